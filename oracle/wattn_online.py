"""O2: online-softmax window attention by index arithmetic, float64 (test infrastructure).

An independent second route to the same quantity as O1 (wattn_ref), used to
cross-check O1.  Only tests, the smoke check and the benchmark's CPU-baseline
leg use this module.  It shares no helper with O1:

* no roll and no reshape-partition: each window of the shifted frame gathers
  its tokens from the original grid with (wy*M + r + s) mod Hp and
  (wx*M + c + s) mod Wp, and results are scattered back to the same tokens;
  Hp, Wp are Hg, Wg rounded up to multiples of M, and a window token whose row
  is >= Hg or column >= Wg is padding: never a key, never written back (the
  padded-grid reading of O1);
* the region of a shifted-frame row Y is (Y >= Hp-M) + (Y >= Hp-s) (likewise
  for columns), compared as a pair;
* RoPE is a complex phase: channel pair (a, b) is z = a + i*b and the rotated
  pair is z * exp(i*phi) ([FS] Abstract and Figure 1(B): window-local 2D RoPE
  on Q and K; [FS] = the paper card "FLASHSWIN: Unlocking Large Windows and
  Dense Tokens in Swin Vision Transformers with Memory Efficient Attention");
* the softmax is streamed over key tiles with a running maximum and running
  sum (the "exact softmax without materializing the score matrix" of the
  [FS] Abstract), the tile size deliberately not dividing N;
* the backward recomputes P from the saved log-sum-exp and uses
  D_i = sum_d dO_i * O_i, and takes the theta gradient as
  Re(conj(dz~) * i z~) * position.

Parity: checked against O1 in tests/test_oracle.py; O1 is pinned there by
brute force, closed forms, library attention and finite differences.
"""

import numpy as np


def _window_coords(Hg, Wg, M, s, wy, wx):
    """Padded-grid rows/cols of shifted-frame window (wy, wx), region ids of its tokens and whether
    each token (n = r*M + c) is a grid token rather than padding."""
    Hp, Wp = -(-Hg // M) * M, -(-Wg // M) * M
    Y = wy * M + np.arange(M)
    X = wx * M + np.arange(M)
    ys = (Y + s) % Hp
    xs = (X + s) % Wp
    if s > 0:
        ry = (Y >= Hp - M).astype(np.int64) + (Y >= Hp - s).astype(np.int64)
        rx = (X >= Wp - M).astype(np.int64) + (X >= Wp - s).astype(np.int64)
    else:
        ry = np.zeros(M, dtype=np.int64)
        rx = np.zeros(M, dtype=np.int64)
    reg_r = np.repeat(ry, M)
    reg_c = np.tile(rx, M)
    real = (np.repeat(ys, M) < Hg) & (np.tile(xs, M) < Wg)
    return ys, xs, reg_r, reg_c, real


def _gather(x, ys, xs):
    """x [B,Hg,Wg,heads,(d)] -> [B, heads, M*M, (d)] for the window rows ys, cols xs; padding rows and
    columns (>= Hg, >= Wg) read as zero."""
    Hg, Wg = x.shape[1:3]
    w = x[:, np.minimum(ys, Hg - 1)][:, :, np.minimum(xs, Wg - 1)]  # B, M, M, heads, (d)
    keep = (ys < Hg)[:, None] & (xs < Wg)[None, :]
    w = np.where(keep.reshape((1, len(ys), len(xs)) + (1,) * (w.ndim - 3)), w, 0.0)
    B, M1, M2 = w.shape[:3]
    w = w.reshape((B, M1 * M2) + w.shape[3:])
    return np.moveaxis(w, 2, 1).astype(np.float64)


def _scatter(dst, w, ys, xs):
    """Inverse of _gather for dst [B,Hg,Wg,heads,(d)] and w [B, heads, N, (d)]: grid tokens only."""
    Hg, Wg = dst.shape[1:3]
    B, H, N = w.shape[:3]
    M = len(ys)
    t = np.moveaxis(w, 1, 2).reshape((B, M, M, H) + w.shape[3:])
    ry, cx = np.nonzero(ys < Hg)[0], np.nonzero(xs < Wg)[0]
    dst[np.ix_(np.arange(B), ys[ry], xs[cx])] = t[:, ry][:, :, cx]


def _phase(theta_row, theta_col, M):
    """exp(i*phi) for every (head, token, pair), [heads, N, d/2] complex.

    Pairs 0..d/4-1 are the row axis (angle theta_row * r), pairs d/4..d/2-1 the
    column axis (angle theta_col * c).
    """
    r = np.repeat(np.arange(M), M).astype(np.float64)
    c = np.tile(np.arange(M), M).astype(np.float64)
    phi = np.concatenate([theta_row[:, None, :] * r[None, :, None],
                          theta_col[:, None, :] * c[None, :, None]], axis=-1)
    return np.exp(1j * phi), np.concatenate(
        [np.broadcast_to(r[:, None], (M * M, theta_row.shape[1])),
         np.broadcast_to(c[:, None], (M * M, theta_col.shape[1]))], axis=-1)


def _to_complex(x):
    return x[..., 0::2] + 1j * x[..., 1::2]


def _to_real(z):
    out = np.empty(z.shape[:-1] + (2 * z.shape[-1],), dtype=np.float64)
    out[..., 0::2] = z.real
    out[..., 1::2] = z.imag
    return out


def wattn_fwd_online(q, k, v, theta_row, theta_col, M, shift, key_tile=24):
    """Forward by streamed keys; returns (out [B,Hg,Wg,heads,d], lse [B,Hg,Wg,heads]) in float64."""
    q = np.asarray(q)
    B, Hg, Wg, H, D = q.shape
    theta_row = np.asarray(theta_row, dtype=np.float64)
    theta_col = np.asarray(theta_col, dtype=np.float64)
    N = M * M
    ph, _ = _phase(theta_row, theta_col, M)
    out = np.zeros((B, Hg, Wg, H, D), dtype=np.float64)
    lse = np.zeros((B, Hg, Wg, H), dtype=np.float64)
    inv_sqrt_d = 1.0 / np.sqrt(D)
    for wy in range(-(-Hg // M)):
        for wx in range(-(-Wg // M)):
            ys, xs, reg_r, reg_c, real = _window_coords(Hg, Wg, M, shift, wy, wx)
            qt = _to_real(_to_complex(_gather(q, ys, xs)) * ph[None])
            kt = _to_real(_to_complex(_gather(k, ys, xs)) * ph[None])
            vt = _gather(v, ys, xs)
            run_max = np.full((B, H, N), -np.inf)
            run_sum = np.zeros((B, H, N))
            acc = np.zeros((B, H, N, D))
            for j0 in range(0, N, key_tile):
                j1 = min(N, j0 + key_tile)
                s = qt @ np.swapaxes(kt[:, :, j0:j1], -1, -2) * inv_sqrt_d
                same = (reg_r[:, None] == reg_r[None, j0:j1]) & (reg_c[:, None] == reg_c[None, j0:j1])
                same &= real[None, j0:j1]
                s = np.where(same[None, None], s, -np.inf)
                new_max = np.maximum(run_max, s.max(axis=-1))
                ref = np.where(np.isfinite(new_max), new_max, 0.0)
                alpha = np.exp(run_max - ref)
                p = np.exp(s - ref[..., None])
                run_sum = alpha * run_sum + p.sum(axis=-1)
                acc = alpha[..., None] * acc + p @ vt[:, :, j0:j1]
                run_max = new_max
            with np.errstate(divide="ignore", invalid="ignore"):  # padding queries: dropped by _scatter
                _scatter(out, acc / run_sum[..., None], ys, xs)
                _scatter(lse, run_max + np.log(run_sum), ys, xs)
    return out, lse


def wattn_bwd_online(q, k, v, out, lse, dout, theta_row, theta_col, M, shift, key_tile=24):
    """Backward from the saved (out, lse): returns (dq, dk, dv, dtheta_row, dtheta_col), float64."""
    q = np.asarray(q)
    B, Hg, Wg, H, D = q.shape
    theta_row = np.asarray(theta_row, dtype=np.float64)
    theta_col = np.asarray(theta_col, dtype=np.float64)
    N = M * M
    ph, pos = _phase(theta_row, theta_col, M)
    dq = np.zeros((B, Hg, Wg, H, D))
    dk = np.zeros((B, Hg, Wg, H, D))
    dv = np.zeros((B, Hg, Wg, H, D))
    dphi_pos = np.zeros((H, D // 2))  # accumulated p * dL/dphi per (head, pair)
    inv_sqrt_d = 1.0 / np.sqrt(D)
    for wy in range(-(-Hg // M)):
        for wx in range(-(-Wg // M)):
            ys, xs, reg_r, reg_c, real = _window_coords(Hg, Wg, M, shift, wy, wx)
            zq = _to_complex(_gather(q, ys, xs)) * ph[None]
            zk = _to_complex(_gather(k, ys, xs)) * ph[None]
            qt, kt = _to_real(zq), _to_real(zk)
            vt = _gather(v, ys, xs)
            ot = _gather(out, ys, xs)
            dot = _gather(dout, ys, xs)
            l_w = _gather(lse[..., None], ys, xs)[..., 0]  # B, H, N
            Drow = (dot * ot).sum(axis=-1)  # B, H, N
            dqt = np.zeros_like(qt)
            dkt = np.zeros_like(kt)
            dvt = np.zeros_like(vt)
            for j0 in range(0, N, key_tile):
                j1 = min(N, j0 + key_tile)
                s = qt @ np.swapaxes(kt[:, :, j0:j1], -1, -2) * inv_sqrt_d
                same = (reg_r[:, None] == reg_r[None, j0:j1]) & (reg_c[:, None] == reg_c[None, j0:j1])
                same &= real[:, None] & real[None, j0:j1]
                p = np.where(same[None, None], np.exp(s - l_w[..., None]), 0.0)
                dvt[:, :, j0:j1] = np.swapaxes(p, -1, -2) @ dot
                dp = dot @ np.swapaxes(vt[:, :, j0:j1], -1, -2)
                ds = p * (dp - Drow[..., None])
                dqt += ds @ kt[:, :, j0:j1] * inv_sqrt_d
                dkt[:, :, j0:j1] = np.swapaxes(ds, -1, -2) @ qt * inv_sqrt_d
            dzq, dzk = _to_complex(dqt), _to_complex(dkt)
            # dL/dphi for z~ = z e^{i phi}: Re(conj(dz~) * i z~)
            for dz, zt in ((dzq, zq), (dzk, zk)):
                g = np.real(np.conj(dz) * 1j * zt)  # B, H, N, d/2
                dphi_pos += (g * pos[None, None]).sum(axis=(0, 2))
            _scatter(dq, _to_real(dzq * np.conj(ph)[None]), ys, xs)
            _scatter(dk, _to_real(dzk * np.conj(ph)[None]), ys, xs)
            _scatter(dv, dvt, ys, xs)
    q4 = D // 4
    return dq, dk, dv, dphi_pos[:, :q4], dphi_pos[:, q4:]
