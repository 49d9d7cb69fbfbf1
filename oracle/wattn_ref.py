"""O1: materialized window attention with window-local 2D RoPE, float64 (test infrastructure).

Only tests, the smoke check and the benchmark's CPU-baseline leg use this
module.  It is deliberately plain: numpy float64, a full N x N score matrix per
window-head, no tiling, no fusion.

What is computed ([FS] = the paper card "FLASHSWIN: Unlocking Large Windows and
Dense Tokens in Swin Vision Transformers with Memory Efficient Attention"):

* exact softmax attention inside each M x M window ([FS] Abstract: windowed
  attention computed exactly, without the additive relative-position bias);
* positions restored by window-local 2D RoPE applied to Q and K ([FS] Abstract;
  Figure 1(B)); theta is the per-head angular frequency in rad/token, the
  exp(omega) parameterisation of [FS] Figure S4 lives in the caller;
* Swin's shifted windows: roll the grid by -shift, partition, attend with the
  region mask, un-partition, roll back by +shift (the shifted configuration
  of the workload; the pages themselves do not describe the mask).

Conventions the pages leave open, and the reading taken here:

* token-grid layout [B, Hg, Wg, heads, d]; window token index n = r*M + c;
* channels [0, d/2) carry the row axis, pairs (2j, 2j+1) rotated by
  theta_row[h, j] * r; channels [d/2, d) carry the column axis, pairs
  (d/2+2j, d/2+2j+1) rotated by theta_col[h, j] * c, j in [0, d/4);
* rotation (a, b) -> (a cos phi - b sin phi, a sin phi + b cos phi), the same
  for Q and K; positions (r, c) are in the shifted frame;
* scores S = q~ . k~ / sqrt(d); masked pairs are excluded (weight exactly 0);
* LSE = natural log of sum_j exp(S_ij) over the live keys;
* a grid whose sides are not multiples of M is extended to the next multiples
  Hp x Wp (as Swin pads its feature map before the shift); the roll, the
  windows and the regions are those of the Hp x Wp grid, and the added tokens
  are absent: they are no key of any query, and have no output.

The forward also takes an optional relative-position bias, the term that the
standard Swin window attention adds to its materialized scores and FlashSwin
drops ([FS] Abstract).  It is used only to check the materialized comparison
path.  Reading (the pages give no index convention): a per-head table
bias[h, 2M-1, 2M-1], and the pair (query i, key j) at in-window positions
(r_i, c_i), (r_j, c_j) gets bias[h, r_i - r_j + M - 1, c_i - c_j + M - 1].

The forward and backward also take an optional rank-r additive bias, the learned low-rank bias
factorization of the FlashBias comparison model ([FS] Table S1 and the Table 4 caption: a trainable
rank-16 bias factorization whose parameters grow with M^2).  Reading: per head, factors
U, W [heads, N, r] over the in-window token index n = r*M + c (the shifted frame, as for RoPE); the
pair (query i, key j) adds sum_t U[h, n_i, t] W[h, n_j, t] to its scaled score, before the mask.
Factors shared by all heads are the same array repeated per head.  The backward then also returns
dU = sum over windows of dS W and dW = sum over windows of dS^T U.

Parity: pinned by tests/test_oracle.py (brute force, library attention for
theta = 0, constant-V, closed-form RoPE pair, region decomposition, finite
differences, invariants, agreement with O2).  The RoPE conventions above are
"parity unpinned" against the pages (they print none).
"""

import numpy as np

SUPPORTED_D = (4, 8, 16, 32, 64)


def check_bias(bias, heads, M):
    """Validate an optional relative-position bias table [heads, 2M-1, 2M-1]."""
    if bias is not None and tuple(np.shape(bias)) != (heads, 2 * M - 1, 2 * M - 1):
        raise ValueError("bias must be [heads, 2M-1, 2M-1]")


def check_lowrank(lowrank, heads, M):
    """Validate optional rank-r bias factors (U, W), each [heads, M*M, r] with r >= 1."""
    if lowrank is None:
        return
    U, W = lowrank
    su, sw = np.shape(U), np.shape(W)
    if len(su) != 3 or su != sw or su[:2] != (heads, M * M) or su[2] < 1:
        raise ValueError("lowrank factors must both be [heads, M*M, r], r >= 1")


def lowrank_bias(lowrank):
    """The bias of every (query i, key j) pair of a window, [heads, N, N]: U[h] @ W[h]^T."""
    U, W = (np.asarray(x, dtype=np.float64) for x in lowrank)
    return U @ np.swapaxes(W, -1, -2)


def check_args(shape, theta_row_shape, theta_col_shape, M, shift):
    """Validate a call; raises ValueError with the reason.

    shape = (B, Hg, Wg, heads, d).  Hg, Wg >= 1 (grids that M does not divide
    are padded, see the module notes), 0 <= shift < M, d a multiple of 4,
    theta arrays of shape [heads, d/4].
    """
    if len(shape) != 5:
        raise ValueError("q/k/v must be [B, Hg, Wg, heads, d]")
    B, Hg, Wg, heads, d = shape
    if B < 0 or heads < 1:
        raise ValueError("need B >= 0 and heads >= 1")
    if M < 1 or Hg < 1 or Wg < 1:
        raise ValueError("need Hg, Wg, M >= 1")
    if not (0 <= shift < M):
        raise ValueError("need 0 <= shift < M")
    if d % 4 or d < 4:
        raise ValueError("d must be a positive multiple of 4")
    if tuple(theta_row_shape) != (heads, d // 4) or tuple(theta_col_shape) != (heads, d // 4):
        raise ValueError("theta_row/theta_col must be [heads, d/4]")


def _roll(x, s):
    """Swin cyclic shift: result[Y, X] = x[(Y + s) mod Hg, (X + s) mod Wg]."""
    if s == 0:
        return x
    return np.roll(x, shift=(-s, -s), axis=(1, 2))


def _unroll(x, s):
    if s == 0:
        return x
    return np.roll(x, shift=(s, s), axis=(1, 2))


def _padded(n, M):
    """The multiple of M that a grid side of n tokens is extended to."""
    return -(-n // M) * M


def _pad(x, M):
    """[B, Hg, Wg, *rest] -> [B, Hp, Wp, *rest], the added tokens zero (they are masked out)."""
    Hg, Wg = x.shape[1:3]
    Hp, Wp = _padded(Hg, M), _padded(Wg, M)
    if (Hp, Wp) == (Hg, Wg):
        return x
    widths = [(0, 0), (0, Hp - Hg), (0, Wp - Wg)] + [(0, 0)] * (x.ndim - 3)
    return np.pad(x, widths)


def _partition(x, M):
    """[B, Hg, Wg, *rest] -> [B*nH*nW, M*M, *rest], window index (b, wy, wx), token n = r*M + c."""
    B, Hg, Wg = x.shape[:3]
    rest = x.shape[3:]
    x = x.reshape(B, Hg // M, M, Wg // M, M, *rest)
    x = np.swapaxes(x, 2, 3)  # B, nH, nW, M(r), M(c), rest
    return x.reshape(B * (Hg // M) * (Wg // M), M * M, *rest)


def _unpartition(xw, B, Hg, Wg, M):
    rest = xw.shape[2:]
    x = xw.reshape(B, Hg // M, Wg // M, M, M, *rest)
    x = np.swapaxes(x, 2, 3)
    return x.reshape(B, Hg, Wg, *rest)


def region_labels(Hg, Wg, M, s):
    """Swin region label of every token of every window, shape [nH, nW, M*M].

    In the shifted frame the rows are cut into [0, Hg-M), [Hg-M, Hg-s),
    [Hg-s, Hg) (likewise the columns); label = 3*row_region + col_region.
    With s == 0 every label is 0 (no mask).
    """
    row_lab = np.zeros(Hg, dtype=np.int64)
    col_lab = np.zeros(Wg, dtype=np.int64)
    if s > 0:
        row_lab[Hg - M:Hg - s] = 1
        row_lab[Hg - s:] = 2
        col_lab[Wg - M:Wg - s] = 1
        col_lab[Wg - s:] = 2
    grid = 3 * row_lab[:, None] + col_lab[None, :]  # [Hg, Wg]
    nH, nW = Hg // M, Wg // M
    g = grid.reshape(nH, M, nW, M).swapaxes(1, 2)  # nH, nW, r, c
    return g.reshape(nH, nW, M * M)


def _angles(theta, pos):
    """phi[h, n, j] = theta[h, j] * pos[n]."""
    return theta[:, None, :] * pos[None, :, None]


def rope_rotate(xw, theta_row, theta_col, M, inverse=False):
    """Rotate channel pairs of windowed x [nWin, heads, N, d] by the 2D RoPE angles.

    inverse=True applies the transpose rotation (angle -phi), used to pull
    gradients of the rotated tensor back to the unrotated one.
    """
    d = xw.shape[-1]
    h2 = d // 2
    n = np.arange(M * M)
    r = (n // M).astype(np.float64)
    c = (n % M).astype(np.float64)
    sign = -1.0 if inverse else 1.0
    out = np.empty_like(xw)
    for lo, theta, pos in ((0, theta_row, r), (h2, theta_col, c)):
        phi = sign * _angles(np.asarray(theta, dtype=np.float64), pos)  # [heads, N, d/4]
        cs, sn = np.cos(phi)[None], np.sin(phi)[None]
        a = xw[..., lo:lo + h2:2]
        b = xw[..., lo + 1:lo + h2:2]
        out[..., lo:lo + h2:2] = a * cs - b * sn
        out[..., lo + 1:lo + h2:2] = a * sn + b * cs
    return out


def _windows(x, M, s):
    """Grid tensor [B, Hg, Wg, heads, d] -> windowed float64 [nWin, heads, N, d] (grid padded to Hp x Wp)."""
    xw = _partition(_roll(_pad(np.asarray(x, dtype=np.float64), M), s), M)
    return np.ascontiguousarray(np.swapaxes(xw, 1, 2))


def _grid_back(xw, B, Hg, Wg, M, s):
    """Inverse of _windows for [nWin, heads, N, ...]: un-partition the Hp x Wp grid, roll back, crop."""
    Hp, Wp = _padded(Hg, M), _padded(Wg, M)
    return _unroll(_unpartition(np.swapaxes(xw, 1, 2), B, Hp, Wp, M), s)[:, :Hg, :Wg]


def _window_mask(B, Hg, Wg, M, s):
    """Boolean live-pair mask [nWin, 1, N, N]: same Swin region and a key that is a grid token (not
    padding); None when every pair is live (no shift, no padding)."""
    Hp, Wp = _padded(Hg, M), _padded(Wg, M)
    if s == 0 and (Hp, Wp) == (Hg, Wg):
        return None
    lab = region_labels(Hp, Wp, M, s).reshape(-1, M * M)  # [nH*nW, N]
    live = lab[:, :, None] == lab[:, None, :]
    real = np.zeros((1, Hp, Wp), dtype=bool)
    real[:, :Hg, :Wg] = True
    real_w = _partition(_roll(real, s), M)  # [nH*nW, N]: is window token n a grid token
    live = live & real_w[:, None, :]
    live = np.broadcast_to(live[None], (B,) + live.shape).reshape(-1, 1, M * M, M * M)
    return live


def relative_bias(bias, M):
    """The bias of every (query i, key j) pair of a window, [heads, N, N]:
    bias[h, r_i - r_j + M - 1, c_i - c_j + M - 1], token n = r*M + c."""
    n = np.arange(M * M)
    r, c = n // M, n % M
    dr = r[:, None] - r[None, :] + M - 1
    dc = c[:, None] - c[None, :] + M - 1
    return np.asarray(bias, dtype=np.float64)[:, dr, dc]


def window_scores_ref(q, k, theta_row, theta_col, M, shift, bias=None):
    """Materialized scaled scores S [nWin, heads, N, N] (masked pairs = -inf). Small inputs only."""
    B, Hg, Wg, heads, d = np.shape(q)
    check_bias(bias, heads, M)
    qw = rope_rotate(_windows(q, M, shift), theta_row, theta_col, M)
    kw = rope_rotate(_windows(k, M, shift), theta_row, theta_col, M)
    S = qw @ np.swapaxes(kw, -1, -2) / np.sqrt(d)
    if bias is not None:
        S = S + relative_bias(bias, M)[None]
    live = _window_mask(B, Hg, Wg, M, shift)
    if live is not None:
        S = np.where(live, S, -np.inf)
    return S


# Memory bound on one materialized block of score matrices (float64).  Windows are independent, so
# the forward and backward walk the windows in consecutive slices that fit it; the value only sets
# how many windows share one batched matmul, never what is computed.
CHUNK_BUDGET_BYTES = 256 << 20


def _chunks(n_win, heads, N):
    """Consecutive window slices covering [0, n_win), each holding at most CHUNK_BUDGET_BYTES of
    float64 scores (at least one window per slice)."""
    per = max(1, CHUNK_BUDGET_BYTES // (heads * N * N * 8))
    for lo in range(0, n_win, per):
        yield slice(lo, min(n_win, lo + per))


def _softmax_rows(S):
    """Row softmax of S (masked entries -inf): (P, row max m, row sum of exp(S - m)).  A row with no
    live entry (only a padding query, whose result is dropped) gets P = 0."""
    m = S.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(S - m)
    ssum = e.sum(axis=-1, keepdims=True)
    return e / np.where(ssum > 0, ssum, 1.0), m, ssum


def wattn_fwd_ref(q, k, v, theta_row, theta_col, M, shift, bias=None, lowrank=None):
    """Forward: returns (out [B,Hg,Wg,heads,d] float64, lse [B,Hg,Wg,heads] float64).

    bias: optional relative-position bias table [heads, 2M-1, 2M-1] added to the scores.
    lowrank: optional rank-r bias factors (U, W), each [heads, M*M, r]; U W^T is added to the scores."""
    q = np.asarray(q)
    B, Hg, Wg, heads, d = q.shape
    theta_row = np.asarray(theta_row, dtype=np.float64)
    theta_col = np.asarray(theta_col, dtype=np.float64)
    check_args(q.shape, theta_row.shape, theta_col.shape, M, shift)
    check_bias(bias, heads, M)
    check_lowrank(lowrank, heads, M)
    N = M * M
    rb = None if bias is None else relative_bias(bias, M)[None]
    if lowrank is not None:
        lb = lowrank_bias(lowrank)[None]
        rb = lb if rb is None else rb + lb
    qw = rope_rotate(_windows(q, M, shift), theta_row, theta_col, M)
    kw = rope_rotate(_windows(k, M, shift), theta_row, theta_col, M)
    vw = _windows(v, M, shift)
    live_all = _window_mask(B, Hg, Wg, M, shift)
    ow = np.empty_like(vw)
    lw = np.empty(vw.shape[:3], dtype=np.float64)
    for sl in _chunks(qw.shape[0], heads, N):
        S = qw[sl] @ np.swapaxes(kw[sl], -1, -2) / np.sqrt(d)
        if rb is not None:
            S = S + rb
        if live_all is not None:
            S = np.where(live_all[sl], S, -np.inf)
        P, m, ssum = _softmax_rows(S)
        ow[sl] = P @ vw[sl]
        with np.errstate(divide="ignore"):
            lw[sl] = (m + np.log(ssum))[..., 0]
    return _grid_back(ow, B, Hg, Wg, M, shift), _grid_back(lw, B, Hg, Wg, M, shift)


def _dtheta_terms(xt, dxt, M):
    """Per-pair dtheta integrand summed over windows and tokens.

    For a pair (a, b) rotated by phi = theta * p, d x~_a / d phi = -x~_b and
    d x~_b / d phi = x~_a, so dL/dtheta = sum p * (dx~_b * x~_a - dx~_a * x~_b).
    xt, dxt: [nWin, heads, N, d] (rotated tensor and the gradient w.r.t. it).
    Returns (row [heads, d/4], col [heads, d/4]).
    """
    d = xt.shape[-1]
    h2 = d // 2
    n = np.arange(M * M)
    r = (n // M).astype(np.float64)
    c = (n % M).astype(np.float64)
    res = []
    for lo, pos in ((0, r), (h2, c)):
        a, b = xt[..., lo:lo + h2:2], xt[..., lo + 1:lo + h2:2]
        da, db = dxt[..., lo:lo + h2:2], dxt[..., lo + 1:lo + h2:2]
        integrand = (db * a - da * b) * pos[None, None, :, None]
        res.append(integrand.sum(axis=(0, 2)))
    return res[0], res[1]


def wattn_bwd_ref(q, k, v, dout, theta_row, theta_col, M, shift, lowrank=None):
    """Analytic backward of wattn_fwd_ref.

    Returns (dq, dk, dv [B,Hg,Wg,heads,d], dtheta_row, dtheta_col [heads,d/4]), float64, and with
    lowrank = (U, W) also (dU, dW [heads, M*M, r]).
    dV = P^T dO; dP = dO V^T; D_i = sum_j P_ij dP_ij; dS = P o (dP - D);
    dq~ = dS k~ / sqrt(d); dk~ = dS^T q~ / sqrt(d); dq = R^T dq~, dk = R^T dk~;
    dU = sum over windows of dS W; dW = sum over windows of dS^T U.
    """
    q = np.asarray(q)
    B, Hg, Wg, heads, d = q.shape
    theta_row = np.asarray(theta_row, dtype=np.float64)
    theta_col = np.asarray(theta_col, dtype=np.float64)
    check_args(q.shape, theta_row.shape, theta_col.shape, M, shift)
    check_lowrank(lowrank, heads, M)
    N = M * M
    lb = None if lowrank is None else lowrank_bias(lowrank)[None]
    if lowrank is not None:
        U, W = (np.asarray(x, dtype=np.float64) for x in lowrank)
        dU = np.zeros_like(U)
        dW = np.zeros_like(W)
    qw = rope_rotate(_windows(q, M, shift), theta_row, theta_col, M)
    kw = rope_rotate(_windows(k, M, shift), theta_row, theta_col, M)
    vw = _windows(v, M, shift)
    dow = _windows(dout, M, shift)
    live_all = _window_mask(B, Hg, Wg, M, shift)
    dqt = np.empty_like(qw)
    dkt = np.empty_like(kw)
    dvw = np.empty_like(vw)
    scale = 1.0 / np.sqrt(d)
    for sl in _chunks(qw.shape[0], heads, N):
        S = qw[sl] @ np.swapaxes(kw[sl], -1, -2) * scale
        if lb is not None:
            S = S + lb
        if live_all is not None:
            S = np.where(live_all[sl], S, -np.inf)
        P = _softmax_rows(S)[0]
        dvw[sl] = np.swapaxes(P, -1, -2) @ dow[sl]
        dP = dow[sl] @ np.swapaxes(vw[sl], -1, -2)
        Dr = (P * dP).sum(axis=-1, keepdims=True)
        dS = P * (dP - Dr)
        dqt[sl] = dS @ kw[sl] * scale
        dkt[sl] = np.swapaxes(dS, -1, -2) @ qw[sl] * scale
        if lowrank is not None:
            dU += (dS @ W[None]).sum(axis=0)
            dW += (np.swapaxes(dS, -1, -2) @ U[None]).sum(axis=0)
    tr_q, tc_q = _dtheta_terms(qw, dqt, M)
    tr_k, tc_k = _dtheta_terms(kw, dkt, M)
    dqw = rope_rotate(dqt, theta_row, theta_col, M, inverse=True)
    dkw = rope_rotate(dkt, theta_row, theta_col, M, inverse=True)

    def back(xw):
        return _grid_back(xw, B, Hg, Wg, M, shift)

    grads = (back(dqw), back(dkw), back(dvw), tr_q + tr_k, tc_q + tc_k)
    return grads if lowrank is None else grads + (dU, dW)
