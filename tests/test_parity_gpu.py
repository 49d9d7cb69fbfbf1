"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle, element by element.

Tolerances (written here, applied to every output):
  float32 tensors: max-abs <= 1e-5 and relative L2 <= 1e-5 (forward O and LSE); the backward's
    dQ/dK/dV use max-abs <= 1e-5 * max(1, max|ref|) and rel-L2 <= 1e-5.
  bf16 tensors: max-abs <= 2e-2 and relative L2 <= 5e-3 for O, LSE, dQ, dK, dV.
  dtheta (a float32 sum over the whole batch): rel-L2 <= 5e-3 and max-abs <= 2e-2 * max|ref| for
    bf16, 1e-5 relative for float32.
  LSE with large logits (inputs built to exercise the softmax reference): the score operands are
    rounded to the MFMA format (unit roundoff u = 2^-11 for fp16, 2^-8 for bf16), which moves a
    logit by at most (2u + u^2) |q_i| |k_j| / sqrt(d), and a log-sum-exp moves by at most the
    largest logit change; so |dLSE_i| <= 2e-2 + (2u + 2^-16) |q_i| max_j |k_j| / sqrt(d) over the
    keys of the query's window (lse_rounding_bound).
Small cases run the oracle on the whole input (several tiles and a ragged tail); the full-size
workloads compare sampled images (windows never cross images, so the oracle on those images is
exact for them) in the same launch configuration the benchmark times.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
import vision_transformer_windowed_amd as F
from vision_transformer_windowed_amd.inputs import WORKLOADS, make_device_inputs, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _seed(case):
    return zlib.crc32(repr(case).encode()) % 100000


def _np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def tol(dtype, kind):
    if dtype == "f32":
        return (1e-5, 1e-5)
    return (2e-2, 5e-3)


def assert_close(name, got, ref, max_abs, rel_l2, scale_abs=False):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    ma = max_abs * (max(1.0, np.abs(ref).max()) if scale_abs else 1.0)
    l2 = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    print(f"  {name}: max-abs {err.max():.3e} (tol {ma:.1e})  rel-L2 {l2:.3e} (tol {rel_l2:.1e})", flush=True)
    assert err.max() <= ma, f"{name}: max-abs {err.max():.3e} > {ma:.1e}"
    assert l2 <= rel_l2, f"{name}: rel-L2 {l2:.3e} > {rel_l2:.1e}"


def assert_close_rowwise(name, got, ref, bound, rel_l2):
    """Per-element absolute bound (an array broadcastable to ref) and a relative-L2 bound."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    l2 = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    worst = float((err / bound).max())
    print(f"  {name}: max-abs {err.max():.3e}, worst err/bound {worst:.3f}  rel-L2 {l2:.3e} (tol {rel_l2:.1e})",
          flush=True)
    assert worst <= 1.0, f"{name}: error above the rounding bound (ratio {worst:.3f})"
    assert l2 <= rel_l2, f"{name}: rel-L2 {l2:.3e} > {rel_l2:.1e}"


def window_max(a, M, s):
    """a [B, Hg, Wg, H] >= 0 -> for every token, the maximum of a over the tokens of its shifted window
    (a grid that M does not divide is padded with zeros to the next multiple, as the kernels see it)."""
    B, Hg, Wg, H = a.shape
    Hp, Wp = -(-Hg // M) * M, -(-Wg // M) * M
    a = np.pad(a, [(0, 0), (0, Hp - Hg), (0, Wp - Wg), (0, 0)])
    r = np.roll(a, (-s, -s), axis=(1, 2)).reshape(B, Hp // M, M, Wp // M, M, H)
    m = r.max(axis=(2, 4), keepdims=True)
    m = np.broadcast_to(m, r.shape).reshape(B, Hp, Wp, H)
    return np.roll(m, (s, s), axis=(1, 2))[:, :Hg, :Wg]


def lse_rounding_bound(q, k, M, s, u):
    """2e-2 + (2u + 2^-16) |q_i| max_j |k_j| / sqrt(d), max over the keys of the query's window (RoPE
    keeps norms, so the raw q and k give the norms of the rotated operands)."""
    d = q.shape[-1]
    qn = np.linalg.norm(q, axis=-1)
    kn = window_max(np.linalg.norm(k, axis=-1), M, s)
    return 2e-2 + (2 * u + 2.0 ** -16) * qn * kn / np.sqrt(d)


U_FP16, U_BF16 = 2.0 ** -11, 2.0 ** -8


def to_dev(x):
    return {k: v.to(DEV) for k, v in x.items()}


def oracle_args(x, batch=None):
    sel = slice(None) if batch is None else batch
    return [x[n][sel].double().numpy() for n in ("q", "k", "v")], x["theta_row"].double().numpy(), \
        x["theta_col"].double().numpy()


# ----------------------------------------------------------------------------------- forward

FWD_SMALL = [
    # B, Hg, Wg, heads, d, M, shift, dtype
    (1, 16, 16, 2, 32, 8, 0, "f32"),
    (2, 8, 8, 3, 32, 4, 2, "f32"),
    (1, 12, 12, 1, 16, 6, 3, "f32"),
    (1, 10, 10, 2, 8, 5, 2, "f32"),
    (1, 14, 14, 2, 64, 7, 3, "f32"),
    (1, 24, 24, 2, 32, 12, 5, "f32"),
    (1, 32, 32, 1, 32, 32, 16, "f32"),
    (2, 64, 64, 3, 32, 8, 0, "bf16"),
    (2, 16, 24, 3, 32, 8, 3, "bf16"),
    (1, 64, 64, 3, 32, 32, 0, "bf16"),
    (1, 64, 64, 6, 32, 32, 16, "bf16"),
    (2, 32, 32, 3, 32, 32, 16, "bf16"),
    (1, 40, 40, 2, 32, 20, 7, "bf16"),
    (1, 24, 24, 2, 32, 12, 5, "bf16"),
    (1, 10, 10, 2, 32, 5, 2, "bf16"),
    (1, 33, 33, 1, 32, 11, 4, "bf16"),
    (1, 6, 6, 2, 32, 1, 0, "bf16"),
    (1, 14, 14, 2, 64, 7, 3, "bf16"),
    (1, 16, 16, 2, 16, 8, 4, "bf16"),
    (1, 32, 48, 2, 32, 16, 8, "bf16"),
    (1, 64, 96, 2, 32, 32, 16, "bf16"),
    (1, 16, 16, 20, 32, 8, 3, "bf16"),
    (1, 8, 8, 2, 32, 8, 3, "bf16"),
    (1, 32, 32, 2, 32, 32, 16, "bf16"),
    (1, 64, 64, 1, 32, 32, 31, "bf16"),
    (1, 64, 64, 1, 32, 32, 1, "bf16"),
    (1, 8, 16, 40, 32, 8, 3, "bf16"),
    # d = 64 on MFMA (windows of up to 512 padded tokens); M = 23 runs the float32-arithmetic kernels
    (1, 16, 16, 2, 64, 8, 3, "bf16"),
    (1, 33, 33, 1, 64, 11, 4, "bf16"),
    (1, 24, 24, 2, 64, 12, 5, "bf16"),
    (1, 32, 32, 2, 64, 16, 0, "bf16"),
    (1, 48, 32, 3, 64, 16, 8, "bf16"),
    (1, 40, 40, 2, 64, 20, 7, "bf16"),
    (1, 44, 44, 1, 64, 22, 5, "bf16"),
    (1, 46, 46, 1, 64, 23, 0, "bf16"),
    # windows larger than 32 x 32 (the float32-arithmetic kernels stream the keys)
    (1, 40, 80, 1, 32, 40, 0, "bf16"),
    (1, 64, 64, 1, 32, 64, 32, "bf16"),
    (1, 48, 96, 2, 16, 48, 7, "f32"),
    (1, 64, 64, 1, 64, 64, 0, "f32"),
] + [
    # grids that M does not divide (padded to the next multiple; the padding tokens are absent)
    (1, 10, 13, 2, 32, 4, 0, "f32"),
    (1, 10, 9, 1, 16, 4, 2, "f32"),
    (2, 7, 13, 2, 8, 6, 5, "f32"),
    (1, 3, 2, 1, 32, 4, 1, "f32"),
    (1, 50, 75, 3, 32, 8, 4, "bf16"),
    (1, 50, 38, 2, 32, 16, 8, "bf16"),
    (1, 40, 29, 2, 64, 12, 6, "bf16"),
    (1, 100, 70, 1, 32, 32, 16, "bf16"),
]


@pytest.mark.parametrize("case", FWD_SMALL, ids=lambda c: "B{}_{}x{}_h{}_d{}_M{}_s{}_{}".format(*c))
def test_forward_small(case):
    B, Hg, Wg, H, D, M, s, dt = case
    x = make_inputs(B, Hg, Wg, H, D, dt, seed=_seed(case))
    xd = to_dev(x)
    out, lse = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], M, s)
    torch.cuda.synchronize()
    (q, k, v), tr, tc = oracle_args(x)
    ro, rl = oracle.wattn_fwd_ref(q, k, v, tr, tc, M, s)
    ma, rl2 = tol(dt, "fwd")
    assert_close("O", _np(out), ro, ma, rl2)
    assert_close("LSE", _np(lse), rl, ma, rl2)


def test_forward_theta_zero_is_plain_attention():
    B, Hg, Wg, H, D, M = 1, 64, 64, 3, 32, 32
    x = make_inputs(B, Hg, Wg, H, D, "bf16", seed=77)
    x["theta_row"].zero_()
    x["theta_col"].zero_()
    xd = to_dev(x)
    out, _ = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], M, 0)
    # plain attention per window through torch (float32 on the CPU)
    def win(t):
        return t.float().reshape(B, Hg // M, M, Wg // M, M, H, D).permute(0, 1, 3, 5, 2, 4, 6).reshape(-1, H, M * M, D)
    ref = torch.nn.functional.scaled_dot_product_attention(win(x["q"]), win(x["k"]), win(x["v"]))
    ref = ref.reshape(B, Hg // M, Wg // M, H, M, M, D).permute(0, 1, 4, 2, 5, 3, 6).reshape(B, Hg, Wg, H, D)
    assert_close("O", _np(out), ref.double().numpy(), 2e-2, 5e-3)


def test_forward_without_lse_matches():
    x = make_inputs(1, 64, 64, 3, 32, "bf16", seed=5)
    xd = to_dev(x)
    o1, l1 = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], 32, 16)
    o2, l2 = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], 32, 16, need_lse=False)
    assert l2 is None
    assert torch.equal(o1, o2)


def test_forward_nan_stays_in_its_window_region():
    B, Hg, Wg, H, D, M, s = 1, 64, 64, 2, 32, 32, 16
    x = make_inputs(B, Hg, Wg, H, D, "bf16", seed=9)
    ky, kx = 5, 40
    x["k"][0, ky, kx, 0, 3] = float("nan")
    xd = to_dev(x)
    out, _ = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], M, s)
    bad = torch.isnan(out.float()).any(dim=-1)[0, :, :, 0].cpu().numpy()

    def where(y, xx):
        Y, X = (y - s) % Hg, (xx - s) % Wg
        reg = lambda t, size: int(t >= size - M) + int(t >= size - s)  # noqa: E731
        return (Y // M, X // M, reg(Y, Hg), reg(X, Wg))

    assert bad.sum() > 0
    for y in range(Hg):
        for xx in range(Wg):
            assert bad[y, xx] == (where(y, xx) == where(ky, kx)), (y, xx)
    assert not torch.isnan(out[..., 1, :].float()).any()  # other head untouched


@pytest.mark.parametrize("M,shift,grid,D", [(32, 16, 64, 32), (32, 0, 64, 32), (8, 3, 32, 32), (12, 5, 36, 32),
                                            (16, 8, 32, 64), (20, 7, 40, 64), (16, 8, 40, 32)])
def test_forward_loose_bound_falls_back(M, shift, grid, D):
    """One key with a large norm makes max|q| * max|k| overshoot the true row maximum of most
    queries by more than 80 (log2 units): their sums under the bound reference fall below
    2^-80 and the kernels redo those rows with the exact maximum.  Logits reach ~40 here; the
    operands stay in fp16 range, so LSE is held to the fp16 rounding bound (lse_rounding_bound)."""
    H = 2
    x = make_inputs(1, grid, grid, H, D, "bf16", seed=31 + M)
    ky, kx = grid // 2 + 1, 3
    x["k"][0, ky, kx, 0] *= 14.0
    xd = to_dev(x)
    out, lse = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], M, shift)
    torch.cuda.synchronize()
    (q, k, v), tr, tc = oracle_args(x)
    ro, rl = oracle.wattn_fwd_ref(q, k, v, tr, tc, M, shift)
    # the case is meant: some query's row maximum sits more than 90 below |q_i^| * max|k| (log2
    # units, q^ = q log2(e) / sqrt(d)), which is at most any wave's bound for that query
    l2e = 1.4426950408889634
    qn = np.linalg.norm(q[0, :, :, 0], axis=-1) * l2e / np.sqrt(D)
    kmax = np.linalg.norm(k[0, :, :, 0], axis=-1).max()
    assert np.any(rl[0, :, :, 0] * l2e < qn * kmax - 90.0)
    assert_close("O", _np(out), ro, 2e-2, 5e-3)
    assert_close_rowwise("LSE", _np(lse), rl, lse_rounding_bound(q, k, M, shift, U_FP16), 5e-3)


def _aligned_large_inputs(B, grid, H, D, amp, seed):
    """q = k with entries +-amp (random signs), so every token has the same norm amp * sqrt(d) and
    each query's own key gives the largest score, equal to the Cauchy-Schwarz bound; v ~ N(0, 1)."""
    x = make_inputs(B, grid, grid, H, D, "bf16", seed=seed)
    g = torch.Generator().manual_seed(seed + 7)
    sign = torch.randint(0, 2, (B, grid, grid, H, D), generator=g).float() * 2 - 1
    x["q"] = (sign * amp).to(torch.bfloat16)
    x["k"] = x["q"].clone()
    return x


@pytest.mark.parametrize("M,shift,grid,amp,u,D", [
    (32, 16, 64, 1024.0, U_FP16, 32), (32, 0, 64, 4096.0, U_BF16, 32), (8, 3, 32, 1024.0, U_FP16, 32),
    (8, 0, 32, 4096.0, U_BF16, 32), (16, 8, 32, 1024.0, U_FP16, 32), (12, 5, 36, 4096.0, U_BF16, 32),
    (16, 8, 32, 1024.0, U_FP16, 64), (20, 0, 40, 4096.0, U_BF16, 64), (32, 16, 80, 1024.0, U_FP16, 32)])
def test_forward_aligned_large_norms(M, shift, grid, amp, u, D):
    """Aligned queries and keys with large norms (q = k): the computed score of a query with its own
    key sits at the bound up to operand rounding, which alone can exceed it by far more than 128
    (log2 units).  The widened reference keeps every exponent finite, the sums underflow, and the
    exact-maximum pass gives O = v of the query's own token.  amp = 1024 keeps the rotated operands in
    fp16 range (|k~| = 5793 at d = 32, 8192 at d = 64); amp = 4096 (|k~| = 23170, 32768) takes the
    bf16 operand path."""
    H = 2
    x = _aligned_large_inputs(1, grid, H, D, amp, seed=71 + M + shift)
    xd = to_dev(x)
    out, lse = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], M, shift)
    torch.cuda.synchronize()
    (q, k, v), tr, tc = oracle_args(x)
    ro, rl = oracle.wattn_fwd_ref(q, k, v, tr, tc, M, shift)
    assert_close("O", _np(out), ro, 2e-2, 5e-3)
    assert_close_rowwise("LSE", _np(lse), rl, lse_rounding_bound(q, k, M, shift, u), 5e-3)


def _scaled_window_inputs(case, seed, with_dout):
    """Inputs where the tokens of one shifted-frame window (the last window row and column: the one
    with the most Swin regions when shifted) have K scaled by 2^12 and Q by 2^-12.  The logits are
    unchanged, but |k| ~ 2^12 sqrt(d) leaves fp16 range, so that window-head takes the bf16 operand
    path of every kernel while the others take fp16."""
    B, Hg, Wg, H, D, M, s = case
    x = make_inputs(B, Hg, Wg, H, D, "bf16", seed=seed, with_dout=with_dout)
    rows = [((Hg // M - 1) * M + r + s) % Hg for r in range(M)]
    cols = [((Wg // M - 1) * M + c + s) % Wg for c in range(M)]
    sel = np.zeros((Hg, Wg), dtype=bool)
    sel[np.ix_(rows, cols)] = True
    mask = torch.from_numpy(sel)[None, :, :, None, None]
    x["k"] = torch.where(mask, x["k"].float() * 4096.0, x["k"].float()).to(torch.bfloat16)
    x["q"] = torch.where(mask, x["q"].float() / 4096.0, x["q"].float()).to(torch.bfloat16)
    return x, sel


BF16_PATH_CASES = [(1, 64, 64, 2, 32, 32, 16), (1, 64, 64, 2, 32, 32, 0), (2, 32, 32, 3, 32, 8, 3),
                   (1, 32, 32, 3, 32, 8, 0), (1, 32, 48, 2, 32, 16, 8), (1, 24, 24, 2, 32, 12, 5),
                   (1, 32, 48, 2, 64, 16, 8), (1, 40, 40, 1, 64, 20, 3)]


@pytest.mark.parametrize("case", BF16_PATH_CASES, ids=lambda c: "B{}_{}x{}_h{}_d{}_M{}_s{}".format(*c))
def test_bf16_operand_path(case):
    """Forward and backward with one window-head on bf16 score operands, against the oracle.  The
    scaling is an exact power of two, so the true dq of the scaled window is 2^12 times, and its dk
    2^-12 times, that of an ordinary window: both sides are rescaled by the same powers of two before
    the ordinary tolerances apply.  dtheta is unchanged by the scaling."""
    B, Hg, Wg, H, D, M, s = case
    x, sel = _scaled_window_inputs(case, seed=_seed(case) + 3, with_dout=True)
    xd = to_dev(x)
    out, lse = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], M, s)
    dq, dk, dv, dtr, dtc = F.wattn_bwd(xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"],
                                       xd["theta_col"], M, s)
    torch.cuda.synchronize()
    (q, k, v), tr, tc = oracle_args(x)
    ro, rl = oracle.wattn_fwd_ref(q, k, v, tr, tc, M, s)
    assert_close("O", _np(out), ro, 2e-2, 5e-3)
    assert_close("LSE", _np(lse), rl, 2e-2, 5e-3)
    g = oracle.wattn_bwd_ref(q, k, v, x["dout"].double().numpy(), tr, tc, M, s)
    back = np.where(sel[None, :, :, None, None], 2.0 ** -12, 1.0)
    assert_close("dQ (rescaled)", _np(dq) * back, g[0] * back, 2e-2, 5e-3)
    assert_close("dK (rescaled)", _np(dk) / back, g[1] / back, 2e-2, 5e-3)
    assert_close("dV", _np(dv), g[2], 2e-2, 5e-3)
    assert_close("dtheta_row", _np(dtr), g[3], 2e-2, 5e-3, scale_abs=True)
    assert_close("dtheta_col", _np(dtc), g[4], 2e-2, 5e-3, scale_abs=True)


@pytest.mark.parametrize("M,shift,grid", [(32, 16, 64), (8, 3, 32), (16, 0, 32)])
def test_backward_nan_in_dout_stays_in_its_window_head(M, shift, grid):
    """A NaN in dO at one token and head makes that window-head's maxima non-finite (the backward
    then takes bf16 operands and unit scales there).  Every other window-head's dq, dk, dv, and
    dtheta of the other heads, still match the oracle run on the same inputs with the NaN zeroed;
    dtheta of the NaN's head is NaN."""
    H, D = 2, 32
    x = make_inputs(1, grid, grid, H, D, "bf16", seed=90 + M, with_dout=True)
    ty, tx = 1, grid - 2
    x["dout"][0, ty, tx, 1, 5] = float("nan")
    xd = to_dev(x)
    out, lse = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], M, shift)
    dq, dk, dv, dtr, dtc = F.wattn_bwd(xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"],
                                       xd["theta_col"], M, shift)
    torch.cuda.synchronize()
    (q, k, v), tr, tc = oracle_args(x)
    do = x["dout"].double().numpy()
    do[0, ty, tx, 1, 5] = 0.0
    g = oracle.wattn_bwd_ref(q, k, v, do, tr, tc, M, shift)
    # tokens of the NaN's shifted window
    Y, X = (ty - shift) % grid, (tx - shift) % grid
    rows = [(Y // M * M + r + shift) % grid for r in range(M)]
    cols = [(X // M * M + c + shift) % grid for c in range(M)]
    inwin = np.zeros((grid, grid), dtype=bool)
    inwin[np.ix_(rows, cols)] = True
    keep = ~(inwin[None, :, :, None, None] & (np.arange(H) == 1)[None, None, None, :, None])
    keep = np.broadcast_to(keep, q.shape)
    for name, got, ref in (("dQ", dq, g[0]), ("dK", dk, g[1]), ("dV", dv, g[2])):
        assert_close(name + " (other window-heads)", _np(got)[keep], ref[keep], 2e-2, 5e-3)
    assert_close("dtheta_row (head 0)", _np(dtr)[0], g[3][0], 2e-2, 5e-3, scale_abs=True)
    assert_close("dtheta_col (head 0)", _np(dtc)[0], g[4][0], 2e-2, 5e-3, scale_abs=True)
    assert np.isnan(_np(dtr)[1]).all() and np.isnan(_np(dtc)[1]).all()


# ------------------------------------------------------------------------- forward, full workloads

SAMPLE_IMAGES = {
    "swin_t_s1_p4_m8": [0, 1, 127],
    "flashswin_t_s1_p2_m32": [0, 127],
    "flashswin_t_s2_shift16_m32": [0, 64, 127],
    "wide_heads_s1_p2_m16_d64": [0, 63],
}


@pytest.mark.parametrize("name,s", [("tiny_f32_m8", 0), ("swin_t_s1_p4_m8", 0), ("flashswin_t_s1_p2_m32", 0),
                                    ("flashswin_t_s2_shift16_m32", 16), ("wide_heads_s1_p2_m16_d64", 0),
                                    ("wide_heads_s1_p2_m16_d64", 8)])
def test_forward_workload(name, s):
    w = WORKLOADS[name]
    assert s in w["shifts"]
    x = workload_inputs(name, with_dout=False)
    xd = to_dev(x)
    out, lse = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], w["M"], s)
    torch.cuda.synchronize()
    imgs = SAMPLE_IMAGES.get(name, list(range(w["B"])))
    (q, k, v), tr, tc = oracle_args(x, imgs)
    ro, rl = oracle.wattn_fwd_ref(q, k, v, tr, tc, w["M"], s)
    ma, rl2 = tol(w["dtype"], "fwd")
    assert_close("O", _np(out[imgs]), ro, ma, rl2)
    assert_close("LSE", _np(lse[imgs]), rl, ma, rl2)


# ----------------------------------------------------------------------------------- backward

BWD_SMALL = [
    (1, 16, 16, 2, 32, 8, 0, "f32"),
    (2, 8, 8, 3, 32, 4, 2, "f32"),
    (1, 10, 10, 2, 8, 5, 2, "f32"),
    (1, 14, 14, 1, 64, 7, 3, "f32"),
    (1, 32, 32, 1, 32, 32, 16, "f32"),
    (2, 16, 16, 3, 32, 8, 0, "bf16"),
    (1, 16, 24, 3, 32, 8, 3, "bf16"),
    (1, 64, 64, 3, 32, 32, 0, "bf16"),
    (1, 64, 64, 3, 32, 32, 16, "bf16"),
    (1, 24, 24, 2, 32, 12, 5, "bf16"),
    (1, 40, 40, 2, 32, 20, 7, "bf16"),
    (1, 33, 33, 1, 32, 11, 4, "bf16"),
    (1, 10, 10, 2, 32, 5, 2, "bf16"),
    (1, 16, 16, 2, 16, 8, 4, "bf16"),
    (1, 32, 32, 2, 32, 16, 15, "bf16"),
    (2, 16, 32, 3, 32, 16, 1, "bf16"),
    (1, 32, 48, 2, 32, 16, 8, "bf16"),
    (1, 64, 96, 2, 32, 32, 16, "bf16"),
    (1, 16, 16, 20, 32, 8, 3, "bf16"),
    (1, 8, 8, 2, 32, 8, 3, "bf16"),
    (1, 32, 32, 2, 32, 32, 16, "bf16"),
    (1, 64, 64, 1, 32, 32, 31, "bf16"),
    (1, 64, 64, 1, 32, 32, 1, "bf16"),
    (1, 8, 16, 40, 32, 8, 3, "bf16"),
    # windows larger than 32 x 32
    (1, 40, 40, 1, 32, 40, 13, "bf16"),
    (1, 64, 64, 1, 32, 64, 0, "bf16"),
    (1, 48, 48, 1, 16, 48, 24, "f32"),
    # d = 64 on MFMA (windows of up to 256 tokens); M = 20 runs the float32-arithmetic kernels
    (2, 8, 8, 2, 64, 4, 1, "bf16"),
    (1, 16, 16, 2, 64, 8, 3, "bf16"),
    (1, 33, 33, 1, 64, 11, 4, "bf16"),
    (1, 24, 24, 2, 64, 12, 5, "bf16"),
    (1, 32, 32, 2, 64, 16, 0, "bf16"),
    (1, 48, 32, 3, 64, 16, 8, "bf16"),
    (1, 40, 40, 1, 64, 20, 7, "bf16"),
    # grids that M does not divide (padded)
    (1, 10, 13, 2, 32, 4, 1, "f32"),
    (2, 7, 13, 1, 16, 6, 5, "f32"),
    (1, 10, 9, 1, 8, 4, 2, "f32"),
    (1, 50, 75, 2, 32, 8, 4, "bf16"),
    (1, 50, 38, 1, 32, 16, 8, "bf16"),
    (1, 40, 29, 1, 64, 12, 6, "bf16"),
    (1, 70, 100, 1, 32, 32, 16, "bf16"),
    (1, 45, 20, 2, 32, 20, 7, "bf16"),
    (1, 30, 47, 1, 64, 16, 8, "bf16"),
    (2, 9, 7, 1, 32, 4, 3, "bf16"),
]


def _bwd_check(x, M, s, dt, batch=None):
    xd = to_dev(x)
    out, lse = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], M, s)
    dq, dk, dv, dtr, dtc = F.wattn_bwd(xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"],
                                       xd["theta_col"], M, s)
    torch.cuda.synchronize()
    (q, k, v), tr, tc = oracle_args(x)
    g = oracle.wattn_bwd_ref(q, k, v, x["dout"].double().numpy(), tr, tc, M, s)
    if dt == "f32":
        for name, got, ref in (("dQ", dq, g[0]), ("dK", dk, g[1]), ("dV", dv, g[2])):
            assert_close(name, _np(got), ref, 1e-5, 1e-5, scale_abs=True)
        for name, got, ref in (("dtheta_row", dtr, g[3]), ("dtheta_col", dtc, g[4])):
            assert_close(name, _np(got), ref, 1e-5, 1e-5, scale_abs=True)
    else:
        for name, got, ref in (("dQ", dq, g[0]), ("dK", dk, g[1]), ("dV", dv, g[2])):
            assert_close(name, _np(got), ref, 2e-2, 5e-3)
        for name, got, ref in (("dtheta_row", dtr, g[3]), ("dtheta_col", dtc, g[4])):
            assert_close(name, _np(got), ref, 2e-2, 5e-3, scale_abs=True)


@pytest.mark.parametrize("case", BWD_SMALL, ids=lambda c: "B{}_{}x{}_h{}_d{}_M{}_s{}_{}".format(*c))
def test_backward_small(case):
    B, Hg, Wg, H, D, M, s, dt = case
    x = make_inputs(B, Hg, Wg, H, D, dt, seed=_seed(case) + 1, with_dout=True)
    _bwd_check(x, M, s, dt)


# (B, Hg, Wg, heads, d, M, shift, offset): bf16 padded grids on the MFMA backward (d = 64 whole-window
# kernels, d = 32 chunked kernels) whose padding, rolled by the shift, reaches the second-to-last
# window row and column (shift + padding > M)
FAR_NEGATIVE_CASES = [(1, 40, 29, 1, 64, 12, 6, 4.5), (1, 50, 38, 1, 32, 16, 8, 5.0),
                      (1, 26, 37, 2, 64, 16, 12, 4.5)]


@pytest.mark.parametrize("case", FAR_NEGATIVE_CASES, ids=lambda c: "{}x{}_d{}_M{}_s{}".format(*c[1:3], *c[4:7]))
def test_backward_padded_far_negative_scores(case):
    """Q near -a and K near +a in every channel with theta = 0 put every score of a real pair near
    -a^2 sqrt(d) (all far below -89), so exp(-LSE) overflows float32; V = 0.  Then O = 0, dP = dO V^T = 0 and
    Delta = 0, so dS = P (dP - Delta) = 0 for every real pair: dQ, dK and dtheta are exactly zero, and
    dV = P^T dO carries the probabilities.  A padding key (a zero vector, score 0) must get P = 0
    exactly rather than exp(0 - LSE) = inf, which would make its dS = inf * 0 = NaN and dQ = dS K
    NaN.  Padding sits in interior windows as well as in the last window row and column.  LSE is
    compared within the large-logit rounding bound of the module docstring (fp16 operands: every
    component is far inside fp16 range)."""
    B, Hg, Wg, H, D, M, s, a = case
    Hp, Wp = -(-Hg // M) * M, -(-Wg // M) * M
    assert s + Hp - Hg > M and s + Wp - Wg > M and a * a * D ** 0.5 > 128
    x = make_inputs(B, Hg, Wg, H, D, "bf16", seed=_seed(case) + 2, with_dout=True)
    x["q"] = (x["q"].float() - a).to(torch.bfloat16)
    x["k"] = (x["k"].float() + a).to(torch.bfloat16)
    x["v"].zero_()
    x["theta_row"].zero_()
    x["theta_col"].zero_()
    xd = to_dev(x)
    out, lse = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], M, s)
    dq, dk, dv, dtr, dtc = F.wattn_bwd(xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"],
                                       xd["theta_col"], M, s)
    torch.cuda.synchronize()
    (q, k, v), tr, tc = oracle_args(x)
    ro, rl = oracle.wattn_fwd_ref(q, k, v, tr, tc, M, s)
    g = oracle.wattn_bwd_ref(q, k, v, x["dout"].double().numpy(), tr, tc, M, s)
    assert rl.max() < -89.0  # exp(-LSE) is beyond float32 for every query
    assert not out.any()
    assert_close_rowwise("LSE", _np(lse), rl, lse_rounding_bound(q, k, M, s, U_FP16), 5e-3)
    for name, got in (("dQ", dq), ("dK", dk), ("dtheta_row", dtr), ("dtheta_col", dtc)):
        print(f"  {name}: {int((got != 0).sum())} nonzero, {int((~torch.isfinite(got)).sum())} non-finite",
              flush=True)
        assert not got.any(), name
    # dV = P^T dO sums up to a window of dO rows (entries reach 20 and more) and P carries the
    # large-logit LSE rounding, so its max-abs bound is relative to max|dV|
    assert_close("dV", _np(dv), g[2], 2e-2, 5e-3, scale_abs=True)


def oracle_bwd_over_batch(x, M, s, got, chunk=4):
    """Run the oracle's backward over the whole batch in chunks of `chunk` images (windows never cross
    images, so each chunk is exact for its images) and compare dq, dk, dv of every image with `got`
    (GPU tensors); dtheta, a sum over the batch, is accumulated and compared at the end.  The
    tolerances are the bf16 ones of the module docstring, over the whole batch."""
    B = x["q"].shape[0]
    tr, tc = x["theta_row"].double().numpy(), x["theta_col"].double().numpy()
    stats = {n: [0.0, 0.0, 0.0] for n in ("dQ", "dK", "dV")}
    dtr = np.zeros(tr.shape)
    dtc = np.zeros(tc.shape)
    for b0 in range(0, B, chunk):
        sl = slice(b0, min(B, b0 + chunk))
        q, k, v, do = (x[n][sl].double().numpy() for n in ("q", "k", "v", "dout"))
        g = oracle.wattn_bwd_ref(q, k, v, do, tr, tc, M, s)
        for (name, ref), t in zip((("dQ", g[0]), ("dK", g[1]), ("dV", g[2])), got[:3]):
            mine = _np(t[sl])
            assert np.all(np.isfinite(mine)), name
            st = stats[name]
            st[0] = max(st[0], float(np.abs(mine - ref).max()))
            st[1] += float(((mine - ref) ** 2).sum())
            st[2] += float((ref ** 2).sum())
        dtr += g[3]
        dtc += g[4]
    for name, (ma, se, sr) in stats.items():
        l2 = (se / sr) ** 0.5
        print(f"  {name} (all {B} images): max-abs {ma:.3e} (tol 2.0e-02)  rel-L2 {l2:.3e} (tol 5.0e-03)", flush=True)
        assert ma <= 2e-2 and l2 <= 5e-3, name
    assert_close(f"dtheta_row (all {B} images)", _np(got[3]), dtr, 2e-2, 5e-3, scale_abs=True)
    assert_close(f"dtheta_col (all {B} images)", _np(got[4]), dtc, 2e-2, 5e-3, scale_abs=True)


@pytest.mark.parametrize("shift", [0, 16])
def test_backward_workload(shift):
    """Full-size backward workload ([32,128,128,3,32], M = 32): dq, dk, dv of all 32 images and the
    full-batch dtheta against the oracle; determinism; dtheta also by batch linearity."""
    name = "flashswin_t_s1_p2_m32_bwd"
    w = WORKLOADS[name]
    M = w["M"]
    x = workload_inputs(name, with_dout=True)
    xd = to_dev(x)
    out, lse = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], M, shift)
    got = F.wattn_bwd(xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"], xd["theta_col"], M,
                      shift)
    # determinism: a second run is bit-identical
    again = F.wattn_bwd(xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"], xd["theta_col"], M,
                        shift)
    torch.cuda.synchronize()
    for a, b in zip(got, again):
        assert torch.equal(a, b)
    oracle_bwd_over_batch(x, M, shift, got)
    # dtheta is a sum over images: the full-batch value equals the sum of per-chunk calls
    tr_sum = torch.zeros_like(got[3], dtype=torch.float64)
    tc_sum = torch.zeros_like(got[4], dtype=torch.float64)
    chunk = 4
    for b0 in range(0, w["B"], chunk):
        sl = slice(b0, b0 + chunk)
        sub = {n: xd[n][sl].contiguous() for n in ("q", "k", "v", "dout")}
        o_c, l_c = F.wattn_fwd(sub["q"], sub["k"], sub["v"], xd["theta_row"], xd["theta_col"], M, shift)
        r = F.wattn_bwd(sub["q"], sub["k"], sub["v"], o_c, sub["dout"], l_c, xd["theta_row"], xd["theta_col"], M,
                        shift)
        tr_sum += r[3].double()
        tc_sum += r[4].double()
    assert_close("dtheta_row (batch sum)", _np(got[3]), tr_sum.cpu().numpy(), 1e-5, 1e-5, scale_abs=True)
    assert_close("dtheta_col (batch sum)", _np(got[4]), tc_sum.cpu().numpy(), 1e-5, 1e-5, scale_abs=True)


@pytest.mark.parametrize("shift", [0, 8])
def test_m16_workload(shift):
    """M = 16 at full size (128 images of 128 x 128 tokens, 3 heads): forward on sampled images, and
    the backward's dq, dk, dv of all images and its full-batch dtheta, against the oracle."""
    name = "flashswin_t_s1_p2_m16"
    w = WORKLOADS[name]
    M = w["M"]
    x = workload_inputs(name, with_dout=True)
    xd = to_dev(x)
    out, lse = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], M, shift)
    got = F.wattn_bwd(xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"], xd["theta_col"], M,
                      shift)
    torch.cuda.synchronize()
    imgs = [0, w["B"] - 1]
    (q, k, v), tr, tc = oracle_args(x, imgs)
    ro, rl = oracle.wattn_fwd_ref(q, k, v, tr, tc, M, shift)
    assert_close("O", _np(out[imgs]), ro, 2e-2, 5e-3)
    assert_close("LSE", _np(lse[imgs]), rl, 2e-2, 5e-3)
    oracle_bwd_over_batch(x, M, shift, got, chunk=16)


@pytest.mark.parametrize("shift", [0, 8])
def test_d64_workload(shift):
    """64-wide heads at M = 16 at full size (64 images of 128 x 128 tokens, 3 heads of d = 64): forward on
    sampled images, and the backward's dq, dk, dv of all images and its full-batch dtheta, against the
    oracle."""
    name = "wide_heads_s1_p2_m16_d64"
    w = WORKLOADS[name]
    M = w["M"]
    x = workload_inputs(name, with_dout=True)
    xd = to_dev(x)
    out, lse = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], M, shift)
    got = F.wattn_bwd(xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"], xd["theta_col"], M,
                      shift)
    torch.cuda.synchronize()
    imgs = [0, w["B"] - 1]
    (q, k, v), tr, tc = oracle_args(x, imgs)
    ro, rl = oracle.wattn_fwd_ref(q, k, v, tr, tc, M, shift)
    assert_close("O", _np(out[imgs]), ro, 2e-2, 5e-3)
    assert_close("LSE", _np(lse[imgs]), rl, 2e-2, 5e-3)
    oracle_bwd_over_batch(x, M, shift, got, chunk=8)


def test_autograd_matches_backward_entry_point():
    x = make_inputs(1, 32, 32, 2, 32, "bf16", seed=3, with_dout=True)
    xd = to_dev(x)
    leaves = {n: xd[n].clone().requires_grad_(True) for n in ("q", "k", "v", "theta_row", "theta_col")}
    out = F.window_attention(leaves["q"], leaves["k"], leaves["v"], leaves["theta_row"], leaves["theta_col"], 16, 4)
    out.backward(xd["dout"])
    o, l = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], 16, 4)
    ref = F.wattn_bwd(xd["q"], xd["k"], xd["v"], o, xd["dout"], l, xd["theta_row"], xd["theta_col"], 16, 4)
    for n, r in zip(("q", "k", "v", "theta_row", "theta_col"), ref):
        assert torch.equal(leaves[n].grad, r), n


def test_caller_workspace_any_dtype_or_too_small():
    """A caller's workspace is sized in bytes whatever its dtype, and one that is too small is
    replaced; the gradients are bit-identical to those with the binding's own workspace."""
    x = make_inputs(2, 32, 32, 3, 32, "bf16", seed=11, with_dout=True)
    xd = to_dev(x)
    out, lse = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], 16, 8)
    args = (xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"], xd["theta_col"], 16, 8)
    ref = F.wattn_bwd(*args)
    nbytes = F.bwd_workspace_bytes(xd["q"], 16, 8)
    for ws in (torch.empty((nbytes + 3) // 4, device=DEV, dtype=torch.float32),
               torch.empty(16, device=DEV, dtype=torch.uint8)):
        got = F.wattn_bwd(*args, workspace=ws)
        for a, b in zip(ref, got):
            assert torch.equal(a, b)


def test_empty_batch():
    x = make_inputs(0, 16, 16, 2, 32, "bf16", seed=1, with_dout=True)
    xd = to_dev(x)
    out, lse = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], 8, 4)
    assert out.shape == (0, 16, 16, 2, 32) and lse.shape == (0, 16, 16, 2)


def test_large_tensors_64bit_offsets():
    """Tensors above 4 GiB, so byte offsets pass 2^32 in every kernel (and the backward prologue takes
    its 64-bit addressing): [1400, 128, 128, 3, 32] bf16, M = 32, shift 16, inputs drawn on the GPU.
    The first, middle and last images against the oracle (dtheta sums over all images: not checked)."""
    B, Hg, Wg, H, D, M, s = 1400, 128, 128, 3, 32, 32, 16
    assert B * Hg * Wg * H * D * 2 > 2 ** 32
    x = make_device_inputs(B, Hg, Wg, H, D, "bf16", seed=1777, device=DEV, with_dout=True)
    out, lse = F.wattn_fwd(x["q"], x["k"], x["v"], x["theta_row"], x["theta_col"], M, s)
    dq, dk, dv, _, _ = F.wattn_bwd(x["q"], x["k"], x["v"], out, x["dout"], lse, x["theta_row"], x["theta_col"],
                                   M, s)
    torch.cuda.synchronize()
    imgs = [0, B // 2, B - 1]
    q, k, v, dout = (_np(x[n][imgs]) for n in ("q", "k", "v", "dout"))
    tr, tc = _np(x["theta_row"]), _np(x["theta_col"])
    ro, rl = oracle.wattn_fwd_ref(q, k, v, tr, tc, M, s)
    assert_close("O", _np(out[imgs]), ro, 2e-2, 5e-3)
    assert_close("LSE", _np(lse[imgs]), rl, 2e-2, 5e-3)
    g = oracle.wattn_bwd_ref(q, k, v, dout, tr, tc, M, s)
    for nm, got, ref in (("dQ", dq[imgs], g[0]), ("dK", dk[imgs], g[1]), ("dV", dv[imgs], g[2])):
        assert_close(nm, _np(got), ref, 2e-2, 5e-3)


def test_huge_image_64bit_in_image_offsets():
    """One image whose tensors exceed 4 GiB (6.4 GB: [1, 4096, 8192, 3, 32] bf16), so offsets within
    a single image pass 2^32 bytes.  Shift 0, so a window is a 32 x 32 sub-grid: windows at the start,
    middle and far end of the image against the oracle on those windows alone."""
    B, Hg, Wg, H, D, M = 1, 4096, 8192, 3, 32, 32
    assert Hg * Wg * H * D * 2 > 2 ** 32
    x = make_device_inputs(B, Hg, Wg, H, D, "bf16", seed=2024, device=DEV, with_dout=True)
    out, lse = F.wattn_fwd(x["q"], x["k"], x["v"], x["theta_row"], x["theta_col"], M, 0)
    dq, dk, dv, _, _ = F.wattn_bwd(x["q"], x["k"], x["v"], out, x["dout"], lse, x["theta_row"], x["theta_col"],
                                   M, 0)
    torch.cuda.synchronize()
    tr, tc = _np(x["theta_row"]), _np(x["theta_col"])
    for wy, wx in ((0, 0), (64, 128), (Hg // M - 1, Wg // M - 1)):
        sl = (slice(None), slice(wy * M, wy * M + M), slice(wx * M, wx * M + M))
        q, k, v, dout = (_np(x[n][sl]) for n in ("q", "k", "v", "dout"))
        ro, rl = oracle.wattn_fwd_ref(q, k, v, tr, tc, M, 0)
        assert_close(f"O {wy},{wx}", _np(out[sl]), ro, 2e-2, 5e-3)
        assert_close(f"LSE {wy},{wx}", _np(lse[sl]), rl, 2e-2, 5e-3)
        g = oracle.wattn_bwd_ref(q, k, v, dout, tr, tc, M, 0)
        for nm, got, ref in (("dQ", dq[sl], g[0]), ("dK", dk[sl], g[1]), ("dV", dv[sl], g[2])):
            assert_close(f"{nm} {wy},{wx}", _np(got), ref, 2e-2, 5e-3)
