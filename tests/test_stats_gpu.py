"""GPU checks of the forward's operand summary (flashswin_wattn_fwd_stats / _bwd_stats).

The summary holds, per window-head, the largest |component| of the window's q, k and v rows of that
head; the backward sizes its fp16 operand scaling from it instead of reading q, k and v again.  Checks:
  - the summary equals those maxima computed here on the host (exact: a maximum of bf16 magnitudes
    is a bf16 value), for the MFMA forward (with and without split query workgroups, d 32 and 64,
    shifted and padded grids, a low-rank bias, the one-wave M = 8 kernel) and for the float32-arithmetic
    forward followed by the separate maxima pass (windows above 32 x 32); out and LSE are bit-identical
    to the plain forward;
  - the backward with the summary is bit-identical to the plain backward on grids that M divides
    (the maxima, hence every scale, are the same), and on padded grids within the bf16 tolerance of
    the fp64 oracle (max-abs 2e-2, relative L2 5e-3), since its maxima then cover only grid tokens;
  - float32 tensors: the summary is not written and the backward ignores it.
The summary's layout is the library's own: {max |q| of a first workgroup's queries, of a second
(0 when one workgroup takes all), max |k|, max |v|}.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
import vision_transformer_windowed_amd as F
from vision_transformer_windowed_amd.inputs import lowrank_factors, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# B, Hg, Wg, heads, d, M, shift, rank
CASES = [
    (2, 32, 32, 3, 32, 8, 3, 0),       # M = 8: one-wave forward
    (1, 16, 16, 40, 32, 8, 3, 0),      # M = 8 with 40 heads: the whole-window instance
    (1, 48, 32, 3, 32, 16, 8, 0),      # M = 16 instance
    (1, 64, 64, 2, 32, 32, 16, 0),     # M = 32 instance, shifted
    (1, 256, 256, 8, 32, 32, 0, 0),    # 512 window-heads: 64 of them split over two workgroups
    (1, 24, 24, 2, 32, 12, 5, 0),      # run-time M
    (1, 32, 32, 2, 64, 16, 0, 0),      # d = 64
    (1, 48, 32, 3, 64, 16, 8, 0),
    (1, 44, 44, 1, 64, 22, 5, 0),      # d = 64, 512 padded tokens (the float32-arithmetic backward)
    (1, 80, 40, 1, 32, 40, 0, 0),      # M = 40: float32-arithmetic forward, then the maxima pass
    (1, 46, 46, 1, 64, 23, 4, 0),      # d = 64 beyond 512 padded tokens: the same at d = 64
    (1, 20, 18, 2, 32, 8, 3, 4),       # a bias on a padded grid: float32-arithmetic forward and backward
    (1, 50, 38, 2, 32, 16, 8, 0),      # padded grids
    (1, 40, 29, 2, 64, 12, 6, 0),
    (1, 100, 70, 1, 32, 32, 16, 0),
    (1, 32, 32, 2, 32, 16, 0, 16),     # low-rank bias
    (2, 24, 24, 3, 32, 8, 3, 5),
    (1, 48, 32, 1, 32, 16, 0, 20),
]


def _ids(c):
    return "B{}_{}x{}_h{}_d{}_M{}_s{}_r{}".format(*c)


def _seed(case):
    return zlib.crc32(repr(case).encode()) % 100000


def _inputs(case, dtype="bf16"):
    B, Hg, Wg, H, D, M, s, r = case
    x = make_inputs(B, Hg, Wg, H, D, dtype, seed=_seed(case), with_dout=True)
    xd = {n: t.to(DEV) for n, t in x.items()}
    if r:
        U, W = lowrank_factors(H, M, r, seed=_seed(case) + 7)
        xd["U"], xd["W"] = U.to(DEV), W.to(DEV)
    return x, xd


def window_head_max(x, M, s):
    """x [B, Hg, Wg, H, d] (host) -> max |component| per window-head, window-major with heads fastest:
    the grid padded with zeros to multiples of M, rolled by -s over the padded extents, partitioned."""
    a = x.float().abs().amax(dim=-1).numpy()
    B, Hg, Wg, H = a.shape
    Hp, Wp = -(-Hg // M) * M, -(-Wg // M) * M
    a = np.pad(a, [(0, 0), (0, Hp - Hg), (0, Wp - Wg), (0, 0)])
    a = np.roll(a, (-s, -s), axis=(1, 2)).reshape(B, Hp // M, M, Wp // M, M, H)
    return a.max(axis=(2, 4)).reshape(-1)


def _fwd(xd, case, stats=None):
    M, s, r = case[5], case[6], case[7]
    args = (xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"])
    if r:
        return F.wattn_fwd_lowrank(*args, xd["U"], xd["W"], M, s, stats=stats)
    return F.wattn_fwd(*args, M, s, stats=stats)


def _bwd(xd, case, out, lse, stats=None):
    M, s, r = case[5], case[6], case[7]
    args = (xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"], xd["theta_col"])
    if r:
        return F.wattn_bwd_lowrank(*args, xd["U"], xd["W"], M, s, stats=stats)
    return F.wattn_bwd(*args, M, s, stats=stats)


def _padded(case):
    _, Hg, Wg, _, _, M, _, _ = case
    return Hg % M != 0 or Wg % M != 0


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_summary_is_the_window_maxima(case):
    print("case", _ids(case), flush=True)
    x, xd = _inputs(case)
    M, s = case[5], case[6]
    stats = torch.full((F.flashswin_wattn_stats_bytes(*case[:7], F.FSW_BF16) // 4,), float("nan"), device=DEV)
    o1, l1 = _fwd(xd, case, stats)
    o0, l0 = _fwd(xd, case)
    torch.cuda.synchronize()
    assert torch.equal(o1, o0) and torch.equal(l1, l0)
    st = stats.cpu().numpy().reshape(-1, 4)
    assert np.all(np.isfinite(st)) and np.all(st >= 0)
    np.testing.assert_array_equal(np.maximum(st[:, 0], st[:, 1]), window_head_max(x["q"], M, s))
    np.testing.assert_array_equal(st[:, 2], window_head_max(x["k"], M, s))
    np.testing.assert_array_equal(st[:, 3], window_head_max(x["v"], M, s))


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_backward_with_summary(case):
    print("case", _ids(case), flush=True)
    x, xd = _inputs(case)
    M, s, r = case[5], case[6], case[7]
    stats = F.new_stats(xd["q"], M, s)
    out, lse = _fwd(xd, case, stats)
    got = _bwd(xd, case, out, lse, stats)
    ref = _bwd(xd, case, out, lse)
    torch.cuda.synchronize()
    names = ("dQ", "dK", "dV", "dtheta_row", "dtheta_col", "dU", "dW")
    if not _padded(case) or r:
        # grids that M divides (the same maxima as the prologue's own), and a bias on a padded grid (the
        # float32-arithmetic backward, which reads no summary)
        for n, a, b in zip(names, got, ref):
            assert torch.equal(a, b), n
        return
    # a padded grid on the MFMA backward: the oracle decides
    (q, k, v) = [x[n].double().numpy() for n in ("q", "k", "v")]
    g = oracle.wattn_bwd_ref(q, k, v, x["dout"].double().numpy(), x["theta_row"].double().numpy(),
                             x["theta_col"].double().numpy(), M, s)
    for i, n in enumerate(names[:5]):
        a = got[i].detach().to("cpu", torch.float64).numpy()
        err = np.abs(a - g[i]).max()
        l2 = np.linalg.norm(a - g[i]) / max(np.linalg.norm(g[i]), 1e-300)
        bound = 2e-2 * (max(1.0, np.abs(g[i]).max()) if i >= 3 else 1.0)
        print(f"  {n}: max-abs {err:.3e} (tol {bound:.1e})  rel-L2 {l2:.3e}", flush=True)
        assert err <= bound and l2 <= 5e-3, n


def test_nan_component_gives_an_infinite_summary():
    """A NaN in q makes its window-head's max |q| infinite (as the backward's own prologue counts it):
    the backward then takes bf16 operands there, exactly as without the summary."""
    case = (1, 32, 32, 2, 32, 16, 0, 0)
    x, xd = _inputs(case)
    xd["q"][0, 3, 5, 1, 7] = float("nan")  # window (0, 0), head 1
    stats = F.new_stats(xd["q"], 16, 0)
    out, lse = _fwd(xd, case, stats)
    got = _bwd(xd, case, out, lse, stats)
    ref = _bwd(xd, case, out, lse)
    torch.cuda.synchronize()
    st = stats.cpu().numpy().reshape(-1, 4)
    assert np.isinf(max(st[1, 0], st[1, 1])) and np.all(np.isfinite(np.delete(st, 1, axis=0)))
    for n, a, b in zip(("dQ", "dK", "dV", "dtheta_row", "dtheta_col"), got, ref):
        assert torch.equal(torch.nan_to_num(a, nan=7.0), torch.nan_to_num(b, nan=7.0)), n
        assert torch.equal(torch.isnan(a), torch.isnan(b)), n


def test_float32_summary_is_not_written():
    case = (1, 16, 16, 2, 32, 8, 0, 0)
    x, xd = _inputs(case, "f32")
    stats = torch.full((F.flashswin_wattn_stats_bytes(*case[:7], F.FSW_F32) // 4,), -3.0, device=DEV)
    out, lse = _fwd(xd, case, stats)
    got = _bwd(xd, case, out, lse, stats)
    ref = _bwd(xd, case, out, lse)
    torch.cuda.synchronize()
    assert torch.all(stats == -3.0)
    for n, a, b in zip(("dQ", "dK", "dV", "dtheta_row", "dtheta_col"), got, ref):
        assert torch.equal(a, b), n


def _small_bf16_cases():
    from test_parity_gpu import BWD_SMALL
    return [c for c in BWD_SMALL if c[-1] == "bf16"]


@pytest.mark.parametrize("case", _small_bf16_cases(), ids=lambda c: "B{}_{}x{}_h{}_d{}_M{}_s{}_{}".format(*c))
def test_summary_path_matches_oracle_on_the_small_backward_cases(case):
    """Every bf16 case of the small backward set (MFMA and float32-arithmetic kernels, shifts, padded
    grids, d = 16, 32, 64, windows up to 64 x 64) through the calls with the operand summary, against
    the fp64 oracle at the backward's bf16 tolerances (max-abs 2e-2, relative L2 5e-3; dtheta max-abs
    relative to max |ref|)."""
    B, Hg, Wg, H, D, M, s, dt = case
    print("case", case, flush=True)
    x = make_inputs(B, Hg, Wg, H, D, dt, seed=_seed(case) + 5, with_dout=True)
    xd = {n: t.to(DEV) for n, t in x.items()}
    stats = F.new_stats(xd["q"], M, s)
    out, lse = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], M, s, stats=stats)
    got = F.wattn_bwd(xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"], xd["theta_col"], M, s,
                      stats=stats)
    torch.cuda.synchronize()
    q, k, v = (x[n].double().numpy() for n in ("q", "k", "v"))
    tr, tc = x["theta_row"].double().numpy(), x["theta_col"].double().numpy()
    g = oracle.wattn_bwd_ref(q, k, v, x["dout"].double().numpy(), tr, tc, M, s)
    for i, n in enumerate(("dQ", "dK", "dV", "dtheta_row", "dtheta_col")):
        a = got[i].detach().to("cpu", torch.float64).numpy()
        err = np.abs(a - g[i]).max()
        l2 = np.linalg.norm(a - g[i]) / max(np.linalg.norm(g[i]), 1e-300)
        bound = 2e-2 * (max(1.0, np.abs(g[i]).max()) if i >= 3 else 1.0)
        print(f"  {n}: max-abs {err:.3e} (tol {bound:.1e})  rel-L2 {l2:.3e}", flush=True)
        assert np.all(np.isfinite(a)) and err <= bound and l2 <= 5e-3, n


@pytest.mark.parametrize("name,rank", [("flashswin_t_s1_p2_m32", 0), ("flashswin_t_s1_p2_m16", 0),
                                       ("wide_heads_s1_p2_m16_d64", 0), ("flashswin_t_s1_p2_m16", 16)])
def test_benchmark_workloads_with_summary_are_bit_identical(name, rank):
    """The benchmark's full-size workloads, in the launch configuration it times: the forward with the
    summary returns the plain forward's out and LSE, and the backward with the summary the plain
    backward's gradients, bit for bit (the plain calls are held to the oracle by the workload tests)."""
    from vision_transformer_windowed_amd.inputs import WORKLOADS, workload_inputs
    w = WORKLOADS[name]
    M = w["M"]
    print("workload", name, "rank", rank, flush=True)
    xd = {n: t.to(DEV) for n, t in workload_inputs(name, with_dout=True).items()}
    case = (w["B"], w["Hg"], w["Wg"], w["heads"], w["d"], M, 0, rank)
    if rank:
        U, W = lowrank_factors(w["heads"], M, rank, seed=2024)
        xd["U"], xd["W"] = U.to(DEV), W.to(DEV)
    stats = F.new_stats(xd["q"], M, 0)
    o1, l1 = _fwd(xd, case, stats)
    o0, l0 = _fwd(xd, case)
    assert torch.equal(o1, o0) and torch.equal(l1, l0)
    g1 = _bwd(xd, case, o0, l0, stats)
    g0 = _bwd(xd, case, o0, l0)
    torch.cuda.synchronize()
    for n, a, b in zip(("dQ", "dK", "dV", "dtheta_row", "dtheta_col", "dU", "dW"), g1, g0):
        assert torch.equal(a, b), n
