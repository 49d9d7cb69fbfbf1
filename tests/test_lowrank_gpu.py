"""GPU parity of the rank-r additive bias (flashswin_wattn_fwd_lowrank / flashswin_wattn_bwd_lowrank)
against the fp64 oracle: O, LSE, dQ, dK, dV, dtheta and the factor gradients dU, dW.

bf16 d = 32 with windows of at most 256 tokens runs the whole-window MFMA backward (the bias as extra
score channels; the factor gradients summed over groups of windows); larger windows, other d, float32
and padded grids run the float32-arithmetic kernels.

The factors are N(0, 0.5^2) per entry; the oracle adds U[h, n_i] . W[h, n_j] to the scaled score of
every pair before the region mask.  Tolerances are those of test_parity_gpu.py: bf16 inputs, max-abs
<= 2e-2 and relative L2 <= 5e-3 (for dtheta, dU and dW, which are sums over the whole batch, max-abs
relative to max|ref|); float32 inputs, 1e-5 both, max-abs relative to max|ref| when that exceeds 1.
A bf16 output is stored rounded, up to 2^-9 of its own magnitude, which at |dV| of 4 and more is
itself near 2e-2: for bf16 tensors the per-element bound is 2e-2 + 2^-8 |ref|."""

import numpy as np
import pytest
import torch

import oracle
import vision_transformer_windowed_amd as F
from vision_transformer_windowed_amd.inputs import WORKLOADS, lowrank_factors, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _close(name, got, ref, max_abs, rel, scale_abs=False, bf16_store=False):
    diff = np.abs(got - ref)
    err = diff.max()
    l2 = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    bound = max_abs * max(1.0, np.abs(ref).max()) if scale_abs else max_abs
    ratio = (diff / (bound + (2.0 ** -8 * np.abs(ref) if bf16_store else 0.0))).max()
    print(f"  {name}: max-abs {err:.3e} (bound {bound:.3e}{' + 2^-8 |ref|' if bf16_store else ''}, worst ratio "
          f"{ratio:.3f}, max|ref| {np.abs(ref).max():.3e}) rel-L2 {l2:.3e}", flush=True)
    assert np.all(np.isfinite(got)), name
    assert ratio <= 1.0 and l2 <= rel, name


def _factors(H, M, r, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn((H, M * M, r), generator=g) * 0.5, torch.randn((H, M * M, r), generator=g) * 0.5)


CASES = [
    # B, Hg, Wg, heads, d, M, shift, rank, dtype
    (1, 16, 16, 2, 32, 8, 0, 16, "f32"),
    (2, 12, 12, 1, 16, 6, 3, 4, "f32"),
    (1, 10, 13, 2, 32, 4, 1, 3, "f32"),      # padded grid
    (1, 32, 32, 2, 32, 8, 4, 16, "bf16"),
    (1, 32, 48, 1, 32, 16, 8, 16, "bf16"),
    (1, 64, 64, 1, 32, 32, 16, 8, "bf16"),
    (1, 24, 24, 2, 64, 12, 5, 32, "bf16"),
    (1, 14, 14, 1, 8, 7, 2, 1, "bf16"),
    (1, 50, 38, 1, 32, 16, 8, 16, "bf16"),   # padded grid
    # bf16, d = 32, windows of up to 512 tokens: the MFMA forward with the bias as extra score channels
    (2, 16, 16, 2, 32, 8, 3, 32, "bf16"),
    (1, 24, 24, 2, 32, 12, 5, 20, "bf16"),
    (1, 32, 32, 3, 32, 16, 0, 1, "bf16"),
    (1, 40, 40, 2, 32, 20, 7, 16, "bf16"),
    (1, 44, 44, 1, 32, 22, 0, 32, "bf16"),
    (1, 10, 10, 2, 32, 5, 2, 9, "bf16"),
    # enough window-heads that the MFMA backward gives each workgroup several windows of one head:
    # 135 windows x 16 heads (2 per group, the last group one window), 279 x 30 (8 per group, the last 7)
    (15, 24, 24, 16, 32, 8, 3, 16, "bf16"),
    (31, 24, 24, 30, 32, 8, 5, 24, "bf16"),
    (2, 64, 64, 3, 32, 16, 8, 16, "bf16"),
    # M = 16 (the forward instances that load the factors with K, V and Q): ranks that leave part of
    # an 8-channel group or of the second 16-channel step empty
    (1, 32, 32, 2, 32, 16, 8, 20, "bf16"),
    (1, 48, 32, 1, 32, 16, 0, 9, "bf16"),
]


def _run(case):
    B, Hg, Wg, H, D, M, s, r, dt = case
    x = make_inputs(B, Hg, Wg, H, D, dt, seed=900 + M + s + r, with_dout=True)
    U, W = _factors(H, M, r, seed=950 + M + r)
    xd = {n: t.to(DEV) for n, t in x.items()}
    Ud, Wd = U.to(DEV), W.to(DEV)
    out, lse = F.wattn_fwd_lowrank(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], Ud, Wd, M, s)
    grads = F.wattn_bwd_lowrank(xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"], xd["theta_col"],
                                Ud, Wd, M, s)
    torch.cuda.synchronize()
    q, k, v, do = (x[n].double().numpy() for n in ("q", "k", "v", "dout"))
    tr, tc = x["theta_row"].double().numpy(), x["theta_col"].double().numpy()
    lr = (U.double().numpy(), W.double().numpy())
    ref_fwd = oracle.wattn_fwd_ref(q, k, v, tr, tc, M, s, lowrank=lr)
    ref_bwd = oracle.wattn_bwd_ref(q, k, v, do, tr, tc, M, s, lowrank=lr)
    return (out, lse), grads, ref_fwd, ref_bwd


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_{}x{}_h{}_d{}_M{}_s{}_r{}_{}".format(*c))
def test_lowrank_matches_oracle(case):
    dt = case[-1]
    (out, lse), grads, (ro, rl), rg = _run(case)
    if dt == "f32":
        tol = dict(max_abs=1e-5, rel=1e-5, scale_abs=True)
        _close("O", _np(out), ro, **tol)
        _close("LSE", _np(lse), rl, **tol)
    else:
        _close("O", _np(out), ro, 2e-2, 5e-3, bf16_store=True)
        _close("LSE", _np(lse), rl, 2e-2, 5e-3)
    names = ("dQ", "dK", "dV", "dtheta_row", "dtheta_col", "dU", "dW")
    for i, (name, got, ref) in enumerate(zip(names, grads, rg)):
        if dt == "f32":
            _close(name, _np(got), ref, 1e-5, 1e-5, scale_abs=True)
        else:
            _close(name, _np(got), ref, 2e-2, 5e-3, scale_abs=i >= 3, bf16_store=i < 3)


def test_lowrank_factor_gradients_are_reproducible():
    """dU and dW are per-window sums reduced in a fixed order: two calls give identical bits."""
    B, Hg, Wg, H, D, M, s, r = 2, 32, 32, 2, 32, 8, 4, 8
    x = make_inputs(B, Hg, Wg, H, D, "bf16", seed=971, with_dout=True)
    U, W = (t.to(DEV) for t in _factors(H, M, r, seed=972))
    xd = {n: t.to(DEV) for n, t in x.items()}
    out, lse = F.wattn_fwd_lowrank(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], U, W, M, s)
    g1 = F.wattn_bwd_lowrank(xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"], xd["theta_col"], U,
                             W, M, s)
    g2 = F.wattn_bwd_lowrank(xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"], xd["theta_col"], U,
                             W, M, s)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_lowrank_zero_factors_equal_the_plain_forward():
    """U = W = 0 adds nothing: the low-rank forward (float32-arithmetic kernels) equals the plain forward
    of the same inputs on the float32 path."""
    B, Hg, Wg, H, D, M, s = 1, 16, 16, 2, 32, 8, 3
    x = make_inputs(B, Hg, Wg, H, D, "f32", seed=973)
    xd = {n: t.to(DEV) for n, t in x.items()}
    Z = torch.zeros((H, M * M, 2), device=DEV)
    o1, l1 = F.wattn_fwd_lowrank(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], Z, Z, M, s)
    o0, l0 = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], M, s)
    torch.cuda.synchronize()
    assert torch.allclose(o1, o0, rtol=0, atol=1e-6) and torch.allclose(l1, l0, rtol=0, atol=1e-6)


@pytest.mark.parametrize("M,shift,rank", [(16, 8, 16), (12, 5, 32)])
def test_lowrank_bf16_operand_path(M, shift, rank):
    """W scaled by 2^14 and U by 2^-14 leaves every bias term unchanged, but max|W| of every head leaves
    fp16 range (about 2.5 sigma of thousands of entries times 2^13 > 2^14), so the MFMA forward and
    backward take bf16 operands for every window-head.  O and LSE against the oracle, and dU times 2^-14
    and dW times 2^14 (the unscaled magnitudes)."""
    B, Hg, Wg, H, D = 1, 2 * M, 2 * M, 2, 32
    x = make_inputs(B, Hg, Wg, H, D, "bf16", seed=980 + M, with_dout=True)
    U, W = _factors(H, M, rank, seed=985 + M)
    U, W = U * 2.0 ** -14, W * 2.0 ** 14
    assert float(W.abs().amax(dim=(1, 2)).min()) >= 2.0 ** 14
    xd = {n: t.to(DEV) for n, t in x.items()}
    out, lse = F.wattn_fwd_lowrank(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], U.to(DEV),
                                   W.to(DEV), M, shift)
    grads = F.wattn_bwd_lowrank(xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"], xd["theta_col"],
                                U.to(DEV), W.to(DEV), M, shift)
    torch.cuda.synchronize()
    q, k, v, do = (x[n].double().numpy() for n in ("q", "k", "v", "dout"))
    tr, tc = x["theta_row"].double().numpy(), x["theta_col"].double().numpy()
    lr = (U.double().numpy(), W.double().numpy())
    ro, rl = oracle.wattn_fwd_ref(q, k, v, tr, tc, M, shift, lowrank=lr)
    _close("O", _np(out), ro, 2e-2, 5e-3)
    _close("LSE", _np(lse), rl, 2e-2, 5e-3)
    rg = oracle.wattn_bwd_ref(q, k, v, do, tr, tc, M, shift, lowrank=lr)
    _close("dU (x 2^-14)", _np(grads[5]) * 2.0 ** -14, rg[5] * 2.0 ** -14, 2e-2, 5e-3, scale_abs=True)
    _close("dW (x 2^14)", _np(grads[6]) * 2.0 ** 14, rg[6] * 2.0 ** 14, 2e-2, 5e-3, scale_abs=True)


def test_lowrank_large_bias_falls_back():
    """A key whose W row has an entry of 200 in a column that every U row leaves at 0 adds nothing to
    any score but makes max|k'| about 200, so the bound max|q'| max|k'| overshoots every row's maximum
    by far more than 80 (log2 units): the MFMA forward redoes the rows with the exact maximum."""
    B, Hg, Wg, H, D, M, s, r = 1, 32, 32, 2, 32, 16, 8, 4
    x = make_inputs(B, Hg, Wg, H, D, "bf16", seed=990)
    U, W = _factors(H, M, r, seed=991)
    U[:, :, 0] = 0.0
    W[:, 5, 0] = 200.0
    xd = {n: t.to(DEV) for n, t in x.items()}
    out, lse = F.wattn_fwd_lowrank(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], U.to(DEV),
                                   W.to(DEV), M, s)
    torch.cuda.synchronize()
    q, k, v = (x[n].double().numpy() for n in ("q", "k", "v"))
    tr, tc = x["theta_row"].double().numpy(), x["theta_col"].double().numpy()
    ro, rl = oracle.wattn_fwd_ref(q, k, v, tr, tc, M, s, lowrank=(U.double().numpy(), W.double().numpy()))
    _close("O", _np(out), ro, 2e-2, 5e-3)
    _close("LSE", _np(lse), rl, 2e-2, 5e-3)


def test_lowrank_workload():
    """The rank-16 bias at the size and launch configuration the benchmark times (flashswin_t_s1_p2_m16:
    128 images of 128 x 128 tokens, 3 heads, M = 16, s = 0; the benchmark's factors, seed 2024; the
    MFMA backward walks 8 windows per workgroup): the forward on sampled images; the backward's dq, dk,
    dv of every image and its full-batch dtheta, dU and dW, against the oracle run over the batch in
    chunks of 16 images (windows never cross images; dtheta, dU and dW are sums over the chunks)."""
    name, rank, seed = "flashswin_t_s1_p2_m16", 16, 2024
    w = WORKLOADS[name]
    B, M = w["B"], w["M"]
    x = workload_inputs(name, with_dout=True)
    U, W = lowrank_factors(w["heads"], M, rank, seed)
    xd = {n: t.to(DEV) for n, t in x.items()}
    out, lse = F.wattn_fwd_lowrank(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], U.to(DEV),
                                   W.to(DEV), M, 0)
    grads = F.wattn_bwd_lowrank(xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"], xd["theta_col"],
                                U.to(DEV), W.to(DEV), M, 0)
    torch.cuda.synchronize()
    tr, tc = x["theta_row"].double().numpy(), x["theta_col"].double().numpy()
    lr = (U.double().numpy(), W.double().numpy())
    imgs = [0, B - 1]
    q, k, v = (x[n][imgs].double().numpy() for n in ("q", "k", "v"))
    ro, rl = oracle.wattn_fwd_ref(q, k, v, tr, tc, M, 0, lowrank=lr)
    _close("O (images 0, B-1)", _np(out[imgs]), ro, 2e-2, 5e-3, bf16_store=True)
    _close("LSE (images 0, B-1)", _np(lse[imgs]), rl, 2e-2, 5e-3)
    worst = {n: 0.0 for n in ("dQ", "dK", "dV")}
    sq = {n: [0.0, 0.0] for n in worst}
    sums = [np.zeros(tr.shape), np.zeros(tc.shape), np.zeros(lr[0].shape), np.zeros(lr[1].shape)]
    for b0 in range(0, B, 16):
        sl = slice(b0, b0 + 16)
        q, k, v, do = (x[n][sl].double().numpy() for n in ("q", "k", "v", "dout"))
        g = oracle.wattn_bwd_ref(q, k, v, do, tr, tc, M, 0, lowrank=lr)
        for name_, ref, t in zip(("dQ", "dK", "dV"), g[:3], grads[:3]):
            mine = _np(t[sl])
            assert np.all(np.isfinite(mine)), name_
            worst[name_] = max(worst[name_], float((np.abs(mine - ref) / (2e-2 + 2.0 ** -8 * np.abs(ref))).max()))
            sq[name_][0] += float(((mine - ref) ** 2).sum())
            sq[name_][1] += float((ref ** 2).sum())
        for acc, part in zip(sums, g[3:]):
            acc += part
    for name_ in worst:
        l2 = (sq[name_][0] / sq[name_][1]) ** 0.5
        print(f"  {name_} (all {B} images): worst err / (2e-2 + 2^-8 |ref|) {worst[name_]:.3f}, rel-L2 {l2:.3e}",
              flush=True)
        assert worst[name_] <= 1.0 and l2 <= 5e-3, name_
    for name_, got, ref in zip(("dtheta_row", "dtheta_col", "dU", "dW"), grads[3:], sums):
        _close(f"{name_} (all {B} images)", _np(got), ref, 2e-2, 5e-3, scale_abs=True)
