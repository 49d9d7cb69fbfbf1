"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle, element by element.

Tolerances (written here, applied to every output):
  float32 tensors: max-abs <= 1e-5 and relative L2 <= 1e-5 (forward O and LSE); the backward's
    dQ/dK/dV use max-abs <= 1e-5 * max(1, max|ref|) and rel-L2 <= 1e-5.
  bf16 tensors: max-abs <= 2e-2 and relative L2 <= 5e-3 for O, LSE, dQ, dK, dV.
  dtheta (a float32 sum over the whole batch): rel-L2 <= 5e-3 and max-abs <= 2e-2 * max|ref| for
    bf16, 1e-5 relative for float32.
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


@pytest.mark.parametrize("M,shift,grid", [(32, 16, 64), (32, 0, 64), (8, 3, 32), (12, 5, 36)])
def test_forward_loose_bound_falls_back(M, shift, grid):
    """One key with a large norm makes max|q| * max|k| overshoot the true row maximum of most
    queries by more than 80 (log2 units): their sums under the bound reference fall below
    2^-80 and the kernels redo those rows with the exact maximum.  Logits reach ~40 here, and
    operand rounding errors grow with the logit, so max-abs is taken relative to max |ref|."""
    H, D = 2, 32
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
    assert_close("LSE", _np(lse), rl, 2e-2, 5e-3, scale_abs=True)


# ------------------------------------------------------------------------- forward, full workloads

SAMPLE_IMAGES = {
    "swin_t_s1_p4_m8": [0, 1, 127],
    "flashswin_t_s1_p2_m32": [0, 127],
    "flashswin_t_s2_shift16_m32": [0, 64, 127],
}


@pytest.mark.parametrize("name", ["tiny_f32_m8", "swin_t_s1_p4_m8", "flashswin_t_s1_p2_m32",
                                  "flashswin_t_s2_shift16_m32"])
def test_forward_workload(name):
    w = WORKLOADS[name]
    x = workload_inputs(name, with_dout=False)
    xd = to_dev(x)
    s = w["shifts"][0]
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


@pytest.mark.parametrize("shift", [0, 16])
def test_backward_workload(shift):
    """Full-size backward workload: sampled images against the oracle, dtheta by batch linearity."""
    name = "flashswin_t_s1_p2_m32_bwd"
    w = WORKLOADS[name]
    M = w["M"]
    x = workload_inputs(name, with_dout=True)
    xd = to_dev(x)
    out, lse = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], M, shift)
    dq, dk, dv, dtr, dtc = F.wattn_bwd(xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"],
                                       xd["theta_col"], M, shift)
    # determinism: a second run is bit-identical
    dq2, dk2, dv2, dtr2, dtc2 = F.wattn_bwd(xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"],
                                            xd["theta_col"], M, shift)
    torch.cuda.synchronize()
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2), (dtr, dtr2), (dtc, dtc2)):
        assert torch.equal(a, b)
    imgs = [0, w["B"] - 1]
    (q, k, v), tr, tc = oracle_args(x, imgs)
    g = oracle.wattn_bwd_ref(q, k, v, x["dout"][imgs].double().numpy(), tr, tc, M, shift)
    for nm, got, ref in (("dQ", dq[imgs], g[0]), ("dK", dk[imgs], g[1]), ("dV", dv[imgs], g[2])):
        assert_close(nm, _np(got), ref, 2e-2, 5e-3)
    # dtheta is a sum over images: the full-batch value equals the sum of per-chunk values
    tr_sum = torch.zeros_like(dtr, dtype=torch.float64)
    tc_sum = torch.zeros_like(dtc, dtype=torch.float64)
    chunk = 4
    for b0 in range(0, w["B"], chunk):
        sl = slice(b0, b0 + chunk)
        sub = {n: xd[n][sl].contiguous() for n in ("q", "k", "v", "dout")}
        o_c, l_c = F.wattn_fwd(sub["q"], sub["k"], sub["v"], xd["theta_row"], xd["theta_col"], M, shift)
        r = F.wattn_bwd(sub["q"], sub["k"], sub["v"], o_c, sub["dout"], l_c, xd["theta_row"], xd["theta_col"], M,
                        shift)
        tr_sum += r[3].double()
        tc_sum += r[4].double()
        if b0 == 0:
            first = (r[3], r[4])
    assert_close("dtheta_row (batch sum)", _np(dtr), tr_sum.cpu().numpy(), 1e-5, 1e-5, scale_abs=True)
    assert_close("dtheta_col (batch sum)", _np(dtc), tc_sum.cpu().numpy(), 1e-5, 1e-5, scale_abs=True)
    # and the first chunk's dtheta against the oracle on those images
    (q, k, v), tr, tc = oracle_args(x, slice(0, chunk))
    g = oracle.wattn_bwd_ref(q, k, v, x["dout"][:chunk].double().numpy(), tr, tc, M, shift)
    assert_close("dtheta_row (chunk)", _np(first[0]), g[3], 2e-2, 5e-3, scale_abs=True)
    assert_close("dtheta_col (chunk)", _np(first[1]), g[4], 2e-2, 5e-3, scale_abs=True)


@pytest.mark.parametrize("shift", [0, 8])
def test_m16_workload(shift):
    """M = 16 at full size (128 images of 128 x 128 tokens, 3 heads): forward and backward on sampled
    images against the oracle."""
    name = "flashswin_t_s1_p2_m16"
    w = WORKLOADS[name]
    M = w["M"]
    x = workload_inputs(name, with_dout=True)
    xd = to_dev(x)
    out, lse = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], M, shift)
    dq, dk, dv, _, _ = F.wattn_bwd(xd["q"], xd["k"], xd["v"], out, xd["dout"], lse, xd["theta_row"],
                                   xd["theta_col"], M, shift)
    torch.cuda.synchronize()
    imgs = [0, w["B"] - 1]
    (q, k, v), tr, tc = oracle_args(x, imgs)
    ro, rl = oracle.wattn_fwd_ref(q, k, v, tr, tc, M, shift)
    assert_close("O", _np(out[imgs]), ro, 2e-2, 5e-3)
    assert_close("LSE", _np(lse[imgs]), rl, 2e-2, 5e-3)
    g = oracle.wattn_bwd_ref(q, k, v, x["dout"][imgs].double().numpy(), tr, tc, M, shift)
    for nm, got, ref in (("dQ", dq[imgs], g[0]), ("dK", dk[imgs], g[1]), ("dV", dv[imgs], g[2])):
        assert_close(nm, _np(got), ref, 2e-2, 5e-3)


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
