"""GPU tests of the packed-qkv entry points (qkv [B, Hg, Wg, 3, heads, d] read in place, dqkv written
packed): results are bit-identical to the separate-tensor entry points on the three slices, which
the other GPU tests hold to the oracle, and the packed forward and backward are also compared with
the oracle directly."""

import numpy as np
import pytest
import torch

import oracle
import vision_transformer_windowed_amd as F
from vision_transformer_windowed_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (B, Hg, Wg, heads, d, M, shift, dtype): the M=32, M=8, M=16 and general MFMA kernels, the
# float32 kernels and d = 64
CASES = [
    (1, 64, 64, 2, 32, 32, 16, "bf16"),
    (2, 32, 32, 3, 32, 8, 0, "bf16"),
    (1, 24, 24, 2, 32, 12, 5, "bf16"),
    (1, 16, 16, 2, 32, 8, 3, "f32"),
    (1, 14, 14, 2, 64, 7, 3, "bf16"),
    (1, 32, 48, 2, 32, 16, 8, "bf16"),
]
IDS = ["B{}_{}x{}_h{}_d{}_M{}_s{}_{}".format(*c) for c in CASES]


def packed_inputs(case, seed, with_dout=False):
    B, Hg, Wg, H, D, M, s, dt = case
    x = make_inputs(B, Hg, Wg, H, D, dt, seed=seed, with_dout=with_dout)
    qkv = torch.stack([x["q"], x["k"], x["v"]], dim=3).contiguous().to(DEV)
    return x, qkv


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_packed_forward_equals_separate(case):
    B, Hg, Wg, H, D, M, s, dt = case
    x, qkv = packed_inputs(case, seed=11)
    tr, tc = x["theta_row"].to(DEV), x["theta_col"].to(DEV)
    out_p, lse_p = F.wattn_fwd_packed(qkv, tr, tc, M, s)
    q, k, v = (qkv[:, :, :, i].contiguous() for i in range(3))
    out_s, lse_s = F.wattn_fwd(q, k, v, tr, tc, M, s)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_s)
    assert torch.equal(lse_p, lse_s)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_packed_backward_equals_separate(case):
    B, Hg, Wg, H, D, M, s, dt = case
    x, qkv = packed_inputs(case, seed=12, with_dout=True)
    tr, tc = x["theta_row"].to(DEV), x["theta_col"].to(DEV)
    dout = x["dout"].to(DEV)
    out, lse = F.wattn_fwd_packed(qkv, tr, tc, M, s)
    dqkv, dtr_p, dtc_p = F.wattn_bwd_packed(qkv, out, dout, lse, tr, tc, M, s)
    q, k, v = (qkv[:, :, :, i].contiguous() for i in range(3))
    dq, dk, dv, dtr_s, dtc_s = F.wattn_bwd(q, k, v, out, dout, lse, tr, tc, M, s)
    torch.cuda.synchronize()
    for i, g in enumerate((dq, dk, dv)):
        assert torch.equal(dqkv[:, :, :, i], g), i
    assert torch.equal(dtr_p, dtr_s)
    assert torch.equal(dtc_p, dtc_s)


def test_packed_forward_matches_oracle():
    case = (1, 64, 64, 2, 32, 32, 16, "bf16")
    B, Hg, Wg, H, D, M, s, dt = case
    x, qkv = packed_inputs(case, seed=13)
    out, lse = F.wattn_fwd_packed(qkv, x["theta_row"].to(DEV), x["theta_col"].to(DEV), M, s)
    torch.cuda.synchronize()
    ro, rl = oracle.wattn_fwd_ref(x["q"].double().numpy(), x["k"].double().numpy(), x["v"].double().numpy(),
                                  x["theta_row"].double().numpy(), x["theta_col"].double().numpy(), M, s)
    for name, got, ref in (("O", out, ro), ("LSE", lse, rl)):
        g = got.to("cpu", torch.float64).numpy()
        err = np.abs(g - ref)
        l2 = np.linalg.norm(g - ref) / np.linalg.norm(ref)
        print(f"  {name}: max-abs {err.max():.3e} rel-L2 {l2:.3e}", flush=True)
        assert err.max() <= 2e-2 and l2 <= 5e-3, name


@pytest.mark.parametrize("case", [(1, 64, 64, 2, 32, 32, 16, "bf16"), (2, 32, 32, 3, 32, 8, 3, "bf16")],
                         ids=["M32_s16", "M8_s3"])
def test_packed_backward_matches_oracle(case):
    """The packed backward's dq, dk, dv slices of dqkv and its dtheta against the oracle (bf16
    tolerances: max-abs 2e-2 and rel-L2 5e-3; dtheta max-abs 2e-2 max|ref|)."""
    B, Hg, Wg, H, D, M, s, dt = case
    x, qkv = packed_inputs(case, seed=15, with_dout=True)
    tr, tc = x["theta_row"].to(DEV), x["theta_col"].to(DEV)
    out, lse = F.wattn_fwd_packed(qkv, tr, tc, M, s)
    dqkv, dtr, dtc = F.wattn_bwd_packed(qkv, out, x["dout"].to(DEV), lse, tr, tc, M, s)
    torch.cuda.synchronize()
    g = oracle.wattn_bwd_ref(x["q"].double().numpy(), x["k"].double().numpy(), x["v"].double().numpy(),
                             x["dout"].double().numpy(), x["theta_row"].double().numpy(),
                             x["theta_col"].double().numpy(), M, s)
    got = [dqkv[:, :, :, i] for i in range(3)] + [dtr, dtc]
    for i, name in enumerate(("dQ", "dK", "dV", "dtheta_row", "dtheta_col")):
        mine = got[i].to("cpu", torch.float64).numpy()
        ref = g[i]
        err = np.abs(mine - ref).max()
        l2 = np.linalg.norm(mine - ref) / np.linalg.norm(ref)
        lim = 2e-2 * (np.abs(ref).max() if i >= 3 else 1.0)
        print(f"  {name}: max-abs {err:.3e} (tol {lim:.1e}) rel-L2 {l2:.3e}", flush=True)
        assert err <= lim and l2 <= 5e-3, name


def test_packed_autograd_matches_separate():
    case = (1, 32, 32, 2, 32, 8, 4, "bf16")
    B, Hg, Wg, H, D, M, s, dt = case
    x, qkv0 = packed_inputs(case, seed=14, with_dout=True)
    w = x["dout"].to(DEV)
    tr0, tc0 = x["theta_row"].to(DEV), x["theta_col"].to(DEV)
    qkv, tr, tc = qkv0.clone().requires_grad_(), tr0.clone().requires_grad_(), tc0.clone().requires_grad_()
    (F.window_attention_packed(qkv, tr, tc, M, s).float() * w.float()).sum().backward()
    q, k, v = (qkv0[:, :, :, i].contiguous().requires_grad_() for i in range(3))
    tr2, tc2 = tr0.clone().requires_grad_(), tc0.clone().requires_grad_()
    (F.window_attention(q, k, v, tr2, tc2, M, s).float() * w.float()).sum().backward()
    torch.cuda.synchronize()
    for i, t in enumerate((q, k, v)):
        assert torch.equal(qkv.grad[:, :, :, i], t.grad), i
    assert torch.equal(tr.grad, tr2.grad)
    assert torch.equal(tc.grad, tc2.grad)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_packed_with_summary_equals_separate(case):
    """The packed calls with the operand summary: the summary, out, LSE and the packed gradient are
    bit-identical to the separate-tensor calls with the summary on the slices (every case above has a
    grid that M divides)."""
    B, Hg, Wg, H, D, M, s, dt = case
    print("case", case, flush=True)
    x, qkv = packed_inputs(case, seed=21, with_dout=True)
    tr, tc, dout = x["theta_row"].to(DEV), x["theta_col"].to(DEV), x["dout"].to(DEV)
    q, k, v = (qkv[:, :, :, i].contiguous() for i in range(3))
    st_p, st_s = F.new_stats(q, M, s), F.new_stats(q, M, s)
    st_p.fill_(-1.0)
    st_s.fill_(-1.0)
    out_p, lse_p = F.wattn_fwd_packed(qkv, tr, tc, M, s, stats=st_p)
    out_s, lse_s = F.wattn_fwd(q, k, v, tr, tc, M, s, stats=st_s)
    dqkv, dtr_p, dtc_p = F.wattn_bwd_packed(qkv, out_p, dout, lse_p, tr, tc, M, s, stats=st_p)
    dq, dk, dv, dtr_s, dtc_s = F.wattn_bwd(q, k, v, out_s, dout, lse_s, tr, tc, M, s, stats=st_s)
    torch.cuda.synchronize()
    assert torch.equal(st_p, st_s)
    assert torch.equal(out_p, out_s) and torch.equal(lse_p, lse_s)
    for i, t in enumerate((dq, dk, dv)):
        assert torch.equal(dqkv[:, :, :, i], t), i
    assert torch.equal(dtr_p, dtr_s) and torch.equal(dtc_p, dtc_s)
