"""GPU parity of the materialized comparison path (flashswin_wattn_fwd_materialized: scores in HBM,
softmax, P.V) against the fp64 oracle, with and without a relative-position bias table.

Tolerances are the bf16 ones of test_parity_gpu.py: max-abs <= 2e-2 and relative L2 <= 5e-3 for O and
LSE.  The bias tables are N(0, 1); the oracle adds bias[h, r_i - r_j + M - 1, c_i - c_j + M - 1]."""

import numpy as np
import pytest
import torch

import oracle
import vision_transformer_windowed_amd as F
from vision_transformer_windowed_amd.inputs import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _close(name, got, ref, max_abs=2e-2, rel=5e-3):
    err = np.abs(got - ref).max()
    l2 = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    print(f"  {name}: max-abs {err:.3e} rel-L2 {l2:.3e}", flush=True)
    assert np.all(np.isfinite(got)), name
    assert err <= max_abs and l2 <= rel, name


CASES = [
    # B, Hg, Wg, heads, M, shift, with bias
    (2, 32, 32, 3, 8, 0, False),
    (1, 24, 16, 2, 8, 3, True),
    (1, 24, 24, 2, 12, 5, True),
    (1, 32, 48, 2, 16, 8, False),
    (1, 64, 64, 2, 32, 16, True),
    (1, 64, 32, 1, 32, 0, True),
    (1, 10, 10, 2, 5, 2, True),
    (1, 14, 14, 1, 7, 0, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_{}x{}_h{}_M{}_s{}_bias{}".format(*c))
def test_materialized_matches_oracle(case):
    B, Hg, Wg, H, M, s, with_bias = case
    x = make_inputs(B, Hg, Wg, H, 32, "bf16", seed=700 + M + s)
    bias = None
    if with_bias:
        bias = torch.from_numpy(np.random.default_rng(M).standard_normal((H, 2 * M - 1, 2 * M - 1))).float()
    xd = {n: t.to(DEV) for n, t in x.items()}
    out, lse, nbytes = F.wattn_fwd_materialized(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], M, s,
                                                bias=None if bias is None else bias.to(DEV))
    torch.cuda.synchronize()
    N = M * M
    assert nbytes == B * (Hg // M) * (Wg // M) * H * N * ((N + 31) // 32 * 32) * 4
    ro, rl = oracle.wattn_fwd_ref(*(x[n].double().numpy() for n in ("q", "k", "v")), x["theta_row"].double().numpy(),
                                  x["theta_col"].double().numpy(), M, s,
                                  bias=None if bias is None else bias.double().numpy())
    _close("O", _np(out), ro)
    _close("LSE", _np(lse), rl)


@pytest.mark.parametrize("name,imgs", [("swin_t_s1_p4_m8", [0, 127]), ("flashswin_t_s1_p2_m32", [0, 127])])
def test_materialized_workload(name, imgs):
    """Full-size workloads (M = 8: 0.4 GB of scores; M = 32: 25.8 GB), sampled images against the oracle,
    and the whole output against the fused forward within twice the bf16 tolerance."""
    w = WORKLOADS[name]
    x = workload_inputs(name, with_dout=False)
    xd = {n: t.to(DEV) for n, t in x.items()}
    out, lse, nbytes = F.wattn_fwd_materialized(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], w["M"],
                                                0)
    fo, fl = F.wattn_fwd(xd["q"], xd["k"], xd["v"], xd["theta_row"], xd["theta_col"], w["M"], 0)
    torch.cuda.synchronize()
    print(f"  workspace {nbytes / 1e9:.2f} GB", flush=True)
    ro, rl = oracle.wattn_fwd_ref(*(x[n][imgs].double().numpy() for n in ("q", "k", "v")),
                                  x["theta_row"].double().numpy(), x["theta_col"].double().numpy(), w["M"], 0)
    _close("O", _np(out[imgs]), ro)
    _close("LSE", _np(lse[imgs]), rl)
    d = (out.float() - fo.float()).abs().max().item()
    dl = (lse - fl).abs().max().item()
    print(f"  materialized vs fused: O max-abs {d:.3e}, LSE max-abs {dl:.3e}", flush=True)
    assert d <= 4e-2 and dl <= 4e-2
