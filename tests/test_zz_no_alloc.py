"""The backward entry point that allocates nothing (flashswin_wattn_bwd_noalloc), called through the
C ABI: two calls in a row, the second on a smaller input, each bit-identical to flashswin_wattn_bwd
with a caller workspace (same kernels; only the workspace's address differs), which the other GPU
tests hold to the oracle.  Shapes whose workspace exceeds the fixed scratch are refused before any
HIP call."""

import pytest
import torch

import vision_transformer_windowed_amd as F
from vision_transformer_windowed_amd.inputs import make_inputs

DEV = "cuda:0"

# (B, Hg, Wg, heads, d, M, shift, dtype): the bf16 M = 32 MFMA kernels, then a smaller input on the
# M = 8 MFMA kernels, then float32 (the float32-arithmetic kernels), the d = 64 MFMA kernels, and a
# padded grid (the MFMA instances with padding checks)
CALLS = [(4, 64, 64, 3, 32, 32, 16, "bf16"), (1, 32, 32, 2, 32, 8, 3, "bf16"), (1, 16, 16, 2, 32, 8, 4, "f32"),
         (2, 32, 32, 2, 64, 16, 8, "bf16"), (1, 50, 38, 2, 32, 16, 8, "bf16")]


def _args(x, out, lse, grads):
    p = lambda t: t.data_ptr()  # noqa: E731
    return [p(x["q"]), p(x["k"]), p(x["v"]), p(out), p(x["dout"]), p(lse), p(x["theta_row"]), p(x["theta_col"])] + \
        [p(g) for g in grads]


def _one(case, seed):
    B, Hg, Wg, H, D, M, s, dt = case
    x = {n: t.to(DEV) for n, t in make_inputs(B, Hg, Wg, H, D, dt, seed=seed, with_dout=True).items()}
    out, lse = F.wattn_fwd(x["q"], x["k"], x["v"], x["theta_row"], x["theta_col"], M, s)
    code = F.FSW_BF16 if dt == "bf16" else F.FSW_F32
    stream = torch.cuda.current_stream(DEV).cuda_stream

    def grads():
        return [torch.full_like(x["q"], float("nan")) for _ in range(3)] + \
            [torch.full_like(x["theta_row"], float("nan")) for _ in range(2)]

    mine = grads()
    st = F.flashswin_wattn_bwd_noalloc(*_args(x, out, lse, mine), B, Hg, Wg, H, D, M, s, code, stream)
    assert st == F.FSW_OK, F.flashswin_status_string(st)
    ref = grads()
    nbytes = F.flashswin_wattn_bwd_workspace_size(B, Hg, Wg, H, D, M, s, code)
    assert 0 < nbytes <= F.SCRATCH_BYTES
    ws = torch.empty(nbytes, device=DEV, dtype=torch.uint8)
    st = F.flashswin_wattn_bwd(*_args(x, out, lse, ref), ws.data_ptr(), nbytes, B, Hg, Wg, H, D, M, s, code, stream)
    assert st == F.FSW_OK, F.flashswin_status_string(st)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv", "dtheta_row", "dtheta_col"), mine, ref):
        assert not torch.isnan(a).any(), name
        assert torch.equal(a, b), name


@pytest.mark.gpu
def test_noalloc_backward_matches_workspace_backward_on_consecutive_calls():
    for i, case in enumerate(CALLS):
        print(f"  call {i}: {case}", flush=True)
        _one(case, seed=500 + i)


def test_noalloc_refuses_shapes_beyond_the_scratch():
    """200 images of 128 x 128 tokens, 3 heads, bf16, M = 32 need a 41.9 MB workspace: refused with
    FSW_ERR_SCRATCH before any HIP call (the pointers are never dereferenced)."""
    fake = 1 << 20
    B, Hg, Wg, H, D, M, s, code = 200, 128, 128, 3, 32, 32, 0, F.FSW_BF16
    assert F.flashswin_wattn_bwd_workspace_size(B, Hg, Wg, H, D, M, s, code) > F.SCRATCH_BYTES
    ptrs = [fake + i * (1 << 34) for i in range(13)]
    assert F.flashswin_wattn_bwd_noalloc(*ptrs, B, Hg, Wg, H, D, M, s, code, None) == F.FSW_ERR_SCRATCH
    assert "FSW_ERR_SCRATCH" in F.flashswin_status_string(F.FSW_ERR_SCRATCH)
