"""C-ABI checks that need no GPU: the library loads, exports every declared symbol, and rejects
invalid arguments with the documented status before any HIP call is made."""

import os
import re

import pytest

import vision_transformer_windowed_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashswin.h")

pytestmark = pytest.mark.skipif(not os.path.exists(F.LIB_PATH), reason="libflashswin.so not built")

FAKE = 1 << 20  # a 256-byte aligned, non-null address never dereferenced (validation fails first)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flashswin_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = F.load()
    names = declared_functions()
    assert set(names) == set(F.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert F.flashswin_version() >= 102
    for code in range(5):
        assert F.flashswin_status_string(code).startswith("FSW_")
    assert "unknown" in F.flashswin_status_string(99)


GIB = 1 << 30  # buffers of the fixtures below sit 1 GiB apart, so none overlaps another


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, tr=FAKE + 3 * GIB, tc=FAKE + 3 * GIB + 256, out=FAKE + GIB, lse=FAKE + 2 * GIB,
             B=1, Hg=16, Wg=16, heads=2, d=32, M=8, shift=0, dtype=F.FSW_BF16)
    a.update(kw)
    return F.flashswin_wattn_fwd(a["q"], a["k"], a["v"], a["tr"], a["tc"], a["out"], a["lse"], a["B"], a["Hg"],
                                 a["Wg"], a["heads"], a["d"], a["M"], a["shift"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(Hg=0), F.FSW_ERR_INVALID_ARG),           # empty grid side
    (dict(Wg=-3), F.FSW_ERR_INVALID_ARG),
    (dict(shift=8), F.FSW_ERR_INVALID_ARG),        # shift >= M
    (dict(shift=-1), F.FSW_ERR_INVALID_ARG),       # negative shift
    (dict(d=6), F.FSW_ERR_INVALID_ARG),            # d not a multiple of 4
    (dict(d=12), F.FSW_ERR_UNSUPPORTED),           # valid d without a kernel
    (dict(d=128), F.FSW_ERR_UNSUPPORTED),
    (dict(Hg=256, Wg=256, M=256), F.FSW_ERR_UNSUPPORTED),  # windows beyond 128 x 128
    (dict(heads=0), F.FSW_ERR_INVALID_ARG),
    (dict(B=-1), F.FSW_ERR_INVALID_ARG),
    (dict(M=0), F.FSW_ERR_INVALID_ARG),
    (dict(dtype=7), F.FSW_ERR_INVALID_ARG),
    (dict(q=None), F.FSW_ERR_INVALID_ARG),
    (dict(tr=None), F.FSW_ERR_INVALID_ARG),
    (dict(out=None), F.FSW_ERR_INVALID_ARG),
    (dict(q=FAKE + 2), F.FSW_ERR_INVALID_ARG),     # misaligned
    (dict(out=FAKE + 8), F.FSW_ERR_INVALID_ARG),
    (dict(tc=FAKE + 2), F.FSW_ERR_INVALID_ARG),
    (dict(lse=FAKE + 1), F.FSW_ERR_INVALID_ARG),
    (dict(out=FAKE), F.FSW_ERR_INVALID_ARG),       # out aliases q
    (dict(out=FAKE + 4096), F.FSW_ERR_INVALID_ARG),  # out overlaps the tail of q (32 KiB)
    (dict(lse=FAKE + GIB + 1024), F.FSW_ERR_INVALID_ARG),  # lse inside out
    (dict(tr=FAKE + GIB + 64), F.FSW_ERR_INVALID_ARG),  # theta inside out
    (dict(B=1 << 40), F.FSW_ERR_UNSUPPORTED),      # index space overflow
])
def test_forward_rejects_before_launch(kw, status):
    assert fwd(**kw) == status


def test_forward_empty_batch_is_a_no_op():
    assert fwd(B=0, q=None, k=None, v=None, out=None, lse=None, tr=None, tc=None) == F.FSW_OK


def bwd(**kw):
    a = dict(q=FAKE, k=FAKE + GIB, v=FAKE + 2 * GIB, out=FAKE + 3 * GIB, dout=FAKE + 4 * GIB,
             lse=FAKE + 5 * GIB, tr=FAKE + 6 * GIB, tc=FAKE + 6 * GIB + 256, dq=FAKE + 7 * GIB,
             dk=FAKE + 8 * GIB, dv=FAKE + 9 * GIB, dtr=FAKE + 10 * GIB, dtc=FAKE + 10 * GIB + 256,
             ws=FAKE + 11 * GIB, wsb=None,
             B=1, Hg=16, Wg=16, heads=2, d=32, M=8, shift=4, dtype=F.FSW_BF16)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = F.flashswin_wattn_bwd_workspace_size(a["B"], a["Hg"], a["Wg"], a["heads"], a["d"], a["M"],
                                                        a["shift"], a["dtype"])
    return F.flashswin_wattn_bwd(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["tr"], a["tc"], a["dq"],
                                 a["dk"], a["dv"], a["dtr"], a["dtc"], a["ws"], a["wsb"], a["B"], a["Hg"], a["Wg"],
                                 a["heads"], a["d"], a["M"], a["shift"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(Hg=0), F.FSW_ERR_INVALID_ARG),
    (dict(shift=9), F.FSW_ERR_INVALID_ARG),
    (dict(lse=None), F.FSW_ERR_INVALID_ARG),       # the backward needs the forward's LSE
    (dict(dout=None), F.FSW_ERR_INVALID_ARG),
    (dict(dtr=None), F.FSW_ERR_INVALID_ARG),
    (dict(dq=FAKE + 4), F.FSW_ERR_INVALID_ARG),
    (dict(dk=FAKE), F.FSW_ERR_INVALID_ARG),        # dk aliases q
    (dict(dv=FAKE + 8 * GIB), F.FSW_ERR_INVALID_ARG),  # dv aliases dk
    (dict(dv=FAKE + 8 * GIB + 4096), F.FSW_ERR_INVALID_ARG),  # dv overlaps the tail of dk
    (dict(dq=FAKE + 3 * GIB + 16384), F.FSW_ERR_INVALID_ARG),  # dq overlaps out
    (dict(dtc=FAKE + 10 * GIB), F.FSW_ERR_INVALID_ARG),  # dtheta_col aliases dtheta_row
    (dict(dtr=FAKE + 5 * GIB + 256), F.FSW_ERR_INVALID_ARG),  # dtheta_row inside lse
    (dict(ws=FAKE + 4 * GIB), F.FSW_ERR_INVALID_ARG),  # workspace over dout
    (dict(ws=None), F.FSW_ERR_WORKSPACE),
    (dict(ws=FAKE + 11 * GIB + 4), F.FSW_ERR_WORKSPACE),  # misaligned workspace
    (dict(wsb=16), F.FSW_ERR_WORKSPACE),           # too small
    (dict(d=12), F.FSW_ERR_UNSUPPORTED),
])
def test_backward_rejects_before_launch(kw, status):
    assert bwd(**kw) == status


def test_workspace_size():
    ws = F.flashswin_wattn_bwd_workspace_size
    assert ws(0, 16, 16, 2, 32, 8, 0, 1) == 0
    assert ws(1, 0, 16, 2, 32, 8, 0, 1) == 0            # invalid shape
    small = ws(1, 16, 16, 2, 32, 8, 0, 1)
    big = ws(4, 16, 16, 2, 32, 8, 0, 1)
    assert 0 < small < big
    assert small % 256 == 0
    # at least the per-token Delta buffer
    assert ws(32, 128, 128, 3, 32, 32, 16, 1) >= 32 * 128 * 128 * 3 * 4


# ----------------------------------------------------------------------- packed qkv entry points
# Shape 1 x 16 x 16 tokens, 2 heads, d 32, bf16: one tensor of q's shape is 32 KiB, packed qkv 96 KiB.
TENS = 16 * 16 * 2 * 32 * 2


def fwd_packed(**kw):
    a = dict(qkv=FAKE, tr=FAKE + 4 * TENS, tc=FAKE + 4 * TENS + 256, out=FAKE + 3 * TENS,
             lse=FAKE + 4 * TENS + 512, B=1, Hg=16, Wg=16, heads=2, d=32, M=8, shift=0, dtype=F.FSW_BF16)
    a.update(kw)
    return F.flashswin_wattn_fwd_packed(a["qkv"], a["tr"], a["tc"], a["out"], a["lse"], a["B"], a["Hg"], a["Wg"],
                                        a["heads"], a["d"], a["M"], a["shift"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(Wg=0), F.FSW_ERR_INVALID_ARG),
    (dict(qkv=None), F.FSW_ERR_INVALID_ARG),
    (dict(qkv=FAKE + 8), F.FSW_ERR_INVALID_ARG),            # misaligned
    (dict(out=None), F.FSW_ERR_INVALID_ARG),
    (dict(out=FAKE + TENS), F.FSW_ERR_INVALID_ARG),         # out is the k slice
    (dict(out=FAKE + 3 * TENS - 4096), F.FSW_ERR_INVALID_ARG),  # out overlaps the tail of qkv
    (dict(d=12), F.FSW_ERR_UNSUPPORTED),
    (dict(B=1 << 38), F.FSW_ERR_UNSUPPORTED),               # 3x the elements of q overflow the index space
])
def test_packed_forward_rejects_before_launch(kw, status):
    assert fwd_packed(**kw) == status


def test_packed_forward_empty_batch_is_a_no_op():
    assert fwd_packed(B=0, qkv=None, out=None, lse=None, tr=None, tc=None) == F.FSW_OK


def bwd_packed(**kw):
    base = FAKE + 16 * TENS
    a = dict(qkv=FAKE, out=base, dout=base + TENS, lse=base + 2 * TENS, tr=base + 2 * TENS + 4096,
             tc=base + 2 * TENS + 4352, dqkv=FAKE + 4 * TENS, dtr=base + 2 * TENS + 4608,
             dtc=base + 2 * TENS + 4864, ws=base + 4 * TENS, wsb=None,
             B=1, Hg=16, Wg=16, heads=2, d=32, M=8, shift=4, dtype=F.FSW_BF16)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = F.flashswin_wattn_bwd_workspace_size(a["B"], a["Hg"], a["Wg"], a["heads"], a["d"], a["M"],
                                                        a["shift"], a["dtype"])
    return F.flashswin_wattn_bwd_packed(a["qkv"], a["out"], a["dout"], a["lse"], a["tr"], a["tc"], a["dqkv"],
                                        a["dtr"], a["dtc"], a["ws"], a["wsb"], a["B"], a["Hg"], a["Wg"],
                                        a["heads"], a["d"], a["M"], a["shift"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(qkv=None), F.FSW_ERR_INVALID_ARG),
    (dict(dqkv=None), F.FSW_ERR_INVALID_ARG),
    (dict(lse=None), F.FSW_ERR_INVALID_ARG),
    (dict(dqkv=FAKE + 2 * TENS), F.FSW_ERR_INVALID_ARG),    # dqkv overlaps qkv
    (dict(out=FAKE + 5 * TENS), F.FSW_ERR_INVALID_ARG),     # out inside dqkv
    (dict(dout=FAKE + 6 * TENS - 64), F.FSW_ERR_INVALID_ARG),  # dout overlaps the end of dqkv
    (dict(dqkv=FAKE + 4 * TENS + 2), F.FSW_ERR_INVALID_ARG),  # misaligned
    (dict(ws=None), F.FSW_ERR_WORKSPACE),
    (dict(wsb=16), F.FSW_ERR_WORKSPACE),
    (dict(shift=8), F.FSW_ERR_INVALID_ARG),
])
def test_packed_backward_rejects_before_launch(kw, status):
    assert bwd_packed(**kw) == status


def mat(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, tr=FAKE + 3 * GIB, tc=FAKE + 3 * GIB + 256, bias=None, out=FAKE + GIB,
             lse=FAKE + 2 * GIB, ws=FAKE + 4 * GIB, wsb=1 << 30, B=1, Hg=16, Wg=16, heads=2, d=32, M=8, shift=0,
             dtype=F.FSW_BF16)
    a.update(kw)
    return F.flashswin_wattn_fwd_materialized(a["q"], a["k"], a["v"], a["tr"], a["tc"], a["bias"], a["out"], a["lse"],
                                              a["ws"], a["wsb"], a["B"], a["Hg"], a["Wg"], a["heads"], a["d"], a["M"],
                                              a["shift"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=F.FSW_F32), F.FSW_ERR_UNSUPPORTED),   # bf16 only
    (dict(d=16), F.FSW_ERR_UNSUPPORTED),              # d = 32 only
    (dict(Hg=64, Wg=64, M=64), F.FSW_ERR_UNSUPPORTED),  # M <= 32 only
    (dict(Hg=12), F.FSW_ERR_UNSUPPORTED),             # padded grids: the fused kernels only
    (dict(Hg=0), F.FSW_ERR_INVALID_ARG),
    (dict(wsb=1024), F.FSW_ERR_WORKSPACE),            # too small
    (dict(ws=None), F.FSW_ERR_WORKSPACE),
    (dict(ws=FAKE + 4 * GIB + 16), F.FSW_ERR_WORKSPACE),  # not 256-byte aligned
    (dict(bias=FAKE + 5 * GIB + 2), F.FSW_ERR_INVALID_ARG),  # misaligned bias
    (dict(bias=FAKE + GIB), F.FSW_ERR_INVALID_ARG),   # bias inside out
    (dict(ws=FAKE), F.FSW_ERR_INVALID_ARG),           # workspace over the inputs
    (dict(q=None), F.FSW_ERR_INVALID_ARG),
])
def test_materialized_rejects_before_launch(kw, status):
    assert mat(**kw) == status


def test_materialized_workspace_size():
    # 16 x 16 grid, M = 8: 4 windows x 2 heads x 64 rows x 64 floats
    assert F.flashswin_wattn_fwd_materialized_workspace_size(1, 16, 16, 2, 32, 8, 0, F.FSW_BF16) == 4 * 2 * 64 * 64 * 4
    # M = 5: N = 25 rows of 32 floats
    assert F.flashswin_wattn_fwd_materialized_workspace_size(1, 10, 10, 1, 32, 5, 2, F.FSW_BF16) == 4 * 25 * 32 * 4
    assert F.flashswin_wattn_fwd_materialized_workspace_size(1, 16, 16, 2, 32, 8, 0, F.FSW_F32) == 0
    assert F.flashswin_wattn_fwd_materialized_workspace_size(1, 12, 16, 2, 32, 8, 0, F.FSW_BF16) == 0  # padded


def test_padded_grid_workspace_counts_padded_windows():
    """A 10 x 13 grid with M = 4 is padded to 12 x 16: 3 x 4 windows.  The backward workspace holds
    Delta for the 130 grid tokens, per-window-head maxima and the float32-arithmetic kernels' dtheta
    partial rows (one row per kernel, window-head and 128-query block), 256-byte aligned sections."""
    def al(n):
        return (n + 255) // 256 * 256
    B, Hg, Wg, H, d, M = 2, 10, 13, 3, 32, 4
    nwin = B * 3 * 4
    want = al(B * Hg * Wg * H * 4) + al(nwin * H * 4 * 4) + al(H * 2 * nwin * 1 * (d // 2) * 4)
    for dt in (F.FSW_BF16, F.FSW_F32):
        assert F.flashswin_wattn_bwd_workspace_size(B, Hg, Wg, H, d, M, 1, dt) == want


# ----------------------------------------------------------------------- low-rank bias entry points
# Shape 1 x 16 x 16 tokens, 2 heads, d 32, M 8: factors [2, 64, rank] float32.

def fwd_lr(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, tr=FAKE + 3 * GIB, tc=FAKE + 3 * GIB + 256, bu=FAKE + 4 * GIB,
             bw=FAKE + 5 * GIB, rank=4, out=FAKE + GIB, lse=FAKE + 2 * GIB, B=1, Hg=16, Wg=16, heads=2, d=32, M=8,
             shift=0, dtype=F.FSW_BF16)
    a.update(kw)
    return F.flashswin_wattn_fwd_lowrank(a["q"], a["k"], a["v"], a["tr"], a["tc"], a["bu"], a["bw"], a["rank"],
                                         a["out"], a["lse"], a["B"], a["Hg"], a["Wg"], a["heads"], a["d"], a["M"],
                                         a["shift"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(rank=0), F.FSW_ERR_INVALID_ARG),
    (dict(rank=-2), F.FSW_ERR_INVALID_ARG),
    (dict(rank=F.MAX_RANK + 1), F.FSW_ERR_UNSUPPORTED),
    (dict(bu=None), F.FSW_ERR_INVALID_ARG),
    (dict(bw=None), F.FSW_ERR_INVALID_ARG),
    (dict(bu=FAKE + 4 * GIB + 2), F.FSW_ERR_INVALID_ARG),  # misaligned factor
    (dict(out=FAKE + 4 * GIB), F.FSW_ERR_INVALID_ARG),     # out over the U factor
    (dict(lse=FAKE + 5 * GIB + 64), F.FSW_ERR_INVALID_ARG),  # lse inside the W factor (2 x 64 x 4 floats)
    (dict(shift=8), F.FSW_ERR_INVALID_ARG),
    (dict(d=12), F.FSW_ERR_UNSUPPORTED),
])
def test_lowrank_forward_rejects_before_launch(kw, status):
    assert fwd_lr(**kw) == status


def test_lowrank_forward_empty_batch_is_a_no_op():
    assert fwd_lr(B=0, q=None, k=None, v=None, out=None, lse=None, tr=None, tc=None) == F.FSW_OK


def test_lowrank_workspace_adds_the_per_window_factor_gradients():
    """float32 kernels: their plain workspace plus two [windows][heads][N][rank] float blocks.  bf16 MFMA
    kernels (d = 32, windows of at most 256 tokens): Delta, the four maxima per window-head, one dtheta
    row of d/2 floats per window-head and side, then the same two blocks, up to 64 floats of alignment,
    both factors zero-padded to 32 channels and two factor maxima per head."""
    def al(n):
        return (n + 255) // 256 * 256
    nwin, heads, N, r = 4, 2, 64, 5
    lr = 2 * nwin * heads * N * r * 4
    base = F.flashswin_wattn_bwd_workspace_size(1, 16, 16, 2, 32, 8, 4, F.FSW_F32)  # the float32-arithmetic layout
    assert F.flashswin_wattn_bwd_lowrank_workspace_size(1, 16, 16, 2, 32, 8, 4, F.FSW_F32, r) == base + al(lr)
    nwh = nwin * heads
    extra = (64 + 2 * heads * N * F.MAX_RANK + 2 * heads) * 4
    mfma = al(16 * 16 * heads * 4) + al(nwh * 4 * 4) + al(2 * nwh * 16 * 4) + al(lr + extra)
    assert F.flashswin_wattn_bwd_lowrank_workspace_size(1, 16, 16, 2, 32, 8, 4, F.FSW_BF16, r) == mfma
    assert F.flashswin_wattn_bwd_lowrank_workspace_size(1, 16, 16, 2, 32, 8, 4, F.FSW_BF16, 0) == 0
    assert F.flashswin_wattn_bwd_lowrank_workspace_size(1, 16, 16, 2, 32, 8, 4, F.FSW_BF16, F.MAX_RANK + 1) == 0


def bwd_lr(**kw):
    a = dict(q=FAKE, k=FAKE + GIB, v=FAKE + 2 * GIB, out=FAKE + 3 * GIB, dout=FAKE + 4 * GIB,
             lse=FAKE + 5 * GIB, tr=FAKE + 6 * GIB, tc=FAKE + 6 * GIB + 256, bu=FAKE + 12 * GIB, bw=FAKE + 13 * GIB,
             rank=3, dq=FAKE + 7 * GIB, dk=FAKE + 8 * GIB, dv=FAKE + 9 * GIB, dtr=FAKE + 10 * GIB,
             dtc=FAKE + 10 * GIB + 256, dbu=FAKE + 14 * GIB, dbw=FAKE + 15 * GIB, ws=FAKE + 11 * GIB, wsb=None,
             B=1, Hg=16, Wg=16, heads=2, d=32, M=8, shift=4, dtype=F.FSW_BF16)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = F.flashswin_wattn_bwd_lowrank_workspace_size(a["B"], a["Hg"], a["Wg"], a["heads"], a["d"], a["M"],
                                                                a["shift"], a["dtype"], max(a["rank"], 1))
    return F.flashswin_wattn_bwd_lowrank(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["tr"], a["tc"],
                                         a["bu"], a["bw"], a["rank"], a["dq"], a["dk"], a["dv"], a["dtr"], a["dtc"],
                                         a["dbu"], a["dbw"], a["ws"], a["wsb"], a["B"], a["Hg"], a["Wg"], a["heads"],
                                         a["d"], a["M"], a["shift"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(rank=0), F.FSW_ERR_INVALID_ARG),
    (dict(rank=F.MAX_RANK + 1), F.FSW_ERR_UNSUPPORTED),
    (dict(dbu=None), F.FSW_ERR_INVALID_ARG),
    (dict(dbw=FAKE + 15 * GIB + 1), F.FSW_ERR_INVALID_ARG),  # misaligned
    (dict(dbu=FAKE + 12 * GIB), F.FSW_ERR_INVALID_ARG),      # dU over U
    (dict(dbw=FAKE + 14 * GIB + 128), F.FSW_ERR_INVALID_ARG),  # dW inside dU (2 x 64 x 3 floats)
    (dict(dbu=FAKE + 11 * GIB + 512), F.FSW_ERR_INVALID_ARG),  # dU inside the workspace
    (dict(wsb=1024), F.FSW_ERR_WORKSPACE),
    (dict(lse=None), F.FSW_ERR_INVALID_ARG),
])
def test_lowrank_backward_rejects_before_launch(kw, status):
    assert bwd_lr(**kw) == status


# ------------------------------------------------------------------ forward operand summary entry points
# Shape 1 x 16 x 16 tokens, 2 heads, d 32, M 8: 4 windows x 2 heads x 4 floats of summary.

def test_stats_bytes():
    assert F.flashswin_wattn_stats_bytes(1, 16, 16, 2, 32, 8, 0, F.FSW_BF16) == 4 * 2 * 16
    assert F.flashswin_wattn_stats_bytes(3, 10, 13, 5, 64, 4, 1, F.FSW_BF16) == 3 * 3 * 4 * 5 * 16  # padded grid
    assert F.flashswin_wattn_stats_bytes(1, 16, 16, 2, 32, 8, 8, F.FSW_BF16) == 0  # shift >= M: rejected


def fwd_st(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, tr=FAKE + 3 * GIB, tc=FAKE + 3 * GIB + 256, bu=None, bw=None, rank=0,
             out=FAKE + GIB, lse=FAKE + 2 * GIB, st=FAKE + 6 * GIB, B=1, Hg=16, Wg=16, heads=2, d=32, M=8, shift=0,
             dtype=F.FSW_BF16)
    a.update(kw)
    return F.flashswin_wattn_fwd_stats(a["q"], a["k"], a["v"], a["tr"], a["tc"], a["bu"], a["bw"], a["rank"],
                                       a["out"], a["lse"], a["st"], a["B"], a["Hg"], a["Wg"], a["heads"], a["d"],
                                       a["M"], a["shift"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(st=None), F.FSW_ERR_INVALID_ARG),
    (dict(st=FAKE + 6 * GIB + 2), F.FSW_ERR_INVALID_ARG),    # misaligned
    (dict(st=FAKE + GIB + 64), F.FSW_ERR_INVALID_ARG),       # inside out
    (dict(st=FAKE + 3 * GIB + 8), F.FSW_ERR_INVALID_ARG),    # over theta_row
    (dict(rank=-1), F.FSW_ERR_INVALID_ARG),
    (dict(rank=2), F.FSW_ERR_INVALID_ARG),                   # a bias rank without factors
    (dict(rank=F.MAX_RANK + 1, bu=FAKE + 4 * GIB, bw=FAKE + 5 * GIB), F.FSW_ERR_UNSUPPORTED),
    (dict(rank=2, bu=FAKE + 4 * GIB, bw=FAKE + 5 * GIB, st=FAKE + 5 * GIB + 16), F.FSW_ERR_INVALID_ARG),  # in W
    (dict(shift=8), F.FSW_ERR_INVALID_ARG),
    (dict(d=12), F.FSW_ERR_UNSUPPORTED),
])
def test_stats_forward_rejects_before_launch(kw, status):
    assert fwd_st(**kw) == status


def test_stats_forward_empty_batch_is_a_no_op():
    assert fwd_st(B=0, q=None, k=None, v=None, out=None, lse=None, tr=None, tc=None, st=None) == F.FSW_OK


def bwd_st(**kw):
    a = dict(q=FAKE, k=FAKE + GIB, v=FAKE + 2 * GIB, out=FAKE + 3 * GIB, dout=FAKE + 4 * GIB,
             lse=FAKE + 5 * GIB, tr=FAKE + 6 * GIB, tc=FAKE + 6 * GIB + 256, bu=None, bw=None, rank=0,
             st=FAKE + 16 * GIB, dq=FAKE + 7 * GIB, dk=FAKE + 8 * GIB, dv=FAKE + 9 * GIB, dtr=FAKE + 10 * GIB,
             dtc=FAKE + 10 * GIB + 256, dbu=None, dbw=None, ws=FAKE + 11 * GIB, wsb=None,
             B=1, Hg=16, Wg=16, heads=2, d=32, M=8, shift=4, dtype=F.FSW_BF16)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = (F.flashswin_wattn_bwd_lowrank_workspace_size(a["B"], a["Hg"], a["Wg"], a["heads"], a["d"],
                                                                 a["M"], a["shift"], a["dtype"], a["rank"])
                    if a["rank"] > 0 else
                    F.flashswin_wattn_bwd_workspace_size(a["B"], a["Hg"], a["Wg"], a["heads"], a["d"], a["M"],
                                                         a["shift"], a["dtype"]))
    return F.flashswin_wattn_bwd_stats(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["tr"], a["tc"],
                                       a["bu"], a["bw"], a["rank"], a["st"], a["dq"], a["dk"], a["dv"], a["dtr"],
                                       a["dtc"], a["dbu"], a["dbw"], a["ws"], a["wsb"], a["B"], a["Hg"], a["Wg"],
                                       a["heads"], a["d"], a["M"], a["shift"], a["dtype"], None)


LR = dict(rank=3, bu=FAKE + 12 * GIB, bw=FAKE + 13 * GIB, dbu=FAKE + 14 * GIB, dbw=FAKE + 15 * GIB)


@pytest.mark.parametrize("kw,status", [
    (dict(st=None), F.FSW_ERR_INVALID_ARG),
    (dict(st=FAKE + 16 * GIB + 1), F.FSW_ERR_INVALID_ARG),  # misaligned
    (dict(st=FAKE + 7 * GIB + 32), F.FSW_ERR_INVALID_ARG),  # inside dq
    (dict(st=FAKE + 11 * GIB + 512), F.FSW_ERR_INVALID_ARG),  # inside the workspace
    (dict(wsb=1024), F.FSW_ERR_WORKSPACE),
    (dict(lse=None), F.FSW_ERR_INVALID_ARG),
    (dict(LR, dbu=None), F.FSW_ERR_INVALID_ARG),
    (dict(LR, bw=None), F.FSW_ERR_INVALID_ARG),
    (dict(LR, dbw=FAKE + 14 * GIB + 128), F.FSW_ERR_INVALID_ARG),  # dW inside dU
    (dict(LR, st=FAKE + 15 * GIB + 64), F.FSW_ERR_INVALID_ARG),   # dW over the summary
    (dict(rank=F.MAX_RANK + 1, bu=FAKE + 12 * GIB, bw=FAKE + 13 * GIB), F.FSW_ERR_UNSUPPORTED),
])
def test_stats_backward_rejects_before_launch(kw, status):
    assert bwd_st(**kw) == status


def test_stats_backward_empty_batch_is_a_no_op():
    assert bwd_st(B=0, wsb=0, q=None, k=None, v=None, out=None, dout=None, lse=None, st=None) == F.FSW_OK


def fwd_pst(**kw):
    a = dict(qkv=FAKE, tr=FAKE + 4 * GIB, tc=FAKE + 4 * GIB + 256, out=FAKE + GIB, lse=FAKE + 2 * GIB,
             st=FAKE + 6 * GIB, B=1, Hg=16, Wg=16, heads=2, d=32, M=8, shift=0, dtype=F.FSW_BF16)
    a.update(kw)
    return F.flashswin_wattn_fwd_packed_stats(a["qkv"], a["tr"], a["tc"], a["out"], a["lse"], a["st"], a["B"],
                                              a["Hg"], a["Wg"], a["heads"], a["d"], a["M"], a["shift"], a["dtype"],
                                              None)


@pytest.mark.parametrize("kw,status", [
    (dict(st=None), F.FSW_ERR_INVALID_ARG),
    (dict(st=FAKE + 6 * GIB + 2), F.FSW_ERR_INVALID_ARG),  # misaligned
    (dict(st=FAKE + 64), F.FSW_ERR_INVALID_ARG),           # inside qkv
    (dict(st=FAKE + 2 * GIB + 16), F.FSW_ERR_INVALID_ARG),  # inside lse
    (dict(shift=8), F.FSW_ERR_INVALID_ARG),
])
def test_packed_stats_forward_rejects_before_launch(kw, status):
    assert fwd_pst(**kw) == status


def bwd_pst(**kw):
    a = dict(qkv=FAKE, out=FAKE + 3 * GIB, dout=FAKE + 4 * GIB, lse=FAKE + 5 * GIB, tr=FAKE + 6 * GIB,
             tc=FAKE + 6 * GIB + 256, st=FAKE + 16 * GIB, dqkv=FAKE + 7 * GIB, dtr=FAKE + 10 * GIB,
             dtc=FAKE + 10 * GIB + 256, ws=FAKE + 11 * GIB, wsb=None, B=1, Hg=16, Wg=16, heads=2, d=32, M=8,
             shift=4, dtype=F.FSW_BF16)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = F.flashswin_wattn_bwd_workspace_size(a["B"], a["Hg"], a["Wg"], a["heads"], a["d"], a["M"],
                                                         a["shift"], a["dtype"])
    return F.flashswin_wattn_bwd_packed_stats(a["qkv"], a["out"], a["dout"], a["lse"], a["tr"], a["tc"], a["st"],
                                              a["dqkv"], a["dtr"], a["dtc"], a["ws"], a["wsb"], a["B"], a["Hg"],
                                              a["Wg"], a["heads"], a["d"], a["M"], a["shift"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(st=None), F.FSW_ERR_INVALID_ARG),
    (dict(st=FAKE + 16 * GIB + 1), F.FSW_ERR_INVALID_ARG),   # misaligned
    (dict(st=FAKE + 7 * GIB + 32), F.FSW_ERR_INVALID_ARG),   # inside dqkv
    (dict(st=FAKE + 11 * GIB + 512), F.FSW_ERR_INVALID_ARG),  # inside the workspace
    (dict(wsb=1024), F.FSW_ERR_WORKSPACE),
])
def test_packed_stats_backward_rejects_before_launch(kw, status):
    assert bwd_pst(**kw) == status


def test_packed_stats_empty_batch_is_a_no_op():
    assert fwd_pst(B=0, qkv=None, out=None, lse=None, tr=None, tc=None, st=None) == F.FSW_OK
    assert bwd_pst(B=0, wsb=0, qkv=None, out=None, dout=None, lse=None, st=None, dqkv=None) == F.FSW_OK
