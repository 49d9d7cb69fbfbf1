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
    assert F.flashswin_version() >= 100
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
    (dict(Hg=12), F.FSW_ERR_INVALID_ARG),          # Hg not a multiple of M
    (dict(Wg=20), F.FSW_ERR_INVALID_ARG),          # Wg not a multiple of M
    (dict(shift=8), F.FSW_ERR_INVALID_ARG),        # shift >= M
    (dict(shift=-1), F.FSW_ERR_INVALID_ARG),       # negative shift
    (dict(d=6), F.FSW_ERR_INVALID_ARG),            # d not a multiple of 4
    (dict(d=12), F.FSW_ERR_UNSUPPORTED),           # valid d without a kernel
    (dict(d=128), F.FSW_ERR_UNSUPPORTED),
    (dict(Hg=64, Wg=64, M=64), F.FSW_ERR_UNSUPPORTED),  # windows beyond 32 x 32
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
    (dict(Hg=10), F.FSW_ERR_INVALID_ARG),
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
    assert ws(1, 12, 16, 2, 32, 8, 0, 1) == 0           # invalid shape
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
    (dict(Hg=12), F.FSW_ERR_INVALID_ARG),
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
