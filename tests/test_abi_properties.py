"""Property tests of the C ABI's shape validation (CPU only: no argument set here reaches the device).

The model below restates the shape rules that include/flashswin.h documents for every entry point:
B >= 0, Hg, Wg >= 1, heads >= 1, 1 <= M, 0 <= shift < M, d a positive multiple of 4 and dtype
FSW_F32 or FSW_BF16 (else FSW_ERR_INVALID_ARG); d in {8, 16, 32, 64} and M <= 128 (else
FSW_ERR_UNSUPPORTED).  For random argument sets it checks that
  - every set the model rejects is rejected by the forward with the model's status, before any HIP
    call (the pointers are fake), and that the size queries return 0 for it;
  - every accepted set gets the documented operand-summary size, B * ceil(Hg/M) * ceil(Wg/M) * heads
    * 16 bytes, and a nonzero backward workspace unless B == 0;
  - B == 0 is a no-op that touches no pointer.
"""

import os

import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import vision_transformer_windowed_amd as F

pytestmark = pytest.mark.skipif(not os.path.exists(F.LIB_PATH), reason="libflashswin.so not built")

FAKE = 1 << 20
GIB = 1 << 30


def model_status(B, Hg, Wg, heads, d, M, shift, dtype):
    if B < 0 or Hg < 1 or Wg < 1 or heads < 1 or M < 1 or d < 1:
        return F.FSW_ERR_INVALID_ARG
    if shift < 0 or shift >= M or d % 4 != 0 or dtype not in (F.FSW_F32, F.FSW_BF16):
        return F.FSW_ERR_INVALID_ARG
    if d not in (8, 16, 32, 64) or M > 128:
        return F.FSW_ERR_UNSUPPORTED
    return F.FSW_OK


shapes = st.tuples(
    st.integers(-2, 3),                  # B
    st.integers(-1, 70),                 # Hg
    st.integers(-1, 70),                 # Wg
    st.integers(-1, 5),                  # heads
    st.sampled_from([-4, 0, 4, 6, 8, 12, 16, 24, 32, 48, 64, 128]),  # d
    st.integers(-1, 140),                # M
    st.integers(-2, 140),                # shift
    st.sampled_from([F.FSW_F32, F.FSW_BF16, 2, -1]),  # dtype
)


def fwd_fake(B, Hg, Wg, heads, d, M, shift, dtype):
    return F.flashswin_wattn_fwd(FAKE, FAKE, FAKE, FAKE + 3 * GIB, FAKE + 3 * GIB + 4096, FAKE + GIB,
                                 FAKE + 2 * GIB, B, Hg, Wg, heads, d, M, shift, dtype, None)


@settings(max_examples=400, deadline=None, derandomize=True)
@given(shapes)
def test_rejected_shapes_never_reach_the_device(shape):
    want = model_status(*shape)
    if want == F.FSW_OK:
        return
    assert fwd_fake(*shape) == want
    assert F.flashswin_wattn_stats_bytes(*shape) == 0
    assert F.flashswin_wattn_bwd_workspace_size(*shape) == 0


@st.composite
def valid_shapes(draw):
    M = draw(st.integers(1, 128))
    return (draw(st.integers(0, 3)), draw(st.integers(1, 300)), draw(st.integers(1, 300)), draw(st.integers(1, 8)),
            draw(st.sampled_from([8, 16, 32, 64])), M, draw(st.integers(0, M - 1)),
            draw(st.sampled_from([F.FSW_F32, F.FSW_BF16])))


@settings(max_examples=400, deadline=None, derandomize=True)
@given(valid_shapes())
def test_accepted_shapes_have_the_documented_sizes(shape):
    B, Hg, Wg, heads, d, M, shift, dtype = shape
    assert model_status(*shape) == F.FSW_OK
    nwin = B * (-(-Hg // M)) * (-(-Wg // M))
    assert F.flashswin_wattn_stats_bytes(*shape) == nwin * heads * 16
    ws = F.flashswin_wattn_bwd_workspace_size(*shape)
    assert (ws == 0) == (B == 0)
    if B > 0:  # at least Delta (one float per token and head) and the maxima (16 bytes per window-head)
        assert ws >= B * Hg * Wg * heads * 4 + nwin * heads * 16
        assert ws % 256 == 0
    else:
        assert F.flashswin_wattn_fwd(None, None, None, None, None, None, None, B, Hg, Wg, heads, d, M, shift, dtype,
                                     None) == F.FSW_OK
