"""ctypes binding of libflashswin.so: argument marshalling only.

Every computation happens in the HIP kernels behind the C ABI declared in
include/flashswin.h.  This module only checks tensor properties torch knows
about (device, dtype, contiguity, shape), allocates outputs and the backward
workspace through torch's caching allocator, and passes raw device pointers and
the current HIP stream.  There is no CPU fallback: if the library is missing
or no GPU is present, calls raise.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflashswin.so")

FSW_OK, FSW_ERR_INVALID_ARG, FSW_ERR_UNSUPPORTED, FSW_ERR_WORKSPACE, FSW_ERR_HIP, FSW_ERR_SCRATCH = range(6)
SCRATCH_BYTES = 32 * 1024 * 1024  # FLASHSWIN_SCRATCH_BYTES of include/flashswin.h
MAX_RANK = 32  # FLASHSWIN_MAX_RANK of include/flashswin.h
FSW_F32, FSW_BF16 = 0, 1

EXPORTED = (
    "flashswin_wattn_fwd",
    "flashswin_wattn_bwd_workspace_size",
    "flashswin_wattn_bwd",
    "flashswin_wattn_fwd_packed",
    "flashswin_wattn_bwd_packed",
    "flashswin_wattn_bwd_noalloc",
    "flashswin_wattn_fwd_materialized_workspace_size",
    "flashswin_wattn_fwd_materialized",
    "flashswin_wattn_fwd_lowrank",
    "flashswin_wattn_bwd_lowrank_workspace_size",
    "flashswin_wattn_bwd_lowrank",
    "flashswin_wattn_stats_bytes",
    "flashswin_wattn_fwd_stats",
    "flashswin_wattn_bwd_stats",
    "flashswin_wattn_fwd_packed_stats",
    "flashswin_wattn_bwd_packed_stats",
    "flashswin_status_string",
    "flashswin_version",
)

_lib = None


class FlashSwinError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load():
    """Load the shared library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m vision_transformer_windowed_amd.build` "
            "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.flashswin_wattn_fwd.restype = i32
    lib.flashswin_wattn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, i32, i32, i32, vp]
    lib.flashswin_wattn_bwd_workspace_size.restype = sz
    lib.flashswin_wattn_bwd_workspace_size.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32]
    lib.flashswin_wattn_bwd.restype = i32
    lib.flashswin_wattn_bwd.argtypes = [vp] * 13 + [vp, sz, i64, i64, i64, i32, i32, i32, i32, i32, vp]
    lib.flashswin_wattn_fwd_packed.restype = i32
    lib.flashswin_wattn_fwd_packed.argtypes = [vp] * 5 + [i64, i64, i64, i32, i32, i32, i32, i32, vp]
    lib.flashswin_wattn_bwd_packed.restype = i32
    lib.flashswin_wattn_bwd_packed.argtypes = [vp] * 9 + [vp, sz, i64, i64, i64, i32, i32, i32, i32, i32, vp]
    lib.flashswin_wattn_bwd_noalloc.restype = i32
    lib.flashswin_wattn_bwd_noalloc.argtypes = [vp] * 13 + [i64, i64, i64, i32, i32, i32, i32, i32, vp]
    lib.flashswin_wattn_fwd_materialized_workspace_size.restype = sz
    lib.flashswin_wattn_fwd_materialized_workspace_size.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32]
    lib.flashswin_wattn_fwd_materialized.restype = i32
    lib.flashswin_wattn_fwd_materialized.argtypes = [vp] * 9 + [sz, i64, i64, i64, i32, i32, i32, i32, i32, vp]
    lib.flashswin_wattn_fwd_lowrank.restype = i32
    lib.flashswin_wattn_fwd_lowrank.argtypes = [vp] * 7 + [i32, vp, vp, i64, i64, i64, i32, i32, i32, i32, i32, vp]
    lib.flashswin_wattn_bwd_lowrank_workspace_size.restype = sz
    lib.flashswin_wattn_bwd_lowrank_workspace_size.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32, i32]
    lib.flashswin_wattn_bwd_lowrank.restype = i32
    lib.flashswin_wattn_bwd_lowrank.argtypes = ([vp] * 10 + [i32] + [vp] * 8 + [sz, i64, i64, i64, i32, i32, i32, i32, i32,
                                                                        vp])
    lib.flashswin_wattn_stats_bytes.restype = sz
    lib.flashswin_wattn_stats_bytes.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32]
    lib.flashswin_wattn_fwd_stats.restype = i32
    lib.flashswin_wattn_fwd_stats.argtypes = [vp] * 7 + [i32] + [vp] * 3 + [i64, i64, i64, i32, i32, i32, i32, i32, vp]
    lib.flashswin_wattn_bwd_stats.restype = i32
    lib.flashswin_wattn_bwd_stats.argtypes = ([vp] * 10 + [i32] + [vp] * 9 + [sz, i64, i64, i64, i32, i32, i32, i32,
                                                                          i32, vp])
    lib.flashswin_wattn_fwd_packed_stats.restype = i32
    lib.flashswin_wattn_fwd_packed_stats.argtypes = [vp] * 6 + [i64, i64, i64, i32, i32, i32, i32, i32, vp]
    lib.flashswin_wattn_bwd_packed_stats.restype = i32
    lib.flashswin_wattn_bwd_packed_stats.argtypes = [vp] * 10 + [vp, sz, i64, i64, i64, i32, i32, i32, i32, i32, vp]
    lib.flashswin_status_string.restype = ctypes.c_char_p
    lib.flashswin_status_string.argtypes = [i32]
    lib.flashswin_version.restype = i32
    lib.flashswin_version.argtypes = []
    _lib = lib
    return lib


def status_string(status):
    return load().flashswin_status_string(int(status)).decode()


# ------------------------------------------------------------------ raw C-ABI calls (same names)

def flashswin_wattn_fwd(q, k, v, theta_row, theta_col, out, lse, B, Hg, Wg, heads, d, M, shift, dtype, stream):
    """Raw call: pointers are ints (device addresses) or None; returns the status code."""
    return load().flashswin_wattn_fwd(q, k, v, theta_row, theta_col, out, lse, B, Hg, Wg, heads, d, M, shift,
                                      dtype, stream)


def flashswin_wattn_bwd_workspace_size(B, Hg, Wg, heads, d, M, shift, dtype):
    return load().flashswin_wattn_bwd_workspace_size(B, Hg, Wg, heads, d, M, shift, dtype)


def flashswin_wattn_bwd(q, k, v, out, dout, lse, theta_row, theta_col, dq, dk, dv, dtheta_row, dtheta_col,
                        workspace, workspace_bytes, B, Hg, Wg, heads, d, M, shift, dtype, stream):
    return load().flashswin_wattn_bwd(q, k, v, out, dout, lse, theta_row, theta_col, dq, dk, dv, dtheta_row,
                                      dtheta_col, workspace, workspace_bytes, B, Hg, Wg, heads, d, M, shift, dtype,
                                      stream)


def flashswin_wattn_fwd_packed(qkv, theta_row, theta_col, out, lse, B, Hg, Wg, heads, d, M, shift, dtype, stream):
    return load().flashswin_wattn_fwd_packed(qkv, theta_row, theta_col, out, lse, B, Hg, Wg, heads, d, M, shift,
                                             dtype, stream)


def flashswin_wattn_bwd_packed(qkv, out, dout, lse, theta_row, theta_col, dqkv, dtheta_row, dtheta_col, workspace,
                               workspace_bytes, B, Hg, Wg, heads, d, M, shift, dtype, stream):
    return load().flashswin_wattn_bwd_packed(qkv, out, dout, lse, theta_row, theta_col, dqkv, dtheta_row,
                                             dtheta_col, workspace, workspace_bytes, B, Hg, Wg, heads, d, M, shift,
                                             dtype, stream)


def flashswin_wattn_bwd_noalloc(q, k, v, out, dout, lse, theta_row, theta_col, dq, dk, dv, dtheta_row, dtheta_col,
                                B, Hg, Wg, heads, d, M, shift, dtype, stream):
    """Raw call of the backward that uses the library's fixed per-GPU scratch instead of a workspace."""
    return load().flashswin_wattn_bwd_noalloc(q, k, v, out, dout, lse, theta_row, theta_col, dq, dk, dv,
                                              dtheta_row, dtheta_col, B, Hg, Wg, heads, d, M, shift, dtype, stream)


def flashswin_wattn_fwd_materialized_workspace_size(B, Hg, Wg, heads, d, M, shift, dtype):
    return load().flashswin_wattn_fwd_materialized_workspace_size(B, Hg, Wg, heads, d, M, shift, dtype)


def flashswin_wattn_fwd_materialized(q, k, v, theta_row, theta_col, bias, out, lse, workspace, workspace_bytes, B,
                                     Hg, Wg, heads, d, M, shift, dtype, stream):
    """Raw call of the materialized comparison forward (scores in the caller's workspace)."""
    return load().flashswin_wattn_fwd_materialized(q, k, v, theta_row, theta_col, bias, out, lse, workspace,
                                                   workspace_bytes, B, Hg, Wg, heads, d, M, shift, dtype, stream)


def flashswin_wattn_fwd_lowrank(q, k, v, theta_row, theta_col, bias_u, bias_w, rank, out, lse, B, Hg, Wg, heads, d,
                                M, shift, dtype, stream):
    """Raw call of the forward with a rank-r additive bias U W^T on the scores."""
    return load().flashswin_wattn_fwd_lowrank(q, k, v, theta_row, theta_col, bias_u, bias_w, rank, out, lse, B, Hg,
                                              Wg, heads, d, M, shift, dtype, stream)


def flashswin_wattn_bwd_lowrank_workspace_size(B, Hg, Wg, heads, d, M, shift, dtype, rank):
    return load().flashswin_wattn_bwd_lowrank_workspace_size(B, Hg, Wg, heads, d, M, shift, dtype, rank)


def flashswin_wattn_bwd_lowrank(q, k, v, out, dout, lse, theta_row, theta_col, bias_u, bias_w, rank, dq, dk, dv,
                                dtheta_row, dtheta_col, dbias_u, dbias_w, workspace, workspace_bytes, B, Hg, Wg, heads,
                                d, M, shift, dtype, stream):
    return load().flashswin_wattn_bwd_lowrank(q, k, v, out, dout, lse, theta_row, theta_col, bias_u, bias_w, rank, dq,
                                              dk, dv, dtheta_row, dtheta_col, dbias_u, dbias_w, workspace,
                                              workspace_bytes, B, Hg, Wg, heads, d, M, shift, dtype, stream)


def flashswin_wattn_stats_bytes(B, Hg, Wg, heads, d, M, shift, dtype):
    return load().flashswin_wattn_stats_bytes(B, Hg, Wg, heads, d, M, shift, dtype)


def flashswin_wattn_fwd_stats(q, k, v, theta_row, theta_col, bias_u, bias_w, rank, out, lse, stats, B, Hg, Wg, heads,
                              d, M, shift, dtype, stream):
    """Raw call of the forward (rank 0: no bias) that also writes the operand summary for the backward."""
    return load().flashswin_wattn_fwd_stats(q, k, v, theta_row, theta_col, bias_u, bias_w, rank, out, lse, stats, B,
                                            Hg, Wg, heads, d, M, shift, dtype, stream)


def flashswin_wattn_bwd_stats(q, k, v, out, dout, lse, theta_row, theta_col, bias_u, bias_w, rank, stats, dq, dk, dv,
                              dtheta_row, dtheta_col, dbias_u, dbias_w, workspace, workspace_bytes, B, Hg, Wg, heads,
                              d, M, shift, dtype, stream):
    """Raw call of the backward that takes the forward's operand summary (its prologue reads only O, dO)."""
    return load().flashswin_wattn_bwd_stats(q, k, v, out, dout, lse, theta_row, theta_col, bias_u, bias_w, rank,
                                            stats, dq, dk, dv, dtheta_row, dtheta_col, dbias_u, dbias_w, workspace,
                                            workspace_bytes, B, Hg, Wg, heads, d, M, shift, dtype, stream)


def flashswin_wattn_fwd_packed_stats(qkv, theta_row, theta_col, out, lse, stats, B, Hg, Wg, heads, d, M, shift, dtype,
                                     stream):
    return load().flashswin_wattn_fwd_packed_stats(qkv, theta_row, theta_col, out, lse, stats, B, Hg, Wg, heads, d, M,
                                                   shift, dtype, stream)


def flashswin_wattn_bwd_packed_stats(qkv, out, dout, lse, theta_row, theta_col, stats, dqkv, dtheta_row, dtheta_col,
                                     workspace, workspace_bytes, B, Hg, Wg, heads, d, M, shift, dtype, stream):
    return load().flashswin_wattn_bwd_packed_stats(qkv, out, dout, lse, theta_row, theta_col, stats, dqkv, dtheta_row,
                                                   dtheta_col, workspace, workspace_bytes, B, Hg, Wg, heads, d, M,
                                                   shift, dtype, stream)


def flashswin_status_string(status):
    return status_string(status)


def new_stats(q, M, shift=0):
    """An uninitialised operand-summary tensor (float32) for wattn_fwd(..., stats=) of q's shape."""
    B, Hg, Wg, H, D = q.shape
    n = flashswin_wattn_stats_bytes(B, Hg, Wg, H, D, int(M), int(shift), _dtype_code(q)) // 4
    return torch.empty(max(n, 1), device=q.device, dtype=torch.float32)


def _check_stats(stats, q, M, shift):
    B, Hg, Wg, H, D = q.shape
    n = flashswin_wattn_stats_bytes(B, Hg, Wg, H, D, int(M), int(shift), _dtype_code(q)) // 4
    if not stats.is_cuda or stats.device != q.device or stats.dtype != torch.float32 or not stats.is_contiguous():
        raise ValueError(f"stats must be a contiguous float32 tensor on {q.device}")
    if stats.numel() < n:
        raise ValueError(f"stats holds {stats.numel()} floats, the shape needs {n}")


def bwd_workspace_bytes(q, M, shift=0):
    B, Hg, Wg, H, D = q.shape
    return flashswin_wattn_bwd_workspace_size(B, Hg, Wg, H, D, int(M), int(shift), _dtype_code(q))


def flashswin_version():
    return load().flashswin_version()


# ------------------------------------------------------------------ torch-tensor helpers

def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return FSW_BF16
    if t.dtype == torch.float32:
        return FSW_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _check_grid(name, t, shape, dtype, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device} (all tensors on one GPU)")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _workspace(workspace, nbytes, device):
    """The caller's workspace when it is a contiguous GPU tensor on `device` of at least `nbytes`
    bytes, else a fresh one; returns (tensor, its size in bytes)."""
    if workspace is not None:
        if not workspace.is_cuda or workspace.device != device or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous tensor on {device}")
        size = workspace.numel() * workspace.element_size()
        if size >= nbytes:
            return workspace, size
    ws = torch.empty(max(nbytes, 1), device=device, dtype=torch.uint8)
    return ws, ws.numel()


def wattn_fwd(q, k, v, theta_row, theta_col, M, shift=0, out=None, lse=None, need_lse=True, stats=None):
    """Forward window attention on the GPU.  Returns (out, lse); lse is None when need_lse=False.

    `stats` (from new_stats) is filled with the operand summary that wattn_bwd(..., stats=) takes.
    """
    if q.dim() != 5:
        raise ValueError("q must be [B, Hg, Wg, heads, d]")
    B, Hg, Wg, H, D = q.shape
    code = _dtype_code(q)
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_grid(name, t, q.shape, q.dtype, dev)
    for name, t in (("theta_row", theta_row), ("theta_col", theta_col)):
        _check_grid(name, t, (H, D // 4), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _check_grid("out", out, q.shape, q.dtype, dev)
    if need_lse:
        if lse is None:
            lse = torch.empty((B, Hg, Wg, H), device=dev, dtype=torch.float32)
        _check_grid("lse", lse, (B, Hg, Wg, H), torch.float32, dev)
    else:
        lse = None
    if stats is not None:
        _check_stats(stats, q, M, shift)
        with torch.cuda.device(dev):
            st = flashswin_wattn_fwd_stats(_ptr(q), _ptr(k), _ptr(v), _ptr(theta_row), _ptr(theta_col), None, None, 0,
                                           _ptr(out), _ptr(lse), _ptr(stats), B, Hg, Wg, H, D, int(M), int(shift),
                                           code, _stream(dev))
        if st != FSW_OK:
            raise FlashSwinError(st, "flashswin_wattn_fwd_stats")
        return out, lse
    with torch.cuda.device(dev):
        st = flashswin_wattn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(theta_row), _ptr(theta_col), _ptr(out),
                                 _ptr(lse), B, Hg, Wg, H, D, int(M), int(shift), code, _stream(dev))
    if st != FSW_OK:
        raise FlashSwinError(st, "flashswin_wattn_fwd")
    return out, lse


def wattn_fwd_materialized(q, k, v, theta_row, theta_col, M, shift=0, bias=None, out=None, lse=None,
                           workspace=None, need_lse=True):
    """The materialized comparison forward (scores in HBM, then softmax, then P.V; bf16, d = 32), with an
    optional relative-position bias [heads, 2M-1, 2M-1].  Returns (out, lse, workspace bytes used)."""
    B, Hg, Wg, H, D = q.shape
    code = _dtype_code(q)
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_grid(name, t, q.shape, q.dtype, dev)
    for name, t in (("theta_row", theta_row), ("theta_col", theta_col)):
        _check_grid(name, t, (H, D // 4), torch.float32, dev)
    if bias is not None:
        _check_grid("bias", bias, (H, 2 * int(M) - 1, 2 * int(M) - 1), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _check_grid("out", out, q.shape, q.dtype, dev)
    if need_lse:
        if lse is None:
            lse = torch.empty((B, Hg, Wg, H), device=dev, dtype=torch.float32)
        _check_grid("lse", lse, (B, Hg, Wg, H), torch.float32, dev)
    else:
        lse = None
    nbytes = flashswin_wattn_fwd_materialized_workspace_size(B, Hg, Wg, H, D, int(M), int(shift), code)
    workspace, wbytes = _workspace(workspace, nbytes, dev)
    with torch.cuda.device(dev):
        st = flashswin_wattn_fwd_materialized(_ptr(q), _ptr(k), _ptr(v), _ptr(theta_row), _ptr(theta_col),
                                              _ptr(bias), _ptr(out), _ptr(lse), _ptr(workspace), wbytes, B, Hg, Wg,
                                              H, D, int(M), int(shift), code, _stream(dev))
    if st != FSW_OK:
        raise FlashSwinError(st, "flashswin_wattn_fwd_materialized")
    return out, lse, nbytes


def wattn_bwd(q, k, v, out, dout, lse, theta_row, theta_col, M, shift=0, workspace=None, grads=None, stats=None):
    """Backward on the GPU.  Returns (dq, dk, dv, dtheta_row, dtheta_col).

    `grads` may hold preallocated (dq, dk, dv, dtheta_row, dtheta_col) to write into.  `stats`: the
    summary that wattn_fwd(..., stats=) wrote for these q, k, v (the prologue then reads only O, dO).
    """
    B, Hg, Wg, H, D = q.shape
    code = _dtype_code(q)
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _check_grid(name, t, q.shape, q.dtype, dev)
    _check_grid("lse", lse, (B, Hg, Wg, H), torch.float32, dev)
    for name, t in (("theta_row", theta_row), ("theta_col", theta_col)):
        _check_grid(name, t, (H, D // 4), torch.float32, dev)
    if grads is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        dtr = torch.empty_like(theta_row)
        dtc = torch.empty_like(theta_col)
    else:
        dq, dk, dv, dtr, dtc = grads
        for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
            _check_grid(name, t, q.shape, q.dtype, dev)
        for name, t in (("dtheta_row", dtr), ("dtheta_col", dtc)):
            _check_grid(name, t, (H, D // 4), torch.float32, dev)
    nbytes = flashswin_wattn_bwd_workspace_size(B, Hg, Wg, H, D, int(M), int(shift), code)
    workspace, wbytes = _workspace(workspace, nbytes, dev)
    if stats is not None:
        _check_stats(stats, q, M, shift)
        with torch.cuda.device(dev):
            st = flashswin_wattn_bwd_stats(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                                           _ptr(theta_row), _ptr(theta_col), None, None, 0, _ptr(stats), _ptr(dq),
                                           _ptr(dk), _ptr(dv), _ptr(dtr), _ptr(dtc), None, None, _ptr(workspace),
                                           wbytes, B, Hg, Wg, H, D, int(M), int(shift), code, _stream(dev))
        if st != FSW_OK:
            raise FlashSwinError(st, "flashswin_wattn_bwd_stats")
        return dq, dk, dv, dtr, dtc
    with torch.cuda.device(dev):
        st = flashswin_wattn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(theta_row),
                                 _ptr(theta_col), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dtr), _ptr(dtc),
                                 _ptr(workspace), wbytes, B, Hg, Wg, H, D, int(M), int(shift), code, _stream(dev))
    if st != FSW_OK:
        raise FlashSwinError(st, "flashswin_wattn_bwd")
    return dq, dk, dv, dtr, dtc


def _check_factors(bias_u, bias_w, H, M, dev):
    if bias_u.dim() != 3:
        raise ValueError("bias_u must be [heads, M*M, rank]")
    rank = bias_u.shape[2]
    for name, t in (("bias_u", bias_u), ("bias_w", bias_w)):
        _check_grid(name, t, (H, int(M) * int(M), rank), torch.float32, dev)
    return rank


def wattn_fwd_lowrank(q, k, v, theta_row, theta_col, bias_u, bias_w, M, shift=0, out=None, lse=None, need_lse=True,
                      stats=None):
    """Forward with a rank-r additive bias bias_u[n_i] . bias_w[n_j] on the scores (factors float32
    [heads, M*M, rank]).  Returns (out, lse).  `stats`: as in wattn_fwd."""
    B, Hg, Wg, H, D = q.shape
    code = _dtype_code(q)
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_grid(name, t, q.shape, q.dtype, dev)
    for name, t in (("theta_row", theta_row), ("theta_col", theta_col)):
        _check_grid(name, t, (H, D // 4), torch.float32, dev)
    rank = _check_factors(bias_u, bias_w, H, M, dev)
    if out is None:
        out = torch.empty_like(q)
    _check_grid("out", out, q.shape, q.dtype, dev)
    if need_lse:
        if lse is None:
            lse = torch.empty((B, Hg, Wg, H), device=dev, dtype=torch.float32)
        _check_grid("lse", lse, (B, Hg, Wg, H), torch.float32, dev)
    else:
        lse = None
    if stats is not None:
        _check_stats(stats, q, M, shift)
        with torch.cuda.device(dev):
            st = flashswin_wattn_fwd_stats(_ptr(q), _ptr(k), _ptr(v), _ptr(theta_row), _ptr(theta_col), _ptr(bias_u),
                                           _ptr(bias_w), rank, _ptr(out), _ptr(lse), _ptr(stats), B, Hg, Wg, H, D,
                                           int(M), int(shift), code, _stream(dev))
        if st != FSW_OK:
            raise FlashSwinError(st, "flashswin_wattn_fwd_stats")
        return out, lse
    with torch.cuda.device(dev):
        st = flashswin_wattn_fwd_lowrank(_ptr(q), _ptr(k), _ptr(v), _ptr(theta_row), _ptr(theta_col), _ptr(bias_u),
                                         _ptr(bias_w), rank, _ptr(out), _ptr(lse), B, Hg, Wg, H, D, int(M), int(shift),
                                         code, _stream(dev))
    if st != FSW_OK:
        raise FlashSwinError(st, "flashswin_wattn_fwd_lowrank")
    return out, lse


def wattn_bwd_lowrank(q, k, v, out, dout, lse, theta_row, theta_col, bias_u, bias_w, M, shift=0, workspace=None,
                      stats=None):
    """Backward of wattn_fwd_lowrank.  Returns (dq, dk, dv, dtheta_row, dtheta_col, dbias_u, dbias_w).
    `stats`: as in wattn_bwd."""
    B, Hg, Wg, H, D = q.shape
    code = _dtype_code(q)
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _check_grid(name, t, q.shape, q.dtype, dev)
    _check_grid("lse", lse, (B, Hg, Wg, H), torch.float32, dev)
    for name, t in (("theta_row", theta_row), ("theta_col", theta_col)):
        _check_grid(name, t, (H, D // 4), torch.float32, dev)
    rank = _check_factors(bias_u, bias_w, H, M, dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dtr, dtc = torch.empty_like(theta_row), torch.empty_like(theta_col)
    dbu, dbw = torch.empty_like(bias_u), torch.empty_like(bias_w)
    nbytes = flashswin_wattn_bwd_lowrank_workspace_size(B, Hg, Wg, H, D, int(M), int(shift), code, rank)
    workspace, wbytes = _workspace(workspace, nbytes, dev)
    if stats is not None:
        _check_stats(stats, q, M, shift)
        with torch.cuda.device(dev):
            st = flashswin_wattn_bwd_stats(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                                           _ptr(theta_row), _ptr(theta_col), _ptr(bias_u), _ptr(bias_w), rank,
                                           _ptr(stats), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dtr), _ptr(dtc), _ptr(dbu),
                                           _ptr(dbw), _ptr(workspace), wbytes, B, Hg, Wg, H, D, int(M), int(shift),
                                           code, _stream(dev))
        if st != FSW_OK:
            raise FlashSwinError(st, "flashswin_wattn_bwd_stats")
        return dq, dk, dv, dtr, dtc, dbu, dbw
    with torch.cuda.device(dev):
        st = flashswin_wattn_bwd_lowrank(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                                         _ptr(theta_row), _ptr(theta_col), _ptr(bias_u), _ptr(bias_w), rank, _ptr(dq),
                                         _ptr(dk), _ptr(dv), _ptr(dtr), _ptr(dtc), _ptr(dbu), _ptr(dbw),
                                         _ptr(workspace), wbytes, B, Hg, Wg, H, D, int(M), int(shift), code,
                                         _stream(dev))
    if st != FSW_OK:
        raise FlashSwinError(st, "flashswin_wattn_bwd_lowrank")
    return dq, dk, dv, dtr, dtc, dbu, dbw


def _packed_shape(qkv):
    if qkv.dim() != 6 or qkv.shape[3] != 3:
        raise ValueError("qkv must be [B, Hg, Wg, 3, heads, d]")
    B, Hg, Wg, _, H, D = qkv.shape
    return B, Hg, Wg, H, D


def wattn_fwd_packed(qkv, theta_row, theta_col, M, shift=0, out=None, lse=None, need_lse=True, stats=None):
    """Forward from packed qkv [B, Hg, Wg, 3, heads, d], read in place.  Returns (out, lse).  `stats`:
    as in wattn_fwd (new_stats of a q-shaped tensor, or of qkv[..., 0, :, :])."""
    B, Hg, Wg, H, D = _packed_shape(qkv)
    code = _dtype_code(qkv)
    dev = qkv.device
    _check_grid("qkv", qkv, qkv.shape, qkv.dtype, dev)
    for name, t in (("theta_row", theta_row), ("theta_col", theta_col)):
        _check_grid(name, t, (H, D // 4), torch.float32, dev)
    if out is None:
        out = torch.empty((B, Hg, Wg, H, D), device=dev, dtype=qkv.dtype)
    _check_grid("out", out, (B, Hg, Wg, H, D), qkv.dtype, dev)
    if need_lse:
        if lse is None:
            lse = torch.empty((B, Hg, Wg, H), device=dev, dtype=torch.float32)
        _check_grid("lse", lse, (B, Hg, Wg, H), torch.float32, dev)
    else:
        lse = None
    if stats is not None:
        _check_stats(stats, out, M, shift)
        with torch.cuda.device(dev):
            st = flashswin_wattn_fwd_packed_stats(_ptr(qkv), _ptr(theta_row), _ptr(theta_col), _ptr(out), _ptr(lse),
                                                  _ptr(stats), B, Hg, Wg, H, D, int(M), int(shift), code, _stream(dev))
        if st != FSW_OK:
            raise FlashSwinError(st, "flashswin_wattn_fwd_packed_stats")
        return out, lse
    with torch.cuda.device(dev):
        st = flashswin_wattn_fwd_packed(_ptr(qkv), _ptr(theta_row), _ptr(theta_col), _ptr(out), _ptr(lse), B, Hg,
                                        Wg, H, D, int(M), int(shift), code, _stream(dev))
    if st != FSW_OK:
        raise FlashSwinError(st, "flashswin_wattn_fwd_packed")
    return out, lse


def wattn_bwd_packed(qkv, out, dout, lse, theta_row, theta_col, M, shift=0, workspace=None, grads=None, stats=None):
    """Backward of wattn_fwd_packed.  Returns (dqkv, dtheta_row, dtheta_col), dqkv packed like qkv.

    `grads` may hold preallocated (dqkv, dtheta_row, dtheta_col) to write into.  `stats`: the summary
    wattn_fwd_packed(..., stats=) wrote for this qkv.
    """
    B, Hg, Wg, H, D = _packed_shape(qkv)
    code = _dtype_code(qkv)
    dev = qkv.device
    _check_grid("qkv", qkv, qkv.shape, qkv.dtype, dev)
    for name, t in (("out", out), ("dout", dout)):
        _check_grid(name, t, (B, Hg, Wg, H, D), qkv.dtype, dev)
    _check_grid("lse", lse, (B, Hg, Wg, H), torch.float32, dev)
    for name, t in (("theta_row", theta_row), ("theta_col", theta_col)):
        _check_grid(name, t, (H, D // 4), torch.float32, dev)
    if grads is None:
        dqkv, dtr, dtc = torch.empty_like(qkv), torch.empty_like(theta_row), torch.empty_like(theta_col)
    else:
        dqkv, dtr, dtc = grads
        _check_grid("dqkv", dqkv, qkv.shape, qkv.dtype, dev)
        for name, t in (("dtheta_row", dtr), ("dtheta_col", dtc)):
            _check_grid(name, t, (H, D // 4), torch.float32, dev)
    nbytes = flashswin_wattn_bwd_workspace_size(B, Hg, Wg, H, D, int(M), int(shift), code)
    workspace, wbytes = _workspace(workspace, nbytes, dev)
    if stats is not None:
        _check_stats(stats, out, M, shift)
        with torch.cuda.device(dev):
            st = flashswin_wattn_bwd_packed_stats(_ptr(qkv), _ptr(out), _ptr(dout), _ptr(lse), _ptr(theta_row),
                                                  _ptr(theta_col), _ptr(stats), _ptr(dqkv), _ptr(dtr), _ptr(dtc),
                                                  _ptr(workspace), wbytes, B, Hg, Wg, H, D, int(M), int(shift), code,
                                                  _stream(dev))
        if st != FSW_OK:
            raise FlashSwinError(st, "flashswin_wattn_bwd_packed_stats")
        return dqkv, dtr, dtc
    with torch.cuda.device(dev):
        st = flashswin_wattn_bwd_packed(_ptr(qkv), _ptr(out), _ptr(dout), _ptr(lse), _ptr(theta_row),
                                        _ptr(theta_col), _ptr(dqkv), _ptr(dtr), _ptr(dtc), _ptr(workspace), wbytes,
                                        B, Hg, Wg, H, D, int(M), int(shift), code, _stream(dev))
    if st != FSW_OK:
        raise FlashSwinError(st, "flashswin_wattn_bwd_packed")
    return dqkv, dtr, dtc


class WindowAttention(torch.autograd.Function):
    """Autograd wrapper: forward saves LSE, backward recomputes P (no score matrix is stored)."""

    @staticmethod
    def forward(ctx, q, k, v, theta_row, theta_col, M, shift):
        # the operand summary (16 bytes per window-head) spares the backward's prologue q, k and v
        stats = new_stats(q, M, shift)
        out, lse = wattn_fwd(q, k, v, theta_row, theta_col, M, shift, stats=stats)
        ctx.save_for_backward(q, k, v, out, lse, theta_row, theta_col, stats)
        ctx.M, ctx.shift = M, shift
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, lse, tr, tc, stats = ctx.saved_tensors
        dq, dk, dv, dtr, dtc = wattn_bwd(q, k, v, out, dout.contiguous(), lse, tr, tc, ctx.M, ctx.shift, stats=stats)
        return dq, dk, dv, dtr, dtc, None, None


def window_attention(q, k, v, theta_row, theta_col, M, shift=0):
    """Differentiable windowed attention with window-local 2D RoPE; q/k/v [B, Hg, Wg, heads, d]."""
    return WindowAttention.apply(q, k, v, theta_row, theta_col, M, shift)


class WindowAttentionPacked(torch.autograd.Function):
    """Autograd wrapper over packed qkv [B, Hg, Wg, 3, heads, d]; the gradient comes back packed."""

    @staticmethod
    def forward(ctx, qkv, theta_row, theta_col, M, shift):
        stats = new_stats(qkv[:, :, :, 0], M, shift)  # the operand summary, as in WindowAttention
        out, lse = wattn_fwd_packed(qkv, theta_row, theta_col, M, shift, stats=stats)
        ctx.save_for_backward(qkv, out, lse, theta_row, theta_col, stats)
        ctx.M, ctx.shift = M, shift
        return out

    @staticmethod
    def backward(ctx, dout):
        qkv, out, lse, tr, tc, stats = ctx.saved_tensors
        dqkv, dtr, dtc = wattn_bwd_packed(qkv, out, dout.contiguous(), lse, tr, tc, ctx.M, ctx.shift, stats=stats)
        return dqkv, dtr, dtc, None, None


def window_attention_packed(qkv, theta_row, theta_col, M, shift=0):
    """Differentiable windowed attention reading packed qkv [B, Hg, Wg, 3, heads, d] in place."""
    return WindowAttentionPacked.apply(qkv, theta_row, theta_col, M, shift)
