"""ctypes binding of liblce.so (the C ABI in include/lce.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  If the library is missing this module raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# The in-tree build (lm_head_projection_amd/build.py); no other library is loaded.
LIB_PATH = os.path.join(PKG, "liblce.so")

LCE_DTYPE_F32 = 0
LCE_DTYPE_BF16 = 1

LCE_OK = 0
LCE_OK_EMPTY = 1
LCE_ERR_ARG = -1
LCE_ERR_LABEL = -2
LCE_ERR_WORKSPACE = -3
LCE_ERR_HIP = -4
LCE_ERR_UNSUPPORTED = -5
LCE_ERR_SCRATCH = -6

LCE_REDUCTION_MEAN = 0
LCE_REDUCTION_SUM = 1
LCE_REDUCTION_NONE = 2
LCE_FILTER_DH = 1
LCE_FILTER_BOTH = 3
REDUCTIONS = {"mean": LCE_REDUCTION_MEAN, "sum": LCE_REDUCTION_SUM, "none": LCE_REDUCTION_NONE}

# Every entry point that include/lce.h declares.
EXPORTS = (
    "lce_workspace_size",
    "lce_forward_workspace_size",
    "lce_backward_workspace_size",
    "lce_compact_valid",
    "lce_forward",
    "lce_backward",
    "lce_forward_ex",
    "lce_forward_ex_noalloc",
    "lce_backward_ex",
    "lce_backward_filtered",
    "lce_forward_shard",
    "lce_merge_shards",
    "lce_backward_shard",
    "lce_status_string",
    "lce_profile_start",
    "lce_profile_stop",
    "lce_profile_count",
    "lce_profile_entry",
)

_lib = None


class LCEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def load() -> ctypes.CDLL:
    """Loads liblce.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m lm_head_projection_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    lib.lce_workspace_size.argtypes = [i64, i64, i64, ctypes.c_int]
    lib.lce_workspace_size.restype = sz
    lib.lce_forward_workspace_size.argtypes = [i64, i64, i64, ctypes.c_int]
    lib.lce_forward_workspace_size.restype = sz
    lib.lce_backward_workspace_size.argtypes = [i64, i64, i64, i64, ctypes.c_int]
    lib.lce_backward_workspace_size.restype = sz
    lib.lce_compact_valid.argtypes = [vp, vp, i64, i64, i64, vp, ctypes.POINTER(i64), vp, sz, vp]
    lib.lce_compact_valid.restype = ctypes.c_int
    lib.lce_forward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                vp, vp, vp, vp, vp, sz, vp]
    lib.lce_forward.restype = ctypes.c_int
    lib.lce_backward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                 vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.lce_backward.restype = ctypes.c_int
    dbl = ctypes.c_double
    lib.lce_forward_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                   ctypes.c_int, vp, dbl, vp, vp, vp, vp, sz, vp]
    lib.lce_forward_ex.restype = ctypes.c_int
    lib.lce_forward_ex_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                           ctypes.c_int, vp, dbl, vp, vp, vp, vp]
    lib.lce_forward_ex_noalloc.restype = ctypes.c_int
    lib.lce_backward_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int,
                                    ctypes.c_int, vp, dbl, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.lce_backward_ex.restype = ctypes.c_int
    lib.lce_backward_filtered.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, vp,
                                          dbl, vp, vp, vp, ctypes.c_float, i32, vp, vp, vp, vp, sz, vp]
    lib.lce_backward_filtered.restype = ctypes.c_int
    lib.lce_forward_shard.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int, vp, vp, sz, vp]
    lib.lce_forward_shard.restype = ctypes.c_int
    lib.lce_merge_shards.argtypes = [vp, i32, ctypes.POINTER(i64), vp, vp, i64, i64, ctypes.c_int, vp, dbl, vp, vp,
                                     vp, vp, sz, vp]
    lib.lce_merge_shards.restype = ctypes.c_int
    lib.lce_backward_shard.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int, ctypes.c_int, vp,
                                       dbl, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.lce_backward_shard.restype = ctypes.c_int
    lib.lce_status_string.argtypes = [ctypes.c_int]
    lib.lce_status_string.restype = ctypes.c_char_p
    lib.lce_profile_start.argtypes = [i32]
    lib.lce_profile_start.restype = ctypes.c_int
    lib.lce_profile_stop.argtypes = []
    lib.lce_profile_stop.restype = ctypes.c_int
    lib.lce_profile_count.argtypes = []
    lib.lce_profile_count.restype = i32
    lib.lce_profile_entry.argtypes = [i32, ctypes.c_char_p, i32, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_double)]
    lib.lce_profile_entry.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().lce_status_string(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def dtype_code(dtype) -> int:
    import torch
    if dtype == torch.bfloat16:
        return LCE_DTYPE_BF16
    if dtype == torch.float32:
        return LCE_DTYPE_F32
    raise TypeError(f"unsupported dtype {dtype} (bf16 or fp32)")


def lce_workspace_size(N: int, D: int, V: int, dtype) -> int:
    return int(load().lce_workspace_size(N, D, V, dtype_code(dtype)))


def lce_forward_workspace_size(N: int, D: int, V: int, dtype) -> int:
    return int(load().lce_forward_workspace_size(N, D, V, dtype_code(dtype)))


def lce_backward_workspace_size(N: int, C: int, D: int, V: int, dtype) -> int:
    return int(load().lce_backward_workspace_size(N, C, D, V, dtype_code(dtype)))


def lce_compact_valid(labels, mask, V: int, ignore_index: int, valid_idx, ws, stream=None):
    """Returns (status, C).  labels int64[N], mask uint8[N] or None, valid_idx int32[N]."""
    C = ctypes.c_int64(0)
    st = load().lce_compact_valid(_ptr(labels), _ptr(mask), labels.numel(), V, ignore_index,
                                  _ptr(valid_idx), ctypes.byref(C), _ptr(ws), ws.numel(),
                                  _stream_ptr(stream))
    return st, int(C.value)


def lce_forward(H, W, b, labels, valid_idx, C: int, loss, m, logs, row_loss, ws, stream=None) -> int:
    N, D = H.shape
    V = W.shape[0]
    return load().lce_forward(_ptr(H), _ptr(W), _ptr(b), _ptr(labels), _ptr(valid_idx), C, N, D, V,
                              dtype_code(H.dtype), _ptr(loss), _ptr(m), _ptr(logs), _ptr(row_loss),
                              _ptr(ws), ws.numel(), _stream_ptr(stream))


def lce_backward(H, W, b, labels, valid_idx, C: int, m, logs, grad_loss, dH, dW, db, ws,
                 stream=None) -> int:
    N, D = H.shape
    V = W.shape[0]
    return load().lce_backward(_ptr(H), _ptr(W), _ptr(b), _ptr(labels), _ptr(valid_idx), C, N, D, V,
                               dtype_code(H.dtype), _ptr(m), _ptr(logs), _ptr(grad_loss), _ptr(dH),
                               _ptr(dW), _ptr(db), _ptr(ws), ws.numel(), _stream_ptr(stream))


def lce_forward_ex(H, W, b, labels, valid_idx, C: int, reduction: int, loss_weights,
                   num_label_tokens: float, loss, m, logs, ws, stream=None) -> int:
    N, D = H.shape
    V = W.shape[0]
    return load().lce_forward_ex(_ptr(H), _ptr(W), _ptr(b), _ptr(labels), _ptr(valid_idx), C, N, D, V,
                                 dtype_code(H.dtype), int(reduction), _ptr(loss_weights),
                                 float(num_label_tokens), _ptr(loss), _ptr(m), _ptr(logs), _ptr(ws),
                                 ws.numel(), _stream_ptr(stream))


def lce_forward_ex_noalloc(H, W, b, labels, valid_idx, C: int, reduction: int, loss_weights,
                           num_label_tokens: float, loss, m, logs, stream=None) -> int:
    N, D = H.shape
    V = W.shape[0]
    return load().lce_forward_ex_noalloc(_ptr(H), _ptr(W), _ptr(b), _ptr(labels), _ptr(valid_idx), C, N, D, V,
                                         dtype_code(H.dtype), int(reduction), _ptr(loss_weights),
                                         float(num_label_tokens), _ptr(loss), _ptr(m), _ptr(logs),
                                         _stream_ptr(stream))


def lce_backward_ex(H, W, b, labels, valid_idx, C: int, reduction: int, loss_weights,
                    num_label_tokens: float, m, logs, grad_loss, dH, dW, db, ws, stream=None) -> int:
    N, D = H.shape
    V = W.shape[0]
    return load().lce_backward_ex(_ptr(H), _ptr(W), _ptr(b), _ptr(labels), _ptr(valid_idx), C, N, D, V,
                                  dtype_code(H.dtype), int(reduction), _ptr(loss_weights),
                                  float(num_label_tokens), _ptr(m), _ptr(logs), _ptr(grad_loss), _ptr(dH),
                                  _ptr(dW), _ptr(db), _ptr(ws), ws.numel(), _stream_ptr(stream))


def lce_backward_filtered(H, W, b, labels, valid_idx, C: int, reduction: int, loss_weights, num_label_tokens: float,
                          m, logs, grad_loss, eps: float, dH, dW, db, ws, stream=None,
                          which: int = 3) -> int:
    """which: LCE_FILTER_DH (1: dH filtered, dW exact) or LCE_FILTER_BOTH (3)."""
    N, D = H.shape
    V = W.shape[0]
    return load().lce_backward_filtered(_ptr(H), _ptr(W), _ptr(b), _ptr(labels), _ptr(valid_idx), C, N, D, V,
                                        dtype_code(H.dtype), int(reduction), _ptr(loss_weights),
                                        float(num_label_tokens), _ptr(m), _ptr(logs), _ptr(grad_loss), float(eps),
                                        int(which), _ptr(dH), _ptr(dW), _ptr(db), _ptr(ws), ws.numel(),
                                        _stream_ptr(stream))


def lce_forward_shard(H, W_shard, b_shard, labels, valid_idx, C: int, v_begin: int, part, ws, stream=None) -> int:
    N, D = H.shape
    Vs = W_shard.shape[0]
    return load().lce_forward_shard(_ptr(H), _ptr(W_shard), _ptr(b_shard), _ptr(labels), _ptr(valid_idx), C, N, D,
                                    Vs, v_begin, dtype_code(H.dtype), _ptr(part), _ptr(ws), ws.numel(),
                                    _stream_ptr(stream))


def lce_merge_shards(parts, shard_begin, labels, valid_idx, C: int, reduction: int, loss_weights,
                     num_label_tokens: float, loss, m, logs, ws, stream=None) -> int:
    """parts: float32[P, 3*C] (device); shard_begin: P+1 ints (host)."""
    P = len(shard_begin) - 1
    arr = (ctypes.c_int64 * (P + 1))(*[int(x) for x in shard_begin])
    N = labels.numel()
    return load().lce_merge_shards(_ptr(parts), P, arr, _ptr(labels), _ptr(valid_idx), C, N, int(reduction),
                                   _ptr(loss_weights), float(num_label_tokens), _ptr(loss), _ptr(m), _ptr(logs),
                                   _ptr(ws), ws.numel(), _stream_ptr(stream))


def lce_backward_shard(H, W_shard, b_shard, labels, valid_idx, C: int, v_begin: int, reduction: int, loss_weights,
                       num_label_tokens: float, m, logs, grad_loss, dH_part, dW_shard, db_shard, ws,
                       stream=None) -> int:
    N, D = H.shape
    Vs = W_shard.shape[0]
    return load().lce_backward_shard(_ptr(H), _ptr(W_shard), _ptr(b_shard), _ptr(labels), _ptr(valid_idx), C, N, D,
                                     Vs, v_begin, dtype_code(H.dtype), int(reduction), _ptr(loss_weights),
                                     float(num_label_tokens), _ptr(m), _ptr(logs), _ptr(grad_loss), _ptr(dH_part),
                                     _ptr(dW_shard), _ptr(db_shard), _ptr(ws), ws.numel(), _stream_ptr(stream))


def profile_start(max_launches: int = 65536) -> None:
    st = load().lce_profile_start(max_launches)
    if st != LCE_OK:
        raise LCEError(st, "lce_profile_start")


def profile_stop() -> dict:
    """Stops recording; returns {kernel: (total_ms, launches, flops)}, flops
    being the launches' algorithmic floating-point operations (0 outside the
    GEMM kernels)."""
    lib = load()
    st = lib.lce_profile_stop()
    if st != LCE_OK:
        raise LCEError(st, "lce_profile_stop")
    out = {}
    buf = ctypes.create_string_buffer(128)
    for i in range(lib.lce_profile_count()):
        ms = ctypes.c_double(0)
        n = ctypes.c_int64(0)
        fl = ctypes.c_double(0)
        lib.lce_profile_entry(i, buf, 128, ctypes.byref(ms), ctypes.byref(n), ctypes.byref(fl))
        out[buf.value.decode()] = (ms.value, n.value, fl.value)
    return out
