"""ctypes binding of ``libbsa_bwd.so``: argument marshalling only.

Every function here has the name and the argument order of the C entry point
it wraps (``include/bsa_bwd.h``).  Tensors are torch tensors (or None for a
null pointer); torch supplies device memory and the stream, nothing else.  All
arithmetic happens in the library's HIP kernels; if the library is missing the
functions raise instead of computing anything another way.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
# BSA_LIBRARY may name another build of the same library (same ABI)
LIB_PATH = os.environ.get("BSA_LIBRARY") or os.path.join(PKG, "libbsa_bwd.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "bsa_bwd.h")

BSA_OK = 0
BSA_ERR_PARAM_NULLPTR = 161001
BSA_ERR_PARAM_INVALID = 161002
BSA_ERR_RUNTIME = 361001
BSA_ERR_INNER = 561002

BSA_DTYPE_F16 = 1
BSA_DTYPE_BF16 = 2
BSA_DTYPE_F32 = 3
BSA_DTYPE_BOOL = 4
BSA_DTYPE_FP8_E4M3FN = 5
BSA_DTYPE_FP8_E5M2 = 6

NO_WINDOW = 2147483647
WS_REGIONS = ("seq", "delta", "lse2", "row_cnt", "row_list", "col_cnt", "col_list", "plan", "partial",
              "amask", "stage", "dq_acc", "total")
# dq_mode of bsa_bwd_ex
BSA_DQ_RECOMPUTE = 0
BSA_DQ_ATOMIC = 1


class bsa_tensor(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * 4),
        ("stride", ctypes.c_int64 * 4),
    ]


class BsaError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code
        self.message = message


_PT = ctypes.POINTER(bsa_tensor)
_PI64 = ctypes.POINTER(ctypes.c_int64)
_COMMON = [_PT] * 8 + [
    _PI64, ctypes.c_int64,           # block_shape
    _PI64, ctypes.c_int64,           # actual_seq_lengths
    _PI64, ctypes.c_int64,           # actual_seq_lengths_kv
    ctypes.c_char_p, ctypes.c_char_p,  # layouts
    ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_int64, ctypes.c_int64,
    _PT, _PT, _PT,
]

# forward: query, key, value, mask, atten_mask, ... (the common scalars) ..., attention_out, softmax_lse
_FWD = [_PT] * 5 + _COMMON[8:-3] + [_PT, _PT]

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it first (python -m block_sparse_attention_bwd_amd.build)")
    lib = ctypes.CDLL(path)
    lib.bsa_bwd_workspace_size.argtypes = _COMMON + [ctypes.POINTER(ctypes.c_uint64)]
    lib.bsa_bwd_workspace_size.restype = ctypes.c_int
    lib.bsa_bwd.argtypes = _COMMON + [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
    lib.bsa_bwd.restype = ctypes.c_int
    lib.bsa_bwd_workspace_layout.argtypes = _COMMON + [ctypes.POINTER(ctypes.c_uint64), _PI64]
    lib.bsa_bwd_workspace_layout.restype = ctypes.c_int
    lib.bsa_bwd_noalloc.argtypes = _COMMON + [ctypes.c_void_p]
    lib.bsa_bwd_noalloc.restype = ctypes.c_int
    lib.bsa_bwd_ex_workspace_size.argtypes = _COMMON + [ctypes.c_int32, ctypes.POINTER(ctypes.c_uint64)]
    lib.bsa_bwd_ex_workspace_size.restype = ctypes.c_int
    lib.bsa_bwd_ex.argtypes = _COMMON + [ctypes.c_int32, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
    lib.bsa_bwd_ex.restype = ctypes.c_int
    lib.bsa_fwd_workspace_size.argtypes = _FWD + [ctypes.POINTER(ctypes.c_uint64)]
    lib.bsa_fwd_workspace_size.restype = ctypes.c_int
    lib.bsa_fwd.argtypes = _FWD + [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
    lib.bsa_fwd.restype = ctypes.c_int
    _pd = ctypes.POINTER(ctypes.c_double)
    lib.bsa_bwd_fp8_workspace_size.argtypes = _COMMON + [_pd, ctypes.POINTER(ctypes.c_uint64)]
    lib.bsa_bwd_fp8_workspace_size.restype = ctypes.c_int
    lib.bsa_bwd_fp8.argtypes = _COMMON + [_pd, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
    lib.bsa_bwd_fp8.restype = ctypes.c_int
    lib.bsa_fwd_fp8_workspace_size.argtypes = _FWD + [_pd, ctypes.POINTER(ctypes.c_uint64)]
    lib.bsa_fwd_fp8_workspace_size.restype = ctypes.c_int
    lib.bsa_fwd_fp8.argtypes = _FWD + [_pd, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
    lib.bsa_fwd_fp8.restype = ctypes.c_int
    lib.bsa_last_error.argtypes = []
    lib.bsa_last_error.restype = ctypes.c_char_p
    lib.bsa_profile_start.argtypes = [ctypes.c_int32]
    lib.bsa_profile_start.restype = ctypes.c_int
    lib.bsa_profile_stop.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.c_int32,
                                     ctypes.POINTER(ctypes.c_int32)]
    lib.bsa_profile_stop.restype = ctypes.c_int
    lib.bsa_stage_name.argtypes = [ctypes.c_int32]
    lib.bsa_stage_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


def header_functions(path: str = HEADER) -> list:
    """Names of the functions ``include/bsa_bwd.h`` declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(bsa_\w+)\s*\(", text, flags=re.M)))


def _dtype_code(t) -> int:
    import torch
    return {
        torch.float16: BSA_DTYPE_F16,
        torch.bfloat16: BSA_DTYPE_BF16,
        torch.float32: BSA_DTYPE_F32,
        torch.bool: BSA_DTYPE_BOOL,
        torch.uint8: BSA_DTYPE_BOOL,
        torch.float8_e4m3fn: BSA_DTYPE_FP8_E4M3FN,
        torch.float8_e5m2: BSA_DTYPE_FP8_E5M2,
    }.get(t.dtype, 0)


def _desc(t):
    if t is None:
        return None
    if isinstance(t, bsa_tensor):
        return ctypes.pointer(t)
    if t.dim() > 4:
        raise ValueError("tensors have at most 4 dimensions")
    d = bsa_tensor()
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = _dtype_code(t)
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return ctypes.pointer(d)


def _i64_array(xs):
    if xs is None:
        return None, 0
    xs = [int(x) for x in xs]
    arr = (ctypes.c_int64 * max(1, len(xs)))(*xs)
    return arr, len(xs)


def _marshal(dout, query, key, value, attention_out, softmax_lse, block_sparse_mask, atten_mask,
             block_shape, actual_seq_lengths, actual_seq_lengths_kv, q_input_layout, kv_input_layout,
             num_key_value_heads, mask_type, scale_value, pre_tokens, next_tokens, dq, dk, dv):
    bs, bs_n = _i64_array(block_shape)
    aq, aq_n = _i64_array(actual_seq_lengths)
    ak, ak_n = _i64_array(actual_seq_lengths_kv)
    enc = lambda s: None if s is None else s.encode()
    return [
        _desc(dout), _desc(query), _desc(key), _desc(value), _desc(attention_out), _desc(softmax_lse),
        _desc(block_sparse_mask), _desc(atten_mask),
        bs, bs_n, aq, aq_n, ak, ak_n, enc(q_input_layout), enc(kv_input_layout),
        int(num_key_value_heads), int(mask_type), float(scale_value), int(pre_tokens), int(next_tokens),
        _desc(dq), _desc(dk), _desc(dv),
    ]


def _marshal_fwd(query, key, value, block_sparse_mask, atten_mask, block_shape, actual_seq_lengths,
                 actual_seq_lengths_kv, q_input_layout, kv_input_layout, num_key_value_heads, mask_type,
                 scale_value, pre_tokens, next_tokens, attention_out, softmax_lse):
    a = _marshal(None, query, key, value, attention_out, softmax_lse, block_sparse_mask, atten_mask,
                 block_shape, actual_seq_lengths, actual_seq_lengths_kv, q_input_layout, kv_input_layout,
                 num_key_value_heads, mask_type, scale_value, pre_tokens, next_tokens, None, None, None)
    # reorder to the forward's argument list
    return [a[1], a[2], a[3], a[6], a[7]] + a[8:21] + [a[4], a[5]]


def _check(rc: int):
    if rc != BSA_OK:
        msg = load_library().bsa_last_error()
        raise BsaError(rc, msg.decode() if msg else "")


def bsa_bwd_workspace_size(dout, query, key, value, attention_out, softmax_lse, block_sparse_mask=None,
                           atten_mask=None, block_shape=None, actual_seq_lengths=None,
                           actual_seq_lengths_kv=None, q_input_layout="BNSD", kv_input_layout="BNSD",
                           num_key_value_heads=1, mask_type=0, scale_value=1.0, pre_tokens=NO_WINDOW,
                           next_tokens=NO_WINDOW, dq=None, dk=None, dv=None) -> int:
    """Phase 1: validate and return the workspace size in bytes (host only)."""
    lib = load_library()
    args = _marshal(dout, query, key, value, attention_out, softmax_lse, block_sparse_mask, atten_mask,
                    block_shape, actual_seq_lengths, actual_seq_lengths_kv, q_input_layout,
                    kv_input_layout, num_key_value_heads, mask_type, scale_value, pre_tokens,
                    next_tokens, dq, dk, dv)
    size = ctypes.c_uint64(0)
    _check(lib.bsa_bwd_workspace_size(*args, ctypes.byref(size)))
    return size.value


def bsa_bwd_workspace_layout(dout, query, key, value, attention_out, softmax_lse, block_sparse_mask=None,
                             atten_mask=None, block_shape=None, actual_seq_lengths=None,
                             actual_seq_lengths_kv=None, q_input_layout="BNSD", kv_input_layout="BNSD",
                             num_key_value_heads=1, mask_type=0, scale_value=1.0, pre_tokens=NO_WINDOW,
                             next_tokens=NO_WINDOW, dq=None, dk=None, dv=None):
    """Workspace region offsets ({name: byte offset}) and the block grid (bx, by, nQB, nKB)."""
    lib = load_library()
    args = _marshal(dout, query, key, value, attention_out, softmax_lse, block_sparse_mask, atten_mask,
                    block_shape, actual_seq_lengths, actual_seq_lengths_kv, q_input_layout,
                    kv_input_layout, num_key_value_heads, mask_type, scale_value, pre_tokens,
                    next_tokens, dq, dk, dv)
    offs = (ctypes.c_uint64 * len(WS_REGIONS))()
    dims = (ctypes.c_int64 * 4)()
    _check(lib.bsa_bwd_workspace_layout(*args, offs, dims))
    return dict(zip(WS_REGIONS, list(offs))), tuple(dims)


def bsa_bwd(dout, query, key, value, attention_out, softmax_lse, block_sparse_mask=None, atten_mask=None,
            block_shape=None, actual_seq_lengths=None, actual_seq_lengths_kv=None, q_input_layout="BNSD",
            kv_input_layout="BNSD", num_key_value_heads=1, mask_type=0, scale_value=1.0,
            pre_tokens=NO_WINDOW, next_tokens=NO_WINDOW, dq=None, dk=None, dv=None, workspace=None,
            workspace_size=None, stream=None) -> None:
    """Phase 2: enqueue the backward on ``stream`` (default: torch's current stream).

    All tensors must be GPU tensors; ``workspace`` is a uint8 GPU tensor of at
    least the phase-1 size.
    """
    import torch
    lib = load_library()
    for name, t in (("dout", dout), ("query", query), ("key", key), ("value", value),
                    ("attention_out", attention_out), ("softmax_lse", softmax_lse),
                    ("block_sparse_mask", block_sparse_mask), ("dq", dq), ("dk", dk), ("dv", dv),
                    ("workspace", workspace)):
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    args = _marshal(dout, query, key, value, attention_out, softmax_lse, block_sparse_mask, atten_mask,
                    block_shape, actual_seq_lengths, actual_seq_lengths_kv, q_input_layout,
                    kv_input_layout, num_key_value_heads, mask_type, scale_value, pre_tokens,
                    next_tokens, dq, dk, dv)
    if workspace_size is None:
        workspace_size = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ws_ptr = None if workspace is None or workspace.numel() == 0 else workspace.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream()
    handle = stream if isinstance(stream, int) else stream.cuda_stream
    _check(lib.bsa_bwd(*args, ws_ptr, int(workspace_size), ctypes.c_void_p(handle)))


def bsa_bwd_noalloc(dout, query, key, value, attention_out, softmax_lse, block_sparse_mask=None, atten_mask=None,
                    block_shape=None, actual_seq_lengths=None, actual_seq_lengths_kv=None, q_input_layout="BNSD",
                    kv_input_layout="BNSD", num_key_value_heads=1, mask_type=0, scale_value=1.0,
                    pre_tokens=NO_WINDOW, next_tokens=NO_WINDOW, dq=None, dk=None, dv=None, stream=None) -> None:
    """The backward on the library's own scratch array (no workspace argument, no
    allocation): enqueued on ``stream`` (default: torch's current stream)."""
    lib = load_library()
    _need_gpu(dout=dout, query=query, key=key, value=value, attention_out=attention_out,
              softmax_lse=softmax_lse, block_sparse_mask=block_sparse_mask, dq=dq, dk=dk, dv=dv)
    args = _marshal(dout, query, key, value, attention_out, softmax_lse, block_sparse_mask, atten_mask,
                    block_shape, actual_seq_lengths, actual_seq_lengths_kv, q_input_layout,
                    kv_input_layout, num_key_value_heads, mask_type, scale_value, pre_tokens,
                    next_tokens, dq, dk, dv)
    _check(lib.bsa_bwd_noalloc(*args, _launch_args(None, 0, stream)[2]))


def bsa_bwd_ex_workspace_size(dout, query, key, value, attention_out, softmax_lse, block_sparse_mask=None,
                              atten_mask=None, block_shape=None, actual_seq_lengths=None,
                              actual_seq_lengths_kv=None, q_input_layout="BNSD", kv_input_layout="BNSD",
                              num_key_value_heads=1, mask_type=0, scale_value=1.0, pre_tokens=NO_WINDOW,
                              next_tokens=NO_WINDOW, dq=None, dk=None, dv=None, dq_mode=BSA_DQ_RECOMPUTE) -> int:
    """Phase 1 of the backward with a dQ mode (BSA_DQ_RECOMPUTE / BSA_DQ_ATOMIC)."""
    lib = load_library()
    args = _marshal(dout, query, key, value, attention_out, softmax_lse, block_sparse_mask, atten_mask,
                    block_shape, actual_seq_lengths, actual_seq_lengths_kv, q_input_layout,
                    kv_input_layout, num_key_value_heads, mask_type, scale_value, pre_tokens,
                    next_tokens, dq, dk, dv)
    size = ctypes.c_uint64(0)
    _check(lib.bsa_bwd_ex_workspace_size(*args, int(dq_mode), ctypes.byref(size)))
    return size.value


def bsa_bwd_ex(dout, query, key, value, attention_out, softmax_lse, block_sparse_mask=None, atten_mask=None,
               block_shape=None, actual_seq_lengths=None, actual_seq_lengths_kv=None, q_input_layout="BNSD",
               kv_input_layout="BNSD", num_key_value_heads=1, mask_type=0, scale_value=1.0,
               pre_tokens=NO_WINDOW, next_tokens=NO_WINDOW, dq=None, dk=None, dv=None, dq_mode=BSA_DQ_RECOMPUTE,
               workspace=None, workspace_size=None, stream=None) -> None:
    """Phase 2 of the backward with a dQ mode, enqueued on ``stream``."""
    lib = load_library()
    _need_gpu(dout=dout, query=query, key=key, value=value, attention_out=attention_out,
              softmax_lse=softmax_lse, block_sparse_mask=block_sparse_mask, dq=dq, dk=dk, dv=dv,
              workspace=workspace)
    args = _marshal(dout, query, key, value, attention_out, softmax_lse, block_sparse_mask, atten_mask,
                    block_shape, actual_seq_lengths, actual_seq_lengths_kv, q_input_layout,
                    kv_input_layout, num_key_value_heads, mask_type, scale_value, pre_tokens,
                    next_tokens, dq, dk, dv)
    _check(lib.bsa_bwd_ex(*args, int(dq_mode), *_launch_args(workspace, workspace_size, stream)))


def bsa_fwd_workspace_size(query, key, value, block_sparse_mask=None, atten_mask=None, block_shape=None,
                           actual_seq_lengths=None, actual_seq_lengths_kv=None, q_input_layout="BNSD",
                           kv_input_layout="BNSD", num_key_value_heads=1, mask_type=0, scale_value=1.0,
                           pre_tokens=NO_WINDOW, next_tokens=NO_WINDOW, attention_out=None,
                           softmax_lse=None) -> int:
    """Forward phase 1: validate and return the workspace size in bytes (host only)."""
    lib = load_library()
    args = _marshal_fwd(query, key, value, block_sparse_mask, atten_mask, block_shape, actual_seq_lengths,
                        actual_seq_lengths_kv, q_input_layout, kv_input_layout, num_key_value_heads,
                        mask_type, scale_value, pre_tokens, next_tokens, attention_out, softmax_lse)
    size = ctypes.c_uint64(0)
    _check(lib.bsa_fwd_workspace_size(*args, ctypes.byref(size)))
    return size.value


def bsa_fwd(query, key, value, block_sparse_mask=None, atten_mask=None, block_shape=None,
            actual_seq_lengths=None, actual_seq_lengths_kv=None, q_input_layout="BNSD",
            kv_input_layout="BNSD", num_key_value_heads=1, mask_type=0, scale_value=1.0,
            pre_tokens=NO_WINDOW, next_tokens=NO_WINDOW, attention_out=None, softmax_lse=None,
            workspace=None, workspace_size=None, stream=None) -> None:
    """Forward phase 2: enqueue O and LSE on ``stream`` (default: torch's current stream)."""
    import torch
    lib = load_library()
    for name, t in (("query", query), ("key", key), ("value", value), ("block_sparse_mask", block_sparse_mask),
                    ("attention_out", attention_out), ("softmax_lse", softmax_lse), ("workspace", workspace)):
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
    args = _marshal_fwd(query, key, value, block_sparse_mask, atten_mask, block_shape, actual_seq_lengths,
                        actual_seq_lengths_kv, q_input_layout, kv_input_layout, num_key_value_heads,
                        mask_type, scale_value, pre_tokens, next_tokens, attention_out, softmax_lse)
    if workspace_size is None:
        workspace_size = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ws_ptr = None if workspace is None or workspace.numel() == 0 else workspace.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream()
    handle = stream if isinstance(stream, int) else stream.cuda_stream
    _check(lib.bsa_fwd(*args, ws_ptr, int(workspace_size), ctypes.c_void_p(handle)))


def _descale(descale, n):
    """Host array of n dequantisation factors for the fp8 entry points (None -> NULL = all 1)."""
    if descale is None:
        return None
    vals = [float(x) for x in descale]
    if len(vals) != n:
        raise ValueError(f"descale needs {n} factors, got {len(vals)}")
    return (ctypes.c_double * n)(*vals)


def _launch_args(workspace, workspace_size, stream):
    import torch
    if workspace_size is None:
        workspace_size = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ws_ptr = None if workspace is None or workspace.numel() == 0 else workspace.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream()
    handle = stream if isinstance(stream, int) else stream.cuda_stream
    return ws_ptr, int(workspace_size), ctypes.c_void_p(handle)


def _need_gpu(**tensors):
    for name, t in tensors.items():
        if t is not None and not isinstance(t, bsa_tensor) and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")


def bsa_bwd_fp8_workspace_size(dout, query, key, value, attention_out, softmax_lse, block_sparse_mask=None,
                               atten_mask=None, block_shape=None, actual_seq_lengths=None,
                               actual_seq_lengths_kv=None, q_input_layout="BNSD", kv_input_layout="BNSD",
                               num_key_value_heads=1, mask_type=0, scale_value=1.0, pre_tokens=NO_WINDOW,
                               next_tokens=NO_WINDOW, dq=None, dk=None, dv=None, descale=None) -> int:
    """fp8 backward, phase 1.  ``descale``: factors of (dout, query, key, value, attention_out)."""
    lib = load_library()
    args = _marshal(dout, query, key, value, attention_out, softmax_lse, block_sparse_mask, atten_mask,
                    block_shape, actual_seq_lengths, actual_seq_lengths_kv, q_input_layout,
                    kv_input_layout, num_key_value_heads, mask_type, scale_value, pre_tokens,
                    next_tokens, dq, dk, dv)
    size = ctypes.c_uint64(0)
    _check(lib.bsa_bwd_fp8_workspace_size(*args, _descale(descale, 5), ctypes.byref(size)))
    return size.value


def bsa_bwd_fp8(dout, query, key, value, attention_out, softmax_lse, block_sparse_mask=None, atten_mask=None,
                block_shape=None, actual_seq_lengths=None, actual_seq_lengths_kv=None, q_input_layout="BNSD",
                kv_input_layout="BNSD", num_key_value_heads=1, mask_type=0, scale_value=1.0,
                pre_tokens=NO_WINDOW, next_tokens=NO_WINDOW, dq=None, dk=None, dv=None, descale=None,
                workspace=None, workspace_size=None, stream=None) -> None:
    """fp8 backward, phase 2: fp8 dout/query/key/value/attention_out, bf16 dq/dk/dv."""
    lib = load_library()
    _need_gpu(dout=dout, query=query, key=key, value=value, attention_out=attention_out,
              softmax_lse=softmax_lse, block_sparse_mask=block_sparse_mask, dq=dq, dk=dk, dv=dv,
              workspace=workspace)
    args = _marshal(dout, query, key, value, attention_out, softmax_lse, block_sparse_mask, atten_mask,
                    block_shape, actual_seq_lengths, actual_seq_lengths_kv, q_input_layout,
                    kv_input_layout, num_key_value_heads, mask_type, scale_value, pre_tokens,
                    next_tokens, dq, dk, dv)
    _check(lib.bsa_bwd_fp8(*args, _descale(descale, 5), *_launch_args(workspace, workspace_size, stream)))


def bsa_fwd_fp8_workspace_size(query, key, value, block_sparse_mask=None, atten_mask=None, block_shape=None,
                               actual_seq_lengths=None, actual_seq_lengths_kv=None, q_input_layout="BNSD",
                               kv_input_layout="BNSD", num_key_value_heads=1, mask_type=0, scale_value=1.0,
                               pre_tokens=NO_WINDOW, next_tokens=NO_WINDOW, attention_out=None,
                               softmax_lse=None, descale=None) -> int:
    """fp8 forward, phase 1.  ``descale``: factors of (query, key, value)."""
    lib = load_library()
    args = _marshal_fwd(query, key, value, block_sparse_mask, atten_mask, block_shape, actual_seq_lengths,
                        actual_seq_lengths_kv, q_input_layout, kv_input_layout, num_key_value_heads,
                        mask_type, scale_value, pre_tokens, next_tokens, attention_out, softmax_lse)
    size = ctypes.c_uint64(0)
    _check(lib.bsa_fwd_fp8_workspace_size(*args, _descale(descale, 3), ctypes.byref(size)))
    return size.value


def bsa_fwd_fp8(query, key, value, block_sparse_mask=None, atten_mask=None, block_shape=None,
                actual_seq_lengths=None, actual_seq_lengths_kv=None, q_input_layout="BNSD",
                kv_input_layout="BNSD", num_key_value_heads=1, mask_type=0, scale_value=1.0,
                pre_tokens=NO_WINDOW, next_tokens=NO_WINDOW, attention_out=None, softmax_lse=None,
                descale=None, workspace=None, workspace_size=None, stream=None) -> None:
    """fp8 forward, phase 2: fp8 query/key/value, bf16 attention_out, fp32 softmax_lse."""
    lib = load_library()
    _need_gpu(query=query, key=key, value=value, block_sparse_mask=block_sparse_mask,
              attention_out=attention_out, softmax_lse=softmax_lse, workspace=workspace)
    args = _marshal_fwd(query, key, value, block_sparse_mask, atten_mask, block_shape, actual_seq_lengths,
                        actual_seq_lengths_kv, q_input_layout, kv_input_layout, num_key_value_heads,
                        mask_type, scale_value, pre_tokens, next_tokens, attention_out, softmax_lse)
    _check(lib.bsa_fwd_fp8(*args, _descale(descale, 3), *_launch_args(workspace, workspace_size, stream)))


def block_sparse_attention(query, key, value, block_sparse_mask=None,
                           block_shape: Optional[Sequence[int]] = None, actual_seq_lengths=None,
                           actual_seq_lengths_kv=None, layout="BNSD",
                           num_key_value_heads: Optional[int] = None, scale_value: Optional[float] = None,
                           stream=None):
    """Allocate O, LSE and the workspace with torch, then run the forward.

    Returns ``(attention_out, softmax_lse)`` with LSE shaped [B, N, S] (BNSD)
    or [T, N] (TND); the work is enqueued on ``stream`` and not synchronised.
    """
    import torch
    if num_key_value_heads is None:
        num_key_value_heads = key.shape[1]
    if scale_value is None:
        scale_value = query.shape[-1] ** -0.5
    out = torch.empty_like(query)
    lse = torch.empty(query.shape[:-1], dtype=torch.float32, device=query.device)
    kw = dict(block_sparse_mask=block_sparse_mask, atten_mask=None, block_shape=block_shape,
              actual_seq_lengths=actual_seq_lengths, actual_seq_lengths_kv=actual_seq_lengths_kv,
              q_input_layout=layout, kv_input_layout=layout, num_key_value_heads=num_key_value_heads,
              mask_type=0, scale_value=scale_value, pre_tokens=NO_WINDOW, next_tokens=NO_WINDOW,
              attention_out=out, softmax_lse=lse)
    ws = bsa_fwd_workspace_size(query, key, value, **kw)
    workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=query.device)
    bsa_fwd(query, key, value, **kw, workspace=workspace, workspace_size=ws, stream=stream)
    _hold_until_done(workspace, stream)
    return out, lse


def _hold_until_done(t, stream) -> None:
    """Keep torch's caching allocator from handing out ``t`` (freed when the caller
    returns) before the work enqueued on ``stream`` has finished with it.  With the
    default stream (torch's current one) frees are already ordered on it; a raw
    stream handle is wrapped so that the same bookkeeping applies."""
    import torch
    if stream is None:
        return
    if isinstance(stream, int):
        stream = torch.cuda.ExternalStream(stream, device=t.device)
    t.record_stream(stream)


def bsa_last_error() -> str:
    msg = load_library().bsa_last_error()
    return msg.decode() if msg else ""


def bsa_profile_start(max_calls: int) -> None:
    _check(load_library().bsa_profile_start(int(max_calls)))


def bsa_profile_stop(n_stages: Optional[int] = None):
    """Returns ({stage name: summed ms}, number of profiled calls) for every stage."""
    lib = load_library()
    if n_stages is None:
        n_stages = 0
        while bsa_stage_name(n_stages) is not None:
            n_stages += 1
    ms = (ctypes.c_double * n_stages)()
    calls = ctypes.c_int32(0)
    _check(lib.bsa_profile_stop(ms, n_stages, ctypes.byref(calls)))
    names = [bsa_stage_name(i) for i in range(n_stages)]
    return dict(zip(names, list(ms))), calls.value


def bsa_stage_name(stage: int) -> Optional[str]:
    n = load_library().bsa_stage_name(int(stage))
    return n.decode() if n else None


def block_sparse_attention_grad(dout, query, key, value, attention_out, softmax_lse,
                                block_sparse_mask=None, block_shape: Optional[Sequence[int]] = None,
                                actual_seq_lengths=None, actual_seq_lengths_kv=None, layout="BNSD",
                                num_key_value_heads: Optional[int] = None,
                                scale_value: Optional[float] = None, stream=None):
    """Allocate dq/dk/dv and the workspace with torch, then run both phases.

    Returns ``(dq, dk, dv)``; the work is enqueued on ``stream`` (torch's
    current stream by default) and not synchronised.
    """
    import torch
    if num_key_value_heads is None:
        num_key_value_heads = key.shape[1]
    if scale_value is None:
        scale_value = query.shape[-1] ** -0.5
    dq = torch.empty_like(query)
    dk = torch.empty_like(key)
    dv = torch.empty_like(value)
    kw = dict(block_sparse_mask=block_sparse_mask, atten_mask=None, block_shape=block_shape,
              actual_seq_lengths=actual_seq_lengths, actual_seq_lengths_kv=actual_seq_lengths_kv,
              q_input_layout=layout, kv_input_layout=layout, num_key_value_heads=num_key_value_heads,
              mask_type=0, scale_value=scale_value, pre_tokens=NO_WINDOW, next_tokens=NO_WINDOW,
              dq=dq, dk=dk, dv=dv)
    ws = bsa_bwd_workspace_size(dout, query, key, value, attention_out, softmax_lse, **kw)
    workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=query.device)
    bsa_bwd(dout, query, key, value, attention_out, softmax_lse, **kw, workspace=workspace,
            workspace_size=ws, stream=stream)
    _hold_until_done(workspace, stream)
    return dq, dk, dv
