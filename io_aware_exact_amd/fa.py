"""ctypes binding of libfa.so (the C ABI in include/fa.h).

Argument marshalling only: every step of the attention computation runs in the
library's HIP kernels.  Tensors are PyTorch-allocated device tensors; work is
enqueued on the current torch stream.  The library is required: if it has not
been built, or a call fails, an exception is raised -- there is no fallback.
"""
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_BF16 = 0
FA_FP32 = 1
FA_FP8_E4M3 = 2
_DTYPES = {torch.bfloat16: FA_BF16, torch.float32: FA_FP32}


class FaError(RuntimeError):
    """A libfa entry point returned a nonzero fa_status."""

    def __init__(self, call, status, message):
        super().__init__(f"{call} failed: status {status} ({message})")
        self.status = status


class FaTensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_s", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class FwdArgs(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("Sq", ctypes.c_int32),
                ("Sk", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float),
                ("q", FaTensor), ("k", FaTensor), ("v", FaTensor), ("o", FaTensor),
                ("lse", ctypes.c_void_p), ("q_descale", ctypes.c_void_p),
                ("k_descale", ctypes.c_void_p), ("v_descale", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class FwdVarlenArgs(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("nseq", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("max_seqlen_q", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32),
                ("total_q", ctypes.c_int32), ("total_k", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p),
                ("q_stride_t", ctypes.c_int64), ("q_stride_h", ctypes.c_int64),
                ("k_stride_t", ctypes.c_int64), ("k_stride_h", ctypes.c_int64),
                ("v_stride_t", ctypes.c_int64), ("v_stride_h", ctypes.c_int64),
                ("o_stride_t", ctypes.c_int64), ("o_stride_h", ctypes.c_int64),
                ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
                ("lse", ctypes.c_void_p)]


class BwdArgs(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("Sq", ctypes.c_int32),
                ("Sk", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float),
                ("q", FaTensor), ("k", FaTensor), ("v", FaTensor), ("o", FaTensor),
                ("dout", FaTensor), ("dq", FaTensor), ("dk", FaTensor), ("dv", FaTensor),
                ("lse", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("stages", ctypes.c_int32),
                ("q_descale", ctypes.c_void_p), ("k_descale", ctypes.c_void_p),
                ("v_descale", ctypes.c_void_p)]


class BwdVarlenArgs(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("nseq", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("max_seqlen_q", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32),
                ("total_q", ctypes.c_int32), ("total_k", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("o", ctypes.c_void_p), ("dout", ctypes.c_void_p),
                ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
                ("q_stride_t", ctypes.c_int64), ("q_stride_h", ctypes.c_int64),
                ("k_stride_t", ctypes.c_int64), ("k_stride_h", ctypes.c_int64),
                ("v_stride_t", ctypes.c_int64), ("v_stride_h", ctypes.c_int64),
                ("o_stride_t", ctypes.c_int64), ("o_stride_h", ctypes.c_int64),
                ("do_stride_t", ctypes.c_int64), ("do_stride_h", ctypes.c_int64),
                ("dq_stride_t", ctypes.c_int64), ("dq_stride_h", ctypes.c_int64),
                ("dk_stride_t", ctypes.c_int64), ("dk_stride_h", ctypes.c_int64),
                ("dv_stride_t", ctypes.c_int64), ("dv_stride_h", ctypes.c_int64),
                ("cu_seqlens_q", ctypes.c_void_p), ("cu_seqlens_k", ctypes.c_void_p),
                ("lse", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


class FwdKvcacheArgs(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("Sq", ctypes.c_int32),
                ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("Snew", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float),
                ("q", FaTensor), ("o", FaTensor), ("lse", ctypes.c_void_p),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("k_stride_page", ctypes.c_int64), ("k_stride_s", ctypes.c_int64),
                ("k_stride_h", ctypes.c_int64),
                ("v_stride_page", ctypes.c_int64), ("v_stride_s", ctypes.c_int64),
                ("v_stride_h", ctypes.c_int64),
                ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_pages_per_seq", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32),
                ("block_table", ctypes.c_void_p), ("block_table_stride", ctypes.c_int64),
                ("cache_seqlens", ctypes.c_void_p),
                ("k_new", FaTensor), ("v_new", FaTensor),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class FwdMxfp8Args(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Sq", ctypes.c_int32), ("Sk", ctypes.c_int32),
                ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("q", FaTensor), ("k", FaTensor), ("v", FaTensor), ("o", FaTensor),
                ("lse", ctypes.c_void_p), ("q_scale", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p)]


class MergeArgs(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("nparts", ctypes.c_int32), ("B", ctypes.c_int32),
                ("S", ctypes.c_int32), ("H", ctypes.c_int32), ("d", ctypes.c_int32),
                ("o_parts", ctypes.c_void_p), ("lse_parts", ctypes.c_void_p), ("o", FaTensor),
                ("lse", ctypes.c_void_p)]


FA_BWD_ALL, FA_BWD_PREPROCESS, FA_BWD_DKDV, FA_BWD_DQ = 0, 1, 2, 4


# Every symbol include/fa.h declares.
EXPORTS = ["fa_abi_version", "fa_status_string", "fa_fwd_workspace_size",
           "fa_bwd_workspace_size", "fa_fwd", "fa_fwd_varlen", "fa_bwd",
           "fa_bwd_varlen_workspace_size", "fa_bwd_varlen", "fa_fwd_kvcache_workspace_size",
           "fa_fwd_kvcache", "fa_quantize_fp8", "fa_fwd_mxfp8", "fa_quantize_mxfp8",
           "fa_merge", "fa_bwd_noalloc"]

_lib = None


def lib():
    """Open libfa.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m io_aware_exact_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        L.fa_abi_version.restype = ctypes.c_int32
        L.fa_status_string.restype = ctypes.c_char_p
        L.fa_status_string.argtypes = [ctypes.c_int]
        L.fa_fwd_workspace_size.restype = ctypes.c_size_t
        L.fa_fwd_workspace_size.argtypes = [ctypes.POINTER(FwdArgs)]
        L.fa_bwd_workspace_size.restype = ctypes.c_size_t
        L.fa_bwd_workspace_size.argtypes = [ctypes.POINTER(BwdArgs)]
        L.fa_fwd.restype = ctypes.c_int
        L.fa_fwd.argtypes = [ctypes.POINTER(FwdArgs), vp]
        L.fa_fwd_varlen.restype = ctypes.c_int
        L.fa_fwd_varlen.argtypes = [ctypes.POINTER(FwdVarlenArgs), vp]
        L.fa_bwd.restype = ctypes.c_int
        L.fa_bwd.argtypes = [ctypes.POINTER(BwdArgs), vp]
        L.fa_bwd_noalloc.restype = ctypes.c_int
        L.fa_bwd_noalloc.argtypes = [ctypes.POINTER(BwdArgs), vp]
        L.fa_bwd_varlen_workspace_size.restype = ctypes.c_size_t
        L.fa_bwd_varlen_workspace_size.argtypes = [ctypes.POINTER(BwdVarlenArgs)]
        L.fa_bwd_varlen.restype = ctypes.c_int
        L.fa_bwd_varlen.argtypes = [ctypes.POINTER(BwdVarlenArgs), vp]
        L.fa_fwd_kvcache_workspace_size.restype = ctypes.c_size_t
        L.fa_fwd_kvcache_workspace_size.argtypes = [ctypes.POINTER(FwdKvcacheArgs)]
        L.fa_fwd_kvcache.restype = ctypes.c_int
        L.fa_fwd_kvcache.argtypes = [ctypes.POINTER(FwdKvcacheArgs), vp]
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        L.fa_quantize_fp8.restype = ctypes.c_int
        L.fa_quantize_fp8.argtypes = [vp, i64, i64, i64, i32, i32, i32, i32, i32, vp, vp, vp]
        L.fa_fwd_mxfp8.restype = ctypes.c_int
        L.fa_fwd_mxfp8.argtypes = [ctypes.POINTER(FwdMxfp8Args), vp]
        L.fa_merge.restype = ctypes.c_int
        L.fa_merge.argtypes = [ctypes.POINTER(MergeArgs), vp]
        L.fa_quantize_mxfp8.restype = ctypes.c_int
        L.fa_quantize_mxfp8.argtypes = [vp, i64, i64, i64, i32, i32, i32, i32, i32, vp, vp, vp]
        _lib = L
    return _lib


def _check(call, status):
    if status != 0:
        raise FaError(call, status, lib().fa_status_string(status).decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _t4(x):
    """fa_tensor of a [B,S,H,d] tensor (d contiguous)."""
    _need(x.dim() == 4 and x.stride(3) == 1, "a [B,S,H,d] tensor with d contiguous is required")
    return FaTensor(x.data_ptr(), x.stride(0), x.stride(1), x.stride(2))


def _scale(d, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


# ---- argument checks ---------------------------------------------------------
# The C ABI takes one dtype and raw element strides for every tensor of a call,
# so a tensor of the wrong dtype, shape or device would be read or written out
# of bounds on the GPU.  The wrappers check every tensor against q before any
# library call and raise ValueError.

def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _on_device(dev, **ts):
    """Every named tensor (None allowed) is a GPU tensor on device `dev`."""
    for name, t in ts.items():
        if t is None:
            continue
        _need(t.device.type == "cuda" and t.device == dev,
              f"{name} must be a GPU tensor on {dev} (got {t.device})")


def _shape(name, t, shape, dtype=None):
    _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None:
        _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")


def _lse(name, t, shape):
    _shape(name, t, shape, torch.float32)
    _need(t.is_contiguous(), f"{name} must be contiguous")


def _workspace(ws):
    if ws is not None:
        _need(ws.dtype == torch.uint8 and ws.is_contiguous(), "workspace must be a contiguous uint8 tensor")


def _check_dense(q, k, v, dtypes):
    """q [B,Sq,Hq,d], k and v [B,Sk,Hkv,d] of one dtype in `dtypes`."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t.dim() == 4, f"{name} must be [B,S,H,d]")
    _need(q.dtype in dtypes, f"q dtype {q.dtype} is not supported here")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k and v must share one dtype")
    _need(tuple(k.shape) == tuple(v.shape), "k and v must have the same shape")
    _need(k.shape[0] == q.shape[0] and k.shape[3] == q.shape[3],
          "k and v must have q's batch size and head dimension")


def _check_packed(q, k, v, dtypes):
    """q [Tq,Hq,d], k and v [Tk,Hkv,d] of one dtype in `dtypes`."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t.dim() == 3, f"{name} must be [T,H,d]")
    _need(q.dtype in dtypes, f"q dtype {q.dtype} is not supported here")
    _need(k.dtype == q.dtype and v.dtype == q.dtype, "q, k and v must share one dtype")
    _need(tuple(k.shape) == tuple(v.shape), "k and v must have the same shape")
    _need(k.shape[2] == q.shape[2], "k and v must have q's head dimension")


def _check_cu(cu_q, cu_k, dev):
    for name, t in (("cu_seqlens_q", cu_q), ("cu_seqlens_k", cu_k)):
        _need(t.dtype == torch.int32 and t.dim() == 1 and t.is_contiguous(),
              f"{name} must be a contiguous int32 vector")
    _need(cu_q.numel() == cu_k.numel() and cu_q.numel() >= 1,
          "cu_seqlens_q and cu_seqlens_k must both have nseq + 1 entries")
    _on_device(dev, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k)


def fwd_args(q, k, v, out, lse, causal, scale, workspace=None):
    _check_dense(q, k, v, (torch.bfloat16, torch.float32))
    B, Sq, Hq, d = q.shape
    _shape("out", out, q.shape, torch.float32 if q.dtype == torch.float32 else torch.bfloat16)
    _lse("lse", lse, (B, Hq, Sq))
    _workspace(workspace)
    _on_device(q.device, q=q, k=k, v=v, out=out, lse=lse, workspace=workspace)
    Sk, Hkv = k.shape[1], k.shape[2]
    dt = _DTYPES.get(q.dtype, -1)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return FwdArgs(dt, B, Sq, Sk, Hq, Hkv, d, int(bool(causal)), _scale(d, scale),
                   _t4(q), _t4(k), _t4(v), _t4(out), lse.data_ptr(), None, None, None,
                   ws_ptr, ws_bytes)


def fwd_workspace_bytes(q, k, v, causal=False, scale=None):
    """Bytes of workspace the split-KV decode path wants (0: not applicable)."""
    _check_dense(q, k, v, (torch.bfloat16, torch.float32))
    B, Sq, Hq, d = q.shape
    dummy = torch.empty(0)
    a = FwdArgs(FA_BF16, B, Sq, k.shape[1], Hq, k.shape[2], d, int(bool(causal)),
                _scale(d, scale), _t4(q), _t4(k), _t4(v), _t4(q), dummy.data_ptr(),
                None, None, None, None, 0)
    return int(lib().fa_fwd_workspace_size(ctypes.byref(a)))


def fwd(q, k, v, causal=False, scale=None, out=None, lse=None, workspace=None):
    """Dense forward.  q [B,Sq,Hq,d], k/v [B,Sk,Hkv,d] bf16 (or fp32) on the
    GPU.  Returns (o [B,Sq,Hq,d] bf16 (fp32 for fp32 inputs), lse [B,Hq,Sq]
    fp32).  With a `workspace`
    (uint8 device tensor of fwd_workspace_bytes) decode-shaped calls take the
    split-KV path."""
    _check_dense(q, k, v, (torch.bfloat16, torch.float32))
    B, Sq, Hq, d = q.shape
    if out is None:
        odt = torch.float32 if q.dtype == torch.float32 else torch.bfloat16
        out = torch.empty((B, Sq, Hq, d), dtype=odt, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    a = fwd_args(q, k, v, out, lse, causal, scale, workspace)
    _check("fa_fwd", lib().fa_fwd(ctypes.byref(a), _stream()))
    return out, lse


def fwd_decode(q, k, v, causal=False, scale=None, out=None, lse=None):
    """Forward that allocates the split-KV workspace when the decode path
    applies (M = Sq * Hq / Hkv <= 32, or M <= 128 in fewer 32-row blocks than
    Hq / Hkv), else the plain dense forward."""
    n = fwd_workspace_bytes(q, k, v, causal, scale)
    ws = torch.empty(n, dtype=torch.uint8, device=q.device) if n > 0 else None
    return fwd(q, k, v, causal, scale, out, lse, ws)


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
               causal=False, scale=None, out=None, lse=None):
    """Packed forward.  q [Tq,Hq,d], k/v [Tk,Hkv,d] bf16; cu_seqlens_* int32
    [nseq+1] on the GPU.  Returns (o [Tq,Hq,d] bf16, lse [Hq,Tq] fp32)."""
    _check_packed(q, k, v, (torch.bfloat16,))
    Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    for x in (q, k, v):
        _need(x.stride(2) == 1, "the last dimension must be contiguous")
    nseq = cu_seqlens_q.numel() - 1
    if out is None:
        out = torch.empty((Tq, Hq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    _shape("out", out, q.shape, torch.bfloat16)
    _need(out.stride(2) == 1, "out: the last dimension must be contiguous")
    _lse("lse", lse, (Hq, Tq))
    _check_cu(cu_seqlens_q, cu_seqlens_k, q.device)
    _on_device(q.device, q=q, k=k, v=v, out=out, lse=lse)
    dt = FA_BF16 if q.dtype == torch.bfloat16 else -1
    a = FwdVarlenArgs(dt, nseq, Hq, Hkv, d, int(max_seqlen_q), int(max_seqlen_k), Tq, Tk,
                      int(bool(causal)), _scale(d, scale),
                      q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                      q.stride(0), q.stride(1), k.stride(0), k.stride(1),
                      v.stride(0), v.stride(1), out.stride(0), out.stride(1),
                      cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), lse.data_ptr())
    _check("fa_fwd_varlen", lib().fa_fwd_varlen(ctypes.byref(a), _stream()))
    return out, lse


def kvcache_args(q, k_cache, v_cache, cache_seqlens, block_table, k_new, v_new, out, lse,
                 causal, scale, max_seqlen_k=0, workspace=None):
    """fa_fwd_kvcache_args.  Caches [pages, page_size, Hkv, d] (without a
    block table: [B, capacity, Hkv, d]); block_table int32 [B, max_pages] or
    None; cache_seqlens int32 [B]; k_new/v_new [B, Snew, Hkv, d] or None."""
    _need(q.dim() == 4 and q.dtype == torch.bfloat16, "q must be a bf16 [B,Sq,Hq,d] tensor")
    B, Sq, Hq, d = q.shape
    for name, x in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(x.dim() == 4 and x.stride(3) == 1 and x.dtype == torch.bfloat16,
              f"{name} must be a bf16 [pages, page_size, Hkv, d] tensor, d contiguous")
    _need(tuple(k_cache.shape) == tuple(v_cache.shape) and k_cache.shape[3] == d,
          "k_cache and v_cache must have the same shape and q's head dimension")
    npages, page_size, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    _need(cache_seqlens.dtype == torch.int32 and tuple(cache_seqlens.shape) == (B,)
          and cache_seqlens.is_contiguous(), "cache_seqlens must be a contiguous int32 [B] tensor")
    _need((k_new is None) == (v_new is None), "k_new and v_new go together")
    if k_new is not None:
        _shape("k_new", k_new, (B, k_new.shape[1], Hkv, d), torch.bfloat16)
        _shape("v_new", v_new, k_new.shape, torch.bfloat16)
    if block_table is not None:
        _need(block_table.dim() == 2 and block_table.shape[0] == B, "block_table must be [B, max_pages]")
    _shape("out", out, q.shape, torch.bfloat16)
    _lse("lse", lse, (B, Hq, Sq))
    _workspace(workspace)
    _on_device(q.device, q=q, k_cache=k_cache, v_cache=v_cache, cache_seqlens=cache_seqlens,
               block_table=block_table, k_new=k_new, v_new=v_new, out=out, lse=lse,
               workspace=workspace)
    snew = 0 if k_new is None else k_new.shape[1]
    dt = FA_BF16 if q.dtype == torch.bfloat16 else -1
    none4 = FaTensor(None, 0, 0, 0)
    if block_table is not None:
        _need(block_table.dtype == torch.int32 and block_table.stride(1) == 1,
              "block_table must be int32 with contiguous rows")
        bt_ptr, bt_stride, maxp = block_table.data_ptr(), block_table.stride(0), block_table.shape[1]
    else:
        bt_ptr, bt_stride, maxp = None, 0, 0
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return FwdKvcacheArgs(dt, B, Sq, Hq, Hkv, d, snew, int(bool(causal)), _scale(d, scale),
                          _t4(q), _t4(out), lse.data_ptr(),
                          k_cache.data_ptr(), v_cache.data_ptr(),
                          k_cache.stride(0), k_cache.stride(1), k_cache.stride(2),
                          v_cache.stride(0), v_cache.stride(1), v_cache.stride(2),
                          npages, page_size, maxp, int(max_seqlen_k), bt_ptr, bt_stride,
                          cache_seqlens.data_ptr(),
                          _t4(k_new) if snew else none4, _t4(v_new) if snew else none4,
                          ws_ptr, ws_bytes)


def fwd_kvcache(q, k_cache, v_cache, cache_seqlens, block_table=None, k_new=None, v_new=None,
                causal=False, scale=None, max_seqlen_k=0, out=None, lse=None, workspace=None):
    """KV-cache attention: appends k_new/v_new ([B,Snew,Hkv,d]) to the cache
    at positions cache_seqlens[b].., then q [B,Sq,Hq,d] attends to the
    cache_seqlens[b] + Snew tokens of each sequence (see kvcache_args for the
    cache layout).  cache_seqlens is not updated.  Returns (o, lse).  When
    `workspace` is None and the split-KV path applies, one is allocated."""
    B, Sq, Hq, d = q.shape
    if out is None:
        out = torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if workspace is None:
        a = kvcache_args(q, k_cache, v_cache, cache_seqlens, block_table, k_new, v_new, out, lse,
                         causal, scale, max_seqlen_k)
        n = int(lib().fa_fwd_kvcache_workspace_size(ctypes.byref(a)))
        if n > 0:
            workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    a = kvcache_args(q, k_cache, v_cache, cache_seqlens, block_table, k_new, v_new, out, lse,
                     causal, scale, max_seqlen_k, workspace)
    _check("fa_fwd_kvcache", lib().fa_fwd_kvcache(ctypes.byref(a), _stream()))
    return out, lse


def bwd_args(q, k, v, o, dout, lse, dq, dk, dv, causal, scale, workspace=None, stages=0):
    _check_dense(q, k, v, (torch.bfloat16,))
    B, Sq, Hq, d = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    for name, t, like in (("o", o, q), ("dout", dout, q), ("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _shape(name, t, like.shape, torch.bfloat16)
    _lse("lse", lse, (B, Hq, Sq))
    _workspace(workspace)
    _on_device(q.device, q=q, k=k, v=v, o=o, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv,
               workspace=workspace)
    dt = FA_BF16 if q.dtype == torch.bfloat16 else -1
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return BwdArgs(dt, B, Sq, Sk, Hq, Hkv, d, int(bool(causal)), _scale(d, scale),
                   _t4(q), _t4(k), _t4(v), _t4(o), _t4(dout), _t4(dq), _t4(dk), _t4(dv),
                   lse.data_ptr(), ws_ptr, ws_bytes, int(stages))


def bwd(q, k, v, o, dout, lse, causal=False, scale=None, out=None, workspace=None, stages=0):
    """Dense backward.  Returns (dq, dk, dv) bf16.  `out` = (dq, dk, dv) and
    `workspace` (uint8 device tensor) may be passed in to reuse buffers;
    `stages` selects FA_BWD_* stages (0: all)."""
    if out is None:
        out = (torch.empty_like(q, dtype=torch.bfloat16),
               torch.empty(k.shape, dtype=torch.bfloat16, device=k.device),
               torch.empty(v.shape, dtype=torch.bfloat16, device=v.device))
    dq, dk, dv = out
    if workspace is None:
        a = bwd_args(q, k, v, o, dout, lse, dq, dk, dv, causal, scale)
        nbytes = lib().fa_bwd_workspace_size(ctypes.byref(a))
        workspace = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=q.device)
    a = bwd_args(q, k, v, o, dout, lse, dq, dk, dv, causal, scale, workspace, stages)
    _check("fa_bwd", lib().fa_bwd(ctypes.byref(a), _stream()))
    return dq, dk, dv


def bwd_fp8_args(q8, k8, v8, descales, o, dout, lse, dq, dk, dv, causal, scale, workspace=None,
                 stages=0):
    """fa_bwd_args for the FP8 backward: E4M3 codes q8 [B,Sq,Hq,d], k8/v8
    [B,Sk,Hkv,d] with the forward's fp32 block scales (q, k, v descales);
    o, dout and the gradients bf16."""
    _check_fp8_codes(q8, k8, v8)
    B, Sq, Hq, d = q8.shape
    Sk, Hkv = k8.shape[1], k8.shape[2]
    q_descale, k_descale, v_descale = descales
    _lse("q_descale", q_descale, (B, Hq, (Sq + 127) // 128))
    _lse("k_descale", k_descale, (B, Hkv, (Sk + 127) // 128))
    _lse("v_descale", v_descale, (B, Hkv, (Sk + 127) // 128))
    for name, t, shape in (("o", o, q8.shape), ("dout", dout, q8.shape), ("dq", dq, q8.shape),
                           ("dk", dk, k8.shape), ("dv", dv, k8.shape)):
        _shape(name, t, shape, torch.bfloat16)
    _lse("lse", lse, (B, Hq, Sq))
    _workspace(workspace)
    _on_device(q8.device, q8=q8, k8=k8, v8=v8, q_descale=q_descale, k_descale=k_descale,
               v_descale=v_descale, o=o, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv, workspace=workspace)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() if workspace is not None else 0
    a = BwdArgs(FA_FP8_E4M3, B, Sq, Sk, Hq, Hkv, d, int(bool(causal)), _scale(d, scale),
                _t4(q8), _t4(k8), _t4(v8), _t4(o), _t4(dout), _t4(dq), _t4(dk), _t4(dv),
                lse.data_ptr(), ws_ptr, ws_bytes, int(stages))
    a.q_descale, a.k_descale, a.v_descale = (q_descale.data_ptr(), k_descale.data_ptr(),
                                             v_descale.data_ptr())
    return a


def bwd_fp8(q8, k8, v8, descales, o, dout, lse, causal=False, scale=None, out=None,
            workspace=None, stages=0):
    """FP8 backward (the gradient of fwd_fp8 with respect to the dequantised
    q, k, v): all five products on FP8 matrix instructions.  descales =
    (q_descale, k_descale, v_descale) as for fwd_fp8; o, dout bf16, lse from
    the forward.  Returns (dq, dk, dv) bf16."""
    B, Sq, Hq, d = q8.shape
    if out is None:
        out = (torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device=q8.device),
               torch.empty(k8.shape, dtype=torch.bfloat16, device=k8.device),
               torch.empty(v8.shape, dtype=torch.bfloat16, device=v8.device))
    dq, dk, dv = out
    if workspace is None:
        a = bwd_fp8_args(q8, k8, v8, descales, o, dout, lse, dq, dk, dv, causal, scale)
        nbytes = lib().fa_bwd_workspace_size(ctypes.byref(a))
        workspace = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=q8.device)
    a = bwd_fp8_args(q8, k8, v8, descales, o, dout, lse, dq, dk, dv, causal, scale, workspace, stages)
    _check("fa_bwd", lib().fa_bwd(ctypes.byref(a), _stream()))
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, dout, lse, causal=False, scale=None, out=None, stages=0):
    """Dense backward through fa_bwd_noalloc: no workspace and no allocation
    in the library (its scratch is a fixed per-device array shared by every
    call on that GPU).  Returns (dq, dk, dv) bf16; `out` may be passed in."""
    if out is None:
        out = (torch.empty_like(q, dtype=torch.bfloat16),
               torch.empty(k.shape, dtype=torch.bfloat16, device=k.device),
               torch.empty(v.shape, dtype=torch.bfloat16, device=v.device))
    dq, dk, dv = out
    a = bwd_args(q, k, v, o, dout, lse, dq, dk, dv, causal, scale, None, stages)
    _check("fa_bwd_noalloc", lib().fa_bwd_noalloc(ctypes.byref(a), _stream()))
    return dq, dk, dv


def bwd_varlen_args(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_k,
                    max_seqlen_q, max_seqlen_k, causal, scale, workspace=None):
    _check_packed(q, k, v, (torch.bfloat16,))
    Tq, Hq, d = q.shape
    Tk, Hkv = k.shape[0], k.shape[1]
    for name, t, like in (("o", o, q), ("dout", dout, q), ("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _shape(name, t, like.shape, torch.bfloat16)
    for x in (q, k, v, o, dout, dq, dk, dv):
        _need(x.stride(2) == 1, "packed [T,H,d] tensors need a contiguous last dimension")
    _lse("lse", lse, (Hq, Tq))
    _check_cu(cu_seqlens_q, cu_seqlens_k, q.device)
    _workspace(workspace)
    _on_device(q.device, q=q, k=k, v=v, o=o, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv,
               workspace=workspace)
    dt = FA_BF16 if q.dtype == torch.bfloat16 else -1
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return BwdVarlenArgs(dt, cu_seqlens_q.numel() - 1, Hq, Hkv, d, int(max_seqlen_q),
                         int(max_seqlen_k), Tq, Tk, int(bool(causal)), _scale(d, scale),
                         q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                         dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                         q.stride(0), q.stride(1), k.stride(0), k.stride(1), v.stride(0), v.stride(1),
                         o.stride(0), o.stride(1), dout.stride(0), dout.stride(1),
                         dq.stride(0), dq.stride(1), dk.stride(0), dk.stride(1),
                         dv.stride(0), dv.stride(1), cu_seqlens_q.data_ptr(),
                         cu_seqlens_k.data_ptr(), lse.data_ptr(), ws_ptr, ws_bytes)


def bwd_varlen(q, k, v, o, dout, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
               causal=False, scale=None, out=None, workspace=None):
    """Packed variable-length backward.  q, o, dout [Tq,Hq,d], k/v [Tk,Hkv,d]
    bf16, lse [Hq,Tq] from fwd_varlen.  Returns (dq, dk, dv) bf16."""
    if out is None:
        out = (torch.empty(q.shape, dtype=torch.bfloat16, device=q.device),
               torch.empty(k.shape, dtype=torch.bfloat16, device=k.device),
               torch.empty(v.shape, dtype=torch.bfloat16, device=v.device))
    dq, dk, dv = out
    if workspace is None:
        a = bwd_varlen_args(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_k,
                            max_seqlen_q, max_seqlen_k, causal, scale)
        nbytes = lib().fa_bwd_varlen_workspace_size(ctypes.byref(a))
        workspace = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=q.device)
    a = bwd_varlen_args(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens_q, cu_seqlens_k,
                        max_seqlen_q, max_seqlen_k, causal, scale, workspace)
    _check("fa_bwd_varlen", lib().fa_bwd_varlen(ctypes.byref(a), _stream()))
    return dq, dk, dv


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal, scale):
        o, lse = fwd(q, k, v, causal, scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale = causal, scale
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = bwd(q, k, v, o, do.contiguous(), lse, ctx.causal, ctx.scale)
        return dq, dk, dv, None, None


def attention(q, k, v, causal=False, scale=None):
    """Exact attention with autograd: q [B,Sq,Hq,d], k/v [B,Sk,Hkv,d] bf16."""
    return _Attention.apply(q, k, v, causal, scale)


def quantize_fp8(x, per_tensor=False):
    """x [B,S,H,d] fp32 on the GPU (d contiguous) -> (codes uint8 [B,S,H,d]
    OCP E4M3, scales fp32 [B,H,ceil(S/128)]).  Per-block: one scale per
    (batch, head, 128 tokens); per-tensor: one scale written to every entry."""
    _need(x.dtype == torch.float32 and x.dim() == 4 and x.stride(3) == 1,
          "x must be fp32 [B,S,H,d] with d contiguous")
    _on_device(x.device, x=x)
    B, S, H, d = x.shape
    codes = torch.empty((B, S, H, d), dtype=torch.uint8, device=x.device)
    scales = torch.empty((B, H, (S + 127) // 128), dtype=torch.float32, device=x.device)
    _check("fa_quantize_fp8", lib().fa_quantize_fp8(
        x.data_ptr(), x.stride(0), x.stride(1), x.stride(2), B, S, H, d, int(bool(per_tensor)),
        codes.data_ptr(), scales.data_ptr(), _stream()))
    return codes, scales


def _check_fp8_codes(q8, k8, v8):
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        _need(t.dim() == 4 and t.dtype in (torch.uint8, torch.float8_e4m3fn),
              f"{name} must be E4M3 codes (uint8 or float8_e4m3fn) [B,S,H,d]")
    _need(tuple(k8.shape) == tuple(v8.shape), "k8 and v8 must have the same shape")
    _need(k8.shape[0] == q8.shape[0] and k8.shape[3] == q8.shape[3],
          "k8 and v8 must have q8's batch size and head dimension")


def fwd_fp8(q8, k8, v8, q_descale, k_descale, v_descale, causal=False, scale=None,
            out=None, lse=None):
    """FP8 forward: q8 [B,Sq,Hq,d], k8/v8 [B,Sk,Hkv,d] E4M3 codes (uint8 or
    float8_e4m3fn) with fp32 scales [B,H,ceil(S/128)].  Returns (o bf16, lse)."""
    _check_fp8_codes(q8, k8, v8)
    B, Sq, Hq, d = q8.shape
    Sk, Hkv = k8.shape[1], k8.shape[2]
    _lse("q_descale", q_descale, (B, Hq, (Sq + 127) // 128))
    _lse("k_descale", k_descale, (B, Hkv, (Sk + 127) // 128))
    _lse("v_descale", v_descale, (B, Hkv, (Sk + 127) // 128))
    if out is None:
        out = torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q8.device)
    _shape("out", out, q8.shape, torch.bfloat16)
    _lse("lse", lse, (B, Hq, Sq))
    _on_device(q8.device, q8=q8, k8=k8, v8=v8, q_descale=q_descale, k_descale=k_descale,
               v_descale=v_descale, out=out, lse=lse)
    a = FwdArgs(FA_FP8_E4M3, B, Sq, Sk, Hq, Hkv, d, int(bool(causal)), _scale(d, scale),
                _t4(q8), _t4(k8), _t4(v8), _t4(out), lse.data_ptr(), q_descale.data_ptr(),
                k_descale.data_ptr(), v_descale.data_ptr(), None, 0)
    _check("fa_fwd", lib().fa_fwd(ctypes.byref(a), _stream()))
    return out, lse


def merge(o_parts, lse_parts, out=None, lse=None):
    """Exact merge of partial results over disjoint key shards: o_parts
    [P,B,S,H,d] (bf16 or fp32) and lse_parts [P,B,H,S] fp32, contiguous ->
    (o [B,S,H,d] bf16, lse [B,H,S] fp32)."""
    P, B, S, H, d = o_parts.shape
    _need(o_parts.is_contiguous() and lse_parts.is_contiguous(), "the parts must be contiguous")
    _need(o_parts.dtype in (torch.bfloat16, torch.float32), "o_parts must be bf16 or fp32")
    _lse("lse_parts", lse_parts, (P, B, H, S))
    if out is None:
        out = torch.empty((B, S, H, d), dtype=torch.bfloat16, device=o_parts.device)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=o_parts.device)
    _shape("out", out, (B, S, H, d), torch.bfloat16)
    _lse("lse", lse, (B, H, S))
    _on_device(o_parts.device, o_parts=o_parts, lse_parts=lse_parts, out=out, lse=lse)
    dt = {torch.bfloat16: FA_BF16, torch.float32: FA_FP32}.get(o_parts.dtype, -1)
    a = MergeArgs(dt, P, B, S, H, d, o_parts.data_ptr(), lse_parts.data_ptr(), _t4(out),
                  lse.data_ptr())
    _check("fa_merge", lib().fa_merge(ctypes.byref(a), _stream()))
    return out, lse


def quantize_mxfp8(x, axis):
    """MX quantisation of x [B,S,H,d] fp32 on the GPU (d contiguous): codes
    uint8 [B,S,H,d] OCP E4M3 and E8M0 scale bytes, one per 32 elements --
    axis 0 (q, k): along d, scales [B,S,H,d/32]; axis 1 (v): along the
    tokens, scales [B,H,ceil(S/32),d]."""
    _need(x.dtype == torch.float32 and x.dim() == 4 and x.stride(3) == 1,
          "x must be fp32 [B,S,H,d] with d contiguous")
    _on_device(x.device, x=x)
    B, S, H, d = x.shape
    codes = torch.empty((B, S, H, d), dtype=torch.uint8, device=x.device)
    shape = (B, S, H, d // 32) if axis == 0 else (B, H, (S + 31) // 32, d)
    scales = torch.empty(shape, dtype=torch.uint8, device=x.device)
    _check("fa_quantize_mxfp8", lib().fa_quantize_mxfp8(
        x.data_ptr(), x.stride(0), x.stride(1), x.stride(2), B, S, H, d, int(axis),
        codes.data_ptr(), scales.data_ptr(), _stream()))
    return codes, scales


def fwd_mxfp8(q8, k8, v8, q_scale, k_scale, v_scale, causal=False, scale=None, out=None,
              lse=None):
    """MX FP8 forward: E4M3 codes q8 [B,Sq,Hq,d], k8/v8 [B,Sk,Hkv,d] with the
    E8M0 scale bytes of quantize_mxfp8 (q, k: axis 0; v: axis 1).  Returns
    (o bf16, lse)."""
    _check_fp8_codes(q8, k8, v8)
    B, Sq, Hq, d = q8.shape
    Sk, Hkv = k8.shape[1], k8.shape[2]
    for name, t, shape in (("q_scale", q_scale, (B, Sq, Hq, d // 32)),
                           ("k_scale", k_scale, (B, Sk, Hkv, d // 32)),
                           ("v_scale", v_scale, (B, Hkv, (Sk + 31) // 32, d))):
        _shape(name, t, shape, torch.uint8)
        _need(t.is_contiguous(), f"{name} must be contiguous")
    if out is None:
        out = torch.empty((B, Sq, Hq, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q8.device)
    _shape("out", out, q8.shape, torch.bfloat16)
    _lse("lse", lse, (B, Hq, Sq))
    _on_device(q8.device, q8=q8, k8=k8, v8=v8, q_scale=q_scale, k_scale=k_scale,
               v_scale=v_scale, out=out, lse=lse)
    a = FwdMxfp8Args(B, Sq, Sk, Hq, Hkv, d, int(bool(causal)), _scale(d, scale),
                     _t4(q8), _t4(k8), _t4(v8), _t4(out), lse.data_ptr(), q_scale.data_ptr(),
                     k_scale.data_ptr(), v_scale.data_ptr())
    _check("fa_fwd_mxfp8", lib().fa_fwd_mxfp8(ctypes.byref(a), _stream()))
    return out, lse


def attention_fp8(q8, k8, v8, descales, causal=False, scale=None):
    """FP8 forward (no backward); descales = (q_descale, k_descale, v_descale).
    Returns o [B,Sq,Hq,d] bf16."""
    return fwd_fp8(q8, k8, v8, *descales, causal=causal, scale=scale)[0]


def attention_decode(q, k, v, causal=False, scale=None):
    """Forward for KV-cache decoding (few query rows against a long cache);
    returns o [B,Sq,Hq,d]."""
    return fwd_decode(q, k, v, causal, scale)[0]


class _AttentionVarlen(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, cu_q, cu_k, max_q, max_k, causal, scale):
        o, lse = fwd_varlen(q, k, v, cu_q, cu_k, max_q, max_k, causal, scale)
        ctx.save_for_backward(q, k, v, o, lse, cu_q, cu_k)
        ctx.meta = (max_q, max_k, causal, scale)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse, cu_q, cu_k = ctx.saved_tensors
        max_q, max_k, causal, scale = ctx.meta
        dq, dk, dv = bwd_varlen(q, k, v, o, do.contiguous(), lse, cu_q, cu_k, max_q, max_k,
                                causal, scale)
        return dq, dk, dv, None, None, None, None, None, None


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                     causal=False, scale=None):
    """Packed variable-length attention with autograd: q [Tq,Hq,d], k/v
    [Tk,Hkv,d] bf16, cu_seqlens_* int32 [nseq+1]; returns o [Tq,Hq,d]."""
    return _AttentionVarlen.apply(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                                  max_seqlen_k, causal, scale)
