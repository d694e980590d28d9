"""ctypes binding of ``libattn.so`` (the C ABI declared in ``include/attn.h``).

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind the C ABI.  Torch supplies device memory and the current
stream.  There is no fallback: if the library is missing or a call fails,
``AttnError`` is raised.
"""
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, 1, 2, 3
ATTN_F32, ATTN_BF16, ATTN_FP8_E4M3 = 0, 1, 2
ATTN_P_E4M3, ATTN_P_E4M3_LEAN = 1, 2

# every symbol include/attn.h declares
EXPORTED = ("attn_fwd", "attn_fwd_fp8", "attn_fwd_partial", "attn_merge", "attn_splitkv_workspace_bytes",
            "attn_fwd_splitkv", "attn_fwd_splitkv_noalloc", "attn_quantize_fp8", "attn_fwd_fp8_blocks", "attn_bwd_workspace_bytes", "attn_bwd", "attn_fwd_fp8_p", "attn_fwd_exp_poly",
            "attn_status_string",
            "attn_last_error", "attn_version")


class AttnError(RuntimeError):
    """A failed call into the attention library (or the library is missing)."""

    def __init__(self, status, msg):
        super().__init__(msg)
        self.status = status


_lib = None


def lib():
    """Load ``libattn.so`` once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise AttnError(-1, f"{LIB_PATH} is missing: build it with `python -m exact_io_aware_attn_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, ci, cf = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, cf, ci, vp]
    L.attn_fwd.restype = ci
    L.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, cf, vp, vp, vp, vp]
    L.attn_fwd_fp8.restype = ci
    L.attn_fwd_partial.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, cf, ci, i64, i64,
                                   vp, vp, vp, vp]
    L.attn_fwd_partial.restype = ci
    L.attn_merge.argtypes = [vp, vp, i64, vp, vp, i64, i64, i64, i64, ci, vp]
    L.attn_merge.restype = ci
    L.attn_splitkv_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    L.attn_splitkv_workspace_bytes.restype = ctypes.c_size_t
    L.attn_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, cf, ci, vp, vp, vp,
                                   i64, vp, ctypes.c_size_t, vp]
    L.attn_fwd_splitkv.restype = ci
    L.attn_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, cf, ci, vp, vp, vp,
                                           i64, vp]
    L.attn_fwd_splitkv_noalloc.restype = ci
    L.attn_quantize_fp8.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp, vp]
    L.attn_quantize_fp8.restype = ci
    L.attn_fwd_fp8_blocks.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, cf, vp, vp, vp, vp]
    L.attn_fwd_fp8_blocks.restype = ci
    L.attn_fwd_exp_poly.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, cf, vp]
    L.attn_fwd_exp_poly.restype = ci
    L.attn_fwd_fp8_p.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ci, cf, vp, vp, vp, ci, vp]
    L.attn_fwd_fp8_p.restype = ci
    L.attn_bwd_workspace_bytes.argtypes = [i64, i64, i64]
    L.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.attn_bwd.argtypes = [vp] * 9 + [i64] * 6 + [ci, cf, ci, vp, ctypes.c_size_t, vp]
    L.attn_bwd.restype = ci
    L.attn_status_string.argtypes = [ci]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_last_error.argtypes = []
    L.attn_last_error.restype = ctypes.c_char_p
    L.attn_version.argtypes = []
    L.attn_version.restype = ci
    _lib = L
    return L


def _check(status):
    if status != ATTN_OK:
        L = lib()
        raise AttnError(status, f"{L.attn_status_string(status).decode()}: {L.attn_last_error().decode()}")


def raw_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, causal, scale, dtype, stream=0):
    """Call ``attn_fwd`` with raw integer pointers; returns the status code."""
    return lib().attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, int(causal), float(scale), int(dtype), stream)


def raw_fwd_fp8(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, causal, scale, dq, dk, dv, stream=0):
    """Call ``attn_fwd_fp8`` with raw integer pointers; returns the status code."""
    return lib().attn_fwd_fp8(q, k, v, o, lse, B, Hq, Hkv, Nq, Nkv, D, int(causal), float(scale), dq, dk, dv,
                              stream)


def _shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D (B, H, N, D)")
    B, Hq, Nq, D = q.shape
    Bk, Hkv, Nkv, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
    return B, Hq, Hkv, Nq, Nkv, D


def _buffer(t, name, shape, dtype, device):
    """A caller-supplied output buffer, checked before any kernel writes it:
    exactly ``shape`` and ``dtype``, contiguous, on ``device``.  ``None``
    allocates one."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _workspace(ws, need, device):
    """A caller-supplied workspace of at least ``need`` bytes on ``device``
    (contiguous), or a new one."""
    if ws is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    if not isinstance(ws, torch.Tensor) or ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, {need} needed")
    return ws


def _stream_ptr(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def fwd(q, k, v, causal=False, scale=None, out=None, lse=None, return_lse=True, stream=None):
    """Exact attention forward on the GPU.

    q: (B, Hq, Nq, D), k/v: (B, Hkv, Nkv, D); dtype float32 or bfloat16.
    Returns (o, lse): o has q's dtype, lse is float32 (B, Hq, Nq) (None if
    ``return_lse`` is False).  ``scale`` defaults to 1/sqrt(D).
    """
    B, Hq, Hkv, Nq, Nkv, D = _shapes(q, k, v)
    if q.dtype == torch.float32:
        dt = ATTN_F32
    elif q.dtype == torch.bfloat16:
        dt = ATTN_BF16
    else:
        raise ValueError(f"unsupported dtype {q.dtype} (use fwd_fp8 for e4m3)")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = _buffer(out, "out", (B, Hq, Nq, D), q.dtype, q.device)
    if lse is not None or return_lse:
        lse = _buffer(lse, "lse", (B, Hq, Nq), torch.float32, q.device)
    _check(raw_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                   lse.data_ptr() if lse is not None else None,
                   B, Hq, Hkv, Nq, Nkv, D, causal, scale, dt, _stream_ptr(stream)))
    return out, lse


def fwd_fp8(q, k, v, descale_q=None, descale_k=None, descale_v=None, causal=False, scale=None, out=None,
            lse=None, return_lse=True, stream=None):
    """Exact attention forward on per-tensor-scaled e4m3fn inputs (bf16 out).

    q/k/v: ``torch.float8_e4m3fn`` device tensors; descales: one-element
    float32 device tensors (or None for 1.0).  ``scale`` defaults to 1/sqrt(D).
    """
    B, Hq, Hkv, Nq, Nkv, D = _shapes(q, k, v)
    for t in (q, k, v):
        if t.dtype != torch.float8_e4m3fn:
            raise ValueError("fwd_fp8 takes torch.float8_e4m3fn tensors")
    ptrs = []
    for d in (descale_q, descale_k, descale_v):
        if d is None:
            ptrs.append(None)
            continue
        if d.dtype != torch.float32 or not d.is_cuda or d.numel() < 1:
            raise ValueError("descales must be float32 device tensors with one element")
        ptrs.append(d.data_ptr())
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = _buffer(out, "out", (B, Hq, Nq, D), torch.bfloat16, q.device)
    if lse is not None or return_lse:
        lse = _buffer(lse, "lse", (B, Hq, Nq), torch.float32, q.device)
    _check(raw_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                       lse.data_ptr() if lse is not None else None,
                       B, Hq, Hkv, Nq, Nkv, D, causal, scale, *ptrs, _stream_ptr(stream)))
    return out, lse


def _dtype_code(q, k, v):
    if q.dtype == torch.float32:
        dt = ATTN_F32
    elif q.dtype == torch.bfloat16:
        dt = ATTN_BF16
    elif q.dtype == torch.float8_e4m3fn:
        dt = ATTN_FP8_E4M3
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    return dt


def _descale_ptrs(dt, descales):
    if descales is None:
        return [None, None, None]
    if dt != ATTN_FP8_E4M3:
        raise ValueError("descales apply to float8_e4m3fn inputs only")
    ptrs = []
    for d in descales:
        if d is None:
            ptrs.append(None)
            continue
        if d.dtype != torch.float32 or not d.is_cuda or d.numel() < 1:
            raise ValueError("descales must be float32 device tensors with one element")
        ptrs.append(d.data_ptr())
    return ptrs


def fwd_partial(q, k, v, kv_begin, kv_end, causal=False, scale=None, descales=None, stream=None):
    """Attention of q over the keys kv_begin <= j < kv_end of k/v (the whole
    sequence's causal alignment).  ``descales``: (dq, dk, dv) one-element
    float32 device tensors for e4m3 inputs, or None.  Returns float32
    (o_part, lse_part)."""
    B, Hq, Hkv, Nq, Nkv, D = _shapes(q, k, v)
    dt = _dtype_code(q, k, v)
    dptr = _descale_ptrs(dt, descales)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty((B, Hq, Nq, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _check(lib().attn_fwd_partial(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  B, Hq, Hkv, Nq, Nkv, D, int(causal), float(scale), dt, int(kv_begin), int(kv_end),
                                  *dptr, _stream_ptr(stream)))
    return o, lse


def merge(o_parts, lse_parts, out_dtype=torch.bfloat16, return_lse=True, stream=None):
    """Merge float32 partial results (P, B, Hq, Nq, D) / (P, B, Hq, Nq) by LSE."""
    if o_parts.dim() != 5 or lse_parts.dim() != 4 or tuple(o_parts.shape[:4]) != tuple(lse_parts.shape):
        raise ValueError("o_parts must be (P, B, Hq, Nq, D) and lse_parts (P, B, Hq, Nq)")
    for t in (o_parts, lse_parts):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("partial results must be contiguous float32 device tensors")
    P, B, Hq, Nq, D = o_parts.shape
    code = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16}.get(out_dtype)
    if code is None:
        raise ValueError("out_dtype must be float32 or bfloat16")
    o = torch.empty((B, Hq, Nq, D), dtype=out_dtype, device=o_parts.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=o_parts.device) if return_lse else None
    _check(lib().attn_merge(o_parts.data_ptr(), lse_parts.data_ptr(), P, o.data_ptr(),
                            lse.data_ptr() if lse is not None else None, B, Hq, Nq, D, code, _stream_ptr(stream)))
    return o, lse


def splitkv_workspace_bytes(B, Hq, Nq, D, n_splits):
    return int(lib().attn_splitkv_workspace_bytes(B, Hq, Nq, D, n_splits))


def fwd_splitkv(q, k, v, n_splits, causal=False, scale=None, descales=None, workspace=None, out=None, lse=None,
                stream=None):
    """``fwd`` (or ``fwd_fp8`` with ``descales``) computed as ``n_splits`` key
    ranges in one launch plus a merge.

    ``workspace``: optional uint8 device tensor of at least
    ``splitkv_workspace_bytes`` bytes (allocated here by torch otherwise).
    Returns (o, lse) like ``fwd``.
    """
    B, Hq, Hkv, Nq, Nkv, D = _shapes(q, k, v)
    dt = _dtype_code(q, k, v)
    dptr = _descale_ptrs(dt, descales)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = splitkv_workspace_bytes(B, Hq, Nq, D, n_splits)
    workspace = _workspace(workspace, need, q.device)
    o = _buffer(out, "out", (B, Hq, Nq, D), torch.float32 if dt == ATTN_F32 else torch.bfloat16, q.device)
    lse = _buffer(lse, "lse", (B, Hq, Nq), torch.float32, q.device)
    _check(lib().attn_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  B, Hq, Hkv, Nq, Nkv, D, int(causal), float(scale), dt, *dptr, int(n_splits),
                                  workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  _stream_ptr(stream)))
    return o, lse


NOALLOC_SCRATCH_BYTES = 64 << 20  # ATTN_NOALLOC_SCRATCH_BYTES of include/attn.h


def fwd_splitkv_noalloc(q, k, v, n_splits, causal=False, scale=None, descales=None, out=None, lse=None,
                        stream=None):
    """``fwd_splitkv`` through ``attn_fwd_splitkv_noalloc``: the partial
    results live in the library's fixed per-GPU scratch area, so the C call
    allocates nothing (``out`` and ``lse`` are allocated here unless given).
    Calls that overlap on one GPU race on that area."""
    B, Hq, Hkv, Nq, Nkv, D = _shapes(q, k, v)
    dt = _dtype_code(q, k, v)
    dptr = _descale_ptrs(dt, descales)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = _buffer(out, "out", (B, Hq, Nq, D), torch.float32 if dt == ATTN_F32 else torch.bfloat16, q.device)
    lse = _buffer(lse, "lse", (B, Hq, Nq), torch.float32, q.device)
    _check(lib().attn_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                          B, Hq, Hkv, Nq, Nkv, D, int(causal), float(scale), dt, *dptr,
                                          int(n_splits), _stream_ptr(stream)))
    return o, lse

def quantize_fp8(x, signs=None, codes=None, descales=None, stream=None):
    """Block e4m3 quantisation of a bf16 (B, H, N, D) device tensor, one
    descale per 64 rows, rows rotated by diag(signs) H_D / sqrt(D) first if
    ``signs`` (an int8 device tensor of D values +-1) is given.  Returns
    (codes as torch.float8_e4m3fn, descales float32 (B, H, ceil(N/64)))."""
    if x.dim() != 4 or x.dtype != torch.bfloat16 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous bfloat16 (B, H, N, D) device tensor")
    B, H, N, D = x.shape
    sp = None
    if signs is not None:
        if signs.dtype != torch.int8 or not signs.is_cuda or signs.numel() != D:
            raise ValueError("signs must be an int8 device tensor of D values")
        sp = signs.data_ptr()
    codes = _buffer(codes, "codes", (B, H, N, D), torch.float8_e4m3fn, x.device)
    descales = _buffer(descales, "descales", (B, H, (N + 63) // 64), torch.float32, x.device)
    desc = descales
    _check(lib().attn_quantize_fp8(x.data_ptr(), codes.data_ptr(), desc.data_ptr(), B, H, N, D, sp,
                                   _stream_ptr(stream)))
    return codes, desc


def fwd_fp8_blocks(q, k, v, dq_blocks, dk_blocks, dv_blocks, causal=False, scale=None, out=None, lse=None,
                   return_lse=True, stream=None):
    """Exact attention on e4m3 inputs with one descale per 64-row block (the
    layout ``quantize_fp8`` returns).  bf16 output, float32 LSE."""
    B, Hq, Hkv, Nq, Nkv, D = _shapes(q, k, v)
    for t in (q, k, v):
        if t.dtype != torch.float8_e4m3fn:
            raise ValueError("fwd_fp8_blocks takes torch.float8_e4m3fn tensors")
    for d, H, N in ((dq_blocks, Hq, Nq), (dk_blocks, Hkv, Nkv), (dv_blocks, Hkv, Nkv)):
        if d.dtype != torch.float32 or not d.is_cuda or tuple(d.shape) != (B, H, (N + 63) // 64):
            raise ValueError("block descales must be float32 device tensors of shape (B, H, ceil(N/64))")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = _buffer(out, "out", (B, Hq, Nq, D), torch.bfloat16, q.device)
    if lse is not None or return_lse:
        lse = _buffer(lse, "lse", (B, Hq, Nq), torch.float32, q.device)
    _check(lib().attn_fwd_fp8_blocks(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     lse.data_ptr() if lse is not None else None, B, Hq, Hkv, Nq, Nkv, D,
                                     int(causal), float(scale), dq_blocks.data_ptr(), dk_blocks.data_ptr(),
                                     dv_blocks.data_ptr(), _stream_ptr(stream)))
    return out, lse


def bwd_workspace_bytes(B, Hq, Nq):
    return int(lib().attn_bwd_workspace_bytes(B, Hq, Nq))


def bwd(q, k, v, o, lse, dout, causal=False, scale=None, workspace=None, dq=None, dk=None, dv=None, stream=None):
    """Gradients (dq, dk, dv) of bf16 attention given the forward outputs o
    and lse (natural log) and the upstream gradient dout."""
    B, Hq, Hkv, Nq, Nkv, D = _shapes(q, k, v)
    for t in (q, k, v, o, dout):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("bwd takes contiguous bfloat16 device tensors")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o and dout must have q's shape")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Nq) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 (B, Hq, Nq) tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    for t in (o, lse, dout):
        if t.device != q.device:
            raise ValueError("o, lse and dout must be on q's device")
    need = bwd_workspace_bytes(B, Hq, Nq)
    workspace = _workspace(workspace, need, q.device)
    dq = _buffer(dq, "dq", tuple(q.shape), torch.bfloat16, q.device)
    dk = _buffer(dk, "dk", tuple(k.shape), torch.bfloat16, q.device)
    dv = _buffer(dv, "dv", tuple(v.shape), torch.bfloat16, q.device)
    _check(lib().attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                          dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Nq, Nkv, D, int(causal),
                          float(scale), ATTN_BF16, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                          _stream_ptr(stream)))
    return dq, dk, dv


def fwd_fp8_p(q, k, v, descale_q=None, descale_k=None, descale_v=None, causal=False, scale=None, lean=False,
              out=None, lse=None, return_lse=True, stream=None):
    """e4m3 attention with e4m3 probabilities (both products on the fp8
    matrix instruction); ``lean`` selects Lean P codes.  bf16 O, fp32 LSE."""
    B, Hq, Hkv, Nq, Nkv, D = _shapes(q, k, v)
    for t in (q, k, v):
        if t.dtype != torch.float8_e4m3fn:
            raise ValueError("fwd_fp8_p takes torch.float8_e4m3fn tensors")
    ptrs = []
    for d in (descale_q, descale_k, descale_v):
        if d is None:
            ptrs.append(None)
            continue
        if d.dtype != torch.float32 or not d.is_cuda or d.numel() < 1:
            raise ValueError("descales must be float32 device tensors with one element")
        ptrs.append(d.data_ptr())
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = _buffer(out, "out", (B, Hq, Nq, D), torch.bfloat16, q.device)
    if lse is not None or return_lse:
        lse = _buffer(lse, "lse", (B, Hq, Nq), torch.float32, q.device)
    _check(lib().attn_fwd_fp8_p(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                lse.data_ptr() if lse is not None else None, B, Hq, Hkv, Nq, Nkv, D, int(causal),
                                float(scale), *ptrs, ATTN_P_E4M3_LEAN if lean else ATTN_P_E4M3, _stream_ptr(stream)))
    return out, lse


def fwd_exp_poly(q, k, v, causal=False, scale=None, out=None, lse=None, return_lse=True, stream=None):
    """bf16 attention with the probabilities' exponentials from a cubic
    polynomial (relative error <= 8.6e-5) instead of the transcendental unit."""
    B, Hq, Hkv, Nq, Nkv, D = _shapes(q, k, v)
    for t in (q, k, v):
        if t.dtype != torch.bfloat16:
            raise ValueError("fwd_exp_poly takes bfloat16 tensors")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = _buffer(out, "out", (B, Hq, Nq, D), torch.bfloat16, q.device)
    if lse is not None or return_lse:
        lse = _buffer(lse, "lse", (B, Hq, Nq), torch.float32, q.device)
    _check(lib().attn_fwd_exp_poly(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                   lse.data_ptr() if lse is not None else None, B, Hq, Hkv, Nq, Nkv, D, int(causal),
                                   float(scale), _stream_ptr(stream)))
    return out, lse
