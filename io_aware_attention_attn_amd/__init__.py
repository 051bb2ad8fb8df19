"""Python binding of libfa.so, the MI355X (gfx950) FlashAttention forward library.

The C ABI is declared in ``include/fa.h``.  This module only marshals arguments:
it checks what it needs to read sizes off torch tensors, allocates outputs and
workspace with torch (device memory plumbing, allocated in the stream order of the
stream the kernels run on), passes raw device pointers and that stream (default:
torch's current stream), and turns a negative status into ``ValueError``.  Every step
of the computation runs in the library's HIP kernels; there is no fallback path.

Functions (same names as the C entry points):
  fa_forward(q, k, v, scale=None, causal=False, o=None, lse=None, stream=None)
  fa_forward_f32(q, k, v, scale=None, causal=False, o=None, lse=None, stream=None)
  fa_forward_fp8(q8, k8, v8, q_descale, k_descale, v_descale, scale=None, causal=False, o=None,
                 lse=None, stream=None)
  fa_forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                    scale=None, causal=False, o=None, lse=None, stream=None)
  fa_backward_workspace_bytes(B, Hq, Nq)
  fa_backward(q, k, v, o, lse, dout, scale=None, causal=False, dq=None, dk=None, dv=None,
              workspace=None, stream=None)
  fa_decode_splitkv_workspace_bytes(B, Hq, Nk_max, d, chunk=256)
  fa_decode_splitkv(q, k_cache, v_cache, seqlens_k, scale=None, chunk=256, o=None,
                    lse=None, workspace=None, stream=None)
  fa_decode_splitkv_noalloc(q, k_cache, v_cache, seqlens_k, scale=None, chunk=256, o, lse,
                            stream=None)
  fa_decode_paged(q, k_pages, v_pages, block_table, seqlens_k, scale=None, chunk=256,
                  o=None, lse=None, workspace=None, stream=None)
  fa_status_str(status)
  fa_probe_mfma_bf16_operand_bytes(blocks), fa_probe_mfma_bf16(operands, out, blocks, iters,
                     stream=None)   (measurement helper: the matrix cores' sustained rate)
  fa_probe_stream_read(buf, out, blocks, stream=None)
                        (measurement helper: the HBM streaming-read rate)

Allocation helper (not a C entry point; torch device memory only):
  kv_cache_empty(shape, device=None) -> (k_cache, v_cache)
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")

FA_OK = 0
FA_ERR_NULL = -1
FA_ERR_SHAPE = -2
FA_ERR_UNSUPPORTED = -3
FA_ERR_ALIGN = -4
FA_ERR_WORKSPACE = -5
FA_ERR_HIP = -6
FA_ERR_SCRATCH = -7

_lib = None


class FAError(ValueError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_str(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load libfa.so (raises if it has not been built; there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m io_aware_attention_attn_amd._build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.fa_forward.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    L.fa_forward.restype = i
    L.fa_forward_f32.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    L.fa_forward_f32.restype = i
    L.fa_forward_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, f, f, f, vp]
    L.fa_forward_fp8.restype = i
    L.fa_forward_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i,
                                    i, i, i, vp]
    L.fa_forward_varlen.restype = i
    L.fa_backward_workspace_bytes.argtypes = [i, i, i]
    L.fa_backward_workspace_bytes.restype = sz
    L.fa_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz,
                              vp]
    L.fa_backward.restype = i
    L.fa_decode_splitkv_workspace_bytes.argtypes = [i, i, i, i, i]
    L.fa_decode_splitkv_workspace_bytes.restype = sz
    L.fa_decode_splitkv.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    L.fa_decode_splitkv.restype = i
    L.fa_decode_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.fa_decode_splitkv_noalloc.restype = i
    L.fa_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    L.fa_decode_paged.restype = i
    L.fa_status_str.argtypes = [i]
    L.fa_status_str.restype = ctypes.c_char_p
    L.fa_probe_mfma_bf16_operand_bytes.argtypes = [i]
    L.fa_probe_mfma_bf16_operand_bytes.restype = sz
    L.fa_probe_mfma_bf16.argtypes = [vp, sz, vp, i, i, vp]
    L.fa_probe_mfma_bf16.restype = i
    L.fa_probe_stream_read.argtypes = [vp, sz, vp, i, vp]
    L.fa_probe_stream_read.restype = i
    _lib = L
    return L


def fa_status_str(status: int) -> str:
    return lib().fa_status_str(int(status)).decode()


def fa_probe_mfma_bf16_operand_bytes(blocks: int) -> int:
    return int(lib().fa_probe_mfma_bf16_operand_bytes(int(blocks)))


def fa_probe_mfma_bf16(operands, out, blocks: int, iters: int, stream=None):
    """Measurement helper: `blocks` x 256 threads of independent bf16 32x32x16 MFMAs on
    the operands in `operands` (a device tensor of at least
    fa_probe_mfma_bf16_operand_bytes(blocks) bytes), each thread's accumulator sum to
    `out` (float32, blocks * 256).  Returns the FLOP count of the launch."""
    import torch
    if not isinstance(operands, torch.Tensor) or not operands.is_cuda:
        raise ValueError("operands must be a CUDA tensor")
    _check_tensor(out, "out", torch.float32, 1)
    if out.numel() < int(blocks) * 256:
        raise ValueError("out is too small")
    ts = _torch_stream(stream)
    st = lib().fa_probe_mfma_bf16(_ptr(operands), operands.numel() * operands.element_size(),
                                  _ptr(out), int(blocks), int(iters), int(ts.cuda_stream))
    if st != FA_OK:
        raise FAError(st, "fa_probe_mfma_bf16")
    return int(blocks) * 4 * int(iters) * 4 * 32768


def fa_probe_stream_read(buf, out, blocks: int, stream=None):
    """Measurement helper: `blocks` x 256 threads read every byte of `buf` (a contiguous
    device tensor, 16-byte aligned, size a multiple of 16 bytes, at most 2^31) once and
    write per-thread XORs of the 32-bit words read to `out` (int32, blocks * 256).
    Returns the number of bytes read."""
    import torch
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous CUDA tensor")
    _check_tensor(out, "out", torch.int32, 1)
    if out.numel() < int(blocks) * 256:
        raise ValueError("out is too small")
    nbytes = buf.numel() * buf.element_size()
    ts = _torch_stream(stream)
    st = lib().fa_probe_stream_read(_ptr(buf), nbytes, _ptr(out), int(blocks),
                                    int(ts.cuda_stream))
    if st != FA_OK:
        raise FAError(st, "fa_probe_stream_read")
    return nbytes


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _torch_stream(stream):
    """The torch stream object for ``stream`` (None = the current stream; a raw
    hipStream_t handle is wrapped without taking ownership)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _empty(shape, dtype, device, ts):
    """Uninitialised device memory allocated in the stream order of ``ts``, the stream
    the kernels will run on: when the tensor is freed (a workspace when the call
    returns), torch's caching allocator hands the block only to later work ordered
    after the kernels on that stream."""
    import torch
    with torch.cuda.stream(ts):
        return torch.empty(shape, dtype=dtype, device=device)


def _check_tensor(t, name, dtype, ndim):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _forward(entry, q, k, v, scale, causal, o, lse, stream, dtype) -> Tuple:
    import torch
    _check_tensor(q, "q", dtype, 4)
    _check_tensor(k, "k", dtype, 4)
    _check_tensor(v, "v", dtype, 4)
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ts = _torch_stream(stream)
    if o is None:
        o = _empty((B, Nq, Hq, d), torch.float32, q.device, ts)
    if lse is None:
        lse = _empty((B, Hq, Nq), torch.float32, q.device, ts)
    _check_tensor(o, "o", torch.float32, 4)
    _check_tensor(lse, "lse", torch.float32, 3)
    if tuple(o.shape) != (B, Nq, Hq, d) or tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("o / lse have the wrong shape")
    st = entry(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
               float(scale), 1 if causal else 0, int(ts.cuda_stream))
    if st != FA_OK:
        raise FAError(st, entry.__name__)
    return o, lse


def fa_forward(q, k, v, scale: Optional[float] = None, causal: bool = False, o=None, lse=None,
               stream=None):
    """bf16 q [B,Nq,Hq,d], k/v [B,Nk,Hkv,d] -> (O fp32 [B,Nq,Hq,d], LSE fp32 [B,Hq,Nq])."""
    import torch
    return _forward(lib().fa_forward, q, k, v, scale, causal, o, lse, stream, torch.bfloat16)


def fa_forward_f32(q, k, v, scale: Optional[float] = None, causal: bool = False, o=None,
                   lse=None, stream=None):
    """fp32 variant of fa_forward (no 16-bit rounding anywhere)."""
    import torch
    return _forward(lib().fa_forward_f32, q, k, v, scale, causal, o, lse, stream, torch.float32)


def fa_forward_fp8(q8, k8, v8, q_descale: float, k_descale: float, v_descale: float,
                   scale: Optional[float] = None, causal: bool = False, o=None, lse=None,
                   stream=None):
    """torch.float8_e4m3fn q8 [B,Nq,Hq,d], k8/v8 [B,Nk,Hkv,d] with per-tensor descales
    (value = code * descale) -> (O fp32 [B,Nq,Hq,d], LSE fp32 [B,Hq,Nq])."""
    import torch
    for t, n in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        _check_tensor(t, n, torch.float8_e4m3fn, 4)
    B, Nq, Hq, d = q8.shape
    Bk, Nk, Hkv, dk = k8.shape
    if tuple(v8.shape) != tuple(k8.shape) or Bk != B or dk != d:
        raise ValueError(f"shape mismatch: q {tuple(q8.shape)} k {tuple(k8.shape)} v {tuple(v8.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ts = _torch_stream(stream)
    if o is None:
        o = _empty((B, Nq, Hq, d), torch.float32, q8.device, ts)
    if lse is None:
        lse = _empty((B, Hq, Nq), torch.float32, q8.device, ts)
    _check_tensor(o, "o", torch.float32, 4)
    _check_tensor(lse, "lse", torch.float32, 3)
    if tuple(o.shape) != (B, Nq, Hq, d) or tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("o / lse have the wrong shape")
    st = lib().fa_forward_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq,
                              Nk, d, float(scale), 1 if causal else 0, float(q_descale),
                              float(k_descale), float(v_descale), int(ts.cuda_stream))
    if st != FA_OK:
        raise FAError(st, "fa_forward_fp8")
    return o, lse


def _check_token_rows(t, name):
    """[total, H, d] bf16 GPU tensor whose tokens may be strided (a view of a packed
    QKV tensor) but whose heads and head dims are dense."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != torch.bfloat16 or t.dim() != 3 or not t.is_cuda:
        raise ValueError(f"{name} must be a 3-dim bf16 GPU tensor, got {t.dtype} {tuple(t.shape)}")
    if t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name}: heads and head dims must be dense (strides {t.stride()})")


def fa_forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                      max_seqlen_k: int, scale: Optional[float] = None, causal: bool = False, o=None, lse=None,
                      stream=None):
    """Packed variable-length batch: q bf16 [total_q,Hq,d], k/v bf16 [total_k,Hkv,d] (token
    stride free, e.g. views of one QKV tensor), cu_seqlens_q/k int32 [B+1] on the GPU
    -> (O fp32 [total_q,Hq,d], LSE fp32 [Hq,total_q])."""
    import torch
    _check_token_rows(q, "q")
    _check_token_rows(k, "k")
    _check_token_rows(v, "v")
    _check_tensor(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    _check_tensor(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    total_q, Hq, d = q.shape
    total_k, Hkv, dk = k.shape
    B = cu_seqlens_q.shape[0] - 1
    if (tuple(v.shape) != tuple(k.shape) or dk != d or cu_seqlens_k.shape[0] != B + 1
            or v.stride(0) != k.stride(0)):
        raise ValueError(f"varlen shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} "
                         f"v {tuple(v.shape)} cu {B + 1}/{cu_seqlens_k.shape[0]}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ts = _torch_stream(stream)
    if o is None:
        o = _empty((total_q, Hq, d), torch.float32, q.device, ts)
    if lse is None:
        lse = _empty((Hq, total_q), torch.float32, q.device, ts)
    _check_tensor(o, "o", torch.float32, 3)
    _check_tensor(lse, "lse", torch.float32, 2)
    if tuple(o.shape) != (total_q, Hq, d) or tuple(lse.shape) != (Hq, total_q):
        raise ValueError("o / lse have the wrong shape")
    st = lib().fa_forward_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens_q),
                                 _ptr(cu_seqlens_k), B, Hq, Hkv, int(max_seqlen_q),
                                 int(max_seqlen_k), total_q,
                                 total_k, d, float(scale), 1 if causal else 0, q.stride(0),
                                 k.stride(0), v.stride(0), int(ts.cuda_stream))
    if st != FA_OK:
        raise FAError(st, "fa_forward_varlen")
    return o, lse


def fa_backward_workspace_bytes(B: int, Hq: int, Nq: int) -> int:
    return int(lib().fa_backward_workspace_bytes(B, Hq, Nq))


def fa_backward(q, k, v, o, lse, dout, scale: Optional[float] = None, causal: bool = False,
                dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients of fa_forward: bf16 q/dout [B,Nq,Hq,d], k/v [B,Nk,Hkv,d]; the forward's
    fp32 o [B,Nq,Hq,d] and lse [B,Hq,Nq] -> (dq fp32 [B,Nq,Hq,d], dk, dv fp32 [B,Nk,Hkv,d])."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (dout, "dout")):
        _check_tensor(t, n, torch.bfloat16, 4)
    _check_tensor(o, "o", torch.float32, 4)
    _check_tensor(lse, "lse", torch.float32, 3)
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk_ = k.shape
    if (tuple(v.shape) != tuple(k.shape) or Bk != B or dk_ != d or tuple(o.shape) != tuple(q.shape)
            or tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, Nq)):
        raise ValueError("backward shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ts = _torch_stream(stream)
    if dq is None:
        dq = _empty((B, Nq, Hq, d), torch.float32, q.device, ts)
    if dk is None:
        dk = _empty((B, Nk, Hkv, d), torch.float32, q.device, ts)
    if dv is None:
        dv = _empty((B, Nk, Hkv, d), torch.float32, q.device, ts)
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check_tensor(t, n, torch.float32, 4)
    if tuple(dq.shape) != tuple(q.shape) or tuple(dk.shape) != tuple(k.shape) or tuple(dv.shape) != tuple(k.shape):
        raise ValueError("dq / dk / dv have the wrong shape")
    need = fa_backward_workspace_bytes(B, Hq, Nq)
    if workspace is None:
        workspace = _empty((max(need, 1),), torch.uint8, q.device, ts)
    st = lib().fa_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                           _ptr(dk), _ptr(dv), B, Hq, Hkv, Nq, Nk, d, float(scale),
                           1 if causal else 0, _ptr(workspace),
                           int(workspace.numel() * workspace.element_size()), int(ts.cuda_stream))
    if st != FA_OK:
        raise FAError(st, "fa_backward")
    return dq, dk, dv


# Start of the V cache relative to the K cache, modulo 1 KiB, that kv_cache_empty sets up.
KV_V_OFFSET_MOD_1K = 256


def kv_cache_empty(shape, device=None, dtype=None):
    """Uninitialised bf16 K and V caches of ``shape`` ([B, Nk_max, Hkv, d] for
    fa_decode_splitkv, [num_pages, page_size, Hkv, d] for fa_decode_paged) carved out of
    one allocation, with the V cache starting 256 bytes past a 1 KiB boundary relative to
    the K cache.

    The K row and the V row of one token and head are always V_start - K_start bytes
    apart, and the decode kernels read a head's K and V rows at the same time.  When the
    two caches start at addresses congruent modulo 1 KiB (two separate allocations, which
    are 2 MiB aligned), those reads fall in the same 256-byte address class and the
    split kernel streams about 5% slower on MI355X (measured: 253 us against 240 us on
    the 16-sequence GQA decode).  Any other offset modulo 1 KiB is as fast; 256 is used.
    """
    import torch
    dtype = torch.bfloat16 if dtype is None else dtype
    shape = tuple(int(x) for x in shape)
    nbytes = math.prod(shape) * torch.empty((), dtype=dtype).element_size()
    pad = (KV_V_OFFSET_MOD_1K - nbytes) % 1024  # V start = nbytes + pad = 256 (mod 1 KiB)
    buf = torch.empty(2 * nbytes + pad, dtype=torch.uint8, device=device)
    k = buf[:nbytes].view(dtype).view(shape)
    v = buf[nbytes + pad:nbytes + pad + nbytes].view(dtype).view(shape)
    return k, v


def fa_decode_splitkv_workspace_bytes(B: int, Hq: int, Nk_max: int, d: int, chunk: int = 256) -> int:
    return int(lib().fa_decode_splitkv_workspace_bytes(B, Hq, Nk_max, d, chunk))


def fa_decode_splitkv(q, k_cache, v_cache, seqlens_k, scale: Optional[float] = None,
                      chunk: int = 256, o=None, lse=None, workspace=None, stream=None):
    """q bf16 [B,Hq,d]; caches bf16 [B,Nk_max,Hkv,d]; seqlens_k int32 [B] on the GPU
    -> (O fp32 [B,Hq,d], LSE fp32 [B,Hq])."""
    import torch
    _check_tensor(q, "q", torch.bfloat16, 3)
    _check_tensor(k_cache, "k_cache", torch.bfloat16, 4)
    _check_tensor(v_cache, "v_cache", torch.bfloat16, 4)
    _check_tensor(seqlens_k, "seqlens_k", torch.int32, 1)
    B, Hq, d = q.shape
    Bc, Nk_max, Hkv, dc = k_cache.shape
    if tuple(v_cache.shape) != tuple(k_cache.shape) or Bc != B or dc != d or seqlens_k.shape[0] != B:
        raise ValueError("decode shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ts = _torch_stream(stream)
    if o is None:
        o = _empty((B, Hq, d), torch.float32, q.device, ts)
    if lse is None:
        lse = _empty((B, Hq), torch.float32, q.device, ts)
    need = fa_decode_splitkv_workspace_bytes(B, Hq, Nk_max, d, chunk)
    if workspace is None:
        workspace = _empty((max(need, 1),), torch.uint8, q.device, ts)
    st = lib().fa_decode_splitkv(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens_k), _ptr(o),
                                 _ptr(lse), B, Hq, Hkv, Nk_max, d, float(scale), int(chunk),
                                 _ptr(workspace), int(workspace.numel() * workspace.element_size()),
                                 int(ts.cuda_stream))
    if st != FA_OK:
        raise FAError(st, "fa_decode_splitkv")
    return o, lse


def fa_decode_splitkv_noalloc(q, k_cache, v_cache, seqlens_k, o, lse,
                              scale: Optional[float] = None, chunk: int = 256, stream=None):
    """fa_decode_splitkv without a workspace: the library's fixed per-GPU device scratch
    holds the partial results, and nothing is allocated (the caller passes o fp32 [B,Hq,d]
    and lse fp32 [B,Hq]).  Calls that overlap in time on one GPU race on that scratch.
    Raises FAError (FA_ERR_SCRATCH) when the request does not fit it."""
    import torch
    _check_tensor(q, "q", torch.bfloat16, 3)
    _check_tensor(k_cache, "k_cache", torch.bfloat16, 4)
    _check_tensor(v_cache, "v_cache", torch.bfloat16, 4)
    _check_tensor(seqlens_k, "seqlens_k", torch.int32, 1)
    _check_tensor(o, "o", torch.float32, 3)
    _check_tensor(lse, "lse", torch.float32, 2)
    B, Hq, d = q.shape
    Bc, Nk_max, Hkv, dc = k_cache.shape
    if (tuple(v_cache.shape) != tuple(k_cache.shape) or Bc != B or dc != d
            or seqlens_k.shape[0] != B or tuple(o.shape) != (B, Hq, d) or tuple(lse.shape) != (B, Hq)):
        raise ValueError("decode shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib().fa_decode_splitkv_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens_k),
                                         _ptr(o), _ptr(lse), B, Hq, Hkv, Nk_max, d, float(scale),
                                         int(chunk), int(_torch_stream(stream).cuda_stream))
    if st != FA_OK:
        raise FAError(st, "fa_decode_splitkv_noalloc")
    return o, lse


def fa_decode_paged(q, k_pages, v_pages, block_table, seqlens_k, scale: Optional[float] = None,
                    chunk: int = 256, o=None, lse=None, workspace=None, stream=None):
    """q bf16 [B,Hq,d]; page pools bf16 [num_pages,page_size,Hkv,d]; block_table int32
    [B,max_pages] and seqlens_k int32 [B] on the GPU -> (O fp32 [B,Hq,d], LSE fp32 [B,Hq])."""
    import torch
    _check_tensor(q, "q", torch.bfloat16, 3)
    _check_tensor(k_pages, "k_pages", torch.bfloat16, 4)
    _check_tensor(v_pages, "v_pages", torch.bfloat16, 4)
    _check_tensor(block_table, "block_table", torch.int32, 2)
    _check_tensor(seqlens_k, "seqlens_k", torch.int32, 1)
    B, Hq, d = q.shape
    num_pages, page_size, Hkv, dc = k_pages.shape
    max_pages = block_table.shape[1]
    if (tuple(v_pages.shape) != tuple(k_pages.shape) or dc != d or seqlens_k.shape[0] != B
            or block_table.shape[0] != B):
        raise ValueError("paged decode shape mismatch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    ts = _torch_stream(stream)
    if o is None:
        o = _empty((B, Hq, d), torch.float32, q.device, ts)
    if lse is None:
        lse = _empty((B, Hq), torch.float32, q.device, ts)
    need = fa_decode_splitkv_workspace_bytes(B, Hq, max_pages * page_size, d, chunk)
    if workspace is None:
        workspace = _empty((max(need, 1),), torch.uint8, q.device, ts)
    st = lib().fa_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                               _ptr(seqlens_k), _ptr(o), _ptr(lse), B, Hq, Hkv, num_pages,
                               page_size, max_pages, d, float(scale), int(chunk), _ptr(workspace),
                               int(workspace.numel() * workspace.element_size()), int(ts.cuda_stream))
    if st != FA_OK:
        raise FAError(st, "fa_decode_paged")
    return o, lse
