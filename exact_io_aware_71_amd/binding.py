"""ctypes binding of libexact_attn.so: argument marshalling only.

Every step of attention runs in the HIP library; this module only checks tensor metadata,
passes raw device pointers, sizes and the current HIP stream, and turns non-OK status codes
into exceptions.  It fails loudly when the library has not been built — there is no
fallback path.

Function names match the C entry points declared in include/attn.h.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libexact_attn.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = range(5)
ATTN_F32, ATTN_BF16 = 0, 1

EXPORTS = (
    "attn_abi_version", "attn_status_str", "attn_last_error", "attn_fwd", "attn_fwd_kv", "attn_fwd_varlen",
    "attn_fwd_blocksparse",
    "attn_bwd_workspace_bytes", "attn_bwd", "attn_bwd_varlen_workspace_bytes", "attn_bwd_varlen",
    "attn_bwd_blocksparse", "attn_decode_auto_splits",
    "attn_decode_workspace_bytes", "attn_decode", "attn_decode_noalloc", "attn_decode_varlen",
    "attn_decode_multi_workspace_bytes", "attn_decode_multi",
)

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status


_STATUS_NAMES = {1: "ATTN_ERR_INVALID_ARG", 2: "ATTN_ERR_UNSUPPORTED", 3: "ATTN_ERR_WORKSPACE", 4: "ATTN_ERR_HIP"}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library once; raises if it is missing (build it with exact_io_aware_71_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m exact_io_aware_71_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_abi_version.restype = i
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_status_str.argtypes = [i]
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_fwd.restype = i
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    lib.attn_fwd_kv.restype = i
    lib.attn_fwd_kv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp]
    lib.attn_fwd_blocksparse.restype = i
    lib.attn_fwd_blocksparse.argtypes = [vp] * 6 + [ctypes.c_longlong, ctypes.c_longlong] + [i] * 8 + [f, vp]
    lib.attn_fwd_varlen.restype = i
    lib.attn_fwd_varlen.argtypes = [vp] * 7 + [i, i, i, i, i, i, i, i, i, f, vp]
    lib.attn_bwd_workspace_bytes.restype = sz
    lib.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.attn_bwd.restype = i
    lib.attn_bwd.argtypes = [vp] * 9 + [i, i, i, i, i, i, i, f, vp, sz, vp]
    lib.attn_bwd_blocksparse.restype = i
    lib.attn_bwd_blocksparse.argtypes = [vp] * 10 + [ctypes.c_longlong, ctypes.c_longlong] + [i] * 7 + [f, vp, sz, vp]
    lib.attn_bwd_varlen_workspace_bytes.restype = sz
    lib.attn_bwd_varlen_workspace_bytes.argtypes = [i, i, i]
    lib.attn_bwd_varlen.restype = i
    lib.attn_bwd_varlen.argtypes = [vp] * 11 + [i] * 10 + [f, vp, sz, vp]
    lib.attn_decode_auto_splits.restype = i
    lib.attn_decode_auto_splits.argtypes = [i, i, i, i, i]
    lib.attn_decode_workspace_bytes.restype = sz
    lib.attn_decode_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.attn_decode.restype = i
    lib.attn_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.attn_decode_noalloc.restype = i
    lib.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.attn_decode_multi_workspace_bytes.restype = sz
    lib.attn_decode_multi_workspace_bytes.argtypes = [i] * 7
    lib.attn_decode_multi.restype = i
    lib.attn_decode_multi.argtypes = [vp] * 6 + [i] * 8 + [f, i, vp, sz, vp]
    lib.attn_decode_varlen.restype = i
    lib.attn_decode_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz, vp]
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != ATTN_OK:
        raise AttnError(status, load().attn_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def attn_fwd(q, k, v, causal: bool, scale: float, o=None, lse=None, want_lse: bool = True, stream=None):
    """O (and LSE [B,Hq,N] fp32) for q [B,Hq,N,d], k/v [B,Hkv,N,d] on the GPU."""
    import torch
    lib = load()
    _require(q.is_cuda and q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "q, k, v must be 4-D CUDA tensors")
    _require(all(t.is_contiguous() for t in (q, k, v)), "q, k, v must be contiguous")
    _require(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    _require(tuple(k.shape) == (B, Hkv, N, d) and tuple(v.shape) == (B, Hkv, N, d), "k/v shape mismatch")
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _check(lib.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d, _dtype_code(q),
                        int(bool(causal)), float(scale), _stream(stream)))
    return o, lse


def attn_fwd_kv(q, k, v, causal: bool, scale: float, o=None, lse=None, want_lse: bool = True, stream=None):
    """q [B,Hq,Nq,d] against k/v [B,Hkv,Nk,d]; causal masks are aligned at the bottom right
    (query i sees keys j <= i + Nk - Nq)."""
    import torch
    lib = load()
    _require(q.is_cuda and q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "q, k, v must be 4-D CUDA tensors")
    _require(all(t.is_contiguous() for t in (q, k, v)), "q, k, v must be contiguous")
    _require(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _require(tuple(k.shape) == (B, Hkv, Nk, d) and tuple(v.shape) == (B, Hkv, Nk, d), "k/v shape mismatch")
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _check(lib.attn_fwd_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, _dtype_code(q),
                           int(bool(causal)), float(scale), _stream(stream)))
    return o, lse


SPARSE_BLOCK = 128


def attn_fwd_blocksparse(q, k, v, block_mask, causal: bool, scale: float, o=None, lse=None, want_lse: bool = True,
                         stream=None):
    """attn_fwd_kv restricted to the 128x128 (query block, key block) pairs block_mask keeps.
    block_mask: uint8 CUDA tensor [B, Hq, nqb, nkb], [Hq, nqb, nkb] or [nqb, nkb] (shared over
    the missing leading dims), nqb = ceil(Nq/128), nkb = ceil(Nk/128); the last two dims dense."""
    import torch
    lib = load()
    _require(q.is_cuda and q.dim() == 4 and k.dim() == 4 and v.dim() == 4, "q, k, v must be 4-D CUDA tensors")
    _require(all(t.is_contiguous() for t in (q, k, v)), "q, k, v must be contiguous")
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _require(tuple(k.shape) == (B, Hkv, Nk, d) and tuple(v.shape) == (B, Hkv, Nk, d), "k/v shape mismatch")
    nqb, nkb = -(-Nq // SPARSE_BLOCK), -(-Nk // SPARSE_BLOCK)
    m = block_mask
    _require(m.is_cuda and m.dtype == torch.uint8 and 2 <= m.dim() <= 4, "block_mask must be a uint8 CUDA tensor")
    _require(tuple(m.shape[-2:]) == (nqb, nkb), f"block_mask must end in [{nqb}, {nkb}]")
    _require(m.stride(-1) == 1 and m.stride(-2) == nkb, "block_mask rows must be dense")
    sb = m.stride(0) if m.dim() == 4 else 0
    sh = m.stride(-3) if m.dim() >= 3 else 0
    if m.dim() == 4:
        _require(m.shape[0] in (1, B), "block_mask batch dim must be 1 or B")
        sb = 0 if m.shape[0] == 1 else sb
    if m.dim() >= 3:
        _require(m.shape[-3] in (1, Hq), "block_mask head dim must be 1 or Hq")
        sh = 0 if m.shape[-3] == 1 else sh
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _check(lib.attn_fwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(m), sb, sh, B, Hq, Hkv, Nq,
                                    Nk, d, _dtype_code(q), int(bool(causal)), float(scale), _stream(stream)))
    return o, lse


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, causal: bool, scale: float, o=None,
                    lse=None, want_lse: bool = True, stream=None):
    """Packed variable-length forward: q [Hq,total_q,d], k/v [Hkv,total_k,d]; sequence b owns rows
    cu_seqlens_q[b]..cu_seqlens_q[b+1]-1 of q (likewise for k/v); int32 offsets on the device."""
    import torch
    lib = load()
    _require(q.dim() == 3 and k.dim() == 3 and v.dim() == 3, "q [Hq,total_q,d], k/v [Hkv,total_k,d]")
    for t in (q, k, v, cu_seqlens_q, cu_seqlens_k):
        _require(t.is_cuda and t.is_contiguous(), "inputs must be contiguous CUDA tensors")
    _require(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    Hq, total_q, d = q.shape
    Hkv, total_k = k.shape[0], k.shape[1]
    _require(tuple(v.shape) == tuple(k.shape) and k.shape[2] == d, "k/v shape mismatch")
    _require(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_k.dtype == torch.int32, "cu_seqlens must be int32")
    _require(cu_seqlens_q.dim() == 1 and cu_seqlens_q.shape == cu_seqlens_k.shape and cu_seqlens_q.numel() >= 2,
             "cu_seqlens must be [B+1]")
    B = cu_seqlens_q.numel() - 1
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    _check(lib.attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens_q),
                               _ptr(cu_seqlens_k), B, Hq, Hkv, total_q, total_k, int(max_seqlen_q), d,
                               _dtype_code(q), int(bool(causal)), float(scale), _stream(stream)))
    return o, lse


def attn_bwd_workspace_bytes(B, Hq, Hkv, N, d) -> int:
    return int(load().attn_bwd_workspace_bytes(B, Hq, Hkv, N, d))


def attn_bwd(q, k, v, o, lse, dout, causal: bool, scale: float, dq=None, dk=None, dv=None, workspace=None,
             stream=None):
    """dQ, dK, dV by recomputation from the forward's O and LSE."""
    import torch
    lib = load()
    for t in (q, k, v, o, lse, dout):
        _require(t.is_cuda and t.is_contiguous(), "all inputs must be contiguous CUDA tensors")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    _require(tuple(lse.shape) == (B, Hq, N) and lse.dtype == torch.float32, "lse must be fp32 [B,Hq,N]")
    _require(tuple(dout.shape) == tuple(q.shape) and tuple(o.shape) == tuple(q.shape), "o/dout shape mismatch")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = attn_bwd_workspace_bytes(B, Hq, Hkv, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                        B, Hq, Hkv, N, d, _dtype_code(q), int(bool(causal)), float(scale), _ptr(workspace),
                        workspace.numel() * workspace.element_size(), _stream(stream)))
    return dq, dk, dv


def _mask_strides(m, B, Hq, nqb, nkb):
    """Validated byte strides (batch, head) of a uint8 block mask [B|1, Hq|1, nqb, nkb] or a
    lower-rank broadcast of it."""
    import torch
    _require(m.is_cuda and m.dtype == torch.uint8 and 2 <= m.dim() <= 4, "block_mask must be a uint8 CUDA tensor")
    _require(tuple(m.shape[-2:]) == (nqb, nkb), f"block_mask must end in [{nqb}, {nkb}]")
    _require(m.stride(-1) == 1 and m.stride(-2) == nkb, "block_mask rows must be dense")
    sb = sh = 0
    if m.dim() == 4:
        _require(m.shape[0] in (1, B), "block_mask batch dim must be 1 or B")
        sb = 0 if m.shape[0] == 1 else m.stride(0)
    if m.dim() >= 3:
        _require(m.shape[-3] in (1, Hq), "block_mask head dim must be 1 or Hq")
        sh = 0 if m.shape[-3] == 1 else m.stride(-3)
    return sb, sh


def attn_bwd_blocksparse(q, k, v, o, lse, dout, block_mask, causal: bool, scale: float, dq=None, dk=None, dv=None,
                         workspace=None, stream=None):
    """Backward of attn_fwd_blocksparse for square attention (q/k/v [B,H,N,d])."""
    import torch
    lib = load()
    for t in (q, k, v, o, lse, dout):
        _require(t.is_cuda and t.is_contiguous(), "all inputs must be contiguous CUDA tensors")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    _require(tuple(k.shape) == (B, Hkv, N, d) == tuple(v.shape), "k/v shape mismatch (square attention only)")
    _require(tuple(lse.shape) == (B, Hq, N) and lse.dtype == torch.float32, "lse must be fp32 [B,Hq,N]")
    nb = -(-N // SPARSE_BLOCK)
    sb, sh = _mask_strides(block_mask, B, Hq, nb, nb)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = attn_bwd_workspace_bytes(B, Hq, Hkv, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.attn_bwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                                    _ptr(dv), _ptr(block_mask), sb, sh, B, Hq, Hkv, N, d, _dtype_code(q),
                                    int(bool(causal)), float(scale), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(stream)))
    return dq, dk, dv


def attn_bwd_varlen_workspace_bytes(B, Hq, total_q) -> int:
    return int(load().attn_bwd_varlen_workspace_bytes(B, Hq, total_q))


def attn_bwd_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                    causal: bool, scale: float, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Packed variable-length backward: q/o/dout [Hq,total_q,d], k/v [Hkv,total_k,d],
    lse [Hq,total_q] fp32, int32 offsets [B+1] on the device."""
    import torch
    lib = load()
    for t in (q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k):
        _require(t.is_cuda and t.is_contiguous(), "all inputs must be contiguous CUDA tensors")
    _require(q.dim() == 3 and k.dim() == 3 and tuple(v.shape) == tuple(k.shape), "q [Hq,total_q,d], k/v [Hkv,total_k,d]")
    Hq, total_q, d = q.shape
    Hkv, total_k = k.shape[0], k.shape[1]
    _require(tuple(o.shape) == tuple(q.shape) == tuple(dout.shape), "o/dout shape mismatch")
    _require(tuple(lse.shape) == (Hq, total_q) and lse.dtype == torch.float32, "lse must be fp32 [Hq,total_q]")
    _require(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_k.dtype == torch.int32, "cu_seqlens must be int32")
    _require(cu_seqlens_q.dim() == 1 and cu_seqlens_q.shape == cu_seqlens_k.shape and cu_seqlens_q.numel() >= 2,
             "cu_seqlens must be [B+1]")
    B = cu_seqlens_q.numel() - 1
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = attn_bwd_varlen_workspace_bytes(B, Hq, total_q)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                               _ptr(dv), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, Hq, Hkv, total_q, total_k,
                               int(max_seqlen_q), int(max_seqlen_k), d, _dtype_code(q), int(bool(causal)),
                               float(scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _stream(stream)))
    return dq, dk, dv


def attn_decode_auto_splits(B, Hq, Hkv, L, d) -> int:
    return int(load().attn_decode_auto_splits(B, Hq, Hkv, L, d))


def attn_decode_workspace_bytes(B, Hq, Hkv, L, d, num_splits=0) -> int:
    return int(load().attn_decode_workspace_bytes(B, Hq, Hkv, L, d, num_splits))


def attn_decode(q, k_cache, v_cache, scale: float, num_splits: int = 0, o=None, lse=None, want_lse=True,
                workspace=None, stream=None):
    """Single-token decode: q [B,Hq,d] against caches [B,Hkv,L,d]."""
    import torch
    lib = load()
    _require(q.dim() == 3 and k_cache.dim() == 4 and v_cache.dim() == 4, "q [B,Hq,d], caches [B,Hkv,L,d]")
    for t in (q, k_cache, v_cache):
        _require(t.is_cuda and t.is_contiguous(), "inputs must be contiguous CUDA tensors")
    B, Hq, d = q.shape
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    _require(tuple(k_cache.shape) == (B, Hkv, L, d) == tuple(v_cache.shape), "cache shape mismatch")
    o = torch.empty_like(q) if o is None else o
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = attn_decode_workspace_bytes(B, Hq, Hkv, L, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), B, Hq, Hkv, L, d,
                           _dtype_code(q), float(scale), int(num_splits), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(stream)))
    return o, lse


# Scratch the library holds per GPU for attn_decode_noalloc (ATTN_DECODE_NOALLOC_SCRATCH_BYTES).
DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20


def attn_decode_noalloc(q, k_cache, v_cache, scale: float, num_splits: int = 0, o=None, lse=None, want_lse=True,
                        stream=None):
    """attn_decode with no workspace: the split partials go to the library's own scratch array.
    With o (and lse) given, nothing is allocated on the device."""
    import torch
    lib = load()
    _require(q.dim() == 3 and k_cache.dim() == 4 and v_cache.dim() == 4, "q [B,Hq,d], caches [B,Hkv,L,d]")
    for t in (q, k_cache, v_cache):
        _require(t.is_cuda and t.is_contiguous(), "inputs must be contiguous CUDA tensors")
    B, Hq, d = q.shape
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    _require(tuple(k_cache.shape) == (B, Hkv, L, d) == tuple(v_cache.shape), "cache shape mismatch")
    o = torch.empty_like(q) if o is None else o
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check(lib.attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), B, Hq, Hkv, L, d,
                                   _dtype_code(q), float(scale), int(num_splits), _stream(stream)))
    return o, lse


def attn_decode_varlen(q, k_cache, v_cache, seqlens, scale: float, num_splits: int = 0, o=None, lse=None,
                       want_lse=True, workspace=None, stream=None):
    """attn_decode where sequence b attends to its first seqlens[b] cached keys (int32 [B], on
    the device)."""
    import torch
    lib = load()
    _require(q.dim() == 3 and k_cache.dim() == 4 and v_cache.dim() == 4, "q [B,Hq,d], caches [B,Hkv,L,d]")
    for t in (q, k_cache, v_cache, seqlens):
        _require(t.is_cuda and t.is_contiguous(), "inputs must be contiguous CUDA tensors")
    B, Hq, d = q.shape
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    _require(tuple(k_cache.shape) == (B, Hkv, L, d) == tuple(v_cache.shape), "cache shape mismatch")
    _require(tuple(seqlens.shape) == (B,) and seqlens.dtype == torch.int32, "seqlens must be int32 [B]")
    o = torch.empty_like(q) if o is None else o
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = attn_decode_workspace_bytes(B, Hq, Hkv, L, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.attn_decode_varlen(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o), _ptr(lse), B, Hq,
                                  Hkv, L, d, _dtype_code(q), float(scale), int(num_splits), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))
    return o, lse


def attn_decode_multi_workspace_bytes(B, Hq, Hkv, T, L, d, num_splits=0) -> int:
    return int(load().attn_decode_multi_workspace_bytes(B, Hq, Hkv, T, L, d, num_splits))


def attn_decode_multi(q, k_cache, v_cache, scale: float, causal: bool = True, seqlens=None, num_splits: int = 0,
                      o=None, lse=None, want_lse=True, workspace=None, stream=None):
    """T tokens per sequence: q [B,Hq,T,d] against caches [B,Hkv,L,d] (optional int32 seqlens [B]);
    causal: token t sees keys j <= len - T + t."""
    import torch
    lib = load()
    _require(q.dim() == 4 and k_cache.dim() == 4 and v_cache.dim() == 4, "q [B,Hq,T,d], caches [B,Hkv,L,d]")
    for t in (q, k_cache, v_cache) + (() if seqlens is None else (seqlens,)):
        _require(t.is_cuda and t.is_contiguous(), "inputs must be contiguous CUDA tensors")
    B, Hq, T, d = q.shape
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    _require(tuple(k_cache.shape) == (B, Hkv, L, d) == tuple(v_cache.shape), "cache shape mismatch")
    if seqlens is not None:
        _require(tuple(seqlens.shape) == (B,) and seqlens.dtype == torch.int32, "seqlens must be int32 [B]")
    o = torch.empty_like(q) if o is None else o
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    need = attn_decode_multi_workspace_bytes(B, Hq, Hkv, T, L, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.attn_decode_multi(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                 T, L, d, _dtype_code(q), int(bool(causal)), float(scale), int(num_splits),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))
    return o, lse
