"""Python binding of libhca.so: HCA / DSA attention (forward, decode upkeep, backward) for MI355X (gfx950).

Each function here has the name of the C entry point it wraps and only
marshals arguments: it reads device pointers, strides and sizes from torch
tensors, allocates outputs and workspaces with torch when the caller does not
pass them, and calls the library on the current HIP stream.  All arithmetic
runs in the HIP kernels of libhca.so.  Without the built library (or without a
GPU) every call raises; there is no CPU fallback.

Layouts follow the C header ``include/hca.h``: tensors are
[batch, seq, head, dim] with the dim axis contiguous.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhca.so")

HCA_OK, HCA_ERR_INVALID, HCA_ERR_UNSUPPORTED, HCA_ERR_WORKSPACE, HCA_ERR_HIP = range(5)
HCA_DTYPE_F32, HCA_DTYPE_BF16 = 0, 1

EXPORTS = (
    "hca_abi_version", "hca_last_error", "hca_compress_kv", "hca_append_kv", "hca_attn_fwd_workspace_size",
    "hca_attn_fwd", "dsa_index_topk_workspace_size", "dsa_index_topk", "dsa_sparse_attn_fwd",
    "dsa_index_topk_decode_workspace_size", "dsa_index_topk_decode", "dsa_sparse_attn_decode",
    "dsa_sparse_attn_decode_workspace_size",
    "hca_attn_bwd_workspace_size", "hca_attn_bwd", "hca_compress_kv_bwd", "hca_attn_compress_bwd",
    "dsa_sparse_attn_bwd_workspace_size", "dsa_sparse_attn_bwd",
    "csa_index_topk_workspace_size", "csa_index_topk", "csa_sparse_attn_fwd", "attn_output_epilogue",
    "hca_attn_fwd_noalloc",
)


class HcaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


class Strides(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seq", ctypes.c_int64), ("head", ctypes.c_int64)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libhca.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libhca.so not found at {path}; build it with `python -m sparse_attention_hca_amd.build`")
    lib = ctypes.CDLL(path)
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    S = Strides
    lib.hca_abi_version.restype = I
    lib.hca_abi_version.argtypes = []
    lib.hca_last_error.restype = ctypes.c_char_p
    lib.hca_last_error.argtypes = []
    lib.hca_compress_kv.restype = I
    lib.hca_compress_kv.argtypes = [I, P, S, P, S, P, P, P, S, P, S, I, I, I, I, I, P]
    lib.hca_append_kv.restype = I
    lib.hca_append_kv.argtypes = [I, P, S, P, S, P, S, P, S, I, P, P, P, S, P, S, I, I64, I, I, I, I, P]
    lib.hca_attn_fwd_workspace_size.restype = SZ
    lib.hca_attn_fwd_workspace_size.argtypes = [I, I, I, I, I, I, I]
    lib.hca_attn_fwd.restype = I
    lib.hca_attn_fwd.argtypes = [I, P, S, P, S, P, S, P, S, P, S, P, S, P,
                                 I, I, I64, I, I64, I, I, I, I, I, I, F, P, SZ, P]
    lib.hca_attn_fwd_noalloc.restype = I
    lib.hca_attn_fwd_noalloc.argtypes = [I, P, S, P, S, P, S, P, S, P, S, P, S, P,
                                         I, I, I64, I, I64, I, I, I, I, I, I, F, P]
    lib.dsa_index_topk_workspace_size.restype = SZ
    lib.dsa_index_topk_workspace_size.argtypes = [I, I, I]
    lib.dsa_index_topk.restype = I
    lib.dsa_index_topk.argtypes = [P, P, P, P, I, I, I, I, I, P, SZ, P]
    lib.dsa_sparse_attn_fwd.restype = I
    lib.dsa_sparse_attn_fwd.argtypes = [I, P, S, P, S, P, S, P, P, S, P, I, I, I, I, I, I, I, F, P]
    lib.dsa_index_topk_decode_workspace_size.restype = SZ
    lib.dsa_index_topk_decode_workspace_size.argtypes = [I, I, I]
    lib.dsa_index_topk_decode.restype = I
    lib.dsa_index_topk_decode.argtypes = [P, P, P, P, I, I, I, I, I, P, SZ, P]
    lib.dsa_sparse_attn_decode.restype = I
    lib.dsa_sparse_attn_decode.argtypes = [I, P, S, P, S, P, S, P, P, S, P, I, I, I, I, I, I, I, F, P, SZ, P]
    lib.dsa_sparse_attn_decode_workspace_size.restype = SZ
    lib.dsa_sparse_attn_decode_workspace_size.argtypes = [I, I, I]
    lib.csa_index_topk_workspace_size.restype = SZ
    lib.csa_index_topk_workspace_size.argtypes = [I, I, I, I]
    lib.csa_index_topk.restype = I
    lib.csa_index_topk.argtypes = [P, P, P, P, I, I, I, I, I, I, I, P, SZ, P]
    lib.csa_sparse_attn_fwd.restype = I
    lib.csa_sparse_attn_fwd.argtypes = [I, P, S, P, S, P, S, P, P, S, P, I, I, I, I, I, I, I, I, F, P]
    lib.attn_output_epilogue.restype = I
    lib.attn_output_epilogue.argtypes = [I, P, S, P, S, P, P, P, P, S, I, I, I, I, I, I, P]
    lib.hca_attn_bwd_workspace_size.restype = SZ
    lib.hca_attn_bwd_workspace_size.argtypes = [I, I, I, I64, I, I, I, I, I, I]
    lib.hca_attn_bwd.restype = I
    lib.hca_attn_bwd.argtypes = [I, P, S, P, S, P, S, P, S, P, S, P, S, P, P, S, P, S, P, S, P, S, P, S, P, S,
                                 I, I, I64, I, I64, I, I, I, I, I, I, F, P, SZ, P]
    lib.hca_attn_compress_bwd.restype = I
    lib.hca_attn_compress_bwd.argtypes = [I, P, S, P, S, P, S, P, S, P, S, P, S, P, P, S, P, P, P, S, P, S, P, S,
                                          P, S, P, S, P, P, I, I, I, I, I, I, I, I, F, P, SZ, P]
    lib.hca_compress_kv_bwd.restype = I
    lib.hca_compress_kv_bwd.argtypes = [I, P, S, P, S, P, S, P, S, P, P, P, S, P, S, P, P, I, I, I, I, I, P]
    lib.dsa_sparse_attn_bwd_workspace_size.restype = SZ
    lib.dsa_sparse_attn_bwd_workspace_size.argtypes = [I, I, I, I, I, I, I, I]
    lib.dsa_sparse_attn_bwd.restype = I
    lib.dsa_sparse_attn_bwd.argtypes = [I, P, S, P, S, P, S, P, P, S, P, P, S, P, S, P, S, P, S,
                                        I, I, I, I, I, I, I, F, P, SZ, P]
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != HCA_OK:
        raise HcaError(status, load_library().hca_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return HCA_DTYPE_BF16
    if t.dtype == torch.float32:
        return HCA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _strides(t: torch.Tensor) -> Strides:
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [batch, seq, head, dim] tensor with a contiguous dim axis")
    return Strides(t.stride(0), t.stride(1), t.stride(2))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def hca_abi_version() -> int:
    return load_library().hca_abi_version()


def hca_last_error() -> str:
    return load_library().hca_last_error().decode()


def hca_compress_kv(k: torch.Tensor, v: torch.Tensor, w_k: torch.Tensor, w_v: torch.Tensor, block: int,
                    kc: Optional[torch.Tensor] = None, vc: Optional[torch.Tensor] = None
                    ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Weighted block compression of K and V: returns (kc, vc) [B, S // block, H_kv, d]."""
    lib = load_library()
    _dev(k, v, w_k, w_v)
    B, S, H, d = k.shape
    nb = S // block
    if kc is None:
        kc = torch.empty((B, nb, H, d), dtype=k.dtype, device=k.device)
    if vc is None:
        vc = torch.empty((B, nb, H, d), dtype=v.dtype, device=v.device)
    w_k = w_k.contiguous()
    w_v = w_v.contiguous()
    _check(lib.hca_compress_kv(_dt(k), _ptr(k), _strides(k), _ptr(v), _strides(v), _ptr(w_k), _ptr(w_v),
                               _ptr(kc), _strides(kc), _ptr(vc), _strides(vc), B, S, H, d, block, _stream()))
    return kc, vc


def hca_append_kv(k_new: torch.Tensor, v_new: torch.Tensor, k_ring: torch.Tensor, v_ring: torch.Tensor,
                  t: int, block: int, w_k: Optional[torch.Tensor] = None, w_v: Optional[torch.Tensor] = None,
                  kc: Optional[torch.Tensor] = None, vc: Optional[torch.Tensor] = None) -> None:
    """Append the K/V rows of position t ([B, 1, H_kv, d]) to the mirrored rings ([B, 2R, H_kv, d]);
    when t closes a block, write its compressed row into kc/vc ([B, n_blocks, H_kv, d])."""
    lib = load_library()
    _dev(k_new, v_new, k_ring, v_ring)
    B, _, H, d = k_new.shape
    ring = k_ring.shape[1] // 2
    n_blocks = 0 if kc is None else kc.shape[1]
    if w_k is not None:
        w_k = w_k.contiguous()
    if w_v is not None:
        w_v = w_v.contiguous()
    _check(lib.hca_append_kv(_dt(k_new), _ptr(k_new), _strides(k_new), _ptr(v_new), _strides(v_new),
                             _ptr(k_ring), _strides(k_ring), _ptr(v_ring), _strides(v_ring), ring,
                             _ptr(w_k), _ptr(w_v), _ptr(kc), _strides(kc) if kc is not None else Strides(0, 0, 0),
                             _ptr(vc), _strides(vc) if vc is not None else Strides(0, 0, 0), n_blocks, t,
                             B, H, d, block, _stream()))


def hca_attn_fwd_workspace_size(batch: int, seqlen_q: int, h_q: int, h_kv: int, head_dim: int,
                                n_blocks: int, window: int) -> int:
    return load_library().hca_attn_fwd_workspace_size(batch, seqlen_q, h_q, h_kv, head_dim, n_blocks, window)


def hca_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kc: Optional[torch.Tensor],
                 vc: Optional[torch.Tensor], *, window: int, block: int, scale: Optional[float] = None,
                 q_pos0: int = 0, kv_pos0: int = 0, o: Optional[torch.Tensor] = None, return_lse: bool = True,
                 lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None
                 ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """HCA attention over compressed entries plus the raw window; returns (o, lse)."""
    lib = load_library()
    _dev(q, k, v, kc, vc)
    B, Sq, Hq, d = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    nb = 0 if kc is None else kc.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty((B, Sq, Hq, v.shape[3]), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    wsz = lib.hca_attn_fwd_workspace_size(B, Sq, Hq, Hkv, d, nb, window)
    if workspace is None and wsz:
        workspace = torch.empty(wsz, dtype=torch.uint8, device=q.device)
    zs = Strides(0, 0, 0)
    _check(lib.hca_attn_fwd(_dt(q), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
                            _ptr(kc), zs if kc is None else _strides(kc), _ptr(vc), zs if vc is None else _strides(vc),
                            _ptr(o), _strides(o), _ptr(lse), B, Sq, q_pos0, Skv, kv_pos0, nb, Hq, Hkv, d, block,
                            window, float(scale), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                            _stream()))
    return o, lse


HCA_NOALLOC_SCRATCH_BYTES = 16 << 20   # the fixed scratch array of hca_attn_fwd_noalloc (include/hca.h)


def hca_attn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kc: Optional[torch.Tensor],
                         vc: Optional[torch.Tensor], o: torch.Tensor, lse: Optional[torch.Tensor], *, window: int,
                         block: int, scale: Optional[float] = None, q_pos0: int = 0, kv_pos0: int = 0) -> None:
    """hca_attn_fwd writing into the given o (and lse, may be None) with the
    library's fixed scratch array instead of a workspace; allocates nothing."""
    lib = load_library()
    _dev(q, k, v, kc, vc, o, lse)
    B, Sq, Hq, d = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    nb = 0 if kc is None else kc.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    zs = Strides(0, 0, 0)
    _check(lib.hca_attn_fwd_noalloc(_dt(q), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
                                    _ptr(kc), zs if kc is None else _strides(kc), _ptr(vc),
                                    zs if vc is None else _strides(vc), _ptr(o), _strides(o), _ptr(lse), B, Sq,
                                    q_pos0, Skv, kv_pos0, nb, Hq, Hkv, d, block, window, float(scale), _stream()))


def dsa_index_topk_workspace_size(batch: int, seqlen: int, topk: int) -> int:
    return load_library().dsa_index_topk_workspace_size(batch, seqlen, topk)


def dsa_index_topk(q_idx: torch.Tensor, k_idx: torch.Tensor, w_idx: torch.Tensor, topk: int,
                   idx: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """ReLU-weighted indexer + causal top-k; returns idx [B, S, topk] int32 (-1 padded, unordered)."""
    lib = load_library()
    _dev(q_idx, k_idx, w_idx)
    B, S, hi, di = q_idx.shape
    for t in (q_idx, k_idx, w_idx):
        if not t.is_contiguous() or t.dtype != torch.float32:
            raise ValueError("indexer inputs must be contiguous float32")
    if idx is None:
        idx = torch.empty((B, S, topk), dtype=torch.int32, device=q_idx.device)
    wsz = lib.dsa_index_topk_workspace_size(B, S, topk)
    if workspace is None and wsz:
        workspace = torch.empty(wsz, dtype=torch.uint8, device=q_idx.device)
    _check(lib.dsa_index_topk(_ptr(q_idx), _ptr(k_idx), _ptr(w_idx), _ptr(idx), B, S, hi, di, topk,
                              _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream()))
    return idx


def dsa_sparse_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                        scale: Optional[float] = None, o: Optional[torch.Tensor] = None, return_lse: bool = True,
                        lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Attention over the positions listed in idx (-1 skipped); returns (o, lse)."""
    lib = load_library()
    _dev(q, k, v, idx)
    B, S, Hq, dqk = q.shape
    Hkv, dv = k.shape[2], v.shape[3]
    topk = idx.shape[2]
    if not idx.is_contiguous() or idx.dtype != torch.int32:
        raise ValueError("idx must be contiguous int32 [B, S, topk]")
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if o is None:
        o = torch.empty((B, S, Hq, dv), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _check(lib.dsa_sparse_attn_fwd(_dt(q), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
                                   _ptr(idx), _ptr(o), _strides(o), _ptr(lse), B, S, Hq, Hkv, dqk, dv, topk,
                                   float(scale), _stream()))
    return o, lse


def dsa_index_topk_decode_workspace_size(batch: int, n_keys: int, topk: int) -> int:
    return load_library().dsa_index_topk_decode_workspace_size(batch, n_keys, topk)


def dsa_index_topk_decode(q_idx: torch.Tensor, k_idx: torch.Tensor, w_idx: torch.Tensor, topk: int,
                          idx: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None
                          ) -> torch.Tensor:
    """Indexer + top-k for one query per sequence (q_idx [B, 1, h_i, d_i], w_idx [B, 1, h_i]) over the
    keys k_idx [B, n_keys, d_i]; returns idx [B, 1, topk] int32 (-1 padded, unordered)."""
    lib = load_library()
    _dev(q_idx, k_idx, w_idx)
    B, _, hi, di = q_idx.shape
    n = k_idx.shape[1]
    for t in (q_idx, k_idx, w_idx):
        if not t.is_contiguous() or t.dtype != torch.float32:
            raise ValueError("indexer inputs must be contiguous float32")
    if idx is None:
        idx = torch.empty((B, 1, topk), dtype=torch.int32, device=q_idx.device)
    if workspace is None:
        workspace = torch.empty(lib.dsa_index_topk_decode_workspace_size(B, n, topk), dtype=torch.uint8,
                                device=q_idx.device)
    _check(lib.dsa_index_topk_decode(_ptr(q_idx), _ptr(k_idx), _ptr(w_idx), _ptr(idx), B, n, hi, di, topk,
                                     _ptr(workspace), workspace.numel(), _stream()))
    return idx


def dsa_sparse_attn_decode_workspace_size(batch: int, h_q: int, topk: int) -> int:
    return load_library().dsa_sparse_attn_decode_workspace_size(batch, h_q, topk)


def dsa_sparse_attn_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                           scale: Optional[float] = None, o: Optional[torch.Tensor] = None, return_lse: bool = True,
                           lse: Optional[torch.Tensor] = None, split: bool = True,
                           workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Attention of one query per sequence (q [B, 1, Hq, d]) over the positions listed in idx [B, 1, topk]
    of k, v [B, n_keys, Hkv, d]; returns (o [B, 1, Hq, dv], lse [B, Hq]).  With split (the default) the
    index row runs in slices merged by a second kernel, in `workspace` (uint8, allocated when not given)."""
    lib = load_library()
    _dev(q, k, v, idx)
    B, _, Hq, dqk = q.shape
    n, Hkv, dv = k.shape[1], k.shape[2], v.shape[3]
    topk = idx.shape[2]
    if not idx.is_contiguous() or idx.dtype != torch.int32:
        raise ValueError("idx must be contiguous int32 [B, 1, topk]")
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if o is None:
        o = torch.empty((B, 1, Hq, dv), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    ws_bytes = lib.dsa_sparse_attn_decode_workspace_size(B, Hq, topk) if split else 0
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    if not ws_bytes:
        workspace = None
    _check(lib.dsa_sparse_attn_decode(_dt(q), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
                                      _ptr(idx), _ptr(o), _strides(o), _ptr(lse), B, n, Hq, Hkv, dqk, dv, topk,
                                      float(scale), _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                      _stream()))
    return o, lse


def csa_index_topk_workspace_size(batch: int, seqlen: int, n_entries: int, topk: int) -> int:
    return load_library().csa_index_topk_workspace_size(batch, seqlen, n_entries, topk)


def csa_index_topk(q_idx: torch.Tensor, k_idx: torch.Tensor, w_idx: torch.Tensor, topk: int, block: int,
                   idx: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Indexer + top-k over the compressed entries k_idx [B, n_entries, d_i] visible to each position
    (entry j once (j + 1) * block - 1 <= t); returns idx [B, S, topk] int32 (-1 padded, unordered)."""
    lib = load_library()
    _dev(q_idx, k_idx, w_idx)
    B, S, hi, di = q_idx.shape
    n = k_idx.shape[1]
    for t in (q_idx, k_idx, w_idx):
        if not t.is_contiguous() or t.dtype != torch.float32:
            raise ValueError("indexer inputs must be contiguous float32")
    if idx is None:
        idx = torch.empty((B, S, topk), dtype=torch.int32, device=q_idx.device)
    if workspace is None:
        workspace = torch.empty(lib.csa_index_topk_workspace_size(B, S, n, topk), dtype=torch.uint8,
                                device=q_idx.device)
    _check(lib.csa_index_topk(_ptr(q_idx), _ptr(k_idx), _ptr(w_idx), _ptr(idx), B, S, n, block, hi, di, topk,
                              _ptr(workspace), workspace.numel(), _stream()))
    return idx


def csa_sparse_attn_fwd(q: torch.Tensor, kc: torch.Tensor, vc: torch.Tensor, idx: torch.Tensor,
                        scale: Optional[float] = None, o: Optional[torch.Tensor] = None, return_lse: bool = True,
                        lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Attention of q [B, S, Hq, d] over the compressed entries kc, vc [B, n_entries, Hkv, d] listed in
    idx [B, S, topk]; returns (o, lse)."""
    lib = load_library()
    _dev(q, kc, vc, idx)
    B, S, Hq, dqk = q.shape
    n, Hkv, dv = kc.shape[1], kc.shape[2], vc.shape[3]
    topk = idx.shape[2]
    if not idx.is_contiguous() or idx.dtype != torch.int32:
        raise ValueError("idx must be contiguous int32 [B, S, topk]")
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    if o is None:
        o = torch.empty((B, S, Hq, dv), dtype=q.dtype, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _check(lib.csa_sparse_attn_fwd(_dt(q), _ptr(q), _strides(q), _ptr(kc), _strides(kc), _ptr(vc), _strides(vc),
                                   _ptr(idx), _ptr(o), _strides(o), _ptr(lse), B, S, n, Hq, Hkv, dqk, dv, topk,
                                   float(scale), _stream()))
    return o, lse


def attn_output_epilogue(o: torch.Tensor, c: torch.Tensor, w_g: torch.Tensor, u: torch.Tensor, v: torch.Tensor,
                         y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = sigmoid(c w_g^T) * (o + (u v) o across heads) for o [B, S, H, d_v] and the query latent
    c [B, S, d_c] (bf16), w_g [H*d_v, d_c] (bf16), u [H, r], v [r, H] (fp32)."""
    lib = load_library()
    _dev(o, c, w_g, u, v, y)
    B, S, H, dv = o.shape
    dc = c.shape[-1]
    r = u.shape[1]
    c4 = c.reshape(B, S, 1, dc) if c.dim() == 3 else c
    w_g = w_g.contiguous()
    u = u.contiguous().float()
    v = v.contiguous().float()
    if y is None:
        y = torch.empty((B, S, H, dv), dtype=o.dtype, device=o.device)
    _check(lib.attn_output_epilogue(_dt(o), _ptr(o), _strides(o), _ptr(c4), _strides(c4), _ptr(w_g), _ptr(u), _ptr(v),
                                    _ptr(y), _strides(y), B, S, H, dv, dc, r, _stream()))
    return y


def hca_attn_bwd_workspace_size(dtype: torch.dtype, batch: int, seqlen_q: int, q_pos0: int, n_blocks: int, h_q: int,
                                h_kv: int, head_dim: int, block: int, window: int) -> int:
    dt = HCA_DTYPE_BF16 if dtype == torch.bfloat16 else HCA_DTYPE_F32
    return load_library().hca_attn_bwd_workspace_size(dt, batch, seqlen_q, q_pos0, n_blocks, h_q, h_kv, head_dim,
                                                      block, window)


def hca_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kc: Optional[torch.Tensor],
                 vc: Optional[torch.Tensor], o: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor, *, window: int,
                 block: int, scale: Optional[float] = None, q_pos0: int = 0, kv_pos0: int = 0,
                 workspace: Optional[torch.Tensor] = None):
    """Gradients of hca_attn_fwd's output given dout, the forward's o and lse:
    returns fp32 (dq, dk, dv, dkc, dvc) shaped like q, k, v, kc, vc (dkc/dvc None without entries)."""
    lib = load_library()
    _dev(q, k, v, kc, vc, o, lse, dout)
    B, Sq, Hq, d = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    nb = 0 if kc is None else kc.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, Hq, Sq]")
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty(q.shape, **f32)
    dk = torch.empty(k.shape, **f32)
    dv = torch.empty(v.shape, **f32)
    dkc = torch.empty(kc.shape, **f32) if nb else None
    dvc = torch.empty(vc.shape, **f32) if nb else None
    if workspace is None:
        workspace = torch.empty(lib.hca_attn_bwd_workspace_size(_dt(q), B, Sq, q_pos0, nb, Hq, Hkv, d, block, window),
                                dtype=torch.uint8, device=q.device)
    zs = Strides(0, 0, 0)
    st = lambda t: zs if t is None else _strides(t)
    _check(lib.hca_attn_bwd(_dt(q), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
                            _ptr(kc), st(kc), _ptr(vc), st(vc), _ptr(o), _strides(o), _ptr(lse), _ptr(dout),
                            _strides(dout), _ptr(dq), _strides(dq), _ptr(dk), _strides(dk), _ptr(dv), _strides(dv),
                            _ptr(dkc), st(dkc), _ptr(dvc), st(dvc), B, Sq, q_pos0, Skv, kv_pos0, nb, Hq, Hkv, d,
                            block, window, float(scale), _ptr(workspace), workspace.numel(), _stream()))
    return dq, dk, dv, dkc, dvc


def hca_compress_kv_bwd(k: torch.Tensor, v: torch.Tensor, dkc: torch.Tensor, dvc: torch.Tensor, w_k: torch.Tensor,
                        w_v: torch.Tensor, block: int, dk: Optional[torch.Tensor] = None,
                        dv: Optional[torch.Tensor] = None):
    """Backward of hca_compress_kv: adds w * dkc (w * dvc) into the fp32 dk (dv) over the whole blocks
    (zeros are allocated when dk/dv are not given) and returns (dk, dv, dw_k, dw_v)."""
    lib = load_library()
    _dev(k, v, dkc, dvc, w_k, w_v, dk, dv)
    B, S, H, d = k.shape
    f32 = dict(dtype=torch.float32, device=k.device)
    if dk is None:
        dk = torch.zeros(k.shape, **f32)
    if dv is None:
        dv = torch.zeros(v.shape, **f32)
    for t in (dkc, dvc, dk, dv):
        if t.dtype != torch.float32:
            raise ValueError("gradients must be float32")
    w_k = w_k.contiguous()
    w_v = w_v.contiguous()
    dw_k = torch.empty((H, block), **f32)
    dw_v = torch.empty((H, block), **f32)
    _check(lib.hca_compress_kv_bwd(_dt(k), _ptr(k), _strides(k), _ptr(v), _strides(v), _ptr(dkc), _strides(dkc),
                                   _ptr(dvc), _strides(dvc), _ptr(w_k), _ptr(w_v), _ptr(dk), _strides(dk), _ptr(dv),
                                   _strides(dv), _ptr(dw_k), _ptr(dw_v), B, S, H, d, block, _stream()))
    return dk, dv, dw_k, dw_v


def hca_attn_compress_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kc: Optional[torch.Tensor],
                          vc: Optional[torch.Tensor], o: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor,
                          w_k: torch.Tensor, w_v: torch.Tensor, *, window: int, block: int,
                          scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None):
    """Backward of compression + attention for a sequence from position 0: returns fp32
    (dq, dk, dv, dkc, dvc, dw_k, dw_v); dk/dv include the compressor's share."""
    lib = load_library()
    _dev(q, k, v, kc, vc, o, lse, dout, w_k, w_v)
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    nb = 0 if kc is None else kc.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, Hq, S]")
    w_k = w_k.contiguous()
    w_v = w_v.contiguous()
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty(q.shape, **f32)
    dk = torch.empty(k.shape, **f32)
    dv = torch.empty(v.shape, **f32)
    dkc = torch.empty(kc.shape, **f32) if nb else None
    dvc = torch.empty(vc.shape, **f32) if nb else None
    dw_k = torch.empty((Hkv, block), **f32)
    dw_v = torch.empty((Hkv, block), **f32)
    if workspace is None:
        workspace = torch.empty(lib.hca_attn_bwd_workspace_size(_dt(q), B, S, 0, nb, Hq, Hkv, d, block, window),
                                dtype=torch.uint8, device=q.device)
    zs = Strides(0, 0, 0)
    st = lambda t: zs if t is None else _strides(t)
    _check(lib.hca_attn_compress_bwd(_dt(q), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
                                     _ptr(kc), st(kc), _ptr(vc), st(vc), _ptr(o), _strides(o), _ptr(lse), _ptr(dout),
                                     _strides(dout), _ptr(w_k), _ptr(w_v), _ptr(dq), _strides(dq), _ptr(dk),
                                     _strides(dk), _ptr(dv), _strides(dv), _ptr(dkc), st(dkc), _ptr(dvc), st(dvc),
                                     _ptr(dw_k), _ptr(dw_v), B, S, nb, Hq, Hkv, d, block, window, float(scale),
                                     _ptr(workspace), workspace.numel(), _stream()))
    return dq, dk, dv, dkc, dvc, dw_k, dw_v


def dsa_sparse_attn_bwd_workspace_size(dtype: torch.dtype, batch: int, seqlen: int, h_q: int, h_kv: int, d_qk: int,
                                       d_v: int, topk: int) -> int:
    dt = HCA_DTYPE_BF16 if dtype == torch.bfloat16 else HCA_DTYPE_F32
    return load_library().dsa_sparse_attn_bwd_workspace_size(dt, batch, seqlen, h_q, h_kv, d_qk, d_v, topk)


def dsa_sparse_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor, o: torch.Tensor,
                        lse: torch.Tensor, dout: torch.Tensor, scale: Optional[float] = None,
                        workspace: Optional[torch.Tensor] = None):
    """Gradients of dsa_sparse_attn_fwd's output given dout, the forward's o and lse and the same idx:
    returns fp32 (dq, dk, dv) shaped like q, k, v."""
    lib = load_library()
    _dev(q, k, v, idx, o, lse, dout)
    B, S, Hq, dqk = q.shape
    Hkv, dv_ = k.shape[2], v.shape[3]
    topk = idx.shape[2]
    if not idx.is_contiguous() or idx.dtype != torch.int32:
        raise ValueError("idx must be contiguous int32 [B, S, topk]")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, Hq, S]")
    if scale is None:
        scale = 1.0 / math.sqrt(dqk)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty(q.shape, **f32)
    dk = torch.empty(k.shape, **f32)
    dv = torch.empty(v.shape, **f32)
    if workspace is None:
        workspace = torch.empty(lib.dsa_sparse_attn_bwd_workspace_size(_dt(q), B, S, Hq, Hkv, dqk, dv_, topk),
                                dtype=torch.uint8, device=q.device)
    _check(lib.dsa_sparse_attn_bwd(_dt(q), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
                                   _ptr(idx), _ptr(o), _strides(o), _ptr(lse), _ptr(dout), _strides(dout),
                                   _ptr(dq), _strides(dq), _ptr(dk), _strides(dk), _ptr(dv), _strides(dv),
                                   B, S, Hq, Hkv, dqk, dv_, topk, float(scale), _ptr(workspace), workspace.numel(),
                                   _stream()))
    return dq, dk, dv


__all__ = [
    "load_library", "HcaError", "Strides", "EXPORTS",
    "hca_abi_version", "hca_last_error", "hca_compress_kv", "hca_append_kv", "hca_attn_fwd_workspace_size",
    "hca_attn_fwd",
    "dsa_index_topk_workspace_size", "dsa_index_topk", "dsa_sparse_attn_fwd",
    "dsa_index_topk_decode_workspace_size", "dsa_index_topk_decode", "dsa_sparse_attn_decode",
    "dsa_sparse_attn_decode_workspace_size",
    "hca_attn_bwd_workspace_size", "hca_attn_bwd", "hca_compress_kv_bwd", "hca_attn_compress_bwd",
    "dsa_sparse_attn_bwd_workspace_size", "dsa_sparse_attn_bwd",
    "csa_index_topk_workspace_size", "csa_index_topk", "csa_sparse_attn_fwd", "attn_output_epilogue",
]
