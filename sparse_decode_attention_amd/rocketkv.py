"""Thin ctypes binding of librocketkv.so (declared in include/rocketkv.h).

Argument marshalling only: every step of the hot path runs in the HIP kernels
of the library.  Tensors are torch tensors on the current GPU (torch is used
for device memory and streams); sizes and strides are read from their shapes.
Importing this module loads the library and raises ImportError if it has not
been built -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librocketkv.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m sparse_decode_attention_amd.build`")
_lib = ctypes.CDLL(_LIB_PATH)

RK_OK, RK_EINVAL, RK_EUNSUPPORTED, RK_EWORKSPACE, RK_EDEVICE = range(5)
RK_F32, RK_BF16 = 0, 1


class RkShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int)]


class RkSplitOut(ctypes.Structure):
    _fields_ = [("r", ctypes.c_double), ("c1", ctypes.c_double), ("c2", ctypes.c_double),
                ("budget_t", ctypes.c_double), ("n_keep", ctypes.c_int64),
                ("k2_blocks", ctypes.c_int32), ("paper_page", ctypes.c_int32),
                ("paper_k1", ctypes.c_double), ("paper_k1_channels", ctypes.c_int32),
                ("paper_k2_blocks", ctypes.c_int32)]


_i32, _i64, _f64, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_size_t
_SP = ctypes.POINTER(RkShape)

_lib.rk_split.argtypes = [_f64, _i64, _i32, _i32, _i32, ctypes.POINTER(RkSplitOut)]
_lib.rk_snapkv_workspace_bytes.argtypes = [_SP, _i64, _i32]
_lib.rk_snapkv_workspace_bytes.restype = _sz
_lib.rk_snapkv_evict.argtypes = [_SP, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _i64, _vp, _vp, _vp,
                                 _i64, _vp, _vp, _vp, _i64, _i32, _vp, _sz, _vp]
_lib.rk_snapkv_evict_pool.argtypes = [_SP, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _i64, _vp, _vp,
                                      _vp, _i64, _vp, _vp, _vp, _i64, _i32, _vp, _sz, _vp]
_lib.rk_snapkv_evict_pool.restype = ctypes.c_int
# pooling operations (rk_pool_op)
POOL_OPS = {"sum": 0, "max": 1}
_lib.rk_hsa_build_aux.argtypes = [_SP, _vp, _i64, _vp, _i64, _i64, _i64, _i32, _vp, _vp, _i64, _vp]
_lib.rk_hsa_workspace_bytes.argtypes = [_SP, _i64, _i32, _i32, _i32]
_lib.rk_hsa_workspace_bytes.restype = _sz
_lib.rk_hsa_decode.argtypes = [_SP, _vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i32, _i32, _i32,
                               _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.rk_hsa_decode_mt.argtypes = [_SP, _vp, _vp, _vp, _i64, _vp, _i64, _i64, _vp, _vp, _i64, _i32,
                                  _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.rk_status_string.argtypes = [ctypes.c_int]
_lib.rk_status_string.restype = ctypes.c_char_p
_lib.rk_last_error.argtypes = []
_lib.rk_last_error.restype = ctypes.c_char_p
for _f in ("rk_split", "rk_snapkv_evict", "rk_hsa_build_aux", "rk_hsa_decode", "rk_hsa_decode_mt"):
    getattr(_lib, _f).restype = ctypes.c_int


class RocketKVError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        name = _lib.rk_status_string(status).decode()
        super().__init__(f"{what}: {name}: {_lib.rk_last_error().decode()}")


def _check(status: int, what: str):
    if status != RK_OK:
        raise RocketKVError(status, what)


def _ptr(t):
    """Device address of a tensor argument (None passes NULL).  Every tensor the
    library reads or writes lives in GPU memory: a host tensor is refused here,
    before a kernel could dereference its address."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor arguments must be on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _need_dtype(dtype, *ts):
    """Index, count and float32 output arguments have one fixed element type."""
    for t in ts:
        if t is not None and t.dtype != dtype:
            raise TypeError(f"expected {dtype} tensor, got {t.dtype}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return RK_F32
    if t.dtype == torch.bfloat16:
        return RK_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def shape_of(batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, dtype) -> RkShape:
    code = dtype if isinstance(dtype, int) else (RK_F32 if dtype == torch.float32 else RK_BF16)
    return RkShape(batch, n_q_heads, n_kv_heads, head_dim, code)


def _need_contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _ws(nbytes: int, like: torch.Tensor, ws, stream=None):
    """The caller's workspace, or a new one.  A new one is allocated on the
    current stream; when the call runs on another stream it is recorded there
    too, so the caching allocator does not hand its memory out again while
    that stream may still use it."""
    if ws is not None:
        return ws
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=like.device)
    if stream is not None and stream != torch.cuda.current_stream(like.device):
        ws.record_stream(stream)
    return ws


# --------------------------------------------------------------------------
def rk_split(c: float, seq_len: int, window: int, block: int, head_dim: int) -> dict:
    out = RkSplitOut()
    _check(_lib.rk_split(c, seq_len, window, block, head_dim, ctypes.byref(out)), "rk_split")
    return {f: getattr(out, f) for f, _ in RkSplitOut._fields_}


def rk_snapkv_workspace_bytes(shape: RkShape, seq_len: int, window: int) -> int:
    return _lib.rk_snapkv_workspace_bytes(ctypes.byref(shape), seq_len, window)


def rk_snapkv_evict(q_win, k, v, seq_len, window, pool_kernel, n_keep, kept_idx,
                    k_out=None, v_out=None, pooled=None, ws=None, stream=None,
                    kmax=None, kmin=None, block=16, pool_op="sum"):
    """Stage 1.  q_win [B,Hq,W,d]; k, v [B,Hkv,cap,d]; kept_idx [B,Hkv,n_keep] int32;
    k_out, v_out [B,Hkv,out_cap,d] or None (RocketKV-MT); pooled [B,Hkv,S-W] fp32 or None;
    kmax, kmin [B,Hkv,d,nblk_cap] or None: also build the compact cache's Kmax/Kmin in
    pages of `block` tokens; pool_op "sum" (rk_snapkv_evict) or "max"
    (rk_snapkv_evict_pool with RK_POOL_MAX)."""
    _need_contig(q_win, k, v, kept_idx, k_out, v_out, pooled, kmax, kmin)
    _need_dtype(k.dtype, q_win, v, k_out, v_out, kmax, kmin)
    _need_dtype(torch.int32, kept_idx)
    _need_dtype(torch.float32, pooled)
    B, Hq, W, d = q_win.shape
    shape = shape_of(B, Hq, k.shape[1], d, _dtype_code(k))
    nbytes = rk_snapkv_workspace_bytes(shape, seq_len, window)
    ws = _ws(nbytes, k, ws, stream)
    out_cap = k_out.shape[2] if k_out is not None else 0
    nblk_cap = kmax.shape[3] if kmax is not None else 0
    if pool_op == "sum":
        _check(_lib.rk_snapkv_evict(ctypes.byref(shape), _ptr(q_win), _ptr(k), _ptr(v), k.shape[2],
                                    seq_len, window, pool_kernel, n_keep, _ptr(kept_idx), _ptr(k_out),
                                    _ptr(v_out), out_cap, _ptr(pooled), _ptr(kmax), _ptr(kmin), nblk_cap,
                                    block, _ptr(ws), ws.numel(), _stream(stream)), "rk_snapkv_evict")
    else:
        _check(_lib.rk_snapkv_evict_pool(ctypes.byref(shape), _ptr(q_win), _ptr(k), _ptr(v), k.shape[2],
                                         seq_len, window, pool_kernel, POOL_OPS.get(pool_op, -1), n_keep,
                                         _ptr(kept_idx), _ptr(k_out), _ptr(v_out), out_cap, _ptr(pooled),
                                         _ptr(kmax), _ptr(kmin), nblk_cap, block, _ptr(ws), ws.numel(),
                                         _stream(stream)), "rk_snapkv_evict_pool")
    return ws


def rk_hsa_build_aux(k, n_tokens, first_token, block, kmax, kmin, n_q_heads=None, idx=None,
                     stream=None):
    """HSA step 1.  k [B,Hkv,cap,d]; kmax, kmin [B,Hkv,d,nblk_cap] (kmin None: Kmax only);
    idx [B,Hkv,stride] int32 or None (page token n is row idx[n])."""
    _need_contig(k, kmax, kmin, idx)
    _need_dtype(k.dtype, kmax, kmin)
    _need_dtype(torch.int32, idx)
    B, Hkv, cap, d = k.shape
    shape = shape_of(B, n_q_heads or Hkv, Hkv, d, _dtype_code(k))
    _check(_lib.rk_hsa_build_aux(ctypes.byref(shape), _ptr(k), cap, _ptr(idx),
                                 idx.shape[2] if idx is not None else 0, n_tokens, first_token,
                                 block, _ptr(kmax), _ptr(kmin), kmax.shape[3], _stream(stream)),
           "rk_hsa_build_aux")


_lib.rk_append_kv.argtypes = [_SP, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _i64, _i32, _vp]
_lib.rk_append_kv.restype = ctypes.c_int
_lib.rk_hsa_append_decode.argtypes = [_SP, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _vp, _i64, _i32,
                                      _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.rk_hsa_append_decode.restype = ctypes.c_int


def rk_append_kv(k_new, v_new, k, v, pos, kmax, kmin, block, n_q_heads=None, stream=None):
    """Append row `pos` (k_new, v_new [B,Hkv,d]) to k, v [B,Hkv,cap,d] and fold it
    into page pos // block of kmax, kmin [B,Hkv,d,nblk_cap]."""
    _need_contig(k_new, v_new, k, v, kmax, kmin)
    _need_dtype(k.dtype, k_new, v_new, v, kmax, kmin)
    B, Hkv, cap, d = k.shape
    shape = shape_of(B, n_q_heads or Hkv, Hkv, d, _dtype_code(k))
    _check(_lib.rk_append_kv(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _ptr(k), _ptr(v), cap, pos,
                             _ptr(kmax), _ptr(kmin), kmax.shape[3], block, _stream(stream)), "rk_append_kv")


def rk_hsa_workspace_bytes(shape: RkShape, n_tokens: int, block: int, k1: int, k2: int) -> int:
    return _lib.rk_hsa_workspace_bytes(ctypes.byref(shape), n_tokens, block, k1, k2)


def rk_hsa_decode(q, k, v, kmax, kmin, n_tokens, block, k1, k2, out, sel_blocks=None,
                  sel_channels=None, block_scores=None, ws=None, stream=None):
    """HSA steps 2-3.  q [B,Hq,d]; k, v [B,Hkv,cap,d]; kmax/kmin [B,Hkv,d,nblk_cap];
    out [B,Hq,d] fp32; optional sel_blocks [B,Hkv,min(k2,nblk)], sel_channels [B,Hkv,k1],
    block_scores [B,Hkv,nblk]."""
    _need_contig(q, k, v, kmax, kmin, out, sel_blocks, sel_channels, block_scores)
    _need_dtype(k.dtype, q, v, kmax, kmin)
    _need_dtype(torch.int32, sel_blocks, sel_channels)
    _need_dtype(torch.float32, out, block_scores)
    B, Hq, d = q.shape
    shape = shape_of(B, Hq, k.shape[1], d, _dtype_code(k))
    ws = _ws(rk_hsa_workspace_bytes(shape, n_tokens, block, k1, k2), k, ws, stream)
    _check(_lib.rk_hsa_decode(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), k.shape[2],
                              _ptr(kmax), _ptr(kmin), kmax.shape[3], n_tokens, block, k1, k2,
                              _ptr(out), _ptr(sel_blocks), _ptr(sel_channels), _ptr(block_scores),
                              _ptr(ws), ws.numel(), _stream(stream)), "rk_hsa_decode")
    return ws


def rk_hsa_append_decode(q, k_new, v_new, k, v, pos, kmax, kmin, block, k1, k2, out,
                         sel_blocks=None, sel_channels=None, block_scores=None, ws=None,
                         stream=None):
    """rk_append_kv at pos followed by rk_hsa_decode over pos + 1 tokens, in one call."""
    _need_contig(q, k_new, v_new, k, v, kmax, kmin, out, sel_blocks, sel_channels, block_scores)
    _need_dtype(k.dtype, q, k_new, v_new, v, kmax, kmin)
    _need_dtype(torch.int32, sel_blocks, sel_channels)
    _need_dtype(torch.float32, out, block_scores)
    B, Hq, d = q.shape
    shape = shape_of(B, Hq, k.shape[1], d, _dtype_code(k))
    ws = _ws(rk_hsa_workspace_bytes(shape, pos + 1, block, k1, k2), k, ws, stream)
    _check(_lib.rk_hsa_append_decode(ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new),
                                     _ptr(k), _ptr(v), k.shape[2], pos, _ptr(kmax), _ptr(kmin),
                                     kmax.shape[3], block, k1, k2, _ptr(out), _ptr(sel_blocks),
                                     _ptr(sel_channels), _ptr(block_scores), _ptr(ws), ws.numel(),
                                     _stream(stream)), "rk_hsa_append_decode")
    return ws


_lib.rk_hsa_decode_noalloc.argtypes = [_SP, _vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i32, _i32, _i32,
                                       _vp, _vp, _vp, _vp, _vp]
_lib.rk_hsa_decode_noalloc.restype = ctypes.c_int
_lib.rk_hsa_decode_noalloc_max_bytes.argtypes = []
_lib.rk_hsa_decode_noalloc_max_bytes.restype = _sz


def rk_hsa_decode_noalloc(q, k, v, kmax, kmin, n_tokens, block, k1, k2, out, sel_blocks=None,
                          sel_channels=None, block_scores=None, stream=None):
    """rk_hsa_decode with the library's static scratch instead of a workspace:
    allocates nothing (every tensor, out included, comes from the caller)."""
    _need_contig(q, k, v, kmax, kmin, out, sel_blocks, sel_channels, block_scores)
    _need_dtype(k.dtype, q, v, kmax, kmin)
    _need_dtype(torch.int32, sel_blocks, sel_channels)
    _need_dtype(torch.float32, out, block_scores)
    B, Hq, d = q.shape
    shape = shape_of(B, Hq, k.shape[1], d, _dtype_code(k))
    _check(_lib.rk_hsa_decode_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), k.shape[2],
                                      _ptr(kmax), _ptr(kmin), kmax.shape[3], n_tokens, block, k1, k2,
                                      _ptr(out), _ptr(sel_blocks), _ptr(sel_channels), _ptr(block_scores),
                                      _stream(stream)), "rk_hsa_decode_noalloc")


def rk_hsa_decode_noalloc_max_bytes() -> int:
    return _lib.rk_hsa_decode_noalloc_max_bytes()


def rk_hsa_decode_mt(q, k, v, cand_idx, n_cand, kmax, kmin, block, k1, k2, out, sel_blocks=None,
                     sel_channels=None, block_scores=None, ws=None, stream=None):
    """RocketKV-MT decode over the candidate rows cand_idx [B,Hkv,stride] of the full k, v."""
    _need_contig(q, k, v, cand_idx, kmax, kmin, out, sel_blocks, sel_channels, block_scores)
    _need_dtype(k.dtype, q, v, kmax, kmin)
    _need_dtype(torch.int32, cand_idx, sel_blocks, sel_channels)
    _need_dtype(torch.float32, out, block_scores)
    B, Hq, d = q.shape
    shape = shape_of(B, Hq, k.shape[1], d, _dtype_code(k))
    ws = _ws(rk_hsa_workspace_bytes(shape, n_cand, block, k1, k2), k, ws, stream)
    _check(_lib.rk_hsa_decode_mt(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), k.shape[2],
                                 _ptr(cand_idx), cand_idx.shape[2], n_cand, _ptr(kmax), _ptr(kmin),
                                 kmax.shape[3], block, k1, k2, _ptr(out), _ptr(sel_blocks),
                                 _ptr(sel_channels), _ptr(block_scores), _ptr(ws), ws.numel(),
                                 _stream(stream)), "rk_hsa_decode_mt")
    return ws


RK_SEL = {"hsa": 0, "quest": 1, "sparq": 2, "exact": 3}


class RkSelectPlan(ctypes.Structure):
    _fields_ = [("page", ctypes.c_int32), ("channels", ctypes.c_int32), ("k2", ctypes.c_int32),
                ("attn_tokens", ctypes.c_int64), ("budget_t", ctypes.c_double), ("est_pairs", ctypes.c_double)]


_lib.rk_select_plan.argtypes = [ctypes.c_int, _f64, _i64, _i32, ctypes.POINTER(RkSelectPlan)]
_lib.rk_select_plan.restype = ctypes.c_int
_lib.rk_select_decode.argtypes = [_SP, ctypes.c_int, _vp, _vp, _vp, _i64, _vp, _vp, _i64, _i64, _i32, _i32,
                                  _i32, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.rk_select_decode.restype = ctypes.c_int


def rk_select_plan(method: str, c: float, seq_len: int, head_dim: int) -> dict:
    """Page, channels and attended pages of a selection method ('hsa', 'quest',
    'sparq', 'exact') at total compression c."""
    out = RkSelectPlan()
    _check(_lib.rk_select_plan(RK_SEL[method], c, seq_len, head_dim, ctypes.byref(out)), "rk_select_plan")
    return {f: getattr(out, f) for f, _ in RkSelectPlan._fields_}


def rk_select_decode(method, q, k, v, kmax, kmin, n_tokens, page, channels, k2, out, sel=None, scores=None,
                     ws=None, stream=None):
    """One decode step of a selection method.  kmax/kmin: aux in pages of `page`
    tokens (hsa, quest); the block-1 Kmax (sparq, kmin may be None); None (exact)."""
    _need_contig(q, k, v, kmax, kmin, out, sel, scores)
    _need_dtype(k.dtype, q, v, kmax, kmin)
    _need_dtype(torch.int32, sel)
    _need_dtype(torch.float32, out, scores)
    B, Hq, d = q.shape
    shape = shape_of(B, Hq, k.shape[1], d, _dtype_code(k))
    ws = _ws(rk_hsa_workspace_bytes(shape, n_tokens, page, channels, k2), k, ws, stream)
    _check(_lib.rk_select_decode(ctypes.byref(shape), RK_SEL[method], _ptr(q), _ptr(k), _ptr(v), k.shape[2],
                                 _ptr(kmax), _ptr(kmin), kmax.shape[3] if kmax is not None else 0, n_tokens,
                                 page, channels, k2, _ptr(out), _ptr(sel), _ptr(scores), _ptr(ws), ws.numel(),
                                 _stream(stream)), "rk_select_decode")
    return ws


class RkPagedKv(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("table_stride", ctypes.c_int64), ("n_pages", ctypes.c_int64),
                ("page_tokens", ctypes.c_int32)]


_PP = ctypes.POINTER(RkPagedKv)
_lib.rk_paged_write_kv.argtypes = [_SP, _vp, _vp, _i64, _i64, _i64, _vp, _vp, _PP, _vp]
_lib.rk_paged_build_aux.argtypes = [_SP, _vp, _PP, _i64, _i64, _i32, _vp, _vp, _i64, _vp]
_lib.rk_paged_append_kv.argtypes = [_SP, _vp, _vp, _vp, _vp, _PP, _i64, _vp, _vp, _i64, _i32, _vp]
_lib.rk_paged_hsa_decode.argtypes = [_SP, _vp, _vp, _vp, _PP, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _vp, _vp,
                                     _vp, _vp, _vp, _sz, _vp]
_lib.rk_paged_hsa_append_decode.argtypes = [_SP, _vp, _vp, _vp, _vp, _vp, _PP, _i64, _vp, _vp, _i64, _i32, _i32,
                                            _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
for _f in ("rk_paged_write_kv", "rk_paged_build_aux", "rk_paged_append_kv", "rk_paged_hsa_decode",
           "rk_paged_hsa_append_decode"):
    getattr(_lib, _f).restype = ctypes.c_int


def paged_kv(block_table, n_pages: int, page_tokens: int) -> RkPagedKv:
    """Descriptor of a paged pool: block_table [B, stride] int32 on the device."""
    _need_contig(block_table)
    _need_dtype(torch.int32, block_table)
    return RkPagedKv(_ptr(block_table).value, block_table.shape[1], n_pages, page_tokens)


def rk_paged_write_kv(k_src, v_src, first_token, n_tokens, k_pool, v_pool, pages: RkPagedKv, n_q_heads=None,
                      stream=None):
    """Copy rows [first, first + n) of k_src, v_src [B,Hkv,cap,d] into the paged pool."""
    _need_contig(k_src, v_src, k_pool, v_pool)
    _need_dtype(k_pool.dtype, k_src, v_src, v_pool)
    B, Hkv, cap, d = k_src.shape
    shape = shape_of(B, n_q_heads or Hkv, Hkv, d, _dtype_code(k_src))
    _check(_lib.rk_paged_write_kv(ctypes.byref(shape), _ptr(k_src), _ptr(v_src), cap, first_token, n_tokens,
                                  _ptr(k_pool), _ptr(v_pool), ctypes.byref(pages), _stream(stream)),
           "rk_paged_write_kv")


def rk_paged_build_aux(k_pool, pages: RkPagedKv, batch, n_tokens, first_token, block, kmax, kmin,
                       n_q_heads=None, stream=None):
    """HSA step 1 over a paged pool k_pool [n_pages,Hkv,P,d]; kmax, kmin [B,Hkv,d,nblk_cap]."""
    _need_contig(k_pool, kmax, kmin)
    _need_dtype(k_pool.dtype, kmax, kmin)
    _, Hkv, _, d = k_pool.shape
    shape = shape_of(batch, n_q_heads or Hkv, Hkv, d, _dtype_code(k_pool))
    _check(_lib.rk_paged_build_aux(ctypes.byref(shape), _ptr(k_pool), ctypes.byref(pages), n_tokens, first_token,
                                   block, _ptr(kmax), _ptr(kmin), kmax.shape[3], _stream(stream)),
           "rk_paged_build_aux")


def rk_paged_append_kv(k_new, v_new, k_pool, v_pool, pages: RkPagedKv, pos, kmax, kmin, block, n_q_heads=None,
                       stream=None):
    _need_contig(k_new, v_new, k_pool, v_pool, kmax, kmin)
    _need_dtype(k_pool.dtype, k_new, v_new, v_pool, kmax, kmin)
    B, Hkv, d = k_new.shape
    shape = shape_of(B, n_q_heads or Hkv, Hkv, d, _dtype_code(k_new))
    _check(_lib.rk_paged_append_kv(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool),
                                   ctypes.byref(pages), pos, _ptr(kmax), _ptr(kmin), kmax.shape[3], block,
                                   _stream(stream)), "rk_paged_append_kv")


def rk_paged_hsa_decode(q, k_pool, v_pool, pages: RkPagedKv, kmax, kmin, n_tokens, block, k1, k2, out,
                        sel_blocks=None, sel_channels=None, block_scores=None, ws=None, stream=None):
    _need_contig(q, k_pool, v_pool, kmax, kmin, out, sel_blocks, sel_channels, block_scores)
    _need_dtype(k_pool.dtype, q, v_pool, kmax, kmin)
    _need_dtype(torch.int32, sel_blocks, sel_channels)
    _need_dtype(torch.float32, out, block_scores)
    B, Hq, d = q.shape
    shape = shape_of(B, Hq, k_pool.shape[1], d, _dtype_code(k_pool))
    ws = _ws(rk_hsa_workspace_bytes(shape, n_tokens, block, k1, k2), k_pool, ws, stream)
    _check(_lib.rk_paged_hsa_decode(ctypes.byref(shape), _ptr(q), _ptr(k_pool), _ptr(v_pool), ctypes.byref(pages),
                                    _ptr(kmax), _ptr(kmin), kmax.shape[3], n_tokens, block, k1, k2, _ptr(out),
                                    _ptr(sel_blocks), _ptr(sel_channels), _ptr(block_scores), _ptr(ws),
                                    ws.numel(), _stream(stream)), "rk_paged_hsa_decode")
    return ws


def rk_paged_hsa_append_decode(q, k_new, v_new, k_pool, v_pool, pages: RkPagedKv, pos, kmax, kmin, block, k1,
                               k2, out, sel_blocks=None, sel_channels=None, block_scores=None, ws=None,
                               stream=None):
    _need_contig(q, k_new, v_new, k_pool, v_pool, kmax, kmin, out, sel_blocks, sel_channels, block_scores)
    _need_dtype(k_pool.dtype, q, k_new, v_new, v_pool, kmax, kmin)
    _need_dtype(torch.int32, sel_blocks, sel_channels)
    _need_dtype(torch.float32, out, block_scores)
    B, Hq, d = q.shape
    shape = shape_of(B, Hq, k_pool.shape[1], d, _dtype_code(k_pool))
    ws = _ws(rk_hsa_workspace_bytes(shape, pos + 1, block, k1, k2), k_pool, ws, stream)
    _check(_lib.rk_paged_hsa_append_decode(ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_pool),
                                           _ptr(v_pool), ctypes.byref(pages), pos, _ptr(kmax), _ptr(kmin),
                                           kmax.shape[3], block, k1, k2, _ptr(out), _ptr(sel_blocks),
                                           _ptr(sel_channels), _ptr(block_scores), _ptr(ws), ws.numel(),
                                           _stream(stream)), "rk_paged_hsa_append_decode")
    return ws


_lib.rk_adakv_evict.argtypes = [_SP, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _i64, _vp,
                                _vp, _vp, _i64, _i32, _vp, _sz, _vp]
_lib.rk_adakv_evict.restype = ctypes.c_int
_lib.rk_adakv_evict_pool.argtypes = [_SP, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp,
                                     _i64, _vp, _vp, _vp, _i64, _i32, _vp, _sz, _vp]
_lib.rk_adakv_evict_pool.restype = ctypes.c_int
_lib.rk_hsa_decode_ragged.argtypes = [_SP, _vp, _vp, _vp, _i64, _vp, _vp, _i64, _vp, _i64, _i32, _i32, _i32, _vp,
                                      _vp, _vp, _vp, _vp, _sz, _vp]
_lib.rk_hsa_decode_ragged.restype = ctypes.c_int


def adakv_capacity(n_kv_heads: int, seq_len: int, window: int, n_keep: int) -> int:
    """Rows a unit may keep under the shared budget: min(S, Hkv * (n_keep - W) + W)."""
    return min(seq_len, n_kv_heads * (n_keep - window) + window)


def rk_adakv_evict(q_win, k, v, seq_len, window, pool_kernel, n_keep, kept_idx, kept_count, k_out=None,
                   v_out=None, pooled=None, ws=None, stream=None, kmax=None, kmin=None, block=16,
                   pool_op="sum"):
    """Stage 1 with the shared (Ada-KV) budget.  kept_idx [B,Hkv,out_cap], kept_count [B,Hkv] int32;
    k_out, v_out [B,Hkv,out_cap,d] or None; kmax/kmin and pool_op as rk_snapkv_evict."""
    _need_contig(q_win, k, v, kept_idx, kept_count, k_out, v_out, pooled, kmax, kmin)
    _need_dtype(k.dtype, q_win, v, k_out, v_out, kmax, kmin)
    _need_dtype(torch.int32, kept_idx, kept_count)
    _need_dtype(torch.float32, pooled)
    B, Hq, W, d = q_win.shape
    shape = shape_of(B, Hq, k.shape[1], d, _dtype_code(k))
    ws = _ws(rk_snapkv_workspace_bytes(shape, seq_len, window), k, ws, stream)
    out_cap = kept_idx.shape[2]
    nblk_cap = kmax.shape[3] if kmax is not None else 0
    _check(_lib.rk_adakv_evict_pool(ctypes.byref(shape), _ptr(q_win), _ptr(k), _ptr(v), k.shape[2], seq_len,
                                    window, pool_kernel, POOL_OPS.get(pool_op, -1), n_keep, _ptr(kept_idx),
                                    _ptr(kept_count), _ptr(k_out), _ptr(v_out), out_cap, _ptr(pooled), _ptr(kmax),
                                    _ptr(kmin), nblk_cap, block, _ptr(ws), ws.numel(), _stream(stream)),
           "rk_adakv_evict_pool")
    return ws


def rk_hsa_decode_ragged(q, k, v, kmax, kmin, unit_tokens, max_tokens, block, k1, k2, out, sel_blocks=None,
                         sel_channels=None, block_scores=None, ws=None, stream=None):
    """rk_hsa_decode with a token count per unit (unit_tokens [B,Hkv] int32 on the device)."""
    _need_contig(q, k, v, kmax, kmin, unit_tokens, out, sel_blocks, sel_channels, block_scores)
    _need_dtype(k.dtype, q, v, kmax, kmin)
    _need_dtype(torch.int32, unit_tokens, sel_blocks, sel_channels)
    _need_dtype(torch.float32, out, block_scores)
    B, Hq, d = q.shape
    shape = shape_of(B, Hq, k.shape[1], d, _dtype_code(k))
    ws = _ws(rk_hsa_workspace_bytes(shape, max_tokens, block, k1, k2), k, ws, stream)
    _check(_lib.rk_hsa_decode_ragged(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), k.shape[2], _ptr(kmax),
                                     _ptr(kmin), kmax.shape[3], _ptr(unit_tokens), max_tokens, block, k1, k2,
                                     _ptr(out), _ptr(sel_blocks), _ptr(sel_channels), _ptr(block_scores),
                                     _ptr(ws), ws.numel(), _stream(stream)), "rk_hsa_decode_ragged")
    return ws


def aux_capacity(n_tokens: int, block: int) -> int:
    """Smallest valid nblk_cap for n_tokens: the page count rounded up to 8."""
    return (-(-n_tokens // block) + 7) // 8 * 8


def library_path() -> str:
    return _LIB_PATH


def raw_library() -> ctypes.CDLL:
    """The loaded ctypes library (for tests of the raw C ABI)."""
    return _lib


class RkKernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


_lib.rk_profile_begin.argtypes = []
_lib.rk_profile_begin.restype = ctypes.c_int
_lib.rk_profile_end.argtypes = [ctypes.POINTER(RkKernelTime), ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
_lib.rk_profile_end.restype = ctypes.c_int


def rk_profile_begin():
    """Start bracketing every library kernel with HIP events on its stream."""
    _check(_lib.rk_profile_begin(), "rk_profile_begin")


def rk_profile_end(cap: int = 64) -> dict:
    """Stop, wait for the events and return {kernel: (launches, total_ms)}."""
    arr = (RkKernelTime * cap)()
    n = ctypes.c_int32(0)
    _check(_lib.rk_profile_end(arr, cap, ctypes.byref(n)), "rk_profile_end")
    return {arr[i].name.decode(): (int(arr[i].launches), float(arr[i].total_ms)) for i in range(n.value)}
