"""ctypes binding of libkvq (include/kvq.h). Argument marshalling only: every step of
encode, dequantise and attention runs in the library's HIP kernels. PyTorch provides
device memory and the stream; there is no fallback path."""

from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libkvq.so not found at {LIB_PATH}; build it with "
        "`python rotated_angle_quantization_amd/build.py` (hipcc, gfx950)")

lib = ctypes.CDLL(LIB_PATH)

KVQ_F16, KVQ_F32 = 0, 1
STATUS = {0: "OK", 1: "INVALID_ARGUMENT", 2: "UNSUPPORTED", 3: "CAPACITY", 4: "WORKSPACE",
          5: "HIP"}


class LayerDesc(ctypes.Structure):
    """kvq_layer_desc: one layer's cache geometry and codec parameters."""

    _fields_ = [("head_dim", ctypes.c_uint32), ("num_kv_heads", ctypes.c_uint32),
                ("batch", ctypes.c_uint32), ("capacity", ctypes.c_uint32),
                ("n_bins_k", ctypes.c_uint32), ("n_bins_v", ctypes.c_uint32),
                ("layer", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
                ("seed", ctypes.c_uint64)]

    def __repr__(self):
        return (f"LayerDesc(d={self.head_dim}, hkv={self.num_kv_heads}, B={self.batch}, "
                f"cap={self.capacity}, n=({self.n_bins_k},{self.n_bins_v}), "
                f"layer={self.layer}, seed={self.seed})")


class Paging(ctypes.Structure):
    """kvq_paging: page table (device int32 [batch][pages_per_seq]) of a paged cache."""

    _fields_ = [("page_table", ctypes.c_void_p), ("pages_per_seq", ctypes.c_uint32),
                ("num_pages", ctypes.c_uint32)]


class KvqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.kvq_status_string(status).decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({msg})")


_P = ctypes.POINTER(LayerDesc)
_v = ctypes.c_void_p
_u32, _u64, _i64, _f32, _sz = (ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int64,
                               ctypes.c_float, ctypes.c_size_t)

_SIGS = {
    "kvq_abi_version": (ctypes.c_int, []),
    "kvq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kvq_cache_bytes": (_sz, [_P]),
    "kvq_tile_bytes": (_sz, [_u32, _u32, _u32]),
    "kvq_layer_signs": (ctypes.c_int, [_u64, _u32, _u32, ctypes.POINTER(ctypes.c_int8)]),
    "kvq_encode": (ctypes.c_int, [_P, _v, _v, _v, ctypes.c_int, _i64, _i64, _i64, _u32, _u32,
                                  _v]),
    "kvq_append": (ctypes.c_int, [_P, _v, _v, _v, ctypes.c_int, _i64, _i64, _v, _v]),
    "kvq_decode": (ctypes.c_int, [_P, _v, _v, _v, ctypes.c_int, _u32, _u32, _v]),
    "kvq_attn_workspace_bytes": (_sz, [_P, _u32, _u32]),
    "kvq_attn_num_splits": (_u32, [_P, _u32, _u32]),
    "kvq_attn_decode": (ctypes.c_int, [_P, _v, _v, ctypes.c_int, _u32, _u32, _f32, _v,
                                       ctypes.c_int, _v, _sz, _v]),
    "kvq_attn_decode_varlen": (ctypes.c_int, [_P, _v, _v, ctypes.c_int, _u32, _v, _u32, _f32,
                                              _v, ctypes.c_int, _v, _sz, _v]),
    "kvq_paged_pool_bytes": (_sz, [_P, _u32]),
    "kvq_encode_paged": (ctypes.c_int, [_P, _v, ctypes.POINTER(Paging), _v, _v, ctypes.c_int, _i64,
                                        _i64, _i64, _u32, _u32, _v]),
    "kvq_append_paged": (ctypes.c_int, [_P, _v, ctypes.POINTER(Paging), _v, _v, ctypes.c_int, _i64,
                                        _i64, _v, _v]),
    "kvq_decode_paged": (ctypes.c_int, [_P, _v, ctypes.POINTER(Paging), _v, _v, ctypes.c_int, _u32,
                                        _u32, _v]),
    "kvq_attn_decode_paged": (ctypes.c_int, [_P, _v, ctypes.POINTER(Paging), _v, ctypes.c_int, _u32,
                                             _v, _u32, _f32, _v, ctypes.c_int, _v, _sz, _v]),
    "kvq_attn_decode_append": (ctypes.c_int, [_P, _v, ctypes.POINTER(Paging), _v, _v,
                                              ctypes.c_int, _i64, _i64, _v, _v, ctypes.c_int,
                                              _u32, _u32, _f32, _v, ctypes.c_int, _v, _sz, _v]),
    "kvq_attn_multi_workspace_bytes": (_sz, [_P, _u32, _u32, _u32]),
    "kvq_attn_multi_paged": (ctypes.c_int, [_P, _v, ctypes.POINTER(Paging), _v, ctypes.c_int,
                                            _u32, _u32, _v, _u32, _f32, _v, ctypes.c_int, _v,
                                            _sz, _v]),
    "kvq_attn_multi_varlen": (ctypes.c_int, [_P, _v, _v, ctypes.c_int, _u32, _u32, _v, _u32,
                                             _f32, _v, ctypes.c_int, _v, _sz, _v]),
    "kvq_attn_multi": (ctypes.c_int, [_P, _v, _v, ctypes.c_int, _u32, _u32, _u32, _f32, _v,
                                      ctypes.c_int, _v, _sz, _v]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTS = tuple(_SIGS)


def _check(status: int, where: str):
    if status != 0:
        raise KvqError(status, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return KVQ_F16
    if t.dtype == torch.float32:
        return KVQ_F32
    raise TypeError(f"unsupported dtype {t.dtype} (float16 or float32)")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def make_desc(head_dim, num_kv_heads, batch, capacity, n_bins_k, n_bins_v, layer=0,
              seed=0) -> LayerDesc:
    return LayerDesc(head_dim, num_kv_heads, batch, capacity, n_bins_k, n_bins_v, layer, 0,
                     seed)


def abi_version() -> int:
    return lib.kvq_abi_version()


def cache_bytes(desc: LayerDesc) -> int:
    return lib.kvq_cache_bytes(ctypes.byref(desc))


def tile_bytes(head_dim: int, n_bins_k: int, n_bins_v: int) -> int:
    return lib.kvq_tile_bytes(head_dim, n_bins_k, n_bins_v)


def layer_signs(seed: int, layer: int, d: int) -> list[int]:
    buf = (ctypes.c_int8 * d)()
    _check(lib.kvq_layer_signs(seed, layer, d, buf), "kvq_layer_signs")
    return list(buf)


def alloc_cache(desc: LayerDesc, device="cuda") -> torch.Tensor:
    n = cache_bytes(desc)
    if n == 0:
        raise KvqError(1, "kvq_cache_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def encode(desc: LayerDesc, cache: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
           t0: int = 0) -> None:
    """Append K/V tokens [t0, t0 + ntok): k, v are [B, ntok, Hkv, d] with matching strides."""
    if k.shape != v.shape or k.stride() != v.stride() or k.dtype != v.dtype:
        raise ValueError("k and v must share shape, strides and dtype")
    if k.dim() != 4 or k.stride(3) != 1:
        raise ValueError("k/v must be [B, ntok, Hkv, d] with d contiguous")
    ntok = k.shape[1]
    _check(lib.kvq_encode(ctypes.byref(desc), cache.data_ptr(), k.data_ptr(), v.data_ptr(),
                          _dtype_code(k), k.stride(0), k.stride(1), k.stride(2), t0, ntok,
                          _stream(cache.device)), "kvq_encode")


def append(desc: LayerDesc, cache: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
           positions: torch.Tensor):
    """Encode one token per sequence at slot positions[b] of sequence b.
    k, v: [B, Hkv, d] (or [B, 1, Hkv, d]) with d contiguous, fp16 or fp32; positions:
    int32 device tensor [B]."""
    if k.dim() == 4 and k.shape[1] == 1:
        k, v = k[:, 0], v[:, 0]
    if k.dim() != 3 or k.shape != v.shape or k.stride() != v.stride() or k.stride(2) != 1:
        raise ValueError("k/v must be [B, Hkv, d] with d contiguous and equal strides")
    if k.dtype != v.dtype:
        raise ValueError("k and v must have the same dtype")
    if positions.dtype not in (torch.int32, torch.uint32) or not positions.is_contiguous() \
            or positions.numel() != k.shape[0] or positions.device != k.device:
        raise ValueError("positions must be a contiguous int32 device tensor [B] on k's device")
    _check(lib.kvq_append(ctypes.byref(desc), cache.data_ptr(), k.data_ptr(), v.data_ptr(),
                          _dtype_code(k), k.stride(0), k.stride(1), positions.data_ptr(),
                          _stream(cache.device)), "kvq_append")


def decode(desc: LayerDesc, cache: torch.Tensor, t0: int, ntok: int,
           out_dtype=torch.float16, out: tuple | None = None):
    """Dequantise tokens [t0, t0 + ntok) -> (k_hat, v_hat), each [B, ntok, Hkv, d]."""
    shape = (desc.batch, ntok, desc.num_kv_heads, desc.head_dim)
    if out is None:
        k_out = torch.empty(shape, dtype=out_dtype, device=cache.device)
        v_out = torch.empty(shape, dtype=out_dtype, device=cache.device)
    else:
        k_out, v_out = out
    _check(lib.kvq_decode(ctypes.byref(desc), cache.data_ptr(), k_out.data_ptr(),
                          v_out.data_ptr(), _dtype_code(k_out), t0, ntok,
                          _stream(cache.device)), "kvq_decode")
    return k_out, v_out


def attn_workspace_bytes(desc: LayerDesc, num_q_heads: int, seq_len: int) -> int:
    return lib.kvq_attn_workspace_bytes(ctypes.byref(desc), num_q_heads, seq_len)


def attn_num_splits(desc: LayerDesc, num_q_heads: int, seq_len: int) -> int:
    return lib.kvq_attn_num_splits(ctypes.byref(desc), num_q_heads, seq_len)


def alloc_workspace(desc: LayerDesc, num_q_heads: int, seq_len: int, device="cuda"):
    """Zero-filled attention workspace (the library keeps its split counters at zero
    between calls, so it can be reused for any later call that fits)."""
    n = attn_workspace_bytes(desc, num_q_heads, seq_len)
    if n == 0:
        raise KvqError(1, "kvq_attn_workspace_bytes")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def attn_decode(desc: LayerDesc, cache: torch.Tensor, q: torch.Tensor, seq_len: int,
                softmax_scale: float = 0.0, out_dtype=None, workspace=None, out=None):
    """o[b, h] = softmax(scale q.k_hat) v_hat over the first seq_len cached tokens.
    q: contiguous [B, Hq, d] (fp16 or fp32); returns [B, Hq, d]."""
    if not q.is_contiguous():
        raise ValueError("q must be contiguous [B, Hq, d]")
    hq = q.shape[1]
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(desc, hq, seq_len, q.device)
    _check(lib.kvq_attn_decode(ctypes.byref(desc), cache.data_ptr(), q.data_ptr(),
                               _dtype_code(q), hq, seq_len, float(softmax_scale),
                               out.data_ptr(), _dtype_code(out), workspace.data_ptr(),
                               workspace.numel(), _stream(q.device)), "kvq_attn_decode")
    return out


def attn_decode_varlen(desc: LayerDesc, cache: torch.Tensor, q: torch.Tensor,
                       seq_lens: torch.Tensor, max_seq_len: int, softmax_scale: float = 0.0,
                       out_dtype=None, workspace=None, out=None):
    """attn_decode with a length per sequence: entry b attends to its first seq_lens[b]
    cached tokens. seq_lens: int32 (or uint32 bits) device tensor [B], every entry
    <= max_seq_len (larger entries count as max_seq_len; 0 gives a zero output)."""
    if not q.is_contiguous():
        raise ValueError("q must be contiguous [B, Hq, d]")
    if seq_lens.dtype not in (torch.int32, torch.uint32) or not seq_lens.is_contiguous() \
            or seq_lens.numel() != q.shape[0] or seq_lens.device != q.device:
        raise ValueError("seq_lens must be a contiguous int32 device tensor [B] on q's device")
    hq = q.shape[1]
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(desc, hq, max_seq_len, q.device)
    _check(lib.kvq_attn_decode_varlen(ctypes.byref(desc), cache.data_ptr(), q.data_ptr(),
                                      _dtype_code(q), hq, seq_lens.data_ptr(), max_seq_len,
                                      float(softmax_scale), out.data_ptr(), _dtype_code(out),
                                      workspace.data_ptr(), workspace.numel(),
                                      _stream(q.device)), "kvq_attn_decode_varlen")
    return out


def attn_multi_workspace_bytes(desc: LayerDesc, num_q_heads: int, num_queries: int,
                               seq_len: int) -> int:
    return lib.kvq_attn_multi_workspace_bytes(ctypes.byref(desc), num_q_heads, num_queries,
                                              seq_len)


def attn_multi(desc: LayerDesc, cache: torch.Tensor, q: torch.Tensor, seq_len: int,
               softmax_scale: float = 0.0, out_dtype=None, workspace=None, out=None,
               paging: Paging | None = None, seq_lens: torch.Tensor | None = None):
    """Multi-query attention: q contiguous [B, NQ, Hq, d]; query token j attends to the
    first seq_len - NQ + j + 1 cached tokens. Returns [B, NQ, Hq, d]. With paging, cache
    is the pool (kvq_attn_multi_paged); with seq_lens (int32 device tensor [B]) sequence b
    holds min(seq_lens[b], seq_len) tokens (kvq_attn_multi_varlen)."""
    if not q.is_contiguous() or q.dim() != 4:
        raise ValueError("q must be contiguous [B, NQ, Hq, d]")
    nq, hq = q.shape[1], q.shape[2]
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if workspace is None:
        n = attn_multi_workspace_bytes(desc, hq, nq, seq_len)
        if n == 0:
            raise KvqError(1, "kvq_attn_multi_workspace_bytes")
        workspace = torch.zeros(n, dtype=torch.uint8, device=q.device)
    lens = seq_lens.data_ptr() if seq_lens is not None else None
    if paging is not None:
        _check(lib.kvq_attn_multi_paged(ctypes.byref(desc), cache.data_ptr(), ctypes.byref(paging),
                                        q.data_ptr(), _dtype_code(q), hq, nq, lens, seq_len,
                                        float(softmax_scale), out.data_ptr(), _dtype_code(out),
                                        workspace.data_ptr(), workspace.numel(),
                                        _stream(q.device)), "kvq_attn_multi_paged")
        return out
    if seq_lens is not None:
        _check(lib.kvq_attn_multi_varlen(ctypes.byref(desc), cache.data_ptr(), q.data_ptr(),
                                         _dtype_code(q), hq, nq, lens, seq_len,
                                         float(softmax_scale), out.data_ptr(), _dtype_code(out),
                                         workspace.data_ptr(), workspace.numel(),
                                         _stream(q.device)), "kvq_attn_multi_varlen")
        return out
    _check(lib.kvq_attn_multi(ctypes.byref(desc), cache.data_ptr(), q.data_ptr(),
                              _dtype_code(q), hq, nq, seq_len, float(softmax_scale),
                              out.data_ptr(), _dtype_code(out), workspace.data_ptr(),
                              workspace.numel(), _stream(q.device)), "kvq_attn_multi")
    return out


def paged_pool_bytes(desc: LayerDesc, num_pages: int) -> int:
    return lib.kvq_paged_pool_bytes(ctypes.byref(desc), num_pages)


def make_paging(page_table: torch.Tensor, num_pages: int) -> Paging:
    """page_table: contiguous int32 device tensor [batch, pages_per_seq]. The tensor must
    stay alive while calls that use the returned description are in flight."""
    if page_table.dtype != torch.int32 or page_table.dim() != 2 or not page_table.is_contiguous():
        raise ValueError("page_table must be a contiguous int32 tensor [batch, pages_per_seq]")
    return Paging(page_table.data_ptr(), page_table.shape[1], num_pages)


def encode_paged(desc: LayerDesc, pool: torch.Tensor, paging: Paging, k: torch.Tensor,
                 v: torch.Tensor, t0: int = 0):
    if k.dim() != 4 or k.stride(3) != 1 or k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k/v must be [B, ntok, Hkv, d] with d contiguous and equal strides")
    _check(lib.kvq_encode_paged(ctypes.byref(desc), pool.data_ptr(), ctypes.byref(paging),
                                k.data_ptr(), v.data_ptr(), _dtype_code(k), k.stride(0),
                                k.stride(1), k.stride(2), t0, k.shape[1], _stream(pool.device)),
           "kvq_encode_paged")


def append_paged(desc: LayerDesc, pool: torch.Tensor, paging: Paging, k: torch.Tensor,
                 v: torch.Tensor, positions: torch.Tensor):
    if k.dim() == 4 and k.shape[1] == 1:
        k, v = k[:, 0], v[:, 0]
    if k.dim() != 3 or k.shape != v.shape or k.stride() != v.stride() or k.stride(2) != 1:
        raise ValueError("k/v must be [B, Hkv, d] with d contiguous and equal strides")
    _check(lib.kvq_append_paged(ctypes.byref(desc), pool.data_ptr(), ctypes.byref(paging),
                                k.data_ptr(), v.data_ptr(), _dtype_code(k), k.stride(0),
                                k.stride(1), positions.data_ptr(), _stream(pool.device)),
           "kvq_append_paged")


def decode_paged(desc: LayerDesc, pool: torch.Tensor, paging: Paging, t0: int, ntok: int,
                 out_dtype=torch.float16):
    shape = (desc.batch, ntok, desc.num_kv_heads, desc.head_dim)
    k_out = torch.empty(shape, dtype=out_dtype, device=pool.device)
    v_out = torch.empty(shape, dtype=out_dtype, device=pool.device)
    _check(lib.kvq_decode_paged(ctypes.byref(desc), pool.data_ptr(), ctypes.byref(paging),
                                k_out.data_ptr(), v_out.data_ptr(), _dtype_code(k_out), t0, ntok,
                                _stream(pool.device)), "kvq_decode_paged")
    return k_out, v_out


def attn_decode_paged(desc: LayerDesc, pool: torch.Tensor, paging: Paging, q: torch.Tensor,
                      max_seq_len: int, seq_lens: torch.Tensor | None = None,
                      softmax_scale: float = 0.0, out_dtype=None, workspace=None, out=None):
    if not q.is_contiguous():
        raise ValueError("q must be contiguous [B, Hq, d]")
    hq = q.shape[1]
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(desc, hq, max_seq_len, q.device)
    lens = seq_lens.data_ptr() if seq_lens is not None else None
    _check(lib.kvq_attn_decode_paged(ctypes.byref(desc), pool.data_ptr(), ctypes.byref(paging),
                                     q.data_ptr(), _dtype_code(q), hq, lens, max_seq_len,
                                     float(softmax_scale), out.data_ptr(), _dtype_code(out),
                                     workspace.data_ptr(), workspace.numel(), _stream(q.device)),
           "kvq_attn_decode_paged")
    return out


def attn_decode_append(desc: LayerDesc, cache: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       positions: torch.Tensor, q: torch.Tensor, max_seq_len: int,
                       paging: Paging | None = None, softmax_scale: float = 0.0,
                       out_dtype=None, workspace=None, out=None):
    """One decode step in one launch: code the token k/v [B, Hkv, d] of sequence b at slot
    positions[b] (int32 device tensor [B]), then attend with q [B, Hq, d] over
    min(positions[b] + 1, max_seq_len) tokens. cache is the pool when paging is given."""
    if k.dim() == 4 and k.shape[1] == 1:
        k, v = k[:, 0], v[:, 0]
    if k.dim() != 3 or k.shape != v.shape or k.stride() != v.stride() or k.stride(2) != 1:
        raise ValueError("k/v must be [B, Hkv, d] with d contiguous and equal strides")
    if k.dtype != v.dtype:
        raise ValueError("k and v must have the same dtype")
    if positions.dtype not in (torch.int32, torch.uint32) or not positions.is_contiguous() \
            or positions.numel() != k.shape[0] or positions.device != k.device:
        raise ValueError("positions must be a contiguous int32 device tensor [B] on k's device")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous [B, Hq, d]")
    hq = q.shape[1]
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(desc, hq, max_seq_len, q.device)
    pg = ctypes.byref(paging) if paging is not None else None
    _check(lib.kvq_attn_decode_append(ctypes.byref(desc), cache.data_ptr(), pg, k.data_ptr(),
                                      v.data_ptr(), _dtype_code(k), k.stride(0), k.stride(1),
                                      positions.data_ptr(), q.data_ptr(), _dtype_code(q), hq,
                                      max_seq_len, float(softmax_scale), out.data_ptr(),
                                      _dtype_code(out), workspace.data_ptr(), workspace.numel(),
                                      _stream(q.device)), "kvq_attn_decode_append")
    return out


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
