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


class TriDesc(ctypes.Structure):
    """kvq_tri_desc: one triplet-coded layer (head dim 64/128, bits per square coordinate,
    per triplet norm and per leftover coordinate)."""

    _fields_ = [("head_dim", ctypes.c_uint32), ("num_kv_heads", ctypes.c_uint32),
                ("batch", ctypes.c_uint32), ("capacity", ctypes.c_uint32),
                ("bits_dir", ctypes.c_uint32), ("bits_norm", ctypes.c_uint32),
                ("bits_rest", ctypes.c_uint32), ("layer", ctypes.c_uint32),
                ("seed", ctypes.c_uint64)]

    def __repr__(self):
        return (f"TriDesc(d={self.head_dim}, hkv={self.num_kv_heads}, B={self.batch}, "
                f"cap={self.capacity}, bits=({self.bits_dir},{self.bits_norm},"
                f"{self.bits_rest}), layer={self.layer}, seed={self.seed})")


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
_PT = ctypes.POINTER(TriDesc)
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
    "kvq_tri_record_words": (_u32, [_PT]),
    "kvq_tri_tile_bytes": (_sz, [_PT]),
    "kvq_tri_cache_bytes": (_sz, [_PT]),
    "kvq_tri_codebook_doubles": (_sz, [_PT]),
    "kvq_tri_codebook": (ctypes.c_int, [_PT, ctypes.POINTER(ctypes.c_double)]),
    "kvq_tri_encode": (ctypes.c_int, [_PT, _v, _v, _v, _v, ctypes.c_int, _i64, _i64, _i64, _u32,
                                      _u32, _v]),
    "kvq_tri_decode": (ctypes.c_int, [_PT, _v, _v, _v, _v, ctypes.c_int, _u32, _u32, _v]),
    "kvq_tri_attn_workspace_bytes": (_sz, [_PT, _u32, _u32]),
    "kvq_tri_attn_decode": (ctypes.c_int, [_PT, _v, _v, _v, ctypes.c_int, _u32, _u32, _f32, _v,
                                           ctypes.c_int, _v, _sz, _v]),
    "kvq_probe_read": (ctypes.c_int, [_v, _sz, _v, _v]),
    "kvq_attn_static_scratch_bytes": (_sz, []),
    "kvq_attn_decode_static": (ctypes.c_int, [_P, _v, _v, ctypes.c_int, _u32, _u32, _f32, _v,
                                              ctypes.c_int, _v]),
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


# Argument checks made before any library call: the kernels take raw pointers, so a
# buffer smaller than the descriptor says, a tensor of the wrong shape, type or layout,
# or one in host memory would be read or written out of bounds on the device. Shapes
# and types are checked first, devices last.


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _float_tensor(t, name: str, shape: tuple, contiguous: bool = True) -> None:
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch tensor")
    _need(tuple(t.shape) == tuple(shape), f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    _need(t.dtype in (torch.float16, torch.float32), f"{name} must be float16 or float32, not {t.dtype}")
    if contiguous:
        _need(t.is_contiguous(), f"{name} must be contiguous")


def _index_tensor(t, name: str, n: int) -> None:
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch tensor")
    _need(t.dtype in (torch.int32, torch.uint32), f"{name} must be int32 (or uint32), not {t.dtype}")
    _need(t.dim() == 1 and t.numel() == n and t.is_contiguous(),
          f"{name} must be a contiguous 1-d tensor of {n} entries, got shape {tuple(t.shape)}")


def _byte_buffer(t, name: str, nbytes: int) -> None:
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch tensor")
    _need(t.dtype == torch.uint8 and t.is_contiguous(), f"{name} must be a contiguous uint8 tensor")
    _need(t.numel() >= nbytes, f"{name} holds {t.numel()} bytes, {nbytes} are needed")


def _kv_rows(k, v, shape: tuple) -> None:
    """K and V rows: the given shape, d contiguous, one dtype and one set of strides."""
    for t, name in ((k, "k"), (v, "v")):
        _float_tensor(t, name, shape, contiguous=False)
        _need(t.stride(-1) == 1, f"{name} must have its last (head_dim) axis contiguous")
    _need(k.dtype == v.dtype and k.stride() == v.stride(), "k and v must share dtype and strides")


def _same_device(*named) -> None:
    """Every tensor on one CUDA (HIP) device."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        _need(t.device.type == "cuda", f"{name} must be in GPU memory, not on {t.device}")
        if dev is None:
            dev = t.device
        _need(t.device == dev, f"{name} is on {t.device}, other arguments on {dev}")


def _layer_cache(desc, cache, name: str = "cache") -> None:
    n = cache_bytes(desc)
    _need(n > 0, f"invalid layer descriptor {desc!r}")
    _byte_buffer(cache, name, n)


def _check_out(out, q_shape) -> None:
    if out is not None:
        _float_tensor(out, "out", q_shape)


def _attn_out(out, q_shape, out_dtype, q):
    if out is None:
        return torch.empty(q_shape, dtype=out_dtype or q.dtype, device=q.device)
    return out


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
    _need(isinstance(k, torch.Tensor) and k.dim() == 4, "k/v must be [B, ntok, Hkv, d]")
    ntok = k.shape[1]
    _kv_rows(k, v, (desc.batch, ntok, desc.num_kv_heads, desc.head_dim))
    _layer_cache(desc, cache)
    _same_device(("cache", cache), ("k", k), ("v", v))
    _check(lib.kvq_encode(ctypes.byref(desc), cache.data_ptr(), k.data_ptr(), v.data_ptr(),
                          _dtype_code(k), k.stride(0), k.stride(1), k.stride(2), t0, ntok,
                          _stream(cache.device)), "kvq_encode")


def _token_rows(desc, k, v):
    """One token per sequence: [B, Hkv, d] (or [B, 1, Hkv, d]), d contiguous."""
    if isinstance(k, torch.Tensor) and isinstance(v, torch.Tensor) and k.dim() == 4 \
            and k.shape[1] == 1 and v.dim() == 4:
        k, v = k[:, 0], v[:, 0]
    _kv_rows(k, v, (desc.batch, desc.num_kv_heads, desc.head_dim))
    return k, v


def append(desc: LayerDesc, cache: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
           positions: torch.Tensor):
    """Encode one token per sequence at slot positions[b] of sequence b.
    k, v: [B, Hkv, d] (or [B, 1, Hkv, d]) with d contiguous, fp16 or fp32; positions:
    int32 device tensor [B]."""
    k, v = _token_rows(desc, k, v)
    _index_tensor(positions, "positions", desc.batch)
    _layer_cache(desc, cache)
    _same_device(("cache", cache), ("k", k), ("v", v), ("positions", positions))
    _check(lib.kvq_append(ctypes.byref(desc), cache.data_ptr(), k.data_ptr(), v.data_ptr(),
                          _dtype_code(k), k.stride(0), k.stride(1), positions.data_ptr(),
                          _stream(cache.device)), "kvq_append")


def decode(desc: LayerDesc, cache: torch.Tensor, t0: int, ntok: int,
           out_dtype=torch.float16, out: tuple | None = None):
    """Dequantise tokens [t0, t0 + ntok) -> (k_hat, v_hat), each [B, ntok, Hkv, d]."""
    shape = (desc.batch, ntok, desc.num_kv_heads, desc.head_dim)
    _layer_cache(desc, cache)
    if out is None:
        _same_device(("cache", cache))
        k_out = torch.empty(shape, dtype=out_dtype, device=cache.device)
        v_out = torch.empty(shape, dtype=out_dtype, device=cache.device)
    else:
        k_out, v_out = out
        _float_tensor(k_out, "k_out", shape)
        _float_tensor(v_out, "v_out", shape)
        _need(k_out.dtype == v_out.dtype, "k_out and v_out must share a dtype")
    _same_device(("cache", cache), ("k_out", k_out), ("v_out", v_out))
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
        # the shape's own status (INVALID_ARGUMENT, UNSUPPORTED or CAPACITY): the library
        # checks the shape before any pointer, so null pointers reach no device work
        st = lib.kvq_attn_decode(ctypes.byref(desc), None, None, KVQ_F16, num_q_heads, seq_len,
                                 0.0, None, KVQ_F16, None, 0, None)
        raise KvqError(st if st else 1, "kvq_attn_workspace_bytes")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def _query(desc, q, nq: int | None = None) -> int:
    """Query rows [B, Hq, d] (or [B, NQ, Hq, d] when nq is given); returns Hq."""
    _need(isinstance(q, torch.Tensor), "q must be a torch tensor")
    if nq is None:
        _need(q.dim() == 3, f"q must be [B, Hq, d], got shape {tuple(q.shape)}")
        hq = q.shape[1]
        _float_tensor(q, "q", (desc.batch, hq, desc.head_dim))
    else:
        _need(q.dim() == 4, f"q must be [B, NQ, Hq, d], got shape {tuple(q.shape)}")
        hq = q.shape[2]
        _float_tensor(q, "q", (desc.batch, nq, hq, desc.head_dim))
    return hq


def attn_decode(desc: LayerDesc, cache: torch.Tensor, q: torch.Tensor, seq_len: int,
                softmax_scale: float = 0.0, out_dtype=None, workspace=None, out=None):
    """o[b, h] = softmax(scale q.k_hat) v_hat over the first seq_len cached tokens.
    q: contiguous [B, Hq, d] (fp16 or fp32); returns [B, Hq, d]."""
    hq = _query(desc, q)
    _layer_cache(desc, cache)
    _check_out(out, q.shape)
    _same_device(("cache", cache), ("q", q), ("out", out), ("workspace", workspace))
    out = _attn_out(out, q.shape, out_dtype, q)
    if workspace is None:
        workspace = alloc_workspace(desc, hq, seq_len, q.device)
    _byte_buffer(workspace, "workspace", attn_workspace_bytes(desc, hq, seq_len))
    _check(lib.kvq_attn_decode(ctypes.byref(desc), cache.data_ptr(), q.data_ptr(),
                               _dtype_code(q), hq, seq_len, float(softmax_scale),
                               out.data_ptr(), _dtype_code(out), workspace.data_ptr(),
                               workspace.numel(), _stream(q.device)), "kvq_attn_decode")
    return out


def attn_decode_static(desc: LayerDesc, cache: torch.Tensor, q: torch.Tensor, seq_len: int,
                       softmax_scale: float = 0.0, out_dtype=None, out=None):
    """attn_decode without a workspace (kvq_attn_decode_static): the library's own fixed
    device scratch array serves as the workspace; nothing is allocated when out is
    given. Calls that may overlap on one GPU must be serialised by the caller."""
    _query(desc, q)
    _layer_cache(desc, cache)
    _check_out(out, q.shape)
    _same_device(("cache", cache), ("q", q), ("out", out))
    out = _attn_out(out, q.shape, out_dtype, q)
    _check(lib.kvq_attn_decode_static(ctypes.byref(desc), cache.data_ptr(), q.data_ptr(),
                                      _dtype_code(q), q.shape[1], seq_len, float(softmax_scale),
                                      out.data_ptr(), _dtype_code(out), _stream(q.device)),
           "kvq_attn_decode_static")
    return out


def attn_static_scratch_bytes() -> int:
    return lib.kvq_attn_static_scratch_bytes()


def attn_decode_varlen(desc: LayerDesc, cache: torch.Tensor, q: torch.Tensor,
                       seq_lens: torch.Tensor, max_seq_len: int, softmax_scale: float = 0.0,
                       out_dtype=None, workspace=None, out=None):
    """attn_decode with a length per sequence: entry b attends to its first seq_lens[b]
    cached tokens. seq_lens: int32 (or uint32 bits) device tensor [B], every entry
    <= max_seq_len (larger entries count as max_seq_len; 0 gives a zero output)."""
    hq = _query(desc, q)
    _index_tensor(seq_lens, "seq_lens", desc.batch)
    _layer_cache(desc, cache)
    _check_out(out, q.shape)
    _same_device(("cache", cache), ("q", q), ("seq_lens", seq_lens), ("out", out),
                 ("workspace", workspace))
    out = _attn_out(out, q.shape, out_dtype, q)
    if workspace is None:
        workspace = alloc_workspace(desc, hq, max_seq_len, q.device)
    _byte_buffer(workspace, "workspace", attn_workspace_bytes(desc, hq, max_seq_len))
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
    _need(isinstance(q, torch.Tensor) and q.dim() == 4, "q must be [B, NQ, Hq, d]")
    nq = q.shape[1]
    hq = _query(desc, q, nq)
    if seq_lens is not None:
        _index_tensor(seq_lens, "seq_lens", desc.batch)
    if paging is not None:
        _paging(desc, paging)
        _byte_buffer(cache, "pool", paged_pool_bytes(desc, paging.num_pages))
    else:
        _layer_cache(desc, cache)
    _check_out(out, q.shape)
    _same_device(("cache", cache), ("q", q), ("seq_lens", seq_lens), ("out", out),
                 ("workspace", workspace),
                 ("page_table", paging.table if paging is not None else None))
    out = _attn_out(out, q.shape, out_dtype, q)
    n = attn_multi_workspace_bytes(desc, hq, nq, seq_len)
    if n == 0:
        raise KvqError(1, "kvq_attn_multi_workspace_bytes")
    if workspace is None:
        workspace = torch.zeros(n, dtype=torch.uint8, device=q.device)
    _byte_buffer(workspace, "workspace", n)
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
    pg = Paging(page_table.data_ptr(), page_table.shape[1], num_pages)
    pg.table = page_table  # kept alive with the description, and checked against the layer
    return pg


def _paging(desc, paging) -> None:
    """The page table covers every sequence of the layer."""
    _need(isinstance(paging, Paging), "paging must come from make_paging")
    table = getattr(paging, "table", None)
    _need(table is not None, "paging must come from make_paging (it keeps the table tensor)")
    _need(table.shape[0] >= desc.batch, f"page table has {table.shape[0]} rows, the layer "
                                         f"has {desc.batch} sequences")


def encode_paged(desc: LayerDesc, pool: torch.Tensor, paging: Paging, k: torch.Tensor,
                 v: torch.Tensor, t0: int = 0):
    _need(isinstance(k, torch.Tensor) and k.dim() == 4, "k/v must be [B, ntok, Hkv, d]")
    _kv_rows(k, v, (desc.batch, k.shape[1], desc.num_kv_heads, desc.head_dim))
    _paging(desc, paging)
    _byte_buffer(pool, "pool", paged_pool_bytes(desc, paging.num_pages))
    _same_device(("pool", pool), ("k", k), ("v", v), ("page_table", paging.table))
    _check(lib.kvq_encode_paged(ctypes.byref(desc), pool.data_ptr(), ctypes.byref(paging),
                                k.data_ptr(), v.data_ptr(), _dtype_code(k), k.stride(0),
                                k.stride(1), k.stride(2), t0, k.shape[1], _stream(pool.device)),
           "kvq_encode_paged")


def append_paged(desc: LayerDesc, pool: torch.Tensor, paging: Paging, k: torch.Tensor,
                 v: torch.Tensor, positions: torch.Tensor):
    k, v = _token_rows(desc, k, v)
    _index_tensor(positions, "positions", desc.batch)
    _paging(desc, paging)
    _byte_buffer(pool, "pool", paged_pool_bytes(desc, paging.num_pages))
    _same_device(("pool", pool), ("k", k), ("v", v), ("positions", positions),
                 ("page_table", paging.table))
    _check(lib.kvq_append_paged(ctypes.byref(desc), pool.data_ptr(), ctypes.byref(paging),
                                k.data_ptr(), v.data_ptr(), _dtype_code(k), k.stride(0),
                                k.stride(1), positions.data_ptr(), _stream(pool.device)),
           "kvq_append_paged")


def decode_paged(desc: LayerDesc, pool: torch.Tensor, paging: Paging, t0: int, ntok: int,
                 out_dtype=torch.float16):
    shape = (desc.batch, ntok, desc.num_kv_heads, desc.head_dim)
    _paging(desc, paging)
    _byte_buffer(pool, "pool", paged_pool_bytes(desc, paging.num_pages))
    _same_device(("pool", pool), ("page_table", paging.table))
    k_out = torch.empty(shape, dtype=out_dtype, device=pool.device)
    v_out = torch.empty(shape, dtype=out_dtype, device=pool.device)
    _check(lib.kvq_decode_paged(ctypes.byref(desc), pool.data_ptr(), ctypes.byref(paging),
                                k_out.data_ptr(), v_out.data_ptr(), _dtype_code(k_out), t0, ntok,
                                _stream(pool.device)), "kvq_decode_paged")
    return k_out, v_out


def attn_decode_paged(desc: LayerDesc, pool: torch.Tensor, paging: Paging, q: torch.Tensor,
                      max_seq_len: int, seq_lens: torch.Tensor | None = None,
                      softmax_scale: float = 0.0, out_dtype=None, workspace=None, out=None):
    hq = _query(desc, q)
    if seq_lens is not None:
        _index_tensor(seq_lens, "seq_lens", desc.batch)
    _paging(desc, paging)
    _byte_buffer(pool, "pool", paged_pool_bytes(desc, paging.num_pages))
    _check_out(out, q.shape)
    _same_device(("pool", pool), ("q", q), ("seq_lens", seq_lens), ("out", out),
                 ("workspace", workspace), ("page_table", paging.table))
    out = _attn_out(out, q.shape, out_dtype, q)
    if workspace is None:
        workspace = alloc_workspace(desc, hq, max_seq_len, q.device)
    _byte_buffer(workspace, "workspace", attn_workspace_bytes(desc, hq, max_seq_len))
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
    k, v = _token_rows(desc, k, v)
    _index_tensor(positions, "positions", desc.batch)
    hq = _query(desc, q)
    if paging is not None:
        _paging(desc, paging)
        _byte_buffer(cache, "pool", paged_pool_bytes(desc, paging.num_pages))
    else:
        _layer_cache(desc, cache)
    _check_out(out, q.shape)
    _same_device(("cache", cache), ("k", k), ("v", v), ("positions", positions), ("q", q),
                 ("out", out), ("workspace", workspace),
                 ("page_table", paging.table if paging is not None else None))
    out = _attn_out(out, q.shape, out_dtype, q)
    if workspace is None:
        workspace = alloc_workspace(desc, hq, max_seq_len, q.device)
    _byte_buffer(workspace, "workspace", attn_workspace_bytes(desc, hq, max_seq_len))
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


# ------------------------------------------------------------------ triplet codec


def make_tri_desc(head_dim, num_kv_heads, batch, capacity, bits_dir, bits_norm, bits_rest,
                  layer=0, seed=0) -> TriDesc:
    return TriDesc(head_dim, num_kv_heads, batch, capacity, bits_dir, bits_norm, bits_rest,
                   layer, seed)


def tri_cache_bytes(desc: TriDesc) -> int:
    return lib.kvq_tri_cache_bytes(ctypes.byref(desc))


def tri_tile_bytes(desc: TriDesc) -> int:
    return lib.kvq_tri_tile_bytes(ctypes.byref(desc))


def tri_record_words(desc: TriDesc) -> int:
    return lib.kvq_tri_record_words(ctypes.byref(desc))


def tri_codebook(desc: TriDesc):
    """The layer's Lloyd-Max tables as computed by the library on the host (a float64
    numpy array; see kvq_tri_codebook for its order)."""
    import numpy as np
    n = lib.kvq_tri_codebook_doubles(ctypes.byref(desc))
    if n == 0:
        raise KvqError(1, "kvq_tri_codebook_doubles")
    buf = (ctypes.c_double * n)()
    _check(lib.kvq_tri_codebook(ctypes.byref(desc), buf), "kvq_tri_codebook")
    return np.frombuffer(buf, dtype=np.float64).copy()


def tri_codebook_device(desc: TriDesc, device="cuda") -> torch.Tensor:
    return torch.from_numpy(tri_codebook(desc)).to(device)


def alloc_tri_cache(desc: TriDesc, device="cuda") -> torch.Tensor:
    n = tri_cache_bytes(desc)
    if n == 0:
        raise KvqError(1, "kvq_tri_cache_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _tri_cache(desc, cache, codebook) -> None:
    n = tri_cache_bytes(desc)
    _need(n > 0, f"invalid triplet descriptor {desc!r}")
    _byte_buffer(cache, "cache", n)
    nd = lib.kvq_tri_codebook_doubles(ctypes.byref(desc))
    _need(isinstance(codebook, torch.Tensor) and codebook.dtype == torch.float64
          and codebook.is_contiguous() and codebook.numel() == nd,
          f"codebook must be the contiguous float64 table of {nd} values (tri_codebook_device)")


def tri_encode(desc: TriDesc, cache: torch.Tensor, codebook: torch.Tensor, k: torch.Tensor,
               v: torch.Tensor, t0: int = 0) -> None:
    """Triplet-code K/V tokens [t0, t0 + ntok): k, v [B, ntok, Hkv, d], d contiguous."""
    _need(isinstance(k, torch.Tensor) and k.dim() == 4, "k/v must be [B, ntok, Hkv, d]")
    ntok = k.shape[1]
    _kv_rows(k, v, (desc.batch, ntok, desc.num_kv_heads, desc.head_dim))
    _tri_cache(desc, cache, codebook)
    _same_device(("cache", cache), ("codebook", codebook), ("k", k), ("v", v))
    _check(lib.kvq_tri_encode(ctypes.byref(desc), cache.data_ptr(), codebook.data_ptr(),
                              k.data_ptr(), v.data_ptr(), _dtype_code(k), k.stride(0),
                              k.stride(1), k.stride(2), t0, ntok, _stream(cache.device)),
           "kvq_tri_encode")


def tri_decode(desc: TriDesc, cache: torch.Tensor, codebook: torch.Tensor, t0: int, ntok: int,
               out_dtype=torch.float16):
    """Dequantise tokens [t0, t0 + ntok) -> (k_hat, v_hat), each [B, ntok, Hkv, d]."""
    _tri_cache(desc, cache, codebook)
    _same_device(("cache", cache), ("codebook", codebook))
    shape = (desc.batch, ntok, desc.num_kv_heads, desc.head_dim)
    k_out = torch.empty(shape, dtype=out_dtype, device=cache.device)
    v_out = torch.empty(shape, dtype=out_dtype, device=cache.device)
    _check(lib.kvq_tri_decode(ctypes.byref(desc), cache.data_ptr(), codebook.data_ptr(),
                              k_out.data_ptr(), v_out.data_ptr(), _dtype_code(k_out), t0, ntok,
                              _stream(cache.device)), "kvq_tri_decode")
    return k_out, v_out


def tri_attn_workspace_bytes(desc: TriDesc, num_q_heads: int, seq_len: int) -> int:
    return lib.kvq_tri_attn_workspace_bytes(ctypes.byref(desc), num_q_heads, seq_len)


def tri_attn_decode(desc: TriDesc, cache: torch.Tensor, codebook: torch.Tensor, q: torch.Tensor,
                    seq_len: int, softmax_scale: float = 0.0, out_dtype=None, workspace=None,
                    out=None):
    """Decode attention over a triplet-coded cache: q [B, Hq, d] -> [B, Hq, d]."""
    _need(isinstance(q, torch.Tensor) and q.dim() == 3, "q must be [B, Hq, d]")
    hq = q.shape[1]
    _float_tensor(q, "q", (desc.batch, hq, desc.head_dim))
    _tri_cache(desc, cache, codebook)
    _check_out(out, q.shape)
    _same_device(("cache", cache), ("codebook", codebook), ("q", q), ("out", out),
                 ("workspace", workspace))
    out = _attn_out(out, q.shape, out_dtype, q)
    n = tri_attn_workspace_bytes(desc, hq, seq_len)
    if n == 0:
        raise KvqError(2, "kvq_tri_attn_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    _byte_buffer(workspace, "workspace", n)
    _check(lib.kvq_tri_attn_decode(ctypes.byref(desc), cache.data_ptr(), codebook.data_ptr(),
                                   q.data_ptr(), _dtype_code(q), hq, seq_len,
                                   float(softmax_scale), out.data_ptr(), _dtype_code(out),
                                   workspace.data_ptr(), workspace.numel(), _stream(q.device)),
           "kvq_tri_attn_decode")
    return out


# ------------------------------------------------------------------ streaming probe


def probe_read(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Read every byte of `buf` once on the device (kvq_probe_read); sink: a device
    tensor of at least 256 bytes on the same device."""
    _need(isinstance(buf, torch.Tensor) and buf.is_contiguous(), "buf must be a contiguous tensor")
    _need(isinstance(sink, torch.Tensor) and sink.is_contiguous()
          and sink.numel() * sink.element_size() >= 256, "sink must hold at least 256 bytes")
    _same_device(("buf", buf), ("sink", sink))
    nbytes = buf.numel() * buf.element_size()
    _check(lib.kvq_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), _stream(buf.device)),
           "kvq_probe_read")
