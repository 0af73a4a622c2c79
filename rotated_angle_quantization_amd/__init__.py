"""kvq: angle-quantised KV cache and decode attention for AMD MI355X (gfx950).

Python face of libkvq (C ABI in include/kvq.h). The codec follows "TurboAngle:
Near-Lossless KV Cache Compression via Uniform Angle Quantization" (arXiv 2603.27467),
Abstract. Importing this package loads libkvq.so and fails if it has not been built.
"""

from ._lib import (  # noqa: F401
    EXPORTS, KVQ_F16, KVQ_F32, KvqError, LayerDesc, Paging, abi_version, alloc_cache, append,
    append_paged, attn_decode_append, attn_decode_paged, decode_paged, encode_paged, make_paging,
    paged_pool_bytes,
    alloc_workspace, attn_decode, attn_decode_static, attn_decode_varlen, attn_multi,
    attn_multi_workspace_bytes, attn_static_scratch_bytes,
    attn_num_splits,
    attn_workspace_bytes, cache_bytes, decode, default_scale, encode, layer_signs, lib,
    make_desc, tile_bytes,
    TriDesc, alloc_tri_cache, make_tri_desc, tri_attn_decode, tri_attn_workspace_bytes,
    tri_cache_bytes, tri_codebook, tri_codebook_device, tri_decode, tri_encode,
    tri_record_words, tri_tile_bytes, probe_read)
