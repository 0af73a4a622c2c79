/*
 * kvq.h - C ABI of libkvq: an angle-quantised, bit-packed KV cache for AMD MI355X
 * (gfx950), with decode attention that runs directly on the packed codes.
 *
 * The codec is the one described in "TurboAngle: Near-Lossless KV Cache Compression
 * via Uniform Angle Quantization" (arXiv 2603.27467), Abstract: each head vector is
 * multiplied by a seeded random sign diagonal and put through a normalised fast
 * Walsh-Hadamard transform; neighbouring coordinates are paired into (radius, angle);
 * each angle is rounded to one of n evenly spaced directions (n set per layer and
 * separately for K and V); key radii get 8 linear bits against a per-vector fp16
 * scale, value radii 4 bits on a log scale between per-vector fp16 min and max.
 * Attention reconstructs keys and values from the codes on the fly and never writes
 * a dequantised cache, the property stressed for fused codec kernels in "OCTOPUS:
 * Joint Triplet Quantization for KV Cache via Octahedral Parametrization" (TL;DR and
 * Why it matters).
 *
 * Readings of steps the abstract leaves open (bin placement, tie rules, fp16
 * parameters, sign generator, byte layout) are stated at each declaration.
 *
 * General conventions
 *  - Every buffer is owned by the caller: the cache, inputs, outputs and workspace.
 *    The library allocates no device memory and never synchronises; its only
 *    global state is a per-device cache of an occupancy query (filled on first use,
 *    the same value on every thread). All device pointers must come from
 *    hipMalloc-class allocations on the current device.
 *  - Device work is enqueued on `hip_stream` (a hipStream_t; NULL = the null
 *    stream). KVQ_OK means the work was enqueued; kernel faults surface at the
 *    caller's next synchronisation on that stream.
 *  - Arguments are validated on the host before any HIP call; a rejected call
 *    enqueues nothing. Calls are thread-safe and re-entrant.
 *  - Inputs must be finite; non-finite values are outside the contract.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 10
#define KVQ_TILE_TOKENS 64

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad shape, stride or alignment */
  KVQ_ERR_UNSUPPORTED = 2,      /* valid request that this build has no kernel for */
  KVQ_ERR_CAPACITY = 3,         /* token range beyond the cache capacity */
  KVQ_ERR_WORKSPACE = 4,        /* workspace missing or smaller than required */
  KVQ_ERR_HIP = 5               /* the HIP runtime rejected a launch */
} kvq_status;

typedef enum { KVQ_F16 = 0, KVQ_F32 = 1 } kvq_dtype;

/*
 * One layer's compressed cache. Plain data: read during a call, never retained.
 *  head_dim     d; 64 or 128 (a power of two; the pairing needs d even).
 *  num_kv_heads Hkv >= 1.  batch B >= 1.
 *  capacity     token slots per (batch, kv head), in [1, 2^31 - 64]; rounded up to
 *               whole tiles of 64 slots in the byte layout.
 *  n_bins_k/v   angle bins n for K and V, in [2, 256]; each code takes ceil(log2 n)
 *               bits (per-layer early boost = a different pair per layer).
 *  layer, seed  select the sign diagonal (see kvq_layer_signs).
 */
typedef struct {
  uint32_t head_dim;
  uint32_t num_kv_heads;
  uint32_t batch;
  uint32_t capacity;
  uint32_t n_bins_k;
  uint32_t n_bins_v;
  uint32_t layer;
  uint32_t reserved; /* must be 0 */
  uint64_t seed;
} kvq_layer_desc;

int kvq_abi_version(void);
const char* kvq_status_string(kvq_status status);

/*
 * Bytes of one layer's cache, or 0 if the descriptor is invalid. Host only.
 *
 * Byte layout (this library's own; the abstract fixes no format). P = d/2 pairs,
 * bk = ceil(log2 n_bins_k), bv = ceil(log2 n_bins_v). The cache is
 * [batch][kv_head][tile][tile_bytes], tile = 64 token slots; every entry point takes
 * the cache pointer 16-byte aligned (tiles are read as 16-byte vectors; tile_bytes is
 * a multiple of 16). A tile holds, in order:
 *   KA key angle codes   token-major 32-bit words: word w of slot t at 4*(w*64+t);
 *                        slot t's bit string (P*bk bits) has pair i's code at bits
 *                        [i*bk, (i+1)*bk)
 *   KR key radius codes  token-major words, word w of slot t at 4*(w*64+t); byte j
 *                        of word w = 8-bit code of pair 4w+j
 *   KS key scale         fp16 per slot, slot t at 2t
 *   VA value angle codes pair-major words: word w of pair i at 4*(w*P+i); pair i's
 *                        bit string (64*bv bits) has slot t's code at [t*bv, (t+1)*bv)
 *   VR value radius codes pair-major words: word w of pair i at 4*(w*P+i); slot t's
 *                        4-bit code at bits [4t, 4t+4)
 *   VP value parameters  (s_min fp16, s_max fp16) per slot, slot t at 4t
 * Bit strings are little-endian (bit b = bit b%32 of word b/32). Key planes are
 * token-major so a wave reads them with one lane per token; value planes are
 * pair-major so a wave reads them with one lane per pair.
 */
size_t kvq_cache_bytes(const kvq_layer_desc* desc);

/* Bytes of one 64-slot tile (see kvq_cache_bytes), or 0 if invalid. Host only. */
size_t kvq_tile_bytes(uint32_t head_dim, uint32_t n_bins_k, uint32_t n_bins_v);

/*
 * The sign diagonal of (seed, layer), written to out_host[0..d) as +1 / -1.
 * Host only. Reading of the abstract's random diagonal rotation: one diagonal per
 * layer, shared by K, V and all heads, drawn with SplitMix64 (Steele, Lea, Flood,
 * OOPSLA 2014): mix(z) adds 0x9E3779B97F4A7C15 then applies the two published
 * xor-shift-multiply rounds; sign[i] = -1 iff bit 63 of mix(mix(seed ^ layer) + i)
 * is set. d must be a power of two in [1, 4096].
 */
kvq_status kvq_layer_signs(uint64_t seed, uint32_t layer, uint32_t d, int8_t* out_host);

/*
 * Encode (append) tokens [t0, t0 + ntok) of K and V into the cache.
 *
 * k, v: device tensors of shape [B, ntok, Hkv, d] with element strides
 * (stride_b, stride_t, stride_h) shared by k and v, and d contiguous; element
 * [b, j, h, e] is at k + b*stride_b + j*stride_t + h*stride_h + e. dtype f16 or f32.
 * Pointers must be aligned to two elements and the strides even.
 *
 * Per (token, kv head) vector x (TurboAngle, Abstract, with this library's readings):
 *   y = H_d (sign * x) / sqrt(d)           natural (Sylvester) order
 *   pair i = (y[2i], y[2i+1]); r = hypot; theta = atan2(y[2i+1], y[2i])
 *   angle code = floor(theta * n / (2 pi) + 1/2) mod n; zero pair -> 0
 *     (bin centres at 2 pi c / n)
 *   keys:   s = fp16(max r) (round to nearest even, saturated at 65504);
 *           radius code = clamp(floor(255 r / s + 1/2), 0, 255); s = 0 -> codes 0
 *   values: s_max = fp16(max r), s_min = fp16(max(min r, 2^-14));
 *           L = ln(s_max / s_min); code = 0 if r < s_min, else
 *           clamp(floor(15 ln(r / s_min) / L + 1/2), 0, 15); s_max <= s_min -> 0
 * The transform and the fp16 parameters are computed in IEEE binary64. Each code is
 * taken from an fp32 estimate only when the estimate is farther from the decision
 * boundary than its worst-case error; otherwise the binary64 formula above decides.
 * Codes are therefore those of a binary64 evaluation, reproducible across runs and
 * launch shapes. Slots outside [t0, t0 + ntok) are left unchanged, so a chunked
 * append produces the same bytes as a one-shot encode.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (d not 64/128), CAPACITY (t0 + ntok >
 * capacity), HIP. ntok = 0 enqueues nothing and returns KVQ_OK.
 */
kvq_status kvq_encode(const kvq_layer_desc* desc, void* cache, const void* k, const void* v,
                      kvq_dtype in_dtype, int64_t stride_b, int64_t stride_t,
                      int64_t stride_h, uint32_t t0, uint32_t ntok, void* hip_stream);

/*
 * Append one token per sequence, each at its own slot: the decode-loop step for a batch
 * whose sequences have different lengths. Sequence b's new K and V rows are encoded
 * into slot positions[b] of its cache, with exactly the codes and bytes kvq_encode
 * would write for that token (neighbouring slots keep their bytes).
 * k, v: device tensors holding one token per sequence; element i of kv head h of
 *   sequence b at k[b * stride_b + h * stride_h + i] (elements), d contiguous,
 *   in_dtype f16 or f32, pointers aligned to two elements, strides even.
 * positions: device array of B slots (uint32, 4-byte aligned), read by the kernel on
 *   the given stream; an entry >= capacity writes nothing for that sequence.
 * Errors: INVALID_ARGUMENT (also a null or misaligned positions), UNSUPPORTED (d not
 * 64/128), HIP.
 */
kvq_status kvq_append(const kvq_layer_desc* desc, void* cache, const void* k, const void* v,
                      kvq_dtype in_dtype, int64_t stride_b, int64_t stride_h,
                      const uint32_t* positions, void* hip_stream);

/*
 * Dequantise tokens [t0, t0 + ntok) back to vectors, inverting the encoding of
 * "TurboAngle: Near-Lossless KV Cache Compression via Uniform Angle Quantization"
 * (arXiv 2603.27467), Abstract: x_hat = sign * H_d y_hat / sqrt(d)
 * with y_hat[2i] = r_hat cos(2 pi c / n), y_hat[2i+1] = r_hat sin(2 pi c / n);
 * key r_hat = code * s / 255; value r_hat = s_min * exp(code * L / 15) (s_max when
 * s_max <= s_min). Arithmetic in fp32.
 * k_out, v_out: contiguous device tensors [B, ntok, Hkv, d] of out_dtype, 16-byte
 * aligned (rows are written as 8- and 16-byte vectors).
 * Errors: as kvq_encode.
 */
kvq_status kvq_decode(const kvq_layer_desc* desc, const void* cache, void* k_out,
                      void* v_out, kvq_dtype out_dtype, uint32_t t0, uint32_t ntok,
                      void* hip_stream);

/*
 * Decode attention for one new query token per sequence, straight from the codes of
 * "TurboAngle: Near-Lossless KV Cache Compression via Uniform Angle Quantization"
 * (arXiv 2603.27467), Abstract, reconstructing keys and values on the fly without
 * writing a dequantised cache ("OCTOPUS: Joint Triplet Quantization for KV Cache via
 * Octahedral Parametrization", Why it matters):
 *   o[b, h] = sum_j softmax_j(scale <q[b, h], k_hat[b, j, h/G]>) v_hat[b, j, h/G]
 * over j < seq_len, G = Hq / Hkv (grouped-query attention: query head h reads kv
 * head floor(h / G)). Scores are formed in the rotated domain (the query is rotated
 * once; <q, k_hat> = <R q, y_hat_k>), probabilities weight rotated-domain values,
 * and one inverse transform per output head brings o back. Work is split over the
 * sequence (flash-decoding style); the last workgroup of each (batch, kv head) to
 * finish merges the partial (max, sum, vector) triples with a log-sum-exp combine, so
 * the whole operation is one kernel launch. Scores, softmax and
 * all sums in fp32; where the value sum runs on the matrix cores (the variants chosen
 * for most shapes) its operands, weights and rebuilt value elements, are rounded to
 * fp16 (about 2^-11 relative per term; measured within 5.4e-4 relative L2 of the
 * float64 definition, against a bound of 2e-3).
 *
 * q:   contiguous device tensor [B, Hq, d], q_dtype f16 or f32.
 * out: contiguous device tensor [B, Hq, d], out_dtype f16 or f32.
 * softmax_scale <= 0 selects 1/sqrt(d).
 * workspace: device buffer of at least kvq_attn_workspace_bytes(desc, Hq, seq_len)
 *   bytes, 256-byte aligned, owned by the caller. It must be zero-filled once after
 *   allocation; every call that completes leaves it ready for the next (its split
 *   counters back at zero). It holds the rotated queries and split partials and, for a
 *   layer with n <= 32 for K or V, a copy of the first ceil(seq_len / 64) tiles of
 *   every (sequence, kv head) with those 1- to 5-bit angle codes re-packed at 6 bits
 *   (the kernels read 6- to 8-bit codes; the copy is written by a launch of its own on
 *   the same stream before the attention launch) and B lengths for the fused step.
 *   Calls that share one workspace must not run concurrently (one stream).
 * Supported: Hq = G * Hkv with G in {1, 2, 4, 8}; every n in [2, 256] for K and V;
 *   1 <= seq_len <= capacity. kvq_attn_workspace_bytes returns 0 for shapes outside
 *   this set (and for invalid arguments).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED, CAPACITY, WORKSPACE, HIP.
 */
size_t kvq_attn_workspace_bytes(const kvq_layer_desc* desc, uint32_t num_q_heads,
                                uint32_t seq_len);

kvq_status kvq_attn_decode(const kvq_layer_desc* desc, const void* cache, const void* q,
                           kvq_dtype q_dtype, uint32_t num_q_heads, uint32_t seq_len,
                           float softmax_scale, void* out, kvq_dtype out_dtype,
                           void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * kvq_attn_decode with a length per sequence, for batches whose sequences have grown
 * to different lengths (a decode loop over ragged requests). Entry b attends to its
 * first seq_lens[b] cached tokens.
 * seq_lens: device array of B lengths (uint32, 4-byte aligned, one per sequence), read
 *   by the kernel on the given stream, so it may be produced by earlier work on that
 *   stream. Entries above max_seq_len are treated as max_seq_len; an entry of 0 gives
 *   an all-zero output for that sequence.
 * max_seq_len: host bound, 1 <= max_seq_len <= capacity; the split plan and the
 *   workspace size are those of kvq_attn_decode at seq_len = max_seq_len (use
 *   kvq_attn_workspace_bytes(desc, Hq, max_seq_len)). Workgroups of splits past an
 *   entry's length exit at once.
 * Everything else (q, out, scale, workspace contract, supported shapes) is as for
 * kvq_attn_decode; with every entry equal to max_seq_len the result is bitwise that
 * of kvq_attn_decode(..., seq_len = max_seq_len, ...).
 * Errors: INVALID_ARGUMENT (also a null or misaligned seq_lens), UNSUPPORTED, CAPACITY,
 * WORKSPACE, HIP.
 */
kvq_status kvq_attn_decode_varlen(const kvq_layer_desc* desc, const void* cache, const void* q,
                                  kvq_dtype q_dtype, uint32_t num_q_heads,
                                  const uint32_t* seq_lens, uint32_t max_seq_len,
                                  float softmax_scale, void* out, kvq_dtype out_dtype,
                                  void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Multi-query attention over the compressed cache: num_queries query tokens per
 * sequence (a chunk of prefill, or the draft tokens of a speculative step under
 * verification), whose own K/V are the last num_queries of the seq_len cached tokens.
 * Query token j (0-based) attends causally to tokens [0, seq_len - num_queries + j + 1):
 *   o[b, j, h] = sum_t softmax_t(scale <q[b, j, h], k_hat[b, t, h/G]>) v_hat[b, t, h/G].
 * The num_queries * G query rows of a kv head share every key and value, so the scores
 * and the value sum are dense products and run on the matrix cores with fp16 operands
 * (rotated queries, reconstructed rotated keys, probabilities, reconstructed rotated
 * values) and fp32 accumulation; softmax and the merge are fp32. Same rotated-domain
 * formulation and single inverse transform per output row as kvq_attn_decode.
 * q:   contiguous device tensor [B, num_queries, Hq, d], q_dtype f16 or f32.
 * out: contiguous device tensor [B, num_queries, Hq, d], out_dtype f16 or f32.
 * workspace: at least kvq_attn_multi_workspace_bytes(desc, Hq, num_queries, seq_len)
 *   bytes, 256-byte aligned, zero-filled once after allocation; every completed call
 *   leaves its split counters at zero. Calls sharing a workspace must not overlap.
 * Supported: d in {64, 128}; G in {1, 2, 4, 8}; num_queries * G <= 32; every n in
 *   [2, 256] for K and V (n <= 32 through the widened copy described at
 *   kvq_attn_workspace_bytes, after the partials in the workspace; not for the paged
 *   form); 1 <= num_queries <= seq_len <= capacity.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED, CAPACITY, WORKSPACE, HIP.
 */
size_t kvq_attn_multi_workspace_bytes(const kvq_layer_desc* desc, uint32_t num_q_heads,
                                      uint32_t num_queries, uint32_t seq_len);

kvq_status kvq_attn_multi(const kvq_layer_desc* desc, const void* cache, const void* q,
                          kvq_dtype q_dtype, uint32_t num_q_heads, uint32_t num_queries,
                          uint32_t seq_len, float softmax_scale, void* out, kvq_dtype out_dtype,
                          void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Paged caches. A paged layer keeps its tiles in a pool of pages shared by all
 * sequences, laid out [page][kv_head][tile_bytes] (one page = one 64-slot tile of every
 * kv head), and a page table maps tile t of sequence b to page
 * page_table[b * pages_per_seq + t]. Sequences then grow page by page without a
 * contiguous reservation, and a page can be dropped from attention by mapping it to no
 * page. The codes and bytes of a tile are exactly those of the contiguous layout. (The
 * pages describe the codec and its attention, not how cache memory is handed out: this
 * layout is the usual serving one, a pool of pages plus a table per sequence.)
 * page_table: device int32 array [batch][pages_per_seq], 4-byte aligned, read by the
 *   kernels on the given stream. An entry outside [0, num_pages) maps its tile to no
 *   page: encode and append write nothing there, dequantisation returns zero vectors
 *   for its slots, attention treats its slots as absent (a sequence with no present
 *   slot gives a zero output).
 * pages_per_seq >= ceil(capacity / 64); num_pages >= 1 (pages in the pool).
 * Each *_paged call is its contiguous counterpart with the cache argument replaced by
 * (pool, paging); arguments and errors are as documented there, plus INVALID_ARGUMENT
 * for a null or misaligned paging description.
 */
typedef struct {
  const int32_t* page_table;
  uint32_t pages_per_seq;
  uint32_t num_pages;
} kvq_paging;

/* Bytes of a pool of num_pages pages for this layer (0 if the descriptor is invalid). */
size_t kvq_paged_pool_bytes(const kvq_layer_desc* desc, uint32_t num_pages);

kvq_status kvq_encode_paged(const kvq_layer_desc* desc, void* pool, const kvq_paging* paging,
                            const void* k, const void* v, kvq_dtype in_dtype, int64_t stride_b,
                            int64_t stride_t, int64_t stride_h, uint32_t t0, uint32_t ntok,
                            void* hip_stream);

kvq_status kvq_append_paged(const kvq_layer_desc* desc, void* pool, const kvq_paging* paging,
                            const void* k, const void* v, kvq_dtype in_dtype, int64_t stride_b,
                            int64_t stride_h, const uint32_t* positions, void* hip_stream);

kvq_status kvq_decode_paged(const kvq_layer_desc* desc, const void* pool,
                            const kvq_paging* paging, void* k_out, void* v_out,
                            kvq_dtype out_dtype, uint32_t t0, uint32_t ntok, void* hip_stream);

/* Decode attention over a paged cache; seq_lens may be null (every sequence attends to
 * max_seq_len tokens) or a device array of per-sequence lengths as for
 * kvq_attn_decode_varlen. Workspace as kvq_attn_decode at seq_len = max_seq_len.
 * Layers with n <= 32 for K or V return UNSUPPORTED (no widened copy of a pool). */
kvq_status kvq_attn_decode_paged(const kvq_layer_desc* desc, const void* pool,
                                 const kvq_paging* paging, const void* q, kvq_dtype q_dtype,
                                 uint32_t num_q_heads, const uint32_t* seq_lens,
                                 uint32_t max_seq_len, float softmax_scale, void* out,
                                 kvq_dtype out_dtype, void* workspace, size_t workspace_bytes,
                                 void* hip_stream);

/* Multi-query attention over a ragged batch: sequence b holds L_b = min(seq_lens[b],
 * max_seq_len) tokens (seq_lens: device uint32 array [B], 4-byte aligned) whose last
 * num_queries are the query tokens' own, so query j attends to tokens
 * [0, L_b - num_queries + j + 1); a query that sees no token (L_b < num_queries - j)
 * gives a zero row. Sizes, workspace and errors as kvq_attn_multi at
 * seq_len = max_seq_len (num_queries <= max_seq_len). With every length equal to
 * max_seq_len the result is that of kvq_attn_multi. */
kvq_status kvq_attn_multi_varlen(const kvq_layer_desc* desc, const void* cache, const void* q,
                                 kvq_dtype q_dtype, uint32_t num_q_heads, uint32_t num_queries,
                                 const uint32_t* seq_lens, uint32_t max_seq_len,
                                 float softmax_scale, void* out, kvq_dtype out_dtype,
                                 void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * One decode step in one launch: kvq_append, then decode attention over the appended
 * sequences. For every sequence b, the token with K/V rows k, v [B, Hkv, d] (element
 * strides stride_b, stride_h; d contiguous; fp16 or fp32 as in_dtype) is coded into
 * slot positions[b] (device uint32 array [B]) exactly as kvq_append codes it, and query
 * q [B, Hq, d] then attends to min(positions[b] + 1, max_seq_len) tokens. The codes are
 * those of "TurboAngle: Near-Lossless KV Cache Compression via Uniform Angle
 * Quantization" (arXiv 2603.27467), Abstract, so the cache bytes and the output equal
 * those of kvq_append followed by kvq_attn_decode_varlen with seq_lens = positions + 1.
 * A slot at or past the capacity is not written (its sequence attends to max_seq_len
 * tokens); with paging, a slot whose page is absent is not written either. The token is
 * coded inside the attention kernel by the wave that reads its tile, while the other
 * waves stream their tiles.
 * paging: null for a contiguous cache, else the pool's page table as for the *_paged
 * calls (cache is then the pool). Workspace as kvq_attn_decode at seq_len = max_seq_len.
 * Layers with n <= 32 for K or V run as kvq_append, a launch that writes the lengths
 * min(positions[b] + 1, max_seq_len) into the workspace, and kvq_attn_decode_varlen
 * over the widened copy (same results, three launches; every argument is checked before
 * the cache is written); with a paged pool they return UNSUPPORTED.
 * Errors: as kvq_attn_decode (max_seq_len in [1, capacity]) and kvq_append.
 */
kvq_status kvq_attn_decode_append(const kvq_layer_desc* desc, void* cache,
                                  const kvq_paging* paging, const void* k, const void* v,
                                  kvq_dtype in_dtype, int64_t stride_b, int64_t stride_h,
                                  const uint32_t* positions, const void* q, kvq_dtype q_dtype,
                                  uint32_t num_q_heads, uint32_t max_seq_len,
                                  float softmax_scale, void* out, kvq_dtype out_dtype,
                                  void* workspace, size_t workspace_bytes, void* hip_stream);

/* Multi-query attention over a paged cache: kvq_attn_multi with the cache replaced by
 * (pool, paging); tokens of tiles mapped to no page are left out of every query's
 * softmax (a query that sees no present token gives a zero row). seq_lens: null (every
 * sequence is max_seq_len tokens long) or per-sequence lengths as for
 * kvq_attn_multi_varlen. */
kvq_status kvq_attn_multi_paged(const kvq_layer_desc* desc, const void* pool,
                                const kvq_paging* paging, const void* q, kvq_dtype q_dtype,
                                uint32_t num_q_heads, uint32_t num_queries,
                                const uint32_t* seq_lens, uint32_t max_seq_len,
                                float softmax_scale, void* out, kvq_dtype out_dtype,
                                void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Allocation-free decode attention, for callers that cannot allocate device memory or
 * pass a workspace (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): kvq_attn_decode with its workspace taken from a fixed device
 * array inside this library, kvq_attn_static_scratch_bytes() = 8 MiB on each GPU the
 * library runs on (held until the process ends; its address is looked up once per
 * device). Arguments, results and errors are those of kvq_attn_decode, except that a
 * shape whose kvq_attn_workspace_bytes exceeds the array returns KVQ_ERR_WORKSPACE
 * before any device work. The call enqueues a small fill kernel that zeroes the split
 * counters, then the attention kernel; it allocates nothing. All calls on one GPU share
 * its array, which keeps the last call's contents: calls that may overlap on one GPU
 * (different streams, or concurrent host threads) race and must be serialised by the
 * caller.
 */
size_t kvq_attn_static_scratch_bytes(void);

kvq_status kvq_attn_decode_static(const kvq_layer_desc* desc, const void* cache, const void* q,
                                  kvq_dtype q_dtype, uint32_t num_q_heads, uint32_t seq_len,
                                  float softmax_scale, void* out, kvq_dtype out_dtype,
                                  void* hip_stream);

/* Number of sequence splits (workgroups per (batch, kv head)) kvq_attn_decode uses for
 * this shape (host only; 0 if the arguments are invalid or the shape is one decode
 * attention does not serve). Each split covers a whole number of 64-token tiles. */
uint32_t kvq_attn_num_splits(const kvq_layer_desc* desc, uint32_t num_q_heads,
                             uint32_t seq_len);

/* ===================================================================================
 * Triplet (octahedral) codec: the variant summarised for "OCTOPUS: Joint Triplet
 * Quantization for KV Cache via Octahedral Parametrization" (TL;DR, What is new). After
 * the same seeded sign diagonal and normalised Walsh-Hadamard transform, a vector y is
 * scaled to unit length by its norm N (stored as fp16); its coordinates are taken three
 * at a time; each triplet's direction goes to the square [-1, 1]^2 through the
 * octahedral parametrisation, and the two square coordinates and the triplet's norm are
 * quantised with Lloyd-Max quantisers fitted to the exact marginals these quantities
 * have for a uniformly random unit vector (the page's "implementation-matched
 * marginals"); the 1 or 2 coordinates left over (d = 64 or 128) get a Lloyd-Max
 * quantiser of their own. The bit split between direction and norm is a parameter.
 * Readings of the open steps:
 *  - octahedral map: p = w / |w|_1; p3 >= 0 keeps (p1, p2), otherwise the point folds to
 *    ((1 - |p2|) sgn p1, (1 - |p1|) sgn p2), sgn(0) = +1; a zero triplet maps to (0, 0);
 *  - marginals: square coordinate f(s) = [2(1-s)/(2s^2+(1-s)^2) + 2s/(s^2+2(1-s)^2)]
 *    / sqrt(s^2+(1-s)^2) for s = |s| (up to a constant); triplet norm
 *    r^2 (1 - r^2)^((d-5)/2) on [0, 1]; one coordinate (1 - u^2)^((d-3)/2) on [-1, 1];
 *  - Lloyd-Max: the fixed point of the centroid conditions (every level the conditional
 *    mean of its cell, boundaries at midpoints), started at the (i + 1/2) / 2^b
 *    quantiles and solved to a residual of 1e-15; cell integrals by 40-point
 *    Gauss-Legendre rules, cells split at 0 for the symmetric densities; a value takes
 *    the nearest level, the lower one at an exact midpoint;
 *  - reconstruction: N_hat rho_hat w_hat per triplet (w_hat = the inverse octahedral
 *    map of the two levels, normalised), N_hat u_hat per leftover coordinate, then the
 *    inverse rotation; keys and values use the same codec.
 * =================================================================================== */

/*
 * One triplet-coded layer.
 *  head_dim           64 or 128.
 *  num_kv_heads, batch, capacity   as in kvq_layer_desc (capacity <= 2^31 - 64).
 *  bits_dir           bits of each of the two square coordinates, 1..6.
 *  bits_norm          bits of the triplet norm, 1..6.
 *  bits_rest          bits of each leftover coordinate, 1..8.
 *  layer, seed        select the sign diagonal (kvq_layer_signs).
 */
typedef struct {
  uint32_t head_dim;
  uint32_t num_kv_heads;
  uint32_t batch;
  uint32_t capacity;
  uint32_t bits_dir;
  uint32_t bits_norm;
  uint32_t bits_rest;
  uint32_t layer;
  uint64_t seed;
} kvq_tri_desc;

/*
 * Sizes (host only; 0 for an invalid descriptor). A token-head record is the bit string
 * (LSB-first in 32-bit words): the fp16 bits of N in [0, 16), then triplet j's fields at
 * 16 + j * (2 bits_dir + bits_norm): s code, t code, norm code (in that order, each
 * LSB-first), then the leftover codes of bits_rest bits; padded to whole words. A tile of
 * 64 slots holds the key plane then the value plane, each word-interleaved by slot (word
 * w of slot t at 4 (w * 64 + t)); the cache is [batch][kv head][tile][tile bytes].
 */
uint32_t kvq_tri_record_words(const kvq_tri_desc* desc);
size_t kvq_tri_tile_bytes(const kvq_tri_desc* desc);
size_t kvq_tri_cache_bytes(const kvq_tri_desc* desc);

/*
 * The layer's quantisers (host only): writes kvq_tri_codebook_doubles(desc) doubles to
 * out_host: the square-coordinate levels (2^bits_dir), the norm levels (2^bits_norm),
 * the leftover levels (2^bits_rest), then the three sets of decision boundaries
 * (2^b - 1 each, the midpoints), all ascending. Computed on the host by Newton's method
 * on the Lloyd-Max centroid conditions (milliseconds to a few seconds); the caller keeps
 * the table in device memory and passes it to the calls below. Depends only on
 * (head_dim, bits).
 */
size_t kvq_tri_codebook_doubles(const kvq_tri_desc* desc);
kvq_status kvq_tri_codebook(const kvq_tri_desc* desc, double* out_host);

/*
 * Encode K/V tokens [t0, t0 + ntok) (inputs as for kvq_encode: [B, ntok, Hkv, d],
 * strides in elements, d contiguous, fp16 or fp32). The transform, N, the triplet norms,
 * the square coordinates and every decision are taken in IEEE binary64. codebook: the
 * device copy of kvq_tri_codebook's table. Slots outside the range keep their bytes.
 * Errors: INVALID_ARGUMENT (also for batch * ntok * num_kv_heads above 2^32 - 256),
 * UNSUPPORTED (d not 64/128), CAPACITY, HIP.
 */
kvq_status kvq_tri_encode(const kvq_tri_desc* desc, void* cache, const double* codebook,
                          const void* k, const void* v, kvq_dtype in_dtype, int64_t stride_b,
                          int64_t stride_t, int64_t stride_h, uint32_t t0, uint32_t ntok,
                          void* hip_stream);

/* Dequantise tokens [t0, t0 + ntok) to contiguous [B, ntok, Hkv, d] outputs (fp32
 * arithmetic). Errors as kvq_tri_encode. */
kvq_status kvq_tri_decode(const kvq_tri_desc* desc, const void* cache, const double* codebook,
                          void* k_out, void* v_out, kvq_dtype out_dtype, uint32_t t0,
                          uint32_t ntok, void* hip_stream);

/*
 * Decode attention over a triplet-coded cache: the definition of kvq_attn_decode with
 * keys and values reconstructed from the triplet codes (rotated domain, one inverse
 * transform per output). Two launches: the splits write partial (max, sum, vector)
 * triples to the workspace, then a merge kernel combines them. The workspace
 * (kvq_tri_attn_workspace_bytes, 256-byte aligned) needs no initialisation. G in
 * {1, 2, 4, 8}. Errors: INVALID_ARGUMENT, UNSUPPORTED, CAPACITY, WORKSPACE, HIP.
 */
size_t kvq_tri_attn_workspace_bytes(const kvq_tri_desc* desc, uint32_t num_q_heads,
                                    uint32_t seq_len);
kvq_status kvq_tri_attn_decode(const kvq_tri_desc* desc, const void* cache,
                               const double* codebook, const void* q, kvq_dtype q_dtype,
                               uint32_t num_q_heads, uint32_t seq_len, float softmax_scale,
                               void* out, kvq_dtype out_dtype, void* workspace,
                               size_t workspace_bytes, void* hip_stream);

/* ===================================================================================
 * Read-only streaming probe (context for the roofline of the cache-reading kernels; no
 * codec work): reads `bytes` of device memory at `buf` once with 16-byte loads, as a
 * plain streaming kernel would, and returns. `sink` is a device buffer of at least 256
 * bytes that the kernel may write to (in practice it never does: a store happens only
 * when the XOR of the words one lane read equals one fixed 32-bit constant). buf 16-byte
 * aligned, bytes a multiple of 16 (0 enqueues nothing). Errors: INVALID_ARGUMENT, HIP.
 * =================================================================================== */
kvq_status kvq_probe_read(const void* buf, size_t bytes, void* sink, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
