// C ABI of libkvq: host-side validation, sign generation, sizing and dispatch.
// Nothing here touches the device before every argument has been checked.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "kvq_internal.h"

using namespace kvq;

namespace {

constexpr double kTwoPi = 6.283185307179586476925286766559;

// SplitMix64 output function (Steele, Lea, Flood, OOPSLA 2014): add the golden
// gamma, then two xor-shift-multiply rounds, all modulo 2^64.
uint64_t splitmix64_mix(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

bool is_pow2(uint32_t v) { return v && !(v & (v - 1)); }

SignMask sign_mask(uint64_t seed, uint32_t layer, uint32_t d) {
  SignMask m;
  memset(&m, 0, sizeof(m));
  const uint64_t base = splitmix64_mix(seed ^ (uint64_t)layer);
  for (uint32_t i = 0; i < d; ++i)
    if (splitmix64_mix(base + i) >> 63) m.w[i >> 6] |= 1ull << (i & 63);
  return m;
}

// Structural validity of a descriptor (independent of what kernels exist).
bool desc_ok(const kvq_layer_desc* d) {
  if (!d) return false;
  if (d->reserved != 0) return false;
  if (d->head_dim < 64 || d->head_dim > 256 || !is_pow2(d->head_dim)) return false;
  // token positions and tile counts are kept in int
  if (d->num_kv_heads == 0 || d->batch == 0 || d->capacity == 0 || d->capacity > kMaxCapacity)
    return false;
  if (d->n_bins_k < 2 || d->n_bins_k > 256 || d->n_bins_v < 2 || d->n_bins_v > 256)
    return false;
  return true;
}

bool head_dim_supported(uint32_t d) { return d == 64 || d == 128; }

int tiles_per_seq(const kvq_layer_desc* d) {
  return (int)((d->capacity + kTile - 1) / kTile);
}

TileGeom geom_of(const kvq_layer_desc* d) {
  return tile_geom((int)d->head_dim, code_bits(d->n_bins_k), code_bits(d->n_bins_v));
}

CodecArgs codec_args(const kvq_layer_desc* d, uint32_t t0, uint32_t ntok) {
  CodecArgs a;
  a.batch = (int)d->batch;
  a.hkv = (int)d->num_kv_heads;
  a.tiles_per_seq = tiles_per_seq(d);
  a.t0 = (int)t0;
  a.ntok = (int)ntok;
  a.tile_lo = (int)(t0 / kTile);
  a.tiles_touched = (int)((t0 + ntok + kTile - 1) / kTile) - a.tile_lo;
  a.n_k = (int)d->n_bins_k;
  a.n_v = (int)d->n_bins_v;
  a.bk = code_bits(d->n_bins_k);
  a.bv = code_bits(d->n_bins_v);
  a.inv_sqrt_d = 1.0 / sqrt((double)d->head_dim);
  a.k_bins_per_rad = (double)d->n_bins_k / kTwoPi;
  a.v_bins_per_rad = (double)d->n_bins_v / kTwoPi;
  a.sign = sign_mask(d->seed, d->layer, d->head_dim);
  a.positions = nullptr;
  a.capacity = (int)d->capacity;
  a.pg = Paging{nullptr, 0, 0};
  return a;
}

// Code widths the decode-attention kernels read: 6 to 8 bits. Narrower codebooks
// (n <= 32) are attended through a copy of the attended tiles re-packed at 6 bits
// (launch_widen), placed in the workspace after the split partials.
constexpr int kAttnMinBits = 6;
int attn_bits(uint32_t n) {
  const int b = code_bits(n);
  return b < kAttnMinBits ? kAttnMinBits : b;
}
bool attn_widens(const kvq_layer_desc* d) {
  return code_bits(d->n_bins_k) < kAttnMinBits || code_bits(d->n_bins_v) < kAttnMinBits;
}

// Decode-attention variant for this shape (see attn_mode in kvq_internal.h). Builds
// with KVQ_ATTN_ALL_MODES compiled in every variant and read KVQ_ATTN_MODE (0-3, 5-7)
// to force one, for comparisons.
int key_table_mode(const kvq_layer_desc* d, uint32_t hq) {
  const int g = (int)(hq / d->num_kv_heads);
  const int bk = attn_bits(d->n_bins_k), bv = attn_bits(d->n_bins_v);
#ifdef KVQ_ATTN_ALL_MODES
  if (const char* e = getenv("KVQ_ATTN_MODE")) {
    const int m = atoi(e);
    const bool half_ok = d->n_bins_k == (1u << bk);
    if (m >= 0 && m <= 7 && m != 4 && ((m & 3) != 2 || half_ok) &&
        attn_lds_bytes((int)d->head_dim, g, bk, bv, m) <= kLdsBytesMax)
      return m;
  }
#endif
  return attn_mode((int)d->head_dim, g, (int)d->n_bins_k, bk, bv);
}

// Sequence split for decode attention. Each wave of a workgroup streams whole tiles; aim
// for one workgroup per compute unit when the key table fills the LDS (256 workgroups),
// two otherwise, with at least 4 tiles per split and no empty split. Short sequences
// gain from more splits even with idle waves: a wave's tile is a chain of dependent
// loads, so running tiles side by side beats fewer, longer splits (a 4096-token layer
// at 4 kv heads: 8 tiles per split 20.0 us, 4 per split 17.8 us, 1 per split 22.4 us).
void split_plan(uint32_t units, uint32_t seq_len, bool key_table, int* nsplit,
                int* tiles_per_split) {
  const int ntiles = (int)((seq_len + kTile - 1) / kTile);
  const int target_wgs = key_table ? 256 : 512;
  int s = (int)((target_wgs + units - 1) / units);
  int max_s = (ntiles + 3) / 4;
  if (max_s < 1) max_s = 1;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  int tps = (ntiles + s - 1) / s;
  *tiles_per_split = tps;
  *nsplit = (ntiles + tps - 1) / tps;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct AttnLayout {
  size_t tickets, qrot, ml, acc, wide, lens, total;
};

// Workspace: split tickets (must read zero before a call; every call leaves them zero),
// the rotated queries, the per-split partial results, then (narrow codebooks only) the
// widened copy of the attended tiles and the fused decode step's per-sequence lengths.
AttnLayout attn_layout(const kvq_layer_desc* d, uint32_t hq, int nsplit, uint32_t seq_len) {
  AttnLayout l;
  const size_t units = (size_t)d->batch * d->num_kv_heads;
  const size_t bh = (size_t)d->batch * hq;
  l.tickets = 0;
  l.qrot = align256(units * sizeof(unsigned));
  l.ml = align256(l.qrot + bh * d->head_dim * sizeof(float));
  l.acc = align256(l.ml + bh * (size_t)nsplit * 2 * sizeof(float));
  l.total = align256(l.acc + bh * (size_t)nsplit * d->head_dim * sizeof(float));
  l.wide = l.lens = l.total;
  if (attn_widens(d)) {
    const size_t ntiles = (seq_len + kTile - 1) / kTile;
    const TileGeom gw = tile_geom((int)d->head_dim, attn_bits(d->n_bins_k), attn_bits(d->n_bins_v));
    l.lens = align256(l.wide + units * ntiles * (size_t)gw.bytes);
    l.total = align256(l.lens + (size_t)d->batch * sizeof(unsigned));
  }
  return l;
}

kvq_status attn_check(const kvq_layer_desc* d, uint32_t hq, uint32_t seq_len) {
  if (!desc_ok(d)) return KVQ_ERR_INVALID_ARGUMENT;
  if (hq == 0 || hq % d->num_kv_heads) return KVQ_ERR_INVALID_ARGUMENT;
  if (seq_len == 0) return KVQ_ERR_INVALID_ARGUMENT;
  if (seq_len > d->capacity) return KVQ_ERR_CAPACITY;
  const uint32_t g = hq / d->num_kv_heads;
  if (!head_dim_supported(d->head_dim)) return KVQ_ERR_UNSUPPORTED;
  if (g != 1 && g != 2 && g != 4 && g != 8) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

kvq_status attn_args(const kvq_layer_desc* d, uint32_t hq, uint32_t seq_len, float scale,
                     void* workspace, size_t workspace_bytes, AttnArgs* a,
                     uint8_t** wide = nullptr) {
  kvq_status st = attn_check(d, hq, seq_len);
  if (st != KVQ_OK) return st;
  int nsplit, tps;
  const int ktm = key_table_mode(d, hq);
  split_plan(d->batch * d->num_kv_heads, seq_len, ktm != 0, &nsplit, &tps);
  const AttnLayout l = attn_layout(d, hq, nsplit, seq_len);
  if (!workspace || ((uintptr_t)workspace & 255) || workspace_bytes < l.total)
    return KVQ_ERR_WORKSPACE;
  if (wide) *wide = (uint8_t*)workspace + l.wide;
  a->batch = (int)d->batch;
  a->hkv = (int)d->num_kv_heads;
  a->hq = (int)hq;
  a->group = (int)(hq / d->num_kv_heads);
  a->seq_len = (int)seq_len;
  a->tiles_per_seq = tiles_per_seq(d);
  a->ntiles = (int)((seq_len + kTile - 1) / kTile);
  a->nsplit = nsplit;
  a->tiles_per_split = tps;
  a->n_k = (int)d->n_bins_k;
  a->n_v = (int)d->n_bins_v;
  a->bk = attn_bits(d->n_bins_k);
  a->bv = attn_bits(d->n_bins_v);
  a->key_table = ktm;
  const double sc = scale > 0.0f ? (double)scale : 1.0 / sqrt((double)d->head_dim);
  a->q_scale = (float)(sc * 1.4426950408889634 / 255.0);
  a->inv_sqrt_d = (float)(1.0 / sqrt((double)d->head_dim));
  a->sign = sign_mask(d->seed, d->layer, d->head_dim);
  char* base = (char*)workspace;
  a->tickets = (unsigned*)(base + l.tickets);
  a->qrot = (float*)(base + l.qrot);
  a->part_ml = (float*)(base + l.ml);
  a->part_acc = (float*)(base + l.acc);
  a->seq_lens = nullptr;
  a->nq = 1;
  a->q0 = 0;
  a->nqc = 1;
  a->pg = Paging{nullptr, 0, 0};
  return KVQ_OK;
}

kvq_status hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

const AppendArgs kNoAppend = {nullptr, nullptr, nullptr, 0, 0, 0, 0, 0.0, 0.0, 0.0};

// Cache, query and output pointers and types of a decode-attention call.
kvq_status attn_io_check(const void* cache, const void* q, kvq_dtype q_dtype, const void* out,
                         kvq_dtype out_dtype) {
  if (!cache || !q || !out || ((uintptr_t)cache % 16)) return KVQ_ERR_INVALID_ARGUMENT;
  if ((q_dtype != KVQ_F16 && q_dtype != KVQ_F32) || (out_dtype != KVQ_F16 && out_dtype != KVQ_F32))
    return KVQ_ERR_INVALID_ARGUMENT;
  if ((uintptr_t)q % (q_dtype == KVQ_F32 ? 8 : 4)) return KVQ_ERR_INVALID_ARGUMENT;
  if ((uintptr_t)out % (out_dtype == KVQ_F32 ? 8 : 4)) return KVQ_ERR_INVALID_ARGUMENT;
  return KVQ_OK;
}

kvq_status attn_run(const kvq_layer_desc* d, const void* cache, const Paging& pg, const void* q,
                    kvq_dtype q_dtype, uint32_t hq, uint32_t seq_len, const uint32_t* seq_lens,
                    float scale, void* out, kvq_dtype out_dtype, void* ws, size_t ws_bytes,
                    void* stream, const AppendArgs& app = kNoAppend) {
  AttnArgs a;
  uint8_t* wide = nullptr;
  kvq_status st = attn_args(d, hq, seq_len, scale, ws, ws_bytes, &a, &wide);
  if (st != KVQ_OK) return st;
  st = attn_io_check(cache, q, q_dtype, out, out_dtype);
  if (st != KVQ_OK) return st;
  if (attn_widens(d)) {
    // a paged pool or a fused append would need the copy to follow the page table or
    // take the new token: not served for narrow codebooks
    if (pg.table || app.positions) return KVQ_ERR_UNSUPPORTED;
    const hipError_t e = launch_widen((const uint8_t*)cache, a.tiles_per_seq, wide,
                                      (int)d->head_dim, code_bits(d->n_bins_k),
                                      code_bits(d->n_bins_v), a.batch * a.hkv, a.ntiles,
                                      (hipStream_t)stream);
    if (e != hipSuccess) return KVQ_ERR_HIP;
    a.tiles_per_seq = a.ntiles;
    cache = wide;
  }
  a.q = q;
  a.q_f32 = q_dtype == KVQ_F32;
  a.out = out;
  a.out_f32 = out_dtype == KVQ_F32;
  a.seq_lens = seq_lens;
  a.pg = pg;
  return hip_status(
      launch_attn_decode(a, app, (int)d->head_dim, (const uint8_t*)cache, (hipStream_t)stream));
}

// Multi-query attention: rows = nq * G query rows per kv head, padded to 16 or 32.
constexpr uint32_t kMultiMaxRows = 32;
int multi_rows(uint32_t rows) { return rows <= 16 ? 16 : 32; }

kvq_status multi_check(const kvq_layer_desc* d, uint32_t hq, uint32_t nq, uint32_t seq_len) {
  if (!desc_ok(d)) return KVQ_ERR_INVALID_ARGUMENT;
  if (hq == 0 || hq % d->num_kv_heads || nq == 0 || seq_len == 0 || nq > seq_len)
    return KVQ_ERR_INVALID_ARGUMENT;
  if (seq_len > d->capacity) return KVQ_ERR_CAPACITY;
  const uint32_t g = hq / d->num_kv_heads;
  if (!head_dim_supported(d->head_dim)) return KVQ_ERR_UNSUPPORTED;
  if (g != 1 && g != 2 && g != 4 && g != 8) return KVQ_ERR_UNSUPPORTED;
  if ((uint64_t)nq * g > kMultiMaxRows) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

// Sequence split for multi-query attention: one workgroup per compute unit fits its
// LDS, so aim for 256 workgroups, with at least four tiles per split and no empty split.
void multi_split_plan(uint32_t units, uint32_t seq_len, int* nsplit, int* tiles_per_split) {
  const int ntiles = (int)((seq_len + kTile - 1) / kTile);
  int s = (int)((256 + units - 1) / units);
  int max_s = (ntiles + 3) / 4;
  if (max_s < 1) max_s = 1;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  const int tps = (ntiles + s - 1) / s;
  *tiles_per_split = tps;
  *nsplit = (ntiles + tps - 1) / tps;
}

struct MultiLayout {
  size_t tickets, ml, acc, wide, total;
};
// Split counters, partials, then (narrow codebooks) the widened tile copy, as for
// decode attention.
MultiLayout multi_layout(const kvq_layer_desc* d, uint32_t rows, int nsplit, uint32_t seq_len) {
  MultiLayout l;
  const size_t units = (size_t)d->batch * d->num_kv_heads;
  const size_t m = (size_t)multi_rows(rows);
  l.tickets = 0;
  l.ml = align256(units * sizeof(unsigned));
  l.acc = align256(l.ml + units * nsplit * m * 2 * sizeof(float));
  l.total = align256(l.acc + units * nsplit * m * d->head_dim * sizeof(float));
  l.wide = l.total;
  if (attn_widens(d)) {
    const size_t ntiles = (seq_len + kTile - 1) / kTile;
    const TileGeom gw = tile_geom((int)d->head_dim, attn_bits(d->n_bins_k), attn_bits(d->n_bins_v));
    l.total = align256(l.wide + units * ntiles * (size_t)gw.bytes);
  }
  return l;
}

const Paging kNoPaging = {nullptr, 0, 0};

kvq_status paging_args(const kvq_layer_desc* d, const kvq_paging* p, Paging* out) {
  if (!desc_ok(d) || !p || !p->page_table || ((uintptr_t)p->page_table % 4))
    return KVQ_ERR_INVALID_ARGUMENT;
  if (p->num_pages == 0 || p->num_pages > 0x7fffffffu) return KVQ_ERR_INVALID_ARGUMENT;
  if (p->pages_per_seq < (uint32_t)tiles_per_seq(d)) return KVQ_ERR_INVALID_ARGUMENT;
  out->table = p->page_table;
  out->pages_per_seq = (int)p->pages_per_seq;
  out->num_pages = (int)p->num_pages;
  return KVQ_OK;
}

kvq_status encode_impl(const kvq_layer_desc* d, void* cache, const Paging& pg, const void* k, const void* v,
                      kvq_dtype in_dtype, int64_t sb, int64_t st, int64_t sh, uint32_t t0,
                      uint32_t ntok, void* stream) {
  if (!desc_ok(d)) return KVQ_ERR_INVALID_ARGUMENT;
  if (in_dtype != KVQ_F16 && in_dtype != KVQ_F32) return KVQ_ERR_INVALID_ARGUMENT;
  if ((uint64_t)t0 + ntok > d->capacity) return KVQ_ERR_CAPACITY;
  if (!head_dim_supported(d->head_dim)) return KVQ_ERR_UNSUPPORTED;
  if (ntok == 0) return KVQ_OK;
  if (!cache || !k || !v || ((uintptr_t)cache % 16)) return KVQ_ERR_INVALID_ARGUMENT;
  const size_t esz = in_dtype == KVQ_F32 ? 4 : 2;
  if (((uintptr_t)k % (2 * esz)) || ((uintptr_t)v % (2 * esz))) return KVQ_ERR_INVALID_ARGUMENT;
  if ((sb & 1) || (st & 1) || (sh & 1) || sb < 0 || st < 0 || sh < 0)
    return KVQ_ERR_INVALID_ARGUMENT;
  CodecArgs a = codec_args(d, t0, ntok);
  a.pg = pg;
  return hip_status(launch_encode(a, (int)d->head_dim, geom_of(d), (uint8_t*)cache, k, v,
                                  in_dtype == KVQ_F32, sb, st, sh, (hipStream_t)stream));
}

kvq_status append_impl(const kvq_layer_desc* d, void* cache, const Paging& pg, const void* k, const void* v,
                      kvq_dtype in_dtype, int64_t sb, int64_t sh, const uint32_t* positions,
                      void* stream) {
  if (!desc_ok(d)) return KVQ_ERR_INVALID_ARGUMENT;
  if (in_dtype != KVQ_F16 && in_dtype != KVQ_F32) return KVQ_ERR_INVALID_ARGUMENT;
  if (!head_dim_supported(d->head_dim)) return KVQ_ERR_UNSUPPORTED;
  if (!cache || !k || !v || !positions || ((uintptr_t)cache % 16) || ((uintptr_t)positions % 4))
    return KVQ_ERR_INVALID_ARGUMENT;
  const size_t esz = in_dtype == KVQ_F32 ? 4 : 2;
  if (((uintptr_t)k % (2 * esz)) || ((uintptr_t)v % (2 * esz))) return KVQ_ERR_INVALID_ARGUMENT;
  if ((sb & 1) || (sh & 1) || sb < 0 || sh < 0) return KVQ_ERR_INVALID_ARGUMENT;
  CodecArgs a = codec_args(d, 0, 1);
  a.positions = positions;
  a.pg = pg;
  return hip_status(launch_append(a, (int)d->head_dim, geom_of(d), (uint8_t*)cache, k, v,
                                  in_dtype == KVQ_F32, sb, sh, (hipStream_t)stream));
}

kvq_status decode_impl(const kvq_layer_desc* d, const void* cache, const Paging& pg, void* k_out, void* v_out,
                      kvq_dtype out_dtype, uint32_t t0, uint32_t ntok, void* stream) {
  if (!desc_ok(d)) return KVQ_ERR_INVALID_ARGUMENT;
  if (out_dtype != KVQ_F16 && out_dtype != KVQ_F32) return KVQ_ERR_INVALID_ARGUMENT;
  if ((uint64_t)t0 + ntok > d->capacity) return KVQ_ERR_CAPACITY;
  if (!head_dim_supported(d->head_dim)) return KVQ_ERR_UNSUPPORTED;
  if (ntok == 0) return KVQ_OK;
  if (!cache || !k_out || !v_out || ((uintptr_t)cache % 16)) return KVQ_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)k_out % 16) || ((uintptr_t)v_out % 16)) return KVQ_ERR_INVALID_ARGUMENT;
  CodecArgs a = codec_args(d, t0, ntok);
  a.pg = pg;
  return hip_status(launch_decode(a, (int)d->head_dim, geom_of(d), (const uint8_t*)cache,
                                  k_out, v_out, out_dtype == KVQ_F32, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int kvq_abi_version(void) { return KVQ_ABI_VERSION; }

const char* kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID_ARGUMENT: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVQ_ERR_CAPACITY: return "token range exceeds cache capacity";
    case KVQ_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case KVQ_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

size_t kvq_tile_bytes(uint32_t head_dim, uint32_t n_bins_k, uint32_t n_bins_v) {
  if (head_dim < 64 || head_dim > 256 || !is_pow2(head_dim)) return 0;
  if (n_bins_k < 2 || n_bins_k > 256 || n_bins_v < 2 || n_bins_v > 256) return 0;
  return (size_t)tile_geom((int)head_dim, code_bits(n_bins_k), code_bits(n_bins_v)).bytes;
}

size_t kvq_cache_bytes(const kvq_layer_desc* d) {
  if (!desc_ok(d)) return 0;
  return (size_t)d->batch * d->num_kv_heads * (size_t)tiles_per_seq(d) *
         kvq_tile_bytes(d->head_dim, d->n_bins_k, d->n_bins_v);
}

kvq_status kvq_layer_signs(uint64_t seed, uint32_t layer, uint32_t d, int8_t* out_host) {
  if (!out_host || !is_pow2(d) || d > 4096) return KVQ_ERR_INVALID_ARGUMENT;
  const uint64_t base = splitmix64_mix(seed ^ (uint64_t)layer);
  for (uint32_t i = 0; i < d; ++i) out_host[i] = (splitmix64_mix(base + i) >> 63) ? -1 : 1;
  return KVQ_OK;
}

kvq_status kvq_encode(const kvq_layer_desc* d, void* cache, const void* k, const void* v,
                      kvq_dtype in_dtype, int64_t sb, int64_t st, int64_t sh, uint32_t t0,
                      uint32_t ntok, void* stream) {
  return encode_impl(d, cache, kNoPaging, k, v, in_dtype, sb, st, sh, t0, ntok, stream);
}

kvq_status kvq_append(const kvq_layer_desc* d, void* cache, const void* k, const void* v,
                      kvq_dtype in_dtype, int64_t sb, int64_t sh, const uint32_t* positions,
                      void* stream) {
  return append_impl(d, cache, kNoPaging, k, v, in_dtype, sb, sh, positions, stream);
}

kvq_status kvq_decode(const kvq_layer_desc* d, const void* cache, void* k_out, void* v_out,
                      kvq_dtype out_dtype, uint32_t t0, uint32_t ntok, void* stream) {
  return decode_impl(d, cache, kNoPaging, k_out, v_out, out_dtype, t0, ntok, stream);
}

size_t kvq_paged_pool_bytes(const kvq_layer_desc* d, uint32_t num_pages) {
  if (!desc_ok(d)) return 0;
  return (size_t)num_pages * d->num_kv_heads * kvq_tile_bytes(d->head_dim, d->n_bins_k, d->n_bins_v);
}

kvq_status kvq_encode_paged(const kvq_layer_desc* d, void* pool, const kvq_paging* paging,
                            const void* k, const void* v, kvq_dtype in_dtype, int64_t sb,
                            int64_t st, int64_t sh, uint32_t t0, uint32_t ntok, void* stream) {
  Paging pg;
  const kvq_status st0 = paging_args(d, paging, &pg);
  if (st0 != KVQ_OK) return st0;
  return encode_impl(d, pool, pg, k, v, in_dtype, sb, st, sh, t0, ntok, stream);
}

kvq_status kvq_append_paged(const kvq_layer_desc* d, void* pool, const kvq_paging* paging,
                            const void* k, const void* v, kvq_dtype in_dtype, int64_t sb,
                            int64_t sh, const uint32_t* positions, void* stream) {
  Paging pg;
  const kvq_status st0 = paging_args(d, paging, &pg);
  if (st0 != KVQ_OK) return st0;
  return append_impl(d, pool, pg, k, v, in_dtype, sb, sh, positions, stream);
}

kvq_status kvq_decode_paged(const kvq_layer_desc* d, const void* pool, const kvq_paging* paging,
                            void* k_out, void* v_out, kvq_dtype out_dtype, uint32_t t0,
                            uint32_t ntok, void* stream) {
  Paging pg;
  const kvq_status st0 = paging_args(d, paging, &pg);
  if (st0 != KVQ_OK) return st0;
  return decode_impl(d, pool, pg, k_out, v_out, out_dtype, t0, ntok, stream);
}

uint32_t kvq_attn_num_splits(const kvq_layer_desc* d, uint32_t hq, uint32_t seq_len) {
  if (attn_check(d, hq, seq_len) != KVQ_OK) return 0;  // invalid or not served
  int nsplit, tps;
  split_plan(d->batch * d->num_kv_heads, seq_len, key_table_mode(d, hq) != 0, &nsplit, &tps);
  return (uint32_t)nsplit;
}

size_t kvq_attn_workspace_bytes(const kvq_layer_desc* d, uint32_t hq, uint32_t seq_len) {
  const uint32_t s = kvq_attn_num_splits(d, hq, seq_len);
  if (!s) return 0;
  return attn_layout(d, hq, (int)s, seq_len).total;
}

kvq_status kvq_attn_decode(const kvq_layer_desc* d, const void* cache, const void* q,
                           kvq_dtype q_dtype, uint32_t hq, uint32_t seq_len, float scale,
                           void* out, kvq_dtype out_dtype, void* ws, size_t ws_bytes,
                           void* stream) {
  return attn_run(d, cache, kNoPaging, q, q_dtype, hq, seq_len, nullptr, scale, out, out_dtype,
                  ws, ws_bytes, stream);
}

kvq_status kvq_attn_decode_varlen(const kvq_layer_desc* d, const void* cache, const void* q,
                                  kvq_dtype q_dtype, uint32_t hq, const uint32_t* seq_lens,
                                  uint32_t max_seq_len, float scale, void* out,
                                  kvq_dtype out_dtype, void* ws, size_t ws_bytes,
                                  void* stream) {
  if (!seq_lens || ((uintptr_t)seq_lens % 4)) {
    // shape errors take precedence, as in kvq_attn_decode
    const kvq_status st = attn_check(d, hq, max_seq_len);
    return st != KVQ_OK ? st : KVQ_ERR_INVALID_ARGUMENT;
  }
  return attn_run(d, cache, kNoPaging, q, q_dtype, hq, max_seq_len, seq_lens, scale, out,
                  out_dtype, ws, ws_bytes, stream);
}

kvq_status kvq_attn_decode_paged(const kvq_layer_desc* d, const void* pool,
                                 const kvq_paging* paging, const void* q, kvq_dtype q_dtype,
                                 uint32_t hq, const uint32_t* seq_lens, uint32_t max_seq_len,
                                 float scale, void* out, kvq_dtype out_dtype, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (seq_lens && ((uintptr_t)seq_lens % 4)) return KVQ_ERR_INVALID_ARGUMENT;
  Paging pg;
  const kvq_status st0 = paging_args(d, paging, &pg);
  if (st0 != KVQ_OK) return st0;
  return attn_run(d, pool, pg, q, q_dtype, hq, max_seq_len, seq_lens, scale, out, out_dtype,
                  ws, ws_bytes, stream);
}

kvq_status kvq_attn_decode_append(const kvq_layer_desc* d, void* cache,
                                  const kvq_paging* paging, const void* k, const void* v,
                                  kvq_dtype in_dtype, int64_t sb, int64_t sh,
                                  const uint32_t* positions, const void* q, kvq_dtype q_dtype,
                                  uint32_t hq, uint32_t max_seq_len, float scale, void* out,
                                  kvq_dtype out_dtype, void* ws, size_t ws_bytes,
                                  void* stream) {
  // shape errors first, as in kvq_attn_decode
  const kvq_status st = attn_check(d, hq, max_seq_len);
  if (st != KVQ_OK) return st;
  if (in_dtype != KVQ_F16 && in_dtype != KVQ_F32) return KVQ_ERR_INVALID_ARGUMENT;
  if (!k || !v || !positions || ((uintptr_t)positions % 4)) return KVQ_ERR_INVALID_ARGUMENT;
  const size_t esz = in_dtype == KVQ_F32 ? 4 : 2;
  if (((uintptr_t)k % (2 * esz)) || ((uintptr_t)v % (2 * esz))) return KVQ_ERR_INVALID_ARGUMENT;
  if ((sb & 1) || (sh & 1) || sb < 0 || sh < 0) return KVQ_ERR_INVALID_ARGUMENT;
  Paging pg = kNoPaging;
  if (paging) {
    const kvq_status sp = paging_args(d, paging, &pg);
    if (sp != KVQ_OK) return sp;
  }
  if (attn_widens(d)) {
    // narrow codebooks: kvq_append, the lengths positions + 1, then the ragged attention
    // over the widened copy (every argument checked before the cache is written)
    if (pg.table) return KVQ_ERR_UNSUPPORTED;
    AttnArgs chk;
    kvq_status s2 = attn_args(d, hq, max_seq_len, scale, ws, ws_bytes, &chk);
    if (s2 == KVQ_OK) s2 = attn_io_check(cache, q, q_dtype, out, out_dtype);
    if (s2 == KVQ_OK && !cache) s2 = KVQ_ERR_INVALID_ARGUMENT;
    if (s2 != KVQ_OK) return s2;
    s2 = append_impl(d, cache, kNoPaging, k, v, in_dtype, sb, sh, positions, stream);
    if (s2 != KVQ_OK) return s2;
    unsigned* lens = (unsigned*)((char*)ws + attn_layout(d, hq, chk.nsplit, max_seq_len).lens);
    if (launch_lengths(positions, lens, (int)d->batch, max_seq_len, (hipStream_t)stream) !=
        hipSuccess)
      return KVQ_ERR_HIP;
    return attn_run(d, cache, kNoPaging, q, q_dtype, hq, max_seq_len, lens, scale, out,
                    out_dtype, ws, ws_bytes, stream);
  }
  const CodecArgs c = codec_args(d, 0, 1);
  AppendArgs app;
  app.positions = positions;
  app.k = k;
  app.v = v;
  app.sb = sb;
  app.sh = sh;
  app.f32 = in_dtype == KVQ_F32;
  app.capacity = (int)d->capacity;
  app.inv_sqrt_d = c.inv_sqrt_d;
  app.k_bins_per_rad = c.k_bins_per_rad;
  app.v_bins_per_rad = c.v_bins_per_rad;
  return attn_run(d, cache, pg, q, q_dtype, hq, max_seq_len, nullptr, scale, out, out_dtype,
                  ws, ws_bytes, stream, app);
}

size_t kvq_attn_multi_workspace_bytes(const kvq_layer_desc* d, uint32_t hq, uint32_t nq,
                                      uint32_t seq_len) {
  if (multi_check(d, hq, nq, seq_len) != KVQ_OK) return 0;
  int nsplit, tps;
  multi_split_plan(d->batch * d->num_kv_heads, seq_len, &nsplit, &tps);
  return multi_layout(d, nq * (hq / d->num_kv_heads), nsplit, seq_len).total;
}

}  // extern "C"

namespace {

kvq_status multi_run(const kvq_layer_desc* d, const void* cache, const Paging& pg,
                     const void* q, kvq_dtype q_dtype, uint32_t hq, uint32_t nq,
                     const uint32_t* seq_lens, uint32_t seq_len, float scale, void* out,
                     kvq_dtype out_dtype, void* ws, size_t ws_bytes, void* stream) {
  kvq_status st = multi_check(d, hq, nq, seq_len);
  if (st != KVQ_OK) return st;
  int nsplit, tps;
  multi_split_plan(d->batch * d->num_kv_heads, seq_len, &nsplit, &tps);
  const uint32_t g = hq / d->num_kv_heads;
  const MultiLayout l = multi_layout(d, nq * g, nsplit, seq_len);
  if (!ws || ((uintptr_t)ws & 255) || ws_bytes < l.total) return KVQ_ERR_WORKSPACE;
  if (!cache || !q || !out || ((uintptr_t)cache % 16)) return KVQ_ERR_INVALID_ARGUMENT;
  if ((q_dtype != KVQ_F16 && q_dtype != KVQ_F32) || (out_dtype != KVQ_F16 && out_dtype != KVQ_F32))
    return KVQ_ERR_INVALID_ARGUMENT;
  if ((uintptr_t)q % (q_dtype == KVQ_F32 ? 8 : 4)) return KVQ_ERR_INVALID_ARGUMENT;
  if ((uintptr_t)out % (out_dtype == KVQ_F32 ? 8 : 4)) return KVQ_ERR_INVALID_ARGUMENT;
  AttnArgs a = {};
  a.batch = (int)d->batch;
  a.hkv = (int)d->num_kv_heads;
  a.hq = (int)hq;
  a.group = (int)g;
  a.nq = (int)nq;
  a.seq_len = (int)seq_len;
  a.tiles_per_seq = tiles_per_seq(d);
  a.ntiles = (int)((seq_len + kTile - 1) / kTile);
  a.nsplit = nsplit;
  a.tiles_per_split = tps;
  a.n_k = (int)d->n_bins_k;
  a.n_v = (int)d->n_bins_v;
  a.bk = attn_bits(d->n_bins_k);
  a.bv = attn_bits(d->n_bins_v);
  const double sc = scale > 0.0f ? (double)scale : 1.0 / sqrt((double)d->head_dim);
  a.q_scale = (float)(sc * 1.4426950408889634);  // the key radius carries s / 255 here
  a.inv_sqrt_d = (float)(1.0 / sqrt((double)d->head_dim));
  a.sign = sign_mask(d->seed, d->layer, d->head_dim);
  a.q = q;
  a.q_f32 = q_dtype == KVQ_F32;
  a.out = out;
  a.out_f32 = out_dtype == KVQ_F32;
  char* base = (char*)ws;
  a.tickets = (unsigned*)(base + l.tickets);
  a.part_ml = (float*)(base + l.ml);
  a.part_acc = (float*)(base + l.acc);
  a.seq_lens = seq_lens;
  a.pg = pg;
  if (attn_widens(d)) {
    if (pg.table) return KVQ_ERR_UNSUPPORTED;  // no widened copy of a pool
    const hipError_t e = launch_widen((const uint8_t*)cache, a.tiles_per_seq, (uint8_t*)ws + l.wide,
                                      (int)d->head_dim, code_bits(d->n_bins_k),
                                      code_bits(d->n_bins_v), a.batch * a.hkv, a.ntiles,
                                      (hipStream_t)stream);
    if (e != hipSuccess) return KVQ_ERR_HIP;
    a.tiles_per_seq = a.ntiles;
    cache = (const uint8_t*)ws + l.wide;
  }
  // one launch for up to 32 query rows: the 16-row kernel, or the 32-row one, which
  // reads the cache once for all of them
  const uint32_t per = 32 / g;
  for (uint32_t q0 = 0; q0 < nq; q0 += per) {
    a.q0 = (int)q0;
    a.nqc = (int)(nq - q0 < per ? nq - q0 : per);
    const hipError_t e = launch_attn_multi(a, (int)d->head_dim, a.nqc * (int)g,
                                           (const uint8_t*)cache, (hipStream_t)stream);
    if (e != hipSuccess) return KVQ_ERR_HIP;
  }
  return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_attn_multi(const kvq_layer_desc* d, const void* cache, const void* q,
                          kvq_dtype q_dtype, uint32_t hq, uint32_t nq, uint32_t seq_len,
                          float scale, void* out, kvq_dtype out_dtype, void* ws,
                          size_t ws_bytes, void* stream) {
  return multi_run(d, cache, kNoPaging, q, q_dtype, hq, nq, nullptr, seq_len, scale, out,
                   out_dtype, ws, ws_bytes, stream);
}

kvq_status kvq_attn_multi_varlen(const kvq_layer_desc* d, const void* cache, const void* q,
                                 kvq_dtype q_dtype, uint32_t hq, uint32_t nq,
                                 const uint32_t* seq_lens, uint32_t max_seq_len, float scale,
                                 void* out, kvq_dtype out_dtype, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (!seq_lens || ((uintptr_t)seq_lens % 4)) {
    const kvq_status st = multi_check(d, hq, nq, max_seq_len);  // shape errors first
    return st != KVQ_OK ? st : KVQ_ERR_INVALID_ARGUMENT;
  }
  return multi_run(d, cache, kNoPaging, q, q_dtype, hq, nq, seq_lens, max_seq_len, scale, out,
                   out_dtype, ws, ws_bytes, stream);
}

kvq_status kvq_attn_multi_paged(const kvq_layer_desc* d, const void* pool,
                                const kvq_paging* paging, const void* q, kvq_dtype q_dtype,
                                uint32_t hq, uint32_t nq, const uint32_t* seq_lens,
                                uint32_t max_seq_len, float scale, void* out,
                                kvq_dtype out_dtype, void* ws, size_t ws_bytes, void* stream) {
  if (seq_lens && ((uintptr_t)seq_lens % 4)) return KVQ_ERR_INVALID_ARGUMENT;
  Paging pg;
  const kvq_status st0 = paging_args(d, paging, &pg);
  if (st0 != KVQ_OK) return st0;
  return multi_run(d, pool, pg, q, q_dtype, hq, nq, seq_lens, max_seq_len, scale, out,
                   out_dtype, ws, ws_bytes, stream);
}

}  // extern "C"

// ------------------------------------------------------------ allocation-free variant
//
// For callers that cannot allocate device memory (code under graph capture, tight
// serving loops, harnesses that forbid allocation): kvq_attn_decode with the workspace
// taken from a fixed-size device array of this library, one copy per GPU (each device
// holds its own copy at its own address, looked up once per device with
// hipGetSymbolAddress and kept). Every call on a GPU shares that GPU's array.

namespace {

constexpr size_t kStaticScratchBytes = (size_t)8 << 20;
constexpr int kScratchDevices = 64;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// Zero-fills the split counters at the start of the workspace (a kernel rather than a
// memset, so the call can also be recorded into a graph).
__global__ void zero_words_kernel(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Device address of the current device's scratch array (looked up on first use per
// device; relaxed atomics: threads that race on the first call store the same value).
hipError_t scratch_address(void** out) {
  static std::atomic<void*> addr[kScratchDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_relaxed);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_relaxed);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t kvq_attn_static_scratch_bytes(void) { return kStaticScratchBytes; }

kvq_status kvq_attn_decode_static(const kvq_layer_desc* d, const void* cache, const void* q,
                                  kvq_dtype q_dtype, uint32_t hq, uint32_t seq_len,
                                  float scale, void* out, kvq_dtype out_dtype, void* stream) {
  // every argument is checked before the first HIP call
  kvq_status st = attn_check(d, hq, seq_len);
  if (st != KVQ_OK) return st;
  st = attn_io_check(cache, q, q_dtype, out, out_dtype);
  if (st != KVQ_OK) return st;
  const size_t need = kvq_attn_workspace_bytes(d, hq, seq_len);
  if (need == 0) return KVQ_ERR_INVALID_ARGUMENT;
  if (need > kStaticScratchBytes) return KVQ_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return KVQ_ERR_HIP;
  // the split counters must read zero; the array keeps the last call's contents
  const int words = (int)(d->batch * d->num_kv_heads);
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, static_cast<unsigned*>(ws), words);
  if (hipGetLastError() != hipSuccess) return KVQ_ERR_HIP;
  return attn_run(d, cache, kNoPaging, q, q_dtype, hq, seq_len, nullptr, scale, out, out_dtype,
                  ws, need, stream);
}

}  // extern "C"
