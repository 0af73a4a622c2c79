// Private definitions shared by the libkvq HIP sources: tile geometry, the per-layer
// sign mask and the kernel launchers the C ABI dispatches to.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

constexpr int kTile = KVQ_TILE_TOKENS;  // token slots per tile
// Largest capacity a descriptor may state: slot and tile arithmetic is done in int.
constexpr uint32_t kMaxCapacity = 0x7FFFFFFFu - (kTile - 1);
constexpr int kMaxHeadDim = 128;

// Angle code width for n bins: ceil(log2 n).
inline int code_bits(uint32_t n) {
  int b = 0;
  while ((1u << b) < n) ++b;
  return b;
}

// Byte geometry of one tile (see the layout comment in kvq.h).
struct TileGeom {
  int d, pairs, bk, bv;
  int ka, kr, ks, va, vr, vp, bytes;  // plane byte offsets and total tile bytes
  int wka, wkr, wva, wvr;             // words per token (K planes) or per pair (V)
};

inline TileGeom tile_geom(int d, int bk, int bv) {
  TileGeom g;
  g.d = d;
  g.pairs = d / 2;
  g.bk = bk;
  g.bv = bv;
  g.wka = g.pairs * bk / 32;
  g.wkr = g.pairs / 4;
  g.wva = 2 * bv;
  g.wvr = 8;
  g.ka = 0;
  g.kr = g.ka + kTile * g.wka * 4;
  g.ks = g.kr + kTile * g.wkr * 4;
  g.va = g.ks + 2 * kTile;
  g.vr = g.va + g.pairs * g.wva * 4;
  g.vp = g.vr + g.pairs * g.wvr * 4;
  g.bytes = g.vp + 4 * kTile;
  return g;
}

// Sign diagonal as a bit mask: bit e set <=> sign[e] = -1. d <= 256.
struct SignMask {
  uint64_t w[4];
};

// Optional page table: tile t of sequence b of a paged cache lives in page
// table[b * pages_per_seq + t] of a pool laid out [page][kv head][tile bytes]. Without a
// table the cache is contiguous, [batch][kv head][tile][tile bytes].
struct Paging {
  const int* table;  // null: contiguous cache
  int pages_per_seq, num_pages;
};

// Byte offset of tile `tile` of (sequence b, kv head h), or -1 when the page table maps
// it to no page of the pool (an entry outside [0, num_pages)).
__host__ __device__ __attribute__((always_inline)) inline long long tile_offset(
    Paging pg, int b, int h, int hkv, int tiles_per_seq, int tile, int bytes) {
  if (!pg.table) return ((long long)(b * hkv + h) * tiles_per_seq + tile) * bytes;
  const int page = pg.table[(long long)b * pg.pages_per_seq + tile];
  if (page < 0 || page >= pg.num_pages) return -1;
  return ((long long)page * hkv + h) * bytes;
}

// Runtime parameters of one encode/decode launch.
struct CodecArgs {
  int batch, hkv, tiles_per_seq;
  int t0, ntok;               // token range
  int tile_lo, tiles_touched;  // first tile and count of tiles the range touches
  int n_k, n_v, bk, bv;
  double inv_sqrt_d;        // fp64 value of 1/sqrt(d)
  double k_bins_per_rad;    // n_k / (2 pi) in fp64
  double v_bins_per_rad;    // n_v / (2 pi) in fp64
  SignMask sign;
  const unsigned* positions;  // append: [B] slot of each sequence's new token
  int capacity;               // tokens per sequence
  Paging pg;
};

hipError_t launch_append(const CodecArgs& a, int d, TileGeom geom, uint8_t* cache,
                         const void* k, const void* v, bool f32_in, int64_t sb, int64_t sh,
                         hipStream_t stream);
hipError_t launch_encode(const CodecArgs& a, int d, TileGeom geom, uint8_t* cache,
                         const void* k, const void* v, bool f32_in, int64_t sb, int64_t st,
                         int64_t sh, hipStream_t stream);

hipError_t launch_decode(const CodecArgs& a, int d, TileGeom geom, const uint8_t* cache,
                         void* k_out, void* v_out, bool f32_out, hipStream_t stream);

// Decode attention.
struct AttnArgs {
  int batch, hkv, hq, group;
  int seq_len, tiles_per_seq, ntiles, nsplit, tiles_per_split;
  int n_k, n_v, bk, bv;
  int key_table;       // score table in LDS: 0 none, 1 full, 2 half (sign-symmetric)
  int q_f32, out_f32;  // element types of q and out (else fp16)
  float q_scale;       // softmax scale * log2(e) / 255, folded into the rotated query
  float inv_sqrt_d;    // fp32 1/sqrt(d)
  SignMask sign;
  const void* q;       // [B, Hq, d]
  void* out;           // [B, Hq, d]
  unsigned* tickets;   // [B * Hkv] split counters; zero between calls
  float* qrot;         // [B, Hq, d] rotated queries (kernels without the key table)
  float* part_ml;      // [B, Hq, nsplit, 2]
  float* part_acc;     // [B, Hq, nsplit, d]
  const unsigned* seq_lens;  // [B] per-entry lengths (device), or null: seq_len for all
  int nq;                    // query tokens per sequence (multi-query attention; else 1)
  int q0, nqc;               // multi-query: first query token and count of this launch
  Paging pg;
};

// Bytes of the per-workgroup key-score table (pairs x 2^bk codes x heads x fp32) and
// the largest table the decode kernel keeps in LDS.
constexpr int kKeyTableMaxBytes = 128 * 1024;
inline long key_table_bytes(int d, int group, int bk) { return (long)(d / 2) * (1L << bk) * group * 4; }

// Decode-attention kernel variants ("mode"): bits 0-1 choose how scores are formed
// (0: rotated query through scalar loads, 1: full LDS score table, 2: half score table
// for power-of-two n, 3: matrix-core products), bit 2 puts the value sum on the matrix
// cores. The LDS a variant needs mirrors the kernel's own layout (cos/sin tables, the
// rotated query, a flag word, then the score table and the waves' fp16 value rows, or
// the merge buffers after the tile loop; with a score table and matrix-core values the
// query moves into that union, beside the merge buffers).
constexpr int kLdsBytesMax = 160 * 1024;
// Waves per workgroup: 12 (three per SIMD) with the key table at up to four heads per
// kv head and for both products on the matrix cores at d = 128 (within 168 VGPRs; 4%
// faster than 8 on the 70B-shaped layers, while d = 64 would spill at 12), else 8.
constexpr int attn_waves(int mode, int group, int d) {
  return (mode & 3) == 3 ? (mode == 7 && d == 128 ? 12 : 8)
                         : ((mode & 3) != 0 && group <= 4 ? 12 : 8);
}
constexpr long attn_lds_bytes(int d, int group, int bk, int bv, int mode) {
  const int p = d / 2, nw = attn_waves(mode, group, d);
  const int hg = group > 4 ? group / 4 : 1;
  const long tab = (mode & 3) == 1 ? (long)p * (1 << bk) * group * 4
                   : (mode & 3) == 2 ? (long)p * (1 << (bk - 1)) * group * 4 : 0;
  const long rows = (mode & 4) ? (long)nw * (hg * 4 * 64 + 64 * 16) * 2 : 0;
  const long qb = (long)group * d * 4;
  const bool qu = tab > 0 && (mode & 4);  // the query lives in the union
  const long merge = (long)nw * group * (d + 2) * 4 + (qu ? qb : 0);
  const long loop = tab + rows;
  return (1L << bk) * 8 + (1L << bv) * 8 + (qu ? 0 : qb) + 16 + (loop > merge ? loop : merge);
}
// The variant run for a shape, as measured fastest on MI355X: for up to four heads per
// kv head, the score table with the value sum on the matrix cores when both fit in LDS.
// Power-of-two n admits the half table (mode 6: one more sign operation per pair, half
// the LDS): it is the faster one at four heads (51.4 against 52.5 us per
// Mistral-7B-shaped 7/6-bit layer), the full table (mode 5) at one and two (41.7
// against 42.5-42.9 us at two), and the full table is the only one for other n. Where
// neither fits (four heads with 8-bit key codes, whose 128 KiB half table leaves no room
// for the value rows): 8-bit codes take the matrix cores for both products, which beats
// the score table with the vector value sum by 3-12% (61 against 63-69 us per
// Mistral-7B-shaped 8/8-bit layer); narrower codes keep that table (their matrix-core
// key loop spills registers at four heads). Eight heads, and shapes where no table
// fits: the matrix cores for both.
constexpr int attn_mode(int d, int group, int n_k, int bk, int bv) {
  const bool pow2 = n_k == (1 << bk);
  if (group <= 4) {
    const bool full = attn_lds_bytes(d, group, bk, bv, 1 | 4) <= kLdsBytesMax;
    const bool half = pow2 && attn_lds_bytes(d, group, bk, bv, 2 | 4) <= kLdsBytesMax;
    if (full && (group <= 2 || !half)) return 1 | 4;
    if (half) return 2 | 4;
    const int tabmode = pow2 ? 2 : 1;
    if (bk < 8 && attn_lds_bytes(d, group, bk, bv, tabmode) <= kLdsBytesMax) return tabmode;
  }
  return 3 | 4;
}

// Fused append of decode attention: the new token of sequence b (K/V rows at
// k / v + b * sb + h * sh elements, d contiguous) is coded into slot positions[b] before
// that slot's tile is read; the sequence attends to min(positions[b] + 1, seq_len)
// tokens. positions == null: no append. (A kernel argument of its own: enlarging
// AttnArgs past a couple of hundred bytes costs the kernels without a key table their
// scalar query loads.)
struct AppendArgs {
  const unsigned* positions;
  const void* k;
  const void* v;
  int64_t sb, sh;
  int f32, capacity;
  double inv_sqrt_d, k_bins_per_rad, v_bins_per_rad;  // the layer's encode constants
};

// Copy of tiles [0, ntiles) of every (sequence, kv head) of a contiguous cache whose
// angle codes are bk / bv bits wide, with each width below 6 re-packed at 6 bits, into
// dst laid out [batch][kv head][ntiles][tile bytes at the new widths].
hipError_t launch_widen(const uint8_t* src, int src_tiles_per_seq, uint8_t* dst, int d, int bk,
                        int bv, int units, int ntiles, hipStream_t stream);
// lens[b] = min(positions[b] + 1, max_len) for b < batch (device arrays).
hipError_t launch_lengths(const unsigned* positions, unsigned* lens, int batch, unsigned max_len,
                          hipStream_t stream);

hipError_t launch_attn_decode(const AttnArgs& a, const AppendArgs& app, int d,
                              const uint8_t* cache, hipStream_t stream);
// rows = nq * group query rows per kv head (at most 32)
hipError_t launch_attn_multi(const AttnArgs& a, int d, int rows, const uint8_t* cache,
                             hipStream_t stream);

}  // namespace kvq
