// Triplet (octahedral) codec: encode, dequantise and decode attention, plus the host
// side of its C ABI (the Lloyd-Max quantisers are computed here, on the host).
//
// Method: "OCTOPUS: Joint Triplet Quantization for KV Cache via Octahedral
// Parametrization" (TL;DR, What is new): rotated coordinates are quantised three at a
// time; a triplet's direction goes to the square [-1, 1]^2 through the octahedral
// parametrisation, and the two square coordinates and the triplet norm are Lloyd-Max
// quantised against the marginals these quantities actually have after the rotation.
// The rotation is the angle codec's (seeded sign diagonal, normalised Walsh-Hadamard
// transform), and the readings of the steps the page leaves open are stated at the
// declarations in kvq.h.
//
// Kernels (the lane maps follow the data):
//   encode     a wave per (batch, kv head, 64-token tile), sixteen token-heads per step
//              with a quarter vector per lane through the binary64 transform (its
//              cross-lane stages as row swaps); each lane then codes the triplets starting
//              in its block of d/4 consecutive elements, in binary64, with branch-free
//              searches of the boundaries in LDS (compiled for the 4/2/3 allocation,
//              generic otherwise), and ORs the fields into the tokens' records in LDS.
//   decode     lane j rebuilds its triplet (or leftover) in fp32 from the levels, the
//              elements are permuted back to two per lane for the inverse transform.
//   attention  split kernel (grid: splits x batch * kv heads, four waves, a wave per
//              64-token tile): scores with one lane per token, the key plane staged in
//              LDS (rows padded by a word) and a table of the 2^(2 bits_dir)
//              reconstructed directions; online softmax per wave; values with one lane
//              per triplet, summing p * N * rho * w over the tile's tokens; both products
//              on the matrix cores in fp32 (four query heads per instruction); waves
//              merge in LDS and each split writes (max, sum, rotated vector) per query
//              head. A merge kernel (a wave per output row) combines the splits with a
//              log-sum-exp and applies the inverse transform. Far more arithmetic per
//              byte than the angle codec (a few bits per element): this path is bound by
//              the rebuild of the operands (VALU and LDS).
#include <math.h>
#include <string.h>

#include <cmath>
#include <vector>

#include "kvq_attn_common.h"
#include "kvq_codec_dev.h"

namespace kvq {
namespace {

constexpr int kTriMaxLevelsDir = 64, kTriMaxLevelsNorm = 64, kTriMaxLevelsRest = 256;
// longest record: d = 128 at 6/6/8 bits, 16 + 42 * 18 + 2 * 8 = 788 bits
constexpr int kTriMaxRecordWords = 25;

// Geometry of one configuration (device and host).
struct TriGeom {
  int d, T, R;           // head dim, triplets, leftover coordinates
  int bd, bn, br, B;     // field widths; B = 2 bd + bn
  int words;             // record words per token-head
  int nd, nn, nr;        // levels per quantiser
};

__host__ __device__ constexpr TriGeom tri_geom(int d, int bd, int bn, int br) {
  TriGeom g{};
  g.d = d;
  g.T = d / 3;
  g.R = d - 3 * g.T;
  g.bd = bd;
  g.bn = bn;
  g.br = br;
  g.B = 2 * bd + bn;
  g.words = (16 + g.T * g.B + g.R * br + 31) / 32;
  g.nd = 1 << bd;
  g.nn = 1 << bn;
  g.nr = 1 << br;
  return g;
}

// Bit offset and width of field f (f < T: triplet f; f >= T: leftover f - T).
__host__ __device__ inline int field_off(const TriGeom& g, int f) {
  return f < g.T ? 16 + f * g.B : 16 + g.T * g.B + (f - g.T) * g.br;
}
__host__ __device__ inline int field_width(const TriGeom& g, int f) { return f < g.T ? g.B : g.br; }

struct TriArgs {
  TriGeom g;
  int batch, hkv, tiles_per_seq;
  int t0, ntok;
  double inv_sqrt_d;
  SignMask sign;
  const double* cb;  // codebook: levels dir, norm, rest; then bounds dir, norm, rest
};

__device__ inline int cb_bounds_off(const TriGeom& g) { return g.nd + g.nn + g.nr; }

// Number of boundaries below x (the nearest level; the lower one at an exact midpoint),
// for 2^bits levels, without a data-dependent loop: steps of
// 2^(bits-1), .., 1, each taken when the boundary it lands on is still below x (the
// index never passes 2^bits - 1, the last boundary's count). Straight-line code, so the
// searches of different values overlap their LDS reads. BITS > 0 fixes the width at
// compile time; BITS = 0 reads it from bits (steps past the width skipped, a uniform
// test).
template <int BITS>
__device__ __forceinline__ int nearest_steps(const double* bounds, int bits, double x) {
  int idx = 0;
  if constexpr (BITS > 0) {
#pragma unroll
    for (int step = 1 << (BITS - 1); step >= 1; step >>= 1)
      if (bounds[idx + step - 1] < x) idx += step;
  } else {
#pragma unroll
    for (int step = 128; step >= 1; step >>= 1)
      if ((step << 1) <= (1 << bits) && bounds[idx + step - 1] < x) idx += step;
  }
  return idx;
}

__device__ __forceinline__ double sgn64(double x) { return x < 0.0 ? -1.0 : 1.0; }
__device__ __forceinline__ float sgn32(float x) { return x < 0.f ? -1.f : 1.f; }


// ------------------------------------------------------------------------------ encode

// Encode, sixteen token-heads per wave. One wave per (batch, kv head, tile of 64 tokens),
// coded in steps of 16 tokens: the token is the lane's position in its 16-lane row and
// the row is the quarter of the vector. The binary64 transform runs as in the angle
// encoder: in-lane butterflies for element strides 1, 2, 4 and 32 (and 64), then the
// stride 8 as a row swap (v_permlane16_swap) on two of the lane's values at once.
// d = 128: the stride 16 is a row swap too (v_permlane32_swap), after which row q holds
// elements 32 q .. 32 q + 31 of its token; block q is row q. d = 64: after the stride-8
// swap, row (q1, q0) already holds elements 32 q0 + 16 q1 .. + 15 (block 2 q0 + q1), and
// the stride 16 is a plain exchange between rows q1 = 0 and 1 (a swap of each value with
// a copy of itself, then a signed add) that keeps those sets. Triplet j (elements
// 3j .. 3j + 2) is coded by the lane whose block holds its first element; a block's last
// triplet may take one or two elements of the next block (through a lane permute), and
// the last block also codes the leftover coordinates. Triplets per block: 11, 11, 10, 10
// at d = 128; 6, 5, 5, 5 at d = 64. The decisions are
// those of tri_encode_kernel, in binary64: triplet norm rho = |c| / N, the octahedral
// point from c / |c|_1 (the same point as from u = y / N: the map is scale-free), the
// leftover coordinates y / N; each is located among the quantiser's boundaries in LDS.
// Results can differ from a u = y / N evaluation only in the last bits, i.e. only for
// values within rounding distance of a boundary. Fields are ORed into the tokens'
// records in LDS, and a row of 16 lanes stores one record word of 16 consecutive slots.
constexpr int kTriRowWaves = 4;

template <bool ROWS32>
__device__ __forceinline__ void tri_row_butterfly(double& x, double& y) {
  const uint64_t a = (uint64_t)__double_as_longlong(x), b = (uint64_t)__double_as_longlong(y);
  uint32_t lo0, lo1, hi0, hi1;
  if constexpr (ROWS32) {
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)a, (uint32_t)b, false, false);
    const auto hi =
        __builtin_amdgcn_permlane32_swap((uint32_t)(a >> 32), (uint32_t)(b >> 32), false, false);
    lo0 = lo[0]; lo1 = lo[1]; hi0 = hi[0]; hi1 = hi[1];
  } else {
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)a, (uint32_t)b, false, false);
    const auto hi =
        __builtin_amdgcn_permlane16_swap((uint32_t)(a >> 32), (uint32_t)(b >> 32), false, false);
    lo0 = lo[0]; lo1 = lo[1]; hi0 = hi[0]; hi1 = hi[1];
  }
  // (value of the lower lane, value of the upper lane) in every lane: see the encoder
  const double u = __longlong_as_double((long long)(((uint64_t)hi0 << 32) | lo0));
  const double w = __longlong_as_double((long long)(((uint64_t)hi1 << 32) | lo1));
  x = u + w;
  y = u - w;
}

// BD, BN, BR: the bit allocation fixed at compile time (the searches' step counts), or 0
// for the widths of the descriptor.
// spw: 16-token steps per wave, 4 (a whole tile) or 1 (a quarter tile each, for launches
// with too few tiles to fill the GPU).
template <int D, bool F32, int BD, int BN, int BR>
__global__ __launch_bounds__(kTriRowWaves * 64) void tri_encode_rows_kernel(
    TriArgs a, uint8_t* cache, const void* k, const void* v, int64_t sb, int64_t st, int64_t sh,
    int spw) {
  constexpr int E = D / 4, PL = E / 2, TPS = 16;
  constexpr int T = D / 3, R = D - 3 * T;
  constexpr int MAXT = D == 128 ? 11 : 6;  // triplets of the fullest block
  const TriGeom& g = a.g;
  __shared__ double s_bd[kTriMaxLevelsDir], s_bn[kTriMaxLevelsNorm], s_br[kTriMaxLevelsRest];
  __shared__ uint32_t s_rec_all[kTriRowWaves][TPS][kTriMaxRecordWords + 1];
  const int bo = cb_bounds_off(g);
  for (int i = threadIdx.x; i < g.nd - 1; i += kTriRowWaves * 64) s_bd[i] = a.cb[bo + i];
  for (int i = threadIdx.x; i < g.nn - 1; i += kTriRowWaves * 64) s_bn[i] = a.cb[bo + g.nd - 1 + i];
  for (int i = threadIdx.x; i < g.nr - 1; i += kTriRowWaves * 64)
    s_br[i] = a.cb[bo + g.nd - 1 + g.nn - 1 + i];
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tq = lane & 15, q = lane >> 4;  // token within the step, quarter of the vector
  uint32_t(*s_rec)[kTriMaxRecordWords + 1] = s_rec_all[wave];
  const int tile_lo = a.t0 / kTile;
  const int tiles_touched = (a.t0 + a.ntok - 1) / kTile - tile_lo + 1;
  const int parts = 4 / spw;  // waves per tile
  const int task = blockIdx.x * kTriRowWaves + wave;
  if (task >= a.batch * a.hkv * tiles_touched * parts) return;  // no barrier follows
  const int tt_task = task / parts, part = task % parts;
  const int bh = tt_task / tiles_touched, b = bh / a.hkv, h = bh % a.hkv;
  const int tile = tile_lo + tt_task % tiles_touched, tok_base = tile * kTile;
  // this wave's slots of the tile: the part's steps, within the encoded range
  const int j_lo = max(max(a.t0 - tok_base, 0), part * spw * TPS);
  const int j_hi = min(min(a.t0 + a.ntok - tok_base, kTile), (part + 1) * spw * TPS);
  if (j_lo >= j_hi) return;
  const size_t tile_bytes = (size_t)2 * g.words * kTile * 4;
  uint32_t* tp = reinterpret_cast<uint32_t*>(
      cache + ((size_t)(b * a.hkv + h) * a.tiles_per_seq + tile) * tile_bytes);

  // lane slots 8m + r hold elements 32m + 8q + r before the row stages; bit 8m + r of
  // sbits is that element's sign, and for fp16 input hmask[k] flips the sign bits of the
  // packed pair k
  uint32_t sbits = 0;
#pragma unroll
  for (int m = 0; m < E / 8; ++m)
    sbits |= (uint32_t)((a.sign.w[(32 * m + 8 * q) >> 6] >> ((32 * m + 8 * q) & 63)) & 0xFFu) << (8 * m);
  uint32_t hmask[PL];
#pragma unroll
  for (int kk = 0; kk < PL; ++kk)
    hmask[kk] = (((sbits >> (2 * kk)) & 1u) << 15) | (((sbits >> (2 * kk + 1)) & 1u) << 31);

  // this lane's block of E consecutive elements, its triplets (the first is J0, whose
  // first element is local slot o) and the row holding the next block
  const int blk = D == 128 ? q : 2 * (q & 1) + (q >> 1);
  const int J0 = D == 128 ? (blk == 0 ? 0 : blk == 1 ? 11 : blk == 2 ? 22 : 32)
                          : (blk == 0 ? 0 : blk == 1 ? 6 : blk == 2 ? 11 : 16);
  const int ntri = D == 128 ? (blk < 2 ? 11 : 10) : (blk == 0 ? 6 : 5);
  const int o = 3 * J0 - E * blk;  // d = 128: 0, 1, 2, 0; d = 64: 0, 2, 1, 0
  const int q_next = D == 128 ? ((q + 1) & 3) : (blk == 0 ? 2 : 1);  // blocks 2, 3 need none
  const double qsgn = (q >> 1) ? -1.0 : 1.0;  // d = 64, stride 16: upper rows keep u - v

  auto row_offset = [&](int jb) {
    const int jr = min(jb + tq, j_hi - 1);
    return (int64_t)b * sb + (int64_t)(tok_base + jr - a.t0) * st + (int64_t)h * sh + 8 * q;
  };
  uint32_t raw[2][PL];
  auto load_raw = [&](int kv, int jb) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(
        static_cast<const __half*>(kv == 0 ? k : v) + row_offset(jb));
#pragma unroll
    for (int kk = 0; kk < PL; ++kk) raw[kv][kk] = p[16 * (kk >> 2) + (kk & 3)];
  };
  if (!F32) {
    load_raw(0, j_lo);
    load_raw(1, j_lo);
  }

  for (int jb = j_lo; jb < j_hi; jb += TPS) {
    const int j = jb + tq;
    const bool act = j < j_hi;
    const int64_t row_off = row_offset(jb);
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {  // unrolled: raw[kv] stays in registers
      double y[E + 5];
      if (F32) {
        const float* p = static_cast<const float*>(kv == 0 ? k : v) + row_off;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          float f = p[32 * (e >> 3) + (e & 7)];
          if (!act) f = 0.f;
          if ((sbits >> e) & 1u) f = -f;
          y[e] = (double)f;
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < PL; ++kk) {
          const uint32_t w = (act ? raw[kv][kk] : 0u) ^ hmask[kk];
          y[2 * kk] = (double)__half2float(__ushort_as_half((uint16_t)(w & 0xFFFFu)));
          y[2 * kk + 1] = (double)__half2float(__ushort_as_half((uint16_t)(w >> 16)));
        }
        load_raw(kv, jb + TPS);  // clamped row past the range: re-read, discarded
      }
#pragma unroll
      for (int hs = 1; hs < E; hs <<= 1) {
#pragma unroll
        for (int i = 0; i < E; ++i) {
          if (i & hs) continue;
          const double u = y[i], w = y[i + hs];
          y[i] = u + w;
          y[i + hs] = u - w;
        }
      }
#pragma unroll
      for (int i = 0; i < E; ++i)
        if (!(i & 8)) tri_row_butterfly<false>(y[i], y[i + 8]);
      if constexpr (D == 128) {
#pragma unroll
        for (int i = 0; i < E; ++i)
          if (!(i & 16)) tri_row_butterfly<true>(y[i], y[i + 16]);
      } else {
        // each value against its partner in the other half of the wave: the swap leaves
        // (lower lane's value, upper lane's value) in every lane
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const uint64_t u = (uint64_t)__double_as_longlong(y[i]);
          const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
          const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32),
                                                           false, false);
          const double lw = __longlong_as_double((long long)(((uint64_t)hi[0] << 32) | lo[0]));
          const double up = __longlong_as_double((long long)(((uint64_t)hi[1] << 32) | lo[1]));
          y[i] = fma(up, qsgn, lw);
        }
      }
      // slot s now holds element E blk + s
      double n2 = 0.0;
#pragma unroll
      for (int i = 0; i < E; ++i) {
        y[i] *= a.inv_sqrt_d;
        n2 = fma(y[i], y[i], n2);
      }
      n2 += shfl_xor_f64(n2, 16);
      n2 += shfl_xor_f64(n2, 32);
      const double nrm = sqrt(n2);
      const double rn = nrm > 0.0 ? 1.0 / nrm : 0.0;
      // the next block's first two elements (for the triplets that straddle blocks)
      y[E] = __shfl(y[0], tq + 16 * q_next, 64);
      y[E + 1] = __shfl(y[1], tq + 16 * q_next, 64);
#pragma unroll
      for (int i = E + 2; i < E + 5; ++i) y[i] = 0.0;

      // the records of this step's tokens: word 0 starts as the fp16 bits of N
      for (int i = lane; i < TPS * g.words; i += 64) {
        const int tt = i / g.words, w = i - tt * g.words;
        s_rec[tt][w] = 0u;
      }
      asm volatile("" ::: "memory");  // a wave's LDS accesses complete in order
      if (q == 0) s_rec[tq][0] = (uint32_t)fp16_bits(fp16_round_pos(fmin(nrm, kFp16Max)));
      asm volatile("" ::: "memory");
      auto put = [&](int f, uint32_t field) {
        const int off = field_off(g, f), wd = field_width(g, f);
        const int wi = off >> 5, sh = off & 31;
        atomicOr(&s_rec[tq][wi], field << sh);
        if (sh + wd > 32) atomicOr(&s_rec[tq][wi + 1], field >> (32 - sh));
      };
#pragma unroll
      for (int i = 0; i < MAXT; ++i) {
        if (i < ntri) {
          double c[3];
#pragma unroll
          for (int m = 0; m < 3; ++m) {
            const int s0 = 3 * i + m;  // element slot for o = 0; o = 1, 2 read one or two on
            c[m] = o == 0 ? y[s0] : o == 1 ? y[s0 + 1] : y[s0 + 2];
          }
          const double rho = sqrt(fma(c[2], c[2], fma(c[1], c[1], c[0] * c[0]))) * rn;
          const double l1 = fabs(c[0]) + fabs(c[1]) + fabs(c[2]);
          const double rl = 1.0 / (l1 > 0.0 ? l1 : 1.0);
          const double p1 = c[0] * rl, p2 = c[1] * rl;
          const bool up = c[2] * rl >= 0.0;
          const double sx = up ? p1 : (1.0 - fabs(p2)) * sgn64(p1);
          const double tx = up ? p2 : (1.0 - fabs(p1)) * sgn64(p2);
          const uint32_t cs = (uint32_t)nearest_steps<BD>(s_bd, g.bd, sx);
          const uint32_t ct = (uint32_t)nearest_steps<BD>(s_bd, g.bd, tx);
          const uint32_t cr = (uint32_t)nearest_steps<BN>(s_bn, g.bn, rho);
          put(J0 + i, cs | (ct << (BD > 0 ? BD : g.bd)) | (cr << (2 * (BD > 0 ? BD : g.bd))));
        }
      }
      if (blk == 3) {
#pragma unroll
        for (int r = 0; r < R; ++r)
          put(T + r, (uint32_t)nearest_steps<BR>(s_br, g.br, y[E - R + r] * rn));
      }
      asm volatile("" ::: "memory");
      if (act)
        for (int w = q; w < g.words; w += 4) tp[(size_t)(kv * g.words + w) * kTile + j] = s_rec[tq][w];
      asm volatile("" ::: "memory");  // the next plane's clear stays after these reads
    }
  }
}

// ------------------------------------------------------------------------------ decode

template <int D, bool F32OUT>
__global__ __launch_bounds__(256) void tri_decode_kernel(TriArgs a, const uint8_t* cache,
                                                         void* k_out, void* v_out) {
  constexpr int P = D / 2;
  const TriGeom& g = a.g;
  __shared__ float s_ld[kTriMaxLevelsDir], s_ln[kTriMaxLevelsNorm], s_lr[kTriMaxLevelsRest];
  for (int i = threadIdx.x; i < g.nd; i += 256) s_ld[i] = (float)a.cb[i];
  for (int i = threadIdx.x; i < g.nn; i += 256) s_ln[i] = (float)a.cb[g.nd + i];
  for (int i = threadIdx.x; i < g.nr; i += 256) s_lr[i] = (float)a.cb[g.nd + g.nn + i];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  // token-head index in 32 bits (the host keeps B * ntok * Hkv below 2^32)
  const unsigned item = blockIdx.x * 4u + (unsigned)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const unsigned total = (unsigned)a.batch * (unsigned)a.ntok * (unsigned)a.hkv;
  if (item >= total) return;
  const int h = (int)(item % (unsigned)a.hkv);
  const unsigned bj = item / (unsigned)a.hkv;
  const int j = (int)(bj % (unsigned)a.ntok), b = (int)(bj / (unsigned)a.ntok);
  const int slot = a.t0 + j, tile = slot / kTile, t = slot % kTile;
  const size_t tile_bytes = (size_t)2 * g.words * kTile * 4;
  const uint32_t* tp = reinterpret_cast<const uint32_t*>(
      cache + ((size_t)(b * a.hkv + h) * a.tiles_per_seq + tile) * tile_bytes);
  const int nf = g.T + g.R;
  const int f = lane < nf ? lane : 0;
  const int off = field_off(g, f), wd = field_width(g, f);
  const int i = lane & (P - 1);
  const float isd = (float)a.inv_sqrt_d;

#pragma unroll 1
  for (int kv = 0; kv < 2; ++kv) {
    const uint32_t* rec = tp + (size_t)kv * g.words * kTile + t;
    const float nu = __half2float(__ushort_as_half((uint16_t)(rec[0] & 0xFFFFu)));
    const int wi = off >> 5;
    const uint32_t lo = rec[(size_t)wi * kTile];
    const uint32_t hi = wi + 1 < g.words ? rec[(size_t)(wi + 1) * kTile] : 0u;
    const uint64_t win = ((uint64_t)hi << 32) | lo;
    const uint32_t val = (uint32_t)(win >> (off & 31)) & ((1u << wd) - 1u);
    float c0 = 0.f, c1 = 0.f, c2 = 0.f;
    if (f < g.T) {
      const float s = s_ld[val & (g.nd - 1)], tt = s_ld[(val >> g.bd) & (g.nd - 1)];
      const float rho = s_ln[val >> (2 * g.bd)];
      const float z = 1.f - fabsf(s) - fabsf(tt);
      const float x = z >= 0.f ? s : (1.f - fabsf(tt)) * sgn32(s);
      const float y = z >= 0.f ? tt : (1.f - fabsf(s)) * sgn32(tt);
      const float sc = nu * rho * rsqrtf(x * x + y * y + z * z);
      c0 = x * sc;
      c1 = y * sc;
      c2 = z * sc;
    } else {
      c0 = nu * s_lr[val];
    }
    // elements 2i, 2i+1 back to lane i
    float e[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int el = 2 * i + m;
      const int srcl = el < 3 * g.T ? el / 3 : g.T + (el - 3 * g.T);
      const int comp = el < 3 * g.T ? el % 3 : 0;
      const float v0 = __shfl(c0, srcl, 64), v1 = __shfl(c1, srcl, 64), v2 = __shfl(c2, srcl, 64);
      e[m] = comp == 0 ? v0 : (comp == 1 ? v1 : v2);
    }
    float a0 = e[0], a1 = e[1];
    fwht_pairs_f32<P>(a0, a1, i);
    a0 *= isd;
    a1 *= isd;
    if (sign_neg(a.sign, 2 * i)) a0 = -a0;
    if (sign_neg(a.sign, 2 * i + 1)) a1 = -a1;
    if (lane < P) {
      const size_t row = ((size_t)(b * a.ntok + j) * a.hkv + h) * D;
      void* out = kv == 0 ? k_out : v_out;
      if (F32OUT)
        reinterpret_cast<float2*>(out)[(row >> 1) + i] = make_float2(a0, a1);
      else
        reinterpret_cast<__half2*>(out)[(row >> 1) + i] = __floats2half2_rn(a0, a1);
    }
  }
}

// --------------------------------------------------------------------------- attention

struct TriAttnArgs {
  TriGeom g;
  int batch, hkv, hq, group, tiles_per_seq;
  int seq_len, ntiles, nsplit, tiles_per_split;
  int q_f32, out_f32;
  float q_scale;      // softmax scale * log2(e), folded into the rotated query
  float inv_sqrt_d;
  SignMask sign;
  const double* cb;
  const void* q;      // [B, Hq, d]
  void* out;          // [B, Hq, d]
  float* part_ml;     // [B * Hq][nsplit][2]
  float* part_acc;    // [B * Hq][nsplit][d] (rotated domain, element order of the codec)
};

constexpr int kTriWaves = 4;
constexpr int kTriMaxWords = 32;  // record words the attention kernel serves

typedef float mf4 __attribute__((ext_vector_type(4)));
typedef _Float16 th4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ mf4 tri_mfma(float a, float b, mf4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

// A plane staged in LDS as [words][kPlaneRow]: a row of 64 slots plus one pad word, so
// the words of one slot (read together when a lane owns a field and loops over slots)
// fall in different banks.
constexpr int kPlaneRow = kTile + 1;

// Field f of the record of slot `slot` in a staged plane.
__device__ __forceinline__ uint32_t staged_field(const uint32_t* plane, int off, int wd, int words,
                                                 int slot) {
  const int wi = off >> 5;
  const uint32_t lo = plane[wi * kPlaneRow + slot];
  const uint32_t hi = wi + 1 < words ? plane[(wi + 1) * kPlaneRow + slot] : 0u;
  const uint64_t win = ((uint64_t)hi << 32) | lo;
  return (uint32_t)(win >> (off & 31)) & ((1u << wd) - 1u);
}

// BD, BN, BR != 0: the bit allocation fixed at compile time (then every field offset,
// mask and table index of the key loop is a constant and the record length is known);
// 0: taken from the descriptor.
template <int D, int G, int DIRB, int BD = 0, int BN = 0, int BR = 0>
__global__ __launch_bounds__(kTriWaves * 64) void tri_attn_split_kernel(TriAttnArgs a,
                                                                         const uint8_t* cache) {
  constexpr int P = D / 2, T = D / 3, R = D - 3 * T;
  constexpr bool FIXED = BD != 0;
  const TriGeom g = FIXED ? tri_geom(D, BD, BN, BR) : a.g;
  // LDS: direction table (2^(2 bd) unit vectors indexed by the t code then the s code,
  // so a triplet field's low 2 bd bits are the index; sized for bd <= DIRB), norm and
  // leftover levels, the rotated query as padded triplets, then per wave: the staged
  // plane and the token weights
  __shared__ float4 s_dir[(1 << DIRB) * (1 << DIRB)];
  __shared__ float s_ln[kTriMaxLevelsNorm], s_lr[kTriMaxLevelsRest];
  __shared__ float4 s_q3[G][T + 1];        // (q~[3j], q~[3j+1], q~[3j+2], 0); row T: leftovers
  __shared__ uint32_t s_plane[kTriWaves][32 * kPlaneRow];  // up to 32 record words
  // p * N per head and token, fp16 (the value products' operand type), rows of 64
  __shared__ __align__(16) _Float16 s_w[kTriWaves][G][kTile];
  __shared__ float s_ml[kTriWaves][G][2];
  __shared__ float s_acc[kTriWaves][G][D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int split = blockIdx.x, bk = blockIdx.y, b = bk / a.hkv;
  const int nd = g.nd;
  for (int idx = tid; idx < nd * nd; idx += kTriWaves * 64) {
    const float s = (float)a.cb[idx % nd], tt = (float)a.cb[idx / nd];
    const float z = 1.f - fabsf(s) - fabsf(tt);
    const float x = z >= 0.f ? s : (1.f - fabsf(tt)) * sgn32(s);
    const float y = z >= 0.f ? tt : (1.f - fabsf(s)) * sgn32(tt);
    const float r = rsqrtf(x * x + y * y + z * z);
    s_dir[idx] = make_float4(x * r, y * r, z * r, 0.f);
  }
  for (int idx = tid; idx < g.nn; idx += kTriWaves * 64) s_ln[idx] = (float)a.cb[nd + idx];
  for (int idx = tid; idx < g.nr; idx += kTriWaves * 64) s_lr[idx] = (float)a.cb[nd + g.nn + idx];
  // rotated query: wave w < G rotates head w (lane p < P holds elements 2p, 2p+1)
  for (int hh = wave; hh < G; hh += kTriWaves) {
    const size_t qoff = ((size_t)bk * G + hh) * D;
    float x0, x1;
    const int p = lane & (P - 1);
    if (a.q_f32) {
      const float2 v = reinterpret_cast<const float2*>(a.q)[(qoff >> 1) + p];
      x0 = v.x;
      x1 = v.y;
    } else {
      const __half2 v = reinterpret_cast<const __half2*>(a.q)[(qoff >> 1) + p];
      x0 = __low2float(v);
      x1 = __high2float(v);
    }
    if (sign_neg(a.sign, 2 * p)) x0 = -x0;
    if (sign_neg(a.sign, 2 * p + 1)) x1 = -x1;
    fwht_pairs_f32<P>(x0, x1, p);
    const float sc = a.inv_sqrt_d * a.q_scale;
    x0 *= sc;
    x1 *= sc;
    float* row = reinterpret_cast<float*>(&s_q3[hh][0]);
    if (lane < P) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int el = 2 * p + m;
        const float val = m ? x1 : x0;
        const int slotq = el < 3 * T ? (el / 3) * 4 + el % 3 : T * 4 + (el - 3 * T);
        row[slotq] = val;
      }
      if (lane < T + 1) row[lane * 4 + 3] = 0.f;
      if (lane == 0 && R < 3) {
        for (int r = R; r < 3; ++r) row[T * 4 + r] = 0.f;
      }
    }
  }
  __syncthreads();

  const int tile_begin = split * a.tiles_per_split;
  const int tile_end = min(tile_begin + a.tiles_per_split, a.ntiles);
  const size_t tile_bytes = (size_t)2 * g.words * kTile * 4;
  const uint8_t* base = cache + (size_t)bk * a.tiles_per_seq * tile_bytes;
  const int nf = T + R;
  const int f = lane < nf ? lane : 0;
  const int foff = field_off(g, f), fwd = field_width(g, f);

  // Both products run on the matrix cores (sixteen 4 x 4 blocks: lane 4b + i supplies
  // row i of block b's A operand, lane 4b + j column j of B, and lane 4b + j accumulates
  // D[b][i][j]); with the query heads as the rows, A in lane l is head 4 hg + (l & 3)'s
  // operand. Scores, v_mfma_f32_4x4x1f32 in fp32: lane = token, B = the token's rebuilt
  // key element rho * w[c]. Values, v_mfma_f32_4x4x4f16 (fp16 operands, fp32 sums,
  // four tokens per instruction): lane = triplet (or leftover), B = its element of four
  // tokens' rebuilt values, A = those tokens' weights. The scores stay fp32, as in the
  // angle codec's kernel (large logits); fp16 operands add about 2^-11 per value term.
  constexpr int HG = G > 4 ? G / 4 : 1;
  const int hl = lane & 3;
  float m[G], l[G];
  mf4 ax[HG], ay[HG], az[HG];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
  }
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) ax[hg] = ay[hg] = az[hg] = mf4{0.f, 0.f, 0.f, 0.f};
  uint32_t* plane = s_plane[wave];
  // Both planes of a tile are loaded into registers at once (all loads in flight), the
  // next tile's as soon as the current value plane is staged, so their latency overlaps
  // the value sum.
  uint32_t kw[kTriMaxWords], vw[kTriMaxWords];
  const int words = g.words;
  auto load_tile = [&](int tile) {
    const uint32_t* tw = reinterpret_cast<const uint32_t*>(base + (size_t)tile * tile_bytes);
#pragma unroll
    for (int w = 0; w < kTriMaxWords; ++w)
      if (w < words) {
        kw[w] = tw[w * kTile + lane];
        vw[w] = tw[(words + w) * kTile + lane];
      }
  };
  if (tile_begin + wave < tile_end) load_tile(tile_begin + wave);
  for (int tile = tile_begin + wave; tile < tile_end; tile += kTriWaves) {
    const int nvalid = min(a.seq_len - tile * kTile, kTile);
    const bool valid = lane < nvalid;
    // ---- keys: stage the key plane, one lane per token
#pragma unroll
    for (int w = 0; w < kTriMaxWords; ++w)
      if (w < words) plane[w * kPlaneRow + lane] = kw[w];
    asm volatile("" ::: "memory");  // a wave's LDS accesses complete in order
    const float nu_k = __half2float(__ushort_as_half((uint16_t)(plane[lane] & 0xFFFFu)));
    mf4 kx[HG], ky[HG], kz[HG];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) kx[hg] = ky[hg] = kz[hg] = mf4{0.f, 0.f, 0.f, 0.f};
    auto key_triplet = [&](int jt) {
      const uint32_t val = staged_field(plane, 16 + jt * g.B, g.B, g.words, lane);
      const float4 w4 = s_dir[val & (nd * nd - 1)];
      const float rho = s_ln[val >> (2 * g.bd)];
      const float bx = rho * w4.x, by = rho * w4.y, bz = rho * w4.z;
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        const float4 q4 = s_q3[min(4 * hg + hl, G - 1)][jt];  // rows past G: unused sums
        kx[hg] = tri_mfma(q4.x, bx, kx[hg]);
        ky[hg] = tri_mfma(q4.y, by, ky[hg]);
        kz[hg] = tri_mfma(q4.z, bz, kz[hg]);
      }
    };
    if constexpr (FIXED) {
#pragma unroll
      for (int jt = 0; jt < T; ++jt) key_triplet(jt);
    } else {
      for (int jt = 0; jt < T; ++jt) key_triplet(jt);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t val = staged_field(plane, 16 + T * g.B + r * g.br, g.br, g.words, lane);
      const float u = s_lr[val];
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        const float4 q4 = s_q3[min(4 * hg + hl, G - 1)][T];
        kx[hg] = tri_mfma(r == 0 ? q4.x : (r == 1 ? q4.y : q4.z), u, kx[hg]);
      }
    }
    // ---- value plane staged (the next tile's planes are requested), then the softmax
    // weights p * N per token
    const float nu_v = __half2float(__ushort_as_half((uint16_t)(vw[0] & 0xFFFFu)));
    asm volatile("" ::: "memory");
#pragma unroll
    for (int w = 0; w < kTriMaxWords; ++w)
      if (w < words) plane[w * kPlaneRow + lane] = vw[w];
    if (tile + kTriWaves < tile_end) load_tile(tile + kTriWaves);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float sc = kx[hh >> 2][hh & 3] + ky[hh >> 2][hh & 3] + kz[hh >> 2][hh & 3];
      const float s = valid ? sc * nu_k : -INFINITY;
      const float mnew = fmaxf(m[hh], wave_max(s));
      const float alpha = mnew == -INFINITY ? 1.f : fast_exp2(m[hh] - mnew);
      l[hh] *= alpha;
      ax[hh >> 2][hh & 3] *= alpha;
      ay[hh >> 2][hh & 3] *= alpha;
      az[hh >> 2][hh & 3] *= alpha;
      m[hh] = mnew;
      const float pv = m[hh] == -INFINITY ? 0.f : fast_exp2(s - m[hh]);
      l[hh] += pv;
      s_w[wave][hh][lane] = (_Float16)(valid ? pv * nu_v : 0.f);
    }
    asm volatile("" ::: "memory");
    // ---- values: lane f rebuilds its triplet (or leftover) of every token; the matrix
    // instructions (fp16 operands, fp32 sums, four tokens each) run on the whole wave,
    // lanes past the fields contributing zero
    for (int t4 = 0; t4 < kTile; t4 += 4) {
      float c[3][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t val = staged_field(plane, foff, fwd, g.words, t4 + u);
        float c0 = 0.f, c1 = 0.f, c2 = 0.f;
        if (f < T) {
          const float4 w4 = s_dir[val & (nd * nd - 1)];
          const float rho = s_ln[val >> (2 * g.bd)];
          c0 = rho * w4.x;
          c1 = rho * w4.y;
          c2 = rho * w4.z;
        } else {
          c0 = s_lr[val];
        }
        if (lane >= nf) c0 = c1 = c2 = 0.f;
        c[0][u] = c0;
        c[1][u] = c1;
        c[2][u] = c2;
      }
      const th4 bx = th4{(_Float16)c[0][0], (_Float16)c[0][1], (_Float16)c[0][2], (_Float16)c[0][3]};
      const th4 by = th4{(_Float16)c[1][0], (_Float16)c[1][1], (_Float16)c[1][2], (_Float16)c[1][3]};
      const th4 bz = th4{(_Float16)c[2][0], (_Float16)c[2][1], (_Float16)c[2][2], (_Float16)c[2][3]};
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        const th4 wgt = *reinterpret_cast<const th4*>(&s_w[wave][min(4 * hg + hl, G - 1)][t4]);
        ax[hg] = __builtin_amdgcn_mfma_f32_4x4x4f16(wgt, bx, ax[hg], 0, 0, 0);
        ay[hg] = __builtin_amdgcn_mfma_f32_4x4x4f16(wgt, by, ay[hg], 0, 0, 0);
        az[hg] = __builtin_amdgcn_mfma_f32_4x4x4f16(wgt, bz, az[hg], 0, 0, 0);
      }
    }
    asm volatile("" ::: "memory");
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) l[hh] = wave_sum(l[hh]);
  // ---- waves merge in LDS (rotated-domain element order of the codec)
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      s_ml[wave][hh][0] = m[hh];
      s_ml[wave][hh][1] = l[hh];
    }
  }
  if (lane < nf) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float v0 = ax[hh >> 2][hh & 3], v1 = ay[hh >> 2][hh & 3], v2 = az[hh >> 2][hh & 3];
      if (f < T) {
        s_acc[wave][hh][3 * f] = v0;
        s_acc[wave][hh][3 * f + 1] = v1;
        s_acc[wave][hh][3 * f + 2] = v2;
      } else {
        s_acc[wave][hh][3 * T + (f - T)] = v0;
      }
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += kTriWaves * 64) {
    const int hh = idx / D, e = idx % D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kTriWaves; ++w) mm = fmaxf(mm, s_ml[w][hh][0]);
    float ll = 0.f, aa = 0.f;
#pragma unroll
    for (int w = 0; w < kTriWaves; ++w) {
      const float fct = mm == -INFINITY ? 0.f : fast_exp2(s_ml[w][hh][0] - mm);
      ll += s_ml[w][hh][1] * fct;
      aa += s_acc[w][hh][e] * fct;
    }
    const size_t rowi = ((size_t)bk * G + hh) * a.nsplit + split;
    a.part_acc[rowi * D + e] = aa;
    if (e == 0) {
      a.part_ml[2 * rowi] = mm;
      a.part_ml[2 * rowi + 1] = ll;
    }
  }
}

// One wave per output row (batch, query head): log-sum-exp over the splits, then the
// inverse transform of acc / l (lane p holds elements 2p, 2p+1). The partials come from
// other compute units through memory, so their loads are issued together rather than
// one split after another: lane s takes the (max, sum) of splits s, s + 64, ..., the
// per-split factors go through LDS, and the accumulator loads of kMergeUnroll splits are
// in flight at once (a dependent load per split had made this kernel 12.7 us at 32
// splits).
constexpr int kTriMaxSplits = 1024;  // tri_split_plan's ceiling
constexpr int kMergeUnroll = 16;
template <int D>
__global__ __launch_bounds__(64) void tri_attn_merge_kernel(TriAttnArgs a) {
  constexpr int P = D / 2;
  __shared__ float s_f[kTriMaxSplits];  // exp2(m_s - max) of split s
  const int lane = threadIdx.x;
  const size_t row = blockIdx.x;
  const int ns = a.nsplit;
  const float* ml = a.part_ml + 2 * row * ns;
  const float* pa = a.part_acc + row * ns * D;
  const int p = lane & (P - 1);
  float mm = -INFINITY;
  for (int s = lane; s < ns; s += 64) mm = fmaxf(mm, ml[2 * s]);
  mm = wave_max(mm);
  float ll = 0.f;
  for (int s = lane; s < ns; s += 64) {
    const float fct = mm == -INFINITY ? 0.f : fast_exp2(ml[2 * s] - mm);
    s_f[s] = fct;
    ll += ml[2 * s + 1] * fct;
  }
  ll = wave_sum(ll);
  __syncthreads();
  float a0 = 0.f, a1 = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kMergeUnroll) {
    float2 v[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u)
      v[u] = *reinterpret_cast<const float2*>(pa + (size_t)min(s0 + u, ns - 1) * D + 2 * p);
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      if (s0 + u < ns) {
        const float fct = s_f[s0 + u];
        a0 += v[u].x * fct;
        a1 += v[u].y * fct;
      }
    }
  }
  const float inv = ll > 0.f ? 1.f / ll : 0.f;
  a0 *= inv;
  a1 *= inv;
  fwht_pairs_f32<P>(a0, a1, p);
  a0 *= a.inv_sqrt_d;
  a1 *= a.inv_sqrt_d;
  if (sign_neg(a.sign, 2 * p)) a0 = -a0;
  if (sign_neg(a.sign, 2 * p + 1)) a1 = -a1;
  if (lane < P) {
    const size_t o = row * D;
    if (a.out_f32)
      reinterpret_cast<float2*>(a.out)[(o >> 1) + p] = make_float2(a0, a1);
    else
      reinterpret_cast<__half2*>(a.out)[(o >> 1) + p] = __floats2half2_rn(a0, a1);
  }
}

// ------------------------------------------------------------------- host: quantisers

// 40-point Gauss-Legendre rule on [-1, 1]: nodes are the roots of P_40 (Newton's method
// on the three-term recurrence from the standard initial guesses), weights
// 2 / ((1 - x^2) P_40'(x)^2).
struct GaussRule {
  double x[40], w[40];
};

GaussRule gauss_legendre40() {
  constexpr int n = 40;
  GaussRule r;
  for (int i = 0; i < n; ++i) {
    double x = cos(M_PI * (i + 0.75) / (n + 0.5));
    double dp = 1.0;
    for (int it = 0; it < 100; ++it) {
      double p0 = 1.0, p1 = x;
      for (int k = 1; k < n; ++k) {
        const double p2 = ((2.0 * k + 1.0) * x * p1 - k * p0) / (k + 1.0);
        p0 = p1;
        p1 = p2;
      }
      dp = n * (x * p1 - p0) / (x * x - 1.0);
      const double dx = p1 / dp;
      x -= dx;
      if (fabs(dx) < 1e-16) break;
    }
    double p0 = 1.0, p1 = x;
    for (int k = 1; k < n; ++k) {
      const double p2 = ((2.0 * k + 1.0) * x * p1 - k * p0) / (k + 1.0);
      p0 = p1;
      p1 = p2;
    }
    dp = n * (x * p1 - p0) / (x * x - 1.0);
    r.x[n - 1 - i] = x;  // ascending
    r.w[n - 1 - i] = 2.0 / ((1.0 - x * x) * dp * dp);
  }
  return r;
}

enum Marginal { kOct = 0, kNorm = 1, kCoord = 2 };

// The marginals (up to constants, which cancel in the means and quantiles).
double marginal(int kind, int d, double x) {
  if (kind == kOct) {
    const double s = fabs(x), c = s * s + (1.0 - s) * (1.0 - s);
    return (2.0 * (1.0 - s) / (2.0 * s * s + (1.0 - s) * (1.0 - s)) +
            2.0 * s / (s * s + 2.0 * (1.0 - s) * (1.0 - s))) / sqrt(c);
  }
  const double q = 1.0 - x * x;
  if (q <= 0.0) return 0.0;
  if (kind == kNorm) return x * x * pow(q, (d - 5) / 2.0);
  return pow(q, (d - 3) / 2.0);
}

struct LloydMax {
  const GaussRule& gl;
  int kind, d;
  double lo, hi;
  bool split0;  // cells are split at 0

  void cell(double a, double b, double* mass, double* mom) const {
    double ms = 0.0, mo = 0.0;
    double edges[3] = {a, b, b};
    int ne = 2;
    if (split0) {
      edges[1] = fmin(fmax(0.0, a), b);
      edges[2] = b;
      ne = 3;
    }
    for (int p = 0; p + 1 < ne; ++p) {
      const double x0 = edges[p], x1 = edges[p + 1];
      const double half = 0.5 * (x1 - x0), mid = 0.5 * (x1 + x0);
      double sm = 0.0, sx = 0.0;
      for (int i = 0; i < 40; ++i) {
        const double x = mid + half * gl.x[i];
        const double fx = marginal(kind, d, x);
        sm += gl.w[i] * fx;
        sx += gl.w[i] * fx * x;
      }
      ms += half * sm;
      mo += half * sx;
    }
    *mass = ms;
    *mom = mo;
  }
  double cdf(double x) const {
    double m, mu;
    cell(lo, x, &m, &mu);
    return m;
  }
  void fit(int bits, double* levels) const {
    const int n = 1 << bits;
    const double total = cdf(hi);
    for (int i = 0; i < n; ++i) {
      const double q = (i + 0.5) / n;
      double a = lo, b = hi;
      for (int it = 0; it < 200; ++it) {
        const double mid = 0.5 * (a + b);
        if (mid <= a || mid >= b) break;
        if (cdf(mid) < q * total) a = mid;
        else b = mid;
      }
      levels[i] = 0.5 * (a + b);
    }
    // Lloyd's iteration (each level to the centroid of its cell) converges linearly
    // with a rate near 1 - O(1/n^2), too slowly for 7-8 bit quantisers; its fixed point
    // F(l) = l - centroid(l) = 0 is solved by Newton's method instead. Cell i's centroid
    // c_i = M1_i / M0_i over [a_i, b_i] moves with its edges as
    //   dc_i/da_i = f(a_i) (c_i - a_i) / M0_i,   dc_i/db_i = f(b_i) (b_i - c_i) / M0_i,
    // and the inner edges are midpoints of adjacent levels, so the Jacobian of F is
    // tridiagonal. Steps are halved until the levels stay ascending inside the support;
    // Lloyd steps finish the job should Newton stall.
    std::vector<double> a(n), b(n), c(n), m0(n), F(n), lo_d(n), di(n), up_d(n), step(n), nl(n);
    const auto residual = [&](const double* l) {
      double r = 0.0;
      for (int i = 0; i < n; ++i) {
        a[i] = i == 0 ? lo : 0.5 * (l[i - 1] + l[i]);
        b[i] = i == n - 1 ? hi : 0.5 * (l[i] + l[i + 1]);
        double mass, mom;
        cell(a[i], b[i], &mass, &mom);
        m0[i] = mass;
        c[i] = mass > 0.0 ? mom / mass : l[i];
        F[i] = l[i] - c[i];
        r = fmax(r, fabs(F[i]));
      }
      return r;
    };
    double r = residual(levels);
    for (int it = 0; it < 100 && r > 1e-15; ++it) {
      for (int i = 0; i < n; ++i) {
        const double dca = (i == 0 || m0[i] <= 0.0) ? 0.0 : marginal(kind, d, a[i]) * (c[i] - a[i]) / m0[i];
        const double dcb = (i == n - 1 || m0[i] <= 0.0) ? 0.0 : marginal(kind, d, b[i]) * (b[i] - c[i]) / m0[i];
        lo_d[i] = -0.5 * dca;
        di[i] = 1.0 - 0.5 * (dca + dcb);
        up_d[i] = -0.5 * dcb;
      }
      // Thomas algorithm on (lo_d, di, up_d) step = F
      for (int i = 0; i < n; ++i) step[i] = F[i];
      for (int i = 1; i < n; ++i) {
        const double w = lo_d[i] / di[i - 1];
        di[i] -= w * up_d[i - 1];
        step[i] -= w * step[i - 1];
      }
      step[n - 1] /= di[n - 1];
      for (int i = n - 2; i >= 0; --i) step[i] = (step[i] - up_d[i] * step[i + 1]) / di[i];
      bool moved = false;
      for (double t = 1.0; t > 1e-6; t *= 0.5) {
        bool ok = true;
        for (int i = 0; i < n; ++i) {
          nl[i] = levels[i] - t * step[i];
          ok = ok && std::isfinite(nl[i]) && nl[i] > lo && nl[i] < hi && (i == 0 || nl[i] > nl[i - 1]);
        }
        if (!ok) continue;
        for (int i = 0; i < n; ++i) levels[i] = nl[i];
        moved = true;
        break;
      }
      if (!moved) break;
      r = residual(levels);
    }
    for (int it = 0; it < 200000 && r > 1e-14; ++it) {
      for (int i = 0; i < n; ++i) levels[i] = c[i];
      r = residual(levels);
    }
  }
};

bool tri_desc_ok(const kvq_tri_desc* d) {
  if (!d) return false;
  if (d->head_dim != 64 && d->head_dim != 128) return false;
  // token positions and tile counts are kept in int
  if (d->num_kv_heads == 0 || d->batch == 0 || d->capacity == 0 || d->capacity > kMaxCapacity)
    return false;
  if (d->bits_dir < 1 || d->bits_dir > 6 || d->bits_norm < 1 || d->bits_norm > 6) return false;
  if (d->bits_rest < 1 || d->bits_rest > 8) return false;
  return true;
}

TriGeom geom_of_tri(const kvq_tri_desc* d) {
  return tri_geom((int)d->head_dim, (int)d->bits_dir, (int)d->bits_norm, (int)d->bits_rest);
}

SignMask tri_sign_mask(const kvq_tri_desc* d) {
  // the angle codec's generator, through its public entry point
  int8_t s[128];
  SignMask m;
  memset(&m, 0, sizeof(m));
  kvq_layer_signs(d->seed, d->layer, d->head_dim, s);
  for (uint32_t i = 0; i < d->head_dim; ++i)
    if (s[i] < 0) m.w[i >> 6] |= 1ull << (i & 63);
  return m;
}

int tri_tiles(const kvq_tri_desc* d) { return (int)((d->capacity + kTile - 1) / kTile); }

kvq_status tri_hip(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

TriArgs tri_args(const kvq_tri_desc* d, const double* cb, uint32_t t0, uint32_t ntok) {
  TriArgs a;
  a.g = geom_of_tri(d);
  a.batch = (int)d->batch;
  a.hkv = (int)d->num_kv_heads;
  a.tiles_per_seq = tri_tiles(d);
  a.t0 = (int)t0;
  a.ntok = (int)ntok;
  a.inv_sqrt_d = 1.0 / sqrt((double)d->head_dim);
  a.sign = tri_sign_mask(d);
  a.cb = cb;
  return a;
}

void tri_split_plan(uint32_t units, uint32_t seq_len, int* nsplit, int* tps) {
  const int ntiles = (int)((seq_len + kTile - 1) / kTile);
  int s = (int)((kTriMaxSplits + units - 1) / units);  // never more than kTriMaxSplits
  int max_s = (ntiles + 3) / 4;
  if (max_s < 1) max_s = 1;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  *tps = (ntiles + s - 1) / s;
  *nsplit = (ntiles + *tps - 1) / *tps;
}

size_t tri_align256(size_t v) { return (v + 255) & ~(size_t)255; }

template <int D, int DIRB>
hipError_t tri_attn_split(const TriAttnArgs& a, const uint8_t* cache, hipStream_t s) {
  const dim3 grid((unsigned)a.nsplit, (unsigned)(a.batch * a.hkv));
  if constexpr (DIRB == 4) {
    // 4 + 4 bits of direction, 2 of norm and 3 per leftover (3.5 bits per element at
    // d = 128) compiled with the allocation fixed
    if (a.g.bd == 4 && a.g.bn == 2 && a.g.br == 3) {
      switch (a.group) {
        case 1: hipLaunchKernelGGL((tri_attn_split_kernel<D, 1, 4, 4, 2, 3>), grid, dim3(kTriWaves * 64), 0, s, a, cache); return hipSuccess;
        case 2: hipLaunchKernelGGL((tri_attn_split_kernel<D, 2, 4, 4, 2, 3>), grid, dim3(kTriWaves * 64), 0, s, a, cache); return hipSuccess;
        case 4: hipLaunchKernelGGL((tri_attn_split_kernel<D, 4, 4, 4, 2, 3>), grid, dim3(kTriWaves * 64), 0, s, a, cache); return hipSuccess;
        case 8: hipLaunchKernelGGL((tri_attn_split_kernel<D, 8, 4, 4, 2, 3>), grid, dim3(kTriWaves * 64), 0, s, a, cache); return hipSuccess;
        default: return hipErrorInvalidValue;
      }
    }
  }
  switch (a.group) {
    case 1: hipLaunchKernelGGL((tri_attn_split_kernel<D, 1, DIRB>), grid, dim3(kTriWaves * 64), 0, s, a, cache); break;
    case 2: hipLaunchKernelGGL((tri_attn_split_kernel<D, 2, DIRB>), grid, dim3(kTriWaves * 64), 0, s, a, cache); break;
    case 4: hipLaunchKernelGGL((tri_attn_split_kernel<D, 4, DIRB>), grid, dim3(kTriWaves * 64), 0, s, a, cache); break;
    case 8: hipLaunchKernelGGL((tri_attn_split_kernel<D, 8, DIRB>), grid, dim3(kTriWaves * 64), 0, s, a, cache); break;
    default: return hipErrorInvalidValue;
  }
  return hipSuccess;
}

template <int D>
hipError_t tri_attn_launch(const TriAttnArgs& a, const uint8_t* cache, hipStream_t s) {
  // direction tables of up to 4 bits per coordinate take 4 KiB of LDS, 6 bits 64 KiB
  const hipError_t e0 = a.g.bd <= 4 ? tri_attn_split<D, 4>(a, cache, s) : tri_attn_split<D, 6>(a, cache, s);
  if (e0 != hipSuccess) return e0;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.nsplit > kTriMaxSplits) return hipErrorInvalidValue;  // the merge's LDS table
  hipLaunchKernelGGL((tri_attn_merge_kernel<D>), dim3((unsigned)(a.batch * a.hq)), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace
}  // namespace kvq

using namespace kvq;

extern "C" {

uint32_t kvq_tri_record_words(const kvq_tri_desc* d) {
  if (!tri_desc_ok(d)) return 0;
  return (uint32_t)geom_of_tri(d).words;
}

size_t kvq_tri_tile_bytes(const kvq_tri_desc* d) {
  if (!tri_desc_ok(d)) return 0;
  return (size_t)2 * geom_of_tri(d).words * kTile * 4;
}

size_t kvq_tri_cache_bytes(const kvq_tri_desc* d) {
  if (!tri_desc_ok(d)) return 0;
  return (size_t)d->batch * d->num_kv_heads * tri_tiles(d) * kvq_tri_tile_bytes(d);
}

size_t kvq_tri_codebook_doubles(const kvq_tri_desc* d) {
  if (!tri_desc_ok(d)) return 0;
  const TriGeom g = geom_of_tri(d);
  return (size_t)2 * (g.nd + g.nn + g.nr) - 3;
}

kvq_status kvq_tri_codebook(const kvq_tri_desc* d, double* out) {
  if (!tri_desc_ok(d) || !out) return KVQ_ERR_INVALID_ARGUMENT;
  const TriGeom g = geom_of_tri(d);
  const GaussRule gl = gauss_legendre40();
  const LloydMax dir{gl, kOct, g.d, -1.0, 1.0, true};
  const LloydMax nrm{gl, kNorm, g.d, 0.0, 1.0, false};
  const LloydMax rst{gl, kCoord, g.d, -1.0, 1.0, true};
  double* ld = out;
  double* ln = ld + g.nd;
  double* lr = ln + g.nn;
  dir.fit(g.bd, ld);
  nrm.fit(g.bn, ln);
  rst.fit(g.br, lr);
  double* b = lr + g.nr;
  for (int i = 0; i + 1 < g.nd; ++i) *b++ = 0.5 * (ld[i] + ld[i + 1]);
  for (int i = 0; i + 1 < g.nn; ++i) *b++ = 0.5 * (ln[i] + ln[i + 1]);
  for (int i = 0; i + 1 < g.nr; ++i) *b++ = 0.5 * (lr[i] + lr[i + 1]);
  return KVQ_OK;
}

kvq_status kvq_tri_encode(const kvq_tri_desc* d, void* cache, const double* cb, const void* k,
                          const void* v, kvq_dtype in_dtype, int64_t sb, int64_t st, int64_t sh,
                          uint32_t t0, uint32_t ntok, void* stream) {
  if (!tri_desc_ok(d)) return KVQ_ERR_INVALID_ARGUMENT;
  if (in_dtype != KVQ_F16 && in_dtype != KVQ_F32) return KVQ_ERR_INVALID_ARGUMENT;
  if ((uint64_t)t0 + ntok > d->capacity) return KVQ_ERR_CAPACITY;
  if (ntok == 0) return KVQ_OK;
  if (!cache || !cb || !k || !v || ((uintptr_t)cache % 16) || ((uintptr_t)cb % 8))
    return KVQ_ERR_INVALID_ARGUMENT;
  const size_t esz = in_dtype == KVQ_F32 ? 4 : 2;
  if (((uintptr_t)k % (2 * esz)) || ((uintptr_t)v % (2 * esz))) return KVQ_ERR_INVALID_ARGUMENT;
  if ((sb & 1) || (st & 1) || (sh & 1) || sb < 0 || st < 0 || sh < 0) return KVQ_ERR_INVALID_ARGUMENT;
  const TriArgs a = tri_args(d, cb, t0, ntok);
  // one wave per (batch, kv head, touched tile), sixteen token-heads per step
  const long long tiles = (long long)(t0 + ntok - 1) / kTile - t0 / kTile + 1;
  const long long tile_tasks = (long long)d->batch * d->num_kv_heads * tiles;
  // a whole tile per wave where there are enough tiles for 16 waves per compute unit,
  // else a quarter tile per wave
  const int spw = tile_tasks >= 4096 ? 4 : 1;
  const long long tasks = tile_tasks * (4 / spw);
  if (tasks > 0x7fffffffLL) return KVQ_ERR_INVALID_ARGUMENT;
  const dim3 rgrid((unsigned)((tasks + kTriRowWaves - 1) / kTriRowWaves)), rblock(kTriRowWaves * 64);
  hipStream_t s = (hipStream_t)stream;
  const bool f32 = in_dtype == KVQ_F32;
  const bool b423 = d->bits_dir == 4 && d->bits_norm == 2 && d->bits_rest == 3;
#define KVQ_TRI_ENC(DD, F, A, B, C)                                                              \
  hipLaunchKernelGGL((tri_encode_rows_kernel<DD, F, A, B, C>), rgrid, rblock, 0, s, a,           \
                     (uint8_t*)cache, k, v, sb, st, sh, spw)
  if (d->head_dim == 64) {
    if (f32 && b423) KVQ_TRI_ENC(64, true, 4, 2, 3);
    else if (f32) KVQ_TRI_ENC(64, true, 0, 0, 0);
    else if (b423) KVQ_TRI_ENC(64, false, 4, 2, 3);
    else KVQ_TRI_ENC(64, false, 0, 0, 0);
  } else {
    if (f32 && b423) KVQ_TRI_ENC(128, true, 4, 2, 3);
    else if (f32) KVQ_TRI_ENC(128, true, 0, 0, 0);
    else if (b423) KVQ_TRI_ENC(128, false, 4, 2, 3);
    else KVQ_TRI_ENC(128, false, 0, 0, 0);
  }
#undef KVQ_TRI_ENC
  return tri_hip(hipGetLastError());
}

kvq_status kvq_tri_decode(const kvq_tri_desc* d, const void* cache, const double* cb, void* k_out,
                          void* v_out, kvq_dtype out_dtype, uint32_t t0, uint32_t ntok,
                          void* stream) {
  if (!tri_desc_ok(d)) return KVQ_ERR_INVALID_ARGUMENT;
  if (out_dtype != KVQ_F16 && out_dtype != KVQ_F32) return KVQ_ERR_INVALID_ARGUMENT;
  if ((uint64_t)t0 + ntok > d->capacity) return KVQ_ERR_CAPACITY;
  if (ntok == 0) return KVQ_OK;
  if (!cache || !cb || !k_out || !v_out || ((uintptr_t)cache % 16) || ((uintptr_t)cb % 8))
    return KVQ_ERR_INVALID_ARGUMENT;
  if (((uintptr_t)k_out % 8) || ((uintptr_t)v_out % 8)) return KVQ_ERR_INVALID_ARGUMENT;
  const TriArgs a = tri_args(d, cb, t0, ntok);
  const long long items = (long long)d->batch * ntok * d->num_kv_heads;
  if (items > 0xFFFFFF00LL) return KVQ_ERR_INVALID_ARGUMENT;
  const dim3 grid((unsigned)((items + 3) / 4)), block(256);
  hipStream_t s = (hipStream_t)stream;
  const uint8_t* c = (const uint8_t*)cache;
  const bool f32 = out_dtype == KVQ_F32;
  if (d->head_dim == 64) {
    if (f32) hipLaunchKernelGGL((tri_decode_kernel<64, true>), grid, block, 0, s, a, c, k_out, v_out);
    else hipLaunchKernelGGL((tri_decode_kernel<64, false>), grid, block, 0, s, a, c, k_out, v_out);
  } else {
    if (f32) hipLaunchKernelGGL((tri_decode_kernel<128, true>), grid, block, 0, s, a, c, k_out, v_out);
    else hipLaunchKernelGGL((tri_decode_kernel<128, false>), grid, block, 0, s, a, c, k_out, v_out);
  }
  return tri_hip(hipGetLastError());
}

size_t kvq_tri_attn_workspace_bytes(const kvq_tri_desc* d, uint32_t hq, uint32_t seq_len) {
  if (!tri_desc_ok(d) || hq == 0 || hq % d->num_kv_heads || seq_len == 0 || seq_len > d->capacity)
    return 0;
  const uint32_t g = hq / d->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return 0;
  if (geom_of_tri(d).words > 32) return 0;
  int nsplit, tps;
  tri_split_plan(d->batch * d->num_kv_heads, seq_len, &nsplit, &tps);
  const size_t rows = (size_t)d->batch * hq * nsplit;
  return tri_align256(rows * 2 * sizeof(float)) + tri_align256(rows * d->head_dim * sizeof(float));
}

kvq_status kvq_tri_attn_decode(const kvq_tri_desc* d, const void* cache, const double* cb,
                               const void* q, kvq_dtype q_dtype, uint32_t hq, uint32_t seq_len,
                               float scale, void* out, kvq_dtype out_dtype, void* ws,
                               size_t ws_bytes, void* stream) {
  if (!tri_desc_ok(d)) return KVQ_ERR_INVALID_ARGUMENT;
  if (hq == 0 || hq % d->num_kv_heads || seq_len == 0) return KVQ_ERR_INVALID_ARGUMENT;
  if (seq_len > d->capacity) return KVQ_ERR_CAPACITY;
  const uint32_t g = hq / d->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return KVQ_ERR_UNSUPPORTED;
  if (geom_of_tri(d).words > 32) return KVQ_ERR_UNSUPPORTED;
  const size_t need = kvq_tri_attn_workspace_bytes(d, hq, seq_len);
  if (!ws || ((uintptr_t)ws & 255) || ws_bytes < need) return KVQ_ERR_WORKSPACE;
  if (!cache || !cb || !q || !out || ((uintptr_t)cache % 16) || ((uintptr_t)cb % 8))
    return KVQ_ERR_INVALID_ARGUMENT;
  if ((q_dtype != KVQ_F16 && q_dtype != KVQ_F32) || (out_dtype != KVQ_F16 && out_dtype != KVQ_F32))
    return KVQ_ERR_INVALID_ARGUMENT;
  if ((uintptr_t)q % (q_dtype == KVQ_F32 ? 8 : 4)) return KVQ_ERR_INVALID_ARGUMENT;
  if ((uintptr_t)out % (out_dtype == KVQ_F32 ? 8 : 4)) return KVQ_ERR_INVALID_ARGUMENT;
  TriAttnArgs a;
  a.g = geom_of_tri(d);
  a.batch = (int)d->batch;
  a.hkv = (int)d->num_kv_heads;
  a.hq = (int)hq;
  a.group = (int)g;
  a.tiles_per_seq = tri_tiles(d);
  a.seq_len = (int)seq_len;
  a.ntiles = (int)((seq_len + kTile - 1) / kTile);
  tri_split_plan(d->batch * d->num_kv_heads, seq_len, &a.nsplit, &a.tiles_per_split);
  a.q_f32 = q_dtype == KVQ_F32;
  a.out_f32 = out_dtype == KVQ_F32;
  const double sc = scale > 0.0f ? (double)scale : 1.0 / sqrt((double)d->head_dim);
  a.q_scale = (float)(sc * 1.4426950408889634);
  a.inv_sqrt_d = (float)(1.0 / sqrt((double)d->head_dim));
  a.sign = tri_sign_mask(d);
  a.cb = cb;
  a.q = q;
  a.out = out;
  const size_t rows = (size_t)d->batch * hq * a.nsplit;
  a.part_ml = (float*)ws;
  a.part_acc = (float*)((char*)ws + tri_align256(rows * 2 * sizeof(float)));
  const hipError_t e = d->head_dim == 64 ? tri_attn_launch<64>(a, (const uint8_t*)cache, (hipStream_t)stream)
                                          : tri_attn_launch<128>(a, (const uint8_t*)cache, (hipStream_t)stream);
  return tri_hip(e);
}

}  // extern "C"
