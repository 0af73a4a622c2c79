// Encode (append) kernel: x -> sign diagonal -> normalised fast Walsh-Hadamard
// transform -> pairs -> (radius, angle) -> codes -> bit-packed tile planes.
//
// Method: "TurboAngle: Near-Lossless KV Cache Compression via Uniform Angle
// Quantization" (arXiv 2603.27467), Abstract. Readings (bin placement, ties, fp16
// parameters, log-radius floor) are documented with kvq_encode in kvq.h.
//
// Exactness. The transform runs in binary64; for fp16 inputs every partial sum is
// exact there (at most ~40 significant bits), so the rotated pairs equal a float64
// reference's. Each integer decision (angle bin, key and value radius level) is first
// taken from fp32 estimates whose error is bounded; when the estimate lies within that
// bound (times a safety factor) of a decision boundary, the decision is recomputed
// with the binary64 formula. Per-vector fp16 parameters are always formed in
// binary64. So the codes match a float64 reference except where a float64 angle
// itself sits within rounding distance of a bin boundary.
//
// Work split: one 64-lane wave per (batch, kv head, tile of 64 tokens), or, for launches
// with fewer tiles than fill the GPU, one workgroup per tile (a 16-token step per wave);
// a lane owns a quarter of one vector (d/4 elements in interleaved 8-element chunks), so
// 16 tokens are coded per step: the token is the lane's position in its 16-lane row and
// the quarter is the row.
// The transform's first log2(d/4) stages are in-lane; the last two pair the rows
// (quarter bit 0: rows 0 <-> 1 and 2 <-> 3; quarter bit 1: rows 0, 1 <-> 2, 3). Each of
// those is taken on two of the lane's values at once with gfx950's row swaps
// (v_permlane16_swap, v_permlane32_swap): after a swap of values s and s' between
// partner lanes, each lane holds both operands of one butterfly (the lower lane's value
// in the first register, the upper's in the second) and keeps both of its outputs, so
// one swap per 32-bit word and one add or subtract per value replace two lane moves and
// a multiply-add. The lanes' element sets change with it; for d = 128 each lane ends
// with 32 consecutive elements. Per-vector maxima, minima and parameters are reduced
// over the token's four lanes. Codes of the tile are staged in LDS as bytes and then
// packed: key planes one lane per token, value planes one lane per pair, matching the
// layout's word order so every store is a coalesced dword.
#include <hip/hip_fp16.h>

#include "kvq_codec_dev.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

__device__ __forceinline__ bool sign_neg(const SignMask& m, int e) {
  return (m.w[e >> 6] >> (e & 63)) & 1ull;
}

// Maximum or minimum of x over the four rows' lanes at the same row position (the four
// quarters of a token), by lane permutes.
__device__ __forceinline__ double rows_max(double x) {
  x = fmax(x, shfl_xor_f64(x, 16));
  return fmax(x, shfl_xor_f64(x, 32));
}
__device__ __forceinline__ double rows_min(double x) {
  x = fmin(x, shfl_xor_f64(x, 16));
  return fmin(x, shfl_xor_f64(x, 32));
}

// Row-pair butterfly of two doubles x, y held by every lane, between the lanes of rows
// that differ in bit 0 of the row index (ROWS32 false: v_permlane16_swap exchanges odd
// rows of its first operand with even rows of its second) or in bit 1 (ROWS32 true:
// v_permlane32_swap exchanges lanes 32-63 of its first operand with lanes 0-31 of its
// second). After the swap the lower lane holds (own x, partner's x) and the upper lane
// (partner's y, own y), both as (value of the lower lane, value of the upper lane), so
// every lane forms sum and difference in the same way: the lower lane's outputs are
// those of x's butterfly, the upper lane's those of y's.
template <bool ROWS32>
__device__ __forceinline__ void row_butterfly(double& x, double& y) {
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
  const double u = __longlong_as_double((long long)(((uint64_t)hi0 << 32) | lo0));
  const double v = __longlong_as_double((long long)(((uint64_t)hi1 << 32) | lo1));
  x = u + v;
  y = u - v;
}

constexpr int kRow = 68;  // LDS row stride (bytes) of the per-token code staging

// NC codes of width B (one per byte, four per dword in cw) as an LSB-first bit string
// of NC * B / 32 words, word w stored at dst[w * stride].
template <int B, int NC>
__device__ __forceinline__ void store_packed_w(const uint32_t (&cw)[NC / 4], uint32_t* dst,
                                               int stride) {
  if constexpr (B == 8) {
#pragma unroll
    for (int w = 0; w < NC / 4; ++w) dst[w * stride] = cw[w];
  } else {
    uint32_t out[NC * B / 32];
#pragma unroll
    for (int w = 0; w < NC * B / 32; ++w) out[w] = 0u;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const uint32_t c = (cw[i >> 2] >> (8 * (i & 3))) & 0xFFu;
      const int bit = B * i, w = bit >> 5, sh = bit & 31;
      out[w] |= c << sh;
      if (sh + B > 32) out[w + 1] |= c >> (32 - sh);
    }
#pragma unroll
    for (int w = 0; w < NC * B / 32; ++w) dst[w * stride] = out[w];
  }
}

// Same for a runtime width: unrolled kernels for 6, 7 and 8 bits, a loop otherwise.
template <int NC>
__device__ __forceinline__ void store_packed(const uint32_t (&cw)[NC / 4], int bits, uint32_t* dst,
                                             int stride) {
  switch (bits) {
    case 6: store_packed_w<6, NC>(cw, dst, stride); return;
    case 7: store_packed_w<7, NC>(cw, dst, stride); return;
    case 8: store_packed_w<8, NC>(cw, dst, stride); return;
    default: break;
  }
  uint64_t acc = 0;
  int nb = 0, w = 0;
  for (int i = 0; i < NC; ++i) {
    acc |= (uint64_t)((cw[i >> 2] >> (8 * (i & 3))) & 0xFFu) << nb;
    nb += bits;
    if (nb >= 32) {
      dst[w * stride] = (uint32_t)acc;
      acc >>= 32;
      nb -= 32;
      ++w;
    }
  }
}

// Eight 4-bit values held one per byte in lo, hi (values < 16) as one word of nibbles.
__device__ __forceinline__ uint32_t nibbles8(uint32_t lo, uint32_t hi) {
  lo = (lo | (lo >> 4)) & 0x00FF00FFu;
  lo = (lo | (lo >> 8)) & 0x0000FFFFu;
  hi = (hi | (hi >> 4)) & 0x00FF00FFu;
  hi = (hi | (hi >> 8)) & 0x0000FFFFu;
  return lo | (hi << 16);
}

constexpr int kEncWaves = 4;  // waves (tiles) per workgroup, sharing the edge tables

// wg_tile = 0: each wave codes a tile of its own (four per workgroup). wg_tile = 1 (for
// launches with too few tiles to fill the GPU): the four waves of a workgroup code one
// tile together, a 16-token step each, staging into one shared set of code rows, and
// wave 0 packs the tile after the barrier.
template <int D, bool F32IN>
__global__ __launch_bounds__(kEncWaves * 64) void encode_kernel(CodecArgs a, TileGeom g,
                                                    uint8_t* __restrict__ cache,
                                                    const void* __restrict__ kin,
                                                    const void* __restrict__ vin,
                                                    int64_t sb, int64_t st, int64_t sh,
                                                    int wg_tile) {
  constexpr int P = D / 2;    // pairs per vector
  constexpr int E = D / 4;    // elements per lane
  constexpr int PL = E / 2;   // pairs per lane
  constexpr int TPS = 16;     // tokens per step (4 lanes each)
  // code staging: keys [token][pair], values [pair][token] (the order each plane is
  // packed in), one byte per code, rows padded to kRow bytes
  __shared__ uint8_t s_code[kEncWaves][4][kTile][kRow];  // key angle, key radius, value angle, value radius
  __shared__ uint16_t s_ks_all[kEncWaves][kTile];
  __shared__ uint32_t s_vp_all[kEncWaves][kTile];
  __shared__ double2 s_kedge[256], s_vedge[256];  // bin edges (k + 1/2) 2 pi / n

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tq = lane & 15, q = lane >> 4;  // token within the step, quarter of the vector
  for (int k = threadIdx.x; k < 256; k += kEncWaves * 64) {
    s_kedge[k] = bin_edge(k, a.n_k);
    s_vedge[k] = bin_edge(k, a.n_v);
  }
  __syncthreads();
  const int slot = wg_tile ? 0 : wave;  // the staging rows of this wave's tile
  uint8_t(*s_kc)[kRow] = s_code[slot][0];
  uint8_t(*s_kr)[kRow] = s_code[slot][1];
  uint8_t(*s_vc)[kRow] = s_code[slot][2];
  uint8_t(*s_vr)[kRow] = s_code[slot][3];
  uint16_t* s_ks = s_ks_all[slot];
  uint32_t* s_vp = s_vp_all[slot];
  // one tile per wave (or per workgroup); waves past the last tile do no work (but take
  // the barrier)
  const int task = wg_tile ? (int)blockIdx.x : (int)blockIdx.x * kEncWaves + wave;
  const int ntasks = a.batch * a.hkv * a.tiles_touched;
  const bool live = task < ntasks;
  const int tile_rel = task % a.tiles_touched;
  const int bh = live ? task / a.tiles_touched : 0;
  const int b = bh / a.hkv, h = bh % a.hkv;
  const int tile = a.tile_lo + tile_rel;
  const int tok_base = tile * kTile;
  // a tile the page table maps to no page is not written
  const long long toff = live ? tile_offset(a.pg, b, h, a.hkv, a.tiles_per_seq, tile, g.bytes) : -1;
  const int j_lo = max(a.t0 - tok_base, 0);
  const int j_hi = toff >= 0 ? min(a.t0 + a.ntok - tok_base, kTile) : j_lo;
  // the slots this wave codes: the tile's range, or its step of it (possibly none)
  const int js = wg_tile ? max(j_lo, TPS * wave) : j_lo;
  const int je = wg_tile ? max(js, min(j_hi, TPS * wave + TPS)) : j_hi;

  // The token's lane in row q owns the 8-element chunks m*4 + q (elements
  // 32m + 8q + r, r < 8) in local slots 8m + r: the transform's in-lane stages are the
  // element strides 1, 2, 4 and 32, 64; strides 8 and 16 are the row swaps. Local
  // bit 8m + r of sbits is the sign of element 32m + 8q + r; for fp16 input the per-pair
  // xor masks flip the fp16 sign bits (bits 15 and 31 of a packed pair).
  uint32_t sbits = 0;
#pragma unroll
  for (int m = 0; m < E / 8; ++m)
    sbits |= (uint32_t)((a.sign.w[(32 * m + 8 * q) >> 6] >> ((32 * m + 8 * q) & 63)) & 0xFFu) << (8 * m);
  uint32_t hmask[PL];
#pragma unroll
  for (int k = 0; k < PL; ++k)
    hmask[k] = (((sbits >> (2 * k)) & 1u) << 15) | (((sbits >> (2 * k + 1)) & 1u) << 31);
  const float kbpr = (float)a.k_bins_per_rad, vbpr = (float)a.v_bins_per_rad;  // n / (2 pi)
  const float ktrust = angle_trust(kbpr), vtrust = angle_trust(vbpr);

  // Element offset of this lane's part of the row of step jb; lanes past the range
  // read the last valid row and discard it.
  auto row_offset = [&](int jb) {
    const int jr = min(jb + tq, je - 1);
    return (int64_t)b * sb + (int64_t)(tok_base + jr - a.t0) * st + (int64_t)h * sh + 8 * q;
  };
  // fp16 input: one buffer per plane; a plane's words of the next step are requested as
  // soon as this step's have been widened, so they load while the rest is coded
  uint32_t raw[2][PL];
  auto load_raw = [&](int kv, int jb) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(
        static_cast<const __half*>(kv == 0 ? kin : vin) + row_offset(jb));
#pragma unroll
    for (int k = 0; k < PL; ++k) raw[kv][k] = p[16 * (k >> 2) + (k & 3)];
  };
  if (!F32IN && js < je) {
    load_raw(0, js);
    load_raw(1, js);
  }

  for (int jb = js; jb < je; jb += TPS) {
    const int j = jb + tq;
    const bool act = j < je;
    const int64_t row_off = row_offset(jb);
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      const void* src = kv == 0 ? kin : vin;
      // load, apply the sign diagonal, widen to binary64
      double y[E];
      if (F32IN) {
        const float* p = static_cast<const float*>(src) + row_off;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          float f = p[32 * (e >> 3) + (e & 7)];
          if (!act) f = 0.f;
          if ((sbits >> e) & 1u) f = -f;
          y[e] = (double)f;
        }
      } else {
#pragma unroll
        for (int k = 0; k < PL; ++k) {
          const uint32_t w = (act ? raw[kv][k] : 0u) ^ hmask[k];
          y[2 * k] = (double)__half2float(__ushort_as_half((uint16_t)(w & 0xFFFFu)));
          y[2 * k + 1] = (double)__half2float(__ushort_as_half((uint16_t)(w >> 16)));
        }
        // unconditional: past the range the clamped row is re-read (just loaded, so
        // a cache hit), and a conditional load would make the buffer a copy
        load_raw(kv, jb + TPS);
      }
      // Walsh-Hadamard: in-lane stages, then the two row stages
#pragma unroll
      for (int hs = 1; hs < E; hs <<= 1) {
#pragma unroll
        for (int i = 0; i < E; ++i) {
          if (i & hs) continue;
          const double u = y[i], v = y[i + hs];
          y[i] = u + v;
          y[i + hs] = u - v;
        }
      }
      // Quarter bit 0 (element stride 8): local slots s and s + 8 (chunk bit 0). After
      // it, slot 8 (2 m1 + c) + r of lane (q1, q0) holds element
      // 32 (2 m1 + q0) + 8 (2 q1 + c) + r.
#pragma unroll
      for (int i = 0; i < E; ++i)
        if (!(i & 8)) row_butterfly<false>(y[i], y[i + 8]);
      // Quarter bit 1 (element stride 16). d = 128: slots s and s + 16 (m1); after it
      // slot s holds element 32 q + s. d = 64 (m1 = 0): slots s and s + 8 (c); after it
      // slot 8 c + r holds element 32 q0 + 16 c + 8 q1 + r.
#pragma unroll
      for (int i = 0; i < E; ++i) {
        constexpr int kPart = E > 16 ? 16 : 8;
        if (!(i & kPart)) row_butterfly<true>(y[i], y[i + kPart]);
      }
#pragma unroll
      for (int i = 0; i < E; ++i) y[i] *= a.inv_sqrt_d;

      double r2[PL];
      double mx = 0.0, mn = INFINITY;
#pragma unroll
      for (int k = 0; k < PL; ++k) {
        r2[k] = fma(y[2 * k + 1], y[2 * k + 1], y[2 * k] * y[2 * k]);
        mx = fmax(mx, r2[k]);
        mn = fmin(mn, r2[k]);
      }
      mx = rows_max(mx);

      uint8_t cc[PL], rr[PL];
      if (kv == 0) {
        const KeyScale ksc = key_scale(mx);
        const auto edge = [&](int e) { return s_kedge[e]; };
#pragma unroll
        for (int k = 0; k < PL; ++k) {
          cc[k] = (uint8_t)angle_code<F32IN>(y[2 * k], y[2 * k + 1], r2[k] == 0.0, a.n_k, kbpr,
                                             ktrust, edge);
          rr[k] = (uint8_t)key_level<F32IN>(r2[k], ksc);
        }
        if (act && q == 0) s_ks[j] = fp16_bits(ksc.s);
      } else {
        mn = rows_min(mn);
        const ValueScale vsc = value_scale(mx, mn);
        const auto edge = [&](int e) { return s_vedge[e]; };
#pragma unroll
        for (int k = 0; k < PL; ++k) {
          cc[k] = (uint8_t)angle_code<F32IN>(y[2 * k], y[2 * k + 1], r2[k] == 0.0, a.n_v, vbpr,
                                             vtrust, edge);
          rr[k] = (uint8_t)value_level(r2[k], vsc);
        }
        if (act && q == 0)
          s_vp[j] = (uint32_t)fp16_bits(vsc.smin) | ((uint32_t)fp16_bits(vsc.smax) << 16);
      }
      if (act) {
        // local pair k (slots 2k, 2k + 1) of the vector: 16 q + k for d = 128,
        // 16 q0 + 8 (k / 4) + 4 q1 + k % 4 for d = 64 (the element maps above)
#pragma unroll
        for (int k = 0; k < PL; ++k) {
          const int i = D == 128 ? 16 * q + k : 16 * (q & 1) + 8 * (k >> 2) + 4 * (q >> 1) + (k & 3);
          if (kv == 0) {
            s_kc[j][i] = cc[k];
            s_kr[j][i] = rr[k];
          } else {
            s_vc[i][j] = cc[k];
            s_vr[i][j] = rr[k];
          }
        }
      }
    }
  }
  __syncthreads();
  if (wg_tile && wave != 0) return;  // no barrier follows

  uint8_t* tp = cache + (toff >= 0 ? toff : 0);

  // Key planes and per-token parameters: one lane per token slot; slots outside the
  // range are not written (their words belong to them alone).
  {
    const int t = lane;
    if (t >= j_lo && t < j_hi) {
      uint32_t cw[P / 4], rw[P / 4];  // the token's codes, four per dword
      const uint32_t* crow = reinterpret_cast<const uint32_t*>(s_kc[t]);
      const uint32_t* rrow = reinterpret_cast<const uint32_t*>(s_kr[t]);
#pragma unroll
      for (int w = 0; w < P / 4; ++w) {
        cw[w] = crow[w];
        rw[w] = rrow[w];
      }
      uint32_t* ka = reinterpret_cast<uint32_t*>(tp + g.ka);
      store_packed<P>(cw, a.bk, ka + t, kTile);
      uint32_t* kr = reinterpret_cast<uint32_t*>(tp + g.kr);
#pragma unroll
      for (int w = 0; w < P / 4; ++w) kr[w * kTile + t] = rw[w];
      reinterpret_cast<uint16_t*>(tp + g.ks)[t] = s_ks[t];
      reinterpret_cast<uint32_t*>(tp + g.vp)[t] = s_vp[t];
    }
  }

  // Value planes: one lane per pair. A whole tile is packed straight from the pair's
  // staged row; for a partial tile, a word shared with slots outside the range is
  // merged with the bits already stored (this wave owns the whole tile here).
  if (lane < P) {
    const int i = lane;
    uint32_t* va = reinterpret_cast<uint32_t*>(tp + g.va);
    uint32_t* vrw = reinterpret_cast<uint32_t*>(tp + g.vr);
    if (j_lo == 0 && j_hi == kTile) {
      uint32_t cw[kTile / 4], rw[kTile / 4];
      const uint32_t* crow = reinterpret_cast<const uint32_t*>(s_vc[i]);
      const uint32_t* rrow = reinterpret_cast<const uint32_t*>(s_vr[i]);
#pragma unroll
      for (int w = 0; w < kTile / 4; ++w) {
        cw[w] = crow[w];
        rw[w] = rrow[w];
      }
      store_packed<kTile>(cw, a.bv, va + i, P);
      // radius nibbles: 8 tokens per word (bytes hold values < 16)
#pragma unroll
      for (int w8 = 0; w8 < 8; ++w8) vrw[w8 * P + i] = nibbles8(rw[2 * w8], rw[2 * w8 + 1]);
    } else {
      uint64_t acc = 0, macc = 0;
      int nb = 0, w = 0;
      const uint64_t cmask = (1ull << a.bv) - 1;
      for (int t = 0; t < kTile; ++t) {
        const bool in = t >= j_lo && t < j_hi;
        acc |= (uint64_t)(in ? s_vc[i][t] : 0) << nb;
        macc |= (in ? cmask : 0ull) << nb;
        nb += a.bv;
        if (nb >= 32) {
          uint32_t* dst = va + w * P + i;
          const uint32_t mk = (uint32_t)macc;
          if (mk == 0xffffffffu)
            *dst = (uint32_t)acc;
          else if (mk)
            *dst = (*dst & ~mk) | ((uint32_t)acc & mk);
          acc >>= 32;
          macc >>= 32;
          nb -= 32;
          ++w;
        }
      }
      for (int w8 = 0; w8 < 8; ++w8) {
        uint32_t word = 0, mk = 0;
        for (int q = 0; q < 8; ++q) {
          const int t = w8 * 8 + q;
          if (t >= j_lo && t < j_hi) {
            word |= (uint32_t)s_vr[i][t] << (4 * q);
            mk |= 0xFu << (4 * q);
          }
        }
        uint32_t* dst = vrw + w8 * P + i;
        if (mk == 0xffffffffu)
          *dst = word;
        else if (mk)
          *dst = (*dst & ~mk) | word;
      }
    }
  }
}

// Append: one token per sequence, each at its own slot (positions[b]). One wave per
// (batch, kv head) runs the one-token append, so a decode step waits for this kernel's
// latency, not its throughput.
template <int D, bool F32IN>
__global__ __launch_bounds__(64) void append_kernel(CodecArgs a, TileGeom g,
                                                    uint8_t* __restrict__ cache,
                                                    const void* __restrict__ kin,
                                                    const void* __restrict__ vin, int64_t sb,
                                                    int64_t sh) {
  const int lane = threadIdx.x;
  const int bh = blockIdx.x, b = bh / a.hkv, h = bh % a.hkv;
  const unsigned pos = a.positions[b];
  if (pos >= (unsigned)a.capacity) return;  // nothing to write for this sequence
  const int tile = (int)pos / kTile, t = (int)pos % kTile;
  const long long toff = tile_offset(a.pg, b, h, a.hkv, a.tiles_per_seq, tile, g.bytes);
  if (toff < 0) return;  // the page table maps this tile to no page
  const int64_t off = (int64_t)b * sb + (int64_t)h * sh;
  const size_t esz = F32IN ? 4 : 2;
  append_token<D>(a, g, cache + toff, t, static_cast<const char*>(kin) + off * esz,
                  static_cast<const char*>(vin) + off * esz, F32IN, lane);
}

}  // namespace

hipError_t launch_append(const CodecArgs& a, int d, TileGeom geom, uint8_t* cache,
                         const void* k, const void* v, bool f32_in, int64_t sb, int64_t sh,
                         hipStream_t stream) {
  const long long blocks = (long long)a.batch * a.hkv;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(64);
  if (d == 64 && f32_in)
    hipLaunchKernelGGL((append_kernel<64, true>), grid, block, 0, stream, a, geom, cache, k, v, sb, sh);
  else if (d == 64)
    hipLaunchKernelGGL((append_kernel<64, false>), grid, block, 0, stream, a, geom, cache, k, v, sb, sh);
  else if (d == 128 && f32_in)
    hipLaunchKernelGGL((append_kernel<128, true>), grid, block, 0, stream, a, geom, cache, k, v, sb, sh);
  else if (d == 128)
    hipLaunchKernelGGL((append_kernel<128, false>), grid, block, 0, stream, a, geom, cache, k, v, sb, sh);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_encode(const CodecArgs& a, int d, TileGeom geom, uint8_t* cache,
                         const void* k, const void* v, bool f32_in, int64_t sb, int64_t st,
                         int64_t sh, hipStream_t stream) {
  const long long blocks = (long long)a.batch * a.hkv * a.tiles_touched;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  // a tile per wave where there are tiles for 16 waves per compute unit, else a tile per
  // workgroup (its four waves a step each)
  const int wg_tile = blocks < 4096 ? 1 : 0;
  const dim3 grid((unsigned)(wg_tile ? blocks : (blocks + kEncWaves - 1) / kEncWaves)),
      block(kEncWaves * 64);
  if (d == 64 && f32_in)
    hipLaunchKernelGGL((encode_kernel<64, true>), grid, block, 0, stream, a, geom, cache, k, v, sb, st, sh, wg_tile);
  else if (d == 64)
    hipLaunchKernelGGL((encode_kernel<64, false>), grid, block, 0, stream, a, geom, cache, k, v, sb, st, sh, wg_tile);
  else if (d == 128 && f32_in)
    hipLaunchKernelGGL((encode_kernel<128, true>), grid, block, 0, stream, a, geom, cache, k, v, sb, st, sh, wg_tile);
  else if (d == 128)
    hipLaunchKernelGGL((encode_kernel<128, false>), grid, block, 0, stream, a, geom, cache, k, v, sb, st, sh, wg_tile);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kvq
