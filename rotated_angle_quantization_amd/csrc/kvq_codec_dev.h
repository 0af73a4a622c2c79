// Device helpers of the encoder shared by the encode, append and fused append-attention
// kernels: exact fp16 rounding of parameters, the fp32-estimate / binary64-fallback code
// decisions, cross-lane transform stages, and the one-token append.
//
// Method: "TurboAngle: Near-Lossless KV Cache Compression via Uniform Angle
// Quantization" (arXiv 2603.27467), Abstract (angles of rotated pairs quantised
// uniformly; 8-bit linear key radii, 4-bit log value radii, fp16 per-vector parameters).
#pragma once

#include <hip/hip_fp16.h>
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr double kFp16Max = 65504.0;
constexpr double kFp16MinNormal = 6.103515625e-05;  // 2^-14
constexpr double kFp16Subnormal = 5.9604644775390625e-08;  // 2^-24

// Nearest fp16 value of a non-negative x <= 65504, ties to even, computed exactly in
// binary64: the fp16 spacing at x is 2^(e-10) (2^-24 below the normal range), so
// rint(x / q) * q rounds to 11 significant bits with no double rounding.
__device__ __forceinline__ double pow2(int e) {  // 2^e for -1022 <= e <= 1023
  return __longlong_as_double((long long)(e + 1023) << 52);
}
__device__ __forceinline__ double fp16_round_pos(double x) {
  if (x == 0.0) return 0.0;
  // 2^(e-10) with x in [2^e, 2^(e+1)); frexp's exponent is e + 1
  const int e = x < kFp16MinNormal ? -14 : __builtin_amdgcn_frexp_exp(x) - 1;
  return rint(x * pow2(10 - e)) * pow2(e - 10);  // scaling by powers of two is exact
}

__device__ __forceinline__ uint16_t fp16_bits(double exact_fp16_value) {
  return __half_as_ushort(__float2half_rn((float)exact_fp16_value));
}

// atan(z) on [0, 1]: odd polynomial z * sum_k c_k z^2k, the minimax fit to atan on a
// dense grid (Lawson's reweighted least squares) rounded to fp32, as printed by
// fit_atan01.py beside this file: maximum error 2.5e-7 rad in exact arithmetic, 3.3e-7
// rad evaluated in fp32 as below.
__device__ __forceinline__ float atan01(float z) {
  const float s = z * z;
  float p = 0.006811870262026787f;
  p = fmaf(p, s, -0.0336044542491436f);
  p = fmaf(p, s, 0.07962393760681152f);
  p = fmaf(p, s, -0.13233356177806854f);
  p = fmaf(p, s, 0.1980782002210617f);
  p = fmaf(p, s, -0.3331736922264099f);
  p = fmaf(p, s, 0.9999961256980896f);
  return p * z;
}

// Angle of a nonzero pair in fp32, by octant reduction: |error| <= 3.3e-7 (polynomial)
// + 1.2e-7 (z = min/max through the reciprocal) + 6e-8 (rounding the pair to fp32)
// + 2.4e-7 (the two reflections about pi/2 and pi) < 8e-7 rad. The reflections and the
// sign use the fp32 values' sign bits (exact: rounding keeps the sign).
__device__ __forceinline__ float angle_f32(float a, float b) {
  const float ax = fabsf(a), ay = fabsf(b);
  const float mx = fmaxf(ax, ay), mn = fminf(ax, ay);
  const float p = atan01(mn * __builtin_amdgcn_rcpf(mx));
  float t = ay > ax ? 1.5707963267948966f - p : p;
  t = a < 0.f ? 3.141592653589793f - t : t;
  return __builtin_copysignf(t, b);
}

// Angle code: nearest of n centres 2 pi c / n, i.e. floor(theta n / (2 pi) + 1/2) mod n;
// 0 for a zero pair. The fp32 estimate theta32 (error < 8e-7 rad) gives the position
// x = theta32 n / (2 pi) in bins, the centre cf = rint(x) and the residual x - cf (exact);
// x carries the estimate's error times n / (2 pi) plus < 2^-24 n (the fp32 factor and
// product). When |x - cf| exceeds 1/2 - kAngleMargin n / (2 pi) (the trust bound, from
// angle_trust), i.e. the pair may lie within kAngleMargin rad of a bin edge, it is
// compared in binary64 with the edge's direction (bedge[k] = (cos, sin) of
// (k + 1/2) 2 pi / n): on or past the edge means the upper bin, as the floor above gives
// at an exact half. The error bound assumes the pair rounds to normal fp32 numbers well
// inside the range, where the reciprocal is exact to an ulp: a pair whose larger
// component lies outside [2^-60, 2^60] (tiny vectors, whose fp32 values are subnormal or
// zero, or fp32 inputs near the top of the range, which overflow fp32 after rotation) is
// first scaled by a power of two in binary64 (exact, and the angle is unchanged) and
// estimated again; a non-finite estimate also fails the margin test. The estimate runs
// for zero pairs too and the zero test only selects the result, so no branch surrounds
// the common path. kWide = false states that the pair comes from fp16 inputs: its
// nonzero components are then sums of multiples of 2^-24 scaled by 1/sqrt(d) <= 1 and
// bounded by 65504 sqrt(d), inside [2^-60, 2^60] for every d the library serves, so the
// range test is skipped (the exact branch still scales, which then changes nothing).
constexpr float kAngleMargin = 8e-6f;  // rad, > 6x the estimate's worst-case error
constexpr float kAngleRangeLo = 0x1p-60f, kAngleRangeHi = 0x1p60f;
// The bound on |x - cf| below which the estimate's code is kept (n / (2 pi) in fp32 given).
__device__ __forceinline__ float angle_trust(float bins_per_rad_f) {
  return 0.5f - kAngleMargin * bins_per_rad_f;
}
template <bool kWide = true, class Edge>  // edge(k) = (cos, sin) of (k + 1/2) 2 pi / n
__device__ __forceinline__ int angle_code(double a, double b, bool zero, int n,
                                          float bins_per_rad_f, float trust,
                                          const Edge& edge) {
  float af = (float)a, bf = (float)b;
  float x = angle_f32(af, bf) * bins_per_rad_f;  // position in bins
  float cf = rintf(x);
  float res = x - cf;  // from the estimated centre, in bins
  int c = (int)cf;  // in [-n/2, n/2]
  const float mxf = fmaxf(fabsf(af), fabsf(bf));
  const bool in_range = !kWide || (mxf >= kAngleRangeLo && mxf <= kAngleRangeHi);
  const bool near_edge = !(fabsf(res) <= trust);  // NaN: near
  if (__builtin_expect((near_edge || !in_range) && !zero, 0)) {
    if (!in_range) {
      // larger component scaled into [1/2, 1): exact in binary64
      const double sc = pow2(-__builtin_amdgcn_frexp_exp(fmax(fabs(a), fabs(b))));
      af = (float)(a * sc);
      bf = (float)(b * sc);
      x = angle_f32(af, bf) * bins_per_rad_f;
      cf = rintf(x);
      res = x - cf;
      c = (int)cf;
    }
    const int k = res > 0.f ? c : c - 1;  // edge between centres k and k + 1
    const int kk = k < 0 ? k + n : (k >= n ? k - n : k);
    const double2 e = edge(kk);
    // the sign of the cross product with the edge direction is that of the pair's
    // angle relative to the edge (exact scaling leaves it unchanged)
    c = fma(e.x, b, -e.y * a) >= 0.0 ? k + 1 : k;
  }
  // c is in [-n/2 - 1, n/2 + 1]: wrap into [0, n) as min(c + n, c) in unsigned terms
  const unsigned cu = (unsigned)(c + n);
  const unsigned wrapped = min(cu, cu - (unsigned)n);
  return zero ? 0 : (int)wrapped;
}

// Bin edge k of an n-bin codebook, (cos, sin) of (k + 1/2) 2 pi / n in binary64; the
// encode kernel tabulates these values, the append kernel computes them when needed.
__device__ __forceinline__ double2 bin_edge(int k, int n) {
  double sn, co;
  sincospi((2.0 * k + 1.0) / n, &sn, &co);
  return make_double2(co, sn);
}

// Key scale and radius level: s = fp16(max r); level = floor(255 r / s + 1/2). Estimate
// in fp32: hardware sqrt (<= 2 ulp) of the rounded r^2, times 255/s: relative error
// < 4e-7, i.e. < 1.1e-4 levels with the final rounding. Within 5e-4 of a half-integer
// the level is decided by comparing r^2 with ((m - 1/2) s / 255)^2 in binary64.
struct KeyScale {
  double s, s_255;
  float sc255;
};
__device__ __forceinline__ KeyScale key_scale(double max_r2) {
  KeyScale k;
  k.s = fp16_round_pos(fmin(sqrt(max_r2), kFp16Max));
  k.sc255 = k.s > 0.0 ? 255.0f * __builtin_amdgcn_rcpf((float)k.s) : 0.f;
  k.s_255 = k.s * (1.0 / 255.0);
  return k;
}
// kWide = false (fp16 inputs): r <= |x| <= 65504 sqrt(d), and s is max r rounded to fp16
// (or 65504 past that), so r / s <= sqrt(d) and t < 255 sqrt(d) + 1 needs no cap before
// the conversion.
template <bool kWide = true>
__device__ __forceinline__ int key_level(double r2, const KeyScale& k) {
  int rho = 0;
  if (k.s > 0.0) {
    // capped so that a radius past the fp32 range (fp32 inputs near its top) converts
    // to a level above 255 rather than to an undefined integer
    float t = __builtin_amdgcn_sqrtf((float)r2) * k.sc255 + 0.5f;
    if (kWide) t = fminf(t, 256.f);
    const float m = rintf(t);
    rho = (int)t;  // t >= 1/2: truncation is the floor
    if (__builtin_expect(fabsf(t - m) < 5e-4f, 0)) {
      const double thr = ((double)m - 0.5) * k.s_255;
      rho = r2 >= thr * thr ? (int)m : (int)m - 1;
    }
    rho = min(max(rho, 0), 255);
  }
  return rho;
}

// Value parameters and radius level: s_max = fp16(max r), s_min = fp16(max(min r,
// 2^-14)); level = floor(15 ln(r / s_min) / L + 1/2), L = ln(s_max / s_min). Estimate:
// 7.5 log2f(r^2 / s_min^2) / log2(s_max / s_min) from fp32; its error is bounded by
// (7.5 / L2) (3 * 2^-24 / ln 2 + ulp(|log2|)) plus the rounding of the sum, which the
// margin below covers with a factor of >= 4.
struct ValueScale {
  double smin, smax, smin2;
  bool spread;
  float scale, inv_smin2;
  float trust;  // |frac(t) - 1/2| above this: the estimate's level is trusted
};
__device__ __forceinline__ ValueScale value_scale(double max_r2, double min_r2) {
  ValueScale v;
  v.smax = fp16_round_pos(fmin(sqrt(max_r2), kFp16Max));
  v.smin = fp16_round_pos(fmin(fmax(sqrt(min_r2), kFp16MinNormal), kFp16Max));
  v.spread = v.smax > v.smin;
  v.smin2 = v.smin * v.smin;
  // log2(s_max / s_min) from the fp32 ratio (s_max, s_min are fp16 values, exact in
  // fp32): error < 4e-7 absolute
  const float l2f =
      v.spread ? __log2f((float)v.smax * __builtin_amdgcn_rcpf((float)v.smin)) : 1.f;
  v.scale = 7.5f * __builtin_amdgcn_rcpf(l2f);
  v.inv_smin2 = __builtin_amdgcn_rcpf((float)v.smin2);
  // The margin of value_level below, with |lr| bounded for the whole vector: every
  // radius coded by its estimate lies in [s_min, max r], and max r <= s_max (1 + 2^-11)
  // unless s_max was clipped at 65504, so 0 <= lr <= 2 l2 + 0.0015 up to rounding,
  // below 2 l2 + 1. Radii with lr past 2 l2 + 1 (clipped s_max only) have t >= 15.5 +
  // 7.5 / l2 >= 15.6 (l2 < 48 for fp16 parameters), so both the estimate and the
  // binary64 formula give level 15 after the clamp.
  v.trust = 0.5f - (v.scale * (4e-6f + 1e-6f * (2.f * l2f + 1.f)) + 2e-5f);
  return v;
}
__device__ __forceinline__ int value_level(double r2, const ValueScale& v) {
  int rho = 0;
  if (v.spread && r2 >= v.smin2) {
    // lr = log2(r^2 / s_min^2) <= 2 l2; t = 7.5 lr / l2 + 1/2. With absolute errors
    // <= 7e-7 (lr) and 4e-7 (l2), |dt| <= 7.5 (7e-7 + 2 * 4e-7) / l2 plus ~1e-6 of fp32
    // rounding; the margin below is more than twice that.
    // The margin scale (4e-6 + 1e-6 |lr|) + 2e-5 is applied with |lr| at its bound for
    // the vector (ValueScale::trust): the estimate is trusted only when the fractional
    // part of t lies farther than that from 0 and 1.
    const float lr = __log2f((float)r2 * v.inv_smin2);
    const float t = fminf(lr * v.scale + 0.5f, 16.f);  // capped: r^2 past the fp32 range
    const float fl = floorf(t);
    rho = (int)fl;
    if (__builtin_expect(!(fabsf(t - fl - 0.5f) <= v.trust), 0)) {
      // s_max passes through an empty asm statement here, so the compiler cannot hoist
      // the binary64 log of s_max / s_min (shared by every pair of the vector) out of
      // this rarely taken branch into the common path
      double smax = v.smax;
      asm volatile("" : "+v"(smax));
      rho = (int)floor(15.0 * log(sqrt(r2) / v.smin) / log(smax / v.smin) + 0.5);
    }
    rho = min(max(rho, 0), 15);
  }
  return rho;
}

// Exchange of a double with lane (lane ^ mask) of the wave.
__device__ __forceinline__ double shfl_xor_f64(double v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// Maximum / minimum over the lanes of groups of 2^k consecutive lanes (masks < group).
template <int GROUP>
__device__ __forceinline__ double group_max(double x) {
#pragma unroll
  for (int m = 1; m < GROUP; m <<= 1) x = fmax(x, shfl_xor_f64(x, m));
  return x;
}
template <int GROUP>
__device__ __forceinline__ double group_min(double x) {
#pragma unroll
  for (int m = 1; m < GROUP; m <<= 1) x = fmin(x, shfl_xor_f64(x, m));
  return x;
}

// Transform stage across lanes: the pair held by this lane is combined with the pair of
// lane ^ mask; the lane whose bit is clear keeps low + high, the other low - high (the
// operations of the encode kernel's stages, so the results are the same doubles).
__device__ __forceinline__ void lane_stage(double& y0, double& y1, int lane, int mask) {
  const double p0 = shfl_xor_f64(y0, mask), p1 = shfl_xor_f64(y1, mask);
  if (lane & mask) {
    y0 = p0 - y0;
    y1 = p1 - y1;
  } else {
    y0 = y0 + p0;
    y1 = y1 + p1;
  }
}

// Append of one token of one (sequence, kv head) at slot t of the tile at tp. One wave;
// lane i owns pair i (elements 2i, 2i + 1), so one token's coding is spread over the
// wave. The transform stages run in the encode kernel's order (element strides 1, 2, 4,
// 32, 64, then 8, 16) with the same operations, and the decisions call the same
// functions, so the codes and bytes are those of the encode kernel. For d = 64 the upper
// 32 lanes repeat the lower 32 and do not store. k, v: this row's d elements (fp16, or
// fp32 when f32in). The codes are gathered for packing with lane permutes, so the
// function touches no LDS and orders no memory beyond its own stores. Value words shared
// with other slots are rewritten with only this slot's bits changed, so no other wave
// may write the same tile meanwhile.
template <int D>
__device__ __forceinline__ void append_token(const CodecArgs& a, const TileGeom& g, uint8_t* tp,
                                             int t, const void* k, const void* v, bool f32in,
                                             int lane) {
  constexpr int P = D / 2;
  const int i = lane & (P - 1);  // pair
  const bool store = lane < P;
  const int e0 = 2 * i;
  const uint64_t sw = e0 < 64 ? a.sign.w[0] : a.sign.w[1];  // d <= 128
  const bool neg0 = (sw >> (e0 & 63)) & 1ull, neg1 = (sw >> ((e0 + 1) & 63)) & 1ull;

  // both rows are loaded before either is coded
  float x[2][2];
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const void* src = kv == 0 ? k : v;
    if (f32in) {
      const float2 f = *reinterpret_cast<const float2*>(static_cast<const float*>(src) + e0);
      x[kv][0] = f.x;
      x[kv][1] = f.y;
    } else {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const __half*>(src) + e0);
      x[kv][0] = __half2float(__ushort_as_half((uint16_t)(w & 0xFFFFu)));
      x[kv][1] = __half2float(__ushort_as_half((uint16_t)(w >> 16)));
    }
  }
  const float kbpr = (float)a.k_bins_per_rad, vbpr = (float)a.v_bins_per_rad;
  const float ktrust = angle_trust(kbpr), vtrust = angle_trust(vbpr);

#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    double y0 = (double)(neg0 ? -x[kv][0] : x[kv][0]);
    double y1 = (double)(neg1 ? -x[kv][1] : x[kv][1]);
    {
      const double u = y0, w = y1;
      y0 = u + w;
      y1 = u - w;
    }
    lane_stage(y0, y1, lane, 1);
    lane_stage(y0, y1, lane, 2);
    lane_stage(y0, y1, lane, 16);
    if (D == 128) lane_stage(y0, y1, lane, 32);
    lane_stage(y0, y1, lane, 4);
    lane_stage(y0, y1, lane, 8);
    y0 *= a.inv_sqrt_d;
    y1 *= a.inv_sqrt_d;
    const double r2 = fma(y1, y1, y0 * y0);
    const double mx = group_max<P>(fmax(0.0, r2));

    if (kv == 0) {
      const KeyScale ksc = key_scale(mx);
      const int nk = a.n_k;
      const auto edge = [&](int e) { return bin_edge(e, nk); };
      const int c = angle_code(y0, y1, r2 == 0.0, nk, kbpr, ktrust, edge);
      const int rho = key_level(r2, ksc);
      // key angle words: word w of the slot's bit string holds the pairs with bits in
      // [32w, 32w + 32), at most 32 / 6 + 2 of them; lane w gathers them (every lane
      // takes part in the permutes, lanes past the word count discard the result)
      {
        const int lo = 32 * lane, p0 = lo / a.bk;
        uint32_t acc = 0;
#pragma unroll
        for (int u = 0; u < 7; ++u) {
          const int p = p0 + u;
          const uint32_t cp = (uint32_t)__shfl(c, min(p, P - 1), 64);
          const int s = p * a.bk - lo;
          if (p < P && s < 32) acc |= s >= 0 ? cp << s : cp >> -s;
        }
        if (lane < g.wka) reinterpret_cast<uint32_t*>(tp + g.ka)[lane * kTile + t] = acc;
      }
      // key radius words: bytes of pairs 4w .. 4w + 3
      {
        uint32_t acc = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc |= (uint32_t)__shfl(rho, min(4 * lane + u, P - 1), 64) << (8 * u);
        if (lane < g.wkr) reinterpret_cast<uint32_t*>(tp + g.kr)[lane * kTile + t] = acc;
      }
      if (lane == 0) reinterpret_cast<uint16_t*>(tp + g.ks)[t] = fp16_bits(ksc.s);
    } else {
      const double mn = group_min<P>(r2);
      const ValueScale vsc = value_scale(mx, mn);
      const int nv = a.n_v;
      const auto edge = [&](int e) { return bin_edge(e, nv); };
      const uint32_t c = (uint32_t)angle_code(y0, y1, r2 == 0.0, nv, vbpr, vtrust, edge);
      const uint32_t rho = (uint32_t)value_level(r2, vsc);
      if (store) {
        // this slot's bits in pair i's strings; the other slots' bits are kept
        uint32_t* va = reinterpret_cast<uint32_t*>(tp + g.va);
        const int bit = t * a.bv, w0 = bit >> 5, s0 = bit & 31;
        const uint32_t mask = (1u << a.bv) - 1u;
        uint32_t* d0 = va + w0 * P + i;
        *d0 = (*d0 & ~(mask << s0)) | (c << s0);
        if (s0 + a.bv > 32) {
          uint32_t* d1 = va + (w0 + 1) * P + i;
          const int hb = s0 + a.bv - 32;  // bits in the next word
          *d1 = (*d1 & ~((1u << hb) - 1u)) | (c >> (32 - s0));
        }
        uint32_t* vr = reinterpret_cast<uint32_t*>(tp + g.vr) + (t >> 3) * P + i;
        const int ns = 4 * (t & 7);
        *vr = (*vr & ~(0xFu << ns)) | (rho << ns);
      }
      if (lane == 0)
        reinterpret_cast<uint32_t*>(tp + g.vp)[t] =
            (uint32_t)fp16_bits(vsc.smin) | ((uint32_t)fp16_bits(vsc.smax) << 16);
    }
  }
}

}  // namespace
}  // namespace kvq
