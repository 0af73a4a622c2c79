// Device helpers shared by the decode-attention kernels: sign diagonal, cross-lane
// transform of query and output rows, wave reductions, code fields and tile geometry.
#pragma once

#include <hip/hip_fp16.h>
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

// Sign bit of element e < 128, selecting the word without indexing the kernel-argument
// array by a lane-dependent value (which would turn into a per-lane memory load).
__device__ __forceinline__ bool sign_neg(const SignMask& m, int e) {
  const uint64_t w = e < 64 ? m.w[0] : m.w[1];
  return (w >> (e & 63)) & 1ull;
}

template <int P>
__device__ __forceinline__ void fwht_pairs_f32(float& a, float& b, int p) {
  const float s = a + b, t = a - b;
  a = s;
  b = t;
#pragma unroll
  for (int m = 1; m < P; m <<= 1) {
    const float pa = __shfl_xor(a, m), pb = __shfl_xor(b, m);
    if (p & m) {
      a = pa - a;
      b = pb - b;
    } else {
      a = a + pa;
      b = b + pb;
    }
  }
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// DPP lane moves within rows of 16: xor 1, xor 2 (quad permutes), then the half-row
// and row mirrors, which pair lanes whose partial results are already row-uniform.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, 0));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

// Wave-wide max / sum: four DPP steps make each row of 16 uniform, then the four row
// results are combined from scalar registers (readlane), so the result is uniform.
// The maximum runs on integers ordered like the floats (a non-negative float's bits
// compare like a signed integer; a negative one's magnitude bits are flipped, which
// reverses their order and keeps them below zero): the DPP moves then fuse into
// v_max_i32, the row results combine on the scalar unit, and none of the NaN
// canonicalisation that a float maximum of lane-moved values costs is needed (scores
// are never NaN).
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, 0);
}
__device__ __forceinline__ int float_order(int b) { return b ^ ((b >> 31) & 0x7fffffff); }
__device__ __forceinline__ float wave_max(float x) {
  int i = float_order(__float_as_int(x));
  i = max(i, dpp_i<kDppXor1>(i));
  i = max(i, dpp_i<kDppXor2>(i));
  i = max(i, dpp_i<kDppHalfMirror>(i));
  i = max(i, dpp_i<kDppMirror>(i));
  const int r = max(max(__builtin_amdgcn_readlane(i, 0), __builtin_amdgcn_readlane(i, 16)),
                    max(__builtin_amdgcn_readlane(i, 32), __builtin_amdgcn_readlane(i, 48)));
  return __int_as_float(float_order(r));  // the map is its own inverse
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  x += dpp<kDppMirror>(x);
  return (readlane_f(x, 0) + readlane_f(x, 16)) + (readlane_f(x, 32) + readlane_f(x, 48));
}

// 2^x with the hardware instruction; arguments here are either <= 0 (softmax) or
// log2 of fp16-range radii, so no range scaling is needed (underflow gives 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Field `idx` of width B from a register-resident little-endian word string; with
// idx a compile-time constant this is one bit-field extract (or an align + mask when
// the field straddles two words).
template <int B, int N>
__device__ __forceinline__ uint32_t field(const uint32_t (&w)[N], int idx) {
  const int bit = idx * B;
  const int wi = bit >> 5, sh = bit & 31;
  if (sh + B <= 32) return (w[wi] >> sh) & ((1u << B) - 1u);
  return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & ((1u << B) - 1u);
}

template <int D, int BK, int BV>
struct Geo {
  static constexpr int P = D / 2;
  static constexpr int WKA = P * BK / 32;
  static constexpr int WKR = P / 4;
  static constexpr int OFF_KR = kTile * WKA * 4;
  static constexpr int OFF_KS = OFF_KR + kTile * WKR * 4;
  static constexpr int OFF_VA = OFF_KS + 2 * kTile;
  static constexpr int OFF_VR = OFF_VA + P * 2 * BV * 4;
  static constexpr int OFF_VP = OFF_VR + P * 8 * 4;
  static constexpr int BYTES = OFF_VP + 4 * kTile;
};

// Rotated query of one head: lane p < D/2 returns elements 2p, 2p+1 of
// q~ = H diag(sign) q / sqrt(d), times the softmax scale * log2(e) / 255. Split into the
// load and the arithmetic so callers can issue other loads in between.
// Raw bits of elements 2p, 2p+1: two dwords for fp32 input, one (read twice) for fp16,
// with no branch, so the loads can stay in flight while other loads are issued.
__device__ __forceinline__ uint2 load_query_pair(const AttnArgs& a, size_t qoff, int lane) {
  const uint32_t* base = static_cast<const uint32_t*>(a.q);
  const size_t w0 = a.q_f32 ? qoff + 2 * lane : (qoff >> 1) + lane;
  const size_t w1 = a.q_f32 ? w0 + 1 : w0;
  return make_uint2(base[w0], base[w1]);
}

template <int D>
__device__ __forceinline__ float2 rotate_query_pair(const AttnArgs& a, uint2 raw, int lane) {
  constexpr int P = D / 2;
  const int e0 = 2 * lane;
  float x0 = a.q_f32 ? __uint_as_float(raw.x) : __half2float(__ushort_as_half((uint16_t)(raw.x & 0xFFFFu)));
  float x1 = a.q_f32 ? __uint_as_float(raw.y) : __half2float(__ushort_as_half((uint16_t)(raw.x >> 16)));
  if (sign_neg(a.sign, e0)) x0 = -x0;
  if (sign_neg(a.sign, e0 + 1)) x1 = -x1;
  fwht_pairs_f32<P>(x0, x1, lane);
  const float sc = a.inv_sqrt_d * a.q_scale;
  return make_float2(x0 * sc, x1 * sc);
}

template <int D>
__device__ __forceinline__ float2 rotate_query(const AttnArgs& a, size_t qoff, int lane) {
  return rotate_query_pair<D>(a, load_query_pair(a, qoff, lane), lane);
}

// Output of one head from its rotated-domain sum: lane p < D/2 holds elements 2p, 2p+1
// of acc / l; o = sign * H (acc / l) / sqrt(d).
template <int D>
__device__ __forceinline__ void store_output(const AttnArgs& a, size_t ooff, int lane, float a0,
                                             float a1) {
  constexpr int P = D / 2;
  fwht_pairs_f32<P>(a0, a1, lane);
  const int e0 = 2 * lane;
  a0 *= a.inv_sqrt_d;
  a1 *= a.inv_sqrt_d;
  if (sign_neg(a.sign, e0)) a0 = -a0;
  if (sign_neg(a.sign, e0 + 1)) a1 = -a1;
  if (a.out_f32)
    reinterpret_cast<float2*>(a.out)[(ooff + e0) >> 1] = make_float2(a0, a1);
  else
    reinterpret_cast<__half2*>(a.out)[(ooff + e0) >> 1] = __floats2half2_rn(a0, a1);
}

}  // namespace
}  // namespace kvq
