// Decode attention straight from the packed angle codes.
//
// Method: the codec of "TurboAngle: Near-Lossless KV Cache Compression via Uniform
// Angle Quantization" (arXiv 2603.27467), Abstract, consumed without writing a
// dequantised cache (the fused-reconstruction point made in "OCTOPUS: Joint Triplet
// Quantization for KV Cache via Octahedral Parametrization", Why it matters).
//
// The transform R = H diag(sign) / sqrt(d) is orthogonal, so with q~ = R q and
// y^_j the rotated-domain reconstruction of key j,
//   <q, k^_j> = <q~, y^_j> = (s_j / 255) sum_i rho_ji (q~_2i cos t_ji + q~_2i+1 sin t_ji)
// and the output is o = R^T (sum_j p_j z^_j) with z^_j the rotated-domain values:
// one inverse transform per output head instead of one per cached token.
//
// Three launches on one stream:
//   prepare  q~ = R q, pre-multiplied by softmax_scale * log2(e) / 255, into the
//            workspace (read back by the split kernel through scalar loads).
//   split    grid (splits, batch * kv heads), 4 waves per workgroup; each wave
//            streams whole 64-token tiles. Keys: one lane per token, codes unpacked
//            from registers with compile-time bit offsets, cos/sin from an LDS table,
//            q~ from SGPRs. Online softmax per wave (base-2). Values: one lane per
//            pair, probabilities broadcast with readlane, rotated-domain accumulate.
//            Waves merge through LDS; each split writes (max, sum, acc[d]) per head.
//   merge    per (batch, query head): log-sum-exp combine of the splits, divide,
//            inverse transform, sign, store.
#include <hip/hip_fp16.h>
#include <math.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

__device__ __forceinline__ bool sign_neg(const SignMask& m, int e) {
  return (m.w[e >> 6] >> (e & 63)) & 1ull;
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

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

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

// ---------------------------------------------------------------------------- prepare

template <int D>
__global__ __launch_bounds__(64) void attn_prepare_kernel(AttnArgs a, const void* __restrict__ q,
                                                          int f32_q) {
  constexpr int P = D / 2;
  const int bh = blockIdx.x;
  const int lane = threadIdx.x;
  if (lane >= P) return;
  const int e0 = 2 * lane;
  float x0, x1;
  if (f32_q) {
    const float2 v = reinterpret_cast<const float2*>(q)[((size_t)bh * D + e0) >> 1];
    x0 = v.x;
    x1 = v.y;
  } else {
    const __half2 v = reinterpret_cast<const __half2*>(q)[((size_t)bh * D + e0) >> 1];
    x0 = __half2float(__low2half(v));
    x1 = __half2float(__high2half(v));
  }
  if (sign_neg(a.sign, e0)) x0 = -x0;
  if (sign_neg(a.sign, e0 + 1)) x1 = -x1;
  fwht_pairs_f32<P>(x0, x1, lane);
  const float sc = a.inv_sqrt_d * a.q_scale;
  reinterpret_cast<float2*>(a.qrot)[((size_t)bh * D + e0) >> 1] = make_float2(x0 * sc, x1 * sc);
}

// ---------------------------------------------------------------------------- split

template <int D, int G, int BK, int BV>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnArgs a,
                                                         const uint8_t* __restrict__ cache,
                                                         const float* __restrict__ qrot) {
  using GE = Geo<D, BK, BV>;
  constexpr int P = GE::P;
  constexpr int NT = (P == 64) ? 64 : 32;  // value tokens per lane per tile
  constexpr int WVA = NT * BV / 32;        // value-angle words per lane
  constexpr int WVR = NT * 4 / 32;         // value-radius words per lane

  __shared__ float2 lut_k[256], lut_v[256];
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ float s_acc[4][G][D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x, bk = blockIdx.y;  // bk = b * hkv + kv head

  for (int c = tid; c < 256; c += 256) {
    double s, co;
    float2 ek = make_float2(0.f, 0.f), ev = make_float2(0.f, 0.f);
    if (c < a.n_k) {
      sincospi(2.0 * c / a.n_k, &s, &co);
      ek = make_float2((float)co, (float)s);
    }
    if (c < a.n_v) {
      sincospi(2.0 * c / a.n_v, &s, &co);
      ev = make_float2((float)co, (float)s);
    }
    lut_k[c] = ek;
    lut_v[c] = ev;
  }
  __syncthreads();

  const float* qg = qrot + (size_t)bk * G * D;
  const int tile_begin = split * a.tiles_per_split;
  const int tile_end = min(tile_begin + a.tiles_per_split, a.ntiles);
  const uint8_t* base = cache + (size_t)bk * a.tiles_per_seq * GE::BYTES;

  const int vpair = lane % P, vhalf = lane / P;  // value lane -> (pair, token half)

  float m[G], l[G], acc0[G], acc1[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
    acc0[g] = 0.f;
    acc1[g] = 0.f;
  }

  for (int tile = tile_begin + wave; tile < tile_end; tile += 4) {
    const uint8_t* tp = base + (size_t)tile * GE::BYTES;
    const int nvalid = min(a.seq_len - tile * kTile, kTile);

    // ---- keys: lane = token slot
    uint32_t ka[GE::WKA], kr[GE::WKR];
#pragma unroll
    for (int w = 0; w < GE::WKA; ++w) ka[w] = reinterpret_cast<const uint32_t*>(tp)[w * kTile + lane];
#pragma unroll
    for (int w = 0; w < GE::WKR; ++w)
      kr[w] = reinterpret_cast<const uint32_t*>(tp + GE::OFF_KR)[w * kTile + lane];
    const float kscale =
        __half2float(__ushort_as_half(reinterpret_cast<const uint16_t*>(tp + GE::OFF_KS)[lane]));
    // value-plane words for this lane (issued early to overlap with the key math)
    uint32_t va[WVA], vr[WVR];
#pragma unroll
    for (int w = 0; w < WVA; ++w)
      va[w] = reinterpret_cast<const uint32_t*>(tp + GE::OFF_VA)[(w + vhalf * WVA) * P + vpair];
#pragma unroll
    for (int w = 0; w < WVR; ++w)
      vr[w] = reinterpret_cast<const uint32_t*>(tp + GE::OFF_VR)[(w + vhalf * WVR) * P + vpair];
    const uint32_t vpar = reinterpret_cast<const uint32_t*>(tp + GE::OFF_VP)[lane];

    float sc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) sc[g] = 0.f;
    // q~ is read with scalar loads in chunks of CH pairs (2 * G * CH = 64 SGPRs); the
    // empty asm makes the chunk's base opaque so the loads are not hoisted out of the
    // tile loop (512+ live values would spill).
    constexpr int CH = 32 / G < P ? 32 / G : P;
#pragma unroll
    for (int i0 = 0; i0 < P; i0 += CH) {
      const float* qc = qg + 2 * i0;
      asm volatile("" : "+s"(qc));
#pragma unroll
      for (int ii = 0; ii < CH; ++ii) {
        const int i = i0 + ii;
        const uint32_t c = field<BK>(ka, i);
        const float rho = (float)((kr[i >> 2] >> (8 * (i & 3))) & 0xFFu);
        const float2 cs = lut_k[c];
        const float x = rho * cs.x, y = rho * cs.y;
#pragma unroll
        for (int g = 0; g < G; ++g)
          sc[g] = fmaf(x, qc[g * D + 2 * ii], fmaf(y, qc[g * D + 2 * ii + 1], sc[g]));
      }
    }
    const bool valid = lane < nvalid;
    float pr[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float s = valid ? sc[g] * kscale : -INFINITY;
      const float mnew = fmaxf(m[g], wave_max(s));
      const float alpha = exp2f(m[g] - mnew);
      const float pv = exp2f(s - mnew);
      l[g] = l[g] * alpha + wave_sum(pv);
      acc0[g] *= alpha;
      acc1[g] *= alpha;
      m[g] = mnew;
      pr[g] = pv;
    }

    // ---- per-token value radius parameters (lane = token): r = 2^(lg + rho * beta)
    float lg = 0.f, beta = 0.f;
    if (valid) {
      const float smin = __half2float(__ushort_as_half((uint16_t)(vpar & 0xFFFFu)));
      const float smax = __half2float(__ushort_as_half((uint16_t)(vpar >> 16)));
      if (smax > smin) {
        lg = __log2f(smin);
        beta = (__log2f(smax) - lg) * (1.0f / 15.0f);
      } else {
        lg = __log2f(smax);
      }
    }

    // ---- values: lane = pair (d = 64: the two half-waves take tokens j and j + 32)
#pragma unroll
    for (int jj = 0; jj < NT; ++jj) {
      if (jj >= nvalid) break;
      float lgj, bj, pj[G];
      if (NT == 64) {
        lgj = readlane_f(lg, jj);
        bj = readlane_f(beta, jj);
#pragma unroll
        for (int g = 0; g < G; ++g) pj[g] = readlane_f(pr[g], jj);
      } else {
        const float l0 = readlane_f(lg, jj), l1 = readlane_f(lg, jj + 32);
        const float b0 = readlane_f(beta, jj), b1 = readlane_f(beta, jj + 32);
        lgj = vhalf ? l1 : l0;
        bj = vhalf ? b1 : b0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float p0 = readlane_f(pr[g], jj), p1 = readlane_f(pr[g], jj + 32);
          pj[g] = vhalf ? p1 : p0;
        }
      }
      const uint32_t c = field<BV>(va, jj);
      const uint32_t rho = (vr[jj >> 3] >> (4 * (jj & 7))) & 0xFu;
      const float r = exp2f(fmaf((float)rho, bj, lgj));
      const float2 cs = lut_v[c];
      const float vx = r * cs.x, vy = r * cs.y;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        acc0[g] = fmaf(pj[g], vx, acc0[g]);
        acc1[g] = fmaf(pj[g], vy, acc1[g]);
      }
    }
  }

  // ---- merge the four waves, then this split's partial per query head
  if (P == 32) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      acc0[g] += __shfl_xor(acc0[g], 32);
      acc1[g] += __shfl_xor(acc1[g], 32);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      s_m[wave][g] = m[g];
      s_l[wave][g] = l[g];
    }
  }
  if (lane < P) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      s_acc[wave][g][2 * lane] = acc0[g];
      s_acc[wave][g][2 * lane + 1] = acc1[g];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += 256) {
    const int g = idx / D, e = idx % D;
    float mm = s_m[0][g];
#pragma unroll
    for (int w = 1; w < 4; ++w) mm = fmaxf(mm, s_m[w][g]);
    float ll = 0.f, aa = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = exp2f(s_m[w][g] - mm);
      ll += s_l[w][g] * f;
      aa += s_acc[w][g][e] * f;
    }
    const size_t row = ((size_t)bk * G + g) * a.nsplit + split;
    a.part_acc[row * D + e] = aa;
    if (e == 0) {
      a.part_ml[2 * row] = mm;
      a.part_ml[2 * row + 1] = ll;
    }
  }
}

// ---------------------------------------------------------------------------- merge

template <int D>
__global__ __launch_bounds__(64) void attn_merge_kernel(AttnArgs a, void* __restrict__ out,
                                                        int f32_out) {
  constexpr int P = D / 2;
  const int bh = blockIdx.x;  // b * hq + h
  const int lane = threadIdx.x;
  const float* ml = a.part_ml + (size_t)bh * a.nsplit * 2;
  const float* acc = a.part_acc + (size_t)bh * a.nsplit * D;
  float mloc = -INFINITY;
  for (int s = lane; s < a.nsplit; s += 64) mloc = fmaxf(mloc, ml[2 * s]);
  const float mm = wave_max(mloc);
  float lloc = 0.f;
  for (int s = lane; s < a.nsplit; s += 64) lloc += ml[2 * s + 1] * exp2f(ml[2 * s] - mm);
  const float ll = wave_sum(lloc);
  if (lane >= P) return;
  float a0 = 0.f, a1 = 0.f;
  for (int s = 0; s < a.nsplit; ++s) {
    const float f = exp2f(ml[2 * s] - mm);
    const float2 v = reinterpret_cast<const float2*>(acc + (size_t)s * D)[lane];
    a0 = fmaf(f, v.x, a0);
    a1 = fmaf(f, v.y, a1);
  }
  const float inv_l = 1.0f / ll;
  a0 *= inv_l;
  a1 *= inv_l;
  fwht_pairs_f32<P>(a0, a1, lane);
  const int e0 = 2 * lane;
  a0 *= a.inv_sqrt_d;
  a1 *= a.inv_sqrt_d;
  if (sign_neg(a.sign, e0)) a0 = -a0;
  if (sign_neg(a.sign, e0 + 1)) a1 = -a1;
  const size_t off = (size_t)bh * D + e0;
  if (f32_out)
    reinterpret_cast<float2*>(out)[off >> 1] = make_float2(a0, a1);
  else
    reinterpret_cast<__half2*>(out)[off >> 1] = __floats2half2_rn(a0, a1);
}

template <int D, int G, int BK>
hipError_t split_bv(const AttnArgs& a, const uint8_t* cache, dim3 grid, hipStream_t s) {
  switch (a.bv) {
    case 6: hipLaunchKernelGGL((attn_split_kernel<D, G, BK, 6>), grid, dim3(256), 0, s, a, cache, a.qrot); break;
    case 7: hipLaunchKernelGGL((attn_split_kernel<D, G, BK, 7>), grid, dim3(256), 0, s, a, cache, a.qrot); break;
    case 8: hipLaunchKernelGGL((attn_split_kernel<D, G, BK, 8>), grid, dim3(256), 0, s, a, cache, a.qrot); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int G>
hipError_t split_bk(const AttnArgs& a, const uint8_t* cache, dim3 grid, hipStream_t s) {
  switch (a.bk) {
    case 6: return split_bv<D, G, 6>(a, cache, grid, s);
    case 7: return split_bv<D, G, 7>(a, cache, grid, s);
    case 8: return split_bv<D, G, 8>(a, cache, grid, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t split_g(const AttnArgs& a, const uint8_t* cache, dim3 grid, hipStream_t s) {
  switch (a.group) {
    case 1: return split_bk<D, 1>(a, cache, grid, s);
    case 2: return split_bk<D, 2>(a, cache, grid, s);
    case 4: return split_bk<D, 4>(a, cache, grid, s);
    case 8: return split_bk<D, 8>(a, cache, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_prepare(const AttnArgs& a, int d, const void* q, bool f32_q,
                               hipStream_t stream) {
  const dim3 grid((unsigned)(a.batch * a.hq)), block(64);
  if (d == 64)
    hipLaunchKernelGGL(attn_prepare_kernel<64>, grid, block, 0, stream, a, q, (int)f32_q);
  else if (d == 128)
    hipLaunchKernelGGL(attn_prepare_kernel<128>, grid, block, 0, stream, a, q, (int)f32_q);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attn_split(const AttnArgs& a, int d, TileGeom geom, const uint8_t* cache,
                             hipStream_t stream) {
  (void)geom;
  const dim3 grid((unsigned)a.nsplit, (unsigned)(a.batch * a.hkv));
  if (d == 64) return split_g<64>(a, cache, grid, stream);
  if (d == 128) return split_g<128>(a, cache, grid, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_merge(const AttnArgs& a, int d, void* out, bool f32_out,
                             hipStream_t stream) {
  const dim3 grid((unsigned)(a.batch * a.hq)), block(64);
  if (d == 64)
    hipLaunchKernelGGL(attn_merge_kernel<64>, grid, block, 0, stream, a, out, (int)f32_out);
  else if (d == 128)
    hipLaunchKernelGGL(attn_merge_kernel<128>, grid, block, 0, stream, a, out, (int)f32_out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kvq
