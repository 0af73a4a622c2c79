// Dequantise kernel: codes -> rotated-domain pairs r_hat (cos, sin) -> inverse
// Walsh-Hadamard transform -> sign diagonal -> fp16/fp32 vectors.
//
// The inverse of the encode in "TurboAngle: Near-Lossless KV Cache Compression via
// Uniform Angle Quantization" (arXiv 2603.27467), Abstract: the normalised transform
// H/sqrt(d) is symmetric and its own inverse, so x_hat = sign * H y_hat / sqrt(d).
// fp32 arithmetic; reconstruction angles come from an LDS table of cos/sin(2 pi c / n).
//
// Work split: one 64-lane wave per (batch, kv head, tile); a lane owns one pair of a
// vector (two vectors per step when d = 64), so each output row is written by one
// coalesced 4- or 8-byte store per lane.
#include <hip/hip_fp16.h>

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

// Code of width `bits` starting at bit `pos` of a little-endian word string.
__device__ __forceinline__ uint32_t read_bits(const uint32_t* words, int stride_words, int pos,
                                              int bits) {
  const int w = pos >> 5, sh = pos & 31;
  uint64_t v = words[w * stride_words];
  if (sh + bits > 32) v |= (uint64_t)words[(w + 1) * stride_words] << 32;
  return (uint32_t)(v >> sh) & ((1u << bits) - 1u);
}

__device__ __forceinline__ void store_pair(void* base, bool f32, int64_t off, float x0, float x1) {
  if (f32)
    *reinterpret_cast<float2*>(static_cast<float*>(base) + off) = make_float2(x0, x1);
  else
    *reinterpret_cast<__half2*>(static_cast<__half*>(base) + off) = __floats2half2_rn(x0, x1);
}

template <int D>
__global__ __launch_bounds__(64) void decode_kernel(CodecArgs a, TileGeom g,
                                                    const uint8_t* __restrict__ cache,
                                                    void* __restrict__ kout,
                                                    void* __restrict__ vout, int f32_out) {
  constexpr int P = D / 2;
  constexpr int VPW = 64 / P;
  __shared__ float2 lut_k[256], lut_v[256];
  const int lane = threadIdx.x;
  for (int c = lane; c < a.n_k; c += 64) {
    double s, co;
    sincospi(2.0 * c / a.n_k, &s, &co);
    lut_k[c] = make_float2((float)co, (float)s);
  }
  for (int c = lane; c < a.n_v; c += 64) {
    double s, co;
    sincospi(2.0 * c / a.n_v, &s, &co);
    lut_v[c] = make_float2((float)co, (float)s);
  }
  __syncthreads();

  const int tile_rel = blockIdx.x % a.tiles_touched;
  const int bh = blockIdx.x / a.tiles_touched;
  const int b = bh / a.hkv, h = bh % a.hkv;
  const int tile = a.tile_lo + tile_rel;
  const int tok_base = tile * kTile;
  const int j_lo = max(a.t0 - tok_base, 0);
  const int j_hi = min(a.t0 + a.ntok - tok_base, kTile);
  const uint8_t* tp =
      cache + ((size_t)(b * a.hkv + h) * a.tiles_per_seq + tile) * (size_t)g.bytes;
  const uint32_t* ka = reinterpret_cast<const uint32_t*>(tp + g.ka);
  const uint32_t* kr = reinterpret_cast<const uint32_t*>(tp + g.kr);
  const uint16_t* ks = reinterpret_cast<const uint16_t*>(tp + g.ks);
  const uint32_t* va = reinterpret_cast<const uint32_t*>(tp + g.va);
  const uint32_t* vrw = reinterpret_cast<const uint32_t*>(tp + g.vr);
  const uint32_t* vp = reinterpret_cast<const uint32_t*>(tp + g.vp);

  const int p = lane % P, sub = lane / P;
  const int e0 = 2 * p;
  const float sg0 = sign_neg(a.sign, e0) ? -1.0f : 1.0f;
  const float sg1 = sign_neg(a.sign, e0 + 1) ? -1.0f : 1.0f;
  const float inv_sqrt_d = (float)a.inv_sqrt_d;

  for (int jb = j_lo; jb < j_hi; jb += VPW) {
    const int j = min(jb + sub, j_hi - 1);  // a spare half-wave repeats the last token
    const bool act = jb + sub < j_hi;
    // keys: token-major planes, word w of slot j at w * 64 + j
    const uint32_t kc = read_bits(ka + j, kTile, p * a.bk, a.bk);
    const uint32_t krho = (kr[(p >> 2) * kTile + j] >> (8 * (p & 3))) & 0xFFu;
    const float kscale = __half2float(__ushort_as_half(ks[j]));
    const float krh = (float)krho * (kscale / 255.0f);
    float k0 = krh * lut_k[kc].x, k1 = krh * lut_k[kc].y;
    fwht_pairs_f32<P>(k0, k1, p);
    // values: pair-major planes, word w of pair p at w * P + p
    const uint32_t vc = read_bits(va + p, P, j * a.bv, a.bv);
    const uint32_t vrho = (vrw[(j >> 3) * P + p] >> (4 * (j & 7))) & 0xFu;
    const uint32_t vpar = vp[j];
    const float smin = __half2float(__ushort_as_half((uint16_t)(vpar & 0xFFFFu)));
    const float smax = __half2float(__ushort_as_half((uint16_t)(vpar >> 16)));
    float vrh = smax;
    if (smax > smin) vrh = smin * expf((float)vrho * logf(smax / smin) / 15.0f);
    float v0 = vrh * lut_v[vc].x, v1 = vrh * lut_v[vc].y;
    fwht_pairs_f32<P>(v0, v1, p);
    if (act) {
      const int64_t off =
          (((int64_t)b * a.ntok + (tok_base + j - a.t0)) * a.hkv + h) * D + e0;
      store_pair(kout, f32_out, off, k0 * inv_sqrt_d * sg0, k1 * inv_sqrt_d * sg1);
      store_pair(vout, f32_out, off, v0 * inv_sqrt_d * sg0, v1 * inv_sqrt_d * sg1);
    }
  }
}

}  // namespace

hipError_t launch_decode(const CodecArgs& a, int d, TileGeom geom, const uint8_t* cache,
                         void* k_out, void* v_out, bool f32_out, hipStream_t stream) {
  const long long blocks = (long long)a.batch * a.hkv * a.tiles_touched;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(64);
  if (d == 64)
    hipLaunchKernelGGL(decode_kernel<64>, grid, block, 0, stream, a, geom, cache, k_out, v_out,
                       (int)f32_out);
  else if (d == 128)
    hipLaunchKernelGGL(decode_kernel<128>, grid, block, 0, stream, a, geom, cache, k_out,
                       v_out, (int)f32_out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kvq
