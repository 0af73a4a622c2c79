// Dequantise kernel: codes -> rotated-domain pairs r_hat (cos, sin) -> inverse
// Walsh-Hadamard transform -> sign diagonal -> fp16/fp32 vectors.
//
// The inverse of the encode in "TurboAngle: Near-Lossless KV Cache Compression via
// Uniform Angle Quantization" (arXiv 2603.27467), Abstract: the normalised transform
// H/sqrt(d) is symmetric and its own inverse, so x_hat = sign * H y_hat / sqrt(d).
// fp32 arithmetic; reconstruction angles come from an LDS table of cos/sin(2 pi c / n).
//
// Work split: one 64-lane wave per (batch, kv head, tile). The tile is copied to LDS
// with coalesced loads; a lane then owns a quarter of one vector (d/4 elements in
// interleaved 8-element chunks, 16 tokens per step), so the inverse transform is
// in-lane except for two DPP quad exchanges, the sign diagonal is applied as an xor on
// the packed output, and each store instruction writes 64 contiguous bytes per token.
#include <hip/hip_fp16.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

// Lane exchange inside a quad (lanes 4k..4k+3): xor 1 or xor 2.
template <int CTRL>
__device__ __forceinline__ float quad_xor(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E;

// LDS copy of one tile, one pad word after every 64 so that the 16 tokens x 4
// quarters of a step, reading different words of the same token column, fall in
// different banks.
__device__ __forceinline__ int padded(int word) { return word + (word >> 6); }

template <int D, bool F32OUT>
__global__ __launch_bounds__(64) void decode_kernel(CodecArgs a, TileGeom g,
                                                    const uint8_t* __restrict__ cache,
                                                    void* __restrict__ kout,
                                                    void* __restrict__ vout) {
  constexpr int P = D / 2;   // pairs per vector
  constexpr int E = D / 4;   // elements per lane (one quarter of a vector)
  constexpr int PL = E / 2;  // pairs per lane
  constexpr int TPS = 16;    // tokens per step
  // largest tile (8-bit angle codes): KA 64P*8/8 + KR 64P + KS 128 + VA 64P + VR 32P + VP 256
  constexpr int MAX_WORDS = (kTile * P + kTile * P + 2 * kTile + P * 2 * 8 * 4 + P * 32 + 4 * kTile) / 4;
  __shared__ float2 lut_k[256], lut_v[256];
  __shared__ uint32_t tw[MAX_WORDS + MAX_WORDS / 64 + 1];

  const int lane = threadIdx.x;
  const int tq = lane >> 2, q = lane & 3;
  const int tile_rel = blockIdx.x % a.tiles_touched;
  const int bh = blockIdx.x / a.tiles_touched;
  const int b = bh / a.hkv, h = bh % a.hkv;
  const int tile = a.tile_lo + tile_rel;
  const int tok_base = tile * kTile;
  const int j_lo = max(a.t0 - tok_base, 0);
  const int j_hi = min(a.t0 + a.ntok - tok_base, kTile);
  const uint32_t* tp = reinterpret_cast<const uint32_t*>(
      cache + ((size_t)(b * a.hkv + h) * a.tiles_per_seq + tile) * (size_t)g.bytes);
  const int nwords = g.bytes / 4;
  for (int w = lane; w < nwords; w += 64) tw[padded(w)] = tp[w];
  for (int c = lane; c < 256; c += 64) {
    float sn = 0.f, co = 0.f;
    if (c < a.n_k) sincospif(2.0f * (float)c / (float)a.n_k, &sn, &co);
    lut_k[c] = make_float2(co, sn);
    sn = 0.f;
    co = 0.f;
    if (c < a.n_v) sincospif(2.0f * (float)c / (float)a.n_v, &sn, &co);
    lut_v[c] = make_float2(co, sn);
  }
  __syncthreads();

  // Lane q of a token's quad owns the 8-element chunks m*4 + q (elements
  // 32m + 8q + r, r < 8); local slot 8m + r. The transform's in-lane stages are the
  // element strides 1, 2, 4 (r) and 32, 64 (m); strides 8 and 16 are the quad xor 1
  // and xor 2 exchanges. Local bit 8m + r of sbits is the sign of element 32m + 8q + r.
  uint32_t sbits = 0;
#pragma unroll
  for (int m = 0; m < E / 8; ++m)
    sbits |= (uint32_t)((a.sign.w[(32 * m + 8 * q) >> 6] >> ((32 * m + 8 * q) & 63)) & 0xFFu) << (8 * m);
  const float qsgn1 = (q & 1) ? -1.0f : 1.0f, qsgn2 = (q & 2) ? -1.0f : 1.0f;
  const float inv_sqrt_d = (float)a.inv_sqrt_d;
  const int ka = g.ka / 4, kr = g.kr / 4, va = g.va / 4, vr = g.vr / 4;
  const int bk = a.bk, bv = a.bv;

  for (int jb = j_lo; jb < j_hi; jb += TPS) {
    const int j = min(jb + tq, j_hi - 1);  // lanes past the range repeat the last token
    const bool act = jb + tq < j_hi;
    const int64_t out_off = (((int64_t)b * a.ntok + (tok_base + j - a.t0)) * a.hkv + h) * D + 8 * q;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      float y[E];
      if (kv == 0) {
        const float ks = __half2float(__ushort_as_half(
            (uint16_t)(tw[padded((g.ks + 2 * j) / 4)] >> (16 * (j & 1)))));
        const float rs = ks * (1.0f / 255.0f) * inv_sqrt_d;
#pragma unroll
        for (int k = 0; k < PL; ++k) {
          const int i = 16 * (k >> 2) + 4 * q + (k & 3);  // pair of local slots 2k, 2k+1
          const int pos = i * bk, w = pos >> 5, sh = pos & 31;
          uint64_t bits = tw[padded(ka + w * kTile + j)];
          if (sh + bk > 32) bits |= (uint64_t)tw[padded(ka + (w + 1) * kTile + j)] << 32;
          const uint32_t c = (uint32_t)(bits >> sh) & ((1u << bk) - 1u);
          const uint32_t rho = (tw[padded(kr + (i >> 2) * kTile + j)] >> (8 * (i & 3))) & 0xFFu;
          const float rh = (float)rho * rs;
          const float2 cs = lut_k[c];
          y[2 * k] = rh * cs.x;
          y[2 * k + 1] = rh * cs.y;
        }
      } else {
        const uint32_t vp = tw[padded((g.vp + 4 * j) / 4)];
        const float smin = __half2float(__ushort_as_half((uint16_t)(vp & 0xFFFFu)));
        const float smax = __half2float(__ushort_as_half((uint16_t)(vp >> 16)));
        const bool spread = smax > smin;
        const float lam = spread ? logf(smax / smin) * (1.0f / 15.0f) : 0.f;
        const float r0 = (spread ? smin : smax) * inv_sqrt_d;
        const int pos = j * bv, w = pos >> 5, sh = pos & 31;
#pragma unroll
        for (int k = 0; k < PL; ++k) {
          const int i = 16 * (k >> 2) + 4 * q + (k & 3);
          uint64_t bits = tw[padded(va + w * P + i)];
          if (sh + bv > 32) bits |= (uint64_t)tw[padded(va + (w + 1) * P + i)] << 32;
          const uint32_t c = (uint32_t)(bits >> sh) & ((1u << bv) - 1u);
          const uint32_t rho = (tw[padded(vr + (j >> 3) * P + i)] >> (4 * (j & 7))) & 0xFu;
          const float rh = r0 * expf((float)rho * lam);
          const float2 cs = lut_v[c];
          y[2 * k] = rh * cs.x;
          y[2 * k + 1] = rh * cs.y;
        }
      }
      // inverse transform (H is its own inverse up to the 1/sqrt(d) already applied)
#pragma unroll
      for (int hs = 1; hs < E; hs <<= 1) {
#pragma unroll
        for (int i = 0; i < E; ++i) {
          if (i & hs) continue;
          const float u = y[i], v = y[i + hs];
          y[i] = u + v;
          y[i + hs] = u - v;
        }
      }
#pragma unroll
      for (int i = 0; i < E; ++i) y[i] = fmaf(y[i], qsgn1, quad_xor<kQuadXor1>(y[i]));
#pragma unroll
      for (int i = 0; i < E; ++i) y[i] = fmaf(y[i], qsgn2, quad_xor<kQuadXor2>(y[i]));
      if (act) {
        void* dst = kv == 0 ? kout : vout;
        if (F32OUT) {
          float* o = static_cast<float*>(dst) + out_off;
#pragma unroll
          for (int e = 0; e < E; e += 4) {
            float4 v4;
            v4.x = __uint_as_float(__float_as_uint(y[e]) ^ (((sbits >> e) & 1u) << 31));
            v4.y = __uint_as_float(__float_as_uint(y[e + 1]) ^ (((sbits >> (e + 1)) & 1u) << 31));
            v4.z = __uint_as_float(__float_as_uint(y[e + 2]) ^ (((sbits >> (e + 2)) & 1u) << 31));
            v4.w = __uint_as_float(__float_as_uint(y[e + 3]) ^ (((sbits >> (e + 3)) & 1u) << 31));
            *reinterpret_cast<float4*>(o + 32 * (e >> 3) + (e & 7)) = v4;
          }
        } else {
          __half* o = static_cast<__half*>(dst) + out_off;
#pragma unroll
          for (int m = 0; m < E / 8; ++m) {
            uint32_t w4[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int e = 8 * m + 2 * t;
              const uint32_t msk = (((sbits >> e) & 1u) << 15) | (((sbits >> (e + 1)) & 1u) << 31);
              w4[t] = __builtin_bit_cast(uint32_t, __floats2half2_rn(y[e], y[e + 1])) ^ msk;
            }
            *reinterpret_cast<uint4*>(o + 32 * m) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
          }
        }
      }
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
  if (d == 64 && f32_out)
    hipLaunchKernelGGL((decode_kernel<64, true>), grid, block, 0, stream, a, geom, cache, k_out, v_out);
  else if (d == 64)
    hipLaunchKernelGGL((decode_kernel<64, false>), grid, block, 0, stream, a, geom, cache, k_out, v_out);
  else if (d == 128 && f32_out)
    hipLaunchKernelGGL((decode_kernel<128, true>), grid, block, 0, stream, a, geom, cache, k_out, v_out);
  else if (d == 128)
    hipLaunchKernelGGL((decode_kernel<128, false>), grid, block, 0, stream, a, geom, cache, k_out, v_out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kvq
