// Dequantise kernel: codes -> rotated-domain pairs r_hat (cos, sin) -> inverse
// Walsh-Hadamard transform -> sign diagonal -> fp16/fp32 vectors.
//
// The inverse of the encode in "TurboAngle: Near-Lossless KV Cache Compression via
// Uniform Angle Quantization" (arXiv 2603.27467), Abstract: the normalised transform
// H/sqrt(d) is symmetric and its own inverse, so x_hat = sign * H y_hat / sqrt(d).
// fp32 arithmetic; reconstruction angles come from an LDS table of cos/sin(2 pi c / n).
//
// Work split: a 256-thread workgroup walks tiles (batch, kv head, 64-slot tile) in
// grid-stride order and keeps the next tile's bytes in flight in registers while it
// decodes the current one from LDS. Wave w decodes slots 16w..16w+15 of every tile; a
// lane owns a quarter of one vector (d/4 elements in interleaved 8-element chunks), so
// the inverse transform is in-lane except for two DPP quad exchanges, and every LDS
// address a lane reads is the same in every tile. Per-vector scales leave the
// transform: the key scale is applied at the output conversion and the value scale
// enters the exponent of the radius decoder.
#include <hip/hip_fp16.h>

#include <atomic>

#include "kvq_internal.h"

namespace kvq {
namespace {

// Lane exchange inside a quad (lanes 4k..4k+3): xor 1 or xor 2.
template <int CTRL>
__device__ __forceinline__ float quad_xor(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E;

// Staged tile in LDS: every plane is cut into rows (64 slot words for the key planes,
// P pair words for the value planes, one row each for the key scales and the value
// parameters) stored kRowStride words apart. The 8-word pad puts the four rows that
// the four quarter-lanes of a token read, for 8 tokens at a time, in distinct banks;
// a multiple of four keeps every row 16-byte aligned for 128-bit LDS writes.
constexpr int kRowStride = 72;
constexpr int kMaxDevices = 64;

// 16-byte word group (a plain vector type: loads and stores stay single instructions)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// LDS word index of tile word x (x a multiple of 4).
__device__ __forceinline__ int staged_word(int x, const TileGeom& g, int pairs) {
  const int ks = g.ks >> 2, va = g.va >> 2, vp = g.vp >> 2;
  const int rks = ks >> 6;  // key planes are whole 64-word rows
  if (x < ks) return (x >> 6) * kRowStride + (x & 63);
  if (x < va) return rks * kRowStride + (x - ks);
  if (x < vp) {
    const int y = x - va;
    return (rks + 1 + y / pairs) * kRowStride + y % pairs;
  }
  return (rks + 1 + g.wva + g.wvr) * kRowStride + (x - vp);
}

template <int D, bool F32OUT>
__global__ __launch_bounds__(256) void decode_kernel(CodecArgs a, TileGeom g,
                                                     const uint8_t* __restrict__ cache,
                                                     void* __restrict__ kout,
                                                     void* __restrict__ vout) {
  constexpr int P = D / 2;   // pairs per vector
  constexpr int E = D / 4;   // elements per lane (one quarter of a vector)
  constexpr int NM = E / 8;  // 8-element chunks per lane
  constexpr int RS = kRowStride;
  // rows at the widest codes (8 bits): KA P/4, KR P/4, KS 1, VA 16, VR 8, VP 1
  constexpr int MAX_ROWS = P / 4 + P / 4 + 1 + 16 + 8 + 1;
  constexpr int MAX_V4 = (kTile * (P / 4) * 2 + 32 + P * 24 + kTile) / 4;
  constexpr int NV4 = (MAX_V4 + 255) / 256;  // 16-byte loads per thread per tile
  __shared__ float2 lut_k[256], lut_v[256];
  __shared__ u32x4 stage[MAX_ROWS * RS / 4 + 1];  // + a spare slot for loads past the tile
  const uint32_t* tw = reinterpret_cast<const uint32_t*>(stage);

  const int tid = threadIdx.x;
  const int lane = tid & 63, q = lane & 3;
  const int j = 16 * (tid >> 6) + (lane >> 2);  // slot decoded by this lane
  const int ntasks = a.batch * a.hkv * a.tiles_touched;
  const int nv4 = g.bytes >> 4;

  int dst[NV4];  // LDS uint4 index of each loaded uint4 (the spare slot past the tile)
  int src[NV4];  // uint4 index in the tile (clamped, so every load is in bounds)
#pragma unroll
  for (int s = 0; s < NV4; ++s) {
    const int u = tid + 256 * s;
    dst[s] = u < nv4 ? staged_word(4 * u, g, P) >> 2 : MAX_ROWS * RS / 4;
    src[s] = min(u, nv4 - 1);
  }
  // Tiles are taken in grid-stride order; pre holds the next tile's bytes.
  const size_t tile_bytes = (size_t)g.bytes;
  // A tile the page table maps to no page decodes as all-zero bytes (zero vectors).
  (void)tile_bytes;
  auto tile_ptr = [&](int t) -> const u32x4* {
    const int tile_rel = t % a.tiles_touched, bh = t / a.tiles_touched;
    const long long off = tile_offset(a.pg, bh / a.hkv, bh % a.hkv, a.hkv, a.tiles_per_seq,
                                      a.tile_lo + tile_rel, g.bytes);
    return off >= 0 ? reinterpret_cast<const u32x4*>(cache + off) : nullptr;
  };
  auto fetch = [&](u32x4 (&dstv)[NV4], int t) {
    const u32x4* tp = tile_ptr(t);
    if (tp) {
#pragma unroll
      for (int s = 0; s < NV4; ++s) dstv[s] = tp[src[s]];
    } else {
#pragma unroll
      for (int s = 0; s < NV4; ++s) dstv[s] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  u32x4 pre[NV4];
  int task = blockIdx.x;
  if (task < ntasks) fetch(pre, task);

  // Angle tables hold (cos + sin, cos - sin) of 2 pi c / n: the transform's first
  // stage (element stride 1) combines the two components of each pair.
  {
    float sn = 0.f, co = 0.f;
    if (tid < a.n_k) sincospif(2.0f * (float)tid / (float)a.n_k, &sn, &co);
    lut_k[tid] = make_float2(co + sn, co - sn);
    sn = 0.f;
    co = 0.f;
    if (tid < a.n_v) sincospif(2.0f * (float)tid / (float)a.n_v, &sn, &co);
    lut_v[tid] = make_float2(co + sn, co - sn);
  }

  // Lane q of a token's quad owns the 8-element chunks m*4 + q (elements
  // 32m + 8q + r, r < 8); local slot 8m + r, pair 16m + 4q + r/2. The in-lane stages
  // are the element strides 1, 2, 4 (r) and 32, 64 (m); strides 8 and 16 are the quad
  // exchanges, computed as w + s*partner(w) with s = -1 on lanes with q bit 0 (then
  // bit 1) set. That leaves each lane's result times s1*s2, which the output's sign
  // flip takes back.
  const int bk = a.bk, bv = a.bv;
  const int rks = g.ks >> 8, rv0 = rks + 1;
  int ka_addr[NM], ka_sh[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const int pos = (16 * m + 4 * q) * bk;
    ka_addr[m] = (pos >> 5) * RS + j;
    ka_sh[m] = pos & 31;
  }
  const int kr_addr = (g.wka + q) * RS + j;  // chunk m adds 4m rows
  const int ks_addr = rks * RS + (j >> 1), ks_sh = 16 * (j & 1);
  const int vpos = j * bv;
  const int va_addr = (rv0 + (vpos >> 5)) * RS + 4 * q;  // pair 16m + 4q + r adds 16m + r
  const int va_sh = vpos & 31;
  const int vr_addr = (rv0 + g.wva + (j >> 3)) * RS + 4 * q;
  const int vr_sh = 4 * (j & 7);
  const int vp_addr = (rv0 + g.wva + g.wvr) * RS + j;

  uint32_t smask[E / 2];  // sign flips of output elements 2t (bit 15) and 2t + 1 (bit 31)
  {
    const uint32_t flip = (q == 1 || q == 2) ? 0x80008000u : 0u;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      // elements 32m + 8q .. +7 lie in mask word m / 2 (8q + 8 <= 32)
      const uint32_t byte = (uint32_t)(a.sign.w[m >> 1] >> (32 * (m & 1) + 8 * q)) & 0xFFu;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        smask[4 * m + t] = flip ^ (((byte >> (2 * t)) & 1u) << 15) ^ (((byte >> (2 * t + 1)) & 1u) << 31);
    }
  }
  float s1 = (q & 1) ? -1.0f : 1.0f, s2 = (q & 2) ? -1.0f : 1.0f;
  // opaque to the optimiser, so the products stay multiplies that take the DPP
  // operand instead of becoming sign selects
  asm volatile("" : "+v"(s1), "+v"(s2));
  const float inv_sqrt_d = (float)a.inv_sqrt_d;

  for (; task < ntasks; task += gridDim.x) {
    __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll
    for (int s = 0; s < NV4; ++s) stage[dst[s]] = pre[s];
    __syncthreads();
    if (task + (int)gridDim.x < ntasks) fetch(pre, task + (int)gridDim.x);

    const int tile_rel = task % a.tiles_touched, bh = task / a.tiles_touched;
    const int b = bh / a.hkv, h = bh % a.hkv;
    const int tok_base = (a.tile_lo + tile_rel) * kTile;
    const bool act = tok_base + j >= a.t0 && tok_base + j < a.t0 + a.ntok;
    const int64_t out_off = (((int64_t)b * a.ntok + (tok_base + j - a.t0)) * a.hkv + h) * D + 8 * q;

#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      float y[E];
      if (kv == 0) {
        const float ks = __half2float(__ushort_as_half((uint16_t)(tw[ks_addr] >> ks_sh)));
        const float kscale = ks * (1.0f / 255.0f) * inv_sqrt_d;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const uint32_t bits = __builtin_amdgcn_alignbit(tw[ka_addr[m] + RS], tw[ka_addr[m]], ka_sh[m]);
          const uint32_t rw = tw[kr_addr + 4 * m * RS];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float2 t = lut_k[__builtin_amdgcn_ubfe(bits, r * bk, bk)];
            const float rho = (float)((rw >> (8 * r)) & 0xFFu) * kscale;
            y[8 * m + 2 * r] = rho * t.x;
            y[8 * m + 2 * r + 1] = rho * t.y;
          }
        }
      } else {
        // r_hat = s_min exp(code L / 15) / sqrt(d) = exp2(code * l2 + l0)
        const uint32_t vp = tw[vp_addr];
        const float smin = __half2float(__ushort_as_half((uint16_t)(vp & 0xFFFFu)));
        const float smax = __half2float(__ushort_as_half((uint16_t)(vp >> 16)));
        const bool spread = smax > smin;
        const float l2 = spread ? log2f(smax / smin) * (1.0f / 15.0f) : 0.f;
        const float l0 = log2f((spread ? smin : smax) * inv_sqrt_d);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int col = 16 * m + r;
            const uint32_t c = __builtin_amdgcn_ubfe(
                __builtin_amdgcn_alignbit(tw[va_addr + col + RS], tw[va_addr + col], va_sh), 0, bv);
            const float2 t = lut_v[c];
            const float rho = (float)__builtin_amdgcn_ubfe(tw[vr_addr + col], vr_sh, 4);
            const float rh = __builtin_amdgcn_exp2f(fmaf(rho, l2, l0));
            y[8 * m + 2 * r] = rh * t.x;
            y[8 * m + 2 * r + 1] = rh * t.y;
          }
        }
      }
      // inverse transform (H is its own inverse up to the 1/sqrt(d) in the scales)
#pragma unroll
      for (int hs = 2; hs < E; hs <<= 1) {
#pragma unroll
        for (int i = 0; i < E; ++i) {
          if (i & hs) continue;
          const float u = y[i], v = y[i + hs];
          y[i] = u + v;
          y[i + hs] = u - v;
        }
      }
      {
#pragma clang fp contract(off)
#pragma unroll
        for (int i = 0; i < E; ++i) y[i] = y[i] + quad_xor<kQuadXor1>(y[i]) * s1;
#pragma unroll
        for (int i = 0; i < E; ++i) y[i] = y[i] + quad_xor<kQuadXor2>(y[i]) * s2;
      }
      // finish the transform on every lane before the stores' lane mask
#pragma unroll
      for (int i = 0; i < E; ++i) asm volatile("" : "+v"(y[i]));
      if (act) {
        void* dstp = kv == 0 ? kout : vout;
        if (F32OUT) {
          float* o = static_cast<float*>(dstp) + out_off;
#pragma unroll
          for (int m = 0; m < NM; ++m) {
#pragma unroll
            for (int h4 = 0; h4 < 2; ++h4) {
              const int e = 8 * m + 4 * h4;
              const uint32_t m0 = smask[e >> 1], m1 = smask[(e >> 1) + 1];
              float4 v4;
              v4.x = __uint_as_float(__float_as_uint(y[e]) ^ (m0 << 16));
              v4.y = __uint_as_float(__float_as_uint(y[e + 1]) ^ (m0 & 0x80000000u));
              v4.z = __uint_as_float(__float_as_uint(y[e + 2]) ^ (m1 << 16));
              v4.w = __uint_as_float(__float_as_uint(y[e + 3]) ^ (m1 & 0x80000000u));
              *reinterpret_cast<float4*>(o + 32 * m + 4 * h4) = v4;
            }
          }
        } else {
          __half* o = static_cast<__half*>(dstp) + out_off;
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            uint32_t w4[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int e = 8 * m + 2 * t;
              w4[t] = __builtin_bit_cast(uint32_t, __floats2half2_rn(y[e], y[e + 1])) ^
                      smask[4 * m + t];
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
  const long long tasks = (long long)a.batch * a.hkv * a.tiles_touched;
  if (tasks <= 0) return hipSuccess;
  if (tasks > 0x7fffffffLL) return hipErrorInvalidValue;
  const void* fn = d == 64 ? (f32_out ? (const void*)decode_kernel<64, true> : (const void*)decode_kernel<64, false>)
                 : d == 128 ? (f32_out ? (const void*)decode_kernel<128, true> : (const void*)decode_kernel<128, false>)
                            : nullptr;
  if (!fn) return hipErrorInvalidValue;
  // One resident wave of workgroups: each walks tiles in grid-stride order, so the
  // grid is the number that fit on the device at once (cached per device and kernel).
  // (relaxed atomics: threads that race on the first call store the same value)
  static std::atomic<int> resident_cache[kMaxDevices][4];
  const int kidx = (d == 128 ? 2 : 0) + (f32_out ? 1 : 0);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int resident = dev >= 0 && dev < kMaxDevices
                     ? resident_cache[dev][kidx].load(std::memory_order_relaxed)
                     : 0;
  if (resident <= 0) {
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0);
    if (e != hipSuccess) return e;
    resident = (cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
    if (dev >= 0 && dev < kMaxDevices)
      resident_cache[dev][kidx].store(resident, std::memory_order_relaxed);
  }
  const dim3 grid((unsigned)(tasks < resident ? tasks : resident)), block(256);
  if (d == 64 && f32_out)
    hipLaunchKernelGGL((decode_kernel<64, true>), grid, block, 0, stream, a, geom, cache, k_out, v_out);
  else if (d == 64)
    hipLaunchKernelGGL((decode_kernel<64, false>), grid, block, 0, stream, a, geom, cache, k_out, v_out);
  else if (d == 128 && f32_out)
    hipLaunchKernelGGL((decode_kernel<128, true>), grid, block, 0, stream, a, geom, cache, k_out, v_out);
  else
    hipLaunchKernelGGL((decode_kernel<128, false>), grid, block, 0, stream, a, geom, cache, k_out, v_out);
  return hipGetLastError();
}

}  // namespace kvq
