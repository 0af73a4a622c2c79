// Widened tile copies for decode attention over narrow codebooks.
//
// The decode-attention kernels read angle codes of 6 to 8 bits. A layer whose K or V
// codebook has at most 32 bins (codes of 1 to 5 bits; TurboAngle abstract: n is set per
// layer and separately for K and V) is attended through a copy of its first `ntiles`
// tiles per (sequence, kv head) in which each such plane is re-packed at 6 bits. Code
// values, radius codes and per-token parameters are copied unchanged, and the angle of
// code c stays 2 pi c / n, so attention over the copy computes what it would over the
// original layout.
//
// One 64-lane workgroup per tile. The narrow plane is staged in LDS; each lane then
// rebuilds one bit string (a token's key string, a pair's value string) at the new
// width and stores it with the tile's usual word order. The other planes are copied
// with 16-byte loads and stores.

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWideBits = 6;
// Largest narrow plane staged: key angles at d = 128, 5 bits (64 tokens x 10 words).
constexpr int kStageWords = 64 * 10;

// Bits [off, off + bits) of a bit string whose word w sits at s[w * stride]
// (bits <= 5: a field spans at most two words).
__device__ __forceinline__ uint32_t field_at(const uint32_t* s, int stride, int off, int bits) {
  const int w = off >> 5, sh = off & 31;
  uint32_t x = s[w * stride] >> sh;
  if (sh + bits > 32) x |= s[(w + 1) * stride] << (32 - sh);
  return x & ((1u << bits) - 1u);
}

// n fields of `bits` each, read in order from `s`, re-packed at 6 bits into `out`
// (n * 6 / 32 words, n a multiple of 16).
template <int N>
__device__ __forceinline__ void repack6(const uint32_t* s, int stride, int bits,
                                        uint32_t (&out)[N * kWideBits / 32]) {
#pragma unroll
  for (int w = 0; w < N * kWideBits / 32; ++w) out[w] = 0u;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t c = field_at(s, stride, i * bits, bits);
    const int o = i * kWideBits;  // compile-time once unrolled
    out[o >> 5] |= c << (o & 31);
    if ((o & 31) > 32 - kWideBits) out[(o >> 5) + 1] |= c >> (32 - (o & 31));
  }
}

// Copies `bytes` (a multiple of 16) from s to d, 16 bytes per lane and step.
__device__ __forceinline__ void copy16(uint8_t* d, const uint8_t* s, int bytes, int lane) {
  using u32x4 = __attribute__((ext_vector_type(4))) unsigned;
  const u32x4* s4 = reinterpret_cast<const u32x4*>(s);
  u32x4* d4 = reinterpret_cast<u32x4*>(d);
  for (int i = lane; i < bytes / 16; i += 64) d4[i] = s4[i];
}

template <int D>
__global__ void __launch_bounds__(64) widen_kernel(const uint8_t* __restrict__ src,
                                                   uint8_t* __restrict__ dst, TileGeom gs,
                                                   TileGeom gd, int src_tiles_per_seq,
                                                   int ntiles) {
  constexpr int P = D / 2;
  __shared__ uint32_t s_w[kStageWords];
  const int lane = threadIdx.x;
  const int tile = blockIdx.x, bh = blockIdx.y;
  const uint8_t* ts = src + ((size_t)bh * src_tiles_per_seq + tile) * gs.bytes;
  uint8_t* td = dst + ((size_t)bh * ntiles + tile) * gd.bytes;

  // key radii and key scales (adjacent in both layouts), value radii and parameters
  copy16(td + gd.kr, ts + gs.kr, gs.va - gs.kr, lane);
  copy16(td + gd.vr, ts + gs.vr, gs.bytes - gs.vr, lane);

  // key angles: token-major words, word w of token t at w * 64 + t
  if (gs.bk == gd.bk) {
    copy16(td + gd.ka, ts + gs.ka, gs.kr - gs.ka, lane);
  } else {
    const uint32_t* ka = reinterpret_cast<const uint32_t*>(ts + gs.ka);
    for (int i = lane; i < kTile * gs.wka; i += 64) s_w[i] = ka[i];
    __syncthreads();
    uint32_t out[P * kWideBits / 32];
    repack6<P>(s_w + lane, kTile, gs.bk, out);
    uint32_t* kd = reinterpret_cast<uint32_t*>(td + gd.ka);
#pragma unroll
    for (int w = 0; w < P * kWideBits / 32; ++w) kd[w * kTile + lane] = out[w];
    __syncthreads();  // s_w is reused below
  }

  // value angles: pair-major words, word w of pair i at w * P + i
  if (gs.bv == gd.bv) {
    copy16(td + gd.va, ts + gs.va, gs.vr - gs.va, lane);
  } else {
    const uint32_t* va = reinterpret_cast<const uint32_t*>(ts + gs.va);
    for (int i = lane; i < P * gs.wva; i += 64) s_w[i] = va[i];
    __syncthreads();
    if (lane < P) {
      uint32_t out[kTile * kWideBits / 32];
      repack6<kTile>(s_w + lane, P, gs.bv, out);
      uint32_t* vd = reinterpret_cast<uint32_t*>(td + gd.va);
#pragma unroll
      for (int w = 0; w < kTile * kWideBits / 32; ++w) vd[w * P + lane] = out[w];
    }
  }
}

// lens[b] = min(positions[b] + 1, max_len), without wrapping at 2^32 - 1.
__global__ void lengths_kernel(const unsigned* __restrict__ positions, unsigned* __restrict__ lens,
                               int batch, unsigned max_len) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) {
    const unsigned p = positions[b];
    lens[b] = p >= max_len ? max_len : p + 1u;
  }
}

}  // namespace

hipError_t launch_lengths(const unsigned* positions, unsigned* lens, int batch, unsigned max_len,
                          hipStream_t stream) {
  if (batch <= 0) return hipSuccess;
  hipLaunchKernelGGL(lengths_kernel, dim3((unsigned)((batch + 255) / 256)), dim3(256), 0, stream,
                     positions, lens, batch, max_len);
  return hipGetLastError();
}

hipError_t launch_widen(const uint8_t* src, int src_tiles_per_seq, uint8_t* dst, int d, int bk,
                        int bv, int units, int ntiles, hipStream_t stream) {
  const TileGeom gs = tile_geom(d, bk, bv);
  const TileGeom gd = tile_geom(d, bk < kWideBits ? kWideBits : bk, bv < kWideBits ? kWideBits : bv);
  if (units <= 0 || ntiles <= 0) return hipSuccess;
  if (ntiles > src_tiles_per_seq || (bk < kWideBits && gs.wka * kTile > kStageWords) ||
      (bv < kWideBits && gs.wva * gs.pairs > kStageWords))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)ntiles, (unsigned)units);
  if (d == 128)
    hipLaunchKernelGGL(widen_kernel<128>, grid, dim3(64), 0, stream, src, dst, gs, gd,
                       src_tiles_per_seq, ntiles);
  else if (d == 64)
    hipLaunchKernelGGL(widen_kernel<64>, grid, dim3(64), 0, stream, src, dst, gs, gd,
                       src_tiles_per_seq, ntiles);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kvq
