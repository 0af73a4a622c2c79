// Encode (append) kernel: x -> sign diagonal -> normalised fast Walsh-Hadamard
// transform -> pairs -> (radius, angle) -> codes -> bit-packed tile planes.
//
// Method: "TurboAngle: Near-Lossless KV Cache Compression via Uniform Angle
// Quantization" (arXiv 2603.27467), Abstract. Readings (bin placement, ties, fp16
// parameters, log-radius floor) are documented with kvq_encode in kvq.h.
//
// Every decision that turns a real number into an integer (angle bin, radius level,
// fp16 rounding of the per-vector parameters) is taken in IEEE binary64, so the codes
// do not depend on launch shape and agree with a float64 reference except where an
// angle falls within rounding distance of a bin boundary.
//
// Work split: one 64-lane wave per (batch, kv head, tile of 64 tokens). A lane owns
// one coordinate pair of a vector (d = 128: one vector per step; d = 64: two vectors
// per step, one per half-wave), so the transform's first stage is in-lane and the
// others are cross-lane exchanges. Codes of the whole tile are staged in LDS as bytes
// and then packed: key planes with one lane per token, value planes with one lane
// per pair, matching the layout's word order so every store is a coalesced dword.
#include <hip/hip_fp16.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr double kFp16Max = 65504.0;
constexpr double kFp16MinNormal = 6.103515625e-05;  // 2^-14
constexpr double kFp16Subnormal = 5.9604644775390625e-08;  // 2^-24

// Nearest fp16 value of a non-negative x <= 65504, ties to even, computed exactly in
// binary64: the fp16 spacing at x is 2^(e-10) (2^-24 below the normal range), so
// rint(x / q) * q rounds to 11 significant bits with no double rounding.
__device__ __forceinline__ double fp16_round_pos(double x) {
  if (x == 0.0) return 0.0;
  const double q = x < kFp16MinNormal ? kFp16Subnormal : ldexp(1.0, ilogb(x) - 10);
  return rint(x / q) * q;
}

__device__ __forceinline__ uint16_t fp16_bits(double exact_fp16_value) {
  return __half_as_ushort(__float2half_rn((float)exact_fp16_value));
}

__device__ __forceinline__ bool sign_neg(const SignMask& m, int e) {
  return (m.w[e >> 6] >> (e & 63)) & 1ull;
}

// In-place Walsh-Hadamard transform of one vector held as (a, b) = elements
// (2p, 2p+1) in lane p of a P-lane group: stage h = 1 is in-lane, stage h = 2m pairs
// lane p with lane p ^ m. Natural (Sylvester) output order.
template <int P>
__device__ __forceinline__ void fwht_pairs(double& a, double& b, int p) {
  const double s = a + b, t = a - b;
  a = s;
  b = t;
#pragma unroll
  for (int m = 1; m < P; m <<= 1) {
    const double pa = __shfl_xor(a, m), pb = __shfl_xor(b, m);
    if (p & m) {
      a = pa - a;
      b = pb - b;
    } else {
      a = a + pa;
      b = b + pb;
    }
  }
}

template <int P>
__device__ __forceinline__ double group_max(double x) {
#pragma unroll
  for (int m = 1; m < P; m <<= 1) x = fmax(x, __shfl_xor(x, m));
  return x;
}

template <int P>
__device__ __forceinline__ double group_min(double x) {
#pragma unroll
  for (int m = 1; m < P; m <<= 1) x = fmin(x, __shfl_xor(x, m));
  return x;
}

// Uniform angle quantiser: nearest of n centres 2 pi c / n; zero pair -> 0.
__device__ __forceinline__ int angle_code(double r, double theta, double bins_per_rad, int n) {
  if (r == 0.0) return 0;
  int c = (int)floor(theta * bins_per_rad + 0.5);
  c %= n;
  if (c < 0) c += n;
  return c;
}

__device__ __forceinline__ void load_pair(const void* base, bool f32, int64_t off, double& x0,
                                          double& x1) {
  if (f32) {
    const float2 v = *reinterpret_cast<const float2*>(static_cast<const float*>(base) + off);
    x0 = v.x;
    x1 = v.y;
  } else {
    const __half2 v = *reinterpret_cast<const __half2*>(static_cast<const __half*>(base) + off);
    x0 = __half2float(__low2half(v));
    x1 = __half2float(__high2half(v));
  }
}

constexpr int kRow = 68;  // LDS row stride (bytes) of the per-token code staging

template <int D>
__global__ __launch_bounds__(64) void encode_kernel(CodecArgs a, TileGeom g,
                                                    uint8_t* __restrict__ cache,
                                                    const void* __restrict__ kin,
                                                    const void* __restrict__ vin, int f32_in,
                                                    int64_t sb, int64_t st, int64_t sh) {
  constexpr int P = D / 2;
  constexpr int VPW = 64 / P;  // vectors per wave step
  __shared__ uint8_t s_kc[kTile][kRow], s_kr[kTile][kRow], s_vc[kTile][kRow], s_vr[kTile][kRow];
  __shared__ uint16_t s_ks[kTile];
  __shared__ uint32_t s_vp[kTile];

  const int lane = threadIdx.x;
  const int tile_rel = blockIdx.x % a.tiles_touched;
  const int bh = blockIdx.x / a.tiles_touched;
  const int b = bh / a.hkv, h = bh % a.hkv;
  const int tile = a.tile_lo + tile_rel;
  const int tok_base = tile * kTile;
  const int j_lo = max(a.t0 - tok_base, 0);
  const int j_hi = min(a.t0 + a.ntok - tok_base, kTile);

  const int p = lane % P;    // pair index within the vector
  const int sub = lane / P;  // which vector of the wave step
  const int e0 = 2 * p;
  const double sg0 = sign_neg(a.sign, e0) ? -1.0 : 1.0;
  const double sg1 = sign_neg(a.sign, e0 + 1) ? -1.0 : 1.0;

  for (int jb = j_lo; jb < j_hi; jb += VPW) {
    const int j = jb + sub;
    const bool act = j < j_hi;
    double k0 = 0.0, k1 = 0.0, v0 = 0.0, v1 = 0.0;
    if (act) {
      const int64_t off =
          (int64_t)b * sb + (int64_t)(tok_base + j - a.t0) * st + (int64_t)h * sh + e0;
      load_pair(kin, f32_in, off, k0, k1);
      load_pair(vin, f32_in, off, v0, v1);
    }
    // keys
    k0 *= sg0;
    k1 *= sg1;
    fwht_pairs<P>(k0, k1, p);
    k0 *= a.inv_sqrt_d;
    k1 *= a.inv_sqrt_d;
    const double kr = hypot(k0, k1);
    const int kc = angle_code(kr, atan2(k1, k0), a.k_bins_per_rad, a.n_k);
    const double ks = fp16_round_pos(fmin(group_max<P>(kr), kFp16Max));
    int krho = 0;
    if (ks > 0.0) krho = (int)fmin(fmax(floor(255.0 * kr / ks + 0.5), 0.0), 255.0);
    // values
    v0 *= sg0;
    v1 *= sg1;
    fwht_pairs<P>(v0, v1, p);
    v0 *= a.inv_sqrt_d;
    v1 *= a.inv_sqrt_d;
    const double vr = hypot(v0, v1);
    const int vc = angle_code(vr, atan2(v1, v0), a.v_bins_per_rad, a.n_v);
    const double vmax = group_max<P>(vr), vmin = group_min<P>(vr);
    const double smax = fp16_round_pos(fmin(vmax, kFp16Max));
    const double smin = fp16_round_pos(fmin(fmax(vmin, kFp16MinNormal), kFp16Max));
    int vrho = 0;
    if (smax > smin && vr >= smin) {
      const double lam = log(smax / smin);
      vrho = (int)fmin(fmax(floor(15.0 * log(vr / smin) / lam + 0.5), 0.0), 15.0);
    }
    if (act) {
      s_kc[j][p] = (uint8_t)kc;
      s_kr[j][p] = (uint8_t)krho;
      s_vc[j][p] = (uint8_t)vc;
      s_vr[j][p] = (uint8_t)vrho;
      if (p == 0) {
        s_ks[j] = fp16_bits(ks);
        s_vp[j] = (uint32_t)fp16_bits(smin) | ((uint32_t)fp16_bits(smax) << 16);
      }
    }
  }
  __syncthreads();

  uint8_t* tp = cache + ((size_t)(b * a.hkv + h) * a.tiles_per_seq + tile) * (size_t)g.bytes;

  // Key planes and per-token parameters: one lane per token slot; slots outside the
  // range are not written (their words belong to them alone).
  {
    const int t = lane;
    if (t >= j_lo && t < j_hi) {
      uint32_t* ka = reinterpret_cast<uint32_t*>(tp + g.ka);
      uint64_t acc = 0;
      int nb = 0, w = 0;
      for (int i = 0; i < P; ++i) {
        acc |= (uint64_t)s_kc[t][i] << nb;
        nb += a.bk;
        if (nb >= 32) {
          ka[w * kTile + t] = (uint32_t)acc;
          acc >>= 32;
          nb -= 32;
          ++w;
        }
      }
      uint32_t* kr = reinterpret_cast<uint32_t*>(tp + g.kr);
      for (int w4 = 0; w4 < P / 4; ++w4) {
        const uint32_t word = (uint32_t)s_kr[t][4 * w4] | ((uint32_t)s_kr[t][4 * w4 + 1] << 8) |
                              ((uint32_t)s_kr[t][4 * w4 + 2] << 16) |
                              ((uint32_t)s_kr[t][4 * w4 + 3] << 24);
        kr[w4 * kTile + t] = word;
      }
      reinterpret_cast<uint16_t*>(tp + g.ks)[t] = s_ks[t];
      reinterpret_cast<uint32_t*>(tp + g.vp)[t] = s_vp[t];
    }
  }

  // Value planes: one lane per pair. A word shared with slots outside the range is
  // merged with the bits already stored (this wave owns the whole tile here).
  if (lane < P) {
    const int i = lane;
    uint32_t* va = reinterpret_cast<uint32_t*>(tp + g.va);
    uint32_t* vrw = reinterpret_cast<uint32_t*>(tp + g.vr);
    uint64_t acc = 0, macc = 0;
    int nb = 0, w = 0;
    const uint64_t cmask = (1ull << a.bv) - 1;
    for (int t = 0; t < kTile; ++t) {
      const bool in = t >= j_lo && t < j_hi;
      acc |= (uint64_t)(in ? s_vc[t][i] : 0) << nb;
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
          word |= (uint32_t)s_vr[t][i] << (4 * q);
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

}  // namespace

hipError_t launch_encode(const CodecArgs& a, int d, TileGeom geom, uint8_t* cache,
                         const void* k, const void* v, bool f32_in, int64_t sb, int64_t st,
                         int64_t sh, hipStream_t stream) {
  const long long blocks = (long long)a.batch * a.hkv * a.tiles_touched;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(64);
  if (d == 64)
    hipLaunchKernelGGL(encode_kernel<64>, grid, block, 0, stream, a, geom, cache, k, v,
                       (int)f32_in, sb, st, sh);
  else if (d == 128)
    hipLaunchKernelGGL(encode_kernel<128>, grid, block, 0, stream, a, geom, cache, k, v,
                       (int)f32_in, sb, st, sh);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kvq
