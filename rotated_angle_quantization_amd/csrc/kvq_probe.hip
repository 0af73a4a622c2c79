// Read-only streaming probe: the bandwidth a plain, well-formed read of device memory
// reaches on this GPU, measured as context for the roofline of the cache-reading
// kernels (it performs none of the codec's work).
//
// Each wave reads its own contiguous 8 KiB chunk (512 16-byte words): eight 16-byte
// loads per lane in flight, a wave's load instruction covering 1 KiB contiguous, and
// folds what it read into an XOR; the result is stored only when it equals a fixed
// constant, so the loads cannot be dropped and practically nothing is written. Word k is
// read by wave k / 512 at lane k % 64. Of the patterns timed on MI355X (grid-stride
// loops over 4,096 to 65,536 workgroups; per-wave chunks of 4 KiB to 256 KiB with four
// or eight loads in flight) this one read fastest.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace {

constexpr int kProbeThreads = 256;
constexpr int kChunk16 = 512;  // 16-byte words per wave
constexpr int kInFlight = 8;   // loads per lane per round
constexpr uint32_t kProbeMagic = 0x9E3779B9u;

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const uint4* __restrict__ p,
                                                                   size_t n16, uint32_t* sink) {
  uint32_t acc = 0u;
  const size_t base = ((size_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)) * kChunk16;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < kChunk16; i += 64 * kInFlight) {
    uint4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const size_t k = base + i + u * 64 + lane;
      v[u] = k < n16 ? p[k] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == kProbeMagic) sink[threadIdx.x & 63] = acc;
}

}  // namespace

extern "C" kvq_status kvq_probe_read(const void* buf, size_t bytes, void* sink, void* stream) {
  if (!buf || !sink || ((uintptr_t)buf & 15) || (bytes & 15) || ((uintptr_t)sink & 3))
    return KVQ_ERR_INVALID_ARGUMENT;
  if (bytes == 0) return KVQ_OK;
  const size_t n16 = bytes / 16;
  const size_t per_block = (size_t)(kProbeThreads / 64) * kChunk16;
  const size_t blocks = (n16 + per_block - 1) / per_block;
  if (blocks > 0x7fffffffULL) return KVQ_ERR_INVALID_ARGUMENT;
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0,
                     (hipStream_t)stream, static_cast<const uint4*>(buf), n16,
                     static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}
