// Read-only streaming probe: the bandwidth a plain, well-formed read of device memory
// reaches on this GPU, measured as context for the roofline of the cache-reading
// kernels (it performs none of the codec's work).
//
// Each thread issues four 16-byte loads per iteration, grid-stride (a wave reads 1 KiB
// contiguous per load instruction), and folds what it read into an XOR; the result is
// stored only when it equals a fixed constant, so the loads cannot be dropped and
// practically nothing is written.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace {

constexpr int kProbeThreads = 256;
constexpr uint32_t kProbeMagic = 0x9E3779B9u;

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const uint4* __restrict__ p,
                                                                   size_t n16, uint32_t* sink) {
  uint32_t acc = 0u;
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
    acc ^= c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == kProbeMagic) sink[threadIdx.x & 63] = acc;
}

}  // namespace

extern "C" kvq_status kvq_probe_read(const void* buf, size_t bytes, void* sink, void* stream) {
  if (!buf || !sink || ((uintptr_t)buf & 15) || (bytes & 15) || ((uintptr_t)sink & 3))
    return KVQ_ERR_INVALID_ARGUMENT;
  if (bytes == 0) return KVQ_OK;
  const size_t n16 = bytes / 16;
  // 16 workgroups per compute unit (256 CUs) at most; fewer when the buffer is small
  const size_t per_block = (size_t)kProbeThreads * 4;
  size_t blocks = (n16 + per_block - 1) / per_block;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0,
                     (hipStream_t)stream, static_cast<const uint4*>(buf), n16,
                     static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_ERR_HIP;
}
