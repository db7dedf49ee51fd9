// Streaming-read probe: the HBM read bandwidth reachable with the load shape
// the decode kernels use (16-byte loads, eight in flight per lane, full
// device grid).  A measurement aid for the roofline, not part of the method.
#include "ekv_device.h"
#include "ekv_kernels.h"

namespace ekv {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocks = EKV_READ_PROBE_SINK / (kProbeThreads / kWave);

__global__ __launch_bounds__(kProbeThreads) void k_read_probe(
    const uint4 *__restrict__ p, size_t n, uint32_t *__restrict__ sink) {
  constexpr int U = 8;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int k = 0; k < U; ++k) v[k] = p[i + k * stride];
#pragma unroll
    for (int k = 0; k < U; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n; i += stride) {
    const uint4 v = p[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0)
    sink[blockIdx.x * (kProbeThreads / kWave) + threadIdx.x / kWave] = acc;
}

hipError_t launch_read_probe(const void *buf, size_t bytes, uint32_t *sink,
                             hipStream_t stream) {
  hipLaunchKernelGGL(k_read_probe, dim3(kProbeBlocks), dim3(kProbeThreads), 0,
                     stream, static_cast<const uint4 *>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace ekv
