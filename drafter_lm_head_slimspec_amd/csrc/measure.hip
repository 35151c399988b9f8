// Measurement helper (not a step of the method): the attainable HBM read rate of this part,
// the second denominator of the streaming kernels' roofline next to the 8 TB/s peak.
//   k_read_probe   1024 workgroups of 256 threads stride over the buffer in 16-byte loads,
//                  four in flight per thread (the flat order, so that at any moment the grid
//                  reads one contiguous window); every 32-bit word is folded into one XOR per
//                  workgroup, added to *sink with a device atomic, so no load can be dropped
//                  and the result is the same in any order.
#include <hip/hip_ext.h>

#include "device_common.h"
#include "launch.h"
#include "trace.h"

namespace sh {

namespace {
constexpr int kProbeThreads = 256;
constexpr int kProbeGrid = 1024;
constexpr int kProbeUnroll = 4;
}  // namespace

__global__ __launch_bounds__(kProbeThreads) void k_read_probe(const void* __restrict__ buf, uint32_t bytes,
                                                            uint32_t* __restrict__ sink) {
  const rsrc_t rs = make_rsrc(buf, bytes);
  const uint32_t stride = gridDim.x * kProbeThreads * 16u;
  uint32_t acc = 0u;
  for (uint32_t off = (blockIdx.x * kProbeThreads + threadIdx.x) * 16u; off < bytes;
       off += stride * kProbeUnroll) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const uint32_t o = off + u * stride;   // past `bytes` the descriptor returns zeros
      v[u] = buffer_load16(rs, o < bytes ? o : kOutOfRange);
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) acc ^= __shfl_xor(acc, s);
  __shared__ uint32_t wacc[kProbeThreads / kWave];
  if (lane_id() == 0) wacc[wave_id()] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0u;
    for (int w = 0; w < kProbeThreads / kWave; ++w) t ^= wacc[w];
    atomicXor(sink, t);
  }
}

hipError_t launch_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t st) {
  if (bytes == 0 || bytes % 16 != 0 || bytes > 0xFFFFFFF0ull) return hipErrorInvalidValue;
  TraceScope ts("read_probe", st, true);
  hipExtLaunchKernelGGL(k_read_probe, dim3(kProbeGrid), dim3(kProbeThreads), 0, st, ts.start(), ts.stop(), 0, buf,
                        static_cast<uint32_t>(bytes), sink);
  return hipGetLastError();
}

}  // namespace sh
