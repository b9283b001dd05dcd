// Measurement helper: a plain streaming read of device memory, the ceiling
// the HBM-bound expert kernels are compared against on the same GPU.
#include <hip/hip_runtime.h>

#include "../../include/ds4moe.h"
#include "common.h"
#include "launch.h"

namespace ds4 {

constexpr int kReadThreads = 256;
constexpr int kReadDepth = 8;  // 16-byte loads in flight per thread

// Every thread folds the 16-byte vectors of a grid-stride loop, kReadDepth at
// a time, into one XOR; each workgroup writes one word, so no load is dead.
__global__ __launch_bounds__(kReadThreads) void k_stream_read(const u4 *__restrict__ p, uint64_t n16,
                                                              uint32_t *__restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * kReadThreads;
  uint64_t i = (uint64_t)blockIdx.x * kReadThreads + threadIdx.x;
  u4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kReadDepth - 1) * stride < n16; i += kReadDepth * stride) {
    u4 v[kReadDepth];
#pragma unroll
    for (int j = 0; j < kReadDepth; ++j) v[j] = p[i + j * stride];
#pragma unroll
    for (int j = 0; j < kReadDepth; ++j) acc ^= v[j];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  uint32_t r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  __shared__ uint32_t red[kReadThreads / 64];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) r ^= (uint32_t)__shfl_xor((int)r, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = r;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace ds4

extern "C" int ds4moe_read_probe(const void *buf, size_t bytes, int32_t n_workgroups, uint32_t *sink,
                                 void *start_event, void *stop_event, void *stream) {
  if (!buf || !sink) return DS4MOE_ERR_NULL;
  if (bytes == 0 || bytes % 16 || n_workgroups < 1 || n_workgroups > (1 << 20)) return DS4MOE_ERR_SHAPE;
  if ((uintptr_t)buf % 16 || (uintptr_t)sink % 4) return DS4MOE_ERR_ALIGN;
  if ((start_event == nullptr) != (stop_event == nullptr)) return DS4MOE_ERR_NULL;
  ds4::Timing t{(hipEvent_t)start_event, (hipEvent_t)stop_event};
  const ds4::Timing *tm = start_event ? &t : nullptr;
  DS4_LAUNCH(tm, ds4::k_stream_read, dim3(n_workgroups), dim3(ds4::kReadThreads), 0, (hipStream_t)stream,
             (const u4 *)buf, (uint64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? DS4MOE_OK : DS4MOE_ERR_HIP;
}
