// A plain streaming read of device memory (measurement only; see
// include/read_probe.h).  Workgroup b reads the contiguous span
// [b * per, (b + 1) * per) of 16-byte chunks, each lane eight loads in
// flight, and folds the words it read into one value.  The store of that
// value is conditional on a constant no sum of random data will hit in
// practice, so the loads cannot be dropped and nothing is written.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "read_probe.h"

namespace {

constexpr uint32_t kNever = 0x9E3779B9u;
constexpr int kInFlight = 8;

__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ p, int64_t n16, int64_t per,
                                                         uint32_t* __restrict__ sink) {
  const int64_t beg = (int64_t)blockIdx.x * per;
  const int64_t end = beg + per < n16 ? beg + per : n16;
  uint32_t acc = 0;
  int64_t i = beg + threadIdx.x;
  for (; i + (kInFlight - 1) * 256 < end; i += kInFlight * 256) {
    uint4 v[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) v[k] = p[i + k * 256];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) acc ^= v[k].x + v[k].y + v[k].z + v[k].w;
  }
  for (; i < end; i += 256) {
    const uint4 a = p[i];
    acc ^= a.x + a.y + a.z + a.w;
  }
  if (acc == kNever) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" int32_t splitkv_read_probe(const void* buf, int64_t bytes, int32_t workgroups, void* sink,
                                      void* stream) {
  if (!buf || !sink || (uintptr_t)buf % 16 || bytes <= 0 || bytes % 16 || workgroups <= 0) return -1;
  (void)hipGetLastError();   // report this launch's status, not an earlier call's
  const int64_t n16 = bytes / 16;
  const int64_t per = (n16 + workgroups - 1) / workgroups;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream,
                     (const uint4*)buf, n16, per, (uint32_t*)sink);
  return (int32_t)hipGetLastError();
}
