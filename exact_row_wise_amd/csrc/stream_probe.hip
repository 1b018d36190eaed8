// stream_probe.hip -- a plain streaming read of device memory, to measure
// the HBM read rate a trivial kernel reaches (the measured roofline of the
// top-k kernels) and to evict earlier inputs from the Infinity Cache before a
// timed region.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "libtopk_probe.h"

namespace {

constexpr int kNT = 256;

// One 16-byte vector per lane; the XOR of its words decides a store that the
// caller's zero fill never triggers, so the loads are kept and nothing is
// written.
__global__ __launch_bounds__(kNT) void stream_read16(const uint4* __restrict__ src, uint64_t nvec,
                                                     uint32_t* __restrict__ sink) {
  const uint64_t i = (uint64_t)blockIdx.x * kNT + threadIdx.x;
  const uint4 v = i < nvec ? src[i] : make_uint4(0u, 0u, 0u, 0u);
  const uint32_t x = v.x ^ v.y ^ v.z ^ v.w;
  if (x == 0x9E3779B9u) sink[threadIdx.x] = x;
}

}  // namespace

extern "C" int topk_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink,
                                      void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || bytes > (int64_t(1) << 40)) return -1;
  if (bytes == 0) return 0;
  if (!src || !sink || ((uintptr_t)src & 15u) != 0) return -1;
  const uint64_t nvec = (uint64_t)bytes / 16;
  const uint64_t grid = (nvec + kNT - 1) / kNT;
  if (grid > 0x7FFFFFFFull) return -1;
  hipLaunchKernelGGL(stream_read16, dim3((unsigned)grid), dim3(kNT), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const uint4*>(src),
                     nvec, sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
