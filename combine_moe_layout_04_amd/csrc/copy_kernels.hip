// Plain device copy: the reference kernel for calibrating HBM traffic
// counters against a known byte count, and for measuring the achievable HBM
// rate of a streaming kernel next to the spec peak.  Not part of the method.
//
// One 16-byte chunk per thread and no loop: a grid-stride loop over a large
// buffer measured about 10% slower than a grid that covers it once.
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void copy_kernel(u32x4* __restrict__ dst,
                                                   const u32x4* __restrict__ src, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

}  // namespace

hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  if (blocks > 0xFFFFFFFFull) return hipErrorInvalidValue;  // one grid dimension
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), n);
  return hipGetLastError();
}

}  // namespace moe
