// Device-to-device copy with 16-byte non-temporal loads and stores: the
// practical HBM ceiling of a streaming kernel on this part.  The row softmax
// moves one read and one write per byte as well ("5.2 CUDA Online Softmax",
// section 6: one read and one write is the floor of a register-cached row), so
// this copy, timed in the same run, is what its bandwidth is compared with
// beside the published peak.  It is also the kernel of known size that
// calibrates the byte counters of a profile.
//
// Each workgroup of 256 threads copies one 16 KiB chunk: every thread issues
// its four 16-byte loads before its four stores, so a wave keeps 4 KiB in
// flight, and each load or store instruction of a wave covers 1 KiB of
// contiguous memory.
#include "common.h"
#include "kernels.h"

namespace osm {
namespace {

typedef unsigned u32x4c __attribute__((ext_vector_type(4)));
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(kCopyThreads) void stream_copy(const u32x4c* __restrict__ x,
                                                             u32x4c* __restrict__ y, size_t n16) {
  const size_t base = (size_t)blockIdx.x * (kCopyThreads * kCopyUnroll) + threadIdx.x;
  u32x4c v[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const size_t i = base + (size_t)u * kCopyThreads;
    if (i < n16) v[u] = __builtin_nontemporal_load(x + i);
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const size_t i = base + (size_t)u * kCopyThreads;
    if (i < n16) __builtin_nontemporal_store(v[u], y + i);
  }
}

}  // namespace

uint64_t stream_copy_blocks(uint64_t bytes) {
  const uint64_t per = (uint64_t)kCopyThreads * kCopyUnroll * 16;
  return (bytes + per - 1) / per;
}

hipError_t launch_stream_copy(const void* x, void* y, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  const u32x4c* xp = static_cast<const u32x4c*>(x);
  u32x4c* yp = static_cast<u32x4c*>(y);
  void* args[] = {(void*)&xp, (void*)&yp, (void*)&n16};
  return hipLaunchKernel((const void*)stream_copy, dim3((unsigned)stream_copy_blocks(bytes)),
                         dim3(kCopyThreads), args, 0, stream);
}

}  // namespace osm
