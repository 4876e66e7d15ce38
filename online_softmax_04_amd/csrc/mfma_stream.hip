// A stream of 32x32x16 bf16 MFMAs with operands held in registers: what the
// matrix units sustain chip-wide when nothing else runs.  The attention forward
// is a dense contraction ("Online Softmax: Tiling Across a Reduction", the
// matrix-unit paragraphs), and on this part the rate the matrix units hold
// depends on the operand data: with operands that switch many bits the power
// draw lowers the clock.  Benchmarks time this kernel on operands drawn like
// the attention inputs and report the attention rate against it beside the
// published peak.
//
// Each workgroup of 8 waves (two per SIMD) streams iters x 8 MFMAs per wave into
// four accumulators.  A wave reads its 16 operand fragments (8 A, 8 B; 16 bytes
// per lane each, a lane's 16 fragments contiguous) from one of kVariants operand
// sets, picked by its global wave index, and writes the sum of its accumulators
// per lane to out.  The sustained rate depends on the compiled code beyond the
// loop's instructions: the same loop with the fragments read fragment-major
// (another register assignment) ran 15-25% slower chip-wide, on zero operands
// as well, which a hand-placed assembly loop did not reproduce.
#include "common.h"
#include "kernels.h"
#include "mfma_tile.h"

namespace osm {
namespace {

constexpr int kStreamThreads = 512;

__global__ __launch_bounds__(kStreamThreads) void mfma_stream(const u32x4* __restrict__ operands,
                                                               float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * (kStreamThreads / 64) + (threadIdx.x >> 6);
  const u32x4* src = operands + (size_t)(gw % kMfmaStreamVariants) * kMfmaStreamFragments * 64;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = __builtin_bit_cast(bf16x8, src[lane * kMfmaStreamFragments + j]);
    b[j] = __builtin_bit_cast(bf16x8, src[lane * kMfmaStreamFragments + 8 + j]);
  }
  f32x16 c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) c[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
    // consecutive MFMAs differ in both operands and in the accumulator
#pragma unroll
    for (int k = 0; k < 8; ++k)
      c[k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[(3 * k + 1) & 7], c[k & 3], 0, 0, 0);
  }
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc += c[j][r];
  out[(size_t)blockIdx.x * kStreamThreads + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_mfma_stream(const void* operands, float* out, int blocks, int iters,
                              hipStream_t stream) {
  const u32x4* op = static_cast<const u32x4*>(operands);
  void* args[] = {(void*)&op, (void*)&out, (void*)&iters};
  return hipLaunchKernel((const void*)mfma_stream, dim3(blocks), dim3(kStreamThreads), args, 0,
                         stream);
}

}  // namespace osm
