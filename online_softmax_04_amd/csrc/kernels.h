// Internal launchers of the HIP library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

namespace osm {

enum class Elem { bf16, f16, f32 };

// Attention forward on `stream`; arguments already validated by the C ABI layer.
hipError_t launch_attn_fwd(Elem elem, const void* q, const void* k, const void* v, void* o,
                           float* lse, int B, int H, int N, int d, float scale, bool causal,
                           hipStream_t stream);
hipError_t attn_fwd_attributes(Elem elem, int d, bool causal, hipFuncAttributes* attr,
                               int* threads, int* blocks_per_cu);

// Row softmax on `stream`; vec_ok = 16-byte aligned pointers and cols % 4 == 0.
hipError_t launch_softmax(const float* x, float* y, int rows, int cols, bool vec_ok,
                          hipStream_t stream);
hipError_t softmax_attributes(int cols, bool vec_ok, hipFuncAttributes* attr, int* threads,
                              int* blocks_per_cu);

}  // namespace osm
