// Tile helpers shared by the attention kernels (gfx950, wave64): buffer
// descriptors, the 32x32x16 and 16x16x32 MFMAs for 16-bit operands, 16-bit packing, the LDS
// chunk swizzles and the direct global-to-LDS load.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace osm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format,
// no swizzle): out-of-range loads return zero and out-of-range stores are dropped.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kBufferWord3);
}

template <typename T>
struct Mma;
template <>
struct Mma<__bf16> {
  using v8 = bf16x8;
  static __device__ __forceinline__ f32x16 run(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // 16x16x32: lane l holds row (A) / column (B) l % 16 and 8 k values of group
  // l / 16; accumulator register r of lane l is element (4 (l / 16) + r, l % 16)
  static __device__ __forceinline__ f32x4v run16(v8 a, v8 b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mma<_Float16> {
  using v8 = f16x8;
  static __device__ __forceinline__ f32x16 run(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4v run16(v8 a, v8 b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

template <typename T>
__device__ __forceinline__ unsigned pack2(float a, float b) {
  return (unsigned)__builtin_bit_cast(unsigned short, (T)a) |
         ((unsigned)__builtin_bit_cast(unsigned short, (T)b) << 16);
}

// 16-byte chunk swizzles of the K and V tiles in LDS (rows of D bf16/fp16
// values, unpadded): physical chunk = logical chunk ^ swizzle(row).  They make
// the MFMA operand reads conflict-free on gfx950's LDS: K is read as 16-byte
// pieces of 32 consecutive rows at one chunk position, V through transposed
// 8-byte reads of 4 consecutive rows x 32 bytes per 16 lanes.
template <int D>
__device__ __forceinline__ int kswz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int vswz(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// One wave-wide buffer load straight into LDS: lane i's 16 bytes (at byte
// offset voff of the buffer) land at lds + 16 i.  Kept out of the kernel
// templates: used in a template body, this builtin makes the host pass drop
// the kernel's launch stub.
__device__ __forceinline__ void load16_to_lds(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}

// s_waitcnt with only the vector-memory count set (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt and lgkmcnt left at their maxima).  Unlike the
// same instruction in inline assembly, the compiler sees it and knows which
// direct-to-LDS loads it retires.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// The same with the non-temporal cache policy (gfx940-family NT bit), for data
// read exactly once: it streams past the caches instead of displacing reused lines.
__device__ __forceinline__ void load16_to_lds_nt(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 2);
}

// The same for 4 bytes per lane: lane i's word lands at lds + 4 i.
__device__ __forceinline__ void load4_to_lds(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voff, 0, 0, 0);
}

// A compile-time stage index for double-buffered LDS tiles.  Kernels keep one
// __shared__ array per stage and name it through this tag: the compiler tracks
// pending direct-to-LDS loads per array, so with the stage known at compile time
// a read of one stage does not wait for the loads into the other.
template <int S>
struct StageTag {
  static constexpr int value = S;
};

// Direct loads write LDS behind the compiler's back: wait for all of this
// wave's vector-memory operations explicitly before publishing.
__device__ __forceinline__ void vmem_landed() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace osm
