// Single-wave probes of the gfx950 instruction behaviour the attention kernels
// rely on, for tests/test_layout_probe.py (test infrastructure; the library
// never loads this file's code).  Each entry point launches one 64-lane
// workgroup on the given device buffers (sizes fixed and stated below) and
// returns the launch status; the test compares the outputs with what the
// kernels assume.
//
//  * mfma_bf16_probe: D = A B on v_mfma_f32_32x32x16_bf16 with lane l holding row
//    l % 32 of A and column l % 32 of B, 8 consecutive k from 8 (l / 32); writes
//    each lane's 16 accumulator values.  A [32][16], B [16][32] bf16 bits (row
//    major), out [64][16] fp32.
//  * mfma16_bf16_probe: D = A B on v_mfma_f32_16x16x32_bf16 with lane l holding
//    row l % 16 of A and column l % 16 of B, 8 consecutive k from 8 (l / 16);
//    writes each lane's 4 accumulator values.  A [16][32], B [32][16] bf16 bits
//    (row major), out [64][4] fp32.
//  * permlane32_probe: v_permlane32_swap with both operands x; in [64] u32,
//    out [2][64] u32 (result halves 0 and 1 per lane).
//  * ds_read_tr16_probe: LDS filled with in [64][64] u16 (row major); lane l
//    reads ds_read_b64_tr_b16 at the byte offset addr[l]; out [64][4] u16.
//  * mfma_fp8_probe: D = A B on the 32x32x64 fp8 MFMA (E4M3 A and B, no scales)
//    with lane l holding row (column) l % 32 and 32 consecutive k from
//    32 (l / 32); A [32][64], B [64][32] E4M3 codes, out [64][16] fp32.
//  * cvt_fp8_probe: v_cvt_pk_fp8_f32 of in [64][4] fp32 into 4 E4M3 codes per
//    lane; out [64][4] u8.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8p __attribute__((ext_vector_type(8)));
typedef float f32x16p __attribute__((ext_vector_type(16)));
typedef float f32x4p __attribute__((ext_vector_type(4)));
typedef short s16x4p __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4p lds_s16x4p;
typedef int i32x8p __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(64) void k_mfma_bf16(const uint16_t* A, const uint16_t* B, float* out) {
  const int l = threadIdx.x, r = l % 32, kb = 8 * (l / 32);
  bf16x8p a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = __builtin_bit_cast(__bf16, A[r * 16 + kb + i]);
    b[i] = __builtin_bit_cast(__bf16, B[(kb + i) * 32 + r]);
  }
  f32x16p c = {};
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  for (int i = 0; i < 16; ++i) out[l * 16 + i] = c[i];
}

__global__ __launch_bounds__(64) void k_mfma16_bf16(const uint16_t* A, const uint16_t* B, float* out) {
  const int l = threadIdx.x, r = l % 16, kb = 8 * (l / 16);
  bf16x8p a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = __builtin_bit_cast(__bf16, A[r * 32 + kb + i]);
    b[i] = __builtin_bit_cast(__bf16, B[(kb + i) * 16 + r]);
  }
  f32x4p c = {};
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  for (int i = 0; i < 4; ++i) out[l * 4 + i] = c[i];
}

__global__ __launch_bounds__(64) void k_permlane32(const unsigned* in, unsigned* out) {
  const int l = threadIdx.x;
  const unsigned x = in[l];
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  out[l] = (unsigned)r[0];
  out[64 + l] = (unsigned)r[1];
}

__global__ __launch_bounds__(64) void k_ds_read_tr16(const uint16_t* in, const int* addr, uint16_t* out) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[64 * 64];
  const int l = threadIdx.x;
  for (int i = l; i < 64 * 64; i += 64) lds[i] = in[i];
  __syncthreads();
  const int a = addr[l] & (64 * 64 * 2 - 8);  // inside the array, 8-byte aligned
  const s16x4p v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4p*)((unsigned char*)lds + a));
  for (int i = 0; i < 4; ++i) out[l * 4 + i] = (uint16_t)v[i];
}

__global__ __launch_bounds__(64) void k_mfma_fp8(const uint8_t* A, const uint8_t* B, float* out) {
  const int l = threadIdx.x, r = l % 32, kb = 32 * (l / 32);
  i32x8p a, b;
  for (int w = 0; w < 8; ++w) {
    unsigned ua = 0, ub = 0;
    for (int i = 0; i < 4; ++i) {
      ua |= (unsigned)A[r * 64 + kb + 4 * w + i] << (8 * i);
      ub |= (unsigned)B[(kb + 4 * w + i) * 32 + r] << (8 * i);
    }
    a[w] = (int)ua;
    b[w] = (int)ub;
  }
  f32x16p c = {};
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  // the fp8 MFMA's results are read only after enough wait states
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 15\n s_nop 15" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  for (int i = 0; i < 16; ++i) out[l * 16 + i] = c[i];
}

__global__ __launch_bounds__(64) void k_cvt_fp8(const float* in, uint8_t* out) {
  const int l = threadIdx.x;
  int x = __builtin_amdgcn_cvt_pk_fp8_f32(in[4 * l], in[4 * l + 1], 0, false);
  x = __builtin_amdgcn_cvt_pk_fp8_f32(in[4 * l + 2], in[4 * l + 3], x, true);
  for (int i = 0; i < 4; ++i) out[4 * l + i] = (uint8_t)((unsigned)x >> (8 * i));
}

extern "C" {
int mfma_bf16_probe(const void* A, const void* B, void* out) {
  hipLaunchKernelGGL(k_mfma_bf16, dim3(1), dim3(64), 0, 0, (const uint16_t*)A, (const uint16_t*)B, (float*)out);
  return (int)hipGetLastError();
}
int mfma16_bf16_probe(const void* A, const void* B, void* out) {
  hipLaunchKernelGGL(k_mfma16_bf16, dim3(1), dim3(64), 0, 0, (const uint16_t*)A, (const uint16_t*)B, (float*)out);
  return (int)hipGetLastError();
}
int permlane32_probe(const void* in, void* out) {
  hipLaunchKernelGGL(k_permlane32, dim3(1), dim3(64), 0, 0, (const unsigned*)in, (unsigned*)out);
  return (int)hipGetLastError();
}
int ds_read_tr16_probe(const void* in, const void* addr, void* out) {
  hipLaunchKernelGGL(k_ds_read_tr16, dim3(1), dim3(64), 0, 0, (const uint16_t*)in, (const int*)addr,
                     (uint16_t*)out);
  return (int)hipGetLastError();
}
int mfma_fp8_probe(const void* A, const void* B, void* out) {
  hipLaunchKernelGGL(k_mfma_fp8, dim3(1), dim3(64), 0, 0, (const uint8_t*)A, (const uint8_t*)B, (float*)out);
  return (int)hipGetLastError();
}
int cvt_fp8_probe(const void* in, void* out) {
  hipLaunchKernelGGL(k_cvt_fp8, dim3(1), dim3(64), 0, 0, (const float*)in, (uint8_t*)out);
  return (int)hipGetLastError();
}
}
