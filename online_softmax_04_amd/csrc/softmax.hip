// Row-wise online softmax for gfx950.
//
// Method (infra-guide "5.2 CUDA Online Softmax"): the row maximum m and the
// sum of exponentials d are gathered in one fused pass; partial (m, d) pairs
// held by different lanes merge with the associative rule
//     m = max(m1, m2),  d = d1 * e^(m1 - m) + d2 * e^(m2 - m)      (section 4.2)
// and a second pass normalises.  Two kernels:
//
//  * softmax_cached: the whole row is held in VGPRs (section 6, "register
//    cache"), so the row is read from HBM once and written once -- the floor of
//    8 bytes per fp32 element.  Each lane caches NV f32x4 chunks; chunk i of
//    lane t is element group i*THREADS + t, so every load and store instruction
//    of a wave covers 1 KiB of contiguous memory.  Instead of the per-element
//    recurrence, a lane takes its slice as one tile: its max m_t, then
//    e = 2^((x - m_t) log2 e) kept in place of x and d_t = sum e.  After the
//    (m, d) merge, y = e * 2^((m_t - m) log2 e) / d, so no element is
//    exponentiated twice.  Loads and stores are non-temporal: every byte is
//    touched once.
//
//  * softmax_stream: rows longer than the cache, or not 16-byte aligned /
//    not a multiple of 4 columns: pass 1 runs the per-chunk online recurrence
//    while streaming the row (sections 2.2, 5), pass 2 re-reads and normalises.
//
// One workgroup per row; the grid is the row count (the hardware dispatcher
// keeps every CU fed, so no software grid-stride loop is needed).
#include "common.h"
#include "kernels.h"
#include "mfma_tile.h"

namespace osm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Merge (mo, lo) into (m, l).  A side with m = -inf carries l = 0.
__device__ __forceinline__ void merge_ml(float& m, float& l, float mo, float lo) {
  const float M = fmaxf(m, mo);
  const float Ms = (M == kNegInf) ? 0.f : M;  // both empty: keep l = 0, avoid -inf - -inf
  l = l * exp2_fast((m - Ms) * kLog2e) + lo * exp2_fast((mo - Ms) * kLog2e);
  m = M;
}

// Merge (m, l) over the workgroup; every thread returns the same pair.
template <int THREADS>
__device__ __forceinline__ void block_merge(float& m, float& l) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float mo = __shfl_xor(m, off);
    const float lo = __shfl_xor(l, off);
    merge_ml(m, l, mo, lo);  // symmetric: both partners compute the same bits
  }
  constexpr int W = THREADS / 64;
  if constexpr (W > 1) {
    __shared__ float sm[W], sl[W];
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
      sm[wave] = m;
      sl[wave] = l;
    }
    __syncthreads();
    m = sm[0];
    l = sl[0];
#pragma unroll
    for (int w = 1; w < W; ++w) merge_ml(m, l, sm[w], sl[w]);
  }
}

__device__ __forceinline__ float max4(f32x4 v) { return fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)); }

// At 1024 threads the instance is held to 64 VGPRs (8 waves per SIMD), so two
// rows are resident per compute unit; at the compiler's own choice (69) only one is.
template <int THREADS, int NV>
__global__ __launch_bounds__(THREADS)
__attribute__((amdgpu_waves_per_eu(THREADS >= 1024 ? 8 : 1, 8))) void softmax_cached(const float* __restrict__ x,
                                                          float* __restrict__ y, int cols) {
  const size_t row = blockIdx.x;
  const f32x4* xr = reinterpret_cast<const f32x4*>(x + row * (size_t)cols);
  f32x4* yr = reinterpret_cast<f32x4*>(y + row * (size_t)cols);
  const int nvec = cols >> 2;
  const int t = threadIdx.x;

  f32x4 c[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = i * THREADS + t;
    if (idx < nvec) {
      c[i] = __builtin_nontemporal_load(xr + idx);
    } else {
      c[i] = f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
    }
  }
  // the lane's slice as one tile: max, then exponentials against it
  float m = kNegInf;
#pragma unroll
  for (int i = 0; i < NV; ++i) m = fmaxf(m, max4(c[i]));
  const float m_lane = m;
  // x - m first, then the log2(e) factor: x - m <= 0, so the product can only
  // overflow towards -inf (exponential 0), even for inputs near -FLT_MAX.
  const float ms = (m == kNegInf) ? 0.f : m;  // a lane without elements keeps l = 0
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    c[i] = (c[i] - ms) * kLog2e;
    c[i].x = exp2_fast(c[i].x);
    c[i].y = exp2_fast(c[i].y);
    c[i].z = exp2_fast(c[i].z);
    c[i].w = exp2_fast(c[i].w);
    l += (c[i].x + c[i].y) + (c[i].z + c[i].w);
  }
  block_merge<THREADS>(m, l);
  // y = e * 2^((m_lane - m) log2 e) / l   (a lane without elements never stores)
  const float f = exp2_fast((m_lane - m) * kLog2e) / l;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int idx = i * THREADS + t;
    if (idx < nvec) {
      const f32x4 v = c[i] * f;
      __builtin_nontemporal_store(v, yr + idx);
    }
  }
}

// Persistent form of the register-cached kernel for many rows: one workgroup
// per compute unit walks rows blockIdx.x, blockIdx.x + gridDim.x, ... with two
// register caches, issuing the loads of its next row before it reduces,
// normalises and stores the current one, so the memory system sees no gap
// between the rows of a compute unit.  The arithmetic is softmax_cached's.
template <int THREADS, int NV>
__global__ __launch_bounds__(THREADS) void softmax_persist(const float* __restrict__ x,
                                                           float* __restrict__ y, int rows,
                                                           int cols) {
  constexpr int W = THREADS / 64;
  __shared__ float sm[2][W], sl[2][W];  // per-parity wave partials: rows r and r + 1 never share
  const int nvec = cols >> 2;
  const int t = threadIdx.x;
  f32x4 a[NV], b[NV];
  // Branch-free loads and stores through buffer descriptors bounded by the row
  // (out-of-range lanes read zeros, replaced by -inf, and their stores are
  // dropped), so the compiler can count the loads still in flight and wait
  // only for the current row's, not for the prefetched one's.
  auto load = [&](f32x4 (&c)[NV], int row) __attribute__((always_inline)) {
    const auto r = make_rsrc(x + row * (size_t)cols, row < rows ? (int64_t)cols * 4 : 0);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = i * THREADS + t;
      const f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, idx * 16, 0, 2));
      c[i] = idx < nvec ? v : f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
    }
    // keep the scheduler from sinking the loads towards their first use
    __builtin_amdgcn_sched_barrier(0);
  };
  auto process = [&](f32x4 (&c)[NV], int row, int par) __attribute__((always_inline)) {
    float m = kNegInf;
#pragma unroll
    for (int i = 0; i < NV; ++i) m = fmaxf(m, max4(c[i]));
    const float m_lane = m;
    const float ms = (m == kNegInf) ? 0.f : m;
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      c[i] = (c[i] - ms) * kLog2e;
      c[i].x = exp2_fast(c[i].x);
      c[i].y = exp2_fast(c[i].y);
      c[i].z = exp2_fast(c[i].z);
      c[i].w = exp2_fast(c[i].w);
      l += (c[i].x + c[i].y) + (c[i].z + c[i].w);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float mo = __shfl_xor(m, off);
      const float lo = __shfl_xor(l, off);
      merge_ml(m, l, mo, lo);
    }
    const int wave = t >> 6;
    if ((t & 63) == 0) {
      sm[par][wave] = m;
      sl[par][wave] = l;
    }
    __syncthreads();
    m = sm[par][0];
    l = sl[par][0];
#pragma unroll
    for (int w = 1; w < W; ++w) merge_ml(m, l, sm[par][w], sl[par][w]);
    const float f = exp2_fast((m_lane - m) * kLog2e) / l;
    const auto ry = make_rsrc(y + row * (size_t)cols, row < rows ? (int64_t)nvec * 16 : 0);
#pragma unroll
    for (int i = 0; i < NV; ++i)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, c[i] * f), ry,
                                             (i * THREADS + t) * 16, 0, 2);
  };
  // Rows are taken two at a time in one straight-line body: the loads of the
  // next row sit in the same block as the work on the current one, where the
  // compiler leaves them.  A row index past the end gets empty descriptors: its
  // loads fetch nothing and its stores are dropped.
  int row = blockIdx.x;
  if (row >= rows) return;  // workgroup-uniform
  load(a, row);
  for (; row < rows; row += 2 * gridDim.x) {
    const int n1 = row + gridDim.x;
    load(b, n1);
    process(a, row, 0);
    load(a, n1 + gridDim.x);
    process(b, n1, 1);
  }
}

template <int THREADS, bool VEC>
__global__ __launch_bounds__(THREADS) void softmax_stream(const float* __restrict__ x,
                                                          float* __restrict__ y, int cols) {
  const size_t row = blockIdx.x;
  const float* xr = x + row * (size_t)cols;
  float* yr = y + row * (size_t)cols;
  const int t = threadIdx.x;
  float m = kNegInf, l = 0.f;
  if constexpr (VEC) {
    const int nvec = cols >> 2;
    const f32x4* x4 = reinterpret_cast<const f32x4*>(xr);
    for (int idx = t; idx < nvec; idx += THREADS) {
      const f32x4 v = x4[idx];
      const float mn = fmaxf(m, max4(v));  // step 1: new running max
      const f32x4 e = (v - mn) * kLog2e;
      l = l * exp2_fast((m - mn) * kLog2e) +  // step 2: rescale, add the chunk
          (exp2_fast(e.x) + exp2_fast(e.y)) + (exp2_fast(e.z) + exp2_fast(e.w));
      m = mn;
    }
  } else {
    for (int j = t; j < cols; j += THREADS) {
      const float v = xr[j];
      const float mn = fmaxf(m, v);
      l = l * exp2_fast((m - mn) * kLog2e) + exp2_fast((v - mn) * kLog2e);
      m = mn;
    }
  }
  block_merge<THREADS>(m, l);
  const float inv = 1.f / l;
  if constexpr (VEC) {
    const int nvec = cols >> 2;
    const f32x4* x4 = reinterpret_cast<const f32x4*>(xr);
    f32x4* y4 = reinterpret_cast<f32x4*>(yr);
    for (int idx = t; idx < nvec; idx += THREADS) {
      const f32x4 e = (x4[idx] - m) * kLog2e;
      const f32x4 o = f32x4{exp2_fast(e.x), exp2_fast(e.y), exp2_fast(e.z), exp2_fast(e.w)} * inv;
      __builtin_nontemporal_store(o, y4 + idx);
    }
  } else {
    for (int j = t; j < cols; j += THREADS) yr[j] = exp2_fast((xr[j] - m) * kLog2e) * inv;
  }
}

// ---- split rows: several workgroups per row (few rows, very long rows) -----------
// Pass 1: workgroup (row, chunk) reduces its chunk to (m, l) with the per-chunk
// online recurrence.  Pass 2: each workgroup of the row merges the row's chunk
// pairs with the associative rule, then re-reads its chunk and normalises it.
// No workgroup waits on another inside a kernel; the kernel boundary orders the
// passes.  12 bytes per element move (two reads, one write).
template <int THREADS, bool VEC>
__device__ __forceinline__ void chunk_ml(const float* __restrict__ xr, int j0, int j1, float& m,
                                         float& l) {
  const int t = threadIdx.x;
  m = kNegInf;
  l = 0.f;
  if constexpr (VEC) {
    const f32x4* x4 = reinterpret_cast<const f32x4*>(xr);
    for (int idx = (j0 >> 2) + t; idx < (j1 >> 2); idx += THREADS) {
      const f32x4 v = x4[idx];  // cached: pass 2 reads it again
      const float mn = fmaxf(m, max4(v));
      const f32x4 e = (v - mn) * kLog2e;
      l = l * exp2_fast((m - mn) * kLog2e) +
          (exp2_fast(e.x) + exp2_fast(e.y)) + (exp2_fast(e.z) + exp2_fast(e.w));
      m = mn;
    }
  } else {
    for (int j = j0 + t; j < j1; j += THREADS) {
      const float v = xr[j];
      const float mn = fmaxf(m, v);
      l = l * exp2_fast((m - mn) * kLog2e) + exp2_fast((v - mn) * kLog2e);
      m = mn;
    }
  }
  block_merge<THREADS>(m, l);
}

template <int THREADS, bool VEC>
__global__ __launch_bounds__(THREADS) void softmax_split_partials(const float* __restrict__ x,
                                                                  float2* __restrict__ part,
                                                                  int cols, int chunk, int nchunks) {
  const int row = blockIdx.x / nchunks, c = blockIdx.x - row * nchunks;
  const int j0 = c * chunk, j1 = min(cols, j0 + chunk);
  float m, l;
  chunk_ml<THREADS, VEC>(x + (size_t)row * cols, j0, j1, m, l);
  if (threadIdx.x == 0) part[blockIdx.x] = make_float2(m, l);
}

template <int THREADS, bool VEC>
__global__ __launch_bounds__(THREADS) void softmax_split_normalise(const float* __restrict__ x,
                                                                   float* __restrict__ y,
                                                                   const float2* __restrict__ part,
                                                                   int cols, int chunk, int nchunks) {
  const int row = blockIdx.x / nchunks, c = blockIdx.x - row * nchunks;
  const int t = threadIdx.x;
  float m = kNegInf, l = 0.f;
  for (int i = t; i < nchunks; i += THREADS) {
    const float2 p = part[(size_t)row * nchunks + i];
    merge_ml(m, l, p.x, p.y);
  }
  block_merge<THREADS>(m, l);
  const float inv = 1.f / l;
  const int j0 = c * chunk, j1 = min(cols, j0 + chunk);
  const float* xr = x + (size_t)row * cols;
  float* yr = y + (size_t)row * cols;
  if constexpr (VEC) {
    const f32x4* x4 = reinterpret_cast<const f32x4*>(xr);
    f32x4* y4 = reinterpret_cast<f32x4*>(yr);
    for (int idx = (j0 >> 2) + t; idx < (j1 >> 2); idx += THREADS) {
      const f32x4 e = (__builtin_nontemporal_load(x4 + idx) - m) * kLog2e;
      const f32x4 o = f32x4{exp2_fast(e.x), exp2_fast(e.y), exp2_fast(e.z), exp2_fast(e.w)} * inv;
      __builtin_nontemporal_store(o, y4 + idx);
    }
  } else {
    for (int j = j0 + t; j < j1; j += THREADS) yr[j] = exp2_fast((xr[j] - m) * kLog2e) * inv;
  }
}

struct CachedConfig {
  int capacity;  // columns
  const void* fn;
  int threads;
};

}  // namespace

// Smallest register-cache instance that holds the row, or the streaming kernel.
static void pick_softmax(int cols, bool vec_ok, const void** fn, int* threads) {
  static const CachedConfig table[] = {
      {256, (const void*)softmax_cached<64, 1>, 64},
      {1024, (const void*)softmax_cached<64, 4>, 64},
      {2048, (const void*)softmax_cached<128, 4>, 128},
      {4096, (const void*)softmax_cached<256, 4>, 256},
      {8192, (const void*)softmax_cached<256, 8>, 256},
      {16384, (const void*)softmax_cached<512, 8>, 512},
      {32768, (const void*)softmax_cached<1024, 8>, 1024},
  };
  if (vec_ok) {
    for (const auto& c : table) {
      if (cols <= c.capacity) {
        *fn = c.fn;
        *threads = c.threads;
        return;
      }
    }
    *fn = (const void*)softmax_stream<512, true>;
  } else {
    *fn = (const void*)softmax_stream<512, false>;
  }
  *threads = 512;
}

// Compute units of the current device (looked up once per device).
static int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

hipError_t launch_softmax(const float* x, float* y, int rows, int cols, bool vec_ok,
                          hipStream_t stream) {
  const void* fn;
  int threads;
  pick_softmax(cols, vec_ok, &fn, &threads);
  if (fn == (const void*)softmax_cached<1024, 8>) {
    // many rows of 16385 .. 32768 columns: one persistent workgroup per compute unit
    const int cus = device_cus();
    if (rows >= 2 * cus) {
      const void* pf = (const void*)softmax_persist<1024, 8>;
      void* pargs[] = {(void*)&x, (void*)&y, (void*)&rows, (void*)&cols};
      return hipLaunchKernel(pf, dim3(cus), dim3(1024), pargs, 0, stream);
    }
  }
  void* args[] = {(void*)&x, (void*)&y, (void*)&cols};
  return hipLaunchKernel(fn, dim3(rows), dim3(threads), args, 0, stream);
}

// Chunking of the split path: enough workgroups to fill the chip (about 2048 in
// all), chunks of at least 4096 columns (two 16-byte vectors per lane), chunk
// lengths a multiple of 4 so that every chunk of an aligned row starts 16-byte
// aligned.
void softmax_split_plan(int rows, int cols, int* chunk, int* nchunks) {
  int64_t n = (2048 + (int64_t)rows - 1) / rows;
  const int64_t by_len = ((int64_t)cols + 4095) / 4096;
  if (n > by_len) n = by_len;
  if (n < 1) n = 1;
  int64_t ch = ((int64_t)cols + n - 1) / n;
  ch = (ch + 3) & ~(int64_t)3;
  *chunk = (int)ch;
  *nchunks = (int)(((int64_t)cols + ch - 1) / ch);
}

hipError_t launch_softmax_split(const float* x, float* y, int rows, int cols, bool vec_ok,
                                float* workspace, hipStream_t stream) {
  int chunk, nchunks;
  softmax_split_plan(rows, cols, &chunk, &nchunks);
  constexpr int T = 512;
  const void* f1 = vec_ok ? (const void*)softmax_split_partials<T, true>
                          : (const void*)softmax_split_partials<T, false>;
  const void* f2 = vec_ok ? (const void*)softmax_split_normalise<T, true>
                          : (const void*)softmax_split_normalise<T, false>;
  float2* part = reinterpret_cast<float2*>(workspace);
  const float2* cpart = part;
  const int grid = rows * nchunks;
  void* a1[] = {(void*)&x, (void*)&part, (void*)&cols, (void*)&chunk, (void*)&nchunks};
  hipError_t e = hipLaunchKernel(f1, dim3(grid), dim3(T), a1, 0, stream);
  if (e != hipSuccess) return e;
  void* a2[] = {(void*)&x, (void*)&y, (void*)&cpart, (void*)&cols, (void*)&chunk, (void*)&nchunks};
  return hipLaunchKernel(f2, dim3(grid), dim3(T), a2, 0, stream);
}

hipError_t softmax_attributes(int cols, bool vec_ok, hipFuncAttributes* attr, int* threads,
                              int* blocks_per_cu) {
  const void* fn;
  pick_softmax(cols, vec_ok, &fn, threads);
  hipError_t e = hipFuncGetAttributes(attr, fn);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, *threads, 0);
}

}  // namespace osm
