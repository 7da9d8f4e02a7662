// ra_softmax.hip -- standalone ra_softmax along the rows of a [rows, cols] matrix.
//
// "Ra-Family: Rational Neural Architecture", section 3, item ra_softmax:
// Delta = max - x, u = Delta/16, phi = ((1-u)/(1+u))^8 for u < 1 else 0, p = phi / sum(phi).
// -inf entries are masked (p = 0, excluded from max and sum); an all -inf row gives p = 0.
//
// HBM-bound: one workgroup per row.  When the row fits in registers (cols <= 256 threads x
// CPT 16-byte chunks and rows are 16-byte aligned) it is read once and written once, with
// nontemporal loads and stores (6-10% faster than cached ones at [16384, 8192], measured);
// otherwise the row is streamed three times (max, sum, write), the re-reads served by L2.
#include <limits.h>

#include "ra_device.h"
#include "ra_internal.h"

namespace ra {

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// Block-wide reductions over 256 threads; `red` is 4 floats of LDS.
__device__ __forceinline__ float block_max(float x, float* red) {
  x = wave_max(x);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}
__device__ __forceinline__ float block_sum(float x, float* red) {
  x = wave_sum(x);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

constexpr float kInvWidth = 1.0f / 16.0f;

// Row held in registers: thread t owns 16-byte chunks t, t + 256, ...
template <typename T, int CPT>
__global__ __launch_bounds__(kThreads) void softmax_rows_reg(const T* x, T* p, int cols) {
  constexpr int CE = 16 / sizeof(T);
  __shared__ float red[kWaves];
  const int tid = threadIdx.x;
  const size_t base = (size_t)blockIdx.x * cols;
  const int nchunk = cols / CE;
  float v[CPT][CE];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = c * kThreads + tid;
    if (ch < nchunk) {
      const u32x4 raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + base + (size_t)ch * CE));
      const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
      for (int j = 0; j < CE; ++j) v[c][j] = to_f32(e[j]);
    } else {
#pragma unroll
      for (int j = 0; j < CE; ++j) v[c][j] = -INFINITY;
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int j = 0; j < CE; ++j) m = fmaxf(m, v[c][j]);
  m = block_max(m, red);
  const bool empty = (m == -INFINITY);
  float l = 0.0f;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int j = 0; j < CE; ++j) {
      const float f = empty ? 0.0f : ra_phi_t(m - v[c][j], kInvWidth);
      v[c][j] = f;
      l += f;
    }
  l = block_sum(l, red);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = c * kThreads + tid;
    if (ch < nchunk) {
      u32x4 raw;
      T* e = reinterpret_cast<T*>(&raw);
#pragma unroll
      for (int j = 0; j < CE; ++j) e[j] = from_f32<T>(v[c][j] * inv);
      __builtin_nontemporal_store(raw, reinterpret_cast<u32x4*>(p + base + (size_t)ch * CE));
    }
  }
}

// Any shape: three strided passes over the row.
template <typename T>
__global__ __launch_bounds__(kThreads) void softmax_rows_stream(const T* x, T* p, int cols) {
  __shared__ float red[kWaves];
  const int tid = threadIdx.x;
  const size_t base = (size_t)blockIdx.x * cols;
  float m = -INFINITY;
  for (int j = tid; j < cols; j += kThreads) m = fmaxf(m, to_f32(x[base + j]));
  m = block_max(m, red);
  const bool empty = (m == -INFINITY);
  float l = 0.0f;
  if (!empty)
    for (int j = tid; j < cols; j += kThreads) l += ra_phi_t(m - to_f32(x[base + j]), kInvWidth);
  l = block_sum(l, red);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  for (int j = tid; j < cols; j += kThreads) {
    const float f = empty ? 0.0f : ra_phi_t(m - to_f32(x[base + j]), kInvWidth);
    p[base + j] = from_f32<T>(f * inv);
  }
}

template <typename T>
static hipError_t launch_rows(const T* x, T* p, int64_t rows, int64_t cols, hipStream_t stream) {
  constexpr int CE = 16 / sizeof(T);
  const bool vec = (cols % CE) == 0 && ((uintptr_t)x % 16) == 0 && ((uintptr_t)p % 16) == 0;
  const int64_t chunks = cols / CE;
  dim3 grid((unsigned)rows), block(kThreads);
  const int c = (int)cols;
  if (vec && chunks <= 1 * kThreads)
    hipLaunchKernelGGL((softmax_rows_reg<T, 1>), grid, block, 0, stream, x, p, c);
  else if (vec && chunks <= 2 * kThreads)
    hipLaunchKernelGGL((softmax_rows_reg<T, 2>), grid, block, 0, stream, x, p, c);
  else if (vec && chunks <= 4 * kThreads)
    hipLaunchKernelGGL((softmax_rows_reg<T, 4>), grid, block, 0, stream, x, p, c);
  else if (vec && chunks <= 8 * kThreads)
    hipLaunchKernelGGL((softmax_rows_reg<T, 8>), grid, block, 0, stream, x, p, c);
  else
    hipLaunchKernelGGL((softmax_rows_stream<T>), grid, block, 0, stream, x, p, c);
  return hipGetLastError();
}

hipError_t launch_softmax_rows(const void* x, void* p, int64_t rows, int64_t cols, bool is_bf16,
                               hipStream_t stream) {
  if (is_bf16)
    return launch_rows<bf16>(static_cast<const bf16*>(x), static_cast<bf16*>(p), rows, cols, stream);
  return launch_rows<float>(static_cast<const float*>(x), static_cast<float*>(p), rows, cols, stream);
}

// ---------------------------------------------------------------- backward
// Gradient dL/dx of p = ra_softmax(x) given g = dL/dp, from the same section of the page (the
// closed-form derivative d(phi)/du = -16 phi / (1 - u^2), u < 1).  With c = sum_j p_j g_j:
//   G_j = p_j (g_j - c) / (1 - u_j^2) = (g_j - c) / l * q_j^7 / (1 + u_j)^2   (0 off the support),
// and since the row max m = x_a itself depends on x, R = -sum_j G_j is added at a, the lowest
// index attaining the max: dx = G + R e_a.  Everything is recomputed from x in fp32; an all -inf
// row gives dx = 0.  Every element of dx is written after its own x and g have been read, so dx
// may be the same buffer as x or dp.

__device__ __forceinline__ float2 block_sum2(float a, float b, float* red) {
  a = wave_sum(a);
  b = wave_sum(b);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) {
    red[wave] = a;
    red[kWaves + wave] = b;
  }
  __syncthreads();
  return make_float2((red[0] + red[1]) + (red[2] + red[3]), (red[4] + red[5]) + (red[6] + red[7]));
}
__device__ __forceinline__ int block_min_i(int x, int* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = min(x, __shfl_xor(x, off));
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wave] = x;
  __syncthreads();
  return min(min(red[0], red[1]), min(red[2], red[3]));
}

// Row held in registers (x and dp): thread t owns 16-byte chunks t, t + 256, ...
template <typename T, int CPT>
__global__ __launch_bounds__(kThreads) void softmax_rows_bwd_reg(const T* x, const T* dp, T* dx, int cols) {
  constexpr int CE = 16 / sizeof(T);
  __shared__ float red[2 * kWaves];
  __shared__ int redi[kWaves];
  const int tid = threadIdx.x;
  const size_t base = (size_t)blockIdx.x * cols;
  const int nchunk = cols / CE;
  float v[CPT][CE], g[CPT][CE];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = c * kThreads + tid;
    if (ch < nchunk) {
      const u32x4 rx = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + base + (size_t)ch * CE));
      const u32x4 rg = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(dp + base + (size_t)ch * CE));
      const T* ex = reinterpret_cast<const T*>(&rx);
      const T* eg = reinterpret_cast<const T*>(&rg);
#pragma unroll
      for (int j = 0; j < CE; ++j) {
        v[c][j] = to_f32(ex[j]);
        g[c][j] = to_f32(eg[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < CE; ++j) {
        v[c][j] = -INFINITY;
        g[c][j] = 0.0f;
      }
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int j = 0; j < CE; ++j) m = fmaxf(m, v[c][j]);
  m = block_max(m, red);
  const bool empty = (m == -INFINITY);
  // l = sum phi, sd = sum phi g, am = lowest index of the max
  float l = 0.0f, sd = 0.0f;
  int am = INT_MAX;
  if (!empty) {
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int j = 0; j < CE; ++j) {
        const float f = ra_phi_t(m - v[c][j], kInvWidth);
        l += f;
        sd = fmaf(f, g[c][j], sd);
        if (v[c][j] == m) am = min(am, (c * kThreads + tid) * CE + j);
      }
  }
  const float2 ls = block_sum2(l, sd, red);
  am = block_min_i(am, redi);
  const float il = ls.x > 0.0f ? 1.0f / ls.x : 0.0f;
  const float cil = ls.y * il * il;   // c / l with c = sum(phi g) / l
  float rs = 0.0f;
#pragma unroll
  for (int c = 0; c < CPT; ++c)
#pragma unroll
    for (int j = 0; j < CE; ++j) {
      float pj;
      const float gj = empty ? 0.0f : ra_grad_t(m - v[c][j], kInvWidth, fmaf(g[c][j], il, -cil), il, &pj);
      g[c][j] = gj;
      rs += gj;
    }
  const float R = -block_sum(rs, red);
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int ch = c * kThreads + tid;
    if (ch < nchunk) {
      u32x4 raw;
      T* e = reinterpret_cast<T*>(&raw);
#pragma unroll
      for (int j = 0; j < CE; ++j) e[j] = from_f32<T>(ch * CE + j == am ? g[c][j] + R : g[c][j]);
      __builtin_nontemporal_store(raw, reinterpret_cast<u32x4*>(dx + base + (size_t)ch * CE));
    }
  }
}

// Any shape: four strided passes over the row (max; sums and argmax; sum of G; write).
template <typename T>
__global__ __launch_bounds__(kThreads) void softmax_rows_bwd_stream(const T* x, const T* dp, T* dx, int cols) {
  __shared__ float red[2 * kWaves];
  __shared__ int redi[kWaves];
  const int tid = threadIdx.x;
  const size_t base = (size_t)blockIdx.x * cols;
  float m = -INFINITY;
  for (int j = tid; j < cols; j += kThreads) m = fmaxf(m, to_f32(x[base + j]));
  m = block_max(m, red);
  if (m == -INFINITY) {   // every entry masked (uniform across the workgroup)
    for (int j = tid; j < cols; j += kThreads) dx[base + j] = from_f32<T>(0.0f);
    return;
  }
  float l = 0.0f, sd = 0.0f;
  int am = INT_MAX;
  for (int j = tid; j < cols; j += kThreads) {
    const float xv = to_f32(x[base + j]);
    const float f = ra_phi_t(m - xv, kInvWidth);
    l += f;
    sd = fmaf(f, to_f32(dp[base + j]), sd);
    if (xv == m) am = min(am, j);
  }
  const float2 ls = block_sum2(l, sd, red);
  am = block_min_i(am, redi);
  const float il = 1.0f / ls.x;   // l >= 1: phi = 1 at the max
  const float cil = ls.y * il * il;
  float rs = 0.0f;
  for (int j = tid; j < cols; j += kThreads) {
    float pj;
    rs += ra_grad_t(m - to_f32(x[base + j]), kInvWidth, fmaf(to_f32(dp[base + j]), il, -cil), il, &pj);
  }
  const float R = -block_sum(rs, red);
  for (int j = tid; j < cols; j += kThreads) {
    float pj;
    const float gj = ra_grad_t(m - to_f32(x[base + j]), kInvWidth, fmaf(to_f32(dp[base + j]), il, -cil), il, &pj);
    dx[base + j] = from_f32<T>(j == am ? gj + R : gj);
  }
}

template <typename T>
static hipError_t launch_rows_bwd(const T* x, const T* dp, T* dx, int64_t rows, int64_t cols,
                                  hipStream_t stream) {
  constexpr int CE = 16 / sizeof(T);
  const bool vec = (cols % CE) == 0 && ((uintptr_t)x % 16) == 0 && ((uintptr_t)dp % 16) == 0 &&
                   ((uintptr_t)dx % 16) == 0;
  const int64_t chunks = cols / CE;
  dim3 grid((unsigned)rows), block(kThreads);
  const int c = (int)cols;
  if (vec && chunks <= 1 * kThreads)
    hipLaunchKernelGGL((softmax_rows_bwd_reg<T, 1>), grid, block, 0, stream, x, dp, dx, c);
  else if (vec && chunks <= 2 * kThreads)
    hipLaunchKernelGGL((softmax_rows_bwd_reg<T, 2>), grid, block, 0, stream, x, dp, dx, c);
  else if (vec && chunks <= 4 * kThreads)
    hipLaunchKernelGGL((softmax_rows_bwd_reg<T, 4>), grid, block, 0, stream, x, dp, dx, c);
  else if (vec && chunks <= 8 * kThreads)
    hipLaunchKernelGGL((softmax_rows_bwd_reg<T, 8>), grid, block, 0, stream, x, dp, dx, c);
  else
    hipLaunchKernelGGL((softmax_rows_bwd_stream<T>), grid, block, 0, stream, x, dp, dx, c);
  return hipGetLastError();
}

hipError_t launch_softmax_rows_bwd(const void* x, const void* dp, void* dx, int64_t rows,
                                   int64_t cols, bool is_bf16, hipStream_t stream) {
  if (is_bf16)
    return launch_rows_bwd<bf16>(static_cast<const bf16*>(x), static_cast<const bf16*>(dp),
                                 static_cast<bf16*>(dx), rows, cols, stream);
  return launch_rows_bwd<float>(static_cast<const float*>(x), static_cast<const float*>(dp),
                                static_cast<float*>(dx), rows, cols, stream);
}

// ---------------------------------------------------------------- fills

template <typename U>
__global__ void fill_kernel(U* dst, U value, size_t count) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < count; i += stride) dst[i] = value;
}

__global__ void fill_pairs_kernel(float* dst, float a, float b, size_t pairs) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < pairs; i += stride) {
    dst[2 * i] = a;
    dst[2 * i + 1] = b;
  }
}

static dim3 fill_grid(size_t count) {
  size_t blocks = (count + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) blocks = 1;
  return dim3((unsigned)blocks);
}

hipError_t launch_fill_u32(void* dst, uint32_t value, size_t count, hipStream_t stream) {
  hipLaunchKernelGGL((fill_kernel<uint32_t>), fill_grid(count), dim3(kThreads), 0, stream,
                     static_cast<uint32_t*>(dst), value, count);
  return hipGetLastError();
}
hipError_t launch_fill_u16(void* dst, uint16_t value, size_t count, hipStream_t stream) {
  hipLaunchKernelGGL((fill_kernel<uint16_t>), fill_grid(count), dim3(kThreads), 0, stream,
                     static_cast<uint16_t*>(dst), value, count);
  return hipGetLastError();
}
hipError_t launch_fill_pairs(float* dst, float a, float b, size_t pairs, hipStream_t stream) {
  hipLaunchKernelGGL(fill_pairs_kernel, fill_grid(pairs), dim3(kThreads), 0, stream, dst, a, b, pairs);
  return hipGetLastError();
}

}  // namespace ra
