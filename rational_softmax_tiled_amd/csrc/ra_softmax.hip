// ra_softmax.hip -- standalone ra_softmax along the rows of a [rows, cols] matrix.
//
// "Ra-Family: Rational Neural Architecture", section 3, item ra_softmax:
// Delta = max - x, u = Delta/16, phi = ((1-u)/(1+u))^8 for u < 1 else 0, p = phi / sum(phi).
// -inf entries are masked (p = 0, excluded from max and sum); an all -inf row gives p = 0.
//
// HBM-bound: one workgroup per row.  When the row fits in registers (cols <= 256 threads x
// CPT 16-byte chunks and rows are 16-byte aligned) it is read once and written once;
// otherwise the row is streamed three times (max, sum, write), the re-reads served by L2.
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
      const u32x4 raw = *reinterpret_cast<const u32x4*>(x + base + (size_t)ch * CE);
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
      *reinterpret_cast<u32x4*>(p + base + (size_t)ch * CE) = raw;
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
