// ra_rope.hip -- split-halves (NEOX) rotary position embedding for gfx950.
//
// "Primitives" page, section "Attention and transformers" (RoPE: channel j of a head is paired
// with channel j + D/2) and the nurl page, section "Layers" (nn_rope, NEOX half-split rotary).
// With inv_freq_j = theta^(-2j/D) (the frequency schedule the pages leave open) and
// angle = position * inv_freq_j:
//   y_j = x_j cos - x_{j+D/2} sin,   y_{j+D/2} = x_{j+D/2} cos + x_j sin,
// and the inverse (the transpose, used for gradients) rotates by -angle.
//
// HBM-bound.  One thread per (position, pair): the angle is formed and reduced in fp64 (large
// positions lose the phase in fp32) once, and applied to that pair of every [N, D] matrix of the
// tensor, so consecutive threads touch consecutive channels of a row.
#include "ra_device.h"
#include "ra_internal.h"

namespace ra {

template <typename T>
__global__ __launch_bounds__(kThreads) void rope_neox_kernel(const T* x, T* y, const int* positions,
                                                             int64_t mats, int N, int D, double theta,
                                                             bool inverse) {
  const int half = D / 2;
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (t >= (int64_t)N * half) return;
  const int n = (int)(t / half), j = (int)(t % half);
  const double pos = positions ? (double)positions[n] : (double)n;
  const double ang = pos * pow(theta, -2.0 * j / D);
  double sd, cd;
  sincos(ang, &sd, &cd);
  const float c = (float)cd, s = inverse ? -(float)sd : (float)sd;
  for (int64_t m = 0; m < mats; ++m) {
    const size_t base = ((size_t)m * N + n) * D + j;
    const float x1 = (float)x[base], x2 = (float)x[base + half];
    y[base] = (T)(x1 * c - x2 * s);
    y[base + half] = (T)(fmaf(x1, s, x2 * c));
  }
}

hipError_t launch_rope_neox(const void* x, void* y, const int* positions, int64_t mats, int64_t N,
                            int64_t D, double theta, bool inverse, bool is_bf16, hipStream_t stream) {
  const int64_t pairs = N * (D / 2);
  const dim3 grid((unsigned)((pairs + kThreads - 1) / kThreads)), block(kThreads);
  if (is_bf16)
    hipLaunchKernelGGL((rope_neox_kernel<bf16>), grid, block, 0, stream, static_cast<const bf16*>(x),
                       static_cast<bf16*>(y), positions, mats, (int)N, (int)D, theta, inverse);
  else
    hipLaunchKernelGGL((rope_neox_kernel<float>), grid, block, 0, stream, static_cast<const float*>(x),
                       static_cast<float*>(y), positions, mats, (int)N, (int)D, theta, inverse);
  return hipGetLastError();
}

}  // namespace ra
