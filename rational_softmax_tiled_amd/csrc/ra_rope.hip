// ra_rope.hip -- split-halves (NEOX) rotary position embedding for gfx950.
//
// "Primitives" page, section "Attention and transformers" (RoPE: channel j of a head is paired
// with channel j + D/2) and the nurl page, section "Layers" (nn_rope, NEOX half-split rotary).
// With inv_freq_j = theta^(-2j/D) (the frequency schedule the pages leave open) and
// angle = position * inv_freq_j:
//   y_j = x_j cos - x_{j+D/2} sin,   y_{j+D/2} = x_{j+D/2} cos + x_j sin,
// and the inverse (the transpose, used for gradients) rotates by -angle.
//
// HBM-bound: each element is read once and written once.  A thread owns V consecutive pairs of
// one row (V = 8 for bf16, 4 for fp32: one 16-byte load from each half of the row) and a run of
// up to kMatsPerThread matrices: it forms the V angles once (rope_rate, rope_cs, fp64) and applies
// them to that slice of each matrix of its run.  Rows whose half is not a multiple of V take the
// V = 1 path.
#include "ra_device.h"
#include "ra_internal.h"

namespace ra {

namespace {

constexpr int kRopeThreads = 256;
constexpr int kMatsPerThread = 8;

template <typename T, int V>
struct RopeVec;
template <>
struct RopeVec<bf16, 8> {
  using type = bf16x8;
};
template <>
struct RopeVec<float, 4> {
  using type = f32x4;
};
template <typename T>
struct RopeVec<T, 1> {
  using type = T;
};

template <typename T, int V>
__device__ __forceinline__ T lane_of(const typename RopeVec<T, V>::type& v, int i) {
  if constexpr (V == 1) return v;
  else return v[i];
}
template <typename T, int V>
__device__ __forceinline__ void set_lane(typename RopeVec<T, V>::type& v, int i, T x) {
  if constexpr (V == 1) v = x;
  else v[i] = x;
}

template <typename T, int V>
__global__ __launch_bounds__(kRopeThreads) void rope_neox_kernel(const T* x, T* y, const int* positions,
                                                             int64_t mats, int N, int D,
                                                             double log2_theta, bool inverse,
                                                             int mats_per_thread) {
  using vec_t = typename RopeVec<T, V>::type;
  const int half = D / 2;
  const int per_row = half / V;
  const int64_t t = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
  if (t >= (int64_t)N * per_row) return;
  const int n = (int)(t / per_row), j0 = (int)(t % per_row) * V;
  const double pos = positions ? (double)positions[n] : (double)n;
  float c[V], s[V];
#pragma unroll
  for (int i = 0; i < V; ++i) rope_cs(pos, rope_rate(j0 + i, D, log2_theta), inverse, c[i], s[i]);
  const int64_t m0 = (int64_t)blockIdx.y * mats_per_thread;
  const int64_t m1 = min(mats, m0 + mats_per_thread);
  auto turn = [&](const vec_t& a, const vec_t& b, size_t base) {
    vec_t ya, yb;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      float y1, y2;
      rope_pair((float)lane_of<T, V>(a, i), (float)lane_of<T, V>(b, i), c[i], s[i], y1, y2);
      set_lane<T, V>(ya, i, (T)y1);
      set_lane<T, V>(yb, i, (T)y2);
    }
    *reinterpret_cast<vec_t*>(y + base) = ya;
    *reinterpret_cast<vec_t*>(y + base + half) = yb;
  };
  // four matrices at a time: their eight loads go out together (one matrix at a time left two
  // loads in flight per thread; measured 2.5% slower)
  constexpr int U = 4;
  int64_t m = m0;
  for (; m + U <= m1; m += U) {
    vec_t a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t base = ((size_t)(m + u) * N + n) * D + j0;
      a[u] = *reinterpret_cast<const vec_t*>(x + base);
      b[u] = *reinterpret_cast<const vec_t*>(x + base + half);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) turn(a[u], b[u], ((size_t)(m + u) * N + n) * D + j0);
  }
  for (; m < m1; ++m) {
    const size_t base = ((size_t)m * N + n) * D + j0;
    turn(*reinterpret_cast<const vec_t*>(x + base), *reinterpret_cast<const vec_t*>(x + base + half), base);
  }
}

template <typename T, int V>
hipError_t launch_v(const void* x, void* y, const int* positions, int64_t mats, int64_t N,
                    int64_t D, double l2t, bool inverse, hipStream_t stream) {
  const int64_t items = N * (D / 2 / V);
  const int64_t runs_needed = (mats + kMatsPerThread - 1) / kMatsPerThread;
  // grid.y is limited to 65535: longer runs per thread when there are more matrices
  const int64_t per = runs_needed <= 65535 ? kMatsPerThread : (mats + 65534) / 65535;
  const dim3 grid((unsigned)((items + kRopeThreads - 1) / kRopeThreads), (unsigned)((mats + per - 1) / per));
  hipLaunchKernelGGL((rope_neox_kernel<T, V>), grid, dim3(kRopeThreads), 0, stream,
                     static_cast<const T*>(x), static_cast<T*>(y), positions, mats, (int)N, (int)D,
                     l2t, inverse, (int)per);
  return hipGetLastError();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_rope_neox(const void* x, void* y, const int* positions, int64_t mats, int64_t N,
                            int64_t D, double theta, bool inverse, bool is_bf16, hipStream_t stream) {
  const double l2t = log2(theta);
  const int half = (int)(D / 2);
  const bool vec_ok = aligned16(x) && aligned16(y);
  if (is_bf16)
    return vec_ok && half % 8 == 0 ? launch_v<bf16, 8>(x, y, positions, mats, N, D, l2t, inverse, stream)
                                   : launch_v<bf16, 1>(x, y, positions, mats, N, D, l2t, inverse, stream);
  return vec_ok && half % 4 == 0 ? launch_v<float, 4>(x, y, positions, mats, N, D, l2t, inverse, stream)
                                 : launch_v<float, 1>(x, y, positions, mats, N, D, l2t, inverse, stream);
}

}  // namespace ra
