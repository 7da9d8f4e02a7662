// ra_device.h -- device-side building blocks of the rational-softmax attention kernels (gfx950).
//
// Matrix-core conventions (CDNA 32x32 MFMA, wave64):
//   * v_mfma_f32_32x32x16_bf16: lane l supplies A[m = l%32][k = 8*(l/32) + j] and
//     B[k = 8*(l/32) + j][n = l%32] for j = 0..7; the 32x32 fp32 result leaves lane l holding
//     column n = l%32 and rows m = 8*(i/4) + 4*(l/32) + i%4 in accumulator element i.
//   * For fp32 operands the same 16-wide K chunk is covered by eight v_mfma_f32_32x32x2_f32,
//     the j-th using element j of each lane's 8-element fragment, so fragments have one layout
//     for both types: "8 consecutive K-elements starting at 8*(l/32)".
//   * The order of the K (contraction) index inside a chunk is free as long as both operands
//     agree; the P.V product uses this to consume the score accumulator in place (see
//     key_slot below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include "ra_internal.h"

namespace ra {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short short8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kWaves = 4;               // waves per workgroup
constexpr int kThreads = kWave * kWaves;
constexpr int kRowsPerWave = 32;        // query (or key) rows one wave owns
constexpr int kNumXcd = 8;              // MI355X: 8 accelerator dies, each with its own L2

template <typename T> struct Ty;
template <> struct Ty<bf16> {
  using frag = bf16x8;                  // 8 x bf16 = 16 bytes
  using quad = bf16x4;
  static constexpr int chunk = 8;       // elements per 16-byte chunk
};
template <> struct Ty<float> {
  using frag = f32x8;                   // 8 x fp32 = 32 bytes
  using quad = f32x4;
  static constexpr int chunk = 4;
};

// ---------------------------------------------------------------- fragments

__device__ __forceinline__ bf16x8 load_frag(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ f32x8 load_frag(const float* p) {
  f32x4 lo = *reinterpret_cast<const f32x4*>(p);
  f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
  return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <typename T> __device__ __forceinline__ typename Ty<T>::frag zero_frag() {
  return typename Ty<T>::frag{};
}

__device__ __forceinline__ void mma(f32x16& c, const bf16x8& a, const bf16x8& b) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16& c, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
}

// Row index (inside a 32x32 accumulator) of element i for this lane.
__device__ __forceinline__ int acc_row(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// Keeps the entries of a 32 x 32 accumulator block whose row offset acc_row(i, lane) -
// 4 (lane >> 5) = 8 (i >> 2) + (i & 3) lies in [lo, hi) and sets the others to -inf.  The causal
// and tail tests of a block reduce to these two per-lane bounds (compared with constants).
constexpr int kNoBound = 1 << 30;
__device__ __forceinline__ void keep_rows(f32x16& s, int lo, int hi) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 8 * (i >> 2) + (i & 3);
    if (r < lo || r >= hi) s[i] = -INFINITY;
  }
}

// Keeps the entries of 32-key block sb of a 64-key tile whose key bit is set in keep (bit l: key
// l of the tile) and sets the others to -inf.  Entry i of a lane is key 8 (i/4) + 4 (lane/32) +
// i%4 of the block.
__device__ __forceinline__ void keep_keys(f32x16& s, unsigned long long keep, int sb, int lane) {
  const unsigned w = (unsigned)(keep >> (32 * sb)) >> (4 * (lane >> 5));
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (!((w >> (8 * (i >> 2) + (i & 3))) & 1u)) s[i] = -INFINITY;
}

// Eight accumulator values (elements 8*ks .. 8*ks+7) as the B fragment of the next product.
__device__ __forceinline__ bf16x8 pack_frag_bf16(const f32x16& s, int ks) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (bf16)s[8 * ks + j];   // v_cvt_pk_bf16_f32: nearest-even
  return r;
}
__device__ __forceinline__ f32x8 pack_frag_f32(const f32x16& s, int ks) {
  f32x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = s[8 * ks + j];
  return r;
}

// Accumulator rows 16*ks + 8*(l/32) + j (j = 0..7) of lane l, produced by elements 8*ks + j,
// are stored at "slot" 16*ks + 8*(l/32) + j of a transposed LDS tile so that an A fragment
// read of 8 consecutive slots pairs with them.  key_slot maps a row (0..31) to its slot;
// groups of four consecutive rows stay contiguous.
__device__ __host__ constexpr int key_slot(int r) {
  return 16 * ((r >> 4) & 1) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3);
}
__device__ __host__ constexpr int quad_slot(int quad) {   // quad = 4 consecutive rows
  return 32 * (quad >> 3) + key_slot((quad & 7) * 4);
}

// ---------------------------------------------------------------- rational softmax

// phi for one entry from the raw score s, with c = scale / 16 and kd = 1 + m * c for the row's
// raw max m: 1 + u = fma(s, -c, kd) (+inf for a masked entry, s = -inf); q = (1-u)/(1+u) =
// 2/(1+u) - 1, clamped to [0, 1] so that u >= 1 gives exactly 0; phi = q^8 by three squarings.
// ("Ra-Family: Rational Neural Architecture", section 3, ra_softmax.)
__device__ __forceinline__ float ra_phi(float s, float c, float kd) {
  const float d = fmaf(s, -c, kd);
  const float r = __builtin_amdgcn_rcpf(d);
  const float q = fminf(fmaxf(fmaf(r, 2.0f, -1.0f), 0.0f), 1.0f);
  const float q2 = q * q;
  const float q4 = q2 * q2;
  return q4 * q4;
}

// The same with Delta given directly in units where u = t * c (t >= 0, +inf when masked).
__device__ __forceinline__ float ra_phi_t(float t, float c) {
  const float d = fmaf(t, c, 1.0f);
  const float r = __builtin_amdgcn_rcpf(d);
  const float q = fminf(fmaxf(fmaf(r, 2.0f, -1.0f), 0.0f), 1.0f);
  const float q2 = q * q;
  const float q4 = q2 * q2;
  return q4 * q4;
}

// The direct gradient factor for one entry: (dP - c) / l * q^7 / (1+u)^2, given t = m - s in
// raw units and dpc = (dP - c) / l.  q is clamped exactly as in the forward, so entries off the
// support (and masked ones, t = +inf) give 0.  Also returns p = q^8 / l through *p.
__device__ __forceinline__ float ra_grad_t(float t, float c16, float dpc, float il, float* p) {
  const float d = fmaf(t, c16, 1.0f);
  const float r = __builtin_amdgcn_rcpf(d);
  const float q = fminf(fmaxf(fmaf(r, 2.0f, -1.0f), 0.0f), 1.0f);
  const float q2 = q * q;
  const float q4 = q2 * q2;
  const float q6 = q4 * q2;
  *p = (q4 * q4) * il;
  return dpc * ((q6 * q) * (r * r));
}

// ---------------------------------------------------------------- NEOX rotary embedding
// Split halves ("Primitives" page, section "Attention and transformers", RoPE; the nurl page,
// section "Layers", nn_rope): channel j < D/2 of a row at position pos pairs with j + D/2 and
// turns by pos * theta^(-2j/D) (the frequency schedule the pages leave open).  The rate
// theta^(-2j/D) is formed in fp64 from log2(theta) (computed once on the host); kernels keep the
// D/2 rates in a small table.  The angle is formed and reduced to [-pi, pi] in fp64 (large
// positions lose the phase in fp32); its cos and sin are then evaluated in fp32.  Every kernel
// that rotates uses these helpers, so a rotation fused into another kernel is bit-identical to
// the standalone one.
__device__ __forceinline__ double rope_rate(int j, int D, double log2_theta) {
  return exp2((double)(-2 * j) / (double)D * log2_theta);
}
__device__ __forceinline__ void rope_cs(double pos, double rate, bool inverse, float& c, float& s) {
  constexpr double kTwoPi = 6.283185307179586476925286766559;
  const double ang = pos * rate;
  const double red = fma(-kTwoPi, rint(ang * (1.0 / kTwoPi)), ang);
  float sf, cf;
  sincosf((float)red, &sf, &cf);
  c = cf;
  s = inverse ? -sf : sf;
}
// (x_j, x_{j+D/2}) -> (x_j c - x_{j+D/2} s, x_j s + x_{j+D/2} c), in fp32 with fixed contractions
__device__ __forceinline__ void rope_pair(float x1, float x2, float c, float s, float& y1, float& y2) {
  y1 = fmaf(x1, c, -(x2 * s));
  y2 = fmaf(x1, s, x2 * c);
}

// ---------------------------------------------------------------- wave / block helpers

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, unrolled at compile time
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_min(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fminf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Max over the 64 lanes with DPP row operations only (no LDS round trip): quad swaps and row
// rotations leave every lane of a 16-lane row with the row max; row_bcast:15 then folds row r-1
// into rows 1 and 3, and row_bcast:31 folds lane 31 into rows 2 and 3.  Exact in lane 63 (other
// lanes hold partial maxima).  Rows a broadcast does not target keep x (old operand = x).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float v) {
  const int i = __builtin_bit_cast(int, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(i, i, CTRL, ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_max_lane63(float x) {
  x = fmaxf(x, dpp_f32<0xB1, 0xf>(x));    // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f32<0x4E, 0xf>(x));    // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_f32<0x124, 0xf>(x));   // row_ror:4
  x = fmaxf(x, dpp_f32<0x128, 0xf>(x));   // row_ror:8
  x = fmaxf(x, dpp_f32<0x142, 0xa>(x));   // row_bcast:15 into rows 1, 3
  x = fmaxf(x, dpp_f32<0x143, 0xc>(x));   // row_bcast:31 into rows 2, 3
  return x;
}

// Workgroups are dispatched round-robin over the 8 XCDs.  Give each XCD a contiguous range
// of logical workgroup ids so that neighbours (which share K/V) share one L2.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int per = n / kNumXcd, rem = n % kNumXcd;
  const int x = i % kNumXcd, j = i / kNumXcd;
  return (x < rem) ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j;
}

// ---------------------------------------------------------------- LDS staging

// Copy `ROWS` rows of a row-major [*, D] tile into LDS with row pitch PITCH (elements);
// rows >= nvalid are zero-filled.  16-byte chunks, consecutive threads on consecutive
// chunks of a row.
template <typename T, int D, int ROWS, int PITCH>
__device__ __forceinline__ void stage_rows(T* lds, const T* g, int nvalid, int tid) {
  constexpr int CE = 16 / sizeof(T);
  constexpr int CPR = D / CE;
  constexpr int TOTAL = ROWS * CPR;
#pragma unroll
  for (int it = 0; it < (TOTAL + kThreads - 1) / kThreads; ++it) {
    const int c = it * kThreads + tid;
    if (TOTAL % kThreads == 0 || c < TOTAL) {
      const int r = c / CPR, cc = c % CPR;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (r < nvalid) val = *reinterpret_cast<const u32x4*>(g + (size_t)r * D + cc * CE);
      *reinterpret_cast<u32x4*>(lds + r * PITCH + cc * CE) = val;
    }
  }
}

// Copy `ROWS` rows of a row-major [*, D] tile into LDS transposed: lds[d * PITCH + slot(row)],
// with the slot order of key_slot inside every 32-row block.  Each thread moves a 4-row x
// 8-column block: four 8-element global loads, eight 4-element LDS stores.  Consecutive lanes
// take consecutive row quads of one column chunk, so the 16 lanes of an LDS store cycle fill
// one contiguous slot row (no bank conflicts whatever the pitch).
template <typename T, int D, int ROWS, int PITCH>
__device__ __forceinline__ void stage_rows_transposed(T* lds, const T* g, int nvalid, int tid) {
  using quad_t = typename Ty<T>::quad;
  constexpr int QUADS = ROWS / 4;
  constexpr int UNITS = QUADS * (D / 8);
#pragma unroll
  for (int it = 0; it < (UNITS + kThreads - 1) / kThreads; ++it) {
    const int u = it * kThreads + tid;
    if (UNITS % kThreads == 0 || u < UNITS) {
      const int quad = u % QUADS, dc = u / QUADS;
      typename Ty<T>::frag rows[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * quad + r;
        rows[r] = row < nvalid ? load_frag(g + (size_t)row * D + 8 * dc) : zero_frag<T>();
      }
      const int slot = quad_slot(quad);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        quad_t col = {rows[0][e], rows[1][e], rows[2][e], rows[3][e]};
        *reinterpret_cast<quad_t*>(lds + (8 * dc + e) * PITCH + slot) = col;
      }
    }
  }
}

// ---------------------------------------------------------------- register-staged tiles
// Two-phase versions of the stagers: load() issues the global loads into registers (they stay
// in flight while the caller computes), store() writes them to LDS.  With two LDS buffers this
// gives one barrier per tile and hides the global-load latency behind the tile's math.
// Loads go through a buffer resource whose size is the tile's valid rows: the hardware returns
// zeros past it, so ragged tails need no per-lane branch.

// Buffer resource word 3 for raw (untyped) dword loads on gfx9-family parts.
constexpr int kBufferWord3 = 0x00020000;

// base and valid_rows must be the same in every lane (a resource lives in scalar registers).
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const T* base, int valid_rows, int D) {
  const int bytes = __builtin_amdgcn_readfirstlane(valid_rows > 0 ? valid_rows * D * (int)sizeof(T) : 0);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), (short)0, bytes, kBufferWord3);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

template <typename T>
__device__ __forceinline__ typename Ty<T>::frag buf_load_frag(__amdgpu_buffer_rsrc_t r, int elem_off) {
  if constexpr (sizeof(T) == 2) {
    const u32x4 v = buf_load16(r, elem_off * 2);
    return __builtin_bit_cast(bf16x8, v);
  } else {
    const u32x4 lo = buf_load16(r, elem_off * 4);
    const u32x4 hi = buf_load16(r, elem_off * 4 + 16);
    const f32x4 flo = __builtin_bit_cast(f32x4, lo), fhi = __builtin_bit_cast(f32x4, hi);
    return f32x8{flo[0], flo[1], flo[2], flo[3], fhi[0], fhi[1], fhi[2], fhi[3]};
  }
}

template <typename T, int D, int ROWS>
struct RowTile {
  static constexpr int CE = 16 / sizeof(T);
  static constexpr int CPR = D / CE;
  static constexpr int TOTAL = ROWS * CPR;
  static constexpr int PER = (TOTAL + kThreads - 1) / kThreads;
  u32x4 v[PER];

  // rows [0, nvalid) of the tile at g; the rest read as zeros
  __device__ __forceinline__ void load(const T* g, int nvalid, int tid) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(g, min(nvalid, ROWS), D);
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int c = (TOTAL % kThreads == 0) ? it * kThreads + tid : min(it * kThreads + tid, TOTAL - 1);
      v[it] = buf_load16(r, c * 16);
    }
  }
  template <int PITCH>
  __device__ __forceinline__ void store(T* lds, int tid) const {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int c = it * kThreads + tid;
      if (TOTAL % kThreads == 0 || c < TOTAL) {
        const int r = c / CPR, cc = c % CPR;
        *reinterpret_cast<u32x4*>(lds + r * PITCH + cc * CE) = v[it];
      }
    }
  }
};

template <typename T, int D, int ROWS>
struct TransTile {
  using frag_t = typename Ty<T>::frag;
  using quad_t = typename Ty<T>::quad;
  static constexpr int QUADS = ROWS / 4;
  static constexpr int UNITS = QUADS * (D / 8);
  static constexpr int PER = (UNITS + kThreads - 1) / kThreads;
  frag_t rows[PER > 0 ? PER : 1][4];   // ROWS == 0: an unused placeholder

  __device__ __forceinline__ void load(const T* g, int nvalid, int tid) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(g, min(nvalid, ROWS), D);
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int u = (UNITS % kThreads == 0) ? it * kThreads + tid : min(it * kThreads + tid, UNITS - 1);
      const int quad = u % QUADS, dc = u / QUADS;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) rows[it][rr] = buf_load_frag<T>(r, (4 * quad + rr) * D + 8 * dc);
    }
  }
  template <int PITCH>
  __device__ __forceinline__ void store(T* lds, int tid) const {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int u = it * kThreads + tid;
      if (UNITS % kThreads == 0 || u < UNITS) {
        const int quad = u % QUADS, dc = u / QUADS;
        const int slot = quad_slot(quad);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          quad_t col = {rows[it][0][e], rows[it][1][e], rows[it][2][e], rows[it][3][e]};
          *reinterpret_cast<quad_t*>(lds + (8 * dc + e) * PITCH + slot) = col;
        }
      }
    }
  }
};

// ---------------------------------------------------------------- swizzled row tiles
// A tile of rows x D elements stored without padding; the 16-byte chunk cc of row r sits at
// chunk position cc ^ swz(r).  The LDS serves 256 bytes per cycle (64 banks): 16 lanes of a
// 16-byte read, 32 lanes of an 8-byte read.  swz makes both access patterns conflict-free:
//   * row reads (16 consecutive rows, one chunk each): swz is a permutation over any 16
//     consecutive rows (for 128-byte rows: over the 8 rows of each row parity);
//   * transposed 8-byte reads (4 consecutive rows, 64 contiguous bytes each): the four rows'
//     chunk groups of four land on distinct bank groups.
template <typename T, int D>
__device__ __forceinline__ constexpr int swz(int row) {
  constexpr int CPR = D * (int)sizeof(T) / 16;   // chunks per row
  if constexpr (CPR >= 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Element offset of logical chunk cc of row r.
template <typename T, int D>
__device__ __forceinline__ int swz_off(int r, int cc) {
  constexpr int CE = 16 / (int)sizeof(T);
  return r * D + ((cc ^ swz<T, D>(r)) * CE);
}

// Row fragment: 8 consecutive elements starting at element column col (a multiple of 8).
template <typename T, int D>
__device__ __forceinline__ typename Ty<T>::frag swz_frag(const T* tile, int r, int col) {
  constexpr int CE = 16 / (int)sizeof(T);
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const bf16x8*>(tile + swz_off<T, D>(r, col / CE));
  } else {
    const f32x4 lo = *reinterpret_cast<const f32x4*>(tile + swz_off<T, D>(r, col / CE));
    const f32x4 hi = *reinterpret_cast<const f32x4*>(tile + swz_off<T, D>(r, col / CE + 1));
    return f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
}

// Transposed A fragment from a swizzled bf16 row tile T[row][col]: lane l receives
// T[k0 + s(j)][c0 + l%32] for the 8 contraction slots j, where the row order
// s = {4*(l/32) + 0..3, 8 + 4*(l/32) + 0..3} matches the accumulator layout of a 32x32
// product (key_slot).  Two ds_read_b64_tr_b16: within each 16-lane group, lane L addresses
// row rb + L/4, columns cb + 4*(L%4) .. +3, and receives column cb + L of rows rb .. rb+3.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const bf16* tile, int k0, int c0, int lane) {
  typedef __attribute__((address_space(3))) short lds_short;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const int g = lane >> 4, L = lane & 15;
  const int row = k0 + 4 * (g >> 1) + (L >> 2);
  const int col = c0 + 16 * (g & 1) + 4 * (L & 3);
  const int sub = col & 7;
  const int o1 = swz_off<bf16, D>(row, col >> 3) + sub;
  const int o2 = swz_off<bf16, D>(row + 8, col >> 3) + sub;
  const lds_short* base = (const lds_short*)(tile);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + o1));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + o2));
  const short8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Register-prefetched swizzled row tile (store() writes chunk cc of row r at its swizzled spot).
template <typename T, int D, int ROWS>
struct SwzTile {
  static constexpr int CE = 16 / sizeof(T);
  static constexpr int CPR = D / CE;
  static constexpr int TOTAL = ROWS * CPR;
  static constexpr int PER = (TOTAL + kThreads - 1) / kThreads;
  u32x4 v[PER > 0 ? PER : 1];   // ROWS == 0: an unused placeholder

  __device__ __forceinline__ void load(const T* g, int nvalid, int tid) {
    const __amdgpu_buffer_rsrc_t r = tile_rsrc(g, min(nvalid, ROWS), D);
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int c = (TOTAL % kThreads == 0) ? it * kThreads + tid : min(it * kThreads + tid, TOTAL - 1);
      v[it] = buf_load16(r, c * 16);
    }
  }
  __device__ __forceinline__ void store(T* lds, int tid) const {
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int c = it * kThreads + tid;
      if (TOTAL % kThreads == 0 || c < TOTAL) {
        const int r = c / CPR, cc = c % CPR;
        *reinterpret_cast<u32x4*>(lds + swz_off<T, D>(r, cc)) = v[it];
      }
    }
  }
};

// ---------------------------------------------------------------- LDS DMA (bf16 row tiles)
// Loads a ROWS x D bf16 row tile straight into LDS with buffer_load ... lds (no registers):
// every instruction fills 1 KiB of LDS, lane l writing chunk position l.  Choosing which global
// chunk each lane fetches lays the tile out swizzled (swz).  Rows >= nvalid read as zeros.
// The NW waves of the workgroup share the 1 KiB blocks.  The caller waits (vmcnt) and issues a
// barrier before any wave reads the tile.
// LDS byte address of a __shared__ object: one address-space conversion, kept in a scalar register
// by callers that add constant offsets to it rather than converting every pointer.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (unsigned)(unsigned long)(const __attribute__((address_space(3))) char*)p);
}

// Raw buffer resource words for [g, g + bytes) (stride 0, raw dword format; zeros past the end).
// g and bytes must be the same in every lane.
__device__ __forceinline__ u32x4 dma_rsrc(const void* g, int bytes) {
  const unsigned long long addr = (unsigned long long)g;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((unsigned)addr);
  r[1] = __builtin_amdgcn_readfirstlane((unsigned)(addr >> 32) & 0xffffu);   // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(bytes > 0 ? bytes : 0);               // num_records
  r[3] = kBufferWord3;
  return r;
}

// One LDS DMA instruction from a prepared resource: every lane fetches SIZE bytes at byte offset
// voffset + soffset of the buffer and lane l stores them at LDS byte address m0 + SIZE * l.  The
// one wait state between the M0 write and the load is the hazard the ISA requires.
template <int SIZE>
__device__ __forceinline__ void lds_dma_at(const u32x4& rsrc, unsigned m0, int voffset, int soffset) {
  static_assert(SIZE == 4 || SIZE == 16, "dword or dwordx4");
  if constexpr (SIZE == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voffset), "s"(rsrc),
                    "s"(__builtin_amdgcn_readfirstlane(soffset))
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voffset), "s"(rsrc),
                    "s"(__builtin_amdgcn_readfirstlane(soffset))
                 : "memory", "m0");
}

// One LDS DMA instruction: every lane fetches SIZE bytes (4 or 16) at byte offset
// voffset + soffset of the buffer [g, g + bytes) (zeros past its end) and lane l stores them at LDS bytes
// [SIZE*l, SIZE*l + SIZE) after `lds`.  Issued from inline assembly so that the compiler does
// not track it as a pending LDS write, for which it would wait (vmcnt) before every later LDS
// read and so serialise the prefetch; callers wait for it themselves (wait_vmem) and then issue
// a barrier before reading what it wrote.  g, bytes and lds must be the same in every lane.  The
// one wait state between the M0 write and the load is the hazard the ISA requires.
template <int SIZE>
__device__ __forceinline__ void lds_dma(const void* g, int bytes, const void* lds, int voffset,
                                        int soffset = 0) {
  lds_dma_at<SIZE>(dma_rsrc(g, bytes), lds_addr(lds), voffset, soffset);
}

// Per-lane byte offset of dma_block's copies when the NW waves' blocks share one lane layout (the
// case dma_block calls kSharedLaneOffset): block b = i * NW + wave then sits at scalar offset
// i * NW * 1024 of the tile and LDS bytes b * 1024.
template <int D, int NW>
__device__ __forceinline__ int dma_lane_offset(int wave, int lane) {
  static_assert((NW * 512 / D) % 16 == 0, "the waves' blocks must share the lane layout");
  constexpr int CPR = D / 8;
  const int p = wave * 64 + lane;
  const int row = p / CPR, pos = p % CPR;
  return (row * CPR + (pos ^ swz<bf16, D>(row))) * 16;
}

// Block i of this wave's share of a ROWS x D tile copy (blocks i*NW + wave); a no-op past the end.
template <int D, int ROWS, int NW = kWaves>
__device__ __forceinline__ void dma_block(bf16* lds, const bf16* g, int nvalid, int wave, int lane, int i) {
  constexpr int CPR = D / 8;                       // 16-byte chunks per row
  constexpr int BLOCKS = ROWS * D * 2 / 1024;      // 1 KiB blocks in the tile
  static_assert((ROWS * D * 2) % 1024 == 0, "tile must be whole 1 KiB blocks");
  const int b = i * NW + wave;
  if (BLOCKS % NW == 0 || b < BLOCKS) {
    // the swizzle depends on the row modulo 16 only; a block spans 1024 / (2 D) rows, so when
    // NW blocks cover a multiple of 16 rows every block of a wave has the same per-lane offset
    // relative to the block's first byte (passed as the scalar offset)
    constexpr bool kSharedLaneOffset = (NW * 512 / D) % 16 == 0;
    const int bb = kSharedLaneOffset ? wave : b;
    const int p = bb * 64 + lane;                  // chunk position inside the tile
    const int row = p / CPR, pos = p % CPR;
    const int cc = pos ^ swz<bf16, D>(row);        // logical chunk stored at that position
    const int lane_off = (row * CPR + cc) * 16;
    if constexpr (kSharedLaneOffset)
      lds_dma<16>(g, min(nvalid, ROWS) * D * 2, lds + b * 512, lane_off, (b - bb) * 1024);
    else
      lds_dma<16>(g, min(nvalid, ROWS) * D * 2, lds + b * 512, lane_off);
  }
}
// Number of dma_block calls that cover this wave's share of the tile.
template <int D, int ROWS, int NW = kWaves>
constexpr int dma_blocks_per_wave() { return (ROWS * D * 2 / 1024 + NW - 1) / NW; }

template <int D, int ROWS, int NW = kWaves>
__device__ __forceinline__ void dma_tile(bf16* lds, const bf16* g, int nvalid, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < dma_blocks_per_wave<D, ROWS, NW>(); ++i) dma_block<D, ROWS, NW>(lds, g, nvalid, wave, lane, i);
}

// dma_tile from a resource over a whole matrix (the tile starts at byte tile_off of it; rows past
// the resource's end read as zeros) to LDS byte address m0, with lane_off = dma_lane_offset: no
// per-tile pointer arithmetic or address-space conversion.
template <int D, int ROWS, int NW = kWaves>
__device__ __forceinline__ void dma_tile_at(const u32x4& rsrc, int tile_off, unsigned m0, int lane_off,
                                            int wave) {
  constexpr int BLOCKS = ROWS * D * 2 / 1024;
  static_assert(BLOCKS % NW == 0, "every wave copies the same number of blocks");
#pragma unroll
  for (int i = 0; i < BLOCKS / NW; ++i)
    lds_dma_at<16>(rsrc, m0 + (i * NW + wave) * 1024, lane_off, tile_off + i * NW * 1024);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left alone): every outstanding vector-memory load,
// LDS DMA included, has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(N): at most the N youngest vector-memory loads still outstanding (loads
// complete in issue order, so every older one, LDS DMA included, has landed).
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// ---------------------------------------------------------------- explicit attention masks
// Element (b, h, i, j) of a mask (query head h, query row i, key j) sits at element offset
// b*sb + h*sh + i*sq + j*sk; zero strides broadcast.  kMaskBool: uint8, nonzero = attend, zero
// masks the score.  kMaskAdd: additive, in the dtype of q, added to the scaled score; the kernels
// work on raw dot products, so it enters as bias / scale.  One (b, h) slice is read through a
// buffer resource of `bytes` bytes: offsets past it read as zero (a masked-out bool, a zero bias),
// and every offset inside the slice fits in 31 bits (the host checks both).
enum { kMaskNone = 0, kMaskBool = 1, kMaskAdd = 2 };

struct MaskArgs {
  const void* ptr;       // nullptr: no explicit mask
  long long sb, sh;      // element strides over batch and query head
  int sq, sk;            // element strides over query rows and keys
  int bytes;             // bytes of one (b, h) slice, tails included
  int kind;
  float inv_scale;       // 1 / scale
  // keys contiguous (sk = 1), every row and slice start a multiple of 4 elements, Nk a multiple of
  // 4 and the mask 4-byte aligned: a row's 32-key block loads in 16-byte pieces, half per lane of a
  // pair (boolean masks, and additive ones of 2-byte elements; see MaskSlice)
  int packed;
};

inline MaskArgs mask_args(const AttnProblem& p) {
  MaskArgs m;
  m.ptr = p.mask_kind != kMaskNone ? p.mask : nullptr;
  m.sb = p.msb;
  m.sh = p.msh;
  m.sq = p.msq;
  m.sk = p.msk;
  m.bytes = p.mask_bytes;
  m.kind = p.mask_kind;
  m.inv_scale = 1.0f / p.scale;
  m.packed = p.mask_kind != kMaskNone && p.msk == 1 && p.msq % 4 == 0 && p.msb % 4 == 0 && p.msh % 4 == 0 &&
             p.Nk % 4 == 0 && reinterpret_cast<unsigned long long>(p.mask) % 4 == 0;
  return m;
}

// Does a raw mask value keep its entry at all (boolean: kept; additive: anything but -inf)?
__device__ __forceinline__ bool mask_alive(int kind, unsigned v) {
  return kind == kMaskBool ? v != 0u : v != 0xff800000u;
}

// A score with its mask element applied (v as MaskSlice::load returns it).
__device__ __forceinline__ float mask_value(int kind, float inv_scale, float s, unsigned v) {
  return kind == kMaskBool ? (v != 0u ? s : -INFINITY) : fmaf(__uint_as_float(v), inv_scale, s);
}

// The (b, h) slice of a mask with its 32 x 32 block loads.  `step` is the byte distance between
// the elements of consecutive accumulator rows (the key stride when keys sit on the accumulator
// rows, the query-row stride when query rows do); element i of a lane is read at voff plus the
// offset of its accumulator row, which is the same in every lane (a scalar offset).
template <typename T>
struct MaskSlice {
  __amdgpu_buffer_rsrc_t r;
  int sq, sk, kind;
  float inv_scale;
  bool packed;

  __device__ __forceinline__ MaskSlice(const MaskArgs& m, int b, int h) {
    const int es = m.kind == kMaskBool ? 1 : (int)sizeof(T);
    const unsigned long long addr =
        reinterpret_cast<unsigned long long>(m.ptr) + (unsigned long long)(b * m.sb + h * m.sh) * es;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)addr);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(addr >> 32));
    void* base = reinterpret_cast<void*>(((unsigned long long)hi << 32) | lo);
    r = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, __builtin_amdgcn_readfirstlane(m.bytes), kBufferWord3);
    sq = m.sq * es;
    sk = m.sk * es;
    kind = m.kind;
    inv_scale = m.inv_scale;
    packed = __builtin_amdgcn_readfirstlane(m.packed) != 0;
  }

  // raw values of the 16 elements of a lane (bool: the byte; additive: the bits as fp32).
  // Element i sits at voff + (8 (i >> 2) + (i & 3)) * step bytes: four runs of four, one load
  // per element.
  __device__ __forceinline__ void load(unsigned (&v)[16], int voff, int step) const {
    if (kind == kMaskBool) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b8(r, voff, uniform((8 * (i >> 2) + (i & 3)) * step), 0);
    } else if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        v[i] = (unsigned)__builtin_amdgcn_raw_buffer_load_b16(r, voff, uniform((8 * (i >> 2) + (i & 3)) * step), 0) << 16;
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, uniform((8 * (i >> 2) + (i & 3)) * step), 0);
    }
  }

  // load() along keys (step = sk) for a lane holding one query row.  In the packed layout a
  // boolean mask's block comes as words (below); with RUNS (kernels for additive masks of 2-byte
  // elements in that layout), an additive one likewise: its four runs are 8 bytes each, lanes l
  // and l + 32 load their halves of the row's 64 bytes (keys 16 h to 16 h + 15) in two 16-byte
  // loads and trade the 8-byte runs the other needs.  Per element, each load touched a cache line
  // per lane.  Called by the whole wave.
  template <bool RUNS = false>
  __device__ __forceinline__ void load_keys(unsigned (&v)[16], int voff) const {
    if (packed && kind == kMaskBool) {
      unsigned w[4];
      load_words(w, voff);
      expand_words(w, v);
    } else if (RUNS && sizeof(T) == 2 && packed && kind == kMaskAdd) {
      u32x4 x0, x1;
      load_run_pairs(voff, x0, x1);
      unsigned d[8];
      runs_of_pairs(x0, x1, d);
      expand_runs(d, v);
    } else {
      load(v, voff, sk);
    }
  }
  // the packed boolean layout's four runs as words (byte e of word j: element 4 j + e).  Lanes l
  // and l + 32 hold the same row, at keys 8 j + 4 h + e of the block (h = l / 32): each loads
  // its half of the row's 32 bytes (keys 16 h to 16 h + 15) in one 16-byte load
  // (load_word_pairs, voff the offset of the lane's element 0, keys contiguous), and the pair
  // trade the two words each needs from the other (words_of_pairs, by the whole wave, when the
  // words are needed: the trade waits for the load).  Four 4-byte loads per lane, each touching a
  // cache line per row, measured 0.13 ms of a masked forward that took 0.65 ms.
  __device__ __forceinline__ u32x4 load_word_pairs(int voff) const {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff + 12 * ((threadIdx.x >> 5) & 1), 0, 0);
  }
  static __device__ __forceinline__ void words_of_pairs(const u32x4& x, unsigned (&w)[4]) {
    const int h = (threadIdx.x >> 5) & 1;
    const unsigned lo = __shfl_xor(h ? x[0] : x[1], 32);
    const unsigned hi = __shfl_xor(h ? x[2] : x[3], 32);
    w[0] = h ? lo : x[0];
    w[1] = h ? hi : x[2];
    w[2] = h ? x[1] : lo;
    w[3] = h ? x[3] : hi;
  }
  __device__ __forceinline__ void load_words(unsigned (&w)[4], int voff) const {
    words_of_pairs(load_word_pairs(voff), w);
  }
  static __device__ __forceinline__ void expand_words(const unsigned (&w)[4], unsigned (&v)[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * j + e] = (w[j] >> (8 * e)) & 0xffu;
  }

  // The packed additive layout of 2-byte elements, the same way: lanes l and l + 32 load their
  // halves of the row's 64 bytes (keys 16 h to 16 h + 15, voff the offset of the lane's element
  // 0) in two 16-byte loads (load_run_pairs), and the trade hands each the two 8-byte runs it
  // needs from the other (runs_of_pairs, by the whole wave; run j of the lane, keys 8 j + 4 h to
  // 8 j + 4 h + 3, in d[2 j] and d[2 j + 1], two elements per dword, the lower key in the low half).
  __device__ __forceinline__ void load_run_pairs(int voff, u32x4& x0, u32x4& x1) const {
    const int o = voff + 24 * ((threadIdx.x >> 5) & 1);
    x0 = __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0);        // keys +0 to +7 of the half
    x1 = __builtin_amdgcn_raw_buffer_load_b128(r, o + 16, 0, 0);   // keys +8 to +15
  }
  static __device__ __forceinline__ void runs_of_pairs(const u32x4& x0, const u32x4& x1, unsigned (&d)[8]) {
    const int h = (threadIdx.x >> 5) & 1;
    // h = 0 keeps the runs at +0 and +8 of its half and sends +4 and +12; h = 1 the reverse
    const unsigned r0 = __shfl_xor(h ? x0[0] : x0[2], 32), r1 = __shfl_xor(h ? x0[1] : x0[3], 32);
    const unsigned r2 = __shfl_xor(h ? x1[0] : x1[2], 32), r3 = __shfl_xor(h ? x1[1] : x1[3], 32);
    d[0] = h ? r0 : x0[0];
    d[1] = h ? r1 : x0[1];
    d[2] = h ? r2 : x1[0];
    d[3] = h ? r3 : x1[1];
    d[4] = h ? x0[2] : r0;
    d[5] = h ? x0[3] : r1;
    d[6] = h ? x1[2] : r2;
    d[7] = h ? x1[3] : r3;
  }
  // the elements as load() gives them (bf16 bits in the high half of an fp32)
  static __device__ __forceinline__ void expand_runs(const unsigned (&d)[8], unsigned (&v)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = (i & 1) ? (d[i >> 1] & 0xffff0000u) : (d[i >> 1] << 16);
  }
  // Bit 15 and bit 31 of a dword of two bf16 elements: set where the element is not -inf (a kept
  // key), and where it is neither -inf nor +-0 (a bias that changes the score).  A 16-bit lane x
  // is nonzero iff bit 15 of ((x & 0x7fff) + 0x7fff) | x is set; the sum never carries out of it.
  static __device__ __forceinline__ unsigned kept_halves(unsigned dw) {
    const unsigned x = dw ^ 0xff80ff80u;
    return (((x & 0x7fff7fffu) + 0x7fff7fffu) | x) & 0x80008000u;
  }
  static __device__ __forceinline__ unsigned biased_halves(unsigned dw) {
    return ((dw & 0x7fff7fffu) + 0x7fff7fffu) & kept_halves(dw);
  }
  // Flags of a lane's runs as loaded (before the trade): `nz` nonzero when some element is not
  // +-0, `ni` nonzero when some element is not -inf.  Taken over the wave, they find the blocks
  // that are all zero or all -inf without the trade.
  static __device__ __forceinline__ void run_flags(const u32x4& x0, const u32x4& x1, unsigned& nz, unsigned& ni) {
    nz = 0;
    ni = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      nz |= (x0[i] | x1[i]) & 0x7fff7fffu;
      ni |= (x0[i] ^ 0xff80ff80u) | (x1[i] ^ 0xff80ff80u);
    }
  }
  // A 0 / -inf block as the boolean words above (byte e of word j: element 4 j + e, 0x80 where
  // kept, 0 where -inf): the bytes holding bits 15 and 31 of the two dwords' flags, by a byte
  // permute.  ORs into `biased` where an element is neither, and then the words do not describe
  // the block.
  static __device__ __forceinline__ void add_words_of_runs(const unsigned (&d)[8], unsigned (&w)[4],
                                                           unsigned& biased) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[j] = __builtin_amdgcn_perm(kept_halves(d[2 * j + 1]), kept_halves(d[2 * j]), 0x07050301u);
      biased |= biased_halves(d[2 * j]) | biased_halves(d[2 * j + 1]);
    }
  }

  // load() along query rows, where a zero stride (a mask broadcast over rows, as key padding is)
  // takes one load for all sixteen elements
  __device__ __forceinline__ void load_rows(unsigned (&v)[16], int voff, int step) const {
    if (step == 0) {
      unsigned x;
      if (kind == kMaskBool) x = __builtin_amdgcn_raw_buffer_load_b8(r, voff, 0, 0);
      else if constexpr (sizeof(T) == 2) x = (unsigned)__builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0) << 16;
      else x = __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = x;
      return;
    }
    load(v, voff, step);
  }

  __device__ __forceinline__ float apply(float s, unsigned v) const { return mask_value(kind, inv_scale, s, v); }
};

}  // namespace ra
