// ra_internal.h -- host-side problem descriptions and kernel launchers behind the C ABI.
// The ABI layer validates every argument first; launchers assume valid, non-empty problems.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ra {

struct AttnProblem {
  const void* q;
  const void* k;
  const void* v;
  int B, Hq, Hkv, Nq, Nk, D;
  bool causal;   // the causal kernels: key j allowed for query i iff j <= i + coff
  int coff;      // 0 top-left, Nk - Nq bottom-right, Nk for an explicit mask without causality
  float scale;
  bool bf16;     // false: fp32
  // explicit mask (kind 0: none); element strides, slice bytes as in MaskArgs (ra_device.h)
  const void* mask;
  int mask_kind;
  long long msb, msh;
  int msq, msk, mask_bytes;
  // NEOX rotary embedding fused into the kernels (rope): the forward rotates Q on load (rows at
  // q_pos, nullable: 0..Nq-1) and writes the rotated rows to q_rot when non-null; the backward
  // turns dQ and dK back (keys at k_pos, nullable: 0..Nk-1)
  bool rope = false;
  double rope_theta = 0.0;
  const int* q_pos = nullptr;
  const int* k_pos = nullptr;
  void* q_rot = nullptr;
};

// The rotary embedding of the fused entry points (theta, positions of query rows and keys).
struct RopeArgs {
  double theta;
  const int* q_pos;
  const int* k_pos;
};

// Forward: o (and stats when non-null); counters non-null selects the counting variant;
// o == nullptr computes the statistics only (stats must then be non-null).
hipError_t launch_attn_fwd(const AttnProblem& p, void* o, float* stats,
                           unsigned long long* counters, hipStream_t stream);

// Backward.  Workspace layout: see bwd_workspace_layout.
struct BwdWorkspace {
  float* stats;   // [B*Hq*Nq*2] (m, l), used when the caller passes none
  float* c;       // [B*Hq*Nq]  dO_i . O_i
  float* r;       // [B*Hq*Nq]  row-max gradient R_i
  int* amax;      // [B*Hq*Nq]  lowest key index of the row max
  float* kd;      // [B*Hq*Nq]  1 + (scale/16) m_i
  float* il;      // [B*Hq*Nq]  1 / l_i (0 when l_i = 0)
  float* cil;     // [B*Hq*Nq]  c_i / l_i
};
size_t bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq);
BwdWorkspace bwd_workspace_layout(void* base, int64_t B, int64_t Hq, int64_t Nq);
// phases: kBwdDq (dQ and the per-row terms c, R, argmax into ws), kBwdDkdv (dK, dV from those
// terms), or both.  stats == nullptr: the dQ phase recomputes (m, l) into ws.stats and the
// dK/dV phase reads them there.
enum { kBwdDq = 1, kBwdDkdv = 2, kBwdAll = 3 };
hipError_t launch_attn_bwd(const AttnProblem& p, const void* o, const void* d_o,
                           const float* stats, void* dq, void* dk, void* dv,
                           const BwdWorkspace& ws, int phases, hipStream_t stream);

// Split-KV decode (bf16 or fp32): R = (Hq / Hkv) * Nq <= 32 query rows per K/V head against caches of
// Nk rows, sample b using its first seqlens[b] (nullable: all).  causal: 0, 1 top-left,
// 2 bottom-right per sample.
struct DecodeProblem {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* stats;
  const int* seqlens;
  int B, Hq, Hkv, Nq, Nk, D;
  int causal;
  float scale;
  bool bf16;
};
// The bounds of the keys per wave (the launch picks the size inside them from the actual cache
// lengths), the most chunks a (batch, K/V head) group can take, the waves launched and the
// workspace carve-up: a function of the sizes only, so the size query and the launch agree.
struct DecodePlan {
  int64_t chunk_min, chunk_max, S, waves;
  size_t scores_bytes, pmax_bytes, psum_bytes, pacc_bytes, gmax_bytes, bytes;
};
DecodePlan decode_plan(int64_t B, int64_t Hkv, int64_t Nk, int64_t R, int64_t D);
hipError_t launch_attn_decode(const DecodeProblem& p, void* workspace, hipStream_t stream);

// Row softmax.
hipError_t launch_softmax_rows(const void* x, void* p, int64_t rows, int64_t cols, bool bf16,
                               hipStream_t stream);
hipError_t launch_softmax_rows_bwd(const void* x, const void* dp, void* dx, int64_t rows,
                                   int64_t cols, bool bf16, hipStream_t stream);

// NEOX rotary embedding of `mats` [N, D] matrices (positions nullable: 0..N-1).
hipError_t launch_rope_neox(const void* x, void* y, const int* positions, int64_t mats, int64_t N,
                            int64_t D, double theta, bool inverse, bool bf16, hipStream_t stream);

// Fill helpers (a kernel, not hipMemsetAsync, so the calls stay graph-capture friendly).
hipError_t launch_fill_u32(void* dst, uint32_t value, size_t count, hipStream_t stream);
hipError_t launch_fill_u16(void* dst, uint16_t value, size_t count, hipStream_t stream);
hipError_t launch_fill_pairs(float* dst, float a, float b, size_t pairs, hipStream_t stream);

}  // namespace ra
