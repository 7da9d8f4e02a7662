// ra_abi.hip -- the extern "C" entry points declared in include/ra_attn.h.
// Every check runs before any launch; on error nothing is launched or written.
#include <math.h>
#include <stdint.h>

#include "ra_attn.h"
#include "ra_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kIndexLimit = (int64_t)1 << 31;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return RA_OK;
  g_last_hip_error = (int)e;
  return RA_ERR_HIP;
}

// a * b * c < 2^31 for non-negative a, b, c, without overflow.
bool below_limit(int64_t a, int64_t b, int64_t c) {
  const __int128 prod = (__int128)a * (__int128)b * (__int128)c;
  return prod < (__int128)kIndexLimit;
}

// Shared validation of the attention size arguments.
int check_sizes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, float scale,
                int dtype) {
  if (dtype != RA_F32 && dtype != RA_BF16) return RA_ERR_DTYPE;
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0 || D < 0) return RA_ERR_SHAPE;
  if ((Hq > 0 || Hkv > 0) && (Hkv == 0 || Hq % Hkv != 0)) return RA_ERR_GQA;
  if (D != 64 && D != 128) return RA_ERR_HEADDIM;
  if (!(scale > 0.0f) || !isfinite(scale)) return RA_ERR_SCALE;
  if (!below_limit(Nq, D, 1) || !below_limit(Nk, D, 1)) return RA_ERR_TOO_LARGE;
  if (!below_limit(B, Hq, Nq) || !below_limit(B, Hkv, Nk)) return RA_ERR_TOO_LARGE;
  return RA_OK;
}

ra::AttnProblem make_problem(const void* q, const void* k, const void* v, int64_t B, int64_t Hq,
                             int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal, float scale,
                             int dtype) {
  ra::AttnProblem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.B = (int)B;
  p.Hq = (int)Hq;
  p.Hkv = (int)Hkv;
  p.Nq = (int)Nq;
  p.Nk = (int)Nk;
  p.D = (int)D;
  p.causal = causal != 0;
  p.scale = scale;
  p.bf16 = dtype == RA_BF16;
  return p;
}

size_t elem_size(int dtype) { return dtype == RA_BF16 ? 2 : 4; }

int fill_zero(void* dst, size_t elems, int dtype, hipStream_t s) {
  if (elems == 0) return RA_OK;
  if (dtype == RA_BF16) return hip_status(ra::launch_fill_u16(dst, 0, elems, s));
  return hip_status(ra::launch_fill_u32(dst, 0u, elems, s));
}

int fwd_common(const void* q, const void* k, const void* v, void* o, float* stats, int64_t B,
               int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal, float scale,
               int dtype, unsigned long long* counters, void* stream) {
  int st = check_sizes(B, Hq, Hkv, Nq, Nk, D, scale, dtype);
  if (st != RA_OK) return st;
  const int64_t rows = B * Hq * Nq;
  if (rows == 0) return RA_OK;
  if (q == nullptr || o == nullptr) return RA_ERR_NULLPTR;
  if (Nk > 0 && (k == nullptr || v == nullptr)) return RA_ERR_NULLPTR;
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(k, 16) || !aligned(v, 16)) return RA_ERR_ALIGN;
  if (stats != nullptr && !aligned(stats, 4)) return RA_ERR_ALIGN;
  if (counters != nullptr && !aligned(counters, 8)) return RA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (Nk == 0) {
    st = fill_zero(o, (size_t)rows * D, dtype, s);
    if (st == RA_OK && stats != nullptr)
      st = hip_status(ra::launch_fill_pairs(stats, -INFINITY, 0.0f, (size_t)rows, s));
    return st;
  }
  ra::AttnProblem p = make_problem(q, k, v, B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype);
  return hip_status(ra::launch_attn_fwd(p, o, stats, counters, s));
}

}  // namespace

extern "C" {

const char* ra_status_string(int status) {
  switch (status) {
    case RA_OK: return "RA_OK";
    case RA_ERR_NULLPTR: return "RA_ERR_NULLPTR: a required pointer is NULL";
    case RA_ERR_SHAPE: return "RA_ERR_SHAPE: negative or inconsistent size";
    case RA_ERR_GQA: return "RA_ERR_GQA: Hq must be a positive multiple of Hkv";
    case RA_ERR_HEADDIM: return "RA_ERR_HEADDIM: head dim must be 64 or 128";
    case RA_ERR_DTYPE: return "RA_ERR_DTYPE: dtype must be RA_F32 or RA_BF16";
    case RA_ERR_SCALE: return "RA_ERR_SCALE: scale must be finite and > 0";
    case RA_ERR_WORKSPACE: return "RA_ERR_WORKSPACE: workspace missing or too small";
    case RA_ERR_ALIGN: return "RA_ERR_ALIGN: pointer misaligned";
    case RA_ERR_TOO_LARGE: return "RA_ERR_TOO_LARGE: size beyond the supported index range";
    case RA_ERR_HIP: return "RA_ERR_HIP: HIP runtime error at launch";
    default: return "unknown ra_status";
  }
}

int ra_last_hip_error(void) { return g_last_hip_error; }

int ra_attn_fwd(const void* q, const void* k, const void* v, void* o, float* stats, int64_t B,
                int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal, float scale,
                int dtype, void* stream) {
  return fwd_common(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype, nullptr, stream);
}

int ra_attn_fwd_counted(const void* q, const void* k, const void* v, void* o, float* stats,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                        int causal, float scale, int dtype, unsigned long long* counters,
                        void* stream) {
  if (counters == nullptr) return RA_ERR_NULLPTR;
  return fwd_common(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype, counters,
                    stream);
}

size_t ra_attn_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                                   int64_t D, int dtype) {
  if (check_sizes(B, Hq, Hkv, Nq, Nk, D, 1.0f, dtype) != RA_OK) return 0;
  return ra::bwd_workspace_bytes(B, Hq, Nq);
}

// Shared by ra_attn_bwd and its two phases.  A phase's own outputs and inputs are required;
// the rest may be NULL.
static int attn_bwd_common(const void* q, const void* k, const void* v, const void* o,
                           const void* d_o, const float* stats, void* dq, void* dk, void* dv,
                           const void* workspace, size_t workspace_bytes, int64_t B, int64_t Hq,
                           int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal, float scale,
                           int dtype, int phases, void* stream) {
  int st = check_sizes(B, Hq, Hkv, Nq, Nk, D, scale, dtype);
  if (st != RA_OK) return st;
  const int64_t qrows = B * Hq * Nq, krows = B * Hkv * Nk;
  if (qrows == 0 && krows == 0) return RA_OK;
  const bool need_q = qrows > 0, need_k = krows > 0;
  const bool ph_dq = (phases & ra::kBwdDq) != 0, ph_kv = (phases & ra::kBwdDkdv) != 0;
  if (need_q && (q == nullptr || d_o == nullptr)) return RA_ERR_NULLPTR;
  if (need_q && ph_dq && (dq == nullptr || o == nullptr)) return RA_ERR_NULLPTR;
  if (need_k && (k == nullptr || v == nullptr)) return RA_ERR_NULLPTR;
  if (need_k && ph_kv && (dk == nullptr || dv == nullptr)) return RA_ERR_NULLPTR;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(d_o, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return RA_ERR_ALIGN;
  if (stats != nullptr && !aligned(stats, 4)) return RA_ERR_ALIGN;
  const size_t need_ws = ra::bwd_workspace_bytes(B, Hq, Nq);
  if (need_q && need_k) {
    if (workspace == nullptr || workspace_bytes < need_ws) return RA_ERR_WORKSPACE;
    if (!aligned(workspace, 4)) return RA_ERR_ALIGN;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!need_k) return ph_dq ? fill_zero(dq, (size_t)qrows * D, dtype, s) : RA_OK;   // Nk == 0
  if (!need_q) {                                                                      // no query rows
    if (!ph_kv) return RA_OK;
    st = fill_zero(dk, (size_t)krows * D, dtype, s);
    if (st == RA_OK) st = fill_zero(dv, (size_t)krows * D, dtype, s);
    return st;
  }
  ra::AttnProblem p = make_problem(q, k, v, B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype);
  ra::BwdWorkspace ws = ra::bwd_workspace_layout(const_cast<void*>(workspace), B, Hq, Nq);
  return hip_status(ra::launch_attn_bwd(p, o, d_o, stats, dq, dk, dv, ws, phases, s));
}

int ra_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                const float* stats, void* dq, void* dk, void* dv, void* workspace,
                size_t workspace_bytes, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                int64_t D, int causal, float scale, int dtype, void* stream) {
  return attn_bwd_common(q, k, v, o, d_o, stats, dq, dk, dv, workspace, workspace_bytes, B, Hq,
                         Hkv, Nq, Nk, D, causal, scale, dtype, ra::kBwdAll, stream);
}

int ra_attn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                   const float* stats, void* dq, void* workspace, size_t workspace_bytes,
                   int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                   int causal, float scale, int dtype, void* stream) {
  return attn_bwd_common(q, k, v, o, d_o, stats, dq, nullptr, nullptr, workspace, workspace_bytes,
                         B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype, ra::kBwdDq, stream);
}

int ra_attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* d_o,
                     const float* stats, void* dk, void* dv, const void* workspace,
                     size_t workspace_bytes, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                     int64_t Nk, int64_t D, int causal, float scale, int dtype, void* stream) {
  return attn_bwd_common(q, k, v, nullptr, d_o, stats, nullptr, dk, dv, workspace, workspace_bytes,
                         B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype, ra::kBwdDkdv, stream);
}

int ra_softmax_rows(const void* x, void* p, int64_t rows, int64_t cols, int dtype, void* stream) {
  if (dtype != RA_F32 && dtype != RA_BF16) return RA_ERR_DTYPE;
  if (rows < 0 || cols < 0) return RA_ERR_SHAPE;
  if (rows >= kIndexLimit || cols >= kIndexLimit) return RA_ERR_TOO_LARGE;
  if (rows == 0 || cols == 0) return RA_OK;
  if (x == nullptr || p == nullptr) return RA_ERR_NULLPTR;
  if (!aligned(x, elem_size(dtype)) || !aligned(p, elem_size(dtype))) return RA_ERR_ALIGN;
  return hip_status(ra::launch_softmax_rows(x, p, rows, cols, dtype == RA_BF16,
                                            static_cast<hipStream_t>(stream)));
}

int ra_softmax_rows_bwd(const void* x, const void* dp, void* dx, int64_t rows, int64_t cols,
                        int dtype, void* stream) {
  if (dtype != RA_F32 && dtype != RA_BF16) return RA_ERR_DTYPE;
  if (rows < 0 || cols < 0) return RA_ERR_SHAPE;
  if (rows >= kIndexLimit || cols >= kIndexLimit) return RA_ERR_TOO_LARGE;
  if (rows == 0 || cols == 0) return RA_OK;
  if (x == nullptr || dp == nullptr || dx == nullptr) return RA_ERR_NULLPTR;
  const int es = elem_size(dtype);
  if (!aligned(x, es) || !aligned(dp, es) || !aligned(dx, es)) return RA_ERR_ALIGN;
  return hip_status(ra::launch_softmax_rows_bwd(x, dp, dx, rows, cols, dtype == RA_BF16,
                                                static_cast<hipStream_t>(stream)));
}

int ra_rope_neox(const void* x, void* y, const int32_t* positions, int64_t mats, int64_t N,
                 int64_t D, double theta, int inverse, int dtype, void* stream) {
  if (dtype != RA_F32 && dtype != RA_BF16) return RA_ERR_DTYPE;
  if (mats < 0 || N < 0 || D < 0) return RA_ERR_SHAPE;
  if (D % 2 != 0) return RA_ERR_HEADDIM;
  if (!(theta > 0.0) || !isfinite(theta)) return RA_ERR_SCALE;
  if (N >= kIndexLimit || D >= kIndexLimit || (__int128)N * D >= kIndexLimit) return RA_ERR_TOO_LARGE;
  if (mats == 0 || N == 0 || D == 0) return RA_OK;
  if (x == nullptr || y == nullptr) return RA_ERR_NULLPTR;
  const int es = elem_size(dtype);
  if (!aligned(x, es) || !aligned(y, es) || (positions != nullptr && !aligned(positions, 4)))
    return RA_ERR_ALIGN;
  return hip_status(ra::launch_rope_neox(x, y, positions, mats, N, D, theta, inverse != 0,
                                         dtype == RA_BF16, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
