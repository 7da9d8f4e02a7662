// ra_abi.hip -- the extern "C" entry points declared in include/ra_attn.h.
// Every check runs before any launch; on error nothing is launched or written.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "ra_attn.h"
#include "ra_device.h"
#include "ra_internal.h"

static_assert(RA_MASK_BOOL == ra::kMaskBool && RA_MASK_ADD == ra::kMaskAdd && RA_MASK_NONE == ra::kMaskNone,
              "mask kinds of the ABI and the kernels agree");

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kIndexLimit = (int64_t)1 << 31;
// Rows past the end of a matrix that a tile may address (the largest tile is 256 rows).
constexpr int64_t kTailRows = 256;

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
  // The kernels form byte offsets inside one head's [N, D] matrix (buffer sizes, tile offsets,
  // including a tile tail of up to kTailRows rows past the end) in signed 32-bit integers.
  const int64_t row_bytes = D * (dtype == RA_BF16 ? 2 : 4);
  if (!below_limit(Nq + kTailRows, row_bytes, 1) || !below_limit(Nk + kTailRows, row_bytes, 1))
    return RA_ERR_TOO_LARGE;
  if (!below_limit(B, Hq, Nq) || !below_limit(B, Hkv, Nk)) return RA_ERR_TOO_LARGE;
  return RA_OK;
}

size_t elem_size(int dtype) { return dtype == RA_BF16 ? 2 : 4; }

bool mask_present(const ra_mask* mask) { return mask != nullptr && mask->kind != RA_MASK_NONE; }

// The causal mode and the mask descriptor.  Besides the slice itself, every offset a kernel
// forms (tile tails included: up to 64 query rows past Nq and 128 keys past Nk) must stay below
// 2^31 bytes; the kernels read those tails through a resource that ends at the slice.
int check_mask(const ra_mask* mask, int causal, int64_t B, int64_t Hq, int64_t Nq, int64_t Nk,
               int dtype) {
  if (causal != RA_CAUSAL_NONE && causal != RA_CAUSAL_TOP_LEFT && causal != RA_CAUSAL_BOTTOM_RIGHT)
    return RA_ERR_MASK;
  if (!mask_present(mask)) return RA_OK;
  if (mask->kind != RA_MASK_BOOL && mask->kind != RA_MASK_ADD) return RA_ERR_MASK;
  if (mask->stride_b < 0 || mask->stride_h < 0 || mask->stride_q < 0 || mask->stride_k < 0)
    return RA_ERR_MASK;
  if (B * Hq * Nq > 0 && Nk > 0 && mask->data == nullptr) return RA_ERR_NULLPTR;
  const int64_t es = mask->kind == RA_MASK_BOOL ? 1 : (int64_t)elem_size(dtype);
  if (!aligned(mask->data, (uintptr_t)es)) return RA_ERR_ALIGN;
  const __int128 reach = ((__int128)(Nq + 64) * mask->stride_q + (__int128)(Nk + 128) * mask->stride_k + 1) * es;
  if (reach >= (__int128)kIndexLimit) return RA_ERR_TOO_LARGE;
  const __int128 heads = ((__int128)(B > 0 ? B - 1 : 0) * mask->stride_b +
                          (__int128)(Hq > 0 ? Hq - 1 : 0) * mask->stride_h) * es;
  if (heads >= ((__int128)1 << 62)) return RA_ERR_TOO_LARGE;
  return RA_OK;
}

ra::AttnProblem make_problem(const void* q, const void* k, const void* v, int64_t B, int64_t Hq,
                             int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal, float scale,
                             int dtype, const ra_mask* mask) {
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
  p.scale = scale;
  p.bf16 = dtype == RA_BF16;
  const bool masked = mask_present(mask);
  // the masked kernels always test the causal diagonal; without causality it sits past the keys
  p.causal = causal != RA_CAUSAL_NONE || masked;
  p.coff = causal == RA_CAUSAL_BOTTOM_RIGHT ? (int)(Nk - Nq) : causal == RA_CAUSAL_TOP_LEFT ? 0 : (int)Nk;
  p.mask = masked ? mask->data : nullptr;
  p.mask_kind = masked ? mask->kind : RA_MASK_NONE;
  p.msb = masked ? mask->stride_b : 0;
  p.msh = masked ? mask->stride_h : 0;
  p.msq = masked ? (int)mask->stride_q : 0;
  p.msk = masked ? (int)mask->stride_k : 0;
  const int64_t es = masked && mask->kind == RA_MASK_BOOL ? 1 : (int64_t)elem_size(dtype);
  p.mask_bytes = masked ? (int)(((Nq - 1) * mask->stride_q + (Nk - 1) * mask->stride_k + 1) * es) : 0;
  return p;
}

int fill_zero(void* dst, size_t elems, int dtype, hipStream_t s) {
  if (elems == 0) return RA_OK;
  if (dtype == RA_BF16) return hip_status(ra::launch_fill_u16(dst, 0, elems, s));
  return hip_status(ra::launch_fill_u32(dst, 0u, elems, s));
}

int fwd_common(const void* q, const void* k, const void* v, void* o, float* stats, int64_t B,
               int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal, float scale,
               int dtype, const ra_mask* mask, unsigned long long* counters, void* stream) {
  int st = check_sizes(B, Hq, Hkv, Nq, Nk, D, scale, dtype);
  if (st != RA_OK) return st;
  st = check_mask(mask, causal, B, Hq, Nq, Nk, dtype);
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
  ra::AttnProblem p = make_problem(q, k, v, B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype, mask);
  return hip_status(ra::launch_attn_fwd(p, o, stats, counters, s));
}

}  // namespace

// ---- the backward for callers that cannot allocate device memory
// Its per-row terms live in `scratch`, a fixed array of the library's code object (one copy per
// device, held from the code object's load on that device until the process ends).  In host code
// `scratch` only names the host-side shadow of the array; its device address comes from
// hipGetSymbolAddress, resolved once per device with that device current, and only that address
// is passed to kernels.  Every call on a device shares the device's copy: calls that overlap on
// one device race.
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, once resolved

// Device address of `scratch` on the current device.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return hip_status(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (p == nullptr) return hip_status(hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return RA_OK;
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
    case RA_ERR_MASK: return "RA_ERR_MASK: invalid causal mode or mask descriptor";
    default: return "unknown ra_status";
  }
}

int ra_last_hip_error(void) { return g_last_hip_error; }

int ra_attn_fwd(const void* q, const void* k, const void* v, void* o, float* stats, int64_t B,
                int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal, float scale,
                int dtype, void* stream) {
  return fwd_common(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype, nullptr, nullptr,
                    stream);
}

int ra_attn_fwd_masked(const void* q, const void* k, const void* v, void* o, float* stats,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                       int causal, float scale, int dtype, const ra_mask* mask, void* stream) {
  return fwd_common(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype, mask, nullptr,
                    stream);
}

int ra_attn_fwd_counted(const void* q, const void* k, const void* v, void* o, float* stats,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                        int causal, float scale, int dtype, unsigned long long* counters,
                        void* stream) {
  if (counters == nullptr) return RA_ERR_NULLPTR;
  return fwd_common(q, k, v, o, stats, B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype, nullptr, counters,
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
                           int dtype, const ra_mask* mask, int phases, void* stream,
                           const ra::RopeArgs* rope = nullptr) {
  int st = check_sizes(B, Hq, Hkv, Nq, Nk, D, scale, dtype);
  if (st != RA_OK) return st;
  st = check_mask(mask, causal, B, Hq, Nq, Nk, dtype);
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
  ra::AttnProblem p = make_problem(q, k, v, B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype, mask);
  if (rope != nullptr) {
    p.rope = true;
    p.rope_theta = rope->theta;
    p.q_pos = rope->q_pos;
    p.k_pos = rope->k_pos;
  }
  ra::BwdWorkspace ws = ra::bwd_workspace_layout(const_cast<void*>(workspace), B, Hq, Nq);
  return hip_status(ra::launch_attn_bwd(p, o, d_o, stats, dq, dk, dv, ws, phases, s));
}

int ra_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                const float* stats, void* dq, void* dk, void* dv, void* workspace,
                size_t workspace_bytes, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                int64_t D, int causal, float scale, int dtype, void* stream) {
  return attn_bwd_common(q, k, v, o, d_o, stats, dq, dk, dv, workspace, workspace_bytes, B, Hq,
                         Hkv, Nq, Nk, D, causal, scale, dtype, nullptr, ra::kBwdAll, stream);
}

int ra_attn_bwd_masked(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                       const float* stats, void* dq, void* dk, void* dv, void* workspace,
                       size_t workspace_bytes, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                       int64_t Nk, int64_t D, int causal, float scale, int dtype,
                       const ra_mask* mask, void* stream) {
  return attn_bwd_common(q, k, v, o, d_o, stats, dq, dk, dv, workspace, workspace_bytes, B, Hq,
                         Hkv, Nq, Nk, D, causal, scale, dtype, mask, ra::kBwdAll, stream);
}

int ra_attn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                   const float* stats, void* dq, void* workspace, size_t workspace_bytes,
                   int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                   int causal, float scale, int dtype, void* stream) {
  return attn_bwd_common(q, k, v, o, d_o, stats, dq, nullptr, nullptr, workspace, workspace_bytes,
                         B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype, nullptr, ra::kBwdDq, stream);
}

int ra_attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* d_o,
                     const float* stats, void* dk, void* dv, const void* workspace,
                     size_t workspace_bytes, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                     int64_t Nk, int64_t D, int causal, float scale, int dtype, void* stream) {
  return attn_bwd_common(q, k, v, nullptr, d_o, stats, nullptr, dk, dv, workspace, workspace_bytes,
                         B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype, nullptr, ra::kBwdDkdv, stream);
}

// ra_attn_bwd with its workspace in `scratch` (declared above); allocates nothing.
int ra_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                        const void* d_o, const float* stats, void* dq, void* dk, void* dv,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                        int causal, float scale, int dtype, void* stream) {
  int st = check_sizes(B, Hq, Hkv, Nq, Nk, D, scale, dtype);   // bounds the products below
  if (st != RA_OK) return st;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (B * Hq * Nq > 0 && B * Hkv * Nk > 0) {   // the only case that uses a workspace
    if (ra::bwd_workspace_bytes(B, Hq, Nq) > kNoallocScratchBytes) return RA_ERR_TOO_LARGE;
    st = scratch_address(&ws);
    if (st != RA_OK) return st;
    ws_bytes = kNoallocScratchBytes;
  }
  return attn_bwd_common(q, k, v, o, d_o, stats, dq, dk, dv, ws, ws_bytes, B, Hq, Hkv, Nq, Nk, D,
                         causal, scale, dtype, nullptr, ra::kBwdAll, stream);
}

// ---- attention with the NEOX rotary embedding fused in
static int check_rope(double theta, int dtype, const int32_t* q_positions, const int32_t* k_positions) {
  if (dtype != RA_BF16 && dtype != RA_F32) return RA_ERR_DTYPE;
  if (!(theta > 0.0) || !isfinite(theta)) return RA_ERR_SCALE;
  if ((q_positions != nullptr && !aligned(q_positions, 4)) || (k_positions != nullptr && !aligned(k_positions, 4)))
    return RA_ERR_ALIGN;
  return RA_OK;
}

int ra_attn_fwd_rope(const void* q, const void* k, const void* v, void* o, float* stats, void* q_rot,
                     void* k_rot, const int32_t* q_positions, const int32_t* k_positions, double theta,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal,
                     float scale, int dtype, const ra_mask* mask, void* stream) {
  int st = check_sizes(B, Hq, Hkv, Nq, Nk, D, scale, dtype);
  if (st != RA_OK) return st;
  st = check_mask(mask, causal, B, Hq, Nq, Nk, dtype);
  if (st != RA_OK) return st;
  st = check_rope(theta, dtype, q_positions, k_positions);
  if (st != RA_OK) return st;
  const int64_t rows = B * Hq * Nq;
  if (rows == 0) return RA_OK;
  if (q == nullptr || o == nullptr) return RA_ERR_NULLPTR;
  if (Nk > 0 && (k == nullptr || v == nullptr || k_rot == nullptr)) return RA_ERR_NULLPTR;
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(q_rot, 16) ||
      !aligned(k_rot, 16))
    return RA_ERR_ALIGN;
  if (stats != nullptr && !aligned(stats, 4)) return RA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (Nk == 0) {   // no key: o = 0; the rotated queries are still produced when asked for
    st = fill_zero(o, (size_t)rows * D, dtype, s);
    if (st == RA_OK && stats != nullptr)
      st = hip_status(ra::launch_fill_pairs(stats, -INFINITY, 0.0f, (size_t)rows, s));
    if (st == RA_OK && q_rot != nullptr)
      st = hip_status(ra::launch_rope_neox(q, q_rot, q_positions, B * Hq, Nq, D, theta, false, dtype == RA_BF16, s));
    return st;
  }
  // K once, by the standalone rotation, into k_rot; Q in the attention kernel, on load
  st = hip_status(ra::launch_rope_neox(k, k_rot, k_positions, B * Hkv, Nk, D, theta, false, dtype == RA_BF16, s));
  if (st != RA_OK) return st;
  ra::AttnProblem p = make_problem(q, k_rot, v, B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype, mask);
  p.rope = true;
  p.rope_theta = theta;
  p.q_pos = q_positions;
  p.q_rot = q_rot;
  return hip_status(ra::launch_attn_fwd(p, o, stats, nullptr, s));
}

int ra_attn_bwd_rope(const void* q_rot, const void* k_rot, const void* v, const void* o,
                     const void* d_o, const float* stats, void* dq, void* dk, void* dv, void* workspace,
                     size_t workspace_bytes, const int32_t* q_positions, const int32_t* k_positions,
                     double theta, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                     int causal, float scale, int dtype, const ra_mask* mask, void* stream) {
  int st = check_rope(theta, dtype, q_positions, k_positions);
  if (st != RA_OK) return st;
  ra::RopeArgs rope;
  rope.theta = theta;
  rope.q_pos = q_positions;
  rope.k_pos = k_positions;
  return attn_bwd_common(q_rot, k_rot, v, o, d_o, stats, dq, dk, dv, workspace, workspace_bytes, B, Hq,
                         Hkv, Nq, Nk, D, causal, scale, dtype, mask, ra::kBwdAll, stream, &rope);
}

// Decode: the query rows of one K/V head (rep * Nq) must fit one wave's 32 MFMA columns.
static int check_decode(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                        int causal, float scale, int dtype) {
  int st = check_sizes(B, Hq, Hkv, Nq, Nk, D, scale, dtype);
  if (st != RA_OK) return st;
  if (causal != RA_CAUSAL_NONE && causal != RA_CAUSAL_TOP_LEFT && causal != RA_CAUSAL_BOTTOM_RIGHT)
    return RA_ERR_MASK;
  if (Hkv > 0 && (Hq / Hkv) * Nq > 32) return RA_ERR_SHAPE;
  return RA_OK;
}

size_t ra_attn_decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                                      int64_t D, int dtype) {
  if (check_decode(B, Hq, Hkv, Nq, Nk, D, RA_CAUSAL_NONE, 1.0f, dtype) != RA_OK) return 0;
  if (B * Hq * Nq == 0 || Nk == 0) return 0;
  return ra::decode_plan(B, Hkv, Nk, (Hq / Hkv) * Nq, D).bytes;
}

int ra_attn_decode(const void* q, const void* k, const void* v, void* o, float* stats,
                   const int32_t* seqlens, void* workspace, size_t workspace_bytes, int64_t B,
                   int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal,
                   float scale, int dtype, void* stream) {
  int st = check_decode(B, Hq, Hkv, Nq, Nk, D, causal, scale, dtype);
  if (st != RA_OK) return st;
  const int64_t rows = B * Hq * Nq;
  if (rows == 0) return RA_OK;
  if (q == nullptr || o == nullptr) return RA_ERR_NULLPTR;
  if (Nk > 0 && (k == nullptr || v == nullptr)) return RA_ERR_NULLPTR;
  if (!aligned(q, 16) || !aligned(o, 16) || !aligned(k, 16) || !aligned(v, 16)) return RA_ERR_ALIGN;
  if ((stats != nullptr && !aligned(stats, 4)) || (seqlens != nullptr && !aligned(seqlens, 4)))
    return RA_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (Nk == 0) {
    st = fill_zero(o, (size_t)rows * D, dtype, s);
    if (st == RA_OK && stats != nullptr)
      st = hip_status(ra::launch_fill_pairs(stats, -INFINITY, 0.0f, (size_t)rows, s));
    return st;
  }
  const size_t need = ra::decode_plan(B, Hkv, Nk, (Hq / Hkv) * Nq, D).bytes;
  if (workspace == nullptr || workspace_bytes < need) return RA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return RA_ERR_ALIGN;
  ra::DecodeProblem p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.stats = stats;
  p.seqlens = seqlens;
  p.B = (int)B;
  p.Hq = (int)Hq;
  p.Hkv = (int)Hkv;
  p.Nq = (int)Nq;
  p.Nk = (int)Nk;
  p.D = (int)D;
  p.causal = causal;
  p.scale = scale;
  p.bf16 = dtype == RA_BF16;
  return hip_status(ra::launch_attn_decode(p, workspace, s));
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
