/*
 * ra_attn.h -- C ABI of the rational-softmax attention library for AMD gfx950 (MI355X).
 *
 * The operation ("Ra-Family: Rational Neural Architecture", section 3 "Rational Attention &
 * Softmax"): for each row of scores s, Delta_j = max(s) - s_j, u_j = Delta_j / 16,
 * phi_j = ((1 - u_j) / (1 + u_j))^8 when u_j < 1 and exactly 0 otherwise, p_j = phi_j / sum(phi).
 * Attention computes O = p(scale * Q K^T) V tile by tile without storing the score matrix
 * (same section, item ra_attention, the functional drop-in for scaled_dot_product_attention).
 * Grouped-query attention: query head h reads K/V head h / (Hq / Hkv) (noeira "Primitives"
 * page, section "Attention and transformers", RepeatKVHeads).
 *
 * Conventions shared by every entry point
 *   - Tensors are contiguous, row-major, in device memory: q, o, dq, d_o are [B, Hq, Nq, D];
 *     k, v, dk, dv are [B, Hkv, Nk, D].  Output dtype equals input dtype.
 *   - dtype: RA_F32 (fp32 storage, fp32 matrix-core products) or RA_BF16 (bf16 storage,
 *     fp32 accumulation; probabilities are rounded to bf16 to nearest-even before the
 *     P.V product).
 *   - causal: RA_CAUSAL_NONE (0); RA_CAUSAL_TOP_LEFT (1) allows key j for query i iff j <= i
 *     (scaled_dot_product_attention's is_causal); RA_CAUSAL_BOTTOM_RIGHT (2) allows j <= i +
 *     Nk - Nq, so the last query sees every key (queries that continue the key sequence; the
 *     pages fix no alignment for Nq != Nk, and the two agree when Nq == Nk).  Any other value
 *     -> RA_ERR_MASK.  Masked keys get p = 0 and take no part in the row max or the sum of
 *     phi.  A query row with no allowed key gives o = 0 (stats m = -inf, l = 0) and dq = 0,
 *     not NaN ("Primitives" page, CrossAttention: a fully masked row gives a zero context).
 *   - stream is a hipStream_t (NULL = the default stream).  Kernels run asynchronously on it;
 *     the caller keeps every buffer alive until the stream has passed the call.
 *   - The caller owns all memory.  The library allocates nothing, frees nothing, does not
 *     synchronise, keeps no pointer after returning and holds no global state; calls are
 *     thread-safe.
 *   - Every argument check runs before any launch: on an error status nothing is launched and
 *     no output is written.  A failed launch returns RA_ERR_HIP.  Nothing is printed, nothing
 *     aborts, no C++ exception crosses the ABI.
 *   - Device tensors must be 16-byte aligned; stats and workspace 4-byte aligned.
 *   - Supported head dims: D = 64 and D = 128.  scale must be finite and > 0.
 *   - Inputs are assumed finite; NaN or Inf inputs give unspecified outputs.
 */
#ifndef RA_ATTN_H
#define RA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ra_dtype { RA_F32 = 0, RA_BF16 = 1 } ra_dtype;

typedef enum ra_status {
  RA_OK = 0,
  RA_ERR_NULLPTR = 1,   /* a required pointer is NULL */
  RA_ERR_SHAPE = 2,     /* a size is negative or B/H/N inconsistent */
  RA_ERR_GQA = 3,       /* Hkv == 0 with Hq > 0, or Hq is not a multiple of Hkv */
  RA_ERR_HEADDIM = 4,   /* D not in {64, 128} */
  RA_ERR_DTYPE = 5,     /* dtype not RA_F32 / RA_BF16 */
  RA_ERR_SCALE = 6,     /* scale not finite or <= 0 */
  RA_ERR_WORKSPACE = 7, /* workspace NULL or smaller than ra_attn_bwd_workspace_bytes */
  RA_ERR_ALIGN = 8,     /* a pointer breaks the alignment rule above */
  RA_ERR_TOO_LARGE = 9, /* a size exceeds the library's index range (see each call) */
  RA_ERR_HIP = 10,      /* the HIP runtime reported an error at launch */
  RA_ERR_MASK = 11      /* causal mode not 0/1/2, or an invalid ra_mask (kind, strides) */
} ra_status;

typedef enum ra_causal {
  RA_CAUSAL_NONE = 0,
  RA_CAUSAL_TOP_LEFT = 1,
  RA_CAUSAL_BOTTOM_RIGHT = 2
} ra_causal;

/*
 * ra_mask -- an explicit attention mask, the attn_mask of the scaled_dot_product_attention
 * drop-in (Ra-Family page, section 3, item ra_attention) and the CrossAttention key padding
 * mask ("Primitives" page, section "Attention and transformers": 1 = attend, 0 = ignore).
 *   Element (b, h, i, j) -- batch b, query head h, query row i, key j -- is read at element
 *   offset b*stride_b + h*stride_h + i*stride_q + j*stride_k of data (device memory; strides
 *   >= 0, a zero stride broadcasts).  A [B, Nk] key padding mask is strides (Nk, 0, 0, 1); one
 *   [Nq, Nk] mask shared by every batch and head is (0, 0, Nk, 1).
 *   kind RA_MASK_BOOL: uint8 elements, nonzero = attend, zero = masked.
 *   kind RA_MASK_ADD: elements of the attention dtype (fp32 or bf16), added to the scaled score
 *     scale * q_i . k_j before the row max; -inf masks the entry.  Finite values or -inf only.
 *   kind RA_MASK_NONE (or a NULL ra_mask pointer): no mask.
 *   The mask is an input constant: no gradient is computed for it.
 *   Limits: every offset of one (b, h) slice plus tile tails, ((Nq + 64) * stride_q +
 *   (Nk + 128) * stride_k + 1) elements, below 2^31 bytes -> else RA_ERR_TOO_LARGE.
 *   data must be aligned to its element size (RA_ERR_ALIGN).
 */
typedef enum ra_mask_kind { RA_MASK_NONE = 0, RA_MASK_BOOL = 1, RA_MASK_ADD = 2 } ra_mask_kind;

typedef struct ra_mask {
  const void* data;
  int kind;
  int64_t stride_b, stride_h, stride_q, stride_k;
} ra_mask;

/* Human-readable name of a status code (static storage; never NULL). */
const char* ra_status_string(int status);

/* HIP error code (hipError_t as int) behind the last RA_ERR_HIP returned on this thread. */
int ra_last_hip_error(void);

/*
 * ra_attn_fwd -- forward rational-softmax attention.
 *   Source: Ra-Family page, section 3, items ra_softmax and ra_attention.
 *   o[b,h,i,:] = sum_j p_ij v[b,g,j,:], p_i = ra_softmax(scale * q[b,h,i,:] . k[b,g,j,:] over
 *   the allowed keys j), g = h / (Hq / Hkv).
 *   stats: optional (NULL to skip), float [B, Hq, Nq, 2]: (m, l) per query row, where m is the
 *   row max of the UNSCALED dot products q_i . k_j (the score max is scale * m) and l is the
 *   sum of phi.  ra_attn_bwd consumes it unchanged.
 *   Two passes over the keys: the first finds m, the second evaluates phi, sum(phi) and P.V;
 *   a key tile whose entries all lie outside the compact support (u >= 1) for a group of
 *   query rows is skipped for them, which leaves the result bit-identical.
 *   Sizes: B*Hq*Nq == 0 -> RA_OK, nothing launched.  Nk == 0 -> o = 0 (and stats m = -inf,
 *   l = 0): a row with no allowed key yields a zero output, not NaN.
 *   Limits (RA_ERR_TOO_LARGE otherwise): (Nq + 256) * D * elem_size and (Nk + 256) * D *
 *   elem_size below 2^31 bytes (elem_size 2 for RA_BF16, 4 for RA_F32: the kernels form byte
 *   offsets inside one head's matrix, tile tails included, in 32-bit integers), and
 *   B * Hq * Nq, B * Hkv * Nk below 2^31.
 */
int ra_attn_fwd(const void* q, const void* k, const void* v, void* o, float* stats,
                int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                int causal, float scale, int dtype, void* stream);

/*
 * ra_attn_fwd_masked -- ra_attn_fwd with an explicit mask (see ra_mask; NULL = none), on top
 *   of the causal mode.  p_i = ra_softmax over the allowed keys of scale * q_i . k_j (+ the
 *   additive mask).  stats m is then the row max of q_i . k_j + mask_ij / scale (the unscaled
 *   units of ra_attn_fwd).  Same checks, sizes and limits as ra_attn_fwd, plus the ra_mask
 *   checks (RA_ERR_MASK, RA_ERR_ALIGN, RA_ERR_TOO_LARGE).
 */
int ra_attn_fwd_masked(const void* q, const void* k, const void* v, void* o, float* stats,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                       int causal, float scale, int dtype, const ra_mask* mask, void* stream);

/*
 * ra_attn_fwd_counted -- ra_attn_fwd plus tile-skip counters (diagnostics, not for timing).
 *   counters: device pointer to 4 uint64, which the call ADDS to (zero them first):
 *     [0] (wave, key-tile) pairs inside the causal range of the second pass (a wave holds 32
 *         query rows, a key tile 64 keys for bf16 and 32 for fp32),
 *     [1] of those, pairs skipped because every entry lies outside the support (skipped by the
 *         wave alone or by its whole workgroup),
 *     [2] (workgroup, key-tile) pairs of the second pass,
 *     [3] of those, tiles whose K/V load was skipped for the whole workgroup.
 *   Everything else as ra_attn_fwd.
 */
int ra_attn_fwd_counted(const void* q, const void* k, const void* v, void* o, float* stats,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                        int64_t D, int causal, float scale, int dtype,
                        unsigned long long* counters, void* stream);

/*
 * ra_attn_bwd_workspace_bytes -- size of the scratch buffer ra_attn_bwd needs (0 on invalid
 * sizes).  The caller allocates it; its contents need not be initialised.
 */
size_t ra_attn_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                                   int64_t D, int dtype);

/*
 * ra_attn_bwd -- gradients of L = sum(O * dO) for ra_attn_fwd.
 *   Source: Ra-Family page, section 3, item ra_softmax (closed-form derivative
 *   d(phi)/du = -16 phi / (1 - u^2) for u < 1, recomputed from the saved row statistics
 *   rather than stored powers) and item ra_attention ("closed-form backward recomputation",
 *   saved state O(B*H*Nq*D)).  With dP = dO V^T and c_i = dO_i . O_i:
 *     G_ij = p_ij (dP_ij - c_i) / (1 - u_ij^2) on the support, 0 elsewhere;
 *     the row max also depends on the scores, which adds R_i = -sum_j G_ij at the lowest
 *     key index attaining the max: dS = G + R e_{argmax};
 *     dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO,
 *   with dK and dV summed over the Hq/Hkv query heads sharing a K/V head (RepeatKVHeads).
 *   o and stats must come from ra_attn_fwd with the same inputs; stats == NULL makes the
 *   call recompute them first.  dq, dk, dv are overwritten (no accumulation).
 *   workspace: at least ra_attn_bwd_workspace_bytes(...) bytes of device memory.
 *   The result is deterministic (no floating-point atomics).
 *   Sizes and limits as ra_attn_fwd; Nk == 0 -> dq = 0; B*Hkv*Nk > 0 with B*Hq*Nq == 0 ->
 *   dk = dv = 0.
 */
int ra_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                const float* stats, void* dq, void* dk, void* dv, void* workspace,
                size_t workspace_bytes, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                int64_t Nk, int64_t D, int causal, float scale, int dtype, void* stream);

/*
 * ra_attn_bwd_masked -- ra_attn_bwd for ra_attn_fwd_masked: the same mask (and causal mode)
 *   must be passed as to the forward that produced o and stats.  Masked entries get P = 0 and
 *   dS = 0; the mask receives no gradient.  Checks as ra_attn_bwd plus the ra_mask checks.
 */
int ra_attn_bwd_masked(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                       const float* stats, void* dq, void* dk, void* dv, void* workspace,
                       size_t workspace_bytes, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                       int64_t Nk, int64_t D, int causal, float scale, int dtype,
                       const ra_mask* mask, void* stream);

/*
 * ra_attn_bwd_dq, ra_attn_bwd_dkdv -- the two phases of ra_attn_bwd, callable on their own
 * (same sources and formulas).  ra_attn_bwd is exactly ra_attn_bwd_dq followed by
 * ra_attn_bwd_dkdv on the same stream, with the same arguments and workspace.
 *   ra_attn_bwd_dq: query-parallel.  Writes dq and, into workspace, the per-row terms the
 *     second phase needs: c_i = dO_i . O_i, the row-max gradient R_i and the lowest key index
 *     of the row max.  With stats == NULL it first recomputes (m, l) into workspace.
 *   ra_attn_bwd_dkdv: key-parallel.  Writes dk and dv from those per-row terms, so the
 *     workspace must hold what ra_attn_bwd_dq wrote for the same inputs (stream order or an
 *     explicit synchronisation between the two calls); pass the same stats pointer (NULL
 *     reads the copy the first phase recomputed).  The workspace is only read.
 *   Pointers a phase does not use (dk, dv for the first; o, dq for the second) may be NULL.
 *   Checks, sizes, limits and determinism as ra_attn_bwd.
 */
int ra_attn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                   const float* stats, void* dq, void* workspace, size_t workspace_bytes,
                   int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                   int causal, float scale, int dtype, void* stream);
int ra_attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* d_o,
                     const float* stats, void* dk, void* dv, const void* workspace,
                     size_t workspace_bytes, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq,
                     int64_t Nk, int64_t D, int causal, float scale, int dtype, void* stream);

/*
 * ra_attn_bwd_noalloc -- ra_attn_bwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight training loops, harnesses that
 * forbid hipMalloc.  The call allocates nothing; the per-row terms ra_attn_bwd keeps in its
 * workspace go to a fixed 64 MiB array inside the library instead, one copy per device, held from
 * the library's first use on that device until the process ends.
 *   Limit: ra_attn_bwd_workspace_bytes(...) <= 64 MiB, i.e. B * Hq * Nq <= 1,864,128 query rows
 *   (36 bytes each plus 256) -> else RA_ERR_TOO_LARGE, nothing launched.
 *   Every call on one device shares that device's array, which keeps the last call's contents:
 *   calls that overlap on one device (on other streams or from other threads) race, and the caller
 *   must order them (calls on one stream are ordered by the stream).
 *   Arguments, checks, sizes and results as ra_attn_bwd (the same kernels: the outputs equal
 *   ra_attn_bwd's bit for bit).  A failure to resolve the array's device address returns
 *   RA_ERR_HIP.
 */
int ra_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                        const void* d_o, const float* stats, void* dq, void* dk, void* dv,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D,
                        int causal, float scale, int dtype, void* stream);

/*
 * ra_attn_decode_workspace_bytes -- scratch size ra_attn_decode needs for these sizes (0 when the
 * sizes are invalid for it or there is nothing to compute).  Caller-allocated, 256-byte aligned,
 * contents need not be initialised.
 */
size_t ra_attn_decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                                      int64_t D, int dtype);

/*
 * ra_attn_decode -- attention of a few query rows per head against a key/value cache, split over
 * the keys (decode and short-prefix steps).
 *   Source: Ra-Family page, section 3, items ra_softmax and ra_attention.  phi has no online
 *   rescaling, so partial results over key ranges cannot be merged as exp-softmax partials are:
 *   the call makes three passes on the stream -- (1) scores and per-range row maxima, (2) with the
 *   row max over all ranges, phi, its partial sums and partial P.V per range, (3) the sums over
 *   ranges in a fixed order and the division.  K and V are each read once.
 *   q, o: [B, Hq, Nq, D]; k, v: [B, Hkv, Nk, D], the caches, of which sample b uses its first
 *   seqlens[b] keys (seqlens: device int32 [B], or NULL for all Nk; values are clamped to
 *   [0, Nk]).  causal: RA_CAUSAL_NONE; RA_CAUSAL_TOP_LEFT (query i takes keys j <= i);
 *   RA_CAUSAL_BOTTOM_RIGHT (query i is position seqlens[b] - Nq + i of its sequence and takes
 *   keys j <= seqlens[b] - Nq + i).  stats (optional) as ra_attn_fwd.  Equivalent to
 *   ra_attn_fwd on each sample's cache prefix; a sample with seqlens[b] = 0 (or a row with no
 *   allowed key) gives o = 0.
 *   dtype RA_BF16 (bf16 products) or RA_F32 (fp32 products), as ra_attn_fwd; fp32 sums either way.
 *   Restrictions: (Hq / Hkv) * Nq <= 32, the query rows of one K/V head (RA_ERR_SHAPE otherwise;
 *   use ra_attn_fwd for longer query blocks).
 *   Forward only.  Deterministic.  Other checks, sizes and limits as ra_attn_fwd; workspace at
 *   least ra_attn_decode_workspace_bytes(...) bytes, 256-byte aligned (RA_ERR_WORKSPACE,
 *   RA_ERR_ALIGN).
 */
int ra_attn_decode(const void* q, const void* k, const void* v, void* o, float* stats,
                   const int32_t* seqlens, void* workspace, size_t workspace_bytes, int64_t B,
                   int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t D, int causal,
                   float scale, int dtype, void* stream);

/*
 * ra_softmax_rows -- ra_softmax along the last axis of a [rows, cols] matrix.
 *   Source: Ra-Family page, section 3, item ra_softmax (ra_softmax(logits, dim=-1)).
 *   Entries equal to -inf are masked: p = 0 there, and they take no part in the max or the
 *   sum.  A row whose entries are all -inf gives p = 0.  x and p may alias (in-place).
 *   Limits: rows < 2^31, cols < 2^31.  rows == 0 or cols == 0 -> RA_OK, nothing launched.
 */
int ra_softmax_rows(const void* x, void* p, int64_t rows, int64_t cols, int dtype,
                    void* stream);

/*
 * ra_softmax_rows_bwd -- gradient of ra_softmax_rows: dx = dL/dx given dp = dL/dp.
 *   Source: Ra-Family page, section 3, item ra_softmax (closed-form derivative
 *   d(phi)/du = -16 phi / (1 - u^2) for u < 1).  Per row, with p = ra_softmax(x),
 *   c = sum_j p_j dp_j and u_j = (max - x_j) / 16:
 *     G_j = p_j (dp_j - c) / (1 - u_j^2) on the support (u_j < 1), 0 elsewhere;
 *   the row max depends on x as well, which adds R = -sum_j G_j at the lowest index attaining
 *   the max: dx = G + R e_argmax.  p is recomputed from x (it is not an argument).
 *   x, dp, dx: [rows, cols] of dtype.  Masked (-inf) entries of x get dx = 0; a row whose entries
 *   are all -inf gives dx = 0.  dx may be the same buffer as x or as dp (each element of dx is
 *   written after its own x and dp are read); other overlaps are not allowed.
 *   Limits, sizes and errors as ra_softmax_rows.
 */
int ra_softmax_rows_bwd(const void* x, const void* dp, void* dx, int64_t rows, int64_t cols,
                        int dtype, void* stream);

/*
 * ra_rope_neox -- split-halves (NEOX) rotary position embedding, for the queries and keys of
 * ra_attn_fwd (the step before the attention call).
 *   Source: "Primitives" page, section "Attention and transformers" (RoPE: channel j of a head
 *   is paired with channel j + D/2, not j + 1) and the nurl page, section "Layers" (nn_rope).
 *   For each of the `mats` contiguous [N, D] matrices of x (e.g. mats = B * H for [B, H, N, D]),
 *   position p_n of row n and pair j < D/2, with angle = p_n * theta^(-2j/D):
 *     y[n, j] = x[n, j] cos - x[n, j + D/2] sin,  y[n, j + D/2] = x[n, j + D/2] cos + x[n, j] sin.
 *   inverse != 0 rotates by -angle: the transpose, which maps dL/dy to dL/dx.
 *   positions: device int32 [N], or NULL for 0..N-1.  The angle is formed and reduced to
 *   [-pi, pi] in fp64; its cosine and sine, and the products, run in fp32, and the result rounds
 *   once to dtype.  y may be x (in place); other overlaps are not allowed.
 *   Errors: D odd -> RA_ERR_HEADDIM; theta not finite or <= 0 -> RA_ERR_SCALE; N * D >= 2^31
 *   -> RA_ERR_TOO_LARGE; mats, N or D == 0 -> RA_OK, nothing launched.
 */
int ra_rope_neox(const void* x, void* y, const int32_t* positions, int64_t mats, int64_t N,
                 int64_t D, double theta, int inverse, int dtype, void* stream);

/*
 * ra_attn_fwd_rope -- ra_attn_fwd on queries and keys rotated by the NEOX rotary embedding,
 * with the query rotation done inside the attention kernel as its rows are loaded.
 *   Source: nurl page, section "Layers" (nn_rope applied to the queries and keys ahead of the
 *   attention core), "Primitives" page, section "Attention and transformers" (split-halves
 *   pairing), Ra-Family page, section 3, item ra_attention.
 *   Result: bit-identical to ra_rope_neox(q -> q_rot), ra_rope_neox(k -> k_rot), then
 *   ra_attn_fwd(q_rot, k_rot, v): the query rows the kernel multiplies are the bf16 rows
 *   ra_rope_neox would produce.
 *   q: [B, Hq, Nq, D] and k: [B, Hkv, Nk, D], unrotated.  k_rot: caller's [B, Hkv, Nk, D] buffer
 *   that receives the rotated keys (one rotation pass over K before the attention kernel); it
 *   may be k itself (k is then overwritten).  q_rot: optional [B, Hq, Nq, D] (NULL to skip)
 *   that receives the rotated queries, for ra_attn_bwd_rope.  q_rot and k_rot must not
 *   overlap q, v, o or stats (k_rot may be k, see above).
 *   q_positions: device int32 [Nq], k_positions: int32 [Nk], or NULL for 0..N-1, shared by
 *   every batch and head; they set the rotation only (the causal mode still compares row and
 *   key indices).  theta: the base of the frequency schedule theta^(-2j/D).
 *   o, stats, causal, scale: as ra_attn_fwd, on the rotated rows.  mask: an explicit mask as
 *   in ra_attn_fwd_masked (NULL = none), with its checks.
 *   dtype: RA_BF16 or RA_F32 (for fp32 the rotated rows are the fp32 rows ra_rope_neox gives).
 *   theta not finite or <= 0 ->
 *   RA_ERR_SCALE.  Sizes, limits and the other errors as ra_attn_fwd; k_rot NULL with Nk > 0
 *   -> RA_ERR_NULLPTR.  Nk == 0: o = 0, stats (-inf, 0), and q_rot is still written.
 */
int ra_attn_fwd_rope(const void* q, const void* k, const void* v, void* o, float* stats,
                     void* q_rot, void* k_rot, const int32_t* q_positions,
                     const int32_t* k_positions, double theta, int64_t B, int64_t Hq, int64_t Hkv,
                     int64_t Nq, int64_t Nk, int64_t D, int causal, float scale, int dtype,
                     const ra_mask* mask, void* stream);

/*
 * ra_attn_bwd_rope -- the backward of ra_attn_fwd_rope: the gradients with respect to the
 * UNROTATED q and k, and v.
 *   Source: as ra_attn_fwd_rope; the rotation is orthogonal, so the gradient of a rotated row
 *   maps back by the rotation with the negative angle.
 *   q_rot, k_rot: the rotated rows ra_attn_fwd_rope wrote (q_rot requested there).  v, o, d_o,
 *   stats (nullable: recomputed), workspace, workspace_bytes (ra_attn_bwd_workspace_bytes),
 *   causal, scale: as ra_attn_bwd; mask as ra_attn_bwd_masked (NULL = none).  q_positions,
 *   k_positions, theta: those of the forward.
 *   dq [B, Hq, Nq, D], dk [B, Hkv, Nk, D]: rotated back inside the kernels' epilogues (each
 *   element is the fp32 accumulator rotated by the negative angle, rounded once to the dtype);
 *   dv as ra_attn_bwd.
 *   dtype: RA_BF16 or RA_F32.  Errors as ra_attn_bwd, plus RA_ERR_SCALE as ra_attn_fwd_rope.
 */
int ra_attn_bwd_rope(const void* q_rot, const void* k_rot, const void* v, const void* o,
                     const void* d_o, const float* stats, void* dq, void* dk, void* dv,
                     void* workspace, size_t workspace_bytes, const int32_t* q_positions,
                     const int32_t* k_positions, double theta, int64_t B, int64_t Hq, int64_t Hkv,
                     int64_t Nq, int64_t Nk, int64_t D, int causal, float scale, int dtype,
                     const ra_mask* mask, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RA_ATTN_H */
