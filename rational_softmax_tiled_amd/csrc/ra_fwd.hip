// ra_fwd.hip -- forward rational-softmax attention for gfx950.
//
// "Ra-Family: Rational Neural Architecture", section 3 "Rational Attention & Softmax":
// O = ra_softmax(scale * Q K^T) V computed tile by tile; the [B, H, Nq, Nk] scores never
// reach memory.  phi has no online rescaling (phi(D + d) is not a multiple of phi(D)), so the
// row max must be final before any phi is summed: pass 1 finds it, pass 2 evaluates phi,
// sum(phi) and P.V.  Tiles whose entries all fall outside the compact support are skipped.
//
// Work decomposition
//   * One wave owns 32 query rows of one head; a workgroup is 4 waves that share one K/V head
//     (grouped-query: the REP query heads of a K/V head are packed into the same workgroup, so
//     each K/V tile staged in LDS serves all of them).  Tasks (head-in-group, 32-row block)
//     are enumerated head-fastest and dealt four per workgroup.
//   * Scores are computed transposed, S^T = K Q^T (keys on the accumulator rows, queries on
//     the lanes), so every lane owns one query row: its running max, phi sum and the
//     P^T operand of O^T = V^T P^T stay in that lane, with no register shuffle.  K and V are
//     staged as XOR-swizzled row tiles; the V^T operand is read with the LDS transposing load
//     in the slot order that matches the accumulator layout (fp32: V staged transposed).
//   * Pass 1 keeps, per wave and key tile, the max score of the tile; after pass 1 a tile is
//     skipped for a wave when 1 + u >= 2 already at the tile max against the smallest row max
//     of the wave, evaluated with the same monotone floating-point steps as phi itself, so
//     skipping never changes a result bit.  A tile
//     skipped by all four waves is not even loaded.  Causal tiles beyond a wave's diagonal are
//     recorded as -inf and skipped the same way.
#include <type_traits>

#include "ra_device.h"
#include "ra_internal.h"

namespace ra {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* stats;
  unsigned long long* counters;
  int Hq, Hkv, Nq, Nk, rep;
  int tasks_per_group;   // rep * ceil(Nq / 32)
  int wg_per_group;      // ceil(tasks_per_group / 4)
  int total_wg;
  float c;               // scale / 16
  int coff;              // causal diagonal: key j allowed for query row i iff j <= i + coff
  MaskArgs mask;         // explicit mask (MASKED kernels)
  // ROPE kernels: Q is rotated (NEOX) as its fragments are loaded; row i sits at position
  // q_pos[i] (nullable: i); the rotated rows go to q_rot when it is non-null
  const int* q_pos;
  double log2_theta;
  void* q_rot;
};

constexpr int kMaxTiles = 512;   // key tiles with a recorded maximum (skip test); beyond: no skip

template <typename T>
__device__ __forceinline__ void store_quad(T* dst, f32x16 acc, int base, float s);

template <>
__device__ __forceinline__ void store_quad<bf16>(bf16* dst, f32x16 acc, int base, float s) {
  bf16x4 v = {(bf16)(acc[base] * s), (bf16)(acc[base + 1] * s), (bf16)(acc[base + 2] * s),
              (bf16)(acc[base + 3] * s)};
  *reinterpret_cast<bf16x4*>(dst) = v;
}
template <>
__device__ __forceinline__ void store_quad<float>(float* dst, f32x16 acc, int base, float s) {
  f32x4 v = {acc[base] * s, acc[base + 1] * s, acc[base + 2] * s, acc[base + 3] * s};
  *reinterpret_cast<f32x4*>(dst) = v;
}

// Does a raw explicit-mask value leave its score as it is (boolean: kept; additive: a zero bias)?
__device__ __forceinline__ bool mask_identity(int kind, unsigned v) {
  return kind == kMaskBool ? v != 0u : (v << 1) == 0u;
}

// The explicit-mask values of a 32x32 S^T block (keys on the accumulator rows, query row qrow on
// the lane), one per entry of the lane.
template <bool RUNS, typename T>
__device__ __forceinline__ void load_mask_block(const MaskSlice<T>& ms, unsigned (&mv)[16], int key0, int qrow,
                                                int lane) {
  ms.template load_keys<RUNS>(mv, qrow * ms.sq + (key0 + 4 * (lane >> 5)) * ms.sk);
}

// Mask entries of a 32x32 S^T block: the explicit mask values mv first (MASKED), then key >= Nk or
// key > qrow + coff (coff = Nk: no causal limit).  With `ident`, also reports (the same in every
// lane) whether the explicit mask left every entry of the block as it was.
template <bool MASKED, typename T>
__device__ __forceinline__ void apply_mask_block(f32x16& s, const unsigned (&mv)[16], int key0, int qrow, int lane,
                                                 int Nk, int coff, const MaskSlice<T>& ms, bool* ident = nullptr) {
  if constexpr (MASKED) {
    bool all = true;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      all = all && mask_identity(ms.kind, mv[i]);
      s[i] = ms.apply(s[i], mv[i]);
    }
    if (ident != nullptr) *ident = !__any(!all);
  }
  // key = key0 + 4 (lane >> 5) + r is kept iff key < Nk and key <= qrow + coff
  const int lb = key0 + 4 * (lane >> 5);
  keep_rows(s, -kNoBound, min(Nk - lb, qrow + coff + 1 - lb));
}

// RUNS: an additive mask in the packed layout may come (see MaskSlice::load_keys)
template <bool MASKED, bool RUNS = false, typename T>
__device__ __forceinline__ void mask_block(f32x16& s, int key0, int qrow, int lane, int Nk, int coff,
                                           const MaskSlice<T>& ms, bool* ident = nullptr) {
  unsigned mv[16] = {};
  if constexpr (MASKED) load_mask_block<RUNS>(ms, mv, key0, qrow, lane);
  apply_mask_block<MASKED>(s, mv, key0, qrow, lane, Nk, coff, ms, ident);
}

// S^T block (32 keys x 32 query rows) of key sub-block sb of the staged (swizzled) K tile.
template <typename T, int D>
__device__ __forceinline__ f32x16 score_block(const T* k_tile, const typename Ty<T>::frag* qf, int sb,
                                              int frow, int fcol) {
  f32x16 s = {};
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) mma(s, swz_frag<T, D>(k_tile, sb * 32 + frow, 16 * kc + fcol), qf[kc]);
  return s;
}

// Both 32-key blocks of a 64-key bf16 tile.  All K fragments of block 0 are read before its
// products start and block 1's are read under them, so no product waits on a read issued just
// before it (LDS latency is several product times).
template <int D>
__device__ __forceinline__ void score_pair(const bf16* k_tile, const bf16x8* qf, int frow, int fcol,
                                           f32x16& s0, f32x16& s1) {
  constexpr int KC = D / 16;
  bf16x8 kf0[KC], kf1[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) kf0[kc] = swz_frag<bf16, D>(k_tile, frow, 16 * kc + fcol);
  __builtin_amdgcn_sched_barrier(0);
  s0 = f32x16{};
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    mma(s0, kf0[kc], qf[kc]);
    kf1[kc] = swz_frag<bf16, D>(k_tile, 32 + frow, 16 * kc + fcol);
  }
  // issue order: product, read, product, read, ...
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  s1 = f32x16{};
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) mma(s1, kf1[kc], qf[kc]);
  __builtin_amdgcn_sched_barrier(0);
}

// Every launch takes the causal form: key j is allowed for query row i iff j <= i + coff, with
// coff = 0 (top-left), Nk - Nq (bottom-right) or Nk (not causal: every key allowed).
// KEYPAD: a boolean mask that depends on the key only (the same for every query row and head:
// key padding).  Its bytes reach LDS with each pass-1 K tile, so the kernel keeps the four-stage
// K ring and the interleaved pass-2 path of the unmasked kernel (MASKED is false): pass 1 turns a
// tile's 64 mask bytes into 64 keep bits, drops a tile with none (its maximum stays -inf, so
// pass 2 skips it too) and masks a partial one; pass 2 masks the partial tiles again from the
// recorded bits and runs full tiles on the interleaved path.
// ROPE: q holds the rows before the rotary embedding; each wave rotates its Q fragments once, on
// load (the pair of channel j, j + D/2 lies in fragments kc, kc + KC/2 of the same lane), and may
// store them (q_rot) for a backward pass.
// MADD (with MASKED, bf16): the mask is additive in the packed layout (see MaskSlice), read ahead
// the way a boolean one is; a variant of its own, so the boolean kernels keep their registers.
template <typename T, int D, int BN, bool COUNT, bool WRITE_O, bool MASKED, bool KEYPAD = false,
          bool ROPE = false, bool MADD = false>
// bf16: two waves per SIMD (at most 256 VGPRs), the second wave fills the first one's waits.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : 1))) void attn_fwd_kernel(FwdArgs a) {
  using frag_t = typename Ty<T>::frag;
  // bf16: V stays a swizzled row tile and the P.V operand is read transposed (ds_read_b64_tr_b16);
  // fp32 has no transposed read: V is staged transposed, [d][key slot], row pitch PV.
  constexpr bool VTR = sizeof(T) == 2;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int PV = BN + PAD;
  constexpr int V_ELEMS = VTR ? BN * D : D * PV;
  constexpr int KC = D / 16;     // 16-wide K chunks of the QK^T contraction
  constexpr int SB = BN / 32;    // 32-key blocks per tile
  constexpr int DB = D / 32;     // 32-row blocks of O^T

  __shared__ __attribute__((aligned(16))) T k_lds[2][BN * D];
  __shared__ __attribute__((aligned(16))) T v_lds[WRITE_O ? 2 : 1][WRITE_O ? V_ELEMS : 8];
  __shared__ float tmax_lds[kWaves][kMaxTiles];
  __shared__ float kmin_lds[kWaves];
  static_assert(!KEYPAD || (sizeof(T) == 2 && WRITE_O && !MASKED && BN == kWave), "key padding path");
  static_assert(!MADD || (sizeof(T) == 2 && MASKED), "packed additive masks: bf16 masked kernels");
  static_assert(!ROPE || (WRITE_O && !COUNT), "rotary path");
  __shared__ __attribute__((aligned(16))) unsigned mstage_lds[KEYPAD ? 4 : 1][KEYPAD ? kWave : 1];
  __shared__ unsigned long long keep_lds[KEYPAD ? kMaxTiles : 1];
  // MASKED: per wave and key tile, 1 when the explicit mask keeps every entry of the wave's block
  // as it is (recorded in pass 1); pass 2 then treats the tile as unmasked
  __shared__ unsigned char mfree_lds[MASKED ? kWaves : 1][MASKED ? kMaxTiles : 1];
  __shared__ double rate_lds[ROPE ? D / 2 : 1];   // ROPE: theta^(-2j/D) per pair j

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // ---- work assignment
  const int logical = xcd_remap(blockIdx.x, a.total_wg);
  const int bg = logical / a.wg_per_group;
  int wig = logical % a.wg_per_group;
  wig = a.wg_per_group - 1 - wig;   // long (late) query blocks first
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int task = wig * kWaves + wave;
  const bool active = task < a.tasks_per_group;
  const int h = g * a.rep + (active ? task % a.rep : 0);
  const int q0 = (active ? task / a.rep : 0) * kRowsPerWave;
  const int last_task = min(wig * kWaves + kWaves - 1, a.tasks_per_group - 1);
  const int wg_qmax = min((last_task / a.rep) * kRowsPerWave + kRowsPerWave - 1, a.Nq - 1);
  const int key_end = max(0, min(a.Nk, wg_qmax + a.coff + 1));
  // tile counts of the workgroup and of the wave: the same in every lane of a wave, read from the
  // first lane so that the tile loops and skip tests branch on scalar registers
  const int nt = uniform((key_end + BN - 1) / BN);
  const int wave_qmax = min(q0 + kRowsPerWave - 1, a.Nq - 1);
  const int key_end_w = !active ? 0 : max(0, min(a.Nk, wave_qmax + a.coff + 1));
  const int nt_w = uniform((key_end_w + BN - 1) / BN);

  const T* qh = static_cast<const T*>(a.q) + (size_t)(b * a.Hq + h) * a.Nq * D;
  const T* kg = static_cast<const T*>(a.k) + (size_t)(b * a.Hkv + g) * a.Nk * D;
  const T* vg = static_cast<const T*>(a.v) + (size_t)(b * a.Hkv + g) * a.Nk * D;

  // ---- Q fragments stay in registers for both passes (B operand of S^T = K Q^T)
  const int qi = q0 + (lane & 31);
  const int qrow = min(qi, a.Nq - 1);   // tail rows duplicate the last real row
  frag_t qf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) qf[kc] = load_frag(qh + (size_t)qrow * D + 16 * kc + 8 * (lane >> 5));
  // ROPE: the row's position and, in wave 0, the table of rates theta^(-2j/D)
  int rope_pos = 0;
  if constexpr (ROPE) {
    rope_pos = a.q_pos != nullptr ? a.q_pos[qrow] : qrow;
    if (tid < D / 2) rate_lds[tid] = rope_rate(tid, D, a.log2_theta);
  }
  // settle these loads here: otherwise the compiler waits for them (vmcnt) inside the tile loops,
  // where the count would also cover the tile prefetch in flight
  wait_vmem();
  if constexpr (ROPE) {
    asm volatile("" : "+v"(rope_pos));   // landed: no wait after the copies below
    __syncthreads();                     // the rate table is written
  }

  // ROPE: turn the Q fragments by the NEOX rotary embedding.  Channel j < D/2 and its partner
  // j + D/2 sit in fragments kc and kc + KC/2 of the same lane (element j % 8), so the rotation is
  // lane-local.  The (cos, sin) pairs go through LDS, the second V buffer (stage 3 of the bf16
  // K ring, free until pass 1's first step; for fp32 idle until pass 2), so that the angle loops
  // stay rolled while the fragments are indexed statically.  When
  // the four waves hold the same query rows (rep a multiple of four) they split one table;
  // otherwise each wave fills its own, one fragment pair at a time.  For bf16 it runs while pass
  // 1's first tiles are in flight; q_rot, when given, receives the rotated rows.
  auto rope_rotate = [&]() {
    if constexpr (ROPE) {
      constexpr int NP = D / 4;   // pairs per lane
      constexpr int STAGE = (int)sizeof(v_lds[0]);
      // pairs per chunk of the per-wave tables: the four tables share stage 3
      constexpr int CH = STAGE / (kWaves * kWave * (int)sizeof(f32x2)) < 8
                             ? STAGE / (kWaves * kWave * (int)sizeof(f32x2)) : 8;
      static_assert(NP * kWave * (int)sizeof(f32x2) <= STAGE && CH >= 1 && 8 % CH == 0,
                    "cos/sin tables fit stage 3");
      f32x2* tab = reinterpret_cast<f32x2*>(v_lds[1]);
      const double pos = (double)rope_pos;
      auto angle = [&](int pr) {   // pair pr of the lane: channel 16 (pr / 8) + 8 (lane / 32) + pr % 8
        float c, sn;
        rope_cs(pos, rate_lds[16 * (pr >> 3) + 8 * (lane >> 5) + (pr & 7)], false, c, sn);
        return f32x2{c, sn};
      };
      // pairs p0 .. p0 + n - 1 (within one fragment pair) from t: [pair - p0][lane]
      auto turn = [&](auto p0_c, auto n_c, const f32x2* t) {
        constexpr int p0 = decltype(p0_c)::value, n = decltype(n_c)::value, kc = p0 / 8;
#pragma unroll
        for (int e = 0; e < n; ++e) {
          const f32x2 v = t[e * kWave + lane];
          float y1, y2;
          rope_pair((float)qf[kc][p0 % 8 + e], (float)qf[kc + KC / 2][p0 % 8 + e], v[0], v[1], y1, y2);
          qf[kc][p0 % 8 + e] = (T)y1;
          qf[kc + KC / 2][p0 % 8 + e] = (T)y2;
        }
      };
      if (a.rep % kWaves == 0) {
        constexpr int PW = NP / kWaves;
#pragma unroll 2
        for (int i = 0; i < PW; ++i) tab[(wave * PW + i) * kWave + lane] = angle(wave * PW + i);
        __syncthreads();
        static_for<NP / 8>([&](auto kc) {
          constexpr int p0 = decltype(kc)::value * 8;
          turn(std::integral_constant<int, p0>{}, std::integral_constant<int, 8>{}, tab + p0 * kWave);
        });
      } else {
        f32x2* own = tab + wave * CH * kWave;
        static_for<NP / CH>([&](auto c) {
          constexpr int p0 = decltype(c)::value * CH;
#pragma unroll 2
          for (int e = 0; e < CH; ++e) own[e * kWave + lane] = angle(p0 + e);
          turn(std::integral_constant<int, p0>{}, std::integral_constant<int, CH>{}, own);
        });
      }
      if (a.q_rot != nullptr && active && qi < a.Nq) {
        T* qr = static_cast<T*>(a.q_rot) + ((size_t)(b * a.Hq + h) * a.Nq + qi) * D + 8 * (lane >> 5);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) *reinterpret_cast<frag_t*>(qr + 16 * kc) = qf[kc];
      }
    }
  };

  const int frow = lane & 31;           // A-fragment row inside a 32-row block
  const int fcol = 8 * (lane >> 5);     // A-fragment column offset

  auto needs_mask = [&](int key0) { return MASKED || key0 + 31 > q0 + a.coff || key0 + 32 > a.Nk; };
  auto at_edge = [&](int key0) { return key0 + 31 > q0 + a.coff || key0 + 32 > a.Nk; };
  const MaskSlice<T> ms(a.mask, b, h);

  // ---- pass 1: row max of the raw dot products (K tiles double-buffered through LDS)
  // Tiles reach LDS by DMA (bf16) or through registers (fp32), one tile ahead of the math.
  SwzTile<T, D, (sizeof(T) == 2 ? 0 : BN)> kreg;
  // bf16: one resource per matrix (K, V of the head), the tile picked by a scalar offset
  const u32x4 k_rsrc = dma_rsrc(kg, a.Nk * D * (int)sizeof(T));
  const u32x4 v_rsrc = dma_rsrc(vg, a.Nk * D * (int)sizeof(T));
  const int lane_off = sizeof(T) == 2 ? dma_lane_offset<D, kWaves>(wave, lane) : 0;
  auto k_issue = [&](int kt, T* dst) {
    if constexpr (sizeof(T) == 2) dma_tile_at<D, BN>(k_rsrc, kt * BN * D * 2, lds_addr(dst), lane_off, wave);
    else kreg.load(kg + (size_t)kt * BN * D, a.Nk - kt * BN, tid);
  };
  auto k_land = [&](T* dst) {
    if constexpr (sizeof(T) == 2) wait_vmem();
    else kreg.store(dst, tid);
  };
  // KEYPAD: wave 0 copies tile kt's 64 mask bytes (lanes 0-15; the other lanes' dwords are not
  // read) into the stage of its K tile
  u32x4 m_rsrc = {};
  if constexpr (KEYPAD) m_rsrc = dma_rsrc(static_cast<const char*>(a.mask.ptr) + (size_t)b * a.mask.sb, a.Nk);
  auto m_issue = [&](int kt, int stage) {
    if constexpr (KEYPAD)
      if (wave == 0) lds_dma_at<4>(m_rsrc, lds_addr(mstage_lds[stage]), lane * 4, kt * BN);
  };
  float mx = -INFINITY;
  // MASKED with a boolean mask in the packed layout: pass 1 reads each tile's mask words one step
  // ahead (they land with the step's copies, so deciding on them waits for nothing), drops a tile
  // the mask empties for every row of the wave before its products, and applies the words to the
  // tiles it computes.  (A wait for words loaded in the same step would also wait for the step's
  // K copy, issued before them, which counts in the same in-order counter.)  A bf16 additive mask
  // in that layout takes the same path: its elements, read one step ahead, become boolean words
  // (-inf drops the key, anything else keeps it), and a block holding a bias other than 0 or -inf
  // reads its values again where they are applied.
  const bool mpack = MASKED && ms.packed && (MADD || ms.kind == kMaskBool);
  // the slice the words are applied as: boolean (an additive mask's words stand for 0 / -inf)
  MaskSlice<T> mword = ms;
  if constexpr (MADD) mword.kind = kMaskBool;
  u32x4 mw_next[SB];    // the words in pairs as loaded (additive: keys +0 to +7 of the half),
  u32x4 mw_next2[SB];   // traded when the tile's step starts (additive: keys +8 to +15)
  auto load_tile_words = [&](int kt, u32x4 (&w)[SB]) {
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      if constexpr (MADD) ms.load_run_pairs(qrow * ms.sq + (kt * BN + sb * 32 + 4 * (lane >> 5)) * ms.sk, w[sb], mw_next2[sb]);
      else w[sb] = ms.load_word_pairs(qrow * ms.sq + (kt * BN + sb * 32 + 4 * (lane >> 5)) * ms.sk);
    }
  };
  // bf16 with V buffers: pass 1 streams K through four LDS stages (the V buffers are idle until
  // pass 2), three tiles ahead of the math.  Only without a mask: the mask loads are vector
  // loads too, and the counted waits below assume the copies are the only ones in flight.
  constexpr bool DEEP = sizeof(T) == 2 && WRITE_O && !MASKED;
  constexpr int kCopies = DEEP ? BN * D * 2 / 1024 / kWaves : 1;   // DMA loads per wave per tile
  // Stage s of the K ring sits at a fixed LDS address, so with the stage a compile-time constant
  // every fragment read is a loop-invariant lane address plus an immediate offset.
  constexpr int kStages = DEEP ? 4 : 2;
  // every copy of the n youngest tiles may still be in flight (wave 0 of KEYPAD copies one more
  // per tile)
  auto wait_younger = [&](auto n_c) {
    constexpr int n = decltype(n_c)::value;
    if (KEYPAD && wave == 0) wait_vmem_n<n * (kCopies + 1)>();
    else wait_vmem_n<n * kCopies>();
  };
  auto k_stage = [&](auto S) -> T* {
    constexpr int st = decltype(S)::value;
    if constexpr (st < 2) return k_lds[st];
    else return v_lds[st - 2];
  };
  if constexpr (DEEP) {
    k_issue(0, k_stage(std::integral_constant<int, 0>{}));
    m_issue(0, 0);
    if (nt > 1) {
      k_issue(1, k_stage(std::integral_constant<int, 1>{}));
      m_issue(1, 1);
    }
    if (nt > 2) {
      k_issue(2, k_stage(std::integral_constant<int, 2>{}));
      m_issue(2, 2);
    }
    if constexpr (ROPE) rope_rotate();
    // tile 0 landed; the copies of tiles 1 and 2 may stay in flight
    if (nt >= 3) wait_younger(std::integral_constant<int, 2>{});
    else if (nt == 2) wait_younger(std::integral_constant<int, 1>{});
    else wait_vmem();
  } else {
    if constexpr (ROPE) rope_rotate();
    if (nt > 0) {
      k_issue(0, k_lds[0]);
      if (mpack && nt_w > 0) load_tile_words(0, mw_next);
      k_land(k_lds[0]);
    }
  }
  __syncthreads();
  // one step of pass 1 on tile kt, held in stage S
  auto p1_step = [&](int kt, auto S) {
    constexpr int st = decltype(S)::value;
    // MASKED, packed: tile kt's words (read in the previous step) decide before anything is issued
    bool alive = true;
    unsigned mw[SB][4];
    unsigned mbias = 0;   // MADD: bit sb set when block sb holds a bias other than 0 or -inf (every lane)
    if constexpr (MASKED) {
      if (mpack && kt < nt_w) {
        unsigned any = 0;
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
          if constexpr (MADD) {
            // a block of only +-0 keeps everything, one of only -inf nothing: no trade for either
            unsigned nz, ni;
            MaskSlice<T>::run_flags(mw_next[sb], mw_next2[sb], nz, ni);
            const bool all_zero = !__any(nz != 0u), all_ninf = !__any(ni != 0u);
            if (all_zero || all_ninf) {
#pragma unroll
              for (int j = 0; j < 4; ++j) mw[sb][j] = all_zero ? 0x80808080u : 0u;
            } else {
              unsigned d[8], biased = 0;
              MaskSlice<T>::runs_of_pairs(mw_next[sb], mw_next2[sb], d);
              MaskSlice<T>::add_words_of_runs(d, mw[sb], biased);
              if (__any(biased != 0u)) mbias |= 1u << sb;
            }
          } else {
            MaskSlice<T>::words_of_pairs(mw_next[sb], mw[sb]);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) any |= mw[sb][j];
        }
        alive = __any(any != 0u);
      }
    }
    // the stage receiving tile kt + kStages - 1 was last read in step kt - 1, which every wave
    // has left (barrier at the end of each step)
    constexpr int st_in = (st + kStages - 1) % kStages;
    if (kt + kStages - 1 < nt) {
      k_issue(kt + kStages - 1, k_stage(std::integral_constant<int, st_in>{}));
      m_issue(kt + kStages - 1, st_in);
    }
    if (MASKED && mpack && kt + 1 < nt_w) load_tile_words(kt + 1, mw_next);
    const T* kt_lds = k_stage(S);
    float tl = -INFINITY;
    unsigned long long keep = ~0ull;   // KEYPAD: bit l set when key kt BN + l is kept
    if constexpr (KEYPAD) {
      keep = __ballot(reinterpret_cast<const unsigned char*>(mstage_lds[st])[lane] != 0);
      if (wave == 0 && lane == 0) keep_lds[kt] = keep;
    }
    bool mfree = true;   // MASKED: the mask leaves both blocks of the tile as they are
    // the block's mask, from the words read one step ahead or loaded now
    // A block whose words hold no zero byte in any lane keeps every entry: only the causal and
    // tail limits apply (at an edge), without the per-entry mask arithmetic.
    auto p1_mask = [&](f32x16& sc, int sb, int key0, bool& id) {
      if (MASKED && mpack && !(MADD && ((mbias >> sb) & 1u))) {
        unsigned zero = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) zero |= (mw[sb][j] - 0x01010101u) & ~mw[sb][j] & 0x80808080u;
        if (!__any(zero != 0u)) {
          id = true;
          if (at_edge(key0)) mask_block<false>(sc, key0, qrow, lane, a.Nk, a.coff, ms);
          return;
        }
        unsigned mv[16];
        MaskSlice<T>::expand_words(mw[sb], mv);
        apply_mask_block<MASKED>(sc, mv, key0, qrow, lane, a.Nk, a.coff, mword, &id);
      } else {
        mask_block<MASKED, MADD>(sc, key0, qrow, lane, a.Nk, a.coff, ms, &id);
      }
    };
    if (kt < nt_w && keep != 0 && alive) {
      if constexpr (sizeof(T) == 2 && SB == 2) {
        f32x16 sc[2];
        score_pair<D>(kt_lds, qf, frow, fcol, sc[0], sc[1]);
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const int key0 = kt * BN + sb * 32;
          bool id = true;
          if (needs_mask(key0)) p1_mask(sc[sb], sb, key0, id);
          mfree = mfree && id;
          if constexpr (KEYPAD)
            if (keep != ~0ull) keep_keys(sc[sb], keep, sb, lane);
#pragma unroll
          for (int i = 0; i < 16; ++i) tl = fmaxf(tl, sc[sb][i]);
        }
      } else {
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
          f32x16 sc = score_block<T, D>(kt_lds, qf, sb, frow, fcol);
          const int key0 = kt * BN + sb * 32;
          bool id = true;
          if (needs_mask(key0)) p1_mask(sc, sb, key0, id);
          mfree = mfree && id;
#pragma unroll
          for (int i = 0; i < 16; ++i) tl = fmaxf(tl, sc[i]);
        }
      }
    }
    mx = fmaxf(mx, tl);
    if (kt < kMaxTiles) {
      const float wm = wave_max_lane63(tl);
      if (lane == 63) tmax_lds[wave][kt] = wm;
      if (MASKED && lane == 0) mfree_lds[MASKED ? wave : 0][MASKED ? kt : 0] = mfree ? 1 : 0;
    }
    if constexpr (DEEP) {
      // tile kt + 1 landed; the copies issued after it (tiles kt + 2, kt + 3) may stay in flight
      if (kt + 3 < nt) wait_younger(std::integral_constant<int, 2>{});
      else if (kt + 2 < nt) wait_younger(std::integral_constant<int, 1>{});
      else if (kt + 1 < nt) wait_vmem();
    } else {
      if (kt + 1 < nt) k_land(k_stage(std::integral_constant<int, (st + 1) % kStages>{}));
    }
    __syncthreads();
  };
  for (int kt = 0; kt < nt;) {
    p1_step(kt, std::integral_constant<int, 0>{});
    if (++kt >= nt) break;
    p1_step(kt, std::integral_constant<int, 1>{});
    ++kt;
    if constexpr (kStages == 4) {
      if (kt >= nt) break;
      p1_step(kt, std::integral_constant<int, 2 % kStages>{});
      if (++kt >= nt) break;
      p1_step(kt, std::integral_constant<int, 3 % kStages>{});
      ++kt;
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32));   // lanes l and l+32 hold the same query row
  // 1 + u = fma(s, -c, kd) with kd = 1 + m c; the smallest kd of the wave bounds every row.  A
  // row with no allowed key (m = -inf) takes kd = +inf: every 1 + u is then +inf, phi = 0.
  const float kd = mx == -INFINITY ? INFINITY : fmaf(mx, a.c, 1.0f);
  {
    const float km = wave_min(kd);
    if (lane == 0) kmin_lds[wave] = km;
  }
  __syncthreads();

  // A tile is skipped for a wave when every entry has 1 + u >= fma(tile max, -c, min kd) >= 2
  // (phi = 0), and not even loaded when that holds for all four waves.  The tests are evaluated
  // for 64 tiles at once, one tile per lane, and kept as bits in scalar registers: evaluated per
  // tile they were chains of dependent LDS reads at the head of every step.
  float kmin_w[kWaves];
#pragma unroll
  for (int w = 0; w < kWaves; ++w) kmin_w[w] = kmin_lds[w];
  auto wave_skips = [&](int w, int kt) -> bool {
    const float tm = tmax_lds[w][kt];
    return (tm == -INFINITY) || (fmaf(tm, -a.c, kmin_w[w]) >= 2.0f);
  };
  unsigned long long wg_bits = 0, my_bits = 0;   // window win: skipped by all waves / this wave
  int win = -1;
  auto load_window = [&](int kt) {
    if ((kt >> 6) == win) return;
    win = kt >> 6;
    const int t = (kt & ~63) + lane;
    bool all = false, mine = t >= nt_w;
    if (t < kMaxTiles) {
      const bool s0 = wave_skips(0, t), s1 = wave_skips(1, t), s2 = wave_skips(2, t), s3 = wave_skips(3, t);
      all = s0 && s1 && s2 && s3;
      mine = wave == 0 ? s0 : wave == 1 ? s1 : wave == 2 ? s2 : s3;
    }
    wg_bits = __ballot(all);
    my_bits = __ballot(mine);
  };
  auto wg_skips = [&](int kt) -> bool {
    load_window(kt);
    return (wg_bits >> (kt & 63)) & 1ull;
  };

  // ---- pass 2: phi, sum(phi), O^T = V^T P^T
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float lsum = 0.0f;
  unsigned long long n_wave_tiles = 0, n_wave_skip = 0, n_wg_skip = 0;

  TransTile<T, D, (VTR ? 0 : BN)> vreg;   // fp32 only: V^T staged through registers
  auto v_issue = [&](int kt, T* dst) {
    if constexpr (VTR) dma_tile_at<D, BN>(v_rsrc, kt * BN * D * 2, lds_addr(dst), lane_off, wave);
    else vreg.load(vg + (size_t)kt * BN * D, a.Nk - kt * BN, tid);
  };
  auto v_land = [&](T* dst) {
    if constexpr (!VTR) vreg.template store<PV>(dst, tid);
  };
  // counting variant: a tile the whole workgroup drops is a skipped tile of every wave whose
  // causal range holds it
  auto count_dropped = [&](int lo, int hi) {
    if (COUNT) {
      n_wg_skip += hi - lo;
      const int in_range = max(0, min(hi, nt_w) - lo);
      n_wave_tiles += in_range;
      n_wave_skip += in_range;
    }
  };
  int cur = 0;
  while (cur < nt && wg_skips(cur)) ++cur;
  cur = uniform(cur);   // every lane computed the same index from the same LDS values
  count_dropped(0, cur);
  if (cur < nt) {
    k_issue(cur, k_lds[0]);
    if constexpr (WRITE_O) v_issue(cur, v_lds[0]);
    k_land(k_lds[0]);
    if constexpr (WRITE_O) v_land(v_lds[0]);
  }
  __syncthreads();
  // one step of pass 2 on tile cur, held in buffer BUF (a compile-time constant, so every LDS
  // read is a loop-invariant lane address plus an immediate offset)
  auto p2_step = [&](auto BUF) {
    constexpr int buf = decltype(BUF)::value;
    // KEYPAD: a tile with every key kept takes the interleaved path (a uniform flag, read first)
    bool keys_full = true;
    if constexpr (KEYPAD) keys_full = uniform(keep_lds[cur] == ~0ull ? 1 : 0) != 0;
    int nxt = cur + 1;
    while (nxt < nt && wg_skips(nxt)) ++nxt;
    nxt = uniform(nxt);
    count_dropped(cur + 1, nxt);
    load_window(cur);
    const bool my_skip = (my_bits >> (cur & 63)) & 1ull;
    if (COUNT && cur < nt_w) {
      n_wave_tiles += 1;
      n_wave_skip += my_skip ? 1 : 0;
    }
    bool done = my_skip;
    // MASKED: a tile whose explicit mask pass 1 found to keep every entry of the wave's blocks as
    // they are runs as an unmasked one (no mask reads; the interleaved path when away from edges)
    bool mfree = false;
    if constexpr (MASKED) mfree = cur < kMaxTiles && uniform((int)mfree_lds[wave][cur]) != 0;
    const bool fast = VTR && WRITE_O && SB == 2 && !done && !(MASKED && !mfree) && !at_edge(cur * BN + 32) &&
                      keys_full;
    if (nxt < nt) {
      k_issue(nxt, k_lds[buf ^ 1]);
      if constexpr (WRITE_O) v_issue(nxt, v_lds[buf ^ 1]);
    }
    if constexpr (VTR && WRITE_O && SB == 2) {
      // Unmasked tile: one straight-line block whose issue order is pinned so that the wave's
      // own VALU work overlaps its own MFMAs (issue is in order): S1 products run under the phi
      // math of block 0, the P.V products of block 0 under the phi math of block 1, and LDS
      // reads run ahead of the products that consume them.
      if (fast) {
        constexpr int NV = 2 * DB;            // P.V products (and V fragments) per 32-key block
        constexpr int EB = 16 / KC;           // phi elements per S1 product (stage B)
        constexpr int EC = 16 / NV;           // phi elements per P.V0 product (stage C)
        const bf16* kt_ = k_lds[buf];
        const bf16* vt_ = v_lds[buf];
        bf16x8 kf0[KC], kf1[KC], va[NV], vb[NV];
        f32x16 s0 = {}, s1 = {};
        // stage A: S0 = K0 Q^T, K1 fragments read behind it (all K0 reads issued first)
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) kf0[kc] = swz_frag<bf16, D>(kt_, frow, 16 * kc + fcol);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          mma(s0, kf0[kc], qf[kc]);
          kf1[kc] = swz_frag<bf16, D>(kt_, 32 + frow, 16 * kc + fcol);
        }
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // stage B: S1 products under phi(S0); V fragments of block 0 read
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          mma(s1, kf1[c], qf[c]);
#pragma unroll
          for (int e = 0; e < EB; ++e) s0[c * EB + e] = ra_phi(s0[c * EB + e], a.c, kd);
          if (c < NV) va[c] = tr_frag<D>(vt_, 16 * (c / DB), 32 * (c % DB), lane);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int c = KC; c < NV; ++c) va[c] = tr_frag<D>(vt_, 16 * (c / DB), 32 * (c % DB), lane);
        bf16x8 p0[2], p1[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          p0[ks] = pack_frag_bf16(s0, ks);
#pragma unroll
          for (int j = 0; j < 8; j += 2)
            lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p0[ks][j], p0[ks][j + 1]},
                                                   bf16x2{(bf16)1.0f, (bf16)1.0f}, lsum, false);
        }
        __builtin_amdgcn_sched_barrier(0);
        // stage C: P.V products of block 0 under phi(S1); V fragments of block 1 read
#pragma unroll
        for (int c = 0; c < NV; ++c) {
          mma(oacc[c % DB], va[c], p0[c / DB]);
#pragma unroll
          for (int e = 0; e < EC; ++e) s1[c * EC + e] = ra_phi(s1[c * EC + e], a.c, kd);
          vb[c] = tr_frag<D>(vt_, 32 + 16 * (c / DB), 32 * (c % DB), lane);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          p1[ks] = pack_frag_bf16(s1, ks);
#pragma unroll
          for (int j = 0; j < 8; j += 2)
            lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{p1[ks][j], p1[ks][j + 1]},
                                                   bf16x2{(bf16)1.0f, (bf16)1.0f}, lsum, false);
        }
        // stage D: P.V products of block 1
#pragma unroll
        for (int c = 0; c < NV; ++c) mma(oacc[c % DB], vb[c], p1[c / DB]);
        done = true;
      }
    }
    if (!done) {
      // both score blocks first, so the phi math of one overlaps the products of the other
      f32x16 s[SB];
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) s[sb] = score_block<T, D>(k_lds[buf], qf, sb, frow, fcol);
#pragma unroll
      for (int sb = 0; sb < SB; ++sb) {
        const int key0 = cur * BN + sb * 32;
        if (MASKED && !mfree) mask_block<MASKED, MADD>(s[sb], key0, qrow, lane, a.Nk, a.coff, ms);
        else if (at_edge(key0)) mask_block<false>(s[sb], key0, qrow, lane, a.Nk, a.coff, ms);
        if constexpr (KEYPAD) {
          const unsigned long long keep = keep_lds[cur];
          if (keep != ~0ull) keep_keys(s[sb], keep, sb, lane);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) s[sb][i] = ra_phi(s[sb][i], a.c, kd);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          frag_t pf;
          if constexpr (sizeof(T) == 2) {
            pf = pack_frag_bf16(s[sb], ks);
            // sum the rounded probabilities that enter the product, two per instruction
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
              bf16x2 pr = {pf[j], pf[j + 1]};
              lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, bf16x2{(bf16)1.0f, (bf16)1.0f}, lsum, false);
            }
          } else {
            pf = pack_frag_f32(s[sb], ks);
#pragma unroll
            for (int j = 0; j < 8; ++j) lsum += pf[j];
          }
          if constexpr (WRITE_O) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              if constexpr (VTR)
                mma(oacc[db], tr_frag<D>(v_lds[buf], sb * 32 + 16 * ks, db * 32, lane), pf);
              else
                mma(oacc[db], load_frag(v_lds[buf] + (db * 32 + frow) * PV + sb * 32 + 16 * ks + fcol), pf);
            }
          }
        }
      }
    }
    if (nxt < nt) {
      k_land(k_lds[buf ^ 1]);
      if constexpr (WRITE_O) v_land(v_lds[buf ^ 1]);
    }
    __syncthreads();
    cur = nxt;
  };
  while (cur < nt) {
    p2_step(std::integral_constant<int, 0>{});
    if (cur >= nt) break;
    p2_step(std::integral_constant<int, 1>{});
  }

  // ---- epilogue: O = acc / l
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  if (active && qi < a.Nq) {
    if constexpr (WRITE_O) {
      T* orow = static_cast<T*>(a.o) + ((size_t)(b * a.Hq + h) * a.Nq + qi) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          store_quad<T>(orow + db * 32 + 8 * r4 + 4 * (lane >> 5), oacc[db], 4 * r4, inv);
    }
    if (a.stats != nullptr && lane < 32) {
      float* st = a.stats + ((size_t)(b * a.Hq + h) * a.Nq + qi) * 2;
      st[0] = mx;
      st[1] = ltot;
    }
  }
  if (COUNT && lane == 0) {
    atomicAdd(a.counters + 0, n_wave_tiles);
    atomicAdd(a.counters + 1, n_wave_skip);
    if (wave == 0) {
      atomicAdd(a.counters + 2, (unsigned long long)nt);
      atomicAdd(a.counters + 3, n_wg_skip);
    }
  }
}


template <typename T, int D, int BN>
static hipError_t launch_typed(const AttnProblem& p, void* o, float* stats,
                               unsigned long long* counters, hipStream_t stream) {
  FwdArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.o = o;
  a.stats = stats;
  a.counters = counters;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.Nq = p.Nq;
  a.Nk = p.Nk;
  a.rep = p.Hq / p.Hkv;
  a.tasks_per_group = a.rep * ((p.Nq + kRowsPerWave - 1) / kRowsPerWave);
  a.wg_per_group = (a.tasks_per_group + kWaves - 1) / kWaves;
  a.total_wg = p.B * p.Hkv * a.wg_per_group;
  a.c = p.scale / 16.0f;
  a.coff = p.coff;
  a.mask = mask_args(p);
  a.q_pos = p.q_pos;
  a.log2_theta = p.rope ? log2(p.rope_theta) : 0.0;
  a.q_rot = p.q_rot;
  dim3 grid(a.total_wg), block(kThreads);
  const bool madd = sizeof(T) == 2 && p.mask_kind == kMaskAdd && a.mask.packed;
  // a boolean key padding mask ([B, Nk] broadcast over heads and rows, keys contiguous, every
  // sample's row 4-byte aligned and a whole number of dwords long for the dword copies, whose
  // resource ends at Nk bytes) with the output: the four-stage path
  const bool keypad = sizeof(T) == 2 && o != nullptr && !counters && p.mask_kind == kMaskBool && p.msq == 0 &&
                      p.msh == 0 && p.msk == 1 && p.msb % 4 == 0 && p.Nk % 4 == 0 &&
                      reinterpret_cast<unsigned long long>(p.mask) % 4 == 0 && (p.Nk + BN - 1) / BN <= kMaxTiles;
  if (p.rope) {   // always with an output; the host rejects counters with the rotary embedding
    if (o == nullptr || counters != nullptr) return hipErrorInvalidValue;
    if (keypad) {
      if constexpr (sizeof(T) == 2 && BN == kWave)
        hipLaunchKernelGGL((attn_fwd_kernel<T, D, BN, false, true, false, true, true>), grid, block, 0, stream, a);
    } else if (p.mask_kind != kMaskNone) {
      if constexpr (sizeof(T) == 2)
        if (madd) {
          hipLaunchKernelGGL((attn_fwd_kernel<T, D, BN, false, true, true, false, true, true>), grid, block, 0, stream, a);
          return hipGetLastError();
        }
      hipLaunchKernelGGL((attn_fwd_kernel<T, D, BN, false, true, true, false, true>), grid, block, 0, stream, a);
    } else {
      hipLaunchKernelGGL((attn_fwd_kernel<T, D, BN, false, true, false, false, true>), grid, block, 0, stream, a);
    }
  } else if (keypad) {
    if constexpr (sizeof(T) == 2 && BN == kWave)
      hipLaunchKernelGGL((attn_fwd_kernel<T, D, BN, false, true, false, true>), grid, block, 0, stream, a);
  } else if (p.mask_kind != kMaskNone) {
    if constexpr (sizeof(T) == 2)
      if (madd) {
        if (o == nullptr) hipLaunchKernelGGL((attn_fwd_kernel<T, D, BN, false, false, true, false, false, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_fwd_kernel<T, D, BN, false, true, true, false, false, true>), grid, block, 0, stream, a);
        return hipGetLastError();
      }
    if (o == nullptr) hipLaunchKernelGGL((attn_fwd_kernel<T, D, BN, false, false, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<T, D, BN, false, true, true>), grid, block, 0, stream, a);
  } else if (o == nullptr) {   // statistics only (m, l), for a backward without saved stats
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, BN, false, false, false>), grid, block, 0, stream, a);
  } else if (counters) {
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, BN, true, true, false>), grid, block, 0, stream, a);
  } else {
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, BN, false, true, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const AttnProblem& p, void* o, float* stats,
                           unsigned long long* counters, hipStream_t stream) {
  if (p.bf16) {
    if (p.D == 64) return launch_typed<bf16, 64, 64>(p, o, stats, counters, stream);
    return launch_typed<bf16, 128, 64>(p, o, stats, counters, stream);
  }
  if (p.D == 64) return launch_typed<float, 64, 32>(p, o, stats, counters, stream);
  return launch_typed<float, 128, 32>(p, o, stats, counters, stream);
}

}  // namespace ra
