// ra_bwd.hip -- backward rational-softmax attention for gfx950.
//
// Gradients of L = sum(O * dO).  From "Ra-Family: Rational Neural Architecture", section 3:
// the closed-form derivative d(phi)/du = -16 phi / (1 - u^2) (u < 1), evaluated from recomputed
// scores and the saved row statistics (m, l) only ("closed-form backward recomputation").
// With dP = dO V^T, c_i = dO_i . O_i and u = (m_i - s_ij) / 16 (scaled scores):
//   G_ij = p_ij (dP_ij - c_i) / (1 - u^2) = (dP_ij - c_i) / l_i * q^7 / (1 + u)^2,
// the second form having no division by 1 - u^2 (q = (1-u)/(1+u), so q^8 / (1 - u^2) =
// q^7 / (1+u)^2), and G = 0 off the support.  Unlike exp, phi is not shift-equivariant: the
// row max m_i = s_{i,a_i} carries R_i = -sum_j G_ij, so dS = G + R e_{a_i}, a_i the lowest key
// index attaining the max.  dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO, with dK and dV
// summed over the query heads that share a K/V head.
//
// Two kernels, no floating-point atomics (deterministic):
//   1. query-parallel (the forward's decomposition and S^T = K Q^T layout, so scores are
//      bit-identical to the forward's): c_i from O and dO, dP^T = V dO^T, G^T,
//      dQ^T += K^T G^T with K^T staged transposed, R_i and a_i; its epilogue adds the
//      row-max term scale * R_i * k_{a_i} to dQ and saves c, R, a.
//   2. key-parallel (one wave owns 32 keys, S = Q K^T so keys sit on the lanes): recomputes
//      P and G, adds R_i at (i, a_i), accumulates dV^T += dO^T P and dK^T += Q^T dS over all
//      query rows of the group's heads, with Q^T and dO^T staged transposed.
#include <limits.h>

#include "ra_device.h"
#include "ra_internal.h"

namespace ra {

size_t bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq) {
  const size_t rows = (size_t)B * Hq * Nq;
  return rows * (2 * sizeof(float) + 3 * sizeof(float) + sizeof(int) + 3 * sizeof(float)) + 256;
}

BwdWorkspace bwd_workspace_layout(void* base, int64_t B, int64_t Hq, int64_t Nq) {
  const size_t rows = (size_t)B * Hq * Nq;
  char* p = static_cast<char*>(base);
  BwdWorkspace ws;
  ws.stats = reinterpret_cast<float*>(p);
  p += rows * 2 * sizeof(float);
  ws.c = reinterpret_cast<float*>(p);
  p += rows * sizeof(float);
  ws.r = reinterpret_cast<float*>(p);
  p += rows * sizeof(float);
  ws.amax = reinterpret_cast<int*>(p);
  p += rows * sizeof(int);
  ws.kd = reinterpret_cast<float*>(p);
  p += rows * sizeof(float);
  ws.il = reinterpret_cast<float*>(p);
  p += rows * sizeof(float);
  ws.cil = reinterpret_cast<float*>(p);
  return ws;
}

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* d_o;
  const float* stats;
  void* dq;
  void* dk;
  void* dv;
  float* c;
  float* r;
  int* amax;
  float* kd;    // per-row terms for the key-parallel kernel: 1 + c16 m, 1/l, c/l
  float* il;
  float* cil;
  int Hq, Hkv, Nq, Nk, rep;
  int tasks_per_group, wg_per_group, total_wg;   // query-parallel kernel
  int kwg_per_group, total_kwg;                  // key-parallel kernel
  float scale, c16;                              // c16 = scale / 16
  int coff;        // causal diagonal: key j allowed for query row i iff j <= i + coff
  MaskArgs mask;   // explicit mask (MASKED kernels)
  // ROPE kernels: q and k hold the rotated rows, and dQ, dK are turned back by the inverse rotation
  // before they are stored (rows at q_pos, keys at k_pos; nullable: 0..N-1)
  const int* q_pos;
  const int* k_pos;
  double log2_theta;
};

// Stores the channels a lane holds of one dQ or dK row (row pointer at channel 0) after turning
// them back by the inverse rotary embedding: element 4 r4 + e of acc[db] is channel
// db*32 + 8 r4 + 4 (lane/32) + e, so channel j < D/2 and its pair j + D/2 (acc[db + DB/2]) lie in
// the same lane.  The value turned is s * (acc + radd * add), as store_quad_scaled forms it;
// add[db][r4][e] holds the matching addend.  cs(pr, j) gives (cos, sin) of the inverse turn of
// pair pr = (db * 4 + r4) * 4 + e of the lane, channel j.
template <typename T, int D, typename CS>
__device__ __forceinline__ void store_row_unrotated(T* row, const f32x16* acc, float s,
                                                    const float (*add)[4][4], float radd, CS&& cs,
                                                    int lane) {
  constexpr int DB = D / 32;
  using quad_t = typename Ty<T>::quad;
#pragma unroll
  for (int db = 0; db < DB / 2; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d0 = db * 32 + 8 * r4 + 4 * (lane >> 5);
      quad_t lo, hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x1 = s * fmaf(radd, add[db][r4][e], acc[db][4 * r4 + e]);
        const float x2 = s * fmaf(radd, add[db + DB / 2][r4][e], acc[db + DB / 2][4 * r4 + e]);
        const f32x2 v = cs((db * 4 + r4) * 4 + e, d0 + e);
        float y1, y2;
        rope_pair(x1, x2, v[0], v[1], y1, y2);
        lo[e] = (T)y1;
        hi[e] = (T)y2;
      }
      *reinterpret_cast<quad_t*>(row + d0) = lo;
      *reinterpret_cast<quad_t*>(row + d0 + D / 2) = hi;
    }
}

// Channel of pair pr = (db * 4 + r4) * 4 + e of a lane in store_row_unrotated.
__device__ __forceinline__ int unrot_channel(int pr, int lane) {
  return (pr >> 4) * 32 + 8 * ((pr >> 2) & 3) + 4 * (lane >> 5) + (pr & 3);
}

// Row statistics of a row with no allowed key (m = -inf) are mapped so that every entry lands
// off the support: t = m - s = +inf, 1 + u = +inf.  The argmax test compares with NaN instead,
// so such a row records no argmax.
__device__ __forceinline__ float live_max(float m) { return m == -INFINITY ? INFINITY : m; }
__device__ __forceinline__ float argmax_probe(float m) { return m == -INFINITY ? __builtin_nanf("") : m; }

constexpr int kKeysPerWg = kWaves * kRowsPerWave;   // key-parallel kernel: 128 keys per workgroup
constexpr int kQTile = 32;                           // query rows per step of the key-parallel kernel

__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }

template <typename T>
__device__ __forceinline__ void store_quad_scaled(T* dst, const f32x16& acc, int base, float s,
                                                 const float* add, float radd);

template <>
__device__ __forceinline__ void store_quad_scaled<bf16>(bf16* dst, const f32x16& acc, int base,
                                                        float s, const float* add, float radd) {
  bf16x4 v = {(bf16)(s * fmaf(radd, add[0], acc[base])), (bf16)(s * fmaf(radd, add[1], acc[base + 1])),
              (bf16)(s * fmaf(radd, add[2], acc[base + 2])), (bf16)(s * fmaf(radd, add[3], acc[base + 3]))};
  *reinterpret_cast<bf16x4*>(dst) = v;
}
template <>
__device__ __forceinline__ void store_quad_scaled<float>(float* dst, const f32x16& acc, int base,
                                                         float s, const float* add, float radd) {
  f32x4 v = {s * fmaf(radd, add[0], acc[base]), s * fmaf(radd, add[1], acc[base + 1]),
             s * fmaf(radd, add[2], acc[base + 2]), s * fmaf(radd, add[3], acc[base + 3])};
  *reinterpret_cast<f32x4*>(dst) = v;
}

// Sum of a fragment's elements (bf16: the rounded values, two per dot instruction).
__device__ __forceinline__ float frag_sum(const bf16x8& f, float acc) {
#pragma unroll
  for (int j = 0; j < 8; j += 2)
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{f[j], f[j + 1]}, bf16x2{(bf16)1.0f, (bf16)1.0f}, acc, false);
  return acc;
}
__device__ __forceinline__ float frag_sum(const f32x8& f, float acc) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc += f[j];
  return acc;
}

template <typename T> __device__ __forceinline__ typename Ty<T>::frag pack_frag(const f32x16& s, int ks);
template <> __device__ __forceinline__ bf16x8 pack_frag<bf16>(const f32x16& s, int ks) { return pack_frag_bf16(s, ks); }
template <> __device__ __forceinline__ f32x8 pack_frag<float>(const f32x16& s, int ks) { return pack_frag_f32(s, ks); }

// ------------------------------------------------------------------ query-parallel: dQ, R, a

// ROPE: q and k hold the rotated rows; dQ is turned back by the inverse rotation before it is
// stored (the angles formed per lane in the epilogue).
template <typename T, int D, int BN, bool CAUSAL, bool MASKED, bool ROPE = false>
__global__ __launch_bounds__(kThreads) void attn_bwd_dq_kernel(BwdArgs a) {
  using frag_t = typename Ty<T>::frag;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int PK = D + PAD;
  constexpr int PT = BN + PAD;
  constexpr int KC = D / 16, SB = BN / 32, DB = D / 32;

  __shared__ __attribute__((aligned(16))) T k_lds[BN * PK];
  __shared__ __attribute__((aligned(16))) T v_lds[BN * PK];
  __shared__ __attribute__((aligned(16))) T kt_lds[D * PT];
  __shared__ double rate_lds[ROPE ? D / 2 : 1];   // ROPE: theta^(-2j/D) per pair j

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if constexpr (ROPE) {
    if (tid < D / 2) rate_lds[tid] = rope_rate(tid, D, a.log2_theta);
    __syncthreads();
  }
  const int logical = xcd_remap(blockIdx.x, a.total_wg);
  const int bg = logical / a.wg_per_group;
  int wig = logical % a.wg_per_group;
  if (CAUSAL) wig = a.wg_per_group - 1 - wig;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int task = wig * kWaves + wave;
  const bool active = task < a.tasks_per_group;
  const int h = g * a.rep + (active ? task % a.rep : 0);
  const int q0 = (active ? task / a.rep : 0) * kRowsPerWave;
  const int last_task = min(wig * kWaves + kWaves - 1, a.tasks_per_group - 1);
  const int wg_qmax = min((last_task / a.rep) * kRowsPerWave + kRowsPerWave - 1, a.Nq - 1);
  const int nt = ((CAUSAL ? max(0, min(a.Nk, wg_qmax + a.coff + 1)) : a.Nk) + BN - 1) / BN;
  const int wave_qmax = min(q0 + kRowsPerWave - 1, a.Nq - 1);
  const int nt_w = !active ? 0 : ((CAUSAL ? max(0, min(a.Nk, wave_qmax + a.coff + 1)) : a.Nk) + BN - 1) / BN;

  const size_t head = (size_t)(b * a.Hq + h) * a.Nq;
  const T* kg = static_cast<const T*>(a.k) + (size_t)(b * a.Hkv + g) * a.Nk * D;
  const T* vg = static_cast<const T*>(a.v) + (size_t)(b * a.Hkv + g) * a.Nk * D;
  const int qi = q0 + (lane & 31);
  const int qrow = min(qi, a.Nq - 1);
  const int frow = lane & 31, fcol = 8 * (lane >> 5);

  const T* qp = static_cast<const T*>(a.q) + (head + qrow) * D;
  const T* dop = static_cast<const T*>(a.d_o) + (head + qrow) * D;
  const T* op = static_cast<const T*>(a.o) + (head + qrow) * D;
  frag_t qf[KC], df[KC];
  float cpart = 0.0f;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    qf[kc] = load_frag(qp + 16 * kc + fcol);
    df[kc] = load_frag(dop + 16 * kc + fcol);
    const frag_t of = load_frag(op + 16 * kc + fcol);
#pragma unroll
    for (int j = 0; j < 8; ++j) cpart = fmaf(to_f(df[kc][j]), to_f(of[j]), cpart);
  }
  const float cval = cpart + __shfl_xor(cpart, 32);   // c_i = dO_i . O_i
  const float m = a.stats[(head + qrow) * 2];
  const float l = a.stats[(head + qrow) * 2 + 1];
  const float il = l > 0.0f ? 1.0f / l : 0.0f;
  const float cil = cval * il;
  const float mt = live_max(m), mprobe = argmax_probe(m);
  const MaskSlice<T> ms(a.mask, b, h);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float rsum = 0.0f;
  int amax = INT_MAX;

  for (int kt = 0; kt < nt; ++kt) {
    __syncthreads();
    const T* kt_g = kg + (size_t)kt * BN * D;
    stage_rows<T, D, BN, PK>(k_lds, kt_g, a.Nk - kt * BN, tid);
    stage_rows<T, D, BN, PK>(v_lds, vg + (size_t)kt * BN * D, a.Nk - kt * BN, tid);
    stage_rows_transposed<T, D, BN, PT>(kt_lds, kt_g, a.Nk - kt * BN, tid);
    __syncthreads();
    if (kt >= nt_w) continue;
#pragma unroll
    for (int sb = 0; sb < SB; ++sb) {
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) mma(s, load_frag(k_lds + (sb * 32 + frow) * PK + 16 * kc + fcol), qf[kc]);
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) mma(dp, load_frag(v_lds + (sb * 32 + frow) * PK + 16 * kc + fcol), df[kc]);
      const int key0 = kt * BN + sb * 32;
      if (MASKED || (CAUSAL && key0 + 31 > q0 + a.coff) || key0 + 32 > a.Nk) {
        if constexpr (MASKED) {
          unsigned mv[16];
          ms.load_keys(mv, qrow * ms.sq + (key0 + 4 * (lane >> 5)) * ms.sk);
#pragma unroll
          for (int i = 0; i < 16; ++i) s[i] = ms.apply(s[i], mv[i]);
        }
        const int lb = key0 + 4 * (lane >> 5);
        keep_rows(s, -kNoBound, min(a.Nk - lb, CAUSAL ? qrow + a.coff + 1 - lb : kNoBound));
      }
      // lowest key attaining the row max (rare: only the tile holding it takes the branch)
      float lm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) lm = fmaxf(lm, s[i]);
      if (__any(lm == mprobe)) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (s[i] == mprobe) amax = min(amax, key0 + acc_row(i, lane));
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p;
        s[i] = ra_grad_t(mt - s[i], a.c16, fmaf(dp[i], il, -cil), il, &p);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const frag_t gf = pack_frag<T>(s, ks);
        rsum = frag_sum(gf, rsum);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          mma(acc[db], load_frag(kt_lds + (db * 32 + frow) * PT + sb * 32 + 16 * ks + fcol), gf);
      }
    }
  }

  const float R = -(rsum + __shfl_xor(rsum, 32));
  amax = min(amax, __shfl_xor(amax, 32));
  if (active && qi < a.Nq) {
    T* dqrow = static_cast<T*>(a.dq) + (head + qi) * D;
    const bool has_max = amax < a.Nk;
    const T* krow = kg + (size_t)(has_max ? amax : 0) * D;
    const float radd = has_max ? R : 0.0f;
    if constexpr (ROPE) {
      float kv[DB][4][4];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
          for (int e = 0; e < 4; ++e) kv[db][r4][e] = to_f(krow[db * 32 + 8 * r4 + 4 * (lane >> 5) + e]);
      const double pos = a.q_pos != nullptr ? (double)a.q_pos[qi] : (double)qi;
      store_row_unrotated<T, D>(dqrow, acc, a.scale, kv, radd, [&](int, int j) {
        float c, sn;
        rope_cs(pos, rate_lds[j], true, c, sn);
        return f32x2{c, sn};
      }, lane);
    } else {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = db * 32 + 8 * r4 + 4 * (lane >> 5);
          float kv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) kv[e] = to_f(krow[d0 + e]);
          store_quad_scaled<T>(dqrow + d0, acc[db], 4 * r4, a.scale, kv, radd);
        }
    }
    if (lane < 32) {
      a.c[head + qi] = cval;
      a.r[head + qi] = R;
      a.amax[head + qi] = has_max ? amax : -1;
      a.kd[head + qi] = m == -INFINITY ? INFINITY : fmaf(m, a.c16, 1.0f);
      a.il[head + qi] = il;
      a.cil[head + qi] = cil;
    }
  }
}

// ------------------------------------------------------------------ key-parallel: dK, dV

// ROPE: dK is turned back by the inverse rotation before it is stored.
template <typename T, int D, bool CAUSAL, bool MASKED, bool ROPE = false>
__global__ __launch_bounds__(kThreads) void attn_bwd_dkdv_kernel(BwdArgs a) {
  using frag_t = typename Ty<T>::frag;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int PQ = D + PAD;
  constexpr int PT = kQTile + PAD;
  constexpr int KC = D / 16, DB = D / 32;
  // Q and dO row tiles (A operands of S and dP) go through LDS unless that would push the
  // static LDS past 64 KiB (fp32, D = 128): then the fragments are read from global memory.
  constexpr bool ROWS_IN_LDS = sizeof(T) == 2 || D == 64;
  constexpr int ROW_TILE = ROWS_IN_LDS ? kQTile * PQ : 8;

  __shared__ __attribute__((aligned(16))) T q_lds[ROW_TILE];
  __shared__ __attribute__((aligned(16))) T do_lds[ROW_TILE];
  __shared__ __attribute__((aligned(16))) T qt_lds[D * PT];
  __shared__ __attribute__((aligned(16))) T dot_lds[D * PT];
  __shared__ __attribute__((aligned(16))) float st_m[kQTile];
  __shared__ __attribute__((aligned(16))) float st_il[kQTile];
  __shared__ __attribute__((aligned(16))) float st_cil[kQTile];
  __shared__ __attribute__((aligned(16))) float st_r[kQTile];
  __shared__ __attribute__((aligned(16))) int st_a[kQTile];
  __shared__ double rate_lds[ROPE ? D / 2 : 1];   // ROPE: theta^(-2j/D) per pair j

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if constexpr (ROPE) {
    if (tid < D / 2) rate_lds[tid] = rope_rate(tid, D, a.log2_theta);
    __syncthreads();
  }
  const int logical = xcd_remap(blockIdx.x, a.total_kwg);
  const int bg = logical / a.kwg_per_group;
  const int kb = logical % a.kwg_per_group;   // low key blocks (most causal work) first
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int key0_wg = kb * kKeysPerWg;
  const int j0 = key0_wg + wave * kRowsPerWave;
  const bool active = j0 < a.Nk;
  const int frow = lane & 31, fcol = 8 * (lane >> 5);
  const int key = j0 + frow;
  const int krow = min(key, a.Nk - 1);

  const size_t kvbase = (size_t)(b * a.Hkv + g) * a.Nk;
  const T* kp = static_cast<const T*>(a.k) + (kvbase + krow) * D;
  const T* vp = static_cast<const T*>(a.v) + (kvbase + krow) * D;
  frag_t kf[KC], vf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    kf[kc] = load_frag(kp + 16 * kc + fcol);
    vf[kc] = load_frag(vp + 16 * kc + fcol);
  }
  f32x16 acc_dk[DB], acc_dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    acc_dk[db] = f32x16{};
    acc_dv[db] = f32x16{};
  }

  const int nqt = (a.Nq + kQTile - 1) / kQTile;
  // first query tile holding a row i >= key0_wg - coff (the lowest key's first allowed row)
  const int qt0 = CAUSAL ? min(max(key0_wg - a.coff, 0) / kQTile, nqt) : 0;
  for (int hh = 0; hh < a.rep; ++hh) {
    const int h = g * a.rep + hh;
    const MaskSlice<T> ms(a.mask, b, h);
    const size_t head = (size_t)(b * a.Hq + h) * a.Nq;
    const T* qh = static_cast<const T*>(a.q) + head * D;
    const T* doh = static_cast<const T*>(a.d_o) + head * D;
    for (int qt = qt0; qt < nqt; ++qt) {
      const int i0 = qt * kQTile;
      __syncthreads();
      if constexpr (ROWS_IN_LDS) {
        stage_rows<T, D, kQTile, PQ>(q_lds, qh + (size_t)i0 * D, a.Nq - i0, tid);
        stage_rows<T, D, kQTile, PQ>(do_lds, doh + (size_t)i0 * D, a.Nq - i0, tid);
      }
      stage_rows_transposed<T, D, kQTile, PT>(qt_lds, qh + (size_t)i0 * D, a.Nq - i0, tid);
      stage_rows_transposed<T, D, kQTile, PT>(dot_lds, doh + (size_t)i0 * D, a.Nq - i0, tid);
      if (tid < kQTile) {
        const int qi = i0 + tid;
        if (qi < a.Nq) {
          const float l = a.stats[(head + qi) * 2 + 1];
          const float il = l > 0.0f ? 1.0f / l : 0.0f;
          st_m[tid] = live_max(a.stats[(head + qi) * 2]);
          st_il[tid] = il;
          st_cil[tid] = a.c[head + qi] * il;
          st_r[tid] = a.r[head + qi];
          st_a[tid] = a.amax[head + qi];
        } else {
          st_m[tid] = 0.0f;
          st_il[tid] = 0.0f;
          st_cil[tid] = 0.0f;
          st_r[tid] = 0.0f;
          st_a[tid] = -1;
        }
      }
      __syncthreads();
      if (!active || (CAUSAL && i0 + kQTile - 1 + a.coff < j0)) continue;
      f32x16 s = {}, dp = {};
      if constexpr (ROWS_IN_LDS) {
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) mma(s, load_frag(q_lds + frow * PQ + 16 * kc + fcol), kf[kc]);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) mma(dp, load_frag(do_lds + frow * PQ + 16 * kc + fcol), vf[kc]);
      } else {
        const int qr = min(i0 + frow, a.Nq - 1);   // rows past Nq are masked below
        const T* qrp = qh + (size_t)qr * D + fcol;
        const T* dorp = doh + (size_t)qr * D + fcol;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) mma(s, load_frag(qrp + 16 * kc), kf[kc]);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) mma(dp, load_frag(dorp + 16 * kc), vf[kc]);
      }
      const bool edge = MASKED || (CAUSAL && j0 + 31 > i0 + a.coff) || i0 + kQTile > a.Nq || j0 + 32 > a.Nk;
      if (edge) {
        if constexpr (MASKED) {
          unsigned mv[16];
          ms.load(mv, key * ms.sk + (i0 + 4 * (lane >> 5)) * ms.sq, ms.sq);
#pragma unroll
          for (int i = 0; i < 16; ++i) s[i] = ms.apply(s[i], mv[i]);
        }
        // query row i0 + 4 (lane >> 5) + r is kept iff r < Nq - i0 - 4 (lane >> 5), key <= row +
        // coff (causal) and key < Nk
        const int lb = 4 * (lane >> 5);
        keep_rows(s, (CAUSAL ? key - a.coff - i0 : -kNoBound) - lb, key >= a.Nk ? -kNoBound : a.Nq - i0 - lb);
      }
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int r0 = 8 * i4 + 4 * (lane >> 5);   // four consecutive query rows of this lane
        const f32x4 m4 = *reinterpret_cast<const f32x4*>(st_m + r0);
        const f32x4 il4 = *reinterpret_cast<const f32x4*>(st_il + r0);
        const f32x4 cil4 = *reinterpret_cast<const f32x4*>(st_cil + r0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * i4 + e;
          float p;
          const float gv = ra_grad_t(m4[e] - s[i], a.c16, fmaf(dp[i], il4[e], -cil4[e]), il4[e], &p);
          s[i] = p;
          dp[i] = gv;
        }
      }
      // row-max term: R_i joins dS at the lowest argmax key of row i
      {
        const int am = st_a[lane & 31];
        if (__any(am >= j0 && am < j0 + 32)) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = acc_row(i, lane);
            if (st_a[r] == key) dp[i] += st_r[r];
          }
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const frag_t pf = pack_frag<T>(s, ks);
        const frag_t gf = pack_frag<T>(dp, ks);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          mma(acc_dv[db], load_frag(dot_lds + (db * 32 + frow) * PT + 16 * ks + fcol), pf);
          mma(acc_dk[db], load_frag(qt_lds + (db * 32 + frow) * PT + 16 * ks + fcol), gf);
        }
      }
    }
  }

  if (active && key < a.Nk) {
    T* dkrow = static_cast<T*>(a.dk) + (kvbase + key) * D;
    T* dvrow = static_cast<T*>(a.dv) + (kvbase + key) * D;
    const float zero4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (ROPE) {
      const float zero[DB][4][4] = {};
      const double pos = a.k_pos != nullptr ? (double)a.k_pos[key] : (double)key;
      store_row_unrotated<T, D>(dkrow, acc_dk, a.scale, zero, 0.0f, [&](int, int j) {
        float c, sn;
        rope_cs(pos, rate_lds[j], true, c, sn);
        return f32x2{c, sn};
      }, lane);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + 8 * r4 + 4 * (lane >> 5);
        if constexpr (!ROPE) store_quad_scaled<T>(dkrow + d0, acc_dk[db], 4 * r4, a.scale, zero4, 0.0f);
        store_quad_scaled<T>(dvrow + d0, acc_dv[db], 4 * r4, 1.0f, zero4, 0.0f);
      }
  }
}

// ------------------------------------------------------------------ bf16 kernels
// Same mathematics as the kernels above, laid out for gfx950: K/V (query-parallel kernel) and
// Q/dO (key-parallel kernel) tiles are brought into LDS by DMA as XOR-swizzled row tiles,
// double-buffered with one barrier per step; every transposed operand (K^T for dQ, Q^T for dK,
// dO^T for dV) is read with the LDS transposing load from the same row tile, so nothing is
// staged twice and no register holds a tile in flight.

// Direct gradient and probability of one entry: with d = 1 + u = fma(s, -c, kd),
// q = clamp(2/d - 1), p = q^8 * il and G = (dP * il - c * il) * q^7 / d^2.
// Fragment reads at an LDS byte address (a register plus an immediate offset in the instruction):
// a row fragment (16 bytes), and a transposed fragment from its two 8-byte halves (rows 0-7 and
// 8-15 of its 16-row block, as tr_frag reads them).
__device__ __forceinline__ bf16x8 lds_frag_at(unsigned addr) {
  typedef __attribute__((address_space(3))) const bf16x8 lds_frag_t;
  return *reinterpret_cast<lds_frag_t*>((size_t)addr);
}
__device__ __forceinline__ bf16x8 lds_tr_frag_at(unsigned a1, unsigned a2) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t)a1);
  const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t)a2);
  const short8 v = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float ra_grad(float s, float c16, float kd, float dp, float il, float cil,
                                         float* p) {
  const float d = fmaf(s, -c16, kd);
  const float r = __builtin_amdgcn_rcpf(d);
  const float q = fminf(fmaxf(fmaf(r, 2.0f, -1.0f), 0.0f), 1.0f);
  const float q2 = q * q;
  const float q4 = q2 * q2;
  const float q6 = q4 * q2;
  *p = (q4 * q4) * il;
  return fmaf(dp, il, -cil) * ((q6 * q) * (r * r));
}

// The gradient alone (the dQ kernel needs no p): q^7 r^2 as (q^3 r)^2 q, six multiplications
// instead of seven.
__device__ __forceinline__ float ra_grad_only(float s, float c16, float kd, float dp, float il, float cil) {
  const float d = fmaf(s, -c16, kd);
  const float r = __builtin_amdgcn_rcpf(d);
  const float q = fminf(fmaxf(fmaf(r, 2.0f, -1.0f), 0.0f), 1.0f);
  const float q3 = (q * q) * q;
  const float w = q3 * r;
  return fmaf(dp, il, -cil) * ((w * w) * q);
}

// KEYPAD (with MASKED false): a boolean key padding mask.  Wave 0 copies each tile's 64 mask bytes
// with its K and V tiles; the 64 keep bits drop whole padded blocks and mask the partial ones.
// MADD (with MASKED): the mask is additive in the packed layout, read as 16-byte runs; a variant
// of its own, so the boolean kernel keeps its registers.
template <int D, bool CAUSAL, bool MASKED, bool KEYPAD = false, bool ROPE = false, bool MADD = false>
__global__ __launch_bounds__(kThreads) void attn_bwd_dq_bf16_kernel(BwdArgs a) {
  constexpr int BN = 64, KC = D / 16, SB = BN / 32, DB = D / 32;
  static_assert(!(KEYPAD && MASKED), "key padding runs the unmasked paths");
  static_assert(!MADD || MASKED, "packed additive masks: masked kernels");
  // the K and V tiles, two buffers each, in one array (K0, K1, V0, V1): every buffer then lies at
  // a constant offset below 64 KiB from the first, an immediate of the LDS read instructions
  __shared__ __attribute__((aligned(16))) bf16 kv_lds[4][BN * D];
  bf16 (*const k_lds)[BN * D] = kv_lds;
  bf16 (*const v_lds)[BN * D] = kv_lds + 2;
  __shared__ __attribute__((aligned(16))) unsigned m_lds[KEYPAD ? 2 : 1][KEYPAD ? kWave : 1];
  __shared__ double rate_lds[ROPE ? D / 2 : 1];   // ROPE: theta^(-2j/D) per pair j

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if constexpr (ROPE) {
    if (tid < D / 2) rate_lds[tid] = rope_rate(tid, D, a.log2_theta);
    __syncthreads();
  }
  const int logical = xcd_remap(blockIdx.x, a.total_wg);
  const int bg = logical / a.wg_per_group;
  int wig = logical % a.wg_per_group;
  if (CAUSAL) wig = a.wg_per_group - 1 - wig;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int task = wig * kWaves + wave;
  const bool active = task < a.tasks_per_group;
  const int h = g * a.rep + (active ? task % a.rep : 0);
  const int q0 = (active ? task / a.rep : 0) * kRowsPerWave;
  const int last_task = min(wig * kWaves + kWaves - 1, a.tasks_per_group - 1);
  const int wg_qmax = min((last_task / a.rep) * kRowsPerWave + kRowsPerWave - 1, a.Nq - 1);
  const int nt = ((CAUSAL ? max(0, min(a.Nk, wg_qmax + a.coff + 1)) : a.Nk) + BN - 1) / BN;
  const int wave_qmax = min(q0 + kRowsPerWave - 1, a.Nq - 1);
  const int nt_w = !active ? 0 : ((CAUSAL ? max(0, min(a.Nk, wave_qmax + a.coff + 1)) : a.Nk) + BN - 1) / BN;

  const size_t head = (size_t)(b * a.Hq + h) * a.Nq;
  const bf16* kg = static_cast<const bf16*>(a.k) + (size_t)(b * a.Hkv + g) * a.Nk * D;
  const bf16* vg = static_cast<const bf16*>(a.v) + (size_t)(b * a.Hkv + g) * a.Nk * D;
  const int qi = q0 + (lane & 31);
  const int qrow = min(qi, a.Nq - 1);
  const int frow = lane & 31, fcol = 8 * (lane >> 5);

  // one resource per matrix (K, V of the group), the tile picked by a scalar offset
  const u32x4 k_rsrc = dma_rsrc(kg, a.Nk * D * 2), v_rsrc = dma_rsrc(vg, a.Nk * D * 2);
  const int lane_off = dma_lane_offset<D, kWaves>(wave, lane);
  const unsigned k_m0[2] = {lds_addr(k_lds[0]), lds_addr(k_lds[1])};
  const unsigned v_m0[2] = {lds_addr(v_lds[0]), lds_addr(v_lds[1])};
  u32x4 m_rsrc = {};
  if constexpr (KEYPAD) m_rsrc = dma_rsrc(static_cast<const char*>(a.mask.ptr) + (size_t)b * a.mask.sb, a.Nk);
  auto m_issue = [&](int kt, int slot) {   // the tile's 64 mask bytes (lanes 0-15)
    if constexpr (KEYPAD)
      if (wave == 0) lds_dma_at<4>(m_rsrc, lds_addr(m_lds[slot]), lane * 4, kt * BN);
  };
  // tile 0 is in flight while the row terms are prepared
  if (nt > 0) {
    dma_tile_at<D, BN>(k_rsrc, 0, k_m0[0], lane_off, wave);
    dma_tile_at<D, BN>(v_rsrc, 0, v_m0[0], lane_off, wave);
    m_issue(0, 0);
  }
  const bf16* qp = static_cast<const bf16*>(a.q) + (head + qrow) * D;
  const bf16* dop = static_cast<const bf16*>(a.d_o) + (head + qrow) * D;
  const bf16* op = static_cast<const bf16*>(a.o) + (head + qrow) * D;
  bf16x8 qf[KC], df[KC];
  float cpart = 0.0f;
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    qf[kc] = load_frag(qp + 16 * kc + fcol);
    df[kc] = load_frag(dop + 16 * kc + fcol);
    const bf16x8 of = load_frag(op + 16 * kc + fcol);
#pragma unroll
    for (int j = 0; j < 8; ++j) cpart = fmaf((float)df[kc][j], (float)of[j], cpart);
  }
  const float cval = cpart + __shfl_xor(cpart, 32);   // c_i = dO_i . O_i
  const float m = a.stats[(head + qrow) * 2];
  const float l = a.stats[(head + qrow) * 2 + 1];
  const float il = l > 0.0f ? 1.0f / l : 0.0f;
  const float cil = cval * il;
  const float kd = m == -INFINITY ? INFINITY : fmaf(m, a.c16, 1.0f);
  const float mprobe = argmax_probe(m);
  const MaskSlice<bf16> ms(a.mask, b, h);
  const bool madd = MADD && ms.packed;
  const bool mpack = MASKED && ms.packed && (MADD || ms.kind == kMaskBool);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float rsum = 0.0f;
  int amax = INT_MAX;

  // Fragment reads.  The unmasked kernels address them from the first buffer: one opaque register
  // per fragment this lane reads, to which the buffer, the 32-key block and the 16-row block add
  // immediate offsets (swz(r + 16) = swz(r)), and their tile loop is unrolled over the two buffers.
  // With the buffer in a register, every read cost address instructions in each step.  The masked
  // kernels keep the rolled loop: they have no registers to spare.
  constexpr unsigned TB = BN * D * 2;   // bytes of one tile buffer
  static_assert(swz<bf16, D>(5) == swz<bf16, D>(21) && swz<bf16, D>(14) == swz<bf16, D>(62),
                "16-row block offsets");
  unsigned ad_row[KC] = {}, ad_tr[2 * DB] = {};
  if constexpr (!MASKED) {
    const unsigned b0 = lds_addr(kv_lds);
    const int g4 = lane >> 4, l16 = lane & 15;
    const int trow = 4 * (g4 >> 1) + (l16 >> 2);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      ad_row[kc] = b0 + 2u * swz_off<bf16, D>(frow, 2 * kc + (lane >> 5));
      asm volatile("" : "+v"(ad_row[kc]));
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = 32 * db + 16 * (g4 & 1) + 4 * (l16 & 3);
      ad_tr[2 * db] = b0 + 2u * (swz_off<bf16, D>(trow, col >> 3) + (col & 7));
      ad_tr[2 * db + 1] = b0 + 2u * (swz_off<bf16, D>(trow + 8, col >> 3) + (col & 7));
      asm volatile("" : "+v"(ad_tr[2 * db]));
      asm volatile("" : "+v"(ad_tr[2 * db + 1]));
    }
  }
  auto k_row = [&](int buf, int sb, int kc) -> bf16x8 {   // K rows sb 32 + frow (A of S^T)
    if constexpr (MASKED) return swz_frag<bf16, D>(k_lds[buf], sb * 32 + frow, 16 * kc + fcol);
    else return lds_frag_at(ad_row[kc] + buf * TB + sb * 32 * D * 2);
  };
  auto v_row = [&](int buf, int sb, int kc) -> bf16x8 {
    if constexpr (MASKED) return swz_frag<bf16, D>(v_lds[buf], sb * 32 + frow, 16 * kc + fcol);
    else return lds_frag_at(ad_row[kc] + (2 + buf) * TB + sb * 32 * D * 2);
  };
  auto k_tr = [&](int buf, int k0, int db) -> bf16x8 {     // K^T rows k0 .. k0 + 15, columns 32 db
    if constexpr (MASKED) return tr_frag<D>(k_lds[buf], k0, db * 32, lane);
    else return lds_tr_frag_at(ad_tr[2 * db] + buf * TB + k0 * D * 2, ad_tr[2 * db + 1] + buf * TB + k0 * D * 2);
  };
  wait_vmem();
  __syncthreads();

  constexpr int U = MASKED ? 1 : 2;   // tiles per iteration
  for (int kt0 = 0; kt0 < nt; kt0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kt = kt0 + u;
      if (U > 1 && kt >= nt) break;
      const int buf = U > 1 ? u : kt & 1;
      if (kt + 1 < nt) {
        dma_tile_at<D, BN>(k_rsrc, (kt + 1) * BN * D * 2, k_m0[buf ^ 1], lane_off, wave);
        dma_tile_at<D, BN>(v_rsrc, (kt + 1) * BN * D * 2, v_m0[buf ^ 1], lane_off, wave);
        m_issue(kt + 1, buf ^ 1);
      }
      unsigned long long keep = ~0ull;   // KEYPAD: bit l set when key kt BN + l is kept
      if constexpr (KEYPAD) keep = __ballot(reinterpret_cast<const unsigned char*>(m_lds[buf])[lane] != 0);
      if (kt < nt_w) {
#pragma unroll
        for (int sb = 0; sb < SB; ++sb) {
          if (KEYPAD && ((keep >> (32 * sb)) & 0xffffffffull) == 0) continue;   // all padding
          // MASKED with a boolean mask in the packed layout: the block's mask words are read
          // before its products and tested after them (a wait before them would also wait for
          // the next tile's copies, issued earlier in the step), and a block the mask empties for
          // every row of the wave stops there (its entries add nothing to dQ, R or the argmax).
          // An additive mask in that layout the same way, with its elements (all -inf: empty).
          u32x4 mwp, mwp2;
          if constexpr (MADD) {
            if (madd) ms.load_run_pairs(qrow * ms.sq + (kt * BN + sb * 32 + 4 * (lane >> 5)) * ms.sk, mwp, mwp2);
          } else if constexpr (MASKED) {
            if (mpack) mwp = ms.load_word_pairs(qrow * ms.sq + (kt * BN + sb * 32 + 4 * (lane >> 5)) * ms.sk);
          }
          f32x16 s = {}, dp = {};
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) mma(s, k_row(buf, sb, kc), qf[kc]);
#pragma unroll
          for (int kc = 0; kc < KC; ++kc) mma(dp, v_row(buf, sb, kc), df[kc]);
          unsigned mw[4], md[8];
          bool mzero = false;   // MADD: every element of the block is +-0 (the same in every lane)
          if constexpr (MADD) {
            if (madd) {
              unsigned nz, ni;
              MaskSlice<bf16>::run_flags(mwp, mwp2, nz, ni);
              if (!__any(ni != 0u)) continue;   // only -inf
              mzero = !__any(nz != 0u);
              if (!mzero) MaskSlice<bf16>::runs_of_pairs(mwp, mwp2, md);
            }
          } else if constexpr (MASKED) {
            if (mpack) {
              MaskSlice<bf16>::words_of_pairs(mwp, mw);
              if (!__any((mw[0] | mw[1] | mw[2] | mw[3]) != 0u)) continue;
            }
          }
          const int key0 = kt * BN + sb * 32;
          if (MASKED || (CAUSAL && key0 + 31 > q0 + a.coff) || key0 + 32 > a.Nk) {
            if constexpr (MASKED) {
              if (!mzero) {
                unsigned mv[16];
                if (MADD && madd) MaskSlice<bf16>::expand_runs(md, mv);
                else if (!MADD && mpack) MaskSlice<bf16>::expand_words(mw, mv);
                else ms.load_keys(mv, qrow * ms.sq + (key0 + 4 * (lane >> 5)) * ms.sk);
#pragma unroll
                for (int i = 0; i < 16; ++i) s[i] = ms.apply(s[i], mv[i]);
              }
            }
            const int lb = key0 + 4 * (lane >> 5);
            keep_rows(s, -kNoBound, min(a.Nk - lb, CAUSAL ? qrow + a.coff + 1 - lb : kNoBound));
          }
          if constexpr (KEYPAD)
            if (keep != ~0ull) keep_keys(s, keep, sb, lane);
          float lm = -INFINITY;
#pragma unroll
          for (int i = 0; i < 16; ++i) lm = fmaxf(lm, s[i]);
          if (__any(lm == mprobe)) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (s[i] == mprobe) amax = min(amax, key0 + acc_row(i, lane));
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) s[i] = ra_grad_only(s[i], a.c16, kd, dp[i], il, cil);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 gf = pack_frag_bf16(s, ks);
            rsum = frag_sum(gf, rsum);
#pragma unroll
            for (int db = 0; db < DB; ++db)
              mma(acc[db], k_tr(buf, sb * 32 + 16 * ks, db), gf);
          }
        }
      }
      wait_vmem();
      __syncthreads();
    }
  }

  const float R = -(rsum + __shfl_xor(rsum, 32));
  amax = min(amax, __shfl_xor(amax, 32));
  // ROPE: the (cos, sin) pairs of the inverse turn, [pair][lane], in the K/V buffers (idle after
  // the loop).  When the four waves hold the same rows (rep a multiple of four) they split one
  // table; otherwise each wave fills its own.  Rolled loops, so that the angles' code is not
  // repeated per pair.
  const f32x2* cs_tab = nullptr;
  if constexpr (ROPE) {
    constexpr int NP = D / 4;
    static_assert(2 * NP * kWave * sizeof(f32x2) <= 2 * BN * D * sizeof(bf16), "cos/sin tables fit the K/V buffers");
    f32x2* tab = reinterpret_cast<f32x2*>(&k_lds[0][0]);
    const double pos = a.q_pos != nullptr ? (double)a.q_pos[qrow] : (double)qrow;
    if (a.rep % kWaves == 0) {
      constexpr int PW = NP / kWaves;
#pragma unroll 2
      for (int i = 0; i < PW; ++i) {
        const int pr = wave * PW + i;
        float c, sn;
        rope_cs(pos, rate_lds[unrot_channel(pr, lane)], true, c, sn);
        tab[pr * kWave + lane] = f32x2{c, sn};
      }
      __syncthreads();
    } else {   // waves 0, 1 in the K buffers, 2, 3 in the V buffers
      tab = reinterpret_cast<f32x2*>(wave < 2 ? &k_lds[0][0] : &v_lds[0][0]) + (wave & 1) * NP * kWave;
#pragma unroll 2
      for (int pr = 0; pr < NP; ++pr) {
        float c, sn;
        rope_cs(pos, rate_lds[unrot_channel(pr, lane)], true, c, sn);
        tab[pr * kWave + lane] = f32x2{c, sn};
      }
    }
    cs_tab = tab;
  }
  if (active && qi < a.Nq) {
    bf16* dqrow = static_cast<bf16*>(a.dq) + (head + qi) * D;
    const bool has_max = amax < a.Nk;
    const bf16* krow = kg + (size_t)(has_max ? amax : 0) * D;
    const float radd = has_max ? R : 0.0f;
    if constexpr (ROPE) {
      float kv[DB][4][4];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
          for (int e = 0; e < 4; ++e) kv[db][r4][e] = (float)krow[db * 32 + 8 * r4 + 4 * (lane >> 5) + e];
      store_row_unrotated<bf16, D>(dqrow, acc, a.scale, kv, radd,
                             [&](int pr, int) { return cs_tab[pr * kWave + lane]; }, lane);
    } else {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = db * 32 + 8 * r4 + 4 * (lane >> 5);
          float kv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) kv[e] = (float)krow[d0 + e];
          store_quad_scaled<bf16>(dqrow + d0, acc[db], 4 * r4, a.scale, kv, radd);
        }
    }
    if (lane < 32) {
      a.c[head + qi] = cval;
      a.r[head + qi] = R;
      a.amax[head + qi] = has_max ? amax : -1;
      a.kd[head + qi] = m == -INFINITY ? INFINITY : fmaf(m, a.c16, 1.0f);
      a.il[head + qi] = il;
      a.cil[head + qi] = cil;
    }
  }
}

// bf16 dK/dV: eight waves, two per SIMD.  The workgroup owns 128 keys whose K and V rows stay in
// LDS; waves w and w+4 own the same 32 keys and split each 64-row query tile: the upper half
// (waves 0-3) takes rows 0-31, the lower half (waves 4-7) rows 32-63.  Each keeps its own
// dK^T/dV^T partial sums, added through LDS at the end (fixed order: deterministic).
//
// A step of a wave has three phases: products S, dP (MFMA), the phi-derivative arithmetic
// (VALU), products dV, dK (MFMA).  The lower half runs one phase behind the upper one: in step t
// it finishes tile t-1 (arithmetic, then dV/dK) and then forms S, dP of tile t, which it keeps in
// registers across the barrier.  The two waves of a SIMD are then in different phases most of
// the step, so one's vector work runs under the other's matrix products.  Each half has its own
// loop (the half is fixed per wave), and both take steps + 1 barriers.
//
// LDS: K, V rows; the upper half-tiles (Q and dO rows 0-31) in two slots (tile t, t+1); the lower
// half-tiles in three (t-1, t, t+1); the per-row terms of a tile in three.  Tile t+1 is fetched
// by LDS DMA during step t, issued by the upper half after its own products.
constexpr int kDkdvWaves = 8;
constexpr int kDkdvThreads = kDkdvWaves * kWave;
constexpr int kDkdvRows = 64;   // query rows per step (32 per half of the workgroup)

// KEYPAD (with MASKED false): a boolean mask that depends on the key only (key padding).  A lane
// owns one key for the whole kernel, so the mask is one keep flag per lane, read once; the
// kernel keeps the unmasked paths, and a wave whose keys are all padding computes nothing.
template <int D, bool CAUSAL, bool MASKED, bool KEYPAD = false, bool ROPE = false>
__global__ __launch_bounds__(kDkdvThreads) void attn_bwd_dkdv_bf16_kernel(BwdArgs a) {
  constexpr int KC = D / 16, DB = D / 32, QT = kDkdvRows, HR = QT / 2, NW = kDkdvWaves;
  constexpr int HTILE = HR * D;           // elements of one half-tile (32 rows of Q or dO)
  constexpr int KV = kKeysPerWg * D;      // elements of the K (or V) rows
  // K | V | Q_up[2] | dO_up[2] | Q_lo[3] | dO_lo[3]; after the loop the same bytes hold the
  // partial sums
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * KV + 10 * HTILE];
  static_assert(4 * 2 * DB * 16 * kWave * sizeof(float) <= sizeof(bf16) * (2 * KV + 10 * HTILE),
                "partial sums must fit in the tile buffers");
  // per-row terms of a tile [slot][term][row]: 1 + c16*m, 1/l, c/l, R, argmax (int bits)
  __shared__ __attribute__((aligned(16))) float st_lds[3][5][QT];
  __shared__ double rate_lds[ROPE ? D / 2 : 1];   // ROPE: theta^(-2j/D) per pair j
  if constexpr (ROPE) {
    if (threadIdx.x < D / 2) rate_lds[threadIdx.x] = rope_rate(threadIdx.x, D, a.log2_theta);
    __syncthreads();
  }
  bf16* const k_lds = smem;
  bf16* const v_lds = smem + KV;
  auto q_up = [&](int slot) { return smem + 2 * KV + slot * HTILE; };
  auto do_up = [&](int slot) { return smem + 2 * KV + (2 + slot) * HTILE; };
  auto q_lo = [&](int slot) { return smem + 2 * KV + (4 + slot) * HTILE; };
  auto do_lo = [&](int slot) { return smem + 2 * KV + (7 + slot) * HTILE; };

  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int kg = wave & 3, half = wave >> 2;
  const int logical = xcd_remap(blockIdx.x, a.total_kwg);
  const int bg = logical / a.kwg_per_group;
  const int kb = logical % a.kwg_per_group;   // low key blocks (most causal work) first
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int key0_wg = kb * kKeysPerWg;
  const int j0 = key0_wg + kg * kRowsPerWave;
  const bool active = j0 < a.Nk;
  const int frow = lane & 31, fcol = 8 * (lane >> 5);
  const int key = j0 + frow;
  const int kr = 32 * kg + frow;     // B-fragment row of this lane inside the K/V rows

  const int nqt = (a.Nq + QT - 1) / QT;
  const int qt0 = CAUSAL ? min(max(key0_wg - a.coff, 0) / QT, nqt) : 0;
  const int per_head = nqt - qt0;
  const int steps = a.rep * per_head;
  const bf16* qbase = static_cast<const bf16*>(a.q);
  const bf16* dobase = static_cast<const bf16*>(a.d_o);
  static_assert(QT == kWave, "one row term per lane of a DMA instruction");

  // Step -> (query head hh of the group, query tile qt, slot of the three-slot buffers), advanced
  // one step at a time: the steps walk the tiles qt0 .. nqt-1 of each head in turn.  Scalar
  // divisions and pointer conversions per step cost more than they seem: a wave issues at most
  // one instruction every four cycles.
  struct Cursor {
    int hh, qt, slot3;
  };
  auto advance = [&](Cursor c) {
    c.slot3 = c.slot3 == 2 ? 0 : c.slot3 + 1;
    if (++c.qt == nqt) {
      c.qt = qt0;
      ++c.hh;
    }
    return c;
  };
  auto head_row = [&](const Cursor& c) { return (b * a.Hq + g * a.rep + c.hh) * a.Nq; };
  // Q/dO half-tiles and the tile's per-row terms (written by the query-parallel kernel) by LDS
  // DMA, issued by the upper half at the start of the step before the tile is needed; rows past
  // Nq read as zeros, which the masking of those rows makes harmless.  One resource covers the
  // 64 rows of Q (and of dO): the lower half-tile is its second 8 KiB.
  const float* term = kg == 0 ? a.kd : kg == 1 ? a.il : kg == 2 ? a.cil : a.r;
  const unsigned smem_b = lds_addr(smem), st_b = lds_addr(&st_lds[0][0][0]);
  const int tile_lane = dma_lane_offset<D, NW / 2>(kg, lane);
  constexpr int TILE_BLOCKS = dma_blocks_per_wave<D, HR, NW / 2>();
  auto issue = [&](const Cursor& c, int slot2) {
    const int row = head_row(c), i0 = c.qt * QT;
    const int rows = min(a.Nq - i0, QT);
    const u32x4 tr = dma_rsrc(term + row + i0, rows * 4);
    lds_dma_at<4>(tr, st_b + (c.slot3 * 5 + kg) * QT * 4, lane * 4, 0);
    if (kg == 3) lds_dma_at<4>(dma_rsrc(a.amax + row + i0, rows * 4), st_b + (c.slot3 * 5 + 4) * QT * 4, lane * 4, 0);
    const u32x4 qr = dma_rsrc(qbase + (size_t)(row + i0) * D, rows * D * 2);
    const u32x4 dr = dma_rsrc(dobase + (size_t)(row + i0) * D, rows * D * 2);
    const unsigned up = smem_b + (2 * KV + slot2 * HTILE) * 2, lo = smem_b + (2 * KV + (4 + c.slot3) * HTILE) * 2;
#pragma unroll
    for (int i = 0; i < TILE_BLOCKS; ++i) {
      const int blk = (i * (NW / 2) + kg) * 1024, soff = i * (NW / 2) * 1024;
      lds_dma_at<16>(qr, up + blk, tile_lane, soff);
      lds_dma_at<16>(dr, up + 2 * HTILE * 2 + blk, tile_lane, soff);
      lds_dma_at<16>(qr, lo + blk, tile_lane, soff + HR * D * 2);
      lds_dma_at<16>(dr, lo + 3 * HTILE * 2 + blk, tile_lane, soff + HR * D * 2);
    }
  };
  // does this wave's 32 x 32 block of the tile at query row i0 hold any allowed score?
  static_assert(!(KEYPAD && MASKED), "key padding runs the unmasked paths");
  bool key_kept = true, keys_all = true, keys_none = false;
  if constexpr (KEYPAD) {
    const unsigned char* mrow = static_cast<const unsigned char*>(a.mask.ptr) + (size_t)b * a.mask.sb;
    key_kept = active && key < a.Nk && mrow[key] != 0;
    keys_all = !__any(!key_kept);
    keys_none = !__any(key_kept);
  }
  auto block_live = [&](const Cursor& c) {
    const int i0 = c.qt * QT + HR * half;
    return active && !keys_none && i0 < a.Nq && !(CAUSAL && i0 + 31 + a.coff < j0);
  };
  // explicit mask elements of this wave's block (read ahead of the products)
  auto mask_load = [&](const Cursor& c, unsigned (&mv)[16]) {
    if constexpr (MASKED) {
      const MaskSlice<bf16> ms(a.mask, b, g * a.rep + c.hh);
      ms.load_rows(mv, key * ms.sk + (c.qt * QT + HR * half + 4 * (lane >> 5)) * ms.sq, ms.sq);
    }
  };
  // does the mask keep any entry of the wave's block?  A block it empties adds nothing to dK or
  // dV: the lower half skips all of its work, the upper half the work after its S/dP products (a
  // wait before them would also wait for the next tile's copies, which it issues at the start of
  // the step)
  auto mask_keeps_any = [&](const unsigned (&mv)[16]) {
    if constexpr (!MASKED) return true;
    bool any = false;
#pragma unroll
    for (int i = 0; i < 16; ++i) any = any || mask_alive(a.mask.kind, mv[i]);
    return __any(any) != 0;
  };

  // Q/dO half-tiles are addressed from the half's slot-0 Q tile hb: Q of slot t at byte offset
  // qo = t HTB, dO at doo.  The unmasked kernels read them through QdoAddr: the LDS address of
  // every fragment this lane reads from hb, one opaque register each, to which the slot, the matrix
  // and the second 16-row block add immediate offsets (all below 64 KiB).  With the slot in a
  // register instead, each fragment read cost two address instructions per step, and with the
  // slots' absolute addresses as constants (above 64 KiB, too large for an immediate) the
  // compiler kept one register per slot and spilled.
  constexpr unsigned HTB = HTILE * 2;
  struct QdoAddr {
    unsigned row[KC];      // row fragment kc: row frow, 16-byte chunk 2 kc + lane / 32
    unsigned tr[2 * DB];   // transposed fragment db: rows 0-7 [2 db] and 8-15 [2 db + 1]
  };
  auto qdo_addr = [&](const bf16* hb) {
    QdoAddr ad;
    const unsigned b0 = lds_addr(hb);
    const int g4 = lane >> 4, l16 = lane & 15;
    const int trow = 4 * (g4 >> 1) + (l16 >> 2);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      ad.row[kc] = b0 + 2u * swz_off<bf16, D>(frow, 2 * kc + (lane >> 5));
      asm volatile("" : "+v"(ad.row[kc]));
    }
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int col = 32 * db + 16 * (g4 & 1) + 4 * (l16 & 3);
      ad.tr[2 * db] = b0 + 2u * (swz_off<bf16, D>(trow, col >> 3) + (col & 7));
      ad.tr[2 * db + 1] = b0 + 2u * (swz_off<bf16, D>(trow + 8, col >> 3) + (col & 7));
      asm volatile("" : "+v"(ad.tr[2 * db]));
      asm volatile("" : "+v"(ad.tr[2 * db + 1]));
    }
    return ad;
  };
  // the second 16-row block of a transposed read: swz(r + 16) = swz(r), so it is an offset
  static_assert(swz<bf16, D>(5) == swz<bf16, D>(21) && swz<bf16, D>(14) == swz<bf16, D>(30),
                "16-row block offset");

  // S^T and dP^T of this wave's block: lane = key, registers = the half-tile's 32 query rows
  // S and dP run as two independent chains with their four operand reads pinned two products
  // ahead (left alone, the compiler read each operand just before its product, so every product
  // waited out an LDS latency)
  auto products_sdp = [&](const bf16* hb, const QdoAddr& ad, unsigned qo, unsigned doo, f32x16& s, f32x16& dp) {
    s = f32x16{};
    dp = f32x16{};
    if constexpr (MASKED) {   // no registers to spare for the read-ahead
      const bf16* qt_ = hb + qo / 2;
      const bf16* dot_ = hb + doo / 2;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        mma(s, swz_frag<bf16, D>(qt_, frow, 16 * kc + fcol), swz_frag<bf16, D>(k_lds, kr, 16 * kc + fcol));
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        mma(dp, swz_frag<bf16, D>(dot_, frow, 16 * kc + fcol), swz_frag<bf16, D>(v_lds, kr, 16 * kc + fcol));
      return;
    }
    bf16x8 qa[KC], ka[KC], da[KC], va[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      qa[kc] = lds_frag_at(ad.row[kc] + qo);
      ka[kc] = swz_frag<bf16, D>(k_lds, kr, 16 * kc + fcol);
      da[kc] = lds_frag_at(ad.row[kc] + doo);
      va[kc] = swz_frag<bf16, D>(v_lds, kr, 16 * kc + fcol);
    }
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      mma(s, qa[kc], ka[kc]);
      mma(dp, da[kc], va[kc]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int kc = 0; kc < KC - 2; ++kc) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // s -> P, dp -> G (+ R at the argmax) for the half-tile rows starting at query row i0
  auto derivative = [&](f32x16& s, f32x16& dp, const unsigned (&mv)[16], int i0, int slot) {
    const bool edge = MASKED || (CAUSAL && j0 + 31 > i0 + a.coff) || i0 + 32 > a.Nq || j0 + 32 > a.Nk;
    if (edge) {   // one uniform branch around the whole block's masking
      if constexpr (MASKED) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = mask_value(a.mask.kind, a.mask.inv_scale, s[i], mv[i]);
      }
      // query row i0 + 4 (lane >> 5) + r is kept iff r < Nq - i0 - 4 (lane >> 5), key <= row + coff
      // (causal) and key < Nk
      const int lb = 4 * (lane >> 5);
      keep_rows(s, (CAUSAL ? key - a.coff - i0 : -kNoBound) - lb, key >= a.Nk ? -kNoBound : a.Nq - i0 - lb);
    }
    if constexpr (KEYPAD) {
      if (!keys_all) {   // a padded key: its whole column of the block goes
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = key_kept ? s[i] : -INFINITY;
      }
    }
    const float* st = &st_lds[slot][0][HR * half];
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      // one group of four rows at a time: hoisting all groups' row terms costs 48 registers
      __builtin_amdgcn_sched_barrier(0);
      const int r0 = 8 * i4 + 4 * (lane >> 5);   // four consecutive query rows of this lane
      const f32x4 kd4 = *reinterpret_cast<const f32x4*>(st + 0 * QT + r0);
      const f32x4 il4 = *reinterpret_cast<const f32x4*>(st + 1 * QT + r0);
      const f32x4 cil4 = *reinterpret_cast<const f32x4*>(st + 2 * QT + r0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * i4 + e;
        float p;
        const float gv = ra_grad(s[i], a.c16, kd4[e], dp[i], il4[e], cil4[e], &p);
        s[i] = p;
        dp[i] = gv;
      }
    }
    const int am = __float_as_int(st[4 * QT + (lane & 31)]);
    if constexpr (MASKED) {   // no registers to spare for the batched reads below
      if (__any(am >= j0 && am < j0 + 32)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = acc_row(i, lane);
          if (__float_as_int(st[4 * QT + r]) == key) dp[i] += st[3 * QT + r];
        }
      }
    } else if (__any(am >= j0 && am < j0 + 32)) {
      // this lane's 16 rows are four runs of four consecutive rows: eight 16-byte reads issued
      // together (one read and wait per element serialised sixteen LDS latencies)
      f32x4 am4[4], r4[4];
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int r0 = 8 * i4 + 4 * (lane >> 5);
        am4[i4] = *reinterpret_cast<const f32x4*>(st + 4 * QT + r0);
        r4[i4] = *reinterpret_cast<const f32x4*>(st + 3 * QT + r0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (__float_as_int(am4[i >> 2][i & 3]) == key) dp[i] += r4[i >> 2][i & 3];
    }
  };
  f32x16 acc_dk[DB], acc_dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    acc_dk[db] = f32x16{};
    acc_dv[db] = f32x16{};
  }
  // dV^T += dO^T P^T, dK^T += Q^T G^T over the half-tile's 32 rows
  auto products_dkdv = [&](const f32x16& s, const f32x16& dp, const bf16* hb, const QdoAddr& ad, unsigned qo,
                           unsigned doo) {
    if constexpr (MASKED) {
      const bf16* qt_ = hb + qo / 2;
      const bf16* dot_ = hb + doo / 2;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 pf = pack_frag_bf16(s, ks);
        const bf16x8 gf = pack_frag_bf16(dp, ks);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          mma(acc_dv[db], tr_frag<D>(dot_, 16 * ks, db * 32, lane), pf);
          mma(acc_dk[db], tr_frag<D>(qt_, 16 * ks, db * 32, lane), gf);
        }
      }
      return;
    }
    // transposed operand reads (two ds_read_b64_tr_b16 each) pinned two products ahead
    constexpr int NP = 2 * DB;
    bf16x8 pf[2], gf[2], ta[NP], tb[NP];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      pf[ks] = pack_frag_bf16(s, ks);
      gf[ks] = pack_frag_bf16(dp, ks);
    }
#pragma unroll
    for (int c = 0; c < NP; ++c) {
      const unsigned blk = (c / DB) * 16 * D * 2;   // second 16-row block
      const int db = c % DB;
      ta[c] = lds_tr_frag_at(ad.tr[2 * db] + doo + blk, ad.tr[2 * db + 1] + doo + blk);
      tb[c] = lds_tr_frag_at(ad.tr[2 * db] + qo + blk, ad.tr[2 * db + 1] + qo + blk);
    }
#pragma unroll
    for (int c = 0; c < NP; ++c) {
      mma(acc_dv[c % DB], ta[c], pf[c / DB]);
      mma(acc_dk[c % DB], tb[c], gf[c / DB]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int c = 0; c < NP - 2; ++c) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  const size_t kv0 = ((size_t)(b * a.Hkv + g) * a.Nk + key0_wg) * D;
  dma_tile<D, kKeysPerWg, NW>(k_lds, static_cast<const bf16*>(a.k) + kv0, a.Nk - key0_wg, wave, lane);
  dma_tile<D, kKeysPerWg, NW>(v_lds, static_cast<const bf16*>(a.v) + kv0, a.Nk - key0_wg, wave, lane);
  const Cursor first{0, qt0, 0};
  if (steps > 0 && half == 0) issue(first, 0);
  wait_vmem();
  __syncthreads();

  // The unmasked kernels unroll the loops over the slots, so that every slot offset is an
  // immediate; the masked ones keep them rolled (no registers to spare).
  if (half == 0) {
    const bf16* hb = q_up(0);   // Q slots 0, 1, then dO slots 0, 1
    QdoAddr ad{};
    if constexpr (!MASKED) ad = qdo_addr(hb);
    Cursor cur = first, nxt = advance(first);   // steps st and st + 1
    auto up_step = [&](int st, int par) {       // par = st & 1: the Q/dO slot of tile st
      // the next tile's copies go out first: their buffers were last read before the barrier
      // that ended step st - 1, and they have the whole step to land
      if (st + 1 < steps) issue(nxt, par ^ 1);
      if (st < steps && block_live(cur)) {
        f32x16 s, dp;
        unsigned mv[16];
        mask_load(cur, mv);
        products_sdp(hb, ad, par * HTB, (2 + par) * HTB, s, dp);
        if (mask_keeps_any(mv)) {
          derivative(s, dp, mv, cur.qt * QT, cur.slot3);
          products_dkdv(s, dp, hb, ad, par * HTB, (2 + par) * HTB);
        }
      }
      wait_vmem();
      __syncthreads();
      cur = nxt;
      nxt = advance(nxt);
    };
    if constexpr (MASKED) {
      for (int st = 0; st <= steps; ++st) up_step(st, st & 1);
    } else {
      for (int st = 0; st <= steps; st += 2) {
        up_step(st, 0);
        if (st + 1 <= steps) up_step(st + 1, 1);
      }
    }
  } else {
    const bf16* hb = q_lo(0);   // Q slots 0-2, then dO slots 0-2
    QdoAddr ad{};
    if constexpr (!MASKED) ad = qdo_addr(hb);
    f32x16 s = {}, dp = {};
    unsigned mv[16];
    bool carried = false;   // s, dp (and mv) hold S, dP (and the mask block) of tile st - 1
    Cursor prev = first, cur = first;
    auto lo_step = [&](int st, int sp, int sc) {   // sp, sc: slots of tiles st - 1 and st
      if (carried) {
        derivative(s, dp, mv, prev.qt * QT + HR, sp);
        products_dkdv(s, dp, hb, ad, sp * HTB, (3 + sp) * HTB);
      }
      carried = st < steps && block_live(cur);
      if (carried) {
        mask_load(cur, mv);
        carried = mask_keeps_any(mv);
        if (carried) products_sdp(hb, ad, sc * HTB, (3 + sc) * HTB, s, dp);
      }
      wait_vmem();
      __syncthreads();
      prev = cur;
      cur = advance(cur);
    };
    if constexpr (MASKED) {
      for (int st = 0; st <= steps; ++st) lo_step(st, prev.slot3, cur.slot3);
    } else {   // tile st sits in slot st % 3
      for (int st = 0; st <= steps; st += 3) {
        lo_step(st, 2, 0);
        if (st + 1 > steps) break;
        lo_step(st + 1, 0, 1);
        if (st + 2 > steps) break;
        lo_step(st + 2, 1, 2);
      }
    }
  }

  // the lower half hands its partial sums to the upper half through LDS ([kg][dk|dv][db][i4][lane]
  // float4, 1 KiB per store instruction); every wave has left its loop behind a barrier
  f32x4* part = reinterpret_cast<f32x4*>(smem);
  auto slot = [&](int which, int db, int i4) { return ((((kg * 2 + which) * DB + db) * 4 + i4) * kWave) + lane; };
  if (half == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        part[slot(0, db, i4)] = f32x4{acc_dk[db][4 * i4], acc_dk[db][4 * i4 + 1], acc_dk[db][4 * i4 + 2], acc_dk[db][4 * i4 + 3]};
        part[slot(1, db, i4)] = f32x4{acc_dv[db][4 * i4], acc_dv[db][4 * i4 + 1], acc_dv[db][4 * i4 + 2], acc_dv[db][4 * i4 + 3]};
      }
  }
  __syncthreads();
  if (half == 0 && active && key < a.Nk) {
    const size_t kvbase = (size_t)(b * a.Hkv + g) * a.Nk;
    bf16* dkrow = static_cast<bf16*>(a.dk) + (kvbase + key) * D;
    bf16* dvrow = static_cast<bf16*>(a.dv) + (kvbase + key) * D;
    if constexpr (ROPE) {
      float ak[DB][4][4];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 pk = part[slot(0, db, i4)];
#pragma unroll
          for (int e = 0; e < 4; ++e) ak[db][i4][e] = pk[e];
        }
      const double pos = a.k_pos != nullptr ? (double)a.k_pos[key] : (double)key;
      store_row_unrotated<bf16, D>(dkrow, acc_dk, a.scale, ak, 1.0f, [&](int, int j) {
        float c, sn;
        rope_cs(pos, rate_lds[j], true, c, sn);
        return f32x2{c, sn};
      }, lane);
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = db * 32 + 8 * i4 + 4 * (lane >> 5);
        const f32x4 pk = part[slot(0, db, i4)];
        const f32x4 pv = part[slot(1, db, i4)];
        const float ak[4] = {pk[0], pk[1], pk[2], pk[3]};
        const float av[4] = {pv[0], pv[1], pv[2], pv[3]};
        if constexpr (!ROPE) store_quad_scaled<bf16>(dkrow + d0, acc_dk[db], 4 * i4, a.scale, ak, 1.0f);
        store_quad_scaled<bf16>(dvrow + d0, acc_dv[db], 4 * i4, 1.0f, av, 1.0f);
      }
  }
}

template <typename T, int D, int BN>
static hipError_t launch_bwd_typed(const AttnProblem& p, const void* o, const void* d_o,
                                   const float* stats, void* dq, void* dk, void* dv,
                                   const BwdWorkspace& ws, int phases, hipStream_t stream) {
  BwdArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.o = o;
  a.d_o = d_o;
  a.stats = stats;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.c = ws.c;
  a.r = ws.r;
  a.amax = ws.amax;
  a.kd = ws.kd;
  a.il = ws.il;
  a.cil = ws.cil;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.Nq = p.Nq;
  a.Nk = p.Nk;
  a.rep = p.Hq / p.Hkv;
  a.tasks_per_group = a.rep * ((p.Nq + kRowsPerWave - 1) / kRowsPerWave);
  a.wg_per_group = (a.tasks_per_group + kWaves - 1) / kWaves;
  a.total_wg = p.B * p.Hkv * a.wg_per_group;
  a.kwg_per_group = (p.Nk + kKeysPerWg - 1) / kKeysPerWg;
  a.total_kwg = p.B * p.Hkv * a.kwg_per_group;
  a.scale = p.scale;
  a.c16 = p.scale / 16.0f;
  a.coff = p.coff;
  a.mask = mask_args(p);
  a.q_pos = p.q_pos;
  a.k_pos = p.k_pos;
  a.log2_theta = p.rope ? log2(p.rope_theta) : 0.0;
  constexpr bool kBf16 = sizeof(T) == 2;
  const dim3 qgrid(a.total_wg), kgrid(a.total_kwg), block(kThreads);
  const dim3 kblock(kBf16 ? kDkdvThreads : kThreads);
  // the masked kernels are the causal ones (coff = Nk when there is no causality)
  const bool masked = p.mask_kind != kMaskNone;
  const bool madd = kBf16 && p.mask_kind == kMaskAdd && a.mask.packed;   // the packed additive dQ
  // a boolean key padding mask ([B, Nk] broadcast over heads and rows, keys contiguous, every
  // sample's row 4-byte aligned and a whole number of dwords long for the dword copies, whose
  // resource ends at Nk bytes): the unmasked kernels with keep bits
  const bool keypad = kBf16 && p.mask_kind == kMaskBool && p.msq == 0 && p.msh == 0 && p.msk == 1 &&
                      p.msb % 4 == 0 && p.Nk % 4 == 0 &&
                      reinterpret_cast<unsigned long long>(p.mask) % 4 == 0;
  if (p.rope) {   // the same kernel choice as below, each with the epilogue turn
    if (phases & kBwdDq) {
      if constexpr (kBf16) {
        if (keypad) hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, true, false, true, true>), qgrid, block, 0, stream, a);
        else if (madd) hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, true, true, false, true, true>), qgrid, block, 0, stream, a);
        else if (masked) hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, true, true, false, true>), qgrid, block, 0, stream, a);
        else if (p.causal) hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, true, false, false, true>), qgrid, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, false, false, false, true>), qgrid, block, 0, stream, a);
      } else {
        if (masked) hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D, BN, true, true, true>), qgrid, block, 0, stream, a);
        else if (p.causal) hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D, BN, true, false, true>), qgrid, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D, BN, false, false, true>), qgrid, block, 0, stream, a);
      }
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (phases & kBwdDkdv) {
      if constexpr (kBf16) {
        if (keypad) hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D, true, false, true, true>), kgrid, kblock, 0, stream, a);
        else if (masked) hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D, true, true, false, true>), kgrid, kblock, 0, stream, a);
        else if (p.causal) hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D, true, false, false, true>), kgrid, kblock, 0, stream, a);
        else hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D, false, false, false, true>), kgrid, kblock, 0, stream, a);
      } else {
        if (masked) hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D, true, true, true>), kgrid, kblock, 0, stream, a);
        else if (p.causal) hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D, true, false, true>), kgrid, kblock, 0, stream, a);
        else hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D, false, false, true>), kgrid, kblock, 0, stream, a);
      }
    }
    return hipGetLastError();
  }
  if (phases & kBwdDq) {
    if (keypad) {
      if constexpr (kBf16) hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, true, false, true>), qgrid, block, 0, stream, a);
    } else if (masked) {
      if constexpr (kBf16) {
        if (madd) hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, true, true, false, false, true>), qgrid, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, true, true>), qgrid, block, 0, stream, a);
      } else {
        hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D, BN, true, true>), qgrid, block, 0, stream, a);
      }
    } else if (p.causal) {
      if constexpr (kBf16) hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, true, false>), qgrid, block, 0, stream, a);
      else hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D, BN, true, false>), qgrid, block, 0, stream, a);
    } else {
      if constexpr (kBf16) hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, false, false>), qgrid, block, 0, stream, a);
      else hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D, BN, false, false>), qgrid, block, 0, stream, a);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & kBwdDkdv) {
    if (keypad) {
      if constexpr (kBf16) hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D, true, false, true>), kgrid, kblock, 0, stream, a);
    } else if (masked) {
      if constexpr (kBf16) hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D, true, true>), kgrid, kblock, 0, stream, a);
      else hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D, true, true>), kgrid, kblock, 0, stream, a);
    } else if (p.causal) {
      if constexpr (kBf16) hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D, true, false>), kgrid, kblock, 0, stream, a);
      else hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D, true, false>), kgrid, kblock, 0, stream, a);
    } else {
      if constexpr (kBf16) hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D, false, false>), kgrid, kblock, 0, stream, a);
      else hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D, false, false>), kgrid, kblock, 0, stream, a);
    }
  }
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const AttnProblem& p, const void* o, const void* d_o,
                           const float* stats, void* dq, void* dk, void* dv,
                           const BwdWorkspace& ws, int phases, hipStream_t stream) {
  if (stats == nullptr) {
    if (phases & kBwdDq) {   // recompute (m, l) with the forward's statistics-only variant
      AttnProblem ps = p;
      ps.rope = false;       // with the rotary embedding q and k already hold the rotated rows
      const hipError_t e = launch_attn_fwd(ps, nullptr, ws.stats, nullptr, stream);
      if (e != hipSuccess) return e;
    }
    stats = ws.stats;
  }
  if (p.bf16) {
    if (p.D == 64) return launch_bwd_typed<bf16, 64, 64>(p, o, d_o, stats, dq, dk, dv, ws, phases, stream);
    return launch_bwd_typed<bf16, 128, 64>(p, o, d_o, stats, dq, dk, dv, ws, phases, stream);
  }
  if (p.D == 64) return launch_bwd_typed<float, 64, 32>(p, o, d_o, stats, dq, dk, dv, ws, phases, stream);
  return launch_bwd_typed<float, 128, 32>(p, o, d_o, stats, dq, dk, dv, ws, phases, stream);
}

}  // namespace ra
