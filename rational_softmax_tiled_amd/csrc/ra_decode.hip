// ra_decode.hip -- split-KV decode for gfx950: a few query rows per head against a long K/V cache.
//
// "Ra-Family: Rational Neural Architecture", section 3 "Rational Attention & Softmax": phi has no
// online rescaling (phi(D + d) is not a multiple of phi(D)), so partial results over key ranges
// cannot be merged the way exp-softmax partials are; every phi needs the final row max.  Split
// over the keys, the computation therefore takes two synchronisation points, one after the max
// and one after the sums, which here are kernel boundaries on one stream:
//   1. scores: each wave owns one chunk of keys of one (batch, K/V head) group, computes the raw
//      dot products of the group's R = rep * Nq query rows with them (MFMA; K rows loaded
//      coalesced into registers, then staged through the wave's LDS tile), stores them in the
//      wave's lane layout and writes the chunk's row maxima;
//   2. phi and P.V: each wave takes the row max over all chunks of its group, evaluates phi on
//      its stored scores, sums it and accumulates P.V (V staged through LDS, read transposed),
//      and writes the unnormalised partial output and partial sum of phi;
//   3. combine: per query row, sum the partials of the chunks in a fixed order and divide.
// K and V are each read from HBM once; the scores (R x 4 bytes per key) and partials are small
// beside them.  Decode is memory-bound: a wave's 32 query columns are padded past R, and that
// idle matrix-core and vector work hides under the K/V streams.
// bf16 and fp32 share the split and the first and last kernels; the fp32 scores take fp32
// products (eight 32x32x2 per 16 columns) with twice the bytes per block, so their register ring
// holds two blocks instead of three, and the fp32 P.V reads V straight into the product's
// operand layout (below) instead of through LDS.
#include <type_traits>

#include "ra_device.h"
#include "ra_internal.h"

namespace ra {

struct DecodeArgs {
  const void* q;        // [B, Hq, Nq, D] of the attention dtype, as k, v and o
  const void* k;
  const void* v;
  void* o;
  float* stats;
  const int* seqlens;   // [B] cache lengths (nullptr: all Nk)
  float* scores;        // [groups][nk32 / 32][R][2][16] raw dot products, by 32-key block
  float* pmax;          // [groups][S][R] row max of a chunk
  float* psum;          // [groups][S][R] sum of phi of a chunk
  float* pacc;          // [groups][S][R][D] unnormalised P.V of a chunk
  float* gmax;          // [groups][R] row max over all chunks (written by chunk 0's wave)
  int B, Hq, Hkv, Nq, Nk, rep, R;
  int nk32;             // Nk rounded up to 32: the keys of a group in the scores
  int chunk_min, chunk_max;   // bounds of the keys per wave, multiples of 32
  int S;                // partial-result slots per group: ceil(Nk / chunk_min)
  int waves;            // waves launched
  int causal;           // 0 none, 1 top-left, 2 bottom-right (per sample)
  float c;              // scale / 16
};

__device__ __forceinline__ int cache_len(const DecodeArgs& a, int b) {
  return a.seqlens != nullptr ? min(max(a.seqlens[b], 0), a.Nk) : a.Nk;
}

// The last key query row r (head-major: r = hq * Nq + i) may see in a cache of length len.
__device__ __forceinline__ int key_limit(const DecodeArgs& a, int len, int r) {
  const int i = r % a.Nq;
  int lim = len - 1;
  if (a.causal == 1) lim = min(lim, i);
  else if (a.causal == 2) lim = min(lim, i + len - a.Nq);
  return lim;
}

// The work split of the step over the actual cache lengths, the same in every wave and in the
// combine: every wave takes `chunk` consecutive keys of one (batch, K/V head) group.  Groups are
// numbered bg = b Hkv + g; the chunks of all groups are numbered in that order, and wave v takes
// chunk v.  The launch has W = groups ceil(Nk / chunk_max) waves, the count that full caches
// need.  With shorter caches the chunk shrinks to total / (W - groups) keys (rounded up to 32,
// at least chunk_min), so the chunks still number at most total / chunk + groups <= W and
// every wave has about the same number of keys: no SIMD idles while others stream twice the
// keys.
// Cache policy of the K and V loads: nontemporal (the aux bit of the buffer load), since every
// cache row is read once; measured 8% faster on the step than cached loads.
constexpr int kStreamOnce = 2;
constexpr int kDecodeTarget = 1024;
// chunk size from the total number of keys
__device__ __forceinline__ int decode_chunk_of(const DecodeArgs& a, long long total) {
  const long long spare = (long long)a.waves - (long long)a.B * a.Hkv;
  if (spare <= 0) return a.chunk_max;   // one chunk per group already
  long long c = (total + spare - 1) / spare;
  c = (c + 31) / 32 * 32;
  c = c < a.chunk_min ? a.chunk_min : (c > a.chunk_max ? a.chunk_max : c);
  return uniform((int)c);
}
__device__ __forceinline__ int wave_sum_int(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ int decode_chunk(const DecodeArgs& a) {
  const int lane = threadIdx.x & 63;
  long long total = 0;
  for (int b0 = 0; b0 < a.B; b0 += kWave) {
    const int b = b0 + lane;
    total += wave_sum_int(b < a.B ? cache_len(a, b) : 0);
  }
  return decode_chunk_of(a, total * a.Hkv);
}
// A pointer the same in every lane, rebuilt from its first lane so that the compiler keeps buffer
// resources made from it in scalar registers (no per-load waterfall loop).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const unsigned long long x = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)x);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(x >> 32));
  return reinterpret_cast<T*>(((unsigned long long)hi << 32) | lo);
}
struct DecodeWork {
  int chunk;
  int bg, s;      // group and chunk; bg < 0: no work for this wave
  int len;        // the group's cache length
};
// The chunk of wave v among one window of batches (lane l holds len_l, the cache length of
// batch b0 + l), whose chunks start at `base`; false when it lies past the window.
__device__ __forceinline__ bool decode_find(const DecodeArgs& a, int chunk, int v, int b0, int len_l,
                                            int& base, DecodeWork& w) {
  const int lane = threadIdx.x & 63;
  const int per = (len_l + chunk - 1) / chunk;   // chunks per group of batch b0 + lane
  int incl = per * a.Hkv;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  const int tot = __shfl(incl, kWave - 1);
  if (v >= base + tot) {
    base += tot;
    return false;
  }
  // the first batch whose chunks end past v
  const int hit = __builtin_ctzll(__ballot(base + incl > v));
  const int per_h = __shfl(per, hit);
  const int local = v - (base + __shfl(incl, hit) - per_h * a.Hkv);
  w.chunk = chunk;
  w.bg = uniform((b0 + hit) * a.Hkv + local / per_h);
  w.s = uniform(local % per_h);
  w.len = uniform(__shfl(len_l, hit));
  return true;
}
__device__ __forceinline__ DecodeWork decode_work(const DecodeArgs& a, int v) {
  const int lane = threadIdx.x & 63;
  DecodeWork w{0, -1, 0, 0};
  int base = 0;
  if (a.B <= kWave) {   // one load of the lengths serves both the size and the search
    const int len_l = lane < a.B ? cache_len(a, lane) : 0;
    w.chunk = decode_chunk_of(a, (long long)wave_sum_int(len_l) * a.Hkv);
    decode_find(a, w.chunk, v, 0, len_l, base, w);
    return w;
  }
  w.chunk = decode_chunk(a);
  for (int b0 = 0; b0 < a.B; b0 += kWave) {
    const int b = b0 + lane;
    if (decode_find(a, w.chunk, v, b0, b < a.B ? cache_len(a, b) : 0, base, w)) break;
  }
  return w;
}

// Blocks of 32 keys stream through a ring of three register sets, two blocks ahead of the math:
// the data in flight per CU is then bounded by the register file, not by LDS.
// step(slot, t): compute block t, held in ring slot t % 3 (slot is a compile-time constant, so
// the ring stays in registers); before that it loads block t + 2 into the slot block t - 1 used.
// Every load and store of the loop is issued unconditionally, through buffer resources that end
// at the chunk (loads past the end read zeros, stores past it are dropped), so the compiler can
// count the two newer blocks as still in flight when it waits for the oldest.
template <typename F>
__device__ __forceinline__ void ring3(int nb, F&& step) {
  for (int t = 0; t < nb; t += 3) {
    step(std::integral_constant<int, 0>{}, t);
    if (t + 1 >= nb) break;
    step(std::integral_constant<int, 1>{}, t + 1);
    if (t + 2 >= nb) break;
    step(std::integral_constant<int, 2>{}, t + 2);
  }
}
// The same with two register sets, one block ahead (fp32: a block is twice the bytes, so the
// data in flight per wave stays that of the bf16 ring).
template <typename F>
__device__ __forceinline__ void ring2(int nb, F&& step) {
  for (int t = 0; t < nb; t += 2) {
    step(std::integral_constant<int, 0>{}, t);
    if (t + 1 >= nb) break;
    step(std::integral_constant<int, 1>{}, t + 1);
  }
}

template <typename T, int D>
__device__ __forceinline__ void decode_scores(const DecodeArgs& a) {
  constexpr int KC = D / 16;
  constexpr int CPR = D * (int)sizeof(T) / 16, PER = 32 * CPR / kWave;
  // register ring slots: bf16 three, two blocks ahead of the math; fp32 (a block is twice the
  // bytes, and the Q fragments take 64 registers at D = 128) one, refilled with the next block as
  // soon as this one is in LDS, so one block is in flight under the products
  constexpr int NS = sizeof(T) == 2 ? 3 : 1;
  __shared__ __attribute__((aligned(16))) T k_lds[kWaves][32 * D];
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const DecodeWork work = decode_work(a, blockIdx.x * kWaves + wave);
  if (work.bg < 0) return;   // whole wave: no barrier in this kernel
  const int chunk = uniform(work.chunk), bg = uniform(work.bg), s = uniform(work.s), len = uniform(work.len);
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int k0 = s * chunk;
  const int nkeys = min(chunk, len - k0), nb = (nkeys + 31) / 32;

  // B operand: query row r = lane % 32 of the group (rows past R repeat the last one)
  const int r = lane & 31, rr = min(r, a.R - 1);
  const int h = g * a.rep + rr / a.Nq;
  const T* qrow = static_cast<const T*>(a.q) + ((size_t)(b * a.Hq + h) * a.Nq + rr % a.Nq) * D;
  const int fcol = 8 * (lane >> 5);
  typename Ty<T>::frag qf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) qf[kc] = load_frag(qrow + 16 * kc + fcol);
  const int lim = key_limit(a, len, rr);

  // K rows: coalesced 16-byte loads into the register ring (lane l takes chunks l, l + 64, ... of
  // a block; rows past the chunk's keys read as zeros), stored swizzled into this wave's LDS
  // tile, from which the A fragments are read (the previous block's reads have returned: their
  // results fed the products, and a wave's LDS operations execute in order)
  const __amdgpu_buffer_rsrc_t kr =
      tile_rsrc(uniform_ptr(static_cast<const T*>(a.k) + ((size_t)bg * a.Nk + k0) * D), nkeys, D);
  u32x4 ring[NS][PER];
  auto load = [&](int slot, int t) {
#pragma unroll
    for (int j = 0; j < PER; ++j)
      ring[slot][j] = __builtin_amdgcn_raw_buffer_load_b128(kr, (j * kWave + lane) * 16,
                                                            uniform(t * 32 * D * (int)sizeof(T)), kStreamOnce);
  };
  T* ktile = k_lds[wave];
  // this chunk's scores, [block][R rows][2 lane halves][16]; padded rows store past the end
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(a.scores + ((size_t)bg * a.nk32 + k0) * a.R), (short)0, uniform(nb * 32 * a.R * 4), kBufferWord3);
  const int s_off = r < a.R ? (r * 2 + (lane >> 5)) * 64 : 0x40000000;
  float mx = -INFINITY;
  auto step = [&](auto slot_c, int t) {
    constexpr int slot = decltype(slot_c)::value;
    if constexpr (NS > 1) load((slot + NS - 1) % NS, t + NS - 1);
    // S^T = K Q^T: keys on the accumulator rows, query row r on the lane
    f32x16 sacc = {};
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int c = j * kWave + lane, row = c / CPR, cc = c % CPR;
      *reinterpret_cast<u32x4*>(ktile + swz_off<T, D>(row, cc)) = ring[slot][j];
    }
    if constexpr (NS == 1) load(0, t + 1);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) mma(sacc, swz_frag<T, D>(ktile, lane & 31, 16 * kc + fcol), qf[kc]);
    // key k0 + 32 t + 4 (lane >> 5) + row offset is kept iff it is <= lim (which is < len)
    keep_rows(sacc, -kNoBound, lim + 1 - (k0 + 32 * t + 4 * (lane >> 5)));
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(u32x4, f32x4{sacc[4 * q4], sacc[4 * q4 + 1], sacc[4 * q4 + 2], sacc[4 * q4 + 3]}),
          sr, s_off + 16 * q4, uniform(t * 32 * a.R * 4), 0);
  };
#pragma unroll
  for (int t = 0; t < (NS > 1 ? NS - 1 : 1); ++t) load(t, t);
  if constexpr (NS == 3) ring3(nb, step);
  else for (int t = 0; t < nb; ++t) step(std::integral_constant<int, 0>{}, t);
  mx = fmaxf(mx, __shfl_xor(mx, 32));   // lanes l and l + 32 hold the same row
  if (lane < a.R) a.pmax[((size_t)bg * a.S + s) * a.R + lane] = mx;
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_scores_kernel(DecodeArgs a) {
  decode_scores<bf16, D>(a);
}
// fp32: the Q fragments take 64 registers at D = 128 and each ring slot 64 more
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_scores_f32_kernel(DecodeArgs a) {
  decode_scores<float, D>(a);
}

// The row max of query row r (lanes r and r + 32) over every chunk of the group that holds keys:
// the two lanes take the even and odd chunks, eight loads in flight per round.  The wave of
// chunk 0 records it for the stats.
__device__ __forceinline__ float decode_row_max(const DecodeArgs& a, int bg, int s, int nlive, int lane, bool live) {
  float m = -INFINITY;
  if (live) {
    const float* pm = a.pmax + (size_t)bg * a.S * a.R + (lane & 31);
    for (int s2 = lane >> 5; s2 < nlive; s2 += 16) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = s2 + 2 * j < nlive ? pm[(size_t)(s2 + 2 * j) * a.R] : -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, x[j]);
    }
  }
  m = fmaxf(m, __shfl_xor(m, 32));
  if (s == 0 && lane < a.R) a.gmax[(size_t)bg * a.R + lane] = m;
  return m;
}

// A chunk's scores as the first kernel stored them, block by block, in its lane layout; padded
// rows and blocks past the chunk read zeros.
struct ChunkScores {
  __amdgpu_buffer_rsrc_t sr;
  int s_off, stride;
  __device__ __forceinline__ ChunkScores(const DecodeArgs& a, int bg, int k0, int nb, int lane, bool live) {
    sr = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(a.scores + ((size_t)bg * a.nk32 + k0) * a.R), (short)0,
                                           uniform(nb * 32 * a.R * 4), kBufferWord3);
    s_off = live ? ((lane & 31) * 2 + (lane >> 5)) * 64 : 0x40000000;
    stride = 32 * a.R * 4;
  }
  __device__ __forceinline__ f32x16 load(int t) const {
    f32x16 v;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 x = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, s_off + 16 * q4, uniform(t * stride), 0));
      v[4 * q4] = x[0];
      v[4 * q4 + 1] = x[1];
      v[4 * q4 + 2] = x[2];
      v[4 * q4 + 3] = x[3];
    }
    return v;
  }
};

template <int D>
__device__ __forceinline__ void decode_pv_bf16(const DecodeArgs& a) {
  constexpr int DB = D / 32, TILE = 32 * D;
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int PER = 32 * CPR / kWave;   // chunks of a 32-row tile per lane
  __shared__ __attribute__((aligned(16))) bf16 v_lds[kWaves][TILE];

  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const DecodeWork work = decode_work(a, blockIdx.x * kWaves + wave);
  if (work.bg < 0) return;
  const int chunk = uniform(work.chunk), bg = uniform(work.bg), s = uniform(work.s), len = uniform(work.len);
  const int k0 = s * chunk;
  const int nkeys = min(chunk, len - k0), nb = (nkeys + 31) / 32;
  const int r = lane & 31;
  const bool live = r < a.R;

  // V rows: coalesced 16-byte loads into a register ring (lane l takes chunks l, l + 64, ... of
  // a block), then stored swizzled into this wave's LDS tile and read transposed
  const __amdgpu_buffer_rsrc_t vr =
      tile_rsrc(uniform_ptr(static_cast<const bf16*>(a.v) + ((size_t)bg * a.Nk + k0) * D), nkeys, D);
  u32x4 ring[3][PER];
  auto load = [&](int slot, int t) {
#pragma unroll
    for (int j = 0; j < PER; ++j)
      ring[slot][j] = __builtin_amdgcn_raw_buffer_load_b128(vr, (j * kWave + lane) * 16, uniform(t * 32 * D * 2), kStreamOnce);
  };
  bf16* tile = v_lds[wave];
  load(0, 0);
  load(1, 1);

  const float m = decode_row_max(a, bg, s, (len + chunk - 1) / chunk, lane, live);
  // 1 + u = fma(s, -c, kd); a row with no allowed key (m = -inf) takes kd = +inf: phi = 0
  const float kd = m == -INFINITY ? INFINITY : fmaf(m, a.c, 1.0f);

  const ChunkScores sc(a, bg, k0, nb, lane, live);
  f32x16 sv = sc.load(0);
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float lsum = 0.0f;
  ring3(nb, [&](auto slot_c, int t) {
    constexpr int slot = decltype(slot_c)::value;
    load((slot + 2) % 3, t + 2);
    const f32x16 sn = sc.load(t + 1);
    // this wave's LDS tile takes block t (the previous block's transposed reads have returned:
    // their results fed the products; a wave's LDS operations execute in order)
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int c = j * kWave + lane, row = c / CPR, cc = c % CPR;
      *reinterpret_cast<u32x4*>(tile + swz_off<bf16, D>(row, cc)) = ring[slot][j];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int i = 0; i < 16; ++i) sv[i] = ra_phi(sv[i], a.c, kd);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 pf = pack_frag_bf16(sv, ks);
      // the sum of phi is taken over the rounded values that enter the product
#pragma unroll
      for (int j = 0; j < 8; j += 2)
        lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pf[j], pf[j + 1]}, bf16x2{(bf16)1.0f, (bf16)1.0f}, lsum, false);
#pragma unroll
      for (int db = 0; db < DB; ++db) mma(oacc[db], tr_frag<D>(tile, 16 * ks, 32 * db, lane), pf);
    }
    sv = sn;
  });
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (!live) return;
  const size_t row = ((size_t)bg * a.S + s) * a.R + r;
  if (lane < 32) a.psum[row] = ltot;
  float* dst = a.pacc + row * D;
  // O^T block db: lane (row r) holds d = 32 db + 8 (i / 4) + 4 (lane / 32) + i % 4
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * q4 + 4 * (lane >> 5)) =
          f32x4{oacc[db][4 * q4], oacc[db][4 * q4 + 1], oacc[db][4 * q4 + 2], oacc[db][4 * q4 + 3]};
}

// fp32 P.V as O = P V (fp32 products): the A operand is P as phi leaves it (lane (r, h) holds
// keys 16 ks + 8 (j / 4) + 4 h + j % 4 of row r in element 8 ks + j), and the B operand V is read
// from HBM straight into that layout: lane (n, h) loads, for each of those 16 keys, the D / 32
// consecutive values at columns (D / 32) n ...; product block db takes column (D / 32) n + db on
// lane n.  One 16-byte (D = 128) or 8-byte (D = 64) load per key serves every column block, and
// the 32 lanes of a half read a key's whole row.
template <int D>
__device__ __forceinline__ void decode_pv_f32(const DecodeArgs& a) {
  constexpr int DB = D / 32;
  static_assert(DB == 2 || DB == 4, "D = 64 or 128");
  using vec = std::conditional_t<DB == 4, f32x4, f32x2>;

  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const DecodeWork work = decode_work(a, blockIdx.x * kWaves + wave);
  if (work.bg < 0) return;
  const int chunk = uniform(work.chunk), bg = uniform(work.bg), s = uniform(work.s), len = uniform(work.len);
  const int k0 = s * chunk;
  const int nkeys = min(chunk, len - k0), nb = (nkeys + 31) / 32;
  const bool live = (lane & 31) < a.R;

  // keys past the chunk read zeros (and meet phi = 0)
  const __amdgpu_buffer_rsrc_t vr =
      tile_rsrc(uniform_ptr(static_cast<const float*>(a.v) + ((size_t)bg * a.Nk + k0) * D), nkeys, D);
  const int voff = (4 * (lane >> 5) * D + DB * (lane & 31)) * 4;
  vec ring[2][16];
  auto load = [&](int slot, int t) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = 16 * (e >> 3) + 8 * ((e & 7) >> 2) + (e & 3);
      if constexpr (DB == 4)
        ring[slot][e] = __builtin_bit_cast(vec, __builtin_amdgcn_raw_buffer_load_b128(vr, voff, uniform(t * 32 * D * 4) + key * D * 4, kStreamOnce));
      else
        ring[slot][e] = __builtin_bit_cast(vec, __builtin_amdgcn_raw_buffer_load_b64(vr, voff, uniform(t * 32 * D * 4) + key * D * 4, kStreamOnce));
    }
  };
  load(0, 0);

  const float m = decode_row_max(a, bg, s, (len + chunk - 1) / chunk, lane, live);
  const float kd = m == -INFINITY ? INFINITY : fmaf(m, a.c, 1.0f);

  const ChunkScores sc(a, bg, k0, nb, lane, live);
  f32x16 sv = sc.load(0);
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float lsum = 0.0f;
  ring2(nb, [&](auto slot_c, int t) {
    constexpr int slot = decltype(slot_c)::value;
    load(slot ^ 1, t + 1);
    const f32x16 sn = sc.load(t + 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sv[i] = ra_phi(sv[i], a.c, kd);
      lsum += sv[i];
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const f32x8 pf = pack_frag_f32(sv, ks);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x8 vf;
#pragma unroll
        for (int j = 0; j < 8; ++j) vf[j] = ring[slot][8 * ks + j][db];
        mma(oacc[db], pf, vf);
      }
    }
    sv = sn;
  });
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const size_t row0 = ((size_t)bg * a.S + s) * a.R;
  if (lane < a.R) a.psum[row0 + lane] = ltot;
  // O block db: lane (n, h) holds rows acc_row(i, lane) of column (D / 32) n + db
  float* dst = a.pacc + row0 * D + DB * (lane & 31);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = acc_row(i, lane);
    vec x;
#pragma unroll
    for (int db = 0; db < DB; ++db) x[db] = oacc[db][i];
    if (r < a.R) *reinterpret_cast<vec*>(dst + (size_t)r * D) = x;
  }
}

// ---- fp32 with at most 16 query rows per K/V head: 16x16x4 fp32 products, half the matrix cycles
// of the 32-column form per key.  Product layout (16x16x4): lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; it holds D[4 (l / 16) + v][l % 16], v = 0..3.
//
// Scores S^T = K Q^T per 16-key half sb of a 32-key block: lane (i, g) = (l % 16, l / 16) feeds
// key 16 sb + i, columns (D / 4) g + kc, kc = 0..D/4-1 (one product per kc), so each lane reads
// a contiguous quarter of its key's row from LDS, and Q row l % 16 the same quarter from
// registers.  Lane (r, g) then holds the scores of row r for keys 16 sb + 4 g + v: eight values
// per block, stored in that order ([block][R rows][4 groups][8]).
template <int D>
__device__ __forceinline__ void decode_scores_f32_16(const DecodeArgs& a) {
  constexpr int DQ = D / 4;                      // contraction columns per lane group
  constexpr int CPR = D * 4 / 16, PER = 32 * CPR / kWave;
  __shared__ __attribute__((aligned(16))) float k_lds[kWaves][32 * D];
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const DecodeWork work = decode_work(a, blockIdx.x * kWaves + wave);
  if (work.bg < 0) return;   // whole wave: no barrier in this kernel
  const int chunk = uniform(work.chunk), bg = uniform(work.bg), s = uniform(work.s), len = uniform(work.len);
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int k0 = s * chunk;
  const int nkeys = min(chunk, len - k0), nb = (nkeys + 31) / 32;
  const int r = lane & 15, grp = lane >> 4, rr = min(r, a.R - 1);
  const int h = g * a.rep + rr / a.Nq;
  const float* qrow = static_cast<const float*>(a.q) + ((size_t)(b * a.Hq + h) * a.Nq + rr % a.Nq) * D + DQ * grp;
  float qf[DQ];
#pragma unroll
  for (int c = 0; c < DQ / 4; ++c) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(qrow + 4 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) qf[4 * c + e] = x[e];
  }
  const int lim = key_limit(a, len, rr);

  const __amdgpu_buffer_rsrc_t kr =
      tile_rsrc(uniform_ptr(static_cast<const float*>(a.k) + ((size_t)bg * a.Nk + k0) * D), nkeys, D);
  u32x4 ring[2][PER];
  auto load = [&](int slot, int t) {
#pragma unroll
    for (int j = 0; j < PER; ++j)
      ring[slot][j] = __builtin_amdgcn_raw_buffer_load_b128(kr, (j * kWave + lane) * 16, uniform(t * 32 * D * 4), kStreamOnce);
  };
  float* ktile = k_lds[wave];
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(a.scores + ((size_t)bg * a.nk32 + k0) * a.R), (short)0, uniform(nb * 32 * a.R * 4), kBufferWord3);
  const int s_off = r < a.R ? (r * 4 + grp) * 32 : 0x40000000;
  float mx = -INFINITY;
  load(0, 0);
  ring2(nb, [&](auto slot_c, int t) {
    constexpr int slot = decltype(slot_c)::value;
    load(slot ^ 1, t + 1);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int c = j * kWave + lane, row = c / CPR, cc = c % CPR;
      *reinterpret_cast<u32x4*>(ktile + swz_off<float, D>(row, cc)) = ring[slot][j];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    f32x4 sacc[2] = {};
#pragma unroll
    for (int c = 0; c < DQ / 4; ++c)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(ktile + swz_off<float, D>(16 * sb + r, (DQ / 4) * grp + c));
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sacc[sb] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[e], qf[4 * c + e], sacc[sb], 0, 0, 0);
      }
    // key k0 + 32 t + 16 sb + 4 grp + v is kept iff it is <= lim (which is < len)
    const int room = lim - (k0 + 32 * t + 4 * grp);
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (16 * sb + v > room) sacc[sb][v] = -INFINITY;
        mx = fmaxf(mx, sacc[sb][v]);
      }
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sacc[sb]), sr, s_off + 16 * sb,
                                             uniform(t * 32 * a.R * 4), 0);
  });
  mx = fmaxf(mx, __shfl_xor(mx, 16));   // lanes r, r + 16, r + 32, r + 48 hold the same row
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  if (lane < a.R) a.pmax[((size_t)bg * a.S + s) * a.R + lane] = mx;
}

// P.V as O = P V with 16x16x4 fp32 products: in product kc (0..7) of a block, lane (r, g) feeds
// P[r][key 16 (kc / 4) + 4 g + kc % 4], its own stored score kc after phi, and V[that key]
// [column 4 j + 64 (db / 4) + db % 4] as B on lane (j, g) for product block db: the 16 lanes of
// a group read 256 contiguous bytes of a key's row per load, one or two loads per key serving
// every column block.
template <int D>
__device__ __forceinline__ void decode_pv_f32_16(const DecodeArgs& a) {
  constexpr int DBL = D / 16;                 // column blocks, columns per lane
  constexpr int NL = DBL / 4;                 // 16-byte loads per key
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const DecodeWork work = decode_work(a, blockIdx.x * kWaves + wave);
  if (work.bg < 0) return;
  const int chunk = uniform(work.chunk), bg = uniform(work.bg), s = uniform(work.s), len = uniform(work.len);
  const int k0 = s * chunk;
  const int nkeys = min(chunk, len - k0), nb = (nkeys + 31) / 32;
  const int r = lane & 15, grp = lane >> 4;
  const bool live = r < a.R;

  const __amdgpu_buffer_rsrc_t vr =
      tile_rsrc(uniform_ptr(static_cast<const float*>(a.v) + ((size_t)bg * a.Nk + k0) * D), nkeys, D);
  const int voff = (4 * grp * D + 4 * r) * 4;
  f32x4 ring[2][8][NL];
  auto load = [&](int slot, int t) {
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const int key = 16 * (kc >> 2) + (kc & 3);
#pragma unroll
      for (int n = 0; n < NL; ++n)
        ring[slot][kc][n] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
            vr, voff + 256 * n, uniform(t * 32 * D * 4) + key * D * 4, kStreamOnce));
    }
  };
  load(0, 0);

  // row max over the chunks: the four lanes of row r take chunks r mod 4 apart
  float m = -INFINITY;
  const int nlive = (len + chunk - 1) / chunk;
  if (live) {
    const float* pm = a.pmax + (size_t)bg * a.S * a.R + r;
    for (int s2 = grp; s2 < nlive; s2 += 32) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = s2 + 4 * j < nlive ? pm[(size_t)(s2 + 4 * j) * a.R] : -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) m = fmaxf(m, x[j]);
    }
  }
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  if (s == 0 && lane < a.R) a.gmax[(size_t)bg * a.R + lane] = m;
  const float kd = m == -INFINITY ? INFINITY : fmaf(m, a.c, 1.0f);

  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(a.scores + ((size_t)bg * a.nk32 + k0) * a.R), (short)0, uniform(nb * 32 * a.R * 4), kBufferWord3);
  const int s_off = live ? (r * 4 + grp) * 32 : 0x40000000;
  auto load_scores = [&](int t, f32x4 (&v)[2]) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      v[h2] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, s_off + 16 * h2, uniform(t * 32 * a.R * 4), 0));
  };
  f32x4 sv[2], sn[2];
  load_scores(0, sv);
  f32x4 oacc[DBL];
#pragma unroll
  for (int db = 0; db < DBL; ++db) oacc[db] = f32x4{};
  float lsum = 0.0f;
  ring2(nb, [&](auto slot_c, int t) {
    constexpr int slot = decltype(slot_c)::value;
    load(slot ^ 1, t + 1);
    load_scores(t + 1, sn);
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const float p = ra_phi(sv[kc >> 2][kc & 3], a.c, kd);
      lsum += p;
#pragma unroll
      for (int db = 0; db < DBL; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(p, ring[slot][kc][db >> 2][db & 3], oacc[db], 0, 0, 0);
    }
    sv[0] = sn[0];
    sv[1] = sn[1];
  });
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  const size_t row0 = ((size_t)bg * a.S + s) * a.R;
  if (lane < a.R) a.psum[row0 + lane] = lsum;
  // O block db: lane (j, g) holds rows 4 g + v of column 4 j + 64 (db / 4) + db % 4
  float* dst = a.pacc + row0 * D + 4 * r;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int row = 4 * grp + v;
    if (row < a.R) {
#pragma unroll
      for (int n = 0; n < NL; ++n)
        *reinterpret_cast<f32x4*>(dst + (size_t)row * D + 64 * n) =
            f32x4{oacc[4 * n][v], oacc[4 * n + 1][v], oacc[4 * n + 2][v], oacc[4 * n + 3][v]};
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_pv_kernel(DecodeArgs a) {
  decode_pv_bf16<D>(a);
}
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_pv_f32_kernel(DecodeArgs a) {
  decode_pv_f32<D>(a);
}
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_scores_f32x16_kernel(DecodeArgs a) {
  decode_scores_f32_16<D>(a);
}
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_pv_f32x16_kernel(DecodeArgs a) {
  decode_pv_f32_16<D>(a);
}

// One workgroup per group: O = (sum of the chunks' partial P.V) / (sum of their phi sums), in
// chunk order; stats (m, l) as ra_attn_fwd writes them.
template <typename T, int D>
__device__ __forceinline__ void decode_combine(const DecodeArgs& a) {
  const int bg = blockIdx.x;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int len = cache_len(a, b);
  const int chunk = decode_chunk(a);
  const int nlive = (len + chunk - 1) / chunk;
  T* o = static_cast<T*>(a.o);
  for (int e = threadIdx.x; e < a.R * D; e += kThreads) {
    const int r = e / D, d = e % D;
    float acc = 0.0f, l = 0.0f;
#pragma unroll 8
    for (int s2 = 0; s2 < nlive; ++s2) {
      const size_t row = ((size_t)bg * a.S + s2) * a.R + r;
      acc += a.pacc[row * D + d];
      l += a.psum[row];
    }
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    const int h = g * a.rep + r / a.Nq, i = r % a.Nq;
    const size_t orow = (size_t)(b * a.Hq + h) * a.Nq + i;
    o[orow * D + d] = (T)(acc * inv);
    if (d == 0 && a.stats != nullptr) {
      a.stats[orow * 2] = nlive > 0 ? a.gmax[(size_t)bg * a.R + r] : -INFINITY;
      a.stats[orow * 2 + 1] = l;
    }
  }
}
template <int D>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(DecodeArgs a) {
  decode_combine<bf16, D>(a);
}
template <int D>
__global__ __launch_bounds__(kThreads) void decode_combine_f32_kernel(DecodeArgs a) {
  decode_combine<float, D>(a);
}

// The keys per wave come from the cache lengths at run time (decode_chunk): the total over about
// kDecodeTarget waves.  Measured on the B=16, Hq=32, Hkv=8 decode step (caches of 16384 and of
// mixed lengths), about 1024 waves in all beat 2048-8192 by 3-10%, the per-wave start-up (Q
// fragments, the first two blocks' latency) outweighing the finer load balance.  The plan bounds
// the size: at most the chunk that spreads full caches over that many waves, at least a quarter
// of it (and kDecodeMinChunk keys), which bounds the partial-result slots per group.
constexpr int64_t kDecodeMinChunk = 64;
constexpr int64_t kDecodeShrink = 4;

DecodePlan decode_plan(int64_t B, int64_t Hkv, int64_t Nk, int64_t R, int64_t D) {
  const int64_t groups = B * Hkv;
  auto up32 = [](int64_t x) { return (x + 31) / 32 * 32; };
  const int64_t nk32 = up32(Nk);
  int64_t cmax = up32((groups * Nk + kDecodeTarget - 1) / kDecodeTarget);
  cmax = cmax < kDecodeMinChunk ? kDecodeMinChunk : cmax;
  if (cmax > nk32) cmax = nk32 > 0 ? nk32 : 32;
  int64_t cmin = up32((cmax + kDecodeShrink - 1) / kDecodeShrink);
  cmin = cmin < kDecodeMinChunk ? kDecodeMinChunk : cmin;
  if (cmin > cmax) cmin = cmax;
  DecodePlan p;
  p.chunk_min = cmin;
  p.chunk_max = cmax;
  p.S = (Nk + cmin - 1) / cmin;
  // the waves full caches need; shorter ones take at most as many chunks (decode_chunk)
  p.waves = groups * ((Nk + cmax - 1) / cmax);
  const int64_t rows = groups * p.S * R;
  auto round256 = [](size_t n) { return (n + 255) / 256 * 256; };   // every region 16-byte aligned
  p.scores_bytes = round256((size_t)(groups * nk32 * R) * sizeof(float));
  p.pmax_bytes = round256((size_t)rows * sizeof(float));
  p.psum_bytes = round256((size_t)rows * sizeof(float));
  p.pacc_bytes = round256((size_t)(rows * D) * sizeof(float));
  p.gmax_bytes = round256((size_t)(groups * R) * sizeof(float));
  p.bytes = p.scores_bytes + p.pmax_bytes + p.psum_bytes + p.pacc_bytes + p.gmax_bytes;
  return p;
}

template <typename T, int D>
static hipError_t launch_decode_typed(const DecodeProblem& p, const DecodePlan& plan, void* ws,
                                      hipStream_t stream) {
  constexpr bool kBf16 = sizeof(T) == 2;
  DecodeArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.o = p.o;
  a.stats = p.stats;
  a.seqlens = p.seqlens;
  char* w = static_cast<char*>(ws);
  a.scores = reinterpret_cast<float*>(w);
  a.pmax = reinterpret_cast<float*>(w + plan.scores_bytes);
  a.psum = reinterpret_cast<float*>(w + plan.scores_bytes + plan.pmax_bytes);
  a.pacc = reinterpret_cast<float*>(w + plan.scores_bytes + plan.pmax_bytes + plan.psum_bytes);
  a.gmax = reinterpret_cast<float*>(w + plan.scores_bytes + plan.pmax_bytes + plan.psum_bytes + plan.pacc_bytes);
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.Nq = p.Nq;
  a.Nk = p.Nk;
  a.rep = p.Hq / p.Hkv;
  a.R = a.rep * p.Nq;
  a.nk32 = (p.Nk + 31) / 32 * 32;
  a.chunk_min = (int)plan.chunk_min;
  a.chunk_max = (int)plan.chunk_max;
  a.S = (int)plan.S;
  a.waves = (int)plan.waves;
  a.causal = p.causal;
  a.c = p.scale / 16.0f;
  const int groups = p.B * p.Hkv;
  const dim3 grid((a.waves + kWaves - 1) / kWaves), block(kThreads);
  // fp32 with at most 16 rows per K/V head: the 16-column products
  const bool narrow = !kBf16 && a.R <= 16;
  if constexpr (kBf16) hipLaunchKernelGGL((decode_scores_kernel<D>), grid, block, 0, stream, a);
  else if (narrow) hipLaunchKernelGGL((decode_scores_f32x16_kernel<D>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((decode_scores_f32_kernel<D>), grid, block, 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (kBf16) hipLaunchKernelGGL((decode_pv_kernel<D>), grid, block, 0, stream, a);
  else if (narrow) hipLaunchKernelGGL((decode_pv_f32x16_kernel<D>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((decode_pv_f32_kernel<D>), grid, block, 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (kBf16) hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(groups), block, 0, stream, a);
  else hipLaunchKernelGGL((decode_combine_f32_kernel<D>), dim3(groups), block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_decode(const DecodeProblem& p, void* workspace, hipStream_t stream) {
  const DecodePlan plan = decode_plan(p.B, p.Hkv, p.Nk, (int64_t)(p.Hq / p.Hkv) * p.Nq, p.D);
  if (p.bf16) {
    if (p.D == 64) return launch_decode_typed<bf16, 64>(p, plan, workspace, stream);
    return launch_decode_typed<bf16, 128>(p, plan, workspace, stream);
  }
  if (p.D == 64) return launch_decode_typed<float, 64>(p, plan, workspace, stream);
  return launch_decode_typed<float, 128>(p, plan, workspace, stream);
}

}  // namespace ra
