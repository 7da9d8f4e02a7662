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
#include <type_traits>

#include "ra_device.h"
#include "ra_internal.h"

namespace ra {

struct DecodeArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* stats;
  const int* seqlens;   // [B] cache lengths (nullptr: all Nk)
  float* scores;        // [groups][S][chunk / 32][R][2][16] raw dot products
  float* pmax;          // [groups][S][R] row max of a chunk
  float* psum;          // [groups][S][R] sum of phi of a chunk
  float* pacc;          // [groups][S][R][D] unnormalised P.V of a chunk
  float* gmax;          // [groups][R] row max over all chunks (written by chunk 0's wave)
  int Hq, Hkv, Nq, Nk, rep, R;
  int chunk;            // keys per wave, a multiple of 32
  int S;                // chunks per group: ceil(Nk / chunk)
  int wg_per_group;     // ceil(S / kWaves)
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

template <int D>
__global__ __launch_bounds__(kThreads) void decode_scores_kernel(DecodeArgs a) {
  constexpr int KC = D / 16;
  constexpr int CPR = D / 8, PER = 32 * CPR / kWave;
  __shared__ __attribute__((aligned(16))) bf16 k_lds[kWaves][32 * D];
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int bg = blockIdx.x / a.wg_per_group;
  const int s = (blockIdx.x % a.wg_per_group) * kWaves + wave;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int len = cache_len(a, b);
  const int k0 = s * a.chunk;
  if (s >= a.S || k0 >= len) return;   // whole wave: no barrier in this kernel
  const int nkeys = min(a.chunk, len - k0), nb = (nkeys + 31) / 32;

  // B operand: query row r = lane % 32 of the group (rows past R repeat the last one)
  const int r = lane & 31, rr = min(r, a.R - 1);
  const int h = g * a.rep + rr / a.Nq;
  const bf16* qrow = a.q + ((size_t)(b * a.Hq + h) * a.Nq + rr % a.Nq) * D;
  const int fcol = 8 * (lane >> 5);
  bf16x8 qf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) qf[kc] = load_frag(qrow + 16 * kc + fcol);
  const int lim = key_limit(a, len, rr);

  // K rows: coalesced 16-byte loads into the register ring (lane l takes chunks l, l + 64, ... of
  // a block; rows past the chunk's keys read as zeros), stored swizzled into this wave's LDS
  // tile, from which the A fragments are read (the previous block's reads have returned: their
  // results fed the products, and a wave's LDS operations execute in order)
  const __amdgpu_buffer_rsrc_t kr = tile_rsrc(a.k + ((size_t)bg * a.Nk + k0) * D, nkeys, D);
  u32x4 ring[3][PER];
  auto load = [&](int slot, int t) {
#pragma unroll
    for (int j = 0; j < PER; ++j)
      ring[slot][j] = __builtin_amdgcn_raw_buffer_load_b128(kr, (j * kWave + lane) * 16, uniform(t * 32 * D * 2), 0);
  };
  bf16* ktile = k_lds[wave];
  // this chunk's scores, [block][R rows][2 lane halves][16]; padded rows store past the end
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      a.scores + ((size_t)bg * a.S + s) * a.chunk * a.R, (short)0, uniform(nb * 32 * a.R * 4), kBufferWord3);
  const int s_off = r < a.R ? (r * 2 + (lane >> 5)) * 64 : 0x40000000;
  float mx = -INFINITY;
  load(0, 0);
  load(1, 1);
  ring3(nb, [&](auto slot_c, int t) {
    constexpr int slot = decltype(slot_c)::value;
    load((slot + 2) % 3, t + 2);
    // S^T = K Q^T: keys on the accumulator rows, query row r on the lane
    f32x16 sacc = {};
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int c = j * kWave + lane, row = c / CPR, cc = c % CPR;
      *reinterpret_cast<u32x4*>(ktile + swz_off<bf16, D>(row, cc)) = ring[slot][j];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) mma(sacc, swz_frag<bf16, D>(ktile, lane & 31, 16 * kc + fcol), qf[kc]);
    // key k0 + 32 t + 4 (lane >> 5) + row offset is kept iff it is <= lim (which is < len)
    keep_rows(sacc, -kNoBound, lim + 1 - (k0 + 32 * t + 4 * (lane >> 5)));
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(u32x4, f32x4{sacc[4 * q4], sacc[4 * q4 + 1], sacc[4 * q4 + 2], sacc[4 * q4 + 3]}),
          sr, s_off + 16 * q4, uniform(t * 32 * a.R * 4), 0);
  });
  mx = fmaxf(mx, __shfl_xor(mx, 32));   // lanes l and l + 32 hold the same row
  if (lane < a.R) a.pmax[((size_t)bg * a.S + s) * a.R + lane] = mx;
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_pv_kernel(DecodeArgs a) {
  constexpr int DB = D / 32, TILE = 32 * D;
  constexpr int CPR = D / 8;              // 16-byte chunks per row
  constexpr int PER = 32 * CPR / kWave;   // chunks of a 32-row tile per lane
  __shared__ __attribute__((aligned(16))) bf16 v_lds[kWaves][TILE];

  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int bg = blockIdx.x / a.wg_per_group;
  const int s = (blockIdx.x % a.wg_per_group) * kWaves + wave;
  const int b = bg / a.Hkv;
  const int len = cache_len(a, b);
  const int k0 = s * a.chunk;
  if (s >= a.S || k0 >= len) return;
  const int nkeys = min(a.chunk, len - k0), nb = (nkeys + 31) / 32;
  const int r = lane & 31;
  const bool live = r < a.R;

  // V rows: coalesced 16-byte loads into a register ring (lane l takes chunks l, l + 64, ... of
  // a block), then stored swizzled into this wave's LDS tile and read transposed
  const __amdgpu_buffer_rsrc_t vr = tile_rsrc(a.v + ((size_t)bg * a.Nk + k0) * D, nkeys, D);
  u32x4 ring[3][PER];
  auto load = [&](int slot, int t) {
#pragma unroll
    for (int j = 0; j < PER; ++j)
      ring[slot][j] = __builtin_amdgcn_raw_buffer_load_b128(vr, (j * kWave + lane) * 16, uniform(t * 32 * D * 2), 0);
  };
  bf16* tile = v_lds[wave];
  load(0, 0);
  load(1, 1);

  // the row max over every chunk of the group that holds keys: lanes r and r + 32 take the even
  // and odd chunks, eight loads in flight per round
  const int nlive = (len + a.chunk - 1) / a.chunk;
  float m = -INFINITY;
  if (live) {
    const float* pm = a.pmax + (size_t)bg * a.S * a.R + r;
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
  // 1 + u = fma(s, -c, kd); a row with no allowed key (m = -inf) takes kd = +inf: phi = 0
  const float kd = m == -INFINITY ? INFINITY : fmaf(m, a.c, 1.0f);

  // this chunk's scores as the first kernel stored them; padded rows (kd = +inf, so phi = 0
  // whatever they read) and blocks past the chunk read zeros
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      a.scores + ((size_t)bg * a.S + s) * a.chunk * a.R, (short)0, uniform(nb * 32 * a.R * 4), kBufferWord3);
  const int s_off = live ? (r * 2 + (lane >> 5)) * 64 : 0x40000000;
  auto load_scores = [&](int t) {
    f32x16 v;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 x = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, s_off + 16 * q4, uniform(t * 32 * a.R * 4), 0));
      v[4 * q4] = x[0];
      v[4 * q4 + 1] = x[1];
      v[4 * q4 + 2] = x[2];
      v[4 * q4 + 3] = x[3];
    }
    return v;
  };
  f32x16 sv = load_scores(0);
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float lsum = 0.0f;
  ring3(nb, [&](auto slot_c, int t) {
    constexpr int slot = decltype(slot_c)::value;
    load((slot + 2) % 3, t + 2);
    const f32x16 sn = load_scores(t + 1);
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

// One workgroup per group: O = (sum of the chunks' partial P.V) / (sum of their phi sums), in
// chunk order; stats (m, l) as ra_attn_fwd writes them.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(DecodeArgs a) {
  const int bg = blockIdx.x;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int len = cache_len(a, b);
  const int nlive = (len + a.chunk - 1) / a.chunk;
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
    a.o[orow * D + d] = (bf16)(acc * inv);
    if (d == 0 && a.stats != nullptr) {
      a.stats[orow * 2] = nlive > 0 ? a.gmax[(size_t)bg * a.R + r] : -INFINITY;
      a.stats[orow * 2 + 1] = l;
    }
  }
}

// Measured on the B=16, Hq=32, Hkv=8 decode step (caches of 16384 and of mixed lengths): about
// 1024 waves in all beat 2048-8192 by 3-10%, the per-wave start-up (Q fragments, the first two
// blocks' latency) outweighing the finer load balance.
constexpr int64_t kDecodeWaves = 1024;
constexpr int64_t kDecodeMinChunk = 64;

DecodePlan decode_plan(int64_t B, int64_t Hkv, int64_t Nk, int64_t R, int64_t D) {
  // about kDecodeWaves waves over the chip, at least kDecodeMinChunk keys per wave
  const int64_t groups = B * Hkv;
  int64_t chunk = (groups * Nk + kDecodeWaves - 1) / kDecodeWaves;
  chunk = ((chunk + 31) / 32) * 32;
  chunk = chunk < kDecodeMinChunk ? kDecodeMinChunk : chunk;
  const int64_t nk32 = ((Nk + 31) / 32) * 32;
  if (chunk > nk32) chunk = nk32 > 0 ? nk32 : 32;
  DecodePlan p;
  p.chunk = chunk;
  p.S = (Nk + chunk - 1) / chunk;
  const int64_t rows = groups * p.S * R;
  auto round256 = [](size_t n) { return (n + 255) / 256 * 256; };   // every region 16-byte aligned
  p.scores_bytes = round256((size_t)(rows * chunk) * sizeof(float));
  p.pmax_bytes = round256((size_t)rows * sizeof(float));
  p.psum_bytes = round256((size_t)rows * sizeof(float));
  p.pacc_bytes = round256((size_t)(rows * D) * sizeof(float));
  p.gmax_bytes = round256((size_t)(groups * R) * sizeof(float));
  p.bytes = p.scores_bytes + p.pmax_bytes + p.psum_bytes + p.pacc_bytes + p.gmax_bytes;
  return p;
}

template <int D>
static hipError_t launch_decode_typed(const DecodeProblem& p, const DecodePlan& plan, void* ws,
                                      hipStream_t stream) {
  DecodeArgs a;
  a.q = static_cast<const bf16*>(p.q);
  a.k = static_cast<const bf16*>(p.k);
  a.v = static_cast<const bf16*>(p.v);
  a.o = static_cast<bf16*>(p.o);
  a.stats = p.stats;
  a.seqlens = p.seqlens;
  char* w = static_cast<char*>(ws);
  a.scores = reinterpret_cast<float*>(w);
  a.pmax = reinterpret_cast<float*>(w + plan.scores_bytes);
  a.psum = reinterpret_cast<float*>(w + plan.scores_bytes + plan.pmax_bytes);
  a.pacc = reinterpret_cast<float*>(w + plan.scores_bytes + plan.pmax_bytes + plan.psum_bytes);
  a.gmax = reinterpret_cast<float*>(w + plan.scores_bytes + plan.pmax_bytes + plan.psum_bytes + plan.pacc_bytes);
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.Nq = p.Nq;
  a.Nk = p.Nk;
  a.rep = p.Hq / p.Hkv;
  a.R = a.rep * p.Nq;
  a.chunk = (int)plan.chunk;
  a.S = (int)plan.S;
  a.wg_per_group = (a.S + kWaves - 1) / kWaves;
  a.causal = p.causal;
  a.c = p.scale / 16.0f;
  const int groups = p.B * p.Hkv;
  const dim3 grid(groups * a.wg_per_group), block(kThreads);
  hipLaunchKernelGGL((decode_scores_kernel<D>), grid, block, 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_pv_kernel<D>), grid, block, 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(groups), block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_decode(const DecodeProblem& p, void* workspace, hipStream_t stream) {
  const DecodePlan plan = decode_plan(p.B, p.Hkv, p.Nk, (int64_t)(p.Hq / p.Hkv) * p.Nq, p.D);
  if (p.D == 64) return launch_decode_typed<64>(p, plan, workspace, stream);
  return launch_decode_typed<128>(p, plan, workspace, stream);
}

}  // namespace ra
