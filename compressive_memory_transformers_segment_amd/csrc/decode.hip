// Streaming decode for gfx950: a chunk of C new query rows per (batch, query
// head) attends causally to the rows of the current segment held in a K/V
// cache, retrieves from the memory state before that segment, and mixes the
// two with the head's gate.
//
// [HF-repro] "Infini-Attention メカニズム": steps Local Attention (causal
// attention inside the current segment), Memory Retrieval (sigma(q) M /
// (sigma(q) z + eps) against the pre-segment state), Integration (gate), and
// State Transfer (only (M, z) and the current segment's rows are kept).
//
// The work is a few query rows against at most one segment of keys, so it is
// bound by reading the cache (and M) once, not by arithmetic: it runs on the
// vector ALUs in fp32, in two kernels.
//   * decode_partial: one workgroup per (split of 64 keys, batch x kv head,
//     block of queries), so a 2048-row cache of 8 kv heads already gives 256
//     workgroups for one new row. Queries are (query head of the group, chunk
//     row) pairs: the g heads that share a kv head share one read of its keys.
//     The split's keys, values and the block's queries move to LDS with
//     16-byte loads (all issued before the first LDS write, widened to fp32);
//     lane j of a wave scores key j against the wave's queries (one per wave
//     when a kv head has at most four, else four), the split's max and sum
//     come from DPP and lane-swap reductions, and P V accumulates with the
//     lanes over value columns. Each split writes its unnormalised partial
//     (acc, max m, sum l).
//   * The retrieval sigma(q) M / (sigma(q).z + eps) of four queries takes one
//     workgroup: its four waves split the rows of M (each wave issues all its
//     loads at once) and multiply them with the four sigma(q) from LDS. With
//     at most four queries per kv head (single-row decode), that workgroup
//     runs in the split launch, beside the splits, and writes a partial slot
//     of its own; with more, the split launch already fills the chip and the
//     merge workgroup of the four queries computes it.
//   * decode_combine: one wave per query merges the split partials with the
//     usual max-rescaling, adds the retrieval, applies the gate and stores the
//     row.

#include <mutex>

#include "common.h"
#include "launch.h"

namespace ia {

// Fixed scratch of the allocation-free decode entry point: the key-split
// partials live here instead of in a buffer the handle grows. In host code
// this name is only a stand-in for the symbol; the device address of each
// device's copy comes from decode_scratch().
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

namespace {

constexpr int kDecKeys = 64;  // keys per workgroup (one split)

// x of another lane of the same 16-lane row, by DPP control CTRL: quad_perm
// 0xB1 = lane ^ 1, 0x4E = lane ^ 2; row_half_mirror 0x141 = lane 7 - i within
// 8; row_mirror 0x140 = lane 15 - i within 16.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Reductions over the 64 lanes; every lane ends with the same value (each
// step combines a lane with its partner by a commutative operation).
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Value column of lane `lane` for its e-th accumulator (D = 32: lanes 32..63
// mirror lanes 0..31 and store nothing).
template <int D>
__device__ __forceinline__ int dec_col(int lane, int e) {
  return D >= 64 ? lane + 64 * e : (lane & (D - 1));
}

// 8 consecutive elements of a q/k/v tensor as fp32 (one 16-byte load for
// bf16, two for fp32); the address is 16-byte aligned.
__device__ __forceinline__ void load8(const uint16_t *p, float (&x)[8]) {
  const u32x4 w = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = lo_bf16(w[i]);
    x[2 * i + 1] = hi_bf16(w[i]);
  }
}
__device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}

// Retrieval of queries q0 .. q0 + 3 of (batch x kv head) bh (the query
// order of the split kernel; slots past nq are empty), by the whole
// workgroup: sigma(q) goes to LDS (smem[0, 4 D)), wave w multiplies rows
// [w D/4, (w + 1) D/4) of M (row-major [d_k][d_v]; every load of the wave is
// issued before the FMAs) with the four sigma(q) and leaves its partial
// numerators in smem[4 D + (w 4 + r) D + c]; wave r leaves sigma(q_r).z + eps
// in smem[20 D + r]. Ends with a barrier: then numerator c of query r is the
// sum of the four waves' partials at (r, c), in wave order.
template <typename T, int D>
__device__ __forceinline__ void retrieval4(const T *__restrict__ q, const float *__restrict__ M,
                                           const float *__restrict__ z, float eps, float *smem,
                                           int bh, int Hq, int Hkv, int C, int q0) {
  constexpr int NE = D >= 64 ? D / 64 : 1;
  constexpr int RPW = D / 4;  // rows of M per wave
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int g = Hq / Hkv, nq = g * C;
  const int b = bh / Hkv, kvh = bh % Hkv;
  float(*sSq)[D] = reinterpret_cast<float(*)[D]>(smem);                  // [query][D]
  float(*sNum)[4][D] = reinterpret_cast<float(*)[4][D]>(smem + 4 * D);  // [wave][query][D]
  float *sDen = smem + 20 * D;
  const float *Mh = M + static_cast<size_t>(bh) * D * D;
  float mv[RPW][NE];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
    for (int e = 0; e < NE; ++e)
      mv[rr][e] = Mh[static_cast<size_t>(w * RPW + rr) * D + dec_col<D>(lane, e)];
  for (int x = tid; x < 4 * D; x += 256) {
    const int r = x / D, c = x % D, qi = q0 + r;
    float v = 0.f;
    if (qi < nq) {
      const size_t qrow = (static_cast<size_t>(b * Hq + kvh * g + qi / C) * C + qi % C) * D;
      v = elu1(load_as_f32(q, qrow + c));
    }
    sSq[r][c] = v;
  }
  __syncthreads();
  float num[4][NE];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int e = 0; e < NE; ++e) num[r][e] = 0.f;
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float sq = sSq[r][w * RPW + rr];  // same address in every lane
#pragma unroll
      for (int e = 0; e < NE; ++e) num[r][e] += sq * mv[rr][e];
    }
  }
  if (D >= 64 || lane < 32) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int e = 0; e < NE; ++e) sNum[w][r][dec_col<D>(lane, e)] = num[r][e];
  }
  const float *zh = z + static_cast<size_t>(bh) * D;
  float den = 0.f;
#pragma unroll
  for (int t = 0; t < (D + 63) / 64; ++t) {
    const int kk = lane + 64 * t;
    den += kk < D ? sSq[w][kk] * zh[kk] : 0.f;
  }
  den = wave_sum(den);
  if (lane == 0) sDen[w] = den + eps;
  __syncthreads();
}

// The split launch: workgroups x < n_splits take 64 keys each (local
// attention partials). With one query per wave (QPW = 1: a block of four
// queries), workgroup x = n_splits of each (batch x kv head, block) computes
// the block's retrieval numerators sigma(q) M and denominators
// sigma(q).z + eps instead, so that the merge kernel reads only partials. Partial slot (bh, x, query) holds D values and two scalars: for a
// key split the unnormalised sum P V, the split's max m and sum l; for the
// retrieval slot the numerator and the denominator (last scalar unused).
// QPW queries per wave (QB = 4 QPW per workgroup): 1 when a kv head has at
// most four new query rows, so that no wave scores empty query slots.
template <typename T, int D, int QPW>
__global__ __launch_bounds__(256) void decode_partial_kernel(
    const T *__restrict__ q, const T *__restrict__ kc, const T *__restrict__ vc,
    const float *__restrict__ M, const float *__restrict__ z, float *__restrict__ part, int Hq,
    int Hkv, int C, int cap, int n_past, int n_splits, float scale, float eps) {
  constexpr int QB = 4 * QPW;
  constexpr int KP = D + 4;                 // padded K row (floats)
  constexpr int NE = D >= 64 ? D / 64 : 1;  // value columns per lane
  constexpr int U = D / 8;                  // 8-element units per row
  constexpr int ATT = kDecKeys * KP + kDecKeys * D + QB * D + 4 * kDecKeys * QPW;
  constexpr int RET = 20 * D + 4;
  __shared__ __attribute__((aligned(16))) float smem[ATT > RET ? ATT : RET];

  const int split = blockIdx.x, bh = blockIdx.y, qb = blockIdx.z;
  const int g = Hq / Hkv, nq = g * C;
  const int b = bh / Hkv, kvh = bh % Hkv;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const size_t sstride = static_cast<size_t>(nq) * (D + 2);
  float *pbase = part + (static_cast<size_t>(bh) * (n_splits + 1) + min(split, n_splits)) * sstride;

  if (QPW == 1 && split >= n_splits) {
    // Retrieval numerators and denominators of the block's four queries.
    const int q0 = qb * QB;
    retrieval4<T, D>(q, M, z, eps, smem, bh, Hq, Hkv, C, q0);
    const float(*sNum)[4][D] = reinterpret_cast<const float(*)[4][D]>(smem + 4 * D);
    const float *sDen = smem + 20 * D;
    for (int x = tid; x < 4 * D; x += 256) {
      const int r = x / D, c = x % D, qi = q0 + r;
      if (qi < nq)
        pbase[qi * (D + 2) + c] = sNum[0][r][c] + sNum[1][r][c] + sNum[2][r][c] + sNum[3][r][c];
    }
    if (tid < 4 && q0 + tid < nq) pbase[(q0 + tid) * (D + 2) + D] = sDen[tid];
    return;
  }

  float(*sK)[KP] = reinterpret_cast<float(*)[KP]>(smem);
  float(*sV)[D] = reinterpret_cast<float(*)[D]>(smem + kDecKeys * KP);
  float(*sQ)[D] = reinterpret_cast<float(*)[D]>(smem + kDecKeys * KP + kDecKeys * D);
  float(*sP)[kDecKeys][QPW] = reinterpret_cast<float(*)[kDecKeys][QPW]>(
      smem + kDecKeys * KP + kDecKeys * D + QB * D);
  const int k0 = split * kDecKeys;
  const int k1 = min(k0 + kDecKeys, n_past + C);

  // Stage the split's keys and values and the block's queries (8 elements per
  // unit, all loads issued before the LDS writes).
  constexpr int KVU = kDecKeys * U / 256;  // K (and V) units per thread
  constexpr int QU = (QB * U + 255) / 256;
  float kx[KVU][8], vx[KVU][8], qx[QU][8];
#pragma unroll
  for (int it = 0; it < KVU; ++it) {
    const int u = tid + 256 * it, r = u / U, c = 8 * (u % U);
    const int row = min(k0 + r, k1 - 1);  // rows past the end: copies, zeroed below
    const size_t off = (static_cast<size_t>(bh) * cap + row) * D + c;
    load8(kc + off, kx[it]);
    load8(vc + off, vx[it]);
  }
#pragma unroll
  for (int it = 0; it < QU; ++it) {
    const int u = tid + 256 * it, r = u / U, c = 8 * (u % U);
    const int qi = min(qb * QB + r, nq - 1);
    const int hh = qi / C, i = qi % C;
    if (u < QB * U)
      load8(q + (static_cast<size_t>(b * Hq + kvh * g + hh) * C + i) * D + c, qx[it]);
  }
#pragma unroll
  for (int it = 0; it < KVU; ++it) {
    const int u = tid + 256 * it, r = u / U, c = 8 * (u % U);
    const bool in = k0 + r < k1;
#pragma unroll
    for (int j = 0; j < 8; j += 4) {
      *reinterpret_cast<f32x4 *>(&sK[r][c + j]) =
          in ? f32x4{kx[it][j], kx[it][j + 1], kx[it][j + 2], kx[it][j + 3]} : f32x4{};
      *reinterpret_cast<f32x4 *>(&sV[r][c + j]) =
          in ? f32x4{vx[it][j], vx[it][j + 1], vx[it][j + 2], vx[it][j + 3]} : f32x4{};
    }
  }
#pragma unroll
  for (int it = 0; it < QU; ++it) {
    const int u = tid + 256 * it, r = u / U, c = 8 * (u % U);
    if (u < QB * U) {
#pragma unroll
      for (int j = 0; j < 8; j += 4)
        *reinterpret_cast<f32x4 *>(&sQ[r][c + j]) =
            f32x4{qx[it][j], qx[it][j + 1], qx[it][j + 2], qx[it][j + 3]};
    }
  }
  __syncthreads();

  // Scores: lane j takes key k0 + j against the wave's queries w, w + 4, ...
  // Four independent partial sums per query (one per column of a 4-column
  // group), so that the dependent chain is D / 4 long instead of D: with a
  // single wave per SIMD nothing else hides its latency.
  float s4[QPW][4];
#pragma unroll
  for (int r = 0; r < QPW; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) s4[r][i] = 0.f;
#pragma unroll 8
  for (int c = 0; c < D; c += 4) {
    const f32x4 kk = *reinterpret_cast<const f32x4 *>(&sK[lane][c]);
#pragma unroll
    for (int r = 0; r < QPW; ++r) {
      const f32x4 qq = *reinterpret_cast<const f32x4 *>(&sQ[w + 4 * r][c]);
#pragma unroll
      for (int i = 0; i < 4; ++i) s4[r][i] = __builtin_fmaf(kk[i], qq[i], s4[r][i]);
    }
  }
  float s[QPW];
#pragma unroll
  for (int r = 0; r < QPW; ++r) s[r] = (s4[r][0] + s4[r][1]) + (s4[r][2] + s4[r][3]);
  const int key = k0 + lane;
  float m[QPW], l[QPW];
#pragma unroll
  for (int r = 0; r < QPW; ++r) {
    const int qi = qb * QB + w + 4 * r;
    const int lim = qi < nq ? n_past + qi % C : -1;  // last key the query sees
    const float sc = key <= lim && key < k1 ? s[r] * scale : -INFINITY;
    m[r] = wave_max(sc);  // -inf when the query sees no key of this split
    const float p = m[r] == -INFINITY ? 0.f : __expf(sc - m[r]);
    l[r] = wave_sum(p);
    sP[w][lane][r] = p;
  }
  // (sP[w] is written and read by wave w only: the wave's own LDS ordering
  // suffices, no workgroup barrier.)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  // P V with keys j and j + kDecKeys / 2 in separate partial sums (two
  // dependent chains of half the length per value).
  float acc2[2][QPW][NE];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int r = 0; r < QPW; ++r)
#pragma unroll
      for (int e = 0; e < NE; ++e) acc2[h][r][e] = 0.f;
#pragma unroll 8
  for (int j = 0; j < kDecKeys / 2; ++j) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int jj = j + h * (kDecKeys / 2);
      float pj[QPW];
#pragma unroll
      for (int r = 0; r < QPW; ++r) pj[r] = sP[w][jj][r];
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const float vv = sV[jj][dec_col<D>(lane, e)];
#pragma unroll
        for (int r = 0; r < QPW; ++r) acc2[h][r][e] = __builtin_fmaf(pj[r], vv, acc2[h][r][e]);
      }
    }
  }
  float acc[QPW][NE];
#pragma unroll
  for (int r = 0; r < QPW; ++r)
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[r][e] = acc2[0][r][e] + acc2[1][r][e];

#pragma unroll
  for (int r = 0; r < QPW; ++r) {
    const int qi = qb * QB + w + 4 * r;
    if (qi < nq) {
      float *pp = pbase + static_cast<size_t>(qi) * (D + 2);
      if (D >= 64 || lane < 32) {
#pragma unroll
        for (int e = 0; e < NE; ++e) pp[dec_col<D>(lane, e)] = acc[r][e];
      }
      if (lane == 0) {
        pp[D] = m[r];
        pp[D + 1] = l[r];
      }
    }
  }
}

// Merge: wave w of workgroup (x, bh) finishes query 4 x + w from the split
// partials and the retrieval, applies the gate and stores the row. RET: the
// workgroup computes the retrieval of its four queries itself (blocks of more
// than four queries per kv head, whose split launch already fills the chip);
// otherwise it reads the retrieval slot the split launch wrote.
constexpr int kCB = 32;  // key splits merged per batch in the combine kernel

template <typename T, int D, bool RET>
__global__ __launch_bounds__(256) void decode_combine_kernel(
    const T *__restrict__ q, const float *__restrict__ M, const float *__restrict__ z,
    const float *__restrict__ part, const float *__restrict__ beta, T *__restrict__ out, int Hq,
    int Hkv, int C, int n_splits, float eps) {
  constexpr int NE = D >= 64 ? D / 64 : 1;
  __shared__ __attribute__((aligned(16))) float smem[RET ? 20 * D + 4 : 1];
  const int bh = blockIdx.y;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = Hq / Hkv, nq = g * C;
  const int b = bh / Hkv, kvh = bh % Hkv;
  const int qi = blockIdx.x * 4 + w;
  const size_t sstride = static_cast<size_t>(nq) * (D + 2);
  const float *pp =
      part + static_cast<size_t>(bh) * (n_splits + 1) * sstride + static_cast<size_t>(qi) * (D + 2);
  float num[NE], den;
  if constexpr (RET) {
    retrieval4<T, D>(q, M, z, eps, smem, bh, Hq, Hkv, C, blockIdx.x * 4);
    if (qi >= nq) return;  // after the only barrier
    const float(*sNum)[4][D] = reinterpret_cast<const float(*)[4][D]>(smem + 4 * D);
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int c = dec_col<D>(lane, e);
      num[e] = sNum[0][w][c] + sNum[1][w][c] + sNum[2][w][c] + sNum[3][w][c];
    }
    den = smem[20 * D + w];
  } else {
    if (qi >= nq) return;  // no barrier on this path
    // Retrieval slot (issued first; used last).
    const float *pr = pp + n_splits * sstride;
#pragma unroll
    for (int e = 0; e < NE; ++e) num[e] = pr[dec_col<D>(lane, e)];
    den = pr[D];
  }
  const int hh = qi / C, i = qi % C;
  const int h = kvh * g + hh;
  const size_t qrow = (static_cast<size_t>(b * Hq + h) * C + i) * D;

  // A_dot: merge the splits, kCB at a time. Every load of a batch is issued
  // before the first use (one memory round trip per batch): lane j < kCB
  // reads split s0 + j's max and sum, and every lane reads its columns of
  // every split of the batch. Batches merge with the usual rescaling; every
  // query sees key 0, so the final max is finite.
  float mt = -INFINITY, lt = 0.f, a[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) a[e] = 0.f;
  for (int s0 = 0; s0 < n_splits; s0 += kCB) {
    const int nb = min(kCB, n_splits - s0);
    const float *pb = pp + static_cast<size_t>(s0) * sstride;
    const int sj = min(lane, nb - 1);
    const float ms = pb[sj * sstride + D], ls = pb[sj * sstride + D + 1];
    float vb[kCB][NE];
#pragma unroll
    for (int j = 0; j < kCB; ++j)
#pragma unroll
      for (int e = 0; e < NE; ++e) vb[j][e] = pb[min(j, nb - 1) * sstride + dec_col<D>(lane, e)];
    const float mb = wave_max(lane < nb ? ms : -INFINITY);
    const float mn = fmaxf(mt, mb);
    // weight of split s0 + lane (0 for lanes past the batch and for splits
    // that saw no key); the running sums rescale to the new max
    const float wl = (lane < nb && ms != -INFINITY) ? __expf(ms - mn) : 0.f;
    const float sc = mt == -INFINITY ? 0.f : __expf(mt - mn);
    lt = lt * sc + wave_sum(wl * ls);
#pragma unroll
    for (int e = 0; e < NE; ++e) a[e] *= sc;
#pragma unroll
    for (int j = 0; j < kCB; ++j) {
      const float wj = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wl), j));
#pragma unroll
      for (int e = 0; e < NE; ++e) a[e] += wj * vb[j][e];
    }
    mt = mn;
  }

  // A_mem = sigma(q) M / (sigma(q) z + eps), gate, store.
  const float gam = 1.f / (1.f + __expf(-beta[h]));
  const float inv_den = 1.f / den, inv_l = 1.f / lt;
  if (D >= 64 || lane < 32) {
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int c = dec_col<D>(lane, e);
      store_from_f32(out, qrow + c, gam * (num[e] * inv_den) + (1.f - gam) * (a[e] * inv_l));
    }
  }
}

template <typename T, int D, int QPW>
hipError_t launch_decode_q(const DecodeGeometry &g, const T *q, const T *kc, const T *vc,
                           const float *beta, const float *M, const float *z, float *part, T *out,
                           hipStream_t stream) {
  constexpr int QB = 4 * QPW;
  const int nq = (g.Hq / g.Hkv) * g.C;
  const int bh = g.B * g.Hkv;
  const int n_splits = decode_splits(g.n_past + g.C);
  const dim3 grid1(n_splits + (QPW > 1 ? 0 : 1), bh, (nq + QB - 1) / QB);
  decode_partial_kernel<T, D, QPW><<<grid1, 256, 0, stream>>>(
      q, kc, vc, M, z, part, g.Hq, g.Hkv, g.C, g.cap, g.n_past, n_splits,
      1.f / sqrtf(static_cast<float>(D)), g.eps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid2((nq + 3) / 4, bh);
  // One query per wave: the split launch computes the retrieval in
  // workgroups of its own; four: the merge does.
  decode_combine_kernel<T, D, (QPW > 1)><<<grid2, 256, 0, stream>>>(
      q, M, z, part, beta, out, g.Hq, g.Hkv, g.C, n_splits, g.eps);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_t(const DecodeGeometry &g, const T *q, const T *kc, const T *vc,
                           const float *beta, const float *M, const float *z, float *part, T *out,
                           hipStream_t stream) {
  if ((g.Hq / g.Hkv) * g.C <= 4)
    return launch_decode_q<T, D, 1>(g, q, kc, vc, beta, M, z, part, out, stream);
  return launch_decode_q<T, D, 4>(g, q, kc, vc, beta, M, z, part, out, stream);
}

template <typename T>
hipError_t launch_decode_d(const DecodeGeometry &g, const T *q, const T *kc, const T *vc,
                           const float *beta, const float *M, const float *z, float *part, T *out,
                           hipStream_t stream) {
  switch (g.D) {
    case 32: return launch_decode_t<T, 32>(g, q, kc, vc, beta, M, z, part, out, stream);
    case 64: return launch_decode_t<T, 64>(g, q, kc, vc, beta, M, z, part, out, stream);
    case 128: return launch_decode_t<T, 128>(g, q, kc, vc, beta, M, z, part, out, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int decode_splits(int n_keys) { return (n_keys + kDecKeys - 1) / kDecKeys; }

hipError_t decode_scratch(int dev, float **ptr) {
  static std::mutex mu;
  static float *addr[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // Each device holds its own copy of the array at its own address; the
    // caller has made `dev` current.
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float *>(p);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t decode_partial_floats(const DecodeGeometry &g) {
  return static_cast<size_t>(g.B) * g.Hkv * (decode_splits(g.n_past + g.C) + 1) *
         (static_cast<size_t>(g.Hq / g.Hkv) * g.C) * (g.D + 2);
}

hipError_t launch_decode_bf16(const DecodeGeometry &g, const uint16_t *q, const uint16_t *kc,
                              const uint16_t *vc, const float *beta, const float *M,
                              const float *z, float *part, uint16_t *out, hipStream_t stream) {
  return launch_decode_d<uint16_t>(g, q, kc, vc, beta, M, z, part, out, stream);
}

hipError_t launch_decode_f32(const DecodeGeometry &g, const float *q, const float *kc,
                             const float *vc, const float *beta, const float *M, const float *z,
                             float *part, float *out, hipStream_t stream) {
  return launch_decode_d<float>(g, q, kc, vc, beta, M, z, part, out, stream);
}

}  // namespace ia
