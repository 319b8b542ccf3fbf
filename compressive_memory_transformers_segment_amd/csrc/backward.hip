// Backward pass of the Infini-attention forward: gradients of
//   loss = <d_out, out> + <d_M, M_S> + <d_z, z_S>
// with respect to q, k, v, beta, M_0 and z_0, by backpropagation through time
// over the segments (the training setting of [LNCB-review] "実装上の流れ" and of
// [HF-repro]'s reproduction, where the memory carries gradient from each
// segment back to the earlier ones). Everything is computed in fp32.
//
// Notation per (b, kv head j) and segment s: (Mp, zp) = (M_{s-1}, z_{s-1}) is
// the state the segment reads, (gM_s, gz_s) the gradient of the state after
// it, sq = sigma(q), sk = sigma(k), den = sq . zp + eps, denk = sk . zp + eps.
//
// The work splits into parts that are independent per segment and short
// chains over the segments:
//   states per (b, kv head, segment): the column sums of sigma(K) (then their
//          prefix, z before each segment), H_s = sigma(K)^T V and, for the
//          delta rule, G_s; then the d x d chain M_s = (I - G_s) M_{s-1} + H_s
//          (G_s = 0 for the linear rule) gives the state every segment reads;
//   query  per (b, q head, segment, 128 query rows): the local attention's dQ
//          (softmax backward with the row statistics recomputed), the
//          retrieval backward (dnum = g dO / den, dden = -g sum(dO num) / den^2,
//          dq += (dnum Mp^T + dden zp) sigma'(q)) and the gate's d beta;
//   key    per (b, kv head, segment, 128 keys): the local attention's dK, dV
//          over every query row and query head of the group that sees the keys;
//   outer  per (b, kv head, segment): R_s = sum sq^T dnum and r_s = sum sq^T dden
//          over the group's query heads, and for the delta rule
//          G_s = sk^T diag(1 / denk) sk;
//   chain  gM_{s-1} = gM_s + R_s (linear), (I - G_s) gM_s + R_s (delta): the
//          delta update is affine in the state, M_s = (I - G_s) M_{s-1} + H_s;
//   update per (b, kv head, segment, 32 rows): with Y = sk gM_s,
//          dv += Y; linear: dsk = v gM_s^T; delta: with numk = sk Mp,
//          W = v - numk / denk, ddenk = sum(Y numk) / denk^2,
//          dsk = W gM_s^T - (Y / denk) Mp^T + ddenk zp, and the z gradient
//          picks up qz_s = sk^T ddenk;
//   z chain gz_{s-1} = gz_s + r_s + qz_s, a reverse prefix sum once every gM_s
//          is known (no product with gM sits on this chain), after which
//          dk += gz_s sigma'(k) row by row.
// sigma'(x) = 1 for x > 0 and exp(x) = sigma(x) otherwise, i.e. min(sigma(x), 1).

#include <type_traits>

#include "common.h"
#include "launch.h"

namespace ia {
namespace {

constexpr int kThreads = 256;
constexpr int kKT = 32;  // keys (or state rows) per LDS chunk

// acc[i][j] += sum_{kk < kn} A(r0 + 16 i, kk) * B(kk, c0 + 16 j), with
// (r0, c0) = (thread / 16, thread % 16): the 16 lanes sharing r0 sit side by
// side in one wave, so a row reduction is a shuffle over 16 lanes.
template <int MI, int NJ, class FA, class FB>
__device__ __forceinline__ void mm16(float (&acc)[MI][NJ], int kn, const FA &fa, const FB &fb) {
  const int r0 = threadIdx.x >> 4, c0 = threadIdx.x & 15;
  for (int kk = 0; kk < kn; ++kk) {
    float av[MI], bv[NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i) av[i] = fa(r0 + 16 * i, kk);
#pragma unroll
    for (int j = 0; j < NJ; ++j) bv[j] = fb(kk, c0 + 16 * j);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
  }
}

template <int MI, int NJ>
__device__ __forceinline__ void zero(float (&acc)[MI][NJ]) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = 0.f;
}

__device__ __forceinline__ float sum16(float x) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) x += __shfl_xor(x, m, 16);
  return x;
}

__device__ __forceinline__ float gate(float beta) { return 1.f / (1.f + expf(-beta)); }

constexpr float kLog2e = 1.4426950408889634f;

// A lane's value combined with that of the lane 32 away (v_permlane32_swap
// returns {x, x of lane ^ 32} in some order; max and sum are symmetric).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// sigma'(x) from sigma(x): 1 where x > 0 (sigma > 1), sigma itself elsewhere.
__device__ __forceinline__ float elu1_grad_from(float s) { return fminf(s, 1.f); }

// Rows [row0, row0 + kn) of a [rows][D] tensor into LDS (zero past `valid`).
template <typename T, int D, int P>
__device__ __forceinline__ void load_rows(float (*dst)[P], const T *src, int kn, int valid,
                                          bool apply_sigma) {
  for (int idx = threadIdx.x; idx < kn * D; idx += kThreads) {
    const int r = idx / D, c = idx % D;
    float x = 0.f;
    if (r < valid) {
      x = load_as_f32(src, static_cast<size_t>(r) * D + c);
      if (apply_sigma) x = elu1(x);
    }
    dst[r][c] = x;
  }
}

// ---------------------------------------------------------------------------
// The two local-attention kernels run their products on the fp32 matrix
// cores (v_mfma_f32_32x32x2_f32: one 32x32 block, two contraction steps per
// instruction, full fp32). In a 32x32 result block, lane l owns column l % 32
// and the rows kappa(r, g) = 8 (r / 4) + 4 g + r % 4 of its 16 registers r,
// g = l / 32. A product whose contraction index is the row index of a result
// block takes that block straight from registers as its B operand: step s
// (of 16) of lane group g contracts over index kappa(s, g), and the A operand
// reads the same index. The hardware sums over (step, lane group) pairs, so
// any bijection between them and the contraction index gives the same sum as
// long as both operands use it.

__device__ __forceinline__ int kappa(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// bf16 storage: a product of two stored bf16 tensors runs as
// v_mfma_f32_32x32x16_bf16. Products of bf16 values are exact in fp32 and the
// accumulation is fp32, so this is the same arithmetic as the fp32 path. Lane
// group g supplies the 8 contraction indices 16 t + 8 g + e (e < 8) of step t
// in both operands.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t *p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p));
}

// Rows [0, kn) of a [rows][D] bf16 tensor into an LDS tile with row stride
// PB (zero past `valid`), 16 bytes at a time.
template <int D, int PB>
__device__ __forceinline__ void load_rows_bf16(uint16_t (*dst)[PB], const uint16_t *src, int kn,
                                               int valid) {
  constexpr int U = D / 8;
  for (int idx = threadIdx.x; idx < kn * U; idx += kThreads) {
    const int r = idx / U, c = 8 * (idx % U);
    u32x4 x = {0u, 0u, 0u, 0u};
    if (r < valid) x = *reinterpret_cast<const u32x4 *>(src + static_cast<size_t>(r) * D + c);
    *reinterpret_cast<u32x4 *>(&dst[r][c]) = x;
  }
}

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): the pair carries x to
// about 2^-17 relative, so a product of x with a stored bf16 operand runs as
// two bf16 MFMAs at fp32-level accuracy. Element e of the pair holds x[e].
__device__ __forceinline__ void split_bf16x8(const float *x, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = static_cast<__bf16>(x[e]);
    hi[e] = h;
    lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(h));
  }
}

// The 8 values of column c at rows kappa(8 st + e, g), e < 8, of a bf16 LDS
// tile: the A operand matching a result block's registers 8 st .. 8 st + 7
// used as the B operand (the contraction runs over the block's rows). Those
// rows are R .. R + 3 and R + 8 .. R + 11 with R = 16 st + 4 g, so two
// transposing LDS reads (ds_read_b64_tr_b16) fetch them. In each group of 16
// lanes, lane i receives element i % 4 of the 8-byte pieces addressed by
// lanes i / 4 + 4 j, j = 0 .. 3, in that order; lane A of the group addresses
// row R + A / 4, columns c0 + 4 (A % 4) .. + 3, so lane i receives rows
// R .. R + 3 of column c0 + i. The caller passes c = (a multiple of 32) +
// lane % 32, and the whole wave takes part.
template <int PB>
__device__ __forceinline__ bf16x8 gather_rows(const uint16_t (*tile)[PB], int st, int g, int c) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const int A = static_cast<int>(threadIdx.x) & 15;
  const int c0 = c - A;
  auto rd = [&](int R) __attribute__((always_inline)) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s *)(&tile[R + A / 4][c0 + 4 * (A % 4)]));
  };
  const u32x2 lo = __builtin_bit_cast(u32x2, rd(16 * st + 4 * g));
  const u32x2 hi = __builtin_bit_cast(u32x2, rd(16 * st + 8 + 4 * g));
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Workgroup barrier that orders LDS only: __syncthreads() also waits for the
// wave's outstanding global loads, which would drain the next tile's
// prefetch.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// query: dq, the softmax row statistics (lse, E) and gamma / den, dden for the
// outer products, and the gate's contribution to d beta. 128 query rows per
// workgroup, 32 per wave; key tiles of 32.
//   S^T = K Q^T and (dO V^T)^T = V dO^T put one query per lane, so the row
//   statistics of the softmax are per lane (plus the lane 32 away);
//   dq^T = K^T dS^T takes dS^T from registers;
//   retrieval: num^T = Mp^T sigma(Q)^T and dsq^T = Mp dnum^T, one 32-row
//   chunk of Mp^T in LDS at a time.
// MODE 0 runs both passes over the keys in one launch. For bf16 storage they
// are two launches over the same grid: MODE 1 (statistics only: lse and E,
// 120 registers, three workgroups per CU) and MODE 2 (reads them back, then
// dq, the retrieval and d beta, two workgroups per CU); the pair is about 3%
// faster at the Llama-3-8B shape than the single launch, whose register
// budget the second pass sets for the first as well.
template <typename T, int D, int MODE>
__global__ __launch_bounds__(kThreads, (std::is_same<T, uint16_t>::value ? (MODE == 1 ? 3 : 2) : 1)) void bwd_query_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ dout, const float *__restrict__ beta, const float *__restrict__ mt,
    const float *__restrict__ zpre, int Hq, int Hkv, int L, int N, int S, float eps,
    float *__restrict__ dq, float *__restrict__ lse_out, float *__restrict__ e_out,
    float *__restrict__ gd_out, float *__restrict__ dden_out, float *__restrict__ dbeta_part) {
  constexpr int P = D + 1;
  constexpr int NB = D / 32;  // 32-wide blocks along d
  constexpr int QT = 128;
  constexpr bool BF = std::is_same<T, uint16_t>::value;
  constexpr int PB = D + 8;   // bf16 row stride: 16-byte aligned rows
  __shared__ float sK[BF ? 1 : kKT][P];  // fp32 storage: key tile, 32-row chunks of Mp^T
  __shared__ float sV[BF ? 1 : kKT][P];
  __shared__ __attribute__((aligned(16))) uint16_t sKb[BF ? kKT : 1][PB];  // bf16 key tile
  __shared__ __attribute__((aligned(16))) uint16_t sVb[BF ? kKT : 1][PB];
  // bf16: the workgroup's d_out rows (each lane reads back only the row it
  // wrote), which keeps them out of the register file.
  __shared__ __attribute__((aligned(16))) uint16_t sOw[BF ? QT : 1][PB];
  __shared__ float sZ[D];
  __shared__ float sAcc[kThreads / 64];

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int s = blockIdx.y, bh = blockIdx.z;
  const int b = bh / Hq, h = bh % Hq;
  const int grp = Hq / Hkv;
  const size_t kvh = static_cast<size_t>(b) * Hkv + h / grp;
  const int a = s * N, e = min(a + N, L);
  const int i0 = a + blockIdx.x * QT;
  // This block's slot of the gate gradient's partial sums (summed in a fixed
  // order afterwards): head h, then (b, s, row block).
  float *dbeta_slot =
      dbeta_part + static_cast<size_t>(h) * (static_cast<size_t>(gridDim.z / Hq) * S * gridDim.x) +
      (static_cast<size_t>(b) * S + s) * gridDim.x + blockIdx.x;
  if (i0 >= e) {
    if (MODE != 1 && t == 0) *dbeta_slot = 0.f;
    return;
  }
  const int kend = min(i0 + QT, e);  // keys this tile's rows can see: [a, kend)
  const int wq0 = i0 + 32 * w;       // this wave's first query row
  const bool wave_live = wq0 < e;
  const int qi = wq0 + l32;          // this lane's query row
  const bool qvalid = qi < e;
  const float gam = gate(beta[h]);
  const float scale = 1.f / sqrtf(static_cast<float>(D));
  const size_t qbase = static_cast<size_t>(bh) * L;
  const T *kb = k + kvh * L * D;
  const T *vb = v + kvh * L * D;
  for (int c = t; c < D; c += kThreads) sZ[c] = zpre[(kvh * (S + 1) + s) * D + c];

  // This lane's query row and d_out row as B operands: element 2 u + g (fp32
  // storage), elements 16 t + 8 g + e (bf16 storage).
  float qr[BF ? 1 : D / 2], orow[BF ? 1 : D / 2];
  bf16x8 qb8[BF ? D / 16 : 1];
  if constexpr (BF) {
    const bf16x8 z8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
      const size_t o = (qbase + qi) * D + 16 * u + 8 * g;
      qb8[u] = qvalid ? ld_bf16x8(reinterpret_cast<const uint16_t *>(q) + o) : z8;
      *reinterpret_cast<bf16x8 *>(&sOw[32 * w + l32][16 * u + 8 * g]) =
          qvalid ? ld_bf16x8(reinterpret_cast<const uint16_t *>(dout) + o) : z8;
    }
  } else {
#pragma unroll
    for (int u = 0; u < D / 2; ++u) {
      const size_t o = (qbase + qi) * D + 2 * u + g;
      qr[u] = qvalid ? load_as_f32(q, o) : 0.f;
      orow[u] = qvalid ? load_as_f32(dout, o) : 0.f;
    }
  }

  // fp32 storage: the key tile j0 staged synchronously.
  auto load_kv = [&](int j0) {
    __syncthreads();
    load_rows<T, D, P>(sK, kb + static_cast<size_t>(j0) * D, kKT, kend - j0, false);
    load_rows<T, D, P>(sV, vb + static_cast<size_t>(j0) * D, kKT, kend - j0, false);
    __syncthreads();
  };
  // bf16 storage: the next key tile's rows travel in registers (KVN 16-byte
  // units of K and of V per thread) while the current tile is worked on.
  constexpr int U16 = D / 8;
  constexpr int KVN = (kKT * U16 + kThreads - 1) / kThreads;
  u32x4 pk[BF ? KVN : 1], pv[BF ? KVN : 1];
  auto fetch = [&](int j0) __attribute__((always_inline)) {
    const uint16_t *k16 = reinterpret_cast<const uint16_t *>(kb);
    const uint16_t *v16 = reinterpret_cast<const uint16_t *>(vb);
#pragma unroll
    for (int it = 0; it < KVN; ++it) {
      const int idx = t + kThreads * it, r = idx / U16, c = 8 * (idx % U16);
      if (idx < kKT * U16) {
        const size_t o = static_cast<size_t>(min(j0 + r, kend - 1)) * D + c;
        pk[it] = *reinterpret_cast<const u32x4 *>(k16 + o);
        pv[it] = *reinterpret_cast<const u32x4 *>(v16 + o);
      }
    }
  };
  auto stage = [&](int j0) __attribute__((always_inline)) {  // rows past kend: zero
#pragma unroll
    for (int it = 0; it < KVN; ++it) {
      const int idx = t + kThreads * it, r = idx / U16, c = 8 * (idx % U16);
      if (idx < kKT * U16) {
        const bool in = j0 + r < kend;
        *reinterpret_cast<u32x4 *>(&sKb[r][c]) = in ? pk[it] : u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4 *>(&sVb[r][c]) = in ? pv[it] : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto scores = [&](f32x16 &st, f32x16 &ot) {
    st = zero16();
    ot = zero16();
    if constexpr (BF) {
#pragma unroll
      for (int u = 0; u < D / 16; ++u) {
        st = mfma32(ld_bf16x8(&sKb[l32][16 * u + 8 * g]), qb8[u], st);
        ot = mfma32(ld_bf16x8(&sVb[l32][16 * u + 8 * g]),
                    ld_bf16x8(&sOw[32 * w + l32][16 * u + 8 * g]), ot);
      }
    } else {
#pragma unroll
      for (int u = 0; u < D / 2; ++u) {
        st = mfma32(sK[l32][2 * u + g], qr[u], st);
        ot = mfma32(sV[l32][2 * u + g], orow[u], ot);
      }
    }
  };
  // Key row kk, column c of the current key tile as fp32.
  auto key_at = [&](int kk, int c) -> float {
    if constexpr (BF) return bf16_to_f32(sKb[kk][c]);
    else return sK[kk][c];
  };
  // Key tile j0 is visible to some row of this wave.
  auto wave_sees = [&](int j0) { return wave_live && j0 <= wq0 + 31; };
  // One pass over the key tiles [a, kend): body(j0) for the tiles this wave
  // sees. bf16: the tile is staged from registers between two LDS-only
  // barriers, then the next tile's loads are issued, so they are in flight
  // during the work and the next stage waits for them.
  auto pass = [&](auto &&body) __attribute__((always_inline)) {
    if constexpr (BF) {
      fetch(a);
      for (int j0 = a; j0 < kend; j0 += kKT) {
        lds_barrier();
        stage(j0);
        lds_barrier();
        if (j0 + kKT < kend) fetch(j0 + kKT);
        if (wave_sees(j0)) body(j0);
      }
    } else {
      for (int j0 = a; j0 < kend; j0 += kKT) {
        load_kv(j0);
        if (wave_sees(j0)) body(j0);
      }
    }
  };

  // Pass 1: online max, sum and E = sum_j P_ij (dO_i . v_j) of each row.
  // Scores are masked only on tiles that hold a key some row of the wave must
  // not see (the diagonal tile, keys past the segment end); elsewhere every
  // key is visible to every row of the wave (rows past the segment end are
  // never stored). The exponentials take the scale and log2(e) in one FMA.
  const float sc2 = scale * kLog2e;
  auto mask_scores = [&](f32x16 &st, int j0) __attribute__((always_inline)) {
    if (j0 + kKT - 1 > wq0 || j0 + kKT > e) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + kappa(r, g);
        if (!(key <= qi && key < e)) st[r] = -INFINITY;
      }
    }
  };
  float lse, E;
  if constexpr (MODE == 2) {
    // The statistics launch stored them; rows past the segment end take a
    // shift of -inf, so their (never stored) dS is zero.
    lse = qvalid ? lse_out[qbase + qi] : INFINITY;
    E = qvalid ? e_out[qbase + qi] : 0.f;
  } else {
    float m = -INFINITY, l = 0.f, ea = 0.f;  // m: running max of the scaled scores
    pass([&](int j0) __attribute__((always_inline)) {
      f32x16 st, ot;
      scores(st, ot);
      mask_scores(st, j0);
      float mx = fmaxf(st[0], st[1]);
#pragma unroll
      for (int r = 2; r < 16; r += 2) mx = fmaxf(mx, fmaxf(st[r], st[r + 1]));
      mx = max_xor32(mx) * scale;  // the scale is positive: max(s) scale = max(s scale)
      const float mn = fmaxf(m, mx);
      const float nb = -mn * kLog2e;
      float ps = 0.f, pe = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], sc2, nb));
        ps += p;
        pe = __builtin_fmaf(p, ot[r], pe);
      }
      ps = sum_xor32(ps);
      pe = sum_xor32(pe);
      const float f = __builtin_amdgcn_exp2f((m - mn) * kLog2e);
      l = l * f + ps;
      ea = ea * f + pe;
      m = mn;
    });
    lse = m + __logf(l);
    E = ea / l;
  }
  if constexpr (MODE == 1) {
    if (qvalid && g == 0) {
      lse_out[qbase + qi] = lse;
      e_out[qbase + qi] = E;
    }
    return;
  }

  // Pass 2: dS^T = (1 - g) P^T (dO V^T - E)^T, dq^T += K^T dS^T.
  f32x16 dqa[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) dqa[cb] = zero16();
  // (1 - g) P in one exponential: log2(1 - g) joins the row's shift (-inf,
  // and so zero probabilities, when the gate is fully open).
  const float bq = __log2f(1.f - gam) - lse * kLog2e;
  pass([&](int j0) __attribute__((always_inline)) {
    f32x16 st, ot;
    scores(st, ot);
    mask_scores(st, j0);
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
      ds[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], sc2, bq)) * (ot[r] - E);
    if constexpr (BF) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bf16x8 hi, lo;
        split_bf16x8(ds + 8 * st, hi, lo);
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
          const bf16x8 ak = gather_rows<PB>(sKb, st, g, 32 * cb + l32);
          dqa[cb] = mfma32(ak, hi, dqa[cb]);
          dqa[cb] = mfma32(ak, lo, dqa[cb]);
        }
      }
    } else {
#pragma unroll
      for (int cb = 0; cb < NB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqa[cb] = mfma32(key_at(kappa(r, g), 32 * cb + l32), ds[r], dqa[cb]);
    }
  });

  // Retrieval backward from the pre-segment snapshot (Mp^T in mt, zp in zpre).
  const float *mtp = mt + (kvh * S + s) * D * D;
  f32x16 dsq[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) dsq[cb] = zero16();
  float s1 = 0.f;  // dO_i . num_i, this lane's part
  float den = 0.f;
  if constexpr (BF) {
    // bf16 storage: both products of the retrieval backward run on the bf16
    // matrix cores. Their fp32 factors (sigma(q), Mp, dnum) are carried as
    // bf16 pairs hi + lo, and each product takes hi.hi + hi.lo + lo.hi
    // (about 2^-16 relative; the lo.lo term is below that).
    //   num^T = Mp^T sigma(Q)^T: sigma(q) of this lane's query at d =
    //   16 t + 8 g + e is the B operand of step t;
    //   dsq^T = Mp dnum^T: dnum from registers, as dS in the dq product.
    const uint16_t *q16 = reinterpret_cast<const uint16_t *>(q);
    const uint16_t *o16 = reinterpret_cast<const uint16_t *>(dout);
    bf16x8 sqh[D / 16], sql[D / 16];
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
      const u32x4 wq = qvalid ? *reinterpret_cast<const u32x4 *>(q16 + (qbase + qi) * D + 16 * u +
                                                                  8 * g)
                              : u32x4{0u, 0u, 0u, 0u};
      float x[8];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        x[2 * e2] = elu1(lo_bf16(wq[e2]));
        x[2 * e2 + 1] = elu1(hi_bf16(wq[e2]));
      }
#pragma unroll
      for (int e2 = 0; e2 < 8; ++e2) den += x[e2] * sZ[16 * u + 8 * g + e2];
      split_bf16x8(x, sqh[u], sql[u]);
    }
    den = sum_xor32(den) + eps;
    const float gd = gam / den;
    if (qvalid && g == 0) gd_out[qbase + qi] = gd;
    for (int jb = 0; jb < NB; ++jb) {
      __syncthreads();
      // Rows 32 jb .. 32 jb + 31 of Mp^T as bf16 hi (sKb) and lo (sVb) parts.
      for (int idx = t; idx < kKT * D / 4; idx += kThreads) {
        const int jj = idx / (D / 4), c = 4 * (idx % (D / 4));
        const float4 m4 = *reinterpret_cast<const float4 *>(mtp + static_cast<size_t>(32 * jb + jj) *
                                                                      D + c);
        const float mv[4] = {m4.x, m4.y, m4.z, m4.w};
        uint32_t hw[2], lw[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const __bf16 h0 = static_cast<__bf16>(mv[2 * i]), h1 = static_cast<__bf16>(mv[2 * i + 1]);
          hw[i] = pack_bf16x2(static_cast<float>(h0), static_cast<float>(h1));
          lw[i] = pack_bf16x2(mv[2 * i] - static_cast<float>(h0), mv[2 * i + 1] - static_cast<float>(h1));
        }
        *reinterpret_cast<u32x2 *>(&sKb[jj][c]) = u32x2{hw[0], hw[1]};
        *reinterpret_cast<u32x2 *>(&sVb[jj][c]) = u32x2{lw[0], lw[1]};
      }
      __syncthreads();
      if (!wave_live) continue;
      f32x16 num = zero16();  // num^T rows 32 jb + kappa, column = this lane's query
#pragma unroll
      for (int u = 0; u < D / 16; ++u) {
        const bf16x8 mh = ld_bf16x8(&sKb[l32][16 * u + 8 * g]);
        const bf16x8 ml = ld_bf16x8(&sVb[l32][16 * u + 8 * g]);
        num = mfma32(mh, sqh[u], num);
        num = mfma32(mh, sql[u], num);
        num = mfma32(ml, sqh[u], num);
      }
      float dn[16];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int j = 32 * jb + 8 * r4 + 4 * g;
        const u32x2 wo = qvalid ? *reinterpret_cast<const u32x2 *>(o16 + (qbase + qi) * D + j)
                                : u32x2{0u, 0u};
        const float o4[4] = {lo_bf16(wo[0]), hi_bf16(wo[0]), lo_bf16(wo[1]), hi_bf16(wo[1])};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s1 += o4[i] * num[4 * r4 + i];
          dn[4 * r4 + i] = gd * o4[i];
        }
      }
      // dsq^T[c][i] += sum_j Mp[c][j] dnum[i][j], j = 32 jb + kappa(r, g).
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bf16x8 dh, dl;
        split_bf16x8(dn + 8 * st, dh, dl);
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
          const bf16x8 mh = gather_rows<PB>(sKb, st, g, 32 * cb + l32);
          const bf16x8 ml = gather_rows<PB>(sVb, st, g, 32 * cb + l32);
          dsq[cb] = mfma32(mh, dh, dsq[cb]);
          dsq[cb] = mfma32(mh, dl, dsq[cb]);
          dsq[cb] = mfma32(ml, dh, dsq[cb]);
        }
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < D / 2; ++u) qr[u] = elu1(qr[u]);  // sigma(q), element 2 u + g
#pragma unroll
    for (int u = 0; u < D / 2; ++u) den += qr[u] * sZ[2 * u + g];
    den += __shfl_xor(den, 32) + eps;
    const float gd = gam / den;
    if (qvalid && g == 0) gd_out[qbase + qi] = gd;
    for (int jb = 0; jb < NB; ++jb) {
      __syncthreads();
      for (int idx = t; idx < kKT * D; idx += kThreads) {
        const int jj = idx / D, c = idx % D;  // sK[jj][c] = Mp^T[32 jb + jj][c]
        sK[jj][c] = mtp[static_cast<size_t>(32 * jb + jj) * D + c];
      }
      __syncthreads();
      if (!wave_live) continue;
      f32x16 num = zero16();  // num^T rows 32 jb + kappa, column = this lane's query
#pragma unroll
      for (int u = 0; u < D / 2; ++u) num = mfma32(sK[l32][2 * u + g], qr[u], num);
      float dn[16];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int j = 32 * jb + 8 * r4 + 4 * g;
        float o4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          o4[i] = qvalid ? load_as_f32(dout, (qbase + qi) * D + j + i) : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s1 += o4[i] * num[4 * r4 + i];
          dn[4 * r4 + i] = gd * o4[i];
        }
      }
      // dsq^T[c][i] += sum_j Mp[c][j] dnum[i][j], j = 32 jb + kappa(r, g).
#pragma unroll
      for (int cb = 0; cb < NB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dsq[cb] = mfma32(sK[kappa(r, g)][32 * cb + l32], dn[r], dsq[cb]);
    }
  }
  s1 += __shfl_xor(s1, 32);
  const float dden = -gam * s1 / (den * den);
  if (qvalid && g == 0) {
    dden_out[qbase + qi] = dden;
    if constexpr (MODE == 0) {
      lse_out[qbase + qi] = lse;
      e_out[qbase + qi] = E;
    }
  }
  if (qvalid) {
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int c = 32 * cb + 8 * r4 + 4 * g;
        float res[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sg = elu1_grad_from(elu1(load_as_f32(q, (qbase + qi) * D + c + i)));
          res[i] = dqa[cb][4 * r4 + i] * scale + (dsq[cb][4 * r4 + i] + dden * sZ[c + i]) * sg;
        }
        *reinterpret_cast<float4 *>(dq + (qbase + qi) * D + c) =
            make_float4(res[0], res[1], res[2], res[3]);
      }
  }
  // d beta: sum over rows of dO . (A_mem - A_dot), times g (1 - g).
  // Summed in a fixed order: a butterfly within the wave, then the waves in
  // index order, so the result does not depend on timing.
  float contrib = (qvalid && g == 0) ? s1 / den - E : 0.f;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) contrib += __shfl_xor(contrib, o);
  if (lane == 0) sAcc[w] = contrib;
  __syncthreads();
  if (t == 0) {
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) tot += sAcc[i];
    *dbeta_slot = tot * gam * (1.f - gam);
  }
}

// ---------------------------------------------------------------------------
// key: dK, dV of the local attention for 128 keys of one segment (32 per
// wave, K and V rows in registers), over every query head of the kv group and
// every query row at or after the keys, in chunks of 32 rows staged in LDS
// for all four waves.
//   S = Q K^T and dO V^T put one key per lane;
//   dv^T = dO^T P and dk^T = Q^T dS take P and dS from registers.
template <typename T, int D>
__global__ __launch_bounds__(kThreads, (std::is_same<T, uint16_t>::value ? 2 : 1)) void bwd_key_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ dout, const float *__restrict__ beta, const float *__restrict__ lse,
    const float *__restrict__ E, int Hq, int Hkv, int L, int N, float *__restrict__ dk,
    float *__restrict__ dv) {
  constexpr int P = D + 1;
  constexpr int NB = D / 32;
  constexpr int KT = 128;
  constexpr bool BF = std::is_same<T, uint16_t>::value;
  constexpr int PB = D + 8;
  __shared__ float sQ[BF ? 1 : 32][P];
  __shared__ float sO[BF ? 1 : 32][P];
  __shared__ __attribute__((aligned(16))) uint16_t sQb[BF ? 32 : 1][PB];
  __shared__ __attribute__((aligned(16))) uint16_t sOb[BF ? 32 : 1][PB];
  // bf16: the workgroup's V rows (each lane reads back only the row it wrote),
  // which keeps them out of the register file.
  __shared__ __attribute__((aligned(16))) uint16_t sVw[BF ? KT : 1][PB];
  __shared__ __attribute__((aligned(16))) float sL[32];
  __shared__ __attribute__((aligned(16))) float sE[32];

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int s = blockIdx.y, kvh = blockIdx.z;
  const int b = kvh / Hkv, j = kvh % Hkv;
  const int grp = Hq / Hkv;
  const int a = s * N, e = min(a + N, L);
  const int j0 = a + blockIdx.x * KT;
  if (j0 >= e) return;
  const int wk0 = j0 + 32 * w;  // this wave's first key
  const bool wave_live = wk0 < e;
  const int key = wk0 + l32;    // this lane's key
  const bool kvalid = key < e;
  const float scale = 1.f / sqrtf(static_cast<float>(D));
  const float sc2 = scale * kLog2e;
  const size_t krow = static_cast<size_t>(kvh) * L + key;
  // Row shift of a chunk's rows as kept in sL: log2(1 - g) - lse log2(e).
  auto row_shift = [&](int hl, float lse_row) __attribute__((always_inline)) {
    return __log2f(1.f - gate(beta[j * grp + hl])) - lse_row * kLog2e;
  };

  float kr[BF ? 1 : D / 2], vr[BF ? 1 : D / 2];
  bf16x8 kb8[BF ? D / 16 : 1];
  if constexpr (BF) {
    const bf16x8 z8 = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
      const size_t o = krow * D + 16 * u + 8 * g;
      kb8[u] = kvalid ? ld_bf16x8(reinterpret_cast<const uint16_t *>(k) + o) : z8;
      *reinterpret_cast<bf16x8 *>(&sVw[32 * w + l32][16 * u + 8 * g]) =
          kvalid ? ld_bf16x8(reinterpret_cast<const uint16_t *>(v) + o) : z8;
    }
  } else {
#pragma unroll
    for (int u = 0; u < D / 2; ++u) {
      kr[u] = kvalid ? load_as_f32(k, krow * D + 2 * u + g) : 0.f;
      vr[u] = kvalid ? load_as_f32(v, krow * D + 2 * u + g) : 0.f;
    }
  }
  auto q_at = [&](int r, int c) -> float {
    if constexpr (BF) return bf16_to_f32(sQb[r][c]);
    else return sQ[r][c];
  };
  auto o_at = [&](int r, int c) -> float {
    if constexpr (BF) return bf16_to_f32(sOb[r][c]);
    else return sO[r][c];
  };
  f32x16 gk[NB], gv[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    gk[cb] = zero16();
    gv[cb] = zero16();
  }
  // One chunk: query head hl of the group, rows i0 .. i0 + 31 (staged in
  // sQb / sOb or sQ / sO, with their lse and E in sL / sE).
  auto chunk = [&](int hl, int i0) __attribute__((always_inline)) {
    f32x16 st = zero16(), ot = zero16();
    if constexpr (BF) {
#pragma unroll
      for (int u = 0; u < D / 16; ++u) {
        st = mfma32(ld_bf16x8(&sQb[l32][16 * u + 8 * g]), kb8[u], st);
        ot = mfma32(ld_bf16x8(&sOb[l32][16 * u + 8 * g]), ld_bf16x8(&sVw[32 * w + l32][16 * u + 8 * g]),
                    ot);
      }
    } else {
#pragma unroll
      for (int u = 0; u < D / 2; ++u) {
        st = mfma32(sQ[l32][2 * u + g], kr[u], st);
        ot = mfma32(sO[l32][2 * u + g], vr[u], ot);
      }
    }
    // Masked only where some key of the wave is after some row of the chunk
    // or past the segment end, or some row is past it. sL holds each row's
    // log2(1 - g) - lse log2(e), so one FMA and one exponential give (1 - g) P.
    if (wk0 + 31 > i0 || i0 + 32 > e || wk0 + 32 > e) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i0 + kappa(r, g);
        if (!(key <= row && row < e && kvalid)) st[r] = -INFINITY;
      }
    }
    float pw[16], ds[16];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const float4 bl = *reinterpret_cast<const float4 *>(&sL[8 * r4 + 4 * g]);
      const float4 ee = *reinterpret_cast<const float4 *>(&sE[8 * r4 + 4 * g]);
      const float blv[4] = {bl.x, bl.y, bl.z, bl.w}, eev[4] = {ee.x, ee.y, ee.z, ee.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * r4 + i;
        pw[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[r], sc2, blv[i]));
        ds[r] = pw[r] * (ot[r] - eev[i]);
      }
    }
    if constexpr (BF) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bf16x8 phi, plo, dhi, dlo;
        split_bf16x8(pw + 8 * st, phi, plo);
        split_bf16x8(ds + 8 * st, dhi, dlo);
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
          const bf16x8 ao = gather_rows<PB>(sOb, st, g, 32 * cb + l32);
          const bf16x8 aq = gather_rows<PB>(sQb, st, g, 32 * cb + l32);
          gv[cb] = mfma32(ao, phi, gv[cb]);
          gv[cb] = mfma32(ao, plo, gv[cb]);
          gk[cb] = mfma32(aq, dhi, gk[cb]);
          gk[cb] = mfma32(aq, dlo, gk[cb]);
        }
      }
    } else {
#pragma unroll
      for (int cb = 0; cb < NB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          gv[cb] = mfma32(o_at(kappa(r, g), 32 * cb + l32), pw[r], gv[cb]);
          gk[cb] = mfma32(q_at(kappa(r, g), 32 * cb + l32), ds[r], gk[cb]);
        }
    }
  };
  const int nci = (e - j0 + 31) / 32;  // row chunks per query head
  if constexpr (BF) {
    // The next chunk's rows travel in registers (KVN 16-byte units of q and
    // of d_out per thread, lse and E for threads < 32) while the current one
    // is worked on; it is staged between two LDS-only barriers.
    constexpr int U16 = D / 8;
    constexpr int KVN = (32 * U16 + kThreads - 1) / kThreads;
    u32x4 pq[KVN], po[KVN];
    float pl = 0.f, pe = 0.f;
    const uint16_t *q16 = reinterpret_cast<const uint16_t *>(q);
    const uint16_t *o16 = reinterpret_cast<const uint16_t *>(dout);
    // Chunk (hl, ci): query head hl of the group, rows j0 + 32 ci .. + 31.
    auto fetch = [&](int hl, int ci) __attribute__((always_inline)) {
      const int i0 = j0 + 32 * ci;
      const size_t hrow = (static_cast<size_t>(b) * Hq + j * grp + hl) * L;
#pragma unroll
      for (int it = 0; it < KVN; ++it) {
        const int idx = t + kThreads * it, r = idx / U16, c8 = 8 * (idx % U16);
        if (idx < 32 * U16) {
          const size_t o = (hrow + min(i0 + r, e - 1)) * D + c8;
          pq[it] = *reinterpret_cast<const u32x4 *>(q16 + o);
          po[it] = *reinterpret_cast<const u32x4 *>(o16 + o);
        }
      }
      if (t < 32) {
        pl = lse[hrow + min(i0 + t, e - 1)];
        pe = E[hrow + min(i0 + t, e - 1)];
      }
    };
    auto stage = [&](int hl, int ci) __attribute__((always_inline)) {  // rows past e: zero
      const int rows = min(32, e - (j0 + 32 * ci));
#pragma unroll
      for (int it = 0; it < KVN; ++it) {
        const int idx = t + kThreads * it, r = idx / U16, c8 = 8 * (idx % U16);
        if (idx < 32 * U16) {
          const bool in = r < rows;
          *reinterpret_cast<u32x4 *>(&sQb[r][c8]) = in ? pq[it] : u32x4{0u, 0u, 0u, 0u};
          *reinterpret_cast<u32x4 *>(&sOb[r][c8]) = in ? po[it] : u32x4{0u, 0u, 0u, 0u};
        }
      }
      if (t < 32) {
        sL[t] = t < rows ? row_shift(hl, pl) : 0.f;
        sE[t] = t < rows ? pe : 0.f;
      }
    };
    // (The chunk index advances as a (head, row chunk) pair: no divisions.)
    fetch(0, 0);
    for (int hl = 0, ci = 0; hl < grp;) {
      lds_barrier();
      stage(hl, ci);
      lds_barrier();
      int nhl = hl, nci2 = ci + 1;
      if (nci2 == nci) {
        nci2 = 0;
        ++nhl;
      }
      if (nhl < grp) fetch(nhl, nci2);
      const int i0 = j0 + 32 * ci;
      if (wave_live && wk0 <= i0 + 31) chunk(hl, i0);  // else: every key after every row
      hl = nhl;
      ci = nci2;
    }
  } else {
    for (int hl = 0; hl < grp; ++hl) {
      const size_t hrow = (static_cast<size_t>(b) * Hq + j * grp + hl) * L;
      for (int i0 = j0; i0 < e; i0 += 32) {
        const int rows = min(32, e - i0);
        __syncthreads();
        load_rows<T, D, P>(sQ, q + (hrow + i0) * D, 32, rows, false);
        load_rows<T, D, P>(sO, dout + (hrow + i0) * D, 32, rows, false);
        if (t < 32) {
          sL[t] = t < rows ? row_shift(hl, lse[hrow + i0 + t]) : 0.f;
          sE[t] = t < rows ? E[hrow + i0 + t] : 0.f;
        }
        __syncthreads();
        if (!wave_live || wk0 > i0 + 31) continue;  // every key after every row
        chunk(hl, i0);
      }
    }
  }
  if (!kvalid) return;
#pragma unroll
  for (int cb = 0; cb < NB; ++cb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int c = 32 * cb + 8 * r4 + 4 * g;
      *reinterpret_cast<float4 *>(dk + krow * D + c) =
          make_float4(gk[cb][4 * r4] * scale, gk[cb][4 * r4 + 1] * scale,
                      gk[cb][4 * r4 + 2] * scale, gk[cb][4 * r4 + 3] * scale);
      *reinterpret_cast<float4 *>(dv + krow * D + c) =
          make_float4(gv[cb][4 * r4], gv[cb][4 * r4 + 1], gv[cb][4 * r4 + 2], gv[cb][4 * r4 + 3]);
    }
}

// ---------------------------------------------------------------------------
// outer: per (b, kv head, segment), out += A^T B over a range of rows.
//   kind 0 (R): rows = (query head of the group, row of the segment),
//               A = sigma(q), B = dnum = gd dO (x2 = d_out, gd = gamma / den
//               per row, the product formed as in the query kernel);
//               r_s = sum A^T dden as well.
//   kind 1 (G): rows = rows of the segment, A = sigma(k), B = sigma(k) / denk.
//   kind 2 (H): rows = rows of the segment, A = sigma(k), B = v (x2).
// Each block writes the partial sum of its row range, D x D floats and then
// (kind 0) D floats of r, to part[unit][block]; bwd_sum_parts_kernel adds the
// blocks of a unit in index order, so the result does not depend on timing.
template <typename T, int D, int KIND>
__global__ __launch_bounds__(kThreads) void bwd_outer_kernel(
    const T *__restrict__ x, const T *__restrict__ x2, const float *__restrict__ gd,
    const float *__restrict__ dden, const float *__restrict__ zpre, int Hq, int Hkv, int L, int N,
    int S, float eps, int rows_per_block, float *__restrict__ part) {
  // The D x D sum of outer products over a range of rows runs on the bf16
  // matrix cores: each fp32 factor is staged as a bf16 pair hi + lo, and each
  // product takes hi.hi + hi.lo + lo.hi (about 2^-16 relative; kind 2 with
  // bf16 storage has an exact bf16 v, so its lo part is zero and skipped).
  // A 32-row chunk is staged row-major; the MFMA operands read it with
  // transposing LDS reads, both sides in the same row order, so the
  // contraction runs over the chunk's rows. The 32 x 32 output blocks are
  // split over the four waves.
  constexpr bool BF = std::is_same<T, uint16_t>::value;
  constexpr bool B_EXACT = KIND == 2 && BF;
  constexpr int PB = D + 8;
  constexpr int NC = D / 32;                        // 32-wide blocks per side
  constexpr int NBLK = NC * NC;
  constexpr int BPW = NBLK >= 4 ? NBLK / 4 : 1;     // output blocks per wave
  __shared__ __attribute__((aligned(16))) uint16_t sAh[kKT][PB];
  __shared__ __attribute__((aligned(16))) uint16_t sAl[kKT][PB];
  __shared__ __attribute__((aligned(16))) uint16_t sBh[kKT][PB];
  __shared__ __attribute__((aligned(16))) uint16_t sBl[B_EXACT ? 1 : kKT][PB];
  __shared__ float sX[kKT];
  __shared__ float sZ[D];

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int s = blockIdx.y, kvh = blockIdx.z;
  const int b = kvh / Hkv, j = kvh % Hkv;
  const int grp = Hq / Hkv;
  const int a = s * N, n = min(a + N, L) - a;
  const int total = KIND == 0 ? grp * n : n;
  const int u0 = blockIdx.x * rows_per_block;
  const int u1 = min(u0 + rows_per_block, total);
  constexpr int kPart = D * D + (KIND == 0 ? D : 0);  // floats of one block's partial
  const size_t unit = static_cast<size_t>(kvh) * S + s;
  float *o = part + (unit * gridDim.x + blockIdx.x) * kPart;
  if (u0 >= u1) {  // no rows (short last segment): a zero partial
    for (int i = t; i < kPart; i += kThreads) o[i] = 0.f;
    return;
  }
  if (KIND == 1)
    for (int c = t; c < D; c += kThreads) sZ[c] = zpre[(static_cast<size_t>(kvh) * (S + 1) + s) * D + c];

  // Source row (of x, and of d_out, gd and dden for kind 0) of unit row u.
  auto src_row = [&](int u) -> size_t {
    if (KIND == 0) {
      const int hl = u / n, i = a + u % n;
      return (static_cast<size_t>(b) * Hq + j * grp + hl) * L + i;
    }
    return static_cast<size_t>(kvh) * L + a + u;
  };
  // Split four values into bf16 hi and lo parts and store them at (r, c).
  auto put4 = [&](uint16_t (*th)[PB], uint16_t (*tl)[PB], int r, int c, const float (&v)[4])
                  __attribute__((always_inline)) {
    uint32_t hw[2], lw[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float h0 = static_cast<float>(static_cast<__bf16>(v[2 * i]));
      const float h1 = static_cast<float>(static_cast<__bf16>(v[2 * i + 1]));
      hw[i] = pack_bf16x2(h0, h1);
      lw[i] = pack_bf16x2(v[2 * i] - h0, v[2 * i + 1] - h1);
    }
    *reinterpret_cast<u32x2 *>(&th[r][c]) = u32x2{hw[0], hw[1]};
    if (tl != nullptr) *reinterpret_cast<u32x2 *>(&tl[r][c]) = u32x2{lw[0], lw[1]};
  };

  // The next chunk's rows travel in registers (raw words: bf16 pairs or
  // fp32) while the current chunk is worked on; the barriers inside the loop
  // order LDS only, so that they do not wait for those loads.
  constexpr int IT = kKT * D / 4 / kThreads;  // 4-element groups per thread
  static_assert(IT >= 1 && IT * kThreads == kKT * D / 4, "whole groups per thread");
  using Raw = typename std::conditional<BF, u32x2, float4>::type;
  auto raw_load = [&](const T *src, size_t row, int c) __attribute__((always_inline)) {
    if constexpr (BF)
      return *reinterpret_cast<const u32x2 *>(reinterpret_cast<const uint16_t *>(src) + row * D + c);
    else
      return *reinterpret_cast<const float4 *>(src + row * D + c);
  };
  auto raw_f32 = [&](const Raw &w2) __attribute__((always_inline)) {
    if constexpr (BF)
      return make_float4(lo_bf16(w2[0]), hi_bf16(w2[0]), lo_bf16(w2[1]), hi_bf16(w2[1]));
    else
      return w2;
  };
  Raw fa[IT], fb[IT];
  float fg[IT], fx = 0.f;
  auto fetch = [&](int c0u) __attribute__((always_inline)) {
    const int cnt = min(kKT, u1 - c0u);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = t + kThreads * it, r = idx / (D / 4), c = 4 * (idx % (D / 4));
      // rows past the range read the range's first row; staging zeroes them
      const size_t row = src_row(c0u + (r < cnt ? r : 0));
      fa[it] = raw_load(x, row, c);
      if (KIND == 0) fg[it] = gd[row];
      if (KIND != 1) fb[it] = raw_load(x2, row, c);
    }
    if (KIND == 0 && t < kKT) fx = t < cnt ? dden[src_row(c0u + t)] : 0.f;
  };

  f32x16 acc[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) acc[i] = zero16();
  float racc = 0.f;
  fetch(u0);
  for (int c0u = u0; c0u < u1; c0u += kKT) {
    const int cnt = min(kKT, u1 - c0u);
    lds_barrier();
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int idx = t + kThreads * it, r = idx / (D / 4), c = 4 * (idx % (D / 4));
      float av[4] = {0.f, 0.f, 0.f, 0.f}, bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (r < cnt) {
        const float4 xa = raw_f32(fa[it]);
        av[0] = elu1(xa.x);
        av[1] = elu1(xa.y);
        av[2] = elu1(xa.z);
        av[3] = elu1(xa.w);
        if (KIND == 0) {
          const float gr = fg[it];
          const float4 o4 = raw_f32(fb[it]);
          bv[0] = gr * o4.x; bv[1] = gr * o4.y; bv[2] = gr * o4.z; bv[3] = gr * o4.w;
        } else if (KIND == 2) {
          const float4 v4 = raw_f32(fb[it]);
          bv[0] = v4.x; bv[1] = v4.y; bv[2] = v4.z; bv[3] = v4.w;
        }
      }
      put4(sAh, sAl, r, c, av);
      if (KIND != 1) put4(sBh, B_EXACT ? nullptr : sBl, r, c, bv);
    }
    if (KIND == 0 && t < kKT) sX[t] = fx;
    if (c0u + kKT < u1) fetch(c0u + kKT);
    lds_barrier();
    if (KIND == 1) {
      // B = sigma(k) / (sigma(k) . z + eps), row by row: eight threads per
      // row take D / 8 columns each, then add their sums in a butterfly (the
      // same order on every lane of the eight).
      {
        static_assert(kThreads == 8 * kKT, "eight threads per staged row");
        const int r = t >> 3, part = t & 7;
        float d = 0.f;
#pragma unroll
        for (int c = part * (D / 8); c < (part + 1) * (D / 8); ++c)
          d += (bf16_to_f32(sAh[r][c]) + bf16_to_f32(sAl[r][c])) * sZ[c];
        d += __shfl_xor(d, 1);
        d += __shfl_xor(d, 2);
        d += __shfl_xor(d, 4);
        if (part == 0) sX[r] = 1.f / (d + eps);
      }
      lds_barrier();
      for (int idx = t; idx < kKT * D / 4; idx += kThreads) {
        const int r = idx / (D / 4), c = 4 * (idx % (D / 4));
        float bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          bv[i] = (bf16_to_f32(sAh[r][c + i]) + bf16_to_f32(sAl[r][c + i])) * sX[r];
        put4(sBh, sBl, r, c, bv);
      }
      lds_barrier();
    }
    if (KIND == 0 && t < D)
      for (int kk = 0; kk < kKT; ++kk)
        racc += (bf16_to_f32(sAh[kk][t]) + bf16_to_f32(sAl[kk][t])) * sX[kk];
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int ib = w * BPW + i;
      if (ib >= NBLK) break;
      const int rb = ib / NC, cb = ib % NC;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8 ah = gather_rows<PB>(sAh, st, g, 32 * rb + l32);
        const bf16x8 al = gather_rows<PB>(sAl, st, g, 32 * rb + l32);
        const bf16x8 bh = gather_rows<PB>(sBh, st, g, 32 * cb + l32);
        acc[i] = mfma32(ah, bh, acc[i]);
        acc[i] = mfma32(al, bh, acc[i]);
        if constexpr (!B_EXACT) {
          const bf16x8 bl = gather_rows<PB>(sBl, st, g, 32 * cb + l32);
          acc[i] = mfma32(ah, bl, acc[i]);
        }
      }
    }
  }
  // Lane (l32, g) holds output column 32 cb + l32, rows 32 rb + kappa(r, g).
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int ib = w * BPW + i;
    if (ib >= NBLK) break;
    const int rb = ib / NC, cb = ib % NC;
#pragma unroll
    for (int r = 0; r < 16; ++r) o[(32 * rb + kappa(r, g)) * D + 32 * cb + l32] = acc[i][r];
  }
  if (KIND == 0 && t < D) o[D * D + t] = racc;
}

// out_mat[u][i] (i < mat) and out_vec[u][i - mat] (mat <= i < mat + vec) =
// sum over b = 0 .. nblk - 1, in that order, of part[u][b][i].
// Grid: (units, ceil((mat + vec) / kThreads)).
__global__ __launch_bounds__(kThreads) void bwd_sum_parts_kernel(
    const float *__restrict__ part, int nblk, int mat, int vec, float *__restrict__ out_mat,
    float *__restrict__ out_vec) {
  const int i = blockIdx.y * kThreads + threadIdx.x;
  const int per = mat + vec;
  if (i >= per) return;
  const size_t u = blockIdx.x;
  const float *p = part + u * nblk * static_cast<size_t>(per) + i;
  float acc = 0.f;
  for (int b = 0; b < nblk; ++b) acc += p[static_cast<size_t>(b) * per];
  if (i < mat)
    out_mat[u * mat + i] = acc;
  else
    out_vec[u * vec + (i - mat)] = acc;
}

// ---------------------------------------------------------------------------
// chain: X <- X - G_s X + R_s (the G term for the delta rule only), 32
// columns per workgroup (column c of the result depends on column c of X
// only).
//   backward (FWD = false): X = gM, walked from s = S-1 down to 0; writes gM_s
//     (the gradient of the state after segment s) for every s, and gM_0.
//   forward (FWD = true): X = M, R = H, walked from s = 0 up; the delta
//     update is affine in the state, M_s = (I - G_s) M_{s-1} + H_s, with
//     H_s = sigma(K_s)^T V_s. Writes M_{s-1}^T for every s (the snapshot
//     layout), nothing at the end.
template <int D, bool FWD>
__global__ __launch_bounds__(kThreads) void bwd_gm_chain_kernel(
    const float *__restrict__ R, const float *__restrict__ G, const float *__restrict__ dM,
    int S, int delta, float *__restrict__ gma, float *__restrict__ dM0) {
  constexpr int MI = D / 16;
  __shared__ float sG[kKT][D + 1];  // sG[kk][r] = G[r][k0 + kk]
  __shared__ float sM[D][kKT + 1];  // this block's columns of gM_s
  const int t = threadIdx.x, r0 = t >> 4, c0 = t & 15;
  const int col0 = blockIdx.x * kKT;
  const size_t kvh = blockIdx.y;
  float g[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
      g[i][jj] = dM ? dM[kvh * D * D + (r0 + 16 * i) * D + col0 + c0 + 16 * jj] : 0.f;
  // G chunks travel through registers one chunk ahead of their use (the next
  // step's first chunk during the last chunk of a step), and each step's R
  // is loaded before its G product: the chain's steps are otherwise bound by
  // the latency of these loads.
  constexpr int SU = kKT * D / kThreads;  // G elements per thread and chunk
  float pre[SU];
  auto base_of = [&](int step) {
    return (kvh * S + static_cast<size_t>(FWD ? step : S - 1 - step)) * D * D;
  };
  auto fetch_g = [&](size_t gbase, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int idx = t + kThreads * i;
      pre[i] = G[gbase + static_cast<size_t>(idx / kKT) * D + k0 + idx % kKT];
    }
  };
  if (delta && S > 0) fetch_g(base_of(0), 0);
  for (int step = 0; step < S; ++step) {
    const size_t base = base_of(step);
    float rv[MI][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) rv[i][jj] = R[base + (r0 + 16 * i) * D + col0 + c0 + 16 * jj];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int r = r0 + 16 * i, c = col0 + c0 + 16 * jj;
        gma[base + (FWD ? c * D + r : r * D + c)] = g[i][jj];
      }
    if (delta) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) sM[r0 + 16 * i][c0 + 16 * jj] = g[i][jj];
      float acc[MI][2];
      zero(acc);
#pragma unroll 1
      for (int k0 = 0; k0 < D; k0 += kKT) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < SU; ++i) {
          const int idx = t + kThreads * i;
          sG[idx % kKT][idx / kKT] = pre[i];
        }
        __syncthreads();
        if (k0 + kKT < D) fetch_g(base, k0 + kKT);
        else if (step + 1 < S) fetch_g(base_of(step + 1), 0);
        mm16<MI, 2>(acc, kKT, [&](int r, int kk) { return sG[kk][r]; },
                    [&](int kk, int c) { return sM[k0 + kk][c]; });
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) g[i][jj] -= acc[i][jj];
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) g[i][jj] += rv[i][jj];
  }
  if (!FWD) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        dM0[kvh * D * D + (r0 + 16 * i) * D + col0 + c0 + 16 * jj] = g[i][jj];
  }
}

// Per-segment column sums of sigma(k): dz[unit][c] = sum over the segment's
// rows of sigma(k[i][c]).
constexpr int kZsumThreads = 512;

// Column sums of sigma(k) over one segment's rows. Each thread reads 8
// columns of a row (16 bytes for bf16 storage) and walks rows with a stride
// of RG = 512 / (D / 8) row groups, four rows in flight; the row groups are
// then added in index order, so the result does not depend on timing.
template <typename T, int D>
__global__ __launch_bounds__(kZsumThreads) void bwd_zsum_kernel(const T *__restrict__ k, int L,
                                                                int N, int S, float *__restrict__ dz) {
  constexpr int CPR = D / 8;                 // threads per row
  constexpr int RG = kZsumThreads / CPR;     // row groups
  __shared__ float part[RG][D + 1];
  const int t = threadIdx.x, c8 = 8 * (t % CPR), rg = t / CPR;
  const int s = blockIdx.x;
  const size_t kvh = blockIdx.y;
  const int a = s * N, e = min(a + N, L);
  const T *kb = k + kvh * L * D;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add_row = [&](int i) __attribute__((always_inline)) {
    float x[8];
    if constexpr (std::is_same<T, uint16_t>::value) {
      const u32x4 w4 = *reinterpret_cast<const u32x4 *>(
          reinterpret_cast<const uint16_t *>(kb) + static_cast<size_t>(i) * D + c8);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        x[2 * h] = lo_bf16(w4[h]);
        x[2 * h + 1] = hi_bf16(w4[h]);
      }
    } else {
      const float4 f0 = *reinterpret_cast<const float4 *>(kb + static_cast<size_t>(i) * D + c8);
      const float4 f1 = *reinterpret_cast<const float4 *>(kb + static_cast<size_t>(i) * D + c8 + 4);
      x[0] = f0.x; x[1] = f0.y; x[2] = f0.z; x[3] = f0.w;
      x[4] = f1.x; x[5] = f1.y; x[6] = f1.z; x[7] = f1.w;
    }
#pragma unroll
    for (int h = 0; h < 8; ++h) acc[h] += elu1(x[h]);
  };
  int i = a + rg;
  for (; i + 3 * RG < e; i += 4 * RG) {
    add_row(i);
    add_row(i + RG);
    add_row(i + 2 * RG);
    add_row(i + 3 * RG);
  }
  for (; i < e; i += RG) add_row(i);
#pragma unroll
  for (int h = 0; h < 8; ++h) part[rg][c8 + h] = acc[h];
  __syncthreads();
  if (t < D) {
    float z = 0.f;
    for (int j = 0; j < RG; ++j) z += part[j][t];
    dz[(kvh * S + s) * D + t] = z;
  }
}

// z before every segment: z_pre[kvh][s] = z0 + sum_{t < s} dz[t] (slot S: the final z).
__global__ void bwd_zprefix_kernel(const float *__restrict__ dz, const float *__restrict__ z0,
                                   int S, int D, float *__restrict__ zpre) {
  const size_t kvh = blockIdx.x;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    float z = z0[kvh * D + c];
    for (int s = 0; s < S; ++s) {
      zpre[(kvh * (S + 1) + s) * D + c] = z;
      z += dz[(kvh * S + s) * D + c];
    }
    zpre[(kvh * (S + 1) + S) * D + c] = z;
  }
}

// ---------------------------------------------------------------------------
// update: the memory write's gradient into v and k (without the gz_s term,
// added once the z chain is done), and qz_s = sk^T ddenk for the delta rule.
// One workgroup per 32 rows of a segment. The four d x d products per chunk
// run on the fp32 matrix cores (v_mfma_f32_32x32x2_f32): wave w computes the
// 32-column block w of each result (d = 128: four blocks, one per wave), with
// A = 32 rows of a chunk tile in LDS and B staged 32 rows at a time.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_update_kernel(
    const T *__restrict__ k, const T *__restrict__ v, const float *__restrict__ mt,
    const float *__restrict__ zpre, const float *__restrict__ gma, int L, int N, int S, float eps,
    int delta, float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ qz_part) {
  constexpr int P = D + 1;
  constexpr int NBC = D / 32;  // 32-column result blocks
  constexpr int SU = kKT * D / kThreads;  // B elements staged per thread
  __shared__ float sK[kKT][P];  // sigma(k)
  __shared__ float sV[kKT][P];  // v, then W = v - numk / denk
  __shared__ float sY[kKT][P];  // Y / denk
  __shared__ float sB[kKT][P];  // 32 rows of gM_s, Mp or their transposes; Y * numk
  __shared__ float sZ[D];
  __shared__ float sDen[kKT], sDd[kKT];

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int s = blockIdx.y, kvh = blockIdx.z;
  const int a = s * N, e = min(a + N, L);
  const int i0 = a + blockIdx.x * kKT;
  const size_t unit = static_cast<size_t>(kvh) * S + s;
  // This chunk's partial of qz_s (delta rule), summed in chunk order later.
  float *qzp = qz_part + (unit * gridDim.x + blockIdx.x) * D;
  if (i0 >= e) {
    if (delta)
      for (int c = t; c < D; c += kThreads) qzp[c] = 0.f;
    return;
  }
  const int rows = min(kKT, e - i0);
  const size_t row0 = static_cast<size_t>(kvh) * L + i0;
  const float *gm = gma + unit * D * D;
  const float *mtp = mt + unit * D * D;  // M_{s-1}^T: mtp[j * D + c] = Mp[c][j]
  load_rows<T, D, P>(sK, k + row0 * D, kKT, rows, true);
  load_rows<T, D, P>(sV, v + row0 * D, kKT, rows, false);
  for (int c = t; c < D; c += kThreads) sZ[c] = zpre[(static_cast<size_t>(kvh) * (S + 1) + s) * D + c];

  const bool owns = w < NBC;     // this wave holds a result block
  const int col = 32 * w + l32;  // its column (owners)
  // Rows [r0, r0 + 32) of the B operand into sB: B(kk, c) = src(r0 + kk, c),
  // every load issued before the first store.
  auto stage = [&](auto &&src, int r0) __attribute__((always_inline)) {
    __syncthreads();  // every wave is done with the previous chunk
    float x[SU];
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int idx = t + kThreads * i;
      x[i] = src(r0 + idx % kKT, idx / kKT);
    }
#pragma unroll
    for (int i = 0; i < SU; ++i) {
      const int idx = t + kThreads * i;
      sB[idx % kKT][idx / kKT] = x[i];
    }
    __syncthreads();
  };
  // acc += sgn A[:, r0 .. r0 + 31] B (the staged chunk), A a 32-row LDS tile.
  auto mm = [&](f32x16 &acc, const float (*A)[P], int r0, float sgn) __attribute__((always_inline)) {
    if (!owns) return;
#pragma unroll 8
    for (int kk = 0; kk < kKT; kk += 2) acc = mfma32(sgn * A[l32][r0 + kk + g], sB[kk + g][col], acc);
  };
  auto gm_rows = [&](int kk, int c) { return gm[static_cast<size_t>(kk) * D + c]; };   // gM_s
  auto gm_cols = [&](int kk, int c) { return gm[static_cast<size_t>(c) * D + kk]; };   // gM_s^T
  auto mp_rows = [&](int kk, int c) { return mtp[static_cast<size_t>(c) * D + kk]; }; // Mp
  auto mp_cols = [&](int kk, int c) { return mtp[static_cast<size_t>(kk) * D + c]; }; // Mp^T

  // Y = sk gM_s; dv += Y.
  f32x16 Y = zero16();
  for (int k0 = 0; k0 < D; k0 += kKT) {
    stage(gm_rows, k0);
    mm(Y, sK, k0, 1.f);
  }
  if (owns) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = kappa(i, g);
      if (r < rows) dv[(row0 + r) * D + col] += Y[i];
    }
  }

  if (delta) {
    // numk = sk Mp; denk = sk . zp + eps; W = v - numk / denk into sV,
    // Y / denk into sY, Y * numk into sB, whose row sums give ddenk.
    f32x16 nk = zero16();
    for (int k0 = 0; k0 < D; k0 += kKT) {
      stage(mp_rows, k0);
      mm(nk, sK, k0, 1.f);
    }
    if (t < kKT) {
      float d = eps;
      for (int c = 0; c < D; ++c) d += sK[t][c] * sZ[c];
      sDen[t] = d;
    }
    __syncthreads();  // sDen written; every wave is done with sB
    if (owns) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = kappa(i, g);
        const float den = sDen[r];
        sV[r][col] -= nk[i] / den;  // owner-only element
        sY[r][col] = Y[i] / den;
        sB[r][col] = Y[i] * nk[i];
      }
    }
    __syncthreads();
    if (t < kKT) {
      float part = 0.f;
      for (int c = 0; c < D; ++c) part += sB[t][c];
      const float den = sDen[t];
      sDd[t] = t < rows ? part / (den * den) : 0.f;
    }
    __syncthreads();
    if (t < D) {
      float acc = 0.f;
      for (int r = 0; r < kKT; ++r) acc += sK[r][t] * sDd[r];
      qzp[t] = acc;
    }
  }

  // dsk = W gM_s^T (linear: v gM_s^T) - (Y / denk) Mp^T + ddenk zp.
  f32x16 dsk = zero16();
  for (int j0 = 0; j0 < D; j0 += kKT) {
    stage(gm_cols, j0);
    mm(dsk, sV, j0, 1.f);
  }
  if (delta) {
    for (int j0 = 0; j0 < D; j0 += kKT) {
      stage(mp_cols, j0);
      mm(dsk, sY, j0, -1.f);
    }
  }
  if (owns) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = kappa(i, g);
      if (r < rows) {
        const float gr = dsk[i] + (delta ? sDd[r] * sZ[col] : 0.f);
        dk[(row0 + r) * D + col] += gr * elu1_grad_from(sK[r][col]);
      }
    }
  }
}

// update on the bf16 matrix cores (bf16 storage, d = 128): the same
// gradients as bwd_update_kernel for 128 rows of a segment (32 per wave).
// Every product is taken transposed, so that its result sits with one row
// per lane, which is the B-operand layout of the next product:
//   Y^T  = gM^T sk^T,  nk^T = Mp^T sk^T       (sk = sigma(k) of the rows)
//   dsk^T = gM W^T - Mp (Y / denk)^T           (linear: gM v^T)
// with W = v - nk / denk. The fp32 factors are bf16 pairs hi + lo and each
// product takes hi.hi + hi.lo + lo.hi (about 2^-16 relative); v is exact in
// bf16. gM_s and M_{s-1}^T are staged once per workgroup as bf16 hi / lo
// tiles; A operands that contract over a tile's rows use transposing LDS
// reads, those along a row two 8-byte reads (contraction index kappa order
// on both sides). One workgroup per CU (139 KB of LDS).
template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_update_mfma_kernel(
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, const float *__restrict__ mt,
    const float *__restrict__ zpre, const float *__restrict__ gma, int L, int N, int S, float eps,
    int delta, float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ qz_part) {
  constexpr int PB = D + 8;
  constexpr int NC = D / 32;  // 32-wide blocks along d
  constexpr int RW = 32 * (kThreads / 64);  // rows per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t sGh[D][PB];  // gM_s, hi
  __shared__ __attribute__((aligned(16))) uint16_t sGl[D][PB];  // gM_s, lo
  __shared__ __attribute__((aligned(16))) uint16_t sMh[D][PB];  // M_{s-1}^T, hi
  __shared__ __attribute__((aligned(16))) uint16_t sMl[D][PB];  // M_{s-1}^T, lo
  __shared__ float sZ[D];
  static_assert(static_cast<size_t>(RW) * (D + 1) * 4 <= sizeof(sGh) + sizeof(sGl),
                "the qz reduction reuses the gM tiles");

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int s = blockIdx.y, kvh = blockIdx.z;
  const int a = s * N, e = min(a + N, L);
  const int i0 = a + blockIdx.x * RW;
  const size_t unit = static_cast<size_t>(kvh) * S + s;
  float *qzp = qz_part + (unit * gridDim.x + blockIdx.x) * D;
  if (i0 >= e) {
    if (delta)
      for (int c = t; c < D; c += kThreads) qzp[c] = 0.f;
    return;
  }
  const int r = i0 + 32 * w + l32;  // this lane's row
  const bool rvalid = r < e;
  const size_t roff = (static_cast<size_t>(kvh) * L + r) * D;
  const float *gm = gma + unit * D * D;
  const float *mtp = mt + unit * D * D;
  for (int c = t; c < D; c += kThreads) sZ[c] = zpre[(static_cast<size_t>(kvh) * (S + 1) + s) * D + c];
  // gM_s and M_{s-1}^T as bf16 hi / lo tiles (row-major, as stored).
  auto split4 = [](const float4 &x, u32x2 &h, u32x2 &l) __attribute__((always_inline)) {
    const float xv[4] = {x.x, x.y, x.z, x.w};
    float hf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hf[i] = static_cast<float>(static_cast<__bf16>(xv[i]));
    h = u32x2{pack_bf16x2(hf[0], hf[1]), pack_bf16x2(hf[2], hf[3])};
    l = u32x2{pack_bf16x2(xv[0] - hf[0], xv[1] - hf[1]), pack_bf16x2(xv[2] - hf[2], xv[3] - hf[3])};
  };
  for (int idx = t; idx < D * D / 4; idx += kThreads) {
    const int row = idx / (D / 4), c = 4 * (idx % (D / 4));
    u32x2 h, l;
    split4(*reinterpret_cast<const float4 *>(gm + static_cast<size_t>(row) * D + c), h, l);
    *reinterpret_cast<u32x2 *>(&sGh[row][c]) = h;
    *reinterpret_cast<u32x2 *>(&sGl[row][c]) = l;
    if (delta) {
      split4(*reinterpret_cast<const float4 *>(mtp + static_cast<size_t>(row) * D + c), h, l);
      *reinterpret_cast<u32x2 *>(&sMh[row][c]) = h;
      *reinterpret_cast<u32x2 *>(&sMl[row][c]) = l;
    }
  }

  // This lane's row of k (sk = sigma(k)) and v at columns 32 kb + kappa(8 st + e, g):
  // the B operand of contraction step (kb, st), and the result registers of
  // block kb (register 8 st + e).
  auto row8 = [&](const uint16_t *src, int kb, int st) __attribute__((always_inline)) {
    const int c0 = 32 * kb + 16 * st + 4 * g;
    const u32x2 lo = rvalid ? *reinterpret_cast<const u32x2 *>(src + roff + c0) : u32x2{0u, 0u};
    const u32x2 hi = rvalid ? *reinterpret_cast<const u32x2 *>(src + roff + c0 + 8) : u32x2{0u, 0u};
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  auto unpack8 = [](const u32x4 &w4, float (&x)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      x[2 * h] = lo_bf16(w4[h]);
      x[2 * h + 1] = hi_bf16(w4[h]);
    }
  };
  bf16x8 skh[NC][2], skl[NC][2];
  float skv[NC][16];  // sigma(k) in result-register order
  float dpart = 0.f;
#pragma unroll
  for (int kb = 0; kb < NC; ++kb)
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      float x[8];
      unpack8(row8(k, kb, st), x);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[i] = rvalid ? elu1(x[i]) : 0.f;  // rows past the segment end: zero
        skv[kb][8 * st + i] = x[i];
        dpart += x[i] * sZ[32 * kb + kappa(8 * st + i, g)];
      }
      split_bf16x8(x, skh[kb][st], skl[kb][st]);
    }
  const float denk = sum_xor32(dpart) + eps;
  __syncthreads();  // the tiles are staged

  // A operand of output block cb, contraction step (kb, st): rows 32 cb + l32
  // of a tile taken along its row (two 8-byte reads), or its column 32 cb +
  // l32 taken over rows 32 kb + kappa (transposing reads).
  auto along = [&](const uint16_t (*tile)[PB], int cb, int kb, int st) __attribute__((always_inline)) {
    const uint16_t *p = &tile[32 * cb + l32][32 * kb + 16 * st + 4 * g];
    const u32x2 lo = *reinterpret_cast<const u32x2 *>(p);
    const u32x2 hi = *reinterpret_cast<const u32x2 *>(p + 8);
    return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
  };
  auto across = [&](const uint16_t (*tile)[PB], int cb, int kb, int st) __attribute__((always_inline)) {
    return gather_rows<PB>(tile + 32 * kb, st, g, 32 * cb + l32);
  };

  // Y^T = gM^T sk^T (A = gM over rows: transposing reads).
  f32x16 Y[NC];
#pragma unroll
  for (int cb = 0; cb < NC; ++cb) {
    Y[cb] = zero16();
#pragma unroll
    for (int kb = 0; kb < NC; ++kb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8 ah = across(sGh, cb, kb, st), al = across(sGl, cb, kb, st);
        Y[cb] = mfma32(ah, skh[kb][st], Y[cb]);
        Y[cb] = mfma32(ah, skl[kb][st], Y[cb]);
        Y[cb] = mfma32(al, skh[kb][st], Y[cb]);
      }
  }
  // dv += Y (four consecutive columns per register group).
  if (rvalid) {
#pragma unroll
    for (int cb = 0; cb < NC; ++cb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float4 *p = reinterpret_cast<float4 *>(dv + roff + 32 * cb + 8 * r4 + 4 * g);
        float4 x = *p;
        x.x += Y[cb][4 * r4];
        x.y += Y[cb][4 * r4 + 1];
        x.z += Y[cb][4 * r4 + 2];
        x.w += Y[cb][4 * r4 + 3];
        *p = x;
      }
  }

  // B operands of dsk^T, contraction over c: W^T and -(Y / denk)^T (delta),
  // or v^T (linear), from this lane's result registers.
  bf16x8 bwh[NC][2], bwl[NC][2], byh[NC][2], byl[NC][2];
  float ddenk = 0.f;
  if (delta) {
    // nk^T = Mp^T sk^T (A = M_{s-1}^T along rows).
    float yn = 0.f;
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
      f32x16 nk = zero16();
#pragma unroll
      for (int kb = 0; kb < NC; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const bf16x8 ah = along(sMh, cb, kb, st), al = along(sMl, cb, kb, st);
          nk = mfma32(ah, skh[kb][st], nk);
          nk = mfma32(ah, skl[kb][st], nk);
          nk = mfma32(al, skh[kb][st], nk);
        }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float vx[8], wx[8], yx[8];
        unpack8(row8(v, cb, st), vx);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float nki = nk[8 * st + i], yi = Y[cb][8 * st + i];
          yn += yi * nki;
          wx[i] = vx[i] - nki / denk;
          yx[i] = -(yi / denk);
        }
        split_bf16x8(wx, bwh[cb][st], bwl[cb][st]);
        split_bf16x8(yx, byh[cb][st], byl[cb][st]);
      }
    }
    ddenk = sum_xor32(yn) / (denk * denk);
  } else {
#pragma unroll
    for (int cb = 0; cb < NC; ++cb)
#pragma unroll
      for (int st = 0; st < 2; ++st) bwh[cb][st] = __builtin_bit_cast(bf16x8, row8(v, cb, st));
  }

  // dsk^T = gM W^T - Mp (Y / denk)^T (A = gM along rows, Mp = (M^T)^T over rows).
#pragma unroll
  for (int cb = 0; cb < NC; ++cb) {
    f32x16 ds = zero16();
#pragma unroll
    for (int kb = 0; kb < NC; ++kb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8 gh = along(sGh, cb, kb, st), gl = along(sGl, cb, kb, st);
        ds = mfma32(gh, bwh[kb][st], ds);
        ds = mfma32(gl, bwh[kb][st], ds);
        if (delta) {
          ds = mfma32(gh, bwl[kb][st], ds);
          const bf16x8 mh = across(sMh, cb, kb, st), ml = across(sMl, cb, kb, st);
          ds = mfma32(mh, byh[kb][st], ds);
          ds = mfma32(mh, byl[kb][st], ds);
          ds = mfma32(ml, byh[kb][st], ds);
        }
      }
    // dk += (dsk + ddenk zp) sigma'(k).
    if (rvalid) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int c = 32 * cb + 8 * r4 + 4 * g;
        float4 *p = reinterpret_cast<float4 *>(dk + roff + c);
        float4 x = *p;
        float gr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          gr[i] = (ds[4 * r4 + i] + (delta ? ddenk * sZ[c + i] : 0.f)) *
                  elu1_grad_from(skv[cb][4 * r4 + i]);
        x.x += gr[0];
        x.y += gr[1];
        x.z += gr[2];
        x.w += gr[3];
        *p = x;
      }
    }
  }

  if (delta) {
    // qz_s partial over the workgroup's rows, added in row order: the gM
    // tiles' LDS (no longer read) holds sk * ddenk row by row.
    float (*sQ)[D + 1] = reinterpret_cast<float (*)[D + 1]>(&sGh[0][0]);
    __syncthreads();  // every wave is done with the tiles
#pragma unroll
    for (int cb = 0; cb < NC; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sQ[32 * w + l32][32 * cb + kappa(i, g)] = skv[cb][i] * ddenk;
    __syncthreads();
    if (t < D) {
      float acc = 0.f;
      for (int rr = 0; rr < RW; ++rr) acc += sQ[rr][t];
      qzp[t] = acc;
    }
  }
}

// The same update on the vector ALUs (d < 128: the matrix-core version
// would leave waves idle with fewer than four 32-column blocks).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_update_valu_kernel(
    const T *__restrict__ k, const T *__restrict__ v, const float *__restrict__ mt,
    const float *__restrict__ zpre, const float *__restrict__ gma, int L, int N, int S, float eps,
    int delta, float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ qz_part) {
  constexpr int P = D + 1;
  constexpr int NJ = D / 16;
  __shared__ float sK[kKT][P];  // sigma(k)
  __shared__ float sV[kKT][P];  // v, then W = v - numk / denk
  __shared__ float sY[kKT][P];  // Y / denk
  __shared__ float sB[kKT][P];  // chunk of gM_s or Mp
  __shared__ float sZ[D];
  __shared__ float sDen[kKT], sDd[kKT];

  const int t = threadIdx.x, r0 = t >> 4, c0 = t & 15;
  const int s = blockIdx.y, kvh = blockIdx.z;
  const int a = s * N, e = min(a + N, L);
  const int i0 = a + blockIdx.x * kKT;
  const size_t unit = static_cast<size_t>(kvh) * S + s;
  // This chunk's partial of qz_s (delta rule), summed in chunk order later.
  float *qzp = qz_part + (unit * gridDim.x + blockIdx.x) * D;
  if (i0 >= e) {
    if (delta)
      for (int c = t; c < D; c += kThreads) qzp[c] = 0.f;
    return;
  }
  const int rows = min(kKT, e - i0);
  const size_t row0 = static_cast<size_t>(kvh) * L + i0;
  const float *gm = gma + unit * D * D;
  const float *mtp = mt + unit * D * D;
  load_rows<T, D, P>(sK, k + row0 * D, kKT, rows, true);
  load_rows<T, D, P>(sV, v + row0 * D, kKT, rows, false);
  for (int c = t; c < D; c += kThreads) sZ[c] = zpre[(static_cast<size_t>(kvh) * (S + 1) + s) * D + c];

  // Y = sk gM_s.
  float Y[2][NJ];
  zero(Y);
  for (int k0 = 0; k0 < D; k0 += kKT) {
    __syncthreads();
    for (int idx = t; idx < kKT * D; idx += kThreads) {
      const int kk = idx / D, c = idx % D;
      sB[kk][c] = gm[static_cast<size_t>(k0 + kk) * D + c];
    }
    __syncthreads();
    mm16<2, NJ>(Y, kKT, [&](int r, int kk) { return sK[r][k0 + kk]; },
                [&](int kk, int c) { return sB[kk][c]; });
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = r0 + 16 * i;
    if (r >= rows) continue;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) dv[(row0 + r) * D + c0 + 16 * jj] += Y[i][jj];
  }

  float ddk[2] = {0.f, 0.f};
  if (delta) {
    float nk[2][NJ];
    zero(nk);
    for (int k0 = 0; k0 < D; k0 += kKT) {
      __syncthreads();
      for (int idx = t; idx < kKT * D; idx += kThreads) {
        const int kk = idx % kKT, jc = idx / kKT;  // sB[kk][jc] = Mp[k0 + kk][jc] = mt[jc][k0 + kk]
        sB[kk][jc] = mtp[static_cast<size_t>(jc) * D + k0 + kk];
      }
      __syncthreads();
      mm16<2, NJ>(nk, kKT, [&](int r, int kk) { return sK[r][k0 + kk]; },
                  [&](int kk, int c) { return sB[kk][c]; });
    }
    if (t < kKT) {
      float d = eps;
      for (int c = 0; c < D; ++c) d += sK[t][c] * sZ[c];
      sDen[t] = d;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = r0 + 16 * i;
      const float den = sDen[r];
      float part = 0.f;
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        const int c = c0 + 16 * jj;
        part += Y[i][jj] * nk[i][jj];
        sV[r][c] -= nk[i][jj] / den;  // owner-only element
        sY[r][c] = Y[i][jj] / den;
      }
      ddk[i] = sum16(part) / (den * den);
      if (c0 == 0) sDd[r] = r < rows ? ddk[i] : 0.f;
    }
    __syncthreads();
    if (t < D) {
      float acc = 0.f;
      for (int r = 0; r < kKT; ++r) acc += sK[r][t] * sDd[r];
      qzp[t] = acc;
    }
  }

  // dsk = W gM_s^T (linear: v gM_s^T) - (Y / denk) Mp^T + ddenk zp.
  float dsk[2][NJ];
  zero(dsk);
  for (int j0 = 0; j0 < D; j0 += kKT) {
    __syncthreads();
    for (int idx = t; idx < kKT * D; idx += kThreads) {
      const int jj = idx % kKT, c = idx / kKT;  // sB[jj][c] = gM_s[c][j0 + jj]
      sB[jj][c] = gm[static_cast<size_t>(c) * D + j0 + jj];
    }
    __syncthreads();
    mm16<2, NJ>(dsk, kKT, [&](int r, int kk) { return sV[r][j0 + kk]; },
                [&](int kk, int c) { return sB[kk][c]; });
  }
  if (delta) {
    for (int j0 = 0; j0 < D; j0 += kKT) {
      __syncthreads();
      for (int idx = t; idx < kKT * D; idx += kThreads) {
        const int jj = idx / D, c = idx % D;  // sB[jj][c] = Mp[c][j0 + jj] = mt[j0 + jj][c]
        sB[jj][c] = mtp[static_cast<size_t>(j0 + jj) * D + c];
      }
      __syncthreads();
      mm16<2, NJ>(dsk, kKT, [&](int r, int kk) { return -sY[r][j0 + kk]; },
                  [&](int kk, int c) { return sB[kk][c]; });
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = r0 + 16 * i;
    if (r >= rows) continue;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int c = c0 + 16 * jj;
      const float g = dsk[i][jj] + (delta ? ddk[i] * sZ[c] : 0.f);
      dk[(row0 + r) * D + c] += g * elu1_grad_from(sK[r][c]);
    }
  }
}

// ---------------------------------------------------------------------------
// z chain: gz backwards over the segments; one thread per state row.
__global__ void bwd_gz_chain_kernel(const float *__restrict__ rvec, const float *__restrict__ qz,
                                    const float *__restrict__ dz, int S, int D,
                                    float *__restrict__ gza, float *__restrict__ dz0) {
  const size_t kvh = blockIdx.x;
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    float g = dz ? dz[kvh * D + c] : 0.f;
    for (int s = S - 1; s >= 0; --s) {
      const size_t o = (kvh * S + s) * D + c;
      gza[o] = g;
      g += rvec[o] + qz[o];
    }
    dz0[kvh * D + c] = g;
  }
}

// dk += gz_s sigma'(k) for every row of segment s, four consecutive
// elements per thread (D is a multiple of 4, so they share a row).
template <typename T>
__global__ void bwd_dk_gz_kernel(const T *__restrict__ k, const float *__restrict__ gza, int L,
                                 int N, int S, int D, size_t total4, float *__restrict__ dk) {
  const size_t idx4 = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx4 >= total4) return;
  const size_t idx = 4 * idx4;
  const int c = static_cast<int>(idx % D);
  const size_t row = idx / D;
  const size_t kvh = row / L;
  const int i = static_cast<int>(row % L);
  const int s = i / N;
  float kv[4];
  if constexpr (std::is_same<T, uint16_t>::value) {
    const u32x2 w2 = *reinterpret_cast<const u32x2 *>(reinterpret_cast<const uint16_t *>(k) + idx);
    kv[0] = lo_bf16(w2[0]);
    kv[1] = hi_bf16(w2[0]);
    kv[2] = lo_bf16(w2[1]);
    kv[3] = hi_bf16(w2[1]);
  } else {
    const float4 f = *reinterpret_cast<const float4 *>(k + idx);
    kv[0] = f.x;
    kv[1] = f.y;
    kv[2] = f.z;
    kv[3] = f.w;
  }
  const float4 gz = *reinterpret_cast<const float4 *>(gza + (kvh * S + s) * D + c);
  const float gv[4] = {gz.x, gz.y, gz.z, gz.w};
  float4 *p = reinterpret_cast<float4 *>(dk + idx);
  float4 x = *p;
  float r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = gv[j] * (kv[j] > 0.f ? 1.f : __expf(kv[j]));
  x.x += r[0];
  x.y += r[1];
  x.z += r[2];
  x.w += r[3];
  *p = x;
}

// Sum the per-block partials of `units` units in block order (see
// bwd_sum_parts_kernel).
hipError_t sum_parts(const float *part, size_t units, int nblk, int mat, int vec, float *out_mat,
                     float *out_vec, hipStream_t st) {
  if (units == 0) return hipSuccess;
  if (units > 0x7fffffffu) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(units), (mat + vec + kThreads - 1) / kThreads);
  bwd_sum_parts_kernel<<<grid, kThreads, 0, st>>>(part, nblk, mat, vec, out_mat, out_vec);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_t(const Geometry &g, const T *q, const T *k, const T *v, const T *dout,
                        const float *beta, const float *M0, const float *z0, const float *dM,
                        const float *dz, int delta, const BwdWorkspace &w, float *dq, float *dk,
                        float *dv, float *dbeta, float *dM0, float *dz0, hipStream_t st) {
  const int grp = g.Hq / g.Hkv;
  const int kvheads = g.B * g.Hkv;
  const size_t units = static_cast<size_t>(kvheads) * g.S;
  const BwdBlocks nb = backward_blocks(g);
  if ((static_cast<long long>(grp) * g.N + nb.rows_per - 1) / nb.rows_per > 0x7fffffffLL)
    return hipErrorInvalidConfiguration;
  // The forward's state before every segment: z prefix, then G_s (delta) and
  // H_s in parallel, then the d x d chain.
  bwd_zsum_kernel<T, D><<<dim3(g.S, kvheads), kZsumThreads, 0, st>>>(k, g.L, g.N, g.S, w.dzs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_zprefix_kernel<<<kvheads, D, 0, st>>>(w.dzs, z0, g.S, D, w.z_pre);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (delta) {
    bwd_outer_kernel<T, D, 1><<<dim3(nb.rows, g.S, kvheads), kThreads, 0, st>>>(
        k, nullptr, nullptr, nullptr, w.z_pre, g.Hq, g.Hkv, g.L, g.N, g.S, g.eps, nb.rows_per,
        w.part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = sum_parts(w.part, units, nb.rows, D * D, 0, w.G, nullptr, st)) != hipSuccess)
      return e;
  }
  bwd_outer_kernel<T, D, 2><<<dim3(nb.rows, g.S, kvheads), kThreads, 0, st>>>(
      k, v, nullptr, nullptr, w.z_pre, g.Hq, g.Hkv, g.L, g.N, g.S, g.eps, nb.rows_per, w.part);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = sum_parts(w.part, units, nb.rows, D * D, 0, w.H, nullptr, st)) != hipSuccess) return e;
  bwd_gm_chain_kernel<D, true><<<dim3(D / kKT, kvheads), kThreads, 0, st>>>(w.H, w.G, M0, g.S,
                                                                           delta, w.mt, nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if constexpr (std::is_same<T, uint16_t>::value) {
    bwd_query_kernel<T, D, 1><<<dim3(nb.qblocks, g.S, g.B * g.Hq), kThreads, 0, st>>>(
        q, k, v, dout, beta, w.mt, w.z_pre, g.Hq, g.Hkv, g.L, g.N, g.S, g.eps, dq, w.lse, w.erow,
        w.gd, w.dden, w.dbeta_part);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    bwd_query_kernel<T, D, 2><<<dim3(nb.qblocks, g.S, g.B * g.Hq), kThreads, 0, st>>>(
        q, k, v, dout, beta, w.mt, w.z_pre, g.Hq, g.Hkv, g.L, g.N, g.S, g.eps, dq, w.lse, w.erow,
        w.gd, w.dden, w.dbeta_part);
  } else {
    bwd_query_kernel<T, D, 0><<<dim3(nb.qblocks, g.S, g.B * g.Hq), kThreads, 0, st>>>(
        q, k, v, dout, beta, w.mt, w.z_pre, g.Hq, g.Hkv, g.L, g.N, g.S, g.eps, dq, w.lse, w.erow,
        w.gd, w.dden, w.dbeta_part);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = sum_parts(w.dbeta_part, g.Hq, g.B * g.S * nb.qblocks, 1, 0, dbeta, nullptr, st)) !=
      hipSuccess)
    return e;
  bwd_key_kernel<T, D><<<dim3(nb.qblocks, g.S, kvheads), kThreads, 0, st>>>(
      q, k, v, dout, beta, w.lse, w.erow, g.Hq, g.Hkv, g.L, g.N, dk, dv);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_outer_kernel<T, D, 0><<<dim3(nb.group_rows, g.S, kvheads), kThreads, 0, st>>>(
      q, dout, w.gd, w.dden, w.z_pre, g.Hq, g.Hkv, g.L, g.N, g.S, g.eps, nb.rows_per, w.part);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = sum_parts(w.part, units, nb.group_rows, D * D, D, w.R, w.r, st)) != hipSuccess)
    return e;
  bwd_gm_chain_kernel<D, false><<<dim3(D / kKT, kvheads), kThreads, 0, st>>>(w.R, w.G, dM, g.S, delta,
                                                                      w.gma, dM0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // Blocks of qz_s partials per unit: 128-row blocks on the matrix-core
  // path for bf16 storage at d = 128, 32-row chunks otherwise.
  int upd_blocks = nb.chunks;
  if constexpr (D == 128 && std::is_same<T, uint16_t>::value) {
    upd_blocks = nb.qblocks;
    bwd_update_mfma_kernel<D><<<dim3(nb.qblocks, g.S, kvheads), kThreads, 0, st>>>(
        k, v, w.mt, w.z_pre, w.gma, g.L, g.N, g.S, g.eps, delta, dk, dv, w.qz_part);
  } else if constexpr (D == 128) {
    bwd_update_kernel<T, D><<<dim3(nb.chunks, g.S, kvheads), kThreads, 0, st>>>(
        k, v, w.mt, w.z_pre, w.gma, g.L, g.N, g.S, g.eps, delta, dk, dv, w.qz_part);
  } else {
    bwd_update_valu_kernel<T, D><<<dim3(nb.chunks, g.S, kvheads), kThreads, 0, st>>>(
        k, v, w.mt, w.z_pre, w.gma, g.L, g.N, g.S, g.eps, delta, dk, dv, w.qz_part);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (delta && (e = sum_parts(w.qz_part, units, upd_blocks, D, 0, w.qz, nullptr, st)) != hipSuccess)
    return e;
  bwd_gz_chain_kernel<<<kvheads, D, 0, st>>>(w.r, w.qz, dz, g.S, D, w.gza, dz0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t total4 = static_cast<size_t>(kvheads) * g.L * D / 4;
  const size_t blocks = (total4 + 255) / 256;
  bwd_dk_gz_kernel<T><<<static_cast<unsigned>(blocks), 256, 0, st>>>(k, w.gza, g.L, g.N, g.S, D,
                                                                      total4, dk);
  return hipGetLastError();
}

}  // namespace

BwdBlocks backward_blocks(const Geometry &g) {
  BwdBlocks nb;
  nb.rows_per = 1024;
  nb.rows = (g.N + nb.rows_per - 1) / nb.rows_per;
  nb.group_rows = static_cast<int>(
      (static_cast<long long>(g.Hq / g.Hkv) * g.N + nb.rows_per - 1) / nb.rows_per);
  nb.qblocks = (g.N + 127) / 128;
  nb.chunks = (g.N + kKT - 1) / kKT;
  return nb;
}

template <typename T>
hipError_t launch_backward(const Geometry &g, const T *q, const T *k, const T *v, const T *dout,
                           const float *beta, const float *M0, const float *z0, const float *dM,
                           const float *dz, int delta, const BwdWorkspace &w, float *dq, float *dk,
                           float *dv, float *dbeta, float *dM0, float *dz0, hipStream_t stream) {
  switch (g.D) {
    case 32:
      return launch_bwd_t<T, 32>(g, q, k, v, dout, beta, M0, z0, dM, dz, delta, w, dq, dk, dv,
                                 dbeta, dM0, dz0, stream);
    case 64:
      return launch_bwd_t<T, 64>(g, q, k, v, dout, beta, M0, z0, dM, dz, delta, w, dq, dk, dv,
                                 dbeta, dM0, dz0, stream);
    case 128:
      return launch_bwd_t<T, 128>(g, q, k, v, dout, beta, M0, z0, dM, dz, delta, w, dq, dk, dv,
                                  dbeta, dM0, dz0, stream);
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_backward<float>(const Geometry &, const float *, const float *,
                                           const float *, const float *, const float *,
                                           const float *, const float *, const float *,
                                           const float *, int, const BwdWorkspace &,
                                           float *, float *, float *, float *, float *, float *,
                                           hipStream_t);
template hipError_t launch_backward<uint16_t>(const Geometry &, const uint16_t *, const uint16_t *,
                                              const uint16_t *, const uint16_t *, const float *,
                                              const float *, const float *, const float *,
                                              const float *, int,
                                              const BwdWorkspace &, float *, float *, float *,
                                              float *, float *, float *, hipStream_t);

}  // namespace ia
