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
// The work splits into parts that are independent per segment and two short
// chains that run backwards over the segments:
//   query  per (b, q head, segment, 64 query rows): the local attention's dQ
//          (softmax backward with the row statistics recomputed), the
//          retrieval backward (dnum = g dO / den, dden = -g sum(dO num) / den^2,
//          dq += (dnum Mp^T + dden zp) sigma'(q)) and the gate's d beta;
//   key    per (b, kv head, segment, 32 keys): the local attention's dK, dV
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

#include "common.h"
#include "launch.h"

namespace ia {
namespace {

constexpr int kThreads = 256;
constexpr int kQT = 64;  // query rows per tile
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

__device__ __forceinline__ float max16(float x) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, 16));
  return x;
}

__device__ __forceinline__ float gate(float beta) { return 1.f / (1.f + expf(-beta)); }

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
// query: dq, the softmax row statistics (lse, E) and dnum / dden for the
// outer products, and the gate's contribution to d beta.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_query_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ dout, const float *__restrict__ beta, const float *__restrict__ mt,
    const float *__restrict__ zpre, int Hq, int Hkv, int L, int N, int S, float eps,
    float *__restrict__ dq, float *__restrict__ lse_out, float *__restrict__ e_out,
    float *__restrict__ dnum_out, float *__restrict__ dden_out, float *__restrict__ dbeta) {
  constexpr int P = D + 1;
  constexpr int NJ = D / 16;
  __shared__ float sQ[kQT][P];   // q rows; sigma(q) for the retrieval part
  __shared__ float sO[kQT][P];   // d_out rows; dnum for the retrieval part
  __shared__ float sK[kKT][P];   // key tile, then chunks of the state
  __shared__ float sV[kKT][P];   // value tile
  __shared__ float sP[kQT][kKT + 1];
  __shared__ float sZ[D];
  __shared__ float sDen[kQT];
  __shared__ float sAcc;

  const int t = threadIdx.x, r0 = t >> 4, c0 = t & 15;
  const int s = blockIdx.y, bh = blockIdx.z;
  const int b = bh / Hq, h = bh % Hq;
  const int grp = Hq / Hkv;
  const size_t kvh = static_cast<size_t>(b) * Hkv + h / grp;
  const int a = s * N, e = min(a + N, L);
  const int i0 = a + blockIdx.x * kQT;
  if (i0 >= e) return;
  const int rows = min(kQT, e - i0);
  const int kend = min(i0 + kQT, e);  // keys this tile's rows can see: [a, kend)
  const float gam = gate(beta[h]);
  const float scale = 1.f / sqrtf(static_cast<float>(D));

  const size_t qrow0 = static_cast<size_t>(bh) * L + i0;
  load_rows<T, D, P>(sQ, q + qrow0 * D, kQT, rows, false);
  load_rows<T, D, P>(sO, dout + qrow0 * D, kQT, rows, false);
  if (t == 0) sAcc = 0.f;
  const T *kb = k + kvh * L * D;
  const T *vb = v + kvh * L * D;

  auto qk = [&](float (&sc)[4][2]) {
    zero(sc);
    mm16<4, 2>(sc, D, [&](int r, int kk) { return sQ[r][kk]; },
               [&](int kk, int c) { return sK[c][kk]; });
  };
  auto ov = [&](float (&o)[4][2]) {
    zero(o);
    mm16<4, 2>(o, D, [&](int r, int kk) { return sO[r][kk]; },
               [&](int kk, int c) { return sV[c][kk]; });
  };
  auto visible = [&](int i, int jj, int j0) {
    const int row = i0 + r0 + 16 * i, col = j0 + c0 + 16 * jj;
    return col <= row && col < e;
  };

  // Pass 1: row max and sum of the causal softmax -> lse.
  float m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
  }
  for (int j0 = a; j0 < kend; j0 += kKT) {
    __syncthreads();
    load_rows<T, D, P>(sK, kb + static_cast<size_t>(j0) * D, kKT, kend - j0, false);
    __syncthreads();
    float sc[4][2];
    qk(sc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x0 = visible(i, 0, j0) ? sc[i][0] * scale : -INFINITY;
      float x1 = visible(i, 1, j0) ? sc[i][1] * scale : -INFINITY;
      const float mn = fmaxf(m[i], max16(fmaxf(x0, x1)));
      const float add = sum16(__expf(x0 - mn) + __expf(x1 - mn));
      l[i] = l[i] * __expf(m[i] - mn) + add;
      m[i] = mn;
    }
  }
  float lse[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lse[i] = m[i] + __logf(l[i]);

  // Pass 2: E_i = sum_j P_ij (dO_i . v_j), i.e. dO_i . A_dot_i.
  float ep[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = a; j0 < kend; j0 += kKT) {
    __syncthreads();
    load_rows<T, D, P>(sK, kb + static_cast<size_t>(j0) * D, kKT, kend - j0, false);
    load_rows<T, D, P>(sV, vb + static_cast<size_t>(j0) * D, kKT, kend - j0, false);
    __syncthreads();
    float sc[4][2], o[4][2];
    qk(sc);
    ov(o);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        if (visible(i, jj, j0)) ep[i] += __expf(sc[i][jj] * scale - lse[i]) * o[i][jj];
  }
  float E[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) E[i] = sum16(ep[i]);

  // Pass 3: dS = (1 - g) P (dO V^T - E), dq_attn = scale dS K.
  float acc[4][NJ];
  zero(acc);
  for (int j0 = a; j0 < kend; j0 += kKT) {
    __syncthreads();
    load_rows<T, D, P>(sK, kb + static_cast<size_t>(j0) * D, kKT, kend - j0, false);
    load_rows<T, D, P>(sV, vb + static_cast<size_t>(j0) * D, kKT, kend - j0, false);
    __syncthreads();
    float sc[4][2], o[4][2];
    qk(sc);
    ov(o);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const float p = visible(i, jj, j0) ? __expf(sc[i][jj] * scale - lse[i]) : 0.f;
        sP[r0 + 16 * i][c0 + 16 * jj] = (1.f - gam) * p * (o[i][jj] - E[i]);
      }
    __syncthreads();
    mm16<4, NJ>(acc, kKT, [&](int r, int kk) { return sP[r][kk]; },
                [&](int kk, int c) { return sK[kk][c]; });
  }

  // Retrieval backward from the pre-segment snapshot (Mp^T in mt, zp in zpre).
  const size_t unit = kvh * S + s;
  const float *mtp = mt + unit * D * D;
  __syncthreads();
  for (int idx = t; idx < kQT * D; idx += kThreads) {
    const int r = idx / D, c = idx % D;
    sQ[r][c] = r < rows ? elu1(sQ[r][c]) : 0.f;
  }
  for (int c = t; c < D; c += kThreads) sZ[c] = zpre[(kvh * (S + 1) + s) * D + c];
  float num[4][NJ];
  zero(num);
  for (int k0 = 0; k0 < D; k0 += kKT) {
    __syncthreads();
    for (int idx = t; idx < kKT * D; idx += kThreads) {
      const int kk = idx % kKT, j = idx / kKT;  // sK[kk][j] = Mp[k0 + kk][j] = mt[j][k0 + kk]
      sK[kk][j] = mtp[static_cast<size_t>(j) * D + k0 + kk];
    }
    __syncthreads();
    mm16<4, NJ>(num, kKT, [&](int r, int kk) { return sQ[r][k0 + kk]; },
                [&](int kk, int c) { return sK[kk][c]; });
  }
  if (t < kQT) {
    float d = eps;
    for (int c = 0; c < D; ++c) d += sQ[t][c] * sZ[c];
    sDen[t] = d;
  }
  __syncthreads();
  float dden[4];
  float mem_dot = 0.f;  // sum over this thread's rows of dO . A_mem (lanes c0 == 0)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + 16 * i;
    const float den = sDen[r];
    float part = 0.f;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) part += sO[r][c0 + 16 * jj] * num[i][jj];
    const float s1 = sum16(part);  // dO_i . num_i
    dden[i] = -gam * s1 / (den * den);
    if (c0 == 0 && r < rows) mem_dot += s1 / den;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int c = c0 + 16 * jj;
      const float dn = gam * sO[r][c] / den;
      sO[r][c] = dn;  // each element is read and written by its owner only
      if (r < rows) dnum_out[(qrow0 + r) * D + c] = dn;
    }
    if (c0 == 0 && r < rows) {
      dden_out[qrow0 + r] = dden[i];
      lse_out[qrow0 + r] = lse[i];
      e_out[qrow0 + r] = E[i];
    }
  }
  float dsq[4][NJ];
  zero(dsq);
  for (int j0 = 0; j0 < D; j0 += kKT) {
    __syncthreads();
    for (int idx = t; idx < kKT * D; idx += kThreads) {
      const int jj = idx / D, c = idx % D;  // sK[jj][c] = Mp[c][j0 + jj] = mt[j0 + jj][c]
      sK[jj][c] = mtp[static_cast<size_t>(j0 + jj) * D + c];
    }
    __syncthreads();
    mm16<4, NJ>(dsq, kKT, [&](int r, int kk) { return sO[r][j0 + kk]; },
                [&](int kk, int c) { return sK[kk][c]; });
  }
  float att_dot = 0.f;  // sum over this thread's rows of dO . A_dot = E (lanes c0 == 0)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = r0 + 16 * i;
    if (r >= rows) continue;
    if (c0 == 0) att_dot += E[i];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int c = c0 + 16 * jj;
      const float g = acc[i][jj] * scale + (dsq[i][jj] + dden[i] * sZ[c]) * elu1_grad_from(sQ[r][c]);
      dq[(qrow0 + r) * D + c] = g;
    }
  }
  // d beta: sum over rows of dO . (A_mem - A_dot), times g (1 - g).
  const float contrib = mem_dot - att_dot;
  if (contrib != 0.f) atomicAdd(&sAcc, contrib);
  __syncthreads();
  if (t == 0) atomicAdd(dbeta + h, sAcc * gam * (1.f - gam));
}

// ---------------------------------------------------------------------------
// key: dK, dV of the local attention for 32 keys of one segment, over every
// query head of the kv group and every query row at or after the keys.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_key_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ dout, const float *__restrict__ beta, const float *__restrict__ lse,
    const float *__restrict__ E, int Hq, int Hkv, int L, int N, float *__restrict__ dk,
    float *__restrict__ dv) {
  constexpr int P = D + 1;
  constexpr int NJ = D / 16;
  __shared__ float sK[kKT][P];
  __shared__ float sV[kKT][P];
  __shared__ float sQ[kQT][P];
  __shared__ float sO[kQT][P];
  __shared__ float sPt[kKT][kQT + 1];  // (1 - g) P^T
  __shared__ float sSt[kKT][kQT + 1];  // dS^T
  __shared__ float sL[kQT], sE[kQT];

  const int t = threadIdx.x, r0 = t >> 4, c0 = t & 15;
  const int s = blockIdx.y, kvh = blockIdx.z;
  const int b = kvh / Hkv, j = kvh % Hkv;
  const int grp = Hq / Hkv;
  const int a = s * N, e = min(a + N, L);
  const int j0 = a + blockIdx.x * kKT;
  if (j0 >= e) return;
  const int keys = min(kKT, e - j0);
  const float scale = 1.f / sqrtf(static_cast<float>(D));
  const size_t krow0 = static_cast<size_t>(kvh) * L + j0;
  load_rows<T, D, P>(sK, k + krow0 * D, kKT, keys, false);
  load_rows<T, D, P>(sV, v + krow0 * D, kKT, keys, false);

  float gk[2][NJ], gv[2][NJ];
  zero(gk);
  zero(gv);
  for (int hl = 0; hl < grp; ++hl) {
    const int h = j * grp + hl;
    const float gam = gate(beta[h]);
    const size_t hrow = (static_cast<size_t>(b) * Hq + h) * L;
    for (int i0 = j0; i0 < e; i0 += kQT) {
      const int rows = min(kQT, e - i0);
      __syncthreads();
      load_rows<T, D, P>(sQ, q + (hrow + i0) * D, kQT, rows, false);
      load_rows<T, D, P>(sO, dout + (hrow + i0) * D, kQT, rows, false);
      if (t < kQT) {
        sL[t] = t < rows ? lse[hrow + i0 + t] : 0.f;
        sE[t] = t < rows ? E[hrow + i0 + t] : 0.f;
      }
      __syncthreads();
      float st[2][4], ot[2][4];
      zero(st);
      zero(ot);
      mm16<2, 4>(st, D, [&](int r, int kk) { return sK[r][kk]; },
                 [&](int kk, int c) { return sQ[c][kk]; });
      mm16<2, 4>(ot, D, [&](int r, int kk) { return sV[r][kk]; },
                 [&](int kk, int c) { return sO[c][kk]; });
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = r0 + 16 * i, c = c0 + 16 * jj;
          const int key = j0 + r, row = i0 + c;
          const bool vis = key <= row && row < e && key < e;
          const float p = vis ? __expf(st[i][jj] * scale - sL[c]) : 0.f;
          sPt[r][c] = (1.f - gam) * p;
          sSt[r][c] = (1.f - gam) * p * (ot[i][jj] - sE[c]);
        }
      __syncthreads();
      mm16<2, NJ>(gv, kQT, [&](int r, int kk) { return sPt[r][kk]; },
                  [&](int kk, int c) { return sO[kk][c]; });
      mm16<2, NJ>(gk, kQT, [&](int r, int kk) { return sSt[r][kk]; },
                  [&](int kk, int c) { return sQ[kk][c]; });
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = r0 + 16 * i;
    if (r >= keys) continue;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const size_t o = (krow0 + r) * D + c0 + 16 * jj;
      dk[o] = gk[i][jj] * scale;
      dv[o] = gv[i][jj];
    }
  }
}

// ---------------------------------------------------------------------------
// outer: per (b, kv head, segment), out += A^T B over a range of rows.
//   kind 0 (R): rows = (query head of the group, row of the segment),
//               A = sigma(q), B = dnum; r_s = sum A^T dden as well.
//   kind 1 (G): rows = rows of the segment, A = sigma(k), B = sigma(k) / denk.
// out must be zeroed first; the row ranges of one unit add atomically.
template <typename T, int D, int KIND>
__global__ __launch_bounds__(kThreads) void bwd_outer_kernel(
    const T *__restrict__ x, const float *__restrict__ dnum, const float *__restrict__ dden,
    const float *__restrict__ zpre, int Hq, int Hkv, int L, int N, int S, float eps,
    int rows_per_block, float *__restrict__ out, float *__restrict__ rvec) {
  constexpr int P = D + 1;
  constexpr int MI = D / 16;
  __shared__ float sA[kKT][P];
  __shared__ float sB[kKT][P];
  __shared__ float sX[kKT];
  __shared__ float sZ[D];

  const int t = threadIdx.x, r0 = t >> 4, c0 = t & 15;
  const int s = blockIdx.y, kvh = blockIdx.z;
  const int b = kvh / Hkv, j = kvh % Hkv;
  const int grp = Hq / Hkv;
  const int a = s * N, n = min(a + N, L) - a;
  const int total = KIND == 0 ? grp * n : n;
  const int u0 = blockIdx.x * rows_per_block;
  const int u1 = min(u0 + rows_per_block, total);
  if (u0 >= u1) return;
  if (KIND == 1)
    for (int c = t; c < D; c += kThreads) sZ[c] = zpre[(static_cast<size_t>(kvh) * (S + 1) + s) * D + c];

  // Source row (of x, and of dnum / dden for kind 0) of unit row u.
  auto src_row = [&](int u) -> size_t {
    if (KIND == 0) {
      const int hl = u / n, i = a + u % n;
      return (static_cast<size_t>(b) * Hq + j * grp + hl) * L + i;
    }
    return static_cast<size_t>(kvh) * L + a + u;
  };

  float acc[MI][MI];
  zero(acc);
  float racc = 0.f;
  for (int c0u = u0; c0u < u1; c0u += kKT) {
    const int cnt = min(kKT, u1 - c0u);
    __syncthreads();
    for (int idx = t; idx < kKT * D; idx += kThreads) {
      const int r = idx / D, c = idx % D;
      float av = 0.f, bv = 0.f;
      if (r < cnt) {
        const size_t row = src_row(c0u + r);
        av = elu1(load_as_f32(x, row * D + c));
        bv = KIND == 0 ? dnum[row * D + c] : av;
      }
      sA[r][c] = av;
      sB[r][c] = bv;
    }
    if (KIND == 0 && t < kKT) sX[t] = t < cnt ? dden[src_row(c0u + t)] : 0.f;
    __syncthreads();
    if (KIND == 1) {
      if (t < kKT) {
        float d = eps;
        for (int c = 0; c < D; ++c) d += sA[t][c] * sZ[c];
        sX[t] = 1.f / d;
      }
      __syncthreads();
      mm16<MI, MI>(acc, kKT, [&](int r, int kk) { return sA[kk][r]; },
                   [&](int kk, int c) { return sB[kk][c] * sX[kk]; });
    } else {
      mm16<MI, MI>(acc, kKT, [&](int r, int kk) { return sA[kk][r]; },
                   [&](int kk, int c) { return sB[kk][c]; });
      if (t < D)
        for (int kk = 0; kk < kKT; ++kk) racc += sA[kk][t] * sX[kk];
    }
  }
  const size_t unit = static_cast<size_t>(kvh) * S + s;
  float *o = out + unit * D * D;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int jj = 0; jj < MI; ++jj) atomicAdd(o + (r0 + 16 * i) * D + c0 + 16 * jj, acc[i][jj]);
  if (KIND == 0 && t < D) atomicAdd(rvec + unit * D + t, racc);
}

// ---------------------------------------------------------------------------
// chain: gM backwards over the segments, 32 columns per workgroup (column c of
// gM_{s-1} depends on column c of gM_s only). Writes gM_s (the gradient of the
// state after segment s) for every s, and gM_0 into dM0.
template <int D>
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
  for (int s = S - 1; s >= 0; --s) {
    const size_t base = (kvh * S + s) * D * D;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        gma[base + (r0 + 16 * i) * D + col0 + c0 + 16 * jj] = g[i][jj];
    if (delta) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) sM[r0 + 16 * i][c0 + 16 * jj] = g[i][jj];
      float acc[MI][2];
      zero(acc);
      for (int k0 = 0; k0 < D; k0 += kKT) {
        __syncthreads();
        for (int idx = t; idx < kKT * D; idx += kThreads) {
          const int kk = idx % kKT, r = idx / kKT;
          sG[kk][r] = G[base + static_cast<size_t>(r) * D + k0 + kk];
        }
        __syncthreads();
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
      for (int jj = 0; jj < 2; ++jj) g[i][jj] += R[base + (r0 + 16 * i) * D + col0 + c0 + 16 * jj];
  }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) dM0[kvh * D * D + (r0 + 16 * i) * D + col0 + c0 + 16 * jj] = g[i][jj];
}

// ---------------------------------------------------------------------------
// update: the memory write's gradient into v and k (without the gz_s term,
// added once the z chain is done), and qz_s = sk^T ddenk for the delta rule.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_update_kernel(
    const T *__restrict__ k, const T *__restrict__ v, const float *__restrict__ mt,
    const float *__restrict__ zpre, const float *__restrict__ gma, int L, int N, int S, float eps,
    int delta, float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ qz) {
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
  if (i0 >= e) return;
  const int rows = min(kKT, e - i0);
  const size_t row0 = static_cast<size_t>(kvh) * L + i0;
  const size_t unit = static_cast<size_t>(kvh) * S + s;
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
      atomicAdd(qz + unit * D + t, acc);
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

// dk += gz_s sigma'(k) for every row of segment s.
template <typename T>
__global__ void bwd_dk_gz_kernel(const T *__restrict__ k, const float *__restrict__ gza, int L,
                                 int N, int S, int D, size_t total, float *__restrict__ dk) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int c = static_cast<int>(idx % D);
  const size_t row = idx / D;
  const size_t kvh = row / L;
  const int i = static_cast<int>(row % L);
  const int s = i / N;
  const float kv = load_as_f32(k, idx);
  const float sg = kv > 0.f ? 1.f : __expf(kv);
  dk[idx] += gza[(kvh * S + s) * D + c] * sg;
}

template <typename T, int D>
hipError_t launch_bwd_t(const Geometry &g, const T *q, const T *k, const T *v, const T *dout,
                        const float *beta, const float *dM, const float *dz, int delta,
                        const BwdWorkspace &w, float *dq, float *dk, float *dv, float *dbeta,
                        float *dM0, float *dz0, hipStream_t st) {
  const int grp = g.Hq / g.Hkv;
  const int kvheads = g.B * g.Hkv;
  bwd_query_kernel<T, D><<<dim3((g.N + kQT - 1) / kQT, g.S, g.B * g.Hq), kThreads, 0, st>>>(
      q, k, v, dout, beta, w.mt, w.z_pre, g.Hq, g.Hkv, g.L, g.N, g.S, g.eps, dq, w.lse, w.erow,
      w.dnum, w.dden, dbeta);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_key_kernel<T, D><<<dim3((g.N + kKT - 1) / kKT, g.S, kvheads), kThreads, 0, st>>>(
      q, k, v, dout, beta, w.lse, w.erow, g.Hq, g.Hkv, g.L, g.N, dk, dv);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int rows_r = 1024;
  bwd_outer_kernel<T, D, 0><<<dim3((grp * g.N + rows_r - 1) / rows_r, g.S, kvheads), kThreads, 0,
                              st>>>(q, w.dnum, w.dden, w.z_pre, g.Hq, g.Hkv, g.L, g.N, g.S, g.eps,
                                    rows_r, w.R, w.r);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (delta) {
    bwd_outer_kernel<T, D, 1><<<dim3((g.N + rows_r - 1) / rows_r, g.S, kvheads), kThreads, 0,
                                st>>>(k, nullptr, nullptr, w.z_pre, g.Hq, g.Hkv, g.L, g.N, g.S,
                                      g.eps, rows_r, w.G, nullptr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  bwd_gm_chain_kernel<D><<<dim3(D / kKT, kvheads), kThreads, 0, st>>>(w.R, w.G, dM, g.S, delta,
                                                                      w.gma, dM0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_update_kernel<T, D><<<dim3((g.N + kKT - 1) / kKT, g.S, kvheads), kThreads, 0, st>>>(
      k, v, w.mt, w.z_pre, w.gma, g.L, g.N, g.S, g.eps, delta, dk, dv, w.qz);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_gz_chain_kernel<<<kvheads, D, 0, st>>>(w.r, w.qz, dz, g.S, D, w.gza, dz0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t total = static_cast<size_t>(kvheads) * g.L * D;
  const size_t blocks = (total + 255) / 256;
  bwd_dk_gz_kernel<T><<<static_cast<unsigned>(blocks), 256, 0, st>>>(k, w.gza, g.L, g.N, g.S, D,
                                                                      total, dk);
  return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t launch_backward(const Geometry &g, const T *q, const T *k, const T *v, const T *dout,
                           const float *beta, const float *dM, const float *dz, int delta,
                           const BwdWorkspace &w, float *dq, float *dk, float *dv, float *dbeta,
                           float *dM0, float *dz0, hipStream_t stream) {
  switch (g.D) {
    case 32:
      return launch_bwd_t<T, 32>(g, q, k, v, dout, beta, dM, dz, delta, w, dq, dk, dv, dbeta, dM0,
                                 dz0, stream);
    case 64:
      return launch_bwd_t<T, 64>(g, q, k, v, dout, beta, dM, dz, delta, w, dq, dk, dv, dbeta, dM0,
                                 dz0, stream);
    case 128:
      return launch_bwd_t<T, 128>(g, q, k, v, dout, beta, dM, dz, delta, w, dq, dk, dv, dbeta,
                                  dM0, dz0, stream);
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_backward<float>(const Geometry &, const float *, const float *,
                                           const float *, const float *, const float *,
                                           const float *, const float *, int, const BwdWorkspace &,
                                           float *, float *, float *, float *, float *, float *,
                                           hipStream_t);
template hipError_t launch_backward<uint16_t>(const Geometry &, const uint16_t *, const uint16_t *,
                                              const uint16_t *, const uint16_t *, const float *,
                                              const float *, const float *, int,
                                              const BwdWorkspace &, float *, float *, float *,
                                              float *, float *, float *, hipStream_t);

}  // namespace ia
