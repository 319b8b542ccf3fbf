// Fused per-segment kernel, fp32 storage path (fp32 arithmetic throughout).
//
// For each (batch, query head, segment, 64-row query tile):
//   A_dot = causal softmax(Q K^T / sqrt(d_k)) V inside the segment
//           ([HF-repro] "Infini-Attention メカニズム", step Local Attention),
//   A_mem = sigma(Q) M_{s-1} / (sigma(Q) z_{s-1} + eps)   (step Memory Retrieval),
//   out   = g A_mem + (1 - g) A_dot, g = sigmoid(beta_h)  (step Integration).
// M_{s-1}, z_{s-1} are the snapshots the segment scan wrote for this segment.
//
// Layout: 256 threads = 64 query rows x 4 lanes; lane qd of a row owns the
// interleaved columns {4c + qd}, so the four lanes of a row read four adjacent
// LDS words (no bank conflicts) and the row's dot products are finished with
// two xor-shuffles. Online softmax over 64-row key tiles staged in LDS.

#include "common.h"
#include "launch.h"

namespace ia {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 64;  // query rows per workgroup
constexpr int kBN = 64;  // key rows per tile
constexpr int kKC = 32;  // state rows staged per retrieval chunk

template <int D>
__global__ __launch_bounds__(kThreads) void fused_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ beta, const float *__restrict__ z_pre,
    const float *__restrict__ mt_pre, float *__restrict__ out, Layout lq, Layout lkv, Layout lo,
    int Hq, int Hkv, int L, int N, int S, float eps) {
  constexpr int DQ = D / 4;
  constexpr int SA = kBN * D > kBM * (kKC + 1) ? kBN * D : kBM * (kKC + 1);
  __shared__ float sA[SA];       // K tile; later sigma(Q) chunk (row stride kKC + 1)
  __shared__ float sB[kBN * D];  // V tile; later M^T chunk
  __shared__ float sZ[D];

  const int t = threadIdx.x;
  const int row = t >> 2, qd = t & 3;
  const int s = blockIdx.y;
  const int bhq = blockIdx.z;
  const int b = bhq / Hq, h = bhq - b * Hq;
  const int hk = h / (Hq / Hkv);
  const int a = s * N;
  const int e = min(a + N, L);
  const int q0 = a + blockIdx.x * kBM;
  if (q0 >= e) return;  // short last segment: whole workgroup idle
  const int qi = q0 + row;
  const bool valid = qi < e;

  // Row i of this head's q, k, v at qp + i * lq.sr, kp / vp + i * lkv.sr.
  const float *qp = q + head_offset(lq, bhq, Hq);
  const long long kvoff = head_offset(lkv, b * Hkv + hk, Hkv);
  const float *kp = k + kvoff;
  const float *vp = v + kvoff;

  float qv[DQ], o[DQ];
#pragma unroll
  for (int c = 0; c < DQ; ++c) {
    qv[c] = valid ? qp[qi * lq.sr + 4 * c + qd] : 0.f;
    o[c] = 0.f;
  }
  const float scale = rsqrtf(static_cast<float>(D));
  float m = -INFINITY, l = 0.f;
  const int kv_end = min(q0 + kBM, e);

  for (int kv0 = a; kv0 < kv_end; kv0 += kBN) {
    __syncthreads();
    for (int idx = t; idx < kBN * D; idx += kThreads) {
      const int r = idx / D, c = idx % D;
      const bool in = kv0 + r < e;
      sA[idx] = in ? kp[(kv0 + r) * lkv.sr + c] : 0.f;
      sB[idx] = in ? vp[(kv0 + r) * lkv.sr + c] : 0.f;
    }
    __syncthreads();
    float sc[kBN];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kBN; ++j) {
      float p = 0.f;
#pragma unroll
      for (int c = 0; c < DQ; ++c) p += qv[c] * sA[j * D + 4 * c + qd];
      p += __shfl_xor(p, 1);
      p += __shfl_xor(p, 2);
      const int kj = kv0 + j;
      p = (kj > qi || kj >= e) ? -INFINITY : p * scale;
      sc[j] = p;
      mx = fmaxf(mx, p);
    }
    const float m_new = fmaxf(m, mx);  // finite: key a <= qi is always in the first tile
    const float alpha = __expf(m - m_new);
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < kBN; ++j) {
      sc[j] = __expf(sc[j] - m_new);
      psum += sc[j];
    }
    l = l * alpha + psum;
    m = m_new;
#pragma unroll
    for (int c = 0; c < DQ; ++c) o[c] *= alpha;
#pragma unroll
    for (int j = 0; j < kBN; ++j) {
#pragma unroll
      for (int c = 0; c < DQ; ++c) o[c] += sc[j] * sB[j * D + 4 * c + qd];
    }
  }

  // Retrieval from the pre-segment snapshot (M^T stored [d_v][d_k]).
  const size_t snap = (static_cast<size_t>(b) * Hkv + hk) * S + s;
  const float *mt = mt_pre + snap * D * D;
  const float *zs = z_pre + ((static_cast<size_t>(b) * Hkv + hk) * (S + 1) + s) * D;
  __syncthreads();
  if (t < D) sZ[t] = zs[t];
  __syncthreads();
  float den = 0.f;
#pragma unroll
  for (int c = 0; c < DQ; ++c) den += elu1(qv[c]) * sZ[4 * c + qd];
  den += __shfl_xor(den, 1);
  den += __shfl_xor(den, 2);
  den += eps;

  float am[DQ];
#pragma unroll
  for (int c = 0; c < DQ; ++c) am[c] = 0.f;
  for (int k0 = 0; k0 < D; k0 += kKC) {
    __syncthreads();
    // sigma(Q)[row][k0:k0+KC] and M^T[:, k0:k0+KC]
    for (int idx = t; idx < kBM * kKC; idx += kThreads) {
      const int r = idx / kKC, c = idx % kKC;
      const int qr = q0 + r;
      sA[r * (kKC + 1) + c] = (qr < e) ? elu1(qp[qr * lq.sr + k0 + c]) : 0.f;
    }
    for (int idx = t; idx < D * kKC; idx += kThreads) {
      const int jv = idx / kKC, c = idx % kKC;
      sB[c * D + jv] = mt[static_cast<size_t>(jv) * D + k0 + c];
    }
    __syncthreads();
    for (int c = 0; c < kKC; ++c) {
      const float sq = sA[row * (kKC + 1) + c];
#pragma unroll
      for (int cc = 0; cc < DQ; ++cc) am[cc] += sq * sB[c * D + 4 * cc + qd];
    }
  }

  const float gam = 1.f / (1.f + __expf(-beta[h]));
  const float inv_l = 1.f / l;
  if (valid) {
    float *op = out + head_offset(lo, bhq, Hq) + qi * lo.sr;
#pragma unroll
    for (int c = 0; c < DQ; ++c) op[4 * c + qd] = gam * (am[c] / den) + (1.f - gam) * (o[c] * inv_l);
  }
}

template <int D>
hipError_t launch_t(const Geometry &g, const float *q, const float *k, const float *v,
                    const float *beta, const Workspace &ws, float *out, hipStream_t stream) {
  dim3 grid((g.N + kBM - 1) / kBM, g.S, g.B * g.Hq);
  fused_f32_kernel<D><<<grid, kThreads, 0, stream>>>(q, k, v, beta, ws.z_pre, ws.mt_pre_f32, out,
                                                     g.lq, g.lkv, g.lo, g.Hq, g.Hkv, g.L, g.N,
                                                     g.S, g.eps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fused_f32(const Geometry &g, const float *q, const float *k, const float *v,
                            const float *beta, const Workspace &ws, float *out,
                            hipStream_t stream) {
  switch (g.D) {
    case 32: return launch_t<32>(g, q, k, v, beta, ws, out, stream);
    case 64: return launch_t<64>(g, q, k, v, beta, ws, out, stream);
    case 128: return launch_t<128>(g, q, k, v, beta, ws, out, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace ia
