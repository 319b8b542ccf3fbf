// Segment scan for fp32 storage: the only state that crosses segments is
// (M, z); this kernel carries it in fp32 through all S segments of every
// (batch, kv head) with fp32 VALU arithmetic throughout (the precision path;
// bf16 storage uses the MFMA scan).
//
//   [HF-repro] "Infini-Attention メカニズム", steps Memory Update and State
//   Transfer; [LNCB-review] "メモリの更新" (outer-product write; delta rule).
//
//   LINEAR: M_s = M_{s-1} + sigma(K_s)^T V_s
//   DELTA:  M_s = M_{s-1} + sigma(K_s)^T (V_s - sigma(K_s) M_{s-1} / (sigma(K_s) z_{s-1} + eps))
//   both:   z_s = z_{s-1} + sum_i sigma(k_i)
//
// Column j of M evolves using only column j of M and z (the delta rule's
// retrieval divides row-wise by a scalar that depends on z alone), so the
// columns are split over workgroups with no communication, and every column
// goes through the same operations in the same order whatever the split. Each
// workgroup owns CB columns of one (b, kv head), keeps them in registers, and
// walks the
// segments in order, R rows at a time. Before each segment it writes the
// pre-segment snapshot (M_{s-1} transposed, z_{s-1}) that the fused attention
// kernel reads for that segment's retrieval.

#include "common.h"
#include "launch.h"

namespace ia {
namespace {

constexpr int kThreads = 256;
constexpr int kR = 64;   // rows of a segment processed per chunk

// Columns of M per workgroup: as few as keep every thread busy (threads
// sharing one state row hold one column each), so that B * Hkv * D / CB
// workgroups fill the chip.
template <int D>
constexpr int scan_cols() { return kThreads / D > 4 ? kThreads / D : 4; }

template <typename T, int D, int kCB>
__global__ __launch_bounds__(kThreads) void segment_scan_kernel(
    const T *__restrict__ k, const T *__restrict__ v, Layout lkv, int Hkv,
    float *__restrict__ M, const float *__restrict__ z, int L, int N, int S, float eps, int delta,
    float *__restrict__ z_pre, float *__restrict__ mt_f32, uint16_t *__restrict__ mt_bf16) {
  static_assert(D <= kThreads && kThreads % D == 0 && D % kCB == 0, "tile shape");
  constexpr int JSTEP = kThreads / D;  // threads sharing one row k of the state
  constexpr int JPT = kCB / JSTEP;     // state columns per thread
  static_assert(JPT >= 1 && kCB % JSTEP == 0, "column split");
  constexpr int ISTEP = kThreads / kCB;

  __shared__ float sK[kR][D + 1];   // sigma(K) of the chunk (pad: conflict-free rows)
  __shared__ float sU[kR][kCB + 1]; // V columns of the chunk, then the write U
  __shared__ float sM[D][kCB + 1];  // M_{s-1}[:, c0:c0+CB]
  __shared__ float sZ[D];           // z_{s-1}
  __shared__ float sDen[kR];        // sigma(k_i) . z_{s-1} + eps

  const int t = threadIdx.x;
  const int cb = blockIdx.x;
  const int bh = blockIdx.y;  // b * Hkv + j
  const int c0 = cb * kCB;
  // Row i of this head's k, v starts i * lkv.sr elements after kb, vb.
  const T *kb = k + head_offset(lkv, bh, Hkv);
  const T *vb = v + head_offset(lkv, bh, Hkv);
  float *Mb = M + static_cast<size_t>(bh) * D * D;

  // Ownership: thread t holds state rows kk = t % D, columns c0 + j0 + JSTEP*r.
  const int kk = t % D;
  const int j0 = t / D;
  float m_reg[JPT];
#pragma unroll
  for (int r = 0; r < JPT; ++r) m_reg[r] = Mb[kk * D + c0 + j0 + JSTEP * r];
  float zval = z[static_cast<size_t>(bh) * D + kk];

  // The next chunk's K and V values are fetched into registers while the
  // current chunk is processed, so a chunk never waits on memory latency.
  constexpr int KPT = kR * D / kThreads;                  // K values per thread
  constexpr int VPT = (kR * kCB + kThreads - 1) / kThreads;  // V values per thread
  float pk[KPT], pv[VPT];
  auto fetch = [&](int i0, int rows) {
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int idx = t + r * kThreads, i = idx / D, c = idx % D;
      pk[r] = i < rows ? load_as_f32(kb, static_cast<size_t>((i0 + i) * lkv.sr + c)) : 0.f;
    }
#pragma unroll
    for (int r = 0; r < VPT; ++r) {
      const int idx = t + r * kThreads, i = idx / kCB, c = idx % kCB;
      pv[r] = (idx < kR * kCB && i < rows)
                  ? load_as_f32(vb, static_cast<size_t>((i0 + i) * lkv.sr + c0 + c)) : 0.f;
    }
  };
  if (L > 0) fetch(0, min(kR, min(N, L)));

  for (int s = 0; s < S; ++s) {
    const int a = s * N;
    const int e = min(a + N, L);
    __syncthreads();  // previous segment finished reading sM / sZ
#pragma unroll
    for (int r = 0; r < JPT; ++r) sM[kk][j0 + JSTEP * r] = m_reg[r];
    if (t < D) sZ[t] = zval;
    // Snapshot of the state before segment s (transposed M: row j, column kk).
    const size_t snap = static_cast<size_t>(bh) * S + s;
#pragma unroll
    for (int r = 0; r < JPT; ++r) {
      const size_t idx = snap * D * D + static_cast<size_t>(c0 + j0 + JSTEP * r) * D + kk;
      if (mt_f32) mt_f32[idx] = m_reg[r];
      else mt_bf16[idx] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(m_reg[r]));
    }
    if (cb == 0 && t < D) z_pre[(static_cast<size_t>(bh) * (S + 1) + s) * D + t] = zval;

    float dm[JPT];
#pragma unroll
    for (int r = 0; r < JPT; ++r) dm[r] = 0.f;
    float dz = 0.f;

    for (int i0 = a; i0 < e; i0 += kR) {
      const int rows = min(kR, e - i0);
      __syncthreads();  // sK / sU free; sM / sZ visible
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        const int idx = t + r * kThreads, i = idx / D, c = idx % D;
        sK[i][c] = (i < rows) ? elu1(pk[r]) : 0.f;
      }
#pragma unroll
      for (int r = 0; r < VPT; ++r) {
        const int idx = t + r * kThreads;
        if (idx < kR * kCB) sU[idx / kCB][idx % kCB] = pv[r];
      }
      {  // the chunk after this one: the rest of this segment, else the next segment
        const int nx = i0 + kR < e ? i0 + kR : e;
        const int nend = nx == e ? min(e + N, L) : e;
        if (nx < L) fetch(nx, min(kR, nend - nx));
      }
      __syncthreads();
      if (delta) {
        if (t < kR) {
          float acc = eps;
          for (int c = 0; c < D; ++c) acc += sK[t][c] * sZ[c];
          sDen[t] = acc;
        }
        __syncthreads();
        const int jj = t % kCB;
        for (int i = t / kCB; i < kR; i += ISTEP) {
          float acc = 0.f;
          for (int c = 0; c < D; ++c) acc += sK[i][c] * sM[c][jj];
          sU[i][jj] -= acc / sDen[i];  // rows past the segment end: 0 - 0/eps = 0
        }
        __syncthreads();
      }
      // All kR rows: rows past the chunk's end are zero in sK and sU and add
      // exact zeros, and a fixed trip count lets the LDS reads pipeline.
#pragma unroll 16
      for (int i = 0; i < kR; ++i) {
        const float kv = sK[i][kk];
        dz += kv;
#pragma unroll
        for (int r = 0; r < JPT; ++r) dm[r] += kv * sU[i][j0 + JSTEP * r];
      }
    }
#pragma unroll
    for (int r = 0; r < JPT; ++r) m_reg[r] += dm[r];
    zval += dz;
  }
#pragma unroll
  for (int r = 0; r < JPT; ++r) Mb[kk * D + c0 + j0 + JSTEP * r] = m_reg[r];
  // Final z goes to snapshot slot S; the host copies it into z after this kernel,
  // because other workgroups of this head may still be reading the initial z.
  if (cb == 0 && t < D) z_pre[(static_cast<size_t>(bh) * (S + 1) + S) * D + t] = zval;
}

template <typename T, int D>
hipError_t launch_scan_t(const Geometry &g, const T *k, const T *v, float *M, const float *z,
                         int delta, const Workspace &ws, hipStream_t stream) {
  constexpr int CB = scan_cols<D>();
  dim3 grid(D / CB, g.B * g.Hkv);
  segment_scan_kernel<T, D, CB><<<grid, kThreads, 0, stream>>>(
      k, v, g.lkv, g.Hkv, M, z, g.L, g.N, g.S, g.eps, delta,
      ws.z_pre, ws.mt_pre_f32, ws.mt_pre_bf16);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_segment_scan_f32(const Geometry &g, const float *k, const float *v, float *M,
                                   const float *z, int delta, const Workspace &ws,
                                   hipStream_t stream) {
  switch (g.D) {
    case 32: return launch_scan_t<float, 32>(g, k, v, M, z, delta, ws, stream);
    case 64: return launch_scan_t<float, 64>(g, k, v, M, z, delta, ws, stream);
    case 128: return launch_scan_t<float, 128>(g, k, v, M, z, delta, ws, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace ia
