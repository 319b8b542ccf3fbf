// Fused per-segment kernel, bf16 storage path: MFMA bf16 with fp32 accumulate.
//
// For each (batch, query head, segment, query tile):
//   A_dot = causal softmax(Q K^T / sqrt(d_k)) V inside the segment
//           ([HF-repro] "Infini-Attention メカニズム", step Local Attention;
//           [LNCB-review] "基本アイデア"),
//   A_mem = sigma(Q) M_{s-1} / (sigma(Q) z_{s-1} + eps)
//           (step Memory Retrieval; [LNCB-review] "メモリの読み出し"),
//   out   = g A_mem + (1 - g) A_dot with g = sigmoid(beta_h)
//           (step Integration; [LNCB-review] "長期情報と短期情報の統合").
//
// Design (gfx950, wave64, v_mfma_f32_32x32x16_bf16):
//   * A workgroup is 8 waves. Each wave owns 32 query rows of one query head;
//     the workgroup covers HPW query heads that read the same kv head (grouped
//     heads) times 256 / HPW rows. Every K / V tile staged in LDS is consumed by
//     all 8 waves, so K / V movement per MFMA is half that of a 4-wave,
//     one-head workgroup, and for grouped heads the tile is shared across heads.
//   * Everything is computed transposed: S^T = K Q^T and O^T = V^T P^T. In the
//     32x32 MFMA result layout a lane owns one column, so with queries as
//     columns every lane owns one query row: the running max / sum of the
//     online softmax are per lane (plus one exchange with the lane 32 away),
//     and the probabilities P leave the first MFMA already in the operand
//     layout of the second (the key index is the contraction index of P V, and
//     the order in which the hardware walks a contraction does not matter as
//     long as both operands agree).
//   * Q stays in registers for the whole key loop (its d-contiguous rows are
//     exactly the B operand of S^T = K Q^T).
//   * K tiles are staged row-major in LDS (A operand of S^T, d-contiguous).
//     V tiles are staged transposed in LDS, [d][key], with the keys of each
//     16-key step permuted so that the 8 keys a lane contributes to one
//     O^T = V^T P^T MFMA (two runs of 4 in the S^T result layout) are
//     adjacent: the A operand is one 16-byte LDS read. Two LDS buffers: the next
//     tile's global loads are issued before the current tile's MFMAs and it is
//     written into the idle buffer afterwards, one barrier per key tile.
//   * Causal skipping: a workgroup visits key tiles up to its last query row;
//     a wave skips tiles entirely in its future and masks only diagonal tiles.
//   * Online softmax with a lazy rescale: the running max m of a row moves
//     (and O, l are rescaled) only when a tile's max exceeds m by more than
//     kLazy (log2 units), so probabilities stay <= 2^kLazy and most tiles skip
//     the rescale. The 1/sqrt(d) scale is folded into the exponent's FMA, and
//     the row sum is a bf16 dot2 over the same rounded P the MFMA consumes.
//     The kernel runs with the IEEE mode bit off (no NaN quieting on max).
//   * Block order is remapped so that consecutive work items share an XCD
//     (blocks are dealt round-robin to the 8 XCDs): the query heads that read
//     one kv head land on one XCD and share its L2.
//   * Epilogue: the pre-segment snapshot M^T (bf16, [d_v][d_k]) is staged in
//     LDS once for all heads of the workgroup and multiplied with sigma(Q)
//     (computed from the Q registers) on MFMA; the denominator sigma(Q).z is a
//     per-lane dot product plus one exchange.

#include "common.h"
#include "launch.h"

namespace ia {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;       // key rows per tile
constexpr float kLazy = 8.f;  // rescale threshold, log2 units
constexpr int kXcds = 8;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

// Combine a lane's value with that of the lane 32 away. v_permlane32_swap
// exchanges the two 32-lane halves between its two operands, so with both
// operands equal to x the pair it returns is {x, x of lane ^ 32} in some
// order in every lane; max and sum are order-independent.
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

template <int D>
struct Tile {
  static constexpr int KSTR = D + 8;    // sK row stride in bf16 (16-byte pad)
  static constexpr int VSTR = kBN + 8;  // sVt row stride in bf16: 36 dwords, 16 rows hit distinct banks
  static constexpr int MSTR = D + 8;    // staged M^T row stride in bf16
  static constexpr int KCHUNKS = kBN * D / 8;                 // 16-byte K chunks per tile
  static constexpr int KCH = (KCHUNKS + kThreads - 1) / kThreads;  // per thread
  static constexpr int VC = (D / 32) > 2 ? (D / 32) : 2;      // V columns per item (x 4 rows)
  static constexpr int VITEMS = 16 * (D / VC);                // 4-row x VC-column items
  static constexpr int BUF = kBN * KSTR + D * VSTR;           // one K tile + one V^T tile
  static constexpr int LDS_ATT = 2 * BUF;
  static constexpr int LDS_MEM = D * MSTR;
  static constexpr int LDS = LDS_ATT > LDS_MEM ? LDS_ATT : LDS_MEM;
  static_assert(VITEMS <= kThreads, "one V staging item per thread");
};

// Load VC consecutive bf16 (VC in {2, 4}) as VC/2 packed words.
template <int VC>
__device__ __forceinline__ void load_cols(const uint16_t *p, uint32_t (&w)[VC / 2]) {
  if constexpr (VC == 4) {
    const u32x2 x = *reinterpret_cast<const u32x2 *>(p);
    w[0] = x[0];
    w[1] = x[1];
  } else {
    w[0] = *reinterpret_cast<const uint32_t *>(p);
  }
}

template <int D, int HPW>
__global__ __launch_bounds__(kThreads, 2) void fused_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const float *__restrict__ beta,
    const float *__restrict__ z_pre, const uint16_t *__restrict__ mt_pre,
    uint16_t *__restrict__ out, int Hq, int Hkv, int L, int N, int S, int n_qt, float eps,
    float scale_log2, int xcd_chunk) {
  using TL = Tile<D>;
  constexpr int NT = D / 16;          // k-steps over d
  constexpr int ND = D / 32;          // 32-row d tiles of O^T
  constexpr int RW = kWaves / HPW;    // waves (32-row strips) per head
  constexpr int BM = 32 * RW;         // query rows per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t smem[TL::LDS];
  __shared__ float sZ[D];
  const int tid = threadIdx.x;
  // The wave index is uniform across the wave; readfirstlane puts it (and all
  // per-wave bounds derived from it) in scalar registers, so the mask and
  // skip conditions below are real branches rather than per-lane selects.
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 5, l32 = lane & 31;

  // Work item: dispatch index -> XCD-contiguous order (when the grid divides
  // evenly), then (query tile, segment, head unit) with the query tile fastest;
  // longest query tiles (most key tiles under the mask) first. A head unit is
  // HPW consecutive query heads of one kv head.
  int wi = blockIdx.x;
  if (xcd_chunk > 0) wi = (wi % kXcds) * xcd_chunk + wi / kXcds;
  const int grp = Hq / Hkv;
  const int units = grp / HPW;  // head units per kv head
  const int qt = n_qt - 1 - wi % n_qt;
  const int s = (wi / n_qt) % S;
  const int unit = wi / (n_qt * S);
  const int b = unit / (Hkv * units);
  const int hk = (unit / units) % Hkv;
  const int h = hk * grp + (unit % units) * HPW + w / RW;  // this wave's query head
  const int bhq = b * Hq + h;
  const int a = s * N;
  const int e = min(a + N, L);
  const int q0 = a + qt * BM;
  if (q0 >= e) return;  // short last segment: whole workgroup idle
  const int qw = q0 + (w % RW) * 32;  // first query row of this wave
  const int qrow = qw + l32;          // query row owned by this lane
  const bool wave_live = qw < e;

  const uint16_t *qp = q + static_cast<size_t>(bhq) * L * D;
  const size_t kvoff = (static_cast<size_t>(b) * Hkv + hk) * L * D;
  const uint16_t *kp = k + kvoff;
  const uint16_t *vp = v + kvoff;

  // Q^T operand: k-step t covers d in [16t, 16t+16); lane holds d = 16t + 8g + 0..7.
  u32x4 qf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    qf[t] = (qrow < e) ? *reinterpret_cast<const u32x4 *>(qp + static_cast<size_t>(qrow) * D +
                                                          16 * t + 8 * g)
                       : u32x4{0u, 0u, 0u, 0u};
  }

  f32x16 o[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) o[dt] = f32x16{};
  float m = -INFINITY;  // running max of this row, log2 domain
  float lsum = 0.f;     // running sum over this lane's key slots

  const int kv_end = min(q0 + BM, e);

  // Register staging of the next K / V tile.
  u32x4 kreg[TL::KCH];
  uint32_t vreg[4][TL::VC / 2];
  const int v_kg = tid & 15;  // 4-row key group
  const int v_cc = tid >> 4;  // VC-column chunk
  const bool v_has = tid < TL::VITEMS;
  // K chunk r of this thread: chunk tid + kThreads * r = row c / (D/8), col (c % (D/8)) * 8.
  constexpr int KROWS = kThreads / (D / 8);
  const int koff = (tid / (D / 8)) * D + (tid % (D / 8)) * 8;
  const int voff = 4 * v_kg * D + v_cc * TL::VC;

  auto load_tile = [&](int kv0) {
    const uint16_t *kt = kp + static_cast<size_t>(kv0) * D;
    const uint16_t *vt = vp + static_cast<size_t>(kv0) * D + voff;
    if (kv0 + kBN <= e) {  // whole tile inside the segment: no per-row guards
#pragma unroll
      for (int r = 0; r < TL::KCH; ++r)
        if (tid + kThreads * r < TL::KCHUNKS)
          kreg[r] = *reinterpret_cast<const u32x4 *>(kt + koff + r * KROWS * D);
      if (v_has) {
#pragma unroll
        for (int r = 0; r < 4; ++r) load_cols<TL::VC>(vt + r * D, vreg[r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < TL::KCH; ++r) {
        const int row = (tid + kThreads * r) / (D / 8);
        if (tid + kThreads * r < TL::KCHUNKS)
          kreg[r] = (kv0 + row < e)
                        ? *reinterpret_cast<const u32x4 *>(kt + koff + r * KROWS * D)
                        : u32x4{0u, 0u, 0u, 0u};
      }
      if (v_has) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (kv0 + 4 * v_kg + r < e) {
            load_cols<TL::VC>(vt + r * D, vreg[r]);
          } else {
#pragma unroll
            for (int i = 0; i < TL::VC / 2; ++i) vreg[r][i] = 0u;
          }
        }
      }
    }
  };

  // Key group kg (keys 4 kg .. 4 kg + 3 of the tile) = 16-key step kg / 4,
  // run h = (kg / 2) % 2, lane group g = kg % 2 of the S^T layout; it is
  // stored at 4-key position (kg / 4, g, h), i.e. bits 0 and 1 swapped.
  const int v_pos = 4 * ((v_kg & ~3) | ((v_kg & 1) << 1) | ((v_kg >> 1) & 1));

  auto store_tile = [&](uint16_t *sK, uint16_t *sVt) {
#pragma unroll
    for (int r = 0; r < TL::KCH; ++r) {
      const int c = tid + kThreads * r;
      if (c < TL::KCHUNKS) {
        const int row = c / (D / 8), col8 = c % (D / 8);
        *reinterpret_cast<u32x4 *>(sK + row * TL::KSTR + col8 * 8) = kreg[r];
      }
    }
    if (v_has) {
      // Transpose 4 rows x VC columns: one 8-byte write of 4 keys per column.
      // v_perm picks the low (resp. high) bf16 of two rows into one word.
#pragma unroll
      for (int i = 0; i < TL::VC / 2; ++i) {
        const uint32_t r0 = vreg[0][i], r1 = vreg[1][i], r2 = vreg[2][i], r3 = vreg[3][i];
        const u32x2 lo = {__builtin_amdgcn_perm(r1, r0, 0x05040100u),
                          __builtin_amdgcn_perm(r3, r2, 0x05040100u)};
        const u32x2 hi = {__builtin_amdgcn_perm(r1, r0, 0x07060302u),
                          __builtin_amdgcn_perm(r3, r2, 0x07060302u)};
        const int col = v_cc * TL::VC + 2 * i;
        *reinterpret_cast<u32x2 *>(sVt + col * TL::VSTR + v_pos) = lo;
        *reinterpret_cast<u32x2 *>(sVt + (col + 1) * TL::VSTR + v_pos) = hi;
      }
    }
  };

  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};

  load_tile(a);
  store_tile(smem, smem + kBN * TL::KSTR);
  __syncthreads();
  int buf = 0;
  for (int kv0 = a; kv0 < kv_end; kv0 += kBN) {
    const uint16_t *sK = smem + buf * TL::BUF;
    const uint16_t *sVt = sK + kBN * TL::KSTR;
    const bool has_next = kv0 + kBN < kv_end;
    if (has_next) load_tile(kv0 + kBN);  // global loads in flight during the MFMAs

    if (wave_live && kv0 <= qw + 31) {
      // S^T tile pair: rows = keys kv0 + 32T + ..., columns = this wave's
      // queries; two independent accumulation chains, interleaved.
      f32x16 st[2] = {f32x16{}, f32x16{}};
      const uint16_t *krow = sK + l32 * TL::KSTR + 8 * g;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4 ka0 = *reinterpret_cast<const u32x4 *>(krow + 16 * t);
        const u32x4 ka1 = *reinterpret_cast<const u32x4 *>(krow + 32 * TL::KSTR + 16 * t);
        st[0] = mfma32(as_bf16x8(ka0), as_bf16x8(qf[t]), st[0]);
        st[1] = mfma32(as_bf16x8(ka1), as_bf16x8(qf[t]), st[1]);
      }
      // Mask future keys and keys past the segment end (diagonal tiles only).
      if ((kv0 + kBN - 1 > qw) || (kv0 + kBN > e)) {
        __asm__ volatile("" ::: "memory");  // keep this a branch (diagonal tiles only)
        const int lim = min(qrow, e - 1) - kv0 - 4 * g;  // key offsets above lim are masked
#pragma unroll
        for (int T = 0; T < 2; ++T) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if (32 * T + (i >> 2) * 8 + (i & 3) > lim) st[T][i] = -INFINITY;
          }
        }
      }
      float mx = fmaxf(st[0][0], st[1][0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(st[0][i], st[1][i]));
      mx = max_xor32(mx) * scale_log2;  // finite: key a is always visible
      const bool grow = mx > m + kLazy;
      if (__any(grow)) {
        __asm__ volatile("" ::: "memory");  // keep this a branch (rarely taken)
        const float m_new = grow ? mx : m;
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 1 where m stays
        m = m_new;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) o[dt] *= alpha;
      }
      // p = 2^(s c - m) rounded to bf16; the row sum is taken over the same
      // rounded values (bf16 dot2 with ones), so numerator and denominator
      // of the softmax see identical weights. O^T += V^T P^T as soon as each
      // 16-key group of P is packed: pair idx holds elements 2 (idx % 8), +1
      // of the 32-key half idx / 8, and group tu = idx / 4 is the P operand of
      // key step tu (slot j of lane group g is key 16 tu + 8 (j / 4) + 4 g +
      // j % 4, matching the S^T result layout; sVt holds it at position
      // 16 tu + 8 g + j).
      const float neg_m = -m;
      const uint16_t *vrow = sVt + l32 * TL::VSTR + 8 * g;
#pragma unroll
      for (int tu = 0; tu < 4; ++tu) {
        // The V fragments of this key step are read first, so their LDS
        // latency overlaps the exponentials.
        u32x4 va[ND];
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
          va[dt] = *reinterpret_cast<const u32x4 *>(vrow + 32 * dt * TL::VSTR + 16 * tu);
        uint32_t pw[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int idx = 4 * tu + jj;
          const int T = idx >> 3, i = 2 * (idx & 7);
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[T][i], scale_log2, neg_m));
          const float p1 =
              __builtin_amdgcn_exp2f(__builtin_fmaf(st[T][i + 1], scale_log2, neg_m));
          pw[jj] = pack_bf16x2(p0, p1);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[jj]), ones, lsum,
                                                 false);
        }
        const u32x4 pb = {pw[0], pw[1], pw[2], pw[3]};
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) o[dt] = mfma32(as_bf16x8(va[dt]), as_bf16x8(pb), o[dt]);
      }
    }
    if (has_next) {
      // The idle buffer was last read before the previous barrier.
      uint16_t *nK = smem + (buf ^ 1) * TL::BUF;
      store_tile(nK, nK + kBN * TL::KSTR);
    }
    __syncthreads();
    buf ^= 1;
  }

  // ---- retrieval from the pre-segment snapshot and the gate ----
  const size_t head = static_cast<size_t>(b) * Hkv + hk;
  const uint16_t *mt = mt_pre + (head * S + s) * D * D;
  const float *zs = z_pre + (head * (S + 1) + s) * D;
  // (the loop ended with a barrier: smem is free for M^T)
  for (int c = tid; c < D * D / 8; c += kThreads) {
    const int row = c / (D / 8), col8 = c % (D / 8);
    *reinterpret_cast<u32x4 *>(smem + row * TL::MSTR + col8 * 8) =
        *reinterpret_cast<const u32x4 *>(mt + static_cast<size_t>(row) * D + col8 * 8);
  }
  if (tid < D) sZ[tid] = zs[tid];
  __syncthreads();

  if (!wave_live) return;
  // sigma(Q) as the B operand, and this lane's part of sigma(q).z.
  float den = 0.f;
  u32x4 sq[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    uint32_t wv[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float x0 = elu1(lo_bf16(qf[t][jj]));
      const float x1 = elu1(hi_bf16(qf[t][jj]));
      den += x0 * sZ[16 * t + 8 * g + 2 * jj] + x1 * sZ[16 * t + 8 * g + 2 * jj + 1];
      wv[jj] = pack_bf16x2(x0, x1);
    }
    sq[t] = u32x4{wv[0], wv[1], wv[2], wv[3]};
  }
  den = sum_xor32(den) + eps;
  const float inv_den = 1.f / den;
  const float inv_l = 1.f / sum_xor32(lsum);  // both halves' key slots
  const float gam = 1.f / (1.f + __expf(-beta[h]));
  const float w_mem = gam * inv_den;
  const float w_dot = (1.f - gam) * inv_l;

  uint16_t *op = out + (static_cast<size_t>(bhq) * L + qrow) * D;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) {
    f32x16 am = f32x16{};
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x4 ma = *reinterpret_cast<const u32x4 *>(smem + (32 * dt + l32) * TL::MSTR +
                                                       16 * t + 8 * g);
      am = mfma32(as_bf16x8(ma), as_bf16x8(sq[t]), am);
    }
    if (qrow < e) {
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        uint32_t pk[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int i0 = 4 * gi + 2 * jj;
          pk[jj] = pack_bf16x2(w_mem * am[i0] + w_dot * o[dt][i0],
                               w_mem * am[i0 + 1] + w_dot * o[dt][i0 + 1]);
        }
        *reinterpret_cast<u32x2 *>(op + 32 * dt + 8 * gi + 4 * g) = u32x2{pk[0], pk[1]};
      }
    }
  }
}

template <int D, int HPW>
hipError_t launch_t(const Geometry &g, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const float *beta, const Workspace &ws, uint16_t *out, hipStream_t stream) {
  constexpr int BM = 32 * kWaves / HPW;
  const int rows = g.N < g.L ? g.N : g.L;
  const int n_qt = (rows + BM - 1) / BM;
  const long long units = static_cast<long long>(g.B) * g.Hkv * (g.Hq / g.Hkv / HPW);
  const long long nblk = static_cast<long long>(n_qt) * g.S * units;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int xcd_chunk = (nblk % kXcds == 0) ? static_cast<int>(nblk / kXcds) : 0;
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  fused_bf16_kernel<D, HPW><<<dim3(static_cast<unsigned>(nblk)), kThreads, 0, stream>>>(
      q, k, v, beta, ws.z_pre, ws.mt_pre_bf16, out, g.Hq, g.Hkv, g.L, g.N, g.S, n_qt, g.eps,
      scale_log2, xcd_chunk);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Geometry &g, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const float *beta, const Workspace &ws, uint16_t *out, hipStream_t stream) {
  // Share each K / V tile across two query heads when they read the same kv head.
  if ((g.Hq / g.Hkv) % 2 == 0) return launch_t<D, 2>(g, q, k, v, beta, ws, out, stream);
  return launch_t<D, 1>(g, q, k, v, beta, ws, out, stream);
}

}  // namespace

hipError_t launch_fused_bf16(const Geometry &g, const uint16_t *q, const uint16_t *k,
                             const uint16_t *v, const float *beta, const Workspace &ws,
                             uint16_t *out, hipStream_t stream) {
  switch (g.D) {
    case 32: return launch_d<32>(g, q, k, v, beta, ws, out, stream);
    case 64: return launch_d<64>(g, q, k, v, beta, ws, out, stream);
    case 128: return launch_d<128>(g, q, k, v, beta, ws, out, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace ia
