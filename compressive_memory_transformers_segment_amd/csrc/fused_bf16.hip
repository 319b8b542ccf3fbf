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
//   * Tiles move from HBM to LDS by direct loads (global_load_lds: no
//     register staging, no LDS store instructions) through a ring of three
//     buffers: tile t + 2 is in flight while tile t is consumed, and each
//     wave waits only for its own loads of tile t + 1 before the one barrier
//     per key tile. K tiles are row-major with a 16-byte-unit XOR swizzle so
//     that the 32 rows an MFMA operand reads hit distinct banks. V arrives
//     already transposed, [d][key], from the segment scan, which writes it per
//     64-key tile with the keys of each 16-key step permuted so that the 8
//     keys a lane contributes to one O^T = V^T P^T MFMA (two runs of 4 in the
//     S^T result layout) are adjacent and bank-swizzled: every MFMA operand
//     read from LDS is one 16-byte read.
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
//   * Epilogue: the pre-segment snapshot M^T (bf16, [d_v][d_k]) arrives in its
//     own LDS buffer by direct loads ahead of the first key tile, once for all
//     heads of the workgroup, and is multiplied with sigma(Q)
//     (computed from the Q registers) on MFMA; the denominator sigma(Q).z is a
//     per-lane dot product plus one exchange.

#include <type_traits>

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

// Wait until at most VM vector-memory operations of this wave are in flight
// and all of its LDS operations are done (s_waitcnt, gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 left at its maximum, lgkmcnt 11:8 = 0).
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
}

#define IA_LDS(p) ((__attribute__((address_space(3))) void *)(p))

template <int D>
struct Tile {
  static constexpr int CPR = D / 8;          // 16-byte units per K (and M^T) row
  static constexpr int RP = 16 / CPR;        // K rows per 256-byte bank line
  static constexpr int KU = kBN * CPR;       // K units per tile
  static constexpr int VU = D * 8;           // V^T units per tile (64 keys per row)
  static constexpr int BUFU = KU + VU;       // units per ring buffer
  static constexpr int BUF = BUFU * 8;       // bf16 per ring buffer
  static constexpr int IPW = BUFU / kThreads;  // direct loads per wave per tile
  static constexpr int MU = D * CPR;         // M^T units
  static constexpr int MPW = (MU + kThreads - 1) / kThreads;  // direct loads per wave for M^T
  static_assert(BUFU % kThreads == 0, "whole direct loads per wave");
  static_assert(KU % 64 == 0, "a direct load never straddles K and V^T");

};

// 16-byte unit of (row r, unit c) in a swizzled row-major tile of D columns
// (K tiles and M^T): 16 consecutive rows read at one unit index land on
// distinct banks.
template <int D>
__device__ __forceinline__ int swz_unit(int r, int c) {
  using TL = Tile<D>;
  return r * TL::CPR + (c ^ ((r / TL::RP) % TL::CPR));
}

template <int D, int HPW>
__global__ __launch_bounds__(kThreads, 2) void fused_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ vt, int vt_tiles, const float *__restrict__ beta,
    const float *__restrict__ z_pre, const uint16_t *__restrict__ mt_pre,
    uint16_t *__restrict__ out, int Hq, int Hkv, int L, int N, int S, int n_qt, float eps,
    float scale_log2, int xcd_chunk) {
  using TL = Tile<D>;
  constexpr int NT = D / 16;          // k-steps over d
  constexpr int ND = D / 32;          // 32-row d tiles of O^T
  constexpr int RW = kWaves / HPW;    // waves (32-row strips) per head
  constexpr int BM = 32 * RW;         // query rows per workgroup
  // Three separate arrays, so that the compiler can tell the buffers apart
  // when it orders LDS reads after direct loads into another buffer.
  __shared__ __attribute__((aligned(16))) uint16_t sB0[TL::BUF];
  __shared__ __attribute__((aligned(16))) uint16_t sB1[TL::BUF];
  __shared__ __attribute__((aligned(16))) uint16_t sB2[TL::BUF];
  __shared__ __attribute__((aligned(16))) uint16_t sM[TL::MU * 8];
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
  const size_t head = static_cast<size_t>(b) * Hkv + hk;
  const uint16_t *kp = k + head * L * D;
  const uint16_t *vtp = vt + (head * S + s) * vt_tiles * (D * 64);  // this segment's V^T tiles
  const uint16_t *mt = mt_pre + (head * S + s) * D * D;
  const float *zs = z_pre + (head * (S + 1) + s) * D;
  const float zreg = tid < D ? zs[tid] : 0.f;

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

  const int n_tiles = (kv_end - a + kBN - 1) / kBN;

  // Direct loads: load i of wave w moves units [(8 i + w) 64, +64) of a ring
  // buffer, one 16-byte unit per lane, into consecutive LDS (the hardware
  // writes lane l's unit at the wave's LDS base + 16 l). Units below KU are K
  // (lane picks its source through the swizzle; rows past the segment end
  // read its last row, whose scores are masked anyway), the rest V^T, copied
  // verbatim from the scan's tile.
  auto dma_tile = [&](int t, uint16_t *buf) {
    const int kv0 = a + t * kBN;
    const uint16_t *vsrc = vtp + static_cast<size_t>(t) * (D * 64);
#pragma unroll
    for (int i = 0; i < TL::IPW; ++i) {
      const int u0 = (8 * i + w) * 64;  // wave-uniform
      const int U = u0 + lane;
      const int r = U / TL::CPR, cp = U % TL::CPR;
      const uint16_t *ksrc =
          kp + static_cast<size_t>(min(kv0 + r, e - 1)) * D + 8 * (cp ^ ((r / TL::RP) % TL::CPR));
      const uint16_t *vsrc_u = vsrc + 8 * (U - TL::KU);
      // For D >= 64 the first KU / 512 loads of every wave are K; for D = 32
      // the first load is K in waves 0..3 and V^T in waves 4..7. A select, not
      // a branch, so the loads form straight-line code.
      const bool is_k = (TL::KU % kThreads == 0) ? (i < TL::KU / kThreads) : (u0 < TL::KU);
      __builtin_amdgcn_global_load_lds(is_k ? ksrc : vsrc_u, IA_LDS(buf + 8 * u0), 16, 0, 0);
    }
  };
  // M^T of the segment, swizzled like a K tile.
  auto dma_mem = [&]() {
#pragma unroll
    for (int i = 0; i < TL::MPW; ++i) {
      const int u0 = (8 * i + w) * 64;
      if (u0 < TL::MU) {
        const int U = u0 + lane;
        const int r = U / TL::CPR, cp = U % TL::CPR;
        const int c = cp ^ ((r / TL::RP) % TL::CPR);
        __builtin_amdgcn_global_load_lds(mt + static_cast<size_t>(r) * D + 8 * c,
                                         IA_LDS(sM + 8 * u0), 16, 0, 0);
      }
    }
  };

  // Per-lane LDS offsets (bf16 elements) of the MFMA operands: K row l32 (+32
  // for the second key half), unit 2 t + g; V^T row l32 (+32 dt), unit 2 tu + g.
  int koff[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) koff[t] = 8 * swz_unit<D>(l32, 2 * t + g);
  int voff[4];
#pragma unroll
  for (int tu = 0; tu < 4; ++tu) voff[tu] = 8 * (TL::KU + l32 * 8 + vt_unit_pos(l32, 2 * tu + g));

  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};

  auto compute = [&](int kv0, const uint16_t *buf) {
    // S^T tile pair: rows = keys kv0 + 32T + ..., columns = this wave's
    // queries; two independent accumulation chains, interleaved.
    f32x16 st[2] = {f32x16{}, f32x16{}};
    // K fragments are read two k-steps ahead of their MFMAs (two register
    // sets); the scheduling fences keep the compiler from sinking the reads
    // next to their uses.
    u32x4 kf[2][2];
    auto kread = [&](int t, u32x4 (&kk)[2]) __attribute__((always_inline)) {
      kk[0] = *reinterpret_cast<const u32x4 *>(buf + koff[t]);
      kk[1] = *reinterpret_cast<const u32x4 *>(buf + koff[t] + 32 * D);
    };
    kread(0, kf[0]);
    if (NT > 1) kread(1, kf[1]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      __builtin_amdgcn_sched_barrier(0);
      st[0] = mfma32(as_bf16x8(kf[t & 1][0]), as_bf16x8(qf[t]), st[0]);
      st[1] = mfma32(as_bf16x8(kf[t & 1][1]), as_bf16x8(qf[t]), st[1]);
      if (t + 2 < NT) kread(t + 2, kf[t & 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
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
    // j % 4, matching the S^T result layout and the V^T tile's unit order).
    const float neg_m = -m;
    // V fragments of step tu + 1 are read right after the MFMAs of step tu,
    // so their latency overlaps the exponentials of step tu + 1.
    u32x4 vf[2][ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
      vf[0][dt] = *reinterpret_cast<const u32x4 *>(buf + voff[0] + 32 * dt * 64);
#pragma unroll
    for (int tu = 0; tu < 4; ++tu) {
      u32x4 (&va)[ND] = vf[tu & 1];
      uint32_t pw[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int idx = 4 * tu + jj;
        const int T = idx >> 3, i = 2 * (idx & 7);
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[T][i], scale_log2, neg_m));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[T][i + 1], scale_log2, neg_m));
        pw[jj] = pack_bf16x2(p0, p1);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[jj]), ones, lsum,
                                               false);
      }
      const u32x4 pb = {pw[0], pw[1], pw[2], pw[3]};
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) o[dt] = mfma32(as_bf16x8(va[dt]), as_bf16x8(pb), o[dt]);
      if (tu + 1 < 4) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
          vf[(tu + 1) & 1][dt] =
              *reinterpret_cast<const u32x4 *>(buf + voff[tu + 1] + 32 * dt * 64);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Iteration t: direct loads of tile t + 2 into the buffer tile t - 1 left
  // (past the end, the last tile again: every iteration issues the same
  // loads, so issue and wait form one pattern whose count the compiler's own
  // wait analysis can follow; nothing reads that buffer before it is
  // reloaded); the tile's MFMAs; then this wave's loads of tile t + 1 are
  // awaited and the workgroup meets at the barrier that publishes them.
  //
  // The compiler's wait analysis loses track of which buffer a direct load
  // targets where control flow merges (the loop head) and waits for all of
  // them before the next LDS read; the first iteration after the loop head
  // therefore issues its loads after its MFMAs (LATE), so that this wait
  // covers only tile t + 1, issued a whole tile earlier.
  auto step = [&](auto late, int t, const uint16_t *cur, uint16_t *nx2) {
    if (!late.value) dma_tile(min(t + 2, n_tiles - 1), nx2);
    const int kv0 = a + t * kBN;
    if (wave_live && kv0 <= qw + 31) compute(kv0, cur);
    if (late.value) dma_tile(min(t + 2, n_tiles - 1), nx2);
    wait_vm_lgkm0<TL::IPW>();
    __builtin_amdgcn_s_barrier();
  };
  using LATE = std::true_type;
  using EARLY = std::false_type;

  // M^T first (its own buffer, needed only after the loop), then tiles 0, 1.
  dma_mem();
  dma_tile(0, sB0);
  dma_tile(min(1, n_tiles - 1), sB1);
  wait_vm_lgkm0<TL::IPW>();
  __builtin_amdgcn_s_barrier();
  for (int t = 0;;) {
    step(LATE{}, t, sB0, sB2);
    if (++t >= n_tiles) break;
    step(EARLY{}, t, sB1, sB0);
    if (++t >= n_tiles) break;
    step(EARLY{}, t, sB2, sB1);
    if (++t >= n_tiles) break;
  }

  // ---- retrieval from the pre-segment snapshot and the gate ----
  if (tid < D) sZ[tid] = zreg;
  wait_vm_lgkm0<0>();
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
      const u32x4 ma =
          *reinterpret_cast<const u32x4 *>(sM + 8 * swz_unit<D>(32 * dt + l32, 2 * t + g));
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
      q, k, ws.vt, ws.vt_tiles, beta, ws.z_pre, ws.mt_pre_bf16, out, g.Hq, g.Hkv, g.L, g.N, g.S,
      n_qt, g.eps, scale_log2, xcd_chunk);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Geometry &g, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const float *beta, const Workspace &ws, uint16_t *out, hipStream_t stream) {
  // Share each K / V tile across up to four query heads that read the same kv
  // head (64 rows each); otherwise two heads of 128 rows or one of 256.
  if ((g.Hq / g.Hkv) % 4 == 0) return launch_t<D, 4>(g, q, k, v, beta, ws, out, stream);
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
