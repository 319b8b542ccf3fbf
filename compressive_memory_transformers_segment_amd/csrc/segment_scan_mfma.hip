// Segment scan for bf16 storage on MFMA.
//
// Memory update per segment s ([HF-repro] "Infini-Attention メカニズム", steps
// Memory Update and State Transfer; [LNCB-review] "メモリの更新"):
//   LINEAR: M_s = M_{s-1} + H_s
//   DELTA:  M_s = M_{s-1} + sigma(K_s)^T (V_s - sigma(K_s) M_{s-1} / (sigma(K_s) z_{s-1} + eps))
//             = (I - G_s) M_{s-1} + H_s
//   with H_s = sigma(K_s)^T V_s and G_s = sigma(K_s)^T diag(1 / (sigma(K_s) z_{s-1} + eps)) sigma(K_s),
//   z_s = z_{s-1} + sum_i sigma(k_i).
// The delta rule is written in this affine form so that the only work left on
// the sequential path is one d x d by d x d product per segment; everything
// that touches the N x d segment data is done for all segments in parallel.
//
// Four launches, in stream order:
//   zsum    (segment, head)     dz_s = column sums of sigma(K_s)             [VALU]
//   zprefix (head)              z_{s-1} for every s, and z_S                  [VALU]
//   gh      (segment, head)     G_s (delta only) and H_s, contraction over    [MFMA bf16]
//                               the segment's rows, stored in MFMA fragment
//                               order: H_s as fp32, G_s as a bf16 hi/lo pair;
//                               also writes the segment's V^T in 64-key tiles
//                               (the fused kernel's LDS layout)
//   seq     (column tile, head) M_s = M_{s-1} - G_s M_{s-1} + H_s with the    [MFMA bf16 x3]
//                               product as G_hi M_hi + G_hi M_lo + G_lo M_hi
//                               (about 16 mantissa bits); fp32 state in
//                               registers; writes the bf16 snapshot M_{s-1}^T
//                               the fused kernel reads, and M_S.
//
// Fragment order: a d x d matrix is stored as (D/32)^2 tiles of 32 x 32; tile
// (rt, ct) holds, for MFMA-result register r and lane l, the element at row
// 32 rt + kappa(r, l / 32), column 32 ct + l % 32, where
// kappa(r, g) = 8 (r / 4) + 4 g + r % 4 is the 32x32 MFMA result row map.
// A lane's 16 values (words) of a tile are kept as four 16-byte quarters, and
// quarter q of all 64 lanes is contiguous, so that every 16-byte load or store
// of a wave covers one contiguous kilobyte:
//   H_s (fp32): element index (((rt * (D/32) + ct) * 4 + r / 4) * 64 + l) * 4 + r % 4.
//   G_s (bf16 hi/lo): 32-bit word (((rt * (D/32) + ct) * 4 + w / 4) * 64 + l) * 4 + w % 4,
//     where word 4 h + p (h, p < 2, 4) packs the hi parts of registers 8 h + 2 p
//     (low half) and 8 h + 2 p + 1 (high half), and word 8 + 4 h + p the lo
//     parts; so quarter h (hi) and quarter 2 + h (lo) are directly the 8-slot
//     bf16 A operands of a 32x32x16 MFMA over rows 32 rt + 16 h .. + 15. G_s is
//     symmetric, so tile (kt, ct) read this way is the A operand for output
//     rows of tile ct.

#include "common.h"
#include "launch.h"

namespace ia {
namespace {

constexpr int kStr = 64 + 4;  // transposed staging row stride (bf16): 64 keys + 8-byte pad

__device__ __forceinline__ f32x16 mfma_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ int kappa(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// x of another lane of the same 16-lane row, by DPP control CTRL (all lanes
// active): quad_perm 0xB1 = lane ^ 1, 0x4E = lane ^ 2; row_half_mirror 0x141
// = lane 7 - i within 8; row_mirror 0x140 = lane 15 - i within 16.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Workgroup barrier that orders LDS only. __syncthreads() also waits for every
// outstanding global load and store of the wave, which would drain the
// prefetches the loops below keep in flight across their barriers; these
// barriers only ever guard LDS buffers.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// zsum: dz[head][s][part][c] = sum over rows of part `part` of segment s of
// sigma(k_ic). A segment is split into `parts` row ranges so that short
// launches (few segments) still spread over the chip; zprefix adds the parts.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void zsum_kernel(const uint16_t *__restrict__ k, Layout lk,
                                                   int Hkv, float *__restrict__ dz, int L, int N,
                                                   int S, int parts) {
  constexpr int CCH = D / 8;      // 16-byte chunks per row
  constexpr int RG = 256 / CCH;   // rows in flight per pass
  constexpr int UNROLL = 4;
  __shared__ float red[RG][D + 1];
  const int s = blockIdx.x / parts, part = blockIdx.x % parts;
  const int head = blockIdx.y;
  const int a = s * N, e = min(a + N, L);
  const int span = (e - a + parts - 1) / parts;
  const int pa = min(a + part * span, e), pe = min(pa + span, e);
  const int t = threadIdx.x, cc = t % CCH, rg = t / CCH;
  const uint16_t *kp = k + head_offset(lk, head, Hkv) + cc * 8;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  for (int i = pa + rg; i < pe; i += RG * UNROLL) {
    u32x4 w[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int row = i + u * RG;
      w[u] = row < pe ? *reinterpret_cast<const u32x4 *>(kp + row * lk.sr)
                      : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      if (i + u * RG < pe) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          acc[2 * jj] += elu1(lo_bf16(w[u][jj]));
          acc[2 * jj + 1] += elu1(hi_bf16(w[u][jj]));
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red[rg][cc * 8 + j] = acc[j];
  __syncthreads();
  if (t < D) {
    float sum = 0.f;
    for (int r = 0; r < RG; ++r) sum += red[r][t];
    dz[((static_cast<size_t>(head) * S + s) * parts + part) * D + t] = sum;
  }
}

// ---------------------------------------------------------------------------
// zprefix: z_pre[head][s] = z_{s-1} (the state before segment s), slot S = z_S.
// With z_hl, also z_{s-1} as two bf16 rows: hi = bf16(z), lo = bf16(z - hi)
// (about 16 significant bits together), the operand from which the fused
// kernel forms sigma(q).z on the matrix cores.
// One workgroup per (32-column block, head); thread (grp, c) owns column c of
// a contiguous range of segments. Pass 1 sums the range, the workgroup
// prefix-sums the ranges in LDS, pass 2 writes the running value. dz is read
// in batches of kZB independent loads so that the sequential part waits on
// memory only once per batch.
// ---------------------------------------------------------------------------
constexpr int kZB = 16;
constexpr int kZThreads = 1024;
constexpr int kZCols = 32;  // columns per workgroup

// The final z also goes to z_final, which may be z0 itself (the caller's
// in/out state): every thread reads z0 before the barrier that precedes that
// store, and each workgroup touches only its own columns.
__global__ __launch_bounds__(kZThreads) void zprefix_kernel(const float *z0,
                                                            const float *__restrict__ dz,
                                                            float *__restrict__ z_pre,
                                                            uint16_t *__restrict__ z_hl, int S,
                                                            int D, int parts, float *z_final) {
  __shared__ float tot[kZThreads];
  const int head = blockIdx.y, G = kZThreads / kZCols;
  const int cl = threadIdx.x % kZCols, grp = threadIdx.x / kZCols;
  const int c = blockIdx.x * kZCols + cl;
  const int per = (S + G - 1) / G;
  const int s0 = min(grp * per, S), s1 = min(s0 + per, S);
  const int f0 = s0 * parts, f1 = s1 * parts;  // flat (segment, part) range
  const float *d = dz + static_cast<size_t>(head) * S * parts * D + c;

  float sum = 0.f;
  for (int f = f0; f < f1; f += kZB) {
    float x[kZB];
#pragma unroll
    for (int i = 0; i < kZB; ++i) x[i] = f + i < f1 ? d[static_cast<size_t>(f + i) * D] : 0.f;
#pragma unroll
    for (int i = 0; i < kZB; ++i) sum += x[i];
  }
  tot[grp * kZCols + cl] = sum;
  __syncthreads();
  float z = z0[static_cast<size_t>(head) * D + c];
  for (int q = 0; q < grp; ++q) z += tot[q * kZCols + cl];

  float *out = z_pre + static_cast<size_t>(head) * (S + 1) * D + c;
  for (int f = f0; f < f1; f += kZB) {
    float x[kZB];
#pragma unroll
    for (int i = 0; i < kZB; ++i) x[i] = f + i < f1 ? d[static_cast<size_t>(f + i) * D] : 0.f;
#pragma unroll
    for (int i = 0; i < kZB; ++i) {
      if (f + i < f1) {
        if ((f + i) % parts == 0) {
          const int s = (f + i) / parts;
          out[static_cast<size_t>(s) * D] = z;
          if (z_hl) {
            const __bf16 hi = static_cast<__bf16>(z);
            const __bf16 lo = static_cast<__bf16>(z - static_cast<float>(hi));
            uint16_t *zh = z_hl + (static_cast<size_t>(head) * S + s) * 2 * D + c;
            zh[0] = __builtin_bit_cast(uint16_t, hi);
            zh[D] = __builtin_bit_cast(uint16_t, lo);
          }
        }
        z += x[i];
      }
    }
  }
  float zs = 0.f;
  if (grp == G - 1) {
    zs = z0[static_cast<size_t>(head) * D + c];
    for (int q = 0; q < G; ++q) zs += tot[q * kZCols + cl];
    out[static_cast<size_t>(S) * D] = zs;
  }
  __syncthreads();  // every read of z0 in this workgroup is done
  if (grp == G - 1) z_final[static_cast<size_t>(head) * D + c] = zs;
}

// ---------------------------------------------------------------------------
// gh: [G_s | H_s] = sigma(K_s)^T [diag(1/den) sigma(K_s) | V_s], den_i = sigma(k_i).z_{s-1} + eps
// ---------------------------------------------------------------------------
// RG row groups of four waves share a workgroup: group q takes the chunks
// q, q + RG, ... of the segment with its own staging buffers, and the groups'
// partial sums are added through LDS at the end (fixed order, so the result
// does not depend on timing). Two groups fill a CU's wave slots when the grid
// alone would leave one workgroup per CU.
template <int D, bool DELTA, int CS, int RG>
__global__ __launch_bounds__(256 * RG) void gh_kernel(const uint16_t *k,  // not restrict:
                                                      const uint16_t *v,  // see load_chunk
                                                      Layout lkv, int Hkv,
                                                      const float *__restrict__ z_pre,
                                                      float *__restrict__ gh,
                                                      uint16_t *__restrict__ vt, int vt_tiles,
                                                      int L, int N, int S, float eps) {
  constexpr int ND = D / 32;
  constexpr int CCH = D / 8;            // 8-column chunks per row
  constexpr int ITEMS = 16 * CCH;       // staging items: 4 rows x 8 columns each
  constexpr int NPAIR = DELTA ? 2 * ND : ND;  // (matrix, column tile) pairs
  constexpr int PPW = (NPAIR + 4 * CS - 1) / (4 * CS);  // pairs per wave
  constexpr int NB = DELTA ? 3 : 2;     // staging buffers per group: sigma(K)^T, V^T, (W^T)
  static_assert(ITEMS <= 256, "one staging item per thread of a group");
  static_assert(RG == 1 || 4 * PPW * ND * 16 * 64 * 4 <= RG * NB * D * kStr * 2,
                "the partial sums of a group fit in the staging buffers");

  // Per group: sigma(K)^T, V^T and (delta) (sigma(K)/den)^T, [col][key].
  __shared__ __attribute__((aligned(16))) uint16_t sStage[RG][NB][D * kStr];
  __shared__ float sZ[D];

  // Work item wi = (head * S + s) * CS + cs. When the launch divides evenly,
  // consecutive work items go to one XCD (hardware hands out workgroups
  // round-robin over the 8 XCDs), so the CS workgroups that read the same rows
  // share that XCD's L2. Column split: workgroup cs owns pairs [p_lo, p_hi);
  // every workgroup stages the whole chunk.
  int wi = blockIdx.y * gridDim.x + blockIdx.x;
  const int total = gridDim.x * gridDim.y;
  if (CS > 1 && total % (8 * CS) == 0) wi = (wi % 8) * (total / 8) + wi / 8;
  const int cs = wi % CS, s = (wi / CS) % S, head = wi / CS / S;
  const int p_lo = cs * NPAIR / CS, p_hi = (cs + 1) * NPAIR / CS;
  const int a = s * N, e = min(a + N, L);
  const int tid = threadIdx.x, lane = tid & 63;
  // Wave within the group and thread within the group (written without a
  // mask when there is one group: the compiler then keeps the wave index
  // scalar and the accumulators in place).
  const int w = RG > 1 ? (__builtin_amdgcn_readfirstlane(tid >> 6) & 3) : (tid >> 6);
  const int grp = RG > 1 ? (tid >> 8) : 0;  // row group
  const int tg = RG > 1 ? (tid & 255) : tid;
  const int g = lane >> 5, l32 = lane & 31;
  uint16_t *sKt = sStage[grp][0];
  uint16_t *sVt = sStage[grp][1];
  uint16_t *sWt = sStage[grp][NB - 1];  // delta only
  const uint16_t *kp = k + head_offset(lkv, head, Hkv);
  const uint16_t *vp = v + head_offset(lkv, head, Hkv);
  if (tid < D) sZ[tid] = z_pre[(static_cast<size_t>(head) * (S + 1) + s) * D + tid];

  f32x16 acc[PPW][ND];
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi)
#pragma unroll
    for (int rt = 0; rt < ND; ++rt) acc[pi][rt] = f32x16{};

  // Chunk iterations of every group (the groups take chunks grp, grp + RG, ...).
  const int iters = ((e - a + 63) / 64 + RG - 1) / RG;
  const bool has = tg < ITEMS;
  // Rows 4 kg .. 4 kg + 3, columns 8 cc .. 8 cc + 7. The column chunks of a row
  // lie in consecutive lanes, so that each load of a wave reads whole rows.
  const int kg = tg / CCH, cc = tg % CCH;
  // The staging buffers hold [column][key], with key unit (4 keys, 8 bytes) u
  // of column c at position u ^ kswz(c). An 8-byte write is served per half
  // wave (32 lanes, 64 banks of 4 bytes). Column c = 8 cc + j of a row
  // (stride 34 words) starts at bank 16 cc + 34 j (mod 64), so the chunks cc
  // and cc + 4 of one write would meet. The swizzle XORs the unit with a
  // different multiple of 32 / CCH in each group of 32 columns (d = 128:
  // 2 ((c >> 5) & 3); d = 64: 4 ((c >> 5) & 1); d = 32: none), which moves
  // those chunks onto distinct banks: every write is conflict-free. The
  // operand reads take one unit of 32 consecutive columns, whose swizzle is
  // one value, so their pattern (conflict-free) is unchanged.
  auto kswz = [](int col) __attribute__((always_inline)) {
    return ((col >> 5) & (CCH / 4 - 1)) * (32 / CCH);
  };
  auto kpos = [&](int col, int unit) __attribute__((always_inline)) {
    return col * kStr + 4 * (unit ^ kswz(col));
  };

  // Register staging of 64-row chunks (4 rows x 8 columns per item), two
  // register sets: a chunk's loads are issued two chunks before it is staged.
  // Every item issues all its loads (rows past the segment end read its last
  // row, and staging masks them), so the compiler's count of loads in flight
  // is the same on every path and its waits cover exactly the chunk being
  // staged. The empty asm statements keep the loads where they are issued
  // (k and v are not restrict, so they cannot be moved across them).
  struct Stage {
    u32x4 k[4], v[4];
  };
  auto load_chunk = [&](Stage &st, int i0) __attribute__((always_inline)) {
    if (has) {
      __asm__ volatile("" ::: "memory");
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const long long row = min(i0 + 4 * kg + r, e - 1);
        st.k[r] = *reinterpret_cast<const u32x4 *>(kp + row * lkv.sr + cc * 8);
        st.v[r] = *reinterpret_cast<const u32x4 *>(vp + row * lkv.sr + cc * 8);
      }
      __asm__ volatile("" ::: "memory");
    }
  };

  auto chunk = [&](int i0, Stage &cur) {
    lds_barrier();  // previous chunk consumed; sZ visible
    const u32x4 *kw = cur.k;
    const u32x4 *vv = cur.v;
    float kf[4][8];
    if (has) {
      uint32_t vw[4][4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool in = i0 + 4 * kg + r < e;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          // rows past the segment end contribute nothing: sigma forced to 0
          kf[r][2 * jj] = in ? elu1(lo_bf16(kw[r][jj])) : 0.f;
          kf[r][2 * jj + 1] = in ? elu1(hi_bf16(kw[r][jj])) : 0.f;
          vw[r][jj] = in ? vv[r][jj] : 0u;
        }
      }
      // transposed stores: one 8-byte write of 4 keys per column
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const u32x2 kk2 = {pack_bf16x2(kf[0][j], kf[1][j]), pack_bf16x2(kf[2][j], kf[3][j])};
        *reinterpret_cast<u32x2 *>(sKt + kpos(cc * 8 + j, kg)) = kk2;
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const uint32_t r0 = vw[0][jj], r1 = vw[1][jj], r2 = vw[2][jj], r3 = vw[3][jj];
        const u32x2 lo = {(r0 & 0xffffu) | (r1 << 16), (r2 & 0xffffu) | (r3 << 16)};
        const u32x2 hi = {(r0 >> 16) | (r1 & 0xffff0000u), (r2 >> 16) | (r3 & 0xffff0000u)};
        *reinterpret_cast<u32x2 *>(sVt + kpos(cc * 8 + 2 * jj, kg)) = lo;
        *reinterpret_cast<u32x2 *>(sVt + kpos(cc * 8 + 2 * jj + 1, kg)) = hi;
      }
      if constexpr (DELTA) {
        // den_i = sigma(k_i).z + eps: this thread's 8 columns, then the
        // row's CCH chunks, which sit in consecutive lanes (DPP: lane pairs,
        // quads, mirrored halves of 8 and of 16 lanes; every lane ends with
        // the same sum). Then (sigma(K) / den)^T, one 8-byte write per column.
        float rd[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) x += kf[r][j] * sZ[cc * 8 + j];
          x += dpp_f32<0xB1>(x);  // lane ^ 1
          x += dpp_f32<0x4E>(x);  // lane ^ 2
          if constexpr (CCH >= 8) x += dpp_f32<0x141>(x);  // lane i <-> 7 - i
          if constexpr (CCH >= 16) x += dpp_f32<0x140>(x);  // lane i <-> 15 - i
          // (v_rcp_f32, within 1 ulp: W is rounded to bf16 right after.)
          rd[r] = __builtin_amdgcn_rcpf(x + eps);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const u32x2 w2 = {pack_bf16x2(kf[0][j] * rd[0], kf[1][j] * rd[1]),
                            pack_bf16x2(kf[2][j] * rd[2], kf[3][j] * rd[3])};
          *reinterpret_cast<u32x2 *>(sWt + kpos(cc * 8 + j, kg)) = w2;
        }
      }
    }
    lds_barrier();
    if (cs == 0 && i0 < e) {
      // V^T of this 64-key chunk (rows past the segment end are zero), in the
      // unit order and bank swizzle of vt_unit_pos. Stored before the next
      // loads are issued, so that waiting for those never waits for these.
      uint16_t *vtile =
          vt + ((static_cast<size_t>(head) * S + s) * vt_tiles + (i0 - a) / 64) * (D * 64);
#pragma unroll
      for (int uu = 0; uu < D * 8 / 256; ++uu) {
        const int u = tg + 256 * uu;
        const int d = u >> 3;
        const int q = vt_unit_pos(d, u & 7);  // the swizzle is its own inverse
        const int u0 = 4 * (q >> 1) + (q & 1);  // key units u0 and u0 + 2
        const u32x2 r0 = *reinterpret_cast<const u32x2 *>(sVt + kpos(d, u0));
        const u32x2 r1 = *reinterpret_cast<const u32x2 *>(sVt + kpos(d, u0 + 2));
        *reinterpret_cast<u32x4 *>(vtile + u * 8) = u32x4{r0[0], r0[1], r1[0], r1[1]};
      }
    }
    // cur is free once staged: load the chunk this set takes next (copies of
    // the last row, for a chunk the loop never stages).
    load_chunk(cur, i0 + 128 * RG);

    // Contraction over the 64 keys of the chunk, 16 per MFMA. Slot j of lane
    // group g is key kb + 8 (j / 4) + 4 g + j % 4 in both operands.
#pragma unroll
    for (int kb = 0; kb < 64; kb += 16) {
      u32x4 av[ND];
#pragma unroll
      for (int rt = 0; rt < ND; ++rt) {
        const int col = 32 * rt + l32;
        const u32x2 x0 = *reinterpret_cast<const u32x2 *>(sKt + kpos(col, kb / 4 + g));
        const u32x2 x1 = *reinterpret_cast<const u32x2 *>(sKt + kpos(col, kb / 4 + 2 + g));
        av[rt] = u32x4{x0[0], x0[1], x1[0], x1[1]};
      }
#pragma unroll
      for (int pi = 0; pi < PPW; ++pi) {
        const int pr = p_lo + w + 4 * pi;
        if (pr < p_hi) {
          const bool is_g = DELTA && pr < ND;
          const int ct = pr % ND;
          const uint16_t *src = is_g ? sWt : sVt;
          const int col = 32 * ct + l32;
          const u32x2 x0 = *reinterpret_cast<const u32x2 *>(src + kpos(col, kb / 4 + g));
          const u32x2 x1 = *reinterpret_cast<const u32x2 *>(src + kpos(col, kb / 4 + 2 + g));
          const u32x4 bv = {x0[0], x0[1], x1[0], x1[1]};
#pragma unroll
          for (int rt = 0; rt < ND; ++rt) acc[pi][rt] = mfma_bf16(av[rt], bv, acc[pi][rt]);
        }
      }
    }
  };
  // Group grp takes chunks grp, grp + RG, ...; every group runs the same
  // number of iterations (the barriers are workgroup-wide), a chunk past the
  // segment end contributing nothing.
  Stage sa, sb;
  load_chunk(sa, a + 64 * grp);
  load_chunk(sb, a + 64 * (RG + grp));
  // Whole pairs of chunks, then an odd last one: a loop with a single exit,
  // so that the loop head is reached only after both sets' loads were issued.
  int j = 0;
  for (; j + 2 <= iters; j += 2) {
    chunk(a + 64 * (RG * j + grp), sa);
    chunk(a + 64 * (RG * (j + 1) + grp), sb);
  }
  if (j < iters) chunk(a + 64 * (RG * j + grp), sa);
  if constexpr (RG > 1) {
    // Add the other groups' partial sums into group 0 (staging buffers reused).
    float *sAcc = reinterpret_cast<float *>(&sStage[0][0][0]);
    lds_barrier();
    for (int q = 1; q < RG; ++q) {
      if (grp == q) {
#pragma unroll
        for (int pi = 0; pi < PPW; ++pi)
#pragma unroll
          for (int rt = 0; rt < ND; ++rt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              sAcc[(((w * PPW + pi) * ND + rt) * 16 + r) * 64 + lane] = acc[pi][rt][r];
      }
      lds_barrier();
      if (grp == 0) {
#pragma unroll
        for (int pi = 0; pi < PPW; ++pi)
#pragma unroll
          for (int rt = 0; rt < ND; ++rt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              acc[pi][rt][r] += sAcc[(((w * PPW + pi) * ND + rt) * 16 + r) * 64 + lane];
      }
      lds_barrier();
    }
    if (grp != 0) return;
  }

  // Store in fragment order: matrix 0 = G as bf16 hi/lo operand words
  // (hi = bf16(x), lo = bf16(x - hi)), matrix 1 = H as fp32.
  float *base = gh + (static_cast<size_t>(head) * S + s) * 2 * D * D;
#pragma unroll
  for (int pi = 0; pi < PPW; ++pi) {
    const int pr = p_lo + w + 4 * pi;
    if (pr < p_hi) {
      const int mat = (DELTA && pr < ND) ? 0 : 1;
      const int ct = pr % ND;
#pragma unroll
      for (int rt = 0; rt < ND; ++rt) {
        if (mat == 0) {
          uint32_t wd[16];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float x0 = acc[pi][rt][2 * q], x1 = acc[pi][rt][2 * q + 1];
            const uint32_t hw = pack_bf16x2(x0, x1);
            wd[q] = hw;
            wd[8 + q] = pack_bf16x2(x0 - lo_bf16(hw), x1 - hi_bf16(hw));
          }
          u32x4 *f = reinterpret_cast<u32x4 *>(base) + (rt * ND + ct) * 256 + lane;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            f[64 * q] = u32x4{wd[4 * q], wd[4 * q + 1], wd[4 * q + 2], wd[4 * q + 3]};
        } else {
          f32x4 *f = reinterpret_cast<f32x4 *>(base + static_cast<size_t>(D) * D) +
                     (rt * ND + ct) * 256 + lane;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            f[64 * q] = f32x4{acc[pi][rt][4 * q], acc[pi][rt][4 * q + 1], acc[pi][rt][4 * q + 2],
                         acc[pi][rt][4 * q + 3]};
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// seq: the recurrence over segments for one 32-column tile of M.
// Wave w holds rows 32 w .. 32 w + 31 of the tile in MFMA-result layout
// (lane: column 32 jt + l % 32; register r: row 32 w + kappa(r, l / 32)).
// The tile's current state is also kept in LDS, transposed, as bf16 hi and lo
// parts (sMh[n][c], sMl[n][c]: column n of the tile, row c of M), which is the
// B operand of G_s M_{s-1}. Its hi part is the bf16 snapshot M_{s-1}^T.
//
// The affine steps M_s = (I - G_s) M_{s-1} + H_s compose associatively, so a
// long chain is also run as a chunked scan (modes below, chunks of C
// segments): PRODUCT runs every chunk at once from the states [I | 0],
// giving X_c = [P_c | h_c] with P_c the product of the chunk's (I - G_s) and
// h_c its chain from zero; chain_pack_kernel turns each into one affine step
// (G' = I - P_c, H' = h_c); CHAIN runs those steps over the chunks,
// recording the fp32 state before each chunk; APPLY reruns every chunk at
// once from its recorded state and writes the per-segment snapshots.
//   FULL     grid (D/32, heads): segments 0 .. S - 1 from M, snapshots, M_S.
//   PRODUCT  grid (2 D/32, heads x chunks): tile jt < D/32 is column tile jt
//            of P_c (starts as I, no H), tile D/32 + jt that of h_c (starts
//            at 0); writes X [heads][chunks][D][2D] (fp32, row-major).
//   CHAIN    grid (D/32, heads): steps over the chunks (gh = packed steps),
//            fp32 state before each chunk into states, M_S into M.
//   APPLY    grid (D/32, heads x chunks): from states, the chunk's segments,
//            snapshots.
// ---------------------------------------------------------------------------
enum SeqMode { kSeqFull = 0, kSeqProduct = 1, kSeqChain = 2, kSeqApply = 3 };

struct SeqArgs {
  const float *gh;   // [heads][S][2][D*D] fragments of (G_s, H_s) (CHAIN: packed chunk steps)
  int S;             // steps per head in gh
  int C;             // segments per chunk (PRODUCT, APPLY)
  int nchunks;       // chunks per head (PRODUCT, APPLY)
  float *M;          // FULL, CHAIN: initial state in, final state out
  uint16_t *mt_pre;  // FULL, APPLY: bf16 M^T before each segment [heads][S][D][D]
  float *states;     // CHAIN (out), APPLY (in): fp32 state before each chunk [heads][chunks][D][D]
  float *X;          // PRODUCT (out): [heads][chunks][D][2D]
};

template <int D, bool DELTA, int MODE>
__global__ __launch_bounds__(64 * (D / 32)) void seq_kernel(SeqArgs args) {
  constexpr int ND = D / 32;
  constexpr int MS = D + 4;  // sMh / sMl row stride (bf16)
  static_assert(DELTA || MODE == kSeqFull, "chunked modes are for the delta rule");
  __shared__ __attribute__((aligned(16))) uint16_t sMh[DELTA ? 32 * MS : 4];
  __shared__ __attribute__((aligned(16))) uint16_t sMl[DELTA ? 32 * MS : 4];
  // (gh is not restrict: see step().)
  const float *gh = args.gh;
  const int S = args.S;
  // Workgroups are dealt round-robin to the 8 XCDs, each with its own L2.
  // All column tiles of a head read the whole G_s, so when the grid allows it
  // they are placed on one XCD: linear id (8 (jt + nt u8) + u % 8), with u8 =
  // u / 8, holds tile jt of unit u (a head, or a (head, chunk) pair).
  // (PRODUCT and APPLY: the same for the tiles of one (head, chunk) unit.)
  int jt = blockIdx.x, unit = blockIdx.y, chunk = 0;
  if (gridDim.y % 8 == 0) {
    const int nt = gridDim.x;  // column tiles per unit
    const int id = blockIdx.y * nt + blockIdx.x;
    jt = (id >> 3) % nt;
    unit = (id & 7) + 8 * ((id >> 3) / nt);
  }
  int head = unit;
  if (MODE == kSeqProduct || MODE == kSeqApply) {
    head = unit / args.nchunks;
    chunk = unit % args.nchunks;
  }
  const int s_begin = (MODE == kSeqProduct || MODE == kSeqApply) ? chunk * args.C : 0;
  const int s_end = (MODE == kSeqProduct || MODE == kSeqApply) ? min(s_begin + args.C, S) : S;
  const int lane = threadIdx.x & 63, ct = threadIdx.x >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  // This tile's columns of the state (PRODUCT: of [P | h]) and of H.
  const int j = 32 * jt + l32;
  const int jh = (MODE == kSeqProduct) ? 32 * (jt % ND) + l32 : j;
  const bool add_h = MODE != kSeqProduct || jt >= ND;

  f32x16 m;
  if (MODE == kSeqFull || MODE == kSeqChain) {
    const float *Mh = args.M + static_cast<size_t>(head) * D * D;
#pragma unroll
    for (int r = 0; r < 16; ++r) m[r] = Mh[static_cast<size_t>(32 * ct + kappa(r, g)) * D + j];
  } else if (MODE == kSeqApply) {
    const float *X0 =
        args.states + (static_cast<size_t>(head) * args.nchunks + chunk) * D * D;
#pragma unroll
    for (int r = 0; r < 16; ++r) m[r] = X0[static_cast<size_t>(32 * ct + kappa(r, g)) * D + j];
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) m[r] = (jt < ND && 32 * ct + kappa(r, g) == j) ? 1.f : 0.f;
  }

  // The state before segment st: the global bf16 snapshot M_{st-1}^T (st < S)
  // and, for the delta rule, the hi/lo operand copy in LDS. This lane holds
  // rows 32 ct + 8 q4 + 4 g + 0..3, which are contiguous in the transposed
  // layouts.
  // The two lanes holding one row of the snapshot (32 apart) swap halves
  // first (upper half of the first operand with the lower half of the
  // second), so that each lane stores 8 contiguous values: rows
  // 32 ct + 16 p + 8 g + 0..7, one 16-byte store per p.
  auto snapshot = [&](int st) __attribute__((always_inline)) {
    if (MODE == kSeqChain) {
      // fp32 state before chunk st, row-major.
      float *xs = args.states + (static_cast<size_t>(head) * S + st) * D * D + j;
#pragma unroll
      for (int r = 0; r < 16; ++r) xs[static_cast<size_t>(32 * ct + kappa(r, g)) * D] = m[r];
      return;
    }
    if (MODE == kSeqProduct) return;
    uint16_t *mt = args.mt_pre + (static_cast<size_t>(head) * S + st) * D * D +
                   static_cast<size_t>(j) * D + 32 * ct + 8 * g;
    uint32_t wd[4][2];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      wd[q4][0] = pack_bf16x2(m[4 * q4], m[4 * q4 + 1]);
      wd[q4][1] = pack_bf16x2(m[4 * q4 + 2], m[4 * q4 + 3]);
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      uint32_t x[2], y[2];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const auto r = __builtin_amdgcn_permlane32_swap(wd[2 * p][jj], wd[2 * p + 1][jj], false,
                                                        false);
        x[jj] = r[0];
        y[jj] = r[1];
      }
      *reinterpret_cast<u32x4 *>(mt + 16 * p) = u32x4{x[0], x[1], y[0], y[1]};
    }
  };
  auto operand = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const uint32_t h0 = pack_bf16x2(m[4 * q4], m[4 * q4 + 1]);
      const uint32_t h1 = pack_bf16x2(m[4 * q4 + 2], m[4 * q4 + 3]);
      const int off = l32 * MS + 32 * ct + 8 * q4 + 4 * g;
      *reinterpret_cast<u32x2 *>(sMh + off) = u32x2{h0, h1};
      *reinterpret_cast<u32x2 *>(sMl + off) =
          u32x2{pack_bf16x2(m[4 * q4] - lo_bf16(h0), m[4 * q4 + 1] - hi_bf16(h0)),
                pack_bf16x2(m[4 * q4 + 2] - lo_bf16(h1), m[4 * q4 + 3] - hi_bf16(h1))};
    }
  };

  // G_s / H_s fragments of a step, loaded R - 1 steps ahead through a ring of
  // R register sets (the loop is unrolled R times, so the sets do not move):
  // 3 for the delta rule's chains (80 registers a set), 8 for the linear rule
  // (16). G: 4
  // operand vectors (hi h = 0, 1, lo h = 0, 1) per 32-row tile kt of the
  // contraction; H: this lane's 16 values. Every step issues its loads (past
  // the last segment of the range it reloads the last one), so that the wait
  // before a step's work covers exactly the loads R - 1 steps old.
  // (The chunk-parallel passes run thousands of independent workgroups,
  // whose latencies overlap each other: they keep a shorter ring, so that two
  // waves fit on a SIMD.)
  constexpr int NG = DELTA ? ND : 1;
  constexpr int R = (MODE == kSeqProduct || MODE == kSeqApply) ? 2 : (DELTA ? 3 : 8);
  struct Frags {
    u32x4 g[NG][4];
    f32x4 h[4];
  };
  auto load_step = [&](int st, Frags &f) __attribute__((always_inline)) {
    st = min(st, s_end - 1);
    const float *ghs = gh + (static_cast<size_t>(head) * S + st) * 2 * D * D;
    const f32x4 *hf = reinterpret_cast<const f32x4 *>(ghs + static_cast<size_t>(D) * D) +
                      (ct * ND + jh / 32) * 256 + lane;
#pragma unroll
    for (int q = 0; q < 4; ++q) f.h[q] = hf[64 * q];
    if constexpr (DELTA) {
#pragma unroll
      for (int kt = 0; kt < ND; ++kt) {
        const u32x4 *gf = reinterpret_cast<const u32x4 *>(ghs) + (kt * ND + ct) * 256 + lane;
#pragma unroll
        for (int q = 0; q < 4; ++q) f.g[kt][q] = gf[64 * q];
      }
    }
  };
  // One segment: store the snapshot of the state before it, start the loads
  // of the segment R - 1 ahead, then M += H_s (- G_s M for the delta rule).
  auto step = [&](int s, const Frags &cur, Frags &ahead) __attribute__((always_inline)) {
    // (The empty asm statements keep the snapshot stores and the loads at the
    // top of their step: the compiler would otherwise sink loads whose values
    // are needed two steps later past the loop exits toward their use. They
    // can only do so because gh is not declared restrict.)
    __asm__ volatile("" ::: "memory");
    snapshot(s);
    load_step(s + R - 1, ahead);
    __asm__ volatile("" ::: "memory");
    if constexpr (DELTA) {
      // (G M)[32 ct + m][j] = sum_c G[c][32 ct + m] M[c][j] over c = 32 kt +
      // 16 h + 8 (slot / 4) + 4 g + slot % 4 in both operands.
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kt = 0; kt < ND; ++kt) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int off = l32 * MS + 32 * kt + 16 * h + 4 * g;
          const u32x2 h0 = *reinterpret_cast<const u32x2 *>(sMh + off);
          const u32x2 h1 = *reinterpret_cast<const u32x2 *>(sMh + off + 8);
          const u32x2 l0 = *reinterpret_cast<const u32x2 *>(sMl + off);
          const u32x2 l1 = *reinterpret_cast<const u32x2 *>(sMl + off + 8);
          const u32x4 bh = {h0[0], h0[1], h1[0], h1[1]};
          const u32x4 bl = {l0[0], l0[1], l1[0], l1[1]};
          acc = mfma_bf16(cur.g[kt][h], bh, acc);
          acc = mfma_bf16(cur.g[kt][h], bl, acc);
          acc = mfma_bf16(cur.g[kt][2 + h], bh, acc);
        }
      }
      lds_barrier();  // every wave has read M_{s-1} from LDS
      if (add_h) {
#pragma unroll
        for (int r = 0; r < 16; ++r) m[r] = m[r] - acc[r] + cur.h[r / 4][r % 4];
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) m[r] = m[r] - acc[r];
      }
      operand();
      lds_barrier();
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) m[r] += cur.h[r / 4][r % 4];
    }
  };

  Frags f[R];
  if (s_end > s_begin) {
#pragma unroll
    for (int r = 0; r + 1 < R; ++r) load_step(s_begin + r, f[r]);
    if constexpr (DELTA) {
      operand();
      lds_barrier();
    }
    // Whole rounds of R steps, then the rest (fewer than R). The rounds have
    // no exits inside, so every path into the loop head has the same loads in
    // flight and the waits stay exact.
    int s = s_begin;
    for (; s + R <= s_end; s += R) {
#pragma unroll
      for (int r = 0; r < R; ++r) step(s + r, f[r], f[(r + R - 1) % R]);
    }
#pragma unroll
    for (int r = 0; r + 1 < R; ++r)
      if (s + r < s_end) step(s + r, f[r], f[(r + R - 1) % R]);
  }
  if (MODE == kSeqFull || MODE == kSeqChain) {
    float *Mh = args.M + static_cast<size_t>(head) * D * D;
#pragma unroll
    for (int r = 0; r < 16; ++r) Mh[static_cast<size_t>(32 * ct + kappa(r, g)) * D + j] = m[r];
  } else if (MODE == kSeqProduct) {
    float *Xc = args.X + (static_cast<size_t>(head) * args.nchunks + chunk) * D * (2 * D) + j;
#pragma unroll
    for (int r = 0; r < 16; ++r) Xc[static_cast<size_t>(32 * ct + kappa(r, g)) * (2 * D)] = m[r];
  }
  // The loads issued past the last segment land before the wave ends (vmcnt 0,
  // lgkmcnt 0, expcnt at its maximum; gfx9 s_waitcnt encoding).
  __builtin_amdgcn_s_waitcnt(7 << 4);
}

// One affine step per chunk from X_c = [P_c | h_c]: G' = I - P_c, stored
// transposed in the G fragment format (the recurrence reads tile (kt, ct)
// of G as its operand for output rows ct, contracting over the rows of tile
// kt, i.e. it applies the transpose of what is stored), as bf16 hi/lo words;
// H' = h_c in the H fragment format (fp32). One thread per (unit, tile, lane).
template <int D>
__global__ __launch_bounds__(256) void chain_pack_kernel(const float *__restrict__ X,
                                                         float *__restrict__ gh2, int units) {
  constexpr int ND = D / 32;
  const long long tid = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
  if (tid >= static_cast<long long>(units) * ND * ND * 64) return;
  const int lane = static_cast<int>(tid % 64);
  const int tile = static_cast<int>((tid / 64) % (ND * ND));
  const size_t unit = static_cast<size_t>(tid / (64 * ND * ND));
  const int rt = tile / ND, ct = tile % ND;
  const int g = lane >> 5, l32 = lane & 31;
  const float *Xu = X + unit * D * (2 * D);
  float gv[16], hv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 32 * rt + kappa(r, g), col = 32 * ct + l32;
    // stored element (row, col) of G' = (I - P)[col][row]
    gv[r] = (row == col ? 1.f : 0.f) - Xu[static_cast<size_t>(col) * (2 * D) + row];
    hv[r] = Xu[static_cast<size_t>(row) * (2 * D) + D + col];
  }
  float *base = gh2 + unit * 2 * D * D;
  uint32_t wd[16];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t hw = pack_bf16x2(gv[2 * q], gv[2 * q + 1]);
    wd[q] = hw;
    wd[8 + q] = pack_bf16x2(gv[2 * q] - lo_bf16(hw), gv[2 * q + 1] - hi_bf16(hw));
  }
  u32x4 *fg = reinterpret_cast<u32x4 *>(base) + tile * 256 + lane;
  f32x4 *fh = reinterpret_cast<f32x4 *>(base + static_cast<size_t>(D) * D) + tile * 256 + lane;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    fg[64 * q] = u32x4{wd[4 * q], wd[4 * q + 1], wd[4 * q + 2], wd[4 * q + 3]};
    fh[64 * q] = f32x4{hv[4 * q], hv[4 * q + 1], hv[4 * q + 2], hv[4 * q + 3]};
  }
}

template <int D>
hipError_t launch_d(const Geometry &g, const uint16_t *k, const uint16_t *v, float *M,
                    float *z, int delta, const Workspace &ws, hipStream_t stream) {
  const int heads = g.B * g.Hkv;
  const int parts = ws.z_parts;
  // Few (segment, head) pairs: split each one's output tiles over two
  // workgroups so that the launch still covers the chip.
  const bool split = g.S * heads < 512;
  const dim3 ghgrid(g.S * (split ? 2 : 1), heads), seqgrid(D / 32, heads);
  // With the column split, two row groups per workgroup (512 threads) fill
  // the CU's wave slots; without it the accumulators leave room for one.
  zsum_kernel<D><<<dim3(g.S * parts, heads), 256, 0, stream>>>(k, g.lkv, g.Hkv, ws.dz, g.L, g.N,
                                                                g.S, parts);
  zprefix_kernel<<<dim3(D / kZCols, heads), kZThreads, 0, stream>>>(z, ws.dz, ws.z_pre, ws.z_hl,
                                                                     g.S, D, parts, z);
  if (delta) {
    if (split)
      gh_kernel<D, true, 2, 2><<<ghgrid, 512, 0, stream>>>(k, v, g.lkv, g.Hkv, ws.z_pre, ws.gh,
                                                        ws.vt, ws.vt_tiles, g.L, g.N, g.S, g.eps);
    else
      gh_kernel<D, true, 1, 1><<<ghgrid, 256, 0, stream>>>(k, v, g.lkv, g.Hkv, ws.z_pre, ws.gh,
                                                        ws.vt, ws.vt_tiles, g.L, g.N, g.S, g.eps);
    SeqArgs a{ws.gh, g.S, 0, 0, M, ws.mt_pre_bf16, nullptr, nullptr};
    if (ws.chunk_len > 0) {
      // Chunked scan of the affine chain (see seq_kernel).
      const int C = ws.chunk_len, nc = (g.S + C - 1) / C;
      const long long units = static_cast<long long>(heads) * nc;
      a.C = C;
      a.nchunks = nc;
      a.X = ws.chain_x;
      seq_kernel<D, true, kSeqProduct><<<dim3(2 * D / 32, static_cast<unsigned>(units)),
                                         64 * (D / 32), 0, stream>>>(a);
      const long long threads = units * (D / 32) * (D / 32) * 64;
      chain_pack_kernel<D><<<static_cast<unsigned>((threads + 255) / 256), 256, 0, stream>>>(
          ws.chain_x, ws.chain_gh, static_cast<int>(units));
      SeqArgs c{ws.chain_gh, nc, 0, 0, M, nullptr, ws.chain_states, nullptr};
      seq_kernel<D, true, kSeqChain><<<seqgrid, 64 * (D / 32), 0, stream>>>(c);
      a.states = ws.chain_states;
      seq_kernel<D, true, kSeqApply><<<dim3(D / 32, static_cast<unsigned>(units)), 64 * (D / 32),
                                       0, stream>>>(a);
    } else {
      seq_kernel<D, true, kSeqFull><<<seqgrid, 64 * (D / 32), 0, stream>>>(a);
    }
  } else {
    if (split)
      gh_kernel<D, false, 2, 2><<<ghgrid, 512, 0, stream>>>(k, v, g.lkv, g.Hkv, ws.z_pre, ws.gh,
                                                         ws.vt, ws.vt_tiles, g.L, g.N, g.S, g.eps);
    else
      gh_kernel<D, false, 1, 1><<<ghgrid, 256, 0, stream>>>(k, v, g.lkv, g.Hkv, ws.z_pre, ws.gh,
                                                         ws.vt, ws.vt_tiles, g.L, g.N, g.S, g.eps);
    SeqArgs a{ws.gh, g.S, 0, 0, M, ws.mt_pre_bf16, nullptr, nullptr};
    seq_kernel<D, false, kSeqFull><<<seqgrid, 64 * (D / 32), 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

int chain_chunk_len(int S, int heads) {
  if (S < 64) return 0;
  int C = static_cast<int>(sqrtf(static_cast<float>(S) / 2.f) + 0.5f);
  C = C < 4 ? 4 : C;
  const long long units = static_cast<long long>(heads) * ((S + C - 1) / C);
  return units > 65535 ? 0 : C;
}

hipError_t launch_segment_scan_bf16(const Geometry &g, const uint16_t *k, const uint16_t *v,
                                    float *M, float *z, int delta, const Workspace &ws,
                                    hipStream_t stream) {
  switch (g.D) {
    case 32: return launch_d<32>(g, k, v, M, z, delta, ws, stream);
    case 64: return launch_d<64>(g, k, v, M, z, delta, ws, stream);
    case 128: return launch_d<128>(g, k, v, M, z, delta, ws, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace ia
