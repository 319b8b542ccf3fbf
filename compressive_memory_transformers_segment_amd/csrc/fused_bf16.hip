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
//   * Q stays in registers for the whole key loop of a work item (its
//     d-contiguous rows are exactly the B operand of S^T = K Q^T).
//   * Persistent workgroups (as many as fit on the chip at once) work through
//     a static schedule of work items (query tile x head unit x segment) that
//     alternates long and short query tiles, so every workgroup gets about
//     the same number of key tiles. All data a workgroup needs moves from HBM
//     to LDS by direct loads (buffer_load ... lds for the key tiles, whose
//     per-lane offsets are the same for every tile, global_load_lds for the
//     per-item slots: no register staging, no LDS store instructions)
//     through a ring of three buffers, as one continuous stream of slots
//     across items: per item its key tiles (padded to a
//     multiple of three slots), M^T of the segment, then the next item's Q
//     rows. The loads run two slots ahead of the work, so the next item's Q,
//     tiles and snapshot are in flight while the current one finishes and no
//     item waits for its inputs. Each wave waits only for its own loads of the
//     next slot before the one barrier per slot.
//   * K tiles (and M^T, Q) are row-major with a 16-byte-unit XOR swizzle so
//     that the 32 rows an MFMA operand reads hit distinct banks. V arrives
//     already transposed, [d][key], from the segment scan, which writes it per
//     64-key tile with the keys of each 16-key step permuted so that the 8
//     keys a lane contributes to one O^T = V^T P^T MFMA (two runs of 4 in the
//     S^T result layout) are adjacent and bank-swizzled: every MFMA operand
//     read from LDS is one 16-byte read.
//   * Causal skipping: an item visits key tiles up to its last query row; a
//     wave skips tiles entirely in its future and masks only diagonal tiles.
//   * Online softmax with a lazy rescale: the running max m of a row moves
//     (and O, l are rescaled) only when a tile's max exceeds m by more than
//     kLazy (log2 units), so probabilities stay <= 2^kLazy and most tiles skip
//     the rescale. The 1/sqrt(d) scale is folded into the exponent's FMA, and
//     the row sum is a bf16 dot2 over the same rounded P the MFMA consumes.
//     The kernel runs with the IEEE mode bit off (no NaN quieting on max).
//   * In every round the workgroups of one XCD (workgroups are dealt
//     round-robin to the 8 XCDs) take consecutive items: the query tiles that
//     read one kv head's segment share that XCD's L2.
//   * Epilogue: the pre-segment snapshot M^T (bf16, [d_v][d_k]) arrives as a
//     ring slot, once for all heads of the workgroup, and is multiplied with
//     sigma(Q) (computed in place of the Q registers) on MFMA; so is the
//     denominator sigma(Q).z, from the same bf16 sigma(Q) and z split into
//     bf16 hi and lo parts (z and the gate parameters travel in a side area
//     of the snapshot's slot).
//     Rows are stored through a buffer resource that ends at the segment end,
//     so every wave issues the same stores and the hardware drops those past
//     it. The two lanes that hold one row exchange halves first, so that each
//     store writes 16 contiguous bytes per lane (32 per row and instruction).

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

// sigma(x) = ELU(x) + 1 without a compare and select: the exponential clamped
// to [0, 1] (the clamp is a free output modifier of v_exp) is exp(x) for
// x <= 0 and exactly 1 for x > 0, so adding max(x, 0) gives x + 1 there and
// leaves exp(x) otherwise; the same values as the select form, bit for bit.
// (A NaN in q may come out of it as a number, but its row's scores, and so
// the row's output, are NaN regardless.)
__device__ __forceinline__ float elu1_clamped(float x) {
  return __builtin_amdgcn_fmed3f(__expf(x), 0.f, 1.f) + fmaxf(x, 0.f);
}

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

// One 16-byte-per-lane direct load from a buffer resource into LDS (lane l's
// unit lands at lds + 16 l bytes); voffset per lane, soffset uniform.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, uint16_t *lds,
                                                  int voffset, int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, IA_LDS(lds), 16, voffset, soffset, 0, 0);
}

template <int D>
struct Tile {
  static constexpr int CPR = D / 8;          // 16-byte units per K (and M^T, Q) row
  static constexpr int RP = 16 / CPR;        // K rows per 256-byte bank line
  static constexpr int KU = kBN * CPR;       // K units per tile
  static constexpr int VU = D * 8;           // V^T units per tile (64 keys per row)
  static constexpr int BUFU = KU + VU;       // 16-byte units per ring slot
  static constexpr int SIDE = kWaves * 64;   // words in a slot's side area (z, beta)
  static constexpr int BUF = BUFU * 8 + 2 * SIDE;  // bf16 per ring slot
  static constexpr int IPW = BUFU / kThreads;  // 16-byte direct loads per wave per slot
  static constexpr int MU = D * CPR;         // M^T units
  static_assert(BUFU % kThreads == 0, "whole direct loads per wave");
  static_assert(KU % 64 == 0, "a direct load never straddles K and V^T");
  static_assert(4 * 32 * CPR == BUFU, "the Q rows of four waves fill one slot");
  static_assert(MU <= BUFU, "M^T fits one slot");
};

// 16-byte unit of (row r, unit c) in a swizzled row-major tile of D columns
// (K tiles and M^T): 16 consecutive rows read at one unit index land on
// distinct banks.
template <int D>
__device__ __forceinline__ int swz_unit(int r, int c) {
  using TL = Tile<D>;
  return r * TL::CPR + (c ^ ((r / TL::RP) % TL::CPR));
}

// One work item of the persistent schedule: a query tile of one head unit
// (HPW query heads of one kv head) in one segment. Uniform across the
// workgroup.
struct FusedItem {
  int k;     // round of the item in its workgroup's schedule; -1 past the last item
  int a, e;  // rows [a, e) of the segment
  int q0;    // first query row of the tile
  int T;     // key tiles under the causal mask
  int bq;    // b * Hq + first query head of the head unit
  int head;  // b * Hkv + kv head
  int s;     // segment index
};

// Unsigned division by a divisor fixed for the launch (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994):
// with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1, the quotient of
// any 32-bit x is (t + ((x - t) >> s1)) >> s2, t = the high word of m x,
// s1 = min(l, 1), s2 = max(l - 1, 0). A multiply-high, a subtraction, two
// shifts and an add, all scalar for uniform x, where a division would expand
// into a vector sequence.
struct FastDiv {
  uint32_t d, m, s1, s2;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while (l < 32 && (uint64_t{1} << l) < d) ++l;
  FastDiv f;
  f.d = d;
  f.m = static_cast<uint32_t>(((uint64_t{(uint64_t{1} << l) - d}) << 32) / d + 1);
  f.s1 = l > 0 ? 1 : 0;
  f.s2 = l > 0 ? l - 1 : 0;
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t x, const FastDiv &f) {
  const uint32_t t = static_cast<uint32_t>((static_cast<uint64_t>(x) * f.m) >> 32);
  return (t + ((x - t) >> f.s1)) >> f.s2;
}

// Divisors of the item index: query tiles per segment, segments, head units
// per kv head, kv heads.
struct ItemDivs {
  FastDiv qt, seg, unit, hkv;
};

// Round k gives the workgroup in slot r item k G + r on even rounds and
// k G + G - 1 - r on odd ones. Items are ordered with the query tile fastest
// and longest first, so a workgroup alternates long and short query tiles;
// items without rows (short last segment) are skipped. Every input is
// uniform (readfirstlane states it for k), so the search runs on the scalar
// unit.
template <int HPW>
__device__ __forceinline__ FusedItem fused_item(int k, int G, int r, int n_items,
                                                const ItemDivs &dv, int N, int L, int Hq,
                                                int Hkv) {
  constexpr int BM = 32 * kWaves / HPW;
  const int grp = Hq / Hkv;
  FusedItem it;
  for (uint32_t kk = __builtin_amdgcn_readfirstlane(k);; ++kk) {
    // Below 2^32: n_items < 2^31 and kk G is at most n_items + 2 G.
    const uint32_t j = kk * static_cast<uint32_t>(G) + static_cast<uint32_t>((kk & 1) ? G - 1 - r : r);
    if (j >= static_cast<uint32_t>(n_items)) {
      it.k = -1;
      it.a = it.e = it.q0 = it.T = it.bq = it.head = it.s = 0;
      return it;
    }
    const uint32_t j1 = fdiv(j, dv.qt);        // (unit, segment) index
    const uint32_t unit = fdiv(j1, dv.seg);     // head unit
    const uint32_t u1 = fdiv(unit, dv.unit);    // b * Hkv + kv head
    const int qt = static_cast<int>(dv.qt.d - 1 - (j - j1 * dv.qt.d));
    const int s = static_cast<int>(j1 - unit * dv.seg.d);
    const int a = s * N;
    const int e = min(a + N, L);
    const int q0 = a + qt * BM;
    if (q0 >= e) continue;
    const uint32_t b = fdiv(u1, dv.hkv);
    const int hk = static_cast<int>(u1 - b * dv.hkv.d);
    const int hu = static_cast<int>(unit - u1 * dv.unit.d);  // head unit within the kv head
    // The fields are uniform by construction; readfirstlane states it, so
    // that they live in scalar registers.
    it.k = __builtin_amdgcn_readfirstlane(static_cast<int>(kk));
    it.a = __builtin_amdgcn_readfirstlane(a);
    it.e = __builtin_amdgcn_readfirstlane(e);
    it.q0 = __builtin_amdgcn_readfirstlane(q0);
    it.T = __builtin_amdgcn_readfirstlane((min(q0 + BM, e) - a + kBN - 1) / kBN);
    it.bq = __builtin_amdgcn_readfirstlane(static_cast<int>(b) * Hq + hk * grp + hu * HPW);
    it.head = __builtin_amdgcn_readfirstlane(static_cast<int>(b) * Hkv + hk);
    it.s = __builtin_amdgcn_readfirstlane(s);
    return it;
  }
}

template <int D, int HPW>
__global__ __launch_bounds__(kThreads, 2) void fused_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ vt, int vt_tiles, const float *__restrict__ beta,
    const uint16_t *__restrict__ z_hl, const uint16_t *__restrict__ mt_pre,
    uint16_t *__restrict__ out, Layout lq, Layout lkv, Layout lo, int Hq, int Hkv, int L, int N,
    int S, ItemDivs dv, int n_items, int G, float eps, float scale_log2) {
  using TL = Tile<D>;
  constexpr int NT = D / 16;          // k-steps over d
  constexpr int ND = D / 32;          // 32-row d tiles of O^T
  constexpr int RW = kWaves / HPW;    // waves (32-row strips) per head
  // Three separate arrays, so that the compiler can tell the ring slots apart
  // when it orders LDS reads after direct loads into another slot.
  __shared__ __attribute__((aligned(16))) uint16_t sB0[TL::BUF];
  __shared__ __attribute__((aligned(16))) uint16_t sB1[TL::BUF];
  __shared__ __attribute__((aligned(16))) uint16_t sB2[TL::BUF];
  const int tid = threadIdx.x;
  // The wave index is uniform across the wave; readfirstlane puts it (and all
  // per-wave bounds derived from it) in scalar registers, so the mask and
  // skip conditions below are real branches rather than per-lane selects.
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int g = lane >> 5, l32 = lane & 31;

  // Slot of this workgroup in the schedule. Workgroups are dealt round-robin
  // to the 8 XCDs; when the grid divides evenly, the slots of one XCD are
  // contiguous, so in every round an XCD works on consecutive items (the
  // query tiles of one head unit and segment, which read the same K / V
  // tiles and share that XCD's L2).
  const int r = (G % kXcds == 0) ? (blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds
                                 : static_cast<int>(blockIdx.x);
  auto item = [&](int kk) __attribute__((always_inline)) {
    return fused_item<HPW>(kk, G, r, n_items, dv, N, L, Hq, Hkv);
  };

  // The workgroup's items form one stream of ring slots. Item i with T key
  // tiles occupies 3 n slots, n = ceil((T + 3) / 3), so that every item starts
  // at ring buffer 0:
  //   slots 0 .. T-1        key tiles (K swizzled, V^T as the scan wrote it)
  //   slots T .. 3n-4       padding (no work; the last tile is loaded again)
  //   slot 3n-3             M^T of the segment (swizzled like K)
  //   slots 3n-2, 3n-1      Q rows of the next item for waves 0..3, 4..7
  //                         (32 rows per wave, swizzled like K)
  // (the first item's Q slots come before its first tile). Every slot also
  // carries a side area of one word per lane of every wave: z before the
  // item's segment as bf16 hi and lo rows (waves 0..6) and beta of its heads
  // (wave 7). Loads run two slots ahead of the work.
  FusedItem cur = item(0);
  if (cur.k < 0) return;

  // Direct loads of one slot: load i of wave w moves units [(8 i + w) 64, +64)
  // of the slot, one 16-byte unit per lane, into consecutive LDS (the hardware
  // writes lane l's unit at the wave's LDS base + 16 l). The 64 units of a
  // load are 512 / D consecutive rows of one 32-row block b_i = (8 i + w) 16 /
  // D of the slot (uniform per wave); the lane's row within the block and its
  // swizzled column are the same for every i (the rows a load covers advance
  // by a multiple of 32, the swizzle period divides 32), so two per-lane
  // values serve all loads. The Q and M^T slots read source row min(row0 +
  // lr, rowmax): rows past the segment end read its last row, whose results
  // are dropped. The key tiles are buffer loads (below): rows past the
  // segment end read as zero, and those keys are masked.
  const int lr = ((w * 64 + lane) / TL::CPR) % 32;
  const int lcol = 8 * ((lane % TL::CPR) ^ ((((w * 64 + lane) / TL::CPR) / TL::RP) % TL::CPR));
  auto blk = [&](int i) __attribute__((always_inline)) { return (8 * i + w) * 16 / D; };
  auto ld = [&](const uint16_t *src, uint16_t *buf, int i) __attribute__((always_inline)) {
    __builtin_amdgcn_global_load_lds(src, IA_LDS(buf + 8 * (8 * i + w) * 64), 16, 0, 0);
  };
  // (The lane values pass through an empty asm statement at each use, so the
  // compiler does not hoist per-lane addresses out of the loops and keep them
  // in registers the MFMA work needs.)
  auto rowsrc = [&](const uint16_t *base, int row0, int rowmax, long long stride)
                    __attribute__((always_inline)) {
    int r = lr, c = lcol;
    __asm__ volatile("" : "+v"(r), "+v"(c));
    return base + min(row0 + r, rowmax) * stride + c;
  };
  auto linsrc = [&](const uint16_t *base) __attribute__((always_inline)) {
    int ln = lane;
    __asm__ volatile("" : "+v"(ln));
    return base + 8 * ln;
  };
  // Key tile t of an item: K rows swizzled, then V^T copied verbatim.
  auto dma_tile = [&](const FusedItem &it, int t, uint16_t *buf) __attribute__((always_inline)) {
    // Buffer loads: the resource of K covers the segment's rows (rows past
    // its end read as zero, and those keys are masked), that of V^T the
    // segment's tiles; the per-lane byte offset is the same for every load
    // of a kind, the rest is a scalar offset.
    auto uniform_ptr = [](const uint16_t *p) __attribute__((always_inline)) {
      const uint64_t a = reinterpret_cast<uint64_t>(p);
      const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
      const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
      return reinterpret_cast<uint16_t *>((static_cast<uint64_t>(hi) << 32) | lo);
    };
    const uint16_t *kseg = k + head_offset(lkv, it.head, Hkv) + it.a * lkv.sr;
    const uint16_t *vseg = vt + (static_cast<size_t>(it.head) * S + it.s) * vt_tiles * (D * 64);
    // (The resource ends with the segment's last row; its rows lie
    // lkv.sr elements apart.)
    const auto krs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(kseg), 0,
        __builtin_amdgcn_readfirstlane(static_cast<int>(((it.e - it.a - 1) * lkv.sr + D) * 2)),
        0x00020000);
    const auto vrs = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(vseg), 0, __builtin_amdgcn_readfirstlane(vt_tiles * D * 64 * 2), 0x00020000);
    int kvo = static_cast<int>((lr * lkv.sr + lcol) * 2), vvo = 16 * lane;
    __asm__ volatile("" : "+v"(kvo), "+v"(vvo));
#pragma unroll
    for (int i = 0; i < TL::IPW; ++i) {
      const int u0 = (8 * i + w) * 64;  // wave-uniform
      // For D >= 64 the first KU / 512 loads of every wave are K; for D = 32
      // the first load is K in waves 0..3 and V^T in waves 4..7.
      const bool is_k = (TL::KU % kThreads == 0) ? (i < TL::KU / kThreads) : (u0 < TL::KU);
      if (is_k)
        buffer_load_lds16(
            krs, buf + 8 * (8 * i + w) * 64, kvo,
            __builtin_amdgcn_readfirstlane(static_cast<int>((t * kBN + 32 * blk(i)) * lkv.sr * 2)));
      else
        buffer_load_lds16(vrs, buf + 8 * (8 * i + w) * 64, vvo,
                          __builtin_amdgcn_readfirstlane((t * D * 64 + 8 * (u0 - TL::KU)) * 2));
    }
  };
  // M^T of an item's segment, swizzled like K, and the side area (one word
  // per lane of every wave) with z before the segment as bf16 hi and lo rows
  // (waves 0..6) and beta of the item's heads (wave 7).
  auto dma_mem = [&](const FusedItem &it, uint16_t *buf) __attribute__((always_inline)) {
    const uint16_t *mt = mt_pre + (static_cast<size_t>(it.head) * S + it.s) * D * D;
#pragma unroll
    for (int i = 0; i < TL::IPW; ++i) ld(rowsrc(mt, 32 * blk(i), D - 1, D), buf, i);  // rows past D (D < 128): unread copies
    // z as hi and lo bf16 rows (2 D bf16 = D words), repeated over waves 0..6.
    const float *zs = reinterpret_cast<const float *>(
        z_hl + (static_cast<size_t>(it.head) * S + it.s) * 2 * D);
    const float *side = (w == kWaves - 1) ? beta + it.bq % Hq + (lane < HPW ? lane : 0)
                                          : zs + (64 * w + lane) % D;
    __builtin_amdgcn_global_load_lds(side, IA_LDS(buf + TL::BUFU * 8 + 128 * w), 4, 0, 0);
  };
  // Q rows of an item for the waves of half `half` (waves 4 half .. 4 half + 3).
  auto dma_q = [&](const FusedItem &it, int half, uint16_t *buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TL::IPW; ++i) {
      const int wv = 4 * half + blk(i);  // the wave that reads this block
      ld(rowsrc(q + head_offset(lq, it.bq + wv / RW, Hq), it.q0 + (wv % RW) * 32, it.e - 1,
                lq.sr),
         buf, i);
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

  // Q^T operand: k-step t covers d in [16t, 16t+16); lane holds d = 16t + 8g + 0..7.
  u32x4 qf[NT];
  f32x16 o[ND];
  float m = -INFINITY;  // running max of this row, log2 domain
  float lsum = 0.f;     // running sum over this lane's key slots

  auto compute = [&](int kv0, const uint16_t *buf, int qw, int qrow, int e)
                     __attribute__((always_inline)) {
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

  // Retrieval from the pre-segment snapshot M^T (this slot), the gate and the
  // store of this wave's 32 rows. Every wave runs it (waves past the segment
  // end included) and issues the same stores: the buffer range ends at the
  // segment end, and the hardware drops stores beyond it.
  auto epilogue = [&](const uint16_t *buf, int qw) __attribute__((always_inline)) {
    const float *side = reinterpret_cast<const float *>(buf + TL::BUFU * 8);
    // sigma(Q) as the B operand, computed in place of Q (the next item's Q
    // slots reload every wave's registers before its first key tile).
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        qf[t][jj] = pack_bf16x2(elu1_clamped(lo_bf16(qf[t][jj])),
                                elu1_clamped(hi_bf16(qf[t][jj])));
    }
    // sigma(q).z on the matrix cores, from the same bf16 sigma(q) as the
    // numerator: row i of the A operand is z's hi part for even i and its lo
    // part for odd i, so registers 0 and 1 of every lane (result rows 4 g and
    // 4 g + 1) hold hi.sigma(q) and lo.sigma(q) of the lane's query.
    const uint16_t *zrow = reinterpret_cast<const uint16_t *>(side) + (l32 & 1) * D + 8 * g;
    f32x16 zacc = f32x16{};
#pragma unroll
    for (int t = 0; t < NT; ++t)
      zacc = mfma32(as_bf16x8(*reinterpret_cast<const u32x4 *>(zrow + 16 * t)), as_bf16x8(qf[t]),
                    zacc);
    const float inv_den = 1.f / (zacc[0] + zacc[1] + eps);
    const float inv_l = 1.f / sum_xor32(lsum);  // both halves' key slots
    const float gam = 1.f / (1.f + __expf(-side[(kWaves - 1) * 64 + w / RW]));
    const float w_mem = gam * inv_den;
    const float w_dot = (1.f - gam) * inv_l;

    // The buffer's base and size are wave-uniform (readfirstlane states it;
    // a buffer resource must be in scalar registers).
    const int nrows = __builtin_amdgcn_readfirstlane(max(0, min(32, cur.e - qw)));
    const size_t obase = head_offset(lo, cur.bq + w / RW, Hq) + qw * lo.sr;
    const uint32_t ob_lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(obase));
    const uint32_t ob_hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(obase >> 32));
    uint16_t *ob = out + ((static_cast<size_t>(ob_hi) << 32) | ob_lo);
    // The resource ends with this wave's last row in the segment (rows lo.sr
    // elements apart); lanes past it address the next row and are dropped.
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(
        ob, 0, nrows > 0 ? static_cast<int>(((nrows - 1) * lo.sr + D) * 2) : 0, 0x00020000);
    const int lane_off = static_cast<int>((l32 < nrows ? l32 : nrows) * lo.sr * 2);
    // One 32-row block of A_mem^T at a time (the fences keep the four
    // accumulation chains from being interleaved, which would hold four
    // accumulators at once). Row 32 dt + l32 of M^T has the swizzle of row
    // l32 (the pattern repeats every 16 rows), so the K operand offsets serve
    // here too. The fragments of block dt + 1 are read as soon as the MFMAs of
    // block dt have been issued, so their latency hides behind the output
    // work of block dt.
    u32x4 ma[NT];
    auto mread = [&](int dt) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        ma[t] = *reinterpret_cast<const u32x4 *>(buf + koff[t] + 32 * dt * D);
    };
    mread(0);
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      __builtin_amdgcn_sched_barrier(0);
      f32x16 am = f32x16{};
#pragma unroll
      for (int t = 0; t < NT; ++t) am = mfma32(as_bf16x8(ma[t]), as_bf16x8(qf[t]), am);
      if (dt + 1 < ND) mread(dt + 1);
      __builtin_amdgcn_sched_barrier(0);
      uint32_t pk[4][2];
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int i0 = 4 * gi + 2 * jj;
          pk[gi][jj] = pack_bf16x2(w_mem * am[i0] + w_dot * o[dt][i0],
                                   w_mem * am[i0 + 1] + w_dot * o[dt][i0 + 1]);
        }
      }
      // Lane group g holds values 8 gi + 4 g + 0..3 of the block; swapping the
      // words of chunks 2p, 2p + 1 with the lane 32 away (upper half of the
      // first operand with the lower half of the second) leaves values
      // 16 p + 8 g + 0..7 in the lane: one 16-byte store per p.
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        uint32_t a[2], b[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const auto r = __builtin_amdgcn_permlane32_swap(pk[2 * p][jj], pk[2 * p + 1][jj], false,
                                                          false);
          a[jj] = r[0];
          b[jj] = r[1];
        }
        __builtin_amdgcn_raw_buffer_store_b128(u32x4{a[0], a[1], b[0], b[1]}, rsrc,
                                               lane_off + (32 * dt + 16 * p + 8 * g) * 2, 0, 0);
      }
    }
  };

  // Q rows of this item for the waves of half `half` (0: waves 0..3, 1:
  // waves 4..7); the online-softmax state starts over with the first half.
  auto take_q = [&](int half, const uint16_t *buf) __attribute__((always_inline)) {
    if (half == 0) {
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) o[dt] = f32x16{};
      m = -INFINITY;
      lsum = 0.f;
    }
    if ((w >> 2) == half) {
      // Row l32 of this wave's 32-row block, swizzled like K row l32. (The
      // block offset passes through an empty asm statement, so that the eight
      // addresses are formed here rather than hoisted and kept.)
      int qo = (w & 3) * 32 * D;
      __asm__ volatile("" : "+v"(qo));
#pragma unroll
      for (int t = 0; t < NT; ++t) qf[t] = *reinterpret_cast<const u32x4 *>(buf + qo + koff[t]);
    }
  };

  // One step: the direct loads of the slot two ahead (EARLY: before the work;
  // LATE: after it), the work on this slot, then this wave's loads of the next
  // slot are awaited and the workgroup meets at the barrier that publishes
  // them. Direct loads complete in issue order, so allowing only this step's
  // own loads (NLD of them) to be outstanding means the next slot has landed.
  //
  // The compiler's wait analysis loses track of which buffer a direct load
  // targets where the paths into a loop head merge, and waits for all of them
  // before the next LDS read; the first step after a loop head therefore
  // issues its loads LATE, so that this wait covers only the next slot, issued
  // a whole step earlier. Elsewhere the steps are straight-line code after a
  // single predecessor and issue EARLY.
  auto step = [&](auto late, auto nld, auto &&load, auto &&work) __attribute__((always_inline)) {
    if (!late.value) load();
    work();
    if (late.value) load();
    wait_vm_lgkm0<decltype(nld)::value>();
    __builtin_amdgcn_s_barrier();
  };
  using LATE = std::true_type;
  using EARLY = std::false_type;
  using NT_ = std::integral_constant<int, TL::IPW>;      // key tile or Q slot
  using NM_ = std::integral_constant<int, TL::IPW + 1>;  // M^T slot with its side area
#define IA_DO(...) [&]() __attribute__((always_inline)) { __VA_ARGS__; }

  // The first item's Q slots (as if a previous item had ended).
  dma_q(cur, 0, sB1);
  dma_q(cur, 1, sB2);
  wait_vm_lgkm0<TL::IPW>();
  __builtin_amdgcn_s_barrier();
  step(EARLY{}, NT_{}, IA_DO(dma_tile(cur, 0, sB0)), IA_DO(take_q(0, sB1)));
  step(EARLY{}, NT_{}, IA_DO(dma_tile(cur, min(1, cur.T - 1), sB1)), IA_DO(take_q(1, sB2)));
  for (;;) {
    const FusedItem nxt = item(cur.k + 1);
    const int n3 = (cur.T + 5) / 3 * 3;  // slots of this item
    const int qw = cur.q0 + (w % RW) * 32;  // first query row of this wave
    const bool live = qw < cur.e;
    const int tlast = cur.T - 1;
    auto tile = [&](int pos, const uint16_t *buf) __attribute__((always_inline)) {
      const int kv0 = cur.a + pos * kBN;
      if (pos < cur.T && live && kv0 <= qw + 31) compute(kv0, buf, qw, qw + l32, cur.e);
    };
    // Slots 0 .. n3 - 7, three per iteration; every slot loaded from here on
    // is a key tile (padding: the last tile again).
    int pos = 0;
    while (pos < n3 - 6) {
      step(LATE{}, NT_{}, IA_DO(dma_tile(cur, min(pos + 2, tlast), sB2)), IA_DO(tile(pos, sB0)));
      step(EARLY{}, NT_{}, IA_DO(dma_tile(cur, min(pos + 3, tlast), sB0)),
           IA_DO(tile(pos + 1, sB1)));
      step(EARLY{}, NT_{}, IA_DO(dma_tile(cur, min(pos + 4, tlast), sB1)),
           IA_DO(tile(pos + 2, sB2)));
      pos += 3;
    }
    // The last three tile slots load M^T and the next item's Q; then the
    // retrieval and output of this item, and the next item's Q. Past the last
    // item, the Q slots load M^T again (any valid source; nobody reads it).
    step(LATE{}, NT_{}, IA_DO(dma_tile(cur, min(n3 - 4, tlast), sB2)), IA_DO(tile(n3 - 6, sB0)));
    step(EARLY{}, NM_{}, IA_DO(dma_mem(cur, sB0)), IA_DO(tile(n3 - 5, sB1)));
    if (nxt.k >= 0) {
      step(EARLY{}, NT_{}, IA_DO(dma_q(nxt, 0, sB1)), IA_DO(tile(n3 - 4, sB2)));
      step(EARLY{}, NT_{}, IA_DO(dma_q(nxt, 1, sB2)), IA_DO(epilogue(sB0, qw)));
    } else {
      step(EARLY{}, NT_{}, IA_DO(dma_tile(cur, tlast, sB1)), IA_DO(tile(n3 - 4, sB2)));
      step(EARLY{}, NT_{}, IA_DO(dma_tile(cur, tlast, sB2)), IA_DO(epilogue(sB0, qw)));
      break;
    }
    cur = nxt;
    step(EARLY{}, NT_{}, IA_DO(dma_tile(cur, 0, sB0)), IA_DO(take_q(0, sB1)));
    step(EARLY{}, NT_{}, IA_DO(dma_tile(cur, min(1, cur.T - 1), sB1)), IA_DO(take_q(1, sB2)));
  }
#undef IA_DO
  // Loads of slots past the end are still in flight; they must land before
  // the workgroup's LDS is handed to another workgroup.
  wait_vm_lgkm0<0>();
}

// Compute units of a device and resident workgroups per compute unit of a
// kernel, cached per device (the values do not change for a process).
int device_cus(int dev) {
  static int cached[64] = {};
  if (dev >= 0 && dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    n = 1;
  if (dev >= 0 && dev < 64) cached[dev] = n;
  return n;
}

template <int D, int HPW>
int fused_per_cu(int dev) {
  static int cached[64] = {};  // per template instance
  if (dev >= 0 && dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, reinterpret_cast<const void *>(&fused_bf16_kernel<D, HPW>), kThreads, 0) !=
          hipSuccess ||
      n < 1)
    n = 1;
  if (dev >= 0 && dev < 64) cached[dev] = n;
  return n;
}

template <int D, int HPW>
hipError_t launch_t(const Geometry &g, const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    const float *beta, const Workspace &ws, uint16_t *out, hipStream_t stream) {
  constexpr int BM = 32 * kWaves / HPW;
  const int rows = g.N < g.L ? g.N : g.L;
  const int n_qt = (rows + BM - 1) / BM;
  const long long units = static_cast<long long>(g.B) * g.Hkv * (g.Hq / g.Hkv / HPW);
  const long long n_items = static_cast<long long>(n_qt) * g.S * units;
  if (n_items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (n_items == 0) return hipSuccess;
  // Persistent workgroups: as many as can be resident at once (one per
  // compute unit at d = 128, where the ring fills most of a CU's LDS), each
  // working through its items in one stream of ring slots.
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const long long slots = static_cast<long long>(fused_per_cu<D, HPW>(dev)) * device_cus(dev);
  const long long grid = n_items < slots ? n_items : slots;
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  const ItemDivs dv{make_fastdiv(static_cast<uint32_t>(n_qt)),
                    make_fastdiv(static_cast<uint32_t>(g.S)),
                    make_fastdiv(static_cast<uint32_t>(g.Hq / g.Hkv / HPW)),
                    make_fastdiv(static_cast<uint32_t>(g.Hkv))};
  fused_bf16_kernel<D, HPW><<<dim3(static_cast<unsigned>(grid)), kThreads, 0, stream>>>(
      q, k, ws.vt, ws.vt_tiles, beta, ws.z_hl, ws.mt_pre_bf16, out, g.lq, g.lkv, g.lo, g.Hq,
      g.Hkv, g.L, g.N, g.S, dv, static_cast<int>(n_items), static_cast<int>(grid), g.eps,
      scale_log2);
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
