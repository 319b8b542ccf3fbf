// Internal launch interface between the host library and the gfx950 kernels.
// Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "infini_attn.h"

namespace ia {

// Where row i of head h of batch b of a q / k / v / out tensor starts, in
// elements: b * sb + h * sh + i * sr (its d elements are contiguous). The C
// ABI's tensors are head-major [B, H, L, d] (sb = H L d, sh = L d, sr = d);
// the block hands the kernels its row-major projections [B, L, ..., H, d]
// (sb = L W, sh = d, sr = W for rows of W elements) without regrouping them.
struct Layout {
  long long sb, sh, sr;
};

__host__ __device__ inline Layout head_major(int H, int L, int D) {
  return Layout{static_cast<long long>(H) * L * D, static_cast<long long>(L) * D, D};
}

// Offset of row 0 of flattened head bh = b * H + h.
__host__ __device__ inline long long head_offset(const Layout &l, int bh, int H) {
  return (bh / H) * l.sb + (bh % H) * l.sh;
}

// Problem geometry of one forward call, already validated on the host.
struct Geometry {
  int B, Hq, Hkv, L, D;  // D = d_k = d_v
  int N;                 // segment length
  int S;                 // number of segments, ceil(L / N)
  float eps;
  Layout lq, lkv, lo;    // of q, of k and v, of out
};

// Per-segment state snapshots written by the scan and read by the fused
// kernel. Index (b * Hkv + j) * S + s holds the state *before* segment s.
struct Workspace {
  float *z_pre;           // [B*Hkv][S+1][D] fp32; slot S receives the final z
  uint16_t *z_hl;         // [B*Hkv][S][2][D] bf16 (bf16 path): z before segment s as its
                          // bf16 rounding (row 0) and the bf16 rounding of the rest (row 1)
  float *mt_pre_f32;      // [B*Hkv][S][D(v)][D(k)] fp32, M^T (fp32 storage path)
  uint16_t *mt_pre_bf16;  // [B*Hkv][S][D(v)][D(k)] bf16 bits, M^T (bf16 storage path)
  float *dz;              // [B*Hkv][S][z_parts][D] partial sums of sigma(k) (bf16 path)
  int z_parts;            // row ranges per segment in dz
  float *gh;              // [B*Hkv][S][2][D*D] G_s, H_s in MFMA fragment order (bf16 path)
  uint16_t *vt;           // [B*Hkv][S][vt_tiles][D*64] V^T per 64-key tile (bf16 path)
  int vt_tiles;           // 64-key tiles per segment, ceil(N / 64)
  // Chunked scan of the delta rule's chain (bf16 path, long chains only):
  // chunk_len segments per chunk (0: one sequential chain), and per chunk
  // [P | h] (D x 2D fp32), its packed affine step (G', H' fragments) and the
  // fp32 state before it.
  int chunk_len;
  float *chain_x;       // [B*Hkv][chunks][D][2D]
  float *chain_gh;      // [B*Hkv][chunks][2][D*D]
  float *chain_states;  // [B*Hkv][chunks][D][D]
};

// Segments per chunk of the chunked chain scan for S segments of B * Hkv
// heads, or 0 when one sequential chain is used: chains of at least 64
// segments are split into about sqrt(S / 2) segments a chunk, which balances
// the two chunk-parallel passes against the sequential pass over the chunks.
int chain_chunk_len(int S, int heads);

// Layout of one 64-key V^T tile (bf16 path), written by the scan and copied
// verbatim into LDS by the fused kernel. Row d (one per value column) holds
// the tile's 64 keys as 8 units of 16 bytes. Unit q of the row holds the
// keys of 16-key step q / 2 that lane group q % 2 of a 32x32x16 MFMA operand
// contributes: keys 16 (q/2) + 4 (q%2) + {0..3} and 16 (q/2) + 8 + 4 (q%2) +
// {0..3}. Unit q is stored at position q ^ ((d / 2) % 8) of the row, so that
// 16 consecutive rows read at one unit index hit distinct LDS banks.
__host__ __device__ inline int vt_unit_pos(int d, int q) { return q ^ ((d >> 1) & 7); }

// Segment scan, fp32 storage: carries fp32 (M, z) across segments for every
// (b, kv head) on VALU, writing the pre-segment snapshots (z_pre, mt_pre_f32)
// and the final M in place; the final z lands in z_pre slot S.
hipError_t launch_segment_scan_f32(const Geometry &g, const float *k, const float *v, float *M,
                                   const float *z, int delta, const Workspace &ws,
                                   hipStream_t stream);

// Segment scan, bf16 storage: per-segment statistics on MFMA in parallel, then
// the fp32 recurrence; writes z_pre (slot S = final z), mt_pre_bf16, and the
// final M and z in place (z is read as z_0 first).
hipError_t launch_segment_scan_bf16(const Geometry &g, const uint16_t *k, const uint16_t *v,
                                    float *M, float *z, int delta, const Workspace &ws,
                                    hipStream_t stream);

// Fused per-segment kernel: local causal attention, retrieval from the
// snapshot, gate, store. bf16 storage path (MFMA).
hipError_t launch_fused_bf16(const Geometry &g, const uint16_t *q, const uint16_t *k,
                             const uint16_t *v, const float *beta, const Workspace &ws,
                             uint16_t *out, hipStream_t stream);

// Same operation for the fp32 storage path (fp32 arithmetic throughout).
hipError_t launch_fused_f32(const Geometry &g, const float *q, const float *k, const float *v,
                            const float *beta, const Workspace &ws, float *out,
                            hipStream_t stream);

// Scratch of the backward pass (fp32 throughout). Units are (b, kv head,
// segment) in that order; rows are [B][Hq][L] for the per-query-row arrays.
struct BwdWorkspace {
  float *z_pre;  // [B*Hkv][S+1][D] z before every segment (scan output)
  float *mt;     // [B*Hkv][S][D(v)][D(k)] M^T before every segment (scan output)
  float *lse;    // [B*Hq*L] log-sum-exp of each query row's causal softmax
  float *erow;   // [B*Hq*L] dO_i . A_dot_i
  float *gd;     // [B*Hq*L] gamma / den of each query row: the retrieval numerator's
                 // gradient is gd dO_i, formed again where it is needed
  float *dden;   // [B*Hq*L] gradient of the retrieval denominator
  float *R;      // [units][D][D] sum of sigma(q)^T (gd dO) over the group (zeroed)
  float *r;      // [units][D] sum of sigma(q)^T dden over the group (zeroed)
  float *G;      // [units][D][D] delta rule's sigma(k)^T diag(1/denk) sigma(k) (zeroed)
  float *qz;     // [units][D] delta rule's sigma(k)^T ddenk (zeroed)
  float *gma;    // [units][D][D] gradient of M after each segment
  float *gza;    // [units][D] gradient of z after each segment
  float *H;      // [units][D][D] sigma(k)^T v of each segment (zeroed)
  float *dzs;    // [units][D] column sums of sigma(k) over each segment
  // Per-block partial sums, added in a fixed order so that every gradient is
  // the same from run to run:
  float *part;        // [units][blocks][D*D (+ D)] of the G, H and R, r products
  float *qz_part;     // [units][chunks][D] of qz (delta rule)
  float *dbeta_part;  // [Hq][B][S][qblocks] of dbeta
};

// Blocks per unit of the backward's kernels (see backward.hip), which size the
// partial-sum scratch: rows_per rows per block of the G and H products (rows
// of them), of the R product (group_rows of them, over every query head of the
// group), 128-row query blocks, and 32-row chunks of the update's gradient.
struct BwdBlocks {
  int rows_per, rows, group_rows, qblocks, chunks;
};
BwdBlocks backward_blocks(const Geometry &g);

// Backward pass: dq, dk, dv (fp32, the shapes of q, k, v), dbeta (zeroed by
// the caller), dM0, dz0, for the forward that starts from (M0, z0), whose
// per-segment states it recomputes into z_pre and mt; dM, dz may be null
// (zero). R, r, G, qz and H must be zeroed.
template <typename T>
hipError_t launch_backward(const Geometry &g, const T *q, const T *k, const T *v, const T *dout,
                           const float *beta, const float *M0, const float *z0, const float *dM,
                           const float *dz, int delta, const BwdWorkspace &w, float *dq, float *dk,
                           float *dv, float *dbeta, float *dM0, float *dz0, hipStream_t stream);

// Geometry of one streaming-decode call: C new query rows per (batch, query
// head) against rows [0, n_past + C) of a K/V cache of cap rows per kv head.
struct DecodeGeometry {
  int B, Hq, Hkv, D;
  int C;       // new query rows per head
  int cap;     // cache rows per (batch, kv head): the row stride of the cache
  int n_past;  // cache rows before the new ones
  float eps;
};

// Key splits (workgroups along the keys) for n_keys visible keys, and the
// fp32 scratch the split partials and the retrieval slot need.
int decode_splits(int n_keys);
size_t decode_partial_floats(const DecodeGeometry &g);

// The allocation-free decode keeps its split partials in a fixed device array
// of this many bytes (one per device, held until the process ends).
constexpr size_t kDecodeScratchBytes = INFINI_ATTN_DECODE_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// Device address of the fixed decode scratch on device `dev`, which must be
// the current device; looked up once per device and cached.
hipError_t decode_scratch(int dev, float **ptr);

// Streaming decode: split partials of the local attention into `part`, then
// merge, retrieval from (M, z), gate and store into out [B][Hq][C][D].
hipError_t launch_decode_bf16(const DecodeGeometry &g, const uint16_t *q, const uint16_t *kc,
                              const uint16_t *vc, const float *beta, const float *M,
                              const float *z, float *part, uint16_t *out, hipStream_t stream);
hipError_t launch_decode_f32(const DecodeGeometry &g, const float *q, const float *kc,
                             const float *vc, const float *beta, const float *M, const float *z,
                             float *part, float *out, hipStream_t stream);

// Infini-attention block: the dense projections through rocBLAS (statuses
// are INFINI_ATTN_* codes). Row-major C (rows x n, leading dimension ldc) =
// X (rows x k, ldx) W^T, W row-major n x k (ldw).
int blas_create(void **blas, hipStream_t stream);
void blas_destroy(void *blas);
int blas_gemm_xwt(void *blas, int dtype, int rows, int n, int k, const void *x, int ldx,
                  const void *w, int ldw, void *c, int ldc);

}  // namespace ia
