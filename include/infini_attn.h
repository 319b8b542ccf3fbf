/*
 * infini_attn.h — C ABI of the gfx950 Infini-attention forward library.
 *
 * The operation (per batch element b and query head h, reading kv head
 * j = h / (Hq / Hkv)):
 *   the sequence of L rows is cut into segments of seg_len rows, the last one
 *   possibly shorter ([HF-repro] "Infini-Attention メカニズム", step
 *   Segmentation). For every segment s, in order:
 *     A_dot = softmax(mask(Q_s K_s^T / sqrt(d_k))) V_s, causal inside the
 *             segment only (step Local Attention; [LNCB-review] "基本アイデア");
 *     A_mem = sigma(Q_s) M_{s-1} / (sigma(Q_s) z_{s-1} + eps), row by row, with
 *             sigma = ELU + 1 (step Memory Retrieval; [LNCB-review]
 *             "メモリの読み出し");
 *     out_s = g_h A_mem + (1 - g_h) A_dot, g_h = 1 / (1 + exp(-beta_h)) (step
 *             Integration; [LNCB-review] "長期情報と短期情報の統合");
 *   then, per kv head, the segment is written into the memory (step Memory
 *   Update; [LNCB-review] "メモリの更新"):
 *     LINEAR: M_s = M_{s-1} + sigma(K_s)^T V_s
 *     DELTA:  M_s = M_{s-1} + sigma(K_s)^T (V_s - sigma(K_s) M_{s-1} /
 *                                              (sigma(K_s) z_{s-1} + eps))
 *     both:   z_s = z_{s-1} + sum over the segment's rows of sigma(k)
 *   and only (M, z) passes to the next segment (step State Transfer).
 *
 * Pages cited: [HF-repro] "Hugging Face Infini-Attention 再現分析";
 * [LNCB-review] the abeam-guide review of "Leave No Context Behind: Efficient
 * Infinite Context Transformers with Infini-attention".
 *
 * Conventions shared by every entry point:
 *   - Every function returns an int status: INFINI_ATTN_OK (0) or a negative
 *     INFINI_ATTN_ERR_* code. No C++ exception crosses this boundary.
 *   - Device pointers point to device memory of the handle's device. The caller
 *     owns every tensor; the library owns only its handle and the workspace
 *     inside it.
 *   - Work is enqueued on the handle's stream and the call returns without
 *     waiting for it. Errors raised by the kernels themselves surface at the
 *     caller's next synchronisation. A handle must not be used by two host
 *     threads or two streams at once.
 */
#ifndef INFINI_ATTN_H
#define INFINI_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define INFINI_ATTN_OK 0
#define INFINI_ATTN_ERR_INVALID (-1)     /* null/misaligned pointer, bad size, mode or dtype */
#define INFINI_ATTN_ERR_UNSUPPORTED (-2) /* valid request this build has no kernel for */
#define INFINI_ATTN_ERR_HIP (-3)         /* HIP runtime or launch failure, no device */
#define INFINI_ATTN_ERR_OOM (-4)         /* workspace allocation failed */
#define INFINI_ATTN_ERR_SCRATCH (-5)     /* request larger than a fixed scratch array */

/* Bytes of the fixed per-device scratch array of infini_attn_decode_noalloc. */
#define INFINI_ATTN_DECODE_SCRATCH_BYTES (16u << 20)

/* Storage type of q, k, v and out. beta, M and z are always fp32. */
#define INFINI_ATTN_F32 0
#define INFINI_ATTN_BF16 1

/* Memory update rule ([LNCB-review] "メモリの更新"). */
#define INFINI_ATTN_LINEAR 0
#define INFINI_ATTN_DELTA 1

typedef struct infini_attn_desc {
  int32_t batch;      /* B >= 1 */
  int32_t n_q_heads;  /* Hq >= 1, a multiple of n_kv_heads */
  int32_t n_kv_heads; /* Hkv >= 1; query head h reads kv head h / (Hq / Hkv) */
  int32_t seq_len;    /* L rows per call, 0 .. 2^30 (larger: ERR_UNSUPPORTED) */
  int32_t d_k;        /* key / query width; supported: 32, 64, 128 */
  int32_t d_v;        /* value width; this build requires d_v == d_k */
  int32_t dtype;      /* INFINI_ATTN_F32 or INFINI_ATTN_BF16 */
  float eps;          /* retrieval denominator offset, > 0 and finite (1e-6 typical) */
  void *stream;       /* hipStream_t to enqueue on; NULL = the null stream */
  int32_t device;     /* HIP device ordinal of every pointer passed to forward */
} infini_attn_desc;

typedef struct infini_attn_handle infini_attn_t;

/*
 * Validate a descriptor and the per-call arguments of infini_attn_forward
 * without touching any device. Returns OK, ERR_INVALID or ERR_UNSUPPORTED.
 * Pure host code: safe to call on a machine with no GPU.
 */
int infini_attn_check(const infini_attn_desc *desc, int32_t seg_len, int32_t update_mode);

/*
 * Bytes of device workspace a handle with this descriptor allocates for a
 * forward call with this segment length: the per-segment state snapshots
 * (M_{s-1}, z_{s-1}) that the segment-scan kernel writes and the fused
 * attention kernel reads, and for bf16 storage the scan's per-segment
 * statistics and a transposed copy of V in 64-key tiles. Writes the size to
 * *bytes. Host only.
 */
int infini_attn_workspace_size(const infini_attn_desc *desc, int32_t seg_len, size_t *bytes);

/*
 * Create a handle for one problem shape. Validates *desc, makes desc->device
 * current, and records the stream. *h receives the handle, or NULL on error.
 * The workspace is allocated by the first forward call that needs it and
 * grown (never shrunk) by later calls with more segments.
 * Errors: ERR_INVALID (null h/desc or bad field), ERR_UNSUPPORTED, ERR_HIP
 * (no device, or the device cannot be selected).
 */
int infini_attn_create(infini_attn_t **h, const infini_attn_desc *desc);

/*
 * One forward pass over seq_len rows.
 *   q    [B, Hq,  L, d_k]  dtype, contiguous, 16-byte aligned (device)
 *   k    [B, Hkv, L, d_k]  dtype, contiguous, 16-byte aligned (device)
 *   v    [B, Hkv, L, d_v]  dtype, contiguous, 16-byte aligned (device)
 *   beta [Hq]              fp32, one gate parameter per query head (device)
 *   M    [B, Hkv, d_k, d_v] fp32 in/out (device): M_0 on entry, M_S on exit
 *   z    [B, Hkv, d_k]      fp32 in/out (device): z_0 on entry, z_S on exit
 *   seg_len     >= 1 rows per segment; S = ceil(L / seg_len) segments (any
 *               seg_len >= L is one segment of L rows; workspace and launches
 *               are sized by min(seg_len, L))
 *   update_mode INFINI_ATTN_LINEAR or INFINI_ATTN_DELTA
 *   out  [B, Hq, L, d_v]   dtype (device), written; must not overlap any input
 * Passing (M_S, z_S) back with the next L rows continues the same stream of
 * segments when the previous L was a multiple of seg_len.
 * Errors: ERR_INVALID (null or misaligned pointer, seg_len < 1, bad mode),
 * ERR_OOM (workspace), ERR_HIP (launch failure). After an error M and z are
 * unspecified.
 */
int infini_attn_forward(infini_attn_t *h, const void *q, const void *k, const void *v,
                        const float *beta, float *M, float *z, int32_t seg_len,
                        int32_t update_mode, void *out);

/*
 * Streaming decode: n_new new query rows per (batch, query head), at positions
 * n_past .. n_past + n_new - 1 of the current segment, against the segment's
 * rows held in a K/V cache. Per new row (position p): causal attention over
 * cache rows 0 .. p, retrieval from the state before the segment, gate mix —
 * the same rows infini_attn_forward produces for these positions
 * ([HF-repro] "Infini-Attention メカニズム", steps Local Attention, Memory
 * Retrieval, Integration and State Transfer: only (M, z) and the current
 * segment's K/V are kept; [LNCB-review] "実装上の流れ").
 * The handle's desc.seq_len is the cache capacity (rows per kv head).
 *   q       [B, Hq,  n_new, d_k] dtype, contiguous, 16-byte aligned (device)
 *   k_cache [B, Hkv, seq_len, d_k] dtype, 16-byte aligned (device); rows
 *           0 .. n_past + n_new - 1 hold the segment's keys, the new rows'
 *           own keys included (the caller appends them first)
 *   v_cache [B, Hkv, seq_len, d_v] dtype, same rows as k_cache
 *   n_past  >= 0 cached rows before the new ones; n_past + n_new <= seq_len
 *   beta    [Hq] fp32 (device)
 *   M, z    [B, Hkv, d_k, d_v], [B, Hkv, d_k] fp32 (device), the state before
 *           the current segment; read only
 *   out     [B, Hq, n_new, d_v] dtype (device), written
 * The library keeps a scratch buffer for the key-split partials and the
 * retrieval in the handle, grown on demand:
 * 4 (d_v + 2) B Hq n_new (ceil((n_past + n_new) / 64) + 1) bytes, small for a
 * few new rows; a long chunk is better served by
 * infini_attn_forward. The chunk must not cross a segment boundary: at
 * the boundary, fold the finished segment into (M, z) with
 * infini_attn_update and start the cache again at row 0.
 * Errors: ERR_INVALID (null or misaligned pointer, n_new < 1, n_past < 0,
 * n_past + n_new > seq_len), ERR_UNSUPPORTED (more than 1048560 query rows
 * per kv head), ERR_OOM (scratch), ERR_HIP (launch failure).
 */
int infini_attn_decode(infini_attn_t *h, const void *q, int32_t n_new, const void *k_cache,
                       const void *v_cache, int32_t n_past, const float *beta, const float *M,
                       const float *z, void *out);

/*
 * Allocation-free variant of infini_attn_decode, for callers that cannot
 * allocate device memory during the call: code under HIP graph capture, tight
 * serving loops, and harnesses that forbid hipMalloc. Same arguments, same
 * kernels and the same result as infini_attn_decode, but the key-split
 * partials go to a fixed array of INFINI_ATTN_DECODE_SCRATCH_BYTES that the
 * library's code object holds on every device it runs on (until the process
 * ends), instead of a buffer the handle grows: the call allocates nothing and
 * calls no allocating library routine. Its address on a device is looked up
 * by infini_attn_create, with that device current.
 * The partials (one slot per 64-key split and one for the retrieval) need
 * 4 (d_v + 2) B Hq n_new (ceil((n_past + n_new) / 64) + 1) bytes; a larger
 * request returns ERR_SCRATCH before anything is enqueued (one new row against
 * a full 2048-row segment of the Llama-3-8B attention shape takes 549 KB). Every call on one device shares that device's array and overwrites
 * what the previous call left there (nothing in it needs to start at zero):
 * calls that may overlap on one device, from any handle or stream, race and
 * must be serialised by the caller.
 * Errors: as infini_attn_decode, with ERR_SCRATCH in place of ERR_OOM.
 */
int infini_attn_decode_noalloc(infini_attn_t *h, const void *q, int32_t n_new,
                               const void *k_cache, const void *v_cache, int32_t n_past,
                               const float *beta, const float *M, const float *z, void *out);

/*
 * Memory update of one finished segment: the desc.seq_len rows of k, v are
 * written into (M, z) in place by the rule update_mode (step Memory Update;
 * [LNCB-review] "メモリの更新"), exactly as infini_attn_forward writes a
 * segment. Used with infini_attn_decode at segment boundaries; for a shorter
 * last segment, use a handle whose seq_len is that segment's length.
 *   k  [B, Hkv, seq_len, d_k] dtype, contiguous, 16-byte aligned (device)
 *   v  [B, Hkv, seq_len, d_v] dtype, contiguous, 16-byte aligned (device)
 *   M, z  fp32 in/out (device): the state before the segment on entry, after
 *         it on exit
 * seq_len = 0 or batch = 0 leaves (M, z) unchanged.
 * Errors: ERR_INVALID (null or misaligned pointer, bad mode), ERR_OOM
 * (workspace), ERR_HIP (launch failure).
 */
int infini_attn_update(infini_attn_t *h, const void *k, const void *v, float *M, float *z,
                       int32_t update_mode);

/*
 * The Infini-attention block: projections of the layer input, the forward
 * pass above, and the output projection ([HF-repro] "Infini-Attention
 * メカニズム": the mechanism takes the layer's own query, key and value
 * states; [LNCB-review] "基本アイデア": it stands in for the attention of each
 * layer's block):
 *   Q = x Wq^T, K = x Wk^T, V = x Wv^T (head h takes columns h d .. h d + d - 1
 *   of the product), O = infini_attn_forward(Q, K, V, beta, M, z, seg_len,
 *   update_mode), y = O' Wo^T, with O' the heads of each row side by side
 *   [B, L, Hq d]. Weights are [out, in] row-major, the layout a linear layer
 *   usually keeps (and the one the library GEMM runs fastest on):
 *   d_model  >= 1 width of the layer input and output
 *   x   [B, L, d_model]        dtype, contiguous (device)
 *   wq  [Hq * d_k, d_model]    dtype, row-major (device)
 *   wk  [Hkv * d_k, d_model]   dtype, row-major (device)
 *   wv  [Hkv * d_v, d_model]   dtype, row-major (device)
 *   wo  [d_model, Hq * d_v]    dtype, row-major (device)
 *   beta, M, z, seg_len, update_mode as for infini_attn_forward (M, z in/out)
 *   y   [B, L, d_model]        dtype (device), written
 * The projections run on rocBLAS with fp32 accumulation, and Q, K, V, O are
 * rounded to dtype. Q, K and V land side by side in one row-major buffer
 * [B, L, (Hq + 2 Hkv) d] that the attention kernels read in place, and O is
 * written row-major [B, L, Hq d] for the output projection; nothing is
 * regrouped. The handle keeps these two buffers in its own scratch, grown on
 * demand, and a rocBLAS handle on its stream.
 * Errors: as infini_attn_forward; ERR_INVALID also for d_model < 1;
 * ERR_UNSUPPORTED for B * L > 2^31 - 1.
 */
int infini_attn_block_forward(infini_attn_t *h, int32_t d_model, const void *x, const void *wq,
                              const void *wk, const void *wv, const void *wo, const float *beta,
                              float *M, float *z, int32_t seg_len, int32_t update_mode, void *y);

/*
 * The same block with the three projection weights fused into one matrix, as
 * models that store a single query-key-value projection keep them:
 *   wqkv [(Hq + 2 Hkv) d_k, d_model] dtype, row-major (device): rows
 *        0 .. Hq d - 1 are Wq, then Hkv d rows of Wk, then Hkv d of Wv
 * so that Q, K and V come from one GEMM. Every other argument, the result and
 * the errors are those of infini_attn_block_forward.
 */
int infini_attn_block_forward_qkv(infini_attn_t *h, int32_t d_model, const void *x,
                                  const void *wqkv, const void *wo, const float *beta, float *M,
                                  float *z, int32_t seg_len, int32_t update_mode, void *y);

/*
 * Backward pass of infini_attn_forward: the gradients of
 *   loss = <d_out, out> + <d_M, M_S> + <d_z, z_S>
 * with respect to q, k, v, beta and the initial state (M_0, z_0), taken by
 * backpropagation through time over the segments, the way the memory is
 * trained end to end ([LNCB-review] "実装上の流れ": the segments are processed
 * in order with the memory carried between them; [HF-repro] "Infini-Attention
 * メカニズム", step State Transfer: the state is the only link between
 * segments, so it is the only path by which later segments' gradients reach
 * earlier ones). The forward quantities (softmax statistics, the state
 * before each segment) are recomputed in fp32; nothing from a forward call
 * is needed.
 *   q, k, v, beta, seg_len, update_mode  as for infini_attn_forward (device)
 *   M0  [B, Hkv, d_k, d_v] fp32, z0 [B, Hkv, d_k] fp32: the state the forward
 *       started from (read only)
 *   d_out [B, Hq, L, d_v] dtype (device): gradient of the loss w.r.t. out
 *   d_M [B, Hkv, d_k, d_v], d_z [B, Hkv, d_k] fp32 (device), or NULL for zero:
 *       gradient w.r.t. the final state
 *   dq [B, Hq, L, d_k], dk [B, Hkv, L, d_k], dv [B, Hkv, L, d_v] fp32, 16-byte
 *       aligned (device), written; dk and dv sum over the query heads of each
 *       kv group
 *   dbeta [Hq] fp32 (device), written
 *   dM0 [B, Hkv, d_k, d_v], dz0 [B, Hkv, d_k] fp32 (device), written
 * Every arithmetic step is fp32: for bf16 storage, products of two stored
 * tensors run on the bf16 matrix cores, exact in fp32 with fp32 accumulation;
 * the other products run on the fp32 matrix cores. Output buffers must not
 * alias inputs. The
 * handle keeps fp32 scratch of about (B Hq L (d + 3) + 5 B Hkv S d^2 +
 * B Hkv S (d^2 + d) ceil(max(seg_len, (Hq / Hkv) seg_len) / 1024)) floats,
 * grown on demand. Every sum over blocks of rows is taken in a fixed order
 * (per-block partials, then an ordered sum; no floating-point atomics), so
 * repeated calls on the same inputs and device return bitwise identical
 * gradients. B = 0 writes dbeta = 0; L = 0 also passes (d_M, d_z) through to
 * (dM0, dz0).
 * Errors: as infini_attn_forward; ERR_INVALID also for a null d_out, dq, dk,
 * dv, dbeta, M0, z0, dM0 or dz0 where the shapes are non-empty.
 */
int infini_attn_backward(infini_attn_t *h, const void *q, const void *k, const void *v,
                         const float *beta, const float *M0, const float *z0, int32_t seg_len,
                         int32_t update_mode, const void *d_out, const float *d_M,
                         const float *d_z, float *dq, float *dk, float *dv, float *dbeta,
                         float *dM0, float *dz0);

/*
 * Per-kernel timing for profiling. With timing enabled, every forward call
 * records HIP events on the handle's stream around its segment-scan kernel
 * and its fused attention kernel. infini_attn_get_timing waits for the
 * recorded events, returns the number of timed calls since the previous get
 * and the summed durations (milliseconds) of the two kernels over those
 * calls, and clears the record. Any output pointer may be NULL.
 * Errors: ERR_INVALID (null handle), ERR_HIP (event failure).
 */
int infini_attn_set_timing(infini_attn_t *h, int32_t enable);
int infini_attn_get_timing(infini_attn_t *h, int32_t *calls, float *scan_ms, float *fused_ms);

/* Free the workspace and the handle. destroy(NULL) returns OK. */
int infini_attn_destroy(infini_attn_t *h);

/* Static, human-readable text for a status code. */
const char *infini_attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* INFINI_ATTN_H */
