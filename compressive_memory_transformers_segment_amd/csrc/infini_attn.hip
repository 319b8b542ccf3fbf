// Host side of the C ABI declared in include/infini_attn.h: argument
// validation, the handle and its workspace, and the launch sequences
//   forward:  segment scan  ->  fused per-segment attention  ->  copy of the final z
//   update:   segment scan over one segment  ->  copy of the final z
//   decode:   split partials of the local attention  ->  merge, retrieval, gate
//   block:    Q/K/V projections (rocBLAS) and regrouping  ->  forward  ->  regroup
//             ->  output projection
//   backward: the forward's per-segment states (parallel sums, a d x d chain)
//             ->  per-segment gradient kernels, the reverse state chains and
//             the memory write's gradient
// enqueued on the handle's stream with no host synchronisation.

#include "infini_attn.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <new>
#include <vector>

#include "launch.h"

struct TimedCall {
  hipEvent_t ev[3];  // before scan, after scan, after fused kernel
};

struct infini_attn_handle {
  infini_attn_desc desc;
  hipStream_t stream;
  void *ws;
  size_t ws_bytes;
  void *dec_ws;  // split partials of the streaming decode
  size_t dec_ws_bytes;
  void *blk_ws;  // the block's projections and regrouped attention output
  size_t blk_ws_bytes;
  void *blas;    // rocBLAS handle of the block's projections (created on first use)
  void *bwd_ws;  // the backward pass's snapshots and per-segment gradients
  size_t bwd_ws_bytes;
  bool timing;
  std::vector<TimedCall> recorded;  // calls timed since the last get
  std::vector<TimedCall> spare;     // event triples ready for reuse
};

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_desc(const infini_attn_desc *d) {
  if (!d) return INFINI_ATTN_ERR_INVALID;
  if (d->batch < 0 || d->seq_len < 0) return INFINI_ATTN_ERR_INVALID;
  if (d->n_q_heads < 1 || d->n_kv_heads < 1 || d->d_k < 1 || d->d_v < 1)
    return INFINI_ATTN_ERR_INVALID;
  if (d->n_q_heads % d->n_kv_heads != 0) return INFINI_ATTN_ERR_INVALID;
  if (d->dtype != INFINI_ATTN_F32 && d->dtype != INFINI_ATTN_BF16) return INFINI_ATTN_ERR_INVALID;
  if (!(d->eps > 0.f) || !(d->eps < 3.0e38f)) return INFINI_ATTN_ERR_INVALID;  // rejects NaN/inf
  if (d->device < 0) return INFINI_ATTN_ERR_INVALID;
  if (d->d_k != d->d_v) return INFINI_ATTN_ERR_UNSUPPORTED;
  if (d->d_k != 32 && d->d_k != 64 && d->d_k != 128) return INFINI_ATTN_ERR_UNSUPPORTED;
  // Every tensor is addressed with 64-bit offsets, but grid dimensions are
  // limited: B * Hq blocks along one axis. Rows per call stay below 2^30, so
  // that row counts rounded up to a tile in 32-bit arithmetic cannot overflow.
  if (static_cast<int64_t>(d->batch) * d->n_q_heads > 65535) return INFINI_ATTN_ERR_UNSUPPORTED;
  if (d->seq_len > (1 << 30)) return INFINI_ATTN_ERR_UNSUPPORTED;
  return INFINI_ATTN_OK;
}

// ceil(L / N), in 64-bit so that any seg_len up to INT32_MAX is safe.
int n_segments(int L, int N) {
  return L == 0 ? 0 : static_cast<int>((static_cast<int64_t>(L) + N - 1) / N);
}

// Segment length the kernels see: a segment never holds more rows than the
// call has, so seg_len >= L is one segment of L rows (the same result), and
// workspace and grids are sized by rows that exist.
int effective_seg(int L, int seg_len) { return (L > 0 && seg_len > L) ? L : seg_len; }

// Workspace layout (each part 256-byte aligned), in this order:
//   z_pre  [B*Hkv][S+1][D] fp32   (slot S receives the final z)
//   mt_pre [B*Hkv][S][D][D]       fp32 or bf16 by storage type
//   dz     [B*Hkv][S][P][D] fp32  (bf16 storage only; P = z_parts(N) row ranges)
//   gh     [B*Hkv][S][2][D][D] fp32 (bf16 storage only)
//   vt     [B*Hkv][S][T][D][64] bf16 (bf16 storage only; T = ceil(N / 64)
//          64-key tiles per segment, V^T in the fused kernel's LDS layout)
//   chain  (bf16 storage, chains of 64+ segments) per chunk: [P | h], the
//          packed affine step and the state before the chunk, all fp32
//   zhl    [B*Hkv][S][2][D] bf16 (bf16 storage only): z_pre as hi + lo parts
struct WsLayout {
  size_t z, mt, dz, gh, vt, chain_x, chain_gh, chain_states, zhl, total;
  int chunk_len;
};

int vt_tiles(int N) { return (N + 63) / 64; }

// Row ranges per segment for the sigma(k) column sums: about 512 rows each.
int z_parts(int N) {
  const int p = (N + 511) / 512;
  return p < 1 ? 1 : (p > 8 ? 8 : p);
}

WsLayout ws_layout(const infini_attn_desc *d, int S, int N) {
  const size_t heads = static_cast<size_t>(d->batch) * d->n_kv_heads;
  const size_t D = static_cast<size_t>(d->d_k);
  const bool bf16 = d->dtype == INFINI_ATTN_BF16;
  WsLayout w;
  w.z = round_up(heads * (S + 1) * D * sizeof(float));
  w.mt = round_up(heads * S * D * D * (bf16 ? sizeof(uint16_t) : sizeof(float)));
  w.dz = bf16 ? round_up(heads * S * z_parts(N) * D * sizeof(float)) : 0;
  w.gh = bf16 ? round_up(heads * S * 2 * D * D * sizeof(float)) : 0;
  w.vt = bf16 ? round_up(heads * S * vt_tiles(N) * D * 64 * sizeof(uint16_t)) : 0;
  w.chunk_len = bf16 ? ia::chain_chunk_len(S, static_cast<int>(heads)) : 0;
  const size_t nc = w.chunk_len > 0 ? (S + w.chunk_len - 1) / w.chunk_len : 0;
  w.chain_x = round_up(heads * nc * D * 2 * D * sizeof(float));
  w.chain_gh = round_up(heads * nc * 2 * D * D * sizeof(float));
  w.chain_states = round_up(heads * nc * D * D * sizeof(float));
  w.zhl = bf16 ? round_up(heads * S * 2 * D * sizeof(uint16_t)) : 0;
  w.total = w.z + w.mt + w.dz + w.gh + w.vt + w.chain_x + w.chain_gh + w.chain_states + w.zhl;
  return w;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return INFINI_ATTN_OK;
  if (e == hipErrorOutOfMemory) return INFINI_ATTN_ERR_OOM;
  return INFINI_ATTN_ERR_HIP;
}

// Makes `dev` current for the lifetime of the guard and restores the caller's
// device afterwards.
struct DeviceGuard {
  int prev = -1;
  hipError_t err = hipSuccess;
  explicit DeviceGuard(int dev) {
    err = hipGetDevice(&prev);
    if (err == hipSuccess && prev != dev) err = hipSetDevice(dev);
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

// Grows *buf to at least `need` bytes (contents not kept).
int ensure_buffer(void **buf, size_t *bytes, size_t need) {
  if (need <= *bytes) return INFINI_ATTN_OK;
  if (*buf) {
    // hipFree waits for work still using the old buffer.
    if (hipFree(*buf) != hipSuccess) return INFINI_ATTN_ERR_HIP;
    *buf = nullptr;
    *bytes = 0;
  }
  void *p = nullptr;
  const hipError_t e = hipMalloc(&p, need);
  if (e != hipSuccess) return e == hipErrorOutOfMemory ? INFINI_ATTN_ERR_OOM : INFINI_ATTN_ERR_HIP;
  *buf = p;
  *bytes = need;
  return INFINI_ATTN_OK;
}

// The scan's and the fused kernel's workspace for geometry g, grown as needed.
int bind_workspace(infini_attn_handle *h, const ia::Geometry &g, ia::Workspace *ws) {
  const infini_attn_desc &d = h->desc;
  const WsLayout lay = ws_layout(&d, g.S, g.N);
  const int st = ensure_buffer(&h->ws, &h->ws_bytes, lay.total);
  if (st != INFINI_ATTN_OK) return st;
  char *base = static_cast<char *>(h->ws);
  ws->z_pre = reinterpret_cast<float *>(base);
  void *mt = base + lay.z;
  const bool bf16 = d.dtype == INFINI_ATTN_BF16;
  ws->mt_pre_f32 = bf16 ? nullptr : static_cast<float *>(mt);
  ws->mt_pre_bf16 = bf16 ? static_cast<uint16_t *>(mt) : nullptr;
  ws->dz = bf16 ? reinterpret_cast<float *>(base + lay.z + lay.mt) : nullptr;
  ws->z_parts = z_parts(g.N);
  ws->gh = bf16 ? reinterpret_cast<float *>(base + lay.z + lay.mt + lay.dz) : nullptr;
  ws->vt = bf16 ? reinterpret_cast<uint16_t *>(base + lay.z + lay.mt + lay.dz + lay.gh) : nullptr;
  ws->vt_tiles = vt_tiles(g.N);
  char *chain = base + lay.z + lay.mt + lay.dz + lay.gh + lay.vt;
  ws->chunk_len = lay.chunk_len;
  ws->chain_x = lay.chunk_len > 0 ? reinterpret_cast<float *>(chain) : nullptr;
  ws->chain_gh = lay.chunk_len > 0 ? reinterpret_cast<float *>(chain + lay.chain_x) : nullptr;
  ws->chain_states =
      lay.chunk_len > 0 ? reinterpret_cast<float *>(chain + lay.chain_x + lay.chain_gh) : nullptr;
  ws->z_hl = bf16 ? reinterpret_cast<uint16_t *>(chain + lay.chain_x + lay.chain_gh +
                                                 lay.chain_states)
                  : nullptr;
  return INFINI_ATTN_OK;
}

hipError_t launch_scan(const infini_attn_handle *h, const ia::Geometry &g, const void *k,
                       const void *v, float *M, float *z, int delta,
                       const ia::Workspace &ws) {
  return h->desc.dtype == INFINI_ATTN_BF16
             ? ia::launch_segment_scan_bf16(g, static_cast<const uint16_t *>(k),
                                            static_cast<const uint16_t *>(v), M, z, delta, ws,
                                            h->stream)
             : ia::launch_segment_scan_f32(g, static_cast<const float *>(k),
                                           static_cast<const float *>(v), M, z, delta, ws,
                                           h->stream);
}

// Final z: slot S of every head's snapshot row -> z [B*Hkv][D]. (The bf16
// scan's z prefix kernel writes it in place; the fp32 scan leaves it here.)
hipError_t copy_final_z(const infini_attn_handle *h, const ia::Geometry &g, float *z,
                        const ia::Workspace &ws) {
  if (h->desc.dtype == INFINI_ATTN_BF16) return hipSuccess;
  const size_t row = static_cast<size_t>(g.D) * sizeof(float);
  return hipMemcpy2DAsync(z, row, ws.z_pre + static_cast<size_t>(g.S) * g.D, (g.S + 1) * row, row,
                          static_cast<size_t>(g.B) * g.Hkv, hipMemcpyDeviceToDevice, h->stream);
}

// The forward pass on tensors of the given layouts (the C ABI's head-major
// ones, or the block's row-major projections).
int forward_impl(infini_attn_handle *h, const void *q, const void *k, const void *v,
                 const float *beta, float *M, float *z, int32_t seg_len, int32_t update_mode,
                 void *out, const ia::Layout &lq, const ia::Layout &lkv, const ia::Layout &lo) {
  if (!h) return INFINI_ATTN_ERR_INVALID;
  const infini_attn_desc &d = h->desc;
  int st = infini_attn_check(&d, seg_len, update_mode);
  if (st != INFINI_ATTN_OK) return st;
  if (d.batch == 0 || d.seq_len == 0) return INFINI_ATTN_OK;  // nothing to do; state unchanged
  if (!q || !k || !v || !beta || !M || !z || !out) return INFINI_ATTN_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return INFINI_ATTN_ERR_INVALID;
  if (!aligned(beta, 4) || !aligned(M, 4) || !aligned(z, 4)) return INFINI_ATTN_ERR_INVALID;

  DeviceGuard guard(d.device);
  if (guard.err != hipSuccess) return INFINI_ATTN_ERR_HIP;

  ia::Geometry g;
  g.B = d.batch;
  g.Hq = d.n_q_heads;
  g.Hkv = d.n_kv_heads;
  g.L = d.seq_len;
  g.D = d.d_k;
  g.N = effective_seg(d.seq_len, seg_len);
  g.S = n_segments(d.seq_len, g.N);
  g.eps = d.eps;
  g.lq = lq;
  g.lkv = lkv;
  g.lo = lo;
  // The bf16 kernels address a segment's rows (and a tile's) through 32-bit
  // buffer offsets.
  const int64_t elt = d.dtype == INFINI_ATTN_BF16 ? 2 : 4;
  if ((static_cast<int64_t>(g.N) * std::max(lq.sr, std::max(lkv.sr, lo.sr)) + d.d_k) * elt >
      INT32_MAX)
    return INFINI_ATTN_ERR_UNSUPPORTED;

  ia::Workspace ws;
  st = bind_workspace(h, g, &ws);
  if (st != INFINI_ATTN_OK) return st;
  const bool bf16 = d.dtype == INFINI_ATTN_BF16;

  TimedCall tc{};
  if (h->timing) {
    if (!h->spare.empty()) {
      tc = h->spare.back();
      h->spare.pop_back();
    } else {
      for (int i = 0; i < 3; ++i) {
        if (hipEventCreate(&tc.ev[i]) != hipSuccess) {
          for (int j = 0; j < i; ++j) (void)hipEventDestroy(tc.ev[j]);
          return INFINI_ATTN_ERR_HIP;
        }
      }
    }
    h->recorded.push_back(tc);
    if (hipEventRecord(tc.ev[0], h->stream) != hipSuccess) return INFINI_ATTN_ERR_HIP;
  }
  const int delta = update_mode == INFINI_ATTN_DELTA;
  hipError_t e = launch_scan(h, g, k, v, M, z, delta, ws);
  if (e != hipSuccess) return hip_status(e);
  if (h->timing && hipEventRecord(tc.ev[1], h->stream) != hipSuccess) return INFINI_ATTN_ERR_HIP;
  if (bf16) {
    e = ia::launch_fused_bf16(g, static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                              static_cast<const uint16_t *>(v), beta, ws,
                              static_cast<uint16_t *>(out), h->stream);
  } else {
    e = ia::launch_fused_f32(g, static_cast<const float *>(q), static_cast<const float *>(k),
                             static_cast<const float *>(v), beta, ws, static_cast<float *>(out),
                             h->stream);
  }
  if (e != hipSuccess) return hip_status(e);
  if (h->timing && hipEventRecord(tc.ev[2], h->stream) != hipSuccess) return INFINI_ATTN_ERR_HIP;
  return hip_status(copy_final_z(h, g, z, ws));
}

// Streaming decode. The split partials go to the handle's buffer (grown on
// demand) or, for the allocation-free variant, to the fixed per-device
// scratch array, which bounds the request size and is shared by every call
// on the device.
int decode_call(infini_attn_handle *h, const void *q, int32_t n_new, const void *k_cache,
                const void *v_cache, int32_t n_past, const float *beta, const float *M,
                const float *z, void *out, bool noalloc) {
  if (!h) return INFINI_ATTN_ERR_INVALID;
  const infini_attn_desc &d = h->desc;
  int st = check_desc(&d);
  if (st != INFINI_ATTN_OK) return st;
  if (n_new < 1 || n_past < 0 || static_cast<int64_t>(n_past) + n_new > d.seq_len)
    return INFINI_ATTN_ERR_INVALID;
  const int64_t nq = static_cast<int64_t>(d.n_q_heads / d.n_kv_heads) * n_new;
  if ((nq + 15) / 16 > 65535) return INFINI_ATTN_ERR_UNSUPPORTED;  // grid z of the split kernel
  if (d.batch == 0) return INFINI_ATTN_OK;
  if (!q || !k_cache || !v_cache || !beta || !M || !z || !out) return INFINI_ATTN_ERR_INVALID;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
    return INFINI_ATTN_ERR_INVALID;
  if (!aligned(beta, 4) || !aligned(M, 4) || !aligned(z, 4)) return INFINI_ATTN_ERR_INVALID;
  ia::DecodeGeometry g;
  g.B = d.batch;
  g.Hq = d.n_q_heads;
  g.Hkv = d.n_kv_heads;
  g.D = d.d_k;
  g.C = n_new;
  g.cap = d.seq_len;
  g.n_past = n_past;
  g.eps = d.eps;
  const size_t part_bytes = ia::decode_partial_floats(g) * sizeof(float);
  if (noalloc && part_bytes > ia::kDecodeScratchBytes) return INFINI_ATTN_ERR_SCRATCH;
  DeviceGuard guard(d.device);
  if (guard.err != hipSuccess) return INFINI_ATTN_ERR_HIP;
  float *part = nullptr;
  if (noalloc) {
    // Looked up by infini_attn_create with the device current; cached.
    if (ia::decode_scratch(d.device, &part) != hipSuccess) return INFINI_ATTN_ERR_HIP;
  } else {
    st = ensure_buffer(&h->dec_ws, &h->dec_ws_bytes, part_bytes);
    if (st != INFINI_ATTN_OK) return st;
    part = static_cast<float *>(h->dec_ws);
  }
  const hipError_t e =
      d.dtype == INFINI_ATTN_BF16
          ? ia::launch_decode_bf16(g, static_cast<const uint16_t *>(q),
                                   static_cast<const uint16_t *>(k_cache),
                                   static_cast<const uint16_t *>(v_cache), beta, M, z, part,
                                   static_cast<uint16_t *>(out), h->stream)
          : ia::launch_decode_f32(g, static_cast<const float *>(q),
                                  static_cast<const float *>(k_cache),
                                  static_cast<const float *>(v_cache), beta, M, z, part,
                                  static_cast<float *>(out), h->stream);
  return hip_status(e);
}

// The Infini-attention block. Weights are [out][in] row-major. The
// projections land row-major in one buffer, QKV [B, L, W] with W = (Hq +
// 2 Hkv) d (the query heads' columns, then the key heads', then the value
// heads'): one GEMM against a fused weight (Wq's rows, then Wk's, then Wv's),
// or one GEMM per weight writing its column block. The attention
// kernels read their heads' rows of it in place (row stride W) and write O
// row-major [B, L, Hq d], the output projection's input; nothing is
// regrouped.
int block_call(infini_attn_handle *h, int32_t d_model, const void *x, const void *wq,
               const void *wk, const void *wv, const void *wqkv, const void *wo,
               const float *beta, float *M, float *z, int32_t seg_len, int32_t update_mode,
               void *y) {
  if (!h) return INFINI_ATTN_ERR_INVALID;
  const infini_attn_desc &d = h->desc;
  int st = infini_attn_check(&d, seg_len, update_mode);
  if (st != INFINI_ATTN_OK) return st;
  if (d_model < 1) return INFINI_ATTN_ERR_INVALID;
  if (d.batch == 0 || d.seq_len == 0) return INFINI_ATTN_OK;
  if (!x || !wo || !beta || !M || !z || !y) return INFINI_ATTN_ERR_INVALID;
  const int64_t rows = static_cast<int64_t>(d.batch) * d.seq_len;
  const int64_t D = d.d_k, Hq = d.n_q_heads, Hkv = d.n_kv_heads;
  const int64_t W = (Hq + 2 * Hkv) * D;
  if (rows > INT32_MAX || W > INT32_MAX) return INFINI_ATTN_ERR_UNSUPPORTED;
  DeviceGuard guard(d.device);
  if (guard.err != hipSuccess) return INFINI_ATTN_ERR_HIP;
  if (!h->blas) {
    st = ia::blas_create(&h->blas, h->stream);
    if (st != INFINI_ATTN_OK) return st;
  }
  const size_t elt = d.dtype == INFINI_ATTN_BF16 ? 2 : 4;
  // QKV [rows][W], then O [rows][Hq D] (each part 256-byte aligned).
  const size_t o_off = round_up(static_cast<size_t>(rows) * W * elt);
  st = ensure_buffer(&h->blk_ws, &h->blk_ws_bytes, o_off + round_up(rows * Hq * D * elt));
  if (st != INFINI_ATTN_OK) return st;
  char *qkv = static_cast<char *>(h->blk_ws);
  char *o = qkv + o_off;
  const int n = static_cast<int>(rows);
  if (wqkv) {
    st = ia::blas_gemm_xwt(h->blas, d.dtype, n, static_cast<int>(W), d_model, x, d_model, wqkv,
                           d_model, qkv, static_cast<int>(W));
    if (st != INFINI_ATTN_OK) return st;
  } else {
    const struct {
      const void *w;
      int64_t col, width;
    } proj[3] = {{wq, 0, Hq * D}, {wk, Hq * D, Hkv * D}, {wv, (Hq + Hkv) * D, Hkv * D}};
    for (const auto &pj : proj) {
      st = ia::blas_gemm_xwt(h->blas, d.dtype, n, static_cast<int>(pj.width), d_model, x,
                             d_model, pj.w, d_model, qkv + pj.col * elt, static_cast<int>(W));
      if (st != INFINI_ATTN_OK) return st;
    }
  }
  const ia::Layout lrow{d.seq_len * W, D, W};
  const ia::Layout lout{d.seq_len * Hq * D, D, Hq * D};
  st = forward_impl(h, qkv, qkv + Hq * D * elt, qkv + (Hq + Hkv) * D * elt, beta, M, z, seg_len,
                    update_mode, o, lrow, lrow, lout);
  if (st != INFINI_ATTN_OK) return st;
  return ia::blas_gemm_xwt(h->blas, d.dtype, n, d_model, static_cast<int>(Hq * D), o,
                           static_cast<int>(Hq * D), wo, static_cast<int>(Hq * D), y, d_model);
}

}  // namespace

extern "C" {

int infini_attn_check(const infini_attn_desc *desc, int32_t seg_len, int32_t update_mode) {
  const int st = check_desc(desc);
  if (st != INFINI_ATTN_OK) return st;
  if (seg_len < 1) return INFINI_ATTN_ERR_INVALID;
  if (update_mode != INFINI_ATTN_LINEAR && update_mode != INFINI_ATTN_DELTA)
    return INFINI_ATTN_ERR_INVALID;
  if (static_cast<int64_t>(n_segments(desc->seq_len, seg_len)) > 65535)
    return INFINI_ATTN_ERR_UNSUPPORTED;
  return INFINI_ATTN_OK;
}

int infini_attn_workspace_size(const infini_attn_desc *desc, int32_t seg_len, size_t *bytes) {
  if (!bytes) return INFINI_ATTN_ERR_INVALID;
  const int st = infini_attn_check(desc, seg_len, INFINI_ATTN_LINEAR);
  if (st != INFINI_ATTN_OK) return st;
  const int N = effective_seg(desc->seq_len, seg_len);
  *bytes = ws_layout(desc, n_segments(desc->seq_len, N), N).total;
  return INFINI_ATTN_OK;
}

int infini_attn_create(infini_attn_t **h, const infini_attn_desc *desc) {
  if (!h) return INFINI_ATTN_ERR_INVALID;
  *h = nullptr;
  const int st = check_desc(desc);
  if (st != INFINI_ATTN_OK) return st;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return INFINI_ATTN_ERR_HIP;
  if (desc->device >= count) return INFINI_ATTN_ERR_INVALID;
  DeviceGuard guard(desc->device);
  if (guard.err != hipSuccess) return INFINI_ATTN_ERR_HIP;
  // The allocation-free decode's scratch address on this device, looked up
  // once per device with the device current (no allocation: the array is
  // part of the library's code object).
  float *scratch_addr = nullptr;
  if (ia::decode_scratch(desc->device, &scratch_addr) != hipSuccess) return INFINI_ATTN_ERR_HIP;
  infini_attn_handle *p = new (std::nothrow) infini_attn_handle;
  if (!p) return INFINI_ATTN_ERR_OOM;
  p->desc = *desc;
  p->stream = static_cast<hipStream_t>(desc->stream);
  p->ws = nullptr;
  p->ws_bytes = 0;
  p->dec_ws = nullptr;
  p->dec_ws_bytes = 0;
  p->blk_ws = nullptr;
  p->blk_ws_bytes = 0;
  p->blas = nullptr;
  p->bwd_ws = nullptr;
  p->bwd_ws_bytes = 0;
  p->timing = false;
  *h = p;
  return INFINI_ATTN_OK;
}

int infini_attn_forward(infini_attn_t *h, const void *q, const void *k, const void *v,
                        const float *beta, float *M, float *z, int32_t seg_len,
                        int32_t update_mode, void *out) {
  if (!h) return INFINI_ATTN_ERR_INVALID;
  const infini_attn_desc &d = h->desc;
  const ia::Layout lq = ia::head_major(d.n_q_heads, d.seq_len, d.d_k);
  const ia::Layout lkv = ia::head_major(d.n_kv_heads, d.seq_len, d.d_k);
  return forward_impl(h, q, k, v, beta, M, z, seg_len, update_mode, out, lq, lkv, lq);
}

int infini_attn_update(infini_attn_t *h, const void *k, const void *v, float *M, float *z,
                       int32_t update_mode) {
  if (!h) return INFINI_ATTN_ERR_INVALID;
  const infini_attn_desc &d = h->desc;
  const int32_t rows = d.seq_len;
  int st = infini_attn_check(&d, rows > 0 ? rows : 1, update_mode);
  if (st != INFINI_ATTN_OK) return st;
  if (d.batch == 0 || rows == 0) return INFINI_ATTN_OK;  // nothing to write
  if (!k || !v || !M || !z) return INFINI_ATTN_ERR_INVALID;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(M, 4) || !aligned(z, 4))
    return INFINI_ATTN_ERR_INVALID;
  DeviceGuard guard(d.device);
  if (guard.err != hipSuccess) return INFINI_ATTN_ERR_HIP;
  ia::Geometry g;
  g.B = d.batch;
  g.Hq = d.n_q_heads;
  g.Hkv = d.n_kv_heads;
  g.L = rows;
  g.D = d.d_k;
  g.N = rows;  // one segment
  g.S = 1;
  g.eps = d.eps;
  g.lkv = ia::head_major(d.n_kv_heads, rows, d.d_k);
  g.lq = g.lo = ia::head_major(d.n_q_heads, rows, d.d_k);
  ia::Workspace ws;
  st = bind_workspace(h, g, &ws);
  if (st != INFINI_ATTN_OK) return st;
  hipError_t e = launch_scan(h, g, k, v, M, z, update_mode == INFINI_ATTN_DELTA, ws);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(copy_final_z(h, g, z, ws));
}

int infini_attn_decode(infini_attn_t *h, const void *q, int32_t n_new, const void *k_cache,
                       const void *v_cache, int32_t n_past, const float *beta, const float *M,
                       const float *z, void *out) {
  return decode_call(h, q, n_new, k_cache, v_cache, n_past, beta, M, z, out, false);
}

int infini_attn_decode_noalloc(infini_attn_t *h, const void *q, int32_t n_new,
                               const void *k_cache, const void *v_cache, int32_t n_past,
                               const float *beta, const float *M, const float *z, void *out) {
  return decode_call(h, q, n_new, k_cache, v_cache, n_past, beta, M, z, out, true);
}

int infini_attn_block_forward(infini_attn_t *h, int32_t d_model, const void *x, const void *wq,
                              const void *wk, const void *wv, const void *wo, const float *beta,
                              float *M, float *z, int32_t seg_len, int32_t update_mode, void *y) {
  if (!wq || !wk || !wv) return INFINI_ATTN_ERR_INVALID;
  return block_call(h, d_model, x, wq, wk, wv, nullptr, wo, beta, M, z, seg_len, update_mode, y);
}

int infini_attn_block_forward_qkv(infini_attn_t *h, int32_t d_model, const void *x,
                                  const void *wqkv, const void *wo, const float *beta, float *M,
                                  float *z, int32_t seg_len, int32_t update_mode, void *y) {
  if (!wqkv) return INFINI_ATTN_ERR_INVALID;
  return block_call(h, d_model, x, nullptr, nullptr, nullptr, wqkv, wo, beta, M, z, seg_len,
                    update_mode, y);
}

int infini_attn_set_timing(infini_attn_t *h, int32_t enable) {
  if (!h) return INFINI_ATTN_ERR_INVALID;
  h->timing = enable != 0;
  return INFINI_ATTN_OK;
}

int infini_attn_get_timing(infini_attn_t *h, int32_t *calls, float *scan_ms, float *fused_ms) {
  if (!h) return INFINI_ATTN_ERR_INVALID;
  DeviceGuard guard(h->desc.device);
  if (guard.err != hipSuccess) return INFINI_ATTN_ERR_HIP;
  double scan = 0.0, fused = 0.0;
  int st = INFINI_ATTN_OK;
  for (TimedCall &tc : h->recorded) {
    float a = 0.f, b = 0.f;
    if (hipEventSynchronize(tc.ev[2]) != hipSuccess ||
        hipEventElapsedTime(&a, tc.ev[0], tc.ev[1]) != hipSuccess ||
        hipEventElapsedTime(&b, tc.ev[1], tc.ev[2]) != hipSuccess) {
      st = INFINI_ATTN_ERR_HIP;
    }
    scan += a;
    fused += b;
    h->spare.push_back(tc);
  }
  if (calls) *calls = static_cast<int32_t>(h->recorded.size());
  if (scan_ms) *scan_ms = static_cast<float>(scan);
  if (fused_ms) *fused_ms = static_cast<float>(fused);
  h->recorded.clear();
  return st;
}

int infini_attn_backward(infini_attn_t *h, const void *q, const void *k, const void *v,
                         const float *beta, const float *M0, const float *z0, int32_t seg_len,
                         int32_t update_mode, const void *d_out, const float *d_M,
                         const float *d_z, float *dq, float *dk, float *dv, float *dbeta,
                         float *dM0, float *dz0) {
  if (!h) return INFINI_ATTN_ERR_INVALID;
  const infini_attn_desc &d = h->desc;
  int st = infini_attn_check(&d, seg_len, update_mode);
  if (st != INFINI_ATTN_OK) return st;
  if (!dbeta || !aligned(dbeta, 4)) return INFINI_ATTN_ERR_INVALID;
  const size_t D = static_cast<size_t>(d.d_k);
  const size_t kvheads = static_cast<size_t>(d.batch) * d.n_kv_heads;
  if (kvheads > 0) {
    if (!M0 || !z0 || !dM0 || !dz0) return INFINI_ATTN_ERR_INVALID;
    if (!aligned(M0, 4) || !aligned(z0, 4) || !aligned(dM0, 4) || !aligned(dz0, 4))
      return INFINI_ATTN_ERR_INVALID;
    if ((d_M && !aligned(d_M, 4)) || (d_z && !aligned(d_z, 4))) return INFINI_ATTN_ERR_INVALID;
  }
  const bool rows = d.batch > 0 && d.seq_len > 0;
  if (rows) {
    if (!q || !k || !v || !beta || !d_out || !dq || !dk || !dv) return INFINI_ATTN_ERR_INVALID;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(d_out, 16) ||
        !aligned(beta, 4) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
      return INFINI_ATTN_ERR_INVALID;
  }
  DeviceGuard guard(d.device);
  if (guard.err != hipSuccess) return INFINI_ATTN_ERR_HIP;
  hipStream_t stream = h->stream;
  hipError_t e = hipMemsetAsync(dbeta, 0, sizeof(float) * d.n_q_heads, stream);
  if (e != hipSuccess) return hip_status(e);
  if (kvheads == 0) return INFINI_ATTN_OK;
  const size_t state_bytes = kvheads * D * D * sizeof(float);
  const size_t z_bytes = kvheads * D * sizeof(float);
  if (!rows) {  // no rows: the state passes through unchanged
    e = d_M ? hipMemcpyAsync(dM0, d_M, state_bytes, hipMemcpyDeviceToDevice, stream)
            : hipMemsetAsync(dM0, 0, state_bytes, stream);
    if (e == hipSuccess)
      e = d_z ? hipMemcpyAsync(dz0, d_z, z_bytes, hipMemcpyDeviceToDevice, stream)
              : hipMemsetAsync(dz0, 0, z_bytes, stream);
    return hip_status(e);
  }

  ia::Geometry g;
  g.B = d.batch;
  g.Hq = d.n_q_heads;
  g.Hkv = d.n_kv_heads;
  g.L = d.seq_len;
  g.D = d.d_k;
  g.N = effective_seg(d.seq_len, seg_len);
  g.S = n_segments(d.seq_len, g.N);
  g.eps = d.eps;
  g.lq = g.lo = ia::head_major(d.n_q_heads, d.seq_len, d.d_k);
  g.lkv = ia::head_major(d.n_kv_heads, d.seq_len, d.d_k);
  const int delta = update_mode == INFINI_ATTN_DELTA;

  // Scratch layout (each part 256-byte aligned): z_pre, mt, dzs, lse, erow,
  // gd, dden, R, r, G (delta only), qz, H, gma, gza, and the per-block
  // partial sums (products, qz, dbeta).
  const size_t units = kvheads * g.S;
  const size_t qrows = static_cast<size_t>(g.B) * g.Hq * g.L;
  const ia::BwdBlocks nb = ia::backward_blocks(g);
  const size_t part_floats =
      units * std::max(static_cast<size_t>(nb.rows) * D * D,
                       static_cast<size_t>(nb.group_rows) * (D * D + D));
  const size_t sz[17] = {
      round_up(kvheads * (g.S + 1) * D * sizeof(float)), round_up(units * D * D * sizeof(float)),
      round_up(units * D * sizeof(float)), round_up(qrows * sizeof(float)),
      round_up(qrows * sizeof(float)), round_up(qrows * sizeof(float)),
      round_up(qrows * sizeof(float)), round_up(units * D * D * sizeof(float)),
      round_up(units * D * sizeof(float)), delta ? round_up(units * D * D * sizeof(float)) : 0,
      round_up(units * D * sizeof(float)), round_up(units * D * D * sizeof(float)),
      round_up(units * D * D * sizeof(float)), round_up(units * D * sizeof(float)),
      round_up(part_floats * sizeof(float)),
      round_up(units * nb.chunks * D * sizeof(float)),
      round_up(static_cast<size_t>(g.Hq) * g.B * g.S * nb.qblocks * sizeof(float))};
  size_t total = 0;
  for (size_t x : sz) total += x;
  st = ensure_buffer(&h->bwd_ws, &h->bwd_ws_bytes, total);
  if (st != INFINI_ATTN_OK) return st;
  float *part[17];
  char *base = static_cast<char *>(h->bwd_ws);
  for (int i = 0; i < 17; ++i) {
    part[i] = reinterpret_cast<float *>(base);
    base += sz[i];
  }
  ia::BwdWorkspace w;
  w.z_pre = part[0];
  w.mt = part[1];
  w.dzs = part[2];
  w.lse = part[3];
  w.erow = part[4];
  w.gd = part[5];
  w.dden = part[6];
  w.R = part[7];
  w.r = part[8];
  w.G = delta ? part[9] : nullptr;
  w.qz = part[10];
  w.H = part[11];
  w.gma = part[12];
  w.gza = part[13];
  w.part = part[14];
  w.qz_part = part[15];
  w.dbeta_part = part[16];

  // R, r, G, H, qz (delta) and dbeta are written whole by the ordered sums of
  // their partials; the linear rule has no qz term.
  if (!delta) {
    e = hipMemsetAsync(w.qz, 0, sz[10], stream);
    if (e != hipSuccess) return hip_status(e);
  }
  if (d.dtype == INFINI_ATTN_BF16) {
    const uint16_t *qb = static_cast<const uint16_t *>(q), *kb = static_cast<const uint16_t *>(k),
                   *vb = static_cast<const uint16_t *>(v),
                   *ob = static_cast<const uint16_t *>(d_out);
    e = ia::launch_backward<uint16_t>(g, qb, kb, vb, ob, beta, M0, z0, d_M, d_z, delta, w, dq, dk,
                                      dv, dbeta, dM0, dz0, stream);
  } else {
    const float *qf = static_cast<const float *>(q), *kf = static_cast<const float *>(k),
                *vf = static_cast<const float *>(v), *of = static_cast<const float *>(d_out);
    e = ia::launch_backward<float>(g, qf, kf, vf, of, beta, M0, z0, d_M, d_z, delta, w, dq, dk,
                                   dv, dbeta, dM0, dz0, stream);
  }
  return hip_status(e);
}

int infini_attn_destroy(infini_attn_t *h) {
  if (!h) return INFINI_ATTN_OK;
  int st = INFINI_ATTN_OK;
  {
    DeviceGuard guard(h->desc.device);
    for (auto *list : {&h->recorded, &h->spare})
      for (TimedCall &tc : *list)
        for (hipEvent_t ev : tc.ev) (void)hipEventDestroy(ev);
  }
  if (h->blas) {
    DeviceGuard guard(h->desc.device);
    ia::blas_destroy(h->blas);
  }
  for (void *buf : {h->ws, h->dec_ws, h->blk_ws, h->bwd_ws}) {
    if (!buf) continue;
    DeviceGuard guard(h->desc.device);
    if (guard.err != hipSuccess || hipFree(buf) != hipSuccess) st = INFINI_ATTN_ERR_HIP;
  }
  delete h;
  return st;
}

const char *infini_attn_strerror(int status) {
  switch (status) {
    case INFINI_ATTN_OK: return "ok";
    case INFINI_ATTN_ERR_INVALID: return "invalid argument";
    case INFINI_ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case INFINI_ATTN_ERR_HIP: return "HIP runtime or launch failure";
    case INFINI_ATTN_ERR_OOM: return "out of device memory";
    case INFINI_ATTN_ERR_SCRATCH:
      return "request larger than the fixed scratch of the allocation-free entry point";
  }
  return "unknown status";
}

}  // extern "C"
