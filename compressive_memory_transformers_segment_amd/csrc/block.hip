// The Infini-attention block around the attention kernels: Q/K/V projections
// of the layer input, the Infini-attention forward, and the output projection
// ([HF-repro] "Infini-Attention メカニズム": the layer's own query, key and
// value states feed the mechanism; [LNCB-review] "基本アイデア": it replaces
// the attention inside each layer's block).
//
//   x [B, L, d_model]  ->  QKV = x [Wq | Wk | Wv]  [B, L, (Hq + 2 Hkv) d]
//   (one d-column slice per head, heads side by side in each row)
//   ->  O = InfiniAttention(Q, K, V; beta, M, z), read from QKV in place and
//       written as [B, L, Hq d] (the heads of a row side by side)
//   ->  y = O Wo  [B, L, d_model].
//
// The projections are plain dense GEMMs over all B * L rows at once and go to
// rocBLAS (fp32 accumulation, results rounded to the storage type). The
// attention kernels take the row stride of these row-major buffers, so no
// tensor is regrouped between the GEMMs and the kernels.

#include "infini_attn.h"

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <stdint.h>

#include "common.h"

namespace {

int blas_status(rocblas_status s) {
  if (s == rocblas_status_success) return INFINI_ATTN_OK;
  if (s == rocblas_status_memory_error) return INFINI_ATTN_ERR_OOM;
  return INFINI_ATTN_ERR_HIP;
}

}  // namespace

namespace ia {

int blas_create(void **blas, hipStream_t stream) {
  rocblas_handle hb = nullptr;
  int st = blas_status(rocblas_create_handle(&hb));
  if (st != INFINI_ATTN_OK) return st;
  st = blas_status(rocblas_set_stream(hb, stream));
  if (st != INFINI_ATTN_OK) {
    (void)rocblas_destroy_handle(hb);
    return st;
  }
  *blas = hb;
  return INFINI_ATTN_OK;
}

void blas_destroy(void *blas) {
  if (blas) (void)rocblas_destroy_handle(static_cast<rocblas_handle>(blas));
}

// Row-major C (rows x n, leading dimension ldc) = X (rows x k, ldx) W^T with
// W row-major n x k (ldw), fp32 accumulation; passed to the column-major BLAS
// as C^T = W X^T (W read transposed from its column-major k x n view). Weights
// stored [out][in] make the library's faster kernels apply: 13-14% over
// [in][out] weights at the Llama-3-8B projection shapes.
int blas_gemm_xwt(void *blas, int dtype, int rows, int n, int k, const void *x, int ldx,
                  const void *w, int ldw, void *c, int ldc) {
  const float one = 1.f, zero = 0.f;
  const rocblas_datatype t = dtype == INFINI_ATTN_BF16 ? rocblas_datatype_bf16_r
                                                       : rocblas_datatype_f32_r;
  const rocblas_status s = rocblas_gemm_ex(
      static_cast<rocblas_handle>(blas), rocblas_operation_transpose, rocblas_operation_none, n,
      rows, k, &one, w, t, ldw, x, t, ldx, &zero, c, t, ldc, c, t, ldc, rocblas_datatype_f32_r,
      rocblas_gemm_algo_standard, 0, 0);
  return blas_status(s);
}

}  // namespace ia
