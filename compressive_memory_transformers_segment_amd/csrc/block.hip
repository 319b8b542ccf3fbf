// The Infini-attention block around the attention kernels: Q/K/V projections
// of the layer input, the Infini-attention forward, and the output projection
// ([HF-repro] "Infini-Attention メカニズム": the layer's own query, key and
// value states feed the mechanism; [LNCB-review] "基本アイデア": it replaces
// the attention inside each layer's block).
//
//   x [B, L, d_model]  ->  Q = x Wq, K = x Wk, V = x Wv, one d-column slice
//   per head, written head-major [B, H, L, d] (the layout the kernels read)
//   ->  O = InfiniAttention(Q, K, V; beta, M, z)  [B, Hq, L, d]
//   ->  O' = O regrouped as [B, L, Hq * d] (the heads of a row side by side)
//   ->  y = O' Wo  [B, L, d_model].
//
// The projections are plain dense GEMMs over all B * L rows at once and go to
// rocBLAS (fp32 accumulation, results rounded to the storage type). Their
// row-major results are regrouped head-major for the kernels, and O back to
// row-major for the output projection, by a row copy kernel (each (b, h, l)
// row of d elements moves as whole 16-byte units). A strided batch of per-head
// GEMMs would write head-major directly, but every head would then read all
// of x again. Row-major matrices are
// passed to the column-major BLAS as their transposes: C = A B row-major is
// C^T = B^T A^T column-major.

#include "infini_attn.h"

#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <stdint.h>

#include "common.h"

namespace {

// Regrouping between head-major [B][H][L][D] and row-major [B][L][H][D],
// 16-byte units; TO_ROWS: head-major -> row-major, else the inverse. Unit u
// walks the head-major side in order.
template <int UPR, bool TO_ROWS>  // 16-byte units per row of D elements
__global__ __launch_bounds__(256) void regroup_kernel(const ia::u32x4 *__restrict__ src,
                                                      ia::u32x4 *__restrict__ dst, int H, int L,
                                                      long long n_units) {
  for (long long u = blockIdx.x * 256ll + threadIdx.x; u < n_units; u += 256ll * gridDim.x) {
    const long long row = u / UPR;
    const int part = static_cast<int>(u % UPR);
    const int l = static_cast<int>(row % L);
    const long long bh = row / L;
    const int h = static_cast<int>(bh % H);
    const long long b = bh / H;
    const long long r = ((b * L + l) * H + h) * UPR + part;
    if (TO_ROWS)
      dst[r] = src[u];
    else
      dst[u] = src[r];
  }
}

template <bool TO_ROWS>
hipError_t regroup(const void *src, void *dst, int B, int H, int L, int row_bytes,
                   hipStream_t stream) {
  const long long units = static_cast<long long>(B) * H * L * (row_bytes / 16);
  if (units == 0) return hipSuccess;
  const long long want = (units + 255) / 256;
  const unsigned grid = static_cast<unsigned>(want < 8192 ? want : 8192);
  const auto *s = static_cast<const ia::u32x4 *>(src);
  auto *d = static_cast<ia::u32x4 *>(dst);
  switch (row_bytes / 16) {
    case 4: regroup_kernel<4, TO_ROWS><<<grid, 256, 0, stream>>>(s, d, H, L, units); break;
    case 8: regroup_kernel<8, TO_ROWS><<<grid, 256, 0, stream>>>(s, d, H, L, units); break;
    case 16: regroup_kernel<16, TO_ROWS><<<grid, 256, 0, stream>>>(s, d, H, L, units); break;
    case 32: regroup_kernel<32, TO_ROWS><<<grid, 256, 0, stream>>>(s, d, H, L, units); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int blas_status(rocblas_status s) {
  if (s == rocblas_status_success) return INFINI_ATTN_OK;
  if (s == rocblas_status_memory_error) return INFINI_ATTN_ERR_OOM;
  return INFINI_ATTN_ERR_HIP;
}

}  // namespace

namespace ia {

hipError_t launch_heads_to_rows(const void *src, void *dst, int B, int H, int L, int row_bytes,
                                hipStream_t stream) {
  return regroup<true>(src, dst, B, H, L, row_bytes, stream);
}

hipError_t launch_rows_to_heads(const void *src, void *dst, int B, int H, int L, int row_bytes,
                                hipStream_t stream) {
  return regroup<false>(src, dst, B, H, L, row_bytes, stream);
}

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

// Row-major C[i] (rows x n, ldc = n) = X (rows x k, ld = ldx) W[i], where W[i]
// is the k x n column slice i of a k x ldw row-major matrix (slices at stride
// n) and C[i] lies at stride rows * n: the head-major projection for batch =
// heads; batch 1 with n = ldw is a plain GEMM.
int blas_gemm_rowmajor(void *blas, int dtype, int rows, int n, int k, const void *x, int ldx,
                       const void *w, int ldw, void *c, int batch) {
  const float one = 1.f, zero = 0.f;
  const rocblas_datatype t = dtype == INFINI_ATTN_BF16 ? rocblas_datatype_bf16_r
                                                       : rocblas_datatype_f32_r;
  const rocblas_status s = rocblas_gemm_strided_batched_ex(
      static_cast<rocblas_handle>(blas), rocblas_operation_none, rocblas_operation_none, n, rows,
      k, &one, w, t, ldw, static_cast<rocblas_stride>(n), x, t, ldx, 0, &zero, c, t, n,
      static_cast<rocblas_stride>(rows) * n, c, t, n, static_cast<rocblas_stride>(rows) * n,
      batch, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  return blas_status(s);
}

}  // namespace ia
