// Internal launch interface between the host library and the gfx950 kernels.
// Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ia {

// Problem geometry of one forward call, already validated on the host.
struct Geometry {
  int B, Hq, Hkv, L, D;  // D = d_k = d_v
  int N;                 // segment length
  int S;                 // number of segments, ceil(L / N)
  float eps;
};

// Per-segment state snapshots written by the scan and read by the fused
// kernel. Index (b * Hkv + j) * S + s holds the state *before* segment s.
struct Workspace {
  float *z_pre;           // [B*Hkv][S+1][D] fp32; slot S receives the final z
  float *mt_pre_f32;      // [B*Hkv][S][D(v)][D(k)] fp32, M^T (fp32 storage path)
  uint16_t *mt_pre_bf16;  // [B*Hkv][S][D(v)][D(k)] bf16 bits, M^T (bf16 storage path)
  float *dz;              // [B*Hkv][S][z_parts][D] partial sums of sigma(k) (bf16 path)
  int z_parts;            // row ranges per segment in dz
  float *gh;              // [B*Hkv][S][2][D*D] G_s, H_s in MFMA fragment order (bf16 path)
};

// Segment scan, fp32 storage: carries fp32 (M, z) across segments for every
// (b, kv head) on VALU, writing the pre-segment snapshots (z_pre, mt_pre_f32)
// and the final M in place; the final z lands in z_pre slot S.
hipError_t launch_segment_scan_f32(const Geometry &g, const float *k, const float *v, float *M,
                                   const float *z, int delta, const Workspace &ws,
                                   hipStream_t stream);

// Segment scan, bf16 storage: per-segment statistics on MFMA in parallel, then
// the fp32 recurrence; writes z_pre (slot S = final z), mt_pre_bf16 and M.
hipError_t launch_segment_scan_bf16(const Geometry &g, const uint16_t *k, const uint16_t *v,
                                    float *M, const float *z, int delta, const Workspace &ws,
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

}  // namespace ia
