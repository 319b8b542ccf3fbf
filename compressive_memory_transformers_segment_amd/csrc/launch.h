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
  float *z_pre;        // [B*Hkv][S][D] fp32
  float *mt_pre_f32;   // [B*Hkv][S][D(v)][D(k)] fp32, M^T (fp32 storage path)
  uint16_t *mt_pre_bf16;  // [B*Hkv][S][D(v)][D(k)] bf16 bits, M^T (bf16 storage path)
};

// Segment scan: carries fp32 (M, z) across segments for every (b, kv head),
// writing the pre-segment snapshots and the final state (in place in M, z).
// `bf16_inputs` selects the storage type of k and v.
hipError_t launch_segment_scan(const Geometry &g, bool bf16_inputs, const void *k, const void *v,
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

}  // namespace ia
