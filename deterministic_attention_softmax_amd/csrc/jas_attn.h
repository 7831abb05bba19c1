// jas_attn.h -- internal interface of the fused attention forward
// (jas_attn.hip), kept apart from the row-softmax kernels' jas_internal.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jas_internal.h"

namespace jas {

// Fused attention forward (QK, the row softmax, PV).
struct AttnArgs {
  const void *q, *k, *v;  // [B,H,Sq,D], [B,Hkv,N,D], [B,Hkv,N,D]
  void *out;              // [B,H,Sq,D]
  const float *mask;      // nullptr when no mask
  int64_t msb, msh, msq;
  Exclusion ex;
  const float *sink;      // nullptr when no sink
  float *p_sink, *lse;    // [rows] or nullptr
  void *probs;            // optional [B,H,Sq,N], dtype
  float *scores;          // optional [B,H,Sq,N], binary32
  float scale;
  int64_t B, H, Hkv, Sq, N;
  int D, T;               // head dim, 256-key tiles
};

// qblocks: 16-query blocks per wave (1 or 2), 0 = chosen from the shape
hipError_t launch_attn_fwd(int dtype, const AttnArgs &a, int qblocks, hipStream_t stream);

}  // namespace jas
