// Device helpers for the per-tensor scale state, used by the bookkeeping
// kernel and by the fused quantizer.
#pragma once

#include "fp8vit_internal.h"

namespace fp8vit {

// descale = max(fp32(A / 448), 1e-10f). __fdiv_rn is the IEEE round-to-nearest
// division, matching the formula's fp32 divide.
__device__ __forceinline__ float descale_from_amax(float A) {
  float d = __fdiv_rn(A, kFp8Max);
  return d > kDescaleFloor ? d : kDescaleFloor;
}

// Window maximum per tensor after (virtually) writing `amax` into slot
// count % 16, and the resulting descales. Reads the ring only; callers that
// run on many blocks read it before any block commits.
__device__ __forceinline__ void ring_window_descales(const DevState* st, uint32_t count,
                                                     const float amax[3], float descale[3]) {
  const uint32_t slot = count % FP8VIT_RING_SLOTS;
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    float w = amax[x];
#pragma unroll
    for (int i = 0; i < FP8VIT_RING_SLOTS; ++i) {
      float r = st->ring[x][i];
      w = (i != (int)slot && r > w) ? r : w;
    }
    descale[x] = descale_from_amax(w);
  }
}

// Push a recorded amax triple into ring slot count % 16: one thread only, at
// a point where no other thread reads the ring.
__device__ __forceinline__ void ring_push(DevState* st, const float amax[3]) {
  const uint32_t count = st->count;
  const uint32_t slot = count % FP8VIT_RING_SLOTS;
#pragma unroll
  for (int x = 0; x < 3; ++x) st->ring[x][slot] = amax[x];
  st->count = count + 1;
}

// Push the amax the last dynamic quantize pass left pending, if any.
__device__ __forceinline__ void ring_push_pending(DevState* st) {
  if (st->pending != 0u) {
    const float a[3] = {st->pending_amax[0], st->pending_amax[1], st->pending_amax[2]};
    ring_push(st, a);
    st->pending = 0u;
  }
}

// Record this forward's amax and descales; the ring push stays pending.
__device__ __forceinline__ void record_pending(DevState* st, const float amax[3], const float descale[3]) {
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    st->pending_amax[x] = amax[x];
    st->amax_last[x] = amax[x];
    st->descale_used[x] = descale[x];
  }
  st->pending = 1u;
}

}  // namespace fp8vit
