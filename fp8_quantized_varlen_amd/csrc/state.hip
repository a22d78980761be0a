// Scale bookkeeping kernels: state reset, static values, dynamic ring update.
//
// The ring follows the vLLM page "FP8 ViT Encoder Attention", Usage: a
// 16-entry circular buffer of observed Q/K/V amax drives the per-forward scale.
// This forward's amax goes into slot count % 16 and the descale comes from the
// maximum over all 16 slots after that push; empty slots hold 0, which never
// wins since amax >= 0. descale = max(A / 448, 1e-10) with an IEEE division
// (atrex-bench #025 per_token_group_quant_fp8, Reference Implementation).
#include "fp8vit_internal.h"
#include "state_device.h"

namespace fp8vit {

__global__ void state_init_kernel(DevState* st) {
  uint32_t* w = reinterpret_cast<uint32_t*>(st);
  for (int i = threadIdx.x; i < (int)(sizeof(DevState) / 4); i += blockDim.x) w[i] = 0u;
}

__global__ void state_set_static_kernel(DevState* st, float q, float k, float v) {
  if (threadIdx.x == 0) {
    st->static_values[0] = q;
    st->static_values[1] = k;
    st->static_values[2] = v;
  }
}

// Set the option bits; the saturation counts start again from zero.
__global__ void state_set_flags_kernel(DevState* st, uint32_t flags) {
  if (threadIdx.x == 0) {
    st->flags = flags;
#pragma unroll
    for (int x = 0; x < 3; ++x) st->saturated[x] = 0ull;
  }
}

// One workgroup checks every boundary of cu_seqlens and writes the FP8VIT_CU_*
// bits of the conditions it violates.
__global__ void check_cu_seqlens_kernel(const int32_t* cu, int32_t nseg, int32_t T, int32_t max_seqlen,
                                        DevState* st) {
  __shared__ uint32_t bits;
  if (threadIdx.x == 0) {
    bits = 0u;
    if (cu[0] != 0) bits |= FP8VIT_CU_FIRST_NOT_ZERO;
    if (cu[nseg] != T) bits |= FP8VIT_CU_LAST_NOT_T;
  }
  __syncthreads();
  uint32_t b = 0u;
  for (int i = threadIdx.x; i < nseg; i += blockDim.x) {
    const int64_t a = cu[i], c = cu[i + 1];
    if (c < a) b |= FP8VIT_CU_DECREASING;
    if (c - a > (int64_t)max_seqlen) b |= FP8VIT_CU_LONGER_THAN_MAX;
  }
  if (b != 0u) atomicOr(&bits, b);
  __syncthreads();
  if (threadIdx.x == 0) st->cu_check = bits;
}

__global__ void scales_update_kernel(DevState* st, const float* amax) {
  if (threadIdx.x == 0) {
    float a[3] = {amax[0], amax[1], amax[2]};
    float d[3];
    ring_push_pending(st);
    ring_window_descales(st, st->count, a, d);
    ring_push(st, a);
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      st->amax_last[x] = a[x];
      st->descale_used[x] = d[x];
    }
  }
}

hipError_t launch_state_init(DevState* st, hipStream_t s) {
  hipLaunchKernelGGL(state_init_kernel, dim3(1), dim3(256), 0, s, st);
  return hipGetLastError();
}

hipError_t launch_state_set_static(DevState* st, float q, float k, float v, hipStream_t s) {
  hipLaunchKernelGGL(state_set_static_kernel, dim3(1), dim3(64), 0, s, st, q, k, v);
  return hipGetLastError();
}

hipError_t launch_scales_update(DevState* st, const float* d_amax, hipStream_t s) {
  hipLaunchKernelGGL(scales_update_kernel, dim3(1), dim3(64), 0, s, st, d_amax);
  return hipGetLastError();
}

hipError_t launch_state_set_flags(DevState* st, uint32_t flags, hipStream_t s) {
  hipLaunchKernelGGL(state_set_flags_kernel, dim3(1), dim3(64), 0, s, st, flags);
  return hipGetLastError();
}

hipError_t launch_check_cu_seqlens(const int32_t* cu, int32_t nseg, int32_t total_tokens, int32_t max_seqlen,
                                   DevState* st, hipStream_t s) {
  hipLaunchKernelGGL(check_cu_seqlens_kernel, dim3(1), dim3(256), 0, s, cu, nseg, total_tokens, max_seqlen, st);
  return hipGetLastError();
}

}  // namespace fp8vit
