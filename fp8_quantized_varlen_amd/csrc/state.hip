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

}  // namespace fp8vit
