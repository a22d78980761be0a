// Internal declarations shared by the host library and the HIP kernels.
// Not part of the public ABI (include/fp8vit.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8vit.h"

namespace fp8vit {

// Per-layer device state. The caller allocates fp8vit_state_bytes() bytes.
struct alignas(256) DevState {
  float ring[3][FP8VIT_RING_SLOTS];  // observed amax of q, k, v
  uint32_t count;                    // dynamic forwards recorded so far
  float static_values[3];            // static q/k/v values (margin included)
  float descale_used[3];             // descales of the last quantize / update
  float amax_last[3];                // amax of the last dynamic forward
  uint32_t flags;                    // reserved: 0
  uint32_t reserved0;
  uint32_t amax_bits[2][4];          // atomic-max scratch of the amax pass (row 0); 0 between forwards
  uint32_t bar_arrived;              // blocks of the amax pass that finished; 0 between forwards
  uint32_t reserved2;
  uint32_t reserved1[54];
};
static_assert(sizeof(DevState) == 512, "state layout");

constexpr float kFp8Max = 448.0f;
constexpr float kDescaleFloor = 1e-10f;

// Launch wrappers (defined in the .hip files). All return hipError_t of the launch.
hipError_t launch_state_init(DevState* st, hipStream_t s);
hipError_t launch_state_set_static(DevState* st, float q, float k, float v, hipStream_t s);
hipError_t launch_scales_update(DevState* st, const float* d_amax, hipStream_t s);

struct QuantArgs {
  const uint16_t* x[3];
  int64_t ld[3];
  uint8_t* y[3];
  int32_t T;
  int32_t row8;   // H*d/8 (16-byte chunks per token row)
  DevState* st;
};
hipError_t launch_quantize(const QuantArgs& a, bool dynamic, hipStream_t s);

struct AttnArgs {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8;
  const int32_t* cu;
  int32_t nseg;
  int32_t H;
  int32_t ntiles_ub;     // upper bound on query tiles per head (set by launch_attn)
  uint32_t tensor_bytes; // T * H * d: bytes of each of q8, k8, v8
  const DevState* st;
  uint16_t* out;           // bf16 output (out8 == nullptr)
  uint8_t* out8;           // e4m3 output, or nullptr
  const float* out_descale;  // device fp32, with out8
  int64_t ld_out;          // token stride of the output, elements
  float softmax_scale;
};
// Picks the workgroup shape and sets a.ntiles_ub for it.
hipError_t launch_attn(const AttnArgs& a, int head_dim, int total_tokens, int max_seqlen, hipStream_t s);
int attn_block_m(int head_dim);

}  // namespace fp8vit
