// Internal declarations shared by the host library and the HIP kernels.
// Not part of the public ABI (include/fp8vit.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fp8vit.h"

namespace fp8vit {

// Workgroups of the first dynamic pass: at most this many per-block partials
// fit in the state.
constexpr int kAmaxSlots = 1024;

// Per-layer device state. The caller allocates fp8vit_state_bytes() bytes.
// The first 512 bytes hold what fp8vit_state_read reports (plus the pending
// ring push and the first dynamic pass's window); the rest is that pass's
// per-block partials (amax, and clamp counts when they are counted).
//
// Dynamic bookkeeping is split over the two launches of a forward. Pass 1
// reads the ring (with the previous forward's pending push applied in its
// reading, not written) and quantizes with the window maximum over the other
// 15 slots, recording per-block partial maxima. Pass 2 reduces them to this
// forward's amax; one of its threads pushes the previous pending amax and
// records this one as pending (no other thread reads the ring in pass 2);
// every workgroup re-quantizes its share of a tensor whose amax raised the
// window (and so its descale). fp8vit_scales_update pushes a pending amax
// first, and fp8vit_state_read applies one to the view it returns.
struct alignas(256) DevState {
  float ring[3][FP8VIT_RING_SLOTS];  // observed amax of q, k, v
  uint32_t count;                    // dynamic forwards pushed into the ring
  float static_values[3];            // static q/k/v values (margin included)
  float descale_used[3];             // descales of the last quantize / update
  float amax_last[3];                // amax of the last dynamic forward
  uint32_t flags;                    // FP8VIT_FLAG_* bits (fp8vit_state_set_flags)
  uint32_t pending;                  // 1: pending_amax still has to be pushed
  float pending_amax[3];
  uint32_t cu_check;                 // FP8VIT_CU_* bits of the last fp8vit_check_cu_seqlens
  unsigned long long saturated[3];   // elements clamped at +-448 (with FP8VIT_FLAG_COUNT_SATURATION)
  float win_other[3];                // dynamic pass 1: window max over the other 15 ring slots
  uint32_t reserved0[55];
  uint32_t amax_part[kAmaxSlots][4];  // dynamic pass 1, block b: |q|, |k|, |v| maxima (bf16 magnitude bits)
  uint32_t sat_part[kAmaxSlots][4];   // dynamic pass 1, block b: clamped q, k, v elements (flag set)
};
constexpr size_t kStateViewBytes = 512;   // the reported part, before the per-block partials
static_assert(offsetof(DevState, amax_part) == kStateViewBytes, "state layout");
static_assert(offsetof(DevState, saturated) == 256, "state layout");
static_assert(sizeof(DevState) == 512 + 32 * kAmaxSlots, "state layout");

// Compute units of the current device (cached per device; 0 on error).
int device_cus();

constexpr float kFp8Max = 448.0f;
constexpr float kDescaleFloor = 1e-10f;

// Launch wrappers (defined in the .hip files). All return hipError_t of the launch.
hipError_t launch_state_init(DevState* st, hipStream_t s);
hipError_t launch_state_set_static(DevState* st, float q, float k, float v, hipStream_t s);
hipError_t launch_scales_update(DevState* st, const float* d_amax, hipStream_t s);
hipError_t launch_state_set_flags(DevState* st, uint32_t flags, hipStream_t s);
hipError_t launch_check_cu_seqlens(const int32_t* cu, int32_t nseg, int32_t total_tokens, int32_t max_seqlen,
                                   DevState* st, hipStream_t s);

struct QuantArgs {
  const uint16_t* x[3];
  int64_t ld[3];
  uint8_t* y[3];
  int32_t T;
  int32_t row8;   // H*d/8 (16-byte chunks per token row)
  int32_t amax_blocks;  // workgroups of dynamic pass 1 (partials to reduce)
  uint32_t quant_mask;  // tensors the quantize pass writes (bit 0 q, 1 k, 2 v)
  DevState* st;
};
hipError_t launch_quantize(const QuantArgs& a, bool dynamic, hipStream_t s);
// Block-scaled e4m3 codes [T, H, d] and E8M0 scales [T, H, 4] of two bf16
// tensors (Q and K), one launch.
struct MxArgs {
  const uint16_t* x[2];
  int64_t ld[2];
  uint8_t* codes[2];
  uint8_t* scales[2];
  int32_t T;
  int32_t H;
};
hipError_t launch_quantize_mx(const MxArgs& a, int32_t d, hipStream_t s);

struct AttnArgs {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8;
  const int32_t* cu;
  int32_t nseg;
  int32_t H;
  int32_t ntiles_ub;     // upper bound on query tiles per head (set by launch_attn)
  uint32_t tensor_bytes; // T * H * d: bytes of each of q8, k8, v8
  int32_t T;             // tokens (every segment is clamped to [0, T])
  const DevState* st;
  uint16_t* out;           // bf16 output (out8 == nullptr)
  uint8_t* out8;           // e4m3 output, or nullptr
  const float* out_descale;  // device fp32, with out8
  int64_t ld_out;          // token stride of the output, elements
  float softmax_scale;
  // Block-scaled variant: E8M0 scales of Q and K, four bytes per (token,
  // head); null for the per-tensor path.
  const uint8_t* qs;
  const uint8_t* ks;
  // Key split (the wide hd72 kernel): every (head, query tile) item's key
  // tiles are cut into up to nsplit pieces, one workgroup each; the pieces
  // leave normalised partial outputs in ws_slots, and a second kernel
  // combines them.
  int32_t nsplit;            // 1: no split
  uint8_t* ws_slots;         // [H * ntiles_ub * nsplit] partial records of kSplitSlotBytes
};
// Partial record of one key piece of a 256-query item: O / l as f16
// [256][72], then the reference max m (log2 units) [256] and the row sum l
// [256] as fp32.
constexpr int kSplitQueries = 256;
constexpr size_t kSplitSlotBytes = (size_t)kSplitQueries * 72 * 2 + 2 * kSplitQueries * 4;
// Key split for this problem within a workspace budget: returns the number of
// pieces per item (1: no split) and sets *bytes to the workspace it uses (0
// with no split).
int attn_split_plan(int head_dim, int num_heads, int total_tokens, int num_segments, int max_seqlen,
                    size_t workspace_bytes, size_t* bytes);
// Size of the library-owned split workspace of fp8vit_attn_varlen_noalloc:
// every plan (at most 4 rounds of one piece per CU) fits on up to 269 CUs.
constexpr size_t kNoAllocScratchBytes = (size_t)40 << 20;
// Device address of that workspace on the current device (looked up once per
// device with hipGetSymbolAddress).
hipError_t noalloc_scratch(void** ptr);
// Picks the workgroup shape and sets a.ntiles_ub for it (and the split when
// a.ws_slots is given).
hipError_t launch_attn(const AttnArgs& a, int head_dim, int total_tokens, int max_seqlen, hipStream_t s);
int attn_block_m(int head_dim);

}  // namespace fp8vit
