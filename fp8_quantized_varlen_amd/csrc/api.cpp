// C ABI of the library: argument validation, then launches on the caller's stream.
// Every check happens on the host before any HIP call; nothing is allocated.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>

#include "fp8vit.h"
#include "fp8vit_internal.h"

using fp8vit::DevState;

namespace {

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline fp8vit_status from_hip(hipError_t e) { return e == hipSuccess ? FP8VIT_OK : FP8VIT_ERR_HIP; }

}  // namespace

extern "C" {

size_t fp8vit_state_bytes(void) { return sizeof(DevState); }

fp8vit_status fp8vit_state_init(void* d_state, void* stream) {
  if (!d_state) return FP8VIT_ERR_INVALID_ARGUMENT;
  if (!aligned(d_state, 256)) return FP8VIT_ERR_UNSUPPORTED;
  return from_hip(fp8vit::launch_state_init(static_cast<DevState*>(d_state), as_stream(stream)));
}

fp8vit_status fp8vit_state_set_static(void* d_state, const float values_qkv[3], void* stream) {
  if (!d_state || !values_qkv) return FP8VIT_ERR_INVALID_ARGUMENT;
  if (!aligned(d_state, 256)) return FP8VIT_ERR_UNSUPPORTED;
  for (int i = 0; i < 3; ++i)
    if (!std::isfinite(values_qkv[i]) || !(values_qkv[i] > 0.0f)) return FP8VIT_ERR_INVALID_ARGUMENT;
  return from_hip(fp8vit::launch_state_set_static(static_cast<DevState*>(d_state), values_qkv[0], values_qkv[1],
                                                  values_qkv[2], as_stream(stream)));
}

fp8vit_status fp8vit_scales_update(void* d_state, const float* d_amax_qkv, void* stream) {
  if (!d_state || !d_amax_qkv) return FP8VIT_ERR_INVALID_ARGUMENT;
  if (!aligned(d_state, 256) || !aligned(d_amax_qkv, 4)) return FP8VIT_ERR_UNSUPPORTED;
  return from_hip(fp8vit::launch_scales_update(static_cast<DevState*>(d_state), d_amax_qkv, as_stream(stream)));
}

fp8vit_status fp8vit_state_set_flags(void* d_state, uint32_t flags, void* stream) {
  if (!d_state || (flags & ~FP8VIT_FLAG_COUNT_SATURATION) != 0u) return FP8VIT_ERR_INVALID_ARGUMENT;
  if (!aligned(d_state, 256)) return FP8VIT_ERR_UNSUPPORTED;
  return from_hip(fp8vit::launch_state_set_flags(static_cast<DevState*>(d_state), flags, as_stream(stream)));
}

fp8vit_status fp8vit_check_cu_seqlens(const int32_t* d_cu_seqlens, int32_t num_segments, int32_t total_tokens,
                                      int32_t max_seqlen, void* d_state, void* stream) {
  if (!d_cu_seqlens || !d_state || num_segments < 0 || total_tokens < 0 || max_seqlen < 0)
    return FP8VIT_ERR_INVALID_ARGUMENT;
  if (!aligned(d_state, 256) || !aligned(d_cu_seqlens, 4)) return FP8VIT_ERR_UNSUPPORTED;
  return from_hip(fp8vit::launch_check_cu_seqlens(d_cu_seqlens, num_segments, total_tokens, max_seqlen,
                                                  static_cast<DevState*>(d_state), as_stream(stream)));
}

namespace {

// Validation and launch of the per-tensor quantize passes; quant_mask selects
// which of Q, K, V (bits 0, 1, 2) get codes. Dynamic mode's amax and ring
// bookkeeping always cover all three tensors.
fp8vit_status quantize_common(const void* q, const void* k, const void* v, int64_t ld_q, int64_t ld_k, int64_t ld_v,
                              int32_t total_tokens, int32_t num_heads, int32_t head_dim, int32_t mode, void* q8,
                              void* k8, void* v8, void* d_state, uint32_t quant_mask, void* stream) {
  if (!d_state || total_tokens < 0 || num_heads <= 0 || head_dim <= 0) return FP8VIT_ERR_INVALID_ARGUMENT;
  // Empty tensors may come with null data pointers; the kernel then reads nothing.
  if (total_tokens > 0 && (!q || !k || !v || !q8 || !k8 || !v8)) return FP8VIT_ERR_INVALID_ARGUMENT;
  if (mode != FP8VIT_DYNAMIC && mode != FP8VIT_STATIC) return FP8VIT_ERR_INVALID_ARGUMENT;
  const int64_t row = (int64_t)num_heads * head_dim;
  if (ld_q < row || ld_k < row || ld_v < row) return FP8VIT_ERR_INVALID_ARGUMENT;
  if (row % 8 != 0 || ld_q % 8 || ld_k % 8 || ld_v % 8) return FP8VIT_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(q8, 16) || !aligned(k8, 16) ||
      !aligned(v8, 16) || !aligned(d_state, 256))
    return FP8VIT_ERR_UNSUPPORTED;
  // Chunk indices are 32-bit on the device.
  if ((int64_t)total_tokens * (row / 8) >= ((int64_t)1 << 31)) return FP8VIT_ERR_UNSUPPORTED;
  fp8vit::QuantArgs a;
  a.x[0] = static_cast<const uint16_t*>(q);
  a.x[1] = static_cast<const uint16_t*>(k);
  a.x[2] = static_cast<const uint16_t*>(v);
  a.ld[0] = ld_q;
  a.ld[1] = ld_k;
  a.ld[2] = ld_v;
  a.y[0] = static_cast<uint8_t*>(q8);
  a.y[1] = static_cast<uint8_t*>(k8);
  a.y[2] = static_cast<uint8_t*>(v8);
  a.T = total_tokens;
  a.row8 = (int32_t)(row / 8);
  a.amax_blocks = 0;
  a.quant_mask = quant_mask;
  a.st = static_cast<DevState*>(d_state);
  return from_hip(fp8vit::launch_quantize(a, mode == FP8VIT_DYNAMIC, as_stream(stream)));
}

}  // namespace

fp8vit_status fp8vit_quantize_qkv(const void* q, const void* k, const void* v, int64_t ld_q, int64_t ld_k,
                                  int64_t ld_v, int32_t total_tokens, int32_t num_heads, int32_t head_dim,
                                  int32_t mode, void* q8, void* k8, void* v8, void* d_state, void* stream) {
  return quantize_common(q, k, v, ld_q, ld_k, ld_v, total_tokens, num_heads, head_dim, mode, q8, k8, v8, d_state, 7u,
                         stream);
}

fp8vit_status fp8vit_quantize_qkv_mx(const void* q, const void* k, const void* v, int64_t ld_q, int64_t ld_k,
                                     int64_t ld_v, int32_t total_tokens, int32_t num_heads, int32_t head_dim,
                                     int32_t mode, void* q8, void* k8, void* v8, void* q_scales, void* k_scales,
                                     void* d_state, void* stream) {
  if (total_tokens > 0 && (!q_scales || !k_scales)) return FP8VIT_ERR_INVALID_ARGUMENT;
  if (head_dim != 72 && head_dim != 128) return FP8VIT_ERR_UNSUPPORTED;
  if (!aligned(q_scales, 4) || !aligned(k_scales, 4)) return FP8VIT_ERR_UNSUPPORTED;
  // V (and, in dynamic mode, the amax ring of Q, K and V) as fp8vit_quantize_qkv
  // does; Q and K then get the block-scaled codes.
  const fp8vit_status st = quantize_common(q, k, v, ld_q, ld_k, ld_v, total_tokens, num_heads, head_dim, mode, q8,
                                           k8, v8, d_state, 4u, stream);
  if (st != FP8VIT_OK || total_tokens == 0) return st;
  fp8vit::MxArgs m;
  m.x[0] = static_cast<const uint16_t*>(q);
  m.x[1] = static_cast<const uint16_t*>(k);
  m.ld[0] = ld_q;
  m.ld[1] = ld_k;
  m.codes[0] = static_cast<uint8_t*>(q8);
  m.codes[1] = static_cast<uint8_t*>(k8);
  m.scales[0] = static_cast<uint8_t*>(q_scales);
  m.scales[1] = static_cast<uint8_t*>(k_scales);
  m.T = total_tokens;
  m.H = num_heads;
  return from_hip(fp8vit::launch_quantize_mx(m, head_dim, as_stream(stream)));
}

namespace {
// Shared validation and launch of the bf16- and e4m3-output entry points.
fp8vit_status attn_common(const void* q8, const void* k8, const void* v8, const int32_t* d_cu_seqlens,
                          int32_t num_segments, int32_t max_seqlen, int32_t total_tokens, int32_t num_heads,
                          int32_t head_dim, float softmax_scale, const void* d_state, void* out, bool out_fp8,
                          const float* d_out_descale, int64_t ld_out, void* d_workspace, size_t workspace_bytes,
                          bool library_scratch, void* stream, const void* q_scales = nullptr,
                          const void* k_scales = nullptr) {
  if (workspace_bytes > 0 && (!d_workspace || !aligned(d_workspace, 256)))
    return d_workspace ? FP8VIT_ERR_UNSUPPORTED : FP8VIT_ERR_INVALID_ARGUMENT;
  if (!d_cu_seqlens || !d_state) return FP8VIT_ERR_INVALID_ARGUMENT;
  if (out_fp8 && !d_out_descale) return FP8VIT_ERR_INVALID_ARGUMENT;
  if (num_segments < 0 || max_seqlen < 0 || total_tokens < 0 || num_heads <= 0) return FP8VIT_ERR_INVALID_ARGUMENT;
  // Empty tensors may come with null data pointers.
  if (total_tokens > 0 && (!q8 || !k8 || !v8 || !out)) return FP8VIT_ERR_INVALID_ARGUMENT;
  if (head_dim != 72 && head_dim != 128) return FP8VIT_ERR_UNSUPPORTED;
  if (!std::isfinite(softmax_scale)) return FP8VIT_ERR_INVALID_ARGUMENT;
  const int64_t row = (int64_t)num_heads * head_dim;
  if (ld_out < row) return FP8VIT_ERR_INVALID_ARGUMENT;
  if (ld_out % 4) return FP8VIT_ERR_UNSUPPORTED;
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v8, 16) || !aligned(out, out_fp8 ? 4 : 8) ||
      !aligned(d_cu_seqlens, 4) || !aligned(d_state, 256) || (out_fp8 && !aligned(d_out_descale, 4)))
    return FP8VIT_ERR_UNSUPPORTED;
  if (num_segments == 0 || total_tokens == 0 || max_seqlen == 0) return FP8VIT_OK;  // no rows to write
  const int bm = fp8vit::attn_block_m(head_dim);   // the smallest shape: the most tiles
  const int64_t by_total = ((int64_t)total_tokens + bm - 1) / bm + num_segments;
  const int64_t by_max = (int64_t)num_segments * (((int64_t)max_seqlen + bm - 1) / bm);
  const int64_t ntiles = by_total < by_max ? by_total : by_max;
  if (ntiles * num_heads >= ((int64_t)1 << 31)) return FP8VIT_ERR_UNSUPPORTED;
  // The kernel's buffer descriptors address each e4m3 tensor with 31-bit
  // offsets, including up to three tiles read past the end of a segment.
  if (((int64_t)total_tokens + 384) * row >= ((int64_t)1 << 31)) return FP8VIT_ERR_UNSUPPORTED;
  fp8vit::AttnArgs a;
  a.q8 = static_cast<const uint8_t*>(q8);
  a.k8 = static_cast<const uint8_t*>(k8);
  a.v8 = static_cast<const uint8_t*>(v8);
  a.cu = d_cu_seqlens;
  a.nseg = num_segments;
  a.H = num_heads;
  a.ntiles_ub = (int32_t)ntiles;
  a.tensor_bytes = (uint32_t)((int64_t)total_tokens * row);
  a.T = total_tokens;
  a.st = static_cast<const DevState*>(d_state);
  a.out = out_fp8 ? nullptr : static_cast<uint16_t*>(out);
  a.out8 = out_fp8 ? static_cast<uint8_t*>(out) : nullptr;
  a.out_descale = d_out_descale;
  a.ld_out = ld_out;
  a.softmax_scale = softmax_scale > 0.0f ? softmax_scale : (float)(1.0 / std::sqrt((double)head_dim));
  a.qs = static_cast<const uint8_t*>(q_scales);
  a.ks = static_cast<const uint8_t*>(k_scales);
  a.nsplit = 1;
  a.ws_slots = nullptr;
  if (library_scratch) {
    // The library's own workspace: take the plan the caller's workspace would
    // get, and refuse a problem whose plan does not fit.
    size_t need = 0;
    (void)fp8vit::attn_split_plan(head_dim, num_heads, total_tokens, num_segments, max_seqlen, (size_t)-1, &need);
    if (need > fp8vit::kNoAllocScratchBytes) return FP8VIT_ERR_UNSUPPORTED;
    if (need > 0) {
      const hipError_t e = fp8vit::noalloc_scratch(&d_workspace);
      if (e != hipSuccess) return FP8VIT_ERR_HIP;
      workspace_bytes = fp8vit::kNoAllocScratchBytes;
    }
  }
  if (workspace_bytes > 0) {
    size_t need = 0;
    const int sp = fp8vit::attn_split_plan(head_dim, num_heads, total_tokens, num_segments, max_seqlen,
                                           workspace_bytes, &need);
    if (sp > 1) {
      a.nsplit = sp;
      a.ws_slots = static_cast<uint8_t*>(d_workspace);
    }
  }
  return from_hip(fp8vit::launch_attn(a, head_dim, total_tokens, max_seqlen, as_stream(stream)));
}
}  // namespace

fp8vit_status fp8vit_attn_varlen(const void* q8, const void* k8, const void* v8, const int32_t* d_cu_seqlens,
                                 int32_t num_segments, int32_t max_seqlen, int32_t total_tokens, int32_t num_heads,
                                 int32_t head_dim, float softmax_scale, const void* d_state, void* out,
                                 int64_t ld_out, void* stream) {
  return attn_common(q8, k8, v8, d_cu_seqlens, num_segments, max_seqlen, total_tokens, num_heads, head_dim,
                     softmax_scale, d_state, out, false, nullptr, ld_out, nullptr, 0, false, stream);
}

size_t fp8vit_attn_workspace_bytes(int32_t num_segments, int32_t max_seqlen, int32_t total_tokens,
                                   int32_t num_heads, int32_t head_dim) {
  if (num_segments <= 0 || max_seqlen <= 0 || total_tokens <= 0 || num_heads <= 0) return 0;
  size_t need = 0;
  (void)fp8vit::attn_split_plan(head_dim, num_heads, total_tokens, num_segments, max_seqlen, (size_t)-1, &need);
  return need;
}

fp8vit_status fp8vit_attn_varlen_ws(const void* q8, const void* k8, const void* v8, const int32_t* d_cu_seqlens,
                                    int32_t num_segments, int32_t max_seqlen, int32_t total_tokens,
                                    int32_t num_heads, int32_t head_dim, float softmax_scale, const void* d_state,
                                    void* out, int64_t ld_out, void* d_workspace, size_t workspace_bytes,
                                    void* stream) {
  return attn_common(q8, k8, v8, d_cu_seqlens, num_segments, max_seqlen, total_tokens, num_heads, head_dim,
                     softmax_scale, d_state, out, false, nullptr, ld_out, d_workspace, workspace_bytes, false,
                     stream);
}

fp8vit_status fp8vit_attn_varlen_noalloc(const void* q8, const void* k8, const void* v8,
                                         const int32_t* d_cu_seqlens, int32_t num_segments, int32_t max_seqlen,
                                         int32_t total_tokens, int32_t num_heads, int32_t head_dim,
                                         float softmax_scale, const void* d_state, void* out, int64_t ld_out,
                                         void* stream) {
  return attn_common(q8, k8, v8, d_cu_seqlens, num_segments, max_seqlen, total_tokens, num_heads, head_dim,
                     softmax_scale, d_state, out, false, nullptr, ld_out, nullptr, 0, true, stream);
}

fp8vit_status fp8vit_attn_varlen_mx(const void* q8, const void* k8, const void* v8, const void* d_q_scales,
                                    const void* d_k_scales, const int32_t* d_cu_seqlens, int32_t num_segments,
                                    int32_t max_seqlen, int32_t total_tokens, int32_t num_heads, int32_t head_dim,
                                    float softmax_scale, const void* d_state, void* out, int64_t ld_out,
                                    void* stream) {
  if (total_tokens > 0 && num_segments > 0 && (!d_q_scales || !d_k_scales)) return FP8VIT_ERR_INVALID_ARGUMENT;
  if (!aligned(d_q_scales, 4) || !aligned(d_k_scales, 4)) return FP8VIT_ERR_UNSUPPORTED;
  // Empty problems return before any launch; otherwise the non-null scales
  // select the block-scaled kernels. The (T + 2 tiles) * H scale dwords stay
  // far below the 31-bit offsets the code tensors are bounded by.
  return attn_common(q8, k8, v8, d_cu_seqlens, num_segments, max_seqlen, total_tokens, num_heads, head_dim,
                     softmax_scale, d_state, out, false, nullptr, ld_out, nullptr, 0, false, stream, d_q_scales,
                     d_k_scales);
}

fp8vit_status fp8vit_attn_varlen_fp8out(const void* q8, const void* k8, const void* v8,
                                        const int32_t* d_cu_seqlens, int32_t num_segments, int32_t max_seqlen,
                                        int32_t total_tokens, int32_t num_heads, int32_t head_dim,
                                        float softmax_scale, const void* d_state, const float* d_out_descale,
                                        void* out8, int64_t ld_out8, void* stream) {
  return attn_common(q8, k8, v8, d_cu_seqlens, num_segments, max_seqlen, total_tokens, num_heads, head_dim,
                     softmax_scale, d_state, out8, true, d_out_descale, ld_out8, nullptr, 0, false, stream);
}

fp8vit_status fp8vit_state_read(const void* d_state, fp8vit_state_view* out, void* stream) {
  if (!d_state || !out) return FP8VIT_ERR_INVALID_ARGUMENT;
  if (!aligned(d_state, 256)) return FP8VIT_ERR_UNSUPPORTED;
  DevState h;
  hipError_t e = hipMemcpyAsync(&h, d_state, fp8vit::kStateViewBytes, hipMemcpyDeviceToHost, as_stream(stream));
  if (e != hipSuccess) return FP8VIT_ERR_HIP;
  e = hipStreamSynchronize(as_stream(stream));
  if (e != hipSuccess) return FP8VIT_ERR_HIP;
  std::memcpy(out->ring, h.ring, sizeof(out->ring));
  out->count = h.count;
  // The last dynamic forward's amax may still be pending: report the ring as
  // it is once pushed (what the next dynamic forward's pass 2 does on the device).
  if (h.pending != 0u) {
    for (int x = 0; x < 3; ++x) out->ring[x][h.count % FP8VIT_RING_SLOTS] = h.pending_amax[x];
    out->count = h.count + 1;
  }
  for (int i = 0; i < 3; ++i) {
    out->static_values[i] = h.static_values[i];
    out->descale_used[i] = h.descale_used[i];
    out->amax_last[i] = h.amax_last[i];
  }
  out->flags = h.flags;
  out->cu_check = h.cu_check;
  for (int i = 0; i < 3; ++i) out->saturated[i] = h.saturated[i];
  return FP8VIT_OK;
}

fp8vit_status fp8vit_state_write(void* d_state, const fp8vit_state_view* in, void* stream) {
  if (!d_state || !in) return FP8VIT_ERR_INVALID_ARGUMENT;
  if (!aligned(d_state, 256)) return FP8VIT_ERR_UNSUPPORTED;
  if ((in->flags & ~FP8VIT_FLAG_COUNT_SATURATION) != 0u) return FP8VIT_ERR_INVALID_ARGUMENT;
  auto nonneg = [](float x) { return std::isfinite(x) && x >= 0.0f; };
  for (int x = 0; x < 3; ++x) {
    for (int i = 0; i < FP8VIT_RING_SLOTS; ++i)
      if (!nonneg(in->ring[x][i])) return FP8VIT_ERR_INVALID_ARGUMENT;
    if (!nonneg(in->static_values[x]) || !nonneg(in->descale_used[x]) || !nonneg(in->amax_last[x]))
      return FP8VIT_ERR_INVALID_ARGUMENT;
  }
  // No push is pending, and the partial maxima start from zero, as after
  // fp8vit_state_init.
  static_assert(sizeof(DevState) <= 65536, "state copied through the stack");
  DevState h;
  std::memset(&h, 0, sizeof(h));
  std::memcpy(h.ring, in->ring, sizeof(h.ring));
  h.count = in->count;
  for (int i = 0; i < 3; ++i) {
    h.static_values[i] = in->static_values[i];
    h.descale_used[i] = in->descale_used[i];
    h.amax_last[i] = in->amax_last[i];
  }
  h.flags = in->flags;
  h.cu_check = in->cu_check;
  for (int i = 0; i < 3; ++i) h.saturated[i] = in->saturated[i];
  hipError_t e = hipMemcpyAsync(d_state, &h, sizeof(DevState), hipMemcpyHostToDevice, as_stream(stream));
  if (e != hipSuccess) return FP8VIT_ERR_HIP;
  // `h` lives on this stack frame: wait for the copy before returning.
  return from_hip(hipStreamSynchronize(as_stream(stream)));
}

fp8vit_status fp8vit_calibrated_values(const void* d_state, float margin, float out_qkv[3], void* stream) {
  if (!d_state || !out_qkv) return FP8VIT_ERR_INVALID_ARGUMENT;
  if (!std::isfinite(margin) || !(margin > 0.0f)) return FP8VIT_ERR_INVALID_ARGUMENT;
  fp8vit_state_view v;
  const fp8vit_status st = fp8vit_state_read(d_state, &v, stream);
  if (st != FP8VIT_OK) return st;
  float vals[3];
  for (int x = 0; x < 3; ++x) {
    float w = 0.0f;
    for (int i = 0; i < FP8VIT_RING_SLOTS; ++i) w = v.ring[x][i] > w ? v.ring[x][i] : w;
    vals[x] = margin * w;  // one fp32 product
    if (!(vals[x] > 0.0f)) return FP8VIT_ERR_NOT_FOUND;
    if (!std::isfinite(vals[x])) return FP8VIT_ERR_INVALID_ARGUMENT;
  }
  for (int i = 0; i < 3; ++i) out_qkv[i] = vals[i];
  return FP8VIT_OK;
}

const char* fp8vit_status_str(fp8vit_status status) {
  switch (status) {
    case FP8VIT_OK: return "ok";
    case FP8VIT_ERR_INVALID_ARGUMENT: return "invalid argument";
    case FP8VIT_ERR_UNSUPPORTED: return "unsupported (head_dim, alignment or size)";
    case FP8VIT_ERR_HIP: return "HIP runtime error";
    case FP8VIT_ERR_IO: return "file could not be read";
    case FP8VIT_ERR_PARSE: return "malformed scale file";
    case FP8VIT_ERR_NOT_FOUND: return "layer or key not found";
  }
  return "unknown status";
}

}  // extern "C"
