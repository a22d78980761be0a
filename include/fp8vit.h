/*
 * fp8vit -- FP8 ViT-encoder attention for AMD MI355X (gfx950), C ABI.
 *
 * What the library computes (web sources, cited by page title and section):
 *   - vLLM page "FP8 ViT Encoder Attention", intro and Usage: Q, K and V of a
 *     ViT encoder attention layer are quantized to FP8 immediately before the
 *     attention call, with one scale per tensor; by default the scales are
 *     dynamic, driven by a 16-entry circular buffer of observed Q/K/V amax.
 *   - same page, Calibrate-Once Reuse Workflow and Scale File Format: static
 *     per-layer q/k/v values, saved with a margin (default 1.5), read from a
 *     JSON object keyed by layer name; q_scale/k_scale/v_scale are aliases.
 *   - same page, note on ROCm: packed variable-length image and video batches
 *     are attended natively (segment boundaries in cu_seqlens, no padding).
 *   - atrex-bench operator #025 "per_token_group_quant_fp8", Reference
 *     Implementation: scale = max(amax / 448, 1e-10); code = e4m3fn of
 *     clamp(x_fp32 / scale, -448, 448).
 *
 * Conventions for every entry point:
 *   - Plain pointers and sizes only. "d_" pointers are device memory on the
 *     current HIP device; "stream" is a hipStream_t passed as void* (NULL is
 *     the null stream). The caller owns every buffer and the stream; the
 *     library allocates nothing and keeps no mutable global state (one cached
 *     device-property query per device).
 *   - Launch functions are asynchronous on `stream`. They validate their
 *     arguments on the host before any HIP call and return a status code;
 *     nothing is printed, thrown or aborted. A kernel fault surfaces at the
 *     caller's next synchronisation with that stream.
 *   - One state object must not be used by two streams at the same time.
 *   - Layouts: bf16 and fp8 tensors are [tokens, heads, head_dim] with
 *     head_dim contiguous; bf16 inputs may have a token stride ld >= H*d
 *     (for example views into a fused [T, 3, H, d] QKV buffer).
 */
#ifndef FP8VIT_H
#define FP8VIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp8vit_status {
  FP8VIT_OK = 0,
  FP8VIT_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, bad value */
  FP8VIT_ERR_UNSUPPORTED = 2,      /* head_dim not in {72, 128}, misaligned pointer or stride */
  FP8VIT_ERR_HIP = 3,              /* a HIP runtime call or kernel launch failed */
  FP8VIT_ERR_IO = 4,               /* file could not be opened or read */
  FP8VIT_ERR_PARSE = 5,            /* file is not valid JSON of the expected shape */
  FP8VIT_ERR_NOT_FOUND = 6         /* layer name or q/k/v key absent from the file */
} fp8vit_status;

/* Scaling modes for fp8vit_quantize_qkv. */
#define FP8VIT_DYNAMIC 0 /* amax of this forward pushed into the 16-slot ring */
#define FP8VIT_STATIC 1  /* values set by fp8vit_state_set_static */

#define FP8VIT_RING_SLOTS 16

/* Host snapshot of one layer's scale state (see fp8vit_state_read). */
typedef struct fp8vit_state_view {
  float ring[3][FP8VIT_RING_SLOTS]; /* observed amax of q, k, v; zeros when unused */
  uint32_t count;                   /* dynamic forwards so far (next slot = count % 16) */
  float static_values[3];           /* values given to fp8vit_state_set_static */
  float descale_used[3];            /* descales of the last quantize (or scales_update) */
  float amax_last[3];               /* amax observed by the last dynamic forward */
  uint32_t flags;                   /* reserved: 0 */
} fp8vit_state_view;

/* Bytes of device memory one layer's state needs. The caller allocates it
 * (256-byte aligned) and calls fp8vit_state_init before first use. */
size_t fp8vit_state_bytes(void);

/* Reset a state: empty ring (zeros), count 0, static values 0, descales 0.
 * Asynchronous (a small fill kernel, safe inside graph capture). */
fp8vit_status fp8vit_state_init(void* d_state, void* stream);

/* Host only. Read the static q/k/v values of `layer_name` from the JSON scale
 * file at `json_path` (vLLM page "FP8 ViT Encoder Attention", Scale File
 * Format: {"layer": {"q": .., "k": .., "v": ..}}, with q_scale/k_scale/v_scale
 * accepted as aliases). Values are returned as stored: the calibration margin
 * is already in them. Numbers are parsed as doubles and rounded to float.
 * Errors: ERR_INVALID_ARGUMENT (null argument; a value that is not a finite
 * number > 0; a key given both plainly and as alias), ERR_IO (cannot open or
 * read the file), ERR_PARSE (not JSON, or the layer entry is not an object),
 * ERR_NOT_FOUND (no such layer, or one of q/k/v missing). Unknown keys are
 * ignored; for repeated keys the last occurrence wins. out_qkv is written only
 * on FP8VIT_OK. */
fp8vit_status fp8vit_load_static_scales(const char* json_path, const char* layer_name,
                                        float out_qkv[3]);

/* Store static q/k/v values (as read from the scale file) in the state.
 * Values must be finite and > 0 (else ERR_INVALID_ARGUMENT). Asynchronous:
 * the values travel as kernel arguments, so `values_qkv` may be freed on
 * return. The ring is not touched. */
fp8vit_status fp8vit_state_set_static(void* d_state, const float values_qkv[3], void* stream);

/* Dynamic scale bookkeeping alone (the same device code the fused quantizer
 * runs after its amax pass): push the three amax values at d_amax_qkv
 * (device, float[3], finite and >= 0) into the ring slot count % 16, advance
 * count, and set descale_used[i] = max(fp32(W_i / 448), 1e-10) where W_i is
 * the maximum over all 16 ring slots after the push (vLLM page, Usage: the
 * 16-entry circular buffer of amax values drives the scale update;
 * atrex-bench #025 for the division and the floor). One thread on `stream`. */
fp8vit_status fp8vit_scales_update(void* d_state, const float* d_amax_qkv, void* stream);

/* Quantize Q, K and V to e4m3: one kernel launch in static mode, two in
 * dynamic mode.
 *   q, k, v      bf16 device tensors [total_tokens, num_heads, head_dim] with
 *                token strides ld_q, ld_k, ld_v (elements, >= H*d, multiples
 *                of 8); base pointers 16-byte aligned.
 *   mode         FP8VIT_DYNAMIC: amax of each whole tensor (all tokens, all
 *                heads) is pushed into the ring and the descale comes from the
 *                16-slot window max including this forward (an amax pass,
 *                whose last block does the ring bookkeeping, then the
 *                quantize pass). FP8VIT_STATIC: descale from the
 *                stored static values; no amax pass, ring untouched.
 *   q8, k8, v8   uint8 e4m3fn outputs, contiguous [total_tokens, H, d],
 *                16-byte aligned.
 * Per element: y = x / descale (IEEE fp32 division, nearest), clamped to
 * [-448, 448], rounded to the nearest e4m3 code with ties to even; the sign is
 * kept (a negative value that rounds to zero gives 0x80) (atrex-bench #025,
 * Reference Implementation). descale_used[3] in the state is written with the
 * descales used. total_tokens == 0 is allowed (tensor pointers may then be
 * null; dynamic mode records amax 0). Errors: ERR_INVALID_ARGUMENT (null pointer, negative size, unknown
 * mode, ld < H*d), ERR_UNSUPPORTED (misalignment, H*d not a multiple of 8),
 * ERR_HIP. */
fp8vit_status fp8vit_quantize_qkv(const void* q, const void* k, const void* v,
                                  int64_t ld_q, int64_t ld_k, int64_t ld_v,
                                  int32_t total_tokens, int32_t num_heads, int32_t head_dim,
                                  int32_t mode, void* q8, void* k8, void* v8, void* d_state,
                                  void* stream);

/* Non-causal FP8 flash attention over packed variable-length segments.
 *   q8, k8, v8    e4m3 tensors [total_tokens, H, d] as written by
 *                 fp8vit_quantize_qkv (16-byte aligned).
 *   (with total_tokens == 0 the tensor pointers may be null: nothing to do)
 *   d_cu_seqlens  device int32 [num_segments + 1]: cu[0] = 0, non-decreasing,
 *                 cu[num_segments] = total_tokens. Queries of segment i attend
 *                 to the keys of segment i only (self-attention). Zero-length
 *                 segments are allowed. Not validated on the device.
 *   max_seqlen    >= the longest segment (used to size the launch).
 *   head_dim      72 or 128.
 *   softmax_scale fp32 multiplier of Q K^T; <= 0 selects fp32(1/sqrt(d)).
 *   d_state       descale_used[3] of the last quantize is read on the device.
 *   out           bf16 [total_tokens, H, d], token stride ld_out (elements,
 *                 >= H*d, multiple of 4), 8-byte aligned. Every element of
 *                 every row of every segment is written.
 * O = softmax(Q^ K^T * scale) V^ per segment and head, where Q^ K^ V^ are the
 * dequantized e4m3 tensors. Q^ K^T runs on the FP8 MFMA with fp32
 * accumulation; the probabilities reach the P.V product with more than e4m3
 * precision: rounded once to f16 against V widened exactly to f16 (the
 * kernels for grids that cover the chip), or as two e4m3 terms on the FP8
 * MFMA (the smaller grids). fp32 accumulation throughout.
 * Errors: ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED (also when
 * (total_tokens + 384) * H * d reaches 2^31: the kernel addresses each e4m3
 * tensor with 31-bit offsets), ERR_HIP. */
fp8vit_status fp8vit_attn_varlen(const void* q8, const void* k8, const void* v8,
                                 const int32_t* d_cu_seqlens, int32_t num_segments,
                                 int32_t max_seqlen, int32_t total_tokens, int32_t num_heads,
                                 int32_t head_dim, float softmax_scale, const void* d_state,
                                 void* out, int64_t ld_out, void* stream);

/* fp8vit_attn_varlen with an e4m3 output, to feed an FP8 output projection
 * without a separate quantization pass (the fused fp8-output request on the
 * vLLM issue page "Add support for fused fp8 output to FlashAttention 3").
 *   d_out_descale device fp32[1]: the output's static per-tensor descale s
 *                 (finite, > 0; read on the device, so it may change between
 *                 calls without a host sync).
 *   out8          e4m3 [total_tokens, H, d], token stride ld_out8 (bytes,
 *                 >= H*d, multiple of 4), 4-byte aligned.
 * Each element is the input quantization formula applied to the attention
 * output O as formed in fp32: e4m3 RNE of clamp(fp32(O / s), +-448). Other
 * arguments and errors as fp8vit_attn_varlen (ERR_INVALID_ARGUMENT also for a
 * null d_out_descale). */
fp8vit_status fp8vit_attn_varlen_fp8out(const void* q8, const void* k8, const void* v8,
                                        const int32_t* d_cu_seqlens, int32_t num_segments,
                                        int32_t max_seqlen, int32_t total_tokens, int32_t num_heads,
                                        int32_t head_dim, float softmax_scale, const void* d_state,
                                        const float* d_out_descale, void* out8, int64_t ld_out8,
                                        void* stream);

/* Synchronous read-back of a state for tests and calibration (copies on
 * `stream`, then waits for it). Not for the hot path. */
fp8vit_status fp8vit_state_read(const void* d_state, fp8vit_state_view* out, void* stream);

/* Synchronous write of a whole state, the inverse of fp8vit_state_read: ring,
 * count, static values, last descales, last amax and flags are taken from
 * `in`; the internal atomic-max scratch and arrival counter are cleared as by
 * fp8vit_state_init. With it a calibration or a dynamic ring can be saved and
 * resumed: the forwards that follow behave as they would have in the process
 * that read the state. Ring, static, descale and amax entries must be finite
 * and >= 0 (else ERR_INVALID_ARGUMENT). Copies on `stream` and waits for it,
 * so it is not for graph capture. */
fp8vit_status fp8vit_state_write(void* d_state, const fp8vit_state_view* in, void* stream);

/* Synchronous. The values a calibration saves (vLLM page "FP8 ViT Encoder
 * Attention", Calibrate-Once Reuse Workflow: dynamic scaling over the
 * calibration passes, then the learned values times a margin, default 1.5):
 * out_qkv[i] = fp32(margin * W_i), one fp32 product, where W_i is the maximum
 * over the 16 ring slots of tensor i. Errors: ERR_INVALID_ARGUMENT (null
 * pointer, margin not finite or <= 0, a product that overflows),
 * ERR_NOT_FOUND (a tensor whose ring holds no amax > 0: no dynamic forward has
 * been recorded, or every input was zero), ERR_HIP. out_qkv is written only on
 * FP8VIT_OK. */
fp8vit_status fp8vit_calibrated_values(const void* d_state, float margin, float out_qkv[3], void* stream);

/* Host only. Store one layer's static q/k/v values in the JSON scale file at
 * `json_path` (vLLM page, Scale File Format and Calibrate-Once Reuse Workflow:
 * the file maps layer names to {"q", "k", "v"} values that already include the
 * margin), so that fp8vit_load_static_scales reads back exactly these floats.
 * An existing file keeps its other entries (in order, numbers as written,
 * strings re-escaped, whitespace normalised); an entry named
 * `layer_name` is replaced in place (later duplicates of it are dropped), or
 * appended. A missing or whitespace-only file starts an empty object. The new
 * file is written beside the target and renamed over it. Values are written
 * as the shortest decimal that reads back to the same float. Errors:
 * ERR_INVALID_ARGUMENT (null argument; a value that is not finite and > 0),
 * ERR_PARSE (the existing file is not a JSON object: it is left untouched),
 * ERR_IO (cannot read the existing file, or cannot write or rename). */
fp8vit_status fp8vit_save_static_scales(const char* json_path, const char* layer_name,
                                        const float values_qkv[3]);

/* Static string naming a status code. */
const char* fp8vit_status_str(fp8vit_status status);

#ifdef __cplusplus
}
#endif

#endif /* FP8VIT_H */
