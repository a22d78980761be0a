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

/* Option bits of a state (fp8vit_state_set_flags). */
#define FP8VIT_FLAG_COUNT_SATURATION 1u /* quantize passes count clamped elements */

/* Bits of fp8vit_state_view.cu_check (fp8vit_check_cu_seqlens). */
#define FP8VIT_CU_FIRST_NOT_ZERO 1u   /* cu_seqlens[0] != 0 */
#define FP8VIT_CU_DECREASING 2u       /* cu_seqlens[i+1] < cu_seqlens[i] for some i */
#define FP8VIT_CU_LAST_NOT_T 4u       /* cu_seqlens[num_segments] != total_tokens */
#define FP8VIT_CU_LONGER_THAN_MAX 8u  /* a segment longer than max_seqlen */

/* Host snapshot of one layer's scale state (see fp8vit_state_read). */
typedef struct fp8vit_state_view {
  float ring[3][FP8VIT_RING_SLOTS]; /* observed amax of q, k, v; zeros when unused */
  uint32_t count;                   /* dynamic forwards so far (next slot = count % 16) */
  float static_values[3];           /* values given to fp8vit_state_set_static */
  float descale_used[3];            /* descales of the last quantize (or scales_update) */
  float amax_last[3];               /* amax observed by the last dynamic forward */
  uint32_t flags;                   /* FP8VIT_FLAG_* bits; 0 after fp8vit_state_init */
  uint32_t cu_check;                /* FP8VIT_CU_* bits of the last fp8vit_check_cu_seqlens */
  uint64_t saturated[3];            /* q, k, v elements clamped at +-448 since the flag was set */
} fp8vit_state_view;

/* Bytes of device memory one layer's state needs. The caller allocates it
 * (256-byte aligned) and calls fp8vit_state_init before first use. The state
 * holds the 16-slot amax ring and count, the static values, the descales in
 * use and the first dynamic pass's per-block partials (33,280 bytes).
 * Source: vLLM page "FP8 ViT Encoder Attention", Usage (a 16-entry circular
 * buffer of observed Q/K/V amax drives each forward's scale) and Scale File
 * Format (per-layer static q/k/v values). */
size_t fp8vit_state_bytes(void);

/* Reset a state: empty ring (zeros), count 0, static values 0, descales 0.
 * Asynchronous (a small fill kernel, safe inside graph capture).
 * Errors: ERR_INVALID_ARGUMENT (null), ERR_UNSUPPORTED (not 256-byte
 * aligned), ERR_HIP.
 * Source: vLLM page "FP8 ViT Encoder Attention", Usage (dynamic scaling with
 * no scale file starts from an empty amax ring). */
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
 * on FP8VIT_OK.
 * Source: vLLM page "FP8 ViT Encoder Attention", Scale File Format (layer ->
 * {"q", "k", "v"}; q_scale/k_scale/v_scale aliases) and Calibrate-Once Reuse
 * Workflow (the saved values already carry the margin). */
fp8vit_status fp8vit_load_static_scales(const char* json_path, const char* layer_name,
                                        float out_qkv[3]);

/* Store static q/k/v values (as read from the scale file) in the state.
 * Values must be finite and > 0 (else ERR_INVALID_ARGUMENT). Asynchronous:
 * the values travel as kernel arguments, so `values_qkv` may be freed on
 * return. The ring is not touched. A later FP8VIT_STATIC quantize uses
 * descale = max(fp32(value / 448), 1e-10).
 * Source: vLLM page "FP8 ViT Encoder Attention", Calibrate-Once Reuse
 * Workflow, step 2 (serve with static scales: no dynamic overhead). */
fp8vit_status fp8vit_state_set_static(void* d_state, const float values_qkv[3], void* stream);

/* Dynamic scale bookkeeping alone (what the dynamic quantizer's second pass
 * does, as a call of its own): push the three amax values at d_amax_qkv
 * (device, float[3], finite and >= 0) into the ring slot count % 16, advance
 * count, and set descale_used[i] = max(fp32(W_i / 448), 1e-10) where W_i is
 * the maximum over all 16 ring slots after the push (vLLM page, Usage: the
 * 16-entry circular buffer of amax values drives the scale update;
 * atrex-bench #025 for the division and the floor). One thread on `stream`.
 * Errors: ERR_INVALID_ARGUMENT (null), ERR_UNSUPPORTED (misaligned), ERR_HIP.
 * Source: vLLM page "FP8 ViT Encoder Attention", Usage; atrex-bench operator
 * #025 "per_token_group_quant_fp8", Reference Implementation. */
fp8vit_status fp8vit_scales_update(void* d_state, const float* d_amax_qkv, void* stream);

/* Set the option bits of a state (FP8VIT_FLAG_*; other bits:
 * ERR_INVALID_ARGUMENT) and restart the saturation counts from zero.
 * With FP8VIT_FLAG_COUNT_SATURATION, every per-tensor quantize pass (of
 * fp8vit_quantize_qkv, and the V pass of fp8vit_quantize_qkv_mx) adds to
 * saturated[q, k, v] the number of elements whose fp32 quotient x / descale
 * is larger than 448 in magnitude, i.e. the elements the clamp changes (one
 * 64-bit atomic add per workgroup and tensor); without it the passes do not
 * count. Block-scaled Q and K never clamp (their block scale is at least the
 * block amax / 448). Asynchronous, one small kernel.
 * Errors: ERR_INVALID_ARGUMENT (null state, unknown bits), ERR_UNSUPPORTED
 * (state not 256-byte aligned), ERR_HIP.
 * Source: vLLM page "FP8 ViT Encoder Attention", Calibrate-Once Reuse
 * Workflow (the saved values carry a margin that leaves headroom for
 * activations beyond the calibration maximum; the count shows when it does
 * not). */
fp8vit_status fp8vit_state_set_flags(void* d_state, uint32_t flags, void* stream);

/* Check a packed batch description on the device and write the FP8VIT_CU_*
 * bits of the conditions it violates (0 when valid) into the state's
 * cu_check, which fp8vit_state_read reports. d_cu_seqlens: num_segments + 1
 * int32 entries (device). The attention kernels themselves clamp every
 * segment to [0, total_tokens], so an invalid cu_seqlens gives unspecified
 * output rows but no access outside the tensors; this check is the way to
 * tell. Asynchronous, one workgroup.
 * Errors: ERR_INVALID_ARGUMENT (null pointer, num_segments, total_tokens or
 * max_seqlen < 0), ERR_UNSUPPORTED (state not 256-byte aligned), ERR_HIP.
 * Source: vLLM page "FP8 ViT Encoder Attention", note on ROCm (packed
 * variable-length batches described by cumulative segment boundaries). */
fp8vit_status fp8vit_check_cu_seqlens(const int32_t* d_cu_seqlens, int32_t num_segments, int32_t total_tokens,
                                      int32_t max_seqlen, void* d_state, void* stream);

/* Quantize Q, K and V to e4m3: one kernel launch in static mode, two in
 * dynamic mode.
 *   q, k, v      bf16 device tensors [total_tokens, num_heads, head_dim] with
 *                token strides ld_q, ld_k, ld_v (elements, >= H*d, multiples
 *                of 8); base pointers 16-byte aligned.
 *   mode         FP8VIT_DYNAMIC: amax of each whole tensor (all tokens, all
 *                heads) is pushed into the ring and the descale comes from the
 *                16-slot window max including this forward. Pass 1 quantizes
 *                at the descale of the other 15 slots while it reduces the
 *                amax; pass 2 does the ring bookkeeping and quantizes a
 *                tensor again only if its amax changed that descale (the
 *                first forward, and in steady state about one forward in
 *                16), so the codes are those of the window including this
 *                forward in every case. FP8VIT_STATIC: descale from the
 *                stored static values; no amax, ring untouched.
 *   q8, k8, v8   uint8 e4m3fn outputs, contiguous [total_tokens, H, d],
 *                16-byte aligned.
 * Per element: y = x / descale (IEEE fp32 division, nearest), clamped to
 * [-448, 448], rounded to the nearest e4m3 code with ties to even; the sign is
 * kept (a negative value that rounds to zero gives 0x80) (atrex-bench #025,
 * Reference Implementation). descale_used[3] in the state is written with the
 * descales used. total_tokens == 0 is allowed (tensor pointers may then be
 * null; dynamic mode records amax 0). Dynamic mode is two launches, not one:
 * the pages ask only that Q, K and V be quantized right before the attention
 * call, and a single cooperative launch with a grid-wide barrier measured
 * slower on MI355X at every size; in the usual case the second launch reads
 * only the first one's per-block maxima.
 * Errors: ERR_INVALID_ARGUMENT (null pointer, negative size, unknown mode,
 * ld < H*d), ERR_UNSUPPORTED (misalignment, H*d not a multiple of 8, or
 * total_tokens * H * d / 8 >= 2^31), ERR_HIP.
 * Source: vLLM page "FP8 ViT Encoder Attention", introduction (Q/K/V are
 * quantized to FP8 on the fly just before the attention call) and Usage
 * (dynamic scaling); atrex-bench operator #025 "per_token_group_quant_fp8",
 * Reference Implementation (scale, division, clamp, e4m3fn cast). */
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
 * tensor with 31-bit offsets), ERR_HIP.
 * Source: vLLM page "FP8 ViT Encoder Attention", Requirements (a varlen
 * FP8 attention call with one scale per tensor) and the note on ROCm (packed
 * variable-length image and video batches attended natively). */
fp8vit_status fp8vit_attn_varlen(const void* q8, const void* k8, const void* v8,
                                 const int32_t* d_cu_seqlens, int32_t num_segments,
                                 int32_t max_seqlen, int32_t total_tokens, int32_t num_heads,
                                 int32_t head_dim, float softmax_scale, const void* d_state,
                                 void* out, int64_t ld_out, void* stream);

/* Bytes of workspace fp8vit_attn_varlen_ws uses for this problem on the
 * current device; 0 when it would not split the keys (the grid already fills
 * the GPU or splitting would not pay, head_dim is 128, or the problem is
 * empty). Host only; a device property query, no launch.
 * Source: vLLM page "FP8 ViT Encoder Attention", Performance (the MI300X
 * AITER table's sequence lengths: at 16 heads and head_dim 72 a short
 * sequence gives fewer (head, query tile) items than the GPU has CUs). */
size_t fp8vit_attn_workspace_bytes(int32_t num_segments, int32_t max_seqlen, int32_t total_tokens,
                                   int32_t num_heads, int32_t head_dim);

/* fp8vit_attn_varlen with a caller workspace that lets the kernel split the
 * keys when the grid of (head, 256-query tile) items is too small to fill the
 * GPU (head_dim 72; for example L = 4096 at 8 heads gives 128 items for 256
 * CUs). Each item's key tiles are cut into equal pieces, one workgroup each;
 * the pieces write normalised partial outputs (O / l as f16, with m and l as
 * fp32) to the workspace, and a second kernel on the same stream combines
 * them in piece order: O = sum_p w_p O_p / sum_p w_p with
 * w_p = l_p 2^(m_p - max m). The split is taken only where a cost model of
 * the kernel (measured on MI355X) predicts a gain of more than 10 %; elsewhere
 * this call is fp8vit_attn_varlen, bit for bit. The result is deterministic
 * and invariant under segment permutation, and agrees with fp8vit_attn_varlen
 * within the attention tolerance (not bitwise: the partials are rounded to
 * f16).
 *   d_workspace      device buffer, 256-byte aligned, of workspace_bytes
 *                    bytes; its contents need no initialisation. Calls that
 *                    share a workspace must not overlap.
 *   workspace_bytes  its size. With less than fp8vit_attn_workspace_bytes()
 *                    the call splits less or not at all; 0 (d_workspace may
 *                    then be NULL) is fp8vit_attn_varlen.
 * Other arguments, layout and errors as fp8vit_attn_varlen (also
 * ERR_INVALID_ARGUMENT for a NULL workspace with workspace_bytes > 0, and
 * ERR_UNSUPPORTED for a misaligned one).
 * Source: vLLM page "FP8 ViT Encoder Attention", Requirements (varlen FP8
 * attention with one scale per tensor) and Performance (the MI300X AITER
 * table's sequence lengths, where smaller images give fewer query tiles). */
fp8vit_status fp8vit_attn_varlen_ws(const void* q8, const void* k8, const void* v8,
                                    const int32_t* d_cu_seqlens, int32_t num_segments,
                                    int32_t max_seqlen, int32_t total_tokens, int32_t num_heads,
                                    int32_t head_dim, float softmax_scale, const void* d_state,
                                    void* out, int64_t ld_out, void* d_workspace,
                                    size_t workspace_bytes, void* stream);

/* fp8vit_attn_varlen_ws for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the key split's workspace is the library's own, a 40 MiB
 * static device array per GPU that each GPU the library runs on holds until
 * the process ends. The call itself allocates nothing (no hipMalloc, no
 * allocating library routine); the first call on a device looks the array's
 * address up once. The split plan, kernels and result are those of
 * fp8vit_attn_varlen_ws with a workspace of fp8vit_attn_workspace_bytes();
 * the array needs no initial contents and keeps the last call's partials.
 * All calls on one GPU share the array: calls that overlap on one GPU (two
 * streams, two threads) race and must be serialised by the caller.
 * Arguments, layout and errors as fp8vit_attn_varlen, and ERR_UNSUPPORTED when
 * the split this problem would take needs more than the 40 MiB (at most four
 * rounds of one piece per CU: never on GPUs of up to 269 CUs).
 * Source: for callers that cannot allocate (no page defines this entry). */
fp8vit_status fp8vit_attn_varlen_noalloc(const void* q8, const void* k8, const void* v8,
                                         const int32_t* d_cu_seqlens, int32_t num_segments,
                                         int32_t max_seqlen, int32_t total_tokens, int32_t num_heads,
                                         int32_t head_dim, float softmax_scale, const void* d_state,
                                         void* out, int64_t ld_out, void* stream);

/* Block-scaled ("MX") variant of fp8vit_quantize_qkv: Q and K get one
 * power-of-two scale per 32-element block of head_dim instead of one per
 * tensor; V is quantized exactly as by fp8vit_quantize_qkv (per-tensor scale
 * from `mode`; in dynamic mode the amax ring of Q, K and V is kept as there).
 *   q8, k8        e4m3 codes [T, H, d] (16-byte aligned): code of
 *                 clamp(x / 2^s_b, +-448), nearest-even, where s_b is the
 *                 block's scale exponent (the product x * 2^-s_b is exact).
 *   q_scales,
 *   k_scales      uint8 [T, H, 4] (4-byte aligned): byte b is the E8M0 scale
 *                 (s_b + 127) of block b = elements 32b .. min(d, 32b + 32);
 *                 head_dim 72 has three blocks (the third of 8 elements) and
 *                 byte 3 = 0; head_dim 128 has four.
 *   s_b          the smallest integer with 448 * 2^s_b >= the block's amax
 *                 (so no element saturates), -127 for a block of zeros.
 * v8, state, mode, strides, alignment and errors as fp8vit_quantize_qkv, and
 * ERR_UNSUPPORTED for head_dim other than 72 or 128. Two launches in static
 * mode (V; then Q and K together), three in dynamic mode (V's two passes,
 * which also take the amax of Q and K for the ring; then Q and K).
 * Source: FlashInfer PR 5283 analysis ("experimental NVFP4 attention"), Code
 * analysis section 1 (a scale per block of the head dimension from the block
 * amax over the element format's largest value); PR 3684 analysis
 * ("asymmetric VO-split NVFP4"), section 3 (one scale factor per block). */
fp8vit_status fp8vit_quantize_qkv_mx(const void* q, const void* k, const void* v,
                                     int64_t ld_q, int64_t ld_k, int64_t ld_v,
                                     int32_t total_tokens, int32_t num_heads, int32_t head_dim,
                                     int32_t mode, void* q8, void* k8, void* v8, void* q_scales,
                                     void* k_scales, void* d_state, void* stream);

/* fp8vit_attn_varlen for block-scaled Q and K (as written by
 * fp8vit_quantize_qkv_mx): S = Q^ K^T with each 32-element block of Q and K
 * dequantized by its own power-of-two scale, applied by the gfx950 matrix
 * core (v_mfma_scale_f32_16x16x128_f8f6f4, which takes one E8M0 byte per
 * operand row and 32-element block); V uses the per-tensor descale in d_state.
 * Runs the kernel shapes fp8vit_attn_varlen chooses, with no key split
 * (head_dim 72 wide: v_mfma_scale_f32_32x32x64_f8f6f4 for d 0..63; d 64..71
 * as the exact bf16 values code * 2^(s_b) on the 32x32x16 bf16 product, where
 * a block scale byte of 0 counts as scale 0 and so drops only values below
 * 448 * 2^-127). bf16 output only. Arguments, layout and errors as
 * fp8vit_attn_varlen, with d_q_scales and d_k_scales
 * the [T, H, 4] scale bytes (device, 4-byte aligned, non-null unless the
 * problem is empty).
 * Source: FlashInfer PR 5283 analysis, Code analysis section 1 (attention on
 * block-scaled Q and K); vLLM page "FP8 ViT Encoder Attention", Requirements
 * (varlen FP8 attention). */
fp8vit_status fp8vit_attn_varlen_mx(const void* q8, const void* k8, const void* v8,
                                    const void* d_q_scales, const void* d_k_scales,
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
 * null d_out_descale).
 * Source: vLLM issue 29920 "Add support for fused fp8 output to
 * FlashAttention 3" (attention writing FP8 for the next FP8 GEMM); the
 * formula is atrex-bench operator #025, Reference Implementation. */
fp8vit_status fp8vit_attn_varlen_fp8out(const void* q8, const void* k8, const void* v8,
                                        const int32_t* d_cu_seqlens, int32_t num_segments,
                                        int32_t max_seqlen, int32_t total_tokens, int32_t num_heads,
                                        int32_t head_dim, float softmax_scale, const void* d_state,
                                        const float* d_out_descale, void* out8, int64_t ld_out8,
                                        void* stream);

/* Synchronous read-back of a state for tests and calibration (copies on
 * `stream`, then waits for it). Not for the hot path.
 * Errors: ERR_INVALID_ARGUMENT (null), ERR_UNSUPPORTED (misaligned), ERR_HIP.
 * Source: vLLM page "FP8 ViT Encoder Attention", Calibrate-Once Reuse
 * Workflow, step 1 (the scales learned by dynamic scaling are read out and
 * dumped). */
fp8vit_status fp8vit_state_read(const void* d_state, fp8vit_state_view* out, void* stream);

/* Synchronous write of a whole state, the inverse of fp8vit_state_read: ring,
 * count, static values, last descales, last amax, flags, cu_check and the
 * saturation counts are taken from `in`; dynamic pass 1's partials are
 * cleared as by fp8vit_state_init, and no push is pending (a view from
 * fp8vit_state_read already has a pending push applied). With it a
 * calibration or a dynamic ring can be saved and resumed: the forwards that
 * follow behave as they would have in the process that read the state. Ring,
 * static, descale and amax entries must be finite and >= 0, and flags only
 * FP8VIT_FLAG_* bits (else ERR_INVALID_ARGUMENT). Copies on `stream` and
 * waits for it, so it is not for graph capture.
 * Source: vLLM page "FP8 ViT Encoder Attention", Usage (the ring carries over
 * from forward to forward, so resuming it needs its whole contents). */
fp8vit_status fp8vit_state_write(void* d_state, const fp8vit_state_view* in, void* stream);

/* Synchronous. The values a calibration saves (vLLM page "FP8 ViT Encoder
 * Attention", Calibrate-Once Reuse Workflow: dynamic scaling over the
 * calibration passes, then the learned values times a margin, default 1.5):
 * out_qkv[i] = fp32(margin * W_i), one fp32 product, where W_i is the maximum
 * over the 16 ring slots of tensor i. Errors: ERR_INVALID_ARGUMENT (null
 * pointer, margin not finite or <= 0, a product that overflows),
 * ERR_NOT_FOUND (a tensor whose ring holds no amax > 0: no dynamic forward has
 * been recorded, or every input was zero), ERR_HIP. out_qkv is written only on
 * FP8VIT_OK.
 * Source: vLLM page "FP8 ViT Encoder Attention", Calibrate-Once Reuse
 * Workflow (16 dynamic passes, learned scales times the save margin). */
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
 * ERR_IO (cannot read the existing file, or cannot write or rename).
 * Source: vLLM page "FP8 ViT Encoder Attention", Scale File Format and
 * Calibrate-Once Reuse Workflow, step 1 (dump the learned scales to JSON). */
fp8vit_status fp8vit_save_static_scales(const char* json_path, const char* layer_name,
                                        const float values_qkv[3]);

/* Static string naming a status code; never NULL (unknown codes give
 * "unknown status").
 * Source: the failure cases of the calls above; the file errors (IO, PARSE,
 * NOT_FOUND) are those of reading the vLLM page's Scale File Format. */
const char* fp8vit_status_str(fp8vit_status status);

#ifdef __cplusplus
}
#endif

#endif /* FP8VIT_H */
