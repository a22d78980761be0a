// Varlen non-causal FP8 flash attention for gfx950 (CDNA4).
//
// What it computes (vLLM page "FP8 ViT Encoder Attention": FP8 Q/K/V with one
// scale per tensor; packed variable-length image/video batches handled
// natively): for every segment [cu[i], cu[i+1]) and head h,
//     O = softmax(dq*dk*scale * Q8 K8^T) (dv * V8),
// with Q8/K8/V8 the e4m3 codes and dq/dk/dv the per-tensor descales.
//
// Design (MI355X-first, not a port of any kernel on the pages):
//  * A workgroup owns BM = 16*QB*WAVES queries of one (segment, head); each
//    wave owns 16*QB of them and runs over every key of the segment.
//  * K/V tiles of 128 keys go global -> LDS by the buffer-load LDS DMA
//    (buffer_load_dwordx4 ... lds): no staging registers, no LDS store
//    instructions, issued a whole iteration before the tile is needed and
//    bounds-checked by the buffer descriptor (reads past the tensor give 0).
//  * S^T = K Q^T on v_mfma_f32_16x16x128_f8f6f4 (K rows as the A operand, Q as
//    B), d zero-padded to 128 for head_dim 72. A rows are permuted so that lane
//    group g holds keys 32g..32g+31 of its query: the fp32 S^T registers turn
//    in place into the B operand of the P.V product (no LDS round trip).
//  * O^T = V^T P^T on the same MFMA; V^T comes from row-major V in LDS through
//    ds_read_b64_tr_b8 (byte transpose on read). The A operand row of column
//    72 (hd72) is replaced by 1.0 in registers, and hd128 appends a constant
//    ones block, so the same MFMAs accumulate the row sum of the
//    probabilities actually used.
//  * Software pipeline over key tiles: iteration j holds the whole S(j) tile
//    in registers, so its maximum is known before any probability is formed;
//    S(j+1) and the previous tile's P(j-1).V(j-1) run on the matrix core while
//    the VALU forms P(j). Lazy reference max m_ref: P~ = 2^7 * exp2(t - m_ref)
//    and m_ref moves only when a score exceeds m_ref + 1.75 (P~ could then pass
//    448, e4m3's largest value); O is rescaled at the end of that iteration.
//  * P~ needs more than e4m3 precision (a single e4m3 term adds ~2.5%
//    relative error to O). The wide shapes round it once to f16 and run P.V
//    on the f16 MFMA against V widened (exactly) into an f16 copy in LDS; the
//    narrow shapes give the FP8 MFMA two e4m3 terms, hi = e4m3(P~) and
//    lo = e4m3(P~ - hi). The wide hd72 kernel (attn_w32_kernel) works on
//    32x32 MFMA blocks, so that d = 72 costs 80 columns of S = K Q^T work
//    instead of 128.
//  * Work items are (head, query tile); consecutive items of one head are
//    mapped to the same XCD so that K/V re-reads hit that XCD's L2.
#include <atomic>
#include <type_traits>

#include "fp8vit_internal.h"

namespace fp8vit {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) v4i lds_v4i;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBN = 128;             // keys per tile
constexpr float kExpBias = 7.0f;     // P~ = 2^7 * exp2(t - m_ref)
constexpr float kLazy = 1.75f;       // log2 growth of the max tolerated before rescaling
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format

template <int D> struct Cfg;
// KS/VS: LDS row strides of K and V tiles in bytes (multiples of 16: the DMA
// moves 16-byte chunks, so a row holds the head's D bytes followed by the
// first bytes of the next head; those only ever meet zero Q bytes or
// discarded O columns). KOP: K is stored in operand order instead of rows
// (see the K placement below; hd128: +6 %, hd72: -1.5 % for 60 % more DMA).
// NCB: 16-column blocks of O^T including the ones column. VH_COLS: columns of
// the f16 copy of V (the wide hd128 shape; no hd72 shape of attn_kernel
// widens V).
template <> struct Cfg<72> {
  static constexpr int KS = 80, VS = 80, NCB = 5, ONES_CB = 4, ONES_LANE0 = 32, VH_COLS = 0;
  static constexpr bool KOP = false;
};
template <> struct Cfg<128> {
  static constexpr int KS = 144, VS = 144, NCB = 9, ONES_CB = 8, ONES_LANE0 = 0, VH_COLS = 128;
  static constexpr bool KOP = true;
};
// Workgroup shapes of attn_kernel: WAVES x QB x 16 = BM queries per
// workgroup, each wave owning QB blocks of 16 queries that share every K and
// V operand it reads. The wide shapes (256 queries per workgroup, 2 waves per
// SIMD: hd128 with two query blocks per wave here, hd72 in attn_w32_kernel
// below) halve the LDS reads and the K/V staging per query; they are used
// unless the problem is too small to spread their workgroups over the chip.
template <int D, bool WIDE> struct Shape;
// XT: the P.V products of tile j-1 run interleaved with the softmax of tile
// j (a second P register set) instead of as a burst at the end of tile j-1.
// P16: P~ goes to the P.V product as one f16 term on the f16 MFMA, with V
// widened once per tile into a transposed f16 copy in LDS (instead of two
// e4m3 terms against e4m3 V).
template <> struct Shape<72, false> {
  static constexpr int WAVES = 8, QB = 1, MIN_WAVES_PER_EU = 4, BM = 128;
  static constexpr bool XT = false, P16 = false;
};
template <> struct Shape<128, false> {
  static constexpr int WAVES = 8, QB = 1, MIN_WAVES_PER_EU = 2, BM = 128;
  static constexpr bool XT = true, P16 = false;
};
template <> struct Shape<128, true> {
  static constexpr int WAVES = 8, QB = 2, MIN_WAVES_PER_EU = 2, BM = 256;
  static constexpr bool XT = false, P16 = true;
};

// Segment i of the packed batch, clamped to [0, T]: a cu_seqlens that does
// not describe the batch (fp8vit_check_cu_seqlens tells) can leave output rows
// unwritten but never makes a kernel address memory outside the tensors.
__device__ __forceinline__ void segment_bounds(const AttnArgs& a, int i, int& b0, int& b1) {
  b0 = min(max(a.cu[i], 0), a.T);
  b1 = min(max(a.cu[i + 1], b0), a.T);
}

// LDS placement of a tile. S^T block t (0..7) row i16 is key
// 32 (i16 / 4) + 4 t + i16 % 4 (k_block_key); its A operand lane (g, i16)
// holds d bytes 32 g .. 32 g + 31 of that key, as two 16-byte reads.
//  K rows (KOP false): key k sits in row 4*(k%32) + k/32, so the 16 keys of
//     one S^T block occupy 16 consecutive rows 16t..16t+15. hd72: lane groups
//     2 and 3 both read bytes 64..95 (8 data bytes, then bytes that only meet
//     zero Q bytes; row 127 runs into 32 zero bytes after the tile).
//  K in operand order (KOP true): the chunk lane (g, i16) reads for (t, half h)
//     sits at (2t + h) * 1024 + 16 * (16 g + i16), so every operand read of a
//     wave is one contiguous kilobyte; the DMA gathers the chunks.
//  V: key k sits in row k (VS-byte rows).
__device__ __forceinline__ int k_block_key(int t, int i16) { return 32 * (i16 >> 2) + 4 * t + (i16 & 3); }
__device__ __forceinline__ int k_key(int row) { return 32 * (row & 3) + (row >> 2); }

template <int D, int WAVES> struct Stage {
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int KZERO = kBN * Cfg<D>::KS;   // rows: 32 zero bytes after the K rows
  static constexpr int KBUF = Cfg<D>::KOP ? 16 * 1024 : KZERO + 32, VBUF = kBN * Cfg<D>::VS;
  // Widened V, f16, in the order of the operand reads: the 16-byte chunk of
  // column 16 cb + i16 holding keys 32 g + 8 c .. + 7 sits at
  // ((4 cb + c) * 64 + 16 g + i16) * 16, so that every read (and every
  // widening store) of a wave is one contiguous kilobyte.
  static constexpr int VHBUF = (Cfg<D>::VH_COLS / 16) * 4 * 1024;
  // DMA: one wave instruction moves 64 chunks of 16 bytes (1 KB) of a tile.
  static constexpr int NIK = (Cfg<D>::KOP ? 16 * 1024 : KZERO) / 1024;   // instructions per K tile
  static constexpr int NIV = kBN * Cfg<D>::VS / 1024;            // instructions per V tile
  static constexpr int NIW = (NIK + NIV + WAVES - 1) / WAVES;    // per wave, K and V together
  static_assert(kBN * Cfg<D>::VS % 1024 == 0 && kBN * Cfg<D>::KS % 1024 == 0, "DMA tiling");
};

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// A operand of S^T block t (see the K placement above). `kl` is the lane's
// byte offset for t = 0 (k_lane_offset).
//  MX (block scales): the scaled MFMA takes the scale of K positions
//     32 j .. 32 j + 31 from lane group j, while lane group g's operand holds
//     positions 16 g .. 16 g + 15 (low four dwords) and 64 + 16 g .. + 15
//     (high four). So the MX operands hold d in that natural order: the low
//     chunk is d bytes 16 g .., the high chunk d bytes 64 + 16 g .. (hd72:
//     only lane group 0 has a high chunk, d 64..79; the others hold zeros).
template <int D, bool MX = false>
__device__ __forceinline__ int k_lane_offset(int g, int i16, int lane) {
  if (Cfg<D>::KOP) return 16 * lane;
  const int krow = 4 * (i16 & 3) + (i16 >> 2);            // row of key 32*(i16/4) + i16%4
  if (MX) return krow * Cfg<D>::KS + 16 * g;
  return krow * Cfg<D>::KS + (D == 72 ? min(32 * g, 64) : 32 * g);
}
// hi_keep: MX hd72 only, false where the lane group has no high chunk.
template <int D, bool MX = false>
__device__ __forceinline__ v8i k_operand(const lds_u8* kl, int t, bool hi_keep = true) {
  const lds_u8* kp = kl + (Cfg<D>::KOP ? 2048 * t : 16 * t * Cfg<D>::KS);
  const v4i k0 = *(const lds_v4i*)(kp);
  if constexpr (MX && !Cfg<D>::KOP) {
    static_assert(D == 72, "MX rows placement is the hd72 one");
    // lane group 0 reads row bytes 64..79; the others read their low chunk
    // again (in bounds) and drop it
    const v4i k1 = *(const lds_v4i*)(kp + (hi_keep ? 64 : 0));
    const v4i z = v4i{0, 0, 0, 0};
    return __builtin_shufflevector(k0, hi_keep ? k1 : z, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  const v4i k1 = *(const lds_v4i*)(kp + (Cfg<D>::KOP ? 1024 : 16));
  return __builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7);
}

// A operand of O^T block cb: lane row i16 <-> V column 16cb + i16, keys 32g..32g+31,
// gathered from row-major V by the byte-transposing LDS read. `vl` is the lane's
// byte offset (v_lane_offset); the 8-key steps and the column block are constants.
template <int D>
__device__ __forceinline__ int v_lane_offset(int g, int i16) {
  return (32 * g + (i16 >> 1)) * Cfg<D>::VS + 8 * (i16 & 1);
}
template <int D>
__device__ __forceinline__ v8i v_operand(const lds_u8* vl, int cb) {
  v8i r;
#pragma unroll
  for (int sidx = 0; sidx < 4; ++sidx) {
    const lds_u8* vp = vl + 8 * sidx * Cfg<D>::VS + 16 * cb;
    const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vp));
    r[2 * sidx] = x[0];
    r[2 * sidx + 1] = x[1];
  }
  return r;
}

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v8h lds_v8h;

// One wave's share of widening an e4m3 V tile (row-major, VS-byte rows) into
// the f16 tile of the wide hd128 shape (the wide hd72 kernel has its own
// layout, attn_w32_kernel). Unit i = (column block cb, 8-key step sidx) is one
// byte-transposing read: lane (g, i16) gets keys 32g + 8 sidx .. + 7 of
// column 16 cb + i16, converts them and stores its 16 B at 1024 i + 16 lane.
template <int D, int WAVES>
__device__ __forceinline__ void widen_v(const uint8_t* v8, uint8_t* vh, int wave, int g, int i16, int vl_lane) {
  static_assert(D == 128, "the f16 P.V path of attn_kernel is the wide hd128 shape");
  constexpr int NU = (Cfg<D>::VH_COLS / 16) * 4;
#pragma unroll
  for (int n = 0; n < (NU + WAVES - 1) / WAVES; ++n) {
    const int i = wave + WAVES * n;   // wave-uniform
    if (i < NU) {
      const int cb = i >> 2, sidx = i & 3;
      const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (lds_v2i*)((const lds_u8*)v8 + vl_lane + 8 * sidx * Cfg<D>::VS + 16 * cb));
      v4i y;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        y[2 * h] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[h], 1.0f, false));
        y[2 * h + 1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[h], 1.0f, true));
      }
      *(lds_v4i*)((lds_u8*)vh + 1024 * i + 16 * (16 * g + i16)) = y;
    }
  }
}

// A operand of the f16 product of column block cb and 32-key chunk c: lane
// (g, i16) reads keys 32g + 8c .. + 7 of column 16 cb + i16. `vhl` is the
// lane's byte offset (16 * lane).
__device__ __forceinline__ v8h vh_operand(const lds_u8* vhl, int cb, int c) {
  return *(const lds_v8h*)(vhl + 1024 * (4 * cb + c));
}

// Two e4m3 terms of four probabilities P~ = exp2(s*c + nb), packed as one
// dword of the P^T operand (hi) and one of the correction term (lo).
// old_hi/old_lo: the dwords being replaced. The first conversion of each pair
// keeps the upper half of its tied "old" operand (the second one overwrites
// it), so passing the dead destination dword lets the result land in place.
__device__ __forceinline__ int2 probs_to_fp8(const v4f& s, float c, float nb, int old_hi, int old_lo) {
  const float p0 = __builtin_amdgcn_exp2f(fmaf(s[0], c, nb));
  const float p1 = __builtin_amdgcn_exp2f(fmaf(s[1], c, nb));
  const float p2 = __builtin_amdgcn_exp2f(fmaf(s[2], c, nb));
  const float p3 = __builtin_amdgcn_exp2f(fmaf(s[3], c, nb));
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, old_hi, false);
  h = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, h, true);
  const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
  const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
  int l = __builtin_amdgcn_cvt_pk_fp8_f32(p0 - h01[0], p1 - h01[1], old_lo, false);
  l = __builtin_amdgcn_cvt_pk_fp8_f32(p2 - h23[0], p3 - h23[1], l, true);
  return make_int2(h, l);
}

// This wave's share of the DMA of one K tile (koff: its global byte offset)
// into kdst and, with_v, one V tile into vdst. Instruction i = wave + WAVES*n
// of a tile moves LDS kilobyte i of K (i < NIK) or kilobyte i - NIK of V;
// dma_off[n] holds the lane's global offset for tile 0.
template <int D, int WAVES>
__device__ __forceinline__ void dma_issue(__amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                          const uint32_t* dma_off, int wave, uint32_t koff, uint8_t* kdst,
                                          uint32_t voff, uint8_t* vdst, bool with_v) {
  using S = Stage<D, WAVES>;
#pragma unroll
  for (int n = 0; n < S::NIW; ++n) {
    const int i = wave + WAVES * n;   // wave-uniform
    if (i < S::NIK) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(kdst + 1024 * i), 16, dma_off[n] + koff, 0, 0, 0);
    } else if (i < S::NIK + S::NIV && with_v) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(vdst + 1024 * (i - S::NIK)), 16, dma_off[n] + voff, 0,
                                               0, 0);
    }
  }
}

// MX: the block-scaled variant. Q and K carry one E8M0 scale per 32-element
// block of head_dim (a.qs, a.ks: four bytes per (token, head)); the S^T MFMA
// applies them per lane (lane group g supplies the scale of block g of its
// row; the operands hold d in the MFMA's natural K order, see the K placement
// above), so S comes out in true units and the softmax constant is
// softmax_scale * log2(e). V keeps its per-tensor scale.
template <int D, bool OUT8, bool WIDE, bool MX = false>
__global__ __launch_bounds__((64 * Shape<D, WIDE>::WAVES))
__attribute__((amdgpu_waves_per_eu(Shape<D, WIDE>::MIN_WAVES_PER_EU))) void attn_kernel(AttnArgs a) {
  using C = Cfg<D>;
  using SH = Shape<D, WIDE>;
  using S = Stage<D, SH::WAVES>;
  constexpr int QB = SH::QB;
  constexpr int BMW = 16 * QB;
  constexpr int kBM = SH::BM;
  static_assert(SH::WAVES * BMW == kBM, "block shape");
  // Two K and two V buffers, as separate objects: the compiler can then tell
  // the DMA's target apart from the buffer being read and does not wait for
  // the DMA before each LDS read.
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[S::KBUF];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[S::KBUF];
  __shared__ __attribute__((aligned(256))) uint32_t ks_lds0[MX ? kBN : 1];   // K block scales of a tile, per key
  __shared__ __attribute__((aligned(256))) uint32_t ks_lds1[MX ? kBN : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[S::VBUF];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[S::VBUF];
  __shared__ __attribute__((aligned(1024))) uint8_t vh_lds0[SH::P16 ? S::VHBUF : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t vh_lds1[SH::P16 ? S::VHBUF : 16];

  // ---- work item: XCD-grouped (head, query tile) -> segment by prefix scan ----
  const int G = gridDim.x;
  const int w = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int h = w / a.ntiles_ub;
  int tile = w - h * a.ntiles_ub;
  if (h >= a.H) return;
  int s0 = 0, L = -1;
  for (int i = 0; i < a.nseg; ++i) {
    int b0, b1;
    segment_bounds(a, i, b0, b1);
    const int n = (b1 - b0 + kBM - 1) / kBM;
    if (tile < n) { s0 = b0; L = b1 - b0; break; }
    tile -= n;
  }
  if (L <= 0) return;
  const int q0 = tile * kBM;
  const int ntiles = (L + kBN - 1) / kBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i16 = lane & 15;

  // ---- DMA geometry ----
  // Buffer descriptors start at key 0 of the segment for this head; their
  // record count ends at the end of the tensor, so chunks past it read 0.
  const uint32_t row_stride = (uint32_t)a.H * D;
  const uint32_t seg_off = ((uint32_t)s0 * (uint32_t)a.H + (uint32_t)h) * D;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.k8 + seg_off), (short)0, (int)(a.tensor_bytes - seg_off), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.v8 + seg_off), (short)0, (int)(a.tensor_bytes - seg_off), kRsrcWord3);
  // This wave's DMA instructions n = 0..NIW-1 are instruction i = wave + WAVES*n
  // of the tile (K for i < NIK, V after). dma_off: lane l's byte offset in
  // global memory for tile 0. K in operand order, instruction i = 2t + h: the
  // chunk of lane (g, i16) in the K placement above. Rows (K or V),
  // instruction ii: chunk c = 64*ii + l of the image, row c / (S/16), piece
  // c % (S/16) for the row stride S.
  uint32_t dma_off[S::NIW];
#pragma unroll
  for (int n = 0; n < S::NIW; ++n) {
    const int i = wave + SH::WAVES * n;
    if (i < S::NIK && C::KOP) {
      dma_off[n] = (uint32_t)k_block_key(i >> 1, i16) * row_stride +
                   (MX ? 16u * g + 64u * (i & 1) : 32u * g + 16u * (i & 1));
    } else if (i < S::NIK) {
      const int c = 64 * i + lane;
      const int row = c / (C::KS / 16), piece = c % (C::KS / 16);
      dma_off[n] = (uint32_t)k_key(row) * row_stride + 16u * (uint32_t)piece;
    } else {
      const int c = 64 * (i - S::NIK) + lane;
      dma_off[n] = (uint32_t)(c / (C::VS / 16)) * row_stride + 16u * (uint32_t)(c % (C::VS / 16));
    }
  }
  // MX: the K tile's scale dwords (four E8M0 bytes per key) come with it,
  // 4 bytes per lane, waves 0 and 1 moving 64 keys each.
  __amdgpu_buffer_rsrc_t ksrs;
  if constexpr (MX) {
    const uint32_t rows = a.tensor_bytes / D;   // T * H
    const uint32_t first = (uint32_t)s0 * (uint32_t)a.H + (uint32_t)h;
    ksrs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.ks + 4u * first), (short)0, (int)(4u * (rows - first)),
                                             kRsrcWord3);
  }
  // Issue this wave's DMA of K tile tk into kdst (with its scales into ksdst,
  // MX) and (with_v) V tile tv into vdst.
  auto dma_tiles = [&](int tk, uint8_t* kdst, uint32_t* ksdst, int tv, uint8_t* vdst, bool with_v) {
    dma_issue<D, SH::WAVES>(krs, vrs, dma_off, wave, (uint32_t)tk * kBN * row_stride, kdst, (uint32_t)tv * kBN * row_stride,
                 vdst, with_v);
    if constexpr (MX) {
      if (wave < 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ksrs, (lds_void*)(ksdst + 64 * wave), 4,
                                                 ((uint32_t)tk * kBN + 64u * wave + lane) * 4u * (uint32_t)a.H, 0, 0, 0);
    }
  };

  dma_tiles(0, k_lds0, ks_lds0, 0, v_lds0, !SH::XT);    // K(0), and V(0) unless iteration 0 loads it
  dma_tiles(1, k_lds1, ks_lds1, 1, v_lds1, SH::P16);    // K(1), and V(1) for the widening pipeline
  if constexpr (!C::KOP) {
    // Zero the 32 bytes after each K tile (read only against zero Q bytes).
    for (int r = tid; r < 2 * 4; r += S::THREADS)
      *reinterpret_cast<uint2*>((r < 4 ? k_lds0 : k_lds1) + S::KZERO + 8 * (r % 4)) = make_uint2(0u, 0u);
  }

  const float dq = a.st->descale_used[0], dk = a.st->descale_used[1], dv = a.st->descale_used[2];
  // raw score -> log2 units (> 0); MX scores already carry the block scales
  const float cexp = MX ? a.softmax_scale * kLog2e : a.softmax_scale * dq * dk * kLog2e;

  // ---- Q operands (B of S^T): lane holds query i16 of its block, d bytes 32g.. ----
  v8i qop[QB];
  int qsc[QB];   // MX: E8M0 scale of this lane's block g of its query (127 = 1.0 where no query)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qop[qb] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    qsc[qb] = 127;
    const int qr = q0 + wave * BMW + qb * 16 + i16;
    if (qr < L) {
      if (MX) qsc[qb] = a.qs[((int64_t)(s0 + qr) * a.H + h) * 4 + g];
      const uint8_t* src = a.q8 + ((int64_t)(s0 + qr) * a.H + h) * D;
      if (MX && D == 72) {
        // natural K order: d 16 g .. 16 g + 15, then (lane group 0) d 64..71
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          uint2 u = *reinterpret_cast<const uint2*>(src + 16 * g + 8 * j);
          qop[qb][2 * j] = (int)u.x;
          qop[qb][2 * j + 1] = (int)u.y;
        }
        if (g == 0) {
          uint2 u = *reinterpret_cast<const uint2*>(src + 64);
          qop[qb][4] = (int)u.x;
          qop[qb][5] = (int)u.y;
        }
      } else if (MX) {
        const v4i u0 = *reinterpret_cast<const v4i*>(src + 16 * g);
        const v4i u1 = *reinterpret_cast<const v4i*>(src + 64 + 16 * g);
        qop[qb] = __builtin_shufflevector(u0, u1, 0, 1, 2, 3, 4, 5, 6, 7);
      } else if (D == 72) {
        if (g < 2) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint2 u = *reinterpret_cast<const uint2*>(src + 32 * g + 8 * j);
            qop[qb][2 * j] = (int)u.x;
            qop[qb][2 * j + 1] = (int)u.y;
          }
        } else if (g == 2) {
          uint2 u = *reinterpret_cast<const uint2*>(src + 64);
          qop[qb][0] = (int)u.x;
          qop[qb][1] = (int)u.y;
        }
      } else {
        const v4i u0 = *reinterpret_cast<const v4i*>(src + 32 * g);
        const v4i u1 = *reinterpret_cast<const v4i*>(src + 32 * g + 16);
        qop[qb] = __builtin_shufflevector(u0, u1, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
  }

  v4f o[QB][C::NCB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int cb = 0; cb < C::NCB; ++cb) o[qb][cb] = v4f{0.f, 0.f, 0.f, 0.f};
  float mref[QB], thr[QB];   // reference max (log2 units); raw-score threshold (m_ref + lazy) / c
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) mref[qb] = thr[qb] = -INFINITY;
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};

  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's DMA of K(0), K(1), V(0)
  __syncthreads();
  const int kl_lane = k_lane_offset<D, MX>(g, i16, lane);
  const bool k_hi = (D != 72) || (g == 0);   // MX hd72: lane groups with a high K chunk
  const int vl_lane = v_lane_offset<D>(g, i16);
  const int vhl_lane = 16 * lane;
  if constexpr (SH::P16) widen_v<D, SH::WAVES>(v_lds0, vh_lds0, wave, g, i16, vl_lane);   // V(0)

  // Software pipeline over key tiles. Iteration j holds S(j) in registers
  // (computed during iteration j-1), so the tile's maximum is known before
  // any probability is formed; its S(j+1) = K(j+1) Q^T products run on the
  // matrix core while the VALU forms P(j), and the O^T += V(j)^T P(j)^T
  // products follow at its end. LDS: an iteration reads K(j+1) and V(j) while
  // the DMA fills the other buffer of each pair with K(j+2) and V(j+1); one
  // barrier per iteration, at its start.
  v8i phi[QB], plo[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) phi[qb] = plo[qb] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  constexpr int kOne8 = 0x38383838;   // four e4m3 1.0
  // hd128: constant A operand of the ones block (row 0 = 1.0); hd72: the A
  // operand row of column 72 (lanes with i16 == 8 of block 4) is set to 1.0.
  const v8i ones_op = (i16 == 0) ? v8i{kOne8, kOne8, kOne8, kOne8, kOne8, kOne8, kOne8, kOne8}
                                 : v8i{0, 0, 0, 0, 0, 0, 0, 0};
  const bool ones_row = (D == 72) && (i16 == 8);
  auto v_op = [&](const lds_u8* vbp, int cb) -> v8i {
    if (D == 128 && cb == 8) return ones_op;
    v8i r = v_operand<D>(vbp, cb);
    if (D == 72 && cb == C::ONES_CB) {
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = ones_row ? kOne8 : r[e];
    }
    return r;
  };

  // S^T block t of one query block: K rows as A, Q as B. MX: the lane's row of
  // block t is key 32 (i16 / 4) + 4 t + i16 % 4; its scale byte g comes from
  // the tile's scale dwords in LDS.
  const int ks_key0 = 32 * (i16 >> 2) + (i16 & 3);
  auto k_scale = [&](const uint32_t* ksbuf, int t) -> int {
    if constexpr (MX) {
      const uint32_t w = ((const __attribute__((address_space(3))) uint32_t*)ksbuf)[ks_key0 + 4 * t];
      return (int)((w >> (8 * g)) & 0xffu);
    }
    return 0;
  };
  auto s_mfma = [&](const v8i& kop, int ksv, int qb) -> v4f {
    if constexpr (MX) return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kop, qop[qb], zero4, 0, 0, 0, ksv, 0, qsc[qb]);
    return mfma_fp8(kop, qop[qb], zero4);
  };

  // S(0)
  v4f sc[QB][8];
  {
    uint32_t kbase = (uint32_t)kl_lane;
    asm volatile("" : "+v"(kbase));
    const lds_u8* kl = (const lds_u8*)k_lds0 + kbase;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const v8i kop = k_operand<D, MX>(kl, t, k_hi);
      const int ksv = k_scale(ks_lds0, t);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sc[qb][t] = s_mfma(kop, ksv, qb);
    }
  }

  // One iteration; LAST: keys of S(j) past the segment end are masked and
  // there is no S(j+1). ODD = j & 1 selects the buffers.
  auto iteration = [&](auto last_c, auto odd_c, int j) {
    constexpr bool LAST = decltype(last_c)::value;
    constexpr bool ODD = decltype(odd_c)::value;
    uint8_t* const k_fill = ODD ? k_lds1 : k_lds0;         // K(j+2)
    uint32_t* const ks_fill = ODD ? ks_lds1 : ks_lds0;
    uint8_t* const v_fill = ODD ? v_lds0 : v_lds1;         // V(j+1)
    const uint8_t* const k_read = ODD ? k_lds0 : k_lds1;   // K(j+1)
    const uint32_t* const ks_read = ODD ? ks_lds0 : ks_lds1;
    const uint8_t* const v_read = ODD ? v_lds1 : v_lds0;   // V(j)
    // The previous iteration's reads of the buffers refilled below are done,
    // and this wave's DMA of K(j+1) and V(j) has landed, on every wave.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    dma_tiles(j + 2, k_fill, ks_fill, j + 1, v_fill, true);
    if (LAST) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sc[qb][t][r] = (j * kBN + 32 * g + 4 * t + r >= L) ? -INFINITY : sc[qb][t][r];
    }
    // Lazy reference max: only when a score exceeds its row's threshold is the
    // row max reduced across the four lane groups, m_ref moved and O rescaled.
    float lm[QB];
    bool over = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        m0 = fmaxf(fmaxf(fmaxf(fmaxf(m0, sc[qb][t][0]), sc[qb][t][1]), sc[qb][t][2]), sc[qb][t][3]);
        m1 = fmaxf(fmaxf(fmaxf(fmaxf(m1, sc[qb][t + 1][0]), sc[qb][t + 1][1]), sc[qb][t + 1][2]), sc[qb][t + 1][3]);
      }
      lm[qb] = fmaxf(m0, m1);
      over = over || (lm[qb] > thr[qb]);
    }
    if (__ballot(over) != 0ull) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float m = lm[qb];
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        const float mn = fmaxf(mref[qb], m * cexp);
        const float alpha = __builtin_amdgcn_exp2f(mref[qb] - mn);
        mref[qb] = mn;
        thr[qb] = (mn + kLazy) / cexp;
#pragma unroll
        for (int cb = 0; cb < C::NCB; ++cb) o[qb][cb] *= alpha;
      }
    }
    float nb[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) nb[qb] = kExpBias - mref[qb];

    uint32_t kbase = (uint32_t)kl_lane, vbase = (uint32_t)vl_lane;
    asm volatile("" : "+v"(kbase), "+v"(vbase));
    const lds_u8* kl = (const lds_u8*)k_read + kbase;
    const lds_u8* vl = (const lds_u8*)v_read + vbase;
    // P(j) block by block, each followed by the S(j+1) product of that block
    // (its K operand read one step ahead).
    v8i kop;
    if (!LAST) kop = k_operand<D, MX>(kl, 0, k_hi);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int2 p = probs_to_fp8(sc[qb][t], cexp, nb[qb], phi[qb][t], plo[qb][t]);
        phi[qb][t] = p.x;
        plo[qb][t] = p.y;
      }
      if (!LAST) {
        const v8i kcur = kop;
        if (t + 1 < 8) kop = k_operand<D, MX>(kl, t + 1, k_hi);
        const int ksv = k_scale(ks_read, t);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sc[qb][t] = s_mfma(kcur, ksv, qb);
      }
      // One query block per wave (4 waves/SIMD, 128 VGPRs): keep the steps
      // apart, since hoisting later LDS reads or softmax work into this step
      // would spill. Two query blocks (256 VGPRs): let the scheduler overlap
      // adjacent steps (+1 %).
      if (QB == 1) __builtin_amdgcn_sched_barrier(0);
    }
    // O^T += V(j)^T P(j)^T, block cb's lo term issued after block cb+1's hi
    // term, so no product waits on the one just issued.
    v8i vprev = v_op(vl, 0);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) o[qb][0] = mfma_fp8(vprev, phi[qb], o[qb][0]);
#pragma unroll
    for (int cb = 1; cb < C::NCB; ++cb) {
      const v8i vcur = v_op(vl, cb);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) o[qb][cb] = mfma_fp8(vcur, phi[qb], o[qb][cb]);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) o[qb][cb - 1] = mfma_fp8(vprev, plo[qb], o[qb][cb - 1]);
      vprev = vcur;
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) o[qb][C::NCB - 1] = mfma_fp8(vprev, plo[qb], o[qb][C::NCB - 1]);
  };
  // f16 P variant: iteration j reads K(j+1), the widened V(j) and the e4m3
  // V(j+1) (which it widens into the other f16 buffer), while the DMA fills
  // the other K buffer with K(j+2) and the other e4m3 V buffer with V(j+2).
  // P(j) becomes f16: for 32-key chunk c the lane packs its rows of S^T
  // blocks 2c and 2c+1, keys 32g + 8c .. + 7, which is the B operand of the
  // 16x16x32 f16 product whose A operand is the widened V^T.
  int p16[QB][16];
  const v8h ones16 = __builtin_bit_cast(v8h, (i16 == 0) ? v4i{0x3c003c00, 0x3c003c00, 0x3c003c00, 0x3c003c00}
                                                          : v4i{0, 0, 0, 0});
  auto iteration_p16 = [&](auto last_c, auto odd_c, int j) {
    constexpr bool LAST = decltype(last_c)::value;
    constexpr bool ODD = decltype(odd_c)::value;
    uint8_t* const k_fill = ODD ? k_lds1 : k_lds0;          // K(j+2)
    uint32_t* const ks_fill = ODD ? ks_lds1 : ks_lds0;
    uint8_t* const v_fill = ODD ? v_lds1 : v_lds0;          // e4m3 V(j+2)
    const uint8_t* const v_conv = ODD ? v_lds0 : v_lds1;    // e4m3 V(j+1)
    uint8_t* const vh_fill = ODD ? vh_lds0 : vh_lds1;       // f16 V(j+1)
    const uint8_t* const k_read = ODD ? k_lds0 : k_lds1;    // K(j+1)
    const uint32_t* const ks_read = ODD ? ks_lds0 : ks_lds1;
    const uint8_t* const vh_read = ODD ? vh_lds1 : vh_lds0; // f16 V(j)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    dma_tiles(j + 2, k_fill, ks_fill, j + 2, v_fill, true);
    if (!LAST) widen_v<D, SH::WAVES>(v_conv, vh_fill, wave, g, i16, vl_lane);
    if (LAST) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sc[qb][t][r] = (j * kBN + 32 * g + 4 * t + r >= L) ? -INFINITY : sc[qb][t][r];
    }
    float lm[QB];
    bool over = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        m0 = fmaxf(fmaxf(fmaxf(fmaxf(m0, sc[qb][t][0]), sc[qb][t][1]), sc[qb][t][2]), sc[qb][t][3]);
        m1 = fmaxf(fmaxf(fmaxf(fmaxf(m1, sc[qb][t + 1][0]), sc[qb][t + 1][1]), sc[qb][t + 1][2]), sc[qb][t + 1][3]);
      }
      lm[qb] = fmaxf(m0, m1);
      over = over || (lm[qb] > thr[qb]);
    }
    if (__ballot(over) != 0ull) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float m = lm[qb];
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        const float mn = fmaxf(mref[qb], m * cexp);
        const float alpha = __builtin_amdgcn_exp2f(mref[qb] - mn);
        mref[qb] = mn;
        thr[qb] = (mn + kLazy) / cexp;
#pragma unroll
        for (int cb = 0; cb < C::NCB; ++cb) o[qb][cb] *= alpha;
      }
    }
    float nb[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) nb[qb] = kExpBias - mref[qb];

    uint32_t kbase = (uint32_t)kl_lane, vbase = (uint32_t)vhl_lane;
    asm volatile("" : "+v"(kbase), "+v"(vbase));
    const lds_u8* kl = (const lds_u8*)k_read + kbase;
    const lds_u8* vhl = (const lds_u8*)vh_read + vbase;
    v8i kop;
    if (!LAST) kop = k_operand<D, MX>(kl, 0, k_hi);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[qb][t][0], cexp, nb[qb]));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[qb][t][1], cexp, nb[qb]));
        const float p2 = __builtin_amdgcn_exp2f(fmaf(sc[qb][t][2], cexp, nb[qb]));
        const float p3 = __builtin_amdgcn_exp2f(fmaf(sc[qb][t][3], cexp, nb[qb]));
        p16[qb][2 * t] = __builtin_bit_cast(int, (v2h){(_Float16)p0, (_Float16)p1});
        p16[qb][2 * t + 1] = __builtin_bit_cast(int, (v2h){(_Float16)p2, (_Float16)p3});
      }
      if (!LAST) {
        const v8i kcur = kop;
        if (t + 1 < 8) kop = k_operand<D, MX>(kl, t + 1, k_hi);
        const int ksv = k_scale(ks_read, t);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sc[qb][t] = s_mfma(kcur, ksv, qb);
      }
      // O^T += V(j)^T P(j)^T for the 32-key chunk whose P is now complete,
      // so the P.V products spread over the softmax work of the tile.
      if (t & 1) {
        const int c = t >> 1;
#pragma unroll
        for (int cb = 0; cb < C::NCB; ++cb) {
          // hd128: block 8 is the constant ones block (row 0 = 1.0)
          const v8h va = (D == 128 && cb == 8) ? ones16 : vh_operand(vhl, cb, c);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const v8h pb = __builtin_bit_cast(
                v8h, v4i{p16[qb][4 * c], p16[qb][4 * c + 1], p16[qb][4 * c + 2], p16[qb][4 * c + 3]});
            o[qb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb, o[qb][cb], 0, 0, 0);
          }
        }
      }
      if (QB == 1) __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Cross-tile variant: iteration j reads K(j+1) and V(j-1) while the DMA
  // fills the other buffer of each pair with K(j+2) and V(j); its steps run
  // O^T += V(j-1)^T P(j-1)^T block by block next to the softmax of S(j), so P
  // lives in two register sets. A rescale found at the start of iteration j
  // is applied at its end, after the products of P(j-1) (formed with the old
  // reference max) have been added.
  struct PSet { v8i hi[QB], lo[QB]; };
  PSet pa, pb;
  auto pv_block = [&](const PSet& pp, const v8i& vop, int cb) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) o[qb][cb] = mfma_fp8(vop, pp.hi[qb], o[qb][cb]);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) o[qb][cb] = mfma_fp8(vop, pp.lo[qb], o[qb][cb]);
  };
  auto iteration_xt = [&](auto first_c, auto last_c, auto odd_c, int j, PSet& cur, const PSet& prev) {
    constexpr bool FIRST = decltype(first_c)::value;
    constexpr bool LAST = decltype(last_c)::value;
    constexpr bool ODD = decltype(odd_c)::value;
    uint8_t* const k_fill = ODD ? k_lds1 : k_lds0;         // K(j+2)
    uint32_t* const ks_fill = ODD ? ks_lds1 : ks_lds0;
    uint8_t* const v_fill = ODD ? v_lds1 : v_lds0;         // V(j)
    const uint8_t* const k_read = ODD ? k_lds0 : k_lds1;   // K(j+1)
    const uint32_t* const ks_read = ODD ? ks_lds0 : ks_lds1;
    const uint8_t* const v_read = ODD ? v_lds0 : v_lds1;   // V(j-1)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    dma_tiles(j + 2, k_fill, ks_fill, j, v_fill, true);
    if (LAST) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sc[qb][t][r] = (j * kBN + 32 * g + 4 * t + r >= L) ? -INFINITY : sc[qb][t][r];
    }
    float lm[QB];
    bool over = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        m0 = fmaxf(fmaxf(fmaxf(fmaxf(m0, sc[qb][t][0]), sc[qb][t][1]), sc[qb][t][2]), sc[qb][t][3]);
        m1 = fmaxf(fmaxf(fmaxf(fmaxf(m1, sc[qb][t + 1][0]), sc[qb][t + 1][1]), sc[qb][t + 1][2]), sc[qb][t + 1][3]);
      }
      lm[qb] = fmaxf(m0, m1);
      over = over || (lm[qb] > thr[qb]);
    }
    const bool rescale = __ballot(over) != 0ull;
    float alpha[QB];
    if (rescale) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float m = lm[qb];
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        const float mn = fmaxf(mref[qb], m * cexp);
        alpha[qb] = __builtin_amdgcn_exp2f(mref[qb] - mn);
        mref[qb] = mn;
        thr[qb] = (mn + kLazy) / cexp;
      }
    }
    float nb[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) nb[qb] = kExpBias - mref[qb];

    uint32_t kbase = (uint32_t)kl_lane, vbase = (uint32_t)vl_lane;
    asm volatile("" : "+v"(kbase), "+v"(vbase));
    const lds_u8* kl = (const lds_u8*)k_read + kbase;
    const lds_u8* vl = (const lds_u8*)v_read + vbase;
    v8i kop, vop;
    if (!LAST) kop = k_operand<D, MX>(kl, 0, k_hi);
    if (!FIRST) vop = v_op(vl, 0);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (!FIRST) {
        if (t < C::NCB) {
          const v8i vcur = vop;
          if (t + 1 < C::NCB) vop = v_op(vl, t + 1);
          pv_block(prev, vcur, t);
        }
        if (t == 7 && C::NCB > 8) pv_block(prev, vop, 8);
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int2 p = probs_to_fp8(sc[qb][t], cexp, nb[qb], cur.hi[qb][t], cur.lo[qb][t]);
        cur.hi[qb][t] = p.x;
        cur.lo[qb][t] = p.y;
        // consumed only by the next iteration: keep its computation here
        asm volatile("" : "+v"(cur.hi[qb]), "+v"(cur.lo[qb]));
      }
      if (!LAST) {
        const v8i kcur = kop;
        if (t + 1 < 8) kop = k_operand<D, MX>(kl, t + 1, k_hi);
        const int ksv = k_scale(ks_read, t);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sc[qb][t] = s_mfma(kcur, ksv, qb);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (rescale) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int cb = 0; cb < C::NCB; ++cb) o[qb][cb] *= alpha[qb];
    }
  };
  // P.V of the last tile J; its V was loaded by iteration J into buffer J % 2.
  auto final_pv = [&](const PSet& pp, const uint8_t* vbuf) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    uint32_t vbase = (uint32_t)vl_lane;
    asm volatile("" : "+v"(vbase));
    const lds_u8* vl = (const lds_u8*)vbuf + vbase;
#pragma unroll
    for (int cb = 0; cb < C::NCB; ++cb) pv_block(pp, v_op(vl, cb), cb);
  };

  using T_ = std::true_type;
  using F_ = std::false_type;
  if constexpr (SH::P16) {
    int j = 0;
    for (; j + 2 < ntiles; j += 2) {
      iteration_p16(F_{}, F_{}, j);
      iteration_p16(F_{}, T_{}, j + 1);
    }
    if (j + 1 < ntiles) {
      iteration_p16(F_{}, F_{}, j);
      iteration_p16(T_{}, T_{}, j + 1);
    } else {
      iteration_p16(T_{}, F_{}, j);
    }
  } else if constexpr (!SH::XT) {
    int j = 0;
    for (; j + 2 < ntiles; j += 2) {
      iteration(F_{}, F_{}, j);
      iteration(F_{}, T_{}, j + 1);
    }
    if (j + 1 < ntiles) {
      iteration(F_{}, F_{}, j);
      iteration(T_{}, T_{}, j + 1);
    } else {
      iteration(T_{}, F_{}, j);
    }
  } else {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) pa.hi[qb] = pa.lo[qb] = pb.hi[qb] = pb.lo[qb] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    if (ntiles == 1) {
      iteration_xt(T_{}, T_{}, F_{}, 0, pa, pb);
      final_pv(pa, v_lds0);
    } else {
      iteration_xt(T_{}, F_{}, F_{}, 0, pa, pb);
      int j = 1;
      for (; j + 2 < ntiles; j += 2) {
        iteration_xt(F_{}, F_{}, T_{}, j, pb, pa);
        iteration_xt(F_{}, F_{}, F_{}, j + 1, pa, pb);
      }
      if (j + 1 < ntiles) {
        iteration_xt(F_{}, F_{}, T_{}, j, pb, pa);
        iteration_xt(F_{}, T_{}, F_{}, j + 1, pa, pb);
        final_pv(pa, v_lds0);
      } else {
        iteration_xt(F_{}, T_{}, T_{}, j, pb, pa);
        final_pv(pb, v_lds1);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no DMA in flight past the loop

  // ---- epilogue: divide by the row sum (ones column), scale by dv; bf16 RNE,
  // or e4m3 of O / out_descale (the input formula: fp32 quotient, formed as
  // RN32(O * RN64(1/out_descale)) which equals the IEEE fp32 division for
  // fp32 O, clamp to +-448, nearest-even code) ----
  double out_rcp = 0.0;
  if (OUT8) out_rcp = 1.0 / (double)(*a.out_descale);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lsum = __shfl(o[qb][C::ONES_CB][0], C::ONES_LANE0 + i16, 64);
    const float f = dv / lsum;
    const int qr = q0 + wave * BMW + qb * 16 + i16;
    if (qr < L) {
      const int64_t row = (int64_t)(s0 + qr) * a.ld_out + (int64_t)h * D;
#pragma unroll
      for (int cb = 0; cb < C::NCB; ++cb) {
        const int col = 16 * cb + 4 * g;
        if (col + 4 <= D) {
          const v4f x = o[qb][cb] * f;
          if (OUT8) {
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              y[e] = __builtin_amdgcn_fmed3f((float)((double)x[e] * out_rcp), -kFp8Max, kFp8Max);
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
            *reinterpret_cast<int*>(a.out8 + row + col) = w;
          } else {
            uint2 pk;
            pk.x = bf16_rne(x[0]) | (bf16_rne(x[1]) << 16);
            pk.y = bf16_rne(x[2]) | (bf16_rne(x[3]) << 16);
            *reinterpret_cast<uint2*>(a.out + row + col) = pk;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// hd72, 256 queries per workgroup, on 32x32 MFMA blocks.
//
// Each wave owns 32 queries; lane l works on query l % 32, lane half
// hf = l / 32. S^T = K Q^T comes in four 32-key blocks u per 128-key tile,
// each from one v_mfma_f32_32x32x64_f8f6f4 (d bytes 0..63) and one
// v_mfma_f32_32x32x16_fp8_fp8 (d bytes 64..79; Q bytes 72..79 are zero), so
// d = 72 costs 80 columns of MFMA work instead of 128. Output layout of a
// 32x32 block: lane l, register r holds row 8 (r/4) + 4 hf + r % 4, column
// l % 32. P~ goes as f16 into O^T += V^T P^T on v_mfma_f32_32x32x16_f16,
// O^T in three 32-row blocks (d 0..95; row 72 is the row-sum column).
//
// K in LDS, per 32-key block u at u * 2560: bytes 0..2047 hold the A operand
// of the 32x32x64 product, half hh of lane l at hh * 1024 + 16 l (key
// 32u + l%32, d bytes 32 (l/32) + 16 hh); bytes 2048..2559 hold d bytes 64..79
// of key 32u + m at 16 m (lane l reads 8 bytes at 16 (l%32) + 8 (l/32)).
// The DMA gathers these 16-byte chunks: 10 KB per tile, as for rows.
//
// 16-key chunk (u, qq) of the P.V product: B operand lane l holds the f16 P~
// of S registers 8qq..8qq+7 of block u, i.e. keys 32u + 16qq + 4 hf + e for
// e in {0,1,2,3,8,9,10,11}; the widened V^T holds, for d row 32 db + l%32,
// the same keys in the same order at ((8 db + 2u + qq) * 64 + l) * 16, so
// every operand read and every widening store is contiguous.
// ---------------------------------------------------------------------------
namespace w32 {
constexpr int WAVES = 8, BM = 256, KBUF = 10240, VBUF = kBN * 80, VHBUF = 3 * 8 * 1024;
constexpr int NIW = (10 + 10 + WAVES - 1) / WAVES;
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) long lds_i64;

__device__ __forceinline__ v16f mfma64(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ v16f mfma16(long a, long b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a, b, c, 0, 0, 0);
}

// MX: d 64..71 (the 8 elements of block 2) as bf16 values code * 2^(e - 127),
// exact (an e4m3 value times a power of two, inside bf16's range), for the
// 32x32x16 bf16 product. e8 is the block's E8M0 byte; byte 0 (2^-127) gives
// scale 0, which drops only values below 448 * 2^-127 in magnitude.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v8bf tail_bf16(long codes, uint32_t e8) {
  const float sc = __uint_as_float(e8 << 23);
  const int lo = (int)codes, hi = (int)(codes >> 32);
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, sc, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, sc, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// One wave's share of widening the e4m3 V tile (80-byte rows) into the f16
// operand layout above. Unit i = (16-column block cb, 8-key step sidx): lane
// (g, i16) reads keys 32g + 8 sidx .. + 7 of column c = 16 cb + i16; keys
// e = 0..3 go to lane half 0 and e = 4..7 to half 1 of chunk (db = c/32, u = g,
// qq = sidx/2), as its 8-byte half sidx % 2. Column 72 is written as 1.0,
// 73..79 as 0.
__device__ __forceinline__ void widen(const uint8_t* v8, uint8_t* vh, int wave, int g, int i16, int vl_lane) {
#pragma unroll
  for (int n = 0; n < (20 + WAVES - 1) / WAVES; ++n) {
    const int i = wave + WAVES * n;
    if (i < 20) {
      const int cb = i >> 2, sidx = i & 3;
      const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (lds_v2i*)((const lds_u8*)v8 + vl_lane + 8 * sidx * 80 + 16 * cb));
      const int c = 16 * cb + i16;
      v2i lo, hi;   // keys e = 0..3 and 4..7 as f16
      lo[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[0], 1.0f, false));
      lo[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[0], 1.0f, true));
      hi[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[1], 1.0f, false));
      hi[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[1], 1.0f, true));
      // Only the units of column block 4 (the last n) reach column 72; the
      // test on n is a constant once the loop is unrolled.
      if (16 * ((WAVES * n + WAVES - 1) >> 2) + 15 >= 72 && c >= 72) {
        const int f = c == 72 ? 0x3c003c00 : 0;
        lo = v2i{f, f};
        hi = v2i{f, f};
      }
      const int chunk = 8 * (c >> 5) + 2 * g + (sidx >> 1);
      lds_u8* base = (lds_u8*)vh + chunk * 1024 + 8 * (sidx & 1);
      *(lds_v2i*)(base + 16 * (c & 31)) = lo;
      *(lds_v2i*)(base + 16 * (32 + (c & 31))) = hi;
    }
  }
}
}  // namespace w32

// Key split of attn_w32_kernel: a piece of a split item leaves O / l (f16),
// m_ref and l for its queries in its record (kSplitSlotBytes per (item,
// piece): O at [query][72], then m and l as fp32 [256] each).
__device__ __forceinline__ void split_write_partial(const AttnArgs& a, const w32::v16f* o, float lsum, float mref,
                                                    int item, int piece, int L, int q0, int wave, int l32, int hf) {
  constexpr int D = 72;
  const int ql = wave * 32 + l32;   // query within the item
  if (q0 + ql >= L) return;
  uint8_t* slot = a.ws_slots + ((size_t)item * a.nsplit + piece) * kSplitSlotBytes;
  const float f = 1.0f / lsum;
#pragma unroll
  for (int db = 0; db < 3; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = 32 * db + 8 * i + 4 * hf;
      if (col + 4 <= D) {
        const v2h lo = {(_Float16)(o[db][4 * i] * f), (_Float16)(o[db][4 * i + 1] * f)};
        const v2h hi = {(_Float16)(o[db][4 * i + 2] * f), (_Float16)(o[db][4 * i + 3] * f)};
        *reinterpret_cast<uint2*>(slot + (size_t)ql * (D * 2) + col * 2) =
            make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
      }
    }
  if (hf == 0) {
    float* ml = reinterpret_cast<float*>(slot + (size_t)kSplitQueries * D * 2);
    ml[ql] = mref;
    ml[kSplitQueries + ql] = lsum;
  }
}

// Combine of the key split (launched after attn_w32_kernel on the same
// stream, so every record is complete and visible): one workgroup per item,
// two threads per query, 36 columns each. The pieces are combined in piece
// order (deterministic):
//   M = max_p m_p, w_p = l_p 2^(m_p - M), O = dv * sum_p w_p O_p / sum_p w_p,
// then written as the unsplit epilogue writes (bf16, or e4m3 of O / out_descale).
// Items that were not split (one piece) were written by the attention kernel.
template <bool OUT8>
__global__ __launch_bounds__(2 * kSplitQueries) void attn_split_combine_kernel(AttnArgs a) {
  constexpr int D = 72, BM = kSplitQueries;
  const int item = blockIdx.x;
  const int h = item / a.ntiles_ub;
  int tile = item - h * a.ntiles_ub;
  if (h >= a.H) return;
  int s0 = 0, L = -1;
  for (int i = 0; i < a.nseg; ++i) {
    int b0, b1;
    segment_bounds(a, i, b0, b1);
    const int n = (b1 - b0 + BM - 1) / BM;
    if (tile < n) { s0 = b0; L = b1 - b0; break; }
    tile -= n;
  }
  if (L <= 0) return;
  const int q0 = tile * BM;
  const int np = min(a.nsplit, (L + kBN - 1) / kBN);
  if (np <= 1) return;
  const int q = threadIdx.x >> 1, half = threadIdx.x & 1;
  if (q0 + q >= L) return;
  const float dv = a.st->descale_used[2];
  const uint8_t* slots = a.ws_slots + (size_t)item * a.nsplit * kSplitSlotBytes;
  // all m and l loads first, then all O loads: a couple of memory round trips
  constexpr int kMaxPieces = 16;
  float mp[kMaxPieces], lp[kMaxPieces];
#pragma unroll
  for (int p = 0; p < kMaxPieces; ++p) {
    if (p < np) {
      const float* ml = reinterpret_cast<const float*>(slots + (size_t)p * kSplitSlotBytes + (size_t)kSplitQueries * D * 2);
      mp[p] = ml[q];
      lp[p] = ml[kSplitQueries + q];
    }
  }
  float mx = mp[0];
#pragma unroll
  for (int p = 1; p < kMaxPieces; ++p)
    if (p < np) mx = fmaxf(mx, mp[p]);
  float acc[36];
#pragma unroll
  for (int c = 0; c < 36; ++c) acc[c] = 0.f;
  float den = 0.f;
#pragma unroll
  for (int p = 0; p < kMaxPieces; ++p) {
    if (p < np) {
      const float wgt = lp[p] * __builtin_amdgcn_exp2f(mp[p] - mx);
      den += wgt;
      const uint8_t* row = slots + (size_t)p * kSplitSlotBytes + (size_t)q * (D * 2) + half * 72;
      uint2 raw[9];
#pragma unroll
      for (int c = 0; c < 9; ++c) raw[c] = *reinterpret_cast<const uint2*>(row + 8 * c);
#pragma unroll
      for (int c = 0; c < 9; ++c) {
        const v2h lo = __builtin_bit_cast(v2h, raw[c].x), hi = __builtin_bit_cast(v2h, raw[c].y);
        acc[4 * c] = fmaf(wgt, (float)lo[0], acc[4 * c]);
        acc[4 * c + 1] = fmaf(wgt, (float)lo[1], acc[4 * c + 1]);
        acc[4 * c + 2] = fmaf(wgt, (float)hi[0], acc[4 * c + 2]);
        acc[4 * c + 3] = fmaf(wgt, (float)hi[1], acc[4 * c + 3]);
      }
    }
  }
  const float f = dv / den;
  const int64_t orow = (int64_t)(s0 + q0 + q) * a.ld_out + (int64_t)h * D + 36 * half;
  if (OUT8) {
    const double out_rcp = 1.0 / (double)(*a.out_descale);
#pragma unroll
    for (int c = 0; c < 9; ++c) {
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        y[e] = __builtin_amdgcn_fmed3f((float)((double)(acc[4 * c + e] * f) * out_rcp), -kFp8Max, kFp8Max);
      int t = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      t = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], t, true);
      *reinterpret_cast<int*>(a.out8 + orow + 4 * c) = t;
    }
  } else {
#pragma unroll
    for (int c = 0; c < 9; ++c) {
      uint2 pk;
      pk.x = bf16_rne(acc[4 * c] * f) | (bf16_rne(acc[4 * c + 1] * f) << 16);
      pk.y = bf16_rne(acc[4 * c + 2] * f) | (bf16_rne(acc[4 * c + 3] * f) << 16);
      *reinterpret_cast<uint2*>(a.out + orow + 4 * c) = pk;
    }
  }
}

template <bool OUT8, bool MX = false>
__global__ __launch_bounds__(64 * w32::WAVES) __attribute__((amdgpu_waves_per_eu(2)))
void attn_w32_kernel(AttnArgs a) {
  using namespace w32;
  constexpr int D = 72;
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[KBUF];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[KBUF];
  __shared__ __attribute__((aligned(256))) uint32_t ks_lds0[MX ? kBN : 1];   // MX: K block scales, per key
  __shared__ __attribute__((aligned(256))) uint32_t ks_lds1[MX ? kBN : 1];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[VBUF];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[VBUF];
  __shared__ __attribute__((aligned(1024))) uint8_t vh_lds0[VHBUF];
  __shared__ __attribute__((aligned(1024))) uint8_t vh_lds1[VHBUF];

  // ---- work item: XCD-grouped (head, query tile, key piece) -> segment by prefix scan ----
  const int G = gridDim.x;
  const int w = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int item = w / a.nsplit;
  const int piece = w - item * a.nsplit;
  const int h = item / a.ntiles_ub;
  int tile = item - h * a.ntiles_ub;
  if (h >= a.H) return;
  int s0 = 0, L = -1;
  for (int i = 0; i < a.nseg; ++i) {
    int b0, b1;
    segment_bounds(a, i, b0, b1);
    const int n = (b1 - b0 + BM - 1) / BM;
    if (tile < n) { s0 = b0; L = b1 - b0; break; }
    tile -= n;
  }
  if (L <= 0) return;
  const int q0 = tile * BM;
  const int ntiles = (L + kBN - 1) / kBN;
  // This workgroup's key tiles [ja, jb): piece `piece` of np near-equal pieces.
  const int np = min(a.nsplit, ntiles);
  if (piece >= np) return;
  const int ja = (int)(((int64_t)piece * ntiles) / np), jb = (int)(((int64_t)(piece + 1) * ntiles) / np);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i16 = lane & 15;
  const int hf = lane >> 5, l32 = lane & 31;

  // ---- DMA geometry (chunks as described above) ----
  const uint32_t row_stride = (uint32_t)a.H * D;
  const uint32_t seg_off = ((uint32_t)s0 * (uint32_t)a.H + (uint32_t)h) * D;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.k8 + seg_off), (short)0, (int)(a.tensor_bytes - seg_off), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.v8 + seg_off), (short)0, (int)(a.tensor_bytes - seg_off), kRsrcWord3);
  uint32_t dma_off[NIW];
#pragma unroll
  for (int n = 0; n < NIW; ++n) {
    const int i = wave + WAVES * n;
    if (i < 10) {
      const int c = 64 * i + lane, u = c / 160, r = c % 160;
      if (r < 128) {
        const int hh = r >> 6, ln = r & 63;
        dma_off[n] = (uint32_t)(32 * u + (ln & 31)) * row_stride +
                     (MX ? 16u * (uint32_t)(ln >> 5) + 32u * hh : 32u * (uint32_t)(ln >> 5) + 16u * hh);
      } else {
        dma_off[n] = (uint32_t)(32 * u + (r - 128)) * row_stride + 64u;
      }
    } else {
      const int c = 64 * (i - 10) + lane;
      dma_off[n] = (uint32_t)(c / 5) * row_stride + 16u * (uint32_t)(c % 5);
    }
  }
  // MX: the K tile's scale dwords (four E8M0 bytes per key), 4 bytes per
  // lane, waves 0 and 1 moving 64 keys each.
  __amdgpu_buffer_rsrc_t ksrs;
  if constexpr (MX) {
    const uint32_t rows = a.tensor_bytes / D;   // T * H
    const uint32_t first = (uint32_t)s0 * (uint32_t)a.H + (uint32_t)h;
    ksrs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.ks + 4u * first), (short)0, (int)(4u * (rows - first)),
                                             kRsrcWord3);
  }
  auto dma_tiles = [&](int tk, uint8_t* kdst, uint32_t* ksdst, int tv, uint8_t* vdst, bool with_v) {
    dma_issue<D, WAVES>(krs, vrs, dma_off, wave, (uint32_t)tk * kBN * row_stride, kdst,
                        (uint32_t)tv * kBN * row_stride, vdst, with_v);
    if constexpr (MX) {
      if (wave < 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ksrs, (lds_void*)(ksdst + 64 * wave), 4,
                                                 ((uint32_t)tk * kBN + 64u * wave + lane) * 4u * (uint32_t)a.H, 0, 0, 0);
    }
  };
  dma_tiles(ja, k_lds0, ks_lds0, ja, v_lds0, true);
  dma_tiles(ja + 1, k_lds1, ks_lds1, ja + 1, v_lds1, true);
  // Rows 80..95 of the widened V^T (no V columns) stay zero: in each buffer,
  // chunks 16..23 (block db = 2), lanes with l % 32 >= 16.
  for (int r = tid; r < 2 * 256; r += 64 * WAVES) {
    const int idx = r & 255, ln = 32 * ((idx >> 4) & 1) + 16 + (idx & 15);
    uint8_t* vb = (r < 256 ? vh_lds0 : vh_lds1) + (16 + (idx >> 5)) * 1024 + 16 * ln;
    *reinterpret_cast<uint4*>(vb) = make_uint4(0u, 0u, 0u, 0u);
  }

  const float dq = a.st->descale_used[0], dk = a.st->descale_used[1], dv = a.st->descale_used[2];
  // raw score -> log2 units; MX scores already carry the block scales
  const float cexp = MX ? a.softmax_scale * kLog2e : a.softmax_scale * dq * dk * kLog2e;

  // ---- Q operands: lane l: query l%32, d bytes 32 hf .. + 31 (MX: 16 hf .. + 15
  // and 32 + 16 hf .. + 15), and 64 + 8 hf .. + 7 (MX: 64 .. 71 in lane half 0) ----
  v8i qa = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  long qbv = 0;
  int qs01 = 127, qs2 = 127;   // MX: E8M0 scales of the query's block hf and block 2
  {
    const int qr = q0 + wave * 32 + l32;
    if (qr < L) {
      const uint8_t* src = a.q8 + ((int64_t)(s0 + qr) * a.H + h) * D;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint2 u2 = *reinterpret_cast<const uint2*>(src + (MX ? 16 * hf + 32 * (j >> 1) + 8 * (j & 1)
                                                                   : 32 * hf + 8 * j));
        qa[2 * j] = (int)u2.x;
        qa[2 * j + 1] = (int)u2.y;
      }
      if (hf == 0) qbv = *reinterpret_cast<const long*>(src + 64);
      if (MX) {
        const uint8_t* qsp = a.qs + ((int64_t)(s0 + qr) * a.H + h) * 4;
        qs01 = qsp[hf];
        qs2 = qsp[2];
      }
    }
  }
  // MX: d 64..71 (block 2) go through the 32x32x16 bf16 product as exact
  // scaled values (lane half 0; half 1 and rows past the segment are zero).
  v8bf qt;
  if constexpr (MX) qt = tail_bf16(qbv, (uint32_t)qs2);

  v16f o[3];
#pragma unroll
  for (int db = 0; db < 3; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float mref = -INFINITY, thr = -INFINITY;
  v16f zero16;
#pragma unroll
  for (int r = 0; r < 16; ++r) zero16[r] = 0.f;

  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's DMA of K(ja), K(ja+1), V(ja), V(ja+1)
  __syncthreads();
  const int vl_lane = v_lane_offset<D>(g, i16);
  widen(v_lds0, vh_lds0, wave, g, i16, vl_lane);      // V(ja)

  const int ka_lane = 16 * lane, kb_lane = 2048 + 16 * l32 + (MX ? 0 : 8 * hf);   // MX: d 64..71 in both halves
  auto k_a = [&](const lds_u8* kb, int u) -> v8i {
    const v4i x0 = *(const lds_v4i*)(kb + u * 2560 + ka_lane);
    const v4i x1 = *(const lds_v4i*)(kb + u * 2560 + ka_lane + 1024);
    return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto k_b = [&](const lds_u8* kb, int u) -> long { return *(const lds_i64*)(kb + u * 2560 + kb_lane); };
  // S^T block u of the wave's queries from K buffer kb (MX: with the scale
  // dwords ksb; lane l's row is key 32u + l%32).
  auto s_block = [&](const lds_u8* kb, const uint32_t* ksb, int u) -> v16f {
    if constexpr (MX) {
      // d 0..63 on the scaled 32x32x64 product (blocks 0 and 1), d 64..71 as
      // scaled bf16 values (lane half 1 holds the same key's bytes, which meet
      // zero Q values).
      const uint32_t ksw = ((const __attribute__((address_space(3))) uint32_t*)ksb)[32 * u + l32];
      const v16f s01 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          k_a(kb, u), qa, zero16, 0, 0, 0, (int)((ksw >> (8 * hf)) & 0xffu), 0, qs01);
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(tail_bf16(k_b(kb, u), (ksw >> 16) & 0xffu), qt, s01, 0, 0, 0);
    }
    return mfma16(k_b(kb, u), qbv, mfma64(k_a(kb, u), qa, zero16));
  };

  // S(ja)
  v16f sc[4];
  {
    const lds_u8* kb = (const lds_u8*)k_lds0;
#pragma unroll
    for (int u = 0; u < 4; ++u) sc[u] = s_block(kb, ks_lds0, u);
  }

  int pf[4][8];   // f16 P~ of block u: dwords 4qq .. 4qq+3 are chunk (u, qq)
  auto iteration = [&](auto last_c, auto odd_c, int j) {
    constexpr bool LAST = decltype(last_c)::value;
    constexpr bool ODD = decltype(odd_c)::value;
    uint8_t* const k_fill = ODD ? k_lds1 : k_lds0;          // K(j+2)
    uint32_t* const ks_fill = ODD ? ks_lds1 : ks_lds0;      // its scales (MX)
    uint8_t* const v_fill = ODD ? v_lds1 : v_lds0;          // e4m3 V(j+2)
    const uint8_t* const v_conv = ODD ? v_lds0 : v_lds1;    // e4m3 V(j+1)
    uint8_t* const vh_fill = ODD ? vh_lds0 : vh_lds1;       // f16 V(j+1)
    const uint8_t* const k_read = ODD ? k_lds0 : k_lds1;    // K(j+1)
    const uint32_t* const ks_read = ODD ? ks_lds0 : ks_lds1;
    const uint8_t* const vh_read = ODD ? vh_lds1 : vh_lds0; // f16 V(j)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    dma_tiles(j + 2, k_fill, ks_fill, j + 2, v_fill, true);
    if (!LAST) widen(v_conv, vh_fill, wave, g, i16, vl_lane);
    if (LAST) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sc[u][r] = (j * kBN + 32 * u + 8 * (r >> 2) + 4 * hf + (r & 3) >= L) ? -INFINITY : sc[u][r];
    }
    // Lazy reference max (see the narrow kernels): the row of query l%32 is
    // split over lanes l and l ^ 32.
    float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 16; r += 8) {
        m0 = fmaxf(fmaxf(fmaxf(fmaxf(m0, sc[u][r]), sc[u][r + 1]), sc[u][r + 2]), sc[u][r + 3]);
        m1 = fmaxf(fmaxf(fmaxf(fmaxf(m1, sc[u][r + 4]), sc[u][r + 5]), sc[u][r + 6]), sc[u][r + 7]);
      }
    const float lm = fmaxf(m0, m1);
    if (__ballot(lm > thr) != 0ull) {
      const float m = fmaxf(lm, __shfl_xor(lm, 32, 64));
      const float mn = fmaxf(mref, m * cexp);
      const float alpha = __builtin_amdgcn_exp2f(mref - mn);
      mref = mn;
      thr = (mn + kLazy) / cexp;
#pragma unroll
      for (int db = 0; db < 3; ++db) o[db] *= alpha;
    }
    const float nb = kExpBias - mref;

    uint32_t kbase = 0, vbase = (uint32_t)(16 * lane);
    asm volatile("" : "+v"(kbase), "+v"(vbase));
    const lds_u8* kb = (const lds_u8*)k_read + kbase;
    const lds_u8* vhl = (const lds_u8*)vh_read + vbase;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[u][r], cexp, nb));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[u][r + 1], cexp, nb));
        pf[u][r >> 1] = __builtin_bit_cast(int, (v2h){(_Float16)p0, (_Float16)p1});
      }
      if (!LAST) sc[u] = s_block(kb, ks_read, u);
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const v8h pb = __builtin_bit_cast(v8h, v4i{pf[u][4 * qq], pf[u][4 * qq + 1], pf[u][4 * qq + 2], pf[u][4 * qq + 3]});
#pragma unroll
        for (int db = 0; db < 3; ++db) {
          const v8h va = *(const lds_v8h*)(vhl + (8 * db + 2 * u + qq) * 1024);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb, o[db], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);   // keep each u step's exps ahead of its own MFMAs
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  // Buffer parity is relative to ja (the prologue filled buffers 0 with tile
  // ja). The last iteration of a piece has no S(j+1); its key mask only
  // removes keys past the segment end, so it is a no-op before the last tile.
  int j = ja;
  for (; j + 2 < jb; j += 2) {
    iteration(F_{}, F_{}, j);
    iteration(F_{}, T_{}, j + 1);
  }
  if (j + 1 < jb) {
    iteration(F_{}, F_{}, j);
    iteration(T_{}, T_{}, j + 1);
  } else {
    iteration(T_{}, F_{}, j);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no DMA in flight past the loop

  // ---- epilogue: row sum = O^T row 72 (block 2, register 4 of half 0) ----
  const float lsum = __shfl(o[2][4], l32, 64);
  const int qr = q0 + wave * 32 + l32;
  if (np > 1) {
    // one piece of a split item: leave its partial for attn_split_combine_kernel
    split_write_partial(a, o, lsum, mref, item, piece, L, q0, wave, l32, hf);
    return;
  }
  double out_rcp = 0.0;
  if (OUT8) out_rcp = 1.0 / (double)(*a.out_descale);
  const float f = dv / lsum;
  if (qr < L) {
    const int64_t row = (int64_t)(s0 + qr) * a.ld_out + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < 3; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = 32 * db + 8 * i + 4 * hf;
        if (col + 4 <= D) {
          const v4f x = v4f{o[db][4 * i], o[db][4 * i + 1], o[db][4 * i + 2], o[db][4 * i + 3]} * f;
          if (OUT8) {
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              y[e] = __builtin_amdgcn_fmed3f((float)((double)x[e] * out_rcp), -kFp8Max, kFp8Max);
            int wv = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
            wv = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], wv, true);
            *reinterpret_cast<int*>(a.out8 + row + col) = wv;
          } else {
            uint2 pk;
            pk.x = bf16_rne(x[0]) | (bf16_rne(x[1]) << 16);
            pk.y = bf16_rne(x[2]) | (bf16_rne(x[3]) << 16);
            *reinterpret_cast<uint2*>(a.out + row + col) = pk;
          }
        }
      }
  }
}

int attn_block_m(int head_dim) { return head_dim == 72 ? Shape<72, false>::BM : Shape<128, false>::BM; }

// Library-owned workspace of the key split for callers that cannot allocate
// (fp8vit_attn_varlen_noalloc). One copy per GPU, held until the process
// ends; every call on that GPU shares it (overlapping calls race). The split
// records need no initial contents. In host code `scratch` names a host-side
// stand-in: kernels get the device address from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  void* p = (dev >= 0 && dev < kMaxScratchDevices) ? g_scratch_ptr[dev].load(std::memory_order_relaxed) : nullptr;
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    if (dev >= 0 && dev < kMaxScratchDevices) g_scratch_ptr[dev].store(p, std::memory_order_relaxed);
  }
  *ptr = p;
  return hipSuccess;
}

namespace {
// Upper bound on query tiles of BM rows per head: every segment adds at most
// one partial tile.
int64_t tiles_ub(int bm, int64_t total_tokens, int64_t nseg, int64_t max_seqlen) {
  const int64_t by_total = (total_tokens + bm - 1) / bm + nseg;
  const int64_t by_max = nseg * ((max_seqlen + bm - 1) / bm);
  return by_total < by_max ? by_total : by_max;
}

template <int D, bool WIDE, bool MX = false>
hipError_t launch_shape(AttnArgs a, int total_tokens, int max_seqlen, hipStream_t s) {
  a.ntiles_ub = (int32_t)tiles_ub(Shape<D, WIDE>::BM, total_tokens, a.nseg, max_seqlen);
  a.nsplit = 1;   // the key split exists in the wide hd72 kernel only
  const int64_t items = (int64_t)a.H * a.ntiles_ub;
  const int64_t grid = ((items + 7) / 8) * 8;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 block(64 * Shape<D, WIDE>::WAVES);
  if constexpr (MX) {
    // block-scaled Q and K: bf16 output only
    if (a.out8 != nullptr) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_kernel<D, false, WIDE, true>), dim3((unsigned)grid), block, 0, s, a);
  } else if (a.out8 != nullptr) {
    hipLaunchKernelGGL((attn_kernel<D, true, WIDE>), dim3((unsigned)grid), block, 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_kernel<D, false, WIDE>), dim3((unsigned)grid), block, 0, s, a);
  }
  return hipGetLastError();
}
hipError_t launch_w32(AttnArgs a, int total_tokens, int max_seqlen, hipStream_t s) {
  a.ntiles_ub = (int32_t)tiles_ub(w32::BM, total_tokens, a.nseg, max_seqlen);
  if (a.nsplit < 1 || a.ws_slots == nullptr) a.nsplit = 1;
  const int64_t items = (int64_t)a.H * a.ntiles_ub * a.nsplit;
  const int64_t grid = ((items + 7) / 8) * 8;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 block(64 * w32::WAVES);
  if (a.qs != nullptr) {
    // block-scaled Q and K: bf16 output only
    if (a.out8 != nullptr) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_w32_kernel<false, true>), dim3((unsigned)grid), block, 0, s, a);
  } else if (a.out8 != nullptr) {
    hipLaunchKernelGGL((attn_w32_kernel<true>), dim3((unsigned)grid), block, 0, s, a);
  } else {
    hipLaunchKernelGGL((attn_w32_kernel<false>), dim3((unsigned)grid), block, 0, s, a);
  }
  if (a.nsplit == 1) return hipGetLastError();
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 cgrid((unsigned)((int64_t)a.H * a.ntiles_ub)), cblock(2 * kSplitQueries);
  if (a.out8 != nullptr)
    hipLaunchKernelGGL(attn_split_combine_kernel<true>, cgrid, cblock, 0, s, a);
  else
    hipLaunchKernelGGL(attn_split_combine_kernel<false>, cgrid, cblock, 0, s, a);
  return hipGetLastError();
}
}  // namespace

// Key split of the wide hd72 kernel. It pays only where the grid of
// (head, 256-query tile) items leaves CUs idle: with one workgroup per CU, a
// grid of `items` < CUs runs in one round of nkt key tiles. Cut every item
// into s pieces and the same work runs in ceil(items * s / CUs) rounds of
// ceil(nkt / s) tiles, each piece paying a fixed cost (Q load, pipeline fill
// and drain, record write) of about kSplitFixed tiles, and the combine kernel
// about kSplitCombine tiles. Measured on MI355X (graph replays): L = 4096 at
// 8 heads, one round of two pieces, 72.5 -> 44 us for the attention kernel;
// L = 2304 at 16 heads, two rounds of three pieces, 43.8 -> 40 us, which the
// combine eats. The plan takes the s with the smallest modelled time that
// fits the workspace, and splits only if that beats the unsplit model by more
// than 10 %. At most kSplitMaxRounds rounds, which also bounds the workspace
// (kSplitMaxRounds * CUs partial records: 39.8 MB on 256 CUs).
constexpr int kSplitMax = 16;   // the combine holds up to 16 pieces' m and l in registers
constexpr int kSplitMaxRounds = 4;
constexpr float kSplitFixed = 2.5f, kSplitCombine = 3.0f;

int attn_split_plan(int head_dim, int num_heads, int total_tokens, int num_segments, int max_seqlen,
                    size_t workspace_bytes, size_t* bytes) {
  *bytes = 0;
  if (head_dim != 72 || num_heads <= 0 || total_tokens <= 0 || num_segments <= 0 || max_seqlen <= 0) return 1;
  const int cus = device_cus();
  if (cus <= 0) return 1;
  const int64_t items = (int64_t)num_heads * tiles_ub(w32::BM, total_tokens, num_segments, max_seqlen);
  if (2 * items < cus || items >= cus) return 1;   // narrow kernel, or the grid already fills the chip
  const int64_t nkt = ((int64_t)max_seqlen + kBN - 1) / kBN;
  const float unsplit = (float)nkt + kSplitFixed;
  int best = 1;
  float best_cost = 0.9f * unsplit;
  for (int sp = 2; sp <= kSplitMax && sp <= nkt; ++sp) {
    const size_t need = (size_t)items * sp * kSplitSlotBytes;
    if (need > workspace_bytes) break;
    const int64_t rounds = (items * sp + cus - 1) / cus;
    if (rounds > kSplitMaxRounds) break;
    const float cost = (float)rounds * ((float)((nkt + sp - 1) / sp) + kSplitFixed) + kSplitCombine;
    if (cost < best_cost) {
      best_cost = cost;
      best = sp;
    }
  }
  if (best > 1) *bytes = (size_t)items * best * kSplitSlotBytes;
  return best;
}

hipError_t launch_attn(const AttnArgs& a, int head_dim, int total_tokens, int max_seqlen, hipStream_t s) {
  // The wide shape once its workgroups occupy at least half of the CUs (by
  // the same upper bound on tiles the grid uses): measured faster from 144
  // workgroups on 256 CUs (L = 2304, 16 heads) up, slower at 16 (L = 256).
  const int cus = device_cus();
  if (cus == 0) return hipErrorInvalidDevice;
  static_assert(w32::BM == 256 && Shape<128, true>::BM == 256, "wide shapes");
  const int64_t wide_items = (int64_t)a.H * tiles_ub(256, total_tokens, a.nseg, max_seqlen);
  const bool wide = 2 * wide_items >= (int64_t)cus;
  if (a.qs != nullptr) {
    // Block-scaled Q and K: the same shapes with the block scales fed to the
    // scaled MFMAs (one E8M0 byte per operand row and 32-element block).
    if (head_dim == 128)
      return wide ? launch_shape<128, true, true>(a, total_tokens, max_seqlen, s)
                  : launch_shape<128, false, true>(a, total_tokens, max_seqlen, s);
    return wide ? launch_w32(a, total_tokens, max_seqlen, s) : launch_shape<72, false, true>(a, total_tokens, max_seqlen, s);
  }
  if (head_dim == 128)
    return wide ? launch_shape<128, true>(a, total_tokens, max_seqlen, s)
                : launch_shape<128, false>(a, total_tokens, max_seqlen, s);
  return wide ? launch_w32(a, total_tokens, max_seqlen, s) : launch_shape<72, false>(a, total_tokens, max_seqlen, s);
}

}  // namespace fp8vit
