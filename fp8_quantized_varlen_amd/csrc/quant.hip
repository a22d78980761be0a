// Per-tensor e4m3 quantization of Q, K and V: one launch in static mode, two
// in dynamic mode.
//
// Per element (atrex-bench #025 per_token_group_quant_fp8, Reference
// Implementation, with one group per tensor): y = x / descale as an IEEE fp32
// division, clamped to [-448, 448], then rounded to the nearest e4m3fn code,
// ties to even (the hardware v_cvt_pk_fp8_f32 conversion; its rounding is
// checked against an exact software model over every bf16 input).
//
// The fp32 quotient is formed as RN32(RN64(x * r)) with r = RN64(1/descale),
// which equals RN32(x / descale) for every bf16 x: the fp64 product is within
// 2^-52 (relative) of x/descale, while x/descale (8 significant bits over 24)
// is either an fp32 number or at least 2^-49 (relative) away from every fp32
// rounding midpoint, which would need 25 significant bits in x. Overflow
// gives inf on both sides and then 448. Three VALU instructions instead of
// the ~10 of a correctly rounded fp32 division.
//
// Dynamic mode (vLLM page "FP8 ViT Encoder Attention", Usage): the amax of
// each whole tensor joins the 16-slot ring, and the window maximum sets this
// forward's descale. Two launches, one pass over the input in the usual case:
//   pass 1 quantizes with the descale of the window over the other 15 slots
//     (known before the pass) and records per-block partial maxima;
//   pass 2 reduces them to this forward's amax. The true descale is that of
//     max(window, amax); where it equals pass 1's (the amax did not raise the
//     window, or raised it without changing the fp32 descale) the codes are
//     already the right ones, bit for bit, and pass 2 only does the
//     bookkeeping. Otherwise its workgroups quantize that tensor again.
// Once the ring is full of like amaxes (steady state) a tensor is redone only
// when its amax is the largest of the 16, about one forward in 16; the first
// forward always redoes (empty ring). The ring push of this forward's amax is
// left pending in the state and done by the next forward's pass 2 (see
// DevState). A single cooperative launch with a grid-wide barrier between an
// amax pass and the quantize pass measured slower on MI355X at every size
// (the cooperative launch itself adds ~17 us, and a barrier across eight XCDs
// costs several device-scope atomic round trips).
//
// Data layout: bf16 rows of H*d elements with token stride ld; every thread
// moves 16-byte chunks (8 elements) in and 8-byte chunks out, consecutive
// lanes on consecutive chunks (fully coalesced for contiguous inputs).
#include "fp8vit_internal.h"
#include "state_device.h"

namespace fp8vit {

// Quantize passes: one 16-byte chunk of each of Q, K and V per thread and
// iteration. Static mode: up to 16 workgroups per CU, each chunk loaded,
// converted and stored in turn (a small grid with several chunks in flight
// per thread measured 9-14 % slower). Dynamic pass 1: up to 4 workgroups per
// CU (one resident round, and at most kAmaxSlots partials), the first loads
// issued before the prologue and each next chunk loaded before the current
// one is stored. Dynamic pass 2: one workgroup per CU.
constexpr int kQuantThreads = 512;
constexpr int kGridPerCu = 16;
constexpr int kGridPerCuDynamic = 4;
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_lo(uint32_t w) { return w << 16; }
__device__ __forceinline__ uint32_t bf16_hi(uint32_t w) { return w & 0xffff0000u; }

// r = RN64(1 / descale), see the header comment: the fp32 quotient x / descale.
__device__ __forceinline__ float quotient(uint32_t fbits, double r) {
  return (float)((double)__uint_as_float(fbits) * r);
}
__device__ __forceinline__ float quant_value(uint32_t fbits, double r) {
  return __builtin_amdgcn_fmed3f(quotient(fbits, r), -kFp8Max, kFp8Max);
}

// 8 bf16 (one 16-byte chunk) -> 8 e4m3 codes (8 bytes), element order kept.
__device__ __forceinline__ uint2 quant_chunk(uint4 w, double r) {
  // The first conversion of a pair keeps the upper half of its tied "old"
  // operand (overwritten by the second): pass the consumed input word.
  uint32_t a = __builtin_amdgcn_cvt_pk_fp8_f32(quant_value(bf16_lo(w.x), r), quant_value(bf16_hi(w.x), r), (int)w.x,
                                               false);
  a = __builtin_amdgcn_cvt_pk_fp8_f32(quant_value(bf16_lo(w.y), r), quant_value(bf16_hi(w.y), r), a, true);
  uint32_t b = __builtin_amdgcn_cvt_pk_fp8_f32(quant_value(bf16_lo(w.z), r), quant_value(bf16_hi(w.z), r), (int)w.z,
                                               false);
  b = __builtin_amdgcn_cvt_pk_fp8_f32(quant_value(bf16_lo(w.w), r), quant_value(bf16_hi(w.w), r), b, true);
  return make_uint2(a, b);
}

// Elements of the chunk whose quotient exceeds 448 in magnitude: the ones the
// clamp changes (the same quotients quant_chunk forms).
__device__ __forceinline__ uint32_t chunk_saturated(uint4 w, double r) {
  uint32_t n = 0;
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    n += fabsf(quotient(bf16_lo(v[i]), r)) > kFp8Max ? 1u : 0u;
    n += fabsf(quotient(bf16_hi(v[i]), r)) > kFp8Max ? 1u : 0u;
  }
  return n;
}

// Largest |x| of the chunk as 15-bit bf16 magnitude bits (finite inputs:
// magnitude bits order like the values).
__device__ __forceinline__ uint32_t chunk_absmax_bits(uint4 w) {
  uint32_t m = 0;
  const uint32_t v[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = v[i] & 0x7fffu, hi = (v[i] >> 16) & 0x7fffu;
    m = max(m, max(lo, hi));
  }
  return m;
}

template <bool CONTIG>
__device__ __forceinline__ const uint4* chunk_src(const uint16_t* x, int64_t ld, int32_t row8, uint32_t c) {
  if (CONTIG) return reinterpret_cast<const uint4*>(x) + c;
  uint32_t t = c / (uint32_t)row8, j = c - t * (uint32_t)row8;
  return reinterpret_cast<const uint4*>(x + (int64_t)t * ld + 8 * (int64_t)j);
}

// NT: non-temporal loads and stores. They speed up a pass that re-reads what
// the previous pass has just read (the redo of dynamic pass 2) by ~10 % and
// slow the static pass slightly.
template <bool NT>
__device__ __forceinline__ uint4 ld16(const uint4* p) {
  if (NT) {
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  }
  return *p;
}
template <bool NT>
__device__ __forceinline__ void st8(uint2* p, uint2 v) {
  if (NT) __builtin_nontemporal_store(v2u{v.x, v.y}, reinterpret_cast<v2u*>(p));
  else *p = v;
}
// Chunk c of each tensor (zeros past the end). ALL: every tensor (for the
// amax); otherwise the tensors the pass writes.
template <bool CONTIG, bool NT, bool ALL = false>
__device__ __forceinline__ void load3(const QuantArgs& a, uint32_t c, uint32_t n8, uint4 w[3]) {
#pragma unroll
  for (int x = 0; x < 3; ++x)
    w[x] = (c < n8 && (ALL || (a.quant_mask >> x & 1u))) ? ld16<NT>(chunk_src<CONTIG>(a.x[x], a.ld[x], a.row8, c))
                                                         : make_uint4(0, 0, 0, 0);
}

// Quantize this thread's chunks c = gtid + i * gstride of Q, K and V.
// PRELOADED: `w` already holds chunk gtid of each tensor (loaded before the
// descales were known, so that the load latency overlaps the kernel's
// prologue), and the next chunk's loads are issued before the current one is
// converted and stored. Otherwise each chunk is loaded, converted and stored
// in turn (`w` is scratch).
// SAT: also count, per tensor, the elements the clamp changes (into sat[3]).
template <bool CONTIG, bool NT, bool PRELOADED, bool SAT>
__device__ __forceinline__ void quantize_all(const QuantArgs& a, uint32_t n8, const double* r, uint32_t gtid,
                                             uint32_t gstride, uint4 w[3], uint32_t* sat) {
  for (uint32_t c = gtid; c < n8; c += gstride) {
    uint4 cur[3];
    if (PRELOADED) {
#pragma unroll
      for (int x = 0; x < 3; ++x) cur[x] = w[x];
      load3<CONTIG, NT>(a, c + gstride, n8, w);
    } else {
      load3<CONTIG, NT>(a, c, n8, cur);
    }
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      if (a.quant_mask >> x & 1u) {
        st8<NT>(reinterpret_cast<uint2*>(a.y[x]) + c, quant_chunk(cur[x], r[x]));
        if (SAT) sat[x] += chunk_saturated(cur[x], r[x]);
      }
    }
  }
}

// Dynamic pass 1 over this thread's chunks c = gtid + i * gstride: the
// largest |x| bits of each of Q, K and V (all three, for the ring) and the
// codes of the tensors the pass writes, at the descales r of the window over
// the other ring slots. `w` holds chunk gtid on entry (loaded before the
// descales were known); each next chunk is loaded before the current one is
// converted. SAT: also count clamped elements (into sat[3]).
template <bool CONTIG, bool SAT>
__device__ __forceinline__ void dyn_pass1_all(const QuantArgs& a, uint32_t n8, const double* r, uint32_t gtid,
                                              uint32_t gstride, uint4 w[3], uint32_t m[3], uint32_t* sat) {
  for (uint32_t c = gtid; c < n8; c += gstride) {
    uint4 cur[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) cur[x] = w[x];
    load3<CONTIG, false, true>(a, c + gstride, n8, w);
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      m[x] = max(m[x], chunk_absmax_bits(cur[x]));
      if (a.quant_mask >> x & 1u) {
        st8<false>(reinterpret_cast<uint2*>(a.y[x]) + c, quant_chunk(cur[x], r[x]));
        if (SAT) sat[x] += chunk_saturated(cur[x], r[x]);
      }
    }
  }
}

// Largest value of m[0..2] over the workgroup, in every thread (red: LDS
// scratch of one triple per wave).
__device__ __forceinline__ void block_max3(uint32_t m[3], uint32_t (*red)[3]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int x = 0; x < 3; ++x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m[x] = max(m[x], (uint32_t)__shfl_xor((int)m[x], off, 64));
  }
  if (lane == 0) {
#pragma unroll
    for (int x = 0; x < 3; ++x) red[wave][x] = m[x];
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    m[x] = red[0][x];
#pragma unroll
    for (int w = 1; w < kQuantThreads / 64; ++w) m[x] = max(m[x], red[w][x]);
  }
}

__device__ __forceinline__ void block_sum3(uint32_t n[3], uint32_t (*red)[3]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int x = 0; x < 3; ++x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) n[x] += (uint32_t)__shfl_xor((int)n[x], off, 64);
  }
  if (lane == 0) {
#pragma unroll
    for (int x = 0; x < 3; ++x) red[wave][x] = n[x];
  }
  __syncthreads();
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    n[x] = red[0][x];
#pragma unroll
    for (int w = 1; w < kQuantThreads / 64; ++w) n[x] += red[w][x];
  }
}

// Static quantize pass: the descales come from the stored static values
// (block 0 records them as the descales in use).
template <bool CONTIG>
__global__ __launch_bounds__(kQuantThreads) void quant_static_kernel(QuantArgs a) {
  __shared__ double rcp[3];
  __shared__ uint32_t red[kQuantThreads / 64][3];
  const uint32_t gtid = blockIdx.x * kQuantThreads + threadIdx.x;
  const uint32_t gstride = gridDim.x * kQuantThreads;
  const uint32_t n8 = (uint32_t)a.T * (uint32_t)a.row8;
  DevState* st = a.st;
  uint4 w[3];
  if (threadIdx.x == 0) {
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const float d = descale_from_amax(st->static_values[x]);
      rcp[x] = 1.0 / (double)d;
      if (blockIdx.x == 0) st->descale_used[x] = d;
    }
  }
  __syncthreads();
  const double r[3] = {rcp[0], rcp[1], rcp[2]};
  if ((st->flags & FP8VIT_FLAG_COUNT_SATURATION) != 0u) {
    // Diagnostic: count the clamped elements; one atomic add per tensor and workgroup.
    uint32_t sat[3] = {0u, 0u, 0u};
    quantize_all<CONTIG, false, false, true>(a, n8, r, gtid, gstride, w, sat);
    block_sum3(sat, red);
    if (threadIdx.x == 0) {
#pragma unroll
      for (int x = 0; x < 3; ++x)
        if (sat[x] != 0u) atomicAdd(&st->saturated[x], (unsigned long long)sat[x]);
    }
  } else {
    quantize_all<CONTIG, false, false, false>(a, n8, r, gtid, gstride, w, nullptr);
  }
}

// Dynamic pass 1: quantize at the descales of the window over the other 15
// ring slots and leave per-block partial maxima (and clamp counts) in the
// state. Reads the ring only; block 0 also records the window for pass 2.
template <bool CONTIG>
__global__ __launch_bounds__(kQuantThreads) void quant_dyn_kernel(QuantArgs a) {
  __shared__ double rcp[3];
  __shared__ uint32_t red[kQuantThreads / 64][3];
  __shared__ uint32_t red_sat[kQuantThreads / 64][3];
  const uint32_t gtid = blockIdx.x * kQuantThreads + threadIdx.x;
  const uint32_t gstride = gridDim.x * kQuantThreads;
  const uint32_t n8 = (uint32_t)a.T * (uint32_t)a.row8;
  DevState* st = a.st;
  uint4 w[3];
  load3<CONTIG, false, true>(a, gtid, n8, w);   // in flight during the prologue
  if (threadIdx.x < 64) {
    // Window maximum per tensor over the ring slots other than this
    // forward's, reading the ring as it is once the push the previous forward
    // left pending is done (that push goes to slot count % 16 and this
    // forward's slot is the next one). The loads are spread over wave 0 so
    // that they are all in flight at once: lane 16 x + i holds slot i of
    // tensor x.
    const int lane = threadIdx.x, x = (lane >> 4) % 3, i = lane & 15;
    const float ring = st->ring[x][i], pa = st->pending_amax[x];
    const uint32_t count = st->count;
    const bool pend = st->pending != 0u;
    const uint32_t slot_p = count % FP8VIT_RING_SLOTS;
    const uint32_t slot_this = (count + (pend ? 1u : 0u)) % FP8VIT_RING_SLOTS;
    float v = (pend && i == (int)slot_p) ? pa : ring;
    v = (lane < 48 && i != (int)slot_this) ? v : 0.0f;
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    if (lane < 48 && i == 0) {
      rcp[x] = 1.0 / (double)descale_from_amax(v);
      if (blockIdx.x == 0) st->win_other[x] = v;
    }
  }
  __syncthreads();
  const double r[3] = {rcp[0], rcp[1], rcp[2]};
  uint32_t m[3] = {0u, 0u, 0u};
  if ((st->flags & FP8VIT_FLAG_COUNT_SATURATION) != 0u) {
    uint32_t sat[3] = {0u, 0u, 0u};
    dyn_pass1_all<CONTIG, true>(a, n8, r, gtid, gstride, w, m, sat);
    block_sum3(sat, red_sat);
    if (threadIdx.x == 0) *reinterpret_cast<uint4*>(st->sat_part[blockIdx.x]) = make_uint4(sat[0], sat[1], sat[2], 0u);
  } else {
    dyn_pass1_all<CONTIG, false>(a, n8, r, gtid, gstride, w, m, nullptr);
  }
  block_max3(m, red);
  if (threadIdx.x == 0) *reinterpret_cast<uint4*>(st->amax_part[blockIdx.x]) = make_uint4(m[0], m[1], m[2], 0u);
}

// Dynamic pass 2: every block reduces pass 1's partials to this forward's
// amax and the true descales, max(window, amax) / 448 with the floor. Block
// 0's first thread does the bookkeeping: the previous forward's pending push,
// this forward's amax as pending, the descales in use and, when counting,
// pass 1's clamp counts of the tensors that stand. A tensor whose descale
// differs from pass 1's is quantized again by all blocks.
template <bool CONTIG>
__global__ __launch_bounds__(kQuantThreads) void quant_fix_kernel(QuantArgs a) {
  __shared__ double rcp[3];
  __shared__ uint32_t redo_sh;
  __shared__ uint32_t red[kQuantThreads / 64][3];
  __shared__ uint32_t red_sat[kQuantThreads / 64][3];
  DevState* st = a.st;
  const bool count_sat = (st->flags & FP8VIT_FLAG_COUNT_SATURATION) != 0u;
  // Everything the bookkeeping reads, loaded before the reduction so that the
  // loads overlap it (only block 0's first thread writes the state below).
  float wo[3], pa[3] = {0.0f, 0.0f, 0.0f};
  uint32_t count = 0u, pend = 0u;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int x = 0; x < 3; ++x) wo[x] = st->win_other[x];
    if (blockIdx.x == 0) {
#pragma unroll
      for (int x = 0; x < 3; ++x) pa[x] = st->pending_amax[x];
      count = st->count;
      pend = st->pending;
    }
  }
  uint32_t m[3] = {0u, 0u, 0u}, sat[3] = {0u, 0u, 0u};
  for (int b = threadIdx.x; b < a.amax_blocks; b += kQuantThreads) {
    const uint4 part = *reinterpret_cast<const uint4*>(st->amax_part[b]);
    m[0] = max(m[0], part.x);
    m[1] = max(m[1], part.y);
    m[2] = max(m[2], part.z);
    if (count_sat && blockIdx.x == 0) {
      const uint4 sp = *reinterpret_cast<const uint4*>(st->sat_part[b]);
      sat[0] += sp.x;
      sat[1] += sp.y;
      sat[2] += sp.z;
    }
  }
  block_max3(m, red);
  if (count_sat && blockIdx.x == 0) block_sum3(sat, red_sat);
  if (threadIdx.x == 0) {
    float amax[3], d[3];
    uint32_t redo = 0u;
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      amax[x] = __uint_as_float(m[x] << 16);
      d[x] = descale_from_amax(amax[x] > wo[x] ? amax[x] : wo[x]);
      if ((a.quant_mask >> x & 1u) && d[x] != descale_from_amax(wo[x])) redo |= 1u << x;
      rcp[x] = 1.0 / (double)d[x];
    }
    redo_sh = redo;
    if (blockIdx.x == 0) {
      // the previous forward's pending push (ring_push_pending, from the
      // values loaded above), then this forward's amax as pending
      if (pend != 0u) {
#pragma unroll
        for (int x = 0; x < 3; ++x) st->ring[x][count % FP8VIT_RING_SLOTS] = pa[x];
        st->count = count + 1u;
      }
      record_pending(st, amax, d);
      if (count_sat) {
#pragma unroll
        for (int x = 0; x < 3; ++x)
          if (!(redo >> x & 1u) && sat[x] != 0u) atomicAdd(&st->saturated[x], (unsigned long long)sat[x]);
      }
    }
  }
  __syncthreads();
  const uint32_t redo = redo_sh;
  if (redo == 0u) return;
  QuantArgs ar = a;
  ar.quant_mask = redo;
  const double r[3] = {rcp[0], rcp[1], rcp[2]};
  const uint32_t gtid = blockIdx.x * kQuantThreads + threadIdx.x;
  const uint32_t gstride = gridDim.x * kQuantThreads;
  const uint32_t n8 = (uint32_t)a.T * (uint32_t)a.row8;
  uint4 w[3];
  if (count_sat) {
    uint32_t cnt[3] = {0u, 0u, 0u};
    quantize_all<CONTIG, true, false, true>(ar, n8, r, gtid, gstride, w, cnt);
    __syncthreads();   // red_sat may still be read by block 0's sum above
    block_sum3(cnt, red_sat);
    if (threadIdx.x == 0) {
#pragma unroll
      for (int x = 0; x < 3; ++x)
        if ((redo >> x & 1u) && cnt[x] != 0u) atomicAdd(&st->saturated[x], (unsigned long long)cnt[x]);
    }
  } else {
    quantize_all<CONTIG, true, false, false>(ar, n8, r, gtid, gstride, w, nullptr);
  }
}

// Block-scaled (MX) e4m3 quantization of one tensor (Q or K of the
// block-scaled variant; FlashInfer PR 5283 analysis, Code analysis section 1:
// a scale per block of the head dimension from the block's amax over the
// element format's largest value). Per (token, head, 32-element block of
// head_dim; a trailing partial block is its own block):
//   s = the smallest integer with 448 * 2^s >= block amax (-127 for a zero or
//       subnormal-only block; never above 120 for finite bf16 inputs),
//   code_i = e4m3 RNE of clamp(x_i * 2^-s, +-448) (the product is exact),
//   scale byte = s + 127 (E8M0), four bytes per (token, head), unused ones 0.
// From the bf16 bits of the amax 2^E * (1 + m/128): 448 * 2^(E-8) = 1.75 * 2^E,
// so s = E - 8 when m <= 96 (1 + m/128 <= 1.75) and E - 7 otherwise.
//
// Q and K in one launch. A wave takes kMxTiles groups of whole (token, head)
// rows of each tensor; a group is D/8 16-byte chunks per row (hd72: 7 rows =
// 63 chunks, lane 63 idle; hd128: 4 rows = 64), lane l on chunk l, so the
// loads and the code stores of a wave are contiguous. All 2 * kMxTiles loads
// of a lane are issued before any conversion. A block's maximum is the
// maximum over its adjacent lanes (4, or 1 for hd72's third block).
constexpr int kMxTiles = 2;

template <int D>
__device__ __forceinline__ void mx_quant_chunk(uint4 w, int lane, int jj, bool active, int64_t row,
                                               uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int b = jj >> 2;                                   // block of this chunk
  const int nchunks = (D == 72 && b == 2) ? 1 : 4;         // chunks in that block
  const int g0 = lane - (jj & 3);                          // the block's first lane
  const uint32_t m = chunk_absmax_bits(w);
  uint32_t bm = m;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t o = (uint32_t)__shfl((int)m, g0 + k, 64);
    bm = k < nchunks ? max(bm, o) : bm;
  }
  const int efield = (int)(bm >> 7), mant = (int)(bm & 0x7f);
  const int sexp = efield == 0 ? -127 : max(efield - 127 - 8 + (mant > 96 ? 1 : 0), -127);
  const float rs = __uint_as_float((uint32_t)(127 - sexp) << 23);   // 2^-s, a normal float for s in [-127, 120]
  if (!active) return;
  const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
  uint32_t out[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const float y0 = __builtin_amdgcn_fmed3f(__uint_as_float(bf16_lo(wv[2 * hh])) * rs, -kFp8Max, kFp8Max);
    const float y1 = __builtin_amdgcn_fmed3f(__uint_as_float(bf16_hi(wv[2 * hh])) * rs, -kFp8Max, kFp8Max);
    const float y2 = __builtin_amdgcn_fmed3f(__uint_as_float(bf16_lo(wv[2 * hh + 1])) * rs, -kFp8Max, kFp8Max);
    const float y3 = __builtin_amdgcn_fmed3f(__uint_as_float(bf16_hi(wv[2 * hh + 1])) * rs, -kFp8Max, kFp8Max);
    const int p = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
    out[hh] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, p, true);
  }
  *reinterpret_cast<uint2*>(codes + row * D + 8 * jj) = make_uint2(out[0], out[1]);
  if ((jj & 3) == 0) {
    scales[row * 4 + b] = (uint8_t)(sexp + 127);
    if (D == 72 && b == 2) scales[row * 4 + 3] = 0;
  }
}

template <int D>
__global__ __launch_bounds__(256) void mx_quant_kernel(MxArgs a) {
  constexpr int CPR = D / 8;      // chunks per row
  constexpr int RPW = 64 / CPR;   // rows per group
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int r = lane / CPR, jj = lane - r * CPR;   // row within a group, chunk within the row
  const int64_t nrows = (int64_t)a.T * a.H;
  uint4 w[2][kMxTiles];
  int64_t rows[kMxTiles];
  bool active[kMxTiles];
#pragma unroll
  for (int k = 0; k < kMxTiles; ++k) {
    rows[k] = (wave * kMxTiles + k) * RPW + r;
    active[k] = r < RPW && rows[k] < nrows;
    const int64_t t = active[k] ? rows[k] / a.H : 0, h = active[k] ? rows[k] - t * a.H : 0;
#pragma unroll
    for (int z = 0; z < 2; ++z)
      w[z][k] = active[k] ? *reinterpret_cast<const uint4*>(a.x[z] + t * a.ld[z] + h * D + 8 * jj)
                          : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int z = 0; z < 2; ++z)
#pragma unroll
    for (int k = 0; k < kMxTiles; ++k) mx_quant_chunk<D>(w[z][k], lane, jj, active[k], rows[k], a.codes[z], a.scales[z]);
}

hipError_t launch_quantize_mx(const MxArgs& a, int32_t d, hipStream_t s) {
  const int64_t rows = (int64_t)a.T * a.H;
  if (rows == 0) return hipSuccess;
  const int rpw = d == 72 ? 64 / 9 : 64 / 16;
  const int64_t waves = (rows + (int64_t)rpw * kMxTiles - 1) / ((int64_t)rpw * kMxTiles);
  const int64_t blocks = (waves + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (d == 72)
    hipLaunchKernelGGL(mx_quant_kernel<72>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else if (d == 128)
    hipLaunchKernelGGL(mx_quant_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs& a, bool dynamic, hipStream_t s) {
  const int cus = device_cus();
  if (cus == 0) return hipErrorInvalidDevice;
  const bool contig = a.ld[0] == 8LL * a.row8 && a.ld[1] == 8LL * a.row8 && a.ld[2] == 8LL * a.row8;
  const uint64_t n8 = (uint64_t)a.T * (uint64_t)a.row8;
  uint64_t g = (n8 + (uint64_t)kQuantThreads - 1) / (uint64_t)kQuantThreads;
  if (g < 1) g = 1;
  const dim3 block(kQuantThreads);
  if (!dynamic) {
    const uint64_t gs = g < (uint64_t)cus * kGridPerCu ? g : (uint64_t)cus * kGridPerCu;
    if (contig)
      hipLaunchKernelGGL(quant_static_kernel<true>, dim3((unsigned)gs), block, 0, s, a);
    else
      hipLaunchKernelGGL(quant_static_kernel<false>, dim3((unsigned)gs), block, 0, s, a);
    return hipGetLastError();
  }
  uint64_t g1 = g < (uint64_t)cus * kGridPerCuDynamic ? g : (uint64_t)cus * kGridPerCuDynamic;
  if (g1 > (uint64_t)kAmaxSlots) g1 = kAmaxSlots;
  const uint64_t g2 = g < (uint64_t)cus ? g : (uint64_t)cus;
  QuantArgs ad = a;
  ad.amax_blocks = (int32_t)g1;
  if (contig)
    hipLaunchKernelGGL(quant_dyn_kernel<true>, dim3((unsigned)g1), block, 0, s, ad);
  else
    hipLaunchKernelGGL(quant_dyn_kernel<false>, dim3((unsigned)g1), block, 0, s, ad);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (contig)
    hipLaunchKernelGGL(quant_fix_kernel<true>, dim3((unsigned)g2), block, 0, s, ad);
  else
    hipLaunchKernelGGL(quant_fix_kernel<false>, dim3((unsigned)g2), block, 0, s, ad);
  return hipGetLastError();
}

}  // namespace fp8vit
