// Varlen non-causal FP8 flash attention for gfx950 (CDNA4).
//
// What it computes (vLLM page "FP8 ViT Encoder Attention": FP8 Q/K/V with one
// scale per tensor; packed variable-length image/video batches handled
// natively): for every segment [cu[i], cu[i+1]) and head h,
//     O = softmax(dq*dk*scale * Q8 K8^T) (dv * V8),
// with Q8/K8/V8 the e4m3 codes and dq/dk/dv the per-tensor descales.
//
// Design (MI355X-first, not a port of any kernel on the pages):
//  * A workgroup owns 128 queries of one (segment, head): WAVES waves of
//    QB 16-query MFMA column blocks each (8x1 or 4x2).
//  * K/V tiles of 128 keys are double-buffered in LDS. The next tile's global
//    loads are issued into registers when a tile starts and stored into the
//    other buffer halfway through it: one barrier per tile, global latency
//    hidden behind the MFMA/softmax work.
//  * S^T = K Q^T on v_mfma_f32_16x16x128_f8f6f4 (K rows as the A operand, Q as
//    B), d zero-padded to 128 for head_dim 72. A rows are permuted so that lane
//    group g holds keys 32g..32g+31 of its query: the fp32 S^T registers turn
//    in place into the B operand of the next product (no LDS round trip).
//  * O^T = V^T P^T on the same MFMA; V^T comes from row-major V in LDS through
//    ds_read_b64_tr_b8 (byte transpose on read). Column 72 of the hd72 V tile
//    holds 1.0, so the same MFMAs accumulate the row sum of the probabilities
//    actually used; hd128 appends a constant ones block.
//  * One-pass online softmax in exp2 units with a lazy reference max m_ref:
//    P~ = 2^7 * exp2(t - m_ref) is formed right after each 16-key S^T block
//    while a per-lane running max is kept; S^T of the next block is already on
//    the matrix core. Only if some score of the tile exceeds m_ref + 1.75
//    (then P~ could pass 448, e4m3's largest value) is the row max reduced
//    across lanes, O rescaled and the tile's probabilities recomputed. The
//    first tile always takes that path (m_ref = -inf).
//  * P~ goes to the FP8 MFMA as two e4m3 terms, hi = e4m3(P~) and
//    lo = e4m3(P~ - hi): a single e4m3 term adds ~2.5% relative error to O.
//  * Work items are (head, query tile); consecutive items of one head are
//    mapped to the same XCD so that K/V re-reads hit that XCD's L2.
#include <type_traits>

#include "fp8vit_internal.h"

namespace fp8vit {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) v4i lds_v4i;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kBN = 128;             // keys per tile
constexpr float kExpBias = 7.0f;     // P~ = 2^7 * exp2(t - m_ref)
constexpr float kLazy = 1.75f;       // log2 growth of the max tolerated before rescaling
constexpr float kLog2e = 1.4426950408889634f;

template <int D> struct Cfg;
// KS/VS: LDS row strides in bytes. NCB: 16-column blocks of O^T including the
// ones column. CHB x ROWCH: bytes per global load x loads per K/V row.
// WAVES x QB x 16 = BM queries per workgroup.
// hd72: K rows are 80 bytes (72 + 8 zero bytes); the d-padding lanes of the
// S^T operand read past their row into the next one, which only meets the
// zero bytes of the Q operand, or read a 32-byte zero block after the tile.
template <> struct Cfg<72> {
  static constexpr int KS = 80, VS = 80, NCB = 5, CHB = 8, ROWCH = 9, ONES_CB = 4, ONES_LANE0 = 32;
  static constexpr int WAVES = 4, QB = 1, MIN_WAVES_PER_EU = 3, BM = 64;
};
template <> struct Cfg<128> {
  static constexpr int KS = 144, VS = 144, NCB = 9, CHB = 16, ROWCH = 8, ONES_CB = 8, ONES_LANE0 = 0;
  static constexpr int WAVES = 8, QB = 1, MIN_WAVES_PER_EU = 2, BM = 128;
};

// LDS placement of a tile's rows.
//  K: key k sits in row 4*(k%32) + k/32, so the 16 keys of one S^T block
//     (32a + 4t + b, a, b = 0..3) occupy 16 consecutive rows 16t..16t+15,
//     whose 16-byte pieces fall on distinct banks.
//  V: key k sits at byte k*VS + 64*(k/32); the 64-byte gap between 32-key
//     groups spreads the four lane groups of a transpose read over the banks.
__device__ __forceinline__ int k_row(int key) { return 4 * (key & 31) + (key >> 5); }
template <int D> __device__ __forceinline__ int v_off(int key) { return key * Cfg<D>::VS + 64 * (key >> 5); }

template <int D> struct Stage {
  static constexpr int THREADS = 64 * Cfg<D>::WAVES;
  // Staging: TPR threads per K/V row, each moving CPT chunks starting at
  // chunk P0_STEP * (tid % TPR) (neighbours may overlap by a chunk; both then
  // store the same bytes).
  static constexpr int TPR = THREADS / kBN;
  static constexpr int CPT = (Cfg<D>::ROWCH + TPR - 1) / TPR;
  static constexpr int P0_STEP = TPR > 1 ? (Cfg<D>::ROWCH - CPT) / (TPR - 1) : 0;
  static_assert(TPR >= 1 && THREADS % kBN == 0, "staging shape");
  static_assert(P0_STEP * (TPR - 1) + CPT == Cfg<D>::ROWCH && P0_STEP <= CPT, "staging covers each row");
  static constexpr int KZERO = kBN * Cfg<D>::KS;                       // 32 bytes after the rows
  static constexpr int KBUF = KZERO + 32, VBUF = kBN * Cfg<D>::VS + 64 * (kBN / 32 - 1);
  using chunk_t = typename std::conditional<Cfg<D>::CHB == 8, u32x2, u32x4>::type;
};

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Global -> register prefetch of this thread's chunks of one K/V row of a
// tile. Rows past the segment end read the last valid row: those keys are
// masked or multiplied by P = 0. kg/vg point at this thread's first chunk of
// key 0 of the segment for this head.
template <int D>
__device__ __forceinline__ void prefetch_row(const uint8_t* kg, const uint8_t* vg, uint32_t row_stride, int key,
                                             typename Stage<D>::chunk_t* kr, typename Stage<D>::chunk_t* vr) {
  using S = Stage<D>;
  const uint32_t off = (uint32_t)key * row_stride;
#pragma unroll
  for (int i = 0; i < S::CPT; ++i) {
    kr[i] = *reinterpret_cast<const typename S::chunk_t*>(kg + off + Cfg<D>::CHB * i);
    vr[i] = *reinterpret_cast<const typename S::chunk_t*>(vg + off + Cfg<D>::CHB * i);
  }
}

template <int D>
__device__ __forceinline__ void commit_row(uint8_t* kdst, uint8_t* vdst, const typename Stage<D>::chunk_t* kr,
                                           const typename Stage<D>::chunk_t* vr) {
  using S = Stage<D>;
#pragma unroll
  for (int i = 0; i < S::CPT; ++i) {
    *reinterpret_cast<typename S::chunk_t*>(kdst + Cfg<D>::CHB * i) = kr[i];
    *reinterpret_cast<typename S::chunk_t*>(vdst + Cfg<D>::CHB * i) = vr[i];
  }
}

// A operand of S^T block t: lane row i16 <-> key 32*(i16/4) + 4t + i16%4, d bytes
// 32g..32g+31. `kl` is the lane's byte offset for t = 0 (k_lane_offset); block t
// adds 16 rows. hd72: lane groups 2 and 3 read bytes 64..95 (8 data bytes, then
// bytes that only meet zero bytes of the Q operand).
template <int D>
__device__ __forceinline__ int k_lane_offset(int g, int i16) {
  const int krow = 4 * (i16 & 3) + (i16 >> 2);            // = k_row(32*(i16/4) + i16%4)
  return krow * Cfg<D>::KS + (D == 72 ? min(32 * g, 64) : 32 * g);
}
template <int D>
__device__ __forceinline__ v8i k_operand(const lds_u8* kl, int t) {
  const lds_u8* kp = kl + 16 * t * Cfg<D>::KS;
  const v4i k0 = *(const lds_v4i*)(kp);
  const v4i k1 = *(const lds_v4i*)(kp + 16);
  return __builtin_shufflevector(k0, k1, 0, 1, 2, 3, 4, 5, 6, 7);
}

// A operand of O^T block cb: lane row i16 <-> V column 16cb + i16, keys 32g..32g+31,
// gathered from row-major V by the byte-transposing LDS read. `vl` is the lane's
// byte offset (v_lane_offset); the 8-key steps and the column block are constants.
template <int D>
__device__ __forceinline__ int v_lane_offset(int g, int i16) {
  return v_off<D>(32 * g + (i16 >> 1)) + 8 * (i16 & 1);
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

// Two e4m3 terms of four probabilities P~ = exp2(s*c + nb), packed as one
// dword of the P^T operand (hi) and one of the correction term (lo).
__device__ __forceinline__ int2 probs_to_fp8(const v4f& s, float c, float nb) {
  const float p0 = __builtin_amdgcn_exp2f(fmaf(s[0], c, nb));
  const float p1 = __builtin_amdgcn_exp2f(fmaf(s[1], c, nb));
  const float p2 = __builtin_amdgcn_exp2f(fmaf(s[2], c, nb));
  const float p3 = __builtin_amdgcn_exp2f(fmaf(s[3], c, nb));
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
  h = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, h, true);
  const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
  const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
  int l = __builtin_amdgcn_cvt_pk_fp8_f32(p0 - h01[0], p1 - h01[1], 0, false);
  l = __builtin_amdgcn_cvt_pk_fp8_f32(p2 - h23[0], p3 - h23[1], l, true);
  return make_int2(h, l);
}

template <int D>
__global__ __launch_bounds__(64 * Cfg<D>::WAVES) __attribute__((amdgpu_waves_per_eu(Cfg<D>::MIN_WAVES_PER_EU)))
void attn_kernel(AttnArgs a) {
  using C = Cfg<D>;
  using S = Stage<D>;
  constexpr int QB = C::QB;
  constexpr int BMW = 16 * QB;
  constexpr int kBM = C::BM;
  static_assert(C::WAVES * BMW == kBM, "block shape");
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[2 * S::KBUF];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[3 * S::VBUF];

  // ---- work item: XCD-grouped (head, query tile) -> segment by prefix scan ----
  const int G = gridDim.x;
  const int w = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int h = w / a.ntiles_ub;
  int tile = w - h * a.ntiles_ub;
  if (h >= a.H) return;
  int s0 = 0, L = -1;
  for (int i = 0; i < a.nseg; ++i) {
    const int b0 = a.cu[i], b1 = a.cu[i + 1];
    const int n = (b1 - b0 + kBM - 1) / kBM;
    if (tile < n) { s0 = b0; L = b1 - b0; break; }
    tile -= n;
  }
  if (L <= 0) return;
  const int q0 = tile * kBM;
  const int ntiles = (L + kBN - 1) / kBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, i16 = lane & 15;

  // ---- staging geometry; first K/V tile in flight while the constants are written ----
  const int srow = tid / S::TPR;
  const int schunk = S::P0_STEP * (tid % S::TPR);
  const uint32_t row_stride = (uint32_t)a.H * D;
  const int64_t seg_off = ((int64_t)s0 * a.H + h) * D + Cfg<D>::CHB * schunk;
  const uint8_t* kg = a.k8 + seg_off;
  const uint8_t* vg = a.v8 + seg_off;
  const int k_stage = k_row(srow) * C::KS + Cfg<D>::CHB * schunk;   // LDS offsets within a buffer
  const int v_stage = v_off<D>(srow) + Cfg<D>::CHB * schunk;
  typename S::chunk_t kr[S::CPT], vr[S::CPT];
  prefetch_row<D>(kg, vg, row_stride, min(srow, L - 1), kr, vr);
  for (int r = tid; r < 2 * (kBN + 4); r += S::THREADS) {
    uint8_t* kr0 = k_lds + (r / (kBN + 4)) * S::KBUF;
    const int rr = r % (kBN + 4);
    if (rr < kBN) {
#pragma unroll
      for (int b = D; b < C::KS; b += 8) *reinterpret_cast<uint2*>(kr0 + rr * C::KS + b) = make_uint2(0u, 0u);
    } else {
      *reinterpret_cast<uint2*>(kr0 + S::KZERO + 8 * (rr - kBN)) = make_uint2(0u, 0u);
    }
  }
  for (int r = tid; r < 3 * kBN; r += S::THREADS) {
    uint8_t* vr0 = v_lds + (r / kBN) * S::VBUF + v_off<D>(r % kBN);
#pragma unroll
    for (int b = 0; b < C::VS; b += 8)
      *reinterpret_cast<uint2*>(vr0 + b) = make_uint2((D == 72 && b == 72) ? 0x38u : 0u, 0u);
  }

  const float dq = a.st->descale_used[0], dk = a.st->descale_used[1], dv = a.st->descale_used[2];
  const float cexp = a.softmax_scale * dq * dk * kLog2e;   // raw score -> log2 units (> 0)

  // ---- Q operands (B of S^T): lane holds query i16 of its block, d bytes 32g.. ----
  v8i qop[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    qop[qb] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    const int qr = q0 + wave * BMW + qb * 16 + i16;
    if (qr < L) {
      const uint8_t* src = a.q8 + ((int64_t)(s0 + qr) * a.H + h) * D;
      if (D == 72) {
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

  __syncthreads();   // zero fill above overlaps the rows stored next
  commit_row<D>(k_lds + k_stage, v_lds + v_stage, kr, vr);
  __syncthreads();
  const int kl_lane = k_lane_offset<D>(g, i16);
  const int vl_lane = v_lane_offset<D>(g, i16);

  // P of the previous tile: its O^T += V^T P^T products are interleaved with
  // the softmax VALU work of the current tile (matrix core and VALU overlap
  // inside each wave). V is triple-buffered so that the previous tile's V
  // stays in LDS while the next one is being stored. Before the first tile the
  // "previous" P is zero and its V buffer holds zeros, so the products add 0.
  v8i phi_prev[QB], plo_prev[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) phi_prev[qb] = plo_prev[qb] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  const v8i ones_op = (i16 == 0) ? v8i{0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838,
                                       0x38383838, 0x38383838}
                                 : v8i{0, 0, 0, 0, 0, 0, 0, 0};
  auto pv_block = [&](const lds_u8* vbp, int cb) {
    const v8i vop = (D == 128 && cb == 8) ? ones_op : v_operand<D>(vbp, cb);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      o[qb][cb] = mfma_fp8(vop, phi_prev[qb], o[qb][cb]);
      o[qb][cb] = mfma_fp8(vop, plo_prev[qb], o[qb][cb]);
    }
  };

  // One pass over the 8 S^T blocks of a tile. Template flags keep the
  // unrolled body free of branches: PARTIAL masks keys past the segment end
  // (last tile only), WITH_PV interleaves the previous tile's P.V, COMMIT
  // stores the prefetched next tile after block 3.
  v8i phi[QB], plo[QB];
  float lm[QB];
  auto run_pass = [&](auto partial_c, auto pv_c, auto commit_c, int j) {
    constexpr bool PARTIAL = decltype(partial_c)::value;
    constexpr bool WITH_PV = decltype(pv_c)::value;
    constexpr bool COMMIT = decltype(commit_c)::value;
    const int kv0 = j * kBN;
    // One base register per operand and tile; the per-block steps become
    // immediate offsets of the LDS reads (the empty asm keeps the compiler
    // from hoisting one precomputed address per read out of the loop).
    uint32_t kbase = (uint32_t)((j & 1) * S::KBUF + kl_lane);
    uint32_t vbase = (uint32_t)(((j + 2) % 3) * S::VBUF + vl_lane);
    asm volatile("" : "+v"(kbase), "+v"(vbase));
    const lds_u8* kl = (const lds_u8*)k_lds + kbase;
    const lds_u8* vprev = (const lds_u8*)v_lds + vbase;   // V of tile j-1
    float nb[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      nb[qb] = kExpBias - mref[qb];
      lm[qb] = -INFINITY;
    }
    v8i kop = k_operand<D>(kl, 0);
    v4f sa[QB], sb[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) sa[qb] = mfma_fp8(kop, qop[qb], zero4);
    kop = k_operand<D>(kl, 1);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t + 1 < 8) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) sb[qb] = mfma_fp8(kop, qop[qb], zero4);
        if (t + 2 < 8) kop = k_operand<D>(kl, t + 2);
      }
      if (WITH_PV) {                     // one 16-column block per 16-key block
        if (t < C::NCB) pv_block(vprev, t);
        if (t == 7 && C::NCB > 8) pv_block(vprev, 8);
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (PARTIAL) {
#pragma unroll
          for (int r = 0; r < 4; ++r) sa[qb][r] = (kv0 + 32 * g + 4 * t + r >= L) ? -INFINITY : sa[qb][r];
        }
        lm[qb] = fmaxf(fmaxf(fmaxf(fmaxf(lm[qb], sa[qb][0]), sa[qb][1]), sa[qb][2]), sa[qb][3]);
        const int2 p = probs_to_fp8(sa[qb], cexp, nb[qb]);
        phi[qb][t] = p.x;
        plo[qb][t] = p.y;
        if (t + 1 < 8) sa[qb] = sb[qb];
      }
      // The buffers of the next tile are free since the last barrier: store
      // it early so its registers do not stay live through the pass.
      if (COMMIT && t == 3)
        commit_row<D>(k_lds + ((j + 1) & 1) * S::KBUF + k_stage, v_lds + ((j + 1) % 3) * S::VBUF + v_stage, kr, vr);
    }
  };
  // Overflow check after a pass: a score above its row's threshold means P~
  // may exceed 448. Then reduce the row max over the four lane groups, move
  // the reference max, rescale O (which holds every earlier tile by now) and
  // recompute this tile's probabilities.
  auto need_redo = [&]() {
    // Keep the pass' probabilities computed here, interleaved with its MFMAs,
    // rather than sunk past the branch into the common path.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) asm volatile("" : "+v"(phi[qb]), "+v"(plo[qb]));
    bool over = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) over = over || (lm[qb] > thr[qb]);
    if (__ballot(over) == 0ull) return false;
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
    return true;
  };
  auto shift_p = [&]() {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      phi_prev[qb] = phi[qb];
      plo_prev[qb] = plo[qb];
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

  // full tiles
  for (int j = 0; j + 1 < ntiles; ++j) {
    prefetch_row<D>(kg, vg, row_stride, min((j + 1) * kBN + srow, L - 1), kr, vr);
    run_pass(F_{}, T_{}, T_{}, j);
    if (need_redo()) run_pass(F_{}, F_{}, F_{}, j);
    shift_p();
    __syncthreads();
  }
  // last tile (keys past the segment end masked), then its own P.V
  {
    const int j = ntiles - 1;
    run_pass(T_{}, T_{}, F_{}, j);
    if (need_redo()) run_pass(T_{}, F_{}, F_{}, j);
    shift_p();
    const lds_u8* vlast = (const lds_u8*)v_lds + (j % 3) * S::VBUF + vl_lane;
#pragma unroll
    for (int cb = 0; cb < C::NCB; ++cb) pv_block(vlast, cb);
  }

  // ---- epilogue: divide by the row sum (ones column), scale by dv, bf16 ----
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lsum = __shfl(o[qb][C::ONES_CB][0], C::ONES_LANE0 + i16, 64);
    const float f = dv / lsum;
    const int qr = q0 + wave * BMW + qb * 16 + i16;
    if (qr < L) {
      uint16_t* dst = a.out + (int64_t)(s0 + qr) * a.ld_out + (int64_t)h * D;
#pragma unroll
      for (int cb = 0; cb < C::NCB; ++cb) {
        const int col = 16 * cb + 4 * g;
        if (col + 4 <= D) {
          const v4f x = o[qb][cb] * f;
          uint2 pk;
          pk.x = bf16_rne(x[0]) | (bf16_rne(x[1]) << 16);
          pk.y = bf16_rne(x[2]) | (bf16_rne(x[3]) << 16);
          *reinterpret_cast<uint2*>(dst + col) = pk;
        }
      }
    }
  }
}

int attn_block_m(int head_dim) { return head_dim == 72 ? Cfg<72>::BM : Cfg<128>::BM; }

hipError_t launch_attn(const AttnArgs& a, int head_dim, int total_tokens, hipStream_t s) {
  const int64_t items = (int64_t)a.H * a.ntiles_ub;
  const int64_t grid = ((items + 7) / 8) * 8;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  (void)total_tokens;
  if (head_dim == 72)
    hipLaunchKernelGGL(attn_kernel<72>, dim3((unsigned)grid), dim3(64 * Cfg<72>::WAVES), 0, s, a);
  else
    hipLaunchKernelGGL(attn_kernel<128>, dim3((unsigned)grid), dim3(64 * Cfg<128>::WAVES), 0, s, a);
  return hipGetLastError();
}

}  // namespace fp8vit
