// Varlen non-causal FP8 flash attention for gfx950 (CDNA4).
//
// What it computes (vLLM page "FP8 ViT Encoder Attention": FP8 Q/K/V with one
// scale per tensor; packed variable-length image/video batches handled
// natively): for every segment [cu[i], cu[i+1]) and head h,
//     O = softmax(dq*dk*scale * Q8 K8^T) (dv * V8),
// with Q8/K8/V8 the e4m3 codes and dq/dk/dv the per-tensor descales.
//
// Design (MI355X-first, not a port of any kernel on the pages):
//  * One workgroup = 4 waves = 128 queries of one (segment, head); each wave
//    owns 32 queries (two 16-query MFMA column blocks).
//  * K/V tiles of 128 keys are staged in LDS. S^T = K Q^T is computed with
//    v_mfma_f32_16x16x128_f8f6f4 (K rows as the A operand, Q as B), d padded to
//    128 with zeros for head_dim 72. The A rows are permuted so that lane group
//    g ends up holding keys 32g..32g+31 of its query: the fp32 S^T registers
//    convert in place into the B operand of the next product, no LDS round trip.
//  * O^T = V^T P^T on the same MFMA: V^T comes from row-major V in LDS through
//    ds_read_b64_tr_b8 (byte transpose on read). Column 72 of the hd72 V tile
//    holds 1.0, so the same MFMAs accumulate the row sum of the probabilities
//    actually used; hd128 appends a constant ones block.
//  * Online softmax in exp2 units with a lazy reference max: O is rescaled only
//    when a row max grows by more than 1.75, and P~ = 2^7 * exp2(t - m_ref) stays
//    below 2^8.75 < 448, inside e4m3's range.
//  * P~ goes to the FP8 MFMA in two e4m3 terms, hi = e4m3(P~) and
//    lo = e4m3(P~ - hi): a single e4m3 term adds ~2.5% relative error to O.
//  * Work items are (head, query tile); consecutive items of one head are
//    mapped to the same XCD so K/V re-reads hit that XCD's L2.
#include "fp8vit_internal.h"

namespace fp8vit {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBMW = 32;             // queries per wave
constexpr int kBM = kWaves * kBMW;   // queries per workgroup
constexpr int kBN = 128;             // keys per tile
constexpr float kExpBias = 7.0f;     // P~ = 2^7 * exp2(t - m_ref)
constexpr float kLazy = 1.75f;       // log2 growth of the max tolerated before rescaling
constexpr float kLog2e = 1.4426950408889634f;

template <int D> struct Cfg;
// KS/VS: LDS row strides (bytes) chosen so 16 lanes reading 16 B from 16 rows,
// or 8 rows x 16 B for the transpose read, touch distinct banks.
// NCB: 16-column blocks of O^T including the ones column. CH x CHB: global
// chunks per K/V row.
template <> struct Cfg<72> {
  static constexpr int KS = 112, VS = 80, NCB = 5, CH = 9, CHB = 8, ONES_CB = 4, ONES_LANE0 = 32;
};
template <> struct Cfg<128> {
  static constexpr int KS = 144, VS = 144, NCB = 9, CH = 8, CHB = 16, ONES_CB = 8, ONES_LANE0 = 0;
};

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kBN * C::KS];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds[kBN * C::VS];

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

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, i16 = lane & 15;

  // ---- constant parts of the LDS tiles: zero padding, ones column ----
  for (int r = tid; r < kBN; r += kThreads) {
#pragma unroll
    for (int b = D; b < C::KS; b += 8) *reinterpret_cast<uint2*>(k_lds + r * C::KS + b) = make_uint2(0u, 0u);
#pragma unroll
    for (int b = D; b < C::VS; b += 8)
      *reinterpret_cast<uint2*>(v_lds + r * C::VS + b) = make_uint2((D == 72 && b == 72) ? 0x38u : 0u, 0u);
  }

  const float dq = a.st->descale_used[0], dk = a.st->descale_used[1], dv = a.st->descale_used[2];
  const float cexp = a.softmax_scale * dq * dk * kLog2e;   // raw score -> log2 units

  // ---- Q operands (B of S^T): lane holds query i16 of its block, d bytes 32g.. ----
  v8i qop[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    qop[qb] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    const int qr = q0 + wave * kBMW + qb * 16 + i16;
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
        uint4 u0 = *reinterpret_cast<const uint4*>(src + 32 * g);
        uint4 u1 = *reinterpret_cast<const uint4*>(src + 32 * g + 16);
        qop[qb] = v8i{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
      }
    }
  }

  v4f o[2][C::NCB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int cb = 0; cb < C::NCB; ++cb) o[qb][cb] = v4f{0.f, 0.f, 0.f, 0.f};
  float mref[2] = {-INFINITY, -INFINITY};
  const v8i ones_op = (i16 == 0) ? v8i{0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838,
                                       0x38383838, 0x38383838}
                                 : v8i{0, 0, 0, 0, 0, 0, 0, 0};
  const v4f zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int kv0 = 0; kv0 < L; kv0 += kBN) {
    // ---- stage K and V rows kv0..kv0+127 (zeros past the segment end) ----
    __syncthreads();
    for (int c = tid; c < kBN * C::CH; c += kThreads) {
      const int row = c / C::CH, part = c - row * C::CH;
      const int key = kv0 + row;
      if (C::CHB == 8) {
        uint2 kk = make_uint2(0u, 0u), vv = make_uint2(0u, 0u);
        if (key < L) {
          const int64_t off = ((int64_t)(s0 + key) * a.H + h) * D + 8 * part;
          kk = *reinterpret_cast<const uint2*>(a.k8 + off);
          vv = *reinterpret_cast<const uint2*>(a.v8 + off);
        }
        *reinterpret_cast<uint2*>(k_lds + row * C::KS + 8 * part) = kk;
        *reinterpret_cast<uint2*>(v_lds + row * C::VS + 8 * part) = vv;
      } else {
        uint4 kk = make_uint4(0u, 0u, 0u, 0u), vv = make_uint4(0u, 0u, 0u, 0u);
        if (key < L) {
          const int64_t off = ((int64_t)(s0 + key) * a.H + h) * D + 16 * part;
          kk = *reinterpret_cast<const uint4*>(a.k8 + off);
          vv = *reinterpret_cast<const uint4*>(a.v8 + off);
        }
        *reinterpret_cast<uint4*>(k_lds + row * C::KS + 16 * part) = kk;
        *reinterpret_cast<uint4*>(v_lds + row * C::VS + 16 * part) = vv;
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T: 8 key tiles x 2 query blocks ----
    float s[2][8][4];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int krow = 32 * (i16 >> 2) + 4 * t + (i16 & 3);
      const int koff = (D == 72 && g == 3) ? 80 : 32 * g;
      const uint8_t* kp = k_lds + krow * C::KS + koff;
      const uint4 k0 = *reinterpret_cast<const uint4*>(kp);
      const uint4 k1 = *reinterpret_cast<const uint4*>(kp + 16);
      const v8i kop = {(int)k0.x, (int)k0.y, (int)k0.z, (int)k0.w, (int)k1.x, (int)k1.y, (int)k1.z, (int)k1.w};
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const v4f acc = mfma_fp8(kop, qop[qb], zero4);
#pragma unroll
        for (int r = 0; r < 4; ++r) s[qb][t][r] = acc[r];
      }
    }
    // keys of this lane: kv0 + 32g + 4t + r
    if (kv0 + kBN > L) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (kv0 + 32 * g + 4 * t + r >= L) s[qb][t][r] = -INFINITY;
    }

    // ---- row max (4 lane groups share a query) and lazy rescale ----
    float mt[2];
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float m = s[qb][0][0];
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, s[qb][t][r]);
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      mt[qb] = m * cexp;
      need = need || (mt[qb] > mref[qb] + kLazy);
    }
    if (__ballot(need) != 0ull) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float mn = fmaxf(mref[qb], mt[qb]);
        const float alpha = __builtin_amdgcn_exp2f(mref[qb] - mn);
        mref[qb] = mn;
#pragma unroll
        for (int cb = 0; cb < C::NCB; ++cb) o[qb][cb] *= alpha;
      }
    }

    // ---- P~ in two e4m3 terms, packed straight into the B operand layout ----
    v8i phi[2], plo[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float nb = kExpBias - mref[qb];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[qb][t][0], cexp, nb));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[qb][t][1], cexp, nb));
        const float p2 = __builtin_amdgcn_exp2f(fmaf(s[qb][t][2], cexp, nb));
        const float p3 = __builtin_amdgcn_exp2f(fmaf(s[qb][t][3], cexp, nb));
        int hi = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, hi, true);
        const auto h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
        const auto h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
        int lo = __builtin_amdgcn_cvt_pk_fp8_f32(p0 - h01[0], p1 - h01[1], 0, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(p2 - h23[0], p3 - h23[1], lo, true);
        phi[qb][t] = hi;
        plo[qb][t] = lo;
      }
    }

    // ---- O^T += V^T P^T (hi and lo terms) ----
#pragma unroll
    for (int cb = 0; cb < C::NCB; ++cb) {
      v8i vop;
      if (D == 128 && cb == 8) {
        vop = ones_op;
      } else {
#pragma unroll
        for (int sidx = 0; sidx < 4; ++sidx) {
          const uint8_t* vp = v_lds + (32 * g + 8 * sidx + (i16 >> 1)) * C::VS + 16 * cb + 8 * (i16 & 1);
          const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vp));
          vop[2 * sidx] = r[0];
          vop[2 * sidx + 1] = r[1];
        }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        o[qb][cb] = mfma_fp8(vop, phi[qb], o[qb][cb]);
        o[qb][cb] = mfma_fp8(vop, plo[qb], o[qb][cb]);
      }
    }
  }

  // ---- epilogue: divide by the row sum (ones column), scale by dv, bf16 ----
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lsum = __shfl(o[qb][C::ONES_CB][0], C::ONES_LANE0 + i16, 64);
    const float f = dv / lsum;
    const int qr = q0 + wave * kBMW + qb * 16 + i16;
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

int attn_block_m() { return kBM; }

hipError_t launch_attn(const AttnArgs& a, int head_dim, int total_tokens, hipStream_t s) {
  const int64_t items = (int64_t)a.H * a.ntiles_ub;
  const int64_t grid = ((items + 7) / 8) * 8;
  if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  (void)total_tokens;
  if (head_dim == 72)
    hipLaunchKernelGGL(attn_kernel<72>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(attn_kernel<128>, dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace fp8vit
