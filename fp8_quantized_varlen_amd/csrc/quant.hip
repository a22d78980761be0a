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
// each whole tensor is reduced first, pushed into the 16-slot ring, and the
// window maximum sets this forward's descale. Two launches: the amax pass
// (whose last block to finish does the ring bookkeeping) and the quantize
// pass, which reads the descales from the state. A single cooperative launch
// with a grid-wide barrier between the passes reads the input once, but on
// MI355X it measured slower at every size: the cooperative launch itself adds
// ~17 us and a barrier across eight XCDs costs several device-scope atomic
// round trips, against ~7 us for re-reading 57 MB (L = 8192, 16 heads, d = 72).
//
// Data layout: bf16 rows of H*d elements with token stride ld; every thread
// moves 16-byte chunks (8 elements) in and 8-byte chunks out, consecutive
// lanes on consecutive chunks (fully coalesced for contiguous inputs).
#include "fp8vit_internal.h"
#include "state_device.h"

namespace fp8vit {

// Quantize pass: one 16-byte chunk of each of Q, K and V per thread and
// iteration, up to 16 workgroups per CU (a small grid with several chunks in
// flight per thread measured 9-14 % slower).
constexpr int kQuantThreads = 512;
constexpr int kUnroll = 1;
constexpr int kGridPerCu = 16;
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
constexpr int kAmaxBlocks = 128;
constexpr int kAmaxUnroll = 4;
__device__ __forceinline__ uint32_t bf16_lo(uint32_t w) { return w << 16; }
__device__ __forceinline__ uint32_t bf16_hi(uint32_t w) { return w & 0xffff0000u; }

// r = RN64(1 / descale), see the header comment.
__device__ __forceinline__ float quant_value(uint32_t fbits, double r) {
  const float q = (float)((double)__uint_as_float(fbits) * r);
  return __builtin_amdgcn_fmed3f(q, -kFp8Max, kFp8Max);
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

// Quantize Q, K and V together: each thread keeps kUnroll chunks of each of
// the three tensors in flight before converting and storing them.
// NT: non-temporal loads and stores. They speed up the quantize pass of
// dynamic mode (which re-reads what the amax pass has just read) by ~10 % and
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
template <bool CONTIG, bool NT>
__device__ __forceinline__ void quantize_all(const QuantArgs& a, uint32_t n8, const double* r, uint32_t gtid,
                                             uint32_t gstride) {
  for (uint32_t base = gtid; base < n8; base += gstride * kUnroll) {
    uint4 w[3][kUnroll];
#pragma unroll
    for (int x = 0; x < 3; ++x)
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t c = base + u * gstride;
        w[x][u] = c < n8 ? ld16<NT>(chunk_src<CONTIG>(a.x[x], a.ld[x], a.row8, c)) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
    for (int x = 0; x < 3; ++x)
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t c = base + u * gstride;
        if (c < n8) st8<NT>(reinterpret_cast<uint2*>(a.y[x]) + c, quant_chunk(w[x][u], r[x]));
      }
  }
}

// Largest |x| bits of each of Q, K, V over this thread's chunks (the same
// chunk pattern as quantize_all), with 3 * kAmaxUnroll loads in flight.
template <bool CONTIG>
__device__ __forceinline__ void absmax_all(const QuantArgs& a, uint32_t n8, uint32_t gtid, uint32_t gstride,
                                           uint32_t m[3]) {
  m[0] = m[1] = m[2] = 0;
  for (uint32_t base = gtid; base < n8; base += gstride * kAmaxUnroll) {
    uint4 w[3][kAmaxUnroll];
#pragma unroll
    for (int x = 0; x < 3; ++x)
#pragma unroll
      for (int u = 0; u < kAmaxUnroll; ++u) {
        const uint32_t c = base + u * gstride;
        w[x][u] = c < n8 ? *chunk_src<CONTIG>(a.x[x], a.ld[x], a.row8, c) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
    for (int x = 0; x < 3; ++x)
#pragma unroll
      for (int u = 0; u < kAmaxUnroll; ++u) m[x] = max(m[x], chunk_absmax_bits(w[x][u]));
  }
}

template <int THREADS>
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < THREADS / 64; ++i) r = max(r, red[i]);
  __syncthreads();
  return r;
}

// Quantize pass. Static mode: the descales come from the stored static
// values (block 0 records them). Dynamic mode: the amax pass already wrote
// them to the state.
template <bool CONTIG, bool DYNAMIC>
__global__ __launch_bounds__(kQuantThreads) void quant_kernel(QuantArgs a) {
  __shared__ double rcp[3];
  const uint32_t gtid = blockIdx.x * kQuantThreads + threadIdx.x;
  const uint32_t gstride = gridDim.x * kQuantThreads;
  const uint32_t n8 = (uint32_t)a.T * (uint32_t)a.row8;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const float d = DYNAMIC ? a.st->descale_used[x] : descale_from_amax(a.st->static_values[x]);
      rcp[x] = 1.0 / (double)d;
      if (!DYNAMIC && blockIdx.x == 0) a.st->descale_used[x] = d;
    }
  }
  __syncthreads();
  const double r[3] = {rcp[0], rcp[1], rcp[2]};
  quantize_all<CONTIG, DYNAMIC>(a, n8, r, gtid, gstride);
}

// Amax pass of dynamic mode. Each block reduces its chunks of Q, K and V and
// atomic-maxes the three results into the state's scratch; then it arrives at
// a counter. The block that arrives last sees every other block's maxima
// (each arrival is a release, the last one an acquire), pushes the triple
// into ring slot count % 16, writes the descales from the window maximum
// including it, and clears the scratch and the counter for the next forward.
template <bool CONTIG>
__global__ __launch_bounds__(kQuantThreads) void amax_kernel(QuantArgs a) {
  __shared__ uint32_t red[kQuantThreads / 64];
  __shared__ uint32_t is_last;
  const uint32_t gtid = blockIdx.x * kQuantThreads + threadIdx.x;
  const uint32_t gstride = gridDim.x * kQuantThreads;
  const uint32_t n8 = (uint32_t)a.T * (uint32_t)a.row8;
  DevState* st = a.st;
  uint32_t mt[3];
  absmax_all<CONTIG>(a, n8, gtid, gstride, mt);
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    const uint32_t m = block_max<kQuantThreads>(mt[x], red);
    if (threadIdx.x == 0 && m != 0u)
      __hip_atomic_fetch_max(&st->amax_bits[0][x], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(&st->bar_arrived, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    is_last = prev + 1 == gridDim.x;
  }
  __syncthreads();
  if (is_last && threadIdx.x == 0) {
    float amax[3], d[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const uint32_t bits = __hip_atomic_load(&st->amax_bits[0][x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      amax[x] = __uint_as_float(bits << 16);
    }
    const uint32_t count = st->count;
    ring_window_descales(st, count, amax, d);
    ring_commit(st, count, amax, d);
#pragma unroll
    for (int x = 0; x < 3; ++x)
      __hip_atomic_store(&st->amax_bits[0][x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&st->bar_arrived, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

namespace {
int g_cus[64];

int device_cus() {
  int dev = 0;
  (void)hipGetDevice(&dev);
  int& n = g_cus[dev & 63];
  if (n == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) n = v;
  }
  return n;
}
}  // namespace

hipError_t launch_quantize(const QuantArgs& a, bool dynamic, hipStream_t s) {
  const int cus = device_cus();
  if (cus == 0) return hipErrorInvalidDevice;
  const bool contig = a.ld[0] == 8LL * a.row8 && a.ld[1] == 8LL * a.row8 && a.ld[2] == 8LL * a.row8;
  const uint64_t n8 = (uint64_t)a.T * (uint64_t)a.row8;
  uint64_t g = (n8 + (uint64_t)kQuantThreads * kUnroll - 1) / ((uint64_t)kQuantThreads * kUnroll);
  if (g < 1) g = 1;
  if (g > (uint64_t)cus * kGridPerCu) g = (uint64_t)cus * kGridPerCu;
  const dim3 grid((unsigned)g), block(kQuantThreads);
  if (dynamic) {
    const dim3 agrid((unsigned)(g < (uint64_t)kAmaxBlocks ? g : (uint64_t)kAmaxBlocks));
    if (contig)
      hipLaunchKernelGGL(amax_kernel<true>, agrid, block, 0, s, a);
    else
      hipLaunchKernelGGL(amax_kernel<false>, agrid, block, 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (contig)
      hipLaunchKernelGGL((quant_kernel<true, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((quant_kernel<false, true>), grid, block, 0, s, a);
  } else {
    if (contig)
      hipLaunchKernelGGL((quant_kernel<true, false>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((quant_kernel<false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace fp8vit
