// Fused per-tensor e4m3 quantization of Q, K and V in one launch.
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
// window maximum sets this forward's descale. The amax pass and the quantize
// pass share one cooperative launch separated by a grid-wide barrier, so the
// three tensors cost a single launch instead of a reduction launch plus three
// quantization launches (the same page names "3 quantization kernel launches"
// as the small-image overhead).
//
// Data layout: bf16 rows of H*d elements with token stride ld; every thread
// moves 16-byte chunks (8 elements) in and 8-byte chunks out, consecutive
// lanes on consecutive chunks (fully coalesced for contiguous inputs).
#include "fp8vit_internal.h"
#include "state_device.h"

namespace fp8vit {

constexpr int kQuantThreads = 512;
constexpr int kUnroll = 4;   // chunks per tensor in flight per thread (12 for the three)
// Dynamic mode: one block of 1024 threads per CU. When every thread's share
// is at most kResident chunks per tensor (up to 8M elements per tensor on 256
// CUs), the chunks loaded for the amax stay in registers across the grid
// barrier and are quantized from there: the input is read once.
constexpr int kDynThreads = 1024;
constexpr int kResident = 8;
// Upper bound on one grid-barrier wait, in ticks of the 100 MHz real-time
// counter (20 ms). Reaching it means the co-residency assumption failed; the
// state flag records it and the kernel still runs to completion.
constexpr uint64_t kBarrierTimeoutTicks = 2000000ull;

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
template <bool CONTIG>
__device__ __forceinline__ void quantize_all(const QuantArgs& a, uint32_t n8, const double* r, uint32_t gtid,
                                             uint32_t gstride) {
  for (uint32_t base = gtid; base < n8; base += gstride * kUnroll) {
    uint4 w[3][kUnroll];
#pragma unroll
    for (int x = 0; x < 3; ++x)
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t c = base + u * gstride;
        w[x][u] = c < n8 ? *chunk_src<CONTIG>(a.x[x], a.ld[x], a.row8, c) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
    for (int x = 0; x < 3; ++x)
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t c = base + u * gstride;
        if (c < n8) reinterpret_cast<uint2*>(a.y[x])[c] = quant_chunk(w[x][u], r[x]);
      }
  }
}

// Largest |x| bits of each of Q, K, V over this thread's chunks (the same
// chunks quantize_all visits), with 3 * kUnroll loads in flight.
template <bool CONTIG>
__device__ __forceinline__ void absmax_all(const QuantArgs& a, uint32_t n8, uint32_t gtid, uint32_t gstride,
                                           uint32_t m[3]) {
  m[0] = m[1] = m[2] = 0;
  for (uint32_t base = gtid; base < n8; base += gstride * kUnroll) {
    uint4 w[3][kUnroll];
#pragma unroll
    for (int x = 0; x < 3; ++x)
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t c = base + u * gstride;
        w[x][u] = c < n8 ? *chunk_src<CONTIG>(a.x[x], a.ld[x], a.row8, c) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
    for (int x = 0; x < 3; ++x)
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) m[x] = max(m[x], chunk_absmax_bits(w[x][u]));
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

// Sense-free generation barrier over all blocks of a cooperative launch. The
// wait is bounded: on timeout the state's flag is raised and the block goes on,
// so every wave always exits.
__device__ void grid_barrier(DevState* st, uint32_t nblocks) {
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t gen = __hip_atomic_load(&st->bar_generation, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t prev = __hip_atomic_fetch_add(&st->bar_arrived, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (prev + 1 == nblocks) {
      __hip_atomic_store(&st->bar_arrived, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(&st->bar_generation, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (__hip_atomic_load(&st->bar_generation, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen) {
        __builtin_amdgcn_s_sleep(8);
        if (__builtin_amdgcn_s_memrealtime() - t0 > kBarrierTimeoutTicks) {
          __hip_atomic_fetch_or(&st->flags, kFlagBarrierTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
      __atomic_thread_fence(__ATOMIC_ACQUIRE);
    }
  }
  __syncthreads();
}

template <bool CONTIG>
__global__ __launch_bounds__(kQuantThreads) void quant_static_kernel(QuantArgs a) {
  __shared__ double rcp[3];
  const uint32_t gtid = blockIdx.x * kQuantThreads + threadIdx.x;
  const uint32_t gstride = gridDim.x * kQuantThreads;
  const uint32_t n8 = (uint32_t)a.T * (uint32_t)a.row8;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const float d = descale_from_amax(a.st->static_values[x]);
      rcp[x] = 1.0 / (double)d;
      if (blockIdx.x == 0) a.st->descale_used[x] = d;
    }
  }
  __syncthreads();
  const double r[3] = {rcp[0], rcp[1], rcp[2]};
  quantize_all<CONTIG>(a, n8, r, gtid, gstride);
}

template <bool CONTIG>
__global__ __launch_bounds__(kDynThreads) void quant_dynamic_kernel(QuantArgs a) {
  __shared__ uint32_t red[kDynThreads / 64];
  __shared__ double rcp[3];
  const uint32_t gtid = blockIdx.x * kDynThreads + threadIdx.x;
  const uint32_t gstride = gridDim.x * kDynThreads;
  const uint32_t n8 = (uint32_t)a.T * (uint32_t)a.row8;
  const bool resident = n8 <= gstride * (uint32_t)kResident;   // grid-uniform
  DevState* st = a.st;
  // Ring and count are read before the barrier; block 0 rewrites them after it.
  const uint32_t count = st->count;
  const uint32_t par = count & 1u;
  float ring_max_other[3];
  {
    const uint32_t slot = count % FP8VIT_RING_SLOTS;
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      float w = 0.0f;
#pragma unroll
      for (int i = 0; i < FP8VIT_RING_SLOTS; ++i) {
        float r = st->ring[x][i];
        w = (i != (int)slot && r > w) ? r : w;
      }
      ring_max_other[x] = w;
    }
  }
  // Phase A: amax of each tensor.
  uint4 held[3][kResident];
  uint32_t mt[3] = {0, 0, 0};
  if (resident) {
#pragma unroll
    for (int x = 0; x < 3; ++x)
#pragma unroll
      for (int u = 0; u < kResident; ++u) {
        const uint32_t c = gtid + u * gstride;
        held[x][u] = c < n8 ? *chunk_src<CONTIG>(a.x[x], a.ld[x], a.row8, c) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
    for (int x = 0; x < 3; ++x)
#pragma unroll
      for (int u = 0; u < kResident; ++u) mt[x] = max(mt[x], chunk_absmax_bits(held[x][u]));
  } else {
    absmax_all<CONTIG>(a, n8, gtid, gstride, mt);
  }
#pragma unroll
  for (int x = 0; x < 3; ++x) {
    const uint32_t m = block_max<kDynThreads>(mt[x], red);
    if (threadIdx.x == 0 && m != 0u)
      __hip_atomic_fetch_max(&st->amax_bits[par][x], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  grid_barrier(st, gridDim.x);
  // Phase B: descales from the window max including this forward (one
  // thread per block; the reciprocals go to the block through LDS).
  if (threadIdx.x == 0) {
    float amax[3], d[3];
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      uint32_t bits = __hip_atomic_load(&st->amax_bits[par][x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      amax[x] = __uint_as_float(bits << 16);
      float w = amax[x] > ring_max_other[x] ? amax[x] : ring_max_other[x];
      d[x] = descale_from_amax(w);
      rcp[x] = 1.0 / (double)d[x];
    }
    if (blockIdx.x == 0) {
      ring_commit(st, count, amax, d);
#pragma unroll
      for (int x = 0; x < 3; ++x) st->amax_bits[par ^ 1u][x] = 0u;   // scratch of the next forward
    }
  }
  __syncthreads();
  // Phase C: quantize.
  const double r[3] = {rcp[0], rcp[1], rcp[2]};
  if (resident) {
#pragma unroll
    for (int x = 0; x < 3; ++x)
#pragma unroll
      for (int u = 0; u < kResident; ++u) {
        const uint32_t c = gtid + u * gstride;
        if (c < n8) reinterpret_cast<uint2*>(a.y[x])[c] = quant_chunk(held[x][u], r[x]);
      }
  } else {
    quantize_all<CONTIG>(a, n8, r, gtid, gstride);
  }
}

namespace {
struct DeviceInfo {
  int cus = 0;
  int coop_blocks_contig = 0;
  int coop_blocks_strided = 0;
};
DeviceInfo g_info[64];

const DeviceInfo& device_info() {
  int dev = 0;
  (void)hipGetDevice(&dev);
  DeviceInfo& di = g_info[dev & 63];
  if (di.cus == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) == hipSuccess) {
      int b1 = 0, b2 = 0;
      (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&b1, quant_dynamic_kernel<true>, kDynThreads, 0);
      (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&b2, quant_dynamic_kernel<false>, kDynThreads, 0);
      di.coop_blocks_contig = (b1 > 0 ? b1 : 1) * p.multiProcessorCount;
      di.coop_blocks_strided = (b2 > 0 ? b2 : 1) * p.multiProcessorCount;
      di.cus = p.multiProcessorCount;
    }
  }
  return di;
}
}  // namespace

hipError_t launch_quantize(const QuantArgs& a, bool dynamic, hipStream_t s) {
  const DeviceInfo& di = device_info();
  if (di.cus == 0) return hipErrorInvalidDevice;
  const bool contig = a.ld[0] == 8LL * a.row8 && a.ld[1] == 8LL * a.row8 && a.ld[2] == 8LL * a.row8;
  const uint64_t n8 = (uint64_t)a.T * (uint64_t)a.row8;
  const uint64_t want = (n8 + (uint64_t)kQuantThreads * kUnroll - 1) / ((uint64_t)kQuantThreads * kUnroll);
  if (!dynamic) {
    uint64_t g = want < 1 ? 1 : want;
    const uint64_t cap = (uint64_t)di.cus * 4;
    if (g > cap) g = cap;
    if (contig)
      hipLaunchKernelGGL(quant_static_kernel<true>, dim3((unsigned)g), dim3(kQuantThreads), 0, s, a);
    else
      hipLaunchKernelGGL(quant_static_kernel<false>, dim3((unsigned)g), dim3(kQuantThreads), 0, s, a);
    return hipGetLastError();
  }
  // At most one block per CU, all on the chip together while they wait at the
  // grid barrier (the cooperative launch refuses grids that could not be);
  // just enough blocks for the register-resident path when it applies.
  const uint64_t per_block = (uint64_t)kDynThreads * kResident;
  uint64_t g = (n8 + per_block - 1) / per_block;
  if (g < 1) g = 1;
  uint64_t cap = (uint64_t)di.cus;
  const uint64_t coresident = (uint64_t)(contig ? di.coop_blocks_contig : di.coop_blocks_strided);
  if (cap > coresident) cap = coresident;
  if (g > cap) g = cap;
  QuantArgs args = a;
  void* params[] = {&args};
  const void* fn = contig ? reinterpret_cast<const void*>(quant_dynamic_kernel<true>)
                          : reinterpret_cast<const void*>(quant_dynamic_kernel<false>);
  return hipLaunchCooperativeKernel(fn, dim3((unsigned)g), dim3(kDynThreads), params, 0, s);
}

}  // namespace fp8vit
