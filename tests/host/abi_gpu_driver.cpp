// A plain C++ program that runs the FP8 ViT attention path through the C ABI
// of libfp8vit.so (include/fp8vit.h) and the HIP runtime alone, without
// PyTorch or Python: it saves and reloads the static scales through the JSON
// scale-file calls, quantizes Q, K and V, and runs the varlen attention with a
// workspace it sizes with fp8vit_attn_workspace_bytes.
//
// Usage: abi_gpu_driver <problem.bin> <result.bin> <scratch.json>
// problem.bin (little-endian): int32 T, H, d, nseg, max_seqlen, mode (0 dynamic,
//   1 static); float32 static values[3]; int32 cu_seqlens[nseg + 1]; then the
//   bf16 bits (uint16) of q, k and v, [T, H, d] each.
// result.bin: uint8 q8, k8, v8 [T * H * d each]; float32 descale_used[3];
//   uint16 (bf16 bits) output [T * H * d].
// Any failing call prints its status string and exits with status 2.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "fp8vit.h"

namespace {

void check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    std::exit(2);
  }
}

void check(fp8vit_status st, const char* what) {
  if (st != FP8VIT_OK) {
    std::fprintf(stderr, "%s: %s\n", what, fp8vit_status_str(st));
    std::exit(2);
  }
}

template <typename T>
void read_into(std::FILE* f, T* p, size_t n) {
  if (std::fread(p, sizeof(T), n, f) != n) {
    std::fprintf(stderr, "short problem file\n");
    std::exit(2);
  }
}

template <typename T>
T* device_copy(const std::vector<T>& h) {
  T* d = nullptr;
  check_hip(hipMalloc(&d, h.size() * sizeof(T) + 256), "hipMalloc");
  if (!h.empty()) check_hip(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice), "hipMemcpy");
  return d;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 4) {
    std::fprintf(stderr, "usage: %s problem.bin result.bin scratch.json\n", argv[0]);
    return 2;
  }
  std::FILE* f = std::fopen(argv[1], "rb");
  if (!f) return 2;
  int32_t hdr[6];
  float static_values[3];
  read_into(f, hdr, 6);
  read_into(f, static_values, 3);
  const int32_t T = hdr[0], H = hdr[1], d = hdr[2], nseg = hdr[3], max_seqlen = hdr[4], mode = hdr[5];
  const size_t n = (size_t)T * H * d;
  std::vector<int32_t> cu(nseg + 1);
  std::vector<uint16_t> q(n), k(n), v(n);
  read_into(f, cu.data(), cu.size());
  read_into(f, q.data(), n);
  read_into(f, k.data(), n);
  read_into(f, v.data(), n);
  std::fclose(f);

  hipStream_t stream;
  check_hip(hipStreamCreate(&stream), "hipStreamCreate");
  void* state = nullptr;
  check_hip(hipMalloc(&state, fp8vit_state_bytes()), "hipMalloc state");
  check(fp8vit_state_init(state, stream), "fp8vit_state_init");
  if (mode == FP8VIT_STATIC) {
    // the calibrate-once file round trip: save the values, read them back
    check(fp8vit_save_static_scales(argv[3], "visual.blocks.0.attn.attn", static_values),
          "fp8vit_save_static_scales");
    float loaded[3];
    check(fp8vit_load_static_scales(argv[3], "visual.blocks.0.attn.attn", loaded), "fp8vit_load_static_scales");
    for (int i = 0; i < 3; ++i)
      if (loaded[i] != static_values[i]) {
        std::fprintf(stderr, "scale file round trip changed value %d\n", i);
        return 2;
      }
    check(fp8vit_state_set_static(state, loaded, stream), "fp8vit_state_set_static");
  }
  uint16_t* dq = device_copy(q);
  uint16_t* dk = device_copy(k);
  uint16_t* dv = device_copy(v);
  int32_t* dcu = device_copy(cu);
  uint8_t *q8 = nullptr, *k8 = nullptr, *v8 = nullptr;
  uint16_t* out = nullptr;
  check_hip(hipMalloc(&q8, n + 256), "hipMalloc");
  check_hip(hipMalloc(&k8, n + 256), "hipMalloc");
  check_hip(hipMalloc(&v8, n + 256), "hipMalloc");
  check_hip(hipMalloc(&out, 2 * n + 256), "hipMalloc");
  const int64_t row = (int64_t)H * d;
  check(fp8vit_quantize_qkv(dq, dk, dv, row, row, row, T, H, d, mode, q8, k8, v8, state, stream),
        "fp8vit_quantize_qkv");
  const size_t ws_bytes = fp8vit_attn_workspace_bytes(nseg, max_seqlen, T, H, d);
  void* ws = nullptr;
  check_hip(hipMalloc(&ws, ws_bytes > 256 ? ws_bytes : 256), "hipMalloc workspace");
  check(fp8vit_attn_varlen_ws(q8, k8, v8, dcu, nseg, max_seqlen, T, H, d, 0.0f, state, out, row, ws, ws_bytes,
                              stream),
        "fp8vit_attn_varlen_ws");
  fp8vit_state_view view;
  check(fp8vit_state_read(state, &view, stream), "fp8vit_state_read");   // waits for the stream

  std::vector<uint8_t> c8(3 * n);
  std::vector<uint16_t> o(n);
  check_hip(hipMemcpy(c8.data(), q8, n, hipMemcpyDeviceToHost), "hipMemcpy");
  check_hip(hipMemcpy(c8.data() + n, k8, n, hipMemcpyDeviceToHost), "hipMemcpy");
  check_hip(hipMemcpy(c8.data() + 2 * n, v8, n, hipMemcpyDeviceToHost), "hipMemcpy");
  check_hip(hipMemcpy(o.data(), out, 2 * n, hipMemcpyDeviceToHost), "hipMemcpy");
  std::FILE* g = std::fopen(argv[2], "wb");
  if (!g) return 2;
  std::fwrite(c8.data(), 1, c8.size(), g);
  std::fwrite(view.descale_used, sizeof(float), 3, g);
  std::fwrite(o.data(), sizeof(uint16_t), n, g);
  std::fclose(g);
  for (void* p : {(void*)dq, (void*)dk, (void*)dv, (void*)dcu, (void*)q8, (void*)k8, (void*)v8, (void*)out, ws, state})
    check_hip(hipFree(p), "hipFree");
  check_hip(hipStreamDestroy(stream), "hipStreamDestroy");
  std::printf("ok: T=%d H=%d d=%d segments=%d workspace=%zu\n", T, H, d, nseg, ws_bytes);
  return 0;
}
