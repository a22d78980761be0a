// Host-only harness for the JSON scale-file reader and writer
// (fp8_quantized_varlen_amd/csrc/json_scales.cpp), built with g++ and
// -fsanitize=address,undefined by tests/test_json_sanitized.py. Every file named
// on the command line goes through the reader for two layer names, then through
// the writer (which rewrites it in place when it holds a JSON object), then
// through the reader again. One line per file: the four status codes and the
// values of the last read; a memory error
// or undefined behaviour aborts the run with a sanitizer report.
#include <cstdio>

#include "fp8vit.h"

int main(int argc, char** argv) {
  const char* layers[2] = {"visual.blocks.0.attn.attn", "visual.blocks.1.attn.attn"};
  for (int i = 1; i < argc; ++i) {
    float v[3] = {0.f, 0.f, 0.f};
    std::printf("%s", argv[i]);
    for (const char* layer : layers) std::printf(" %d", (int)fp8vit_load_static_scales(argv[i], layer, v));
    const float w[3] = {1.5f, 2.25f, 3.0f};
    std::printf(" %d", (int)fp8vit_save_static_scales(argv[i], layers[1], w));
    const int st = (int)fp8vit_load_static_scales(argv[i], layers[1], v);
    std::printf(" %d %.9g %.9g %.9g\n", st, (double)v[0], (double)v[1], (double)v[2]);
  }
  return 0;
}
