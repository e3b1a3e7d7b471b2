// Sustained rate of v_mfma_f32_32x32x16_bf16 on the whole chip: a measurement of the matrix-core
// ceiling the attention kernel runs against, next to the published dense bf16 peak.
//
// Every wave keeps four independent 16-register accumulators and issues products from registers
// only (no memory traffic in the loop); 2048 workgroups x 4 waves = 8 waves per SIMD.  The operand
// values decide the power drawn: "random" fills the operands with bf16 values of magnitude 1..2 and
// random signs, "zero" with zeros.  Prints TFLOP/s per launch (12 launches, the first ones warm up).
//
// Build and run:  hipcc --offload-arch=gfx950 -O3 mfma_rate.hip -o mfma_rate && ./mfma_rate random
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <vector>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kIn = 4096;  // operand pool (elements); every index below is masked into it

__global__ __launch_bounds__(256) void mfma_rate_kernel(const unsigned short* in, float* out, int iters) {
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8_t a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = __builtin_bit_cast(__bf16, in[(gid * 8 + e) & (kIn - 1)]);
    b[e] = __builtin_bit_cast(__bf16, in[(gid * 8 + e + 3) & (kIn - 1)]);
  }
  f32x16_t acc[4];
  for (int i = 0; i < 4; ++i)
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.f;
  for (int i = 0; i < 4; ++i)
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  out[gid] = s;  // keeps the products live
}

#define CHECK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));            \
      return 1;                                                               \
    }                                                                         \
  } while (0)

int main(int argc, char** argv) {
  const bool zero = argc > 1 && std::strcmp(argv[1], "zero") == 0;
  std::vector<unsigned short> h(kIn);
  unsigned x = 12345;
  for (auto& v : h) {
    x = x * 1664525u + 1013904223u;
    v = zero ? 0 : (unsigned short)((0x3f80 | ((x >> 16) & 0x7f)) ^ ((x >> 8) & 0x8000));
  }
  const int blocks = 256 * 8, threads = 256, iters = 20000;
  unsigned short* din = nullptr;
  float* dout = nullptr;
  CHECK(hipMalloc(&din, kIn * sizeof(unsigned short)));
  CHECK(hipMalloc(&dout, (size_t)blocks * threads * sizeof(float)));
  CHECK(hipMemcpy(din, h.data(), kIn * sizeof(unsigned short), hipMemcpyHostToDevice));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  const double flops = 2.0 * 32 * 32 * 16 * 4.0 * iters * (blocks * threads / 64);
  std::printf("operands: %s\n", zero ? "zero" : "random");
  for (int rep = 0; rep < 12; ++rep) {
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(threads), 0, 0, din, dout, iters);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    std::printf("launch %2d: %8.3f ms %8.1f TFLOP/s\n", rep, ms, flops / (ms * 1e-3) / 1e12);
  }
  CHECK(hipFree(din));
  CHECK(hipFree(dout));
  return 0;
}
