// Co-execution of vector work with the matrix core: how much do v_exp_f32 (the softmax's
// exponentials) and plain FMAs cost when interleaved with v_mfma_f32_32x32x16_bf16 in one wave, at
// 1, 2 and 4 waves per SIMD?  A measurement that informs the attention kernel's schedule.
//
// Each wave loops over 8 products on 4 independent accumulators from registers, and/or 16-32
// independent exp2 / fma chains (sched_group_barrier interleaves one product with a few vector
// instructions).  No memory traffic in the loop; one float per thread is written at the end.
// Prints the best of launches 2..5 per variant, in ns per loop iteration.
//
// Build and run:  hipcc --offload-arch=gfx950 -O3 coexec_rate.hip -o coexec_rate && ./coexec_rate
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kIn = 4096;

// MODE: 0 = 8 mfma; 1 = 32 exp; 2 = 8 mfma + 32 exp; 3 = 8 mfma + 32 fma; 4 = 8 mfma + 16 exp;
//       5 = 32 fma; 6 = 8 mfma + 16 exp + 16 fma
template <int MODE>
__global__ __launch_bounds__(256) void coexec_kernel(const unsigned short* in, float* out, int iters) {
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8_t a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = __builtin_bit_cast(__bf16, in[(gid * 8 + e) & (kIn - 1)]);
    b[e] = __builtin_bit_cast(__bf16, in[(gid * 8 + e + 3) & (kIn - 1)]);
  }
  f32x16_t acc[4];
  for (int i = 0; i < 4; ++i)
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float x[32];
  for (int i = 0; i < 32; ++i) x[i] = 0.25f + 0.01f * (float)((gid + i) & 31);
  constexpr bool MF = MODE == 0 || MODE == 2 || MODE == 3 || MODE == 4 || MODE == 6;
  constexpr int NEXP = MODE == 1 || MODE == 2 ? 32 : (MODE == 4 || MODE == 6 ? 16 : 0);
  constexpr int NFMA = MODE == 3 || MODE == 5 ? 32 : (MODE == 6 ? 16 : 0);
  for (int it = 0; it < iters; ++it) {
    if constexpr (MF) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i & 3], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NEXP; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
#pragma unroll
    for (int i = 0; i < NFMA; ++i) x[31 - i] = __builtin_fmaf(x[31 - i], 0.75f, 0.125f);
    if constexpr (MF && (NEXP + NFMA) > 0) {
      // one matrix product, then (NEXP + NFMA) / 8 vector instructions, eight times
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, (NEXP + NFMA) / 8, 0);
      }
    }
  }
  float s = 0.f;
  for (int i = 0; i < 4; ++i)
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  for (int i = 0; i < 32; ++i) s += x[i];
  out[gid] = s;
}

#define CHECK(x)                                                              \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));            \
      return 1;                                                               \
    }                                                                         \
  } while (0)

template <int MODE>
static int run(const unsigned short* din, float* dout, int blocks, int iters, const char* name) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  float best = 1e30f;
  for (int rep = 0; rep < 6; ++rep) {
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(coexec_kernel<MODE>, dim3(blocks), dim3(256), 0, 0, din, dout, iters);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    if (rep >= 2 && ms < best) best = ms;
  }
  // per wave and iteration, in ns
  std::printf("%-26s blocks %5d  %8.3f ms  %8.2f ns/iter\n", name, blocks, best, best * 1e6 / iters);
  return 0;
}

int main(int argc, char** argv) {
  std::vector<unsigned short> h(kIn);
  unsigned x = 12345;
  for (auto& v : h) {
    x = x * 1664525u + 1013904223u;
    v = (unsigned short)((0x3f80 | ((x >> 16) & 0x7f)) ^ ((x >> 8) & 0x8000));
  }
  const int iters = 20000;
  unsigned short* din = nullptr;
  float* dout = nullptr;
  const int max_blocks = 256 * 8;
  CHECK(hipMalloc(&din, kIn * sizeof(unsigned short)));
  CHECK(hipMalloc(&dout, (size_t)max_blocks * 256 * sizeof(float)));
  CHECK(hipMemcpy(din, h.data(), kIn * sizeof(unsigned short), hipMemcpyHostToDevice));
  for (int wps : {1, 2, 4}) {
    const int blocks = 256 * wps;  // 4 waves per block: wps waves per SIMD when all resident
    std::printf("-- %d wave(s) per SIMD\n", wps);
    run<0>(din, dout, blocks, iters, "8 mfma");
    run<1>(din, dout, blocks, iters, "32 exp");
    run<5>(din, dout, blocks, iters, "32 fma");
    run<2>(din, dout, blocks, iters, "8 mfma + 32 exp");
    run<4>(din, dout, blocks, iters, "8 mfma + 16 exp");
    run<3>(din, dout, blocks, iters, "8 mfma + 32 fma");
    run<6>(din, dout, blocks, iters, "8 mfma + 16 exp + 16 fma");
  }
  CHECK(hipFree(din));
  CHECK(hipFree(dout));
  return 0;
}
