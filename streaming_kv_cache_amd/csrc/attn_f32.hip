// fp32 attention over the visible key ranges (small fp32 configurations).
//
// out_i = softmax(q_i K^T / sqrt(D)) V with fp32 arithmetic end to end (no
// reduced-precision matrix instructions): one wave per (head, 64 queries), one
// query row per lane, K/V tiles of 64 keys staged in LDS and read as
// broadcasts.  Online softmax over chunks of 16 keys (max, rescale, exp2).
// V is read through general strides, so the transposed V store and token-major
// V (cross attention) share the kernel.
#include "skv_device.hpp"
#include "skv_kernels.hpp"

namespace skv {

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(AttnArgs a) {
  constexpr int BN = 64, KC = 16;
  __shared__ __attribute__((aligned(16))) float Ks[BN][D];
  __shared__ __attribute__((aligned(16))) float Vs[BN][D];
  const int lane = threadIdx.x;
  const int n_qt = (a.Lq + 63) / 64;
  const int h = blockIdx.x / n_qt, qt = blockIdx.x % n_qt;
  const int qi = qt * 64 + lane;
  const bool q_ok = qi < a.Lq;
  const float* qp = (const float*)a.q + ((int64_t)qi * a.H + h) * D;
  float q[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    f32x4_t v = q_ok ? *(const f32x4_t*)(qp + d) : f32x4_t{0.f, 0.f, 0.f, 0.f};
    q[d] = v[0] * a.sl2;
    q[d + 1] = v[1] * a.sl2;
    q[d + 2] = v[2] * a.sl2;
    q[d + 3] = v[3] * a.sl2;
    acc[d] = acc[d + 1] = acc[d + 2] = acc[d + 3] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int si = 0; si < a.nseg; ++si) {
    if (si == a.alt_seg) {  // ranges from here on use the queries at q_alt
      const float* qa = (const float*)a.q_alt + ((int64_t)qi * a.H + h) * D;
#pragma unroll
      for (int d = 0; d < D; d += 4) {
        f32x4_t v = q_ok ? *(const f32x4_t*)(qa + d) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        q[d] = v[0] * a.sl2;
        q[d + 1] = v[1] * a.sl2;
        q[d + 2] = v[2] * a.sl2;
        q[d + 3] = v[3] * a.sl2;
      }
    }
    const KvSeg sg = a.seg[si];
    const float* kb = (const float*)sg.k + h * sg.k_hs;
    const float* vb = (const float*)sg.v + h * sg.v_hs;
    for (int off = 0; off < sg.n; off += BN) {
      const int nk = sg.n - off < BN ? sg.n - off : BN;
      __syncthreads();
      for (int idx = lane; idx < BN * D / 4; idx += 64) {
        const int key = idx / (D / 4), c = (idx % (D / 4)) * 4;
        f32x4_t kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
        if (key < nk) {
          kv = *(const f32x4_t*)(kb + (int64_t)(off + key) * sg.k_rs + c);
          const float* vr = vb + (int64_t)(off + key) * sg.v_rs;
          if (sg.v_ds == 1) {
            vv = *(const f32x4_t*)(vr + c);
          } else {  // transposed V
            vv = f32x4_t{vr[c * sg.v_ds], vr[(c + 1) * sg.v_ds], vr[(c + 2) * sg.v_ds], vr[(c + 3) * sg.v_ds]};
          }
        }
        *(f32x4_t*)&Ks[key][c] = kv;
        *(f32x4_t*)&Vs[key][c] = vv;
      }
      __syncthreads();
      for (int j0 = 0; j0 < nk; j0 += KC) {
        float s[KC];
        float mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < KC; ++j) {
          float dot = 0.f;
#pragma unroll
          for (int d = 0; d < D; ++d) dot = fmaf(q[d], Ks[j0 + j][d], dot);
          s[j] = (j0 + j < nk) ? dot : -INFINITY;
          mt = fmaxf(mt, s[j]);
        }
        const float mn = fmaxf(m, mt);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        l *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
        for (int j = 0; j < KC; ++j) {
          const float p = __builtin_amdgcn_exp2f(s[j] - mn);
          l += p;
#pragma unroll
          for (int d = 0; d < D; ++d) acc[d] = fmaf(p, Vs[j0 + j][d], acc[d]);
        }
        m = mn;
      }
    }
  }
  if (!q_ok) return;
  const float inv = 1.f / l;
  float* op = (float*)a.out + ((int64_t)qi * a.H + h) * D;
#pragma unroll
  for (int d = 0; d < D; d += 4)
    *(f32x4_t*)(op + d) = f32x4_t{acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv};
}

hipError_t launch_attention_f32(const AttnArgs& a, int D, hipStream_t stream) {
  const int n_qt = (a.Lq + 63) / 64;
  dim3 grid(n_qt * a.H);
  switch (D) {
    case 32: hipLaunchKernelGGL(attn_f32_kernel<32>, grid, dim3(64), 0, stream, a); break;
    case 64: hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace skv
