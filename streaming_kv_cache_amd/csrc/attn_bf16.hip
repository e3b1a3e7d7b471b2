// bf16 flash attention over the visible key ranges on CDNA4 matrix cores.
//
// out_i = softmax(q_i K^T / sqrt(D)) V, where K/V are the concatenation of up
// to four key ranges (visible sinks, two runs of the ring, the current chunk):
// [LB-fast] "3. KV 缓存 滚动窗口" (attention over the window slice) and
// [ABot-stream] 机制二 (a chunk's queries see the visible history and the whole
// chunk, so no mask is needed inside a range).  Tiles never cross a range, so
// only the last tile of each range is partial.
//
// Two kernels share the score / softmax / output code path:
//   * attn_bf16_vt_kernel (the cache path): V arrives transposed (V^T[h][d][key],
//     the layout the V store keeps), K and V^T tiles are moved global -> LDS with
//     direct-to-LDS loads into XOR-swizzled layouts, 4 waves x 32 query rows per
//     workgroup, two workgroups per CU (two waves per SIMD, so one wave's softmax
//     overlaps the other's matrix work);
//   * attn_bf16_tokv_kernel (cross attention over caller-provided token-major V):
//     tiles staged through registers, V transposed on its way into LDS.
//
// Work decomposition (wave64, gfx950):
//   * a workgroup owns BM = NW*32*QB query rows of one head; each wave owns
//     32*QB rows; workgroup ids are remapped so that the workgroups one XCD runs
//     work on consecutive tiles of the same head (they share K/V in that XCD's L2);
//   * the key loop walks tiles of 64 keys; K rows and V^T are staged in LDS
//     (double-buffered, loads for tile t+1 in flight while tile t is computed);
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows, B = Q^T kept in
//     registers), so each lane holds scores of ONE query: row max and row sum
//     need a single cross-lane step (lanes l and l^32);
//   * the K rows feeding the A operand are read in an order that swaps bits 2
//     and 3 of the row index, which makes the score registers come out in the
//     key order the P^T B operand of the second product needs;
//   * O^T += V^T P^T with P rounded to bf16; online softmax in fp32 with exp2,
//     rescaling the accumulators only when the running max grows by more than
//     2^8 (the result is the same; P stays below 256);
//   * deterministic: no atomics, fixed reduction order.
#include "skv_device.hpp"
#include "skv_kernels.hpp"

namespace skv {

namespace {

constexpr int kBN = 64;  // keys per tile

__device__ __forceinline__ bf16x8_t ld_bf16x8(const void* p) {
  return __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)p);
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Key (0..31 inside a 32-key block) held by score register r in half hf.
__device__ __forceinline__ constexpr int score_key(int r, int hf) {
  return 16 * ((r >> 3) & 1) + 8 * hf + 4 * ((r >> 2) & 1) + (r & 3);
}

// K row read for A-operand row m: bits 2 and 3 swapped.
__device__ __forceinline__ int k_row_perm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <int D, int NW, int QB>
struct Cfg {
  static constexpr int BM = NW * 32 * QB;
  static constexpr int NT = NW * 64;
  static constexpr int KP = D + 8;        // K tile row pitch (elements)
  static constexpr int VP = kBN + 8;      // V^T tile row pitch (elements)
  static constexpr int KSTEPS = D / 16;   // k-steps of Q K^T
  static constexpr int MBLK = D / 32;     // 32-row blocks of O^T
  static constexpr int KCH = kBN * D / 8; // 16-byte chunks of a K tile
  static constexpr int KCH_T = (KCH + NT - 1) / NT;
  static constexpr int VUN = (kBN / 4) * (D / 8);  // (4 keys x 8 dims) units of a V tile
  static constexpr int VUN_T = (VUN + NT - 1) / NT;
};

}  // namespace

template <int D, int NW, int QB>
__global__ __launch_bounds__(NW * 64) void attn_bf16_tokv_kernel(AttnArgs a) {
  using C = Cfg<D, NW, QB>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBN * C::KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * C::VP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int n_qt = (a.Lq + C::BM - 1) / C::BM;
  const int tile = xcd_remap(blockIdx.x, n_qt * a.H);
  const int h = tile / n_qt, qt = tile - h * n_qt;
  const int q_base = qt * C::BM + wave * 32 * QB;

  // Q^T (B operand): lane (query l32, half hf) holds d = 16*ks + 8*hf .. +8.
  bf16x8_t qreg[QB][C::KSTEPS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = q_base + qb * 32 + l32;
    const bool ok = qi < a.Lq;
    const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)(ok ? qi : 0) * a.H + h) * D + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      u32x4_t v = ok ? *(const u32x4_t*)(qp + 16 * ks) : u32x4_t{0u, 0u, 0u, 0u};
      qreg[qb][ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  f32x16_t o[QB][C::MBLK];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < C::MBLK; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[qb][mb][r] = 0.f;
  }

  // ---- tile cursor over the key ranges
  int cseg = 0, coff = 0;
  auto skip_empty = [&]() {
    while (cseg < a.nseg && coff >= a.seg[cseg].n) {
      ++cseg;
      coff = 0;
    }
  };
  skip_empty();
  if (cseg >= a.nseg) return;  // no keys: the host never launches this

  u32x4_t kst[C::KCH_T];
  u32x4_t vst[C::VUN_T][4];
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};

  auto load_tile = [&](int si, int off) -> int {
    const KvSeg sg = a.seg[si];
    const int nk = sg.n - off < kBN ? sg.n - off : kBN;
    const uint16_t* kb = (const uint16_t*)sg.k + h * sg.k_hs + (int64_t)off * sg.k_rs;
    const uint16_t* vb = (const uint16_t*)sg.v + h * sg.v_hs + (int64_t)off * sg.v_rs;
#pragma unroll
    for (int i = 0; i < C::KCH_T; ++i) {
      const int c = tid + i * C::NT;
      const int key = c / (D / 8), ch = c % (D / 8);
      kst[i] = (c < C::KCH && key < nk) ? *(const u32x4_t*)(kb + (int64_t)key * sg.k_rs + ch * 8) : zero4;
    }
#pragma unroll
    for (int i = 0; i < C::VUN_T; ++i) {
      const int u = tid + i * C::NT;
      const int g = u / (D / 8), j = u % (D / 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 4 * g + r;
        vst[i][r] = (u < C::VUN && key < nk) ? *(const u32x4_t*)(vb + (int64_t)key * sg.v_rs + j * 8) : zero4;
      }
    }
    return nk;
  };

  auto store_tile = [&](int buf) {
    uint16_t* kd = Ks[buf];
    uint16_t* vd = Vt[buf];
#pragma unroll
    for (int i = 0; i < C::KCH_T; ++i) {
      const int c = tid + i * C::NT;
      if (c < C::KCH) {
        const int key = c / (D / 8), ch = c % (D / 8);
        *(u32x4_t*)(kd + key * C::KP + ch * 8) = kst[i];
      }
    }
#pragma unroll
    for (int i = 0; i < C::VUN_T; ++i) {
      const int u = tid + i * C::NT;
      if (u < C::VUN) {
        const int g = u / (D / 8), j = u % (D / 8);
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          const int w = dd >> 1;
          uint32_t lo, hi;
          if (dd & 1) {
            lo = (vst[i][0][w] >> 16) | (vst[i][1][w] & 0xffff0000u);
            hi = (vst[i][2][w] >> 16) | (vst[i][3][w] & 0xffff0000u);
          } else {
            lo = (vst[i][0][w] & 0xffffu) | (vst[i][1][w] << 16);
            hi = (vst[i][2][w] & 0xffffu) | (vst[i][3][w] << 16);
          }
          *(u32x2_t*)(vd + (8 * j + dd) * C::VP + 4 * g) = u32x2_t{lo, hi};
        }
      }
    }
  };

  int nk_cur = load_tile(cseg, coff);
  coff += kBN;
  skip_empty();
  store_tile(0);
  __syncthreads();

  const float sl2 = a.sl2;
  int buf = 0;
  while (true) {
    const bool has_next = cseg < a.nseg;
    int nk_next = 0;
    if (has_next) {
      nk_next = load_tile(cseg, coff);
      coff += kBN;
      skip_empty();
    }

    // ---- S^T = K Q^T for two 32-key blocks
    const uint16_t* Kb = Ks[buf];
    const uint16_t* Vb = Vt[buf];
    f32x16_t s[2][QB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8_t av = ld_bf16x8(Kb + (kb * 32 + k_row_perm(l32)) * C::KP + ks * 16 + 8 * hf);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qreg[qb][ks], s[kb][qb], 0, 0, 0);
      }
    }
    if (nk_cur < kBN) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + score_key(r, hf) >= nk_cur)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[kb][qb][r] = -INFINITY;
    }

    // ---- online softmax; P^T packed to bf16 in the B-operand order
    bf16x8_t pb[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = s[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
      mx = fmaxf(mx, xor32(mx)) * sl2;
      if (__any(mx > m_run[qb] + 8.0f)) {
        const float mn = fmaxf(m_run[qb], mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - mn);
        m_run[qb] = mn;
        l_run[qb] *= alpha;
#pragma unroll
        for (int mb = 0; mb < C::MBLK; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[qb][mb][r] *= alpha;
      }
      const float mneg = -m_run[qb];
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4_t pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 8 * half + 2 * e;
            const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][r], sl2, mneg));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][r + 1], sl2, mneg));
            lsum += p0 + p1;
            pk[e] = pack_bf16x2(p0, p1);
          }
          pb[qb][2 * kb + half] = __builtin_bit_cast(bf16x8_t, pk);
        }
      }
      l_run[qb] += lsum;
    }

    // ---- O^T += V^T P^T, four 16-key steps
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int mb = 0; mb < C::MBLK; ++mb) {
        const bf16x8_t av = ld_bf16x8(Vb + (mb * 32 + l32) * C::VP + st * 16 + 8 * hf);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          o[qb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[qb][st], o[qb][mb], 0, 0, 0);
      }
    }

    if (!has_next) break;
    store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    nk_cur = nk_next;
  }

  // ---- normalise and write: lane holds O^T[d][query l32] for d = 32mb + 8g + 4hf + 0..3
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l_run[qb] + xor32(l_run[qb]);
    const float inv = 1.f / lt;
    const int qi = q_base + qb * 32 + l32;
    if (qi >= a.Lq) continue;
    uint16_t* op = (uint16_t*)a.out + ((int64_t)qi * a.H + h) * D + 4 * hf;
#pragma unroll
    for (int mb = 0; mb < C::MBLK; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2_t w = {pack_bf16x2(o[qb][mb][4 * g] * inv, o[qb][mb][4 * g + 1] * inv),
                           pack_bf16x2(o[qb][mb][4 * g + 2] * inv, o[qb][mb][4 * g + 3] * inv)};
        *(u32x2_t*)(op + 32 * mb + 8 * g) = w;
      }
  }
}

template <int D, int NW, int QB>
static hipError_t launch_tokv_cfg(const AttnArgs& a, hipStream_t stream) {
  using C = Cfg<D, NW, QB>;
  const int n_qt = (a.Lq + C::BM - 1) / C::BM;
  dim3 grid(n_qt * a.H);
  hipLaunchKernelGGL((attn_bf16_tokv_kernel<D, NW, QB>), grid, dim3(C::NT), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attention_bf16_tokv(const AttnArgs& a, int D, hipStream_t stream) {
  switch (D) {
    case 64: return launch_tokv_cfg<64, 4, 1>(a, stream);
    case 128: return launch_tokv_cfg<128, 4, 1>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace skv

// ============================================================================
// Cache-path kernel: transposed V, direct-to-LDS tiles, two workgroups per CU.
// ============================================================================
namespace skv {

namespace {

__device__ __forceinline__ __attribute__((address_space(3))) void* lds_ptr(void* p) {
  return (__attribute__((address_space(3))) void*)p;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(256, 2) void attn_bf16_vt_kernel(AttnArgs a) {
  constexpr int NW = 4, BM = 128;
  constexpr int KRB = 2 * D;          // bytes per K row
  constexpr int KRP = 256 / KRB;      // K rows per 256-byte bank period
  constexpr int KCPR = KRB / 16;      // 16-byte chunks per K row
  constexpr int TB = kBN * KRB;       // bytes of a K tile (== bytes of a V^T tile: D rows x 64 keys)
  constexpr int NI = TB / 1024 / NW;  // 1-KB direct loads per wave, per tile and tensor
  constexpr int KSTEPS = D / 16, MBLK = D / 32;
  // [buffer][K tile | V^T tile].  K row r keeps 16-byte chunk c at c ^ ((r / KRP) % KCPR);
  // V^T row d (64 keys, 128 bytes) keeps chunk c at c ^ ((d / 2) % 8): the A-operand reads of
  // both products then touch every bank once per 16 lanes.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[4 * TB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int n_qt = (a.Lq + BM - 1) / BM;
  const int tile = xcd_remap(blockIdx.x, n_qt * a.H);
  const int h = tile / n_qt, qt = tile - h * n_qt;
  const int q_base = qt * BM + wave * 32;

  bf16x8_t qreg[KSTEPS];
  {
    const int qi = q_base + l32;
    const bool ok = qi < a.Lq;
    const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)(ok ? qi : 0) * a.H + h) * D + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4_t v = ok ? *(const u32x4_t*)(qp + 16 * ks) : u32x4_t{0u, 0u, 0u, 0u};
      qreg[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
  f32x16_t o[MBLK];
#pragma unroll
  for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  int cseg = 0, coff = 0;
  auto skip_empty = [&]() {
    while (cseg < a.nseg && coff >= a.seg[cseg].n) {
      ++cseg;
      coff = 0;
    }
  };
  skip_empty();
  if (cseg >= a.nseg) return;  // no keys: the host never launches this

  // Issue the loads of one K tile and one V^T tile into buffer b; returns the valid key count.
  auto issue = [&](int b, int si, int off) -> int {
    const KvSeg sg = a.seg[si];
    const int nk = sg.n - off < kBN ? sg.n - off : kBN;
    uint8_t* kt = smem + b * 2 * TB;
    uint8_t* vt = kt + TB;
    const uint8_t* kg = (const uint8_t*)sg.k + 2 * (h * sg.k_hs + (int64_t)off * sg.k_rs);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int blk = wave * NI + i;
      const int ob = blk * 1024 + lane * 16;
      const int r = ob / KRB, p = (ob % KRB) / 16;
      const int c = p ^ ((r / KRP) % KCPR);
      const int rr = r < nk ? r : 0;  // rows past the range: any valid row (scores are masked)
      __builtin_amdgcn_global_load_lds(kg + 2 * (int64_t)rr * sg.k_rs + 16 * c, lds_ptr(kt + blk * 1024), 16, 0, 0);
    }
    const uint8_t* vg = (const uint8_t*)sg.v + 2 * (h * sg.v_hs + (int64_t)off);
    if (sg.v_al16) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int blk = wave * NI + i;
        const int ob = blk * 1024 + lane * 16;
        const int d = ob / 128, p = (ob % 128) / 16;
        const int c = p ^ ((d >> 1) & 7);
        const int cc = 8 * c < nk ? c : 0;  // chunks past the range: any valid chunk (P is 0 there)
        __builtin_amdgcn_global_load_lds(vg + 2 * (int64_t)d * sg.v_ds + 16 * cc, lds_ptr(vt + blk * 1024), 16,
                                         0, 0);
      }
    } else {
      // ranges whose keys are not 16-byte aligned: element copies through registers
      for (int idx = tid; idx < D * kBN; idx += NW * 64) {
        const int d = idx / kBN, e = idx % kBN;
        const int key = 8 * ((e / 8) ^ ((d >> 1) & 7)) + (e % 8);
        const int kk = key < nk ? key : 0;
        ((uint16_t*)(vt + d * 128))[e] = ((const uint16_t*)vg)[(int64_t)d * sg.v_ds + kk];
      }
    }
    return nk;
  };

  int nk_cur = issue(0, cseg, coff);
  coff += kBN;
  skip_empty();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // per-lane LDS byte offsets of the A operands
  int krow_off[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) krow_off[kb] = (kb * 32 + k_row_perm(l32)) * KRB;
  int kswz[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) kswz[kb] = ((kb * 32 + k_row_perm(l32)) / KRP) % KCPR;
  const int vswz = (l32 >> 1) & 7;  // (d / 2) % 8 for d = 32*mb + l32

  const float sl2 = a.sl2;
  int buf = 0;
  while (true) {
    const bool has_next = cseg < a.nseg;
    int nk_next = 0;
    if (has_next) {
      nk_next = issue(buf ^ 1, cseg, coff);
      coff += kBN;
      skip_empty();
    }
    const uint8_t* kt = smem + buf * 2 * TB;
    const uint8_t* vt = kt + TB;

    // ---- S^T = K Q^T
    f32x16_t s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int c = 2 * ks + hf;
        const bf16x8_t av = ld_bf16x8(kt + krow_off[kb] + ((c ^ kswz[kb]) << 4));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qreg[ks], s[kb], 0, 0, 0);
      }
    }
    if (nk_cur < kBN) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + score_key(r, hf) >= nk_cur) s[kb][r] = -INFINITY;
    }

    // ---- online softmax; P^T packed to bf16 in the B-operand order
    bf16x8_t pb[4];
    {
      float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s[0][r], s[1][r]));
      mx = fmaxf(mx, xor32(mx)) * sl2;
      if (__any(mx > m_run + 8.0f)) {
        const float mn = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
        m_run = mn;
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[mb][r] *= alpha;
      }
      const float mneg = -m_run;
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4_t pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 8 * half + 2 * e;
            const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][r], sl2, mneg));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][r + 1], sl2, mneg));
            lsum += p0 + p1;
            pk[e] = pack_bf16x2(p0, p1);
          }
          pb[2 * kb + half] = __builtin_bit_cast(bf16x8_t, pk);
        }
      }
      l_run += lsum;
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int st = 0; st < 4; ++st) {
#pragma unroll
      for (int mb = 0; mb < MBLK; ++mb) {
        const int c = 2 * st + hf;
        const bf16x8_t av = ld_bf16x8(vt + (mb * 32 + l32) * 128 + ((c ^ vswz) << 4));
        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[st], o[mb], 0, 0, 0);
      }
    }

    if (!has_next) break;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    buf ^= 1;
    nk_cur = nk_next;
  }

  const float lt = l_run + xor32(l_run);
  const float inv = 1.f / lt;
  const int qi = q_base + l32;
  if (qi < a.Lq) {
    uint16_t* op = (uint16_t*)a.out + ((int64_t)qi * a.H + h) * D + 4 * hf;
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2_t w = {pack_bf16x2(o[mb][4 * g] * inv, o[mb][4 * g + 1] * inv),
                           pack_bf16x2(o[mb][4 * g + 2] * inv, o[mb][4 * g + 3] * inv)};
        *(u32x2_t*)(op + 32 * mb + 8 * g) = w;
      }
  }
}

hipError_t launch_attention_bf16_vt(const AttnArgs& a, int D, hipStream_t stream) {
  const int n_qt = (a.Lq + 127) / 128;
  dim3 grid(n_qt * a.H);
  switch (D) {
    case 64: hipLaunchKernelGGL(attn_bf16_vt_kernel<64>, grid, dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL(attn_bf16_vt_kernel<128>, grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace skv
