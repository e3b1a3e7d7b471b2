// bf16 flash attention over the visible key ranges on CDNA4 matrix cores.
//
// out_i = softmax(q_i K^T / sqrt(D)) V, where K/V are the concatenation of up
// to four key ranges (visible sinks, two runs of the ring, the current chunk):
// [LB-fast] "3. KV 缓存 滚动窗口" (attention over the window slice) and
// [ABot-stream] 机制二 (a chunk's queries see the visible history and the whole
// chunk, so no mask is needed inside a range).  Tiles never cross a range, so
// only the last tile of each range is partial.
//
// Three kernels:
//   * attn_bf16_vt_kernel (the cache path): V arrives transposed, in the V store's
//     tiles of 64 keys (V^T[h][key / 64][d][key % 64]); K rows and V^T tiles go global -> LDS with
//     direct-to-LDS buffer loads into padded, conflict-free layouts.  Two shapes:
//     4 waves x 32 query rows with two stages (two workgroups per CU), or 8 waves
//     x 32 rows with four stages (one workgroup per CU); the host picks the one
//     that needs fewer dispatch rounds;
//   * attn_bf16_tokv_kernel (cross attention over caller-provided token-major V):
//     tiles staged through registers, V transposed on its way into LDS;
//   * attn_merge_kernel: when a grid would leave most of the chip idle (few heads), the
//     cache-path kernel splits each query tile's keys over several workgroups, which write
//     partial (O, running max, row sum); this pass combines them (log-sum-exp weights).
//
// Work decomposition (wave64, gfx950):
//   * a workgroup owns the query rows of its waves for one head; workgroup ids are
//     remapped so that the workgroups one XCD runs work on consecutive tiles of
//     the same head (they share K/V in that XCD's L2);
//   * the key loop walks tiles of 64 keys, loads running one or two tiles ahead;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows, B = Q^T kept in
//     registers), so each lane holds scores of ONE query: row max and row sum
//     need a single cross-lane step (lanes l and l^32);
//   * the K rows feeding the A operand are read in an order that swaps bits 2
//     and 3 of the row index, which makes the score registers come out in the
//     key order the P^T B operand of the second product needs;
//   * O^T += V^T P^T with P rounded to bf16; softmax in fp32 with exp2 against a
//     running max that is raised only when a row sum would pass 2^60 (the result
//     is the same for any max); each 64-key tile is done in two 32-key halves so
//     the exponentials of one half overlap the matrix products of the other;
//   * the A operands (K rows, V^T rows) sit in one rolling set of registers: the LDS
//     reads of the next product group are issued one behind each product of the
//     current group, so they land under the matrix core (the 8-wave shape also
//     moves its tile barrier before the last product group, so the next tile's
//     first K reads roll behind it too);
//   * deterministic: no atomics, fixed reduction order.
#include <cstdlib>

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
// Cache-path kernel: transposed V, direct-to-LDS tiles, NW waves, NSTAGE tile stages.
// ============================================================================
namespace skv {

namespace {

__device__ __forceinline__ __attribute__((address_space(3))) void* lds_ptr(void* p) {
  return (__attribute__((address_space(3))) void*)p;
}

}  // namespace

// Word 3 of a raw (stride 0) buffer resource on gfx9-family parts: 32-bit data format, no swizzle.
constexpr int kRsrcWord3 = 0x00020000;

// 16 bytes per lane from base + voff + soff straight into LDS (lane l writes lds + 16 l).
// A buffer load rather than a global one: the compiler then tracks it as a plain vector-memory
// load, and LDS reads issued after it keep their partial lgkmcnt waits.  Offsets stay below 2^31
// (the host checks the ranges).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7fffffff, kRsrcWord3);
}
__device__ __forceinline__ void buf_lds16(__amdgpu_buffer_rsrc_t r, void* lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(lds), 16, voff, soff, 0, 0);
}

// Wait until at most N vector-memory loads of this wave are in flight and all LDS
// operations are done, then barrier.  Written out because a fenced barrier also waits
// for the direct-to-LDS loads that are meant to stay in flight.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  // s_waitcnt fields (gfx9): vmcnt [3:0] and [15:14], expcnt [6:4] (7 = no wait), lgkmcnt [11:8]
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
}

// Cross-half (lanes l and l^32) reductions.
__device__ __forceinline__ float half_swap_max(float x) { return fmaxf(x, xor32(x)); }
__device__ __forceinline__ float half_swap_sum(float x) { return x + xor32(x); }

// FOLLOW (masked only): the running max follows every half tile from -inf, for rows that may see no
// key of the first tiles (no sinks).  With sinks every row sees key 0 of its workgroup's first tile,
// so the max starts there and is raised only on overflow, as unmasked.
template <int D, int NW, int NSTAGE, bool MASKED, bool FOLLOW = MASKED>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void attn_bf16_vt_kernel(AttnBatch ab) {
  static_assert(NSTAGE == 2 || NSTAGE == 4, "two or four stages");
  constexpr int BM = NW * 32;
  constexpr int KP = 2 * D + 16;          // LDS pitch of a K row (bytes): data + one 16-byte pad
  constexpr int VP = 2 * kBN + 16;        // LDS pitch of a V^T row (64 keys + pad)
  constexpr int KT_B = kBN * KP, VT_B = D * VP;
  constexpr int KBLK = KT_B / 1024, VBLK = VT_B / 1024;  // 1-KB direct loads per tile
  constexpr int KI = (KBLK + NW - 1) / NW, VI = (VBLK + NW - 1) / NW;
  constexpr int KCPR = 2 * D / 16;        // data chunks per K row
  constexpr int KSTEPS = D / 16, MBLK = D / 32;
  static_assert(KT_B % 1024 == 0 && VT_B % 1024 == 0, "tiles must be whole 1-KB blocks");
  // fewest direct loads any wave issues per K / V^T tile: the in-order vmcnt thresholds
  constexpr int KMIN = KBLK / NW, VMIN = VBLK / NW;
  // [K stages | V^T stages].  A padded pitch of 68 (K) or 36 (V^T)
  // dwords puts the 16 rows a 16-lane group reads on 16 distinct 4-bank groups, so both
  // products read conflict-free with addresses that are a lane constant plus an immediate.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTAGE * (KT_B + VT_B)];

  const int tid = threadIdx.x, lane = tid & 63;
  // uniform (scalar branches on it) and known to be below NW
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (NW - 1);
  const int l32 = lane & 31, hf = lane >> 5;
  // every batch element has the same Lq, H and split count; split index slowest, so that the
  // workgroups next to each other share the key range of their split
  const int n_qt = (ab.b[0].Lq + BM - 1) / BM;
  const int per = n_qt * ab.b[0].H;
  const int nsp = (!MASKED && ab.b[0].nsplit > 1) ? ab.b[0].nsplit : 1;
  const int tile = xcd_remap(blockIdx.x, per * ab.nb * nsp);
  const int sp = tile / (per * ab.nb), tl = tile - sp * per * ab.nb;
  const int bi = tl / per, rest = tl - bi * per;
  const AttnArgs& a = ab.b[bi];
  const int h = rest / n_qt, qt = rest - h * n_qt;
  const int q_base = qt * BM + wave * 32;
  const float sl2 = a.sl2;

  // Q^T, pre-multiplied by softmax scale * log2(e): scores come out in log2 units.  fetch_q issues
  // the loads, scale_q (which waits for them) converts in place; the prologue issues the first K/V
  // tiles in between, so the latencies of the query rows and of the first tiles overlap.
  bf16x8_t qreg[KSTEPS];
  auto fetch_q = [&](const void* src) {
    const int qi = q_base + l32;
    const bool ok = qi < a.Lq;
    const uint16_t* qp = (const uint16_t*)src + ((int64_t)(ok ? qi : 0) * a.H + h) * D + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qreg[ks] = __builtin_bit_cast(bf16x8_t, ok ? *(const u32x4_t*)(qp + 16 * ks) : u32x4_t{0u, 0u, 0u, 0u});
  };
  auto scale_q = [&]() {
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4_t v = __builtin_bit_cast(u32x4_t, qreg[ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = pack_bf16x2(bf16_lo_to_f32(v[e]) * sl2, bf16_hi_to_f32(v[e]) * sl2);
      qreg[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  };
  auto load_q = [&](const void* src) {
    fetch_q(src);
    scale_q();
  };
  f32x16_t o[MBLK];
#pragma unroll
  for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;
  // unmasked: the running max starts at the first half tile's max; masked: at -inf (a row may
  // see no key of the first tiles) and follows every half tile's max
  float m_run = FOLLOW ? -INFINITY : 0.f, l_run = 0.f;
  // unmasked: -m_run in every entry, the accumulator the score products start from, so the
  // scores come out already relative to the running max (no subtraction per score)
  f32x16_t negm;
#pragma unroll
  for (int r = 0; r < 16; ++r) negm[r] = 0.f;

  // Masked (many chunks at once): query row r lies in frame q0 + r / F of the chunk ending at
  // frame e(r); it sees keys of frames j < e with j < S or j >= e - (W - S).  This workgroup's
  // keys are the visible sinks [0, min(S, e_b) F) and the window [max(S, e_a - (W - S)) F, e_b F),
  // e_a / e_b the chunk ends of its first / last rows; lanes mask what their own row may not see.
  int e_a = 0, e_b = 0, sink_keys = 0, ring0 = 0, ring_keys = 0, vis_hi = 0, ring_lo = 0;
  if constexpr (MASKED) {
    const int r_last = (qt * BM + BM < a.Lq ? qt * BM + BM : a.Lq) - 1;
    auto chunk_end = [&](int row) { return a.mq0 + a.mc * ((row / a.mF) / a.mc + 1); };
    e_a = chunk_end(qt * BM);
    e_b = chunk_end(r_last);
    sink_keys = (a.mS < e_b ? a.mS : e_b) * a.mF;
    const int r0f = a.mS > e_a - (a.mW - a.mS) ? a.mS : e_a - (a.mW - a.mS);
    ring0 = r0f * a.mF;
    ring_keys = e_b * a.mF - ring0 > 0 ? e_b * a.mF - ring0 : 0;
    const int qr = q_base + l32 < a.Lq ? q_base + l32 : r_last;
    const int er = chunk_end(qr);
    vis_hi = er * a.mF;
    ring_lo = (a.mS > er - (a.mW - a.mS) ? a.mS : er - (a.mW - a.mS)) * a.mF;
  }
  const int nseg = MASKED ? 2 : a.nseg;

  // Lane part of the direct loads.  Lane l of block blk fills LDS bytes [blk*1024 + 16 l, +16);
  // lanes that land on a pad chunk fetch a harmless valid chunk (row 0, chunk 0).
  // `ln` is the lane id passed through an empty asm so that the partial-tile paths recompute
  // their offsets instead of keeping them live in registers across the loop.
  auto k_lane = [&](int i, int ln, int& row, int& c16) {
    const int ob = (wave + NW * i) * 1024 + 16 * ln;
    row = ob / KP;
    const int ch = (ob % KP) / 16;
    if (ch >= KCPR || row >= kBN) row = 0, c16 = 0; else c16 = 16 * ch;
  };
  auto v_lane = [&](int i, int ln, int& d, int& ch) {
    const int ob = (wave + NW * i) * 1024 + 16 * ln;
    d = ob / VP;
    ch = (ob % VP) / 16;
    if (ch >= 8 || d >= D) d = 0, ch = 0;
  };
  int kq_off[KI], vq_off[VI];  // byte offsets for whole tiles of the current range

  // Two uniform tile iterators over the key ranges (one for K, one for V^T; they advance together).
  auto seg_n = [&](int s_) -> int { return MASKED ? (s_ == 0 ? sink_keys : ring_keys) : a.seg[s_].n; };
  auto seg_start = [&](int s_) -> int { return MASKED ? (s_ == 0 ? 0 : ring0) : 0; };
  int n_tiles = 0, alt_tiles = 1 << 30;  // tiles before the ranges that use the queries at q_alt
  for (int s_ = 0; s_ < nseg; ++s_) {
    if (!MASKED && s_ == a.alt_seg) alt_tiles = n_tiles;
    n_tiles += (seg_n(s_) + kBN - 1) / kBN;
  }
  if (n_tiles == 0) return;  // no keys: the host never launches this
  // split keys: this workgroup's tiles [t_begin, t_begin + n_tiles) of the sequence
  int t_begin = 0;
  if (nsp > 1) {
    t_begin = sp * a.split_tiles;
    const int t_end = n_tiles < t_begin + a.split_tiles ? n_tiles : t_begin + a.split_tiles;
    n_tiles = t_end - t_begin;
    alt_tiles -= t_begin;  // local index of the query switch
    if (n_tiles <= 0) {
      // an empty split (a batch element with fewer tiles than the others): contributes nothing
      const int qi = q_base + l32;
      if (qi < a.Lq) {
        const int64_t row = ((int64_t)sp * a.Lq + qi) * a.H + h;
        float* po = a.part_o + row * D + 4 * hf;
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
          for (int g = 0; g < 4; ++g) *(f32x4_t*)(po + 32 * mb + 8 * g) = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (hf == 0) {
          a.part_ml[2 * row] = -INFINITY;
          a.part_ml[2 * row + 1] = 0.f;
        }
      }
      return;
    }
  }
  // queries of the first tile (from the switch on: at q_alt); converted once the first tiles are issued
  if (alt_tiles <= 0) {
    fetch_q(a.q_alt);
    alt_tiles = 1 << 30;
  } else {
    fetch_q(a.q);
  }
  int ksi = 0, krem = 0, k_rs_b = 0;
  const uint8_t* kp = nullptr;
  
  int k_so = 0, kkey = 0;  // kkey: sequence index of the next K tile's first key (masked)
  __amdgpu_buffer_rsrc_t krs = buf_rsrc(nullptr);  // the current K range of this head (k_so: offset in it)
  auto k_seg = [&](int s_) {
    const KvSeg sg = a.seg[MASKED ? 0 : s_];
    const int start = seg_start(s_);
    kp = (const uint8_t*)sg.k + 2 * ((int64_t)h * sg.k_hs + (int64_t)start * sg.k_rs);
    k_so = 0;
    krs = buf_rsrc(kp);
    kkey = start;
    k_rs_b = (int)(2 * sg.k_rs);
    krem = seg_n(s_);
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      int row, c16;
      k_lane(i, lane, row, c16);
      kq_off[i] = row * k_rs_b + c16;
    }
  };
  // V^T in 64-key tiles: the current range starts at position vph of the tile at vp; the tile
  // iterator advances by whole tiles (v_so), so a lane's offset inside the range is fixed.
  constexpr int VTILE_B = 2 * kVtKeys * D;  // bytes of one tile (every d of 64 keys)
  int vsi = 0, vrem = 0, v_al16 = 1, vph = 0;
  const uint8_t* vp = nullptr;
  int v_so = 0;
  __amdgpu_buffer_rsrc_t vrs = buf_rsrc(nullptr);
  // byte offset from vp of the keys starting at range key r (a multiple of 8 when aligned), dim d
  auto v_off = [&](int d, int r) -> int {
    const int p = vph + r;
    return (p >> 6) * VTILE_B + d * (2 * kVtKeys) + 2 * (p & 63);
  };
  auto v_seg = [&](int s_) {
    const KvSeg sg = a.seg[MASKED ? 0 : s_];
    const int pe = sg.v_phase + seg_start(s_);
    vp = (const uint8_t*)sg.v + 2 * (int64_t)h * sg.v_hs + (int64_t)(pe >> 6) * VTILE_B;
    vph = pe & 63;
    v_so = 0;
    vrs = buf_rsrc(vp);
    vrem = seg_n(s_);
    v_al16 = sg.v_al16 && (vph & 7) == 0;
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      int d, ch;
      v_lane(i, lane, d, ch);
      vq_off[i] = v_off(d, 8 * ch);
    }
  };
  k_seg(0);
  while (krem <= 0 && ++ksi < nseg) k_seg(ksi);
  v_seg(0);
  while (vrem <= 0 && ++vsi < nseg) v_seg(vsi);
  // split keys: move both iterators (they walk the same ranges) to tile t_begin
  for (int skip = t_begin; skip > 0;) {
    const int left = (krem + kBN - 1) / kBN;  // tiles left in the current range
    if (left <= 0) break;                       // no range left (cannot happen: t_begin < tiles)
    if (skip < left) {
      k_so += skip * kBN * k_rs_b;
      kkey += skip * kBN;
      krem -= skip * kBN;
      v_so += skip * VTILE_B;
      vp += skip * VTILE_B;
      vrem -= skip * kBN;
      skip = 0;
    } else {
      skip -= left;
      krem = 0;
      vrem = 0;
      while (krem <= 0 && ++ksi < nseg) k_seg(ksi);
      while (vrem <= 0 && ++vsi < nseg) v_seg(vsi);
    }
  }

  // Issue the next K tile into stage st; returns its valid key count (and, masked, the
  // sequence index of its first key in key0).
  int key0 = 0;
  auto issue_k = [&](int st) -> int {
    const int nk = krem < kBN ? krem : kBN;
    key0 = kkey;
    kkey += kBN;
    uint8_t* dst = smem + st * KT_B;
    if (nk == kBN) {
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        const int blk = wave + NW * i;
        if (blk < KBLK) buf_lds16(krs, dst + blk * 1024, kq_off[i], k_so);
      }
    } else {
      int ln = lane;
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        const int blk = wave + NW * i;
        if (blk < KBLK) {
          int row, c16;
          k_lane(i, ln, row, c16);
          const int rr = row < nk ? row : 0;  // rows past the range: a valid row (masked)
          buf_lds16(krs, dst + blk * 1024, rr * k_rs_b + c16, k_so);
        }
      }
    }
    krem -= kBN;
    k_so += kBN * k_rs_b;
    while (krem <= 0 && ++ksi < nseg) k_seg(ksi);
    return nk;
  };
  // Issue the next V^T tile into stage st.
  auto issue_v = [&](int st) {
    const int nk = vrem < kBN ? vrem : kBN;
    uint8_t* dst = smem + NSTAGE * KT_B + st * VT_B;
    if (v_al16 && nk == kBN) {
#pragma unroll
      for (int i = 0; i < VI; ++i) {
        const int blk = wave + NW * i;
        if (blk < VBLK) buf_lds16(vrs, dst + blk * 1024, vq_off[i], v_so);
      }
    } else if (v_al16) {
      int ln = lane;
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int i = 0; i < VI; ++i) {
        const int blk = wave + NW * i;
        if (blk < VBLK) {
          int d, ch;
          v_lane(i, ln, d, ch);
          const int cc = 8 * ch < nk ? ch : 0;  // chunks past the range: valid data, P is 0
          buf_lds16(vrs, dst + blk * 1024, v_off(d, 8 * cc), v_so);
        }
      }
    } else {
      // ranges whose first key does not start a 16-byte piece: element copies through registers
      for (int idx = tid; idx < D * kBN; idx += NW * 64) {
        const int d = idx / kBN, e = idx % kBN;
        const int kk = e < nk ? e : 0;
        ((uint16_t*)(dst + d * VP))[e] = *(const uint16_t*)(vp + v_off(d, kk));
      }
    }
    vrem -= kBN;
    vp += VTILE_B;
    v_so += VTILE_B;
    while (vrem <= 0 && ++vsi < nseg) v_seg(vsi);
  };

  // per-lane LDS byte offsets of the A operands (plus immediates per k-step)
  int koff[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) koff[kb] = (kb * 32 + k_row_perm(l32)) * KP + 16 * hf;
  const int voff = l32 * VP + 16 * hf;
  const uint32_t one2 = 0x3f803f80u;  // bf16 pair (1, 1)

  // Whole K/V tiles NSTAGE-1 ahead (two stages: one ahead), one barrier per tile.
  int nkq[3] = {0, 0, 0}, k0q[3] = {0, 0, 0};  // valid keys / first key of the tiles in flight, oldest first
#pragma unroll
  for (int i = 0; i < NSTAGE - 1; ++i)
    if (i < n_tiles) {
      nkq[i] = issue_k(i);
      k0q[i] = key0;
      issue_v(i);
    }
  scale_q();

  // P = exp2(S' - sub) for one 32-key half, packed to bf16 in B-operand order; returns the
  // row sum of the rounded values.
  auto exp_half = [&](const f32x16_t& sv, float sub, bf16x8_t& p0, bf16x8_t& p1) -> float {
    float ls = 0.f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4_t pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 8 * half + 2 * e;
        const uint32_t w = pack_bf16x2(__builtin_amdgcn_exp2f(sv[r] - sub), __builtin_amdgcn_exp2f(sv[r + 1] - sub));
        ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, one2), ls,
                                             false);
        pk[e] = w;
      }
      (half ? p1 : p0) = __builtin_bit_cast(bf16x8_t, pk);
    }
    return ls;
  };
  auto max_half = [&](const f32x16_t& sv) -> float {
    float ma = fmaxf(fmaxf(sv[0], sv[1]), sv[2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) ma = fmaxf(fmaxf(ma, sv[r]), sv[r + 1]);
    return half_swap_max(fmaxf(ma, sv[15]));
  };
  // Raise the running max by up: rescale what has been accumulated.
  auto raise_by = [&](float up) {
    const float alpha = __builtin_amdgcn_exp2f(-up);
    l_run *= alpha;
#pragma unroll
    for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[mb][r] *= alpha;
    m_run += up;
  };
  // Masked: the running max follows the max of every half tile (rows may have seen nothing
  // yet: -inf until their first visible key); returns the offset the exponentials use.
  auto follow_max = [&](const f32x16_t& sv) -> float {
    const float mn = fmaxf(m_run, max_half(sv));
    if (__any(mn > m_run)) {
      const float alpha = mn > m_run ? __builtin_amdgcn_exp2f(m_run - mn) : 1.f;  // m_run = -inf: 0
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[mb][r] *= alpha;
      m_run = mn;
    }
    return m_run == -INFINITY ? 0.f : m_run;
  };
  // Masked: scores of keys this lane's row may not see (or past the range) -> -inf.  kbase is the
  // sequence index of the half tile's first key, nvalid its valid key count.
  auto mask_half = [&](f32x16_t& sv, int kbase, int nvalid) {
    const int kend = kbase + (nvalid < 32 ? nvalid : 32);
    const bool all_seen = kend <= e_a * a.mF &&
                          (kend <= a.mS * a.mF || kbase >= (a.mS > e_b - (a.mW - a.mS) ? a.mS : e_b - (a.mW - a.mS)) * a.mF);
    if (all_seen && nvalid >= 32) return;
    // key score_key(r, hf) = kbase + score_key(r, 0) + 8 hf: compare score_key(r, 0) with shifted bounds
    const int off = kbase + 8 * hf;
    int t_hi = vis_hi - off, t_sink = a.mS * a.mF - off, t_ring = ring_lo - off, t_n = nvalid - 8 * hf;
    asm volatile("" : "+v"(t_hi), "+v"(t_sink), "+v"(t_ring), "+v"(t_n));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = score_key(r, 0);
      if (!(kk < t_hi && kk < t_n && (kk < t_sink || kk >= t_ring))) sv[r] = -INFINITY;
    }
  };

  // Scheduling of the LDS operand reads.  All shapes keep the A operands in one rolling set of
  // registers and read K of keys 32..63 behind the first score products.  The 8-wave shape also
  // reads V behind the preceding products, and moves the tile's barrier from the top of the tile
  // to before its last product group, so that K of the next tile's keys 0..31 is read behind that
  // group too.  Each was measured faster for the 8-wave shape and slower for the 4-wave one (two
  // workgroups per CU, whose waves already cover each other's waits).
  constexpr bool ROLL_ALL = NW == 8;
  static_assert(KSTEPS == 2 * MBLK, "K steps and V blocks share the operand slots");
  bf16x8_t ob[KSTEPS];
  if constexpr (ROLL_ALL) {
    // tile 0 landed (later tiles may still be in flight), then K of its keys 0..31
    if constexpr (NSTAGE == 2)
      wait_vm_barrier<0>();
    else if (n_tiles > 2)
      wait_vm_barrier<2 * (KMIN + VMIN)>();
    else if (n_tiles > 1)
      wait_vm_barrier<KMIN + VMIN>();
    else
      wait_vm_barrier<0>();
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) ob[ks] = ld_bf16x8(smem + koff[0] + 32 * ks);
  }

  for (int t = 0; t < n_tiles; ++t) {
    const int st = t % NSTAGE;
    const bool more = t + 1 < n_tiles;
    if constexpr (!ROLL_ALL) {
      // tile t landed (later tiles may still be in flight), then everyone is done with tile t-1
      if constexpr (NSTAGE == 2)
        wait_vm_barrier<0>();
      else if (t + 2 < n_tiles)
        wait_vm_barrier<2 * (KMIN + VMIN)>();
      else if (more)
        wait_vm_barrier<KMIN + VMIN>();
      else
        wait_vm_barrier<0>();
    }
    const int nk = nkq[0], k0 = k0q[0];
    nkq[0] = nkq[1];
    nkq[1] = nkq[2];
    k0q[0] = k0q[1];
    k0q[1] = k0q[2];
    // the stage of tile t-1, which every wave is done with (behind the last barrier), takes
    // tile t + NSTAGE - 1: K here; V here too with four waves, behind the first score products
    // with eight (the eight waves' loads then reach the memory pipeline in two bursts: 480P
    // -0.8 to -1.7 %, 720P -1.9 % per pass, measured interleaved; the same in the four-wave
    // shape, and moving K as well, were slower)
    const bool fill = t + NSTAGE - 1 < n_tiles;
    if (fill) {
      const int sn = (t + NSTAGE - 1) % NSTAGE;
      nkq[NSTAGE - 2] = issue_k(sn);
      k0q[NSTAGE - 2] = key0;
      if constexpr (!ROLL_ALL) issue_v(sn);
    }

    if (t == alt_tiles) load_q(a.q_alt);
    const uint8_t* kt = smem + st * KT_B;
    const uint8_t* vt = smem + NSTAGE * KT_B + st * VT_B;
    // The LDS reads of the next product group are issued one after each product of the current
    // group, into the operand slots it has just consumed, so they land while the matrix core works
    // instead of stalling the next group's first product (and the exponentials queued behind it).
    constexpr bool RV = ROLL_ALL;
    if constexpr (!ROLL_ALL) {
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) ob[ks] = ld_bf16x8(kt + koff[0] + 32 * ks);
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- keys 0..31: S'^T = K (Q^T * scale * log2 e); K of keys 32..63 read behind the products
    // Wave priorities (s_setprio) order the two waves that share a SIMD: the first score products
    // (products and LDS reads only) issue at priority 3, both P.V groups at 1, the second score
    // group (products under the exponentials of the first half) at 0.  A wave that can feed the
    // matrix core from operands already in registers then wins the issue slots over one that is
    // about to wait on its exponentials.  Measured, interleaved: ABot (4 waves) 0.559 -> 0.539 ms
    // per pass, 480P (8 waves) -1 %.
    __builtin_amdgcn_s_setprio(3);
    f32x16_t s0 = negm;
    if constexpr (FOLLOW) s0 = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ob[ks], qreg[ks], s0, 0, 0, 0);
      ob[ks] = ld_bf16x8(kt + koff[1] + 32 * ks);
    }
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    if constexpr (ROLL_ALL)
      if (fill) issue_v((t + NSTAGE - 1) % NSTAGE);
    float sub0 = 0.f;
    if constexpr (MASKED) mask_half(s0, k0, nk);
    if constexpr (FOLLOW) {
      sub0 = follow_max(s0);
    } else {
      if (!MASKED && nk < 32) {
        int nkh = nk - 8 * hf;  // key score_key(r, hf) >= nk  <=>  score_key(r, 0) >= nk - 8 hf
        asm volatile("" : "+v"(nkh));
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (score_key(r, 0) >= nkh) s0[r] = -INFINITY;
      }
      if (t == 0) {
        // first tile: the running max starts at the max of its first half (key 0 is always valid)
        m_run = max_half(s0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s0[r] -= m_run;
          negm[r] = -m_run;
        }
      }
      sub0 = 0.f;
    }

    // ---- keys 32..63 on the matrix cores while P of keys 0..31 is formed (8 waves: and V of
    // keys 0..31 is read)
    f32x16_t s1 = negm;
    if constexpr (FOLLOW) s1 = f32x16_t{};
    bf16x8_t pb[4];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ob[ks], qreg[ks], s1, 0, 0, 0);
      if constexpr (RV) ob[ks] = ld_bf16x8(vt + voff + (ks % MBLK) * 32 * VP + 32 * (ks / MBLK));
    }
    float lsum = exp_half(s0, sub0, pb[0], pb[1]);
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (RV) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 48 / KSTEPS, 0);
    }
    // The running max is raised only when some score exceeds it by a lot (a row sum past
    // 2^60): the result is the same for any max, and P stays far below overflow.
    if (!FOLLOW && __any(lsum > 0x1p60f)) {
      // scores are relative to the old max (s1 too, its product started from the old -m_run)
      const float up = fmaxf(max_half(s0), 0.f);
      raise_by(up);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[r] -= up;
        s1[r] -= up;
        negm[r] = -m_run;
      }
      lsum = exp_half(s0, 0.f, pb[0], pb[1]);
    }
    l_run += lsum;
    if constexpr (MASKED) {
      mask_half(s1, k0 + 32, nk - 32);
    } else if (nk < kBN) {
      int nkh = nk - 32 - 8 * hf;
      asm volatile("" : "+v"(nkh));
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (score_key(r, 0) >= nkh) s1[r] = -INFINITY;
    }

    // ---- O^T += V^T P^T over keys 0..31 while P of keys 32..63 is formed (8 waves: and V of
    // keys 32..63 is read)
    __builtin_amdgcn_s_setprio(1);
    if constexpr (!RV) {
#pragma unroll
      for (int stp = 0; stp < 2; ++stp)
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb) ob[stp * MBLK + mb] = ld_bf16x8(vt + voff + mb * 32 * VP + 32 * stp);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int stp = 0; stp < 2; ++stp)
#pragma unroll
      for (int mb = 0; mb < MBLK; ++mb) {
        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ob[stp * MBLK + mb], pb[stp], o[mb], 0, 0, 0);
        if constexpr (RV) ob[stp * MBLK + mb] = ld_bf16x8(vt + voff + mb * 32 * VP + 32 * (stp + 2));
      }
    if constexpr (FOLLOW) {
      lsum = exp_half(s1, follow_max(s1), pb[2], pb[3]);
      if constexpr (RV) {
#pragma unroll
        for (int i = 0; i < 2 * MBLK; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    } else {
      lsum = exp_half(s1, 0.f, pb[2], pb[3]);
#pragma unroll
      for (int i = 0; i < 2 * MBLK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (RV) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 48 / (2 * MBLK), 0);
      }
      if (__any(lsum > 0x1p60f)) {
        const float up = fmaxf(max_half(s1), 0.f);
        raise_by(up);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s1[r] -= up;
          negm[r] = -m_run;
        }
        lsum = exp_half(s1, 0.f, pb[2], pb[3]);
      }
    }
    l_run += lsum;
    __builtin_amdgcn_s_setprio(0);
    if constexpr (!RV) {
#pragma unroll
      for (int stp = 2; stp < 4; ++stp)
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb) ob[(stp - 2) * MBLK + mb] = ld_bf16x8(vt + voff + mb * 32 * VP + 32 * stp);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (ROLL_ALL) {
      // tile t+1 landed, and every wave holds all it reads of tile t (the wait includes the LDS
      // reads), so tile t's stage is free from here on
      if (more) {
        if constexpr (NSTAGE == 2)
          wait_vm_barrier<0>();
        else if (t + 3 < n_tiles)
          wait_vm_barrier<2 * (KMIN + VMIN)>();
        else if (t + 2 < n_tiles)
          wait_vm_barrier<KMIN + VMIN>();
        else
          wait_vm_barrier<0>();
      }
      // ---- O^T += V^T P^T over keys 32..63, K of keys 0..31 of tile t+1 read behind the products
      // (after the last tile: a read of a stage nobody writes any more, never used)
      const uint8_t* kn = smem + ((t + 1) % NSTAGE) * KT_B;
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int stp = 2; stp < 4; ++stp)
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb) {
          const int i = (stp - 2) * MBLK + mb;
          o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ob[i], pb[stp], o[mb], 0, 0, 0);
          ob[i] = ld_bf16x8(kn + koff[0] + 32 * i);
        }
#pragma unroll
      for (int i = 0; i < 2 * MBLK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
    } else {
      // ---- O^T += V^T P^T over keys 32..63
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int stp = 2; stp < 4; ++stp)
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb)
          o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ob[(stp - 2) * MBLK + mb], pb[stp], o[mb], 0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
    }
  }

  const float l_row = half_swap_sum(l_run);
  const int qi = q_base + l32;
  if (nsp > 1) {
    // split keys: unnormalised O, running max and row sum of this split for the merge pass
    if (qi < a.Lq) {
      const int64_t row = ((int64_t)sp * a.Lq + qi) * a.H + h;
      float* po = a.part_o + row * D + 4 * hf;
#pragma unroll
      for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(f32x4_t*)(po + 32 * mb + 8 * g) = f32x4_t{o[mb][4 * g], o[mb][4 * g + 1], o[mb][4 * g + 2], o[mb][4 * g + 3]};
      if (hf == 0) {
        a.part_ml[2 * row] = m_run;
        a.part_ml[2 * row + 1] = l_row;
      }
    }
    return;
  }
  // Normalise, then write whole output rows: a lane holds O^T[d][query l32] for d = 32 mb + 8 g +
  // 4 hf + 0..3, so written directly every store instruction would touch 16 bytes of 32 rows.  The
  // wave's 32 rows go through its own part of the (now idle) tile stages instead and leave as
  // 16-byte pieces of consecutive bytes (4 or 8 whole rows per instruction).
  const float inv = 1.f / l_row;
  constexpr int OP = 2 * D + 16;  // LDS pitch of an output row: data + a 16-byte pad
  static_assert(NW * 32 * OP <= NSTAGE * (KT_B + VT_B), "output rows fit the tile stages");
  __syncthreads();  // every wave is done with the stages
  uint8_t* ob_lds = smem + wave * 32 * OP;
#pragma unroll
  for (int mb = 0; mb < MBLK; ++mb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2_t w = {pack_bf16x2(o[mb][4 * g] * inv, o[mb][4 * g + 1] * inv),
                         pack_bf16x2(o[mb][4 * g + 2] * inv, o[mb][4 * g + 3] * inv)};
      *(u32x2_t*)(ob_lds + l32 * OP + 2 * (32 * mb + 8 * g + 4 * hf)) = w;
    }
  constexpr int CPR = 2 * D / 16;   // 16-byte pieces per row
  constexpr int RPI = 64 / CPR;     // rows per instruction
#pragma unroll
  for (int j = 0; j < 32 / RPI; ++j) {
    const int r = RPI * j + lane / CPR, c = lane % CPR;
    const u32x4_t v = *(const u32x4_t*)(ob_lds + r * OP + 16 * c);
    if (q_base + r < a.Lq) *(u32x4_t*)((uint8_t*)a.out + ((int64_t)(q_base + r) * a.H + h) * (2 * D) + 16 * c) = v;
  }
}

// Split keys: merge the partial results of nsplit key ranges into out (bf16).  Thread i handles
// row r = i / (D / 4) of the [Lq * H] rows and its dims 4 (i % (D / 4)) .. +3:
// out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s with M = max_s m_s (empty splits: m = -inf).
// One thread per (row, 4 consecutive d): out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the
// splits in a fixed order.  The split loop is unrolled to the most splits the workspace holds, so
// every partial load of a thread is in flight at once (the pass is short and latency-bound).
constexpr int kMaxSplit = 16;
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* part_o, const float* part_ml, int nsplit,
                                                         int64_t rows, int D, uint16_t* out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int q4 = D / 4;
  if (i >= rows * q4) return;
  const int64_t r = i / q4;
  const int d = 4 * (int)(i - r * q4);
  float m[kMaxSplit], l[kMaxSplit];
  f32x4_t o[kMaxSplit];
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s) {
    if (s < nsplit) {
      const f32x2_t ml = *(const f32x2_t*)(part_ml + 2 * (s * rows + r));
      m[s] = ml[0];
      l[s] = ml[1];
      o[s] = *(const f32x4_t*)(part_o + (s * rows + r) * D + d);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s)
    if (s < nsplit) M = fmaxf(M, m[s]);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s) {
    if (s < nsplit && m[s] != -INFINITY) {
      const float w = __builtin_amdgcn_exp2f(m[s] - M);
      L += w * l[s];
      acc += w * o[s];
    }
  }
  const float inv = 1.f / L;
  *(u32x2_t*)(out + r * D + d) = u32x2_t{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
}

// Two shapes of the same kernel: 4 waves x 32 queries with two stages (two workgroups per CU),
// or 8 waves x 32 queries with four stages (one workgroup per CU; each K/V tile feeds twice the
// queries and loads run two tiles ahead).  The larger one runs about 10% faster per query once
// the grid fills the chip; with few query tiles its coarser grid leaves CUs idle, so pick by
// the number of dispatch rounds each needs on 256 CUs.  A grid that fills less than half of one
// round (few heads, e.g. one GPU's share of a head-sharded model) has its keys split so that the
// chip fills, when the caller's workspace holds the partial results.
template <bool MASKED>
static hipError_t launch_vt(const AttnBatch& in, int D, hipStream_t stream) {
  AttnBatch a = in;
  const AttnArgs& a0 = a.b[0];
  const int64_t wg4 = (int64_t)((a0.Lq + 127) / 128) * a0.H * a.nb, wg8 = (int64_t)((a0.Lq + 255) / 256) * a0.H * a.nb;
  const double rounds4 = (double)((wg4 + 511) / 512), rounds8 = 0.9 * (double)((wg8 + 255) / 256);
  // SKV_ATTN_WAVES=4 or 8 forces one shape (tests cover both on small inputs)
  const char* env = std::getenv("SKV_ATTN_WAVES");
  const int forced = (env && *env) ? std::atoi(env) : 0;
  // short key sequences (e.g. cross attention over a few hundred text tokens): a workgroup's
  // prologue and pipeline fill are a large part of its life, and two 4-wave workgroups per CU
  // overlap them where one 8-wave workgroup cannot (480P x 512 text tokens: 92 -> 88 us)
  int seq_tiles = 0;
  for (int i = 0; i < a.nb; ++i) {
    int nt = 0;
    for (int s_ = 0; s_ < a.b[i].nseg; ++s_) nt += (a.b[i].seg[s_].n + kBN - 1) / kBN;
    seq_tiles = nt > seq_tiles ? nt : seq_tiles;
  }
  bool big = forced == 8 || (forced != 4 && !(!MASKED && seq_tiles <= 16) && rounds8 < rounds4);
  // split keys: SKV_ATTN_SPLIT=0 never, =1 whenever the buffers allow (tests), unset: grids that fill
  // at most half of one dispatch round
  int nsplit = 1;
  if (!MASKED) {
    const char* se = std::getenv("SKV_ATTN_SPLIT");
    const int mode = (se && *se) ? std::atoi(se) : -1;
    int cap = kMaxSplit, max_tiles = 0;  // the merge pass handles at most kMaxSplit partials per row
    for (int i = 0; i < a.nb; ++i) {
      cap = a.b[i].split_cap < cap ? a.b[i].split_cap : cap;
      int nt = 0;
      for (int s_ = 0; s_ < a.b[i].nseg; ++s_) nt += (a.b[i].seg[s_].n + kBN - 1) / kBN;
      max_tiles = nt > max_tiles ? nt : max_tiles;
    }
    // splits a shape would take: as many as fit the grid into one round
    auto splits = [&](int64_t wgs, int64_t slots) -> int {
      if (mode == 0 || cap <= 1 || (mode != 1 && 2 * wgs > slots)) return 1;
      int want = (int)(slots / wgs);
      if (mode == 1 && want < 2) want = 2;
      want = want < cap ? want : cap;
      return want < max_tiles ? want : max_tiles;
    };
    const int s4 = splits(wg4, 512), s8 = splits(wg8, 256);
    // both shapes fit one round once split: take the one whose split grid fills more of the chip
    // (equal fill: the 8-wave shape, faster per tile)
    if (!forced && (s4 > 1 || s8 > 1)) big = (double)(wg8 * s8) / 256.0 >= (double)(wg4 * s4) / 512.0;
    nsplit = big ? s8 : s4;
    if (nsplit > 1) {
      for (int i = 0; i < a.nb; ++i) {
        int nt = 0;
        for (int s_ = 0; s_ < a.b[i].nseg; ++s_) nt += (a.b[i].seg[s_].n + kBN - 1) / kBN;
        a.b[i].nsplit = nsplit;
        a.b[i].split_tiles = (nt + nsplit - 1) / nsplit;
      }
    } else {
      for (int i = 0; i < a.nb; ++i) a.b[i].nsplit = 1;
    }
  }
  const int64_t wg = big ? wg8 : wg4;
  const dim3 grid((unsigned)(wg * nsplit));
  // masked with sinks: every row sees key 0, so the running max need not follow every half tile
  const bool follow = MASKED && a0.mS == 0;
  const int key = D * (big ? -1 : 1);
  if (!follow) {
    switch (key) {
      case 64: hipLaunchKernelGGL((attn_bf16_vt_kernel<64, 4, 2, MASKED, false>), grid, dim3(256), 0, stream, a); break;
      case 128: hipLaunchKernelGGL((attn_bf16_vt_kernel<128, 4, 2, MASKED, false>), grid, dim3(256), 0, stream, a); break;
      case -64: hipLaunchKernelGGL((attn_bf16_vt_kernel<64, 8, 4, MASKED, false>), grid, dim3(512), 0, stream, a); break;
      case -128: hipLaunchKernelGGL((attn_bf16_vt_kernel<128, 8, 4, MASKED, false>), grid, dim3(512), 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
  } else if constexpr (MASKED) {
    switch (key) {
      case 64: hipLaunchKernelGGL((attn_bf16_vt_kernel<64, 4, 2, true, true>), grid, dim3(256), 0, stream, a); break;
      case 128: hipLaunchKernelGGL((attn_bf16_vt_kernel<128, 4, 2, true, true>), grid, dim3(256), 0, stream, a); break;
      case -64: hipLaunchKernelGGL((attn_bf16_vt_kernel<64, 8, 4, true, true>), grid, dim3(512), 0, stream, a); break;
      case -128: hipLaunchKernelGGL((attn_bf16_vt_kernel<128, 8, 4, true, true>), grid, dim3(512), 0, stream, a); break;
      default: return hipErrorInvalidValue;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsplit <= 1) return e;
  for (int i = 0; i < a.nb && e == hipSuccess; ++i) {
    const int64_t rows = (int64_t)a.b[i].Lq * a.b[i].H;
    const int64_t threads = rows * (D / 4);
    hipLaunchKernelGGL(attn_merge_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream,
                       (const float*)a.b[i].part_o, (const float*)a.b[i].part_ml, nsplit, rows, D,
                       (uint16_t*)a.b[i].out);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_attention_bf16_vt(const AttnBatch& a, int D, hipStream_t stream) { return launch_vt<false>(a, D, stream); }

hipError_t launch_attention_bf16_masked(const AttnBatch& a, int D, hipStream_t stream) {
  return launch_vt<true>(a, D, stream);
}

}  // namespace skv
