// Device-side helpers shared by the gfx950 kernels: vector types, bf16
// conversion, and the argument blocks the host fills.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// bf16 <-> f32.  Widening is exact; narrowing rounds to nearest even.
__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

// One run of frames for the frame-copy and rotary kernels: frames
// [start, start+count) of the launch read source frame src0+(i-start) and
// write destination frame dst0+(i-start).
struct FrameRun {
  int32_t start, count, src0, dst0;
};

// Strided view of a [frames*F tokens, H, D] tensor:
// element (token t, head h, d) is at base + t*tok_stride + h*head_stride + d.
struct TokView {
  void* base;
  int64_t tok_stride, head_stride;
};

// Transposed bf16 values (V^T) are kept in tiles of kVtKeys keys: tile b of head h holds
// V^T[h][d][64 b + j] for all d at h*hs + b*64*D + d*64 + j (16 KB for D = 128), so a write of
// 64 keys and a read of one attention tile are whole, contiguous tiles when 64-aligned.
constexpr int kVtKeys = 64;

// One contiguous range of visible keys for the attention kernels.
// Key j of the range, head h, dim d: K at k + j*k_rs + h*k_hs + d.
// V: token-major (fp32 and the cross-attention kernel): v + h*v_hs + j*v_rs + d*v_ds
// (v_rs = H*D, v_ds = 1); transposed fp32 rows: v_rs = 1, v_ds = row length;
// transposed bf16 (tiled, the cache-path kernel): v points at the tile that holds the range's
// first key, which sits at position v_phase of it, so key j is at
// v + h*v_hs + ((v_phase + j) / 64)*64*D + d*64 + (v_phase + j) % 64.
struct KvSeg {
  const void* k;
  const void* v;
  int64_t k_hs, k_rs, v_hs, v_rs, v_ds;
  int32_t n;
  int32_t v_al16;   // transposed V: 16-byte pieces of 8 keys line up (row starts / v_phase + start)
  int32_t v_phase;  // tiled bf16 V^T: position of the range's first key in its tile
};

struct AttnArgs {
  const void* q;   // [Lq, H, D]
  void* out;       // [Lq, H, D]
  KvSeg seg[4];
  int32_t nseg;
  int32_t Lq, H;
  float sl2;       // softmax scale * log2(e)
  // key ranges from seg[alt_seg] on are attended with the queries at q_alt (same layout as q)
  const void* q_alt;
  int32_t alt_seg;
  // many chunks at once under the sink + window block-causal mask (masked kernel only):
  // frames of mF tokens, query frames from mq0 in chunks of mc frames, mS sinks, window mW;
  // seg[0] then describes the keys / V^T of the whole sequence
  int32_t mF, mq0, mc, mS, mW;
  // split keys (unmasked kernel): nsplit workgroups per query tile, split s taking tiles
  // [s * split_tiles, (s + 1) * split_tiles) of the key sequence, write instead of out the
  // unnormalised O to part_o [nsplit][Lq][H][D] and (running max in log2 units, row sum) to
  // part_ml [nsplit][Lq][H][2]; a merge pass combines them.  nsplit <= 1: no split.  split_cap:
  // the most splits the part buffers hold (set by the host; 0: never split).
  float* part_o;
  float* part_ml;
  int32_t split_cap;
  int32_t nsplit, split_tiles;
};

// Up to kMaxAttnBatch independent attention problems of one shape (same Lq, H, D) in one
// launch, e.g. the conditional and unconditional caches of guidance: workgroup ids cover the
// query tiles of element 0, then of element 1, ...
constexpr int kMaxAttnBatch = 4;
struct AttnBatch {
  AttnArgs b[kMaxAttnBatch];
  int32_t nb;
};

// Bijective remap of a workgroup id so that workgroups the dispatcher sends to
// the same XCD (ids congruent mod 8) work on consecutive tiles.
__device__ __forceinline__ int xcd_remap(int pid, int total) {
  const int q = total >> 3, r = total & 7;
  const int xcd = pid & 7, idx = pid >> 3;
  return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

}  // namespace skv
