/*
 * skv.h — streaming KV cache for chunk-causal video attention on MI355X (gfx950).
 *
 * C ABI of the hot path the LingBot-World 2.0 and ABot-World pages describe:
 * a new latent chunk of c frames attends to a bounded KV cache that holds S
 * never-evicted sink frames plus a sliding window of recent frames, with 3D
 * rotary embeddings that carry time either as an absolute frame offset or as a
 * relative slot index.  Pages cited below:
 *   [LB-causal]   "LingBot-World 2.0因果预训练范式深度剖析" (sheratonhq.com)
 *   [LB-fast]     "从40步到4步：LingBot-World 2.0实时推理蒸馏（causal_fast）原理与关键代码解读" (hmyw.cn)
 *   [LB-src]      LingBot-World 2.0 wan/ source map (kwkr.cn)
 *   [ABot-stream] "ABot-World流式因果推理深度解析：KV缓存与块级注意力如何让24小时连续生成不漂移" (lpnh.cn)
 *
 * Conventions shared by every entry point
 *   - Tensors are [tokens, heads, head_dim], row-major, tokens frame-major and
 *     row-major inside a latent frame of grid_h x grid_w tokens (F tokens).
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; it must be
 *     16-byte aligned.  The library allocates only the small host-side handle.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *     call only enqueues work on that stream and never synchronises, except
 *     kv_cache_gather, which fills a host array from host state.
 *   - Arguments are validated before anything is enqueued; on a validation error
 *     nothing is enqueued and the handle is unchanged.  A failed HIP launch
 *     returns SKV_ERR_HIP and poisons the handle: every later call on it returns
 *     SKV_ERR_STATE until kv_cache_reset.
 *   - Cache bookkeeping lives on the host and advances at enqueue time, so calls
 *     on one handle must be issued in order on one stream.  A handle is not
 *     thread-safe; separate handles are independent (one handle per layer).
 */
#ifndef SKV_H
#define SKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SKV_ABI_VERSION 5

typedef enum {
  SKV_OK = 0,
  SKV_ERR_NULL = 1,    /* a required pointer is NULL */
  SKV_ERR_CONFIG = 2,  /* invalid or unsupported configuration */
  SKV_ERR_SHAPE = 3,   /* n_frames / token counts out of range */
  SKV_ERR_ALIGN = 4,   /* a tensor pointer is not 16-byte aligned */
  SKV_ERR_STATE = 5,   /* call not valid in the handle's state (or poisoned handle) */
  SKV_ERR_HIP = 6      /* a HIP launch or runtime call failed */
} skv_status;

typedef enum { SKV_F32 = 0, SKV_BF16 = 1 } skv_dtype;

/* Time axis of the rotary embedding.
 *   ABS: frame f's key is stored already rotated at time id f; a chunk starting
 *        at frame s rotates its queries/keys at ids s..s+c-1 ([LB-src] 改造③,
 *        rope_apply(..., start_frame)).
 *   REL: the cache stores un-rotated keys (k_raw); each chunk rotates only the
 *        visible window, at time id = slot index in the visible sequence, clamped
 *        to [0, window_frames-1] ([ABot-stream] 机制三). */
typedef enum { SKV_ROPE_ABS = 0, SKV_ROPE_REL = 1 } skv_rope_mode;

typedef struct {
  int32_t heads, head_dim;      /* H, D.  bf16: D in {64, 128}; f32: D in {32, 64, 128} */
  int32_t grid_h, grid_w;       /* F = grid_h * grid_w tokens per latent frame */
  int32_t chunk_frames;         /* c >= 1: frames per generated chunk */
  int32_t sink_frames;          /* S >= 0: first frames never evicted */
  int32_t window_frames;        /* W >= S + c: frames visible to a chunk, sinks and chunk included */
  int32_t rope_t, rope_h, rope_w; /* head_dim split; 0,0,0 -> D-4*(D/6), 2*(D/6), 2*(D/6); each even, sum D */
  double rope_theta;            /* rotary base; 0 -> 10000 */
  int32_t rope_mode;            /* skv_rope_mode */
  int32_t dtype;                /* skv_dtype of every tensor the handle touches */
  int32_t fused_rope;           /* 0: the protocol above; 1: the library rotates (see below) */
} skv_config;

/* fused_rope = 1: callers pass UN-rotated q and k everywhere; rope_apply_window is
 * not used (SKV_ERR_STATE).  kv_cache_append_evict rotates k at each frame's
 * absolute id f while writing it (both modes), chunk_attention rotates q and
 * k_cur itself (into the workspace) before attending.  REL keeps its meaning: a
 * score depends only on the difference of the two time ids, and for ring and
 * current-chunk keys the slot-index difference equals the frame-number
 * difference, so those are attended with queries rotated at absolute ids
 * (start frame T + i); only the sink frames, whose slot ids are their frame
 * numbers, need the queries at their slot ids n_vis - c + i.  The window is
 * therefore never rotated again after the write-back (no per-chunk window pass,
 * no window workspace); kv_cache_gather returns keys rotated at absolute ids. */

typedef struct {
  int64_t n_appended;   /* frames appended since init/reset (T) */
  int32_t n_cached;     /* frames the cache holds now */
  int32_t n_sink_vis;   /* sink frames a chunk of c frames would see now */
  int32_t n_ring_vis;   /* non-sink history frames it would see */
  int32_t n_vis;        /* n_sink_vis + n_ring_vis + c */
  int32_t ring_start;   /* physical slot of the oldest visible non-sink frame (-1 if none) */
  int32_t window_ready; /* REL: 1 if rope_apply_window ran since the last append/reset */
  int32_t poisoned;     /* 1 after a failed launch, until kv_cache_reset */
} kv_cache_info_t;

typedef struct skv_cache skv_cache; /* opaque host-side handle */

/* ABI version (SKV_ABI_VERSION) and a static message for a status code. */
int skv_abi_version(void);
const char* skv_status_string(skv_status s);

/* Bytes the caller must allocate for each of the K store and the V store (one
 * size for both: H*D*P elements of cfg->dtype, P = W*F rounded up to a multiple
 * of 64) and for the workspace.  Physical layouts:
 *   K store  [H][W*F][D]   (head-major; slot s holds tokens [s*F, (s+1)*F));
 *   V store  V transposed per head, same key numbering: bf16 in tiles of 64 keys,
 *            [H][P/64][D][64] (element (h, d, key) at ((h*P/64 + key/64)*D + d)*64
 *            + key%64), fp32 in rows [H][D][P];
 *   workspace: first (REL only) the rotated visible window [H][(W-c)*F][D] (with
 *   fused_rope instead: q at absolute ids, k_cur at absolute ids and, REL, q at
 *   slot ids, [c*F][H][D] each), then the staged current-chunk values [H][D][P]
 *   with P = c*F rounded up to 64; then, for bf16 chunks whose attention grid
 *   would fill less than half of the chip (few heads: e.g. one GPU's share of
 *   a head-sharded model), at the next 256-byte boundary the fp32 partial
 *   results of up to 16 key splits ([splits][c*F][H][D], then [splits][c*F][H][2]),
 *   which chunk_attention merges.
 * Frame f < S lives in slot f, frame f >= S in slot S + (f-S) mod (W-S). */
skv_status kv_cache_bytes(const skv_config* cfg, size_t* store_bytes_each, size_t* workspace_bytes);

/* Bind caller-allocated stores and workspace (kv_cache_bytes gives the sizes) to
 * a new handle with zero frames appended ([ABot-stream] reset_stream()).  The
 * device memory is not touched.  *out receives the handle. */
skv_status kv_cache_init(const skv_config* cfg, void* k_store, void* v_store, void* workspace,
                         skv_cache** out);

/* Start a new stream on the same stores: forget every frame (counters to zero,
 * nothing on the device is touched) and clear the poisoned flag.  [ABot-stream]
 * "一次流式生成的完整链路": reset_stream() rebuilds the KV caches for a new
 * stream, while a prompt change (set_prompts) rebuilds only the text cache and
 * keeps the history, so a prompt swap never calls this.  Errors: SKV_ERR_NULL. */
skv_status kv_cache_reset(skv_cache* cache);

/* Free the host handle (device memory stays the caller's). NULL is a no-op. */
skv_status kv_cache_destroy(skv_cache* cache);

/* Write back n_frames clean frames ([LB-fast] 3. KV 缓存 滚动窗口; [ABot-stream]
 * 机制二 clean-context write-back).  k, v: [n_frames*F, H, D].  ABS: k must be
 * the rotated keys; REL: the raw keys.  Frames go to their ring slots; a frame
 * written to a ring slot evicts the frame that held it, which is the oldest
 * non-sink frame, so the logical cache is exactly the one the pages obtain by
 * shifting the post-sink entries left.  Requires 1 <= n_frames <= W - S. */
skv_status kv_cache_append_evict(skv_cache* cache, const void* k, const void* v, int32_t n_frames,
                                 void* stream);

/* 3D rotary embedding of x_in [n_frames*F, H, D] into x_out (may alias x_in)
 * ([LB-src] "改造③因果 RoPE 定位": a chunk's frames are rotated from start_frame on,
 * so they continue the absolute time axis of the frames before them; [ABot-stream]
 * 机制三: relative ids, the chunk takes the last slots of the visible window).
 * Token (frame i, row r, col w) is rotated at positions (t_i, r, w): head_dim
 * is split [time | height | width] and each adjacent pair (x_2k, x_2k+1) turns
 * by position * theta^(-2k/d_axis).  ABS: t_i = start_frame + i (start_frame >= 0).
 * REL: n_frames must equal c and t_i = n_vis - c + i (the chunk's slots);
 * start_frame is ignored.  fp32 arithmetic, angles reduced in fp64. */
skv_status rope_apply(const skv_cache* cache, const void* x_in, void* x_out, int32_t n_frames,
                      int64_t start_frame, void* stream);

/* q and k_cur of one chunk share their time ids ([LB-src] 改造③ rotates both with the
 * same start_frame; [ABot-stream] 机制三 places both in the chunk's slots), so one
 * launch rotates both: the same result as rope_apply(q_in -> q_out) followed by
 * rope_apply(k_in -> k_out) with these n_frames / start_frame.  Each output may
 * alias its own input; the q and k tensors must not overlap each other. */
skv_status rope_apply_qk(const skv_cache* cache, const void* q_in, void* q_out, const void* k_in, void* k_out,
                         int32_t n_frames, int64_t start_frame, void* stream);

/* REL only ([ABot-stream] 机制三: the cache keeps un-rotated keys and only the
 * visible window is rotated, at ids counted from the window's start and clamped
 * to [0, window-1]): rotate the visible history k_raw (sinks, then the visible ring
 * frames oldest first) at time ids 0..n_vis-c-1 into the workspace, once per
 * chunk; its result serves every pass until the next append or reset.
 * Errors: SKV_ERR_STATE in ABS mode or under fused rotation. */
skv_status rope_apply_window(skv_cache* cache, void* stream);

/* Stage the current chunk's values v_cur [c*F, H, D] in the workspace, in the
 * transposed layout the attention kernel reads (the V store's layout over c*F
 * keys, padded with zeros to a multiple of 64 keys).  chunk_attention does this itself when
 * it is given v_cur; calling it separately lets a caller time or overlap it.
 * n_frames must equal c. */
skv_status kv_cache_stage_v(skv_cache* cache, const void* v_cur, int32_t n_frames, void* stream);

/* Everything an attention pass needs before chunk_attention, in one launch: the
 * result of rope_apply_qk(q_in -> q_out, k_in -> k_out, n_frames, start_frame)
 * followed by kv_cache_stage_v(v_cur) ([LB-src] 改造③ rotates q and k with one
 * start_frame; [LB-fast] 3. KV 缓存 滚动窗口 feeds the chunk's own K/V to the
 * window attention).  bf16 runs the rotary blocks and the staging blocks in one
 * grid, fp32 as two launches.  n_frames must equal c; argument errors are those
 * of the two calls, and SKV_ERR_STATE under fused rotation (chunk_attention then
 * rotates q and k_cur and stages v_cur itself, in one launch).  v_cur must not
 * overlap q_out or k_out.  Then call chunk_attention(q_out, k_out, NULL). */
skv_status kv_cache_prepare_pass(skv_cache* cache, const void* q_in, void* q_out, const void* k_in, void* k_out,
                                 const void* v_cur, int32_t n_frames, int64_t start_frame, void* stream);

/* Chunk attention ([LB-fast] 3. KV 缓存 滚动窗口: attention over the window
 * slice; [ABot-stream] 机制二: block-causal, frames of a chunk see each other).
 * q, k_cur, v_cur: [c*F, H, D], q and k_cur already rotated with rope_apply;
 * v_cur may be NULL to use the values staged by kv_cache_stage_v (since the
 * last append or reset; SKV_ERR_STATE otherwise).
 * out[i] = softmax(q_i . K^T / sqrt(D)) V over the visible keys: the visible
 * sink frames, the visible ring frames, and the current chunk.  The cache is
 * read only.  fp32 softmax and accumulation; out in cfg dtype.  n_frames must
 * equal c.  REL mode with cached history requires rope_apply_window first.
 * bf16 runs one of two kernel shapes (4 or 8 waves per workgroup), chosen from
 * the grid size; the environment variable SKV_ATTN_WAVES=4 or 8, read at each
 * call, forces one of them (the two may round differently).  A bf16 grid that
 * would fill at most half of the chip (few heads, e.g. one GPU's share of a
 * head-sharded model) has each query tile's keys split over several
 * workgroups, whose partial results (in the workspace) a second kernel merges
 * on the same stream; SKV_ATTN_SPLIT=0 disables that, =1 splits whenever the
 * workspace has room (results differ from the unsplit ones by rounding only). */
skv_status chunk_attention(const skv_cache* cache, const void* q, const void* k_cur, const void* v_cur,
                           int32_t n_frames, void* out, void* stream);

/* Several chunk_attention calls of one shape in one launch ([LB-fast] table of
 * inference modes: causal_pretrain runs every step twice, with and without the
 * prompt, for classifier-free guidance; each of the two keeps its own cache).
 * caches[i], q[i], k_cur[i], v_cur[i], out[i] (host arrays of n_caches device
 * pointers, 1 <= n_caches <= 4) mean what they mean for chunk_attention; v_cur
 * may be NULL (every element uses its staged values) and so may any v_cur[i].
 * Every handle must have the same configuration (SKV_ERR_CONFIG otherwise) and
 * appear once (SKV_ERR_STATE).  All elements are checked before anything is
 * enqueued; then given values are staged and one kernel covers all elements
 * (bf16; fp32 launches once per element).  A failed launch poisons every
 * handle of the batch. */
skv_status chunk_attention_batch(const skv_cache* const* caches, int32_t n_caches, const void* const* q,
                                 const void* const* k_cur, const void* const* v_cur, int32_t n_frames,
                                 void* const* out, void* stream);

/* Cross attention over cached text K/V ([LB-causal] CrossAttention_KVCache;
 * [ABot-stream] 512 text tokens computed once): out = softmax(q K_text^T / sqrt(D)) V_text,
 * no rotary embedding, no mask.  q/out [n_q, H, D]; k_text/v_text [n_text, H, D].
 * Independent of any cache handle (a prompt swap keeps the KV history). */
skv_status cross_attention(const void* q, int32_t n_q, const void* k_text, const void* v_text,
                           int32_t n_text, int32_t heads, int32_t head_dim, int32_t dtype, void* out,
                           void* stream);

/* Prepared text cache for cross attention.  The text K/V are computed once per
 * prompt and reused by every later chunk and pass ([LB-fast] "3. KV 缓存 滚动窗口",
 * its note on the cross-attention cache; [ABot-stream] "一次流式生成的完整链路",
 * step 1: the 512-token text cache is built once, and a prompt change rebuilds
 * only it), so their layout is fixed once:
 * text_cache_prepare lays k_text and v_text out into `store`, a caller-allocated
 * device buffer of text_cache_bytes(...) bytes, 256-byte aligned.  bf16, with
 * P = roundup(n_text, 64) and the keys past n_text zero: K head-major [H][P][D]
 * (one head's keys contiguous, as in the K store), then, at the next 256-byte
 * boundary, V^T in tiles of 64 keys, [H][P/64][D][64]; fp32: copies of k_text
 * and v_text ([n_text, H, D]) back to back, the second at a 256-byte boundary.
 * cross_attention_cached then attends q/out [n_q, H, D] over the store with the
 * same result definition as cross_attention (bf16: the matrix-core kernel of
 * chunk_attention, which reads V^T with direct-to-LDS loads).  The store is
 * read-only for cross_attention_cached; replacing the prompt means preparing
 * again.  Same checks as cross_attention (heads 1..4096; bf16 D 64/128, fp32 D
 * 32/64/128; 1 <= n_text <= 2^30); SKV_ERR_SHAPE also when a head's keys do not
 * fit the bf16 kernel's 32-bit offsets. */
skv_status text_cache_bytes(int32_t n_text, int32_t heads, int32_t head_dim, int32_t dtype, size_t* bytes);
skv_status text_cache_prepare(const void* k_text, const void* v_text, int32_t n_text, int32_t heads,
                              int32_t head_dim, int32_t dtype, void* store, void* stream);
skv_status cross_attention_cached(const void* q, int32_t n_q, const void* store, int32_t n_text,
                                  int32_t heads, int32_t head_dim, int32_t dtype, void* out, void* stream);

/* Host-side bookkeeping of the handle. */
skv_status kv_cache_info(const skv_cache* cache, kv_cache_info_t* info);

/* Logical snapshot: the cache as the pages describe it ([LB-fast] "3. KV 缓存
 * 滚动窗口" and [LB-causal] "Attention Sink": the first S frames, then the most
 * recent frames, oldest first), copied into k_out/v_out [n_cached*F, H, D]
 * (device; keys as stored: rotated in ABS mode and under fused rotation, raw in
 * REL mode) with their frame ids in frame_ids_host[n_cached] (host; may be NULL;
 * kv_cache_info gives n_cached).  The ids are filled before returning; the copies
 * are enqueued on stream.  Errors: SKV_ERR_NULL / SKV_ERR_ALIGN on k_out, v_out;
 * SKV_ERR_STATE on a poisoned handle. */
skv_status kv_cache_gather(const skv_cache* cache, void* k_out, void* v_out, int64_t* frame_ids_host,
                           void* stream);

/* Restore a snapshot taken with kv_cache_gather, on a handle of the same
 * configuration (a stream resumed where it stopped; [ABot-stream] "一次流式生成的
 * 完整链路": a stream keeps its KV history until reset_stream).  k, v: the gathered
 * [n_frames*F, H, D] device tensors; frame_ids_host: the n_frames gathered ids.
 * Each frame goes back to the slot its id maps to, so the handle afterwards holds
 * what it held when gathered (n_appended = last id + 1; bytes, slots and the
 * visible ranges identical, and with them every later result).  n_frames == 0
 * leaves an empty cache (as kv_cache_reset).  REL mode needs rope_apply_window
 * again before the next attention.  Errors: SKV_ERR_NULL / SKV_ERR_ALIGN on
 * pointers; SKV_ERR_SHAPE when the ids are not exactly the ones kv_cache_gather
 * reports for n_appended = last id + 1; SKV_ERR_STATE on a poisoned handle. */
skv_status kv_cache_restore(skv_cache* cache, const void* k, const void* v, const int64_t* frame_ids_host,
                            int32_t n_frames, void* stream);

/* Many chunks at once under the sink + window block-causal mask ([ABot-stream]
 * 机制二: a chunk's queries see their own chunk and the window of earlier chunks,
 * frames inside a chunk see each other; the same mask serves training, where it is
 * FlexAttention's block_mask.  [LB-fast] "3. KV 缓存 滚动窗口": the window keeps the
 * first S frames and the most recent frames).  No cache handle: cfg gives H, D,
 * F = grid_h * grid_w, c, S, W and dtype (bf16 only).
 * k, v: [n_frames*F, H, D], the keys already rotated (e.g. rope_apply at absolute
 * frame ids); q, out: [(n_frames - q_frame0)*F, H, D], the rotated queries of frames
 * q_frame0 .. n_frames-1 (frames before q_frame0 are context only, e.g. reference
 * sinks).  Query frame i lies in the chunk ending at e = q_frame0 + c*((i-q_frame0)/c + 1)
 * and sees key frame j iff j < e and (j < S or j >= e - (W - S)): exactly the keys a
 * chunk sees when it is streamed through a cache with S sinks and window W.
 * workspace: block_causal_workspace_bytes(cfg, n_frames) bytes of device memory
 * (the values are transposed there first, in the V store's bf16 tile layout).
 * Requires (n_frames - q_frame0) % c == 0.
 * Errors: SKV_ERR_NULL / SKV_ERR_ALIGN on pointers; SKV_ERR_CONFIG for an invalid or
 * non-bf16 cfg; SKV_ERR_SHAPE for frame counts out of range or a sequence too long
 * for 32-bit offsets within one head. */
skv_status block_causal_workspace_bytes(const skv_config* cfg, int32_t n_frames, size_t* bytes);
skv_status block_causal_attention(const skv_config* cfg, const void* q, const void* k, const void* v,
                                  int32_t n_frames, int32_t q_frame0, void* workspace, void* out, void* stream);

/* block_causal_attention for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same result, with the workspace taken from a static device array the library
 * owns (SKV_NOALLOC_SCRATCH_BYTES = 64 MiB on each device it runs on, held until
 * the process ends) instead of a caller's buffer.  It allocates nothing: the
 * array's address is looked up once per device on the first call (with that
 * device current).  Every call on a device uses that device's one array, so
 * calls that overlap on one device race (one at a time per device, e.g. one
 * stream).  Arguments and errors are those of block_causal_attention, plus
 * SKV_ERR_SHAPE when block_causal_workspace_bytes(cfg, n_frames) exceeds
 * SKV_NOALLOC_SCRATCH_BYTES and SKV_ERR_HIP when the array cannot be located. */
#define SKV_NOALLOC_SCRATCH_BYTES (64u << 20)
skv_status block_causal_attention_noalloc(const skv_config* cfg, const void* q, const void* k, const void* v,
                                          int32_t n_frames, int32_t q_frame0, void* out, void* stream);

/* One step of the few-step sampler between attention passes ([LB-fast]
 * "2. 4 步采样": the forward gives a flow-matching velocity, x0 is recovered in
 * one step and re-noised to the next, smaller timestep unless it was the last;
 * the conversion runs in double precision).  Element-wise over n elements of
 * dtype (any layout):
 *   v      = v_cond, or v_uncond + cfg_scale * (v_cond - v_uncond) when
 *            v_uncond is not NULL (guidance of the causal_pretrain mode);
 *   x0     = x_t - sigma * v                       -> x0_out (if not NULL);
 *   x_next = (1 - sigma_next) * x0 + sigma_next * noise -> x_next_out (if not NULL;
 *            needs noise).
 * Arithmetic in fp64, results rounded to dtype (bf16: to fp32, then to bf16,
 * each to nearest even).  Outputs may alias x_t (each element is read before it
 * is written).  sigma for timestep t of 1000 training steps is t / 1000 in the
 * schedules the tests use; the call takes the sigmas themselves.
 * Errors: NULL x_t / v_cond, both outputs NULL, or x_next_out without noise ->
 * SKV_ERR_NULL; misaligned pointer -> SKV_ERR_ALIGN; bad dtype or non-finite
 * scalar -> SKV_ERR_CONFIG; n < 0 -> SKV_ERR_SHAPE; n == 0 enqueues nothing. */
skv_status sampler_step(const void* x_t, const void* v_cond, const void* v_uncond, double cfg_scale,
                        const void* noise, int64_t n, double sigma, double sigma_next, int32_t dtype,
                        void* x0_out, void* x_next_out, void* stream);

/* Test hook for the failure path: the next n launches or device copies the
 * library makes (any entry point) report a HIP failure without launching
 * anything, as a failed launch would (SKV_ERR_HIP; a handle's call is then
 * poisoned until kv_cache_reset).  n <= 0 disarms it.  Process-wide; for tests
 * of the error handling only, no GPU work is involved. */
void skv_debug_fail_launches(int32_t n);

#ifdef __cplusplus
}
#endif
#endif /* SKV_H */
