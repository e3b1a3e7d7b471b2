"""Plain float64 CPU oracle of chunk-causal attention over a sink + sliding-window KV cache.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the product path.

The pages this follows (cited below by the short name in brackets):

* [LB-causal]  "LingBot-World 2.0因果预训练范式深度剖析：为什么它能持续生成视频而不'掉画质'"
               (sheratonhq.com/news/156439)
* [LB-fast]    "从40步到4步：LingBot-World 2.0实时推理蒸馏（causal_fast）原理与关键代码解读"
               (hmyw.cn/news/135683)
* [LB-src]     the LingBot-World 2.0 ``wan/`` source-map page (kwkr.cn/news/564388)
* [ABot-stream] "ABot-World流式因果推理深度解析：KV缓存与块级注意力如何让24小时连续生成不漂移"
               (lpnh.cn/news/2488095)
* [ABot-LF]    "无限生成的秘密：ABot-World如何用Causal Forcing与LongForcing蒸馏实现无限世界推演"
               (nxmr.cn/news/121609)

Where the pages leave a step open, the reading taken here is stated at the
function that implements it.  Nothing here is blocked, fused or reordered
beyond what the definitions state; row blocking in ``attention`` only bounds
memory and keeps every row's softmax exact.

Tensor layout everywhere: ``[tokens, heads, head_dim]``, tokens frame-major and,
inside a latent frame of ``grid_h x grid_w`` tokens, row-major.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

THETA_DEFAULT = 10000.0


# --------------------------------------------------------------------------- RoPE
def rope_split(head_dim: int) -> Tuple[int, int, int]:
    """Split of head_dim into (time, height, width) rotary parts.

    [LB-fast] section "3. KV 缓存 滚动窗口" and [LB-src] section "改造③因果 RoPE 定位"
    only say the rotary embedding is three-dimensional; no split is printed.
    Reading taken: height and width get 2*floor(D/6) dims each and time gets the
    rest, which gives 24/20/20 at D=64 and 44/42/42 at D=128.
    """
    d = int(head_dim)
    hw = 2 * (d // 6)
    return d - 2 * hw, hw, hw


def axis_frequencies(d_axis: int, theta: float = THETA_DEFAULT) -> np.ndarray:
    """Angular frequencies of one rotary axis: omega_k = theta^(-2k/d_axis), k < d_axis/2.

    Textbook rotary embedding (RoFormer); base theta = 10000 because the pages
    name none.
    """
    k = np.arange(d_axis // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * k / float(d_axis))


def token_grid_positions(grid_h: int, grid_w: int) -> Tuple[np.ndarray, np.ndarray]:
    """Row and column index of every token of one latent frame (row-major order)."""
    idx = np.arange(grid_h * grid_w)
    return idx // grid_w, idx % grid_w


def rope_3d(x: np.ndarray, frame_time_ids: Sequence[float], grid_h: int, grid_w: int,
            split: Optional[Tuple[int, int, int]] = None,
            theta: float = THETA_DEFAULT) -> np.ndarray:
    """3D rotary embedding of ``x`` [n_frames*F, H, D] (float64), returned as a new array.

    Token (frame i, row r, col c) has positions (t_i, r, c); ``frame_time_ids``
    gives t_i per frame.  head_dim is cut into [time | height | width] parts; in
    each part, the adjacent pair (x_2k, x_2k+1) is turned by the angle
    position * omega_k, i.e. (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a).

    [LB-causal] "Attention Sink" section and [LB-src] "改造③": the frame offset
    (start_frame) places a new chunk's frames at their true time position.
    """
    x = np.asarray(x, dtype=np.float64)
    n_tok, _, d = x.shape
    f = grid_h * grid_w
    t_ids = np.asarray(frame_time_ids, dtype=np.float64)
    if n_tok != len(t_ids) * f:
        raise ValueError("token count does not match frames x grid")
    split = rope_split(d) if split is None else tuple(split)
    if sum(split) != d or any(s % 2 for s in split):
        raise ValueError("bad rotary split")
    rows, cols = token_grid_positions(grid_h, grid_w)
    pos_t = np.repeat(t_ids, f)
    pos_h = np.tile(rows, len(t_ids)).astype(np.float64)
    pos_w = np.tile(cols, len(t_ids)).astype(np.float64)
    out = x.copy()
    off = 0
    for d_axis, pos in zip(split, (pos_t, pos_h, pos_w)):
        if d_axis:
            ang = pos[:, None] * axis_frequencies(d_axis, theta)[None, :]   # [tokens, d_axis/2]
            cos = np.cos(ang)[:, None, :]
            sin = np.sin(ang)[:, None, :]
            x0 = x[:, :, off:off + d_axis:2]
            x1 = x[:, :, off + 1:off + d_axis:2]
            out[:, :, off:off + d_axis:2] = x0 * cos - x1 * sin
            out[:, :, off + 1:off + d_axis:2] = x0 * sin + x1 * cos
        off += d_axis
    return out


# ------------------------------------------------------------------ cache list
class CacheList:
    """The logical KV cache: an ordered list of (frame id, K_f, V_f).

    [LB-causal] "滑动窗口 KV 缓存" / "Attention Sink" sections and [LB-fast]
    "3. KV 缓存 滚动窗口": the cache holds at most ``window`` frames; when a new
    frame would overflow it, the oldest frame after the first ``sink`` frames is
    pushed out and the rest shift left; the first ``sink`` frames are never
    evicted.  [ABot-stream] "机制一" describes the same roll with the reference
    latents pinned at the front.

    Readings: eviction is by whole frames (the pages speak of frames and of
    tokens); ``window`` counts sink frames too ("6 permanent + 12 sliding" = 18).
    """

    def __init__(self, sink: int, window: int):
        if sink < 0 or window <= 0 or sink > window:
            raise ValueError("need 0 <= sink <= window, window > 0")
        self.sink = int(sink)
        self.window = int(window)
        self.entries: List[Tuple[int, np.ndarray, np.ndarray]] = []
        self.n_appended = 0

    def append(self, k_frames: Sequence[np.ndarray], v_frames: Sequence[np.ndarray]) -> None:
        """Push frames one by one; after each push, evict entry [sink] while over capacity."""
        n = len(k_frames)
        if n != len(v_frames):
            raise ValueError("k/v frame count mismatch")
        if n < 1 or n > self.window - self.sink:
            raise ValueError("append size must be in [1, window - sink]")
        for kf, vf in zip(k_frames, v_frames):
            self.entries.append((self.n_appended, kf, vf))
            self.n_appended += 1
            while len(self.entries) > self.window:
                del self.entries[self.sink]

    def frame_ids(self) -> List[int]:
        return [e[0] for e in self.entries]


def visible_history(entries: Sequence, chunk: int, sink: int, window: int) -> list:
    """Cached entries visible to a new chunk of ``chunk`` frames.

    [LB-fast] "3. KV 缓存 滚动窗口": attention is taken over the last
    ``max_attention_size`` positions of the cache after the new chunk is written,
    and the sink frames are kept.  Equivalently, before writing: the whole cache
    while it and the chunk fit in the window, else the sink frames plus the most
    recent (window - sink - chunk) frames.  The chunk itself is always visible
    in full to each of its queries ([ABot-stream] "机制二": frames inside a block
    see each other; future blocks are never seen).
    """
    entries = list(entries)
    if len(entries) + chunk <= window:
        return entries
    keep = window - sink - chunk
    tail = entries[len(entries) - keep:] if keep > 0 else []
    return entries[:sink] + tail


# ------------------------------------------------------------------ attention
def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
              rows: Optional[np.ndarray] = None, scale: Optional[float] = None,
              block_rows: int = 1024) -> np.ndarray:
    """softmax(q k^T * scale) v per head, float64; scale defaults to 1/sqrt(head_dim).

    q [Lq, H, D], k/v [Lk, H, D].  ``rows`` selects a subset of query rows (the
    result then has len(rows) rows).  The 1/sqrt(D) scale is the textbook one;
    the pages do not print it.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if rows is not None:
        q = q[np.asarray(rows)]
    lq, h, d = q.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = np.empty((lq, h, v.shape[2]), dtype=np.float64)
    for hh in range(h):
        kh = k[:, hh, :]
        vh = v[:, hh, :]
        for r0 in range(0, lq, block_rows):
            s = (q[r0:r0 + block_rows, hh, :] @ kh.T) * scale
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[r0:r0 + block_rows, hh, :] = p @ vh
    return out


def block_causal_visible(n_frames: int, q_frame0: int, chunk_frames: int, sink_frames: int,
                         window_frames: int) -> np.ndarray:
    """[n_frames - q_frame0, n_frames] boolean: may query frame i (row i - q_frame0) see key frame j?

    [ABot-stream] 机制二 (block-causal mask: a chunk's queries see their own chunk and
    the window of earlier chunks, frames of a chunk see each other; the same structure
    in training, with FlexAttention's block_mask) and [LB-fast] "3. KV 缓存 滚动窗口"
    (the window keeps the sink frames and the most recent frames).  Query frame i lies
    in the chunk ending (exclusive) at e = q_frame0 + c * ((i - q_frame0) // c + 1);
    it sees key frame j iff j < e and (j < S or j >= e - (W - S)): the sinks plus the
    last W - S frames up to its chunk's end, i.e. exactly what streaming chunk by chunk
    shows that chunk.
    """
    if (n_frames - q_frame0) % chunk_frames or not 0 <= q_frame0 < n_frames:
        raise ValueError("query frames must be whole chunks")
    i = np.arange(q_frame0, n_frames)[:, None]
    j = np.arange(n_frames)[None, :]
    e = q_frame0 + chunk_frames * ((i - q_frame0) // chunk_frames + 1)
    return (j < e) & ((j < sink_frames) | (j >= e - (window_frames - sink_frames)))


def block_causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, frame_tokens: int, chunk_frames: int,
                           sink_frames: int, window_frames: int, q_frame0: int = 0,
                           rows: Optional[np.ndarray] = None, block_rows: int = 1024) -> np.ndarray:
    """Many chunks at once under the sink + window block-causal mask (plain definition).

    q: the already-rotated queries of frames q_frame0 .. n_frames-1 ([(n - q0) F, H, D]);
    k, v: the already-rotated keys and the values of all n frames ([n F, H, D]).  Each
    query row is a softmax over the keys its frame may see (``block_causal_visible``),
    scaled by 1/sqrt(D).  ``rows`` selects query rows.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    f = int(frame_tokens)
    n = k.shape[0] // f
    vis = block_causal_visible(n, q_frame0, chunk_frames, sink_frames, window_frames)
    row_ids = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    q = q[row_ids]
    lq, h, d = q.shape
    scale = 1.0 / math.sqrt(d)
    key_frame = np.arange(n * f) // f
    out = np.empty((lq, h, v.shape[2]), dtype=np.float64)
    for r0 in range(0, lq, block_rows):
        rr = row_ids[r0:r0 + block_rows]
        allowed = vis[rr // f][:, key_frame]          # [rows, keys]
        for hh in range(h):
            s = (q[r0:r0 + block_rows, hh, :] @ k[:, hh, :].T) * scale
            s = np.where(allowed, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=1, keepdims=True)
            out[r0:r0 + block_rows, hh, :] = p @ v[:, hh, :]
    return out


def cross_attention(q: np.ndarray, k_text: np.ndarray, v_text: np.ndarray,
                    rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Attention of video queries over cached text keys/values: no RoPE, no mask.

    [LB-causal] end of the "Attention Sink" section and [LB-fast] "另外两个缓存":
    the text K/V are computed once and reused by every chunk; [ABot-stream]
    "一次流式生成的完整链路" gives 512 text tokens.  Reading: all text tokens are
    valid (no padding mask).
    """
    return attention(q, k_text, v_text, rows=rows)


# ------------------------------------------------------------ streaming model
class StreamingOracle:
    """One attention layer's streaming state: cache list + rotary bookkeeping.

    Modes ([LB-src] "改造③" for ``abs``; [ABot-stream] "机制三" for ``rel``):

    * ``abs``: frame f's key is stored already rotated at time id f; a new chunk
      starting at frame s rotates its queries/keys at ids s .. s+c-1.
    * ``rel``: the cache stores un-rotated keys (k_raw); at each chunk the visible
      keys are rotated at their slot index j in the visible sequence (history then
      the chunk), time ids clamped to [0, window-1]; queries take the ids of the
      chunk's slots.  Reading: ids are slot indices, so the clamp never binds while
      the visible sequence is at most ``window`` frames; it is kept as a guard.

    Per chunk the caller runs any number of attention passes with the cache
    unchanged and then appends the clean chunk ([LB-fast] "3. KV 缓存 滚动窗口";
    [ABot-stream] "机制二" clean-context write-back).
    """

    def __init__(self, heads: int, head_dim: int, grid_h: int, grid_w: int,
                 chunk_frames: int, sink_frames: int, window_frames: int,
                 rope_mode: str = "abs", theta: float = THETA_DEFAULT,
                 split: Optional[Tuple[int, int, int]] = None):
        if rope_mode not in ("abs", "rel"):
            raise ValueError("rope_mode must be 'abs' or 'rel'")
        if window_frames < sink_frames + chunk_frames:
            raise ValueError("window must hold sink + chunk")
        self.h, self.d = int(heads), int(head_dim)
        self.gh, self.gw = int(grid_h), int(grid_w)
        self.f = self.gh * self.gw
        self.c, self.s, self.w = int(chunk_frames), int(sink_frames), int(window_frames)
        self.mode = rope_mode
        self.theta = float(theta)
        self.split = rope_split(self.d) if split is None else tuple(split)
        self.cache = CacheList(self.s, self.w)

    # -- bookkeeping
    @property
    def n_appended(self) -> int:
        return self.cache.n_appended

    def visible(self) -> list:
        return visible_history(self.cache.entries, self.c, self.s, self.w)

    def n_vis(self, n_frames: Optional[int] = None) -> int:
        n = self.c if n_frames is None else n_frames
        return len(visible_history(self.cache.entries, n, self.s, self.w)) + n

    def _rope(self, x: np.ndarray, ids: Sequence[float]) -> np.ndarray:
        return rope_3d(x, ids, self.gh, self.gw, self.split, self.theta)

    def _clamp(self, ids):
        return [min(max(int(i), 0), self.w - 1) for i in ids]

    def query_time_ids(self) -> List[int]:
        if self.mode == "abs":
            s0 = self.n_appended
            return list(range(s0, s0 + self.c))
        nv = self.n_vis()
        return self._clamp(range(nv - self.c, nv))

    def frames_of(self, x: np.ndarray, n: int) -> List[np.ndarray]:
        x = np.asarray(x, dtype=np.float64)
        if x.shape != (n * self.f, self.h, self.d):
            raise ValueError(f"expected {(n * self.f, self.h, self.d)}, got {x.shape}")
        return [x[i * self.f:(i + 1) * self.f] for i in range(n)]

    # -- the method
    def append(self, k_raw: np.ndarray, v: np.ndarray) -> None:
        """Write back the clean chunk: abs stores rotated keys (id = own frame), rel stores k_raw."""
        n = np.asarray(k_raw).shape[0] // self.f
        kf = self.frames_of(k_raw, n)
        vf = self.frames_of(v, n)
        if self.mode == "abs":
            f0 = self.n_appended
            kf = [self._rope(kk, [f0 + i]) for i, kk in enumerate(kf)]
        self.cache.append(kf, vf)

    def keys_values(self, k_raw_cur: np.ndarray, v_cur: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
        """Rotated visible keys and values [n_vis*F, H, D] for the current chunk."""
        hist = self.visible()
        if self.mode == "abs":
            s0 = self.n_appended
            k_hist = [e[1] for e in hist]
            k_cur = self._rope(k_raw_cur, range(s0, s0 + self.c))
        else:
            nv = len(hist) + self.c
            k_hist = [self._rope(e[1], self._clamp([j])) for j, e in enumerate(hist)]
            k_cur = self._rope(k_raw_cur, self._clamp(range(nv - self.c, nv)))
        k_all = np.concatenate(k_hist + [k_cur], axis=0)
        v_all = np.concatenate([e[2] for e in hist] + [np.asarray(v_cur, np.float64)], axis=0)
        return k_all, v_all

    def chunk_attention(self, q_raw: np.ndarray, k_raw_cur: np.ndarray, v_cur: np.ndarray,
                        rows: Optional[np.ndarray] = None) -> np.ndarray:
        """Output of one pass for the current chunk: softmax(q~ K~^T / sqrt(D)) V over the visible set."""
        self.frames_of(q_raw, self.c)
        self.frames_of(k_raw_cur, self.c)
        self.frames_of(v_cur, self.c)
        q = self._rope(q_raw, self.query_time_ids())
        k_all, v_all = self.keys_values(k_raw_cur, v_cur)
        return attention(q, k_all, v_all, rows=rows)

    def gather(self) -> Tuple[np.ndarray, np.ndarray, List[int]]:
        """Logical cache contents (oldest first) and their frame ids."""
        ent = self.cache.entries
        if not ent:
            z = np.zeros((0, self.h, self.d))
            return z, z.copy(), []
        k = np.concatenate([e[1] for e in ent], axis=0)
        v = np.concatenate([e[2] for e in ent], axis=0)
        return k, v, [e[0] for e in ent]
