"""Python binding of ``libskv.so`` (C ABI in ``include/skv.h``): argument marshalling only.

Every step of the hot path runs in the library's HIP kernels.  torch is used for
device memory (the stores, the workspace, inputs and outputs) and for the
current HIP stream.  Importing this package fails loudly when the library has
not been built (``python streaming_kv_cache_amd/build.py``); there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libskv.so")

OK, ERR_NULL, ERR_CONFIG, ERR_SHAPE, ERR_ALIGN, ERR_STATE, ERR_HIP = range(7)
F32, BF16 = 0, 1
ROPE_ABS, ROPE_REL = 0, 1

EXPORTED = (
    "skv_abi_version", "skv_status_string", "kv_cache_bytes", "kv_cache_init", "kv_cache_reset",
    "kv_cache_destroy", "kv_cache_append_evict", "rope_apply", "rope_apply_window", "chunk_attention",
    "cross_attention", "kv_cache_info", "kv_cache_gather", "kv_cache_stage_v", "sampler_step",
    "chunk_attention_batch", "block_causal_workspace_bytes", "block_causal_attention",
    "text_cache_bytes", "text_cache_prepare", "cross_attention_cached", "rope_apply_qk", "kv_cache_prepare_pass",
    "kv_cache_restore", "skv_debug_fail_launches", "block_causal_attention_noalloc",
)


class SkvConfig(ctypes.Structure):
    _fields_ = [
        ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32),
        ("chunk_frames", ctypes.c_int32), ("sink_frames", ctypes.c_int32), ("window_frames", ctypes.c_int32),
        ("rope_t", ctypes.c_int32), ("rope_h", ctypes.c_int32), ("rope_w", ctypes.c_int32),
        ("rope_theta", ctypes.c_double),
        ("rope_mode", ctypes.c_int32), ("dtype", ctypes.c_int32), ("fused_rope", ctypes.c_int32),
    ]


class KvCacheInfo(ctypes.Structure):
    _fields_ = [
        ("n_appended", ctypes.c_int64), ("n_cached", ctypes.c_int32), ("n_sink_vis", ctypes.c_int32),
        ("n_ring_vis", ctypes.c_int32), ("n_vis", ctypes.c_int32), ("ring_start", ctypes.c_int32),
        ("window_ready", ctypes.c_int32), ("poisoned", ctypes.c_int32),
    ]


class SkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python streaming_kv_cache_amd/build.py`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int
    sig = {
        "skv_abi_version": ([], ctypes.c_int),
        "skv_status_string": ([st], ctypes.c_char_p),
        "kv_cache_bytes": ([ctypes.POINTER(SkvConfig), ctypes.POINTER(ctypes.c_size_t),
                            ctypes.POINTER(ctypes.c_size_t)], st),
        "kv_cache_init": ([ctypes.POINTER(SkvConfig), vp, vp, vp, ctypes.POINTER(vp)], st),
        "kv_cache_reset": ([vp], st),
        "kv_cache_destroy": ([vp], st),
        "kv_cache_append_evict": ([vp, vp, vp, i32, vp], st),
        "rope_apply": ([vp, vp, vp, i32, i64, vp], st),
        "rope_apply_qk": ([vp, vp, vp, vp, vp, i32, i64, vp], st),
        "kv_cache_prepare_pass": ([vp, vp, vp, vp, vp, vp, i32, i64, vp], st),
        "rope_apply_window": ([vp, vp], st),
        "chunk_attention": ([vp, vp, vp, vp, i32, vp, vp], st),
        "cross_attention": ([vp, i32, vp, vp, i32, i32, i32, i32, vp, vp], st),
        "kv_cache_info": ([vp, ctypes.POINTER(KvCacheInfo)], st),
        "kv_cache_gather": ([vp, vp, vp, ctypes.POINTER(ctypes.c_int64), vp], st),
        "kv_cache_restore": ([vp, vp, vp, ctypes.POINTER(ctypes.c_int64), i32, vp], st),
        "skv_debug_fail_launches": ([i32], None),
        "kv_cache_stage_v": ([vp, vp, i32, vp], st),
        "chunk_attention_batch": ([ctypes.POINTER(vp), i32, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                   i32, ctypes.POINTER(vp), vp], st),
        "block_causal_workspace_bytes": ([ctypes.POINTER(SkvConfig), i32, ctypes.POINTER(ctypes.c_size_t)], st),
        "block_causal_attention": ([ctypes.POINTER(SkvConfig), vp, vp, vp, i32, i32, vp, vp, vp], st),
        "block_causal_attention_noalloc": ([ctypes.POINTER(SkvConfig), vp, vp, vp, i32, i32, vp, vp], st),
        "sampler_step": ([vp, vp, vp, ctypes.c_double, vp, i64, ctypes.c_double, ctypes.c_double, i32, vp, vp, vp],
                         st),
        "text_cache_bytes": ([i32, i32, i32, i32, ctypes.POINTER(ctypes.c_size_t)], st),
        "text_cache_prepare": ([vp, vp, i32, i32, i32, i32, vp, vp], st),
        "cross_attention_cached": ([vp, i32, vp, i32, i32, i32, i32, vp, vp], st),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.skv_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != OK:
        raise SkvError(status, where)


def _stream(stream: Optional[torch.cuda.Stream] = None) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    raise ValueError(f"unsupported dtype {dt}")


@dataclass(frozen=True)
class Config:
    """Mirror of ``skv_config``.  Rotary split 0/0/0 and theta 0 select the defaults."""
    heads: int
    head_dim: int
    grid_h: int
    grid_w: int
    chunk_frames: int
    sink_frames: int
    window_frames: int
    rope_mode: int = ROPE_ABS
    dtype: int = BF16
    rope_split: tuple = (0, 0, 0)
    rope_theta: float = 0.0
    fused_rope: bool = False   # callers pass raw q/k; the library rotates (see skv.h)

    @property
    def tokens_per_frame(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPE[self.dtype]

    def c_struct(self) -> SkvConfig:
        t, h, w = self.rope_split
        return SkvConfig(self.heads, self.head_dim, self.grid_h, self.grid_w, self.chunk_frames,
                         self.sink_frames, self.window_frames, t, h, w, float(self.rope_theta),
                         int(self.rope_mode), int(self.dtype), int(bool(self.fused_rope)))


def cache_bytes(cfg: Config):
    """(bytes of one store, bytes of the REL workspace) for ``cfg``."""
    c = cfg.c_struct()
    s, w = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.kv_cache_bytes(ctypes.byref(c), ctypes.byref(s), ctypes.byref(w)), "kv_cache_bytes")
    return s.value, w.value


class KVCache:
    """One layer's streaming KV cache: device stores owned here (torch), bookkeeping in the library."""

    def __init__(self, cfg: Config, device="cuda"):
        self.cfg = cfg
        store, ws = cache_bytes(cfg)
        self.k_store = torch.empty(store, dtype=torch.uint8, device=device)
        self.v_store = torch.empty(store, dtype=torch.uint8, device=device)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=device) if ws else None
        h = ctypes.c_void_p()
        c = cfg.c_struct()
        _check(lib.kv_cache_init(ctypes.byref(c), _ptr(self.k_store), _ptr(self.v_store),
                                 _ptr(self.workspace), ctypes.byref(h)), "kv_cache_init")
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and lib is not None:   # lib is None during interpreter shutdown
            lib.kv_cache_destroy(h)
            self._h = None

    # -- argument checks (shape/dtype/device/contiguity); the library checks the rest
    def _tensor(self, x: torch.Tensor, n_frames: int, name: str) -> torch.Tensor:
        cfg = self.cfg
        want = (n_frames * cfg.tokens_per_frame, cfg.heads, cfg.head_dim)
        if tuple(x.shape) != want:
            raise ValueError(f"{name}: expected shape {want}, got {tuple(x.shape)}")
        if x.dtype != cfg.torch_dtype or not x.is_cuda or not x.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous {cfg.torch_dtype} CUDA tensor")
        return x

    def reset(self) -> None:
        _check(lib.kv_cache_reset(self._h), "kv_cache_reset")

    def info(self) -> KvCacheInfo:
        i = KvCacheInfo()
        _check(lib.kv_cache_info(self._h, ctypes.byref(i)), "kv_cache_info")
        return i

    def append_evict(self, k: torch.Tensor, v: torch.Tensor, stream=None) -> None:
        n = k.shape[0] // self.cfg.tokens_per_frame
        self._tensor(k, n, "k")
        self._tensor(v, n, "v")
        _check(lib.kv_cache_append_evict(self._h, _ptr(k), _ptr(v), n, _stream(stream)), "kv_cache_append_evict")

    def rope_apply(self, x: torch.Tensor, out: Optional[torch.Tensor] = None, start_frame: int = 0,
                   stream=None) -> torch.Tensor:
        n = x.shape[0] // self.cfg.tokens_per_frame
        self._tensor(x, n, "x")
        out = torch.empty_like(x) if out is None else self._tensor(out, n, "out")
        _check(lib.rope_apply(self._h, _ptr(x), _ptr(out), n, int(start_frame), _stream(stream)), "rope_apply")
        return out

    def rope_apply_qk(self, q: torch.Tensor, k: torch.Tensor, q_out: Optional[torch.Tensor] = None,
                      k_out: Optional[torch.Tensor] = None, start_frame: int = 0, stream=None):
        """q and k of one chunk rotated at the same time ids in one launch; returns (q_out, k_out)."""
        n = q.shape[0] // self.cfg.tokens_per_frame
        self._tensor(q, n, "q")
        self._tensor(k, n, "k")
        q_out = torch.empty_like(q) if q_out is None else self._tensor(q_out, n, "q_out")
        k_out = torch.empty_like(k) if k_out is None else self._tensor(k_out, n, "k_out")
        _check(lib.rope_apply_qk(self._h, _ptr(q), _ptr(q_out), _ptr(k), _ptr(k_out), n, int(start_frame),
                                 _stream(stream)), "rope_apply_qk")
        return q_out, k_out

    def prepare_pass(self, q: torch.Tensor, k: torch.Tensor, v_cur: torch.Tensor,
                     q_out: Optional[torch.Tensor] = None, k_out: Optional[torch.Tensor] = None,
                     start_frame: int = 0, stream=None):
        """rope_apply_qk and stage_v in one call (one launch in bf16); returns (q_out, k_out)."""
        c = self.cfg.chunk_frames
        self._tensor(q, c, "q")
        self._tensor(k, c, "k")
        self._tensor(v_cur, c, "v_cur")
        q_out = torch.empty_like(q) if q_out is None else self._tensor(q_out, c, "q_out")
        k_out = torch.empty_like(k) if k_out is None else self._tensor(k_out, c, "k_out")
        _check(lib.kv_cache_prepare_pass(self._h, _ptr(q), _ptr(q_out), _ptr(k), _ptr(k_out), _ptr(v_cur), c,
                                         int(start_frame), _stream(stream)), "kv_cache_prepare_pass")
        return q_out, k_out

    def rope_apply_window(self, stream=None) -> None:
        _check(lib.rope_apply_window(self._h, _stream(stream)), "rope_apply_window")

    def stage_v(self, v_cur: torch.Tensor, stream=None) -> None:
        c = self.cfg.chunk_frames
        self._tensor(v_cur, c, "v_cur")
        _check(lib.kv_cache_stage_v(self._h, _ptr(v_cur), c, _stream(stream)), "kv_cache_stage_v")

    def chunk_attention(self, q: torch.Tensor, k_cur: torch.Tensor, v_cur: Optional[torch.Tensor],
                        out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """v_cur=None uses the values staged by stage_v."""
        c = self.cfg.chunk_frames
        self._tensor(q, c, "q")
        self._tensor(k_cur, c, "k_cur")
        if v_cur is not None:
            self._tensor(v_cur, c, "v_cur")
        out = torch.empty_like(q) if out is None else self._tensor(out, c, "out")
        _check(lib.chunk_attention(self._h, _ptr(q), _ptr(k_cur), _ptr(v_cur), c, _ptr(out), _stream(stream)),
               "chunk_attention")
        return out

    def gather(self, stream=None):
        """Logical cache contents (oldest first) and frame ids: (k, v, ids)."""
        n = self.info().n_cached
        cfg = self.cfg
        shape = (n * cfg.tokens_per_frame, cfg.heads, cfg.head_dim)
        k = torch.empty(shape, dtype=cfg.torch_dtype, device=self.k_store.device)
        v = torch.empty_like(k)
        ids = (ctypes.c_int64 * max(n, 1))()
        if n:
            _check(lib.kv_cache_gather(self._h, _ptr(k), _ptr(v), ids, _stream(stream)), "kv_cache_gather")
        return k, v, [int(ids[i]) for i in range(n)]

    def restore(self, k: torch.Tensor, v: torch.Tensor, frame_ids, stream=None) -> None:
        """Put back a snapshot from gather(): afterwards the cache holds exactly what it held then."""
        n = len(frame_ids)
        ids = (ctypes.c_int64 * max(n, 1))(*[int(i) for i in frame_ids])
        if n:
            self._tensor(k, n, "k")
            self._tensor(v, n, "v")
        _check(lib.kv_cache_restore(self._h, _ptr(k if n else None), _ptr(v if n else None), ids, n,
                                    _stream(stream)), "kv_cache_restore")


def debug_fail_launches(n: int) -> None:
    """Test hook: the next n launches of the library report a HIP failure without launching."""
    lib.skv_debug_fail_launches(int(n))


def chunk_attention_batch(caches, qs, ks, vs, outs=None, stream=None):
    """chunk_attention for several caches of one configuration in one launch (e.g. the two caches of
    classifier-free guidance).  ``vs`` may be None or hold None entries (use the staged values)."""
    n = len(caches)
    if not (len(qs) == len(ks) == n and (vs is None or len(vs) == n)):
        raise ValueError("one q, k_cur (and v_cur) per cache")
    c = caches[0].cfg.chunk_frames
    for i, cache in enumerate(caches):
        cache._tensor(qs[i], c, "q")
        cache._tensor(ks[i], c, "k_cur")
        if vs is not None and vs[i] is not None:
            cache._tensor(vs[i], c, "v_cur")
    outs = [torch.empty_like(q) for q in qs] if outs is None else list(outs)
    arr = lambda ptrs: (ctypes.c_void_p * n)(*[p.value for p in ptrs])  # noqa: E731
    vp = None if vs is None else arr([_ptr(v) for v in vs])
    _check(lib.chunk_attention_batch(arr([cache._h for cache in caches]), n, arr([_ptr(q) for q in qs]),
                                     arr([_ptr(k) for k in ks]), vp, c, arr([_ptr(o) for o in outs]),
                                     _stream(stream)), "chunk_attention_batch")
    return outs


def block_causal_workspace_bytes(cfg: Config, n_frames: int) -> int:
    c = cfg.c_struct()
    b = ctypes.c_size_t()
    _check(lib.block_causal_workspace_bytes(ctypes.byref(c), int(n_frames), ctypes.byref(b)),
           "block_causal_workspace_bytes")
    return b.value


def block_causal_attention(cfg: Config, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_frame0: int = 0,
                           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """Many chunks at once under the sink + window block-causal mask (see skv.h).  k, v: all frames;
    q: frames q_frame0.. ; everything already rotated."""
    f = cfg.tokens_per_frame
    n = k.shape[0] // f
    for name, t, rows in (("k", k, n * f), ("v", v, n * f), ("q", q, (n - q_frame0) * f)):
        if tuple(t.shape) != (rows, cfg.heads, cfg.head_dim) or t.dtype != cfg.torch_dtype or not t.is_cuda \
                or not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous {cfg.torch_dtype} CUDA tensor of shape "
                             f"{(rows, cfg.heads, cfg.head_dim)}")
    if workspace is None:
        workspace = torch.empty(block_causal_workspace_bytes(cfg, n), dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q) if out is None else out
    c = cfg.c_struct()
    _check(lib.block_causal_attention(ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), n, int(q_frame0), _ptr(workspace),
                                      _ptr(out), _stream(stream)), "block_causal_attention")
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20


def block_causal_attention_noalloc(cfg: Config, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                                   q_frame0: int = 0, stream=None) -> torch.Tensor:
    """block_causal_attention with the workspace in the library's static device array (the call allocates
    nothing; ``out`` is the caller's).  At most NOALLOC_SCRATCH_BYTES of workspace (see skv.h)."""
    f = cfg.tokens_per_frame
    n = k.shape[0] // f
    for name, t, rows in (("k", k, n * f), ("v", v, n * f), ("q", q, (n - q_frame0) * f), ("out", out, (n - q_frame0) * f)):
        if tuple(t.shape) != (rows, cfg.heads, cfg.head_dim) or t.dtype != cfg.torch_dtype or not t.is_cuda \
                or not t.is_contiguous():
            raise ValueError(f"{name}: expected a contiguous {cfg.torch_dtype} CUDA tensor of shape "
                             f"{(rows, cfg.heads, cfg.head_dim)}")
    c = cfg.c_struct()
    _check(lib.block_causal_attention_noalloc(ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), n, int(q_frame0), _ptr(out),
                                              _stream(stream)), "block_causal_attention_noalloc")
    return out


def cross_attention(q: torch.Tensor, k_text: torch.Tensor, v_text: torch.Tensor,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """softmax(q K_text^T / sqrt(D)) V_text per head; tensors [tokens, H, D] on the GPU."""
    if q.dim() != 3 or k_text.dim() != 3 or k_text.shape != v_text.shape or q.shape[1:] != k_text.shape[1:]:
        raise ValueError("q [n_q, H, D] and k_text/v_text [n_text, H, D] expected")
    for t in (q, k_text, v_text):
        if t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError("contiguous CUDA tensors of one dtype expected")
    out = torch.empty_like(q) if out is None else out
    _check(lib.cross_attention(_ptr(q), q.shape[0], _ptr(k_text), _ptr(v_text), k_text.shape[0], q.shape[1],
                               q.shape[2], _dtype_code(q.dtype), _ptr(out), _stream(stream)), "cross_attention")
    return out


def text_cache_bytes(n_text: int, heads: int, head_dim: int, dtype: int) -> int:
    b = ctypes.c_size_t()
    _check(lib.text_cache_bytes(int(n_text), int(heads), int(head_dim), int(dtype), ctypes.byref(b)),
           "text_cache_bytes")
    return b.value


def text_cache_prepare(k_text: torch.Tensor, v_text: torch.Tensor, store: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """Lay the text K/V out once for cross_attention_cached (see skv.h); returns the store (uint8)."""
    if k_text.dim() != 3 or k_text.shape != v_text.shape:
        raise ValueError("k_text/v_text [n_text, H, D] expected")
    for t in (k_text, v_text):
        if t.dtype != k_text.dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError("contiguous CUDA tensors of one dtype expected")
    n, h, d = k_text.shape
    dt = _dtype_code(k_text.dtype)
    if store is None:
        store = torch.empty(text_cache_bytes(n, h, d, dt), dtype=torch.uint8, device=k_text.device)
    _check(lib.text_cache_prepare(_ptr(k_text), _ptr(v_text), n, h, d, dt, _ptr(store), _stream(stream)),
           "text_cache_prepare")
    return store


def cross_attention_cached(q: torch.Tensor, store: torch.Tensor, n_text: int, out: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """cross_attention over a store laid out by text_cache_prepare; q [n_q, H, D] on the GPU."""
    if q.dim() != 3 or not q.is_cuda or not q.is_contiguous() or not store.is_cuda:
        raise ValueError("contiguous CUDA q [n_q, H, D] and a CUDA store expected")
    out = torch.empty_like(q) if out is None else out
    _check(lib.cross_attention_cached(_ptr(q), q.shape[0], _ptr(store), int(n_text), q.shape[1], q.shape[2],
                                      _dtype_code(q.dtype), _ptr(out), _stream(stream)), "cross_attention_cached")
    return out


class TextCache:
    """Text K/V of one prompt, laid out once (text_cache_prepare) and attended by every chunk and pass."""

    def __init__(self, k_text: torch.Tensor, v_text: torch.Tensor, stream=None):
        self.n_text, self.heads, self.head_dim = k_text.shape
        self.dtype = k_text.dtype
        self.store = text_cache_prepare(k_text, v_text, stream=stream)

    def attend(self, q: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        if q.dtype != self.dtype or tuple(q.shape[1:]) != (self.heads, self.head_dim):
            raise ValueError(f"q: expected [n_q, {self.heads}, {self.head_dim}] of {self.dtype}")
        return cross_attention_cached(q, self.store, self.n_text, out=out, stream=stream)


def sampler_step(x_t: torch.Tensor, v_cond: torch.Tensor, sigma: float, sigma_next: float = 0.0,
                 noise: Optional[torch.Tensor] = None, v_uncond: Optional[torch.Tensor] = None,
                 cfg_scale: float = 1.0, x0_out: Optional[torch.Tensor] = None,
                 x_next_out: Optional[torch.Tensor] = None, want_x0: bool = True, stream=None):
    """One sampler step (see ``sampler_step`` in skv.h).  Returns (x0, x_next); x_next is None without noise."""
    ts = [t for t in (x_t, v_cond, v_uncond, noise, x0_out, x_next_out) if t is not None]
    for t in ts:
        if t.dtype != x_t.dtype or t.numel() != x_t.numel() or not t.is_cuda or not t.is_contiguous():
            raise ValueError("contiguous CUDA tensors of one dtype and size expected")
    if want_x0 and x0_out is None:
        x0_out = torch.empty_like(x_t)
    if noise is not None and x_next_out is None:
        x_next_out = torch.empty_like(x_t)
    _check(lib.sampler_step(_ptr(x_t), _ptr(v_cond), _ptr(v_uncond), float(cfg_scale), _ptr(noise), x_t.numel(),
                            float(sigma), float(sigma_next), _dtype_code(x_t.dtype), _ptr(x0_out),
                            _ptr(x_next_out), _stream(stream)), "sampler_step")
    return x0_out, x_next_out
