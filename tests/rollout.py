"""Drivers shared by the GPU tests: the same seeded inputs through the HIP path and the oracle.

The per-chunk schedule follows the pages ([LB-fast] "3. KV 缓存 滚动窗口",
[ABot-stream] 机制二): 4 denoise passes with the cache read only, then the clean
write-back pass, whose keys/values are appended (rotated keys in ABS mode,
raw keys in REL mode).  The oracle receives the exact fp64 upcast of the same
bf16/fp32 inputs and never sees a value produced by the GPU.
"""
from __future__ import annotations

import numpy as np
import torch

import seeded_inputs as si
import streaming_kv_cache_amd as skv
from oracle import skv_oracle as so

WRITE_BACK = 4


def oracle_for(wl):
    c = wl.cfg
    return so.StreamingOracle(c.heads, c.head_dim, c.grid_h, c.grid_w, c.chunk_frames, c.sink_frames,
                              c.window_frames, rope_mode="rel" if c.rope_mode == skv.ROPE_REL else "abs",
                              split=None if tuple(c.rope_split) == (0, 0, 0) else tuple(c.rope_split))


def draw(wl, n_frames, chunk, pass_idx, tensor_id, base=0):
    c = wl.cfg
    shape = (n_frames * c.tokens_per_frame, c.heads, c.head_dim)
    return si.draw(shape, base, chunk, pass_idx, tensor_id, c.torch_dtype)


def f64(x):
    return si.to_f64(x)


def fused(wl):
    """The same workload with the library rotating q / k (callers pass raw tensors everywhere)."""
    import dataclasses
    return dataclasses.replace(wl, cfg=dataclasses.replace(wl.cfg, fused_rope=True))


def gpu_pass(cache, q, k, v):
    """rope(q), rope(k) at the chunk's ids, then chunk attention; returns (out, k to append, v).
    With fused rotation the raw tensors go in as they are.  Chunks alternate between two call
    sequences so that both meet the oracle: rope_apply twice then chunk_attention with v, and
    kv_cache_prepare_pass (one launch) then chunk_attention over the staged values."""
    t = cache.info().n_appended
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    if cache.cfg.fused_rope:
        return cache.chunk_attention(qd, kd, vd), kd, vd
    if (t // cache.cfg.chunk_frames) % 2 == 1:
        qr, kr = cache.prepare_pass(qd, kd, vd, start_frame=t)
        out = cache.chunk_attention(qr, kr, None)
    else:
        qr = cache.rope_apply(qd, start_frame=t)
        kr = cache.rope_apply(kd, start_frame=t)
        out = cache.chunk_attention(qr, kr, vd)
    k_store = kr if cache.cfg.rope_mode == skv.ROPE_ABS else kd
    return out, k_store, vd


def prefill(wl, cache, orc, base=0):
    if not wl.prefill:
        return
    sk = draw(wl, wl.prefill, 0, 0, si.SINK_K, base)
    sv = draw(wl, wl.prefill, 0, 0, si.SINK_V, base)
    if cache.cfg.rope_mode == skv.ROPE_ABS and not cache.cfg.fused_rope:
        kd = cache.rope_apply(sk.cuda(), start_frame=cache.info().n_appended)
    else:
        kd = sk.cuda()
    cache.append_evict(kd, sv.cuda())
    if orc is not None:
        orc.append(f64(sk), f64(sv))


def rollout(wl, n_chunks, passes=(0, 1, 2, 3, WRITE_BACK), base=0, with_oracle=True, rows=None,
            oracle_chunks=None):
    """Yield (chunk, pass, gpu_out, oracle_out or None) for every pass of every chunk."""
    cache = skv.KVCache(wl.cfg)
    orc = oracle_for(wl) if with_oracle else None
    prefill(wl, cache, orc, base)
    for ch in range(n_chunks):
        if wl.cfg.rope_mode == skv.ROPE_REL and not wl.cfg.fused_rope:
            cache.rope_apply_window()
        for p in passes:
            q = draw(wl, wl.cfg.chunk_frames, ch, p, si.Q, base)
            k = draw(wl, wl.cfg.chunk_frames, ch, p, si.K, base)
            v = draw(wl, wl.cfg.chunk_frames, ch, p, si.V, base)
            out, k_app, v_app = gpu_pass(cache, q, k, v)
            ref = None
            if orc is not None and (oracle_chunks is None or ch in oracle_chunks):
                ref = orc.chunk_attention(f64(q), f64(k), f64(v), rows=rows)
            yield ch, p, out, ref
            if p == WRITE_BACK:
                cache.append_evict(k_app, v_app)
                if orc is not None:
                    orc.append(f64(k), f64(v))


def errors(got: torch.Tensor, ref: np.ndarray):
    g = got.detach().float().cpu().double().numpy()
    e = np.abs(g - ref)
    rel_rms = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300))
    return float(e.max()), float(e.mean()), rel_rms


def assert_close(got, ref, dtype, what=""):
    """bf16: max-abs 2e-2, mean-abs 2e-3 and relative RMS 1e-2; fp32: max-abs 1e-5."""
    mx, mean, rr = errors(got, ref)
    if dtype == skv.F32:
        assert mx <= 1e-5, f"{what}: max-abs {mx:.3g} > 1e-5"
    else:
        assert mx <= 2e-2 and mean <= 2e-3 and rr <= 1e-2, \
            f"{what}: max-abs {mx:.3g} (2e-2), mean-abs {mean:.3g} (2e-3), rel-rms {rr:.3g} (1e-2)"
    return mx, mean, rr
