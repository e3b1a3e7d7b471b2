"""Pins of the CPU oracle: each check raises AssertionError when the oracle is wrong.

The checks compare the oracle with things other than itself: closed forms, brute
force over a whole sequence, a library routine (torch's scaled dot-product
attention, numpy complex arithmetic), special cases with exact answers, and the
configuration figures the pages print (``tests/golden/page_figures.json``).
They are functions so that ``test_oracle_mutations.py`` can plant mistakes in the
oracle and confirm that some check fails.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import skv_oracle as so

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_figures.json")


def _rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ RoPE pins
def check_rope_identity_at_origin():
    """All three positions zero (1x1 grid, time id 0): the rotation is the identity."""
    x = _rng(1).standard_normal((1, 3, 64))
    y = so.rope_3d(x, [0], 1, 1)
    assert np.array_equal(x, y)


def check_rope_norm_preserved():
    """Each rotated pair keeps its Euclidean norm."""
    x = _rng(2).standard_normal((2 * 12, 2, 128))
    y = so.rope_3d(x, [7, 1033], 3, 4)
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.allclose(n0, n1, rtol=1e-12, atol=1e-12)


def check_rope_complex():
    """Each pair equals complex multiplication by exp(i * position * omega) (numpy complex)."""
    gh, gw, d = 3, 5, 64
    x = _rng(3).standard_normal((2 * gh * gw, 2, d))
    t_ids = [4, 9]
    y = so.rope_3d(x, t_ids, gh, gw)
    d_t, d_h, d_w = 24, 20, 20
    z = x[..., 0::2] + 1j * x[..., 1::2]          # [tok, H, D/2]
    tok = np.arange(2 * gh * gw)
    pos = {"t": np.repeat(t_ids, gh * gw), "h": (tok % (gh * gw)) // gw, "w": tok % gw}
    # textbook frequencies written out per axis: theta^(-2k/d_axis)
    freqs = []
    for name, d_a in (("t", d_t), ("h", d_h), ("w", d_w)):
        for kk in range(d_a // 2):
            freqs.append((name, 10000.0 ** (-(2.0 * kk) / d_a)))
    phase = np.stack([pos[name] * w for name, w in freqs], axis=1)     # [tok, D/2]
    zr = z * np.exp(1j * phase)[:, None, :]
    assert np.allclose(y[..., 0::2], zr.real, atol=1e-12)
    assert np.allclose(y[..., 1::2], zr.imag, atol=1e-12)


def check_rope_axes():
    """Unit probes: the first pair of each axis turns by exactly (t, row, col) radians."""
    gh, gw = 4, 6
    f = gh * gw
    x = np.zeros((f, 1, 64))
    x[:, 0, 0] = 1.0       # first time pair
    x[:, 0, 24] = 1.0      # first height pair
    x[:, 0, 44] = 1.0      # first width pair
    t = 3.0
    y = so.rope_3d(x, [t], gh, gw)
    for tok in range(f):
        r, c = divmod(tok, gw)
        assert abs(y[tok, 0, 0] - math.cos(t)) < 1e-15 and abs(y[tok, 0, 1] - math.sin(t)) < 1e-15
        assert abs(y[tok, 0, 24] - math.cos(r)) < 1e-15 and abs(y[tok, 0, 25] - math.sin(r)) < 1e-15
        assert abs(y[tok, 0, 44] - math.cos(c)) < 1e-15 and abs(y[tok, 0, 45] - math.sin(c)) < 1e-15
    # last pair of the time axis: omega = theta^(-(d_t-2)/d_t)
    x2 = np.zeros((1, 1, 64))
    x2[0, 0, 22] = 1.0
    y2 = so.rope_3d(x2, [100.0], 1, 1)
    a = 100.0 * 10000.0 ** (-22.0 / 24.0)
    assert abs(y2[0, 0, 22] - math.cos(a)) < 1e-13 and abs(y2[0, 0, 23] - math.sin(a)) < 1e-13


def check_rope_relative_shift():
    """RoFormer's relative property: shifting every time id by delta keeps all scores."""
    gh, gw = 2, 3
    rng = _rng(4)
    q = rng.standard_normal((2 * 6, 2, 128))
    k = rng.standard_normal((3 * 6, 2, 128))
    for delta in (1, 17, 1000):
        s0 = np.einsum("qhd,khd->hqk", so.rope_3d(q, [5, 6], gh, gw), so.rope_3d(k, [0, 2, 6], gh, gw))
        s1 = np.einsum("qhd,khd->hqk", so.rope_3d(q, [5 + delta, 6 + delta], gh, gw),
                       so.rope_3d(k, [delta, 2 + delta, 6 + delta], gh, gw))
        assert np.allclose(s0, s1, atol=1e-9)


def check_rope_split_figures():
    assert so.rope_split(64) == (24, 20, 20)
    assert so.rope_split(128) == (44, 42, 42)


# ------------------------------------------------------------------ cache pins
def _closed_form(hist, sink, window):
    t = len(hist)
    return hist[:min(sink, t)] + hist[max(sink, t - (window - sink)):t]


def check_cache_closed_form(seed=5):
    """After every append the list equals hist[0:S] ++ hist[-(W-S):] (brute-force history)."""
    rng = _rng(seed)
    for sink, window in ((0, 1), (1, 4), (2, 7), (6, 18), (5, 21), (0, 5), (3, 3)):
        cl = so.CacheList(sink, window)
        hist = []
        for _ in range(60):
            n = int(rng.integers(1, window - sink + 1)) if window > sink else 0
            if n == 0:
                break
            ks = [np.full((1,), float(len(hist) + i)) for i in range(n)]
            cl.append(ks, ks)
            hist.extend(range(len(hist), len(hist) + n))
            assert cl.frame_ids() == _closed_form(hist, sink, window), (sink, window)
            for fid, kf, vf in cl.entries:
                assert kf[0] == fid and vf[0] == fid


def check_cache_rejects_oversize():
    cl = so.CacheList(2, 6)
    try:
        cl.append([np.zeros(1)] * 5, [np.zeros(1)] * 5)
    except ValueError:
        return
    raise AssertionError("append of more than window - sink frames must be rejected")


def check_sink_identity():
    """Sink frames are the same bytes after 300 chunks of evictions."""
    rng = _rng(6)
    cl = so.CacheList(6, 18)
    sink_frames = None
    for ch in range(300):
        ks = [rng.standard_normal((4, 2)) for _ in range(4)]
        vs = [rng.standard_normal((4, 2)) for _ in range(4)]
        cl.append(ks, vs)
        if ch == 1:
            sink_frames = [(e[1].copy(), e[2].copy()) for e in cl.entries[:6]]
    assert len(cl.entries) == 18
    for (k0, v0), e in zip(sink_frames, cl.entries[:6]):
        assert k0.tobytes() == e[1].tobytes() and v0.tobytes() == e[2].tobytes()
    assert cl.frame_ids() == list(range(6)) + list(range(1200 - 12, 1200))


def check_visible_matches_append_then_slice(seed=7):
    """'attend, then append' equals 'evict + append the chunk, then take the window'."""
    rng = _rng(seed)
    for sink, chunk, window in ((1, 2, 4), (6, 4, 18), (5, 3, 21), (0, 2, 5), (2, 3, 5)):
        cl = so.CacheList(sink, window)
        for _ in range(25):
            vis = so.visible_history(cl.entries, chunk, sink, window)
            probe = so.CacheList(sink, window)
            probe.entries = list(cl.entries)
            probe.n_appended = cl.n_appended
            probe.append([np.zeros(1)] * chunk, [np.zeros(1)] * chunk)
            expect = probe.frame_ids()
            got = [e[0] for e in vis] + list(range(cl.n_appended, cl.n_appended + chunk))
            assert got == expect, (sink, chunk, window)
            n = int(rng.integers(1, window - sink + 1))
            cl.append([np.zeros(1)] * n, [np.zeros(1)] * n)


# ------------------------------------------------------------------ attention pins
def _one_shot_masked(q_all, k_all, v_all, visible_mask, scale):
    """Whole-sequence attention with an explicit [L, L] boolean mask (separate code path)."""
    lq, h, d = q_all.shape
    out = np.zeros_like(q_all)
    for hh in range(h):
        s = (q_all[:, hh] @ k_all[:, hh].T) * scale
        s = np.where(visible_mask, s, -np.inf)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, hh] = (w / w.sum(axis=1, keepdims=True)) @ v_all[:, hh]
    return out


def _stream(cfg, n_chunks, seed, prefill=0):
    """Run the streaming oracle; return per-chunk outputs plus all raw inputs."""
    h, d, gh, gw, c, s, w, mode = cfg
    f = gh * gw
    rng = _rng(seed)
    o = so.StreamingOracle(h, d, gh, gw, c, s, w, rope_mode=mode)
    raws = []
    if prefill:
        kp = rng.standard_normal((prefill * f, h, d))
        vp = rng.standard_normal((prefill * f, h, d))
        o.append(kp, vp)
        raws.append((None, kp, vp))
    outs = []
    for _ in range(n_chunks):
        q = rng.standard_normal((c * f, h, d))
        k = rng.standard_normal((c * f, h, d))
        v = rng.standard_normal((c * f, h, d))
        outs.append(o.chunk_attention(q, k, v))
        o.append(k, v)
        raws.append((q, k, v))
    return outs, raws, o


def _one_shot_abs(cfg, raws, sink, window):
    """Absolute-RoPE reference: rotate the whole sequence once, mask with the closed form."""
    h, d, gh, gw, c, s, w, mode = cfg
    f = gh * gw
    q_parts, chunk_start, k_parts, v_parts = [], [], [], []
    frame = 0
    for q, k, v in raws:
        if q is not None:
            q_parts.append(q)
            chunk_start.append(frame)
        k_parts.append(k)
        v_parts.append(v)
        frame += k.shape[0] // f
    k_all = np.concatenate(k_parts)
    v_all = np.concatenate(v_parts)
    n_frames = k_all.shape[0] // f
    k_rot = so.rope_3d(k_all, range(n_frames), gh, gw)
    q_rot = np.concatenate([so.rope_3d(qq, range(st, st + c), gh, gw) for qq, st in zip(q_parts, chunk_start)])
    key_frame = np.repeat(np.arange(n_frames), f)[None, :]
    # every query of the chunk starting at st sees keys of frames j < e = st + c ...
    e = np.concatenate([[st + c] * (c * f) for st in chunk_start])[:, None]
    # ... restricted to the sinks and the last (window - sink) frames before e
    mask = (key_frame < e) & ((key_frame < sink) | (key_frame >= e - (window - sink)))
    return _one_shot_masked(q_rot, k_rot, v_all, mask, 1.0 / math.sqrt(d))


def check_full_window_block_causal():
    """W >= total frames: streaming equals one whole-sequence block-causal masked softmax."""
    for cfg, n_chunks, prefill in (((2, 64, 2, 3, 2, 1, 64, "abs"), 6, 0),
                                   ((1, 32, 3, 2, 3, 2, 64, "abs"), 4, 2)):
        outs, raws, _ = _stream(cfg, n_chunks, seed=8, prefill=prefill)
        ref = _one_shot_abs(cfg, raws, cfg[5], cfg[6])
        got = np.concatenate(outs)
        assert np.allclose(got, ref, atol=1e-11), np.abs(got - ref).max()


def check_sink_window_mask():
    """General window (abs): streaming equals the closed-form sink+window block-causal mask."""
    for cfg, n_chunks, prefill in (((2, 64, 2, 2, 2, 1, 4, "abs"), 8, 0),
                                   ((2, 32, 2, 3, 3, 5, 11, "abs"), 7, 5),
                                   ((1, 64, 1, 3, 4, 6, 18, "abs"), 9, 0),
                                   ((1, 32, 2, 2, 2, 0, 3, "abs"), 6, 0),
                                   ((1, 32, 2, 2, 3, 2, 5, "abs"), 6, 0)):
        outs, raws, _ = _stream(cfg, n_chunks, seed=9, prefill=prefill)
        ref = _one_shot_abs(cfg, raws, cfg[5], cfg[6])
        got = np.concatenate(outs)
        assert np.allclose(got, ref, atol=1e-11), (cfg, np.abs(got - ref).max())


def check_block_causal_matches_streaming():
    """The many-chunk masked attention equals streaming the same sequence chunk by chunk (abs)."""
    for cfg, n_chunks, prefill in (((2, 64, 2, 2, 2, 1, 4, "abs"), 8, 0),
                                   ((2, 32, 2, 3, 3, 5, 11, "abs"), 7, 5),
                                   ((1, 64, 1, 3, 4, 6, 18, "abs"), 9, 0),
                                   ((1, 32, 2, 2, 2, 0, 3, "abs"), 6, 0)):
        h, d, gh, gw, c, s, w, _ = cfg
        f = gh * gw
        outs, raws, _ = _stream(cfg, n_chunks, seed=10, prefill=prefill)
        k_all = np.concatenate([r[1] for r in raws])
        v_all = np.concatenate([r[2] for r in raws])
        n = k_all.shape[0] // f
        k_rot = so.rope_3d(k_all, range(n), gh, gw)
        q_rot = np.concatenate([so.rope_3d(r[0], range(prefill + i * c, prefill + (i + 1) * c), gh, gw)
                                for i, r in enumerate(raws[1:] if prefill else raws)])
        got = so.block_causal_attention(q_rot, k_rot, v_all, f, c, s, w, q_frame0=prefill)
        assert np.allclose(got, np.concatenate(outs), atol=1e-11), (cfg, np.abs(got - np.concatenate(outs)).max())
        # a row subset gives the same rows
        rows = np.array([0, 5, got.shape[0] - 1])
        sub = so.block_causal_attention(q_rot, k_rot, v_all, f, c, s, w, q_frame0=prefill, rows=rows)
        assert np.allclose(sub, got[rows], atol=1e-13)


def check_block_causal_counts_and_full():
    """Each query frame sees min(e, W) frames (e = its chunk's end); one chunk with a large window is
    plain full attention (torch scaled_dot_product_attention, fp64, no mask)."""
    import torch
    for n, q0, c, s, w in ((20, 0, 4, 6, 18), (23, 5, 3, 5, 21), (9, 1, 2, 0, 5), (12, 0, 2, 3, 5)):
        vis = so.block_causal_visible(n, q0, c, s, w)
        for row, i in enumerate(range(q0, n)):
            e = q0 + c * ((i - q0) // c + 1)
            assert vis[row].sum() == min(e, w), (n, q0, c, s, w, i)
            assert vis[row, :s].all() or e < s        # sinks stay visible
            assert not vis[row, e:].any()             # nothing after the chunk's end
    r = _rng(11)
    f, h, d = 6, 2, 32
    q = r.standard_normal((3 * f, h, d))
    k = r.standard_normal((3 * f, h, d))
    v = r.standard_normal((3 * f, h, d))
    got = so.block_causal_attention(q, k, v, f, 3, 1, 8, q_frame0=0)
    tq, tk, tv = (torch.from_numpy(x).permute(1, 0, 2) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(1, 0, 2).numpy()
    assert np.allclose(got, ref, atol=1e-12)


def check_rel_equals_abs_cases():
    """rel == abs when nothing was evicted yet, and when there are no sinks (shift invariance)."""
    for s, w, n_chunks in ((1, 64, 5), (0, 5, 9), (0, 7, 8)):
        cfg_a = (2, 64, 2, 2, 2, s, w, "abs")
        cfg_r = (2, 64, 2, 2, 2, s, w, "rel")
        oa, _, _ = _stream(cfg_a, n_chunks, seed=10)
        orl, _, _ = _stream(cfg_r, n_chunks, seed=10)
        for a, r in zip(oa, orl):
            assert np.allclose(a, r, atol=1e-10)
    # with sinks and eviction the two readings must differ (ids are not a common shift)
    oa, _, _ = _stream((2, 64, 2, 2, 2, 1, 4, "abs"), 8, seed=10)
    orl, _, _ = _stream((2, 64, 2, 2, 2, 1, 4, "rel"), 8, seed=10)
    assert not np.allclose(oa[-1], orl[-1], atol=1e-6)


def check_rel_ids_bounded():
    """rel time ids stay inside [0, W-1] and span it exactly once the window is full."""
    o = so.StreamingOracle(1, 64, 1, 1, 3, 5, 21, rope_mode="rel")
    o.append(np.zeros((5, 1, 64)), np.zeros((5, 1, 64)))
    seen_max = 0
    for _ in range(40):
        ids = o.query_time_ids()
        assert min(ids) >= 0 and max(ids) <= 20
        seen_max = max(seen_max, max(ids))
        o.append(np.zeros((3, 1, 64)), np.zeros((3, 1, 64)))
    assert seen_max == 20
    assert o.n_vis() == 21


def check_probe_zero_query():
    """q = 0: every score is equal, so o = mean of the visible V rows (per head)."""
    h, d, gh, gw, c, s, w = 2, 64, 2, 2, 2, 1, 4
    f = gh * gw
    rng = _rng(11)
    o = so.StreamingOracle(h, d, gh, gw, c, s, w)
    hist_v = []
    for ch in range(7):
        k = rng.standard_normal((c * f, h, d))
        v = rng.standard_normal((c * f, h, d))
        out = o.chunk_attention(np.zeros((c * f, h, d)), k, v)
        t = len(hist_v)
        frames = list(range(t))
        e = t + c
        vis = [j for j in frames if (j < s or j >= e - (w - s))] + list(range(t, e))
        all_v = hist_v + [v[i * f:(i + 1) * f] for i in range(c)]
        mean = np.concatenate([all_v[j] for j in vis]).mean(axis=0)
        assert np.allclose(out, mean[None], atol=1e-13)
        o.append(k, v)
        hist_v.extend(v[i * f:(i + 1) * f] for i in range(c))


def check_probe_onehot():
    """V of frame f = one-hot(f): with q = 0, o = 1/n_vis on exactly the visible frames."""
    h, d, gh, gw, c, s, w = 1, 64, 2, 3, 3, 5, 11
    f = gh * gw
    o = so.StreamingOracle(h, d, gh, gw, c, s, w, rope_mode="rel")

    def onehot(frames):
        v = np.zeros((len(frames) * f, h, d))
        for i, fr in enumerate(frames):
            v[i * f:(i + 1) * f, :, fr % d] = 1.0
        return v

    rng = _rng(12)
    o.append(rng.standard_normal((s * f, h, d)), onehot(range(s)))
    for ch in range(12):
        t = o.n_appended
        fr = list(range(t, t + c))
        out = o.chunk_attention(np.zeros((c * f, h, d)), rng.standard_normal((c * f, h, d)), onehot(fr))
        e = t + c
        vis = [j for j in range(e) if j < s or j >= e - (w - s)]
        expect = np.zeros(d)
        expect[[j % d for j in vis]] = 1.0 / len(vis)
        assert np.allclose(out, expect[None, None], atol=1e-14), ch
        o.append(rng.standard_normal((c * f, h, d)), onehot(fr))


def check_sdpa():
    """Single-chunk and cross attention equal torch's scaled_dot_product_attention (CPU, fp64)."""
    import torch
    import torch.nn.functional as F
    rng = _rng(13)
    for lq, lk, h, d in ((32, 64, 2, 64), (50, 512, 3, 128), (7, 1, 1, 32)):
        q = rng.standard_normal((lq, h, d))
        k = rng.standard_normal((lk, h, d))
        v = rng.standard_normal((lk, h, d))
        ref = F.scaled_dot_product_attention(torch.from_numpy(q).permute(1, 0, 2),
                                             torch.from_numpy(k).permute(1, 0, 2),
                                             torch.from_numpy(v).permute(1, 0, 2)).permute(1, 0, 2).numpy()
        assert np.allclose(so.attention(q, k, v), ref, atol=1e-12)
        assert np.allclose(so.cross_attention(q, k, v), ref, atol=1e-12)
        rows = np.array([0, lq - 1])
        assert np.allclose(so.attention(q, k, v, rows=rows), ref[rows], atol=1e-12)


# ------------------------------------------------------------------ page figures
def check_page_figures():
    """The configuration arithmetic the pages print."""
    g = json.load(open(GOLDEN))
    val = {k: v["value"] for k, v in g.items() if not k.startswith("_")}
    # ABot: cache of 21 frames x 880 tokens, relative ids 0..20, five reference sinks, 3-frame blocks
    o = so.StreamingOracle(1, 8, 1, 1, val["abot_block_frames"], val["abot_ref_slots"],
                           val["abot_window_frames"], rope_mode="rel")
    o.append(np.zeros((5, 1, 8)), np.zeros((5, 1, 8)))
    for _ in range(10):
        o.append(np.zeros((3, 1, 8)), np.zeros((3, 1, 8)))
    assert len(o.cache.entries) * val["abot_tokens_per_frame"] == 21 * 880
    ids = o.query_time_ids()
    nv = o.n_vis()
    assert [0, nv - 1] == val["abot_rel_time_id_range"] and ids[-1] == 20
    assert o.cache.frame_ids()[:5] == list(range(5))
    # LingBot: 6 sink + 12 sliding = 18 frames, chunks of 4
    cl = so.CacheList(val["lingbot_sink_frames"], val["lingbot_window_frames"])
    for _ in range(30):
        cl.append([np.zeros(1)] * 4, [np.zeros(1)] * 4)
    ids = cl.frame_ids()
    assert len(ids) == val["lingbot_sink_frames"] + val["lingbot_sliding_frames"] == 18
    assert ids[:6] == list(range(6)) and ids[6:] == list(range(120 - 12, 120))
    # 361 pixel frames -> 91 latent frames (temporal stride 4, frame_num = 4n+1) -> 22 chunks of 4 -> 88
    latent = (val["lingbot_pixel_frames"] - 1) // 4 + 1
    assert latent == val["lingbot_latent_frames"]
    chunks = latent // val["lingbot_chunk_frames"]
    assert chunks == val["lingbot_chunks"] and chunks * 4 == val["lingbot_forwards"]


ALL_CHECKS = [
    check_rope_identity_at_origin, check_rope_norm_preserved, check_rope_complex, check_rope_axes,
    check_rope_relative_shift, check_rope_split_figures, check_cache_closed_form, check_cache_rejects_oversize,
    check_sink_identity, check_visible_matches_append_then_slice, check_full_window_block_causal,
    check_sink_window_mask, check_rel_equals_abs_cases, check_rel_ids_bounded, check_probe_zero_query,
    check_probe_onehot, check_sdpa, check_page_figures, check_block_causal_matches_streaming,
    check_block_causal_counts_and_full,
]
