"""GPU parity of block_causal_attention (many chunks under the sink + window mask) with the oracle.

Keys are rotated at their absolute frame ids and queries at theirs (rope_apply of an
absolute-RoPE handle of the same configuration), so the masked attention over the whole
sequence is what streaming the chunks through a cache computes (the oracle's pin).  Small
shapes cover: frames whose token count is not a multiple of 8 (unaligned V^T ranges), a
context prefix before the first query frame, no sinks, query chunks inside the sink range,
both kernel shapes; a 480P-sized sequence and an ABot 720P-sized one (5 context frames, then 22
chunks of 3) are checked on sampled rows.
"""
import numpy as np
import pytest
import torch

import seeded_inputs as si
import streaming_kv_cache_amd as skv
from oracle import skv_oracle as so
from tests import rollout as ro

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


CASES = {
    # name: (H, D, gh, gw, c, S, W, n_frames, q_frame0)
    "odd_frame": (3, 128, 7, 9, 2, 2, 7, 14, 0),
    "aligned": (2, 128, 4, 8, 2, 2, 7, 16, 0),
    "prefix": (2, 128, 5, 8, 3, 2, 9, 17, 2),
    "no_sink": (2, 128, 4, 9, 2, 0, 5, 12, 0),
    "chunk_in_sinks": (2, 128, 3, 8, 2, 3, 7, 14, 0),
    "d64": (2, 64, 6, 11, 2, 1, 6, 12, 0),
}


def _run(name, h, d, gh, gw, c, s, w, n, q0, rows=None, base=0):
    cfg = skv.Config(h, d, gh, gw, c, s, w, skv.ROPE_ABS, skv.BF16)
    f = gh * gw
    k = si.draw((n * f, h, d), base, 0, 0, si.K, torch.bfloat16)
    v = si.draw((n * f, h, d), base, 0, 0, si.V, torch.bfloat16)
    q = si.draw(((n - q0) * f, h, d), base, 0, 0, si.Q, torch.bfloat16)
    cache = skv.KVCache(cfg)       # only for rope_apply at absolute ids
    kr = cache.rope_apply(k.cuda(), start_frame=0)
    qr = cache.rope_apply(q.cuda(), start_frame=q0)
    out = skv.block_causal_attention(cfg, qr, kr, v.cuda(), q_frame0=q0)
    torch.cuda.synchronize()
    kx = so.rope_3d(ro.f64(k), range(n), gh, gw)
    qx = so.rope_3d(ro.f64(q), range(q0, n), gh, gw)
    ref = so.block_causal_attention(qx, kx, ro.f64(v), f, c, s, w, q_frame0=q0, rows=rows)
    got = out if rows is None else out[torch.as_tensor(rows, device=out.device)]
    return got, ref


@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_block_causal_small(name, waves, monkeypatch):
    monkeypatch.setenv("SKV_ATTN_WAVES", waves)
    say(f"[block-causal] {name} waves={waves} {CASES[name]}")
    got, ref = _run(name, *CASES[name])
    ro.assert_close(got, ref, skv.BF16, f"{name} waves {waves}")


@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("name", ["odd_frame", "no_sink", "d64"])
def test_block_causal_hot_key(name, waves, monkeypatch):
    """One key of frame 3 scores ~200 (log2 units) against every other query row: rows that see it
    raise their running max past the first tile (with sinks) or follow it (without), and their
    output concentrates on its value; all rows stay within the oracle's tolerance.  The key and the
    queries use only the lowest-frequency time pair, so the rotation keeps their dot product."""
    monkeypatch.setenv("SKV_ATTN_WAVES", waves)
    h, d, gh, gw, c, s_, w, n, q0 = CASES[name]
    say(f"[block-causal hot key] {name} waves={waves}")
    cfg = skv.Config(h, d, gh, gw, c, s_, w, skv.ROPE_ABS, skv.BF16)
    f = gh * gw
    hot_dim = so.rope_split(d)[0] - 2
    k = si.draw((n * f, h, d), 0, 0, 0, si.K, torch.bfloat16).clone()
    v = si.draw((n * f, h, d), 0, 0, 0, si.V, torch.bfloat16).clone()
    q = si.draw(((n - q0) * f, h, d), 0, 0, 0, si.Q, torch.bfloat16).clone()
    hot_tok = 3 * f + f // 2
    k[hot_tok] = 0
    k[hot_tok, :, hot_dim] = 40.0
    v[hot_tok] = 0.5
    hot = torch.arange((n - q0) * f) % 2 == 0
    q[hot] = 0
    q[hot, :, hot_dim] = 40.0
    cache = skv.KVCache(cfg)
    kr = cache.rope_apply(k.cuda(), start_frame=0)
    qr = cache.rope_apply(q.cuda(), start_frame=q0)
    out = skv.block_causal_attention(cfg, qr, kr, v.cuda(), q_frame0=q0)
    torch.cuda.synchronize()
    kx = so.rope_3d(ro.f64(k), range(n), gh, gw)
    qx = so.rope_3d(ro.f64(q), range(q0, n), gh, gw)
    ref = so.block_causal_attention(qx, kx, ro.f64(v), f, c, s_, w, q_frame0=q0)
    # rows of the query frames that see frame 3 concentrate on the planted value
    vis = so.block_causal_visible(n, q0, c, s_, w)[:, 3].astype(bool)          # per query frame
    sees = np.repeat(vis, f) & hot.numpy()
    assert sees.any()
    assert np.abs(ref[sees] - 0.5).max() < 1e-6
    ro.assert_close(out, ref, skv.BF16, f"{name} waves {waves}")
    g = out.float().cpu().double().numpy()
    assert np.abs(g[sees] - 0.5).max() <= 2.0 ** -8


def test_block_causal_probe_visibility():
    """q = 0 and one-hot values (frame j -> channel j): each output is 1/|visible| on exactly the
    visible frames, which a wrong frame would move by at least 1/W."""
    h, d, gh, gw, c, s, w, n, q0 = 1, 128, 4, 8, 2, 2, 7, 20, 0
    cfg = skv.Config(h, d, gh, gw, c, s, w, skv.ROPE_ABS, skv.BF16)
    f = gh * gw
    k = si.draw((n * f, h, d), 3, 0, 0, si.K, torch.bfloat16).cuda()
    v = torch.zeros(n * f, h, d)
    for j in range(n):
        v[j * f:(j + 1) * f, :, j] = 1.0
    q = torch.zeros((n - q0) * f, h, d, dtype=torch.bfloat16, device="cuda")
    out = skv.block_causal_attention(cfg, q, k, v.to(torch.bfloat16).cuda(), q_frame0=q0)
    torch.cuda.synchronize()
    vis = so.block_causal_visible(n, q0, c, s, w)
    expect = vis / vis.sum(axis=1, keepdims=True)                     # [query frames, frames]
    g = out.float().cpu().numpy()[:, 0, :n].reshape(n - q0, f, n)
    assert np.abs(g - expect[:, None, :]).max() <= 2.0 ** -8 * expect.max() + 1e-6


def test_block_causal_480p_sampled():
    """A LingBot 480P training-length sequence (22 chunks of 4 frames, 40 heads): sampled rows
    from the first chunk, the chunk where the window starts sliding, and the last chunk."""
    h, d, gh, gw, c, s, w = 40, 128, 30, 52, 4, 6, 18
    n = 88
    f = gh * gw
    rows = np.concatenate([np.arange(0, 4 * f, 997), np.arange(12 * f, 16 * f, 1499),
                           np.arange((n - 4) * f, n * f, 577)])
    say(f"[block-causal] 480P n_frames={n} rows={len(rows)}")
    got, ref = _run("lb480", h, d, gh, gw, c, s, w, n, 0, rows=rows)
    ro.assert_close(got, ref, skv.BF16, "480P sampled rows")


def test_block_causal_abot720_sampled():
    """The ABot 720P shape the bench's many-chunk leg times: 24 heads, 5 context frames (the sinks)
    then 22 chunks of 3 frames, window 21: sampled rows from the first chunk, the chunk where the
    window starts sliding and the last chunk."""
    h, d, gh, gw, c, s, w = 24, 128, 22, 40, 3, 5, 21
    q0, n = 5, 5 + 22 * 3
    f = gh * gw
    rows = np.concatenate([np.arange(0, 3 * f, 97), np.arange(15 * f, 18 * f, 151),
                           np.arange((n - q0 - 3) * f, (n - q0) * f, 89)])
    say(f"[block-causal] ABot 720P n_frames={n} q_frame0={q0} rows={len(rows)}")
    got, ref = _run("abot720", h, d, gh, gw, c, s, w, n, q0, rows=rows)
    ro.assert_close(got, ref, skv.BF16, "ABot 720P sampled rows")
