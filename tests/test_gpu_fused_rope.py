"""GPU tests of the fused-rotation protocol (fused_rope = 1): callers pass raw q / k, the library
rotates them (q and the current keys before each pass, the written-back keys at their absolute
frame ids), and REL attends ring and current keys with queries at absolute ids, sinks with
queries at slot ids.  The oracle is the unchanged streaming oracle: the same REL / ABS results."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
import streaming_kv_cache_amd as skv
from streaming_kv_cache_amd.workloads import WORKLOADS
from tests import rollout as ro

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("name", ["tiny", "small_abs", "small_rel", "small_d64", "small_f32_rel", "small_nosink"])
def test_fused_rollout_parity(name, waves, monkeypatch):
    monkeypatch.setenv("SKV_ATTN_WAVES", waves)
    wl = ro.fused(WORKLOADS[name])
    say(f"[fused] {name} waves={waves} chunks={wl.n_chunks}")
    for ch, p, out, ref in ro.rollout(wl, wl.n_chunks):
        torch.cuda.synchronize()
        ro.assert_close(out, ref, wl.cfg.dtype, f"fused {name} chunk {ch} pass {p}")


@pytest.mark.parametrize("name", ["small_abs", "small_rel"])
def test_fused_store_holds_keys_at_absolute_ids(name):
    """The fused write-back stores exactly what rope_apply at the absolute ids gives (same kernel),
    so the fused cache's gather equals an absolute-mode cache fed rotated keys, bit for bit."""
    wl = WORKLOADS[name]
    f_cfg = ro.fused(wl).cfg
    a_cfg = skv.Config(f_cfg.heads, f_cfg.head_dim, f_cfg.grid_h, f_cfg.grid_w, f_cfg.chunk_frames,
                       f_cfg.sink_frames, f_cfg.window_frames, skv.ROPE_ABS, f_cfg.dtype)
    fc, ac = skv.KVCache(f_cfg), skv.KVCache(a_cfg)
    n = f_cfg.chunk_frames
    for ch in range(wl.n_chunks):
        k = ro.draw(wl, n, ch, ro.WRITE_BACK, si.K).cuda()
        v = ro.draw(wl, n, ch, ro.WRITE_BACK, si.V).cuda()
        t = ac.info().n_appended
        fc.append_evict(k, v)
        ac.append_evict(ac.rope_apply(k, start_frame=t), v)
    kf, vf, idf = fc.gather()
    ka, va, ida = ac.gather()
    torch.cuda.synchronize()
    assert idf == ida
    assert torch.equal(kf, ka) and torch.equal(vf, va)


def test_fused_abot720_sampled():
    """ABot 720P shapes (relative RoPE, 5 reference sinks, window 21) through the steady state,
    sampled query rows against the oracle."""
    wl = ro.fused(WORKLOADS["abot720"])
    rows = np.unique(np.linspace(0, wl.lq - 1, 48).astype(np.int64))
    last = wl.steady_chunk + 1
    say(f"[fused] abot720 to chunk {last}, {len(rows)} rows")
    checked = 0
    for ch, p, out, ref in ro.rollout(wl, last + 1, passes=(0, ro.WRITE_BACK), rows=rows,
                                      oracle_chunks={0, wl.steady_chunk, last}):
        if ref is None:
            continue
        torch.cuda.synchronize()
        got = out[torch.as_tensor(rows, device=out.device)]
        e = ro.assert_close(got, ref, wl.cfg.dtype, f"fused abot720 chunk {ch} pass {p}")
        say(f"  chunk {ch} pass {p}: max {e[0]:.3g} mean {e[1]:.3g} relrms {e[2]:.3g}")
        checked += 1
    assert checked == 6
