"""Snapshot and restore of a stream on the GPU: kv_cache_gather, then kv_cache_restore on another
handle (or on the same one after kv_cache_reset), gives back exactly the cache that was gathered:
the same bytes and frame ids, and bit-identical attention for the chunks that follow.

Resuming keeps the history ([ABot-stream] "一次流式生成的完整链路": a stream's KV caches live until
reset_stream; a prompt change keeps them).  Also checked: the plain re-append of the snapshot in
logical order after a reset holds the same bytes (frame ids renumbered from 0), and its next chunk
matches the oracle when the queries keep their absolute time ids.
"""
import sys

import pytest
import torch

import seeded_inputs as si
from tests import rollout as ro

skv = pytest.importorskip("streaming_kv_cache_amd")
from streaming_kv_cache_amd.workloads import WORKLOADS  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _chunk(wl, cache, ch, passes=(0, ro.WRITE_BACK)):
    """One chunk of the schedule on one handle: outputs of the passes, then the write-back append."""
    c = wl.cfg
    if c.rope_mode == skv.ROPE_REL and not c.fused_rope:
        cache.rope_apply_window()
    outs = []
    for p in passes:
        q, k, v = (ro.draw(wl, c.chunk_frames, ch, p, t) for t in (si.Q, si.K, si.V))
        out, k_app, v_app = ro.gpu_pass(cache, q, k, v)
        outs.append(out)
        if p == ro.WRITE_BACK:
            cache.append_evict(k_app, v_app)
    return outs


def _same_state(a, b):
    ia, ib = a.info(), b.info()
    fields = ("n_appended", "n_cached", "n_sink_vis", "n_ring_vis", "n_vis", "ring_start")
    return all(getattr(ia, f) == getattr(ib, f) for f in fields)


@pytest.mark.parametrize("name,fused", [("small_abs", False), ("small_rel", False), ("small_nosink", False),
                                        ("small_d64", False), ("small_f32_rel", False), ("small_rel", True),
                                        ("small_abs", True), ("abot720", False)])
def test_gather_restore_round_trip(name, fused):
    wl = ro.fused(WORKLOADS[name]) if fused else WORKLOADS[name]
    c = wl.cfg
    n0 = wl.steady_chunk + 3          # past the first wrap of the ring
    say(f"[snapshot] {name} fused={fused}: {n0} chunks, restore, 3 more chunks on both handles")
    a = skv.KVCache(c)
    ro.prefill(wl, a, None)
    for ch in range(n0):
        _chunk(wl, a, ch, passes=(ro.WRITE_BACK,))
    k, v, ids = a.gather()
    # a second handle, restored from the snapshot
    b = skv.KVCache(c)
    b.restore(k, v, ids)
    kb, vb, idb = b.gather()
    torch.cuda.synchronize()
    assert idb == ids and torch.equal(kb, k) and torch.equal(vb, v)
    assert _same_state(a, b)
    # the same handle, reset and restored
    a2 = skv.KVCache(c)
    ro.prefill(wl, a2, None)
    _chunk(wl, a2, 0, passes=(ro.WRITE_BACK,))
    a2.reset()
    a2.restore(k, v, ids)
    assert _same_state(a, a2)
    # the stream continues identically on all three
    for ch in range(n0, n0 + 3):
        oa = _chunk(wl, a, ch)
        ob = _chunk(wl, b, ch)
        o2 = _chunk(wl, a2, ch)
        torch.cuda.synchronize()
        for x, y, z in zip(oa, ob, o2):
            assert torch.equal(x, y) and torch.equal(x, z), f"chunk {ch}"
    ka, va, ia = a.gather()
    kb, vb, ib = b.gather()
    torch.cuda.synchronize()
    assert ia == ib and torch.equal(ka, kb) and torch.equal(va, vb)


@pytest.mark.parametrize("name", ["small_abs", "lb480"])
def test_reset_and_reappend_in_logical_order(name):
    """ABS: after a reset, appending the snapshot's frames oldest first stores the same bytes (ids
    0..n-1); the next chunk, rotated at its true start frame, still matches the oracle."""
    wl = WORKLOADS[name]
    c = wl.cfg
    f = c.tokens_per_frame
    n0 = wl.steady_chunk + 2
    say(f"[re-append] {name}: {n0} chunks")
    cache = skv.KVCache(c)
    orc = ro.oracle_for(wl)
    for ch in range(n0):
        k = ro.draw(wl, c.chunk_frames, ch, ro.WRITE_BACK, si.K)
        v = ro.draw(wl, c.chunk_frames, ch, ro.WRITE_BACK, si.V)
        t = cache.info().n_appended
        cache.append_evict(cache.rope_apply(k.cuda(), start_frame=t), v.cuda())
        orc.append(ro.f64(k), ro.f64(v))
    k, v, ids = cache.gather()
    t_true = cache.info().n_appended
    cache.reset()
    n = len(ids)
    step = c.window_frames - c.sink_frames
    for i0 in range(0, n, step):
        i1 = min(n, i0 + step)
        cache.append_evict(k[i0 * f:i1 * f].contiguous(), v[i0 * f:i1 * f].contiguous())
    k2, v2, ids2 = cache.gather()
    torch.cuda.synchronize()
    assert ids2 == list(range(n)) and torch.equal(k2, k) and torch.equal(v2, v)
    # next chunk: queries and keys at the true absolute ids
    q, kc, vc = (ro.draw(wl, c.chunk_frames, n0, 0, t) for t in (si.Q, si.K, si.V))
    qr, kr = cache.rope_apply_qk(q.cuda(), kc.cuda(), start_frame=t_true)
    out = cache.chunk_attention(qr, kr, vc.cuda())
    torch.cuda.synchronize()
    rows = None if wl.lq <= 512 else torch.arange(0, wl.lq, 97).numpy()
    ref = orc.chunk_attention(ro.f64(q), ro.f64(kc), ro.f64(vc), rows=rows)
    got = out if rows is None else out[torch.as_tensor(rows, device=out.device)]
    e = ro.assert_close(got, ref, c.dtype, f"{name} after re-append")
    say(f"  next chunk: max {e[0]:.3g} mean {e[1]:.3g} relrms {e[2]:.3g}")
