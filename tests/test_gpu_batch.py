"""GPU tests of chunk_attention_batch: the two caches of classifier-free guidance in one launch.

Two caches (conditional / unconditional) of one configuration advance in lockstep on
different seeded inputs (seed bases 0 and 500).  Every pass of the batch call must
(a) match the oracle of each cache to the usual tolerance and (b) equal, bit for bit,
the output of a single chunk_attention call on the same inputs run with the same
kernel shape (the shape is forced, since the batch grid may select the other one).
"""
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
@pytest.mark.parametrize("name", ["small_abs", "small_rel", "small_f32_rel"])
def test_guidance_batch(name, waves, monkeypatch):
    monkeypatch.setenv("SKV_ATTN_WAVES", waves)
    # bit-equality with single calls needs the same key split: a batch's grid may choose another
    monkeypatch.setenv("SKV_ATTN_SPLIT", "0")
    wl = WORKLOADS[name]
    cfg = wl.cfg
    bases = (0, 500)
    caches = [skv.KVCache(cfg) for _ in bases]
    orcs = [ro.oracle_for(wl) for _ in bases]
    for cache, orc, b in zip(caches, orcs, bases):
        ro.prefill(wl, cache, orc, b)
    say(f"[batch] {name} waves={waves} chunks={wl.n_chunks}")
    for ch in range(wl.n_chunks):
        if cfg.rope_mode == skv.ROPE_REL:
            for cache in caches:
                cache.rope_apply_window()
        for p in (0, 1, ro.WRITE_BACK):
            qs, ks, vs, qr, kr = [], [], [], [], []
            for cache, b in zip(caches, bases):
                t = cache.info().n_appended
                q, k, v = (ro.draw(wl, cfg.chunk_frames, ch, p, tid, b) for tid in (si.Q, si.K, si.V))
                qs.append(q), ks.append(k), vs.append(v)
                qr.append(cache.rope_apply(q.cuda(), start_frame=t))
                kr.append(cache.rope_apply(k.cuda(), start_frame=t))
            vd = [v.cuda() for v in vs]
            # staged values for the second element (v_cur NULL), given values for the first
            caches[1].stage_v(vd[1])
            outs = skv.chunk_attention_batch(caches, qr, kr, [vd[0], None])
            singles = [cache.chunk_attention(qr[i], kr[i], vd[i]) for i, cache in enumerate(caches)]
            torch.cuda.synchronize()
            for i in range(2):
                assert torch.equal(outs[i], singles[i]), f"chunk {ch} pass {p} element {i}: batch != single"
                ref = orcs[i].chunk_attention(ro.f64(qs[i]), ro.f64(ks[i]), ro.f64(vs[i]))
                ro.assert_close(outs[i], ref, cfg.dtype, f"{name} chunk {ch} pass {p} element {i}")
            if p == ro.WRITE_BACK:
                for i, cache in enumerate(caches):
                    cache.append_evict(kr[i] if cfg.rope_mode == skv.ROPE_ABS else ks[i].cuda(), vd[i])
                    orcs[i].append(ro.f64(ks[i]), ro.f64(vs[i]))


def test_guidance_batch_then_sampler():
    """Guided velocity from the two batch outputs (sampler_step with v_uncond) equals the oracle's
    guidance of the oracle outputs, within the attention tolerance scaled by the guidance."""
    import numpy as np
    from oracle import sampler as sp
    wl = WORKLOADS["small_abs"]
    cfg = wl.cfg
    caches = [skv.KVCache(cfg) for _ in range(2)]
    orcs = [ro.oracle_for(wl) for _ in range(2)]
    q, k, v = [], [], []
    for b in (0, 500):
        q.append(ro.draw(wl, cfg.chunk_frames, 0, 0, si.Q, b))
        k.append(ro.draw(wl, cfg.chunk_frames, 0, 0, si.K, b))
        v.append(ro.draw(wl, cfg.chunk_frames, 0, 0, si.V, b))
    qr = [c.rope_apply(x.cuda(), start_frame=0) for c, x in zip(caches, q)]
    kr = [c.rope_apply(x.cuda(), start_frame=0) for c, x in zip(caches, k)]
    outs = skv.chunk_attention_batch(caches, qr, kr, [x.cuda() for x in v])
    x_t = ro.draw(wl, cfg.chunk_frames, 0, 0, si.NOISE, 0).cuda()
    x0, _ = skv.sampler_step(x_t, outs[0], 0.75, v_uncond=outs[1], cfg_scale=5.0)
    torch.cuda.synchronize()
    refs = [o.chunk_attention(ro.f64(a), ro.f64(b), ro.f64(c)) for o, a, b, c in zip(orcs, q, k, v)]
    ex0, _ = sp.sampler_step(ro.f64(x_t.cpu()), refs[0], 0.75, v_uncond=refs[1], cfg_scale=5.0)
    err = np.abs(x0.float().cpu().double().numpy() - ex0)
    # attention error (<= 2e-2 each) times 0.75 * (5 + 4), plus the bf16 rounding of x0
    assert err.max() <= 0.75 * 9 * 2e-2 + 2.0 ** -7 * np.abs(ex0).max(), err.max()


@pytest.mark.parametrize("nb", [3, 4])
def test_wide_batch(nb, monkeypatch):
    """Three and four caches (the batch limit) of 40 heads x 4 query tiles (160 four-wave workgroups
    each, so four make a grid past one dispatch round): every element equals its single
    chunk_attention call bit for bit, and element 0 matches the oracle."""
    from streaming_kv_cache_amd.workloads import Workload
    monkeypatch.setenv("SKV_ATTN_SPLIT", "0")   # bit-equality with single calls: same (no) key split
    cfg = skv.Config(40, 128, 8, 16, 4, 1, 6, skv.ROPE_ABS, skv.BF16)
    wl = Workload("batch_wide", cfg, n_chunks=3)
    say(f"[batch split] nb={nb} heads={cfg.heads} lq={cfg.chunk_frames * cfg.tokens_per_frame}")
    bases = tuple(100 * i for i in range(nb))
    caches = [skv.KVCache(cfg) for _ in bases]
    orc = ro.oracle_for(wl)
    for ch in range(wl.n_chunks):
        qr, kr, vd, raw0 = [], [], [], None
        for cache, b in zip(caches, bases):
            t = cache.info().n_appended
            q, k, v = (ro.draw(wl, cfg.chunk_frames, ch, 0, tid, b) for tid in (si.Q, si.K, si.V))
            if b == 0:
                raw0 = (q, k, v)
            rq, rk = cache.rope_apply_qk(q.cuda(), k.cuda(), start_frame=t)
            qr.append(rq), kr.append(rk), vd.append(v.cuda())
        outs = skv.chunk_attention_batch(caches, qr, kr, vd)
        singles = [cache.chunk_attention(qr[i], kr[i], vd[i]) for i, cache in enumerate(caches)]
        torch.cuda.synchronize()
        for i in range(nb):
            assert torch.equal(outs[i], singles[i]), f"chunk {ch} element {i}: batch != single"
        ref = orc.chunk_attention(*(ro.f64(x) for x in raw0))
        ro.assert_close(outs[0], ref, cfg.dtype, f"batch_wide chunk {ch} element 0")
        for i, cache in enumerate(caches):
            cache.append_evict(kr[i], vd[i])
        orc.append(ro.f64(raw0[1]), ro.f64(raw0[2]))


@pytest.mark.parametrize("name", ["small_abs", "small_rel"])
def test_guidance_batch_split(name):
    """With key splits (the default for these small grids) the batch still matches the oracle."""
    wl = WORKLOADS[name]
    cfg = wl.cfg
    bases = (0, 500)
    caches = [skv.KVCache(cfg) for _ in bases]
    orcs = [ro.oracle_for(wl) for _ in bases]
    for cache, orc, b in zip(caches, orcs, bases):
        ro.prefill(wl, cache, orc, b)
    say(f"[batch split] {name}")
    for ch in range(wl.n_chunks):
        if cfg.rope_mode == skv.ROPE_REL:
            for cache in caches:
                cache.rope_apply_window()
        qs, ks, vs, qr, kr = [], [], [], [], []
        for cache, b in zip(caches, bases):
            t = cache.info().n_appended
            q, k, v = (ro.draw(wl, cfg.chunk_frames, ch, ro.WRITE_BACK, tid, b) for tid in (si.Q, si.K, si.V))
            qs.append(q), ks.append(k), vs.append(v)
            a, bk = cache.rope_apply_qk(q.cuda(), k.cuda(), start_frame=t)
            qr.append(a), kr.append(bk)
        vd = [v.cuda() for v in vs]
        outs = skv.chunk_attention_batch(caches, qr, kr, vd)
        torch.cuda.synchronize()
        for i in range(2):
            ref = orcs[i].chunk_attention(ro.f64(qs[i]), ro.f64(ks[i]), ro.f64(vs[i]))
            ro.assert_close(outs[i], ref, cfg.dtype, f"{name} chunk {ch} element {i}")
        for i, cache in enumerate(caches):
            cache.append_evict(kr[i] if cfg.rope_mode == skv.ROPE_ABS else ks[i].cuda(), vd[i])
            orcs[i].append(ro.f64(ks[i]), ro.f64(vs[i]))
