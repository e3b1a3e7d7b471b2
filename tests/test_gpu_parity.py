"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Bars: cache contents bit-exact; attention within max-abs 2e-2 / mean-abs 2e-3 /
relative RMS 1e-2 in bf16 and max-abs 1e-5 in fp32; RoPE within one bf16 ulp
(fp32: 1e-6 of the pair norm) of the fp64 value.
"""
import sys

import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import skv_oracle as so
from tests import rollout as ro

skv = pytest.importorskip("streaming_kv_cache_amd")
from streaming_kv_cache_amd.workloads import WORKLOADS  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


SMALL = ["tiny", "small_abs", "small_rel", "small_d64", "small_f32_rel", "small_nosink"]


# ------------------------------------------------------------------ cache update
@pytest.mark.parametrize("name", SMALL)
def test_append_gather_bitexact(name):
    wl = WORKLOADS[name]
    c = wl.cfg
    say(f"[append/gather] {name}")
    cache = skv.KVCache(c)
    cl = so.CacheList(c.sink_frames, c.window_frames)
    rng = np.random.default_rng(1)
    for step in range(40):
        n = c.chunk_frames if rng.random() < 0.6 else int(rng.integers(1, c.window_frames - c.sink_frames + 1))
        k = ro.draw(wl, n, step, 0, si.K)
        v = ro.draw(wl, n, step, 0, si.V)
        cache.append_evict(k.cuda(), v.cuda())
        f = c.tokens_per_frame
        cl.append([k[i * f:(i + 1) * f] for i in range(n)], [v[i * f:(i + 1) * f] for i in range(n)])
        gk, gv, ids = cache.gather()
        torch.cuda.synchronize()
        assert ids == cl.frame_ids()
        ek = torch.cat([e[1] for e in cl.entries])
        ev = torch.cat([e[2] for e in cl.entries])
        assert torch.equal(gk.cpu(), ek) and torch.equal(gv.cpu(), ev), f"step {step}"


def test_sinks_survive_300_chunks():
    wl = WORKLOADS["small_abs"]
    c = wl.cfg
    say("[sinks] small_abs 300 chunks")
    cache = skv.KVCache(c)
    f = c.tokens_per_frame
    first = []
    for ch in range(300):
        k = ro.draw(wl, c.chunk_frames, ch, 0, si.K).cuda()
        v = ro.draw(wl, c.chunk_frames, ch, 0, si.V).cuda()
        cache.append_evict(k, v)
        if ch == 0:
            first = [k.clone(), v.clone()]
    gk, gv, ids = cache.gather()
    torch.cuda.synchronize()
    s = c.sink_frames
    assert ids[:s] == list(range(s)) and ids[-1] == 300 * c.chunk_frames - 1
    assert torch.equal(gk[:s * f], first[0][:s * f]) and torch.equal(gv[:s * f], first[1][:s * f])


# ------------------------------------------------------------------ RoPE
def _rope_close(got, ref, dtype):
    g = got.float().cpu().double().numpy()
    if dtype == skv.F32:
        pair = np.abs(ref[..., 0::2]) + np.abs(ref[..., 1::2])
        bound = 1e-6 * np.repeat(pair, 2, axis=-1) + 1e-30
        assert np.all(np.abs(g - ref) <= bound)
    else:
        # one bf16 ulp of the exact value, plus the fp32 rounding of the rotation itself
        a = np.abs(ref)
        ulp = np.where(a > 0, 2.0 ** (np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7), 2.0 ** -133)
        pair = np.repeat(np.abs(ref[..., 0::2]) + np.abs(ref[..., 1::2]), 2, axis=-1)
        bound = ulp + 2.0 ** -20 * pair
        assert np.all(np.abs(g - ref) <= bound), float(np.max(np.abs(g - ref) / bound))


@pytest.mark.parametrize("name", ["tiny", "small_abs", "small_d64", "lb480"])
@pytest.mark.parametrize("start", [0, 7, 1199])
def test_rope_abs(name, start):
    wl = WORKLOADS[name]
    c = wl.cfg
    say(f"[rope abs] {name} start={start}")
    cache = skv.KVCache(c)
    x = ro.draw(wl, c.chunk_frames, start, 0, si.Q)
    got = cache.rope_apply(x.cuda(), start_frame=start)
    torch.cuda.synchronize()
    orc = ro.oracle_for(wl)
    ref = so.rope_3d(ro.f64(x), range(start, start + c.chunk_frames), c.grid_h, c.grid_w, orc.split)
    _rope_close(got, ref, c.dtype)
    # in place
    xd = x.cuda()
    cache.rope_apply(xd, out=xd, start_frame=start)
    torch.cuda.synchronize()
    assert torch.equal(xd, got)


@pytest.mark.parametrize("name", ["tiny", "small_abs", "small_rel", "small_f32_rel", "lb480", "abot720"])
def test_rope_apply_qk_matches_two_calls(name):
    """One launch over q and k gives exactly the bytes of two rope_apply calls (same ids, same math),
    in place too; REL after a few appends so the chunk's slot ids are past the first frames."""
    wl = WORKLOADS[name]
    c = wl.cfg
    say(f"[rope qk] {name}")
    cache = skv.KVCache(c)
    ro.prefill(wl, cache, None)
    for ch in range(3):
        cache.append_evict(ro.draw(wl, c.chunk_frames, ch, 4, si.K).cuda(), ro.draw(wl, c.chunk_frames, ch, 4, si.V).cuda())
    start = cache.info().n_appended
    q = ro.draw(wl, c.chunk_frames, 5, 0, si.Q).cuda()
    k = ro.draw(wl, c.chunk_frames, 5, 0, si.K).cuda()
    rq = cache.rope_apply(q, start_frame=start)
    rk = cache.rope_apply(k, start_frame=start)
    gq, gk = cache.rope_apply_qk(q, k, start_frame=start)
    q2, k2 = q.clone(), k.clone()
    cache.rope_apply_qk(q2, k2, q_out=q2, k_out=k2, start_frame=start)
    torch.cuda.synchronize()
    assert torch.equal(gq, rq) and torch.equal(gk, rk)
    assert torch.equal(q2, rq) and torch.equal(k2, rk)


@pytest.mark.parametrize("name", ["tiny", "small_abs", "small_rel", "small_d64", "small_f32_rel", "lb480", "abot720"])
def test_prepare_pass_matches_separate_calls(name):
    """kv_cache_prepare_pass (rotary and V^T staging blocks in one grid for bf16) writes exactly the bytes
    of rope_apply_qk followed by kv_cache_stage_v: the rotated q and k compare bitwise, and attention over
    the values it staged equals, bitwise, attention that stages the same values itself."""
    wl = WORKLOADS[name]
    c = wl.cfg
    say(f"[prepare pass] {name}")
    cache = skv.KVCache(c)
    ro.prefill(wl, cache, None)
    for ch in range(3):
        cache.append_evict(ro.draw(wl, c.chunk_frames, ch, 4, si.K).cuda(), ro.draw(wl, c.chunk_frames, ch, 4, si.V).cuda())
    if c.rope_mode == skv.ROPE_REL:
        cache.rope_apply_window()
    start = cache.info().n_appended
    q = ro.draw(wl, c.chunk_frames, 5, 0, si.Q).cuda()
    k = ro.draw(wl, c.chunk_frames, 5, 0, si.K).cuda()
    v = ro.draw(wl, c.chunk_frames, 5, 0, si.V).cuda()
    rq, rk = cache.rope_apply_qk(q, k, start_frame=start)
    ref = cache.chunk_attention(rq, rk, v)
    cache.stage_v(ro.draw(wl, c.chunk_frames, 6, 0, si.V).cuda())  # other values in the staging area first
    gq, gk = cache.prepare_pass(q, k, v, start_frame=start)
    got = cache.chunk_attention(gq, gk, None)
    torch.cuda.synchronize()
    assert torch.equal(gq, rq) and torch.equal(gk, rk)
    assert torch.equal(got, ref)


@pytest.mark.parametrize("name", ["small_rel", "small_f32_rel", "abot720"])
def test_rope_rel_and_window(name):
    wl = WORKLOADS[name]
    c = wl.cfg
    say(f"[rope rel] {name}")
    cache = skv.KVCache(c)
    orc = ro.oracle_for(wl)
    ro.prefill(wl, cache, orc)
    f = c.tokens_per_frame
    for ch in range(wl.steady_chunk + 3):
        x = ro.draw(wl, c.chunk_frames, ch, 1, si.Q)
        got = cache.rope_apply(x.cuda())
        cache.rope_apply_window()
        torch.cuda.synchronize()
        ref = orc._rope(ro.f64(x), orc.query_time_ids())
        _rope_close(got, ref, c.dtype)
        # window: visible history k_raw rotated at slot ids, logical order, head-major workspace
        hist = orc.visible()
        if hist and (ch % 2 == 0 or ch == wl.steady_chunk + 2):
            nh = len(hist)
            nwin = c.heads * (c.window_frames - c.chunk_frames) * f * c.head_dim
            ws = cache.workspace.view(c.torch_dtype)[:nwin].view(c.heads, (c.window_frames - c.chunk_frames) * f,
                                                                 c.head_dim)[:, :nh * f]
            wsd = ws.permute(1, 0, 2).contiguous()
            refw = np.concatenate([orc._rope(e[1], [j]) for j, e in enumerate(hist)])
            _rope_close(wsd, refw, c.dtype)
        k = ro.draw(wl, c.chunk_frames, ch, 4, si.K)
        v = ro.draw(wl, c.chunk_frames, ch, 4, si.V)
        cache.append_evict(k.cuda(), v.cuda())
        orc.append(ro.f64(k), ro.f64(v))


# ------------------------------------------------------------------ attention
@pytest.mark.parametrize("name", SMALL)
def test_rollout_parity(name):
    wl = WORKLOADS[name]
    say(f"[rollout] {name} chunks={wl.n_chunks}")
    worst = (0.0, 0.0, 0.0)
    for ch, p, out, ref in ro.rollout(wl, wl.n_chunks):
        torch.cuda.synchronize()
        e = ro.assert_close(out, ref, wl.cfg.dtype, f"{name} chunk {ch} pass {p}")
        worst = tuple(max(a, b) for a, b in zip(worst, e))
    say(f"  worst max/mean/relrms = {worst}")


@pytest.mark.parametrize("split", ["0", "auto"])
@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("name", ["small_abs", "small_rel", "small_d64", "small_nosink"])
def test_rollout_parity_kernel_shapes(name, waves, split, monkeypatch):
    """Both bf16 kernel shapes (4 waves / two stages, 8 waves / four stages) on the same rollouts,
    with the keys split over workgroups (the default for these small grids) and without."""
    monkeypatch.setenv("SKV_ATTN_WAVES", waves)
    if split == "0":
        monkeypatch.setenv("SKV_ATTN_SPLIT", "0")
    else:
        monkeypatch.delenv("SKV_ATTN_SPLIT", raising=False)
    wl = WORKLOADS[name]
    say(f"[rollout] {name} waves={waves} split={split} chunks={wl.n_chunks}")
    for ch, p, out, ref in ro.rollout(wl, wl.n_chunks):
        torch.cuda.synchronize()
        ro.assert_close(out, ref, wl.cfg.dtype, f"{name} waves {waves} chunk {ch} pass {p}")


def _edge_workloads():
    from streaming_kv_cache_amd.workloads import Workload
    C = skv.Config
    return {
        # one head, one-frame chunks, ring of two frames, relative ids
        "edge_h1_c1_rel": Workload("edge_h1_c1_rel", C(1, 128, 3, 5, 1, 1, 3, skv.ROPE_REL, skv.BF16), n_chunks=7),
        # one token per frame: every range start is unaligned (element-copy V path), one partial tile
        "edge_f1_abs": Workload("edge_f1_abs", C(2, 64, 1, 1, 2, 1, 5, skv.ROPE_ABS, skv.BF16), n_chunks=8),
        # W = S + c with relative ids: a chunk sees only the sinks and itself
        "edge_rel_tight": Workload("edge_rel_tight", C(2, 128, 4, 4, 2, 2, 4, skv.ROPE_REL, skv.BF16), n_chunks=6),
        # a chunk of 6 frames in a window of 7 without sinks: the ring wraps inside every append
        "edge_bigc_nosink": Workload("edge_bigc_nosink", C(2, 128, 5, 7, 6, 0, 7, skv.ROPE_ABS, skv.BF16),
                                     n_chunks=5),
        # fp32, D = 32, one token per frame, no sinks, window 2, one-frame chunks
        "edge_f1_f32_rel": Workload("edge_f1_f32_rel", C(1, 32, 1, 1, 1, 0, 2, skv.ROPE_REL, skv.F32), n_chunks=6),
    }


EDGE = list(_edge_workloads())


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("name", EDGE)
def test_edge_shapes(name, waves, fused, monkeypatch):
    """Degenerate shapes through every pass of a rollout against the oracle: both kernel shapes, the
    pages' protocol and the fused rotation."""
    wl = _edge_workloads()[name]
    if wl.cfg.dtype == skv.F32 and waves == "8":
        pytest.skip("one fp32 kernel shape")
    monkeypatch.setenv("SKV_ATTN_WAVES", waves)
    if fused:
        wl = ro.fused(wl)
    say(f"[edge] {name} waves={waves} fused={fused} chunks={wl.n_chunks}")
    for ch, p, out, ref in ro.rollout(wl, wl.n_chunks):
        torch.cuda.synchronize()
        ro.assert_close(out, ref, wl.cfg.dtype, f"{name} chunk {ch} pass {p}")


@pytest.mark.parametrize("name", EDGE)
def test_edge_append_gather(name):
    """Cache contents after every append equal the closed form bit for bit on the degenerate shapes."""
    wl = _edge_workloads()[name]
    c = wl.cfg
    say(f"[edge gather] {name}")
    cache = skv.KVCache(c)
    hist_k, hist_v = [], []
    for ch in range(wl.n_chunks + 2):
        k = ro.draw(wl, c.chunk_frames, ch, 4, si.K)
        v = ro.draw(wl, c.chunk_frames, ch, 4, si.V)
        cache.append_evict(k.cuda(), v.cuda())
        f = c.tokens_per_frame
        hist_k += [k[i * f:(i + 1) * f] for i in range(c.chunk_frames)]
        hist_v += [v[i * f:(i + 1) * f] for i in range(c.chunk_frames)]
        t = len(hist_k)
        keep = list(range(min(c.sink_frames, t))) + list(range(max(c.sink_frames, t - (c.window_frames - c.sink_frames)), t))
        gk, gv, ids = cache.gather()
        torch.cuda.synchronize()
        assert list(ids) == keep
        assert torch.equal(gk.cpu(), torch.cat([hist_k[i] for i in keep]))
        assert torch.equal(gv.cpu(), torch.cat([hist_v[i] for i in keep]))


def _probe_rollout(wl, mode):
    """q = 0 with one-hot (mode 'onehot') or random (mode 'zeroq') values: the answer is a plain mean."""
    c = wl.cfg
    f = c.tokens_per_frame
    cache = skv.KVCache(c)
    orc = ro.oracle_for(wl)
    ro.prefill(wl, cache, orc)
    lq = c.chunk_frames * f

    def values(first_frame, n, ch):
        if mode == "zeroq":
            return ro.draw(wl, n, ch, 2, si.V)
        v = torch.zeros(n * f, c.heads, c.head_dim)
        for i in range(n):
            v[i * f:(i + 1) * f, :, (first_frame + i) % c.head_dim] = 1.0
        return v.to(c.torch_dtype)

    if wl.prefill:  # replace the random sink values by probe values (same frames)
        cache.reset()
        orc = ro.oracle_for(wl)
        sk = ro.draw(wl, wl.prefill, 0, 0, si.SINK_K)
        sv = values(0, wl.prefill, 0)
        cache.append_evict(sk.cuda(), sv.cuda())
        orc.append(ro.f64(sk), ro.f64(sv))
    for ch in range(wl.n_chunks):
        t = cache.info().n_appended
        if c.rope_mode == skv.ROPE_REL:
            cache.rope_apply_window()
        q = torch.zeros(lq, c.heads, c.head_dim, dtype=c.torch_dtype)
        k = ro.draw(wl, c.chunk_frames, ch, 1, si.K)
        v = values(t, c.chunk_frames, ch)
        out, k_app, v_app = ro.gpu_pass(cache, q, k, v)
        torch.cuda.synchronize()
        ref = orc.chunk_attention(ro.f64(q), ro.f64(k), ro.f64(v))
        g = out.float().cpu().double().numpy()
        if mode == "onehot":
            # exact closed form: 1/n_vis on each visible frame's channel
            vis = [e[0] for e in orc.visible()] + list(range(t, t + c.chunk_frames))
            expect = np.zeros(c.head_dim)
            for fr in vis:
                expect[fr % c.head_dim] += 1.0 / len(vis)
            assert np.allclose(ref, expect[None, None], atol=1e-12)
            tol = 1e-5 if c.dtype == skv.F32 else 2.0 ** -8 * expect.max() + 1e-6
            assert np.abs(g - expect[None, None]).max() <= tol, f"chunk {ch}"
        else:
            ro.assert_close(out, ref, c.dtype, f"zero-q chunk {ch}")
        cache.append_evict(k_app, v_app)
        orc.append(ro.f64(k), ro.f64(v))


@pytest.mark.parametrize("name", ["small_abs", "small_rel", "tiny", "small_nosink"])
@pytest.mark.parametrize("mode", ["onehot", "zeroq"])
def test_visibility_probes(name, mode):
    say(f"[probe] {name} {mode}")
    _probe_rollout(WORKLOADS[name], mode)


@pytest.mark.parametrize("dtype,n_q,n_text,h,d", [
    (skv.BF16, 1000, 512, 5, 128), (skv.BF16, 130, 77, 3, 64), (skv.F32, 70, 512, 2, 128), (skv.F32, 33, 9, 1, 32),
])
def test_cross_attention(dtype, n_q, n_text, h, d):
    say(f"[cross] dtype={dtype} n_q={n_q} n_text={n_text} h={h} d={d}")
    tdt = torch.bfloat16 if dtype == skv.BF16 else torch.float32
    q = si.draw((n_q, h, d), 0, 0, 0, si.Q, tdt)
    kt = si.draw((n_text, h, d), 0, 0, 0, si.TEXT_K, tdt)
    vt = si.draw((n_text, h, d), 0, 0, 0, si.TEXT_V, tdt)
    out = skv.cross_attention(q.cuda(), kt.cuda(), vt.cuda())
    torch.cuda.synchronize()
    ref = so.cross_attention(ro.f64(q), ro.f64(kt), ro.f64(vt))
    ro.assert_close(out, ref, dtype, "cross")


@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("dtype,n_q,n_text,h,d", [
    (skv.BF16, 1000, 512, 5, 128), (skv.BF16, 130, 77, 3, 64), (skv.BF16, 6240, 512, 40, 128),
    (skv.F32, 70, 512, 2, 128), (skv.F32, 33, 9, 1, 32),
])
def test_cross_attention_cached(dtype, n_q, n_text, h, d, waves, monkeypatch):
    """Prepared text cache (copy of K, V^T rows) + the matrix-core kernel against the oracle's
    cross attention; both kernel shapes; the largest case is the 480P chunk against 512 text tokens."""
    if dtype == skv.F32 and waves == "8":
        pytest.skip("one fp32 kernel shape")
    monkeypatch.setenv("SKV_ATTN_WAVES", waves)
    say(f"[cross cached] dtype={dtype} n_q={n_q} n_text={n_text} h={h} d={d} waves={waves}")
    tdt = torch.bfloat16 if dtype == skv.BF16 else torch.float32
    q = si.draw((n_q, h, d), 0, 0, 0, si.Q, tdt)
    kt = si.draw((n_text, h, d), 0, 0, 0, si.TEXT_K, tdt)
    vt = si.draw((n_text, h, d), 0, 0, 0, si.TEXT_V, tdt)
    tc = skv.TextCache(kt.cuda(), vt.cuda())
    out = tc.attend(q.cuda())
    again = tc.attend(q.cuda())
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    rows = _rows(n_q) if n_q > 2000 else np.arange(n_q)
    ref = so.cross_attention(ro.f64(q[torch.as_tensor(rows)]), ro.f64(kt), ro.f64(vt))
    ro.assert_close(out[torch.as_tensor(rows, device=out.device)], ref, dtype, "cross cached")


@pytest.mark.parametrize("dtype,n_text,h,d", [(skv.BF16, 77, 3, 64), (skv.BF16, 512, 4, 128), (skv.F32, 9, 2, 32)])
def test_text_cache_layout(dtype, n_text, h, d):
    """The prepared store holds the bytes the header states.  bf16: K head-major ([h][key][d], rows up
    to roundup(n_text, 64), past n_text zero), then V^T in tiles of 64 keys ([h][key / 64][d][key % 64],
    keys past n_text zero); fp32: copies of K and V.  The second part starts at a 256-byte boundary."""
    say(f"[text store] dtype={dtype} n_text={n_text} h={h} d={d}")
    tdt = torch.bfloat16 if dtype == skv.BF16 else torch.float32
    kt = si.draw((n_text, h, d), 0, 0, 1, si.TEXT_K, tdt).cuda()
    vt = si.draw((n_text, h, d), 0, 0, 1, si.TEXT_V, tdt).cuda()
    store = skv.text_cache_prepare(kt, vt)
    torch.cuda.synchronize()
    pad = (n_text + 63) // 64 * 64
    kb = (h * pad * d if dtype == skv.BF16 else n_text * h * d) * kt.element_size()
    off = (kb + 255) // 256 * 256
    assert store.numel() == skv.text_cache_bytes(n_text, h, d, dtype)
    if dtype == skv.BF16:
        k_hm = store[:kb].view(tdt).view(h, pad, d)
        assert torch.equal(k_hm[:, :n_text], kt.permute(1, 0, 2))
        assert not k_hm[:, n_text:].any()
    else:
        assert torch.equal(store[:kb].view(tdt).view(n_text, h, d), kt)
    if dtype == skv.BF16:
        tiles = store[off:].view(tdt).view(h, pad // 64, d, 64)
        v_t = tiles.permute(0, 2, 1, 3).reshape(h, d, pad)      # back to [h][d][key]
        assert torch.equal(v_t[:, :, :n_text], vt.permute(1, 2, 0))
        assert not v_t[:, :, n_text:].any()
    else:
        assert torch.equal(store[off:off + kb].view(tdt).view(n_text, h, d), vt)


def test_determinism():
    say("[determinism] small_rel twice")
    wl = WORKLOADS["small_rel"]
    a = [o.clone() for _, _, o, _ in ro.rollout(wl, 6, with_oracle=False)]
    b = [o.clone() for _, _, o, _ in ro.rollout(wl, 6, with_oracle=False)]
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_edge_window_equals_sink_plus_chunk():
    """W = S + c: a chunk sees only the sinks and itself."""
    say("[edge] W = S + c")
    cfg = skv.Config(2, 128, 3, 7, 2, 1, 3, skv.ROPE_ABS, skv.BF16)
    from streaming_kv_cache_amd.workloads import Workload
    wl = Workload("edge", cfg, n_chunks=6)
    for ch, p, out, ref in ro.rollout(wl, 6, passes=(0, ro.WRITE_BACK)):
        torch.cuda.synchronize()
        ro.assert_close(out, ref, cfg.dtype, f"edge chunk {ch}")


# ------------------------------------------------------------------ full-size shapes
def _rows(lq, n=48, seed=0):
    rng = np.random.default_rng(seed)
    r = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, lq - 1], rng.integers(0, lq, n)]))
    return r[r < lq]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["abot720", "lb480", "lb720", "abot720_h3", "lb480_h5"])
def test_full_size_sampled(name):
    """Roll out to the first steady chunk and one past it; compare sampled query rows (all heads)."""
    wl = WORKLOADS[name]
    rows = _rows(wl.lq)
    last = wl.steady_chunk + 1
    say(f"[full] {name} to chunk {last}, {len(rows)} rows")
    checked = 0
    for ch, p, out, ref in ro.rollout(wl, last + 1, passes=(0, ro.WRITE_BACK), rows=rows,
                                      oracle_chunks={0, wl.steady_chunk, last}):
        if ref is None:
            continue
        torch.cuda.synchronize()
        got = out[torch.as_tensor(rows, device=out.device)]
        e = ro.assert_close(got, ref, wl.cfg.dtype, f"{name} chunk {ch} pass {p}")
        say(f"  chunk {ch} pass {p}: max {e[0]:.3g} mean {e[1]:.3g} relrms {e[2]:.3g}")
        checked += 1
    assert checked == 6


@pytest.mark.parametrize("name", ["abot720_h3", "lb480_h5"])
def test_split_matches_unsplit(name, monkeypatch):
    """One GPU's share of a head-sharded model (ABot 3 of 24 heads, LingBot 480P 5 of 40): the key
    split the small grid takes agrees with the unsplit kernel on every row (the two differ only in
    summation order), and the split path is the one taken by default."""
    wl = WORKLOADS[name]
    c = wl.cfg
    say(f"[split] {name}")
    cache = skv.KVCache(c)
    ro.prefill(wl, cache, None)
    while cache.info().n_vis < c.window_frames:
        k = ro.draw(wl, c.chunk_frames, 0, 4, si.K).cuda()
        cache.append_evict(k if c.rope_mode == skv.ROPE_REL else cache.rope_apply(k, start_frame=cache.info().n_appended),
                           ro.draw(wl, c.chunk_frames, 0, 4, si.V).cuda())
    if c.rope_mode == skv.ROPE_REL:
        cache.rope_apply_window()
    t = cache.info().n_appended
    q, k = cache.rope_apply_qk(ro.draw(wl, c.chunk_frames, 1, 0, si.Q).cuda(), ro.draw(wl, c.chunk_frames, 1, 0, si.K).cuda(),
                               start_frame=t)
    v = ro.draw(wl, c.chunk_frames, 1, 0, si.V).cuda()
    monkeypatch.delenv("SKV_ATTN_SPLIT", raising=False)
    split = cache.chunk_attention(q, k, v)
    monkeypatch.setenv("SKV_ATTN_SPLIT", "0")
    whole = cache.chunk_attention(q, k, v)
    torch.cuda.synchronize()
    e = ro.errors(split, whole.float().cpu().double().numpy())
    say(f"  split vs unsplit: max {e[0]:.3g} mean {e[1]:.3g} relrms {e[2]:.3g}")
    # both outputs are bf16 roundings (relative error <= 2^-9 each) of sums whose P were rounded to
    # bf16 against different running maxima: they may differ by 2^-8 relative
    assert e[0] <= 2 ** -7 and e[2] <= 2 ** -8


def test_staged_v_matches_direct():
    """kv_cache_stage_v + chunk_attention(v_cur=NULL) gives the same bytes as passing v_cur."""
    wl = WORKLOADS["small_rel"]
    c = wl.cfg
    say("[staged v] small_rel")
    cache = skv.KVCache(c)
    ro.prefill(wl, cache, None)
    for ch in range(4):
        cache.rope_apply_window()
        q = cache.rope_apply(ro.draw(wl, c.chunk_frames, ch, 0, si.Q).cuda())
        k = cache.rope_apply(ro.draw(wl, c.chunk_frames, ch, 0, si.K).cuda())
        v = ro.draw(wl, c.chunk_frames, ch, 0, si.V).cuda()
        direct = cache.chunk_attention(q, k, v)
        cache.stage_v(v)
        staged = cache.chunk_attention(q, k, None)
        torch.cuda.synchronize()
        assert torch.equal(direct, staged)
        cache.append_evict(ro.draw(wl, c.chunk_frames, ch, 4, si.K).cuda(), v)
    with pytest.raises(skv.SkvError):
        cache.chunk_attention(q, k, None)   # append cleared the staged values
