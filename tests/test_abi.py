"""The C ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments before touching the GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "skv.h")

skv = pytest.importorskip("streaming_kv_cache_amd")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 13, names
    lib = ctypes.CDLL(skv._LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in skv.h but not exported"
    assert set(names) == set(skv.EXPORTED)


def test_version_and_strings():
    assert skv.lib.skv_abi_version() == 5
    for code in range(7):
        assert skv.status_string(code)
    assert skv.status_string(99) == "unknown status"


ABOT = skv.Config(24, 128, 22, 40, 3, 5, 21, rope_mode=skv.ROPE_REL)
LB480 = skv.Config(40, 128, 30, 52, 4, 6, 18)


def test_cache_bytes():
    # workspace = REL window keys [(W-c)*F, H, D] + current-chunk V^T [H, D, c*F rounded up to 64]
    def pad64(n):
        return (n + 63) // 64 * 64
    # one size serves both stores: the V store's V^T, W*F keys per head padded to 64-key tiles
    store, ws = skv.cache_bytes(ABOT)
    assert store == pad64(21 * 880) * 24 * 128 * 2
    assert ws == (21 - 3) * 880 * 24 * 128 * 2 + 24 * 128 * pad64(3 * 880) * 2
    store, ws = skv.cache_bytes(LB480)
    assert store == pad64(18 * 1560) * 40 * 128 * 2 and ws == 40 * 128 * pad64(4 * 1560) * 2
    tiny = skv.Config(2, 64, 4, 4, 2, 1, 4, dtype=skv.F32)
    assert skv.cache_bytes(tiny) == (4 * 16 * 2 * 64 * 4, 2 * 64 * 64 * 4)
    # 3 heads of 480P: 49 query tiles x 3 heads = 147 four-wave workgroups fill less than half of
    # the 512 slots, so the workspace also holds floor(512 / 147) = 3 key splits of fp32 partials
    lb_h3 = skv.Config(3, 128, 30, 52, 4, 6, 18)
    base = 3 * 128 * pad64(4 * 1560) * 2
    store, ws = skv.cache_bytes(lb_h3)
    assert ws == (base + 255) // 256 * 256 + 3 * 4 * 1560 * 3 * (128 + 2) * 4
    # small grids: at most 16 splits
    small = skv.Config(3, 128, 5, 13, 3, 2, 9, rope_mode=skv.ROPE_REL)
    base = (9 - 3) * 65 * 3 * 128 * 2 + 3 * 128 * pad64(3 * 65) * 2
    assert skv.cache_bytes(small)[1] == (base + 255) // 256 * 256 + 16 * 3 * 65 * 3 * (128 + 2) * 4


@pytest.mark.parametrize("bad", [
    dict(heads=0), dict(head_dim=96), dict(head_dim=32), dict(grid_h=0), dict(chunk_frames=0),
    dict(sink_frames=-1), dict(window_frames=7), dict(rope_split=(40, 40, 40)), dict(rope_split=(43, 43, 42)),
    dict(rope_theta=-1.0), dict(dtype=7), dict(rope_mode=3),
])
def test_bad_configs(bad):
    base = dict(heads=2, head_dim=128, grid_h=3, grid_w=3, chunk_frames=2, sink_frames=2, window_frames=8)
    base.update({k: v for k, v in bad.items() if k in base})
    cfg = skv.Config(**base, **{k: v for k, v in bad.items() if k not in base})
    if bad == dict(window_frames=7):
        cfg = skv.Config(2, 128, 3, 3, 4, 4, 7)
    with pytest.raises(skv.SkvError) as e:
        skv.cache_bytes(cfg)
    assert e.value.status == skv.ERR_CONFIG


def _init(cfg, k=0x10000, v=0x20000, ws=0x30000):
    h = ctypes.c_void_p()
    c = cfg.c_struct()
    st = skv.lib.kv_cache_init(ctypes.byref(c), ctypes.c_void_p(k), ctypes.c_void_p(v), ctypes.c_void_p(ws),
                               ctypes.byref(h))
    return st, h


def test_init_validation_and_info():
    # the handle records pointers only; fake aligned addresses never reach the GPU here
    assert _init(LB480, k=0)[0] == skv.ERR_NULL
    assert _init(LB480, k=0x10008)[0] == skv.ERR_ALIGN
    assert _init(ABOT, ws=0)[0] == skv.ERR_NULL
    st, h = _init(ABOT)
    assert st == skv.OK
    info = skv.KvCacheInfo()
    assert skv.lib.kv_cache_info(h, ctypes.byref(info)) == skv.OK
    assert (info.n_appended, info.n_cached, info.n_vis, info.ring_start, info.poisoned) == (0, 0, 3, -1, 0)
    nul = ctypes.c_void_p(0)
    p = ctypes.c_void_p(0x40000)
    # argument checks that return before anything is enqueued
    assert skv.lib.kv_cache_append_evict(h, p, p, 0, nul) == skv.ERR_SHAPE
    assert skv.lib.kv_cache_append_evict(h, p, p, 17, nul) == skv.ERR_SHAPE
    assert skv.lib.kv_cache_append_evict(h, nul, p, 3, nul) == skv.ERR_NULL
    assert skv.lib.kv_cache_append_evict(h, ctypes.c_void_p(0x40004), p, 3, nul) == skv.ERR_ALIGN
    assert skv.lib.rope_apply(h, p, p, 2, 0, nul) == skv.ERR_SHAPE          # rel: n_frames must equal c
    assert skv.lib.chunk_attention(h, p, p, p, 2, p, nul) == skv.ERR_SHAPE
    assert skv.lib.chunk_attention(h, nul, p, p, 3, p, nul) == skv.ERR_NULL
    assert skv.lib.chunk_attention(h, p, p, nul, 3, p, nul) == skv.ERR_STATE   # nothing staged yet
    assert skv.lib.kv_cache_stage_v(h, nul, 3, nul) == skv.ERR_NULL
    assert skv.lib.kv_cache_stage_v(h, p, 2, nul) == skv.ERR_SHAPE
    assert skv.lib.kv_cache_gather(h, nul, p, None, nul) == skv.ERR_NULL
    assert skv.lib.kv_cache_reset(h) == skv.OK
    assert skv.lib.kv_cache_destroy(h) == skv.OK
    assert skv.lib.kv_cache_destroy(nul) == skv.OK
    st, h = _init(LB480)
    assert skv.lib.rope_apply_window(h, nul) == skv.ERR_STATE              # abs mode has no window
    assert skv.lib.rope_apply(h, p, p, 4, -1, nul) == skv.ERR_SHAPE         # abs: start_frame >= 0
    qk = skv.lib.rope_apply_qk
    assert qk(h, p, p, p, p, 4, -1, nul) == skv.ERR_SHAPE
    assert qk(h, p, p, nul, p, 4, 0, nul) == skv.ERR_NULL
    assert qk(h, p, p, p, nul, 4, 0, nul) == skv.ERR_NULL
    assert qk(h, p, ctypes.c_void_p(0x40008), p, p, 4, 0, nul) == skv.ERR_ALIGN
    assert qk(h, p, p, p, p, 0, 0, nul) == skv.ERR_SHAPE
    pp = skv.lib.kv_cache_prepare_pass  # rope_apply_qk's checks, then v_cur's, and n_frames == c
    assert pp(h, p, p, p, p, p, 4, -1, nul) == skv.ERR_SHAPE
    assert pp(h, p, p, nul, p, p, 4, 0, nul) == skv.ERR_NULL
    assert pp(h, p, p, p, p, nul, 4, 0, nul) == skv.ERR_NULL
    assert pp(h, p, p, p, p, ctypes.c_void_p(0x40008), 4, 0, nul) == skv.ERR_ALIGN
    assert pp(h, p, p, p, p, p, 3, 0, nul) == skv.ERR_SHAPE                   # abs too: staging needs c frames
    assert pp(nul, p, p, p, p, p, 4, 0, nul) == skv.ERR_NULL
    skv.lib.kv_cache_destroy(h)
    st, h = _init(ABOT)
    assert skv.lib.rope_apply_qk(h, p, p, p, p, 2, 0, nul) == skv.ERR_SHAPE   # rel: n_frames must equal c
    assert skv.lib.kv_cache_prepare_pass(h, p, p, p, p, p, 2, 0, nul) == skv.ERR_SHAPE
    skv.lib.kv_cache_destroy(h)


def test_cross_attention_validation():
    p, nul = ctypes.c_void_p(0x40000), ctypes.c_void_p(0)
    f = skv.lib.cross_attention
    assert f(nul, 8, p, p, 512, 40, 128, skv.BF16, p, nul) == skv.ERR_NULL
    assert f(p, 8, p, p, 512, 40, 96, skv.BF16, p, nul) == skv.ERR_CONFIG
    assert f(p, 8, p, p, 0, 40, 128, skv.BF16, p, nul) == skv.ERR_SHAPE
    assert f(p, 0, p, p, 512, 40, 128, skv.BF16, p, nul) == skv.ERR_SHAPE
    assert f(p, 8, p, p, 512, 0, 128, skv.BF16, p, nul) == skv.ERR_CONFIG


def test_text_cache_sizes_and_validation():
    """Store size formula, and every error path of the prepared text cache returns before anything is
    enqueued (no GPU needed)."""
    # bf16: K head-major and V^T, each over the keys padded to a multiple of 64, V^T at a 256-byte boundary
    assert skv.text_cache_bytes(512, 40, 128, skv.BF16) == 2 * 512 * 40 * 128 * 2
    assert skv.text_cache_bytes(77, 3, 64, skv.BF16) == 3 * 128 * 64 * 2 + 3 * 64 * 128 * 2
    assert skv.text_cache_bytes(77, 3, 64, skv.F32) == (77 * 3 * 64 * 4 + 255) // 256 * 256 + 77 * 3 * 64 * 4
    b = ctypes.c_size_t()
    f = skv.lib.text_cache_bytes
    assert f(512, 40, 128, skv.BF16, None) == skv.ERR_NULL
    assert f(512, 40, 96, skv.BF16, ctypes.byref(b)) == skv.ERR_CONFIG       # bf16 D in {64, 128}
    assert f(512, 40, 32, skv.F32, ctypes.byref(b)) == skv.OK
    assert f(0, 40, 128, skv.BF16, ctypes.byref(b)) == skv.ERR_SHAPE
    assert f(512, 0, 128, skv.BF16, ctypes.byref(b)) == skv.ERR_CONFIG
    assert f((1 << 23) + 1, 40, 128, skv.BF16, ctypes.byref(b)) == skv.ERR_SHAPE   # past 32-bit offsets per head
    p, p16, nul = ctypes.c_void_p(0x40000), ctypes.c_void_p(0x40010), ctypes.c_void_p(0)
    g = skv.lib.text_cache_prepare
    assert g(nul, p, 512, 40, 128, skv.BF16, p, nul) == skv.ERR_NULL
    assert g(p, p, 512, 40, 128, skv.BF16, nul, nul) == skv.ERR_NULL
    assert g(p, p, 512, 40, 128, skv.BF16, p16, nul) == skv.ERR_ALIGN        # store: 256-byte aligned
    assert g(p, p16, 512, 40, 96, skv.BF16, p, nul) == skv.ERR_CONFIG
    assert g(p, p, 0, 40, 128, skv.BF16, p, nul) == skv.ERR_SHAPE
    h = skv.lib.cross_attention_cached
    assert h(nul, 8, p, 512, 40, 128, skv.BF16, p, nul) == skv.ERR_NULL
    assert h(p, 8, nul, 512, 40, 128, skv.BF16, p, nul) == skv.ERR_NULL
    assert h(p, 8, p16, 512, 40, 128, skv.BF16, p, nul) == skv.ERR_ALIGN
    assert h(p, 0, p, 512, 40, 128, skv.BF16, p, nul) == skv.ERR_SHAPE
    assert h(p, 8, p, 512, 40, 128, 7, p, nul) == skv.ERR_CONFIG


def test_sampler_step_validation():
    """Every error path of sampler_step returns before anything is enqueued (no GPU needed)."""
    p, q, nul = ctypes.c_void_p(0x40000), ctypes.c_void_p(0x50000), ctypes.c_void_p(0)
    f = skv.lib.sampler_step
    ok = (p, p, nul, 1.0, p, 1024, 0.75, 0.5, skv.BF16, q, q, nul)

    def call(**kw):
        a = list(ok)
        names = ["x_t", "v_cond", "v_uncond", "cfg", "noise", "n", "sigma", "sigma_next", "dtype", "x0", "xn", "s"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(x_t=nul) == skv.ERR_NULL
    assert call(v_cond=nul) == skv.ERR_NULL
    assert call(x0=nul, xn=nul) == skv.ERR_NULL
    assert call(noise=nul) == skv.ERR_NULL                      # re-noised output without noise
    assert call(x_t=ctypes.c_void_p(0x40008)) == skv.ERR_ALIGN
    assert call(v_uncond=ctypes.c_void_p(0x40004)) == skv.ERR_ALIGN
    assert call(xn=ctypes.c_void_p(0x50002)) == skv.ERR_ALIGN
    assert call(dtype=7) == skv.ERR_CONFIG
    assert call(sigma=float("nan")) == skv.ERR_CONFIG
    assert call(cfg=float("inf")) == skv.ERR_CONFIG
    assert call(n=-1) == skv.ERR_SHAPE
    assert call(n=0) == skv.OK                                   # nothing to do, nothing enqueued


def test_chunk_attention_batch_validation():
    """Batch checks return before anything is enqueued (fake aligned device addresses, no GPU)."""
    V = ctypes.c_void_p
    p, nul = V(0x40000), V(0)
    st, h1 = _init(LB480)
    st2, h2 = _init(LB480, k=0x50000, v=0x60000, ws=0x70000)
    st3, h3 = _init(skv.Config(40, 128, 30, 52, 4, 6, 20), k=0x80000, v=0x90000, ws=0xA0000)
    assert st == st2 == st3 == skv.OK
    f = skv.lib.chunk_attention_batch

    def arr(*xs):
        return (V * len(xs))(*[x.value for x in xs])

    two = arr(p, p)
    assert f(None, 2, two, two, two, 4, two, nul) == skv.ERR_NULL
    assert f(arr(h1, h2), 0, two, two, two, 4, two, nul) == skv.ERR_SHAPE
    five = arr(h1, h2, h1, h2, h1)
    assert f(five, 5, five, five, five, 4, five, nul) == skv.ERR_SHAPE
    assert f(arr(h1, nul), 2, two, two, two, 4, two, nul) == skv.ERR_NULL
    assert f(arr(h1, h1), 2, two, two, two, 4, two, nul) == skv.ERR_STATE       # one handle twice
    assert f(arr(h1, h3), 2, two, two, two, 4, two, nul) == skv.ERR_CONFIG      # different windows
    assert f(arr(h1, h2), 2, two, two, None, 4, two, nul) == skv.ERR_STATE      # nothing staged
    assert f(arr(h1, h2), 2, two, arr(p, nul), two, 4, two, nul) == skv.ERR_NULL
    assert f(arr(h1, h2), 2, two, two, two, 3, two, nul) == skv.ERR_SHAPE
    for h in (h1, h2, h3):
        skv.lib.kv_cache_destroy(h)


def test_block_causal_validation():
    """Size query and argument checks of block_causal_attention (no GPU work reaches a launch)."""
    V = ctypes.c_void_p
    p, nul = V(0x40000), V(0)
    c = LB480.c_struct()
    b = ctypes.c_size_t()
    assert skv.lib.block_causal_workspace_bytes(ctypes.byref(c), 88, ctypes.byref(b)) == skv.OK
    assert b.value == 40 * 128 * ((88 * 1560 + 63) // 64 * 64) * 2
    assert skv.lib.block_causal_workspace_bytes(ctypes.byref(c), 0, ctypes.byref(b)) == skv.ERR_SHAPE
    assert skv.lib.block_causal_workspace_bytes(ctypes.byref(c), 88, None) == skv.ERR_NULL
    f = skv.lib.block_causal_attention
    assert f(ctypes.byref(c), nul, p, p, 88, 0, p, p, nul) == skv.ERR_NULL
    assert f(ctypes.byref(c), p, p, p, 88, 0, V(0x40008), p, nul) == skv.ERR_ALIGN
    assert f(ctypes.byref(c), p, p, p, 87, 0, p, p, nul) == skv.ERR_SHAPE        # not whole chunks
    assert f(ctypes.byref(c), p, p, p, 88, 88, p, p, nul) == skv.ERR_SHAPE       # no query frames
    assert f(ctypes.byref(c), p, p, p, 88, -1, p, p, nul) == skv.ERR_SHAPE
    assert f(ctypes.byref(c), p, p, p, 2000, 0, p, p, nul) == skv.ERR_SHAPE      # past 32-bit head offsets
    f32 = skv.Config(2, 64, 4, 4, 2, 1, 4, skv.ROPE_ABS, skv.F32).c_struct()
    assert f(ctypes.byref(f32), p, p, p, 8, 0, p, p, nul) == skv.ERR_CONFIG      # bf16 only
    ab = ABOT.c_struct()
    assert skv.lib.block_causal_workspace_bytes(ctypes.byref(ab), 5 + 3 * 7, ctypes.byref(b)) == skv.OK


def test_fused_rope_config():
    """fused_rope: 0/1 only; the workspace holds the rotated chunk copies instead of the REL window;
    the window call and the separate pass preparation are not used."""
    import dataclasses
    bad = dataclasses.replace(ABOT, fused_rope=True).c_struct()
    bad.fused_rope = 2
    s, w = ctypes.c_size_t(), ctypes.c_size_t()
    assert skv.lib.kv_cache_bytes(ctypes.byref(bad), ctypes.byref(s), ctypes.byref(w)) == skv.ERR_CONFIG
    lq_elems = 3 * 880 * 24 * 128
    vt = 24 * 128 * ((3 * 880 + 63) // 64 * 64)
    assert skv.cache_bytes(dataclasses.replace(ABOT, fused_rope=True))[1] == (3 * lq_elems + vt) * 2
    assert skv.cache_bytes(dataclasses.replace(LB480, fused_rope=True))[1] == \
        (2 * 4 * 1560 * 40 * 128 + 40 * 128 * ((4 * 1560 + 63) // 64 * 64)) * 2
    st, h = _init(dataclasses.replace(ABOT, fused_rope=True))
    assert st == skv.OK
    assert skv.lib.rope_apply_window(h, ctypes.c_void_p(0)) == skv.ERR_STATE
    p = ctypes.c_void_p(0x40000)
    # chunk_attention rotates and stages by itself under fused rotation
    assert skv.lib.kv_cache_prepare_pass(h, p, p, p, p, p, 3, 0, ctypes.c_void_p(0)) == skv.ERR_STATE
    skv.lib.kv_cache_destroy(h)
