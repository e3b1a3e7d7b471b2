"""The failure path of the C ABI on the CPU: a launch that fails poisons its handle until
kv_cache_reset, and kv_cache_restore checks the frame ids of a snapshot.

The library's test hook (skv_debug_fail_launches) makes the next launches report a HIP failure
without launching anything, so no GPU is involved: the handles here point at fake, aligned device
addresses that are never dereferenced.
"""
import ctypes

import pytest

skv = pytest.importorskip("streaming_kv_cache_amd")

NUL = ctypes.c_void_p(0)
P = ctypes.c_void_p(0x40000)
ABOT = skv.Config(24, 128, 22, 40, 3, 5, 21, rope_mode=skv.ROPE_REL)
LB480 = skv.Config(40, 128, 30, 52, 4, 6, 18)


def _handle(cfg):
    h = ctypes.c_void_p()
    c = cfg.c_struct()
    assert skv.lib.kv_cache_init(ctypes.byref(c), ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000),
                                 ctypes.c_void_p(0x30000), ctypes.byref(h)) == skv.OK
    return h


def _info(h):
    i = skv.KvCacheInfo()
    assert skv.lib.kv_cache_info(h, ctypes.byref(i)) == skv.OK
    return i


@pytest.fixture(autouse=True)
def _disarm():
    skv.debug_fail_launches(0)
    yield
    skv.debug_fail_launches(0)


def _ids(values):
    return (ctypes.c_int64 * max(len(values), 1))(*values)


def test_failed_launch_poisons_until_reset():
    h = _handle(LB480)
    skv.debug_fail_launches(1)
    # a validation error comes first and leaves the armed failure for the next launch
    assert skv.lib.kv_cache_append_evict(h, P, P, 0, NUL) == skv.ERR_SHAPE
    assert _info(h).poisoned == 0
    assert skv.lib.kv_cache_append_evict(h, P, P, 4, NUL) == skv.ERR_HIP
    i = _info(h)
    assert i.poisoned == 1 and i.n_appended == 0     # the failed append did not advance the ring
    # every call on the poisoned handle is refused before anything is enqueued
    assert skv.lib.kv_cache_append_evict(h, P, P, 4, NUL) == skv.ERR_STATE
    assert skv.lib.rope_apply(h, P, P, 4, 0, NUL) == skv.ERR_STATE
    assert skv.lib.rope_apply_qk(h, P, P, P, P, 4, 0, NUL) == skv.ERR_STATE
    assert skv.lib.kv_cache_prepare_pass(h, P, P, P, P, P, 4, 0, NUL) == skv.ERR_STATE
    assert skv.lib.kv_cache_stage_v(h, P, 4, NUL) == skv.ERR_STATE
    assert skv.lib.chunk_attention(h, P, P, P, 4, P, NUL) == skv.ERR_STATE
    assert skv.lib.kv_cache_gather(h, P, P, None, NUL) == skv.ERR_STATE
    assert skv.lib.kv_cache_restore(h, P, P, _ids([]), 0, NUL) == skv.ERR_STATE
    arr = (ctypes.c_void_p * 1)(h.value)
    assert skv.lib.chunk_attention_batch(arr, 1, (ctypes.c_void_p * 1)(P.value), (ctypes.c_void_p * 1)(P.value),
                                         None, 4, (ctypes.c_void_p * 1)(P.value), NUL) == skv.ERR_STATE
    # reset recovers the handle: counters to zero, not poisoned
    assert skv.lib.kv_cache_reset(h) == skv.OK
    i = _info(h)
    assert (i.poisoned, i.n_appended, i.n_cached) == (0, 0, 0)
    assert skv.lib.kv_cache_destroy(h) == skv.OK


def test_rel_window_and_attention_launch_failures_poison():
    h = _handle(ABOT)
    # a snapshot of 8 frames (5 sinks + frames 5..7): its write fails -> poisoned, nothing restored
    skv.debug_fail_launches(1)
    assert skv.lib.kv_cache_restore(h, P, P, _ids(list(range(8))), 8, NUL) == skv.ERR_HIP
    assert _info(h).poisoned == 1 and _info(h).n_appended == 0
    assert skv.lib.kv_cache_reset(h) == skv.OK
    # an empty snapshot needs no launch: an empty cache
    assert skv.lib.kv_cache_restore(h, NUL, NUL, _ids([]), 0, NUL) == skv.OK
    # with no history there is nothing to rotate: the window pass launches nothing
    assert skv.lib.rope_apply_window(h, NUL) == skv.OK and _info(h).window_ready == 1
    # the chunk's own rotation fails -> poisoned
    skv.debug_fail_launches(1)
    assert skv.lib.rope_apply(h, P, P, 3, 0, NUL) == skv.ERR_HIP
    assert _info(h).poisoned == 1
    assert skv.lib.kv_cache_reset(h) == skv.OK
    # attention with v given: the staging launch fails -> poisoned
    skv.debug_fail_launches(1)
    assert skv.lib.chunk_attention(h, P, P, P, 3, P, NUL) == skv.ERR_HIP
    assert _info(h).poisoned == 1
    assert skv.lib.kv_cache_reset(h) == skv.OK
    assert _info(h).poisoned == 0
    assert skv.lib.kv_cache_destroy(h) == skv.OK


def test_handle_free_calls_report_failure():
    skv.debug_fail_launches(3)
    assert skv.lib.cross_attention(P, 64, P, P, 16, 2, 128, skv.BF16, P, NUL) == skv.ERR_HIP
    assert skv.lib.sampler_step(P, P, None, 1.0, None, 64, 0.5, 0.0, skv.BF16, P, None, NUL) == skv.ERR_HIP
    store = ctypes.c_void_p(0x100000)
    assert skv.lib.cross_attention_cached(P, 64, store, 16, 2, 128, skv.BF16, P, NUL) == skv.ERR_HIP
    # disarmed: validation errors are unchanged
    skv.debug_fail_launches(0)
    assert skv.lib.cross_attention(NUL, 64, P, P, 16, 2, 128, skv.BF16, P, NUL) == skv.ERR_NULL


def test_restore_checks_the_snapshot_ids():
    """kv_cache_restore accepts exactly the ids kv_cache_gather reports for T = last id + 1: the S
    sinks 0..S-1, then the most recent min(T - S, W - S) frames."""
    h = _handle(LB480)   # S = 6, W = 18: ring of 12 slots
    r = skv.lib.kv_cache_restore
    assert r(h, P, P, _ids([0, 1, 2]), -1, NUL) == skv.ERR_SHAPE
    assert r(h, P, P, None, 3, NUL) == skv.ERR_NULL
    assert r(h, NUL, P, _ids([0, 1, 2]), 3, NUL) == skv.ERR_NULL
    assert r(h, ctypes.c_void_p(0x40008), P, _ids([0, 1, 2]), 3, NUL) == skv.ERR_ALIGN
    assert r(h, P, P, _ids([1, 2, 3]), 3, NUL) == skv.ERR_SHAPE                 # sinks must start at 0
    assert r(h, P, P, _ids([0, 1, 3]), 3, NUL) == skv.ERR_SHAPE                 # a gap
    assert r(h, P, P, _ids(list(range(6)) + [7]), 7, NUL) == skv.ERR_SHAPE     # frame 6 is still cached
    full = list(range(6)) + list(range(100, 112))
    assert r(h, P, P, _ids(full[:-1]), 17, NUL) == skv.ERR_SHAPE               # a full ring holds 12 frames
    assert r(h, P, P, _ids(full[:6] + full[7:]), 17, NUL) == skv.ERR_SHAPE
    assert _info(h).poisoned == 0 and _info(h).n_appended == 0                  # nothing changed
    # a valid snapshot reaches the (failing) launch, which then counts as a failed write
    skv.debug_fail_launches(1)
    assert r(h, P, P, _ids(full), 18, NUL) == skv.ERR_HIP
    assert skv.lib.kv_cache_reset(h) == skv.OK
    assert skv.lib.kv_cache_destroy(h) == skv.OK
