"""The library's calls enqueue kernels only (no allocation, no memset, no host synchronisation), so a
pass can be captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.  Each replay, with eager
work and synchronisation in between, must give the eager result bit for bit."""
import pytest
import torch

import seeded_inputs as si
import streaming_kv_cache_amd as skv
from streaming_kv_cache_amd.workloads import WORKLOADS
from tests import rollout as ro

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("split", ["0", "auto"])
@pytest.mark.parametrize("name", ["small_abs", "small_rel"])
def test_pass_capture_replay(name, split, monkeypatch):
    if split == "0":
        monkeypatch.setenv("SKV_ATTN_SPLIT", "0")
    else:
        monkeypatch.delenv("SKV_ATTN_SPLIT", raising=False)
    wl = WORKLOADS[name]
    c = wl.cfg
    say(f"[graph] {name} split={split}")
    cache = skv.KVCache(c)
    ro.prefill(wl, cache, None)
    for ch in range(3):
        k = ro.draw(wl, c.chunk_frames, ch, 4, si.K).cuda()
        k = k if c.rope_mode == skv.ROPE_REL else cache.rope_apply(k, start_frame=cache.info().n_appended)
        cache.append_evict(k, ro.draw(wl, c.chunk_frames, ch, 4, si.V).cuda())
    if c.rope_mode == skv.ROPE_REL:
        cache.rope_apply_window()
    t = cache.info().n_appended
    q, k, v = (ro.draw(wl, c.chunk_frames, 3, 0, tid).cuda() for tid in (si.Q, si.K, si.V))
    qr, kr = torch.empty_like(q), torch.empty_like(k)
    out_g = torch.empty_like(q)

    def one_pass(out):
        cache.rope_apply_qk(q, k, q_out=qr, k_out=kr, start_frame=t)
        cache.stage_v(v)
        cache.chunk_attention(qr, kr, None, out=out)

    eager = torch.empty_like(q)
    one_pass(eager)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one_pass(out_g)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one_pass(out_g)
    scratch = torch.zeros(1 << 20, device="cuda")
    for r in range(3):
        out_g.zero_()
        g.replay()
        scratch.add_(1.0)          # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out_g, eager), f"replay {r} differs from the eager pass"
