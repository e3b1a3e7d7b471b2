"""block_causal_attention_noalloc (workspace in the library's static device array) against
block_causal_attention (caller's workspace) through the C ABI: the same kernels, so the outputs
must be bit-identical; two calls in a row, the second on a smaller input, and a size past the
static array's limit refused before anything is enqueued."""
import sys

import pytest
import torch

import seeded_inputs as si

skv = pytest.importorskip("streaming_kv_cache_amd")

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _inputs(cfg, n_frames, q_frame0, base):
    f = cfg.tokens_per_frame
    k = si.draw((n_frames * f, cfg.heads, cfg.head_dim), base, 0, 0, si.K, cfg.torch_dtype).cuda()
    v = si.draw((n_frames * f, cfg.heads, cfg.head_dim), base, 0, 0, si.V, cfg.torch_dtype).cuda()
    q = si.draw(((n_frames - q_frame0) * f, cfg.heads, cfg.head_dim), base, 0, 0, si.Q, cfg.torch_dtype).cuda()
    return q, k, v


def test_noalloc_matches_workspace_call():
    # ABot-like 720P layer (24 heads, 880 tokens per frame, chunks of 3, 5 reference sinks, window 21):
    # 5 + 2 chunks -> V^T of 11 frames = 59.8 MB of the 64 MiB array; then a small shape
    abot = skv.Config(24, 128, 22, 40, 3, 5, 21, skv.ROPE_ABS, skv.BF16)
    small = skv.Config(3, 128, 5, 13, 3, 2, 9, skv.ROPE_ABS, skv.BF16)
    cases = [(abot, 11, 5, 0), (small, 8, 2, 1)]
    for cfg, n, q0, base in cases:
        need = skv.block_causal_workspace_bytes(cfg, n)
        assert need <= skv.NOALLOC_SCRATCH_BYTES
        say(f"[noalloc] H={cfg.heads} F={cfg.tokens_per_frame} frames={n} q_frame0={q0}: {need / 2**20:.1f} MiB")
        q, k, v = _inputs(cfg, n, q0, base)
        out_ref = skv.block_causal_attention(cfg, q, k, v, q_frame0=q0)
        out = torch.full_like(q, float("nan"))
        skv.block_causal_attention_noalloc(cfg, q, k, v, out, q_frame0=q0)
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref)
    # past the limit: refused on the host, nothing enqueued, the output untouched
    n = 14
    assert skv.block_causal_workspace_bytes(abot, n) > skv.NOALLOC_SCRATCH_BYTES
    q, k, v = _inputs(abot, n, 5, 2)
    out = torch.zeros_like(q)
    with pytest.raises(skv.SkvError) as e:
        skv.block_causal_attention_noalloc(abot, q, k, v, out, q_frame0=5)
    assert e.value.status == skv.ERR_SHAPE
    torch.cuda.synchronize()
    assert not out.any()
