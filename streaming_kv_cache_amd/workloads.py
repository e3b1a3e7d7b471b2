"""Named workloads: the shapes of the pages' two systems plus small test shapes.

Shapes follow the pages: [ABot-stream] 机制一/二/三 (21-frame window of 880
tokens, 3-frame blocks, 5 reference sinks, relative RoPE, 30 blocks, 512 text
tokens) and [LB-causal] / [LB-fast] (18-frame window with 6 sinks, chunks of 4,
about 1560 tokens per frame at 480P, absolute RoPE with start_frame, 40 heads
of 128 in a 5120-wide model, 22 chunks for 361 frames).  Small shapes exercise
several tiles and ragged tails at sizes the CPU oracle finishes in seconds.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import BF16, F32, ROPE_ABS, ROPE_REL, Config


@dataclass(frozen=True)
class Workload:
    name: str
    cfg: Config
    n_chunks: int
    prefill: int = 0        # frames appended before chunk 0 (reference sinks)
    passes: int = 5         # 4 denoise passes + 1 clean write-back pass per chunk
    text_tokens: int = 0    # cross-attention keys (0: none)
    layers: int = 1
    steady_chunk: int = 0   # first chunk whose visible set is the full window
    # timesteps (of 1000 training steps) of the denoise passes; the sampler runs after each
    # of them with sigma = t / 1000 (the write-back pass runs at t = 0 and is not sampled)
    timesteps: tuple = ()

    @property
    def lq(self) -> int:
        return self.cfg.chunk_frames * self.cfg.tokens_per_frame

    @property
    def steady_lkv(self) -> int:
        return self.cfg.window_frames * self.cfg.tokens_per_frame


# [ABot-stream] 机制二: denoising_step_list.  [LB-fast] 2. 4 步采样: indices 0, 179, 358, 679 into the
# 1000-step training table, read as the descending table 1000, 999, ..., 1.
ABOT_STEPS = (1000, 750, 500, 250)
LINGBOT_STEPS = tuple(1000 - i for i in (0, 179, 358, 679))

WORKLOADS = {
    # the small fp32 case: 2 heads x 64, 4x4 tokens, chunk 2, sink 1, window 4, absolute RoPE, 8 chunks
    "tiny": Workload("tiny", Config(2, 64, 4, 4, 2, 1, 4, ROPE_ABS, F32), n_chunks=8, steady_chunk=1),
    # ABot-like 720P: 24 heads x 128, 22x40 tokens, chunk 3, window 21 incl. 5 reference sinks, relative RoPE
    "abot720": Workload("abot720", Config(24, 128, 22, 40, 3, 5, 21, ROPE_REL, BF16), n_chunks=40,
                        prefill=5, steady_chunk=5, timesteps=ABOT_STEPS),
    # LingBot-like 480P: 40 heads x 128, 30x52 tokens, chunk 4, window 18 incl. sink 6, absolute RoPE
    "lb480": Workload("lb480", Config(40, 128, 30, 52, 4, 6, 18, ROPE_ABS, BF16), n_chunks=22, steady_chunk=4,
                      timesteps=LINGBOT_STEPS),
    # LingBot-like 720P: 40 heads x 128, 45x80 tokens
    "lb720": Workload("lb720", Config(40, 128, 45, 80, 4, 6, 18, ROPE_ABS, BF16), n_chunks=8, steady_chunk=4,
                      timesteps=LINGBOT_STEPS),
    # 40 layers of the 480P layer, cross attention to 512 cached text tokens, 300 chunks
    "fulldepth480": Workload("fulldepth480", Config(40, 128, 30, 52, 4, 6, 18, ROPE_ABS, BF16), n_chunks=300,
                             text_tokens=512, layers=40, steady_chunk=4, timesteps=LINGBOT_STEPS),
    # one GPU's share of a model sharded by heads over 8 GPUs (ABot 24 / 8 = 3 heads, LingBot 40 / 8 = 5):
    # the real per-GPU shape, whose attention grid alone leaves most of the chip idle
    "abot720_h3": Workload("abot720_h3", Config(3, 128, 22, 40, 3, 5, 21, ROPE_REL, BF16), n_chunks=40,
                           prefill=5, steady_chunk=5, timesteps=ABOT_STEPS),
    "lb480_h5": Workload("lb480_h5", Config(5, 128, 30, 52, 4, 6, 18, ROPE_ABS, BF16), n_chunks=22,
                         steady_chunk=4, timesteps=LINGBOT_STEPS),
    # small shapes: several 64-key tiles, ragged frame sizes, ring wrap-around
    "small_abs": Workload("small_abs", Config(3, 128, 7, 9, 2, 2, 7, ROPE_ABS, BF16), n_chunks=12, steady_chunk=3),
    "small_rel": Workload("small_rel", Config(3, 128, 5, 13, 3, 2, 9, ROPE_REL, BF16), n_chunks=10, prefill=2,
                          steady_chunk=2),
    "small_d64": Workload("small_d64", Config(2, 64, 6, 11, 2, 1, 6, ROPE_ABS, BF16), n_chunks=10, steady_chunk=2),
    "small_f32_rel": Workload("small_f32_rel", Config(2, 128, 3, 5, 2, 1, 5, ROPE_REL, F32), n_chunks=8,
                              steady_chunk=2),
    "small_nosink": Workload("small_nosink", Config(2, 128, 4, 9, 2, 0, 5, ROPE_ABS, BF16), n_chunks=9,
                             steady_chunk=2),
}
