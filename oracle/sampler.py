"""Plain float64 CPU oracle of the few-step sampler between attention passes.

TEST INFRASTRUCTURE ONLY: imported by ``tests/`` and nothing in the product path.

Pages (short names as in ``skv_oracle``):

* [LB-fast]     "从40步到4步：LingBot-World 2.0实时推理蒸馏（causal_fast）原理与关键代码解读",
                section "2. 4 步采样" (four timestep indices out of 1000 training steps; per
                step: one forward gives a flow-matching velocity, x0 is recovered in one
                analytic step from x_t, sigma_t and the velocity, then re-noised to the next,
                smaller timestep unless it was the last one) and the "精度" remark of the
                engineering-details section (the flow -> x0 conversion runs in double);
                the table at the top (causal_pretrain: 40 steps with CFG scale 5.0).
* [ABot-stream] "ABot-World流式因果推理深度解析", 机制二 (denoising_step_list
                [1000, 750, 500, 250]; clean write-back at timestep 0, context_noise 0).

Readings where the pages are silent (each also listed in the design notes):

* sigma of a timestep t out of ``num_train`` training steps is ``t / num_train`` (a plain
  linear flow-matching schedule; no shift is given on the pages);
* the 1000-entry training timestep table that [LB-fast]'s indices point into is
  ``T[i] = num_train - i`` (descending, step 1), so index 0 is the noisiest step;
* re-noising to sigma' is the flow-matching forward interpolation
  ``x' = (1 - sigma') x0 + sigma' eps`` with fresh noise eps; it is the process under which
  ``x0 = x_t - sigma_t v`` is exact for the velocity ``v = eps - x0``;
* classifier-free guidance combines two velocity predictions as
  ``v = v_uncond + scale (v_cond - v_uncond)``.
"""
from __future__ import annotations

from typing import Callable, List, Optional, Sequence

import numpy as np

NUM_TRAIN_TIMESTEPS = 1000


def sigma_of(t: float, num_train: int = NUM_TRAIN_TIMESTEPS) -> float:
    """Noise level of timestep t (reading: linear schedule, sigma = t / num_train)."""
    return float(t) / float(num_train)


def timesteps_from_indices(indices: Sequence[int], num_train: int = NUM_TRAIN_TIMESTEPS) -> List[int]:
    """[LB-fast] 2. 4 步采样: the sampled timesteps are entries of the training timestep table.

    Reading: the table is num_train, num_train - 1, ..., 1 (descending).
    """
    out = []
    for i in indices:
        if not 0 <= int(i) < num_train:
            raise ValueError("timestep index out of range")
        out.append(num_train - int(i))
    return out


def flow_to_x0(x_t: np.ndarray, v: np.ndarray, sigma: float) -> np.ndarray:
    """[LB-fast] 2. 4 步采样: x0 = x_t - sigma_t * (velocity prediction), in float64."""
    return np.asarray(x_t, np.float64) - float(sigma) * np.asarray(v, np.float64)


def renoise(x0: np.ndarray, noise: np.ndarray, sigma_next: float) -> np.ndarray:
    """Re-noise a clean estimate to the next timestep (reading: flow-matching interpolation)."""
    s = float(sigma_next)
    return (1.0 - s) * np.asarray(x0, np.float64) + s * np.asarray(noise, np.float64)


def cfg_combine(v_cond: np.ndarray, v_uncond: np.ndarray, scale: float) -> np.ndarray:
    """Classifier-free guidance of two velocity predictions ([LB-fast] table: causal_pretrain, scale 5.0)."""
    vu = np.asarray(v_uncond, np.float64)
    return vu + float(scale) * (np.asarray(v_cond, np.float64) - vu)


def sampler_step(x_t: np.ndarray, v_cond: np.ndarray, sigma: float, sigma_next: Optional[float] = None,
                 noise: Optional[np.ndarray] = None, v_uncond: Optional[np.ndarray] = None,
                 cfg_scale: float = 1.0):
    """One step of the loop: (guided) velocity -> x0 -> re-noised x at sigma_next (None on the last step).

    Returns (x0, x_next); x_next is None when ``noise`` is None (last step: x0 is the output).
    """
    v = v_cond if v_uncond is None else cfg_combine(v_cond, v_uncond, cfg_scale)
    x0 = flow_to_x0(x_t, v, sigma)
    if noise is None:
        return x0, None
    if sigma_next is None:
        raise ValueError("sigma_next is needed to re-noise")
    return x0, renoise(x0, noise, sigma_next)


def denoise_chunk(x_start: np.ndarray, timesteps: Sequence[float], velocity: Callable[[np.ndarray, float], np.ndarray],
                  noises: Sequence[np.ndarray], num_train: int = NUM_TRAIN_TIMESTEPS) -> np.ndarray:
    """The per-chunk few-step loop of [LB-fast] 2. 4 步采样 / [ABot-stream] 机制二.

    ``x_start`` is the chunk's latent at the first (noisiest) timestep; ``velocity(x, t)``
    stands in for the forward pass; ``noises[i]`` re-noises after step i (one per step
    but the last).  Returns the clean latent of the last step.
    """
    ts = list(timesteps)
    if len(noises) < len(ts) - 1:
        raise ValueError("one noise tensor per step but the last")
    x = np.asarray(x_start, np.float64)
    x0 = x
    for i, t in enumerate(ts):
        v = velocity(x, t)
        x0 = flow_to_x0(x, v, sigma_of(t, num_train))
        if i + 1 < len(ts):
            x = renoise(x0, noises[i], sigma_of(ts[i + 1], num_train))
    return x0
