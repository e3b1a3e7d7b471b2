"""Pins of the sampler oracle (``oracle/sampler.py``) and planted-mistake checks.

Pins: the flow-matching round trip (re-noising a clean latent and recovering it
with the velocity that generated it), the endpoint cases sigma = 0 and 1, the
special cases of guidance, the timestep figures the pages print, and the loop's
trajectory under an exact velocity field.
"""
import json
import os
import types

import numpy as np
import pytest

from oracle import sampler as sp

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "sampler.py")
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_figures.json")


def _rng(seed):
    return np.random.default_rng(seed)


def check_round_trip(m):
    """x_t = renoise(x0, eps, s); with v = eps - x0 the one-step conversion returns x0."""
    r = _rng(1)
    x0, eps = r.standard_normal((3, 50)), r.standard_normal((3, 50))
    for s in (0.25, 0.5, 0.821, 1.0):
        x_t = m.renoise(x0, eps, s)
        assert np.allclose(m.flow_to_x0(x_t, eps - x0, s), x0, rtol=0, atol=1e-13)
        # the interpolation moves linearly from x0 (s = 0) toward the noise (s = 1)
        assert np.allclose(x_t - x0, s * (eps - x0), rtol=0, atol=1e-13)


def check_endpoints(m):
    """sigma 0: the latent is already clean; re-noising to 1 gives pure noise, to 0 the clean latent."""
    r = _rng(2)
    x, v, eps = r.standard_normal(40), r.standard_normal(40), r.standard_normal(40)
    assert np.array_equal(m.flow_to_x0(x, v, m.sigma_of(0)), x)
    assert np.array_equal(m.renoise(x, eps, 1.0), eps)
    assert np.array_equal(m.renoise(x, eps, 0.0), x)
    assert m.sigma_of(m.NUM_TRAIN_TIMESTEPS) == 1.0 and m.sigma_of(0) == 0.0


def check_guidance_cases(m):
    """scale 1 keeps the conditional prediction, scale 0 the unconditional one; equal inputs are fixed points."""
    r = _rng(3)
    a, b = r.standard_normal(30), r.standard_normal(30)
    assert np.allclose(m.cfg_combine(a, b, 1.0), a, atol=1e-15)
    assert np.array_equal(m.cfg_combine(a, b, 0.0), b)
    assert np.allclose(m.cfg_combine(a, a, 5.0), a, atol=1e-14)
    # scale 5 moves five times as far from the unconditional prediction as scale 1
    assert np.allclose(m.cfg_combine(a, b, 5.0) - b, 5.0 * (m.cfg_combine(a, b, 1.0) - b), atol=1e-13)


def check_page_timesteps(m):
    """The printed schedules: ABot's list starts at pure noise and falls; LingBot's indices pick falling steps."""
    g = {k: v["value"] for k, v in json.load(open(GOLDEN)).items() if not k.startswith("_")}
    sig = [m.sigma_of(t) for t in g["abot_denoise_steps"]]
    assert sig == [1.0, 0.75, 0.5, 0.25]
    ts = m.timesteps_from_indices(g["lingbot_timesteps_index"])
    assert ts[0] == m.NUM_TRAIN_TIMESTEPS and all(a > b > 0 for a, b in zip(ts, ts[1:]))
    assert ts == [1000, 821, 642, 321]


def check_loop_trajectory(m):
    """Exact velocity field for a target x0*: every step recovers x0*, and the latent seen at step i
    is x0* re-noised with noise i-1 to that step's sigma."""
    r = _rng(4)
    target = r.standard_normal((2, 16))
    noises = [r.standard_normal((2, 16)) for _ in range(3)]
    start_noise = r.standard_normal((2, 16))
    steps = [1000, 750, 500, 250]
    seen = []

    def velocity(x, t):
        seen.append((x.copy(), t))
        s = m.sigma_of(t)
        return (x - target) / s  # the velocity that maps this x back to the target in one step

    x_start = m.renoise(target, start_noise, m.sigma_of(steps[0]))
    out = m.denoise_chunk(x_start, steps, velocity, noises)
    assert np.allclose(out, target, atol=1e-12)
    assert [t for _, t in seen] == steps
    for i in range(1, len(steps)):
        s = steps[i] / 1000.0
        expect = (1.0 - s) * target + s * noises[i - 1]
        assert np.allclose(seen[i][0], expect, atol=1e-12), f"step {i}"


def check_sampler_step_modes(m):
    """sampler_step: guided velocity feeds x0; the last step (no noise) returns no re-noised latent."""
    r = _rng(5)
    x, vc, vu, eps = (r.standard_normal(20) for _ in range(4))
    x0, xn = m.sampler_step(x, vc, 0.5, 0.25, eps, v_uncond=vu, cfg_scale=5.0)
    v = vu + 5.0 * (vc - vu)
    assert np.allclose(x0, x - 0.5 * v, atol=1e-13)
    assert np.allclose(xn, 0.75 * x0 + 0.25 * eps, atol=1e-13)
    x0b, none = m.sampler_step(x, vc, 0.5)
    assert none is None and np.allclose(x0b, x - 0.5 * vc, atol=1e-14)


CHECKS = [check_round_trip, check_endpoints, check_guidance_cases, check_page_timesteps, check_loop_trajectory,
          check_sampler_step_modes]


@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__)
def test_sampler_pin(check):
    check(sp)


MUTATIONS = {
    "flow_sign": ("- float(sigma) * np.asarray(v, np.float64)", "+ float(sigma) * np.asarray(v, np.float64)"),
    "renoise_weights_swapped": ("return (1.0 - s) * np.asarray(x0, np.float64) + s * np.asarray(noise, np.float64)",
                                "return s * np.asarray(x0, np.float64) + (1.0 - s) * np.asarray(noise, np.float64)"),
    "cfg_on_uncond": ("return vu + float(scale) * (np.asarray(v_cond, np.float64) - vu)",
                      "return np.asarray(v_cond, np.float64) + float(scale) * (vu - np.asarray(v_cond, np.float64))"),
    "sigma_reversed": ("return float(t) / float(num_train)", "return 1.0 - float(t) / float(num_train)"),
    "table_ascending": ("out.append(num_train - int(i))", "out.append(int(i) + 1)"),
    "renoise_with_current_sigma": ("x = renoise(x0, noises[i], sigma_of(ts[i + 1], num_train))",
                                   "x = renoise(x0, noises[i], sigma_of(ts[i], num_train))"),
    "loop_returns_noisy": ("            x = renoise(x0, noises[i], sigma_of(ts[i + 1], num_train))\n    return x0",
                           "            x = renoise(x0, noises[i], sigma_of(ts[i + 1], num_train))\n    return x"),
    "noise_index_shift": ("renoise(x0, noises[i], sigma_of", "renoise(x0, noises[max(i - 1, 0)], sigma_of"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_sampler_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("sampler_mutant")
    exec(compile(src.replace(old, new, 1), "sampler_mutant", "exec"), mod.__dict__)
    failed = []
    for check in CHECKS:
        try:
            check(mod)
        except (AssertionError, ValueError, IndexError):
            failed.append(check.__name__)
    assert failed, f"no pin caught mutation {name}"
