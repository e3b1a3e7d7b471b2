"""GPU parity of the sampler step (sampler_step in skv.h) against the fp64 oracle.

The kernel computes in fp64 and rounds once to the output dtype (bf16 through fp32),
so each output must lie within one unit in the last place of the output dtype of the
oracle's exact fp64 value (half a unit for the rounding, the rest for the two-step
bf16 rounding and for a fused multiply-add).
"""
import numpy as np
import pytest
import torch

import seeded_inputs as si
import streaming_kv_cache_amd as skv
from oracle import sampler as sp

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _ulp(x: np.ndarray, dtype) -> np.ndarray:
    """Spacing of the output dtype at |x| (fp32: 2^-23 relative, bf16: 2^-7), normal range."""
    mant = 23 if dtype == torch.float32 else 7
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - mant)


def _draw(n, tid, dtype):
    return si.draw((n,), 11, 0, 0, tid, dtype)


def _f64(t):
    return t.detach().float().cpu().double().numpy()


def _check(gpu, exact, dtype, what):
    g = _f64(gpu)
    err = np.abs(g - exact)
    bad = err > _ulp(exact, dtype) * 1.0000001
    assert not bad.any(), f"{what}: {bad.sum()} elements beyond 1 ulp, worst {err.max():.3g}"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n", [1, 7, 8, 13, 4096 + 5, 2640 * 24 * 128])
def test_sampler_step_parity(dtype, n):
    say(f"[sampler] dtype={dtype} n={n}")
    x, vc, vu, e = (_draw(n, t, dtype) for t in (si.Q, si.K, si.V, si.TEXT_K))
    xd, vcd, vud, ed = (t.cuda() for t in (x, vc, vu, e))
    for cfg in (None, 5.0):
        for sig, sig_n in ((1.0, 0.75), (0.821, 0.642), (0.25, None)):
            x0, xn = skv.sampler_step(xd, vcd, sig, sig_n or 0.0, noise=ed if sig_n else None,
                                      v_uncond=vud if cfg else None, cfg_scale=cfg or 1.0)
            torch.cuda.synchronize()
            ex0, exn = sp.sampler_step(_f64(x), _f64(vc), sig, sig_n, _f64(e) if sig_n else None,
                                       v_uncond=_f64(vu) if cfg else None, cfg_scale=cfg or 1.0)
            _check(x0, ex0, dtype, f"x0 cfg={cfg} sigma={sig}")
            if sig_n:
                _check(xn, exn, dtype, f"x_next cfg={cfg} sigma={sig}")
            else:
                assert xn is None


def test_sampler_step_in_place_and_outputs():
    """x_next written over x_t; x0 not requested; the pair of calls matches the oracle."""
    n = 3 * 880 + 3
    dtype = torch.bfloat16
    x, v, e = (_draw(n, t, dtype) for t in (si.Q, si.K, si.V))
    xd = x.cuda()
    x0, xn = skv.sampler_step(xd, v.cuda(), 0.75, 0.5, noise=e.cuda(), x_next_out=xd, want_x0=False)
    torch.cuda.synchronize()
    assert x0 is None and xn.data_ptr() == xd.data_ptr()
    _, exn = sp.sampler_step(_f64(x), _f64(v), 0.75, 0.5, _f64(e))
    _check(xd, exn, dtype, "in-place x_next")


def test_denoise_loop_fp32():
    """The four-step loop (ABot's denoising_step_list) run with sampler_step matches the oracle's loop
    when the velocity of each step is a fixed synthetic field."""
    n = 2 * 880 * 8
    steps = [1000, 750, 500, 250]
    x_start = _draw(n, si.Q, torch.float32)
    vel = [si.draw((n,), 12, 0, i, si.K, torch.float32) for i in range(4)]
    noises = [si.draw((n,), 12, 0, i, si.V, torch.float32) for i in range(3)]
    x = x_start.cuda()
    out = None
    for i, t in enumerate(steps):
        last = i + 1 == len(steps)
        x0, xn = skv.sampler_step(x, vel[i].cuda(), sp.sigma_of(t), 0.0 if last else sp.sigma_of(steps[i + 1]),
                                  noise=None if last else noises[i].cuda())
        out, x = (x0, xn) if not last else (x0, None)
    torch.cuda.synchronize()
    table = {s: _f64(v) for s, v in zip(steps, vel)}
    ref = sp.denoise_chunk(_f64(x_start), steps, lambda xx, t: table[t], [_f64(z) for z in noises])
    err = np.abs(_f64(out) - ref)
    # each step rounds x to fp32 once (rel 2^-24) and the later steps scale that error by at most 1
    assert err.max() <= 8 * 2.0 ** -24 * (np.abs(ref).max() + 1.0), err.max()
