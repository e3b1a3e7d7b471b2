"""Ring-slot bookkeeping (host C++, built with g++ without HIP) against the oracle's cache list.

A physical slot array is simulated from the slots the bookkeeping reports for
each appended frame; the frames it then reads back (cache in logical order, and
the visible set a chunk attends to) must equal the oracle's list exactly.
"""
import json
import os
import subprocess

import numpy as np
import pytest

from oracle import skv_oracle as so

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "tests", "host", "ring_probe.cpp"),
       os.path.join(ROOT, "streaming_kv_cache_amd", "csrc", "skv_core.cpp")]
EXE = os.path.join(ROOT, "_build", "ring_probe")


@pytest.fixture(scope="module")
def probe():
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-fsanitize=address,undefined",
                    "-I", os.path.join(ROOT, "include"), *SRC, "-o", EXE], check=True)
    return EXE


def run(exe, s, w, c, appends):
    inp = f"cfg {s} {w} {c}\n" + "".join(f"append {n}\n" for n in appends)
    r = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True)
    return [json.loads(l) for l in r.stdout.splitlines()]


CASES = [(1, 4, 2), (6, 18, 4), (5, 21, 3), (0, 5, 2), (2, 7, 2), (2, 5, 3), (0, 3, 3), (3, 9, 1), (4, 40, 5)]


@pytest.mark.parametrize("s,w,c", CASES)
def test_ring_matches_oracle(probe, s, w, c):
    rng = np.random.default_rng(s * 100 + w * 10 + c)
    # first append may be a prefill of the sinks; then mostly chunks of c, sometimes other sizes
    appends = ([s] if s else []) + [c if rng.random() < 0.7 else int(rng.integers(1, w - s + 1)) for _ in range(80)]
    outs = run(probe, s, w, c, appends)
    cl = so.CacheList(s, w)
    slots = {}
    t = 0
    for n, o in zip(appends, outs):
        for i, sl in enumerate(o["slots"]):
            slots[sl] = t + i
        cl.append([np.zeros(1)] * n, [np.zeros(1)] * n)
        t += n
        assert o["T"] == t
        # cache in logical order read back from the physical slots
        assert [f for f, _ in o["cached"]] == cl.frame_ids()
        assert [slots[sl] for _, sl in o["cached"]] == cl.frame_ids()
        # visible history read from the plan's slot runs
        vis = so.visible_history(cl.entries, c, s, w)
        got = []
        for slot0, frames, logical0 in o["runs"]:
            assert logical0 == len(got)
            got.extend(slots[slot0 + j] for j in range(frames))
        assert got == [e[0] for e in vis]
        assert o["n_hist"] == len(vis) and o["n_vis"] == len(vis) + c
        assert len(o["runs"]) <= 3


def test_bad_config_rejected(probe):
    r = subprocess.run([probe], input="cfg 3 4 2\n", capture_output=True, text=True, check=True)
    assert json.loads(r.stdout)["error"] == 2
