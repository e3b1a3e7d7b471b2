"""Plant plausible mistakes in the oracle (a copy of its source, on the CPU) and check a pin fails.

Each mutation is a textual edit of ``oracle/skv_oracle.py``; the edited source is
loaded as a throw-away module and every pin of ``oracle_checks`` is run against it.
At least one pin must fail for each mutation.
"""
import importlib.util
import os
import types

import pytest

from tests import oracle_checks as oc

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "skv_oracle.py")

MUTATIONS = {
    "evict_wrong_index": ("del self.entries[self.sink]", "del self.entries[min(self.sink + 1, len(self.entries) - 1)]"),
    "evict_sink_too": ("del self.entries[self.sink]", "del self.entries[0]"),
    "window_keeps_one_less": ("keep = window - sink - chunk", "keep = window - sink - chunk - 1"),
    "window_ignores_chunk": ("if len(entries) + chunk <= window:", "if len(entries) <= window:"),
    "rope_sign_flip": ("x0 * cos - x1 * sin", "x0 * cos + x1 * sin"),
    "rope_pairs_swapped": ("out[:, :, off:off + d_axis:2] = x0 * cos - x1 * sin",
                           "out[:, :, off:off + d_axis:2] = x1 * cos - x0 * sin"),
    "rope_hw_transposed": ("return idx // grid_w, idx % grid_w", "return idx % grid_w, idx // grid_w"),
    "rope_time_dropped": ("pos_t = np.repeat(t_ids, f)", "pos_t = np.repeat(t_ids * 0.0, f)"),
    "rope_freq_exponent": ("-2.0 * k / float(d_axis)", "-1.0 * k / float(d_axis)"),
    "rope_split_swapped": ("return d - 2 * hw, hw, hw", "return hw, d - 2 * hw, hw"),
    "scale_wrong": ("1.0 / math.sqrt(d) if scale is None", "1.0 / d if scale is None"),
    "v_is_k": ("out[r0:r0 + block_rows, hh, :] = p @ vh", "out[r0:r0 + block_rows, hh, :] = p @ kh"),
    "abs_query_offset": ("return list(range(s0, s0 + self.c))", "return list(range(s0 + 1, s0 + 1 + self.c))"),
    "abs_key_offset": ("kf = [self._rope(kk, [f0 + i]) for i, kk in enumerate(kf)]",
                       "kf = [self._rope(kk, [f0 + i + 1]) for i, kk in enumerate(kf)]"),
    "rel_ids_frame_based": ("k_hist = [self._rope(e[1], self._clamp([j])) for j, e in enumerate(hist)]",
                            "k_hist = [self._rope(e[1], self._clamp([e[0]])) for j, e in enumerate(hist)]"),
    "rel_query_ids_off": ("return self._clamp(range(nv - self.c, nv))", "return self._clamp(range(nv - self.c - 1, nv - 1))"),
    "bc_chunk_end_early": ("e = q_frame0 + chunk_frames * ((i - q_frame0) // chunk_frames + 1)",
                           "e = q_frame0 + chunk_frames * ((i - q_frame0) // chunk_frames)"),
    "bc_window_short": ("(j >= e - (window_frames - sink_frames))", "(j >= e - (window_frames - sink_frames) + 1)"),
    "bc_no_sinks": ("(j < sink_frames) | (j >= e", "(j < 0) | (j >= e"),
    "bc_frame_causal": ("return (j < e) &", "return (j <= i) &"),
    "abs_stores_raw": ("if self.mode == \"abs\":\n            f0 = self.n_appended", "if False:\n            f0 = self.n_appended"),
}


def _load_mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    mod = types.ModuleType("skv_oracle_mutant")
    exec(compile(src, "skv_oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    old, new = MUTATIONS[name]
    mutant = _load_mutant(old, new)
    monkeypatch.setattr(oc, "so", mutant)
    failed = []
    for check in oc.ALL_CHECKS:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            failed.append(check.__name__)
    assert failed, f"no pin caught mutation {name}"
