"""The named workloads of inputs.py against their definitions, restated in
tests/golden/workloads.json: every shape, dtype, decay, initial-state and
segment field, the decay schedule's values, and the statistics of small draws
of each recipe (scales of q, k, v and S0).  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

from long_sequence_causal_amd import inputs

HERE = os.path.dirname(os.path.abspath(__file__))
SPEC = json.load(open(os.path.join(HERE, "golden", "workloads.json")))["workloads"]


def test_the_same_workloads_are_defined():
    assert set(inputs.WORKLOADS) == set(SPEC)


@pytest.mark.parametrize("name", sorted(SPEC))
def test_workload_fields_match_their_definition(name):
    w, s = inputs.WORKLOADS[name], SPEC[name]
    for key in ("B", "H", "L", "d", "dtype", "decay", "s0_std", "nseg", "backward"):
        assert getattr(w, key) == s[key], (name, key)
    assert w.L % w.nseg == 0 and (w.L // w.nseg) % 64 == 0
    if "same_seed_as" in s:
        assert w.seed == inputs.WORKLOADS[s["same_seed_as"]].seed
    seeds = [x.seed for n, x in inputs.WORKLOADS.items() if "same_seed_as" not in SPEC[n]]
    assert len(set(seeds)) == len(seeds)  # otherwise distinct draws


def test_segment_length_of_the_segmented_workload():
    w = inputs.WORKLOADS["segmented_1m"]
    assert w.L // w.nseg == 16384


@pytest.mark.parametrize("H", [2, 16, 32])
def test_decay_schedule_values(H):
    lam = inputs.decay_schedule(H)
    assert lam.dtype == torch.float32 and lam.shape == (H,)
    for h in range(H):
        want = np.float32(math.exp(-(2.0 ** (-(5.0 + 8.0 * h / H)))))
        assert lam[h].item() == want
    assert bool((lam > 0).all()) and bool((lam < 1).all())
    assert bool((lam[1:] > lam[:-1]).all())  # slower decay for later heads
    assert bool((inputs.decay_schedule(H, decay=False) == 1).all())


@pytest.mark.parametrize("name", sorted(SPEC))
def test_draws_follow_the_recipe(name):
    """A short draw (same B, H, d, dtype; L cut to 2048) has the stated
    scales: std(q) = std(k) = 1/sqrt(d), std(v) = 1, std(S0) = s0_std."""
    s = SPEC[name]
    inp = inputs.workload_inputs(name, device="cpu", L=2048)
    q, k, v, S0 = inp["q"], inp["k"], inp["v"], inp["S0"]
    want_dtype = torch.bfloat16 if s["dtype"] == "bf16" else torch.float32
    for t in (q, k, v):
        assert t.dtype == want_dtype and t.shape == (s["B"], s["H"], 2048, s["d"])
    assert abs(float(q.float().std()) * math.sqrt(s["d"]) - 1) < 0.03
    assert abs(float(k.float().std()) * math.sqrt(s["d"]) - 1) < 0.03
    assert abs(float(v.float().std()) - 1) < 0.03
    if s["s0_std"] > 0:
        assert S0.dtype == torch.float32 and S0.shape == (s["B"], s["H"], 1, s["d"], s["d"])
        assert abs(float(S0.std()) / s["s0_std"] - 1) < 0.03
    else:
        assert S0 is None
    assert (inp["dO"] is not None) == s["backward"]
    lam = inp["lam"]
    assert torch.equal(lam, inputs.decay_schedule(s["H"], s["decay"]))
