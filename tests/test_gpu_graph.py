"""HIP graph replay of the benchmark's mixed serving step.

The benchmark captures its timed steps as one HIP graph (launches, the side
stream's fork and join, and event-record nodes) and replays it.  These tests
capture a small two-layer version of the same plan, replay it several times
with the program's own eager work (state restores, output poisoning) and
synchronisations between the replays, and require every replay to reproduce
the eager step bit for bit: o, the prefill tokens' q/k/v, the conv rows and
the recurrent states of every layer.
"""
import math
import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from linear_attention_layers_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu

# three ragged prefill sequences (one of a single token) and four decode tokens
LENGTHS = [300, 64, 1, 1, 1, 1, 1]
N_PREFILL = 3


def small_mixed_layer(layer):
    lb = inputs.make_layer(inputs.GEO_6144, LENGTHS, "bf16", 7000 + 10 * layer,
                           conv_state_std=math.sqrt(0.1), state_std=math.sqrt(0.1))
    lb.meta["n_prefill"] = N_PREFILL
    return lb


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _setup():
    dev = torch.device("cuda", 0)
    plan = bench.plan_mixed(dev, layers=2, make_layer=small_mixed_layer)
    runner = bench.Runner(plan, torch.cuda.current_stream())
    mutable = [t for d in plan.keep for t in (d["cs"], d["st"])]
    init = [t.clone() for t in mutable]
    outs = []
    for d in plan.keep:
        npre = int(d["cu_pre"][-1])
        outs += [d["o"], d["q"][:npre], d["k"][:npre], d["v"][:npre], d["cs"], d["st"]]
    poison = [d[nm] for d in plan.keep for nm in ("o", "q", "k", "v")]

    def restore():
        for t, t0 in zip(mutable, init):
            t.copy_(t0)
        for t in poison:
            t.fill_(float("nan"))

    return plan, runner, outs, restore


def test_graph_replays_match_the_eager_step():
    plan, runner, outs, restore = _setup()
    restore()
    runner.step()
    torch.cuda.synchronize()
    ref = [_bits(t).clone() for t in outs]
    assert all(torch.isfinite(t).all() for t in outs)

    graph = runner.capture(steps=1)
    for rep in range(3):
        restore()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outs, ref)):
            assert torch.equal(_bits(t), r), f"replay {rep}: output {i} differs from the eager step"


def test_graph_with_timing_nodes_matches_and_times_the_prefill():
    plan, runner, outs, restore = _setup()
    restore()
    runner.step()
    torch.cuda.synchronize()
    ref = [_bits(t).clone() for t in outs]

    events = [runner.events()]
    graph = runner.capture(events, only="prefill")
    for rep in range(2):
        restore()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outs, ref)):
            assert torch.equal(_bits(t), r), f"replay {rep}: output {i} differs from the eager step"
        ms = runner.stage_ms(events[0], only="prefill")["prefill"]
        assert 0.0 < ms < 1000.0
