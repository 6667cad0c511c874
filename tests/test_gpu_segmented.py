"""Segment-parallel prefill (gdn_delta_rule_prefill_segmented) against the
oracle: its o and final state against the per-token rule, and the
transitions it leaves in the workspace (R_p, P_p and the chained entering
states X_p) against the oracle's segment transition, on ragged batches with
empty and one-token sequences and trailing empty segments."""
import numpy as np
import pytest
import torch

import gdn_testlib as TL
from oracle import gdn_oracle as O

pytestmark = pytest.mark.gpu

gdn = pytest.importorskip("linear_attention_layers_amd.gdn")
from linear_attention_layers_amd import inputs as I  # noqa: E402

DEV = "cuda"

# (geometry, lengths, has_init, nseg)
SEG_CASES = [
    (I.Geometry(Hk=2, Hv=4), [700], [1], 2),
    (I.Geometry(Hk=2, Hv=4), [1000], [1], 4),
    (I.Geometry(Hk=1, Hv=2), [300, 1, 0, 900], [1, 0, 1, 1], 3),
    (I.GEO_TINY, [130, 64], [0, 1], 5),           # 3 and 1 chunks: trailing segments empty
    (I.Geometry(Hk=2, Hv=4), [2000, 129], [1, 1], 7),
]


def _segmented(lb, out, nseg):
    st = lb.state.to(DEV).contiguous()
    ws = torch.full((gdn.gdn_prefill_segmented_workspace(lb.nseq, lb.geo.Hv, nseg),), 0xFF,
                    dtype=torch.uint8, device=DEV)   # NaN-filled: nothing may read it unwritten
    o = gdn.gdn_delta_rule_prefill_segmented(out["q"], out["k"], out["v"], out["g"], out["beta"],
                                             out["cu"], st, nseg, out["hi"], workspace=ws)
    torch.cuda.synchronize()
    return o, st, ws


@pytest.mark.parametrize("case", range(len(SEG_CASES)))
def test_segmented_prefill_parity(case):
    geo, lengths, hinit, nseg = SEG_CASES[case]
    print(f"segmented case {case}: lengths {lengths} nseg {nseg}", flush=True)
    lb = I.make_layer(geo, lengths, "bf16", 700 + case, state_std=0.3, has_init=hinit)
    out = TL.gpu_layer(lb)
    o, st, _ = _segmented(lb, out, nseg)
    o_ref, st_ref = O.delta_rule_recurrent(TL.np64(out["q"]), TL.np64(out["k"]), TL.np64(out["v"]),
                                           TL.np64(lb.g), TL.np64(lb.beta), TL.np64(lb.state),
                                           lb.has_init.numpy(), lb.cu_seqlens.tolist(), geo.Hk, geo.Hv)
    TL.check_normwise(TL.np64(o), o_ref, TL.REC_BF16, axes=(2,), what="o")
    TL.check_normwise(TL.np64(st), st_ref, TL.REC_BF16, axes=(2, 3), what="state")
    # and against the unsegmented prefill of the same inputs (rounding only)
    TL.check_normwise(TL.np64(o), TL.np64(out["o"]), TL.REC_BF16, axes=(2,), what="o vs prefill")
    TL.check_normwise(TL.np64(st), TL.np64(out["state"]), TL.REC_BF16, axes=(2, 3),
                      what="state vs prefill")


@pytest.mark.parametrize("case", [1, 2])
def test_segmented_prefill_workspace_transitions(case):
    geo, lengths, hinit, nseg = SEG_CASES[case]
    lb = I.make_layer(geo, lengths, "bf16", 700 + case, state_std=0.3, has_init=hinit)
    out = TL.gpu_layer(lb)
    _, _, ws = _segmented(lb, out, nseg)
    Hk, Hv = geo.Hk, geo.Hv
    W = ws.view(torch.float32).view(3, lb.nseq, nseg, Hv, 128, 128)
    q, k, v = TL.np64(out["q"]), TL.np64(out["k"]), TL.np64(out["v"])
    g, b, S0 = TL.np64(lb.g), TL.np64(lb.beta), TL.np64(lb.state)
    bounds = O.segment_bounds(lb.cu_seqlens.tolist(), nseg)
    for s in range(lb.nseq):
        # entering state of each segment, by the per-token rule over the prefix
        for p in range(1, nseg):
            b0, e0 = int(bounds[s, p, 0]), int(bounds[s, p, 1])
            P_ref = O.segment_transition(k, g, b, [b0, e0], Hk, Hv)[0]
            _, R_ref = O.delta_rule_recurrent(q, k, v, g, b, S0[s:s + 1], [0], [b0, e0], Hk, Hv)
            _, X_ref = O.delta_rule_recurrent(q, k, v, g, b, S0[s:s + 1], [int(lb.has_init[s])],
                                              [int(lb.cu_seqlens[s]), b0], Hk, Hv)
            what = f"seq {s} segment {p} [{b0},{e0})"
            TL.check_normwise(TL.np64(W[2, s, p]), P_ref, TL.REC_BF16, axes=(1, 2), what="P " + what)
            if e0 > b0:
                TL.check_normwise(TL.np64(W[1, s, p]), R_ref[0], TL.REC_BF16, axes=(1, 2), what="R " + what)
            else:
                assert torch.equal(W[1, s, p].cpu(), torch.zeros_like(W[1, s, p].cpu()))
                assert torch.equal(W[2, s, p].cpu(), torch.eye(128).expand(Hv, 128, 128))
            TL.check_normwise(TL.np64(W[0, s, p]), X_ref[0], TL.REC_BF16, axes=(1, 2), what="X " + what)


def test_segmented_prefill_one_segment_is_the_prefill():
    geo = I.Geometry(Hk=2, Hv=4)
    lb = I.make_layer(geo, [300, 77], "bf16", 760, state_std=0.3, has_init=[1, 0])
    out = TL.gpu_layer(lb)
    o, st, _ = _segmented(lb, out, 1)
    assert torch.equal(o, out["o"]) and torch.equal(st, out["state"])


def test_segmented_prefill_ignores_poisoned_state_without_init():
    geo = I.GEO_TINY
    lb = I.make_layer(geo, [200, 5], "bf16", 761, state_std=0.3, has_init=[0, 0])
    out = TL.gpu_layer(lb)
    lb.state[:] = float("nan")
    o, st, _ = _segmented(lb, out, 3)
    assert torch.isfinite(o.float()).all() and torch.isfinite(st).all()
