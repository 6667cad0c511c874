"""The no-allocation segmented prefill (gdn_delta_rule_prefill_segmented_noalloc,
scratch inside the library) against the allocating entry point with a
caller workspace: same kernels, so the outputs and final states must be
bitwise equal.  Two calls in a row, the second on a smaller input (the
scratch keeps the first call's contents); the call recorded into a HIP graph
by stream capture and replayed; then a call over the scratch limit, which
must be refused before any launch."""
import pytest
import torch

import gdn_testlib as TL

pytestmark = pytest.mark.gpu

gdn = pytest.importorskip("linear_attention_layers_amd.gdn")
from linear_attention_layers_amd import inputs as I  # noqa: E402

DEV = "cuda"

CASES = [
    # geometry, lengths, has_init, nseg: the second is smaller in every size
    (I.Geometry(Hk=2, Hv=4), [2600, 700, 1], [1, 0, 1], 5),
    (I.Geometry(Hk=1, Hv=2), [500], [1], 3),
]


def _both(geo, lengths, hinit, nseg, seed):
    lb = I.make_layer(geo, lengths, "bf16", seed, state_std=0.3, has_init=hinit)
    out = TL.gpu_layer(lb)               # q, k, v from the conv and post-conv
    args = (out["q"], out["k"], out["v"], out["g"], out["beta"], out["cu"])
    st1 = lb.state.to(DEV).contiguous()
    o1 = torch.empty_like(out["v"])
    gdn.gdn_delta_rule_prefill_segmented_noalloc(*args, st1, nseg, out["hi"], o=o1)
    st2 = lb.state.to(DEV).contiguous()
    ws = torch.full((gdn.gdn_prefill_segmented_workspace(lb.nseq, geo.Hv, nseg),), 0xFF, dtype=torch.uint8,
                    device=DEV)
    o2 = gdn.gdn_delta_rule_prefill_segmented(*args, st2, nseg, out["hi"], workspace=ws)
    torch.cuda.synchronize()
    return o1, st1, o2, st2


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    for i, (geo, lengths, hinit, nseg) in enumerate(CASES):
        print(f"no-alloc call {i}: lengths {lengths} nseg {nseg} Hv {geo.Hv}", flush=True)
        o1, st1, o2, st2 = _both(geo, lengths, hinit, nseg, 1900 + i)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"call {i}: o differs"
        assert torch.equal(st1.view(torch.int32), st2.view(torch.int32)), f"call {i}: state differs"
        assert torch.isfinite(o1.float()).all() and torch.isfinite(st1).all()


def test_noalloc_replays_from_a_captured_graph():
    # the callers this entry point is for: launches recorded by stream
    # capture and replayed; each replay (after eager restores of the state
    # and poisoned outputs) must give the eager call's bits
    geo, lengths, hinit, nseg = CASES[0]
    lb = I.make_layer(geo, lengths, "bf16", 1960, state_std=0.3, has_init=hinit)
    out = TL.gpu_layer(lb)
    args = (out["q"], out["k"], out["v"], out["g"], out["beta"], out["cu"])
    st0 = lb.state.to(DEV).contiguous()
    st, o = st0.clone(), torch.empty_like(out["v"])
    gdn.gdn_delta_rule_prefill_segmented_noalloc(*args, st, nseg, out["hi"], o=o)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    stc, oc = st0.clone(), torch.empty_like(o)
    with torch.cuda.graph(graph):
        gdn.gdn_delta_rule_prefill_segmented_noalloc(*args, stc, nseg, out["hi"], o=oc)
    for rep in range(3):
        stc.copy_(st0)
        oc.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(oc.view(torch.int16), o.view(torch.int16)), f"replay {rep}: o differs"
        assert torch.equal(stc.view(torch.int32), st.view(torch.int32)), f"replay {rep}: state differs"


def test_noalloc_refuses_more_than_its_scratch():
    geo = I.Geometry(Hk=16, Hv=32)
    lb = I.make_layer(geo, [130, 130], "bf16", 1950, state_std=0.3)
    out = TL.gpu_layer(lb)
    # 3 x 2 sequences x 8 segments x 32 heads x 64 KiB = 96 MiB > 24 MiB
    with pytest.raises(gdn.GdnError) as exc:
        gdn.gdn_delta_rule_prefill_segmented_noalloc(out["q"], out["k"], out["v"], out["g"], out["beta"],
                                                     out["cu"], lb.state.to(DEV), 8, out["hi"],
                                                     o=torch.empty_like(out["v"]))
    assert exc.value.status == 7     # GDN_ERR_CAPACITY
