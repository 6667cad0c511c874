"""GPU parity of the paths that short runs do not reach: hand-derived float32
L2 scale values, decode / verify windows longer than one 16-token block,
the tiny float32 layer's step form, a float32 commit, a long chain of
committed one-token steps, and empty sequences (with and without an
initial state, stored buffers poisoned with NaN) through every entry point
that writes a final state.  Every call goes through the C ABI; the
reference is the CPU oracle, except for a batch cut into groups of
consecutive sequences, which must give the bits of one launch."""
import os

import numpy as np
import pytest
import torch

import gdn_testlib as TL
from oracle import gdn_oracle as O

pytestmark = pytest.mark.gpu

gdn = pytest.importorskip("linear_attention_layers_amd.gdn")
from linear_attention_layers_amd import inputs as I  # noqa: E402

DEV = "cuda"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- L2 scale

def _l2_scale_cases():
    """tests/golden/l2_scale_cases.txt: (name, eps, y head, q_hat bits)."""
    def parse(spec, conv):
        vals, fill = {}, None
        for part in spec.split(";"):
            key, val = [p.strip() for p in part.split(":")]
            if key == "rest":
                fill = conv(val)
            else:
                vals[int(key)] = conv(val)
        return [vals.get(i, fill) for i in range(128)]

    out = []
    with open(os.path.join(GOLDEN, "l2_scale_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, eps, yspec, qspec = [p.strip() for p in line.split("|")]
            out.append((name, float(eps), parse(yspec, float), parse(qspec, lambda h: int(h, 16))))
    return out


@pytest.mark.parametrize("case", _l2_scale_cases(), ids=lambda c: c[0])
def test_postconv_f32_arm_gives_hand_derived_scale(case):
    """The float32 output arm rounds 1/sqrt(sum + eps) and then multiplies:
    its bits equal the values worked out by hand (a divide, or eps outside
    the square root, gives other bits)."""
    name, eps, yh, want = case
    geo = I.Geometry(Hk=1, Hv=1)
    y = torch.tensor([yh * 3] * 5, dtype=torch.float32)          # q, k and v heads, 5 tokens
    q, k, v = gdn.gdn_postconv_l2(y.to(DEV), 1, 1, eps, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for got in (q, k):
        bits = got.cpu().view(torch.int32).numpy().astype(np.uint32)
        assert (bits == np.array(want, dtype=np.uint32)[None, None]).all(), name
    assert torch.equal(v.cpu(), y[:, 2 * 128:].reshape(5, 1, 128))
    # the fused conv + post-conv arm gives the same bits: a conv with the
    # current-token tap 1 passes y through unchanged in float32
    w = torch.zeros(geo.C, 4)
    w[:, 3] = 1.0
    cu = torch.tensor([0, 5], dtype=torch.int32, device=DEV)
    cs = torch.zeros(1, 3, geo.C, device=DEV)
    q2, k2, _ = gdn.gdn_conv_postconv_fwd(y.to(DEV), w.to(DEV), None, cs, None, cu, None, False,
                                          1, 1, eps)
    torch.cuda.synchronize()
    assert torch.equal(q2.cpu().view(torch.int32), q.cpu().view(torch.int32))
    assert torch.equal(k2.cpu().view(torch.int32), k.cpu().view(torch.int32))


# ---------------------------------------------------------------- step windows

def _step_layer(act, geo, lengths, hinit, seed, commit, gate="softplus"):
    """conv + post-conv (oracle-checked elsewhere) then the step, all on the
    GPU; returns the batch and the device tensors."""
    lb = I.make_layer(geo, lengths, act, seed, state_std=0.3, has_init=hinit, gate=gate)
    cu, hi = lb.cu_seqlens.to(DEV), lb.has_init.to(DEV)
    cs = lb.conv_state.to(DEV)
    y = gdn.gdn_causal_conv_fwd(lb.x.to(DEV), lb.conv_w.to(DEV), None, cs, hi, cu,
                                gdn.gdn_make_chunks_device(cu, lb.N), commit)
    q, k, v = gdn.gdn_postconv_l2(y, geo.Hk, geo.Hv, 1e-6)
    st = lb.state.to(DEV)
    g, beta = lb.g.to(DEV), lb.beta.to(DEV)
    o = gdn.gdn_delta_rule_step(q, k, v, g, beta, cu, st, hi, commit_state=commit)
    torch.cuda.synchronize()
    return lb, dict(q=q, k=k, v=v, o=o, state=st, g=g, beta=beta, cu=cu, hi=hi, conv_state=cs)


def _check_step(lb, out, act, commit, what):
    o_ref, st_ref = O.delta_rule_recurrent(TL.np64(out["q"]), TL.np64(out["k"]), TL.np64(out["v"]),
                                           TL.np64(lb.g), TL.np64(lb.beta), TL.np64(lb.state),
                                           lb.has_init.numpy(), lb.cu_seqlens.tolist(),
                                           lb.geo.Hk, lb.geo.Hv)
    tol = TL.REC_F32 if act == "f32" else TL.REC_BF16
    wo = TL.check_normwise(TL.np64(out["o"]), o_ref, tol, axes=(2,), what=f"{what} o")
    ws = 0.0
    if commit:
        ws = TL.check_normwise(TL.np64(out["state"]), st_ref, tol, axes=(2, 3), what=f"{what} state")
    else:
        assert torch.equal(out["state"].cpu(), lb.state)
    print(f"{what}: worst o {wo:.2e}, state {ws:.2e} (bound {tol})", flush=True)


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("commit", [True, False])
def test_step_multi_block_windows_match_oracle(act, commit):
    """Windows of 17..40 tokens run the 16-token block loop two or three
    times, carrying the state between blocks."""
    lengths = [17, 24, 33, 40, 16, 1, 31]
    hinit = [1, 0, 1, 1, 0, 1, 1]
    print(f"step windows {lengths} act {act} commit {commit}", flush=True)
    lb, out = _step_layer(act, I.GEO_TINY, lengths, hinit, 1500 + (act == "f32") + 2 * commit, commit)
    _check_step(lb, out, act, commit, f"windows {act} commit={commit}")


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_step_gqa_ratio_two_long_window(act):
    lb, out = _step_layer(act, I.Geometry(Hk=2, Hv=4), [48, 20], [1, 1], 1510, True)
    _check_step(lb, out, act, True, f"gqa {act}")


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_tiny_layer_step_form_matches_oracle(act):
    """The tiny float32 layer (1 sequence, T = 64, C = 1024, zero initial
    recurrent state, conv_state ~N(0,1)) in its step form: conv, post-conv,
    then one 64-token committing step (four 16-token blocks), against the
    oracle chain.  The bf16 run takes the same draws in bf16."""
    base = I.tiny_f32()
    lb = I.make_layer(base.geo, [64], act, 1000, conv_state_std=1.0, state_std=0.0, has_init=[1])
    if act == "f32":
        assert torch.equal(lb.x, base.x) and torch.equal(lb.conv_state, base.conv_state)
    cu, hi = lb.cu_seqlens.to(DEV), lb.has_init.to(DEV)
    cs = lb.conv_state.to(DEV)
    y = gdn.gdn_causal_conv_fwd(lb.x.to(DEV), lb.conv_w.to(DEV), None, cs, hi, cu,
                                gdn.gdn_make_chunks_device(cu, 64), True)
    q, k, v = gdn.gdn_postconv_l2(y, 2, 4, 1e-6)
    st = lb.state.to(DEV)
    o = gdn.gdn_delta_rule_step(q, k, v, lb.g.to(DEV), lb.beta.to(DEV), cu, st, hi, commit_state=True)
    torch.cuda.synchronize()
    # the whole chain from raw inputs, in float64
    y_ref, cs_ref = O.causal_conv(TL.np64(lb.x), TL.np64(lb.conv_w), None, TL.np64(lb.conv_state),
                                  [1], [0, 64], True)
    assert np.array_equal(TL.np64(cs), cs_ref)
    TL.check_conv(TL.np64(y), y_ref, TL.conv_scale(TL.np64(lb.x), TL.np64(lb.conv_w), None,
                                                   TL.np64(lb.conv_state), [1], [0, 64]), act)
    qr, kr, vr = O.postconv_l2(O.round_to(y_ref, act), 2, 4, 128, 128, 1e-6)
    qr, kr, vr = (O.round_to(a, act) for a in (qr, kr, vr))
    o_ref, st_ref = O.delta_rule_recurrent(qr, kr, vr, TL.np64(lb.g), TL.np64(lb.beta),
                                           TL.np64(lb.state), [1], [0, 64], 2, 4)
    # stage-isolated at the recurrence bound, and the whole chain from raw
    # inputs (a few float32 ulps of q, k, v in front of the recurrence)
    _check_step(lb, dict(q=q, k=k, v=v, o=o, state=st), act, True, f"tiny layer step {act}")
    chain = 1e-4 if act == "f32" else TL.REC_BF16
    TL.check_normwise(TL.np64(o), o_ref, chain, axes=(2,), what="chain o")
    TL.check_normwise(TL.np64(st), st_ref, chain, axes=(2, 3), what="chain state")


# ---------------------------------------------------------------- commit f32

def test_commit_f32_matches_oracle_and_committing_step():
    geo = I.GEO_TINY
    L = 2
    lengths = [1, 8, 5, 3, 20, 2]
    n_keep = [0, 8, 2, 3, 17, 1]
    hinit = [1, 1, 1, 0, 1, 1]
    layers, runs = [], []
    for layer in range(L):
        lb, out = _step_layer("f32", geo, lengths, hinit, 1600 + 10 * layer, False)
        out["x"] = lb.x.to(DEV)
        runs.append((lb, out))
        layers.append(dict(x=out["x"], conv_state=out["conv_state"], state=out["state"],
                           k=out["k"], v=out["v"], g=out["g"], beta=out["beta"]))
    table = gdn.gdn_layer_table(layers, DEV)
    nk = torch.tensor(n_keep, dtype=torch.int32, device=DEV)
    cu, hi = runs[0][1]["cu"], runs[0][1]["hi"]
    gdn.gdn_commit(table, L, cu, nk, hi, geo.C, geo.Hk, geo.Hv, torch.float32)
    torch.cuda.synchronize()
    keep_idx = torch.cat([torch.arange(c, c + n) for c, n in zip(runs[0][0].cu_seqlens[:-1].tolist(), n_keep)])
    cu_keep = I.cu_from_lengths(n_keep).to(DEV)
    for layer, (lb, out) in enumerate(runs):
        cs_ref, st_ref = O.commit(TL.np64(lb.x), TL.np64(lb.conv_state), TL.np64(lb.state),
                                  TL.np64(out["k"]), TL.np64(out["v"]), TL.np64(lb.g), TL.np64(lb.beta),
                                  lb.has_init.numpy(), lb.cu_seqlens.tolist(), n_keep, geo.Hk, geo.Hv)
        assert np.array_equal(TL.np64(out["conv_state"]), cs_ref)
        TL.check_normwise(TL.np64(out["state"]), st_ref, TL.REC_F32, axes=(2, 3), what=f"layer {layer} state")
        kd = keep_idx.to(DEV)
        st2 = lb.state.to(DEV)
        gdn.gdn_delta_rule_step(out["q"][kd].contiguous(), out["k"][kd].contiguous(), out["v"][kd].contiguous(),
                                out["g"][kd].contiguous(), out["beta"][kd].contiguous(), cu_keep, st2, hi,
                                commit_state=True)
        torch.cuda.synchronize()
        assert torch.equal(st2, out["state"]), f"layer {layer}: commit differs from a committing step"


# ---------------------------------------------------------------- long chain

@pytest.mark.parametrize("gate", ["softplus", "slow"])
def test_long_chain_of_committed_decode_steps(gate):
    """512 one-token decode steps per sequence, each committing its state
    (bf16 activations, float32 state), against the per-token oracle over
    the whole run: the rounding of each step must not drift.  "slow" draws
    decays near one (log a ~ -U(0.001, 0.05)), so errors fade slowly."""
    geo = I.GEO_TINY
    nseq, T = 4, 512
    g_ = torch.Generator().manual_seed(1700 + (gate == "slow"))
    q = torch.nn.functional.normalize(torch.randn(T, nseq, geo.Hk, 128, generator=g_, dtype=torch.float64), dim=-1)
    k = torch.nn.functional.normalize(torch.randn(T, nseq, geo.Hk, 128, generator=g_, dtype=torch.float64), dim=-1)
    v = torch.randn(T, nseq, geo.Hv, 128, generator=g_, dtype=torch.float64)
    q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    if gate == "slow":
        g = -(0.001 + 0.049 * torch.rand(T, nseq, geo.Hv, generator=g_))
    else:
        g = -torch.nn.functional.softplus(torch.randn(T, nseq, geo.Hv, generator=g_))
    beta = torch.sigmoid(torch.randn(T, nseq, geo.Hv, generator=g_))
    state0 = torch.randn(nseq, geo.Hv, 128, 128, generator=g_) * 0.3
    st = state0.to(DEV)
    cu = torch.arange(nseq + 1, dtype=torch.int32, device=DEV)
    qd, kd, vd, gd, bd = (t.to(DEV) for t in (q, k, v, g.float(), beta.float()))
    os_ = []
    for t in range(T):
        os_.append(gdn.gdn_delta_rule_step(qd[t], kd[t], vd[t], gd[t], bd[t], cu, st, None, commit_state=True))
    o = torch.stack(os_, 1)                                   # [nseq, T, Hv, 128]
    torch.cuda.synchronize()
    # the oracle runs each sequence's 512 tokens as one sequence
    perm = lambda a: TL.np64(a.transpose(0, 1).reshape(nseq * T, *a.shape[2:]))  # noqa: E731
    cu_ref = [T * s for s in range(nseq + 1)]
    o_ref, st_ref = O.delta_rule_recurrent(perm(q), perm(k), perm(v), perm(g), perm(beta),
                                           TL.np64(state0), [1] * nseq, cu_ref, geo.Hk, geo.Hv)
    o_got = TL.np64(o).reshape(nseq * T, geo.Hv, 128)
    err = np.max(np.abs(o_got - o_ref), axis=2) / np.maximum(np.max(np.abs(o_ref), axis=2), 1e-30)
    per_block = [float(err[:, :][np.arange(nseq * T) % T // 64 == b].max()) for b in range(T // 64)]
    print(f"long chain ({gate}): worst o ratio per 64 steps {['%.2e' % x for x in per_block]}", flush=True)
    TL.check_normwise(o_got, o_ref, TL.REC_BF16, axes=(2,), what="o")
    ws = TL.check_normwise(TL.np64(st), st_ref, TL.REC_BF16, axes=(2, 3), what="final state")
    print(f"long chain ({gate}): final state worst ratio {ws:.2e}", flush=True)
    # no drift: the last 64 steps are no worse than a few times the first 128
    assert per_block[-1] <= max(3 * max(per_block[:2]), 1e-2), per_block
    # the chunked prefill over the same 512-token sequences (8 chunks each)
    cu_d = torch.tensor(cu_ref, dtype=torch.int32, device=DEV)
    st_p = state0.to(DEV)
    o_p = gdn.gdn_delta_rule_prefill(*(torch.from_numpy(perm(a)).to(torch.bfloat16).to(DEV).contiguous()
                                       for a in (q, k, v)),
                                     torch.from_numpy(perm(g)).float().to(DEV).contiguous(),
                                     torch.from_numpy(perm(beta)).float().to(DEV).contiguous(), cu_d, st_p)
    torch.cuda.synchronize()
    wp = TL.check_normwise(TL.np64(o_p), o_ref, TL.REC_BF16, axes=(2,), what="prefill o")
    wps = TL.check_normwise(TL.np64(st_p), st_ref, TL.REC_BF16, axes=(2, 3), what="prefill state")
    print(f"long chain ({gate}): prefill over the same tokens: worst o {wp:.2e}, state {wps:.2e}", flush=True)


# ---------------------------------------------------------------- empty sequences

EMPTY_LENGTHS = [0, 5, 0, 70, 0]
EMPTY_INIT = [0, 1, 1, 0, 0]


def _poisoned(lb):
    """Stored states of sequences without an initial state set to NaN."""
    cs = lb.conv_state.clone()
    st = lb.state.clone()
    for s, h in enumerate(lb.has_init.tolist()):
        if not h:
            cs[s] = float("nan")
            st[s] = float("nan")
    return cs, st


def _check_final_conv_rows(lb, cs_in, cs_gpu):
    ref_y, ref = O.causal_conv(TL.np64(lb.x), TL.np64(lb.conv_w), None, TL.np64(cs_in), lb.has_init.numpy(),
                               lb.cu_seqlens.tolist(), True)
    got = TL.np64(cs_gpu)
    assert np.isfinite(got).all()
    assert np.array_equal(got, ref)
    for s, (L, h) in enumerate(zip(np.diff(lb.cu_seqlens.numpy()), lb.has_init.tolist())):
        if L == 0 and not h:
            assert np.all(got[s] == 0)
        if L == 0 and h:
            assert torch.equal(cs_gpu[s].cpu(), cs_in[s])


def _check_final_states(lb, st_in, st_gpu, q, k, v, act):
    _, ref = O.delta_rule_recurrent(TL.np64(q), TL.np64(k), TL.np64(v), TL.np64(lb.g), TL.np64(lb.beta),
                                    TL.np64(st_in), lb.has_init.numpy(), lb.cu_seqlens.tolist(),
                                    lb.geo.Hk, lb.geo.Hv)
    got = TL.np64(st_gpu)
    assert np.isfinite(got).all()
    tol = TL.REC_F32 if act == "f32" else TL.REC_BF16
    TL.check_normwise(got, ref, tol, axes=(2, 3), what="state")
    for s, (L, h) in enumerate(zip(np.diff(lb.cu_seqlens.numpy()), lb.has_init.tolist())):
        if L == 0 and not h:
            assert np.all(got[s] == 0)
        if L == 0 and h:
            assert torch.equal(st_gpu[s].cpu(), st_in[s])


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("path", ["conv", "convpost", "convpost_derived"])
def test_empty_sequences_conv_final_rows(act, path):
    lb = I.make_layer(I.GEO_TINY, EMPTY_LENGTHS, act, 1800, state_std=0.3, has_init=EMPTY_INIT)
    cs_in, _ = _poisoned(lb)
    print(f"empty sequences: {path} {act}", flush=True)
    cu, hi, w, x = lb.cu_seqlens.to(DEV), lb.has_init.to(DEV), lb.conv_w.to(DEV), lb.x.to(DEV)
    cs = cs_in.to(DEV)
    chunks = gdn.gdn_make_chunks_device(cu, lb.N)
    if path == "conv":
        gdn.gdn_causal_conv_fwd(x, w, None, cs, hi, cu, chunks, True)
    else:
        gdn.gdn_conv_postconv_fwd(x, w, None, cs, hi, cu, chunks if path == "convpost" else None, True, 2, 4, 1e-6)
    torch.cuda.synchronize()
    _check_final_conv_rows(lb, cs_in, cs.cpu())
    # write_state = 0 writes nothing, NaN included
    cs2 = cs_in.to(DEV)
    if path == "conv":
        gdn.gdn_causal_conv_fwd(x, w, None, cs2, hi, cu, chunks, False)
    else:
        gdn.gdn_conv_postconv_fwd(x, w, None, cs2, hi, cu, chunks if path == "convpost" else None, False, 2, 4, 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(cs2.cpu().view(torch.int32), cs_in.view(torch.int32))


# the segmented prefill takes bf16 activations only
@pytest.mark.parametrize("path, act", [(p, a) for p in ("prefill", "step", "fused", "segmented")
                                       for a in ("f32", "bf16") if not (p == "segmented" and a == "f32")])
def test_empty_sequences_recurrent_final_state(act, path):
    lb = I.make_layer(I.GEO_TINY, EMPTY_LENGTHS, act, 1810, state_std=0.3, has_init=EMPTY_INIT)
    cs_in, st_in = _poisoned(lb)
    print(f"empty sequences: {path} {act}", flush=True)
    cu, hi, w, x = lb.cu_seqlens.to(DEV), lb.has_init.to(DEV), lb.conv_w.to(DEV), lb.x.to(DEV)
    cs, st = cs_in.to(DEV), st_in.to(DEV)
    g, beta = lb.g.to(DEV), lb.beta.to(DEV)
    if path == "fused":
        k = torch.empty(lb.N, 2, 128, dtype=x.dtype, device=DEV)
        v = torch.empty(lb.N, 4, 128, dtype=x.dtype, device=DEV)
        gdn.gdn_decode_fused(x, w, None, cs, cu, g, beta, st, 2, 4, 1e-6, hi, write_conv_state=True,
                             commit_state=True, k_out=k, v_out=v)
        torch.cuda.synchronize()
        _check_final_conv_rows(lb, cs_in, cs.cpu())
        q = None
    else:
        q, k, v = gdn.gdn_conv_postconv_fwd(x, w, None, cs, hi, cu, None, True, 2, 4, 1e-6)
        if path == "prefill":
            gdn.gdn_delta_rule_prefill(q, k, v, g, beta, cu, st, hi)
        elif path == "step":
            gdn.gdn_delta_rule_step(q, k, v, g, beta, cu, st, hi, commit_state=True)
        else:
            gdn.gdn_delta_rule_prefill_segmented(q, k, v, g, beta, cu, st, 3, hi)
        torch.cuda.synchronize()
    if q is not None:
        _check_final_states(lb, st_in, st.cpu(), q, k, v, act)
    else:
        # the fused path keeps q on chip (its bitwise equality with the three
        # calls is tested elsewhere): the zero / untouched rule exactly
        got = TL.np64(st.cpu())
        assert np.isfinite(got).all()
        for s, (L, h) in enumerate(zip(EMPTY_LENGTHS, EMPTY_INIT)):
            if L == 0 and not h:
                assert np.all(got[s] == 0)
            if L == 0 and h:
                assert torch.equal(st.cpu()[s], st_in[s])


@pytest.mark.parametrize("path", ["conv", "convpost", "step", "fused", "prefill"])
def test_batch_without_tokens_writes_only_zero_states(path):
    """N = 0 with two sequences: the one without an initial state gets zero
    final states, the other keeps its bits; no token buffer is touched."""
    geo = I.GEO_TINY
    lb = I.make_layer(geo, [0, 0], "bf16", 1820, state_std=0.3, has_init=[0, 1])
    cs_in, st_in = _poisoned(lb)
    cu, hi = lb.cu_seqlens.to(DEV), lb.has_init.to(DEV)
    cs, st = cs_in.to(DEV), st_in.to(DEV)
    x = torch.empty(0, geo.C, dtype=torch.bfloat16, device=DEV)
    w = lb.conv_w.to(DEV)
    q = torch.empty(0, 2, 128, dtype=torch.bfloat16, device=DEV)
    v = torch.empty(0, 4, 128, dtype=torch.bfloat16, device=DEV)
    g = torch.empty(0, 4, device=DEV)
    print(f"no tokens: {path}", flush=True)
    if path == "conv":
        gdn.gdn_causal_conv_fwd(x, w, None, cs, hi, cu, gdn.gdn_make_chunks_device(cu, 0), True)
    elif path == "convpost":
        gdn.gdn_conv_postconv_fwd(x, w, None, cs, hi, cu, None, True, 2, 4, 1e-6)
    elif path == "step":
        gdn.gdn_delta_rule_step(q, q, v, g, g, cu, st, hi, commit_state=True)
    elif path == "fused":
        gdn.gdn_decode_fused(x, w, None, cs, cu, g, g, st, 2, 4, 1e-6, hi)
    else:
        gdn.gdn_delta_rule_prefill(q, q, v, g, g, cu, st, hi)
    torch.cuda.synchronize()
    if path in ("conv", "convpost", "fused"):
        assert torch.all(cs[0].cpu() == 0)
        assert torch.equal(cs[1].cpu(), cs_in[1])
    if path in ("step", "fused", "prefill"):
        assert torch.all(st[0].cpu() == 0)
        assert torch.equal(st[1].cpu(), st_in[1])


# ------------------------------------------------ a batch cut into groups

SPLIT_LENGTHS = [300, 70, 0, 1, 129, 64, 500, 17]
SPLIT_INIT = [1, 0, 1, 1, 0, 1, 1, 0]
SPLIT_GROUPS = [(0, 2), (2, 5), (5, 8)]


@pytest.mark.parametrize("path", ["conv", "convpost", "prefill", "segmented", "step", "fused"])
def test_batch_split_into_consecutive_groups_equals_one_launch(path):
    """A batch cut into runs of consecutive sequences, each run launched on
    views of its own token rows, conv rows, states and flags with
    cu_seqlens rebased to its first token, gives the bits of one launch over
    the whole batch: a sequence's results depend on its own tokens and
    states only, not on the batch around it."""
    geo = I.Geometry(Hk=2, Hv=4)
    lb = I.make_layer(geo, SPLIT_LENGTHS, "bf16", 1840, state_std=0.3, has_init=SPLIT_INIT)
    Hk, Hv = geo.Hk, geo.Hv
    cuh = lb.cu_seqlens.tolist()
    x, w = lb.x.to(DEV), lb.conv_w.to(DEV)
    cu, hi = lb.cu_seqlens.to(DEV), lb.has_init.to(DEV)
    g, beta = lb.g.to(DEV).contiguous(), lb.beta.to(DEV).contiguous()
    cs0, st0 = lb.conv_state.to(DEV).contiguous(), lb.state.to(DEV).contiguous()
    q, k, v = gdn.gdn_conv_postconv_fwd(x, w, None, cs0.clone(), hi, cu, None, True, Hk, Hv, 1e-6)

    def launch(cu_, hi_, cs, st, x_, q_, k_, v_, g_, b_, o_):
        if path == "conv":   # y (in q_'s place) with the chunk list of this batch
            gdn.gdn_causal_conv_fwd(x_, w, None, cs, hi_, cu_, gdn.gdn_make_chunks_device(cu_, x_.shape[0]), True,
                                    y=q_)
        elif path == "fused":
            gdn.gdn_decode_fused(x_, w, None, cs, cu_, g_, b_, st, Hk, Hv, 1e-6, hi_, o=o_)
        elif path == "convpost":
            gdn.gdn_conv_postconv_fwd(x_, w, None, cs, hi_, cu_, None, True, Hk, Hv, 1e-6, q=q_, k=k_, v=v_)
        elif path == "prefill":
            gdn.gdn_delta_rule_prefill(q_, k_, v_, g_, b_, cu_, st, hi_, o=o_)
        elif path == "segmented":
            gdn.gdn_delta_rule_prefill_segmented(q_, k_, v_, g_, b_, cu_, st, 3, hi_, o=o_)
        else:
            gdn.gdn_delta_rule_step(q_, k_, v_, g_, b_, cu_, st, hi_, o=o_, commit_state=True)

    def outputs():
        if path == "conv":
            return torch.full_like(x, float("nan")), None, None
        if path == "convpost":
            return (torch.full_like(q, float("nan")), torch.full_like(k, float("nan")),
                    torch.full_like(v, float("nan")))
        return q, k, v

    print(f"batch split: {path}", flush=True)
    whole_cs, whole_st, whole_o = cs0.clone(), st0.clone(), torch.full_like(v, float("nan"))
    wq, wk, wv = outputs()
    launch(cu, hi, whole_cs, whole_st, x, wq, wk, wv, g, beta, whole_o)
    part_cs, part_st, part_o = cs0.clone(), st0.clone(), torch.full_like(v, float("nan"))
    pq, pk, pv = outputs()
    for s0, s1 in SPLIT_GROUPS:
        t0, t1 = cuh[s0], cuh[s1]
        cug = (cu[s0:s1 + 1] - t0).contiguous()
        cut = (lambda t: None if t is None else t[t0:t1])
        launch(cug, hi[s0:s1], part_cs[s0:s1], part_st[s0:s1], x[t0:t1], cut(pq), cut(pk), cut(pv),
               g[t0:t1], beta[t0:t1], part_o[t0:t1])
    torch.cuda.synchronize()
    if path in ("conv", "convpost"):
        for a, b, nm in ((wq, pq, "q / y"), (wk, pk, "k"), (wv, pv, "v")):
            if a is not None:
                assert torch.equal(a.view(torch.int16), b.view(torch.int16)), nm
        assert torch.equal(whole_cs.view(torch.int32), part_cs.view(torch.int32)), "conv_state"
    else:
        if path == "fused":
            assert torch.equal(whole_cs.view(torch.int32), part_cs.view(torch.int32)), "conv_state"
        assert torch.equal(whole_o.view(torch.int16), part_o.view(torch.int16)), "o"
        assert torch.equal(whole_st.view(torch.int32), part_st.view(torch.int32)), "state"
        assert torch.isfinite(whole_o.float()).all()


# ------------------------------------------ batches of more than 64 sequences

def test_batch_of_70_sequences():
    """70 sequences: past 64 the prefill runs them in index order instead
    of longest first, and the conv + post-conv needs chunk descriptors.
    The prefill is checked against the per-token oracle, and both launches
    must give the bits of the same batch cut into two runs of 35 sequences
    (the longest-first prefill and the in-launch chunk derivation)."""
    geo = I.Geometry(Hk=1, Hv=2)
    rng = np.random.default_rng(1870)
    lengths = [int(v) for v in rng.choice([0, 1, 2, 17, 63, 64, 65, 130], size=70)]
    hinit = [int(v) for v in rng.integers(0, 2, size=70)]
    lb = I.make_layer(geo, lengths, "bf16", 1870, state_std=0.3, has_init=hinit)
    Hk, Hv = geo.Hk, geo.Hv
    cuh = lb.cu_seqlens.tolist()
    x, w = lb.x.to(DEV), lb.conv_w.to(DEV)
    cu, hi = lb.cu_seqlens.to(DEV), lb.has_init.to(DEV)
    g, beta = lb.g.to(DEV).contiguous(), lb.beta.to(DEV).contiguous()
    cs0, st0 = lb.conv_state.to(DEV).contiguous(), lb.state.to(DEV).contiguous()
    print(f"70 sequences: {lb.N} tokens", flush=True)

    # whole batch: conv + post-conv with descriptors, then the prefill
    cs_w, st_w = cs0.clone(), st0.clone()
    q, k, v = gdn.gdn_conv_postconv_fwd(x, w, None, cs_w, hi, cu, gdn.gdn_make_chunks_device(cu, lb.N), True,
                                        Hk, Hv, 1e-6)
    o = gdn.gdn_delta_rule_prefill(q, k, v, g, beta, cu, st_w, hi)
    # two runs of 35 sequences (each on its own views, cu rebased)
    cs_p, st_p = cs0.clone(), st0.clone()
    qp, kp, vp = (torch.full_like(t, float("nan")) for t in (q, k, v))
    op = torch.full_like(o, float("nan"))
    for s0, s1 in ((0, 35), (35, 70)):
        t0, t1 = cuh[s0], cuh[s1]
        cug = (cu[s0:s1 + 1] - t0).contiguous()
        gdn.gdn_conv_postconv_fwd(x[t0:t1], w, None, cs_p[s0:s1], hi[s0:s1], cug, None, True, Hk, Hv, 1e-6,
                                  q=qp[t0:t1], k=kp[t0:t1], v=vp[t0:t1])
        gdn.gdn_delta_rule_prefill(qp[t0:t1], kp[t0:t1], vp[t0:t1], g[t0:t1], beta[t0:t1], cug, st_p[s0:s1],
                                   hi[s0:s1], o=op[t0:t1])
    torch.cuda.synchronize()
    for a, b, nm in ((q, qp, "q"), (k, kp, "k"), (v, vp, "v"), (o, op, "o")):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), nm
    assert torch.equal(cs_w.view(torch.int32), cs_p.view(torch.int32)), "conv_state"
    assert torch.equal(st_w.view(torch.int32), st_p.view(torch.int32)), "state"

    o_ref, st_ref = O.delta_rule_recurrent(TL.np64(q), TL.np64(k), TL.np64(v), TL.np64(lb.g),
                                           TL.np64(lb.beta), TL.np64(lb.state), lb.has_init.numpy(),
                                           cuh, Hk, Hv)
    TL.check_normwise(TL.np64(o), o_ref, TL.REC_BF16, axes=(2,), what="o")
    TL.check_normwise(TL.np64(st_w), st_ref, TL.REC_BF16, axes=(2, 3), what="state")
