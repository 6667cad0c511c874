"""Stage-by-stage parity of the HIP library against the CPU oracle, at sizes
the oracle finishes in seconds, spanning several tiles / chunks with ragged
tails, plus the edge cases of each stage.  Every call goes through the C ABI
(the ctypes binding).  Stage isolation: each oracle stage consumes the GPU's
own output of the previous stage."""
import numpy as np
import pytest
import torch

import gdn_testlib as TL
from oracle import gdn_oracle as O

pytestmark = pytest.mark.gpu

gdn = pytest.importorskip("linear_attention_layers_amd.gdn")
from linear_attention_layers_amd import inputs as I  # noqa: E402

DEV = "cuda"


def _cu(lengths):
    return I.cu_from_lengths(lengths)


# ---------------------------------------------------------------- chunks

@pytest.mark.parametrize("lengths", [[1], [64], [65], [0, 5, 0, 130, 3], [2048] * 3 + [1] * 5,
                                     list(range(0, 300, 7)),
                                     [int(x) for x in np.random.default_rng(3).integers(0, 150, 700)]])
def test_make_chunks_device_bit_exact(lengths):
    cu = _cu(lengths)
    out = gdn.gdn_make_chunks_device(cu.to(DEV), int(cu[-1]))
    ref = O.make_chunks(cu.tolist(), 64)
    got = out.cpu().numpy()
    assert got.shape[0] == gdn.gdn_chunk_capacity(int(cu[-1]), len(lengths))
    assert np.array_equal(got[:len(ref)], ref)
    assert np.all(got[len(ref):, 0] == -1)
    host = gdn.gdn_make_chunks(cu.tolist()).numpy()
    assert np.array_equal(host, ref)


# ---------------------------------------------------------------- conv

CONV_CASES = [
    # act, geometry, lengths, has_init, bias_std, row_pad
    ("f32", I.GEO_TINY, [64], [1], 0.0, 0),
    ("bf16", I.GEO_TINY, [1, 2, 3, 63, 64, 65, 129, 200], [1, 0, 1, 0, 1, 1, 0, 1], 0.3, 0),
    ("f32", I.Geometry(Hk=1, Hv=1), [5, 70, 2, 1], [0, 1, 1, 1], 0.5, 8),
    ("bf16", I.Geometry(Hk=5, Hv=15), [130, 7, 64], [1, 1, 0], 0.0, 16),
]


def _conv_ref(lb, conv_state_in, write_state):
    x = TL.np64(lb.x)
    hi = lb.has_init.numpy()
    cu = lb.cu_seqlens.tolist()
    b = None if lb.conv_b is None else TL.np64(lb.conv_b)
    y, st = O.causal_conv(x, TL.np64(lb.conv_w), b, TL.np64(conv_state_in), hi, cu, write_state)
    scale = TL.conv_scale(x, TL.np64(lb.conv_w), b, TL.np64(conv_state_in), hi, cu)
    return y, st, scale


@pytest.mark.parametrize("case", range(len(CONV_CASES)))
@pytest.mark.parametrize("write_state", [True, False])
def test_conv_parity(case, write_state):
    act, geo, lengths, hinit, bias_std, pad = CONV_CASES[case]
    lb = I.make_layer(geo, lengths, act, 100 + case, bias_std=bias_std, has_init=hinit,
                      x_row_pad=pad)
    # poison the stored rows of sequences without initial state
    cs0 = lb.conv_state.clone()
    for s, h in enumerate(hinit):
        if not h:
            cs0[s] = float("nan")
    cs = cs0.to(DEV)
    xd = lb.x.to(DEV) if pad == 0 else _padded_to_device(lb)
    cu = lb.cu_seqlens.to(DEV)
    chunks = gdn.gdn_make_chunks_device(cu, lb.N)
    y = gdn.gdn_causal_conv_fwd(xd, lb.conv_w.to(DEV), TL.dev(lb.conv_b), cs,
                                lb.has_init.to(DEV), cu, chunks, write_state)
    torch.cuda.synchronize()
    y_ref, st_ref, scale = _conv_ref(lb, cs0, write_state)
    assert np.all(np.isfinite(TL.np64(y)))
    TL.check_conv(TL.np64(y), y_ref, scale, act)
    got_st = cs.cpu().numpy().astype(np.float64)
    if write_state:
        assert np.array_equal(got_st, st_ref)          # exact copies of inputs
    else:
        assert np.array_equal(np.isnan(got_st), np.isnan(cs0.numpy()))
        assert np.array_equal(np.nan_to_num(got_st), np.nan_to_num(cs0.numpy().astype(np.float64)))


def _padded_to_device(lb):
    """Re-create the padded row storage on the device (stride > C)."""
    N, C = lb.x.shape
    stride = lb.x.stride(0)
    full = torch.zeros(N, stride, dtype=lb.x.dtype)
    full[:, :C] = lb.x
    return full.to(DEV)[:, :C]


def test_conv_delta_kernel_is_an_exact_shift():
    geo = I.Geometry(Hk=1, Hv=1)
    lb = I.make_layer(geo, [3, 1, 70], "bf16", 7)
    C = geo.C
    for shift in range(4):
        w = torch.zeros(C, 4)
        w[:, 3 - shift] = 1.0
        cs = lb.conv_state.to(DEV)
        cu = lb.cu_seqlens.to(DEV)
        y = gdn.gdn_causal_conv_fwd(lb.x.to(DEV), w.to(DEV), None, cs, None, cu,
                                    gdn.gdn_make_chunks_device(cu, lb.N), False)
        y_ref, _ = O.causal_conv(TL.np64(lb.x), w.numpy(), None, TL.np64(lb.conv_state), [1, 1, 1],
                                 lb.cu_seqlens.tolist(), False)
        assert np.array_equal(TL.np64(y), O.round_to_bf16(y_ref))


@pytest.mark.parametrize("order", ["reversed", "shuffled"])
def test_conv_state_in_place_is_race_free(order):
    """Sequences longer than one chunk with initial state, in place, with the
    chunk list reordered: every repetition must match the oracle exactly."""
    lb = I.make_layer(I.GEO_TINY, [200, 65, 64, 300, 5], "bf16", 11)
    host = gdn.gdn_make_chunks(lb.cu_seqlens.tolist())
    idx = torch.arange(host.shape[0] - 1, -1, -1) if order == "reversed" else \
        torch.randperm(host.shape[0], generator=torch.Generator().manual_seed(5))
    chunks = host[idx].contiguous().to(DEV)
    cu = lb.cu_seqlens.to(DEV)
    x = lb.x.to(DEV)
    w = lb.conv_w.to(DEV)
    y_ref, st_ref, scale = _conv_ref(lb, lb.conv_state, True)
    y_first = None
    for rep in range(100):
        cs = lb.conv_state.to(DEV)
        y = gdn.gdn_causal_conv_fwd(x, w, None, cs, None, cu, chunks, True)
        got = cs.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, st_ref), f"repetition {rep}"
        if y_first is None:
            y_first = y.clone()
            TL.check_conv(TL.np64(y), y_ref, scale, "bf16")
        else:
            assert torch.equal(y, y_first)


def test_conv_two_calls_equal_one():
    lb = I.make_layer(I.GEO_TINY, [150], "bf16", 12)
    cu_all = lb.cu_seqlens.to(DEV)
    w = lb.conv_w.to(DEV)
    cs_a = lb.conv_state.to(DEV)
    y_all = gdn.gdn_causal_conv_fwd(lb.x.to(DEV), w, None, cs_a, None, cu_all,
                                    gdn.gdn_make_chunks_device(cu_all, 150), True)
    for split in (1, 2, 3, 64, 100):
        cs_b = lb.conv_state.to(DEV)
        parts = []
        for (a, b) in ((0, split), (split, 150)):
            cu = torch.tensor([0, b - a], dtype=torch.int32, device=DEV)
            parts.append(gdn.gdn_causal_conv_fwd(lb.x[a:b].contiguous().to(DEV), w, None, cs_b, None,
                                                 cu, gdn.gdn_make_chunks_device(cu, b - a), True))
        assert torch.equal(torch.cat(parts), y_all)
        assert torch.equal(cs_b, cs_a)


# ---------------------------------------------------------------- post-conv

def _y(geo, N, act, scale=2.0, seed=0, lo=None, hi=None):
    g = torch.Generator().manual_seed(seed)
    if lo is not None:
        y = lo + (hi - lo) * torch.rand(N, geo.C, generator=g)
    else:
        y = torch.randn(N, geo.C, generator=g) * scale
    return y.to(TL.ACT[act])


@pytest.mark.parametrize("act_in", ["f32", "bf16"])
def test_postconv_f32_arm_matches_documented_order(act_in):
    geo = I.Geometry(Hk=3, Hv=6)
    y = _y(geo, 300, act_in, seed=1)
    q, k, v = gdn.gdn_postconv_l2(y.to(DEV), geo.Hk, geo.Hv, 1e-6, out_dtype=torch.float32)
    qr, kr, vr = O.postconv_l2_f32_tree(TL.np64(y), geo.Hk, geo.Hv, 128, 128, 1e-6)
    for got, ref in ((q, qr), (k, kr)):
        d = TL.ulp_dist_f32(got.cpu().numpy(), ref)
        assert d.max() <= TL.L2_ULP_F32, f"max ulp {d.max()}"
    s_ref = O.silu(TL.np64(y))[:, 2 * geo.Hk * 128:].reshape(300, geo.Hv, 128)
    np.testing.assert_allclose(v.cpu().numpy(), s_ref, rtol=TL.SILU_REL_F32, atol=0)
    assert np.array_equal(v.cpu().numpy(), vr)


def test_postconv_silu_identity_region_pins_the_order_exactly():
    """y in [20, 40]: SiLU(y) == y in float32, so q_hat depends only on the
    summation order; it must equal the oracle's documented order bit for bit."""
    geo = I.Geometry(Hk=4, Hv=4)
    y = _y(geo, 2000, "f32", seed=2, lo=20.0, hi=40.0)
    q, k, v = gdn.gdn_postconv_l2(y.to(DEV), geo.Hk, geo.Hv, 1e-6, out_dtype=torch.float32)
    qr, kr, vr = O.postconv_l2_f32_tree(TL.np64(y), geo.Hk, geo.Hv, 128, 128, 1e-6)
    assert np.array_equal(q.cpu().numpy(), qr)
    assert np.array_equal(k.cpu().numpy(), kr)
    assert np.array_equal(v.cpu().numpy(), y[:, 8 * 128:].reshape(2000, 4, 128).numpy())


@pytest.mark.parametrize("act_in", ["f32", "bf16"])
def test_postconv_bf16_output_within_one_step(act_in):
    geo = I.GEO_8192
    y = _y(geo, 96, act_in, seed=3)
    q, k, v = gdn.gdn_postconv_l2(y.to(DEV), geo.Hk, geo.Hv, 1e-6, out_dtype=torch.bfloat16)
    qr, kr, vr = O.postconv_l2(TL.np64(y), geo.Hk, geo.Hv, 128, 128, np.float64(np.float32(1e-6)))
    for got, ref in ((q, qr), (k, kr), (v, vr)):
        d = TL.ulp_dist_bf16(got.float().cpu().numpy(), O.round_to_bf16(ref).astype(np.float32))
        assert d.max() <= TL.L2_ULP_BF16


def test_postconv_closed_forms_and_zero_head():
    geo = I.Geometry(Hk=2, Hv=2)
    y = _y(geo, 40, "f32", seed=4)
    y[3, :128] = -1e4                     # SiLU = -0 on a whole q head
    eps = 1e-3
    q, k, v = gdn.gdn_postconv_l2(y.to(DEV), geo.Hk, geo.Hv, eps, out_dtype=torch.float32)
    s = O.silu(TL.np64(y))
    sq, sk, _ = O.split_heads(s, geo.Hk, geo.Hv, 128, 128)
    for got, raw in ((q, sq), (k, sk)):
        sig = np.sum(raw ** 2, axis=-1)
        np.testing.assert_allclose(np.linalg.norm(got.cpu().numpy().astype(np.float64), axis=-1),
                                   np.sqrt(sig / (sig + eps)), rtol=2e-6)
    assert np.all(q[3, 0].cpu().numpy() == 0)


# ---------------------------------------------------------------- recurrence

def _rec_inputs(act, geo, lengths, has_init, seed, state_std=0.3, gate="softplus"):
    """Run conv + post-conv on the GPU and return the recurrence inputs."""
    lb = I.make_layer(geo, lengths, act, seed, state_std=state_std, has_init=has_init, gate=gate)
    out = TL.gpu_layer(lb)
    return lb, out


def _rec_ref(lb, out, state_in=None):
    hi = lb.has_init.numpy()
    st = TL.np64(lb.state if state_in is None else state_in)
    return O.delta_rule_recurrent(TL.np64(out["q"]), TL.np64(out["k"]), TL.np64(out["v"]),
                                  TL.np64(lb.g), TL.np64(lb.beta), st, hi,
                                  lb.cu_seqlens.tolist(), lb.geo.Hk, lb.geo.Hv)


REC_CASES = [
    ("f32", I.GEO_TINY, [64], [1]),
    ("f32", I.GEO_TINY, [1, 2, 3, 63, 65, 129], [1, 0, 1, 1, 0, 1]),
    ("bf16", I.GEO_TINY, [1, 2, 3, 63, 64, 65, 129, 200], [1, 0, 1, 0, 1, 1, 0, 1]),
    ("bf16", I.Geometry(Hk=1, Hv=3), [130, 7], [1, 0]),
    ("bf16", I.Geometry(Hk=2, Hv=2), [300], [1]),
    # 6 sequences x 32 v-heads, lengths unsorted (longest-first dispatch)
    ("bf16", I.GEO_8192, [1, 63, 65, 130, 200, 7], [1, 0, 1, 1, 0, 1]),
    # more sequences than the longest-first ordering handles (kept in order)
    ("bf16", I.GEO_TINY, [(7 * i) % 41 + 1 for i in range(70)], [i % 2 for i in range(70)]),
]


@pytest.mark.parametrize("case", range(len(REC_CASES)))
def test_prefill_parity(case):
    act, geo, lengths, hinit = REC_CASES[case]
    lb, out = _rec_inputs(act, geo, lengths, hinit, 200 + case)
    torch.cuda.synchronize()
    o_ref, st_ref = _rec_ref(lb, out)
    tol = TL.REC_F32 if act == "f32" else TL.REC_BF16
    TL.check_normwise(TL.np64(out["o"]), o_ref, tol, axes=(2,), what="o")
    TL.check_normwise(TL.np64(out["state"]), st_ref, tol, axes=(2, 3), what="state")


def test_prefill_ignores_poisoned_state_without_init():
    geo = I.GEO_TINY
    lb = I.make_layer(geo, [70, 5], "bf16", 300, state_std=0.3, has_init=[0, 0])
    lb.state[:] = float("nan")
    out = TL.gpu_layer(lb)
    assert torch.isfinite(out["o"].float()).all() and torch.isfinite(out["state"]).all()


def _step_run(act, geo, lengths, hinit, seed, commit):
    lb = I.make_layer(geo, lengths, act, seed, state_std=0.3, has_init=hinit)
    cu = lb.cu_seqlens.to(DEV)
    hi = lb.has_init.to(DEV)
    cs = lb.conv_state.to(DEV)
    y = gdn.gdn_causal_conv_fwd(lb.x.to(DEV), lb.conv_w.to(DEV), None, cs, hi, cu,
                                gdn.gdn_make_chunks_device(cu, lb.N), commit)
    q, k, v = gdn.gdn_postconv_l2(y, geo.Hk, geo.Hv, 1e-6)
    st = lb.state.to(DEV)
    g, beta = lb.g.to(DEV), lb.beta.to(DEV)
    o = gdn.gdn_delta_rule_step(q, k, v, g, beta, cu, st, hi, commit_state=commit)
    return lb, dict(q=q, k=k, v=v, o=o, state=st, g=g, beta=beta, cu=cu, hi=hi, x=lb.x.to(DEV),
                    conv_state=cs)


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("commit", [True, False])
def test_step_parity(act, commit):
    geo = I.GEO_TINY
    lengths = [1, 2, 5, 8, 3, 1]
    hinit = [1, 1, 0, 1, 1, 0]
    lb, out = _step_run(act, geo, lengths, hinit, 400, commit)
    torch.cuda.synchronize()
    o_ref, st_ref = _rec_ref(lb, out)
    tol = TL.REC_F32 if act == "f32" else TL.REC_BF16
    TL.check_normwise(TL.np64(out["o"]), o_ref, tol, axes=(2,), what="o")
    if commit:
        TL.check_normwise(TL.np64(out["state"]), st_ref, tol, axes=(2, 3), what="state")
    else:
        assert torch.equal(out["state"].cpu(), lb.state)


def test_step_window_agrees_with_single_token_steps():
    """T tokens in one call and T one-token calls evaluate the same
    recurrence with a different association (a call's window runs its
    products on MFMA over all of its tokens at once): equal within the
    recurrence bound, token by token and for the final state."""
    geo = I.GEO_TINY
    lengths = [1, 4, 8, 2, 16, 19]
    lb, out = _step_run("bf16", geo, lengths, [1, 1, 1, 0, 1, 1], 500, True)
    cu = lb.cu_seqlens.tolist()
    for s in range(len(lengths)):
        st = lb.state[s:s + 1].to(DEV).contiguous()
        for t in range(cu[s], cu[s + 1]):
            sl = slice(t, t + 1)
            init = torch.tensor([1 if (t > cu[s] or lb.has_init[s]) else 0], dtype=torch.uint8,
                                device=DEV)
            one = torch.tensor([0, 1], dtype=torch.int32, device=DEV)
            o1 = gdn.gdn_delta_rule_step(out["q"][sl].contiguous(), out["k"][sl].contiguous(),
                                         out["v"][sl].contiguous(), out["g"][sl].contiguous(),
                                         out["beta"][sl].contiguous(), one, st, init,
                                         commit_state=True)
            TL.check_normwise(TL.np64(o1), TL.np64(out["o"][sl]), TL.REC_BF16, axes=(2,),
                              what=f"seq {s} token {t}")
        TL.check_normwise(TL.np64(st[0]), TL.np64(out["state"][s]), TL.REC_BF16, axes=(1, 2),
                          what=f"seq {s} state")


def test_step_single_token_window_matches_per_token_formula_f32():
    """One-token windows in float32: o = a S q + d (k . q) with
    d = b (v - a S k), the per-token update written out, to the float32
    recurrence bound."""
    geo = I.GEO_TINY
    lengths = [1, 1, 1]
    lb, out = _step_run("f32", geo, lengths, [1, 1, 1], 510, True)
    torch.cuda.synchronize()
    S = TL.np64(lb.state)
    q, k, v = TL.np64(out["q"]), TL.np64(out["k"]), TL.np64(out["v"])
    g, b = TL.np64(lb.g), TL.np64(lb.beta)
    for s in range(3):
        for h in range(geo.Hv):
            kh = h // (geo.Hv // geo.Hk)
            a = np.exp(g[s, h])
            u = S[s, h] @ k[s, kh]
            d = b[s, h] * (v[s, h] - a * u)
            o_ref = a * (S[s, h] @ q[s, kh]) + d * (k[s, kh] @ q[s, kh])
            st_ref = a * S[s, h] + np.outer(d, k[s, kh])
            TL.check_normwise(TL.np64(out["o"][s, h])[None], o_ref[None], TL.REC_F32, axes=(1,),
                              what="o")
            TL.check_normwise(TL.np64(out["state"][s, h])[None], st_ref[None], TL.REC_F32,
                              axes=(1, 2), what="state")


def test_prefill_and_step_agree_within_tolerance():
    """The chunked and the per-token forms are both correct: not bitwise equal,
    but within the recurrence bound of each other."""
    geo = I.GEO_TINY
    lb = I.make_layer(geo, [1, 8, 64, 100], "bf16", 600, state_std=0.3)
    out = TL.gpu_layer(lb)
    st2 = lb.state.to(DEV)
    o2 = gdn.gdn_delta_rule_step(out["q"], out["k"], out["v"], out["g"], out["beta"], out["cu"],
                                 st2, out["hi"], commit_state=True)
    TL.check_normwise(TL.np64(out["o"]), TL.np64(o2), TL.REC_BF16, axes=(2,), what="o")
    TL.check_normwise(TL.np64(out["state"]), TL.np64(st2), TL.REC_BF16, axes=(2, 3), what="state")


# ---------------------------------------------------------------- commit

def test_commit_parity_and_bitwise_equal_to_step_commit():
    geo = I.GEO_TINY
    L = 3
    lengths = [1, 8, 5, 3, 7, 2]
    n_keep = [0, 8, 2, 3, 0, 1]
    hinit = [1, 1, 1, 0, 1, 1]
    layers, runs = [], []
    for layer in range(L):
        lb, out = _step_run("bf16", geo, lengths, hinit, 700 + 10 * layer, False)
        runs.append((lb, out))
        layers.append(dict(x=out["x"], conv_state=out["conv_state"], state=out["state"],
                           k=out["k"], v=out["v"], g=out["g"], beta=out["beta"]))
    table = gdn.gdn_layer_table(layers, DEV)
    nk = torch.tensor(n_keep, dtype=torch.int32, device=DEV)
    cu = runs[0][1]["cu"]
    hi = runs[0][1]["hi"]
    gdn.gdn_commit(table, L, cu, nk, hi, geo.C, geo.Hk, geo.Hv, torch.bfloat16)
    torch.cuda.synchronize()
    # the kept tokens, packed, for the reference forward with commit
    keep_idx = torch.cat([torch.arange(c, c + n) for c, n in zip(lb.cu_seqlens[:-1].tolist(), n_keep)])
    cu_keep = I.cu_from_lengths(n_keep).to(DEV)
    for layer, (lb, out) in enumerate(runs):
        # oracle
        cs_ref, st_ref = O.commit(TL.np64(lb.x), TL.np64(lb.conv_state), TL.np64(lb.state),
                                  TL.np64(out["k"]), TL.np64(out["v"]), TL.np64(lb.g),
                                  TL.np64(lb.beta), lb.has_init.numpy(), lb.cu_seqlens.tolist(),
                                  n_keep, geo.Hk, geo.Hv)
        assert np.array_equal(out["conv_state"].cpu().numpy().astype(np.float64), cs_ref)
        TL.check_normwise(TL.np64(out["state"]), st_ref, TL.REC_BF16, axes=(2, 3), what="state")
        # n = 0 leaves the state untouched bit for bit
        for s, n in enumerate(n_keep):
            if n == 0:
                assert torch.equal(out["state"][s].cpu(), lb.state[s])
                assert torch.equal(out["conv_state"][s].cpu(), lb.conv_state[s])
        # bitwise equal to a committing step / conv over the kept tokens
        kd = keep_idx.to(DEV)
        st2 = lb.state.to(DEV)
        gdn.gdn_delta_rule_step(out["q"][kd].contiguous(), out["k"][kd].contiguous(),
                                out["v"][kd].contiguous(), out["g"][kd].contiguous(),
                                out["beta"][kd].contiguous(), cu_keep, st2, hi, commit_state=True)
        cs2 = lb.conv_state.to(DEV)
        xk = out["x"][kd].contiguous()
        gdn.gdn_causal_conv_fwd(xk, lb.conv_w.to(DEV), None, cs2, hi, cu_keep,
                                gdn.gdn_make_chunks_device(cu_keep, int(sum(n_keep))), True)
        assert torch.equal(st2, out["state"]), f"layer {layer}"
        assert torch.equal(cs2, out["conv_state"]), f"layer {layer}"


# ---------------------------------------------------------------- fused decode

FUSED_CASES = [
    # act, geometry, lengths, has_init, write_conv_state, commit_state, bias_std
    ("bf16", I.Geometry(Hk=2, Hv=4), [1, 3, 8, 0, 5, 2], [1, 1, 0, 1, 1, 0], True, True, 0.0),
    ("bf16", I.Geometry(Hk=2, Hv=4), [1, 3, 8, 0, 5, 2], [1, 1, 0, 1, 1, 0], False, False, 0.3),
    ("bf16", I.Geometry(Hk=2, Hv=2), [1, 1, 1, 2], [1, 1, 1, 1], True, True, 0.0),
    ("bf16", I.Geometry(Hk=1, Hv=2), [17, 33, 4], [1, 0, 1], True, False, 0.0),
    ("bf16", I.GEO_8192, [1, 1, 4, 1], [1, 1, 1, 0], True, True, 0.0),
    ("f32", I.Geometry(Hk=2, Hv=4), [1, 7, 2, 16], [1, 0, 1, 1], True, True, 0.2),
    ("f32", I.Geometry(Hk=2, Hv=2), [3, 1], [0, 1], False, True, 0.0),
    ("f32", I.Geometry(Hk=1, Hv=1), [20, 0, 1], [1, 1, 0], True, True, 0.0),
]


@pytest.mark.parametrize("case", range(len(FUSED_CASES)))
def test_decode_fused_bitwise_equal_to_three_calls(case):
    act, geo, lengths, hinit, wcs, commit, bias_std = FUSED_CASES[case]
    lb = I.make_layer(geo, lengths, act, 800 + case, state_std=0.3, has_init=hinit,
                      bias_std=bias_std)
    cu = lb.cu_seqlens.to(DEV)
    hi = lb.has_init.to(DEV)
    x, w, b = lb.x.to(DEV), lb.conv_w.to(DEV), TL.dev(lb.conv_b)
    g, beta = lb.g.to(DEV), lb.beta.to(DEV)
    # the three calls
    cs1, st1 = lb.conv_state.to(DEV), lb.state.to(DEV)
    y = gdn.gdn_causal_conv_fwd(x, w, b, cs1, hi, cu, gdn.gdn_make_chunks_device(cu, lb.N), wcs)
    q, k, v = gdn.gdn_postconv_l2(y, geo.Hk, geo.Hv, 1e-6)
    o1 = gdn.gdn_delta_rule_step(q, k, v, g, beta, cu, st1, hi, commit_state=commit)
    # one fused call
    cs2, st2 = lb.conv_state.to(DEV), lb.state.to(DEV)
    keep_kv = case % 2 == 0
    k2 = torch.full_like(k, float("nan")) if keep_kv else None
    v2 = torch.full_like(v, float("nan")) if keep_kv else None
    o2 = gdn.gdn_decode_fused(x, w, b, cs2, cu, g, beta, st2, geo.Hk, geo.Hv, 1e-6, hi,
                              write_conv_state=wcs, commit_state=commit, k_out=k2, v_out=v2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    if keep_kv:
        assert torch.equal(k, k2) and torch.equal(v, v2)
    assert torch.equal(st1, st2)
    assert torch.equal(cs1, cs2)
    if not commit:
        assert torch.equal(st2.cpu(), lb.state)
    if not wcs:
        assert torch.equal(cs2.cpu(), lb.conv_state)


def test_decode_fused_matches_oracle():
    geo = I.Geometry(Hk=2, Hv=4)
    lengths, hinit = [1, 4, 8, 3], [1, 0, 1, 1]
    lb = I.make_layer(geo, lengths, "bf16", 850, state_std=0.3, has_init=hinit)
    cu = lb.cu_seqlens.to(DEV)
    cs, st = lb.conv_state.to(DEV), lb.state.to(DEV)
    o = gdn.gdn_decode_fused(lb.x.to(DEV), lb.conv_w.to(DEV), None, cs, cu, lb.g.to(DEV),
                             lb.beta.to(DEV), st, geo.Hk, geo.Hv, 1e-6, lb.has_init.to(DEV))
    torch.cuda.synchronize()
    hi = lb.has_init.numpy()
    cu_l = lb.cu_seqlens.tolist()
    y_ref, cs_ref = O.causal_conv(TL.np64(lb.x), TL.np64(lb.conv_w), None, TL.np64(lb.conv_state),
                                  hi, cu_l, True)
    assert np.array_equal(TL.np64(cs), cs_ref)
    qr, kr, vr = O.postconv_l2(O.round_to_bf16(y_ref), geo.Hk, geo.Hv, 128, 128, 1e-6)
    o_ref, st_ref = O.delta_rule_recurrent(O.round_to_bf16(qr), O.round_to_bf16(kr),
                                           O.round_to_bf16(vr), TL.np64(lb.g), TL.np64(lb.beta),
                                           TL.np64(lb.state), hi, cu_l, geo.Hk, geo.Hv)
    TL.check_normwise(TL.np64(o), o_ref, TL.REC_BF16, axes=(2,), what="o")
    TL.check_normwise(TL.np64(st), st_ref, TL.REC_BF16, axes=(2, 3), what="state")


# ---------------------------------------------------------------- output norm

def _out_norm_inputs(act, N, Hv, seed, with_w=True):
    g = torch.Generator().manual_seed(seed)
    dt = TL.ACT[act]
    o = (torch.randn(N, Hv, 128, generator=g) * 1.7).to(dt)
    z = (torch.randn(N, Hv, 128, generator=g) * 2.0).to(dt)
    w = (0.5 + torch.rand(128, generator=g)) if with_w else None
    return o, z, w


def _out_norm_check(act, o, z, w, y, eps=1e-6):
    ref = O.out_norm_gated(TL.np64(o), TL.np64(z), None if w is None else TL.np64(w), np.float64(np.float32(eps)))
    got = TL.np64(y)
    if act == "f32":
        np.testing.assert_allclose(got, ref, rtol=2e-6, atol=1e-30)
    else:
        d = TL.ulp_dist_bf16(y.float().cpu().numpy(), O.round_to_bf16(ref).astype(np.float32))
        assert d.max() <= 1, f"max bf16 ulp distance {d.max()}"


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("with_w", [True, False])
@pytest.mark.parametrize("N,Hv", [(1, 1), (37, 3), (64, 16)])
def test_out_norm_parity(act, with_w, N, Hv):
    o, z, w = _out_norm_inputs(act, N, Hv, 900 + N + Hv, with_w)
    y = gdn.gdn_out_norm(o.to(DEV), z.to(DEV), TL.dev(w), 1e-6)
    torch.cuda.synchronize()
    _out_norm_check(act, o, z, w, y)


def test_out_norm_in_place_equals_out_of_place():
    o, z, w = _out_norm_inputs("bf16", 45, 5, 950)
    od, zd, wd = o.to(DEV), z.to(DEV), w.to(DEV)
    y = gdn.gdn_out_norm(od, zd, wd, 1e-6)
    o2 = od.clone()
    r = gdn.gdn_out_norm(o2, zd, wd, 1e-6, y=o2)
    torch.cuda.synchronize()
    assert r.data_ptr() == o2.data_ptr()
    assert torch.equal(y, o2)


def test_out_norm_mixed_serving_size():
    lb = I.mixed_serving_layer(0)
    N, Hv = lb.N, lb.geo.Hv
    o, z, w = _out_norm_inputs("bf16", N, Hv, 960)
    y = gdn.gdn_out_norm(o.to(DEV), z.to(DEV), w.to(DEV), 1e-6)
    torch.cuda.synchronize()
    _out_norm_check("bf16", o, z, w, y)


def test_out_norm_zero_rows_and_zero_gate():
    o = torch.zeros(3, 2, 128, dtype=torch.bfloat16)
    z = torch.randn(3, 2, 128).to(torch.bfloat16)
    o[1] = torch.randn(2, 128).to(torch.bfloat16)
    z[2] = 0
    y = gdn.gdn_out_norm(o.to(DEV), z.to(DEV), None, 1e-6)
    torch.cuda.synchronize()
    yc = y.cpu()
    assert torch.all(yc[0] == 0) and torch.all(yc[2] == 0)
    assert torch.isfinite(yc.float()).all()


# ---------------------------------------------------------------- gates

def _gates_inputs(act, N, Hv, seed, scale=2.0):
    g = torch.Generator().manual_seed(seed)
    ba = (torch.randn(N, Hv, 2, generator=g) * scale).to(TL.ACT[act])
    A_log = torch.log(1.0 + 15.0 * torch.rand(Hv, generator=g))
    dt = torch.randn(Hv, generator=g)
    return ba, A_log, dt


def _gates_check(ba, A_log, dt, g, beta):
    g_ref, b_ref = O.gates(TL.np64(ba), TL.np64(A_log), TL.np64(dt))
    np.testing.assert_allclose(TL.np64(g), g_ref, rtol=4e-6, atol=1e-30)
    np.testing.assert_allclose(TL.np64(beta), b_ref, rtol=4e-6, atol=1e-30)


@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("N,Hv", [(1, 1), (37, 3), (5252, 32)])
def test_gates_parity(act, N, Hv):
    ba, A_log, dt = _gates_inputs(act, N, Hv, 970 + N + Hv)
    g, beta = gdn.gdn_gates(ba.to(DEV), A_log.to(DEV), dt.to(DEV))
    torch.cuda.synchronize()
    _gates_check(ba, A_log, dt, g, beta)


def test_gates_extreme_inputs():
    ba = torch.tensor([[[30.0, 30.0], [-30.0, -30.0], [0.0, 19.5], [0.0, 20.5], [88.0, -88.0], [-88.0, 100.0]]])
    A_log = torch.zeros(6)
    dt = torch.zeros(6)
    g, beta = gdn.gdn_gates(ba.to(DEV), A_log.to(DEV), dt.to(DEV))
    torch.cuda.synchronize()
    assert torch.isfinite(g).all() and torch.isfinite(beta).all()
    assert (g <= 0).all() and (beta >= 0).all() and (beta <= 1).all()
    _gates_check(ba, A_log, dt, g, beta)


# ------------------------------------------------ conv + post-conv in one launch

# (act, geometry, lengths, has_init, bias, x row padding)
CP_CASES = [
    ("f32", I.GEO_TINY, [1, 2, 3, 64, 65, 130], [1, 0, 1, 1, 0, 1], False, 0),
    ("bf16", I.GEO_TINY, [1, 2, 3, 63, 64, 65, 129, 200], [1, 0, 1, 0, 1, 1, 0, 1], True, 0),
    ("bf16", I.Geometry(Hk=1, Hv=1), [70, 5], [1, 1], True, 0),      # C = 384: half a channel group
    ("bf16", I.Geometry(Hk=2, Hv=2), [300], [0], False, 64),          # x rows wider than C
    ("bf16", I.GEO_8192, [1, 63, 65, 130, 200, 7], [1, 0, 1, 1, 0, 1], False, 0),
    ("f32", I.Geometry(Hk=1, Hv=3), [3, 150], [1, 0], True, 8),
]


def _cp_inputs(case):
    act, geo, lengths, hinit, with_bias, pad = CP_CASES[case]
    lb = I.make_layer(geo, lengths, act, 800 + case, state_std=0.3, has_init=hinit)
    x = lb.x
    if pad:
        wide = torch.zeros(lb.N, geo.C + pad, dtype=x.dtype)
        wide[:, :geo.C] = x
        x = wide.to(DEV)[:, :geo.C]
    else:
        x = x.to(DEV)
    g = torch.Generator().manual_seed(900 + case)
    bias = (torch.randn(geo.C, generator=g) * 0.2).to(DEV) if with_bias else None
    return lb, geo, x, bias


@pytest.mark.parametrize("write_state", [True, False])
@pytest.mark.parametrize("case", range(len(CP_CASES)))
def test_conv_postconv_bitwise_equal_to_two_calls(case, write_state):
    lb, geo, x, bias = _cp_inputs(case)
    print(f"conv+postconv case {case} write_state {write_state}", flush=True)
    cu, hi, w = lb.cu_seqlens.to(DEV), lb.has_init.to(DEV), lb.conv_w.to(DEV)
    chunks = gdn.gdn_make_chunks_device(cu, lb.N)
    cs1 = lb.conv_state.to(DEV).contiguous()
    cs2 = cs1.clone()
    y = gdn.gdn_causal_conv_fwd(x, w, bias, cs1, hi, cu, chunks, write_state)
    q1, k1, v1 = gdn.gdn_postconv_l2(y, geo.Hk, geo.Hv, 1e-6)
    q2, k2, v2 = gdn.gdn_conv_postconv_fwd(x, w, bias, cs2, hi, cu, chunks, write_state, geo.Hk, geo.Hv, 1e-6)
    torch.cuda.synchronize()
    for a, b, nm in ((q1, q2, "q"), (k1, k2, "k"), (v1, v2, "v"), (cs1, cs2, "conv_state")):
        ai = a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32)
        bi = b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32)
        assert torch.equal(ai, bi), f"{nm} differs in {(ai != bi).sum().item()} elements"


DERIVE_CASES = [
    ("bf16", I.GEO_TINY, [1, 2, 3, 63, 64, 65, 129, 200]),
    ("bf16", I.GEO_TINY, [5, 0, 70, 0, 1, 0]),                      # empty sequences
    ("f32", I.Geometry(Hk=2, Hv=2), [130, 7, 64, 128]),
    ("bf16", I.GEO_TINY, [(7 * i) % 41 + 1 for i in range(64)]),    # 64 sequences
    ("bf16", I.GEO_TINY, [64 * 3]),
]


@pytest.mark.parametrize("case", range(len(DERIVE_CASES)))
def test_conv_postconv_derived_chunks_bitwise_equal_to_descriptors(case):
    act, geo, lengths = DERIVE_CASES[case]
    hinit = [i % 2 for i in range(len(lengths))]
    lb = I.make_layer(geo, lengths, act, 860 + case, state_std=0.3, has_init=hinit)
    print(f"derived chunks case {case}: {len(lengths)} sequences, N = {lb.N}", flush=True)
    cu, hi, w, x = lb.cu_seqlens.to(DEV), lb.has_init.to(DEV), lb.conv_w.to(DEV), lb.x.to(DEV)
    cs1 = lb.conv_state.to(DEV).contiguous()
    cs2 = cs1.clone()
    q1, k1, v1 = gdn.gdn_conv_postconv_fwd(x, w, None, cs1, hi, cu, gdn.gdn_make_chunks_device(cu, lb.N), True,
                                           geo.Hk, geo.Hv, 1e-6)
    q2, k2, v2 = gdn.gdn_conv_postconv_fwd(x, w, None, cs2, hi, cu, None, True, geo.Hk, geo.Hv, 1e-6)
    torch.cuda.synchronize()
    for a, b, nm in ((q1, q2, "q"), (k1, k2, "k"), (v1, v2, "v"), (cs1, cs2, "conv_state")):
        ai = a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32)
        bi = b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32)
        assert torch.equal(ai, bi), f"{nm} differs in {(ai != bi).sum().item()} elements"


def test_conv_postconv_f32_matches_oracle_chain():
    # the f32 arm against the oracle: conv in float64, rounded to float32,
    # then the post-conv in its documented order
    lb, geo, x, bias = _cp_inputs(0)
    cu, hi = lb.cu_seqlens.to(DEV), lb.has_init.to(DEV)
    cs = lb.conv_state.to(DEV).contiguous()
    q, k, v = gdn.gdn_conv_postconv_fwd(x, lb.conv_w.to(DEV), None, cs, hi, cu,
                                        gdn.gdn_make_chunks_device(cu, lb.N), True, geo.Hk, geo.Hv, 1e-6)
    torch.cuda.synchronize()
    y_ref, cs_ref = O.causal_conv(TL.np64(lb.x), TL.np64(lb.conv_w), None, TL.np64(lb.conv_state),
                                  lb.has_init.numpy(), lb.cu_seqlens.tolist(), True)
    yr = O.round_to(y_ref, "f32")
    qr, kr, vr = O.postconv_l2_f32_tree(yr, geo.Hk, geo.Hv, 128, 128, 1e-6)
    # y itself is within the conv bound of the oracle; q, k, v follow it through
    # SiLU and the L2 scale (each a few float32 ulps)
    for got, ref in ((q, qr), (k, kr), (v, vr)):
        np.testing.assert_allclose(got.cpu().numpy(), ref, rtol=2e-5, atol=2e-6)
    assert np.array_equal(TL.np64(cs), cs_ref)
