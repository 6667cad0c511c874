"""Host-side checks of the benchmark script: the one-GPU contract and the
algorithmic byte model behind its roofline figures (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from linear_attention_layers_amd import inputs as I  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_varlen_byte_model_counts_each_tensor_once():
    lb = I.varlen_prefill()
    N, nseq = lb.N, lb.nseq
    assert (N, nseq) == (sum(I.varlen_lengths()), 8)
    n_init = int(lb.has_init.sum())
    assert n_init == 4                          # even-indexed sequences
    algo = bench.algorithmic_bytes(lb)
    # conv (+ post-conv in one launch): x in and q|k|v out, 8192 bf16 channels
    # per token; taps (4 floats) and the bias slot per channel; 3 float32
    # conv rows read for the 4 sequences with initial state, written for all 8
    assert algo["convpost"] == N * 8192 * 2 * 2 + 8192 * 20 + 4 * 3 * 8192 * 4 + 8 * 3 * 8192 * 4
    # prefill: q and k (16 heads of 128) and v and o (32 heads of 128) in
    # bf16, g and beta per v-head in float32, 128 x 128 float32 states read
    # for 4 sequences and written for 8, 32 heads each
    per_token = (16 * 128 * 2) * 2 + (32 * 128 * 2) * 2 + 32 * 4 * 2
    assert algo["prefill"] == N * per_token + (4 + 8) * 32 * 128 * 128 * 4
    assert bench.prefill_flops(lb) == 11 * 128 * 128 * N * 32


def test_commit_byte_model_skips_sequences_that_keep_nothing():
    # one layer, C = 8192, two sequences keeping 3 and 0 tokens
    got = bench.commit_bytes(1, 8192, 16, 32, 2, [3, 0], 2)
    state = 32 * 128 * 128 * 4 * 2               # read and written, one sequence
    tokens = 3 * (16 * 128 + 32 * 128) * 2 + 3 * 32 * 8 + 3 * 8192 * 2
    conv_rows = 24 * 8192
    assert got == state + tokens + conv_rows


def test_cpu_baseline_units_cover_every_sequence_and_head_once():
    import numpy as np
    for lengths, Hk in ((I.mixed_lengths(), 16), (I.varlen_lengths(), 16), ([1] * 5, 2), ([300], 16),
                        ([0, 7, 0, 400, 3], 4)):
        cu = np.concatenate([[0], np.cumsum(lengths)])
        cover = np.zeros((len(lengths), Hk), dtype=int)
        for s0, s1, kh0, nk in bench._cpu_units(cu, Hk):
            cover[s0:s1, kh0:kh0 + nk] += 1
        assert (cover == 1).all(), (lengths, Hk)


def test_cpu_baseline_units_compute_the_whole_layer():
    # the per-unit oracle runs (a run of sequences x a group of heads, on that
    # group's channels) add up to the oracle on the whole batch
    import numpy as np
    from oracle import gdn_oracle as O
    lb = I.make_layer(I.Geometry(Hk=2, Hv=4), [70, 1, 1, 300], "bf16", 77, state_std=0.3,
                      has_init=[1, 0, 1, 1])
    bench._CPU.clear()
    bench._CPU.update(x=lb.x.float().numpy(), w=lb.conv_w.numpy().astype(np.float64),
                      cs=lb.conv_state.numpy().astype(np.float64), st=lb.state.numpy().astype(np.float64),
                      g=lb.g.numpy().astype(np.float64), beta=lb.beta.numpy().astype(np.float64),
                      hi=lb.has_init.numpy(), cu=lb.cu_seqlens.numpy().astype(np.int64), Hk=2, Hv=4, act="bf16")
    units = bench._cpu_units(bench._CPU["cu"], 2, min_tokens=64)
    assert len(units) > 2
    total = sum(bench._cpu_unit(u) for u in units)
    bench._CPU.clear()
    cu = lb.cu_seqlens.tolist()
    y, _ = O.causal_conv(lb.x.float().numpy().astype(np.float64), lb.conv_w.numpy(), None,
                         lb.conv_state.numpy(), lb.has_init.numpy(), cu, True)
    q, k, v = (O.round_to_bf16(a) for a in O.postconv_l2(O.round_to_bf16(y), 2, 4, 128, 128, 1e-6))
    o, _ = O.delta_rule_recurrent(q, k, v, lb.g.numpy(), lb.beta.numpy(), lb.state.numpy(),
                                  lb.has_init.numpy(), cu, 2, 4)
    assert abs(total - float(np.abs(o).sum())) <= 1e-9 * float(np.abs(o).sum())


def test_default_workload_is_the_mixed_serving_step():
    import argparse  # noqa: F401
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert 'ap.add_argument("--workload", choices=sorted(PLANS), default="mixed")' in src
    lb, layers = bench.cpu_sample("mixed")
    assert layers == 24 and lb.geo.C == 6144 and lb.nseq == 32 and lb.N == sum(I.mixed_lengths())


def test_timing_stride_picks_every_nth_launch_of_the_kernel():
    p = bench.Plan()
    for layer in range(6):
        p.add("convpost", None, 1)
        p.add("prefill", None, 1)
        p.add("fused", None, 1, stream=1)
    r = bench.Runner.__new__(bench.Runner)
    r.plan = p
    pre = [i for i, (nm, _) in enumerate(p.launches) if nm == "prefill"]
    assert r.timed("prefill", 1) == set(pre)
    assert r.timed("prefill", 4) == {pre[0], pre[4]}
    assert r.timed("prefill", 24) == {pre[0]}
    assert r.timed(None) == set(range(18))
