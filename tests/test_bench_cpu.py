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
