"""GDN layer hot-path benchmark on one MI355X.

Default workload (the headline metric): the bf16 varlen prefill.  One step
is one pass of the whole hot path over one batch: exact 64-token conv chunks
(derived from cu_seqlens inside the conv launch; --chunk-descriptors runs
the descriptor builder instead), causal conv with the conv_state update and
post-conv (SiLU, split, L2) in one launch, and the chunked delta-rule
prefill with the state update, on 8
sequences with lengths uniform in [128, 2048], 8192 packed channels = 16 q
+ 16 k heads and 32 v heads of 128, half of the sequences with initial
states.  Inputs are synthetic and seeded, resident in HBM before timing
starts.

Prints ONE JSON line: throughput in tokens/s, the roofline of the dominant
kernel (per-launch HIP-event time of each kernel inside the timed region),
the CPU oracle timed on a bounded sample of the same workload, and a
cold-cache pass (`cold_cache`: up to 20 more steps, each after a 1 GiB read
that evicts L2 and the Infinity Cache, timed with events; context beside
`value`, which is the warm timed region).

Other workloads (--workload), each one JSON line with per-kernel stages and
the dominant kernel's roofline, throughput in layer-tokens/s:
  verify  speculative verify: 36 layers of conv shift + post-conv + decode
          step (no state write), then one batched commit of n_keep tokens
          (32 sequences, 1..8 draft tokens each)
  long    one 32768-token prefill layer
  mixed   24 layers of a serving step: 8 prefill sequences (log-uniform
          lengths in [256, 8192]) and 24 single-token decode sequences,
          6144 channels (16 q, 16 k, 16 v heads)
  verify-fused, mixed-fused
          the same, with the decode / draft tokens' conv, post-conv and
          step in one fused launch per layer
  out-norm
          the gated output norm on the mixed serving step's o, 24 layers
  gates   the gate computation for the mixed serving step, 24 layers

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                  [--workload varlen|verify|long|mixed|verify-fused|mixed-fused|out-norm|gates]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFS = 2500.0
METRIC = "GDN layer tokens/s (conv+postconv+delta-rule) and % of HBM roofline, 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_varlen_prefill_bf16.json")
KERNEL_SOURCES = {
    "conv": ["conv.hip", "device_common.hpp"],
    "convpost": ["conv.hip", "device_common.hpp"],
    "postconv": ["postconv.hip", "device_common.hpp"],
    "prefill": ["prefill.hip", "mfma.hpp", "device_common.hpp"],
    "step": ["step.hip", "mfma.hpp", "device_common.hpp"],
    "commit": ["step.hip", "mfma.hpp", "device_common.hpp"],
    "fused": ["step.hip", "mfma.hpp", "device_common.hpp"],
    "out_norm": ["outnorm.hip", "mfma.hpp", "device_common.hpp"],
    "gates": ["gates.hip", "mfma.hpp", "device_common.hpp"],
}
STATE_BYTES = 128 * 128 * 4   # one float32 state matrix (dv x dk)


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "linear_attention_layers_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------ algorithmic bytes
# Bytes each kernel must move at minimum (one launch).  e = activation bytes.

def conv_bytes(N, C, e, n_init, nseq, write_state):
    """x read, y written, weights (16 B) + bias slot (4 B) per channel, the
    three float32 conv_state rows read for sequences with initial state and
    written (when write_state) for every sequence."""
    return 2 * N * C * e + 20 * C + n_init * 12 * C + (nseq * 12 * C if write_state else 0)


def postconv_bytes(N, C, e):
    return 2 * N * C * e


# The conv and the post-conv run as one launch (gdn_conv_postconv_fwd) unless
# --split-conv asks for the two separate launches.  The fused launch moves
# conv_bytes: x in, q|k|v (N x C) out instead of y.  It derives the 64-token
# chunks from cu_seqlens itself unless --chunk-descriptors (or --split-conv,
# whose conv needs them) asks for the descriptor builder's launch.
SPLIT_CONV = False
CHUNK_DESCRIPTORS = False


def descriptors_needed() -> bool:
    return SPLIT_CONV or CHUNK_DESCRIPTORS


def add_conv_post(p, x, w, cs, hi, cu, chunks, write_state, Hk, Hv, N, C, n_init, nseq, y, q, k, v):
    from linear_attention_layers_amd import gdn
    if SPLIT_CONV:
        p.add("conv", lambda: gdn.gdn_causal_conv_fwd(x, w, None, cs, hi, cu, chunks, write_state, y=y),
              conv_bytes(N, C, 2, n_init, nseq, write_state))
        p.add("postconv", lambda: gdn.gdn_postconv_l2(y, Hk, Hv, 1e-6, q=q, k=k, v=v), postconv_bytes(N, C, 2))
    else:
        p.add("convpost", lambda: gdn.gdn_conv_postconv_fwd(x, w, None, cs, hi, cu, chunks, write_state, Hk, Hv,
                                                            1e-6, q=q, k=k, v=v),
              conv_bytes(N, C, 2, n_init, nseq, write_state))


def recurrence_bytes(N, Hk, Hv, e, n_state_read, n_state_write):
    """q, k, v read, o written, g and beta read, plus whole float32 states."""
    return (N * (2 * Hk * 128 + Hv * 128) * e + N * Hv * 8 + N * Hv * 128 * e
            + (n_state_read + n_state_write) * Hv * STATE_BYTES)


def fused_bytes(N, C, Hk, Hv, e, nseq, write_conv, n_state_write, kv_out):
    """The fused decode/verify launch: x read, weights and bias slot, the
    stored conv rows of every sequence read (and written when write_conv),
    g and beta read, o written, every state read (and written when
    committing), plus the kept k and v when kv_out."""
    return (N * C * e + 20 * C + nseq * 12 * C * (2 if write_conv else 1) + N * Hv * 8
            + N * Hv * 128 * e + (nseq + n_state_write) * Hv * STATE_BYTES
            + (N * (Hk + Hv) * 128 * e if kv_out else 0))


def commit_bytes(L, C, Hk, Hv, e, n_keep, nseq):
    """Per layer, for each sequence that keeps n > 0 tokens: its state read
    and written, the kept tokens' k, v, g, beta, and the conv_state rows
    rebuilt from the kept x rows (12 B per channel read and written)."""
    kept = sum(n_keep)
    active = sum(1 for n in n_keep if n > 0)
    per_layer = (active * Hv * 2 * STATE_BYTES + kept * (Hk * 128 + Hv * 128) * e + kept * Hv * 8
                 + kept * C * e + active * 24 * C)
    return L * per_layer


def algorithmic_bytes(lb) -> dict:
    """Per-kernel bytes of the default varlen step (one launch each)."""
    N, C = lb.N, lb.geo.C
    e = 2 if lb.act == "bf16" else 4
    n_init = int(lb.has_init.sum())
    return {"conv": conv_bytes(N, C, e, n_init, lb.nseq, True),
            "postconv": postconv_bytes(N, C, e),
            "convpost": conv_bytes(N, C, e, n_init, lb.nseq, True),
            "prefill": recurrence_bytes(N, lb.geo.Hk, lb.geo.Hv, e, n_init, lb.nseq)}


def prefill_flops(lb) -> float:
    """Dense contraction flops of the chunked form, 11 d^2 per token per
    v-head (K K^T, Q K^T, T R, K S^T, Q S^T, P U, state update)."""
    return 11.0 * 128 * 128 * lb.N * lb.geo.Hv


def cpu_baseline(lb) -> dict:
    """The oracle (unchanged) on the same batch: conv, post-conv and the
    per-token recurrence for every token and head, single-threaded float64
    numpy.  The whole varlen batch is about 10 s of CPU work, so the sample
    is the full workload."""
    import numpy as np
    from oracle import gdn_oracle as O
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:                              # pragma: no cover
        limiter = None
    cu = lb.cu_seqlens.tolist()
    x = lb.x.float().numpy().astype(np.float64)
    w = lb.conv_w.numpy().astype(np.float64)
    cs = lb.conv_state.numpy().astype(np.float64)
    st = lb.state.numpy().astype(np.float64)
    g = lb.g.numpy().astype(np.float64)
    b = lb.beta.numpy().astype(np.float64)
    hi = lb.has_init.numpy()
    Hk, Hv = lb.geo.Hk, lb.geo.Hv
    t0 = time.perf_counter()
    y, _ = O.causal_conv(x, w, None, cs, hi, cu, True)
    q, k, v = O.postconv_l2(O.round_to_bf16(y), Hk, Hv, 128, 128, 1e-6)
    del y
    q, k, v = O.round_to_bf16(q), O.round_to_bf16(k), O.round_to_bf16(v)
    O.delta_rule_recurrent(q, k, v, g, b, st, hi, cu, Hk, Hv)
    dt = time.perf_counter() - t0
    if limiter is not None and hasattr(limiter, "unregister"):
        limiter.unregister()
    return {"value": lb.N / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"the full batch ({lb.nseq} sequences, {lb.N} tokens): conv, post-conv "
                      f"and per-token recurrence over all {Hv} v-heads, float64 numpy, one thread",
            "seconds": round(dt, 2)}


# ------------------------------------------------------------------ workloads
# Each builder returns a plan: the ordered kernel launches of one step, the
# algorithmic bytes per kernel name (summed over the step), the tokens of
# one step and the config dict.

class Plan:
    def __init__(self):
        self.launches = []       # (kernel name, callable)
        self.bytes = {}          # kernel name -> bytes per step
        self.count = {}          # kernel name -> launches per step
        self.flops = {}          # kernel name -> dense flops per step
        self.tokens = 0
        self.dtype = "bf16"      # arithmetic type of the step's activations
        self.config = {}
        self.keep = []           # tensors kept alive

    def add(self, name, fn, nbytes, flops=0.0):
        self.launches.append((name, fn))
        self.bytes[name] = self.bytes.get(name, 0) + nbytes
        self.count[name] = self.count.get(name, 0) + 1
        if flops:
            self.flops[name] = self.flops.get(name, 0.0) + flops


def _layer_on_device(lb, dev):
    import torch
    d = dict(x=lb.x.to(dev), w=lb.conv_w.to(dev), cs=lb.conv_state.to(dev), st=lb.state.to(dev),
             g=lb.g.to(dev), beta=lb.beta.to(dev), cu=lb.cu_seqlens.to(dev),
             hi=lb.has_init.to(dev))
    N, C, Hk, Hv = lb.N, lb.geo.C, lb.geo.Hk, lb.geo.Hv
    d["y"] = torch.empty(N, C, dtype=lb.x.dtype, device=dev)
    d["q"] = torch.empty(N, Hk, 128, dtype=lb.x.dtype, device=dev)
    d["k"] = torch.empty_like(d["q"])
    d["v"] = torch.empty(N, Hv, 128, dtype=lb.x.dtype, device=dev)
    d["o"] = torch.empty_like(d["v"])
    return d


def plan_varlen(dev):
    import torch
    from linear_attention_layers_amd import gdn, inputs
    lb = inputs.varlen_prefill()
    d = _layer_on_device(lb, dev)
    Hk, Hv, N = lb.geo.Hk, lb.geo.Hv, lb.N
    chunks = torch.empty(gdn.gdn_chunk_capacity(N, lb.nseq), 4, dtype=torch.int32, device=dev)
    algo = algorithmic_bytes(lb)
    p = Plan()
    if descriptors_needed():
        p.add("chunks", lambda: gdn.gdn_make_chunks_device(d["cu"], N, out=chunks), 0)
    add_conv_post(p, d["x"], d["w"], d["cs"], d["hi"], d["cu"], chunks if descriptors_needed() else None,
                  True, Hk, Hv, N, lb.geo.C,
                  int(lb.has_init.sum()), lb.nseq, d["y"], d["q"], d["k"], d["v"])
    p.add("prefill", lambda: gdn.gdn_delta_rule_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                                        d["cu"], d["st"], d["hi"], o=d["o"]),
          algo["prefill"], prefill_flops(lb))
    p.tokens = N
    p.config = {"workload": "varlen_prefill_bf16", "nseq": lb.nseq, "tokens": N,
                "channels": lb.geo.C, "Hk": Hk, "Hv": Hv, "head_dim": 128, "layers": 1,
                "state_dtype": "f32", "seed": 2000}
    p.keep = [d, chunks]
    p.lb = lb
    return p


def plan_verify(dev, fused=False):
    import torch
    from linear_attention_layers_amd import gdn, inputs
    L = 36
    lengths, n_keep = inputs.spec_verify_window()
    p = Plan()
    table_layers = []
    lb0 = None
    for layer in range(L):
        lb = inputs.spec_verify_layer(layer)
        lb0 = lb0 or lb
        d = _layer_on_device(lb, dev)
        N, C, Hk, Hv = lb.N, lb.geo.C, lb.geo.Hk, lb.geo.Hv
        chunks = gdn.gdn_make_chunks_device(d["cu"], N)
        d["chunks"] = chunks
        if fused:
            # k and v are kept for the commit's replay
            p.add("fused", lambda d=d, Hk=Hk, Hv=Hv: gdn.gdn_decode_fused(
                      d["x"], d["w"], None, d["cs"], d["cu"], d["g"], d["beta"], d["st"], Hk, Hv, 1e-6,
                      None, o=d["o"], write_conv_state=False, commit_state=False, k_out=d["k"],
                      v_out=d["v"]),
                  fused_bytes(N, C, Hk, Hv, 2, lb.nseq, False, 0, True))
        else:
            add_conv_post(p, d["x"], d["w"], d["cs"], None, d["cu"], d["chunks"] if descriptors_needed() else None,
                          False, Hk, Hv, N, C,
                          lb.nseq, lb.nseq, d["y"], d["q"], d["k"], d["v"])
            p.add("step", lambda d=d: gdn.gdn_delta_rule_step(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                                              d["cu"], d["st"], None, o=d["o"],
                                                              commit_state=False),
                  recurrence_bytes(N, Hk, Hv, 2, lb.nseq, 0))
        p.keep.append(d)
        table_layers.append(dict(x=d["x"], conv_state=d["cs"], state=d["st"], k=d["k"], v=d["v"],
                                 g=d["g"], beta=d["beta"]))
    table = gdn.gdn_layer_table(table_layers, dev)
    cu0 = lb0.cu_seqlens.to(dev)
    nk = lb0.n_keep.to(dev)
    p.keep += [table, cu0, nk]
    C, Hk, Hv = lb0.geo.C, lb0.geo.Hk, lb0.geo.Hv
    p.add("commit", lambda: gdn.gdn_commit(table, L, cu0, nk, None, C, Hk, Hv, torch.bfloat16),
          commit_bytes(L, C, Hk, Hv, 2, n_keep, len(lengths)))
    p.tokens = L * sum(lengths)
    p.config = {"workload": "spec_verify_36L_bf16" + ("_fused" if fused else ""),
                "nseq": len(lengths), "tokens": sum(lengths),
                "kept_tokens": sum(n_keep), "channels": C, "Hk": Hk, "Hv": Hv, "head_dim": 128,
                "layers": L, "state_dtype": "f32", "seed": 3000}
    return p


def plan_long(dev, nseg=1):
    import torch
    from linear_attention_layers_amd import gdn, inputs
    lb = inputs.long_prefill()
    d = _layer_on_device(lb, dev)
    Hk, Hv, N, C = lb.geo.Hk, lb.geo.Hv, lb.N, lb.geo.C
    chunks = torch.empty(gdn.gdn_chunk_capacity(N, lb.nseq), 4, dtype=torch.int32, device=dev)
    p = Plan()
    if descriptors_needed():
        p.add("chunks", lambda: gdn.gdn_make_chunks_device(d["cu"], N, out=chunks), 0)
    add_conv_post(p, d["x"], d["w"], d["cs"], d["hi"], d["cu"], chunks if descriptors_needed() else None,
                  True, Hk, Hv, N, C, 0, 1, d["y"],
                  d["q"], d["k"], d["v"])
    if nseg == 1:
        run = lambda: gdn.gdn_delta_rule_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"],
                                                 d["st"], d["hi"], o=d["o"])
    else:
        # the three launches of the segmented prefill are one stage; its
        # bytes and flops are the unsegmented algorithm's
        d["ws"] = torch.empty(gdn.gdn_prefill_segmented_workspace(1, Hv, nseg), dtype=torch.uint8,
                              device=dev)
        run = lambda: gdn.gdn_delta_rule_prefill_segmented(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                                           d["cu"], d["st"], nseg, d["hi"], o=d["o"],
                                                           workspace=d["ws"])
    p.add("prefill", run, recurrence_bytes(N, Hk, Hv, 2, 0, 1), prefill_flops(lb))
    p.tokens = N
    p.config = {"workload": "long_prefill_32k_bf16" + (f"_seg{nseg}" if nseg > 1 else ""), "nseq": 1,
                "tokens": N, "channels": C, "Hk": Hk, "Hv": Hv, "head_dim": 128, "layers": 1,
                "state_dtype": "f32", "seed": 4000}
    if nseg > 1:
        p.config["segments"] = nseg
    p.keep = [d, chunks]
    return p


def plan_mixed(dev, fused=False):
    from linear_attention_layers_amd import gdn, inputs
    L = 24
    p = Plan()
    for layer in range(L):
        lb = inputs.mixed_serving_layer(layer)
        d = _layer_on_device(lb, dev)
        npre = lb.meta["n_prefill"]
        Npre = int(lb.cu_seqlens[npre])
        N, C, Hk, Hv = lb.N, lb.geo.C, lb.geo.Hk, lb.geo.Hv
        ndec = lb.nseq - npre
        d["chunks"] = gdn.gdn_make_chunks_device(d["cu"], N)
        d["cu_pre"] = d["cu"][:npre + 1]
        d["cu_dec"] = (d["cu"][npre:] - Npre).contiguous()
        if fused:
            # conv and post-conv over the prefill tokens only; the decode
            # tokens go through the fused launch
            d["chunks_pre"] = gdn.gdn_make_chunks_device(d["cu_pre"], Npre)
            add_conv_post(p, d["x"][:Npre], d["w"], d["cs"][:npre], None, d["cu_pre"],
                          d["chunks_pre"] if descriptors_needed() else None, True,
                          Hk, Hv, Npre, C, npre, npre, d["y"][:Npre], d["q"][:Npre], d["k"][:Npre],
                          d["v"][:Npre])
        else:
            add_conv_post(p, d["x"], d["w"], d["cs"], None, d["cu"], d["chunks"] if descriptors_needed() else None,
                          True, Hk, Hv, N, C,
                          lb.nseq, lb.nseq, d["y"], d["q"], d["k"], d["v"])
        p.add("prefill", lambda d=d, n=Npre, m=npre: gdn.gdn_delta_rule_prefill(
                  d["q"][:n], d["k"][:n], d["v"][:n], d["g"][:n], d["beta"][:n], d["cu_pre"],
                  d["st"][:m], None, o=d["o"][:n]),
              recurrence_bytes(Npre, Hk, Hv, 2, npre, npre), 11.0 * 128 * 128 * Npre * Hv)
        if fused:
            p.add("fused", lambda d=d, n=Npre, m=npre, Hk=Hk, Hv=Hv: gdn.gdn_decode_fused(
                      d["x"][n:], d["w"], None, d["cs"][m:], d["cu_dec"], d["g"][n:], d["beta"][n:],
                      d["st"][m:], Hk, Hv, 1e-6, None, o=d["o"][n:], write_conv_state=True,
                      commit_state=True),
                  fused_bytes(N - Npre, C, Hk, Hv, 2, ndec, True, ndec, False))
        else:
            p.add("step", lambda d=d, n=Npre, m=npre: gdn.gdn_delta_rule_step(
                      d["q"][n:], d["k"][n:], d["v"][n:], d["g"][n:], d["beta"][n:], d["cu_dec"],
                      d["st"][m:], None, o=d["o"][n:], commit_state=True),
                  recurrence_bytes(N - Npre, Hk, Hv, 2, ndec, ndec))
        p.keep.append(d)
        p.tokens += N
        p.config = {"workload": "mixed_serving_24L_bf16" + ("_fused" if fused else ""),
                    "prefill_seqs": npre, "decode_seqs": ndec,
                    "tokens_per_layer": N, "channels": C, "Hk": Hk, "Hv": Hv, "head_dim": 128,
                    "layers": L, "state_dtype": "f32", "seed": 5000}
    return p


def plan_out_norm(dev):
    """The gated output norm on every layer's o of the mixed serving step
    (24 layers, its token count, 16 v-heads of 128, bf16, with a weight).
    o, z and the weight are drawn on the device (seeded)."""
    import torch
    from linear_attention_layers_amd import gdn, inputs
    L = 24
    N = sum(inputs.mixed_lengths(5000))
    Hv = inputs.GEO_6144.Hv
    p = Plan()
    gen = torch.Generator(device=dev).manual_seed(6000)
    for layer in range(L):
        o = torch.randn(N, Hv, 128, generator=gen, device=dev).to(torch.bfloat16)
        z = (2.0 * torch.randn(N, Hv, 128, generator=gen, device=dev)).to(torch.bfloat16)
        w = 0.5 + torch.rand(128, generator=gen, device=dev)
        y = torch.empty_like(o)
        p.add("out_norm", lambda o=o, z=z, w=w, y=y: gdn.gdn_out_norm(o, z, w, 1e-6, y=y),
              3 * N * Hv * 128 * 2 + 128 * 4)
        p.keep.append((o, z, w, y))
        p.tokens += N
    p.config = {"workload": "out_norm_24L_bf16", "tokens_per_layer": N, "Hv": Hv, "head_dim": 128,
                "layers": L, "seed": 6000}
    return p


def plan_gates(dev):
    """The gate computation for every layer of the mixed serving step (24
    layers, its token count, 16 v-heads): packed float32 (b, a) in, float32
    g and beta out.  Inputs drawn on the device (seeded)."""
    import torch
    from linear_attention_layers_amd import gdn, inputs
    L = 24
    N = sum(inputs.mixed_lengths(5000))
    Hv = inputs.GEO_6144.Hv
    p = Plan()
    gen = torch.Generator(device=dev).manual_seed(7000)
    for layer in range(L):
        ba = 2.0 * torch.randn(N, Hv, 2, generator=gen, device=dev)
        A_log = torch.log(1.0 + 15.0 * torch.rand(Hv, generator=gen, device=dev))
        dt = torch.randn(Hv, generator=gen, device=dev)
        g = torch.empty(N, Hv, device=dev)
        beta = torch.empty_like(g)
        p.add("gates", lambda ba=ba, A_log=A_log, dt=dt, g=g, beta=beta: gdn.gdn_gates(ba, A_log, dt, g=g, beta=beta),
              N * Hv * 16 + Hv * 8)
        p.keep.append((ba, A_log, dt, g, beta))
        p.tokens += N
    p.config = {"workload": "gates_24L_f32", "tokens_per_layer": N, "Hv": Hv, "layers": L, "seed": 7000}
    p.dtype = "f32"
    return p


PLANS = {"varlen": plan_varlen, "verify": plan_verify, "long": plan_long, "mixed": plan_mixed,
         "verify-fused": lambda dev: plan_verify(dev, fused=True),
         "mixed-fused": lambda dev: plan_mixed(dev, fused=True), "out-norm": plan_out_norm,
         "gates": plan_gates, "long-seg": lambda dev: plan_long(dev, nseg=4)}


def cold_pass(plan, stream, reps):
    """Each of `reps` steps runs right after a 1 GiB read of an unrelated
    buffer (clean lines: it evicts L2 and the Infinity Cache without leaving
    write-backs behind), with HIP events on the launch stream around every
    kernel and around the step; the read itself is outside the events."""
    import torch
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=stream.device)
    names = list(dict.fromkeys(nm for nm, _ in plan.launches))
    acc = {nm: 0.0 for nm in names}
    total = 0.0
    for _ in range(reps):
        scratch.sum()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(plan.launches) + 1)]
        ev[0].record(stream)
        for i, (_, fn) in enumerate(plan.launches):
            fn()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        for j, (nm, _) in enumerate(plan.launches):
            acc[nm] += ev[j].elapsed_time(ev[j + 1])
        total += ev[0].elapsed_time(ev[-1])
    del scratch
    stages = {}
    for nm in names:
        rec = {"us_per_launch": round(acc[nm] / reps * 1e3 / plan.count[nm], 2)}
        if plan.bytes.get(nm):
            rec["hbm_frac"] = round(plan.bytes[nm] / (acc[nm] / reps / 1e3) / 1e9 / HBM_PEAK_GBS, 4)
        stages[nm] = rec
    ms = total / reps
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(plan.tokens / (ms / 1e3), 1),
            "steps": reps, "flush_bytes": 1 << 30, "stages": stages}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", choices=sorted(PLANS), default="varlen")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache pass (steps run after a 1 GiB read that evicts L2 and the "
                         "256 MB Infinity Cache; reported beside the timed region, never as value)")
    ap.add_argument("--chunk-descriptors", action="store_true",
                    help="build the conv chunk descriptors in their own launch (gdn_make_chunks_device) "
                         "instead of deriving them inside the conv launch")
    ap.add_argument("--split-conv", action="store_true",
                    help="run the conv and the post-conv as two launches instead of the fused one")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 5 times (the reference "
                         "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the GDN hot path shards by sequence and head group with no exchange; "
              "multi-GPU runs are not part of this build)", file=sys.stderr)
        sys.exit(2)
    default_steps = {"varlen": 100, "verify": 20, "long": 20, "mixed": 10, "verify-fused": 20,
                     "mixed-fused": 10, "out-norm": 20, "gates": 20, "long-seg": 20}[args.workload]
    steps = args.steps if args.steps is not None else default_steps
    warmup = args.warmup if args.warmup is not None else max(2, steps // 10)

    import torch

    dev = torch.device("cuda", 0)
    if args.copy_calibration:
        nbytes = 256 << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": nbytes, "launches": 5}), flush=True)
        return

    global SPLIT_CONV, CHUNK_DESCRIPTORS
    SPLIT_CONV = args.split_conv
    CHUNK_DESCRIPTORS = args.chunk_descriptors
    plan = PLANS[args.workload](dev)
    stream = torch.cuda.current_stream()
    n_l = len(plan.launches)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        for i, (_, fn) in enumerate(plan.launches):
            fn()
            if ev is not None:
                ev[i + 1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_l + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    names = list(dict.fromkeys(nm for nm, _ in plan.launches))
    per_step_ms = {nm: 0.0 for nm in names}
    for ev in events:
        for j, (nm, _) in enumerate(plan.launches):
            per_step_ms[nm] += ev[j].elapsed_time(ev[j + 1])
    per_step_ms = {nm: t / steps for nm, t in per_step_ms.items()}

    ms_per_step = wall * 1e3 / steps
    tokens_per_s = plan.tokens / (ms_per_step / 1e3)
    stages = {}
    for nm in names:
        t = per_step_ms[nm] / 1e3
        rec = {"us_per_launch": round(per_step_ms[nm] * 1e3 / plan.count[nm], 2),
               "launches": plan.count[nm]}
        if plan.bytes.get(nm):
            rec["GB/s"] = round(plan.bytes[nm] / t / 1e9, 1)
            rec["hbm_frac"] = round(plan.bytes[nm] / t / 1e9 / HBM_PEAK_GBS, 4)
        if plan.flops.get(nm):
            tf = plan.flops[nm] / t / 1e12
            rec["mfma_TFLOP/s"] = round(tf, 2)
            rec["mfma_frac_bf16_dense"] = round(tf / BF16_MFMA_PEAK_TFS, 4)
        stages[nm] = rec
    timed = [nm for nm in names if plan.bytes.get(nm)]
    dominant = max(timed, key=lambda nm: per_step_ms[nm])
    achieved = plan.bytes[dominant] / (per_step_ms[dominant] / 1e3) / 1e9

    traffic = None
    if args.workload == "varlen":
        try:
            with open(TRAFFIC_FILE) as f:
                rec = json.load(f).get(dominant)
            if rec and rec.get("source_hash") == source_hash(dominant):
                traffic = rec["bytes_per_launch"]
        except (OSError, ValueError):
            pass

    out = {
        "metric": METRIC if args.workload == "varlen" else
        f"GDN {args.workload} step layer-tokens/s and % of HBM roofline, 1 GPU",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": plan.dtype,
        "data": "synthetic",
        "config": plan.config,
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes": plan.bytes[dominant] // plan.count[dominant]},
        "stages": stages,
    }
    if not args.no_cold:
        out["cold_cache"] = cold_pass(plan, stream, min(steps, 20))
    if args.workload == "varlen" and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(plan.lb)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
