"""GDN layer hot-path benchmark on one MI355X.

One step = one pass of the whole hot path over one batch: exact conv chunks
(device builder), causal conv with conv_state update, post-conv (SiLU,
split, L2) and the chunked delta-rule prefill with the state update, on the
bf16 varlen prefill workload (8 sequences with lengths uniform in
[128, 2048], 8192 packed channels = 16 q + 16 k heads and 32 v heads of
128, half of the sequences with initial states).  Inputs are synthetic and
seeded, resident in HBM before timing starts.

Prints ONE JSON line: throughput in tokens/s, the roofline of the dominant
kernel (per-launch HIP-event time of each kernel inside the timed region),
and the CPU oracle timed on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
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
METRIC = "GDN layer tokens/s (conv+postconv+delta-rule) and % of HBM roofline, 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_varlen_prefill_bf16.json")
KERNEL_SOURCES = {
    "conv": ["conv.hip", "device_common.hpp"],
    "postconv": ["postconv.hip", "device_common.hpp"],
    "prefill": ["prefill.hip", "device_common.hpp"],
}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "linear_attention_layers_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(lb) -> dict:
    """Bytes each kernel must move at minimum for this batch (per launch)."""
    N, C = lb.N, lb.geo.C
    Hk, Hv = lb.geo.Hk, lb.geo.Hv
    e = 2 if lb.act == "bf16" else 4
    n_init = int(lb.has_init.sum())
    nseq = lb.nseq
    conv = 2 * N * C * e + 20 * C + n_init * 12 * C + nseq * 12 * C
    post = N * C * e + N * C * e
    state = Hv * 128 * 128 * 4
    pre = (N * (2 * Hk * 128 + Hv * 128) * e      # q, k, v
           + N * Hv * 8                            # g, beta
           + N * Hv * 128 * e                      # o
           + n_init * state + nseq * state)        # state read (if any) + write
    return {"conv": conv, "postconv": post, "prefill": pre}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 5 times (the reference "
                         "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the GDN hot path shards by sequence and head group with no exchange; "
              "multi-GPU runs are not part of this build)", file=sys.stderr)
        sys.exit(2)

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

    from linear_attention_layers_amd import gdn, inputs

    lb = inputs.varlen_prefill()
    Hk, Hv, C, N = lb.geo.Hk, lb.geo.Hv, lb.geo.C, lb.N
    x = lb.x.to(dev)
    w = lb.conv_w.to(dev)
    cs = lb.conv_state.to(dev)
    st = lb.state.to(dev)
    g = lb.g.to(dev)
    beta = lb.beta.to(dev)
    cu = lb.cu_seqlens.to(dev)
    hi = lb.has_init.to(dev)
    cap = gdn.gdn_chunk_capacity(N, lb.nseq)
    chunks = torch.empty(cap, 4, dtype=torch.int32, device=dev)
    y = torch.empty(N, C, dtype=torch.bfloat16, device=dev)
    q = torch.empty(N, Hk, 128, dtype=torch.bfloat16, device=dev)
    k = torch.empty_like(q)
    v = torch.empty(N, Hv, 128, dtype=torch.bfloat16, device=dev)
    o = torch.empty_like(v)
    stream = torch.cuda.current_stream()

    names = ["chunks", "conv", "postconv", "prefill"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        gdn.gdn_make_chunks_device(cu, N, out=chunks)
        mark(1)
        gdn.gdn_causal_conv_fwd(x, w, None, cs, hi, cu, chunks, True, y=y)
        mark(2)
        gdn.gdn_postconv_l2(y, Hk, Hv, 1e-6, q=q, k=k, v=v)
        mark(3)
        gdn.gdn_delta_rule_prefill(q, k, v, g, beta, cu, st, hi, o=o)
        mark(4)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per_kernel_ms = {nm: 0.0 for nm in names}
    for ev in events:
        for j, nm in enumerate(names):
            per_kernel_ms[nm] += ev[j].elapsed_time(ev[j + 1])
    per_kernel_ms = {nm: t / args.steps for nm, t in per_kernel_ms.items()}

    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = N / (ms_per_step / 1e3)
    algo = algorithmic_bytes(lb)
    stages = {}
    for nm in ("conv", "postconv", "prefill"):
        t = per_kernel_ms[nm] / 1e3
        stages[nm] = {"us": round(per_kernel_ms[nm] * 1e3, 2),
                      "GB/s": round(algo[nm] / t / 1e9, 1),
                      "hbm_frac": round(algo[nm] / t / 1e9 / HBM_PEAK_GBS, 4)}
    stages["prefill"]["mfma_TFLOP/s"] = round(prefill_flops(lb) / (per_kernel_ms["prefill"] / 1e3) / 1e12, 2)
    stages["chunks"] = {"us": round(per_kernel_ms["chunks"] * 1e3, 2)}
    dominant = max(("conv", "postconv", "prefill"), key=lambda nm: per_kernel_ms[nm])
    achieved = algo[dominant] / (per_kernel_ms[dominant] / 1e3) / 1e9

    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(dominant)
        if rec and rec.get("source_hash") == source_hash(dominant):
            traffic = rec["bytes_per_launch"]
    except (OSError, ValueError):
        pass

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "varlen_prefill_bf16", "nseq": lb.nseq, "tokens": N,
                   "channels": C, "Hk": Hk, "Hv": Hv, "head_dim": 128, "layers": 1,
                   "state_dtype": "f32", "seed": 2000},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": algo[dominant]},
        "stages": stages,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(lb)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
