"""GDN layer hot-path benchmark on one MI355X.

Default workload (the headline metric): the mixed serving step at
concurrency 32, the largest of the five workloads that fits one GPU.  Each
of 24 layers takes 8 prefill sequences (lengths log-uniform in [256, 8192],
16,333 tokens) and 24 single-token decode sequences, 6144 packed channels
(16 q, 16 k, 16 v heads of 128), bf16 activations, float32 states, all with
initial states.  One step is one pass of the hot path over all 24 layers;
per layer:
  main stream  conv + post-conv of the prefill tokens in one launch (exact
               64-token chunks derived in the launch, conv_state updated),
               then the chunked delta-rule prefill (state updated);
  side stream  the decode tokens' conv, post-conv and committing step in
               one fused launch, started after the layer's conv + post-conv
               and joined before the next layer, so it runs beside the
               prefill (the two touch disjoint sequences).
--serial runs every launch on one stream.  Inputs are synthetic and
seeded, resident in HBM before timing starts.  The K timed steps are
captured once as one HIP graph (launches, cross-stream joins and the
dominant kernel's event records as graph nodes) and replayed, after one warm
replay (the first launch of a graph uploads it); --eager issues them from the
host launch by launch instead.  Inside the timed region events bracket every
4th launch of the dominant kernel in each step (--time-stride; its first
launch included): each bracketed launch puts two marker packets in the queue,
about 7 us of step time on the mixed serving step.  Every event is created
with hipEventDisableSystemFence, so recording one adds no cache write-back.

Prints ONE JSON line: throughput in layer-tokens/s, the roofline of the
dominant kernel (its per-launch HIP-event time inside the timed region, on
the stream it runs on; the warm-up steps, timed per launch, pick it by their
median), every kernel's time from an instrumented pass after the timed
region (with each one's fraction of a plain device copy's bandwidth,
`copy_bandwidth`, measured after the timed region as context), the CPU
oracle timed on a bounded sample of the same workload over a pool of host
processes, and a cold-cache pass (`cold_cache`: up to 20 more steps, each after a 1 GiB read
that evicts L2 and the Infinity Cache, timed with events; context beside
`value`, which is the warm timed region).

Other workloads (--workload), each one JSON line in the same form:
  varlen  the bf16 varlen prefill: 8 sequences with lengths uniform in
          [128, 2048], 8192 channels (16 q, 16 k, 32 v heads), half with
          initial states; conv + post-conv, then the prefill
  verify  speculative verify: 36 layers of conv shift + post-conv + decode
          step (no state write), then one batched commit of n_keep tokens
          (32 sequences, 1..8 draft tokens each)
  long    one 32768-token prefill layer
  mixed-unfused
          the mixed serving step with the decode tokens in the conv +
          post-conv launch and a separate step launch
  verify-fused
          verify with each layer's conv, post-conv and step in one launch
  out-norm
          the gated output norm on the mixed serving step's o, 24 layers
  gates   the gate computation for the mixed serving step, 24 layers
  long-seg
          the 32768-token prefill split into 5 segments

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                  [--serial] [--workload mixed|varlen|verify|...]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import multiprocessing
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFS = 2500.0
METRIC = "GDN layer tokens/s (conv+postconv+delta-rule) and % of HBM roofline, 1 GPU"
# calibrated FETCH_SIZE / WRITE_SIZE traffic per kernel, one file per workload
TRAFFIC_FILES = {"varlen": os.path.join(ROOT, "profiles", "traffic_varlen_prefill_bf16.json"),
                 "mixed": os.path.join(ROOT, "profiles", "traffic_mixed_serving_24L_bf16.json")}
CPU_POOL_MAX = 16          # host processes for the CPU baseline (one GPU's share of the box)
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


# ------------------------------------------------------------ CPU baseline
# The oracle, unchanged, on one layer of the workload, spread over a pool of
# host processes.  The conv is depthwise and every group of k-heads with
# their v-heads is independent of the others, so a unit of work is a run of
# sequences and a group of heads: the oracle's conv, post-conv and per-token
# recurrence on that group's channels.  Units are handed out longest first.

_CPU = {}    # one layer's inputs (numpy), shared with forked workers


def _cpu_unit(unit):
    import numpy as np
    from oracle import gdn_oracle as O
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:                              # pragma: no cover
        pass
    s0, s1, kh0, nk = unit
    d = _CPU
    Hk, Hv, act = d["Hk"], d["Hv"], d["act"]
    G = Hv // Hk
    cu = d["cu"]
    b, e = int(cu[s0]), int(cu[s1])
    cu_l = [int(c) - b for c in cu[s0:s1 + 1]]
    qk = np.arange(kh0 * 128, (kh0 + nk) * 128)
    chans = np.concatenate([qk, Hk * 128 + qk, 2 * Hk * 128 + np.arange(kh0 * G * 128, (kh0 + nk) * G * 128)])
    heads = np.arange(kh0 * G, (kh0 + nk) * G)
    hi = d["hi"][s0:s1]
    y, _ = O.causal_conv(d["x"][b:e][:, chans].astype(np.float64), d["w"][chans], None,
                         d["cs"][s0:s1][:, :, chans], hi, cu_l, True)
    q, k, v = O.postconv_l2(O.round_to(y, act), nk, nk * G, 128, 128, 1e-6)
    q, k, v = (O.round_to(a, act) for a in (q, k, v))
    o, _ = O.delta_rule_recurrent(q, k, v, d["g"][b:e][:, heads], d["beta"][b:e][:, heads],
                                  d["st"][s0:s1][:, heads], hi, cu_l, nk, nk * G)
    return float(np.abs(o).sum())


def _cpu_units(cu, Hk, head_groups=4, min_tokens=256):
    """Runs of consecutive sequences of at least min_tokens tokens (a long
    sequence alone), times head_groups groups of k-heads; longest first."""
    runs, s0 = [], 0
    nseq = len(cu) - 1
    for s in range(nseq):
        if cu[s + 1] - cu[s0] >= min_tokens or s == nseq - 1:
            runs.append((s0, s + 1))
            s0 = s + 1
    nk = max(1, Hk // head_groups)
    units = [(a, b, kh, min(nk, Hk - kh)) for a, b in runs for kh in range(0, Hk, nk)]
    return sorted(units, key=lambda u: -(cu[u[1]] - cu[u[0]]))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(lb, layers: int) -> dict:
    """The oracle on one layer's whole batch (every sequence, every head),
    over min(16, cpu_count) processes forked before the GPU is touched.
    Result in tokens/s of that layer, the metric's unit (layer-tokens/s)."""
    import numpy as np
    import torch
    _CPU.clear()
    _CPU.update(x=lb.x.float().numpy(), w=lb.conv_w.numpy().astype(np.float64),
                cs=lb.conv_state.numpy().astype(np.float64), st=lb.state.numpy().astype(np.float64),
                g=lb.g.numpy().astype(np.float64), beta=lb.beta.numpy().astype(np.float64),
                hi=lb.has_init.numpy(), cu=lb.cu_seqlens.numpy().astype(np.int64),
                Hk=lb.geo.Hk, Hv=lb.geo.Hv, act=lb.act)
    units = _cpu_units(_CPU["cu"], lb.geo.Hk)
    nproc = os.cpu_count() or 1
    workers = min(CPU_POOL_MAX, nproc, len(units))
    if torch.cuda.is_initialized():
        workers = 1          # never fork a process that holds the GPU
    t0 = time.perf_counter()
    if workers > 1:
        with multiprocessing.get_context("fork").Pool(workers) as pool:
            t0 = time.perf_counter()
            list(pool.imap_unordered(_cpu_unit, units, chunksize=1))
            dt = time.perf_counter() - t0
    else:
        for u in units:
            _cpu_unit(u)
        dt = time.perf_counter() - t0
    _CPU.clear()
    return {"value": round(lb.N / dt, 1), "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"one of the {layers} layers: all {lb.nseq} sequences ({lb.N} tokens) and all "
                      f"{lb.geo.Hv} v-heads through the oracle's conv, post-conv and per-token "
                      f"recurrence (float64 numpy), {len(units)} units (a run of sequences x 4 of the "
                      f"{lb.geo.Hk} k-heads with their v-heads) over {workers} host processes",
            "seconds": round(dt, 2), "nproc": nproc, "cpu_model": cpu_model()}


# ------------------------------------------------------------------ workloads
# Each builder returns a plan: the ordered kernel launches of one step, the
# algorithmic bytes per kernel name (summed over the step), the tokens of
# one step and the config dict.

class Plan:
    """The ordered launches of one step.  ops: ("run", name, fn, stream),
    ("mark", key, stream) records an event on a stream, ("wait", key,
    stream) makes a stream wait for it; stream 0 is the caller's stream."""

    def __init__(self):
        self.ops = []
        self.bytes = {}          # kernel name -> bytes per step
        self.count = {}          # kernel name -> launches per step
        self.flops = {}          # kernel name -> dense flops per step
        self.tokens = 0
        self.dtype = "bf16"      # arithmetic type of the step's activations
        self.config = {}
        self.keep = []           # tensors kept alive
        self.lb = None           # one layer's inputs (CPU), for the CPU baseline

    def add(self, name, fn, nbytes, flops=0.0, stream=0):
        self.ops.append(("run", name, fn, stream))
        self.bytes[name] = self.bytes.get(name, 0) + nbytes
        self.count[name] = self.count.get(name, 0) + 1
        if flops:
            self.flops[name] = self.flops.get(name, 0.0) + flops

    def mark(self, key, stream=0):
        self.ops.append(("mark", key, stream))

    def wait(self, key, stream=0):
        self.ops.append(("wait", key, stream))

    @property
    def launches(self):
        return [(op[1], op[2]) for op in self.ops if op[0] == "run"]


# HIP event flags (hip_runtime_api.h).  The bench's events are created with
# hipEventDisableSystemFence: by default recording an event performs a
# system-scope release, which writes the caches back at every record (about
# 9 us per record after a kernel that wrote hundreds of MB, measured on the
# mixed serving step: 5.56 against 5.24 ms per step); a timing or ordering
# marker inside the step should not add that cost.  Work on one device stays
# ordered and visible through the kernels' own dispatch fences.
HIP_EVENT_DISABLE_TIMING = 0x2
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
# hipStreamUpdateCaptureDependencies: replace the capture's dependency set
HIP_STREAM_SET_CAPTURE_DEPENDENCIES = 0x1


class HipEvents:
    """hipEvent_t objects with explicit flags, through the HIP runtime that
    torch loaded (looked up in the process's mappings, so no second runtime
    is loaded)."""

    def __init__(self):
        import ctypes
        path = None
        with open("/proc/self/maps") as f:
            for ln in f:
                if "libamdhip64" in ln:
                    path = ln.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded")
        self.ct = ctypes
        self.lib = ctypes.CDLL(path)

    def create(self, timing=True):
        ev = self.ct.c_void_p()
        flags = HIP_EVENT_DISABLE_SYSTEM_FENCE | (0 if timing else HIP_EVENT_DISABLE_TIMING)
        rc = self.lib.hipEventCreateWithFlags(self.ct.byref(ev), self.ct.c_uint(flags))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags: {rc}")
        return ev

    def record(self, ev, stream, node=False):
        """Record ev on stream.  node=True, for a stream under capture: add
        an event-record node to the graph being captured, after the
        stream's current dependencies, and make it the stream's only
        dependency (an event recorded during capture is otherwise only an
        ordering edge, and this runtime refuses hipEventRecordExternal)."""
        ct, sp = self.ct, self.ct.c_void_p(stream.cuda_stream)
        if not node:
            rc = self.lib.hipEventRecord(ev, sp)
            if rc != 0:
                raise RuntimeError(f"hipEventRecord: {rc}")
            return
        status, cid, graph = ct.c_int(), ct.c_ulonglong(), ct.c_void_p()
        deps, ndeps = ct.POINTER(ct.c_void_p)(), ct.c_size_t()
        rc = self.lib.hipStreamGetCaptureInfo_v2(sp, ct.byref(status), ct.byref(cid), ct.byref(graph),
                                                 ct.byref(deps), ct.byref(ndeps))
        if rc != 0 or not graph:
            raise RuntimeError(f"hipStreamGetCaptureInfo_v2: {rc} (is the stream capturing?)")
        nd = ct.c_void_p()
        rc = self.lib.hipGraphAddEventRecordNode(ct.byref(nd), graph, deps, ndeps, ev)
        if rc != 0:
            raise RuntimeError(f"hipGraphAddEventRecordNode: {rc}")
        rc = self.lib.hipStreamUpdateCaptureDependencies(sp, ct.byref(nd), ct.c_size_t(1),
                                                         ct.c_uint(HIP_STREAM_SET_CAPTURE_DEPENDENCIES))
        if rc != 0:
            raise RuntimeError(f"hipStreamUpdateCaptureDependencies: {rc}")

    def wait(self, stream, ev):
        rc = self.lib.hipStreamWaitEvent(self.ct.c_void_p(stream.cuda_stream), ev, self.ct.c_uint(0))
        if rc != 0:
            raise RuntimeError(f"hipStreamWaitEvent: {rc}")

    def elapsed(self, a, b):
        ms = self.ct.c_float()
        rc = self.lib.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime: {rc}")
        return ms.value


class Runner:
    """Issues a plan's ops on the caller's stream and side streams (default
    priority), optionally bracketing every launch with HIP events on the
    stream it runs on.  serial=True puts everything on the caller's stream."""

    def __init__(self, plan, stream, serial=False):
        import torch
        self.plan = plan
        self.serial = serial
        n = 1 if serial else 1 + max([op[3] if op[0] == "run" else op[2] for op in plan.ops], default=0)
        self.streams = [stream] + [torch.cuda.Stream(device=stream.device) for _ in range(n - 1)]
        self.hip = HipEvents()
        self.marks = {op[1]: self.hip.create(timing=False) for op in plan.ops if op[0] == "mark"}
        self.n_runs = sum(1 for op in plan.ops if op[0] == "run")

    def events(self):
        return [(self.hip.create(), self.hip.create()) for _ in range(self.n_runs)]

    def timed(self, only=None, stride=1):
        """Indices (among the step's launches) that carry events: every
        launch, or every stride-th launch of kernel `only`."""
        names = [nm for nm, _ in self.plan.launches]
        if only is None:
            return set(range(len(names)))
        return set([i for i, nm in enumerate(names) if nm == only][::stride])

    def step(self, ev=None, only=None, capture=False, stride=1):
        """One step; with ev, launches are bracketed by their event pair
        (every stride-th launch of kernel `only` when it is given).  capture:
        the streams are being captured, and the timing records become
        event-record nodes of the graph."""
        import torch
        i = 0
        timed_set = self.timed(only, stride) if ev is not None else set()
        for op in self.plan.ops:
            if op[0] == "run":
                st = self.streams[0 if self.serial else op[3]]
                timed = i in timed_set
                with torch.cuda.stream(st):
                    if timed:
                        self.hip.record(ev[i][0], st, capture)
                    op[2]()
                    if timed:
                        self.hip.record(ev[i][1], st, capture)
                i += 1
            elif self.serial:
                continue
            elif op[0] == "mark":
                self.hip.record(self.marks[op[1]], self.streams[op[2]])
            else:
                self.hip.wait(self.streams[op[2]], self.marks[op[1]])

    def capture(self, events=None, only=None, steps=1, stride=1):
        """A HIP graph of `steps` steps (len(events) when events are given,
        each step's timing records of kernel `only` captured as event-record
        nodes).  The caller's stream hosts the capture and the side streams
        join it through the plan's marks, so replaying the graph issues the
        same launches with the same dependencies as step()."""
        import torch
        g = torch.cuda.CUDAGraph()
        main = self.streams[0]
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            self.streams[0] = torch.cuda.current_stream()
            try:
                for i in range(len(events) if events is not None else steps):
                    self.step(events[i] if events is not None else None, only=only, capture=True,
                              stride=stride)
            finally:
                self.streams[0] = main
        return g

    def stage_ms(self, ev, only=None, stride=1):
        """Per-kernel-name milliseconds of one step from its event pairs (a
        kernel timed on a stride-th of its launches: their mean times its
        launch count)."""
        acc, n = {}, {}
        names = [nm for nm, _ in self.plan.launches]
        timed_set = self.timed(only, stride)
        for i, (nm, (a, b)) in enumerate(zip(names, ev)):
            if i in timed_set:
                acc[nm] = acc.get(nm, 0.0) + self.hip.elapsed(a, b)
                n[nm] = n.get(nm, 0) + 1
        return {nm: acc[nm] / n[nm] * self.plan.count[nm] for nm in acc}

    def instrumented(self, steps, median=False):
        """Per-kernel-name milliseconds per step over `steps` steps with
        every launch bracketed by events: the mean, or with median=True the
        median over the steps after the first (robust to a cold first step)."""
        import torch
        evs = [self.events() for _ in range(steps)]
        for ev in evs:
            self.step(ev)
        torch.cuda.synchronize()
        per = [self.stage_ms(ev) for ev in evs]
        if median and len(per) > 1:
            per = per[1:]
            out = {}
            for nm in per[0]:
                v = sorted(p[nm] for p in per)
                out[nm] = v[len(v) // 2] if len(v) % 2 else 0.5 * (v[len(v) // 2 - 1] + v[len(v) // 2])
            return out
        return {nm: sum(p[nm] for p in per) / len(per) for nm in per[0]}


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


def plan_mixed(dev, fused=True, layers=24, make_layer=None):
    """`layers` layers of the mixed serving step (24; make_layer(layer)
    gives a layer's inputs, inputs.mixed_serving_layer by default).  Per
    layer the decode tokens' launch (fused conv + post-conv + step, or the
    step alone after a conv + post-conv over all tokens when not fused) goes
    to side stream 1 once the layer's conv + post-conv is done, and stream 0
    waits for it before the next layer: it runs beside the prefill, which
    touches other sequences."""
    from linear_attention_layers_amd import gdn, inputs
    L = layers
    make_layer = make_layer or inputs.mixed_serving_layer
    p = Plan()
    for layer in range(L):
        lb = make_layer(layer)
        if layer == 0:
            p.lb = lb
        d = _layer_on_device(lb, dev)
        npre = lb.meta["n_prefill"]
        Npre = int(lb.cu_seqlens[npre])
        N, C, Hk, Hv = lb.N, lb.geo.C, lb.geo.Hk, lb.geo.Hv
        ndec = lb.nseq - npre
        d["chunks"] = gdn.gdn_make_chunks_device(d["cu"], N)
        d["cu_pre"] = d["cu"][:npre + 1]
        d["cu_dec"] = (d["cu"][npre:] - Npre).contiguous()
        # views of the prefill and decode parts, taken once (a view costs the
        # host a few microseconds per launch)
        P_ = {nm: d[nm][:Npre] for nm in ("x", "y", "q", "k", "v", "o", "g", "beta")}
        P_["cs"], P_["st"] = d["cs"][:npre], d["st"][:npre]
        D_ = {nm: d[nm][Npre:] for nm in ("x", "q", "k", "v", "o", "g", "beta")}
        D_["cs"], D_["st"] = d["cs"][npre:], d["st"][npre:]
        d["pre"], d["dec"] = P_, D_
        if fused:
            # conv and post-conv over the prefill tokens only; the decode
            # tokens go through the fused launch
            d["chunks_pre"] = gdn.gdn_make_chunks_device(d["cu_pre"], Npre)
            add_conv_post(p, P_["x"], d["w"], P_["cs"], None, d["cu_pre"],
                          d["chunks_pre"] if descriptors_needed() else None, True,
                          Hk, Hv, Npre, C, npre, npre, P_["y"], P_["q"], P_["k"], P_["v"])
        else:
            add_conv_post(p, d["x"], d["w"], d["cs"], None, d["cu"], d["chunks"] if descriptors_needed() else None,
                          True, Hk, Hv, N, C,
                          lb.nseq, lb.nseq, d["y"], d["q"], d["k"], d["v"])
        p.mark(f"conv{layer}", 0)
        p.wait(f"conv{layer}", 1)
        p.add("prefill", lambda P_=P_, d=d: gdn.gdn_delta_rule_prefill(
                  P_["q"], P_["k"], P_["v"], P_["g"], P_["beta"], d["cu_pre"], P_["st"], None, o=P_["o"]),
              recurrence_bytes(Npre, Hk, Hv, 2, npre, npre), 11.0 * 128 * 128 * Npre * Hv)
        if fused:
            p.add("fused", lambda D_=D_, d=d, Hk=Hk, Hv=Hv: gdn.gdn_decode_fused(
                      D_["x"], d["w"], None, D_["cs"], d["cu_dec"], D_["g"], D_["beta"], D_["st"], Hk, Hv, 1e-6,
                      None, o=D_["o"], write_conv_state=True, commit_state=True),
                  fused_bytes(N - Npre, C, Hk, Hv, 2, ndec, True, ndec, False), stream=1)
        else:
            p.add("step", lambda D_=D_, d=d: gdn.gdn_delta_rule_step(
                      D_["q"], D_["k"], D_["v"], D_["g"], D_["beta"], d["cu_dec"], D_["st"], None, o=D_["o"],
                      commit_state=True),
                  recurrence_bytes(N - Npre, Hk, Hv, 2, ndec, ndec), stream=1)
        p.mark(f"dec{layer}", 1)
        p.wait(f"dec{layer}", 0)
        p.keep.append(d)
        p.tokens += N
        p.config = {"workload": "mixed_serving_24L_bf16" + ("" if fused else "_unfused"),
                    "prefill_seqs": npre, "decode_seqs": ndec,
                    "tokens_per_layer": N, "channels": C, "Hk": Hk, "Hv": Hv, "head_dim": 128,
                    "layers": L, "state_dtype": "f32", "seed": 5000,
                    "decode": ("fused conv + post-conv + step" if fused else "step") + " on a side stream"}
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
         "mixed-unfused": lambda dev: plan_mixed(dev, fused=False), "out-norm": plan_out_norm,
         "gates": plan_gates, "long-seg": lambda dev: plan_long(dev, nseg=5)}


def cpu_sample(workload):
    """(one layer's inputs on the CPU, layers in the workload) for the CPU
    baseline, or None where the workload has no baseline leg."""
    from linear_attention_layers_amd import inputs
    if workload == "varlen":
        return inputs.varlen_prefill(), 1
    if workload == "mixed":
        return inputs.mixed_serving_layer(0), 24
    return None


def cold_pass(runner, reps):
    """Each of `reps` steps runs right after a 1 GiB read of an unrelated
    buffer (clean lines: it evicts L2 and the Infinity Cache without leaving
    write-backs behind), with HIP events around every kernel and around the
    step; the read itself is outside the events."""
    import torch
    plan = runner.plan
    main = runner.streams[0]
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=main.device)
    names = list(dict.fromkeys(nm for nm, _ in plan.launches))
    acc = {nm: 0.0 for nm in names}
    total = 0.0
    for _ in range(reps):
        scratch.sum()
        ev = runner.events()
        t0, t1 = runner.hip.create(), runner.hip.create()
        runner.hip.record(t0, main)
        runner.step(ev)
        for st in runner.streams[1:]:
            main.wait_stream(st)
        runner.hip.record(t1, main)
        torch.cuda.synchronize()
        for nm, ms in runner.stage_ms(ev).items():
            acc[nm] += ms
        total += runner.hip.elapsed(t0, t1)
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


def copy_bandwidth(dev, nbytes: int = 1 << 30, reps: int = 10) -> dict:
    """A plain device-to-device copy of nbytes (torch's copy kernel), timed
    with events after two untimed copies: bytes read and written over the
    median time.  Context for the stages' HBM fractions: a kernel that
    streams its bytes once gets about this far on the same GPU."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(2):
        dst.copy_(src)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) / 1e3)
    del src, dst
    t = sorted(ts)[len(ts) // 2]
    gbs = 2 * nbytes / t / 1e9
    return {"GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "bytes_moved": 2 * nbytes,
            "kernel": "torch copy_ of 1 GiB on one device (hipMemcpyAsync, the HIP runtime's copy kernel), "
                      "median of 10"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--workload", choices=sorted(PLANS), default="mixed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--serial", action="store_true",
                    help="issue every launch on one stream (no side stream for the decode tokens)")
    ap.add_argument("--time-stride", type=int, default=4,
                    help="in the timed region, bracket every n-th launch of the dominant kernel in "
                         "each step with events, its first launch included (1: every launch; each "
                         "bracketed launch adds two marker packets to the queue)")
    ap.add_argument("--eager", action="store_true",
                    help="issue the timed steps' launches from the host one by one instead of "
                         "replaying them as one captured HIP graph")
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
              "this benchmark measures the one-GPU share only)", file=sys.stderr)
        sys.exit(2)
    default_steps = {"varlen": 100, "verify": 20, "long": 20, "mixed": 40, "verify-fused": 20,
                     "mixed-unfused": 20, "out-norm": 20, "gates": 20, "long-seg": 20}[args.workload]
    steps = args.steps if args.steps is not None else default_steps
    warmup = args.warmup if args.warmup is not None else max(2, steps // 10)

    import torch

    # the CPU baseline runs first: its worker processes are forked before
    # this process touches the GPU
    cpu = None
    sample = None if args.no_cpu_baseline or args.copy_calibration else cpu_sample(args.workload)
    if sample is not None:
        cpu = cpu_baseline(*sample)
        del sample

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
    runner = Runner(plan, stream, serial=args.serial)

    # warm-up steps with every launch timed: the kernel with the largest
    # median time per step over them (the first left out) is the dominant one
    names = list(dict.fromkeys(nm for nm, _ in plan.launches))
    warm_ms = runner.instrumented(warmup, median=True)
    dominant = max([nm for nm in names if plan.bytes.get(nm)], key=lambda nm: warm_ms[nm])

    # the timed region: K steps bracketed by synchronisation, events around
    # the dominant kernel's launches only (on the stream each runs on).  By
    # default the K steps are captured once as a HIP graph (their launches,
    # stream joins and the dominant kernel's event records as nodes) and the
    # graph is replayed twice: a warm replay, then the timed one; --eager
    # issues every launch from the host inside the timed region instead.
    events = [runner.events() for _ in range(steps)]
    graph = None
    launch = "eager"
    if not args.eager:
        try:
            graph = runner.capture(events, only=dominant, stride=args.time_stride)
            graph.replay()
            launch = "hip graph (the timed steps captured once, replayed)"
        except Exception as exc:  # noqa: BLE001 - any capture failure falls back to eager launches
            # a runtime that cannot capture these launches still gets its
            # measurement, issued launch by launch (and says so)
            graph = None
            torch.cuda.synchronize()
            launch = f"eager (graph capture failed: {str(exc).splitlines()[0][:120]})"
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        graph.replay()
    else:
        for i in range(steps):
            runner.step(events[i], only=dominant, stride=args.time_stride)
    enqueued = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_ms = sum(runner.stage_ms(ev, only=dominant, stride=args.time_stride)[dominant]
                 for ev in events) / steps
    del graph

    # every kernel's time from an instrumented pass after the timed region;
    # the dominant kernel's entry is the timed region's own measurement
    per_step_ms = runner.instrumented(min(steps, 10))
    per_step_ms[dominant] = dom_ms

    ms_per_step = wall * 1e3 / steps
    tokens_per_s = plan.tokens / (ms_per_step / 1e3)
    copy_bw = copy_bandwidth(dev)
    stages = {}
    for nm in names:
        t = per_step_ms[nm] / 1e3
        rec = {"us_per_launch": round(per_step_ms[nm] * 1e3 / plan.count[nm], 2),
               "launches": plan.count[nm]}
        if plan.bytes.get(nm):
            rec["GB/s"] = round(plan.bytes[nm] / t / 1e9, 1)
            rec["hbm_frac"] = round(plan.bytes[nm] / t / 1e9 / HBM_PEAK_GBS, 4)
            rec["of_copy"] = round(plan.bytes[nm] / t / 1e9 / copy_bw["GB/s"], 4)
        if plan.flops.get(nm):
            tf = plan.flops[nm] / t / 1e12
            rec["mfma_TFLOP/s"] = round(tf, 2)
            rec["mfma_frac_bf16_dense"] = round(tf / BF16_MFMA_PEAK_TFS, 4)
        rec["timing"] = "timed region" if nm == dominant else "instrumented pass"
        stages[nm] = rec
    achieved = plan.bytes[dominant] / (per_step_ms[dominant] / 1e3) / 1e9

    traffic = None
    if args.workload in TRAFFIC_FILES and not (args.split_conv or args.chunk_descriptors or args.serial):
        try:
            with open(TRAFFIC_FILES[args.workload]) as f:
                rec = json.load(f).get(dominant)
            if rec and rec.get("source_hash") == source_hash(dominant):
                traffic = rec["bytes_per_launch"]
        except (OSError, ValueError):
            pass

    roofline = {"bound": "hbm", "kernel": dominant, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "algorithmic_bytes": plan.bytes[dominant] // plan.count[dominant]}
    if plan.flops.get(dominant):
        # the chunked prefill's dense contractions against the bf16 MFMA peak
        roofline["mfma_frac"] = stages[dominant]["mfma_frac_bf16_dense"]
    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "host_enqueue_ms_per_step": round(enqueued * 1e3 / steps, 4),
        "launch": launch,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": plan.dtype,
        "data": "synthetic",
        "config": plan.config,
        "roofline": roofline,
        "stages": stages,
        "copy_bandwidth": copy_bw,
    }
    if not args.no_cold:
        out["cold_cache"] = cold_pass(runner, min(steps, 20))
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
