"""Shared helpers for the GPU parity tests: tensor movement, the comparison
bars, and runners that push a LayerBatch through the HIP library or the
oracle.  The oracle and the library never call each other; tests feed both
the same seeded inputs and compare."""
from __future__ import annotations

import numpy as np
import torch

from oracle import gdn_oracle as O

ACT = {"f32": torch.float32, "bf16": torch.bfloat16}

# Tolerances: conv and SiLU relative bounds in float32, ulp bounds for the
# L2 outputs, normwise relative bounds for the recurrence (per (token, head)
# output vector, per (sequence, head) state matrix).
CONV_REL_F32 = 1e-6
SILU_REL_F32 = 1e-6
L2_ULP_F32 = 2
L2_ULP_BF16 = 1
REC_F32 = 1e-5
REC_BF16 = 2e-2


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype != torch.float64 \
        else t.detach().cpu().numpy()


def dev(t, device="cuda"):
    return None if t is None else t.to(device)


# --------------------------------------------------------------- comparisons

def ulp_dist_f32(a, b) -> np.ndarray:
    """|a - b| in units of float32 spacing (integer distance of the ordered
    bit patterns)."""
    ai = np.asarray(a, dtype=np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, dtype=np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7fffffff), ai)
    bi = np.where(bi < 0, -(bi & 0x7fffffff), bi)
    return np.abs(ai - bi)


def ulp_dist_bf16(a, b) -> np.ndarray:
    """Distance in bf16 steps between two arrays of bf16-representable values."""
    ai = (np.asarray(a, dtype=np.float32).view(np.int32) >> 16).astype(np.int64)
    bi = (np.asarray(b, dtype=np.float32).view(np.int32) >> 16).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7fff), ai)
    bi = np.where(bi < 0, -(bi & 0x7fff), bi)
    return np.abs(ai - bi)


def bf16_ulp(x) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_conv(y_gpu, y_ref, scale, act: str, what="conv"):
    """float32: |dy| <= 1e-6 * (|bias| + sum|w x|); bf16: at most one bf16
    step away from the correctly rounded value, plus the same
    condition-scaled float32 term (under cancellation the float32 sum itself
    may sit on the other side of a rounding boundary)."""
    y_gpu = np.asarray(y_gpu, np.float64)
    if act == "f32":
        err = np.abs(y_gpu - y_ref)
        bound = CONV_REL_F32 * scale
    else:
        y_rb = O.round_to_bf16(y_ref)
        err = np.abs(y_gpu - y_rb)
        bound = bf16_ulp(y_rb) * 1.0 + CONV_REL_F32 * scale
    bad = err > bound + 1e-30
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside bound; worst excess " \
                          f"{np.max(err - bound):.3g}"


def conv_scale(x, w, bias, conv_state, has_init, cu):
    """|bias| + sum_j |w_j x_j| per output element (the conv's condition)."""
    y, _ = O.causal_conv(np.abs(x), np.abs(w), None if bias is None else np.abs(bias),
                         np.abs(conv_state), has_init, cu, write_state=False)
    return y


def check_normwise(got, ref, tol, axes, what):
    """max |got - ref| <= tol * max |ref| over each slice spanned by `axes`."""
    got = np.asarray(got, np.float64)
    err = np.max(np.abs(got - ref), axis=axes)
    mag = np.max(np.abs(ref), axis=axes)
    ratio = err / np.maximum(mag, 1e-30)
    worst = float(np.max(ratio)) if ratio.size else 0.0
    assert worst <= tol, f"{what}: worst normwise relative error {worst:.3g} > {tol}"
    return worst


# --------------------------------------------------------------- runners

def gpu_layer(lb, write_state=True, eps=1e-6, out_dtype=None, device="cuda"):
    """conv -> post-conv -> prefill through the library; returns a dict of
    device tensors (y, q, k, v, o, conv_state, state)."""
    from linear_attention_layers_amd import gdn
    x = dev(lb.x, device)
    cu = dev(lb.cu_seqlens, device)
    hi = dev(lb.has_init, device)
    cs = dev(lb.conv_state, device).contiguous()
    st = dev(lb.state, device).contiguous()
    chunks = gdn.gdn_make_chunks_device(cu, lb.N)
    y = gdn.gdn_causal_conv_fwd(x, dev(lb.conv_w, device), dev(lb.conv_b, device), cs, hi, cu,
                                chunks, write_state)
    q, k, v = gdn.gdn_postconv_l2(y, lb.geo.Hk, lb.geo.Hv, eps, out_dtype=out_dtype)
    g = dev(lb.g, device)
    beta = dev(lb.beta, device)
    o = gdn.gdn_delta_rule_prefill(q, k, v, g, beta, cu, st, hi)
    return dict(y=y, q=q, k=k, v=v, o=o, conv_state=cs, state=st, g=g, beta=beta, cu=cu, hi=hi)
