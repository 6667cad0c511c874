"""Thin ctypes binding over libgdn.so (C ABI in include/gdn.h).

Each function here has the name of the C entry point it calls, turns torch
tensors into pointers, sizes and dtype codes, passes torch's current HIP
stream, and raises GdnError on a non-OK status.  No step of the computation
runs in Python: every one is a HIP kernel inside the library.  Importing
this module fails if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m linear_attention_layers_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)


def _hip_runtimes():
    """Distinct HIP runtime libraries mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


# The library must share torch's HIP runtime: if it was loaded before torch,
# a second runtime is mapped and device pointers and streams would not match.
if len(_hip_runtimes()) > 1:
    raise ImportError("two HIP runtimes are loaded (" + ", ".join(_hip_runtimes()) + "); "
                      "import torch before loading libgdn.so")

GDN_F32 = 0
GDN_BF16 = 1
CHUNK_LEN = 64

_vp = ctypes.c_void_p
_i32 = ctypes.c_int
_i64 = ctypes.c_int64
_f32 = ctypes.c_float


class gdn_chunk(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_int32), ("begin", ctypes.c_int32),
                ("end", ctypes.c_int32), ("flags", ctypes.c_int32)]


class gdn_layer_io(ctypes.Structure):
    _fields_ = [("x", _vp), ("x_row_stride", _i64), ("conv_state", _vp), ("state", _vp),
                ("k", _vp), ("v", _vp), ("g", _vp), ("beta", _vp)]


def _sig(name, args, res=_i32):
    fn = getattr(_lib, name)
    fn.argtypes = args
    fn.restype = res
    return fn


_abi_version = _sig("gdn_abi_version", [])
_status_string = _sig("gdn_status_string", [_i32], ctypes.c_char_p)
_last_error = _sig("gdn_last_error", [], ctypes.c_char_p)
_chunk_capacity = _sig("gdn_chunk_capacity", [_i32, _i32, _i32])
_make_chunks = _sig("gdn_make_chunks", [_vp, _i32, _i32, _vp, _i32])
_make_chunks_device = _sig("gdn_make_chunks_device", [_vp, _i32, _i32, _vp, _i32, _vp])
_conv = _sig("gdn_causal_conv_fwd", [_vp, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                     _i32, _i32, _i32, _vp, _vp])
_conv_post = _sig("gdn_conv_postconv_fwd", [_vp, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                            _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp, _vp])
_postconv = _sig("gdn_postconv_l2", [_vp, _i64, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp,
                                     _vp, _vp, _i32, _vp])
_prefill = _sig("gdn_delta_rule_prefill", [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32,
                                           _i32, _i32, _i32, _vp, _vp, _vp, _vp])
_seg_ws = _sig("gdn_prefill_segmented_workspace", [_i32, _i32, _i32], ctypes.c_size_t)
_prefill_seg = _sig("gdn_delta_rule_prefill_segmented", [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32,
                                                         _i32, _i32, _i32, _i32, _vp, _vp, _vp, _i32, _vp,
                                                         ctypes.c_size_t, _vp])
_prefill_seg_na = _sig("gdn_delta_rule_prefill_segmented_noalloc", [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32,
                                                                    _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                                                    _i32, _vp])
_step = _sig("gdn_delta_rule_step", [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                     _i32, _i32, _vp, _vp, _vp, _i32, _vp])
_commit = _sig("gdn_commit", [_vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                              _vp])
_decode_fused = _sig("gdn_decode_fused", [_vp, _i64, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                          _i32, _i32, _f32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                          _vp])

_out_norm = _sig("gdn_out_norm", [_vp, _vp, _i32, _vp, _i32, _i32, _i32, _f32, _vp, _vp])
_gates = _sig("gdn_gates", [_vp, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp])

EXPORTED = ["gdn_abi_version", "gdn_status_string", "gdn_last_error", "gdn_chunk_capacity",
            "gdn_make_chunks", "gdn_make_chunks_device", "gdn_causal_conv_fwd", "gdn_conv_postconv_fwd",
            "gdn_postconv_l2", "gdn_delta_rule_prefill", "gdn_prefill_segmented_workspace",
            "gdn_delta_rule_prefill_segmented", "gdn_delta_rule_prefill_segmented_noalloc",
            "gdn_delta_rule_step", "gdn_commit",
            "gdn_decode_fused", "gdn_out_norm", "gdn_gates"]


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _last_error().decode(errors="replace")
        super().__init__(f"{where}: {_status_string(status).decode()} ({msg})")


def _check(status: int, where: str):
    if status != 0:
        raise GdnError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else _vp(t.data_ptr())


def _code(dtype) -> int:
    if dtype == torch.float32:
        return GDN_F32
    if dtype == torch.bfloat16:
        return GDN_BF16
    raise TypeError(f"unsupported dtype {dtype}")


def _torch_dtype(code: int):
    return torch.float32 if code == GDN_F32 else torch.bfloat16


def _stream(stream) -> _vp:
    if stream is None:
        stream = torch.cuda.current_stream()
    return _vp(stream.cuda_stream)


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _dense(t: torch.Tensor, name: str):
    _require(t.is_contiguous(), f"{name} must be contiguous")


# ---------------------------------------------------------------- info

def gdn_abi_version() -> int:
    return int(_abi_version())


def gdn_status_string(status: int) -> str:
    return _status_string(status).decode()


def gdn_last_error() -> str:
    return _last_error().decode(errors="replace")


# ---------------------------------------------------------------- chunks

def gdn_chunk_capacity(N: int, nseq: int, chunk_len: int = CHUNK_LEN) -> int:
    return int(_chunk_capacity(N, nseq, chunk_len))


def gdn_make_chunks(cu_seqlens: Sequence[int], chunk_len: int = CHUNK_LEN) -> torch.Tensor:
    """Host chunk list: returns an int32 CPU tensor [n, 4] = (seq, begin, end, flags)."""
    cu = torch.as_tensor(list(int(c) for c in cu_seqlens), dtype=torch.int32)
    nseq = cu.numel() - 1
    cap = max(gdn_chunk_capacity(int(cu[-1]), nseq, chunk_len), 1)
    out = torch.empty(cap, 4, dtype=torch.int32)
    n = int(_make_chunks(_ptr(cu), nseq, chunk_len, _ptr(out), cap))
    if n < 0:
        raise GdnError(-n, "gdn_make_chunks")
    return out[:n].clone()


def gdn_make_chunks_device(cu_seqlens: torch.Tensor, N: int, chunk_len: int = CHUNK_LEN,
                           out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Device chunk list with gdn_chunk_capacity slots (unused slots seq = -1)."""
    _require(cu_seqlens.is_cuda and cu_seqlens.dtype == torch.int32, "cu_seqlens: int32 device tensor")
    nseq = cu_seqlens.numel() - 1
    cap = gdn_chunk_capacity(N, nseq, chunk_len)
    if out is None:
        out = torch.empty(max(cap, 1), 4, dtype=torch.int32, device=cu_seqlens.device)
    _require(out.shape[0] >= cap and out.dtype == torch.int32 and out.is_contiguous(), "out too small")
    st = int(_make_chunks_device(_ptr(cu_seqlens), nseq, chunk_len, _ptr(out), cap, _stream(stream)))
    if st != 0:
        raise GdnError(-st, "gdn_make_chunks_device")
    return out[:cap]


# ---------------------------------------------------------------- conv

def gdn_causal_conv_fwd(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor],
                        conv_state: torch.Tensor, has_initial_state: Optional[torch.Tensor],
                        cu_seqlens: torch.Tensor, chunks: torch.Tensor, write_state: bool,
                        y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    N, C = x.shape
    _require(x.stride(1) == 1, "x rows must be contiguous")
    nseq = cu_seqlens.numel() - 1
    if y is None:
        y = torch.empty(N, C, dtype=x.dtype, device=x.device)
    _dense(y, "y")
    _dense(w, "w")
    _dense(conv_state, "conv_state")
    _require(w.dtype == torch.float32 and conv_state.dtype == torch.float32, "w, conv_state: float32")
    _require(bias is None or bias.dtype == torch.float32, "bias: float32")
    _require(y.dtype == x.dtype, "y dtype must match x")
    _check(_conv(_ptr(x), x.stride(0), _code(x.dtype), _ptr(w), _ptr(bias), _ptr(conv_state),
                 _ptr(has_initial_state), _ptr(cu_seqlens), _ptr(chunks), chunks.shape[0], nseq,
                 N, C, int(bool(write_state)), _ptr(y), _stream(stream)), "gdn_causal_conv_fwd")
    return y


def gdn_conv_postconv_fwd(x: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor],
                          conv_state: torch.Tensor, has_initial_state: Optional[torch.Tensor],
                          cu_seqlens: torch.Tensor, chunks: Optional[torch.Tensor], write_state: bool,
                          Hk: int, Hv: int, eps: float = 1e-6, q: Optional[torch.Tensor] = None,
                          k: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None,
                          stream=None):
    """Conv and post-conv in one launch (C ABI gdn_conv_postconv_fwd);
    returns (q, k, v) in x's dtype, bitwise equal to gdn_causal_conv_fwd
    followed by gdn_postconv_l2.  chunks=None (up to 64 sequences): the
    launch derives the 64-token chunks from cu_seqlens itself."""
    N, C = x.shape
    _require(x.stride(1) == 1, "x rows must be contiguous")
    _require(C == (2 * Hk + Hv) * 128, "C must be (2 Hk + Hv) * 128")
    nseq = cu_seqlens.numel() - 1
    if q is None:
        q = torch.empty(N, Hk, 128, dtype=x.dtype, device=x.device)
    if k is None:
        k = torch.empty(N, Hk, 128, dtype=x.dtype, device=x.device)
    if v is None:
        v = torch.empty(N, Hv, 128, dtype=x.dtype, device=x.device)
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (w, "w"), (conv_state, "conv_state")):
        _dense(t, nm)
    _require(w.dtype == torch.float32 and conv_state.dtype == torch.float32, "w, conv_state: float32")
    _require(bias is None or bias.dtype == torch.float32, "bias: float32")
    _require(q.dtype == k.dtype == v.dtype == x.dtype, "q, k, v dtype must match x")
    _check(_conv_post(_ptr(x), x.stride(0), _code(x.dtype), _ptr(w), _ptr(bias), _ptr(conv_state),
                      _ptr(has_initial_state), _ptr(cu_seqlens), _ptr(chunks), 0 if chunks is None else chunks.shape[0], nseq, N,
                      Hk, Hv, 128, 128, float(eps), int(bool(write_state)), _ptr(q), _ptr(k), _ptr(v),
                      _stream(stream)), "gdn_conv_postconv_fwd")
    return q, k, v


# ---------------------------------------------------------------- post-conv

def gdn_postconv_l2(y: torch.Tensor, Hk: int, Hv: int, eps: float = 1e-6,
                    out_dtype=None, q: Optional[torch.Tensor] = None,
                    k: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None,
                    dk: int = 128, dv: int = 128, stream=None):
    N = y.shape[0]
    _require(y.stride(1) == 1, "y rows must be contiguous")
    out_dtype = y.dtype if out_dtype is None else out_dtype
    dev = y.device
    if q is None:
        q = torch.empty(N, Hk, dk, dtype=out_dtype, device=dev)
    if k is None:
        k = torch.empty(N, Hk, dk, dtype=out_dtype, device=dev)
    if v is None:
        v = torch.empty(N, Hv, dv, dtype=out_dtype, device=dev)
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _dense(t, nm)
        _require(t.dtype == out_dtype, f"{nm} dtype")
    _check(_postconv(_ptr(y), y.stride(0), _code(y.dtype), N, Hk, Hv, dk, dv, float(eps),
                     _ptr(q), _ptr(k), _ptr(v), _code(out_dtype), _stream(stream)),
           "gdn_postconv_l2")
    return q, k, v


# ---------------------------------------------------------------- recurrence

def _recurrence_args(q, k, v, g, beta, cu_seqlens, state, o):
    N, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (g, "g"), (beta, "beta"), (state, "state")):
        _dense(t, nm)
    _require(k.shape == q.shape and v.shape[0] == N, "q, k, v shapes")
    _require(g.dtype == torch.float32 and beta.dtype == torch.float32 and state.dtype == torch.float32,
             "g, beta, state: float32")
    _require(q.dtype == k.dtype == v.dtype, "q, k, v dtypes must match")
    if o is None:
        o = torch.empty(N, Hv, dv, dtype=q.dtype, device=q.device)
    _dense(o, "o")
    nseq = cu_seqlens.numel() - 1
    return N, Hk, Hv, dk, dv, nseq, o


def gdn_delta_rule_prefill(q, k, v, g, beta, cu_seqlens, state, has_initial_state=None,
                           o: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    N, Hk, Hv, dk, dv, nseq, o = _recurrence_args(q, k, v, g, beta, cu_seqlens, state, o)
    _check(_prefill(_ptr(q), _ptr(k), _ptr(v), _code(q.dtype), _ptr(g), _ptr(beta),
                    _ptr(cu_seqlens), nseq, N, Hk, Hv, dk, dv, _ptr(state),
                    _ptr(has_initial_state), _ptr(o), _stream(stream)), "gdn_delta_rule_prefill")
    return o


def gdn_prefill_segmented_workspace(nseq: int, Hv: int, nseg: int) -> int:
    """Workspace bytes gdn_delta_rule_prefill_segmented needs (0 for nseg <= 1)."""
    return int(_seg_ws(nseq, Hv, nseg))


def gdn_delta_rule_prefill_segmented(q, k, v, g, beta, cu_seqlens, state, nseg: int,
                                     has_initial_state=None, o: Optional[torch.Tensor] = None,
                                     workspace: Optional[torch.Tensor] = None,
                                     stream=None) -> torch.Tensor:
    """Prefill with every sequence split into nseg segments (C ABI
    gdn_delta_rule_prefill_segmented).  workspace: a device byte tensor of at
    least gdn_prefill_segmented_workspace(nseq, Hv, nseg) bytes (allocated
    here when not given)."""
    N, Hk, Hv, dk, dv, nseq, o = _recurrence_args(q, k, v, g, beta, cu_seqlens, state, o)
    need = gdn_prefill_segmented_workspace(nseq, Hv, nseg)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_prefill_seg(_ptr(q), _ptr(k), _ptr(v), _code(q.dtype), _ptr(g), _ptr(beta),
                        _ptr(cu_seqlens), nseq, N, Hk, Hv, dk, dv, _ptr(state),
                        _ptr(has_initial_state), _ptr(o), nseg, _ptr(workspace), nbytes,
                        _stream(stream)), "gdn_delta_rule_prefill_segmented")
    return o


def gdn_delta_rule_prefill_segmented_noalloc(q, k, v, g, beta, cu_seqlens, state, nseg: int,
                                             has_initial_state=None, o: Optional[torch.Tensor] = None,
                                             stream=None) -> torch.Tensor:
    """The segmented prefill with the library's own device scratch instead
    of a workspace (C ABI gdn_delta_rule_prefill_segmented_noalloc).  The C
    call allocates nothing; pass o to keep this wrapper from allocating it."""
    N, Hk, Hv, dk, dv, nseq, o = _recurrence_args(q, k, v, g, beta, cu_seqlens, state, o)
    _check(_prefill_seg_na(_ptr(q), _ptr(k), _ptr(v), _code(q.dtype), _ptr(g), _ptr(beta),
                           _ptr(cu_seqlens), nseq, N, Hk, Hv, dk, dv, _ptr(state),
                           _ptr(has_initial_state), _ptr(o), nseg, _stream(stream)),
           "gdn_delta_rule_prefill_segmented_noalloc")
    return o


def gdn_delta_rule_step(q, k, v, g, beta, cu_seqlens, state, has_initial_state=None,
                        o: Optional[torch.Tensor] = None, commit_state: bool = True,
                        stream=None) -> torch.Tensor:
    N, Hk, Hv, dk, dv, nseq, o = _recurrence_args(q, k, v, g, beta, cu_seqlens, state, o)
    _check(_step(_ptr(q), _ptr(k), _ptr(v), _code(q.dtype), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
                 nseq, N, Hk, Hv, dk, dv, _ptr(state), _ptr(has_initial_state), _ptr(o),
                 int(bool(commit_state)), _stream(stream)), "gdn_delta_rule_step")
    return o


def gdn_decode_fused(x, w, bias, conv_state, cu_seqlens, g, beta, state, Hk: int, Hv: int,
                     eps: float = 1e-6, has_initial_state=None, o: Optional[torch.Tensor] = None,
                     write_conv_state: bool = True, commit_state: bool = True,
                     k_out: Optional[torch.Tensor] = None, v_out: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """conv + post-conv + step in one launch (bitwise equal to the three calls).
    k_out [N, Hk, 128] / v_out [N, Hv, 128] (optional, activation dtype)
    receive the normalised k and the v for a later gdn_commit."""
    N, C = x.shape
    _require(x.stride(1) == 1, "x rows must be contiguous")
    for t, nm in ((w, "w"), (conv_state, "conv_state"), (g, "g"), (beta, "beta"), (state, "state")):
        _dense(t, nm)
    _require(w.dtype == torch.float32 and conv_state.dtype == torch.float32 and g.dtype == torch.float32
             and beta.dtype == torch.float32 and state.dtype == torch.float32,
             "w, conv_state, g, beta, state: float32")
    _require(bias is None or bias.dtype == torch.float32, "bias: float32")
    if o is None:
        o = torch.empty(N, Hv, 128, dtype=x.dtype, device=x.device)
    _dense(o, "o")
    for t, nm, H in ((k_out, "k_out", Hk), (v_out, "v_out", Hv)):
        if t is not None:
            _dense(t, nm)
            _require(t.dtype == x.dtype and t.numel() == N * H * 128, f"{nm}: [N, {H}, 128] of x's dtype")
    nseq = cu_seqlens.numel() - 1
    _check(_decode_fused(_ptr(x), x.stride(0), _code(x.dtype), _ptr(w), _ptr(bias), _ptr(conv_state),
                         _ptr(cu_seqlens), nseq, N, Hk, Hv, 128, 128, float(eps), _ptr(g), _ptr(beta),
                         _ptr(state), _ptr(has_initial_state), _ptr(o), _ptr(k_out), _ptr(v_out),
                         int(bool(write_conv_state)),
                         int(bool(commit_state)), _stream(stream)), "gdn_decode_fused")
    return o


# ---------------------------------------------------------------- gates

def gdn_gates(ba: torch.Tensor, A_log: torch.Tensor, dt_bias: torch.Tensor,
              g: Optional[torch.Tensor] = None, beta: Optional[torch.Tensor] = None, stream=None):
    """beta = sigmoid(b), g = -exp(A_log) * softplus(a + dt_bias) from the
    packed ba [N, Hv, 2] = (b, a) (float32 or bf16); returns float32 (g, beta)
    of shape [N, Hv]."""
    _dense(ba, "ba")
    _require(ba.dim() == 3 and ba.shape[2] == 2, "ba: [N, Hv, 2]")
    N, Hv, _ = ba.shape
    for t, nm in ((A_log, "A_log"), (dt_bias, "dt_bias")):
        _dense(t, nm)
        _require(t.dtype == torch.float32 and t.numel() == Hv, f"{nm}: float32 [Hv]")
    if g is None:
        g = torch.empty(N, Hv, dtype=torch.float32, device=ba.device)
    if beta is None:
        beta = torch.empty(N, Hv, dtype=torch.float32, device=ba.device)
    for t, nm in ((g, "g"), (beta, "beta")):
        _dense(t, nm)
        _require(t.dtype == torch.float32 and t.numel() == N * Hv, f"{nm}: float32 [N, Hv]")
    _check(_gates(_ptr(ba), _code(ba.dtype), _ptr(A_log), _ptr(dt_bias), N, Hv, _ptr(g), _ptr(beta),
                  _stream(stream)), "gdn_gates")
    return g, beta


# ---------------------------------------------------------------- output norm

def gdn_out_norm(o: torch.Tensor, z: torch.Tensor, w: Optional[torch.Tensor] = None,
                 eps: float = 1e-6, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y = o / sqrt(mean(o^2) + eps) * w * SiLU(z) per token and v-head;
    o, z [N, Hv, 128]; w float32 [128] or None; y may be o (in place)."""
    _dense(o, "o")
    _dense(z, "z")
    _require(o.dim() == 3 and o.shape == z.shape and o.dtype == z.dtype, "o, z: [N, Hv, 128] of one dtype")
    if w is not None:
        _dense(w, "w")
        _require(w.dtype == torch.float32 and w.numel() == o.shape[2], "w: float32 [dv]")
    if y is None:
        y = torch.empty_like(o)
    _dense(y, "y")
    _require(y.shape == o.shape and y.dtype == o.dtype, "y: like o")
    N, Hv, dv = o.shape
    _check(_out_norm(_ptr(o), _ptr(z), _code(o.dtype), _ptr(w), N, Hv, dv, float(eps), _ptr(y),
                     _stream(stream)), "gdn_out_norm")
    return y


# ---------------------------------------------------------------- commit

def gdn_layer_table(layers: List[dict], device) -> torch.Tensor:
    """Pack per-layer tensors {x, conv_state, state, k, v, g, beta} into a
    device array of gdn_layer_io (kept alive by the caller)."""
    arr = (gdn_layer_io * len(layers))()
    for i, L in enumerate(layers):
        x = L["x"]
        _require(x.stride(1) == 1, "x rows must be contiguous")
        arr[i] = gdn_layer_io(x.data_ptr(), x.stride(0), L["conv_state"].data_ptr(),
                              L["state"].data_ptr(), L["k"].data_ptr(), L["v"].data_ptr(),
                              L["g"].data_ptr(), L["beta"].data_ptr())
    raw = torch.frombuffer(bytearray(bytes(arr)), dtype=torch.uint8)
    return raw.to(device)


def gdn_commit(layer_table: torch.Tensor, L: int, cu_seqlens: torch.Tensor, n_keep: torch.Tensor,
               has_initial_state: Optional[torch.Tensor], C: int, Hk: int, Hv: int, act_dtype,
               dk: int = 128, dv: int = 128, stream=None):
    _require(layer_table.numel() >= L * ctypes.sizeof(gdn_layer_io), "layer table too small")
    nseq = cu_seqlens.numel() - 1
    _check(_commit(_ptr(layer_table), L, _ptr(cu_seqlens), _ptr(n_keep), _ptr(has_initial_state),
                   nseq, C, Hk, Hv, dk, dv, _code(act_dtype), _stream(stream)), "gdn_commit")
