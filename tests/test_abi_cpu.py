"""CPU-side checks of the C ABI: the library loads and exports every entry
point include/gdn.h declares; the host chunk builder is bit-exact against the
oracle; argument validation returns the documented status codes before any
launch (no GPU is touched: every call here fails validation)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch  # noqa: F401  (loaded before libgdn.so so both use torch's HIP runtime)

from oracle import gdn_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "linear_attention_layers_amd", "libgdn.so")
HEADER = os.path.join(ROOT, "include", "gdn.h")

if not os.path.exists(LIB):
    pytest.skip("libgdn.so not built (run __graft_entry__.build())", allow_module_level=True)

lib = ctypes.CDLL(LIB)
vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float

OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, LAUNCH, CAPACITY = range(8)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_hot_path_calls():
    names = declared_functions()
    for required in ("gdn_causal_conv_fwd", "gdn_postconv_l2", "gdn_delta_rule_prefill",
                     "gdn_delta_rule_step", "gdn_commit", "gdn_make_chunks"):
        assert required in names


def test_every_declared_symbol_is_exported():
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_names_match_the_abi():
    # the Python binding is not imported here (it needs torch's HIP stream at
    # call time, not at import); its list of names must equal the header's
    src = open(os.path.join(ROOT, "linear_attention_layers_amd", "gdn.py")).read()
    exported = re.search(r"EXPORTED = \[(.*?)\]", src, re.S).group(1)
    assert sorted(re.findall(r'"(gdn_[a-z0-9_]+)"', exported)) == declared_functions()


def test_abi_version_and_status_strings():
    lib.gdn_abi_version.restype = i32
    assert lib.gdn_abi_version() == 1
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_status_string.argtypes = [i32]
    assert lib.gdn_status_string(0) == b"ok"
    assert lib.gdn_status_string(ALIAS) == b"overlapping buffers"


def _make_chunks(cu, chunk_len=64, cap=None):
    cu = np.asarray(cu, dtype=np.int32)
    nseq = len(cu) - 1
    lib.gdn_chunk_capacity.restype = i32
    lib.gdn_chunk_capacity.argtypes = [i32, i32, i32]
    bound = lib.gdn_chunk_capacity(int(cu[-1]), nseq, chunk_len)
    cap = bound if cap is None else cap
    out = np.zeros((max(cap, 1), 4), dtype=np.int32)
    lib.gdn_make_chunks.restype = i32
    lib.gdn_make_chunks.argtypes = [vp, i32, i32, vp, i32]
    n = lib.gdn_make_chunks(cu.ctypes.data, nseq, chunk_len, out.ctypes.data, cap)
    return n, out, bound


@pytest.mark.parametrize("seed", range(25))
def test_host_make_chunks_bit_exact_and_capacity_is_a_bound(seed):
    r = np.random.default_rng(seed)
    lengths = r.integers(0, 400, int(r.integers(1, 40)))
    cu = np.concatenate([[0], np.cumsum(lengths)])
    M = int(r.choice([3, 16, 63, 64]))
    n, out, bound = _make_chunks(cu, M)
    ref = O.make_chunks(cu, M)
    assert n == len(ref) <= bound
    assert np.array_equal(out[:n], ref)


def test_host_make_chunks_errors():
    n, _, _ = _make_chunks([0, 200], 64, cap=3)
    assert n == -CAPACITY
    n, _, _ = _make_chunks([0, 5, 3], 64)
    assert n == -SHAPE
    n, _, _ = _make_chunks([1, 5], 64)
    assert n == -SHAPE
    lib.gdn_make_chunks.argtypes = [vp, i32, i32, vp, i32]
    assert lib.gdn_make_chunks(None, 1, 64, None, 4) == -NULL


@pytest.mark.parametrize("chunk_len", [-1, 0, 1, 2, 65, 100, 128])
def test_chunk_len_outside_3_to_64_is_rejected(chunk_len):
    # The conv kernels cover at most 64 tokens per descriptor and a
    # non-first chunk reads its 3-row halo from its own sequence: every
    # builder refuses other lengths before touching memory or the GPU.
    n, _, bound = _make_chunks([0, 200, 201], chunk_len)
    assert n == -SHAPE and bound == 0
    dev = lib.gdn_make_chunks_device
    dev.restype = i32
    dev.argtypes = [vp, i32, i32, vp, i32, vp]
    assert dev(FAKE, 2, chunk_len, FAKE + (1 << 24), 8, None) == -SHAPE
    assert dev(FAKE, 2, chunk_len, FAKE + (1 << 24), 0, None) == -SHAPE


@pytest.mark.parametrize("chunk_len", [3, 4, 64])
def test_chunk_len_bounds_are_accepted(chunk_len):
    n, out, bound = _make_chunks([0, 200, 201, 201], chunk_len)
    ref = O.make_chunks([0, 200, 201, 201], chunk_len)
    assert n == len(ref) <= bound and np.array_equal(out[:n], ref)


FAKE = 0x10000000          # 16-byte aligned dummy address; never dereferenced


def _postconv(y, ys, N, Hk, Hv, dk, dv, eps, q, k, v, din=1, dout=1):
    fn = lib.gdn_postconv_l2
    fn.restype = i32
    fn.argtypes = [vp, i64, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp, i32, vp]
    return fn(y, ys, din, N, Hk, Hv, dk, dv, eps, q, k, v, dout, None)


def test_postconv_validation():
    C = 2 * 2 * 128 + 4 * 128
    base = dict(y=FAKE, ys=C, N=4, Hk=2, Hv=4, dk=128, dv=128, eps=1e-6,
                q=FAKE + (1 << 24), k=FAKE + (2 << 24), v=FAKE + (3 << 24))
    assert _postconv(**dict(base, dk=64)) == SHAPE
    assert _postconv(**dict(base, Hv=3)) == SHAPE
    assert _postconv(**dict(base, eps=0.0)) == SHAPE
    assert _postconv(**dict(base, ys=C - 8)) == SHAPE
    assert _postconv(**dict(base, y=None)) == NULL
    assert _postconv(**dict(base, q=FAKE + 8)) == ALIGN
    assert _postconv(**dict(base, q=FAKE + 64)) == ALIAS          # q inside y
    assert _postconv(**dict(base), din=7) == DTYPE
    assert _postconv(**dict(base, N=0)) == OK                      # empty: no launch


def test_conv_validation():
    fn = lib.gdn_causal_conv_fwd
    fn.restype = i32
    fn.argtypes = [vp, i64, i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp]
    C = 1024
    args = [FAKE, C, 1, FAKE + (1 << 24), None, FAKE + (2 << 24), None, FAKE + (3 << 24),
            FAKE + (4 << 24), 4, 2, 100, C, 1, FAKE + (5 << 24), None]

    def call(**kw):
        a = list(args)
        idx = {"x": 0, "xs": 1, "act": 2, "C": 12, "y": 14, "w": 3, "N": 11, "ws": 13, "cs": 5}
        for k_, v_ in kw.items():
            a[idx[k_]] = v_
        return fn(*a)

    assert call(C=1020) == SHAPE
    assert call(xs=C - 8) == SHAPE
    assert call(act=5) == DTYPE
    assert call(w=None) == NULL
    assert call(x=FAKE + 2) == ALIGN
    assert call(y=FAKE + 1024) == ALIAS
    # no tokens and no final rows to write: nothing to do, no launch
    assert call(N=0, ws=0) == OK
    # no tokens but final rows to write (empty sequences are cleared): the
    # state buffer is still required
    assert call(N=0, cs=None) == NULL


def test_recurrence_validation():
    fn = lib.gdn_delta_rule_prefill
    fn.restype = i32
    fn.argtypes = [vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp]
    base = [FAKE, FAKE + (1 << 24), FAKE + (2 << 24), 1, FAKE + (3 << 24), FAKE + (4 << 24),
            FAKE + (5 << 24), 2, 100, 2, 4, 128, 128, FAKE + (6 << 24), None, FAKE + (7 << 24), None]

    def call(**kw):
        a = list(base)
        idx = {"q": 0, "act": 3, "cu": 6, "Hk": 9, "Hv": 10, "dk": 11, "state": 13, "o": 15}
        for k_, v_ in kw.items():
            a[idx[k_]] = v_
        return fn(*a)

    assert call(Hv=3) == SHAPE
    assert call(dk=64) == SHAPE
    assert call(act=2) == DTYPE
    assert call(cu=None) == NULL
    assert call(o=FAKE + 4) == ALIGN
    assert call(o=FAKE + 256) == ALIAS      # o inside q
    step = lib.gdn_delta_rule_step
    step.restype = i32
    step.argtypes = fn.argtypes[:-1] + [i32, vp]
    a = list(base)
    a[9] = 3
    assert step(*(a[:-1] + [1, None])) == SHAPE


def test_prefill_segmented_validation():
    wsz = lib.gdn_prefill_segmented_workspace
    wsz.restype = ctypes.c_size_t
    wsz.argtypes = [i32, i32, i32]
    assert wsz(2, 4, 3) == 3 * 2 * 3 * 4 * 128 * 128 * 4
    assert wsz(2, 4, 1) == 0 and wsz(0, 4, 3) == 0
    fn = lib.gdn_delta_rule_prefill_segmented
    fn.restype = i32
    fn.argtypes = [vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, i32, vp,
                   ctypes.c_size_t, vp]
    need = wsz(2, 4, 3)
    base = [FAKE, FAKE + (1 << 24), FAKE + (2 << 24), 1, FAKE + (3 << 24), FAKE + (4 << 24),
            FAKE + (5 << 24), 2, 100, 2, 4, 128, 128, FAKE + (6 << 24), None, FAKE + (7 << 24),
            3, FAKE + (1 << 30), need, None]

    def call(**kw):
        a = list(base)
        idx = {"act": 3, "Hv": 10, "nseg": 16, "ws": 17, "wsb": 18}
        for k_, v_ in kw.items():
            a[idx[k_]] = v_
        return fn(*a)

    assert call(Hv=3) == SHAPE
    assert call(nseg=0) == SHAPE and call(nseg=65) == SHAPE
    assert call(act=0) == DTYPE                      # float32 activations: unsegmented only
    assert call(ws=None) == NULL
    assert call(ws=FAKE + (1 << 30) + 4) == ALIGN
    assert call(wsb=need - 1) == CAPACITY
    assert call(ws=FAKE + (2 << 24)) == ALIAS        # workspace over v
    assert call(ws=FAKE + (6 << 24) - 4096) == ALIAS   # workspace running into state


def test_conv_postconv_validation():
    fn = lib.gdn_conv_postconv_fwd
    fn.restype = i32
    fn.argtypes = [vp, i64, i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32,
                   vp, vp, vp, vp]
    C = (2 * 2 + 4) * 128
    base = [FAKE, C, 1, FAKE + (1 << 24), None, FAKE + (2 << 24), None, FAKE + (3 << 24), FAKE + (4 << 24),
            3, 2, 100, 2, 4, 128, 128, 1e-6, 1, FAKE + (5 << 24), FAKE + (6 << 24), FAKE + (7 << 24), None]

    def call(**kw):
        a = list(base)
        idx = {"xs": 1, "act": 2, "nseq": 10, "Hv": 13, "dk": 14, "eps": 16, "q": 18, "v": 20, "chunks": 8}
        for k_, v_ in kw.items():
            a[idx[k_]] = v_
        return fn(*a)

    assert call(Hv=3) == SHAPE
    assert call(dk=64) == SHAPE
    assert call(xs=C - 8) == SHAPE
    assert call(eps=0.0) == SHAPE
    assert call(act=5) == DTYPE
    assert call(chunks=None, nseq=65) == SHAPE        # chunks derived in-kernel only up to 64 sequences
    assert call(q=None) == NULL
    assert call(q=FAKE + (5 << 24) + 8) == ALIGN
    assert call(q=FAKE + 1024) == ALIAS                # q inside x
    assert call(v=FAKE + (6 << 24) + 4096) == ALIAS    # v inside k


def test_commit_validation():
    fn = lib.gdn_commit
    fn.restype = i32
    fn.argtypes = [vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp]
    assert fn(FAKE, 2, FAKE, FAKE, None, 4, 1000, 2, 4, 128, 128, 1, None) == SHAPE
    assert fn(None, 2, FAKE, FAKE, None, 4, 1024, 2, 4, 128, 128, 1, None) == NULL
    assert fn(FAKE, 0, FAKE, FAKE, None, 4, 1024, 2, 4, 128, 128, 1, None) == OK


def test_decode_fused_validation():
    fn = lib.gdn_decode_fused
    fn.restype = i32
    fn.argtypes = [vp, i64, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, vp, vp, vp, vp,
                   vp, vp, vp, i32, i32, vp]
    Hk, Hv = 2, 4
    C = 2 * Hk * 128 + Hv * 128
    base = dict(x=FAKE, xs=C, act=1, w=FAKE + (1 << 24), bias=None, cs=FAKE + (2 << 24),
                cu=FAKE + (3 << 24), nseq=2, N=10, Hk=Hk, Hv=Hv, dk=128, dv=128, eps=1e-6,
                g=FAKE + (4 << 24), beta=FAKE + (5 << 24), st=FAKE + (6 << 24), hi=None,
                o=FAKE + (8 << 24), ko=None, vo=None, wcs=1, commit=1)

    def call(**kw):
        a = dict(base, **kw)
        return fn(a["x"], a["xs"], a["act"], a["w"], a["bias"], a["cs"], a["cu"], a["nseq"], a["N"],
                  a["Hk"], a["Hv"], a["dk"], a["dv"], a["eps"], a["g"], a["beta"], a["st"], a["hi"],
                  a["o"], a["ko"], a["vo"], a["wcs"], a["commit"], None)

    assert call(Hv=8) == SHAPE             # only Hv = Hk or 2 Hk
    assert call(Hv=3) == SHAPE
    assert call(dk=64) == SHAPE
    assert call(eps=0.0) == SHAPE
    assert call(xs=C - 8) == SHAPE
    assert call(act=9) == DTYPE
    assert call(x=None) == NULL
    assert call(st=None) == NULL
    assert call(o=FAKE + (8 << 24) + 4) == ALIGN
    assert call(o=FAKE + 64) == ALIAS      # o inside x
    assert call(cs=FAKE + (6 << 24) + 64) == ALIAS   # conv_state inside state
    assert call(ko=FAKE + (9 << 24) + 2) == ALIGN
    assert call(ko=FAKE + (8 << 24) + 256) == ALIAS   # k_out inside o
    assert call(vo=FAKE + (9 << 24), ko=FAKE + (9 << 24) + 4096) == ALIAS   # k_out inside v_out
    assert call(vo=FAKE + 128) == ALIAS     # v_out inside x
    assert call(N=0, wcs=0, commit=0) == OK   # no tokens, no final state: no launch
    assert call(N=0, x=None, o=None, g=None, beta=None, st=None) == NULL   # zero states still need state
    assert call(nseq=0) == OK


def test_out_norm_validation():
    fn = lib.gdn_out_norm
    fn.restype = i32
    fn.argtypes = [vp, vp, i32, vp, i32, i32, i32, f32, vp, vp]
    base = dict(o=FAKE, z=FAKE + (1 << 24), act=1, w=None, N=10, Hv=4, dv=128, eps=1e-6,
                y=FAKE + (2 << 24))

    def call(**kw):
        a = dict(base, **kw)
        return fn(a["o"], a["z"], a["act"], a["w"], a["N"], a["Hv"], a["dv"], a["eps"], a["y"], None)

    assert call(dv=64) == SHAPE
    assert call(Hv=0) == SHAPE
    assert call(N=-1) == SHAPE
    assert call(eps=0.0) == SHAPE
    assert call(eps=float("nan")) == SHAPE
    assert call(act=7) == DTYPE
    assert call(o=None) == NULL
    assert call(y=None) == NULL
    assert call(z=FAKE + (1 << 24) + 8) == ALIGN
    assert call(w=FAKE + (3 << 24) + 4) == ALIGN
    assert call(y=FAKE + 256) == ALIAS                 # partly over o
    assert call(y=FAKE + (1 << 24)) == ALIAS           # over z
    assert call(w=FAKE + (2 << 24) + 512) == ALIAS     # w inside y
    assert call(N=0) == OK                             # empty: no launch


def test_gates_validation():
    fn = lib.gdn_gates
    fn.restype = i32
    fn.argtypes = [vp, i32, vp, vp, i32, i32, vp, vp, vp]
    base = dict(ba=FAKE, act=0, A=FAKE + (1 << 24), dt=FAKE + (2 << 24), N=10, Hv=4,
                g=FAKE + (3 << 24), beta=FAKE + (4 << 24))

    def call(**kw):
        a = dict(base, **kw)
        return fn(a["ba"], a["act"], a["A"], a["dt"], a["N"], a["Hv"], a["g"], a["beta"], None)

    assert call(Hv=0) == SHAPE
    assert call(N=-3) == SHAPE
    assert call(act=5) == DTYPE
    assert call(ba=None) == NULL
    assert call(beta=None) == NULL
    assert call(ba=FAKE + 4) == ALIGN                    # f32 pairs need 8 bytes
    assert call(g=FAKE + (3 << 24) + 2) == ALIGN
    assert call(beta=FAKE + (3 << 24) + 16) == ALIAS     # overlaps g
    assert call(g=FAKE + 40) == ALIAS                    # inside ba
    assert call(N=0) == OK


def _derived_chunks(cu, nslots):
    """Host restatement of the fused conv launch's slot map: slot j belongs
    to the last sequence s with floor(cu[s] / 64) + s <= j, as its chunk
    j - f(s) when that chunk exists."""
    nseq = len(cu) - 1
    f = [cu[s] // 64 + s for s in range(nseq)]
    out = []
    for j in range(nslots):
        s = max(t for t in range(nseq) if f[t] <= j)
        c = j - f[s]
        nc = -(-(cu[s + 1] - cu[s]) // 64)
        if c < nc:
            b = cu[s] + 64 * c
            out.append((s, b, min(b + 64, cu[s + 1]), (1 if c == 0 else 0) | (2 if c == nc - 1 else 0)))
    return out


@pytest.mark.parametrize("seed", range(6))
def test_derived_chunk_slots_give_the_descriptor_list(seed):
    rng = np.random.default_rng(seed)
    nseq = int(rng.integers(1, 65))
    lengths = [int(v) for v in rng.integers(0, 300, nseq)]
    lengths[int(rng.integers(0, nseq))] = int(rng.integers(1, 1000))   # at least one token
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + L)
    got = _derived_chunks(cu, cu[-1] // 64 + nseq)
    ref = [tuple(int(v) for v in row) for row in O.make_chunks(cu, 64)]
    assert got == ref


@pytest.mark.parametrize("lengths", [[1] * 64, [64] * 64, [63] * 64, [65, 63, 1, 127, 0, 129], [0, 0, 5], [4096]])
def test_derived_chunk_slots_edge_batches(lengths):
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + L)
    got = _derived_chunks(cu, cu[-1] // 64 + len(lengths))
    ref = [tuple(int(v) for v in row) for row in O.make_chunks(cu, 64)]
    assert got == ref
