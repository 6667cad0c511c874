"""Slow, plain CPU oracle for the Gated DeltaNet (GDN) layer hot path.

TEST INFRASTRUCTURE ONLY.  This module states, in float64 numpy, what each
stage of the GDN hot path computes.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import it; the HIP library never does, and
nothing here shares code, headers, tables or helpers with it.

Sources (page title, section):
  [vllm155]  "perf(gdn): optimize post-conv and causal-conv kernels" (vllm.cpp
             pull request 155): review sections "Blocker", "What I verified",
             "The one thing I changed in your tests", "New issue #305", and the
             PR description sections "What changed" and "Speed claims".
  [strata]   "Strata pull request 3226" (GDN speculative-verify, decode and
             commit kernels): sections "Problem and result", "Approach",
             "Summary" items 1-4 and "Root Cause & RED / GREEN Verification".
  [GDN]      the gated delta rule itself, S_t = a_t S_{t-1}(I - b_t k_t k_t^T)
             + b_t v_t k_t^T with read-out o_t = S_t q_t (Yang, Kautz and
             Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with Delta
             Rule", 2024); the pages name the kernels that run it but print no
             equation.

Where the pages are silent the plainest reading is taken; each reading is
listed next to the function that depends on it.

Parity pins: every function below is pinned by tests/test_oracle_pins.py
(closed forms, brute force, hand-derived values, library special cases).  No
function here is "parity unpinned"; the only unpinned aspect is fidelity to a
trained model's conventions (tap order, eps, gate parametrisation), for which
the pages hold no weights.
"""
from __future__ import annotations

import numpy as np

CHUNK_FIRST = 1
CHUNK_LAST = 2
CONV_WIDTH = 4


# --------------------------------------------------------------------------
# rounding helpers (storage points)
# --------------------------------------------------------------------------

def round_to_bf16(x):
    """Round float64 values to the nearest bfloat16 (ties to even), returned as
    float64.  bfloat16 keeps 8 significant bits and the float32 exponent
    range; values are rounded directly from float64 (no float32 step), so no
    double rounding.  Subnormal bfloat16 results are not needed by any
    workload here and are flushed through the same formula (values below
    2**-126 keep 8 bits relative to 2**-126)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                 # bf16 min normal 2**-126 = 0.5*2**-125
    r = np.rint(np.ldexp(x, 8 - e))         # 8 significant bits, ties to even
    out = np.ldexp(r, e - 8)
    out = np.where(np.abs(out) > 3.3895313892515355e38, np.copysign(np.inf, x), out)
    return np.where(np.isfinite(x), out, x)


def round_to(x, dtype: str):
    """Round float64 values to the storage dtype ("f32" or "bf16"), as float64."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return round_to_bf16(x)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# a1: exact token chunks
# --------------------------------------------------------------------------

def make_chunks(cu_seqlens, chunk_len: int = 64) -> np.ndarray:
    """Exact conv chunk descriptors [vllm155, "New issue #305"; PR description
    "Before starting" names the exact causal-conv chunk dispatch].

    Every sequence s (tokens cu[s]..cu[s+1]-1) is cut into consecutive pieces
    of chunk_len tokens, the last one possibly shorter.  Each descriptor is
    (seq, begin, end, flags) with flags bit 0 = first chunk of its sequence
    (the one whose window reaches back into the initial conv_state) and bit 1
    = last chunk (the one holding the sequence's final tokens).  Order: by
    sequence, then by position.  Empty sequences emit nothing.
    """
    cu = [int(c) for c in cu_seqlens]
    out = []
    for s in range(len(cu) - 1):
        length = cu[s + 1] - cu[s]
        if length <= 0:
            continue
        nchunks = -(-length // chunk_len)
        for j in range(nchunks):
            begin = cu[s] + j * chunk_len
            end = min(begin + chunk_len, cu[s + 1])
            flags = (CHUNK_FIRST if j == 0 else 0) | (CHUNK_LAST if j == nchunks - 1 else 0)
            out.append((s, begin, end, flags))
    return np.array(out, dtype=np.int32).reshape(-1, 4)


# --------------------------------------------------------------------------
# a2: width-4 depthwise causal conv with per-sequence conv_state
# --------------------------------------------------------------------------

def causal_conv(x, w, bias, conv_state, has_init, cu_seqlens, write_state=True):
    """Width-4 depthwise causal conv1d over the packed q|k|v channels
    [vllm155, "Blocker" (c = 1024 channels, k = 4 taps) and "New issue #305"
    (the initial conv_state is read by the first chunk, the final one is
    written from the last tokens)].

    Readings (the pages are silent): tap w[c, 3] multiplies the current token
    and w[c, 3 - d] the token d steps back (the causal conv1d convention);
    conv_state[s] holds the 3 most recent inputs of sequence s, row 0 the
    oldest, in float32 storage; has_init[s] == 0 means the 3 rows before the
    sequence are zero and the stored rows are never read.

    For sequence s with L tokens, the extended input is
        ext[0:3]   = conv_state[s]        (or zeros)
        ext[3:3+L] = x[cu[s]:cu[s+1]]
    and y[cu[s]+t, c] = bias[c] + sum_j w[c, j] * ext[t + j, c].
    The returned state is ext[L:L+3] (the last 3 rows) when write_state,
    otherwise the input state unchanged.

    Returns (y float64 [N, C], new_state float64 [nseq, 3, C]).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    N, C = x.shape
    b = np.zeros(C) if bias is None else np.asarray(bias, dtype=np.float64)
    st = np.array(conv_state, dtype=np.float64, copy=True)
    cu = [int(c) for c in cu_seqlens]
    nseq = len(cu) - 1
    y = np.zeros((N, C))
    for s in range(nseq):
        L = cu[s + 1] - cu[s]
        init = st[s] if has_init[s] else np.zeros((3, C))
        ext = np.concatenate([init, x[cu[s]:cu[s + 1]]], axis=0)
        for t in range(L):
            acc = b.copy()
            for j in range(CONV_WIDTH):
                acc = acc + w[:, j] * ext[t + j]
            y[cu[s] + t] = acc
        if write_state:
            st[s] = ext[L:L + 3]
    return y, st


# --------------------------------------------------------------------------
# a3: post-conv SiLU + split + per-head L2 norm
# --------------------------------------------------------------------------

def silu(y):
    """SiLU(y) = y * sigmoid(y) = y / (1 + exp(-y)), in float64."""
    y = np.asarray(y, dtype=np.float64)
    with np.errstate(over="ignore"):
        return y / (1.0 + np.exp(-y))


def split_heads(a, Hk, Hv, dk, dv):
    """Split packed channels [..., C] into q [..., Hk, dk], k [..., Hk, dk] and
    v [..., Hv, dv]; the packing is q | k | v [vllm155, "Blocker" c = 1024
    channels; the Strata geometry C = 10240 = 2*16*128 + 48*128 in
    "Benchmark Evidence"]."""
    lead = a.shape[:-1]
    q = a[..., : Hk * dk].reshape(*lead, Hk, dk)
    k = a[..., Hk * dk: 2 * Hk * dk].reshape(*lead, Hk, dk)
    v = a[..., 2 * Hk * dk: 2 * Hk * dk + Hv * dv].reshape(*lead, Hv, dv)
    return q, k, v


def postconv_l2(y, Hk, Hv, dk, dv, eps):
    """Post-conv step in float64 [vllm155, "What I verified" (the reduction
    for the per-head squared norm) and "The one thing I changed in your tests"
    (the 1/sqrtf normalisation)]: s = SiLU(y) over all channels, split q|k|v,
    and q_hat = q / sqrt(sum(q^2) + eps), k_hat likewise, per head.

    Reading: SiLU applies to all channels (v too); L2 applies to q and k only;
    the normaliser is 1/sqrt(sum + eps) with eps > 0 an argument.
    Returns (q_hat, k_hat, v) float64."""
    s = silu(y)
    q, k, v = split_heads(s, Hk, Hv, dk, dv)
    qn = q / np.sqrt(np.sum(q * q, axis=-1, keepdims=True) + eps)
    kn = k / np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + eps)
    return qn, kn, v


def tree_sum_f32(sq):
    """The documented summation order for a head's squared norm, evaluated in
    float32: a pairwise tree, neighbours first.  Level l adds adjacent blocks
    of 2**l elements: (x0+x1), then (x0+x1)+(x2+x3), and so on, each addition
    rounded to float32 (ties to even).  The last axis must be a power of two.
    The pages fix the order only as "fixed and bit-verifiable" [vllm155,
    "What I verified"]; this is the reading taken for every L2 norm here."""
    cur = np.asarray(sq, dtype=np.float32)
    n = cur.shape[-1]
    if n & (n - 1):
        raise ValueError("head size must be a power of two")
    while cur.shape[-1] > 1:
        cur = (cur[..., 0::2] + cur[..., 1::2]).astype(np.float32)
    return cur[..., 0]


def postconv_l2_f32_tree(y, Hk, Hv, dk, dv, eps):
    """The float32 output arm of the post-conv step with the documented order
    [vllm155, "The one thing I changed in your tests": a reduction order is
    only observable in a float32 output].

    s_i = float32(SiLU(y_i) in float64); squares, the neighbours-first tree,
    eps addition, sqrt and the division are each one correctly rounded
    float32 operation; q_hat_i = float32(s_i * inv).  Returns float32 arrays
    (q_hat, k_hat, v)."""
    s = silu(y).astype(np.float32)
    q, k, v = split_heads(s, Hk, Hv, dk, dv)
    e = np.float32(eps)

    def norm(a):
        sq = (a * a).astype(np.float32)
        sig = tree_sum_f32(sq)
        inv = (np.float32(1.0) / np.sqrt((sig + e).astype(np.float32))).astype(np.float32)
        return (a * inv[..., None]).astype(np.float32)

    return norm(q), norm(k), v.astype(np.float32)


# --------------------------------------------------------------------------
# a4/a5: the gated delta rule
# --------------------------------------------------------------------------

def _kv_head_map(Hk, Hv):
    """GQA map: v-head h reads k-head h // (Hv // Hk) (consecutive v-heads
    share a k-head).  Reading of "2 v-heads per k-head" for the 16/32-head
    layout; the pages' own geometry (h_k = 16, h_v = 48) has ratio 3
    [strata, "Benchmark Evidence"]."""
    if Hv % Hk:
        raise ValueError("Hv must be a multiple of Hk")
    return np.arange(Hv) // (Hv // Hk)


def delta_rule_recurrent(q, k, v, g, beta, state0, has_init, cu_seqlens, Hk, Hv):
    """Gated delta rule, token by token, in float64 [GDN; the per-token step
    of strata "Summary" item 3].

    For each sequence s and v-head h (k-head kh = h // (Hv/Hk)):
        S = state0[s, h] if has_init[s] else 0            (dv x dk)
        for each token t of s, with a = exp(g[t, h]), b = beta[t, h]:
            S = a * S (I - b k_t k_t^T) + b v_t k_t^T
            o[t, h] = S q_t          (read-out after the update)
    Returns (o [N, Hv, dv], final states [nseq, Hv, dv, dk]), float64.

    Readings: g is log a_t (float32, <= 0); the state is stored dv x dk
    (k index fastest); no output scale."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    st = np.array(state0, dtype=np.float64, copy=True)
    kmap = _kv_head_map(Hk, Hv)
    cu = [int(c) for c in cu_seqlens]
    N = q.shape[0]
    dv = v.shape[-1]
    o = np.zeros((N, Hv, dv))
    for s in range(len(cu) - 1):
        S = st[s].copy() if has_init[s] else np.zeros_like(st[s])
        for t in range(cu[s], cu[s + 1]):
            a = np.exp(g[t])[:, None, None]
            b = beta[t][:, None, None]
            kt = k[t, kmap]                        # [Hv, dk]
            qt = q[t, kmap]
            Sk = np.einsum("hvc,hc->hv", S, kt)    # S k
            S = a * (S - b * Sk[:, :, None] * kt[:, None, :]) + b * v[t][:, :, None] * kt[:, None, :]
            o[t] = np.einsum("hvc,hc->hv", S, qt)
        st[s] = S
    return o, st


def delta_rule_chunked(q, k, v, g, beta, state0, has_init, cu_seqlens, Hk, Hv,
                       chunk_len=64):
    """The same recurrence in chunked (WY) form, float64.  The pages do not
    print the chunked algorithm (the Strata page leaves its prefill kernels
    untouched, "What This Does NOT Fix"); this is the chunk-64 form derived
    from the per-token rule.  Per sequence, per v-head, per chunk of n tokens
    (local index i, entering state S0):

      1. G_i = sum_{m<=i} g_m,  gamma_i = exp(G_i)
      2. A_ij = b_i exp(G_i - G_j) (k_i . k_j) for j < i, else 0
      3. T = (I + A)^-1             (unit lower triangular)
      4. W = T diag(b gamma) K,  Ut = T diag(b) V
      5. U = Ut - W S0^T            (row i: b_i (v_i - a_i S_{i-1} k_i))
      6. O = diag(gamma) Q S0^T + (Mask_ij exp(G_i - G_j) (q_i . k_j)) U,
         Mask_ij = 1 for j <= i
      7. S = gamma_{n-1} S0 + U^T diag(exp(G_{n-1} - G)) K

    The chunks start at each sequence's first token.  Returns the same as
    delta_rule_recurrent."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    st = np.array(state0, dtype=np.float64, copy=True)
    kmap = _kv_head_map(Hk, Hv)
    cu = [int(c) for c in cu_seqlens]
    N = q.shape[0]
    dv = v.shape[-1]
    o = np.zeros((N, Hv, dv))
    for s in range(len(cu) - 1):
        for h in range(Hv):
            kh = kmap[h]
            S = st[s, h].copy() if has_init[s] else np.zeros_like(st[s, h])
            for c0 in range(cu[s], cu[s + 1], chunk_len):
                c1 = min(c0 + chunk_len, cu[s + 1])
                n = c1 - c0
                Q = q[c0:c1, kh]
                K = k[c0:c1, kh]
                V = v[c0:c1, h]
                b = beta[c0:c1, h]
                G = np.cumsum(g[c0:c1, h])
                gamma = np.exp(G)
                diff = G[:, None] - G[None, :]
                lower = np.tril(np.ones((n, n), dtype=bool), -1)
                lower_eq = np.tril(np.ones((n, n), dtype=bool), 0)
                decay_lt = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
                decay_le = np.where(lower_eq, np.exp(np.where(lower_eq, diff, 0.0)), 0.0)
                A = b[:, None] * decay_lt * (K @ K.T)
                T = _unit_lower_inverse(A)
                W = T @ ((b * gamma)[:, None] * K)
                Ut = T @ (b[:, None] * V)
                U = Ut - W @ S.T
                O = gamma[:, None] * (Q @ S.T) + (decay_le * (Q @ K.T)) @ U
                S = gamma[-1] * S + U.T @ (np.exp(G[-1] - G)[:, None] * K)
                o[c0:c1, h] = O
            st[s, h] = S
    return o, st


def segment_bounds(cu_seqlens, nseg: int, chunk_len: int = 64) -> np.ndarray:
    """Split of every sequence into nseg segments of whole chunks, for the
    segment-parallel evaluation below.  The pages print no such split
    (reading; any split gives the same result, the split only decides which
    transitions exist): with n tokens and nc = ceil(n / chunk_len) chunks,
    segment p covers chunks [b(p), b(p + 1)) with b(0) = 0, b(nseg) = nc and
        b(p) = ceil(nc (2 p + 3) / (2 nseg + 3)),   0 < p < nseg,
    i.e. the first segment spans 5 of the 2 nseg + 3 shares and every later
    one 2, and tokens [bos + min(n, b(p) chunk_len), bos + min(n, b(p + 1)
    chunk_len)); the last segments may be short or empty.  Returns int64
    [nseq, nseg, 2] (begin, end)."""
    cu = [int(c) for c in cu_seqlens]
    out = np.zeros((len(cu) - 1, nseg, 2), dtype=np.int64)
    shares = 2 * nseg + 3
    for s in range(len(cu) - 1):
        n = cu[s + 1] - cu[s]
        nc = -(-n // chunk_len)
        b = [0] + [-(-(nc * (2 * p + 3)) // shares) for p in range(1, nseg)] + [nc]
        for p in range(nseg):
            out[s, p, 0] = cu[s] + min(n, b[p] * chunk_len)
            out[s, p, 1] = cu[s] + min(n, b[p + 1] * chunk_len)
    return out


def segment_transition(k, g, beta, cu_seqlens, Hk, Hv):
    """State transition of the gated delta rule over each sequence [GDN].
    Every token's step is affine in the state:
        S_t = S_{t-1} M_t + b_t v_t k_t^T,   M_t = a_t (I - b_t k_t k_t^T),
    so a run of tokens t_1 .. t_n entering with any S ends at
        S P + R,   P = M_{t_1} M_{t_2} ... M_{t_n}   (dk x dk),
    where R is the state the run reaches from S = 0 (delta_rule_recurrent
    with no initial state).  P depends on k, g and beta only, not on v.  The
    pages print no segment-parallel form (reading: this is the composition
    of the per-token rule).  P is formed token by token, P <- P M_t, from
    P = I.  Returns P [nseq, Hv, dk, dk], float64."""
    k = np.asarray(k, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    kmap = _kv_head_map(Hk, Hv)
    cu = [int(c) for c in cu_seqlens]
    dk = k.shape[-1]
    out = np.zeros((len(cu) - 1, Hv, dk, dk))
    for s in range(len(cu) - 1):
        P = np.broadcast_to(np.eye(dk), (Hv, dk, dk)).copy()
        for t in range(cu[s], cu[s + 1]):
            kt = k[t, kmap]                                          # [Hv, dk]
            M = np.eye(dk)[None] - beta[t][:, None, None] * kt[:, :, None] * kt[:, None, :]
            P = np.exp(g[t])[:, None, None] * (P @ M)
        out[s] = P
    return out


def delta_rule_segmented(q, k, v, g, beta, state0, has_init, cu_seqlens, Hk, Hv, nseg,
                         chunk_len=64):
    """The gated delta rule evaluated segment-parallel [GDN; reading, as
    segment_transition]: each sequence is split by segment_bounds, then
      1. segment 0 runs from the entering state (or 0) and gives X_1, the
         state entering segment 1; every later segment p gives its
         transition (P_p, R_p), independently of the others;
      2. X_{p+1} = X_p P_p + R_p for p = 1 .. nseg - 2;
      3. every segment p >= 1 runs again from X_p, which gives its outputs
         and, for the last segment, the final state.
    Returns the same as delta_rule_recurrent, to which it is equal up to
    rounding.  chunk_len is the split granularity of segment_bounds."""
    cu = [int(c) for c in cu_seqlens]
    bounds = segment_bounds(cu, nseg, chunk_len)
    st0 = np.asarray(state0, dtype=np.float64)
    N = np.asarray(q).shape[0]
    dv = np.asarray(v).shape[-1]
    o = np.zeros((N, Hv, dv))
    final = np.array(st0, copy=True)
    for s in range(len(cu) - 1):
        def run(p, S, init):
            b, e = int(bounds[s, p, 0]), int(bounds[s, p, 1])
            oo, ss = delta_rule_recurrent(q, k, v, g, beta, S[None], [init], [b, e], Hk, Hv)
            return oo[b:e], ss[0], (b, e)
        oo, X, (b, e) = run(0, st0[s], bool(has_init[s]))
        o[b:e] = oo
        Ps, Rs = [None] * nseg, [None] * nseg
        for p in range(1, nseg):
            b, e = int(bounds[s, p, 0]), int(bounds[s, p, 1])
            Ps[p] = segment_transition(k, g, beta, [b, e], Hk, Hv)[0]
            Rs[p] = run(p, np.zeros_like(st0[s]), False)[1]
        Xs = [None, X]
        for p in range(1, nseg - 1):
            Xs.append(Xs[p] @ Ps[p] + Rs[p])
        for p in range(1, nseg):
            oo, S, (b, e) = run(p, Xs[p], True)
            o[b:e] = oo
            X = S
        final[s] = X
    return o, final


def _unit_lower_inverse(A):
    """(I + A)^-1 for strictly lower triangular A, by forward substitution:
    row i of T is e_i - sum_{j<i} A_ij T_j."""
    n = A.shape[0]
    T = np.eye(n)
    for i in range(1, n):
        T[i] = T[i] - A[i, :i] @ T[:i]
    return T


# --------------------------------------------------------------------------
# a6: commit of a speculative window
# --------------------------------------------------------------------------

def gates(ba, A_log, dt_bias):
    """Gate computation before the recurrence [strata, "Root Cause & RED /
    GREEN Verification" names the gate kernels fused_gdn_ab / gdn_ab_multi;
    vllm155, "The one thing I changed in your tests" names their packed
    float32 input dpacked_ba and a bf16 gate-type instantiation; the pages
    print no formula].

    Reading (the plainest one the rest supports, as in the Gated DeltaNet
    layer): the projection gives, per token and v-head, the pair (b, a)
    packed as ba[..., h, 0] = b, ba[..., h, 1] = a; per v-head parameters
    A_log and dt_bias; then
        beta = sigmoid(b),   g = log a_t = -exp(A_log) * softplus(a + dt_bias).
    ba: [N, Hv, 2]; A_log, dt_bias: [Hv].  Returns (g, beta) float64 [N, Hv]."""
    ba = np.asarray(ba, dtype=np.float64)
    b, a = ba[..., 0], ba[..., 1]
    A_log = np.asarray(A_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    beta = 1.0 / (1.0 + np.exp(-b))
    g = -np.exp(A_log) * np.logaddexp(0.0, a + dt_bias)
    return g, beta


def out_norm_gated(o, z, w, eps):
    """Gated output norm after the recurrence [strata, "Summary" item 2 and
    "Code Object Resource Usage": an output-norm kernel consumes o and a gate
    operand z; the pages print no formula].

    Reading (the plainest one the rest supports, as in the Gated DeltaNet
    layer): per token and v-head, root-mean-square normalisation of o over
    its dv channels, an optional per-channel weight w (ones when None), and
    the gate SiLU(z):
        y_i = o_i / sqrt(mean_j(o_j^2) + eps) * w_i * SiLU(z_i).
    o, z: [..., dv]; w: [dv] or None; eps >= 0.  Returns float64."""
    o = np.asarray(o, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    y = o / np.sqrt(ms + eps)
    if w is not None:
        y = y * np.asarray(w, dtype=np.float64)
    return y * silu(z)


def commit(x, conv_state, state, k, v, g, beta, has_init, cu_seqlens, n_keep, Hk, Hv):
    """Commit of one layer after a speculative-verify window [strata,
    "Problem and result" item 2 and "Summary" item 1: the forward ran with
    commit_state=false, the commit then keeps n_keep tokens of the window and
    recomputes the recurrent state by replaying them].

    For each sequence s with n = n_keep[s] (0 <= n <= L_s):
      conv_state[s] = the last 3 rows of [old rows ; x[cu[s] .. cu[s]+n-1]]
      state[s]      = the recurrence run from the old state over those n
                      tokens (same k_hat, v, g, beta as the forward)
    n = 0 leaves both untouched.  has_init[s] == 0 means the old rows/state
    are zero.  Returns (conv_state, state), float64 copies."""
    x = np.asarray(x, dtype=np.float64)
    cs = np.array(conv_state, dtype=np.float64, copy=True)
    st = np.array(state, dtype=np.float64, copy=True)
    cu = [int(c) for c in cu_seqlens]
    for s in range(len(cu) - 1):
        n = int(n_keep[s])
        if n == 0:
            continue
        old = cs[s] if has_init[s] else np.zeros_like(cs[s])
        ext = np.concatenate([old, x[cu[s]:cu[s] + n]], axis=0)
        cs[s] = ext[-3:]
        sub_cu = [0, n]
        sl = slice(cu[s], cu[s] + n)
        _, S = delta_rule_recurrent(k[sl], k[sl], v[sl], g[sl], beta[sl], st[s:s + 1],
                                    [has_init[s]], sub_cu, Hk, Hv)
        st[s] = S[0]
    return cs, st
