/*
 * gdn.h - C ABI of the MI355X (gfx950) Gated DeltaNet layer hot path.
 *
 * The library (libgdn.so) runs every stage as a hand-written HIP kernel:
 *   1. exact token chunks for the conv          gdn_make_chunks / _device
 *   2. width-4 depthwise causal conv             gdn_causal_conv_fwd
 *   3. SiLU + q|k|v split + per-head L2 norm     gdn_postconv_l2
 *      2 and 3 in one launch                     gdn_conv_postconv_fwd
 *   4. chunked gated delta-rule prefill          gdn_delta_rule_prefill
 *      segment-parallel form for long sequences  gdn_delta_rule_prefill_segmented
 *   5. per-token decode / verify step            gdn_delta_rule_step
 *   6. layer-batched commit of a verify window   gdn_commit
 *   7. fused decode / verify: conv + post-conv + step in one launch
 *                                                gdn_decode_fused
 *   8. gated output norm after the recurrence    gdn_out_norm
 *   9. gate computation before the recurrence   gdn_gates
 *
 * Sources (page title, section):
 *   "perf(gdn): optimize post-conv and causal-conv kernels" (vllm.cpp pull
 *   request 155): "Blocker" (conv over c channels with k = 4 taps, row
 *   padding), "What I verified" and "The one thing I changed in your tests"
 *   (post-conv L2 reduction and its float32 output arm), "New issue #305"
 *   (first chunk reads, last chunk writes conv_state; has_initial_state).
 *   "Strata pull request 3226": "Problem and result" and "Summary" items 1-4
 *   (verify forward with commit_state = false, per-token state-resident step,
 *   layer-batched commit of n_keep tokens by state replay).
 *   The recurrence is the gated delta rule
 *       S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = S_t q_t
 *   (Yang, Kautz, Hatamizadeh, "Gated Delta Networks", 2024).
 *
 * Conventions shared by every call
 *   - Pointers marked (device) are device memory; (host) is host memory.
 *     The caller owns every buffer.  The library allocates nothing (the
 *     segmented prefill takes a caller-owned workspace), keeps no state
 *     between calls and is safe to call from several host threads.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  A returned GDN_OK means the launch was accepted.  A call
 *     only launches kernels on that stream (no allocation, copy, memset or
 *     synchronisation), so it can be recorded by HIP stream capture and
 *     replayed from a graph; the replay reads the buffers' contents at
 *     replay time.
 *   - Activations are float32 (GDN_F32) or bfloat16 (GDN_BF16); conv weights,
 *     gates and both states are float32.  Head sizes dk = dv = 128.
 *   - Packed channels: C = 2*Hk*dk + Hv*dv, laid out q | k | v.  v-head h
 *     reads k-head h / (Hv/Hk).
 *   - Varlen batches: cu_seqlens[nseq+1] (device, int32) with cu[0] = 0,
 *     nondecreasing, cu[nseq] = N.  Device-resident integers are
 *     preconditions: they are not read back on the host.  Sequences are
 *     independent: a run of consecutive sequences [s0, s1) can be passed as
 *     its own batch (token pointers advanced by cu[s0] rows, per-sequence
 *     pointers by s0 entries, cu rebased to start at 0), and gives the same
 *     bits as the whole batch.
 *   - has_initial_state[nseq] (device, uint8; NULL = all set): when 0, the
 *     sequence starts from zero conv rows and a zero recurrent state, and
 *     the stored buffers are not read (they may hold anything, NaN included).
 *   - Empty sequences (cu[s+1] == cu[s]): the final conv rows and recurrent
 *     state are the initial ones.  With has_initial_state[s] = 1 they are left
 *     bit-identical; with 0 every call that writes a final state (the conv
 *     with write_state, the prefill, a committing step, the fused step) writes
 *     zeros, as for a sequence whose tokens are all skipped.  N = 0 with
 *     nseq > 0 is valid: only those zero writes happen (token buffers may be
 *     NULL then).  gdn_commit with n_keep[s] = 0 writes nothing.
 *   - Errors: the host validates arguments before any launch and returns a
 *     gdn_status; gdn_last_error() gives a message (thread-local).  No
 *     exception crosses the ABI.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 1

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef enum {
  GDN_OK = 0,
  GDN_ERR_NULL = 1,      /* a required pointer is NULL */
  GDN_ERR_SHAPE = 2,     /* sizes out of range or inconsistent */
  GDN_ERR_DTYPE = 3,     /* unsupported dtype code */
  GDN_ERR_ALIGN = 4,     /* a pointer or row stride is not 16-byte aligned */
  GDN_ERR_ALIAS = 5,     /* an output overlaps an input it must not overlap */
  GDN_ERR_LAUNCH = 6,    /* the HIP runtime rejected a launch */
  GDN_ERR_CAPACITY = 7   /* an output array is too small */
} gdn_status;

/* One exact conv chunk: tokens [begin, end) of sequence `seq` (global token
 * indices).  flags: GDN_CHUNK_FIRST = the sequence's first chunk (its window
 * reaches into conv_state), GDN_CHUNK_LAST = the sequence's last chunk.
 * seq = -1 marks an unused slot (written by gdn_make_chunks_device). */
typedef struct {
  int32_t seq, begin, end, flags;
} gdn_chunk;

#define GDN_CHUNK_FIRST 1
#define GDN_CHUNK_LAST 2
#define GDN_CHUNK_LEN 64

/* One layer's tensors for gdn_commit (all device pointers).  `x`, `k`, `v`,
 * `g`, `beta` are the exact tensors the verify forward consumed for this
 * layer; `conv_state` and `state` are updated in place. */
typedef struct {
  const void* x;          /* conv input  [N][x_row_stride] activations */
  int64_t x_row_stride;   /* elements, >= C */
  float* conv_state;      /* [nseq][3][C] */
  float* state;           /* [nseq][Hv][dv][dk] */
  const void* k;          /* post-conv k_hat [N][Hk][dk] activations */
  const void* v;          /* post-conv v     [N][Hv][dv] activations */
  const float* g;         /* [N][Hv]  log of the decay gate a_t */
  const float* beta;      /* [N][Hv]  b_t */
} gdn_layer_io;

/* ---- library info ------------------------------------------------------ */

int gdn_abi_version(void);
const char* gdn_status_string(int status);
/* Message for the last non-OK status returned on this host thread. */
const char* gdn_last_error(void);

/* ---- 1. exact token chunks ---------------------------------------------
 * Cuts every sequence into consecutive chunks of `chunk_len` tokens, the
 * last one possibly shorter, ordered by sequence then position; empty
 * sequences emit nothing ("New issue #305": exact chunks, first-chunk /
 * last-chunk roles).  Integer work, bit-exact.
 *
 * chunk_len must lie in 3 .. 64 (GDN_CHUNK_LEN): the conv kernels cover at
 * most 64 tokens per descriptor, and a chunk that does not start its
 * sequence reads the 3 rows before it from the same sequence.  Other
 * values are GDN_ERR_SHAPE (and capacity 0).
 *
 * gdn_chunk_capacity: an upper bound on the number of chunks of any batch
 * with N tokens in nseq sequences: floor((N + nseq*(chunk_len-1)) /
 * chunk_len); 0 for invalid arguments.
 *
 * gdn_make_chunks (host): reads cu_seqlens (host, nseq+1 entries), writes
 * at most `cap` descriptors to out (host).  Returns the count (>= 0), or
 * -GDN_ERR_* (NULL pointer, nseq < 0, chunk_len outside 3..64, cu not
 * nondecreasing from 0, or more than cap chunks).
 *
 * gdn_make_chunks_device: the same list built on the GPU from a device
 * cu_seqlens, written to out (device) with exactly `cap` slots; slots past
 * the real count get seq = -1.  cap must be >= gdn_chunk_capacity(N, nseq,
 * chunk_len) for the batch (precondition).  One small launch. */
int gdn_chunk_capacity(int N, int nseq, int chunk_len);
int gdn_make_chunks(const int32_t* cu_seqlens, int nseq, int chunk_len,
                    gdn_chunk* out, int cap);
int gdn_make_chunks_device(const int32_t* cu_seqlens, int nseq, int chunk_len,
                           gdn_chunk* out, int cap, void* stream);

/* ---- 2. causal conv -----------------------------------------------------
 * Width-4 depthwise causal conv1d over the packed channels ("Blocker":
 * c channels, k = 4 taps; "New issue #305"):
 *   y[t][c] = bias[c] + sum_{j=0..3} w[c][j] * xe[t-3+j][c]
 * where xe is the sequence's input preceded by its 3 stored conv rows
 * (row 0 oldest; zeros when has_initial_state is 0).  Tap w[c][3]
 * multiplies the current token.
 * When write_state != 0, conv_state[s] becomes the last 3 rows of
 * [stored rows ; x of sequence s]; otherwise conv_state is not written.
 * Exactly one wave per (sequence, 256-channel group) touches conv_state:
 * wave 0 of the sequence's first chunk reads the stored rows and, later in
 * the same lanes' program order, writes the final rows, so the in-place
 * update has no cross-workgroup race.  Empty sequences have no chunk; one
 * extra workgroup column writes their zero rows (see "Empty sequences").
 * Descriptor preconditions (device data, not checked): each covers at most
 * 64 tokens of one sequence, and one that is not its sequence's first
 * starts at least 3 tokens into it; gdn_make_chunks* with chunk_len in
 * 3..64 produce such lists.
 *   x           (device) [N][x_row_stride] act, x_row_stride >= C, rows
 *               16-byte aligned
 *   w           (device) float [C][4];  bias (device) float [C] or NULL (0)
 *   conv_state  (device) float [nseq][3][C], read and written in place
 *   chunks      (device) nchunks descriptors (from gdn_make_chunks*);
 *               unused slots (seq = -1) are skipped
 *   y           (device) [N][C] act; must not overlap x or conv_state
 * C must be a multiple of 8. */
int gdn_causal_conv_fwd(const void* x, int64_t x_row_stride, int act,
                        const float* w, const float* bias,
                        float* conv_state, const uint8_t* has_initial_state,
                        const int32_t* cu_seqlens, const gdn_chunk* chunks,
                        int nchunks, int nseq, int N, int C, int write_state,
                        void* y, void* stream);

/* ---- 3. post-conv -------------------------------------------------------
 * s = SiLU(y) = y / (1 + exp(-y)) on all C channels; split q | k | v; per q
 * and k head: q_hat = s * (1 / sqrt(sum(s^2) + eps)).  v = s.
 * ("What I verified", "The one thing I changed in your tests".)
 * The squared norm is summed in one fixed order: a pairwise tree,
 * neighbours first (level l adds adjacent blocks of 2^l elements), each
 * step one float32 addition with no fused multiply-add.  For a float32
 * output, sqrt and division are correctly rounded and SiLU is evaluated in
 * float64 and rounded once to float32; for a bf16 output the scale is the
 * hardware reciprocal square root (about one float32 ulp).
 *   y      (device) [N][y_row_stride] act `in`, y_row_stride >= C
 *   q_out, k_out (device) [N][Hk][dk], v_out [N][Hv][dv], dtype `out`;
 *          none may overlap y
 *   eps > 0 (float32). */
int gdn_postconv_l2(const void* y, int64_t y_row_stride, int in, int N,
                    int Hk, int Hv, int dk, int dv, float eps,
                    void* q_out, void* k_out, void* v_out, int out, void* stream);

/* ---- 3b. conv and post-conv in one launch ---------------------------------
 * gdn_causal_conv_fwd followed by gdn_postconv_l2 (out = act), with y kept
 * on chip: each lane forms y for 8 adjacent channels, rounds it to the
 * activation dtype as the stored y would be, and applies SiLU, the head's
 * sum of squares in the documented order (one 128-channel head per 16-lane
 * row, the post-conv kernel's tree) and the L2 scale on q and k.
 * Results are bitwise equal to the two calls ("perf(gdn): optimize
 * post-conv and causal-conv kernels", "What I verified": the fixed order is
 * what makes that checkable).  conv_state is updated as by the conv.
 *   x, x_row_stride, w, bias, conv_state, has_initial_state, cu_seqlens,
 *   chunks, nchunks, nseq, N, write_state: as gdn_causal_conv_fwd, except
 *   that chunks may be NULL when nseq <= 64: the launch then derives the
 *   64-token chunks of gdn_make_chunks from cu_seqlens itself (nchunks is
 *   not used; the same chunks, so the same results), saving the
 *   descriptor-builder launch.  NULL with nseq > 64 is GDN_ERR_SHAPE.
 *   Hk, Hv, dk, dv, eps: as gdn_postconv_l2 (C = 2 Hk dk + Hv dv)
 *   q, k (device) [N][Hk][dk] act; v (device) [N][Hv][dv] act; none may
 *   overlap x, w, conv_state or each other (GDN_ERR_ALIAS). */
int gdn_conv_postconv_fwd(const void* x, int64_t x_row_stride, int act,
                          const float* w, const float* bias, float* conv_state,
                          const uint8_t* has_initial_state, const int32_t* cu_seqlens,
                          const gdn_chunk* chunks, int nchunks, int nseq, int N,
                          int Hk, int Hv, int dk, int dv, float eps, int write_state,
                          void* q, void* k, void* v, void* stream);

/* ---- 4. chunked prefill --------------------------------------------------
 * Gated delta rule over every sequence of a varlen batch in chunks of 64
 * tokens (chunk-local K K^T and Q K^T on MFMA, unit-lower-triangular solve
 * for the WY factors, float32 state carried between chunks).  For sequence
 * s, v-head h (k-head h/(Hv/Hk)), starting from S = state[s][h] (or 0):
 *   S <- a_t S (I - b_t k k^T) + b_t v k^T,  o_t = S q_t,  a_t = exp(g[t][h])
 * and the final S is written back to state[s][h] (always).
 *   q, k   (device) [N][Hk][dk] act;  v (device) [N][Hv][dv] act
 *   g, beta (device) float [N][Hv]
 *   state  (device) float [nseq][Hv][dv][dk] (k index fastest), in place
 *   o      (device) [N][Hv][dv] act; must not overlap any input. */
int gdn_delta_rule_prefill(const void* q, const void* k, const void* v, int act,
                           const float* g, const float* beta,
                           const int32_t* cu_seqlens, int nseq, int N,
                           int Hk, int Hv, int dk, int dv,
                           float* state, const uint8_t* has_initial_state,
                           void* o, void* stream);

/* ---- 4b. segment-parallel prefill ----------------------------------------
 * The prefill of item 4 with every sequence split into nseg segments of
 * whole 64-token chunks, so that one long sequence occupies nseg times the
 * workgroups.  The pages print no such form; it rests on the per-token rule
 * being affine in the state (the gated delta rule of item 4): a run of tokens
 * entering with S ends at S P + R, with P = M_1 ... M_n, M_t = a_t (I - b_t
 * k_t k_t^T) (dk x dk, independent of v) and R the end state from S = 0.
 * With n tokens in nc = ceil(n / 64) chunks, segment p covers chunks
 * [b(p), b(p + 1)), b(0) = 0, b(nseg) = nc, b(p) = ceil(nc (2 p + 3) /
 * (2 nseg + 3)): the first segment spans 5 of 2 nseg + 3 shares, every later
 * one 2 (it is evaluated once, the later ones three times); tokens
 * [bos + min(n, 64 b(p)), bos + min(n, 64 b(p + 1))).  Three launches:
 *   1. segment 0 from the entering state (its end state is X_1); each later
 *      segment p from S = 0 (R_p) and, with v = 0, from S = I (P_p);
 *   2. X_{p+1} = X_p P_p + R_p (float32), p = 1 .. nseg - 2;
 *   3. each segment p >= 1 again from X_p: its o and, for the last one, the
 *      final state.
 * o and the final state equal item 4's up to rounding (the transitions carry
 * the same bf16 operand rounding as the state does inside the prefill).
 * Arguments as gdn_delta_rule_prefill, and
 *   nseg       1..64; 1 runs gdn_delta_rule_prefill (no workspace needed);
 *              nseg > 1 needs act = GDN_BF16 (GDN_ERR_DTYPE otherwise)
 *   workspace  (device) at least gdn_prefill_segmented_workspace(nseq, Hv,
 *              nseg) bytes, 16-byte aligned, owned by the caller, must not
 *              overlap any argument (GDN_ERR_ALIAS); its contents on entry
 *              are ignored, and on return it holds X, R and P, each
 *              [nseq][nseg][Hv][dk][dk] float32 (index p = 0 unused). */
size_t gdn_prefill_segmented_workspace(int nseq, int Hv, int nseg);
int gdn_delta_rule_prefill_segmented(const void* q, const void* k, const void* v, int act,
                                     const float* g, const float* beta,
                                     const int32_t* cu_seqlens, int nseq, int N,
                                     int Hk, int Hv, int dk, int dv,
                                     float* state, const uint8_t* has_initial_state,
                                     void* o, int nseg, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* ---- 4c. segment-parallel prefill without allocation ------------------------
 * For callers that cannot allocate device memory around the call: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * gdn_delta_rule_prefill_segmented with the workspace taken from a scratch
 * array inside the library (GDN_NOALLOC_SCRATCH_BYTES per GPU, held until
 * the process ends) instead of the caller's buffer; no hipMalloc, hipFree or
 * other allocating call is made.  Same arguments and results (bitwise) as
 * item 4b minus the workspace.
 *   - gdn_prefill_segmented_workspace(nseq, Hv, nseg) must not exceed
 *     GDN_NOALLOC_SCRATCH_BYTES (GDN_ERR_CAPACITY otherwise, before any
 *     launch); e.g. one sequence with Hv = 32 and nseg = 4 takes 24 MiB.
 *   - Every call on a GPU shares that GPU's scratch, which keeps the last
 *     call's X, R and P (nothing in it needs to start at zero): calls that
 *     overlap on one GPU (several streams, several host threads) race.
 *     Issue them on one stream, or use item 4b with separate workspaces.
 *   - The scratch address is looked up once per device, on the first call
 *     for the stream's device; a failure there is GDN_ERR_LAUNCH. */
#define GDN_NOALLOC_SCRATCH_BYTES (24u << 20)
int gdn_delta_rule_prefill_segmented_noalloc(const void* q, const void* k, const void* v, int act,
                                             const float* g, const float* beta,
                                             const int32_t* cu_seqlens, int nseq, int N,
                                             int Hk, int Hv, int dk, int dv,
                                             float* state, const uint8_t* has_initial_state,
                                             void* o, int nseg, void* stream);

/* ---- 5. decode / verify step ---------------------------------------------
 * The same recurrence token by token with the state held in registers
 * ("Summary" item 3: state-resident per-token step).  Every sequence's
 * tokens (a decode token or a window of draft tokens) run in one launch.
 * commit_state != 0 writes the final S back to state; commit_state == 0
 * writes no state at all (verify forward; see gdn_commit).
 * Same operands and layouts as gdn_delta_rule_prefill. */
int gdn_delta_rule_step(const void* q, const void* k, const void* v, int act,
                        const float* g, const float* beta,
                        const int32_t* cu_seqlens, int nseq, int N,
                        int Hk, int Hv, int dk, int dv,
                        float* state, const uint8_t* has_initial_state,
                        void* o, int commit_state, void* stream);

/* ---- 6. layer-batched commit ----------------------------------------------
 * After a verify window ran with write_state = 0 / commit_state = 0, keep
 * the first n = n_keep[s] tokens of every sequence in every layer, in ONE
 * launch ("Problem and result" item 2, "Summary" item 1):
 *   conv_state[s] <- last 3 rows of [stored rows ; x_0 .. x_{n-1}]
 *   state[s]      <- the recurrence replayed over those n tokens from the
 *                    stored state, with the same arithmetic as
 *                    gdn_delta_rule_step (bitwise equal to a step with
 *                    commit_state = 1 over the same n tokens)
 * n = 0 leaves both states bit-identical.
 *   layers     (device) gdn_layer_io[L]
 *   cu_seqlens (device) [nseq+1]; n_keep (device) int32 [nseq], 0 <= n_keep[s]
 *              <= cu[s+1]-cu[s] (precondition)
 *   has_initial_state (device) uint8 [nseq] or NULL. */
int gdn_commit(const gdn_layer_io* layers, int L, const int32_t* cu_seqlens,
               const int32_t* n_keep, const uint8_t* has_initial_state, int nseq,
               int C, int Hk, int Hv, int dk, int dv, int act, void* stream);

/* ---- 7. fused decode / verify step ------------------------------------------
 * One launch per layer for decode tokens and draft windows: the causal conv
 * of each sequence's tokens (stored conv rows as history), SiLU, the q / k
 * L2 norm and the recurrence step, without writing y, q, k or v to memory.
 * The result is bitwise equal to gdn_causal_conv_fwd (write_state =
 * write_conv_state) + gdn_postconv_l2 (out dtype = act) +
 * gdn_delta_rule_step (commit_state) on the same inputs.  One workgroup per
 * (sequence, k-head) owns the k-head's q, k channels and the v channels of
 * its v-heads, so the in-place conv_state update is race-free.
 * Fuses the three calls that "Summary" items 2-3 ("Strata pull request
 * 3226") keep as separate verify-forward launches.
 *   x, x_row_stride, w, bias, conv_state: as gdn_causal_conv_fwd
 *   g, beta, state, has_initial_state, o: as gdn_delta_rule_step
 *   k_out, v_out (device, optional, NULL = not written) [N, Hk, dk] and
 *       [N, Hv, dv] in the activation dtype, 16-byte aligned: the normalised
 *       k and the v of every token, bitwise equal to gdn_postconv_l2's k and
 *       v, for a later gdn_commit of a verify window (its replay reads them).
 *   Hv must equal Hk or 2*Hk (GDN_ERR_SHAPE otherwise); eps > 0.
 *   o, k_out, v_out, state and conv_state must not overlap x or each other. */
int gdn_decode_fused(const void* x, int64_t x_row_stride, int act,
                     const float* w, const float* bias, float* conv_state,
                     const int32_t* cu_seqlens, int nseq, int N,
                     int Hk, int Hv, int dk, int dv, float eps,
                     const float* g, const float* beta, float* state,
                     const uint8_t* has_initial_state, void* o,
                     void* k_out, void* v_out,
                     int write_conv_state, int commit_state, void* stream);

/* ---- 8. gated output norm ---------------------------------------------------
 * After the recurrence, per token t and v-head h over the dv = 128 channels:
 *   y[t][h][i] = o[t][h][i] / sqrt(mean_j o[t][h][j]^2 + eps) * w[i] * SiLU(z[t][h][i])
 * ("Strata pull request 3226", "Summary" item 2 and "Code Object Resource
 * Usage" name an output-norm kernel on o and a gate operand z; the pages
 * print no formula, this is the plainest reading).  Arithmetic in float32;
 * the sum of squares uses the post-conv kernel's neighbours-first order.
 *   o, z (device) [N, Hv, dv] in the activation dtype act, 16-byte aligned
 *   w    (device, optional) float32 [dv]; NULL means all ones
 *   y    (device) [N, Hv, dv] in act; may be o itself (in place), otherwise
 *        must not overlap o, z or w (GDN_ERR_ALIAS)
 *   dv must be 128, eps > 0 (GDN_ERR_SHAPE); N = 0 is a no-op. */
int gdn_out_norm(const void* o, const void* z, int act, const float* w,
                 int N, int Hv, int dv, float eps, void* y, void* stream);

/* ---- 9. gate computation ----------------------------------------------------
 * Before the recurrence, per token t and v-head h, from the packed pair
 * ba[t][h] = (b, a) and the per-head parameters A_log, dt_bias:
 *   beta[t][h] = sigmoid(b),  g[t][h] = log a_t = -exp(A_log[h]) * softplus(a + dt_bias[h])
 * ("Strata pull request 3226", "Root Cause & RED / GREEN Verification",
 * names the gate kernels; "perf(gdn): optimize post-conv and causal-conv
 * kernels", "The one thing I changed in your tests", their packed float32
 * input and a bf16 gate type; the pages print no formula, this is the
 * plainest reading).  g and beta are the float32 gates the recurrence
 * entry points take.  Float32 arithmetic with the HIP math library.
 *   ba      (device) [N, Hv, 2] in gate_act (GDN_F32: 8-byte aligned,
 *           GDN_BF16: 4-byte aligned)
 *   A_log, dt_bias (device) float32 [Hv]
 *   g, beta (device) float32 [N, Hv], 4-byte aligned, overlapping nothing
 *   N = 0 is a no-op; Hv >= 1. */
int gdn_gates(const void* ba, int gate_act, const float* A_log, const float* dt_bias,
              int N, int Hv, float* g, float* beta, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
