// C-ABI entry points of libgdn.so: argument validation, then one launch
// each.  Declarations and contracts: include/gdn.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return GDN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int dtype) { return dtype == GDN_F32 ? 4 : 2; }

bool valid_dtype(int d) { return d == GDN_F32 || d == GDN_BF16; }

// [a, a + na) and [b, b + nb) overlap?
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int check_heads(int Hk, int Hv, int dk, int dv) {
  if (dk != 128 || dv != 128) return fail(GDN_ERR_SHAPE, "head sizes must be dk = dv = 128 (got %d, %d)", dk, dv);
  if (Hk < 1 || Hv < 1 || Hv % Hk != 0)
    return fail(GDN_ERR_SHAPE, "need Hk >= 1 and Hv a multiple of Hk (got Hk=%d Hv=%d)", Hk, Hv);
  return GDN_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// The conv kernels cover at most 64 tokens per descriptor, and a non-first
// chunk reads the 3 rows before it from its own sequence, so chunks are
// 3 .. 64 tokens long.
bool valid_chunk_len(int chunk_len) { return chunk_len >= 3 && chunk_len <= GDN_CHUNK_LEN; }

int check_recurrence(const void* q, const void* k, const void* v, int act, const float* g,
                     const float* beta, const int32_t* cu, int nseq, int N, int Hk, int Hv,
                     int dk, int dv, const float* state, const void* o) {
  if (!valid_dtype(act)) return fail(GDN_ERR_DTYPE, "unsupported activation dtype %d", act);
  if (nseq < 0 || N < 0) return fail(GDN_ERR_SHAPE, "negative nseq or N");
  int st = check_heads(Hk, Hv, dk, dv);
  if (st != GDN_OK) return st;
  if (nseq == 0) return GDN_OK;
  if (!cu || !state) return fail(GDN_ERR_NULL, "cu_seqlens and state are required");
  if (N > 0 && (!q || !k || !v || !g || !beta || !o)) return fail(GDN_ERR_NULL, "q, k, v, g, beta and o are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(state) || !aligned16(o))
    return fail(GDN_ERR_ALIGN, "q, k, v, o and state must be 16-byte aligned");
  const size_t e = elem_bytes(act);
  const size_t nq = (size_t)N * Hk * dk * e, nv = (size_t)N * Hv * dv * e;
  const size_t no = (size_t)N * Hv * dv * e, ns = (size_t)nseq * Hv * dv * dk * 4;
  const size_t ng = (size_t)N * Hv * 4;
  if (overlaps(o, no, q, nq) || overlaps(o, no, k, nq) || overlaps(o, no, v, nv) ||
      overlaps(o, no, g, ng) || overlaps(o, no, beta, ng) || overlaps(o, no, state, ns) ||
      overlaps(state, ns, q, nq) || overlaps(state, ns, k, nq) || overlaps(state, ns, v, nv))
    return fail(GDN_ERR_ALIAS, "o and state must not overlap q, k, v, g, beta or each other");
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_string(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL: return "null pointer";
    case GDN_ERR_SHAPE: return "bad shape";
    case GDN_ERR_DTYPE: return "bad dtype";
    case GDN_ERR_ALIGN: return "misaligned pointer or stride";
    case GDN_ERR_ALIAS: return "overlapping buffers";
    case GDN_ERR_LAUNCH: return "launch failed";
    case GDN_ERR_CAPACITY: return "output capacity too small";
    default: return "unknown status";
  }
}

const char* gdn_last_error(void) { return g_last_error; }

int gdn_chunk_capacity(int N, int nseq, int chunk_len) {
  if (N < 0 || nseq < 0 || !valid_chunk_len(chunk_len)) return 0;
  const long long cap = ((long long)N + (long long)nseq * (chunk_len - 1)) / chunk_len;
  return cap > 0x7fffffff ? 0x7fffffff : (int)cap;
}

int gdn_make_chunks(const int32_t* cu, int nseq, int chunk_len, gdn_chunk* out, int cap) {
  if (nseq < 0) return -fail(GDN_ERR_SHAPE, "nseq < 0");
  if (!valid_chunk_len(chunk_len)) return -fail(GDN_ERR_SHAPE, "chunk_len must be in 3..64 (got %d)", chunk_len);
  if (cu == nullptr) return -fail(GDN_ERR_NULL, "cu_seqlens is NULL");
  if (cu[0] != 0) return -fail(GDN_ERR_SHAPE, "cu_seqlens[0] must be 0");
  int count = 0;
  for (int s = 0; s < nseq; ++s) {
    const int b = cu[s], e = cu[s + 1];
    if (e < b) return -fail(GDN_ERR_SHAPE, "cu_seqlens decreases at %d", s);
    for (int j = 0, t = b; t < e; ++j, t += chunk_len) {
      if (count >= cap) return -fail(GDN_ERR_CAPACITY, "more than %d chunks", cap);
      if (out == nullptr) return -fail(GDN_ERR_NULL, "out is NULL");
      gdn_chunk& c = out[count++];
      c.seq = s;
      c.begin = t;
      c.end = (e - t < chunk_len) ? e : t + chunk_len;
      c.flags = (j == 0 ? GDN_CHUNK_FIRST : 0) | (c.end == e ? GDN_CHUNK_LAST : 0);
    }
  }
  return count;
}

int gdn_make_chunks_device(const int32_t* cu, int nseq, int chunk_len, gdn_chunk* out, int cap,
                           void* stream) {
  if (nseq < 0 || cap < 0) return -fail(GDN_ERR_SHAPE, "nseq or cap < 0");
  if (!valid_chunk_len(chunk_len)) return -fail(GDN_ERR_SHAPE, "chunk_len must be in 3..64 (got %d)", chunk_len);
  if (cap == 0) return GDN_OK;
  if (cu == nullptr || out == nullptr) return -fail(GDN_ERR_NULL, "cu_seqlens and out are required");
  const int st = launched(gdn::launch_make_chunks(cu, nseq, chunk_len, out, cap, as_stream(stream)),
                          "make_chunks");
  return st == GDN_OK ? GDN_OK : -st;
}

int gdn_causal_conv_fwd(const void* x, int64_t xs, int act, const float* w, const float* bias,
                        float* conv_state, const uint8_t* has_init, const int32_t* cu,
                        const gdn_chunk* chunks, int nchunks, int nseq, int N, int C,
                        int write_state, void* y, void* stream) {
  if (!valid_dtype(act)) return fail(GDN_ERR_DTYPE, "unsupported activation dtype %d", act);
  if (N < 0 || nseq < 0 || nchunks < 0 || C < 8 || C % 8 != 0 || xs < C)
    return fail(GDN_ERR_SHAPE, "need N, nseq, nchunks >= 0, C a positive multiple of 8, x_row_stride >= C");
  // with no tokens only the final rows of empty sequences are written
  if (N == 0) nchunks = 0;
  if (nseq == 0 || (nchunks == 0 && !write_state)) return GDN_OK;
  if (!conv_state || !cu) return fail(GDN_ERR_NULL, "conv_state and cu_seqlens are required");
  if (N > 0 && (!x || !w || !chunks || !y)) return fail(GDN_ERR_NULL, "x, w, chunks and y are required");
  const int e = elem_bytes(act);
  if (!aligned16(x) || ((size_t)xs * e) % 16 != 0 || !aligned16(w) || !aligned16(conv_state) ||
      !aligned16(y) || (bias && !aligned16(bias)))
    return fail(GDN_ERR_ALIGN, "x rows, w, bias, conv_state and y must be 16-byte aligned");
  const size_t ny = (size_t)N * C * e;
  const size_t nx = N > 0 ? ((size_t)(N - 1) * xs + C) * e : 0;
  const size_t ns = (size_t)nseq * 3 * C * 4;
  if (overlaps(y, ny, x, nx) || overlaps(y, ny, conv_state, ns) || overlaps(y, ny, w, (size_t)C * 16))
    return fail(GDN_ERR_ALIAS, "y must not overlap x, w or conv_state");
  if (overlaps(conv_state, ns, x, nx)) return fail(GDN_ERR_ALIAS, "conv_state must not overlap x");
  return launched(gdn::launch_conv(x, xs, act, w, bias, conv_state, has_init, cu, chunks, nchunks, nseq, C,
                                   write_state, y, as_stream(stream)),
                  "causal_conv");
}

int gdn_conv_postconv_fwd(const void* x, int64_t xs, int act, const float* w, const float* bias,
                          float* conv_state, const uint8_t* has_init, const int32_t* cu,
                          const gdn_chunk* chunks, int nchunks, int nseq, int N, int Hk, int Hv, int dk,
                          int dv, float eps, int write_state, void* q, void* k, void* v, void* stream) {
  if (!valid_dtype(act)) return fail(GDN_ERR_DTYPE, "unsupported activation dtype %d", act);
  int st = check_heads(Hk, Hv, dk, dv);
  if (st != GDN_OK) return st;
  const int C = 2 * Hk * dk + Hv * dv;
  if (N < 0 || nseq < 0 || nchunks < 0 || xs < C)
    return fail(GDN_ERR_SHAPE, "need N, nseq, nchunks >= 0 and x_row_stride >= C");
  if (!(eps > 0.f)) return fail(GDN_ERR_SHAPE, "eps must be > 0");
  // chunks == NULL: the launch derives the 64-token chunks from cu_seqlens
  // (nseq <= 64), over floor(N / 64) + nseq slots; nchunks is not used
  if (chunks == nullptr) {
    if (nseq > 64) return fail(GDN_ERR_SHAPE, "chunks may be NULL only for nseq <= 64 (got %d)", nseq);
    nchunks = N / 64 + nseq;
  }
  // with no tokens only the final rows of empty sequences are written
  if (N == 0) nchunks = 0;
  if (nseq == 0 || (nchunks == 0 && !write_state)) return GDN_OK;
  if (!conv_state || !cu) return fail(GDN_ERR_NULL, "conv_state and cu_seqlens are required");
  if (N > 0 && (!x || !w || !q || !k || !v)) return fail(GDN_ERR_NULL, "x, w, q, k and v are required");
  const int e = elem_bytes(act);
  if (!aligned16(x) || ((size_t)xs * e) % 16 != 0 || !aligned16(w) || !aligned16(conv_state) ||
      (bias && !aligned16(bias)) || !aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(GDN_ERR_ALIGN, "x rows, w, bias, conv_state, q, k and v must be 16-byte aligned");
  const size_t nx = N > 0 ? ((size_t)(N - 1) * xs + C) * e : 0, ns = (size_t)nseq * 3 * C * 4;
  const size_t nq = (size_t)N * Hk * dk * e, nv = (size_t)N * Hv * dv * e;
  struct Buf { const void* p; size_t n; } out[4] = {{q, nq}, {k, nq}, {v, nv}, {conv_state, ns}};
  for (int i = 0; i < 4; ++i) {
    if (overlaps(out[i].p, out[i].n, x, nx) || overlaps(out[i].p, out[i].n, w, (size_t)C * 16))
      return fail(GDN_ERR_ALIAS, "q, k, v and conv_state must not overlap x, w or each other");
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(out[i].p, out[i].n, out[j].p, out[j].n))
        return fail(GDN_ERR_ALIAS, "q, k, v and conv_state must not overlap x, w or each other");
  }
  return launched(gdn::launch_conv_postconv(x, xs, act, w, bias, conv_state, has_init, cu, chunks, nchunks, nseq,
                                            Hk, Hv, eps, write_state, q, k, v, as_stream(stream)),
                  "conv_postconv");
}

int gdn_postconv_l2(const void* y, int64_t ys, int in, int N, int Hk, int Hv, int dk, int dv,
                    float eps, void* q, void* k, void* v, int out, void* stream) {
  if (!valid_dtype(in) || !valid_dtype(out)) return fail(GDN_ERR_DTYPE, "unsupported dtype");
  int st = check_heads(Hk, Hv, dk, dv);
  if (st != GDN_OK) return st;
  const int C = 2 * Hk * dk + Hv * dv;
  if (N < 0 || ys < C) return fail(GDN_ERR_SHAPE, "need N >= 0 and y_row_stride >= C");
  if (!(eps > 0.f)) return fail(GDN_ERR_SHAPE, "eps must be > 0");
  if (N == 0) return GDN_OK;
  if (!y || !q || !k || !v) return fail(GDN_ERR_NULL, "missing required pointer");
  const int ei = elem_bytes(in), eo = elem_bytes(out);
  if (!aligned16(y) || ((size_t)ys * ei) % 16 != 0 || !aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(GDN_ERR_ALIGN, "y rows, q, k and v must be 16-byte aligned");
  const size_t ny = ((size_t)(N - 1) * ys + C) * ei;
  const size_t nq = (size_t)N * Hk * dk * eo, nv = (size_t)N * Hv * dv * eo;
  if (overlaps(q, nq, y, ny) || overlaps(k, nq, y, ny) || overlaps(v, nv, y, ny) ||
      overlaps(q, nq, k, nq) || overlaps(q, nq, v, nv) || overlaps(k, nq, v, nv))
    return fail(GDN_ERR_ALIAS, "q, k, v must not overlap y or each other");
  return launched(gdn::launch_postconv(y, ys, in, N, Hk, Hv, eps, q, k, v, out, as_stream(stream)),
                  "postconv_l2");
}

int gdn_delta_rule_prefill(const void* q, const void* k, const void* v, int act, const float* g,
                           const float* beta, const int32_t* cu, int nseq, int N, int Hk, int Hv,
                           int dk, int dv, float* state, const uint8_t* has_init, void* o,
                           void* stream) {
  int st = check_recurrence(q, k, v, act, g, beta, cu, nseq, N, Hk, Hv, dk, dv, state, o);
  if (st != GDN_OK || nseq == 0) return st;
  return launched(gdn::launch_prefill(q, k, v, act, g, beta, cu, nseq, Hk, Hv, state, has_init, o,
                                      as_stream(stream)),
                  "delta_rule_prefill");
}

size_t gdn_prefill_segmented_workspace(int nseq, int Hv, int nseg) {
  if (nseq <= 0 || Hv <= 0 || nseg <= 1) return 0;
  return (size_t)3 * nseq * nseg * Hv * 128 * 128 * sizeof(float);
}

int gdn_delta_rule_prefill_segmented(const void* q, const void* k, const void* v, int act,
                                     const float* g, const float* beta, const int32_t* cu, int nseq,
                                     int N, int Hk, int Hv, int dk, int dv, float* state,
                                     const uint8_t* has_init, void* o, int nseg, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  int st = check_recurrence(q, k, v, act, g, beta, cu, nseq, N, Hk, Hv, dk, dv, state, o);
  if (st != GDN_OK) return st;
  if (nseg < 1 || nseg > 64) return fail(GDN_ERR_SHAPE, "nseg must be in 1..64 (got %d)", nseg);
  if (nseg == 1) return gdn_delta_rule_prefill(q, k, v, act, g, beta, cu, nseq, N, Hk, Hv, dk, dv, state,
                                               has_init, o, stream);
  if (act != GDN_BF16) return fail(GDN_ERR_DTYPE, "the segmented prefill needs bf16 activations");
  if (nseq == 0) return GDN_OK;
  if ((size_t)nseq * Hv * 2 * (2 * nseg - 1) > (size_t)INT32_MAX) return fail(GDN_ERR_SHAPE, "grid too large");
  const size_t need = gdn_prefill_segmented_workspace(nseq, Hv, nseg);
  if (!workspace) return fail(GDN_ERR_NULL, "workspace is required when nseg > 1");
  if (!aligned16(workspace)) return fail(GDN_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(GDN_ERR_CAPACITY, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  const size_t e = elem_bytes(act);
  const size_t nq = (size_t)N * Hk * dk * e, nv = (size_t)N * Hv * dv * e, ng = (size_t)N * Hv * 4;
  const size_t ns = (size_t)nseq * Hv * dv * dk * 4;
  if (overlaps(workspace, need, q, nq) || overlaps(workspace, need, k, nq) || overlaps(workspace, need, v, nv) ||
      overlaps(workspace, need, g, ng) || overlaps(workspace, need, beta, ng) ||
      overlaps(workspace, need, o, nv) || overlaps(workspace, need, state, ns))
    return fail(GDN_ERR_ALIAS, "workspace must not overlap q, k, v, g, beta, o or state");
  return launched(gdn::launch_prefill_segmented(q, k, v, g, beta, cu, nseq, Hk, Hv, state, has_init, o, nseg,
                                                static_cast<float*>(workspace), as_stream(stream)),
                  "delta_rule_prefill_segmented");
}

int gdn_delta_rule_prefill_segmented_noalloc(const void* q, const void* k, const void* v, int act,
                                             const float* g, const float* beta, const int32_t* cu,
                                             int nseq, int N, int Hk, int Hv, int dk, int dv, float* state,
                                             const uint8_t* has_init, void* o, int nseg, void* stream) {
  int st = check_recurrence(q, k, v, act, g, beta, cu, nseq, N, Hk, Hv, dk, dv, state, o);
  if (st != GDN_OK) return st;
  if (nseg < 1 || nseg > 64) return fail(GDN_ERR_SHAPE, "nseg must be in 1..64 (got %d)", nseg);
  if (nseg == 1) return gdn_delta_rule_prefill(q, k, v, act, g, beta, cu, nseq, N, Hk, Hv, dk, dv, state,
                                               has_init, o, stream);
  if (act != GDN_BF16) return fail(GDN_ERR_DTYPE, "the segmented prefill needs bf16 activations");
  if (nseq == 0) return GDN_OK;
  const size_t need = gdn_prefill_segmented_workspace(nseq, Hv, nseg);
  if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES)
    return fail(GDN_ERR_CAPACITY, "nseq %d x nseg %d x Hv %d needs %zu bytes of scratch; the limit is %zu",
                nseq, nseg, Hv, need, (size_t)GDN_NOALLOC_SCRATCH_BYTES);
  float* ws = nullptr;
  const hipError_t e = gdn::noalloc_scratch(as_stream(stream), &ws);
  if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "scratch address: %s", hipGetErrorString(e));
  return launched(gdn::launch_prefill_segmented(q, k, v, g, beta, cu, nseq, Hk, Hv, state, has_init, o, nseg, ws,
                                                as_stream(stream)),
                  "delta_rule_prefill_segmented_noalloc");
}

int gdn_delta_rule_step(const void* q, const void* k, const void* v, int act, const float* g,
                        const float* beta, const int32_t* cu, int nseq, int N, int Hk, int Hv,
                        int dk, int dv, float* state, const uint8_t* has_init, void* o,
                        int commit_state, void* stream) {
  int st = check_recurrence(q, k, v, act, g, beta, cu, nseq, N, Hk, Hv, dk, dv, state, o);
  // with no tokens a committing step still writes the (zero) states of
  // sequences without an initial state
  if (st != GDN_OK || nseq == 0 || (N == 0 && !commit_state)) return st;
  return launched(gdn::launch_step(q, k, v, act, g, beta, cu, nseq, Hk, Hv, state, has_init, o,
                                   commit_state, as_stream(stream)),
                  "delta_rule_step");
}

int gdn_decode_fused(const void* x, int64_t xs, int act, const float* w, const float* bias,
                     float* conv_state, const int32_t* cu, int nseq, int N, int Hk, int Hv, int dk,
                     int dv, float eps, const float* g, const float* beta, float* state,
                     const uint8_t* has_init, void* o, void* k_out, void* v_out,
                     int write_conv_state, int commit_state, void* stream) {
  if (!valid_dtype(act)) return fail(GDN_ERR_DTYPE, "unsupported activation dtype %d", act);
  if (nseq < 0 || N < 0) return fail(GDN_ERR_SHAPE, "negative nseq or N");
  int st = check_heads(Hk, Hv, dk, dv);
  if (st != GDN_OK) return st;
  if (Hv != Hk && Hv != 2 * Hk) return fail(GDN_ERR_SHAPE, "the fused step needs Hv = Hk or Hv = 2*Hk (got Hk=%d Hv=%d)", Hk, Hv);
  if (!(eps > 0.f)) return fail(GDN_ERR_SHAPE, "eps must be > 0");
  const int C = 2 * Hk * dk + Hv * dv;
  if (xs < C) return fail(GDN_ERR_SHAPE, "x_row_stride must be >= C");
  if (xs > (int64_t)(1 << 24)) return fail(GDN_ERR_SHAPE, "x_row_stride above 2^24 elements");
  if (nseq == 0 || (N == 0 && !write_conv_state && !commit_state)) return GDN_OK;
  if (!conv_state || !cu || !state) return fail(GDN_ERR_NULL, "conv_state, cu_seqlens and state are required");
  if (N > 0 && (!x || !w || !g || !beta || !o))
    return fail(GDN_ERR_NULL, "x, w, g, beta and o are required");
  const size_t e = elem_bytes(act);
  if (!aligned16(x) || ((size_t)xs * e) % 16 != 0 || !aligned16(w) || (bias && !aligned16(bias)) ||
      !aligned16(conv_state) || !aligned16(state) || !aligned16(o) || (k_out && !aligned16(k_out)) ||
      (v_out && !aligned16(v_out)))
    return fail(GDN_ERR_ALIGN, "x rows, w, bias, conv_state, state, o, k_out and v_out must be 16-byte aligned");
  const size_t nx = N > 0 ? ((size_t)(N - 1) * xs + C) * e : 0, ncs = (size_t)nseq * 3 * C * 4;
  const size_t no = (size_t)N * Hv * dv * e, ns = (size_t)nseq * Hv * dv * dk * 4;
  const size_t nk = k_out ? (size_t)N * Hk * dk * e : 0, nv = v_out ? (size_t)N * Hv * dv * e : 0;
  struct Buf { const void* p; size_t n; } out[5] = {{o, no}, {state, ns}, {conv_state, ncs}, {k_out, nk}, {v_out, nv}};
  for (int i = 0; i < 5; ++i) {
    if (overlaps(out[i].p, out[i].n, x, nx))
      return fail(GDN_ERR_ALIAS, "o, k_out, v_out, state and conv_state must not overlap x or each other");
    for (int j = i + 1; j < 5; ++j)
      if (overlaps(out[i].p, out[i].n, out[j].p, out[j].n))
        return fail(GDN_ERR_ALIAS, "o, k_out, v_out, state and conv_state must not overlap x or each other");
  }
  return launched(gdn::launch_decode_fused(x, xs, act, w, bias, conv_state, cu, nseq, Hk, Hv, eps, g, beta,
                                           state, has_init, o, k_out, v_out, write_conv_state, commit_state,
                                           as_stream(stream)),
                  "decode_fused");
}

int gdn_gates(const void* ba, int gate_act, const float* A_log, const float* dt_bias, int N, int Hv,
              float* g, float* beta, void* stream) {
  if (!valid_dtype(gate_act)) return fail(GDN_ERR_DTYPE, "unsupported gate dtype %d", gate_act);
  if (N < 0 || Hv < 1) return fail(GDN_ERR_SHAPE, "need N >= 0 and Hv >= 1");
  const size_t rows = (size_t)N * Hv;
  if (rows * 8 >= 0x7fffffffULL) return fail(GDN_ERR_SHAPE, "N * Hv too large");
  if (N == 0) return GDN_OK;
  if (!ba || !A_log || !dt_bias || !g || !beta)
    return fail(GDN_ERR_NULL, "ba, A_log, dt_bias, g and beta are required");
  const size_t pair = gate_act == GDN_F32 ? 8 : 4;
  if (reinterpret_cast<uintptr_t>(ba) % pair != 0 || reinterpret_cast<uintptr_t>(g) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(beta) % 4 != 0 || reinterpret_cast<uintptr_t>(A_log) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(dt_bias) % 4 != 0)
    return fail(GDN_ERR_ALIGN, "ba must be aligned to its (b, a) pair, the float32 arrays to 4 bytes");
  const size_t nb = rows * pair, ng = rows * 4, np = (size_t)Hv * 4;
  if (overlaps(g, ng, beta, ng) || overlaps(g, ng, ba, nb) || overlaps(beta, ng, ba, nb) ||
      overlaps(g, ng, A_log, np) || overlaps(g, ng, dt_bias, np) || overlaps(beta, ng, A_log, np) ||
      overlaps(beta, ng, dt_bias, np))
    return fail(GDN_ERR_ALIAS, "g and beta must not overlap each other or the inputs");
  return launched(gdn::launch_gates(ba, gate_act, A_log, dt_bias, (int)rows, Hv, g, beta, as_stream(stream)),
                  "gates");
}

int gdn_out_norm(const void* o, const void* z, int act, const float* w, int N, int Hv, int dv,
                 float eps, void* y, void* stream) {
  if (!valid_dtype(act)) return fail(GDN_ERR_DTYPE, "unsupported activation dtype %d", act);
  if (N < 0 || Hv < 1) return fail(GDN_ERR_SHAPE, "need N >= 0 and Hv >= 1");
  if (dv != 128) return fail(GDN_ERR_SHAPE, "dv must be 128 (got %d)", dv);
  if (!(eps > 0.f)) return fail(GDN_ERR_SHAPE, "eps must be > 0");
  const size_t e = elem_bytes(act);
  const size_t n = (size_t)N * Hv * dv * e;
  if (n >= 0x7fffffffULL) return fail(GDN_ERR_SHAPE, "N * Hv * dv elements exceed 2 GiB");
  if (N == 0) return GDN_OK;
  if (!o || !z || !y) return fail(GDN_ERR_NULL, "o, z and y are required");
  if (!aligned16(o) || !aligned16(z) || !aligned16(y) || (w && !aligned16(w)))
    return fail(GDN_ERR_ALIGN, "o, z, y and w must be 16-byte aligned");
  if ((y != o && overlaps(y, n, o, n)) || overlaps(y, n, z, n) || (w && overlaps(y, n, w, dv * 4)))
    return fail(GDN_ERR_ALIAS, "y must be o itself or overlap none of o, z and w");
  return launched(gdn::launch_out_norm(o, z, act, w, N * Hv, eps, y, as_stream(stream)), "out_norm");
}

int gdn_commit(const gdn_layer_io* layers, int L, const int32_t* cu, const int32_t* n_keep,
               const uint8_t* has_init, int nseq, int C, int Hk, int Hv, int dk, int dv, int act,
               void* stream) {
  if (!valid_dtype(act)) return fail(GDN_ERR_DTYPE, "unsupported activation dtype %d", act);
  int st = check_heads(Hk, Hv, dk, dv);
  if (st != GDN_OK) return st;
  if (L < 0 || nseq < 0) return fail(GDN_ERR_SHAPE, "negative L or nseq");
  if (C != 2 * Hk * dk + Hv * dv) return fail(GDN_ERR_SHAPE, "C must equal 2*Hk*dk + Hv*dv");
  if (L == 0 || nseq == 0) return GDN_OK;
  if (!layers || !cu || !n_keep) return fail(GDN_ERR_NULL, "layers, cu_seqlens and n_keep are required");
  const long long blocks = (long long)L * nseq * (Hv + (C + 1023) / 1024);
  if (blocks > 0x7fffffffLL) return fail(GDN_ERR_SHAPE, "too many (layer, sequence) pairs");
  return launched(gdn::launch_commit(layers, L, cu, n_keep, has_init, nseq, C, Hk, Hv, act,
                                     as_stream(stream)),
                  "commit");
}

}  // extern "C"
