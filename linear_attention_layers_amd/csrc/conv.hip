// Exact token chunks and the width-4 depthwise causal conv (gfx950).
//
// Conv semantics ("perf(gdn): optimize post-conv and causal-conv kernels",
// "Blocker": c channels, k = 4 taps; "New issue #305": the first chunk of a
// sequence reads the stored conv rows, the final rows come from the last
// tokens):  y[t][c] = bias[c] + sum_j w[c][j] * xe[t-3+j][c], where xe is the
// sequence input preceded by its 3 stored rows (oldest first).
//
// Layout: one workgroup per (chunk, group of 256 channels); each lane owns
// 4 adjacent channels, so a wave reads and writes every token row as one
// contiguous 512-byte (bf16) span; each of the 4 waves takes 16 of the
// chunk's tokens, requests all of its rows up front and walks them in order
// with the 3-token window in registers (no cross-lane traffic, no LDS).  A
// wave reads its 3-row halo from x unless it starts a sequence.  Outputs
// are written through a buffer resource spanning exactly the wave's tokens,
// so rows past a chunk's end need no branches.  Four channels per lane keep
// the kernel near 100 registers, so five workgroups share a CU and the
// loads of some overlap the stores of others.
//
// conv_state ownership: only wave 0 of the FIRST chunk's workgroup touches a
// sequence's conv_state.  Its lanes read the stored rows, use them for the
// outputs t < 3 (which forces the loads to complete), and afterwards store
// the final rows, taken from the last 3 tokens of x (or from the shifted
// stored rows when the sequence has fewer than 3 tokens).  Each element is
// read and then written by the same lane, in program order, so updating
// conv_state in place cannot race with any other workgroup.  This replaces
// the "last chunk writes" arrangement whose cross-block race the issue
// describes.
#include "launch.hpp"
#include "mfma.hpp"

namespace gdn {

namespace {

constexpr int kConvThreads = 256;                 // 4 waves
constexpr int kConvChannelsPerLane = 4;
constexpr int kConvChannelsPerBlock = 64 * kConvChannelsPerLane;   // 256
constexpr int kConvTokensPerWave = 16;            // 4 waves x 16 = one 64-token chunk

// ------------------------------------------------------------ chunk builder
// One workgroup.  Up to 64 sequences: wave 0 counts each sequence's chunks
// (lane s), an integer prefix sum over the wave gives each its first slot,
// and after one barrier every thread writes slots tid, tid + 256, ...,
// finding the sequence of its slot by binary search over the first slots
// (the last sequence whose first slot is <= the slot; empty sequences share
// their successor's first slot and are passed over).  Larger batches are
// scanned 256 sequences at a time.  Slots past the total are marked unused
// (seq = -1).
__device__ __forceinline__ int wave_prefix_sum_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
  return v;
}

__device__ __forceinline__ gdn_chunk chunk_of(int s, int j, int n, int begin, int len, int chunk_len) {
  gdn_chunk c;
  c.seq = s;
  c.begin = begin + j * chunk_len;
  c.end = min(c.begin + chunk_len, begin + len);
  c.flags = (j == 0 ? GDN_CHUNK_FIRST : 0) | (j == n - 1 ? GDN_CHUNK_LAST : 0);
  return c;
}

__global__ __launch_bounds__(256) void make_chunks_kernel(const int32_t* __restrict__ cu, int nseq,
                                                          int chunk_len, gdn_chunk* __restrict__ out,
                                                          int cap) {
  __shared__ int s_count[256];
  __shared__ int s_first[65];
  __shared__ int s_base;
  const int tid = threadIdx.x;
  if (nseq <= 64) {
    if (tid < 64) {
      const int s = tid;
      int n = 0;
      if (s < nseq) {
        const int len = cu[s + 1] - cu[s];
        n = len > 0 ? (len + chunk_len - 1) / chunk_len : 0;
      }
      const int incl = wave_prefix_sum_i32(n);
      s_first[s] = incl - n;
      if (s == 63) s_first[64] = incl;   // the total
    }
    __syncthreads();
    const int total = s_first[64];
    for (int slot = tid; slot < cap; slot += 256) {
      gdn_chunk c;
      if (slot < total) {
        int lo = 0, hi = nseq - 1;   // last s with first[s] <= slot
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_first[mid] <= slot) lo = mid; else hi = mid - 1;
        }
        const int begin = cu[lo], len = cu[lo + 1] - begin;
        const int n = (len + chunk_len - 1) / chunk_len;
        c = chunk_of(lo, slot - s_first[lo], n, begin, len, chunk_len);
      } else {
        c.seq = -1; c.begin = 0; c.end = 0; c.flags = 0;
      }
      out[slot] = c;
    }
    return;
  }
  if (tid == 0) s_base = 0;
  __syncthreads();
  for (int s0 = 0; s0 < nseq; s0 += 256) {
    const int s = s0 + tid;
    int begin = 0, len = 0, n = 0;
    if (s < nseq) {
      begin = cu[s];
      len = cu[s + 1] - begin;
      n = len > 0 ? (len + chunk_len - 1) / chunk_len : 0;
    }
    s_count[tid] = n;
    __syncthreads();
    // inclusive Hillis-Steele scan over 256 counts
    for (int off = 1; off < 256; off <<= 1) {
      int add = tid >= off ? s_count[tid - off] : 0;
      __syncthreads();
      s_count[tid] += add;
      __syncthreads();
    }
    const int base = s_base;
    const int first = base + s_count[tid] - n;
    for (int j = 0; j < n; ++j) {
      const int slot = first + j;
      if (slot < cap) out[slot] = chunk_of(s, j, n, begin, len, chunk_len);
    }
    __syncthreads();
    if (tid == 255) s_base = base + s_count[255];
    __syncthreads();
  }
  const int total = s_base;
  for (int slot = total + tid; slot < cap; slot += 256) {
    gdn_chunk c;
    c.seq = -1; c.begin = 0; c.end = 0; c.flags = 0;
    out[slot] = c;
  }
}

// ------------------------------------------------- empty sequences
// A sequence with no tokens has no chunk, so no chunk workgroup owns its
// conv_state.  Its final rows are its initial rows: unchanged with an
// initial state, zeros without one.  One extra slot (a workgroup per
// channel group, launched only when the final rows are written) takes the
// second case: wave 0 finds the empty sequences without an initial state
// 64 at a time (lane = sequence, one ballot) and its lanes store zeros into
// the three rows of their CPL channels of the workgroup's channel group.
template <int CPL>
__device__ __forceinline__ void zero_empty_conv_rows(float* conv_state, const uint8_t* __restrict__ has_init,
                                                     const int32_t* __restrict__ cu, int nseq, int C, int c0,
                                                     int lane) {
  for (int s0 = 0; s0 < nseq; s0 += 64) {
    const int s = s0 + lane;
    const bool empty = s < nseq && cu[s + 1] == cu[s] && !seq_flag(has_init, s);
    uint64_t m = __builtin_amdgcn_ballot_w64(empty);
    while (m != 0) {
      const int se = s0 + __builtin_ctzll(m);
      m &= m - 1;
      if (c0 < C) {
        float* st = conv_state + (int64_t)se * 3 * C + c0;
#pragma unroll
        for (int r = 0; r < 3; ++r)
#pragma unroll
          for (int i = 0; i < CPL; i += 4)
            *reinterpret_cast<float4*>(st + (int64_t)r * C + i) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  }
}

// ---------------------------------------------------------------- the conv
// Workgroup = (chunk slot, group of 256 channels); wave w handles tokens
// [16 w, 16 w + 16) of the chunk and lane l channels 4 l .. 4 l + 3 of the
// group.  A lane issues its 3 halo rows and its 16 token rows up front (19
// independent loads), then computes and stores 16 outputs.  Only wave 0 of
// a sequence's first chunk touches conv_state (see the file comment); the
// slot past the last chunk slot clears the rows of empty sequences.
// Four adjacent activations in storage form.
template <class T> struct Act4;
template <> struct Act4<float> {
  using Raw = float4;
  __device__ __forceinline__ static Raw load(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ static void unpack(Raw r, float (&v)[4]) { v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w; }
  __device__ __forceinline__ static void store(__amdgpu_buffer_rsrc_t rs, int off, const float (&v)[4]) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                                 __float_as_uint(v[3])}, rs, off, 0, 0);
  }
};
template <> struct Act4<uint16_t> {
  using Raw = uint2;
  __device__ __forceinline__ static Raw load(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ static void unpack(Raw r, float (&v)[4]) {
    v[0] = bf16_to_f32(r.x & 0xffffu); v[1] = bf16_to_f32(r.x >> 16);
    v[2] = bf16_to_f32(r.y & 0xffffu); v[3] = bf16_to_f32(r.y >> 16);
  }
  __device__ __forceinline__ static void store(__amdgpu_buffer_rsrc_t rs, int off, const float (&v)[4]) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])}, rs, off, 0, 0);
  }
};

// Work item of a conv launch (1-D grid): channel group `group` (the fastest
// index) of chunk slot `slot`, the slots taken last to first, then the extra
// slot `nslots` (empty sequences' rows) after every chunk.  Workgroups are
// dispatched in index order, so the ones running at any moment cover whole
// rows of x and of the outputs (every channel group of a few chunks:
// contiguous memory spread over all HBM channels) rather than one channel
// group of many chunks (pieces one row pitch apart, which crowd a few
// channels: 87 against 75 us for the mixed serving layer's conv and
// post-conv).  The first chunks of the sequences, which the prefill reads
// first, are written last and are still in L2 when it starts.
struct ConvItem {
  int slot, group;
};
__device__ __forceinline__ ConvItem conv_item(int nslots, int ngroups) {
  const int b = __builtin_amdgcn_readfirstlane((int)blockIdx.x);
  const int r = b / ngroups;
  return {r < nslots ? nslots - 1 - r : nslots, b - r * ngroups};
}

template <class T>
__global__ __launch_bounds__(kConvThreads) void conv_kernel(
    const T* __restrict__ x, int64_t xs, const float* __restrict__ w, const float* __restrict__ bias,
    float* conv_state, const uint8_t* __restrict__ has_init, const int32_t* __restrict__ cu,
    const gdn_chunk* __restrict__ chunks, int nslots, int nseq, int C, int write_state, T* __restrict__ y) {
  using A = Act4<T>;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const ConvItem it = conv_item(nslots, (C + kConvChannelsPerBlock - 1) / kConvChannelsPerBlock);
  const int c0 = (it.group * 64 + lane) * kConvChannelsPerLane;
  if (it.slot == nslots) {   // launched only when write_state
    if (wave == 0) zero_empty_conv_rows<kConvChannelsPerLane>(conv_state, has_init, cu, nseq, C, c0, lane);
    return;
  }
  const gdn_chunk ch = chunks[it.slot];
  if (ch.seq < 0 || c0 >= C) return;
  const int s = ch.seq;
  const int t_begin = ch.begin + kConvTokensPerWave * wave;
  const int n = min(kConvTokensPerWave, ch.end - t_begin);
  const bool owner = wave == 0 && (ch.flags & GDN_CHUNK_FIRST) != 0;   // reads and writes conv_state
  if (n <= 0) return;   // an owner's range is never empty: a first chunk starts its sequence

  // all token rows of this wave, requested before any use (rows past the
  // chunk's end re-read its last row; their outputs are dropped)
  typename A::Raw xr[kConvTokensPerWave];
#pragma unroll
  for (int u = 0; u < kConvTokensPerWave; ++u)
    xr[u] = A::load(x + (int64_t)(t_begin + min(u, n - 1)) * xs + c0);

  // window rows xe[t-3], xe[t-2], xe[t-1] for t = t_begin
  float h0[4], h1[4], h2[4];
  float* st = conv_state + ((int64_t)s * 3) * C + c0;
  if (owner) {
    const bool init = seq_flag(has_init, s);
    const float4 a = init ? *reinterpret_cast<const float4*>(st) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 bb = init ? *reinterpret_cast<const float4*>(st + C) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 c = init ? *reinterpret_cast<const float4*>(st + 2 * C) : make_float4(0.f, 0.f, 0.f, 0.f);
    h0[0] = a.x; h0[1] = a.y; h0[2] = a.z; h0[3] = a.w;
    h1[0] = bb.x; h1[1] = bb.y; h1[2] = bb.z; h1[3] = bb.w;
    h2[0] = c.x; h2[1] = c.y; h2[2] = c.z; h2[3] = c.w;
  } else {
    // the 3 rows before t_begin lie in the same sequence: a non-first chunk
    // starts at least 64 tokens in, and waves > 0 start 16 w tokens in
    A::unpack(A::load(x + (int64_t)(t_begin - 3) * xs + c0), h0);
    A::unpack(A::load(x + (int64_t)(t_begin - 2) * xs + c0), h1);
    A::unpack(A::load(x + (int64_t)(t_begin - 1) * xs + c0), h2);
  }
  // the stored rows, kept for sequences shorter than 3 tokens
  float o1[4], o2[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { o1[i] = h1[i]; o2[i] = h2[i]; }

  float w0[4], w1[4], w2[4], w3[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 wv = *reinterpret_cast<const float4*>(w + (int64_t)(c0 + i) * 4);
    w0[i] = wv.x; w1[i] = wv.y; w2[i] = wv.z; w3[i] = wv.w;
    b[i] = 0.f;
  }
  if (bias != nullptr) {
    const float4 bv = *reinterpret_cast<const float4*>(bias + c0);
    b[0] = bv.x; b[1] = bv.y; b[2] = bv.z; b[3] = bv.w;
  }

  const auto ry = buf_rsrc(y + (int64_t)t_begin * C, n * C * (int)sizeof(T));
#pragma unroll
  for (int u = 0; u < kConvTokensPerWave; ++u) {
    float xv[4], out[4];
    A::unpack(xr[u], xv);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float acc = b[i];
      acc = __builtin_fmaf(w0[i], h0[i], acc);
      acc = __builtin_fmaf(w1[i], h1[i], acc);
      acc = __builtin_fmaf(w2[i], h2[i], acc);
      acc = __builtin_fmaf(w3[i], xv[i], acc);
      out[i] = acc;
      h0[i] = h1[i]; h1[i] = h2[i]; h2[i] = xv[i];
    }
    A::store(ry, (u * C + c0) * (int)sizeof(T), out);
  }

  if (owner && write_state) {
    const int bos = cu[s], eos = cu[s + 1];
    const int len = eos - bos;
    // final rows r = 0..2 are xe[len-3+r]: x when that index is >= 0, else the
    // stored row 3 + (len-3+r).
    float r0[4], r1[4], r2[4], x0[4], x1[4];
    A::unpack(xr[0], x0);
    A::unpack(xr[1], x1);
    if (len >= 3) {
      A::unpack(A::load(x + (int64_t)(eos - 3) * xs + c0), r0);
      A::unpack(A::load(x + (int64_t)(eos - 2) * xs + c0), r1);
      A::unpack(A::load(x + (int64_t)(eos - 1) * xs + c0), r2);
    } else if (len == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) { r0[i] = o2[i]; r1[i] = x0[i]; r2[i] = x1[i]; }
    } else {  // len == 1 (a first chunk is never empty)
#pragma unroll
      for (int i = 0; i < 4; ++i) { r0[i] = o1[i]; r1[i] = o2[i]; r2[i] = x0[i]; }
    }
    *reinterpret_cast<float4*>(st) = make_float4(r0[0], r0[1], r0[2], r0[3]);
    *reinterpret_cast<float4*>(st + C) = make_float4(r1[0], r1[1], r1[2], r1[3]);
    *reinterpret_cast<float4*>(st + 2 * C) = make_float4(r2[0], r2[1], r2[2], r2[3]);
  }
}

// ---------------------------------------------------------------------------
// Conv and post-conv in one pass.  Each lane owns 8 adjacent channels (the
// post-conv kernel's layout: a 128-channel head is one 16-lane DPP row, and
// heads never straddle rows) and a wave takes kCPTokens consecutive tokens
// of one chunk.  Per token the lane forms y for its channels as conv_kernel
// does (same taps, same fused multiply-adds in the same order), rounds it
// to the activation dtype as the stored y is rounded, and then runs the
// post-conv kernel's lane function: SiLU, the head's squared norm in the
// documented order, the L2 scale on q and k.  So q, k and v are bitwise
// those of conv_kernel followed by postconv_kernel, and y never reaches
// memory.  conv_state is read and written as in conv_kernel (wave 0 of a
// sequence's first chunk, in place; its stored rows are read again at the
// end for sequences shorter than 3 tokens, before they are overwritten).
template <class T> struct CPShape;
template <> struct CPShape<uint16_t> { static constexpr int kTok = 16; };   // 4 waves per chunk
template <> struct CPShape<float> { static constexpr int kTok = 8; };       // 8 waves per chunk

// The 64-token chunk of slot j, derived from cu_seqlens (nseq <= 64) when no
// descriptor list is given.  f(s) = floor(cu[s] / 64) + s is strictly
// increasing (f(s+1) - f(s) = floor(cu[s+1]/64) - floor(cu[s]/64) + 1 >= 1),
// and sequence s owns slots f(s) .. f(s) + ceil(L_s / 64) - 1, which stay
// below f(s+1): floor(a/64) + ceil(L/64) <= floor((a+L)/64) + 1.  So slot j
// belongs to the last s with f(s) <= j (a prefix of the lanes, counted by a
// ballot), as chunk c = j - f(s) if c < ceil(L_s / 64); otherwise the slot
// is empty (seq = -1).  Slots number floor(N / 64) + nseq.  The chunks and
// their order within a sequence are those of the descriptor builder.
__device__ __forceinline__ gdn_chunk derive_chunk(const int32_t* __restrict__ cu, int nseq, int j, int lane) {
  const int b = lane < nseq ? cu[lane] : 0;
  const int e = lane < nseq ? cu[lane + 1] : 0;
  const int f = (b >> 6) + lane;
  const uint64_t below = __builtin_amdgcn_ballot_w64(lane < nseq && f <= j);
  const int s = __builtin_popcountll(below) - 1;   // f(0) = 0 <= j: s >= 0
  const int bs = __builtin_amdgcn_readlane(b, s), es = __builtin_amdgcn_readlane(e, s);
  const int c = j - __builtin_amdgcn_readlane(f, s);
  const int nc = (es - bs + 63) >> 6;
  gdn_chunk ch;
  ch.seq = c < nc ? s : -1;
  ch.begin = bs + 64 * c;
  ch.end = min(ch.begin + 64, es);
  ch.flags = (c == 0 ? GDN_CHUNK_FIRST : 0) | (c == nc - 1 ? GDN_CHUNK_LAST : 0);
  return ch;
}

template <class T>
__global__ __launch_bounds__(64 * 64 / CPShape<T>::kTok) void conv_post_kernel(
    const T* __restrict__ x, int64_t xs, const float* __restrict__ w, const float* __restrict__ bias,
    float* conv_state, const uint8_t* __restrict__ has_init, const int32_t* __restrict__ cu,
    const gdn_chunk* __restrict__ chunks, int nslots, int nseq, int C, int Hk, int Hv, float eps,
    int write_state, T* __restrict__ q, T* __restrict__ k, T* __restrict__ v) {
  constexpr int TPW = CPShape<T>::kTok;
  using AT = Act<T>;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const ConvItem it = conv_item(nslots, (C + 511) / 512);
  const int c0 = (it.group * 64 + lane) * 8;
  if (it.slot == nslots) {   // launched only when write_state
    if (wave == 0) zero_empty_conv_rows<8>(conv_state, has_init, cu, nseq, C, c0, lane);
    return;
  }
  const gdn_chunk ch = chunks != nullptr ? chunks[it.slot] : derive_chunk(cu, nseq, it.slot, lane);
  if (ch.seq < 0 || c0 >= C) return;   // whole 16-lane rows: C is a multiple of 128
  const int s = ch.seq;
  const int t_begin = ch.begin + TPW * wave;
  const int n = min(TPW, ch.end - t_begin);
  const bool owner = wave == 0 && (ch.flags & GDN_CHUNK_FIRST) != 0;
  if (n <= 0) return;

  // taps and bias, then the window rows, then the token rows (one in-order
  // counter: the first token waits only for what precedes it)
  float w0[8], w1[8], w2[8], w3[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 wv = *reinterpret_cast<const float4*>(w + (int64_t)(c0 + i) * 4);
    w0[i] = wv.x; w1[i] = wv.y; w2[i] = wv.z; w3[i] = wv.w;
    b[i] = 0.f;
  }
  if (bias != nullptr) {
    const float4 b0 = *reinterpret_cast<const float4*>(bias + c0);
    const float4 b1 = *reinterpret_cast<const float4*>(bias + c0 + 4);
    b[0] = b0.x; b[1] = b0.y; b[2] = b0.z; b[3] = b0.w; b[4] = b1.x; b[5] = b1.y; b[6] = b1.z; b[7] = b1.w;
  }
  float h0[8], h1[8], h2[8];
  float* st = conv_state + ((int64_t)s * 3) * C + c0;
  const bool init = owner && seq_flag(has_init, s);
  auto stored_row = [&](int r, float (&o)[8]) {
    const float4 a = init ? *reinterpret_cast<const float4*>(st + (int64_t)r * C) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 c = init ? *reinterpret_cast<const float4*>(st + (int64_t)r * C + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = c.x; o[5] = c.y; o[6] = c.z; o[7] = c.w;
  };
  if (owner) {
    stored_row(0, h0);
    stored_row(1, h1);
    stored_row(2, h2);
  } else {
    // the 3 rows before t_begin lie in the same sequence (a non-first chunk
    // starts 64 tokens in or more, a later wave TPW w tokens in)
    AT::load8(x + (int64_t)(t_begin - 3) * xs + c0, h0);
    AT::load8(x + (int64_t)(t_begin - 2) * xs + c0, h1);
    AT::load8(x + (int64_t)(t_begin - 1) * xs + c0, h2);
  }
  typename AT::Raw xr[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) xr[u] = AT::load_raw(x + (int64_t)(t_begin + min(u, n - 1)) * xs + c0);

  // this lane's output row of token t_begin, and the row stride
  const int qk = Hk * 128;
  const bool is_qk = c0 < 2 * qk;
  const int ors = is_qk ? qk : Hv * 128;
  T* op = c0 < qk ? q + (int64_t)t_begin * qk + c0
          : is_qk ? k + (int64_t)t_begin * qk + (c0 - qk)
                  : v + (int64_t)t_begin * ors + (c0 - 2 * qk);
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    float xv[8], yv[8], sv[8];
    AT::unpack(xr[u], xv);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float acc = b[i];
      acc = __builtin_fmaf(w0[i], h0[i], acc);
      acc = __builtin_fmaf(w1[i], h1[i], acc);
      acc = __builtin_fmaf(w2[i], h2[i], acc);
      acc = __builtin_fmaf(w3[i], xv[i], acc);
      h0[i] = h1[i]; h1[i] = h2[i]; h2[i] = xv[i];
      yv[i] = acc;
    }
    // y as stored (rounded to the activation dtype, two at a time)
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const uint32_t pk = pack_bf16x2(yv[i], yv[i + 1]);
        yv[i] = __uint_as_float(pk << 16);
        yv[i + 1] = __uint_as_float(pk & 0xffff0000u);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) sv[i] = silu<T>(yv[i]);
    // every lane takes part in the row reduction (DPP needs its partners)
    const float sum = head_sum_sq<T>(sv);
    if (u < n) {
      if (is_qk) {
        const float inv = l2_inv<T>(sum, eps);
#pragma unroll
        for (int i = 0; i < 8; ++i) sv[i] = sv[i] * inv;
      }
      AT::store8(op, sv);
    }
    op += ors;
  }

  if (owner && write_state) {
    const int len = cu[s + 1] - cu[s];
    const int eos = cu[s + 1];
    // final rows r = 0..2 are xe[len-3+r]: x when that index is >= 0, else
    // the stored row 3 + (len-3+r)
    float r0[8], r1[8], r2[8];
    if (len >= 3) {
      AT::load8(x + (int64_t)(eos - 3) * xs + c0, r0);
      AT::load8(x + (int64_t)(eos - 2) * xs + c0, r1);
      AT::load8(x + (int64_t)(eos - 1) * xs + c0, r2);
    } else {
      float o1[8], o2[8], x0[8], x1[8];
      stored_row(1, o1);
      stored_row(2, o2);
      AT::unpack(xr[0], x0);
      AT::unpack(xr[1], x1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (len == 2) { r0[i] = o2[i]; r1[i] = x0[i]; r2[i] = x1[i]; }
        else          { r0[i] = o1[i]; r1[i] = o2[i]; r2[i] = x0[i]; }   // len == 1
      }
    }
    auto put = [&](int r, const float (&o)[8]) {
      *reinterpret_cast<float4*>(st + (int64_t)r * C) = make_float4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<float4*>(st + (int64_t)r * C + 4) = make_float4(o[4], o[5], o[6], o[7]);
    };
    put(0, r0);
    put(1, r1);
    put(2, r2);
  }
}

}  // namespace

hipError_t launch_make_chunks(const int32_t* cu, int nseq, int chunk_len, gdn_chunk* out, int cap,
                              hipStream_t st) {
  hipLaunchKernelGGL(make_chunks_kernel, dim3(1), dim3(256), 0, st, cu, nseq, chunk_len, out, cap);
  return hipGetLastError();
}

hipError_t launch_conv_postconv(const void* x, int64_t xs, int act, const float* w, const float* bias,
                                float* conv_state, const uint8_t* has_init, const int32_t* cu,
                                const gdn_chunk* chunks, int nchunks, int nseq, int Hk, int Hv, float eps,
                                int write_state, void* q, void* k, void* v, hipStream_t st) {
  const int C = (2 * Hk + Hv) * 128;
  // (nchunks slots, descriptors or derived, and when the final rows are
  // written one more for the empty sequences) x channel groups, flattened
  // (see conv_item)
  const int64_t nblk = (int64_t)(nchunks + (write_state ? 1 : 0)) * ((C + 511) / 512);
  if (nblk == 0) return hipSuccess;
  if (nblk > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nblk);
  if (act == GDN_F32) {
    hipLaunchKernelGGL(conv_post_kernel<float>, grid, dim3(64 * 64 / CPShape<float>::kTok), 0, st,
                       static_cast<const float*>(x), xs, w, bias, conv_state, has_init, cu, chunks, nchunks, nseq,
                       C, Hk, Hv, eps, write_state, static_cast<float*>(q), static_cast<float*>(k),
                       static_cast<float*>(v));
  } else {
    hipLaunchKernelGGL(conv_post_kernel<uint16_t>, grid, dim3(64 * 64 / CPShape<uint16_t>::kTok), 0, st,
                       static_cast<const uint16_t*>(x), xs, w, bias, conv_state, has_init, cu, chunks, nchunks,
                       nseq, C, Hk, Hv, eps, write_state, static_cast<uint16_t*>(q), static_cast<uint16_t*>(k),
                       static_cast<uint16_t*>(v));
  }
  return hipGetLastError();
}

hipError_t launch_conv(const void* x, int64_t xs, int act, const float* w, const float* bias,
                       float* conv_state, const uint8_t* has_init, const int32_t* cu,
                       const gdn_chunk* chunks, int nchunks, int nseq, int C, int write_state, void* y,
                       hipStream_t st) {
  // one workgroup per chunk slot (and one more slot for the empty sequences
  // when the final rows are written) and channel group, flattened (see
  // conv_item)
  const int64_t nblk = (int64_t)(nchunks + (write_state ? 1 : 0)) *
                      ((C + kConvChannelsPerBlock - 1) / kConvChannelsPerBlock);
  if (nblk == 0) return hipSuccess;
  if (nblk > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nblk);
  if (act == GDN_F32) {
    hipLaunchKernelGGL(conv_kernel<float>, grid, dim3(kConvThreads), 0, st,
                       static_cast<const float*>(x), xs, w, bias, conv_state, has_init, cu, chunks,
                       nchunks, nseq, C, write_state, static_cast<float*>(y));
  } else {
    hipLaunchKernelGGL(conv_kernel<uint16_t>, grid, dim3(kConvThreads), 0, st,
                       static_cast<const uint16_t*>(x), xs, w, bias, conv_state, has_init, cu,
                       chunks, nchunks, nseq, C, write_state, static_cast<uint16_t*>(y));
  }
  return hipGetLastError();
}

}  // namespace gdn
