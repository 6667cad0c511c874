// Per-token gated delta-rule step (decode / speculative verify) and the
// layer-batched commit of a verify window (gfx950).
//
// "Strata pull request 3226": the verify forward runs the per-token step for
// T = 1..8 draft tokens with commit_state = false ("Problem and result");
// the commit later keeps n_keep tokens and recomputes the state by replaying
// them with the same layout and reduction order as the fused step, so the
// two are bitwise equal ("Summary" item 1); all layers commit in one launch
// instead of one launch per layer.
//
// Recurrence (gated delta rule), per token t of a sequence's window, with
// the dv x dk state S:
//   u = S k_t,   d_t = b_t (v_t - a_t u),   S <- a_t S + d_t k_t^T,
//   o_t = S q_t  (after the update).
//
// Evaluation.  The window is taken 16 tokens at a time.  Unrolling the
// recurrence over a block of n <= 16 tokens that enters with state S0, with
// L_t = sum_{s<=t} log a_s and gamma_t = exp(L_t):
//   the deltas d_t solve (I + A) D = R, A_ts = b_t exp(L_t - L_s) (k_t . k_s)
//   for s < t, R_t = b_t (v_t - gamma_t S0 k_t);
//   o_t = gamma_t S0 q_t + sum_{s<=t} exp(L_t - L_s) (q_t . k_s) d_s;
//   S_n = gamma_{n-1} S0 + sum_s exp(L_{n-1} - L_s) d_s k_s^T.
// Row t of D is exactly the per-token delta of token t, so this is the
// per-token recurrence reassociated: S0 is read once per block, the
// products S0 K^T, S0 Q^T, K K^T, Q K^T and the state update run on MFMA,
// and the n-step dependency between tokens is one 16x16 unit-lower-
// triangular inverse.  The kernel is then bound by reading (and, when
// committing, writing) the float32 state.
//
// Layout.  One workgroup of 2 waves per (sequence, v-head); wave w owns
// state rows 64 w .. 64 w + 63 as four 16-row blocks, held TRANSPOSED in
// MFMA accumulators (the prefill's layout).  At two waves per SIMD every
// workgroup of a 32-sequence x 32-head launch is resident at once, so all
// state reads are in flight together instead of in two rounds.  Each wave
// loads half of the block's K and Q rows and stages it in LDS (one barrier
// per block); fragments are read back from LDS where they are used, and
// each wave keeps its own scratch for the inverse.  The commit replays the
// kept tokens through the same function, so its state is bitwise equal to
// the state a committing step over those tokens writes.
#include "launch.hpp"
#include "mfma.hpp"

namespace gdn {

namespace {

constexpr int kStepWaves = 2;                  // waves per (sequence, v-head)
constexpr int kStepThreads = 64 * kStepWaves;
constexpr int kRB = 128 / 16 / kStepWaves;     // 16-row state blocks per wave
constexpr int kRows = 16 * kRB;                // state rows per wave
constexpr int kSlices = 4 / kStepWaves;        // 32-column K / Q slices each wave stages
constexpr int kWin = 16;     // tokens per block of a window
constexpr float kLog2e = 1.4426950408889634f;

// One wave's scratch for a block.
template <class T> struct WaveScratch {
  using E = typename Prec<T>::E;
  static constexpr int LDT = kWin + Prec<T>::PAD;  // rows of T = (I + A)^-1
  E Tm[kWin * LDT];
  float A[kWin][20];
  float W[4][64];           // log2-scaled L, gamma, beta, d of the block's tokens (entries
                            // past 16 are written by the other lanes and never read)
};

// The block's K and Q rows, shared by the workgroup's waves (each wave
// stages one 32-column slice), and every wave's scratch.
template <class T> struct alignas(16) StepSmem {
  using E = typename Prec<T>::E;
  static constexpr int LDK = 128 + Prec<T>::PAD;
  E K[kWin * LDK];
  E Q[kWin * LDK];
  WaveScratch<T> w[kStepWaves];
};

// S^T of rows v0 + 16 b + r16, b0 <= b < b1, in accumulator layout: tile
// cb holds S[v0 + 16 b + r16][16 cb + 4 kg + e].  rs spans the state, or
// nothing (all zeros) when there is no initial state, so the read is
// branch-free.  The row block's offset is wave-uniform and goes in the
// scalar offset, so every read takes one lane offset plus an immediate.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t state_rsrc(const float* base, bool init) {
  return buf_rsrc(base, init ? 128 * 128 * 4 : 0);
}
__device__ __forceinline__ void load_state_rows(__amdgpu_buffer_rsrc_t rs, int v0, int r16, int kg,
                                                f32x4 (&st)[kRB][8], int b0, int b1) {
#pragma unroll
  for (int b = b0; b < b1; ++b)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
      st[b][cb] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (r16 * 128 + 16 * cb + 4 * kg) * 4,
                                                       __builtin_amdgcn_readfirstlane((v0 + 16 * b) * 512), 0));
}

__device__ __forceinline__ void store_state(float* base, int v0, int r16, int kg, const f32x4 (&st)[kRB][8]) {
#pragma unroll
  for (int b = 0; b < kRB; ++b)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
      *reinterpret_cast<float4*>(base + (v0 + 16 * b + r16) * 128 + 16 * cb + 4 * kg) =
          make_float4(st[b][cb][0], st[b][cb][1], st[b][cb][2], st[b][cb][3]);
}

// This wave's state rows set to zero (an empty sequence without an initial
// state, when the final state is written).
__device__ __forceinline__ void store_zero_state(float* base, int v0, int r16, int kg) {
#pragma unroll
  for (int b = 0; b < kRB; ++b)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
      *reinterpret_cast<float4*>(base + (v0 + 16 * b + r16) * 128 + 16 * cb + 4 * kg) = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Token inputs of one block of a window, in registers: this wave's
// 32-column slice of the K and Q rows (staged to LDS for every wave), and
// what the wave alone reads.
template <class T, bool WITH_O> struct BlockIn {
  typename Prec<T>::F32 kf[kSlices], qf[kSlices];   // K, Q slice fragments (token r16)
  float vv[kRB][4];                     // V (token 4 kg + e, state row v0 + 16 b + r16)
  float gl, bl;                         // log a, beta of token `lane` (lanes < 16)
  int n;
  int64_t t0;
};

template <class T, bool WITH_O>
__device__ __forceinline__ void load_block(BlockIn<T, WITH_O>& in, int lane, int wave, const T* q,
                                           const T* k, const T* v, const float* g, const float* beta,
                                           int64_t t0, int n, int Hk, int Hv, int h, int kh, int v0) {
  using PR = Prec<T>;
  constexpr int ES = sizeof(typename PR::E);
  const int r16 = lane & 15, kg = lane >> 4;
  in.n = n;
  in.t0 = t0;
  const auto rg = buf_rsrc(g + t0 * Hv, n * Hv * 4);
  const auto rb = buf_rsrc(beta + t0 * Hv, n * Hv * 4);
  const int goff = ((lane & 15) * Hv + h) * 4;
  in.gl = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, goff, 0, 0));
  in.bl = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, goff, 0, 0));
  const auto rk = buf_rsrc(k + t0 * Hk * 128, n * Hk * 128 * ES);
  const auto rq = buf_rsrc(q + t0 * Hk * 128, n * Hk * 128 * ES);
  const auto rv = buf_rsrc(v + t0 * Hv * 128, n * Hv * 128 * ES);
#pragma unroll
  for (int i = 0; i < kSlices; ++i) {
    const int off = ((r16 * Hk + kh) * 128 + 32 * (kSlices * wave + i) + 4 * kg) * ES;
    in.kf[i] = PR::gfrag32(rk, off);
    if (WITH_O) in.qf[i] = PR::gfrag32(rq, off);
  }
#pragma unroll
  for (int b = 0; b < kRB; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e) in.vv[b][e] = PR::gload1(rv, (((4 * kg + e) * Hv + h) * 128 + v0 + 16 * b + r16) * ES);
}

// This wave's slices of the block's K and Q rows into the shared tiles.
template <class T, bool WITH_O>
__device__ __forceinline__ void stage_block(typename Prec<T>::E* Ks, typename Prec<T>::E* Qs,
                                            const BlockIn<T, WITH_O>& in, int wave, int lane) {
  using PR = Prec<T>;
  constexpr int LDK = StepSmem<T>::LDK;
  const int r16 = lane & 15, kg = lane >> 4;
#pragma unroll
  for (int i = 0; i < kSlices; ++i) {
    const int c = 32 * (kSlices * wave + i) + 4 * kg;
    PR::put_frag32(Ks + r16 * LDK + c, in.kf[i]);
    if (WITH_O) PR::put_frag32(Qs + r16 * LDK + c, in.qf[i]);
  }
}

struct NoMid {
  __device__ void operator()() const {}
};

// One block of a window: o of its tokens (WITH_O) and, when `advance`, the
// state moved past them.  Ks / Qs hold the block's K and Q rows (16 x 128,
// row stride LDK); `wave` selects the state rows kRows wave .. kRows wave +
// kRows - 1.  K and Q fragments are read from the tiles where they are
// used, so they are not held in registers next to the state.  `mid` runs
// between the token side (gate vectors, K K^T, Q K^T, A, T) and the state
// side, which reads st: a caller issues the rest of its state reads there.
template <class T, bool WITH_O, class Mid = NoMid>
__device__ __forceinline__ void run_block(WaveScratch<T>& ws, const typename Prec<T>::E* Ks,
                                          const typename Prec<T>::E* Qs, int wave, int lane,
                                          f32x4 (&st)[kRB][8], const BlockIn<T, WITH_O>& in, T* o,
                                          int Hv, int h, bool advance, Mid mid = Mid{}) {
  using PR = Prec<T>;
  using E = typename PR::E;
  constexpr int ES = sizeof(E);
  constexpr int LDK = StepSmem<T>::LDK, LDT = WaveScratch<T>::LDT;
  const int r16 = lane & 15, kg = lane >> 4;
  const int v0 = kRows * wave;
  const int n = in.n;
  E* Tm = ws.Tm;
  float* Wl = &ws.W[0][0];

  // gate vectors: lane t < 16 holds token t (zero past the block's end);
  // every lane writes its slot, so the loads are never sunk into a branch
  {
    const float gl = lane < kWin ? in.gl : 0.f;
    const float L = wave_prefix_sum(gl) * kLog2e;
    const float Llast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(L), n - 1));
    Wl[lane] = L;
    Wl[64 + lane] = __builtin_amdgcn_exp2f(L);
    Wl[128 + lane] = in.bl;
    Wl[192 + lane] = lane < n ? __builtin_amdgcn_exp2f(Llast - L) : 0.f;
  }

  // transposed token products: lane (r16, kg) element e holds k_j . k_i
  // and k_j . q_i for i = r16, j = 4 kg + e
  f32x4 kk = zero4(), qk = zero4();
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const auto kf = PR::lds32(Ks, LDK, r16, 32 * t, kg);
    kk = PR::mma32(kf, kf, kk);
    if (WITH_O) qk = PR::mma32(kf, PR::lds32(Qs, LDK, r16, 32 * t, kg), qk);
  }

  // A (row i = r16, columns j = 4 kg + e) to LDS, P kept as the B operand
  // of U^T P^T
  float pv[4];
  {
    const float Li = Wl[r16], bi = Wl[128 + r16];
    const float4 Lj = *reinterpret_cast<const float4*>(&Wl[4 * kg]);
    const float lj[4] = {Lj.x, Lj.y, Lj.z, Lj.w};
    float av[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * kg + e;
      const float dec = j <= r16 ? __builtin_amdgcn_exp2f(Li - lj[e]) : 0.f;
      av[e] = j < r16 ? bi * dec * kk[e] : 0.f;
      pv[e] = dec * qk[e];
    }
    *reinterpret_cast<float4*>(&ws.A[r16][4 * kg]) = make_float4(av[0], av[1], av[2], av[3]);
  }

  // T = (I + A)^-1 by forward substitution: lane (c, q) = (lane / 4,
  // lane % 4) owns rows q, q+4, q+8, q+12 of column c; the four lanes of a
  // column form a DPP quad and x_j, once final, is broadcast from the lane
  // owning row j.  Terms with j >= i vanish: A is strictly lower
  // triangular.
  {
    const int c = lane >> 2, qd = lane & 3;
    float x[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) x[m] = (qd + 4 * m == c) ? 1.f : 0.f;
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      float a4[4][4];   // A[qd + 4 m][4 j4 .. 4 j4 + 3]
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float4 t = *reinterpret_cast<const float4*>(&ws.A[qd + 4 * m][4 * j4]);
        a4[m][0] = t.x; a4[m][1] = t.y; a4[m][2] = t.z; a4[m][3] = t.w;
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const float xj = quad_bcast(x[j4], jj);
#pragma unroll
        for (int m = 0; m < 4; ++m) x[m] = __builtin_fmaf(-a4[m][jj], xj, x[m]);
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) PR::put(&Tm[(qd + 4 * m) * LDT + c], x[m]);
  }
  const auto tf = PR::lds16(Tm, LDT, r16, 0, kg);
  // everything above is the token side; a caller may issue work here that
  // must come after it in program order (the rest of its state reads)
  mid();

  // Z = K S0^T (rows: tokens) and (Q S0^T)^T (rows: state rows).  With bf16
  // operands the float32 state enters as hi + lo (two products each): one
  // bf16 rounding of S0 here, taken at every call, costs the outputs and the
  // deltas (v - a S0 k cancels as the rule converges) about 2^-9 of |S0|
  // per token, which a chain of one-token decode steps never averages out.
  f32x4 z[kRB], qt[kRB];
#pragma unroll
  for (int b = 0; b < kRB; ++b) { z[b] = zero4(); qt[b] = zero4(); }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const auto kf = PR::lds32(Ks, LDK, r16, 32 * t, kg);
    typename PR::F32 qf;
    if (WITH_O) qf = PR::lds32(Qs, LDK, r16, 32 * t, kg);
#pragma unroll
    for (int b = 0; b < kRB; ++b) {
      const auto bs = PR::reg32(st[b][2 * t], st[b][2 * t + 1]);
      z[b] = PR::mma32(kf, bs, z[b]);
      if (WITH_O) qt[b] = PR::mma32(bs, qf, qt[b]);
      if constexpr (PR::kSplitState) {
        const auto bl = PR::reg32_lo(st[b][2 * t], st[b][2 * t + 1], bs);
        z[b] = PR::mma32(kf, bl, z[b]);
        if (WITH_O) qt[b] = PR::mma32(bl, qf, qt[b]);
      }
    }
  }

  // R = diag(beta) (V - diag(gamma) Z), D = T R (rows: tokens)
  const float4 ga = *reinterpret_cast<const float4*>(&Wl[64 + 4 * kg]);
  const float4 be = *reinterpret_cast<const float4*>(&Wl[128 + 4 * kg]);
  const float4 dd = *reinterpret_cast<const float4*>(&Wl[192 + 4 * kg]);
  const float gam[4] = {ga.x, ga.y, ga.z, ga.w}, bet[4] = {be.x, be.y, be.z, be.w};
  const float dec4[4] = {dd.x, dd.y, dd.z, dd.w};
  f32x4 dl[kRB];
#pragma unroll
  for (int b = 0; b < kRB; ++b) {
    f32x4 rr;
#pragma unroll
    for (int e = 0; e < 4; ++e) rr[e] = bet[e] * (in.vv[b][e] - gam[e] * z[b][e]);
    dl[b] = PR::mma16(tf, PR::reg16(rr), zero4());
  }

  // O^T = (Q S0^T)^T diag(gamma) + D^T P^T; lane: token r16, state rows
  // v0 + 16 b + 4 kg .. +3.  The 16-wide product is formed on its own
  // accumulator: an accumulator is never carried from a 16x16x32 MFMA into
  // a 16x16x16 one (the hardware needs wait states between the two shapes
  // that the compiler does not insert).
  if (WITH_O) {
    const auto ro = buf_rsrc(o + in.t0 * Hv * 128, n * Hv * 128 * ES);
    const auto pf = PR::reg16(f32x4{pv[0], pv[1], pv[2], pv[3]});
    const float gt = Wl[64 + r16];
#pragma unroll
    for (int b = 0; b < kRB; ++b) {
      const f32x4 pu = PR::mma16(PR::reg16(dl[b]), pf, zero4());
      float ov[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = gt * qt[b][e] + pu[e];
      PR::gstore4(ro, ((r16 * Hv + h) * 128 + v0 + 16 * b + 4 * kg) * ES, ov);
    }
  }

  // S^T <- gamma_{n-1} S^T + K^T diag(d) D
  if (advance) {
    const float gl = __builtin_amdgcn_exp2f(Wl[n - 1]);
    typename PR::F16 du[kRB];
#pragma unroll
    for (int b = 0; b < kRB; ++b) {
      f32x4 t;
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = dl[b][e] * dec4[e];
      du[b] = PR::reg16(t);
    }
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const auto kt = PR::ldsT16(Ks, LDK, 16 * cb, lane);
#pragma unroll
      for (int b = 0; b < kRB; ++b) {
        f32x4 acc;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = gl * st[b][cb][e];
        st[b][cb] = PR::mma16(kt, du[b], acc);
      }
    }
  }
}

// Runs tokens [bos, bos + len) of one (sequence, v-head) through this
// wave's kRows state rows in st; `in` holds the first block's token inputs,
// already requested by the caller (with the state, or with its first part:
// `mid` is the first block's, where the caller requests the rest), so a
// unit's loads are in flight together.  WITH_O writes o; the state is
// advanced over every block except, when !write_state, the last.
template <class T, bool WITH_O, class Mid = NoMid>
__device__ __forceinline__ void run_window(StepSmem<T>& sm, int wave, int lane, f32x4 (&st)[kRB][8],
                                           BlockIn<T, WITH_O>& in, const T* q, const T* k,
                                           const T* v, const float* g, const float* beta, T* o,
                                           int bos, int len, int Hk, int Hv, int h, int kh,
                                           bool write_state, Mid mid = Mid{}) {
  const int v0 = kRows * wave;
  stage_block<T, WITH_O>(sm.K, sm.Q, in, wave, lane);
  __syncthreads();
  run_block<T, WITH_O>(sm.w[wave], sm.K, sm.Q, wave, lane, st, in, o, Hv, h, write_state || len > kWin, mid);
  for (int c0 = kWin; c0 < len; c0 += kWin) {
    load_block<T, WITH_O>(in, lane, wave, q, k, v, g, beta, (int64_t)bos + c0, min(kWin, len - c0), Hk,
                          Hv, h, kh, v0);
    __syncthreads();   // every wave is done with the previous block's rows
    stage_block<T, WITH_O>(sm.K, sm.Q, in, wave, lane);
    __syncthreads();
    run_block<T, WITH_O>(sm.w[wave], sm.K, sm.Q, wave, lane, st, in, o, Hv, h,
                         write_state || c0 + kWin < len);
  }
}

// One workgroup per (sequence, v-head).  The state is read right after the
// first block's token inputs; without an initial state the reads go through
// an empty buffer range and return zeros.  The flag comes from a scalar load
// issued with cu's, so no vector load waits on it.
template <class T>
__global__ __launch_bounds__(kStepThreads, sizeof(T) == 2 ? 2 : 1) void step_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
    int Hk, int Hv, float* state, const uint8_t* __restrict__ has_init, T* __restrict__ o,
    int commit_state) {
  __shared__ StepSmem<T> sm;
  const int s = blockIdx.x / Hv;
  const int h = blockIdx.x % Hv;
  const int kh = h / (Hv / Hk);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, kg = lane >> 4;
  const int v0 = kRows * wave;
  const int bos = cu[s], len = cu[s + 1] - bos;
  const bool init = seq_flag(has_init, s);   // requested with cu (both scalar)
  float* base = state + ((int64_t)s * Hv + h) * (128 * 128);
  if (len <= 0) {
    // no tokens: the final state is the initial one, zero without a flag
    if (commit_state && !init) store_zero_state(base, v0, r16, kg);
    return;
  }
  BlockIn<T, true> in;
  load_block<T, true>(in, lane, wave, q, k, v, g, beta, bos, min(kWin, len), Hk, Hv, h, kh, v0);
  // The state (zeros without an initial state) is requested in two halves,
  // the second between the first block's token side and its state side:
  // with every workgroup asking for its state at once, issuing the reads is
  // paced by the memory system, and a wave runs nothing placed after a
  // read before that read is issued.
  f32x4 st[kRB][8];
  const auto rs = state_rsrc(base, init);
  load_state_rows(rs, v0, r16, kg, st, 0, kRB / 2);
  // the first half is issued before anything uses a read: the scheduler
  // would otherwise hoist the block's conversions between the reads, and
  // the in-order wait for them would hold back the remaining reads
  __builtin_amdgcn_sched_barrier(0);
  run_window<T, true>(sm, wave, lane, st, in, q, k, v, g, beta, o, bos, len, Hk, Hv, h, kh,
                      commit_state != 0, [&]() __attribute__((always_inline)) {
                        __builtin_amdgcn_sched_barrier(0);
                        load_state_rows(rs, v0, r16, kg, st, kRB / 2, kRB);
                        __builtin_amdgcn_sched_barrier(0);
                      });
  if (commit_state) store_state(base, v0, r16, kg, st);
}

// ---------------------------------------------------------------------------
// Fused decode / verify step: the causal conv over the window's x rows, SiLU,
// the q / k L2 norm and the step in one launch, with y, q, k and v kept on
// chip.  One workgroup per (sequence, k-head) holds the G = Hv / Hk v-heads
// that read that k-head (2 waves each), so it owns every channel it reads:
// q and k of the k-head and v of its v-heads.  Its optional in-place
// conv_state update therefore cannot race with another workgroup.
//
// Per block of up to 16 tokens: the block's conv input rows (and, for the
// first block, the stored conv rows) are staged into LDS; phase A computes
// y from them, rounds it to the activation dtype (as the stored y would
// be), applies the post-conv lane function (as the post-conv kernel does)
// and writes q, k and each v-head's v, rounded again, into LDS tiles; phase
// B runs the step's block function on fragments read from those tiles.
// Every value is what the three separate launches produce, so the results
// are bitwise equal to them.
//
// Load order.  One in-order counter covers a wave's vector memory
// operations, so the first block's staged rows, the conv weights and the
// gates are requested before the state: phase A then waits only for them
// while the state is still arriving.  With every workgroup asking for its
// state at once, issuing the state reads is itself paced by the memory
// system, and a wave runs nothing placed after a read before that read is
// issued; so half of the state is requested before phase A and half after
// it, and phase A issues no global stores (the k and v kept for a commit
// are copied out of the tiles after phase B).
template <class T, int G> struct alignas(16) FusedSmem {
  using E = typename Prec<T>::E;
  static constexpr int LDK = 128 + Prec<T>::PAD;
  static constexpr int CH = (2 + G) * 128;                // q, k and G v heads
  static constexpr int NT = kStepThreads * G;
  static constexpr int PE = 16 / sizeof(E);                // elements per 16-byte piece
  static constexpr int XP = (kWin + 3) * CH / PE;          // pieces of the conv input rows
  static constexpr int XI = (XP + NT - 1) / NT;            // ... per thread
  static constexpr int CP = 3 * CH / 4;                    // pieces of the stored rows
  static constexpr int CI = (CP + NT - 1) / NT;
  static constexpr int WI = (CH + NT - 1) / NT;            // conv taps: one piece per channel
  static constexpr int BI = (CH / 4 + NT - 1) / NT;        // bias: four channels per piece
  WaveScratch<T> w[kStepWaves * G];
  E Qs[kWin * LDK];
  E Ks[kWin * LDK];
  E Vs[G][kWin * LDK];
  // conv input rows, row r = block token r - 3, [kWin + 3][CH] row-major
  // (padded to whole pieces per thread); stored rows [3][CH]
  alignas(16) E Xs[XI * NT * PE];
  alignas(16) float Cs[CI * NT * 4];
  alignas(16) float Wt[4][WI * NT];    // taps, transposed: [tap][channel]
  alignas(16) float Bt[BI * NT * 4];   // [CH] bias (zeros without one)
};

template <class T, int G>
__global__ __launch_bounds__(kStepThreads * G, sizeof(T) == 2 ? 2 : 1) void fused_kernel(
    const T* __restrict__ x, int64_t xs, const float* __restrict__ w, const float* __restrict__ bias,
    float* conv_state, const int32_t* __restrict__ cu, int Hk, int Hv, float eps,
    const float* __restrict__ g, const float* __restrict__ beta, float* state,
    const uint8_t* __restrict__ has_init, T* __restrict__ o, T* __restrict__ k_out, T* __restrict__ v_out,
    int write_conv_state, int commit_state) {
  using PR = Prec<T>;
  using E = typename PR::E;
  using SM = FusedSmem<T, G>;
  constexpr int LDK = SM::LDK, CH = SM::CH, NT = SM::NT, PE = SM::PE;
  constexpr int ES = sizeof(E);
  constexpr int NW = kStepWaves * G;                      // waves
  __shared__ SM sm;
  const int s = blockIdx.x / Hk, kh = blockIdx.x % Hk;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / kStepWaves, wl = wave % kStepWaves;
  const int r16 = lane & 15, kg = lane >> 4;
  const int v0 = kRows * wl;
  const int h = kh * G + grp;
  const int C = (2 * Hk + Hv) * 128;
  const int bos = cu[s], len = cu[s + 1] - bos;
  const bool init = seq_flag(has_init, s);   // requested with cu (both scalar)
  float* cs = conv_state + (int64_t)s * 3 * C;
  // global channel of channel c (0 .. CH-1) of this workgroup: slots 0, 1
  // are the q and k heads of k-head kh, slots 2.. its v heads
  auto chan = [=](int c) {
    const int hs = c >> 7;
    const int qk = hs * Hk + kh, vh = 2 * Hk + kh * G + hs - 2;   // both formed, one kept
    return (hs < 2 ? qk : vh) * 128 + (c & 127);
  };
  if (len <= 0) {
    // no tokens: the final states are the initial ones, zero without a flag
    if (!init) {
      if (commit_state) store_zero_state(state + ((int64_t)s * Hv + h) * (128 * 128), v0, r16, kg);
      if (write_conv_state && wave == 0 && (lane >> 4) < 2 + G) {
        const int cg = chan((lane >> 4) * 128 + 8 * (lane & 15));
#pragma unroll
        for (int r = 0; r < 3; ++r) {
          float* p = cs + (int64_t)r * C + cg;
          *reinterpret_cast<float4*>(p) = make_float4(0.f, 0.f, 0.f, 0.f);
          *reinterpret_cast<float4*>(p + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
    return;
  }

  // staged pieces: x rows of block c0 (rows before the sequence read as
  // zeros), and the stored rows for the first block (zeros without an
  // initial state); padding pieces read out of range (zeros)
  u32x4 px[SM::XI], pc[SM::CI], pw[SM::WI], pb[SM::BI];
  auto issue_stage = [&](int c0, int n) {
    const int hb = c0 > 0 ? 3 : 0;   // rows of the previous block inside the range
    const auto rx = buf_rsrc(x + ((int64_t)bos + c0 - hb) * xs, (n + hb) * (int)xs * ES);
#pragma unroll
    for (int i = 0; i < SM::XI; ++i) {
      const int p = tid + NT * i, pp = min(p, SM::XP - 1);
      const int row = pp / (CH / PE), c = (pp % (CH / PE)) * PE;
      const int off = ((row - 3 + hb) * (int)xs + chan(c)) * ES;
      px[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, p < SM::XP ? off : INT_MIN, 0, 0);
    }
    if (c0 == 0) {
      const auto rc = buf_rsrc(cs, init ? 3 * C * 4 : 0);
#pragma unroll
      for (int i = 0; i < SM::CI; ++i) {
        const int p = tid + NT * i, pp = min(p, SM::CP - 1);
        const int row = pp / (CH / 4), c = (pp % (CH / 4)) * 4;
        const int off = (row * C + chan(c)) * 4;
        pc[i] = __builtin_amdgcn_raw_buffer_load_b128(rc, p < SM::CP ? off : INT_MIN, 0, 0);
      }
      const auto rw = buf_rsrc(w, C * 16);
#pragma unroll
      for (int i = 0; i < SM::WI; ++i) {
        const int p = tid + NT * i, off = chan(min(p, CH - 1)) * 16;
        pw[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, p < CH ? off : INT_MIN, 0, 0);
      }
      const auto rb = buf_rsrc(bias, bias != nullptr ? C * 4 : 0);
#pragma unroll
      for (int i = 0; i < SM::BI; ++i) {
        const int p = tid + NT * i, off = chan(4 * min(p, CH / 4 - 1)) * 4;
        pb[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, p < CH / 4 ? off : INT_MIN, 0, 0);
      }
    }
  };
  auto write_stage = [&](int c0) {
#pragma unroll
    for (int i = 0; i < SM::XI; ++i) reinterpret_cast<u32x4*>(sm.Xs)[tid + NT * i] = px[i];
    if (c0 == 0) {
#pragma unroll
      for (int i = 0; i < SM::CI; ++i) reinterpret_cast<u32x4*>(sm.Cs)[tid + NT * i] = pc[i];
      // (the whole piece is reinterpreted, then indexed: a bit cast of one
      // vector element compiled to a read of element 0 for every index)
#pragma unroll
      for (int i = 0; i < SM::WI; ++i) {
        const f32x4 wv = __builtin_bit_cast(f32x4, pw[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j) sm.Wt[j][tid + NT * i] = wv[j];
      }
#pragma unroll
      for (int i = 0; i < SM::BI; ++i) reinterpret_cast<u32x4*>(sm.Bt)[tid + NT * i] = pb[i];
    }
  };

  // phase A lanes: 16-lane row hs = lane / 16 is one head (q, k, v...),
  // lane jl owns its channels 8 jl .. 8 jl + 7; wave wv takes tokens
  // wv, wv + NW, ...  Rows past the 2 + G heads idle.
  const int hs = lane >> 4, jl = lane & 15;
  const bool a_row = hs < 2 + G;

  int n = min(kWin, len);
  issue_stage(0, n);
  float gl, bl;
  auto load_gates = [&](int c0, int nn) {
    const auto rg = buf_rsrc(g + ((int64_t)bos + c0) * Hv, nn * Hv * 4);
    const auto rbt = buf_rsrc(beta + ((int64_t)bos + c0) * Hv, nn * Hv * 4);
    const int goff = ((lane & 15) * Hv + h) * 4;
    gl = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, goff, 0, 0));
    bl = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rbt, goff, 0, 0));
  };
  load_gates(0, n);

  // The state is requested in two halves, the second after the first
  // block's conv and post-conv phase: issuing the reads is paced by the
  // memory system (every workgroup asks for its state at once), and a
  // wave runs nothing placed after a read before that read is issued.
  f32x4 st[kRB][8];
  float* base = state + ((int64_t)s * Hv + h) * (128 * 128);
  const auto rs = state_rsrc(base, init);
  load_state_rows(rs, v0, r16, kg, st, 0, kRB / 2);
  write_stage(0);   // waits for the staged pieces only

  // one block of the window; the first is peeled (a compile-time flag), so
  // the second half of the state reads is issued on every path through it
  // and no merged wait count covers it early
  auto one_block = [&](int c0, auto first_c) __attribute__((always_inline)) {
    constexpr bool first = decltype(first_c)::value;
    n = min(kWin, len - c0);
    if constexpr (!first) {
      issue_stage(c0, n);
      load_gates(c0, n);
      write_stage(c0);
    }
    __syncthreads();

    // phase A
    if (a_row) {
      const int ca = hs * 128 + 8 * jl;   // channel within the workgroup
      for (int t = wave; t < kWin; t += NW) {
        float out[8];
        if (t < n) {
          // y = bias + w_0 x_{t-3} + ... + w_3 x_t, one tap at a time (the
          // conv kernel's order): staging row t + r holds x_{t-3+r}
          float yv[8];
          {
            const float4 b0 = *reinterpret_cast<const float4*>(&sm.Bt[ca]);
            const float4 b1 = *reinterpret_cast<const float4*>(&sm.Bt[ca + 4]);
            yv[0] = b0.x; yv[1] = b0.y; yv[2] = b0.z; yv[3] = b0.w;
            yv[4] = b1.x; yv[5] = b1.y; yv[6] = b1.z; yv[7] = b1.w;
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int sr = t + r;
            float xr[8];
            if (first && sr < 3) {
              const float4 a = *reinterpret_cast<const float4*>(&sm.Cs[sr * CH + ca]);
              const float4 b4 = *reinterpret_cast<const float4*>(&sm.Cs[sr * CH + ca + 4]);
              xr[0] = a.x; xr[1] = a.y; xr[2] = a.z; xr[3] = a.w;
              xr[4] = b4.x; xr[5] = b4.y; xr[6] = b4.z; xr[7] = b4.w;
            } else {
              Act<T>::load8(&sm.Xs[sr * CH + ca], xr);
            }
            const float4 w0 = *reinterpret_cast<const float4*>(&sm.Wt[r][ca]);
            const float4 w1 = *reinterpret_cast<const float4*>(&sm.Wt[r][ca + 4]);
            const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int i = 0; i < 8; ++i) yv[i] = __builtin_fmaf(wv[i], xr[i], yv[i]);
            __builtin_amdgcn_sched_barrier(0);
          }
          // y as stored in the activation dtype
          typename Act<T>::Raw ry;
          {
            E tmp[8];
            Act<T>::store8(tmp, yv);
            ry = Act<T>::load_raw(tmp);
          }
          Act<T>::unpack(ry, yv);
          postconv_lane<T>(yv, hs < 2, eps, out);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) out[i] = 0.f;
        }
        E* dst = hs == 0 ? sm.Qs : hs == 1 ? sm.Ks : sm.Vs[hs - 2];
        Act<T>::store8(dst + t * LDK + 8 * jl, out);
      }
    }
    if constexpr (first) load_state_rows(rs, v0, r16, kg, st, kRB / 2, kRB);
    __syncthreads();

    // phase B: the step's block on this v-head group's waves
    BlockIn<T, true> in;   // K and Q are read from the tiles
    in.n = n;
    in.t0 = (int64_t)bos + c0;
    in.gl = gl;
    in.bl = bl;
#pragma unroll
    for (int b = 0; b < kRB; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) in.vv[b][e] = PR::to_f32(sm.Vs[grp][(4 * kg + e) * LDK + v0 + 16 * b + r16]);
    run_block<T, true>(sm.w[wave], sm.Ks, sm.Qs, wl, lane, st, in, o, Hv, h,
                       commit_state != 0 || c0 + kWin < len);
    // the normalised k and the v kept for a later commit's replay, copied
    // from the tiles (the values phase A wrote there) once the block's
    // state reads are out of the way
    if (k_out != nullptr || v_out != nullptr) {
      constexpr int PR16 = 128 / PE;              // 16-byte pieces per row
      for (int i = tid; i < (1 + G) * n * PR16; i += NT) {
        const int hh = i / (n * PR16), rem = i % (n * PR16), t = rem / PR16, c = (rem % PR16) * PE;
        const int64_t tg = (int64_t)bos + c0 + t;
        if (hh == 0) {
          if (k_out != nullptr)
            *reinterpret_cast<uint4*>(k_out + (tg * Hk + kh) * 128 + c) =
                *reinterpret_cast<const uint4*>(&sm.Ks[t * LDK + c]);
        } else if (v_out != nullptr) {
          *reinterpret_cast<uint4*>(v_out + (tg * Hv + kh * G + hh - 1) * 128 + c) =
              *reinterpret_cast<const uint4*>(&sm.Vs[hh - 1][t * LDK + c]);
        }
      }
    }
    __syncthreads();
  };
  one_block(0, std::true_type{});
  for (int c0 = kWin; c0 < len; c0 += kWin) one_block(c0, std::false_type{});
  if (commit_state) store_state(base, v0, r16, kg, st);

  // conv_state <- the last 3 rows of [stored rows ; x window] for this
  // workgroup's channels, read from LDS: the last block's staged x rows
  // (row r = block token r - 3) hold every final token, and the staged
  // stored rows (zeros without an initial state) the rows before the
  // sequence when it has fewer than 3 tokens.
  if (write_conv_state && a_row && wave == 0) {
    const int cg = chan(hs * 128 + 8 * jl);
    const int ca = hs * 128 + 8 * jl;
    const int c_last = (len - 1) / kWin * kWin;   // first token of the last block
    float v8[3][8];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const int tr = len - 3 + r;   // token index of final row r
      if (tr >= 0) {
        Act<T>::load8(&sm.Xs[(tr - c_last + 3) * CH + ca], v8[r]);
      } else {
        const float4 a = *reinterpret_cast<const float4*>(&sm.Cs[(3 + tr) * CH + ca]);
        const float4 b4 = *reinterpret_cast<const float4*>(&sm.Cs[(3 + tr) * CH + ca + 4]);
        v8[r][0] = a.x; v8[r][1] = a.y; v8[r][2] = a.z; v8[r][3] = a.w;
        v8[r][4] = b4.x; v8[r][5] = b4.y; v8[r][6] = b4.z; v8[r][7] = b4.w;
      }
    }
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      float* p = cs + (int64_t)r * C + cg;
      *reinterpret_cast<float4*>(p) = make_float4(v8[r][0], v8[r][1], v8[r][2], v8[r][3]);
      *reinterpret_cast<float4*>(p + 4) = make_float4(v8[r][4], v8[r][5], v8[r][6], v8[r][7]);
    }
  }
}

// One launch for all layers: block b covers (layer, sequence, role); roles
// 0..Hv-1 replay the state of v-head `role`, roles Hv.. shift the conv rows
// of one group of 8 * kStepThreads channels.  A block whose sequence keeps no token exits
// before touching memory.
template <class T>
__global__ __launch_bounds__(kStepThreads, 1) void commit_kernel(
    const gdn_layer_io* __restrict__ layers, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ n_keep, const uint8_t* __restrict__ has_init, int nseq, int C,
    int Hk, int Hv, int roles) {
  __shared__ StepSmem<T> sm;
  const int b = blockIdx.x;
  const int role = b % roles;
  const int s = (b / roles) % nseq;
  const int layer = b / (roles * nseq);
  const int n = n_keep[s];
  const int bos = cu[s];
  const bool init = seq_flag(has_init, s);   // the three scalar reads overlap
  if (n <= 0) return;
  const gdn_layer_io io = layers[layer];
  if (role < Hv) {
    const int h = role;
    const int kh = h / (Hv / Hk);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r16 = lane & 15, kg = lane >> 4;
    float* base = io.state + ((int64_t)s * Hv + h) * (128 * 128);
    f32x4 st[kRB][8];
    BlockIn<T, false> in;
    load_block<T, false>(in, lane, wave, nullptr, static_cast<const T*>(io.k), static_cast<const T*>(io.v), io.g,
                         io.beta, bos, min(kWin, n), Hk, Hv, h, kh, kRows * wave);
    // the state in two halves around the first block's token side, as in
    // the step
    const auto rs = state_rsrc(base, init);
    load_state_rows(rs, kRows * wave, r16, kg, st, 0, kRB / 2);
    __builtin_amdgcn_sched_barrier(0);   // the first half issued before any use
    run_window<T, false>(sm, wave, lane, st, in, nullptr, static_cast<const T*>(io.k),
                         static_cast<const T*>(io.v), io.g, io.beta, nullptr, bos, n, Hk, Hv, h, kh,
                         true, [&]() __attribute__((always_inline)) {
                           __builtin_amdgcn_sched_barrier(0);
                           load_state_rows(rs, kRows * wave, r16, kg, st, kRB / 2, kRB);
                           __builtin_amdgcn_sched_barrier(0);
                         });
    store_state(base, kRows * wave, r16, kg, st);
  } else {
    const int c0 = ((role - Hv) * kStepThreads + threadIdx.x) * 8;
    if (c0 >= C) return;
    const T* x = static_cast<const T*>(io.x);
    float* st = io.conv_state + ((int64_t)s * 3) * C + c0;
    float rows[3][8];
    // the stored rows (oldest first) followed by the kept tokens; keep the
    // last three
    if (n >= 3) {
#pragma unroll
      for (int r = 0; r < 3; ++r) Act<T>::load8(x + (int64_t)(bos + n - 3 + r) * io.x_row_stride + c0, rows[r]);
    } else {
      float old[3][8];
#pragma unroll
      for (int r = 0; r < 3; ++r) {
#pragma unroll
        for (int i = 0; i < 8; i += 4) {
          float4 a = init ? *reinterpret_cast<const float4*>(st + (int64_t)r * C + i)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
          old[r][i] = a.x; old[r][i + 1] = a.y; old[r][i + 2] = a.z; old[r][i + 3] = a.w;
        }
      }
      float x0[8], x1[8];
      Act<T>::load8(x + (int64_t)bos * io.x_row_stride + c0, x0);
      if (n == 2) Act<T>::load8(x + (int64_t)(bos + 1) * io.x_row_stride + c0, x1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (n == 1) { rows[0][i] = old[1][i]; rows[1][i] = old[2][i]; rows[2][i] = x0[i]; }
        else        { rows[0][i] = old[2][i]; rows[1][i] = x0[i];     rows[2][i] = x1[i]; }
      }
    }
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
      for (int i = 0; i < 8; i += 4)
        *reinterpret_cast<float4*>(st + (int64_t)r * C + i) =
            make_float4(rows[r][i], rows[r][i + 1], rows[r][i + 2], rows[r][i + 3]);
  }
}

}  // namespace

hipError_t launch_step(const void* q, const void* k, const void* v, int act, const float* g,
                       const float* beta, const int32_t* cu, int nseq, int Hk, int Hv,
                       float* state, const uint8_t* has_init, void* o, int commit_state,
                       hipStream_t st) {
  const dim3 grid(nseq * Hv);
  if (act == GDN_F32) {
    hipLaunchKernelGGL(step_kernel<float>, grid, dim3(kStepThreads), 0, st,
                       static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), g, beta, cu, Hk, Hv, state, has_init,
                       static_cast<float*>(o), commit_state);
  } else {
    hipLaunchKernelGGL(step_kernel<uint16_t>, grid, dim3(kStepThreads), 0, st,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), g, beta, cu, Hk, Hv, state, has_init,
                       static_cast<uint16_t*>(o), commit_state);
  }
  return hipGetLastError();
}

hipError_t launch_decode_fused(const void* x, int64_t xs, int act, const float* w, const float* bias,
                               float* conv_state, const int32_t* cu, int nseq, int Hk, int Hv, float eps,
                               const float* g, const float* beta, float* state, const uint8_t* has_init,
                               void* o, void* k_out, void* v_out, int write_conv_state, int commit_state,
                               hipStream_t st) {
  const int G = Hv / Hk;
  const dim3 grid(nseq * Hk);
#define GDN_FUSED_LAUNCH(TT, GG)                                                                   \
  hipLaunchKernelGGL((fused_kernel<TT, GG>), grid, dim3(kStepThreads * GG), 0, st, static_cast<const TT*>(x), xs, w, \
                     bias, conv_state, cu, Hk, Hv, eps, g, beta, state, has_init, static_cast<TT*>(o),     \
                     static_cast<TT*>(k_out), static_cast<TT*>(v_out), write_conv_state, commit_state)
  if (act == GDN_F32) {
    if (G == 1) GDN_FUSED_LAUNCH(float, 1);
    else GDN_FUSED_LAUNCH(float, 2);
  } else {
    if (G == 1) GDN_FUSED_LAUNCH(uint16_t, 1);
    else GDN_FUSED_LAUNCH(uint16_t, 2);
  }
#undef GDN_FUSED_LAUNCH
  return hipGetLastError();
}

hipError_t launch_commit(const gdn_layer_io* layers, int L, const int32_t* cu,
                         const int32_t* n_keep, const uint8_t* has_init, int nseq, int C, int Hk,
                         int Hv, int act, hipStream_t st) {
  const int roles = Hv + (C + kStepThreads * 8 - 1) / (kStepThreads * 8);
  dim3 grid(L * nseq * roles);
  if (act == GDN_F32) {
    hipLaunchKernelGGL(commit_kernel<float>, grid, dim3(kStepThreads), 0, st, layers, cu, n_keep,
                       has_init, nseq, C, Hk, Hv, roles);
  } else {
    hipLaunchKernelGGL(commit_kernel<uint16_t>, grid, dim3(kStepThreads), 0, st, layers, cu,
                       n_keep, has_init, nseq, C, Hk, Hv, roles);
  }
  return hipGetLastError();
}

}  // namespace gdn
