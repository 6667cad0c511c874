// Chunked gated delta-rule prefill (gfx950, MFMA).
//
// Recurrence (gated delta rule, Yang et al. 2024): per sequence and v-head,
//   S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t.
// The pages print no chunked algorithm (the Strata pull request 3226 leaves
// its prefill kernels untouched, "What This Does NOT Fix"); this kernel uses
// the chunk-64 WY form derived from the per-token rule.  For a chunk of n
// tokens (local index i) entering with state S0:
//   G_i = sum_{m<=i} g_m,  gamma_i = exp(G_i),  d_i = exp(G_{n-1} - G_i)
//   A_ij = b_i exp(G_i - G_j) (k_i . k_j)  (j < i)
//   Z = K S0^T,   R_i = b_i (v_i - gamma_i Z_i),   (I + A) U = R
//   O = diag(gamma) Q S0^T + P U,  P_ij = exp(G_i - G_j) (q_i . k_j) (j <= i)
//   S = gamma_{n-1} S0 + (diag(d) U)^T K
// (U = T diag(b) V - T diag(b gamma) K S0^T with T = (I + A)^-1 is the usual
// WY factor; here it is reached by solving (I + A) U = R blockwise.  The bf16
// kernel keeps b out of R: with A = diag(b) A~ it forms R~_i = v_i -
// gamma_i Z_i and U_i = T'_ii (R~_i - sum_{j<i} A~_ij U_j), where T'_ii =
// (I + A_ii)^-1 diag(b_i) and A~_ij = exp(G_i - G_j) (k_i . k_j).)
//
// Work split.  Rows of S (the dv index) evolve independently.  A workgroup
// owns one (sequence, v-head, slice of state rows) and walks the sequence's
// chunks in order; a wave owns 16-row blocks of the state and holds them
// TRANSPOSED (S^T, 8 tiles of 16x16) in MFMA accumulators.  An accumulator
// tile holds element [4*(lane/16) + e][lane % 16], which is exactly the
// B-operand layout of the next product (contraction index = tile row), so
// the chain Z -> R -> U -> (O, S) passes its operands in registers.  Only K,
// Q, the triangular factors and P live in LDS, shared by the waves; the
// K^T operand of the state update is read from K with the transposing LDS
// load ds_read_b64_tr_b16.
//
// Two schedules.  prefill_kernel (float32 activations): every wave stages,
// builds its share of the 10 lower 16x16 tile pairs of K K^T and Q K^T
// (scaled into -A, the diagonal blocks of A, and P) and of the diagonal
// inverses, then runs the state chain; three barriers per chunk, the next
// chunk's inputs prefetched into registers.  prefill_ws_kernel (bf16
// activations): producer waves build the state-independent factors one
// chunk ahead while consumer waves run the state chain (described at that
// kernel).
//
// Precision.  bf16 activations: every contraction is one bf16 MFMA pass
// (v_mfma_f32_16x16x32_bf16, or 16x16x16 for the 16-wide block solve) with
// float32 accumulation; the state is carried in float32 accumulators and
// rounded to bf16 only as an MFMA operand; the 16x16 diagonal inverses are
// float32.  float32 activations: every contraction uses
// v_mfma_f32_16x16x4_f32 on float32 operands.
#include <mutex>
#include <type_traits>

#include "launch.hpp"
#include "mfma.hpp"

namespace gdn {

namespace {

constexpr int BT = 64;    // chunk length
constexpr int DK = 128;   // head size
constexpr float kLog2e = 1.4426950408889634f;


template <class T, int NW> struct __attribute__((aligned(16))) Smem {
  using E = typename Prec<T>::E;
  static constexpr int LDK = DK + Prec<T>::PAD;   // rows of 128 features
  static constexpr int LDT = BT + Prec<T>::PAD;   // rows of 64 tokens
  E K[BT * LDK];        // K (token, feature)
  E Q[BT * LDK];        // Q (token, feature)
  E AT[BT * LDT];       // off-diagonal 16x16 blocks: -A; diagonal blocks: T_bb = (I + A_bb)^-1
  E P[BT * LDT];        // masked, decayed Q K^T
  float Ad[4][16][20];  // diagonal 16x16 blocks of A, row-major (rows 16-byte aligned)
  float W[NW][4][BT];   // per-wave copies of log2-scaled G, gamma, beta, d
};

// The 10 lower 16x16 tile pairs (bi, bj): the four diagonal ones first.
__device__ __forceinline__ void tile_pair(int p, int& bi, int& bj) {
  constexpr int kI[10] = {0, 1, 2, 3, 1, 2, 3, 2, 3, 3};
  constexpr int kJ[10] = {0, 1, 2, 3, 0, 1, 2, 0, 1, 0};
  bi = kI[p];
  bj = kJ[p];
}

// NW waves per workgroup, each owning VB blocks of 16 state rows.
template <class T, int NW, int VB>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
    int Hk, int Hv, float* state, const uint8_t* __restrict__ has_init, T* __restrict__ o) {
  using PR = Prec<T>;
  using E = typename PR::E;
  using SM = Smem<T, NW>;
  constexpr int NT = NW * 64;
  constexpr int DVS = 16 * NW * VB;
  constexpr int NSL = DK / DVS;
  constexpr int LDK = SM::LDK, LDT = SM::LDT;
  constexpr int KQ_ITEMS = BT * (DK / 8) / NT;   // 16-byte pieces of K and of Q per thread
  static_assert(NW == 4, "tile-pair assignment assumes 4 waves");

  __shared__ SM sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, kg = lane >> 4;

  // Blocks are dealt to the 8 XCDs round robin; consecutive units (the
  // slices of one head, then the heads sharing a k-head) go to one XCD so
  // their shared K and Q reads meet in that XCD's L2.
  int u = blockIdx.x;
  if ((gridDim.x & 7) == 0) u = (u & 7) * (gridDim.x >> 3) + (u >> 3);
  const int slice = u % NSL;
  u /= NSL;
  const int h = u % Hv;
  const int s = u / Hv;
  const int kh = h / (Hv / Hk);
  const int bos = cu[s], eos = cu[s + 1];
  const bool init = seq_flag(has_init, s);   // requested with cu (both scalar)
  int v0[VB];                               // this wave's state rows: v0[b] .. v0[b] + 15
#pragma unroll
  for (int b = 0; b < VB; ++b) v0[b] = slice * DVS + 16 * (wave * VB + b);

  // ---- S^T tiles: st[b][cb][e] = S[v0[b] + r16][16 cb + 4 kg + e]
  f32x4 st[VB][8];
  float* const sbase = state + ((int64_t)s * Hv + h) * (DK * DK);
#pragma unroll
  for (int b = 0; b < VB; ++b)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      if (init) {
        const float4 t = *reinterpret_cast<const float4*>(sbase + (int64_t)(v0[b] + r16) * DK + 16 * cb + 4 * kg);
        st[b][cb] = f32x4{t.x, t.y, t.z, t.w};
      } else {
        st[b][cb] = zero4();
      }
    }

  // ---- prefetch registers for one chunk.  Every load is unconditional
  // (rows past the chunk end read the chunk's last row) and kept in storage
  // form; rows >= n are zeroed where the data is used, so no load waits on
  // a branch.
  typename PR::Raw8 pk[KQ_ITEMS], pq[KQ_ITEMS];
  E vpre[VB][4][4];
  float gpre, bpre;
  auto prefetch = [&](int c0) {
    const int last = min(BT, eos - c0) - 1;
#pragma unroll
    for (int it = 0; it < KQ_ITEMS; ++it) {
      const int idx = tid + NT * it;
      const int row = min(idx >> 4, last), c8 = (idx & 15) * 8;
      const int64_t off = ((int64_t)(c0 + row) * Hk + kh) * DK + c8;
      pk[it] = PR::load_raw8(k + off);
      pq[it] = PR::load_raw8(q + off);
    }
#pragma unroll
    for (int b = 0; b < VB; ++b)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = min(16 * ib + 4 * kg + e, last);
          vpre[b][ib][e] = v[((int64_t)(c0 + row) * Hv + h) * DK + v0[b] + r16];
        }
    const int row = min(lane, last);
    gpre = g[(int64_t)(c0 + row) * Hv + h];
    bpre = beta[(int64_t)(c0 + row) * Hv + h];
  };

  if (bos < eos) prefetch(bos);

  float* const WL = sm.W[wave][0];    // log2-scaled G
  float* const Wgam = sm.W[wave][1];
  float* const Wb = sm.W[wave][2];
  float* const Wd = sm.W[wave][3];

  for (int c0 = bos; c0 < eos; c0 += BT) {
    const int n = min(BT, eos - c0);
    __syncthreads();  // the previous chunk is done with K, Q, AT, P, Ad

    // ---- 1. stage K and Q; keep this chunk's V, g, beta; prefetch the next
#pragma unroll
    for (int it = 0; it < KQ_ITEMS; ++it) {
      const int idx = tid + NT * it;
      const int row = idx >> 4, c8 = (idx & 15) * 8;
      const bool ok = row < n;
      PR::store_raw8(&sm.K[row * LDK + c8], ok ? pk[it] : PR::zero_raw8());
      PR::store_raw8(&sm.Q[row * LDK + c8], ok ? pq[it] : PR::zero_raw8());
    }
    float vv[VB][4][4];
#pragma unroll
    for (int b = 0; b < VB; ++b)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vv[b][ib][e] = (16 * ib + 4 * kg + e < n) ? PR::to_f32(vpre[b][ib][e]) : 0.f;
    const float gl = lane < n ? gpre : 0.f, bl = lane < n ? bpre : 0.f;
    if (c0 + BT < eos) prefetch(c0 + BT);

    // cumulative log decay over the chunk, in every wave (lane = token)
    const float L = wave_prefix_sum(gl) * kLog2e;
    const float Llast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(L), n - 1));
    WL[lane] = L;
    Wgam[lane] = exp2f(L);
    Wb[lane] = bl;
    Wd[lane] = lane < n ? exp2f(Llast - L) : 0.f;
    const float gamma_last = exp2f(Llast);
    __syncthreads();

    // ---- 2a. Z = K S0^T and QS = Q S0^T for this wave's rows.  The K and Q
    //          fragments of contraction step t+1 are read while step t runs.
    f32x4 z[VB][4], qs[VB][4];
#pragma unroll
    for (int b = 0; b < VB; ++b)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) { z[b][ib] = zero4(); qs[b][ib] = zero4(); }
    {
      typename PR::F32 fk[2][4], fq[2][4];
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        fk[0][ib] = PR::lds32(sm.K, LDK, 16 * ib + r16, 0, kg);
        fq[0][ib] = PR::lds32(sm.Q, LDK, 16 * ib + r16, 0, kg);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int cur = t & 1, nxt = cur ^ 1;
        if (t < 3) {
#pragma unroll
          for (int ib = 0; ib < 4; ++ib) {
            fk[nxt][ib] = PR::lds32(sm.K, LDK, 16 * ib + r16, 32 * (t + 1), kg);
            fq[nxt][ib] = PR::lds32(sm.Q, LDK, 16 * ib + r16, 32 * (t + 1), kg);
          }
        }
#pragma unroll
        for (int b = 0; b < VB; ++b) {
          const auto bs = PR::reg32(st[b][2 * t], st[b][2 * t + 1]);
#pragma unroll
          for (int ib = 0; ib < 4; ++ib) {
            z[b][ib] = PR::mma32(fk[cur][ib], bs, z[b][ib]);
            qs[b][ib] = PR::mma32(fq[cur][ib], bs, qs[b][ib]);
          }
        }
      }
    }

    // ---- 2b. tile pairs of K K^T and Q K^T -> -A, A_bb, P.  Wave w takes
    //          diagonal pair w (and inverts it) plus off-diagonal pairs
    //          4 + w and, for w < 2, 8 + w.
    for (int p = wave; p < 10; p = (p < 4) ? p + 4 : (p < 6 ? p + 4 : 10)) {
      int bi, bj;
      tile_pair(p, bi, bj);
      f32x4 kk = zero4(), qk = zero4();
#pragma unroll
      for (int kb = 0; kb < DK; kb += 32) {
        const auto bk = PR::lds32(sm.K, LDK, 16 * bj + r16, kb, kg);
        kk = PR::mma32(PR::lds32(sm.K, LDK, 16 * bi + r16, kb, kg), bk, kk);
        qk = PR::mma32(PR::lds32(sm.Q, LDK, 16 * bi + r16, kb, kg), bk, qk);
      }
      // rows i = 16 bi + 4 kg + e (4 consecutive tokens), column j = 16 bj + r16
      const float4 Li = *reinterpret_cast<const float4*>(&WL[16 * bi + 4 * kg]);
      const float4 Bi = *reinterpret_cast<const float4*>(&Wb[16 * bi + 4 * kg]);
      const float Lj = WL[16 * bj + r16];
      const float li[4] = {Li.x, Li.y, Li.z, Li.w};
      const float bb4[4] = {Bi.x, Bi.y, Bi.z, Bi.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * bi + 4 * kg + e, j = 16 * bj + r16;
        const float dec = j <= i ? exp2f(li[e] - Lj) : 0.f;
        PR::put(&sm.P[i * LDT + j], dec * qk[e]);
        const float a = j < i ? bb4[e] * dec * kk[e] : 0.f;
        if (bi == bj) sm.Ad[bi][i - 16 * bi][j - 16 * bj] = a;
        else PR::put(&sm.AT[i * LDT + j], -a);
      }
      if (bi == bj) {
        // T_bb = (I + A_bb)^-1 by forward substitution.  Lane (c, q) =
        // (lane / 4, lane % 4) owns rows q, q+4, q+8, q+12 of column c; the
        // four lanes of a column form a DPP quad, and x_j, once final, is
        // broadcast within the quad from the lane that owns row j.  Terms
        // with j >= i vanish because A_bb is strictly lower triangular.
        __builtin_amdgcn_wave_barrier();   // A_bb above was written by this wave
        const int c = lane >> 2, qd = lane & 3;
        float arow[4][16];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int j4 = 0; j4 < 4; ++j4) {
            const float4 t = *reinterpret_cast<const float4*>(&sm.Ad[bi][qd + 4 * m][4 * j4]);
            arow[m][4 * j4] = t.x; arow[m][4 * j4 + 1] = t.y;
            arow[m][4 * j4 + 2] = t.z; arow[m][4 * j4 + 3] = t.w;
          }
        float x[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) x[m] = (qd + 4 * m == c) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float xj = quad_bcast(x[j >> 2], j & 3);
#pragma unroll
          for (int m = 0; m < 4; ++m) x[m] = __builtin_fmaf(-arow[m][j], xj, x[m]);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) PR::put(&sm.AT[(16 * bi + qd + 4 * m) * LDT + 16 * bi + c], x[m]);
      }
    }
    __syncthreads();

    // ---- 3. R, then (I + A) U = R by block forward substitution:
    //         U_i = T_ii (R_i + sum_{m<i} (-A_im) U_m)
    float gam4[4][4], b4[4][4], d4[4][4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      const float4 ga = *reinterpret_cast<const float4*>(&Wgam[16 * ib + 4 * kg]);
      const float4 bt = *reinterpret_cast<const float4*>(&Wb[16 * ib + 4 * kg]);
      const float4 dd = *reinterpret_cast<const float4*>(&Wd[16 * ib + 4 * kg]);
      gam4[ib][0] = ga.x; gam4[ib][1] = ga.y; gam4[ib][2] = ga.z; gam4[ib][3] = ga.w;
      b4[ib][0] = bt.x; b4[ib][1] = bt.y; b4[ib][2] = bt.z; b4[ib][3] = bt.w;
      d4[ib][0] = dd.x; d4[ib][1] = dd.y; d4[ib][2] = dd.z; d4[ib][3] = dd.w;
    }
    f32x4 uu[VB][4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      f32x4 rr[VB];
#pragma unroll
      for (int b = 0; b < VB; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) rr[b][e] = b4[ib][e] * (vv[b][ib][e] - gam4[ib][e] * z[b][ib][e]);
      if (ib >= 2) {   // blocks 0 and 1 together as one 32-wide step
        const auto a01 = PR::lds32(sm.AT, LDT, 16 * ib + r16, 0, kg);
#pragma unroll
        for (int b = 0; b < VB; ++b) rr[b] = PR::mma32(a01, PR::reg32(uu[b][0], uu[b][1]), rr[b]);
      }
      if (ib == 1 || ib == 3) {
        const auto am = PR::lds16(sm.AT, LDT, 16 * ib + r16, 16 * (ib - 1), kg);
#pragma unroll
        for (int b = 0; b < VB; ++b) rr[b] = PR::mma16(am, PR::reg16(uu[b][ib - 1]), rr[b]);
      }
      const auto td = PR::lds16(sm.AT, LDT, 16 * ib + r16, 16 * ib, kg);
#pragma unroll
      for (int b = 0; b < VB; ++b) uu[b][ib] = PR::mma16(td, PR::reg16(rr[b]), zero4());
    }

    // ---- 4. O = diag(gamma) QS + P U
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      f32x4 pu[VB];
#pragma unroll
      for (int b = 0; b < VB; ++b) pu[b] = zero4();
      if (ib >= 1) {
        const auto p01 = PR::lds32(sm.P, LDT, 16 * ib + r16, 0, kg);
#pragma unroll
        for (int b = 0; b < VB; ++b) pu[b] = PR::mma32(p01, PR::reg32(uu[b][0], uu[b][1]), pu[b]);
      }
      if (ib == 3) {
        const auto p23 = PR::lds32(sm.P, LDT, 16 * ib + r16, 32, kg);
#pragma unroll
        for (int b = 0; b < VB; ++b) pu[b] = PR::mma32(p23, PR::reg32(uu[b][2], uu[b][3]), pu[b]);
      } else if (ib != 1) {   // ib == 0: block 0; ib == 2: block 2
        const auto pd = PR::lds16(sm.P, LDT, 16 * ib + r16, 16 * ib, kg);
#pragma unroll
        for (int b = 0; b < VB; ++b) pu[b] = PR::mma16(pd, PR::reg16(uu[b][ib]), pu[b]);
      }
#pragma unroll
      for (int b = 0; b < VB; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * ib + 4 * kg + e;
          if (i < n) {
            const float ov = gam4[ib][e] * qs[b][ib][e] + pu[b][e];
            Act<T>::store1(o + ((int64_t)(c0 + i) * Hv + h) * DK + v0[b] + r16, ov);
          }
        }
    }

    // ---- 5. S^T <- gamma_last S^T + K^T diag(d) U
    typename PR::F32 du01[VB], du23[VB];
#pragma unroll
    for (int b = 0; b < VB; ++b) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) uu[b][mb][e] *= d4[mb][e];
      du01[b] = PR::reg32(uu[b][0], uu[b][1]);
      du23[b] = PR::reg32(uu[b][2], uu[b][3]);
    }
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const auto kt0 = PR::ldsT32(sm.K, LDK, 16 * cb, 0, lane);
      const auto kt1 = PR::ldsT32(sm.K, LDK, 16 * cb, 32, lane);
#pragma unroll
      for (int b = 0; b < VB; ++b) {
        f32x4 acc;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = gamma_last * st[b][cb][e];
        acc = PR::mma32(kt0, du01[b], acc);
        st[b][cb] = PR::mma32(kt1, du23[b], acc);
      }
    }
  }

  // ---- final state
#pragma unroll
  for (int b = 0; b < VB; ++b)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
      *reinterpret_cast<float4*>(sbase + (int64_t)(v0[b] + r16) * DK + 16 * cb + 4 * kg) =
          make_float4(st[b][cb][0], st[b][cb][1], st[b][cb][2], st[b][cb][3]);
}

// ---------------------------------------------------------------------------
// Warp-specialised variant (bf16 activations).  The part of a chunk that
// does not depend on the state (staging K and Q, the tile pairs of K K^T and
// Q K^T, the decays, -A, P and the diagonal inverses) is built ahead of the
// state chain by four producer waves, while four consumer waves own the
// state and run the chain (Z, R, U, the state update, O) of the current
// chunk.  Each SIMD hosts one wave of each role, so the LDS and MFMA
// latencies of one role are covered by the other's work.  In iteration c
// the consumers run chunk c while the producers build the factors of chunk
// c+1 and stage K, Q and the gate vectors of chunk c+2: K, Q and the gate
// vectors are triple-buffered in LDS, the factors double-buffered, and one
// barrier ends each iteration.
//
// Global accesses go through raw buffer resources that span exactly the
// valid tokens of the chunk, so the hardware range check zero-fills loads
// of tail rows and drops stores to them; no lane masks or address clamps.
// O is formed transposed (the operands of Q S^T and P U swapped), which
// gives each lane four consecutive dv values of one token: 8-byte stores.
// The pair products are formed transposed for the same reason: each lane
// writes four consecutive columns of P and -A.

constexpr int kOrderMax = 64;            // batches up to this size run longest first

// K and Q tiles (64 tokens x 128 features, bf16) hold their rows with the
// 8-byte granules of row r XOR-permuted by sig(r) = 4 (r % 8) +
// 2 ((r / 8) % 2).  A fragment read (32 lanes: 16 rows x 2 granules) and a
// transposing read (32 lanes: 8 rows x 4 consecutive granules) then both
// touch each of the 64 LDS banks exactly once; no plain row padding does
// that for both patterns.  sig(r) is even, so granules 2m and 2m + 1 stay
// adjacent: a 16-byte read of them (16 lanes: 16 rows) also covers the 64
// banks once.  Each 16-row block is followed by 16 bytes of
// padding, which shifts a block's banks uniformly (a read never spans two
// blocks) but keeps any two blocks, and the same position in a K and a Q
// tile, from lying a multiple of 512 bytes apart: the compiler would fuse
// such reads into ds_read2st64_b64, which costs about 3.4x the LDS cycles
// of the separate reads.  Returns the element offset of granule g of row r.
constexpr int kKQTile = BT * DK + 4 * 8;   // elements per tile, with the block padding
__device__ __forceinline__ int kq_at(int r, int g) {
  return 4 * (32 * r + (g ^ (4 * (r & 7) + 2 * ((r >> 3) & 1)))) + 8 * (r >> 4);
}

// Element position of column c in a row of the factor tiles (-A / T and P).
// Within each 32-column group the two 4-column quads a 16x16x32 fragment
// lane reads (columns 4q .. 4q+3 and 16 + 4q .. 16+4q+3) are stored side by
// side, so that fragment is one 16-byte read, and a 16x16x16 fragment (one
// quad) one 8-byte read.
__device__ __forceinline__ constexpr int ft_pos(int c) {
  return 32 * (c >> 5) + 8 * ((c >> 2) & 3) + 4 * ((c >> 4) & 1) + (c & 3);
}

struct __attribute__((aligned(16))) SmemWS {
  static constexpr int LDT = BT + 8;   // rows of 64 tokens (bf16)
  uint16_t K[3][kKQTile];
  uint16_t Q[3][kKQTile];
  uint16_t AT[2][BT * LDT];   // off-diagonal 16x16 blocks: -A~; diagonal blocks: T_bb diag(b)
  uint16_t P[2][BT * LDT];
  float W[3][4][BT];          // per chunk: log2-scaled G, gamma, beta, d
  float Ad[4][16][20];        // diagonal block of A of each producer wave
  uint16_t O[2][BT * 72];     // V / o staging: 64 tokens x 64 state rows, rows padded to 144 B
  int len[kOrderMax];         // sequence lengths, for the longest-first order
  int pick;
};

// Fragment of a swizzled K / Q tile: rows row.., contraction kb.. (as
// Prec<uint16_t>::lds32 on a row-major tile).
__device__ __forceinline__ Prec<uint16_t>::F32 kq_frag(const uint16_t* p, int row, int kb, int kg) {
  const uint2 a = *reinterpret_cast<const uint2*>(p + kq_at(row, (kb >> 2) + kg));
  const uint2 b = *reinterpret_cast<const uint2*>(p + kq_at(row, (kb >> 2) + 4 + kg));
  Prec<uint16_t>::F32 f;
  f.v = make_uint4(a.x, a.y, b.x, b.y);
  return f;
}

// Fragment of a swizzled K / Q tile with the natural contraction order: lane
// (r16, kg) holds k = 32 t + 8 kg .. + 7, logical granules 8 t + 2 kg and
// + 1, which the (even) swizzle keeps adjacent and 16-byte aligned: one
// 16-byte read.  Only for products whose two operands both come from K / Q
// tiles (the tile pairs).
__device__ __forceinline__ Prec<uint16_t>::F32 kq_frag_nat(const uint16_t* p, int row, int t, int kg) {
  Prec<uint16_t>::F32 f;
  f.v = *reinterpret_cast<const uint4*>(p + kq_at(row, 8 * t + 2 * kg));
  return f;
}

// Transposed fragment of a swizzled K tile (as Prec<uint16_t>::ldsT32).
__device__ __forceinline__ Prec<uint16_t>::F32 kq_fragT(const uint16_t* p, int c0, int kb, int lane) {
  const int sl = lane & 15, kg = lane >> 4;
  const int r = kb + 4 * kg + (sl >> 2), g = (c0 >> 2) + (sl & 3);
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + kq_at(r, g)));
  const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + kq_at(r + 16, g)));
  const uint2 ux = __builtin_bit_cast(uint2, x), uy = __builtin_bit_cast(uint2, y);
  Prec<uint16_t>::F32 f;
  f.v = make_uint4(ux.x, ux.y, uy.x, uy.y);
  return f;
}

// Segment roles (SEG != 0).  A sequence of nc = ceil(n / 64) chunks is split
// into nseg segments of whole chunks: segment p covers chunks [b(p),
// b(p + 1)), b(0) = 0, b(nseg) = nc, b(p) = ceil(nc (2 p + 3) / (2 nseg + 3)),
// i.e. segment 0 spans 5 of 2 nseg + 3 shares and every later one 2 (tokens
// clipped to n).  Segment 0 is evaluated once (first pass), a later one
// three times (R, P, then the re-run), so a longer first segment shortens
// the critical path: on one 32k-token sequence (32 v-heads) with 5
// segments the two passes take about 15% less than with 4 equal ones.  The
// per-token rule is
// affine in the state, S_end = S_start P + R, so
//   SEG = 1 (first pass): segment 0 runs from the entering state and writes
//     its end state to X[1]; every later segment p runs twice over its
//     tokens, from S = 0 (end state R[p]) and, with v = 0, from S = I (end
//     state P[p], dk x dk); neither writes o;
//   SEG = 2 (second pass): every segment p >= 1 runs from X[p], written by
//     the combine X[p+1] = X[p] P[p] + R[p]; it writes o, and the last one
//     the final state.
// The workspace holds X, R and P, each [nseq][nseg][Hv][128][128] float32.
template <int VB, int SEG>
__global__ __launch_bounds__(512) void prefill_ws_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
    int Hk, int Hv, float* state, const uint8_t* __restrict__ has_init, uint16_t* __restrict__ o,
    int nseg, float* ws) {
  using PR = Prec<uint16_t>;
  constexpr int DVS = 64 * VB;   // state rows per workgroup (4 consumer waves)
  constexpr int NSL = DK / DVS;
  constexpr int LDT = SmemWS::LDT;
  constexpr int KQ_ITEMS = BT * (DK / 8) / 256;   // 16-byte pieces per producer thread

  __shared__ SmemWS sm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, kg = lane >> 4;
  const int rw = wave & 3;   // index of the wave within its role

  // Work item -> (sequence, v-head, slice).  Blocks are dispatched in
  // index order, so the sequences are taken longest first (for batches of
  // up to kOrderMax sequences): the longest sequence, whose chunks run one
  // after another, starts in the first wave of workgroups.  Within a
  // sequence, block b runs on XCD b % 8 (round-robin dispatch); item
  // i = (b % 8) * (items / 8) + b / 8 keeps the heads sharing a k-head, which
  // read the same K and Q, on one XCD and its L2.
  const int items = Hv * NSL;
  // groups of `items` workgroups per sequence: 1 (plain), 2 nseg - 1 (first
  // segment pass: segment 0, then R and P of each later segment), nseg - 1
  // (second pass)
  const int groups = SEG == 0 ? 1 : SEG == 1 ? 2 * nseg - 1 : nseg - 1;
  const int nseq = gridDim.x / (items * groups);
  const int rank = blockIdx.x / (items * groups);
  const int grp = blockIdx.x / items % groups;
  int item = blockIdx.x % items;
  if ((items & 7) == 0) item = (item & 7) * (items >> 3) + (item >> 3);
  // segment p and role: 0 = the real rows, 1 = R (from 0, no o), 2 = P
  // (from I, v = 0, no o)
  const int p = SEG == 0 ? 0 : SEG == 1 ? (grp + 1) / 2 : grp + 1;
  const int role = SEG == 1 && grp > 0 ? 2 - (grp & 1) : 0;
  int s = rank;
  if (SEG == 0 && nseq > 1 && nseq <= kOrderMax) {
    if (tid < nseq) sm.len[tid] = cu[tid + 1] - cu[tid];
    __syncthreads();
    if (tid < nseq) {
      const int mine = sm.len[tid];
      int r = 0;
      for (int t = 0; t < nseq; ++t) {
        const int other = sm.len[t];
        r += (other > mine || (other == mine && t < tid)) ? 1 : 0;
      }
      if (r == rank) sm.pick = tid;
    }
    __syncthreads();
    s = __builtin_amdgcn_readfirstlane(sm.pick);
  }
  const int slice = item % NSL;
  const int h = item / NSL;
  const int kh = h / (Hv / Hk);
  int bos = cu[s], eos = cu[s + 1];
  const bool init = seq_flag(has_init, s);   // requested with cu (both scalar)
  if (SEG != 0) {
    const int n = eos - bos;
    const int64_t nch = (n + BT - 1) / BT, shares = 2 * nseg + 3;
    auto bound = [&](int pp) -> int {   // first chunk of segment pp
      return pp == 0 ? 0 : pp >= nseg ? (int)nch : (int)((nch * (2 * pp + 3) + shares - 1) / shares);
    };
    eos = bos + min(n, bound(p + 1) * BT);
    bos = bos + min(n, bound(p) * BT);
  }
  const int nc = eos > bos ? (eos - bos + BT - 1) / BT : 0;
  // valid tokens of chunk c (0 past the end)
  auto chunk_len = [&](int c) { return max(0, min(BT, eos - (bos + BT * c))); };

  // the transition roles of the first segment pass write no o: their
  // workgroups run a body without the Q side (no Q tiles, Q K^T pairs, P,
  // Q S^T, P U or o stores)
  const bool o_on_wg = !(SEG == 1 && p > 0);

  if (wave >= 4) {
    // ================================================================ producers
    if (nc == 0) return;
    auto produce = [&](auto wo_c, auto rw_c) __attribute__((always_inline)) {
    constexpr bool WO = decltype(wo_c)::value;
    // the wave's index within its role as a compile-time constant: its tile
    // pairs' block offsets fold into the LDS instructions
    constexpr int rw = decltype(rw_c)::value;
    const int ptid = tid - 256;
    u32x4 pk[KQ_ITEMS], pq[KQ_ITEMS];
    float gr = 0.f, br = 0.f;
    auto load_kq = [&](int c) {
      const int64_t c0 = bos + BT * c;
      const int bytes = chunk_len(c) * Hk * DK * 2;
      const auto rk = buf_rsrc(k + c0 * Hk * DK, bytes);
      const auto rq = buf_rsrc(q + c0 * Hk * DK, bytes);
#pragma unroll
      for (int it = 0; it < KQ_ITEMS; ++it) {
        const int idx = ptid + 256 * it;
        const int off = (((idx >> 4) * Hk + kh) * DK + (idx & 15) * 8) * 2;
        pk[it] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
        if constexpr (WO) pq[it] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
      }
    };
    auto stage_kq = [&](int buf) {
#pragma unroll
      for (int it = 0; it < KQ_ITEMS; ++it) {
        const int idx = ptid + 256 * it;
        const int e = kq_at(idx >> 4, 2 * (idx & 15));
        *reinterpret_cast<u32x4*>(&sm.K[buf][e]) = pk[it];
        if constexpr (WO) *reinterpret_cast<u32x4*>(&sm.Q[buf][e]) = pq[it];
      }
    };
    // gate vectors: one token per lane (wave rw == 3 only, which forms two tile pairs, not three)
    auto load_gates = [&](int c) {
      const int64_t c0 = bos + BT * c;
      const int bytes = chunk_len(c) * Hv * 4;
      const int off = (lane * Hv + h) * 4;
      gr = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buf_rsrc(g + c0 * Hv, bytes), off, 0, 0));
      br = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buf_rsrc(beta + c0 * Hv, bytes), off, 0, 0));
    };
    // cumulative log2-decay of chunk c and the vectors derived from it;
    // lanes past the chunk's end hold g = beta = 0
    auto scan = [&](int c, int buf) {
      const int n = chunk_len(c);
      const float L = wave_prefix_sum(gr) * kLog2e;
      const float Llast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(L), max(n, 1) - 1));
      float* Wc = &sm.W[buf][0][0];
      Wc[lane] = L;
      Wc[BT + lane] = __builtin_amdgcn_exp2f(L);
      Wc[2 * BT + lane] = br;
      Wc[3 * BT + lane] = lane < n ? __builtin_amdgcn_exp2f(Llast - L) : 0.f;
    };
    // P and -A~ of tile pair (bi, bj), bi >= bj, from its products kk, qk
    // (A~ without the row's beta, which the stored T_ii diag(beta) applies;
    // the diagonal block keeps it, for the inverse):
    // lane (r16, kg) holds rows i = 16 bi + r16, columns j = 16 bj + 4 kg + e
    // (transposed products: K_bj-rows as the A operand)
    auto pair_store = [&](auto diag_c, int bi, int bj, f32x4 kk, f32x4 qk, int kb, int ab) __attribute__((always_inline)) {
      // off the diagonal every column precedes every row: no masks
      constexpr bool diag = decltype(diag_c)::value;
      const float* Wl = &sm.W[kb][0][0];
      const int i = 16 * bi + r16, j0 = 16 * bj + 4 * kg;
      const float Li = Wl[i], bti = Wl[2 * BT + i];
      const float4 Lj = *reinterpret_cast<const float4*>(&Wl[j0]);
      const float lj[4] = {Lj.x, Lj.y, Lj.z, Lj.w};
      float pv[4], av[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (diag) {
          const float dec = j0 + e <= i ? __builtin_amdgcn_exp2f(Li - lj[e]) : 0.f;
          pv[e] = dec * qk[e];
          av[e] = j0 + e < i ? bti * dec * kk[e] : 0.f;
        } else {
          const float dec = __builtin_amdgcn_exp2f(Li - lj[e]);
          pv[e] = dec * qk[e];
          av[e] = dec * kk[e];
        }
      }
      if constexpr (WO)
        *reinterpret_cast<u32x2*>(&sm.P[ab][i * LDT + ft_pos(j0)]) =
            u32x2{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])};
      if constexpr (diag)
        *reinterpret_cast<float4*>(&sm.Ad[rw][r16][4 * kg]) = make_float4(av[0], av[1], av[2], av[3]);
      else
        *reinterpret_cast<u32x2*>(&sm.AT[ab][i * LDT + ft_pos(j0)]) =
            u32x2{pack_bf16x2(-av[0], -av[1]), pack_bf16x2(-av[2], -av[3])};
    };
    // this wave's tile pairs of K/Q buffer kb: (rw, rw) on the diagonal, the
    // pair tile_pair(4 + rw) and, for rw < 2, tile_pair(8 + rw) (the ten
    // lower pairs over four waves).  Their fragments are read one 32-wide
    // contraction slice at a time for all pairs together, so the pairs' MFMA
    // chains and LDS reads overlap instead of running one pair after
    // another.  The third pair is a compile-time variant, chosen once.
    auto pairs_t = [&](auto third_c, int kb, int ab) __attribute__((always_inline)) {
      constexpr bool kThird = decltype(third_c)::value;
      const uint16_t* Kb = sm.K[kb];
      const uint16_t* Qb = sm.Q[kb];
      const int bd = rw;                                   // diagonal block
      constexpr int bi1 = rw < 3 ? rw + 1 : 2, bj1 = rw < 3 ? rw : 0;
      constexpr int bi2 = 3, bj2 = rw == 0 ? 1 : 0;
      f32x4 kk0 = zero4(), qk0 = zero4(), kk1 = zero4(), qk1 = zero4(), kk2 = zero4(), qk2 = zero4();
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const auto d0 = kq_frag_nat(Kb, 16 * bd + r16, t, kg);
        const auto b1 = kq_frag_nat(Kb, 16 * bj1 + r16, t, kg);
        const auto a1 = kq_frag_nat(Kb, 16 * bi1 + r16, t, kg);
        kk0 = PR::mma32(d0, d0, kk0);
        kk1 = PR::mma32(b1, a1, kk1);
        if constexpr (WO) {
          const auto q0 = kq_frag_nat(Qb, 16 * bd + r16, t, kg);
          const auto q1 = kq_frag_nat(Qb, 16 * bi1 + r16, t, kg);
          qk0 = PR::mma32(d0, q0, qk0);
          qk1 = PR::mma32(b1, q1, qk1);
        }
        if constexpr (kThird) {
          const auto b2 = kq_frag_nat(Kb, 16 * bj2 + r16, t, kg);
          const auto a2 = kq_frag_nat(Kb, 16 * bi2 + r16, t, kg);
          kk2 = PR::mma32(b2, a2, kk2);
          if constexpr (WO) {
            const auto q2 = kq_frag_nat(Qb, 16 * bi2 + r16, t, kg);
            qk2 = PR::mma32(b2, q2, qk2);
          }
        }
      }
      pair_store(std::true_type{}, bd, bd, kk0, qk0, kb, ab);
      pair_store(std::false_type{}, bi1, bj1, kk1, qk1, kb, ab);
      if constexpr (kThird) pair_store(std::false_type{}, bi2, bj2, kk2, qk2, kb, ab);
    };
    auto pairs = [&](int kb, int ab) __attribute__((always_inline)) {
      pairs_t(std::integral_constant<bool, (rw < 2)>{}, kb, ab);
    };
    // T_bb = (I + A_bb)^-1 of this wave's diagonal block b = rw, by forward
    // substitution.  Lane (c, q) = (lane / 4, lane % 4) owns rows q, q+4,
    // q+8, q+12 of column c; the four lanes of a column form a DPP quad and
    // x_j, once final, is broadcast from the lane owning row j.  Terms with
    // j >= i vanish: A_bb is strictly lower triangular.
    auto invert_diag = [&](int ab, int kbw) {
      const int c = lane >> 2, qd = lane & 3, bb = rw;
      // row q + 4 m has nonzero entries only in columns j < q + 4 m <= 4 m + 3,
      // so its columns past 4 m + 2 are neither read nor applied (they are
      // zero, and subtracting a zero product leaves x unchanged up to the
      // sign of a zero), and x_15 feeds no row
      float arow[4][16];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int j4 = 0; j4 <= m; ++j4) {
          const float4 t = *reinterpret_cast<const float4*>(&sm.Ad[rw][qd + 4 * m][4 * j4]);
          arow[m][4 * j4] = t.x; arow[m][4 * j4 + 1] = t.y;
          arow[m][4 * j4 + 2] = t.z; arow[m][4 * j4 + 3] = t.w;
        }
      float x[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) x[m] = (qd + 4 * m == c) ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < 15; ++j) {
        const float xj = quad_bcast(x[j >> 2], j & 3);
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (j <= 4 * m + 2) x[m] = __builtin_fmaf(-arow[m][j], xj, x[m]);
      }
      // stored as T_bb diag(beta): column c scaled by its token's beta, so
      // the consumers' solve needs no beta
      const float bc = sm.W[kbw][2][16 * bb + c];
#pragma unroll
      for (int m = 0; m < 4; ++m) PR::put(&sm.AT[ab][(16 * bb + qd + 4 * m) * LDT + ft_pos(16 * bb + c)], x[m] * bc);
    };
    // all factors of chunk c (K/Q and gate buffer c % 3 -> factor buffer c & 1)
    auto factors = [&](int c, int kb) __attribute__((always_inline)) {
      const int ab = c & 1;
      pairs(kb, ab);
      invert_diag(ab, kb);
    };

    load_kq(0);
    if constexpr (rw == 3) load_gates(0);
    stage_kq(0);
    if constexpr (rw == 3) scan(0, 0);
    load_kq(1);
    if constexpr (rw == 3) load_gates(1);
    __syncthreads();
    factors(0, 0);
    stage_kq(1);
    if constexpr (rw == 3) scan(1, 1);
    load_kq(2);
    if constexpr (rw == 3) load_gates(2);
    __syncthreads();
    // three chunks per trip: the K / Q buffers staged and read are
    // compile-time constants, so the fragment offsets fold into the
    // LDS instructions
    auto step = [&](int c, auto m_c) __attribute__((always_inline)) {
      constexpr int m = decltype(m_c)::value;   // c % 3
      stage_kq((m + 2) % 3);
      load_kq(c + 3);
      if constexpr (rw == 3) {
        scan(c + 2, (m + 2) % 3);
        load_gates(c + 3);
      }
      factors(c + 1, (m + 1) % 3);
      __syncthreads();
    };
    for (int c = 0; c < nc; c += 3) {
      step(c, std::integral_constant<int, 0>{});
      if (c + 1 >= nc) break;
      step(c + 1, std::integral_constant<int, 1>{});
      if (c + 2 >= nc) break;
      step(c + 2, std::integral_constant<int, 2>{});
    }
    };
    auto by_wave = [&](auto wo_c) __attribute__((always_inline)) {
      switch (rw) {
        case 0: produce(wo_c, std::integral_constant<int, 0>{}); break;
        case 1: produce(wo_c, std::integral_constant<int, 1>{}); break;
        case 2: produce(wo_c, std::integral_constant<int, 2>{}); break;
        default: produce(wo_c, std::integral_constant<int, 3>{}); break;
      }
    };
    if constexpr (SEG == 1) {
      if (o_on_wg) by_wave(std::true_type{});
      else by_wave(std::false_type{});
    } else {
      by_wave(std::true_type{});
    }
    return;
  }

  // ================================================================== consumers
  const int w = wave;
  int v0[VB];
#pragma unroll
  for (int b = 0; b < VB; ++b) v0[b] = slice * DVS + 16 * (w * VB + b);

  f32x4 st[VB][8];
  // entering state (src; none = zero, or the identity for a P role) and
  // where the end state goes (dst; none = not written)
  float* const sbase = state + ((int64_t)s * Hv + h) * (DK * DK);
  const float* src = init ? sbase : nullptr;
  float* dst = sbase;
  bool ident = false, v_on = true, o_on = true;
  if (SEG != 0) {
    auto wsp = [&](int which, int pp) {
      return ws + ((((int64_t)which * nseq + s) * nseg + pp) * Hv + h) * (DK * DK);
    };
    if (SEG == 1 && p == 0) {
      dst = wsp(0, 1);
    } else if (SEG == 1) {
      src = nullptr;
      dst = wsp(role, p);
      ident = role == 2;
      v_on = role == 1;
      o_on = false;
    } else {
      src = wsp(0, p);
      dst = p == nseg - 1 ? sbase : nullptr;
    }
  }
#pragma unroll
  for (int b = 0; b < VB; ++b)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      if (src != nullptr) {
        const float4 t = *reinterpret_cast<const float4*>(src + (int64_t)(v0[b] + r16) * DK + 16 * cb + 4 * kg);
        st[b][cb] = f32x4{t.x, t.y, t.z, t.w};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) st[b][cb][e] = ident && v0[b] + r16 == 16 * cb + 4 * kg + e ? 1.f : 0.f;
      }
    }

  if (nc > 0) {
    // a compile-time constant except in the first segment pass, where it is
    // uniform over the workgroup
    const bool WO = o_on_wg;
    // V enters and o leaves through two LDS tiles X[0], X[1] of 64 tokens x
    // 64 state rows (bf16, rows padded to 144 bytes).  Global memory sees
    // whole 128-byte row pieces only: wave w moves tokens 16 w .. 16 w + 15
    // of all 64 rows, 16 bytes per lane, two accesses per chunk.  The MFMA
    // side works on the wave's own 16 state rows of all tokens.  In
    // iteration c:
    //   top: read V(c) from X[c & 1] (own rows, transposing reads into the
    //        accumulator layout); read o(c-1) from X[(c+1) & 1] (own
    //        tokens), then write V(c+1), loaded one iteration earlier, into
    //        the same place; issue the loads of V(c+2), then the stores of
    //        o(c-1);
    //   end: write o(c) into X[c & 1] (own rows, where V(c) was read).
    // So within an iteration a wave touches X[c & 1] only in its own rows
    // and X[(c+1) & 1] only in its own tokens; what another wave wrote is
    // read only after the barrier that ends the iteration.  The stores come
    // after the V loads: one in-order counter covers loads and stores, so
    // the wait for those loads never includes a store.  Direct global
    // accesses in the accumulator layout moved 32-byte pieces (16 loads of
    // 2 bytes and 4 stores of 8 bytes per lane and chunk) and cost about a
    // fifth of the kernel time.  The row padding makes the 8-byte o writes
    // free of bank conflicts within a half wave.
    static_assert(VB == 1, "the V / o staging tiles hold 64 state rows");
    const int tok_w = 16 * w + (lane >> 3), gq = lane & 7;   // token-side piece: + 8 j
    u32x4 vg[2];
    auto load_v = [&](int c) {
      const int64_t c0 = bos + BT * c;
      const auto rv = buf_rsrc(v + c0 * Hv * DK, v_on ? chunk_len(c) * Hv * DK * 2 : 0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        vg[j] = __builtin_amdgcn_raw_buffer_load_b128(rv, (((tok_w + 8 * j) * Hv + h) * DK + slice * DVS + 8 * gq) * 2, 0, 0);
    };
    auto put_v = [&](int buf) {
#pragma unroll
      for (int j = 0; j < 2; ++j) *reinterpret_cast<u32x4*>(&sm.O[buf][(tok_w + 8 * j) * 72 + 8 * gq]) = vg[j];
    };
    // V(c) of this lane: tokens 16 ib + 4 kg + e of state row 16 w + r16
    // (ds_read_b64_tr_b16: result lane i, slot j comes from source lane
    // 4 j + i / 4, slot i % 4, within each 16-lane group)
    auto get_v = [&](int buf, float (&vv)[4][4]) {
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(&sm.O[buf][(16 * ib + 4 * kg + (r16 >> 2)) * 72 + 4 * (4 * w + (r16 & 3))]));
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[ib][e] = bf16_to_f32(static_cast<uint16_t>(x[e]));
      }
    };
    u32x2 opk[VB][4];
    __amdgpu_buffer_rsrc_t ro_prev = buf_rsrc(o, 0);
    auto stage_o = [&](int buf) {
#pragma unroll
      for (int ib = 0; ib < 4; ++ib)
        *reinterpret_cast<u32x2*>(&sm.O[buf][(16 * ib + r16) * 72 + 16 * w + 4 * kg]) = opk[0][ib];
    };
    u32x4 og[2];
    auto read_o = [&](int buf) {
#pragma unroll
      for (int j = 0; j < 2; ++j) og[j] = *reinterpret_cast<const u32x4*>(&sm.O[buf][(tok_w + 8 * j) * 72 + 8 * gq]);
    };
    auto store_o = [&]() {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(og[j], ro_prev, (((tok_w + 8 * j) * Hv + h) * DK + slice * DVS + 8 * gq) * 2, 0, 0);
    };
#pragma unroll
    for (int b = 0; b < VB; ++b)
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) opk[b][ib] = u32x2{0u, 0u};
    load_v(0);
    put_v(0);
    load_v(1);
    // K, Q, the gates and V of chunk 0 are in LDS after this barrier; the
    // producers form chunk 0's factors until the next one, which chunk 0's
    // iteration takes just before its solve: Z and R overlap those factors
    __syncthreads();

    // The loop runs three chunks per trip so that the K / Q and gate buffer
    // of each chunk (kb = c % 3) is a compile-time constant: the offsets of
    // its 96 fragment reads fold into the instructions, leaving the factor
    // and V / o tiles' (ab = c & 1) few reads with a computed base (mixed
    // serving layer -1%, varlen batch -2% against two chunks per trip with
    // ab constant; six per trip, both constant, spills).
    auto iteration = [&](int c, auto kb_c) __attribute__((always_inline)) {
      constexpr int kb = decltype(kb_c)::value;   // c % 3
      const int ab = c & 1;
      const int n = chunk_len(c);
      const int64_t c0 = bos + BT * c;
      const uint16_t* Kc = sm.K[kb];
      const uint16_t* Qc = sm.Q[kb];
      const uint16_t* ATc = sm.AT[ab];
      const uint16_t* Pc = sm.P[ab];
      const float* Wc = &sm.W[kb][0][0];
      const float gamma_last = __builtin_amdgcn_exp2f(Wc[n - 1]);

      float vv[VB][4][4];
      get_v(ab, vv[0]);
      if (WO && c > 0) read_o(ab ^ 1);
      put_v(ab ^ 1);
      load_v(c + 2);
      if (WO && c > 0) store_o();

      // The chain of the chunk is Z -> R -> the four block steps of the
      // solve -> the state update.  Each U block, once final, immediately
      // feeds its share of the state update and of U P^T.  The Q S0^T
      // products, which no later step of the chain needs, are formed after
      // the state update: anywhere earlier their fragment reads queue ahead
      // of the chain's own LDS reads (LDS returns in order) and their
      // products ahead of its MFMAs (between the block steps, before the
      // solve, and measured 2% slower there than here).  U P^T stays in
      // the solve, where it fills the matrix pipe while a block step waits
      // (3% slower after the update).
      // S0 is read as bf16 operands taken before the update (sb), so the
      // float32 state is updated in place.

      // gate vectors of this lane's rows (tokens 16 ib + 4 kg + e)
      float gam4[4][4], d4[4][4];
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const float4 ga = *reinterpret_cast<const float4*>(&Wc[BT + 16 * ib + 4 * kg]);
        const float4 dd = *reinterpret_cast<const float4*>(&Wc[3 * BT + 16 * ib + 4 * kg]);
        gam4[ib][0] = ga.x; gam4[ib][1] = ga.y; gam4[ib][2] = ga.z; gam4[ib][3] = ga.w;
        d4[ib][0] = dd.x; d4[ib][1] = dd.y; d4[ib][2] = dd.z; d4[ib][3] = dd.w;
      }
      typename PR::F32 sb[VB][4];
#pragma unroll
      for (int b = 0; b < VB; ++b)
#pragma unroll
        for (int t = 0; t < 4; ++t) sb[b][t] = PR::reg32(st[b][2 * t], st[b][2 * t + 1]);

      // ---- Z = K S0^T (rows: tokens)
      f32x4 z[VB][4];
#pragma unroll
      for (int b = 0; b < VB; ++b)
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) z[b][ib] = zero4();
      {
        typename PR::F32 fk[2][4];
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) fk[0][ib] = kq_frag(Kc, 16 * ib + r16, 0, kg);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int cur = t & 1, nxt = cur ^ 1;
          if (t < 3) {
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) fk[nxt][ib] = kq_frag(Kc, 16 * ib + r16, 32 * (t + 1), kg);
          }
#pragma unroll
          for (int b = 0; b < VB; ++b)
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) z[b][ib] = PR::mma32(fk[cur][ib], sb[b][t], z[b][ib]);
        }
      }

      // ---- R~ = V - diag(gamma) Z (beta enters through the stored
      // T_ii diag(beta))
      f32x4 rr[VB][4];
#pragma unroll
      for (int b = 0; b < VB; ++b)
#pragma unroll
        for (int ib = 0; ib < 4; ++ib)
#pragma unroll
          for (int e = 0; e < 4; ++e) rr[b][ib][e] = vv[b][ib][e] - gam4[ib][e] * z[b][ib][e];

      // (Q S0^T)^T (rows: state rows, columns: tokens), one 32-wide slice
      // of the contraction at a time
      f32x4 qt[VB][4];
#pragma unroll
      for (int b = 0; b < VB; ++b)
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) qt[b][ib] = zero4();
      auto qs_step = [&](int t) {
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
          const auto fq = kq_frag(Qc, 16 * ib + r16, 32 * t, kg);
#pragma unroll
          for (int b = 0; b < VB; ++b) qt[b][ib] = PR::mma32(sb[b][t], fq, qt[b][ib]);
        }
      };
      // S^T <- S^T + K^T diag(d) U over tokens kb .. kb+31 (the decay by
      // gamma_last is applied with the first half)
      auto state_half = [&](int kb, const typename PR::F32* du, bool first) {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          const auto kt = kq_fragT(Kc, 16 * cb, kb, lane);
#pragma unroll
          for (int b = 0; b < VB; ++b) {
            f32x4 acc = st[b][cb];
            if (first) {
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[e] = gamma_last * acc[e];
            }
            st[b][cb] = PR::mma32(kt, du[b], acc);
          }
        }
      };

      // ---- block solve U_i = (T_ii diag(beta)) (R~_i - sum_{j<i} A~_ij U_j),
      // interleaved with the products that each finished block enables.  An accumulator is never carried from
      // a 16x16x32 MFMA into a 16x16x16 one: the hardware needs wait states
      // between the two shapes that the compiler does not insert (the
      // second one read stale accumulator elements), so mixed-shape sums are
      // formed on separate accumulators and added.
      if constexpr (kb == 0) {
        if (c == 0) __syncthreads();   // chunk 0's factors are in LDS
      }
      // fragments of the factor tiles (ft_pos layout): fr32 = columns
      // 32 g .. 32 g + 31 of a 16x16x32 fragment (one 16-byte read), fr16 =
      // columns 16 h .. 16 h + 15 of a 16x16x16 one (one 8-byte read)
      // (the offset passes through an empty asm operand, which keeps the
      // compiler from hoisting these reads ahead of the chain's own: LDS
      // returns data in order)
      auto fr32 = [&](const uint16_t* p, int row, int g) __attribute__((always_inline)) {
        int off = row * LDT + 32 * g + 8 * kg;
        asm volatile("" : "+v"(off));
        typename PR::F32 f;
        f.v = *reinterpret_cast<const uint4*>(p + off);
        return f;
      };
      auto fr16 = [&](const uint16_t* p, int row, int h) __attribute__((always_inline)) {
        int off = row * LDT + 32 * (h >> 1) + 8 * kg + 4 * (h & 1);
        asm volatile("" : "+v"(off));
        typename PR::F16 f;
        f.v = *reinterpret_cast<const uint2*>(p + off);
        return f;
      };
      auto lo16 = [](typename PR::F32 f) { typename PR::F16 r; r.v = make_uint2(f.v.x, f.v.y); return r; };
      auto hi16 = [](typename PR::F32 f) { typename PR::F16 r; r.v = make_uint2(f.v.z, f.v.w); return r; };
      f32x4 uu[VB][4], pu[VB][4];
      {
        const auto td = fr16(ATc, r16, 0);
#pragma unroll
        for (int b = 0; b < VB; ++b) uu[b][0] = PR::mma16(td, PR::reg16(rr[b][0]), zero4());
      }
      {
        const auto amtd = fr32(ATc, 16 + r16, 0);
        const auto am = lo16(amtd), td = hi16(amtd);
#pragma unroll
        for (int b = 0; b < VB; ++b) {
          rr[b][1] = PR::mma16(am, PR::reg16(uu[b][0]), rr[b][1]);
          uu[b][1] = PR::mma16(td, PR::reg16(rr[b][1]), zero4());
        }
      }
      {
        // blocks 0 and 1 are final: first half of the state update and
        // their part of O
        typename PR::F32 du[VB], u01[VB];
#pragma unroll
        for (int b = 0; b < VB; ++b) {
          f32x4 d0, d1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            d0[e] = uu[b][0][e] * d4[0][e];
            d1[e] = uu[b][1][e] * d4[1][e];
          }
          du[b] = PR::reg32(d0, d1);
          u01[b] = PR::reg32(uu[b][0], uu[b][1]);
        }
        const auto a2 = fr32(ATc, 32 + r16, 0);
        const auto a3 = fr32(ATc, 48 + r16, 0);
#pragma unroll
        for (int b = 0; b < VB; ++b) {
          rr[b][2] = PR::mma32(a2, u01[b], rr[b][2]);
          rr[b][3] = PR::mma32(a3, u01[b], rr[b][3]);
        }
        if (WO) {
          const auto p0 = fr16(Pc, r16, 0);
#pragma unroll
          for (int b = 0; b < VB; ++b) pu[b][0] = PR::mma16(PR::reg16(uu[b][0]), p0, zero4());
#pragma unroll
          for (int ib = 1; ib < 4; ++ib) {
            const auto p01 = fr32(Pc, 16 * ib + r16, 0);
#pragma unroll
            for (int b = 0; b < VB; ++b) pu[b][ib] = PR::mma32(u01[b], p01, zero4());
          }
        }
        state_half(0, du, true);
      }
      {
        const auto td = fr16(ATc, 32 + r16, 2);
#pragma unroll
        for (int b = 0; b < VB; ++b) uu[b][2] = PR::mma16(td, PR::reg16(rr[b][2]), zero4());
      }
      {
        const auto amtd = fr32(ATc, 48 + r16, 1);
        const auto am = lo16(amtd), td = hi16(amtd);
#pragma unroll
        for (int b = 0; b < VB; ++b) {
          const f32x4 t3 = PR::mma16(am, PR::reg16(uu[b][2]), zero4());
#pragma unroll
          for (int e = 0; e < 4; ++e) rr[b][3][e] += t3[e];
          uu[b][3] = PR::mma16(td, PR::reg16(rr[b][3]), zero4());
        }
      }
      {
        // blocks 2 and 3: second half of the state update and the rest of O
        typename PR::F32 du[VB], u23[VB];
#pragma unroll
        for (int b = 0; b < VB; ++b) {
          f32x4 d2, d3;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            d2[e] = uu[b][2][e] * d4[2][e];
            d3[e] = uu[b][3][e] * d4[3][e];
          }
          du[b] = PR::reg32(d2, d3);
          u23[b] = PR::reg32(uu[b][2], uu[b][3]);
        }
        state_half(32, du, false);
        if (WO) {
          const auto p2 = fr16(Pc, 32 + r16, 2);
          const auto p3 = fr32(Pc, 48 + r16, 1);
#pragma unroll
          for (int b = 0; b < VB; ++b) {
            const f32x4 t2 = PR::mma16(PR::reg16(uu[b][2]), p2, zero4());
#pragma unroll
            for (int e = 0; e < 4; ++e) pu[b][2][e] += t2[e];
            pu[b][3] = PR::mma32(u23[b], p3, pu[b][3]);
          }
        }
      }

      if (WO) {
        qs_step(0);
        qs_step(1);
        qs_step(2);
        qs_step(3);
        // ---- O^T = (Q S0^T)^T diag(gamma) + U^T P^T; lane: token 16 ib + r16,
        // state rows v0 + 4 kg .. +3
        ro_prev = buf_rsrc(o + c0 * Hv * DK, o_on ? n * Hv * DK * 2 : 0);
#pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
          const float gt = Wc[BT + 16 * ib + r16];
#pragma unroll
          for (int b = 0; b < VB; ++b) {
            float ov[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) ov[e] = gt * qt[b][ib][e] + pu[b][ib][e];
            opk[b][ib] = u32x2{pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3])};
          }
        }
        stage_o(ab);
      }
      __syncthreads();
    };
    for (int c = 0; c < nc; c += 3) {
      iteration(c, std::integral_constant<int, 0>{});
      if (c + 1 >= nc) break;
      iteration(c + 1, std::integral_constant<int, 1>{});
      if (c + 2 >= nc) break;
      iteration(c + 2, std::integral_constant<int, 2>{});
    }
    if (WO) {
      read_o((nc - 1) & 1);
      store_o();
    }
  }

  if (dst != nullptr) {
#pragma unroll
    for (int b = 0; b < VB; ++b)
#pragma unroll
      for (int cb = 0; cb < 8; ++cb)
        *reinterpret_cast<float4*>(dst + (int64_t)(v0[b] + r16) * DK + 16 * cb + 4 * kg) =
            make_float4(st[b][cb][0], st[b][cb][1], st[b][cb][2], st[b][cb][3]);
  }
}

template <int VB, int SEG>
hipError_t launch_ws(const void* q, const void* k, const void* v, const float* g, const float* beta,
                     const int32_t* cu, int nseq, int Hk, int Hv, float* state,
                     const uint8_t* has_init, void* o, int nseg, float* ws, hipStream_t st) {
  const int groups = SEG == 0 ? 1 : SEG == 1 ? 2 * nseg - 1 : nseg - 1;
  const dim3 grid(nseq * Hv * (DK / (64 * VB)) * groups);
  hipLaunchKernelGGL((prefill_ws_kernel<VB, SEG>), grid, dim3(512), 0, st, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), g, beta, cu, Hk,
                     Hv, state, has_init, static_cast<uint16_t*>(o), nseg, ws);
  return hipGetLastError();
}

// The segment chain X[p + 1] = X[p] P[p] + R[p], p = 1 .. nseg - 2, for one
// 16-row block of one (sequence, v-head).  Rows of the chain are
// independent (row i of X[p + 1] needs row i of X[p] and all of P[p]), so
// every block runs its own chain, in float32 on 16x16x4 MFMAs: wave w forms
// columns 32 w .. 32 w + 31 (two 16x16 tiles) from the block's X rows and
// P, both staged in LDS, starting from R.  Rows of the LDS copies are padded
// to 132 floats, so a fragment's four strided P rows and its sixteen X rows
// each fall on distinct banks.
__global__ __launch_bounds__(256) void seg_combine_kernel(float* ws, int nseq, int nseg, int Hv) {
  constexpr int LD = DK + 4;
  __shared__ float Pl[DK * LD];
  __shared__ float Xl[16 * LD];
  // block b runs on XCD b % 8 (round-robin dispatch); when the units
  // (sequence, v-head) come in eights, the 8 row blocks of a unit share b % 8,
  // so the unit's P is fetched into one XCD's L2
  const int blk = blockIdx.x;
  const bool by_xcd = ((nseq * Hv) & 7) == 0;
  const int unit = by_xcd ? (blk & 7) + 8 * (blk >> 6) : blk >> 3;
  const int rb = by_xcd ? (blk >> 3) & 7 : blk & 7;
  const int h = unit % Hv, s = unit / Hv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  auto wsp = [&](int which, int pp) {
    return ws + ((((int64_t)which * nseq + s) * nseg + pp) * Hv + h) * (DK * DK);
  };
  // a 128-column matrix of ROWS rows from global memory into LDS rows of LD
  // floats: every piece of a thread is requested before the first is
  // written, so the copy waits for one memory latency, not one per piece
  auto stage = [&](float* dst, const float* src, auto rows_c) {
    constexpr int N = decltype(rows_c)::value * (DK / 4) / 256;
    f32x4 t[N];
#pragma unroll
    for (int j = 0; j < N; ++j) t[j] = reinterpret_cast<const f32x4*>(src)[tid + 256 * j];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int i = tid + 256 * j;
      *reinterpret_cast<f32x4*>(&dst[(i >> 5) * LD + 4 * (i & 31)]) = t[j];
    }
  };
  stage(Xl, wsp(0, 1) + 16 * rb * DK, std::integral_constant<int, 16>{});
  for (int p = 1; p + 1 < nseg; ++p) {
    stage(Pl, wsp(2, p), std::integral_constant<int, DK>{});
    __syncthreads();   // P[p] and X[p] are in LDS
    const float* Rp = wsp(1, p) + 16 * rb * DK;
    f32x4 acc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[j][e] = Rp[(4 * kg + e) * DK + 32 * w + 16 * j + r16];
#pragma unroll 4
    for (int kb = 0; kb < DK; kb += 16) {
      // lane (r16, kg), slot t: X[r16][kb + 4 kg + t] and P[kb + 4 kg + t][column]
      const float4 xa = *reinterpret_cast<const float4*>(&Xl[r16 * LD + kb + 4 * kg]);
      const f32x4 a = f32x4{xa.x, xa.y, xa.z, xa.w};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = 32 * w + 16 * j + r16;
        f32x4 b;
#pragma unroll
        for (int t = 0; t < 4; ++t) b[t] = Pl[(kb + 4 * kg + t) * LD + c];
        acc[j] = Prec<float>::mma4x(a, b, acc[j]);
      }
    }
    __syncthreads();   // every wave is done with Xl and Pl
    // lane (r16, kg) holds rows 4 kg + e of columns 32 w + 16 j + r16
    float* Xn = wsp(0, p + 1) + 16 * rb * DK;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 32 * w + 16 * j + r16;
        Xn[(4 * kg + e) * DK + c] = acc[j][e];
        Xl[(4 * kg + e) * LD + c] = acc[j][e];
      }
  }
}

template <class T, int NW, int VB>
hipError_t launch_t(const void* q, const void* k, const void* v, const float* g, const float* beta,
                    const int32_t* cu, int nseq, int Hk, int Hv, float* state,
                    const uint8_t* has_init, void* o, hipStream_t st) {
  const dim3 grid(nseq * Hv * (DK / (16 * NW * VB)));
  hipLaunchKernelGGL((prefill_kernel<T, NW, VB>), grid, dim3(NW * 64), 0, st, static_cast<const T*>(q),
                     static_cast<const T*>(k), static_cast<const T*>(v), g, beta, cu, Hk, Hv, state,
                     has_init, static_cast<T*>(o));
  return hipGetLastError();
}

}  // namespace

// Device scratch of the no-allocation segmented prefill: the X, R and P
// matrices that the allocating entry point keeps in its caller's workspace,
// at most GDN_NOALLOC_SCRATCH_BYTES.  Each GPU the library runs on holds its
// own copy until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: kernels get the address that
// hipGetSymbolAddress returns for the device.
static __device__ __align__(256) float scratch[GDN_NOALLOC_SCRATCH_BYTES / sizeof(float)];

hipError_t noalloc_scratch(hipStream_t st, float** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = st != nullptr ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // once per device, with that device current
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<float*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_prefill_segmented(const void* q, const void* k, const void* v, const float* g,
                                    const float* beta, const int32_t* cu, int nseq, int Hk, int Hv,
                                    float* state, const uint8_t* has_init, void* o, int nseg,
                                    float* ws, hipStream_t st) {
  hipError_t e = launch_ws<1, 1>(q, k, v, g, beta, cu, nseq, Hk, Hv, state, has_init, o, nseg, ws, st);
  if (e != hipSuccess) return e;
  if (nseg > 2) {
    hipLaunchKernelGGL(seg_combine_kernel, dim3(nseq * Hv * 8), dim3(256), 0, st, ws, nseq, nseg, Hv);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_ws<1, 2>(q, k, v, g, beta, cu, nseq, Hk, Hv, state, has_init, o, nseg, ws, st);
}

hipError_t launch_prefill(const void* q, const void* k, const void* v, int act, const float* g,
                          const float* beta, const int32_t* cu, int nseq, int Hk, int Hv,
                          float* state, const uint8_t* has_init, void* o, hipStream_t st) {
  // float32 activations take the single-role schedule: three K/Q buffers of
  // 4-byte elements do not fit in LDS.
  if (act == GDN_F32) return launch_t<float, 4, 1>(q, k, v, g, beta, cu, nseq, Hk, Hv, state, has_init, o, st);
  return launch_ws<1, 0>(q, k, v, g, beta, cu, nseq, Hk, Hv, state, has_init, o, 1, nullptr, st);
}

}  // namespace gdn
