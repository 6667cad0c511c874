// Chunked gated delta-rule prefill (gfx950, MFMA).
//
// Recurrence (gated delta rule, Yang et al. 2024): per sequence and v-head,
//   S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t.
// The pages print no chunked algorithm (the Strata pull request 3226 leaves
// its prefill kernels untouched, "What This Does NOT Fix"); this kernel uses
// the chunk-64 WY form derived from the per-token rule.  For a chunk of n
// tokens (local index i) entering with state S0:
//   G_i = sum_{m<=i} g_m,  gamma_i = exp(G_i),  d_i = exp(G_{n-1} - G_i)
//   A_ij = b_i exp(G_i - G_j) (k_i . k_j)  (j < i),   T = (I + A)^-1
//   Z = K S0^T,   R_i = b_i (v_i - gamma_i Z_i),   U = T R
//   O = diag(gamma) Q S0^T + P U,  P_ij = exp(G_i - G_j) (q_i . k_j) (j <= i)
//   S = gamma_{n-1} S0 + (U^T diag(d)) K
// (U = T diag(b) V - T diag(b gamma) K S0^T is the usual WY factor; writing it
// as T R needs no separate W = T diag(b gamma) K.)
//
// Work split: rows of S (the dv index) evolve independently, so one
// workgroup owns one (sequence, v-head, slice of DVS state rows) and walks
// the sequence's chunks in order, carrying its DVS x 128 float32 slice of S
// in MFMA accumulator registers.  Per chunk, everything is staged in LDS:
// K, K^T, Q (bf16 exact), V slice, then K K^T and Q K^T (MFMA), the decay /
// beta scaling, the unit-lower-triangular inverse (16x16 diagonal blocks by
// forward substitution in one wave, off-diagonal blocks by block forward
// substitution), and the state-dependent products Z, Q S0^T, U, O and the
// state update (MFMA).
//
// Precision: with bf16 activations the contractions run on
// v_mfma_f32_16x16x32_bf16.  Operands that are bf16 inputs (K, Q) are exact;
// float32 operands (T, P, R, U, S0) are split into hi + lo bf16 parts and
// multiplied as hi*hi + hi*lo + lo*hi, i.e. about 16 significant bits per
// operand with float32 accumulation.  With float32 activations every
// product uses v_mfma_f32_16x16x4_f32.
#include "device_common.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int BT = 64;    // chunk length
constexpr int DK = 128;   // head size
constexpr int NW = 4;     // waves per workgroup
constexpr int NT = NW * 64;

struct ModeBF16 {
  using elem = uint16_t;
  static constexpr int KS = 32;
  static constexpr int PAD = 8;
  static constexpr bool kSplit = true;
};
struct ModeF32 {
  using elem = float;
  static constexpr int KS = 4;
  static constexpr int PAD = 4;
  static constexpr bool kSplit = false;
};

// An LDS matrix operand: element (row i, contraction index k) is at
// hi[i * rs + k * cs]; lo (bf16 mode only, may be null) holds the residual.
template <class M> struct Opnd {
  const typename M::elem* hi;
  const typename M::elem* lo;
  int rs, cs;
};

__device__ __forceinline__ f32x4 mfma_bf16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// acc += A[i0 .. i0+15][k0 .. k1) * B^T[j0 .. j0+15][k0 .. k1)^T.
// Lane l supplies row (l % 16) of A and of B^T for contraction slice l / 16;
// the accumulator holds D[4 (l / 16) + e][l % 16] in element e.
template <class M>
__device__ __forceinline__ f32x4 mma(f32x4 acc, const Opnd<M>& A, int i0, const Opnd<M>& B, int j0,
                                     int k0, int k1, int lane) {
  const int r = lane & 15, kg = lane >> 4;
  if constexpr (M::kSplit) {
    for (int kk = k0; kk < k1; kk += 32) {
      const int off = kk + 8 * kg;
      const uint4 ah = *reinterpret_cast<const uint4*>(A.hi + (i0 + r) * A.rs + off);
      const uint4 bh = *reinterpret_cast<const uint4*>(B.hi + (j0 + r) * B.rs + off);
      if (A.lo != nullptr) {
        const uint4 al = *reinterpret_cast<const uint4*>(A.lo + (i0 + r) * A.rs + off);
        acc = mfma_bf16(al, bh, acc);
      }
      if (B.lo != nullptr) {
        const uint4 bl = *reinterpret_cast<const uint4*>(B.lo + (j0 + r) * B.rs + off);
        acc = mfma_bf16(ah, bl, acc);
      }
      acc = mfma_bf16(ah, bh, acc);
    }
  } else {
    for (int kk = k0; kk < k1; kk += 4) {
      const float a = A.hi[(i0 + r) * A.rs + (kk + kg) * A.cs];
      const float b = B.hi[(j0 + r) * B.rs + (kk + kg) * B.cs];
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
  }
  return acc;
}

// Store a float32 value into an operand matrix (split into hi/lo in bf16 mode).
template <class M>
__device__ __forceinline__ void put(typename M::elem* hi, typename M::elem* lo, int idx, float x) {
  if constexpr (M::kSplit) {
    const uint32_t h = f32_to_bf16(x);
    hi[idx] = static_cast<uint16_t>(h);
    lo[idx] = static_cast<uint16_t>(f32_to_bf16(x - bf16_to_f32(h)));
  } else {
    hi[idx] = x;
  }
}

template <class M>
__device__ __forceinline__ float get(const typename M::elem* hi, const typename M::elem* lo, int idx) {
  if constexpr (M::kSplit) {
    return bf16_to_f32(hi[idx]) + bf16_to_f32(lo[idx]);
  } else {
    return hi[idx];
  }
}

template <class M, int DVS> struct __attribute__((aligned(16))) Smem {
  static constexpr int LDK = DK + M::PAD;   // 128-wide rows
  static constexpr int LDT = BT + M::PAD;   // 64-wide rows
  static constexpr int NS = M::kSplit ? 2 : 1;
  using E = typename M::elem;
  E K[BT * LDK];                          // K rows (token, feature)
  E KT[M::kSplit ? DK * LDT : 4];         // K^T (feature, token), bf16 mode only
  E Q[BT * LDK];
  E V[BT * DVS];                          // this slice of V (token, row)
  float A[BT * (BT + 1)];                 // K K^T, then the scaled strict lower part A
  E T[NS * BT * LDT];                     // (I + A)^-1
  E P[NS * BT * LDT];                     // masked, decayed Q K^T
  E RT[NS * DVS * LDT];                   // R^T (row, token)
  E UT[NS * DVS * LDT];                   // U^T
  union {
    E UdT[NS * DVS * LDT];                // U^T diag(d)
    float X[NW * 16 * 17];                // per-wave scratch of the triangular solve
  };
  E S[NS * DVS * LDK];                    // S0 slice (row, feature)
  float G[BT], Gam[BT], Beta[BT], D[BT];
  float gamma_last;
};

template <class T> struct ModeOf;
template <> struct ModeOf<uint16_t> { using type = ModeBF16; static constexpr int DVS = 32; };
template <> struct ModeOf<float> { using type = ModeF32; static constexpr int DVS = 16; };

template <class T>
__global__ __launch_bounds__(NT) void prefill_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
    int Hk, int Hv, float* state, const uint8_t* __restrict__ has_init, T* __restrict__ o) {
  using M = typename ModeOf<T>::type;
  constexpr int DVS = ModeOf<T>::DVS;
  using SM = Smem<M, DVS>;
  using E = typename M::elem;
  constexpr int LDK = SM::LDK, LDT = SM::LDT;
  constexpr int NSL = DK / DVS;            // slices per head
  constexpr int NVB = DVS / 16;            // 16-row blocks per slice
  constexpr int NZ = (BT / 16) * NVB;      // (token block, row block) tiles of Z / O
  constexpr int NSTILE = NVB * (DK / 16);  // tiles of the state slice
  constexpr int ZPW = (NZ + NW - 1) / NW;
  constexpr int SPW = NSTILE / NW;
  static_assert(NSTILE % NW == 0, "state tiles must split evenly over waves");

  __shared__ SM sm;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, kg = lane >> 4;

  int bid = blockIdx.x;
  const int slice = bid % NSL;
  bid /= NSL;
  const int h = bid % Hv;
  const int s = bid / Hv;
  const int kh = h / (Hv / Hk);
  const int v0 = slice * DVS;
  const int bos = cu[s], eos = cu[s + 1];

  constexpr int NS = SM::NS;
  E* const Thi = sm.T;
  E* const Tlo = M::kSplit ? sm.T + BT * LDT : nullptr;
  E* const Phi = sm.P;
  E* const Plo = M::kSplit ? sm.P + BT * LDT : nullptr;
  E* const RThi = sm.RT;
  E* const RTlo = M::kSplit ? sm.RT + DVS * LDT : nullptr;
  E* const UThi = sm.UT;
  E* const UTlo = M::kSplit ? sm.UT + DVS * LDT : nullptr;
  E* const UdThi = sm.UdT;
  E* const UdTlo = M::kSplit ? sm.UdT + DVS * LDT : nullptr;
  E* const Shi = sm.S;
  E* const Slo = M::kSplit ? sm.S + DVS * LDK : nullptr;
  (void)NS;

  // T and P are lower triangular; their upper 16x16 blocks are read as zeros
  // by the rounded-up contraction ranges and are never written afterwards.
  for (int idx = tid; idx < BT * LDT; idx += NT) {
    Thi[idx] = E(0); Phi[idx] = E(0);
    if constexpr (M::kSplit) { Tlo[idx] = E(0); Plo[idx] = E(0); }
  }

  // ---- initial state slice into accumulators (and LDS as an operand)
  f32x4 Sacc[SPW];
  const bool init = has_init == nullptr || has_init[s] != 0;
  float* const sbase = state + ((int64_t)s * Hv + h) * (DK * DK) + (int64_t)v0 * DK;
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int ts = wave + NW * j;
    const int tv = ts / (DK / 16), tc = ts % (DK / 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int vr = 16 * tv + 4 * kg + e, c = 16 * tc + r16;
      Sacc[j][e] = init ? sbase[vr * DK + c] : 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int ts = wave + NW * j;
    const int tv = ts / (DK / 16), tc = ts % (DK / 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) put<M>(Shi, Slo, (16 * tv + 4 * kg + e) * LDK + 16 * tc + r16, Sacc[j][e]);
  }

  const Opnd<M> opK{sm.K, nullptr, LDK, 1};
  const Opnd<M> opQ{sm.Q, nullptr, LDK, 1};
  const Opnd<M> opS{Shi, Slo, LDK, 1};
  const Opnd<M> opT{Thi, Tlo, LDT, 1};
  const Opnd<M> opP{Phi, Plo, LDT, 1};
  const Opnd<M> opRT{RThi, RTlo, LDT, 1};
  const Opnd<M> opUT{UThi, UTlo, LDT, 1};
  const Opnd<M> opUdT{UdThi, UdTlo, LDT, 1};
  // B operand of the state update: element (feature c, token m) = K[m][c]
  const Opnd<M> opKT = M::kSplit ? Opnd<M>{sm.KT, nullptr, LDT, 1} : Opnd<M>{sm.K, nullptr, 1, LDK};

  for (int c0 = bos; c0 < eos; c0 += BT) {
    const int n = min(BT, eos - c0);
    __syncthreads();  // the previous chunk is done with every LDS buffer

    // ---- 1. stage K, K^T, Q, V slice, g, beta
    for (int it = tid; it < BT * (DK / 8); it += NT) {
      const int row = it / (DK / 8), c8 = (it % (DK / 8)) * 8;
      float kv[8], qv[8];
      if (row < n) {
        const int64_t off = ((int64_t)(c0 + row) * Hk + kh) * DK + c8;
        Act<T>::load8(k + off, kv);
        Act<T>::load8(q + off, qv);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) { kv[i] = 0.f; qv[i] = 0.f; }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (M::kSplit) {
          const uint16_t kb = static_cast<uint16_t>(f32_to_bf16(kv[i]));  // exact: kv came from bf16
          sm.K[row * LDK + c8 + i] = kb;
          sm.KT[(c8 + i) * LDT + row] = kb;
          sm.Q[row * LDK + c8 + i] = static_cast<uint16_t>(f32_to_bf16(qv[i]));
        } else {
          sm.K[row * LDK + c8 + i] = kv[i];
          sm.Q[row * LDK + c8 + i] = qv[i];
        }
      }
    }
    for (int it = tid; it < BT * (DVS / 8); it += NT) {
      const int row = it / (DVS / 8), c8 = (it % (DVS / 8)) * 8;
      float vv[8];
      if (row < n) {
        Act<T>::load8(v + ((int64_t)(c0 + row) * Hv + h) * DK + v0 + c8, vv);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) vv[i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (M::kSplit) sm.V[row * DVS + c8 + i] = static_cast<uint16_t>(f32_to_bf16(vv[i]));
        else sm.V[row * DVS + c8 + i] = vv[i];
      }
    }
    if (tid < BT) {
      const bool ok = tid < n;
      sm.G[tid] = ok ? g[(int64_t)(c0 + tid) * Hv + h] : 0.f;
      sm.Beta[tid] = ok ? beta[(int64_t)(c0 + tid) * Hv + h] : 0.f;
    }
    __syncthreads();

    // ---- 2. cumulative log-decay (wave 0) and K K^T, Q K^T lower tiles
    if (wave == 0) {
      float gv = sm.G[lane];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float t = __shfl_up(gv, off, 64);
        if (lane >= off) gv += t;
      }
      const float glast = __shfl(gv, n - 1, 64);
      sm.G[lane] = gv;
      sm.Gam[lane] = expf(gv);
      sm.D[lane] = lane < n ? expf(glast - gv) : 0.f;
      if (lane == 0) sm.gamma_last = expf(glast);
    }
    // 10 lower tiles of K K^T (jobs 0..9) and of Q K^T (jobs 10..19)
    constexpr int NJOB = 20;
    constexpr int JPW = (NJOB + NW - 1) / NW;
    f32x4 jacc[JPW];
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      const int job = wave + NW * jj;
      jacc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (job < NJOB) {
        const int t = job % 10;
        int bi = 0;
        while ((bi + 1) * (bi + 2) / 2 <= t) ++bi;
        const int bj = t - bi * (bi + 1) / 2;
        jacc[jj] = mma<M>(jacc[jj], job < 10 ? opK : opQ, 16 * bi, opK, 16 * bj, 0, DK, lane);
      }
    }
    __syncthreads();
#pragma unroll
    for (int jj = 0; jj < JPW; ++jj) {
      const int job = wave + NW * jj;
      if (job < NJOB) {
        const int t = job % 10;
        int bi = 0;
        while ((bi + 1) * (bi + 2) / 2 <= t) ++bi;
        const int bj = t - bi * (bi + 1) / 2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * bi + 4 * kg + e, j = 16 * bj + r16;
          const float decay = j <= i ? expf(sm.G[i] - sm.G[j]) : 0.f;
          if (job < 10) {
            sm.A[i * (BT + 1) + j] = j < i ? sm.Beta[i] * decay * jacc[jj][e] : 0.f;
          } else {
            put<M>(Phi, Plo, i * LDT + j, decay * jacc[jj][e]);
          }
        }
      }
    }
    __syncthreads();

    // ---- 3. T = (I + A)^-1
    // 3a. diagonal 16x16 blocks, one per 16-lane group of wave 0: lane
    //     (blk, col) forward-substitutes column col of block blk.
    if (wave == 0) {
      const int blk = kg, col = r16, base = 16 * blk;
      float xcol[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = (i == col) ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < i; ++j) acc -= sm.A[(base + i) * (BT + 1) + base + j] * xcol[j];
        xcol[i] = acc;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) put<M>(Thi, Tlo, (base + i) * LDT + base + col, xcol[i]);
    }
    __syncthreads();
    // 3b. off-diagonal blocks by block forward substitution, level by level:
    //     T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj   (block indices, i - j = lvl)
    for (int lvl = 1; lvl < 4; ++lvl) {
      const int bi = lvl + wave, bj = wave;
      const bool active = bi < 4;
      float* X = sm.X + wave * (16 * 17);
      if (active) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = 4 * kg + e, cc = r16;
          float acc = 0.f;
          for (int bm = bj; bm < bi; ++bm) {
#pragma unroll
            for (int m = 0; m < 16; ++m)
              acc += sm.A[(16 * bi + rr) * (BT + 1) + 16 * bm + m] *
                     get<M>(Thi, Tlo, (16 * bm + m) * LDT + 16 * bj + cc);
          }
          X[rr * 17 + cc] = acc;
        }
      }
      __syncthreads();
      if (active) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = 4 * kg + e, cc = r16;
          float acc = 0.f;
#pragma unroll
          for (int m = 0; m < 16; ++m)
            acc += get<M>(Thi, Tlo, (16 * bi + rr) * LDT + 16 * bi + m) * X[m * 17 + cc];
          put<M>(Thi, Tlo, (16 * bi + rr) * LDT + 16 * bj + cc, -acc);
        }
      }
      __syncthreads();
    }

    // ---- 4. Z = K S0^T and QS = Q S0^T; R = diag(b) (V - diag(gamma) Z)
    f32x4 QS[ZPW];
#pragma unroll
    for (int jj = 0; jj < ZPW; ++jj) {
      const int tz = wave + NW * jj;
      QS[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (tz < NZ) {
        const int ti = tz / NVB, tv = tz % NVB;
        f32x4 z = mma<M>(f32x4{0.f, 0.f, 0.f, 0.f}, opK, 16 * ti, opS, 16 * tv, 0, DK, lane);
        QS[jj] = mma<M>(QS[jj], opQ, 16 * ti, opS, 16 * tv, 0, DK, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * ti + 4 * kg + e, vr = 16 * tv + r16;
          float vv;
          if constexpr (M::kSplit) vv = bf16_to_f32(sm.V[i * DVS + vr]);
          else vv = sm.V[i * DVS + vr];
          const float rv = sm.Beta[i] * (vv - sm.Gam[i] * z[e]);
          put<M>(RThi, RTlo, vr * LDT + i, rv);
        }
      }
    }
    __syncthreads();

    // ---- 5. U = T R  (T is lower triangular: row block ti needs tokens < 16 (ti+1))
#pragma unroll
    for (int jj = 0; jj < ZPW; ++jj) {
      const int tz = wave + NW * jj;
      if (tz < NZ) {
        const int ti = tz / NVB, tv = tz % NVB;
        const int kend = ((16 * (ti + 1) + M::KS - 1) / M::KS) * M::KS;
        f32x4 u = mma<M>(f32x4{0.f, 0.f, 0.f, 0.f}, opT, 16 * ti, opRT, 16 * tv, 0, kend, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * ti + 4 * kg + e, vr = 16 * tv + r16;
          put<M>(UThi, UTlo, vr * LDT + i, u[e]);
          put<M>(UdThi, UdTlo, vr * LDT + i, u[e] * sm.D[i]);
        }
      }
    }
    __syncthreads();

    // ---- 6. O = diag(gamma) QS + P U, and S = gamma_last S0 + (U^T diag(d)) K
#pragma unroll
    for (int jj = 0; jj < ZPW; ++jj) {
      const int tz = wave + NW * jj;
      if (tz < NZ) {
        const int ti = tz / NVB, tv = tz % NVB;
        const int kend = ((16 * (ti + 1) + M::KS - 1) / M::KS) * M::KS;
        f32x4 pu = mma<M>(f32x4{0.f, 0.f, 0.f, 0.f}, opP, 16 * ti, opUT, 16 * tv, 0, kend, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * ti + 4 * kg + e, vr = 16 * tv + r16;
          if (i < n) {
            const float ov = sm.Gam[i] * QS[jj][e] + pu[e];
            Act<T>::store1(o + ((int64_t)(c0 + i) * Hv + h) * DK + v0 + vr, ov);
          }
        }
      }
    }
    const float gl = sm.gamma_last;
#pragma unroll
    for (int j = 0; j < SPW; ++j) {
      const int ts = wave + NW * j;
      const int tv = ts / (DK / 16), tc = ts % (DK / 16);
      f32x4 acc;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = gl * Sacc[j][e];
      Sacc[j] = mma<M>(acc, opUdT, 16 * tv, opKT, 16 * tc, 0, BT, lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) put<M>(Shi, Slo, (16 * tv + 4 * kg + e) * LDK + 16 * tc + r16, Sacc[j][e]);
    }
  }

  // ---- final state slice
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int ts = wave + NW * j;
    const int tv = ts / (DK / 16), tc = ts % (DK / 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) sbase[(16 * tv + 4 * kg + e) * DK + 16 * tc + r16] = Sacc[j][e];
  }
}

}  // namespace

hipError_t launch_prefill(const void* q, const void* k, const void* v, int act, const float* g,
                          const float* beta, const int32_t* cu, int nseq, int Hk, int Hv,
                          float* state, const uint8_t* has_init, void* o, hipStream_t st) {
  if (act == GDN_F32) {
    dim3 grid(nseq * Hv * (DK / ModeOf<float>::DVS));
    hipLaunchKernelGGL(prefill_kernel<float>, grid, dim3(NT), 0, st, static_cast<const float*>(q),
                       static_cast<const float*>(k), static_cast<const float*>(v), g, beta, cu, Hk,
                       Hv, state, has_init, static_cast<float*>(o));
  } else {
    dim3 grid(nseq * Hv * (DK / ModeOf<uint16_t>::DVS));
    hipLaunchKernelGGL(prefill_kernel<uint16_t>, grid, dim3(NT), 0, st,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), g, beta, cu, Hk, Hv, state, has_init,
                       static_cast<uint16_t*>(o));
  }
  return hipGetLastError();
}

}  // namespace gdn
