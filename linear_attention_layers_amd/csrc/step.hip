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
// Recurrence (gated delta rule), per row i of the dv x dk state S:
//   u_i = S_i . k,   w_i = S_i . q,   kq = k . q
//   d_i = b (v_i - a u_i)
//   S_i <- a S_i + d_i k          (= a S_i (I - b k k^T) + b v_i k^T)
//   o_i  = a w_i + d_i kq         (= S_i q after the update)
//
// Layout: one workgroup of 256 lanes per (sequence, v-head).  Lane (rg, cl)
// = (tid / 16, tid % 16) holds rows rg + 16 r (r = 0..7) and columns
// 8 cl .. 8 cl + 7 of S in 64 registers, loaded once with 16-byte accesses
// (16 lanes cover one 512-byte row).  Each token needs the 17 row dot
// products above; each is 8 in-lane FMAs and a 16-lane DPP reduction in the
// fixed xor order, so the state never leaves registers between tokens and
// there is no barrier in the token loop.  All arithmetic in the update is
// written as explicit fmaf / mul so the step and the commit replay (the same
// function) are bitwise identical.
#include "device_common.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int kStepThreads = 256;

struct StateRegs {
  float s[8][8];  // [row r][column j]
};

__device__ __forceinline__ void load_state(const float* __restrict__ base, int rg, int cl,
                                           StateRegs& S) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const float* p = base + (rg + 16 * r) * 128 + 8 * cl;
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    S.s[r][0] = a.x; S.s[r][1] = a.y; S.s[r][2] = a.z; S.s[r][3] = a.w;
    S.s[r][4] = b.x; S.s[r][5] = b.y; S.s[r][6] = b.z; S.s[r][7] = b.w;
  }
}

__device__ __forceinline__ void store_state(float* __restrict__ base, int rg, int cl,
                                            const StateRegs& S) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    float* p = base + (rg + 16 * r) * 128 + 8 * cl;
    *reinterpret_cast<float4*>(p) = make_float4(S.s[r][0], S.s[r][1], S.s[r][2], S.s[r][3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(S.s[r][4], S.s[r][5], S.s[r][6], S.s[r][7]);
  }
}

// Runs tokens [t_begin, t_end) of one (sequence, v-head) through the state
// held in S.  When WRITE_O, o[t][h][row] is written by lane cl == r.
template <class T, bool WRITE_O>
__device__ __forceinline__ void run_tokens(StateRegs& S, const T* __restrict__ q,
                                           const T* __restrict__ k, const T* __restrict__ v,
                                           const float* __restrict__ g,
                                           const float* __restrict__ beta, T* __restrict__ o,
                                           int t_begin, int t_end, int Hk, int Hv, int h, int kh,
                                           int rg, int cl) {
#pragma clang fp contract(off)
  for (int t = t_begin; t < t_end; ++t) {
    float kv[8], qv[8];
    Act<T>::load8(k + ((int64_t)t * Hk + kh) * 128 + 8 * cl, kv);
    if (WRITE_O) {
      Act<T>::load8(q + ((int64_t)t * Hk + kh) * 128 + 8 * cl, qv);
    }
    float vr[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) vr[r] = Act<T>::load1(v + ((int64_t)t * Hv + h) * 128 + rg + 16 * r);
    const float a = expf(g[(int64_t)t * Hv + h]);
    const float b = beta[(int64_t)t * Hv + h];

    float u[8], w[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float pu = S.s[r][0] * kv[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) pu = __builtin_fmaf(S.s[r][j], kv[j], pu);
      u[r] = pu;
      if (WRITE_O) {
        float pw = S.s[r][0] * qv[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) pw = __builtin_fmaf(S.s[r][j], qv[j], pw);
        w[r] = pw;
      }
    }
    float kq = 0.f;
    if (WRITE_O) {
      float p = kv[0] * qv[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) p = __builtin_fmaf(kv[j], qv[j], p);
      kq = row16_sum(p);
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      u[r] = row16_sum(u[r]);
      if (WRITE_O) w[r] = row16_sum(w[r]);
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float d = b * (vr[r] - a * u[r]);
#pragma unroll
      for (int j = 0; j < 8; ++j) S.s[r][j] = __builtin_fmaf(d, kv[j], a * S.s[r][j]);
      if (WRITE_O) {
        const float orow = __builtin_fmaf(d, kq, a * w[r]);
        if (cl == r) Act<T>::store1(o + ((int64_t)t * Hv + h) * 128 + rg + 16 * r, orow);
      }
    }
  }
}

template <class T>
__global__ __launch_bounds__(kStepThreads) void step_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
    int Hk, int Hv, float* state, const uint8_t* __restrict__ has_init, T* __restrict__ o,
    int commit_state) {
  const int s = blockIdx.x / Hv;
  const int h = blockIdx.x % Hv;
  const int kh = h / (Hv / Hk);
  const int rg = threadIdx.x >> 4, cl = threadIdx.x & 15;
  const int bos = cu[s], eos = cu[s + 1];
  if (eos <= bos) return;
  float* base = state + ((int64_t)s * Hv + h) * (128 * 128);
  StateRegs S;
  if (has_init == nullptr || has_init[s] != 0) {
    load_state(base, rg, cl, S);
  } else {
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int j = 0; j < 8; ++j) S.s[r][j] = 0.f;
  }
  run_tokens<T, true>(S, q, k, v, g, beta, o, bos, eos, Hk, Hv, h, kh, rg, cl);
  if (commit_state) store_state(base, rg, cl, S);
}

// One launch for all layers: block b covers (layer, sequence, role); roles
// 0..Hv-1 replay the state of v-head `role`, roles Hv.. shift the conv rows
// of one 2048-channel group.  A block whose sequence keeps no token exits
// before touching memory.
template <class T>
__global__ __launch_bounds__(kStepThreads) void commit_kernel(
    const gdn_layer_io* __restrict__ layers, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ n_keep, const uint8_t* __restrict__ has_init, int nseq, int C,
    int Hk, int Hv, int roles) {
  const int b = blockIdx.x;
  const int role = b % roles;
  const int s = (b / roles) % nseq;
  const int layer = b / (roles * nseq);
  const int n = n_keep[s];
  if (n <= 0) return;
  const gdn_layer_io io = layers[layer];
  const int bos = cu[s];
  const bool init = has_init == nullptr || has_init[s] != 0;
  if (role < Hv) {
    const int h = role;
    const int kh = h / (Hv / Hk);
    const int rg = threadIdx.x >> 4, cl = threadIdx.x & 15;
    float* base = io.state + ((int64_t)s * Hv + h) * (128 * 128);
    StateRegs S;
    if (init) {
      load_state(base, rg, cl, S);
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int j = 0; j < 8; ++j) S.s[r][j] = 0.f;
    }
    run_tokens<T, false>(S, nullptr, static_cast<const T*>(io.k), static_cast<const T*>(io.v),
                         io.g, io.beta, nullptr, bos, bos + n, Hk, Hv, h, kh, rg, cl);
    store_state(base, rg, cl, S);
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
  dim3 grid(nseq * Hv);
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
