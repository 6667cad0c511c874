// Gate computation before the recurrence (gfx950).
//
// "Strata pull request 3226", "Root Cause & RED / GREEN Verification", and
// "perf(gdn): optimize post-conv and causal-conv kernels", "The one thing I
// changed in your tests", name gate kernels on a packed float32 (b, a)
// input with a bf16 gate-type instantiation; the pages print no formula.
// Reading (as in the Gated DeltaNet layer): per token t and v-head h, from
// ba[t][h] = (b, a) and the per-head parameters A_log, dt_bias,
//   beta = sigmoid(b),   g = log a_t = -exp(A_log[h]) * softplus(a + dt_bias[h]).
// One lane per (token, head), grid-stride; the HIP math library's expf and
// log1pf; softplus(x) = x above 20, where log1p(e^x) - x < 3e-9.
#include "launch.hpp"
#include "mfma.hpp"

namespace gdn {

namespace {

template <class TG> struct Pair;
template <> struct Pair<float> {
  __device__ __forceinline__ static void load(const float* p, int i, float& b, float& a) {
    const float2 v = reinterpret_cast<const float2*>(p)[i];
    b = v.x;
    a = v.y;
  }
};
template <> struct Pair<uint16_t> {
  __device__ __forceinline__ static void load(const uint16_t* p, int i, float& b, float& a) {
    const uint32_t v = reinterpret_cast<const uint32_t*>(p)[i];
    b = bf16_to_f32(v & 0xffffu);
    a = bf16_to_f32(v >> 16);
  }
};

template <class TG>
__global__ __launch_bounds__(256) void gates_kernel(const TG* __restrict__ ba, const float* __restrict__ A_log,
                                                   const float* __restrict__ dt_bias, int rows, int Hv,
                                                   float* __restrict__ g, float* __restrict__ beta) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < rows; i += gridDim.x * 256) {
    const int h = i % Hv;
    float b, a;
    Pair<TG>::load(ba, i, b, a);
    const float x = a + dt_bias[h];
    const float sp = x > 20.f ? x : log1pf(expf(x));
    g[i] = -expf(A_log[h]) * sp;
    beta[i] = 1.f / (1.f + expf(-b));
  }
}

}  // namespace

hipError_t launch_gates(const void* ba, int gate_act, const float* A_log, const float* dt_bias, int rows,
                        int Hv, float* g, float* beta, hipStream_t st) {
  const dim3 grid(min((rows + 255) / 256, 4096));
  if (gate_act == GDN_F32)
    hipLaunchKernelGGL(gates_kernel<float>, grid, dim3(256), 0, st, static_cast<const float*>(ba), A_log,
                       dt_bias, rows, Hv, g, beta);
  else
    hipLaunchKernelGGL(gates_kernel<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(ba),
                       A_log, dt_bias, rows, Hv, g, beta);
  return hipGetLastError();
}

}  // namespace gdn
