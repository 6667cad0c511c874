// Post-conv step (gfx950): SiLU on all channels, q|k|v split, per-head L2
// norm of q and k ("perf(gdn): optimize post-conv and causal-conv kernels",
// review sections "What I verified" and "The one thing I changed in your
// tests").
//
// Layout: each lane owns 8 adjacent channels (one 16-byte load of bf16, two
// of float32), so a 128-channel head is one 16-lane DPP row and a wave
// covers 4 heads.  Heads never straddle a row because every region starts
// at a multiple of 128 channels.  A workgroup of 256 lanes covers 2048
// channels of a few tokens.
//
// Documented order of a head's squared norm (all float32, no fused
// multiply-add): each lane squares its 8 elements and adds them as a
// neighbours-first tree ((e0+e1)+(e2+e3))+((e4+e5)+(e6+e7)); the 16 lane
// partials are then combined by xor-1, xor-2, xor-4, xor-8 DPP butterflies.
// Together this is the pairwise tree over the 128 elements in which level l
// adds adjacent blocks of 2^l elements.  inv = 1/sqrt(sum + eps), with
// correctly rounded sqrt and division for a float32 output and the hardware
// reciprocal square root for a bf16 output; q_hat = s * inv.
#include "device_common.hpp"
#include "launch.hpp"

namespace gdn {

namespace {

constexpr int kPostThreads = 256;
constexpr int kPostChannelsPerBlock = kPostThreads * 8;
constexpr int kPostTokensPerBlock = 4;

template <class TI, class TO>
__global__ __launch_bounds__(kPostThreads) void postconv_kernel(
    const TI* __restrict__ y, int64_t ys, int N, int C, int Hk, int Hv, float eps,
    TO* __restrict__ q, TO* __restrict__ k, TO* __restrict__ v) {
  // 1-D grid: channel group fastest, token blocks last to first, so the
  // running workgroups cover whole rows (as the conv launches do)
  const int ngroups = (C + kPostChannelsPerBlock - 1) / kPostChannelsPerBlock;
  const int ntb = (N + kPostTokensPerBlock - 1) / kPostTokensPerBlock;
  const int b = __builtin_amdgcn_readfirstlane((int)blockIdx.x);
  const int r = b / ngroups;
  const int c0 = ((b - r * ngroups) * kPostThreads + threadIdx.x) * 8;
  const bool active = c0 < C;
  const int qk = Hk * 128;
  const int t0 = (ntb - 1 - r) * kPostTokensPerBlock;

  float raw[kPostTokensPerBlock][8];
#pragma unroll
  for (int u = 0; u < kPostTokensPerBlock; ++u) {
    if (active && t0 + u < N) {
      Act<TI>::load8(y + (int64_t)(t0 + u) * ys + c0, raw[u]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) raw[u][i] = 0.f;
    }
  }
#pragma unroll
  for (int u = 0; u < kPostTokensPerBlock; ++u) {
    const int t = t0 + u;
    float s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = silu<TO>(raw[u][i]);
    // every lane takes part in the row reduction (DPP needs its partners)
    const float sum = head_sum_sq<TO>(s);
    if (!active || t >= N) continue;
    if (c0 < 2 * qk) {
      const float inv = l2_inv<TO>(sum, eps);
      float out[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = s[i] * inv;
      TO* dst = c0 < qk ? q + (int64_t)t * qk + c0 : k + (int64_t)t * qk + (c0 - qk);
      Act<TO>::store8(dst, out);
    } else {
      Act<TO>::store8(v + (int64_t)t * (Hv * 128) + (c0 - 2 * qk), s);
    }
  }
}

template <class TI, class TO>
hipError_t launch_t(const void* y, int64_t ys, int N, int Hk, int Hv, float eps, void* q, void* k,
                    void* v, hipStream_t st) {
  const int C = (2 * Hk + Hv) * 128;
  const int64_t nblk = (int64_t)((N + kPostTokensPerBlock - 1) / kPostTokensPerBlock) *
                      ((C + kPostChannelsPerBlock - 1) / kPostChannelsPerBlock);
  if (nblk == 0) return hipSuccess;
  if (nblk > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nblk);
  hipLaunchKernelGGL((postconv_kernel<TI, TO>), grid, dim3(kPostThreads), 0, st,
                     static_cast<const TI*>(y), ys, N, C, Hk, Hv, eps, static_cast<TO*>(q),
                     static_cast<TO*>(k), static_cast<TO*>(v));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_postconv(const void* y, int64_t ys, int in, int N, int Hk, int Hv, float eps,
                           void* q, void* k, void* v, int out, hipStream_t st) {
  if (in == GDN_F32 && out == GDN_F32) return launch_t<float, float>(y, ys, N, Hk, Hv, eps, q, k, v, st);
  if (in == GDN_F32 && out == GDN_BF16) return launch_t<float, uint16_t>(y, ys, N, Hk, Hv, eps, q, k, v, st);
  if (in == GDN_BF16 && out == GDN_F32) return launch_t<uint16_t, float>(y, ys, N, Hk, Hv, eps, q, k, v, st);
  return launch_t<uint16_t, uint16_t>(y, ys, N, Hk, Hv, eps, q, k, v, st);
}

}  // namespace gdn
