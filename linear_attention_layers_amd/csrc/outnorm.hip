// Gated output norm after the recurrence (gfx950).
//
// "Strata pull request 3226", "Summary" item 2 and "Code Object Resource
// Usage": an output-norm kernel consumes the recurrence output o and a gate
// operand z; the pages print no formula.  Reading (the plainest one the rest
// supports): per token and v-head, root-mean-square normalisation of o over
// its 128 channels, an optional per-channel weight w, and the gate SiLU(z):
//   y_i = o_i / sqrt(mean_j(o_j^2) + eps) * w_i * SiLU(z_i).
//
// Layout.  One 16-lane row per (token, v-head): lane j holds channels
// 8 j .. 8 j + 7, so the sum of squares is the post-conv kernel's row
// reduction (neighbours first).  A 256-thread workgroup covers 16 rows.
// Every access goes through a buffer resource spanning exactly the rows, so
// the tail of the last workgroup reads zeros and its stores are dropped.
// Each lane reads its own elements before writing them, so y may be o
// (in place).  The kernel streams o and z in and y out: HBM-bound.
#include "launch.hpp"
#include "mfma.hpp"

namespace gdn {

namespace {

// 8 consecutive elements through a buffer resource, as float
template <class T> struct Buf8;
template <> struct Buf8<uint16_t> {
  __device__ __forceinline__ static void load(__amdgpu_buffer_rsrc_t r, int off, float (&v)[8]) {
    const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32(u[i] & 0xffffu);
      v[2 * i + 1] = bf16_to_f32(u[i] >> 16);
    }
  }
  __device__ __forceinline__ static void store(__amdgpu_buffer_rsrc_t r, int off, const float (&v)[8]) {
    const u32x4 u{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                  pack_bf16x2(v[6], v[7])};
    __builtin_amdgcn_raw_buffer_store_b128(u, r, off, 0, 0);
  }
};
template <> struct Buf8<float> {
  __device__ __forceinline__ static void load(__amdgpu_buffer_rsrc_t r, int off, float (&v)[8]) {
    const f32x4 a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    const f32x4 b = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
  __device__ __forceinline__ static void store(__amdgpu_buffer_rsrc_t r, int off, const float (&v)[8]) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]}), r, off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{v[4], v[5], v[6], v[7]}), r, off + 16, 0,
                                           0);
  }
};

template <class T>
__global__ __launch_bounds__(256) void out_norm_kernel(const T* __restrict__ o, const T* __restrict__ z,
                                                      const float* __restrict__ w, int rows, float eps,
                                                      T* y) {
  constexpr int ES = sizeof(T);
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int jl = threadIdx.x & 15;
  const int bytes = rows * 128 * ES;
  const auto ro = buf_rsrc(o, bytes);
  const auto rz = buf_rsrc(z, bytes);
  const auto ry = buf_rsrc(y, bytes);
  const bool has_w = w != nullptr;
  const auto rw = buf_rsrc(w, has_w ? 128 * 4 : 0);
  const int off = (row * 128 + 8 * jl) * ES;
  float ov[8], zv[8];
  Buf8<T>::load(ro, off, ov);
  Buf8<T>::load(rz, off, zv);
  const f32x4 w0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, 32 * jl, 0, 0));
  const f32x4 w1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, 32 * jl + 16, 0, 0));
  // mean of squares over the head's 128 channels (1/128 is exact)
  const float inv = 1.0f / __builtin_sqrtf(head_sum_sq<float>(ov) * (1.0f / 128.0f) + eps);
  float yv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float wi = has_w ? (i < 4 ? w0[i] : w1[i - 4]) : 1.0f;
    yv[i] = ov[i] * inv * wi * silu<T>(zv[i]);
  }
  Buf8<T>::store(ry, off, yv);
}

}  // namespace

hipError_t launch_out_norm(const void* o, const void* z, int act, const float* w, int rows, float eps,
                           void* y, hipStream_t st) {
  const dim3 grid((rows + 15) / 16);
  if (act == GDN_F32)
    hipLaunchKernelGGL(out_norm_kernel<float>, grid, dim3(256), 0, st, static_cast<const float*>(o),
                       static_cast<const float*>(z), w, rows, eps, static_cast<float*>(y));
  else
    hipLaunchKernelGGL(out_norm_kernel<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(o),
                       static_cast<const uint16_t*>(z), w, rows, eps, static_cast<uint16_t*>(y));
  return hipGetLastError();
}

}  // namespace gdn
