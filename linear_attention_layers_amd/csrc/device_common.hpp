// Device helpers shared by the GDN kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- bfloat16
// bfloat16 is stored as its 16 raw bits (uint16_t).

__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// Two floats to packed bf16 (low half = a), round to nearest, ties to even:
// one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return pack_bf16x2(f, 0.f) & 0xffffu;
}

// Activation storage traits: load / store 8 consecutive elements as float.
template <class T> struct Act;

template <> struct Act<float> {
  static constexpr int kBytes = 4;
  // 8 elements in storage form
  struct Raw { float4 a, b; };
  __device__ __forceinline__ static Raw load_raw(const float* p) {
    Raw r;
    r.a = *reinterpret_cast<const float4*>(p);
    r.b = *reinterpret_cast<const float4*>(p + 4);
    return r;
  }
  __device__ __forceinline__ static void unpack(const Raw& r, float (&v)[8]) {
    v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
    v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
  }
  __device__ __forceinline__ static void load8(const float* p, float (&v)[8]) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ static void store8(float* p, const float (&v)[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
  __device__ __forceinline__ static float load1(const float* p) { return *p; }
  __device__ __forceinline__ static void store1(float* p, float v) { *p = v; }
};

template <> struct Act<uint16_t> {
  static constexpr int kBytes = 2;
  struct Raw { uint4 u; };
  __device__ __forceinline__ static Raw load_raw(const uint16_t* p) {
    Raw r;
    r.u = *reinterpret_cast<const uint4*>(p);
    return r;
  }
  __device__ __forceinline__ static void unpack(const Raw& r, float (&v)[8]) {
    v[0] = bf16_to_f32(r.u.x & 0xffffu); v[1] = bf16_to_f32(r.u.x >> 16);
    v[2] = bf16_to_f32(r.u.y & 0xffffu); v[3] = bf16_to_f32(r.u.y >> 16);
    v[4] = bf16_to_f32(r.u.z & 0xffffu); v[5] = bf16_to_f32(r.u.z >> 16);
    v[6] = bf16_to_f32(r.u.w & 0xffffu); v[7] = bf16_to_f32(r.u.w >> 16);
  }
  __device__ __forceinline__ static void load8(const uint16_t* p, float (&v)[8]) {
    uint4 u = *reinterpret_cast<const uint4*>(p);
    v[0] = bf16_to_f32(u.x & 0xffffu); v[1] = bf16_to_f32(u.x >> 16);
    v[2] = bf16_to_f32(u.y & 0xffffu); v[3] = bf16_to_f32(u.y >> 16);
    v[4] = bf16_to_f32(u.z & 0xffffu); v[5] = bf16_to_f32(u.z >> 16);
    v[6] = bf16_to_f32(u.w & 0xffffu); v[7] = bf16_to_f32(u.w >> 16);
  }
  __device__ __forceinline__ static void store8(uint16_t* p, const float (&v)[8]) {
    uint4 u;
    u.x = pack_bf16x2(v[0], v[1]);
    u.y = pack_bf16x2(v[2], v[3]);
    u.z = pack_bf16x2(v[4], v[5]);
    u.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = u;
  }
  __device__ __forceinline__ static float load1(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store1(uint16_t* p, float v) {
    *p = static_cast<uint16_t>(f32_to_bf16(v));
  }
};

// ------------------------------------------------------ per-sequence flag
// Byte s of a per-sequence uint8 array (NULL = every flag set).  The aligned
// dword that holds the byte is read instead of the byte: at a uniform
// address that is a scalar load, which arrives with the prologue's other
// scalar loads rather than as a vector load that everything after it on the
// in-order vector counter would wait behind.  A 4-byte-aligned dword never
// crosses a page, so reading the bytes beside the flag cannot fault.
__device__ __forceinline__ bool seq_flag(const uint8_t* __restrict__ f, int s) {
  if (f == nullptr) return true;
  const int sub = static_cast<int>((reinterpret_cast<uintptr_t>(f) + static_cast<uintptr_t>(s)) & 3);
  const uint32_t w = *reinterpret_cast<const uint32_t*>(f + s - sub);
  return ((w >> (8 * sub)) & 0xffu) != 0;
}

// ------------------------------------------------------- wave64 DPP moves
// Row-local (16-lane) data movement.  quad_perm xor-1 = 0xB1, xor-2 = 0x4E,
// row_half_mirror = 0x141 (lane i <- 7-i within 8), row_mirror = 0x140
// (lane i <- 15-i within 16); only controls whose every lane has a source
// lane in its row (quad permutations and mirrors).  For those the bound_ctrl
// bit changes no value, and with it set the compiler folds the move into the
// arithmetic that consumes it (one v_add_f32_dpp instead of a DPP move, two
// wait states and an add).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  static_assert((CTRL >= 0x00 && CTRL <= 0xFF) || CTRL == 0x140 || CTRL == 0x141,
                "dpp_mov is for quad permutations and row mirrors");
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Sum over the 16 lanes of a DPP row, result in every lane of the row.
// Order: lanes are combined neighbours first, xor 1, 2, 4, 8.  After each
// level all lanes of a group hold the same value, so the mirror moves used
// for the 4- and 8-lane levels fetch exactly the partner group's sum, and
// a + b == b + a keeps the lanes bit-identical.
__device__ __forceinline__ float row16_sum(float v) {
  v = v + dpp_mov<0xB1>(v);
  v = v + dpp_mov<0x4E>(v);
  v = v + dpp_mov<0x141>(v);
  v = v + dpp_mov<0x140>(v);
  return v;
}

// ---------------------------------------------------------- post-conv math
// Shared by the post-conv kernel and the fused decode kernel, so both give
// bit-identical q, k, v.  A head's 128 channels sit in one 16-lane DPP row,
// 8 adjacent channels per lane.
// SiLU for a float32 output is evaluated in float64 and rounded once, so the
// float32 output arm carries the correctly rounded activation; for a bf16
// output float32 arithmetic suffices (its error is far below a bf16 step).
template <class TO> __device__ __forceinline__ float silu(float y);
template <> __device__ __forceinline__ float silu<float>(float y) {
  const double d = static_cast<double>(y);
  return static_cast<float>(d / (1.0 + exp(-d)));
}
template <> __device__ __forceinline__ float silu<uint16_t>(float y) {
  // y * 1 / (1 + 2^(-y log2 e)) with the hardware exp2 and reciprocal (each
  // about 1 ulp): a few float32 ulps in all, far below a bf16 step.
  // Large |y| saturates correctly: 2^(+inf) = inf -> rcp = 0 -> -0.
  const float e = __builtin_amdgcn_exp2f(-y * 1.4426950408889634f);
  return y * __builtin_amdgcn_rcpf(1.0f + e);
}

// 1 / sqrt(sum + eps), the L2 scale of a q or k head.  A float32 output
// carries the correctly rounded square root and division.  A bf16 output
// takes the hardware reciprocal square root (about one float32 ulp, a
// single transcendental instead of the two correction sequences), whose
// error is far below a bf16 step; the argument is kept at or above the
// smallest normal float32.
template <class TO> __device__ __forceinline__ float l2_inv(float sum, float eps);
template <> __device__ __forceinline__ float l2_inv<float>(float sum, float eps) {
  return 1.0f / __builtin_sqrtf(sum + eps);
}
template <> __device__ __forceinline__ float l2_inv<uint16_t>(float sum, float eps) {
  return __builtin_amdgcn_rsqf(__builtin_fmaxf(sum + eps, 1.17549435e-38f));
}

// Sum of squares of a head's 128 channels (8 per lane, 16 lanes).  A float32
// output keeps the documented order: within the lane the pairwise tree
// ((s0^2 + s1^2) + (s2^2 + s3^2)) + ((s4^2 + s5^2) + (s6^2 + s7^2)), each
// square and sum rounded, then row16_sum.  A bf16 output only needs the sum
// far inside a bf16 step, so the lane's part is two fused multiply-add
// chains over channels 0-3 and 4-7, added (9 instead of 15 operations).
template <class TO> __device__ __forceinline__ float head_sum_sq(const float (&s)[8]);
template <> __device__ __forceinline__ float head_sum_sq<float>(const float (&s)[8]) {
#pragma clang fp contract(off)
  const float p0 = s[0] * s[0] + s[1] * s[1];
  const float p1 = s[2] * s[2] + s[3] * s[3];
  const float p2 = s[4] * s[4] + s[5] * s[5];
  const float p3 = s[6] * s[6] + s[7] * s[7];
  const float lane = (p0 + p1) + (p2 + p3);
  return row16_sum(lane);
}
template <> __device__ __forceinline__ float head_sum_sq<uint16_t>(const float (&s)[8]) {
  float a = s[0] * s[0], b = s[4] * s[4];
#pragma unroll
  for (int i = 1; i < 4; ++i) {
    a = __builtin_fmaf(s[i], s[i], a);
    b = __builtin_fmaf(s[4 + i], s[4 + i], b);
  }
  return row16_sum(a + b);
}


// q_hat (is_qk) or v of one lane's 8 channels from its 8 conv outputs
// (already in the activation dtype); every lane of the row must call it.
template <class TO>
__device__ __forceinline__ void postconv_lane(const float (&raw)[8], bool is_qk, float eps, float (&out)[8]) {
  float s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = silu<TO>(raw[i]);
  const float sum = head_sum_sq<TO>(s);
  const float inv = l2_inv<TO>(sum, eps);
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = is_qk ? s[i] * inv : s[i];
}

}  // namespace gdn
