// MFMA operand helpers shared by the chunked prefill and the windowed step
// (gfx950).  Fragment conventions (16x16 tiles, wave64):
//   A 16 x 16 (rows x contraction) fragment: lane (r, kg) = (lane % 16,
//   lane / 16) holds contraction slots 4kg .. 4kg+3 of row r.  A 16 x 32
//   fragment holds slots 4kg..4kg+3 of the first 16 and then of the second
//   16.  Every operand uses this slot order (a permutation of the
//   contraction index applied identically to both operands).
//   An accumulator tile holds element [4 kg + e][r] in lane (r, kg), element
//   e: the B-operand layout of the next product (contraction index = tile
//   row) and the A-operand layout of its transpose.
#pragma once
#include "device_common.hpp"

namespace gdn {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ------------------------------------------------------------ MFMA operands
// A 16 x 16 (rows x contraction) fragment: lane (r, kg) = (lane % 16,
// lane / 16) holds contraction slots 4kg .. 4kg+3 of row r.  A 16 x 32
// fragment holds slots 4kg..4kg+3 of the first 16 and then of the second 16.
// Every operand uses this slot order, and an accumulator tile's rows
// 4kg..4kg+3 are a lane's slots, so tiles feed the B side directly.
// Raw buffer resource over [p, p + bytes): the hardware range check turns
// loads past the end into zeros and drops stores past the end, so tail rows
// need no lane masks or address clamps.
constexpr int kBufDword3 = 0x00020000;   // raw buffer, 32-bit data format

// The size is made wave-uniform explicitly so the descriptor lives in
// scalar registers (a vector-register descriptor costs a waterfall loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, __builtin_amdgcn_readfirstlane(bytes),
                                           kBufDword3);
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// One 8-byte LDS read kept as its own instruction.  Left alone, the
// compiler fuses two 8-byte reads at a constant distance (here the two
// halves of a fragment, 32 bytes apart) into ds_read2_b64, which gfx950
// services in about 3.4x the LDS cycles of the two separate reads (13.8
// against 2 x 2 cycles per instruction, measured with the bank-conflict
// counter).  The offset passes through an empty asm operand, so the two
// addresses are not known to be a constant apart.
__device__ __forceinline__ uint2 lds_u64(const uint16_t* p, int off) {
  asm volatile("" : "+v"(off));
  return *reinterpret_cast<const uint2*>(p + off);
}

template <class T> struct Prec;

template <> struct Prec<uint16_t> {
  using E = uint16_t;
  static constexpr int PAD = 8;
  struct F16 { uint2 v; };
  struct F32 { uint4 v; };
  // row-major LDS matrix, fragment of rows row0.., contraction kb..
  __device__ __forceinline__ static F16 lds16(const E* p, int ld, int row, int kb, int kg) {
    F16 f;
    f.v = lds_u64(p, row * ld + kb + 4 * kg);
    return f;
  }
  __device__ __forceinline__ static F32 lds32(const E* p, int ld, int row, int kb, int kg) {
    const uint2 a = lds_u64(p, row * ld + kb + 4 * kg);
    const uint2 b = lds_u64(p, row * ld + kb + 16 + 4 * kg);
    F32 f;
    f.v = make_uint4(a.x, a.y, b.x, b.y);
    return f;
  }
  // Transposed fragment of a row-major LDS matrix M: rows = M's columns
  // c0..c0+15, contraction = M's rows kb..kb+31.  In each 16-lane group the
  // transposing load hands lane r, slot j the element loaded by lane
  // 4j + r/4 at slot r%4, so lane s of group kg loads M[kb + 4kg + s/4]
  // [c0 + 4 (s%4) .. +3].
  __device__ __forceinline__ static F32 ldsT32(const E* p, int ld, int c0, int kb, int lane) {
    const int s = lane & 15, kg = lane >> 4;
    const E* a = p + (kb + 4 * kg + (s >> 2)) * ld + c0 + 4 * (s & 3);
    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a));
    const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 16 * ld));
    const uint2 ux = __builtin_bit_cast(uint2, x), uy = __builtin_bit_cast(uint2, y);
    F32 f;
    f.v = make_uint4(ux.x, ux.y, uy.x, uy.y);
    return f;
  }
  __device__ __forceinline__ static F16 reg16(f32x4 d) {
    F16 f;
    f.v = make_uint2(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]));
    return f;
  }
  __device__ __forceinline__ static F32 reg32(f32x4 d0, f32x4 d1) {
    F32 f;
    f.v = make_uint4(pack_bf16x2(d0[0], d0[1]), pack_bf16x2(d0[2], d0[3]), pack_bf16x2(d1[0], d1[1]),
                     pack_bf16x2(d1[2], d1[3]));
    return f;
  }
  // The float32 operand split in two bf16 operands, hi = bf16(x) (reg32's
  // result) and lo = bf16(x - hi): hi + lo carries 16 significant bits, so a
  // product taken as hi * B + lo * B has the operand's rounding error near
  // 2^-17 instead of 2^-9.  x - hi is exact in float32.
  __device__ __forceinline__ static F32 reg32_lo(f32x4 d0, f32x4 d1, F32 hi) {
    const unsigned h[4] = {hi.v.x, hi.v.y, hi.v.z, hi.v.w};
    const float x[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
    unsigned lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lo[i] = pack_bf16x2(x[2 * i] - __uint_as_float(h[i] << 16), x[2 * i + 1] - __uint_as_float(h[i] & 0xffff0000u));
    F32 f;
    f.v = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    return f;
  }
  static constexpr bool kSplitState = true;
  __device__ __forceinline__ static f32x4 mma16(F16 a, F16 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a.v),
                                                     __builtin_bit_cast(s16x4, b.v), c, 0, 0, 0);
  }
  __device__ __forceinline__ static f32x4 mma32(F32 a, F32 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                    __builtin_bit_cast(bf16x8, b.v), c, 0, 0, 0);
  }
  __device__ __forceinline__ static void put(E* p, float x) { *p = static_cast<E>(f32_to_bf16(x)); }
  // 8 consecutive activations in storage form (one 16-byte piece)
  struct Raw8 { uint4 v; };
  __device__ __forceinline__ static Raw8 load_raw8(const uint16_t* p) {
    Raw8 r;
    r.v = *reinterpret_cast<const uint4*>(p);
    return r;
  }
  __device__ __forceinline__ static Raw8 zero_raw8() { Raw8 r; r.v = make_uint4(0, 0, 0, 0); return r; }
  __device__ __forceinline__ static void store_raw8(E* p, Raw8 r) { *reinterpret_cast<uint4*>(p) = r.v; }
  __device__ __forceinline__ static float to_f32(E x) { return bf16_to_f32(x); }
  // Transposed 16-wide fragment of a row-major LDS matrix M: rows = M's
  // columns c0..c0+15, contraction = M's rows 0..15 (one transposing load:
  // lane s of group kg loads M[4kg + s/4][c0 + 4 (s%4) .. +3]).
  __device__ __forceinline__ static F16 ldsT16(const E* p, int ld, int c0, int lane) {
    const int s = lane & 15, kg = lane >> 4;
    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + (4 * kg + (s >> 2)) * ld + c0 + 4 * (s & 3)));
    F16 f;
    f.v = __builtin_bit_cast(uint2, x);
    return f;
  }
  // 16 x 32 fragment read from global memory through a buffer resource:
  // `off` is the byte offset of slot 0 (row, kb + 4 kg); the second half is
  // 16 elements further.
  __device__ __forceinline__ static F32 gfrag32(__amdgpu_buffer_rsrc_t r, int off) {
    const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    const u32x2 b = __builtin_amdgcn_raw_buffer_load_b64(r, off + 32, 0, 0);
    F32 f;
    f.v = make_uint4(a.x, a.y, b.x, b.y);
    return f;
  }
  // the fragment's two halves written back to a row-major LDS row at
  // p (slot 0) and p + 16
  __device__ __forceinline__ static void put_frag32(E* p, F32 f) {
    *reinterpret_cast<uint2*>(p) = make_uint2(f.v.x, f.v.y);
    *reinterpret_cast<uint2*>(p + 16) = make_uint2(f.v.z, f.v.w);
  }
  __device__ __forceinline__ static float gload1(__amdgpu_buffer_rsrc_t r, int off) {
    return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
  }
  __device__ __forceinline__ static void gstore4(__amdgpu_buffer_rsrc_t r, int off, const float (&x)[4]) {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])}, r, off, 0, 0);
  }
};

template <> struct Prec<float> {
  using E = float;
  static constexpr int PAD = 4;
  struct F16 { f32x4 v; };
  struct F32 { f32x4 a, b; };
  __device__ __forceinline__ static F16 lds16(const E* p, int ld, int row, int kb, int kg) {
    F16 f;
    const float4 t = *reinterpret_cast<const float4*>(p + row * ld + kb + 4 * kg);
    f.v = f32x4{t.x, t.y, t.z, t.w};
    return f;
  }
  __device__ __forceinline__ static F32 lds32(const E* p, int ld, int row, int kb, int kg) {
    F32 f;
    f.a = lds16(p, ld, row, kb, kg).v;
    f.b = lds16(p, ld, row, kb + 16, kg).v;
    return f;
  }
  __device__ __forceinline__ static F32 ldsT32(const E* p, int ld, int c0, int kb, int lane) {
    const int r = lane & 15, kg = lane >> 4;
    F32 f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f.a[t] = p[(kb + 4 * kg + t) * ld + c0 + r];
      f.b[t] = p[(kb + 16 + 4 * kg + t) * ld + c0 + r];
    }
    return f;
  }
  __device__ __forceinline__ static F16 reg16(f32x4 d) { F16 f; f.v = d; return f; }
  __device__ __forceinline__ static F32 reg32(f32x4 d0, f32x4 d1) { F32 f; f.a = d0; f.b = d1; return f; }
  // float32 operands are exact: no second part
  __device__ __forceinline__ static F32 reg32_lo(f32x4, f32x4, F32 hi) { return hi; }
  static constexpr bool kSplitState = false;
  // slot t of lane kg is contraction index 4kg + t: four k = 4 steps
  __device__ __forceinline__ static f32x4 mma4x(f32x4 a, f32x4 b, f32x4 c) {
#pragma unroll
    for (int t = 0; t < 4; ++t) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], b[t], c, 0, 0, 0);
    return c;
  }
  __device__ __forceinline__ static f32x4 mma16(F16 a, F16 b, f32x4 c) { return mma4x(a.v, b.v, c); }
  __device__ __forceinline__ static f32x4 mma32(F32 a, F32 b, f32x4 c) {
    c = mma4x(a.a, b.a, c);
    return mma4x(a.b, b.b, c);
  }
  __device__ __forceinline__ static void put(E* p, float x) { *p = x; }
  struct Raw8 { float4 a, b; };
  __device__ __forceinline__ static Raw8 load_raw8(const float* p) {
    Raw8 r;
    r.a = *reinterpret_cast<const float4*>(p);
    r.b = *reinterpret_cast<const float4*>(p + 4);
    return r;
  }
  __device__ __forceinline__ static Raw8 zero_raw8() {
    Raw8 r;
    r.a = make_float4(0.f, 0.f, 0.f, 0.f);
    r.b = r.a;
    return r;
  }
  __device__ __forceinline__ static void store_raw8(E* p, Raw8 r) {
    *reinterpret_cast<float4*>(p) = r.a;
    *reinterpret_cast<float4*>(p + 4) = r.b;
  }
  __device__ __forceinline__ static float to_f32(E x) { return x; }
  __device__ __forceinline__ static F16 ldsT16(const E* p, int ld, int c0, int lane) {
    const int r = lane & 15, kg = lane >> 4;
    F16 f;
#pragma unroll
    for (int t = 0; t < 4; ++t) f.v[t] = p[(4 * kg + t) * ld + c0 + r];
    return f;
  }
  __device__ __forceinline__ static F32 gfrag32(__amdgpu_buffer_rsrc_t r, int off) {
    F32 f;
    f.a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    f.b = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 64, 0, 0));
    return f;
  }
  __device__ __forceinline__ static void put_frag32(E* p, F32 f) {
    *reinterpret_cast<f32x4*>(p) = f.a;
    *reinterpret_cast<f32x4*>(p + 16) = f.b;
  }
  __device__ __forceinline__ static float gload1(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  }
  __device__ __forceinline__ static void gstore4(__amdgpu_buffer_rsrc_t r, int off, const float (&x)[4]) {
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{__builtin_bit_cast(unsigned, x[0]), __builtin_bit_cast(unsigned, x[1]),
                                                 __builtin_bit_cast(unsigned, x[2]), __builtin_bit_cast(unsigned, x[3])},
                                           r, off, 0, 0);
  }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Value of lane `src` (0..3, a constant) of each DPP quad, in all four lanes.
__device__ __forceinline__ float quad_bcast(float v, int src) {
  switch (src) {
    case 0: return dpp_mov<0x00>(v);
    case 1: return dpp_mov<0x55>(v);
    case 2: return dpp_mov<0xAA>(v);
    default: return dpp_mov<0xFF>(v);
  }
}

// v moved by a DPP control; lanes without a source (or outside row_mask)
// read 0.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_or_zero(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf, false));
}

// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4, 8 inside each
// 16-lane row, then the rows' totals are carried forward with row_bcast:15
// and row_bcast:31.
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v += dpp_or_zero<0x111, 0xf>(v);
  v += dpp_or_zero<0x112, 0xf>(v);
  v += dpp_or_zero<0x114, 0xf>(v);
  v += dpp_or_zero<0x118, 0xf>(v);
  v += dpp_or_zero<0x142, 0xa>(v);
  v += dpp_or_zero<0x143, 0xc>(v);
  return v;
}




}  // namespace gdn
