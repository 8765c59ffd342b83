// Device-side building blocks shared by the attention kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace exattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum MaskMode { kMaskNone = 0, kMaskBool = 1, kMaskAdd = 2 };

// D[32x32] += A[32x16] * B[16x32] on one wavefront, bf16 in, fp32 accumulate.
// Operand layout: lane l holds row (A) or column (B) l % 32 and eight k-slots for k-half
// l / 32; the hardware pairs A's lane (i + 32h) slot s with B's lane (j + 32h) slot s, so
// any slot-to-k assignment shared by A and B gives the same product.
// Result layout: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 cvt8(float a0, float a1, float a2, float a3, float a4,
                                       float a5, float a6, float a7) {
  f32x8 f = {a0, a1, a2, a3, a4, a5, a6, a7};
  return __builtin_convertvector(f, bf16x8);
}

__device__ __forceinline__ bf16x8 cat44(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Buffer resource over `bytes` bytes at `base`: loads past the end return zero, so partial
// tiles need no per-row branches (robust buffer access of the gfx9 family).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

// Transposed LDS read (ds_read_b64_tr_b16). Within each 16-lane group, if lane j points at
// row k0 + j/4, columns n0 + 4*(j%4) .. +3 of a row-major bf16 tile, lane i receives
// column n0 + i, rows k0 .. k0+3: an MFMA operand fragment read from the other-major layout.
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<bf16*>(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// Transpose a 4-row x 8-column bf16 block held as four 16-byte rows into eight 8-byte
// columns (column c = rows 0..3 at column c), written as 64 contiguous bytes to `dst`.
// This builds the "key-interleaved" tile layout T[row/4][col][row%4] that lets one lane
// read four consecutive rows of one column with a single 8-byte LDS read.
__device__ __forceinline__ void store_4x8_transposed(bf16* dst, u32x4 r0, u32x4 r1, u32x4 r2,
                                                     u32x4 r3) {
  u32x4 o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // column 2j: low halves; column 2j+1: high halves
    uint32_t a0 = (r0[j] & 0xffffu) | (r1[j] << 16);
    uint32_t a1 = (r2[j] & 0xffffu) | (r3[j] << 16);
    uint32_t b0 = (r0[j] >> 16) | (r1[j] & 0xffff0000u);
    uint32_t b1 = (r2[j] >> 16) | (r3[j] & 0xffff0000u);
    o[j] = u32x4{a0, a1, b0, b1};
  }
  u32x4* d = reinterpret_cast<u32x4*>(dst);
#pragma unroll
  for (int j = 0; j < 4; ++j) d[j] = o[j];
}

// Map a hardware block index to a logical one so that consecutive logical blocks run on
// the same XCD: the dispatcher places block b on XCD b % 8, each XCD having its own L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int per = n >> 3, rem = n & 7;
  const int x = bid & 7, k = bid >> 3;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + k;
}

__device__ __forceinline__ float wave_xor32(float v) { return __shfl_xor(v, 32, 64); }

}  // namespace exattn
