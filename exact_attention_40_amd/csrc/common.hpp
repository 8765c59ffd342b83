// Device-side building blocks shared by the attention kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace exattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum MaskMode { kMaskNone = 0, kMaskBool = 1, kMaskAdd = 2 };
enum DtypeCode { kDtypeBf16 = 0, kDtypeF16 = 1 };   // values of exattn_dtype

// D[32x32] += A[32x16] * B[16x32] on one wavefront, bf16 in, fp32 accumulate.
// Operand layout: lane l holds row (A) or column (B) l % 32 and eight k-slots for k-half
// l / 32; the hardware pairs A's lane (i + 32h) slot s with B's lane (j + 32h) slot s, so
// any slot-to-k assignment shared by A and B gives the same product.
// Result layout: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// The two 16-bit input formats share every data path; only the MFMA instruction (chosen
// by overload) and the rounding of fp32 results differ.
template <class E>
struct Ty;
template <>
struct Ty<bf16> {
  typedef bf16x8 v8;
  typedef bf16x4 v4;
};
template <>
struct Ty<f16> {
  typedef f16x8 v8;
  typedef f16x4 v4;
};

__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// acc + the two 16-bit values packed in `pair` (a dot product with (1, 1): v_dot2c_f32_bf16 or
// _f16), summing exponentials in the rounded form the P.V product consumes them.
template <class E>
__device__ __forceinline__ float add_pair(uint32_t pair, float acc);
template <>
__device__ __forceinline__ float add_pair<__bf16>(uint32_t pair, float acc) {
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2, pair), v2{(__bf16)1.f, (__bf16)1.f}, acc, false);
}
template <>
__device__ __forceinline__ float add_pair<_Float16>(uint32_t pair, float acc) {
  typedef _Float16 v2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(v2, pair), v2{(_Float16)1.f, (_Float16)1.f}, acc, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// exp2(min(x, 0)) in one instruction: exp2 is monotonic, so that is exp2(x) clamped to
// [0, 1], which the output clamp of v_exp_f32 gives (+inf -> 1, -inf -> 0). The clamp maps
// NaN to 0 unless the mode register's DX10_CLAMP bit is clear: kernels that use this call
// nan_passing_clamp() first, so a NaN score or lse stays NaN (a plain min(x, 0) before the
// exponential would turn it into exp2(0) = 1). No other instruction in those kernels
// carries a clamp modifier.
__device__ __forceinline__ float exp2_le1(float x) {
  float r;
  asm("v_exp_f32_e64 %0, %1 clamp" : "=v"(r) : "v"(x));
  return r;
}
// Clear MODE.DX10_CLAMP (bit 8) for this wave: clamped float results keep NaN.
__device__ __forceinline__ void nan_passing_clamp() {
  asm volatile("s_setreg_imm32_b32 hwreg(HW_REG_MODE, 8, 1), 0");
}

// An additive mask value in log2 units, bias * log2(e), rounded once. The product must not
// be contracted into a later add (hipcc fuses across statements by default): the row max
// and the exponent must see the same rounded value, or the exponent picks up the product's
// rounding error, about |bias| * 2^-24, which overflows exp2 for a huge finite bias such as
// -1e30.
__device__ __forceinline__ float bias_log2(float bias) {
#pragma clang fp contract(off)
  return bias * kLog2e;
}


template <bool B>
using bool_c = std::integral_constant<bool, B>;

// Eight fp32 values rounded (to nearest even) to one 16-byte fragment of the input format.
template <class V8 = bf16x8>
__device__ __forceinline__ V8 cvt8(float a0, float a1, float a2, float a3, float a4, float a5,
                                   float a6, float a7) {
  f32x8 f = {a0, a1, a2, a3, a4, a5, a6, a7};
  return __builtin_convertvector(f, V8);
}

__device__ __forceinline__ bf16x8 cat44(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f16x8 cat44(f16x4 lo, f16x4 hi) {
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
template <class V4 = bf16x4>
__device__ __forceinline__ V4 lds_read_tr4(const void* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<void*>(p)));
  return __builtin_bit_cast(V4, v);
}

// Map a hardware block index to a logical one so that consecutive logical blocks run on
// the same XCD: the dispatcher places block b on XCD b % 8, each XCD having its own L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int per = n >> 3, rem = n & 7;
  const int x = bid & 7, k = bid >> 3;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + k;
}

__device__ __forceinline__ float wave_xor32(float v) { return __shfl_xor(v, 32, 64); }

// Rows of packed sequence s: [beg, beg + len). The caller's device offsets are trusted only
// as far as they stay inside the packed tensor: each is clamped into [0, total], the end is
// at least the start, and the length is cut to `cap` (max_seqlen: the grid covers that
// many rows per sequence). So no offset array makes a kernel touch rows outside [0, total).
struct SeqRows {
  int beg, len;
};
__device__ __forceinline__ int clamp_cu(const int32_t* cu, int i, int total) {
  return min(max(cu[i], 0), total);
}
__device__ __forceinline__ SeqRows seq_rows(const int32_t* cu, int s, int total, int cap) {
  const int b = clamp_cu(cu, s, total);
  const int e = max(clamp_cu(cu, s + 1, total), b);
  return {b, min(e - b, cap)};
}

// Whether packed row r (0 <= r < total) is outside the rows the kernels compute: before the
// first or past the last sequence, or past the first `cap` rows of its own sequence. The
// sequence is found by bisection over the clamped offsets (n + 1 entries).
__device__ __forceinline__ bool row_uncovered(const int32_t* cu, int n, int r, int total, int cap) {
  if (r < clamp_cu(cu, 0, total) || r >= clamp_cu(cu, n, total)) return true;
  int lo = 0, hi = n;   // invariant for sorted offsets: cu[lo] <= r < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (clamp_cu(cu, mid, total) <= r) lo = mid;
    else hi = mid;
  }
  const SeqRows sr = seq_rows(cu, lo, total, cap);
  return r - sr.beg >= sr.len;
}

// max and sum of the values held by lanes l and l ^ 32, on both lanes, in one
// v_permlane32_swap (which exchanges the upper half of one register with the lower half of
// another): the two results hold the lower and the upper half on every lane.
__device__ __forceinline__ float pair_max32(float v) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
}
__device__ __forceinline__ float pair_min32(float v) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fminf(__uint_as_float(h[0]), __uint_as_float(h[1]));
}

// LDS model (64 banks of 4 bytes; 16-byte reads serve 16 lanes per cycle, 8-byte and
// transposed reads 32 lanes per cycle). A row-major tile of 256-byte rows whose 16-byte
// chunks are XOR-permuted by a 4x4 transpose of the row's low four bits,
// chunk' = chunk ^ (4*(row & 3) + ((row >> 2) & 3)), is free of bank conflicts both for
// 16-byte reads of 16 consecutive rows at one column and for transposed reads of 4
// consecutive rows x 32 columns. Rows of D = 64 (128 bytes) keep the XOR inside 8 chunks.
template <int D>
__device__ __forceinline__ int swz_f(int row) {
  const int f = 4 * (row & 3) + ((row >> 2) & 3);
  return D == 128 ? f : (f & 7);
}

// Copy R rows of D bf16 (row stride `stride` elements, rows past the buffer range read as
// zero) into a swizzled LDS tile with direct global->LDS loads: each wave instruction
// fills 64 consecutive 16-byte LDS chunks, lane i the i-th, so lane i fetches the global
// chunk that the swizzle places there. Completion is tracked by vmcnt.
template <int D, int R, int NW>
__device__ __forceinline__ void copy_tile_to_lds(unsigned char* dst, __amdgpu_buffer_rsrc_t rs,
                                                 int stride, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int ITER = R * CPR / 64 / NW;
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const int p0 = (i * NW + wave) * 64;
    const int pos = p0 + lane;
    const int row = pos / CPR, pc = pos % CPR;
    const int col = (pc ^ swz_f<D>(row)) * 8;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(dst + p0 * 16), 16,
        (int)((row * stride + col) * 2), 0, 0, 0);
  }
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Asynchronous global -> LDS copies (buffer loads with the LDS bit): lane i writes its
// 16 (or 4) bytes at LDS byte address `lds` + 16*i (or + 4*i); reads past `bytes` of the
// buffer return zero. They are issued from inline assembly so that the compiler does not
// treat them as LDS writes that every later LDS read might alias (it would wait for them
// right away); completion is tracked only through vmcnt by the caller (sync_copies).
// `base` and `lds` must be wave-uniform.
// The descriptor and the LDS address go to scalar registers (readfirstlane: the values are
// wave-uniform, and the instruction takes them from SGPRs).
__device__ __forceinline__ uint32_t sgpr(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}
__device__ __forceinline__ u32x4 copy_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return u32x4{sgpr((uint32_t)p), sgpr((uint32_t)(p >> 32) & 0xffffu), sgpr(bytes), 0x00020000u};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return sgpr((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}
__device__ __forceinline__ void copy16_to_lds(u32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               : : "v"(voff), "s"(rsrc), "s"(lds) : "memory", "m0");
}
// The same as a streaming (non-temporal) load, for data read exactly once.
__device__ __forceinline__ void copy16_to_lds_nt(u32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
               : : "v"(voff), "s"(rsrc), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void copy4_to_lds(u32x4 rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               : : "v"(voff), "s"(rsrc), "s"(lds) : "memory", "m0");
}
// Wait until at most N of this wave's asynchronous copies are in flight (they complete in
// issue order) and its LDS operations are done, then join the workgroup barrier.
template <int N>
__device__ __forceinline__ void sync_copies() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// copy_tile_to_lds with the asynchronous copies above.
template <int D, int R, int NW>
__device__ __forceinline__ void copy_tile_async(unsigned char* dst, u32x4 rs, int stride,
                                                int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int ITER = R * CPR / 64 / NW;
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const int p0 = (i * NW + wave) * 64;
    const int pos = p0 + lane;
    const int row = pos / CPR, pc = pos % CPR;
    const int col = (pc ^ swz_f<D>(row)) * 8;
    copy16_to_lds(rs, (uint32_t)((row * stride + col) * 2), lds_addr(dst + p0 * 16));
  }
}
// The same with `dst` given as an LDS byte address (wave-uniform), so no pointer conversion
// happens per copy.
template <int D, int R, int NW>
__device__ __forceinline__ void copy_tile_async(uint32_t dst, u32x4 rs, int stride,
                                                int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int ITER = R * CPR / 64 / NW;
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const int p0 = (i * NW + wave) * 64;
    const int pos = p0 + lane;
    const int row = pos / CPR, pc = pos % CPR;
    const int col = (pc ^ swz_f<D>(row)) * 8;
    copy16_to_lds(rs, (uint32_t)((row * stride + col) * 2), sgpr(dst + (uint32_t)p0 * 16u));
  }
}

// Wait for every vector-memory operation except the most recent N. The counter retires in
// issue order, so older loads are complete while the newest N (atomics) stay in flight.
template <int N>
__device__ __forceinline__ void wait_vmem_except() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS read at a per-lane byte address plus a compile-time byte offset (the offset folds into
// the instruction's immediate field).
template <class V>
__device__ __forceinline__ V lds_at(const unsigned char* base, int imm) {
  return *reinterpret_cast<const V*>(base + imm);
}
template <class V4 = bf16x4>
__device__ __forceinline__ V4 tr_at(const unsigned char* base, int imm) {
  return lds_read_tr4<V4>(base + imm);
}

// Store a wave's 32 x D result block as bf16 rows, coalesced. `acc[db]` holds the block in
// the MFMA result layout with lane = row (l % 32) and register r = column db*32 +
// acc_row(r, l / 32). The values go through this wave's own 32 * D * 2 bytes of LDS `buf`
// (16-byte chunks XOR-swizzled by the row's low bits, so both the 8-byte writes and the
// 16-byte reads avoid bank conflicts), then each lane stores 16 contiguous bytes: every
// store instruction covers whole rows. Rows r >= nrows are not written. The caller makes
// sure no other wave uses `buf` meanwhile.
template <int D, class E>
__device__ __forceinline__ void wave_store_rows(unsigned char* buf, const f32x16 (&acc)[D / 32],
                                                float scale, E* dst, int64_t row_stride,
                                                int nrows, int lane) {
  typedef typename Ty<E>::v4 V4;
  constexpr int RB = D * 2;
  constexpr int CPR = D / 8;                     // 16-byte chunks per row
  const int half = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int c8 = db * 8 + 2 * rg + half;     // 8-byte chunk of columns 4*c8 .. 4*c8+3
      f32x4 v = {acc[db][4 * rg] * scale, acc[db][4 * rg + 1] * scale, acc[db][4 * rg + 2] * scale,
                 acc[db][4 * rg + 3] * scale};
      *reinterpret_cast<V4*>(buf + l32 * RB + 16 * ((c8 >> 1) ^ (l32 & (CPR - 1))) + 8 * (c8 & 1)) =
          __builtin_convertvector(v, V4);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr int RPI = 64 / CPR;                  // rows per instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / CPR, c = lane % CPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(buf + r * RB + 16 * (c ^ (r & (CPR - 1))));
    if (r < nrows) *reinterpret_cast<u32x4*>(dst + (int64_t)r * row_stride + 8 * c) = v;
  }
}

// Store a wave's 32 x D result block as rows of the input format, coalesced, for an
// accumulator in the other orientation: lane = column, `acc[db]` register r = row
// acc_row(r, l / 32), column db*32 + l % 32. Each value goes to this wave's own 32 * D * 2
// bytes of LDS `buf` (16-byte chunks XOR-swizzled by the row's low bits), then each lane
// stores 16 contiguous bytes, so every store instruction covers whole rows. Rows
// r >= nrows are not written. The caller makes sure no other wave uses `buf` meanwhile.
template <int D, class E>
__device__ __forceinline__ void wave_store_cols(unsigned char* buf, const f32x16 (&acc)[D / 32],
                                                float scale, E* dst, int64_t row_stride,
                                                int nrows, int lane) {
  constexpr int RB = D * 2;
  constexpr int CPR = D / 8;
  const int half = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int col = db * 32 + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = acc_row(r, half);
      *reinterpret_cast<E*>(buf + row * RB + 16 * ((col >> 3) ^ (row & (CPR - 1))) + 2 * (col & 7)) =
          (E)(acc[db][r] * scale);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr int RPI = 64 / CPR;                  // rows per instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / CPR, c = lane % CPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(buf + r * RB + 16 * (c ^ (r & (CPR - 1))));
    if (r < nrows) *reinterpret_cast<u32x4*>(dst + (int64_t)r * row_stride + 8 * c) = v;
  }
}

}  // namespace exattn
