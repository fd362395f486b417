// Device helpers shared by the attention kernels (forward and backward) for
// gfx950: vector types, the bf16 32x32x16 matrix instruction, bf16 packing,
// reductions across the two lane halves, the LDS row swizzle, and the
// global-to-LDS DMA instruction with its wait counter.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
typedef __attribute__((address_space(3))) const bf16x8_t lds_bf16x8;
typedef __attribute__((address_space(3))) const f32x4_t lds_f32x4;

// D = A B + C for a 32x32 block with k = 16 (bf16 in, fp32 out).
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D = A B + C for a 32x32 block with k = 64, A and B in OCP FP8 e4m3 (32
// bytes a lane), fp32 out: the gfx950 block-scaled instruction with every block
// scale at 2^0 (E8M0 127), i.e. the plain product.  Lane (g, i) holds row
// (column) i of A (B) and a half of the 64 k values; any assignment of k
// values to bytes works as long as A and B use the same one.
__device__ __forceinline__ f32x16_t mfma32_fp8(i32x8_t a, i32x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0x7f7f7f7f, 0, 0x7f7f7f7f);
}

// Four fp32 values -> four OCP FP8 e4m3 bytes, round to nearest even.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t r;
  r[0] = (__bf16)a;  // v_cvt_pk_bf16_f32: round to nearest even
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// Reduce over the lane pair (l, l ^ 32): with both operands = x, the swap
// returns x of the lower half and x of the upper half in every lane.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS row swizzle of a row-major tile (256-byte rows, sixteen 16-byte chunks):
// chunk c of row r sits at physical chunk c ^ swz(r).  swz takes 16 distinct
// values over any 16 consecutive rows and distinct top bits over any 4, so
// 16-byte row reads and 8-byte transposing reads are both conflict-free.
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

// Buffer resource word 3: raw buffer, 32-bit data format.  Loads past the
// resource's size (word 2, bytes) return zeros and touch no memory.
constexpr int kBufferDword3 = 0x00020000;

// 64 lanes x 16 bytes from rsrc + voff (per lane) straight into LDS at lds,
// in lane order (buffer_load_dwordx4 ... lds: no VGPR staging).  Awaited with
// the vmcnt counter, explicitly: the compiler cannot see these LDS writes.
__device__ __forceinline__ void lds_dma_dwordx4(const i32x4_t& rsrc, uint32_t voff, uint32_t lds) {
  // One wait state between writing M0 and the LDS-DMA instruction that reads it.
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
               :
               : "v"(voff), "s"(lds), "s"(rsrc)
               : "memory");
}

// s_waitcnt immediate for vmcnt(n) (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

// All of this wave's vector-memory operations have completed.
__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); }

// All but this wave's n most recent vector-memory operations have completed.
template <int n>
__device__ __forceinline__ void dma_wait_all_but() { __builtin_amdgcn_s_waitcnt(vmcnt_imm(n)); }

}  // namespace
}  // namespace h3attn
