// fa2_device.h -- gfx950 building blocks shared by the attention kernels.
//
// Facts these helpers rely on (checked on gfx950 with a lane-layout probe):
//  * v_mfma_f32_32x32x16_bf16, wave64. A (32x16): lane l holds row l%32, k = 8*(l/32)+e.
//    B (16x32): lane l holds column l%32, k = 8*(l/32)+e. C/D (32x32): lane l holds column
//    l%32 and, in register r, row 8*(r/4) + 4*(l/32) + (r%4). An accumulator can therefore be
//    fed back as the B operand of the next product (its rows become the contraction index).
//  * ds_read_b64_tr_b16: inside each group of 16 lanes, output lane t element e is element
//    t%4 of the 8 bytes addressed by lane 4*e + t/4 -- a 4x16 -> 16x4 transpose of bf16.
//  * v_permlane32_swap exchanges the upper half of the first operand with the lower half of
//    the second; swapping a value with itself hands each lane its partner's (lane ^ 32) value.
//  * buffer_load_dwordx4 ... lds writes lane l's 16 bytes at (wave-uniform LDS base) + 16*l;
//    out-of-range buffer offsets read as zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define FA2_LDS __attribute__((address_space(3)))
typedef FA2_LDS char lds_char;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef unsigned u32x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands FP8 E4M3FN (format code 0, the OCP
// encoding: bias 7, largest finite 448) and unit block scales (E8M0 code 127 = 2^0). Lane l
// supplies row (A) / column (B) l%32 and 32 bytes of k; as with the bf16 form, any ordering
// of those bytes used identically by A and B gives the same product (checked on gfx950).
__device__ __forceinline__ f32x16 mfma32x32x64_fp8(u32x8 a, u32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(__builtin_bit_cast(i32x8, a),
                                                         __builtin_bit_cast(i32x8, b), c, 0, 0, 0,
                                                         127, 0, 127);
}

// Buffer resource over [base, base + bytes); loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t rs, uint32_t voffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voffset, 0, 0));
}

// Direct global -> LDS copy of 16 bytes per lane; lane l lands at lds_wave_base + 16*l.
__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t rs, lds_char* lds_wave_base,
                                                  uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (FA2_LDS void*)lds_wave_base, 16, voffset, 0, 0, 0);
}

__device__ __forceinline__ u32x4 lds_read16(const lds_char* p) {
  return *(const FA2_LDS u32x4*)p;
}

__device__ __forceinline__ u32x2 lds_read8_tr(const lds_char* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA2_LDS i16x4*)p);
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(unsigned, v);
}

// acc + lo + hi of a packed bf16 pair, in fp32 (v_dot2c_f32_bf16 against (1, 1)): sums exactly
// the bf16 values an MFMA consumed.
__device__ __forceinline__ float add_bf16_pair(unsigned pk, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk),
                                         __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// An empty asm statement with an AGPR operand. Its presence tells the compiler that the kernel
// uses AGPRs, which makes it select the AGPR-accumulator form of MFMA: the O accumulators then
// stay in AGPRs across the loop instead of being copied out and back every iteration.
__device__ __forceinline__ void agpr_accumulators_hint() { asm volatile("" ::"a"(0.0f)); }

// x + C through an add the optimiser cannot see into (it stays one add, not folded into the
// address arithmetic of every later use).
template <int C>
__device__ __forceinline__ int opaque_add(int x) {
  int r;
  asm("v_add_u32 %0, %1, %2" : "=v"(r) : "i"(C), "v"(x));
  return r;
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// LDS tiles of bf16 rows of D elements (D / 8 chunks of 16 bytes per row). The 64 banks form
// 16 groups of 16 bytes; a row of 256 or 512 bytes starts in group 0, a 128-byte row in group 0
// or 8. SWZ_ROWS rows share one 256-byte bank row, SWZ_SPAN chunks can be permuted.
template <int D>
struct SwzCfg {
  static constexpr int CH = D / 8;
  static constexpr int SWZ_ROWS = CH >= 16 ? 1 : 16 / CH;
  static constexpr int SWZ_SPAN = CH >= 16 ? 16 : CH;
};
// K tile: chunk c of row r is stored at chunk position c ^ swz_k(r). The 16 rows a
// quarter-wave reads at one chunk then land in 16 different bank groups.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  using S = SwzCfg<D>;
  return (r / S::SWZ_ROWS) & (S::SWZ_SPAN - 1);
}
// V tile: chunk c of row r at c ^ swz_v(r). A transposing read touches 4 rows x 4 chunks
// per half-wave; this XOR spreads them over all 16 bank groups.
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  using S = SwzCfg<D>;
  return 4 * ((r / S::SWZ_ROWS) & (S::SWZ_SPAN / 4 - 1));
}

// Calls f(std::integral_constant<int, I>) for I = B .. E-1, fully unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

}  // namespace fa2
