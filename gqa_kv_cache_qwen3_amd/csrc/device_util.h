// Small gfx950 device helpers used by the libmtd kernels: bf16 bit tricks, packed bf16 dot
// products, DPP lane exchanges inside 8-lane groups, and wave-wide scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtd {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// exp2 on the hardware transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// a.lo*b.lo + a.hi*b.hi + c with bf16 pairs packed in 32-bit words, fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Two fp32 -> packed bf16 pair (round to nearest even), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Byte permute: result bytes picked from {lo_src bytes 0..3, hi_src bytes 4..7}.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
  return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}
// (x.lo16, y.lo16) and (x.hi16, y.hi16)
__device__ __forceinline__ uint32_t pack_lo16(uint32_t x, uint32_t y) { return perm_b32(y, x, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi16(uint32_t x, uint32_t y) { return perm_b32(y, x, 0x07060302u); }

// DPP controls (within rows of 16 lanes).
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i within each 8-lane half row

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}

// Sum over each aligned group of 8 lanes; every lane of the group gets the sum.
__device__ __forceinline__ float sum8(float x) {
  x += dpp_f32<kDppQuadXor1>(x);
  x += dpp_f32<kDppQuadXor2>(x);
  x += dpp_f32<kDppRowHalfMirror>(x);
  return x;
}

// The value of lane l ^ 32, for every lane, without a trip through LDS.  v_permlane32_swap with
// both operands holding x leaves x[l % 32] in the first and x[l % 32 + 32] in the second register
// (checked on gfx950); one of the two is x[l ^ 32] and the other x[l] itself, so max / sum of the
// pair is the pair reduction.  Written as inline asm because the compiler folds the intrinsic
// with two equal operands to a no-op.  The s_nop pairs cover the VALU-write -> permlane hazard.
__device__ __forceinline__ void swap_halves(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float max_xor32(float x) {
  float y = x;
  swap_halves(x, y);
  return fmaxf(x, y);
}
__device__ __forceinline__ float sum_xor32(float x) {
  float y = x;
  swap_halves(x, y);
  return x + y;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace mtd
