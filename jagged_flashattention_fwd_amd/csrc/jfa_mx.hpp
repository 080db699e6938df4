// Device helpers shared by the MXFP8 kernels (gfx950): the block-scaled FP8
// product, its operand reads from LDS, E4M3 packing and the small copies of
// scale bytes.
//
// Operand layout of v_mfma_scale_f32_32x32x64_f8f6f4 (checked on the
// device): row m of an operand lives in lanes m and m + 32, 32 bytes each;
// bytes 0-15 of both lanes are one 32-element block, scaled by lane m's scale
// byte, bytes 16-31 of both the next block, scaled by lane m + 32's.  Only
// the pairing of byte positions between the two operands matters, so lane
// m + 32 g holds elements 16 g .. 16 g + 15 of each of its two blocks.  The
// op_sel value of each operand picks the byte of its 32-bit scale register.
// The output has the 32 x 32 fp32 layout of the bf16 product: lane
// n + 32 g holds rows (i / 4) * 8 + 4 g + i % 4 of column n, i = 0..15.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jfa_device.hpp"

namespace jfa {

typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 4 bytes per lane from byte soff + voff of the resource into LDS at
// lds + 4 * lane (buffer_load_dword ... lds); out-of-range lanes write zeros.
__device__ __forceinline__ void dma_copy4_buf(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, %3 offen lds" ::"v"(voff), "s"(rs),
               "s"(__builtin_amdgcn_readfirstlane(lds)), "s"(__builtin_amdgcn_readfirstlane(soff))
               : "m0");
}
#pragma clang diagnostic pop

// Two 16-byte LDS reads forming one lane's 32 operand bytes.
__device__ __forceinline__ i32x8 lds_read32x2(const char* p0, const char* p1) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(p0);
  const u32x4 b = *reinterpret_cast<const u32x4*>(p1);
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

template <int SA, int SB>
__device__ __forceinline__ f32x16 mfma_mx(const i32x8& a, const i32x8& b, const f32x16& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, SA, sa, SB, sb);
}

// a / 2^k and b / 2^k as two E4M3 codes in byte pair HI of `old`, with k
// the exponent of `scale` (only the scale's exponent counts: a scale of 3
// acts as 2), in one instruction (v_cvt_scalef32_pk_fp8_f32: nearest, ties
// to even, E4M3 denormals kept, no saturation: past 464 * 2^k the code is
// NaN, so callers keep |a|, |b| within 448 * 2^k).
template <bool HI>
__device__ __forceinline__ uint32_t cvt_e4m3x2_scaled(float a, float b, float scale, uint32_t old) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  const s16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(__builtin_bit_cast(s16x2, old), a, b, scale, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// Of a block whose largest magnitude has biased exponent be (the block is
// live: be >= 27): the scale 2^(floor(log2 amax) - 8) as a float, and the cap
// 448 times it, 1.75 * 2^floor(log2 amax), applied before the division (exact:
// the division is by a power of two).
__device__ __forceinline__ float mx_block_scale(uint32_t be) { return __uint_as_float((be - 8u) << 23); }
__device__ __forceinline__ float mx_block_cap(uint32_t be) { return __uint_as_float((be << 23) | 0x600000u); }

// One 32-element MX block held as 16 floats in each of two lanes (lane n
// and n + 32: the product output layout above, rows (i / 4) * 8 + 4 g +
// i % 4): its E4M3 codes as the B-operand words of a product that reduces
// over the block, so that lane half g holds elements 16 g .. 16 g + 15, and
// its E8M0 scale code.  The scale is 2^(floor(log2 amax) - 8), the elements
// divided by it and capped at +-448 round to nearest, ties to even.  A block
// whose largest magnitude is below 2^-100 (or zero) quantizes to zeros.
// SIGNED = false: the elements are known non-negative.
template <bool SIGNED>
__device__ __forceinline__ void quantize_block32(const float (&x)[16], uint32_t (&w)[4], uint32_t* code) {
  float am = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) am = fmaxf(am, SIGNED ? fabsf(x[i]) : x[i]);
  am = max_across_halves(am);
  const uint32_t be = __float_as_uint(am) >> 23;  // biased exponent of the block maximum
  const bool live = be >= 27u;
  // a dead block: every element capped to 0
  const float cap = live ? mx_block_cap(be) : 0.f;
  const float scale = live ? mx_block_scale(be) : 1.f;
  *code = live ? be - 8u : 127u;  // E8M0 of 2^(floor(log2 amax) - 8)
  uint32_t c[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float* v = x + 4 * q;
    float a[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] = SIGNED ? __builtin_amdgcn_fmed3f(v[e], -cap, cap) : fminf(v[e], cap);
    const float a0 = a[0], a1 = a[1], a2 = a[2], a3 = a[3];
    c[q] = cvt_e4m3x2_scaled<true>(a2, a3, scale, cvt_e4m3x2_scaled<false>(a0, a1, scale, 0u));
  }
  // c[q] holds rows 8 q + 4 g + {0..3} (q = 0, 1: first 16, q = 2, 3: the
  // others): the lower half takes the upper half's first words, the upper
  // half the lower half's last words.
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    auto sw = __builtin_amdgcn_permlane32_swap(c[q], c[2 + q], false, false);
    w[2 * q] = sw[0];
    w[2 * q + 1] = sw[1];
  }
}

}  // namespace jfa
