// Device-side helpers of the quantized attention kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsdpa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int D = 128;          // head dimension
constexpr int KSTEP = 64;       // keys per online-softmax step (also the K scale block)
constexpr int NPAD = 128;       // token padding of every workspace tensor
constexpr float FP8_MAX = 448.f;
constexpr float FP4_MAX = 6.f;
constexpr float LOG2_448 = 8.807354922057604f;
constexpr float LOG2E = 1.4426950408889634f;

// The two bf16 values held in one 32-bit word (low half = first element).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> two E4M3 codes in the low (hi_word = false) or high 16 bits of
// `old`.  The hardware conversion rounds to nearest even, keeps the sign and
// handles subnormals; magnitudes at or above 464 would become NaN, so callers
// clamp values that can reach them.
template <bool HI_WORD>
__device__ __forceinline__ int cvt_e4m3x2(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI_WORD);
}

__device__ __forceinline__ float clamp448(float x) { return fminf(fmaxf(x, -FP8_MAX), FP8_MAX); }

// E2M1 codes of the eight fp32 values v[0..7] * inv, each clamped to
// [-6, 6], four bytes with v[2k] in the low nibble of byte k.  The hardware
// conversion (v_cvt_scalef32_pk_fp4_f32 at scale 1) rounds to nearest even
// and keeps the sign: ties 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2,
// 2.5 -> 2, 3.5 -> 4, 5 -> 4 go to the even mantissa, and -0 gives code 8.
__device__ __forceinline__ float clamp6(float x) { return __builtin_amdgcn_fmed3f(x, -FP4_MAX, FP4_MAX); }
__device__ __forceinline__ uint32_t e2m1_word8(const float* v, float inv) {
  uint32_t w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, clamp6(v[0] * inv), clamp6(v[1] * inv), 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, clamp6(v[2] * inv), clamp6(v[3] * inv), 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, clamp6(v[4] * inv), clamp6(v[5] * inv), 1.0f, 2);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, clamp6(v[6] * inv), clamp6(v[7] * inv), 1.0f, 3);
}

// MXFP4 (OCP Microscaling v1.0): the E8M0 byte shared by a block of 32
// values whose largest magnitude amax > 0 is 2 below amax's biased exponent
// (2 is E2M1's largest exponent), at least 0; the codes are E2M1 of
// x * 2^(127 - byte), saturating at 6.  The inverse scale 2^(127 - byte) is a
// normal fp32, so x * inv is exact; a block with amax = 0 keeps byte 0 and
// all-zero codes (callers skip the codes there).
__device__ __forceinline__ uint32_t mx_scale_byte(float amax) {
  return (uint32_t)max((int)((__float_as_uint(amax) >> 23) & 0xffu) - 2, 0);
}
__device__ __forceinline__ float mx_inv_scale(uint32_t byte) { return __uint_as_float((254u - byte) << 23); }

// Value of an E2M1 code (sign bit 3, exponent bits 2..1, mantissa bit 0).
__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const float mag = e ? (float)((2u + m) << (e - 1u)) * 0.5f : (float)m * 0.5f;
  return (c & 8u) ? -mag : mag;
}

// FP4 mode: the power of two 2^-E that brings the dequantized values of a
// query row or a 64-key K tile into f16's range before their hi/lo split:
// E = e - 138, e the biased exponent field of the largest fp32 scale (0 for
// zero or subnormal scales).  smax < 2^(e - 126), so the largest magnitude
// 6 * smax * 2^-E stays below 0.75 * 2^15 = 24576 (f16's largest finite value
// is 65504), and values more than 2^28 below it are still f16 normals.
// x * 2^-E is exact (ldexp), so the split keeps its relative precision
// whatever the input magnitude.
__device__ __forceinline__ int fp4_norm_exp(float smax) { return (int)((__float_as_uint(smax) >> 23) & 0xffu) - 138; }

// Bytes of one 64-key tile of FP4-mode K expanded to an f16 hi tile and an
// E4M3 correction tile (2 x 16 KB), and the byte offset of 16-byte chunk c of
// key row `row` inside either: rows of 256 B, chunk c stored at position
// c ^ (row & 15), so the 16 lanes that read one chunk column of 16 rows hit
// 16 different positions.
constexpr int KXTILE = 2 * KSTEP * D * 2;
__device__ __forceinline__ int kh_off(int row, int c) { return row * 256 + ((c ^ (row & 15)) << 4); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

}  // namespace qsdpa
