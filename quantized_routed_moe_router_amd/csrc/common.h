// Device-side types and helpers shared by the ds4moe kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 half_t;
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

// Packed expert layout: one unit = 16 rows x 256 reduction columns.
// Unit of B-bit codes (B = 2, 4 or 6): B/2 code planes of 1024 bytes (16
// bytes per MFMA lane each), then 16 bytes of scales and mins per row, then
// d | dmin<<16 per row.  The scale, min and d layouts do not depend on B.
// The 6-bit unit holds the low 4 bits of each code in two planes laid out as
// in the 4-bit unit and the high 2 bits in a third plane laid out as in the
// 2-bit unit; 5-bit codes use it with their top bit zero.
template <int B>
struct Unit;
template <>
struct Unit<2> {
  static constexpr uint32_t BYTES = 1344, SCALE_OFF = 1024, DD_OFF = 1280;
  static constexpr int LOADS = 3;  // 16-byte loads per lane per unit
};
template <>
struct Unit<4> {
  static constexpr uint32_t BYTES = 2368, SCALE_OFF = 2048, DD_OFF = 2304;
  static constexpr int LOADS = 4;
};
template <>
struct Unit<6> {
  static constexpr uint32_t BYTES = 3392, SCALE_OFF = 3072, DD_OFF = 3328;
  static constexpr int LOADS = 5;
};

// width of the packed unit that holds `bits`-bit codes (5-bit codes: the 6-bit unit)
__host__ __device__ constexpr int unit_bits(int bits) { return bits == 5 ? 6 : bits; }

// canonical block of 256 weights with B-bit codes: scales[16], codes, d, dmin
template <int B>
constexpr int canon_block_bytes() {
  return 16 + 32 * B + 4;
}


__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  half_t h;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}

__device__ __forceinline__ h8 cat8(h2 a, h2 b, h2 c, h2 d) {
  h8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// fp4 (e2m1) nibble pairs -> fp16 pairs.  The scale operand acts as a power
// of two (only its exponent is used); nibble 0b00qq is q/2, so scale 2 gives
// q exactly.  SEL picks the byte of `w`; the low nibble lands in element 0.
#define CVT_FP4(w, scale, SEL) __builtin_amdgcn_cvt_scalef32_pk_f16_fp4((w), (scale), (SEL))

// A-operand fragment of one MFMA step: 8 codes of one sub-block times the
// sub-block scale, exact small integers in fp16.  HALF selects elements 0-7
// (bits 0-1 of each nibble) or 8-15 (bits 2-3).
template <int HALF>
__device__ __forceinline__ h8 dequant_frag(uint32_t raw, h2 sc2) {
  const uint32_t nib = (raw >> (2 * HALF)) & 0x33333333u;
  h2 p0 = CVT_FP4(nib, 2.0f, 0) * sc2;
  h2 p1 = CVT_FP4(nib, 2.0f, 1) * sc2;
  h2 p2 = CVT_FP4(nib, 2.0f, 2) * sc2;
  h2 p3 = CVT_FP4(nib, 2.0f, 3) * sc2;
  return cat8(p0, p1, p2, p3);
}

// fp8 (OCP e4m3) byte pairs -> fp16 pairs.  A byte b <= 15 encodes b * 2^-9
// exactly (exponent field 0 or 1), so scale 512 gives the small integer b.
// HI picks the upper 16 bits of `w`; the low byte lands in element 0.
#define CVT_FP8(w, HI) __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((w), 512.0f, (HI))

// A-operand fragment of one MFMA step with 4-bit codes: the dword holds the
// step's 8 codes, element e in nibble 2e (e < 4) or 2(e-4)+1 (e >= 4), so the
// low nibbles of its bytes are elements 0-3 and the high nibbles 4-7; each
// code (<= 15) converts exactly and sc*q (<= 225) is exact in fp16.
__device__ __forceinline__ h8 dequant_frag4(uint32_t raw, h2 sc2) {
  const uint32_t lo = raw & 0x0F0F0F0Fu, hi = (raw >> 4) & 0x0F0F0F0Fu;
  return cat8(CVT_FP8(lo, false) * sc2, CVT_FP8(lo, true) * sc2, CVT_FP8(hi, false) * sc2,
              CVT_FP8(hi, true) * sc2);
}

// A-operand fragment of one MFMA step with 6-bit codes (5-bit codes: top bit
// zero): the low 4 bits of the step's 8 codes as in dequant_frag4 (dword
// `lo`), the high 2 bits as in dequant_frag (dword `hi`, elements 0-7 or
// 8-15 of its sub-block by HALF), so element e of both is the same weight.
// q = l + 16*h, and q*sc = l*sc + h*(16*sc): every term and the sum are exact
// integers in fp16 (at most 945).
template <int HALF>
__device__ __forceinline__ h8 dequant_frag6(uint32_t lo, uint32_t hi, h2 sc2) {
  const uint32_t l0 = lo & 0x0F0F0F0Fu, l1 = (lo >> 4) & 0x0F0F0F0Fu;
  const uint32_t nib = (hi >> (2 * HALF)) & 0x33333333u;
  h2 s16;
  s16[0] = sc2[0] * (half_t)16.0f;
  s16[1] = sc2[1] * (half_t)16.0f;
  return cat8(CVT_FP4(nib, 2.0f, 0) * s16 + CVT_FP8(l0, false) * sc2,
              CVT_FP4(nib, 2.0f, 1) * s16 + CVT_FP8(l0, true) * sc2,
              CVT_FP4(nib, 2.0f, 2) * s16 + CVT_FP8(l1, false) * sc2,
              CVT_FP4(nib, 2.0f, 3) * s16 + CVT_FP8(l1, true) * sc2);
}

__device__ __forceinline__ h2 splat_h2(float v) {
  h2 r;
  r[0] = (half_t)v;
  r[1] = r[0];
  return r;
}

__device__ __forceinline__ f4 mfma16(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ h8 zero_h8() {
  h8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (half_t)0.0f;
  return z;
}

__device__ __forceinline__ h8 load_h8(const half_t *p) { return *reinterpret_cast<const h8 *>(p); }

// Raw buffer access over one region (wave-uniform descriptor).  Lanes with an
// offset at or beyond the region's length read zeros without touching memory,
// so masked loads need no branch.
constexpr uint32_t DS4_OOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane straight into LDS: lane l's bytes land at lds + 16*l
// (lds wave-uniform); out-of-range lanes write zeros
__device__ __forceinline__ void buf_load_lds16(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, off, 0, 0, 0);
}

// vmcnt(N) with the other counters left alone
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ h8 buf_load_h8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// ---------------------------------------------------------------- token pre-scale
// Each token's activations enter the fp16 operands as x' = x * 2^-e with
// max |x| in [2^e, 2^(e+1)), so max |x'| lies in [1, 2) whatever the range of
// x (bf16 covers far more than fp16).  Gate and up are linear in x, so the
// MFMA sums are g' = g 2^-e and u' = u 2^-e, exactly; the intermediate is
// stored as h' = h 2^-2e = g' u' sigmoid(g' 2^e) and the token's expert
// outputs carry the factor 2^2e back.  Every scaling is by a power of two,
// hence exact while no value leaves the fp32 range.
//
// e for a token whose largest magnitude is `amax` (0 for an all-zero,
// infinite or NaN row, which is then converted unscaled).
__device__ __forceinline__ int token_exp(float amax) {
  return (amax > 0.0f && amax <= 3.40282347e38f) ? ilogbf(amax) : 0;
}

// SwiGLU of a pre-scaled token: h' = silu(g) u 2^-2e from g' = g 2^-e and
// u' = u 2^-e (the same operations as silu(g) * u, each result scaled by a
// power of two).
__device__ __forceinline__ float swiglu_scaled(float gs, float us, int e) {
  const float g = ldexpf(gs, e);
  return gs / (1.0f + expf(-g)) * us;
}

// v * 2^(2e) in two exact steps (2^(2e) itself may not be representable).
__device__ __forceinline__ float scale_2e(float v, int e) { return ldexpf(ldexpf(v, e), e); }
