// Device-side helpers shared by the bfp4moe kernels (gfx950 / CDNA4).
//
// Formats (FlashInfer "flashinfer.fused_moe.alphamoe_nvfp4_aligned_moe", layout paragraph;
// Megatron-Core "core.inference.moe.flashinfer_nvfp4", module data):
//   E2M1 code s.e1e0.m, magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; two codes per byte, the even
//   logical value in the low nibble.  E4M3FN block scales (bias 7, max 448), one per 16 values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bfp4 {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kE4M3Max = 448.0f;
constexpr float kE2M1Max = 6.0f;
constexpr float kEncodeNumerator = 2688.0f;   // kE4M3Max * kE2M1Max, exact

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> BF16 bits, round to nearest even (finite inputs; overflow rounds to infinity).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// E4M3FN byte -> float (sign bit ignored: block scales are non-negative).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
}

// Non-negative finite float -> E4M3FN code: round to nearest even on the E4M3 grid, saturate at
// 448 (code 0x7E).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  if (v >= kE4M3Max) return 0x7Eu;
  if (v < 0x1p-6f) {                       // subnormal range: spacing 2^-9; 8 * 2^-9 is 2^-6
    return (uint32_t)__builtin_rintf(v * 512.0f);
  }
  uint32_t u = __float_as_uint(v);
  uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);   // round the float mantissa to 3 bits
  uint32_t code = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
  return code > 0x7Eu ? 0x7Eu : code;
}

// float -> E2M1 code: nearest magnitude, ties to the even code, saturate at 6, sign bit copied
// (so -0.0 and small negatives give code 0x8).  gfx950's v_cvt_scalef32_pk_fp4_f32 with a scale
// of 1 implements exactly this rule: it was compared with a compare-chain encoder of the rule on
// every finite FP32 bit pattern and on both infinities, with no difference.  It converts two
// values per instruction, the first into the low nibble of the selected byte.
__device__ __forceinline__ uint32_t e2m1_pack2(uint32_t old, float lo, float hi, int sel) {
  switch (sel) {   // the byte selector must be a compile-time constant
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, lo, hi, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, lo, hi, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, lo, hi, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, lo, hi, 1.0f, 3);
  }
}

// E4M3 block scale of a block whose largest magnitude is bmax, for encode scale s_enc (FP32
// steps rounded separately, no FMA: the library is compiled with -ffp-contract=off).  Returns
// the scale code and sets inv, the factor that maps the block's values onto the E2M1 grid.
__device__ __forceinline__ uint32_t block_scale(float bmax, float s_enc, float& inv) {
  const float v = (bmax * s_enc) / kE2M1Max;
  const uint32_t sf = f32_to_e4m3(v);
  const float sfv = e4m3_to_f32(sf);
  inv = (sfv == 0.0f) ? 0.0f : s_enc / sfv;
  return sf;
}

// 8 values -> 8 E2M1 codes of fl32(x * inv) in one dword (value i in bits 4i..4i+3: even value
// in the low nibble of each byte).
__device__ __forceinline__ uint32_t quant8(const float* x, float inv) {
  uint32_t c = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) c = e2m1_pack2(c, x[2 * j] * inv, x[2 * j + 1] * inv, j);
  return c;
}

// Quantize 16 values with encode scale s_enc.  Returns the scale code; codes packed into lo/hi
// (values 0..7 in lo, 8..15 in hi).
__device__ __forceinline__ uint32_t quant_block16(const float (&x)[16], float s_enc, uint32_t& lo,
                                                  uint32_t& hi) {
  float bmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) bmax = __builtin_fmaxf(bmax, __builtin_fabsf(x[i]));
  float inv;
  const uint32_t sf = block_scale(bmax, s_enc, inv);
  lo = quant8(x, inv);
  hi = quant8(x + 8, inv);
  return sf;
}

// MX (E8M0 per 32 values) shared scale of a block with largest magnitude amax, for an element
// format whose largest magnitude has exponent emax (E2M1: 2, E4M3: 8): X = floor(log2(amax)) -
// emax clamped to [-127, 127]; code = X + 127, or 0 for amax 0 or below the FP32 normal range
// (where the clamp gives X = -127 as well).  Returns 2^-X, the exact factor that maps the block
// onto the element grid; a normal float, since amax < 2^128 keeps X <= 127 - emax.
constexpr int kE2M1Emax = 2;
constexpr int kE4M3Emax = 8;
__device__ __forceinline__ float mx_scale_inverse(float amax, int emax, uint32_t& code) {
  const int ebits = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  int X = ebits == 0 ? -127 : ebits - 127 - emax;
  X = X < -127 ? -127 : (X > 127 ? 127 : X);
  code = (amax == 0.0f || ebits == 0) ? 0u : (uint32_t)(X + 127);
  return __uint_as_float((uint32_t)(127 - X) << 23);        // 2^-X, a normal float (|X| <= 127)
}

// Four values -> four signed E4M3FN codes of fl32(x * inv) (value i in byte i): nearest on the
// E4M3 grid with ties to the even code, saturating at 448, sign bit copied from the product.
__device__ __forceinline__ uint32_t e4m3_pack4(const float* x, float inv) {
  uint32_t w = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float y = x[i] * inv;
    const uint32_t sgn = (__float_as_uint(y) >> 31) << 7;
    w |= (sgn | f32_to_e4m3(__builtin_fabsf(y))) << (8 * i);
  }
  return w;
}

// Load one 16-value BF16 block as floats (two 16-byte loads).
__device__ __forceinline__ void load_block16(const uint16_t* p, float (&x)[16]) {
  uint4 a = *reinterpret_cast<const uint4*>(p);
  uint4 b = *reinterpret_cast<const uint4*>(p + 8);
  uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
}

// Encode scale from an FP32 amax: 2688 / amax, 1 when amax is 0, infinity clamped.
__device__ __forceinline__ float encode_scale_from_amax(float amax) {
  if (amax == 0.0f) return 1.0f;
  float s = kEncodeNumerator / amax;
  return (s > 3.40282347e38f) ? 3.40282347e38f : s;
}

// Exact decode of NVFP4 operands to FP16.
// Every E2M1 x E4M3 product has at most 6 significant bits and lies in [2^-10, 2688] (or is 0),
// so it is exact in FP16 (normal range).  v_cvt_scalef32_pk_f16_fp4 converts two E2M1 codes of a
// selected byte and multiplies by a power of two (only the exponent of its scale operand is
// used); 256 is passed so that the E4M3 factor can be applied as the exact FP16 number
// s * 2^-8, whose bit pattern is (code & 0x7F) << 7.
__device__ __forceinline__ uint32_t e4m3_scale_h2(uint32_t sf_byte) {
  uint32_t b = (sf_byte & 0x7Fu) << 7;
  return b | (b << 16);
}

__device__ __forceinline__ uint32_t dec_pair(uint32_t w, h2_t s, int sel) {
  h2_t p;
  switch (sel) {   // the byte selector must be a compile-time constant
    case 0: p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0); break;
    case 1: p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1); break;
    case 2: p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2); break;
    default: p = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3); break;
  }
  return __builtin_bit_cast(uint32_t, p * s);
}

// 8 E2M1 codes (one dword, code k in bits 4k..4k+3) times one E4M3 scale -> 8 exact FP16.
__device__ __forceinline__ h8_t decode8(uint32_t w, uint32_t scale_h2_bits) {
  h2_t s = __builtin_bit_cast(h2_t, scale_h2_bits);
  u32x4_t r;
  r[0] = dec_pair(w, s, 0);
  r[1] = dec_pair(w, s, 1);
  r[2] = dec_pair(w, s, 2);
  r[3] = dec_pair(w, s, 3);
  return __builtin_bit_cast(h8_t, r);
}

// Raw buffer resources and loads (gfx9 resource word 3; stride 0, range checked against `bytes`).
// Offsets: per-lane `voff` (VGPR) plus wave-uniform `soff` (SGPR), both unsigned 32-bit.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint32_t buffer_load_u8(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                   uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t buffer_load_u32(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                    uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint2 buffer_load_u64(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 uint32_t soff) {
  typedef uint32_t v2u __attribute__((ext_vector_type(2)));
  const v2u v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 buffer_load_u128(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                  uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Direct buffer -> LDS load of 16 bytes per lane: lane l's bytes land at lds_wave_base + 16*l
// (lds_wave_base is wave-uniform).  Completion is counted by vmcnt like any vector load.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds_wave_base,
                                                  uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds_wave_base, 16, voff, soff, 0, 0);
}

// s_waitcnt on the vector-memory counter only: at most N of this wave's vector memory
// operations still outstanding (gfx9 encoding: vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wave-wide (64 lanes) reductions.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// LDS barrier that leaves global loads in flight: wait for this wave's LDS operations only.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace bfp4
