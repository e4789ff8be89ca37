// Device helpers shared by the bsq kernels (gfx950 only).
//
// Rounding rules follow "End-to-End 4-Bit Training": FP4 values
// +-{0,0.5,1,1.5,2,3,4,6}, E4M3 block scales (max 448), E8M0 MX scales
// (section "Low-precision formats on Blackwell"); stochastic rounding rounds
// up or down with probability given by the distance to each neighbour
// (section "Re-quantization with stochastic rounding").
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsqd {

constexpr float kFltMinNormal = 1.17549435082228750797e-38f;  // 2^-126
constexpr float kTwoPowM17 = 7.62939453125e-06f;              // 2^-17

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------- E4M3
// Exact decode (hardware convert, OCP E4M3FN on gfx950).
__device__ __forceinline__ float e4m3_val(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}
// Non-negative r -> E4M3 code, round to nearest even, saturating at 448. The
// hardware convert rounds to nearest even for |v| <= 464 and gives NaN above,
// so clamping to 448 first yields exactly the saturating rounding.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float r) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(r, 448.0f), 0.0f, 0, false) & 0xFFu;
}
// Non-negative r -> smallest E4M3 code whose value is >= r, capped at 448.
__device__ __forceinline__ uint32_t e4m3_ru_cap(float r) {
  uint32_t c = e4m3_rne_sat(r);
  if (c < 0x7Eu && e4m3_val(c) < r) c += 1u;
  return c;
}
// Value already on the E4M3 grid (|v| <= 448) -> code (exact).
__device__ __forceinline__ uint32_t e4m3_exact(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xFFu;
}
// Two values on the E4M3 grid -> two codes packed in the low 16 bits.
__device__ __forceinline__ uint32_t e4m3_exact2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// ---------------------------------------------------------------- E2M1
// Two floats -> two E2M1 codes written into byte `sel` of `old` (a in the
// low nibble). With scale 1.0 the hardware convert is round to nearest even,
// saturating at 6, sign kept (checked over every float32 pattern below 12).
#define BSQ_CVT_FP4X2(old, a, b, sel) \
  __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((old), (a), (b), 1.0f, (sel))

// ---------------------------------------------------------------- E8M0
// Smallest e with a <= 448 * 2^e, clamped to [-127, 127]; 0 gives -127.
// 448 = 1.75 * 2^8: a = 2^E * 1.f needs e = E - 8, or E - 7 when 1.f > 1.75.
__device__ __forceinline__ int e8m0_exponent(float a) {
  uint32_t b = __float_as_uint(a);
  int E = (int)(b >> 23) - 127;
  int e = E - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  if (a == 0.0f) e = -127;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// 2^-e as float32 for e in [-127, 126].
__device__ __forceinline__ float pow2_neg(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// ---------------------------------------------------------------- Philox4x32-10
// Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3"
// (SC'11): ten rounds of two 32x32->64 multiplies by 0xD2511F53 / 0xCD9E8D57
// with the key bumped by (0x9E3779B9, 0xBB67AE85) between rounds.
struct U32x4 { uint32_t v[4]; };
__device__ __forceinline__ U32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (i) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    // three-input XORs: one v_bitop3_b32 each (truth table 0x96) instead of two XORs
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  U32x4 r;
  r.v[0] = c0; r.v[1] = c1; r.v[2] = c2; r.v[3] = c3;
  return r;
}
// The four words serving output indices 8*grp .. 8*grp+7 (index i takes half
// i&1 of word (i>>1)&3).
__device__ __forceinline__ U32x4 sr_words(uint64_t seed, uint64_t stream, uint64_t grp) {
  return philox4x32_10((uint32_t)grp, (uint32_t)(grp >> 32), (uint32_t)stream,
                       (uint32_t)(stream >> 32), (uint32_t)seed, (uint32_t)(seed >> 32));
}
__device__ __forceinline__ uint32_t r16_of(const U32x4& w, int i) {
  return (w.v[(i >> 1) & 3] >> (16 * (i & 1))) & 0xFFFFu;
}

// ---------------------------------------------------------------- stochastic rounding
// u = (2 r + 1) / 2^17; round away from zero iff u < delta, delta the position
// of |y| between its two grid neighbours (exact in float32 here).
//
// E4M3 target, |y| <= 448. For |y| >= 2^-6 the grid keeps 3 mantissa bits, so
// delta = t / 2^20 with t the 20 dropped mantissa bits, and
// u < delta  <=>  8 (2 r + 1) < t. Below 2^-6 the step is 2^-9.
__device__ __forceinline__ float sr_e4m3(float y, uint32_t r16) {
  const uint32_t b = __float_as_uint(y);
  const uint32_t s = b & 0x80000000u;
  uint32_t a = b & 0x7FFFFFFFu;
  if (a - 1u >= 0x3C7FFFFFu) {  // |y| >= 2^-6, or exactly 0 (t = 0 keeps it 0)
    const uint32_t t = a & 0xFFFFFu;
    a = (a & 0xFFF00000u) + (((r16 << 4) + 8u < t) ? 0x100000u : 0u);
  } else {
    const float q = __uint_as_float(a) * 512.0f;
    float fl = floorf(q);
    const float u = (float)(2u * r16 + 1u) * kTwoPowM17;
    fl += (u < q - fl) ? 1.0f : 0.0f;
    a = __float_as_uint(fl * 0.001953125f);
  }
  return __uint_as_float(a | s);
}
// Eight values at once, y[i] drawing half i & 1 of word i >> 1 of one Philox
// call (the same draws and decisions as sr_e4m3). When every value is 0 or at
// least 2^-6 in magnitude, rounding away from zero adds one unit at mantissa
// bit 20: adding K = 0xFFFF7 - 16 r to the low 20 bits t carries into bit 20
// exactly when t > 16 r + 8, and K = ((~r) << 4) | 7. The sign bit and zeros
// pass through unchanged. Otherwise every value takes sr_e4m3.
__device__ __forceinline__ void sr_e4m3_x8(float (&y)[8], const U32x4& w) {
  uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < 8; ++i) mn = min(mn, (__float_as_uint(y[i]) & 0x7FFFFFFFu) - 1u);
  if (mn >= 0x3C7FFFFFu) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t nw = ~w.v[q];
      const uint32_t k0 = ((nw << 4) & 0xFFFF0u) | 7u;
      const uint32_t k1 = ((nw >> 12) & 0xFFFF0u) | 7u;
      y[2 * q] = __uint_as_float((__float_as_uint(y[2 * q]) + k0) & 0xFFF00000u);
      y[2 * q + 1] = __uint_as_float((__float_as_uint(y[2 * q + 1]) + k1) & 0xFFF00000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = sr_e4m3(y[i], r16_of(w, i));
  }
}
// One MX block: 32 values z with E8M0 exponent e (codes of y = z 2^-e, |y| <= 448)
// rounded stochastically, value i drawing from the Philox call grp0 + i / 8.
// Scaling by 2^-e keeps the mantissa bits, so when e >= -120 (every z of the
// fast path is then a normal float) and each z of a group of 8 is 0 or at
// least 2^(e-6), the one-add rounding of sr_e4m3_x8 applies to z itself and
// the scaled stochastic-rounding convert (which divides by its power-of-two
// scale and adds the random operand below the kept mantissa bits) makes each
// code, placed into its byte of the word. Other groups take y = z 2^-e and
// sr_e4m3. Codes are the same either way.
__device__ __forceinline__ void sr_block_e4m3(const float (&z)[32], int e, uint64_t seed, uint64_t stream,
                                              uint64_t grp0, uint32_t (&out)[8]) {
  const float scale = __uint_as_float((uint32_t)(e + 127) << 23);  // 2^e, used for e >= -120 only
  const uint32_t thr = ((uint32_t)(e + 121) << 24) - 2u;           // (bits(2^(e-6)) << 1) - 2
  const float pw = pow2_neg(e);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const U32x4 w = sr_words(seed, stream, grp0 + g);
    uint32_t mn = 0xFFFFFFFFu;  // zeros map to 0xFFFFFFFE
#pragma unroll
    for (int q = 0; q < 8; ++q) mn = min(mn, (__float_as_uint(z[8 * g + q]) << 1) - 2u);
    if (e >= -120 && mn >= thr) {
      // The hardware stochastic-rounding convert divides by the scale, adds
      // the top 20 bits of its random operand to the 20 mantissa bits that
      // E4M3 drops and truncates (checked bit for bit on gfx950 over 2^20
      // normal-range values, zeros of both signs and random operands). Giving
      // it K << 12, K = ((~r) << 4) | 7, is the one-add rounding above: the
      // same decisions, in one instruction per value.
      int wd0 = 0, wd1 = 0;
#define BSQ_SR2(wd, q, b0)                                                                                  \
  {                                                                                                         \
    const uint32_t nw = ~w.v[q];                                                                            \
    wd = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(wd, z[8 * g + 2 * (q)], (nw << 16) | 0x7000u, scale, b0); \
    wd = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(wd, z[8 * g + 2 * (q) + 1], (nw & 0xFFFF0000u) | 0x7000u, \
                                                  scale, (b0) + 1);                                         \
  }
      BSQ_SR2(wd0, 0, 0)
      BSQ_SR2(wd0, 1, 2)
      BSQ_SR2(wd1, 2, 0)
      BSQ_SR2(wd1, 3, 2)
#undef BSQ_SR2
      out[2 * g] = (uint32_t)wd0;
      out[2 * g + 1] = (uint32_t)wd1;
    } else {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = sr_e4m3(z[8 * g + q] * pw, r16_of(w, q));
      out[2 * g] = e4m3_exact2(v[0], v[1]) | (e4m3_exact2(v[2], v[3]) << 16);
      out[2 * g + 1] = e4m3_exact2(v[4], v[5]) | (e4m3_exact2(v[6], v[7]) << 16);
    }
  }
}
// E2M1 target: steps 0.5 below 2, 1 in [2, 4), 2 in [4, 6); 6 and above -> 6.
__device__ __forceinline__ float sr_e2m1(float y, uint32_t r16) {
  const float m = fabsf(y);
  const float inv = m < 2.0f ? 2.0f : (m < 4.0f ? 1.0f : 0.5f);
  const float step = m < 2.0f ? 0.5f : (m < 4.0f ? 1.0f : 2.0f);
  const float q = m * inv;
  float fl = floorf(q);
  const float u = (float)(2u * r16 + 1u) * kTwoPowM17;
  fl += (u < q - fl) ? 1.0f : 0.0f;
  const float mag = m >= 6.0f ? 6.0f : fl * step;
  return copysignf(mag, y);
}

// ---------------------------------------------------------------- stores
// 16-byte store with the non-temporal hint, for outputs the kernel does not
// read again and that a wave writes as whole 128-byte lines (measured 0.5-2%
// faster there; where lanes write parts of lines the hint raised the HBM
// write traffic, so those stores stay ordinary).
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt(void* p, uint4 v) {
  __builtin_nontemporal_store(u32x4v{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4v*>(p));
}

// ---------------------------------------------------------------- RHT-32 + S2F6
// (combine codec: the encoder kernel and the w2 GEMM's epilogue)
constexpr uint32_t kInvSqrt32 = 0x3E3504F3u;  // float32 nearest to 1/sqrt(32)

// Unnormalized Walsh-Hadamard transform of v (v H, Sylvester order).
__device__ __forceinline__ void fwht32(float (&v)[32]) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1)
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
}

// Smallest e with a <= (127/64) 2^e for a >= 0, clamped to [-127, 127]; -127
// for a == 0. From the bits: a = f 2^p with f in [1, 2) rounds up to p + 1 when
// f > 127/64, i.e. when the 23-bit fraction exceeds 63 * 2^17.
__device__ __forceinline__ int s2f6_exponent(float a) {
  const uint32_t bits = __float_as_uint(a);
  const uint32_t E = bits >> 23;
  if (E == 0) return bits > 0x7F0000u ? -126 : -127;  // subnormal: below 2^-126
  const int e = (int)E - 127 + ((bits & 0x7FFFFFu) > 0x7E0000u ? 1 : 0);
  return e > 127 ? 127 : e;
}

__device__ __forceinline__ uint32_t s2f6_code(float z, int sh) {
  float y = rintf(ldexpf(z, sh));  // exact scaling, then round half to even
  y = fminf(fmaxf(y, -128.0f), 127.0f);
  return (uint32_t)(int)y & 0xFFu;
}

// Block of 32 values in registers -> S2F6 codes (8 words, 4 per word, element
// 4o + i in byte i of word o) and the UE8M0 scale byte: sign flips by the
// mask, butterfly, times f32(1/sqrt(32)), smallest covering power of two.
__device__ __forceinline__ uint32_t rht_s2f6_block(float (&v)[32], uint32_t signs, uint32_t (&w)[8]) {
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = __uint_as_float(__float_as_uint(v[i]) ^ (((signs >> i) & 1u) << 31));
  fwht32(v);
  const float c = __uint_as_float(kInvSqrt32);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = v[i] * c;
    amax = fmaxf(amax, fabsf(v[i]));
  }
  const int e = s2f6_exponent(amax);
#pragma unroll
  for (int o = 0; o < 8; ++o) {
    w[o] = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[o] |= s2f6_code(v[4 * o + i], 6 - e) << (8 * i);
  }
  return (uint32_t)(e + 127);
}

// ---------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
template <int G>
__device__ __forceinline__ float group_max(float v) {  // over aligned groups of G lanes, G <= 64
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace bsqd
