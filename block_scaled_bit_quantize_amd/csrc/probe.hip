// Per-instruction MFMA throughput on the device: the peak each contraction
// dtype's instruction sustains when nothing but MFMAs runs, with operand data
// of three kinds (the GEMMs run at the chip's power limit, so the rate depends
// on how many operand bits switch).
//
// "End-to-End 4-Bit Training", section "Kernels for low-precision training":
// the MoE kernels are dominated by matrix multiplications whose rate is set by
// the tensor cores; on CDNA4 those are the MFMA instructions timed here:
//   kind 0: v_mfma_f32_32x32x16_f16      (the NVFP4 GEMMs' exact fp16 operands)
//   kind 1: v_mfma_f32_32x32x16_bf16     (the MXFP8 GEMMs' exact bf16 operands)
//   kind 2: v_mfma_f32_32x32x16_fp8_fp8  (K = 16 FP8, the in-register-scale variant)
//   kind 3: v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 operands (block-scaled FP8)
//   kind 4: v_mfma_scale_f32_32x32x64_f8f6f4, E2M1 operands (block-scaled FP4)
// Each wave runs `iters` rounds of four independent accumulator chains over
// four operand sets held in registers; each thread writes one float of its
// accumulators so that no MFMA is dead. Data: 0 random finite values (16-bit
// kinds: random sign and 10 (fp16) or 7 (bf16) mantissa bits, exponents within
// 8 binades; FP8: random E4M3 codes below the NaN code; FP4: random E2M1
// codes), 1 all zeros, 2 values with at most two significant bits (E2M1-like
// magnitudes times a power of two, as the NVFP4 decode forms them).
#include "bsq_device.h"
#include "bsq_internal.h"

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint32_t mix32(uint32_t x) {  // a 32-bit integer hash (xorshift-multiply)
  x ^= x >> 16; x *= 0x7FEB352Du; x ^= x >> 15; x *= 0x846CA68Bu; x ^= x >> 16;
  return x;
}
// one 16-bit operand: random sign, exponent within +-4 of 1, random mantissa (data 0)
// or a signed E2M1 magnitude times 2^e (data 2); `bf` selects bf16 bit layout
__device__ __forceinline__ uint32_t val16(uint32_t h, int data, bool bf) {
  if (data == 1) return 0u;
  const uint32_t s = (h >> 31) << 15;
  const uint32_t e = (h >> 24) & 7u;  // 0..7
  if (data == 0) {
    return bf ? s | ((123u + e) << 7) | (h & 0x7Fu) : s | ((11u + e) << 10) | (h & 0x3FFu);
  }
  // E2M1 magnitudes 0.5 .. 6 as (exponent, leading mantissa bit)
  const uint32_t c = 1u + (h & 7u) % 7u;  // codes 1..7
  const uint32_t ex = c < 2 ? 0u : (c < 4 ? 1u : (c < 6 ? 2u : 3u));
  const uint32_t m1 = (c == 3 || c == 5 || c == 7) ? 1u : 0u;
  return bf ? s | ((123u + e + ex) << 7) | (m1 << 6) : s | ((11u + e + ex) << 10) | (m1 << 9);
}
__device__ __forceinline__ uint32_t word16x2(uint32_t h, int data, bool bf) {
  return val16(mix32(h), data, bf) | (val16(mix32(h ^ 0x5bd1e995u), data, bf) << 16);
}
// four E4M3 bytes (NaN codes avoided) or eight E2M1 nibbles
__device__ __forceinline__ uint32_t word8(uint32_t h, int data, bool fp4) {
  if (data == 1) return 0u;
  const uint32_t r = mix32(h);
  if (fp4) return r;
  return data == 0 ? (r & 0xF7F7F7F7u) : (r & 0xB7B7B7B7u);  // exponents below 15 (no NaN)
}

template <int KIND>
__global__ __launch_bounds__(256) void k_mfma_rate(int data, int64_t iters, float* __restrict__ out) {
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  f32x16 acc[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[s][v] = 0.0f;
  if constexpr (KIND <= 1) {
    typedef typename std::conditional<KIND == 0, half8, bf16x8>::type V;
    V a[4], b[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint32_t wa[4], wb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wa[q] = word16x2(gid * 64u + s * 8u + q, data, KIND == 1);
        wb[q] = word16x2(gid * 64u + s * 8u + q + 4u + 0x9e37u, data, KIND == 1);
      }
      a[s] = __builtin_bit_cast(V, make_uint4(wa[0], wa[1], wa[2], wa[3]));
      b[s] = __builtin_bit_cast(V, make_uint4(wb[0], wb[1], wb[2], wb[3]));
    }
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if constexpr (KIND == 0)
          acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[s], b[(s + 1) & 3], acc[s], 0, 0, 0);
        else
          acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[(s + 1) & 3], acc[s], 0, 0, 0);
      }
    }
  } else if constexpr (KIND == 2) {
    long a[4], b[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      a[s] = (long)(((uint64_t)word8(gid * 64u + s * 8u + 1u, data, false) << 32) | word8(gid * 64u + s * 8u, data, false));
      b[s] = (long)(((uint64_t)word8(gid * 64u + s * 8u + 3u, data, false) << 32) | word8(gid * 64u + s * 8u + 2u, data, false));
    }
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(a[s], b[(s + 1) & 3], acc[s], 0, 0, 0);
    }
  } else {
    constexpr bool FP4 = KIND == 4;
    v8i a[4], b[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        a[s][q] = (int)word8(gid * 128u + s * 16u + q, data, FP4);
        b[s][q] = (int)word8(gid * 128u + s * 16u + q + 8u, data, FP4);
      }
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int s = 0; s < 4; ++s)  // E8M0 scale 127 (a factor of one) for both operands
        acc[s] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[s], b[(s + 1) & 3], acc[s], FP4 ? 4 : 0, FP4 ? 4 : 0,
                                                                 0, 127, 0, 127);
    }
  }
  float r = 0.0f;
#pragma unroll
  for (int s = 0; s < 4; ++s) r += acc[s][threadIdx.x & 15];
  out[gid] = r;
}

}  // namespace

extern "C" int bsq_mfma_rate_probe(int kind, int data, int64_t iters, int64_t workgroups, float* out,
                                   bsq_stream_t stream) {
  BSQ_REQUIRE(kind >= 0 && kind <= 4 && data >= 0 && data <= 2, BSQ_E_ENUM);
  BSQ_REQUIRE(iters >= 1 && iters <= ((int64_t)1 << 24) && workgroups >= 1 && workgroups <= 65535, BSQ_E_SHAPE);
  BSQ_REQUIRE(out, BSQ_E_NULL);
  BSQ_REQUIRE(((uintptr_t)out & 3) == 0, BSQ_E_ALIGN);
  hipStream_t s = bsqh::as_stream(stream);
  const dim3 grid((unsigned)workgroups), block(256);
  switch (kind) {
    case 0: hipLaunchKernelGGL(k_mfma_rate<0>, grid, block, 0, s, data, iters, out); break;
    case 1: hipLaunchKernelGGL(k_mfma_rate<1>, grid, block, 0, s, data, iters, out); break;
    case 2: hipLaunchKernelGGL(k_mfma_rate<2>, grid, block, 0, s, data, iters, out); break;
    case 3: hipLaunchKernelGGL(k_mfma_rate<3>, grid, block, 0, s, data, iters, out); break;
    default: hipLaunchKernelGGL(k_mfma_rate<4>, grid, block, 0, s, data, iters, out); break;
  }
  return bsqh::launch_status();
}
