// Combine codec: 32-point random Hadamard transform + block-scaled S2F6.
//
// "End-to-End 4-Bit Training", section "Quantized communications": before the
// combine exchange each expert output row is rotated by a 32-dimensional
// random Hadamard transform (orthonormal: energy kept, inverted exactly) and
// quantized to S2F6 (fixed point with two signed integer bits and six
// fractional bits, values k/64 for k in [-128, 127]) with one UE8M0 scale per
// 32 values, 8.25 bits per value; the receiver dequantizes and aggregates the
// copies of each token, then inverts the transform.
//
// The transform is H D / sqrt(32) (D: 32 signs given as a bit mask, H the
// Sylvester Hadamard matrix), computed in float32 as the fast Walsh-Hadamard
// butterfly (stages of span 1, 2, 4, 8, 16, each (a, b) -> (a + b, a - b)) and
// one multiply by f32(1/sqrt(32)); the scale is the smallest 2^e with
// max|z| <= (127/64) 2^e (e in [-127, 127], -127 for a zero block) and each
// code is round-half-even(z 2^(6-e)) saturated to [-128, 127]. The combine sums
// a token's dequantized copies in slot order, then applies D H / sqrt(32).
//
// HBM-bound: one thread per block of 32, which it holds in registers; the
// butterfly is 80 additions and 80 subtractions per block (5 per value). A
// wave reads and writes contiguous runs (64 consecutive blocks); the combine's
// gathered rows are whole rows per wave, since the 64 lanes of a wave take 64
// consecutive blocks of one token.
#include "bsq_device.h"
#include "bsq_internal.h"

using namespace bsqd;

namespace {

constexpr int kThreads = 256;

template <typename T>
__global__ __launch_bounds__(kThreads) void k_rht_s2f6_encode(const T* __restrict__ x, int64_t nblk, uint32_t signs,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ scales) {
  const int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (blk >= nblk) return;
  float v[32];
  const uint4* src = reinterpret_cast<const uint4*>(x + blk * 32);
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 w = src[q];
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * q + 2 * i] = bf16_lo(u[i]);
        v[8 * q + 2 * i + 1] = bf16_hi(u[i]);
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint4 w = src[q];
      v[4 * q] = __uint_as_float(w.x);
      v[4 * q + 1] = __uint_as_float(w.y);
      v[4 * q + 2] = __uint_as_float(w.z);
      v[4 * q + 3] = __uint_as_float(w.w);
    }
  }
  uint32_t w[8];
  const uint32_t sc = rht_s2f6_block(v, signs, w);
  uint4* dst = reinterpret_cast<uint4*>(codes + blk * 32);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  scales[blk] = (uint8_t)sc;
}

// Token t, block b of cols/32: sum of the dequantized blocks of rows
// pair_row[t*k + j], j = 0..k-1 (indices clamped into [0, rows)), then the
// inverse transform; OUT_F32 selects float32 or bf16 (round to nearest even).
template <bool OUT_F32>
__global__ __launch_bounds__(kThreads) void k_rht_s2f6_combine(const uint8_t* __restrict__ codes,
                                                              const uint8_t* __restrict__ scales, int64_t rows,
                                                              int64_t bpr, const int32_t* __restrict__ pair_row,
                                                              int64_t tokens, int64_t k, uint32_t signs,
                                                              void* __restrict__ out) {
  const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (id >= tokens * bpr) return;
  const int64_t t = id / bpr, b = id % bpr;
  float v[32];
  for (int64_t j = 0; j < k; ++j) {
    int64_t r = pair_row[t * k + j];
    r = r < 0 ? 0 : (r >= rows ? rows - 1 : r);
    const uint4* src = reinterpret_cast<const uint4*>(codes + (r * bpr + b) * 32);
    const uint4 c0 = src[0], c1 = src[1];
    const int sh = (int)scales[r * bpr + b] - 127 - 6;
    const uint32_t u[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int q = (int)(int8_t)((u[i >> 2] >> (8 * (i & 3))) & 0xFFu);
      const float d = ldexpf((float)q, sh);  // k/64 * 2^e, exact
      v[i] = j == 0 ? d : v[i] + d;
    }
  }
  fwht32(v);
  const float c = __uint_as_float(kInvSqrt32);
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = __uint_as_float(__float_as_uint(v[i] * c) ^ (((signs >> i) & 1u) << 31));
  if constexpr (OUT_F32) {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(out) + id * 32);
#pragma unroll
    for (int q = 0; q < 8; ++q) dst[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  } else {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){v[2 * i], v[2 * i + 1]}, bf2));
    uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + id * 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
  }
}

inline unsigned grid1(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

}  // namespace

extern "C" int bsq_rht_s2f6_encode(const void* x, int dtype, int64_t rows, int64_t cols, uint32_t signs,
                                   uint8_t* codes, uint8_t* scales, bsq_stream_t stream) {
  BSQ_REQUIRE(dtype == BSQ_F32 || dtype == BSQ_BF16, BSQ_E_DTYPE);
  BSQ_REQUIRE(rows >= 0 && cols >= 0 && cols % 32 == 0, BSQ_E_SHAPE);
  // one thread per block: at most 2^38 blocks keeps the grid below 2^31 workgroups
  BSQ_REQUIRE(rows == 0 || cols == 0 || (rows <= ((int64_t)1 << 38) && cols <= ((int64_t)1 << 38) &&
                                         rows <= (((int64_t)1 << 38) / (cols / 32 > 0 ? cols / 32 : 1))),
              BSQ_E_SHAPE);
  const int64_t nblk = rows * (cols / 32);
  if (nblk == 0) return BSQ_OK;
  BSQ_REQUIRE(x && codes && scales, BSQ_E_NULL);
  BSQ_REQUIRE(bsqh::aligned16(x) && bsqh::aligned16(codes), BSQ_E_ALIGN);
  hipStream_t s = bsqh::as_stream(stream);
  if (dtype == BSQ_BF16)
    hipLaunchKernelGGL(k_rht_s2f6_encode<uint16_t>, dim3(grid1(nblk)), dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(x), nblk, signs, codes, scales);
  else
    hipLaunchKernelGGL(k_rht_s2f6_encode<float>, dim3(grid1(nblk)), dim3(kThreads), 0, s,
                       static_cast<const float*>(x), nblk, signs, codes, scales);
  return bsqh::launch_status();
}

extern "C" int bsq_rht_s2f6_combine(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                                    const int32_t* pair_row, int64_t tokens, int64_t k, uint32_t signs, void* out,
                                    int out_dtype, bsq_stream_t stream) {
  BSQ_REQUIRE(out_dtype == BSQ_F32 || out_dtype == BSQ_BF16, BSQ_E_DTYPE);
  BSQ_REQUIRE(rows >= 0 && cols >= 0 && cols % 32 == 0 && tokens >= 0 && k >= 1 && k <= 64, BSQ_E_SHAPE);
  // offsets stay inside int64 and the grid (one thread per token block) below 2^31 workgroups
  BSQ_REQUIRE(cols <= ((int64_t)1 << 31) && rows <= ((int64_t)1 << 40) / (cols > 0 ? cols : 1) &&
                  tokens <= ((int64_t)1 << 38) / (cols / 32 > 0 ? cols / 32 : 1) && tokens <= ((int64_t)1 << 40) / k,
              BSQ_E_SHAPE);
  const int64_t bpr = cols / 32;
  if (tokens == 0 || bpr == 0) return BSQ_OK;
  BSQ_REQUIRE(rows >= 1, BSQ_E_SHAPE);
  BSQ_REQUIRE(codes && scales && pair_row && out, BSQ_E_NULL);
  BSQ_REQUIRE(bsqh::aligned16(codes) && bsqh::aligned16(out) && ((uintptr_t)pair_row & 3) == 0, BSQ_E_ALIGN);
  hipStream_t s = bsqh::as_stream(stream);
  if (out_dtype == BSQ_F32)
    hipLaunchKernelGGL(k_rht_s2f6_combine<true>, dim3(grid1(tokens * bpr)), dim3(kThreads), 0, s, codes, scales,
                       rows, bpr, pair_row, tokens, k, signs, out);
  else
    hipLaunchKernelGGL(k_rht_s2f6_combine<false>, dim3(grid1(tokens * bpr)), dim3(kThreads), 0, s, codes, scales,
                       rows, bpr, pair_row, tokens, k, signs, out);
  return bsqh::launch_status();
}
