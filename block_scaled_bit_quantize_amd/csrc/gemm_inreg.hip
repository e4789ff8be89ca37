// NVFP4 x NVFP4 GEMM with the block scales applied in registers: the other
// way to handle NVFP4's scales on CDNA4, kept to measure it against the
// exact 16-bit decode of gemm.hip.
//
// "End-to-End 4-Bit Training", section "Kernels for low-precision training":
// on hardware without a native NVFP4 MMA the E4M3 scale per 16 values is
// handled either by decoding the values (scale applied before the MMA) or
// by block-wise MMAs whose partial sums are scaled in registers. Section
// "Block-scaled backward passes" defines the product: each 16-value block
// pair contributes s_a * s_w * sum q_a q_w.
//
// Here every 16-value block pair is one FP8 MFMA (v_mfma_f32_32x32x16_fp8_fp8)
// over the E2M1 values converted to E4M3 (exactly: every E2M1 value is an
// E4M3 value). Its 16 products are multiples of 1/4 below 36 in magnitude, so
// the instruction's partial sum is exact; each of the 16 partial sums a lane
// holds is then multiplied into the fp32 accumulator with its own scale
// product s_a(row) * s_w(col) (exact: two 4-bit significands). Accurate, but
// each 16-cycle MFMA brings about 50 vector instructions (scale decode,
// scale products, fused multiply-adds, value conversion), so the kernel is
// bound by the vector ALU far below the FP8 MFMA rate.
//
// Dense single-expert form: out[m, n] = a_outer[m] * b_outer[0] *
// sum_k xq[m, k] wq[n, k], fp32 output. M % 128 == 0, N % 128 == 0,
// K % 64 == 0. Workgroups of 4 waves own 128 x 128 outputs (64 x 64 per
// wave); K advances in chunks of 64 (four blocks) staged in LDS.
#include "bsq_device.h"
#include "bsq_internal.h"

using namespace bsqd;

namespace {

constexpr int TM = 128;       // rows of A (tokens) per workgroup
constexpr int TN = 128;       // rows of B (output columns) per workgroup
constexpr int KC = 64;        // K values per chunk: four NVFP4 blocks
constexpr int P = 36;         // LDS pitch of a row's 32 code bytes (odd dword pitch: conflict-free reads)

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f2 __attribute__((ext_vector_type(2)));

// Eight E2M1 codes (one 32-bit word, element 2k in the low nibble of byte k)
// as eight E4M3 bytes (a 64-bit MFMA operand, element k in byte k).
__device__ __forceinline__ long fp4x8_to_fp8x8(uint32_t w) {
  uint32_t lo = 0, hi = 0;
  f2 v;
  v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], lo, false);
  v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], lo, true);
  v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], hi, false);
  v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], hi, true);
  return (long)(((uint64_t)hi << 32) | lo);
}

__global__ __launch_bounds__(256) void k_gemm_nvfp4_inreg(const uint8_t* __restrict__ a_codes,
                                                         const uint8_t* __restrict__ a_scales,
                                                         const float* __restrict__ a_outer,
                                                         const uint8_t* __restrict__ b_codes,
                                                         const uint8_t* __restrict__ b_scales,
                                                         const float* __restrict__ b_outer, int64_t N, int64_t K,
                                                         float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t sa[TM * P];
  __shared__ __attribute__((aligned(16))) uint8_t sb[TN * P];
  __shared__ uint32_t ssa[TM];  // the chunk's four E4M3 scales of each row
  __shared__ uint32_t ssb[TN];
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int r = lane & 31, h = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.y * TM, n0 = (int64_t)blockIdx.x * TN;
  const int64_t kb_row = K / 2, ks_row = K / 16;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int ld_row = t >> 1, ld_half = t & 1;  // 2 threads per row, 16 code bytes each
  for (int64_t kc = 0; kc < K / KC; ++kc) {
    const uint4 va = *reinterpret_cast<const uint4*>(a_codes + (m0 + ld_row) * kb_row + kc * 32 + 16 * ld_half);
    const uint4 vb = *reinterpret_cast<const uint4*>(b_codes + (n0 + ld_row) * kb_row + kc * 32 + 16 * ld_half);
    uint32_t sc = 0;
    if (t < TM) sc = *reinterpret_cast<const uint32_t*>(a_scales + (m0 + t) * ks_row + 4 * kc);
    else sc = *reinterpret_cast<const uint32_t*>(b_scales + (n0 + t - TM) * ks_row + 4 * kc);
    __syncthreads();  // the previous chunk's reads are done
    uint32_t* da = reinterpret_cast<uint32_t*>(sa + ld_row * P + 16 * ld_half);
    uint32_t* db = reinterpret_cast<uint32_t*>(sb + ld_row * P + 16 * ld_half);
    da[0] = va.x; da[1] = va.y; da[2] = va.z; da[3] = va.w;
    db[0] = vb.x; db[1] = vb.y; db[2] = vb.z; db[3] = vb.w;
    if (t < TM) ssa[t] = sc;
    else ssb[t - TM] = sc;
    __syncthreads();
    // scales of the lane's rows: A row 32 i + r (one per lane and i), B rows
    // 32 j + 8 (v / 4) + 4 h + v % 4 (the 16 output rows of accumulator v)
    uint32_t wa[2], wb[2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i) wa[i] = ssa[wm * 64 + 32 * i + r];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) wb[j][v] = ssb[wn * 64 + 32 * j + 8 * (v >> 2) + 4 * h + (v & 3)];
#pragma unroll
    for (int kb = 0; kb < KC / 16; ++kb) {
      long fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = fp4x8_to_fp8x8(*reinterpret_cast<const uint32_t*>(sa + (wm * 64 + 32 * i + r) * P + 8 * kb + 4 * h));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = fp4x8_to_fp8x8(*reinterpret_cast<const uint32_t*>(sb + (wn * 64 + 32 * j + r) * P + 8 * kb + 4 * h));
      float s_a[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) s_a[i] = e4m3_val((wa[i] >> (8 * kb)) & 0xFFu);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float s_b[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) s_b[v] = e4m3_val((wb[j][v] >> (8 * kb)) & 0xFFu);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          f32x16 zero;
#pragma unroll
          for (int v = 0; v < 16; ++v) zero[v] = 0.0f;
          // C[n][m]: B rows along the output's rows, A rows along its columns (lane's m = 32 i + r)
          const f32x16 part = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(fb[j], fa[i], zero, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][j][v] = fmaf(part[v], s_a[i] * s_b[v], acc[i][j][v]);
        }
      }
    }
  }
  // out[m, n] = acc * f32(a_outer[m] * b_outer): four consecutive n per float4
  const float sw = b_outer[0];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t m = m0 + wm * 64 + 32 * i + r;
    const float s = a_outer[m] * sw;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = n0 + wn * 64 + 32 * j + 8 * q + 4 * h;
        *reinterpret_cast<float4*>(out + m * N + n) =
            make_float4(acc[i][j][4 * q] * s, acc[i][j][4 * q + 1] * s, acc[i][j][4 * q + 2] * s,
                        acc[i][j][4 * q + 3] * s);
      }
  }
}

}  // namespace

extern "C" int bsq_gemm_nvfp4_inreg_scale(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_outer,
                                          const uint8_t* b_codes, const uint8_t* b_scales, const float* b_outer,
                                          int64_t M, int64_t N, int64_t K, float* out, bsq_stream_t stream) {
  BSQ_REQUIRE(M >= 0 && N >= 0 && K >= 0, BSQ_E_SHAPE);
  BSQ_REQUIRE(M % TM == 0 && N % TN == 0 && K % KC == 0, BSQ_E_SHAPE);
  BSQ_REQUIRE(M / TM <= 65535 && N / TN <= 0x7FFFFFFF, BSQ_E_SHAPE);
  if (M == 0 || N == 0) return BSQ_OK;
  BSQ_REQUIRE(K > 0, BSQ_E_SHAPE);
  BSQ_REQUIRE(a_codes && a_scales && a_outer && b_codes && b_scales && b_outer && out, BSQ_E_NULL);
  BSQ_REQUIRE(bsqh::aligned16(a_codes) && bsqh::aligned16(b_codes) && bsqh::aligned16(out), BSQ_E_ALIGN);
  BSQ_REQUIRE(((uintptr_t)a_scales & 3) == 0 && ((uintptr_t)b_scales & 3) == 0, BSQ_E_ALIGN);
  hipLaunchKernelGGL(k_gemm_nvfp4_inreg, dim3((unsigned)(N / TN), (unsigned)(M / TM)), dim3(256), 0,
                     bsqh::as_stream(stream), a_codes, a_scales, a_outer, b_codes, b_scales, b_outer, N, K, out);
  return bsqh::launch_status();
}
