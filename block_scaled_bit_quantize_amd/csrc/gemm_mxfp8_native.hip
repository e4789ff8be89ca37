// MXFP8 expert grouped GEMMs (DGRAD, WGRAD) on the native scaled FP8 MFMA.
//
// Same operations as bsq_grouped_gemm_mxfp8 ("End-to-End 4-Bit Training",
// sections "Block-scaled backward passes" and "Re-quantization with
// stochastic rounding": dx = g w_q and dw = g^T x_q as MXFP8 GEMMs), computed
// with v_mfma_scale_f32_32x32x64_f8f6f4, which takes E4M3 operands and one
// E8M0 scale per 32 K-values per row -- the MX block, natively, at the FP8
// MFMA rate and with no decode.
//
// Accuracy: measured on gfx950, the FP8 dot product inside one instruction
// keeps roughly 15 bits below its largest product (errors of about 2^-15 of
// sum |products| for operands spanning the whole E4M3 range, about 2^-18 for
// quantized Gaussian data), so near-cancelling outputs can miss a relative
// 2e-3 bound; the exact-product path is bsq_grouped_gemm_mxfp8. This entry
// point is the faster alternative for callers that accept that error.
//
// In this instruction lane half h of a row holds K bytes [16h, 16h+16) and
// [32+16h, 48+16h) of the 64-wide K chunk and supplies the scale of K block
// h of that chunk (measured layout). Operands stay as raw bytes in LDS.
//
// Tiles: 256 x 256 outputs per workgroup of 4 waves (each wave 128 x 128 =
// 4 x 4 MFMAs), K steps of 128 double-buffered in LDS (rows padded to 144
// bytes), global loads one step ahead in registers.
//   DGRAD: segments along M. Row r of expert e: out[r, n] = sum_k A[r,k] B[e,n,k].
//   WGRAD: segments along K. out[e, m, n] = sum_t A_e[m,t] B_e[n,t], A_e/B_e in
//          the padded per-segment transposed layout ([M, Kp_e] / [N, Kp_e]).
#include "bsq_device.h"
#include "bsq_internal.h"

using namespace bsqd;

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 128;
constexpr int kThreads = 256;
constexpr int kRow = BK + 16;
constexpr int kMaxE = 1024;
constexpr int kXcds = 8;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));

struct Rows {
  uint4 a[8], b[8];
  uint32_t sa, sb;
};

// 128 bytes of a row starting at k0 (zero beyond klen) and its 4 scales (127 beyond).
__device__ __forceinline__ void load_row128(const uint8_t* codes_row, const uint8_t* scales_row, int64_t k0,
                                            int64_t klen, uint4* v, uint32_t& sc) {
  if (k0 + BK <= klen) {
    const uint4* p = reinterpret_cast<const uint4*>(codes_row + k0);
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = p[c];
    // byte loads: in the per-segment layout a row's scales may start at any byte
    const uint8_t* q = scales_row + (k0 >> 5);
    sc = (uint32_t)q[0] | ((uint32_t)q[1] << 8) | ((uint32_t)q[2] << 16) | ((uint32_t)q[3] << 24);
  } else {
    sc = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = k0 + 16 * c < klen ? reinterpret_cast<const uint4*>(codes_row + k0)[c] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int b = 0; b < 4; ++b) sc |= (k0 + 32 * b < klen ? (uint32_t)scales_row[(k0 >> 5) + b] : 127u) << (8 * b);
  }
}

__device__ __forceinline__ void store_row(uint8_t* dst, const uint4* v) {
#pragma unroll
  for (int c = 0; c < 8; ++c) *reinterpret_cast<uint4*>(dst + 16 * c) = v[c];
}

template <int WGRAD, int OUT_F32>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_mxfp8(const uint8_t* __restrict__ a_codes,
                                                            const uint8_t* __restrict__ a_scales,
                                                            const uint8_t* __restrict__ b_codes,
                                                            const uint8_t* __restrict__ b_scales,
                                                            const int64_t* __restrict__ seg_offsets, int E,
                                                            int64_t Mdim, int64_t N, int64_t K, void* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * kRow];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * kRow];
  __shared__ uint32_t sSA[2][BM];
  __shared__ uint32_t sSB[2][BN];
  __shared__ int64_t s_cum[kMaxE];
  __shared__ int64_t s_part[kThreads];

  const int t = threadIdx.x;
  // ---- per-expert prefix: m-tiles (DGRAD) or padded token counts (WGRAD)
  {
    int64_t loc[4];
    int64_t sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * t + j;
      int64_t n = 0;
      if (e < E) {
        const int64_t len = seg_offsets[e + 1] - seg_offsets[e];
        n = WGRAD ? (len + 31) / 32 * 32 : (len + BM - 1) / BM;
      }
      sum += n;
      loc[j] = sum;
    }
    s_part[t] = sum;
    __syncthreads();
    for (int o = 1; o < kThreads; o <<= 1) {
      const int64_t v = t >= o ? s_part[t - o] : 0;
      __syncthreads();
      s_part[t] += v;
      __syncthreads();
    }
    const int64_t before = s_part[t] - sum;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4 * t + j < E) s_cum[4 * t + j] = before + loc[j];
    __syncthreads();
  }
  const int64_t ntn = N / BN;
  const int64_t ntm_w = Mdim / BM;  // WGRAD: m-tiles per expert
  const int64_t total = WGRAD ? (int64_t)E * ntm_w * ntn : s_cum[E - 1] * ntn;
  const int64_t per_xcd = (total + kXcds - 1) / kXcds;
  const int64_t w = blockIdx.x;
  const int64_t tile = (w % kXcds) * per_xcd + w / kXcds;
  if (w / kXcds >= per_xcd || tile >= total) return;

  int e;
  int64_t m0, n0, Me = 0, seg0 = 0, klen;
  const uint8_t *a_c, *a_s, *b_c, *b_s;
  int64_t a_stride, b_stride;
  if constexpr (WGRAD) {
    e = (int)(tile / (ntm_w * ntn));
    const int64_t r = tile % (ntm_w * ntn);
    m0 = (r / ntn) * BM;
    n0 = (r % ntn) * BN;
    klen = s_cum[e] - (e ? s_cum[e - 1] : 0);  // Kp_e
    const int64_t kbase = e ? s_cum[e - 1] : 0;  // sum of earlier Kp
    a_stride = klen;
    b_stride = klen;
    a_c = a_codes + Mdim * kbase + (m0 + t) * klen;
    a_s = a_scales + (Mdim * kbase + (m0 + t) * klen) / 32;
    b_c = b_codes + N * kbase + (n0 + t) * klen;
    b_s = b_scales + (N * kbase + (n0 + t) * klen) / 32;
  } else {
    const int64_t mtg = tile / ntn;
    n0 = (tile % ntn) * BN;
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_cum[mid] > mtg) hi = mid; else lo = mid + 1;
    }
    e = lo;
    seg0 = seg_offsets[e];
    Me = seg_offsets[e + 1] - seg0;
    if (seg0 < 0 || seg0 + Me > Mdim) return;  // malformed offsets: stay inside the buffers
    m0 = (mtg - (s_cum[e] - (Me + BM - 1) / BM)) * BM;
    klen = K;
    a_stride = K;
    b_stride = K;
    const int64_t m = m0 + t < Me ? m0 + t : Me - 1;
    a_c = a_codes + (seg0 + m) * K;
    a_s = a_scales + (seg0 + m) * (K / 32);
    b_c = b_codes + ((int64_t)e * N + n0 + t) * K;
    b_s = b_scales + ((int64_t)e * N + n0 + t) * (K / 32);
  }
  (void)a_stride;
  (void)b_stride;

  const int wave = t >> 6;
  const int lane = t & 63;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int h = lane >> 5;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (int)((klen + BK - 1) / BK);
  uint4 va[8], vb[8];
  uint32_t sca = 0, scb = 0;
  if (nk > 0) {
    load_row128(a_c, a_s, 0, klen, va, sca);
    load_row128(b_c, b_s, 0, klen, vb, scb);
    store_row(&sA[0][t * kRow], va);
    store_row(&sB[0][t * kRow], vb);
    sSA[0][t] = sca;
    sSB[0][t] = scb;
    if (nk > 1) {
      load_row128(a_c, a_s, BK, klen, va, sca);
      load_row128(b_c, b_s, BK, klen, vb, scb);
    }
  }
  __syncthreads();

  const int frag_off = (lane & 31) * kRow + h * 16;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const uint8_t* pa = &sA[buf][(wm * 128) * kRow + frag_off];
    const uint8_t* pb = &sB[buf][(wn * 128) * kRow + frag_off];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      i32x8 fa[4], fb[4];
      int sa[4], sb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 a0 = *reinterpret_cast<const uint4*>(pa + i * 32 * kRow + kc * 64);
        const uint4 a1 = *reinterpret_cast<const uint4*>(pa + i * 32 * kRow + kc * 64 + 32);
        const uint4 b0 = *reinterpret_cast<const uint4*>(pb + i * 32 * kRow + kc * 64);
        const uint4 b1 = *reinterpret_cast<const uint4*>(pb + i * 32 * kRow + kc * 64 + 32);
        fa[i] = (i32x8){(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        fb[i] = (i32x8){(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
        sa[i] = (int)((sSA[buf][wm * 128 + i * 32 + (lane & 31)] >> (8 * (2 * kc + h))) & 0xFFu);
        sb[i] = (int)((sSB[buf][wn * 128 + i * 32 + (lane & 31)] >> (8 * (2 * kc + h))) & 0xFFu);
      }
      // D = B A^T: output rows are n, columns m (lane keeps 4 consecutive n).
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], 0, 0, 0, sb[j], 0, sa[i]);
    }
    if (kt + 1 < nk) {
      store_row(&sA[buf ^ 1][t * kRow], va);
      store_row(&sB[buf ^ 1][t * kRow], vb);
      sSA[buf ^ 1][t] = sca;
      sSB[buf ^ 1][t] = scb;
      if (kt + 2 < nk) {
        load_row128(a_c, a_s, (int64_t)(kt + 2) * BK, klen, va, sca);
        load_row128(b_c, b_s, (int64_t)(kt + 2) * BK, klen, vb, scb);
      }
    }
    __syncthreads();
  }

  // ---- epilogue: DGRAD rows of the segment, WGRAD the expert's [M, N] block
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + wm * 128 + i * 32 + (lane & 31);
    if (!WGRAD && m >= Me) continue;
    const int64_t obase = (WGRAD ? ((int64_t)e * Mdim + m) : (seg0 + m)) * N + n0 + wn * 128;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = j * 32 + g * 8 + h * 4;
        if constexpr (OUT_F32) {
          *reinterpret_cast<float4*>(static_cast<float*>(out) + obase + n) =
              make_float4(acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
        } else {  // round to nearest even
          const bf2 lo2 = __builtin_convertvector((f2){acc[i][j][4 * g], acc[i][j][4 * g + 1]}, bf2);
          const bf2 hi2 = __builtin_convertvector((f2){acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]}, bf2);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + obase + n) =
              make_uint2(__builtin_bit_cast(uint32_t, lo2), __builtin_bit_cast(uint32_t, hi2));
        }
      }
  }
}

}  // namespace

extern "C" int bsq_grouped_gemm_mxfp8_native(int wgrad, const uint8_t* a_codes, const uint8_t* a_scales,
                                      const uint8_t* b_codes, const uint8_t* b_scales, const int64_t* seg_offsets,
                                      int64_t E, int64_t M_total, int64_t N, int64_t K, void* out,
                                      int out_dtype, bsq_stream_t stream) {
  BSQ_REQUIRE(wgrad == 0 || wgrad == 1, BSQ_E_ENUM);
  BSQ_REQUIRE(out_dtype == BSQ_BF16 || out_dtype == BSQ_F32, BSQ_E_DTYPE);
  BSQ_REQUIRE(E >= 1 && E <= kMaxE && M_total >= 0 && N >= 0 && K >= 0, BSQ_E_SHAPE);
  BSQ_REQUIRE(N % BN == 0, BSQ_E_SHAPE);
  if (wgrad) BSQ_REQUIRE(M_total % BM == 0, BSQ_E_SHAPE);
  else BSQ_REQUIRE(K % BK == 0, BSQ_E_SHAPE);
  if (M_total == 0 || N == 0) return BSQ_OK;
  BSQ_REQUIRE(a_codes && a_scales && b_codes && b_scales && seg_offsets && out, BSQ_E_NULL);
  BSQ_REQUIRE(bsqh::aligned16(a_codes) && bsqh::aligned16(b_codes) && bsqh::aligned16(out), BSQ_E_ALIGN);
  BSQ_REQUIRE(((uintptr_t)a_scales & 3) == 0 && ((uintptr_t)b_scales & 3) == 0, BSQ_E_ALIGN);
  hipStream_t s = bsqh::as_stream(stream);
  if (wgrad) {
    const int64_t tiles = E * (M_total / BM) * (N / BN);
    const int64_t grid = (tiles + kXcds - 1) / kXcds * kXcds;
    if (out_dtype == BSQ_F32)
      hipLaunchKernelGGL((k_gemm_mxfp8<1, 1>), dim3((unsigned)grid), dim3(kThreads), 0, s, a_codes, a_scales, b_codes,
                         b_scales, seg_offsets, (int)E, M_total, N, K, out);
    else
      hipLaunchKernelGGL((k_gemm_mxfp8<1, 0>), dim3((unsigned)grid), dim3(kThreads), 0, s, a_codes, a_scales, b_codes,
                         b_scales, seg_offsets, (int)E, M_total, N, K, out);
  } else {
    if (K == 0) return BSQ_E_SHAPE;
    const int64_t slots = bsqh::tile_bound(M_total, E, BM) * (N / BN);
    const int64_t grid = (slots + kXcds - 1) / kXcds * kXcds;
    if (out_dtype == BSQ_F32)
      hipLaunchKernelGGL((k_gemm_mxfp8<0, 1>), dim3((unsigned)grid), dim3(kThreads), 0, s, a_codes, a_scales, b_codes,
                         b_scales, seg_offsets, (int)E, M_total, N, K, out);
    else
      hipLaunchKernelGGL((k_gemm_mxfp8<0, 0>), dim3((unsigned)grid), dim3(kThreads), 0, s, a_codes, a_scales, b_codes,
                         b_scales, seg_offsets, (int)E, M_total, N, K, out);
  }
  return bsqh::launch_status();
}
