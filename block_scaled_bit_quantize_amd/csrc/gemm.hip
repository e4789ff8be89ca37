// Expert grouped GEMMs: NVFP4 x NVFP4 forward (FPROP) and MXFP8 backward
// (DGRAD, WGRAD), exact-product path.
//
// "End-to-End 4-Bit Training", section "Block-scaled backward passes": the
// forward pass computes y = x_q w_q^T by pairing 16-value blocks of a row of
// x_q and a column of w_q^T and scaling each block sum by both block scales;
// the backward pass computes dx = g w_q and dw = g^T x_q from the transposed
// tensors. Section "Re-quantization with stochastic rounding": the backward
// GEMMs are MXFP8 (E4M3, one E8M0 scale per 32). Section "Quantized
// communications": each expert's GEMM covers the tokens routed to it; WGRAD
// reads the forward-quantized activations. Section "Recipe details": outer
// scales per token (activations) and per expert (weights).
//
// CDNA4 design. CDNA4's scaled FP4/FP8 MFMA takes one E8M0 scale per 32
// K-values: that cannot express NVFP4's E4M3 scale per 16, and (measured) the
// FP8 dot product inside one instruction keeps only about 15 bits below its
// largest product, which loses the small products of wide-range blocks. Both
// formats therefore decode each element once per workgroup tile into LDS as
// an exactly representable 16-bit value and contract on the dense 16-bit
// MFMA (v_mfma_f32_32x32x16_{f16,bf16}) with fp32 accumulation:
//   NVFP4: q * s_b (E2M1 x E4M3: at most 6 significant bits, within
//          [2^-10, 2688]) is exact in fp16; the two FP32 outer scales multiply
//          the fp32 sum in the epilogue.
//   MXFP8: q * 2^(s-127) (E4M3 x E8M0) is exact in bf16 for scale codes
//          10..246 (hardware scaled convert, which applies a power-of-two
//          scale); no epilogue scaling.
// Every product is exact; the only roundings are the fp32 accumulation and
// the output conversion (bf16 round-to-nearest-even, or fp32).
//
// Tiles: 256 x 256 outputs per workgroup of 4 waves (each wave 128 x 128 =
// 4 x 4 MFMAs of 32 x 32 x 16), K steps of 64 double-buffered in LDS (rows
// padded to 144 bytes: conflict-free 16-byte fragment reads), global loads
// one step ahead in registers. Tiles map to (expert, m-tile, n-tile) through
// an in-workgroup scan of the segment offsets; workgroups are remapped so each
// XCD (workgroup w runs on XCD w % 8) works on a contiguous range of tiles,
// keeping an expert's weights and its token rows in that XCD's L2.
//   FPROP/DGRAD (segments along M): row r of expert e reads A row a_row(r)
//     (gathered token for FPROP) and B[e]; out[r, n].
//   WGRAD (segments along K): A_e [M, Kp_e], B_e [N, Kp_e] in the padded
//     per-segment transposed layout; out[e, m, n].
#include "bsq_device.h"
#include "bsq_internal.h"

using namespace bsqd;

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kRow = BK * 2 + 16;  // LDS bytes per decoded row (16-bit values + pad)
constexpr int kMaxE = 1024;
constexpr int kXcds = 8;
enum { FMT_NVFP4 = 0, FMT_MXFP8 = 1 };

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// One row's operand data for one K step of 64 elements.
template <int FMT> struct RowData;
template <> struct RowData<FMT_NVFP4> {
  uint4 c[2];   // 64 E2M1 codes
  uint32_t sc;  // 4 E4M3 scales (one per 16)
};
template <> struct RowData<FMT_MXFP8> {
  uint4 c[4];   // 64 E4M3 codes
  uint32_t sc;  // 2 E8M0 scales (one per 32) in the low 16 bits
};

// Load K elements [k0, k0+64) of a row; elements at or past klen read as zero.
__device__ __forceinline__ void load_row(RowData<FMT_NVFP4>& r, const uint8_t* codes, const uint8_t* scales,
                                         int64_t k0, int64_t) {
  const uint4* p = reinterpret_cast<const uint4*>(codes + (k0 >> 1));
  r.c[0] = p[0];
  r.c[1] = p[1];
  r.sc = *reinterpret_cast<const uint32_t*>(scales + (k0 >> 4));
}
__device__ __forceinline__ void load_row(RowData<FMT_MXFP8>& r, const uint8_t* codes, const uint8_t* scales,
                                         int64_t k0, int64_t klen) {
  const uint4* p = reinterpret_cast<const uint4*>(codes + k0);
  if (k0 + BK <= klen) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.c[i] = p[i];
    r.sc = (uint32_t)scales[k0 >> 5] | ((uint32_t)scales[(k0 >> 5) + 1] << 8);
  } else {  // a segment's last 32 tokens (padded lengths are multiples of 32)
#pragma unroll
    for (int i = 0; i < 4; ++i) r.c[i] = k0 + 16 * i < klen ? p[i] : make_uint4(0, 0, 0, 0);
    r.sc = (uint32_t)scales[k0 >> 5] | (k0 + 32 < klen ? (uint32_t)scales[(k0 >> 5) + 1] << 8 : (127u << 8));
  }
}

// Decode 64 elements into 128 bytes of LDS.
__device__ __forceinline__ void decode_row(const RowData<FMT_NVFP4>& r, uint8_t* dst) {
  const uint32_t w[8] = {r.c[0].x, r.c[0].y, r.c[0].z, r.c[0].w, r.c[1].x, r.c[1].y, r.c[1].z, r.c[1].w};
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const _Float16 s = (_Float16)e4m3_val((r.sc >> (8 * (q >> 1))) & 0xFFu);
    const h2 sv = {s, s};
    const h2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[q], 1.0f, 0) * sv;
    const h2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[q], 1.0f, 1) * sv;
    const h2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[q], 1.0f, 2) * sv;
    const h2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[q], 1.0f, 3) * sv;
    *reinterpret_cast<uint4*>(dst + 16 * q) =
        make_uint4(__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1), __builtin_bit_cast(uint32_t, v2),
                   __builtin_bit_cast(uint32_t, v3));
  }
}
__device__ __forceinline__ void decode_row(const RowData<FMT_MXFP8>& r, uint8_t* dst) {
  const uint32_t w[16] = {r.c[0].x, r.c[0].y, r.c[0].z, r.c[0].w, r.c[1].x, r.c[1].y, r.c[1].z, r.c[1].w,
                          r.c[2].x, r.c[2].y, r.c[2].z, r.c[2].w, r.c[3].x, r.c[3].y, r.c[3].z, r.c[3].w};
  const float s0 = __uint_as_float((r.sc & 0xFFu) << 23);  // 2^(s-127): the convert applies its exponent
  const float s1 = __uint_as_float(((r.sc >> 8) & 0xFFu) << 23);
#pragma unroll
  for (int q = 0; q < 16; q += 2) {
    const float s = q < 8 ? s0 : s1;
    const bf2 v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q], s, false);
    const bf2 v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q], s, true);
    const bf2 v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q + 1], s, false);
    const bf2 v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[q + 1], s, true);
    *reinterpret_cast<uint4*>(dst + 8 * q) =
        make_uint4(__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1), __builtin_bit_cast(uint32_t, v2),
                   __builtin_bit_cast(uint32_t, v3));
  }
}

template <int FMT>
__device__ __forceinline__ f32x16 mfma16(const uint8_t* pa, const uint8_t* pb, f32x16 acc);
template <>
__device__ __forceinline__ f32x16 mfma16<FMT_NVFP4>(const uint8_t* pb, const uint8_t* pa, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(*reinterpret_cast<const half8*>(pb),
                                                *reinterpret_cast<const half8*>(pa), acc, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma16<FMT_MXFP8>(const uint8_t* pb, const uint8_t* pa, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(pb),
                                                 *reinterpret_cast<const bf16x8*>(pa), acc, 0, 0, 0);
}

struct GemmArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_outer;     // NVFP4: per token (a_outer_per_row) or one value
  int a_outer_per_row;
  int64_t a_rows;           // rows of the A table (gather bound)
  const int32_t* a_row_index;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  const float* b_outer;     // NVFP4: per expert
  const int64_t* seg_offsets;
  int E;
  int64_t M;                // M_total (segments along M) or rows per expert (WGRAD)
  int64_t N;
  int64_t K;                // shared K (segments along M)
  void* out;
};

template <int FMT, int WGRAD, int OUT_F32>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(const GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * kRow];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * kRow];
  __shared__ int64_t s_cum[kMaxE];  // inclusive m-tiles (along M) or padded tokens (WGRAD) per expert
  __shared__ int64_t s_part[kThreads];

  const int t = threadIdx.x;
  const int E = g.E;
  {
    int64_t loc[4];
    int64_t sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 4 * t + j;
      int64_t n = 0;
      if (e < E) {
        const int64_t len = g.seg_offsets[e + 1] - g.seg_offsets[e];
        n = len <= 0 ? 0 : (WGRAD ? (len + 31) / 32 * 32 : (len + BM - 1) / BM);
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
  const int64_t ntn = g.N / BN;
  const int64_t ntm_w = g.M / BM;
  const int64_t total = WGRAD ? (int64_t)E * ntm_w * ntn : s_cum[E - 1] * ntn;
  const int64_t per_xcd = (total + kXcds - 1) / kXcds;
  const int64_t w = blockIdx.x;
  const int64_t tile = (w % kXcds) * per_xcd + w / kXcds;
  if (w / kXcds >= per_xcd || tile >= total) return;

  int e;
  int64_t m0, n0, Me = 0, seg0 = 0, klen;
  const uint8_t *a_c, *a_s, *b_c, *b_s;
  if constexpr (WGRAD) {
    e = (int)(tile / (ntm_w * ntn));
    const int64_t r = tile % (ntm_w * ntn);
    m0 = (r / ntn) * BM;
    n0 = (r % ntn) * BN;
    const int64_t kbase = e ? s_cum[e - 1] : 0;  // sum of earlier padded token counts
    klen = s_cum[e] - kbase;
    a_c = g.a_codes + g.M * kbase + (m0 + t) * klen;
    a_s = g.a_scales + (g.M * kbase + (m0 + t) * klen) / 32;
    b_c = g.b_codes + g.N * kbase + (n0 + t) * klen;
    b_s = g.b_scales + (g.N * kbase + (n0 + t) * klen) / 32;
  } else {
    const int64_t mtg = tile / ntn;
    n0 = (tile % ntn) * BN;
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_cum[mid] > mtg) hi = mid; else lo = mid + 1;
    }
    e = lo;
    seg0 = g.seg_offsets[e];
    Me = g.seg_offsets[e + 1] - seg0;
    if (seg0 < 0 || seg0 + Me > g.M) return;  // malformed offsets: stay inside the buffers
    m0 = (mtg - (s_cum[e] - (Me + BM - 1) / BM)) * BM;
    klen = g.K;
    const int64_t m = m0 + t < Me ? m0 + t : Me - 1;
    int64_t arow = g.a_row_index ? (int64_t)g.a_row_index[seg0 + m] : seg0 + m;
    arow = arow < 0 ? 0 : (arow >= g.a_rows ? g.a_rows - 1 : arow);
    const int64_t brow = (int64_t)e * g.N + n0 + t;
    constexpr int CB = FMT == FMT_NVFP4 ? 2 : 1;   // elements per code byte
    constexpr int SB = FMT == FMT_NVFP4 ? 16 : 32;  // elements per scale
    a_c = g.a_codes + arow * (g.K / CB);
    a_s = g.a_scales + arow * (g.K / SB);
    b_c = g.b_codes + brow * (g.K / CB);
    b_s = g.b_scales + brow * (g.K / SB);
  }

  const int wave = t >> 6;
  const int lane = t & 63;
  const int wm = wave >> 1;  // 128-row half of the tile (m)
  const int wn = wave & 1;   // 128-col half of the tile (n)

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int nk = (int)((klen + BK - 1) / BK);
  RowData<FMT> ra, rb;
  if (nk > 0) {
    load_row(ra, a_c, a_s, 0, klen);
    load_row(rb, b_c, b_s, 0, klen);
    decode_row(ra, &sA[0][t * kRow]);
    decode_row(rb, &sB[0][t * kRow]);
    if (nk > 1) {
      load_row(ra, a_c, a_s, BK, klen);
      load_row(rb, b_c, b_s, BK, klen);
    }
  }
  __syncthreads();

  // fragment: lane -> row (lane & 31), k offset 8 * (lane >> 5) within each 16-wide k slice
  const int frag_off = (lane & 31) * kRow + (lane >> 5) * 16;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const uint8_t* pa = &sA[buf][(wm * 128) * kRow + frag_off];
    const uint8_t* pb = &sB[buf][(wn * 128) * kRow + frag_off];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      // D = B A^T: output rows are n, columns m (a lane keeps 4 consecutive n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = mfma16<FMT>(pb + j * 32 * kRow + ks * 32, pa + i * 32 * kRow + ks * 32, acc[i][j]);
    }
    if (kt + 1 < nk) {
      decode_row(ra, &sA[buf ^ 1][t * kRow]);
      decode_row(rb, &sB[buf ^ 1][t * kRow]);
      if (kt + 2 < nk) {
        load_row(ra, a_c, a_s, (int64_t)(kt + 2) * BK, klen);
        load_row(rb, b_c, b_s, (int64_t)(kt + 2) * BK, klen);
      }
    }
    __syncthreads();
  }

  // ---- epilogue
  const float sw = FMT == FMT_NVFP4 ? g.b_outer[e] : 1.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + wm * 128 + i * 32 + (lane & 31);
    if (!WGRAD && m >= Me) continue;
    float s = 1.0f;
    if constexpr (FMT == FMT_NVFP4) {
      float sx = g.a_outer[0];
      if (g.a_outer_per_row) {
        int64_t tok = g.a_row_index ? (int64_t)g.a_row_index[seg0 + m] : seg0 + m;
        tok = tok < 0 ? 0 : (tok >= g.a_rows ? g.a_rows - 1 : tok);
        sx = g.a_outer[tok];
      }
      s = sx * sw;
    }
    const int64_t obase = (WGRAD ? ((int64_t)e * g.M + m) : (seg0 + m)) * g.N + n0 + wn * 128;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = j * 32 + q * 8 + (lane >> 5) * 4;
        float v0 = acc[i][j][4 * q], v1 = acc[i][j][4 * q + 1], v2 = acc[i][j][4 * q + 2], v3 = acc[i][j][4 * q + 3];
        if constexpr (FMT == FMT_NVFP4) {
          v0 *= s; v1 *= s; v2 *= s; v3 *= s;
        }
        if constexpr (OUT_F32) {
          *reinterpret_cast<float4*>(static_cast<float*>(g.out) + obase + n) = make_float4(v0, v1, v2, v3);
        } else {  // round to nearest even
          const bf2 lo2 = __builtin_convertvector((f2){v0, v1}, bf2);
          const bf2 hi2 = __builtin_convertvector((f2){v2, v3}, bf2);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.out) + obase + n) =
              make_uint2(__builtin_bit_cast(uint32_t, lo2), __builtin_bit_cast(uint32_t, hi2));
        }
      }
  }
}

template <int FMT, int WGRAD>
int launch(const GemmArgs& a, int64_t slots, int out_dtype, hipStream_t s) {
  const int64_t grid = (slots + kXcds - 1) / kXcds * kXcds;
  if (out_dtype == BSQ_F32)
    hipLaunchKernelGGL((k_gemm<FMT, WGRAD, 1>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k_gemm<FMT, WGRAD, 0>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return bsqh::launch_status();
}

}  // namespace

extern "C" int bsq_grouped_gemm_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_outer,
                                      int a_outer_per_row, int64_t a_rows, const int32_t* a_row_index,
                                      const uint8_t* b_codes, const uint8_t* b_scales, const float* b_outer,
                                      const int64_t* seg_offsets, int64_t E, int64_t M_total, int64_t N, int64_t K,
                                      void* out, int out_dtype, bsq_stream_t stream) {
  BSQ_REQUIRE(out_dtype == BSQ_BF16 || out_dtype == BSQ_F32, BSQ_E_DTYPE);
  BSQ_REQUIRE(E >= 1 && E <= kMaxE && M_total >= 0 && N >= 0 && K >= 0 && a_rows >= 0, BSQ_E_SHAPE);
  BSQ_REQUIRE(N % BN == 0 && K % BK == 0, BSQ_E_SHAPE);
  if (M_total == 0 || N == 0) return BSQ_OK;
  BSQ_REQUIRE(K > 0 && a_rows > 0, BSQ_E_SHAPE);
  BSQ_REQUIRE(a_codes && a_scales && a_outer && b_codes && b_scales && b_outer && seg_offsets && out, BSQ_E_NULL);
  BSQ_REQUIRE(bsqh::aligned16(a_codes) && bsqh::aligned16(b_codes) && bsqh::aligned16(out), BSQ_E_ALIGN);
  BSQ_REQUIRE(((uintptr_t)a_scales & 3) == 0 && ((uintptr_t)b_scales & 3) == 0, BSQ_E_ALIGN);
  const GemmArgs a{a_codes, a_scales, a_outer, a_outer_per_row, a_rows, a_row_index, b_codes, b_scales, b_outer,
                   seg_offsets, (int)E, M_total, N, K, out};
  return launch<FMT_NVFP4, 0>(a, bsqh::tile_bound(M_total, E, BM) * (N / BN), out_dtype, bsqh::as_stream(stream));
}

extern "C" int bsq_grouped_gemm_mxfp8(int wgrad, const uint8_t* a_codes, const uint8_t* a_scales,
                                      const uint8_t* b_codes, const uint8_t* b_scales, const int64_t* seg_offsets,
                                      int64_t E, int64_t M_total, int64_t N, int64_t K, void* out, int out_dtype,
                                      bsq_stream_t stream) {
  BSQ_REQUIRE(wgrad == 0 || wgrad == 1, BSQ_E_ENUM);
  BSQ_REQUIRE(out_dtype == BSQ_BF16 || out_dtype == BSQ_F32, BSQ_E_DTYPE);
  BSQ_REQUIRE(E >= 1 && E <= kMaxE && M_total >= 0 && N >= 0 && K >= 0, BSQ_E_SHAPE);
  BSQ_REQUIRE(N % BN == 0, BSQ_E_SHAPE);
  if (wgrad) BSQ_REQUIRE(M_total % BM == 0, BSQ_E_SHAPE);
  else BSQ_REQUIRE(K % BK == 0, BSQ_E_SHAPE);
  if (M_total == 0 || N == 0) return BSQ_OK;
  if (!wgrad) BSQ_REQUIRE(K > 0, BSQ_E_SHAPE);
  BSQ_REQUIRE(a_codes && a_scales && b_codes && b_scales && seg_offsets && out, BSQ_E_NULL);
  BSQ_REQUIRE(bsqh::aligned16(a_codes) && bsqh::aligned16(b_codes) && bsqh::aligned16(out), BSQ_E_ALIGN);
  const GemmArgs a{a_codes, a_scales, nullptr, 0, M_total, nullptr, b_codes, b_scales, nullptr,
                   seg_offsets, (int)E, M_total, N, K, out};
  hipStream_t s = bsqh::as_stream(stream);
  if (wgrad) return launch<FMT_MXFP8, 1>(a, E * (M_total / BM) * (N / BN), out_dtype, s);
  return launch<FMT_MXFP8, 0>(a, bsqh::tile_bound(M_total, E, BM) * (N / BN), out_dtype, s);
}
