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

// Decode elements [16c, 16c+16) of a row's K step into 32 bytes at dst + 32c.
__device__ __forceinline__ void decode_chunk(const RowData<FMT_NVFP4>& r, uint8_t* dst, int c) {
  const uint32_t w0 = c < 2 ? (c == 0 ? r.c[0].x : r.c[0].z) : (c == 2 ? r.c[1].x : r.c[1].z);
  const uint32_t w1 = c < 2 ? (c == 0 ? r.c[0].y : r.c[0].w) : (c == 2 ? r.c[1].y : r.c[1].w);
  const _Float16 s = (_Float16)e4m3_val((r.sc >> (8 * c)) & 0xFFu);  // one E4M3 scale per 16
  const h2 sv = {s, s};
#define BSQ_DEC4(w, v0, v1, v2, v3)                                 \
  const h2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sv; \
  const h2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sv; \
  const h2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sv; \
  const h2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sv;
  BSQ_DEC4(w0, a0, a1, a2, a3)
  BSQ_DEC4(w1, b0, b1, b2, b3)
#undef BSQ_DEC4
  uint4* d = reinterpret_cast<uint4*>(dst + 32 * c);
  d[0] = make_uint4(__builtin_bit_cast(uint32_t, a0), __builtin_bit_cast(uint32_t, a1), __builtin_bit_cast(uint32_t, a2),
                    __builtin_bit_cast(uint32_t, a3));
  d[1] = make_uint4(__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1), __builtin_bit_cast(uint32_t, b2),
                    __builtin_bit_cast(uint32_t, b3));
}
__device__ __forceinline__ void decode_chunk(const RowData<FMT_MXFP8>& r, uint8_t* dst, int c) {
  const uint4 v = r.c[c];
  // 2^(s-127) as a float: the scaled convert applies its exponent (one E8M0 scale per 32)
  const float s = __uint_as_float(((r.sc >> (8 * (c >> 1))) & 0xFFu) << 23);
#define BSQ_DEC2(w, p, q)                                              \
  const bf2 p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, s, false); \
  const bf2 q = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, s, true);
  BSQ_DEC2(v.x, a0, a1)
  BSQ_DEC2(v.y, a2, a3)
  BSQ_DEC2(v.z, b0, b1)
  BSQ_DEC2(v.w, b2, b3)
#undef BSQ_DEC2
  uint4* d = reinterpret_cast<uint4*>(dst + 32 * c);
  d[0] = make_uint4(__builtin_bit_cast(uint32_t, a0), __builtin_bit_cast(uint32_t, a1), __builtin_bit_cast(uint32_t, a2),
                    __builtin_bit_cast(uint32_t, a3));
  d[1] = make_uint4(__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1), __builtin_bit_cast(uint32_t, b2),
                    __builtin_bit_cast(uint32_t, b3));
}

template <int FMT> struct Frag { typedef half8 type; };
template <> struct Frag<FMT_MXFP8> { typedef bf16x8 type; };

__device__ __forceinline__ f32x16 mfma16(half8 b, half8 a, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma16(bf16x8 b, bf16x8 a, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc, 0, 0, 0);
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

// WN waves along N (2: 4 waves of 128 x 128, one wave per SIMD; 4: 8 waves of
// 128 x 64, two waves per SIMD so one wave's LDS/VMEM/barrier waits are
// covered by the other's MFMAs).
template <int FMT, int WGRAD, int OUT_F32, int WN>
__global__ __launch_bounds__(128 * WN) void k_gemm(const GemmArgs g) {
  constexpr int NT = 128 * WN;            // threads
  constexpr int TJ = 8 / WN;              // 32-wide n tiles per wave
  constexpr int RPT = (BM + BN) / NT;     // operand rows loaded and decoded per thread
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * kRow];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * kRow];
  __shared__ int64_t s_cum[kMaxE];  // inclusive m-tiles (along M) or padded tokens (WGRAD) per expert
  __shared__ int64_t s_part[256];

  const int t = threadIdx.x;
  const int E = g.E;
  // per-expert unit count: m-tiles (segments along M) or padded tokens (WGRAD)
  auto units = [&](int e) -> int64_t {
    const int64_t len = g.seg_offsets[e + 1] - g.seg_offsets[e];
    return len <= 0 ? 0 : (WGRAD ? (len + 31) / 32 * 32 : (len + BM - 1) / BM);
  };
  int64_t own = 0;  // units of experts 4t .. 4t+3
  if (t < 256) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4 * t + j < E) own += units(4 * t + j);
    s_part[t] = own;
  }
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {  // inclusive scan over the 256 partial sums
    const int64_t v = (t < 256 && t >= o) ? s_part[t - o] : 0;
    __syncthreads();
    if (t < 256) s_part[t] += v;
    __syncthreads();
  }
  if (t < 256) {
    int64_t run = s_part[t] - own;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4 * t + j < E) {
        run += units(4 * t + j);
        s_cum[4 * t + j] = run;
      }
  }
  __syncthreads();
  const int64_t ntn = g.N / BN;
  const int64_t ntm_w = g.M / BM;
  const int64_t total = WGRAD ? (int64_t)E * ntm_w * ntn : s_cum[E - 1] * ntn;
  const int64_t per_xcd = (total + kXcds - 1) / kXcds;
  const int64_t w = blockIdx.x;
  const int64_t tile = (w % kXcds) * per_xcd + w / kXcds;
  if (w / kXcds >= per_xcd || tile >= total) return;

  int e;
  int64_t m0, n0, Me = 0, seg0 = 0, klen;
  if constexpr (WGRAD) {
    e = (int)(tile / (ntm_w * ntn));
    const int64_t r = tile % (ntm_w * ntn);
    m0 = (r / ntn) * BM;
    n0 = (r % ntn) * BN;
    klen = s_cum[e] - (e ? s_cum[e - 1] : 0);  // Kp_e
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
  }

  // ---- the operand rows this thread loads and decodes: tile row id = t + r*NT
  // (ids below BM are A rows, the rest B rows)
  const uint8_t* rcode[RPT];
  const uint8_t* rscal[RPT];
  int ldst[RPT];  // byte offset of the row in sA / sB
  bool isA[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int id = t + r * NT;
    isA[r] = id < BM;
    const int lrow = isA[r] ? id : id - BM;
    ldst[r] = lrow * kRow;
    if constexpr (WGRAD) {
      const int64_t kbase = e ? s_cum[e - 1] : 0;  // sum of earlier padded token counts
      const int64_t off = isA[r] ? g.M * kbase + (m0 + lrow) * klen : g.N * kbase + (n0 + lrow) * klen;
      rcode[r] = (isA[r] ? g.a_codes : g.b_codes) + off;
      rscal[r] = (isA[r] ? g.a_scales : g.b_scales) + off / 32;
    } else {
      constexpr int CB = FMT == FMT_NVFP4 ? 2 : 1;   // elements per code byte
      constexpr int SB = FMT == FMT_NVFP4 ? 16 : 32;  // elements per scale
      int64_t row;
      if (isA[r]) {
        const int64_t m = m0 + lrow < Me ? m0 + lrow : Me - 1;
        row = g.a_row_index ? (int64_t)g.a_row_index[seg0 + m] : seg0 + m;
        row = row < 0 ? 0 : (row >= g.a_rows ? g.a_rows - 1 : row);
      } else {
        row = (int64_t)e * g.N + n0 + lrow;
      }
      rcode[r] = (isA[r] ? g.a_codes : g.b_codes) + row * (g.K / CB);
      rscal[r] = (isA[r] ? g.a_scales : g.b_scales) + row * (g.K / SB);
    }
  }

  const int wave = t >> 6;
  const int lane = t & 63;
  const int wm = wave / WN;  // 128-row half of the tile (m)
  const int wn = wave % WN;  // (256/WN)-column slice of the tile (n)

  f32x16 acc[4][TJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

  const int nk = (int)((klen + BK - 1) / BK);
  typedef typename Frag<FMT>::type V8;
  // fragment: lane -> row (lane & 31), k offset 8 * (lane >> 5) within each 16-wide k slice
  const int frag_off = (lane & 31) * kRow + (lane >> 5) * 16;
  const int a_off = wm * 128 * kRow + frag_off;
  const int b_off = wn * (256 / WN) * kRow + frag_off;
  V8 fa[2][4], fb[2][TJ];
#define BSQ_LOAD_FRAGS(slot, buf, ks)                                                              \
  _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) fa[slot][i_] =                                  \
      *reinterpret_cast<const V8*>(&sA[buf][a_off + i_ * 32 * kRow + (ks) * 32]);                  \
  _Pragma("unroll") for (int j_ = 0; j_ < TJ; ++j_) fb[slot][j_] =                                 \
      *reinterpret_cast<const V8*>(&sB[buf][b_off + j_ * 32 * kRow + (ks) * 32]);
#define BSQ_DST(buf, r) (isA[r] ? &sA[buf][ldst[r]] : &sB[buf][ldst[r]])
  RowData<FMT> rd[RPT];
  if (nk > 0) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      load_row(rd[r], rcode[r], rscal[r], 0, klen);
#pragma unroll
      for (int c = 0; c < 4; ++c) decode_chunk(rd[r], BSQ_DST(0, r), c);
      load_row(rd[r], rcode[r], rscal[r], nk > 1 ? BK : 0, klen);
    }
    __syncthreads();
    BSQ_LOAD_FRAGS(0, 0, 0)
  }

  // Software pipeline per K step (one scheduling region, no branches): for each
  // 16-wide k slice, read the next slice's fragments, run this slice's MFMAs
  // and decode one quarter of the next K step into the other LDS buffer; then
  // fetch the K step after next (clamped: the last iteration decodes and loads
  // a duplicate that is never read) and swap buffers at the barrier.
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3) {
        BSQ_LOAD_FRAGS((ks + 1) & 1, buf, ks + 1)
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = mfma16(fb[ks & 1][j], fa[ks & 1][i], acc[i][j]);
#pragma unroll
      for (int r = 0; r < RPT; ++r) decode_chunk(rd[r], BSQ_DST(buf ^ 1, r), ks);
      // interleave each MFMA with a few decode VALU ops, the fragment reads and the decode stores
#pragma unroll
      for (int m = 0; m < 4 * TJ; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                         // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 12 * RPT / TJ, 0);             // VALU
        if (m < 4 + TJ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);         // DS read
        if (m >= 4 * TJ - 2 * RPT) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
      }
    }
    const int64_t knext = (int64_t)(kt + 2 < nk ? kt + 2 : nk - 1) * BK;
#pragma unroll
    for (int r = 0; r < RPT; ++r) load_row(rd[r], rcode[r], rscal[r], knext, klen);
    __syncthreads();
    BSQ_LOAD_FRAGS(0, buf ^ 1, 0)
  }
#undef BSQ_LOAD_FRAGS
#undef BSQ_DST

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
    const int64_t obase = (WGRAD ? ((int64_t)e * g.M + m) : (seg0 + m)) * g.N + n0 + wn * (256 / WN);
#pragma unroll
    for (int j = 0; j < TJ; ++j)
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

#ifndef BSQ_GEMM_WN
#define BSQ_GEMM_WN 4
#endif

template <int FMT, int WGRAD>
int launch(const GemmArgs& a, int64_t slots, int out_dtype, hipStream_t s) {
  constexpr int WN = BSQ_GEMM_WN;
  const int64_t grid = (slots + kXcds - 1) / kXcds * kXcds;
  if (out_dtype == BSQ_F32)
    hipLaunchKernelGGL((k_gemm<FMT, WGRAD, 1, WN>), dim3((unsigned)grid), dim3(128 * WN), 0, s, a);
  else
    hipLaunchKernelGGL((k_gemm<FMT, WGRAD, 0, WN>), dim3((unsigned)grid), dim3(128 * WN), 0, s, a);
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
