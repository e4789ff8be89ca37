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
// formats therefore contract exactly representable 16-bit values on the
// dense 16-bit MFMA (v_mfma_f32_32x32x16_{f16,bf16}) with fp32 accumulation:
//   NVFP4: q * s_b (E2M1 x E4M3: at most 6 significant bits, within
//          [2^-10, 2688]) is exact in fp16; the two FP32 outer scales multiply
//          the fp32 sum in the epilogue.
//   MXFP8: q * 2^(s-127) (E4M3 x E8M0) is exact in bf16 for scale codes
//          10..246 (the hardware scaled convert applies the power-of-two
//          scale); no epilogue scaling.
// Each element is decoded once per workgroup into LDS (a per-wave decode in
// registers repeats it for every wave that reads the row).
// Every product is exact; the only roundings are the fp32 accumulation and
// the output conversion (bf16 round-to-nearest-even, or fp32).
//
// Tiles: 256 x 256 outputs, 8 waves (2 along m x 4 along n, each wave
// 128 x 64 = 4 x 2 MFMAs of 32 x 32 x 16; two waves per SIMD so one wave's
// LDS, memory and barrier waits are covered by the other's MFMAs), K steps of
// 64 double-buffered in LDS (row pitches chosen so 16-byte fragment reads and
// row writes are bank-conflict free), global loads issued a step ahead into
// two register sets. Persistent workgroups (one per CU) walk contiguous tile
// ranges of their XCD (workgroup w runs on XCD w % 8), keeping an expert's
// weights and token rows in that XCD's L2; tiles map to (expert, m-tile,
// n-tile) through one in-workgroup scan of the segment offsets. A segment's
// last m-tile with at most 128 rows runs as a tail tile: both wave halves
// on its first 128 rows, each over half of every K step's slices.
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
constexpr int kRow = BK * 2 + 16;   // LDS bytes per row of decoded 16-bit values (+ pad)
constexpr int kMaxE = 1024;
constexpr int64_t kMaxRows = 0x7FFFFFFF - 1;  // segments along M: rows (offsets in LDS are int32)
constexpr int kXcds = 8;
#ifndef BSQ_GEMM_WN
#define BSQ_GEMM_WN 4
#endif
// Waves along n. 4: 8 waves of 128 x 64 outputs, two per SIMD, so one wave's
// LDS, memory and barrier waits are covered by the other's MFMAs. 2: 4 waves
// of 128 x 128, one per SIMD (a third fewer LDS bytes per MFMA).
constexpr int WN = BSQ_GEMM_WN;
constexpr int kThreads = 128 * WN;
constexpr int TJ = 8 / WN;          // 32-wide n tiles per wave

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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
  void* out;                // bf16 / fp32 output, or the S2F6 codes [M_total, N]
  uint8_t* out_scales;      // S2F6 output: UE8M0 scales [M_total, N/32]
  uint32_t signs;           // S2F6 output: the RHT's sign mask
};

enum { OUT_BF16 = 0, OUT_F32 = 1, OUT_S2F6 = 2 };


struct Tile {
  int e;
  int64_t m0, n0;
  int64_t Me, seg0;  // segment rows and first row (segments along M)
  int64_t klen;      // K extent (WGRAD: the expert's padded token count)
  int64_t kbase;     // WGRAD: padded tokens of the experts before e
};

// Per-expert unit counts (m-tiles for segments along M, padded tokens for
// WGRAD), scanned inside the workgroup into s_cum (inclusive). Segments along
// M also keep their offsets in s_seg (int32, clamped to [-1, M + 1]: the
// host bounds M below 2^31 - 1, and the clamp keeps every malformed-offset
// test of tile_coords unchanged), so that starting a tile reads no global
// memory: a global read there would wait for the previous tile's stores,
// which share its counter. Every thread calls it; returns the number of
// output tiles.
template <int WGRAD, int TBM>
__device__ int64_t scan_units(const GemmArgs& g, int64_t* s_cum, int64_t* s_part, int32_t* s_seg) {
  const int t = threadIdx.x;
  const int E = g.E;
  if (!WGRAD) {
    for (int e = t; e <= E; e += kThreads) {
      const int64_t v = g.seg_offsets[e];
      s_seg[e] = (int32_t)(v < -1 ? -1 : (v > g.M + 1 ? g.M + 1 : v));
    }
  }
  auto units = [&](int e) -> int64_t {
    const int64_t len = g.seg_offsets[e + 1] - g.seg_offsets[e];
    return len <= 0 ? 0 : (WGRAD ? (len + 31) / 32 * 32 : (len + TBM - 1) / TBM);
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
  return WGRAD ? (int64_t)E * (g.M / TBM) * ntn : s_cum[E - 1] * ntn;
}

// Order of an expert's tiles: groups of GN n-tiles, all m-tiles of a group
// before the next group, n fastest inside a group. The workgroups of one XCD
// run about 32 consecutive tiles at a time, roughly in step along K, so a
// group keeps (rows of the group's m-tiles + rows of its n-tiles) per K step
// in that XCD's L2 rather than every n-tile of the expert. Measured: groups
// of 4 take 1-3% off the MXFP8 GEMMs (16 n-tiles of 256) and 0-2% off the
// NVFP4 forward (6 n-tiles; 8 n-tiles at hidden 7168: 1-2%); groups of 2 no
// better.
template <int GN>
__device__ __forceinline__ void group_mn(int64_t li, int64_t mt, int64_t ntn, int64_t& m, int64_t& n) {
  const int64_t grp = li / (mt * GN);               // the groups before it are whole
  const int64_t rem = li - grp * mt * GN;
  const int64_t n0 = grp * GN;
  const int64_t w = ntn - n0 < GN ? ntn - n0 : GN;
  m = rem / w;
  n = n0 + rem % w;
}

// Coordinates of tile `tile` (tiles run expert by expert, in the group order
// above); false for malformed segment offsets (the tile is skipped, uniformly).
template <int WGRAD, int TBM, int GN>
__device__ bool tile_coords(const GemmArgs& g, const int64_t* s_cum, const int32_t* s_seg, int64_t tile, Tile& tl) {
  const int64_t ntn = g.N / BN;
  tl.Me = 0;
  tl.seg0 = 0;
  tl.kbase = 0;
  if constexpr (WGRAD) {
    const int64_t ntm = g.M / TBM;
    tl.e = (int)(tile / (ntm * ntn));
    int64_t mi, ni;
    group_mn<GN>(tile % (ntm * ntn), ntm, ntn, mi, ni);
    tl.m0 = mi * TBM;
    tl.n0 = ni * BN;
    tl.kbase = tl.e ? s_cum[tl.e - 1] : 0;
    tl.klen = s_cum[tl.e] - tl.kbase;  // Kp_e
  } else {
    int lo = 0, hi = g.E - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_cum[mid] * ntn > tile) hi = mid; else lo = mid + 1;
    }
    tl.e = lo;
    tl.seg0 = s_seg[lo];
    tl.Me = (int64_t)s_seg[lo + 1] - tl.seg0;
    if (tl.seg0 < 0 || tl.seg0 + tl.Me > g.M) return false;  // malformed offsets: stay inside the buffers
    const int64_t mt_e = (tl.Me + TBM - 1) / TBM;
    const int64_t li = tile - (s_cum[lo] - mt_e) * ntn;  // tile index within the expert
    int64_t mi, ni;
    group_mn<GN>(li, mt_e, ntn, mi, ni);
    tl.m0 = mi * TBM;
    tl.n0 = ni * BN;
    tl.klen = g.K;
  }
  return true;
}

// Epilogue. The accumulators pass through LDS so that global stores are
// whole 16-byte pieces of contiguous output rows. OUT_S2F6 (the w2 GEMM of
// the expert chain, "Quantized communications": RHT and S2F6 quantization in
// the epilogue): the fp32 rows are staged as for OUT_F32 and each thread
// turns one 32-wide block of a row into 32 S2F6 codes and a UE8M0 scale (one
// row per lane, so the 16-byte LDS reads of a wave hit every bank once). acc[i][j] holds tile row
// 128 wm + 32 i + (lane & 31) and, in element 4q + u, tile column
// 32 TJ wn + 32 j + 8 q + 4 (lane >> 5) + u. Rows past the segment (FPROP,
// DGRAD) are not stored; NVFP4 sums take the two FP32 outer scales. `stage`
// is the workgroup's LDS (at least 256 x 528 bytes); the caller has made sure
// no wave still reads it.
template <int NVFP4, int WGRAD, int OUT>
__device__ __forceinline__ void store_tile(const GemmArgs& g, const Tile& tl, const f32x16 (&acc)[4][TJ], int wm,
                                           int wn, int lane_in, uint8_t* stage) {
  // The lane's LDS and global offsets are derived here anew for every tile:
  // hoisted out of the tile loop they stay live across the K loop, do not fit
  // in registers beside the accumulators, and their spilled copies would be
  // reloaded after the first half's global stores, a reload that waits for
  // those stores to complete (one vector-memory counter orders both).
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  const float sw = NVFP4 ? g.b_outer[tl.e] : 1.0f;
  float rs[4];  // output scale of each of the lane's rows
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rs[i] = 1.0f;
    if constexpr (NVFP4) {
      const int64_t m = tl.m0 + wm * 128 + i * 32 + (lane & 31);
      float sx = g.a_outer[0];
      if (g.a_outer_per_row) {
        const int64_t mm = m < tl.Me ? m : tl.Me - 1;
        int64_t tok = g.a_row_index ? (int64_t)g.a_row_index[tl.seg0 + mm] : tl.seg0 + mm;
        tok = tok < 0 ? 0 : (tok >= g.a_rows ? g.a_rows - 1 : tok);
        sx = g.a_outer[tok];
      }
      rs[i] = sx * sw;
    }
  }
  const int64_t rows_left = WGRAD ? BM : tl.Me - tl.m0;  // rows of the tile inside the segment
  if constexpr (OUT == OUT_BF16) {
    // bf16 rows of 512 bytes at a 520-byte pitch (rows 2 banks apart)
    constexpr int P = BN * 2 + 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 128 + i * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = wn * 32 * TJ + j * 32 + q * 8 + (lane >> 5) * 4;
          const float s = rs[i];
          const bf2 lo2 = __builtin_convertvector((f2){acc[i][j][4 * q] * s, acc[i][j][4 * q + 1] * s}, bf2);
          const bf2 hi2 = __builtin_convertvector((f2){acc[i][j][4 * q + 2] * s, acc[i][j][4 * q + 3] * s}, bf2);
          *reinterpret_cast<uint2*>(stage + r * P + c * 2) =
              make_uint2(__builtin_bit_cast(uint32_t, lo2), __builtin_bit_cast(uint32_t, hi2));
        }
    }
    __syncthreads();
    // 32 pieces of 16 bytes per row; a wave covers two whole rows
#pragma unroll 4
    for (int k = 0; k < BM * 32 / kThreads; ++k) {
      const int id = t + k * kThreads;
      const int r = id >> 5, c = id & 31;
      if (r < rows_left) {
        const uint4 v = *reinterpret_cast<const uint4*>(stage + r * P + c * 16);
        const int64_t orow = WGRAD ? (int64_t)tl.e * g.M + tl.m0 + r : tl.seg0 + tl.m0 + r;
        store_nt(static_cast<uint16_t*>(g.out) + orow * g.N + tl.n0 + c * 8, v);
      }
    }
  } else {
    // fp32: two passes of 128 rows (1024 bytes each at a 1040-byte pitch)
    constexpr int P = BN * 4 + 16;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half) __syncthreads();  // the first half's reads are done
      if (wm == half) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = i * 32 + (lane & 31);
#pragma unroll
          for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int c = wn * 32 * TJ + j * 32 + q * 8 + (lane >> 5) * 4;
              const float s = rs[i];
              *reinterpret_cast<float4*>(stage + r * P + c * 4) =
                  make_float4(acc[i][j][4 * q] * s, acc[i][j][4 * q + 1] * s, acc[i][j][4 * q + 2] * s,
                              acc[i][j][4 * q + 3] * s);
            }
        }
      }
      __syncthreads();
      if constexpr (OUT == OUT_F32) {
#pragma unroll 4
        for (int k = 0; k < 128 * 64 / kThreads; ++k) {  // 64 pieces of 16 bytes per row
          const int id = t + k * kThreads;
          const int r = id >> 6, c = id & 63;
          if (half * 128 + r < rows_left) {
            const uint4 v = *reinterpret_cast<const uint4*>(stage + r * P + c * 16);
            const int64_t m = tl.m0 + half * 128 + r;
            const int64_t orow = WGRAD ? (int64_t)tl.e * g.M + m : tl.seg0 + m;
            store_nt(static_cast<float*>(g.out) + orow * g.N + tl.n0 + c * 4, v);
          }
        }
      } else {
        for (int k = 0; k < 128 * (BN / 32) / kThreads; ++k) {  // 8 blocks of 32 per row
          const int id = t + k * kThreads;
          const int r = id & 127, b = id >> 7;
          if (half * 128 + r < rows_left) {
            float v[32];
            const float4* src = reinterpret_cast<const float4*>(stage + r * P + b * 128);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const float4 f = src[q];
              v[4 * q] = f.x;
              v[4 * q + 1] = f.y;
              v[4 * q + 2] = f.z;
              v[4 * q + 3] = f.w;
            }
            uint32_t w[8];
            const uint32_t sc = rht_s2f6_block(v, g.signs, w);
            const int64_t orow = tl.seg0 + tl.m0 + half * 128 + r;
            // ordinary stores: a lane's 32 bytes are half of a line (the hint measured +35% HBM writes here)
            uint4* dst = reinterpret_cast<uint4*>(static_cast<uint8_t*>(g.out) + orow * g.N + tl.n0 + b * 32);
            dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
            dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
            g.out_scales[orow * (g.N / 32) + tl.n0 / 32 + b] = (uint8_t)sc;
          }
        }
      }
    }
  }
}

// ============================================================== operand loads

enum { FMT_NVFP4 = 0, FMT_MXFP8 = 1 };

// Byte offset of the codes of row `lrow` of the tile's A (isA) or B operand.
// A row's scales start at offset / (elements per scale / elements per byte).
template <int WGRAD, int CB>
__device__ __forceinline__ int64_t row_off(const GemmArgs& g, const Tile& tl, bool isA, int lrow) {
  if constexpr (WGRAD) {
    return isA ? g.M * tl.kbase + (tl.m0 + lrow) * tl.klen : g.N * tl.kbase + (tl.n0 + lrow) * tl.klen;
  } else {
    int64_t row;
    if (isA) {
      const int64_t m = tl.m0 + lrow < tl.Me ? tl.m0 + lrow : tl.Me - 1;
      row = g.a_row_index ? (int64_t)g.a_row_index[tl.seg0 + m] : tl.seg0 + m;
      row = row < 0 ? 0 : (row >= g.a_rows ? g.a_rows - 1 : row);
    } else {
      row = (int64_t)tl.e * g.N + tl.n0 + lrow;
    }
    return row * (g.K / CB);
  }
}

// The K step's codes are fetched in 16-byte chunks with the lanes of a row
// side by side (CPR chunks per row: 2 for NVFP4's 32 bytes, 4 for MXFP8's
// 64), so one wave instruction reads whole row segments instead of one chunk
// of 64 rows. Thread t holds chunk c = t % CPR of tile rows
// t / CPR + (kThreads / CPR) i, i < R; rows below BM (i < R/2) are A rows.
// The loads never branch and nothing combines loaded values before the
// decode, so a step's loads stay in flight while the previous step computes.
template <int FMT> struct Slab {
  static constexpr int CPR = FMT == FMT_NVFP4 ? 2 : 4;
  static constexpr int R = (BM + BN) * CPR / kThreads;  // rows per thread
  uint4 c[R];      // NVFP4: 32 E2M1 codes; MXFP8: 16 E4M3 codes of each row
  uint32_t m;      // MXFP8: all ones, or 0 when the chunk lies past the K extent
};

// Block scales, fetched for four K steps at a time: the CPR threads that
// share a thread's rows (CPR = R) each load one of those rows' scales of the
// four steps, 16 bytes (NVFP4: 4 E4M3 scales per step) or 8 (MXFP8: 2 E8M0
// scales per step), with one buffer load (reads past the scale array return
// zeros); every step, a broadcast within the group of CPR lanes gives each
// thread its rows' scales of the step. One scale request per row and four
// steps instead of one per row, chunk and step (measured: the per-step
// scale loads cost 0.14-0.17 ms per GEMM beside the code loads).
template <int FMT> struct ScaleGrp;
template <> struct ScaleGrp<FMT_NVFP4> {
  uint32_t w[4];  // the row's scale bytes of steps 4j .. 4j+3 (4 per step)
};
template <> struct ScaleGrp<FMT_MXFP8> {
  uint32_t d[3];  // 12 bytes from the 4-byte boundary at or below the row's scales of step 4j
  uint32_t sh;    // bit offset of those scales in d
};
typedef __amdgpu_buffer_rsrc_t brsrc_t;
typedef int v3i __attribute__((ext_vector_type(3)));
typedef int v4i __attribute__((ext_vector_type(4)));

// Lane c of a group of CPR loads the scales of its row c (A rows for c < R/2)
// for K steps 4j .. 4j+3.
__device__ __forceinline__ void load_group(ScaleGrp<FMT_NVFP4>& gr, brsrc_t ra, brsrc_t rb, const uint32_t* off32,
                                           int c, int64_t j) {
  const uint32_t o = (off32[c] << 2) + 16u * (uint32_t)j;  // scale bytes are an 8th of the code bytes
  const v4i v = c < 1 ? __builtin_amdgcn_raw_buffer_load_b128(ra, (int)o, 0, 0)
                      : __builtin_amdgcn_raw_buffer_load_b128(rb, (int)o, 0, 0);
  gr.w[0] = (uint32_t)v.x; gr.w[1] = (uint32_t)v.y; gr.w[2] = (uint32_t)v.z; gr.w[3] = (uint32_t)v.w;
}
__device__ __forceinline__ void load_group(ScaleGrp<FMT_MXFP8>& gr, brsrc_t ra, brsrc_t rb, const uint32_t* off32,
                                           int c, int64_t j) {
  const uint32_t o = off32[c] + 8u * (uint32_t)j;  // scale bytes are a 32nd of the code bytes
  const v3i v = c < 2 ? __builtin_amdgcn_raw_buffer_load_b96(ra, (int)(o & ~3u), 0, 0)
                      : __builtin_amdgcn_raw_buffer_load_b96(rb, (int)(o & ~3u), 0, 0);
  gr.d[0] = (uint32_t)v.x; gr.d[1] = (uint32_t)v.y; gr.d[2] = (uint32_t)v.z;
  gr.sh = 8u * (o & 3u);
}

// The thread's rows' scales of step s (s % 4 of its group), in the per-row
// form the decode takes: NVFP4 the chunk's two E4M3 bytes, MXFP8 the E8M0
// byte of the chunk's block. Lane i of the group holds row i's scales.
template <int I> __device__ __forceinline__ uint32_t bcast4(uint32_t v) {  // lane I of each group of 4
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, I | (I << 2) | (I << 4) | (I << 6), 0xF, 0xF, false);
}
template <int I> __device__ __forceinline__ uint32_t bcast2(uint32_t v) {  // lane I of each pair
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, I | (I << 2) | ((2 + I) << 4) | ((2 + I) << 6), 0xF, 0xF, false);
}
// The group's word holding step s4's scales (the lane's own row), and the
// shift of the thread's chunk's scales in it.
__device__ __forceinline__ uint32_t step_word(const ScaleGrp<FMT_NVFP4>& gr, int s4) {
  return s4 == 0 ? gr.w[0] : (s4 == 1 ? gr.w[1] : (s4 == 2 ? gr.w[2] : gr.w[3]));
}
__device__ __forceinline__ uint32_t step_word(const ScaleGrp<FMT_MXFP8>& gr, int s4) {
  return s4 < 2 ? __builtin_amdgcn_alignbit(gr.d[1], gr.d[0], gr.sh)   // steps 0, 1 of the group
                : __builtin_amdgcn_alignbit(gr.d[2], gr.d[1], gr.sh);  // steps 2, 3
}
template <int FMT> __device__ __forceinline__ uint32_t step_shift(int s4, int c) {
  return FMT == FMT_NVFP4 ? 16u * (uint32_t)c : 8u * (uint32_t)(2 * (s4 & 1) + (c >> 1));
}
// Row i's scales of the step (i a constant after unrolling): NVFP4 the
// chunk's two E4M3 bytes, MXFP8 the E8M0 byte of the chunk's block.
template <int FMT> __device__ __forceinline__ uint32_t row_scale(uint32_t w, uint32_t shift, int i) {
  uint32_t v;
  if constexpr (FMT == FMT_NVFP4) {
    v = i == 0 ? bcast2<0>(w) : bcast2<1>(w);
    return (v >> shift) & 0xFFFFu;
  } else {
    v = i == 0 ? bcast4<0>(w) : (i == 1 ? bcast4<1>(w) : (i == 2 ? bcast4<2>(w) : bcast4<3>(w)));
    return (v >> shift) & 0xFFu;
  }
}

__device__ __forceinline__ void load_slab(Slab<FMT_NVFP4>& r, const GemmArgs& g, const uint32_t* off32, int c,
                                          int64_t k0, int64_t) {
  constexpr int R = Slab<FMT_NVFP4>::R;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const uint8_t* codes = i < R / 2 ? g.a_codes : g.b_codes;
    const int64_t off = (int64_t)off32[i] << 5;
    r.c[i] = *reinterpret_cast<const uint4*>(codes + off + (k0 >> 1) + 16 * c);
  }
}
// MXFP8 rows of WGRAD end where the expert's padded token count ends, a
// multiple of 32: a last step can hold one 32-wide half, and the chunks of
// its second half then read a duplicate of the first that the decode masks.
__device__ __forceinline__ void load_slab(Slab<FMT_MXFP8>& r, const GemmArgs& g, const uint32_t* off32, int c,
                                          int64_t k0, int64_t klen) {
  constexpr int R = Slab<FMT_MXFP8>::R;
  const bool in = k0 + 16 * c < klen;
  const int64_t k = in ? k0 + 16 * c : k0 + 16 * (c & 1);
  r.m = in ? 0xFFFFFFFFu : 0u;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const uint8_t* codes = i < R / 2 ? g.a_codes : g.b_codes;
    const int64_t off = (int64_t)off32[i] << 5;
    r.c[i] = *reinterpret_cast<const uint4*>(codes + off + k);
  }
}

// Decode quarter q of the slab (16 values) into 32 bytes of LDS.
//   NVFP4: row q / 2, values 16 (q & 1) .. of its chunk, at byte 64c + 32(q & 1);
//   MXFP8: row q, at byte 32c.
template <int FMT> constexpr int quarters() { return FMT == FMT_NVFP4 ? 2 * Slab<FMT>::R : Slab<FMT>::R; }
template <int FMT> constexpr int quarter_row(int q) { return FMT == FMT_NVFP4 ? q >> 1 : q; }
// `scr` is the quarter's row's scales of the step (row_scale).
__device__ __forceinline__ void decode_quarter(const Slab<FMT_NVFP4>& r, uint32_t scr, uint8_t* dst, int q) {
  const int i = q >> 1, h = q & 1;
  const uint32_t w0 = h ? r.c[i].z : r.c[i].x;
  const uint32_t w1 = h ? r.c[i].w : r.c[i].y;
  const _Float16 s = (_Float16)e4m3_val((scr >> (8 * h)) & 0xFFu);  // one E4M3 scale per 16
  const h2 sv = {s, s};
#define BSQ_DEC4(w, v0, v1, v2, v3)                                 \
  const h2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sv; \
  const h2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sv; \
  const h2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sv; \
  const h2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sv;
  BSQ_DEC4(w0, a0, a1, a2, a3)
  BSQ_DEC4(w1, b0, b1, b2, b3)
#undef BSQ_DEC4
  uint4* d = reinterpret_cast<uint4*>(dst);
  d[0] = make_uint4(__builtin_bit_cast(uint32_t, a0), __builtin_bit_cast(uint32_t, a1), __builtin_bit_cast(uint32_t, a2),
                    __builtin_bit_cast(uint32_t, a3));
  d[1] = make_uint4(__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1), __builtin_bit_cast(uint32_t, b2),
                    __builtin_bit_cast(uint32_t, b3));
}
__device__ __forceinline__ void decode_quarter(const Slab<FMT_MXFP8>& r, uint32_t scr, uint8_t* dst, int q) {
  const uint4 v = make_uint4(r.c[q].x & r.m, r.c[q].y & r.m, r.c[q].z & r.m, r.c[q].w & r.m);
  // 2^(s-127) as a float: the scaled convert applies its exponent (code 127,
  // a factor of one, for a masked chunk)
  const uint32_t code = (scr & r.m) | (127u & ~r.m);
  const float s = __uint_as_float(code << 23);
#define BSQ_DEC2(w, p, q_)                                              \
  const bf2 p = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, s, false); \
  const bf2 q_ = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, s, true);
  BSQ_DEC2(v.x, a0, a1)
  BSQ_DEC2(v.y, a2, a3)
  BSQ_DEC2(v.z, b0, b1)
  BSQ_DEC2(v.w, b2, b3)
#undef BSQ_DEC2
  uint4* d = reinterpret_cast<uint4*>(dst);
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

// ============================================================== kernel

// Persistent kernel: one workgroup per CU walks its XCD's range of tiles
// (workgroup w runs on XCD w % 8, so each XCD works on a contiguous range of
// tiles: an expert's weights and token rows stay in that XCD's L2), with one
// segment scan per workgroup and no launch or scan cost per tile.
template <bool B> struct Split { static constexpr bool value = B; };

template <int FMT, int WGRAD, int OUT>
__global__ __launch_bounds__(kThreads) void k_gemm(const GemmArgs g) {
  static_assert(BM == BN, "A and B LDS buffers share one layout");
  static_assert(WN * 4 * TJ * 4 * 64 * 16 <= 4 * BM * kRow, "tail-tile partial sums fit in the operand buffers");
  static_assert(2 * BM % (kThreads / Slab<FMT>::CPR) == 0, "whole slab rows per thread");
  static_assert(BM * (BN * 2 + 8) <= 4 * BM * kRow && 128 * (BN * 4 + 16) <= 4 * BM * kRow, "epilogue staging fits");
  __shared__ __attribute__((aligned(16))) uint8_t s_ab[4][BM * kRow];  // A buffers 0, 1; B buffers 0, 1
  uint8_t (*sA)[BM * kRow] = s_ab;
  uint8_t (*sB)[BM * kRow] = s_ab + 2;
  __shared__ int64_t s_cum[kMaxE];
  __shared__ int64_t s_part[256];
  __shared__ int32_t s_seg[WGRAD ? 1 : kMaxE + 1];
  const int64_t total = scan_units<WGRAD, BM>(g, s_cum, s_part, s_seg);
  const int64_t per_xcd = (total + kXcds - 1) / kXcds;
  const int64_t wpx = gridDim.x / kXcds;  // workgroups per XCD (the grid is a multiple of kXcds)
  const int64_t tile0 = (int64_t)(blockIdx.x % kXcds) * per_xcd;

  // ---- the scale arrays as buffers (reads past them return zeros; the
  // range is rounded up to whole 4-byte words)
  int64_t sa_bytes, sb_bytes;
  if constexpr (FMT == FMT_NVFP4) {
    sa_bytes = g.a_rows * (g.K / 16);
    sb_bytes = (int64_t)g.E * g.N * (g.K / 16);
  } else if constexpr (WGRAD) {
    const int64_t kpt = s_cum[g.E - 1];  // padded tokens of all experts
    sa_bytes = g.M * kpt / 32;
    sb_bytes = g.N * kpt / 32;
  } else {
    sa_bytes = g.M * (g.K / 32);
    sb_bytes = (int64_t)g.E * g.N * (g.K / 32);
  }
  auto nrec = [](int64_t b) -> int {
    b = (b + 3) & ~(int64_t)3;
    return (int)(uint32_t)(b < 0xFFFFFFFCll ? b : 0xFFFFFFFCll);
  };
  const brsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc((void*)g.a_scales, (short)0, nrec(sa_bytes), 0x00020000);
  const brsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc((void*)g.b_scales, (short)0, nrec(sb_bytes), 0x00020000);

  // ---- the slab this thread loads and decodes each K step
  const int t = threadIdx.x;
  constexpr int SR = Slab<FMT>::R;
  constexpr int CPR = Slab<FMT>::CPR;
  constexpr int QK = quarters<FMT>() / 4;  // quarters decoded per 16-wide k slice
  const int chunk = t % CPR;
  int ldst[SR];  // LDS offset of each slab row's decoded chunk in buffer 0 (A rows: sA, B rows: sB)
#pragma unroll
  for (int i = 0; i < SR; ++i) {
    const int row = t / CPR + (kThreads / CPR) * i;  // tile row: A rows below BM, then B rows
    ldst[i] = (i < SR / 2 ? 0 : 2 * BM * kRow) + (row & (BM - 1)) * kRow + chunk * (FMT == FMT_NVFP4 ? 64 : 32);
  }
  uint8_t* const lds0 = sA[0];  // sA[0], sA[1], sB[0], sB[1] are contiguous
  // LDS destination of quarter q in buffer b
  auto qdst = [&](int b, int q) -> uint8_t* {
    return FMT == FMT_NVFP4 ? lds0 + ldst[q >> 1] + b * (BM * kRow) + 32 * (q & 1) : lds0 + ldst[q] + b * (BM * kRow);
  };

  const int wave = t >> 6;
  const int lane = t & 63;
  const int wm = wave / WN;  // 128-row half of the tile (m)
  const int wn = wave % WN;  // 32 TJ-column slice of the tile (n)
  typedef typename Frag<FMT>::type V8;
  // fragment: lane -> row (lane & 31), k offset 8 * (lane >> 5) within each 16-wide k slice
  const int frag_off = (lane & 31) * kRow + (lane >> 5) * 16;
  const int a_off = wm * 128 * kRow + frag_off;
  const int b_off = wn * 32 * TJ * kRow + frag_off;
  // Tail tiles (segments along M, at most 128 rows of the tile inside the
  // segment): both halves of the waves multiply rows 0..127, half wm taking the
  // k slices 2 wm and 2 wm + 1 of every step; the two partial sums are added
  // after the K loop. Half the MFMA work of a full tile, whose second 128 rows
  // would all lie past the segment.
  const int a_off_s = frag_off + 64 * wm;
  const int b_off_s = b_off + 64 * wm;
#define BSQ_LOAD_FRAGS(slot, buf, ks, ao, bo)                                                      \
  _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) fa[slot][i_] =                                  \
      *reinterpret_cast<const V8*>(&sA[buf][(ao) + i_ * 32 * kRow + (ks) * 32]);                   \
  _Pragma("unroll") for (int j_ = 0; j_ < TJ; ++j_) fb[slot][j_] =                                 \
      *reinterpret_cast<const V8*>(&sB[buf][(bo) + j_ * 32 * kRow + (ks) * 32]);

  // One tile: full (256 output rows) or tail (SPLIT); the two K-loop
  // variants are separate instantiations inside the one tile walk below.
  auto tile_body = [&](auto split_tag, const Tile& tl) {
    constexpr bool SPLIT = decltype(split_tag)::value;
    {
      // The thread's slab rows, derived anew per tile from an opaque copy of
      // the thread index: hoisted out of the tile loop they stay live across
      // the K loop and spill, and the reload in the next tile's prologue waits
      // for the previous tile's stores (one counter orders both).
      int tr = t;
      asm volatile("" : "+v"(tr));
      uint32_t off[SR];  // row code offsets in units of 32 bytes (every row starts at a multiple of 32)
#pragma unroll
      for (int i = 0; i < SR; ++i)
        off[i] = (uint32_t)(row_off<WGRAD, FMT == FMT_NVFP4 ? 2 : 1>(g, tl, i < SR / 2,
                                                                      (tr / CPR + (kThreads / CPR) * i) & (BM - 1)) >> 5);

      f32x16 acc[4][TJ];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
      V8 fa[2][4], fb[2][TJ];
      const int nk = (int)((tl.klen + BK - 1) / BK);

      // Software pipeline. At the start of step kt, `cur` holds step kt + 1 as
      // loaded and the loads of step kt + 2 go out into `nxt` (clamped: the last
      // steps load and decode a duplicate that is never read). Each 16-wide k
      // slice then reads the next slice's fragments, runs this slice's MFMAs and
      // decodes one quarter of `cur` into the other LDS buffer; the barrier at the
      // end of the step publishes that buffer (every read of it from the previous
      // step finished before the previous barrier). The two register sets swap
      // roles every step (the loop body is unrolled twice). Tail tiles (SPLIT)
      // run two slices per step, each over two iterations.
      // Scale groups: group j (steps 4j .. 4j+3) is loaded with step 4j's codes
      // (at step 4j - 2) into gnext and becomes gcur when step 4j is decoded.
      Slab<FMT> r0, r1;
      ScaleGrp<FMT> gcur, gnext;
      auto step = [&](int kt, Slab<FMT>& cur, Slab<FMT>& nxt) {
        const int ao = SPLIT ? a_off_s : a_off;
        const int bo = SPLIT ? b_off_s : b_off;
        const int buf = kt & 1;
        load_slab(nxt, g, off, chunk, (int64_t)(kt + 2 < nk ? kt + 2 : nk - 1) * BK, tl.klen);
        if (kt + 2 < nk && ((kt + 2) & 3) == 0) load_group(gnext, rsa, rsb, off, chunk, (kt + 2) >> 2);
        __builtin_amdgcn_sched_barrier(0);  // keep the loads here: a whole step ahead of their use
        const int dstep = kt + 1 < nk ? kt + 1 : nk - 1;  // the step `cur` holds
        if (kt + 1 < nk && (dstep & 3) == 0) gcur = gnext;
        const uint32_t sw = step_word(gcur, dstep & 3);
        const uint32_t ssh = step_shift<FMT>(dstep & 3, chunk);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          if constexpr (SPLIT) {
            // the wave's two slices (fragment slots 0, 1), each in two
            // iterations of half its MFMAs (rows 64 (ks & 1) .. of the 128),
            // so that every iteration still decodes one quarter
            const int sl = ks >> 1, ih = ks & 1;
            if (ks == 1) {
              BSQ_LOAD_FRAGS(1, buf, 1, ao, bo)
            }
#pragma unroll
            for (int i = 2 * ih; i < 2 * ih + 2; ++i)
#pragma unroll
              for (int j = 0; j < TJ; ++j) acc[i][j] = mfma16(fb[sl][j], fa[sl][i], acc[i][j]);
          } else {
            if (ks < 3) {
              BSQ_LOAD_FRAGS((ks + 1) & 1, buf, ks + 1, ao, bo)
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int j = 0; j < TJ; ++j) acc[i][j] = mfma16(fb[ks & 1][j], fa[ks & 1][i], acc[i][j]);
          }
#pragma unroll
          for (int q = ks * QK; q < (ks + 1) * QK; ++q)
            decode_quarter(cur, row_scale<FMT>(sw, ssh, quarter_row<FMT>(q)), qdst(buf ^ 1, q), q);
          // interleave each MFMA with a few decode VALU ops, the fragment reads and the decode stores
          constexpr int NM = SPLIT ? 2 * TJ : 4 * TJ;  // MFMAs of the iteration
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                          // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 48 / NM, 0);                    // VALU
            if (SPLIT ? (ks == 1 && 2 * m < 4 + TJ) : (m < 4 + TJ))
              __builtin_amdgcn_sched_group_barrier(0x100, SPLIT ? 2 : 1, 0);            // DS read
            if (m >= NM - 2 * QK) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);    // DS write
          }
        }
        __syncthreads();
        BSQ_LOAD_FRAGS(0, buf ^ 1, 0, ao, bo)
      };
      if (nk > 0) {
        load_slab(r0, g, off, chunk, 0, tl.klen);
        load_group(gnext, rsa, rsb, off, chunk, 0);
        gcur = gnext;
        const uint32_t sw = step_word(gcur, 0);
        const uint32_t ssh = step_shift<FMT>(0, chunk);
#pragma unroll
        for (int q = 0; q < quarters<FMT>(); ++q)
          decode_quarter(r0, row_scale<FMT>(sw, ssh, quarter_row<FMT>(q)), qdst(0, q), q);
        load_slab(r0, g, off, chunk, nk > 1 ? BK : 0, tl.klen);
        __syncthreads();
        BSQ_LOAD_FRAGS(0, 0, 0, SPLIT ? a_off_s : a_off, SPLIT ? b_off_s : b_off)
      }
      int kt = 0;
      for (; kt + 1 < nk; kt += 2) {
        step(kt, r0, r1);
        step(kt + 1, r1, r0);
      }
      if (kt < nk) step(kt, r0, r1);

      __syncthreads();  // every wave is done with the operand buffers
      if constexpr (SPLIT) {
        // the partial sums of half 1 (slices 2, 3) join those of half 0 through LDS
        float4* red = reinterpret_cast<float4*>(lds0);
        if (wm == 1) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q)
                red[(((wn * 4 + i) * TJ + j) * 4 + q) * 64 + lane] =
                    make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
        __syncthreads();
        if (wm == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const float4 p = red[(((wn * 4 + i) * TJ + j) * 4 + q) * 64 + lane];
                acc[i][j][4 * q] += p.x;
                acc[i][j][4 * q + 1] += p.y;
                acc[i][j][4 * q + 2] += p.z;
                acc[i][j][4 * q + 3] += p.w;
              }
        }
        __syncthreads();  // the partial sums are read before the epilogue stages into LDS
      }
      store_tile<FMT == FMT_NVFP4, WGRAD, OUT>(g, tl, acc, wm, wn, lane, lds0);
      __syncthreads();  // the staging reads are done before the next tile decodes into LDS
    }
  };
  for (int64_t lt = blockIdx.x / kXcds; lt < per_xcd; lt += wpx) {
    const int64_t tile = tile0 + lt;
    if (tile >= total) break;
    Tile tl;
    constexpr int GN = 4;  // n-tiles per group (above)
    if (!tile_coords<WGRAD, BM, GN>(g, s_cum, s_seg, tile, tl)) continue;  // uniform across the workgroup
    if constexpr (WGRAD) {
      tile_body(Split<false>{}, tl);
    } else {
      if (tl.Me - tl.m0 <= 128) tile_body(Split<true>{}, tl);  // uniform: at most 128 rows left
      else tile_body(Split<false>{}, tl);
    }
  }
#undef BSQ_LOAD_FRAGS
}

template <int FMT, int WGRAD>
int launch(const GemmArgs& a, int64_t slots, int out_dtype, hipStream_t s) {
  const int64_t cus = (bsqh::device_cus() + kXcds - 1) / kXcds * kXcds;
  int64_t grid = (slots + kXcds - 1) / kXcds * kXcds;
  if (grid > cus) grid = cus;
  if constexpr (FMT == FMT_NVFP4 && !WGRAD) {
    if (out_dtype == OUT_S2F6) {
      hipLaunchKernelGGL((k_gemm<FMT, WGRAD, OUT_S2F6>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
      return bsqh::launch_status();
    }
  }
  if (out_dtype == BSQ_F32)
    hipLaunchKernelGGL((k_gemm<FMT, WGRAD, OUT_F32>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((k_gemm<FMT, WGRAD, OUT_BF16>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
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
  BSQ_REQUIRE(N % BN == 0 && K % BK == 0 && M_total < kMaxRows, BSQ_E_SHAPE);
  if (M_total == 0 || N == 0) return BSQ_OK;
  BSQ_REQUIRE(K > 0 && a_rows > 0, BSQ_E_SHAPE);
  BSQ_REQUIRE(a_codes && a_scales && a_outer && b_codes && b_scales && b_outer && seg_offsets && out, BSQ_E_NULL);
  BSQ_REQUIRE(bsqh::aligned16(a_codes) && bsqh::aligned16(b_codes) && bsqh::aligned16(out), BSQ_E_ALIGN);
  BSQ_REQUIRE(((uintptr_t)a_scales & 3) == 0 && ((uintptr_t)b_scales & 3) == 0, BSQ_E_ALIGN);
  const GemmArgs a{a_codes, a_scales, a_outer, a_outer_per_row, a_rows, a_row_index, b_codes, b_scales, b_outer,
                   seg_offsets, (int)E, M_total, N, K, out, nullptr, 0u};
  return launch<FMT_NVFP4, 0>(a, bsqh::tile_bound(M_total, E, BM) * (N / BN), out_dtype, bsqh::as_stream(stream));
}

extern "C" int bsq_grouped_gemm_nvfp4_s2f6(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_outer,
                                           int a_outer_per_row, int64_t a_rows, const int32_t* a_row_index,
                                           const uint8_t* b_codes, const uint8_t* b_scales, const float* b_outer,
                                           const int64_t* seg_offsets, int64_t E, int64_t M_total, int64_t N,
                                           int64_t K, uint32_t signs, uint8_t* out_codes, uint8_t* out_scales,
                                           bsq_stream_t stream) {
  BSQ_REQUIRE(E >= 1 && E <= kMaxE && M_total >= 0 && N >= 0 && K >= 0 && a_rows >= 0, BSQ_E_SHAPE);
  BSQ_REQUIRE(N % BN == 0 && K % BK == 0 && M_total < kMaxRows, BSQ_E_SHAPE);
  if (M_total == 0 || N == 0) return BSQ_OK;
  BSQ_REQUIRE(K > 0 && a_rows > 0, BSQ_E_SHAPE);
  BSQ_REQUIRE(a_codes && a_scales && a_outer && b_codes && b_scales && b_outer && seg_offsets && out_codes &&
                  out_scales,
              BSQ_E_NULL);
  BSQ_REQUIRE(bsqh::aligned16(a_codes) && bsqh::aligned16(b_codes) && bsqh::aligned16(out_codes), BSQ_E_ALIGN);
  BSQ_REQUIRE(((uintptr_t)a_scales & 3) == 0 && ((uintptr_t)b_scales & 3) == 0, BSQ_E_ALIGN);
  const GemmArgs a{a_codes, a_scales, a_outer, a_outer_per_row, a_rows, a_row_index, b_codes, b_scales, b_outer,
                   seg_offsets, (int)E, M_total, N, K, out_codes, out_scales, signs};
  return launch<FMT_NVFP4, 0>(a, bsqh::tile_bound(M_total, E, BM) * (N / BN), OUT_S2F6, bsqh::as_stream(stream));
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
  else BSQ_REQUIRE(K % BK == 0 && M_total < kMaxRows, BSQ_E_SHAPE);
  if (M_total == 0 || N == 0) return BSQ_OK;
  if (!wgrad) BSQ_REQUIRE(K > 0, BSQ_E_SHAPE);
  BSQ_REQUIRE(a_codes && a_scales && b_codes && b_scales && seg_offsets && out, BSQ_E_NULL);
  BSQ_REQUIRE(bsqh::aligned16(a_codes) && bsqh::aligned16(b_codes) && bsqh::aligned16(out), BSQ_E_ALIGN);
  const GemmArgs a{a_codes, a_scales, nullptr, 0, M_total, nullptr, b_codes, b_scales, nullptr,
                   seg_offsets, (int)E, M_total, N, K, out, nullptr, 0u};
  hipStream_t s = bsqh::as_stream(stream);
  if (wgrad) return launch<FMT_MXFP8, 1>(a, E * (M_total / BM) * (N / BN), out_dtype, s);
  return launch<FMT_MXFP8, 0>(a, bsqh::tile_bound(M_total, E, BM) * (N / BN), out_dtype, s);
}
