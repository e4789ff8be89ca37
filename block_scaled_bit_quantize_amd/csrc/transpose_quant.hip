// Transposing quantizers: dequantize -> transpose -> stochastic requantize,
// and the transposed MXFP8 quantization of the output gradient.
//
// "End-to-End 4-Bit Training", section "Block-scaled backward passes": the
// backward products dx = g w_q and dw = g^T x_q use the forward tensors
// transposed, so their blocks run along the other axis. Section
// "Re-quantization with stochastic rounding": the forward NVFP4 tensors are
// dequantized, transposed in higher precision and requantized with stochastic
// rounding (to MXFP8 for the backward GEMMs), so that E[w_q] = E[(w_q^T)^T].
// The quantized linear layer figure also quantizes the transposed BF16 output
// gradient to MXFP8 with stochastic rounding for WGRAD. Section "Quantized
// communications": WGRAD reads the forward-quantized activations, i.e. the
// dispatched (gathered) token rows of each expert.
//
// One workgroup turns a tile of 128 input rows (tokens) x 64 channels into 64
// output rows x 128 tokens. Phase 1 loads the rows with 16-byte loads (NVFP4
// rows are decoded to exact fp16 q*s_b with the per-row outer scale kept
// aside), phase 2 reads the tile transposed from LDS: one thread per output
// block of 32 tokens, lanes on consecutive channels (conflict-free 2-byte
// reads), with the block maximum, scale, Philox draws and conversions in
// registers, and 16-byte code stores.
#include "bsq_device.h"
#include "bsq_internal.h"

using namespace bsqd;

namespace {

constexpr int kThreads = 256;
constexpr int TM = 128;  // tokens per tile (input rows)
constexpr int TC = 64;   // column granularity of the transposed layouts
constexpr int64_t kMaxTransposeCols = 1 << 22;  // bf16/float sources: 128 rows of byte offsets below 2^31
enum { SRC_BF16 = 0, SRC_F32 = 1, SRC_NVFP4 = 2 };

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t brsrc_t;

inline unsigned grid1(int64_t n, int t = kThreads) { return (unsigned)((n + t - 1) / t); }
__host__ __device__ inline int64_t pad32(int64_t n) { return (n + 31) / 32 * 32; }

// Tile plan for segmented layouts: slot -> (segment, token tile), and per
// segment its start row, length and output element base (cols * sum of
// earlier padded lengths). Offsets are clamped to [0, rows] and then replaced
// by their running maximum, so segments never overlap and their padded
// lengths sum to at most rows + 31 * nseg: a malformed (e.g. decreasing)
// table cannot send a later kernel outside its buffers.
// One workgroup of 1024 threads; num_segments <= 1024.
__global__ __launch_bounds__(1024) void k_seg_plan(const int64_t* __restrict__ seg_offsets, int nseg, int64_t rows,
                                                   int64_t cols, int tile, int64_t nslots,
                                                   int32_t* __restrict__ slot_seg, int32_t* __restrict__ slot_mt,
                                                   int64_t* __restrict__ seg_base, int64_t* __restrict__ seg_start,
                                                   int64_t* __restrict__ seg_len) {
  __shared__ int64_t s_tiles[1024];
  __shared__ int64_t s_pad[1024];
  __shared__ int64_t s_hi[1024];
  const int t = threadIdx.x;
  auto clampr = [&](int64_t v) { return v < 0 ? 0 : (v > rows ? rows : v); };
  // running maximum of the clamped offsets 0..t (inclusive max scan)
  s_hi[t] = t < nseg ? clampr(seg_offsets[t]) : 0;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int64_t v = t >= o ? s_hi[t - o] : 0;
    __syncthreads();
    s_hi[t] = s_hi[t] > v ? s_hi[t] : v;
    __syncthreads();
  }
  int64_t mp = 0, nt = 0;
  if (t < nseg) {
    const int64_t a = s_hi[t];
    int64_t b = clampr(seg_offsets[t + 1]);
    b = b < a ? a : b;
    seg_start[t] = a;
    seg_len[t] = b - a;
    mp = pad32(b - a);
    nt = (mp + tile - 1) / tile;
  }
  s_tiles[t] = nt;
  s_pad[t] = mp;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive Hillis-Steele scan
    const int64_t a = t >= o ? s_tiles[t - o] : 0;
    const int64_t b = t >= o ? s_pad[t - o] : 0;
    __syncthreads();
    s_tiles[t] += a;
    s_pad[t] += b;
    __syncthreads();
  }
  if (t < nseg) seg_base[t] = (s_pad[t] - mp) * cols;
  const int64_t total = nseg > 0 ? s_tiles[nseg - 1] : 0;
  for (int64_t slot = t; slot < nslots; slot += 1024) {
    int32_t seg = -1, mt = 0;
    if (slot < total) {
      int lo = 0, hi = nseg - 1;  // first segment whose inclusive tile count exceeds slot
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_tiles[mid] > slot) hi = mid; else lo = mid + 1;
      }
      seg = lo;
      mt = (int32_t)(slot - (s_tiles[lo] - ((s_pad[lo] - (lo ? s_pad[lo - 1] : 0)) + tile - 1) / tile));
    }
    slot_seg[slot] = seg;
    slot_mt[slot] = mt;
  }
}

// Largest dequantized magnitude of each batch item of an NVFP4 tensor
// (max over a block of f32(f32(max|q| * s_b) * s_t) equals the max of the
// element-wise dequantization, rounding being monotonic). One thread per block
// of 16; a workgroup whose blocks all belong to one item reduces them and
// issues one atomic (per-thread atomics on one address serialize), otherwise
// each thread merges its own block.
__global__ __launch_bounds__(kThreads) void k_nvfp4_item_amax(const uint8_t* __restrict__ codes,
                                                              const uint8_t* __restrict__ scales,
                                                              const float* __restrict__ outer, int in_mode,
                                                              int64_t nblk, int64_t blk_per_row, int64_t rows_per_item,
                                                              uint32_t* __restrict__ amax_bits) {
  const int64_t first = (int64_t)blockIdx.x * kThreads;
  const int64_t blk = first + threadIdx.x;
  float v = 0.0f;
  int64_t item = 0;
  if (blk < nblk) {
    const uint2 w = *reinterpret_cast<const uint2*>(codes + blk * 8);
    uint32_t mq = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mq = max(mq, (w.x >> (4 * i)) & 7u);
      mq = max(mq, (w.y >> (4 * i)) & 7u);
    }
    const float qmax = mq == 0 ? 0.0f : (mq < 2 ? 0.5f * (float)mq : (mq < 4 ? 1.0f + 0.5f * (float)(mq - 2) : (mq < 6 ? (float)(mq - 2) : (mq == 6 ? 4.0f : 6.0f))));
    const int64_t row = blk / blk_per_row;
    item = row / rows_per_item;
    const float st = in_mode == BSQ_OUTER_ROW ? outer[row] : outer[item];
    v = (qmax * e4m3_val(scales[blk])) * st;
  }
  const int64_t last = (first + kThreads < nblk ? first + kThreads : nblk) - 1;
  const int64_t item0 = first / blk_per_row / rows_per_item;
  if (item0 == last / blk_per_row / rows_per_item) {  // uniform across the workgroup
    __shared__ float red[kThreads / 64];
    const float m = wave_max(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      float r = red[0];
#pragma unroll
      for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
      if (r > 0.0f) atomicMax(amax_bits + item0, __float_as_uint(r));
    }
  } else if (v > 0.0f) {
    atomicMax(amax_bits + item, __float_as_uint(v));
  }
}

template <int SRC> struct TileT { typedef uint16_t type; };
template <> struct TileT<SRC_F32> { typedef float type; };
template <int SRC> constexpr int tile_channels() { return SRC == SRC_NVFP4 ? 128 : 64; }

// The transposing quantizer. SEG: tiles come from the segment plan (gather
// and per-segment padded layout); otherwise batch item e covers input rows
// [e*R, (e+1)*R) and is written as [cols, R]. A workgroup covers 128 tokens x
// TCH channels (128 for NVFP4 sources, whose decoded fp16 tile is small; 64
// for bf16 and float sources, whose 18 KB tile lets more workgroups share a
// CU: measured 5% faster than 128 for the bf16 gradient); in phase 2 a thread
// owns CPT = TCH/64 adjacent channels x 32 tokens.
// ROWS (bf16 and float sources, segmented MXFP8 output): the same launch also
// writes the row-wise MXFP8 quantization of the tile's rows (blocks of 32
// along channels, element index row * C + channel, its own random stream), so
// that a gradient quantized both ways is read from HBM once.
struct RowOut {
  uint8_t* codes = nullptr;   // [rows, C]
  uint8_t* scales = nullptr;  // [rows, C / 32]
  uint64_t stream_id = 0;
};

template <int SRC, int OUTF, int RND, bool SEG, bool ROWS = false>
__global__ __launch_bounds__(kThreads) void k_tq(
    const void* __restrict__ src, const uint8_t* __restrict__ in_scales, const float* __restrict__ in_outer,
    int in_mode, int64_t C, int64_t R, const int32_t* __restrict__ gather, const int64_t* __restrict__ seg_start_p,
    const int64_t* __restrict__ seg_len_p, const int32_t* __restrict__ slot_seg, const int32_t* __restrict__ slot_mt,
    const int64_t* __restrict__ seg_base, const uint32_t* __restrict__ amax_bits, uint64_t seed, uint64_t stream_id,
    uint8_t* __restrict__ out_codes, uint8_t* __restrict__ out_scales, float* __restrict__ out_outer,
    int64_t ntiles, RowOut rows = RowOut{}) {
  static_assert(!ROWS || (SRC != SRC_NVFP4 && OUTF == BSQ_MXFP8 && SEG), "row output: bf16/float source, segmented MXFP8");
  typedef typename TileT<SRC>::type TT;
  constexpr int TCH = tile_channels<SRC>();
  constexpr int CPT = TCH / 64;
  constexpr int LROW = TCH * (int)sizeof(TT) + 16;  // padded LDS row (bytes): conflict-free writes
  __shared__ __attribute__((aligned(16))) uint8_t tile[TM * LROW];
  __shared__ float rowmul[TM];

  // Tiles (token tile x channel tile, channel tiles fastest) are remapped so
  // that each XCD (workgroup w runs on XCD w % 8) takes a contiguous range:
  // the channel tiles of one token tile, which share its rows' code and scale
  // cache lines, then meet in one L2. The grid is 8 * ceil(total / 8).
  const int64_t nct = (C + TCH - 1) / TCH;
  const int64_t total = ntiles * nct;
  const int64_t per_xcd = (total + 7) / 8;
  const int64_t tid = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (tid >= total) return;
  const int64_t bx = tid / nct, by = tid % nct;

  int64_t e, mt, seg_start, Me, Mp, base;
  if constexpr (SEG) {
    const int32_t sg = slot_seg[bx];
    if (sg < 0) return;  // uniform across the workgroup
    e = sg;
    mt = slot_mt[bx];
    seg_start = seg_start_p[e];
    Me = seg_len_p[e];
    Mp = pad32(Me);
    base = seg_base[e];
  } else {
    const int64_t tiles_per = (R + TM - 1) / TM;
    e = bx / tiles_per;
    mt = bx % tiles_per;
    seg_start = e * R;
    Me = R;
    Mp = R;
    base = e * C * R;
  }
  const int64_t c0 = by * TCH;
  const int64_t m0 = mt * TM;
  const int t = threadIdx.x;

  // ---- phase 1: rows m0 .. m0+127 of the segment, channels c0 .. c0+TCH-1
  if constexpr (SRC == SRC_BF16 || SRC == SRC_F32) {
    // 16-byte buffer loads against a resource that starts at the tile's
    // first row and ends with the segment's last row inside the tile: rows
    // past the segment read as zeros, with no branch and one 32-bit offset
    // per load (cols <= 2^22 keeps 128 rows of offsets below 2^31)
    constexpr int VPR = TCH * (int)sizeof(TT) / 16;  // 16-byte vectors per tile row
    constexpr int RPP = kThreads / VPR;              // rows per pass
    const TT* x = static_cast<const TT*>(src);
    const int64_t rows_in = Me - m0 < TM ? Me - m0 : TM;  // >= 1: the tile starts inside the segment
    const int row_bytes = (int)(C * (int64_t)sizeof(TT));
    const brsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(x + (seg_start + m0) * C + c0), (short)0,
        (int)((rows_in - 1) * row_bytes + TCH * (int)sizeof(TT)), 0x00020000);
    const int vi = t % VPR;
#pragma unroll
    for (int p = 0; p < TM / RPP; ++p) {
      const int m = p * RPP + t / VPR;
      const v4i v = __builtin_amdgcn_raw_buffer_load_b128(rs, m * row_bytes + vi * 16, 0, 0);
      *reinterpret_cast<v4i*>(&tile[m * LROW + vi * 16]) = v;
    }
  } else {
    const uint8_t* codes = static_cast<const uint8_t*>(src);
    const int m = t >> 1;          // 2 threads per row, 64 channels each
    const int half = t & 1;
    uint4 w0 = make_uint4(0, 0, 0, 0), w1 = make_uint4(0, 0, 0, 0);
    uint32_t sc = 0;
    float mul = 0.0f;
    if (m0 + m < Me && c0 + 64 * half < C) {
      const int64_t g = seg_start + m0 + m;
      int64_t row = g;
      if (gather) {  // segment mode: R is the number of input rows the indices point into
        row = (int64_t)gather[g];
        row = row < 0 ? 0 : (row >= R ? R - 1 : row);
      }
      const uint4* cp = reinterpret_cast<const uint4*>(codes + row * (C >> 1) + (c0 >> 1) + half * 32);
      w0 = cp[0];
      w1 = cp[1];
      const uint8_t* sp = in_scales + row * (C >> 4) + (c0 >> 4) + half * 4;
      sc = (uint32_t)sp[0] | ((uint32_t)sp[1] << 8) | ((uint32_t)sp[2] << 16) | ((uint32_t)sp[3] << 24);
      mul = in_mode == BSQ_OUTER_ROW ? in_outer[row] : in_outer[SEG ? 0 : e];
    }
    if (half == 0) rowmul[m] = mul;
    const uint32_t wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    // q * s_b is exact in fp16: at most 6 significant bits, within [2^-10, 2688]
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const _Float16 s16 = (_Float16)e4m3_val((sc >> (8 * (q >> 1))) & 0xFFu);
      const h2 sv = {s16, s16};
      const h2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wv[q], 1.0f, 0) * sv;
      const h2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wv[q], 1.0f, 1) * sv;
      const h2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wv[q], 1.0f, 2) * sv;
      const h2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wv[q], 1.0f, 3) * sv;
      *reinterpret_cast<uint4*>(&tile[m * LROW + half * 128 + q * 16]) =
          make_uint4(__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
                     __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3));
    }
  }
  __syncthreads();

  // ---- phase R (ROWS): thread -> tile row t / 2, channels c0 + 32 (t % 2) .. +31
  // (reads the tile only; the phase-2 barrier below orders these reads before
  // the tile buffer is reused as the output stage)
  if constexpr (ROWS) {
    const int m = t >> 1, cb = 32 * (t & 1);
    if (m0 + m < Me && c0 + cb < C) {
      float z[32];
#pragma unroll
      for (int q = 0; q < (SRC == SRC_F32 ? 8 : 4); ++q) {
        const uint4 v = *reinterpret_cast<const uint4*>(&tile[m * LROW + (cb * (int)sizeof(TT)) + 16 * q]);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if constexpr (SRC == SRC_F32) {
            z[4 * q + u] = __uint_as_float(w[u]);
          } else {
            z[8 * q + 2 * u] = __uint_as_float(w[u] << 16);
            z[8 * q + 2 * u + 1] = __uint_as_float(w[u] & 0xFFFF0000u);
          }
        }
      }
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(z[i]));
      const int ex = e8m0_exponent(amax);
      const int64_t idx = (seg_start + m0 + m) * C + c0 + cb;  // element index of z[0] (row-major)
      uint32_t out[8];
      if constexpr (RND == BSQ_SR) {
        sr_block_e4m3(z, ex, seed, rows.stream_id, (uint64_t)(idx >> 3), out);
      } else {
        const float pw = pow2_neg(ex);
#pragma unroll
        for (int o = 0; o < 8; ++o)
          out[o] = e4m3_exact2(z[4 * o] * pw, z[4 * o + 1] * pw) | (e4m3_exact2(z[4 * o + 2] * pw, z[4 * o + 3] * pw) << 16);
      }
      uint4* dst = reinterpret_cast<uint4*>(rows.codes + idx);
      dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
      dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
      rows.scales[idx >> 5] = (uint8_t)(ex + 127);
    }
  }

  // ---- phase 2: thread -> channels c0 + CPT*lane .. +CPT-1, tokens m0 + 32*wave .. +31
  const int cl = CPT * (t & 63);
  const int tb = t >> 6;
  const int64_t mb = m0 + 32 * tb;
  const bool active = mb < Mp && c0 + cl < C;
  // MXFP8 codes are staged through LDS for whole-row stores, except from the
  // gathered, segmented NVFP4 source (requantized activations), where direct
  // 32-byte stores measured faster
  constexpr bool kStage = OUTF == BSQ_MXFP8 && !(SRC == SRC_NVFP4 && SEG);
  if constexpr (!kStage) {
    if (!active) return;  // no barrier follows on these paths
  }
  float z[CPT][32];
  if (!kStage || active) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int m = 32 * tb + i;
      if constexpr (SRC == SRC_F32) {
        z[0][i] = *reinterpret_cast<const float*>(&tile[m * LROW + cl * 4]);
      } else {
        if constexpr (SRC == SRC_BF16 && CPT == 1) {
          z[0][i] = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t*>(&tile[m * LROW + cl * 2]) << 16);
        } else if constexpr (SRC == SRC_BF16) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(&tile[m * LROW + cl * 2]);  // 2 channels
          z[0][i] = __uint_as_float(w << 16);
          z[CPT - 1][i] = __uint_as_float(w & 0xFFFF0000u);
        } else {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(&tile[m * LROW + cl * 2]);  // 2 channels
          const h2 hv = __builtin_bit_cast(h2, w);
          z[0][i] = (float)hv[0] * rowmul[m];
          z[1][i] = (float)hv[1] * rowmul[m];
        }
      }
    }
  }

  if constexpr (OUTF == BSQ_MXFP8) {
    // Codes and scales of the tile go through LDS (the input tile's buffer, free
    // once every phase-2 read is done) so that the output rows, 128 contiguous
    // tokens per channel, leave as whole 128-byte runs (8 lanes per channel)
    // instead of one 32-byte piece per lane and channel.
    constexpr int SP = 144;  // stage pitch: one channel's 128 token codes (+16: 16-byte aligned, 2-way banks)
    static_assert(TCH * SP + TCH * 4 <= TM * LROW, "output stage fits in the tile buffer");
    uint32_t out[CPT][8];
    int ex[CPT];
    if (!kStage || active) {
#pragma unroll
      for (int ch = 0; ch < CPT; ++ch) {
        const int64_t c = c0 + cl + ch;
        const int64_t obase = base + c * Mp + mb;  // output index of z[ch][0]
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(z[ch][i]));
        ex[ch] = e8m0_exponent(amax);
        if constexpr (RND == BSQ_SR) {
          sr_block_e4m3(z[ch], ex[ch], seed, stream_id, (uint64_t)(obase >> 3), out[ch]);
        } else {
          const float pw = pow2_neg(ex[ch]);  // |y| <= 448: the hardware convert is the nearest-even rounding
#pragma unroll
          for (int o = 0; o < 8; ++o)
            out[ch][o] = e4m3_exact2(z[ch][4 * o] * pw, z[ch][4 * o + 1] * pw) |
                         (e4m3_exact2(z[ch][4 * o + 2] * pw, z[ch][4 * o + 3] * pw) << 16);
        }
        if constexpr (!kStage) {  // each channel's codes leave as soon as they are ready
          uint4* dst = reinterpret_cast<uint4*>(out_codes + obase);
          dst[0] = make_uint4(out[ch][0], out[ch][1], out[ch][2], out[ch][3]);
          dst[1] = make_uint4(out[ch][4], out[ch][5], out[ch][6], out[ch][7]);
          out_scales[obase >> 5] = (uint8_t)(ex[ch] + 127);
        }
      }
    }
    if constexpr (!kStage) return;
    __syncthreads();  // every phase-2 read of the input tile is done
    uint8_t* const stage = tile;
    uint8_t* const stage_sc = tile + TCH * SP;
    if (active) {
#pragma unroll
      for (int ch = 0; ch < CPT; ++ch) {
        uint4* d = reinterpret_cast<uint4*>(stage + (cl + ch) * SP + 32 * tb);
        d[0] = make_uint4(out[ch][0], out[ch][1], out[ch][2], out[ch][3]);
        d[1] = make_uint4(out[ch][4], out[ch][5], out[ch][6], out[ch][7]);
        stage_sc[(cl + ch) * 4 + tb] = (uint8_t)(ex[ch] + 127);
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TCH * 8 / kThreads; ++k) {  // 16-byte pieces: channel id / 8, tokens 16 (id % 8) ..
      const int id = t + k * kThreads;
      const int ch = id >> 3, q = id & 7;
      const int64_t c = c0 + ch;
      if (c < C && m0 + 16 * q < Mp)
        store_nt(out_codes + base + c * Mp + m0 + 16 * q, *reinterpret_cast<const uint4*>(stage + ch * SP + 16 * q));
    }
    for (int id = t; id < TCH * 4; id += kThreads) {
      const int ch = id >> 2, b = id & 3;
      const int64_t c = c0 + ch;
      if (c < C && m0 + 32 * b < Mp) out_scales[((base + c * Mp + m0) >> 5) + b] = stage_sc[ch * 4 + b];
    }
  } else {
#pragma unroll
  for (int ch = 0; ch < CPT; ++ch) {
    const int64_t c = c0 + cl + ch;
    const int64_t obase = base + c * Mp + mb;  // output index of z[ch][0]
    {
      // NVFP4 target: outer s_t' from the item maximum, round-up block scales.
      const float am = __uint_as_float(amax_bits[e]);
      const float st = am > 0.0f ? am / 2688.0f : 1.0f;
      if (mt == 0 && by == 0 && t == 0 && ch == 0) out_outer[e] = st;
      const float d = 6.0f * st;
      uint32_t cw[4];
      uint32_t sc2[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(z[ch][16 * hb + i]));
        const uint32_t sc = e4m3_ru_cap(a / d);
        const float D = e4m3_val(sc) * st;
        const float inv = D >= kFltMinNormal ? 1.0f / D : 0.0f;
        sc2[hb] = sc;
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          const int g = 2 * hb + g2;
          uint32_t word = 0;
          float y[8];
          if constexpr (RND == BSQ_SR) {
            const U32x4 w = sr_words(seed, stream_id, (uint64_t)(obase >> 3) + g);
#pragma unroll
            for (int q = 0; q < 8; ++q) y[q] = sr_e2m1(z[ch][8 * g + q] * inv, r16_of(w, q));
          } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) y[q] = z[ch][8 * g + q] * inv;
          }
          word = BSQ_CVT_FP4X2(word, y[0], y[1], 0);
          word = BSQ_CVT_FP4X2(word, y[2], y[3], 1);
          word = BSQ_CVT_FP4X2(word, y[4], y[5], 2);
          word = BSQ_CVT_FP4X2(word, y[6], y[7], 3);
          cw[g] = word;
        }
      }
      // 8-byte stores: with rows % 32 == 16 an output row starts on an 8-byte boundary only
      *reinterpret_cast<uint2*>(out_codes + (obase >> 1)) = make_uint2(cw[0], cw[1]);
      out_scales[obase >> 4] = (uint8_t)sc2[0];
      if (mb + 16 < Mp) {  // else a trailing half block
        *reinterpret_cast<uint2*>(out_codes + (obase >> 1) + 8) = make_uint2(cw[2], cw[3]);
        out_scales[(obase >> 4) + 1] = (uint8_t)sc2[1];
      }
    }
  }
  }
}

__global__ void k_fill_u32(uint32_t* __restrict__ p, uint32_t v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void k_deq_nvfp4(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                            const float* __restrict__ outer, int mode, int64_t n, int64_t C, int64_t R,
                            float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t row = i / C;
  const uint32_t q = (codes[i >> 1] >> (4 * (i & 1))) & 0xFu;
  const float mag = (q & 7u) < 4u ? 0.5f * (float)(q & 7u) : ((q & 7u) < 6u ? (float)((q & 7u) - 2u) : ((q & 7u) == 6u ? 4.0f : 6.0f));
  const float v = (q & 8u) ? -mag : mag;
  const float st = mode == BSQ_OUTER_ROW ? outer[row] : outer[row / R];
  out[i] = (v * e4m3_val(scales[i >> 4])) * st;
}

__global__ void k_deq_mxfp8(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t n,
                            float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int s = (int)scales[i >> 5] - 127;
  out[i] = ldexpf(e4m3_val(codes[i]), s);
}

__global__ void k_rng_bits16(uint64_t seed, uint64_t stream_id, uint64_t first, int64_t n, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint64_t idx = first + (uint64_t)i;
  const U32x4 w = sr_words(seed, stream_id, idx >> 3);
  out[i] = (uint16_t)r16_of(w, (int)(idx & 7));
}

struct Plan {
  int32_t* slot_seg;
  int32_t* slot_mt;
  int64_t* seg_base;
  int64_t* seg_start;
  int64_t* seg_len;
  int64_t nslots;
};

size_t plan_bytes(int64_t rows, int64_t nseg) {
  const int64_t nslots = bsqh::tile_bound(rows, nseg, TM);
  return (size_t)((nseg * 24 + nslots * 8 + 255) / 256 * 256);
}

Plan make_plan(void* ws, int64_t rows, int64_t nseg) {
  Plan p;
  p.nslots = bsqh::tile_bound(rows, nseg, TM);
  p.seg_base = static_cast<int64_t*>(ws);
  p.seg_start = p.seg_base + nseg;
  p.seg_len = p.seg_start + nseg;
  p.slot_seg = reinterpret_cast<int32_t*>(p.seg_len + nseg);
  p.slot_mt = p.slot_seg + p.nslots;
  return p;
}

// 1-D grid of 8 * ceil(tiles / 8) workgroups for k_tq's XCD-aware remap.
inline unsigned tq_grid(int64_t ntiles, int64_t nct) { return (unsigned)((ntiles * nct + 7) / 8 * 8); }

// rows: dispatched rows (segments cover [0, rows)); in_rows: rows of the
// input table that gathered indices point into.
template <int SRC, bool ROWS = false>
int launch_tq_seg(const void* src, const uint8_t* in_scales, const float* in_outer, int in_mode, int64_t C,
                  const int32_t* gather, const int64_t* seg, int64_t nseg, int64_t rows, int64_t in_rows, int rnd,
                  uint64_t seed, uint64_t sid, uint8_t* oc, uint8_t* os, void* ws, hipStream_t s,
                  RowOut row_out = RowOut{}) {
  const Plan p = make_plan(ws, rows, nseg);
  hipLaunchKernelGGL(k_seg_plan, dim3(1), dim3(1024), 0, s, seg, (int)nseg, rows, C, TM, p.nslots, p.slot_seg,
                     p.slot_mt, p.seg_base, p.seg_start, p.seg_len);
  constexpr int TCH = tile_channels<SRC>();
  const dim3 grid(tq_grid(p.nslots, (C + TCH - 1) / TCH));
  if (rnd == BSQ_SR)
    hipLaunchKernelGGL((k_tq<SRC, BSQ_MXFP8, BSQ_SR, true, ROWS>), grid, dim3(kThreads), 0, s, src, in_scales,
                       in_outer, in_mode, C, in_rows, gather, p.seg_start, p.seg_len, p.slot_seg, p.slot_mt,
                       p.seg_base, nullptr, seed, sid, oc, os, nullptr, p.nslots, row_out);
  else
    hipLaunchKernelGGL((k_tq<SRC, BSQ_MXFP8, BSQ_RN, true, ROWS>), grid, dim3(kThreads), 0, s, src, in_scales,
                       in_outer, in_mode, C, in_rows, gather, p.seg_start, p.seg_len, p.slot_seg, p.slot_mt,
                       p.seg_base, nullptr, seed, sid, oc, os, nullptr, p.nslots, row_out);
  return bsqh::launch_status();
}

// One segment covering all rows, for seg_offsets == NULL.
__global__ void k_one_segment(int64_t rows, int64_t* __restrict__ seg) {
  if (threadIdx.x == 0) { seg[0] = 0; seg[1] = rows; }
}

}  // namespace

int bsq_quantize_mxfp8_rows(const void* x, int dtype, int64_t rows, int64_t cols, int rnd, uint64_t seed,
                            uint64_t stream_id, uint8_t* codes, uint8_t* scales, hipStream_t s);

extern "C" size_t bsq_quantize_mxfp8_workspace(int64_t rows, int transpose, int64_t num_segments) {
  if (!transpose || rows < 0) return 0;
  const int64_t nseg = num_segments > 0 ? num_segments : 1;
  return plan_bytes(rows, nseg) + 256;  // + room for a one-segment offset table
}

extern "C" int bsq_quantize_mxfp8(const void* x, int dtype, int64_t rows, int64_t cols, int transpose,
                                  const int64_t* seg_offsets, int64_t num_segments, int rnd, uint64_t seed,
                                  uint64_t stream_id, uint8_t* codes, uint8_t* scales, void* ws, size_t ws_bytes,
                                  bsq_stream_t stream) {
  BSQ_REQUIRE(dtype == BSQ_F32 || dtype == BSQ_BF16, BSQ_E_DTYPE);
  BSQ_REQUIRE(rnd == BSQ_RN || rnd == BSQ_SR, BSQ_E_ENUM);
  BSQ_REQUIRE(transpose == 0 || transpose == 1, BSQ_E_ENUM);
  BSQ_REQUIRE(rows >= 0 && cols >= 0, BSQ_E_SHAPE);
  if (!transpose) {
    BSQ_REQUIRE(cols % 32 == 0, BSQ_E_SHAPE);
    if (rows == 0 || cols == 0) return BSQ_OK;
    BSQ_REQUIRE(x && codes && scales, BSQ_E_NULL);
    BSQ_REQUIRE(bsqh::aligned16(x) && bsqh::aligned16(codes), BSQ_E_ALIGN);
    return bsq_quantize_mxfp8_rows(x, dtype, rows, cols, rnd, seed, stream_id, codes, scales,
                                   bsqh::as_stream(stream));
  }
  BSQ_REQUIRE(cols % TC == 0 && cols <= kMaxTransposeCols, BSQ_E_SHAPE);
  BSQ_REQUIRE(seg_offsets == nullptr || (num_segments >= 1 && num_segments <= 1024), BSQ_E_SHAPE);
  if (rows == 0 || cols == 0) return BSQ_OK;
  BSQ_REQUIRE(x && codes && scales && ws, BSQ_E_NULL);
  BSQ_REQUIRE(bsqh::aligned16(x) && bsqh::aligned16(codes) && bsqh::aligned16(ws), BSQ_E_ALIGN);
  const int64_t nseg = seg_offsets ? num_segments : 1;
  BSQ_REQUIRE(ws_bytes >= bsq_quantize_mxfp8_workspace(rows, 1, nseg), BSQ_E_WORKSPACE);
  hipStream_t s = bsqh::as_stream(stream);
  const int64_t* seg = seg_offsets;
  if (!seg) {
    int64_t* own = reinterpret_cast<int64_t*>(static_cast<char*>(ws) + plan_bytes(rows, 1));
    hipLaunchKernelGGL(k_one_segment, dim3(1), dim3(64), 0, s, rows, own);
    seg = own;
  }
  if (dtype == BSQ_BF16)
    return launch_tq_seg<SRC_BF16>(x, nullptr, nullptr, 0, cols, nullptr, seg, nseg, rows, rows, rnd, seed, stream_id,
                                   codes, scales, ws, s);
  return launch_tq_seg<SRC_F32>(x, nullptr, nullptr, 0, cols, nullptr, seg, nseg, rows, rows, rnd, seed, stream_id,
                                codes, scales, ws, s);
}

extern "C" int bsq_quantize_mxfp8_dual(const void* x, int dtype, int64_t rows, int64_t cols,
                                       const int64_t* seg_offsets, int64_t num_segments, int rnd, uint64_t seed,
                                       uint64_t stream_rows, uint64_t stream_t, uint8_t* codes, uint8_t* scales,
                                       uint8_t* codes_t, uint8_t* scales_t, void* ws, size_t ws_bytes,
                                       bsq_stream_t stream) {
  BSQ_REQUIRE(dtype == BSQ_F32 || dtype == BSQ_BF16, BSQ_E_DTYPE);
  BSQ_REQUIRE(rnd == BSQ_RN || rnd == BSQ_SR, BSQ_E_ENUM);
  BSQ_REQUIRE(rows >= 0 && cols >= 0 && cols % TC == 0 && cols <= kMaxTransposeCols, BSQ_E_SHAPE);
  BSQ_REQUIRE(seg_offsets == nullptr || (num_segments >= 1 && num_segments <= 1024), BSQ_E_SHAPE);
  if (rows == 0 || cols == 0) return BSQ_OK;
  BSQ_REQUIRE(x && codes && scales && codes_t && scales_t && ws, BSQ_E_NULL);
  BSQ_REQUIRE(bsqh::aligned16(x) && bsqh::aligned16(codes) && bsqh::aligned16(codes_t) && bsqh::aligned16(ws),
              BSQ_E_ALIGN);
  const int64_t nseg = seg_offsets ? num_segments : 1;
  BSQ_REQUIRE(ws_bytes >= bsq_quantize_mxfp8_workspace(rows, 1, nseg), BSQ_E_WORKSPACE);
  hipStream_t s = bsqh::as_stream(stream);
  const int64_t* seg = seg_offsets;
  if (!seg) {
    int64_t* own = reinterpret_cast<int64_t*>(static_cast<char*>(ws) + plan_bytes(rows, 1));
    hipLaunchKernelGGL(k_one_segment, dim3(1), dim3(64), 0, s, rows, own);
    seg = own;
  }
  RowOut ro;
  ro.codes = codes;
  ro.scales = scales;
  ro.stream_id = stream_rows;
  if (dtype == BSQ_BF16)
    return launch_tq_seg<SRC_BF16, true>(x, nullptr, nullptr, 0, cols, nullptr, seg, nseg, rows, rows, rnd, seed,
                                         stream_t, codes_t, scales_t, ws, s, ro);
  return launch_tq_seg<SRC_F32, true>(x, nullptr, nullptr, 0, cols, nullptr, seg, nseg, rows, rows, rnd, seed,
                                      stream_t, codes_t, scales_t, ws, s, ro);
}

extern "C" size_t bsq_requant_workspace(int64_t batch, int64_t rows, int64_t num_segments, int out_fmt, int gather) {
  if (gather) return plan_bytes(rows, num_segments > 0 ? num_segments : 1);
  if (out_fmt == BSQ_NVFP4 && batch > 0) return (size_t)((batch * 4 + 255) / 256 * 256);
  return 0;
}

extern "C" int bsq_requant_transpose_sr(const uint8_t* codes, const uint8_t* scales, const float* outer, int in_mode,
                                        int64_t batch, int64_t rows, int64_t cols, int64_t in_rows,
                                        const int32_t* row_gather, const int64_t* seg_offsets, int64_t num_segments,
                                        int out_fmt, int rnd, uint64_t seed, uint64_t stream_id, uint8_t* out_codes,
                                        uint8_t* out_scales, float* out_outer, void* ws, size_t ws_bytes,
                                        bsq_stream_t stream) {
  BSQ_REQUIRE(in_mode == BSQ_OUTER_TENSOR || in_mode == BSQ_OUTER_ROW, BSQ_E_ENUM);
  BSQ_REQUIRE(out_fmt == BSQ_NVFP4 || out_fmt == BSQ_MXFP8, BSQ_E_ENUM);
  BSQ_REQUIRE(rnd == BSQ_RN || rnd == BSQ_SR, BSQ_E_ENUM);
  BSQ_REQUIRE(batch >= 0 && rows >= 0 && cols >= 0 && in_rows >= 0 && cols % TC == 0, BSQ_E_SHAPE);
  const bool gather_mode = row_gather != nullptr || seg_offsets != nullptr;
  hipStream_t s = bsqh::as_stream(stream);
  if (gather_mode) {
    BSQ_REQUIRE(row_gather && seg_offsets, BSQ_E_NULL);
    BSQ_REQUIRE(batch == 1 && out_fmt == BSQ_MXFP8 && num_segments >= 1 && num_segments <= 1024, BSQ_E_SHAPE);
    if (rows == 0 || cols == 0) return BSQ_OK;
    BSQ_REQUIRE(codes && scales && outer && out_codes && out_scales && ws, BSQ_E_NULL);
    BSQ_REQUIRE(bsqh::aligned16(codes) && bsqh::aligned16(out_codes) && bsqh::aligned16(ws), BSQ_E_ALIGN);
    BSQ_REQUIRE(ws_bytes >= bsq_requant_workspace(1, rows, num_segments, out_fmt, 1), BSQ_E_WORKSPACE);
    BSQ_REQUIRE(in_rows >= 1, BSQ_E_SHAPE);
    return launch_tq_seg<SRC_NVFP4>(codes, scales, outer, in_mode, cols, row_gather, seg_offsets, num_segments, rows,
                                    in_rows, rnd, seed, stream_id, out_codes, out_scales, ws, s);
  }
  BSQ_REQUIRE(in_rows == batch * rows, BSQ_E_SHAPE);
  BSQ_REQUIRE(rows % (out_fmt == BSQ_MXFP8 ? 32 : 16) == 0, BSQ_E_SHAPE);
  if (batch == 0 || rows == 0 || cols == 0) return BSQ_OK;
  BSQ_REQUIRE(codes && scales && outer && out_codes && out_scales, BSQ_E_NULL);
  BSQ_REQUIRE(bsqh::aligned16(codes) && bsqh::aligned16(out_codes), BSQ_E_ALIGN);
  const int64_t tiles_per = (rows + TM - 1) / TM;
  constexpr int TCH = tile_channels<SRC_NVFP4>();
  const int64_t ntiles = batch * tiles_per;
  const dim3 grid(tq_grid(ntiles, (cols + TCH - 1) / TCH));
  if (out_fmt == BSQ_MXFP8) {
    if (rnd == BSQ_SR)
      hipLaunchKernelGGL((k_tq<SRC_NVFP4, BSQ_MXFP8, BSQ_SR, false>), grid, dim3(kThreads), 0, s, codes, scales, outer,
                         in_mode, cols, rows, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, seed, stream_id,
                         out_codes, out_scales, nullptr, ntiles, RowOut{});
    else
      hipLaunchKernelGGL((k_tq<SRC_NVFP4, BSQ_MXFP8, BSQ_RN, false>), grid, dim3(kThreads), 0, s, codes, scales, outer,
                         in_mode, cols, rows, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, seed, stream_id,
                         out_codes, out_scales, nullptr, ntiles, RowOut{});
    return bsqh::launch_status();
  }
  BSQ_REQUIRE(out_outer && ws, BSQ_E_NULL);
  BSQ_REQUIRE(((uintptr_t)ws & 3) == 0 && ((uintptr_t)out_outer & 3) == 0, BSQ_E_ALIGN);
  BSQ_REQUIRE(ws_bytes >= bsq_requant_workspace(batch, rows, 0, out_fmt, 0), BSQ_E_WORKSPACE);
  uint32_t* amax = static_cast<uint32_t*>(ws);
  hipLaunchKernelGGL(k_fill_u32, dim3(grid1(batch)), dim3(kThreads), 0, s, amax, 0u, batch);
  const int64_t nblk = batch * rows * cols / 16;
  hipLaunchKernelGGL(k_nvfp4_item_amax, dim3(grid1(nblk)), dim3(kThreads), 0, s, codes, scales, outer, in_mode, nblk,
                     cols / 16, rows, amax);
  if (rnd == BSQ_SR)
    hipLaunchKernelGGL((k_tq<SRC_NVFP4, BSQ_NVFP4, BSQ_SR, false>), grid, dim3(kThreads), 0, s, codes, scales, outer,
                       in_mode, cols, rows, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, amax, seed, stream_id,
                       out_codes, out_scales, out_outer, ntiles, RowOut{});
  else
    hipLaunchKernelGGL((k_tq<SRC_NVFP4, BSQ_NVFP4, BSQ_RN, false>), grid, dim3(kThreads), 0, s, codes, scales, outer,
                       in_mode, cols, rows, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, amax, seed, stream_id,
                       out_codes, out_scales, out_outer, ntiles, RowOut{});
  return bsqh::launch_status();
}

extern "C" int bsq_dequantize_nvfp4(const uint8_t* codes, const uint8_t* scales, const float* outer, int mode,
                                    int64_t batch, int64_t rows, int64_t cols, float* out, bsq_stream_t stream) {
  BSQ_REQUIRE(mode == BSQ_OUTER_TENSOR || mode == BSQ_OUTER_ROW || mode == BSQ_OUTER_GIVEN, BSQ_E_ENUM);
  BSQ_REQUIRE(batch >= 0 && rows >= 0 && cols >= 0 && cols % 16 == 0, BSQ_E_SHAPE);
  const int64_t n = batch * rows * cols;
  if (n == 0) return BSQ_OK;
  BSQ_REQUIRE(codes && scales && outer && out, BSQ_E_NULL);
  hipLaunchKernelGGL(k_deq_nvfp4, dim3(grid1(n)), dim3(kThreads), 0, bsqh::as_stream(stream), codes, scales, outer,
                     mode, n, cols, rows, out);
  return bsqh::launch_status();
}

extern "C" int bsq_dequantize_mxfp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                                    float* out, bsq_stream_t stream) {
  BSQ_REQUIRE(rows >= 0 && cols >= 0 && cols % 32 == 0, BSQ_E_SHAPE);
  const int64_t n = rows * cols;
  if (n == 0) return BSQ_OK;
  BSQ_REQUIRE(codes && scales && out, BSQ_E_NULL);
  hipLaunchKernelGGL(k_deq_mxfp8, dim3(grid1(n)), dim3(kThreads), 0, bsqh::as_stream(stream), codes, scales, n, out);
  return bsqh::launch_status();
}

extern "C" int bsq_rng_bits16(uint64_t seed, uint64_t stream_id, uint64_t first, int64_t n, uint16_t* out,
                              bsq_stream_t stream) {
  BSQ_REQUIRE(n >= 0, BSQ_E_SHAPE);
  if (n == 0) return BSQ_OK;
  BSQ_REQUIRE(out, BSQ_E_NULL);
  hipLaunchKernelGGL(k_rng_bits16, dim3(grid1(n)), dim3(kThreads), 0, bsqh::as_stream(stream), seed, stream_id, first,
                     n, out);
  return bsqh::launch_status();
}
