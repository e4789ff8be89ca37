// Row-wise block quantizers: round-to-nearest NVFP4 and row-wise MXFP8.
//
// "End-to-End 4-Bit Training", section "Low-precision formats on Blackwell":
// each block of 16 consecutive values is scaled from its largest magnitude
// (an E4M3 scale), values round to the nearest FP4 value, and an FP32 outer
// scale over a large group shifts the representable range [2^-10, 2688];
// MXFP8 uses blocks of 32 with E8M0 scales. Section "Recipe details": outer
// scales per token for activations, per expert for weights. The quantized
// linear layer figure (section "Re-quantization with stochastic rounding")
// quantizes the BF16 output gradient to MXFP8 with stochastic rounding.
//
// HBM-bound kernels: each thread owns whole blocks, loads them with 16-byte
// vector loads, reduces the block maximum in registers and writes packed codes
// with one 8- or 16-byte store. Per-row outer scales reduce across the threads
// of a row; per-tensor outer scales take a separate max pass over the tensor.
#include <cstdlib>
#include <type_traits>

#include "bsq_device.h"
#include "bsq_internal.h"

using namespace bsqd;

namespace {

constexpr int kThreads = 256;
// per-tensor outer scales need the group maximum before any block can round:
// one max pass over all items, then the quantize pass
constexpr int kAmaxVecPerThread = 32;  // 16-byte vectors per thread of the max pass
// The one-pass per-item kernel serves items of at least 1 MiB of bf16 (a
// grid-wide wait per item) and at most 4096 items (its slots in the workspace).
inline bool one_pass_items(int64_t B, int64_t R, int64_t C) { return R * C * 2 >= (1 << 20) && B <= 4096; }

// 16 consecutive elements of type T (bf16 bit patterns or float).
template <typename T> struct Blk16;
template <> struct Blk16<uint16_t> {
  uint32_t w[8];
  __device__ __forceinline__ void load(const uint16_t* p) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    const uint4 a = q[0], b = q[1];
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
  __device__ __forceinline__ float get(int i) const { return (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]); }
  __device__ __forceinline__ float absmax() const {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t a = w[i] & 0x7FFF7FFFu;
      const uint32_t lo = a & 0xFFFFu, hi = a >> 16;
      m = max(m, max(lo, hi));
    }
    return __uint_as_float(m << 16);  // magnitudes compare like their bit patterns
  }
};
template <> struct Blk16<float> {
  float w[16];
  __device__ __forceinline__ void load(const float* p) {
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = q[i];
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
  }
  __device__ __forceinline__ float get(int i) const { return w[i]; }
  __device__ __forceinline__ float absmax() const {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(w[i]));
    return m;
  }
};

template <typename T>
__device__ __forceinline__ float absmax16B(const uint4 v);
template <>
__device__ __forceinline__ float absmax16B<uint16_t>(const uint4 v) {
  const uint32_t w[4] = {v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu, v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = max(m, max(w[i] & 0xFFFFu, w[i] >> 16));
  return __uint_as_float(m << 16);
}
template <>
__device__ __forceinline__ float absmax16B<float>(const uint4 v) {
  return fmaxf(fmaxf(fabsf(__uint_as_float(v.x)), fabsf(__uint_as_float(v.y))),
               fmaxf(fabsf(__uint_as_float(v.z)), fabsf(__uint_as_float(v.w))));
}

__global__ void k_fill_u32(uint32_t* __restrict__ p, uint32_t v, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}
__global__ void k_copy_f32(const float* __restrict__ s, float* __restrict__ d, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) d[i] = s[i];
}

// Largest magnitude of each batch item [item0, item0 + gridDim.y), merged
// into amax_bits[item] with an atomic max on the bit pattern (non-negative
// floats order like their bits). Workgroup x of item y reduces the 16-byte
// vectors [x*per_wg, (x+1)*per_wg) of the item with 8 loads in flight per
// thread and issues one atomic.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_amax_items(const T* __restrict__ x, int64_t vec_per_item,
                                                         int64_t per_wg, uint32_t* __restrict__ amax_bits,
                                                         int64_t item0) {
  const int64_t item = item0 + blockIdx.y;
  const uint4* p = reinterpret_cast<const uint4*>(x) + item * vec_per_item;
  const int64_t lo = (int64_t)blockIdx.x * per_wg;
  const int64_t hi = lo + per_wg < vec_per_item ? lo + per_wg : vec_per_item;
  float m = 0.0f;
  int64_t i = lo + threadIdx.x;
  for (; i + 7 * kThreads < hi; i += 8 * kThreads) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[i + u * kThreads];
#pragma unroll
    for (int u = 0; u < 8; ++u) m = fmaxf(m, absmax16B<T>(v[u]));
  }
  for (; i < hi; i += kThreads) m = fmaxf(m, absmax16B<T>(p[i]));
  m = wave_max(m);
  __shared__ float red[kThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, red[w]);
    if (r > 0.0f) atomicMax(amax_bits + item, __float_as_uint(r));
  }
}

// Element codes of one block with scale code sc (outer st): w0 holds
// elements 0..7, w1 elements 8..15.
template <typename T>
__device__ __forceinline__ void nvfp4_codes(const Blk16<T>& b, uint32_t sc, float st, uint32_t& w0, uint32_t& w1) {
  const float D = e4m3_val(sc) * st;
  const float inv = D >= kFltMinNormal ? 1.0f / D : 0.0f;
  w0 = 0;
  w1 = 0;
  w0 = BSQ_CVT_FP4X2(w0, b.get(0) * inv, b.get(1) * inv, 0);
  w0 = BSQ_CVT_FP4X2(w0, b.get(2) * inv, b.get(3) * inv, 1);
  w0 = BSQ_CVT_FP4X2(w0, b.get(4) * inv, b.get(5) * inv, 2);
  w0 = BSQ_CVT_FP4X2(w0, b.get(6) * inv, b.get(7) * inv, 3);
  w1 = BSQ_CVT_FP4X2(w1, b.get(8) * inv, b.get(9) * inv, 0);
  w1 = BSQ_CVT_FP4X2(w1, b.get(10) * inv, b.get(11) * inv, 1);
  w1 = BSQ_CVT_FP4X2(w1, b.get(12) * inv, b.get(13) * inv, 2);
  w1 = BSQ_CVT_FP4X2(w1, b.get(14) * inv, b.get(15) * inv, 3);
}

// Squared quantization error of the block in float32, in element order:
// x^_i = f32(f32(q_i s_b) s_t), e_i = f32(x_i - x^_i), err = sum of f32(e_i^2)
// with each partial sum rounded (no fused operations).
template <typename T>
__device__ __forceinline__ float nvfp4_sq_err(const Blk16<T>& b, uint32_t w0, uint32_t w1, uint32_t sc, float st) {
  typedef float f2v __attribute__((ext_vector_type(2)));
  const float sv = e4m3_val(sc);
  float err = 0.0f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const uint32_t w = p < 4 ? w0 : w1;
    f2v q;
    switch (p & 3) {  // decode two codes (byte p & 3 of the word); the selector must be a constant
      case 0: q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); break;
      case 1: q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); break;
      case 2: q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); break;
      default: q = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); break;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float xh = (q[u] * sv) * st;
      const float e = b.get(2 * p + u) - xh;
      err = err + e * e;
    }
  }
  return err;
}

// One NVFP4 block of 16 (block maximum am, outer scale st): the E4M3 scale
// byte and 8 code bytes. FS (Four Over Six): the block also tries the scale that maps a_b to 4 and
// keeps it when its squared error is strictly smaller (ties keep 6).
template <bool FS, typename T>
__device__ __forceinline__ void nvfp4_block(const Blk16<T>& b, float am, float st, uint8_t* code_dst,
                                            uint8_t* scale_dst) {
  const float d = 6.0f * st;
  const float r = am / d;
  uint32_t sc = e4m3_rne_sat(r);
  uint32_t w0, w1;
  nvfp4_codes(b, sc, st, w0, w1);
  if constexpr (FS) {
    const float d4 = 4.0f * st;
    const float r4 = am / d4;
    const uint32_t sc4 = e4m3_rne_sat(r4);
    uint32_t v0, v1;
    nvfp4_codes(b, sc4, st, v0, v1);
    if (nvfp4_sq_err(b, v0, v1, sc4, st) < nvfp4_sq_err(b, w0, w1, sc, st)) {
      sc = sc4;
      w0 = v0;
      w1 = v1;
    }
  }
  *reinterpret_cast<uint2*>(code_dst) = make_uint2(w0, w1);
  *scale_dst = (uint8_t)sc;
}

// e^x in float32 (Cody and Waite's reduction, degree-7 Taylor polynomial):
// n = round-half-even(f32(x * f32(1/ln 2))) clamped to [-300, 300],
// r = f32(f32(x - n ln2_hi) - f32(n ln2_lo)) with ln2_hi = 0.693145751953125
// (n ln2_hi exact), p(r) = sum r^k / k! in Horner form, each product and sum
// rounded separately (no fused operations), e^x = p 2^n; within 1.2 ulp.
__device__ __forceinline__ float exp_cw(float x) {
  constexpr double kLn2 = 0.69314718055994530942;
  constexpr double c2 = 1.0 / 2, c3 = c2 / 3, c4 = c3 / 4, c5 = c4 / 5, c6 = c5 / 6, c7 = c6 / 7;
  float n = rintf(__fmul_rn(x, (float)(1.0 / kLn2)));
  n = fminf(fmaxf(n, -300.0f), 300.0f);
  float r = __fsub_rn(x, __fmul_rn(n, 0.693145751953125f));
  r = __fsub_rn(r, __fmul_rn(n, (float)(kLn2 - 0.693145751953125)));
  float p = (float)c7;
  p = __fadd_rn(__fmul_rn(p, r), (float)c6);
  p = __fadd_rn(__fmul_rn(p, r), (float)c5);
  p = __fadd_rn(__fmul_rn(p, r), (float)c4);
  p = __fadd_rn(__fmul_rn(p, r), (float)c3);
  p = __fadd_rn(__fmul_rn(p, r), (float)c2);
  p = __fadd_rn(__fmul_rn(p, r), 1.0f);
  p = __fadd_rn(__fmul_rn(p, r), 1.0f);
  return ldexpf(p, (int)n);
}

// SwiGLU of 16 gate and 16 up values: silu(g) * u, silu(g) = g / (1 + e^-g),
// every step rounded to float32.
template <typename T>
__device__ __forceinline__ void swiglu16(const T* gate, const T* up, Blk16<float>& out) {
  Blk16<T> g, u;
  g.load(gate);
  u.load(up);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float gi = g.get(i);
    const float s = gi / __fadd_rn(1.0f, exp_cw(-gi));
    out.w[i] = __fmul_rn(s, u.get(i));
  }
}

// NVFP4 round-to-nearest quantization of rows [row0, row_end). TPR threads
// share a row; each owns up to MAXB blocks of 16 (block j = lane + k*TPR).
// GLU: a row of x holds 2C values, gate [0, C) and up [C, 2C); the quantized
// values are their SwiGLU (the quantization step between the w13 and w2 GEMMs
// of the expert chain).
template <typename T, int TPR, int MAXB, int MODE, bool FS, bool GLU = false>
__global__ __launch_bounds__(kThreads) void k_quant_nvfp4(
    const T* __restrict__ x, int64_t row0, int64_t row_end, int64_t rows_per_item, int64_t C,
    const float* __restrict__ outer_in, const uint32_t* __restrict__ amax_bits,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ outer_out) {
  constexpr int RPW = kThreads / TPR;
  const int tr = threadIdx.x / TPR;
  const int tl = threadIdx.x % TPR;
  const int64_t row = row0 + (int64_t)blockIdx.x * RPW + tr;
  const bool row_ok = row < row_end;
  const int64_t nb = C >> 4;

  typedef typename std::conditional<GLU, Blk16<float>, Blk16<T>>::type Blk;
  Blk blk[MAXB];
  float am[MAXB];
  float rmax = 0.0f;
#pragma unroll
  for (int k = 0; k < MAXB; ++k) {
    const int64_t j = tl + (int64_t)k * TPR;
    am[k] = 0.0f;
    if (row_ok && j < nb) {
      if constexpr (GLU)
        swiglu16(x + row * 2 * C + j * 16, x + row * 2 * C + C + j * 16, blk[k]);
      else
        blk[k].load(x + row * C + j * 16);
      am[k] = blk[k].absmax();
      rmax = fmaxf(rmax, am[k]);
    }
  }

  float st;
  if constexpr (MODE == BSQ_OUTER_ROW) {
    if constexpr (TPR <= 64) {
      rmax = group_max<TPR>(rmax);
    } else {
      __shared__ float red[kThreads / 64];
      const float wm = wave_max(rmax);
      if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = wm;
      __syncthreads();
      rmax = red[tr * (TPR / 64)];
#pragma unroll
      for (int w = 1; w < TPR / 64; ++w) rmax = fmaxf(rmax, red[tr * (TPR / 64) + w]);
    }
    st = rmax > 0.0f ? rmax / 2688.0f : 1.0f;
    if (row_ok && tl == 0) outer_out[row] = st;
  } else {
    const int64_t item = (row_ok ? row : row_end - 1) / rows_per_item;
    if constexpr (MODE == BSQ_OUTER_TENSOR) {
      const float a = __uint_as_float(amax_bits[item]);
      st = a > 0.0f ? a / 2688.0f : 1.0f;
    } else {
      st = outer_in[item];
    }
    if (row_ok && tl == 0 && row % rows_per_item == 0) outer_out[item] = st;
  }

#pragma unroll
  for (int k = 0; k < MAXB; ++k) {
    const int64_t j = tl + (int64_t)k * TPR;
    if (row_ok && j < nb) nvfp4_block<FS>(blk[k], am[k], st, codes + row * (C >> 1) + j * 8, scales + row * nb + j);
  }
}

// Per-item outer scale in one pass over HBM. Each group of the grid (one
// workgroup per CU; two groups when two of the kernel's workgroups fit on a
// CU, so that one group's loads overlap the other's wait and stores) walks its
// items (every groups-th item) in order. A workgroup keeps its shares of up to
// S items in registers (S register sets of at most BPT blocks of 16 per
// thread): it publishes the maximum of its share of an item in its own slot
// slot[e][w] (bit pattern with bit 31 set as the arrival mark: magnitudes
// have it clear) as soon as that share's loads have arrived, waits until
// every slot of an item is marked only when the item is next to be quantized
// (the maximum of the slots is the item's maximum), and has the loads of the
// following items in flight meanwhile (item_pipeline below). One wave polls
// the slots; the others wait at a barrier that waits for LDS operations only,
// so their loads stay in flight (a plain __syncthreads would wait for every
// outstanding load and store).
// The wait is bounded: after spin_limit polls the workgroup reduces the whole
// item itself (the same maximum, from a second read), so every wave always
// finishes. The slots start at zero. Slot accesses are relaxed device-scope
// atomics: no other memory is shared between workgroups (x is only read, each
// output byte has one writer), so no release/acquire (and no L2 write-back or
// invalidation on this multi-XCD device) is needed.
constexpr int kOnePassThreads = 512;
constexpr int kOnePassMaxWg = 512;
constexpr uint32_t kSpinLimit = 1u << 22;  // polls before a workgroup stops waiting (about 0.1 s)
#ifndef BSQ_ONEPASS_GROUPS
#define BSQ_ONEPASS_GROUPS 2
#endif
constexpr int kOnePassGroups = BSQ_ONEPASS_GROUPS;

// The poll limit; the environment variable BSQ_WAIT_POLLS overrides it (tests
// set 0 to take every workgroup through the fallback).
inline uint32_t wait_polls() {
  const char* v = getenv("BSQ_WAIT_POLLS");
  return v ? (uint32_t)strtoul(v, nullptr, 10) : kSpinLimit;
}

// Workgroup barrier that completes this wave's LDS operations first and
// leaves its global loads and stores in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Every thread calls it. Wave 0 polls the nwg (<= kOnePassMaxWg) slots of one
// item until all carry the arrival mark, then leaves their maximum in *out
// (LDS; -1 when spin_limit polls found a slot unmarked); the other waves wait
// at an LDS-only barrier with their loads in flight. Returns *out. A caller
// writes *out again only after another barrier.
__device__ __forceinline__ float poll_slots(const uint32_t* __restrict__ row, int nwg, uint32_t spin_limit,
                                            float* out) {
  const int t = threadIdx.x;
  if (t < 64) {  // lane l polls slots l, l + 64, ...
    float mx = -1.0f;
    for (uint32_t spins = 0; spins < spin_limit; ++spins) {
      // all loads are issued before the first is waited for (lanes past the
      // last slot re-read it), so a poll costs one round trip
      uint32_t v[kOnePassMaxWg / 64];
#pragma unroll
      for (int q = 0; q < kOnePassMaxWg / 64; ++q) {
        const int w = t + 64 * q;
        v[q] = __hip_atomic_load(row + (w < nwg ? w : nwg - 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      bool all = true;
      float m = 0.0f;
#pragma unroll
      for (int q = 0; q < kOnePassMaxWg / 64; ++q) {
        all = all && (v[q] & 0x80000000u) != 0;
        m = fmaxf(m, __uint_as_float(v[q] & 0x7FFFFFFFu));
      }
      if (__all(all)) {  // wave-uniform
        mx = wave_max(m);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (t == 0) *out = mx;
  }
  lds_barrier();
  return *out;
}

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>), in order.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Lambdas of the one-pass kernels are inlined whatever their size: a call
// would put the register sets on the stack.
#define BSQ_AI __attribute__((always_inline))

// The item loop of the one-pass kernels, with S register sets: issue(set, i)
// starts the loads of the workgroup's share of (group-local) item i into a
// set, publish(set, i) reduces and publishes the share's maximum (waiting for
// that set's loads), wait(i) returns item i's outer scale once every
// workgroup has published it, quant(set, i, st) writes item i's codes. Item i
// lives in set i % S. Step i starts the loads of item i + S - 1 (into the set
// item i - 1 has left) and publishes item i + P, then quantizes item i once
// its wait is over. With three sets or more the publish (of item i + S - 2,
// whose loads are the second youngest in flight) comes before the wait for
// item i; with two it comes after it (P = 1: item i + 1's loads are the
// youngest). In the main loop every step issues and publishes
// unconditionally, so the wait the compiler places for one set's loads leaves
// the younger sets' loads in flight; the last 2S - 2 steps check the count.
template <int S, typename Issue, typename Publish, typename Wait, typename Quant>
__device__ __forceinline__ void item_pipeline(int64_t n, Issue&& issue, Publish&& publish, Wait&& wait,
                                              Quant&& quant) {
  static_assert(S >= 2, "one item in flight at least");
  constexpr int P = S == 2 ? 1 : S - 2;
  auto step = [&](auto set, int64_t i, auto tail) BSQ_AI {
    constexpr int sc = decltype(set)::value;
    constexpr bool tl = decltype(tail)::value;
    if (!tl || i + S - 1 < n) issue((sc + S - 1) % S, i + S - 1);
    if constexpr (S == 2) {
      const float st = wait(i);
      if (!tl || i + P < n) publish((sc + P) % S, i + P);
      quant(sc, i, st);
    } else {
      if (!tl || i + P < n) publish((sc + P) % S, i + P);
      quant(sc, i, wait(i));
    }
  };
  // prologue: loads of items 0 .. S - 2, maxima of items 0 .. P - 1
  static_for<S - 1>([&](auto j) BSQ_AI {
    if (j < n) issue(j, j);
  });
  static_for<P>([&](auto j) BSQ_AI {
    if (j < n) publish(j, j);
  });
  int64_t i = 0;
  for (; i + 2 * S - 2 < n; i += S) static_for<S>([&](auto j) BSQ_AI { step(j, i + j, std::false_type{}); });
  static_for<2 * S - 2>([&](auto j) BSQ_AI {
    if (i + j < n) step(std::integral_constant<int, j % S>{}, i + j, std::true_type{});
  });
}

// S register sets of BPT blocks per thread: up to S - 1 items in flight
// besides the one being waited for.
template <typename T, int BPT, int S>
__global__ __launch_bounds__(kOnePassThreads) void k_quant_nvfp4_items(
    const T* __restrict__ x, int64_t B, int64_t bpi, int groups, uint32_t* __restrict__ slot,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ outer_out, uint32_t spin_limit) {
  // `groups` independent grids of nwg workgroups each: group g takes items
  // g, g + groups, ..., so that one group's loads overlap another's wait
  const int nwg = gridDim.x / groups;
  const int grp = blockIdx.x / nwg, wid = blockIdx.x % nwg;
  const int64_t share = (bpi + nwg - 1) / nwg;  // blocks per workgroup and item, <= BPT * threads
  const int64_t lo = (int64_t)wid * share;
  const int64_t hi = lo + share < bpi ? lo + share : bpi;
  const int t = threadIdx.x;
  __shared__ float red[kOnePassThreads / 64];
  __shared__ float slots_max;  // item maximum found by the polling wave; -1: polls ran out
  auto wg_max = [&](float m) BSQ_AI -> float {  // every thread calls it; result in every thread
    m = wave_max(m);
    if ((t & 63) == 0) red[t >> 6] = m;
    lds_barrier();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kOnePassThreads / 64; ++w) r = fmaxf(r, red[w]);
    lds_barrier();
    return r;
  };
  Blk16<T> blk[S][BPT];
  // The thread's first block of a share, from a copy of the thread index the
  // compiler cannot see through: per-block addresses are then recomputed
  // where they are used instead of being held in registers for every set.
  auto first = [&]() BSQ_AI -> int64_t {
    int tr = t;
    asm volatile("" : "+v"(tr));
    return lo + tr;
  };
  // Loads and maxima are branch-free (a thread's blocks past its share load a
  // valid block of the item and count as zero), so the compiler's wait for a
  // set's loads is exact and never also waits for the other sets' loads.
  auto issue = [&](int b, int64_t e) BSQ_AI {  // start the loads of item e's share into set b
    const int64_t j0 = first();
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const int64_t j = j0 + (int64_t)k * kOnePassThreads;
      blk[b][k].load(x + (e * bpi + (j < bpi ? j : bpi - 1)) * 16);
    }
  };
  auto thread_max = [&](int b) BSQ_AI -> float {  // largest block maximum of set b (waits for its loads)
    const int64_t j0 = first();
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const float a = blk[b][k].absmax();
      m = fmaxf(m, j0 + (int64_t)k * kOnePassThreads < hi ? a : 0.0f);
    }
    return m;
  };
  auto publish = [&](int64_t e, float m) BSQ_AI {
    const float r = wg_max(m);
    if (t == 0) __hip_atomic_store(slot + e * nwg + wid, __float_as_uint(r) | 0x80000000u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
  };
  auto outer_scale = [&](int64_t e) BSQ_AI -> float {
    float a = poll_slots(slot + e * nwg, nwg, spin_limit, &slots_max);
    if (a < 0.0f) {  // uniform: the polls ran out; reduce the whole item here
      float m = 0.0f;
      for (int64_t j = t; j < bpi; j += kOnePassThreads) {
        Blk16<T> q;
        q.load(x + (e * bpi + j) * 16);
        m = fmaxf(m, q.absmax());
      }
      a = wg_max(m);
    }
    // slots_max is written again only in the next item's wait, after the
    // barriers of the publish in between
    return a > 0.0f ? a / 2688.0f : 1.0f;
  };
  auto quantize = [&](int b, int64_t e, float st) BSQ_AI {
    if (wid == 0 && t == 0) outer_out[e] = st;
    const int64_t j0 = first();
#pragma unroll
    for (int k = 0; k < BPT; ++k) {
      const int64_t j = j0 + (int64_t)k * kOnePassThreads;
      if (j < hi) nvfp4_block<false>(blk[b][k], blk[b][k].absmax(), st, codes + (e * bpi + j) * 8, scales + e * bpi + j);
    }
  };
  const int64_t n = grp < B ? (B - grp + groups - 1) / groups : 0;  // this group's items
  if (n <= 0) return;
  auto it = [&](int64_t i) BSQ_AI -> int64_t { return grp + i * groups; };
  item_pipeline<S>(
      n, [&](int set, int64_t i) BSQ_AI { issue(set, it(i)); },
      [&](int set, int64_t i) BSQ_AI { publish(it(i), thread_max(set)); },
      [&](int64_t i) BSQ_AI { return outer_scale(it(i)); },
      [&](int set, int64_t i, float st) BSQ_AI { quantize(set, it(i), st); });
}

// Row-wise MXFP8: one thread per block of 32 (element index = blk*32 + i).
template <typename T, int RND>
__global__ __launch_bounds__(kThreads) void k_mxfp8_rows(const T* __restrict__ x, int64_t nblk, uint64_t seed,
                                                         uint64_t stream_id, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales) {
  const int64_t blk = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (blk >= nblk) return;
  Blk16<T> a, b;
  a.load(x + blk * 32);
  b.load(x + blk * 32 + 16);
  const float amax = fmaxf(a.absmax(), b.absmax());
  const int e = e8m0_exponent(amax);
  const float pw = pow2_neg(e);
  uint32_t out[8];
  if constexpr (RND == BSQ_SR) {
    float z[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) z[i] = i < 16 ? a.get(i) : b.get(i - 16);
    sr_block_e4m3(z, e, seed, stream_id, (uint64_t)blk * 4, out);
  } else {
#pragma unroll
    for (int o = 0; o < 8; ++o) {
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 4 * o + q;
        v[q] = (i < 16 ? a.get(i) : b.get(i - 16)) * pw;
      }
      out[o] = e4m3_exact2(v[0], v[1]) | (e4m3_exact2(v[2], v[3]) << 16);
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + blk * 32);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  scales[blk] = (uint8_t)(e + 127);
}

inline unsigned grid1(int64_t n, int t = kThreads) { return (unsigned)((n + t - 1) / t); }

template <typename T, int MODE, bool FS, bool GLU = false>
int launch_quant(const T* x, int64_t row0, int64_t row_end, int64_t R, int64_t C, const float* outer_in,
                 const uint32_t* amax, uint8_t* codes, uint8_t* scales, float* outer_out, hipStream_t s) {
  const int64_t nb = C / 16;
  const int64_t n = row_end - row0;
  if (n <= 0) return BSQ_OK;
#define BSQ_QL(TPR, MAXB)                                                                                      \
  hipLaunchKernelGGL((k_quant_nvfp4<T, TPR, MAXB, MODE, FS, GLU>), dim3(grid1(n, kThreads / TPR)), dim3(kThreads), 0, \
                     s, x, row0, row_end, R, C, outer_in, amax, codes, scales, outer_out)
  // one wave per row up to 512 blocks (the row maximum is a wave reduction),
  // up to 8 blocks (256 bytes of bf16) in flight per thread
  if (nb <= 16) BSQ_QL(16, 1);
  else if (nb <= 64) BSQ_QL(64, 1);
  else if (nb <= 128) BSQ_QL(64, 2);
  else if (nb <= 256) BSQ_QL(64, 4);
  else if (nb <= 512) BSQ_QL(64, 8);
  else if (nb <= 1024) BSQ_QL(256, 4);
  else BSQ_QL(256, 8);
#undef BSQ_QL
  return bsqh::launch_status();
}

// Workgroups of the one-pass kernel (BPT blocks per thread, S register
// sets) that fit on a CU at once (queried once per instantiation).
template <typename T, int BPT, int S>
int items_per_cu() {
  static const int per_cu = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(&k_quant_nvfp4_items<T, BPT, S>),
                                                     kOnePassThreads, 0) != hipSuccess)
      nb = 1;
    return nb;
  }();
  return per_cu;
}

// One launch of the one-pass kernel: `groups` groups of nwg workgroups each
// (the slots, B * nwg words, are cleared first).
template <typename T, int BPT, int S>
void launch_items(const T* x, int64_t B, int64_t bpi, int64_t nwg, int groups, uint32_t* ws, uint8_t* codes,
                  uint8_t* scales, float* outer_out, hipStream_t s) {
  hipLaunchKernelGGL(k_fill_u32, dim3(grid1(B * nwg)), dim3(kThreads), 0, s, ws, 0u, B * nwg);
  hipLaunchKernelGGL((k_quant_nvfp4_items<T, BPT, S>), dim3((unsigned)(nwg * groups)), dim3(kOnePassThreads), 0, s, x,
                     B, bpi, groups, ws, codes, scales, outer_out, wait_polls());
}

// The whole chip per item: one workgroup per CU, and a second group of them
// taking alternate items when two of the kernel's workgroups fit on a CU.
template <typename T, int BPT, int S>
void launch_items_full(const T* x, int64_t B, int64_t bpi, int64_t nwg, uint32_t* ws, uint8_t* codes, uint8_t* scales,
                       float* outer_out, hipStream_t s) {
  launch_items<T, BPT, S>(x, B, bpi, nwg, items_per_cu<T, BPT, S>() >= 2 ? kOnePassGroups : 1, ws, codes, scales,
                          outer_out, s);
}

template <typename T>
int quantize_nvfp4_t(const T* x, int64_t B, int64_t R, int64_t C, int mode, bool fs, const float* outer_in,
                     uint8_t* codes, uint8_t* scales, float* outer_out, uint32_t* ws, hipStream_t s) {
  const int64_t rows = B * R;
  if (mode == BSQ_OUTER_ROW)
    return fs ? launch_quant<T, BSQ_OUTER_ROW, true>(x, 0, rows, R, C, nullptr, nullptr, codes, scales, outer_out, s)
              : launch_quant<T, BSQ_OUTER_ROW, false>(x, 0, rows, R, C, nullptr, nullptr, codes, scales, outer_out, s);
  if (mode == BSQ_OUTER_GIVEN)
    return fs ? launch_quant<T, BSQ_OUTER_GIVEN, true>(x, 0, rows, R, C, outer_in, nullptr, codes, scales, outer_out, s)
              : launch_quant<T, BSQ_OUTER_GIVEN, false>(x, 0, rows, R, C, outer_in, nullptr, codes, scales, outer_out, s);
  // one pass when the items are large (a grid-wide wait per item) and a
  // workgroup's share fits in registers
  const int64_t bpi = R * C / 16;
  const int64_t nwg = bsqh::device_cus() < kOnePassMaxWg ? bsqh::device_cus() : kOnePassMaxWg;
  const int64_t per_thread = ((bpi + nwg - 1) / nwg + kOnePassThreads - 1) / kOnePassThreads;
  // (a float share of 8 blocks per thread would not fit in registers)
  if (!fs && one_pass_items(B, R, C) && per_thread <= (sizeof(T) == 2 ? 8 : 4)) {
    // Many items: two halves of the chip (nwg / 2 workgroups each, one per
    // CU) take alternate items, so each item's wait involves half the
    // workgroups; used where a half's share fits three register sets.
    // Measured 7-12% faster for 64 items of 6-12 MB; with few items the
    // halves' pipelines do not fill (3-5% slower at 3-16 items).
    const int64_t half = nwg / 2;
    const int64_t pt_half = half ? ((bpi + half - 1) / half + kOnePassThreads - 1) / kOnePassThreads : 0;
    if constexpr (sizeof(T) == 2) {
      if (B >= 32 && pt_half >= 2 && pt_half <= 6) {
        if (pt_half <= 2) launch_items<T, 2, 3>(x, B, bpi, half, 2, ws, codes, scales, outer_out, s);
        else if (pt_half <= 3) launch_items<T, 3, 3>(x, B, bpi, half, 2, ws, codes, scales, outer_out, s);
        else if (pt_half <= 4) launch_items<T, 4, 3>(x, B, bpi, half, 2, ws, codes, scales, outer_out, s);
        else if (pt_half <= 5) launch_items<T, 5, 3>(x, B, bpi, half, 2, ws, codes, scales, outer_out, s);
        else launch_items<T, 6, 3>(x, B, bpi, half, 2, ws, codes, scales, outer_out, s);
        return bsqh::launch_status();
      }
    }
    // three register sets where they fit in registers, two for the largest shares
    if (per_thread <= 1) launch_items_full<T, 1, 3>(x, B, bpi, nwg, ws, codes, scales, outer_out, s);
    else if (per_thread <= 2) launch_items_full<T, 2, 3>(x, B, bpi, nwg, ws, codes, scales, outer_out, s);
    else if constexpr (sizeof(T) == 2) {
      if (per_thread <= 3) launch_items_full<T, 3, 3>(x, B, bpi, nwg, ws, codes, scales, outer_out, s);
      else if (per_thread <= 4) launch_items_full<T, 4, 3>(x, B, bpi, nwg, ws, codes, scales, outer_out, s);
      else if (per_thread <= 5) launch_items_full<T, 5, 3>(x, B, bpi, nwg, ws, codes, scales, outer_out, s);
      else if (per_thread <= 6) launch_items_full<T, 6, 3>(x, B, bpi, nwg, ws, codes, scales, outer_out, s);
      else if (per_thread <= 7) launch_items_full<T, 7, 3>(x, B, bpi, nwg, ws, codes, scales, outer_out, s);
      else launch_items_full<T, 8, 2>(x, B, bpi, nwg, ws, codes, scales, outer_out, s);
    } else {
      launch_items_full<T, 4, 2>(x, B, bpi, nwg, ws, codes, scales, outer_out, s);
    }
    return bsqh::launch_status();
  }
  hipLaunchKernelGGL(k_fill_u32, dim3(grid1(B)), dim3(kThreads), 0, s, ws, 0u, B);
  const int64_t vec = R * C * (int64_t)sizeof(T) / 16;  // per item
  const int64_t per_wg = (int64_t)kThreads * kAmaxVecPerThread;
  const int64_t gx = (vec + per_wg - 1) / per_wg;
  for (int64_t i0 = 0; i0 < B; i0 += 65535) {  // grid y limit
    const int64_t ni = (B - i0) < 65535 ? (B - i0) : 65535;
    hipLaunchKernelGGL(k_amax_items<T>, dim3((unsigned)gx, (unsigned)ni), dim3(kThreads), 0, s, x, vec, per_wg, ws,
                       i0);
  }
  return fs ? launch_quant<T, BSQ_OUTER_TENSOR, true>(x, 0, rows, R, C, nullptr, ws, codes, scales, outer_out, s)
            : launch_quant<T, BSQ_OUTER_TENSOR, false>(x, 0, rows, R, C, nullptr, ws, codes, scales, outer_out, s);
}

// ------------------------------------------------------------ square tiles
// The 16x16-tile variant ("Block-scaled backward passes", row-vs-column and
// outlier figures): one E4M3 scale per 16x16 tile from the tile's largest
// magnitude, every element then rounding as in a 1x16 block with that scale.
// Because the tile is square, the quantization of the transpose is the
// transpose of the codes, so one read of x yields both layouts.
//
// A workgroup unit is 128 rows x 64 columns (8 x 4 tiles, 512 threads): wave
// w owns tile row w, lane (tc = lane / 16, j = lane % 16) owns row j of tile
// tc (16 elements), and the tile maximum reduces over the 16 lanes of a tile.
// Row-major codes and scales are stored straight from registers. For the
// transposed layout the codes go through LDS (128 rows of 32 bytes, 8 bytes of
// skew per 16 rows so that the reads below hit 8 different banks); thread
// (c, q) then gathers column c of rows 16q .. 16q + 15 (one byte per row) and
// writes them as one 8-byte run, so a wave's store covers 8 columns x 64
// contiguous bytes.
constexpr int kSqThreads = 512;
constexpr int kSqRows = 128, kSqCols = 64;
constexpr int kSqLdsBytes = kSqRows * 32 + 8 * (kSqRows / 16);

__device__ __forceinline__ int sq_lds(int r, int byte) { return r * 32 + 8 * (r >> 4) + byte; }

struct SqGeom {
  int64_t R, C, nrt, nct;  // units: nrt = ceil(R / 128) down, nct = ceil(C / 64) across
};

// First row and column of unit u of an item. RF: units ordered down the rows
// first (the one-shot kernel: the XCD-local neighbours continue each other's
// transposed runs); else across the columns first (the one-pass kernel: a
// workgroup's units and its XCD neighbours read long runs of each row).
template <bool RF>
__device__ __forceinline__ void sq_origin(const SqGeom& g, int64_t u, int64_t& r0, int64_t& c0) {
  if constexpr (RF) {
    r0 = (u % g.nrt) * kSqRows;
    c0 = (u / g.nrt) * kSqCols;
  } else {
    r0 = (u / g.nct) * kSqRows;
    c0 = (u % g.nct) * kSqCols;
  }
}

// Loads this thread's 16 elements of unit u (column-major unit order) of item
// b; returns their largest magnitude (0 for a thread outside the matrix).
template <bool RF, typename T>
__device__ __forceinline__ float sq_load(const T* __restrict__ x, const SqGeom& g, int64_t b, int64_t u, Blk16<T>& e) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int64_t r0, c0;
  sq_origin<RF>(g, u, r0, c0);
  const int64_t r = r0 + 16 * w, col = c0 + 16 * (lane >> 4);
  if (r >= g.R || col >= g.C) return 0.0f;  // R and C are multiples of 16: whole 16x16 tiles
  e.load(x + (b * g.R + r + (lane & 15)) * g.C + col);
  return e.absmax();
}

// Quantizes unit u of item b from registers with outer scale st. Every thread
// of the workgroup calls it (it holds barriers when TR).
template <bool RF, bool TR, typename T>
__device__ __forceinline__ void sq_unit(const Blk16<T>& e, float m, float st, const SqGeom& g, int64_t b, int64_t u,
                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                        uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t, uint8_t* lds,
                                        uint8_t* lds_sc) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tc = lane >> 4, j = lane & 15;
  int64_t r0, c0;
  sq_origin<RF>(g, u, r0, c0);
  const int64_t row = r0 + 16 * w + j, col = c0 + 16 * tc;
  const bool ok = r0 + 16 * w < g.R && col < g.C;
  m = group_max<16>(m);
  const uint32_t sc = e4m3_rne_sat(m / (6.0f * st));
  uint32_t a0 = 0, a1 = 0;
  if (ok) {
    nvfp4_codes(e, sc, st, a0, a1);
    *reinterpret_cast<uint2*>(codes + ((b * g.R + row) * g.C + col) / 2) = make_uint2(a0, a1);
    scales[(b * g.R + row) * (g.C / 16) + col / 16] = (uint8_t)sc;
  }
  if constexpr (TR) {
    *reinterpret_cast<uint2*>(lds + sq_lds(16 * w + j, tc * 8)) = make_uint2(a0, a1);
    if (j == 0) lds_sc[w * 4 + tc] = (uint8_t)sc;
    lds_barrier();  // LDS only: loads of later items stay in flight
    const int c = threadIdx.x >> 3, q = threadIdx.x & 7;  // column c, rows 16q .. 16q + 15
    const int64_t rr = r0 + 16 * q, cc = c0 + c;
    if (rr < g.R && cc < g.C) {
      const int sh = (c & 1) * 4;
      uint32_t o[2] = {0u, 0u};
#pragma unroll
      for (int p = 0; p < 8; ++p) {  // rows 2p, 2p + 1 of the tile -> output byte p
        const uint32_t lo = (lds[sq_lds(16 * q + 2 * p, c >> 1)] >> sh) & 0xFu;
        const uint32_t hi = (lds[sq_lds(16 * q + 2 * p + 1, c >> 1)] >> sh) & 0xFu;
        o[p >> 2] |= (lo | (hi << 4)) << (8 * (p & 3));
      }
      *reinterpret_cast<uint2*>(codes_t + ((b * g.C + cc) * g.R + rr) / 2) = make_uint2(o[0], o[1]);
      scales_t[(b * g.C + cc) * (g.R / 16) + rr / 16] = lds_sc[q * 4 + (c >> 4)];
    }
    lds_barrier();  // the LDS unit is reused by the next unit of a persistent workgroup
  }
}

// One unit per workgroup; the outer scale comes from amax_bits (TENSOR,
// filled by k_amax_items) or outer_in (GIVEN).
template <typename T, int MODE, bool TR>
__global__ __launch_bounds__(kSqThreads) void k_quant_nvfp4_square(
    const T* __restrict__ x, SqGeom g, int64_t nunits, const float* __restrict__ outer_in,
    const uint32_t* __restrict__ amax_bits, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
    uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t, float* __restrict__ outer_out) {
  __shared__ __align__(16) uint8_t lds[kSqLdsBytes];
  __shared__ uint8_t lds_sc[32];
  // consecutive units run on one XCD (blockIdx.x % 8 picks it)
  const int64_t per_xcd = (nunits + 7) / 8;
  const int64_t unit = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (unit >= nunits) return;  // uniform over the workgroup
  const int64_t per_item = g.nrt * g.nct;
  const int64_t b = unit / per_item, u = unit % per_item;
  float st;
  if constexpr (MODE == BSQ_OUTER_TENSOR) {
    const float a = __uint_as_float(amax_bits[b]);
    st = a > 0.0f ? a / 2688.0f : 1.0f;
  } else {
    st = outer_in[b];
  }
  if (threadIdx.x == 0 && u == 0) outer_out[b] = st;
  Blk16<T> e;
  const float m = sq_load<true>(x, g, b, u, e);
  sq_unit<true, TR>(e, m, st, g, b, u, codes, scales, codes_t, scales_t, lds, lds_sc);
}

// Per-item outer scale in one HBM pass, as k_quant_nvfp4_items (groups of
// resident workgroups, each group walking every groups-th item): logical
// workgroup v of a group (consecutive v on one XCD) owns the contiguous units
// [v*U/n, (v+1)*U/n) of each of its items (U units per item, at most UPW),
// publishes the maximum of its share in slot[item][v], prefetches its share of
// its next item, waits (bounded, with the same re-read fallback) for all slots
// of the item and quantizes its units from registers.
template <typename T, int UPW, bool TR>
__global__ __launch_bounds__(kSqThreads) void k_quant_nvfp4_square_items(
    const T* __restrict__ x, SqGeom g, int64_t B, int groups, uint32_t* __restrict__ slot,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint8_t* __restrict__ codes_t,
    uint8_t* __restrict__ scales_t, float* __restrict__ outer_out, uint32_t spin_limit) {
  __shared__ __align__(16) uint8_t lds[kSqLdsBytes];
  __shared__ uint8_t lds_sc[32];
  __shared__ float red[kSqThreads / 64];
  const int nwg = gridDim.x / groups;  // workgroups per group, a multiple of 8
  const int grp = blockIdx.x / nwg, wid = blockIdx.x % nwg;
  const int v = (wid % 8) * (nwg / 8) + wid / 8;
  const int64_t upi = g.nrt * g.nct;
  const int64_t lo = v * upi / nwg, hi = (v + 1) * upi / nwg;
  const int t = threadIdx.x;
  auto wg_max = [&](float m) -> float {
    m = wave_max(m);
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kSqThreads / 64; ++w) r = fmaxf(r, red[w]);
    __syncthreads();
    return r;
  };
  Blk16<T> blk[2][UPW];
  float am[2][UPW];
  auto load = [&](int s, int64_t e) -> float {
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < UPW; ++k) {
      am[s][k] = 0.0f;
      if (lo + k < hi) {
        am[s][k] = sq_load<false>(x, g, e, lo + k, blk[s][k]);
        m = fmaxf(m, am[s][k]);
      }
    }
    return m;
  };
  auto publish = [&](int64_t e, float m) {
    const float r = wg_max(m);
    if (t == 0)
      __hip_atomic_store(slot + e * nwg + v, __float_as_uint(r) | 0x80000000u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  };
  auto item = [&](int s, int64_t e) {
    float mx = 0.0f;
    uint32_t spins = 0;
    for (;;) {
      uint32_t val = 0x80000000u;
      if (t < nwg) val = __hip_atomic_load(slot + e * nwg + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (!__syncthreads_or((val & 0x80000000u) == 0)) {
        mx = __uint_as_float(val & 0x7FFFFFFFu);
        break;
      }
      if (++spins >= spin_limit) {  // uniform: reduce the whole item here
        const uint4* p = reinterpret_cast<const uint4*>(x + e * g.R * g.C);
        const int64_t nvec = g.R * g.C * (int64_t)sizeof(T) / 16;
        for (int64_t i = t; i < nvec; i += kSqThreads) mx = fmaxf(mx, absmax16B<T>(p[i]));
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    const float a = wg_max(mx);
    const float st = a > 0.0f ? a / 2688.0f : 1.0f;
    if (v == 0 && t == 0) outer_out[e] = st;
#pragma unroll
    for (int k = 0; k < UPW; ++k)
      if (lo + k < hi)  // uniform over the workgroup
        sq_unit<false, TR>(blk[s][k], am[s][k], st, g, e, lo + k, codes, scales, codes_t, scales_t, lds, lds_sc);
  };
  const int64_t n = grp < B ? (B - grp + groups - 1) / groups : 0;  // this group's items
  if (n <= 0) return;
  auto it = [&](int64_t i) -> int64_t { return grp + i * groups; };
  publish(it(0), load(0, it(0)));
  int64_t i = 0;
  for (; i + 1 < n; i += 2) {  // register sets alternate: item i in set 0, i + 1 in set 1
    const float m1 = load(1, it(i + 1));
    item(0, it(i));
    publish(it(i + 1), m1);
    if (i + 2 < n) {
      const float m2 = load(0, it(i + 2));
      item(1, it(i + 1));
      publish(it(i + 2), m2);
    } else {
      item(1, it(i + 1));
    }
  }
  if (i < n && (n & 1)) item(0, it(i));
}

// Workgroups per group of the one-pass square kernel (a multiple of 8, one per
// CU), or 0 when the items are small (see one_pass_items) or need more than
// max_upw units per workgroup.
inline int64_t square_one_pass_wgs(int64_t B, int64_t R, int64_t C, int64_t max_upw) {
  if (!one_pass_items(B, R, C)) return 0;
  const int64_t cus = bsqh::device_cus() < kOnePassMaxWg ? bsqh::device_cus() : kOnePassMaxWg;
  const int64_t nwg = cus / 8 * 8;
  const int64_t upi = ((R + kSqRows - 1) / kSqRows) * ((C + kSqCols - 1) / kSqCols);
  return nwg >= 8 && upi <= max_upw * nwg ? nwg : 0;
}

template <typename T>
int quantize_nvfp4_square_t(const T* x, int64_t B, int64_t R, int64_t C, int mode, const float* outer_in,
                            uint8_t* codes, uint8_t* scales, uint8_t* codes_t, uint8_t* scales_t,
                            float* outer_out, uint32_t* ws, hipStream_t s) {
  const SqGeom g{R, C, (R + kSqRows - 1) / kSqRows, (C + kSqCols - 1) / kSqCols};
  const bool tr = codes_t != nullptr;
  if (mode == BSQ_OUTER_TENSOR) {
    // at most 3 (bf16) or 2 (float) units per workgroup; two groups where a
    // workgroup stays within 128 VGPRs (two per CU)
    const int64_t nwg = square_one_pass_wgs(B, R, C, sizeof(T) == 2 ? 3 : 2);
    if (nwg) {
      const int64_t upw = (g.nrt * g.nct + nwg - 1) / nwg;
      const int grp = sizeof(T) == 2 || upw <= 1 ? kOnePassGroups : 1;
      hipLaunchKernelGGL(k_fill_u32, dim3(grid1(B * nwg)), dim3(kThreads), 0, s, ws, 0u, B * nwg);
#define BSQ_SQI(UPW, TR)                                                                                          \
  hipLaunchKernelGGL((k_quant_nvfp4_square_items<T, UPW, TR>), dim3((unsigned)(nwg * grp)), dim3(kSqThreads), 0, s, \
                     x, g, B, grp, ws, codes, scales, codes_t, scales_t, outer_out, wait_polls())
      if (upw <= 1) { if (tr) BSQ_SQI(1, true); else BSQ_SQI(1, false); }
      else if (upw <= 2) { if (tr) BSQ_SQI(2, true); else BSQ_SQI(2, false); }
      else if constexpr (sizeof(T) == 2) { if (tr) BSQ_SQI(3, true); else BSQ_SQI(3, false); }
#undef BSQ_SQI
      return bsqh::launch_status();
    }
    hipLaunchKernelGGL(k_fill_u32, dim3(grid1(B)), dim3(kThreads), 0, s, ws, 0u, B);
    const int64_t vec = R * C * (int64_t)sizeof(T) / 16;
    const int64_t per_wg = (int64_t)kThreads * kAmaxVecPerThread;
    const int64_t gx = (vec + per_wg - 1) / per_wg;
    for (int64_t i0 = 0; i0 < B; i0 += 65535) {
      const int64_t ni = (B - i0) < 65535 ? (B - i0) : 65535;
      hipLaunchKernelGGL(k_amax_items<T>, dim3((unsigned)gx, (unsigned)ni), dim3(kThreads), 0, s, x, vec, per_wg,
                         ws, i0);
    }
  }
  const int64_t nunits = B * g.nrt * g.nct;
  const dim3 grid((unsigned)((nunits + 7) / 8 * 8));
#define BSQ_SQ(MODE, TR)                                                                                      \
  hipLaunchKernelGGL((k_quant_nvfp4_square<T, MODE, TR>), grid, dim3(kSqThreads), 0, s, x, g, nunits, outer_in, \
                     ws, codes, scales, codes_t, scales_t, outer_out)
  if (mode == BSQ_OUTER_TENSOR) {
    if (tr) BSQ_SQ(BSQ_OUTER_TENSOR, true);
    else BSQ_SQ(BSQ_OUTER_TENSOR, false);
  } else {
    if (tr) BSQ_SQ(BSQ_OUTER_GIVEN, true);
    else BSQ_SQ(BSQ_OUTER_GIVEN, false);
  }
#undef BSQ_SQ
  return bsqh::launch_status();
}

}  // namespace

extern "C" size_t bsq_quantize_nvfp4_workspace(int64_t batch, int64_t rows, int64_t cols, int mode) {
  mode &= ~BSQ_NVFP4_FOUR_OVER_SIX;
  if (mode != BSQ_OUTER_TENSOR || batch <= 0) return 0;
  // per item: the maximum's bits, or one arrival slot per workgroup of the one-pass kernel
  const int64_t words = one_pass_items(batch, rows, cols) ? batch * kOnePassMaxWg : batch;
  return (size_t)((words * 4 + 255) / 256 * 256);
}

extern "C" int bsq_quantize_nvfp4(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols, int mode,
                                  const float* outer_in, uint8_t* codes, uint8_t* scales, float* outer_out,
                                  void* ws, size_t ws_bytes, bsq_stream_t stream) {
  BSQ_REQUIRE(dtype == BSQ_F32 || dtype == BSQ_BF16, BSQ_E_DTYPE);
  const bool fs = (mode & BSQ_NVFP4_FOUR_OVER_SIX) != 0;
  const int flags_in = mode;
  mode &= ~BSQ_NVFP4_FOUR_OVER_SIX;
  BSQ_REQUIRE(mode == BSQ_OUTER_TENSOR || mode == BSQ_OUTER_ROW || mode == BSQ_OUTER_GIVEN, BSQ_E_ENUM);
  BSQ_REQUIRE(batch >= 0 && rows >= 0 && cols >= 0 && cols % 16 == 0 && cols <= 32768, BSQ_E_SHAPE);
  if (batch == 0) return BSQ_OK;
  const bool empty = rows == 0 || cols == 0;
  BSQ_REQUIRE(outer_out && (mode != BSQ_OUTER_GIVEN || outer_in), BSQ_E_NULL);
  BSQ_REQUIRE(empty || (x && codes && scales), BSQ_E_NULL);
  BSQ_REQUIRE(bsqh::aligned16(x) && bsqh::aligned16(codes), BSQ_E_ALIGN);
  BSQ_REQUIRE(((uintptr_t)outer_out & 3) == 0 && ((uintptr_t)outer_in & 3) == 0, BSQ_E_ALIGN);
  const size_t need = empty ? 0 : bsq_quantize_nvfp4_workspace(batch, rows, cols, flags_in);
  if (need) {
    BSQ_REQUIRE(ws, BSQ_E_NULL);
    BSQ_REQUIRE(((uintptr_t)ws & 3) == 0, BSQ_E_ALIGN);
    BSQ_REQUIRE(ws_bytes >= need, BSQ_E_WORKSPACE);
  }
  hipStream_t s = bsqh::as_stream(stream);
  if (empty) {  // empty groups: outer scale 1 (or the given one)
    const int64_t n = mode == BSQ_OUTER_ROW ? batch * rows : batch;
    if (n == 0) return BSQ_OK;
    if (mode == BSQ_OUTER_GIVEN)
      hipLaunchKernelGGL(k_copy_f32, dim3(grid1(n)), dim3(kThreads), 0, s, outer_in, outer_out, n);
    else
      hipLaunchKernelGGL(k_fill_u32, dim3(grid1(n)), dim3(kThreads), 0, s, reinterpret_cast<uint32_t*>(outer_out),
                         0x3F800000u, n);
    return bsqh::launch_status();
  }
  if (dtype == BSQ_BF16)
    return quantize_nvfp4_t<uint16_t>(static_cast<const uint16_t*>(x), batch, rows, cols, mode, fs, outer_in, codes,
                                      scales, outer_out, static_cast<uint32_t*>(ws), s);
  return quantize_nvfp4_t<float>(static_cast<const float*>(x), batch, rows, cols, mode, fs, outer_in, codes, scales,
                                 outer_out, static_cast<uint32_t*>(ws), s);
}

// Row-wise MXFP8 (transpose == 0); the transposed form lives with the
// transpose kernels.
int bsq_quantize_mxfp8_rows(const void* x, int dtype, int64_t rows, int64_t cols, int rnd, uint64_t seed,
                            uint64_t stream_id, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t nblk = rows * cols / 32;
  if (nblk == 0) return BSQ_OK;
  if (dtype == BSQ_BF16) {
    if (rnd == BSQ_SR)
      hipLaunchKernelGGL((k_mxfp8_rows<uint16_t, BSQ_SR>), dim3(grid1(nblk)), dim3(kThreads), 0, s,
                         static_cast<const uint16_t*>(x), nblk, seed, stream_id, codes, scales);
    else
      hipLaunchKernelGGL((k_mxfp8_rows<uint16_t, BSQ_RN>), dim3(grid1(nblk)), dim3(kThreads), 0, s,
                         static_cast<const uint16_t*>(x), nblk, seed, stream_id, codes, scales);
  } else {
    if (rnd == BSQ_SR)
      hipLaunchKernelGGL((k_mxfp8_rows<float, BSQ_SR>), dim3(grid1(nblk)), dim3(kThreads), 0, s,
                         static_cast<const float*>(x), nblk, seed, stream_id, codes, scales);
    else
      hipLaunchKernelGGL((k_mxfp8_rows<float, BSQ_RN>), dim3(grid1(nblk)), dim3(kThreads), 0, s,
                         static_cast<const float*>(x), nblk, seed, stream_id, codes, scales);
  }
  return bsqh::launch_status();
}

extern "C" size_t bsq_quantize_nvfp4_square_workspace(int64_t batch, int64_t rows, int64_t cols, int mode) {
  if (mode != BSQ_OUTER_TENSOR || batch <= 0) return 0;
  // per item: the maximum's bits, or one arrival slot per workgroup of the one-pass kernel
  const int64_t words = one_pass_items(batch, rows, cols) ? batch * kOnePassMaxWg : batch;
  return (size_t)((words * 4 + 255) / 256 * 256);
}

extern "C" int bsq_quantize_nvfp4_square(const void* x, int dtype, int64_t batch, int64_t rows, int64_t cols,
                                         int mode, const float* outer_in, uint8_t* codes, uint8_t* scales,
                                         uint8_t* codes_t, uint8_t* scales_t, float* outer_out, void* ws,
                                         size_t ws_bytes, bsq_stream_t stream) {
  BSQ_REQUIRE(dtype == BSQ_F32 || dtype == BSQ_BF16, BSQ_E_DTYPE);
  BSQ_REQUIRE(mode == BSQ_OUTER_TENSOR || mode == BSQ_OUTER_GIVEN, BSQ_E_ENUM);
  BSQ_REQUIRE(batch >= 0 && rows >= 0 && cols >= 0 && rows % 16 == 0 && cols % 16 == 0, BSQ_E_SHAPE);
  if (batch == 0) return BSQ_OK;
  // element offsets stay far inside int64, the grid inside 2^31 workgroups
  BSQ_REQUIRE(rows <= ((int64_t)1 << 31) && cols <= ((int64_t)1 << 31), BSQ_E_SHAPE);
  BSQ_REQUIRE(batch <= ((int64_t)1 << 46) / (rows * cols > 0 ? rows * cols : 1), BSQ_E_SHAPE);
  const int64_t nunits = batch * ((rows + 127) / 128) * ((cols + 63) / 64);
  BSQ_REQUIRE(nunits <= ((int64_t)1 << 31) - 8, BSQ_E_SHAPE);
  const bool empty = rows == 0 || cols == 0;
  BSQ_REQUIRE(outer_out && (mode != BSQ_OUTER_GIVEN || outer_in), BSQ_E_NULL);
  BSQ_REQUIRE(empty || (x && codes && scales), BSQ_E_NULL);
  BSQ_REQUIRE((codes_t == nullptr) == (scales_t == nullptr), BSQ_E_NULL);
  BSQ_REQUIRE(bsqh::aligned16(x) && bsqh::aligned16(codes) && bsqh::aligned16(codes_t), BSQ_E_ALIGN);
  BSQ_REQUIRE(((uintptr_t)outer_out & 3) == 0 && ((uintptr_t)outer_in & 3) == 0, BSQ_E_ALIGN);
  const size_t need = empty ? 0 : bsq_quantize_nvfp4_square_workspace(batch, rows, cols, mode);
  if (need) {
    BSQ_REQUIRE(ws, BSQ_E_NULL);
    BSQ_REQUIRE(((uintptr_t)ws & 3) == 0, BSQ_E_ALIGN);
    BSQ_REQUIRE(ws_bytes >= need, BSQ_E_WORKSPACE);
  }
  hipStream_t s = bsqh::as_stream(stream);
  if (empty) {
    if (mode == BSQ_OUTER_GIVEN)
      hipLaunchKernelGGL(k_copy_f32, dim3(grid1(batch)), dim3(kThreads), 0, s, outer_in, outer_out, batch);
    else
      hipLaunchKernelGGL(k_fill_u32, dim3(grid1(batch)), dim3(kThreads), 0, s,
                         reinterpret_cast<uint32_t*>(outer_out), 0x3F800000u, batch);
    return bsqh::launch_status();
  }
  if (dtype == BSQ_BF16)
    return quantize_nvfp4_square_t<uint16_t>(static_cast<const uint16_t*>(x), batch, rows, cols, mode, outer_in,
                                             codes, scales, codes_t, scales_t, outer_out,
                                             static_cast<uint32_t*>(ws), s);
  return quantize_nvfp4_square_t<float>(static_cast<const float*>(x), batch, rows, cols, mode, outer_in, codes,
                                        scales, codes_t, scales_t, outer_out, static_cast<uint32_t*>(ws), s);
}

extern "C" int bsq_swiglu_quantize_nvfp4(const void* h13, int dtype, int64_t rows, int64_t ffn, int flags,
                                         uint8_t* codes, uint8_t* scales, float* outer_out, bsq_stream_t stream) {
  BSQ_REQUIRE(dtype == BSQ_F32 || dtype == BSQ_BF16, BSQ_E_DTYPE);
  BSQ_REQUIRE((flags & ~BSQ_NVFP4_FOUR_OVER_SIX) == 0, BSQ_E_ENUM);
  BSQ_REQUIRE(rows >= 0 && ffn >= 0 && ffn % 16 == 0 && ffn <= 32768, BSQ_E_SHAPE);
  if (rows == 0 || ffn == 0) {
    if (rows > 0) {  // empty rows: outer scale 1
      BSQ_REQUIRE(outer_out, BSQ_E_NULL);
      hipLaunchKernelGGL(k_fill_u32, dim3(grid1(rows)), dim3(kThreads), 0, bsqh::as_stream(stream),
                         reinterpret_cast<uint32_t*>(outer_out), 0x3F800000u, rows);
      return bsqh::launch_status();
    }
    return BSQ_OK;
  }
  BSQ_REQUIRE(h13 && codes && scales && outer_out, BSQ_E_NULL);
  BSQ_REQUIRE(bsqh::aligned16(h13) && bsqh::aligned16(codes) && ((uintptr_t)outer_out & 3) == 0, BSQ_E_ALIGN);
  hipStream_t s = bsqh::as_stream(stream);
  const bool fs = (flags & BSQ_NVFP4_FOUR_OVER_SIX) != 0;
  if (dtype == BSQ_BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(h13);
    return fs ? launch_quant<uint16_t, BSQ_OUTER_ROW, true, true>(p, 0, rows, rows, ffn, nullptr, nullptr, codes,
                                                                  scales, outer_out, s)
              : launch_quant<uint16_t, BSQ_OUTER_ROW, false, true>(p, 0, rows, rows, ffn, nullptr, nullptr, codes,
                                                                   scales, outer_out, s);
  }
  const float* p = static_cast<const float*>(h13);
  return fs ? launch_quant<float, BSQ_OUTER_ROW, true, true>(p, 0, rows, rows, ffn, nullptr, nullptr, codes, scales,
                                                             outer_out, s)
            : launch_quant<float, BSQ_OUTER_ROW, false, true>(p, 0, rows, rows, ffn, nullptr, nullptr, codes, scales,
                                                              outer_out, s);
}
