// Routing of tokens to per-expert row segments.
//
// "End-to-End 4-Bit Training", section "Quantized communications": a small
// router decides where each token goes and tokens are dispatched to the
// routed experts. On one GPU the dispatch is a permutation: every (token,
// slot) pair of the top-k routing becomes one row of the expert GEMMs, rows
// grouped by expert and, inside an expert, ordered by token.
//
// Three deterministic passes over chunks of 256 tokens: per-chunk expert
// counts, one scan that turns them into segment offsets and per-chunk bases,
// and a scatter whose within-chunk rank comes from an LDS bitmap of the
// tokens routed to each expert (a popcount of the earlier tokens).
#include <mutex>

#include "bsq_device.h"
#include "bsq_internal.h"

namespace {

constexpr int kChunk = 256;

__global__ __launch_bounds__(kChunk) void k_route_count(const int32_t* __restrict__ ids, int64_t tokens, int k, int E,
                                                        int32_t* __restrict__ counts) {
  extern __shared__ int32_t cnt[];
  for (int e = threadIdx.x; e < E; e += kChunk) cnt[e] = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kChunk + threadIdx.x;
  if (t < tokens) {
    for (int j = 0; j < k; ++j) {
      const int e = ids[t * k + j];
      if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kChunk) counts[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// One workgroup of 1024 threads turns the per-chunk counts into exclusive
// bases (in place) and the segment offsets. Thread (e, p) = (t % E, t / E),
// p < P = 1024 / E, owns expert e's counts in a contiguous range of chunks:
// it sums them (independent loads), the partial sums are scanned over p
// in LDS, the expert totals over e, and each thread then writes its range's
// bases.
__global__ __launch_bounds__(1024) void k_route_scan(int32_t* __restrict__ counts, int64_t nchunks, int E,
                                                     int64_t* __restrict__ seg_offsets) {
  __shared__ int64_t part[1024];
  __shared__ int64_t tot[1024];
  const int t = threadIdx.x;
  const int P = 1024 / E;
  const int e = t % E, p = t / E;
  const bool own = p < P;
  const int64_t per = (nchunks + P - 1) / P;
  const int64_t c0 = own ? (int64_t)p * per : 0;
  const int64_t c1 = own ? (c0 + per < nchunks ? c0 + per : nchunks) : 0;
  int64_t sum = 0;
  for (int64_t c = c0; c < c1; ++c) sum += counts[c * E + e];
  part[t] = sum;  // part[p * E + e] for the owning threads
  __syncthreads();
  int64_t total = 0;
  if (t < E) {  // exclusive prefix of expert t's partial sums over p
    for (int q = 0; q < P; ++q) {
      const int64_t v = part[q * E + t];
      part[q * E + t] = total;
      total += v;
    }
  }
  tot[t] = total;  // zero for t >= E
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {  // inclusive scan of the expert totals
    const int64_t v = t >= o ? tot[t - o] : 0;
    __syncthreads();
    tot[t] += v;
    __syncthreads();
  }
  if (t < E) seg_offsets[t] = tot[t] - total;
  if (t == E - 1) seg_offsets[E] = tot[t];
  if (own) {
    const int64_t start = (e ? tot[e - 1] : 0) + part[t];
    int64_t run = start;
    for (int64_t c = c0; c < c1; ++c) {
      const int32_t v = counts[c * E + e];
      counts[c * E + e] = (int32_t)run;
      run += v;
    }
  }
}

__global__ __launch_bounds__(kChunk) void k_route_scatter(const int32_t* __restrict__ ids, int64_t tokens, int k, int E,
                                                          const int32_t* __restrict__ bases, int32_t* __restrict__ row_index,
                                                          int32_t* __restrict__ pair_row) {
  extern __shared__ uint32_t bits[];  // [E][kChunk / 32]
  constexpr int W = kChunk / 32;
  for (int i = threadIdx.x; i < E * W; i += kChunk) bits[i] = 0;
  __syncthreads();
  const int tl = threadIdx.x;
  const int64_t t = (int64_t)blockIdx.x * kChunk + tl;
  if (t < tokens) {
    for (int j = 0; j < k; ++j) {
      const int e = ids[t * k + j];
      if (e >= 0 && e < E) atomicOr(&bits[e * W + (tl >> 5)], 1u << (tl & 31));
    }
  }
  __syncthreads();
  if (t >= tokens) return;
  for (int j = 0; j < k; ++j) {
    const int e = ids[t * k + j];
    if (e < 0 || e >= E) continue;
    int rank = 0;
    for (int w = 0; w < (tl >> 5); ++w) rank += __popc(bits[e * W + w]);
    rank += __popc(bits[e * W + (tl >> 5)] & ((1u << (tl & 31)) - 1u));
    const int32_t row = bases[(int64_t)blockIdx.x * E + e] + rank;
    row_index[row] = (int32_t)t;
    pair_row[t * k + j] = row;
  }
}

}  // namespace

extern "C" size_t bsq_route_workspace(int64_t tokens, int64_t E) {
  if (tokens <= 0 || E <= 0) return 0;
  const int64_t nchunks = (tokens + kChunk - 1) / kChunk;
  return (size_t)((nchunks * E * 4 + 255) / 256 * 256);
}

// The three passes; `counts` holds nchunks * E int32 (every slot that the
// scan and the scatter read is written by the count pass first).
static int route_launch(const int32_t* topk_ids, int64_t tokens, int64_t k, int64_t E, int32_t* row_index,
                        int64_t* seg_offsets, int32_t* pair_row, int32_t* counts, hipStream_t s) {
  const int64_t nchunks = (tokens + kChunk - 1) / kChunk;
  if (tokens > 0)
    hipLaunchKernelGGL(k_route_count, dim3((unsigned)nchunks), dim3(kChunk), E * sizeof(int32_t), s, topk_ids, tokens,
                       (int)k, (int)E, counts);
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(1024), 0, s, counts, nchunks, (int)E, seg_offsets);
  if (tokens > 0)
    hipLaunchKernelGGL(k_route_scatter, dim3((unsigned)nchunks), dim3(kChunk), E * (kChunk / 32) * sizeof(uint32_t), s,
                       topk_ids, tokens, (int)k, (int)E, static_cast<const int32_t*>(counts), row_index, pair_row);
  return bsqh::launch_status();
}

extern "C" int bsq_route(const int32_t* topk_ids, int64_t tokens, int64_t k, int64_t E, int32_t* row_index,
                         int64_t* seg_offsets, int32_t* pair_row, void* ws, size_t ws_bytes, bsq_stream_t stream) {
  BSQ_REQUIRE(tokens >= 0 && k >= 1 && k <= 64 && E >= 1 && E <= 1024, BSQ_E_SHAPE);
  BSQ_REQUIRE(tokens * k < (int64_t)1 << 31, BSQ_E_SHAPE);
  BSQ_REQUIRE(seg_offsets, BSQ_E_NULL);
  if (tokens > 0) {
    BSQ_REQUIRE(topk_ids && row_index && pair_row && ws, BSQ_E_NULL);
    BSQ_REQUIRE(((uintptr_t)ws & 3) == 0, BSQ_E_ALIGN);
    BSQ_REQUIRE(ws_bytes >= bsq_route_workspace(tokens, E), BSQ_E_WORKSPACE);
  }
  return route_launch(topk_ids, tokens, k, E, row_index, seg_offsets, pair_row, static_cast<int32_t*>(ws),
                      bsqh::as_stream(stream));
}

// ---------------------------------------------------------------- no-alloc
// Routing for callers that cannot allocate: the per-chunk counts live in a
// file-scope device array instead of a caller workspace. Each GPU holds its
// own copy for the life of the process; host code reaches it only through
// the address that hipGetSymbolAddress returns on that device (the array's
// name in host code is a host-side stand-in, not a device address).
constexpr size_t kRouteScratchBytes = BSQ_ROUTE_NOALLOC_MAX_BYTES;
static __device__ __align__(256) uint8_t scratch[kRouteScratchBytes];

constexpr int kMaxDevices = 64;
static void* g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, looked up once per device.
static int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BSQ_E_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BSQ_E_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BSQ_OK;
}

extern "C" int bsq_route_noalloc(const int32_t* topk_ids, int64_t tokens, int64_t k, int64_t E, int32_t* row_index,
                                 int64_t* seg_offsets, int32_t* pair_row, bsq_stream_t stream) {
  BSQ_REQUIRE(tokens >= 0 && k >= 1 && k <= 64 && E >= 1 && E <= 1024, BSQ_E_SHAPE);
  BSQ_REQUIRE(tokens * k < (int64_t)1 << 31, BSQ_E_SHAPE);
  BSQ_REQUIRE(seg_offsets, BSQ_E_NULL);
  if (tokens > 0) BSQ_REQUIRE(topk_ids && row_index && pair_row, BSQ_E_NULL);
  BSQ_REQUIRE(bsq_route_workspace(tokens, E) <= kRouteScratchBytes, BSQ_E_WORKSPACE);
  void* counts = nullptr;
  const int st = scratch_ptr(&counts);
  if (st != BSQ_OK) return st;
  return route_launch(topk_ids, tokens, k, E, row_index, seg_offsets, pair_row, static_cast<int32_t*>(counts),
                      bsqh::as_stream(stream));
}

extern "C" const char* bsq_status_string(int status) {
  switch (status) {
    case BSQ_OK: return "ok";
    case BSQ_E_NULL: return "required pointer is NULL";
    case BSQ_E_SHAPE: return "invalid size or shape";
    case BSQ_E_ALIGN: return "pointer not sufficiently aligned";
    case BSQ_E_DTYPE: return "unknown element type";
    case BSQ_E_ENUM: return "unknown mode, rounding or format";
    case BSQ_E_WORKSPACE: return "workspace too small";
    case BSQ_E_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" int bsq_version(void) { return 100; }
