// Host-side helpers of the C ABI: argument validation and launch checks.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/bsq.h"

namespace bsqh {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline hipStream_t as_stream(bsq_stream_t s) { return reinterpret_cast<hipStream_t>(s); }
inline int launch_status() { return hipGetLastError() == hipSuccess ? BSQ_OK : BSQ_E_LAUNCH; }

// Upper bound on the number of row tiles of height `tile` over `num_segments`
// segments holding `total_rows` rows in all (each segment wastes at most one
// partial tile).
inline int64_t tile_bound(int64_t total_rows, int64_t num_segments, int64_t tile) {
  return (total_rows + tile - 1) / tile + num_segments;
}

// Compute units of the current device (persistent kernels launch one
// workgroup per CU); 256 if the query fails. The per-device cache is atomic:
// threads calling concurrently may each query once and store the same value.
inline int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace bsqh

#define BSQ_REQUIRE(cond, err) \
  do {                         \
    if (!(cond)) return (err); \
  } while (0)
