// Host/device internals of the sketch library: rank-dependent tiling traits,
// the compile-time dispatch over supported ranks, and argument checks.
#pragma once

#include <stdint.h>
#include <stdlib.h>

#include <atomic>
#include <type_traits>

#include <hip/hip_runtime.h>

#include "../../include/rgc.h"
#include "rgc_device.hpp"

namespace rgc {

// Per-call limit on the tiled dimension (tokens for project, d for
// accumulate); keeps every in-kernel offset within 32 bits.
constexpr int64_t kMaxTiledDim = 65536;

// Limit on the leading dimension of X and D: the kernels address a tile of
// up to 256 rows (project) or a 32-row window (accumulate) with 32-bit
// per-lane byte offsets, so 256 * 2^23 * 2 bytes must fit in 32 bits.
constexpr int64_t kMaxLeadingDim = int64_t(1) << 23;

// Bytes of the static device scratch behind rgc_apply_noalloc.
constexpr size_t kNoAllocScratchBytes = RGC_NOALLOC_SCRATCH_BYTES;

// Ranks of the MFMA-tiled kernels: every multiple of 16 up to 256.
inline bool rank_tiled(int64_t r) { return r >= 16 && r <= 256 && r % 16 == 0; }

// Ranks below one MFMA tile (4 and 8) take the small-rank kernels.
inline bool rank_small(int64_t r) { return r == 4 || r == 8; }

inline bool rank_supported(int64_t r) { return rank_tiled(r) || rank_small(r); }

template <int V>
using IntC = std::integral_constant<int, V>;

// Calls f(IntC<i>{}) for i = B .. E-1 (a loop whose index is a constant expression).
template <int B, int E, typename F>
__host__ __device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(IntC<B>{});
    static_for<B + 1, E>(f);
  }
}

// Calls f(IntC<r>{}) for a tiled rank (a multiple of 16 up to 256); returns
// false otherwise.
template <typename F>
bool dispatch_rank(int64_t r, F&& f) {
  bool done = false;
  static_for<1, 17>([&](auto q) {
    constexpr int R = 16 * decltype(q)::value;
    if (r == R) {
      f(IntC<R>{});
      done = true;
    }
  });
  return done;
}

// Calls f(IntC<r>{}) for a small rank (4 or 8); returns false otherwise.
template <typename F>
bool dispatch_small_rank(int64_t r, F&& f) {
  if (r == 4) f(IntC<4>{});
  else if (r == 8) f(IntC<8>{});
  else return false;
  return true;
}

inline bool aligned_to(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }
inline bool aligned16(const void* p) { return aligned_to(p, 16); }

// Compute units of the current device (cached per device; 256 if unknown).
inline int device_compute_units() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  static std::atomic<int> cache[64];
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

}  // namespace rgc
