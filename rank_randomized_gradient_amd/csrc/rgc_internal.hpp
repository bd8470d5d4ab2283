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

// Limit on the leading dimension of X and D: the kernels address a 64-token
// (or 32-token) slab of rows with 32-bit byte offsets.
constexpr int64_t kMaxLeadingDim = int64_t(1) << 24;

// Tiling of the rank dimension r (a multiple of 16, at most 64, or a multiple
// of 64 up to 256). A wave covers RPW rank columns in NG groups of GW columns;
// each lane reads CPL adjacent columns per row of a group (CPL = 4 when the
// group is 64 wide). NR waves cover all of r; KS waves split the K loop
// inside a workgroup so that it has four waves when r is small.
template <int R>
struct RankTraits {
  static_assert(R % 16 == 0 && R >= 16 && R <= 256, "rank");
  static constexpr int CPL = (R % 64 == 0) ? 4 : ((R % 32 == 0) ? 2 : 1);
  static constexpr int RPW = (R <= 64) ? R : 64;
  static constexpr int NR = R / RPW;
  static constexpr int GW = 16 * CPL;
  static constexpr int NG = RPW / GW;
  static constexpr int MT = RPW / 16;
  static constexpr int KS = (NR == 1) ? 4 : (NR == 2 ? 2 : 1);
  static_assert(RPW % GW == 0 && R % RPW == 0, "rank tiling");
};

inline bool rank_supported(int64_t r) {
  return r == 16 || r == 32 || r == 48 || r == 64 || r == 128 || r == 192 || r == 256;
}

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

// Calls f(IntC<r>{}) for a supported rank; returns false otherwise.
template <typename F>
bool dispatch_rank(int64_t r, F&& f) {
  switch (r) {
    case 16: f(IntC<16>{}); return true;
    case 32: f(IntC<32>{}); return true;
    case 48: f(IntC<48>{}); return true;
    case 64: f(IntC<64>{}); return true;
    case 128: f(IntC<128>{}); return true;
    case 192: f(IntC<192>{}); return true;
    case 256: f(IntC<256>{}); return true;
    default: return false;
  }
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

inline int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  int x = atoi(v);
  return x > 0 ? x : dflt;
}

}  // namespace rgc
