// Version and status strings of the C ABI, and the composite entry point that
// applies a received sketch from its projection seed (host only: it enqueues
// the projection sampling and the update through the library's own calls).
#include <stdint.h>

#include "../../include/rgc.h"

extern "C" int rgc_abi_version(void) { return RGC_ABI_VERSION; }

extern "C" const char* rgc_status_string(rgc_status_t status) {
  switch (status) {
    case RGC_OK: return "ok";
    case RGC_ERR_NULL: return "a required pointer is NULL";
    case RGC_ERR_SHAPE: return "invalid shape (negative size, r > k or leading dimension < width)";
    case RGC_ERR_UNSUPPORTED: return "unsupported shape (rank, width multiple or size limit)";
    case RGC_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case RGC_ERR_WORKSPACE: return "workspace missing or too small";
    case RGC_ERR_HIP: return "HIP kernel launch failed";
    case RGC_ERR_VALUE: return "a scalar argument is not finite";
    case RGC_ERR_SCRATCH: return "the call needs more scratch than the library's static buffer holds";
  }
  return "unknown status";
}

namespace rgc {
// Host-side argument checks of the sampling and of the update (defined next
// to those calls); they launch nothing.
rgc_status_t sample_validate(rgc_proj_kind_t kind, int64_t k, int64_t r, const uint16_t* P);
rgc_status_t apply_validate(const uint16_t* W, int64_t ldw, const float* C, const uint16_t* P, int64_t d, int64_t k,
                            int64_t r, bool scaled, float step, const float* stats);
}  // namespace rgc

namespace {

size_t round_up_256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of rgc_apply_from_seed: the regenerated P (k x r bf16), then one
// region that serves the sampling and, after it, the update (the two run in
// that order on the caller's stream, so the sampling scratch is dead when
// the update starts).
size_t projection_bytes(int64_t k, int64_t r) { return round_up_256((size_t)k * (size_t)r * 2); }

size_t shared_scratch_bytes(rgc_proj_kind_t kind, int64_t d, int64_t k, int64_t r) {
  const size_t a = rgc_sample_projection_workspace_size(kind, k, r);
  const size_t b = rgc_apply_workspace_size(d, k, r);
  return a > b ? a : b;
}

}  // namespace

// 0 when the combination is not supported (the regenerated P always needs room).
extern "C" size_t rgc_apply_from_seed_workspace_size(rgc_proj_kind_t kind, int64_t d, int64_t k, int64_t r) {
  if (d <= 0 || k <= 0 || r <= 0 || r > k) return 0;
  if (kind == RGC_PROJ_QR_GAUSSIAN && rgc_sample_projection_workspace_size(kind, k, r) == 0) return 0;
  if (kind != RGC_PROJ_QR_GAUSSIAN && kind != RGC_PROJ_RADEMACHER) return 0;
  if (rgc_apply_workspace_size(d, k, r) == 0) return 0;
  return projection_bytes(k, r) + shared_scratch_bytes(kind, d, k, r);
}

extern "C" rgc_status_t rgc_apply_from_seed(rgc_update_mode_t mode, rgc_proj_kind_t kind, uint64_t proj_seed,
                                            uint16_t* W, int64_t ldw, const float* C, int64_t d, int64_t k,
                                            int64_t r, float step, uint64_t seed, float* stats, void* ws,
                                            size_t ws_bytes, void* stream) {
  if (mode != RGC_UPDATE_NORMALIZED && mode != RGC_UPDATE_SCALED) return RGC_ERR_UNSUPPORTED;
  if (mode == RGC_UPDATE_SCALED && stats) return RGC_ERR_UNSUPPORTED;
  if (d <= 0 || k <= 0 || r <= 0 || r > k || ldw < k) return RGC_ERR_SHAPE;
  if (!ws) return RGC_ERR_WORKSPACE;
  if (((uintptr_t)ws % 256) != 0) return RGC_ERR_ALIGN;
  const size_t need = rgc_apply_from_seed_workspace_size(kind, d, k, r);
  if (need == 0) return RGC_ERR_UNSUPPORTED;
  if (ws_bytes < need) return RGC_ERR_WORKSPACE;
  uint16_t* P = static_cast<uint16_t*>(ws);
  char* scratch = static_cast<char*>(ws) + projection_bytes(k, r);
  const size_t scratch_bytes = ws_bytes - projection_bytes(k, r);
  // Validate both steps before the sampling is enqueued, so that an error
  // leaves nothing launched.
  rgc_status_t st = rgc::sample_validate(kind, k, r, P);
  if (st != RGC_OK) return st;
  st = rgc::apply_validate(W, ldw, C, P, d, k, r, mode == RGC_UPDATE_SCALED, step, stats);
  if (st != RGC_OK) return st;
  st = rgc_sample_projection(kind, proj_seed, k, r, P, scratch, scratch_bytes, stream);
  if (st != RGC_OK) return st;
  if (mode == RGC_UPDATE_SCALED) return rgc_apply_scaled(W, ldw, C, P, d, k, r, step, seed, stream);
  return rgc_apply(W, ldw, C, P, d, k, r, step, seed, stats, scratch, scratch_bytes, stream);
}
