// Normalized update with stochastic rounding [page "Randomized Gradient
// Compression", section "How it works"]:
//
//   W <- SR_bf16(W - s * H),  H = C P^T,  s = tau * ||W||_F / ||H||_F
//
// H is never written to memory. Each wave rebuilds 16 rows x 64 columns of it
// at a time on MFMA (M = columns of W from rows of P, N = rows of W from rows
// of C, K = r), with C split into a bf16 high part and a bf16 remainder so that
// H carries ~16 bits of C's mantissa. The page rebuilds H 128 rows at a time;
// here the height is 64 rows per workgroup (the result does not depend on it).
//
// Two sweeps over W:
//   sweep 1 reads W and rebuilds H to get sum(w^2) and sum(h^2) (fp64 per lane,
//           fixed-order reductions across lanes and waves), one partial pair
//           per workgroup (at most a few hundred workgroups);
//   sweep 2 first sums those partials in a fixed order in every workgroup (all
//           get the identical s and skip flag, with no signalling between
//           workgroups), then reads W again, rebuilds the same H (same code,
//           same order), forms v = fp32(w - fp32(s*h)) and rounds
//           stochastically with 16 bits per element from Philox4x32-10 keyed
//           on (seed, row, column).
//
// Lane layout of a tile: M-tile t row m stands for column
// jb + 16*(m/4) + 4*t + (m%4), which gives lane (g = lane/16, n = lane%16) the
// 16 consecutive columns jb + 16g .. +15 of row ib + n, i.e. two 16-byte loads
// of W and two Philox calls (8 columns each) per lane per tile.
#include "rgc_internal.hpp"

namespace rgc {

enum ApplyMode { kModeNorms = 0, kModeUpdate = 1, kModeReconstruct = 2 };

constexpr int kApplyRowsPerWG = 64;  // 4 waves x 16 rows
constexpr int kApplyColsPerTile = 64;

// The C side of the tile product for the 16 rows a wave owns: K-step q holds
// C[i][32q + 8g .. +7] as bf16 high parts and bf16 remainders.
template <int R>
struct RowOperand {
  static constexpr int KQ = (R + 31) / 32;
  uint32_t hi[KQ][4];
  uint32_t lo[KQ][4];
};

template <int R>
__device__ __forceinline__ void load_row_operand(const float* __restrict__ C, int64_t d, int64_t i, int g,
                                                 RowOperand<R>& op) {
#pragma unroll
  for (int q = 0; q < RowOperand<R>::KQ; ++q) {
    const int c0 = 32 * q + 8 * g;
    float v[8];
    if (i < d && c0 < R) {
      const float4 a = *reinterpret_cast<const float4*>(C + i * R + c0);
      const float4 b = *reinterpret_cast<const float4*>(C + i * R + c0 + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t h0 = f32_to_bf16_rne(v[2 * p]), h1 = f32_to_bf16_rne(v[2 * p + 1]);
      const uint32_t l0 = f32_to_bf16_rne(v[2 * p] - bf16_bits_to_f32(h0));
      const uint32_t l1 = f32_to_bf16_rne(v[2 * p + 1] - bf16_bits_to_f32(h1));
      op.hi[q][p] = pack_bf16x2(h0, h1);
      op.lo[q][p] = pack_bf16x2(l0, l1);
    }
  }
}

// h[x] = H[ib + n][jb + 16g + x], x = 0..15, for this lane.
template <int R>
__device__ __forceinline__ void rebuild_tile(const uint16_t* __restrict__ P, int64_t k, int64_t jb,
                                             const RowOperand<R>& rop, int lane, float (&h)[16]) {
  const int m = lane & 15, g = lane >> 4;
  f32x4_t acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t j = jb + 16 * (m >> 2) + 4 * t + (m & 3);
#pragma unroll
    for (int q = 0; q < RowOperand<R>::KQ; ++q) {
      const int c0 = 32 * q + 8 * g;
      uint32_t a[4] = {0u, 0u, 0u, 0u};
      if (j < k && c0 < R) {
        const uint4 v = *reinterpret_cast<const uint4*>(P + j * R + c0);
        a[0] = v.x; a[1] = v.y; a[2] = v.z; a[3] = v.w;
      }
      acc[t] = mfma_16x16x32(a, rop.hi[q], acc[t]);
      acc[t] = mfma_16x16x32(a, rop.lo[q], acc[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) h[4 * t + e] = acc[t][e];
}

__device__ __forceinline__ void load_w16(const uint16_t* p, uint32_t (&w)[8]) {
  const uint4 a = reinterpret_cast<const uint4*>(p)[0];
  const uint4 b = reinterpret_cast<const uint4*>(p)[1];
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

// Rounding bits for row i, columns 8*cb .. 8*cb+7: word (x/2), low half for
// even x.
__device__ __forceinline__ void rounding_words(uint64_t seed, int64_t i, int64_t cb, uint32_t (&words)[4]) {
  u32x4 c = {(uint32_t)cb, (uint32_t)i, kTagRounding, 0u};
  const u32x4 o = philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  words[0] = o.x; words[1] = o.y; words[2] = o.z; words[3] = o.w;
}

// Fixed-order sum of sweep 1's partials (thread t holds partials t, t+256, ...
// in order; then a butterfly within each wave and the waves in order), and the
// step s = fp32(tau * ||W|| / ||H||); flag = 1 when ||H|| is zero or not finite
// or s is not finite (then s = 0).
__device__ __forceinline__ void step_from_partials(const double* __restrict__ partials, int nparts, float tau, int wave,
                                                   int lane, float& s, uint32_t& flag, double& nw, double& nh) {
  __shared__ double red[2][4];
  double aw = 0.0, ah = 0.0;
  for (int b = threadIdx.x; b < nparts; b += blockDim.x) {
    aw += partials[2 * b];
    ah += partials[2 * b + 1];
  }
  aw = wave_sum(aw);
  ah = wave_sum(ah);
  if (lane == 0) {
    red[0][wave] = aw;
    red[1][wave] = ah;
  }
  __syncthreads();
  const double tw = ((red[0][0] + red[0][1]) + red[0][2]) + red[0][3];
  const double th = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];
  nw = sqrt(tw);
  nh = sqrt(th);
  s = 0.f;
  flag = 0u;
  if (!(nh > 0.0) || !isfinite(nh)) {
    flag = 1u;
  } else {
    s = (float)((double)tau * nw / nh);
    if (!isfinite(s)) {
      s = 0.f;
      flag = 1u;
    }
  }
}

template <int R, int MODE>
__global__ __launch_bounds__(256) void apply_kernel(uint16_t* __restrict__ W, int64_t ldw, const float* __restrict__ C,
                                                    const uint16_t* __restrict__ P, int64_t d, int64_t k,
                                                    int tiles_per_wg, float tau, uint64_t seed,
                                                    float* __restrict__ stats, double* __restrict__ partials,
                                                    int nparts, float* __restrict__ Hout) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int64_t i = (int64_t)blockIdx.x * kApplyRowsPerWG + 16 * wave + n;
  const int64_t col_tiles = (k + kApplyColsPerTile - 1) / kApplyColsPerTile;
  const int64_t tile0 = (int64_t)blockIdx.y * tiles_per_wg;

  float s = 0.f;
  if constexpr (MODE == kModeUpdate) {
    // Every workgroup sums sweep 1's partials in the same fixed order, so all
    // compute the identical step s; workgroup 0 reports it.
    uint32_t flag;
    double nw, nh;
    step_from_partials(partials, nparts, tau, wave, lane, s, flag, nw, nh);
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0 && stats) {
      stats[0] = (float)nw;
      stats[1] = (float)nh;
      stats[2] = s;
      stats[3] = (float)flag;
    }
    if (flag) return;  // zero or non-finite step: leave W untouched
  }

  RowOperand<R> rop;
  load_row_operand<R>(C, d, i, g, rop);

  double sw = 0.0, sh = 0.0;
  for (int tt = 0; tt < tiles_per_wg; ++tt) {
    const int64_t tile = tile0 + tt;
    if (tile >= col_tiles) break;
    const int64_t jb = tile * kApplyColsPerTile;
    float h[16];
    rebuild_tile<R>(P, k, jb, rop, lane, h);
    const int64_t j0 = jb + 16 * g;
    if (i >= d) continue;
    if constexpr (MODE == kModeReconstruct) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if (j0 + 8 * half >= k) continue;
        float4* dst = reinterpret_cast<float4*>(Hout + i * k + j0 + 8 * half);
        dst[0] = make_float4(h[8 * half + 0], h[8 * half + 1], h[8 * half + 2], h[8 * half + 3]);
        dst[1] = make_float4(h[8 * half + 4], h[8 * half + 5], h[8 * half + 6], h[8 * half + 7]);
      }
    } else if constexpr (MODE == kModeNorms) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if (j0 + 8 * half >= k) continue;
        const uint4 wv = *reinterpret_cast<const uint4*>(W + i * ldw + j0 + 8 * half);
        const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const double w0 = (double)bf16_bits_to_f32(wd[p] & 0xFFFFu);
          const double w1 = (double)bf16_bits_to_f32(wd[p] >> 16);
          const double h0 = (double)h[8 * half + 2 * p], h1 = (double)h[8 * half + 2 * p + 1];
          sw += w0 * w0 + w1 * w1;
          sh += h0 * h0 + h1 * h1;
        }
      }
    } else {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int64_t jj = j0 + 8 * half;
        if (jj >= k) continue;
        uint4* wp = reinterpret_cast<uint4*>(W + i * ldw + jj);
        const uint4 wv = *wp;
        const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
        uint32_t rw[4];
        rounding_words(seed, i, jj >> 3, rw);
        uint32_t out[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float w0 = bf16_bits_to_f32(wd[p] & 0xFFFFu), w1 = bf16_bits_to_f32(wd[p] >> 16);
          const float sh0 = s * h[8 * half + 2 * p], sh1 = s * h[8 * half + 2 * p + 1];
          const float v0 = w0 - sh0, v1 = w1 - sh1;
          out[p] = pack_bf16x2(f32_to_bf16_sr(v0, rw[p] & 0xFFFFu), f32_to_bf16_sr(v1, rw[p] >> 16));
        }
        *wp = make_uint4(out[0], out[1], out[2], out[3]);
      }
    }
  }

  if constexpr (MODE == kModeNorms) {
    __shared__ double red[2][4];
    sw = wave_sum(sw);
    sh = wave_sum(sh);
    if (lane == 0) {
      red[0][wave] = sw;
      red[1][wave] = sh;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      const int64_t bid = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
      partials[2 * bid] = ((red[0][0] + red[0][1]) + red[0][2]) + red[0][3];
      partials[2 * bid + 1] = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];
    }
  }
}

// ---------------------------------------------------------------------------
// Test hooks: the rounding stream and the Philox generator alone.
// ---------------------------------------------------------------------------
__global__ void stochastic_round_kernel(const float* __restrict__ v, uint16_t* __restrict__ out, int64_t rows,
                                        int64_t cols, int64_t ld, int64_t row0, int64_t col0, uint64_t seed) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * cols) return;
  const int64_t i = idx / cols, j = idx % cols;
  const int64_t I = row0 + i, J = col0 + j;
  uint32_t words[4];
  rounding_words(seed, I, J >> 3, words);
  const uint32_t w = words[(J & 7) >> 1];
  const uint32_t r16 = (J & 1) ? (w >> 16) : (w & 0xFFFFu);
  out[i * ld + j] = (uint16_t)f32_to_bf16_sr(v[i * ld + j], r16);
}

__global__ void philox_kernel(uint64_t seed, int64_t n, const uint32_t* __restrict__ ctr, uint32_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  u32x4 c = {ctr[4 * idx], ctr[4 * idx + 1], ctr[4 * idx + 2], ctr[4 * idx + 3]};
  const u32x4 o = philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  out[4 * idx] = o.x;
  out[4 * idx + 1] = o.y;
  out[4 * idx + 2] = o.z;
  out[4 * idx + 3] = o.w;
}

namespace {

struct ApplyPlan {
  int64_t row_blocks, col_tiles;
  int tiles_per_wg;
  int64_t col_groups;
};

// Grid over (64-row blocks) x (groups of 64-column tiles) with at most
// `target` workgroups.
ApplyPlan apply_plan(int64_t d, int64_t k, int64_t target) {
  ApplyPlan p;
  p.row_blocks = (d + kApplyRowsPerWG - 1) / kApplyRowsPerWG;
  p.col_tiles = (k + kApplyColsPerTile - 1) / kApplyColsPerTile;
  int64_t tpw = (p.row_blocks * p.col_tiles + target - 1) / target;
  if (tpw < 1) tpw = 1;
  if (tpw > p.col_tiles) tpw = p.col_tiles;
  p.tiles_per_wg = (int)tpw;
  p.col_groups = (p.col_tiles + tpw - 1) / tpw;
  return p;
}
// Sweep 1 writes one partial per workgroup and every sweep-2 workgroup reads
// them all, so sweep 1's grid stays small; sweep 2's is sized for the chip.
ApplyPlan norms_plan(int64_t d, int64_t k) { return apply_plan(d, k, env_int("RGC_NORM_WGS", 256)); }
ApplyPlan update_plan(int64_t d, int64_t k) { return apply_plan(d, k, env_int("RGC_APPLY_WGS", 1024)); }

size_t apply_ws(int64_t d, int64_t k) {
  const ApplyPlan p = norms_plan(d, k);
  return (size_t)p.row_blocks * p.col_groups * 2 * sizeof(double);
}

template <int R>
rgc_status_t apply_launch(uint16_t* W, int64_t ldw, const float* C, const uint16_t* P, int64_t d, int64_t k,
                          float tau, uint64_t seed, float* stats, void* ws, hipStream_t s) {
  const ApplyPlan p1 = norms_plan(d, k), p2 = update_plan(d, k);
  double* partials = static_cast<double*>(ws);
  const int nparts = (int)(p1.row_blocks * p1.col_groups);
  hipLaunchKernelGGL((apply_kernel<R, kModeNorms>), dim3((unsigned)p1.row_blocks, (unsigned)p1.col_groups), dim3(256),
                     0, s, W, ldw, C, P, d, k, p1.tiles_per_wg, tau, seed, nullptr, partials, nparts, nullptr);
  hipLaunchKernelGGL((apply_kernel<R, kModeUpdate>), dim3((unsigned)p2.row_blocks, (unsigned)p2.col_groups), dim3(256),
                     0, s, W, ldw, C, P, d, k, p2.tiles_per_wg, tau, seed, stats, partials, nparts, nullptr);
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

template <int R>
rgc_status_t reconstruct_launch(const float* C, const uint16_t* P, float* H, int64_t d, int64_t k, hipStream_t s) {
  const ApplyPlan p = update_plan(d, k);
  dim3 grid((unsigned)p.row_blocks, (unsigned)p.col_groups);
  hipLaunchKernelGGL((apply_kernel<R, kModeReconstruct>), grid, dim3(256), 0, s, nullptr, k, C, P, d, k,
                     p.tiles_per_wg, 0.f, 0ull, nullptr, nullptr, 0, H);
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

}  // namespace
}  // namespace rgc

using namespace rgc;

extern "C" size_t rgc_apply_workspace_size(int64_t d, int64_t k, int64_t r) {
  if (d <= 0 || k <= 0 || !rank_supported(r)) return 0;
  return apply_ws(d, k);
}

extern "C" rgc_status_t rgc_apply(uint16_t* W, int64_t ldw, const float* C, const uint16_t* P, int64_t d, int64_t k,
                                  int64_t r, float tau, uint64_t seed, float* stats, void* ws, size_t ws_bytes,
                                  void* stream) {
  if (d <= 0 || k <= 0 || r <= 0 || r > k || ldw < k) return RGC_ERR_SHAPE;
  if (!rank_supported(r) || (d % 8) != 0 || (k % 8) != 0) return RGC_ERR_UNSUPPORTED;
  if (!W || !C || !P) return RGC_ERR_NULL;
  if (!aligned16(W) || !aligned16(C) || !aligned16(P) || (ldw % 8) != 0) return RGC_ERR_ALIGN;
  if (stats && !aligned_to(stats, 4)) return RGC_ERR_ALIGN;
  const size_t need = apply_ws(d, k);
  if (!ws || ws_bytes < need) return RGC_ERR_WORKSPACE;
  if (!aligned_to(ws, 256)) return RGC_ERR_ALIGN;
  rgc_status_t st = RGC_OK;
  dispatch_rank(r, [&](auto rc) {
    st = apply_launch<decltype(rc)::value>(W, ldw, C, P, d, k, tau, seed, stats, ws, static_cast<hipStream_t>(stream));
  });
  return st;
}

extern "C" rgc_status_t rgc_test_reconstruct(const float* C, const uint16_t* P, float* H, int64_t d, int64_t k,
                                             int64_t r, void* stream) {
  if (d <= 0 || k <= 0 || r <= 0 || r > k) return RGC_ERR_SHAPE;
  if (!rank_supported(r) || (d % 8) != 0 || (k % 8) != 0) return RGC_ERR_UNSUPPORTED;
  if (!C || !P || !H) return RGC_ERR_NULL;
  if (!aligned16(C) || !aligned16(P) || !aligned16(H)) return RGC_ERR_ALIGN;
  rgc_status_t st = RGC_OK;
  dispatch_rank(r, [&](auto rc) {
    st = reconstruct_launch<decltype(rc)::value>(C, P, H, d, k, static_cast<hipStream_t>(stream));
  });
  return st;
}

extern "C" rgc_status_t rgc_test_stochastic_round(const float* v, uint16_t* out, int64_t rows, int64_t cols,
                                                  int64_t ld, int64_t row0, int64_t col0, uint64_t seed,
                                                  void* stream) {
  if (rows < 0 || cols < 0 || ld < cols || row0 < 0 || col0 < 0) return RGC_ERR_SHAPE;
  if (rows == 0 || cols == 0) return RGC_OK;
  if (!v || !out) return RGC_ERR_NULL;
  if (!aligned_to(v, 4) || !aligned_to(out, 2)) return RGC_ERR_ALIGN;
  const int64_t nel = rows * cols;
  hipLaunchKernelGGL(stochastic_round_kernel, dim3((unsigned)((nel + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), v, out, rows, cols, ld, row0, col0, seed);
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

extern "C" rgc_status_t rgc_test_philox(uint64_t seed, int64_t n, const uint32_t* ctr, uint32_t* out, void* stream) {
  if (n < 0) return RGC_ERR_SHAPE;
  if (n == 0) return RGC_OK;
  if (!ctr || !out) return RGC_ERR_NULL;
  if (!aligned_to(ctr, 4) || !aligned_to(out, 4)) return RGC_ERR_ALIGN;
  hipLaunchKernelGGL(philox_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     seed, n, ctr, out);
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}
