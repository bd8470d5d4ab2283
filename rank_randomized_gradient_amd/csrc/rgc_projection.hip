// Seeded projection P (k x r, bf16), regenerated from a 64-bit seed so that it
// never has to be stored or sent ([page "LoGRA: Low-Rank Gradient Sketches",
// "Why Refreshing the Projection Enables New Update Directions"]).
//
// Rademacher [same page, "Why the Sketch Can Be Accumulated Without a Full
// Gradient"]: entries +-1/sqrt(r) from Philox sign bits.
//
// QR of a Gaussian [page "Randomized Gradient Compression", footnote 1]:
// P = sqrt(k/r) Q with Q the sign-corrected (diag R > 0) thin QR factor of a
// Gaussian k x r matrix. Q is computed by CholeskyQR2 in fp64:
//   A  = Box-Muller normals from Philox                  (gram pass 1 writes A)
//   R1 = chol(A^T A),   Q1 = A R1^-1                      (reduce+factor, trmul)
//   R2 = chol(Q1^T Q1), Q  = Q1 R2^-1                     (gram, reduce+factor, trmul)
// Cholesky factors have a positive diagonal, so Q is the unique factor with
// the standard sign correction; the second pass restores orthogonality to
// fp64 accuracy. The Gram matrices are summed from per-workgroup partials in a
// fixed order, so P is bit-reproducible.
#include <math.h>
#include <string.h>

#include "rgc_internal.hpp"

namespace rgc {

// ---------------------------------------------------------------------------
// Rademacher: one thread per (row, 8 columns).
// ---------------------------------------------------------------------------
__global__ void rademacher_kernel(uint16_t* __restrict__ P, int64_t k, int r, uint64_t seed, uint32_t mag) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int groups = r / 8;
  if (idx >= k * groups) return;
  const int64_t i = idx / groups;
  const int j0 = (int)(idx % groups) * 8;
  u32x4 c = {(uint32_t)i, (uint32_t)(j0 >> 7), kTagRademacher, 0u};
  const u32x4 o = philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  const uint32_t words[4] = {o.x, o.y, o.z, o.w};
  uint32_t out[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t hv[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = j0 + 2 * p + e;
      const uint32_t bit = (words[(j >> 5) & 3] >> (j & 31)) & 1u;
      hv[e] = bit ? (mag | 0x8000u) : mag;
    }
    out[p] = pack_bf16x2(hv[0], hv[1]);
  }
  *reinterpret_cast<uint4*>(P + i * r + j0) = make_uint4(out[0], out[1], out[2], out[3]);
}

// ---------------------------------------------------------------------------
// CholeskyQR2 pieces. R is the rank (<= 128), templated for register tiles.
// ---------------------------------------------------------------------------
constexpr int kQrRowsPerChunk = 16;
constexpr double kTwoPi = 6.283185307179586;  // 2*pi rounded to double

// Normal draws for row i, columns 4q .. 4q+3 (Box-Muller on Philox words).
__device__ __forceinline__ void gaussian4(uint64_t seed, int64_t i, int q, double (&z)[4]) {
  u32x4 c = {(uint32_t)i, (uint32_t)q, kTagGaussian, 0u};
  const u32x4 o = philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  const uint32_t w[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
  for (int pr = 0; pr < 2; ++pr) {
    const double u1 = ((double)w[2 * pr] + 0.5) * 0x1p-32;
    const double u2 = ((double)w[2 * pr + 1] + 0.5) * 0x1p-32;
    const double rho = sqrt(-2.0 * log(u1));
    const double theta = kTwoPi * u2;
    z[2 * pr] = rho * cos(theta);
    z[2 * pr + 1] = rho * sin(theta);
  }
}

// Gram partials: block b sums rows [b*rows_per_block, ...) of M^T M into
// partial[b] (R x R, fp64). GEN: M is drawn here (and stored to M);
// otherwise M is read.
template <int R, bool GEN>
__global__ __launch_bounds__(256) void gram_kernel(double* __restrict__ M, int64_t k, int64_t rows_per_block,
                                                   uint64_t seed, double* __restrict__ partial) {
  constexpr int TU = R / 16;  // each thread owns a TU x TU sub-tile
  __shared__ double rows[kQrRowsPerChunk][R];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  double acc[TU][TU];
#pragma unroll
  for (int u = 0; u < TU; ++u)
#pragma unroll
    for (int v = 0; v < TU; ++v) acc[u][v] = 0.0;
  const int64_t rbeg = (int64_t)blockIdx.x * rows_per_block;
  const int64_t rend = rbeg + rows_per_block < k ? rbeg + rows_per_block : k;
  for (int64_t r0 = rbeg; r0 < rend; r0 += kQrRowsPerChunk) {
    __syncthreads();
    if constexpr (GEN) {
      // kQrRowsPerChunk x R/4 Philox calls for this chunk
      for (int t = threadIdx.x; t < kQrRowsPerChunk * (R / 4); t += blockDim.x) {
        const int lr = t / (R / 4), q = t % (R / 4);
        const int64_t row = r0 + lr;
        double z[4] = {0.0, 0.0, 0.0, 0.0};
        if (row < rend) {
          gaussian4(seed, row, q, z);
#pragma unroll
          for (int e = 0; e < 4; ++e) M[row * R + 4 * q + e] = z[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) rows[lr][4 * q + e] = z[e];
      }
    } else {
      for (int t = threadIdx.x; t < kQrRowsPerChunk * R; t += blockDim.x) {
        const int lr = t / R, c = t % R;
        const int64_t row = r0 + lr;
        rows[lr][c] = row < rend ? M[row * R + c] : 0.0;
      }
    }
    __syncthreads();
#pragma unroll 4
    for (int lr = 0; lr < kQrRowsPerChunk; ++lr) {
      double a[TU], b[TU];
#pragma unroll
      for (int u = 0; u < TU; ++u) a[u] = rows[lr][ty + 16 * u];
#pragma unroll
      for (int v = 0; v < TU; ++v) b[v] = rows[lr][tx + 16 * v];
#pragma unroll
      for (int u = 0; u < TU; ++u)
#pragma unroll
        for (int v = 0; v < TU; ++v) acc[u][v] += a[u] * b[v];
    }
  }
  double* out = partial + (int64_t)blockIdx.x * R * R;
#pragma unroll
  for (int u = 0; u < TU; ++u)
#pragma unroll
    for (int v = 0; v < TU; ++v) out[(ty + 16 * u) * R + tx + 16 * v] = acc[u][v];
}

// Sums the Gram partials in block order (each block a slice of the R x R
// entries); the last block to finish writes U = R^-1 for the upper Cholesky
// factor R of G (G = R^T R, diag R > 0), upper triangular with zeros below.
//
// U comes from one Gaussian elimination of [G | I] without pivoting (stable
// for symmetric positive definite G): with G = L D L^T (L unit lower), the
// eliminated left block is D L^T and the right block is L^-1, so
// R = D^1/2 L^T and R^-1 = L^-T D^-1/2. The symmetric Schur complement is
// kept in g's upper triangle and L^-1 (unit diagonal implied) in its strictly
// lower triangle; each column costs one barrier.
template <int R>
__global__ __launch_bounds__(256) void reduce_factor_kernel(const double* __restrict__ partial, int nparts,
                                                            double* __restrict__ G, double* __restrict__ U,
                                                            uint32_t* __restrict__ counter,
                                                            uint32_t* __restrict__ status) {
  __shared__ double g[R][R + 1];  // +1 pads rows off the same banks
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + tid;
  if (e < (int64_t)R * R) {
    double s = 0.0;
    for (int p = 0; p < nparts; ++p) s += partial[(int64_t)p * R * R + e];
    G[e] = s;
  }
  if (!arrive_last(counter, gridDim.x - 1)) return;
  for (int a = ty; a < R; a += 16)
    for (int c = tx; c < R; c += 16) g[a][c] = (c >= a) ? G[a * R + c] : 0.0;
  __syncthreads();

  for (int j = 0; j < R; ++j) {
    const double piv = g[j][j];
    for (int l = j + 1 + ty; l < R; l += 16) {
      const double f = g[j][l] / piv;  // G(l, j) / G(j, j), using the symmetric upper copy
      for (int m = l + tx; m < R; m += 16) g[l][m] -= f * g[j][m];
      for (int c = tx; c < j; c += 16) g[l][c] -= f * g[j][c];
      if (tx == 0) g[l][j] = -f;  // E(l, j) = 0 - f * E(j, j)
    }
    __syncthreads();
  }
  if (tid == 0) {
    bool ok = true;
    for (int j = 0; j < R; ++j) ok = ok && (g[j][j] > 0.0) && isfinite(g[j][j]);
    *status = ok ? 0u : 1u;
  }
  for (int a = ty; a < R; a += 16)
    for (int c = tx; c < R; c += 16) {
      const double rs = 1.0 / sqrt(g[c][c]);
      double v = 0.0;
      if (c == a) v = rs;
      else if (c > a) v = g[c][a] * rs;
      U[a * R + c] = v;
    }
  if (tid == 0) *counter = 0u;
}

// Y = M U for U upper triangular (R x R). FINAL: P = bf16(fp32(scale * Y)),
// else Y is written in fp64.
template <int R, bool FINAL>
__global__ __launch_bounds__(256) void trmul_kernel(const double* __restrict__ M, const double* __restrict__ U,
                                                    int64_t k, int64_t rows_per_block, double scale,
                                                    double* __restrict__ Y, uint16_t* __restrict__ P) {
  constexpr int TU = R / 16;
  __shared__ double u[R][R];
  __shared__ double rows[kQrRowsPerChunk][R + 1];  // +1: rows read by different lanes sit on different banks
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  for (int t = threadIdx.x; t < R * R; t += blockDim.x) u[t / R][t % R] = U[t];
  const int64_t rbeg = (int64_t)blockIdx.x * rows_per_block;
  const int64_t rend = rbeg + rows_per_block < k ? rbeg + rows_per_block : k;
  for (int64_t r0 = rbeg; r0 < rend; r0 += kQrRowsPerChunk) {
    __syncthreads();
    for (int t = threadIdx.x; t < kQrRowsPerChunk * R; t += blockDim.x) {
      const int lr = t / R, c = t % R;
      const int64_t row = r0 + lr;
      rows[lr][c] = row < rend ? M[row * R + c] : 0.0;
    }
    __syncthreads();
    // thread (tx, ty): row r0 + ty, columns tx + 16 v
    const int64_t row = r0 + ty;
    double y[TU];
#pragma unroll
    for (int v = 0; v < TU; ++v) y[v] = 0.0;
    for (int a = 0; a < R; ++a) {
      const double ma = rows[ty][a];
#pragma unroll
      for (int v = 0; v < TU; ++v) {
        const int c = tx + 16 * v;
        if (a <= c) y[v] += ma * u[a][c];
      }
    }
    if (row < rend) {
#pragma unroll
      for (int v = 0; v < TU; ++v) {
        const int c = tx + 16 * v;
        if constexpr (FINAL) {
          const float f = (float)(scale * y[v]);
          P[row * R + c] = (uint16_t)f32_to_bf16_rne(f);
        } else {
          Y[row * R + c] = y[v];
        }
      }
    }
  }
}

namespace {

struct QrPlan {
  int64_t rows_per_block;
  int blocks;
};

QrPlan qr_plan(int64_t k, int64_t r) {
  QrPlan p;
  // about 2K fp64 multiply-adds per thread in the Gram pass, 8..128 blocks
  int64_t target = (k * r * r + 256 * 2048 - 1) / (256 * 2048);
  if (target < 8) target = 8;
  if (target > 128) target = 128;
  int64_t rpb = (k + target - 1) / target;
  rpb = ((rpb + kQrRowsPerChunk - 1) / kQrRowsPerChunk) * kQrRowsPerChunk;
  if (rpb < kQrRowsPerChunk) rpb = kQrRowsPerChunk;
  p.rows_per_block = rpb;
  p.blocks = (int)((k + rpb - 1) / rpb);
  return p;
}

struct QrLayout {
  size_t a, q1, partial, g, u1, u2, status, total;
};

QrLayout qr_layout(int64_t k, int64_t r) {
  const QrPlan p = qr_plan(k, r);
  QrLayout l;
  size_t off = kCounterBytes;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += (bytes + 255) / 256 * 256;
    return at;
  };
  l.a = take((size_t)k * r * sizeof(double));
  l.q1 = take((size_t)k * r * sizeof(double));
  l.partial = take((size_t)p.blocks * r * r * sizeof(double));
  l.g = take((size_t)r * r * sizeof(double));
  l.u1 = take((size_t)r * r * sizeof(double));
  l.u2 = take((size_t)r * r * sizeof(double));
  l.status = take(256);
  l.total = off;
  return l;
}

template <int R>
rgc_status_t qr_launch(uint64_t seed, int64_t k, uint16_t* P, void* ws, hipStream_t s) {
  const QrPlan p = qr_plan(k, R);
  const QrLayout l = qr_layout(k, R);
  char* base = static_cast<char*>(ws);
  uint32_t* counter = reinterpret_cast<uint32_t*>(base);
  double* A = reinterpret_cast<double*>(base + l.a);
  double* Q1 = reinterpret_cast<double*>(base + l.q1);
  double* part = reinterpret_cast<double*>(base + l.partial);
  double* G = reinterpret_cast<double*>(base + l.g);
  double* U1 = reinterpret_cast<double*>(base + l.u1);
  double* U2 = reinterpret_cast<double*>(base + l.u2);
  uint32_t* status = reinterpret_cast<uint32_t*>(base + l.status);
  const unsigned red_blocks = (unsigned)((R * R + 255) / 256);
  const double scale = sqrt((double)k / (double)R);

  hipLaunchKernelGGL((gram_kernel<R, true>), dim3(p.blocks), dim3(256), 0, s, A, k, p.rows_per_block, seed, part);
  hipLaunchKernelGGL((reduce_factor_kernel<R>), dim3(red_blocks), dim3(256), 0, s, part, p.blocks, G, U1, counter,
                     status);
  hipLaunchKernelGGL((trmul_kernel<R, false>), dim3(p.blocks), dim3(256), 0, s, A, U1, k, p.rows_per_block, 1.0, Q1,
                     nullptr);
  hipLaunchKernelGGL((gram_kernel<R, false>), dim3(p.blocks), dim3(256), 0, s, Q1, k, p.rows_per_block, seed, part);
  hipLaunchKernelGGL((reduce_factor_kernel<R>), dim3(red_blocks), dim3(256), 0, s, part, p.blocks, G, U2, counter,
                     status + 1);
  hipLaunchKernelGGL((trmul_kernel<R, true>), dim3(p.blocks), dim3(256), 0, s, Q1, U2, k, p.rows_per_block, scale,
                     nullptr, P);
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

bool qr_rank_supported(int64_t r) { return r == 16 || r == 32 || r == 48 || r == 64 || r == 128; }

}  // namespace
}  // namespace rgc

using namespace rgc;

extern "C" size_t rgc_sample_projection_workspace_size(rgc_proj_kind_t kind, int64_t k, int64_t r) {
  if (kind == RGC_PROJ_RADEMACHER) return 0;
  if (kind != RGC_PROJ_QR_GAUSSIAN || k <= 0 || !qr_rank_supported(r)) return 0;
  return qr_layout(k, r).total;
}

extern "C" rgc_status_t rgc_sample_projection(rgc_proj_kind_t kind, uint64_t seed, int64_t k, int64_t r, uint16_t* P,
                                              void* ws, size_t ws_bytes, void* stream) {
  if (k <= 0 || r <= 0 || r > k) return RGC_ERR_SHAPE;
  if (kind != RGC_PROJ_RADEMACHER && kind != RGC_PROJ_QR_GAUSSIAN) return RGC_ERR_UNSUPPORTED;
  if (!rank_supported(r) || (k % 8) != 0 || k > (int64_t)0xFFFFFFFF) return RGC_ERR_UNSUPPORTED;
  if (kind == RGC_PROJ_QR_GAUSSIAN && !qr_rank_supported(r)) return RGC_ERR_UNSUPPORTED;
  if (!P) return RGC_ERR_NULL;
  if (!aligned16(P)) return RGC_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == RGC_PROJ_RADEMACHER) {
    // a = bf16(fp32(1/sqrt(r))), both roundings to nearest even
    const float af = (float)(1.0 / sqrt((double)r));
    uint32_t b;
    memcpy(&b, &af, sizeof(b));
    const uint32_t mag = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
    const int64_t n = k * (r / 8);
    hipLaunchKernelGGL(rademacher_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, P, k, (int)r, seed, mag);
    return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
  }
  const size_t need = qr_layout(k, r).total;
  if (!ws || ws_bytes < need) return RGC_ERR_WORKSPACE;
  if (!aligned_to(ws, 256)) return RGC_ERR_ALIGN;
  switch (r) {
    case 16: return qr_launch<16>(seed, k, P, ws, s);
    case 32: return qr_launch<32>(seed, k, P, ws, s);
    case 48: return qr_launch<48>(seed, k, P, ws, s);
    case 64: return qr_launch<64>(seed, k, P, ws, s);
    case 128: return qr_launch<128>(seed, k, P, ws, s);
    default: return RGC_ERR_UNSUPPORTED;
  }
}
