// Seeded projection P (k x r, bf16), regenerated from a 64-bit seed so that it
// never has to be stored or sent ([page "LoGRA: Low-Rank Gradient Sketches",
// "Why Refreshing the Projection Enables New Update Directions"]).
//
// Rademacher [same page, "Why the Sketch Can Be Accumulated Without a Full
// Gradient"]: entries +-1/sqrt(r) from Philox sign bits.
//
// QR of a Gaussian [page "Randomized Gradient Compression", footnote 1]:
// P = sqrt(k/r) Q with Q the sign-corrected (diag R > 0) thin QR factor of a
// Gaussian k x r matrix. Q is computed by CholeskyQR2 in fp64, for a batch of
// matrices of one rank at once (each launch covers every matrix, so the
// latency-bound steps are paid once per batch, not once per matrix):
//   gram     A = Box-Muller normals from Philox (stored), partial Grams of A
//            over 64-row blocks
//   reduce   G1 = A^T A (partials summed in block order)
//   factor   U1 = chol(G1)^-1
//   gram     Q1 = A U1 (stored), partial Grams of Q1, and P = bf16(fp32(
//            sqrt(k/r) * Q1)) as a candidate
//   reduce   G2 = Q1^T Q1
//   factor   U2 = chol(G2)^-1 (G2 is the identity up to rounding, so this is
//            the first-order expansion I - S unless some |G2 - I| >= 1e-7)
//   gram     P = bf16(fp32(sqrt(k/r) * Q1 U2)), skipped (the candidate kept)
//            when every |G2 - I| < 1e-14, as it is for well-conditioned
//            Gaussian matrices
// Cholesky factors have a positive diagonal, so Q is the unique factor with
// the standard sign correction; the second pass restores orthogonality to
// fp64 accuracy. Every reduction has a fixed order, so P is bit-reproducible.
// A Gram matrix that is not numerically positive definite (it does not happen
// for Gaussian matrices with k >= r in practice) makes its factor all NaN, so
// the P of that matrix is all NaN and an update computed from it is skipped.
#include <math.h>
#include <string.h>

#include "rgc_internal.hpp"

namespace rgc {

// ---------------------------------------------------------------------------
// Rademacher: one thread per (row, 8 columns), or per row when r = 4.
// ---------------------------------------------------------------------------
__global__ void rademacher_kernel(uint16_t* __restrict__ P, int64_t k, int r, uint64_t seed, uint32_t mag) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per = r < 8 ? r : 8;  // columns per thread
  const int groups = r / per;
  if (idx >= k * groups) return;
  const int64_t i = idx / groups;
  const int j0 = (int)(idx % groups) * per;
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
  if (per == 8)
    *reinterpret_cast<uint4*>(P + i * r + j0) = make_uint4(out[0], out[1], out[2], out[3]);
  else
    *reinterpret_cast<uint2*>(P + i * r + j0) = make_uint2(out[0], out[1]);
}

// ---------------------------------------------------------------------------
// CholeskyQR2, batched over up to kQrMaxBatch matrices of one rank R <= 128.
// ---------------------------------------------------------------------------
constexpr int kQrMaxBatch = 16;
// Rows per Gram / multiply workgroup: four row tiles of 16, one per wave.
constexpr int kQrBlockRows = 64;

constexpr double kTwoPi = 6.283185307179586;  // 2*pi rounded to double
// When every entry of Q1^T Q1 - I is below this, Q1 (U2 = I - S, |S| below it
// too) already equals the second pass's Q to ~1e-14, far inside the bf16
// rounding of P, and the P written from Q1 by the first multiply is kept.
constexpr double kQrFinalTol = 1e-14;

struct QrBatch {
  int n;
  int64_t k[kQrMaxBatch];
  uint64_t seed[kQrMaxBatch];
  double scale[kQrMaxBatch];
  uint16_t* P[kQrMaxBatch];
  double* A[kQrMaxBatch];     // k x R Gaussian
  double* Q1[kQrMaxBatch];    // k x R after the first pass
  double* part[kQrMaxBatch];  // one R x R partial Gram per row block
  double* U1[kQrMaxBatch];
  double* U2[kQrMaxBatch];
  // status[m]: [0], [1] = factorization failed in pass 1, 2; [2] = the first
  // pass is already orthonormal to kQrFinalTol, so P from it is final
  uint32_t* status[kQrMaxBatch];
  int block_begin[kQrMaxBatch + 1];  // workgroup prefix of the row blocks
};

__device__ __forceinline__ int batch_item(const int* begin, int n, int b) {
  int m = 0;
  while (m + 1 < n && b >= begin[m + 1]) ++m;
  return m;
}

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

// The three block steps on fp64 MFMA (v_mfma_f64_16x16x4_f64):
//   MODE 0: draw the Gaussian rows of the block (into A and LDS), partial Gram of A;
//   MODE 1: Q1 = A U1 (stored, with the candidate P from it), partial Gram of Q1;
//   MODE 2: P = bf16(fp32(scale * Q1 U2)).
// operands come straight from the staged rows, so the products no longer
// wait on one LDS read per multiply-add. A 16 x 16 x 4 product takes, in lane
// l, A[l % 16][l / 16] and B[l / 16][l % 16] and returns D[4 i + l / 16][l % 16]
// in its register i = 0..3 (rows interleaved over the lane groups; measured
// with a probe). Wave w owns row tile w of a multiply (the 64 staged rows are
// four tiles of 16) and row tiles w, w + 4 of a Gram. U is upper triangular:
// only its 16 x 16 tiles on and above the diagonal are staged (tile (rt, tc),
// rt <= tc, at slot tc (tc + 1) / 2 + rt, rows padded to 17), which is what
// lets r = 128 stage U beside the rows, and the multiply skips the zero tiles.
typedef double f64x4_t __attribute__((ext_vector_type(4)));

constexpr int kUTilePitch = 17;                     // doubles per staged U tile row
constexpr int kUTileSize = 16 * kUTilePitch;        // doubles per staged U tile
__host__ __device__ constexpr int utile_slot(int rt, int tc) { return tc * (tc + 1) / 2 + rt; }

template <int R, int MODE>
__global__ __launch_bounds__(256) void qr_block_mfma_kernel(QrBatch b) {
  static_assert(R <= 128 && R % 16 == 0, "r <= 128, multiple of 16");
  constexpr int BR = kQrBlockRows;
  static_assert(BR == 64, "four row tiles, one per wave");
  constexpr int NT = R / 16;
  constexpr int LD = R + 1;             // padded row pitch (doubles)
  __shared__ double rows[BR][LD];
  __shared__ double u[MODE == 0 ? 1 : NT * (NT + 1) / 2 * kUTileSize];
  const int m = batch_item(b.block_begin, b.n, blockIdx.x);
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int li = lane & 15, lg = lane >> 4;
  const int64_t k = b.k[m];
  const int64_t rbeg = (int64_t)(blockIdx.x - b.block_begin[m]) * BR;
  const int64_t rend = rbeg + BR < k ? rbeg + BR : k;
  if constexpr (MODE == 2) {
    if (b.status[m][2] != 0u) return;  // P from the first pass is final
  }
  const double* src = MODE == 2 ? b.Q1[m] : b.A[m];
  if constexpr (MODE == 0) {
    // The Gaussian rows are drawn here (four columns per Philox call) into
    // LDS and into A for the first multiply.
    constexpr int NQ = BR * (R / 4) / 256;
#pragma unroll
    for (int e = 0; e < NQ; ++e) {
      const int t = threadIdx.x + 256 * e;
      const int lr = t / (R / 4), q = t % (R / 4);
      const int64_t row = rbeg + lr;
      double z[4] = {0.0, 0.0, 0.0, 0.0};
      if (row < rend) {
        gaussian4(b.seed[m], row, q, z);
        double* dst = b.A[m] + row * R + 4 * q;
#pragma unroll
        for (int x = 0; x < 4; ++x) dst[x] = z[x];
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) rows[lr][4 * q + x] = z[x];
    }
  } else {
    // every load issued before the first LDS store; rows past the end read
    // a valid row and are zeroed
    constexpr int NS = BR * R / 256, NU = MODE == 0 ? 0 : R * R / 256;
    double sv[NS], uv[NU > 0 ? NU : 1];
#pragma unroll
    for (int e = 0; e < NS; ++e) {
      const int t = threadIdx.x + 256 * e;
      const int64_t row = rbeg + t / R;
      sv[e] = src[(row < rend ? row : rend - 1) * R + t % R];
    }
    if constexpr (MODE != 0) {
      const double* U = MODE == 1 ? b.U1[m] : b.U2[m];
#pragma unroll
      for (int e = 0; e < NU; ++e) uv[e] = U[threadIdx.x + 256 * e];
    }
#pragma unroll
    for (int e = 0; e < NS; ++e) {
      const int t = threadIdx.x + 256 * e;
      rows[t / R][t % R] = rbeg + t / R < rend ? sv[e] : 0.0;
    }
    if constexpr (MODE != 0) {
#pragma unroll
      for (int e = 0; e < NU; ++e) {
        const int t = threadIdx.x + 256 * e;
        const int a = t / R, c = t % R;
        if (a / 16 <= c / 16) u[utile_slot(a / 16, c / 16) * kUTileSize + (a % 16) * kUTilePitch + c % 16] = uv[e];
      }
    }
  }
  __syncthreads();
  if constexpr (MODE != 0) {
    // Y = rows U: row tile `wave`, all column tiles
    f64x4_t y[NT];
#pragma unroll
    for (int tc = 0; tc < NT; ++tc) y[tc] = f64x4_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kk = 0; kk < R / 4; ++kk) {
      const double a = rows[16 * wave + li][4 * kk + lg];
      const int rt = kk / 4;  // U's row tile; tiles left of the diagonal are zero
#pragma unroll
      for (int tc = 0; tc < NT; ++tc)
        if (tc >= rt)
          y[tc] = __builtin_amdgcn_mfma_f64_16x16x4f64(
              a, u[utile_slot(rt, tc) * kUTileSize + (4 * kk + lg - 16 * rt) * kUTilePitch + li], y[tc], 0, 0, 0);
    }
    const double scale = b.scale[m];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int lr = 16 * wave + 4 * i + lg;
      const int64_t row = rbeg + lr;
      if (row >= rend) continue;
#pragma unroll
      for (int tc = 0; tc < NT; ++tc) {
        const int col = 16 * tc + li;
        if constexpr (MODE == 1) b.Q1[m][row * R + col] = y[tc][i];
        b.P[m][row * R + col] = (uint16_t)f32_to_bf16_rne((float)(scale * y[tc][i]));
      }
    }
    if constexpr (MODE == 2) return;
    __syncthreads();  // every wave is done reading the staged rows
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int tc = 0; tc < NT; ++tc) rows[16 * wave + 4 * i + lg][16 * tc + li] = y[tc][i];  // 0 past the end
    __syncthreads();
  }
  // partial Gram of the staged rows: row tiles wave, wave + 4, all column tiles
#pragma unroll
  for (int pass = 0; pass < (NT + 3) / 4; ++pass) {
    const int ti = wave + 4 * pass;
    if (ti >= NT) break;
    f64x4_t acc[NT];
#pragma unroll
    for (int tj = 0; tj < NT; ++tj) acc[tj] = f64x4_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kk = 0; kk < BR / 4; ++kk) {
      const double a = rows[4 * kk + lg][16 * ti + li];
#pragma unroll
      for (int tj = 0; tj < NT; ++tj)
        acc[tj] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, rows[4 * kk + lg][16 * tj + li], acc[tj], 0, 0, 0);
    }
    double* out = b.part[m] + (int64_t)(blockIdx.x - b.block_begin[m]) * R * R;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int tj = 0; tj < NT; ++tj) out[(16 * ti + 4 * i + lg) * R + 16 * tj + li] = acc[tj][i];
  }
}

// The same three block steps for ranks below one MFMA tile (r = 4, 8), on
// the fp64 VALU: one wave per 64-row block, one row per lane. The multiply
// sums a = 0 .. c in order; the block's Gram entries are lane butterflies.
template <int R, int MODE>
__global__ __launch_bounds__(64) void qr_block_small_kernel(QrBatch b) {
  static_assert(R == 4 || R == 8, "small rank");
  const int m = batch_item(b.block_begin, b.n, blockIdx.x);
  const int64_t k = b.k[m];
  const int64_t rbeg = (int64_t)(blockIdx.x - b.block_begin[m]) * kQrBlockRows;
  const int64_t rend = rbeg + kQrBlockRows < k ? rbeg + kQrBlockRows : k;
  if constexpr (MODE == 2) {
    if (b.status[m][2] != 0u) return;  // P from the first pass is final
  }
  const int64_t row = rbeg + threadIdx.x;
  const bool in = row < rend;
  double y[R];
#pragma unroll
  for (int c = 0; c < R; ++c) y[c] = 0.0;
  if constexpr (MODE == 0) {
    if (in) {
#pragma unroll
      for (int q = 0; q < R / 4; ++q) {
        double z[4];
        gaussian4(b.seed[m], row, q, z);
#pragma unroll
        for (int x = 0; x < 4; ++x) y[4 * q + x] = z[x];
      }
#pragma unroll
      for (int c = 0; c < R; ++c) b.A[m][row * R + c] = y[c];
    }
  } else {
    const double* src = MODE == 2 ? b.Q1[m] : b.A[m];
    const double* U = MODE == 1 ? b.U1[m] : b.U2[m];
    double x[R];
#pragma unroll
    for (int a = 0; a < R; ++a) x[a] = in ? src[row * R + a] : 0.0;
#pragma unroll
    for (int c = 0; c < R; ++c) {
      double acc = 0.0;
#pragma unroll
      for (int a = 0; a <= c; ++a) acc += x[a] * U[a * R + c];
      y[c] = acc;
    }
    if (in) {
#pragma unroll
      for (int c = 0; c < R; ++c) {
        if constexpr (MODE == 1) b.Q1[m][row * R + c] = y[c];
        b.P[m][row * R + c] = (uint16_t)f32_to_bf16_rne((float)(b.scale[m] * y[c]));
      }
    }
    if constexpr (MODE == 2) return;
  }
  double* out = b.part[m] + (int64_t)(blockIdx.x - b.block_begin[m]) * R * R;
#pragma unroll
  for (int a = 0; a < R; ++a)
#pragma unroll
    for (int c = 0; c < R; ++c) {
      const double v = wave_sum(y[a] * y[c]);
      if (threadIdx.x == 0) out[a * R + c] = v;
    }
}

// G = sum of a matrix's block partials in block order, upper triangle only
// (one thread per entry, 16 blocks' loads in flight at a time).
template <int R>
__global__ __launch_bounds__(256) void qr_gram_reduce_kernel(QrBatch b, double* __restrict__ G_all) {
  const int m = blockIdx.y;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= b.n || e >= R * R) return;
  const int row = e / R, col = e % R;
  if (col < row) return;
  const int nparts = b.block_begin[m + 1] - b.block_begin[m];
  const double* part = b.part[m];
  double sum = 0.0;
  for (int p0 = 0; p0 < nparts; p0 += 16) {
    double v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = part[(int64_t)(p0 + i < nparts ? p0 + i : nparts - 1) * R * R + e];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (p0 + i < nparts) sum = (p0 + i == 0) ? v[i] : sum + v[i];
  }
  G_all[(int64_t)m * R * R + e] = sum;
}

// One workgroup (NT x NT threads) per matrix: U = chol(G)^-1 (upper triangular,
// zeros below) from the summed Gram G (upper triangle).
//
// U comes from one Gaussian elimination of [G | I] without pivoting (stable
// for symmetric positive definite G): with G = L D L^T (L unit lower), the
// eliminated left block is D L^T and the right block is L^-1, so
// R = D^1/2 L^T and R^-1 = L^-T D^-1/2. Thread (ty, tx) of an NT x NT grid
// keeps elements (ty + NT a, tx + NT c) in registers: the symmetric Schur
// complement in the upper triangle and L^-1 (unit diagonal implied) in the
// strictly lower one. Only the pivot row travels through LDS, double
// buffered, together with its reciprocal pivot, so each column costs one
// barrier and no division on the critical path of the other threads.
template <int R>
struct QrFactorShape {
  // NT x NT threads, each holding TT x TT elements. (16 x 16 threads at
  // r = 64, with cheaper barriers but four times the per-thread work per
  // column, measured twice as slow.)
  static constexpr int NT = 32;
  static constexpr int TT = (R + NT - 1) / NT;
  static constexpr int THREADS = NT * NT;
};

template <int R>
__global__ __launch_bounds__(QrFactorShape<R>::THREADS) void qr_factor_kernel(QrBatch b, const double* __restrict__ G_all,
                                                                             int second) {
  constexpr int NT = QrFactorShape<R>::NT;
  constexpr int TT = QrFactorShape<R>::TT;
  __shared__ double rowbuf[2][R];
  __shared__ double rinv[2];
  __shared__ double diag[R];
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const int tx = tid % NT, ty = tid / NT;
  double* U = second ? b.U2[m] : b.U1[m];
  const double* G = G_all + (int64_t)m * R * R;

  double a[TT][TT];
#pragma unroll
  for (int i = 0; i < TT; ++i)
#pragma unroll
    for (int j = 0; j < TT; ++j) {
      const int l = ty + NT * i, c = tx + NT * j;
      a[i][j] = (l < R && c < R && c >= l) ? G[l * R + c] : 0.0;
      if (l == 0 && c < R) rowbuf[0][c] = a[i][j];
      if (l == 0 && c == 0) rinv[0] = 1.0 / a[i][j];
    }
  if (second) {
    // G2 = Q1^T Q1 is the identity up to rounding (|G2 - I| ~ 1e-15 for the
    // Gaussian matrices here). For G2 = I + E, chol(G2) = I + S with S the
    // upper triangle of E (diagonal halved) up to O(|E|^2), and its inverse
    // is I - S up to O(|E|^2): below 1e-14 when every |E| < 1e-7, so the
    // elimination below is skipped. Otherwise it runs as for G1.
    bool far = false, above_final = false;
#pragma unroll
    for (int i = 0; i < TT; ++i)
#pragma unroll
      for (int j = 0; j < TT; ++j) {
        const int l = ty + NT * i, c = tx + NT * j;
        if (l < R && c < R && c >= l) {
          const double e = fabs(a[i][j] - (c == l ? 1.0 : 0.0));
          far = far || !(e < 1e-7);
          above_final = above_final || !(e < kQrFinalTol);
        }
      }
    const bool keep_first = !__syncthreads_or(above_final);
    if (!__syncthreads_or(far)) {
      if (tid == 0) {
        b.status[m][second] = 0u;
        b.status[m][2] = keep_first ? 1u : 0u;
      }
#pragma unroll
      for (int i = 0; i < TT; ++i)
#pragma unroll
        for (int j = 0; j < TT; ++j) {
          const int l = ty + NT * i, c = tx + NT * j;
          if (l >= R || c >= R) continue;
          U[l * R + c] = c < l ? 0.0 : (c == l ? 1.0 - 0.5 * (a[i][j] - 1.0) : -a[i][j]);
        }
      return;
    }
  }
  for (int j = 0; j < R; ++j) {
    __syncthreads();
    const double* rb = rowbuf[j & 1];
    const double inv = rinv[j & 1];
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      const int l = ty + NT * i;
      if (l <= j || l >= R) continue;
      const double f = rb[l] * inv;  // G(l, j) / G(j, j), from the symmetric upper copy
#pragma unroll
      for (int jj = 0; jj < TT; ++jj) {
        const int c = tx + NT * jj;
        if (c >= R) continue;
        if (c >= l || c < j) a[i][jj] -= f * rb[c];
        else if (c == j) a[i][jj] = -f;  // E(l, j) = 0 - f * E(j, j)
      }
      if (l == j + 1) {
#pragma unroll
        for (int jj = 0; jj < TT; ++jj) {
          const int c = tx + NT * jj;
          if (c < R) rowbuf[(j + 1) & 1][c] = a[i][jj];
          if (c == l) rinv[(j + 1) & 1] = 1.0 / a[i][jj];
        }
      }
    }
  }
  // U[x][y] = E(y, x) / sqrt(D_y) above the diagonal, 1 / sqrt(D_y) on it
#pragma unroll
  for (int i = 0; i < TT; ++i)
#pragma unroll
    for (int j = 0; j < TT; ++j) {
      const int l = ty + NT * i, c = tx + NT * j;
      if (l < R && c == l) diag[l] = a[i][j];
    }
  // A pivot that is not positive and finite means G is not numerically
  // positive definite: the whole factor is then NaN (and so is P).
  bool bad = false;
#pragma unroll
  for (int i = 0; i < TT; ++i)
#pragma unroll
    for (int j = 0; j < TT; ++j) {
      const int l = ty + NT * i, c = tx + NT * j;
      if (l < R && c == l) bad = bad || !(a[i][j] > 0.0 && isfinite(a[i][j]));
    }
  const bool failed = __syncthreads_or(bad) != 0;
  if (tid == 0) {
    b.status[m][second] = failed ? 1u : 0u;
    if (second) b.status[m][2] = 0u;
  }
  const double nan = __builtin_nan("");
#pragma unroll
  for (int i = 0; i < TT; ++i)
#pragma unroll
    for (int j = 0; j < TT; ++j) {
      const int l = ty + NT * i, c = tx + NT * j;
      if (l >= R || c >= R || c > l) continue;
      const double rs = 1.0 / sqrt(diag[l]);
      if (c == l) {
        U[l * R + l] = failed ? nan : rs;
      } else {
        U[c * R + l] = failed ? nan : a[i][j] * rs;
        U[l * R + c] = failed ? nan : 0.0;
      }
    }
}

namespace {

struct QrItemLayout {
  size_t a, q1, part, u1, u2, status, total;
  int blocks;
};

QrItemLayout qr_item_layout(int64_t k, int64_t r) {
  QrItemLayout l;
  l.blocks = (int)((k + kQrBlockRows - 1) / kQrBlockRows);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += (bytes + 255) / 256 * 256;
    return at;
  };
  l.a = take((size_t)k * r * sizeof(double));
  l.q1 = take((size_t)k * r * sizeof(double));
  l.part = take((size_t)l.blocks * r * r * sizeof(double));
  l.u1 = take((size_t)r * r * sizeof(double));
  l.u2 = take((size_t)r * r * sizeof(double));
  l.status = take(3 * sizeof(uint32_t));
  l.total = off;
  return l;
}

size_t qr_gram_bytes(int64_t n, int64_t r) { return ((size_t)n * r * r * sizeof(double) + 255) / 256 * 256; }

template <int R>
rgc_status_t qr_launch(int n, const uint64_t* seeds, const int64_t* ks, uint16_t* const* Ps, void* ws, hipStream_t s) {
  QrBatch b = {};
  b.n = n;
  char* base = static_cast<char*>(ws);
  // the n summed Gram matrices first, then each item's buffers
  double* G_all = reinterpret_cast<double*>(base);
  size_t off = qr_gram_bytes(n, R);
  b.block_begin[0] = 0;
  for (int m = 0; m < n; ++m) {
    const QrItemLayout l = qr_item_layout(ks[m], R);
    b.k[m] = ks[m];
    b.seed[m] = seeds[m];
    b.scale[m] = sqrt((double)ks[m] / (double)R);
    b.P[m] = Ps[m];
    b.A[m] = reinterpret_cast<double*>(base + off + l.a);
    b.Q1[m] = reinterpret_cast<double*>(base + off + l.q1);
    b.part[m] = reinterpret_cast<double*>(base + off + l.part);
    b.U1[m] = reinterpret_cast<double*>(base + off + l.u1);
    b.U2[m] = reinterpret_cast<double*>(base + off + l.u2);
    b.status[m] = reinterpret_cast<uint32_t*>(base + off + l.status);
    b.block_begin[m + 1] = b.block_begin[m] + l.blocks;
    off += l.total;
  }
  const dim3 red_grid((unsigned)((R * R + 255) / 256), (unsigned)n);
  const dim3 blocks((unsigned)b.block_begin[n]);
  auto block_step = [&](auto mode) {
    constexpr int MODE = decltype(mode)::value;
    if constexpr (R < 16)
      hipLaunchKernelGGL((qr_block_small_kernel<R, MODE>), blocks, dim3(64), 0, s, b);
    else
      hipLaunchKernelGGL((qr_block_mfma_kernel<R, MODE>), blocks, dim3(256), 0, s, b);
  };
  block_step(IntC<0>{});
  hipLaunchKernelGGL((qr_gram_reduce_kernel<R>), red_grid, dim3(256), 0, s, b, G_all);
  hipLaunchKernelGGL((qr_factor_kernel<R>), dim3(n), dim3(QrFactorShape<R>::THREADS), 0, s, b, G_all, 0);
  block_step(IntC<1>{});
  hipLaunchKernelGGL((qr_gram_reduce_kernel<R>), red_grid, dim3(256), 0, s, b, G_all);
  hipLaunchKernelGGL((qr_factor_kernel<R>), dim3(n), dim3(QrFactorShape<R>::THREADS), 0, s, b, G_all, 1);
  block_step(IntC<2>{});
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

bool qr_rank_supported(int64_t r) { return rank_small(r) || (r >= 16 && r <= 128 && r % 16 == 0); }

uint32_t rademacher_magnitude(int64_t r) {
  // a = bf16(fp32(1/sqrt(r))), both roundings to nearest even
  const float af = (float)(1.0 / sqrt((double)r));
  uint32_t bits;
  memcpy(&bits, &af, sizeof(bits));
  return (bits + 0x7FFFu + ((bits >> 16) & 1u)) >> 16;
}

rgc_status_t check_item(rgc_proj_kind_t kind, int64_t k, int64_t r, const uint16_t* P) {
  if (k <= 0 || r <= 0 || r > k) return RGC_ERR_SHAPE;
  if (kind != RGC_PROJ_RADEMACHER && kind != RGC_PROJ_QR_GAUSSIAN) return RGC_ERR_UNSUPPORTED;
  if (!rank_supported(r) || (k % 8) != 0 || k > (int64_t)0x7FFFFFFF) return RGC_ERR_UNSUPPORTED;
  if (kind == RGC_PROJ_QR_GAUSSIAN && !qr_rank_supported(r)) return RGC_ERR_UNSUPPORTED;
  if (!P) return RGC_ERR_NULL;
  if (!aligned16(P)) return RGC_ERR_ALIGN;
  return RGC_OK;
}

size_t batch_ws(rgc_proj_kind_t kind, int64_t n, const int64_t* ks, int64_t r) {
  if (kind != RGC_PROJ_QR_GAUSSIAN || !qr_rank_supported(r) || n <= 0 || n > kQrMaxBatch || !ks) return 0;
  size_t total = qr_gram_bytes(n, r);
  for (int64_t m = 0; m < n; ++m) {
    if (ks[m] <= 0) return 0;
    total += qr_item_layout(ks[m], r).total;
  }
  return total;
}

}  // namespace

rgc_status_t sample_validate(rgc_proj_kind_t kind, int64_t k, int64_t r, const uint16_t* P) {
  return check_item(kind, k, r, P);
}

}  // namespace rgc

using namespace rgc;

extern "C" size_t rgc_sample_projection_workspace_size(rgc_proj_kind_t kind, int64_t k, int64_t r) {
  return batch_ws(kind, 1, &k, r);
}

extern "C" size_t rgc_sample_projections_workspace_size(rgc_proj_kind_t kind, int64_t n, const int64_t* ks,
                                                        int64_t r) {
  return batch_ws(kind, n, ks, r);
}

extern "C" rgc_status_t rgc_sample_projections(rgc_proj_kind_t kind, int64_t n, const uint64_t* seeds,
                                               const int64_t* ks, int64_t r, uint16_t* const* Ps, void* ws,
                                               size_t ws_bytes, void* stream) {
  if (n < 0 || n > kQrMaxBatch) return RGC_ERR_UNSUPPORTED;
  if (n == 0) return RGC_OK;
  if (!seeds || !ks || !Ps) return RGC_ERR_NULL;
  for (int64_t m = 0; m < n; ++m) {
    const rgc_status_t st = check_item(kind, ks[m], r, Ps[m]);
    if (st != RGC_OK) return st;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == RGC_PROJ_RADEMACHER) {
    const uint32_t mag = rademacher_magnitude(r);
    for (int64_t m = 0; m < n; ++m) {
      const int64_t cnt = ks[m] * (r < 8 ? 1 : r / 8);  // threads of rademacher_kernel
      hipLaunchKernelGGL(rademacher_kernel, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, s, Ps[m], ks[m], (int)r,
                         seeds[m], mag);
    }
    return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
  }
  const size_t need = batch_ws(kind, n, ks, r);
  if (!ws || ws_bytes < need) return RGC_ERR_WORKSPACE;
  if (!aligned_to(ws, 256)) return RGC_ERR_ALIGN;
  rgc_status_t st = RGC_ERR_UNSUPPORTED;
  if (dispatch_small_rank(r, [&](auto rc) { st = qr_launch<decltype(rc)::value>((int)n, seeds, ks, Ps, ws, s); }))
    return st;
  static_for<1, 9>([&](auto q) {
    constexpr int R = 16 * decltype(q)::value;
    if (r == R) st = qr_launch<R>((int)n, seeds, ks, Ps, ws, s);
  });
  return st;
}

extern "C" rgc_status_t rgc_sample_projection(rgc_proj_kind_t kind, uint64_t seed, int64_t k, int64_t r, uint16_t* P,
                                              void* ws, size_t ws_bytes, void* stream) {
  return rgc_sample_projections(kind, 1, &seed, &k, r, &P, ws, ws_bytes, stream);
}
