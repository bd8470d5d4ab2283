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
//   draw     A = Box-Muller normals from Philox (stored; its own launch,
//            one thread per four values, so that the fp64 transcendentals
//            run at full occupancy)
//   gram     partial Grams of A, one per workgroup of 128 rows (summed in
//            registers over its two 64-row blocks)
//   reduce   G1 = A^T A (partials summed in workgroup order)
//   factor   U1 = chol(G1)^-1
//   gram     Q1 = A U1, partial Grams of Q1, and P = bf16(fp32(sqrt(k/r) *
//            Q1)) as a candidate
//   reduce   G2 = Q1^T Q1
//   factor   U2 = chol(G2)^-1 (G2 is the identity up to rounding, so this is
//            the first-order expansion I - S unless some |G2 - I| >= 1e-7)
//   gram     P = bf16(fp32(sqrt(k/r) * Q1 U2)) with Q1 = A U1 formed again
//            as in the pass before (same bits), skipped (the candidate kept)
//            when every |G2 - I| < 1e-14, as it is for well-conditioned
//            Gaussian matrices
// Q1 is not stored at ranks of 16 and up (the third step, rarely run, forms
// it again). Ranks 4 and 8 run one 64-row block per workgroup on the VALU,
// drawing A in their first step and keeping Q1.
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
// Rows per block of the Gram / multiply steps: four row tiles of 16, one per
// wave.
constexpr int kQrBlockRows = 64;
// Blocks per workgroup of the fp64 MFMA steps: a workgroup sums its blocks'
// Gram in registers and writes one partial, so the partials written and read
// back per pass are half of one per block, and U is staged once per two
// blocks. (More blocks per workgroup leave too few workgroups to fill the
// chip for one transformer block's projections, and make each workgroup hold
// its compute unit longer against other streams' launches.)
constexpr int kQrGroupBlocks = 3;

// Rows per workgroup of a block step at rank r (the small-rank steps run one
// block per workgroup).
__host__ __device__ constexpr int qr_group_rows(int64_t r) {
  return r < 16 ? kQrBlockRows : kQrBlockRows * kQrGroupBlocks;
}

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
  double* Q1[kQrMaxBatch];    // k x R after the first pass (ranks 4 and 8 only)
  double* part[kQrMaxBatch];  // one R x R partial Gram per workgroup
  double* U1[kQrMaxBatch];
  double* U2[kQrMaxBatch];
  // status[m]: [0], [1] = factorization failed in pass 1, 2; [2] = the first
  // pass is already orthonormal to kQrFinalTol, so P from it is final
  uint32_t* status[kQrMaxBatch];
  int block_begin[kQrMaxBatch + 1];  // workgroup prefix (qr_group_rows rows per workgroup)
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

// The Gaussian A of every matrix of the batch: one thread per row and four
// columns (one Philox call), a grid row per matrix.
template <int R>
__global__ __launch_bounds__(256) void qr_gauss_kernel(QrBatch b) {
  const int m = blockIdx.y;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (m >= b.n || t >= b.k[m] * (R / 4)) return;
  const int64_t row = t / (R / 4);
  const int q = (int)(t % (R / 4));
  double z[4];
  gaussian4(b.seed[m], row, q, z);
  double2* dst = reinterpret_cast<double2*>(b.A[m] + row * R + 4 * q);
  dst[0] = make_double2(z[0], z[1]);
  dst[1] = make_double2(z[2], z[3]);
}

// The three block steps on fp64 MFMA (v_mfma_f64_16x16x4_f64), each
// workgroup over up to kQrGroupBlocks blocks of 64 rows of one matrix:
//   MODE 0: partial Gram of A;
//   MODE 1: Q1 = A U1, the candidate P from Q1; partial Gram of Q1;
//   MODE 2: Q1 = A U1 as in MODE 1, P = bf16(fp32(scale * Q1 U2)).
// Operands come straight from the staged rows. A 16 x 16 x 4 product takes,
// in lane l, A[l % 16][l / 16] and B[l / 16][l % 16] and returns
// D[4 i + l / 16][l % 16] in its register i = 0..3 (rows interleaved over the
// lane groups; measured with a probe). Wave w owns row tile w of a multiply
// (the 64 staged rows are four tiles of 16). A Gram is symmetric and only its
// upper triangle is summed later, so only the 16 x 16 tiles (ti, tj) with
// ti <= tj are formed, numbered row by row, tile t by wave t % 4; each wave
// keeps its tiles' sums in registers across the workgroup's blocks. U is
// upper triangular: only its tiles on and above the diagonal are staged
// (tile (rt, tc), rt <= tc, at slot tc (tc + 1) / 2 + rt, rows padded to 17),
// which is what lets r = 128 stage U beside the rows, and the multiply skips
// the zero tiles.
typedef double f64x4_t __attribute__((ext_vector_type(4)));

// LDS pitches. The LDS serves 64 banks of 4 bytes, so a 64-bit read is free
// of bank conflicts when each half-wave's 32 lanes cover all 64 banks.
// The multiply reads its left operand as 16 rows x 4 columns (lane l: row
// l % 16, column l / 16) and the Gram reads both operands as 4 rows x 16
// columns; rows of 2 (mod 32) doubles serve the first, rows of 16 (mod 32)
// doubles the second, so a block is staged at the pitch its reader needs.
// U's tiles are read as 4 rows x 16 columns and are stored unpadded.
constexpr int kUTilePitch = 16;                     // doubles per staged U tile row
constexpr int kUTileSize = 16 * kUTilePitch;        // doubles per staged U tile
__host__ __device__ constexpr int qr_gram_pitch(int R) { return R % 32 == 0 ? R + 16 : R; }
__host__ __device__ constexpr int qr_mul_pitch(int R) { return R % 32 == 0 ? R + 2 : R + 18; }
__host__ __device__ constexpr int utile_slot(int rt, int tc) { return tc * (tc + 1) / 2 + rt; }

// Row and column tile of upper-triangle Gram tile t (row by row: row ti
// holds the nt - ti tiles ti .. nt - 1).
__device__ __forceinline__ void gram_tile(int t, int nt, int& ti, int& tj) {
  int i = 0;
  while (t >= nt - i) {
    t -= nt - i;
    ++i;
  }
  ti = i;
  tj = i + t;
}

// Threads of a block-step workgroup: eight waves, two per SIMD, so that one
// wave's products run while the other waits on LDS or a barrier.
constexpr int kQrThreads = 512;
constexpr int kQrWaves = kQrThreads / 64;

// Stages the upper-triangle tiles of U (R x R, row-major) into LDS, 16 loads
// in flight per thread at a time (few registers, so it can sit beside live
// products).
template <int R>
__device__ __forceinline__ void qr_stage_u(double* u, const double* __restrict__ U) {
  constexpr int CH = 16;
#pragma unroll 1
  for (int t0 = 0; t0 < R * R; t0 += kQrThreads * CH) {
    double uv[CH];
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      const int t = t0 + (int)threadIdx.x + kQrThreads * e;
      uv[e] = t < R * R ? U[t] : 0.0;
    }
#pragma unroll
    for (int e = 0; e < CH; ++e) {
      const int t = t0 + (int)threadIdx.x + kQrThreads * e;
      if (t >= R * R) continue;
      const int a = t / R, c = t % R;
      if (a / 16 <= c / 16) u[utile_slot(a / 16, c / 16) * kUTileSize + (a % 16) * kUTilePitch + c % 16] = uv[e];
    }
  }
}

// Row and column of element e of a thread in a row-major block of R columns
// that the workgroup's threads stride through (flat index threadIdx.x +
// kQrThreads e), from the thread's own row q0 and column c0: one compare per
// element instead of a division.
template <int R>
__device__ __forceinline__ void qr_flat_split(int q0, int c0, int e, int& row, int& col) {
  const int d = kQrThreads * e / R, mm = kQrThreads * e % R;
  const int c = c0 + mm;
  row = q0 + d + (c >= R ? 1 : 0);
  col = c >= R ? c - R : c;
}

// Workgroup barrier for LDS handoff only: this wave's LDS accesses are
// complete when it arrives, and global loads stay in flight across it (the
// next block's rows are fetched while the current block is multiplied).
__device__ __forceinline__ void qr_lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited for
  asm volatile("s_barrier" ::: "memory");
}

// Y = X U for the 16-row tile WR of a staged block (pitch LM) and the column
// tiles tc = 2 j + H (j < NY), U's upper-triangle tiles staged in u.
template <int R, int H>
__device__ __forceinline__ void qr_multiply(const double* rows, const double* u, int wr, int li, int lg,
                                            f64x4_t (&y)[(R / 16 + 1) / 2]) {
  constexpr int NT = R / 16, NY = (NT + 1) / 2, LM = qr_mul_pitch(R);
#pragma unroll
  for (int j = 0; j < NY; ++j) y[j] = f64x4_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int kk = 0; kk < R / 4; ++kk) {
    const double a = rows[(16 * wr + li) * LM + 4 * kk + lg];
    const int rt = kk / 4;  // U's row tile; tiles left of the diagonal are zero
#pragma unroll
    for (int j = 0; j < NY; ++j) {
      const int tc = 2 * j + H;
      if (tc < NT && tc >= rt)
        y[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(
            a, u[utile_slot(rt, tc) * kUTileSize + (4 * kk + lg - 16 * rt) * kUTilePitch + li], y[j], 0, 0, 0);
    }
  }
}

// The three block steps on fp64 MFMA (v_mfma_f64_16x16x4_f64), each
// workgroup over up to kQrGroupBlocks blocks of 64 rows of one matrix:
//   MODE 0: partial Gram of A;
//   MODE 1: Q1 = A U1, the candidate P from Q1; partial Gram of Q1;
//   MODE 2: Q1 = A U1 as in MODE 1, P = bf16(fp32(scale * Q1 U2)).
// Operands come straight from the staged rows. A 16 x 16 x 4 product takes,
// in lane l, A[l % 16][l / 16] and B[l / 16][l % 16] and returns
// D[4 i + l / 16][l % 16] in its register i = 0..3 (rows interleaved over the
// lane groups; measured with a probe). In a multiply, wave w owns row tile
// w % 4 of the block (64 rows, four tiles of 16) and the column tiles of
// parity w / 4. A Gram is symmetric and only its upper triangle is summed
// later, so only the 16 x 16 tiles (ti, tj) with ti <= tj are formed,
// numbered row by row, tile t by wave t % 8; each wave keeps its tiles' sums
// in registers across the workgroup's blocks. U is upper triangular: only its
// tiles on and above the diagonal are staged (tile (rt, tc), rt <= tc, at
// slot tc (tc + 1) / 2 + rt), which is what lets r = 128 stage U beside the
// rows, and the multiply skips the zero tiles.
template <int R, int MODE>
__global__ __launch_bounds__(kQrThreads) void qr_block_mfma_kernel(QrBatch b) {
  static_assert(R <= 128 && R % 16 == 0, "r <= 128, multiple of 16");
  constexpr int BR = kQrBlockRows;
  static_assert(BR == 64 && kQrWaves == 8, "four row tiles, two waves each");
  constexpr int NT = R / 16, NY = (NT + 1) / 2;
  constexpr int LG = qr_gram_pitch(R);            // row pitch of a block the Gram reads
  constexpr int LM = qr_mul_pitch(R);             // row pitch of a block a multiply reads
  constexpr int LA = MODE == 0 ? LG : LM;         // the pitch A is staged at
  constexpr int NTT = NT * (NT + 1) / 2;          // upper-triangle Gram tiles
  constexpr int PW = (NTT + kQrWaves - 1) / kQrWaves;  // Gram tiles per wave (at most)
  constexpr int NS = BR * R / kQrThreads;         // staged doubles per thread and block
  __shared__ double rows[BR * (LG > LM ? LG : LM)];
  __shared__ double u[MODE == 0 ? 1 : NT * (NT + 1) / 2 * kUTileSize];
  const int m = batch_item(b.block_begin, b.n, blockIdx.x);
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int li = lane & 15, lg = lane >> 4;
  const int wr = wave % 4, wh = wave / 4;  // multiply: row tile and column-tile parity
  const int64_t k = b.k[m];
  const int64_t gbeg = (int64_t)(blockIdx.x - b.block_begin[m]) * qr_group_rows(R);
  const int64_t gend = gbeg + qr_group_rows(R) < k ? gbeg + qr_group_rows(R) : k;
  if constexpr (MODE == 2) {
    if (b.status[m][2] != 0u) return;  // P from the first pass is final
  }
  const double* __restrict__ A = b.A[m];
  const double scale = b.scale[m];

  int gti[PW], gtj[PW];
  f64x4_t acc[PW];
#pragma unroll
  for (int sl = 0; sl < PW; ++sl) {
    gti[sl] = -1;
    gtj[sl] = 0;
    if (wave + kQrWaves * sl < NTT) gram_tile(wave + kQrWaves * sl, NT, gti[sl], gtj[sl]);
    acc[sl] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  }
  // The rows of A of a block are loaded into registers one block ahead:
  // every load of the next block is issued before the current block's
  // products, and stored to LDS when those are done. Rows past the end read a
  // valid row and are zeroed.
  // A block's rows are contiguous in A: thread element e is flat element
  // threadIdx.x + kQrThreads e of the block, clamped to the last valid one.
  const int q0 = (int)threadIdx.x / R, c0 = (int)threadIdx.x % R;
  double sv[NS];
  {
    const double* blk = A + gbeg * R;
    const int lim = (int)((gbeg + BR < gend ? gbeg + BR : gend) - gbeg) * R;
#pragma unroll
    for (int e = 0; e < NS; ++e) {
      const int f = (int)threadIdx.x + kQrThreads * e;
      sv[e] = blk[f < lim ? f : lim - 1];
    }
  }
  if constexpr (MODE == 1) qr_stage_u<R>(u, b.U1[m]);

  for (int64_t rbeg = gbeg; rbeg < gend; rbeg += BR) {
    const int64_t rend = rbeg + BR < gend ? rbeg + BR : gend;
    qr_lds_barrier();  // the previous block's readers of rows (and u) are done
    if constexpr (MODE == 2) qr_stage_u<R>(u, b.U1[m]);
    {
      const int lim = (int)(rend - rbeg) * R;
#pragma unroll
      for (int e = 0; e < NS; ++e) {
        int lr, c;
        qr_flat_split<R>(q0, c0, e, lr, c);
        rows[lr * LA + c] = (int)threadIdx.x + kQrThreads * e < lim ? sv[e] : 0.0;
      }
    }
    if (rbeg + BR < gend) {
      const int64_t nbeg = rbeg + BR, nend = nbeg + BR < gend ? nbeg + BR : gend;
      const double* blk = A + nbeg * R;
      const int lim = (int)(nend - nbeg) * R;
#pragma unroll
      for (int e = 0; e < NS; ++e) {
        const int f = (int)threadIdx.x + kQrThreads * e;
        sv[e] = blk[f < lim ? f : lim - 1];
      }
    }
    qr_lds_barrier();
    if constexpr (MODE != 0) {
      // Q1 rows = A rows U1: row tile wr, the column tiles of parity wh
      f64x4_t y[NY];
      if (wh == 0)
        qr_multiply<R, 0>(rows, u, wr, li, lg, y);
      else
        qr_multiply<R, 1>(rows, u, wr, li, lg, y);
      if constexpr (MODE == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t row = rbeg + 16 * wr + 4 * i + lg;
          if (row >= rend) continue;
#pragma unroll
          for (int j = 0; j < NY; ++j) {
            const int tc = 2 * j + wh;
            if (tc < NT) b.P[m][row * R + 16 * tc + li] = (uint16_t)f32_to_bf16_rne((float)(scale * y[j][i]));
          }
        }
      }
      qr_lds_barrier();  // every wave is done reading the staged rows (and U1)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NY; ++j) {  // 0 past the end; MODE 2 multiplies it again, MODE 1 takes its Gram
          const int tc = 2 * j + wh;
          if (tc < NT) rows[(16 * wr + 4 * i + lg) * (MODE == 2 ? LM : LG) + 16 * tc + li] = y[j][i];
        }
      if constexpr (MODE == 2) qr_stage_u<R>(u, b.U2[m]);
      qr_lds_barrier();
      if constexpr (MODE == 2) {
        // P rows = scale * Q1 rows U2
        if (wh == 0)
          qr_multiply<R, 0>(rows, u, wr, li, lg, y);
        else
          qr_multiply<R, 1>(rows, u, wr, li, lg, y);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t row = rbeg + 16 * wr + 4 * i + lg;
          if (row >= rend) continue;
#pragma unroll
          for (int j = 0; j < NY; ++j) {
            const int tc = 2 * j + wh;
            if (tc < NT) b.P[m][row * R + 16 * tc + li] = (uint16_t)f32_to_bf16_rne((float)(scale * y[j][i]));
          }
        }
      }
    }
    if constexpr (MODE != 2) {
      // the block's rows into this wave's upper-triangle Gram tiles
#pragma unroll 4
      for (int kk = 0; kk < BR / 4; ++kk)
#pragma unroll
        for (int sl = 0; sl < PW; ++sl)
          if (gti[sl] >= 0)
            acc[sl] = __builtin_amdgcn_mfma_f64_16x16x4f64(rows[(4 * kk + lg) * LG + 16 * gti[sl] + li],
                                                           rows[(4 * kk + lg) * LG + 16 * gtj[sl] + li], acc[sl], 0,
                                                           0, 0);
    }
  }
  if constexpr (MODE != 2) {
    double* out = b.part[m] + (int64_t)(blockIdx.x - b.block_begin[m]) * R * R;
#pragma unroll
    for (int sl = 0; sl < PW; ++sl) {
      if (gti[sl] < 0) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) out[(16 * gti[sl] + 4 * i + lg) * R + 16 * gtj[sl] + li] = acc[sl][i];
    }
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

// Blocked U = chol(G)^-1 for R = 16 NT (ranks 16 .. 128), one workgroup of
// four waves per matrix, the upper 16 x 16 tiles of G in LDS. With G = R^T R
// (R upper triangular) and V_pp = R_pp^-1, for each block step p:
//   diagonal  V_pp = chol(G_pp)^-1 of the current (Schur-complemented) G_pp,
//             one wave, by eliminating [G_pp | I] as the unblocked factor
//             does (lane (g, i): column i, rows g + 4 t);
//   panel     R_pq = V_pp^T G_pq for q > p (fp64 MFMA);
//   update    G_qq' -= R_pq^T R_pq' for p < q <= q' (fp64 MFMA).
// Then U = R^-1 by block columns, each within one wave: U_qq = V_qq and
// U_pq = -V_pp sum_{p < s <= q} R_ps U_sq for p = q - 1 .. 0, the U tiles
// kept in registers in the MFMA result layout, which is also the layout of
// a B operand. Only the diagonal steps are serial (16 pivots of one wave each);
// the rest is 16 x 16 x 16 products. A pivot that is not positive and finite
// makes the whole U NaN, as in the unblocked factor.
constexpr int kFacPitch = 18;  // doubles per row of an LDS tile (reads of 16 rows x 4 columns hit distinct banks)
constexpr int kFacTile = 16 * kFacPitch;

template <int R>
__global__ __launch_bounds__(256) void qr_factor_blocked_kernel(QrBatch b, const double* __restrict__ G_all,
                                                                int second) {
  static_assert(R % 16 == 0 && R <= 128, "tiled ranks");
  constexpr int NT = R / 16, NTT = NT * (NT + 1) / 2;
  __shared__ double gt[NTT * kFacTile];  // upper tiles of G, then of R
  __shared__ double vt[NT * kFacTile];   // V_pp per diagonal block
  __shared__ double yt[kFacTile];        // a diagonal step's L^-1, read transposed
  __shared__ double dd[16];              // a diagonal step's pivots
  __shared__ int fail_s;
  const int m = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
  const int li = lane & 15, lg = lane >> 4;
  double* U = second ? b.U2[m] : b.U1[m];
  const double* G = G_all + (int64_t)m * R * R;

  constexpr int NE = R * R / 256;  // elements of G per thread (element tid + 256 e)
  if (second) {
    // G2 = I + E (see the unblocked factor): U2 = I - S when every |E| < 1e-7.
    // Every load is issued before the first is used.
    double gv[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) gv[e] = G[tid + 256 * e];
    bool far = false, above_final = false;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int l = (tid + 256 * e) / R, c = (tid + 256 * e) % R;
      if (c < l) continue;
      const double err = fabs(gv[e] - (c == l ? 1.0 : 0.0));
      far = far || !(err < 1e-7);
      above_final = above_final || !(err < kQrFinalTol);
    }
    const bool keep_first = !__syncthreads_or(above_final);
    if (!__syncthreads_or(far)) {
      if (tid == 0) {
        b.status[m][1] = 0u;
        b.status[m][2] = keep_first ? 1u : 0u;
      }
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int l = (tid + 256 * e) / R, c = (tid + 256 * e) % R;
        const double a = gv[e];
        U[tid + 256 * e] = c < l ? 0.0 : (c == l ? 1.0 - 0.5 * (a - 1.0) : -a);
      }
      return;
    }
  }

  // the upper tiles of G (its lower triangle is not summed: diagonal tiles are
  // mirrored), every load issued before the first LDS store
  {
    double gv[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int l = (tid + 256 * e) / R, c = (tid + 256 * e) % R;
      gv[e] = G[c >= l ? l * R + c : c * R + l];
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int l = (tid + 256 * e) / R, c = (tid + 256 * e) % R;
      if (l / 16 <= c / 16) gt[utile_slot(l / 16, c / 16) * kFacTile + (l % 16) * kFacPitch + c % 16] = gv[e];
    }
  }
  if (tid == 0) fail_s = 0;
  __syncthreads();

  for (int p = 0; p < NT; ++p) {
    if (wave == 0) {
      // V_pp from the current G_pp: lane holds column li of rows lg + 4 t
      double* tp = gt + utile_slot(p, p) * kFacTile;
      double x[4], y[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        x[t] = tp[(lg + 4 * t) * kFacPitch + li];
        y[t] = lg + 4 * t == li ? 1.0 : 0.0;
      }
      bool bad = false;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const double piv = __shfl(x[k / 4], 16 * (k % 4) + k);
        bad = bad || !(piv > 0.0 && isfinite(piv));
        const double inv = 1.0 / piv;
        const double bk = __shfl(x[k / 4], 16 * (k % 4) + li);  // pivot row, column li
        const double yk = __shfl(y[k / 4], 16 * (k % 4) + li);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const double bik = __shfl(x[t], 16 * lg + k);  // row lg + 4 t, pivot column
          if (lg + 4 * t > k) {
            const double f = bik * inv;
            x[t] -= f * bk;
            y[t] -= f * yk;
          }
        }
      }
      // V = L^-T D^-1/2: V[i][j] = L^-1[j][i] / sqrt(D_j) for i <= j
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        yt[(lg + 4 * t) * kFacPitch + li] = y[t];
        if (lg + 4 * t == li) dd[li] = x[t];
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
      double* vp = vt + p * kFacTile;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int i = lg + 4 * t;
        vp[i * kFacPitch + li] = i <= li ? yt[li * kFacPitch + i] / sqrt(dd[li]) : 0.0;
      }
      if (bad && lane == 0) fail_s = 1;
    }
    __syncthreads();
    // panel: R_pq = V_pp^T G_pq, tile q by wave (q - p - 1) % 4
    for (int q = p + 1 + wave; q < NT; q += 4) {
      double* tq = gt + utile_slot(p, q) * kFacTile;
      const double* vp = vt + p * kFacTile;
      f64x4_t acc = f64x4_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(vp[(4 * kk + lg) * kFacPitch + li],
                                                    tq[(4 * kk + lg) * kFacPitch + li], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) tq[(4 * i + lg) * kFacPitch + li] = acc[i];
    }
    __syncthreads();
    // update: G_qq' -= R_pq^T R_pq' over the upper tiles of the trailing block
    const int nt2 = NT - p - 1;
    for (int t = wave; t < nt2 * (nt2 + 1) / 2; t += 4) {
      int a_, b_;
      gram_tile(t, nt2, a_, b_);
      const int q = p + 1 + a_, q2 = p + 1 + b_;
      double* tc = gt + utile_slot(q, q2) * kFacTile;
      const double* ra = gt + utile_slot(p, q) * kFacTile;
      const double* rb = gt + utile_slot(p, q2) * kFacTile;
      f64x4_t acc;
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = tc[(4 * i + lg) * kFacPitch + li];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(-ra[(4 * kk + lg) * kFacPitch + li],
                                                    rb[(4 * kk + lg) * kFacPitch + li], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) tc[(4 * i + lg) * kFacPitch + li] = acc[i];
    }
    __syncthreads();
  }

  if (fail_s) {
    const double nan = __builtin_nan("");
    for (int e = tid; e < R * R; e += 256) U[e] = nan;
    if (tid == 0) {
      b.status[m][second] = 1u;
      if (second) b.status[m][2] = 0u;
    }
    return;
  }
  if (tid == 0) {
    b.status[m][second] = 0u;
    if (second) b.status[m][2] = 0u;
  }
  // U by block columns: column q by wave q % 4
  static_for<0, NT>([&](auto qc) {
    constexpr int q = decltype(qc)::value;
    if (q % 4 != wave) return;
    f64x4_t ures[q + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) ures[q][i] = vt[q * kFacTile + (4 * i + lg) * kFacPitch + li];
    static_for<0, q>([&](auto pc) {
      constexpr int p = q - 1 - decltype(pc)::value;
      f64x4_t sacc = f64x4_t{0.0, 0.0, 0.0, 0.0};
      static_for<p + 1, q + 1>([&](auto sc) {
        constexpr int s2 = decltype(sc)::value;
        const double* rp = gt + utile_slot(p, s2) * kFacTile;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          sacc = __builtin_amdgcn_mfma_f64_16x16x4f64(rp[li * kFacPitch + 4 * kk + lg], ures[s2][kk], sacc, 0, 0, 0);
      });
      f64x4_t r = f64x4_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        r = __builtin_amdgcn_mfma_f64_16x16x4f64(-vt[p * kFacTile + li * kFacPitch + 4 * kk + lg], sacc[kk], r, 0, 0,
                                                 0);
      ures[p] = r;
    });
#pragma unroll
    for (int p = 0; p < NT; ++p)
#pragma unroll
      for (int i = 0; i < 4; ++i) U[(16 * p + 4 * i + lg) * R + 16 * q + li] = p <= q ? ures[p <= q ? p : q][i] : 0.0;
  });
}

namespace {

struct QrItemLayout {
  size_t a, q1, part, u1, u2, status, total;
  int blocks;
};

QrItemLayout qr_item_layout(int64_t k, int64_t r) {
  QrItemLayout l;
  l.blocks = (int)((k + qr_group_rows(r) - 1) / qr_group_rows(r));  // workgroups of a block step
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += (bytes + 255) / 256 * 256;
    return at;
  };
  l.a = take((size_t)k * r * sizeof(double));
  l.q1 = take(r < 16 ? (size_t)k * r * sizeof(double) : 0);  // the small-rank steps keep Q1
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
      hipLaunchKernelGGL((qr_block_mfma_kernel<R, MODE>), blocks, dim3(kQrThreads), 0, s, b);
  };
  if constexpr (R >= 16) {
    int64_t kmax = 0;
    for (int m = 0; m < n; ++m) kmax = ks[m] > kmax ? ks[m] : kmax;
    hipLaunchKernelGGL((qr_gauss_kernel<R>), dim3((unsigned)((kmax * (R / 4) + 255) / 256), (unsigned)n), dim3(256),
                       0, s, b);
  }
  auto factor = [&](int second) {
    if constexpr (R < 16)
      hipLaunchKernelGGL((qr_factor_kernel<R>), dim3(n), dim3(QrFactorShape<R>::THREADS), 0, s, b, G_all, second);
    else
      hipLaunchKernelGGL((qr_factor_blocked_kernel<R>), dim3(n), dim3(256), 0, s, b, G_all, second);
  };
  block_step(IntC<0>{});
  hipLaunchKernelGGL((qr_gram_reduce_kernel<R>), red_grid, dim3(256), 0, s, b, G_all);
  factor(0);
  block_step(IntC<1>{});
  hipLaunchKernelGGL((qr_gram_reduce_kernel<R>), red_grid, dim3(256), 0, s, b, G_all);
  factor(1);
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
