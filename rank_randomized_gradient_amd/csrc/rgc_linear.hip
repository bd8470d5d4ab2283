// The layer's own products either side of the sketch, on bf16 MFMA with fp32
// sums and one rounding to bf16 per output element:
//   forward:  [Y | XP] = X [W^T | P]    Y = bf16(X W^T): T x d, XP = bf16(X P): T x r
//   backward: dX = bf16(D W)            T x k; then C += D^T XP (the sketch accumulate)
// ([RGC, "How it works"] = page "Randomized Gradient Compression": the layer
// keeps X P instead of X, and D^T (X P) is what the backward adds to the
// sketch. [LoGRA-M, "Minimal Causal Code"] = page "LoGRA: Low-Rank Gradient
// Sketches": the projection belongs inside the layer's own weight-gradient
// products rather than in a pass of its own.)
//
// One kernel serves both directions: out = A B over K, A: M x K with K
// contiguous (X or D, M = tokens), B either N x K with K contiguous (W in the
// forward: its rows are Y's columns) or K x N with N contiguous (W in the
// backward, where K = d). In the forward, P's r columns ride along: the first
// r / 16 tiles of each tile row also make a 16-column slice of XP from the X
// fragments they already hold (two more MFMAs per 32), so the projection
// adds no pass over X and no tiles of its own. (Where a tile would have to
// carry more than two slices, or r is 8, P's columns are instead one more
// column of tiles of the same grid.)
//
// * A workgroup tile is 256 x 256 outputs; its eight waves (two per SIMD, so
//   that one wave's LDS reads overlap the other's MFMAs) split it 2 x 4, each
//   multiplying a 128 x 64 block with 16x16x32 MFMAs.
// * A K-step is 32 rows of K. The step's A slab (256 x 32), B slab (256 x 32
//   or 32 x 256) and P slices (32 x 16 each) are copied from memory straight
//   into an LDS stage in 1 KB copies that do not pass through VGPRs; four
//   stages, copies running three steps ahead of the step that multiplies.
// * Operands with K contiguous sit in LDS as rows of 64 bytes (four 16-byte
//   chunks) whose chunks are rotated by the row index, so the 16-byte reads
//   of 8 consecutive rows touch distinct bank groups; K-major operands sit as
//   blocks of 4 K rows x 16 columns and are read with transposing LDS reads.
// * The MFMA takes B's fragment on its M side and A's on its N side, so each
//   lane ends with four consecutive output columns of one row: one 8-byte
//   store per 16 x 16 block.
// * Tiles walk groups of 8 M tiles down an N column before moving right, and
//   consecutive tiles go to the same XCD, so the tiles running on one XCD share
//   their A and B slabs through its L2.
// * Each output element is one fp32 sum over K in ascending order: results
//   are bit-reproducible and independent of the launch shape.
#include "rgc_internal.hpp"

namespace rgc {
namespace {

constexpr int kLinTile = 256;        // M and N extent of a workgroup tile
constexpr int kLinKs = 32;           // K rows per step
constexpr int kLinStages = 4;
constexpr int kLinSlab = 16384;      // one operand's slab of a stage
constexpr int kLinSlices = 2;        // XP slices a tile can carry
constexpr int kLinStage = 2 * kLinSlab + 1024 * kLinSlices;  // A slab, B slab, P slices
constexpr int kLinThreads = 512;     // eight waves, two per SIMD
constexpr int kLinGroupRows = 8;     // M tiles walked together
constexpr int kLinMaxItems = 16;
constexpr int kNumXcdsLin = 8;

struct LinItem {
  const uint16_t* A;  // M x K, row stride lda
  int64_t lda;
  const uint16_t* B0;  // segment 0 operand: N0 x K (row stride ldb0) or K x N0 (row stride ldb0)
  int64_t ldb0;
  uint16_t* O0;  // M x N0, row stride ldo0
  int64_t ldo0;
  int64_t N0;
  const uint16_t* B1;  // segment 1 (K x N1, row stride N1), or null
  uint16_t* O1;        // M x N1, row stride N1
  int64_t N1;
  int64_t K;
  const uint16_t* Ps;  // P (K x R) computed as 16-column slices inside segment 0's tiles, or null
  uint16_t* XPs;       // M x R, row stride R
  int64_t R;
};

struct LinBatch {
  int n;
  int64_t M;
  int64_t mtiles;
  int64_t tbase[kLinMaxItems + 1];  // first tile of each item
  int64_t nt0[kLinMaxItems];        // N tiles of segment 0
  int64_t nt[kLinMaxItems];         // N tiles of the item
  LinItem it[kLinMaxItems];
};

__device__ __forceinline__ int64_t lin_window_base(int64_t k0, int64_t end) {
  return k0 + kLinKs <= end ? k0 : (end >= kLinKs ? end - kLinKs : 0);
}

// The hardware hands workgroups to the XCDs round-robin; this numbers them
// so that each XCD gets a contiguous run of tiles.
__device__ __forceinline__ int64_t lin_logical(int64_t b, int64_t G) {
  const int64_t x = b % kNumXcdsLin, pos = b / kNumXcdsLin;
  const int64_t q = G / kNumXcdsLin, rem = G % kNumXcdsLin;
  return x * q + (x < rem ? x : rem) + pos;
}

// K-contiguous slab: copy c (1 KB) holds rows 16c .. 16c+15, 64 bytes (four
// 16-byte chunks of 8 K values) each; chunk q of row t sits at slot
// (q + t / 2) % 4 of its row, so the 16-byte reads of 8 consecutive rows at
// one chunk touch 8 distinct bank groups.
__device__ __forceinline__ int rowslab_offset(int rho, int q) {
  const int c = rho >> 4, t = rho & 15;
  return 1024 * c + 16 * (4 * t + ((q + (t >> 1)) & 3));
}

// The last step of a K extent that is not a multiple of 32 multiplies a
// window whose K offsets outside [lo, hi) are not its own (rows of the step
// before, or re-read copies of the last row): they are set to zero in both
// slabs of the stage, so that they add nothing (an Inf or NaN there would
// otherwise still count). K-contiguous slab: 16-byte granule p = 64c + 4t + s
// holds chunk (s - t / 2) % 4 of row t of copy c; K-major slab: granule p
// holds half of K row 4 (p / 128) + (p % 8) / 2 of a block.
template <bool BKM, int NSL>
__device__ __forceinline__ void zero_stale_k(RGC_LDS char* stage, int lo, int hi) {
  if (NSL > 0 && (int)threadIdx.x < 64 * NSL) {  // P slices: K-major blocks
    const int p = threadIdx.x, kb = 4 * ((p >> 3) & 7) + ((p & 7) >> 1);
    if (kb < lo || kb >= hi) *(RGC_LDS u32x4v_t*)(stage + 2 * kLinSlab + 16 * p) = u32x4v_t{0u, 0u, 0u, 0u};
  }
  for (int p = threadIdx.x; p < 1024; p += kLinThreads) {
    const int t = (p >> 2) & 15, s = p & 3;
    const int kq = 8 * ((s - (t >> 1)) & 3);
    if (kq < lo || kq >= hi) *(RGC_LDS u32x4v_t*)(stage + 16 * p) = u32x4v_t{0u, 0u, 0u, 0u};
    int kb = kq;
    if constexpr (BKM) kb = 4 * (p >> 7) + ((p & 7) >> 1);
    if (kb < lo || kb >= hi) *(RGC_LDS u32x4v_t*)(stage + kLinSlab + 16 * p) = u32x4v_t{0u, 0u, 0u, 0u};
  }
}

// One tile: out[m0 .. m0+255][n0 .. n0+255] of A (rows m0.., K contiguous)
// times B (BKM: K x N, N contiguous; else N x K, K contiguous). Eight waves:
// wave (wm, wn) multiplies rows 128 wm .. +127 by columns 64 wn .. +63.
//
// NSL > 0: the tile also makes NSL 16-column slices of XP = A P (columns
// 16 sl[q] .. +15, P: K x R), from the A fragments it already holds: wave
// (wm, wn) takes rows 128 wm + 32 wn .. +31 of each slice (two more MFMAs per
// 32). Wave q < NSL copies slice q's 1 KB of P per stage.
template <bool BKM, int NSL>
__device__ __forceinline__ void lin_tile(const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B,
                                         int64_t ldb, uint16_t* __restrict__ O, int64_t ldo, int64_t m_rem,
                                         int64_t n_rem, int64_t K, char* smem, const uint16_t* __restrict__ P = nullptr,
                                         uint16_t* __restrict__ XP = nullptr, int64_t R = 0, int sl0 = 0,
                                         int sl1 = 0) {
  constexpr int S = kLinStages;
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int wm = wave & 1, wn = wave >> 1;
  const int g = lane >> 4, li = lane & 15;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(RGC_LDS char*)smem;
  const int64_t rows_k = K >= kLinKs ? kLinKs : K;  // K rows of a window that are valid memory

  // Per-lane offsets of the wave's 4 copies per stage (copies c = wave + 8v:
  // v < 2 fill the A slab, v >= 2 the B slab).
  uint32_t voff[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int c = (wave + 8 * v) & 15;
    if (v < 2 || !BKM) {
      const int t = lane >> 2;
      const int q = ((lane & 3) - (t >> 1)) & 3;  // chunk whose bytes land at 16 * lane
      int64_t row = 16 * c + t;
      const int64_t rmax = (v < 2 ? m_rem : n_rem) - 1;  // rows past the end re-read the last one (never stored)
      row = row < rmax ? row : rmax;
      int64_t kc = 8 * q;
      kc = kc + 8 <= rows_k ? kc : rows_k - 8;
      voff[v] = (uint32_t)((row * (v < 2 ? lda : ldb) + kc) * 2);
    } else {
      const int blk = 8 * c + (lane >> 3);  // block (kq, b) = (blk / 16, blk % 16)
      int64_t kr = 4 * (blk >> 4) + ((lane & 7) >> 1);
      kr = kr < rows_k ? kr : rows_k - 1;
      int64_t col = 16 * (blk & 15) + 8 * (lane & 1);
      col = col + 8 <= n_rem ? col : n_rem - 8;  // past N: a valid chunk (never stored)
      voff[v] = (uint32_t)((kr * ldb + col) * 2);
    }
  }

  // the slice copy of wave q < NSL: lane l reads K row 4 (l / 8) + (l % 8) / 2,
  // columns 16 sl[q] + 8 (l % 2) .. +7 (block l / 8 of the slice)
  const bool slicer = wave < NSL;
  uint32_t voff_p = 0;
  if (NSL > 0) {
    int64_t kr = 4 * (lane >> 3) + ((lane & 7) >> 1);
    kr = kr < rows_k ? kr : rows_k - 1;
    voff_p = (uint32_t)((kr * R + 16 * (wave == 0 ? sl0 : sl1) + 8 * (lane & 1)) * 2);
  }

  const int64_t nsteps = (K + kLinKs - 1) / kLinKs;
  auto issue = [&](int64_t step) {
    const int64_t wb = lin_window_base(step * kLinKs, K);
    const uint16_t* Ab = uniform_ptr(A + wb);
    const uint16_t* Bb = uniform_ptr(BKM ? B + wb * ldb : B + wb);
    const uint32_t st = lds0 + (uint32_t)(step % S) * kLinStage;
#pragma unroll
    for (int v = 0; v < 4; ++v) dma_16b_cached(v < 2 ? Ab : Bb, voff[v], st + 1024 * (wave + 8 * v));
    if (NSL > 0 && slicer) dma_16b_cached(uniform_ptr(P + wb * R), voff_p, st + 2 * kLinSlab + 1024 * wave);
  };

  // A wave with no rows (or, carrying no slices, no columns) of its part
  // inside the tile only copies.
  const bool idle = 128 * wm >= m_rem || (NSL == 0 && 64 * wn >= n_rem);
  f32x4_t acc[8][4];
  f32x4_t accx[NSL > 0 ? NSL : 1][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < (NSL > 0 ? NSL : 1); ++q) accx[q][0] = accx[q][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < S - 1; ++s)
    if (s < nsteps) issue(s);
  for (int64_t step = 0; step < nsteps; ++step) {
    // this step's copies are done once at most the later steps' are pending
    if (step + S - 2 < nsteps) {
      if (NSL > 0 && slicer)
        wait_vmcnt<5 * (S - 2)>();
      else
        wait_vmcnt<4 * (S - 2)>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    RGC_LDS char* st = (RGC_LDS char*)smem + (step % S) * kLinStage;
    const int64_t k0 = step * kLinKs;
    if (k0 + kLinKs > K) {
      const int64_t wb = lin_window_base(k0, K);
      zero_stale_k<BKM, NSL>(st, (int)(k0 - wb), (int)(K - wb));
      lds_barrier();
    }
    // refill the stage every wave finished reading in the previous step
    if (step + S - 1 < nsteps) issue(step + S - 1);
    if (idle) continue;
    const RGC_LDS char* sa = st;
    const RGC_LDS char* sb = st + kLinSlab;
    uint32_t a[8][4], b[4][4];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const u32x4v_t v = *(const RGC_LDS u32x4v_t*)(sa + rowslab_offset(128 * wm + 16 * mt + li, g));
      a[mt][0] = v.x;
      a[mt][1] = v.y;
      a[mt][2] = v.z;
      a[mt][3] = v.w;
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      if constexpr (BKM) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x2v_t v = lds_read_tr16(sb + 128 * ((2 * g + h) * 16 + 4 * wn + nt) + 8 * li);
          b[nt][2 * h] = v.x;
          b[nt][2 * h + 1] = v.y;
        }
      } else {
        const u32x4v_t v = *(const RGC_LDS u32x4v_t*)(sb + rowslab_offset(64 * wn + 16 * nt + li, g));
        b[nt][0] = v.x;
        b[nt][1] = v.y;
        b[nt][2] = v.z;
        b[nt][3] = v.w;
      }
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_16x16x32(b[nt], a[mt], acc[mt][nt]);
#pragma unroll
    for (int q = 0; q < NSL; ++q) {
      uint32_t bp[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x2v_t v = lds_read_tr16(st + 2 * kLinSlab + 1024 * q + 128 * (2 * g + h) + 8 * li);
        bp[2 * h] = v.x;
        bp[2 * h + 1] = v.y;
      }
      // rows 128 wm + 32 wn + 16 u + li are A fragment 2 wn + u of this wave
#pragma unroll
      for (int u = 0; u < 2; ++u) accx[q][u] = mfma_16x16x32(bp, a[2 * wn + u], accx[q][u]);
    }
  }
  if (idle) return;

#pragma unroll
  for (int q = 0; q < NSL; ++q) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t row = 128 * wm + 32 * wn + 16 * u + li;
      if (row >= m_rem) continue;
      const f32x4_t v = accx[q][u];
      *reinterpret_cast<uint2*>(XP + row * R + 16 * (q == 0 ? sl0 : sl1) + 4 * g) =
          make_uint2(f32x2_to_bf16x2_rne(v[0], v[1]),
                     f32x2_to_bf16x2_rne(v[2], v[3]));
    }
  }

  // lane (li, g) holds out[128 wm + 16 mt + li][64 wn + 16 nt + 4 g + e], e = 0..3
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const int64_t row = 128 * wm + 16 * mt + li;
    if (row >= m_rem) continue;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t col = 64 * wn + 16 * nt + 4 * g;
      if (col >= n_rem) continue;  // n_rem is a multiple of 8: four columns are all in or all out
      const f32x4_t v = acc[mt][nt];
      *reinterpret_cast<uint2*>(O + row * ldo + col) =
          make_uint2(f32x2_to_bf16x2_rne(v[0], v[1]),
                     f32x2_to_bf16x2_rne(v[2], v[3]));
    }
  }
}

// Tile t of the batch: item m, M tile i, N tile j (segment 0 first, then
// segment 1). Within an item, tiles walk groups of kLinGroupRows M tiles down
// each N column.
template <bool B0KM>
__global__ __launch_bounds__(kLinThreads, 1) void linear_kernel(LinBatch lb) {
  __shared__ __attribute__((aligned(1024))) char smem[kLinStages * kLinStage];
  const int64_t t = lin_logical(blockIdx.x, gridDim.x);
  int m = 0;
  while (m + 1 < lb.n && t >= lb.tbase[m + 1]) ++m;
  const LinItem& it = lb.it[m];
  const int64_t lt = t - lb.tbase[m];
  const int64_t NT = lb.nt[m];
  const int64_t grp = lt / (kLinGroupRows * NT);
  const int64_t rows = lb.mtiles - grp * kLinGroupRows < kLinGroupRows ? lb.mtiles - grp * kLinGroupRows
                                                                       : kLinGroupRows;
  const int64_t within = lt - grp * kLinGroupRows * NT;
  const int64_t j = within / rows, i = grp * kLinGroupRows + within % rows;
  const int64_t m0 = i * kLinTile;
  const uint16_t* A = it.A + m0 * it.lda;
  const int64_t nt0 = lb.nt0[m];
  if (j < nt0) {
    const int64_t n0 = j * kLinTile;
    const uint16_t* B = B0KM ? it.B0 + n0 : it.B0 + n0 * it.ldb0;
    uint16_t* O = it.O0 + m0 * it.ldo0 + n0;
    if constexpr (!B0KM) {
      // XP slices j and j + nt0 of the R / 16 (at most two per tile)
      const int64_t ns = it.Ps ? it.R / 16 : 0;
      if (j + nt0 < ns) {
        lin_tile<B0KM, 2>(A, it.lda, B, it.ldb0, O, it.ldo0, lb.M - m0, it.N0 - n0, it.K, smem, it.Ps,
                          it.XPs + m0 * it.R, it.R, (int)j, (int)(j + nt0));
        return;
      }
      if (j < ns) {
        lin_tile<B0KM, 1>(A, it.lda, B, it.ldb0, O, it.ldo0, lb.M - m0, it.N0 - n0, it.K, smem, it.Ps,
                          it.XPs + m0 * it.R, it.R, (int)j);
        return;
      }
    }
    lin_tile<B0KM, 0>(A, it.lda, B, it.ldb0, O, it.ldo0, lb.M - m0, it.N0 - n0, it.K, smem);
  } else {
    lin_tile<true, 0>(A, it.lda, it.B1, it.N1, it.O1 + m0 * it.N1, it.N1, lb.M - m0, it.N1, it.K, smem);
  }
}

rgc_status_t check_operand(const void* p, int64_t ld, int64_t width) {
  if (!p) return RGC_ERR_NULL;
  if (ld < width) return RGC_ERR_SHAPE;
  if (ld > kMaxLeadingDim) return RGC_ERR_UNSUPPORTED;
  if (!aligned16(p) || (ld % 8) != 0) return RGC_ERR_ALIGN;
  return RGC_OK;
}

rgc_status_t linear_launch(LinBatch& lb, bool b0_kmajor, hipStream_t stream) {
  lb.mtiles = (lb.M + kLinTile - 1) / kLinTile;
  lb.tbase[0] = 0;
  for (int m = 0; m < lb.n; ++m) {
    lb.nt0[m] = (lb.it[m].N0 + kLinTile - 1) / kLinTile;
    lb.nt[m] = lb.nt0[m] + (lb.it[m].B1 ? 1 : 0);
    lb.tbase[m + 1] = lb.tbase[m] + lb.mtiles * lb.nt[m];
  }
  const int64_t tiles = lb.tbase[lb.n];
  if (tiles == 0) return RGC_OK;
  if (tiles > INT32_MAX) return RGC_ERR_UNSUPPORTED;
  if (b0_kmajor)
    hipLaunchKernelGGL(linear_kernel<true>, dim3((unsigned)tiles), dim3(kLinThreads), 0, stream, lb);
  else
    hipLaunchKernelGGL(linear_kernel<false>, dim3((unsigned)tiles), dim3(kLinThreads), 0, stream, lb);
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

bool linear_rank_ok(int64_t r) { return r == 0 || rank_supported(r); }

rgc_status_t forward_batch_impl(int64_t n, const uint16_t* const* Xs, const int64_t* ldxs, const int64_t* ks,
                                const uint16_t* const* Ws, const int64_t* ldws, const int64_t* ds,
                                const uint16_t* const* Ps, uint16_t* const* Ys, const int64_t* ldys,
                                uint16_t* const* XPs, int64_t T, int64_t r, void* stream) {
  if (n < 0 || T < 0 || r < 0) return RGC_ERR_SHAPE;
  if (n > kLinMaxItems || !linear_rank_ok(r) || T > kMaxTiledDim) return RGC_ERR_UNSUPPORTED;
  if (n == 0 || T == 0) return RGC_OK;
  if (!Xs || !ldxs || !ks || !Ws || !ldws || !ds || !Ys || !ldys || (r > 0 && (!Ps || !XPs))) return RGC_ERR_NULL;
  LinBatch lb{};
  lb.n = (int)n;
  lb.M = T;
  for (int64_t m = 0; m < n; ++m) {
    const int64_t k = ks[m], d = ds[m];
    if (k <= 0 || d <= 0 || r > k) return RGC_ERR_SHAPE;
    if ((k % 8) != 0 || (d % 8) != 0) return RGC_ERR_UNSUPPORTED;
    rgc_status_t st = check_operand(Xs[m], ldxs[m], k);
    if (st == RGC_OK) st = check_operand(Ws[m], ldws[m], k);
    if (st == RGC_OK) st = check_operand(Ys[m], ldys[m], d);
    // (rank 4's P and XP are checked by the small-rank project that makes XP)
    if (st == RGC_OK && r >= 8) st = check_operand(Ps[m], r, r);
    if (st == RGC_OK && r >= 8) st = check_operand(XPs[m], r, r);
    if (st == RGC_OK && r == 4 && (!Ps[m] || !XPs[m])) st = RGC_ERR_NULL;
    if (st != RGC_OK) return st;
    LinItem& it = lb.it[m];
    it.A = Xs[m];
    it.lda = ldxs[m];
    it.B0 = Ws[m];
    it.ldb0 = ldws[m];
    it.O0 = Ys[m];
    it.ldo0 = ldys[m];
    it.N0 = d;
    it.K = k;
    // XP as 16-column slices inside the tiles of Y when r is a multiple of 16
    // and no tile carries more than two; else one more column of tiles
    // (r = 8, or narrow d), and at rank 4 (narrower than a 16-byte chunk of
    // P) from the small-rank project after the tile grid
    const int64_t nt0 = (d + kLinTile - 1) / kLinTile;
    const bool slices = r % 16 == 0 && r > 0 && r / 16 <= kLinSlices * nt0;
    it.Ps = slices ? Ps[m] : nullptr;
    it.XPs = slices ? XPs[m] : nullptr;
    it.R = slices ? r : 0;
    it.B1 = !slices && r >= 8 ? Ps[m] : nullptr;
    it.O1 = !slices && r >= 8 ? XPs[m] : nullptr;
    it.N1 = !slices && r >= 8 ? r : 0;
  }
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  rgc_status_t st = linear_launch(lb, false, hs);
  if (st == RGC_OK && r == 4)
    st = rgc_project_batch(n, Xs, ldxs, ks, Ps, XPs, T, r, nullptr, 0, stream);
  return st;
}

}  // namespace
}  // namespace rgc

using namespace rgc;

extern "C" rgc_status_t rgc_linear_forward_batch(int64_t n, const uint16_t* const* Xs, const int64_t* ldxs,
                                                 const int64_t* ks, const uint16_t* const* Ws, const int64_t* ldws,
                                                 const int64_t* ds, const uint16_t* const* Ps, uint16_t* const* Ys,
                                                 const int64_t* ldys, uint16_t* const* XPs, int64_t T, int64_t r,
                                                 void* stream) {
  return forward_batch_impl(n, Xs, ldxs, ks, Ws, ldws, ds, Ps, Ys, ldys, XPs, T, r, stream);
}

extern "C" rgc_status_t rgc_linear_forward(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw,
                                           const uint16_t* P, uint16_t* Y, int64_t ldy, uint16_t* XP, int64_t T,
                                           int64_t d, int64_t k, int64_t r, void* stream) {
  if (T < 0 || d <= 0 || k <= 0 || r < 0) return RGC_ERR_SHAPE;
  return forward_batch_impl(1, &X, &ldx, &k, &W, &ldw, &d, &P, &Y, &ldy, &XP, T, r, stream);
}

extern "C" size_t rgc_linear_backward_workspace_size(int64_t T, int64_t d, int64_t k, int64_t r) {
  (void)k;
  return r > 0 ? rgc_accumulate_workspace_size(T, d, r) : 0;
}

extern "C" rgc_status_t rgc_linear_backward(const uint16_t* D, int64_t ldd, const uint16_t* W, int64_t ldw,
                                            const uint16_t* XP, float* C, uint16_t* dX, int64_t lddx, int64_t T,
                                            int64_t d, int64_t k, int64_t r, void* ws, size_t ws_bytes,
                                            void* stream) {
  if (T < 0 || d <= 0 || k <= 0 || r < 0) return RGC_ERR_SHAPE;
  if (!linear_rank_ok(r) || T > kMaxTiledDim) return RGC_ERR_UNSUPPORTED;
  if ((k % 8) != 0 || (d % 8) != 0) return RGC_ERR_UNSUPPORTED;
  if (r > k) return RGC_ERR_SHAPE;
  rgc_status_t st = check_operand(D, ldd, d);
  if (st == RGC_OK) st = check_operand(W, ldw, k);
  if (st == RGC_OK) st = check_operand(dX, lddx, k);
  if (st != RGC_OK) return st;
  if (r > 0) {
    if (!XP || !C) return RGC_ERR_NULL;
    const size_t need = rgc_accumulate_workspace_size(T, d, r);
    if (need > 0 && (!ws || ws_bytes < need)) return RGC_ERR_WORKSPACE;
    if (need > 0 && !aligned_to(ws, 256)) return RGC_ERR_ALIGN;
    if (!aligned16(XP) || !aligned16(C)) return RGC_ERR_ALIGN;
  }
  if (T == 0) return RGC_OK;
  LinBatch lb{};
  lb.n = 1;
  lb.M = T;
  LinItem& it = lb.it[0];
  it.A = D;
  it.lda = ldd;
  it.B0 = W;  // K x N: d rows of k
  it.ldb0 = ldw;
  it.O0 = dX;
  it.ldo0 = lddx;
  it.N0 = k;
  it.K = d;
  st = linear_launch(lb, true, static_cast<hipStream_t>(stream));
  // the accumulate follows on the same stream, while D (just streamed by the
  // tile grid) is still in the last-level cache
  if (st == RGC_OK && r > 0) st = rgc_accumulate(D, ldd, XP, C, T, d, r, ws, ws_bytes, stream);
  return st;
}
