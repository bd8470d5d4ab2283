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
// forward: its rows are Y's columns) or K x N with N contiguous (P in the
// forward; W in the backward, where K = d). The forward's output columns are
// d columns of Y followed by r columns of XP: P's columns are one more N
// tile of the same grid, so X is staged into LDS by the same tiles that make
// Y, and the projection adds no pass over X.
//
// * A workgroup tile is 256 x 256 outputs; its four waves split it 2 x 2, so
//   each wave multiplies a 128 x 128 block with 16x16x32 MFMAs (64
//   accumulator tiles).
// * A K-step is 64 rows of K. The step's A slab (256 x 64) and B slab (256 x
//   64 or 64 x 256) are copied from memory straight into an LDS stage (64 KB)
//   by all four waves in 1 KB copies that do not pass through VGPRs; two
//   stages, so the next step's copies run while the current step multiplies.
// * Operands with K contiguous sit in LDS as rows of 128 bytes (eight 16-byte
//   chunks) whose chunks are rotated by the row index, so the 16-byte reads
//   of 8 consecutive rows touch distinct banks; K-major operands sit as blocks
//   of 4 K rows x 16 columns and are read with transposing LDS reads.
// * The MFMA takes B's fragment on its M side and A's on its N side, so each
//   lane ends with four consecutive output columns of one row: one 8-byte
//   store per tile.
// * Tiles walk groups of 8 M tiles down an N column before moving right, and
//   consecutive tiles go to the same XCD, so the tiles running on one XCD share
//   their A and B slabs through its L2.
// * Each output element is one fp32 sum over K in ascending order: results
//   are bit-reproducible and independent of the launch shape.
#include "rgc_internal.hpp"

namespace rgc {
namespace {

constexpr int kLinTile = 256;        // M and N extent of a workgroup tile
constexpr int kLinKs = 64;           // K rows per step
constexpr int kLinStage = 65536;     // one stage: A slab + B slab
constexpr int kLinSlab = 32768;
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

// Byte offset in a stage slab of 16-byte chunk q of row rho (K-contiguous
// layout): copy rho / 8 holds rows 8c .. 8c+7, row t's chunk q at slot
// (q + t + 4 (c % 2)) % 8 of the row's 128 bytes.
__device__ __forceinline__ int rowslab_offset(int rho, int q) {
  const int c = rho >> 3, t = rho & 7;
  return 1024 * c + 16 * (8 * t + ((q + t + 4 * (c & 1)) & 7));
}

// The last step of a K extent that is not a multiple of 64 multiplies a
// window whose K offsets outside [lo, hi) are not its own (rows of the step
// before, or re-read copies of the last row): they are set to zero in both
// slabs of the stage, so that they add nothing (an Inf or NaN there would
// otherwise still count). K-contiguous slab: 16-byte granule p of copy
// p / 64 holds chunk q of a row (8 K values, all inside or all outside since
// lo and hi are multiples of 8); K-major slab: granule p holds half of K row
// 4 (p / 128) + (p % 8) / 2 of a block.
template <bool BKM>
__device__ __forceinline__ void zero_stale_k(RGC_LDS char* stage, int lo, int hi) {
  for (int p = threadIdx.x; p < 2048; p += 256) {
    const int c = p >> 6, t = (p >> 3) & 7, s = p & 7;
    const int q = (s - t - 4 * (c & 1)) & 7;
    if (8 * q < lo || 8 * q >= hi) *(RGC_LDS u32x4v_t*)(stage + 16 * p) = u32x4v_t{0u, 0u, 0u, 0u};
    int kb = 8 * q;
    if constexpr (BKM) kb = 4 * (p >> 7) + ((p & 7) >> 1);
    if (kb < lo || kb >= hi) *(RGC_LDS u32x4v_t*)(stage + kLinSlab + 16 * p) = u32x4v_t{0u, 0u, 0u, 0u};
  }
}

// One tile: out[m0 .. m0+255][n0 .. n0+255] of A (rows m0.., K contiguous)
// times B (BKM: K x N, N contiguous; else N x K, K contiguous).
template <bool BKM>
__device__ __forceinline__ void lin_tile(const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B,
                                         int64_t ldb, uint16_t* __restrict__ O, int64_t ldo, int64_t m_rem,
                                         int64_t n_rem, int64_t K, char* smem) {
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int wm = wave & 1, wn = wave >> 1;
  const int g = lane >> 4, li = lane & 15;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(RGC_LDS char*)smem;
  const int64_t rows_k = K >= kLinKs ? kLinKs : K;  // K rows of a window that are valid memory

  // Per-lane offsets of the wave's 16 copies per stage (copies c = wave + 4v:
  // v < 8 fill the A slab, v >= 8 the B slab).
  uint32_t voff[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int c = (wave + 4 * v) & 31;
    if (v < 8 || !BKM) {
      const int t = lane >> 3;
      const int q = ((lane & 7) - t - 4 * (c & 1)) & 7;  // chunk whose bytes land at 16 * lane
      int64_t row = 8 * c + t;
      const int64_t rmax = (v < 8 ? m_rem : n_rem) - 1;  // rows past the end re-read the last one (never stored)
      row = row < rmax ? row : rmax;
      int64_t kc = 8 * q;
      kc = kc + 8 <= rows_k ? kc : rows_k - 8;
      voff[v] = (uint32_t)((row * (v < 8 ? lda : ldb) + kc) * 2);
    } else {
      const int blk = 8 * c + (lane >> 3);  // block (kq, b) = (blk / 16, blk % 16)
      int64_t kr = 4 * (blk >> 4) + ((lane & 7) >> 1);
      kr = kr < rows_k ? kr : rows_k - 1;
      int64_t col = 16 * (blk & 15) + 8 * (lane & 1);
      col = col + 8 <= n_rem ? col : n_rem - 8;  // past N: a valid chunk (never stored)
      voff[v] = (uint32_t)((kr * ldb + col) * 2);
    }
  }

  const int64_t nsteps = (K + kLinKs - 1) / kLinKs;
  auto issue = [&](int64_t step, int slot) {
    const int64_t wb = lin_window_base(step * kLinKs, K);
    const uint16_t* Ab = uniform_ptr(A + wb);
    const uint16_t* Bb = uniform_ptr(BKM ? B + wb * ldb : B + wb);
    const uint32_t st = lds0 + slot * kLinStage;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int c = wave + 4 * v;
      dma_16b_cached(v < 8 ? Ab : Bb, voff[v], st + 1024 * c);
    }
  };

  // A wave with no rows or no columns of its quarter inside the tile only copies.
  const bool idle = 128 * wm >= m_rem || 128 * wn >= n_rem;
  f32x4_t acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  issue(0, 0);
  int slot = 0;
  for (int64_t step = 0; step < nsteps; ++step) {
    wait_vmcnt<0>();
    lds_barrier();
    const int64_t k0 = step * kLinKs;
    if (k0 + kLinKs > K) {
      const int64_t wb = lin_window_base(k0, K);
      zero_stale_k<BKM>((RGC_LDS char*)smem + slot * kLinStage, (int)(k0 - wb), (int)(K - wb));
      lds_barrier();
    }
    if (step + 1 < nsteps) issue(step + 1, slot ^ 1);
    const RGC_LDS char* sa = (const RGC_LDS char*)smem + slot * kLinStage;
    const RGC_LDS char* sb = sa + kLinSlab;
    slot ^= 1;
    if (idle) continue;
    // the two K-halves of the step, not unrolled: unrolled, both halves'
    // operands are live at once and the accumulators spill
#pragma unroll 1
    for (int kh = 0; kh < 2; ++kh) {
      uint32_t a[8][4], b[8][4];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const u32x4v_t v = *(const RGC_LDS u32x4v_t*)(sa + rowslab_offset(128 * wm + 16 * mt + li, 4 * kh + g));
        a[mt][0] = v.x;
        a[mt][1] = v.y;
        a[mt][2] = v.z;
        a[mt][3] = v.w;
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        if constexpr (BKM) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const u32x2v_t v = lds_read_tr16(sb + 128 * ((8 * kh + 2 * g + h) * 16 + 8 * wn + nt) + 8 * li);
            b[nt][2 * h] = v.x;
            b[nt][2 * h + 1] = v.y;
          }
        } else {
          const u32x4v_t v = *(const RGC_LDS u32x4v_t*)(sb + rowslab_offset(128 * wn + 16 * nt + li, 4 * kh + g));
          b[nt][0] = v.x;
          b[nt][1] = v.y;
          b[nt][2] = v.z;
          b[nt][3] = v.w;
        }
      }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = mfma_16x16x32(b[nt], a[mt], acc[mt][nt]);
    }
  }
  if (idle) return;

  // lane (li, g) holds out[128 wm + 16 mt + li][128 wn + 16 nt + 4 g + e], e = 0..3
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const int64_t row = 128 * wm + 16 * mt + li;
    if (row >= m_rem) continue;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int64_t col = 128 * wn + 16 * nt + 4 * g;
      if (col >= n_rem) continue;  // n_rem is a multiple of 8: four columns are all in or all out
      const f32x4_t v = acc[mt][nt];
      *reinterpret_cast<uint2*>(O + row * ldo + col) =
          make_uint2(pack_bf16x2(f32_to_bf16_rne(v[0]), f32_to_bf16_rne(v[1])),
                     pack_bf16x2(f32_to_bf16_rne(v[2]), f32_to_bf16_rne(v[3])));
    }
  }
}

// Tile t of the batch: item m, M tile i, N tile j (segment 0 first, then
// segment 1). Within an item, tiles walk groups of kLinGroupRows M tiles down
// each N column.
template <bool B0KM>
__global__ __launch_bounds__(256, 1) void linear_kernel(LinBatch lb) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kLinStage];
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
  if (j < lb.nt0[m]) {
    const int64_t n0 = j * kLinTile;
    lin_tile<B0KM>(A, it.lda, B0KM ? it.B0 + n0 : it.B0 + n0 * it.ldb0, it.ldb0, it.O0 + m0 * it.ldo0 + n0, it.ldo0,
                   lb.M - m0, it.N0 - n0, it.K, smem);
  } else {
    lin_tile<true>(A, it.lda, it.B1, it.N1, it.O1 + m0 * it.N1, it.N1, lb.M - m0, it.N1, it.K, smem);
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
    hipLaunchKernelGGL(linear_kernel<true>, dim3((unsigned)tiles), dim3(256), 0, stream, lb);
  else
    hipLaunchKernelGGL(linear_kernel<false>, dim3((unsigned)tiles), dim3(256), 0, stream, lb);
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
    // rank 4 is narrower than a 16-byte chunk of P: its XP comes from the
    // small-rank project after the tile grid
    it.B1 = r >= 8 ? Ps[m] : nullptr;
    it.O1 = r >= 8 ? XPs[m] : nullptr;
    it.N1 = r >= 8 ? r : 0;
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
