// Normalized update with stochastic rounding [page "Randomized Gradient
// Compression", section "How it works"]:
//
//   W <- SR_bf16(W - s * H),  H = C P^T,  s = tau * ||W||_F / ||H||_F
//
// H is never written to memory. The update rebuilds it 64 columns at a time
// on MFMA (M = columns of W from rows of P, N = rows of W from rows of C,
// K = r), with C split into a bf16 high part and a bf16 remainder so that H
// carries ~16 bits of C's mantissa. The page rebuilds H 128 rows at a time;
// here a workgroup rebuilds 128 rows (64 at r = 128) x 64 columns per step
// (the result does not depend on the tile shape).
//
// One batch (e.g. all projections of a block) takes three or four launches:
//   norms:  sum w^2 over W (fp64 partials per 128 KB of W), and ||H||^2 =
//           tr((C^T C)(P^T P)) (the Frobenius norm of a product through the
//           two r x r Gram matrices): a few workgroups per matrix form
//           partial Gram matrices of C and of P (above r = 128 in four
//           groups of block pairs) on MFMA, fp32 partials; every reduction
//           has a fixed order across lanes and waves. Up to r = 64 the W
//           stream and the Gram workgroups share one launch; above, the Gram
//           workgroups' registers would leave the W stream one workgroup per
//           compute unit, so it runs first in a launch of its own;
//   reduce: one workgroup per (matrix, block pair) sums that pair's partials
//           in a fixed order into one term of ||H||^2 (and ||W||^2);
//   update: every wave forms s = fp32(tau ||W|| / ||H||) from its matrix's
//           terms (the skip flag when ||H|| is zero or not finite or s is not
//           finite), rebuilds its H tiles, forms v = fp32(w - fp32(s h)) and
//           rounds stochastically with 16 bits per element from
//           Philox4x32-10 keyed on (seed, row, column).
// Each matrix gets its own workgroups in every launch, as many as its own
// shape alone decides, so a matrix gets the same bits alone or in a batch.
//
// Lane layout of a tile: M-tile t row m stands for column
// jb + 16*(m/4) + 4*t + (m%4), which gives lane (g = lane/16, n = lane%16) the
// 16 consecutive columns jb + 16g .. +15 of its row in each N-tile, i.e. two
// 16-byte reads of W and two Philox calls (8 columns each).
#include <cmath>
#include <mutex>

#include "rgc_internal.hpp"

namespace rgc {

// kModeUpdateCarry: the update that also sums the squares of the bf16
// weights it writes (one fp64 partial per workgroup), for the carried norm.
enum ApplyMode { kModeUpdate = 1, kModeReconstruct = 2, kModeUpdateCarry = 3 };

// Where ||W||^2 comes from (ApplyBatch::carry): streamed from W by the norms
// launch (kCarryNone, kCarryFresh) or the caller's value carried over from
// the previous update (kCarryIn). With kCarryIn and kCarryFresh the caller's
// buffer receives ||W'||^2 of the weights the update wrote.
enum CarryMode { kCarryNone = 0, kCarryIn = 1, kCarryFresh = 2 };

constexpr int kApplyCols = 64;     // columns per tile
constexpr int kApplyWaves = 4;
constexpr int kApplyMaxItems = 16;
constexpr int64_t kMaxApplyDim = int64_t(1) << 30;  // d and k
constexpr int64_t kMaxApplyElems = int64_t(1) << 38;  // d * k (workgroup counts stay within int)

template <int R>
struct ApplyTraits {
  static constexpr int KQ = (R + 31) / 32;              // K-steps of 32 over r
  // Update sweeps: tiles of 128 rows, eight waves of one 16-row N-tile each,
  // so that more waves overlap the per-tile arithmetic with the copies: two
  // workgroups (four waves per SIMD) up to r = 128, one above, where the P
  // stage leaves one workgroup per compute unit (there eight waves against
  // four of two N-tiles: the Qwen3-1.7B-shaped block's apply at r = 256
  // 161 -> 148 us, at r = 192 139 -> 128 us). The 128-row tile halves the P
  // rows re-read per W byte against 64 rows (r = 256: 253 -> 205 us).
  static constexpr int WAVES = 8;  // waves of an update workgroup
  static constexpr int NTW = 1;
  static constexpr int RW = 16 * NTW;                   // rows per wave
  static constexpr int ROWS = WAVES * RW;               // rows per workgroup tile
  static constexpr int THREADS = 64 * WAVES;
};

struct ApplyItem {
  uint16_t* W;
  int64_t ldw;
  const float* C;
  const uint16_t* P;
  int64_t d, k;
  int64_t ctiles;  // column tiles per row block
  int64_t units;   // row blocks x column tiles
  uint64_t seed;
  float* stats;
  float alpha;  // fixed-scale update: the caller's step
};

struct ApplyBatch {
  int n;
  int fixed;  // 1: fixed-scale update (s = it.alpha, no norms, never skipped)
  int carry;  // CarryMode
  float tau;
  int wbase[kApplyMaxItems + 1];  // update workgroups [wbase[m], wbase[m+1]) serve item m
  // Norms: Gram workgroups [gbase[m], gbase[m+1]) (per pair group, the
  // first ncg[m] over rows of C, the rest over rows of P) and W-stream
  // workgroups [sbase[m], sbase[m+1]) (a launch of their own at the tiled
  // ranks; in the small ranks' norms launch they follow the Gram workgroups,
  // from gbase[n]).
  int gbase[kApplyMaxItems + 1];
  int sbase[kApplyMaxItems + 1];
  int ncg[kApplyMaxItems];
  ApplyItem it[kApplyMaxItems];
  double* partials;               // rebuild norms: 2 per workgroup; Gram norms: 1 per W-stream workgroup
  float* gram;                    // Gram norms: GramShape::NE floats per Gram workgroup
  double* hpairs;                 // Gram norms: per item, kGramMaxPairs block-pair terms of ||H||^2
  double* wnorm2;                 // per item, ||W||^2 (the caller's buffer when carrying)
  float* scale;                   // per item s, flag (rebuild norms; Gram norms when carrying)
  double* wpart;                  // carrying: per update workgroup, sum of the written weights' squares
  double* sgram;                  // ranks below 16: one fp64 Gram partial (upper triangle) per Gram workgroup
  float* H;                       // reconstruct target (test hook)
};

__device__ __forceinline__ int apply_item_of(const ApplyBatch& b, int w) {
  int m = 0;
  while (m + 1 < b.n && w >= b.wbase[m + 1]) ++m;
  return m;
}

// The Gram-form norms (below) work on 16-column blocks of C and P and their
// NB (NB + 1) / 2 block pairs a <= c. A workgroup holds the sums of at most
// 36 pairs (the registers of one wave), so above 8 blocks (r > 128) the pairs
// are split into four groups: the pairs within the lower half of the blocks,
// within the upper half, and the pairs across the halves in two groups (by
// the first block). Group g covers the n0(g) blocks from lo0(g) and, for a
// cross group, the n1(g) blocks from lo1(g).
template <int R>
struct GramShape {
  static constexpr int NB = R / 16;
  static constexpr int NG = NB <= 8 ? 1 : 4;             // pair groups
  static constexpr int H = NB <= 8 ? NB : (NB + 1) / 2;  // blocks of the lower half
  static constexpr int U = NB - H, H2 = H / 2;
  static constexpr int lo0(int g) { return g == 1 ? H : (g == 3 ? H2 : 0); }
  static constexpr int n0(int g) { return NG == 1 ? NB : (g == 0 ? H : (g == 1 ? U : (g == 2 ? H2 : H - H2))); }
  static constexpr int lo1(int) { return H; }
  static constexpr int n1(int g) { return NG > 1 && g >= 2 ? U : 0; }
  static constexpr int pairs(int g) { return n1(g) == 0 ? n0(g) * (n0(g) + 1) / 2 : n0(g) * n1(g); }
  static constexpr int poff(int g) { return g == 0 ? 0 : poff(g - 1) + pairs(g - 1); }  // first pair of group g
  static constexpr int NP = NB * (NB + 1) / 2;  // block pairs a <= c
  static constexpr int NE = 36 * 256;           // floats per Gram partial (the pairs of a group)
  // 32-row steps per wave of a Gram workgroup: 512 rows per workgroup keeps
  // its share of the stream (128 KB of C at r = 64) near that of a W-stream
  // workgroup, and the step count (each step waits for one load round) low.
  static constexpr int STEPS = 4;
  static constexpr int64_t ROWS = (int64_t)STEPS * 32 * kApplyWaves;
  static_assert(poff(NG) == NP, "the groups cover every block pair");
};
constexpr int kGramMaxPairs = 136;  // NP at r = 256

// s = fp32(tau * ||W|| / ||H||) from the squared norms; flag = 1 (and s = 0)
// when ||H|| is zero or not finite or s is not finite. stats (if not null)
// receive {||W||, ||H||, s, flag}.
__device__ __forceinline__ void step_scale(float tau, double nw2, double nh2, float& s, float& flag, float* stats) {
  const double nw = sqrt(nw2), nh = sqrt(nh2);
  s = 0.f;
  flag = 0.f;
  if (!(nh > 0.0) || !isfinite(nh)) {
    flag = 1.f;
  } else {
    s = (float)((double)tau * nw / nh);
    if (!isfinite(s)) {
      s = 0.f;
      flag = 1.f;
    }
  }
  if (stats) {
    stats[0] = (float)nw;
    stats[1] = (float)nh;
    stats[2] = s;
    stats[3] = flag;
  }
}

// The C side of the MFMA for the rows of one N-tile: K-step q holds
// C[i][32q + 8g .. +7] as bf16 high parts and bf16 remainders.
template <int R>
struct RowOperand {
  uint32_t hi[ApplyTraits<R>::NTW][ApplyTraits<R>::KQ][4];
  uint32_t lo[ApplyTraits<R>::NTW][ApplyTraits<R>::KQ][4];
};

template <int R>
__device__ __forceinline__ void load_row_operand(const float* __restrict__ C, int64_t d, int64_t row0, int lane,
                                                 RowOperand<R>& op) {
  using Tr = ApplyTraits<R>;
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < Tr::NTW; ++nt) {
    const int64_t i = row0 + 16 * nt + n;
#pragma unroll
    for (int q = 0; q < Tr::KQ; ++q) {
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
        const uint32_t hv = f32x2_to_bf16x2_rne(v[2 * p], v[2 * p + 1]);
        op.hi[nt][q][p] = hv;
        op.lo[nt][q][p] = f32x2_to_bf16x2_rne(v[2 * p] - __uint_as_float(hv << 16),
                                              v[2 * p + 1] - __uint_as_float(hv & 0xFFFF0000u));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The sweeps are software pipelines over the workgroup's tiles: each tile's
// W rows (ROWS x 64 bf16) and P rows (64 x R bf16) are copied from memory
// straight into an LDS stage (1 KB copies that bypass the VGPRs, spread over
// the workgroup's waves), S - 1 tiles ahead of the tile being processed.
//
// W stage layout: copy c holds tile rows 8c .. 8c+7 (128 bytes each); lane l
// reads row 8c + l / 8, 8-column chunk q such that its 16 bytes land at
// 16 * (8 * (l / 8) + (q + (l / 8) / 2 + 4 (c % 2)) % 8). A lane's two
// chunks of its row (columns 16g .. 16g+15) are then two 16-byte reads, and
// the rotations spread the 16 rows a wave reads at once over all banks.
//
// P stage layout: the 64 P rows of the tile row-major (2R bytes each) with
// the 16-byte chunks of row jl rotated by f(jl) (bank spreading for the
// A-operand reads, whose 16 lanes read 16 different rows).
// ---------------------------------------------------------------------------
// Two workgroups per compute unit with up to three stages each (two at r >
// 80, where a stage passes 26 KB): the update's per-tile arithmetic (the H
// rebuild on MFMA, Philox, rounding) is heavy enough that other waves
// overlapping it pay more than deeper staging (measured on the Qwen3-1.7B-
// shaped block and the Qwen3-8B-shaped layer). At r > 128 the P rows make a
// stage too large for two, so one workgroup takes up to six (three at
// r = 256).

template <int R, int MODE>
struct ApplyShape {
  using Tr = ApplyTraits<R>;
  static constexpr int WC = MODE == kModeReconstruct ? 0 : Tr::ROWS / 8;  // W copies per stage
  static constexpr int CH = R / 8;                                          // 16-byte chunks per P row
  static constexpr int PC = 64 * CH / 64;                                   // P copies per stage (= R / 8)
  static constexpr int NI = WC + PC;
  static constexpr int PBASE = 1024 * WC;
  static constexpr int STAGE = 1024 * NI;
  static constexpr int PER_CU = R > 128 ? 1 : 2;                          // resident workgroups per compute unit
  static constexpr int LDS_MAX = (PER_CU == 2 ? 79 : 159) * 1024;        // room for the norm reduction
  static constexpr int SMAX = PER_CU == 2 ? 3 : 6;
  static constexpr int S = SMAX * STAGE <= LDS_MAX ? SMAX : LDS_MAX / STAGE;
  static constexpr int NV_LO = NI / Tr::WAVES, NV_HI = (NI + Tr::WAVES - 1) / Tr::WAVES;  // copies per wave
  static_assert(S >= 2 && S * STAGE <= LDS_MAX, "LDS");
  static_assert((S - 1) * NV_HI <= 63, "vector memory counter");
};

// Chunk rotation of P row jl in the stage.
template <int CH>
__device__ __forceinline__ int p_rotation(int jl) {
  return CH <= 8 ? (2 * (jl >> 4) + ((jl & 3) >> 1)) : (4 * (jl >> 4) + (jl & 3));
}

// h[nt][x] = H[row(nt)][jb + 16g + x], x = 0..15, from the P rows in LDS.
template <int R>
__device__ __forceinline__ void rebuild_tile(const RGC_LDS char* pst, const RowOperand<R>& rop, int lane,
                                             float (&h)[ApplyTraits<R>::NTW][16]) {
  using Tr = ApplyTraits<R>;
  constexpr int CH = R / 8;
  const int m = lane & 15, g = lane >> 4;
  f32x4_t acc[4][Tr::NTW];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int nt = 0; nt < Tr::NTW; ++nt) acc[t][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int jl = 16 * (m >> 2) + 4 * t + (m & 3);
    const int rot = p_rotation<CH>(jl);
#pragma unroll
    for (int q = 0; q < Tr::KQ; ++q) {
      const int ch = 4 * q + g;  // rank columns 32q + 8g .. +7
      uint32_t a[4] = {0u, 0u, 0u, 0u};
      if (32 * q + 32 <= R || ch < CH) {  // columns past R are zero (r = 48)
        const u32x4v_t v = *(const RGC_LDS u32x4v_t*)(pst + jl * (2 * R) + 16 * ((ch + rot) % CH));
        a[0] = v.x;
        a[1] = v.y;
        a[2] = v.z;
        a[3] = v.w;
      }
#pragma unroll
      for (int nt = 0; nt < Tr::NTW; ++nt) {
        acc[t][nt] = mfma_16x16x32(a, rop.hi[nt][q], acc[t][nt]);
        acc[t][nt] = mfma_16x16x32(a, rop.lo[nt][q], acc[t][nt]);
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < Tr::NTW; ++nt)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) h[nt][4 * t + e] = acc[t][nt][e];
}

// Rounding bits for row i, columns 8*cb .. 8*cb+7: word (x/2), low half for
// even x.
__device__ __forceinline__ void rounding_words(uint64_t seed, int64_t i, int64_t cb, uint32_t (&words)[4]) {
  u32x4 c = {(uint32_t)cb, (uint32_t)i, kTagRounding, 0u};
  const u32x4 o = philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  words[0] = o.x; words[1] = o.y; words[2] = o.z; words[3] = o.w;
}

// Tiles are addressed from an origin (wrow, wcol) that keeps the whole
// ROWS x 64 stage inside W (and the 64 P rows inside P): the tile's own
// origin, shifted back at the last row block or column tile. The lanes then
// work in stage coordinates (row wrow + r, column wcol + c) and only the
// elements the tile owns (rows row0 .. row0+ROWS-1, columns jb .. jb+63, and
// inside W) are stored or counted. Matrices with fewer than ROWS rows or 64
// columns use origin 0 and clamp the copied rows and columns instead.
// The hardware hands workgroups to the eight XCDs round-robin; this numbers
// them so that each XCD runs a contiguous run of workgroups (whole row blocks
// of W), so that a row block's C rows are fetched into one XCD's L2, not into
// all eight. The partition of the work over the numbers, and so every sum,
// is unchanged.
__device__ __forceinline__ int apply_logical_workgroup(int b, int G) {
  constexpr int kXcds = 8;
  const int x = b % kXcds, pos = b / kXcds;
  const int q = G / kXcds, rem = G % kXcds;
  return x * q + (x < rem ? x : rem) + pos;
}

template <int R, int MODE>
__global__ __launch_bounds__(ApplyTraits<R>::THREADS, R > 128 ? 1 : 2) void apply_kernel(ApplyBatch b) {  // PER_CU
  using Tr = ApplyTraits<R>;
  using Sh = ApplyShape<R, MODE>;
  constexpr int S = Sh::S;
  __shared__ __attribute__((aligned(1024))) char smem[S * Sh::STAGE];
  __shared__ double red[Tr::WAVES];
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int n = lane & 15, g = lane >> 4;
  const int w = apply_logical_workgroup(blockIdx.x, gridDim.x);
  const int m = apply_item_of(b, w);
  const ApplyItem& it = b.it[m];
  const int64_t wl = w - b.wbase[m], gm = b.wbase[m + 1] - b.wbase[m];
  const int64_t u0 = uniform_i64(wl * it.units / gm), u1 = uniform_i64((wl + 1) * it.units / gm);

  constexpr bool UPD = MODE == kModeUpdate || MODE == kModeUpdateCarry;
  float s = 0.f;
  if constexpr (UPD) {
    if (b.fixed) s = it.alpha;
  }

  double sw = 0.0;
  RowOperand<R> rop;
  uint16_t* wrowp[Tr::NTW];  // update: start of the lane's W row in each N-tile
  int rop_row = -1;  // first row of the loaded row operand
  const int d = (int)it.d, k = (int)it.k, ctiles = (int)it.ctiles;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(RGC_LDS char*)smem;
  const bool more = wave < Sh::NI % Tr::WAVES;
  // Tiles run in unit order, unit = row block * ctiles + column tile; the
  // copy cursor (lrb, lct) and the compute cursor (crb, cct) step through
  // (row block, column tile) without dividing.
  auto origin = [&](int rb, int ct, int& row0, int& jb, int& wrow, int& wcol) {
    row0 = rb * Tr::ROWS;
    jb = ct * kApplyCols;
    wrow = row0 + Tr::ROWS <= d ? row0 : (d >= Tr::ROWS ? d - Tr::ROWS : 0);
    wcol = jb + kApplyCols <= k ? jb : (k >= kApplyCols ? k - kApplyCols : 0);
  };

  // ---- copies: per-lane byte offsets from the tile origin (fixed)
  uint32_t voff[Sh::NV_HI];
#pragma unroll
  for (int v = 0; v < Sh::NV_HI; ++v) {
    const int c = wave + Tr::WAVES * v;
    if (c < Sh::WC) {
      const int t = lane >> 3;
      const int q = ((lane & 7) - (t >> 1) - 4 * (c & 1)) & 7;
      const int row = 8 * c + t < d ? 8 * c + t : d - 1;
      const int col = 8 * q + 8 <= k ? 8 * q : k - 8;
      voff[v] = (uint32_t)(((int64_t)row * it.ldw + col) * 2);
    } else {
      const int e = 64 * (c - Sh::WC) + lane;
      const int jr = e / Sh::CH, sig = e % Sh::CH;
      const int ch = ((sig - p_rotation<Sh::CH>(jr)) % Sh::CH + Sh::CH) % Sh::CH;
      const int prow = jr < k ? jr : k - 1;
      voff[v] = (uint32_t)(((int64_t)prow * R + 8 * ch) * 2);
    }
  }
  int64_t lu = u0;
  int lrb = __builtin_amdgcn_readfirstlane((int)(u0 / ctiles));
  int lct = __builtin_amdgcn_readfirstlane((int)(u0 - (int64_t)lrb * ctiles));
  int crb = lrb, cct = lct;
  uint32_t lslot = 0;
  auto issue = [&]() {
    int row0, jb, wrow, wcol;
    origin(lrb, lct, row0, jb, wrow, wcol);
    if (++lct == ctiles) {
      lct = 0;
      ++lrb;
    }
    const uint16_t* Wb = uniform_ptr(it.W + (int64_t)wrow * it.ldw + wcol);
    const uint16_t* Pb = uniform_ptr(it.P + (int64_t)wcol * R);
    const uint32_t st = lds0 + lslot * Sh::STAGE;
    static_for<0, Sh::NV_HI>([&](auto vc) {
      constexpr int v = decltype(vc)::value;
      const int c = wave + Tr::WAVES * v;  // a W copy if c < WC, a P copy if WC <= c < NI
      if constexpr (Tr::WAVES * v + Tr::WAVES - 1 < Sh::WC) {
        dma_16b_stream(Wb, voff[v], st + 1024 * c);
      } else if constexpr (Tr::WAVES * v >= Sh::WC && Tr::WAVES * v + Tr::WAVES - 1 < Sh::NI) {
        dma_16b_cached(Pb, voff[v], st + 1024 * c);
      } else {
        if (c < Sh::WC)
          dma_16b_stream(Wb, voff[v], st + 1024 * c);
        else if (c < Sh::NI)
          dma_16b_cached(Pb, voff[v], st + 1024 * c);
      }
    });
    ++lu;
    lslot = lslot + 1 == S ? 0 : lslot + 1;
  };
#pragma unroll
  for (int v = 0; v + 1 < S; ++v)
    if (lu < u1) issue();

  if constexpr (UPD) {
    if (!b.fixed) {
      // s from the item's norm terms while the first copies are in flight: the
      // same fixed-order sums in every wave of every workgroup of the item
      // (each lane its terms lane, lane + 64, ... in order, then a butterfly,
      // which gives every lane the same sum), so all agree on s.
      double hp = 0.0;
      for (int q = lane; q < GramShape<R>::NP; q += 64) hp += b.hpairs[m * kGramMaxPairs + q];
      float flag;
      const bool lead = wl == 0 && threadIdx.x == 0;
      step_scale(b.tau, b.wnorm2[m], wave_sum(hp), s, flag, lead ? it.stats : nullptr);
      if constexpr (MODE == kModeUpdateCarry) {
        if (lead) {  // read by the launch that sums the carried norm
          b.scale[2 * m] = s;
          b.scale[2 * m + 1] = flag;
        }
      }
      if (flag != 0.f) {  // zero or non-finite step: W stays as it is
        wait_vmcnt<0>();
        return;
      }
    }
  }

  uint32_t cslot = 0;
  for (int64_t u = u0; u < u1; ++u) {
    if (u + S - 2 < u1) {
      if (more)
        wait_vmcnt<(S - 2) * Sh::NV_HI>();
      else
        wait_vmcnt<(S - 2) * Sh::NV_LO>();
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
    if (lu < u1) issue();
    const RGC_LDS char* st = (const RGC_LDS char*)smem + cslot * Sh::STAGE;
    cslot = cslot + 1 == S ? 0 : cslot + 1;

    int row0, jb, wrow, wcol;
    origin(crb, cct, row0, jb, wrow, wcol);
    if (++cct == ctiles) {
      cct = 0;
      ++crb;
    }
    if (wrow != rop_row) {  // wave-uniform: new rows
      load_row_operand<R>(it.C, it.d, wrow + Tr::RW * wave, lane, rop);
      rop_row = wrow;
      if constexpr (UPD) {
#pragma unroll
        for (int nt = 0; nt < Tr::NTW; ++nt) {
          const int i = wrow + Tr::RW * wave + 16 * nt + n;
          wrowp[nt] = it.W + (int64_t)(i < d ? i : d - 1) * it.ldw;
        }
      }
    }
    float h[Tr::NTW][16];
    rebuild_tile<R>(st + Sh::PBASE, rop, lane, h);
    // Every lane does the arithmetic; only the stores (and the norm sums)
    // depend on whether the tile owns its element.
#pragma unroll
    for (int nt = 0; nt < Tr::NTW; ++nt) {
      const int r = Tr::RW * wave + 16 * nt + n;  // stage row
      const int i = wrow + r;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int cs = 16 * g + 8 * half;  // stage column of the lane's 8-column chunk
        const int jj = wcol + cs;
        const bool inside = i >= row0 && i < d && jj >= jb && jj < k;
        const float* hv = &h[nt][8 * half];
        if constexpr (MODE == kModeReconstruct) {
          if (inside) {
            float4* dst = reinterpret_cast<float4*>(b.H + (int64_t)i * k + jj);
            dst[0] = make_float4(hv[0], hv[1], hv[2], hv[3]);
            dst[1] = make_float4(hv[4], hv[5], hv[6], hv[7]);
          }
        } else {
          const int c = r >> 3, t = r & 7, q = cs >> 3;
          const u32x4v_t wv =
              *(const RGC_LDS u32x4v_t*)(st + 1024 * c + 16 * (8 * t + ((q + (t >> 1) + 4 * (c & 1)) & 7)));
          const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
          {
            uint32_t rw[4];
            rounding_words(it.seed, i, jj >> 3, rw);
            uint32_t out[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const float w0 = __uint_as_float(wd[p] << 16), w1 = __uint_as_float(wd[p] & 0xFFFF0000u);
              const float sh0 = s * hv[2 * p], sh1 = s * hv[2 * p + 1];
              const float v0 = w0 - sh0, v1 = w1 - sh1;
              out[p] = f32x2_to_bf16x2_sr(v0, v1, rw[p]);
            }
            if (inside) *reinterpret_cast<uint4*>(wrowp[nt] + jj) = make_uint4(out[0], out[1], out[2], out[3]);
            if constexpr (MODE == kModeUpdateCarry) {
              float sq = 0.f;
#pragma unroll
              for (int p = 0; p < 4; ++p) {
                const float o0 = __uint_as_float(out[p] << 16), o1 = __uint_as_float(out[p] & 0xFFFF0000u);
                sq += o0 * o0;
                sq += o1 * o1;
              }
              sw += inside ? (double)sq : 0.0;
            }
          }
        }
      }
    }
  }
  wait_vmcnt<0>();

  if constexpr (MODE == kModeUpdateCarry) {
    sw = wave_sum(sw);
    if (lane == 0) red[wave] = sw;
    __syncthreads();
    if (threadIdx.x == 0) {
      double t = red[0];
      for (int v = 1; v < Tr::WAVES; ++v) t += red[v];  // waves in order
      b.wpart[w] = t;
    }
  }
}

// ---------------------------------------------------------------------------
// Gram-form norms.
//
// ||H||_F^2 = ||C P^T||_F^2 = tr(P C^T C P^T) = sum_ab (C^T C)_ab (P^T P)_ab.
// C^T C is formed from C's bf16 high parts and remainders with all four
// products (so only C's own two-term rounding, about 2^-18 relative and of
// either sign, enters), P^T P from P's bf16 values (exact products), both
// with fp32 MFMA sums over at most a few hundred rows per wave and fp64 sums
// across workgroups. The result equals the H-based norm up to rounding. A C
// whose squares leave the fp32 range (|c| above ~1e19) gives a non-finite
// Gram and the update is skipped as for a non-finite ||H||.
//
// Lane layout: the r columns are relabelled so that block a (a < NB = r/16),
// position x stands for column NB*x + a. Lane l (x = l % 16, g = l / 16)
// reads the NB consecutive values NB*x .. NB*x + NB - 1 of each of its rows
// 8g .. 8g+7 of a 32-row step (those of its pair group's blocks), which for
// every block a is the MFMA operand of row x with K = those 8 rows, both as A
// and as B. Block pair (a, b), a <= b, accumulates the 16 x 16 block (a, b)
// of the relabelled Gram matrix. C and P are relabelled alike, so the sum of
// the elementwise product is unchanged; off-diagonal pairs count twice (the
// blocks (b, a) are their transposes).
// ---------------------------------------------------------------------------
// 16-byte chunks of W per W-stream workgroup (128 KB).
constexpr int64_t kWStreamChunks = 8192;

// The values one lane reads in one 32-row step: rows 8g .. 8g+7 of the step,
// for the NL blocks of its pair group (raw bits: fp32 for C, bf16 for P).
// Slot s < N0 holds block LO0 + s, slot N0 + s block LO1 + s; the value of
// block b in lane x is column NB x + b of the row. Rows past row1 are read
// from row row1 - 1 and masked to 0 where they are used (keep), so that the
// loads carry no branch: a load under a per-row branch was followed by a
// wait for it, which serialised every step's sixteen loads.
template <int NL>
struct GramRows {
  uint32_t v[8][NL];
  uint32_t keep[8];  // ~0 for a row below row1, else 0
};

// Blocks LO .. LO+N-1 of one row (p = the row's column NB x) into slots
// S .. S+N-1, with vector loads where the alignment allows.
template <int NB, int LO, int N, int S, int NL>
__device__ __forceinline__ void load_range(const float* __restrict__ p, uint32_t (&v)[NL]) {
  if constexpr (N > 0) {
    if constexpr (NB % 4 == 0 && LO % 4 == 0 && N % 4 == 0) {
#pragma unroll
      for (int i = 0; i < N; i += 4) {
        const uint4 a = *reinterpret_cast<const uint4*>(p + LO + i);
        v[S + i] = a.x; v[S + i + 1] = a.y; v[S + i + 2] = a.z; v[S + i + 3] = a.w;
      }
    } else if constexpr (NB % 2 == 0 && LO % 2 == 0 && N % 2 == 0) {
#pragma unroll
      for (int i = 0; i < N; i += 2) {
        const uint2 a = *reinterpret_cast<const uint2*>(p + LO + i);
        v[S + i] = a.x; v[S + i + 1] = a.y;
      }
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) v[S + i] = __float_as_uint(p[LO + i]);
    }
  }
}
template <int NB, int LO, int N, int S, int NL>
__device__ __forceinline__ void load_range(const uint16_t* __restrict__ p, uint32_t (&v)[NL]) {
  if constexpr (N > 0) {
    if constexpr (NB % 8 == 0 && LO % 8 == 0 && N % 8 == 0) {
#pragma unroll
      for (int i = 0; i < N; i += 8) {
        const uint4 a = *reinterpret_cast<const uint4*>(p + LO + i);
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[S + i + 2 * j] = w[j] & 0xFFFFu;
          v[S + i + 2 * j + 1] = w[j] >> 16;
        }
      }
    } else if constexpr (NB % 4 == 0 && LO % 4 == 0 && N % 4 == 0) {
#pragma unroll
      for (int i = 0; i < N; i += 4) {
        const uint2 a = *reinterpret_cast<const uint2*>(p + LO + i);
        v[S + i] = a.x & 0xFFFFu; v[S + i + 1] = a.x >> 16; v[S + i + 2] = a.y & 0xFFFFu; v[S + i + 3] = a.y >> 16;
      }
    } else if constexpr (NB % 2 == 0 && LO % 2 == 0 && N % 2 == 0) {
#pragma unroll
      for (int i = 0; i < N; i += 2) {
        const uint32_t a = *reinterpret_cast<const uint32_t*>(p + LO + i);
        v[S + i] = a & 0xFFFFu; v[S + i + 1] = a >> 16;
      }
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) v[S + i] = p[LO + i];
    }
  }
}

template <int NB, int LO0, int N0, int LO1, int N1, typename T>
__device__ __forceinline__ void load_gram_rows(const T* __restrict__ src, int64_t base, int64_t row1, int x, int g,
                                               GramRows<N0 + N1>& o) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t row = base + 8 * g + e;
    o.keep[e] = row < row1 ? ~0u : 0u;
    const T* p = src + (row < row1 ? row : row1 - 1) * (16 * NB) + NB * x;
    load_range<NB, LO0, N0, 0>(p, o.v[e]);
    load_range<NB, LO1, N1, N0>(p, o.v[e]);
  }
}

// One 32-row step: MFMA operands of the group's blocks from the lane's rows
// (C: bf16 high part and remainder of each fp32 value, all four products; P:
// the bf16 values), accumulated into the group's block pairs: with N1 = 0
// the pairs (a, c), a <= c < N0, else the pairs (a, N0 + c), in a-major order.
template <int N0, int N1, bool TWO_TERM>
__device__ __forceinline__ void gram_step(const GramRows<N0 + N1>& rw,
                                          f32x4_t (&acc)[N1 == 0 ? N0 * (N0 + 1) / 2 : N0 * N1]) {
  constexpr int NL = N0 + N1;
  uint32_t hi[NL][4], lo[NL][4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int a = 0; a < NL; ++a) {
      if constexpr (TWO_TERM) {
        const float v0 = __uint_as_float(rw.v[2 * p][a] & rw.keep[2 * p]);
        const float v1 = __uint_as_float(rw.v[2 * p + 1][a] & rw.keep[2 * p + 1]);
        const uint32_t hv = f32x2_to_bf16x2_rne(v0, v1);
        hi[a][p] = hv;
        lo[a][p] = f32x2_to_bf16x2_rne(v0 - __uint_as_float(hv << 16), v1 - __uint_as_float(hv & 0xFFFF0000u));
      } else {
        hi[a][p] = pack_bf16x2(rw.v[2 * p][a] & rw.keep[2 * p], rw.v[2 * p + 1][a] & rw.keep[2 * p + 1]);
        lo[a][p] = 0u;
      }
    }
  int q = 0;
#pragma unroll
  for (int a = 0; a < N0; ++a)
#pragma unroll
    for (int c = (N1 == 0 ? a : N0); c < (N1 == 0 ? N0 : NL); ++c) {
      acc[q] = mfma_16x16x32(hi[a], hi[c], acc[q]);
      if constexpr (TWO_TERM) {
        acc[q] = mfma_16x16x32(hi[a], lo[c], acc[q]);
        acc[q] = mfma_16x16x32(lo[a], hi[c], acc[q]);
        acc[q] = mfma_16x16x32(lo[a], lo[c], acc[q]);
      }
      ++q;
    }
}

// Partial Gram matrix of rows [row0, row1) (at most ROWS) of the row-major
// rows x R matrix src (C in fp32 with TWO_TERM, P in bf16 without), for the
// block pairs of group GR, written as out[pair * 256 + 64 j + lane] = entry j
// of the lane's 16 x 16 MFMA output for the group's pair `pair`, summed over
// the four waves in wave order. Wave w takes the steps at rows row0 + 32 w +
// 128 s; each step's loads are issued before the previous step's MFMAs.
template <int R, bool TWO_TERM, int GR, typename T>
__device__ void gram_partial(const T* __restrict__ src, int64_t row0, int64_t row1, float* __restrict__ out,
                             float* red) {
  using Gs = GramShape<R>;
  constexpr int NB = Gs::NB;
  constexpr int LO0 = Gs::lo0(GR), N0 = Gs::n0(GR), LO1 = Gs::lo1(GR), N1 = Gs::n1(GR);
  constexpr int NPG = Gs::pairs(GR);
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int x = lane & 15, g = lane >> 4;
  f32x4_t acc[NPG];
#pragma unroll
  for (int q = 0; q < NPG; ++q) acc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  GramRows<N0 + N1> cur, nxt;
  load_gram_rows<NB, LO0, N0, LO1, N1>(src, row0 + 32 * wave, row1, x, g, cur);
#pragma unroll
  for (int st = 0; st < Gs::STEPS; ++st) {
    if (st + 1 < Gs::STEPS)
      load_gram_rows<NB, LO0, N0, LO1, N1>(src, row0 + 32 * wave + 128 * (st + 1), row1, x, g, nxt);
    gram_step<N0, N1, TWO_TERM>(cur, acc);
    if (st + 1 < Gs::STEPS) cur = nxt;
  }
  // waves add their sums into one slab in wave order: ((w0 + w1) + w2) + w3
#pragma unroll
  for (int w = 0; w < kApplyWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int q = 0; q < NPG; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float* e = red + q * 256 + 64 * j + lane;
          *e = w == 0 ? acc[q][j] : *e + acc[q][j];
        }
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < NPG * 256; e += 256) out[e] = red[e];
}

// Sum of squares of the 16-byte chunks [c0, c1) of W (row-major d x k, row
// stride ldw; chunk c is columns 8 (c % (k/8)) .. +7 of row c / (k/8)):
// fp32 per chunk (the squares of bf16 values are exact in fp32), fp64 across
// chunks, lanes and waves; returned in thread 0. NT: non-temporal loads.
template <bool NT>
__device__ double wstream_sumsq(const uint16_t* __restrict__ W, int64_t ldw, int64_t k, int64_t c0, int64_t c1,
                                double* red) {
  constexpr int U = 8;
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int cpr = (int)(k >> 3);
  const int dr = 256 / cpr, dc = 256 % cpr;  // per 256 chunks: whole rows and remainder
  int64_t c = c0 + threadIdx.x;
  int row = (int)(c / cpr), col = (int)(c % cpr);
  double acc = 0.0;
  for (; c < c1; c += 256 * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const u32x4v_t* src = reinterpret_cast<const u32x4v_t*>(W + (int64_t)row * ldw + 8 * col);
      const u32x4v_t t = c + 256 * u < c1 ? (NT ? __builtin_nontemporal_load(src) : *src) : u32x4v_t{0u, 0u, 0u, 0u};
      v[u] = make_uint4(t.x, t.y, t.z, t.w);
      col += dc;
      row += dr;
      const bool wrap = col >= cpr;
      col -= wrap ? cpr : 0;
      row += wrap ? 1 : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      float sq = 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float w0 = bf16_bits_to_f32(wd[p] & 0xFFFFu), w1 = bf16_bits_to_f32(wd[p] >> 16);
        sq += w0 * w0;
        sq += w1 * w1;
      }
      acc += (double)sq;
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) red[wave] = acc;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}

__device__ __forceinline__ int item_of(const int* base, int n, int w) {
  int m = 0;
  while (m + 1 < n && w >= base[m + 1]) ++m;
  return m;
}

// W-stream workgroup sw: the squares of its kWStreamChunks chunks of one
// matrix into b.partials[sw].
template <bool NT>
__device__ __forceinline__ void wstream_workgroup(const ApplyBatch& b, int sw, double* red) {
  const int m = item_of(b.sbase, b.n, sw);
  const ApplyItem& it = b.it[m];
  const int64_t total = it.d * (it.k >> 3);
  const int64_t c0 = (sw - b.sbase[m]) * kWStreamChunks;
  const int64_t c1 = c0 + kWStreamChunks < total ? c0 + kWStreamChunks : total;
  const double sq = wstream_sumsq<NT>(it.W, it.ldw, it.k, c0, c1, red);
  if (threadIdx.x == 0) b.partials[sw] = sq;
}

// The W stream in a launch of its own (64 < r <= 128): in one launch with the
// Gram workgroups it took their register allocation (one workgroup per
// compute unit) and streamed W at about 4.2 TB/s; alone, with non-temporal
// loads, at 5.5 TB/s (the Qwen3-8B-shaped layer at r = 128: 386 MB in 70 us;
// the apply 295 -> 271 us). Up to r = 64 the shared launch measured faster
// (the Qwen3-1.7B-shaped block: 71 against 78 us), and above r = 128 too,
// where the Gram workgroups take longer than the stream and the shared launch
// hides it behind them (the same block at r = 256: 142 against 135 us per
// update).
__global__ __launch_bounds__(256) void wstream_kernel(ApplyBatch b) {
  __shared__ double red[kApplyWaves];
  wstream_workgroup<true>(b, blockIdx.x, red);
}

// Where the W stream runs at rank R (see wstream_kernel).
template <int R>
constexpr bool wstream_own_launch() { return R > 64 && R <= 128; }

// The norms launch: per item and pair group, the C-row chunks, then the
// P-row chunks; outside 64 < r <= 128 the W-stream workgroups follow.
template <int R>
__global__ __launch_bounds__(256) void gram_norms_kernel(ApplyBatch b) {
  using Gs = GramShape<R>;
  __shared__ __attribute__((aligned(16))) float red[Gs::NE];
  const int w = blockIdx.x;
  const int ng = b.gbase[b.n];
  if (!wstream_own_launch<R>() && w >= ng) {
    wstream_workgroup<false>(b, w - ng, reinterpret_cast<double*>(red));
    return;
  }
  {
    const int m = item_of(b.gbase, b.n, w);
    const ApplyItem& it = b.it[m];
    const int per_group = (b.gbase[m + 1] - b.gbase[m]) / Gs::NG;  // C and P chunks of one group
    const int l = w - b.gbase[m];
    const int grp = l / per_group, lc = l - grp * per_group;
    float* out = b.gram + (int64_t)w * Gs::NE;
    static_for<0, Gs::NG>([&](auto gc) {
      constexpr int GR = decltype(gc)::value;
      if (grp != GR) return;
      if (lc < b.ncg[m]) {
        const int64_t r0 = lc * Gs::ROWS, r1 = r0 + Gs::ROWS < it.d ? r0 + Gs::ROWS : it.d;
        gram_partial<R, true, GR>(it.C, r0, r1, out, red);
      } else {
        const int64_t r0 = (lc - b.ncg[m]) * Gs::ROWS, r1 = r0 + Gs::ROWS < it.k ? r0 + Gs::ROWS : it.k;
        gram_partial<R, false, GR>(it.P, r0, r1, out, red);
      }
    });
  }
}

// Per item: the scale launches sum its norms partials in a fixed order (each
// thread its share in order, passed here as aw and ah; then a butterfly
// within each wave and the waves in order) and form s = fp32(tau * ||W|| /
// ||H||); flag = 1 when ||H|| is zero or not finite or s is not finite (then
// s = 0).
__device__ __forceinline__ void finish_scale(const ApplyBatch& b, int m, double aw, double ah) {
  __shared__ double red[2][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  aw = wave_sum(aw);
  ah = wave_sum(ah);
  if (lane == 0) {
    red[0][wave] = aw;
    red[1][wave] = ah;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  double nw2 = ((red[0][0] + red[0][1]) + red[0][2]) + red[0][3];
  const double nh2 = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];
  if (b.carry == kCarryIn) nw2 = b.wnorm2[m];
  if (b.carry == kCarryFresh) b.wnorm2[m] = nw2;
  float s, flag;
  step_scale(b.tau, nw2, nh2, s, flag, b.it[m].stats);
  b.scale[2 * m] = s;
  b.scale[2 * m + 1] = flag;
}

// Gram form, one workgroup per (item, block pair): thread t sums entry t of
// the pair in the item's C Gram partials and in its P Gram partials (those
// of the pair's group) in partial order (fp64), and the workgroup writes sum
// over its entries of G * M, times 2 for an off-diagonal pair. Pair 0's
// workgroup also sums the item's W-stream partials into ||W||^2.
template <int R>
__global__ __launch_bounds__(256) void gram_reduce_kernel(ApplyBatch b) {
  using Gs = GramShape<R>;
  __shared__ double red[2][4];
  const int m = blockIdx.x / Gs::NP, q = blockIdx.x % Gs::NP;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int grp = 0;
  while (grp + 1 < Gs::NG && q >= Gs::poff(grp + 1)) ++grp;
  const int ql = q - Gs::poff(grp);  // the pair within its group
  const int nc = b.ncg[m], np = (b.gbase[m + 1] - b.gbase[m]) / Gs::NG - nc;
  const float* gc = b.gram + (int64_t)(b.gbase[m] + grp * (nc + np)) * Gs::NE + 256 * ql + threadIdx.x;
  const float* gp = gc + (int64_t)nc * Gs::NE;
  // the C and P partials are loaded together, U of each in flight per thread
  // (row clamped, value masked past the count, so that no load sits under a
  // branch), and summed in partial order
  constexpr int U = 16;
  double G = 0.0, M = 0.0;
  const int nmax = nc > np ? nc : np;
  for (int u = 0; u < nmax; u += U) {
    float vc[U], vp[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      vc[i] = gc[(int64_t)(u + i < nc ? u + i : nc - 1) * Gs::NE];
      vp[i] = gp[(int64_t)(u + i < np ? u + i : np - 1) * Gs::NE];
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      if (u + i < nc) G += (double)vc[i];
      if (u + i < np) M += (double)vp[i];
    }
  }
  // a within-half group lists its pairs (a, c) for a = 0.., c = a .. n0-1
  // (diagonal when c = a); a cross group has no diagonal pair
  bool diag = false;
  if (Gs::n1(grp) == 0) {
    int pq = ql, a = 0;
    while (pq >= Gs::n0(grp) - a) {
      pq -= Gs::n0(grp) - a;
      ++a;
    }
    diag = pq == 0;
  }
  double th = (diag ? 1.0 : 2.0) * G * M;
  double tw = 0.0;
  const bool streamed = q == 0 && b.carry != kCarryIn;  // else ||W||^2 is the caller's carried value
  if (streamed) {
    // thread t sums partials t, t + 256, ... in order, four loads in flight
    const int w1 = b.sbase[m + 1];
    for (int w = b.sbase[m] + (int)threadIdx.x; w < w1; w += 4 * 256) {
      double v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = b.partials[w + 256 * i < w1 ? w + 256 * i : w1 - 1];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (w + 256 * i < w1) tw += v[i];
    }
  }
  th = wave_sum(th);
  tw = wave_sum(tw);
  if (lane == 0) {
    red[0][wave] = th;
    red[1][wave] = tw;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  b.hpairs[m * kGramMaxPairs + q] = ((red[0][0] + red[0][1]) + red[0][2]) + red[0][3];
  if (streamed) b.wnorm2[m] = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];
}

// Carried norm, one workgroup per item: ||W'||^2 = the update workgroups'
// partials summed in a fixed order (as in the scale launch), stored over the
// item's ||W||^2. A skipped update leaves W, and so the value, as it is.
__global__ __launch_bounds__(256) void carry_norm_kernel(ApplyBatch b) {
  __shared__ double red[4];
  const int m = blockIdx.x;
  if (b.scale[2 * m + 1] != 0.f) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double a = 0.0;
  for (int w = b.wbase[m] + (int)threadIdx.x; w < b.wbase[m + 1]; w += 256) a += b.wpart[w];
  a = wave_sum(a);
  if (lane == 0) red[wave] = a;
  __syncthreads();
  if (threadIdx.x == 0) b.wnorm2[m] = ((red[0] + red[1]) + red[2]) + red[3];
}

// ---------------------------------------------------------------------------
// Ranks below one MFMA tile (r = 4, 8). Each element of H = C P^T has only r
// terms, so it is formed on the VALU in fp32, in rank order with every
// product and sum rounded separately: h = ((c0 p0 + c1 p1) + c2 p2) + ...
// ||H||^2 comes from the Gram identity with fp64 Gram matrices of C and P
// (products of fp32 or bf16 values are exact in fp64; fixed-order sums), and
// ||W||^2 from the same W stream as the tiled ranks. The launches mirror the
// tiled ones: norms (Gram and W-stream workgroups), one scale workgroup per
// item, the update (or the reconstruction), and for a carried norm the
// per-item sum of the written squares.
// ---------------------------------------------------------------------------
constexpr int64_t kSmallGramRows = 4096;      // rows of C or P per Gram workgroup
constexpr int64_t kSmallUpdateChunks = 2048;  // 8-column chunks per update workgroup (8 per thread)

template <int R>
struct SmallShape {
  static constexpr int NQ = R * (R + 1) / 2;  // upper-triangle entries of an R x R Gram matrix
};

template <int R>
__device__ __forceinline__ void small_row(const float* __restrict__ C, int64_t row, double (&v)[R]) {
#pragma unroll
  for (int a = 0; a < R; a += 4) {
    const float4 c = *reinterpret_cast<const float4*>(C + row * R + a);
    v[a] = c.x; v[a + 1] = c.y; v[a + 2] = c.z; v[a + 3] = c.w;
  }
}
template <int R>
__device__ __forceinline__ void small_row(const uint16_t* __restrict__ P, int64_t row, double (&v)[R]) {
  float f[R];
  load_bf16_row<R>(P + row * R, f);
#pragma unroll
  for (int a = 0; a < R; ++a) v[a] = f[a];
}

// Upper triangle of the Gram matrix of rows [row0, row1) of src (R columns),
// summed per thread over its rows in order, then lanes by butterfly and
// waves in order; written by threads 0 .. NQ-1.
template <int R, typename T>
__device__ void small_gram_partial(const T* __restrict__ src, int64_t row0, int64_t row1, double* __restrict__ out,
                                   double* red) {
  constexpr int NQ = SmallShape<R>::NQ;
  const int lane = threadIdx.x & 63, wave = wave_index();
  double acc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) acc[q] = 0.0;
  for (int64_t row = row0 + threadIdx.x; row < row1; row += 256) {
    double v[R];
    small_row<R>(src, row, v);
    int q = 0;
#pragma unroll
    for (int a = 0; a < R; ++a)
#pragma unroll
      for (int c = a; c < R; ++c) acc[q++] += v[a] * v[c];
  }
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const double t = wave_sum(acc[q]);
    if (lane == 0) red[wave * NQ + q] = t;
  }
  __syncthreads();
  if (threadIdx.x < NQ) {
    const int q = threadIdx.x;
    out[q] = ((red[q] + red[NQ + q]) + red[2 * NQ + q]) + red[3 * NQ + q];
  }
}

// Gram workgroups first (per item the C-row chunks, then the P-row chunks),
// then the W-stream workgroups.
template <int R>
__global__ __launch_bounds__(256) void small_norms_kernel(ApplyBatch b) {
  constexpr int NQ = SmallShape<R>::NQ;
  __shared__ double red[4 * NQ];
  const int w = blockIdx.x;
  const int ng = b.gbase[b.n];
  if (w < ng) {
    const int m = item_of(b.gbase, b.n, w);
    const ApplyItem& it = b.it[m];
    const int l = w - b.gbase[m];
    double* out = b.sgram + (int64_t)w * NQ;
    if (l < b.ncg[m]) {
      const int64_t r0 = l * kSmallGramRows, r1 = r0 + kSmallGramRows < it.d ? r0 + kSmallGramRows : it.d;
      small_gram_partial<R>(it.C, r0, r1, out, red);
    } else {
      const int64_t r0 = (l - b.ncg[m]) * kSmallGramRows, r1 = r0 + kSmallGramRows < it.k ? r0 + kSmallGramRows : it.k;
      small_gram_partial<R>(it.P, r0, r1, out, red);
    }
    return;
  }
  const int sw = w - ng;
  const int m = item_of(b.sbase, b.n, sw);
  const ApplyItem& it = b.it[m];
  const int64_t total = it.d * (it.k >> 3);
  const int64_t c0 = (sw - b.sbase[m]) * kWStreamChunks;
  const int64_t c1 = c0 + kWStreamChunks < total ? c0 + kWStreamChunks : total;
  const double sq = wstream_sumsq<false>(it.W, it.ldw, it.k, c0, c1, red);
  if (threadIdx.x == 0) b.partials[sw] = sq;
}

// One workgroup per item: the Gram partials summed entry by entry in
// workgroup order, ||H||^2 = sum_ab G_ab M_ab (off-diagonal entries twice),
// ||W||^2 from the W-stream partials (or carried), then s and the flag.
template <int R>
__global__ __launch_bounds__(256) void small_scale_kernel(ApplyBatch b) {
  constexpr int NQ = SmallShape<R>::NQ;
  const int m = blockIdx.x;
  const int t = threadIdx.x;
  double ah = 0.0;
  if (t < NQ) {
    const int nc = b.ncg[m], np = b.gbase[m + 1] - b.gbase[m] - nc;
    const double* gc = b.sgram + (int64_t)b.gbase[m] * NQ + t;
    const double* gp = gc + (int64_t)nc * NQ;
    double G = 0.0, M = 0.0;
    for (int i = 0; i < nc; ++i) G += gc[(int64_t)i * NQ];
    for (int i = 0; i < np; ++i) M += gp[(int64_t)i * NQ];
    int a = 0, q = t;  // entry t of the upper triangle is (a, a + q) after the loop
    while (q >= R - a) {
      q -= R - a;
      ++a;
    }
    ah = (q == 0 ? 1.0 : 2.0) * G * M;
  }
  double aw = 0.0;
  if (b.carry != kCarryIn)
    for (int w = b.sbase[m] + t; w < b.sbase[m + 1]; w += 256) aw += b.partials[w];
  finish_scale(b, m, aw, ah);
}

// One thread per 8-column chunk of a row (eight chunks per thread, a
// workgroup per kSmallUpdateChunks chunks of one item): h of the chunk on the
// VALU, then (MODE) the H store, or v = fp32(w - fp32(s h)) rounded
// stochastically with the chunk's Philox word, as the tiled update rounds it.
template <int R, int MODE>
__global__ __launch_bounds__(256) void small_update_kernel(ApplyBatch b) {
  const int w = blockIdx.x;
  const int m = apply_item_of(b, w);
  const ApplyItem& it = b.it[m];
  constexpr bool UPD = MODE == kModeUpdate || MODE == kModeUpdateCarry;
  float s = 0.f;
  if constexpr (UPD) {
    if (b.fixed) {
      s = it.alpha;
    } else {
      s = b.scale[2 * m];
      if (b.scale[2 * m + 1] != 0.f) return;  // zero or non-finite step: W stays as it is
    }
  }
  const int64_t cpr = it.k >> 3;  // chunks per row
  const int64_t total = it.d * cpr;
  const int64_t c0 = (int64_t)(w - b.wbase[m]) * kSmallUpdateChunks;
  double sw = 0.0;
  for (int u = 0; u < (int)(kSmallUpdateChunks / 256); ++u) {
    const int64_t c = c0 + u * 256 + threadIdx.x;
    if (c >= total) break;
    const int64_t i = c / cpr, j0 = 8 * (c - i * cpr);
    float cv[R];
#pragma unroll
    for (int a = 0; a < R; a += 4) {
      const float4 q = *reinterpret_cast<const float4*>(it.C + i * R + a);
      cv[a] = q.x; cv[a + 1] = q.y; cv[a + 2] = q.z; cv[a + 3] = q.w;
    }
    float h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float p[R];
      load_bf16_row<R>(it.P + (j0 + e) * R, p);
      float acc = cv[0] * p[0];
#pragma unroll
      for (int a = 1; a < R; ++a) acc = acc + cv[a] * p[a];
      h[e] = acc;
    }
    if constexpr (MODE == kModeReconstruct) {
      float4* dst = reinterpret_cast<float4*>(b.H + i * it.k + j0);
      dst[0] = make_float4(h[0], h[1], h[2], h[3]);
      dst[1] = make_float4(h[4], h[5], h[6], h[7]);
    } else {
      uint16_t* wp = it.W + i * it.ldw + j0;
      const uint4 wv = *reinterpret_cast<const uint4*>(wp);
      const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
      uint32_t rw[4];
      rounding_words(it.seed, i, j0 >> 3, rw);
      uint32_t out[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float w0 = __uint_as_float(wd[p] << 16), w1 = __uint_as_float(wd[p] & 0xFFFF0000u);
        const float sh0 = s * h[2 * p], sh1 = s * h[2 * p + 1];
        out[p] = f32x2_to_bf16x2_sr(w0 - sh0, w1 - sh1, rw[p]);
      }
      *reinterpret_cast<uint4*>(wp) = make_uint4(out[0], out[1], out[2], out[3]);
      if constexpr (MODE == kModeUpdateCarry) {
        float sq = 0.f;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float o0 = __uint_as_float(out[p] << 16), o1 = __uint_as_float(out[p] & 0xFFFF0000u);
          sq += o0 * o0;
          sq += o1 * o1;
        }
        sw += (double)sq;
      }
    }
  }
  if constexpr (MODE == kModeUpdateCarry) {
    __shared__ double red[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    sw = wave_sum(sw);
    if (lane == 0) red[wave] = sw;
    __syncthreads();
    if (threadIdx.x == 0) b.wpart[w] = ((red[0] + red[1]) + red[2]) + red[3];
  }
}

// ---------------------------------------------------------------------------
// Test hooks: the rounding stream, the nearest-even conversion and the Philox
// generator alone.
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

__global__ void round_nearest_kernel(const float* __restrict__ v, uint16_t* __restrict__ out, int64_t n) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < n) out[idx] = (uint16_t)f32_to_bf16_rne(v[idx]);
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

// Workgroups per matrix: one per 8 tiles, or per 16 tiles for a matrix of
// at least 2048 tiles, a function of the matrix's own shape only, so that a
// matrix gets the same partition (and so the same norm sums and bits) alone
// or in any batch. Each workgroup loads and splits its C rows once per row
// block it enters, so larger matrices take longer runs: on the Qwen3-8B-
// shaped layer at r = 128 (2048-6144 tiles of 128 x 64 per matrix) 16 tiles
// measured 330 -> 316 us against 8 (32: 315 us); the Qwen3-1.7B-shaped block
// (512-1536 tiles per matrix at r = 64) is fastest with 8 (76 us; 16: 79 us,
// 32: 85 us).
constexpr int64_t kApplyUnitsPerWG = 8;
constexpr int64_t kApplyUnitsPerWGLarge = 16;
constexpr int64_t kApplyLargeUnits = 2048;

template <int R>
void apply_plan(ApplyBatch& b, int n, const int64_t* ds, const int64_t* ks) {
  using Tr = ApplyTraits<R>;
  b.wbase[0] = 0;
  for (int m = 0; m < n; ++m) {
    b.it[m].ctiles = (ks[m] + kApplyCols - 1) / kApplyCols;
    b.it[m].units = (ds[m] + Tr::ROWS - 1) / Tr::ROWS * b.it[m].ctiles;
    const int64_t per = b.it[m].units >= kApplyLargeUnits ? kApplyUnitsPerWGLarge : kApplyUnitsPerWG;
    b.wbase[m + 1] = b.wbase[m] + (int)((b.it[m].units + per - 1) / per);
  }
  b.n = n;
}

// Gram-form norms launch: per matrix and pair group ceil(d / ROWS) C-Gram
// and ceil(k / ROWS) P-Gram workgroups, and one W-stream workgroup per
// kWStreamChunks 16-byte chunks of W.
template <int R>
void gram_plan(ApplyBatch& b, int n, const int64_t* ds, const int64_t* ks) {
  using Gs = GramShape<R>;
  b.gbase[0] = 0;
  b.sbase[0] = 0;
  for (int m = 0; m < n; ++m) {
    b.ncg[m] = (int)((ds[m] + Gs::ROWS - 1) / Gs::ROWS);
    b.gbase[m + 1] = b.gbase[m] + Gs::NG * (b.ncg[m] + (int)((ks[m] + Gs::ROWS - 1) / Gs::ROWS));
    b.sbase[m + 1] = b.sbase[m] + (int)((ds[m] * (ks[m] / 8) + kWStreamChunks - 1) / kWStreamChunks);
  }
}

// Workspace: norm partials (fp64), then Gram partials (fp32), then the
// per-item Gram-form terms (fp64: block pairs, ||W||^2), then (s, flag) per
// item, then the carried norm's per-workgroup partials (fp64), each part
// 256-byte aligned.
struct ApplyWorkspace {
  size_t gram_off, hpairs_off, wnorm2_off, scale_off, wpart_off, total;
};

template <int R>
ApplyWorkspace apply_ws_layout(const ApplyBatch& b) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  ApplyWorkspace l;
  const size_t part = (size_t)b.sbase[b.n] * sizeof(double);
  const size_t gram = (size_t)b.gbase[b.n] * GramShape<R>::NE * sizeof(float);
  l.gram_off = up(part);
  l.hpairs_off = l.gram_off + up(gram);
  l.wnorm2_off = l.hpairs_off + up(kApplyMaxItems * kGramMaxPairs * sizeof(double));
  l.scale_off = l.wnorm2_off + up(kApplyMaxItems * sizeof(double));
  l.wpart_off = l.scale_off + up(2 * kApplyMaxItems * sizeof(float));
  l.total = l.wpart_off + up((size_t)b.wbase[b.n] * sizeof(double));
  return l;
}

// A lone matrix whose update workgroups would leave compute units idle (one
// 4096 x 4096 matrix at r = 64: 2048 tiles in 128 workgroups of 16) takes
// fewer tiles per workgroup, one or two workgroups per compute unit: the
// square layer's update 42.0 -> 34-38 us. Only for the plain and fixed-scale
// updates, whose bits do not depend on the partition; the carried norm's
// partial sums follow it, so that form keeps the per-shape partition (and so
// its values alone and in a batch agree). Giving every matrix of 2048 to 4095
// tiles four tiles per workgroup instead made the Qwen3-8B-shaped layer's
// update slower (264 -> 326 us).
template <int R>
void fill_lone_matrix(ApplyBatch& b) {
  if (b.n != 1) return;
  const int64_t slots = (int64_t)device_compute_units() * ApplyShape<R, kModeUpdate>::PER_CU;
  if (b.wbase[1] >= slots) return;
  const int64_t per = b.it[0].units / slots > 1 ? b.it[0].units / slots : 1;
  b.wbase[1] = (int)((b.it[0].units + per - 1) / per);
}

template <int R>
void apply_plan_all(ApplyBatch& b, int n, const int64_t* ds, const int64_t* ks) {
  apply_plan<R>(b, n, ds, ks);
  gram_plan<R>(b, n, ds, ks);
}

template <int R>
size_t apply_ws_for(int n, const int64_t* ds, const int64_t* ks) {
  ApplyBatch b = {};
  apply_plan_all<R>(b, n, ds, ks);
  return apply_ws_layout<R>(b).total;
}

template <int R>
rgc_status_t apply_launch(int n, uint16_t* const* Ws, const int64_t* ldws, const float* const* Cs,
                          const uint16_t* const* Ps, const int64_t* ds, const int64_t* ks, float tau,
                          const uint64_t* seeds, float* const* stats, void* ws, hipStream_t st,
                          const float* alphas = nullptr, int carry = kCarryNone, double* wnorm2 = nullptr) {
  ApplyBatch b = {};
  apply_plan_all<R>(b, n, ds, ks);
  b.tau = tau;
  b.fixed = alphas ? 1 : 0;
  b.carry = carry;
  for (int m = 0; m < n; ++m) {
    b.it[m].W = Ws[m];
    b.it[m].ldw = ldws[m];
    b.it[m].C = Cs[m];
    b.it[m].P = Ps[m];
    b.it[m].d = ds[m];
    b.it[m].k = ks[m];
    b.it[m].seed = seeds[m];
    b.it[m].stats = stats ? stats[m] : nullptr;
    b.it[m].alpha = alphas ? alphas[m] : 0.f;
  }
  if (alphas) {  // fixed scale: the update sweep alone, no workspace
    fill_lone_matrix<R>(b);
    hipLaunchKernelGGL((apply_kernel<R, kModeUpdate>), dim3((unsigned)b.wbase[n]), dim3(ApplyTraits<R>::THREADS), 0,
                       st, b);
    return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
  }
  const ApplyWorkspace l = apply_ws_layout<R>(b);
  b.partials = static_cast<double*>(ws);
  b.gram = reinterpret_cast<float*>(static_cast<char*>(ws) + l.gram_off);
  b.hpairs = reinterpret_cast<double*>(static_cast<char*>(ws) + l.hpairs_off);
  b.wnorm2 = carry != kCarryNone ? wnorm2 : reinterpret_cast<double*>(static_cast<char*>(ws) + l.wnorm2_off);
  b.scale = reinterpret_cast<float*>(static_cast<char*>(ws) + l.scale_off);
  b.wpart = reinterpret_cast<double*>(static_cast<char*>(ws) + l.wpart_off);
  // with a carried ||W|| there is no W stream
  const int nw = carry == kCarryIn ? 0 : b.sbase[n];
  if (wstream_own_launch<R>()) {
    if (nw > 0) hipLaunchKernelGGL(wstream_kernel, dim3((unsigned)nw), dim3(256), 0, st, b);
    hipLaunchKernelGGL(gram_norms_kernel<R>, dim3((unsigned)b.gbase[n]), dim3(256), 0, st, b);
  } else {
    hipLaunchKernelGGL(gram_norms_kernel<R>, dim3((unsigned)(b.gbase[n] + nw)), dim3(256), 0, st, b);
  }
  hipLaunchKernelGGL(gram_reduce_kernel<R>, dim3((unsigned)(n * GramShape<R>::NP)), dim3(256), 0, st, b);
  constexpr unsigned T = ApplyTraits<R>::THREADS;
  if (carry == kCarryNone) {
    fill_lone_matrix<R>(b);  // the norms launches above took b as it was
    hipLaunchKernelGGL((apply_kernel<R, kModeUpdate>), dim3((unsigned)b.wbase[n]), dim3(T), 0, st, b);
  } else {
    hipLaunchKernelGGL((apply_kernel<R, kModeUpdateCarry>), dim3((unsigned)b.wbase[n]), dim3(T), 0, st, b);
    hipLaunchKernelGGL(carry_norm_kernel, dim3((unsigned)n), dim3(256), 0, st, b);
  }
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

// Small ranks: update workgroups per kSmallUpdateChunks chunks of W, Gram
// workgroups per kSmallGramRows rows of C and of P, W-stream workgroups as
// for the tiled ranks. All functions of each matrix's own shape.
template <int R>
void small_plan(ApplyBatch& b, int n, const int64_t* ds, const int64_t* ks) {
  b.n = n;
  b.wbase[0] = b.gbase[0] = b.sbase[0] = 0;
  for (int m = 0; m < n; ++m) {
    const int64_t chunks = ds[m] * (ks[m] / 8);
    b.wbase[m + 1] = b.wbase[m] + (int)((chunks + kSmallUpdateChunks - 1) / kSmallUpdateChunks);
    b.ncg[m] = (int)((ds[m] + kSmallGramRows - 1) / kSmallGramRows);
    b.gbase[m + 1] = b.gbase[m] + b.ncg[m] + (int)((ks[m] + kSmallGramRows - 1) / kSmallGramRows);
    b.sbase[m + 1] = b.sbase[m] + (int)((chunks + kWStreamChunks - 1) / kWStreamChunks);
  }
}

// Workspace: W-stream partials, Gram partials, ||W||^2, (s, flag), and the
// carried norm's per-workgroup partials, each part 256-byte aligned.
template <int R>
ApplyWorkspace small_ws_layout(const ApplyBatch& b) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  ApplyWorkspace l;
  l.gram_off = up((size_t)b.sbase[b.n] * sizeof(double));
  l.hpairs_off = l.gram_off + up((size_t)b.gbase[b.n] * SmallShape<R>::NQ * sizeof(double));
  l.wnorm2_off = l.hpairs_off;
  l.scale_off = l.wnorm2_off + up(kApplyMaxItems * sizeof(double));
  l.wpart_off = l.scale_off + up(2 * kApplyMaxItems * sizeof(float));
  l.total = l.wpart_off + up((size_t)b.wbase[b.n] * sizeof(double));
  return l;
}

template <int R>
size_t small_ws_for(int n, const int64_t* ds, const int64_t* ks) {
  ApplyBatch b = {};
  small_plan<R>(b, n, ds, ks);
  return small_ws_layout<R>(b).total;
}

template <int R>
rgc_status_t small_apply_launch(int n, uint16_t* const* Ws, const int64_t* ldws, const float* const* Cs,
                                const uint16_t* const* Ps, const int64_t* ds, const int64_t* ks, float tau,
                                const uint64_t* seeds, float* const* stats, void* ws, hipStream_t st,
                                const float* alphas = nullptr, int carry = kCarryNone, double* wnorm2 = nullptr) {
  ApplyBatch b = {};
  small_plan<R>(b, n, ds, ks);
  b.tau = tau;
  b.fixed = alphas ? 1 : 0;
  b.carry = carry;
  for (int m = 0; m < n; ++m) {
    b.it[m].W = Ws[m];
    b.it[m].ldw = ldws[m];
    b.it[m].C = Cs[m];
    b.it[m].P = Ps[m];
    b.it[m].d = ds[m];
    b.it[m].k = ks[m];
    b.it[m].seed = seeds[m];
    b.it[m].stats = stats ? stats[m] : nullptr;
    b.it[m].alpha = alphas ? alphas[m] : 0.f;
  }
  const int G = b.wbase[n];
  if (alphas) {
    hipLaunchKernelGGL((small_update_kernel<R, kModeUpdate>), dim3((unsigned)G), dim3(256), 0, st, b);
    return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
  }
  const ApplyWorkspace l = small_ws_layout<R>(b);
  char* base = static_cast<char*>(ws);
  b.partials = reinterpret_cast<double*>(base);
  b.sgram = reinterpret_cast<double*>(base + l.gram_off);
  b.wnorm2 = carry != kCarryNone ? wnorm2 : reinterpret_cast<double*>(base + l.wnorm2_off);
  b.scale = reinterpret_cast<float*>(base + l.scale_off);
  b.wpart = reinterpret_cast<double*>(base + l.wpart_off);
  const int nw = carry == kCarryIn ? 0 : b.sbase[n];  // with a carried ||W||, no W stream
  hipLaunchKernelGGL(small_norms_kernel<R>, dim3((unsigned)(b.gbase[n] + nw)), dim3(256), 0, st, b);
  hipLaunchKernelGGL(small_scale_kernel<R>, dim3((unsigned)n), dim3(256), 0, st, b);
  if (carry == kCarryNone) {
    hipLaunchKernelGGL((small_update_kernel<R, kModeUpdate>), dim3((unsigned)G), dim3(256), 0, st, b);
  } else {
    hipLaunchKernelGGL((small_update_kernel<R, kModeUpdateCarry>), dim3((unsigned)G), dim3(256), 0, st, b);
    hipLaunchKernelGGL(carry_norm_kernel, dim3((unsigned)n), dim3(256), 0, st, b);
  }
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

template <int R>
rgc_status_t small_reconstruct_launch(const float* C, const uint16_t* P, float* H, int64_t d, int64_t k,
                                      hipStream_t st) {
  ApplyBatch b = {};
  small_plan<R>(b, 1, &d, &k);
  b.it[0].C = C;
  b.it[0].P = P;
  b.it[0].d = d;
  b.it[0].k = k;
  b.H = H;
  hipLaunchKernelGGL((small_update_kernel<R, kModeReconstruct>), dim3((unsigned)b.wbase[1]), dim3(256), 0, st, b);
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

template <int R>
rgc_status_t reconstruct_launch(const float* C, const uint16_t* P, float* H, int64_t d, int64_t k, hipStream_t st) {
  ApplyBatch b = {};
  apply_plan<R>(b, 1, &d, &k);
  b.it[0].C = C;
  b.it[0].P = P;
  b.it[0].d = d;
  b.it[0].k = k;
  b.H = H;
  hipLaunchKernelGGL((apply_kernel<R, kModeReconstruct>), dim3((unsigned)b.wbase[1]), dim3(ApplyTraits<R>::THREADS), 0,
                     st, b);
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

rgc_status_t check_apply_shape(int64_t ldw, int64_t d, int64_t k, int64_t r) {
  return (d <= 0 || k <= 0 || r > k || ldw < k) ? RGC_ERR_SHAPE : RGC_OK;
}

rgc_status_t check_apply_item(const uint16_t* W, int64_t ldw, const float* C, const uint16_t* P, int64_t d,
                              int64_t k, const float* stats) {
  // element indices are 32-bit inside the kernels, and so are the byte
  // offsets of a tile's rows from its origin
  if ((d % 8) != 0 || (k % 8) != 0 || d > kMaxApplyDim || k > kMaxApplyDim || ldw > kMaxLeadingDim ||
      d * k > kMaxApplyElems)
    return RGC_ERR_UNSUPPORTED;
  if (!W || !C || !P) return RGC_ERR_NULL;
  if (!aligned16(W) || !aligned16(C) || !aligned16(P) || (ldw % 8) != 0) return RGC_ERR_ALIGN;
  if (stats && !aligned_to(stats, 4)) return RGC_ERR_ALIGN;
  return RGC_OK;
}

}  // namespace

rgc_status_t apply_validate(const uint16_t* W, int64_t ldw, const float* C, const uint16_t* P, int64_t d, int64_t k,
                            int64_t r, bool scaled, float step, const float* stats) {
  if (check_apply_shape(ldw, d, k, r) != RGC_OK) return RGC_ERR_SHAPE;
  if (!rank_supported(r)) return RGC_ERR_UNSUPPORTED;
  const rgc_status_t st = check_apply_item(W, ldw, C, P, d, k, stats);
  if (st != RGC_OK) return st;
  if (scaled && !std::isfinite(step)) return RGC_ERR_VALUE;
  return RGC_OK;
}

}  // namespace rgc

using namespace rgc;

extern "C" size_t rgc_apply_batch_workspace_size(int64_t n, const int64_t* ds, const int64_t* ks, int64_t r) {
  if (n <= 0 || n > kApplyMaxItems || !ds || !ks || !rank_supported(r)) return 0;
  for (int64_t m = 0; m < n; ++m)
    if (ds[m] <= 0 || ks[m] <= 0) return 0;
  size_t out = 0;
  if (dispatch_small_rank(r, [&](auto rc) { out = small_ws_for<decltype(rc)::value>((int)n, ds, ks); })) return out;
  dispatch_rank(r, [&](auto rc) { out = apply_ws_for<decltype(rc)::value>((int)n, ds, ks); });
  return out;
}

extern "C" rgc_status_t rgc_apply_batch(int64_t n, uint16_t* const* Ws, const int64_t* ldws, const float* const* Cs,
                                        const uint16_t* const* Ps, const int64_t* ds, const int64_t* ks, int64_t r,
                                        float tau, const uint64_t* seeds, float* const* stats, void* ws,
                                        size_t ws_bytes, void* stream) {
  if (n < 0 || r <= 0) return RGC_ERR_SHAPE;
  if (n > kApplyMaxItems) return RGC_ERR_UNSUPPORTED;
  if (n == 0) return RGC_OK;
  if (!Ws || !ldws || !Cs || !Ps || !ds || !ks || !seeds) return RGC_ERR_NULL;
  for (int64_t m = 0; m < n; ++m)
    if (check_apply_shape(ldws[m], ds[m], ks[m], r) != RGC_OK) return RGC_ERR_SHAPE;
  if (!rank_supported(r)) return RGC_ERR_UNSUPPORTED;
  for (int64_t m = 0; m < n; ++m) {
    const rgc_status_t st = check_apply_item(Ws[m], ldws[m], Cs[m], Ps[m], ds[m], ks[m], stats ? stats[m] : nullptr);
    if (st != RGC_OK) return st;
  }
  const size_t need = rgc_apply_batch_workspace_size(n, ds, ks, r);
  if (!ws || ws_bytes < need) return RGC_ERR_WORKSPACE;
  if (!aligned_to(ws, 256)) return RGC_ERR_ALIGN;
  rgc_status_t st = RGC_OK;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (dispatch_small_rank(r, [&](auto rc) {
        st = small_apply_launch<decltype(rc)::value>((int)n, Ws, ldws, Cs, Ps, ds, ks, tau, seeds, stats, ws, hs);
      }))
    return st;
  dispatch_rank(r, [&](auto rc) {
    st = apply_launch<decltype(rc)::value>((int)n, Ws, ldws, Cs, Ps, ds, ks, tau, seeds, stats, ws, hs);
  });
  return st;
}

extern "C" rgc_status_t rgc_apply_carried_batch(int64_t n, uint16_t* const* Ws, const int64_t* ldws,
                                                const float* const* Cs, const uint16_t* const* Ps, const int64_t* ds,
                                                const int64_t* ks, int64_t r, float tau, const uint64_t* seeds,
                                                float* const* stats, double* wnorm2, int fresh, void* ws,
                                                size_t ws_bytes, void* stream) {
  if (n < 0 || r <= 0) return RGC_ERR_SHAPE;
  if (n > kApplyMaxItems) return RGC_ERR_UNSUPPORTED;
  if (n == 0) return RGC_OK;
  if (!Ws || !ldws || !Cs || !Ps || !ds || !ks || !seeds || !wnorm2) return RGC_ERR_NULL;
  for (int64_t m = 0; m < n; ++m)
    if (check_apply_shape(ldws[m], ds[m], ks[m], r) != RGC_OK) return RGC_ERR_SHAPE;
  if (!rank_supported(r)) return RGC_ERR_UNSUPPORTED;
  for (int64_t m = 0; m < n; ++m) {
    const rgc_status_t st = check_apply_item(Ws[m], ldws[m], Cs[m], Ps[m], ds[m], ks[m], stats ? stats[m] : nullptr);
    if (st != RGC_OK) return st;
  }
  if (!aligned_to(wnorm2, 8)) return RGC_ERR_ALIGN;
  const size_t need = rgc_apply_batch_workspace_size(n, ds, ks, r);
  if (!ws || ws_bytes < need) return RGC_ERR_WORKSPACE;
  if (!aligned_to(ws, 256)) return RGC_ERR_ALIGN;
  rgc_status_t st = RGC_OK;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const int carry = fresh ? kCarryFresh : kCarryIn;
  if (dispatch_small_rank(r, [&](auto rc) {
        st = small_apply_launch<decltype(rc)::value>((int)n, Ws, ldws, Cs, Ps, ds, ks, tau, seeds, stats, ws, hs,
                                                     nullptr, carry, wnorm2);
      }))
    return st;
  dispatch_rank(r, [&](auto rc) {
    st = apply_launch<decltype(rc)::value>((int)n, Ws, ldws, Cs, Ps, ds, ks, tau, seeds, stats, ws, hs, nullptr,
                                           carry, wnorm2);
  });
  return st;
}

extern "C" rgc_status_t rgc_apply_carried(uint16_t* W, int64_t ldw, const float* C, const uint16_t* P, int64_t d,
                                          int64_t k, int64_t r, float tau, uint64_t seed, float* stats,
                                          double* wnorm2, int fresh, void* ws, size_t ws_bytes, void* stream) {
  if (d <= 0 || k <= 0 || r <= 0) return RGC_ERR_SHAPE;
  return rgc_apply_carried_batch(1, &W, &ldw, &C, &P, &d, &k, r, tau, &seed, &stats, wnorm2, fresh, ws, ws_bytes,
                                 stream);
}

extern "C" size_t rgc_apply_workspace_size(int64_t d, int64_t k, int64_t r) {
  return rgc_apply_batch_workspace_size(1, &d, &k, r);
}

extern "C" rgc_status_t rgc_apply(uint16_t* W, int64_t ldw, const float* C, const uint16_t* P, int64_t d, int64_t k,
                                  int64_t r, float tau, uint64_t seed, float* stats, void* ws, size_t ws_bytes,
                                  void* stream) {
  if (d <= 0 || k <= 0 || r <= 0) return RGC_ERR_SHAPE;
  return rgc_apply_batch(1, &W, &ldw, &C, &P, &d, &k, r, tau, &seed, &stats, ws, ws_bytes, stream);
}

extern "C" rgc_status_t rgc_apply_scaled_batch(int64_t n, uint16_t* const* Ws, const int64_t* ldws,
                                               const float* const* Cs, const uint16_t* const* Ps, const int64_t* ds,
                                               const int64_t* ks, int64_t r, const float* alphas,
                                               const uint64_t* seeds, void* stream) {
  if (n < 0 || r <= 0) return RGC_ERR_SHAPE;
  if (n > kApplyMaxItems) return RGC_ERR_UNSUPPORTED;
  if (n == 0) return RGC_OK;
  if (!Ws || !ldws || !Cs || !Ps || !ds || !ks || !alphas || !seeds) return RGC_ERR_NULL;
  for (int64_t m = 0; m < n; ++m)
    if (check_apply_shape(ldws[m], ds[m], ks[m], r) != RGC_OK) return RGC_ERR_SHAPE;
  if (!rank_supported(r)) return RGC_ERR_UNSUPPORTED;
  for (int64_t m = 0; m < n; ++m) {
    const rgc_status_t st = check_apply_item(Ws[m], ldws[m], Cs[m], Ps[m], ds[m], ks[m], nullptr);
    if (st != RGC_OK) return st;
    if (!std::isfinite(alphas[m])) return RGC_ERR_VALUE;
  }
  rgc_status_t st = RGC_OK;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (dispatch_small_rank(r, [&](auto rc) {
        st = small_apply_launch<decltype(rc)::value>((int)n, Ws, ldws, Cs, Ps, ds, ks, 0.f, seeds, nullptr, nullptr,
                                                     hs, alphas);
      }))
    return st;
  dispatch_rank(r, [&](auto rc) {
    st = apply_launch<decltype(rc)::value>((int)n, Ws, ldws, Cs, Ps, ds, ks, 0.f, seeds, nullptr, nullptr, hs, alphas);
  });
  return st;
}

extern "C" rgc_status_t rgc_apply_scaled(uint16_t* W, int64_t ldw, const float* C, const uint16_t* P, int64_t d,
                                         int64_t k, int64_t r, float alpha, uint64_t seed, void* stream) {
  if (d <= 0 || k <= 0 || r <= 0) return RGC_ERR_SHAPE;
  return rgc_apply_scaled_batch(1, &W, &ldw, &C, &P, &d, &k, r, &alpha, &seed, stream);
}

extern "C" rgc_status_t rgc_test_reconstruct(const float* C, const uint16_t* P, float* H, int64_t d, int64_t k,
                                             int64_t r, void* stream) {
  if (d <= 0 || k <= 0 || r <= 0 || r > k) return RGC_ERR_SHAPE;
  if (!rank_supported(r) || (d % 8) != 0 || (k % 8) != 0) return RGC_ERR_UNSUPPORTED;
  if (!C || !P || !H) return RGC_ERR_NULL;
  if (!aligned16(C) || !aligned16(P) || !aligned16(H)) return RGC_ERR_ALIGN;
  rgc_status_t st = RGC_OK;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (dispatch_small_rank(r, [&](auto rc) { st = small_reconstruct_launch<decltype(rc)::value>(C, P, H, d, k, hs); }))
    return st;
  dispatch_rank(r, [&](auto rc) { st = reconstruct_launch<decltype(rc)::value>(C, P, H, d, k, hs); });
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

extern "C" rgc_status_t rgc_test_round_nearest(const float* v, uint16_t* out, int64_t n, void* stream) {
  if (n < 0 || n > (int64_t(1) << 31)) return RGC_ERR_SHAPE;
  if (n == 0) return RGC_OK;
  if (!v || !out) return RGC_ERR_NULL;
  if (!aligned_to(v, 4) || !aligned_to(out, 2)) return RGC_ERR_ALIGN;
  hipLaunchKernelGGL(round_nearest_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), v, out, n);
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

// ---------------------------------------------------------------------------
// The normalized update for callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation):
// rgc_apply with its workspace in a static device array instead of a caller
// buffer. Each device holds its own copy of the array (for as long as the
// library stays loaded); every call on a device shares it, so such calls must
// not overlap on one device. The workspace needs no initialisation (every
// partial is written before it is read), so nothing is cleared between calls.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mutex;
void* scratch_addr[kMaxScratchDevices];  // device address of `scratch` on each device, looked up once

// The current device's address of `scratch`, looked up on the first call on
// that device with the device current; the stream must belong to it.
rgc_status_t scratch_for(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return RGC_ERR_HIP;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return RGC_ERR_HIP;
    if (sdev != dev) return RGC_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RGC_ERR_HIP;
    scratch_addr[dev] = p;
  }
  *out = scratch_addr[dev];
  return RGC_OK;
}

}  // namespace

extern "C" rgc_status_t rgc_apply_noalloc(uint16_t* W, int64_t ldw, const float* C, const uint16_t* P, int64_t d,
                                          int64_t k, int64_t r, float tau, uint64_t seed, float* stats,
                                          void* stream) {
  rgc_status_t st = apply_validate(W, ldw, C, P, d, k, r, false, 0.f, stats);
  if (st != RGC_OK) return st;
  const size_t need = rgc_apply_workspace_size(d, k, r);
  if (need == 0 || need > kNoAllocScratchBytes) return RGC_ERR_SCRATCH;
  void* ptr = nullptr;
  st = scratch_for(static_cast<hipStream_t>(stream), &ptr);
  if (st != RGC_OK) return st;
  return rgc_apply(W, ldw, C, P, d, k, r, tau, seed, stats, ptr, kNoAllocScratchBytes, stream);
}
