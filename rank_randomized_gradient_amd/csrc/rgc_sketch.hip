// The two skinny contractions of the sketch, on bf16 MFMA with fp32 sums:
//   project:    XP = bf16(X P)         X: T x k, P: k x r      [RGC, "How it works"]
//   accumulate: C += D^T XP            D: T x d, XP: T x r     [RGC, "How it works";
//                                      LoGRA-S, Key Contributions 1]
// ([RGC] = page "Randomized Gradient Compression"; [LoGRA-S] = page "LoGRA:
// Scaling LLM Reinforcement Learning with Low-Rank Gradient Sketches".)
//
// Both are GEMMs with a long K (k, or tokens), a short M (the rank r) and an N
// (tokens, or d) whose operand is read from HBM exactly once: the "stream"
// operand (X or D) carries nearly all the bytes, the "rank" operand (P or XP)
// is small and re-read from L2 by every N-tile. At r <= 128 they are
// HBM-bound, so the design is about keeping enough stream bytes in flight:
//
// * A wave computes a 64 (N) x RPW (r) tile: four 16x16 MFMA N-tiles per
//   M-tile. A workgroup of NR x KS waves covers all of r and splits each
//   K-block of 32*KS rows among its KS waves (summed through LDS at the end
//   of a tile).
// * The rank operand's register transpose puts r on the MFMA's M side: a lane
//   loads CPL consecutive r columns for eight consecutive K rows and repacks
//   them, so M-tile c row m is r = base + CPL*m + c and each lane's output is
//   a contiguous run of 4*CPL values of r (contiguous C and XP stores). D is
//   token-major, so it gets the same transpose on the N side: lane (n, g)
//   reads d = 4n .. 4n+3 of eight tokens and N-tile c column n is d = 4n + c.
// * Each wave keeps the loads of its next two K-steps in flight while it
//   multiplies the current one (three register stages). Loads are
//   unconditional: out-of-range rows are clamped to valid memory and zeroed
//   only in the last, partial K-step; addresses are a scalar base plus a
//   per-lane 32-bit offset that is fixed for the whole loop.
// * Work is balanced across the chip at K-block granularity ("stream-K"):
//   the (item, tile, K-block) units of the whole batch are cut into one
//   contiguous range per workgroup, one workgroup per compute unit. A tile that lies inside one
//   range is finished in place; a tile cut between ranges gets fp32 partials
//   (at most two per workgroup) that a second launch sums in workgroup order.
//   Every reduction has a fixed order, so results are bit-reproducible, and
//   there is no signalling between workgroups inside a launch (a device-scope
//   release costs an L2 writeback per wave on this part). Consecutive ranges
//   are placed on the same XCD, so the tiles of one item share that XCD's L2
//   for the rank operand.
#include "rgc_internal.hpp"

namespace rgc {

// ---------------------------------------------------------------------------
// Shared pieces
// ---------------------------------------------------------------------------

// A K-step covers 32 rows of the K dimension. Its operands are read through a
// window of 32 rows [wb, wb + 32): in the steady state wb is the step's own
// first row k0; for the last, partial step (and for prefetches past the end)
// the window is moved back to end at the K extent, so that every row it
// touches is valid memory, and rows outside [k0, end) are zeroed before use.
// A K extent below 32 clamps the lanes' row offsets once, up front.
__device__ __forceinline__ int64_t window_base(int64_t k0, int64_t end) {
  return k0 + 32 <= end ? k0 : (end >= 32 ? end - 32 : 0);
}

// Rows of a window that are valid memory for a K extent `end`.
__device__ __forceinline__ int64_t window_rows(int64_t end) { return end >= 32 ? 32 : end; }

// Pins a wave-uniform value to scalar registers. Without it the compiler may
// strength-reduce every load address of the K loop into its own 64-bit
// per-lane induction variable, which costs two VGPRs per load in flight.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ const uint16_t* uniform_ptr(const uint16_t* p) {
  return reinterpret_cast<const uint16_t*>(uniform_u64(reinterpret_cast<uint64_t>(p)));
}
__device__ __forceinline__ int64_t uniform_i64(int64_t v) { return (int64_t)uniform_u64((uint64_t)v); }

// Raw (untransposed) M-side rows of one K-step: for each column group q and
// row j = 0..7, the CPL columns the lane reads, packed in dwords.
template <int R>
struct RankRows {
  static constexpr int W = (RankTraits<R>::CPL + 1) / 2;
  uint32_t v[RankTraits<R>::NG][8][W];
};

// Per-lane byte offsets of eight rows, relative to a window's first row.
struct RowOffsets {
  uint32_t off[8];
};

// Rows 8g + j (j = 0..7) of a row-major bf16 matrix with row stride R, at
// columns CPL*m (m = lane % 16, g = lane / 16), clamped into `rows` rows.
template <int R>
__device__ __forceinline__ RowOffsets rank_row_offsets(int lane, int64_t rows) {
  constexpr int CPL = RankTraits<R>::CPL;
  const int m = lane & 15, g = lane >> 4;
  RowOffsets o;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t row = 8 * g + j < rows ? 8 * g + j : rows - 1;
    o.off[j] = (uint32_t)((row * R + CPL * m) * 2);
  }
  return o;
}

// Loads a K-step's rank rows; `win` points at the window's first row and the
// wave's first column. The rank operand is re-read by every N-tile, so these
// loads keep the default (cached) policy.
template <int R>
__device__ __forceinline__ void load_rank_rows(const uint16_t* win, const RowOffsets& o, RankRows<R>& out) {
  using Tr = RankTraits<R>;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int q = 0; q < Tr::NG; ++q) {
      const uint32_t off = o.off[j] + q * Tr::GW * 2;
      if constexpr (Tr::CPL == 4) {
        const u32x2v_t v = load_cached<u32x2v_t>(win, off);
        out.v[q][j][0] = v.x;
        out.v[q][j][1] = v.y;
      } else if constexpr (Tr::CPL == 2) {
        out.v[q][j][0] = load_cached<uint32_t>(win, off);
      } else {
        out.v[q][j][0] = load_cached<uint16_t>(win, off);
      }
    }
}

// Zeroes the rows of a window that lie outside [k0, end).
template <int R>
__device__ __forceinline__ void mask_rank_rows(int64_t wb, int64_t k0, int64_t end, int lane, RankRows<R>& rows) {
  const int g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t row = wb + 8 * g + j;
    const bool ok = row >= k0 && row < end;
#pragma unroll
    for (int q = 0; q < RankTraits<R>::NG; ++q)
#pragma unroll
      for (int w = 0; w < RankRows<R>::W; ++w) rows.v[q][j][w] = ok ? rows.v[q][j][w] : 0u;
  }
}

template <int R>
__device__ __forceinline__ void transpose_rank_rows(const RankRows<R>& rows, uint32_t (&aop)[RankTraits<R>::MT][4]) {
  using Tr = RankTraits<R>;
#pragma unroll
  for (int q = 0; q < Tr::NG; ++q)
#pragma unroll
    for (int c = 0; c < Tr::CPL; ++c) transpose_8xcpl<Tr::CPL>(rows.v[q], c, aop[q * Tr::CPL + c]);
}

// N-tiles (16 columns each) per wave, and the workgroup's N extent.
constexpr int kNT = 4;
constexpr int kTileN = 16 * kNT;

// The register budget (at most 256 VGPRs + AGPRs per wave) and the LDS of
// the wave reduction are sized so that two workgroups fit on a compute unit.
constexpr int kWorkgroupsPerCU = 2;

// K-steps in flight per wave: the loads of step s + kStages - 1 are issued
// before step s is multiplied. The stage buffers are indexed with
// compile-time constants in an unrolled loop, so rotating them costs no
// register copies (and no early waits).
// (Two for r = 48, whose rank operand takes three column groups of 16-bit
// loads and would not fit three stages in the register budget.)
template <int R>
constexpr int stages() { return R == 48 ? 2 : 3; }

template <int R>
using AccTile = f32x4_t[RankTraits<R>::MT][kNT];

// The N-tiles of a wave's output are split among the KS waves that share an
// r-slice: wave ks owns N-tiles nt with nt % KS == ks, and after the
// reduction below it holds the finished sums for exactly those.
template <int KS>
__device__ __forceinline__ constexpr bool owns_ntile(int nt, int ks) { return (nt % KS) == ks; }

template <int R>
constexpr int reduce_lds_floats() {
  using Tr = RankTraits<R>;
  return Tr::KS > 1 ? Tr::KS * Tr::NR * Tr::MT * kNT * 4 * 64 : 1;
}

// Sums the KS waves' accumulators through LDS: every wave stores all of its
// tile, then each wave adds, for the N-tiles it owns, the KS copies in wave
// order (fixed order, so the result does not depend on timing). The leading
// barrier lets the LDS be reused from one tile to the next.
template <int R>
__device__ __forceinline__ void reduce_waves(AccTile<R>& acc, float* lds, int rw, int ks, int lane) {
  using Tr = RankTraits<R>;
  constexpr int KS = Tr::KS;
  constexpr int E = Tr::MT * kNT * 4;  // floats per lane
  if constexpr (KS > 1) {
    __syncthreads();
    float* mine = lds + (ks * Tr::NR + rw) * E * 64;
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int mt = 0; mt < Tr::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[((nt * Tr::MT + mt) * 4 + i) * 64 + lane] = acc[mt][nt][i];
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      if (!owns_ntile<KS>(nt, ks)) continue;
#pragma unroll
      for (int mt = 0; mt < Tr::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = 0.f;
#pragma unroll
          for (int w = 0; w < KS; ++w) {
            const float x = lds[((w * Tr::NR + rw) * E + (nt * Tr::MT + mt) * 4 + i) * 64 + lane];
            v = (w == 0) ? x : v + x;
          }
          acc[mt][nt][i] = v;
        }
    }
  }
}

// Gathers, for N-tile `nt` and column group q, the 4*CPL contiguous rank
// values a lane owns: out[CPL*i + c] = acc[q*CPL + c][nt][i], which are
// r = base + q*GW + 4*CPL*g + (0 .. 4*CPL-1).
template <int R>
__device__ __forceinline__ void gather_rank_run(const AccTile<R>& acc, int q, int nt,
                                                float (&out)[4 * RankTraits<R>::CPL]) {
  constexpr int CPL = RankTraits<R>::CPL;
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) out[CPL * i + c] = acc[q * CPL + c][nt][i];
}

// Calls f(row, q, run) for every N-tile this wave owns in a finished tile:
// `row` is the tile-relative N index of the lane's column, row_of(nt, n),
// and run holds the lane's 4*CPL consecutive rank values of column group q,
// which start at r = rbase + q*GW + 4*CPL*g.
template <int R, typename RowOf, typename F>
__device__ __forceinline__ void for_owned_runs(const AccTile<R>& acc, int ks, int lane, RowOf row_of, F f) {
  using Tr = RankTraits<R>;
  const int n = lane & 15;
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    if (!owns_ntile<Tr::KS>(nt, ks)) continue;
#pragma unroll
    for (int q = 0; q < Tr::NG; ++q) {
      float run[4 * Tr::CPL];
      gather_rank_run<R>(acc, q, nt, run);
      f(row_of(nt, n), q, run);
    }
  }
}

template <int CPL>
__device__ __forceinline__ void store_run_f32(float* dst, const float (&run)[4 * CPL]) {
#pragma unroll
  for (int v = 0; v < CPL; ++v)
    reinterpret_cast<float4*>(dst)[v] = make_float4(run[4 * v], run[4 * v + 1], run[4 * v + 2], run[4 * v + 3]);
}

template <int CPL>
__device__ __forceinline__ void add_run_f32(float* dst, const float (&run)[4 * CPL]) {
#pragma unroll
  for (int v = 0; v < CPL; ++v) {
    float4 old = reinterpret_cast<float4*>(dst)[v];
    old.x += run[4 * v + 0];
    old.y += run[4 * v + 1];
    old.z += run[4 * v + 2];
    old.w += run[4 * v + 3];
    reinterpret_cast<float4*>(dst)[v] = old;
  }
}

template <int CPL>
__device__ __forceinline__ void store_run_bf16(uint16_t* dst, const float (&run)[4 * CPL]) {
  uint32_t packed[2 * CPL];
#pragma unroll
  for (int e = 0; e < 2 * CPL; ++e) packed[e] = pack_bf16x2(f32_to_bf16_rne(run[2 * e]), f32_to_bf16_rne(run[2 * e + 1]));
  if constexpr (CPL == 4) {
    reinterpret_cast<uint4*>(dst)[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    reinterpret_cast<uint4*>(dst)[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  } else if constexpr (CPL == 2) {
    reinterpret_cast<uint4*>(dst)[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  } else {
    reinterpret_cast<uint2*>(dst)[0] = make_uint2(packed[0], packed[1]);
  }
}

// ---------------------------------------------------------------------------
// Work items and the stream-K schedule. One launch covers a list of
// independent matrices of one rank (e.g. all projections of a transformer
// block). Units are (item, N-tile, K-block) in that order; workgroup w takes
// units [floor(w U / G), floor((w+1) U / G)).
// ---------------------------------------------------------------------------
constexpr int kMaxItems = 16;
constexpr int kNumXcds = 8;

struct Schedule {
  int n;                          // items
  int G;                          // workgroups
  int64_t tile_n;                 // N extent of a tile
  int64_t U;                      // units
  int64_t ubase[kMaxItems + 1];   // first unit of each item
  int64_t nkb[kMaxItems];         // K-blocks per tile
  int64_t tbase[kMaxItems + 1];   // first (batch-wide) tile index of each item
  int64_t kext[kMaxItems];        // K extent
  int64_t next[kMaxItems];        // N extent
};

__device__ __forceinline__ int64_t range_begin(const Schedule& s, int64_t w) { return w * s.U / s.G; }

// The workgroup whose range holds unit u: the largest w with
// range_begin(w) <= u.
__device__ __forceinline__ int64_t range_of(const Schedule& s, int64_t u) { return ((u + 1) * s.G - 1) / s.U; }

__device__ __forceinline__ int item_of_unit(const Schedule& s, int64_t u) {
  int m = 0;
  while (m + 1 < s.n && u >= s.ubase[m + 1]) ++m;
  return m;
}

__device__ __forceinline__ int item_of_tile(const Schedule& s, int64_t t) {
  int m = 0;
  while (m + 1 < s.n && t >= s.tbase[m + 1]) ++m;
  return m;
}

// The hardware hands workgroups to the XCDs round-robin; this numbers them
// so that each XCD gets a contiguous run of ranges.
__device__ __forceinline__ int64_t logical_workgroup(int64_t b, int64_t G) {
  const int64_t x = b % kNumXcds, pos = b / kNumXcds;
  const int64_t q = G / kNumXcds, rem = G % kNumXcds;
  return x * q + (x < rem ? x : rem) + pos;
}

// Partial slots: a workgroup's first segment (if it is a partial tile) goes
// to slot 2w, its last (if partial and not also the first) to slot 2w + 1.
__device__ __forceinline__ int64_t partial_slot(int64_t w, bool first_segment) {
  return 2 * w + (first_segment ? 0 : 1);
}

struct ProjectBatch {
  Schedule s;
  const uint16_t* X[kMaxItems];
  int64_t ldx[kMaxItems];
  const uint16_t* P[kMaxItems];
  uint16_t* XP[kMaxItems];
  float* part;                    // 2 G slots of kTileN x R fp32
};

struct AccumulateBatch {
  Schedule s;
  const uint16_t* D[kMaxItems];
  int64_t ldd[kMaxItems];
  const uint16_t* XP[kMaxItems];
  float* C[kMaxItems];
  float* part;                    // 2 G slots of kTileN x R fp32
};

// Runs the workgroup's range: for each segment (a run of K-blocks of one
// tile) calls begin(m, tile), then load(stage, k0) / step(stage, k0, masked)
// for its K-steps, then finish(m, tile, full, slot) with the tile's sums in
// acc (reduced across the KS waves). Steps whose K-block lies wholly inside
// the K extent run without any masking; only the epilogue, which holds the
// last (possibly partial) K-block, checks.
template <int R, typename Stage, typename Begin, typename Load, typename Step, typename Finish>
__device__ __forceinline__ void run_range(const Schedule& s, int64_t w, int ks, float* lds, int rw, int lane,
                                          AccTile<R>& acc, Begin begin, Load load, Step step, Finish finish) {
  using Tr = RankTraits<R>;
  constexpr int64_t stride = 32 * Tr::KS;
  const int64_t u0 = uniform_i64(range_begin(s, w)), u1 = uniform_i64(range_begin(s, w + 1));
  constexpr int kStages = stages<R>();
  Stage st[kStages];
  for (int64_t u = u0; u < u1;) {
    const int m = item_of_unit(s, u);
    const int64_t nkb = s.nkb[m];
    const int64_t tile = (u - s.ubase[m]) / nkb, kb0 = (u - s.ubase[m]) % nkb;
    const int64_t tile_end = s.ubase[m] + (tile + 1) * nkb;
    const int64_t seg_end = u1 < tile_end ? u1 : tile_end;
    const int64_t kb1 = kb0 + (seg_end - u);
    const int64_t kb_full = s.kext[m] / stride;  // K-blocks wholly inside the K extent
    const int64_t nfull = (kb1 < kb_full ? kb1 : kb_full) - kb0;
    begin(m, tile);
#pragma unroll
    for (int mt = 0; mt < Tr::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // this wave's K-steps start at rows kb*32*KS + 32*ks, kb in [kb0, kb1)
    const int64_t first = kb0 * stride + 32 * ks;
    const int64_t nsteps = kb1 - kb0;
#pragma unroll
    for (int v = 0; v + 1 < kStages; ++v) load(st[v], first + v * stride);
    int64_t s0 = 0;
    for (; s0 + kStages <= nfull; s0 += kStages) {
#pragma unroll
      for (int v = 0; v < kStages; ++v) {
        const int64_t k0 = first + (s0 + v) * stride;
        load(st[(v + kStages - 1) % kStages], k0 + (kStages - 1) * stride);
        // Keep each step's transposes and MFMAs between its own loads and
        // the next step's: hoisting the next step's transposes (which the
        // scheduler likes for ILP) would wait for data still in flight.
        __builtin_amdgcn_sched_barrier(0);
        step(st[v], k0, std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // at most kStages steps remain: the stages hold steps s0 .. s0+kStages-2
#pragma unroll
    for (int v = 0; v < kStages; ++v) {
      if (s0 + v >= nsteps) break;
      const int64_t k0 = first + (s0 + v) * stride;
      if (v == kStages - 1) load(st[v], k0);
      step(st[v], k0, std::true_type{});
    }
    reduce_waves<R>(acc, lds, rw, ks, lane);
    finish(m, tile, kb0 == 0 && kb1 == nkb, partial_slot(w, u == u0));
    u = seg_end;
  }
}

// ---------------------------------------------------------------------------
// project: XP = bf16(X P). N = tokens (N-tile nt column n is token
// tbase + 16*nt + n), K = k.
// ---------------------------------------------------------------------------
struct XRows {
  uint32_t v[kNT][4];  // per N-tile: 8 consecutive k of one token (16 bytes)
};

// Per-lane byte offsets, relative to (token tbase, window column), of the 16
// bytes lane (n, g) reads for N-tile nt: token tbase + 16*nt + n (tokens past
// T read token T-1; their outputs are never stored), k chunk 8g (clamped into
// a window of `rows` valid columns; rows is a multiple of 8).
struct XOffsets {
  uint32_t off[kNT];
};

__device__ __forceinline__ XOffsets x_offsets(int lane, int64_t T, int64_t tbase, int64_t ldx, int64_t rows) {
  const int n = lane & 15, g = lane >> 4;
  const int64_t kc = 8 * g + 8 <= rows ? 8 * g : rows - 8;
  XOffsets o;
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int64_t t = tbase + 16 * nt + n;
    const int64_t tc = t < T ? t : T - 1;
    o.off[nt] = (uint32_t)(((tc - tbase) * ldx + kc) * 2);
  }
  return o;
}

__device__ __forceinline__ void load_x_rows(const uint16_t* win, const XOffsets& o, XRows& out) {
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const u32x4v_t v = load_stream_16b(win, o.off[nt]);
    out.v[nt][0] = v.x;
    out.v[nt][1] = v.y;
    out.v[nt][2] = v.z;
    out.v[nt][3] = v.w;
  }
}

// Zeroes the 8-wide k chunks of a window that lie outside [k0, end).
__device__ __forceinline__ void mask_x_rows(int64_t wb, int64_t k0, int64_t end, int lane, XRows& x) {
  const int64_t c0 = wb + 8 * (lane >> 4);
  const bool ok = c0 >= k0 && c0 < end;
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
    for (int e = 0; e < 4; ++e) x.v[nt][e] = ok ? x.v[nt][e] : 0u;
}

template <int R>
__global__ __launch_bounds__(64 * RankTraits<R>::NR * RankTraits<R>::KS, kWorkgroupsPerCU) void project_kernel(
    ProjectBatch pb) {
  using Tr = RankTraits<R>;
  __shared__ float lds[reduce_lds_floats<R>()];
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int rw = wave % Tr::NR, ks = wave / Tr::NR;
  const int rbase = rw * Tr::RPW;
  const int g = lane >> 4;
  const Schedule& s = pb.s;
  const int64_t w = logical_workgroup(blockIdx.x, s.G);
  const int64_t T = s.next[0];

  struct Stage {
    RankRows<R> p;
    XRows x;
  };
  AccTile<R> acc;
  int64_t kend = 0, tbase = 0;
  const uint16_t* Xt = nullptr;
  const uint16_t* P = nullptr;
  RowOffsets po;
  XOffsets xo;
  auto begin = [&](int m, int64_t tile) {
    kend = uniform_i64(s.kext[m]);
    tbase = tile * kTileN;
    const int64_t ldx = pb.ldx[m];
    Xt = uniform_ptr(pb.X[m] + tbase * ldx);
    P = uniform_ptr(pb.P[m] + rbase);
    po = rank_row_offsets<R>(lane, window_rows(kend));
    xo = x_offsets(lane, T, tbase, ldx, window_rows(kend));
  };
  auto load = [&](Stage& b, int64_t k0) {
    const int64_t wb = window_base(k0, kend);
    load_rank_rows<R>(uniform_ptr(P + wb * R), po, b.p);
    load_x_rows(uniform_ptr(Xt + wb), xo, b.x);
  };
  auto step = [&](Stage& b, int64_t k0, auto masked) {
    if (masked && k0 + 32 > kend) {  // the last, partial K-step (wave-uniform)
      const int64_t wb = window_base(k0, kend);
      mask_rank_rows<R>(wb, k0, kend, lane, b.p);
      mask_x_rows(wb, k0, kend, lane, b.x);
    }
    uint32_t aop[Tr::MT][4];
    transpose_rank_rows<R>(b.p, aop);
#pragma unroll
    for (int mt = 0; mt < Tr::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) acc[mt][nt] = mfma_16x16x32(aop[mt], b.x.v[nt], acc[mt][nt]);
  };
  auto finish = [&](int m, int64_t tile, bool full, int64_t slot) {
    const auto row_of = [](int nt, int n) { return 16 * nt + n; };
    if (full) {
      uint16_t* XP = pb.XP[m];
      for_owned_runs<R>(acc, ks, lane, row_of, [&](int row, int q, const float (&run)[4 * Tr::CPL]) {
        if (tbase + row < T)
          store_run_bf16<Tr::CPL>(XP + (tbase + row) * R + rbase + q * Tr::GW + 4 * Tr::CPL * g, run);
      });
    } else {
      float* part = pb.part + slot * (int64_t)kTileN * R;
      for_owned_runs<R>(acc, ks, lane, row_of, [&](int row, int q, const float (&run)[4 * Tr::CPL]) {
        store_run_f32<Tr::CPL>(part + row * R + rbase + q * Tr::GW + 4 * Tr::CPL * g, run);
      });
    }
  };
  run_range<R, Stage>(s, w, ks, lds, rw, lane, acc, begin, load, step, finish);
}

// ---------------------------------------------------------------------------
// accumulate: C += D^T XP, staged through LDS. N = d, K = tokens.
//
// A workgroup tile is TILE = 64*WN columns of d by all R columns of r; its
// four waves split it WN ways along d and WR ways along r (WN * WR = 4), so
// every wave multiplies a 64 (d) x RW (r) block. A K-step is 32 tokens: the
// step's D slab (32 x TILE) and XP slab (32 x R) are copied from memory
// straight into an LDS stage by all four waves in 1 KB pieces, S stages
// ahead; each wave then reads its MFMA operands from the stage with
// transposing reads, so both token-major operands arrive in MFMA layout
// without register shuffles, and the XP slab is fetched once per workgroup.
//
// LDS layout of a stage: blocks of 4 tokens x 16 columns (128 bytes, four
// rows of four 8-byte chunks). Block (tq, b) of the D slab (b = 16-column
// block of the tile) sits at 128 * (tq * NDB + b); the XP slab's block
// (tq, b) at D_BYTES + 128 * (tq * NRB + b). Copy c fills blocks 8c .. 8c+7:
// lane l reads token (l % 8) / 2 of block 8c + l / 8, columns 8 * (l % 2)
// .. +7, which are exactly the 16 bytes that land at 16 * l.
// ---------------------------------------------------------------------------
constexpr int kAccStages = 6;

template <int R>
struct AccShape {
  static constexpr int WR = R <= 64 ? 1 : (R == 128 ? 2 : 4);  // waves along r
  static constexpr int WN = 4 / WR;                              // waves along d
  static constexpr int RW = R / WR;                              // r per wave
  static constexpr int MT = RW / 16;                             // MFMA M-tiles per wave
  static constexpr int TILE = 64 * WN;                           // d per workgroup tile
  static constexpr int NDB = TILE / 16;                          // D copies per stage
  static constexpr int NRB = R / 16;                             // XP copies per stage
  static constexpr int NI = NDB + NRB;
  static constexpr int D_BYTES = 1024 * NDB;
  static constexpr int STAGE = 1024 * NI;
  static constexpr int S = kAccStages;
  static constexpr int NV_LO = NI / 4, NV_HI = (NI + 3) / 4;  // copies per wave (waves below NI % 4 take one more)
  static_assert(RW % 16 == 0 && RW <= 64, "rank split");
  static_assert(S * STAGE <= 160 * 1024, "LDS");
  static_assert((S - 1) * NV_HI <= 63, "vector memory counter");
};

template <int R>
__global__ __launch_bounds__(256, kWorkgroupsPerCU) void accumulate_kernel(AccumulateBatch ab) {
  using Sh = AccShape<R>;
  constexpr int S = Sh::S;
  __shared__ __attribute__((aligned(1024))) char smem[S * Sh::STAGE];
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int wn = wave % Sh::WN, rw = wave / Sh::WN;
  const int g = lane >> 4, li = lane & 15;
  const Schedule& s = ab.s;
  const int64_t w = logical_workgroup(blockIdx.x, s.G);
  const int64_t T = uniform_i64(s.kext[0]);
  const int64_t u0 = uniform_i64(range_begin(s, w)), u1 = uniform_i64(range_begin(s, w + 1));
  const int64_t rows = window_rows(T);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(RGC_LDS char*)smem;
  const bool more = wave < Sh::NI % 4;  // this wave issues NV_HI copies per stage (else NV_LO)

  // ---- the copy side: a cursor over this workgroup's units, S - 1 ahead
  uint32_t voff[Sh::NV_HI];
  auto set_offsets = [&](int m, int64_t tile) {
    const int64_t d = s.next[m], ldd = ab.ldd[m], dbase = tile * Sh::TILE;
    const int j = (lane & 7) >> 1, half = lane & 1;
#pragma unroll
    for (int v = 0; v < Sh::NV_HI; ++v) {
      const int c = wave + 4 * v;
      if (c < Sh::NDB) {
        const int blk = 8 * c + (lane >> 3);
        int64_t t = 4 * (blk / Sh::NDB) + j;
        t = t < rows ? t : rows - 1;
        int64_t col = dbase + 16 * (blk % Sh::NDB) + 8 * half;
        col = col < d ? col : d - 8;  // past d: any valid chunk (its columns are never stored)
        voff[v] = (uint32_t)((t * ldd + col) * 2);
      } else {
        const int blk = 8 * (c - Sh::NDB) + (lane >> 3);
        int64_t t = 4 * (blk / Sh::NRB) + j;
        t = t < rows ? t : rows - 1;
        voff[v] = (uint32_t)((t * R + 16 * (blk % Sh::NRB) + 8 * half) * 2);
      }
    }
  };
  const int m0 = item_of_unit(s, u0);
  const int64_t tile0 = (u0 - s.ubase[m0]) / s.nkb[m0], k0 = (u0 - s.ubase[m0]) % s.nkb[m0];
  // per-item constants of the copy cursor, reloaded when it moves to the next item
  int lm = m0;
  int64_t ltile = tile0, lk = k0, lu = u0;
  int64_t l_nkb = 0, l_tiles = 0, l_ldd = 0;
  const uint16_t* l_D = nullptr;
  const uint16_t* l_XP = nullptr;
  auto enter_item = [&](int m) {
    l_nkb = uniform_i64(s.nkb[m]);
    l_tiles = uniform_i64(s.tbase[m + 1] - s.tbase[m]);
    l_ldd = uniform_i64(ab.ldd[m]);
    l_D = uniform_ptr(ab.D[m]);
    l_XP = uniform_ptr(ab.XP[m]);
  };
  if (u0 < u1) {
    enter_item(lm);
    set_offsets(lm, ltile);
  }
  uint32_t lslot = 0;  // stage of unit lu
  auto issue = [&]() {
    const int64_t wb = window_base(lk * 32, T);
    const uint16_t* Db = uniform_ptr(l_D + wb * l_ldd);
    const uint16_t* Xb = uniform_ptr(l_XP + wb * R);
    const uint32_t st = lds0 + lslot * Sh::STAGE;
    static_for<0, Sh::NV_HI>([&](auto vc) {
      constexpr int v = decltype(vc)::value;
      // copy c = wave + 4v: a D copy if c < NDB, an XP copy if NDB <= c < NI
      const int c = wave + 4 * v;
      if constexpr (4 * v + 3 < Sh::NDB) {
        dma_16b_stream(Db, voff[v], st + 1024 * c);
      } else if constexpr (4 * v >= Sh::NDB && 4 * v + 3 < Sh::NI) {
        dma_16b_cached(Xb, voff[v], st + 1024 * c);
      } else {
        if (c < Sh::NDB)
          dma_16b_stream(Db, voff[v], st + 1024 * c);
        else if (c < Sh::NI)
          dma_16b_cached(Xb, voff[v], st + 1024 * c);
      }
    });
    ++lu;
    lslot = lslot + 1 == S ? 0 : lslot + 1;
    if (++lk == l_nkb) {
      lk = 0;
      if (++ltile == l_tiles) {
        ltile = 0;
        ++lm;
        if (lu < u1) enter_item(lm);
      }
      if (lu < u1) set_offsets(lm, ltile);
    }
  };

  // ---- the compute side
  f32x4_t acc[Sh::MT][4];
  using Acc = f32x4_t[Sh::MT][4];
  auto finish = [&](const Acc& res, int m, int64_t tile, bool full, int64_t slot) {
    const int64_t d = s.next[m], dbase = tile * Sh::TILE;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t row = 64 * wn + 16 * nt + li;  // tile-relative d
#pragma unroll
      for (int mt = 0; mt < Sh::MT; ++mt) {
        const int rcol = rw * Sh::RW + 16 * mt + 4 * g;
        const f32x4_t v = res[mt][nt];
        if (full) {
          // the tile lies inside this workgroup's range: one add per element,
          // no other writer in this launch
          if (dbase + row < d) {
            float* c = ab.C[m] + (dbase + row) * R + rcol;
#pragma unroll
            for (int e = 0; e < 4; ++e) unsafeAtomicAdd(c + e, v[e]);
          }
        } else {
          float* p = ab.part + slot * Sh::TILE * R + row * R + rcol;
          *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
  };

#pragma unroll
  for (int v = 0; v + 1 < S; ++v)
    if (lu < u1) issue();

  // The first segment's sums are kept in registers and stored after the
  // range's last segment: a store issued while copies are in flight counts
  // in the same counter as the copies, so the next wait would drain the
  // whole pipeline. Later segments (each a whole tile or the range's last
  // piece) are stored as they finish.
  f32x4_t keep[Sh::MT][4];
  bool kept = false, kept_full = false;
  int64_t kept_tile = tile0;

  uint32_t cslot = 0;  // stage of unit u
  int cm = m0;
  int64_t ctile = tile0, ck = k0;
  for (int64_t u = u0; u < u1;) {
    // one segment: K-steps ck .. of tile (cm, ctile), up to the tile's end or the range's
    const int64_t c_nkb = uniform_i64(s.nkb[cm]);
    const int64_t seg_kb0 = ck;
    const int64_t seg_end = u + (c_nkb - ck) < u1 ? u + (c_nkb - ck) : u1;
    const bool tile_end = u + (c_nkb - ck) <= u1;
#pragma unroll
    for (int mt = 0; mt < Sh::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (; u < seg_end; ++u, ++ck) {
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
      uint32_t a[Sh::MT][4], b[4][4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int mt = 0; mt < Sh::MT; ++mt) {
          const u32x2v_t v =
              lds_read_tr16(st + Sh::D_BYTES + 128 * ((2 * g + h) * Sh::NRB + rw * Sh::MT + mt) + 8 * li);
          a[mt][2 * h] = v.x;
          a[mt][2 * h + 1] = v.y;
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const u32x2v_t v = lds_read_tr16(st + 128 * ((2 * g + h) * Sh::NDB + 4 * wn + nt) + 8 * li);
          b[nt][2 * h] = v.x;
          b[nt][2 * h + 1] = v.y;
        }
      }
      const int64_t t0 = ck * 32;
      if (t0 + 32 > T) {
        // the last, partial step: the stage holds tokens wb .. wb+31 (wb <= t0);
        // K slot 8g + 2p (+1) of this lane is token wb + 8g + 2p (+1)
        const int64_t wb = window_base(t0, T);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int64_t tk = wb + 8 * g + 2 * p;
          const uint32_t keep =
              (tk >= t0 && tk < T ? 0x0000FFFFu : 0u) | (tk + 1 >= t0 && tk + 1 < T ? 0xFFFF0000u : 0u);
#pragma unroll
          for (int mt = 0; mt < Sh::MT; ++mt) a[mt][p] &= keep;
        }
      }
#pragma unroll
      for (int mt = 0; mt < Sh::MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_16x16x32(a[mt], b[nt], acc[mt][nt]);
    }
    const bool first_seg = seg_kb0 == k0 && ctile == tile0 && cm == m0;
    if (first_seg && u < u1) {
#pragma unroll
      for (int mt = 0; mt < Sh::MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) keep[mt][nt] = acc[mt][nt];
      kept = true;
      kept_full = seg_kb0 == 0 && tile_end;
      kept_tile = ctile;
    } else {
      finish(acc, cm, ctile, seg_kb0 == 0 && tile_end, partial_slot(w, first_seg));
    }
    if (tile_end) {
      ck = 0;
      if (++ctile == uniform_i64(s.tbase[cm + 1] - s.tbase[cm])) {
        ctile = 0;
        ++cm;
      }
    }
  }
  if (kept) finish(keep, m0, kept_tile, kept_full, partial_slot(w, true));
}

// ---------------------------------------------------------------------------
// Finishing pass over the tiles that were cut between workgroups: workgroup
// (c, t) takes values 1024c .. 1024c+1023 of batch-wide tile t, finds the
// ranges that cover the tile and sums their partials in range order, then
// rounds into XP (project) or adds into C (accumulate). Tiles inside one
// range return at once.
// ---------------------------------------------------------------------------
struct FinishBatch {
  Schedule s;
  const float* part;
  float* C[kMaxItems];            // accumulate targets
  uint16_t* XP[kMaxItems];        // project targets
};

template <int R, bool TO_BF16>
__global__ __launch_bounds__(256) void finish_tiles_kernel(FinishBatch fb) {
  const Schedule& s = fb.s;
  const int64_t t = blockIdx.y;
  const int m = item_of_tile(s, t);
  const int64_t tile = t - s.tbase[m];
  const int64_t ts = s.ubase[m] + tile * s.nkb[m], te = ts + s.nkb[m];
  const int64_t wa = range_of(s, ts), wb = range_of(s, te - 1);
  if (wa == wb) return;
  const int64_t tn = s.tile_n;
  const int64_t left = s.next[m] - tile * tn;
  const int64_t rows = left < tn ? left : tn;
  constexpr int PER = 4;  // floats per thread
  {
    const int64_t e = (int64_t)blockIdx.x * (256 * PER) + threadIdx.x * PER;
    if (e >= rows * R) return;
    f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
    for (int64_t w = wa; w <= wb; ++w) {
      // wa's share is its last segment when its range began in an earlier
      // tile, else its first; every later range begins inside this tile
      const bool first = !(w == wa && range_begin(s, wa) < ts);
      const float4 v = *reinterpret_cast<const float4*>(fb.part + partial_slot(w, first) * tn * R + e);
      const f32x4_t x = {v.x, v.y, v.z, v.w};
      sum = (w == wa) ? x : sum + x;
    }
    const int64_t out = tile * tn * R + e;
    if constexpr (TO_BF16) {
      const uint2 o = make_uint2(pack_bf16x2(f32_to_bf16_rne(sum[0]), f32_to_bf16_rne(sum[1])),
                                 pack_bf16x2(f32_to_bf16_rne(sum[2]), f32_to_bf16_rne(sum[3])));
      *reinterpret_cast<uint2*>(fb.XP[m] + out) = o;
    } else {
      float4 old = *reinterpret_cast<float4*>(fb.C[m] + out);
      old.x += sum[0];
      old.y += sum[1];
      old.z += sum[2];
      old.w += sum[3];
      *reinterpret_cast<float4*>(fb.C[m] + out) = old;
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

// Workgroups per launch: one per compute unit. (Two fit, but measured on
// the Qwen3-1.7B-shaped block one is faster: the second adds L2/request
// pressure rather than hiding latency.)
int64_t sketch_workgroups() {
  const int forced = env_int("RGC_SKETCH_WGS", 0);
  return forced > 0 ? forced : (int64_t)device_compute_units();
}

// The schedule for items with N extents ns[] and K extents ks[].
Schedule make_schedule(int n, const int64_t* ns, const int64_t* ks, int64_t tile_n, int64_t kblock) {
  Schedule s = {};
  s.n = n;
  s.tile_n = tile_n;
  for (int m = 0; m < n; ++m) {
    const int64_t tiles = (ns[m] + tile_n - 1) / tile_n;
    s.nkb[m] = (ks[m] + kblock - 1) / kblock;
    s.kext[m] = ks[m];
    s.next[m] = ns[m];
    s.ubase[m + 1] = s.ubase[m] + tiles * s.nkb[m];
    s.tbase[m + 1] = s.tbase[m] + tiles;
  }
  s.U = s.ubase[n];
  const int64_t G = sketch_workgroups();
  s.G = (int)(s.U < G ? s.U : G);
  return s;
}

template <int R>
size_t partial_bytes(const Schedule& s) {
  return (size_t)2 * s.G * s.tile_n * R * sizeof(float);
}

// One finishing workgroup per 1024 values of a tile (x) and per tile (y).
template <int R>
dim3 finish_grid(const Schedule& s) {
  return dim3((unsigned)((s.tile_n * R + 1023) / 1024), (unsigned)s.tbase[s.n]);
}

template <int R>
Schedule project_schedule(int n, const int64_t* ns, const int64_t* ks) {
  return make_schedule(n, ns, ks, kTileN, 32 * RankTraits<R>::KS);
}

template <int R>
Schedule accumulate_schedule(int n, const int64_t* ns, const int64_t* ks) {
  return make_schedule(n, ns, ks, AccShape<R>::TILE, 32);
}

template <int R>
rgc_status_t project_launch(int n, const uint16_t* const* Xs, const int64_t* ldxs, const int64_t* ks,
                            const uint16_t* const* Ps, uint16_t* const* XPs, int64_t T, void* ws, hipStream_t st) {
  int64_t ns[kMaxItems];
  for (int m = 0; m < n; ++m) ns[m] = T;
  ProjectBatch pb = {};
  pb.s = project_schedule<R>(n, ns, ks);
  FinishBatch fb = {};
  fb.s = pb.s;
  for (int m = 0; m < n; ++m) {
    pb.X[m] = Xs[m];
    pb.ldx[m] = ldxs[m];
    pb.P[m] = Ps[m];
    pb.XP[m] = XPs[m];
    fb.XP[m] = XPs[m];
  }
  pb.part = static_cast<float*>(ws);
  fb.part = pb.part;
  hipLaunchKernelGGL(project_kernel<R>, dim3((unsigned)pb.s.G), dim3(64 * RankTraits<R>::NR * RankTraits<R>::KS), 0,
                     st, pb);
  hipLaunchKernelGGL((finish_tiles_kernel<R, true>), finish_grid<R>(pb.s), dim3(256), 0, st, fb);
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

template <int R>
rgc_status_t accumulate_launch(int n, const uint16_t* const* Ds, const int64_t* ldds, const int64_t* ds,
                               const uint16_t* const* XPs, float* const* Cs, int64_t T, void* ws, hipStream_t st) {
  int64_t ks[kMaxItems];
  for (int m = 0; m < n; ++m) ks[m] = T;
  AccumulateBatch ab = {};
  ab.s = accumulate_schedule<R>(n, ds, ks);
  FinishBatch fb = {};
  fb.s = ab.s;
  for (int m = 0; m < n; ++m) {
    ab.D[m] = Ds[m];
    ab.ldd[m] = ldds[m];
    ab.XP[m] = XPs[m];
    ab.C[m] = Cs[m];
    fb.C[m] = Cs[m];
  }
  ab.part = static_cast<float*>(ws);
  fb.part = ab.part;
  hipLaunchKernelGGL(accumulate_kernel<R>, dim3((unsigned)ab.s.G), dim3(256), 0, st, ab);
  hipLaunchKernelGGL((finish_tiles_kernel<R, false>), finish_grid<R>(ab.s), dim3(256), 0, st, fb);
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

template <int R>
size_t accumulate_workspace(int n, const int64_t* ds, int64_t T) {
  int64_t ks[kMaxItems];
  for (int m = 0; m < n; ++m) ks[m] = T;
  return partial_bytes<R>(accumulate_schedule<R>(n, ds, ks));
}

rgc_status_t check_project_item(const uint16_t* X, int64_t ldx, int64_t k, const uint16_t* P, const uint16_t* XP,
                                int64_t T, int64_t r) {
  if (k <= 0 || r > k || ldx < k) return RGC_ERR_SHAPE;
  if ((k % 8) != 0 || ldx > kMaxLeadingDim) return RGC_ERR_UNSUPPORTED;
  if (T == 0) return RGC_OK;
  if (!X || !P || !XP) return RGC_ERR_NULL;
  if (!aligned16(X) || !aligned16(P) || !aligned16(XP) || (ldx % 8) != 0) return RGC_ERR_ALIGN;
  return RGC_OK;
}

rgc_status_t check_accumulate_item(const uint16_t* D, int64_t ldd, int64_t d, const uint16_t* XP, const float* C,
                                   int64_t T) {
  if (d <= 0 || ldd < d) return RGC_ERR_SHAPE;
  if ((d % 8) != 0 || d > kMaxTiledDim || ldd > kMaxLeadingDim) return RGC_ERR_UNSUPPORTED;
  if (T == 0) return RGC_OK;
  if (!D || !XP || !C) return RGC_ERR_NULL;
  if (!aligned16(D) || !aligned16(XP) || !aligned16(C) || (ldd % 8) != 0) return RGC_ERR_ALIGN;
  return RGC_OK;
}

}  // namespace
}  // namespace rgc

using namespace rgc;

extern "C" size_t rgc_project_batch_workspace_size(int64_t n, const int64_t* ks, int64_t T, int64_t r) {
  if (n <= 0 || n > kMaxItems || !ks || T <= 0) return 0;
  for (int64_t m = 0; m < n; ++m)
    if (ks[m] <= 0) return 0;
  int64_t ns[kMaxItems];
  for (int64_t m = 0; m < n; ++m) ns[m] = T;
  size_t out = 0;
  if (!dispatch_rank(r, [&](auto rc) {
        constexpr int R = decltype(rc)::value;
        out = partial_bytes<R>(project_schedule<R>((int)n, ns, ks));
      }))
    return 0;
  return out;
}

extern "C" size_t rgc_accumulate_batch_workspace_size(int64_t n, const int64_t* ds, int64_t T, int64_t r) {
  if (n <= 0 || n > kMaxItems || !ds || T <= 0) return 0;
  for (int64_t m = 0; m < n; ++m)
    if (ds[m] <= 0) return 0;
  size_t out = 0;
  if (!dispatch_rank(r, [&](auto rc) {
        constexpr int R = decltype(rc)::value;
        out = accumulate_workspace<R>((int)n, ds, T);
      }))
    return 0;
  return out;
}

extern "C" rgc_status_t rgc_project_batch(int64_t n, const uint16_t* const* Xs, const int64_t* ldxs,
                                          const int64_t* ks, const uint16_t* const* Ps, uint16_t* const* XPs,
                                          int64_t T, int64_t r, void* ws, size_t ws_bytes, void* stream) {
  if (n < 0 || T < 0 || r <= 0) return RGC_ERR_SHAPE;
  if (n > kMaxItems || !rank_supported(r) || T > kMaxTiledDim) return RGC_ERR_UNSUPPORTED;
  if (n == 0 || T == 0) return RGC_OK;
  if (!Xs || !ldxs || !ks || !Ps || !XPs) return RGC_ERR_NULL;
  for (int64_t m = 0; m < n; ++m) {
    const rgc_status_t st = check_project_item(Xs[m], ldxs[m], ks[m], Ps[m], XPs[m], T, r);
    if (st != RGC_OK) return st;
  }
  const size_t need = rgc_project_batch_workspace_size(n, ks, T, r);
  if (need > 0 && (!ws || ws_bytes < need)) return RGC_ERR_WORKSPACE;
  if (need > 0 && !aligned_to(ws, 256)) return RGC_ERR_ALIGN;
  rgc_status_t st = RGC_OK;
  dispatch_rank(r, [&](auto rc) {
    st = project_launch<decltype(rc)::value>((int)n, Xs, ldxs, ks, Ps, XPs, T, ws, static_cast<hipStream_t>(stream));
  });
  return st;
}

extern "C" rgc_status_t rgc_accumulate_batch(int64_t n, const uint16_t* const* Ds, const int64_t* ldds,
                                             const int64_t* ds, const uint16_t* const* XPs, float* const* Cs,
                                             int64_t T, int64_t r, void* ws, size_t ws_bytes, void* stream) {
  if (n < 0 || T < 0 || r <= 0) return RGC_ERR_SHAPE;
  if (n > kMaxItems || !rank_supported(r)) return RGC_ERR_UNSUPPORTED;
  if (n == 0 || T == 0) return RGC_OK;
  if (!Ds || !ldds || !ds || !XPs || !Cs) return RGC_ERR_NULL;
  for (int64_t m = 0; m < n; ++m) {
    const rgc_status_t st = check_accumulate_item(Ds[m], ldds[m], ds[m], XPs[m], Cs[m], T);
    if (st != RGC_OK) return st;
  }
  const size_t need = rgc_accumulate_batch_workspace_size(n, ds, T, r);
  if (need > 0 && (!ws || ws_bytes < need)) return RGC_ERR_WORKSPACE;
  if (need > 0 && !aligned_to(ws, 256)) return RGC_ERR_ALIGN;
  rgc_status_t st = RGC_OK;
  dispatch_rank(r, [&](auto rc) {
    st = accumulate_launch<decltype(rc)::value>((int)n, Ds, ldds, ds, XPs, Cs, T, ws, static_cast<hipStream_t>(stream));
  });
  return st;
}

extern "C" size_t rgc_project_workspace_size(int64_t T, int64_t k, int64_t r) {
  return rgc_project_batch_workspace_size(1, &k, T, r);
}

extern "C" size_t rgc_accumulate_workspace_size(int64_t T, int64_t d, int64_t r) {
  return rgc_accumulate_batch_workspace_size(1, &d, T, r);
}

extern "C" rgc_status_t rgc_project(const uint16_t* X, int64_t ldx, const uint16_t* P, uint16_t* XP, int64_t T,
                                    int64_t k, int64_t r, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k <= 0 || r <= 0) return RGC_ERR_SHAPE;
  return rgc_project_batch(1, &X, &ldx, &k, &P, &XP, T, r, ws, ws_bytes, stream);
}

extern "C" rgc_status_t rgc_accumulate(const uint16_t* D, int64_t ldd, const uint16_t* XP, float* C, int64_t T,
                                       int64_t d, int64_t r, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || d <= 0 || r <= 0) return RGC_ERR_SHAPE;
  return rgc_accumulate_batch(1, &D, &ldd, &d, &XP, &C, T, r, ws, ws_bytes, stream);
}
