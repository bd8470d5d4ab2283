// The two skinny contractions of the sketch, on bf16 MFMA with fp32 sums:
//   project:    XP = bf16(X P)         X: T x k, P: k x r      [RGC, "How it works"]
//   accumulate: C += D^T XP            D: T x d, XP: T x r     [RGC, "How it works";
//                                      LoGRA-S, Key Contributions 1]
// ([RGC] = page "Randomized Gradient Compression"; [LoGRA-S] = page "LoGRA:
// Scaling LLM Reinforcement Learning with Low-Rank Gradient Sketches".)
//
// Both are out = A^T B over a long K: A is the small "rank" operand (K x R,
// row-major with row stride R: P for project, XP for accumulate) and B the
// "stream" operand that carries nearly all the bytes (X, K = k, N = tokens;
// D, K = tokens, N = d), read from HBM exactly once. At r <= 128 they are
// HBM-bound, so the design is about keeping enough bytes in flight and
// fetching the rank operand as rarely as possible:
//
// * A workgroup tile is TILE = 64*WN columns of N by all R columns of r; its
//   waves (four or eight, by rank: StageShape below) split it WN ways along
//   N and WR ways along r, so every wave multiplies a 64 (N) x RW (r) block
//   with 16x16x32 MFMAs, r on the M side.
// * A K-step is 32 rows of K (64 for the project). The step's stream slab
//   (32 x TILE) and rank slab (32 x R) are copied from memory straight into
//   an LDS stage by all the waves, in 1 KB copies that do not pass through
//   VGPRs, S - 1 steps ahead of the step being multiplied. The rank slab is
//   fetched once per workgroup and shared by its waves.
// * Each wave reads its A operand from the stage with transposing LDS reads
//   (the rank operand is K-major), and its B operand with plain reads
//   (project: X is already k-contiguous per token) or transposing reads
//   (accumulate: D is token-major).
// * Work is balanced across the chip at K-step granularity ("stream-K"):
//   the (item, tile, K-step) units of the whole batch are cut into one
//   contiguous range per workgroup, about one workgroup per compute unit
//   (the host-side schedule below says how many). A tile
//   that lies inside one range is finished in place; a tile cut between
//   ranges gets fp32 partials (at most two per workgroup) that a second
//   launch sums in workgroup order. Every reduction has a fixed order, so
//   results are bit-reproducible, and there is no signalling between
//   workgroups inside a launch. Consecutive ranges are placed on the same
//   XCD, so the workgroups of one item share that XCD's L2.
#include "rgc_internal.hpp"

namespace rgc {

// ---------------------------------------------------------------------------
// K windows
// ---------------------------------------------------------------------------

// A K-step covers KS rows of the K dimension (32 or 64). Its operands are
// read through a window of KS rows [wb, wb + KS): in the steady state wb is
// the step's own first row k0; for the last, partial step the window is
// moved back to end at the K extent, so that every row it touches is valid
// memory, and rows outside [k0, end) are zeroed before use. A K extent
// below KS clamps the rows once, up front.
__device__ __forceinline__ int64_t window_base(int64_t k0, int64_t end, int64_t ks) {
  return k0 + ks <= end ? k0 : (end >= ks ? end - ks : 0);
}

// Rows of a window that are valid memory for a K extent `end`.
__device__ __forceinline__ int64_t window_rows(int64_t end, int64_t ks) { return end >= ks ? ks : end; }

// K-slot keep mask of a partial step: the stage holds K rows wb .. wb+KS-1;
// in K-half kh, dword p of a lane's operand holds rows 32kh + 8g + 2p and
// 32kh + 8g + 2p + 1 (low and high half). Returns the halves whose rows lie
// in [k0, end).
__device__ __forceinline__ uint32_t kslot_keep(int64_t wb, int kh, int64_t k0, int64_t end, int g, int p) {
  const int64_t k = wb + 32 * kh + 8 * g + 2 * p;
  return (k >= k0 && k < end ? 0x0000FFFFu : 0u) | (k + 1 >= k0 && k + 1 < end ? 0xFFFF0000u : 0u);
}

// ---------------------------------------------------------------------------
// Work items and the stream-K schedule. One launch covers a list of
// independent matrices of one rank (e.g. all projections of a transformer
// block). Units are (item, N-tile, K-step) in that order; workgroup w takes
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
  int64_t nkb[kMaxItems];         // K-steps per tile
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

// Layout of a partial slot (TILE x R fp32 of one segment) in store order: the
// float4 that lane l of wave w holds for N-tile nt and M-tile mt sits at
// float4 position ((w 4 + nt) MT + mt) 64 + l, so that each store instruction
// writes 1 KB contiguously (a row-major tile took 16 rows x 64 bytes each).
// It holds tile row 64 wn + 16 nt + l % 16 and columns rw RW + 16 mt +
// 4 (l / 16) .. +3, with wn = w % WN and rw = w / WN.
template <int MT>
__host__ __device__ __forceinline__ int64_t slot_pos4(int w, int nt, int mt, int l) {
  return ((int64_t)(w * 4 + nt) * MT + mt) * 64 + l;
}

// ---------------------------------------------------------------------------
// Stage geometry and the pipeline shared by both contractions.
//
// A step of KS = 32 KH rows is multiplied as KH K-halves of 32 (one MFMA K
// extent each).
//
// Rank-operand layout in a stage (after the stream slab): blocks of 4 K rows
// x 16 r columns (128 bytes, four rows of four 8-byte chunks); block (kq, b)
// sits at STREAM + 128 * (kq * NRB + b). Rank copy c fills blocks 8c ..
// 8c+7: lane l reads K row (l % 8) / 2 of block 8c + l / 8, columns
// 8 * (l % 2) .. +7, which are exactly the 16 bytes that land at 16 * l. A
// transposing read of block (kq, b) gives lane i column i of rows 4kq ..
// 4kq+3: four K slots of the A operand.
// ---------------------------------------------------------------------------
constexpr int kStages = 6;

// Compute width of the rank operand for a rank of RM columns (a multiple of
// 16): RM itself, except above 128 with an odd number of 16-column blocks
// (144, 176, 208, 240), which take one more block so that two waves can split
// them. The extra block is filled with a copy of a real block and never
// multiplied or stored.
__host__ __device__ constexpr int sketch_width(int RM) { return RM > 128 && (RM / 16) % 2 == 1 ? RM + 16 : RM; }

// Waves along r: up to 128 ranks one (the N tile is 256 wide, each wave holds
// all ranks, up to 8 M-tiles); above 128 two, each with half the ranks (with
// four waves, a split that gave every wave at most 64 ranks re-read the rank
// operand twice as often: measured on the 1.7B block at r = 256 and the 8B
// layer at r = 128). Above 128 the accumulate keeps the 256-wide N tile with
// eight waves (two per SIMD), so that its XP slab (32 tokens x r) is shared
// by 256 columns of D, not 128: the 1.7B block's accumulate at r = 256 71.0
// -> 63.2 us per call. The project's X and P slabs (64 k per step) leave
// room for a 128-wide tile only: four waves, or at r = 192 and 256, where r
// splits into four whole 16-column blocks, eight (four along r, two per
// SIMD), whose second wave per SIMD outweighs the X operand read by four
// waves instead of two (the 1.7B block at r = 256: 78.3 -> 65.1 us per
// call). At r = 64, 96 and 128 both kernels
// run eight waves too, two along r: two waves per SIMD hide more of each
// step's latency, and the first segment's sums fit in registers (the 8B
// layer at r = 128: accumulate 81.5 -> 74 us, project 78 -> 76 us; the 1.7B
// block at r = 64: 33.6 -> 32.9 and 39.6 -> 38.6 us). Ranks with an odd
// number of 16-column blocks up to 128 (48, 80, 112) keep four waves.
//
// WNF > 0 forces WNF waves along N (the narrow accumulate tile below).
template <int R, int KH, int WNF = 0>
struct StageShape {
  static constexpr int WR = KH == 2 && R > 128 && (R / 16) % 4 == 0 ? 4 : R > 128 || (R > 32 && (R / 16) % 2 == 0) ? 2 : 1;
  static constexpr int WN = WNF > 0 ? WNF : R <= 128 || KH == 1 ? 4 : 2;  // waves along N
  static constexpr int WAVES = WR * WN;
  static constexpr int RW = R / WR;                              // r per wave
  static constexpr int MT = RW / 16;                             // MFMA M-tiles per wave
  static constexpr int TILE = 64 * WN;                           // N per workgroup tile
  static constexpr int KS = 32 * KH;                             // K rows per step
  static constexpr int NSC = TILE * KH / 16;                     // stream copies per stage (1 KB each)
  static constexpr int NRB = R / 16;                             // 16-column rank blocks
  static constexpr int NRC = KH * NRB;                           // rank copies per stage
  static constexpr int NI = NSC + NRC;
  static constexpr int STREAM = 1024 * NSC;                      // stream slab bytes
  static constexpr int STAGE = 1024 * NI;
  static constexpr int S = kStages * STAGE <= 160 * 1024 ? kStages : 160 * 1024 / STAGE;
  static constexpr int NV_LO = NI / WAVES, NV_HI = (NI + WAVES - 1) / WAVES;  // copies per wave
  static_assert(RW % 16 == 0 && RW <= 128, "rank split");
  static_assert(S >= 3 && S * STAGE <= 160 * 1024, "LDS");
  static_assert((S - 1) * NV_HI <= 63, "vector memory counter");
};

template <int R>
using AccTile = f32x4_t[StageShape<R, 1>::MT][4];

// Runs a workgroup's range of units. The policy supplies what differs
// between the two contractions:
//   enter_item(m)                          per-item constants of the copy side
//                                          (the copy cursor runs S - 1 units
//                                          ahead, possibly in a later item, so
//                                          the compute side never uses them)
//   stream_offset(m, tile, c, lane, rows)  per-lane byte offset of stream copy c
//   stream_base(m, tile, wb)               wave-uniform base of the window at K row wb
//   rank_base(m, mi)                       rank operand of member mi of the item
//   read_b(stage, kh, wn, g, li, b)        the B operands of the wave's four N-tiles, K-half kh
//   mask_b(b, wb, kh, k0, end, g)          zero B's K slots outside [k0, end)
//   store(res, m, tile, full, slot, wn, rw, g, li)
//
// An item may be a group of GM members that share the stream operand (the
// project of several matrices that read the same X): the rank operand is then
// the members' RM-column operands side by side, GM * RM columns in all, and
// every stream slab in LDS is multiplied by all of them. In a stage the rank
// blocks are laid out member by member (member mi's blocks (kq, b) at block
// mi * 8 KH * NRB_ITEM + kq * NRB_ITEM + b), so that every 1 KB copy comes
// from a single member's operand.
template <int RM, int KH, typename Policy, int GM = 1>
__device__ __forceinline__ void staged_pipeline(const Schedule& s, Policy& pol, char* smem) {
  constexpr int R = sketch_width(GM * RM);  // compute width; each member has RM columns (row stride RM)
  constexpr int NRB_ITEM = RM / 16;         // rank blocks of one member
  constexpr int NRB_MEM = GM * NRB_ITEM;    // rank blocks that exist in memory
  constexpr int CPM = KH * NRB_ITEM;        // rank copies per member and stage
  using Sh = typename Policy::Sh;
  static_assert(Sh::KS == 32 * KH, "policy shape");
  constexpr int S = Sh::S, MT = Sh::MT, KS = Sh::KS;
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int wn = wave % Sh::WN, rw = wave / Sh::WN;
  const int g = lane >> 4, li = lane & 15;
  const int64_t w = logical_workgroup(blockIdx.x, s.G);
  const int64_t u0 = uniform_i64(range_begin(s, w)), u1 = uniform_i64(range_begin(s, w + 1));
  const uint32_t lds0 = (uint32_t)(uintptr_t)(RGC_LDS char*)smem;
  constexpr int NW = Sh::WAVES;
  const bool more = wave < Sh::NI % NW;  // this wave issues NV_HI copies per stage (else NV_LO)

  // ---- the copy side: a cursor over this workgroup's units, S - 1 ahead
  const int m0 = item_of_unit(s, u0);
  const int64_t tile0 = (u0 - s.ubase[m0]) / s.nkb[m0], k0 = (u0 - s.ubase[m0]) % s.nkb[m0];
  int lm = m0;
  int64_t ltile = tile0, lk = k0, lu = u0;
  int64_t l_kext = 0, l_nkb = 0, l_tiles = 0;
  const uint16_t* l_rank[GM];  // the members' rank operands
  uint32_t voff[Sh::NV_HI];
  // the member and the copy within the member of rank copy cr (copies past the
  // members, the padding, repeat the last one)
  auto rank_copy = [&](int cr, int& mi, int& cl) {
    cr = cr < NRB_MEM * KH ? cr : NRB_MEM * KH - 1;
    mi = GM == 1 ? 0 : cr / CPM;
    cl = cr - mi * CPM;
  };
  auto enter_item = [&](int m) {
    l_kext = uniform_i64(s.kext[m]);
    l_nkb = uniform_i64(s.nkb[m]);
    l_tiles = uniform_i64(s.tbase[m + 1] - s.tbase[m]);
#pragma unroll
    for (int mi = 0; mi < GM; ++mi) l_rank[mi] = uniform_ptr(pol.rank_base(m, mi));
    pol.enter_item(m);
  };
  auto set_offsets = [&](int m, int64_t tile) {
    const int64_t rows = window_rows(l_kext, KS);
#pragma unroll
    for (int v = 0; v < Sh::NV_HI; ++v) {
      const int c = wave + NW * v;
      if (c < Sh::NSC) {
        voff[v] = pol.stream_offset(m, tile, c, lane, rows);
      } else {
        int mi = 0, cl = 0;
        rank_copy(c - Sh::NSC, mi, cl);
        const int blk = 8 * cl + (lane >> 3);  // block of member mi
        int64_t kr = 4 * (blk / NRB_ITEM) + ((lane & 7) >> 1);
        kr = kr < rows ? kr : rows - 1;
        voff[v] = (uint32_t)((kr * RM + 16 * (blk % NRB_ITEM) + 8 * (lane & 1)) * 2);
      }
    }
  };
  if (u0 < u1) {
    enter_item(lm);
    set_offsets(lm, ltile);
  }
  uint32_t lslot = 0;  // stage of unit lu
  auto issue = [&]() {
    const int64_t wb = window_base(lk * KS, l_kext, KS);
    const uint16_t* Sb = uniform_ptr(pol.stream_base(lm, ltile, wb));
    const uint32_t st = lds0 + lslot * Sh::STAGE;
    static_for<0, Sh::NV_HI>([&](auto vc) {
      constexpr int v = decltype(vc)::value;
      const int c = wave + NW * v;  // a stream copy if c < NSC, a rank copy if NSC <= c < NI
      const uint16_t* Rb = nullptr;
      if constexpr (NW * v + NW - 1 >= Sh::NSC) {
        if constexpr (GM == 1) {
          Rb = uniform_ptr(l_rank[0] + wb * RM);
        } else {
          int mi = 0, cl = 0;  // the member this slot copies from (wave-uniform)
          rank_copy(c - Sh::NSC, mi, cl);
          const uint16_t* base = l_rank[0];
#pragma unroll
          for (int q = 1; q < GM; ++q) base = mi == q ? l_rank[q] : base;
          Rb = uniform_ptr(base + wb * RM);
        }
      }
      if constexpr (NW * v + NW - 1 < Sh::NSC) {
        dma_16b_stream(Sb, voff[v], st + 1024 * c);
      } else if constexpr (NW * v >= Sh::NSC && NW * v + NW - 1 < Sh::NI) {
        dma_16b_cached(Rb, voff[v], st + 1024 * c);
      } else {
        if (c < Sh::NSC)
          dma_16b_stream(Sb, voff[v], st + 1024 * c);
        else if (c < Sh::NI)
          dma_16b_cached(Rb, voff[v], st + 1024 * c);
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
  f32x4_t acc[MT][4];
  // The first segment's sums are kept in registers and stored after the
  // range's last segment: a store issued while copies are in flight counts
  // in the same counter as the copies, so the next wait would drain the
  // whole pipeline. Later segments (each a whole tile or the range's last
  // piece) are stored as they finish. With 8 M-tiles per wave (r = 256 on
  // two waves along r) the accumulate has no room for a second set of sums
  // (it spilled), so there its first segment is stored as it finishes too.
  constexpr bool KEEP_FIRST = MT <= 4 || Policy::kKeepLargeFirst;
  f32x4_t keep[KEEP_FIRST ? MT : 1][4];
  bool kept = false, kept_full = false;
  int64_t kept_tile = tile0;

#pragma unroll
  for (int v = 0; v + 1 < S; ++v)
    if (lu < u1) issue();

  uint32_t cslot = 0;  // stage of unit u
  int cm = m0;
  int64_t ctile = tile0, ck = k0;
  for (int64_t u = u0; u < u1;) {
    // one segment: K-steps ck .. of tile (cm, ctile), up to the tile's end or the range's
    const int64_t c_nkb = uniform_i64(s.nkb[cm]), c_kext = uniform_i64(s.kext[cm]);
    const int64_t seg_kb0 = ck;
    const int64_t seg_end = u + (c_nkb - ck) < u1 ? u + (c_nkb - ck) : u1;
    const bool tile_end = u + (c_nkb - ck) <= u1;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
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
      const int64_t t0 = ck * KS;
      const bool partial = t0 + KS > c_kext;  // the tile's last, partial step
      const int64_t wb = window_base(t0, c_kext, KS);
#pragma unroll
      for (int kh = 0; kh < KH; ++kh) {
        uint32_t a[MT][4], b[4][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const int B = rw * MT + mt;  // rank block (wave-uniform)
            // A padding block is never multiplied; with one member its read
            // stays inside the stage (it reads some block of the stage), with
            // several it would not, so it is skipped.
            if (GM > 1 && R != RM * GM && B >= NRB_MEM) {
              a[mt][2 * h] = a[mt][2 * h + 1] = 0u;
              continue;
            }
            const int mi = GM == 1 ? 0 : B / NRB_ITEM;
            const u32x2v_t v = lds_read_tr16(
                st + Sh::STREAM + 128 * (mi * 8 * KH * NRB_ITEM + (8 * kh + 2 * g + h) * NRB_ITEM + B - mi * NRB_ITEM) +
                8 * li);
            a[mt][2 * h] = v.x;
            a[mt][2 * h + 1] = v.y;
          }
        pol.read_b(st, kh, wn, g, li, b);
        if (partial) {
          // zero both operands outside [t0, end)
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t keep_p = kslot_keep(wb, kh, t0, c_kext, g, p);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) a[mt][p] &= keep_p;
          }
          pol.mask_b(b, wb, kh, t0, c_kext, g);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (R != RM * GM && rw * MT + mt >= NRB_MEM) continue;  // padding block (wave-uniform)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_16x16x32(a[mt], b[nt], acc[mt][nt]);
        }
      }
    }
    const bool first_seg = seg_kb0 == k0 && ctile == tile0 && cm == m0;
    if (KEEP_FIRST && first_seg && u < u1) {
      if constexpr (KEEP_FIRST) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) keep[mt][nt] = acc[mt][nt];
      }
      kept = true;
      kept_full = seg_kb0 == 0 && tile_end;
      kept_tile = ctile;
    } else {
      pol.store(acc, cm, ctile, seg_kb0 == 0 && tile_end, partial_slot(w, first_seg), wn, rw, g, li);
    }
    if (tile_end) {
      ck = 0;
      if (++ctile == uniform_i64(s.tbase[cm + 1] - s.tbase[cm])) {
        ctile = 0;
        ++cm;
      }
    }
  }
  if constexpr (KEEP_FIRST) {
    if (kept) pol.store(keep, m0, kept_tile, kept_full, partial_slot(w, true), wn, rw, g, li);
  }
}

// ---------------------------------------------------------------------------
// project: XP = bf16(X P). N = tokens, K = k, steps of 64 k (two K-halves),
// so that every copy reads whole 128-byte rows of X.
//
// Stream copy c holds 8 tokens x 64 k (128 bytes per token) of the tile:
// lane l reads token 8c + l / 8, k chunk q (8 values) such that its 16
// bytes land at 16 * (8 * (l / 8) + (q + l / 16 + 4 (c % 2)) % 8). The B
// operand of lane (n, g) for N-tile nt in K-half kh is token 16nt + n,
// k = 32kh + 8g .. +7: one 16-byte read; the rotations spread the 16 lanes
// of a group over all LDS banks.
// ---------------------------------------------------------------------------
constexpr int kProjectKH = 2;
// Members of a project group: matrices that read the same X, projected in one
// pass over it; at most 256 ranks in all.
constexpr int kMaxGroup = 4;

struct ProjectBatch {
  Schedule s;                     // one schedule item per group
  const uint16_t* X[kMaxItems];
  int64_t ldx[kMaxItems];
  const uint16_t* P[kMaxItems][kMaxGroup];
  uint16_t* XP[kMaxItems][kMaxGroup];
  float* part;                    // 2 G slots of TILE x R fp32
};

template <int RM, int GM, int WNF = 0>
struct ProjectPolicy {
  static constexpr int R = sketch_width(GM * RM);
  static constexpr int NRB_ITEM = RM / 16;
  using Sh = StageShape<R, kProjectKH, WNF>;
  // a group's sums leave no room for a second set (measured: spills)
  static constexpr bool kKeepLargeFirst = GM == 1;
  const ProjectBatch& pb;
  int64_t ldx = 0, T = 0;  // of the copy cursor's item
  __device__ void enter_item(int m) {
    ldx = uniform_i64(pb.ldx[m]);
    T = uniform_i64(pb.s.next[m]);
  }
  __device__ const uint16_t* rank_base(int m, int mi) const { return pb.P[m][mi]; }
  __device__ const uint16_t* stream_base(int m, int64_t tile, int64_t wb) const {
    return pb.X[m] + tile * Sh::TILE * ldx + wb;
  }
  __device__ uint32_t stream_offset(int m, int64_t tile, int c, int lane, int64_t rows) const {
    const int tl = lane >> 3;
    const int q = ((lane & 7) - (tl >> 1) - 4 * (c & 1)) & 7;  // k chunk whose bytes land at 16 * lane
    int64_t t = 8 * c + tl;
    const int64_t tmax = T - 1 - tile * Sh::TILE;  // tokens past T read the last one (never stored)
    t = t < tmax ? t : tmax;
    int64_t kc = 8 * q;
    kc = kc + 8 <= rows ? kc : rows - 8;  // rows is a multiple of 8
    return (uint32_t)((t * ldx + kc) * 2);
  }
  __device__ void read_b(const RGC_LDS char* st, int kh, int wn, int g, int li, uint32_t (&b)[4][4]) const {
    const int t = li & 7, half = li >> 3;
    const int sigma = (4 * kh + g + (t >> 1) + 4 * half) & 7;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int c = 2 * (4 * wn + nt) + half;
      const u32x4v_t v = *(const RGC_LDS u32x4v_t*)(st + 1024 * c + 16 * (8 * t + sigma));
      b[nt][0] = v.x;
      b[nt][1] = v.y;
      b[nt][2] = v.z;
      b[nt][3] = v.w;
    }
  }
  __device__ void mask_b(uint32_t (&b)[4][4], int64_t wb, int kh, int64_t k0, int64_t end, int g) const {
    // a lane's 8 K slots are one k chunk: all inside [k0, end) or all outside
    const int64_t k = wb + 32 * kh + 8 * g;
    const uint32_t keep = k >= k0 && k < end ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int p = 0; p < 4; ++p) b[nt][p] &= keep;
  }
  __device__ void store(const f32x4_t (&res)[Sh::MT][4], int m, int64_t tile, bool full, int64_t slot, int wn, int rw, int g,
                        int li) const {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t row = 64 * wn + 16 * nt + li;  // tile-relative token
#pragma unroll
      for (int mt = 0; mt < Sh::MT; ++mt) {
        const int B = rw * Sh::MT + mt;  // rank block
        if (R != RM * GM && B >= GM * NRB_ITEM) continue;  // padding block
        const int rcol = rw * Sh::RW + 16 * mt + 4 * g;
        const f32x4_t v = res[mt][nt];
        if (full) {
          const int64_t t = tile * Sh::TILE + row;
          const int mi = GM == 1 ? 0 : B / NRB_ITEM;
          if (t < pb.s.next[m])
            *reinterpret_cast<uint2*>(pb.XP[m][mi] + t * RM + rcol - mi * RM) =
                make_uint2(f32x2_to_bf16x2_rne(v[0], v[1]),
                           f32x2_to_bf16x2_rne(v[2], v[3]));
        } else {
          reinterpret_cast<float4*>(pb.part + slot * Sh::TILE * R)[slot_pos4<Sh::MT>(rw * Sh::WN + wn, nt, mt,
                                                                                     16 * g + li)] =
              make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
  }
};

template <int RM, int GM, int WNF = 0>
constexpr int prj_threads() { return 64 * StageShape<sketch_width(GM * RM), kProjectKH, WNF>::WAVES; }
template <int RM, int GM>
__global__ __launch_bounds__((prj_threads<RM, GM>()), 1) void project_kernel(ProjectBatch pb) {
  using Sh = StageShape<sketch_width(GM * RM), kProjectKH>;
  __shared__ __attribute__((aligned(1024))) char smem[Sh::S * Sh::STAGE];
  ProjectPolicy<RM, GM> pol{pb};
  staged_pipeline<RM, kProjectKH, ProjectPolicy<RM, GM>, GM>(pb.s, pol, smem);
}
// The narrow tiles (128 tokens, two waves along N) of small one-matrix launches.
template <int RM>
__global__ __launch_bounds__((prj_threads<RM, 1, 2>()), 1) void project_narrow_kernel(ProjectBatch pb) {
  using Sh = StageShape<sketch_width(RM), kProjectKH, 2>;
  __shared__ __attribute__((aligned(1024))) char smem[Sh::S * Sh::STAGE];
  ProjectPolicy<RM, 1, 2> pol{pb};
  staged_pipeline<RM, kProjectKH, ProjectPolicy<RM, 1, 2>, 1>(pb.s, pol, smem);
}

// ---------------------------------------------------------------------------
// accumulate: C += D^T XP. N = d, K = tokens.
//
// Stream layout: blocks of 4 tokens x 16 columns of d (128 bytes, four rows
// of four 8-byte chunks); block (tq, b) sits at 128 * (tq * NSC + b). Stream
// copy c fills blocks 8c .. 8c+7: lane l reads token (l % 8) / 2 of block
// 8c + l / 8, columns 8 * (l % 2) .. +7. A transposing read of block (tq, b)
// gives lane i column i of tokens 4tq .. 4tq+3: four K slots of B.
// ---------------------------------------------------------------------------
struct AccumulateBatch {
  Schedule s;
  const uint16_t* D[kMaxItems];
  int64_t ldd[kMaxItems];
  const uint16_t* XP[kMaxItems];
  float* C[kMaxItems];
  float* part;                    // 2 G slots of TILE x R fp32
  int add_part;                   // 1: add the split tiles' partials to the slots (a later call of a deferred accumulation)
};

template <int RM, int WNF = 0>
struct AccumulatePolicy {
  static constexpr int R = sketch_width(RM);
  using Sh = StageShape<R, 1, WNF>;
  static constexpr bool kKeepLargeFirst = false;
  const AccumulateBatch& ab;
  int64_t ldd = 0, d = 0;  // of the copy cursor's item
  __device__ void enter_item(int m) {
    ldd = uniform_i64(ab.ldd[m]);
    d = uniform_i64(ab.s.next[m]);
  }
  __device__ const uint16_t* rank_base(int m, int) const { return ab.XP[m]; }
  __device__ const uint16_t* stream_base(int m, int64_t tile, int64_t wb) const { return ab.D[m] + wb * ldd; }
  __device__ uint32_t stream_offset(int m, int64_t tile, int c, int lane, int64_t rows) const {
    const int blk = 8 * c + (lane >> 3);
    int64_t t = 4 * (blk / Sh::NSC) + ((lane & 7) >> 1);
    t = t < rows ? t : rows - 1;
    int64_t col = tile * Sh::TILE + 16 * (blk % Sh::NSC) + 8 * (lane & 1);
    col = col < d ? col : d - 8;  // past d: any valid chunk (its columns are never stored)
    return (uint32_t)((t * ldd + col) * 2);
  }
  __device__ void read_b(const RGC_LDS char* st, int kh, int wn, int g, int li, uint32_t (&b)[4][4]) const {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const u32x2v_t v = lds_read_tr16(st + 128 * ((8 * kh + 2 * g + h) * Sh::NSC + 4 * wn + nt) + 8 * li);
        b[nt][2 * h] = v.x;
        b[nt][2 * h + 1] = v.y;
      }
  }
  __device__ void mask_b(uint32_t (&b)[4][4], int64_t wb, int kh, int64_t k0, int64_t end, int g) const {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t keep = kslot_keep(wb, kh, k0, end, g, p);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) b[nt][p] &= keep;
    }
  }
  __device__ void store(const AccTile<R>& res, int m, int64_t tile, bool full, int64_t slot, int wn, int rw, int g,
                        int li) const {
    if (!full && ab.add_part) {
      // A deferred accumulation: this slot already holds the earlier calls'
      // sums of the same segment (the same schedule every call). A load waits
      // for every older memory operation of the wave, the copies in flight
      // included, so the slot is read one N-tile (MT loads) at a time and each
      // wait covers MT loads rather than one.
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        float4* p = reinterpret_cast<float4*>(ab.part + slot * Sh::TILE * R) +
                    slot_pos4<Sh::MT>(rw * Sh::WN + wn, nt, 0, 16 * g + li);
        float4 o[Sh::MT];
#pragma unroll
        for (int mt = 0; mt < Sh::MT; ++mt)
          if (!(R != RM && rw * Sh::RW + 16 * mt >= RM)) o[mt] = p[64 * mt];
#pragma unroll
        for (int mt = 0; mt < Sh::MT; ++mt) {
          if (R != RM && rw * Sh::RW + 16 * mt >= RM) continue;  // padding block
          const f32x4_t v = res[mt][nt];
          p[64 * mt] = make_float4(o[mt].x + v[0], o[mt].y + v[1], o[mt].z + v[2], o[mt].w + v[3]);
        }
      }
      return;
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t row = 64 * wn + 16 * nt + li;  // tile-relative d
#pragma unroll
      for (int mt = 0; mt < Sh::MT; ++mt) {
        if (R != RM && rw * Sh::RW + 16 * mt >= RM) continue;  // padding block
        const int rcol = rw * Sh::RW + 16 * mt + 4 * g;
        const f32x4_t v = res[mt][nt];
        if (full) {
          // the tile lies inside this workgroup's range: one add per element,
          // no other writer in this launch
          if (tile * Sh::TILE + row < ab.s.next[m]) {
            float* c = ab.C[m] + (tile * Sh::TILE + row) * RM + rcol;
#pragma unroll
            for (int e = 0; e < 4; ++e) unsafeAtomicAdd(c + e, v[e]);
          }
        } else {
          reinterpret_cast<float4*>(ab.part + slot * Sh::TILE * R)[slot_pos4<Sh::MT>(rw * Sh::WN + wn, nt, mt,
                                                                                     16 * g + li)] =
              make_float4(v[0], v[1], v[2], v[3]);
        }
      }
    }
  }
};

template <int RM, int WNF = 0>
constexpr int acc_threads() { return 64 * StageShape<sketch_width(RM), 1, WNF>::WAVES; }
template <int RM>
__global__ __launch_bounds__(acc_threads<RM>(), 1) void accumulate_kernel(AccumulateBatch ab) {
  using Sh = StageShape<sketch_width(RM), 1>;
  __shared__ __attribute__((aligned(1024))) char smem[Sh::S * Sh::STAGE];
  AccumulatePolicy<RM> pol{ab};
  staged_pipeline<RM, 1>(ab.s, pol, smem);
}
// The narrow tiles (128 columns of d, two waves along N) of small launches.
template <int RM>
__global__ __launch_bounds__((acc_threads<RM, 2>()), 1) void accumulate_narrow_kernel(AccumulateBatch ab) {
  using Sh = StageShape<sketch_width(RM), 1, 2>;
  __shared__ __attribute__((aligned(1024))) char smem[Sh::S * Sh::STAGE];
  AccumulatePolicy<RM, 2> pol{ab};
  staged_pipeline<RM, 1>(ab.s, pol, smem);
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
  float* C[kMaxItems];                    // accumulate targets
  uint16_t* XP[kMaxItems][kMaxGroup];     // project targets (per group member)
};

template <int RM, int GM, bool TO_BF16, int WNF>
__device__ __forceinline__ void finish_tiles(const FinishBatch& fb) {
  constexpr int R = sketch_width(GM * RM);  // partials are tile_n x R; outputs have row stride RM
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
  // the slots' layout (slot_pos4) is the producing kernel's: the project's
  // tile shape (K-steps of 64) or the accumulate's (32)
  using Sh = StageShape<R, TO_BF16 ? kProjectKH : 1, WNF>;
  constexpr int MAXP = 8;        // partial loads in flight at once
  {
    // one float4 of the slots per thread, at the same store-order position in each
    const int64_t q4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q4 >= tn * R / 4) return;
    const int lane = (int)(q4 % 64);
    const int64_t wq = q4 / 64;
    const int mt = (int)(wq % Sh::MT), nt = (int)(wq / Sh::MT % 4), wv = (int)(wq / Sh::MT / 4);
    const int64_t row = 64 * (wv % Sh::WN) + 16 * nt + (lane & 15);
    const int col = (wv / Sh::WN) * Sh::RW + 16 * mt + 4 * (lane >> 4);
    if (row >= rows) return;
    if (R != RM * GM && col >= RM * GM) return;  // padding columns (a float4 never straddles a member)
    const int mi = col / RM;
    const int64_t out = (tile * tn + row) * RM + col - mi * RM;
    float4 old = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (!TO_BF16) old = *reinterpret_cast<const float4*>(fb.C[m] + out);
    f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
    // The partials of up to MAXP ranges are loaded together, then summed in
    // range order (the order, and so the bits, of a one-at-a-time sum).
    for (int64_t w0 = wa; w0 <= wb; w0 += MAXP) {
      float4 v[MAXP];
#pragma unroll
      for (int i = 0; i < MAXP; ++i) {
        const int64_t w = w0 + i;
        // wa's share is its last segment when its range began in an earlier
        // tile, else its first; every later range begins inside this tile
        const bool first = !(w == wa && range_begin(s, wa) < ts);
        v[i] = w <= wb ? reinterpret_cast<const float4*>(fb.part + partial_slot(w, first) * tn * R)[q4]
                       : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int i = 0; i < MAXP; ++i) {
        const int64_t w = w0 + i;
        const f32x4_t x = {v[i].x, v[i].y, v[i].z, v[i].w};
        if (w <= wb) sum = (w == wa) ? x : sum + x;
      }
    }
    if constexpr (TO_BF16) {
      const uint2 o = make_uint2(f32x2_to_bf16x2_rne(sum[0], sum[1]),
                                 f32x2_to_bf16x2_rne(sum[2], sum[3]));
      *reinterpret_cast<uint2*>(fb.XP[m][mi] + out) = o;
    } else {
      old.x += sum[0];
      old.y += sum[1];
      old.z += sum[2];
      old.w += sum[3];
      *reinterpret_cast<float4*>(fb.C[m] + out) = old;
    }
  }
}

template <int RM, int GM, bool TO_BF16>
__global__ __launch_bounds__(256) void finish_tiles_kernel(FinishBatch fb) {
  finish_tiles<RM, GM, TO_BF16, 0>(fb);
}

// The same over the narrow tiles' partials (their slot layout).
template <int RM, bool TO_BF16>
__global__ __launch_bounds__(256) void finish_narrow_tiles_kernel(FinishBatch fb) {
  finish_tiles<RM, 1, TO_BF16, 2>(fb);
}

// ---------------------------------------------------------------------------
// Ranks below one MFMA tile (r = 4, 8): the rank operand rows are 8 or 16
// bytes, so these contractions stream X or D with plain 16-byte loads and
// sum on the VALU. Products of bf16 values are exact in fp32; the sums are
// fp32 in a fixed order, so results are bit-reproducible.
// ---------------------------------------------------------------------------
struct SmallProjectBatch {
  int n;
  int64_t T;
  const uint16_t* X[kMaxItems];
  int64_t ldx[kMaxItems];
  int64_t k[kMaxItems];
  const uint16_t* P[kMaxItems];
  uint16_t* XP[kMaxItems];
};

// One wave per token row: lane l sums the 8-value chunks l, l + 64, ... of
// the row against the matching P rows, then a butterfly adds the 64 lane
// sums; one rounding to bf16.
template <int R>
__global__ __launch_bounds__(256) void small_project_kernel(SmallProjectBatch b) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int m = (int)(row / b.T);
  if (m >= b.n) return;
  const int64_t t = row - (int64_t)m * b.T;
  const uint16_t* __restrict__ x = b.X[m] + t * b.ldx[m];
  const uint16_t* __restrict__ P = b.P[m];
  const int64_t chunks = b.k[m] / 8;
  float acc[R];
#pragma unroll
  for (int j = 0; j < R; ++j) acc[j] = 0.f;
  for (int64_t c = lane; c < chunks; c += 64) {
    const uint4 xv = *reinterpret_cast<const uint4*>(x + 8 * c);
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xe = __uint_as_float(e & 1 ? (xw[e / 2] & 0xFFFF0000u) : (xw[e / 2] << 16));
      float p[R];
      load_bf16_row<R>(P + (8 * c + e) * R, p);
#pragma unroll
      for (int j = 0; j < R; ++j) acc[j] += xe * p[j];
    }
  }
#pragma unroll
  for (int j = 0; j < R; ++j) acc[j] = wave_sum_f32(acc[j]);
  if (lane == 0) {
    uint32_t o[R / 2];
#pragma unroll
    for (int i = 0; i < R / 2; ++i) o[i] = f32x2_to_bf16x2_rne(acc[2 * i], acc[2 * i + 1]);
    uint16_t* dst = b.XP[m] + t * R;
    if constexpr (R == 4)
      *reinterpret_cast<uint2*>(dst) = make_uint2(o[0], o[1]);
    else
      *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Tokens per partial sum of the small-rank accumulate.
constexpr int kSmallTokenChunk = 128;

struct SmallAccumulateBatch {
  int n;
  int64_t T;
  int64_t chunks;                  // 8-column chunks of all items
  int64_t cbase[kMaxItems + 1];    // first chunk of each item
  const uint16_t* D[kMaxItems];
  int64_t ldd[kMaxItems];
  const uint16_t* XP[kMaxItems];
  float* C[kMaxItems];
  float* part;                     // per (token chunk, column chunk): 8 x R fp32
};

__device__ __forceinline__ int small_item(const int64_t* base, int n, int64_t c) {
  int m = 0;
  while (m + 1 < n && c >= base[m + 1]) ++m;
  return m;
}

// Thread (column chunk, token chunk): the 8 x R sums of D[t][8c .. 8c+7] *
// XP[t][0 .. R-1] over the chunk's tokens in order.
template <int R>
__global__ __launch_bounds__(256) void small_accumulate_kernel(SmallAccumulateBatch b) {
  const int64_t gc = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gc >= b.chunks) return;
  const int m = small_item(b.cbase, b.n, gc);
  const int64_t cc = gc - b.cbase[m];
  const int64_t t0 = (int64_t)blockIdx.y * kSmallTokenChunk;
  const int64_t t1 = t0 + kSmallTokenChunk < b.T ? t0 + kSmallTokenChunk : b.T;
  const uint16_t* __restrict__ D = b.D[m] + 8 * cc;
  const uint16_t* __restrict__ XP = b.XP[m];
  float acc[8][R];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int j = 0; j < R; ++j) acc[e][j] = 0.f;
  for (int64_t t = t0; t < t1; ++t) {
    const uint4 dv = *reinterpret_cast<const uint4*>(D + t * b.ldd[m]);
    const uint32_t dw[4] = {dv.x, dv.y, dv.z, dv.w};
    float xp[R];
    load_bf16_row<R>(XP + t * R, xp);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float de = __uint_as_float(e & 1 ? (dw[e / 2] & 0xFFFF0000u) : (dw[e / 2] << 16));
#pragma unroll
      for (int j = 0; j < R; ++j) acc[e][j] += de * xp[j];
    }
  }
  float4* out = reinterpret_cast<float4*>(b.part + ((int64_t)blockIdx.y * b.chunks + gc) * 8 * R);
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int j = 0; j < R; j += 4) out[(e * R + j) / 4] = make_float4(acc[e][j], acc[e][j + 1], acc[e][j + 2], acc[e][j + 3]);
}

// Thread per C element: its token-chunk partials summed in chunk order, then
// added to C (one writer per element).
template <int R>
__global__ __launch_bounds__(256) void small_accumulate_finish_kernel(SmallAccumulateBatch b, int tchunks) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t gc = idx / (8 * R);
  if (gc >= b.chunks) return;
  const int q = (int)(idx % (8 * R));
  const int m = small_item(b.cbase, b.n, gc);
  const int64_t cc = gc - b.cbase[m];
  float sum = 0.f;
  for (int tc = 0; tc < tchunks; ++tc) {
    const float v = b.part[((int64_t)tc * b.chunks + gc) * 8 * R + q];
    sum = tc == 0 ? v : sum + v;
  }
  float* c = b.C[m] + (8 * cc + q / R) * R + q % R;
  *c += sum;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

template <int R>
rgc_status_t small_project_launch(int n, const uint16_t* const* Xs, const int64_t* ldxs, const int64_t* ks,
                                  const uint16_t* const* Ps, uint16_t* const* XPs, int64_t T, hipStream_t st) {
  SmallProjectBatch b = {};
  b.n = n;
  b.T = T;
  for (int m = 0; m < n; ++m) {
    b.X[m] = Xs[m];
    b.ldx[m] = ldxs[m];
    b.k[m] = ks[m];
    b.P[m] = Ps[m];
    b.XP[m] = XPs[m];
  }
  const int64_t rows = (int64_t)n * T;
  hipLaunchKernelGGL(small_project_kernel<R>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, b);
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

int64_t small_token_chunks(int64_t T) { return (T + kSmallTokenChunk - 1) / kSmallTokenChunk; }

template <int R>
size_t small_accumulate_workspace(int n, const int64_t* ds, int64_t T) {
  int64_t chunks = 0;
  for (int m = 0; m < n; ++m) chunks += ds[m] / 8;
  return (size_t)small_token_chunks(T) * chunks * 8 * R * sizeof(float);
}

template <int R>
rgc_status_t small_accumulate_launch(int n, const uint16_t* const* Ds, const int64_t* ldds, const int64_t* ds,
                                     const uint16_t* const* XPs, float* const* Cs, int64_t T, void* ws,
                                     hipStream_t st) {
  SmallAccumulateBatch b = {};
  b.n = n;
  b.T = T;
  b.cbase[0] = 0;
  for (int m = 0; m < n; ++m) {
    b.D[m] = Ds[m];
    b.ldd[m] = ldds[m];
    b.XP[m] = XPs[m];
    b.C[m] = Cs[m];
    b.cbase[m + 1] = b.cbase[m] + ds[m] / 8;
  }
  b.chunks = b.cbase[n];
  b.part = static_cast<float*>(ws);
  const int64_t tchunks = small_token_chunks(T);
  hipLaunchKernelGGL(small_accumulate_kernel<R>, dim3((unsigned)((b.chunks + 255) / 256), (unsigned)tchunks), dim3(256),
                     0, st, b);
  hipLaunchKernelGGL(small_accumulate_finish_kernel<R>, dim3((unsigned)((b.chunks * 8 * R + 255) / 256)), dim3(256), 0,
                     st, b, (int)tchunks);
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

// Workgroups per launch: one per compute unit (two fit, but measured on the
// Qwen3-1.7B-shaped block one is faster: the second adds L2/request pressure
// rather than hiding latency), or one per two compute units when that would
// leave fewer than kMinUnitsPerWorkgroup K-steps per workgroup: such short
// ranges pay their pipeline fill and their split-tile partials on little
// work (measured on one 4096 x 4096 matrix with 4096-token microbatches:
// 1.49 against 1.62 ms per step).
// `forced` > 0 replaces this choice (the test hooks only: the partition
// decides the fp32 summation order, so the product calls never take it from
// anything but the shapes and the device).
constexpr int64_t kMinUnitsPerWorkgroup = 16;
int64_t sketch_workgroups(int64_t units, int64_t forced) {
  if (forced > 0) return forced;
  const int64_t cus = device_compute_units();
  return units < kMinUnitsPerWorkgroup * cus ? (cus + 1) / 2 : cus;
}

// The schedule for items with N extents ns[] and K extents ks[].
Schedule make_schedule(int n, const int64_t* ns, const int64_t* ks, int64_t tile_n, int64_t kblock,
                       int64_t forced) {
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
  const int64_t G = sketch_workgroups(s.U, forced);
  s.G = (int)(s.U < G ? s.U : G);
  return s;
}

template <int RM, int GM = 1>
size_t partial_bytes(const Schedule& s) {
  return (size_t)2 * s.G * s.tile_n * sketch_width(GM * RM) * sizeof(float);
}

// Whether some tile is cut between ranges (then the finishing launch runs).
bool has_split_tiles(const Schedule& s) {
  for (int m = 0; m < s.n; ++m)
    for (int64_t t = 0; t < s.tbase[m + 1] - s.tbase[m]; ++t) {
      const int64_t ts = s.ubase[m] + t * s.nkb[m], te = ts + s.nkb[m];
      if (((ts + 1) * s.G - 1) / s.U != (te * s.G - 1) / s.U) return true;  // range_of(ts) != range_of(te - 1)
    }
  return false;
}

// One finishing workgroup per 1024 values of a tile (x) and per tile (y).
template <int RM, int GM = 1>
dim3 finish_grid(const Schedule& s) {
  return dim3((unsigned)((s.tile_n * sketch_width(GM * RM) + 1023) / 1024), (unsigned)s.tbase[s.n]);
}

// Waves along N of the narrow tiles (128 columns of N) of small launches:
// only at ranks where the wide tile has WN = 4 and two waves along r, so that
// the narrow one keeps four waves.
constexpr int kNarrowWN = 2;
static_assert(kNarrowWN == 2, "the narrow kernels above take two waves along N");
template <int R, int KH>
constexpr bool narrow_tile_ok() {
  return StageShape<R, KH>::WR == 2 && StageShape<R, KH>::WN != kNarrowWN;
}

template <int RM, int GM = 1, int WNF = 0>
Schedule project_schedule(int n, const int64_t* ns, const int64_t* ks, int64_t forced) {
  using Sh = StageShape<sketch_width(GM * RM), kProjectKH, WNF>;
  Schedule s = make_schedule(n, ns, ks, Sh::TILE, Sh::KS, forced);
  if (WNF > 0 && forced <= 0) {
    // narrow tiles: one workgroup per compute unit (see project_narrow)
    const int64_t cus = device_compute_units();
    s.G = (int)(s.U < cus ? s.U : cus);
  }
  return s;
}

// Narrow project tiles (128 tokens, WN = 2), as for the accumulate: when a
// one-matrix-per-group launch has too few K-steps for one workgroup per
// compute unit with 256-token tiles, the wide schedule takes half the compute
// units with ranges of a few K-steps; 128-token tiles give every compute unit
// such a range, at the same split-tile partial bytes. Only where the narrow
// tile keeps four waves. Never with a forced count.
template <int RM, int GM>
bool project_narrow(int n, const int64_t* ns, const int64_t* ks, int64_t forced) {
  if (GM != 1 || forced > 0 || !narrow_tile_ok<sketch_width(RM), kProjectKH>()) return false;
  const Schedule wide = project_schedule<RM, GM>(n, ns, ks, forced);
  return wide.U < kMinUnitsPerWorkgroup * device_compute_units();
}

// When every tile has the same K-steps (one token count for all items, as in
// the accumulate) and p >= 2 whole copies of the tile list fill at least 90%
// of the workgroups, the schedule takes p x tiles workgroups: every range
// then lies inside one tile and every tile has exactly p partials, instead
// of ranges that straddle tile ends and leave up to two partials each
// (measured on the Qwen3-1.7B-shaped block, 80 tiles: 240 workgroups 41.3 us
// against 256 workgroups 42.9 us per accumulate call). A forced workgroup
// count is kept as it is.
void align_ranges_to_tiles(Schedule& s, int64_t forced) {
  if (forced > 0) return;
  const int64_t tiles = s.tbase[s.n];
  for (int m = 1; m < s.n; ++m)
    if (s.nkb[m] != s.nkb[0]) return;
  const int64_t p = s.G / tiles;
  if (p >= 2 && p <= s.nkb[0] && 10 * p * tiles >= 9 * (int64_t)s.G) s.G = (int)(p * tiles);
}

template <int RM, int WNF = 0>
Schedule accumulate_schedule(int n, const int64_t* ns, const int64_t* ks, int64_t forced) {
  using Sh = StageShape<sketch_width(RM), 1, WNF>;
  Schedule s = make_schedule(n, ns, ks, Sh::TILE, Sh::KS, forced);
  align_ranges_to_tiles(s, forced);
  return s;
}

// Narrow accumulate tiles (128 columns of d, WN = 2): when a launch has too
// few K-steps for one workgroup per compute unit with 256-column tiles (a
// single 4096-wide matrix per microbatch: 16 tiles), the wide schedule takes
// half the compute units; 128-column tiles give twice the tiles, so every
// compute unit streams D, each tile cut no finer than before. Only where the
// narrow tile keeps four waves (two along r). Never with a forced count.
template <int RM>
bool accumulate_narrow(int n, const int64_t* ns, const int64_t* ks, int64_t forced) {
  if (forced > 0 || !narrow_tile_ok<sketch_width(RM), 1>()) return false;
  const Schedule wide = accumulate_schedule<RM>(n, ns, ks, forced);
  return wide.U < kMinUnitsPerWorkgroup * device_compute_units();
}

// Groups of a launch: with `shared`, the matrices that read the same X (same
// pointer, row stride and width) form groups of up to kMaxGroup members and
// at most 256 ranks in all, each projected in one pass over X (rgc_project_
// shared); otherwise every matrix is its own group (the batched project).
// Groups of one size share a launch. (Grouping inside the batched project
// was measured slower on the Qwen3-shaped blocks, 96 against 42 us per
// microbatch at r = 64: per-size launches leave each workgroup a few K-steps
// and many partial sums, and a group's P slabs take the LDS that would keep
// more X in flight.)
struct ProjectGroups {
  int n = 0;                        // groups
  int size[kMaxItems];              // members per group
  int member[kMaxItems][kMaxGroup];  // batch index of each member
};

ProjectGroups project_groups(int n, const uint16_t* const* Xs, const int64_t* ldxs, const int64_t* ks, int64_t r,
                             bool shared) {
  ProjectGroups g;
  const int cap = !shared ? 1 : ((int)(256 / r) < kMaxGroup ? (int)(256 / r) : kMaxGroup);
  for (int m = 0; m < n; ++m) {
    int gi = -1;
    for (int q = 0; q < g.n && gi < 0; ++q) {
      const int f = g.member[q][0];
      if (Xs[f] == Xs[m] && ldxs[f] == ldxs[m] && ks[f] == ks[m] && g.size[q] < cap) gi = q;
    }
    if (gi < 0) {
      gi = g.n++;
      g.size[gi] = 0;
    }
    g.member[gi][g.size[gi]++] = m;
  }
  return g;
}

// The groups with GM members, as one launch's schedule items.
template <int RM, int GM>
rgc_status_t project_launch_groups(const ProjectGroups& gr, const uint16_t* const* Xs, const int64_t* ldxs,
                                   const int64_t* ks, const uint16_t* const* Ps, uint16_t* const* XPs, int64_t T,
                                   void* ws, hipStream_t st, int64_t forced) {
  ProjectBatch pb = {};
  FinishBatch fb = {};
  int64_t ns[kMaxItems], kk[kMaxItems];
  int n = 0;
  for (int q = 0; q < gr.n; ++q) {
    if (gr.size[q] != GM) continue;
    const int f = gr.member[q][0];
    pb.X[n] = Xs[f];
    pb.ldx[n] = ldxs[f];
    for (int i = 0; i < GM; ++i) {
      pb.P[n][i] = Ps[gr.member[q][i]];
      pb.XP[n][i] = XPs[gr.member[q][i]];
      fb.XP[n][i] = XPs[gr.member[q][i]];
    }
    ns[n] = T;
    kk[n] = ks[f];
    ++n;
  }
  if (n == 0) return RGC_OK;
  pb.part = static_cast<float*>(ws);
  fb.part = pb.part;
  if constexpr (GM == 1 && narrow_tile_ok<sketch_width(RM), kProjectKH>()) {
    if (project_narrow<RM, GM>(n, ns, kk, forced)) {
      pb.s = project_schedule<RM, GM, kNarrowWN>(n, ns, kk, forced);
      fb.s = pb.s;
      hipLaunchKernelGGL(project_narrow_kernel<RM>, dim3((unsigned)pb.s.G), dim3((prj_threads<RM, 1, kNarrowWN>())),
                         0, st, pb);
      if (has_split_tiles(pb.s))
        hipLaunchKernelGGL((finish_narrow_tiles_kernel<RM, true>), (finish_grid<RM, GM>(pb.s)), dim3(256), 0, st, fb);
      return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
    }
  }
  pb.s = project_schedule<RM, GM>(n, ns, kk, forced);
  fb.s = pb.s;
  const dim3 grid = finish_grid<RM, GM>(pb.s);
  {
    hipLaunchKernelGGL((project_kernel<RM, GM>), dim3((unsigned)pb.s.G), dim3((prj_threads<RM, GM>())), 0, st, pb);
    if (has_split_tiles(pb.s)) hipLaunchKernelGGL((finish_tiles_kernel<RM, GM, true>), grid, dim3(256), 0, st, fb);
  }
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

// Calls f(IntC<GM>{}) for each group size GM (1 .. kMaxGroup) whose total
// width GM * RM stays within 256 ranks.
template <int RM, typename F>
void for_group_sizes(F&& f) {
  static_for<1, kMaxGroup + 1>([&](auto gm) {
    constexpr int GM = decltype(gm)::value;
    if constexpr (GM * RM <= 256) f(gm);
  });
}

template <int R>
rgc_status_t project_launch(int n, const uint16_t* const* Xs, const int64_t* ldxs, const int64_t* ks,
                            const uint16_t* const* Ps, uint16_t* const* XPs, int64_t T, void* ws, hipStream_t st,
                            int64_t forced, bool shared = false) {
  const ProjectGroups gr = project_groups(n, Xs, ldxs, ks, R, shared);
  rgc_status_t res = RGC_OK;
  for_group_sizes<R>([&](auto gm) {
    if (res == RGC_OK) res = project_launch_groups<R, decltype(gm)::value>(gr, Xs, ldxs, ks, Ps, XPs, T, ws, st, forced);
  });
  return res;
}

// Workspace of a batched project, a bound that holds for any grouping of its
// n items (the query does not see which items share an X): the largest
// partial-sum area of a launch with groups of GM <= n members, at the
// workgroup count of the schedule.
template <int R>
size_t project_workspace(int n, const int64_t* ks, int64_t T, int64_t forced, bool shared = false) {
  size_t out = 0;
  for_group_sizes<R>([&](auto gm) {
    constexpr int GM = decltype(gm)::value;
    if (GM > n || (GM > 1 && !shared)) return;
    int64_t ns[kMaxItems];
    for (int m = 0; m < n; ++m) ns[m] = T;
    // the same items as one group each: at least as many units, so at least
    // as many workgroups as any launch of the call with GM-member groups
    size_t b = partial_bytes<R, GM>(project_schedule<R, GM>(n, ns, ks, forced));
    if constexpr (GM == 1 && narrow_tile_ok<sketch_width(R), kProjectKH>())
      if (project_narrow<R, GM>(n, ns, ks, forced))
        b = partial_bytes<R, GM>(project_schedule<R, GM, kNarrowWN>(n, ns, ks, forced));
    out = b > out ? b : out;
  });
  return out;
}

// phase: bit 0 = the first call of an accumulation (the split tiles' slots are
// written), bit 1 = the last (the finishing launch adds the slots into C);
// 3 for a call that is both, the plain rgc_accumulate_batch.
template <int R>
rgc_status_t accumulate_launch(int n, const uint16_t* const* Ds, const int64_t* ldds, const int64_t* ds,
                               const uint16_t* const* XPs, float* const* Cs, int64_t T, void* ws, hipStream_t st,
                               int64_t forced, int phase) {
  int64_t ks[kMaxItems];
  for (int m = 0; m < n; ++m) ks[m] = T;
  constexpr bool kNarrowOk = narrow_tile_ok<sketch_width(R), 1>();
  const bool narrow = kNarrowOk && accumulate_narrow<R>(n, ds, ks, forced);
  AccumulateBatch ab = {};
  ab.s = narrow ? accumulate_schedule<R, kNarrowOk ? kNarrowWN : 0>(n, ds, ks, forced)
                : accumulate_schedule<R>(n, ds, ks, forced);
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
  ab.add_part = (phase & 1) ? 0 : 1;
  fb.part = ab.part;
  if constexpr (kNarrowOk) {
    if (narrow) {
      hipLaunchKernelGGL(accumulate_narrow_kernel<R>, dim3((unsigned)ab.s.G), dim3((acc_threads<R, kNarrowWN>())), 0,
                         st, ab);
      if ((phase & 2) && has_split_tiles(ab.s))
        hipLaunchKernelGGL((finish_narrow_tiles_kernel<R, false>), finish_grid<R>(ab.s), dim3(256), 0, st, fb);
      return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
    }
  }
  {
    hipLaunchKernelGGL(accumulate_kernel<R>, dim3((unsigned)ab.s.G), dim3(acc_threads<R>()), 0, st, ab);
    if ((phase & 2) && has_split_tiles(ab.s))
      hipLaunchKernelGGL((finish_tiles_kernel<R, 1, false>), finish_grid<R>(ab.s), dim3(256), 0, st, fb);
  }
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

template <int R>
size_t accumulate_workspace(int n, const int64_t* ds, int64_t T, int64_t forced) {
  int64_t ks[kMaxItems];
  for (int m = 0; m < n; ++m) ks[m] = T;
  if constexpr (narrow_tile_ok<sketch_width(R), 1>())
    if (accumulate_narrow<R>(n, ds, ks, forced))
      return partial_bytes<R>(accumulate_schedule<R, kNarrowWN>(n, ds, ks, forced));
  return partial_bytes<R>(accumulate_schedule<R>(n, ds, ks, forced));
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

namespace {

size_t project_ws_impl(int64_t n, const int64_t* ks, int64_t T, int64_t r, int64_t forced) {
  if (n <= 0 || n > kMaxItems || !ks || T <= 0) return 0;
  for (int64_t m = 0; m < n; ++m)
    if (ks[m] <= 0) return 0;
  if (rank_small(r)) return 0;  // no partial sums
  size_t out = 0;
  if (!dispatch_rank(r, [&](auto rc) { out = project_workspace<decltype(rc)::value>((int)n, ks, T, forced); }))
    return 0;
  return out;
}

size_t accumulate_ws_impl(int64_t n, const int64_t* ds, int64_t T, int64_t r, int64_t forced) {
  if (n <= 0 || n > kMaxItems || !ds || T <= 0) return 0;
  for (int64_t m = 0; m < n; ++m)
    if (ds[m] <= 0) return 0;
  size_t out = 0;
  if (dispatch_small_rank(r, [&](auto rc) { out = small_accumulate_workspace<decltype(rc)::value>((int)n, ds, T); }))
    return out;
  if (!dispatch_rank(r, [&](auto rc) {
        constexpr int R = decltype(rc)::value;
        out = accumulate_workspace<R>((int)n, ds, T, forced);
      }))
    return 0;
  return out;
}

rgc_status_t project_batch_impl(int64_t n, const uint16_t* const* Xs, const int64_t* ldxs, const int64_t* ks,
                                const uint16_t* const* Ps, uint16_t* const* XPs, int64_t T, int64_t r, void* ws,
                                size_t ws_bytes, void* stream, int64_t forced) {
  if (n < 0 || T < 0 || r <= 0) return RGC_ERR_SHAPE;
  if (n > kMaxItems || !rank_supported(r) || T > kMaxTiledDim) return RGC_ERR_UNSUPPORTED;
  if (n == 0 || T == 0) return RGC_OK;
  if (!Xs || !ldxs || !ks || !Ps || !XPs) return RGC_ERR_NULL;
  for (int64_t m = 0; m < n; ++m) {
    const rgc_status_t st = check_project_item(Xs[m], ldxs[m], ks[m], Ps[m], XPs[m], T, r);
    if (st != RGC_OK) return st;
  }
  const size_t need = project_ws_impl(n, ks, T, r, forced);
  if (need > 0 && (!ws || ws_bytes < need)) return RGC_ERR_WORKSPACE;
  if (need > 0 && !aligned_to(ws, 256)) return RGC_ERR_ALIGN;
  rgc_status_t st = RGC_OK;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (dispatch_small_rank(r, [&](auto rc) {
        st = small_project_launch<decltype(rc)::value>((int)n, Xs, ldxs, ks, Ps, XPs, T, hs);
      }))
    return st;
  dispatch_rank(r, [&](auto rc) {
    st = project_launch<decltype(rc)::value>((int)n, Xs, ldxs, ks, Ps, XPs, T, ws, hs, forced);
  });
  return st;
}

rgc_status_t accumulate_batch_impl(int64_t n, const uint16_t* const* Ds, const int64_t* ldds, const int64_t* ds,
                                   const uint16_t* const* XPs, float* const* Cs, int64_t T, int64_t r, void* ws,
                                   size_t ws_bytes, void* stream, int64_t forced, int phase = 3) {
  if (n < 0 || T < 0 || r <= 0) return RGC_ERR_SHAPE;
  if (n > kMaxItems || !rank_supported(r)) return RGC_ERR_UNSUPPORTED;
  if (n == 0 || T == 0) return RGC_OK;
  if (!Ds || !ldds || !ds || !XPs || !Cs) return RGC_ERR_NULL;
  for (int64_t m = 0; m < n; ++m) {
    const rgc_status_t st = check_accumulate_item(Ds[m], ldds[m], ds[m], XPs[m], Cs[m], T);
    if (st != RGC_OK) return st;
  }
  const size_t need = accumulate_ws_impl(n, ds, T, r, forced);
  if (need > 0 && (!ws || ws_bytes < need)) return RGC_ERR_WORKSPACE;
  if (need > 0 && !aligned_to(ws, 256)) return RGC_ERR_ALIGN;
  rgc_status_t st = RGC_OK;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (dispatch_small_rank(r, [&](auto rc) {
        st = small_accumulate_launch<decltype(rc)::value>((int)n, Ds, ldds, ds, XPs, Cs, T, ws, hs);
      }))
    return st;
  dispatch_rank(r, [&](auto rc) {
    st = accumulate_launch<decltype(rc)::value>((int)n, Ds, ldds, ds, XPs, Cs, T, ws, hs, forced, phase);
  });
  return st;
}

}  // namespace

extern "C" size_t rgc_project_batch_workspace_size(int64_t n, const int64_t* ks, int64_t T, int64_t r) {
  return project_ws_impl(n, ks, T, r, 0);
}

extern "C" size_t rgc_accumulate_batch_workspace_size(int64_t n, const int64_t* ds, int64_t T, int64_t r) {
  return accumulate_ws_impl(n, ds, T, r, 0);
}

extern "C" rgc_status_t rgc_project_batch(int64_t n, const uint16_t* const* Xs, const int64_t* ldxs,
                                          const int64_t* ks, const uint16_t* const* Ps, uint16_t* const* XPs,
                                          int64_t T, int64_t r, void* ws, size_t ws_bytes, void* stream) {
  return project_batch_impl(n, Xs, ldxs, ks, Ps, XPs, T, r, ws, ws_bytes, stream, 0);
}

extern "C" rgc_status_t rgc_accumulate_batch(int64_t n, const uint16_t* const* Ds, const int64_t* ldds,
                                             const int64_t* ds, const uint16_t* const* XPs, float* const* Cs,
                                             int64_t T, int64_t r, void* ws, size_t ws_bytes, void* stream) {
  return accumulate_batch_impl(n, Ds, ldds, ds, XPs, Cs, T, r, ws, ws_bytes, stream, 0);
}

extern "C" rgc_status_t rgc_accumulate_batch_deferred(int64_t n, const uint16_t* const* Ds, const int64_t* ldds,
                                                      const int64_t* ds, const uint16_t* const* XPs, float* const* Cs,
                                                      int64_t T, int64_t r, void* ws, size_t ws_bytes, int phase,
                                                      void* stream) {
  if (phase < 0 || phase > 3) return RGC_ERR_SHAPE;
  return accumulate_batch_impl(n, Ds, ldds, ds, XPs, Cs, T, r, ws, ws_bytes, stream, 0, phase);
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

// Test hooks: the batched contractions with the workgroup count given by the
// caller (> 0) instead of chosen from the shapes, so that tests can force
// ranges of whole tiles that cross item boundaries.
extern "C" size_t rgc_test_sketch_workspace_size(int contraction, int64_t workgroups, int64_t n,
                                                 const int64_t* widths, int64_t T, int64_t r) {
  if (workgroups <= 0) return 0;
  return contraction == 0 ? project_ws_impl(n, widths, T, r, workgroups)
                          : accumulate_ws_impl(n, widths, T, r, workgroups);
}

extern "C" rgc_status_t rgc_test_project_batch_wgs(int64_t workgroups, int64_t n, const uint16_t* const* Xs,
                                                   const int64_t* ldxs, const int64_t* ks,
                                                   const uint16_t* const* Ps, uint16_t* const* XPs, int64_t T,
                                                   int64_t r, void* ws, size_t ws_bytes, void* stream) {
  if (workgroups <= 0) return RGC_ERR_SHAPE;
  return project_batch_impl(n, Xs, ldxs, ks, Ps, XPs, T, r, ws, ws_bytes, stream, workgroups);
}

extern "C" rgc_status_t rgc_test_accumulate_batch_wgs(int64_t workgroups, int64_t n, const uint16_t* const* Ds,
                                                      const int64_t* ldds, const int64_t* ds,
                                                      const uint16_t* const* XPs, float* const* Cs, int64_t T,
                                                      int64_t r, void* ws, size_t ws_bytes, void* stream) {
  if (workgroups <= 0) return RGC_ERR_SHAPE;
  return accumulate_batch_impl(n, Ds, ldds, ds, XPs, Cs, T, r, ws, ws_bytes, stream, workgroups);
}

extern "C" rgc_status_t rgc_test_accumulate_batch_deferred_wgs(int64_t workgroups, int64_t n,
                                                               const uint16_t* const* Ds, const int64_t* ldds,
                                                               const int64_t* ds, const uint16_t* const* XPs,
                                                               float* const* Cs, int64_t T, int64_t r, void* ws,
                                                               size_t ws_bytes, int phase, void* stream) {
  if (workgroups <= 0 || phase < 0 || phase > 3) return RGC_ERR_SHAPE;
  return accumulate_batch_impl(n, Ds, ldds, ds, XPs, Cs, T, r, ws, ws_bytes, stream, workgroups, phase);
}

// ---- one pass over a shared X ---------------------------------------------
namespace {

size_t project_shared_ws_impl(int64_t n, int64_t T, int64_t k, int64_t r, int64_t forced) {
  if (n <= 0 || n > kMaxGroup || T <= 0 || k <= 0 || !rank_tiled(r) || n * r > 256) return 0;
  int64_t ks[kMaxGroup];
  for (int64_t m = 0; m < n; ++m) ks[m] = k;
  size_t out = 0;
  dispatch_rank(r, [&](auto rc) { out = project_workspace<decltype(rc)::value>((int)n, ks, T, forced, true); });
  return out;
}

rgc_status_t project_shared_impl(int64_t n, const uint16_t* X, int64_t ldx, int64_t k, const uint16_t* const* Ps,
                                 uint16_t* const* XPs, int64_t T, int64_t r, void* ws, size_t ws_bytes, void* stream,
                                 int64_t forced) {
  if (n < 0 || T < 0 || r <= 0 || k <= 0) return RGC_ERR_SHAPE;
  if (n > kMaxGroup || !rank_tiled(r) || n * r > 256 || T > kMaxTiledDim) return RGC_ERR_UNSUPPORTED;
  if (n == 0 || T == 0) return RGC_OK;
  if (!Ps || !XPs) return RGC_ERR_NULL;
  const uint16_t* Xs[kMaxGroup];
  int64_t ldxs[kMaxGroup], ks[kMaxGroup];
  for (int64_t m = 0; m < n; ++m) {
    Xs[m] = X;
    ldxs[m] = ldx;
    ks[m] = k;
    const rgc_status_t st = check_project_item(X, ldx, k, Ps[m], XPs[m], T, r);
    if (st != RGC_OK) return st;
  }
  const size_t need = project_shared_ws_impl(n, T, k, r, forced);
  if (need > 0 && (!ws || ws_bytes < need)) return RGC_ERR_WORKSPACE;
  if (need > 0 && !aligned_to(ws, 256)) return RGC_ERR_ALIGN;
  rgc_status_t st = RGC_OK;
  dispatch_rank(r, [&](auto rc) {
    st = project_launch<decltype(rc)::value>((int)n, Xs, ldxs, ks, Ps, XPs, T, ws, static_cast<hipStream_t>(stream),
                                             forced, true);
  });
  return st;
}

}  // namespace

extern "C" size_t rgc_project_shared_workspace_size(int64_t n, int64_t T, int64_t k, int64_t r) {
  return project_shared_ws_impl(n, T, k, r, 0);
}

extern "C" rgc_status_t rgc_project_shared(int64_t n, const uint16_t* X, int64_t ldx, int64_t k,
                                           const uint16_t* const* Ps, uint16_t* const* XPs, int64_t T, int64_t r,
                                           void* ws, size_t ws_bytes, void* stream) {
  return project_shared_impl(n, X, ldx, k, Ps, XPs, T, r, ws, ws_bytes, stream, 0);
}

extern "C" size_t rgc_test_project_shared_workspace_size(int64_t workgroups, int64_t n, int64_t T, int64_t k,
                                                         int64_t r) {
  return workgroups > 0 ? project_shared_ws_impl(n, T, k, r, workgroups) : 0;
}

extern "C" rgc_status_t rgc_test_project_shared_wgs(int64_t workgroups, int64_t n, const uint16_t* X, int64_t ldx,
                                                    int64_t k, const uint16_t* const* Ps, uint16_t* const* XPs,
                                                    int64_t T, int64_t r, void* ws, size_t ws_bytes, void* stream) {
  if (workgroups <= 0) return RGC_ERR_SHAPE;
  return project_shared_impl(n, X, ldx, k, Ps, XPs, T, r, ws, ws_bytes, stream, workgroups);
}
