// The two skinny contractions of the sketch, on bf16 MFMA with fp32 sums:
//   project:    XP = bf16(X P)         X: T x k, P: k x r      [RGC, "How it works"]
//   accumulate: C += D^T XP            D: T x d, XP: T x r     [RGC, "How it works";
//                                      LoGRA-S, Key Contributions 1]
// ([RGC] = page "Randomized Gradient Compression"; [LoGRA-S] = page "LoGRA:
// Scaling LLM Reinforcement Learning with Low-Rank Gradient Sketches".)
//
// Both kernels put the rank dimension r on the MFMA's M side. Its operand
// (P or XP) is read with a register transpose: a lane loads CPL consecutive r
// columns for eight consecutive K rows and repacks them, so M-tile c row m
// is r = base + CPL*m + c. With that ordering each lane's output is a
// contiguous run of 4*CPL values of r, which is what makes the stores
// (XP rows, C rows) contiguous.
//
// Both are HBM-bound at the ranks of interest (a few flops per byte), so the
// loops are written for memory-level parallelism: every load is unconditional
// (out-of-range rows are clamped to a valid address and their values zeroed),
// addresses are 32-bit offsets from workgroup-uniform bases, and the next
// K-step's loads are issued before the current step's MFMAs.
//
// Work is split over K (k for project, tokens for accumulate) first across the
// waves of a workgroup (summed through LDS, each wave finishing the N-tiles it
// owns) and then, when the output alone has too few tiles to fill the chip,
// across workgroups: each writes an output-shaped fp32 partial and a second,
// fully parallel launch sums the partials in split order. Both reductions
// have a fixed order, so results are bit-reproducible. There is no
// cross-workgroup signalling inside a launch: a device-scope release costs an
// L2 writeback per wave on this part, which serializes across hundreds of
// workgroups, while the launch boundary orders the partials for free.
#include "rgc_internal.hpp"

namespace rgc {

// ---------------------------------------------------------------------------
// Shared pieces
// ---------------------------------------------------------------------------

// Raw (untransposed) M-side rows of one 32-row K-step: for each column group
// q and row j = 0..7, the CPL columns the lane reads, packed in dwords.
template <int R>
struct RankRows {
  static constexpr int W = (RankTraits<R>::CPL + 1) / 2;
  uint32_t v[RankTraits<R>::NG][8][W];
};

// Loads rows krow0 + 8g + j (j = 0..7) of a row-major bf16 matrix with
// compile-time row stride R (src already points at the wave's first column),
// columns q*GW + CPL*m .. +CPL-1, for a lane (m = lane % 16, g = lane / 16).
// Rows >= nrows read row nrows-1 and are zeroed.
template <int R>
__device__ __forceinline__ void load_rank_rows(const uint16_t* __restrict__ src, int64_t krow0, int64_t nrows,
                                               int lane, RankRows<R>& out) {
  using Tr = RankTraits<R>;
  constexpr int CPL = Tr::CPL;
  const int m = lane & 15, g = lane >> 4;
  const int64_t base_row = krow0 < nrows ? krow0 : nrows - 1;  // uniform
  const uint16_t* base = src + base_row * R + CPL * m;
  const int64_t room = nrows - 1 - base_row;  // rows available after base_row
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t want = krow0 + 8 * g + j - base_row;
    const bool ok = krow0 + 8 * g + j < nrows;
    const uint32_t off = (uint32_t)((want < room ? want : room) * R);
#pragma unroll
    for (int q = 0; q < Tr::NG; ++q) {
      const uint16_t* p = base + off + q * Tr::GW;
      if constexpr (CPL == 4) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        out.v[q][j][0] = ok ? v.x : 0u;
        out.v[q][j][1] = ok ? v.y : 0u;
      } else if constexpr (CPL == 2) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
        out.v[q][j][0] = ok ? v : 0u;
      } else {
        const uint32_t v = *p;
        out.v[q][j][0] = ok ? v : 0u;
      }
    }
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

// Gathers, for N-tile `nt` and column group q, the 4*CPL contiguous rank
// values a lane owns: out[CPL*i + c] = acc[q*CPL + c][nt][i].
template <int R>
__device__ __forceinline__ void gather_rank_run(const f32x4_t (&acc)[RankTraits<R>::MT][4], int q, int nt,
                                                float (&out)[4 * RankTraits<R>::CPL]) {
  constexpr int CPL = RankTraits<R>::CPL;
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) out[CPL * i + c] = acc[q * CPL + c][nt][i];
}

__device__ __forceinline__ int g_of(int lane) { return lane >> 4; }

// The four N-tiles of a wave's output are split among the KS waves that share
// an r-slice: wave ks owns N-tiles nt with nt % KS == ks, and after the
// reductions below it holds the finished sums for exactly those.
template <int KS>
__device__ __forceinline__ constexpr bool owns_ntile(int nt, int ks) { return (nt % KS) == ks; }

// Sums the KS waves' accumulators through LDS: every wave stores all of its
// tile, then each wave adds, for the N-tiles it owns, the KS copies in wave
// order (fixed order, so the result does not depend on timing).
// `lds` holds KS * NR * MT * 16 * 64 floats.
template <int R, int KS>
__device__ __forceinline__ void reduce_waves(f32x4_t (&acc)[RankTraits<R>::MT][4], float* lds, int rw, int ks,
                                             int lane) {
  using Tr = RankTraits<R>;
  constexpr int E = Tr::MT * 16;  // floats per lane
  if constexpr (KS > 1) {
    float* mine = lds + (ks * Tr::NR + rw) * E * 64;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int mt = 0; mt < Tr::MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mine[((nt * Tr::MT + mt) * 4 + i) * 64 + lane] = acc[mt][nt][i];
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
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

// Writes the 4*CPL-wide rank runs of the N-tiles this wave owns to an fp32
// row-major buffer with row stride R (an output-shaped split partial). Rows of
// N-tile nt: TOKEN_ROWS (project) row0 + 16*nt + n, else (accumulate)
// row0 + 4*n + nt.
template <int R, int KS, bool TOKEN_ROWS>
__device__ __forceinline__ void store_runs_f32(const f32x4_t (&acc)[RankTraits<R>::MT][4], float* __restrict__ out,
                                               int64_t row0, int64_t nrows, int rbase, int ks, int lane) {
  using Tr = RankTraits<R>;
  const int n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t row = TOKEN_ROWS ? row0 + 16 * nt + n : row0 + 4 * n + nt;
    if (!owns_ntile<KS>(nt, ks) || row >= nrows) continue;
#pragma unroll
    for (int q = 0; q < Tr::NG; ++q) {
      float run[4 * Tr::CPL];
      gather_rank_run<R>(acc, q, nt, run);
      float4* dst = reinterpret_cast<float4*>(out + row * R + rbase + q * Tr::GW + 4 * Tr::CPL * g);
#pragma unroll
      for (int v = 0; v < Tr::CPL; ++v) dst[v] = make_float4(run[4 * v], run[4 * v + 1], run[4 * v + 2], run[4 * v + 3]);
    }
  }
}

// ---------------------------------------------------------------------------
// Work-item tables: one launch covers a list of independent matrices of one
// rank (e.g. all projections of a transformer block). Workgroup b belongs to
// the item whose [wg_begin, wg_begin') range holds b.
// ---------------------------------------------------------------------------
constexpr int kMaxItems = 16;

__device__ __forceinline__ int item_of(const int* begin, int n, int b) {
  int m = 0;
  while (m + 1 < n && b >= begin[m + 1]) ++m;
  return m;
}

struct ProjectBatch {
  int n;
  int64_t T, tiles;                 // tokens (shared) and 64-token tiles per item
  int wg_begin[kMaxItems + 1];      // tiles * splits workgroups per item
  const uint16_t* X[kMaxItems];
  int64_t ldx[kMaxItems];
  int64_t k[kMaxItems];
  const uint16_t* P[kMaxItems];
  uint16_t* XP[kMaxItems];
  int64_t kchunk[kMaxItems];
  int splits[kMaxItems];
  float* part[kMaxItems];           // splits x T x R fp32 when splits > 1
};

struct AccumulateBatch {
  int n;
  int64_t T, tchunk;                // tokens and tokens per split (shared)
  int splits;
  int wg_begin[kMaxItems + 1];      // tiles * splits workgroups per item
  const uint16_t* D[kMaxItems];
  int64_t ldd[kMaxItems];
  int64_t d[kMaxItems];
  int64_t tiles[kMaxItems];
  const uint16_t* XP[kMaxItems];
  float* C[kMaxItems];
  float* part[kMaxItems];           // splits x d x R fp32 when splits > 1
};

// ---------------------------------------------------------------------------
// project: XP = bf16(X P)
// Workgroup = (item, 64-token tile, k-split); its NR x KS waves take r-slices
// x interleaved K-steps.
// ---------------------------------------------------------------------------
struct XRows {
  uint32_t v[4][4];  // per N-tile: 8 consecutive k of one token (16 bytes)
};

__device__ __forceinline__ void load_x_rows(const uint16_t* __restrict__ X, int64_t ldx, int64_t T, int64_t tbase,
                                            int64_t k0, int64_t kend, int lane, XRows& out) {
  const int n = lane & 15, g = lane >> 4;
  const int64_t kc = k0 + 8 * g;
  const bool kok = kc < kend;
  const int64_t kcl = kok ? kc : kend - 8;  // kend is a multiple of 8
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t t = tbase + 16 * nt + n;
    const bool ok = kok && t < T;
    const int64_t tc = t < T ? t : T - 1;
    const u32x4v_t v = load_stream_16b(X + tc * ldx + kcl);
    out.v[nt][0] = ok ? v.x : 0u;
    out.v[nt][1] = ok ? v.y : 0u;
    out.v[nt][2] = ok ? v.z : 0u;
    out.v[nt][3] = ok ? v.w : 0u;
  }
}

template <int R>
__global__ __launch_bounds__(256) void project_kernel(ProjectBatch pb) {
  using Tr = RankTraits<R>;
  constexpr int KS = Tr::KS;
  __shared__ float lds[KS > 1 ? KS * Tr::NR * Tr::MT * 16 * 64 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rw = wave % Tr::NR, ks = wave / Tr::NR;
  const int rbase = rw * Tr::RPW;
  const int n = lane & 15, g = lane >> 4;
  const int m = item_of(pb.wg_begin, pb.n, blockIdx.x);
  const int local = blockIdx.x - pb.wg_begin[m];
  const int64_t T = pb.T;
  const int64_t tbase = (int64_t)(local % pb.tiles) * 64;
  const int split = (int)(local / pb.tiles);
  const int splits = pb.splits[m];
  const int64_t k = pb.k[m], kchunk = pb.kchunk[m];
  const int64_t kbeg = split * kchunk;
  const int64_t kend = kbeg + kchunk < k ? kbeg + kchunk : k;
  const uint16_t* X = pb.X[m];
  const int64_t ldx = pb.ldx[m];
  const uint16_t* P = pb.P[m] + rbase;

  f32x4_t acc[Tr::MT][4];
#pragma unroll
  for (int mt = 0; mt < Tr::MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  int64_t k0 = kbeg + 32 * ks;
  RankRows<R> pa;
  XRows xb;
  load_rank_rows<R>(P, k0, kend, lane, pa);
  load_x_rows(X, ldx, T, tbase, k0, kend, lane, xb);
  for (; k0 < kend; k0 += 32 * KS) {
    RankRows<R> pn;
    XRows xn;
    load_rank_rows<R>(P, k0 + 32 * KS, kend, lane, pn);
    load_x_rows(X, ldx, T, tbase, k0 + 32 * KS, kend, lane, xn);
    uint32_t aop[Tr::MT][4];
    transpose_rank_rows<R>(pa, aop);
#pragma unroll
    for (int mt = 0; mt < Tr::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_16x16x32(aop[mt], xb.v[nt], acc[mt][nt]);
    pa = pn;
    xb = xn;
  }

  reduce_waves<R, KS>(acc, lds, rw, ks, lane);
  if (splits > 1) {  // output-shaped fp32 partial (T x R) for the finishing pass
    store_runs_f32<R, KS, true>(acc, pb.part[m] + (int64_t)split * T * R, tbase, T, rbase, ks, lane);
    return;
  }
  uint16_t* XP = pb.XP[m];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t t = tbase + 16 * nt + n;
    if (!owns_ntile<KS>(nt, ks) || t >= T) continue;
#pragma unroll
    for (int q = 0; q < Tr::NG; ++q) {
      float run[4 * Tr::CPL];
      gather_rank_run<R>(acc, q, nt, run);
      uint16_t* dst = XP + t * R + rbase + q * Tr::GW + 4 * Tr::CPL * g;
      uint32_t packed[2 * Tr::CPL];
#pragma unroll
      for (int e = 0; e < 2 * Tr::CPL; ++e)
        packed[e] = pack_bf16x2(f32_to_bf16_rne(run[2 * e]), f32_to_bf16_rne(run[2 * e + 1]));
      if constexpr (Tr::CPL == 4) {
        reinterpret_cast<uint4*>(dst)[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        reinterpret_cast<uint4*>(dst)[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
      } else if constexpr (Tr::CPL == 2) {
        reinterpret_cast<uint4*>(dst)[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
      } else {
        reinterpret_cast<uint2*>(dst)[0] = make_uint2(packed[0], packed[1]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// accumulate: C += D^T XP
// Workgroup = (item, 64-row d tile, token split); its NR x KS waves take
// r-slices x interleaved 32-token steps. D is token-major, so its operand is
// also transposed in registers: lane (n, g) reads 4 consecutive d for eight
// tokens, and N-tile c column n is d = dbase + 4n + c.
// ---------------------------------------------------------------------------
struct DRows {
  uint32_t v[8][2];  // 8 tokens x 4 consecutive d (bf16 pairs)
};

__device__ __forceinline__ void load_d_rows(const uint16_t* __restrict__ Dm, int64_t ldd, int64_t t0, int64_t tend,
                                            int64_t dcol, bool dvalid, int lane, DRows& out) {
  const int g = lane >> 4;
  const int64_t base_row = t0 < tend ? t0 : tend - 1;  // uniform
  const uint16_t* base = Dm + base_row * ldd + dcol;
  const int64_t room = tend - 1 - base_row;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t want = t0 + 8 * g + j - base_row;
    const bool ok = dvalid && (t0 + 8 * g + j < tend);
    const uint32_t off = (uint32_t)((want < room ? want : room) * ldd);
    const u32x2v_t v = load_stream_8b(base + off);
    out.v[j][0] = ok ? v.x : 0u;
    out.v[j][1] = ok ? v.y : 0u;
  }
}

template <int R>
__global__ __launch_bounds__(256) void accumulate_kernel(AccumulateBatch ab) {
  using Tr = RankTraits<R>;
  constexpr int KS = Tr::KS;
  __shared__ float lds[KS > 1 ? KS * Tr::NR * Tr::MT * 16 * 64 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rw = wave % Tr::NR, ks = wave / Tr::NR;
  const int rbase = rw * Tr::RPW;
  const int n = lane & 15;
  const int m = item_of(ab.wg_begin, ab.n, blockIdx.x);
  const int local = blockIdx.x - ab.wg_begin[m];
  const int64_t tiles = ab.tiles[m];
  const int64_t dbase = (int64_t)(local % tiles) * 64;
  const int split = (int)(local / tiles);
  const int64_t T = ab.T, d = ab.d[m];
  const int64_t tbeg = split * ab.tchunk;
  const int64_t tend = tbeg + ab.tchunk < T ? tbeg + ab.tchunk : T;
  const bool dvalid = dbase + 4 * n < d;  // d % 4 == 0: a lane's 4 columns are all in or all out
  const int64_t dcol = dvalid ? dbase + 4 * n : 0;
  const uint16_t* Dm = ab.D[m];
  const int64_t ldd = ab.ldd[m];
  const uint16_t* XPm = ab.XP[m] + rbase;

  f32x4_t acc[Tr::MT][4];
#pragma unroll
  for (int mt = 0; mt < Tr::MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  int64_t t0 = tbeg + 32 * ks;
  DRows db;
  RankRows<R> xa;
  load_d_rows(Dm, ldd, t0, tend, dcol, dvalid, lane, db);
  load_rank_rows<R>(XPm, t0, tend, lane, xa);
  for (; t0 < tend; t0 += 32 * KS) {
    DRows dn;
    RankRows<R> xn;
    load_d_rows(Dm, ldd, t0 + 32 * KS, tend, dcol, dvalid, lane, dn);
    load_rank_rows<R>(XPm, t0 + 32 * KS, tend, lane, xn);
    uint32_t aop[Tr::MT][4];
    transpose_rank_rows<R>(xa, aop);
    uint32_t bop[4][4];
#pragma unroll
    for (int c = 0; c < 4; ++c) transpose_8xcpl<4>(db.v, c, bop[c]);
#pragma unroll
    for (int mt = 0; mt < Tr::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_16x16x32(aop[mt], bop[nt], acc[mt][nt]);
    db = dn;
    xa = xn;
  }

  reduce_waves<R, KS>(acc, lds, rw, ks, lane);
  if (!dvalid) return;
  if (ab.splits > 1) {  // output-shaped fp32 partial (d x R) for the finishing pass
    store_runs_f32<R, KS, false>(acc, ab.part[m] + (int64_t)split * d * R, dbase, d, rbase, ks, lane);
    return;
  }
  float* C = ab.C[m];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    if (!owns_ntile<KS>(nt, ks)) continue;
    const int64_t drow = dbase + 4 * n + nt;
#pragma unroll
    for (int q = 0; q < Tr::NG; ++q) {
      float run[4 * Tr::CPL];
      gather_rank_run<R>(acc, q, nt, run);
      float* dst = C + drow * R + rbase + q * Tr::GW + 4 * Tr::CPL * g_of(lane);
#pragma unroll
      for (int v = 0; v < Tr::CPL; ++v) {
        float4 old = reinterpret_cast<float4*>(dst)[v];
        old.x += run[4 * v + 0];
        old.y += run[4 * v + 1];
        old.z += run[4 * v + 2];
        old.w += run[4 * v + 3];
        reinterpret_cast<float4*>(dst)[v] = old;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Finishing pass over split partials (fp32, output-shaped, `splits` slabs per
// item): each thread sums four consecutive values over the splits in split
// order, with a batch of splits' loads in flight, then rounds them to bf16
// into XP (project) or adds them to C (accumulate). Workgroup b belongs to
// the item whose [fin_begin, fin_begin') range holds b.
// ---------------------------------------------------------------------------
struct FinishBatch {
  int n;
  int fin_begin[kMaxItems + 1];
  const float* part[kMaxItems];
  int splits[kMaxItems];
  int64_t count[kMaxItems];  // floats per slab
  float* C[kMaxItems];       // accumulate targets
  uint16_t* XP[kMaxItems];   // project targets
};

template <bool TO_BF16>
__global__ __launch_bounds__(256) void finish_splits_kernel(FinishBatch fb) {
  const int m = item_of(fb.fin_begin, fb.n, blockIdx.x);
  const int64_t e = ((int64_t)(blockIdx.x - fb.fin_begin[m]) * blockDim.x + threadIdx.x) * 4;
  const int64_t count = fb.count[m];
  const int splits = fb.splits[m];
  const float* partials = fb.part[m];
  if (e >= count) return;
  constexpr int BATCH = 8;
  f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += BATCH) {
    float4 v[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int sb = s0 + b < splits ? s0 + b : splits - 1;
      v[b] = *reinterpret_cast<const float4*>(partials + (int64_t)sb * count + e);
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      if (s0 + b < splits) {
        const f32x4_t x = {v[b].x, v[b].y, v[b].z, v[b].w};
        sum = (s0 + b == 0) ? x : sum + x;
      }
    }
  }
  if constexpr (TO_BF16) {
    const uint2 out = make_uint2(pack_bf16x2(f32_to_bf16_rne(sum[0]), f32_to_bf16_rne(sum[1])),
                                 pack_bf16x2(f32_to_bf16_rne(sum[2]), f32_to_bf16_rne(sum[3])));
    *reinterpret_cast<uint2*>(fb.XP[m] + e) = out;
  } else {
    float4 old = *reinterpret_cast<float4*>(fb.C[m] + e);
    old.x += sum[0];
    old.y += sum[1];
    old.z += sum[2];
    old.w += sum[3];
    *reinterpret_cast<float4*>(fb.C[m] + e) = old;
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

// Workgroups that keep all 256 compute units streaming (two resident
// workgroups per compute unit).
int target_workgroups() { return env_int("RGC_TARGET_WGS", 512); }

inline size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// Project plan: every item gets a k-chunk of about the same size, so that all
// workgroups carry similar bytes; the chunk shrinks (more splits) until the
// launch has enough workgroups, within 64 splits per item.
struct ProjectPlan {
  int64_t tiles;
  int64_t kchunk[kMaxItems];
  int splits[kMaxItems];
  int wg_begin[kMaxItems + 1];
  size_t part_off[kMaxItems];
  size_t ws_bytes;
};

template <int R>
ProjectPlan project_plan(int n, const int64_t* ks, int64_t T) {
  ProjectPlan p;
  constexpr int step = 32 * RankTraits<R>::KS;
  p.tiles = (T + 63) / 64;
  int64_t kmax = 0;
  for (int m = 0; m < n; ++m) kmax = ks[m] > kmax ? ks[m] : kmax;
  int64_t chunk = ((kmax + step - 1) / step) * step;
  for (;;) {
    int64_t wgs = 0;
    bool capped = false;
    for (int m = 0; m < n; ++m) {
      const int64_t sp = (ks[m] + chunk - 1) / chunk;
      wgs += p.tiles * sp;
      capped = capped || sp >= 64;
    }
    if (wgs >= target_workgroups() || chunk <= step || capped) break;
    chunk = ((chunk / 2 + step - 1) / step) * step;
  }
  size_t off = 0;
  p.wg_begin[0] = 0;
  for (int m = 0; m < n; ++m) {
    p.splits[m] = (int)((ks[m] + chunk - 1) / chunk);
    p.kchunk[m] = chunk;
    p.wg_begin[m + 1] = p.wg_begin[m] + (int)(p.tiles * p.splits[m]);
    p.part_off[m] = off;
    if (p.splits[m] > 1) off += align256((size_t)p.splits[m] * T * R * sizeof(float));
  }
  p.ws_bytes = off;
  return p;
}

// Accumulate plan: one token split count for the whole batch, chosen so that
// the launch has enough workgroups.
struct AccumulatePlan {
  int64_t tiles[kMaxItems];
  int splits;
  int64_t tchunk;
  int wg_begin[kMaxItems + 1];
  size_t part_off[kMaxItems];
  size_t ws_bytes;
};

template <int R>
AccumulatePlan accumulate_plan(int n, const int64_t* ds, int64_t T) {
  AccumulatePlan p;
  constexpr int step = 32 * RankTraits<R>::KS;
  int64_t total = 0;
  for (int m = 0; m < n; ++m) {
    p.tiles[m] = (ds[m] + 63) / 64;
    total += p.tiles[m];
  }
  const int64_t ksteps = (T + step - 1) / step;
  int64_t want = (target_workgroups() + total - 1) / (total > 0 ? total : 1);
  if (want < 1) want = 1;
  if (want > ksteps) want = ksteps > 0 ? ksteps : 1;
  if (want > 64) want = 64;
  p.tchunk = ((ksteps + want - 1) / want) * step;
  p.splits = (int)((T + p.tchunk - 1) / (p.tchunk > 0 ? p.tchunk : 1));
  if (p.splits < 1) p.splits = 1;
  size_t off = 0;
  p.wg_begin[0] = 0;
  for (int m = 0; m < n; ++m) {
    p.wg_begin[m + 1] = p.wg_begin[m] + (int)(p.tiles[m] * p.splits);
    p.part_off[m] = off;
    if (p.splits > 1) off += align256((size_t)p.splits * ds[m] * R * sizeof(float));
  }
  p.ws_bytes = off;
  return p;
}

inline int finish_blocks(int64_t count) { return (int)((count / 4 + 255) / 256); }

template <int R>
rgc_status_t project_launch(int n, const uint16_t* const* Xs, const int64_t* ldxs, const int64_t* ks,
                            const uint16_t* const* Ps, uint16_t* const* XPs, int64_t T, void* ws, hipStream_t s) {
  const ProjectPlan p = project_plan<R>(n, ks, T);
  ProjectBatch pb = {};
  FinishBatch fb = {};
  pb.n = n;
  pb.T = T;
  pb.tiles = p.tiles;
  fb.fin_begin[0] = 0;
  for (int m = 0; m < n; ++m) {
    pb.X[m] = Xs[m];
    pb.ldx[m] = ldxs[m];
    pb.k[m] = ks[m];
    pb.P[m] = Ps[m];
    pb.XP[m] = XPs[m];
    pb.kchunk[m] = p.kchunk[m];
    pb.splits[m] = p.splits[m];
    pb.part[m] = p.splits[m] > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_off[m]) : nullptr;
    pb.wg_begin[m] = p.wg_begin[m];
    if (p.splits[m] > 1) {
      const int f = fb.n++;
      fb.part[f] = pb.part[m];
      fb.splits[f] = p.splits[m];
      fb.count[f] = T * R;
      fb.XP[f] = XPs[m];
      fb.fin_begin[f + 1] = fb.fin_begin[f] + finish_blocks(T * R);
    }
  }
  pb.wg_begin[n] = p.wg_begin[n];
  hipLaunchKernelGGL(project_kernel<R>, dim3(p.wg_begin[n]), dim3(64 * RankTraits<R>::NR * RankTraits<R>::KS), 0, s,
                     pb);
  if (fb.n > 0) hipLaunchKernelGGL(finish_splits_kernel<true>, dim3(fb.fin_begin[fb.n]), dim3(256), 0, s, fb);
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

template <int R>
rgc_status_t accumulate_launch(int n, const uint16_t* const* Ds, const int64_t* ldds, const int64_t* ds,
                               const uint16_t* const* XPs, float* const* Cs, int64_t T, void* ws, hipStream_t s) {
  const AccumulatePlan p = accumulate_plan<R>(n, ds, T);
  AccumulateBatch ab = {};
  FinishBatch fb = {};
  ab.n = n;
  ab.T = T;
  ab.tchunk = p.tchunk;
  ab.splits = p.splits;
  fb.fin_begin[0] = 0;
  for (int m = 0; m < n; ++m) {
    ab.D[m] = Ds[m];
    ab.ldd[m] = ldds[m];
    ab.d[m] = ds[m];
    ab.tiles[m] = p.tiles[m];
    ab.XP[m] = XPs[m];
    ab.C[m] = Cs[m];
    ab.part[m] = p.splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_off[m]) : nullptr;
    ab.wg_begin[m] = p.wg_begin[m];
    if (p.splits > 1) {
      fb.part[m] = ab.part[m];
      fb.splits[m] = p.splits;
      fb.count[m] = ds[m] * R;
      fb.C[m] = Cs[m];
      fb.fin_begin[m + 1] = fb.fin_begin[m] + finish_blocks(ds[m] * R);
    }
  }
  ab.wg_begin[n] = p.wg_begin[n];
  fb.n = p.splits > 1 ? n : 0;
  hipLaunchKernelGGL(accumulate_kernel<R>, dim3(p.wg_begin[n]), dim3(64 * RankTraits<R>::NR * RankTraits<R>::KS), 0,
                     s, ab);
  if (fb.n > 0) hipLaunchKernelGGL(finish_splits_kernel<false>, dim3(fb.fin_begin[fb.n]), dim3(256), 0, s, fb);
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

rgc_status_t check_project_item(const uint16_t* X, int64_t ldx, int64_t k, const uint16_t* P, const uint16_t* XP,
                                int64_t T, int64_t r) {
  if (k <= 0 || r > k || ldx < k) return RGC_ERR_SHAPE;
  if ((k % 8) != 0) return RGC_ERR_UNSUPPORTED;
  if (T == 0) return RGC_OK;
  if (!X || !P || !XP) return RGC_ERR_NULL;
  if (!aligned16(X) || !aligned16(P) || !aligned16(XP) || (ldx % 8) != 0) return RGC_ERR_ALIGN;
  return RGC_OK;
}

rgc_status_t check_accumulate_item(const uint16_t* D, int64_t ldd, int64_t d, const uint16_t* XP, const float* C,
                                   int64_t T) {
  if (d <= 0 || ldd < d) return RGC_ERR_SHAPE;
  if ((d % 8) != 0 || d > kMaxTiledDim) return RGC_ERR_UNSUPPORTED;
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
  size_t out = 0;
  if (!dispatch_rank(r, [&](auto rc) { out = project_plan<decltype(rc)::value>((int)n, ks, T).ws_bytes; })) return 0;
  return out;
}

extern "C" size_t rgc_accumulate_batch_workspace_size(int64_t n, const int64_t* ds, int64_t T, int64_t r) {
  if (n <= 0 || n > kMaxItems || !ds || T <= 0) return 0;
  for (int64_t m = 0; m < n; ++m)
    if (ds[m] <= 0) return 0;
  size_t out = 0;
  if (!dispatch_rank(r, [&](auto rc) { out = accumulate_plan<decltype(rc)::value>((int)n, ds, T).ws_bytes; })) return 0;
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
