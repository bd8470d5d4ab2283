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
// Work is split over K (k for project, tokens for accumulate) first across the
// waves of a workgroup (summed through LDS) and then across workgroups: each
// workgroup writes its partial tile to the workspace and the last one to
// finish a tile (device-scope counter) adds the partials in split order, so
// results are bit-reproducible whatever the arrival order. Both reductions
// are spread over all waves (each owns some of the output's N-tiles), so no
// single wave serializes the tail of the kernel.
#include "rgc_internal.hpp"

namespace rgc {

// ---------------------------------------------------------------------------
// Shared pieces
// ---------------------------------------------------------------------------

// Loads the M-side operand (rank columns) for one K-step of 32 rows starting
// at `krow0` from a row-major bf16 matrix `src` (row stride `ld`, `nrows`
// valid rows). The lane (m = lane % 16, g = lane / 16) reads rows
// krow0 + 8g + j, j = 0..7, columns rbase + q*GW + CPL*m .. +CPL-1 for each
// column group q, then transposes them into MT operands.
template <int R>
__device__ __forceinline__ void load_rank_operand(const uint16_t* __restrict__ src, int64_t ld, int64_t krow0,
                                                  int64_t nrows, int rbase, int lane,
                                                  uint32_t (&aop)[RankTraits<R>::MT][4]) {
  using Tr = RankTraits<R>;
  constexpr int CPL = Tr::CPL;
  constexpr int W = (CPL + 1) / 2;
  const int m = lane & 15, g = lane >> 4;
#pragma unroll
  for (int q = 0; q < Tr::NG; ++q) {
    uint32_t rows[8][W];
    const int col = rbase + q * Tr::GW + CPL * m;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t kr = krow0 + 8 * g + j;
      const uint16_t* p = src + kr * ld + col;
      const bool ok = kr < nrows;
      if constexpr (CPL == 4) {
        uint2 v = ok ? *reinterpret_cast<const uint2*>(p) : make_uint2(0u, 0u);
        rows[j][0] = v.x;
        rows[j][1] = v.y;
      } else if constexpr (CPL == 2) {
        rows[j][0] = ok ? *reinterpret_cast<const uint32_t*>(p) : 0u;
      } else {
        rows[j][0] = ok ? (uint32_t)(*p) : 0u;
      }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) transpose_8xcpl<CPL>(rows, c, aop[q * CPL + c]);
  }
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

// Cross-workgroup split reduction. Every wave stores the N-tiles it owns to
// the workspace (per lane, contiguous); the last workgroup of the tile to
// arrive sums all splits in split order, each wave for its own N-tiles, with
// the loads of several splits in flight at once. Returns true in the
// workgroup that holds the final sums (always, with a single split).
template <int R, int KS>
__device__ __forceinline__ bool combine_splits(f32x4_t (&acc)[RankTraits<R>::MT][4], float* __restrict__ partials,
                                               uint32_t* __restrict__ counter, int tile, int split, int splits,
                                               int rw, int ks, int lane) {
  using Tr = RankTraits<R>;
  constexpr int MT = Tr::MT;
  if (splits == 1) return true;
  auto slot = [&](int s, int nt) {
    return partials + ((((int64_t)tile * splits + s) * Tr::NR + rw) * 4 + nt) * 64 * (MT * 4) + lane * (MT * 4);
  };
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    if (!owns_ntile<KS>(nt, ks)) continue;
    float4* dst = reinterpret_cast<float4*>(slot(split, nt));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) dst[mt] = make_float4(acc[mt][nt][0], acc[mt][nt][1], acc[mt][nt][2], acc[mt][nt][3]);
  }
  if (!arrive_last(counter + tile, (uint32_t)(splits - 1))) return false;
  constexpr int BATCH = 4;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    if (!owns_ntile<KS>(nt, ks)) continue;
    f32x4_t sum[MT];
#pragma unroll 1
    for (int s0 = 0; s0 < splits; s0 += BATCH) {
      float4 v[BATCH][MT];
#pragma unroll
      for (int b = 0; b < BATCH; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          v[b][mt] = (s0 + b < splits) ? reinterpret_cast<const float4*>(slot(s0 + b, nt))[mt] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int b = 0; b < BATCH; ++b) {
        if (s0 + b >= splits) break;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const f32x4_t x = {v[b][mt].x, v[b][mt].y, v[b][mt].z, v[b][mt].w};
          sum[mt] = (s0 + b == 0) ? x : sum[mt] + x;
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt][nt] = sum[mt];
  }
  if (threadIdx.x == 0) counter[tile] = 0u;  // leave the counter zeroed for the next call
  return true;
}

// ---------------------------------------------------------------------------
// project: XP = bf16(X P)
// Grid (ceil(T / 64), splits). A workgroup computes 64 tokens x all r over one
// k-chunk; its NR x KS waves take r-slices x interleaved K-steps.
// ---------------------------------------------------------------------------
template <int R>
__global__ __launch_bounds__(256) void project_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                      const uint16_t* __restrict__ P, uint16_t* __restrict__ XP,
                                                      int64_t T, int64_t k, int64_t kchunk, int splits,
                                                      float* __restrict__ partials, uint32_t* __restrict__ counters) {
  using Tr = RankTraits<R>;
  constexpr int KS = Tr::KS;
  __shared__ float lds[KS > 1 ? KS * Tr::NR * Tr::MT * 16 * 64 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rw = wave % Tr::NR, ks = wave / Tr::NR;
  const int rbase = rw * Tr::RPW;
  const int n = lane & 15, g = lane >> 4;
  const int64_t tbase = (int64_t)blockIdx.x * 64;
  const int split = blockIdx.y;
  const int64_t kbeg = split * kchunk;
  const int64_t kend = kbeg + kchunk < k ? kbeg + kchunk : k;

  f32x4_t acc[Tr::MT][4];
#pragma unroll
  for (int mt = 0; mt < Tr::MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = kbeg + 32 * ks; k0 < kend; k0 += 32 * KS) {
    uint32_t aop[Tr::MT][4];
    load_rank_operand<R>(P, R, k0, kend, rbase, lane, aop);
    uint32_t bop[4][4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t t = tbase + 16 * nt + n;
      const int64_t kc = k0 + 8 * g;
      u32x4v_t v = {0u, 0u, 0u, 0u};
      if (t < T && kc < kend) v = load_stream_16b(X + t * ldx + kc);
      bop[nt][0] = v.x;
      bop[nt][1] = v.y;
      bop[nt][2] = v.z;
      bop[nt][3] = v.w;
    }
#pragma unroll
    for (int mt = 0; mt < Tr::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_16x16x32(aop[mt], bop[nt], acc[mt][nt]);
  }

  reduce_waves<R, KS>(acc, lds, rw, ks, lane);
  if (!combine_splits<R, KS>(acc, partials, counters, blockIdx.x, split, splits, rw, ks, lane)) return;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t t = tbase + 16 * nt + n;
    if (!owns_ntile<KS>(nt, ks) || t >= T) continue;
#pragma unroll
    for (int q = 0; q < Tr::NG; ++q) {
      float run[4 * Tr::CPL];
      gather_rank_run<R>(acc, q, nt, run);
      uint16_t* dst = XP + t * R + rbase + q * Tr::GW + 4 * Tr::CPL * g;
      if constexpr (Tr::CPL == 4) {
        uint4 a, b;
        a.x = pack_bf16x2(f32_to_bf16_rne(run[0]), f32_to_bf16_rne(run[1]));
        a.y = pack_bf16x2(f32_to_bf16_rne(run[2]), f32_to_bf16_rne(run[3]));
        a.z = pack_bf16x2(f32_to_bf16_rne(run[4]), f32_to_bf16_rne(run[5]));
        a.w = pack_bf16x2(f32_to_bf16_rne(run[6]), f32_to_bf16_rne(run[7]));
        b.x = pack_bf16x2(f32_to_bf16_rne(run[8]), f32_to_bf16_rne(run[9]));
        b.y = pack_bf16x2(f32_to_bf16_rne(run[10]), f32_to_bf16_rne(run[11]));
        b.z = pack_bf16x2(f32_to_bf16_rne(run[12]), f32_to_bf16_rne(run[13]));
        b.w = pack_bf16x2(f32_to_bf16_rne(run[14]), f32_to_bf16_rne(run[15]));
        reinterpret_cast<uint4*>(dst)[0] = a;
        reinterpret_cast<uint4*>(dst)[1] = b;
      } else if constexpr (Tr::CPL == 2) {
        uint4 a;
        a.x = pack_bf16x2(f32_to_bf16_rne(run[0]), f32_to_bf16_rne(run[1]));
        a.y = pack_bf16x2(f32_to_bf16_rne(run[2]), f32_to_bf16_rne(run[3]));
        a.z = pack_bf16x2(f32_to_bf16_rne(run[4]), f32_to_bf16_rne(run[5]));
        a.w = pack_bf16x2(f32_to_bf16_rne(run[6]), f32_to_bf16_rne(run[7]));
        reinterpret_cast<uint4*>(dst)[0] = a;
      } else {
        uint2 a;
        a.x = pack_bf16x2(f32_to_bf16_rne(run[0]), f32_to_bf16_rne(run[1]));
        a.y = pack_bf16x2(f32_to_bf16_rne(run[2]), f32_to_bf16_rne(run[3]));
        reinterpret_cast<uint2*>(dst)[0] = a;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// accumulate: C += D^T XP
// Grid (ceil(d / 64), splits). A workgroup computes 64 output rows (d) x all r
// over one token chunk; its NR x KS waves take r-slices x interleaved
// 32-token steps. D is token-major, so its operand is also transposed in
// registers: lane (n, g) reads 4 consecutive d for eight tokens, and N-tile
// c column n is d = dbase + 4n + c.
// ---------------------------------------------------------------------------
template <int R>
__global__ __launch_bounds__(256) void accumulate_kernel(const uint16_t* __restrict__ Dm, int64_t ldd,
                                                         const uint16_t* __restrict__ XPm, float* __restrict__ C,
                                                         int64_t T, int64_t d, int64_t tchunk, int splits,
                                                         float* __restrict__ partials,
                                                         uint32_t* __restrict__ counters) {
  using Tr = RankTraits<R>;
  constexpr int KS = Tr::KS;
  __shared__ float lds[KS > 1 ? KS * Tr::NR * Tr::MT * 16 * 64 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rw = wave % Tr::NR, ks = wave / Tr::NR;
  const int rbase = rw * Tr::RPW;
  const int n = lane & 15, g = lane >> 4;
  const int64_t dbase = (int64_t)blockIdx.x * 64;
  const int split = blockIdx.y;
  const int64_t tbeg = split * tchunk;
  const int64_t tend = tbeg + tchunk < T ? tbeg + tchunk : T;
  const bool dvalid = dbase + 4 * n < d;  // d % 4 == 0: a lane's 4 columns are all in or all out

  f32x4_t acc[Tr::MT][4];
#pragma unroll
  for (int mt = 0; mt < Tr::MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int64_t t0 = tbeg + 32 * ks; t0 < tend; t0 += 32 * KS) {
    uint32_t drows[8][2];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t t = t0 + 8 * g + j;
      u32x2v_t v = {0u, 0u};
      if (t < tend && dvalid) v = load_stream_8b(Dm + t * ldd + dbase + 4 * n);
      drows[j][0] = v.x;
      drows[j][1] = v.y;
    }
    uint32_t aop[Tr::MT][4];
    load_rank_operand<R>(XPm, R, t0, tend, rbase, lane, aop);
    uint32_t bop[4][4];
#pragma unroll
    for (int c = 0; c < 4; ++c) transpose_8xcpl<4>(drows, c, bop[c]);
#pragma unroll
    for (int mt = 0; mt < Tr::MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_16x16x32(aop[mt], bop[nt], acc[mt][nt]);
  }

  reduce_waves<R, KS>(acc, lds, rw, ks, lane);
  if (!combine_splits<R, KS>(acc, partials, counters, blockIdx.x, split, splits, rw, ks, lane)) return;
  if (!dvalid) return;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    if (!owns_ntile<KS>(nt, ks)) continue;
    const int64_t drow = dbase + 4 * n + nt;
#pragma unroll
    for (int q = 0; q < Tr::NG; ++q) {
      float run[4 * Tr::CPL];
      gather_rank_run<R>(acc, q, nt, run);
      float* dst = C + drow * R + rbase + q * Tr::GW + 4 * Tr::CPL * g;
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
// Host side
// ---------------------------------------------------------------------------
namespace {

// Number of workgroups that keeps all 256 compute units streaming.
int target_workgroups() { return env_int("RGC_TARGET_WGS", 256); }

struct SplitPlan {
  int64_t tiles;
  int splits;
  int64_t chunk;  // K elements per split (multiple of 32 * KS)
};

SplitPlan plan_splits(int64_t tiles, int64_t kdim, int ks) {
  SplitPlan p;
  p.tiles = tiles;
  const int64_t step = 32LL * ks;
  const int64_t ksteps = (kdim + step - 1) / step;
  int64_t want = (target_workgroups() + tiles - 1) / (tiles > 0 ? tiles : 1);
  if (want < 1) want = 1;
  if (want > ksteps) want = ksteps > 0 ? ksteps : 1;
  if (want > 64) want = 64;
  p.chunk = ((ksteps + want - 1) / want) * step;
  p.splits = (int)((kdim + p.chunk - 1) / (p.chunk > 0 ? p.chunk : 1));
  if (p.splits < 1) p.splits = 1;
  return p;
}

template <int R>
SplitPlan project_plan(int64_t T, int64_t k) { return plan_splits((T + 63) / 64, k, RankTraits<R>::KS); }
template <int R>
SplitPlan accumulate_plan(int64_t T, int64_t d) { return plan_splits((d + 63) / 64, T, RankTraits<R>::KS); }

template <int R>
size_t project_ws(int64_t T, int64_t k) {
  SplitPlan p = project_plan<R>(T, k);
  if (p.splits <= 1) return 0;
  return kCounterBytes + (size_t)p.tiles * p.splits * 64 * R * sizeof(float);
}
template <int R>
size_t accumulate_ws(int64_t T, int64_t d) {
  SplitPlan p = accumulate_plan<R>(T, d);
  if (p.splits <= 1) return 0;
  return kCounterBytes + (size_t)p.tiles * p.splits * 64 * R * sizeof(float);
}

template <int R>
rgc_status_t project_launch(const uint16_t* X, int64_t ldx, const uint16_t* P, uint16_t* XP, int64_t T, int64_t k,
                            void* ws, hipStream_t s) {
  SplitPlan p = project_plan<R>(T, k);
  float* partials = nullptr;
  uint32_t* counters = nullptr;
  if (p.splits > 1) {
    counters = static_cast<uint32_t*>(ws);
    partials = reinterpret_cast<float*>(static_cast<char*>(ws) + kCounterBytes);
  }
  dim3 grid((unsigned)p.tiles, (unsigned)p.splits);
  hipLaunchKernelGGL(project_kernel<R>, grid, dim3(64 * RankTraits<R>::NR * RankTraits<R>::KS), 0, s, X, ldx, P, XP,
                     T, k, p.chunk, p.splits, partials, counters);
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

template <int R>
rgc_status_t accumulate_launch(const uint16_t* D, int64_t ldd, const uint16_t* XP, float* C, int64_t T, int64_t d,
                               void* ws, hipStream_t s) {
  SplitPlan p = accumulate_plan<R>(T, d);
  float* partials = nullptr;
  uint32_t* counters = nullptr;
  if (p.splits > 1) {
    counters = static_cast<uint32_t*>(ws);
    partials = reinterpret_cast<float*>(static_cast<char*>(ws) + kCounterBytes);
  }
  dim3 grid((unsigned)p.tiles, (unsigned)p.splits);
  hipLaunchKernelGGL(accumulate_kernel<R>, grid, dim3(64 * RankTraits<R>::NR * RankTraits<R>::KS), 0, s, D, ldd, XP,
                     C, T, d, p.chunk, p.splits, partials, counters);
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

}  // namespace
}  // namespace rgc

using namespace rgc;

extern "C" size_t rgc_project_workspace_size(int64_t T, int64_t k, int64_t r) {
  if (T <= 0 || k <= 0) return 0;
  size_t out = 0;
  if (!dispatch_rank(r, [&](auto rc) { out = project_ws<decltype(rc)::value>(T, k); })) return 0;
  return out;
}

extern "C" size_t rgc_accumulate_workspace_size(int64_t T, int64_t d, int64_t r) {
  if (T <= 0 || d <= 0) return 0;
  size_t out = 0;
  if (!dispatch_rank(r, [&](auto rc) { out = accumulate_ws<decltype(rc)::value>(T, d); })) return 0;
  return out;
}

extern "C" rgc_status_t rgc_project(const uint16_t* X, int64_t ldx, const uint16_t* P, uint16_t* XP, int64_t T,
                                    int64_t k, int64_t r, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k <= 0 || r <= 0) return RGC_ERR_SHAPE;
  if (r > k || ldx < k) return RGC_ERR_SHAPE;
  if (!rank_supported(r) || (k % 8) != 0 || T > kMaxTiledDim) return RGC_ERR_UNSUPPORTED;
  if (T == 0) return RGC_OK;
  if (!X || !P || !XP) return RGC_ERR_NULL;
  if (!aligned16(X) || !aligned16(P) || !aligned16(XP) || (ldx % 8) != 0) return RGC_ERR_ALIGN;
  const size_t need = rgc_project_workspace_size(T, k, r);
  if (need > 0 && (!ws || ws_bytes < need)) return RGC_ERR_WORKSPACE;
  if (need > 0 && !aligned_to(ws, 256)) return RGC_ERR_ALIGN;
  rgc_status_t st = RGC_OK;
  dispatch_rank(r, [&](auto rc) {
    st = project_launch<decltype(rc)::value>(X, ldx, P, XP, T, k, ws, static_cast<hipStream_t>(stream));
  });
  return st;
}

extern "C" rgc_status_t rgc_accumulate(const uint16_t* D, int64_t ldd, const uint16_t* XP, float* C, int64_t T,
                                       int64_t d, int64_t r, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || d <= 0 || r <= 0) return RGC_ERR_SHAPE;
  if (ldd < d) return RGC_ERR_SHAPE;
  if (!rank_supported(r) || (d % 8) != 0 || d > kMaxTiledDim) return RGC_ERR_UNSUPPORTED;
  if (T == 0) return RGC_OK;
  if (!D || !XP || !C) return RGC_ERR_NULL;
  if (!aligned16(D) || !aligned16(XP) || !aligned16(C) || (ldd % 8) != 0) return RGC_ERR_ALIGN;
  const size_t need = rgc_accumulate_workspace_size(T, d, r);
  if (need > 0 && (!ws || ws_bytes < need)) return RGC_ERR_WORKSPACE;
  if (need > 0 && !aligned_to(ws, 256)) return RGC_ERR_ALIGN;
  rgc_status_t st = RGC_OK;
  dispatch_rank(r, [&](auto rc) {
    st = accumulate_launch<decltype(rc)::value>(D, ldd, XP, C, T, d, ws, static_cast<hipStream_t>(stream));
  });
  return st;
}
