// Normalized update with stochastic rounding [page "Randomized Gradient
// Compression", section "How it works"]:
//
//   W <- SR_bf16(W - s * H),  H = C P^T,  s = tau * ||W||_F / ||H||_F
//
// H is never written to memory. It is rebuilt 64 columns at a time on MFMA
// (M = columns of W from rows of P, N = rows of W from rows of C, K = r), with
// C split into a bf16 high part and a bf16 remainder so that H carries ~16
// bits of C's mantissa. The page rebuilds H 128 rows at a time; here a
// workgroup rebuilds 128 rows (64 for r > 64) x 64 columns per step (the
// result does not depend on the tile shape).
//
// One batch (e.g. all projections of a block) takes three launches:
//   norms:  every workgroup streams its share of one matrix's W, rebuilds the
//           same H tiles and writes one (sum w^2, sum h^2) pair (fp64 per
//           lane, fixed-order reductions across lanes and waves);
//   scale:  one workgroup per matrix sums that matrix's pairs in workgroup
//           order and forms s = fp32(tau ||W|| / ||H||), or the skip flag when
//           ||H|| is zero or not finite or s is not finite;
//   update: every workgroup reads its matrix's s, rebuilds its H tiles again
//           (same code, same order), forms v = fp32(w - fp32(s h)) and rounds
//           stochastically with 16 bits per element from Philox4x32-10 keyed
//           on (seed, row, column).
// Each matrix gets one workgroup per twelve tiles (its own shape alone
// decides, so a matrix gets the same bits alone or in a batch), and each
// workgroup serves one matrix. Within a workgroup the W and P tiles two steps
// ahead are loaded while the current one is processed (P goes through
// registers into LDS, where the four waves share it).
//
// Lane layout of a tile: M-tile t row m stands for column
// jb + 16*(m/4) + 4*t + (m%4), which gives lane (g = lane/16, n = lane%16) the
// 16 consecutive columns jb + 16g .. +15 of its row in each N-tile, i.e. two
// 16-byte loads of W and two Philox calls (8 columns each).
#include "rgc_internal.hpp"

namespace rgc {

enum ApplyMode { kModeNorms = 0, kModeUpdate = 1, kModeReconstruct = 2 };

constexpr int kApplyCols = 64;     // columns per tile
constexpr int kApplyWaves = 4;
constexpr int kApplyMaxItems = 16;
constexpr int64_t kMaxApplyDim = int64_t(1) << 30;  // d and k

template <int R>
struct ApplyTraits {
  static constexpr int KQ = (R + 31) / 32;              // K-steps of 32 over r
  static constexpr int NTW = R <= 64 ? 2 : 1;           // 16-row N-tiles per wave
  static constexpr int RW = 16 * NTW;                   // rows per wave
  static constexpr int ROWS = kApplyWaves * RW;         // rows per workgroup tile
  static constexpr int RP = 32 * KQ + 8;                // LDS row pitch of the P tile (bf16)
  static constexpr int PCHUNKS = kApplyCols * R / 8;    // 16-byte chunks of a P tile
  static constexpr int PCPT = (PCHUNKS + 255) / 256;    // chunks per thread
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
};

struct ApplyBatch {
  int n;
  float tau;
  int wbase[kApplyMaxItems + 1];  // workgroups [wbase[m], wbase[m+1]) serve item m
  ApplyItem it[kApplyMaxItems];
  double* partials;               // 2 per workgroup of the norms sweep
  float* scale;                   // per item: s, flag
  float* H;                       // reconstruct target (test hook)
};

__device__ __forceinline__ int apply_item_of(const ApplyBatch& b, int w) {
  int m = 0;
  while (m + 1 < b.n && w >= b.wbase[m + 1]) ++m;
  return m;
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
        const uint32_t h0 = f32_to_bf16_rne(v[2 * p]), h1 = f32_to_bf16_rne(v[2 * p + 1]);
        const uint32_t l0 = f32_to_bf16_rne(v[2 * p] - bf16_bits_to_f32(h0));
        const uint32_t l1 = f32_to_bf16_rne(v[2 * p + 1] - bf16_bits_to_f32(h1));
        op.hi[nt][q][p] = pack_bf16x2(h0, h1);
        op.lo[nt][q][p] = pack_bf16x2(l0, l1);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The sweeps are software pipelines over the workgroup's tiles: each tile's
// W rows (ROWS x 64 bf16) and P rows (64 x R bf16) are copied from memory
// straight into an LDS stage (1 KB copies that bypass the VGPRs, spread over
// the four waves), S - 1 tiles ahead of the tile being processed.
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
// Two workgroups per compute unit with three stages each: the update's
// per-tile arithmetic (the H rebuild on MFMA, Philox, rounding) is heavy
// enough that a second workgroup's waves overlapping it pay more than deeper
// staging (measured on the Qwen3-1.7B-shaped block). At r > 128 the P rows
// make a stage too large for two, so one workgroup takes up to six.

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
  static constexpr int NV_LO = NI / 4, NV_HI = (NI + 3) / 4;
  static_assert(S >= 3 && S * STAGE <= LDS_MAX, "LDS");
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
template <int R, int MODE>
__global__ __launch_bounds__(256, R > 128 ? 1 : 2) void apply_kernel(ApplyBatch b) {  // ApplyShape::PER_CU
  using Tr = ApplyTraits<R>;
  using Sh = ApplyShape<R, MODE>;
  constexpr int S = Sh::S;
  __shared__ __attribute__((aligned(1024))) char smem[S * Sh::STAGE];
  __shared__ double red[2][kApplyWaves];
  const int lane = threadIdx.x & 63, wave = wave_index();
  const int n = lane & 15, g = lane >> 4;
  const int w = blockIdx.x;
  const int m = apply_item_of(b, w);
  const ApplyItem& it = b.it[m];
  const int64_t wl = w - b.wbase[m], gm = b.wbase[m + 1] - b.wbase[m];
  const int64_t u0 = uniform_i64(wl * it.units / gm), u1 = uniform_i64((wl + 1) * it.units / gm);

  float s = 0.f;
  if constexpr (MODE == kModeUpdate) {
    s = b.scale[2 * m];
    if (b.scale[2 * m + 1] != 0.f) return;  // zero or non-finite step: W stays as it is
  }

  double sw = 0.0, sh = 0.0;
  RowOperand<R> rop;
  int rop_row = -1;  // first row of the loaded row operand
  const int d = (int)it.d, k = (int)it.k, ctiles = (int)it.ctiles;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(RGC_LDS char*)smem;
  const bool more = wave < Sh::NI % 4;
  auto origin = [&](int64_t u, int& row0, int& jb, int& wrow, int& wcol) {
    row0 = (int)(u / ctiles) * Tr::ROWS;
    jb = (int)(u % ctiles) * kApplyCols;
    wrow = row0 + Tr::ROWS <= d ? row0 : (d >= Tr::ROWS ? d - Tr::ROWS : 0);
    wcol = jb + kApplyCols <= k ? jb : (k >= kApplyCols ? k - kApplyCols : 0);
  };

  // ---- copies: per-lane byte offsets from the tile origin (fixed)
  uint32_t voff[Sh::NV_HI];
#pragma unroll
  for (int v = 0; v < Sh::NV_HI; ++v) {
    const int c = wave + 4 * v;
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
  uint32_t lslot = 0;
  auto issue = [&]() {
    int row0, jb, wrow, wcol;
    origin(lu, row0, jb, wrow, wcol);
    const uint16_t* Wb = uniform_ptr(it.W + (int64_t)wrow * it.ldw + wcol);
    const uint16_t* Pb = uniform_ptr(it.P + (int64_t)wcol * R);
    const uint32_t st = lds0 + lslot * Sh::STAGE;
    static_for<0, Sh::NV_HI>([&](auto vc) {
      constexpr int v = decltype(vc)::value;
      const int c = wave + 4 * v;  // a W copy if c < WC, a P copy if WC <= c < NI
      if constexpr (4 * v + 3 < Sh::WC) {
        dma_16b_stream(Wb, voff[v], st + 1024 * c);
      } else if constexpr (4 * v >= Sh::WC && 4 * v + 3 < Sh::NI) {
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
    origin(u, row0, jb, wrow, wcol);
    if (wrow != rop_row) {  // wave-uniform: new rows
      load_row_operand<R>(it.C, it.d, wrow + Tr::RW * wave, lane, rop);
      rop_row = wrow;
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
          if constexpr (MODE == kModeNorms) {
            double pw = 0.0, ph = 0.0;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const double w0 = (double)bf16_bits_to_f32(wd[p] & 0xFFFFu);
              const double w1 = (double)bf16_bits_to_f32(wd[p] >> 16);
              const double h0 = (double)hv[2 * p], h1 = (double)hv[2 * p + 1];
              pw += w0 * w0 + w1 * w1;
              ph += h0 * h0 + h1 * h1;
            }
            sw += inside ? pw : 0.0;
            sh += inside ? ph : 0.0;
          } else {
            uint32_t rw[4];
            rounding_words(it.seed, i, jj >> 3, rw);
            uint32_t out[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const float w0 = bf16_bits_to_f32(wd[p] & 0xFFFFu), w1 = bf16_bits_to_f32(wd[p] >> 16);
              const float sh0 = s * hv[2 * p], sh1 = s * hv[2 * p + 1];
              const float v0 = w0 - sh0, v1 = w1 - sh1;
              out[p] = pack_bf16x2(f32_to_bf16_sr(v0, rw[p] & 0xFFFFu), f32_to_bf16_sr(v1, rw[p] >> 16));
            }
            if (inside)
              *reinterpret_cast<uint4*>(it.W + (int64_t)i * it.ldw + jj) = make_uint4(out[0], out[1], out[2], out[3]);
          }
        }
      }
    }
  }
  wait_vmcnt<0>();

  if constexpr (MODE == kModeNorms) {
    sw = wave_sum(sw);
    sh = wave_sum(sh);
    if (lane == 0) {
      red[0][wave] = sw;
      red[1][wave] = sh;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      b.partials[2 * w] = ((red[0][0] + red[0][1]) + red[0][2]) + red[0][3];
      b.partials[2 * w + 1] = ((red[1][0] + red[1][1]) + red[1][2]) + red[1][3];
    }
  }
}

// Per item: fixed-order sum of its norms partials (thread t holds partials
// t, t+256, ... in order; then a butterfly within each wave and the waves in
// order), and s = fp32(tau * ||W|| / ||H||); flag = 1 when ||H|| is zero or
// not finite or s is not finite (then s = 0).
__global__ __launch_bounds__(256) void apply_scale_kernel(ApplyBatch b) {
  __shared__ double red[2][4];
  const int m = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int w0 = b.wbase[m], w1 = b.wbase[m + 1];
  double aw = 0.0, ah = 0.0;
  for (int w = w0 + (int)threadIdx.x; w < w1; w += 256) {
    aw += b.partials[2 * w];
    ah += b.partials[2 * w + 1];
  }
  aw = wave_sum(aw);
  ah = wave_sum(ah);
  if (lane == 0) {
    red[0][wave] = aw;
    red[1][wave] = ah;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  const double nw = sqrt(((red[0][0] + red[0][1]) + red[0][2]) + red[0][3]);
  const double nh = sqrt(((red[1][0] + red[1][1]) + red[1][2]) + red[1][3]);
  float s = 0.f, flag = 0.f;
  if (!(nh > 0.0) || !isfinite(nh)) {
    flag = 1.f;
  } else {
    s = (float)((double)b.tau * nw / nh);
    if (!isfinite(s)) {
      s = 0.f;
      flag = 1.f;
    }
  }
  b.scale[2 * m] = s;
  b.scale[2 * m + 1] = flag;
  float* st = b.it[m].stats;
  if (st) {
    st[0] = (float)nw;
    st[1] = (float)nh;
    st[2] = s;
    st[3] = flag;
  }
}

// ---------------------------------------------------------------------------
// Test hooks: the rounding stream and the Philox generator alone.
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

// Workgroups per matrix: one per kApplyUnitsPerWG tiles, a function of the
// matrix's own shape only, so that a matrix gets the same partition (and so
// the same norm sums and bits) alone or in any batch. Eight tiles of 128 x
// 64 give the Qwen3-1.7B-shaped block 768 workgroups (two resident per
// compute unit); measured faster than 4, 6, 10, 16 or 24 tiles.
constexpr int64_t kApplyUnitsPerWG = 8;

template <int R>
void apply_plan(ApplyBatch& b, int n, const int64_t* ds, const int64_t* ks) {
  using Tr = ApplyTraits<R>;
  const int forced = env_int("RGC_APPLY_UNITS", 0);
  const int64_t per = forced > 0 ? forced : kApplyUnitsPerWG;
  b.wbase[0] = 0;
  for (int m = 0; m < n; ++m) {
    b.it[m].ctiles = (ks[m] + kApplyCols - 1) / kApplyCols;
    b.it[m].units = (ds[m] + Tr::ROWS - 1) / Tr::ROWS * b.it[m].ctiles;
    b.wbase[m + 1] = b.wbase[m] + (int)((b.it[m].units + per - 1) / per);
  }
  b.n = n;
}

size_t apply_ws_bytes(int workgroups) {
  return (size_t)((2 * workgroups * sizeof(double) + 255) / 256 * 256) + 2 * kApplyMaxItems * sizeof(float);
}

template <int R>
size_t apply_ws_for(int n, const int64_t* ds, const int64_t* ks) {
  ApplyBatch b = {};
  apply_plan<R>(b, n, ds, ks);
  return apply_ws_bytes(b.wbase[n]);
}

template <int R>
rgc_status_t apply_launch(int n, uint16_t* const* Ws, const int64_t* ldws, const float* const* Cs,
                          const uint16_t* const* Ps, const int64_t* ds, const int64_t* ks, float tau,
                          const uint64_t* seeds, float* const* stats, void* ws, hipStream_t st) {
  ApplyBatch b = {};
  apply_plan<R>(b, n, ds, ks);
  b.tau = tau;
  for (int m = 0; m < n; ++m) {
    b.it[m].W = Ws[m];
    b.it[m].ldw = ldws[m];
    b.it[m].C = Cs[m];
    b.it[m].P = Ps[m];
    b.it[m].d = ds[m];
    b.it[m].k = ks[m];
    b.it[m].seed = seeds[m];
    b.it[m].stats = stats ? stats[m] : nullptr;
  }
  const int G = b.wbase[n];
  b.partials = static_cast<double*>(ws);
  b.scale = reinterpret_cast<float*>(static_cast<char*>(ws) + (apply_ws_bytes(G) - 2 * kApplyMaxItems * sizeof(float)));
  hipLaunchKernelGGL((apply_kernel<R, kModeNorms>), dim3((unsigned)G), dim3(256), 0, st, b);
  hipLaunchKernelGGL(apply_scale_kernel, dim3((unsigned)n), dim3(256), 0, st, b);
  hipLaunchKernelGGL((apply_kernel<R, kModeUpdate>), dim3((unsigned)G), dim3(256), 0, st, b);
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
  hipLaunchKernelGGL((apply_kernel<R, kModeReconstruct>), dim3((unsigned)b.wbase[1]), dim3(256), 0, st, b);
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}

rgc_status_t check_apply_shape(int64_t ldw, int64_t d, int64_t k, int64_t r) {
  return (d <= 0 || k <= 0 || r > k || ldw < k) ? RGC_ERR_SHAPE : RGC_OK;
}

rgc_status_t check_apply_item(const uint16_t* W, int64_t ldw, const float* C, const uint16_t* P, int64_t d,
                              int64_t k, const float* stats) {
  // element indices are 32-bit inside the kernels, and so are the byte
  // offsets of a tile's rows from its origin
  if ((d % 8) != 0 || (k % 8) != 0 || d > kMaxApplyDim || k > kMaxApplyDim || ldw > kMaxLeadingDim)
    return RGC_ERR_UNSUPPORTED;
  if (!W || !C || !P) return RGC_ERR_NULL;
  if (!aligned16(W) || !aligned16(C) || !aligned16(P) || (ldw % 8) != 0) return RGC_ERR_ALIGN;
  if (stats && !aligned_to(stats, 4)) return RGC_ERR_ALIGN;
  return RGC_OK;
}

}  // namespace
}  // namespace rgc

using namespace rgc;

extern "C" size_t rgc_apply_batch_workspace_size(int64_t n, const int64_t* ds, const int64_t* ks, int64_t r) {
  if (n <= 0 || n > kApplyMaxItems || !ds || !ks || !rank_supported(r)) return 0;
  for (int64_t m = 0; m < n; ++m)
    if (ds[m] <= 0 || ks[m] <= 0) return 0;
  size_t out = 0;
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
  dispatch_rank(r, [&](auto rc) {
    st = apply_launch<decltype(rc)::value>((int)n, Ws, ldws, Cs, Ps, ds, ks, tau, seeds, stats, ws,
                                           static_cast<hipStream_t>(stream));
  });
  return st;
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

extern "C" rgc_status_t rgc_test_reconstruct(const float* C, const uint16_t* P, float* H, int64_t d, int64_t k,
                                             int64_t r, void* stream) {
  if (d <= 0 || k <= 0 || r <= 0 || r > k) return RGC_ERR_SHAPE;
  if (!rank_supported(r) || (d % 8) != 0 || (k % 8) != 0) return RGC_ERR_UNSUPPORTED;
  if (!C || !P || !H) return RGC_ERR_NULL;
  if (!aligned16(C) || !aligned16(P) || !aligned16(H)) return RGC_ERR_ALIGN;
  rgc_status_t st = RGC_OK;
  dispatch_rank(r, [&](auto rc) {
    st = reconstruct_launch<decltype(rc)::value>(C, P, H, d, k, static_cast<hipStream_t>(stream));
  });
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

extern "C" rgc_status_t rgc_test_philox(uint64_t seed, int64_t n, const uint32_t* ctr, uint32_t* out, void* stream) {
  if (n < 0) return RGC_ERR_SHAPE;
  if (n == 0) return RGC_OK;
  if (!ctr || !out) return RGC_ERR_NULL;
  if (!aligned_to(ctr, 4) || !aligned_to(out, 4)) return RGC_ERR_ALIGN;
  hipLaunchKernelGGL(philox_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     seed, n, ctr, out);
  return hipGetLastError() == hipSuccess ? RGC_OK : RGC_ERR_HIP;
}
