// Device helpers shared by the gfx950 kernels of the sketch library: the
// global-to-LDS copies and transposing LDS reads of the staged contractions,
// the Philox4x32-10 counter generator, bf16 bit helpers and the bf16 MFMA
// wrapper.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rgc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Staging through LDS.
//
// dma_16b_*: each lane copies the 16 bytes at base + voff (global) into LDS;
// lane l's bytes land at lds_addr + 16*l (lds_addr is wave-uniform and goes
// to M0). The copy does not pass through VGPRs. It is issued from inline asm
// on purpose: the compiler, seeing the builtin, conservatively waits for
// every outstanding copy before any LDS read, which would serialize a
// multi-stage pipeline. Completion is therefore tracked by hand: a copy
// counts in the wave's vector-memory counter until its bytes are in LDS, and
// these counters retire loads in issue order, so wait_vmcnt<N>() returns once
// all but the N most recent of the wave's loads are done. Other waves see the
// bytes after a workgroup barrier that follows that wait.
//
// The leading s_nop 4 supplies wait states that the compiler cannot insert
// into inline asm: a vector memory instruction that reads an SGPR as its base
// needs five wait states after a VALU instruction wrote that SGPR (the
// compiler reloads spilled SGPRs with v_readlane right before the asm), and
// a copy into LDS needs one after M0 was written (the compiler writes M0 for
// the "{m0}" operand right before the asm). Without them the copy may use a
// stale base address.
#define RGC_LDS __attribute__((address_space(3)))
__device__ __forceinline__ void dma_16b_stream(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "{m0}"(lds_addr) : "memory");
}
__device__ __forceinline__ void dma_16b_cached(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_addr) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier for LDS handoff: the wave's own LDS reads are complete
// before it arrives (so a stage read in the previous step may be refilled
// after the barrier). No memory fence beyond that: the copies it orders are
// waited for explicitly with wait_vmcnt.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Transposing LDS read of 16-bit elements (ds_read_b64_tr_b16). Within each
// group of 16 lanes, lane c supplies the address of an 8-byte chunk (four
// elements); lane i receives, as its element j (j = 0..3), element i % 4 of
// the chunk addressed by lane 4j + i / 4 of its group. With the chunks of a
// 4 x 16 block laid out row-major (chunk 4j + q = row j, columns 4q..4q+3),
// lane i therefore gets column i of rows 0..3: the MFMA operand layout for a
// K-major (token-major) matrix. Returned as two dwords, element 0 in the low
// half of dword 0.
__device__ __forceinline__ u32x2v_t lds_read_tr16(const RGC_LDS char* p) {
  typedef short i16x4_t __attribute__((ext_vector_type(4)));
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((RGC_LDS i16x4_t*)p);
  return __builtin_bit_cast(u32x2v_t, v);
}

// Pins a wave-uniform value to scalar registers.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ const uint16_t* uniform_ptr(const uint16_t* p) {
  return reinterpret_cast<const uint16_t*>(uniform_u64(reinterpret_cast<uint64_t>(p)));
}
__device__ __forceinline__ int64_t uniform_i64(int64_t v) { return (int64_t)uniform_u64((uint64_t)v); }

// Index of the calling wave within its workgroup, as a wave-uniform (scalar)
// value, so that branches on it and on values derived from it are scalar
// branches rather than exec-masked ones.
__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

struct u32x4 {
  uint32_t x, y, z, w;
};

// Stream tags (counter word 2): projection signs, Gaussian draws, rounding bits.
constexpr uint32_t kTagRademacher = 1;
constexpr uint32_t kTagGaussian = 2;
constexpr uint32_t kTagRounding = 3;

// Philox4x32-10 (Salmon et al., SC'11): ten rounds, each multiplying counter
// words 0 and 2 by the two round constants (full 64-bit products), mixing the
// halves with words 1 and 3 and the key, and bumping the key by the Weyl
// increments afterwards. The key is wave-uniform, so its schedule lives in
// scalar registers.
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    u32x4 n;
    n.x = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c.y, k0, 0x96);  // three-way xor
    n.y = (uint32_t)p1;
    n.z = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c.w, k1, 0x96);
    n.w = (uint32_t)p0;
    c = n;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16, round to nearest even; NaN becomes a quiet NaN keeping its
// sign and upper payload ((bits >> 16) | 0x40). This is what the conversion
// instruction (v_cvt_pk_bf16_f32) does in the default float mode: compared on
// MI355X with the integer form (b + 0x7FFF + lsb) >> 16, NaN aside, over all
// 2^32 fp32 bit patterns, with no difference; the pair form converts two in
// one instruction.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Stochastic rounding fp32 -> bf16 with 16 random bits: the random integer is
// added to the dropped low half, so the kept half rounds up with probability
// (low half) / 2^16. NaN becomes a quiet NaN keeping its sign. Infinities need
// no case of their own: their low half is zero, so the sum never carries.
// sr_keep returns the 32-bit word whose high half is the result.
// (Selects, not branches: both words are formed for every input.)
__device__ __forceinline__ uint32_t sr_keep(float f, uint32_t r16) {
  const uint32_t b = __float_as_uint(f);
  return __builtin_isnan(f) ? (b | 0x00400000u) : b + r16;
}
__device__ __forceinline__ uint32_t f32_to_bf16_sr(float f, uint32_t r16) { return sr_keep(f, r16) >> 16; }
// Two stochastically rounded values packed in a dword (v0 in the low half),
// with the random halves of one word: low half for v0, high half for v1.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_sr(float v0, float v1, uint32_t rword) {
  // byte select: result bytes 0, 1 = bytes 2, 3 of the first word, bytes 2, 3 = bytes 2, 3 of the second
  return __builtin_amdgcn_perm(sr_keep(v1, rword >> 16), sr_keep(v0, rword & 0xFFFFu), 0x07060302u);
}

// Two bf16 packed in a dword, element 0 in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(uint32_t lo, uint32_t hi) { return (lo & 0xFFFFu) | (hi << 16); }

// D = A B + C for one 16x16 output tile with K = 32 (bf16 in, fp32 out).
// Lane l supplies A row (l % 16) and B column (l % 16), each with the eight
// consecutive K values 8*(l/16) .. 8*(l/16)+7 packed as four bf16 pairs;
// it receives D rows 4*(l/16) .. 4*(l/16)+3 of column (l % 16).
__device__ __forceinline__ f32x4_t mfma_16x16x32(const uint32_t (&a)[4], const uint32_t (&b)[4], f32x4_t c) {
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  u4v av = {a[0], a[1], a[2], a[3]};
  u4v bv = {b[0], b[1], b[2], b[3]};
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv),
                                                 c, 0, 0, 0);
}

// Wave-wide sum of a double (64 lanes) with cross-lane shuffles.
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
// The same for a float. A xor butterfly pairs the same two partial sums in
// both lanes of every exchange, so all 64 lanes end with the same bits.
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// R (4 or 8) consecutive bf16 values at p (8- or 16-byte aligned) as floats.
template <int R>
__device__ __forceinline__ void load_bf16_row(const uint16_t* p, float (&out)[R]) {
  static_assert(R == 4 || R == 8, "small rank");
  uint32_t w[R / 2];
  if constexpr (R == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x; w[1] = v.y;
  } else {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  }
#pragma unroll
  for (int i = 0; i < R / 2; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

}  // namespace rgc
