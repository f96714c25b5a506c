// Device helpers shared by the LoGRA kernels (gfx950 / CDNA4 only).
//
// Method: "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
// Sketches", section 2.1 (equations 2-4).  The sign generator is this
// library's own fixed choice (the paper asks only for independent random
// signs regenerated from a seed, section 2.1 and section 2.2 "Memory and
// synchronization"); it is Philox4x64-10 as defined by Salmon, Moraes, Dror
// and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace logra {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

// One wavefront is 64 lanes on CDNA.
constexpr int kWave = 64;
// Signs per Philox4x64 call (four 64-bit output words).
constexpr int kSignBlock = 256;

// ---------------------------------------------------------------------------
// Philox4x64-10 (SC'11, section 5): two 64x64->128 multiplies per round, key
// bumped by the Weyl constants between rounds.
// ---------------------------------------------------------------------------
constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;

// Full 128-bit product of a and b from four 32x32->64 partial products; each
// maps to one v_mad_u64_u32 with the carry folded into its addend.
__device__ __forceinline__ void mul_wide64(uint64_t a, uint64_t b, uint64_t& hi, uint64_t& lo) {
  const uint32_t a0 = (uint32_t)a, a1 = (uint32_t)(a >> 32);
  const uint32_t b0 = (uint32_t)b, b1 = (uint32_t)(b >> 32);
  const uint64_t p00 = (uint64_t)a0 * b0;
  const uint64_t p01 = (uint64_t)a0 * b1 + (p00 >> 32);
  const uint64_t p10 = (uint64_t)a1 * b0 + (uint32_t)p01;
  hi = (uint64_t)a1 * b1 + (p01 >> 32) + (p10 >> 32);
  lo = (p10 << 32) | (uint32_t)p00;
}

// One Philox4x64-10 block for counter (c0, c1, c2, 0) and key (seed, 0), as
// eight 32-bit halves: w[2q] is the low half of output word q.
__device__ __forceinline__ void philox_block(uint64_t seed, uint64_t c0, uint64_t c1, uint64_t c2, uint32_t w[8]) {
  uint64_t x0 = c0, x1 = c1, x2 = c2, x3 = 0;
  uint64_t k0 = seed, k1 = 0;
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    uint64_t hi0, lo0, hi1, lo1;
    mul_wide64(kPhiloxM0, x0, hi0, lo0);
    mul_wide64(kPhiloxM1, x2, hi1, lo1);
    const uint64_t n0 = hi1 ^ x1 ^ k0;
    const uint64_t n2 = hi0 ^ x3 ^ k1;
    x0 = n0;
    x1 = lo1;
    x2 = n2;
    x3 = lo0;
  }
  w[0] = (uint32_t)x0; w[1] = (uint32_t)(x0 >> 32);
  w[2] = (uint32_t)x1; w[3] = (uint32_t)(x1 >> 32);
  w[4] = (uint32_t)x2; w[5] = (uint32_t)(x2 >> 32);
  w[6] = (uint32_t)x3; w[7] = (uint32_t)(x3 >> 32);
}

// 256 sign bits of sign row `row`, columns [256*cblk, 256*cblk + 256):
// Philox4x64-10(counter = (cblk, row, 0, 0), key = (seed, 0)).  Word q of the
// output holds columns 64q .. 64q+63, least significant bit first; w[2q] is
// the low half of word q.  Bit 1 means sign -1.
__device__ __forceinline__ void philox_sign_block(uint64_t seed, uint32_t row, uint32_t cblk,
                                                  uint32_t w[8]) {
  philox_block(seed, cblk, row, 0, w);
}

// Eight N(0, 1) values of the Gaussian basis, row `row`, columns
// 8*blk .. 8*blk+7: the block Philox4x64-10(counter = (blk, row, 1, 0), key =
// (seed, 0)) gives four Box-Muller pairs (Box and Muller, 1958), pair p from
// halves 2p and 2p+1 as 24-bit uniforms u1 = ((h >> 8) + 1) / 2^24 (in
// (0, 1], never 0) and u2 = (h >> 8) / 2^24; z[2p] = R cos(2 pi u2),
// z[2p+1] = R sin(2 pi u2) with R = sqrt(-2 ln u1).  Both uniforms are exact
// in fp32; sincospi takes 2 u2 exactly.
__device__ __forceinline__ void gauss_block(uint64_t seed, uint32_t row, uint64_t blk, float z[8]) {
  uint32_t w[8];
  philox_block(seed, blk, row, 1, w);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float u1 = (float)((w[2 * p] >> 8) + 1u) * 0x1p-24f;
    const float t = (float)(w[2 * p + 1] >> 8) * 0x1p-23f;  // 2 u2
    const float R = sqrtf(-2.0f * logf(u1));
    float sn, cs;
    sincospif(t, &sn, &cs);
    z[2 * p] = R * cs;
    z[2 * p + 1] = R * sn;
  }
}

// Eight sign bits (bit e -> element e, 1 = negative) to eight bf16 values
// +-1.0 packed two per dword, element 2q in the low half of dword q.  bf16
// +1.0 is 0x3F80; the sign bit is bit 15 of each half.  The byte is copied
// into both 16-bit halves, then one packed 16-bit shift per dword moves bit
// 2q to bit 15 of the low half and bit 2q+1 to bit 15 of the high half.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_shl16(uint32_t x, unsigned short lo, unsigned short hi) {
  const u16x2 v = __builtin_bit_cast(u16x2, x);
  const u16x2 s = {lo, hi};
  return __builtin_bit_cast(uint32_t, (u16x2)(v << s));
}
__device__ __forceinline__ u32x4 signs_to_bf16x8(uint32_t b) {
  const uint32_t d = b * 0x00010001u;  // b < 256: byte in both halves
  u32x4 o;
  o[0] = (pk_shl16(d, 15, 14) & 0x80008000u) | 0x3F803F80u;
  o[1] = (pk_shl16(d, 13, 12) & 0x80008000u) | 0x3F803F80u;
  o[2] = (pk_shl16(d, 11, 10) & 0x80008000u) | 0x3F803F80u;
  o[3] = (pk_shl16(d, 9, 8) & 0x80008000u) | 0x3F803F80u;
  return o;
}

// The same expansion for lane group g straight from a dword holding four
// sign bytes (byte g is this lane's): one v_perm copies byte g into both
// 16-bit halves, then per output dword one packed shift and one and-or with
// the +1.0 pattern kept in a register.
struct SignExpander {
  uint32_t sel;  // v_perm selector: byte g -> bytes 0 and 2, zero elsewhere
  uint32_t one;  // 0x3F803F80 (two bf16 +1.0), held in a VGPR
  __device__ __forceinline__ explicit SignExpander(int g) {
    sel = 0x0C000C00u | ((uint32_t)g << 16) | (uint32_t)g;
    asm volatile("v_mov_b32 %0, 0x3f803f80" : "=v"(one));
  }
  __device__ __forceinline__ u32x4 operator()(uint32_t dw) const {
    const uint32_t d = __builtin_amdgcn_perm(0u, dw, sel);
    u32x4 o;
    o[0] = (pk_shl16(d, 15, 14) & 0x80008000u) | one;
    o[1] = (pk_shl16(d, 13, 12) & 0x80008000u) | one;
    o[2] = (pk_shl16(d, 11, 10) & 0x80008000u) | one;
    o[3] = (pk_shl16(d, 9, 8) & 0x80008000u) | one;
    return o;
  }
};

// ---------------------------------------------------------------------------
// Raw buffer access with the agent-scope coherence bit (sc1): used for the
// partial sums one workgroup hands to another inside a kernel, so that no
// L2 write-back or invalidate of the whole cache is needed.
// ---------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int kSc1 = 16;  // cache-policy bit that sets sc1 on gfx950
__device__ __forceinline__ void store16_agent(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kSc1);
}
__device__ __forceinline__ u32x4 load16_agent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1);
}
// Plain raw-buffer loads: SGPR base + 32-bit byte offset; offsets past the
// descriptor's size read as zero (used for rows beyond the matrix).
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
// s_waitcnt vmcnt(0): every vector memory access of this wave has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------------------
// bf16 <-> fp32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round to nearest, ties to even (v_cvt_pk_bf16_f32; NaN stays NaN).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// x = hi + lo + O(2^-17 |x|) with hi, lo bf16: the pair carries about 16
// significant bits, so an MFMA over (hi, lo) reproduces fp32 operands to well
// below the bf16 rounding error of a single operand.  Two values per call:
// hi and lo come back packed (value a in the low half).
__device__ __forceinline__ void split_hi_lo2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  const float ah = __uint_as_float(hi << 16), bh = __uint_as_float(hi & 0xffff0000u);
  lo = pack_bf16x2(a - ah, b - bh);
}
__device__ __forceinline__ void split_hi_lo(float x, uint32_t& hi, uint32_t& lo) {
  uint32_t h, l;
  split_hi_lo2(x, 0.f, h, l);
  hi = h & 0xffffu;
  lo = l & 0xffffu;
}

// ---------------------------------------------------------------------------
// MFMA 16x16x32 bf16 -> fp32 (CDNA4).  Lane l = 16*g + i supplies
//   A[i][k] and B[k][i] for the eight k in lane group g,
// and receives D[4g + e][i], e = 0..3.  The kernels below always give A and B
// the same (g, element) -> k assignment, so the reduction is right whatever
// order the hardware walks k in.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// MFMAs with the accumulators pinned to AGPRs.  Kernels that keep 256
// accumulator registers per lane (one wave per SIMD) need them in the AGPR
// half of the register file; with the builtin the compiler keeps loop-carried
// accumulators in VGPRs and copies every MFMA result across (thousands of
// v_accvgpr moves and spills).  Inline asm with "a" constraints keeps them in
// AGPRs, but the compiler's hazard recognizer does not look inside it, so
// every block states its own wait states:
//   * it opens with s_nop 2 (three wait states), more than the two a VALU
//     write of a VGPR needs before an MFMA reads it as SrcA/B/C (the
//     operands here are often written by the VALU just before);
//   * MFMAs inside a block write distinct accumulators, and an accumulator
//     is read as SrcC only by a later MFMA of the same shape (exact overlap,
//     which the hardware forwards);
//   * before any non-MFMA instruction reads the accumulators, call
//     mfma_drain(): it waits out the longest MFMA-write -> VALU/memory-read
//     distance, and mfma_touch() orders each later read after that wait.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void mfma4_b(f32x4& c0, f32x4& c1, f32x4& c2, f32x4& c3, const u32x4& a0,
                                        const u32x4& a1, const u32x4& a2, const u32x4& a3, const u32x4& b) {
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %8, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %5, %8, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %6, %8, %2\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %7, %8, %3"
      : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(b));
}
// Eight accumulators sharing one B operand: c_q += a_q * b.
// Two MFMAs sharing the B operand (see mfma4_b).
__device__ __forceinline__ void mfma2_b(f32x4& c0, f32x4& c1, const u32x4& a0, const u32x4& a1, const u32x4& b) {
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %2, %4, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %3, %4, %1"
      : "+a"(c0), "+a"(c1)
      : "v"(a0), "v"(a1), "v"(b));
}

__device__ __forceinline__ void mfma8_b(f32x4 (&c)[8], const u32x4 (&a)[8], const u32x4& b) {
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %8, %16, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %9, %16, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %10, %16, %2\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %11, %16, %3\n\t"
      "v_mfma_f32_16x16x32_bf16 %4, %12, %16, %4\n\t"
      "v_mfma_f32_16x16x32_bf16 %5, %13, %16, %5\n\t"
      "v_mfma_f32_16x16x32_bf16 %6, %14, %16, %6\n\t"
      "v_mfma_f32_16x16x32_bf16 %7, %15, %16, %7"
      : "+a"(c[0]), "+a"(c[1]), "+a"(c[2]), "+a"(c[3]), "+a"(c[4]), "+a"(c[5]), "+a"(c[6]), "+a"(c[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(b));
}
// Four accumulators, each multiplied by its own A operand and two B operands
// in turn (the high and low bf16 halves of one fp32 operand): c_q += a_q*bh,
// then c_q += a_q*bl; the four bh products come first, so dependent MFMAs are
// four apart.
__device__ __forceinline__ void mfma4_hl(f32x4& c0, f32x4& c1, f32x4& c2, f32x4& c3, const u32x4& a0,
                                         const u32x4& a1, const u32x4& a2, const u32x4& a3, const u32x4& bh,
                                         const u32x4& bl) {
  asm volatile(
      "s_nop 2\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %8, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %5, %8, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %6, %8, %2\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %7, %8, %3\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %9, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %5, %9, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %6, %9, %2\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %7, %9, %3"
      : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3)
      : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(bh), "v"(bl));
}
// Wait states after the last MFMA before its results are read by anything
// else (more than the 19 a 16-pass MFMA write needs before a VALU read).
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }
// Orders later reads of c after mfma_drain() (volatile asm keeps its order).
__device__ __forceinline__ void mfma_touch(f32x4& c) { asm volatile("" : "+a"(c)); }

}  // namespace logra
