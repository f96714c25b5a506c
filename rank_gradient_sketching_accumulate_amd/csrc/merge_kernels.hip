// Fused expand-and-merge (gfx950): W <- RNE_bf16(W - scale/sqrt(r) * U s).
// "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
// Sketches", section 2.1, equations 3 and 4 (W <- W - alpha eta U A) and
// Algorithm 1's trainer update.  No d x k update buffer exists: every W tile
// is read once, updated in fp32 and rounded to bf16 once.
//
// One kernel.  A workgroup owns a block of 64*NBW rows and a range of
// columns, which it walks in chunks of 16*CB columns.  Its waves (16*NBW rows
// each) load their U rows once, split them into bf16 hi/lo pairs held in
// registers for the whole range, and keep the W tiles of the next PD chunks
// in flight.  Whenever the walk enters a new 256-column sign block the
// workgroup regenerates that block's signs (Philox, rows 0 .. 32*NK-1, up to
// 512) into LDS and bit-transposes them so that one byte holds 8 rows of a
// column;
// every wave then expands its own MFMA sign operands from those bytes.
//
// MFMA orientation D = s^T U^T: M = 16 columns of W, N = 16 rows of W,
// K = 32 entries of r, so each lane ends with four consecutive columns of
// one W row.  W itself moves in row-contiguous pieces: each wave parks its
// fp32 update tile in a private LDS slice and reads it back as 16*CB/4 lanes
// x 4 columns per row, so one load or store instruction covers whole
// 128-byte rows (the MFMA layout would touch 16 rows per instruction).
#include "logra_device.h"
#include "logra_internal.h"

namespace logra {

__device__ __forceinline__ int xcd_linear_id_m(int bid, int grid) {
  return (bid & 7) * (grid >> 3) + (bid >> 3);
}

// Transpose an 8x8 bit matrix held as 64 bits: bit 8*a + b -> bit 8*b + a.
__device__ __forceinline__ uint64_t transpose8x8(uint64_t x) {
  uint64_t t;
  t = (x ^ (x >> 7)) & 0x00AA00AA00AA00AAull;
  x = x ^ t ^ (t << 7);
  t = (x ^ (x >> 14)) & 0x0000CCCC0000CCCCull;
  x = x ^ t ^ (t << 14);
  t = (x ^ (x >> 28)) & 0x00000000F0F0F0F0ull;
  x = x ^ t ^ (t << 28);
  return x;
}

// The work of one workgroup: tile `lin` (row block lin / n_cr, column range
// lin % n_cr) of the matrix p describes.
// GAUSS: the basis is the dense Gaussian one; its column-major bf16 hi/lo
// planes (p.Athi, p.Atlo) feed the MFMA A operand directly and each product
// takes three MFMAs (hi*hi, hi*lo, lo*hi; lo*lo is below 2^-32 relative).
// HL = 1 (sign basis only): U rounded once to bf16, one MFMA per product.
template <int NBW, int CB, int NK, int PD, bool GAUSS = false, int HL = 2>
__device__ __forceinline__ void merge_tile(const MergeParams& p, int lin) {
  static_assert(HL == 2 || !GAUSS, "the Gaussian basis keeps both halves of U");
  constexpr int STR = 9;        // dwords per row of row-major bits (8 + 1 pad)
  constexpr int CSTR = NK < 8 ? 9 : NK + 1;  // dwords per column of column-major bits (odd)
  constexpr int CW = 16 * CB;   // columns per chunk
  constexpr int KR = 32 * NK;   // sign rows generated (U entries >= r are zero)
  constexpr int RW = 16 * NBW;  // rows per wave
  constexpr int TSTR = CW + 4;  // floats per row of a wave's update tile (conflict-free)
  constexpr int LPR = CW / 4;   // lanes per row in the row-contiguous layout
  constexpr int RPI = 64 / LPR; // rows per W instruction
  constexpr int NI = RW / RPI;  // W instructions per chunk
  __shared__ uint32_t rowbits[KR * STR];
  __shared__ uint32_t colbits[256 * CSTR];
  __shared__ float tiles[4 * RW * TSTR];

  const int rb = lin / p.n_cr;
  const int cr = lin - rb * p.n_cr;
  if (rb >= p.n_rb) return;

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4, i = lane & 15;
  const int64_t rw = (int64_t)rb * 4 * RW + (int64_t)wave * RW;  // first row of this wave
  const int64_t c_begin = (int64_t)cr * p.cr_cols;
  const int64_t c_end = min(p.k, c_begin + p.cr_cols);
  const int nch = (int)((c_end - c_begin + CW - 1) / CW);

  // U rows of this wave: 8 consecutive entries per (K step, row block) and
  // lane.  Entries past r are zeroed; rows past d read as zero through the
  // descriptor.  Queued first, split after the first sign block is built.
  const __amdgpu_buffer_rsrc_t ru = make_rsrc(p.U, (uint32_t)(p.d * p.ldu * 4));
  // RowAdam folded in: the row factors of this wave's rows (rows past d read
  // as zero; without a factor buffer the descriptor is empty and 1 is used).
  const __amdgpu_buffer_rsrc_t rm = make_rsrc(p.rowmul, p.rowmul ? (uint32_t)(p.d * 4) : 0u);
  float fr[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const float f = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rm, (uint32_t)((rw + 16 * nb + i) * 4), 0, 0));
    fr[nb] = p.rowmul ? f : 1.0f;
  }
  float uraw[NK][NBW][8];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int j0 = 32 * kk + 8 * g;
      const uint32_t off = (uint32_t)(((rw + 16 * nb + i) * p.ldu + j0) * 4);
      if (j0 >= p.r) {
#pragma unroll
        for (int e = 0; e < 8; ++e) uraw[kk][nb][e] = 0.f;
      } else if (p.u_vec) {
        const f32x4 x0 = __builtin_bit_cast(f32x4, buf_load16(ru, off));
        const f32x4 x1 = __builtin_bit_cast(f32x4, buf_load16(ru, off + 16));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uraw[kk][nb][e] = x0[e];
          uraw[kk][nb][4 + e] = x1[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          uraw[kk][nb][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ru, off + 4 * e, 0, 0));
      }
      if (j0 < p.r && j0 + 8 > p.r) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (j0 + e >= p.r) uraw[kk][nb][e] = 0.f;
      }
      if (p.rowmul) {
#pragma unroll
        for (int e = 0; e < 8; ++e) uraw[kk][nb][e] *= fr[nb];
      }
    }

  // W tiles of the next PD chunks in the row-contiguous layout: the lane holds
  // row rw + RPI*q + lane/LPR, columns chunk + 4*(lane%LPR) .. +3.  Rows past
  // d read as zero and are never written; columns past k are never written.
  const int lrow = lane / LPR, lcol = 4 * (lane % LPR);
  const __amdgpu_buffer_rsrc_t rwb = make_rsrc(p.W, (uint32_t)(p.d * p.ldw * 2));
  const uint32_t wbase = (uint32_t)(((rw + lrow) * p.ldw + c_begin + lcol) * 2);
  const uint32_t wrowstep = (uint32_t)(RPI * p.ldw * 2);
  u32x2 wv[PD][NI];
  // Loads are unconditional (chunks past the range re-read the last one,
  // which is never used): a load under a branch would make the compiler's
  // wait counts wait for every load in flight.
  auto load_w = [&](int slot, int ch) {
    ch = min(ch, nch - 1);
    uint32_t off = wbase + (uint32_t)(ch * CW * 2);
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      wv[slot][q] = buf_load8(rwb, off);
      off += wrowstep;
    }
  };
#pragma unroll
  for (int q = 0; q < PD; ++q) load_w(q, q);

  // Signs of the 256-column block holding col0: rows 0 .. KR-1 into rowbits,
  // then the columns of this workgroup's range inside the block into colbits.
  auto build_block = [&](int64_t col0) {
    for (int row = threadIdx.x; row < KR; row += 256) {
      uint32_t w[8];
      philox_sign_block(p.seed, (uint32_t)row, (uint32_t)(col0 >> 8), w);
#pragma unroll
      for (int q = 0; q < 8; ++q) rowbits[row * STR + q] = w[q];
    }
    __syncthreads();  // also: every wave is done with the previous colbits
    const uint8_t* rbt = reinterpret_cast<const uint8_t*>(rowbits);
    uint8_t* cbt = reinterpret_cast<uint8_t*>(colbits);
    const int co_lo = (int)(col0 & 255) >> 3;
    const int64_t left = (c_end - col0 + 7) >> 3;
    const int co_hi = left < 32 - co_lo ? co_lo + (int)left : 32;
    const int nco = co_hi - co_lo;
    for (int task = threadIdx.x; task < nco * (KR >> 3); task += 256) {
      const int co = co_lo + task % nco;  // column octet
      const int ro = task / nco;          // row octet
      uint64_t x = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) x |= (uint64_t)rbt[(8 * ro + e) * STR * 4 + co] << (8 * e);
      x = transpose8x8(x);
#pragma unroll
      for (int b = 0; b < 8; ++b) cbt[(8 * co + b) * CSTR * 4 + ro] = (uint8_t)(x >> (8 * b));
    }
    __syncthreads();
  };

  if constexpr (!GAUSS) {
    if (nch > 0) build_block(c_begin);
  }

  u32x4 uh[NK][NBW], ul[NK][HL == 2 ? NBW : 1];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float h0 = uraw[kk][nb][2 * q], h1 = uraw[kk][nb][2 * q + 1];
        if constexpr (HL == 2) {
          uint32_t h, l;
          split_hi_lo2(h0, h1, h, l);
          uh[kk][nb][q] = h;
          ul[kk][nb][q] = l;
        } else {
          uh[kk][nb][q] = pack_bf16x2(h0, h1);
        }
      }

  const SignExpander ex(g);
  const float ns = -p.scale_eff;
  float* tile = tiles + wave * RW * TSTR;
  for (int ch0 = 0; ch0 < nch; ch0 += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      const int ch = ch0 + u;
      if (ch < nch) {
        const int64_t col0 = c_begin + (int64_t)ch * CW;
        if constexpr (!GAUSS) {
          if (ch > 0 && (col0 & 255) == 0) build_block(col0);
        }
        const int cib = (int)(col0 & 255);

        f32x4 acc[CB][NBW];
#pragma unroll
        for (int mb = 0; mb < CB; ++mb)
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
#pragma unroll
          for (int mb = 0; mb < CB; ++mb) {
            if constexpr (GAUSS) {
              const int64_t o = (col0 + 16 * mb + i) * (int64_t)KR + 32 * kk + 8 * g;
              const u32x4 ah = *reinterpret_cast<const u32x4*>(p.Athi + o);
              const u32x4 al = *reinterpret_cast<const u32x4*>(p.Atlo + o);
#pragma unroll
              for (int nb = 0; nb < NBW; ++nb) {
                acc[mb][nb] = mfma_16x16x32(ah, uh[kk][nb], acc[mb][nb]);
                acc[mb][nb] = mfma_16x16x32(ah, ul[kk][nb], acc[mb][nb]);
                acc[mb][nb] = mfma_16x16x32(al, uh[kk][nb], acc[mb][nb]);
              }
            } else {
              const u32x4 a = ex(colbits[(cib + 16 * mb + i) * CSTR + kk]);
#pragma unroll
              for (int nb = 0; nb < NBW; ++nb) {
                acc[mb][nb] = mfma_16x16x32(a, uh[kk][nb], acc[mb][nb]);
                if constexpr (HL == 2) acc[mb][nb] = mfma_16x16x32(a, ul[kk][nb], acc[mb][nb]);
              }
            }
          }

        // Park the tile (row 16*nb + i, columns 16*mb + 4g ..), then read it
        // back row-contiguously.  The slice is private to this wave, whose
        // LDS accesses complete in order.
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
          for (int mb = 0; mb < CB; ++mb)
            *reinterpret_cast<f32x4*>(tile + (16 * nb + i) * TSTR + 16 * mb + 4 * g) = acc[mb][nb];
        __builtin_amdgcn_wave_barrier();
        const int64_t col = col0 + lcol;
#pragma unroll
        for (int q = 0; q < NI; ++q) {
          const f32x4 a = *reinterpret_cast<const f32x4*>(tile + (RPI * q + lrow) * TSTR + lcol);
          const int64_t row = rw + RPI * q + lrow;
          if (row >= p.d || col >= p.k) continue;
          const u32x2 v = wv[u][q];
          const float w0 = __uint_as_float(v[0] << 16), w1 = __uint_as_float(v[0] & 0xffff0000u);
          const float w2 = __uint_as_float(v[1] << 16), w3 = __uint_as_float(v[1] & 0xffff0000u);
          const uint32_t p01 = pack_bf16x2(__fmaf_rn(ns, a[0], w0), __fmaf_rn(ns, a[1], w1));
          const uint32_t p23 = pack_bf16x2(__fmaf_rn(ns, a[2], w2), __fmaf_rn(ns, a[3], w3));
          uint16_t* dst = p.W + row * p.ldw + col;
          if (col + 4 <= p.k) {
            *reinterpret_cast<u32x2*>(dst) = u32x2{p01, p23};
          } else {
            const uint32_t h[4] = {p01 & 0xffffu, p01 >> 16, p23 & 0xffffu, p23 >> 16};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (col + e < p.k) dst[e] = (uint16_t)h[e];
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
      load_w(u, ch + PD);
    }
  }
}

template <int NBW, int CB, int NK, int PD, bool GAUSS = false, int HL = 2>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void merge_kernel(MergeParams p) {
  merge_tile<NBW, CB, NK, PD, GAUSS, HL>(p, xcd_linear_id_m(blockIdx.x, gridDim.x));
}

// Several matrices in one launch (same rank, so the same tiling): the
// logical workgroup ids are dealt to the matrices by the prefix table
// `start`; each matrix's tiles are exactly those of its own launch.
template <int NBW, int CB, int NK, int PD, int HL = 2>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void merge_group_kernel(MergeGroup grp) {
  const int lin = xcd_linear_id_m(blockIdx.x, gridDim.x);
  int j = 0;
  while (j + 1 < grp.count && lin >= grp.start[j + 1]) ++j;
  if (lin >= grp.start[grp.count]) return;
  merge_tile<NBW, CB, NK, PD, false, HL>(grp.p[j], lin - grp.start[j]);
}

namespace {
size_t align_up_m(size_t x, size_t a) { return (x + a - 1) / a * a; }
}  // namespace

MergePlan plan_merge(int64_t d, int64_t k, int r, bool gauss) {
  MergePlan pl{};
  pl.NK = r <= 32 ? 1 : (r <= 64 ? 2 : (r <= 128 ? 4 : (r <= 256 ? 8 : 16)));
  // Tile per wave and chunk (two waves fit per SIMD): one 16-row block x 64
  // columns up to r = 128 with about 2048 workgroups; at r = 256, where the
  // U operands and sign expansion cost more, two 16-row blocks (each expanded
  // sign operand feeds both) with longer column ranges.  Measured
  // with GPU-only timing over layers from 1536 x 1536 to 17408 x 5120.
  // Above r = 256 (NK = 16) one 16-row block x 64 columns: the U operands
  // alone take 128 registers.
  // The Gaussian basis runs the default tiling only.
  int NBW = pl.NK == 8 ? 2 : 1, CB = 4;
  if (!gauss) {
    NBW = env_int("LOGRA_MERGE_NBW", NBW) == 2 ? 2 : 1;
    CB = env_int("LOGRA_MERGE_CB", CB) == 4 ? 4 : 8;
  }
  if (NBW == 2 && CB == 8 && pl.NK >= 4) CB = 4;  // would not fit two waves per SIMD
  if (pl.NK == 16) NBW = 1, CB = 4;
  pl.NBW = NBW;
  pl.CB = CB;
  pl.n_rb = (int)((d + 64 * NBW - 1) / (64 * NBW));
  const int64_t CW = 16 * CB;
  const int64_t chunks = (k + CW - 1) / CW;
  int64_t target = env_int("LOGRA_MERGE_WGS", 0);
  int64_t n_cr;
  if (target <= 0 && pl.NK >= 8) {
    // Above rank 128 a workgroup's column range is long and two workgroups
    // fit per CU (512 at once): choose the number of ranges that minimises
    // rounds x (chunks per range + 3), the 3 standing for a range's fixed
    // cost (U rows, the first sign block); ties go to more workgroups.
    // Against about 1024 workgroups: 27B attention 53 -> 44 us, 7B down
    // 107 -> 87 us, 7B q 37 -> 30 us, 7B up 109 -> 94 us, 27B up 138 -> 128 us.
    int64_t best_cost = -1, best_g = 0;
    n_cr = 1;
    for (int64_t c = 1; c <= chunks; ++c) {
      const int64_t per = (chunks + c - 1) / c;
      const int64_t used = (chunks + per - 1) / per;
      const int64_t g = pl.n_rb * used;
      const int64_t cost = ((g + 511) / 512) * (per + 3);
      if (best_cost < 0 || cost < best_cost || (cost == best_cost && g > best_g)) {
        best_cost = cost;
        best_g = g;
        n_cr = used;
      }
    }
  } else {
    // Otherwise ranges as long as possible while about `target` workgroups
    // remain (2048 up to rank 128).
    if (target <= 0) target = 2048;
    n_cr = (target + pl.n_rb - 1) / pl.n_rb;
  }
  if (n_cr > chunks) n_cr = chunks;
  if (n_cr < 1) n_cr = 1;
  pl.cr_cols = ((chunks + n_cr - 1) / n_cr) * CW;
  pl.n_cr = (int)((k + pl.cr_cols - 1) / pl.cr_cols);
  (void)r;
  return pl;
}

bool merge_launch(const MergePlan& pl, const MergeParams& mp, hipStream_t s) {
  const int grid = (int)align_up_m((size_t)pl.n_cr * pl.n_rb, 8);
  if (mp.Athi) {
#define LOGRA_MERGE_GAUSS(nbw, cb, nk)                                                          \
    if (pl.NBW == nbw && pl.CB == cb && pl.NK == nk) {                                          \
      hipLaunchKernelGGL((merge_kernel<nbw, cb, nk, 2, true>), dim3(grid), dim3(256), 0, s, mp); \
      return true;                                                                              \
    }
    LOGRA_MERGE_GAUSS(1, 4, 1) LOGRA_MERGE_GAUSS(1, 4, 2) LOGRA_MERGE_GAUSS(1, 4, 4)
    LOGRA_MERGE_GAUSS(2, 4, 8) LOGRA_MERGE_GAUSS(1, 4, 16)
#undef LOGRA_MERGE_GAUSS
    return false;
  }
#define LOGRA_MERGE(nbw, cb, nk)                                                                     \
  if (pl.NBW == nbw && pl.CB == cb && pl.NK == nk) {                                                 \
    if (mp.hi_only)                                                                                  \
      hipLaunchKernelGGL((merge_kernel<nbw, cb, nk, 2, false, 1>), dim3(grid), dim3(256), 0, s, mp); \
    else                                                                                             \
      hipLaunchKernelGGL((merge_kernel<nbw, cb, nk, 2>), dim3(grid), dim3(256), 0, s, mp);           \
    return true;                                                                                     \
  }
  LOGRA_MERGE(1, 4, 1) LOGRA_MERGE(1, 8, 1) LOGRA_MERGE(2, 4, 1) LOGRA_MERGE(2, 8, 1)
  LOGRA_MERGE(1, 4, 2) LOGRA_MERGE(1, 8, 2) LOGRA_MERGE(2, 4, 2) LOGRA_MERGE(2, 8, 2)
  LOGRA_MERGE(1, 4, 4) LOGRA_MERGE(1, 8, 4) LOGRA_MERGE(2, 4, 4)
  LOGRA_MERGE(1, 4, 8) LOGRA_MERGE(1, 8, 8) LOGRA_MERGE(2, 4, 8)
  LOGRA_MERGE(1, 4, 16)
#undef LOGRA_MERGE
  return false;
}

}  // namespace logra

namespace logra {

bool merge_group_launch(const MergePlan& pl, const MergeGroup& g, hipStream_t s) {
  const int grid = (int)align_up_m((size_t)g.start[g.count], 8);
#define LOGRA_MERGE_G(nbw, cb, nk)                                                                \
  if (pl.NBW == nbw && pl.CB == cb && pl.NK == nk) {                                              \
    if (g.p[0].hi_only)                                                                           \
      hipLaunchKernelGGL((merge_group_kernel<nbw, cb, nk, 2, 1>), dim3(grid), dim3(256), 0, s, g); \
    else                                                                                          \
      hipLaunchKernelGGL((merge_group_kernel<nbw, cb, nk, 2>), dim3(grid), dim3(256), 0, s, g);    \
    return true;                                                                                  \
  }
  LOGRA_MERGE_G(1, 4, 1) LOGRA_MERGE_G(1, 8, 1) LOGRA_MERGE_G(2, 4, 1) LOGRA_MERGE_G(2, 8, 1)
  LOGRA_MERGE_G(1, 4, 2) LOGRA_MERGE_G(1, 8, 2) LOGRA_MERGE_G(2, 4, 2) LOGRA_MERGE_G(2, 8, 2)
  LOGRA_MERGE_G(1, 4, 4) LOGRA_MERGE_G(1, 8, 4) LOGRA_MERGE_G(2, 4, 4)
  LOGRA_MERGE_G(1, 4, 8) LOGRA_MERGE_G(1, 8, 8) LOGRA_MERGE_G(2, 4, 8)
  LOGRA_MERGE_G(1, 4, 16)
#undef LOGRA_MERGE_G
  return false;
}

}  // namespace logra
