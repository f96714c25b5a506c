// Fused expand-and-merge (gfx950): W <- RNE_bf16(W - scale/sqrt(r) * U s).
// "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
// Sketches", section 2.1, equations 3 and 4 (W <- W - alpha eta U A) and
// Algorithm 1's trainer update.  No d x k update buffer exists: every W tile
// is read once, updated in fp32 and rounded to bf16 once.
//
//   usplit_kernel  U (fp32) -> a bf16 hi/lo pair in MFMA operand order (Uk).
//   merge_kernel   per 256-column block: regenerate the signs of that block
//                  (Philox, LDS), transpose them so a byte holds 8 rows of one
//                  column, MFMA over r with U hi and U lo, update W in place.
//
// MFMA orientation D = s^T U^T: M = 16 columns of W, N = 16 rows of W,
// K = 32 entries of r, so each lane ends with four consecutive columns of
// one W row (one 8-byte access).
//
// Uk layout (rows of U padded to 16, r padded to KR = 32*ceil(r/32)):
//   elem(row, j) = (((row/16)*(KR/32) + j/32)*64 + ((j%32)/8)*16 + row%16)*8 + j%8
#include "logra_device.h"
#include "logra_internal.h"

namespace logra {

__device__ __forceinline__ int xcd_linear_id_m(int bid, int grid) {
  return (bid & 7) * (grid >> 3) + (bid >> 3);
}

// One thread per (16-row block, 32-wide K step, lane): eight values of U.
__global__ __launch_bounds__(256) void usplit_kernel(USplitParams p) {
  const int NK = p.KR >> 5;
  const int64_t nrb = p.dpad >> 4;
  const int64_t total = nrb * NK * 64;
  for (int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x; id < total; id += (int64_t)gridDim.x * 256) {
    const int lane = (int)(id & 63);
    const int64_t blk = id >> 6;
    const int kk = (int)(blk % NK);
    const int64_t rb = blk / NK;
    const int g = lane >> 4, i = lane & 15;
    const int64_t row = rb * 16 + i;
    const int j0 = 32 * kk + 8 * g;
    float u[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = (row < p.d && j0 + e < p.r) ? p.U[row * p.ldu + j0 + e] : 0.f;
    u32x4 hv, lv;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t h, l;
      split_hi_lo2(u[2 * q], u[2 * q + 1], h, l);
      hv[q] = h;
      lv[q] = l;
    }
    *reinterpret_cast<u32x4*>(p.Uhi + id * 8) = hv;
    *reinterpret_cast<u32x4*>(p.Ulo + id * 8) = lv;
  }
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

// A workgroup updates rows [r0, r0 + 64*NBW) x columns [c0, c0 + 256) of W.
// Wave w owns rows r0 + 16*NBW*w .. (+16*NBW) across all 256 columns (16
// column blocks), so its U operands are its own; the sign operands of all 16
// column blocks are expanded once per K step by the whole workgroup into a
// double-buffered LDS stage.
template <int NBW>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  constexpr int MB = 16;   // 16-column blocks per 256-column block
  constexpr int STR = 9;   // dwords per row (row-major bits) / per column (column-major bits)
  __shared__ uint32_t rowbits[256 * STR];
  __shared__ uint32_t colbits[256 * STR];
  __shared__ u32x4 sgn[2][MB * 64];

  const int lin = xcd_linear_id_m(blockIdx.x, gridDim.x);
  const int dt = lin / p.n_cb;
  const int cb = lin - dt * p.n_cb;
  if (dt >= p.n_dt) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, i = lane & 15;
  const int64_t c0 = (int64_t)cb * 256;
  const int64_t rw = (int64_t)dt * 64 * NBW + (int64_t)wave * 16 * NBW;  // first row of this wave
  const int NK = p.KR >> 5;

  // Signs of rows 0 .. KR-1 for this 256-column block.
  if (threadIdx.x < p.KR) {
    uint32_t w[8];
    philox_sign_block(p.seed, threadIdx.x, (uint32_t)cb, w);
#pragma unroll
    for (int q = 0; q < 8; ++q) rowbits[threadIdx.x * STR + q] = w[q];
  }
  __syncthreads();
  {
    const uint8_t* rb = reinterpret_cast<const uint8_t*>(rowbits);
    uint8_t* cbt = reinterpret_cast<uint8_t*>(colbits);
    for (int task = threadIdx.x; task < 32 * (p.KR >> 3); task += 256) {
      const int co = task & 31;  // column octet
      const int ro = task >> 5;  // row octet
      uint64_t x = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) x |= (uint64_t)rb[(8 * ro + e) * STR * 4 + co] << (8 * e);
      x = transpose8x8(x);
#pragma unroll
      for (int b = 0; b < 8; ++b) cbt[(8 * co + b) * STR * 4 + ro] = (uint8_t)(x >> (8 * b));
    }
  }
  __syncthreads();

  // Wave w expands column blocks 4w .. 4w+3 of K step kk into stage buf.
  const SignExpander ex(g);
  auto expand = [&](int kk, int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int mb = 4 * wave + q;
      sgn[buf][mb * 64 + lane] = ex(colbits[(16 * mb + i) * STR + kk]);
    }
  };

  f32x4 acc[MB][NBW];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 bh[2][NBW], bl[2][NBW];
  auto load_u = [&](int kk, int s) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int64_t rb16 = (rw >> 4) + nb;
      const int64_t off = ((rb16 * NK + kk) * 64 + lane) * 8;
      bh[s][nb] = *reinterpret_cast<const u32x4*>(p.Uhi + off);
      bl[s][nb] = *reinterpret_cast<const u32x4*>(p.Ulo + off);
    }
  };

  expand(0, 0);
  load_u(0, 0);
  __syncthreads();
  for (int k0 = 0; k0 < NK; k0 += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kk = k0 + u;
      if (kk < NK) {
        if (kk + 1 < NK) {
          expand(kk + 1, u ^ 1);
          load_u(kk + 1, u ^ 1);
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const u32x4 a = sgn[u][mb * 64 + lane];
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb) {
            acc[mb][nb] = mfma_16x16x32(a, bh[u][nb], acc[mb][nb]);
            acc[mb][nb] = mfma_16x16x32(a, bl[u][nb], acc[mb][nb]);
          }
        }
        __syncthreads();
      }
    }
  }

#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int64_t row = rw + 16 * nb + i;
    if (row >= p.d) continue;
    uint16_t* wrow = p.W + row * p.ldw;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int64_t col = c0 + 16 * mb + 4 * g;
      if (col >= p.k) continue;
      uint16_t* dst = wrow + col;
      uint32_t wb[4];
      const bool full = col + 4 <= p.k;
      if (full) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(dst);
        wb[0] = v[0] & 0xffffu; wb[1] = v[0] >> 16; wb[2] = v[1] & 0xffffu; wb[3] = v[1] >> 16;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) wb[e] = (col + e < p.k) ? dst[e] : 0u;
      }
      float nw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) nw[e] = __fmaf_rn(-p.scale_eff, acc[mb][nb][e], bf16_to_f32(wb[e]));
      const uint32_t p01 = pack_bf16x2(nw[0], nw[1]), p23 = pack_bf16x2(nw[2], nw[3]);
      if (full) {
        *reinterpret_cast<u32x2*>(dst) = u32x2{p01, p23};
      } else {
        const uint32_t h[4] = {p01 & 0xffffu, p01 >> 16, p23 & 0xffffu, p23 >> 16};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < p.k) dst[e] = (uint16_t)h[e];
      }
    }
  }
}

namespace {
size_t align_up_m(size_t x, size_t a) { return (x + a - 1) / a * a; }
}

MergePlan plan_merge(int64_t d, int64_t k, int r) {
  MergePlan pl{};
  const int KR = (r + 31) / 32 * 32;
  pl.n_cb = (int)((k + 255) / 256);
  int NBW = 2;
  if ((int64_t)pl.n_cb * ((d + 127) / 128) < 256) NBW = 1;
  NBW = env_int("LOGRA_MERGE_NBW", NBW);
  if (NBW != 1) NBW = 2;
  pl.NBW = NBW;
  pl.n_dt = (int)((d + 64 * NBW - 1) / (64 * NBW));
  pl.dpad = (int64_t)pl.n_dt * 64 * NBW;
  pl.u_bytes = align_up_m((size_t)pl.dpad * KR * 2, 256);
  return pl;
}

bool merge_launch(const MergePlan& pl, const USplitParams& up, const MergeParams& mp, hipStream_t s) {
  const int64_t items = up.dpad / 16 * (up.KR / 32) * 64;
  int ugrid = (int)((items + 255) / 256);
  if (ugrid > 2048) ugrid = 2048;
  if (ugrid < 1) ugrid = 1;
  hipLaunchKernelGGL(usplit_kernel, dim3(ugrid), dim3(256), 0, s, up);
  const int grid = (int)align_up_m((size_t)pl.n_cb * pl.n_dt, 8);
  if (pl.NBW == 1)
    hipLaunchKernelGGL((merge_kernel<1>), dim3(grid), dim3(256), 0, s, mp);
  else
    hipLaunchKernelGGL((merge_kernel<2>), dim3(grid), dim3(256), 0, s, mp);
  return true;
}

}  // namespace logra
