// Fused expand-and-merge (gfx950): W <- RNE_bf16(W - scale/sqrt(r) * U s).
// "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
// Sketches", section 2.1, equations 3 and 4 (W <- W - alpha eta U A) and
// Algorithm 1's trainer update.  No d x k update buffer exists: every W tile
// is read once, updated in fp32 and rounded to bf16 once.
//
// One kernel.  A workgroup owns rows [r0, r0 + 64*NBW) and 16*CB columns of
// one 256-column sign block.  It regenerates that block's signs (Philox,
// rows 0..KR-1) into LDS, bit-transposes them so that one byte holds 8 rows of
// one column, and per 32-wide step of r expands the sign operands of its
// column blocks once into a double-buffered LDS stage shared by its waves.
// Each wave owns 16*NBW rows: it reads its U rows straight from memory,
// splits them into a bf16 hi/lo pair in registers and runs the MFMAs.  The W
// tile is fetched at the start and rewritten at the end.
//
// MFMA orientation D = s^T U^T: M = 16 columns of W, N = 16 rows of W,
// K = 32 entries of r, so each lane ends with four consecutive columns of
// one W row (one 8-byte access).
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

template <int NBW, int CB>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  constexpr int STR = 9;  // dwords per row (row-major bits) / per column (column-major bits)
  __shared__ uint32_t rowbits[256 * STR];
  __shared__ uint32_t colbits[16 * CB * STR];
  __shared__ u32x4 sgn[2][CB * 64];

  const int lin = xcd_linear_id_m(blockIdx.x, gridDim.x);
  const int dt = lin / p.n_cb;
  const int ct = lin - dt * p.n_cb;  // column tile of 16*CB columns
  if (dt >= p.n_dt) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, i = lane & 15;
  const int64_t c0 = (int64_t)ct * 16 * CB;
  const int sblk = (int)(c0 >> 8);   // 256-column sign block
  const int cofs = (int)(c0 & 255);  // first column inside it
  const int64_t rw = (int64_t)dt * 64 * NBW + (int64_t)wave * 16 * NBW;  // first row of this wave
  const int NK = p.KR >> 5;

  // W tile of this lane: rows rw + 16*nb + i, columns c0 + 16*mb + 4g .. +3.
  // Rows past d read as zero through the descriptor and are never written.
  const __amdgpu_buffer_rsrc_t rwb = make_rsrc(p.W, (uint32_t)(p.d * p.ldw * 2));
  u32x2 wv[CB][NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const uint32_t rowoff = (uint32_t)((rw + 16 * nb + i) * p.ldw * 2);
#pragma unroll
    for (int mb = 0; mb < CB; ++mb)
      wv[mb][nb] = buf_load8(rwb, rowoff + (uint32_t)((c0 + 16 * mb + 4 * g) * 2));
  }

  // Signs of rows 0 .. KR-1 for this 256-column block, then bit-transpose the
  // workgroup's columns so that one byte holds 8 consecutive rows of a column.
  if (threadIdx.x < p.KR) {
    uint32_t w[8];
    philox_sign_block(p.seed, threadIdx.x, (uint32_t)sblk, w);
#pragma unroll
    for (int q = 0; q < 8; ++q) rowbits[threadIdx.x * STR + q] = w[q];
  }
  __syncthreads();
  {
    const uint8_t* rb = reinterpret_cast<const uint8_t*>(rowbits);
    uint8_t* cbt = reinterpret_cast<uint8_t*>(colbits);
    constexpr int NCO = 2 * CB;  // column octets of this workgroup
    for (int task = threadIdx.x; task < NCO * (p.KR >> 3); task += 256) {
      const int co = task % NCO;  // column octet
      const int ro = task / NCO;  // row octet
      uint64_t x = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) x |= (uint64_t)rb[(8 * ro + e) * STR * 4 + (cofs >> 3) + co] << (8 * e);
      x = transpose8x8(x);
#pragma unroll
      for (int b = 0; b < 8; ++b) cbt[(8 * co + b) * STR * 4 + ro] = (uint8_t)(x >> (8 * b));
    }
  }
  __syncthreads();

  // The four waves expand the column blocks of K step kk into stage buf.
  const SignExpander ex(g);
  auto expand = [&](int kk, int buf) {
#pragma unroll
    for (int q = 0; q < (CB + 3) / 4; ++q) {
      const int mb = 4 * q + wave;
      if (mb < CB) sgn[buf][mb * 64 + lane] = ex(colbits[(16 * mb + i) * STR + kk]);
    }
  };

  // U rows of this wave, split into a bf16 hi/lo pair in registers.  Entries
  // past r are zeroed; rows past d read as zero through the descriptor.
  const __amdgpu_buffer_rsrc_t ru = make_rsrc(p.U, (uint32_t)(p.d * p.ldu * 4));
  u32x4 bh[2][NBW], bl[2][NBW];
  auto load_u = [&](int kk, int s) {
    const int j0 = 32 * kk + 8 * g;
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const uint32_t off = (uint32_t)(((rw + 16 * nb + i) * p.ldu + j0) * 4);
      float u[8];
      if (p.u_vec) {
        const f32x4 x0 = __builtin_bit_cast(f32x4, buf_load16(ru, off));
        const f32x4 x1 = __builtin_bit_cast(f32x4, buf_load16(ru, off + 16));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          u[e] = x0[e];
          u[4 + e] = x1[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          u[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ru, off + 4 * e, 0, 0));
      }
      if (j0 + 8 > p.r) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (j0 + e >= p.r) u[e] = 0.f;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t h, l;
        split_hi_lo2(u[2 * q], u[2 * q + 1], h, l);
        bh[s][nb][q] = h;
        bl[s][nb][q] = l;
      }
    }
  };

  f32x4 acc[CB][NBW];
#pragma unroll
  for (int mb = 0; mb < CB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

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
        for (int mb = 0; mb < CB; ++mb) {
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

  const float ns = -p.scale_eff;
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int64_t row = rw + 16 * nb + i;
    if (row >= p.d) continue;
    uint16_t* wrow = p.W + row * p.ldw;
#pragma unroll
    for (int mb = 0; mb < CB; ++mb) {
      const int64_t col = c0 + 16 * mb + 4 * g;
      if (col >= p.k) continue;
      const u32x2 v = wv[mb][nb];
      const float w0 = __uint_as_float(v[0] << 16), w1 = __uint_as_float(v[0] & 0xffff0000u);
      const float w2 = __uint_as_float(v[1] << 16), w3 = __uint_as_float(v[1] & 0xffff0000u);
      const uint32_t p01 = pack_bf16x2(__fmaf_rn(ns, acc[mb][nb][0], w0), __fmaf_rn(ns, acc[mb][nb][1], w1));
      const uint32_t p23 = pack_bf16x2(__fmaf_rn(ns, acc[mb][nb][2], w2), __fmaf_rn(ns, acc[mb][nb][3], w3));
      uint16_t* dst = wrow + col;
      if (col + 4 <= p.k) {
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
}  // namespace

MergePlan plan_merge(int64_t d, int64_t k, int r) {
  MergePlan pl{};
  int NBW = 2, CB = 16;
  auto tiles = [&](int nbw, int cb) {
    return ((k + 16 * cb - 1) / (16 * cb)) * ((d + 64 * nbw - 1) / (64 * nbw));
  };
  if (tiles(NBW, CB) < 512) NBW = 1;
  if (tiles(NBW, CB) < 256) CB = 8;
  NBW = env_int("LOGRA_MERGE_NBW", NBW) == 1 ? 1 : 2;
  CB = env_int("LOGRA_MERGE_CB", CB) == 8 ? 8 : 16;
  pl.NBW = NBW;
  pl.CB = CB;
  pl.n_cb = (int)((k + 16 * CB - 1) / (16 * CB));
  pl.n_dt = (int)((d + 64 * NBW - 1) / (64 * NBW));
  (void)r;
  return pl;
}

bool merge_launch(const MergePlan& pl, const MergeParams& mp, hipStream_t s) {
  const int grid = (int)align_up_m((size_t)pl.n_cb * pl.n_dt, 8);
#define LOGRA_MERGE(nbw, cb)                                                              \
  if (pl.NBW == nbw && pl.CB == cb) {                                                     \
    hipLaunchKernelGGL((merge_kernel<nbw, cb>), dim3(grid), dim3(256), 0, s, mp);         \
    return true;                                                                          \
  }
  LOGRA_MERGE(1, 8) LOGRA_MERGE(1, 16) LOGRA_MERGE(2, 8) LOGRA_MERGE(2, 16)
#undef LOGRA_MERGE
  return false;
}

}  // namespace logra
