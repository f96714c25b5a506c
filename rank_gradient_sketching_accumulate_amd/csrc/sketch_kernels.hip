// Sketch accumulation kernels (gfx950): S += G A^T for one microbatch, with
// G = dY^T X never formed.  "LoGRA: Scaling LLM Reinforcement Learning with
// Low-Rank Gradient Sketches", section 2.1 (equation 2 and the direct
// accumulation of projected microbatch contributions into an fp32 sketch;
// the inputs are projected before the backward derivatives multiply them).
//
//   proj_kernel       P = X s^T        (bf16 x exact +-1 on MFMA, fp32 sums)
//   contract_*        S += dY^T P / sqrt(r)   (P as a bf16 hi/lo pair)
//
// Pk layout of P (tokens x 16*NB columns; one array of high halves, one of
// low halves):
//   elem(t, c) = (((t/32)*NB + c/16)*64 + ((t%32)/8)*16 + c%16)*8 + t%8
// so that lane l of a contraction MFMA step over tokens 32*ks.. and columns
// 16*nb.. reads its eight tokens as one 16-byte word at ((ks*NB + nb)*64 + l)*8.
#include "logra_device.h"
#include "logra_internal.h"

#include <stdlib.h>

namespace logra {

__device__ __forceinline__ int64_t pk_index(int64_t t, int c, int NB) {
  return (((t >> 5) * NB + (c >> 4)) * 64 + ((t & 31) >> 3) * 16 + (c & 15)) * 8 + (t & 7);
}

// Workgroups are dealt to the eight XCDs round-robin by id; renumber them so
// consecutive logical ids share an XCD and its L2.  grid is a multiple of 8.
__device__ __forceinline__ int xcd_linear_id(int bid, int grid) {
  return (bid & 7) * (grid >> 3) + (bid >> 3);
}

// X[t][c .. c+7] as 8 bf16; zeros outside the matrix.
__device__ __forceinline__ u32x4 load_x8(const uint16_t* X, int64_t ldx, int64_t T, int64_t k,
                                         int64_t t, int64_t c) {
  u32x4 v = {0u, 0u, 0u, 0u};
  if (t < T && c < k) {
    const uint16_t* p = X + t * ldx + c;
    if (c + 8 <= k) {
      v = *reinterpret_cast<const u32x4*>(p);
    } else {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = (c + e < k) ? p[e] : 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = h[2 * q] | (h[2 * q + 1] << 16);
    }
  }
  return v;
}

// ===========================================================================
// Projection for small r*k (the signs of the whole k range fit in LDS).
// A workgroup of eight waves owns TT = 16*MBW tokens; the waves split the
// 32-column steps of k evenly.  Every wave issues its X loads first (a ring
// of eight steps), then the workgroup regenerates all sign blocks once, then
// each wave multiplies its steps, and the eight column partials are summed
// through LDS.
// ===========================================================================
template <int NB, int MBW>
__global__ __launch_bounds__(512) void proj_small_kernel(ProjParams p) {
  constexpr int RP = 16 * NB;
  constexpr int NW = 8;
  constexpr int TT = 16 * MBW;
  constexpr int SROW = 9;
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];

  const int tt = blockIdx.x;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4, i = lane & 15;
  const int64_t t0 = (int64_t)tt * TT;
  const int nks = (int)((p.k + 31) >> 5);
  const int q = (nks + NW - 1) / NW;
  const int ks0 = w * q;
  const int nloc = max(0, min(nks, ks0 + q) - ks0);

  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.X, (uint32_t)(p.T * p.ldx * 2));
  uint32_t rowoff[MBW];
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb) rowoff[mb] = (uint32_t)((t0 + 16 * mb + i) * p.ldx * 2);

  f32x4 acc[MBW][NB];
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 xr[8][MBW];
  // Loads are unconditional (steps past the wave's range re-read the last
  // step of k and are never used): a load under a branch would make the
  // compiler's wait counts wait for every load in flight.
  auto issue = [&](u32x4 (&slot)[MBW], int j) {
    const int64_t col = (int64_t)min(ks0 + j, nks - 1) * 32 + 8 * g;
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) slot[mb] = buf_load16(rx, rowoff[mb] + (uint32_t)(col * 2));
  };
  // The last step of a k that is not a multiple of 32: zero the entries past k.
  auto xmask = [&](u32x4 (&slot)[MBW], int ks) {
    if ((int64_t)ks * 32 + 32 <= p.k) return;
    const int64_t nv = p.k - ((int64_t)ks * 32 + 8 * g);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t m = (2 * q < nv ? 0x0000ffffu : 0u) | (2 * q + 1 < nv ? 0xffff0000u : 0u);
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb) slot[mb][q] &= m;
    }
  };
#pragma unroll
  for (int j = 0; j < 7; ++j) issue(xr[j], j);

  for (int b = threadIdx.x; b < RP * p.ncb; b += NW * 64) {
    const int row = b % RP, cb = b / RP;
    uint32_t wd[8];
    philox_sign_block(p.seed, (uint32_t)(p.row0 + row), (uint32_t)cb, wd);
    uint32_t* dst = lds + (cb * RP + row) * SROW;
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = wd[e];
  }
  __syncthreads();

  const SignExpander ex(g);
  for (int j0 = 0; j0 < nloc; j0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u;
      issue(xr[(u + 7) & 7], j + 7);
      if (j < nloc) {
        const int ks = ks0 + j;
        xmask(xr[u], ks);
        const uint32_t* sb = lds + ((ks >> 3) * RP + i) * SROW + (ks & 7);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const u32x4 bsg = ex(sb[16 * nb * SROW]);
#pragma unroll
          for (int mb = 0; mb < MBW; ++mb) acc[mb][nb] = mfma_16x16x32(xr[u][mb], bsg, acc[mb][nb]);
        }
      }
    }
  }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    if (16 * nb + i >= p.r)
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Eight-way sum of the column partials, one 16-token block at a time:
  // every wave parks its accumulators in LDS as whole float4s (1 KB
  // contiguous per column block), then each thread sums one float4 item
  // (four consecutive tokens of one column) over the eight waves and writes
  // their hi/lo pair.
  constexpr int ITEMS = NB * 64;
  f32x4* red = reinterpret_cast<f32x4*>(lds);
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb) {
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) red[w * ITEMS + nb * 64 + lane] = acc[mb][nb];
    __syncthreads();
    for (int v = threadIdx.x; v < ITEMS; v += NW * 64) {
      const int ln = v & 63, nb = v >> 6;  // lane (g, i) of wave 0's layout, column block
      f32x4 sum = red[v];
#pragma unroll
      for (int q = 1; q < NW; ++q) {
        const f32x4 o = red[q * ITEMS + v];
        sum[0] += o[0]; sum[1] += o[1]; sum[2] += o[2]; sum[3] += o[3];
      }
      const int gg = ln >> 4, ii = ln & 15;
      const int64_t e0 = pk_index(t0 + 16 * mb + 4 * gg, 16 * nb + ii, NB);
      uint32_t h0, l0, h1, l1;
      split_hi_lo2(sum[0], sum[1], h0, l0);
      split_hi_lo2(sum[2], sum[3], h1, l1);
      *reinterpret_cast<u32x2*>(p.Phi + e0) = u32x2{h0, h1};
      if (p.hi_only != 1) *reinterpret_cast<u32x2*>(p.Plo + e0) = p.hi_only ? u32x2{0u, 0u} : u32x2{l0, l1};
    }
  }
}

size_t proj_small_lds_bytes(int NB, int ncb) {
  const size_t signs = (size_t)16 * NB * ncb * 9 * 4;
  const size_t red = (size_t)8 * NB * 256 * 4;
  return signs > red ? signs : red;
}

// ===========================================================================
// Projection.  A workgroup owns TT = (4/WK)*16*MBW tokens and the 256-column
// blocks [cbb, cbe) of k.  Its WK wave columns take the blocks of one "round"
// side by side; the 4/WK wave rows take different tokens.  Each round the
// workgroup regenerates the signs of the next round's blocks into LDS while
// it multiplies the current ones, and every wave keeps X loads for the next
// seven 32-column steps in flight in a register ring.
// ===========================================================================
template <int NB, int MBW, int WK, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void proj_kernel(ProjParams p) {
  constexpr int RP = 16 * NB;
  constexpr int NT = NW * 64;  // threads
  constexpr int WT = NW / WK;
  constexpr int TT = WT * 16 * MBW;
  constexpr int SROW = 9;  // 8 dwords of sign bits + 1 pad dword (bank spread)
  constexpr int NGEN = (RP * WK + NT - 1) / NT;
  constexpr int RED = WK > 1 ? (WK - 1) * WT * NB * 256 : 4;
  constexpr int SB = 2 * WK * RP * SROW;
  __shared__ uint32_t smem[SB > RED ? SB : RED];
  uint32_t (*const sbits)[WK * RP * SROW] = reinterpret_cast<uint32_t (*)[WK * RP * SROW]>(smem);
  // After the last round (which ends with a barrier) the sign buffers are free
  // and hold the partial sums of the WK wave columns.
  float* const red = reinterpret_cast<float*>(smem);
  __shared__ int s_last;

  const int lin = xcd_linear_id(blockIdx.x, gridDim.x);
  const int tt = lin / p.n_k;
  const int ksp = lin - tt * p.n_k;
  if (tt >= p.n_tt) return;

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4, i = lane & 15;
  const int wt = wave % WT, wk = wave / WT;
  const int64_t t0 = (int64_t)tt * TT;
  const int64_t tw = t0 + (int64_t)wt * 16 * MBW;
  const int cbb = ksp * p.cbs_per;
  const int cbe = min(p.ncb, cbb + p.cbs_per);
  const int nrounds = (cbe - cbb + WK - 1) / WK;

  f32x4 acc[MBW][NB];
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Philox blocks of round j (rows 0..RP-1, one 256-column block per wave column).
  auto gen = [&](int j, int buf) {
#pragma unroll
    for (int q = 0; q < NGEN; ++q) {
      const int b = threadIdx.x + NT * q;
      if (b < RP * WK) {
        const int row = b % RP, wkk = b / RP;
        const int cb = cbb + j * WK + wkk;
        if (cb < cbe) {
          uint32_t w[8];
          philox_sign_block(p.seed, (uint32_t)(p.row0 + row), (uint32_t)cb, w);
          uint32_t* dst = &sbits[buf][(wkk * RP + row) * SROW];
#pragma unroll
          for (int e = 0; e < 8; ++e) dst[e] = w[e];
        }
      }
    }
  };

  // X through a buffer descriptor: token rows past T read as zero.  Every
  // load is issued unconditionally (a block past the range re-reads the
  // range's last block, which is in cache): a load under a branch would make
  // the compiler's wait counts assume the path without it and wait for every
  // load in flight.  Columns past k, and blocks past the range, are zeroed
  // where the step is used (xmask).
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.X, (uint32_t)(p.T * p.ldx * 2));
  uint32_t rowoff[MBW];
#pragma unroll
  for (int mb = 0; mb < MBW; ++mb) rowoff[mb] = (uint32_t)((tw + 16 * mb + i) * p.ldx * 2);
  u32x4 xr[8][MBW];
  auto issue = [&](u32x4 (&slot)[MBW], int cb, int s) {
    const int cbl = min(cb, cbe - 1);
    const uint32_t coff = (uint32_t)(((int64_t)cbl * 256 + 32 * s + 8 * g) * 2);
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) slot[mb] = buf_load16(rx, rowoff[mb] + coff);
  };
  // Zero the entries of a step's X operands whose columns fall past k (only
  // the last step of k can have any; wave-uniform test).
  auto xmask = [&](u32x4 (&slot)[MBW], int cb, int s) {
    const int64_t c0 = (int64_t)cb * 256 + 32 * s;
    if (c0 + 32 <= p.k) return;
    const int64_t nv = p.k - (c0 + 8 * g);  // valid entries of this lane's eight
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t m = (2 * q < nv ? 0x0000ffffu : 0u) | (2 * q + 1 < nv ? 0xffff0000u : 0u);
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb) slot[mb][q] &= m;
    }
  };

  gen(0, 0);
  {
    const int cbw = cbb + wk;
#pragma unroll
    for (int s = 0; s < 7; ++s) issue(xr[s], cbw, s);
  }
  __syncthreads();

  for (int j = 0; j < nrounds; ++j) {
    const int buf = j & 1;
    if (j + 1 < nrounds) gen(j + 1, buf ^ 1);
    const int cb = cbb + j * WK + wk;
    const uint32_t* sb = &sbits[buf][(wk * RP + i) * SROW];
    const SignExpander ex(g);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s == 0)
        issue(xr[7], cb, 7);
      else
        issue(xr[s - 1], cb + WK, s - 1);
      if (cb < cbe) {
        xmask(xr[s], cb, s);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const u32x4 bsg = ex(sb[16 * nb * SROW + s]);
#pragma unroll
          for (int mb = 0; mb < MBW; ++mb) acc[mb][nb] = mfma_16x16x32(xr[s][mb], bsg, acc[mb][nb]);
        }
      }
    }
    __syncthreads();
  }

  // Columns >= r used sign rows the caller did not ask for.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    if (16 * nb + i >= p.r)
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Sum the WK column partials of each token row of waves through LDS.
  if constexpr (WK > 1) {
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
      if (wk > 0) {
        float* dst = red + ((wk - 1) * WT + wt) * NB * 256;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[(nb * 4 + e) * 64 + lane] = acc[mb][nb][e];
      }
      __syncthreads();
      if (wk == 0) {
#pragma unroll
        for (int w = 1; w < WK; ++w) {
          const float* src = red + ((w - 1) * WT + wt) * NB * 256;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[mb][nb][e] += src[(nb * 4 + e) * 64 + lane];
        }
      }
      __syncthreads();
    }
  }

  if (p.n_k == 1) {
    if (wk == 0) {
#pragma unroll
      for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int64_t e0 = pk_index(tw + 16 * mb + 4 * g, 16 * nb + i, NB);
          uint32_t h0, l0, h1, l1;
          split_hi_lo2(acc[mb][nb][0], acc[mb][nb][1], h0, l0);
          split_hi_lo2(acc[mb][nb][2], acc[mb][nb][3], h1, l1);
          *reinterpret_cast<u32x2*>(p.Phi + e0) = u32x2{h0, h1};
          if (p.hi_only != 1) *reinterpret_cast<u32x2*>(p.Plo + e0) = p.hi_only ? u32x2{0u, 0u} : u32x2{l0, l1};
        }
    }
    return;
  }

  // Column splits across workgroups: each split stores its fp32 partial with
  // agent-coherent (sc1) stores; the last split of the tile to arrive reads
  // them back with agent-coherent loads, sums them in split order and writes
  // the hi/lo pair.  No cache-wide write-back is involved.
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.Ppart, (uint32_t)((int64_t)p.n_k * p.part_stride * 4));
  if (wk == 0) {
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int64_t e0 = (int64_t)ksp * p.part_stride + pk_index(tw + 16 * mb + 4 * g, 16 * nb + i, NB);
        store16_agent(rs, (uint32_t)(e0 * 4), __builtin_bit_cast(u32x4, acc[mb][nb]));
      }
  }
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(p.counters + tt, 1u);
    s_last = (prev == (unsigned)(p.n_k - 1));
  }
  __syncthreads();
  if (!s_last) return;
  // Walk the tile in the units the waves stored: four consecutive tokens of
  // one column (16 bytes of fp32 per split).
  for (int v = threadIdx.x; v < TT * RP / 4; v += NT) {
    const int col = v % RP;
    const int64_t tq = t0 + 4 * (int64_t)(v / RP);
    const int64_t e0 = pk_index(tq, col, NB);
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < p.n_k; ++sp) {
      const uint32_t off = (uint32_t)(((int64_t)sp * p.part_stride + e0) * 4);
      sum += __builtin_bit_cast(f32x4, load16_agent(rs, off));
    }
    uint32_t h0, l0, h1, l1;
    split_hi_lo2(sum[0], sum[1], h0, l0);
    split_hi_lo2(sum[2], sum[3], h1, l1);
    *reinterpret_cast<u32x2*>(p.Phi + e0) = u32x2{h0, h1};
    if (p.hi_only != 1) *reinterpret_cast<u32x2*>(p.Plo + e0) = p.hi_only ? u32x2{0u, 0u} : u32x2{l0, l1};
  }
  if (threadIdx.x == 0) p.counters[tt] = 0u;
}

// ===========================================================================
// Projection for ranks above 32 (NB = 4, 8 or 16), X staged through LDS.
// Eight waves, two per SIMD.  Wave (wn, wk) keeps the workgroup's 64 tokens
// x one half of P's 16*NB columns in accumulators (8*NB*2 registers: 128 at
// NB = 16, pinned to the AGPR half of the wave's registers), so that each
// expanded sign operand feeds four MFMAs.  The k range goes in rounds of
// four 256-column blocks; within a round the four k waves take interleaved
// 32-column slices of one 128-column slab per step (wave wk: columns
// 128 s + 32 wk .. + 31 of the round).  The workgroup loads each slab once:
// thread q moves 16-byte chunk q % 16 of rows q / 16 and q / 16 + 32, so one
// load instruction covers four rows x 256 contiguous bytes (two whole cache
// lines per row) and no X byte is loaded twice by one CU.  (Sixteen rows x
// 64 bytes per instruction, the MFMA operand's own layout, kept the texture
// addresser busy about 70 cycles per load and set the kernel's pace.)  In
// LDS, chunk c of row t sits at slot c ^ (t & 15) of the row's 256 bytes, so
// the sixteen rows of an MFMA operand read fall in distinct banks.  Slab
// u + 2 is loaded into registers during step u and slab u + 1 is stored into
// the other LDS buffer at the end of step u, before the step's barrier.
// Each round first draws the signs of the next round's four blocks into the
// other LDS sign buffer (two Philox blocks per thread at NB = 16, one at
// NB = 8, one for half the threads at NB = 4); the signs never leave
// registers and LDS.  After the last round
// the four wave columns are summed through LDS in two halving rounds, and the wk = 0 waves write P (or, with column
// splits across workgroups, their fp32 partial; the last split to arrive
// sums the partials).
// ===========================================================================
template <int NB>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void proj_lds_kernel(ProjParams p) {
  constexpr int RP = 16 * NB;
  constexpr int NBW = NB / 2;           // column blocks per wave
  constexpr int MT = 4;                 // 16-token blocks per wave: the whole tile
  constexpr int TT = 16 * MT;           // tokens per workgroup
  constexpr int WK = 4;                 // blocks per round
  constexpr int SROW = 9;               // 8 dwords of sign bits + 1 pad dword per row
  constexpr int SBUF = WK * RP * SROW;  // dwords of one sign buffer
  constexpr int XBUF = TT * 64;         // dwords of one X slab: 64 rows x 128 columns
  constexpr int RED = 2 * 2 * NBW * MT * 256;  // floats parked in the first halving round
  constexpr int MAIN = 2 * SBUF + 2 * XBUF;
  constexpr int LDSW = (MAIN > RED) ? MAIN : RED;
  static_assert((2 * SBUF) % 4 == 0, "X slabs on 16-byte boundaries");
  __shared__ __attribute__((aligned(16))) uint32_t smem[LDSW];
  __shared__ int s_last;
  uint32_t* const xlds = smem + 2 * SBUF;

  const int lin = xcd_linear_id(blockIdx.x, gridDim.x);
  const int tt = lin / p.n_k;
  const int ksp = lin - tt * p.n_k;
  if (tt >= p.n_tt) return;

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, i = lane & 15;
  const int wn = wave & 1, wk = wave >> 1;
  const int64_t t0 = (int64_t)tt * TT;
  const int cbb = ksp * p.cbs_per;
  const int cbe = min(p.ncb, cbb + p.cbs_per);
  const int nrounds = (cbe - cbb + WK - 1) / WK;

  f32x4 acc[NBW][MT];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) acc[nb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Signs of round j: rows 0 .. RP-1 of blocks cbb + WK*j .. + WK-1, one
  // Philox block (256 columns of one row) per thread and pass, written to
  // LDS row (wkk * RP + row) with the row stride SROW (the ninth dword only
  // spreads the banks and is never read).  Blocks past k are drawn too;
  // their X is zeroed.
  constexpr int NGEN = (RP * WK + 511) / 512;
  auto gen = [&](int j, int buf) {
#pragma unroll 1
    for (int q = 0; q < NGEN; ++q) {
      const int b = threadIdx.x + 512 * q;
      if (RP * WK % 512 != 0 && b >= RP * WK) break;  // NB = 4: half the threads draw
      const int row = b % RP, wkk = b / RP;
      uint32_t w[8];
      philox_sign_block(p.seed, (uint32_t)(p.row0 + row), (uint32_t)(cbb + WK * j + wkk), w);
      uint32_t* dst = smem + buf * SBUF + (wkk * RP + row) * SROW;
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = w[e];
    }
  };

  // X slabs.  Rows past T read as zero (buffer range); columns past k or
  // past the split's blocks are zeroed when staged.  Loads are unconditional
  // (a slab past the last round reads whatever lies there and is zeroed).
  const int sc = threadIdx.x & 15, srow = threadIdx.x >> 4;  // chunk, row (and row + 32)
  const int64_t xbytes = p.T * p.ldx * 2;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.X, (uint32_t)xbytes);
  // Byte offsets fit 32 bits: the planner keeps (Tpad + 32) * ldx * 2 below
  // 2^32 - 4096, and a slab column never passes ldx + 2304.
  const uint32_t rowoff0 = (uint32_t)((t0 + srow) * p.ldx * 2), rowoff1 = (uint32_t)((t0 + srow + 32) * p.ldx * 2);
  const int lim = (int)min(p.k, (int64_t)cbe * 256);  // first column that stages as zero
  auto slab_base = [&](int u) { return (cbb + WK * (u >> 3)) * 256 + 128 * (u & 7); };  // wave-uniform
  auto xload = [&](u32x4 (&v)[2], int u) {
    const uint32_t c2 = (uint32_t)(slab_base(u) + 8 * sc) * 2u;
    v[0] = buf_load16(rx, rowoff0 + c2);
    v[1] = buf_load16(rx, rowoff1 + c2);
  };
  auto xstore = [&](u32x4 (&v)[2], int u) {
    const int sbase = slab_base(u);
    if (sbase + 128 > lim) {  // a slab that reaches past k or past the split's blocks (uniform test)
      const int nv = lim - (sbase + 8 * sc);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t m = (2 * q < nv ? 0x0000ffffu : 0u) | (2 * q + 1 < nv ? 0xffff0000u : 0u);
        v[0][q] &= m;
        v[1][q] &= m;
      }
    }
    uint32_t* b = xlds + (u & 1) * XBUF;
    *reinterpret_cast<u32x4*>(b + srow * 64 + ((sc ^ (srow & 15)) * 4)) = v[0];
    *reinterpret_cast<u32x4*>(b + (srow + 32) * 64 + ((sc ^ (srow & 15)) * 4)) = v[1];
  };

  u32x4 xv[2][2];
  xload(xv[0], 0);
  xload(xv[1], 1);
  gen(0, 0);
  xstore(xv[0], 0);
  __syncthreads();

  const SignExpander ex(g);
  const int xoff = ((4 * wk + g) ^ i) * 4;  // this lane's chunk slot in its rows
  for (int j = 0; j < nrounds; ++j) {
    const int buf = j & 1;
    if (j + 1 < nrounds) gen(j + 1, buf ^ 1);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int u = 8 * j + s;
      xload(xv[s & 1], u + 2);  // slot of slab u (stored at the end of step u - 1)
      const uint32_t* xb = xlds + (s & 1) * XBUF + i * 64 + xoff;
      u32x4 a[MT];
#pragma unroll
      for (int mb = 0; mb < MT; ++mb) a[mb] = *reinterpret_cast<const u32x4*>(xb + 16 * mb * 64);
      const uint32_t* sb = smem + buf * SBUF + ((s >> 1) * RP + 16 * NBW * wn + i) * SROW + 4 * (s & 1) + wk;
      uint32_t sw[NBW];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) sw[nb] = sb[16 * nb * SROW];
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const u32x4 bsg = ex(sw[nb]);
        mfma4_b(acc[nb][0], acc[nb][1], acc[nb][2], acc[nb][3], a[0], a[1], a[2], a[3], bsg);
      }
      xstore(xv[(s + 1) & 1], u + 1);
      __syncthreads();
    }
  }
  // The accumulators live in AGPRs (pinned by the MFMA asm); from here on the
  // sums are worked on in VGPRs.
  mfma_drain();
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) mfma_touch(acc[nb][mb]);
  f32x4 v[NBW][MT];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) v[nb][mb] = acc[nb][mb];
  // (Columns >= r, from sign rows the caller did not ask for, are left in P:
  // they only feed columns of S that are never stored.)

  // Sum the four wave columns in two halving rounds through LDS (the sign
  // buffers are free: the last round ended with a barrier): wk = 2, 3 park
  // and wk = 0, 1 add, then wk = 1 parks and wk = 0 adds.
  float* const red = reinterpret_cast<float*>(smem);
  auto slot = [&](int half, int nb, int mb) {
    return red + (((half * 2 + wn) * NBW + nb) * MT + mb) * 256 + 4 * lane;
  };
#pragma unroll
  for (int level = 2; level >= 1; level >>= 1) {
    if (wk >= level && wk < 2 * level) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int mb = 0; mb < MT; ++mb) *reinterpret_cast<f32x4*>(slot(wk - level, nb, mb)) = v[nb][mb];
    }
    __syncthreads();
    if (wk < level) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int mb = 0; mb < MT; ++mb) v[nb][mb] += *reinterpret_cast<const f32x4*>(slot(wk, nb, mb));
    }
    __syncthreads();
  }
  const int cb0 = NBW * wn;  // first column block of this wave

  if (p.n_k == 1) {
    if (wk == 0) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
        for (int mb = 0; mb < MT; ++mb) {
          const f32x4 o = v[nb][mb];
          const int64_t e0 = pk_index(t0 + 16 * mb + 4 * g, 16 * (cb0 + nb) + i, NB);
          uint32_t h0, l0, h1, l1;
          split_hi_lo2(o[0], o[1], h0, l0);
          split_hi_lo2(o[2], o[3], h1, l1);
          *reinterpret_cast<u32x2*>(p.Phi + e0) = u32x2{h0, h1};
          if (p.hi_only != 1) *reinterpret_cast<u32x2*>(p.Plo + e0) = p.hi_only ? u32x2{0u, 0u} : u32x2{l0, l1};
        }
    }
    return;
  }

  // Column splits across workgroups (the splits of a token tile are
  // consecutive logical ids, all on one XCD): each split stores its fp32
  // partial with agent-coherent (sc1) stores; the last to arrive sums them
  // in split order and writes P, with all of a thread's loads in flight at
  // once.
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.Ppart, (uint32_t)((int64_t)p.n_k * p.part_stride * 4));
  if (wk == 0) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
      for (int mb = 0; mb < MT; ++mb) {
        const int64_t e0 = (int64_t)ksp * p.part_stride + pk_index(t0 + 16 * mb + 4 * g, 16 * (cb0 + nb) + i, NB);
        store16_agent(rs, (uint32_t)(e0 * 4), __builtin_bit_cast(u32x4, v[nb][mb]));
      }
  }
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(p.counters + tt, 1u);
    s_last = (prev == (unsigned)(p.n_k - 1));
  }
  __syncthreads();
  if (!s_last) return;
  constexpr int ITEMS = TT * RP / 4 / 512;  // float4 items per thread (2, 4 or 8)
  f32x4 sum[ITEMS];
  int64_t e0[ITEMS];
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) {
    const int v = threadIdx.x + 512 * q;
    e0[q] = pk_index(t0 + 4 * (int64_t)(v / RP), v % RP, NB);
    sum[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (int sp = 0; sp < p.n_k; ++sp) {
    f32x4 part[ITEMS];
#pragma unroll
    for (int q = 0; q < ITEMS; ++q)
      part[q] = __builtin_bit_cast(f32x4, load16_agent(rs, (uint32_t)(((int64_t)sp * p.part_stride + e0[q]) * 4)));
#pragma unroll
    for (int q = 0; q < ITEMS; ++q) sum[q] += part[q];
  }
#pragma unroll
  for (int q = 0; q < ITEMS; ++q) {
    uint32_t h0, l0, h1, l1;
    split_hi_lo2(sum[q][0], sum[q][1], h0, l0);
    split_hi_lo2(sum[q][2], sum[q][3], h1, l1);
    *reinterpret_cast<u32x2*>(p.Phi + e0[q]) = u32x2{h0, h1};
    if (p.hi_only != 1) *reinterpret_cast<u32x2*>(p.Plo + e0[q]) = p.hi_only ? u32x2{0u, 0u} : u32x2{l0, l1};
  }
  if (threadIdx.x == 0) p.counters[tt] = 0u;
}

// ===========================================================================
// Projection with the Gaussian basis: P = X Z^T with Z dense (the refreshed
// Gaussian projection), Z's bf16 hi/lo planes generated per call by
// gauss_basis_kernel.  Four waves of 16 tokens (64 per workgroup) x all 16*NB
// columns; k in 32-column steps.  A step's Z columns (hi and lo, 16*NB rows x
// 32) are staged through a two-buffer LDS ring shared by the four waves; X
// is read straight into the MFMA A operand (rows past T read as zero, columns
// past k are zeroed).  Each product takes two MFMAs (X times hi, X times lo).
// ===========================================================================
template <int NB>
__global__ __launch_bounds__(256) void proj_gauss_kernel(ProjParams p) {
  constexpr int RP = 16 * NB;
  constexpr int SW = RP * 4;                  // u32x4 words per plane and step
  constexpr int PER = (2 * SW + 255) / 256;   // words each thread stages per step
  __shared__ u32x4 st[2][2 * SW];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, i = lane & 15;
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int nsteps = (int)(p.kpad / 32);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.X, (uint32_t)(p.T * p.ldx * 2));
  const uint32_t xrow = (uint32_t)((t0 + 16 * wave + i) * p.ldx * 2);

  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Staged word w of a step: plane w / SW, row (w % SW) / 4, quad w % 4
  // (columns 8*quad .. 8*quad+7 of the step).
  u32x4 stg[PER];
  auto load_a = [&](int m) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int w = threadIdx.x + 256 * j;
      if (2 * SW % 256 == 0 || w < 2 * SW) {
        const int q = w % SW;
        const uint16_t* src = (w < SW ? p.Ahi : p.Alo) + (int64_t)(q >> 2) * p.kpad + 32 * (int64_t)m + 8 * (q & 3);
        stg[j] = *reinterpret_cast<const u32x4*>(src);
      }
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int w = threadIdx.x + 256 * j;
      if (2 * SW % 256 == 0 || w < 2 * SW) st[buf][w] = stg[j];
    }
  };

  if (nsteps > 0) {
    load_a(0);
    store_a(0);
  }
  __syncthreads();
  for (int m = 0; m < nsteps; ++m) {
    const int buf = m & 1;
    if (m + 1 < nsteps) load_a(m + 1);
    const int64_t c0 = 32 * (int64_t)m + 8 * g;
    u32x4 xa = buf_load16(rx, xrow + (uint32_t)(c0 * 2));
    if (c0 + 8 > p.k) {
      const int64_t nv = p.k - c0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t mk = (2 * q < nv ? 0x0000ffffu : 0u) | (2 * q + 1 < nv ? 0xffff0000u : 0u);
        xa[q] &= mk;
      }
    }
    const u32x4* ah = &st[buf][0];
    const u32x4* al = &st[buf][SW];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      acc[nb] = mfma_16x16x32(xa, ah[(16 * nb + i) * 4 + g], acc[nb]);
      acc[nb] = mfma_16x16x32(xa, al[(16 * nb + i) * 4 + g], acc[nb]);
    }
    if (m + 1 < nsteps) store_a(buf ^ 1);
    __syncthreads();
  }
  // acc[nb][e] = P[t0 + 16*wave + 4g + e][16*nb + i]: four consecutive tokens
  // of one column, consecutive in Pk order.
  const int64_t t = t0 + 16 * wave + 4 * g;
  if (t < p.Tw) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int64_t e0 = pk_index(t, 16 * nb + i, NB);
      uint32_t h0, l0, h1, l1;
      split_hi_lo2(acc[nb][0], acc[nb][1], h0, l0);
      split_hi_lo2(acc[nb][2], acc[nb][3], h1, l1);
      *reinterpret_cast<u32x2*>(p.Phi + e0) = u32x2{h0, h1};
      if (p.hi_only != 1) *reinterpret_cast<u32x2*>(p.Plo + e0) = p.hi_only ? u32x2{0u, 0u} : u32x2{l0, l1};
    }
  }
}

bool proj_gauss_launch(const SketchPlan& pl, const ProjParams& p, hipStream_t s) {
  const int grid = (int)((p.Tw + 63) / 64);
  if (grid < 1) return true;
  switch (pl.NB) {
    case 1: hipLaunchKernelGGL((proj_gauss_kernel<1>), dim3(grid), dim3(256), 0, s, p); return true;
    case 2: hipLaunchKernelGGL((proj_gauss_kernel<2>), dim3(grid), dim3(256), 0, s, p); return true;
    case 4: hipLaunchKernelGGL((proj_gauss_kernel<4>), dim3(grid), dim3(256), 0, s, p); return true;
    case 8: hipLaunchKernelGGL((proj_gauss_kernel<8>), dim3(grid), dim3(256), 0, s, p); return true;
    case 16: hipLaunchKernelGGL((proj_gauss_kernel<16>), dim3(grid), dim3(256), 0, s, p); return true;
  }
  return false;
}

// ===========================================================================
// Contraction S += (1/sqrt r) dY^T P.
// MFMA: A = dY^T (M = 16 rows of S), B = P (N = 16 columns), K = 32 tokens.
// A lane loads four consecutive columns of dY from eight token rows and a
// register transpose (one v_perm-like op per dword) turns them into the A
// operands of four M-blocks whose rows are d0 + 4*m + c (c = 0..3).
// ===========================================================================
constexpr int kDC = 4;

// dY[t][c .. c+3] as 2 dwords; zeros outside the matrix.
__device__ __forceinline__ u32x2 load_dy4(const uint16_t* dY, int64_t lddy, int64_t T, int64_t d,
                                          int64_t t, int64_t c) {
  u32x2 v = {0u, 0u};
  if (t < T && c < d) {
    const uint16_t* p = dY + t * lddy + c;
    if (c + 4 <= d) {
      v = *reinterpret_cast<const u32x2*>(p);
    } else {
      uint32_t h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) h[e] = (c + e < d) ? p[e] : 0u;
      v = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    }
  }
  return v;
}

// Eight token rows (2 dwords each) -> A operands of the four M-blocks.
__device__ __forceinline__ void transpose_dy(const u32x2 (&y)[8], u32x4 (&a)[kDC]) {
#pragma unroll
  for (int c = 0; c < kDC; ++c)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w0 = y[2 * q][c >> 1], w1 = y[2 * q + 1][c >> 1];
      a[c][q] = (c & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u)) : ((w0 & 0xffffu) | (w1 << 16));
    }
}

// Stores a wave's finished 64 x 16*NBW tile of S.  The store mode and the
// bounds checks are decided once per tile (interior tiles need none), not
// once per element.
template <int NBW, int MODE>
__device__ __forceinline__ void store_s_tile_mode(const ContractParams& p, const f32x4 (&acc)[kDC][NBW], int64_t d0w,
                                                  int nb0, int g, int i, int ts, bool full) {
  float* const base = MODE == 0 ? p.part + (int64_t)ts * p.part_split : p.S;
  const int64_t ld = MODE == 0 ? 16 * p.NB : p.lds;
#pragma unroll
  for (int c = 0; c < kDC; ++c)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int cc = 16 * (nb0 + nb) + i;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = d0w + (int64_t)kDC * (4 * g + e) + c;
        if (full || (cc < p.r && row < p.d)) {
          float* dst = base + row * ld + cc;
          const float val = acc[c][nb][e] * p.inv_sqrt_r;
          if constexpr (MODE == 0)
            *dst = val;
          else if constexpr (MODE == 1)
            atomicAdd(dst, val);
          else
            *dst += val;
        }
      }
    }
}

template <int NBW>
__device__ __forceinline__ void store_s_tile(const ContractParams& p, const f32x4 (&acc)[kDC][NBW], int64_t d0w,
                                             int nb0, int g, int i, int ts) {
  const bool full = d0w + 16 * kDC <= p.d && 16 * (nb0 + NBW) <= p.r;
  if (p.part) {
    if (full) store_s_tile_mode<NBW, 0>(p, acc, d0w, nb0, g, i, ts, true);
    else store_s_tile_mode<NBW, 0>(p, acc, d0w, nb0, g, i, ts, false);
  } else if (p.atomic_out) {
    if (full) store_s_tile_mode<NBW, 1>(p, acc, d0w, nb0, g, i, ts, true);
    else store_s_tile_mode<NBW, 1>(p, acc, d0w, nb0, g, i, ts, false);
  } else {
    if (full) store_s_tile_mode<NBW, 2>(p, acc, d0w, nb0, g, i, ts, true);
    else store_s_tile_mode<NBW, 2>(p, acc, d0w, nb0, g, i, ts, false);
  }
}

// Adds one finished value of S (the LDS-reduced paths): into the caller's S
// (atomically when several token splits share the tile), or as a plain store
// into the split's partial tile.
__device__ __forceinline__ void put_s(const ContractParams& p, int ts, int64_t row, int cc, float val) {
  if (p.part) {
    p.part[(int64_t)ts * p.part_split + row * (16 * p.NB) + cc] = val;
  } else {
    float* dst = p.S + row * p.lds + cc;
    if (p.atomic_out)
      atomicAdd(dst, val);
    else
      *dst += val;
  }
}

// Stream-K split of a contraction: units are (row tile, 32-token step) pairs;
// the grid takes them in equal contiguous runs, tile-major.  With p.bands = 8
// the steps are first cut into eight token bands, one per XCD (workgroup ids
// are dealt round-robin to the eight XCDs), and an XCD's workgroups share the
// units of its band, so that its L2 holds only that band's rows of P.
struct StreamK {
  int64_t kb0, blen, u_beg, u_end;
  __device__ __forceinline__ StreamK(const ContractParams& p, int64_t nks) {
    // Workgroup ids are dealt to the eight XCDs round-robin: with B = 8 each
    // XCD takes one band, with B = 4 the XCDs b and b + 4 share band b.
    const int B = p.bands;
    const int band = (int)(blockIdx.x % B);
    const int64_t gx = gridDim.x / B;  // workgroups sharing the band
    const int64_t jx = blockIdx.x / B;
    kb0 = nks * band / B;
    blen = nks * (band + 1) / B - kb0;
    const int64_t units = (int64_t)p.n_dt * blen;
    u_beg = units * jx / gx;
    u_end = units * (jx + 1) / gx;
  }
  // The segment of the run that starts at unit u0 (one row tile, a range of
  // steps); advances u0 past it.
  __device__ __forceinline__ void segment(int64_t& u0, int& dt, int64_t& ks_beg, int64_t& ks_end) const {
    dt = (int)(u0 / blen);
    ks_beg = kb0 + (u0 - (int64_t)dt * blen);
    ks_end = min(kb0 + blen, ks_beg + (u_end - u0));
    u0 += ks_end - ks_beg;
  }
};

// Small ranks (NB <= 4): eight waves share 64 rows of S and take every
// eighth 32-token step, with the work split stream-K style (StreamK), so that
// every workgroup does the same number of steps however the tiles divide
// among the CUs.  A run crosses a few tile boundaries at most; the workgroup
// keeps the tile's sums in registers over its part of the run and adds them
// into S whenever the tile changes (atomically, unless the segment is the
// whole tile).  A step's dY rows and P words
// travel together in one ring slot (DEPTH steps in flight), so waiting for
// one step never waits for a later one.  dY comes through a buffer
// descriptor: token rows past T read as zero; columns past d only feed rows
// of S that are not stored.
template <int NB, int DEPTH>
__global__ __launch_bounds__(512) void contract_small_kernel(ContractParams p) {
  constexpr int NW = 8;
  // 16-row blocks of the tile reduced per LDS round (64 KB of partials).
  constexpr int CPR = (kDC * NB * 256 * NW * 4 <= 65536) ? kDC : 65536 / (NB * 256 * NW * 4);
  constexpr int ITEMS = CPR * NB * 64;  // float4 items per wave and round
  __shared__ f32x4 red[NW * ITEMS];

  // The wave index is uniform over the wave: keep it (and all derived
  // addressing) in scalar registers.
  const int lane = threadIdx.x & 63, wt = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, i = lane & 15;
  const int64_t nks = (p.T + 31) >> 5;
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.dY, (uint32_t)(p.T * p.lddy * 2));
  const uint32_t rowstep = (uint32_t)(p.lddy * 2);
  const StreamK sk(p, nks);

  for (int64_t u0 = sk.u_beg; u0 < sk.u_end;) {
    int dt;
    int64_t ks_beg, ks_end;
    sk.segment(u0, dt, ks_beg, ks_end);
    const bool whole = ks_beg == 0 && ks_end == nks;  // no other workgroup adds into this tile

    const int64_t d0w = (int64_t)dt * 16 * kDC;
    const uint32_t coloff = (uint32_t)((d0w + kDC * i) * 2);
    const int64_t ks0 = ks_beg + wt;
    const int nsteps = ks_end > ks0 ? (int)((ks_end - ks0 + NW - 1) / NW) : 0;

    f32x4 acc[kDC][NB];
#pragma unroll
    for (int c = 0; c < kDC; ++c)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[c][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x2 y[DEPTH][8];
    u32x4 bh[DEPTH][NB], bl[DEPTH][NB];
    // Loads are unconditional (steps past the wave's share re-read the
    // segment's last step, which is never used): a load under a branch would
    // make the compiler's wait counts wait for every load in flight.
    auto issue = [&](int slot_y, int m) {
      const int64_t ks = min(ks0 + (int64_t)NW * m, ks_end - 1);
      uint32_t off = (uint32_t)((32 * ks + 8 * g) * p.lddy * 2) + coloff;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[slot_y][e] = buf_load8(ry, off);
        off += rowstep;
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int64_t o = ((ks * p.NB + nb) * 64 + lane) * 8;
        bh[slot_y][nb] = *reinterpret_cast<const u32x4*>(p.Phi + o);
        bl[slot_y][nb] = *reinterpret_cast<const u32x4*>(p.Plo + o);
      }
    };

#pragma unroll
    for (int q = 0; q < DEPTH - 1; ++q) issue(q, q);
    for (int m0 = 0; m0 < nsteps; m0 += DEPTH) {
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        const int m = m0 + u;
        issue((u + DEPTH - 1) % DEPTH, m + DEPTH - 1);
        if (m < nsteps) {
          u32x4 a[kDC];
          transpose_dy(y[u], a);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int c = 0; c < kDC; ++c) {
              acc[c][nb] = mfma_16x16x32(a[c], bh[u][nb], acc[c][nb]);
              acc[c][nb] = mfma_16x16x32(a[c], bl[u][nb], acc[c][nb]);
            }
        }
      }
    }

    // Eight-way sum through LDS, CPR 16-row blocks per round: every wave
    // parks its accumulators as whole float4s (one 1 KB contiguous write per
    // block and column block), then each thread sums one float4 item of all
    // eight waves (contiguous 16-byte reads) and adds its four rows into S.
    static_assert(kDC % CPR == 0, "rounds must cover the tile");
#pragma unroll
    for (int c0 = 0; c0 < kDC; c0 += CPR) {
      __syncthreads();  // the previous round's (or segment's) readers are done
#pragma unroll
      for (int cr = 0; cr < CPR; ++cr)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) red[wt * ITEMS + (cr * NB + nb) * 64 + lane] = acc[c0 + cr][nb];
      __syncthreads();
      for (int v = threadIdx.x; v < ITEMS; v += NW * 64) {
        f32x4 sum = red[v];
#pragma unroll
        for (int q = 1; q < NW; ++q) {
          const f32x4 o = red[q * ITEMS + v];
          sum[0] += o[0]; sum[1] += o[1]; sum[2] += o[2]; sum[3] += o[3];
        }
        const int ln = v & 63, cn = v >> 6;  // lane of the item, (cr, nb) of the item
        const int cr = cn / NB, nb = cn - cr * NB;
        const int gg = ln >> 4, ii = ln & 15;
        const int cc = 16 * nb + ii;
        if (cc < p.r) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t row = d0w + (int64_t)kDC * (4 * gg + e) + c0 + cr;
            if (row < p.d) {
              float* dst = p.S + row * p.lds + cc;
              if (whole)
                *dst += sum[e] * p.inv_sqrt_r;
              else
                atomicAdd(dst, sum[e] * p.inv_sqrt_r);
            }
          }
        }
      }
    }
  }
}

// Larger ranks (NB = 8 or 16): waves split the rows (WM) and the columns (WN)
// of the workgroup's S tile and all work on the same 32-token step; the P
// tile of a step (NB KB of high halves, NB KB of low halves) is loaded once
// per workgroup into a double-buffered LDS stage and shared by all waves.
template <int NB, int WN>
__global__ __launch_bounds__(256) void contract_lds_kernel(ContractParams p) {
  constexpr int NBW = NB / WN;
  constexpr int WM = 4 / WN;
  constexpr int PV = NB * 64;            // u32x4 words per half-tile
  constexpr int PER = 2 * PV / 256;      // u32x4 words each thread moves per step
  __shared__ u32x4 pt[2][2 * PV];
  const int lin = xcd_linear_id(blockIdx.x, gridDim.x);
  const int ts = lin / p.n_dt;
  const int dt = lin - ts * p.n_dt;
  if (ts >= p.n_ts) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, i = lane & 15;
  const int wn = wave % WN, wm = wave / WN;
  const int64_t d0w = (int64_t)dt * WM * 16 * kDC + (int64_t)wm * 16 * kDC;
  const int64_t col = d0w + kDC * i;
  const int64_t nks = (p.T + 31) >> 5;
  const int64_t ks_beg = ts * p.ksp;
  const int64_t ks_end = min(nks, ks_beg + p.ksp);
  const int nsteps = ks_end > ks_beg ? (int)(ks_end - ks_beg) : 0;

  f32x4 acc[kDC][NBW];
#pragma unroll
  for (int c = 0; c < kDC; ++c)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[c][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x2 y[2][8];
  u32x4 stg[PER];
  auto load_y = [&](u32x2 (&slot)[8], int m) {
    const int64_t t = 32 * (ks_beg + m) + 8 * g;
#pragma unroll
    for (int e = 0; e < 8; ++e) slot[e] = load_dy4(p.dY, p.lddy, p.T, p.d, t + e, col);
  };
  // Thread q moves words q, q+256, ... of the step's [hi | lo] tile.
  auto load_p = [&](int m) {
    const int64_t base = (ks_beg + m) * (int64_t)PV;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int w = threadIdx.x + 256 * j;
      const uint16_t* src = (w < PV) ? p.Phi + (base + w) * 8 : p.Plo + (base + w - PV) * 8;
      stg[j] = *reinterpret_cast<const u32x4*>(src);
    }
  };
  auto store_p = [&](int buf) {
#pragma unroll
    for (int j = 0; j < PER; ++j) pt[buf][threadIdx.x + 256 * j] = stg[j];
  };

  if (nsteps > 0) {
    load_p(0);
    load_y(y[0], 0);
    store_p(0);
  }
  __syncthreads();
  for (int m0 = 0; m0 < nsteps; m0 += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int m = m0 + u;
      if (m < nsteps) {
        const bool more = m + 1 < nsteps;
        if (more) {
          load_p(m + 1);
          load_y(y[u ^ 1], m + 1);
        }
        u32x4 a[kDC];
        transpose_dy(y[u], a);
        const u32x4* ph = &pt[u][0];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          const u32x4 bh = ph[(wn * NBW + nb) * 64 + lane];
          const u32x4 bl = ph[PV + (wn * NBW + nb) * 64 + lane];
#pragma unroll
          for (int c = 0; c < kDC; ++c) {
            acc[c][nb] = mfma_16x16x32(a[c], bh, acc[c][nb]);
            acc[c][nb] = mfma_16x16x32(a[c], bl, acc[c][nb]);
          }
        }
        if (more) store_p(u ^ 1);
        __syncthreads();
      }
    }
  }
  store_s_tile<NBW>(p, acc, d0w, wn * NBW, g, i, ts);
}

// Larger ranks on big problems: eight waves, each owning 64 rows x 128
// columns of S (128 accumulator registers, two waves per SIMD); WM = 8/WN row
// groups x WN column groups give a 512 x 128 (r <= 128) or 256 x 256 tile.
// The step's P tile sits in a double-buffered LDS stage shared by all waves;
// every wave loads the dY rows of its row group itself.
template <int NB, int WN, int DP>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void contract_big_kernel(ContractParams p) {
  constexpr int NBW = NB / WN;           // column blocks per wave
  constexpr int WM = 8 / WN;             // row groups
  constexpr int PV = NB * 64;            // u32x4 words per half-tile of a step
  constexpr int PER = 2 * PV / 512;      // u32x4 words each thread moves per step
  __shared__ u32x4 pt[2][2 * PV];
  // Token splits vary fastest among consecutive logical ids, so the
  // workgroups that add into the same S tile share an XCD (and its L2).
  const int lin = xcd_linear_id(blockIdx.x, gridDim.x);
  const int dt = lin / p.n_ts;
  const int ts = lin - dt * p.n_ts;
  if (dt >= p.n_dt) return;

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4, i = lane & 15;
  const int wn = wave % WN, wm = wave / WN;
  const int64_t d0w = ((int64_t)dt * WM + wm) * 16 * kDC;
  const uint32_t coloff = (uint32_t)((d0w + kDC * i) * 2);
  const int64_t nks = (p.T + 31) >> 5;
  const int64_t ks_beg = ts * p.ksp;
  const int64_t ks_end = min(nks, ks_beg + p.ksp);
  const int nsteps = ks_end > ks_beg ? (int)(ks_end - ks_beg) : 0;
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.dY, (uint32_t)(p.T * p.lddy * 2));
  const uint32_t rowstep = (uint32_t)(p.lddy * 2);

  f32x4 acc[kDC][NBW];
#pragma unroll
  for (int c = 0; c < kDC; ++c)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[c][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Prefetch distance DP: the loads of step m + DP are issued while step m is
  // multiplied, and P of step m + 1 goes from registers into the other LDS
  // half at the end of step m, DP - 1 steps after it was requested.
  u32x2 y[DP + 1][8];
  u32x4 stg[DP][PER];
  // Loads are issued unconditionally (a step past the range reloads the
  // last one): a load under a branch makes the compiler's wait counts assume
  // the shortest path, which would wait for every prefetch at each step.
  auto load_y = [&](u32x2 (&slot)[8], int m) {
    m = min(m, nsteps - 1);
    uint32_t off = (uint32_t)((32 * (ks_beg + m) + 8 * g) * p.lddy * 2) + coloff;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      slot[e] = buf_load8(ry, off);
      off += rowstep;
    }
  };
  // Thread q moves words q, q + 512, ... of the step's hi plane, then the
  // same words of its lo plane (PER / 2 of each), through buffer loads
  // (SGPR base, 32-bit offsets: the planes span less than 4 GiB).
  constexpr int PH = PER / 2;
  static_assert(PH * 512 == PV, "whole planes per step");
  const __amdgpu_buffer_rsrc_t rph = make_rsrc(p.Phi, 0xFFFFFFF0u);
  const __amdgpu_buffer_rsrc_t rpl = make_rsrc(p.Plo, 0xFFFFFFF0u);
  auto load_p = [&](u32x4 (&sl)[PER], int m) {
    m = min(m, nsteps - 1);
    const uint32_t base = (uint32_t)(((ks_beg + m) * (int64_t)PV + threadIdx.x) * 16);
#pragma unroll
    for (int j = 0; j < PH; ++j) {
      sl[j] = buf_load16(rph, base + 512 * 16 * j);
      sl[PH + j] = buf_load16(rpl, base + 512 * 16 * j);
    }
  };
  auto store_p = [&](const u32x4 (&sl)[PER], int buf) {
#pragma unroll
    for (int j = 0; j < PH; ++j) {
      pt[buf][threadIdx.x + 512 * j] = sl[j];
      pt[buf][PV + threadIdx.x + 512 * j] = sl[PH + j];
    }
  };

  // Steps 0 .. DP - 1 in flight; step 0 staged.  P of step m lives in
  // stg[m % DP] until it is staged, dY of step m in y[m % (DP + 1)]; the loop
  // body covers DP * (DP + 1) steps so that both indices are constants.
  // Every active workgroup has at least one step (token splits are cut so).
  if (nsteps > 0) {
#pragma unroll
  for (int q = 0; q < DP; ++q) {
    load_p(stg[q], q);
    load_y(y[q], q);
  }
  store_p(stg[0], 0);
  __syncthreads();
  constexpr int L = DP * (DP + 1);
  for (int m0 = 0; m0 < nsteps; m0 += L) {
#pragma unroll
    for (int u = 0; u < L; ++u) {
      const int m = m0 + u;
      load_p(stg[u % DP], m + DP);  // stg[m % DP] was staged at the end of step m - 1
      load_y(y[(u + DP) % (DP + 1)], m + DP);
      if (m < nsteps) {
        u32x4 a[kDC];
        transpose_dy(y[u % (DP + 1)], a);
        const u32x4* ph = &pt[u & 1][0];
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          const u32x4 bh = ph[(wn * NBW + nb) * 64 + lane];
          const u32x4 bl = ph[PV + (wn * NBW + nb) * 64 + lane];
#pragma unroll
          for (int c = 0; c < kDC; ++c) {
            acc[c][nb] = mfma_16x16x32(a[c], bh, acc[c][nb]);
            acc[c][nb] = mfma_16x16x32(a[c], bl, acc[c][nb]);
          }
        }
        if (m + 1 < nsteps) store_p(stg[(u + 1) % DP], (u + 1) & 1);
        __syncthreads();
      }
    }
  }
  }
  store_s_tile<NBW>(p, acc, d0w, wn * NBW, g, i, ts);
}

// Rank 256, two workgroups per CU: the 256 x 256 tile of contract_big_kernel
// cut into two column halves, each a workgroup of four waves (one per SIMD,
// 64 rows x 128 columns each, 128 accumulator registers).  The two
// workgroups on a CU have barriers of their own, so one can multiply while
// the other waits on its loads or its barrier; the two halves of a tile are
// consecutive logical ids (one XCD), so the second read of the tile's dY
// rows comes from L2.
// NB = 8 (ranks 65-128): the same workgroup holds all of P's columns (one
// "half" per tile), two workgroups per CU from different (tile, split) pairs.
// HL = 1: P's high bf16 plane only (the single-bf16 contraction: one MFMA per
// product, no low plane loaded).
template <int DP, int NB, int HL = 2>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void contract_half_kernel(ContractParams p) {
  static_assert(NB == 16 || NB == 8, "two halves of 128 columns, or one");
  static_assert(HL == 1 || HL == 2, "one or two planes of P");
  constexpr int NBW = 8;                 // column blocks per wave (half of the tile)
  constexpr int NHALF = NB / NBW;
  constexpr int PVH = NBW * 64;          // u32x4 words per plane and step for the half
  constexpr int PH = PVH / 256;          // words each thread moves per plane and step
  constexpr int PER = HL * PH;           // words each thread moves per step
  static_assert(PH * 256 == PVH, "whole planes per step");
  __shared__ u32x4 pt[2][HL * PVH];
  const int lin = xcd_linear_id(blockIdx.x, gridDim.x);
  const int half = NHALF == 2 ? (lin & 1) : 0;
  const int rest = NHALF == 2 ? (lin >> 1) : lin;
  const int dt = rest / p.n_ts;
  const int ts = rest - dt * p.n_ts;
  if (dt >= p.n_dt) return;

  const int lane = threadIdx.x & 63, wm = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, i = lane & 15;
  const int64_t d0w = ((int64_t)dt * 4 + wm) * 16 * kDC;
  const uint32_t coloff = (uint32_t)((d0w + kDC * i) * 2);
  const int64_t nks = (p.T + 31) >> 5;
  const int64_t ks_beg = ts * p.ksp;
  const int64_t ks_end = min(nks, ks_beg + p.ksp);
  const int nsteps = ks_end > ks_beg ? (int)(ks_end - ks_beg) : 0;
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.dY, (uint32_t)(p.T * p.lddy * 2));
  const uint32_t rowstep = (uint32_t)(p.lddy * 2);

  f32x4 acc[kDC][NBW];
#pragma unroll
  for (int c = 0; c < kDC; ++c)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[c][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x2 y[DP + 1][8];
  u32x4 stg[DP][PER];
  auto load_y = [&](u32x2 (&slot)[8], int m) {
    m = min(m, nsteps - 1);
    uint32_t off = (uint32_t)((32 * (ks_beg + m) + 8 * g) * p.lddy * 2) + coloff;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      slot[e] = buf_load8(ry, off);
      off += rowstep;
    }
  };
  // The half's column blocks are contiguous within a step of each plane.
  const __amdgpu_buffer_rsrc_t rph = make_rsrc(p.Phi, 0xFFFFFFF0u);
  const __amdgpu_buffer_rsrc_t rpl = make_rsrc(p.Plo, 0xFFFFFFF0u);
  auto load_p = [&](u32x4 (&sl)[PER], int m) {
    m = min(m, nsteps - 1);
    const uint32_t base = (uint32_t)((((ks_beg + m) * NB + NBW * half) * 64 + threadIdx.x) * 16);
#pragma unroll
    for (int j = 0; j < PH; ++j) {
      sl[j] = buf_load16(rph, base + 256 * 16 * j);
      if constexpr (HL == 2) sl[PH + j] = buf_load16(rpl, base + 256 * 16 * j);
    }
  };
  auto store_p = [&](const u32x4 (&sl)[PER], int buf) {
#pragma unroll
    for (int j = 0; j < PH; ++j) {
      pt[buf][threadIdx.x + 256 * j] = sl[j];
      if constexpr (HL == 2) pt[buf][PVH + threadIdx.x + 256 * j] = sl[PH + j];
    }
  };

  if (nsteps > 0) {
#pragma unroll
  for (int q = 0; q < DP; ++q) {
    load_p(stg[q], q);
    load_y(y[q], q);
  }
  store_p(stg[0], 0);
  __syncthreads();
  constexpr int L = DP * (DP + 1);
  for (int m0 = 0; m0 < nsteps; m0 += L) {
#pragma unroll
    for (int u = 0; u < L; ++u) {
      const int m = m0 + u;
      load_p(stg[u % DP], m + DP);
      load_y(y[(u + DP) % (DP + 1)], m + DP);
      // Keep the loads at the top of the step: left to itself the scheduler
      // sinks them below the step's MFMAs (their registers then hold the
      // transposed operands), which halves the prefetch distance.
      __builtin_amdgcn_sched_barrier(0);
      if (m < nsteps) {
        u32x4 a[kDC];
        transpose_dy(y[u % (DP + 1)], a);
        const u32x4* ph = &pt[u & 1][0];
        // Raised issue priority over the step's MFMAs: of the two workgroups
        // sharing each SIMD, the one multiplying keeps the matrix core fed
        // while the other issues its loads and transposes.
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          const u32x4 bh = ph[nb * 64 + lane];
          if constexpr (HL == 2) {
            const u32x4 bl = ph[PVH + nb * 64 + lane];
#pragma unroll
            for (int c = 0; c < kDC; ++c) {
              acc[c][nb] = mfma_16x16x32(a[c], bh, acc[c][nb]);
              acc[c][nb] = mfma_16x16x32(a[c], bl, acc[c][nb]);
            }
          } else {
#pragma unroll
            for (int c = 0; c < kDC; ++c) acc[c][nb] = mfma_16x16x32(a[c], bh, acc[c][nb]);
          }
        }
        __builtin_amdgcn_s_setprio(0);
        if (m + 1 < nsteps) store_p(stg[(u + 1) % DP], (u + 1) & 1);
        __syncthreads();
      }
    }
  }
  }
  store_s_tile<NBW>(p, acc, d0w, NBW * half, g, i, ts);
}

// Rank 256 on large layers: four waves, one per SIMD, each owning 64 rows x
// all 256 columns of the workgroup's 256 x 256 S tile (256 accumulator
// registers, pinned to the AGPR half of the register file).  Every wave
// streams its own rows of dY (no two waves load the same bytes: duplicated
// loads from one CU halve the streaming rate), and the step's P tile (hi
// and, unless HL == 1, lo planes) sits in a two-stage LDS ring written by
// all four waves from registers loaded one step ahead, with one barrier per
// step.  Within a step the B operands of column block nb + 1 are read from
// LDS while the MFMAs of block nb run.  HL == 1 contracts with the high
// bf16 half of P only (one MFMA per product).
template <int HL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1))) void contract_wide_kernel(ContractParams p) {
  constexpr int NB = 16;
  constexpr int PV = NB * 64;      // u32x4 words per plane and step
  constexpr int PW = HL * PV;      // u32x4 words per stage
  constexpr int PER = PW / 256;    // words each thread moves per step
  constexpr int DY = 4;            // dY ring depth (steps): loads go out three steps ahead
  constexpr int DPP = 2;           // P register ring depth: loads go out two steps before staging
  __shared__ u32x4 pt[2][PW];
  const int lin = xcd_linear_id(blockIdx.x, gridDim.x);
  const int dt = lin / p.n_ts;
  const int ts = lin - dt * p.n_ts;
  if (dt >= p.n_dt) return;

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, i = lane & 15;
  const int64_t d0w = (int64_t)dt * 256 + (int64_t)wave * 16 * kDC;
  const uint32_t coloff = (uint32_t)((d0w + kDC * i) * 2);
  const int64_t nks = (p.T + 31) >> 5;
  const int64_t ks_beg = ts * p.ksp;
  const int64_t ks_end = min(nks, ks_beg + p.ksp);
  const int nsteps = ks_end > ks_beg ? (int)(ks_end - ks_beg) : 0;
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.dY, (uint32_t)(p.T * p.lddy * 2));
  const uint32_t rowstep = (uint32_t)(p.lddy * 2);

  f32x4 acc[kDC][NB];
#pragma unroll
  for (int c = 0; c < kDC; ++c)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[c][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Loads are unconditional (steps past the range re-read the last step):
  // a load under a branch would make the compiler's wait counts wait for
  // every load in flight.
  u32x2 y[DY][8];
  auto load_y = [&](u32x2 (&slot)[8], int m) {
    m = min(m, nsteps - 1);
    uint32_t off = (uint32_t)((32 * (ks_beg + m) + 8 * g) * p.lddy * 2) + coloff;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      slot[e] = buf_load8(ry, off);
      off += rowstep;
    }
  };
  // Thread q moves words q, q + 256, ... of the step's [hi | lo] tile.
  u32x4 stg[DPP][PER];
  auto load_p = [&](u32x4 (&sl)[PER], int m) {
    m = min(m, nsteps - 1);
    const int64_t base = (ks_beg + m) * (int64_t)PV;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int w = threadIdx.x + 256 * j;
      const uint16_t* src = (w < PV) ? p.Phi + (base + w) * 8 : p.Plo + (base + w - PV) * 8;
      sl[j] = *reinterpret_cast<const u32x4*>(src);
    }
  };
  auto store_p = [&](const u32x4 (&sl)[PER], int buf) {
#pragma unroll
    for (int j = 0; j < PER; ++j) pt[buf][threadIdx.x + 256 * j] = sl[j];
  };

  // Every active workgroup has at least one step (token splits are cut so).
  // P of step m sits in stg[m % DPP] from step m - 2 (when it is requested)
  // to step m - 1 (when it goes into LDS stage m % 2); dY of step m sits in
  // y[m % DY] from step m - 3.  The loop body covers four steps so that all
  // ring indices are constants.
  static_assert(DY == 4 && DPP == 2, "loop body of four steps");
  if (nsteps > 0) {
    load_p(stg[0], 0);
    load_p(stg[1], 1);
    load_y(y[0], 0);
    load_y(y[1], 1);
    load_y(y[2], 2);
    store_p(stg[0], 0);
    load_p(stg[0], 2);
    __syncthreads();
    for (int m0 = 0; m0 < nsteps; m0 += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int m = m0 + u;
        // P of step m + 1 into the other stage (its readers finished step
        // m - 1 before the last barrier), then request step m + 3 into the
        // freed registers and dY of step m + 3.
        store_p(stg[(u + 1) % DPP], (u + 1) & 1);
        load_p(stg[(u + 1) % DPP], m + 3);
        load_y(y[(u + 3) % DY], m + 3);
        if (m < nsteps) {
          u32x4 a[kDC];
          transpose_dy(y[u % DY], a);
          const u32x4* ph = &pt[u & 1][0];
          u32x4 bh = ph[lane], bl = HL == 2 ? ph[PV + lane] : bh;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            u32x4 nh = bh, nl = bl;
            if (nb + 1 < NB) {
              nh = ph[(nb + 1) * 64 + lane];
              if (HL == 2) nl = ph[PV + (nb + 1) * 64 + lane];
            }
            if (HL == 2)
              mfma4_hl(acc[0][nb], acc[1][nb], acc[2][nb], acc[3][nb], a[0], a[1], a[2], a[3], bh, bl);
            else
              mfma4_b(acc[0][nb], acc[1][nb], acc[2][nb], acc[3][nb], a[0], a[1], a[2], a[3], bh);
            bh = nh;
            bl = nl;
          }
        }
        __syncthreads();
      }
    }
  }
  mfma_drain();
#pragma unroll
  for (int c = 0; c < kDC; ++c)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) mfma_touch(acc[c][nb]);
  store_s_tile<NB>(p, acc, d0w, 0, g, i, ts);
}

// Rank 256 on large layers, eight waves (two per SIMD): wave (wm, wn) owns
// 64 rows x 128 columns of the workgroup's 256 x 256 S tile (128 accumulator
// registers).  Both column halves of a row group need the same dY operands,
// and two waves of one CU loading the same bytes halve the streaming rate;
// so the wn = 0 wave alone loads its rows of dY (three steps ahead),
// transposes them into MFMA operands one step ahead and hands them to its
// wn = 1 partner through LDS, while the wn = 1 waves alone move the step's P
// tile (hi and, unless HL == 1, lo planes; requested two steps ahead) into a
// two-stage LDS ring.  One barrier per step publishes both.
template <int HL>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void contract_share_kernel(ContractParams p) {
  constexpr int NB = 16, WN = 2, WM = 4, NBW = NB / WN;
  constexpr int PV = NB * 64;      // u32x4 words per plane and step
  constexpr int PW = HL * PV;      // u32x4 words per stage
  constexpr int PER = PW / 256;    // words each wn = 1 thread moves per step
  constexpr int DY = 4;            // dY ring of the wn = 0 waves (steps)
  __shared__ u32x4 pt[2][PW];
  __shared__ u32x4 at[2][WM][kDC][64];
  const int lin = xcd_linear_id(blockIdx.x, gridDim.x);
  const int dt = lin / p.n_ts;
  const int ts = lin - dt * p.n_ts;
  if (dt >= p.n_dt) return;

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, i = lane & 15;
  const int wn = wave % WN, wm = wave / WN;
  const int64_t d0w = ((int64_t)dt * WM + wm) * 16 * kDC;
  const int64_t nks = (p.T + 31) >> 5;
  const int64_t ks_beg = ts * p.ksp;
  const int64_t ks_end = min(nks, ks_beg + p.ksp);
  const int nsteps = ks_end > ks_beg ? (int)(ks_end - ks_beg) : 0;

  f32x4 acc[kDC][NBW];
#pragma unroll
  for (int c = 0; c < kDC; ++c)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[c][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const u32x4 (&a)[kDC], int buf) {
    const u32x4* ph = &pt[buf][0];
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const u32x4 bh = ph[(wn * NBW + nb) * 64 + lane];
      if constexpr (HL == 2) {
        const u32x4 bl = ph[PV + (wn * NBW + nb) * 64 + lane];
#pragma unroll
        for (int c = 0; c < kDC; ++c) {
          acc[c][nb] = mfma_16x16x32(a[c], bh, acc[c][nb]);
          acc[c][nb] = mfma_16x16x32(a[c], bl, acc[c][nb]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < kDC; ++c) acc[c][nb] = mfma_16x16x32(a[c], bh, acc[c][nb]);
      }
    }
  };

  // Every active workgroup has at least one step (token splits are cut so).
  // Both branches below run the same number of barriers.  Loads are
  // unconditional (steps past the range re-read the last one): a load under
  // a branch would make the compiler's wait counts wait for every load in
  // flight.
  if (nsteps > 0) {
    if (wn == 0) {
      const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.dY, (uint32_t)(p.T * p.lddy * 2));
      const uint32_t rowstep = (uint32_t)(p.lddy * 2);
      const uint32_t coloff = (uint32_t)((d0w + kDC * i) * 2);
      u32x2 y[DY][8];
      auto load_y = [&](u32x2 (&slot)[8], int m) {
        m = min(m, nsteps - 1);
        uint32_t off = (uint32_t)((32 * (ks_beg + m) + 8 * g) * p.lddy * 2) + coloff;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          slot[e] = buf_load8(ry, off);
          off += rowstep;
        }
      };
#pragma unroll
      for (int q = 0; q < DY - 1; ++q) load_y(y[q], q);
      {
        u32x4 a0[kDC];
        transpose_dy(y[0], a0);
#pragma unroll
        for (int c = 0; c < kDC; ++c) at[0][wm][c][lane] = a0[c];
      }
      __syncthreads();
      for (int m0 = 0; m0 < nsteps; m0 += DY) {
#pragma unroll
        for (int u = 0; u < DY; ++u) {
          const int m = m0 + u;
          load_y(y[(u + DY - 1) % DY], m + DY - 1);
          {
            u32x4 an[kDC];
            transpose_dy(y[(u + 1) % DY], an);  // operands of step m + 1
#pragma unroll
            for (int c = 0; c < kDC; ++c) at[(u + 1) & 1][wm][c][lane] = an[c];
          }
          if (m < nsteps) {
            u32x4 a[kDC];
#pragma unroll
            for (int c = 0; c < kDC; ++c) a[c] = at[u & 1][wm][c][lane];
            compute(a, u & 1);
          }
          __syncthreads();
        }
      }
    } else {
      // Thread q of the wn = 1 waves moves words q, q + 256, ... of the
      // step's [hi | lo] tile.
      const int tq = (wm * 64) + lane;
      u32x4 stg[2][PER];
      auto load_p = [&](u32x4 (&sl)[PER], int m) {
        m = min(m, nsteps - 1);
        const uint16_t* hi = p.Phi + ((ks_beg + m) * (int64_t)PV) * 8;
        const uint16_t* lo = p.Plo + ((ks_beg + m) * (int64_t)PV) * 8;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const int w = tq + 256 * j;  // plane fixed at compile time: PV is a multiple of 256
          sl[j] = *reinterpret_cast<const u32x4*>(j * 256 < PV ? hi + (size_t)w * 8 : lo + (size_t)(w - PV) * 8);
        }
      };
      auto store_p = [&](const u32x4 (&sl)[PER], int buf) {
#pragma unroll
        for (int j = 0; j < PER; ++j) pt[buf][tq + 256 * j] = sl[j];
      };
      load_p(stg[0], 0);
      load_p(stg[1], 1);
      store_p(stg[0], 0);
      load_p(stg[0], 2);
      __syncthreads();
      for (int m0 = 0; m0 < nsteps; m0 += DY) {
#pragma unroll
        for (int u = 0; u < DY; ++u) {
          const int m = m0 + u;
          // P of step m + 1 into the other stage (its readers finished step
          // m - 1 before the last barrier), then request step m + 3.
          store_p(stg[(u + 1) & 1], (u + 1) & 1);
          load_p(stg[(u + 1) & 1], m + 3);
          if (m < nsteps) {
            u32x4 a[kDC];
#pragma unroll
            for (int c = 0; c < kDC; ++c) a[c] = at[u & 1][wm][c][lane];
            compute(a, u & 1);
          }
          __syncthreads();
        }
      }
    }
  }
  store_s_tile<NBW>(p, acc, d0w, wn * NBW, g, i, ts);
}

// General tiling for larger ranks: NW waves arranged as WM row groups (64
// rows of S each) x WN column groups (16*NB/WN columns each) x WT token lanes.
// A wave takes every WT-th 32-token step of the workgroup's token range and
// loads its own dY rows and P operands (DEPTH steps in flight, no LDS stage
// and no barrier in the main loop); the WT token-lane partials of each tile
// are summed through LDS at the end.  Small per-workgroup S tiles keep the
// token splits (and so the atomic adds into S) few, at the price of reading
// P from L2 once per 64*WM rows.
template <int NB, int WM, int WN, int NW, int DEPTH>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void contract_tile_kernel(ContractParams p) {
  constexpr int WT = NW / (WM * WN);
  constexpr int NBW = NB / WN;
  static_assert(WT * WM * WN == NW, "wave arrangement");
  // LDS rounds of CPR 16-row blocks: every wave parks CPR x NBW float4 items
  // per lane (64 KB in all).
  constexpr int CPR = (kDC * NBW * 64 * NW * 16 <= 65536) ? kDC : 65536 / (NBW * 64 * NW * 16);
  constexpr int ITEMS = CPR * NBW * 64;  // float4 items per wave and round
  static_assert(CPR >= 1 && kDC % CPR == 0, "rounds must cover the tile");
  __shared__ f32x4 red[WT > 1 ? NW * ITEMS : 1];

  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = lane >> 4, i = lane & 15;
  const int wt = w % WT, wn = (w / WT) % WN, wm = w / (WT * WN);
  const int64_t nks = (p.T + 31) >> 5;
  const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.dY, (uint32_t)(p.T * p.lddy * 2));
  const uint32_t rowstep = (uint32_t)(p.lddy * 2);
  const StreamK sk(p, nks);

  for (int64_t u0 = sk.u_beg; u0 < sk.u_end;) {
    int dt;
    int64_t ks_beg, ks_end;
    sk.segment(u0, dt, ks_beg, ks_end);
    const bool whole = ks_beg == 0 && ks_end == nks;  // no other workgroup adds into this tile

    const int64_t d0w = ((int64_t)dt * WM + wm) * 16 * kDC;
    const uint32_t coloff = (uint32_t)((d0w + kDC * i) * 2);
    const int64_t ks0 = ks_beg + wt;
    const int nsteps = ks_end > ks0 ? (int)((ks_end - ks0 + WT - 1) / WT) : 0;

    f32x4 acc[kDC][NBW];
#pragma unroll
    for (int c = 0; c < kDC; ++c)
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) acc[c][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x2 y[DEPTH][8];
    u32x4 bh[DEPTH][NBW], bl[DEPTH][NBW];
    // Unconditional loads, as in contract_small_kernel.
    auto issue = [&](int slot, int m) {
      const int64_t ks = min(ks0 + (int64_t)WT * m, ks_end - 1);
      uint32_t off = (uint32_t)((32 * ks + 8 * g) * p.lddy * 2) + coloff;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[slot][e] = buf_load8(ry, off);
        off += rowstep;
      }
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const int64_t o = ((ks * p.NB + wn * NBW + nb) * 64 + lane) * 8;
        bh[slot][nb] = *reinterpret_cast<const u32x4*>(p.Phi + o);
        bl[slot][nb] = *reinterpret_cast<const u32x4*>(p.Plo + o);
      }
    };

#pragma unroll
    for (int q = 0; q < DEPTH - 1; ++q) issue(q, q);
    for (int m0 = 0; m0 < nsteps; m0 += DEPTH) {
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        const int m = m0 + u;
        issue((u + DEPTH - 1) % DEPTH, m + DEPTH - 1);
        if (m < nsteps) {
          u32x4 a[kDC];
          transpose_dy(y[u], a);
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
            for (int c = 0; c < kDC; ++c) {
              acc[c][nb] = mfma_16x16x32(a[c], bh[u][nb], acc[c][nb]);
              acc[c][nb] = mfma_16x16x32(a[c], bl[u][nb], acc[c][nb]);
            }
        }
      }
    }

    if constexpr (WT == 1) {
      if (whole) store_s_tile_mode<NBW, 2>(p, acc, d0w, wn * NBW, g, i, 0, d0w + 16 * kDC <= p.d && 16 * (wn + 1) * NBW <= p.r);
      else store_s_tile_mode<NBW, 1>(p, acc, d0w, wn * NBW, g, i, 0, d0w + 16 * kDC <= p.d && 16 * (wn + 1) * NBW <= p.r);
    } else {
      // Sum the WT token lanes of every (row group, column group) through
      // LDS, CPR 16-row blocks per round, as whole float4s (contiguous 1 KB
      // writes and reads).
#pragma unroll
      for (int c0 = 0; c0 < kDC; c0 += CPR) {
        __syncthreads();  // the previous round's (or segment's) readers are done
#pragma unroll
        for (int cr = 0; cr < CPR; ++cr)
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb) red[w * ITEMS + (cr * NBW + nb) * 64 + lane] = acc[c0 + cr][nb];
        __syncthreads();
        for (int v = threadIdx.x; v < (NW / WT) * ITEMS; v += NW * 64) {
          const int gm = v / ITEMS, rest = v - gm * ITEMS;  // gm = wm * WN + wn
          f32x4 sum = red[(gm * WT) * ITEMS + rest];
#pragma unroll
          for (int q = 1; q < WT; ++q) {
            const f32x4 o = red[(gm * WT + q) * ITEMS + rest];
            sum[0] += o[0]; sum[1] += o[1]; sum[2] += o[2]; sum[3] += o[3];
          }
          const int ln = rest & 63, cn = rest >> 6;  // lane, (cr, nb) of the item
          const int cr = cn / NBW, nb = cn - cr * NBW;
          const int gg = ln >> 4, ii = ln & 15;
          const int cc = 16 * ((gm % WN) * NBW + nb) + ii;
          if (cc < p.r) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int64_t row = ((int64_t)dt * WM + gm / WN) * 16 * kDC + (int64_t)kDC * (4 * gg + e) + c0 + cr;
              if (row < p.d) {
                float* dst = p.S + row * p.lds + cc;
                if (whole)
                  *dst += sum[e] * p.inv_sqrt_r;
                else
                  atomicAdd(dst, sum[e] * p.inv_sqrt_r);
              }
            }
          }
        }
      }
    }
  }
}

// S[row][c] += sum over token splits of part[ts][row][c]; one thread per four
// columns of a row.
__global__ __launch_bounds__(256) void sketch_reduce_kernel(ContractParams p, int n_ts) {
  const int RP = 16 * p.NB;
  const int nq = (p.r + 3) >> 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / nq;
  if (row >= p.d) return;
  const int c0 = 4 * (int)(idx - row * nq);
  const float* src = p.part + row * RP + c0;
  // Four splits' loads in flight at a time.
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0, s2 = s0, s3 = s0;
  int t = 0;
  for (; t + 4 <= n_ts; t += 4) {
    s0 += *reinterpret_cast<const f32x4*>(src + (int64_t)t * p.part_split);
    s1 += *reinterpret_cast<const f32x4*>(src + (int64_t)(t + 1) * p.part_split);
    s2 += *reinterpret_cast<const f32x4*>(src + (int64_t)(t + 2) * p.part_split);
    s3 += *reinterpret_cast<const f32x4*>(src + (int64_t)(t + 3) * p.part_split);
  }
  for (; t < n_ts; ++t) s0 += *reinterpret_cast<const f32x4*>(src + (int64_t)t * p.part_split);
  const f32x4 sum = (s0 + s1) + (s2 + s3);
  float* dst = p.S + row * p.lds + c0;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (c0 + e < p.r) dst[e] += sum[e];
}

// ===========================================================================
// Host: plans and launchers.
// ===========================================================================
namespace {
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int pow2_blocks(int r) {
  const int nb = (r + 15) / 16;
  int q = 1;
  while (q < nb) q <<= 1;
  return q;
}
}  // namespace

size_t projection_cache_bytes(int64_t T, int r) {
  return (size_t)cache_tokens(T) * 16 * pow2_blocks(r) * 4;
}

void scratch_layout(SketchPlan& pl, int64_t d, bool proj_part, bool con_part) {
  const size_t RP = 16 * (size_t)pl.NB;
  size_t off = 0;
  pl.off_phi = pl.off_plo = 0;
  pl.off_part = off;
  if (proj_part && pl.n_k > 1) off += align_up((size_t)pl.n_k * pl.Tpad * RP * 4, 256);
  pl.off_cpart = off;
  if (con_part && pl.use_part) off += align_up((size_t)pl.n_ts * d * RP * 4, 256);
  pl.total = off;
}

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return (s && *s) ? atoi(s) : dflt;
}

SketchPlan plan_sketch(int64_t T, int64_t k, int64_t d, int r, bool det, bool hi_only) {
  SketchPlan pl{};
  pl.NB = pow2_blocks(r);
  const int RP = 16 * pl.NB;
  pl.ncb = (int)((k + 255) / 256);
  const int64_t T32 = (T + 31) / 32 * 32;

  // Projection.  Ranks above 64 with at least two 256-column blocks: the
  // LDS-staged kernel (64-token tiles, two waves per SIMD; against the same
  // tiling with X loaded in the MFMA operand's layout, 27B layers 70 -> 57
  // (attention), 70 -> 59 (up), 191 -> 155 us (down), 7B down at r = 128
  // 81 -> 71 us).  Small r*k otherwise: the whole k range's signs fit in
  // 64 KB of LDS.
  // The LDS-staged projection above rank 64; at ranks 33-64 only for long k
  // (7B layers at r = 64: 3584 columns 18.8 -> 18.1 us, 18944 columns
  // 65.4 -> 61.1 us; at 1536 columns the other kernels win, 6.9 against 9.9).
  pl.pwide = ((pl.NB >= 8 && pl.ncb >= 2) || (pl.NB == 4 && pl.ncb >= 14)) ? 1 : 0;
  pl.pwide = env_int("LOGRA_PROJ_WIDE", pl.pwide) != 0 && pl.NB >= 4 ? 1 : 0;
  pl.small_proj = (!pl.pwide && (size_t)RP * pl.ncb * 36 <= 65536 && pl.NB <= 8) ? 1 : 0;
  pl.small_proj = pl.pwide ? 0 : env_int("LOGRA_PROJ_SMALL", pl.small_proj);
  int64_t TT;
  if (pl.pwide) {
    // 64-token tiles; column splits across workgroups (powers of two, so
    // that a tile's splits are consecutive ids on one XCD) until there is a
    // workgroup per CU, each split at least one round of two blocks.
    TT = 64;
    pl.WK = 4;
    pl.MBW = 4;
    pl.n_tt = (int)((T32 + TT - 1) / TT);
    const int rounds = (pl.ncb + 3) / 4;
    int nk = 1;
    while (nk < 8 && (int64_t)pl.n_tt * nk < 256 && 2 * nk <= rounds + 1) nk *= 2;  // at least ~a round per split
    nk = env_int("LOGRA_PROJ_NK", nk);
    if (nk != 1 && nk != 2 && nk != 4 && nk != 8) nk = 1;
    const int rounds_per = (rounds + nk - 1) / nk;
    pl.cbs_per = 4 * rounds_per;
    pl.n_k = (pl.ncb + pl.cbs_per - 1) / pl.cbs_per;
    // the grid must keep each tile's splits on one XCD: n_k a power of two
    // dividing the per-XCD share (the launch rounds the grid up to 8 * n_k)
    while (pl.n_k & (pl.n_k - 1)) ++pl.n_k;
  } else if (pl.small_proj) {
    // More tokens per workgroup amortise the signs; keep >= 256 workgroups.
    int MBW = 4;
    while (MBW > 1 && (MBW * pl.NB > 16 || (T32 + 16 * MBW - 1) / (16 * MBW) < 256)) MBW >>= 1;
    MBW = env_int("LOGRA_PROJ_MB", MBW);
    pl.MBW = MBW;
    pl.WK = 8;
    TT = 16 * MBW;
    pl.n_tt = (int)((T32 + TT - 1) / TT);
    pl.n_k = 1;
    pl.cbs_per = pl.ncb;
  } else {
    // Four waves along k (WK) sharing one token tile, so that each expanded
    // sign operand feeds MBW MFMAs and the grid still has a few hundred
    // workgroups of 32-64 tokens; MBW keeps the accumulators within 128
    // registers (two waves per SIMD).
    int WK = pl.ncb >= 4 ? 4 : (pl.ncb >= 2 ? 2 : 1);
    int MBW = pl.NB >= 8 ? 2 : 32 / pl.NB;
    if (MBW > 4) MBW = 4;
    if (MBW < 1) MBW = 1;
    auto tiles = [&](int mbw, int wk) { return (T32 + (4 / wk) * 16 * mbw - 1) / ((4 / wk) * 16 * mbw); };
    // (rank >= 128 keeps two token blocks per wave and splits k instead)
    while (pl.NB < 8 && MBW > 1 && tiles(MBW, WK) < 512) MBW >>= 1;
    MBW = env_int("LOGRA_PROJ_MB", MBW);
    WK = env_int("LOGRA_PROJ_WK", WK);
    // Eight-wave workgroups (two token rows) halve the sign generation per
    // token at rank >= 128, where Philox costs more than the expansion: for
    // long rows, and for long microbatches, where 64-token tiles still give
    // 256 workgroups without column splits (16384 tokens x 5120 columns at
    // r = 256: 79 -> 71 us; 8192-token microbatches of 3584 columns gained
    // nothing).
    int NW = env_int("LOGRA_PROJ_NW", (k >= 8192 || T32 >= 16384) ? 8 : 4) == 8 ? 8 : 4;
    if (NW == 8 && !(pl.NB >= 8 && MBW == 2 && WK >= 2)) NW = 4;
    pl.PNW = NW;
    pl.MBW = MBW;
    pl.WK = WK;
    TT = (NW / WK) * 16 * MBW;
    // The contraction reads whole 32-token steps of P: cover them all, so the
    // tokens in [T, Tpad) hold P = 0 written by the projection (X reads as 0).
    pl.n_tt = (int)((T32 + TT - 1) / TT);
    // Column splits across workgroups (fp32 partials, last arriver sums) until
    // there are two waves per SIMD: 512 four-wave or 256 eight-wave groups.
    const int64_t want = NW == 8 ? 256 : 512;
    int64_t nk = 1;
    if (pl.n_tt < want) nk = (want + pl.n_tt - 1) / pl.n_tt;
    const int64_t rounds = (pl.ncb + WK - 1) / WK;
    if (nk > rounds) nk = rounds;
    nk = env_int("LOGRA_PROJ_NK", (int)nk);
    if (nk < 1) nk = 1;
    const int64_t rounds_per = (rounds + nk - 1) / nk;
    pl.cbs_per = (int)(rounds_per * WK);
    pl.n_k = (int)((pl.ncb + pl.cbs_per - 1) / pl.cbs_per);
  }
  pl.Tpad = pl.n_tt * TT;

  // Contraction.
  const int64_t nks = T32 / 32;
  int64_t BD, min_steps;
  if (pl.NB <= 4) {
    // Eight waves on every eighth step of 64 rows, stream-K over steps; at
    // NB = 4 the token-lane tiles of 128 or 256 rows (WM = 2, 4) are the
    // alternative: P is re-read from L2 half or a quarter as often, for more
    // atomic adds into S per step.  They pay off only for tall S (18944 x
    // 3584 at r = 64: 99.6 -> 93.1 us per 8192-token call; 1536- and
    // 3584-row layers ran 0-35 % slower).
    const int tile4 = (pl.NB == 4 && !det) ? env_int("LOGRA_CON_TILE", d >= 8192 ? 1 : 0) : 0;
    if (tile4) {
      int wm = env_int("LOGRA_CON_WM", 2);
      if (wm != 1 && wm != 2 && wm != 4) wm = 2;
      pl.WM = wm;
      pl.cvar = 5;
      BD = 16 * kDC * wm;
    } else {
      pl.cvar = 0;
      BD = 16 * kDC;
    }
    min_steps = 16;
  } else {
    // Eight-wave tiles (512 x 128 or 256 x 256) where they still give a few
    // hundred workgroups; the four-wave tiles otherwise.
    // Token-lane tiles (64 rows per workgroup, few token splits) unless the
    // rank is 256 and the microbatch long: there every 64-row tile would read
    // eight times the dY bytes in P, and the 256 x 256 tiles win.
    const int64_t bd8 = pl.NB == 8 ? 8 * 16 * kDC : 4 * 16 * kDC;
    // Large d: the 512 x 128 / 256 x 256 tiles read P from L2 only d/bd8
    // times and, with at least 36 row tiles, need only a few token splits.
    const bool tall = (d + bd8 - 1) / bd8 >= 36;
    pl.few_ts = tall ? 1 : 0;
    const int tile = det ? 1 : env_int("LOGRA_CON_TILE", tall ? 0 : ((pl.NB == 8 || T <= 8192) ? 1 : 0));
    const int big = env_int("LOGRA_CON_BIG", tall ? 1 : -1);
    const bool use_big = big >= 0 ? big != 0 : ((d + bd8 - 1) / bd8) * (nks / 16) >= 256;
    // The half tiles also beat the token-lane tiles on shorter S: 3584-row
    // layers at 8192 tokens, 58-66 -> 49 us above rank 128 and 37 -> 32.5 us
    // at rank 128 (at 1536 rows, 20 -> 26 us: not taken there).
    const int64_t span = ((d + bd8 - 1) / bd8) * (nks / 16);
    const bool half_short = pl.NB == 16 ? span >= 128 : span >= 96;
    // Rank 256 on large layers: the one-wave-per-SIMD 256 x 256 tiles.
    // (With P as a hi/lo pair contract_big_kernel is as fast; the shared-
    // operand kernel serves the single-bf16 contraction, also on the shorter
    // S where the half tiles serve the hi/lo one: 7B q at r = 256 81 -> 73 us
    // per sketch call, 7B down 151 -> 141 us.)
    const int wide = (!det && pl.NB == 16)
                         ? env_int("LOGRA_CON_WIDE", (hi_only && (tall || use_big || half_short)) ? 1 : 0)
                         : 0;
    // Otherwise the 256 x 256 tiles as two 256 x 128 workgroups per CU
    // (27B up layer 336 -> 314 us, attention 110 -> 105, 7B up 185 -> 174).
    // At NB = 8 one such workgroup holds the whole rank: used where the
    // 512 x 128 tiles would be too few for a round (1.5B up layer, r = 128:
    // 78.8 -> 67.1 us); on tall S (7B up) the 512 x 128 tiles stay ahead
    // (105.6 against 111.1 us).
    const int halfk = (!det && !wide && (tall || use_big || half_short))
                          ? env_int("LOGRA_CON_HALF", (pl.NB == 16 || !tall) ? 1 : 0)
                          : 0;
    if (halfk) {
      pl.cvar = 7;  // contract_half_kernel: 256 x 128 workgroups, two per CU
      BD = 256;
    } else if (wide) {
      pl.cvar = 6;
      pl.cwide = wide;  // 1: contract_share_kernel (eight waves), 2: contract_wide_kernel (four)
      BD = 256;
    } else if (tile) {
      // NB = 8: 2 column groups; NB = 16: 4 column groups; WM row groups.
      const int wn = pl.NB / 4;
      int wm = det ? 1 : env_int("LOGRA_CON_WM", 1);
      if (wm < 1 || wm * wn > 8) wm = 1;
      pl.WM = wm;
      pl.cvar = 5;
      BD = 16 * kDC * wm;
    } else if (use_big) {
      pl.cvar = pl.NB == 8 ? 3 : 4;
      BD = bd8;
    } else if (pl.NB == 8) {
      pl.cvar = 1;  // WN = 1, WM = 4
      BD = 4 * 16 * kDC;
    } else {
      pl.cvar = 2;  // WN = 2, WM = 2
      BD = 2 * 16 * kDC;
    }
    min_steps = 16;
  }
  pl.n_dt = (int)((d + BD - 1) / BD);
  int64_t n_ts = (384 + pl.n_dt - 1) / pl.n_dt;
  int64_t max_ts = nks / min_steps;
  if (max_ts < 1) max_ts = 1;
  if (pl.cvar == 6) {
    // One round of one workgroup per CU at most.
    n_ts = 256 / pl.n_dt;
    if (n_ts < 1) n_ts = 1;
  } else if (pl.cvar == 7) {
    // One round of two workgroups per CU at most (at NB = 16 the two column
    // halves of a tile).
    n_ts = 512 / ((pl.NB / 8) * pl.n_dt);
    if (n_ts < 1) n_ts = 1;
    if (n_ts > 8 && pl.few_ts) n_ts = 8;
    // At NB = 16, at least 32 steps per workgroup: shorter splits spend more
    // on the prologue and the partial tiles than the fuller grid gains
    // (3584-row layers at 8192 tokens: 16 splits 53 us, 8 splits 49 us).
    if (pl.NB == 16 && n_ts > nks / 32) n_ts = nks / 32 > 1 ? nks / 32 : 1;
  } else if (pl.cvar >= 3 && pl.few_ts) {
    n_ts = 256 / pl.n_dt;  // one round of 256 eight-wave workgroups at most
    if (n_ts < 1) n_ts = 1;
    if (n_ts > 8) n_ts = 8;
  } else if (pl.cvar >= 3) {
    // One eight-wave workgroup per CU (256 on MI355X): fill whole rounds of
    // the chip, preferring fewer token splits (less atomic traffic into S).
    double best = 0.0;
    for (int R = 1; R <= 4; ++R) {
      int64_t t = (256 * R) / pl.n_dt;
      if (t < 1) t = 1;
      if (t > max_ts) t = max_ts;
      const double eff = (double)(pl.n_dt * t) / (256.0 * ((pl.n_dt * t + 255) / 256));
      if (eff > best + 0.05) {
        best = eff;
        n_ts = t;
      }
    }
  }
  if (n_ts > max_ts) n_ts = max_ts;
  n_ts = env_int("LOGRA_CON_TS", (int)n_ts);
  if (n_ts < 1) n_ts = 1;
  pl.ksp = (nks + n_ts - 1) / n_ts;
  pl.n_ts = (int)((nks + pl.ksp - 1) / pl.ksp);
  if (pl.n_ts < 1) pl.n_ts = 1;
  if (pl.cvar == 0 || pl.cvar == 5) {
    // Stream-K with one eight-wave workgroup per CU at most.  When eight
    // token bands of at least 16 steps times the row tiles fit in one round
    // (n_dt * 8 <= 256), every workgroup takes exactly one (tile, band) pair
    // and each XCD's L2 holds only its band's eighth of P; otherwise one band
    // over 256 workgroups (runs that straddle tiles cost one more set of
    // atomic adds each, and many tiles per band would cut every run up).
    const int64_t units = (int64_t)pl.n_dt * nks;
    // Four bands (one per pair of XCDs) when eight do not fit one round but
    // four do, at r <= 128: 3584-row layers at r = 64 and 128 took 4-7 %
    // less than with one band over 256 workgroups; at r = 256 no gain.
    int bands = 1;
    if (nks >= 128 && pl.n_dt * 8 <= 256) bands = 8;
    else if (nks >= 128 && pl.n_dt * 4 <= 256 && pl.NB <= 8) bands = 4;
    pl.cbands = env_int("LOGRA_CON_BANDS", bands);
    if (pl.cbands != 4 && pl.cbands != 8) pl.cbands = 1;
    int64_t grid = pl.cbands > 1 ? (int64_t)pl.cbands * pl.n_dt : 256;
    grid = env_int("LOGRA_CON_GRID", (int)grid);
    if (grid > units / 8) grid = units / 8;
    if (pl.cbands > 1) grid = grid / pl.cbands * pl.cbands;
    if (grid < 1) {
      grid = 1;
      pl.cbands = 1;
    }
    pl.cgrid = (int)grid;
    if (det) {
      // One workgroup per row tile over all the tokens: every S element is
      // summed in one fixed order and stored without atomic adds.
      pl.cbands = 1;
      pl.cgrid = pl.n_dt;
      pl.n_ts = 1;
      pl.ksp = nks;
    }
  }

  // Split counters (one per token tile) live in a region of their own that
  // nothing else writes (the kernels leave them at zero); see n_counters.
  pl.n_counters = pl.n_k > 1 ? pl.n_tt : 0;
  size_t off = 0;
  pl.off_phi = off;
  off += align_up((size_t)pl.Tpad * RP * 2, 256);
  pl.off_plo = off;
  off += align_up((size_t)pl.Tpad * RP * 2, 256);
  pl.off_part = off;
  if (pl.n_k > 1) off += align_up((size_t)pl.n_k * pl.Tpad * RP * 4, 256);
  // Token splits of the large-rank tilings store partial tiles (a plain,
  // coalesced stream) that one small kernel sums into S: L2 retires fp32
  // atomic adds at about one element per channel and clock.  The half-tile
  // contraction at three splits (the tall 17408- and 18944-row layers) is
  // the exception: there the atomic adds overlap the other half's MFMA work
  // and the extra pass over the partials costs more (27B up 311 -> 300 us).
  const bool part_default = pl.cvar == 7 ? pl.n_ts >= 4 : (pl.n_ts >= 3 || pl.cvar >= 6);
  pl.use_part = !det && env_int("LOGRA_CON_PART", part_default ? 1 : 0) && pl.n_ts > 1 &&
                (pl.cvar == 3 || pl.cvar == 4 || pl.cvar == 6 || pl.cvar == 7);
  pl.bigdp = env_int("LOGRA_CON_BIGDP", 2) == 1 ? 1 : 2;
  pl.off_cpart = off;
  if (pl.use_part) off += align_up((size_t)pl.n_ts * d * RP * 4, 256);
  pl.total = off;
  return pl;
}

bool proj_launch(const SketchPlan& pl, const ProjParams& p, hipStream_t s) {
  if (pl.pwide) {
    const int grid = (int)align_up((size_t)pl.n_tt * pl.n_k, (size_t)8 * pl.n_k);
    if (pl.NB == 16) hipLaunchKernelGGL((proj_lds_kernel<16>), dim3(grid), dim3(512), 0, s, p);
    else if (pl.NB == 8) hipLaunchKernelGGL((proj_lds_kernel<8>), dim3(grid), dim3(512), 0, s, p);
    else if (pl.NB == 4) hipLaunchKernelGGL((proj_lds_kernel<4>), dim3(grid), dim3(512), 0, s, p);
    else return false;
    return true;
  }
  if (pl.small_proj) {
    const size_t shm = proj_small_lds_bytes(pl.NB, pl.ncb);
#define LOGRA_PSMALL(nb, mb)                                                                       \
    if (pl.NB == nb && pl.MBW == mb) {                                                             \
      hipLaunchKernelGGL((proj_small_kernel<nb, mb>), dim3(pl.n_tt), dim3(512), shm, s, p);       \
      return true;                                                                                 \
    }
    LOGRA_PSMALL(1, 1) LOGRA_PSMALL(1, 2) LOGRA_PSMALL(1, 4)
    LOGRA_PSMALL(2, 1) LOGRA_PSMALL(2, 2) LOGRA_PSMALL(2, 4)
    LOGRA_PSMALL(4, 1) LOGRA_PSMALL(4, 2) LOGRA_PSMALL(4, 4)
    LOGRA_PSMALL(8, 1) LOGRA_PSMALL(8, 2)
#undef LOGRA_PSMALL
    return false;
  }
  const int grid = (int)align_up((size_t)pl.n_tt * pl.n_k, 8);
#define LOGRA_PROJ(nb, mb, wk)                                                                \
  if (pl.NB == nb && pl.MBW == mb && pl.WK == wk && pl.PNW == 4) {                            \
    hipLaunchKernelGGL((proj_kernel<nb, mb, wk, 4>), dim3(grid), dim3(256), 0, s, p);         \
    return true;                                                                              \
  }
#define LOGRA_PROJ8(nb, mb, wk)                                                               \
  if (pl.NB == nb && pl.MBW == mb && pl.WK == wk && pl.PNW == 8) {                            \
    hipLaunchKernelGGL((proj_kernel<nb, mb, wk, 8>), dim3(grid), dim3(512), 0, s, p);         \
    return true;                                                                              \
  }
  LOGRA_PROJ(1, 1, 1) LOGRA_PROJ(1, 2, 1) LOGRA_PROJ(1, 4, 1)
  LOGRA_PROJ(1, 1, 2) LOGRA_PROJ(1, 2, 2) LOGRA_PROJ(1, 4, 2)
  LOGRA_PROJ(1, 1, 4) LOGRA_PROJ(1, 2, 4) LOGRA_PROJ(1, 4, 4)
  LOGRA_PROJ(2, 1, 1) LOGRA_PROJ(2, 2, 1) LOGRA_PROJ(2, 4, 1)
  LOGRA_PROJ(2, 1, 2) LOGRA_PROJ(2, 2, 2) LOGRA_PROJ(2, 4, 2)
  LOGRA_PROJ(2, 1, 4) LOGRA_PROJ(2, 2, 4) LOGRA_PROJ(2, 4, 4)
  LOGRA_PROJ(4, 1, 1) LOGRA_PROJ(4, 2, 1) LOGRA_PROJ(4, 4, 1)
  LOGRA_PROJ(4, 1, 2) LOGRA_PROJ(4, 2, 2) LOGRA_PROJ(4, 4, 2)
  LOGRA_PROJ(4, 1, 4) LOGRA_PROJ(4, 2, 4) LOGRA_PROJ(4, 4, 4)
  LOGRA_PROJ(8, 1, 1) LOGRA_PROJ(8, 2, 1)
  LOGRA_PROJ(8, 1, 2) LOGRA_PROJ(8, 2, 2)
  LOGRA_PROJ(16, 1, 1) LOGRA_PROJ(16, 2, 1) LOGRA_PROJ(16, 1, 2) LOGRA_PROJ(16, 2, 2)
  LOGRA_PROJ(16, 1, 4) LOGRA_PROJ(16, 2, 4) LOGRA_PROJ(8, 1, 4) LOGRA_PROJ(8, 2, 4)
  LOGRA_PROJ8(8, 2, 2) LOGRA_PROJ8(8, 2, 4) LOGRA_PROJ8(16, 2, 2) LOGRA_PROJ8(16, 2, 4)
#undef LOGRA_PROJ8
#undef LOGRA_PROJ
  return false;
}

void reduce_launch(const SketchPlan& pl, const ContractParams& p, hipStream_t s) {
  const int64_t n = p.d * ((p.r + 3) / 4);
  hipLaunchKernelGGL(sketch_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, pl.n_ts);
}

bool contract_launch(const SketchPlan& pl, const ContractParams& p, hipStream_t s) {
  const int grid = (int)align_up((size_t)pl.n_dt * pl.n_ts, 8);
  switch (pl.cvar) {
    case 0:
      if (pl.NB == 1) hipLaunchKernelGGL((contract_small_kernel<1, 3>), dim3(pl.cgrid), dim3(512), 0, s, p);
      else if (pl.NB == 2) hipLaunchKernelGGL((contract_small_kernel<2, 3>), dim3(pl.cgrid), dim3(512), 0, s, p);
      else hipLaunchKernelGGL((contract_small_kernel<4, 2>), dim3(pl.cgrid), dim3(512), 0, s, p);
      return true;
    case 1:
      hipLaunchKernelGGL((contract_lds_kernel<8, 1>), dim3(grid), dim3(256), 0, s, p);
      return true;
    case 2:
      hipLaunchKernelGGL((contract_lds_kernel<16, 2>), dim3(grid), dim3(256), 0, s, p);
      return true;
    case 3:
      if (pl.bigdp == 2) hipLaunchKernelGGL((contract_big_kernel<8, 1, 2>), dim3(grid), dim3(512), 0, s, p);
      else hipLaunchKernelGGL((contract_big_kernel<8, 1, 1>), dim3(grid), dim3(512), 0, s, p);
      return true;
    case 4:
      if (pl.bigdp == 2) hipLaunchKernelGGL((contract_big_kernel<16, 2, 2>), dim3(grid), dim3(512), 0, s, p);
      else hipLaunchKernelGGL((contract_big_kernel<16, 2, 1>), dim3(grid), dim3(512), 0, s, p);
      return true;
    case 7:
      if (pl.NB == 16 && p.hi_only)
        hipLaunchKernelGGL((contract_half_kernel<2, 16, 1>), dim3((unsigned)align_up((size_t)pl.n_dt * pl.n_ts * 2, 8)),
                           dim3(256), 0, s, p);
      else if (pl.NB == 16)
        hipLaunchKernelGGL((contract_half_kernel<2, 16>), dim3((unsigned)align_up((size_t)pl.n_dt * pl.n_ts * 2, 8)),
                           dim3(256), 0, s, p);
      else if (pl.NB == 8 && p.hi_only)
        hipLaunchKernelGGL((contract_half_kernel<2, 8, 1>), dim3((unsigned)align_up((size_t)pl.n_dt * pl.n_ts, 8)),
                           dim3(256), 0, s, p);
      else if (pl.NB == 8)
        hipLaunchKernelGGL((contract_half_kernel<2, 8>), dim3((unsigned)align_up((size_t)pl.n_dt * pl.n_ts, 8)),
                           dim3(256), 0, s, p);
      else
        return false;
      return true;
    case 6:
      if (pl.cwide == 2) {
        if (p.hi_only) hipLaunchKernelGGL((contract_wide_kernel<1>), dim3(grid), dim3(256), 0, s, p);
        else hipLaunchKernelGGL((contract_wide_kernel<2>), dim3(grid), dim3(256), 0, s, p);
      } else {
        if (p.hi_only) hipLaunchKernelGGL((contract_share_kernel<1>), dim3(grid), dim3(512), 0, s, p);
        else hipLaunchKernelGGL((contract_share_kernel<2>), dim3(grid), dim3(512), 0, s, p);
      }
      return true;
    case 5: {
#define LOGRA_CT(nb, wm, wn)                                                                          \
      if (pl.NB == nb && pl.WM == wm) {                                                               \
        hipLaunchKernelGGL((contract_tile_kernel<nb, wm, wn, 8, 2>), dim3(pl.cgrid), dim3(512), 0, s, p); \
        return true;                                                                                  \
      }
      LOGRA_CT(4, 1, 1) LOGRA_CT(4, 2, 1) LOGRA_CT(4, 4, 1)
      LOGRA_CT(8, 1, 2) LOGRA_CT(8, 2, 2) LOGRA_CT(8, 4, 2) LOGRA_CT(16, 1, 4) LOGRA_CT(16, 2, 4)
#undef LOGRA_CT
      return false;
    }
  }
  return false;
}

}  // namespace logra
