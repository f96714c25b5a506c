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
// Projection.  A workgroup owns TT = (4/WK)*16*MBW tokens and the 256-column
// blocks [cbb, cbe) of k.  Its WK wave columns take the blocks of one "round"
// side by side; the 4/WK wave rows take different tokens.  Each round the
// workgroup regenerates the signs of the next round's blocks into LDS while
// it multiplies the current ones, and every wave keeps X loads for the next
// seven 32-column steps in flight in a register ring.
// ===========================================================================
template <int NB, int MBW, int WK>
__global__ __launch_bounds__(256) void proj_kernel(ProjParams p) {
  constexpr int RP = 16 * NB;
  constexpr int WT = 4 / WK;
  constexpr int TT = WT * 16 * MBW;
  constexpr int SROW = 9;  // 8 dwords of sign bits + 1 pad dword (bank spread)
  constexpr int NGEN = (RP * WK + 255) / 256;
  constexpr int RED = WK > 1 ? (WK - 1) * WT * NB * 256 : 4;
  __shared__ uint32_t sbits[2][WK * RP * SROW];
  __shared__ float red[RED];
  __shared__ int s_last;

  const int lin = xcd_linear_id(blockIdx.x, gridDim.x);
  const int tt = lin / p.n_k;
  const int ksp = lin - tt * p.n_k;
  if (tt >= p.n_tt) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
      const int b = threadIdx.x + 256 * q;
      if (b < RP * WK) {
        const int row = b % RP, wkk = b / RP;
        const int cb = cbb + j * WK + wkk;
        if (cb < cbe) {
          uint32_t w[8];
          philox_sign_block(p.seed, (uint32_t)row, (uint32_t)cb, w);
          uint32_t* dst = &sbits[buf][(wkk * RP + row) * SROW];
#pragma unroll
          for (int e = 0; e < 8; ++e) dst[e] = w[e];
        }
      }
    }
  };

  u32x4 xr[8][MBW];
  auto issue = [&](u32x4 (&slot)[MBW], int cb, int s) {
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb)
      slot[mb] = (cb < cbe) ? load_x8(p.X, p.ldx, p.T, p.k, tw + 16 * mb + i, (int64_t)cb * 256 + 32 * s + 8 * g)
                            : u32x4{0u, 0u, 0u, 0u};
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
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s == 0)
        issue(xr[7], cb, 7);
      else
        issue(xr[s - 1], cb + WK, s - 1);
      if (cb < cbe) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint32_t dw = sb[16 * nb * SROW + s];
          const u32x4 bsg = signs_to_bf16x8((dw >> (8 * g)) & 0xffu);
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
          uint32_t h[4], l[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) split_hi_lo(acc[mb][nb][e], h[e], l[e]);
          *reinterpret_cast<u32x2*>(p.Phi + e0) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
          *reinterpret_cast<u32x2*>(p.Plo + e0) = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
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
  for (int v = threadIdx.x; v < TT * RP / 4; v += 256) {
    const int col = v % RP;
    const int64_t tq = t0 + 4 * (int64_t)(v / RP);
    const int64_t e0 = pk_index(tq, col, NB);
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < p.n_k; ++sp) {
      const uint32_t off = (uint32_t)(((int64_t)sp * p.part_stride + e0) * 4);
      sum += __builtin_bit_cast(f32x4, load16_agent(rs, off));
    }
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split_hi_lo(sum[e], h[e], l[e]);
    *reinterpret_cast<u32x2*>(p.Phi + e0) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
    *reinterpret_cast<u32x2*>(p.Plo + e0) = u32x2{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
  }
  if (threadIdx.x == 0) p.counters[tt] = 0u;
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

template <int NBW>
__device__ __forceinline__ void store_s_tile(const ContractParams& p, f32x4 (&acc)[kDC][NBW], int64_t d0w,
                                             int nb0, int g, int i) {
#pragma unroll
  for (int c = 0; c < kDC; ++c)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int cc = 16 * (nb0 + nb) + i;
      if (cc >= p.r) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = d0w + (int64_t)kDC * (4 * g + e) + c;
        if (row >= p.d) continue;
        float* dst = p.S + row * p.lds + cc;
        const float val = acc[c][nb][e] * p.inv_sqrt_r;
        if (p.atomic_out)
          atomicAdd(dst, val);
        else
          *dst += val;
      }
    }
}

// Small ranks (NB <= 4): the four waves of a workgroup share 64 rows of S and
// take every fourth 32-token step of the workgroup's token range.  Each wave
// keeps three steps of dY and one step of P in flight.
template <int NB>
__global__ __launch_bounds__(256) void contract_small_kernel(ContractParams p) {
  constexpr int WT = 4;
  __shared__ float red[(WT - 1) * NB * 256];
  const int lin = xcd_linear_id(blockIdx.x, gridDim.x);
  const int ts = lin / p.n_dt;
  const int dt = lin - ts * p.n_dt;
  if (ts >= p.n_ts) return;

  const int lane = threadIdx.x & 63, wt = threadIdx.x >> 6;
  const int g = lane >> 4, i = lane & 15;
  const int64_t d0w = (int64_t)dt * 16 * kDC;
  const int64_t col = d0w + kDC * i;
  const int64_t nks = (p.T + 31) >> 5;
  const int64_t ks_beg = ts * p.ksp;
  const int64_t ks_end = min(nks, ks_beg + p.ksp);
  const int64_t ks0 = ks_beg + wt;
  const int nsteps = ks_end > ks0 ? (int)((ks_end - ks0 + WT - 1) / WT) : 0;

  f32x4 acc[kDC][NB];
#pragma unroll
  for (int c = 0; c < kDC; ++c)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[c][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x2 y[4][8];
  u32x4 bh[2][NB], bl[2][NB];
  auto load_y = [&](u32x2 (&slot)[8], int m) {
    const int64_t t = 32 * (ks0 + (int64_t)WT * m) + 8 * g;
#pragma unroll
    for (int e = 0; e < 8; ++e) slot[e] = load_dy4(p.dY, p.lddy, p.T, p.d, t + e, col);
  };
  auto load_b = [&](u32x4 (&h)[NB], u32x4 (&l)[NB], int m) {
    const int64_t ks = ks0 + (int64_t)WT * m;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int64_t off = ((ks * p.NB + nb) * 64 + lane) * 8;
      h[nb] = *reinterpret_cast<const u32x4*>(p.Phi + off);
      l[nb] = *reinterpret_cast<const u32x4*>(p.Plo + off);
    }
  };

#pragma unroll
  for (int q = 0; q < 3; ++q)
    if (q < nsteps) load_y(y[q], q);
  if (nsteps > 0) load_b(bh[0], bl[0], 0);

  for (int m0 = 0; m0 < nsteps; m0 += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int m = m0 + u;
      if (m < nsteps) {
        if (m + 3 < nsteps) load_y(y[(u + 3) & 3], m + 3);
        if (m + 1 < nsteps) load_b(bh[(u + 1) & 1], bl[(u + 1) & 1], m + 1);
        u32x4 a[kDC];
        transpose_dy(y[u], a);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int c = 0; c < kDC; ++c) {
            acc[c][nb] = mfma_16x16x32(a[c], bh[u & 1][nb], acc[c][nb]);
            acc[c][nb] = mfma_16x16x32(a[c], bl[u & 1][nb], acc[c][nb]);
          }
      }
    }
  }

  // Sum the four waves' partials through LDS, one 16-row block at a time.
#pragma unroll
  for (int c = 0; c < kDC; ++c) {
    if (wt > 0) {
      float* dst = red + (wt - 1) * NB * 256;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(nb * 4 + e) * 64 + lane] = acc[c][nb][e];
    }
    __syncthreads();
    if (wt == 0) {
#pragma unroll
      for (int w = 1; w < WT; ++w) {
        const float* src = red + (w - 1) * NB * 256;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[c][nb][e] += src[(nb * 4 + e) * 64 + lane];
      }
    }
    __syncthreads();
  }
  if (wt == 0) store_s_tile<NB>(p, acc, d0w, 0, g, i);
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
  store_s_tile<NBW>(p, acc, d0w, wn * NBW, g, i);
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

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return (s && *s) ? atoi(s) : dflt;
}

SketchPlan plan_sketch(int64_t T, int64_t k, int64_t d, int r) {
  SketchPlan pl{};
  pl.NB = pow2_blocks(r);
  const int RP = 16 * pl.NB;
  pl.ncb = (int)((k + 255) / 256);

  // Projection: waves along k (WK) so that RP*WK <= 256 sign blocks per round;
  // MBW keeps the accumulators within 128 registers.
  int WK = RP >= 256 ? 1 : (RP >= 128 ? 2 : 4);
  if (WK > pl.ncb) WK = pl.ncb >= 2 ? 2 : 1;
  int MBW = 32 / pl.NB;
  if (MBW > 4) MBW = 4;
  if (MBW < 1) MBW = 1;
  // Fewer tokens per workgroup while that still leaves < 2 workgroups per CU.
  auto tiles = [&](int mbw, int wk) { return (T + (4 / wk) * 16 * mbw - 1) / ((4 / wk) * 16 * mbw); };
  while (MBW > 1 && tiles(MBW, WK) < 512) MBW >>= 1;
  MBW = env_int("LOGRA_PROJ_MB", MBW);
  WK = env_int("LOGRA_PROJ_WK", WK);
  pl.MBW = MBW;
  pl.WK = WK;
  const int64_t TT = (4 / WK) * 16 * MBW;
  // The contraction reads whole 32-token steps of P: cover them all, so the
  // tokens in [T, Tpad) hold P = 0 written by the projection (X reads as 0).
  const int64_t T32 = (T + 31) / 32 * 32;
  pl.n_tt = (int)((T32 + TT - 1) / TT);
  pl.Tpad = pl.n_tt * TT;
  int64_t nk = 1;
  if (pl.n_tt < 256) nk = (256 + pl.n_tt - 1) / pl.n_tt;
  const int64_t rounds = (pl.ncb + WK - 1) / WK;
  if (nk > rounds) nk = rounds;
  nk = env_int("LOGRA_PROJ_NK", (int)nk);
  if (nk < 1) nk = 1;
  const int64_t rounds_per = (rounds + nk - 1) / nk;
  pl.cbs_per = (int)(rounds_per * WK);
  pl.n_k = (int)((pl.ncb + pl.cbs_per - 1) / pl.cbs_per);

  // Contraction.
  const int64_t nks = (T + 31) / 32;
  int64_t BD;
  if (pl.NB <= 4) {
    pl.cvar = 0;
    BD = 16 * kDC;
  } else if (pl.NB == 8) {
    pl.cvar = 1;  // WN = 1, WM = 4
    BD = 4 * 16 * kDC;
  } else {
    pl.cvar = 2;  // WN = 2, WM = 2
    BD = 2 * 16 * kDC;
  }
  pl.n_dt = (int)((d + BD - 1) / BD);
  const int64_t min_steps = pl.cvar == 0 ? 16 : 16;  // 32-token steps per workgroup
  int64_t n_ts = (512 + pl.n_dt - 1) / pl.n_dt;
  int64_t max_ts = nks / min_steps;
  if (max_ts < 1) max_ts = 1;
  if (n_ts > max_ts) n_ts = max_ts;
  n_ts = env_int("LOGRA_CON_TS", (int)n_ts);
  if (n_ts < 1) n_ts = 1;
  pl.ksp = (nks + n_ts - 1) / n_ts;
  pl.n_ts = (int)((nks + pl.ksp - 1) / pl.ksp);
  if (pl.n_ts < 1) pl.n_ts = 1;

  size_t off = 0;
  pl.off_counters = off;
  off += align_up((size_t)pl.n_tt * sizeof(unsigned), 256);
  pl.off_phi = off;
  off += align_up((size_t)pl.Tpad * RP * 2, 256);
  pl.off_plo = off;
  off += align_up((size_t)pl.Tpad * RP * 2, 256);
  pl.off_part = off;
  if (pl.n_k > 1) off += align_up((size_t)pl.n_k * pl.Tpad * RP * 4, 256);
  pl.total = off;
  return pl;
}

bool proj_launch(const SketchPlan& pl, const ProjParams& p, hipStream_t s) {
  const int grid = (int)align_up((size_t)pl.n_tt * pl.n_k, 8);
#define LOGRA_PROJ(nb, mb, wk)                                                            \
  if (pl.NB == nb && pl.MBW == mb && pl.WK == wk) {                                       \
    hipLaunchKernelGGL((proj_kernel<nb, mb, wk>), dim3(grid), dim3(256), 0, s, p);        \
    return true;                                                                          \
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
  LOGRA_PROJ(8, 1, 1) LOGRA_PROJ(8, 2, 1) LOGRA_PROJ(8, 4, 1)
  LOGRA_PROJ(8, 1, 2) LOGRA_PROJ(8, 2, 2) LOGRA_PROJ(8, 4, 2)
  LOGRA_PROJ(16, 1, 1) LOGRA_PROJ(16, 2, 1)
#undef LOGRA_PROJ
  return false;
}

bool contract_launch(const SketchPlan& pl, const ContractParams& p, hipStream_t s) {
  const int grid = (int)align_up((size_t)pl.n_dt * pl.n_ts, 8);
  switch (pl.cvar) {
    case 0:
      if (pl.NB == 1) hipLaunchKernelGGL((contract_small_kernel<1>), dim3(grid), dim3(256), 0, s, p);
      else if (pl.NB == 2) hipLaunchKernelGGL((contract_small_kernel<2>), dim3(grid), dim3(256), 0, s, p);
      else hipLaunchKernelGGL((contract_small_kernel<4>), dim3(grid), dim3(256), 0, s, p);
      return true;
    case 1:
      hipLaunchKernelGGL((contract_lds_kernel<8, 1>), dim3(grid), dim3(256), 0, s, p);
      return true;
    case 2:
      hipLaunchKernelGGL((contract_lds_kernel<16, 2>), dim3(grid), dim3(256), 0, s, p);
      return true;
  }
  return false;
}

}  // namespace logra
