// RowAdam row scaling and the sign dump (gfx950).
//
// RowAdam: "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
// Sketches", appendix B, equation 15.  Per row i of S (d x r):
//   v_i <- beta2 v_i + (1 - beta2) mean_j S_ij^2,  vh_i = v_i / (1 - beta2^t),
//   Ut_i = S_i / (sqrt(vh_i) + eps),  eps = max(eps_rel * mean_i sqrt(vh_i), 1e-30),
//   U = Ut * ||S||_F / ||Ut||_F  (0 when ||Ut||_F = 0).
// The stabiliser statistic (mean over rows) and the norm (Frobenius) are
// this library's readings of words the appendix text lost.
#include "logra_device.h"
#include "logra_internal.h"

namespace logra {

// Rows go to groups of L lanes (L = the smallest power of two >= r/4, at
// most 64), so a wave covers 64/L rows at a time; with 16-byte aligned rows
// and r % 4 == 0 each lane moves float4s.  Three grid-wide kernels: (1) per
// row m_i, the v_i update, sqrt(vh_i) and ||S_i||^2, plus per-block float64
// sums of sqrt(vh) and ||S_i||^2; (2) every block re-sums those partials in a
// fixed order (so every block holds the same eps), then adds
// ||S_i||^2 / (sqrt(vh_i) + eps)^2 over its rows into a second set of
// partials; (3) every block re-sums both sets the same way, forms
// f = ||S|| / ||Ut|| and rescales its rows by f / (sqrt(vh_i) + eps).  Up to
// 2048 rows the second kernel is folded into the third.  All sums are in a
// fixed order: the result is deterministic.
struct RowGroup {
  int L, lane_in_row;
  int64_t row_in_wave;
};

__device__ __forceinline__ double block_sum_256(double x, double* sh) {
  sh[threadIdx.x] = x;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  const double out = sh[0];
  __syncthreads();
  return out;
}

// Fixed-order sum of n values spaced `stride` apart (every block that calls
// it with the same arguments gets the same bits).  Each thread adds its
// values in increasing order; eight loads are issued before their adds so
// that a long list does not wait out one memory latency per value.
__device__ __forceinline__ double sum_partials(const double* p, int n, int stride, double* sh) {
  double a = 0.0;
  int j = threadIdx.x;
  for (; j + 256 * 7 < n; j += 256 * 8) {
    double v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = p[(int64_t)(j + 256 * q) * stride];
#pragma unroll
    for (int q = 0; q < 8; ++q) a += v[q];
  }
  for (; j < n; j += 256) a += p[(int64_t)j * stride];
  return block_sum_256(a, sh);
}

template <bool VEC>
__global__ __launch_bounds__(256) void rowadam_rows_kernel(const float* S, int64_t lds, float* v, int64_t d, int r,
                                                          int L, float beta2, double inv_bias, float* root,
                                                          float* ssq, double* partial) {
  __shared__ double sh[256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & (L - 1);
  const int rpw = 64 / L;                      // rows per wave and pass
  const int64_t rpb = 4 * (int64_t)rpw;        // rows per block and pass
  double sum_root = 0.0, sum_ssq = 0.0;
  for (int64_t base = (int64_t)blockIdx.x * rpb; base < d; base += (int64_t)gridDim.x * rpb) {
    const int64_t row = base + wave * rpw + lane / L;
    float q = 0.f;
    if (row < d) {
      const float* src = S + row * lds;
      if constexpr (VEC) {
        for (int j = 4 * sub; j < r; j += 4 * L) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(src + j);
          q = __fmaf_rn(x[0], x[0], q);
          q = __fmaf_rn(x[1], x[1], q);
          q = __fmaf_rn(x[2], x[2], q);
          q = __fmaf_rn(x[3], x[3], q);
        }
      } else {
        for (int j = sub; j < r; j += L) q = __fmaf_rn(src[j], src[j], q);
      }
    }
    for (int off = L >> 1; off > 0; off >>= 1) q += __shfl_xor(q, off, 64);
    if (sub == 0 && row < d) {
      const float m = q / (float)r;
      const float vn = beta2 * v[row] + (1.f - beta2) * m;
      const float rt = (float)sqrt((double)vn * inv_bias);
      v[row] = vn;
      root[row] = rt;
      ssq[row] = q;
      sum_root += (double)rt;
      sum_ssq += (double)q;
    }
  }
  const double a = block_sum_256(sum_root, sh);
  const double b = block_sum_256(sum_ssq, sh);
  if (threadIdx.x == 0) {
    partial[2 * blockIdx.x] = a;
    partial[2 * blockIdx.x + 1] = b;
  }
}

// eps from the mean of the row roots and ||S||^2, both from the row
// kernel's block partials in a fixed order (every block gets the same bits;
// block 0 stores them in fin[0], fin[1]), then this block's share of
// ||U~||^2 = sum_i ||S_i||^2 / (sqrt(vh_i) + eps)^2 into fin[2 + block].
__global__ __launch_bounds__(256) void rowadam_norm_kernel(const double* partial, int nparts, const float* root,
                                                          const float* ssq, int64_t d, float eps_rel, double* fin) {
  __shared__ double sh[256];
  const double sum_root = sum_partials(partial, nparts, 2, sh);
  const double eps = fmax((double)eps_rel * (sum_root / (double)d), 1e-30);
  double c = 0.0;
  for (int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x; row < d; row += (int64_t)gridDim.x * 256) {
    const double den = (double)root[row] + eps;
    c += (double)ssq[row] / (den * den);
  }
  const double t = block_sum_256(c, sh);
  if (blockIdx.x == 0) {
    const double norm_s2 = sum_partials(partial + 1, nparts, 2, sh);
    if (threadIdx.x == 0) {
      fin[0] = eps;
      fin[1] = norm_s2;
    }
  }
  if (threadIdx.x == 0) fin[2 + blockIdx.x] = t;
}

// FUSED (few rows): every block works eps and the factor out itself from
// the row kernel's nparts block partials (one launch fewer); otherwise it
// reads eps and ||S||^2 from fin and sums the nparts norm partials after them.
template <bool VEC, bool FUSED>
__global__ __launch_bounds__(256) void rowadam_apply_kernel(float* S, int64_t lds, int64_t d, int r, int L,
                                                           const float* root, const float* ssq,
                                                           const double* partial, int nparts,
                                                           const double* fin, float eps_rel, float* rowmul) {
  double eps, fac;
  if constexpr (FUSED) {
    __shared__ double sh[256];
    const double sum_root = sum_partials(partial, nparts, 2, sh);
    const double norm_s2 = sum_partials(partial + 1, nparts, 2, sh);
    eps = fmax((double)eps_rel * (sum_root / (double)d), 1e-30);
    double c = 0.0;
    for (int64_t row = threadIdx.x; row < d; row += 256) {
      const double den = (double)root[row] + eps;
      c += (double)ssq[row] / (den * den);
    }
    const double norm_u2 = block_sum_256(c, sh);
    fac = norm_u2 > 0.0 ? sqrt(norm_s2 / norm_u2) : 0.0;
  } else {
    __shared__ double sh[256];
    eps = fin[0];
    const double norm_u2 = sum_partials(fin + 2, nparts, 1, sh);
    fac = norm_u2 > 0.0 ? sqrt(fin[1] / norm_u2) : 0.0;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & (L - 1);
  const int rpw = 64 / L;
  const int64_t rpb = 4 * (int64_t)rpw;
  for (int64_t base = (int64_t)blockIdx.x * rpb; base < d; base += (int64_t)gridDim.x * rpb) {
    const int64_t row = base + wave * rpw + lane / L;
    if (row >= d) continue;
    const float f = (float)(fac / ((double)root[row] + eps));
    if (rowmul) {
      // Folded into the merge: the row factor only (the merge multiplies
      // each S entry by it in fp32, exactly as below).
      if (sub == 0) rowmul[row] = f;
      continue;
    }
    float* dst = S + row * lds;
    if constexpr (VEC) {
      for (int j = 4 * sub; j < r; j += 4 * L) {
        f32x4 x = *reinterpret_cast<const f32x4*>(dst + j);
        x[0] *= f; x[1] *= f; x[2] *= f; x[3] *= f;
        *reinterpret_cast<f32x4*>(dst + j) = x;
      }
    } else {
      for (int j = sub; j < r; j += L) dst[j] *= f;
    }
  }
}

void rowadam_launch(float* S, int64_t lds, float* v, int64_t d, int r, float beta2, double inv_bias, float eps_rel,
                    float* root, float* ssq, double* partial, double* partial2, hipStream_t s, float* rowmul) {
  const bool vec = (((uintptr_t)S & 15) == 0) && (lds % 4 == 0) && (r % 4 == 0);
  int L = 1;
  while (L < 64 && 4 * L < r) L <<= 1;  // float4 lanes per row (the scalar path uses the same grouping)
  // One pass over the rows per block where the block cap allows: the row
  // statistics are latency-bound (a row's load, its reduction, then v).
  const int64_t rpb = 4 * (int64_t)(64 / L);
  int64_t blocks = (d + rpb - 1) / rpb;
  if (blocks > kRowAdamBlocks) blocks = kRowAdamBlocks;
  if (vec)
    hipLaunchKernelGGL(rowadam_rows_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, S, lds, v, d, r, L, beta2,
                       inv_bias, root, ssq, partial);
  else
    hipLaunchKernelGGL(rowadam_rows_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, S, lds, v, d, r, L, beta2,
                       inv_bias, root, ssq, partial);
  // Up to 2048 rows every rescale block works out eps and the factor itself
  // (at most 16 KB of L2 reads per block) and the middle kernel is skipped:
  // 1536 rows at r = 64 take 11.1 us instead of 12.7.
  if (d <= 2048) {
    if (vec)
      hipLaunchKernelGGL((rowadam_apply_kernel<true, true>), dim3((unsigned)blocks), dim3(256), 0, s, S, lds, d, r, L,
                         root, ssq, partial, (int)blocks, partial2, eps_rel, rowmul);
    else
      hipLaunchKernelGGL((rowadam_apply_kernel<false, true>), dim3((unsigned)blocks), dim3(256), 0, s, S, lds, d, r, L,
                         root, ssq, partial, (int)blocks, partial2, eps_rel, rowmul);
    return;
  }
  int64_t nblocks = (d + 255) / 256;
  if (nblocks > 256) nblocks = 256;
  hipLaunchKernelGGL(rowadam_norm_kernel, dim3((unsigned)nblocks), dim3(256), 0, s, partial, (int)blocks, root, ssq, d,
                     eps_rel, partial2);
  if (vec)
    hipLaunchKernelGGL((rowadam_apply_kernel<true, false>), dim3((unsigned)blocks), dim3(256), 0, s, S, lds, d, r, L,
                       root, ssq, partial, (int)nblocks, partial2, eps_rel, rowmul);
  else
    hipLaunchKernelGGL((rowadam_apply_kernel<false, false>), dim3((unsigned)blocks), dim3(256), 0, s, S, lds, d, r, L,
                       root, ssq, partial, (int)nblocks, partial2, eps_rel, rowmul);
}

// Signs s (r x k) as int8 +-1; one thread per (row, 256-column block).
__global__ __launch_bounds__(256) void signs_kernel(uint64_t seed, int r, int64_t k, int8_t* out) {
  const int64_t ncb = (k + 255) >> 8;
  const int64_t total = (int64_t)r * ncb;
  for (int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x; id < total; id += (int64_t)gridDim.x * 256) {
    const int row = (int)(id / ncb);
    const int64_t cb = id - (int64_t)row * ncb;
    uint32_t w[8];
    philox_sign_block(seed, (uint32_t)row, (uint32_t)cb, w);
    const int64_t c0 = cb * 256;
    for (int j = 0; j < 256 && c0 + j < k; ++j)
      out[(int64_t)row * k + c0 + j] = ((w[j >> 5] >> (j & 31)) & 1u) ? (int8_t)-1 : (int8_t)1;
  }
}

void signs_launch(uint64_t seed, int r, int64_t k, int8_t* out, hipStream_t s) {
  const int64_t total = (int64_t)r * ((k + 255) / 256);
  int grid = (int)((total + 255) / 256);
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(signs_kernel, dim3(grid), dim3(256), 0, s, seed, r, k, out);
}

// Streaming read of n16 16-byte words (a measurement aid: the read ceiling
// for the same bytes a sketch call streams).  Four words per thread are in
// flight; the xor of everything reaches *sink only for one value, so no load
// can be dropped.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                          uint32_t* sink) {
  const int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  u32x4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t idx = base + 256 * u;
    v[u] = idx < n16 ? src[idx] : u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  if (acc == 0x9E3779B9u) *sink = acc;
}

void stream_read_launch(const void* ptr, int64_t n16, uint32_t* sink, hipStream_t s) {
  const int64_t grid = (n16 + 1023) / 1024;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     static_cast<const u32x4*>(ptr), n16, sink);
}

// Zero fill of n16 16-byte words (a kernel rather than a memset node, so that
// a caller may capture the call in a HIP graph).
__global__ __launch_bounds__(256) void zero_fill_kernel(u32x4* __restrict__ dst, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256)
    dst[i] = u32x4{0u, 0u, 0u, 0u};
}

void zero_fill_launch(void* dst, int64_t n16, hipStream_t s) {
  int64_t grid = (n16 + 255) / 256;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)grid), dim3(256), 0, s, static_cast<u32x4*>(dst), n16);
}

// Payload packing (the sync payload of the merge: header, entries, factors).
// Block row j copies factor j (d_j x r fp32, row stride ldu_j) into its
// packed slot (row stride r) and zeroes the slot's 256-byte tail; block
// (0, 0) also writes the header and entry words from the kernel arguments
// and zeroes the rest of the header region, so every byte of the payload is
// defined.
__global__ __launch_bounds__(256) void payload_pack_kernel(PayloadPackArgs a, uint8_t* __restrict__ payload) {
  const int j = blockIdx.y;
  if (blockIdx.x == 0 && j == 0) {
    uint32_t* hw = reinterpret_cast<uint32_t*>(payload);
    for (int w = threadIdx.x; w < a.header_words; w += 256) hw[w] = w < a.n_head_words ? a.head[w] : 0u;
  }
  const int64_t n = a.d[j] * a.r;            // floats of the factor
  const int64_t span = a.span[j] / 4;        // floats of its slot (256-byte multiple)
  float* dst = reinterpret_cast<float*>(payload + a.off[j]);
  const float* src = a.U[j];
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < span; e += (int64_t)gridDim.x * 256) {
    float v = 0.f;
    if (e < n) {
      const int64_t row = e / a.r;
      v = src[row * a.ldu[j] + (e - row * a.r)];
    }
    dst[e] = v;
  }
}

void payload_pack_launch(const PayloadPackArgs& a, void* payload, hipStream_t s) {
  int64_t most = 1;
  for (int j = 0; j < a.count; ++j) most = a.span[j] / 4 > most ? a.span[j] / 4 : most;
  int64_t gx = (most + 255) / 256;
  if (gx > 1024) gx = 1024;
  if (gx < 1) gx = 1;
  hipLaunchKernelGGL(payload_pack_kernel, dim3((unsigned)gx, (unsigned)a.count), dim3(256), 0, s, a,
                     static_cast<uint8_t*>(payload));
}

// Gaussian basis planes (see GaussBasisParams).  One thread per (row, block
// of eight columns); with col_major the rows of a block are consecutive
// threads (the At stores coalesce), otherwise the blocks of a row are.
__global__ __launch_bounds__(256) void gauss_basis_kernel(GaussBasisParams p, int col_major) {
  const int64_t nblk = p.kpad / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)p.RP * nblk) return;
  int i;
  int64_t b;
  if (col_major) {
    b = idx / p.RP;
    i = (int)(idx - b * p.RP);
  } else {
    i = (int)(idx / nblk);
    b = idx - (int64_t)i * nblk;
  }
  float z[8];
  if (i < p.rr && 8 * b < p.k) {
    gauss_block(p.seed, (uint32_t)(p.row0 + i), (uint64_t)b, z);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (8 * b + e >= p.k) z[e] = 0.f;
  if (p.Z && i < p.rr) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (8 * b + e < p.k) p.Z[(int64_t)i * p.k + 8 * b + e] = z[e];
  }
  uint32_t h[4], l[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) split_hi_lo2(z[2 * q], z[2 * q + 1], h[q], l[q]);
  if (p.Ahi) {
    const int64_t o = (int64_t)i * p.kpad + 8 * b;
    *reinterpret_cast<u32x4*>(p.Ahi + o) = u32x4{h[0], h[1], h[2], h[3]};
    *reinterpret_cast<u32x4*>(p.Alo + o) = u32x4{l[0], l[1], l[2], l[3]};
  }
  if (p.Athi) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t o = (8 * b + e) * p.RP + i;
      p.Athi[o] = (uint16_t)(h[e >> 1] >> (16 * (e & 1)));
      p.Atlo[o] = (uint16_t)(l[e >> 1] >> (16 * (e & 1)));
    }
  }
}

void gauss_basis_launch(const GaussBasisParams& p, hipStream_t s) {
  const int64_t n = (int64_t)p.RP * (p.kpad / 8);
  const int64_t grid = (n + 255) / 256;
  hipLaunchKernelGGL(gauss_basis_kernel, dim3((unsigned)(grid > 0 ? grid : 1)), dim3(256), 0, s, p,
                     p.Athi ? 1 : 0);
}

}  // namespace logra
