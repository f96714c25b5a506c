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

// One wave per row: m_i, the v_i update and sqrt(vh_i); per-workgroup fp64
// sums of sqrt(vh) and of ||S_i||^2 into partial[2*block .. 2*block+1].
__global__ __launch_bounds__(256) void rowadam_rows_kernel(const float* S, int64_t lds, float* v, int64_t d,
                                                          int r, float beta2, double inv_bias, float* root,
                                                          float* ssq, double* partial) {
  __shared__ double sh[2][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double sum_root = 0.0, sum_ssq = 0.0;
  for (int64_t row = (int64_t)blockIdx.x * 4 + wave; row < d; row += (int64_t)gridDim.x * 4) {
    float q = 0.f;
    for (int j = lane; j < r; j += 64) {
      const float x = S[row * lds + j];
      q = __fmaf_rn(x, x, q);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) q += __shfl_xor(q, off, 64);
    if (lane == 0) {
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
  if (lane == 0) {
    sh[0][wave] = sum_root;
    sh[1][wave] = sum_ssq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    partial[2 * blockIdx.x] = sh[0][0] + sh[0][1] + sh[0][2] + sh[0][3];
    partial[2 * blockIdx.x + 1] = sh[1][0] + sh[1][1] + sh[1][2] + sh[1][3];
  }
}

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

// One workgroup, fixed summation order (deterministic): scal[0] = eps,
// scal[1] = ||S|| / ||Ut||.
__global__ __launch_bounds__(256) void rowadam_finalize_kernel(const double* partial, int nparts, const float* root,
                                                              const float* ssq, int64_t d, float eps_rel,
                                                              double* scal) {
  __shared__ double sh[256];
  double a = 0.0, b = 0.0;
  for (int j = threadIdx.x; j < nparts; j += 256) {
    a += partial[2 * j];
    b += partial[2 * j + 1];
  }
  const double sum_root = block_sum_256(a, sh);
  const double norm_s2 = block_sum_256(b, sh);
  const double eps = fmax((double)eps_rel * (sum_root / (double)d), 1e-30);
  double c = 0.0;
  for (int64_t row = threadIdx.x; row < d; row += 256) {
    const double den = (double)root[row] + eps;
    c += (double)ssq[row] / (den * den);
  }
  const double norm_u2 = block_sum_256(c, sh);
  if (threadIdx.x == 0) {
    scal[0] = eps;
    scal[1] = norm_u2 > 0.0 ? sqrt(norm_s2 / norm_u2) : 0.0;
  }
}

__global__ __launch_bounds__(256) void rowadam_apply_kernel(float* S, int64_t lds, int64_t d, int r,
                                                           const float* root, const double* scal) {
  const double eps = scal[0], fac = scal[1];
  for (int64_t row = blockIdx.x; row < d; row += gridDim.x) {
    const float f = (float)(fac / ((double)root[row] + eps));
    for (int j = threadIdx.x; j < r; j += 256) S[row * lds + j] *= f;
  }
}

void rowadam_launch(float* S, int64_t lds, float* v, int64_t d, int r, float beta2, double inv_bias, float eps_rel,
                    float* root, float* ssq, double* partial, double* scal, hipStream_t s) {
  int blocks = (int)((d + 3) / 4);
  if (blocks > kRowAdamBlocks) blocks = kRowAdamBlocks;
  hipLaunchKernelGGL(rowadam_rows_kernel, dim3(blocks), dim3(256), 0, s, S, lds, v, d, r, beta2, inv_bias, root,
                     ssq, partial);
  hipLaunchKernelGGL(rowadam_finalize_kernel, dim3(1), dim3(256), 0, s, partial, blocks, root, ssq, d, eps_rel,
                     scal);
  const int ablocks = (int)(d < 4096 ? d : 4096);
  hipLaunchKernelGGL(rowadam_apply_kernel, dim3(ablocks), dim3(256), 0, s, S, lds, d, r, root, scal);
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

}  // namespace logra
