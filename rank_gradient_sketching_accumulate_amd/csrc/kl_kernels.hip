// Predicted KL of a proposed update (gfx950).
//
// "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
// Sketches", section 2.3, equation 6 (derived in appendix A.1):
//
//   q(D) = 1 / (2 |P| T^2) * sum_s Var_{v ~ p(s)}[zdot_v(s)],   p(s) = softmax(z(s) / T)
//
// for logits z and score-change rates zdot over the whole vocabulary at each
// examined context s (one row each).  The pass is one streaming read of both
// arrays: every workgroup owns a column range of one row and keeps, per
// thread, the weighted-moment state of the tokens it has seen:
//
//   m  = the largest z/T seen, in base-2 units (z log2(e) / T),
//   W  = sum of 2^(z log2(e)/T - m)            (softmax numerator, rebased to m),
//   mu = the W-weighted mean of zdot (relative to the row's first rate),
//   M2 = the W-weighted sum of squared deviations of zdot from mu.
//
// Each step a thread holds 16 tokens in registers; their weighted mean and
// squared deviations are taken in two passes over the registers and merged
// into the running state with the pairwise update of Chan, Golub and LeVeque
// (mean shift times the product of the weights over their sum), so no sum of
// squares is ever differenced: peaked rows (one token holding nearly all the
// probability) keep full relative precision.  When a larger logit arrives,
// W and M2 are rescaled by 2^(m_old - m_new); mu does not change.  States
// are merged across the wave with shuffles and across the workgroup through
// LDS in float64, and one small kernel merges a row's column ranges in a
// fixed order (deterministic), writes Var = M2 / W per row and q.
#include <math.h>

#include <type_traits>

#include "logra_device.h"
#include "logra_internal.h"

namespace logra {

namespace {

constexpr int kKLThreads = 256;
constexpr int kKLStep = 16;  // tokens per thread per step (64 bytes fp32 or 32 bytes bf16 of each array)

struct KLState {
  double m, w, mu, m2;
};

__device__ __forceinline__ KLState kl_merge(const KLState& a, const KLState& b) {
  // An empty state (no token with a finite logit) has w == 0; a NaN weight
  // passes through the arithmetic below, so NaN inputs reach the result.
  if (b.w == 0.0) return a;
  if (a.w == 0.0) return b;
  const double m = fmax(a.m, b.m);
  // (the maxima are fp32 values: their difference rounded to fp32 and the
  // hardware exp2 keep the rescale within a few fp32 ulps)
  const double fa = __builtin_amdgcn_exp2f((float)(a.m - m)), fb = __builtin_amdgcn_exp2f((float)(b.m - m));
  const double wa = a.w * fa, wb = b.w * fb;
  const double w = wa + wb;
  const double dl = b.mu - a.mu;
  KLState o;
  o.m = m;
  o.w = w;
  o.mu = a.mu + dl * (wb / w);
  o.m2 = a.m2 * fa + b.m2 * fb + dl * dl * (wa * (wb / w));
  return o;
}

__device__ __forceinline__ KLState kl_shfl_xor(const KLState& s, int off) {
  KLState o;
  o.m = __shfl_xor(s.m, off, 64);
  o.w = __shfl_xor(s.w, off, 64);
  o.mu = __shfl_xor(s.mu, off, 64);
  o.m2 = __shfl_xor(s.m2, off, 64);
  return o;
}

template <bool BF16>
__device__ __forceinline__ void kl_unpack(const u32x4& v, float* out) {
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = bf16_to_f32(v[i] & 0xffffu);
      out[2 * i + 1] = bf16_to_f32(v[i] >> 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
  }
}

}  // namespace

// Grid: n_rows * n_split workgroups; workgroup b covers row b / n_split and
// the column range [sp * span, min(V, (sp + 1) * span)) of it, sp = b % n_split.
template <bool BF16>
__global__ __launch_bounds__(kKLThreads) void kl_rows_kernel(KLParams p) {
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int EPL = 16 / ESZ;         // tokens per 16-byte load
  constexpr int L = kKLStep / EPL;      // loads per array per step
  constexpr int64_t BLK = (int64_t)kKLThreads * kKLStep;
  __shared__ KLState sh[kKLThreads / 64];

  const int64_t row = blockIdx.x / p.n_split;
  const int sp = (int)(blockIdx.x - row * p.n_split);
  const int tid = threadIdx.x;
  // One descriptor per row.  The hardware bounds-checks buffer loads per
  // dword, so the size is the row's bytes rounded up to 16: a bf16 row of odd
  // length keeps its last token (whose dword also holds the next entry).  Rows
  // start on 16-byte boundaries, so the rounded block never leaves the page
  // that holds the row's last token; entries past V are masked below.
  const uint32_t row_bytes = (uint32_t)((p.V * ESZ + 15) / 16 * 16);
  const __amdgpu_buffer_rsrc_t rz =
      make_rsrc(static_cast<const char*>(p.z) + row * p.ldz * ESZ, row_bytes);
  const __amdgpu_buffer_rsrc_t rd =
      make_rsrc(static_cast<const char*>(p.zd) + row * p.ldzd * ESZ, row_bytes);
  const int64_t beg = (int64_t)sp * p.span;
  const int64_t end = min(p.V, beg + p.span);
  const float scale = p.scale;  // log2(e) / T

  // The score rates are taken relative to the row's first one: the variance
  // does not change, and fp32 keeps its digits for the spread when the rates
  // share a large common offset.
  float zref;
  {
    float first[EPL];
    kl_unpack<BF16>(buf_load16(rd, 0), first);
    zref = first[0];
  }

  float m = -INFINITY, W = 0.f, mu = 0.f, M2 = 0.f;
  u32x4 cz[L], cd[L], nz[L], nd[L];
  auto load = [&](u32x4 (&a)[L], u32x4 (&b)[L], int64_t e0) {
#pragma unroll
    for (int u = 0; u < L; ++u) {
      const uint32_t off = (uint32_t)((e0 + (int64_t)(u * kKLThreads + tid) * EPL) * ESZ);
      a[u] = buf_load16(rz, off);
      b[u] = buf_load16(rd, off);
    }
  };
  // One step: 16 entries per thread.  Interior steps (every entry inside the
  // range, the common case) skip the masking; the scale 1/T is folded into
  // the exponent's fma, and the step's maximum is taken on the raw logits
  // (scaling by log2(e)/T > 0 keeps the order).
  auto step = [&](int64_t e0, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    float zr[kKLStep], zv[kKLStep];
#pragma unroll
    for (int u = 0; u < L; ++u) {
      kl_unpack<BF16>(cz[u], zr + u * EPL);
      kl_unpack<BF16>(cd[u], zv + u * EPL);
    }
    float cm = -INFINITY;
#pragma unroll
    for (int u = 0; u < L; ++u)
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = u * EPL + i;
        if constexpr (MASKED) {
          const bool valid = e0 + (int64_t)(u * kKLThreads + tid) * EPL + i < end;
          zr[e] = valid ? zr[e] : -INFINITY;
          zv[e] = valid ? zv[e] - zref : 0.f;
        } else {
          zv[e] -= zref;
        }
        cm = fmaxf(cm, zr[e]);
      }
    const float cms = cm * scale;
    if (cms > m) {
      const float f = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - cms);
      W *= f;
      M2 *= f;
      m = cms;
    }
    if (cms != -INFINITY) {
      const float nm = -m;
      float w[kKLStep], Wc = 0.f, S1 = 0.f;
#pragma unroll
      for (int e = 0; e < kKLStep; ++e) {
        w[e] = __builtin_amdgcn_exp2f(__fmaf_rn(zr[e], scale, nm));
        Wc += w[e];
        S1 = __fmaf_rn(w[e], zv[e], S1);
      }
      if (Wc != 0.f) {  // (a NaN weight takes this branch and propagates)
        const float muc = S1 / Wc;
        float M2c = 0.f;
#pragma unroll
        for (int e = 0; e < kKLStep; ++e) {
          const float dv = zv[e] - muc;
          M2c = __fmaf_rn(w[e] * dv, dv, M2c);
        }
        const float Wn = W + Wc;
        const float dl = muc - mu;
        const float rc = Wc / Wn;
        mu = __fmaf_rn(dl, rc, mu);
        M2 = M2 + M2c + dl * dl * (W * rc);
        W = Wn;
      }
    }
  };

  if (beg < end) load(cz, cd, beg);
  for (int64_t e0 = beg; e0 < end; e0 += BLK) {
    const bool more = e0 + BLK < end;
    if (more) load(nz, nd, e0 + BLK);
    if (e0 + BLK <= end)
      step(e0, std::false_type{});
    else
      step(e0, std::true_type{});
    if (more) {
#pragma unroll
      for (int u = 0; u < L; ++u) {
        cz[u] = nz[u];
        cd[u] = nd[u];
      }
    }
  }

  // Merge the 256 thread states: wave shuffles, then the four waves in order.
  KLState st{(double)m, (double)W, (double)mu, (double)M2};
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) st = kl_merge(st, kl_shfl_xor(st, off));
  const int lane = tid & 63, wave = tid >> 6;
  if (lane == 0) sh[wave] = st;
  __syncthreads();
  if (tid == 0) {
    KLState acc = sh[0];
#pragma unroll
    for (int q = 1; q < kKLThreads / 64; ++q) acc = kl_merge(acc, sh[q]);
    double* out = p.part + 4 * (int64_t)blockIdx.x;
    out[0] = acc.m;
    out[1] = acc.w;
    out[2] = acc.mu;
    out[3] = acc.m2;
  }
}

// One workgroup: each thread merges the column ranges of its rows in order,
// writes Var = M2 / W (NaN for a row with no finite logit), and the fixed
// tree sum of the variances gives q = sum / (2 n T^2).
__global__ __launch_bounds__(256) void kl_finalize_kernel(const double* part, int n_split, int64_t n,
                                                          float* row_var, float* q, double inv_2nt2) {
  __shared__ double sh[256];
  double acc = 0.0;
  for (int64_t row = threadIdx.x; row < n; row += 256) {
    const double* src = part + 4 * row * n_split;
    KLState st{src[0], src[1], src[2], src[3]};
    for (int s = 1; s < n_split; ++s) {
      const double* o = src + 4 * s;
      st = kl_merge(st, KLState{o[0], o[1], o[2], o[3]});
    }
    // (a rounding-negative M2 reads as zero; NaN stays NaN)
    double var = st.w > 0.0 ? st.m2 / st.w : (double)NAN;
    if (var < 0.0) var = 0.0;
    if (row_var) row_var[row] = (float)var;
    acc += var;
  }
  sh[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) q[0] = (float)(sh[0] * inv_2nt2);
}

KLPlan plan_kl(int64_t n, int64_t V) {
  KLPlan pl{};
  const int64_t blk = (int64_t)kKLThreads * kKLStep;
  // Column ranges only when there are fewer than ~2048 rows: on the
  // 2048 x 151,936 probe one range per row ran at 0.92 of the GPU's
  // streaming-read time for the same bytes, and 4, 8 or 16 ranges per row
  // were 3-10 % slower.  Each range keeps at least two steps of its row.
  int64_t want = n > 0 ? (2048 + n - 1) / n : 1;
  const int64_t most = V > 0 ? (V + 2 * blk - 1) / (2 * blk) : 1;
  if (want > most) want = most;
  if (want < 1) want = 1;
  want = env_int("LOGRA_KL_SPLIT", (int)want);
  if (want < 1) want = 1;
  int64_t span = (V + want - 1) / want;
  span = (span + blk - 1) / blk * blk;
  if (span < blk) span = blk;
  pl.span = span;
  pl.n_split = V > 0 ? (int)((V + span - 1) / span) : 1;
  pl.part_bytes = (size_t)n * pl.n_split * 4 * sizeof(double);
  return pl;
}

void kl_launch(const KLPlan& pl, const KLParams& p, int bf16, float* row_var, float* q, double inv_2nt2,
               hipStream_t s) {
  if (p.n > 0) {
    const unsigned grid = (unsigned)(p.n * pl.n_split);
    if (bf16)
      hipLaunchKernelGGL(kl_rows_kernel<true>, dim3(grid), dim3(kKLThreads), 0, s, p);
    else
      hipLaunchKernelGGL(kl_rows_kernel<false>, dim3(grid), dim3(kKLThreads), 0, s, p);
  }
  hipLaunchKernelGGL(kl_finalize_kernel, dim3(1), dim3(256), 0, s, p.part, pl.n_split, p.n, row_var, q, inv_2nt2);
}

}  // namespace logra
