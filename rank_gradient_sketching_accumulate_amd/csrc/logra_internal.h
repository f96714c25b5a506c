// Internal interface between the C ABI (logra_api.hip) and the kernel
// translation units: parameter blocks, launch plans and launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace logra {

// ---------------------------------------------------------------------------
// Sketch accumulation: projection P = X s^T, then S += (1/sqrt r) dY^T P.
// ---------------------------------------------------------------------------
struct ProjParams {
  const uint16_t* X;
  int64_t ldx, T, k;
  uint64_t seed;
  int r;
  int n_tt;         // token tiles
  int n_k;          // column splits across workgroups
  int cbs_per;      // 256-column blocks per split
  int ncb;          // 256-column blocks of k
  uint16_t* Phi;    // P high halves, Pk order
  uint16_t* Plo;    // P low halves, Pk order
  float* Ppart;     // n_k fp32 partial sums, Pk order (n_k > 1 only)
  int64_t part_stride;
  unsigned* counters;  // one per token tile; zero between calls
  int hi_only;      // 0: write P's high and low planes; 1: the high plane only (the
                    // contraction reads no low plane); 2: high plane, zero low plane
  int row0;         // sign row of P's column 0 (256 for the upper half at ranks above 256)
  // Gaussian basis (proj_gauss_kernel): A as bf16 hi/lo planes, 16*NB rows x
  // kpad columns, row-major; P is written for tokens < Tw.
  const uint16_t* Ahi;
  const uint16_t* Alo;
  int64_t kpad, Tw;
};

struct ContractParams {
  const uint16_t* dY;
  int64_t lddy, T, d;
  const uint16_t* Phi;
  const uint16_t* Plo;
  int NB;        // 16-column blocks in Pk
  float* S;
  int64_t lds;
  int r;
  float inv_sqrt_r;
  int n_dt, n_ts;  // d tiles, token splits
  int64_t ksp;     // 32-token steps per token split
  int atomic_out;  // 1 when several workgroups add into the same S tile
  float* part;      // non-null: token split ts stores its tile at part + ts*part_split instead
  int64_t part_split;  // floats per split (d x 16*NB, row stride 16*NB)
  int bands;        // stream-K kernels: token bands, 1, 4 or 8 (grid a multiple of bands)
  int hi_only;      // contract with the high bf16 plane of P only
};

struct SketchPlan {
  int NB;                 // padded rank / 16 (power of two)
  int small_proj;         // 1: proj_small_kernel (all signs of k in LDS)
  int MBW, WK;            // projection: 16-token blocks per wave, waves along k
  int PNW;                // projection (round-based): waves per workgroup (4 or 8)
  int pwide;              // 1: proj_lds_kernel (NB = 4, 8 or 16, 64-token tiles, X staged through LDS)
  int n_tt, n_k, cbs_per, ncb;
  int64_t Tpad;
  int cvar;               // contraction variant (see contract_launch)
  int cwide;              // cvar 6: 1 = eight-wave shared-operand kernel, 2 = four-wave kernel
  int WM;                 // contraction row groups per workgroup (cvar 5)
  int few_ts;             // tall S: at most one round of workgroups, few token splits
  int n_dt, n_ts;
  int64_t ksp;
  int use_part;           // token-split tiles stored as partials, then summed by sketch_reduce
  int cgrid;              // contract_small / contract_tile: workgroups sharing the step units
  int cbands;             // token bands of that split (1; 4 = one per XCD pair; 8 = one per XCD)
  int bigdp;              // contract_big: steps between requesting a step's operands and using them
  int64_t n_counters;     // split counters the projection needs (a separate zeroed region)
  size_t off_phi, off_plo, off_part, off_cpart, total;
};

// det: bitwise-reproducible contraction (one workgroup per row tile of S,
// fixed summation order, no atomic adds).
// hi_only: the contraction uses the high bf16 plane of P only.
SketchPlan plan_sketch(int64_t T, int64_t k, int64_t d, int r, bool det = false, bool hi_only = false);
// Caller-held projection cache of the split project / contract calls: a high
// plane then a low plane, each cache_tokens(T) x 16*NB bf16 entries in Pk
// order.  Every projection tiling's padded token count fits in it (token
// tiles are powers of two of at most 256 tokens).
inline int64_t cache_tokens(int64_t T) { return (T + 255) / 256 * 256; }
size_t projection_cache_bytes(int64_t T, int r);
// Re-lays the library scratch of a plan without the P planes (they live in
// the caller's cache), keeping the projection's column-split partials and/or
// the contraction's token-split partials.
void scratch_layout(SketchPlan& pl, int64_t d, bool proj_part, bool con_part);
bool proj_launch(const SketchPlan& pl, const ProjParams& p, hipStream_t s);
bool contract_launch(const SketchPlan& pl, const ContractParams& p, hipStream_t s);
// S += sum over token splits of the stored partial tiles (use_part plans).
void reduce_launch(const SketchPlan& pl, const ContractParams& p, hipStream_t s);

// ---------------------------------------------------------------------------
// Merge W <- RNE(W - scale_eff * U s).
// ---------------------------------------------------------------------------
struct MergeParams {
  uint16_t* W;
  int64_t ldw, d, k;
  const float* U;
  int64_t ldu;
  int r;
  int u_vec;        // U rows 16-byte aligned (ldu % 4 == 0, aligned base)
  uint64_t seed;
  float scale_eff;  // scale / sqrt(r)
  // Gaussian basis: A^T as bf16 hi/lo planes, one row of 32*NK entries per
  // column of W (rows up to the last chunk's end); null for signs.
  const uint16_t* Athi;
  const uint16_t* Atlo;
  // RowAdam folded into the merge: U = S with row i multiplied by rowmul[i]
  // (fp32) as it is loaded; null for a plain U.
  const float* rowmul;
  // 1: U rounded once to bf16, one MFMA per product (sign basis only);
  // 0: U as a bf16 hi/lo pair, two MFMAs per product.
  int hi_only;
  int n_rb, n_cr;   // row blocks, column ranges
  int64_t cr_cols;  // columns per range (a multiple of the chunk width)
};

struct MergePlan {
  int NK;           // 32-wide steps of r (1, 2, 4, 8 or 16; U zero-padded)
  int NBW;          // 16-row blocks per wave
  int CB;           // 16-column blocks per chunk (4 or 8)
  int n_rb, n_cr;
  int64_t cr_cols;
};

// gauss: the Gaussian basis (default tiling only; no tuning variables).
MergePlan plan_merge(int64_t d, int64_t k, int r, bool gauss = false);
bool merge_launch(const MergePlan& pl, const MergeParams& mp, hipStream_t s);

// Up to kMaxMergeGroup matrices of one rank merged by one launch; matrix j
// owns logical workgroups [start[j], start[j+1]) (its own n_rb * n_cr tiles).
constexpr int kMaxMergeGroup = 16;
struct MergeGroup {
  int count;
  int start[kMaxMergeGroup + 1];
  MergeParams p[kMaxMergeGroup];
};
bool merge_group_launch(const MergePlan& pl, const MergeGroup& g, hipStream_t s);

// ---------------------------------------------------------------------------
// Gaussian basis (the refreshed Gaussian projection): Z for sign rows
// row0 .. row0 + rr - 1 (rows up to RP - 1 and columns k .. kpad - 1 are
// zero) as bf16 hi/lo planes, row-major A (RP x kpad) and/or column-major
// At (kpad x RP), and/or fp32 Z (rr x k, row stride k).
// ---------------------------------------------------------------------------
struct GaussBasisParams {
  uint64_t seed;
  int row0, rr, RP;
  int64_t k, kpad;
  uint16_t* Ahi;
  uint16_t* Alo;
  uint16_t* Athi;
  uint16_t* Atlo;
  float* Z;
};
void gauss_basis_launch(const GaussBasisParams& p, hipStream_t s);
// The projection with a Gaussian basis (P = X Z^T into the hi/lo planes).
bool proj_gauss_launch(const SketchPlan& pl, const ProjParams& p, hipStream_t s);

// ---------------------------------------------------------------------------
// Sync payload packing: header and entry words (little-endian u32 words of
// the documented layout), and per factor its source, rows, byte offset and
// slot size in the payload.
// ---------------------------------------------------------------------------
constexpr int kPayloadMaxItems = 32;
constexpr int kPayloadHeadWords = (32 + 48 * kPayloadMaxItems) / 4;
struct PayloadPackArgs {
  uint32_t head[kPayloadHeadWords];
  int n_head_words;  // words of header + entries actually used
  int header_words;  // words of the header region (a 256-byte multiple)
  int count, r;
  const float* U[kPayloadMaxItems];
  int64_t ldu[kPayloadMaxItems];
  int64_t d[kPayloadMaxItems];
  uint64_t off[kPayloadMaxItems];   // byte offset of the factor's slot
  uint64_t span[kPayloadMaxItems];  // bytes of the slot (d r 4 rounded up to 256)
};
void payload_pack_launch(const PayloadPackArgs& a, void* payload, hipStream_t s);

// ---------------------------------------------------------------------------
// Predicted KL (equation 6): per-row softmax-weighted variance of the score
// rates, then q.
// ---------------------------------------------------------------------------
struct KLParams {
  const void* z;
  int64_t ldz;
  const void* zd;
  int64_t ldzd;
  int64_t n, V;
  float scale;      // log2(e) / temperature
  int n_split;      // workgroups per row
  int64_t span;     // columns per workgroup (a multiple of 256 * 16)
  double* part;     // n * n_split states (m, W, mu, M2)
};

struct KLPlan {
  int n_split;
  int64_t span;
  size_t part_bytes;
};

KLPlan plan_kl(int64_t n, int64_t V);
void kl_launch(const KLPlan& pl, const KLParams& p, int bf16, float* row_var, float* q, double inv_2nt2,
               hipStream_t s);

// ---------------------------------------------------------------------------
// RowAdam and the sign dump.
// ---------------------------------------------------------------------------
// RowAdam: at most kRowAdamBlocks blocks per kernel; partial holds
// 2 * kRowAdamBlocks doubles, partial2 kRowAdamBlocks (its first two hold
// the finished eps and rescale factor).
constexpr int kRowAdamBlocks = 4096;
void rowadam_launch(float* S, int64_t lds, float* v, int64_t d, int r, float beta2, double inv_bias,
                    float eps_rel, float* root, float* ssq, double* partial, double* partial2, hipStream_t s,
                    float* rowmul = nullptr);
void signs_launch(uint64_t seed, int r, int64_t k, int8_t* out, hipStream_t s);
void stream_read_launch(const void* ptr, int64_t n16, uint32_t* sink, hipStream_t s);
// dst[0 .. 16*n16) = 0 (dst 16-byte aligned).
void zero_fill_launch(void* dst, int64_t n16, hipStream_t s);

int env_int(const char* name, int dflt);

}  // namespace logra
