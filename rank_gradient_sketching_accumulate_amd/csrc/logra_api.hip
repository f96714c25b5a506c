// C ABI of the LoGRA hot-path library: argument validation, per-stream
// scratch, launch plans.  Declared in include/logra.h.
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <cstring>
#include <unistd.h>

#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <utility>
#include <vector>
#include <algorithm>

#include "../../include/logra.h"
#include "logra_internal.h"

namespace {

using namespace logra;

thread_local std::string g_last_error;

logra_status fail(logra_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

logra_status hip_fail(hipError_t e, const char* what) {
  return fail(LOGRA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

size_t span_bytes(int64_t rows, int64_t cols, int64_t ld, size_t elem) {
  if (rows <= 0 || cols <= 0) return 0;
  return ((size_t)(rows - 1) * (size_t)ld + (size_t)cols) * elem;
}

// Scratch per (device, purpose, stream).  It grows and never shrinks, and
// it is zeroed when it grows (the split counters must start at zero; the
// kernels leave them at zero).  A buffer it outgrows is retired, not freed:
// a graph captured earlier on the stream may still launch kernels that use
// it.  Retired and current buffers are freed only by logra_workspace_release.
// Growing is refused while the stream is being captured (allocation and
// clearing are not capturable); logra_workspace_reserve grows it beforehand.
enum ArenaKind {
  kArenaSketch = 0,
  kArenaRowAdam = 1,
  kArenaKL = 2,
  kArenaCounters = 3,
  kArenaBasis = 4,  // Gaussian basis planes
  kArenaKinds = 5
};
struct Arena {
  void* ptr = nullptr;
  size_t bytes = 0;
  std::vector<void*> retired;
};
std::mutex g_arena_mu;
std::map<std::pair<std::pair<int, int>, hipStream_t>, Arena> g_arenas;

// Scratch lives on the current device, so the stream must belong to it (a
// stream of another device would run the kernels there, on memory of this
// one).  Handles the runtime cannot map to a device (the null stream and the
// special per-thread handles) are taken to be the current device's.
logra_status stream_on_device(hipStream_t stream, int dev) {
  if (stream == nullptr) return LOGRA_OK;
  hipDevice_t sd = 0;
  if (hipStreamGetDevice(stream, &sd) != hipSuccess) {
    (void)hipGetLastError();
    return LOGRA_OK;
  }
  if ((int)sd != dev)
    return fail(LOGRA_ERR_RANGE, "the stream belongs to device " + std::to_string((int)sd) + " but device " +
                                     std::to_string(dev) + " is current: make the stream's device current");
  return LOGRA_OK;
}

logra_status arena_get(int kind, hipStream_t stream, size_t need, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  const logra_status sd = stream_on_device(stream, dev);
  if (sd != LOGRA_OK) return sd;
  std::lock_guard<std::mutex> lk(g_arena_mu);
  Arena& a = g_arenas[{{dev, kind}, stream}];
  if (a.bytes < need) {
    const char* fa = getenv("LOGRA_TEST_FAIL_ALLOC");
    if (fa && fa[0] == '1') return fail(LOGRA_ERR_NOMEM, "scratch allocation refused (LOGRA_TEST_FAIL_ALLOC=1)");
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone)
      return fail(LOGRA_ERR_NOMEM,
                  "the library's scratch for this stream must grow, but the stream is being captured: "
                  "call logra_workspace_reserve before capturing");
    size_t cap = need < ((size_t)1 << 20) ? ((size_t)1 << 20) : need;
    if (a.bytes && cap < 2 * a.bytes) cap = 2 * a.bytes;  // geometric: retired buffers stay below the current one
    void* np = nullptr;
    e = hipMalloc(&np, cap);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(LOGRA_ERR_NOMEM, std::string("hipMalloc of scratch failed: ") + hipGetErrorString(e));
    }
    e = hipMemsetAsync(np, 0, cap, stream);
    if (e != hipSuccess) {
      (void)hipFree(np);
      return hip_fail(e, "hipMemsetAsync");
    }
    if (a.ptr) a.retired.push_back(a.ptr);
    a.ptr = np;
    a.bytes = cap;
  }
  *out = a.ptr;
  return LOGRA_OK;
}

// Split counters: one unsigned per token tile, in an arena of their own.
logra_status counters_get(hipStream_t stream, int64_t n, unsigned** out) {
  void* p = nullptr;
  logra_status st = arena_get(kArenaCounters, stream, (size_t)(n > 0 ? n : 1) * sizeof(unsigned), &p);
  *out = static_cast<unsigned*>(p);
  return st;
}

// Launch plans depend only on the shape, unless a LOGRA_ variable in the
// environment overrides a choice (tuning and tests): then the plan is worked
// out afresh on every call.  Otherwise each thread keeps the plans it has
// made, so a call costs one scan of the environment, not one lookup per knob.
bool plan_overrides_present() {
  for (char** e = environ; e && *e; ++e)
    if (strncmp(*e, "LOGRA_", 6) == 0) return true;
  return false;
}

// Per-thread switch of logra_set_deterministic.
thread_local bool g_deterministic = false;
// Per-thread switch of logra_set_precision: contract with the high bf16 half
// of P only (one MFMA per product instead of two).
thread_local bool g_precision_hi_only = false;

SketchPlan sketch_plan_for(int64_t T, int64_t k, int64_t d, int r, bool ho) {
  const bool det = g_deterministic;
  if (plan_overrides_present()) return plan_sketch(T, k, d, r, det, ho);
  thread_local std::map<std::tuple<int64_t, int64_t, int64_t, int, bool, bool>, SketchPlan> plans;
  const auto key = std::make_tuple(T, k, d, r, det, ho);
  auto it = plans.find(key);
  if (it != plans.end()) return it->second;
  if (plans.size() >= 1024) plans.clear();
  const SketchPlan pl = plan_sketch(T, k, d, r, det, ho);
  plans.emplace(key, pl);
  return pl;
}

// Per-thread switch of logra_set_basis: the Gaussian basis instead of signs.
thread_local bool g_basis_gauss = false;

MergePlan merge_plan_for(int64_t d, int64_t k, int r) {
  if (g_basis_gauss) return plan_merge(d, k, r, true);
  if (plan_overrides_present()) return plan_merge(d, k, r);
  thread_local std::map<std::tuple<int64_t, int64_t, int>, MergePlan> plans;
  const auto key = std::make_tuple(d, k, r);
  auto it = plans.find(key);
  if (it != plans.end()) return it->second;
  if (plans.size() >= 1024) plans.clear();
  const MergePlan pl = plan_merge(d, k, r);
  plans.emplace(key, pl);
  return pl;
}

// Checks shared by the calls that read X.
logra_status check_x(const void* X, int64_t ldx, int64_t T, int64_t k) {
  if (ldx < k) return fail(LOGRA_ERR_SHAPE, "ldx must be >= k");
  if (((uintptr_t)X & 15) || (ldx & 7))
    return fail(LOGRA_ERR_ALIGN, "X needs a 16-byte aligned base and a row stride that is a multiple of 8");
  if (T > ((int64_t)1 << 31) || k > ((int64_t)1 << 31)) return fail(LOGRA_ERR_SHAPE, "T and k must be below 2^31");
  return LOGRA_OK;
}

// Checks shared by the calls that read dY and add into S.
logra_status check_dy_s(const void* dY, int64_t lddy, int64_t T, int64_t d, const float* S, int64_t lds, int r) {
  if (lddy < d) return fail(LOGRA_ERR_SHAPE, "lddy must be >= d");
  if (((uintptr_t)dY & 15) || (lddy & 7))
    return fail(LOGRA_ERR_ALIGN, "dY needs a 16-byte aligned base and a row stride that is a multiple of 8");
  if ((uintptr_t)S & 3) return fail(LOGRA_ERR_ALIGN, "S must be 4-byte aligned");
  if (overlaps(S, span_bytes(d, r, lds, 4), dY, span_bytes(T, d, lddy, 2)))
    return fail(LOGRA_ERR_ALIAS, "S overlaps X or dY");
  if (T > ((int64_t)1 << 31) || d > ((int64_t)1 << 31)) return fail(LOGRA_ERR_SHAPE, "T and d must be below 2^31");
  return LOGRA_OK;
}

// Kernels address X and dY through buffer descriptors with 32-bit byte
// offsets (rows past T read as zero): each operand must span < 4 GiB.
logra_status check_plan(const SketchPlan& pl, int64_t T, int64_t ldx, int64_t lddy) {
  const uint64_t lim = ((uint64_t)1 << 32) - 4096;
  if ((uint64_t)(pl.Tpad + 32) * (uint64_t)ldx * 2 >= lim || (uint64_t)(pl.Tpad + 32) * (uint64_t)lddy * 2 >= lim)
    return fail(LOGRA_ERR_SHAPE, "X or dY spans 4 GiB or more; split the microbatch into several calls");
  if ((size_t)pl.n_k * pl.Tpad * 16 * pl.NB * 4 > ((size_t)1 << 32) - 64)
    return fail(LOGRA_ERR_SHAPE, "T too large for one call at this rank; split the microbatch");
  (void)T;
  return LOGRA_OK;
}

// Gaussian basis planes (bf16 hi and lo) of rp rows x kpad columns: bytes,
// and generation into the basis region (which the caller has already grown
// to at least that size).
size_t basis_bytes(int rp, int64_t kpad) { return (size_t)2 * rp * (size_t)kpad * 2; }
int64_t basis_kpad_proj(int64_t k) { return (k + 31) / 32 * 32; }
int64_t basis_kpad_merge(int64_t k) { return (k + 127) / 128 * 128; }

logra_status basis_generate(uint64_t seed, int row0, int rr, int rp, int64_t k, int64_t kpad, bool col_major,
                            hipStream_t stream, uint16_t** hi, uint16_t** lo) {
  void* p = nullptr;
  logra_status st = arena_get(kArenaBasis, stream, basis_bytes(rp, kpad), &p);
  if (st != LOGRA_OK) return st;
  GaussBasisParams gp{};
  gp.seed = seed;
  gp.row0 = row0;
  gp.rr = rr;
  gp.RP = rp;
  gp.k = k;
  gp.kpad = kpad;
  uint16_t* h = static_cast<uint16_t*>(p);
  uint16_t* l = h + (size_t)rp * (size_t)kpad;
  if (col_major) {
    gp.Athi = h;
    gp.Atlo = l;
  } else {
    gp.Ahi = h;
    gp.Alo = l;
  }
  gauss_basis_launch(gp, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "basis launch");
  *hi = h;
  *lo = l;
  return LOGRA_OK;
}

// P = X s^T into the hi/lo planes (Pk order); tokens in [T, Tpad) get zeros.
// hi_only: the fused call contracts with P rounded once to bf16: its
// projection writes no low plane when the contraction reads none (the
// single-bf16 and half tilings), or a zero one otherwise.  The split call always
// writes both planes.
// counters: the split counters (zero, n_counters of them), or null to take
// them from the library's per-stream region.
// row0: the sign row of P's first column (256 for the upper half of a rank
// above 256).
// With the Gaussian basis (g_basis_gauss) the basis planes of this half are
// generated into the basis region first and proj_gauss_kernel runs instead.
logra_status enqueue_projection(const SketchPlan& pl, char* base, const void* X, int64_t ldx, int64_t T, int64_t k,
                                uint64_t seed, int r, int row0, uint16_t* Phi, uint16_t* Plo, bool hi_only,
                                hipStream_t stream, unsigned* counters = nullptr) {
  if (g_basis_gauss) {
    const int rp = 16 * pl.NB;
    const int64_t kpad = basis_kpad_proj(k);
    uint16_t *ah = nullptr, *al = nullptr;
    logra_status st = basis_generate(seed, row0, r, rp, k, kpad, false, stream, &ah, &al);
    if (st != LOGRA_OK) return st;
    ProjParams gp{};
    gp.X = static_cast<const uint16_t*>(X);
    gp.ldx = ldx; gp.T = T; gp.k = k; gp.seed = seed; gp.r = r; gp.row0 = row0;
    gp.Phi = Phi;
    gp.Plo = Plo;
    gp.Ahi = ah;
    gp.Alo = al;
    gp.kpad = kpad;
    gp.Tw = (T + 31) / 32 * 32;
    gp.hi_only = !hi_only ? 0 : ((pl.cvar == 6 || pl.cvar == 7) ? 1 : 2);
    if (!proj_gauss_launch(pl, gp, stream)) return fail(LOGRA_ERR_RANGE, "no Gaussian projection kernel for this rank");
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "Gaussian projection launch");
    return LOGRA_OK;
  }
  ProjParams pp{};
  pp.X = static_cast<const uint16_t*>(X);
  pp.ldx = ldx; pp.T = T; pp.k = k; pp.seed = seed; pp.r = r; pp.row0 = row0;
  pp.n_tt = pl.n_tt; pp.n_k = pl.n_k; pp.cbs_per = pl.cbs_per; pp.ncb = pl.ncb;
  pp.Phi = Phi;
  pp.Plo = Plo;
  pp.Ppart = reinterpret_cast<float*>(base + pl.off_part);
  pp.part_stride = pl.Tpad * 16 * pl.NB;
  if (pl.n_k > 1) {
    if (counters) {
      pp.counters = counters;
    } else {
      logra_status st = counters_get(stream, pl.n_counters, &pp.counters);
      if (st != LOGRA_OK) return st;
    }
  }
  pp.hi_only = !hi_only ? 0 : ((pl.cvar == 6 || pl.cvar == 7) ? 1 : 2);
  if (!proj_launch(pl, pp, stream)) return fail(LOGRA_ERR_RANGE, "no projection kernel for this tile");
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "projection launch");
  return LOGRA_OK;
}

// S += (1/sqrt r) dY^T P from the hi/lo planes.
// r: the columns of S this contraction adds into; r_full: the rank whose
// 1/sqrt scales them (r_full > r for the halves of a rank above 256).
logra_status enqueue_contraction(const SketchPlan& pl, char* base, const void* dY, int64_t lddy, int64_t T, int64_t d,
                                 const uint16_t* Phi, const uint16_t* Plo, int r, int r_full, float* S, int64_t lds,
                                 bool hi_only, hipStream_t stream) {
  ContractParams cp{};
  cp.dY = static_cast<const uint16_t*>(dY);
  cp.lddy = lddy; cp.T = T; cp.d = d;
  cp.Phi = Phi; cp.Plo = Plo; cp.NB = pl.NB;
  cp.S = S; cp.lds = lds; cp.r = r;
  cp.inv_sqrt_r = (float)(1.0 / sqrt((double)r_full));
  cp.n_dt = pl.n_dt; cp.n_ts = pl.n_ts; cp.ksp = pl.ksp;
  cp.atomic_out = pl.n_ts > 1 ? 1 : 0;
  cp.bands = pl.cbands;
  cp.hi_only = (hi_only && (pl.cvar == 6 || pl.cvar == 7)) ? 1 : 0;
  if (pl.use_part) {
    cp.part = reinterpret_cast<float*>(base + pl.off_cpart);
    cp.part_split = d * 16 * pl.NB;
  }
  if (!contract_launch(pl, cp, stream)) return fail(LOGRA_ERR_RANGE, "no contraction kernel for this tile");
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "contraction launch");
  if (pl.use_part) {
    reduce_launch(pl, cp, stream);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "partial-sum launch");
  }
  return LOGRA_OK;
}

// Validation and launch parameters of one merge (shared by the single and
// grouped calls).  skip: nothing to do (empty matrix or scale 0).
logra_status prepare_merge(void* W, int64_t ldw, const float* U, int64_t ldu, int64_t d, int64_t k, uint64_t seed,
                           int32_t r, float scale, MergeParams& mp, MergePlan& pl, bool& skip) {
  skip = false;
  if (d < 0 || k < 0) return fail(LOGRA_ERR_SHAPE, "d and k must be >= 0");
  if (r < 1 || r > LOGRA_MAX_RANK) return fail(LOGRA_ERR_RANGE, "r must be in [1, 512]");
  if (ldu < r) return fail(LOGRA_ERR_SHAPE, "ldu must be >= r");
  if (d == 0 || k == 0) {
    skip = true;
    return LOGRA_OK;
  }
  if (!W || !U) return fail(LOGRA_ERR_NULL, "W and U must be non-null");
  if (ldw < k) return fail(LOGRA_ERR_SHAPE, "ldw must be >= k");
  if (((uintptr_t)W & 7) || (ldw & 3)) return fail(LOGRA_ERR_ALIGN, "W needs an 8-byte aligned base and ldw a multiple of 4");
  if ((uintptr_t)U & 3) return fail(LOGRA_ERR_ALIGN, "U must be 4-byte aligned");
  if (!isfinite(scale)) return fail(LOGRA_ERR_RANGE, "scale must be finite");
  if (overlaps(W, span_bytes(d, k, ldw, 2), U, span_bytes(d, r, ldu, 4))) return fail(LOGRA_ERR_ALIAS, "W overlaps U");
  if (d > ((int64_t)1 << 31) || k > ((int64_t)1 << 31)) return fail(LOGRA_ERR_SHAPE, "d and k must be below 2^31");
  if ((uint64_t)d * (uint64_t)ldw * 2 >= ((uint64_t)1 << 32) - 4096 ||
      (uint64_t)d * (uint64_t)ldu * 4 >= ((uint64_t)1 << 32) - 4096)
    return fail(LOGRA_ERR_SHAPE, "W or U spans 4 GiB or more; merge the rows in several calls");
  if (scale == 0.0f) {
    skip = true;
    return LOGRA_OK;
  }
  pl = merge_plan_for(d, k, r);
  mp = MergeParams{};
  mp.hi_only = g_precision_hi_only ? 1 : 0;
  mp.W = static_cast<uint16_t*>(W);
  mp.ldw = ldw; mp.d = d; mp.k = k; mp.U = U; mp.ldu = ldu; mp.r = r;
  mp.u_vec = (((uintptr_t)U & 15) == 0 && (ldu & 3) == 0) ? 1 : 0;
  mp.seed = seed;
  mp.scale_eff = (float)((double)scale / sqrt((double)r));
  mp.n_rb = pl.n_rb; mp.n_cr = pl.n_cr; mp.cr_cols = pl.cr_cols;
  return LOGRA_OK;
}

// RowAdam scratch for d rows: per-row root and squared norm, then the two
// rounds of per-block partial sums.  Returns the total bytes.
size_t rowadam_layout(int64_t d, size_t& off_root, size_t& off_ssq, size_t& off_part, size_t& off_part2) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  off_root = 0;
  off_ssq = up((size_t)d * 4);
  off_part = off_ssq + up((size_t)d * 4);
  off_part2 = off_part + up((size_t)2 * kRowAdamBlocks * 8);
  return off_part2 + up((size_t)kRowAdamBlocks * 8);
}

// Ranks above 256 run as two column halves through the rank <= 256 tilings:
// sign rows [0, 256) into columns [0, 256) of S (and of the projection cache),
// rows [256, r) into columns [256, r).  A sign depends only on (seed, row,
// column), so the halves add exactly the columns one rank-r pass would; both
// scale by 1/sqrt(r).
constexpr int kHalfRank = 256;
int n_halves(int r) { return r > kHalfRank ? 2 : 1; }
int half_rank(int r, int h) { return h == 0 ? std::min(r, kHalfRank) : r - kHalfRank; }
// Projection cache of rank r: one cache per half, back to back.
size_t cache_bytes(int64_t T, int r) {
  size_t b = 0;
  for (int h = 0; h < n_halves(r); ++h) b += projection_cache_bytes(T, half_rank(r, h));
  return b;
}
size_t cache_half_offset(int64_t T, int h) { return h == 0 ? 0 : projection_cache_bytes(T, kHalfRank); }



// Argument checks of the fused sketch calls; *empty: nothing to do.
logra_status check_sketch_args(const void* X, int64_t ldx, const void* dY, int64_t lddy, int64_t T, int64_t k,
                               int64_t d, int32_t r, const float* S, int64_t lds, bool* empty) {
  *empty = false;
  if (T < 0 || k < 0 || d < 0) return fail(LOGRA_ERR_SHAPE, "T, k and d must be >= 0");
  if (r < 1 || r > LOGRA_MAX_RANK) return fail(LOGRA_ERR_RANGE, "r must be in [1, 512]");
  if (lds < r) return fail(LOGRA_ERR_SHAPE, "lds must be >= r");
  if (T == 0 || k == 0 || d == 0) {
    *empty = true;
    return LOGRA_OK;
  }
  if (!X || !dY || !S) return fail(LOGRA_ERR_NULL, "X, dY and S must be non-null");
  logra_status st = check_x(X, ldx, T, k);
  if (st != LOGRA_OK) return st;
  st = check_dy_s(dY, lddy, T, d, S, lds, r);
  if (st != LOGRA_OK) return st;
  if (overlaps(S, span_bytes(d, r, lds, 4), X, span_bytes(T, k, ldx, 2)))
    return fail(LOGRA_ERR_ALIAS, "S overlaps X or dY");
  return LOGRA_OK;
}

}  // namespace

// Scratch of logra_sketch_accumulate_noalloc: a fixed array in device
// memory, one copy per GPU the library runs on, held until the process ends.
// Host code never passes the array's name to a kernel (on the host it only
// stands for the symbol): it uses the device address that hipGetSymbolAddress
// returns for the current device.
static __device__ __align__(256) unsigned char scratch[LOGRA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per
// device).
logra_status noalloc_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(LOGRA_ERR_RANGE, "device ordinal above 63");
  const logra_status sd = stream_on_device(stream, dev);
  if (sd != LOGRA_OK) return sd;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(LOGRA_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LOGRA_OK;
}

}  // namespace

extern "C" {

logra_status logra_sketch_accumulate_noalloc(const void* X, int64_t ldx, const void* dY, int64_t lddy, int64_t T,
                                             int64_t k, int64_t d, uint64_t seed, int32_t r, float* S, int64_t lds,
                                             hipStream_t stream) {
  try {
    g_last_error.clear();
    bool empty = false;
    logra_status st = check_sketch_args(X, ldx, dY, lddy, T, k, d, r, S, lds, &empty);
    if (st != LOGRA_OK || empty) return st;
    if (g_basis_gauss)
      return fail(LOGRA_ERR_RANGE, "the Gaussian basis needs scratch for its planes: use logra_sketch_accumulate");
    // The plan of logra_sketch_accumulate, except that token splits of the
    // contraction add into S directly instead of parking partial tiles (the
    // scratch then holds P, the projection's column-split partials and the
    // split counters only).  Worked out afresh (no plan cache: nothing is
    // allocated on the host either).
    SketchPlan pls[2];
    size_t off_cnt = 0, cnt_bytes = 0;
    for (int h = 0; h < n_halves(r); ++h) {
      SketchPlan& pl = pls[h];
      pl = plan_sketch(T, k, d, half_rank(r, h), g_deterministic, g_precision_hi_only);
      pl.use_part = 0;
      st = check_plan(pl, T, ldx, lddy);
      if (st != LOGRA_OK) return st;
      off_cnt = std::max(off_cnt, (pl.off_cpart + 255) / 256 * 256);
      cnt_bytes = std::max(cnt_bytes, (size_t)(pl.n_k > 1 ? pl.n_counters : 0) * sizeof(unsigned));
    }
    const size_t cnt_span = (cnt_bytes + 15) / 16 * 16;
    const size_t need = off_cnt + cnt_span;
    if (need > (size_t)LOGRA_NOALLOC_SCRATCH_BYTES)
      return fail(LOGRA_ERR_NOMEM, "this call needs " + std::to_string(need) +
                                       " bytes of scratch, more than the static " +
                                       std::to_string((size_t)LOGRA_NOALLOC_SCRATCH_BYTES) +
                                       " bytes: split the microbatch or use logra_sketch_accumulate");
    void* ptr = nullptr;
    st = noalloc_scratch(stream, &ptr);
    if (st != LOGRA_OK) return st;
    char* base = static_cast<char*>(ptr);
    unsigned* counters = nullptr;
    if (cnt_span) {
      // The last call may have left anything here: clear the counters with
      // a kernel (capturable, unlike a memset node).  The projection kernels
      // leave them at zero, so one clear serves both halves.
      counters = reinterpret_cast<unsigned*>(base + off_cnt);
      zero_fill_launch(counters, (int64_t)(cnt_span / 16), stream);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return hip_fail(e, "counter clear launch");
    }
    for (int h = 0; h < n_halves(r); ++h) {
      const SketchPlan& pl = pls[h];
      const int rh = half_rank(r, h);
      uint16_t* Phi = reinterpret_cast<uint16_t*>(base + pl.off_phi);
      uint16_t* Plo = reinterpret_cast<uint16_t*>(base + pl.off_plo);
      st = enqueue_projection(pl, base, X, ldx, T, k, seed, rh, kHalfRank * h, Phi, Plo, g_precision_hi_only, stream,
                              counters);
      if (st != LOGRA_OK) return st;
      st = enqueue_contraction(pl, base, dY, lddy, T, d, Phi, Plo, rh, r, S + kHalfRank * h, lds,
                               g_precision_hi_only, stream);
      if (st != LOGRA_OK) return st;
    }
    return LOGRA_OK;
  } catch (...) {
    return fail(LOGRA_ERR_HIP, "unexpected C++ exception");
  }
}

logra_status logra_sketch_accumulate(const void* X, int64_t ldx, const void* dY, int64_t lddy, int64_t T, int64_t k,
                                     int64_t d, uint64_t seed, int32_t r, float* S, int64_t lds,
                                     hipStream_t stream) {
  try {
    g_last_error.clear();
    bool empty = false;
    logra_status st = check_sketch_args(X, ldx, dY, lddy, T, k, d, r, S, lds, &empty);
    if (st != LOGRA_OK || empty) return st;

    SketchPlan pls[2];
    size_t need = 0;
    int64_t n_cnt = 0;
    for (int h = 0; h < n_halves(r); ++h) {
      pls[h] = sketch_plan_for(T, k, d, half_rank(r, h), g_precision_hi_only);
      st = check_plan(pls[h], T, ldx, lddy);
      if (st != LOGRA_OK) return st;
      need = std::max(need, pls[h].total);
      n_cnt = std::max(n_cnt, pls[h].n_counters);
    }
    // All scratch is obtained before anything is enqueued.
    void* ws = nullptr;
    st = arena_get(kArenaSketch, stream, need, &ws);
    if (st != LOGRA_OK) return st;
    if (n_cnt > 0) {
      unsigned* cnt = nullptr;
      st = counters_get(stream, n_cnt, &cnt);
      if (st != LOGRA_OK) return st;
    }
    if (g_basis_gauss) {
      void* bp = nullptr;
      st = arena_get(kArenaBasis, stream, basis_bytes(16 * pls[0].NB, basis_kpad_proj(k)), &bp);
      if (st != LOGRA_OK) return st;
    }
    char* base = static_cast<char*>(ws);
    for (int h = 0; h < n_halves(r); ++h) {
      const SketchPlan& pl = pls[h];
      const int rh = half_rank(r, h);
      uint16_t* Phi = reinterpret_cast<uint16_t*>(base + pl.off_phi);
      uint16_t* Plo = reinterpret_cast<uint16_t*>(base + pl.off_plo);
      st = enqueue_projection(pl, base, X, ldx, T, k, seed, rh, kHalfRank * h, Phi, Plo, g_precision_hi_only, stream);
      if (st != LOGRA_OK) return st;
      st = enqueue_contraction(pl, base, dY, lddy, T, d, Phi, Plo, rh, r, S + kHalfRank * h, lds,
                               g_precision_hi_only, stream);
      if (st != LOGRA_OK) return st;
    }
    return LOGRA_OK;
  } catch (...) {
    return fail(LOGRA_ERR_HIP, "unexpected C++ exception");
  }
}

int logra_set_precision(int mode) {
  const int prev = g_precision_hi_only ? LOGRA_PRECISION_BF16 : LOGRA_PRECISION_BF16X2;
  g_precision_hi_only = mode == LOGRA_PRECISION_BF16;
  return prev;
}

int logra_set_basis(int basis) {
  const int prev = g_basis_gauss ? LOGRA_BASIS_GAUSSIAN : LOGRA_BASIS_RADEMACHER;
  g_basis_gauss = basis == LOGRA_BASIS_GAUSSIAN;
  return prev;
}

logra_status logra_basis_normals(uint64_t seed, int32_t r, int64_t k, float* out, hipStream_t stream) {
  try {
    g_last_error.clear();
    if (k < 0) return fail(LOGRA_ERR_SHAPE, "k must be >= 0");
    if (r < 1 || r > LOGRA_MAX_RANK) return fail(LOGRA_ERR_RANGE, "r must be in [1, 512]");
    if (k == 0) return LOGRA_OK;
    if (!out) return fail(LOGRA_ERR_NULL, "out must be non-null");
    if ((uintptr_t)out & 3) return fail(LOGRA_ERR_ALIGN, "out must be 4-byte aligned");
    if ((uint64_t)r * (uint64_t)k >= ((uint64_t)1 << 31)) return fail(LOGRA_ERR_SHAPE, "r * k must be below 2^31");
    GaussBasisParams gp{};
    gp.seed = seed;
    gp.row0 = 0;
    gp.rr = r;
    gp.RP = r;
    gp.k = k;
    gp.kpad = (k + 7) / 8 * 8;
    gp.Z = out;
    gauss_basis_launch(gp, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "basis launch");
    return LOGRA_OK;
  } catch (...) {
    return fail(LOGRA_ERR_HIP, "unexpected C++ exception");
  }
}

int logra_set_deterministic(int enable) {
  const int prev = g_deterministic ? 1 : 0;
  g_deterministic = enable != 0;
  return prev;
}

size_t logra_projection_bytes(int64_t T, int32_t r) {
  if (T <= 0 || r < 1 || r > LOGRA_MAX_RANK) return 0;
  return cache_bytes(T, r);
}

logra_status logra_project(const void* X, int64_t ldx, int64_t T, int64_t k, uint64_t seed, int32_t r, void* P,
                           size_t P_bytes, hipStream_t stream) {
  try {
    g_last_error.clear();
    if (T < 0 || k < 0) return fail(LOGRA_ERR_SHAPE, "T and k must be >= 0");
    if (r < 1 || r > LOGRA_MAX_RANK) return fail(LOGRA_ERR_RANGE, "r must be in [1, 512]");
    if (T == 0) return LOGRA_OK;
    if (!P) return fail(LOGRA_ERR_NULL, "P must be non-null");
    const size_t need = cache_bytes(T, r);
    if (P_bytes < need) return fail(LOGRA_ERR_SHAPE, "P_bytes is smaller than logra_projection_bytes(T, r)");
    if ((uintptr_t)P & 15) return fail(LOGRA_ERR_ALIGN, "P must be 16-byte aligned");
    if (k == 0) {
      // X has no columns: P = X s^T is zero (need is a multiple of 16 bytes).
      zero_fill_launch(P, (int64_t)(need / 16), stream);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return hip_fail(e, "zero fill launch");
      return LOGRA_OK;
    }
    if (!X) return fail(LOGRA_ERR_NULL, "X must be non-null");
    logra_status st = check_x(X, ldx, T, k);
    if (st != LOGRA_OK) return st;
    if (overlaps(P, need, X, span_bytes(T, k, ldx, 2))) return fail(LOGRA_ERR_ALIAS, "P overlaps X");

    SketchPlan pls[2];
    size_t ws_need = 0;
    int64_t n_cnt = 0;
    for (int h = 0; h < n_halves(r); ++h) {
      SketchPlan& pl = pls[h];
      pl = sketch_plan_for(T, k, 1, half_rank(r, h), false);
      st = check_plan(pl, T, ldx, 8);
      if (st != LOGRA_OK) return st;
      if (pl.Tpad > cache_tokens(T)) return fail(LOGRA_ERR_RANGE, "projection tile does not fit the cache");
      scratch_layout(pl, 1, true, false);
      ws_need = std::max(ws_need, pl.total);
      n_cnt = std::max(n_cnt, pl.n_counters);
    }
    void* ws = nullptr;
    st = arena_get(kArenaSketch, stream, ws_need, &ws);
    if (st != LOGRA_OK) return st;
    if (n_cnt > 0) {
      unsigned* cnt = nullptr;
      st = counters_get(stream, n_cnt, &cnt);
      if (st != LOGRA_OK) return st;
    }
    if (g_basis_gauss) {
      void* bp = nullptr;
      st = arena_get(kArenaBasis, stream, basis_bytes(16 * pls[0].NB, basis_kpad_proj(k)), &bp);
      if (st != LOGRA_OK) return st;
    }
    for (int h = 0; h < n_halves(r); ++h) {
      const SketchPlan& pl = pls[h];
      uint16_t* Phi = reinterpret_cast<uint16_t*>(static_cast<char*>(P) + cache_half_offset(T, h));
      uint16_t* Plo = Phi + (size_t)cache_tokens(T) * 16 * pl.NB;
      st = enqueue_projection(pl, static_cast<char*>(ws), X, ldx, T, k, seed, half_rank(r, h), kHalfRank * h, Phi,
                              Plo, false, stream);
      if (st != LOGRA_OK) return st;
    }
    return LOGRA_OK;
  } catch (...) {
    return fail(LOGRA_ERR_HIP, "unexpected C++ exception");
  }
}

logra_status logra_contract(const void* dY, int64_t lddy, int64_t T, int64_t d, const void* P, size_t P_bytes,
                            int32_t r, float* S, int64_t lds, hipStream_t stream) {
  try {
    g_last_error.clear();
    if (T < 0 || d < 0) return fail(LOGRA_ERR_SHAPE, "T and d must be >= 0");
    if (r < 1 || r > LOGRA_MAX_RANK) return fail(LOGRA_ERR_RANGE, "r must be in [1, 512]");
    if (lds < r) return fail(LOGRA_ERR_SHAPE, "lds must be >= r");
    if (T == 0 || d == 0) return LOGRA_OK;
    if (!dY || !P || !S) return fail(LOGRA_ERR_NULL, "dY, P and S must be non-null");
    const size_t need = cache_bytes(T, r);
    if (P_bytes < need) return fail(LOGRA_ERR_SHAPE, "P_bytes is smaller than logra_projection_bytes(T, r)");
    if ((uintptr_t)P & 15) return fail(LOGRA_ERR_ALIGN, "P must be 16-byte aligned");
    logra_status st = check_dy_s(dY, lddy, T, d, S, lds, r);
    if (st != LOGRA_OK) return st;
    if (overlaps(S, span_bytes(d, r, lds, 4), P, need)) return fail(LOGRA_ERR_ALIAS, "S overlaps P");

    // The contraction's tiling does not depend on k; 256 stands in for it.
    SketchPlan pls[2];
    size_t ws_need = 0;
    for (int h = 0; h < n_halves(r); ++h) {
      SketchPlan& pl = pls[h];
      pl = sketch_plan_for(T, 256, d, half_rank(r, h), false);
      st = check_plan(pl, T, 8, lddy);
      if (st != LOGRA_OK) return st;
      scratch_layout(pl, d, false, true);
      ws_need = std::max(ws_need, pl.total);
    }
    void* ws = nullptr;
    st = arena_get(kArenaSketch, stream, ws_need, &ws);
    if (st != LOGRA_OK) return st;
    for (int h = 0; h < n_halves(r); ++h) {
      const SketchPlan& pl = pls[h];
      const uint16_t* Phi = reinterpret_cast<const uint16_t*>(static_cast<const char*>(P) + cache_half_offset(T, h));
      const uint16_t* Plo = Phi + (size_t)cache_tokens(T) * 16 * pl.NB;
      st = enqueue_contraction(pl, static_cast<char*>(ws), dY, lddy, T, d, Phi, Plo, half_rank(r, h), r,
                               S + kHalfRank * h, lds, false, stream);
      if (st != LOGRA_OK) return st;
    }
    return LOGRA_OK;
  } catch (...) {
    return fail(LOGRA_ERR_HIP, "unexpected C++ exception");
  }
}

logra_status logra_merge_update(void* W, int64_t ldw, const float* U, int64_t ldu, int64_t d, int64_t k,
                                uint64_t seed, int32_t r, float scale, hipStream_t stream) {
  try {
    g_last_error.clear();
    MergeParams mp{};
    MergePlan pl{};
    bool skip = false;
    logra_status st = prepare_merge(W, ldw, U, ldu, d, k, seed, r, scale, mp, pl, skip);
    if (st != LOGRA_OK || skip) return st;
    if (g_basis_gauss) {
      uint16_t *ah = nullptr, *al = nullptr;
      st = basis_generate(seed, 0, r, 32 * pl.NK, k, basis_kpad_merge(k), true, stream, &ah, &al);
      if (st != LOGRA_OK) return st;
      mp.Athi = ah;
      mp.Atlo = al;
    }
    if (!merge_launch(pl, mp, stream)) return fail(LOGRA_ERR_RANGE, "no merge kernel for this tile");
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "merge launch");
    return LOGRA_OK;
  } catch (...) {
    return fail(LOGRA_ERR_HIP, "unexpected C++ exception");
  }
}

logra_status logra_merge_update_grouped(const logra_merge_item* items, int32_t count, int32_t r,
                                        hipStream_t stream) {
  try {
    g_last_error.clear();
    if (count < 0) return fail(LOGRA_ERR_SHAPE, "count must be >= 0");
    if (count == 0) return LOGRA_OK;
    if (!items) return fail(LOGRA_ERR_NULL, "items must be non-null");
    if (r < 1 || r > LOGRA_MAX_RANK) return fail(LOGRA_ERR_RANGE, "r must be in [1, 512]");
    // Validate everything before anything is enqueued.
    std::vector<MergeParams> mps;
    MergePlan pl0{};
    bool have = false;
    for (int32_t j = 0; j < count; ++j) {
      const logra_merge_item& it = items[j];
      MergeParams mp{};
      MergePlan pl{};
      bool skip = false;
      logra_status st = prepare_merge(it.W, it.ldw, it.U, it.ldu, it.d, it.k, it.seed, r, it.scale, mp, pl, skip);
      if (st != LOGRA_OK)
        return fail(st, "item " + std::to_string(j) + ": " + g_last_error);
      const size_t wb = span_bytes(it.d, it.k, it.ldw, 2);
      for (int32_t i = 0; i < j; ++i)
        if (overlaps(it.W, wb, items[i].W, span_bytes(items[i].d, items[i].k, items[i].ldw, 2)) ||
            overlaps(it.W, wb, items[i].U, span_bytes(items[i].d, r, items[i].ldu, 4)) ||
            overlaps(items[i].W, span_bytes(items[i].d, items[i].k, items[i].ldw, 2), it.U,
                     span_bytes(it.d, r, it.ldu, 4)))
          return fail(LOGRA_ERR_ALIAS, "item " + std::to_string(j) + " overlaps the W or U of item " +
                                           std::to_string(i) + " (a W written by one item is read or written by another)");
      if (skip) continue;
      if (!have) {
        pl0 = pl;
        have = true;
      } else if (pl.NBW != pl0.NBW || pl.CB != pl0.CB || pl.NK != pl0.NK) {
        return fail(LOGRA_ERR_RANGE, "items need the same tiling (set by r)");
      }
      mp.n_rb = pl.n_rb;
      mp.n_cr = pl.n_cr;
      mp.cr_cols = pl.cr_cols;
      mps.push_back(mp);
    }
    if (g_basis_gauss) {
      // One merge per matrix, each after its basis planes (one region, reused
      // in stream order; grown to the largest first).
      size_t most = 0;
      for (const MergeParams& mp : mps) most = std::max(most, basis_bytes(32 * pl0.NK, basis_kpad_merge(mp.k)));
      void* bp = nullptr;
      logra_status st = arena_get(kArenaBasis, stream, most, &bp);
      if (st != LOGRA_OK) return st;
      for (MergeParams mp : mps) {
        uint16_t *ah = nullptr, *al = nullptr;
        st = basis_generate(mp.seed, 0, r, 32 * pl0.NK, mp.k, basis_kpad_merge(mp.k), true, stream, &ah, &al);
        if (st != LOGRA_OK) return st;
        mp.Athi = ah;
        mp.Atlo = al;
        MergePlan pl = pl0;
        pl.n_rb = mp.n_rb;
        pl.n_cr = mp.n_cr;
        pl.cr_cols = mp.cr_cols;
        if (!merge_launch(pl, mp, stream)) return fail(LOGRA_ERR_RANGE, "no merge kernel for this tile");
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "merge launch");
      }
      return LOGRA_OK;
    }
    for (size_t b = 0; b < mps.size(); b += kMaxMergeGroup) {
      MergeGroup g{};
      g.count = (int)std::min<size_t>(kMaxMergeGroup, mps.size() - b);
      g.start[0] = 0;
      for (int j = 0; j < g.count; ++j) {
        g.p[j] = mps[b + j];
        const int64_t next = (int64_t)g.start[j] + (int64_t)g.p[j].n_rb * g.p[j].n_cr;
        if (next >= ((int64_t)1 << 31) - 8) return fail(LOGRA_ERR_SHAPE, "too many workgroups for one launch");
        g.start[j + 1] = (int)next;
      }
      if (!merge_group_launch(pl0, g, stream)) return fail(LOGRA_ERR_RANGE, "no grouped merge kernel for this tile");
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return hip_fail(e, "grouped merge launch");
    }
    return LOGRA_OK;
  } catch (...) {
    return fail(LOGRA_ERR_HIP, "unexpected C++ exception");
  }
}

}  // extern "C"

namespace {

static_assert(sizeof(logra_payload_header) == 32, "payload header is 32 bytes");
static_assert(sizeof(logra_payload_entry) == 48, "payload entry is 48 bytes");
static_assert(LOGRA_PAYLOAD_MAX_ITEMS == kPayloadMaxItems, "one item limit");

size_t up256(size_t x) { return (x + 255) / 256 * 256; }

// Offsets of the factors (and the total) for count items of d_j rows.
void payload_layout(const int64_t* d, int32_t count, int32_t r, uint64_t* off, uint64_t* span, size_t* total) {
  size_t o = up256(32 + 48 * (size_t)count);
  for (int32_t j = 0; j < count; ++j) {
    off[j] = o;
    span[j] = up256((size_t)d[j] * (size_t)r * 4);
    o += span[j];
  }
  *total = o;
}

}  // namespace

extern "C" {

size_t logra_payload_header_bytes(int32_t count) {
  if (count < 1 || count > LOGRA_PAYLOAD_MAX_ITEMS) return 0;
  return up256(32 + 48 * (size_t)count);
}

size_t logra_payload_bytes(const logra_merge_item* items, int32_t count, int32_t r) {
  if (!items || count < 1 || count > LOGRA_PAYLOAD_MAX_ITEMS || r < 1 || r > LOGRA_MAX_RANK) return 0;
  int64_t d[kPayloadMaxItems];
  uint64_t off[kPayloadMaxItems], span[kPayloadMaxItems];
  for (int32_t j = 0; j < count; ++j) {
    if (items[j].d < 0 || items[j].k < 0) return 0;
    d[j] = items[j].d;
  }
  size_t total = 0;
  payload_layout(d, count, r, off, span, &total);
  return total;
}

logra_status logra_payload_pack(const logra_merge_item* items, int32_t count, int32_t r, void* payload,
                                size_t payload_bytes, hipStream_t stream) {
  try {
    g_last_error.clear();
    if (count < 1 || count > LOGRA_PAYLOAD_MAX_ITEMS)
      return fail(LOGRA_ERR_RANGE, "count must be in [1, " + std::to_string(LOGRA_PAYLOAD_MAX_ITEMS) + "]");
    if (r < 1 || r > LOGRA_MAX_RANK) return fail(LOGRA_ERR_RANGE, "r must be in [1, 512]");
    if (!items || !payload) return fail(LOGRA_ERR_NULL, "items and payload must be non-null");
    if ((uintptr_t)payload & 255) return fail(LOGRA_ERR_ALIGN, "payload must be 256-byte aligned");
    PayloadPackArgs a{};
    a.count = count;
    a.r = r;
    for (int32_t j = 0; j < count; ++j) {
      const logra_merge_item& it = items[j];
      const std::string tag = "item " + std::to_string(j) + ": ";
      if (it.d < 0 || it.k < 0) return fail(LOGRA_ERR_SHAPE, tag + "d and k must be >= 0");
      if (it.ldu < r) return fail(LOGRA_ERR_SHAPE, tag + "ldu must be >= r");
      if (it.d > 0 && !it.U) return fail(LOGRA_ERR_NULL, tag + "U must be non-null");
      if ((uintptr_t)it.U & 3) return fail(LOGRA_ERR_ALIGN, tag + "U must be 4-byte aligned");
      if (!isfinite(it.scale)) return fail(LOGRA_ERR_RANGE, tag + "scale must be finite");
      a.U[j] = it.U;
      a.ldu[j] = it.ldu;
      a.d[j] = it.d;
    }
    size_t total = 0;
    payload_layout(a.d, count, r, a.off, a.span, &total);
    if (payload_bytes < total) return fail(LOGRA_ERR_SHAPE, "payload_bytes is smaller than logra_payload_bytes");
    for (int32_t j = 0; j < count; ++j)
      if (overlaps(items[j].U, span_bytes(items[j].d, r, items[j].ldu, 4), payload, total))
        return fail(LOGRA_ERR_ALIAS, "item " + std::to_string(j) + ": U overlaps the payload");
    // Header and entries as little-endian words.
    logra_payload_header h{};
    h.magic = LOGRA_PAYLOAD_MAGIC;
    h.version = LOGRA_PAYLOAD_VERSION;
    h.count = count;
    h.r = r;
    h.total_bytes = total;
    std::memcpy(a.head, &h, sizeof(h));
    for (int32_t j = 0; j < count; ++j) {
      logra_payload_entry e{};
      e.seed = items[j].seed;
      e.d = items[j].d;
      e.k = items[j].k;
      e.scale = items[j].scale;
      e.basis = g_basis_gauss ? LOGRA_BASIS_GAUSSIAN : LOGRA_BASIS_RADEMACHER;
      e.u_offset = a.off[j];
      std::memcpy(reinterpret_cast<char*>(a.head) + 32 + 48 * (size_t)j, &e, sizeof(e));
    }
    a.n_head_words = (32 + 48 * count) / 4;
    a.header_words = (int)(a.off[0] / 4);
    payload_pack_launch(a, payload, stream);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return hip_fail(err, "payload pack launch");
    return LOGRA_OK;
  } catch (...) {
    return fail(LOGRA_ERR_HIP, "unexpected C++ exception");
  }
}

logra_status logra_payload_parse(const void* header_host, size_t bytes, logra_payload_header* header,
                                 logra_payload_entry* entries, int32_t max_entries) {
  try {
    g_last_error.clear();
    if (!header_host || !header) return fail(LOGRA_ERR_NULL, "header_host and header must be non-null");
    if (bytes < sizeof(logra_payload_header)) return fail(LOGRA_ERR_SHAPE, "fewer bytes than a payload header");
    logra_payload_header h;
    std::memcpy(&h, header_host, sizeof(h));
    if (h.magic != LOGRA_PAYLOAD_MAGIC) return fail(LOGRA_ERR_SHAPE, "not a payload (magic)");
    if (h.version != LOGRA_PAYLOAD_VERSION) return fail(LOGRA_ERR_SHAPE, "unknown payload version");
    if (h.reserved != 0) return fail(LOGRA_ERR_SHAPE, "header reserved word is not zero");
    if (h.count < 1 || h.count > LOGRA_PAYLOAD_MAX_ITEMS) return fail(LOGRA_ERR_SHAPE, "entry count out of range");
    if (h.r < 1 || h.r > LOGRA_MAX_RANK) return fail(LOGRA_ERR_SHAPE, "rank out of range");
    const size_t hb = up256(32 + 48 * (size_t)h.count);
    if (bytes < 32 + 48 * (size_t)h.count) return fail(LOGRA_ERR_SHAPE, "header truncated before its entries end");
    if (h.total_bytes < hb) return fail(LOGRA_ERR_SHAPE, "total bytes smaller than the header");
    if (h.count > max_entries) return fail(LOGRA_ERR_RANGE, "more entries than max_entries");
    if (!entries) return fail(LOGRA_ERR_NULL, "entries must be non-null");
    logra_payload_entry es[kPayloadMaxItems];
    for (int32_t j = 0; j < h.count; ++j) {
      std::memcpy(&es[j], static_cast<const char*>(header_host) + 32 + 48 * (size_t)j, sizeof(logra_payload_entry));
      const logra_payload_entry& e = es[j];
      const std::string tag = "entry " + std::to_string(j) + ": ";
      if (e.d < 0 || e.k < 0 || e.d > ((int64_t)1 << 31) || e.k > ((int64_t)1 << 31))
        return fail(LOGRA_ERR_SHAPE, tag + "d or k out of range");
      if (e.reserved1 != 0) return fail(LOGRA_ERR_SHAPE, tag + "reserved word is not zero");
      if (e.basis != LOGRA_BASIS_RADEMACHER && e.basis != LOGRA_BASIS_GAUSSIAN)
        return fail(LOGRA_ERR_SHAPE, tag + "unknown basis");
      if (!isfinite(e.scale)) return fail(LOGRA_ERR_SHAPE, tag + "scale is not finite");
      const uint64_t n = (uint64_t)e.d * (uint64_t)h.r * 4;
      if (e.u_offset % 256 || e.u_offset < hb || e.u_offset > h.total_bytes || n > h.total_bytes - e.u_offset)
        return fail(LOGRA_ERR_SHAPE, tag + "factor outside the payload or misaligned");
      for (int32_t i = 0; i < j; ++i) {
        const uint64_t ni = (uint64_t)es[i].d * (uint64_t)h.r * 4;
        if (n && ni && e.u_offset < es[i].u_offset + ni && es[i].u_offset < e.u_offset + n)
          return fail(LOGRA_ERR_SHAPE, tag + "factor overlaps entry " + std::to_string(i) + "'s");
      }
    }
    *header = h;
    std::memcpy(entries, es, sizeof(logra_payload_entry) * (size_t)h.count);
    return LOGRA_OK;
  } catch (...) {
    return fail(LOGRA_ERR_HIP, "unexpected C++ exception");
  }
}

logra_status logra_payload_apply(const void* payload, size_t payload_bytes, const logra_payload_header* header,
                                 const logra_payload_entry* entries, void* const* W, const int64_t* ldw,
                                 hipStream_t stream) {
  try {
    g_last_error.clear();
    if (!payload || !header || !entries || !W || !ldw)
      return fail(LOGRA_ERR_NULL, "payload, header, entries, W and ldw must be non-null");
    if (header->magic != LOGRA_PAYLOAD_MAGIC || header->version != LOGRA_PAYLOAD_VERSION)
      return fail(LOGRA_ERR_SHAPE, "header is not a parsed payload header");
    if (header->count < 1 || header->count > LOGRA_PAYLOAD_MAX_ITEMS || header->r < 1 || header->r > LOGRA_MAX_RANK)
      return fail(LOGRA_ERR_SHAPE, "header count or rank out of range");
    if (payload_bytes < header->total_bytes) return fail(LOGRA_ERR_SHAPE, "payload_bytes below the header's total");
    if ((uintptr_t)payload & 255) return fail(LOGRA_ERR_ALIGN, "payload must be 256-byte aligned");
    logra_merge_item items[kPayloadMaxItems];
    for (int32_t j = 0; j < header->count; ++j) {
      const logra_payload_entry& e = entries[j];
      const uint64_t n = (uint64_t)e.d * (uint64_t)header->r * 4;
      if (e.d < 0 || e.k < 0 || e.u_offset > header->total_bytes || n > header->total_bytes - e.u_offset)
        return fail(LOGRA_ERR_SHAPE, "entry " + std::to_string(j) + ": factor outside the payload");
      items[j].W = W[j];
      items[j].ldw = ldw[j];
      items[j].U = reinterpret_cast<const float*>(static_cast<const char*>(payload) + e.u_offset);
      items[j].ldu = header->r;
      items[j].d = e.d;
      items[j].k = e.k;
      items[j].seed = e.seed;
      items[j].scale = e.scale;
    }
    // Each entry with its own basis: consecutive entries of one basis go to
    // one grouped call under that basis.
    const bool saved = g_basis_gauss;
    logra_status st = LOGRA_OK;
    for (int32_t j0 = 0; j0 < header->count && st == LOGRA_OK;) {
      int32_t j1 = j0 + 1;
      while (j1 < header->count && entries[j1].basis == entries[j0].basis) ++j1;
      g_basis_gauss = entries[j0].basis == LOGRA_BASIS_GAUSSIAN;
      st = logra_merge_update_grouped(items + j0, j1 - j0, header->r, stream);
      j0 = j1;
    }
    g_basis_gauss = saved;
    return st;
  } catch (...) {
    return fail(LOGRA_ERR_HIP, "unexpected C++ exception");
  }
}

logra_status logra_rowadam_scale(float* S, int64_t lds, float* v, int64_t d, int32_t r, int64_t step, float beta2,
                                 float eps_rel, hipStream_t stream) {
  try {
    g_last_error.clear();
    if (d < 0) return fail(LOGRA_ERR_SHAPE, "d must be >= 0");
    if (r < 1 || r > LOGRA_MAX_RANK) return fail(LOGRA_ERR_RANGE, "r must be in [1, 512]");
    if (lds < r) return fail(LOGRA_ERR_SHAPE, "lds must be >= r");
    if (step < 1) return fail(LOGRA_ERR_RANGE, "step counts RowAdam updates and starts at 1");
    if (!(beta2 >= 0.0f && beta2 < 1.0f)) return fail(LOGRA_ERR_RANGE, "beta2 must be in [0, 1)");
    if (!(eps_rel >= 0.0f) || !isfinite(eps_rel)) return fail(LOGRA_ERR_RANGE, "eps_rel must be finite and >= 0");
    if (d == 0) return LOGRA_OK;
    if (!S || !v) return fail(LOGRA_ERR_NULL, "S and v must be non-null");
    if (((uintptr_t)S & 3) || ((uintptr_t)v & 3)) return fail(LOGRA_ERR_ALIGN, "S and v must be 4-byte aligned");
    if (overlaps(S, span_bytes(d, r, lds, 4), v, (size_t)d * 4)) return fail(LOGRA_ERR_ALIAS, "v overlaps S");

    size_t off_root, off_ssq, off_part, off_part2;
    const size_t total = rowadam_layout(d, off_root, off_ssq, off_part, off_part2);
    void* ws = nullptr;
    logra_status st = arena_get(kArenaRowAdam, stream, total, &ws);
    if (st != LOGRA_OK) return st;
    char* base = static_cast<char*>(ws);
    const double inv_bias = 1.0 / (1.0 - pow((double)beta2, (double)step));
    rowadam_launch(S, lds, v, d, r, beta2, inv_bias, eps_rel, reinterpret_cast<float*>(base + off_root),
                   reinterpret_cast<float*>(base + off_ssq), reinterpret_cast<double*>(base + off_part),
                   reinterpret_cast<double*>(base + off_part2), stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "rowadam launch");
    return LOGRA_OK;
  } catch (...) {
    return fail(LOGRA_ERR_HIP, "unexpected C++ exception");
  }
}

logra_status logra_rowadam_merge(void* W, int64_t ldw, const float* S, int64_t lds, float* v, int64_t d, int64_t k,
                                 uint64_t seed, int32_t r, int64_t step, float beta2, float eps_rel, float scale,
                                 hipStream_t stream) {
  try {
    g_last_error.clear();
    if (d < 0 || k < 0) return fail(LOGRA_ERR_SHAPE, "d and k must be >= 0");
    if (r < 1 || r > LOGRA_MAX_RANK) return fail(LOGRA_ERR_RANGE, "r must be in [1, 512]");
    if (lds < r) return fail(LOGRA_ERR_SHAPE, "lds must be >= r");
    if (step < 1) return fail(LOGRA_ERR_RANGE, "step counts RowAdam updates and starts at 1");
    if (!(beta2 >= 0.0f && beta2 < 1.0f)) return fail(LOGRA_ERR_RANGE, "beta2 must be in [0, 1)");
    if (!(eps_rel >= 0.0f) || !isfinite(eps_rel)) return fail(LOGRA_ERR_RANGE, "eps_rel must be finite and >= 0");
    if (d == 0) return LOGRA_OK;
    if (!S || !v) return fail(LOGRA_ERR_NULL, "S and v must be non-null");
    if (((uintptr_t)S & 3) || ((uintptr_t)v & 3)) return fail(LOGRA_ERR_ALIGN, "S and v must be 4-byte aligned");
    if (overlaps(S, span_bytes(d, r, lds, 4), v, (size_t)d * 4)) return fail(LOGRA_ERR_ALIAS, "v overlaps S");
    // The merge's own checks (W against S as its U), before anything is
    // enqueued; k == 0 still updates v.
    MergeParams mp{};
    MergePlan pl{};
    bool skip = false;
    logra_status st = prepare_merge(W, ldw, S, lds, d, k, seed, r, scale, mp, pl, skip);
    if (st != LOGRA_OK) return st;
    if (!skip && overlaps(W, span_bytes(d, k, ldw, 2), v, (size_t)d * 4)) return fail(LOGRA_ERR_ALIAS, "W overlaps v");
    size_t off_root, off_ssq, off_part, off_part2;
    const size_t total = rowadam_layout(d, off_root, off_ssq, off_part, off_part2);
    const size_t off_mul = total;
    void* ws = nullptr;
    st = arena_get(kArenaRowAdam, stream, total + (size_t)d * 4, &ws);
    if (st != LOGRA_OK) return st;
    if (!skip && g_basis_gauss) {
      void* bp = nullptr;
      st = arena_get(kArenaBasis, stream, basis_bytes(32 * pl.NK, basis_kpad_merge(k)), &bp);
      if (st != LOGRA_OK) return st;
    }
    char* base = static_cast<char*>(ws);
    float* rowmul = reinterpret_cast<float*>(base + off_mul);
    const double inv_bias = 1.0 / (1.0 - pow((double)beta2, (double)step));
    // S is only read: the rescale writes the row factors instead.
    rowadam_launch(const_cast<float*>(S), lds, v, d, r, beta2, inv_bias, eps_rel,
                   reinterpret_cast<float*>(base + off_root), reinterpret_cast<float*>(base + off_ssq),
                   reinterpret_cast<double*>(base + off_part), reinterpret_cast<double*>(base + off_part2), stream,
                   rowmul);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "rowadam launch");
    if (skip) return LOGRA_OK;
    mp.rowmul = rowmul;
    if (g_basis_gauss) {
      uint16_t *ah = nullptr, *al = nullptr;
      st = basis_generate(seed, 0, r, 32 * pl.NK, k, basis_kpad_merge(k), true, stream, &ah, &al);
      if (st != LOGRA_OK) return st;
      mp.Athi = ah;
      mp.Atlo = al;
    }
    if (!merge_launch(pl, mp, stream)) return fail(LOGRA_ERR_RANGE, "no merge kernel for this tile");
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "merge launch");
    return LOGRA_OK;
  } catch (...) {
    return fail(LOGRA_ERR_HIP, "unexpected C++ exception");
  }
}

logra_status logra_predicted_kl(const void* z, int64_t ldz, const void* zdot, int64_t ldzd, int64_t n, int64_t V,
                                int32_t dtype, float temperature, float* row_var, float* q, hipStream_t stream) {
  try {
    g_last_error.clear();
    if (n < 0 || V < 0) return fail(LOGRA_ERR_SHAPE, "n and V must be >= 0");
    if (dtype != LOGRA_DTYPE_F32 && dtype != LOGRA_DTYPE_BF16)
      return fail(LOGRA_ERR_RANGE, "dtype must be LOGRA_DTYPE_F32 or LOGRA_DTYPE_BF16");
    if (!(temperature > 0.0f) || !isfinite(temperature))
      return fail(LOGRA_ERR_RANGE, "temperature must be finite and > 0");
    if (!q) return fail(LOGRA_ERR_NULL, "q must be non-null");
    if ((uintptr_t)q & 3) return fail(LOGRA_ERR_ALIGN, "q must be 4-byte aligned");
    const size_t esz = dtype == LOGRA_DTYPE_BF16 ? 2 : 4;
    if (n > 0) {
      if (V == 0) return fail(LOGRA_ERR_SHAPE, "V must be >= 1 when n > 0 (softmax over an empty vocabulary)");
      if (!z || !zdot) return fail(LOGRA_ERR_NULL, "z and zdot must be non-null");
      if (ldz < V || ldzd < V) return fail(LOGRA_ERR_SHAPE, "ldz and ldzd must be >= V");
      if (((uintptr_t)z & 15) || ((uintptr_t)zdot & 15) ||
          (n > 1 && (((size_t)ldz * esz) % 16 || ((size_t)ldzd * esz) % 16)))
        return fail(LOGRA_ERR_ALIGN, "z and zdot need 16-byte aligned bases and rows that start on 16-byte boundaries");
      if (row_var && ((uintptr_t)row_var & 3)) return fail(LOGRA_ERR_ALIGN, "row_var must be 4-byte aligned");
      if ((uint64_t)V * esz >= ((uint64_t)1 << 31)) return fail(LOGRA_ERR_SHAPE, "a row must span less than 2 GiB");
      const size_t zb = span_bytes(n, V, ldz, esz), db = span_bytes(n, V, ldzd, esz);
      if (overlaps(q, 4, z, zb) || overlaps(q, 4, zdot, db))
        return fail(LOGRA_ERR_ALIAS, "q overlaps z or zdot");
      if (row_var && (overlaps(row_var, (size_t)n * 4, z, zb) || overlaps(row_var, (size_t)n * 4, zdot, db) ||
                      overlaps(row_var, (size_t)n * 4, q, 4)))
        return fail(LOGRA_ERR_ALIAS, "row_var overlaps z, zdot or q");
    }
    const KLPlan pl = plan_kl(n, V);
    if ((uint64_t)n * (uint64_t)pl.n_split >= ((uint64_t)1 << 31))
      return fail(LOGRA_ERR_SHAPE, "too many rows for one call; split them");
    void* ws = nullptr;
    if (n > 0) {
      logra_status st = arena_get(kArenaKL, stream, pl.part_bytes, &ws);
      if (st != LOGRA_OK) return st;
    }
    KLParams kp{};
    kp.z = z; kp.ldz = ldz; kp.zd = zdot; kp.ldzd = ldzd; kp.n = n; kp.V = V;
    kp.scale = (float)(1.4426950408889634 / (double)temperature);  // log2(e) / T
    kp.n_split = pl.n_split;
    kp.span = pl.span;
    kp.part = static_cast<double*>(ws);
    const double t = (double)temperature;
    const double inv_2nt2 = n > 0 ? 1.0 / (2.0 * (double)n * t * t) : 0.0;
    kl_launch(pl, kp, dtype == LOGRA_DTYPE_BF16 ? 1 : 0, row_var, q, inv_2nt2, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "predicted-KL launch");
    return LOGRA_OK;
  } catch (...) {
    return fail(LOGRA_ERR_HIP, "unexpected C++ exception");
  }
}

double logra_kl_step_scale(double q, double delta, double alpha_max) {
  if (!(delta > 0.0) || !(alpha_max > 0.0) || !(q >= 0.0)) return NAN;
  if (q == 0.0) return alpha_max;
  const double a = sqrt(delta / q);
  return a < alpha_max ? a : alpha_max;
}

double logra_kl_budget(int64_t u, int64_t H, double delta_max, double delta_min) {
  if (H < 2) return delta_min;
  if (u < 1) u = 1;
  if (u > H) u = H;
  const double pi = 3.14159265358979323846;
  return delta_min + 0.5 * (delta_max - delta_min) * (1.0 + cos(pi * (double)(u - 1) / (double)(H - 1)));
}

double logra_kl_effective_budget(double delta, double kappa) {
  if (isnan(kappa)) return delta;
  const double k = kappa > 0.0 ? kappa : 0.0;
  const double a = delta - k, b = 0.5 * delta;
  return a > b ? a : b;
}

logra_status logra_signs(uint64_t seed, int32_t r, int64_t k, int8_t* out, hipStream_t stream) {
  g_last_error.clear();
  if (r < 1 || r > LOGRA_MAX_RANK) return fail(LOGRA_ERR_RANGE, "r must be in [1, 512]");
  if (k < 0) return fail(LOGRA_ERR_SHAPE, "k must be >= 0");
  if (k == 0) return LOGRA_OK;
  if (!out) return fail(LOGRA_ERR_NULL, "out must be non-null");
  signs_launch(seed, r, k, out, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "signs launch");
  return LOGRA_OK;
}

logra_status logra_stream_read(const void* ptr, size_t bytes, uint32_t* sink, hipStream_t stream) {
  g_last_error.clear();
  if (bytes == 0) return LOGRA_OK;
  if (!ptr || !sink) return fail(LOGRA_ERR_NULL, "ptr and sink must be non-null");
  if (((uintptr_t)ptr & 15) || (bytes & 15) || ((uintptr_t)sink & 3))
    return fail(LOGRA_ERR_ALIGN, "ptr must be 16-byte aligned, bytes a multiple of 16, sink 4-byte aligned");
  if (bytes / 16 / 1024 >= ((size_t)1 << 31)) return fail(LOGRA_ERR_SHAPE, "bytes too large for one launch");
  stream_read_launch(ptr, (int64_t)(bytes / 16), sink, stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "stream read launch");
  return LOGRA_OK;
}

}  // extern "C"

namespace {

// Scratch the calls for one (T, k, d, r) need on a stream, with the calling
// thread's settings: the sketch region (the fused call's plan covers the
// split calls' partials too), the split counters, and RowAdam's for d rows.
struct WorkspaceNeed {
  size_t sketch = 0, counters = 0, rowadam = 0, basis = 0;
};

WorkspaceNeed workspace_need(int64_t T, int64_t k, int64_t d, int r) {
  WorkspaceNeed w;
  for (int h = 0; h < n_halves(r); ++h) {
    const int rh = half_rank(r, h);
    const SketchPlan pl = sketch_plan_for(T, k, d, rh, g_precision_hi_only);
    w.sketch = std::max(w.sketch, pl.total);
    w.counters = std::max(w.counters, (size_t)std::max<int64_t>(pl.n_counters, 1) * sizeof(unsigned));
    SketchPlan pp = sketch_plan_for(T, k, 1, rh, false);
    scratch_layout(pp, 1, true, false);
    w.sketch = std::max(w.sketch, pp.total);
    w.counters = std::max(w.counters, (size_t)std::max<int64_t>(pp.n_counters, 1) * sizeof(unsigned));
    SketchPlan pc = sketch_plan_for(T, 256, d, rh, false);
    scratch_layout(pc, d, false, true);
    w.sketch = std::max(w.sketch, pc.total);
  }
  if (g_basis_gauss) {
    const int nb0 = sketch_plan_for(T, k, d, half_rank(r, 0), g_precision_hi_only).NB;
    const MergePlan mpl = merge_plan_for(d, k, r);
    w.basis = std::max(basis_bytes(16 * nb0, basis_kpad_proj(k)), basis_bytes(32 * mpl.NK, basis_kpad_merge(k)));
  }
  size_t a, b, c, e;
  w.rowadam = rowadam_layout(d, a, b, c, e);
  return w;
}

}  // namespace

extern "C" {

size_t logra_workspace_bytes(int64_t T, int64_t d, int64_t k, int32_t r) {
  if (T <= 0 || d <= 0 || k <= 0 || r < 1 || r > LOGRA_MAX_RANK) return 0;
  try {
    const WorkspaceNeed w = workspace_need(T, k, d, r);
    return w.sketch + w.counters + w.rowadam + w.basis;
  } catch (...) {
    return 0;
  }
}

logra_status logra_workspace_reserve(int64_t T, int64_t d, int64_t k, int32_t r, hipStream_t stream) {
  try {
    g_last_error.clear();
    if (T < 0 || d < 0 || k < 0) return fail(LOGRA_ERR_SHAPE, "T, d and k must be >= 0");
    if (r < 1 || r > LOGRA_MAX_RANK) return fail(LOGRA_ERR_RANGE, "r must be in [1, 512]");
    if (T == 0 || d == 0 || k == 0) return LOGRA_OK;
    const WorkspaceNeed w = workspace_need(T, k, d, r);
    void* p = nullptr;
    logra_status st = arena_get(kArenaSketch, stream, w.sketch, &p);
    if (st != LOGRA_OK) return st;
    st = arena_get(kArenaCounters, stream, w.counters, &p);
    if (st != LOGRA_OK) return st;
    if (w.basis) {
      st = arena_get(kArenaBasis, stream, w.basis, &p);
      if (st != LOGRA_OK) return st;
    }
    return arena_get(kArenaRowAdam, stream, w.rowadam, &p);
  } catch (...) {
    return fail(LOGRA_ERR_HIP, "unexpected C++ exception");
  }
}

logra_status logra_workspace_release(hipStream_t stream) {
  try {
    g_last_error.clear();
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone)
      return fail(LOGRA_ERR_RANGE, "the stream is being captured: release its scratch after the capture ends");
    // Work already queued on the stream may still use the buffers.
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    std::lock_guard<std::mutex> lk(g_arena_mu);
    for (int kind = 0; kind < kArenaKinds; ++kind) {
      auto it = g_arenas.find({{dev, kind}, stream});
      if (it == g_arenas.end()) continue;
      Arena& a = it->second;
      for (void* q : a.retired) (void)hipFree(q);
      if (a.ptr) (void)hipFree(a.ptr);
      g_arenas.erase(it);
    }
    return LOGRA_OK;
  } catch (...) {
    return fail(LOGRA_ERR_HIP, "unexpected C++ exception");
  }
}

const char* logra_status_string(logra_status s) {
  // A C caller may pass any int; in C++ a value outside the enumerators'
  // range may not be read as the enum, so read the bits as an int.
  int v;
  static_assert(sizeof(v) == sizeof(s), "logra_status is int-sized");
  std::memcpy(&v, &s, sizeof(v));
  switch (v) {
    case LOGRA_OK: return "ok";
    case LOGRA_ERR_NULL: return "null pointer";
    case LOGRA_ERR_SHAPE: return "bad shape";
    case LOGRA_ERR_ALIGN: return "bad alignment";
    case LOGRA_ERR_RANGE: return "argument out of range";
    case LOGRA_ERR_ALIAS: return "overlapping buffers";
    case LOGRA_ERR_HIP: return "HIP runtime error";
    case LOGRA_ERR_NOMEM: return "out of memory";
  }
  return "unknown status";
}

const char* logra_last_error(void) { return g_last_error.c_str(); }

int logra_abi_version(void) { return LOGRA_ABI_VERSION; }

}  // extern "C"
