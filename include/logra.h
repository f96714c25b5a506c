/*
 * logra.h -- C ABI of the LoGRA low-rank gradient sketch library (MI355X, gfx950).
 *
 * Source of the method: "LoGRA: Scaling LLM Reinforcement Learning with
 * Low-Rank Gradient Sketches" (arXiv 2610.06647v2), section 2.1 ("Low-rank
 * gradient sketches": equations 2-4), section 2.2 (Algorithm 1; "Memory and
 * synchronization") and appendix B (RowAdam, equation 15).
 *
 * Notation.  One linear layer Y = X W^T with W in R^{d x k}.  X (T x k) holds
 * the layer inputs of one microbatch of T tokens, dY (T x d) the gradients of
 * the layer outputs, so the weight gradient is G = dY^T X (d x k).  A = s/sqrt(r)
 * with s in {+1,-1}^{r x k} is the random sign projection, S = G A^T (d x r)
 * the sketch.
 *
 * Conventions shared by every entry point.
 *   - Matrices are row-major; `ld*` is the row stride in ELEMENTS and must be
 *     >= the number of columns.
 *   - Every pointer is a DEVICE pointer on the current HIP device, owned by the
 *     caller; the library keeps no reference after the call returns.
 *   - Work is enqueued on `stream` (0 = the null stream) and the call returns
 *     without synchronising.  Scalar arguments are captured by value.  The
 *     stream must belong to the current device: the calls that take library
 *     scratch (allocated on the current device) return LOGRA_ERR_RANGE for a
 *     stream of another device.
 *   - Validation runs before anything is enqueued; on any error nothing is
 *     written and a nonzero status is returned.  logra_last_error() then gives
 *     a thread-local description.  No C++ exception crosses this boundary.
 *   - 1 <= r <= LOGRA_MAX_RANK (512).  The paper asks only r << min(d, k)
 *     (section 2.1).  Ranks above 256 run as two column halves: sign rows
 *     0..255 into columns 0..255 and rows 256..r-1 into columns 256..r-1 (a
 *     sign depends only on seed, row and column), so they cost one more pass
 *     over X per sketch call.
 *   - NaN and Inf in the inputs propagate to the outputs; nothing traps.
 *
 * Sign generator (this library's fixed choice; the paper only requires
 * independent random signs that the rollout side can regenerate from a seed):
 *   s[i][j] = +1 if bit b is 0, -1 if it is 1, where b is bit (q mod 64) of
 *   word (q / 64) of Philox4x64-10(counter = (j / 256, i, 0, 0),
 *   key = (seed, 0)), q = j mod 256.  Philox4x64-10 is the generator of
 *   Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as
 *   1, 2, 3" (SC'11).  The sign of (i, j) does not depend on r or k.
 */
#ifndef LOGRA_H_
#define LOGRA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOGRA_ABI_VERSION 2
#define LOGRA_MAX_RANK 512

typedef enum {
  LOGRA_OK = 0,
  LOGRA_ERR_NULL = 1,   /* a required pointer is NULL                            */
  LOGRA_ERR_SHAPE = 2,  /* negative size, ld < columns, or sizes that disagree   */
  LOGRA_ERR_ALIGN = 3,  /* base pointer or ld breaks the stated alignment        */
  LOGRA_ERR_RANGE = 4,  /* r, step, beta2 or eps_rel out of range; stream of another device */
  LOGRA_ERR_ALIAS = 5,  /* an output overlaps an input it must not overlap       */
  LOGRA_ERR_HIP = 6,    /* a HIP runtime call or kernel launch failed            */
  LOGRA_ERR_NOMEM = 7   /* the library could not obtain its scratch memory       */
} logra_status;

/*
 * Sketch accumulation (paper section 2.1, equation 2, and Algorithm 1's
 * direct sketch accumulation step):
 *
 *     S[d x r] += (1/sqrt(r)) * dY^T[d x T] * ( X[T x k] * s^T[k x r] )
 *
 * i.e. S += G A^T for this microbatch, computed by projecting the inputs first
 * and never forming G.  Call it once per microbatch with the same seed and r;
 * the caller zeroes S once per training step (Algorithm 1) -- the library
 * only adds.
 *
 *   X    bf16, T x k, row stride ldx (elements).  16-byte aligned base,
 *        ldx a multiple of 8.
 *   dY   bf16, T x d, row stride lddy.  16-byte aligned base, lddy a multiple
 *        of 8.
 *   S    fp32, d x r, row stride lds >= r, read and written.  Must not overlap
 *        X or dY.
 *   T, k, d >= 0; T == 0, k == 0 or d == 0 leaves S unchanged.  X and dY
 *   must each span less than 4 GiB (split larger microbatches into several
 *   calls: the sketch is additive over tokens).
 *
 * Internal scratch (the projected inputs P = X s^T, T x r) is held by the
 * library per (device, stream) and grown on first use of a larger size (see
 * logra_workspace_reserve); concurrent calls on different streams are safe,
 * calls that update the same S must be ordered by the caller.  The result is not bitwise reproducible
 * across runs when the token range is split over several workgroups (fp32
 * atomic adds); any order is within the stated error bound.
 */
logra_status logra_sketch_accumulate(const void* X, int64_t ldx,
                                     const void* dY, int64_t lddy,
                                     int64_t T, int64_t k, int64_t d,
                                     uint64_t seed, int32_t r,
                                     float* S, int64_t lds,
                                     hipStream_t stream);

/*
 * logra_sketch_accumulate for callers that cannot allocate device memory:
 * code being captured into a HIP graph, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, validation, settings (precision,
 * determinism) and result as logra_sketch_accumulate, within the same error
 * bound.  It calls no hipMalloc or hipFree and no allocating library routine:
 * its scratch (P as a bf16 hi/lo pair, the projection's column-split partial
 * sums and their counters) lives in a static device array of
 * LOGRA_NOALLOC_SCRATCH_BYTES bytes, one copy per GPU, held until the process
 * ends; token splits of the contraction add into S with atomic adds instead
 * of parking partial tiles.  The array is found on the first call on each
 * device (one hipGetSymbolAddress).  A call whose scratch would exceed the
 * array (roughly T * 16 * 2^ceil(log2(r/16)) * 4 bytes for P, plus the
 * column-split partials of short microbatches) returns LOGRA_ERR_NOMEM before
 * enqueuing anything: split the microbatch (the sketch is additive over
 * tokens) or use logra_sketch_accumulate.
 *
 * Every call on a GPU shares that GPU's array and leaves its contents
 * behind (the split counters are cleared by a kernel at the start of each
 * call): calls that may overlap on one GPU -- on different streams, or from
 * different threads without ordering -- race and give wrong results.  Order
 * them on one stream, or use logra_sketch_accumulate, whose scratch is per
 * stream.
 */
#define LOGRA_NOALLOC_SCRATCH_BYTES (64ull * 1024ull * 1024ull)
logra_status logra_sketch_accumulate_noalloc(const void* X, int64_t ldx,
                                             const void* dY, int64_t lddy,
                                             int64_t T, int64_t k, int64_t d,
                                             uint64_t seed, int32_t r,
                                             float* S, int64_t lds,
                                             hipStream_t stream);

/*
 * Projection basis (a setting of the calling thread; returns the previous
 * one).  LOGRA_BASIS_RADEMACHER (default): A = s / sqrt(r) with the signs
 * above.  LOGRA_BASIS_GAUSSIAN: the refreshed Gaussian basis the paper
 * compares with it (section 3.4.1, Figure 5c), A = Z / sqrt(r) with Z[i][j]
 * ~ N(0, 1) drawn from the same Philox stream in its own counter range:
 *   block  = Philox4x64-10(counter = (j / 8, i, 1, 0), key = (seed, 0)),
 *            halves h[2m] = low and h[2m+1] = high 32 bits of word m;
 *   pair p = (j mod 8) / 2: u1 = ((h[2p] >> 8) + 1) / 2^24,
 *            u2 = (h[2p+1] >> 8) / 2^24;
 *   Z = sqrt(-2 ln u1) cos(2 pi u2) for even j mod 8, sin for odd (Box and
 *   Muller, 1958), computed in fp32 and carried as bf16 hi/lo pairs.
 * Applies to logra_sketch_accumulate, logra_project, logra_merge_update,
 * logra_merge_update_grouped and logra_payload_pack (which records it per
 * entry).  With the Gaussian basis those calls generate the basis planes
 * (2 bf16 per entry of A, 4 r k bytes for the projection or the merge) into
 * a per-stream region like the other scratch, so the merges then allocate on
 * first use too (see logra_workspace_reserve); logra_sketch_accumulate_noalloc
 * refuses it (LOGRA_ERR_RANGE).  The grouped merge runs one launch per
 * matrix under this basis.
 *
 * logra_basis_normals: writes Z (fp32, r x k, row-major, unscaled) of the
 * Gaussian basis for `seed` into the device buffer `out` (test and debug aid,
 * like logra_signs).
 */
#define LOGRA_BASIS_RADEMACHER 0
#define LOGRA_BASIS_GAUSSIAN 1
int logra_set_basis(int basis);
logra_status logra_basis_normals(uint64_t seed, int32_t r, int64_t k, float* out, hipStream_t stream);

/*
 * Bitwise-reproducible sketches (off by default; a setting of the calling
 * thread).  Atomic adds from several workgroups into the same S entries
 * make S depend on their order at the level of fp32 rounding; any such
 * order is within the stated error bound.  When enabled, logra_sketch_
 * accumulate and logra_contract give every row tile of S to one workgroup,
 * which sums all the tokens in one fixed order and stores without atomic
 * adds, so repeated calls on the same inputs give the same bits.  This is a
 * testing and debugging mode: with few row tiles it runs on few compute
 * units.  Returns the previous setting.
 */
int logra_set_deterministic(int enable);

/*
 * Precision of the contraction and of the merge (a setting of the calling
 * thread; returns the previous mode).  The projected inputs P are fp32 sums;
 * the contraction multiplies them on bf16 matrix cores.
 *
 *   LOGRA_PRECISION_BF16X2 (default): P is carried as a bf16 high part plus
 *     a bf16 low part of the remainder (about 16 significant bits) and each
 *     product takes two MFMAs; S matches an fp64 evaluation to about 1e-5
 *     relative (Frobenius).
 *   LOGRA_PRECISION_BF16: P is rounded once to bf16 (round to nearest even)
 *     and each product takes one MFMA; half the matrix-core work and half the
 *     P traffic.  S then carries the error of that one rounding, about
 *     1.6e-3 relative (Frobenius) on iid data.
 *
 * Applies to logra_sketch_accumulate and logra_sketch_accumulate_noalloc.
 * The split calls always use both planes: logra_project writes them and
 * logra_contract reads them.
 *
 * The mode also sets how the merges (logra_merge_update,
 * logra_merge_update_grouped, logra_rowadam_merge) carry the factor U with
 * the random-sign basis: as a bf16 high/low pair (default; two MFMAs per
 * product) or rounded once to bf16 (one MFMA per product).  The latter puts
 * about 1.1e-3 relative (Frobenius) error into the update before W is
 * rounded; on a weight the update only nudges, W stays within the same
 * tolerance either way.  With the Gaussian basis the merges keep both halves.
 * A trainer and a receiver that must agree bitwise (section 2.2's sync
 * apply) merge in the same mode.
 */
#define LOGRA_PRECISION_BF16X2 0
#define LOGRA_PRECISION_BF16 1
int logra_set_precision(int mode);

/*
 * Split sketch accumulation: project at forward time, contract at backward
 * time.  The paper counts cached projections among the memory the method
 * keeps (section 2.2, "Memory and synchronization") and projects the inputs
 * before the backward derivatives multiply them (section 2.1, after
 * equation 2):
 *
 *     logra_project  :  P  = X[T x k] * s^T[k x r]              (forward)
 *     logra_contract :  S += (1/sqrt(r)) * dY^T[d x T] * P       (backward)
 *
 * Together they add exactly what one logra_sketch_accumulate call adds (the
 * same kernels run); between the two calls the caller keeps P instead of X:
 * 4 * roundup(T, 256) * R bytes against 2 * T * k.
 *
 * The projection cache P is a caller-owned device buffer of at least
 * logra_projection_bytes(T, r) bytes, 16-byte aligned.  Its layout for
 * r <= 256: R = 16 * (the smallest power of two >= ceil(r / 16)) columns,
 * Tc = roundup(T, 256) tokens; a plane of bf16 high parts at byte 0 and a
 * plane of bf16 low parts at byte 2 * Tc * R, each Tc * R entries.  For
 * r > 256 two such caches follow each other: columns 0..255 (R = 256) at
 * byte 0, then columns 256..r-1 as a cache of rank r - 256 at byte
 * 4 * Tc * 256.  Within a plane entry (t, c) sits at
 * index ((((t / 32) * (R / 16) + c / 16) * 64 + ((t % 32) / 8) * 16 + c % 16) * 8
 * + t % 8), the order in which the contraction feeds its matrix cores.  For
 * t < T and c < r, high + low equals P[t][c] = sum_j X[t][j] s[c][j] to about
 * 2^-16 relative (fp32 accumulation, then a bf16 high part and a bf16 low
 * part of the remainder); tokens T <= t < roundup(T, 32) hold zeros; other
 * entries are unspecified.  A cache is valid for the T and r it was made
 * with and is read, not written, by logra_contract.
 *
 *   logra_project:  X as in logra_sketch_accumulate; T, k >= 0 (T == 0 is a
 *                   no-op; k == 0 fills P with zeros); P must not overlap X;
 *                   the whole cache is rewritten.
 *   logra_contract: dY and S as in logra_sketch_accumulate; T, d >= 0 (0 is a
 *                   no-op); S must not overlap dY or P.  The same seed and r
 *                   as the projection are implied by P.
 * Both keep their other scratch (column- and token-split partial sums) per
 * (device, stream) like logra_sketch_accumulate, and return
 * LOGRA_ERR_SHAPE when P_bytes < logra_projection_bytes(T, r).
 */
size_t logra_projection_bytes(int64_t T, int32_t r);

logra_status logra_project(const void* X, int64_t ldx, int64_t T, int64_t k,
                           uint64_t seed, int32_t r,
                           void* P, size_t P_bytes, hipStream_t stream);

logra_status logra_contract(const void* dY, int64_t lddy, int64_t T, int64_t d,
                            const void* P, size_t P_bytes, int32_t r,
                            float* S, int64_t lds, hipStream_t stream);

/*
 * Fused expand-and-merge (paper section 2.1, equations 3 and 4; Algorithm 1's
 * trainer update):
 *
 *     W[d x k] <- RNE_bf16( W - scale * (1/sqrt(r)) * U[d x r] * s[r x k] )
 *
 * in place, with scale = alpha * eta supplied by the host.  U is the sketch S,
 * or S after logra_rowadam_scale.  No d x k update buffer exists: each W tile
 * is read, updated in fp32 and rounded to bf16 (round to nearest, ties to
 * even) once.  Inside the kernel U is carried as a bf16 high/low pair
 * (about 2^-16 relative); the call needs no scratch memory.
 *
 *   W    bf16, d x k, row stride ldw, read and written.  8-byte aligned base,
 *        ldw a multiple of 4.
 *   U    fp32, d x r, row stride ldu >= r, 4-byte aligned.  Must not overlap W.
 *   d, k >= 0 (0 is a no-op).  scale may be any finite float; 0 leaves W
 *   bitwise unchanged.
 */
logra_status logra_merge_update(void* W, int64_t ldw,
                                const float* U, int64_t ldu,
                                int64_t d, int64_t k,
                                uint64_t seed, int32_t r, float scale,
                                hipStream_t stream);

/*
 * Grouped merge: the merge above applied to several matrices of one rank in
 * one launch (Algorithm 1's trainer update for every sketched matrix of a
 * layer, and the rollout side's policy synchronisation, where the engine
 * regenerates each A from its seed and applies the received alpha eta U,
 * section 2.2 "Memory and synchronization").  Item j is
 *
 *     W_j <- RNE_bf16( W_j - scale_j * (1/sqrt(r)) * U_j * s(seed_j) )
 *
 * with each item's arguments and rules exactly those of logra_merge_update;
 * every W_j ends bitwise equal to what logra_merge_update gives for the same
 * item (each matrix keeps its own tiling).  The items array is host memory,
 * read during the call.  All items are validated before anything is
 * enqueued; an item's W may not overlap another item's W or U
 * (LOGRA_ERR_ALIAS).  Items with d == 0, k == 0 or scale == 0 are skipped.
 * Sixteen matrices go to one launch; more are split over several launches.
 */
typedef struct {
  void* W;          /* bf16, d x k, row stride ldw (read and written)  */
  int64_t ldw;
  const float* U;   /* fp32, d x r, row stride ldu                      */
  int64_t ldu;
  int64_t d, k;
  uint64_t seed;
  float scale;      /* alpha * eta for this matrix                      */
} logra_merge_item;

logra_status logra_merge_update_grouped(const logra_merge_item* items, int32_t count,
                                        int32_t r, hipStream_t stream);

/*
 * Synchronisation payload (paper section 2.2, "Memory and synchronization";
 * Algorithm 1, the rollout side's update): after the trainer's merge, the
 * rollout engine receives each sketched matrix's factor -- O(d r) values --
 * with its seed and metadata, regenerates the signs from the seed and applies
 * the factor to its own copy of the weights.
 *
 * The payload is one contiguous byte buffer, little-endian:
 *   bytes 0..31    header: u32 magic LOGRA_PAYLOAD_MAGIC ("LGRP"), u32 version
 *                  (LOGRA_PAYLOAD_VERSION), i32 count, i32 r, u64 total
 *                  bytes, u64 zero;
 *   bytes 32..     count entries of 48 bytes (logra_payload_entry): u64 seed,
 *                  i64 d, i64 k, f32 scale (alpha * eta), u32 basis (the
 *                  packing thread's logra_set_basis setting), u64 byte
 *                  offset of the entry's factor, u64 zero;
 *   from logra_payload_header_bytes(count) (a multiple of 256): each factor U
 *                  as fp32 d x r, rows packed (row stride r), at its offset
 *                  (256-byte aligned).
 * U and alpha*eta travel separately, not as one product: the receiver then
 * runs the merge on exactly the trainer's inputs (U bits, seed, r, fp32
 * scale), and a deterministic merge of the same inputs onto the same W bits
 * gives the same W bits.  Receiver and trainer end bitwise equal when both
 * hold the same W before the update and run this library build with the same
 * tiling (no LOGRA_ tuning variables set); a product alpha*eta*U rounded to
 * fp32 would not give that.
 *
 * logra_payload_bytes: total size for items' d (and r); 0 if count is out of
 *   [1, LOGRA_PAYLOAD_MAX_ITEMS], r out of range or some d < 0 or k < 0.
 * logra_payload_pack: writes the whole payload into the device buffer
 *   `payload` (256-byte aligned, at least logra_payload_bytes bytes) on
 *   `stream` from items' U (ldu >= r), d, k, seed and scale (W and ldw are
 *   not read).  U must not overlap the payload.
 * logra_payload_parse: host-side check of a host copy of the first
 *   logra_payload_header_bytes(count) bytes (or more): magic, version, count
 *   in range, every factor inside total bytes and 256-byte aligned, sizes
 *   consistent.  Fills *header and entries[0 .. count-1] (max_entries of
 *   room).  LOGRA_ERR_SHAPE for a malformed or truncated header,
 *   LOGRA_ERR_RANGE when count exceeds max_entries.
 * logra_payload_apply: the receiver's merge: W_j <- RNE_bf16(W_j - scale_j
 *   (1/sqrt(r)) U_j A(seed_j)) for every entry, in the entry's basis
 *   (whatever the calling thread's setting), through
 *   logra_merge_update_grouped with U_j read from the device payload
 *   (`payload_bytes` bytes) at entry j's offset.  W[j] and ldw[j] are the
 *   receiver's weights (host arrays of count pointers and strides); the
 *   header and entries are those logra_payload_parse returned.
 */
#define LOGRA_PAYLOAD_MAGIC 0x5052474Cu
#define LOGRA_PAYLOAD_VERSION 1
#define LOGRA_PAYLOAD_MAX_ITEMS 32
typedef struct {
  uint32_t magic, version;
  int32_t count, r;
  uint64_t total_bytes;
  uint64_t reserved;
} logra_payload_header;
typedef struct {
  uint64_t seed;
  int64_t d, k;
  float scale;
  uint32_t basis;   /* LOGRA_BASIS_RADEMACHER or LOGRA_BASIS_GAUSSIAN */
  uint64_t u_offset;
  uint64_t reserved1;
} logra_payload_entry;

size_t logra_payload_header_bytes(int32_t count);
size_t logra_payload_bytes(const logra_merge_item* items, int32_t count, int32_t r);
logra_status logra_payload_pack(const logra_merge_item* items, int32_t count, int32_t r,
                                void* payload, size_t payload_bytes, hipStream_t stream);
logra_status logra_payload_parse(const void* header_host, size_t bytes, logra_payload_header* header,
                                 logra_payload_entry* entries, int32_t max_entries);
logra_status logra_payload_apply(const void* payload, size_t payload_bytes,
                                 const logra_payload_header* header, const logra_payload_entry* entries,
                                 void* const* W, const int64_t* ldw, hipStream_t stream);

/*
 * RowAdam row scaling (paper appendix B, equation 15), S -> U in place:
 *
 *     m_i   = (1/r) sum_j S_ij^2
 *     v_i  <- beta2 v_i + (1 - beta2) m_i
 *     vh_i  = v_i / (1 - beta2^step)
 *     eps   = max(eps_rel * mean_i sqrt(vh_i), 1e-30)
 *     Ut_i  = S_i / (sqrt(vh_i) + eps)
 *     U     = Ut * ||S||_F / ||Ut||_F        (U = 0 when ||Ut||_F = 0)
 *
 * Readings of words the appendix text lost: the stabiliser uses the MEAN over
 * rows of sqrt(vh); the rescale restores the Frobenius norm of the incoming
 * sketch; the sketch is used as passed in.
 *
 *   S     fp32, d x r, row stride lds >= r, overwritten with U.
 *   v     fp32, d values, the per-row second moment, read and written; starts
 *         at zero and persists across projection refreshes.  Must not overlap S.
 *   step  >= 1, counts RowAdam updates of this matrix.
 *   0 <= beta2 < 1, eps_rel >= 0.
 * All reductions stay on the device; the result is deterministic.
 */
logra_status logra_rowadam_scale(float* S, int64_t lds, float* v,
                                 int64_t d, int32_t r, int64_t step,
                                 float beta2, float eps_rel,
                                 hipStream_t stream);

/*
 * RowAdam folded into the merge: W <- RNE_bf16(W - scale (1/sqrt(r)) U A)
 * with U = RowAdam(S) as logra_rowadam_scale defines it, without writing U:
 * the RowAdam statistics give one fp32 factor per row and the merge
 * multiplies each entry of S by its row's factor as it loads it.  v is
 * updated as by logra_rowadam_scale; S is only read.  W and v end bitwise
 * equal to logra_rowadam_scale on a copy of S followed by logra_merge_update
 * (same basis setting), and one read and write of S fewer.  Arguments and
 * checks are those of the two calls (S in the role of U; W may overlap
 * neither S nor v); k == 0 updates v only.
 */
logra_status logra_rowadam_merge(void* W, int64_t ldw, const float* S, int64_t lds, float* v,
                                 int64_t d, int64_t k, uint64_t seed, int32_t r, int64_t step,
                                 float beta2, float eps_rel, float scale, hipStream_t stream);

/*
 * Predicted KL of a proposed update (paper section 2.3, equation 6; derived in
 * appendix A.1):
 *
 *     q = 1 / (2 n T^2) * sum_{s < n} Var_{v ~ p(s)}[ zdot[s][v] ],
 *     p(s) = softmax(z[s][.] / T) over the V vocabulary entries,
 *
 * where row s of z holds the logits at one examined context and row s of
 * zdot their rates of change along the proposed update D (evaluated before
 * the update is applied; the caller computes them, e.g. with a forward-mode
 * pass through the factors -eta U A, appendix A.1).  Var is the
 * p-weighted variance.  One streaming pass over both arrays; per-row states
 * are merged in a fixed order, so the result is deterministic.
 *
 *   z, zdot  n x V, row strides ldz, ldzd >= V (elements); dtype
 *            LOGRA_DTYPE_F32 (float) or LOGRA_DTYPE_BF16 (bfloat16), the same
 *            for both.  16-byte aligned bases; with n > 1 every row must
 *            start on a 16-byte boundary (ld a multiple of 4 floats or 8 bf16).  A row
 *            spans less than 2 GiB.
 *   temperature  T > 0, finite (the sampling temperature of p).
 *   row_var  optional (NULL to skip): n floats receiving Var per row.
 *   q        one float receiving q.  n == 0 writes q = 0.
 * A row whose logits are all -inf has no distribution: its Var, and q, are
 * NaN.  NaN inputs propagate.  Neither output may overlap z, zdot or the
 * other output.  V == 0 with n > 0 is LOGRA_ERR_SHAPE.  Scratch (32 bytes per
 * row and column range) is held per (device, stream).
 */
#define LOGRA_DTYPE_F32 0
#define LOGRA_DTYPE_BF16 1
logra_status logra_predicted_kl(const void* z, int64_t ldz,
                                const void* zdot, int64_t ldzd,
                                int64_t n, int64_t V, int32_t dtype,
                                float temperature,
                                float* row_var, float* q,
                                hipStream_t stream);

/*
 * Host helpers of the KL-budget step rule (no device work).
 *
 * logra_kl_step_scale: alpha = min(alpha_max, sqrt(delta / q)) (section 2.3,
 *   equation 7; appendix A.2).  q == 0 gives alpha_max, q == +inf gives 0;
 *   NaN for q < 0, NaN q, delta <= 0 or alpha_max <= 0.
 * logra_kl_budget: delta_u = delta_min + (delta_max - delta_min) / 2 *
 *   (1 + cos(pi (u - 1) / (H - 1))) for update u = 1..H (appendix D.1,
 *   equation 16); u is clamped to [1, H] (the budget stays at delta_min after
 *   the schedule); H < 2 gives delta_min.
 * logra_kl_effective_budget: max(delta - kappa, delta / 2) (appendix D.1,
 *   equation 17), kappa the smoothed rollout-minus-trainer log-probability
 *   mismatch, clamped below at zero; NaN kappa (no valid measurement) gives
 *   delta unchanged.
 */
double logra_kl_step_scale(double q, double delta, double alpha_max);
double logra_kl_budget(int64_t u, int64_t H, double delta_max, double delta_min);
double logra_kl_effective_budget(double delta, double kappa);

/*
 * Materialise the signs s (r x k) as int8 (+1 / -1), row-major, row stride k,
 * into `out` (device).  A test and debugging aid: the hot path never stores
 * the signs.
 */
logra_status logra_signs(uint64_t seed, int32_t r, int64_t k, int8_t* out,
                         hipStream_t stream);

/* Measurement aid (not part of the method): streams `bytes` bytes from the
 * device buffer `ptr` with 16-byte loads, four per thread in flight, and
 * discards them (only a one-in-2^32 xor value is written to the device word
 * *sink).  Timing it over the bytes one sketch call reads gives the GPU's
 * streaming-read ceiling for that call.  ptr 16-byte aligned, bytes a
 * multiple of 16 (LOGRA_ERR_ALIGN otherwise); bytes == 0 is a no-op. */
logra_status logra_stream_read(const void* ptr, size_t bytes, uint32_t* sink, hipStream_t stream);

/*
 * Library scratch per (device, stream).  logra_sketch_accumulate, the split
 * calls and logra_rowadam_scale take scratch (P as a bf16 hi/lo pair,
 * column- and token-split partial sums, split counters, RowAdam's row
 * statistics) from regions the library keeps per (device, stream).  A region
 * grows, by hipMalloc and a clearing hipMemsetAsync on the stream, the first
 * time a call needs more than it holds, and never shrinks; a buffer it
 * outgrows is retired, not freed, because a graph captured earlier may still
 * launch kernels that use it.  Growing is refused with LOGRA_ERR_NOMEM while
 * the stream is being captured (allocation cannot be captured): reserve
 * before capturing.
 *
 * logra_workspace_bytes: the scratch, in bytes, that the sketch calls (fused
 * and split) and logra_rowadam_scale need for one shape with the calling
 * thread's settings (precision, determinism); 0 for an empty or invalid
 * shape.  logra_predicted_kl's scratch is not included.
 *
 * logra_workspace_reserve: grows the stream's regions to that size now (on
 * the current device).  After it, calls of that shape, or smaller ones whose
 * plans fit, on that stream allocate nothing and may be captured into a graph.
 * Errors: LOGRA_ERR_SHAPE / LOGRA_ERR_RANGE for bad arguments,
 * LOGRA_ERR_NOMEM when the allocation fails or the stream is being captured.
 *
 * logra_workspace_release: waits for the stream's queued work, then frees
 * every region the library holds for the stream on the current device,
 * current and retired.  A graph captured before must not be launched after
 * it.  Refused (LOGRA_ERR_RANGE) while the stream is being captured.
 */
size_t logra_workspace_bytes(int64_t T, int64_t d, int64_t k, int32_t r);
logra_status logra_workspace_reserve(int64_t T, int64_t d, int64_t k, int32_t r, hipStream_t stream);
logra_status logra_workspace_release(hipStream_t stream);

/* Static text for a status code. */
const char* logra_status_string(logra_status s);

/* Thread-local description of the last failure on this thread ("" if none). */
const char* logra_last_error(void);

/* LOGRA_ABI_VERSION of the built library. */
int logra_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LOGRA_H_ */
