/*
 * rgc.h -- C ABI of the randomized low-rank gradient-sketch library (gfx950).
 *
 * One linear layer W (d x k, out x in) is trained from a rank-r sketch of its
 * gradient instead of the dense gradient:
 *
 *   1. P  = rgc_sample_projection(seed)      k x r, fixed for one accumulation
 *   2. XP = rgc_project(X, P)                the layer keeps XP (T x r), not X
 *   3. C += rgc_accumulate(D, XP)            C = D^T (X P), d x r, fp32
 *   4. W  = rgc_apply(W, C, P)               W <- SR_bf16(W - tau*||W||*H/||H||),
 *                                            H = C P^T rebuilt in tiles, never stored
 *
 * Sources, by page title and section:
 *   [RGC]     "Randomized Gradient Compression": "How it works" (C += D^T (X P),
 *             the saved X P, H = C P^T rebuilt 128 rows at a time, the normalized
 *             update, bf16 weights with stochastic rounding), footnote 1 (the
 *             QR-of-Gaussian frame scaled by sqrt(input width / rank)).
 *   [LoGRA-S] "LoGRA: Scaling LLM Reinforcement Learning with Low-Rank Gradient
 *             Sketches": Key Contributions item 1 (fp32 sketch S = G A^T, d x r,
 *             accumulated per microbatch, never forming G).
 *   [LoGRA-M] "LoGRA: Low-Rank Gradient Sketches": "Why the Sketch Can Be
 *             Accumulated Without a Full Gradient" (random signs scaled by
 *             1/sqrt(r)), "Minimal Causal Code" (caller-zeroed fp32 sketch,
 *             projection regenerated from a seed).
 *
 * Conventions for every call:
 *   - bf16 tensors travel as uint16_t bit patterns; all matrices are row-major.
 *   - Every tensor pointer is a DEVICE pointer owned by the caller. The library
 *     allocates no memory, keeps no pointer after a call returns and has no
 *     mutable global state. Buffers passed to one call must not alias each
 *     other (except where noted).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every
 *     call only enqueues kernels on it and never synchronizes; results are
 *     ready when the stream reaches them.
 *   - Workspaces: device scratch of at least the queried size (0 means none
 *     is needed), 256-byte aligned, owned by the caller. Its contents need no
 *     initialisation and are dead after the call's kernels complete, so one
 *     workspace can serve any sequence of calls ordered on a stream; calls
 *     that may run concurrently need separate workspaces.
 *   - Results depend only on the arguments and the device's compute-unit
 *     count (which sets the work partition and so the fp32 summation order);
 *     no environment variable or other process state changes them.
 *   - Arguments are validated on the host before anything is enqueued; on any
 *     error nothing is launched and no buffer changes. Conditions that are only
 *     known on the device (a zero sketch, non-finite values) are reported
 *     through `stats` (rgc_apply).
 *   - Shape limits: r is 4, 8 or any multiple of 16 up to 256 (QR
 *     projections: 4, 8 or a multiple of 16 up to 128); ranks 4 and 8 run
 *     small-rank kernels (VALU sums; H formed in fp32 in rank order, its norm
 *     from fp64 Gram matrices); d and k are multiples of 8; T >= 0 (T = 0 is a
 *     no-op); T and d at most 65536 per call; leading dimensions are
 *     multiples of 8 elements and at most 2^23 (RGC_ERR_UNSUPPORTED above);
 *     for rgc_apply, d and k at most 2^30 and d*k at most 2^38;
 *     tensor base pointers are 16-byte aligned.
 */
#ifndef RGC_H
#define RGC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RGC_ABI_VERSION 6

typedef enum {
  RGC_OK = 0,
  RGC_ERR_NULL = 1,        /* a required pointer is NULL */
  RGC_ERR_SHAPE = 2,       /* a dimension is negative, r > k, or ld < width */
  RGC_ERR_UNSUPPORTED = 3, /* r or d/k outside the supported set (see the shape limits) */
  RGC_ERR_ALIGN = 4,       /* a base pointer or leading dimension is misaligned */
  RGC_ERR_WORKSPACE = 5,   /* workspace missing or smaller than the query */
  RGC_ERR_HIP = 6,         /* a kernel launch failed */
  RGC_ERR_VALUE = 7,       /* a scalar argument is not finite */
  RGC_ERR_SCRATCH = 8      /* rgc_apply_noalloc: more scratch needed than its static buffer holds */
} rgc_status_t;

typedef enum {
  /* Entries +-bf16(1/sqrt(r)) from counter-based sign bits [LoGRA-M]. */
  RGC_PROJ_RADEMACHER = 0,
  /* sqrt(k/r) * Q, Q the sign-corrected QR factor of a Gaussian k x r matrix,
   * computed by CholeskyQR2 in fp64 and rounded fp64 -> fp32 -> bf16 [RGC, fn 1]. */
  RGC_PROJ_QR_GAUSSIAN = 1
} rgc_proj_kind_t;

int rgc_abi_version(void);
const char* rgc_status_string(rgc_status_t status);

/* ---- 1. Projection ------------------------------------------------------ */

/* Workspace bytes rgc_sample_projection needs for (kind, k, r); 0 means none. */
size_t rgc_sample_projection_workspace_size(rgc_proj_kind_t kind, int64_t k, int64_t r);

/* Fill P (k x r bf16, row-major, leading dimension r) from `seed`.
 * Rademacher: one Philox4x32-10 call (counter (i, j/128, 1, 0), key = seed)
 *   per row i and block of 128 columns; bit (j % 32) of word ((j / 32) % 4) set
 *   gives -a, clear gives +a, a = bf16(1/sqrt(r)).
 * QR-Gaussian: A[i][j] Box-Muller normals from Philox (counter (i, j/4, 2, 0),
 *   key = seed; columns 4q,4q+1 use words 0,1 and 4q+2,4q+3 use words 2,3;
 *   u = (w + 1/2) / 2^32; even column rho*cos, odd column rho*sin); then
 *   Q = A R^-1 with R upper triangular, diag(R) > 0 (CholeskyQR2, fp64);
 *   P = bf16(fp32(sqrt(k/r) * Q)). Needs a workspace (see the query).
 *   If a Cholesky factorization fails (a Gram matrix that is not numerically
 *   positive definite: for a Gaussian draw with k >= r practically never),
 *   P is written as all NaN; every update from such a P is then skipped
 *   (flag = 1 in its stats, W left bit-identical).
 * The same (kind, seed, k, r) always gives the same bits, on any device. */
rgc_status_t rgc_sample_projection(rgc_proj_kind_t kind, uint64_t seed, int64_t k, int64_t r,
                                   uint16_t* P, void* ws, size_t ws_bytes, void* stream);

/* Batched form for the projections of several matrices with the same rank
 * (e.g. all projections of one transformer block): P[m] is filled exactly as
 * rgc_sample_projection(kind, seeds[m], ks[m], r, P[m], ...) would fill it,
 * but each step of the QR pipeline is one launch for the whole batch.
 * seeds, ks and Ps are HOST arrays of n entries (n <= 16); the P[m] are
 * device pointers. The workspace query takes the same ks. */
size_t rgc_sample_projections_workspace_size(rgc_proj_kind_t kind, int64_t n, const int64_t* ks, int64_t r);
rgc_status_t rgc_sample_projections(rgc_proj_kind_t kind, int64_t n, const uint64_t* seeds, const int64_t* ks,
                                    int64_t r, uint16_t* const* Ps, void* ws, size_t ws_bytes, void* stream);

/* ---- 2. Projected activations --------------------------------------------- */

/* Workspace bytes rgc_project needs (split-k partial sums). */
size_t rgc_project_workspace_size(int64_t T, int64_t k, int64_t r);

/* XP = bf16_rne(X P) [RGC, "How it works": the layer keeps X P, not X].
 * X: T x k bf16, row stride ldx (>= k). P: k x r bf16 (row stride r).
 * XP: T x r bf16, row stride r. Products of bf16 in fp32 (MFMA), fp32 sums in a
 * fixed order (deterministic), one rounding to bf16. */
rgc_status_t rgc_project(const uint16_t* X, int64_t ldx, const uint16_t* P, uint16_t* XP,
                         int64_t T, int64_t k, int64_t r, void* ws, size_t ws_bytes, void* stream);

/* Batched form: n independent projections (n <= 16, one rank r, one token
 * count T) in one launch, e.g. all projections of a transformer block for one
 * microbatch (items may share an X, which then streams from cache). Item m
 * computes XPs[m] = bf16(Xs[m] Ps[m]) with X of width ks[m] and row stride
 * ldxs[m], exactly as rgc_project does (same rounding; the fp32 summation
 * order may differ). Xs, ldxs, ks, Ps, XPs are HOST arrays of n entries. */
size_t rgc_project_batch_workspace_size(int64_t n, const int64_t* ks, int64_t T, int64_t r);
rgc_status_t rgc_project_batch(int64_t n, const uint16_t* const* Xs, const int64_t* ldxs, const int64_t* ks,
                               const uint16_t* const* Ps, uint16_t* const* XPs, int64_t T, int64_t r, void* ws,
                               size_t ws_bytes, void* stream);

/* One pass over a shared X [RGC, "How it works": every projection of a layer
 * keeps X P]: XPs[i] = bf16(X Ps[i]) for the n <= 4 projections of the
 * matrices that read the same input X (a block's q, k and v; gate and up),
 * with X streamed from memory once for all of them: the rank operand is the
 * n projections side by side (n * r <= 256 ranks; r a multiple of 16). X: T
 * x k bf16, row stride ldx; Ps[i]: k x r bf16; XPs[i]: T x r bf16; Ps and
 * XPs are HOST arrays of n device pointers. Rounding as rgc_project (the
 * fp32 summation order may differ). rgc_project_batch does not group items
 * itself: on the Qwen3-shaped blocks the grouped schedule measured slower
 * than one item per matrix (per-CU streaming, not the repeated X reads,
 * bounds the project there). */
size_t rgc_project_shared_workspace_size(int64_t n, int64_t T, int64_t k, int64_t r);
rgc_status_t rgc_project_shared(int64_t n, const uint16_t* X, int64_t ldx, int64_t k, const uint16_t* const* Ps,
                                uint16_t* const* XPs, int64_t T, int64_t r, void* ws, size_t ws_bytes, void* stream);

/* ---- 3. Sketch accumulation ----------------------------------------------- */

/* Workspace bytes rgc_accumulate needs (split-token partial sums). */
size_t rgc_accumulate_workspace_size(int64_t T, int64_t d, int64_t r);

/* C += D^T XP over this microbatch's T tokens [RGC, "How it works"; LoGRA-S,
 * Key Contributions 1]. D: T x d bf16 (row stride ldd >= d) = dL/dY of the
 * layer's output. XP: T x r bf16 (row stride r) from rgc_project. C: d x r
 * fp32 (row stride r), read-modify-written; it only adds, so the caller zeroes
 * C once per update (as the pages' loop does). Products in fp32 on MFMA, token
 * partial sums reduced in a fixed order (bit-reproducible). */
rgc_status_t rgc_accumulate(const uint16_t* D, int64_t ldd, const uint16_t* XP, float* C,
                            int64_t T, int64_t d, int64_t r, void* ws, size_t ws_bytes,
                            void* stream);

/* Batched form: n independent accumulations (n <= 16, one rank r, one token
 * count T) in one launch: Cs[m] += Ds[m]^T XPs[m], D of width ds[m] and row
 * stride ldds[m]. All arrays are HOST arrays of n entries. */
size_t rgc_accumulate_batch_workspace_size(int64_t n, const int64_t* ds, int64_t T, int64_t r);
rgc_status_t rgc_accumulate_batch(int64_t n, const uint16_t* const* Ds, const int64_t* ldds, const int64_t* ds,
                                  const uint16_t* const* XPs, float* const* Cs, int64_t T, int64_t r, void* ws,
                                  size_t ws_bytes, void* stream);

/* Deferred form for the microbatches of one accumulation (the calls that add
 * into the same Cs before the next update): the work split between
 * workgroups leaves fp32 partial sums for some tiles, and here they stay in the
 * workspace from call to call, added there, and reach C once, in the call that
 * ends the accumulation, instead of in a finishing pass after every call.
 * phase: bit 0 set = the first call of the accumulation, bit 1 set = the last;
 * 3 = a single call (exactly rgc_accumulate_batch). C holds the full sum only
 * after the last call; in between it holds part of it. Every call of one
 * accumulation must have the same n, ds, T and r, run on the same device and
 * use the same workspace, which no other call may use in between (its contents
 * carry the partial sums; this is not checked). The sum differs from the
 * per-call form's only in the fp32 addition order; it is bit-reproducible.
 * Ranks 4 and 8 complete C in every call whatever the phase. */
rgc_status_t rgc_accumulate_batch_deferred(int64_t n, const uint16_t* const* Ds, const int64_t* ldds,
                                           const int64_t* ds, const uint16_t* const* XPs, float* const* Cs,
                                           int64_t T, int64_t r, void* ws, size_t ws_bytes, int phase,
                                           void* stream);

/* ---- 4. Normalized update with stochastic rounding ------------------------ */

/* Workspace bytes rgc_apply needs (per-workgroup norm partials, for r <= 128
 * also partial Gram matrices, and the step scalar). */
size_t rgc_apply_workspace_size(int64_t d, int64_t k, int64_t r);

/* W <- SR_bf16(W - s * H), H = C P^T, s = fp32(tau * ||W||_F / ||H||_F)
 * [RGC, "How it works"]. W: d x k bf16 (row stride ldw >= k), updated in place;
 * C: d x r fp32; P: k x r bf16. H is rebuilt tile by tile in registers (MFMA,
 * C split into two bf16 terms) and never written to memory. For r <= 128,
 * ||H||_F^2 is taken as sum((C^T C) o (P^T P)) (equal to it up to rounding);
 * a C whose squares overflow fp32 then reads as a non-finite ||H||. The pre-rounding
 * value is v = fp32(w - fp32(s*h)) (no fused multiply-add); stochastic
 * rounding adds 16 random bits to v's low half and keeps the high half, the
 * bits coming from Philox4x32-10 (counter (j/8, i, 3, 0), key = seed; column j
 * uses word (j%8)/2, low half for even j). When ||H|| = 0 or s is not finite
 * the update is skipped: W is left bit-identical and flag = 1.
 * stats: NULL or device float[4] receiving {||W||, ||H||, s, flag}. */
rgc_status_t rgc_apply(uint16_t* W, int64_t ldw, const float* C, const uint16_t* P, int64_t d,
                       int64_t k, int64_t r, float tau, uint64_t seed, float* stats, void* ws,
                       size_t ws_bytes, void* stream);

/* rgc_apply for n <= 16 matrices of one rank r (e.g. the projections of a
 * block) in three or four launches: the norms (W streamed for ||W||, the
 * Gram partials of C and P for ||H||; one launch up to r = 64, two above),
 * one step scalar per matrix, an update sweep. Item m: W Ws[m] (ds[m] x ks[m], row stride
 * ldws[m]), C Cs[m] (ds[m] x r), P Ps[m] (ks[m] x r), rounding seed seeds[m],
 * stats NULL or stats[m] NULL or device float[4]. All arrays are HOST arrays
 * of n entries; tau is shared. Each matrix gets exactly the bits that
 * rgc_apply would give it alone. */
size_t rgc_apply_batch_workspace_size(int64_t n, const int64_t* ds, const int64_t* ks, int64_t r);
rgc_status_t rgc_apply_batch(int64_t n, uint16_t* const* Ws, const int64_t* ldws, const float* const* Cs,
                             const uint16_t* const* Ps, const int64_t* ds, const int64_t* ks, int64_t r,
                             float tau, const uint64_t* seeds, float* const* stats, void* ws,
                             size_t ws_bytes, void* stream);

/* ---- The normalized update without a workspace ---------------------------
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. Computes
 * exactly what rgc_apply computes (same kernels, same partition, same bits),
 * with rgc_apply's workspace taken from a static device buffer of
 * RGC_NOALLOC_SCRATCH_BYTES bytes that the library holds on each device it
 * runs on, for as long as it stays loaded. The call allocates nothing.
 * - Calls whose workspace (rgc_apply_workspace_size(d, k, r)) would exceed
 *   that buffer return RGC_ERR_SCRATCH before anything is enqueued; with
 *   8 MiB this holds e.g. every matrix up to 32768 x 32768 at r <= 128.
 * - Every call on one device shares the buffer: calls that may overlap on one
 *   device (different streams without ordering, or concurrent host threads)
 *   race and must not be made; calls ordered on one stream are fine.
 * - `stream` must belong to the current device (RGC_ERR_UNSUPPORTED
 *   otherwise); the first call on a device looks the buffer's address up.
 * Arguments, stats and the other errors as rgc_apply. */
#define RGC_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
rgc_status_t rgc_apply_noalloc(uint16_t* W, int64_t ldw, const float* C, const uint16_t* P, int64_t d,
                               int64_t k, int64_t r, float tau, uint64_t seed, float* stats, void* stream);

/* ---- The normalized update with a carried ||W|| --------------------------
 *
 * rgc_apply's update ([RGC], "How it works") where ||W||_F^2 is not streamed
 * from W but carried over from the previous update, which summed the squares
 * of the bf16 weights as it wrote them: the apply then reads W once and
 * writes it once (4dk bytes instead of 6dk). The step uses the same formula
 * and the same rounding bits as rgc_apply; its ||W|| is the same number up to
 * the order of the fp64 sum, so s can differ from rgc_apply's in its last
 * bit.
 * wnorm2: device double[n] (8-byte aligned), owned by the caller. fresh != 0:
 *   on entry its contents are ignored and ||W||^2 is streamed from W as in
 *   rgc_apply (first call, or after W changed outside these calls); fresh ==
 *   0: on entry wnorm2[m] must hold ||W_m||_F^2 of the weights as they stand,
 *   normally as a previous call left it. On return wnorm2[m] holds
 *   ||W'_m||_F^2 of the weights this call wrote (fp32 sums of eight squares,
 *   fp64 across them, fixed order, so repeated calls give the same bits); a
 *   skipped update (flag = 1) leaves W and the entry as they were (with
 *   fresh != 0, the streamed ||W||^2). A value that does not match W is not
 *   detected: the step is then scaled by the wrong norm.
 * Other arguments, the workspace (rgc_apply_batch_workspace_size) and errors
 * as rgc_apply_batch; wnorm2 NULL gives RGC_ERR_NULL. Four launches: the
 * norms (at r <= 128 the Gram partials of C and P, plus the W stream only
 * when fresh != 0), one step scalar per matrix, the update with the squares,
 * one sum per matrix. At r > 128 the norms launch rebuilds H from the W tiles
 * it reads, so there it reads W whatever fresh says. */
rgc_status_t rgc_apply_carried_batch(int64_t n, uint16_t* const* Ws, const int64_t* ldws,
                                     const float* const* Cs, const uint16_t* const* Ps, const int64_t* ds,
                                     const int64_t* ks, int64_t r, float tau, const uint64_t* seeds,
                                     float* const* stats, double* wnorm2, int fresh, void* ws,
                                     size_t ws_bytes, void* stream);
rgc_status_t rgc_apply_carried(uint16_t* W, int64_t ldw, const float* C, const uint16_t* P, int64_t d,
                               int64_t k, int64_t r, float tau, uint64_t seed, float* stats,
                               double* wnorm2, int fresh, void* ws, size_t ws_bytes, void* stream);

/* ---- The fixed-scale update ([LoGRA-M], "Minimal Causal Code") -----------
 *
 * W <- SR_bf16(W - alpha * H), H = C P^T: the tutorial's plain-SGD update
 * W -= alpha*eta*(U @ A) with U = S (the sketch, here C) and A = P^T, the
 * step alpha*eta passed as one fp32 scalar `alpha` chosen by the caller (the
 * pages' KL-based step controller stays with the caller). No norms are taken
 * and nothing is skipped: the update runs in one launch, with the same H
 * tiles, pre-rounding value v = fp32(w - fp32(alpha*h)) and rounding bits as
 * rgc_apply (so rgc_apply_scaled with alpha = the s that rgc_apply reports in
 * stats[2] gives rgc_apply's bits). The pages do not say how LoGRA rounds its
 * bf16 weights; this library keeps no fp32 copy and rounds stochastically as
 * for [RGC]. A non-finite alpha returns RGC_ERR_VALUE; non-finite values in C
 * give non-finite weights, as the dense update would. No workspace. */
rgc_status_t rgc_apply_scaled(uint16_t* W, int64_t ldw, const float* C, const uint16_t* P, int64_t d,
                              int64_t k, int64_t r, float alpha, uint64_t seed, void* stream);

/* rgc_apply_scaled for n <= 16 matrices of one rank r in one launch; alphas
 * and the other arrays are HOST arrays of n entries (as rgc_apply_batch). */
rgc_status_t rgc_apply_scaled_batch(int64_t n, uint16_t* const* Ws, const int64_t* ldws,
                                    const float* const* Cs, const uint16_t* const* Ps,
                                    const int64_t* ds, const int64_t* ks, int64_t r,
                                    const float* alphas, const uint64_t* seeds, void* stream);

/* ---- Applying a received sketch from its projection seed ------------------
 *
 * The receiving side of a policy update ([LoGRA-S], Key Contributions item 2;
 * [LoGRA-M], "Why Refreshing the Projection Enables New Update Directions"):
 * only the d x r factor and the projection seed travel; the receiver
 * regenerates P (k x r, `kind`, `proj_seed`) in the workspace and applies the
 * update. mode RGC_UPDATE_NORMALIZED: rgc_apply with tau = `step` (stats as
 * there, may be NULL); RGC_UPDATE_SCALED: rgc_apply_scaled with alpha = `step`
 * (stats must be NULL). Given the same W, C, seeds and step, the result is bit
 * for bit what the sender computes with its own P. */
typedef enum { RGC_UPDATE_NORMALIZED = 0, RGC_UPDATE_SCALED = 1 } rgc_update_mode_t;

size_t rgc_apply_from_seed_workspace_size(rgc_proj_kind_t kind, int64_t d, int64_t k, int64_t r);
rgc_status_t rgc_apply_from_seed(rgc_update_mode_t mode, rgc_proj_kind_t kind, uint64_t proj_seed,
                                 uint16_t* W, int64_t ldw, const float* C, int64_t d, int64_t k,
                                 int64_t r, float step, uint64_t seed, float* stats, void* ws,
                                 size_t ws_bytes, void* stream);

/* ---- The layer's own products either side of the sketch ------------------
 *
 * [RGC, "How it works"]: the forward keeps X P instead of X and the backward
 * adds D^T (X P) to C; [LoGRA-M, "Minimal Causal Code"]: the projection
 * belongs inside the layer's own products. These calls make the layer's
 * dense products themselves on the library's kernels, with the sketch steps
 * attached, so a layer needs no other GEMM:
 *
 * Forward: Y = bf16_rne(X W^T) and XP = bf16_rne(X P) from one tile grid
 * over the output columns [d columns of Y | r columns of XP]: P's columns are
 * one more column of tiles beside W's, so X is staged once per tile row for
 * both and the projection adds no pass of its own over X.
 *   X: T x k bf16, row stride ldx; W: d x k bf16 (out x in), row stride ldw;
 *   P: k x r bf16 (row stride r); Y: T x d bf16, row stride ldy; XP: T x r
 *   bf16 (row stride r). r = 0 (P and XP may then be NULL) computes Y alone.
 *   Each output element is one fp32 sum over k in ascending order (MFMA
 *   products of bf16), then one rounding: bit-reproducible. XP is equal to
 *   rgc_project's up to the fp32 summation order. At r = 4 (narrower than
 *   the kernel's 16-byte P chunks) XP comes from the small-rank project after
 *   the grid, a second pass over X.
 * The batched form takes HOST arrays of n <= 16 entries (one T, one r); items
 * may share X (a block's q, k and v; gate and up). No workspace. */
rgc_status_t rgc_linear_forward(const uint16_t* X, int64_t ldx, const uint16_t* W, int64_t ldw,
                                const uint16_t* P, uint16_t* Y, int64_t ldy, uint16_t* XP, int64_t T,
                                int64_t d, int64_t k, int64_t r, void* stream);
rgc_status_t rgc_linear_forward_batch(int64_t n, const uint16_t* const* Xs, const int64_t* ldxs,
                                      const int64_t* ks, const uint16_t* const* Ws, const int64_t* ldws,
                                      const int64_t* ds, const uint16_t* const* Ps, uint16_t* const* Ys,
                                      const int64_t* ldys, uint16_t* const* XPs, int64_t T, int64_t r,
                                      void* stream);

/* Backward: dX = bf16_rne(D W) (T x k, row stride lddx; one fp32 sum over d
 * in ascending order per element), then C += D^T XP exactly as
 * rgc_accumulate does (same kernels, same bits), both enqueued by this one
 * call on `stream`, the accumulate right after the dX grid while D is still
 * in the last-level cache. D: T x d bf16, row stride ldd; W: d x k bf16, row
 * stride ldw; XP: T x r bf16; C: d x r fp32. r = 0 (XP and C may then be
 * NULL) computes dX alone. The workspace is rgc_accumulate's (query below).
 * Both calls: d and k multiples of 8, ld* multiples of 8, 16-byte aligned
 * pointers, r in {0, 4, 8, 16, 32, ..., 256} and r <= k, T <= 65536;
 * RGC_ERR_SHAPE / _UNSUPPORTED / _ALIGN / _NULL / _WORKSPACE otherwise. */
size_t rgc_linear_backward_workspace_size(int64_t T, int64_t d, int64_t k, int64_t r);
rgc_status_t rgc_linear_backward(const uint16_t* D, int64_t ldd, const uint16_t* W, int64_t ldw,
                                 const uint16_t* XP, float* C, uint16_t* dX, int64_t lddx, int64_t T,
                                 int64_t d, int64_t k, int64_t r, void* ws, size_t ws_bytes,
                                 void* stream);

/* ---- Test hooks (same library; used by the parity tests) ----------------- */

/* out[4*i .. 4*i+3] = Philox4x32-10(counter ctr[4*i .. 4*i+3], key = seed) for
 * i < n. ctr and out: device uint32 arrays of 4*n words. */
rgc_status_t rgc_test_philox(uint64_t seed, int64_t n, const uint32_t* ctr, uint32_t* out,
                             void* stream);

/* out[i] = bf16(v[i]) rounded to nearest even for i < n: the conversion every
 * kernel uses where it rounds to bf16 without randomness (XP, Y, dX, P, the
 * high part and remainder of C in the update); NaN gives a quiet NaN with the
 * input's sign and upper payload bits ((bits >> 16) | 0x40). v: device fp32,
 * out: device bf16, n elements each; 0 <= n <= 2^31 (else RGC_ERR_SHAPE). */
rgc_status_t rgc_test_round_nearest(const float* v, uint16_t* out, int64_t n, void* stream);

/* out[i][j] = SR(v[i][j]) with the rounding bits of weight element
 * (row0 + i, col0 + j) under `seed`: the same bits rgc_apply draws, rounded
 * here one element at a time (the update sweep rounds pairs and packs them
 * with a byte permute; the parity tests pin the update's own written bits
 * against the oracle separately).
 * v: rows x cols fp32 (row stride ld); out: rows x cols bf16 (row stride ld). */
rgc_status_t rgc_test_stochastic_round(const float* v, uint16_t* out, int64_t rows, int64_t cols,
                                       int64_t ld, int64_t row0, int64_t col0, uint64_t seed,
                                       void* stream);

/* rgc_project_batch (contraction 0) and rgc_accumulate_batch (contraction 1)
 * with the number of workgroups given by the caller (workgroups > 0) instead
 * of chosen from the shapes and the device. The partition decides the fp32
 * summation order, so results may differ in their last bits from the product
 * calls'; tests use it to force ranges of whole tiles that cross item
 * boundaries. Arguments, validation and errors otherwise as the product
 * calls; workgroups <= 0 gives RGC_ERR_SHAPE (the query returns 0). */
size_t rgc_test_sketch_workspace_size(int contraction, int64_t workgroups, int64_t n, const int64_t* widths,
                                      int64_t T, int64_t r);
rgc_status_t rgc_test_project_batch_wgs(int64_t workgroups, int64_t n, const uint16_t* const* Xs,
                                        const int64_t* ldxs, const int64_t* ks, const uint16_t* const* Ps,
                                        uint16_t* const* XPs, int64_t T, int64_t r, void* ws, size_t ws_bytes,
                                        void* stream);
rgc_status_t rgc_test_accumulate_batch_wgs(int64_t workgroups, int64_t n, const uint16_t* const* Ds,
                                           const int64_t* ldds, const int64_t* ds, const uint16_t* const* XPs,
                                           float* const* Cs, int64_t T, int64_t r, void* ws, size_t ws_bytes,
                                           void* stream);
rgc_status_t rgc_test_accumulate_batch_deferred_wgs(int64_t workgroups, int64_t n, const uint16_t* const* Ds,
                                                    const int64_t* ldds, const int64_t* ds,
                                                    const uint16_t* const* XPs, float* const* Cs, int64_t T,
                                                    int64_t r, void* ws, size_t ws_bytes, int phase, void* stream);

/* rgc_project_shared with a caller-given workgroup count (as above). */
size_t rgc_test_project_shared_workspace_size(int64_t workgroups, int64_t n, int64_t T, int64_t k, int64_t r);
rgc_status_t rgc_test_project_shared_wgs(int64_t workgroups, int64_t n, const uint16_t* X, int64_t ldx, int64_t k,
                                         const uint16_t* const* Ps, uint16_t* const* XPs, int64_t T, int64_t r,
                                         void* ws, size_t ws_bytes, void* stream);

/* H = C P^T in fp32 through the apply kernel's tile code (d x k, row stride k). */
rgc_status_t rgc_test_reconstruct(const float* C, const uint16_t* P, float* H, int64_t d,
                                  int64_t k, int64_t r, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RGC_H */
