/*
 * muon_step.h -- C ABI of the MI355X (gfx950) Muon optimizer step over flat buffers.
 *
 * What is computed (page "Add initial Muon+M-FSDPv2 implementation",
 * Megatron-LM PR #6425, pseudocode block "Opt step", steps 1, 2, 4 and 6; and
 * class FsdpMuon on the page
 * "core.distributed.fsdp.src.megatron_fsdp.experimental.muon", methods
 * _compute_momentum_inputs, _orthogonalize_updates, _apply_local_updates):
 * for every 2-D matrix described by a muon_matrix_desc_t, with
 * G = gradient, M = momentum, W = weights, all rows x cols row-major,
 *
 *   M  <- beta*M + G                              (state update, step 1)
 *   U  <- G + beta*M   (Nesterov)   or   U <- M   (orthogonalization input, step 2)
 *   O  <- s * NS(U),  s = sqrt(max(1, rows/cols)) (orthogonalization, step 4)
 *   W  <- W*(1 - lr*wd) - lr*O                    (decoupled decay + update, step 6)
 *
 * NS is the quintic Newton-Schulz orthogonalization: X = U (or U^T when
 * rows > cols), X <- X / (||X||_F + 1e-7), then ns_steps times
 * A = X X^T, B = b A + c A A, X <- a X + B X with (a, b, c) =
 * (3.4445, -4.7750, 2.0315); the result is transposed back for tall matrices.
 * The pages name the orthogonalization without fixing its algorithm; the
 * quintic iteration is the one Muon is built on.
 *
 * Numerics.  The elementwise phases run in float32, one rounding per
 * operation, no fused multiply-add, in this order:
 *   M1 = fl(fl(beta*M) + G);  U = fl(fl(beta*M1) + G)  (U = M1 without Nesterov)
 *   f  = fl(1 - fl(lr*wd));   W1 = fl(W*f);  Wn = fl(W1 - fl(lr*O))
 * and bfloat16 weights are rounded once, to nearest even, on store.
 * The Frobenius norm is a deterministic float32 reduction.  Newton-Schulz
 * runs either on bfloat16 MFMA with float32 accumulation and float32
 * epilogues, X/A/B stored as bfloat16 (MUON_GEMM_BF16_MFMA), or entirely in
 * float32 on the float32 MFMA (MUON_GEMM_F32).  Matrices whose shorter side
 * is below 160 run in float32 in both modes (with bfloat16 iterates a matrix
 * with few singular values deviates from the exact iteration by up to ~12%);
 * in float32 no accumulation chain is longer than 32768 products.  The
 * first iterate is stored
 * as U itself (rounded to the Newton-Schulz type) and the normalization is
 * applied in float32 inside the first iteration: A0 = inv^2 (U U^T),
 * X1 = inv (a U + B0 U), inv = 1 / (||U||_F + 1e-7) -- the same iterates as
 * X0 = U / (||U||_F + 1e-7), with one rounding fewer.  Rank-deficient inputs:
 * the exact O lies in U's column and row spaces, and that part is computed to
 * the mode's accuracy; in U's null space each iteration multiplies rounding
 * noise by a = 3.4445, so O also carries a component there, about a^5 times
 * the products' rounding error: below 3e-4 of ||O|| in float32, but of the
 * order of ||O|| itself with bfloat16 iterates (use MUON_GEMM_F32 for inputs
 * of very low rank).  The bfloat16 mode's deviation also grows with
 * ns_steps, since rounding accumulates while the quintic keeps the singular
 * values oscillating in its band: on Gaussian inputs about 2e-3 relative at 2
 * iterations, 1e-2 at 5, 2.4e-2 at 10 and 5e-2 at 64 (float32: below 3e-5 at
 * 64).  With ns_steps == 0,
 * O = fl(s * X0) with X0 rounded to the Newton-Schulz type.  O = fl(s * x)
 * in float32.  Results are deterministic and do not depend on the order of
 * descriptors; muon_step equals muon_apply(muon_orthogonalize(muon_momentum))
 * bit for bit.
 *
 * Buffers.  All buffer pointers are device pointers allocated by the caller,
 * who keeps ownership.  Descriptor arrays are host memory read during the
 * call.  The workspace is caller-owned device memory, 256-byte aligned; its
 * contents are undefined after a call.  Calls that share a workspace must be
 * ordered on one stream.  With muon_workspace_bytes() bytes every matrix is
 * orthogonalized in one wave; a smaller workspace of at least
 * muon_workspace_min_bytes() bytes runs the matrices in waves, each wave's
 * intermediates fitting the workspace (the pages' optimizer likewise works
 * through its buffers one at a time on the caller's stream, FsdpMuon class
 * docstring).  Results do not depend on the wave split, bit for bit.
 *
 * Execution.  All work is enqueued on `stream` (0 = the null stream) and the
 * call returns without waiting for it.  The first call with a new descriptor
 * set (per device, GEMM mode and -- when it runs in waves -- workspace size)
 * builds a launch plan and uploads its tables: one device allocation and a
 * stream synchronization, so make that call outside graph capture and while
 * no stream of the process is being captured in global mode.  Later calls
 * with the same set allocate nothing and do not synchronize the host.  Plans
 * stay in a 64-entry least-recently-used cache; a plan used while its stream
 * is being captured into a HIP graph is pinned (never evicted, kept until the
 * process ends), since the graph keeps pointers to its tables.  An evicted
 * plan's tables are freed after a device synchronization.
 *
 * Errors.  The pages' optimizer validates its parameter-to-group mapping up
 * front and raises rather than run on a bad mapping (FsdpMuon._validate_parameter_groups
 * on the page "core.distributed.fsdp.src.megatron_fsdp.experimental.muon";
 * the review answer on the page "feat(fsdp): expose HSDP and HFSDP through
 * the MFSDP v2 adapter": an inconsistent layout is an error, never a quiet
 * wrong mapping).  Here every entry point returns MUON_OK (0) or a
 * negative muon_status_t instead of raising: nothing is thrown across the
 * ABI.  Every check except MUON_ERR_HIP runs before anything is enqueued, so
 * a failed call leaves every buffer untouched.  muon_last_error() returns a
 * thread-local message describing the last failure of this thread.  Values
 * that are NaN or infinite inside the buffers are not checked: they propagate.
 */
#ifndef MUON_STEP_H
#define MUON_STEP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One 2-D parameter inside the flat buffers (page "core.distributed.fsdp.src.
 * megatron_fsdp.experimental.muon": FsdpMuon handles 2-D parameters only,
 * held in flat FSDP buffers; the owner scatters slices of each full update to
 * their shard destinations, "Opt step" step 5 of PR #6425).
 *
 *   offset        element offset of the row-major rows x cols matrix in the
 *                 flat grads / momentum (and update) buffers; multiple of 4.
 *   rows, cols    matrix shape, each >= 1 and <= 2^20, rows*cols <= 2^34;
 *                 a set's matrices hold at most 2^36 elements in total
 *                 (MUON_ERR_BAD_SHAPE otherwise).
 *   param_offset  element offset of slice 0 in the flat params buffer.
 *   shard_stride  distance in elements between consecutive slices in params
 *                 (>= rows*cols/n_shards; ignored when n_shards == 1).
 *   n_shards      the flattened matrix is cut into n_shards contiguous slices
 *                 of rows*cols/n_shards elements; slice k of the update goes
 *                 to params[param_offset + k*shard_stride ...].  For
 *                 n_shards > 1 the slice length must be a multiple of 8.
 *   group         optimizer group of the matrix for muon_step_grouped
 *                 (0 <= group < n_groups); must be 0 for every other entry
 *                 point (muon_workspace_bytes accepts any group >= 0).
 * Every slice start must be 16-byte aligned within params.  Matrices must not
 * overlap each other in grads/momentum, nor slices each other in params. */
typedef struct muon_matrix_desc {
    int64_t offset;
    int64_t rows;
    int64_t cols;
    int64_t param_offset;
    int64_t shard_stride;
    int32_t n_shards;
    int32_t group;
} muon_matrix_desc_t;

typedef enum muon_status {
    MUON_OK = 0,
    MUON_ERR_NULL_POINTER = -1,        /* a required pointer is NULL */
    MUON_ERR_BAD_SHAPE = -2,           /* rows/cols < 1, numel % n_shards, slice length */
    MUON_ERR_OUT_OF_BOUNDS = -3,       /* a matrix or slice leaves its buffer */
    MUON_ERR_MISALIGNED = -4,          /* a matrix, slice or workspace start misaligned */
    MUON_ERR_OVERLAP = -5,             /* two descriptors' ranges intersect */
    MUON_ERR_ALIAS = -6,               /* two distinct buffers' address ranges intersect */
    MUON_ERR_BAD_ARG = -7,             /* bad n, dtype, mode, ns_steps, group or non-finite scalar */
    MUON_ERR_WORKSPACE_TOO_SMALL = -8, /* workspace smaller than muon_workspace_bytes() */
    MUON_ERR_HIP = -9,                 /* a HIP runtime call failed (message has details) */
    MUON_ERR_INTERNAL = -10            /* should not happen; message has details */
} muon_status_t;

/* Element type of the params buffer.  grads, momentum and updates are float32. */
enum { MUON_DTYPE_F32 = 0, MUON_DTYPE_BF16 = 1 };

/* Arithmetic of the Newton-Schulz chain. */
enum { MUON_GEMM_BF16_MFMA = 0, MUON_GEMM_F32 = 1 };

/* Bytes of device workspace with which muon_step / muon_orthogonalize run
 * these descriptors in one wave, for this GEMM mode (the plan-building
 * analogue of FsdpMuon's owner assignment, which is worked out once when the
 * optimizer is set up).  Host-only: makes no HIP call.  Validates the descriptors' shapes
 * (not their bounds).  out_bytes: host pointer receiving the size. */
int muon_workspace_bytes(const muon_matrix_desc_t* descs, int64_t n, int gemm_mode,
                         size_t* out_bytes);

/* Smallest workspace with which the descriptors run at all: the largest
 * single matrix's intermediates.  Between this and muon_workspace_bytes() the
 * matrices run in waves whose intermediates fit the workspace given (the
 * FsdpMuon class docstring: the step works through the buffers in turn on the
 * caller's stream).  Host-only, same validation as muon_workspace_bytes. */
int muon_workspace_min_bytes(const muon_matrix_desc_t* descs, int64_t n, int gemm_mode,
                             size_t* out_bytes);

/* The whole step ("Opt step" steps 1, 2, 4, 6 of PR #6425; FsdpMuon.step).
 *   params        device, n_param_elems elements of param_dtype; updated in place.
 *   grads         device, float32, n_state_elems elements; read only.
 *   momentum      device, float32, n_state_elems elements; updated in place.
 *   descs, n      host array of n descriptors (n == 0 is a no-op).
 *   lr, weight_decay, beta  finite float32 scalars.
 *   nesterov      0 or 1.   ns_steps  0..64.   gemm_mode  MUON_GEMM_*.
 *   workspace     device, 256-byte aligned, >= muon_workspace_min_bytes()
 *                 (>= muon_workspace_bytes() for one wave).
 * The four buffers must not alias one another. */
int muon_step(void* params, int param_dtype, int64_t n_param_elems, const float* grads,
              float* momentum, int64_t n_state_elems, const muon_matrix_desc_t* descs,
              int64_t n, float lr, float weight_decay, float beta, int nesterov, int ns_steps,
              int gemm_mode, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Momentum update and orthogonalization input alone ("Opt step" steps 1-2;
 * FsdpMuon._compute_momentum_inputs).  Writes U (float32) to u_out at each
 * descriptor's offset; momentum updated in place.  grads, momentum, u_out are
 * device buffers of n_state_elems float32 that must not alias.  Weight decay
 * is applied by muon_apply (decoupled), not here. */
int muon_momentum(const float* grads, float* momentum, float* u_out, int64_t n_state_elems,
                  const muon_matrix_desc_t* descs, int64_t n, float beta, int nesterov,
                  hipStream_t stream);

/* Orthogonalization alone ("Opt step" step 4; FsdpMuon._orthogonalize_updates):
 * o_out = s * NS(u) for every descriptor, both device float32 buffers of
 * n_elems elements laid out like grads.  o_out may equal u (in place) but must
 * not partially overlap it.  Workspace as for muon_step. */
int muon_orthogonalize(const float* u, float* o_out, int64_t n_elems,
                       const muon_matrix_desc_t* descs, int64_t n, int ns_steps, int gemm_mode,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* One optimizer group of muon_step_grouped: the pages' optimizer keeps its
 * settings per parameter group and maps every parameter to its group (page
 * "core.distributed.fsdp.src.megatron_fsdp.experimental.muon", FsdpMuon._step_group,
 * argument tensor_to_optimizer_group_index).  An array of groups lives in DEVICE
 * memory and is read by the kernels when they run, so a captured graph
 * replays with whatever values the array holds at replay time (optimizer
 * CUDA-graph support is among the features the Megatron-Bridge #5933 commit
 * message lists, quoted on the page "feat(fsdp): expose HSDP and HFSDP
 * through the MFSDP v2 adapter", PR #6873).  Values are not checked: NaN and
 * infinities propagate; nesterov is true when non-zero. */
typedef struct muon_group {
    float lr;
    float weight_decay;
    float beta;
    int32_t nesterov;
} muon_group_t;

/* The whole step with per-matrix optimizer groups and an optional bfloat16
 * model copy.  Matrix i uses groups[descs[i].group]; its results equal, bit for
 * bit, those of muon_step called with that group's scalars.
 *   groups, n_groups  DEVICE array of n_groups (1..65536) muon_group_t, read
 *                     during the kernels; must not overlap the other buffers.
 *   model_copy        NULL, or -- with param_dtype MUON_DTYPE_F32 only -- a
 *                     device bfloat16 buffer of n_param_elems elements, 16-byte
 *                     aligned and laid out like params: every updated weight
 *                     is also stored there, rounded to nearest even (float32
 *                     master weights with a refreshed bfloat16 model copy: the
 *                     pages' optimizer updates the model weights from the
 *                     optimizer's own copy, FsdpMuon class docstring and
 *                     FsdpMuon.step; the precision-aware optimizer listed in the
 *                     Megatron-Bridge #5933 commit message on the PR #6873 page).
 * Every other argument as muon_step.  Once the plan for a descriptor set
 * exists (built by the first call with that set, which synchronizes the
 * stream: make it outside graph capture), a call makes no allocation, memset
 * or host synchronization and may be captured into a HIP graph. */
int muon_step_grouped(void* params, int param_dtype, int64_t n_param_elems, void* model_copy,
                      const float* grads, float* momentum, int64_t n_state_elems,
                      const muon_matrix_desc_t* descs, int64_t n, const muon_group_t* groups,
                      int32_t n_groups, int ns_steps, int gemm_mode, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/* Decay and update alone ("Opt step" step 6; FsdpMuon._apply_local_updates):
 * params slice k <- fl(fl(W*f) - fl(lr*O)), f = fl(1 - fl(lr*weight_decay)),
 * with O read from `updates` (device float32, n_update_elems, laid out like
 * grads) and slices scattered as the descriptors say.  params and updates
 * must not alias. */
int muon_apply(void* params, int param_dtype, int64_t n_param_elems, const float* updates,
               int64_t n_update_elems, const muon_matrix_desc_t* descs, int64_t n, float lr,
               float weight_decay, hipStream_t stream);

/* muon_step for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments and results (bit for bit) as muon_step, without the workspace:
 * every intermediate lives in a fixed device array of 320 MiB that the library
 * holds on each GPU it runs on, from its load until the process ends (8 MiB of
 * launch tables, 312 MiB of workspace; matrices that do not fit at once run in
 * waves).  The call makes no hipMalloc, hipFree or other allocation.  A matrix
 * whose intermediates alone exceed 312 MiB (for example 4096 x 16384 with
 * bfloat16 products), or a set whose launch tables exceed 8 MiB, is rejected
 * with MUON_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.  The first
 * call with a new descriptor set on a device copies its launch tables into the
 * array and synchronizes `stream`; later calls with the same set copy nothing
 * and do not synchronize.  Under graph capture only a call with the set whose
 * tables are resident (the device's last one) can run: any other is rejected
 * with MUON_ERR_BAD_ARG before anything is enqueued, leaving the resident
 * tables in place.  All calls on one GPU share its array, which keeps
 * the last call's contents: calls that overlap on one GPU (different streams,
 * or threads without ordering) race and must not be made. */
int muon_step_noalloc(void* params, int param_dtype, int64_t n_param_elems, const float* grads,
                      float* momentum, int64_t n_state_elems, const muon_matrix_desc_t* descs,
                      int64_t n, float lr, float weight_decay, float beta, int nesterov,
                      int ns_steps, int gemm_mode, hipStream_t stream);

/* Kernel timing, a profiling aid (not part of the step's semantics).
 * Between muon_profile_begin() and muon_profile_end(), every kernel the
 * library launches, from any thread, is bracketed by two HIP events recorded
 * on the launch's own stream.  muon_profile_end() stops recording, waits for
 * the recorded events, and aggregates elapsed time by kernel name into `out`
 * (at most max_entries rows, host memory; *n_entries receives the number of
 * distinct kernels, which may exceed max_entries).  Names are
 * "front", "sumsq", "norm", "cast", "apply" and "ns_<stage>_t<tile>_<type>"
 * for the Newton-Schulz products (stage a: X X^T, b: b A + c A A, x: a X + B X;
 * tile 64/128/256; type bf16/f32).  Events come from a pool the library owns;
 * when timing is off the only cost is one flag test per launch. */
typedef struct muon_kernel_time {
    char name[48];
    double total_ms;   /* sum of the launches' event-to-event times */
    int64_t launches;
} muon_kernel_time_t;

int muon_profile_begin(void);
int muon_profile_end(muon_kernel_time_t* out, int max_entries, int* n_entries);

/* Static name of a status code ("MUON_OK", "MUON_ERR_BAD_SHAPE", ...): the
 * kind of a rejected call, which the pages' optimizer reports by raising from
 * its up-front validation (FsdpMuon._validate_parameter_groups, page
 * "core.distributed.fsdp.src.megatron_fsdp.experimental.muon"; errors rather
 * than wrong mappings, review answers on the page "feat(fsdp): expose HSDP and
 * HFSDP through the MFSDP v2 adapter").  Any int is accepted; unknown codes
 * give "MUON_ERR_UNKNOWN".  The string is static: never free it. */
const char* muon_status_string(int status);

/* Message of the calling thread's last failure ("" if none): the text the
 * pages' validation would raise with (same passages as muon_status_string),
 * naming the offending descriptor, buffer or argument.  Thread-local, owned
 * by the library, valid until the thread's next failing call into this
 * library; never free it.  Successful calls leave it unchanged. */
const char* muon_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MUON_STEP_H */
