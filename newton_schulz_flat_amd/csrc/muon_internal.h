// Internal declarations shared by the host runtime (validation, plan, ABI)
// and the gfx950 kernels of the flat-buffer Muon step.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <memory>

#include <hip/hip_runtime_api.h>

#include "muon_step.h"

namespace muon {

// ---------------------------------------------------------------- geometry

// Elements handled by one workgroup of the elementwise kernels: 512, as
// 128 threads x one float4 for the momentum kernel (two 16-byte loads per
// thread) and 64 threads x two float4 for the apply kernel (whose bfloat16
// weight loads are 8 bytes).  Of the shapes measured on gfx950 (512 to 8192
// elements, 64 to 256 threads) these two stream fastest.  One float partial
// sum of squares is produced per chunk.
constexpr int kEwVec = 4;
constexpr int kFrontThreads = 128, kFrontIters = 1;
constexpr int kApplyThreads = 64, kApplyIters = 2;
constexpr int64_t kEwChunk = int64_t(kFrontThreads) * kEwVec * kFrontIters;
static_assert(kEwChunk == int64_t(kApplyThreads) * kEwVec * kApplyIters, "one chunk size");

// Square tile of the normalize/cast/orient kernel.
constexpr int kCastTile = 64;

// GEMM tile of the matrices whose shorter side is below 160.  Their
// Newton-Schulz products run in float32 in every mode: with bfloat16 iterates
// a matrix with few singular values keeps none of the averaging that holds
// large matrices to ~1e-2, and deviates from the exact iteration by up to ~12%.
constexpr int kF32NsTile = 64;

// Alignment of every workspace region, in bytes.
constexpr size_t kWsAlign = 256;

// Largest accepted matrix side and element count, and element count of a
// whole descriptor set (2^36 float32 elements are 256 GiB per buffer; the
// bound keeps every chunk and tile count of a set within int32).
constexpr int64_t kMaxSide = int64_t(1) << 20;
constexpr int64_t kMaxNumel = int64_t(1) << 34;
constexpr int64_t kMaxSetNumel = int64_t(1) << 36;
constexpr int kMaxNsSteps = 64;
constexpr int kMaxGroups = 65536;  // optimizer groups per muon_step_grouped call

// Quintic Newton-Schulz coefficients and the norm epsilon.
constexpr float kNsA = 3.4445f;
constexpr float kNsB = -4.7750f;
constexpr float kNsC = 2.0315f;
constexpr float kNormEps = 1e-7f;

// Per-matrix facts the kernels read (device copy lives in the plan tables).
// All offsets are in elements.  "NS orientation": r = min(R, C) rows and
// c = max(R, C) columns, padded with zeros to rp x cp (multiples of the GEMM
// tile); tall matrices (R > C) are transposed into it.
struct alignas(16) MatInfo {
    int64_t off;        // start of the R x C matrix in the grads/momentum/U/O layout
    int64_t numel;      // R * C
    int64_t poff;       // start of slice 0 in params
    int64_t pstride;    // slice stride in params
    int64_t slice_len;  // numel / n_shards
    int64_t x_off;      // start of X (rp x cp) in each of the two X regions
    int64_t g_off;      // start of the rp x rp Gram block in the A and B regions
    int64_t u_off;      // start of the matrix's U / O in the workspace's compact float32 U region
    int32_t R, C;       // original shape
    int32_t r, c;       // NS-orientation shape
    int32_t rp, cp;     // padded NS-orientation shape
    int32_t tall;       // R > C
    int32_t tile;       // GEMM tile size used for this matrix (64, 128 or 256)
    int32_t chunk_begin, n_chunks;  // elementwise chunks / partial-sum slots
    int32_t cast_begin, n_cast;     // normalize/cast tiles
    float scale;        // (float) sqrt(max(1, R/C))
    int32_t group;      // optimizer group (muon_step_grouped), else 0
    int32_t ns_f32;     // products, X, A and B in float32 (x_off, g_off count floats)
};
static_assert(sizeof(MatInfo) == 128, "MatInfo layout");

// One GEMM tile: matrix index and tile coordinates.
struct alignas(16) GemmTile {
    int32_t mat, ti, tj, pad_;
};

// Byte offsets of the workspace regions.  The compact U / O region is used only
// by muon_step with ns_steps == 0, which uses no X, A or B: it overlays them.
struct WsLayout {
    size_t u;        // float32 U / O, matrix i at MatInfo::u_off (compact, 256-byte aligned)
    size_t x[2];     // X ping-pong (iteration input / output), rp x cp per matrix
    size_t a, b;     // Gram matrices rp x rp per matrix
    size_t partial;  // one float per elementwise chunk
    size_t inv;      // one float per matrix
    size_t total;
};

// Tiles of one GEMM tile size: the upper triangle (ti <= tj) of rp x rp for
// stages A and B (the same tiles, balanced for each stage's contraction
// length), and the full rp x cp grid for stage X.  Device pointers.
struct TileClassDev {
    int tile;
    int n_sym_a, n_sym_b, n_full;
    const GemmTile* sym_a;
    const GemmTile* sym_b;
    const GemmTile* full;
};

// A launch plan for one descriptor set, device and GEMM mode.
struct PlanView {
    int n;                      // matrices
    int gemm_mode;
    int64_t state_extent;       // max over descriptors of offset + numel
    int64_t total_chunks;       // elementwise workgroups
    int64_t total_cast;         // cast workgroups
    WsLayout ws;
    const MatInfo* mats_host;   // n entries
    const MatInfo* mats;        // device, n entries
    const int32_t* chunk_prefix;  // device, n + 1 entries
    const int32_t* cast_prefix;   // device, n + 1 entries
    int n_classes;
    TileClassDev classes[3];
};

// --------------------------------------------------------------- validation

struct Status {
    int code;
    char msg[512];
};

// Shapes, shard geometry and group fields (0 <= group < n_groups) of every descriptor.
int check_desc_shapes(const muon_matrix_desc_t* d, int64_t n, Status* st,
                      int64_t n_groups = 1);
// Matrices inside [0, n_elems) of the float32 state layout, 16-byte aligned,
// pairwise disjoint.
int check_state_ranges(const muon_matrix_desc_t* d, int64_t n, int64_t n_elems, const char* what,
                       Status* st);
// Slices inside [0, n_param_elems) of params, 16-byte aligned, pairwise disjoint.
int check_param_ranges(const muon_matrix_desc_t* d, int64_t n, int64_t n_param_elems,
                       int param_dtype, Status* st);
// Address ranges [ptr, ptr + bytes) of distinct buffers do not intersect.
struct Range {
    const void* ptr;
    size_t bytes;
    const char* name;
};
int check_no_alias(const Range* r, int count, Status* st);
int check_scalar(float v, const char* name, Status* st);

// Everything about a whole step's arguments except the workspace (shapes, mode,
// ns_steps, dtype, model copy, bounds, alignment, aliasing -- also against
// `extra` when non-null); h.groups and n_groups describe muon_step_grouped's
// table.  The scalars of muon_step: nesterov in {0, 1}, finite lr, wd, beta.
struct Hyper;
int check_step_args(Status& st, void* params, int param_dtype, int64_t n_param_elems,
                    void* model_copy, const float* grads, float* momentum, int64_t n_state_elems,
                    const muon_matrix_desc_t* descs, int64_t n, const Hyper& h, int32_t n_groups,
                    int ns_steps, int gemm_mode, const Range* extra);
int check_step_scalars(Status& st, float lr, float weight_decay, float beta, int nesterov);
// Records a failure as the calling thread's last error (muon_last_error);
// returns its code.  report_hip fills st from a HIP error first.
int report(const Status& st);
int report_hip(Status& st, hipError_t e, const char* what);

// --------------------------------------------------------------------- plan

// Workspace bytes for a descriptor set run in one wave (host only; shapes
// must be valid).
size_t workspace_bytes_for(const muon_matrix_desc_t* d, int64_t n, int gemm_mode);
// Smallest workspace that runs the set at all: the largest one-matrix wave.
size_t min_workspace_bytes_for(const muon_matrix_desc_t* d, int64_t n, int gemm_mode);

// A launch plan: the descriptor set cut into waves whose workspace regions fit
// a capacity (one wave when unbounded), each wave with its own tables.
struct StepPlan;
int plan_waves(const StepPlan& p);
const PlanView& wave_view(const StepPlan& p, int wave);

// Cached plan for (device, gemm_mode, capacity, descriptors); builds and
// uploads it on first use (outside graph capture).  capacity: workspace bytes
// available, 0 = one wave.  A plan fetched while `stream` is being captured
// is pinned (kept until the process ends).  The shared pointer keeps the plan
// alive for the caller.
int get_plan(const muon_matrix_desc_t* d, int64_t n, int gemm_mode, size_t capacity,
             hipStream_t stream, std::shared_ptr<const StepPlan>* out, Status* st);

// A plan built on the host only (no device memory): its tables as one blob
// (blob_bytes), to be copied to a device address and bound there.  For callers
// that cannot allocate; not cached.
struct HostPlan;
int build_host_plan(const muon_matrix_desc_t* d, int64_t n, int gemm_mode, size_t capacity,
                    std::shared_ptr<HostPlan>* out, Status* st);
size_t host_plan_blob_bytes(const HostPlan& p);
const void* host_plan_blob(const HostPlan& p);
size_t host_plan_workspace_bytes(const HostPlan& p);  // largest wave's workspace
// Views of every wave with their tables at dev_blob (a device copy of the blob).
int host_plan_waves(const HostPlan& p);
PlanView host_plan_view(const HostPlan& p, int wave, const void* dev_blob);

// ---------------------------------------------------------------- profiling

// Brackets one kernel launch with HIP events on its stream while kernel
// timing is on (muon_profile_begin / muon_profile_end); a no-op otherwise.
class LaunchTimer {
  public:
    LaunchTimer(const char* name, hipStream_t s);
    ~LaunchTimer();
    LaunchTimer(const LaunchTimer&) = delete;
    LaunchTimer& operator=(const LaunchTimer&) = delete;

  private:
    const char* name_;
    hipStream_t stream_;
    void* start_ = nullptr;  // hipEvent_t when active
};

// ------------------------------------------------------------------ kernels

// Optimizer hyperparameters of a launch: one set for every matrix
// (groups == nullptr), or per matrix groups[MatInfo::group], read from device
// memory by the kernels.
struct Hyper {
    const muon_group_t* groups;
    float lr, weight_decay, beta;
    int nesterov;
};


// Momentum + orthogonalization input (+ per-chunk sum of squares of U).  U is
// written at each matrix's offset in the grads layout, or (compact) at its
// u_off in the workspace's U region.
hipError_t launch_front(const PlanView& p, const float* grads, float* momentum, float* u,
                        bool compact, float* partial, const Hyper& h, hipStream_t s);
// Per-chunk sum of squares of an existing U (grads layout).
hipError_t launch_sumsq(const PlanView& p, const float* u, float* partial, hipStream_t s);
// Per-matrix 1 / (sqrt(sum of partials) + eps); partials per elementwise chunk,
// or per 64 x 64 cast tile (per_tile).
hipError_t launch_norm(const PlanView& p, const float* partial, float* inv, bool per_tile,
                       hipStream_t s);
// One pass over the first iterate, one workgroup per 4096 of its elements:
// with u == nullptr, momentum and input from grads and momentum (momentum
// updated); else U is read.  Writes U, rounded to the matrix's product type but
// not normalized, as the first iterate in NS orientation (zero padding) and
// one sum of squares of U per workgroup.  The Newton-Schulz iteration 0 then
// applies 1 / ||U|| (launch_newton_schulz with the norm folded).
hipError_t launch_front_cast(const PlanView& p, const float* grads, float* momentum,
                             const float* u, const Hyper& h, void* ws, float* partial,
                             hipStream_t s);
// X0 = cast(U * inv) in NS orientation into the first X region, zero
// padding; when o_direct is non-null (ns_steps == 0) write O = s * X0 there
// instead.  U and O in the grads layout, or both compact (u_off).
hipError_t launch_cast(const PlanView& p, const float* u, const float* inv, void* ws,
                       float* o_direct, bool compact, hipStream_t s);
// The decay-and-update of the apply phase, for the last Newton-Schulz
// iteration to perform in place of storing O.  model_copy (float32 params
// only, may be null) receives every updated weight rounded to bfloat16.
struct FusedApply {
    void* params;
    int param_dtype;
    Hyper hyper;
    uint16_t* model_copy;
};
// ns_steps >= 1 Newton-Schulz iterations on the first iterate that
// launch_front_cast stored (U unnormalized; iteration 0 scales its products by
// the per-matrix 1 / ||U||: A0 = inv^2 (U U^T), X1 = inv (a U + B0 U)); the last
// writes O = s * X in the original orientation to o, or, with fuse, applies
// W <- fl(fl(W f) - fl(lr O)) to the parameter slices directly (O is then not
// stored).
hipError_t launch_newton_schulz(const PlanView& p, void* ws, float* o, const FusedApply* fuse,
                                int ns_steps, hipStream_t s);
// The whole step (ns_steps >= 1: front_cast, norm, Newton-Schulz with the
// fused apply; ns_steps == 0: front, norm, cast and apply through the compact U
// region), wave after wave on one stream, every wave reusing the workspace.
hipError_t enqueue_step(const PlanView* views, int n_waves, void* params, int param_dtype,
                        uint16_t* copy, const float* grads, float* momentum, const Hyper& h,
                        int ns_steps, void* workspace, hipStream_t stream);
// W <- fl(fl(W*f) - fl(lr*O)) scattered into the slices (and, with
// model_copy, its bfloat16 rounding into the copy).  O in the grads layout, or
// compact (u_off).
hipError_t launch_apply(const PlanView& p, void* params, int param_dtype, const float* o,
                        bool compact, const Hyper& h, uint16_t* model_copy, hipStream_t s);

}  // namespace muon
