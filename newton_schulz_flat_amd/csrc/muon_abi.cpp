// extern "C" entry points of the flat-buffer Muon step (declared, with their
// contracts, in include/muon_step.h).  Each entry point validates everything
// on the host first, then fetches the cached plan and enqueues its kernels on
// the caller's stream.  Nothing is thrown across the ABI.
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include <hip/hip_runtime.h>

#include "muon_internal.h"

using muon::Status;

namespace {

thread_local char t_last_error[512] = "";

int finish(const Status& st) {
    if (st.code != MUON_OK) {
        std::strncpy(t_last_error, st.msg, sizeof(t_last_error) - 1);
        t_last_error[sizeof(t_last_error) - 1] = '\0';
    }
    return st.code;
}

int hip_fail(Status* st, hipError_t e, const char* what) {
    st->code = MUON_ERR_HIP;
    snprintf(st->msg, sizeof(st->msg), "%s: %s", what, hipGetErrorString(e));
    return st->code;
}

size_t param_bytes(int dtype, int64_t n) { return size_t(n) * (dtype == MUON_DTYPE_BF16 ? 2 : 4); }

int check_mode(int gemm_mode, Status* st) {
    if (gemm_mode != MUON_GEMM_BF16_MFMA && gemm_mode != MUON_GEMM_F32) {
        st->code = MUON_ERR_BAD_ARG;
        snprintf(st->msg, sizeof(st->msg), "gemm_mode %d is not MUON_GEMM_BF16_MFMA or _F32",
                 gemm_mode);
        return st->code;
    }
    return MUON_OK;
}

int check_ns_steps(int ns_steps, Status* st) {
    if (ns_steps < 0 || ns_steps > muon::kMaxNsSteps) {
        st->code = MUON_ERR_BAD_ARG;
        snprintf(st->msg, sizeof(st->msg), "ns_steps %d is outside [0, %d]", ns_steps,
                 muon::kMaxNsSteps);
        return st->code;
    }
    return MUON_OK;
}

int check_flag(int v, const char* name, Status* st) {
    if (v != 0 && v != 1) {
        st->code = MUON_ERR_BAD_ARG;
        snprintf(st->msg, sizeof(st->msg), "%s = %d must be 0 or 1", name, v);
        return st->code;
    }
    return MUON_OK;
}

int check_null(const void* p, const char* name, Status* st) {
    if (p == nullptr) {
        st->code = MUON_ERR_NULL_POINTER;
        snprintf(st->msg, sizeof(st->msg), "%s is NULL", name);
        return st->code;
    }
    return MUON_OK;
}

// The workspace must hold the largest single-matrix wave (need_min).  When it
// holds the whole set (need_full), everything runs in one wave (*capacity = 0);
// otherwise the set runs in waves of at most `have` bytes each.
int check_workspace(const void* ws, size_t have, size_t need_full, size_t need_min,
                    size_t* capacity, Status* st) {
    *capacity = 0;
    if (need_full == 0) return MUON_OK;
    if (ws == nullptr) return check_null(ws, "workspace", st);
    if (reinterpret_cast<uintptr_t>(ws) % muon::kWsAlign != 0) {
        st->code = MUON_ERR_MISALIGNED;
        snprintf(st->msg, sizeof(st->msg), "workspace is not %zu-byte aligned", muon::kWsAlign);
        return st->code;
    }
    if (have < need_min) {
        st->code = MUON_ERR_WORKSPACE_TOO_SMALL;
        snprintf(st->msg, sizeof(st->msg),
                 "workspace has %zu bytes; the largest matrix alone needs %zu (%zu for one wave)",
                 have, need_min, need_full);
        return st->code;
    }
    if (have < need_full) *capacity = have;
    return MUON_OK;
}

#define TRY(expr)                                  \
    do {                                           \
        if ((expr) != MUON_OK) return finish(st);  \
    } while (0)

#define TRY_HIP(expr, what)                                      \
    do {                                                         \
        hipError_t e_ = (expr);                                  \
        if (e_ != hipSuccess) return finish((hip_fail(&st, e_, what), st)); \
    } while (0)

}  // namespace

namespace muon {

// Validation of a whole step's arguments except the workspace: descriptors,
// mode, ns_steps, dtype, model copy, buffer bounds, alignment and aliasing of
// the caller's buffers (and of `extra`, when given).  h holds the scalars or
// the device group array (n_groups groups).
int check_step_args(Status& st, void* params, int param_dtype, int64_t n_param_elems,
                    void* model_copy, const float* grads, float* momentum, int64_t n_state_elems,
                    const muon_matrix_desc_t* descs, int64_t n, const Hyper& h, int32_t n_groups,
                    int ns_steps, int gemm_mode, const Range* extra) {
    if (check_desc_shapes(descs, n, &st, n_groups) != MUON_OK) return st.code;
    if (check_mode(gemm_mode, &st) != MUON_OK) return st.code;
    if (check_ns_steps(ns_steps, &st) != MUON_OK) return st.code;
    if (param_dtype != MUON_DTYPE_F32 && param_dtype != MUON_DTYPE_BF16 &&
        check_param_ranges(descs, 0, 0, param_dtype, &st) != MUON_OK)
        return st.code;
    if (model_copy != nullptr && param_dtype != MUON_DTYPE_F32) {
        st.code = MUON_ERR_BAD_ARG;
        snprintf(st.msg, sizeof(st.msg), "model_copy needs float32 params (param_dtype %d)",
                 param_dtype);
        return st.code;
    }
    if (n == 0) return MUON_OK;
    if (check_null(params, "params", &st) != MUON_OK) return st.code;
    if (check_null(grads, "grads", &st) != MUON_OK) return st.code;
    if (check_null(momentum, "momentum", &st) != MUON_OK) return st.code;
    if (check_state_ranges(descs, n, n_state_elems, "grads/momentum", &st) != MUON_OK)
        return st.code;
    if (check_param_ranges(descs, n, n_param_elems, param_dtype, &st) != MUON_OK) return st.code;
    if (model_copy != nullptr && reinterpret_cast<uintptr_t>(model_copy) % 16 != 0) {
        st.code = MUON_ERR_MISALIGNED;
        snprintf(st.msg, sizeof(st.msg), "model_copy is not 16-byte aligned");
        return st.code;
    }
    const Range ranges[6] = {
        {params, param_bytes(param_dtype, n_param_elems), "params"},
        {grads, size_t(n_state_elems) * 4, "grads"},
        {momentum, size_t(n_state_elems) * 4, "momentum"},
        {h.groups, h.groups ? size_t(n_groups) * sizeof(muon_group_t) : 0, "groups"},
        {model_copy, model_copy ? size_t(n_param_elems) * 2 : 0, "model_copy"},
        extra ? *extra : Range{nullptr, 0, "unused"}};
    return check_no_alias(ranges, 6, &st);
}

int check_step_scalars(Status& st, float lr, float weight_decay, float beta, int nesterov) {
    if (check_flag(nesterov, "nesterov", &st) != MUON_OK) return st.code;
    if (check_scalar(lr, "lr", &st) != MUON_OK) return st.code;
    if (check_scalar(weight_decay, "weight_decay", &st) != MUON_OK) return st.code;
    return check_scalar(beta, "beta", &st);
}

int report(const Status& st) { return finish(st); }

int report_hip(Status& st, hipError_t e, const char* what) { return finish((hip_fail(&st, e, what), st)); }

}  // namespace muon

namespace {

// The whole step for muon_step and muon_step_grouped: validation, then the
// launches, in waves when the workspace is smaller than the one-wave size.
int run_step(Status& st, void* params, int param_dtype, int64_t n_param_elems, void* model_copy,
             const float* grads, float* momentum, int64_t n_state_elems,
             const muon_matrix_desc_t* descs, int64_t n, const muon::Hyper& h, int32_t n_groups,
             int ns_steps, int gemm_mode, void* workspace, size_t workspace_bytes,
             hipStream_t stream) {
    const muon::Range ws_range{workspace, workspace_bytes, "workspace"};
    TRY(muon::check_step_args(st, params, param_dtype, n_param_elems, model_copy, grads,
                              momentum, n_state_elems, descs, n, h, n_groups, ns_steps, gemm_mode,
                              &ws_range));
    if (n == 0) return MUON_OK;
    size_t capacity = 0;
    TRY(check_workspace(workspace, workspace_bytes, muon::workspace_bytes_for(descs, n, gemm_mode),
                        muon::min_workspace_bytes_for(descs, n, gemm_mode), &capacity, &st));
    std::shared_ptr<const muon::StepPlan> plan;
    TRY(muon::get_plan(descs, n, gemm_mode, capacity, stream, &plan, &st));
    std::vector<muon::PlanView> views;
    for (int w = 0; w < muon::plan_waves(*plan); ++w) views.push_back(muon::wave_view(*plan, w));
    TRY_HIP(muon::enqueue_step(views.data(), int(views.size()), params, param_dtype,
                               static_cast<uint16_t*>(model_copy), grads, momentum, h, ns_steps,
                               workspace, stream),
            "step");
    return MUON_OK;
}

}  // namespace

namespace muon {

// The step's launches, wave after wave on one stream (each wave reuses the
// whole workspace: stream order keeps the waves apart).
hipError_t enqueue_step(const PlanView* views, int n_waves, void* params, int param_dtype,
                        uint16_t* copy, const float* grads, float* momentum, const Hyper& h,
                        int ns_steps, void* workspace, hipStream_t stream) {
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    for (int w = 0; w < n_waves; ++w) {
        const PlanView& p = views[w];
        float* u = reinterpret_cast<float*>(ws + p.ws.u);
        float* partial = reinterpret_cast<float*>(ws + p.ws.partial);
        float* inv = reinterpret_cast<float*>(ws + p.ws.inv);
        hipError_t e;
        if (ns_steps > 0) {
            // momentum, input and first iterate in one pass; the norm is folded into
            // iteration 0, and the last iteration applies the update itself (same
            // roundings as the apply phase)
            if ((e = launch_front_cast(p, grads, momentum, nullptr, h, ws, partial, stream)) != hipSuccess)
                return e;
            if ((e = launch_norm(p, partial, inv, true, stream)) != hipSuccess) return e;
            const FusedApply fuse{params, param_dtype, h, copy};
            if ((e = launch_newton_schulz(p, ws, nullptr, &fuse, ns_steps, stream)) != hipSuccess)
                return e;
        } else {
            // U and O (in place) in the compact region over the unused X / A / B
            if ((e = launch_front(p, grads, momentum, u, true, partial, h, stream)) != hipSuccess)
                return e;
            if ((e = launch_norm(p, partial, inv, false, stream)) != hipSuccess) return e;
            if ((e = launch_cast(p, u, inv, ws, u, true, stream)) != hipSuccess) return e;
            if ((e = launch_apply(p, params, param_dtype, u, true, h, copy, stream)) != hipSuccess)
                return e;
        }
    }
    return hipSuccess;
}

}  // namespace muon

extern "C" {

int muon_workspace_bytes(const muon_matrix_desc_t* descs, int64_t n, int gemm_mode,
                         size_t* out_bytes) {
    Status st{MUON_OK, ""};
    TRY(check_null(out_bytes, "out_bytes", &st));
    TRY(check_mode(gemm_mode, &st));
    // any group index is fine here: the workspace does not depend on groups
    TRY(muon::check_desc_shapes(descs, n, &st, INT32_MAX));
    *out_bytes = muon::workspace_bytes_for(descs, n, gemm_mode);
    return MUON_OK;
}

int muon_workspace_min_bytes(const muon_matrix_desc_t* descs, int64_t n, int gemm_mode,
                             size_t* out_bytes) {
    Status st{MUON_OK, ""};
    TRY(check_null(out_bytes, "out_bytes", &st));
    TRY(check_mode(gemm_mode, &st));
    TRY(muon::check_desc_shapes(descs, n, &st, INT32_MAX));
    *out_bytes = muon::min_workspace_bytes_for(descs, n, gemm_mode);
    return MUON_OK;
}

int muon_step(void* params, int param_dtype, int64_t n_param_elems, const float* grads,
              float* momentum, int64_t n_state_elems, const muon_matrix_desc_t* descs, int64_t n,
              float lr, float weight_decay, float beta, int nesterov, int ns_steps, int gemm_mode,
              void* workspace, size_t workspace_bytes, hipStream_t stream) {
    Status st{MUON_OK, ""};
    TRY(muon::check_step_scalars(st, lr, weight_decay, beta, nesterov));
    const muon::Hyper h{nullptr, lr, weight_decay, beta, nesterov};
    return run_step(st, params, param_dtype, n_param_elems, nullptr, grads, momentum, n_state_elems,
                    descs, n, h, 1, ns_steps, gemm_mode, workspace, workspace_bytes, stream);
}

int muon_step_grouped(void* params, int param_dtype, int64_t n_param_elems, void* model_copy,
                      const float* grads, float* momentum, int64_t n_state_elems,
                      const muon_matrix_desc_t* descs, int64_t n, const muon_group_t* groups,
                      int32_t n_groups, int ns_steps, int gemm_mode, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
    Status st{MUON_OK, ""};
    if (n_groups < 1 || n_groups > muon::kMaxGroups) {
        st.code = MUON_ERR_BAD_ARG;
        snprintf(st.msg, sizeof(st.msg), "n_groups = %d is outside [1, %d]", n_groups,
                 muon::kMaxGroups);
        return finish(st);
    }
    if (n > 0) TRY(check_null(groups, "groups", &st));
    const muon::Hyper h{groups, 0.f, 0.f, 0.f, 0};
    return run_step(st, params, param_dtype, n_param_elems, model_copy, grads, momentum,
                    n_state_elems, descs, n, h, n_groups, ns_steps, gemm_mode, workspace,
                    workspace_bytes, stream);
}

int muon_momentum(const float* grads, float* momentum, float* u_out, int64_t n_state_elems,
                  const muon_matrix_desc_t* descs, int64_t n, float beta, int nesterov,
                  hipStream_t stream) {
    Status st{MUON_OK, ""};
    TRY(muon::check_desc_shapes(descs, n, &st));
    TRY(check_flag(nesterov, "nesterov", &st));
    TRY(muon::check_scalar(beta, "beta", &st));
    if (n == 0) return MUON_OK;
    TRY(check_null(grads, "grads", &st));
    TRY(check_null(momentum, "momentum", &st));
    TRY(check_null(u_out, "u_out", &st));
    TRY(muon::check_state_ranges(descs, n, n_state_elems, "grads/momentum/u_out", &st));
    const muon::Range ranges[3] = {{grads, size_t(n_state_elems) * 4, "grads"},
                                   {momentum, size_t(n_state_elems) * 4, "momentum"},
                                   {u_out, size_t(n_state_elems) * 4, "u_out"}};
    TRY(muon::check_no_alias(ranges, 3, &st));
    std::shared_ptr<const muon::StepPlan> plan;
    TRY(muon::get_plan(descs, n, MUON_GEMM_BF16_MFMA, 0, stream, &plan, &st));
    const muon::Hyper h{nullptr, 0.f, 0.f, beta, nesterov};
    TRY_HIP(muon::launch_front(muon::wave_view(*plan, 0), grads, momentum, u_out, false, nullptr,
                               h, stream),
            "front");
    return MUON_OK;
}

int muon_orthogonalize(const float* u, float* o_out, int64_t n_elems,
                       const muon_matrix_desc_t* descs, int64_t n, int ns_steps, int gemm_mode,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
    Status st{MUON_OK, ""};
    TRY(muon::check_desc_shapes(descs, n, &st));
    TRY(check_mode(gemm_mode, &st));
    TRY(check_ns_steps(ns_steps, &st));
    if (n == 0) return MUON_OK;
    TRY(check_null(u, "u", &st));
    TRY(check_null(o_out, "o_out", &st));
    TRY(muon::check_state_ranges(descs, n, n_elems, "u/o_out", &st));
    size_t capacity = 0;
    TRY(check_workspace(workspace, workspace_bytes, muon::workspace_bytes_for(descs, n, gemm_mode),
                        muon::min_workspace_bytes_for(descs, n, gemm_mode), &capacity, &st));
    const bool in_place = static_cast<const void*>(u) == static_cast<const void*>(o_out);
    const muon::Range ranges[3] = {{u, size_t(n_elems) * 4, "u"},
                                   {o_out, in_place ? 0 : size_t(n_elems) * 4, "o_out"},
                                   {workspace, workspace_bytes, "workspace"}};
    TRY(muon::check_no_alias(ranges, 3, &st));
    std::shared_ptr<const muon::StepPlan> plan;
    TRY(muon::get_plan(descs, n, gemm_mode, capacity, stream, &plan, &st));
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    for (int w = 0; w < muon::plan_waves(*plan); ++w) {
        const muon::PlanView& p = muon::wave_view(*plan, w);
        float* partial = reinterpret_cast<float*>(ws + p.ws.partial);
        float* inv = reinterpret_cast<float*>(ws + p.ws.inv);
        if (ns_steps > 0) {
            TRY_HIP(muon::launch_front_cast(p, nullptr, nullptr, u, muon::Hyper{}, ws, partial,
                                            stream),
                    "sum of squares and cast");
            TRY_HIP(muon::launch_norm(p, partial, inv, true, stream), "norm");
            TRY_HIP(muon::launch_newton_schulz(p, ws, o_out, nullptr, ns_steps, stream),
                    "newton-schulz");
        } else {
            TRY_HIP(muon::launch_sumsq(p, u, partial, stream), "sum of squares");
            TRY_HIP(muon::launch_norm(p, partial, inv, false, stream), "norm");
            TRY_HIP(muon::launch_cast(p, u, inv, ws, o_out, false, stream), "cast");
        }
    }
    return MUON_OK;
}

int muon_apply(void* params, int param_dtype, int64_t n_param_elems, const float* updates,
               int64_t n_update_elems, const muon_matrix_desc_t* descs, int64_t n, float lr,
               float weight_decay, hipStream_t stream) {
    Status st{MUON_OK, ""};
    TRY(muon::check_desc_shapes(descs, n, &st));
    TRY(muon::check_scalar(lr, "lr", &st));
    TRY(muon::check_scalar(weight_decay, "weight_decay", &st));
    if (param_dtype != MUON_DTYPE_F32 && param_dtype != MUON_DTYPE_BF16)
        TRY(muon::check_param_ranges(descs, 0, 0, param_dtype, &st));
    if (n == 0) return MUON_OK;
    TRY(check_null(params, "params", &st));
    TRY(check_null(updates, "updates", &st));
    TRY(muon::check_state_ranges(descs, n, n_update_elems, "updates", &st));
    TRY(muon::check_param_ranges(descs, n, n_param_elems, param_dtype, &st));
    const muon::Range ranges[2] = {{params, param_bytes(param_dtype, n_param_elems), "params"},
                                   {updates, size_t(n_update_elems) * 4, "updates"}};
    TRY(muon::check_no_alias(ranges, 2, &st));
    std::shared_ptr<const muon::StepPlan> plan;
    TRY(muon::get_plan(descs, n, MUON_GEMM_BF16_MFMA, 0, stream, &plan, &st));
    const muon::Hyper h{nullptr, lr, weight_decay, 0.f, 0};
    TRY_HIP(muon::launch_apply(muon::wave_view(*plan, 0), params, param_dtype, updates, false, h,
                               nullptr, stream),
            "apply");
    return MUON_OK;
}

const char* muon_status_string(int status) {
    switch (status) {
        case MUON_OK: return "MUON_OK";
        case MUON_ERR_NULL_POINTER: return "MUON_ERR_NULL_POINTER";
        case MUON_ERR_BAD_SHAPE: return "MUON_ERR_BAD_SHAPE";
        case MUON_ERR_OUT_OF_BOUNDS: return "MUON_ERR_OUT_OF_BOUNDS";
        case MUON_ERR_MISALIGNED: return "MUON_ERR_MISALIGNED";
        case MUON_ERR_OVERLAP: return "MUON_ERR_OVERLAP";
        case MUON_ERR_ALIAS: return "MUON_ERR_ALIAS";
        case MUON_ERR_BAD_ARG: return "MUON_ERR_BAD_ARG";
        case MUON_ERR_WORKSPACE_TOO_SMALL: return "MUON_ERR_WORKSPACE_TOO_SMALL";
        case MUON_ERR_HIP: return "MUON_ERR_HIP";
        case MUON_ERR_INTERNAL: return "MUON_ERR_INTERNAL";
        default: return "MUON_ERR_UNKNOWN";
    }
}

const char* muon_last_error(void) { return t_last_error; }

}  // extern "C"
