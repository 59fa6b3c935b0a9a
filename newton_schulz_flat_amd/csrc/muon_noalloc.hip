// muon_step_noalloc: the whole Muon step with no device allocation, for
// callers that cannot allocate (code under graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// Every intermediate lives in one file-scope device array, `scratch`, that
// each GPU holds from the library's load until the process ends.  Its head
// (kTableBytes) holds the launch tables of the descriptor set last used on the
// device; the rest is the step's workspace, which the matrices fill in waves
// when they do not fit at once.  Host code never names the array: the device
// address of each GPU's copy comes from hipGetSymbolAddress (once per device,
// with that device current) and is what the copies and the kernels get.
//
// Nothing in the scratch needs clearing: every byte a kernel reads was written
// earlier in the same call (the first iterate with its zero padding, the Gram
// matrices, the partial sums, the norms).  All calls on one GPU share its
// scratch, so calls that overlap on one GPU race.
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "muon_internal.h"

namespace muon {

namespace {

constexpr size_t kScratchBytes = size_t(320) << 20;  // per GPU
constexpr size_t kTableBytes = size_t(8) << 20;      // launch tables at the head

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceState {
    unsigned char* ptr = nullptr;  // this device's copy of `scratch`
    std::string key;               // descriptor set whose tables are resident
    std::shared_ptr<HostPlan> plan;
};

std::mutex g_mu;
DeviceState g_dev[kMaxDevices];

}  // namespace

}  // namespace muon

extern "C" int muon_step_noalloc(void* params, int param_dtype, int64_t n_param_elems,
                                 const float* grads, float* momentum, int64_t n_state_elems,
                                 const muon_matrix_desc_t* descs, int64_t n, float lr,
                                 float weight_decay, float beta, int nesterov, int ns_steps,
                                 int gemm_mode, hipStream_t stream) {
    using namespace muon;
    Status st{MUON_OK, ""};
    if (check_step_scalars(st, lr, weight_decay, beta, nesterov) != MUON_OK) return report(st);
    const Hyper h{nullptr, lr, weight_decay, beta, nesterov};
    if (check_step_args(st, params, param_dtype, n_param_elems, nullptr, grads, momentum,
                        n_state_elems, descs, n, h, 1, ns_steps, gemm_mode, nullptr) != MUON_OK)
        return report(st);
    if (n == 0) return MUON_OK;

    const size_t ws_cap = kScratchBytes - kTableBytes;
    const size_t need_min = min_workspace_bytes_for(descs, n, gemm_mode);
    if (need_min > ws_cap) {
        st.code = MUON_ERR_WORKSPACE_TOO_SMALL;
        snprintf(st.msg, sizeof(st.msg),
                 "the largest matrix needs %zu bytes of intermediates; muon_step_noalloc has "
                 "%zu (use muon_step with a workspace)",
                 need_min, ws_cap);
        return report(st);
    }
    const size_t capacity = workspace_bytes_for(descs, n, gemm_mode) <= ws_cap ? 0 : ws_cap;

    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return report_hip(st, e, "hipGetDevice");
    if (device < 0 || device >= kMaxDevices) {
        st.code = MUON_ERR_INTERNAL;
        snprintf(st.msg, sizeof(st.msg), "device %d beyond the %d supported", device, kMaxDevices);
        return report(st);
    }

    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState& ds = g_dev[device];
    if (ds.ptr == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return report_hip(st, e, "hipGetSymbolAddress of the scratch array");
        ds.ptr = static_cast<unsigned char*>(p);
    }
    std::string key(sizeof(int) + size_t(n) * sizeof(muon_matrix_desc_t), '\0');
    std::memcpy(&key[0], &gemm_mode, sizeof(int));
    std::memcpy(&key[sizeof(int)], descs, size_t(n) * sizeof(muon_matrix_desc_t));
    if (ds.key != key) {
        // a new descriptor set: its tables go to the head of the scratch (once;
        // later calls with the same set copy nothing and do not synchronize).
        // The copy and the synchronization cannot be captured into a graph.
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(stream, &cs);
        if (e != hipSuccess) return report_hip(st, e, "hipStreamIsCapturing");
        if (cs == hipStreamCaptureStatusActive) {
            st.code = MUON_ERR_BAD_ARG;
            snprintf(st.msg, sizeof(st.msg),
                     "the launch tables of this descriptor set are not resident: make one call "
                     "with it outside graph capture first (it copies them and synchronizes)");
            return report(st);
        }
        std::shared_ptr<HostPlan> hp;
        if (build_host_plan(descs, n, gemm_mode, capacity, &hp, &st) != MUON_OK) return report(st);
        const size_t bytes = host_plan_blob_bytes(*hp);
        if (bytes > kTableBytes) {
            st.code = MUON_ERR_WORKSPACE_TOO_SMALL;
            snprintf(st.msg, sizeof(st.msg),
                     "the launch tables of %lld matrices take %zu bytes; muon_step_noalloc "
                     "holds %zu",
                     (long long)n, bytes, kTableBytes);
            return report(st);
        }
        ds.key.clear();
        ds.plan.reset();
        e = hipMemcpyAsync(ds.ptr, host_plan_blob(*hp), bytes, hipMemcpyHostToDevice, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return report_hip(st, e, "upload of the launch tables");
        ds.plan = std::move(hp);
        ds.key = std::move(key);
    }
    std::vector<PlanView> views;
    for (int w = 0; w < host_plan_waves(*ds.plan); ++w)
        views.push_back(host_plan_view(*ds.plan, w, ds.ptr));
    e = enqueue_step(views.data(), int(views.size()), params, param_dtype, nullptr, grads,
                     momentum, h, ns_steps, ds.ptr + kTableBytes, stream);
    if (e != hipSuccess) return report_hip(st, e, "step");
    return MUON_OK;
}
