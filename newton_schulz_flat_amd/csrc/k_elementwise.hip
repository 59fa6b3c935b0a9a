// Elementwise phases of the Muon step on gfx950: momentum update and
// orthogonalization input ("Opt step" steps 1-2 of PR #6425,
// FsdpMuon._compute_momentum_inputs), the per-chunk sum of squares feeding
// the Frobenius norm, and the decoupled decay + update with the scatter of
// update slices to their shard destinations ("Opt step" steps 5-6,
// FsdpMuon._apply_local_updates).
//
// All three are HBM-bound streams: each workgroup owns one chunk of 512
// consecutive elements of one matrix (kEwChunk) and moves them with 16-byte
// (float4) nontemporal loads and stores, consecutive lanes on consecutive
// vectors.
// Floating-point contraction is off so that every multiply and add rounds on
// its own, in the documented order (bit-exact against a same-order float32
// reference).
#include "k_common.h"

#pragma clang fp contract(off)

namespace muon {

namespace {

// Deterministic block sum of one float per thread (fixed shuffle tree, then
// the kWaves wave sums in order).
template <int kWaves>
__device__ __forceinline__ float block_sum(float v, float* lds) {
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if (lane == 0) lds[wave] = v;
    __syncthreads();
    float t = 0.f;
    if (threadIdx.x == 0) {
        t = lds[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) t += lds[w];
    }
    return t;
}

// kMode 0: M <- beta M + G, U <- G + beta M (or M); partial sums of U^2.
// kMode 1: partial sums of U^2 only (U given).
// U element e of a matrix at offset off lives at u[e] (grads layout) or, with
// u_compact, at u[e - off + u_off] (the workspace's compact U region).
// Workgroup x of a launch handles chunk chunk0 + x.
template <int kMode>
__global__ __launch_bounds__(kFrontThreads) void front_kernel(
    const MatInfo* __restrict__ mats, const int32_t* __restrict__ prefix, int n,
    int32_t chunk0, const float* __restrict__ g, float* __restrict__ m,
    float* __restrict__ u_base, int u_compact, float* __restrict__ partial, Hyper h) {
    __shared__ float lds_w[kFrontThreads / 64];
    const int blk = chunk0 + int(blockIdx.x);
    const int mi = owner_of(prefix, n, blk);
    const HyperVals hv = hyper_for(h, mats[mi]);
    const float beta = hv.beta;
    const int nesterov = hv.nesterov;
    const int64_t off = mats[mi].off;
    const int64_t end = off + mats[mi].numel;
    const int64_t base = off + int64_t(blk - mats[mi].chunk_begin) * kEwChunk;
    // U element e (e counts from off, like G and M) is u_base[e + ud]
    const int64_t ud = u_compact ? mats[mi].u_off - off : int64_t(0);
    float ss = 0.f;
#pragma unroll
    for (int it = 0; it < kFrontIters; ++it) {
        const int64_t e = base + (int64_t(it) * kFrontThreads + threadIdx.x) * kEwVec;
        if (e + kEwVec <= end) {
            float4 uv;
            if (kMode == 0) {
                const float4 gv = load4_stream(g + e);
                const float4 mv = load4_stream(m + e);
                float4 m1;
                m1.x = beta * mv.x + gv.x;
                m1.y = beta * mv.y + gv.y;
                m1.z = beta * mv.z + gv.z;
                m1.w = beta * mv.w + gv.w;
                store4_stream(m + e, m1);
                if (nesterov) {
                    uv.x = beta * m1.x + gv.x;
                    uv.y = beta * m1.y + gv.y;
                    uv.z = beta * m1.z + gv.z;
                    uv.w = beta * m1.w + gv.w;
                } else {
                    uv = m1;
                }
                store4_stream(u_base + (e + ud), uv);
            } else {
                uv = load4_stream(u_base + (e + ud));
            }
            ss += uv.x * uv.x;
            ss += uv.y * uv.y;
            ss += uv.z * uv.z;
            ss += uv.w * uv.w;
        } else {
            for (int64_t k = e; k < end && k < e + kEwVec; ++k) {
                float uk;
                if (kMode == 0) {
                    const float gk = g[k];
                    const float m1 = beta * m[k] + gk;
                    m[k] = m1;
                    uk = nesterov ? beta * m1 + gk : m1;
                    u_base[k + ud] = uk;
                } else {
                    uk = u_base[k + ud];
                }
                ss += uk * uk;
            }
        }
    }
    if (partial != nullptr) {
        const float t = block_sum<kFrontThreads / 64>(ss, lds_w);
        if (threadIdx.x == 0) partial[blk] = t;
    }
}

__device__ __forceinline__ void store_w(float* p, float4 v) { store4_stream(p, v); }
__device__ __forceinline__ void store_w(uint16_t* p, float4 v) {
    const uint32_t lo = uint32_t(bf16_rne(v.x)) | (uint32_t(bf16_rne(v.y)) << 16);
    const uint32_t hi = uint32_t(bf16_rne(v.z)) | (uint32_t(bf16_rne(v.w)) << 16);
    store2_stream(reinterpret_cast<uint2*>(p), make_uint2(lo, hi));
}
__device__ __forceinline__ float4 load_w(const float* p) { return load4_stream(p); }
__device__ __forceinline__ float4 load_w(const uint16_t* p) {
    const uint2 b = load2_stream(reinterpret_cast<const uint2*>(p));
    return make_float4(__uint_as_float(b.x << 16), __uint_as_float(b.x & 0xffff0000u),
                       __uint_as_float(b.y << 16), __uint_as_float(b.y & 0xffff0000u));
}
__device__ __forceinline__ float load_w1(const float* p) { return *p; }
__device__ __forceinline__ float load_w1(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void store_w1(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_w1(uint16_t* p, float v) { *p = bf16_rne(v); }

// W1 = fl(W f); Wn = fl(W1 - fl(lr O)); element j of the flattened matrix
// lives in slice j / slice_len at param offset poff + k pstride + j % slice_len.
// O of the matrix at o[off ...] (grads layout) or, with o_compact, at
// o[u_off ...] (the workspace's compact region).
template <typename TW>
__global__ __launch_bounds__(kApplyThreads) void apply_kernel(
    const MatInfo* __restrict__ mats, const int32_t* __restrict__ prefix, int n,
    int32_t chunk0, TW* __restrict__ w, const float* __restrict__ o, int o_compact, Hyper h,
    uint16_t* __restrict__ copy) {
    const int blk = chunk0 + int(blockIdx.x);
    const int mi = owner_of(prefix, n, blk);
    const MatInfo& mt = mats[mi];
    const HyperVals hv = hyper_for(h, mt);
    const float decay = hv.decay, lr = hv.lr;
    const int64_t numel = mt.numel, off = o_compact ? mt.u_off : mt.off, poff = mt.poff;
    const int64_t slice = mt.slice_len, stride = mt.pstride;
    const bool sharded = slice != numel;
    const double inv_slice = 1.0 / double(slice);
    const int64_t base = int64_t(blk - mt.chunk_begin) * kEwChunk;
#pragma unroll
    for (int it = 0; it < kApplyIters; ++it) {
        const int64_t j = base + (int64_t(it) * kApplyThreads + threadIdx.x) * kEwVec;
        if (j + kEwVec <= numel) {
            // slices are multiples of 8 long when sharded: a vector never straddles two
            int64_t dst = poff + j;
            if (sharded) {
                const int64_t k = slice_index(j, slice, inv_slice);
                dst = poff + k * stride + (j - k * slice);
            }
            const float4 ov = load4_stream(o + off + j);
            const float4 wv = load_w(w + dst);
            float4 r;
            r.x = wv.x * decay - lr * ov.x;
            r.y = wv.y * decay - lr * ov.y;
            r.z = wv.z * decay - lr * ov.z;
            r.w = wv.w * decay - lr * ov.w;
            store_w(w + dst, r);
            if (copy != nullptr) store_w(copy + dst, r);
        } else {
            for (int64_t k = j; k < numel && k < j + kEwVec; ++k) {
                const int64_t s = sharded ? slice_index(k, slice, inv_slice) : 0;
                const int64_t dst = poff + s * stride + (k - s * slice);
                const float w1 = load_w1(w + dst) * decay;
                const float t = lr * o[off + k];
                const float wn = w1 - t;
                store_w1(w + dst, wn);
                if (copy != nullptr) store_w1(copy + dst, wn);
            }
        }
    }
}

// A launch's grid counts at most 2^32 - 1 work-items: sets of more than
// kEwGridChunks chunks (8 G elements) run as several launches in chunk order.
constexpr int64_t kEwGridChunks = int64_t(1) << 24;
static_assert(kEwGridChunks * kFrontThreads < (int64_t(1) << 32), "front grid");
static_assert(kEwGridChunks * kApplyThreads < (int64_t(1) << 32), "apply grid");

template <typename F>
hipError_t for_each_grid(int64_t total, F launch) {
    for (int64_t c0 = 0; c0 < total; c0 += kEwGridChunks) {
        launch(int32_t(c0), dim3(unsigned(std::min(kEwGridChunks, total - c0))));
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_front(const PlanView& p, const float* grads, float* momentum, float* u,
                        bool compact, float* partial, const Hyper& h, hipStream_t s) {
    if (p.total_chunks == 0) return hipSuccess;
    LaunchTimer timer("front", s);
    return for_each_grid(p.total_chunks, [&](int32_t c0, dim3 grid) {
        front_kernel<0><<<grid, dim3(kFrontThreads), 0, s>>>(
            p.mats, p.chunk_prefix, p.n, c0, grads, momentum, u, compact ? 1 : 0, partial, h);
    });
}

hipError_t launch_sumsq(const PlanView& p, const float* u, float* partial, hipStream_t s) {
    if (p.total_chunks == 0) return hipSuccess;
    LaunchTimer timer("sumsq", s);
    return for_each_grid(p.total_chunks, [&](int32_t c0, dim3 grid) {
        front_kernel<1><<<grid, dim3(kFrontThreads), 0, s>>>(
            p.mats, p.chunk_prefix, p.n, c0, nullptr, nullptr, const_cast<float*>(u), 0,
            partial, Hyper{});
    });
}

hipError_t launch_apply(const PlanView& p, void* params, int param_dtype, const float* o,
                        bool compact, const Hyper& h, uint16_t* model_copy, hipStream_t s) {
    if (p.total_chunks == 0) return hipSuccess;
    LaunchTimer timer("apply", s);
    const dim3 block{kApplyThreads};
    const int oc = compact ? 1 : 0;
    return for_each_grid(p.total_chunks, [&](int32_t c0, dim3 grid) {
        if (param_dtype == MUON_DTYPE_BF16)
            apply_kernel<uint16_t><<<grid, block, 0, s>>>(p.mats, p.chunk_prefix, p.n, c0,
                                                          static_cast<uint16_t*>(params), o, oc,
                                                          h, nullptr);
        else
            apply_kernel<float><<<grid, block, 0, s>>>(p.mats, p.chunk_prefix, p.n, c0,
                                                       static_cast<float*>(params), o, oc, h,
                                                       model_copy);
    });
}

}  // namespace muon
