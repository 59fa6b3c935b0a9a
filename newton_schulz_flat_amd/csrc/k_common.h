// Device helpers shared by the gfx950 kernels of the Muon step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "muon_internal.h"

namespace muon {

// Matrix owning workgroup b: the largest m with prefix[m] <= b.  prefix has
// n + 1 non-decreasing entries and every matrix owns at least one workgroup.
__device__ __forceinline__ int owner_of(const int32_t* __restrict__ prefix, int n, int b) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (prefix[mid] <= b)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Shard slice of flattened element e of a sharded matrix (0 <= e < numel <=
// 2^34, slices of slice >= 8 elements): e / slice without a 64-bit integer
// division.  inv_slice = 1.0 / slice.  The double estimate e * inv_slice lies
// within q 2^-51 of the quotient q < 2^31, well inside the 1 / slice distance
// from q up to the next integer, so it truncates to floor(q) or, where q is an
// integer, possibly to q - 1; one integer comparison makes it exact.
__device__ __forceinline__ int64_t slice_index(int64_t e, int64_t slice, double inv_slice) {
    int64_t k = int(double(e) * inv_slice);
    k += (k + 1) * slice <= e ? 1 : 0;
    return k;
}

// float32 -> bfloat16 bits, round to nearest even (IEEE-754 definition on the
// bit pattern); NaN becomes a quiet NaN keeping sign and top payload bits.
__device__ __forceinline__ uint16_t bf16_rne(float x) {
    const uint32_t b = __float_as_uint(x);
    if ((b & 0x7fffffffu) > 0x7f800000u) return uint16_t((b >> 16) | 0x40u);
    const uint32_t lsb = (b >> 16) & 1u;
    return uint16_t((b + 0x7fffu + lsb) >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// 16-byte loads and stores of data that is touched once per pass (optimizer
// state streams): nontemporal, so that they do not displace cached operands.
typedef float f32x4_stream __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load4_stream(const float* p) {
    const f32x4_stream t = __builtin_nontemporal_load(reinterpret_cast<const f32x4_stream*>(p));
    return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void store4_stream(float* p, float4 v) {
    const f32x4_stream t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, reinterpret_cast<f32x4_stream*>(p));
}
typedef uint32_t u32x2_stream __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 load2_stream(const uint2* p) {
    const u32x2_stream t = __builtin_nontemporal_load(reinterpret_cast<const u32x2_stream*>(p));
    return make_uint2(t.x, t.y);
}
__device__ __forceinline__ void store2_stream(uint2* p, uint2 v) {
    const u32x2_stream t = {v.x, v.y};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x2_stream*>(p));
}

// One matrix's optimizer scalars; decay = fl(1 - fl(lr * wd)), the same two
// roundings as on the host.
struct HyperVals {
    float lr, decay, beta;
    int nesterov;
};
__device__ __forceinline__ HyperVals hyper_for(const Hyper& h, const MatInfo& mt) {
#pragma clang fp contract(off)
    HyperVals v;
    float wd;
    if (h.groups != nullptr) {
        const muon_group_t g = h.groups[mt.group];
        v.lr = g.lr, wd = g.weight_decay, v.beta = g.beta, v.nesterov = g.nesterov != 0;
    } else {
        v.lr = h.lr, wd = h.weight_decay, v.beta = h.beta, v.nesterov = h.nesterov;
    }
    const float lrwd = v.lr * wd;
    v.decay = 1.0f - lrwd;
    return v;
}

}  // namespace muon
