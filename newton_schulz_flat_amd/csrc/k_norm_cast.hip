// Frobenius normalization and layout change into the Newton-Schulz
// orientation, on gfx950.
//
// norm_kernel: one workgroup per matrix sums that matrix's partial sums of
// squares (per elementwise chunk, or per 64 x 64 tile) in a fixed order and
// stores inv = 1 / (sqrt(sum) + 1e-7).
//
// front_cast_kernel: one workgroup per 4096 elements of the padded
// NS-orientation matrix (as many workgroups as cast_kernel has 64 x 64 tiles).
// It reads the matching elements of G and M (or of U) along U's rows,
// computes M <- fl(fl(beta M) + G) (stored) and U = fl(fl(beta M) + G) (or M)
// in float32 exactly as the elementwise front kernel does, stores U rounded to
// the Newton-Schulz type -- not yet divided by its norm: the first iteration
// applies 1 / ||U|| in its float32 epilogues -- in NS orientation, and writes
// the workgroup's sum of squares of U (fixed order) for norm_kernel.  A wide or
// square matrix keeps its orientation, and each workgroup streams a contiguous
// run of the padded iterate; a tall one is handled in blocks of 32 x 128 (or
// 64 x 64) elements of U transposed through LDS.  G and M are streamed with nontemporal accesses.  One pass
// replaces front + cast.
//
// cast_kernel: one workgroup per 64 x 64 tile of the padded NS-orientation
// matrix X0 (rp x cp).  It reads the matching 64 x 64 block of U in U's own
// row-major orientation (coalesced along U's rows), scales it by inv, and
// writes X0 along its rows, transposing through LDS when the matrix is tall
// (rows > cols: tall matrices are transposed into the wide orientation here).
// Elements outside the r x c matrix are written as zero, which the
// Newton-Schulz products preserve.  With ns_steps == 0 it writes
// O = fl(s * X0) in U's own layout instead.
#include "k_common.h"

#pragma clang fp contract(off)

namespace muon {

namespace {

constexpr int kNormThreads = 256;

__global__ __launch_bounds__(kNormThreads) void norm_kernel(const MatInfo* __restrict__ mats,
                                                            const float* __restrict__ partial,
                                                            float* __restrict__ inv, int per_tile) {
    __shared__ float red[kNormThreads];
    const int mi = blockIdx.x;
    const int begin = per_tile ? mats[mi].cast_begin : mats[mi].chunk_begin;
    const int count = per_tile ? mats[mi].n_cast : mats[mi].n_chunks;
    float s = 0.f;
    for (int i = threadIdx.x; i < count; i += kNormThreads) s += partial[begin + i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = kNormThreads / 2; w >= 1; w >>= 1) {
        if (threadIdx.x < w) red[threadIdx.x] = red[threadIdx.x] + red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) inv[mi] = 1.0f / (sqrtf(red[0]) + kNormEps);
}

__device__ __forceinline__ void store_x4(float* p, const float v[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store_x4(uint16_t* p, const float v[4]) {
    const uint32_t lo = uint32_t(bf16_rne(v[0])) | (uint32_t(bf16_rne(v[1])) << 16);
    const uint32_t hi = uint32_t(bf16_rne(v[2])) | (uint32_t(bf16_rne(v[3])) << 16);
    *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
}
__device__ __forceinline__ float rounded(float v, float*) { return v; }
__device__ __forceinline__ float rounded(float v, uint16_t*) { return bf16_to_f32(bf16_rne(v)); }

// U (and O) of a matrix at its offset in the grads layout, or (compact) at its
// u_off in the workspace's compact region.
template <typename TX>
__global__ __launch_bounds__(256) void cast_kernel(const MatInfo* __restrict__ mats,
                                                   const int32_t* __restrict__ prefix, int n,
                                                   const float* u,  // may equal o_direct
                                                   const float* __restrict__ inv,
                                                   TX* __restrict__ x, float* o_direct,
                                                   int compact) {
    constexpr int T = kCastTile;
    __shared__ float tile[T][T + 1];
    const int blk = blockIdx.x;
    const int mi = owner_of(prefix, n, blk);
    const MatInfo& mt = mats[mi];
    const int t = blk - mt.cast_begin;
    const int ntj = mt.cp / T;
    const int ti = t / ntj, tj = t % ntj;
    const bool tall = mt.tall != 0;
    // Tile origin in U's own (R x C) coordinates.
    const int ur0 = tall ? tj * T : ti * T;
    const int uc0 = tall ? ti * T : tj * T;
    const float scale_inv = inv[mi];
    const int64_t uoff = compact ? mt.u_off : mt.off;
    const float* um = u + uoff;
    for (int idx = threadIdx.x; idx < T * T; idx += 256) {
        const int rr = idx / T, cc = idx % T;
        const int gr = ur0 + rr, gc = uc0 + cc;
        float v = 0.f;
        if (gr < mt.R && gc < mt.C) v = um[int64_t(gr) * mt.C + gc] * scale_inv;
        tile[rr][cc] = v;
    }
    __syncthreads();
    if (o_direct != nullptr) {
        // No iterations: O = fl(s * X0), X0 rounded to the storage type.
        float* om = o_direct + uoff;
        for (int idx = threadIdx.x; idx < T * T; idx += 256) {
            const int rr = idx / T, cc = idx % T;
            const int gr = ur0 + rr, gc = uc0 + cc;
            if (gr < mt.R && gc < mt.C)
                om[int64_t(gr) * mt.C + gc] =
                    mt.scale * (mt.ns_f32 ? tile[rr][cc] : rounded(tile[rr][cc], x));
        }
        return;
    }
    // X0[i][j], i = ti*T + a, j = tj*T + b  (native element tile[a][b] or tile[b][a]);
    // each thread writes 4 consecutive elements of a row
    for (int idx = threadIdx.x; idx < T * T / 4; idx += 256) {
        const int a = idx / (T / 4), b = (idx % (T / 4)) * 4;
        float v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = tall ? tile[b + t][a] : tile[a][b + t];
        const int64_t at = int64_t(ti * T + a) * mt.cp + tj * T + b;
        if (mt.ns_f32)
            store_x4(reinterpret_cast<float*>(x) + mt.x_off + at, v);
        else
            store_x4(x + mt.x_off + at, v);
    }
}

template <typename TX, bool kStep>
__global__ __launch_bounds__(256) void front_cast_kernel(const MatInfo* __restrict__ mats,
                                                         const int32_t* __restrict__ prefix, int n,
                                                         const float* __restrict__ g, float* __restrict__ m,
                                                         const float* __restrict__ u_in, Hyper h,
                                                         TX* __restrict__ x,
                                                         float* __restrict__ partial) {
    constexpr int T = kCastTile;
    constexpr int kIters = T * T / 4 / 256;  // 4-element groups per thread
    // tall blocks: TR rows of TC + 1 floats (TR = 64 or 32)
    __shared__ float tile[T * (T + 1)];
    __shared__ float wsum[4];
    const int blk = blockIdx.x;
    const int mi = owner_of(prefix, n, blk);
    const MatInfo& mt = mats[mi];
    const int t = blk - mt.cast_begin;
    const bool tall = mt.tall != 0;
    const bool vec = (mt.C & 3) == 0;  // rows start 16-byte aligned
    const HyperVals hv = hyper_for(h, mt);
    const float beta = hv.beta;
    const int nesterov = hv.nesterov;
    // Each thread first loads all of its G and M (or U) groups and only then
    // stores: loads and stores share the vector memory counter, and with both
    // kinds pending a wait for a load is a wait for the counter to reach zero
    // (their completion order is not known), store included.
    // G and M (or U, in gv) at 4 consecutive elements of U's row gr from column
    // gc; zero outside R x C.
    auto load4 = [&](int gr, int gc, float gv[4], float mv[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) gv[q] = mv[q] = 0.f;
        if (gr >= mt.R || gc >= mt.C) return;
        const int64_t e = mt.off + int64_t(gr) * mt.C + gc;
        if (vec && gc + 3 < mt.C) {
            const float4 a4 = load4_stream((kStep ? g : u_in) + e);
            gv[0] = a4.x, gv[1] = a4.y, gv[2] = a4.z, gv[3] = a4.w;
            if (kStep) {
                const float4 b4 = load4_stream(m + e);
                mv[0] = b4.x, mv[1] = b4.y, mv[2] = b4.z, mv[3] = b4.w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (gc + q < mt.C) {
                    gv[q] = (kStep ? g : u_in)[e + q];
                    if (kStep) mv[q] = m[e + q];
                }
            }
        }
    };
    // U from the loaded values; with kStep, M <- fl(fl(beta M) + G) is stored
    auto update4 = [&](int gr, int gc, const float gv[4], const float mv[4], float uv[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) uv[q] = 0.f;
        if (gr >= mt.R || gc >= mt.C) return;
        if (!kStep) {
#pragma unroll
            for (int q = 0; q < 4; ++q) uv[q] = gv[q];
            return;
        }
        const int64_t e = mt.off + int64_t(gr) * mt.C + gc;
        float m1[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            m1[q] = beta * mv[q] + gv[q];
            uv[q] = nesterov ? beta * m1[q] + gv[q] : m1[q];
        }
        if (vec && gc + 3 < mt.C) {
            store4_stream(m + e, make_float4(m1[0], m1[1], m1[2], m1[3]));
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (gc + q < mt.C) m[e + q] = m1[q];
                else uv[q] = 0.f;
            }
        }
    };
    // Rows whose length is not a multiple of 4 start at unaligned addresses:
    // their G and M (or U) are read as aligned 4-element vectors covering the
    // workgroup's elements (a vector is read whole when it lies inside the
    // matrix, else element by element), M is stored for the workgroup's own
    // elements only, and U goes through LDS to the iterate.  The values, and
    // the order in which the sum of squares adds them, are those of the aligned
    // path.  Vector at matrix-relative element a (a % 4 == 0; a < 0: none).
    constexpr int kV = 5;  // vectors per thread: <= 1025 (wide) or 1088 (tall) per workgroup
    auto loadv = [&](int64_t a, float gv[4], float mv[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) gv[q] = mv[q] = 0.f;
        if (a < 0) return;
        const int64_t e = mt.off + a;
        if (a + 4 <= mt.numel) {
            const float4 a4 = load4_stream((kStep ? g : u_in) + e);
            gv[0] = a4.x, gv[1] = a4.y, gv[2] = a4.z, gv[3] = a4.w;
            if (kStep) {
                const float4 b4 = load4_stream(m + e);
                mv[0] = b4.x, mv[1] = b4.y, mv[2] = b4.z, mv[3] = b4.w;
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (a + q < mt.numel) {
                    gv[q] = (kStep ? g : u_in)[e + q];
                    if (kStep) mv[q] = m[e + q];
                }
            }
        }
    };
    // U of the vector's elements; with kStep, M is stored for those in [lo, hi)
    auto updv = [&](int64_t a, int64_t lo, int64_t hi, const float gv[4], const float mv[4],
                    float uv[4]) {
        if (!kStep) {
#pragma unroll
            for (int q = 0; q < 4; ++q) uv[q] = gv[q];
            return;
        }
        float m1[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            m1[q] = beta * mv[q] + gv[q];
            uv[q] = nesterov ? beta * m1[q] + gv[q] : m1[q];
        }
        const int64_t e = mt.off + a;
        if (a >= lo && a + 4 <= hi) {
            store4_stream(m + e, make_float4(m1[0], m1[1], m1[2], m1[3]));
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (a + q >= lo && a + q < hi) m[e + q] = m1[q];
        }
    };
    float ss = 0.f;
    // X (NS orientation) at element offset at of this matrix, in its product type
    auto store_iter4 = [&](int64_t at, const float v[4]) {
        if (mt.ns_f32)
            store_x4(reinterpret_cast<float*>(x) + mt.x_off + at, v);
        else
            store_x4(x + mt.x_off + at, v);
    };
    // Tall: workgroup t takes a block of TR rows x TC = 4096 / TR columns of U
    // (iterate tile (ti, tj): TC iterate rows by TR iterate columns), read along
    // U's rows (TC / 4 consecutive threads per row) and transposed through LDS.
    // Consecutive workgroups take consecutive ti, i.e. neighbouring column
    // blocks of the same TR rows of U.  TR = 32 (512-byte runs of G and M)
    // where the iterate's padded row count is a multiple of 128, else 64.
    const int tall_rows = (mt.rp % 128 == 0) ? 32 : 64;
    auto tall_in = [&](auto tr_tag) {
        constexpr int TR = decltype(tr_tag)::value, TC = T * T / TR, kSegs = TC / 4;
        const int nti = mt.rp / TC;
        const int tj = t / nti, ti = t % nti;
        const int ur0 = tj * TR, uc0 = ti * TC;  // block origin in U's (R x C) coordinates
        float gv[kIters][4], mv[kIters][4];
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int seg = it * 256 + int(threadIdx.x);
            load4(ur0 + seg / kSegs, uc0 + (seg % kSegs) * 4, gv[it], mv[it]);
        }
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int seg = it * 256 + int(threadIdx.x);
            const int rr = seg / kSegs, c4 = (seg % kSegs) * 4;
            float uv[4];
            update4(ur0 + rr, uc0 + c4, gv[it], mv[it], uv);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                tile[rr * (TC + 1) + c4 + q] = uv[q];
                ss = ss + uv[q] * uv[q];
            }
        }
    };
    // tall_in for rows not a multiple of 4 long: the block's row segments are
    // read as aligned vectors (row rr: the vectors from its first element's
    // aligned start), U written into the block tile; then, in tall_in's order,
    // the sum of squares, with the tile's entries outside R x C set to zero
    auto tall_in_unaligned = [&](auto tr_tag) {
        constexpr int TR = decltype(tr_tag)::value, TC = T * T / TR, kSegs = TC / 4;
        constexpr int kVpr = TC / 4 + 1;  // vectors per row segment
        const int nti = mt.rp / TC;
        const int tj = t / nti, ti = t % nti;
        const int ur0 = tj * TR, uc0 = ti * TC;
        const int64_t C = mt.C;
        const int64_t cw = uc0 < C ? (C - uc0 < TC ? C - uc0 : TC) : 0;  // real columns
        float gv[kV][4], mv[kV][4];
        int64_t av[kV];
#pragma unroll
        for (int k = 0; k < kV; ++k) {
            const int v = k * 256 + int(threadIdx.x);
            const int rr = v / kVpr, kk = v % kVpr, gr = ur0 + rr;
            const int64_t lo = int64_t(gr) * C + uc0;
            const int64_t a = (lo & ~int64_t(3)) + 4 * kk;
            av[k] = (v < TR * kVpr && gr < mt.R && cw > 0 && a < lo + cw) ? a : -1;
            loadv(av[k], gv[k], mv[k]);
        }
#pragma unroll
        for (int k = 0; k < kV; ++k) {
            if (av[k] < 0) continue;
            const int rr = (k * 256 + int(threadIdx.x)) / kVpr;
            const int64_t lo = int64_t(ur0 + rr) * C + uc0;
            float uv[4];
            updv(av[k], lo, lo + cw, gv[k], mv[k], uv);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t el = av[k] + q;
                if (el >= lo && el < lo + cw) tile[rr * (TC + 1) + int(el - lo)] = uv[q];
            }
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int seg = it * 256 + int(threadIdx.x);
            const int rr = seg / kSegs, c4 = (seg % kSegs) * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float* cell = &tile[rr * (TC + 1) + c4 + q];
                const bool in = ur0 + rr < mt.R && c4 + q < cw;
                const float u = in ? *cell : 0.f;
                if (!in) *cell = 0.f;
                ss = ss + u * u;
            }
        }
    };
    // X[i][j], i = ti*TC + a, j = tj*TR + b = U[j][i] = block element (b, a); each
    // thread writes 4 consecutive elements of a row
    auto tall_out = [&](auto tr_tag) {
        constexpr int TR = decltype(tr_tag)::value, TC = T * T / TR;
        const int nti = mt.rp / TC;
        const int tj = t / nti, ti = t % nti;
        for (int idx = threadIdx.x; idx < T * T / 4; idx += 256) {
            const int a = idx / (TR / 4), b = (idx % (TR / 4)) * 4;
            float v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = tile[(b + q) * (TC + 1) + a];
            store_iter4(int64_t(ti * TC + a) * mt.cp + tj * TR + b, v);
        }
    };
    if (!tall && !vec) {
        // wide, rows not a multiple of 4 long: the workgroup's elements of U are
        // one flat run [lo, hi) of the matrix (its rows are contiguous)
        const int64_t base = int64_t(t) * (T * T);
        const int64_t last = base + T * T - 1;
        const int i0 = int(base / mt.cp), j0 = int(base % mt.cp);
        const int i1 = int(last / mt.cp), j1 = int(last % mt.cp) + 1;
        const int64_t C = mt.C;
        const int64_t lo = i0 < mt.R ? int64_t(i0) * C + (j0 < C ? j0 : C) : mt.numel;
        const int64_t hi = i1 < mt.R ? int64_t(i1) * C + (j1 < C ? j1 : C) : mt.numel;
        const int64_t a0 = lo & ~int64_t(3);
        const int nv = int((hi - a0 + 3) >> 2);
        float gv[kV][4], mv[kV][4];
#pragma unroll
        for (int k = 0; k < kV; ++k) {
            const int v = k * 256 + int(threadIdx.x);
            loadv(v < nv ? a0 + 4 * int64_t(v) : -1, gv[k], mv[k]);
        }
#pragma unroll
        for (int k = 0; k < kV; ++k) {
            const int v = k * 256 + int(threadIdx.x);
            if (v >= nv) continue;
            float uv[4];
            updv(a0 + 4 * int64_t(v), lo, hi, gv[k], mv[k], uv);
#pragma unroll
            for (int q = 0; q < 4; ++q) tile[4 * v + q] = uv[q];
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int e = j0 + (it * 256 + int(threadIdx.x)) * 4;
            const int gr = i0 + e / mt.cp, gc = e % mt.cp;
            float uv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uv[q] = (gr < mt.R && gc + q < C) ? tile[int(int64_t(gr) * C + gc + q - a0)] : 0.f;
                ss = ss + uv[q] * uv[q];
            }
            store_iter4(base + (it * 256 + int(threadIdx.x)) * 4, uv);
        }
    } else if (!tall) {
        // The iterate has U's own orientation: workgroup t takes the 4096
        // consecutive elements [4096 t, 4096 t + 4096) of the row-major rp x cp
        // iterate (rows padded to cp), thread tid the 4-element groups
        // it * 256 + tid, so that G, M and X stream along rows.
        const int64_t base = int64_t(t) * (T * T);
        const int i0 = int(base / mt.cp), j0 = int(base % mt.cp);
        int gr[kIters], gc[kIters];
        float gv[kIters][4], mv[kIters][4];
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            const int e = j0 + (it * 256 + int(threadIdx.x)) * 4;
            gr[it] = i0 + e / mt.cp, gc[it] = e % mt.cp;
            load4(gr[it], gc[it], gv[it], mv[it]);
        }
#pragma unroll
        for (int it = 0; it < kIters; ++it) {
            float uv[4];
            update4(gr[it], gc[it], gv[it], mv[it], uv);
#pragma unroll
            for (int q = 0; q < 4; ++q) ss = ss + uv[q] * uv[q];
            store_iter4(base + (it * 256 + int(threadIdx.x)) * 4, uv);
        }
    } else if (!vec) {
        if (tall_rows == 32)
            tall_in_unaligned(std::integral_constant<int, 32>{});
        else
            tall_in_unaligned(std::integral_constant<int, 64>{});
    } else if (tall_rows == 32) {
        tall_in(std::integral_constant<int, 32>{});
    } else {
        tall_in(std::integral_constant<int, 64>{});
    }
    // deterministic block sum: fixed shuffle tree, then the 4 wave sums in order
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0) partial[blk] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
    if (tall) {
        if (tall_rows == 32)
            tall_out(std::integral_constant<int, 32>{});
        else
            tall_out(std::integral_constant<int, 64>{});
    }
}

}  // namespace

hipError_t launch_norm(const PlanView& p, const float* partial, float* inv, bool per_tile,
                       hipStream_t s) {
    if (p.n == 0) return hipSuccess;
    LaunchTimer timer("norm", s);
    norm_kernel<<<dim3(unsigned(p.n)), dim3(kNormThreads), 0, s>>>(p.mats, partial, inv,
                                                                   per_tile ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_front_cast(const PlanView& p, const float* grads, float* momentum,
                             const float* u, const Hyper& h, void* ws, float* partial,
                             hipStream_t s) {
    if (p.total_cast == 0) return hipSuccess;
    const bool step = u == nullptr;
    LaunchTimer timer(step ? "front_cast" : "sumsq_cast", s);
    unsigned char* w = static_cast<unsigned char*>(ws);
    const dim3 grid{static_cast<unsigned>(p.total_cast)}, block{256};
    if (p.gemm_mode == MUON_GEMM_F32) {
        float* x = reinterpret_cast<float*>(w + p.ws.x[0]);
        if (step)
            front_cast_kernel<float, true><<<grid, block, 0, s>>>(p.mats, p.cast_prefix, p.n, grads,
                                                                  momentum, nullptr, h, x, partial);
        else
            front_cast_kernel<float, false><<<grid, block, 0, s>>>(p.mats, p.cast_prefix, p.n, nullptr,
                                                                   nullptr, u, Hyper{}, x, partial);
    } else {
        uint16_t* x = reinterpret_cast<uint16_t*>(w + p.ws.x[0]);
        if (step)
            front_cast_kernel<uint16_t, true><<<grid, block, 0, s>>>(p.mats, p.cast_prefix, p.n, grads,
                                                                     momentum, nullptr, h, x, partial);
        else
            front_cast_kernel<uint16_t, false><<<grid, block, 0, s>>>(p.mats, p.cast_prefix, p.n,
                                                                      nullptr, nullptr, u, Hyper{}, x,
                                                                      partial);
    }
    return hipGetLastError();
}

hipError_t launch_cast(const PlanView& p, const float* u, const float* inv, void* ws,
                       float* o_direct, bool compact, hipStream_t s) {
    if (p.total_cast == 0) return hipSuccess;
    LaunchTimer timer("cast", s);
    unsigned char* w = static_cast<unsigned char*>(ws);
    const dim3 grid{static_cast<unsigned>(p.total_cast)}, block{256};
    if (p.gemm_mode == MUON_GEMM_F32)
        cast_kernel<float><<<grid, block, 0, s>>>(p.mats, p.cast_prefix, p.n, u, inv,
                                                  reinterpret_cast<float*>(w + p.ws.x[0]),
                                                  o_direct, compact ? 1 : 0);
    else
        cast_kernel<uint16_t><<<grid, block, 0, s>>>(p.mats, p.cast_prefix, p.n, u, inv,
                                                     reinterpret_cast<uint16_t*>(w + p.ws.x[0]),
                                                     o_direct, compact ? 1 : 0);
    return hipGetLastError();
}

}  // namespace muon
