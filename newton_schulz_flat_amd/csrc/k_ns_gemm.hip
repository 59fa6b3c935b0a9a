// Newton-Schulz product chain on gfx950 matrix cores.
//
// One iteration of the quintic Newton-Schulz orthogonalization is three
// products, every one of them of the form C = P Q^T with both operands
// row-major along the contraction index ("NT"):
//
//   stage A   A = X X^T            P = Q = X   (rp x cp), K = cp   symmetric
//   stage B   B = b A + c A A^T    P = Q = A   (rp x rp), K = rp   symmetric
//   stage X   X <- a X + B X       P = B, Q = X^T (cp x rp), K = rp
//
// (A is symmetric, so A A = A A^T, and B X = B (X^T)^T.)  Keeping X^T next to
// X makes every operand load a contiguous run along K, which is exactly what
// the MFMA operand layout wants (8 consecutive K values per lane for bf16).
//
// Symmetric stages compute only tiles with ti <= tj and mirror each
// off-diagonal tile into (tj, ti).  The axpys b A + c (.) and a X + (.) run in
// float32 in the epilogues; the stage-B epilogue reads A and the stage-X
// epilogue reads X from the transposed copies, whose 4 consecutive elements
// match the 4 consecutive output rows each lane holds.  Stage X writes X in
// place (no workgroup reads X during stage X) and X^T into the other
// ping-pong buffer; on the last iteration it writes O = fl(s * X) in the
// matrix's original orientation instead.
//
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid over a TILE x TILE output
// tile; each wave owns (TILE/2)^2 outputs as 32 x 32 MFMA fragments.  K is
// consumed in blocks of 128 bytes per row (64 bf16 / 32 float32), staged
// through double-buffered LDS with rows padded to 144 bytes so that the 16-byte
// fragment reads of 8 consecutive rows hit distinct banks.  One grouped launch
// per stage and tile size covers every matrix, driven by a tile table.
#include <type_traits>

#include "k_common.h"

namespace muon {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum Stage { kStageA = 0, kStageB = 1, kStageX = 2 };

struct NsArgs {
    const MatInfo* mats;
    const GemmTile* tiles;
    void* x;        // X region
    void* xt_cur;   // X^T read by this iteration
    void* xt_next;  // X^T written by this iteration
    void* ga;       // A region
    void* gb;       // B region
    float* o;       // O (last iteration), laid out like the gradients
    float ca, cb, cc;
    int last;
};

constexpr int kRowBytes = 128;  // K block: bytes of one operand row
constexpr int kLdsStride = 144;  // padded LDS row

template <int TILE>
struct TileGeo {
    static constexpr int kOp = TILE * kLdsStride;            // bytes of one operand tile
    static constexpr int kWt = TILE / 2;                     // wave tile side
    static constexpr int kNf = kWt / 32;                     // fragments per wave side
    static constexpr int kLoads = TILE * (kRowBytes / 16) / 256;  // 16-byte loads / thread / operand
};

__device__ __forceinline__ float load_e(const float* p) { return *p; }
__device__ __forceinline__ float load_e(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void store_e(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_e(uint16_t* p, float v) { *p = bf16_rne(v); }

__device__ __forceinline__ void load4(const float* p, float v[4]) {
    const float4 t = *reinterpret_cast<const float4*>(p);
    v[0] = t.x, v[1] = t.y, v[2] = t.z, v[3] = t.w;
}
__device__ __forceinline__ void load4(const uint16_t* p, float v[4]) {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(t.x << 16), v[1] = __uint_as_float(t.x & 0xffff0000u);
    v[2] = __uint_as_float(t.y << 16), v[3] = __uint_as_float(t.y & 0xffff0000u);
}
__device__ __forceinline__ void store4(float* p, const float v[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(uint16_t* p, const float v[4]) {
    const uint32_t lo = uint32_t(bf16_rne(v[0])) | (uint32_t(bf16_rne(v[1])) << 16);
    const uint32_t hi = uint32_t(bf16_rne(v[2])) | (uint32_t(bf16_rne(v[3])) << 16);
    *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
}

template <int TILE, bool BF16, int STAGE>
__global__ __launch_bounds__(256) void ns_gemm_kernel(NsArgs args) {
    using TE = std::conditional_t<BF16, uint16_t, float>;
    using G = TileGeo<TILE>;
    constexpr int kEs = BF16 ? 2 : 4;
    constexpr int kBk = kRowBytes / kEs;  // K elements per block
    constexpr int kNf = G::kNf;
    __shared__ __attribute__((aligned(16))) unsigned char lds[2 * 2 * G::kOp];

    const GemmTile tile = args.tiles[blockIdx.x];
    if (tile.mat < 0) return;  // padding slot of the XCD-interleaved table
    const MatInfo& mt = args.mats[tile.mat];
    const int rp = mt.rp, cp = mt.cp;
    const int ti = tile.ti, tj = tile.tj;

    const TE* P;
    const TE* Q;
    int ld, K;
    if (STAGE == kStageA) {
        const TE* base = static_cast<const TE*>(args.x) + mt.x_off;
        P = base + int64_t(ti) * TILE * cp;
        Q = base + int64_t(tj) * TILE * cp;
        ld = cp;
        K = cp;
    } else if (STAGE == kStageB) {
        const TE* base = static_cast<const TE*>(args.ga) + mt.g_off;
        P = base + int64_t(ti) * TILE * rp;
        Q = base + int64_t(tj) * TILE * rp;
        ld = rp;
        K = rp;
    } else {
        P = static_cast<const TE*>(args.gb) + mt.g_off + int64_t(ti) * TILE * rp;
        Q = static_cast<const TE*>(args.xt_cur) + mt.x_off + int64_t(tj) * TILE * rp;
        ld = rp;
        K = rp;
    }

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 31, hk = lane >> 5;

    uint4 rp_[G::kLoads], rq_[G::kLoads];
    auto gload = [&](int kb) {
#pragma unroll
        for (int l = 0; l < G::kLoads; ++l) {
            const int c = l * 256 + tid;
            const int row = c >> 3, col = (c & 7) * (16 / kEs);
            const int64_t at = int64_t(row) * ld + int64_t(kb) * kBk + col;
            rp_[l] = *reinterpret_cast<const uint4*>(P + at);
            rq_[l] = *reinterpret_cast<const uint4*>(Q + at);
        }
    };
    auto lstore = [&](int buf) {
        unsigned char* lp = lds + buf * 2 * G::kOp;
        unsigned char* lq = lp + G::kOp;
#pragma unroll
        for (int l = 0; l < G::kLoads; ++l) {
            const int c = l * 256 + tid;
            const int row = c >> 3, col16 = c & 7;
            *reinterpret_cast<uint4*>(lp + row * kLdsStride + col16 * 16) = rp_[l];
            *reinterpret_cast<uint4*>(lq + row * kLdsStride + col16 * 16) = rq_[l];
        }
    };

    f32x16 acc[kNf][kNf];
#pragma unroll
    for (int i = 0; i < kNf; ++i)
#pragma unroll
        for (int j = 0; j < kNf; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int nkb = K / kBk;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
        const int cur = kb & 1;
        if (kb + 1 < nkb) gload(kb + 1);
        const unsigned char* lp = lds + cur * 2 * G::kOp;
        const unsigned char* lq = lp + G::kOp;
        // Lane (lr, hk) reads row lr of each fragment, bytes [hk*64, hk*64+64) of the
        // K block, 16 bytes per step q.  P and Q use the same K assignment, so the
        // products cover every K index of the block exactly once.
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            uint4 fa[kNf], fb[kNf];
#pragma unroll
            for (int i = 0; i < kNf; ++i)
                fa[i] = *reinterpret_cast<const uint4*>(
                    lp + (wm * G::kWt + i * 32 + lr) * kLdsStride + hk * 64 + q * 16);
#pragma unroll
            for (int j = 0; j < kNf; ++j)
                fb[j] = *reinterpret_cast<const uint4*>(
                    lq + (wn * G::kWt + j * 32 + lr) * kLdsStride + hk * 64 + q * 16);
            if constexpr (BF16) {
#pragma unroll
                for (int i = 0; i < kNf; ++i)
#pragma unroll
                    for (int j = 0; j < kNf; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, fa[i]), __builtin_bit_cast(bf16x8, fb[j]),
                            acc[i][j], 0, 0, 0);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int i = 0; i < kNf; ++i)
#pragma unroll
                        for (int j = 0; j < kNf; ++j) {
                            const uint32_t ua = e == 0 ? fa[i].x : e == 1 ? fa[i].y : e == 2 ? fa[i].z : fa[i].w;
                            const uint32_t ub = e == 0 ? fb[j].x : e == 1 ? fb[j].y : e == 2 ? fb[j].z : fb[j].w;
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                                __uint_as_float(ua), __uint_as_float(ub), acc[i][j], 0, 0, 0);
                        }
            }
        }
        if (kb + 1 < nkb) lstore(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  Lane (lr, hk) of fragment (i, j) holds, for g = 0..3, the
    // outputs at rows rbase + 0..3 (rbase = i*32 + g*8 + hk*4) and column lr.
    const float ca = args.ca, cb = args.cb, cc = args.cc;
#pragma unroll
    for (int i = 0; i < kNf; ++i) {
#pragma unroll
        for (int j = 0; j < kNf; ++j) {
            const int gj = tj * TILE + wn * G::kWt + j * 32 + lr;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int gi = ti * TILE + wm * G::kWt + i * 32 + g * 8 + hk * 4;
                float v[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = acc[i][j][g * 4 + t];
                if (STAGE == kStageA || STAGE == kStageB) {
                    TE* out = static_cast<TE*>(STAGE == kStageA ? args.ga : args.gb) + mt.g_off;
                    if (STAGE == kStageB) {
                        // A is symmetric: A[gi+t][gj] = A[gj][gi+t], 4 consecutive elements
                        float av[4];
                        load4(static_cast<const TE*>(args.ga) + mt.g_off + int64_t(gj) * rp + gi, av);
#pragma unroll
                        for (int t = 0; t < 4; ++t) v[t] = cb * av[t] + cc * v[t];
                    }
#pragma unroll
                    for (int t = 0; t < 4; ++t) store_e(out + int64_t(gi + t) * rp + gj, v[t]);
                    if (ti != tj) store4(out + int64_t(gj) * rp + gi, v);
                } else {
                    // X[gi+t][gj] = X^T[gj][gi+t]
                    float xv[4];
                    load4(static_cast<const TE*>(args.xt_cur) + mt.x_off + int64_t(gj) * rp + gi, xv);
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = ca * xv[t] + v[t];
                    if (!args.last) {
                        TE* xo = static_cast<TE*>(args.x) + mt.x_off;
#pragma unroll
                        for (int t = 0; t < 4; ++t) store_e(xo + int64_t(gi + t) * cp + gj, v[t]);
                        store4(static_cast<TE*>(args.xt_next) + mt.x_off + int64_t(gj) * rp + gi, v);
                    } else {
                        float* om = args.o + mt.off;
                        const float s = mt.scale;
                        if (!mt.tall) {
                            // O is r x c (R = r, C = c): O[gi+t][gj]
                            if (gj < mt.c) {
#pragma unroll
                                for (int t = 0; t < 4; ++t)
                                    if (gi + t < mt.r) om[int64_t(gi + t) * mt.c + gj] = s * v[t];
                            }
                        } else {
                            // O is c x r (R = c, C = r): O[gj][gi+t], 4 consecutive elements
                            if (gj < mt.c) {
                                float* dst = om + int64_t(gj) * mt.r + gi;
                                const float w4[4] = {s * v[0], s * v[1], s * v[2], s * v[3]};
                                if (gi + 3 < mt.r && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                                    store4(dst, w4);
                                } else {
#pragma unroll
                                    for (int t = 0; t < 4; ++t)
                                        if (gi + t < mt.r) dst[t] = w4[t];
                                }
                            }
                        }
                    }
                }
            }
        }
    }
}

template <int TILE, bool BF16>
hipError_t launch_stage(int stage, int n_tiles, const NsArgs& a, hipStream_t s) {
    if (n_tiles == 0) return hipSuccess;
    const dim3 grid{static_cast<unsigned>(n_tiles)}, block{256};
    switch (stage) {
        case kStageA: ns_gemm_kernel<TILE, BF16, kStageA><<<grid, block, 0, s>>>(a); break;
        case kStageB: ns_gemm_kernel<TILE, BF16, kStageB><<<grid, block, 0, s>>>(a); break;
        default: ns_gemm_kernel<TILE, BF16, kStageX><<<grid, block, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_class(int tile, int stage, int n_tiles, const NsArgs& a, hipStream_t s) {
    switch (tile) {
        case 256: return launch_stage<256, BF16>(stage, n_tiles, a, s);
        case 128: return launch_stage<128, BF16>(stage, n_tiles, a, s);
        default: return launch_stage<64, BF16>(stage, n_tiles, a, s);
    }
}

}  // namespace

hipError_t launch_newton_schulz(const PlanView& p, void* ws, float* o, int ns_steps,
                                hipStream_t s) {
    unsigned char* w = static_cast<unsigned char*>(ws);
    const bool bf16 = p.gemm_mode != MUON_GEMM_F32;
    for (int it = 0; it < ns_steps; ++it) {
        NsArgs a{};
        a.mats = p.mats;
        a.x = w + p.ws.x;
        a.xt_cur = w + p.ws.xt[it & 1];
        a.xt_next = w + p.ws.xt[(it + 1) & 1];
        a.ga = w + p.ws.a;
        a.gb = w + p.ws.b;
        a.o = o;
        a.ca = kNsA;
        a.cb = kNsB;
        a.cc = kNsC;
        a.last = it == ns_steps - 1;
        for (int stage = kStageA; stage <= kStageX; ++stage) {
            for (int c = 0; c < p.n_classes; ++c) {
                const TileClassDev& tc = p.classes[c];
                const int count = stage == kStageX ? tc.n_full : tc.n_sym;
                a.tiles = stage == kStageX ? tc.full : tc.sym;
                const hipError_t e = bf16 ? launch_class<true>(tc.tile, stage, count, a, s)
                                          : launch_class<false>(tc.tile, stage, count, a, s);
                if (e != hipSuccess) return e;
            }
        }
    }
    return hipSuccess;
}

}  // namespace muon
