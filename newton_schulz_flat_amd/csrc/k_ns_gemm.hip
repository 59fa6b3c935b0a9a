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
// (A is symmetric, so A A = A A^T, and B X = B (X^T)^T.)  The MFMA operand
// layout wants each lane to hold consecutive K values of one operand row (8
// for bf16), so operand tiles are staged in LDS as rows along K.  For P and
// for the symmetric stages those are rows of the stored matrices; stage X's
// Q = X^T is never stored: bfloat16 stage X stages K rows of X as they are and
// its fragment reads transpose them (ds_read_b64_tr_b16); float32 stage X
// transposes blocks of X in registers on their way into LDS.
//
// Symmetric stages compute only tiles with ti <= tj and mirror each
// off-diagonal tile into (tj, ti).  The axpys b A + c (.) and a X + (.) run in
// float32 in the epilogues: the bfloat16 epilogues bring their operand into
// the accumulator layout, and their results into row order, through LDS
// transposing reads; the float32 ones exchange values across lane quads.
// X ping-pongs between two buffers (workgroups of stage X still read the
// current X while others write the next one); on the last iteration stage X
// writes O = fl(s * X) in the matrix's original orientation instead, or
// applies the decay and update to the weights at once.  Iteration 0 scales its
// products by the matrix's 1 / ||U|| (the first iterate is U itself).
//
// Workgroup: 4 waves in a 2 x 2 grid over a TILE x TILE output tile (8 waves,
// 2 x 4, for the 256 x 256 bf16 tile); each wave owns its block of outputs as
// 32 x 32 MFMA fragments.  K is consumed in blocks of 128 bytes per row (64
// bf16 / 32 float32), staged through double-buffered LDS with rows padded to
// 144 bytes so that the 16-byte fragment reads of 8 consecutive rows hit
// distinct banks.  One grouped launch per stage and tile size covers every
// matrix, driven by a tile table.  The 64-tiles run in float32 in every mode;
// float32 64/128-tiles restart their accumulation chains every 1024 K blocks.
#include <type_traits>
#include <utility>

#include "k_common.h"

namespace muon {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum Stage { kStageA = 0, kStageB = 1, kStageX = 2 };

struct NsArgs {
    const MatInfo* mats;
    const GemmTile* tiles;
    const void* x_cur;  // X read by this iteration
    void* x_next;       // X written by this iteration (unused on the last)
    void* ga;       // A region
    void* gb;       // B region
    float* o;       // O (last iteration), laid out like the gradients
    float ca, cb, cc;
    int last;
    // Iteration 0 (first != 0) works on U itself: its products are scaled by
    // the matrix's inv = 1 / ||U|| (A0 = inv^2 U U^T, X1 = inv (a U + B0 U)).
    const float* inv;
    int first;
    // fused apply on the last iteration (fuse != 0): W <- fl(fl(W decay) - fl(lr O)),
    // decay and lr of the matrix's optimizer group; model_copy: bfloat16 copy of
    // float32 weights (or null)
    void* params;
    Hyper hyper;
    uint16_t* model_copy;
    int fuse, param_bf16;
    int split;  // mixed launches: table slots below split are 128-tiles, the rest 64-tiles
};

constexpr int kRowBytes = 128;  // K block: bytes of one operand row
constexpr int kLdsStride = 144;  // padded LDS row

// Workgroup geometry.  The 256 x 256 bf16 tile uses 8 waves (two per SIMD,
// each wave 128 x 64 outputs): a wave waiting on memory leaves the matrix
// pipe to its partner, and the two-per-SIMD LDS read rate is about twice
// the one-per-SIMD rate.  Smaller tiles and float32 use 4 waves (2 x 2).
template <int TILE, bool BF16>
struct Geo {
    static constexpr int kWaves = (TILE == 256 && BF16) ? 8 : 4;
    static constexpr int kThreads = kWaves * 64;
    // waves per SIMD the registers must allow: two 128-tile workgroups share a
    // CU (their LDS fits twice), so that one's epilogue overlaps the other's
    // main loop
    static constexpr int kMinWaves = TILE == 128 ? 2 : 1;
    static constexpr int kOp = TILE * kLdsStride;       // bytes of one staged operand tile
    static constexpr int kWm = TILE / 2;                 // wave tile rows
    static constexpr int kWn = TILE / (kWaves / 2);      // wave tile columns
    static constexpr int kMi = kWm / 32, kNj = kWn / 32;  // 32 x 32 fragments per wave
    static constexpr int kRowsPerPass = kThreads / 8;    // operand rows one load pass covers
    static constexpr int kLoads = TILE / kRowsPerPass;   // 16-byte loads per thread per operand
};

__device__ __forceinline__ void store4(float* p, const float v[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

// Raw (undecoded) 4-element operand vectors: loaded in batches so that one
// wave pays one memory latency per batch, not one per vector.
template <typename TE> struct Raw4;
template <> struct Raw4<uint16_t> { uint2 v; };
template <> struct Raw4<float> { float4 v; };
__device__ __forceinline__ Raw4<uint16_t> load_raw4(const uint16_t* p) {
    return {*reinterpret_cast<const uint2*>(p)};
}
__device__ __forceinline__ Raw4<float> load_raw4(const float* p) {
    return {*reinterpret_cast<const float4*>(p)};
}
__device__ __forceinline__ void decode4(const Raw4<uint16_t>& r, float v[4]) {
    v[0] = __uint_as_float(r.v.x << 16), v[1] = __uint_as_float(r.v.x & 0xffff0000u);
    v[2] = __uint_as_float(r.v.y << 16), v[3] = __uint_as_float(r.v.y & 0xffff0000u);
}
__device__ __forceinline__ void decode4(const Raw4<float>& r, float v[4]) {
    v[0] = r.v.x, v[1] = r.v.y, v[2] = r.v.z, v[3] = r.v.w;
}

// Quad transpose: lanes 4m+s (s = 0..3, same half-wave) each hold one column
// of a 4 x 4 block, v[t] = M[t][s]; afterwards lane 4m+s holds row s,
// w[t] = M[s][t].  Two DPP butterflies (xor 2, then xor 1) and a final
// lane-dependent permutation.
__device__ __forceinline__ float dpp_xor1(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ void quad_transpose(const float v[4], float w[4], int s) {
    const bool hi2 = (s & 2) != 0, hi1 = (s & 1) != 0;
    // stage 1: keep rows rb, rb+1 (rb = s & 2) of columns s and s^2
    const float y0 = dpp_xor2(hi2 ? v[0] : v[2]);
    const float y1 = dpp_xor2(hi2 ? v[1] : v[3]);
    const float c0 = hi2 ? v[2] : v[0], c1 = hi2 ? v[3] : v[1];
    // c0 = M[rb][s], c1 = M[rb+1][s], y0 = M[rb][s^2], y1 = M[rb+1][s^2]
    // stage 2: keep row s of columns s and s^2, receive columns s^1 and s^3
    const float z0 = dpp_xor1(hi1 ? c0 : c1);
    const float z1 = dpp_xor1(hi1 ? y0 : y1);
    const float k0 = hi1 ? c1 : c0, k1 = hi1 ? y1 : y0;
    // M[s][s] = k0, M[s][s^1] = z0, M[s][s^2] = k1, M[s][s^3] = z1
    const float e0 = hi1 ? z0 : k0, e1 = hi1 ? k0 : z0;  // columns (s&2), (s&2)+1
    const float e2 = hi1 ? z1 : k1, e3 = hi1 ? k1 : z1;  // columns (s&2)^2, ((s&2)^2)+1
    w[0] = hi2 ? e2 : e0;
    w[1] = hi2 ? e3 : e1;
    w[2] = hi2 ? e0 : e2;
    w[3] = hi2 ? e1 : e3;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane g points at 4 consecutive 16-bit elements of row (g >> 2) of a 4 x 16
// block, at column 4 (g & 3); it receives column g of the block, i.e. the
// elements of rows 0..3 at column g.  p points into LDS.
__device__ __forceinline__ uint2 read_tr1(const unsigned char* p) {
    return __builtin_bit_cast(
        uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(const_cast<unsigned char*>(p))));
}

// Two float32 values rounded to bfloat16 (nearest even) and packed, low first.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

// W <- fl(fl(W decay) - fl(lr O)) for elements e .. e + cnt - 1 (cnt <= 4) of a
// matrix in its own row-major order, each written to its shard slice: the
// decay-and-update of the apply phase, with the same three roundings and the
// same round-to-nearest-even store, applied where O is produced.
__device__ __forceinline__ void load_w4(const float* p, float w[4]) {
    const float4 t = *reinterpret_cast<const float4*>(p);
    w[0] = t.x, w[1] = t.y, w[2] = t.z, w[3] = t.w;
}
__device__ __forceinline__ void load_w4(const uint16_t* p, float w[4]) {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    w[0] = __uint_as_float(t.x << 16), w[1] = __uint_as_float(t.x & 0xffff0000u);
    w[2] = __uint_as_float(t.y << 16), w[3] = __uint_as_float(t.y & 0xffff0000u);
}
__device__ __forceinline__ void store_w4(float* p, const float r[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(r[0], r[1], r[2], r[3]);
}
__device__ __forceinline__ void store_w4(uint16_t* p, const float r[4]) {
    const uint32_t lo = uint32_t(bf16_rne(r[0])) | (uint32_t(bf16_rne(r[1])) << 16);
    const uint32_t hi = uint32_t(bf16_rne(r[2])) | (uint32_t(bf16_rne(r[3])) << 16);
    *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
}
__device__ __forceinline__ float load_w1(const float* p) { return *p; }
__device__ __forceinline__ float load_w1(const uint16_t* p) { return __uint_as_float(uint32_t(*p) << 16); }
__device__ __forceinline__ void store_w1(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_w1(uint16_t* p, float v) { *p = bf16_rne(v); }
// The same four elements where they are not 4-aligned (O rows whose length
// is not a multiple of 4): element accesses.
__device__ __forceinline__ Raw4<float> load_raw4_u(const float* p) { return {make_float4(p[0], p[1], p[2], p[3])}; }
__device__ __forceinline__ Raw4<uint16_t> load_raw4_u(const uint16_t* p) {
    return {make_uint2(uint32_t(p[0]) | (uint32_t(p[1]) << 16), uint32_t(p[2]) | (uint32_t(p[3]) << 16))};
}
template <typename TW>
__device__ __forceinline__ void store_w4_u(TW* p, const float r[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) store_w1(p + u, r[u]);
}

template <typename TW>
__device__ __forceinline__ void apply_span(TW* __restrict__ params, uint16_t* copy, const MatInfo& mt,
                                           int64_t e, int cnt, const float o[4], float decay, float lr) {
#pragma clang fp contract(off)
    const int64_t slice = mt.slice_len;
    const bool sharded = slice != mt.numel;
    if (cnt == 4 && (e & 3) == 0) {
        // sharded slices are multiples of 8 long: an aligned group of 4 never straddles two
        int64_t dst = mt.poff + e;
        if (sharded) {
            const int64_t k = e / slice;
            dst = mt.poff + k * mt.pstride + (e - k * slice);
        }
        float w[4], r[4];
        load_w4(params + dst, w);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float w1 = w[t] * decay;
            const float u = lr * o[t];
            r[t] = w1 - u;
        }
        store_w4(params + dst, r);
        if (copy != nullptr) store_w4(copy + dst, r);
    } else {
        // static indexing only: o[] must stay in registers
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t < cnt) {
                const int64_t j = e + t;
                const int64_t k = sharded ? j / slice : 0;
                const int64_t at = mt.poff + k * mt.pstride + (j - k * slice);
                const float w1 = load_w1(params + at) * decay;
                const float u = lr * o[t];
                const float wn = w1 - u;
                store_w1(params + at, wn);
                if (copy != nullptr) store_w1(copy + at, wn);
            }
        }
    }
}

// One staged 32-row band of O (kT 4-element chunks per lane, chunk t of lane l
// at staged row (64 t + l) / cpr, column 4 ((64 t + l) % cpr), O element
// (a0 + row, b0 + column)) applied to the weights: the weights of every
// aligned 4-element group are loaded before any is updated, so that one wave
// has all of its band's loads in flight at once; ragged groups take
// apply_span.  kU (O rows not a multiple of 4 long, unsharded matrix): every
// complete group is loaded and stored element by element, its loads still
// issued with the band's -- apply_span would wait for a store round trip per
// element, since a load issued after a store is waited for together with it.
template <int kT, int kParts, bool kU, typename TW>
__device__ __forceinline__ void apply_band(TW* __restrict__ params, uint16_t* copy, const MatInfo& mt,
                                           const float* wl, int pitch, int cpr, int a0, int b0,
                                           int rows_o, int cols_o, float decay, float lr, int lane) {
#pragma clang fp contract(off)
    const int64_t slice = mt.slice_len;
    const bool sharded = slice != mt.numel;
    // the loads of a part (the whole band, or a half where registers are short),
    // then its updates
#pragma unroll
    for (int h = 0; h < kParts; ++h) {
        constexpr int kH = kT / kParts;
        int64_t dst[kH];
        Raw4<TW> w[kH];  // undecoded
#pragma unroll
        for (int t = 0; t < kH; ++t) {
            const int ch = (h * kH + t) * 64 + lane, lrow = ch / cpr, lc = (ch % cpr) * 4;
            const int a = a0 + lrow, b = b0 + lc;
            const int64_t e = int64_t(a) * cols_o + b;
            dst[t] = -1;
            w[t] = Raw4<TW>{};
            if constexpr (kU) {
                if (a < rows_o && b + 3 < cols_o) {
                    dst[t] = mt.poff + e;
                    w[t] = load_raw4_u(params + dst[t]);
                }
            } else if (a < rows_o && b + 3 < cols_o && (e & 3) == 0) {
                // sharded slices are multiples of 8 long: an aligned group of 4 never straddles two
                int64_t d = mt.poff + e;
                if (sharded) {
                    const int64_t k = e / slice;
                    d = mt.poff + k * mt.pstride + (e - k * slice);
                }
                dst[t] = d;
                w[t] = load_raw4(params + d);
            }
        }
#pragma unroll
        for (int t = 0; t < kH; ++t) {
            const int ch = (h * kH + t) * 64 + lane, lrow = ch / cpr, lc = (ch % cpr) * 4;
            const int a = a0 + lrow, b = b0 + lc;
            if (a < rows_o && b < cols_o) {
                const float4 q = *reinterpret_cast<const float4*>(wl + lrow * pitch + lc);
                const float ov[4] = {q.x, q.y, q.z, q.w};
                if (dst[t] >= 0) {
                    float wv[4], r[4];
                    decode4(w[t], wv);
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float w1 = wv[u] * decay;
                        const float up = lr * ov[u];
                        r[u] = w1 - up;
                    }
                    if constexpr (kU) {
                        store_w4_u(params + dst[t], r);
                        if (copy != nullptr) store_w4_u(copy + dst[t], r);
                    } else {
                        store_w4(params + dst[t], r);
                        if (copy != nullptr) store_w4(copy + dst[t], r);
                    }
                } else {
                    const int cnt = b + 3 < cols_o ? 4 : cols_o - b;
                    apply_span(params, copy, mt, int64_t(a) * cols_o + b, cnt, ov, decay, lr);
                }
            }
        }
    }
}

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N - 1>{}):
// a loop whose index is a compile-time constant in every instance.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Two transposing LDS reads at p and p + second, as one 8-element MFMA operand.
__device__ __forceinline__ u32x4 read_tr(const unsigned char* p, int second) {
    const uint2 lo = __builtin_bit_cast(
        uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(const_cast<unsigned char*>(p))));
    const uint2 hi = __builtin_bit_cast(
        uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(const_cast<unsigned char*>(p + second))));
    return u32x4{lo.x, lo.y, hi.x, hi.y};
}

// LDS write number w of a thread's Q operand chunks of one K block, at dst.
// Row copies: chunk w (16 bytes of one row) goes to row pass w, `pass` bytes
// apart.  Transposed (float32 stage X): pb[l] holds 4 columns of K row l of
// the thread's block; operand row c (one column of X) takes element c of
// every pb[l], l = 0..kL-1, as kL consecutive K values.
template <bool TRANS, int kL>
__device__ __forceinline__ void store_q(unsigned char* dst, const u32x4 (&pb)[kL], int w, int pass) {
    if constexpr (!TRANS) {
        *reinterpret_cast<u32x4*>(dst + w * pass) = pb[w];
    } else {
        {
            if constexpr (kL == 8) {
                const int c = w >> 1, h = (w & 1) * 4;
                *reinterpret_cast<u32x4*>(dst + c * kLdsStride + h * 4) =
                    u32x4{pb[h][c], pb[h + 1][c], pb[h + 2][c], pb[h + 3][c]};
            } else if constexpr (kL == 4) {
                *reinterpret_cast<u32x4*>(dst + w * kLdsStride) = u32x4{pb[0][w], pb[1][w], pb[2][w], pb[3][w]};
            } else {
                *reinterpret_cast<uint2*>(dst + w * kLdsStride) = make_uint2(pb[0][w], pb[1][w]);
            }
        }
    }
}

// LDS layout of one tile size, type and stage: double-buffered operand tiles.
// How stage X stages its Q = X^T; every other operand is a copy of rows.
//  bf16: K rows of X are copied as they are (an LDS row of kS bytes holds the
//        tile's TILE columns of one K row) and the fragment reads transpose
//        them with ds_read_b64_tr_b16;
//  f32:  blocks of X are transposed in registers on their way into LDS.
template <int TILE, bool BF16, int STAGE>
struct Lds {
    using G = Geo<TILE, BF16>;
    static constexpr int kEs = BF16 ? 2 : 4;
    static constexpr int kBk = kRowBytes / kEs;  // K elements per block
    static constexpr bool kQLdsT = STAGE == kStageX && BF16;
    static constexpr bool kTransQ = STAGE == kStageX && !BF16;
    // kS = 64 (mod 256) bytes: the four K rows one transposing read gathers
    // start in distinct quarters of the 256-byte bank space
    static constexpr int kS = TILE * 2 + 64;
    static constexpr int kOpQ = (kQLdsT && kBk * kS > G::kOp) ? kBk * kS : G::kOp;
    static constexpr int kBuf = G::kOp + kOpQ;  // one stage of the double-buffered operands
    static constexpr int kBytes = 2 * kBuf;
};

// One output tile of one product (the whole work of a workgroup); lds holds
// Lds<TILE, BF16, STAGE>::kBytes bytes.
template <int TILE, bool BF16, int STAGE>
__device__ __forceinline__ void ns_gemm_tile(const NsArgs& args, const GemmTile tile,
                                             unsigned char* __restrict__ lds) {
    using TE = std::conditional_t<BF16, uint16_t, float>;
    using G = Geo<TILE, BF16>;
    using L = Lds<TILE, BF16, STAGE>;
    constexpr int kEs = L::kEs;
    constexpr int kBk = L::kBk;
    constexpr int kMi = G::kMi, kNj = G::kNj;
    constexpr int kL = G::kLoads;
    constexpr bool kQLdsT = L::kQLdsT;
    constexpr bool kTransQ = L::kTransQ;
    constexpr int kS = L::kS;
    constexpr int kBuf = L::kBuf;

    const MatInfo& mt = args.mats[tile.mat];
    const int rp = mt.rp, cp = mt.cp;
    const int ti = tile.ti, tj = tile.tj;

    // Stage X reads its Q operand transposed out of row-major X (see above).
    const TE* P;
    const TE* Q;
    int ld, K;
    if (STAGE == kStageA) {
        const TE* base = static_cast<const TE*>(args.x_cur) + mt.x_off;
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
        Q = static_cast<const TE*>(args.x_cur) + mt.x_off + int64_t(tj) * TILE;  // X[k][tj*TILE + .]
        ld = rp;
        K = rp;
    }

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int lr = lane & 31, hk = lane >> 5;

    // Global -> LDS staging of row operands: thread tid moves 16-byte chunk
    // (tid & 7) of rows (tid >> 3) + l * kRowsPerPass, l = 0..kL-1, of the
    // operand's K block.
    const int lrow = tid >> 3, lchunk = tid & 7;
    const TE* gp = P + int64_t(lrow) * ld + lchunk * (16 / kEs);
    const int64_t rstep = int64_t(G::kRowsPerPass) * ld;
    const int lds_st = lrow * kLdsStride + lchunk * 16;
    constexpr int kLdsPass = G::kRowsPerPass * kLdsStride;
    // Register-transposed staging (float32 stage X): thread tid loads K rows
    // kg*kL .. kg*kL+kL-1 of X at the 16-byte column chunk jb, i.e. a kL x kCpc
    // block, and writes it as kCpc operand rows (jb*kCpc + c) of kL elements
    // each at K offset kg*kL.  Consecutive threads take consecutive kg, so the
    // LDS writes of one wave cover whole 128-byte rows.
    constexpr int kCpc = 16 / kEs;    // elements per 16-byte chunk
    constexpr int kNkg = kBk / kL;    // K-row groups per K block
    static_assert(!kTransQ || kNkg * (TILE / kCpc) == G::kThreads, "transposed loader covers the tile");
    static_assert(!kTransQ || kL == 2 || kL == 4 || kL == 8, "transposed loader block height");
    const int kg = tid % kNkg, jb = tid / kNkg;
    // LDS writes of Q per thread and K block: one per row operand chunk, or one per
    // transposed row (two for float32 rows of 8 elements)
    constexpr int kQW = !kTransQ ? kL : kL < 8 ? kCpc : 2 * kCpc;
    // X-row staging (bf16 stage X): thread tid moves 16-byte chunk (tid % kQc) of
    // K rows tid / kQc + l * kQr of the K block.
    constexpr int kQc = TILE * kEs / 16, kQr = G::kThreads / kQc;
    static_assert(!kQLdsT || kQr * kL == kBk, "X-row loader covers the K block");
    const int qrow = tid / kQc, qch = tid % kQc;
    const TE* gq = kTransQ ? Q + int64_t(kg * kL) * cp + jb * kCpc
                   : kQLdsT ? Q + int64_t(qrow) * cp + qch * kCpc
                            : Q + int64_t(lrow) * ld + lchunk * (16 / kEs);
    // between a thread's Q loads
    const int64_t qstep = kTransQ ? int64_t(cp) : kQLdsT ? int64_t(kQr) * cp : rstep;
    const int q_st = G::kOp + (kTransQ   ? jb * kCpc * kLdsStride + kg * kL * kEs
                               : kQLdsT ? qrow * kS + qch * 16
                                        : lds_st);
    const int q_pass = kQLdsT ? kQr * kS : kLdsPass;
    // Fragment reads: row lr of each 32-row fragment, bytes [hk*64, hk*64 + 64).
    const int fa_off = (wm * G::kWm + lr) * kLdsStride + hk * 64;
    const int fb_off = G::kOp + (wn * G::kWn + lr) * kLdsStride + hk * 64;
    // Transposing reads (bf16 stage X): within each 16-lane group, lane g reads
    // 4 elements of K row (g >> 2) at column 4 (g & 3) and receives column g of
    // the 4 x 16 block; a lane thus gets 4 consecutive K values of operand row
    // lr, and two reads (K rows +0 and +4) make the 8 the MFMA takes.
    const int fbt_off = G::kOp + (hk * 32 + ((lane & 15) >> 2)) * kS +
                        (wn * G::kWn + (lane & 16) + (lane & 3) * 4) * 2;

    f32x16 acc[kMi][kNj];
#pragma unroll
    for (int i = 0; i < kMi; ++i)
#pragma unroll
        for (int j = 0; j < kNj; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // Main loop.  A K block is consumed in four steps q of 16 bf16 (4 float32)
    // per lane; its instruction order is fixed with scheduling barriers so
    // that each MFMA is followed by at most a few memory instructions:
    //   q = 0, 1, 2: fragments of step q+1 are read from LDS (double-buffered
    //                registers); after step 2 all waves meet at the barrier,
    //                after which this block's LDS buffer is free;
    //   q = 3:       the MFMAs run on fragments already in registers while the
    //                fragments of step 0 of the next block are read.
    // Staging: each step writes one share of the staged registers into LDS --
    // step 3 into the freed buffer (block kb + 2), steps 0-2 into the other one
    // (completing block kb + 1 before the barrier) -- and reloads those
    // registers right away, so a global load has one whole K block to arrive
    // and the LDS writes and loads are spread evenly over the steps.  Step 3's
    // MFMAs give the matrix pipe work while every wave refills its fragments.
    // Blocks past the end reload the last block (valid, unused copies) so the
    // loop stays branch free.
    const int nkb = K / kBk;
    constexpr int kMfma = kMi * kNj;  // MFMAs per step q (per K sub-step for bf16)
    // float32 products with long contractions: every kFlushBlocks K blocks the
    // accumulators are added, in order, into this tile's own float32 output
    // region (written by no other workgroup of the launch and read by none) and
    // restarted, so that no accumulation chain runs over more than
    // kFlushBlocks * 32 products -- one float32 chain over 2^20 positive terms
    // drifts by ~5e-4 relative.  The epilogue later overwrites the region.
    // 64- and 128-tiles only: the plan gives float32 256-tiles contractions of
    // at most kFlushBlocks * 32 (their 256 accumulators leave no registers for
    // this path).
    constexpr int kFlushBlocks = 1024;
    constexpr bool kFlush = !BF16 && TILE < 256;
    float* sbase = nullptr;
    int sld = 0;
    if constexpr (kFlush) {
        if (STAGE == kStageX) {
            sbase = static_cast<float*>(args.x_next) + mt.x_off;
            sld = cp;
        } else {
            sbase = static_cast<float*>(STAGE == kStageA ? args.ga : args.gb) + mt.g_off;
            sld = rp;
        }
    }
    const int srow0 = ti * TILE + wm * G::kWm + hk * 4, scol0 = tj * TILE + wn * G::kWn + lr;
    // partial sums: first flush stores, later ones add (earlier segments first);
    // fold == true adds the stored sum into the accumulators instead
    auto flush = [&](bool first, bool fold) {
        // opaque copies: keeps the address arithmetic on this rare path instead
        // of hoisted (and held in registers) across the main loop
        int ld_f = sld, row_f = srow0, col_f = scol0;
        asm volatile("" : "+s"(ld_f));
        asm volatile("" : "+v"(row_f), "+v"(col_f));
        float* const b0 = sbase + int64_t(row_f) * ld_f + col_f;
#pragma unroll
        for (int i = 0; i < kMi; ++i)
#pragma unroll
            for (int j = 0; j < kNj; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float* sp = b0 + int64_t(i * 32 + (e >> 2) * 8 + (e & 3)) * ld_f + j * 32;
                    if (fold) {
                        acc[i][j][e] = *sp + acc[i][j][e];
                    } else {
                        *sp = first ? acc[i][j][e] : *sp + acc[i][j][e];
                        acc[i][j][e] = 0.f;
                    }
                    // one fragment's values in flight at a time
                    if ((e & 15) == 15) asm volatile("" ::: "memory");
                }
    };
    auto q_off = [&](int blk) -> int64_t {
        return (kTransQ || kQLdsT) ? int64_t(blk) * kBk * cp : int64_t(blk) * kBk;
    };
    // Staged register pair l (pa[l], pb[l]) is written to LDS and reloaded at
    // step (3 + l / kPerStep) mod 4, so that every step carries the same share of
    // LDS writes and global loads.  (The register-transposed Q of float32 stage X
    // reads every pb in each write: there all pairs are handled at step 3.)
    constexpr int kPerStep = kTransQ ? kL : (kL + 3) / 4;
    u32x4 pa[kL], pb[kL];
    {
        // block 0 into LDS buffer 0; block 1 into buffer 1 for the pairs handled
        // at step 3 (those are reloaded with block 2), the rest stay in registers
        // and are written during steps 0-2 of block 0
        u32x4 pa1[kL], pb1[kL];
        const int b1 = nkb > 1 ? 1 : 0, b2 = nkb > 2 ? 2 : nkb - 1;
#pragma unroll
        for (int l = 0; l < kL; ++l) {
            pa1[l] = *reinterpret_cast<const u32x4*>(gp + l * rstep);
            pb1[l] = *reinterpret_cast<const u32x4*>(gq + l * qstep);
        }
#pragma unroll
        for (int l = 0; l < kL; ++l) {
            pa[l] = *reinterpret_cast<const u32x4*>(gp + l * rstep + int64_t(b1) * kBk);
            pb[l] = *reinterpret_cast<const u32x4*>(gq + l * qstep + q_off(b1));
        }
#pragma unroll
        for (int l = 0; l < kL; ++l) *reinterpret_cast<u32x4*>(lds + lds_st + l * kLdsPass) = pa1[l];
#pragma unroll
        for (int w = 0; w < kQW; ++w) store_q<kTransQ, kL>(lds + q_st, pb1, w, q_pass);
        if constexpr (kTransQ) {
#pragma unroll
            for (int l = 0; l < kL; ++l) *reinterpret_cast<u32x4*>(lds + kBuf + lds_st + l * kLdsPass) = pa[l];
#pragma unroll
            for (int w = 0; w < kQW; ++w) store_q<kTransQ, kL>(lds + kBuf + q_st, pb, w, q_pass);
#pragma unroll
            for (int l = 0; l < kL; ++l) {
                pa[l] = *reinterpret_cast<const u32x4*>(gp + l * rstep + int64_t(b2) * kBk);
                pb[l] = *reinterpret_cast<const u32x4*>(gq + l * qstep + q_off(b2));
            }
        } else {
#pragma unroll
            for (int l = 0; l < kPerStep && l < kL; ++l) {
                *reinterpret_cast<u32x4*>(lds + kBuf + lds_st + l * kLdsPass) = pa[l];
                *reinterpret_cast<u32x4*>(lds + kBuf + q_st + l * q_pass) = pb[l];
                pa[l] = *reinterpret_cast<const u32x4*>(gp + l * rstep + int64_t(b2) * kBk);
                pb[l] = *reinterpret_cast<const u32x4*>(gq + l * qstep + q_off(b2));
            }
        }
    }
    __syncthreads();

    u32x4 fa[2][kMi], fb[2][kNj];
#pragma unroll
    for (int i = 0; i < kMi; ++i)
        fa[0][i] = *reinterpret_cast<const u32x4*>(lds + fa_off + i * 32 * kLdsStride);
#pragma unroll
    for (int j = 0; j < kNj; ++j)
        fb[0][j] = kQLdsT ? read_tr(lds + fbt_off + j * 64, 4 * kS)
                          : *reinterpret_cast<const u32x4*>(lds + fb_off + j * 32 * kLdsStride);
    for (int kb = 0; kb < nkb; ++kb) {
        // steps 0-2 complete block kb + 1 in the other buffer and load block kb + 2;
        // step 3 starts block kb + 2 in this (now free) buffer and loads block kb + 3
        const int b2 = kb + 2 < nkb ? kb + 2 : nkb - 1;
        const int b3 = kb + 3 < nkb ? kb + 3 : nkb - 1;
        const int64_t k2 = int64_t(b2) * kBk, qk2 = q_off(b2);
        const int64_t k3 = int64_t(b3) * kBk, qk3 = q_off(b3);
        unsigned char* buf = lds + (kb & 1) * kBuf;
        unsigned char* nbuf = lds + ((kb + 1) & 1) * kBuf;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int cur = q & 1;
            const unsigned char* rbuf = q < 3 ? buf : nbuf;
            const int rq = q < 3 ? q + 1 : 0;
            unsigned char* wbuf = q == 3 ? buf : nbuf;
            const int64_t kk = q == 3 ? k3 : k2, qkk = q == 3 ? qk3 : qk2;
            const int l0 = ((q + 1) & 3) * kPerStep;  // first pair of this step
            // Step 3 (after the barrier) runs at raised wave priority, so that a
            // wave already in the next block's step 0 yields issue slots to its
            // partner on the SIMD still in step 3 (measured: llama layer about
            // 1% faster, owner share unchanged).
            if constexpr (BF16 && TILE == 256) {
                if (q == 3) __builtin_amdgcn_s_setprio(1);
            }
#pragma unroll
            for (int m = 0; m < kMfma; ++m) {
                const int i = m / kNj, j = m % kNj;
                if constexpr (BF16) {
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, fa[cur][i]), __builtin_bit_cast(bf16x8, fb[cur][j]),
                        acc[i][j], 0, 0, 0);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            __uint_as_float(fa[cur][i][e]), __uint_as_float(fb[cur][j][e]), acc[i][j],
                            0, 0, 0);
                }
#pragma unroll
                for (int rd = m; rd < kMi + kNj; rd += kMfma) {
                    if (rd < kMi)
                        fa[cur ^ 1][rd] = *reinterpret_cast<const u32x4*>(
                            rbuf + fa_off + rd * 32 * kLdsStride + rq * 16);
                    else if (kQLdsT)
                        fb[cur ^ 1][rd - kMi] =
                            read_tr(rbuf + fbt_off + (rd - kMi) * 64 + rq * 8 * kS, 4 * kS);
                    else
                        fb[cur ^ 1][rd - kMi] = *reinterpret_cast<const u32x4*>(
                            rbuf + fb_off + (rd - kMi) * 32 * kLdsStride + rq * 16);
                }
                if constexpr (kTransQ) {
                    if (q == 3) {
                        // this block's buffer is free: block kb + 2 goes in, then block kb + 3
                        // is loaded (pa right after its write; pb after all writes, below)
#pragma unroll
                        for (int l = m; l < kL + kQW; l += kMfma) {
                            if (l < kL)
                                *reinterpret_cast<u32x4*>(buf + lds_st + l * kLdsPass) = pa[l];
                            else
                                store_q<kTransQ, kL>(buf + q_st, pb, l - kL, q_pass);
                        }
#pragma unroll
                        for (int l = m; l < kL; l += kMfma)
                            pa[l] = *reinterpret_cast<const u32x4*>(gp + l * rstep + k3);
                    }
                } else {
                    // this step's pairs: writes first, then the reloads
#pragma unroll
                    for (int it = m; it < 4 * kPerStep; it += kMfma) {
                        const int l = l0 + (it % (2 * kPerStep)) / 2;
                        const bool is_q = (it & 1) != 0;
                        if (l < kL) {
                            if (it < 2 * kPerStep) {
                                if (is_q)
                                    *reinterpret_cast<u32x4*>(wbuf + q_st + l * q_pass) = pb[l];
                                else
                                    *reinterpret_cast<u32x4*>(wbuf + lds_st + l * kLdsPass) = pa[l];
                            } else {
                                if (is_q)
                                    pb[l] = *reinterpret_cast<const u32x4*>(gq + l * qstep + qkk);
                                else
                                    pa[l] = *reinterpret_cast<const u32x4*>(gp + l * rstep + kk);
                            }
                        }
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (kTransQ && q == 3) {
#pragma unroll
                for (int l = 0; l < kL; ++l)
                    pb[l] = *reinterpret_cast<const u32x4*>(gq + l * qstep + qk3);
            }
            if constexpr (BF16 && TILE == 256) {
                if (q == 3) __builtin_amdgcn_s_setprio(0);
            }
            if (q == 2) __syncthreads();
        }
        if constexpr (kFlush) {
            if ((kb + 1) % kFlushBlocks == 0 && kb + 1 < nkb) flush(kb + 1 == kFlushBlocks, false);
        }
    }
    if constexpr (kFlush) {
        if (nkb > kFlushBlocks) flush(false, true);
    }
    // the last step read (unused) fragments: let every wave finish with LDS
    // before the epilogue reuses it
    __syncthreads();

    // Epilogue.  Lane (lr, hk) of fragment (i, j) holds, for g = 0..3, the
    // outputs at rows gi + 0..3 (gi = wave row + i*32 + g*8 + hk*4) of column gj
    // (column layout).  Column-oriented stores take those 4 values as one
    // vector; the row layout comes from exchanging them across the lane quad,
    // after which lane s of the quad holds row gi + s, columns gj - s .. gj - s + 3.
    // Stage X works in the row layout throughout, so that its operand X is read
    // along rows.
    const int s4 = lr & 3;
    const int row0 = ti * TILE + wm * G::kWm + hk * 4;
    const int col0 = tj * TILE + wn * G::kWn + lr;
    const float ca = args.ca, cb = args.cb, cc = args.cc;
    // iteration-0 normalization (exactly 1 afterwards)
    const float inv0 = args.first ? args.inv[tile.mat] : 1.f;
    const float sa = STAGE == kStageA ? inv0 * inv0 : 1.f;  // stage A: A0 = inv^2 U U^T
    const float xs = inv0;                                  // stage X: X1 = inv (a U + B0 U)
    const TE* xc = static_cast<const TE*>(args.x_cur) + mt.x_off;
    // X (row layout) at fragment (i, j), group g
    auto x_row = [&](int i, int j, int g) {
        return xc + int64_t(row0 + i * 32 + g * 8 + s4) * cp + (col0 + j * 32 - s4);
    };
    if (STAGE != kStageX || !args.last) {
        TE* out_n;  // row-oriented destination, leading dimension ld_n
        int ld_n;
        if (STAGE == kStageX) {
            out_n = static_cast<TE*>(args.x_next) + mt.x_off;
            ld_n = cp;
        } else {
            out_n = static_cast<TE*>(STAGE == kStageA ? args.ga : args.gb) + mt.g_off;
            ld_n = rp;
        }
        TE* const out_t = out_n;  // mirror (symmetric stages), leading dimension rp
        const bool write_t = STAGE != kStageX && ti != tj;
        // stage-B operand A, read along a column (A is symmetric)
        const TE* ga = static_cast<const TE*>(args.ga) + mt.g_off;
        if constexpr (BF16) {
            // bfloat16 tiles go through a wave-private LDS region in three passes,
            // so that every global access is a 16-byte run along a row:
            //  1. (stages B, X) the operand sub-tile is loaded along its rows and
            //     staged row-major; transposing reads then hand each lane the 4
            //     rows x 1 column it holds in the accumulators;
            //  2. the rounded results are staged column-major (staged row = output
            //     column), which a mirrored tile stores as it is;
            //  3. transposing reads of the column-major staging return output rows
            //     for the row-oriented stores.
            // The main loop ended with a barrier, so LDS is free.
            constexpr int kWm = G::kWm, kWn = G::kWn;
            constexpr int kStrideT = kWm * 2 + 16;  // column-major staging: kWn rows of kWm
            constexpr int kStrideO = kWn * 2 + 16;  // operand staging: kWm rows of kWn
            constexpr int kRegion = (kWn * kStrideT > kWm * kStrideO) ? kWn * kStrideT : kWm * kStrideO;
            static_assert(kRegion * G::kWaves <= 2 * kBuf, "epilogue staging exceeds LDS");
            unsigned char* wl = lds + wave * kRegion;
            const int r0w = ti * TILE + wm * kWm, c0w = tj * TILE + wn * kWn;  // wave sub-tile origin
            // transposing-read lane geometry (see read_tr): row (g >> 2), column 4 (g & 3)
            const int tr_r = (lane & 15) >> 2, tr_c = (lane & 3) * 4;
            uint32_t pk[kMi][kNj][4][2];
            if (STAGE != kStageA) {
                const int old = STAGE == kStageB ? rp : cp;
                const TE* src = (STAGE == kStageB ? ga + int64_t(r0w) * rp : xc + int64_t(r0w) * cp) + c0w;
                constexpr int kCpr = kWn / 8;             // 16-byte chunks per operand row
                constexpr int kChunks = kWm * kCpr / 64;  // per lane
                u32x4 ov[kChunks];
#pragma unroll
                for (int t = 0; t < kChunks; ++t) {
                    const int ch = t * 64 + lane, r = ch / kCpr, c16 = ch % kCpr;
                    ov[t] = *reinterpret_cast<const u32x4*>(src + int64_t(r) * old + c16 * 8);
                }
#pragma unroll
                for (int t = 0; t < kChunks; ++t) {
                    const int ch = t * 64 + lane, r = ch / kCpr, c16 = ch % kCpr;
                    *reinterpret_cast<u32x4*>(wl + r * kStrideO + c16 * 16) = ov[t];
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
                for (int i = 0; i < kMi; ++i)
#pragma unroll
                    for (int j = 0; j < kNj; ++j)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            // rows i*32 + g*8 + hk*4 + 0..3, column j*32 + lr of the sub-tile
                            const uint2 x2 = read_tr1(wl + (i * 32 + g * 8 + hk * 4 + tr_r) * kStrideO +
                                                      (j * 32 + (lane & 16) + tr_c) * 2);
                            float ov4[4] = {__uint_as_float(x2.x << 16), __uint_as_float(x2.x & 0xffff0000u),
                                            __uint_as_float(x2.y << 16), __uint_as_float(x2.y & 0xffff0000u)};
                            float v[4];
#pragma unroll
                            for (int t = 0; t < 4; ++t)
                                v[t] = STAGE == kStageB ? cb * ov4[t] + cc * acc[i][j][g * 4 + t]
                                                        : xs * (ca * ov4[t] + acc[i][j][g * 4 + t]);
                            pk[i][j][g][0] = pack_bf16(v[0], v[1]);
                            pk[i][j][g][1] = pack_bf16(v[2], v[3]);
                        }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            } else {
#pragma unroll
                for (int i = 0; i < kMi; ++i)
#pragma unroll
                    for (int j = 0; j < kNj; ++j)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            pk[i][j][g][0] = pack_bf16(sa * acc[i][j][g * 4 + 0], sa * acc[i][j][g * 4 + 1]);
                            pk[i][j][g][1] = pack_bf16(sa * acc[i][j][g * 4 + 2], sa * acc[i][j][g * 4 + 3]);
                        }
            }
            // column-major staging: staged row = output column j*32 + lr, 4 rows per lane
#pragma unroll
            for (int i = 0; i < kMi; ++i)
#pragma unroll
                for (int j = 0; j < kNj; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int sr = j * 32 + lr, sc = i * 32 + g * 8 + hk * 4;
                        *reinterpret_cast<uint2*>(wl + sr * kStrideT + sc * 2) =
                            make_uint2(pk[i][j][g][0], pk[i][j][g][1]);
                    }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (write_t) {
                // mirror tile: staged row c -> global row c0w + c of out_t, columns r0w ..
                constexpr int cpr = kWm / 8;
#pragma unroll 4
                for (int t = 0; t < kWn * cpr / 64; ++t) {
                    const int ch = t * 64 + lane, r = ch / cpr, c16 = ch % cpr;
                    const u32x4 val = *reinterpret_cast<const u32x4*>(wl + r * kStrideT + c16 * 16);
                    *reinterpret_cast<u32x4*>(out_t + int64_t(c0w + r) * rp + r0w + c16 * 8) = val;
                }
            }
            // row-oriented stores: per pass, 16-lane group G takes output rows
            // rb + 0..15 (lane g: row rb + g) and columns cb + 8G .. cb + 8G + 7,
            // read as staged rows cb + 8G + 0..3 and + 4..7 at staged column rb + 4 (g & 3)
#pragma unroll 4
            for (int t = 0; t < (kWm / 16) * (kWn / 32); ++t) {
                const int rb = (t % (kWm / 16)) * 16, cb = (t / (kWm / 16)) * 32 + (lane >> 4) * 8;
                const unsigned char* p = wl + (cb + tr_r) * kStrideT + (rb + tr_c) * 2;
                const u32x4 val = read_tr(p, 4 * kStrideT);
                *reinterpret_cast<u32x4*>(out_n + int64_t(r0w + rb + (lane & 15)) * ld_n + c0w + cb) = val;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kMi; ++i) {
                Raw4<TE> raw[kNj][4];
                if (STAGE != kStageA) {
#pragma unroll
                    for (int j = 0; j < kNj; ++j)
#pragma unroll
                        for (int g = 0; g < 4; ++g)
                            raw[j][g] = STAGE == kStageX
                                            ? load_raw4(x_row(i, j, g))
                                            : load_raw4(ga + int64_t(col0 + j * 32) * rp + row0 + i * 32 + g * 8);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < kNj; ++j) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int gi = row0 + i * 32 + g * 8;
                        const int gj = col0 + j * 32;
                        float v[4], w[4], ov[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) v[t] = sa * acc[i][j][g * 4 + t];
                        if (STAGE == kStageX) {
                            quad_transpose(v, w, s4);
                            decode4(raw[j][g], ov);
#pragma unroll
                            for (int t = 0; t < 4; ++t) w[t] = xs * (ca * ov[t] + w[t]);
                        } else {
                            if (STAGE == kStageB) {
                                decode4(raw[j][g], ov);
#pragma unroll
                                for (int t = 0; t < 4; ++t) v[t] = cb * ov[t] + cc * v[t];
                            }
                            if (write_t) store4(out_t + int64_t(gj) * rp + gi, v);
                            quad_transpose(v, w, s4);
                        }
                        store4(out_n + int64_t(gi + s4) * ld_n + (gj - s4), w);
                    }
                }
            }
        }
    } else {
        // Last iteration: O = fl(s * (a X + B X)) in the matrix's own R x C layout,
        // stored, or (fused apply) used at once to update the weights.  Each
        // 32-row band of the wave's sub-tile is staged in a wave-private LDS region
        // in O's own orientation, then written out along O's rows.
        float* om = args.fuse ? nullptr : args.o + mt.off;  // O is not stored when fused
        const float sc = mt.scale;
        const int r = mt.r, c = mt.c;
        const bool tall = mt.tall != 0;
        const int rows_o = tall ? c : r, cols_o = tall ? r : c;  // O's shape
        const HyperVals hv = hyper_for(args.hyper, mt);
        constexpr int kWn = G::kWn;
        constexpr int kPN = kWn + 4;  // float pitch, wide: 32 O rows of kWn
        constexpr int kPT = 32 + 4;   // float pitch, tall: kWn O rows of 32
        constexpr int kRegionL = (32 * kPN > kWn * kPT ? 32 * kPN : kWn * kPT) * 4;
        static_assert(kRegionL * G::kWaves <= 2 * kBuf, "epilogue staging exceeds LDS");
        float* wl = reinterpret_cast<float*>(lds + wave * kRegionL);
        const int r0w = ti * TILE + wm * G::kWm, c0w = tj * TILE + wn * kWn;
        constexpr int kT = 32 * kWn / 4 / 64;  // 4-element chunks per lane and band
        // the band loop once per output kind (weights of type TW, or O), so that
        // each instance unrolls fully and the accumulators keep static indices
        auto bands = [&](auto* params, uint16_t* copy, auto fuse_tag, auto u_tag) {
            constexpr bool kFuse = decltype(fuse_tag)::value;
            constexpr bool kU = decltype(u_tag)::value;
            // X rows of band 0; band i + 1 is loaded while band i is written out
            Raw4<TE> raw[kNj][4];
#pragma unroll
            for (int j = 0; j < kNj; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) raw[j][g] = load_raw4(x_row(0, j, g));
            static_for<kMi>([&](auto i_tag) {
                constexpr int i = decltype(i_tag)::value;
                __builtin_amdgcn_sched_barrier(0);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // previous band read back
#pragma unroll
                for (int j = 0; j < kNj; ++j) {
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        float v[4], xv[4], w[4];
                        decode4(raw[j][g], xv);  // row layout
                        if (tall) {
                            // O[gj][gi + t] = X[gi + t][gj]: the column layout, 4 consecutive O elements
                            float xcol[4];
                            quad_transpose(xv, xcol, s4);
#pragma unroll
                            for (int t = 0; t < 4; ++t)
                                v[t] = sc * (xs * (ca * xcol[t] + acc[i][j][g * 4 + t]));
                            *reinterpret_cast<float4*>(wl + (j * 32 + lr) * kPT + g * 8 + (lane >> 5) * 4) =
                                make_float4(v[0], v[1], v[2], v[3]);
                        } else {
                            // O[gi + s][gj - s + t]: the row layout after the quad exchange
#pragma unroll
                            for (int t = 0; t < 4; ++t) v[t] = acc[i][j][g * 4 + t];
                            quad_transpose(v, w, s4);
#pragma unroll
                            for (int t = 0; t < 4; ++t) w[t] = sc * (xs * (ca * xv[t] + w[t]));
                            *reinterpret_cast<float4*>(wl + (g * 8 + (lane >> 5) * 4 + s4) * kPN + j * 32 +
                                                       lr - s4) = make_float4(w[0], w[1], w[2], w[3]);
                        }
                    }
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                if constexpr (i + 1 < kMi) {
#pragma unroll
                    for (int j = 0; j < kNj; ++j)
#pragma unroll
                        for (int g = 0; g < 4; ++g) raw[j][g] = load_raw4(x_row(i + 1, j, g));
                }
                // the band is 32 x kWn (wide) or kWn x 32 (tall) O elements; 4 per lane per pass
                const int cpr = tall ? 8 : kWn / 4;  // 4-element chunks per staged row
                const int pitch = tall ? kPT : kPN;
                const int a0 = tall ? c0w : r0w + i * 32, b0 = tall ? r0w + i * 32 : c0w;
                if constexpr (kFuse) {
                    // whole bands in the 64/128-tile kernels and for bfloat16 weights in
                    // the bfloat16 kernels; halves of float32 bands in the 256-tile ones
                    // (their registers)
                    constexpr int kParts =
                        (TILE < 256 || (BF16 && sizeof(std::remove_pointer_t<decltype(params)>) == 2)) ? 1 : 2;
                    apply_band<kT, kParts, kU>(params, copy, mt, wl, pitch, cpr, a0, b0, rows_o, cols_o,
                                               hv.decay, hv.lr, lane);
                } else {
#pragma unroll
                    for (int t = 0; t < kT; ++t) {
                        const int ch = t * 64 + lane, lrow = ch / cpr, lc = (ch % cpr) * 4;
                        const int a = a0 + lrow, b = b0 + lc;
                        if (a < rows_o && b < cols_o) {
                            const float4 q = *reinterpret_cast<const float4*>(wl + lrow * pitch + lc);
                            const float ov[4] = {q.x, q.y, q.z, q.w};
                            const int cnt = b + 3 < cols_o ? 4 : cols_o - b;
                            const int64_t e = int64_t(a) * cols_o + b;
                            if (cnt == 4 && (e & 3) == 0) {
                                store4(om + e, ov);
                            } else {
#pragma unroll
                                for (int u = 0; u < 4; ++u)
                                    if (u < cnt) om[e + u] = ov[u];
                            }
                        }
                    }
                }
            });
        };
        // O rows whose length is not a multiple of 4 (unsharded matrices only:
        // sharded slices may start inside a group) update element by element in
        // the 64/128-tile kernels.  The 256-tile kernels keep the aligned path
        // alone: the second instance costs their other paths registers (spills),
        // and they take the rows of 513..1024-long sides, where the per-element
        // round trips are a smaller share of a tile's time.
        const bool unaligned = TILE < 256 && (cols_o & 3) != 0 && mt.slice_len == mt.numel;
        if (!args.fuse) {
            bands(static_cast<float*>(nullptr), nullptr, std::false_type{}, std::false_type{});
        } else if (!unaligned) {
            if (args.param_bf16)
                bands(static_cast<uint16_t*>(args.params), nullptr, std::true_type{}, std::false_type{});
            else
                bands(static_cast<float*>(args.params), args.model_copy, std::true_type{}, std::false_type{});
        } else if constexpr (TILE < 256) {
            if (args.param_bf16)
                bands(static_cast<uint16_t*>(args.params), nullptr, std::true_type{}, std::true_type{});
            else
                bands(static_cast<float*>(args.params), args.model_copy, std::true_type{}, std::true_type{});
        }
    }
}

template <int TILE, bool BF16, int STAGE>
__global__ __launch_bounds__((Geo<TILE, BF16>::kThreads), (Geo<TILE, BF16>::kMinWaves)) void ns_gemm_kernel(
    NsArgs args) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[Lds<TILE, BF16, STAGE>::kBytes];
    const GemmTile tile = args.tiles[blockIdx.x];
    if (tile.mat < 0) return;  // padding slot of the XCD-interleaved table
    ns_gemm_tile<TILE, BF16, STAGE>(args, tile, lds);
}

// The 128-tile and 64-tile classes of one stage in one launch: table slots
// [0, split) hold 128-tiles (bfloat16 or float32 products), the rest 64-tiles
// (float32).  Both take 4 waves and fit two workgroups per CU, so the small
// 64-tiles fill the CUs the 128-tiles leave idle instead of waiting for a
// launch of their own.
template <bool BF16, int STAGE>
__global__ __launch_bounds__(256, 2) void ns_gemm_mixed_kernel(NsArgs args) {
    static_assert(Geo<128, BF16>::kThreads == 256 && Geo<64, false>::kThreads == 256, "block size");
    constexpr int kA = Lds<128, BF16, STAGE>::kBytes, kB = Lds<64, false, STAGE>::kBytes;
    __shared__ __attribute__((aligned(16))) unsigned char lds[kA > kB ? kA : kB];
    const GemmTile tile = args.tiles[blockIdx.x];
    if (tile.mat < 0) return;  // padding slot of an XCD-interleaved table
    if (int(blockIdx.x) < args.split)
        ns_gemm_tile<128, BF16, STAGE>(args, tile, lds);
    else
        ns_gemm_tile<64, false, STAGE>(args, tile, lds);
}

template <int TILE, bool BF16>
const char* stage_name(int stage) {
    static const char* const names[3] = {
        TILE == 256 ? (BF16 ? "ns_a_t256_bf16" : "ns_a_t256_f32")
                    : TILE == 128 ? (BF16 ? "ns_a_t128_bf16" : "ns_a_t128_f32")
                                  : (BF16 ? "ns_a_t64_bf16" : "ns_a_t64_f32"),
        TILE == 256 ? (BF16 ? "ns_b_t256_bf16" : "ns_b_t256_f32")
                    : TILE == 128 ? (BF16 ? "ns_b_t128_bf16" : "ns_b_t128_f32")
                                  : (BF16 ? "ns_b_t64_bf16" : "ns_b_t64_f32"),
        TILE == 256 ? (BF16 ? "ns_x_t256_bf16" : "ns_x_t256_f32")
                    : TILE == 128 ? (BF16 ? "ns_x_t128_bf16" : "ns_x_t128_f32")
                                  : (BF16 ? "ns_x_t64_bf16" : "ns_x_t64_f32")};
    return names[stage];
}

template <int TILE, bool BF16>
hipError_t launch_stage(int stage, int n_tiles, const NsArgs& a, hipStream_t s) {
    if (n_tiles == 0) return hipSuccess;
    LaunchTimer timer(stage_name<TILE, BF16>(stage), s);
    const dim3 grid{static_cast<unsigned>(n_tiles)}, block{unsigned(Geo<TILE, BF16>::kThreads)};
    switch (stage) {
        case kStageA: ns_gemm_kernel<TILE, BF16, kStageA><<<grid, block, 0, s>>>(a); break;
        case kStageB: ns_gemm_kernel<TILE, BF16, kStageB><<<grid, block, 0, s>>>(a); break;
        default: ns_gemm_kernel<TILE, BF16, kStageX><<<grid, block, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_mixed(int stage, int n_tiles, const NsArgs& a, hipStream_t s) {
    static const char* const names[2][3] = {
        {"ns_a_t128+64_f32", "ns_b_t128+64_f32", "ns_x_t128+64_f32"},
        {"ns_a_t128+64_bf16", "ns_b_t128+64_bf16", "ns_x_t128+64_bf16"}};
    LaunchTimer timer(names[BF16 ? 1 : 0][stage], s);
    const dim3 grid{static_cast<unsigned>(n_tiles)}, block{256u};
    switch (stage) {
        case kStageA: ns_gemm_mixed_kernel<BF16, kStageA><<<grid, block, 0, s>>>(a); break;
        case kStageB: ns_gemm_mixed_kernel<BF16, kStageB><<<grid, block, 0, s>>>(a); break;
        default: ns_gemm_mixed_kernel<BF16, kStageX><<<grid, block, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_class(int tile, int stage, int n_tiles, const NsArgs& a, hipStream_t s) {
    switch (tile) {
        case 256: return launch_stage<256, BF16>(stage, n_tiles, a, s);
        case 128: return launch_stage<128, BF16>(stage, n_tiles, a, s);
        default:
            // 64-tiles run in float32 in every mode (kF32NsTile)
            if constexpr (BF16) return hipErrorInvalidValue;
            else return launch_stage<64, false>(stage, n_tiles, a, s);
    }
}

}  // namespace

hipError_t launch_newton_schulz(const PlanView& p, void* ws, float* o, const FusedApply* fuse,
                                int ns_steps, hipStream_t s) {
    unsigned char* w = static_cast<unsigned char*>(ws);
    const bool bf16 = p.gemm_mode != MUON_GEMM_F32;
    for (int it = 0; it < ns_steps; ++it) {
        NsArgs a{};
        a.mats = p.mats;
        a.x_cur = w + p.ws.x[it & 1];
        a.x_next = w + p.ws.x[(it + 1) & 1];
        a.ga = w + p.ws.a;
        a.gb = w + p.ws.b;
        a.o = o;
        a.ca = kNsA;
        a.cb = kNsB;
        a.cc = kNsC;
        a.last = it == ns_steps - 1;
        a.first = it == 0;
        a.inv = reinterpret_cast<const float*>(w + p.ws.inv);
        if (fuse && a.last) {
            a.params = fuse->params;
            a.hyper = fuse->hyper;
            a.model_copy = fuse->model_copy;
            a.fuse = 1;
            a.param_bf16 = fuse->param_dtype == MUON_DTYPE_BF16;
        }
        for (int stage = kStageA; stage <= kStageX; ++stage) {
            auto count_of = [&](const TileClassDev& tc) {
                return stage == kStageX ? tc.n_full : stage == kStageA ? tc.n_sym_a : tc.n_sym_b;
            };
            auto table_of = [&](const TileClassDev& tc) {
                return stage == kStageX ? tc.full : stage == kStageA ? tc.sym_a : tc.sym_b;
            };
            // the 128- and 64-tile classes share one launch when both have tiles
            // (the plan keeps a stage's class tables contiguous)
            const TileClassDev& t128 = p.classes[1];
            const TileClassDev& t64 = p.classes[2];
            const bool mixed = count_of(t128) > 0 && count_of(t64) > 0 &&
                               table_of(t128) + count_of(t128) == table_of(t64);
            for (int c = 0; c < p.n_classes; ++c) {
                const TileClassDev& tc = p.classes[c];
                const int count = count_of(tc);
                a.tiles = table_of(tc);
                const bool cls_bf16 = bf16 && tc.tile != kF32NsTile;
                hipError_t e;
                if (mixed && c == 1) {
                    a.split = count;
                    e = bf16 ? launch_mixed<true>(stage, count + count_of(t64), a, s)
                             : launch_mixed<false>(stage, count + count_of(t64), a, s);
                } else if (mixed && c == 2) {
                    continue;
                } else {
                    e = cls_bf16 ? launch_class<true>(tc.tile, stage, count, a, s)
                                 : launch_class<false>(tc.tile, stage, count, a, s);
                }
                if (e != hipSuccess) return e;
            }
        }
    }
    return hipSuccess;
}

}  // namespace muon
