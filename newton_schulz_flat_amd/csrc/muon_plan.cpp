// Launch plans: per-matrix geometry, workspace carve-up, elementwise chunk
// prefixes and the grouped GEMM tile tables, cached per descriptor set.
//
// The plan is the single-device analogue of FsdpMuon's owner assignment,
// which the optimizer works out once when it is set up and which balances orthogonalization
// cost across buffers (page "core.distributed.fsdp.src.megatron_fsdp.
// experimental.muon", class FsdpMuon; PR #6425 "Opt step" step 3 picks owners
// by orthogonalization cost).  Here the same cost model orders matrices so
// that the grouped GEMM launches start the most expensive tiles first, and
// the tile tables are laid out so that each of the 8 XCDs works on a
// contiguous run of tiles (neighbouring tiles share operand panels in that
// XCD's L2).
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <numeric>
#include <string>
#include <vector>

#include <hip/hip_runtime.h>

#include "muon_internal.h"
#include "plan_cache.h"

namespace muon {

namespace {

constexpr int kXcds = 8;  // MI355X dispatches workgroup i to XCD i % 8

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// GEMM tile size for a matrix whose NS orientation is r x c.  Large tiles
// give the MFMA pipeline the operand reuse it needs; small matrices use small
// tiles so that zero padding stays a small fraction of the work.  Below a
// shorter side of 1024 a 256-tile matrix has at most 3 x 3 upper-triangle
// tiles and short contractions: such matrices fill 256 CUs poorly and their
// launches are latency-bound, so they take 128-tiles.  float32 products
// longer than kF32ChainK use at most 128-tiles: only those split their
// accumulation chains (the 256-tile has no registers to spare), and every
// contraction of a 256-tile is then at most c.
constexpr int64_t kF32ChainK = 32768;
int choose_tile(int64_t r, int64_t c, int gemm_mode) {
    if (r >= 1024 && (gemm_mode != MUON_GEMM_F32 || c <= kF32ChainK)) return 256;
    if (r >= 160) return 128;
    return 64;
}

int class_index(int tile) { return tile == 256 ? 0 : tile == 128 ? 1 : 2; }

// Running sums of a (sub)set of matrices' workspace needs.
struct Sums {
    int64_t x_bytes = 0, g_bytes = 0, u_floats = 0, chunks = 0, casts = 0, n = 0;
};

// Workspace layout of a set with these sums.  Regions start 256-byte aligned.
// The second X region starts 64 KiB past an alignment boundary so that the two
// iterates never alias at a power-of-two distance.  The compact U / O region
// (muon_step with ns_steps == 0 only, which uses no X, A or B) overlays them.
WsLayout layout_of(const Sums& s) {
    WsLayout w{};
    size_t at = 0;
    w.x[0] = at;
    at = align_up(at + size_t(s.x_bytes), kWsAlign) + (size_t(1) << 16);
    w.x[1] = at;
    at = align_up(at + size_t(s.x_bytes), kWsAlign);
    w.a = at;
    at = align_up(at + size_t(s.g_bytes), kWsAlign);
    w.b = at;
    at = align_up(at + size_t(s.g_bytes), kWsAlign);
    w.u = 0;
    at = std::max(at, align_up(size_t(s.u_floats) * 4, kWsAlign));
    // partial sums: one per elementwise chunk or one per cast tile
    w.partial = at;
    at = align_up(at + size_t(std::max<int64_t>(s.chunks, s.casts)) * 4, kWsAlign);
    w.inv = at;
    at = align_up(at + size_t(s.n) * 4, kWsAlign);
    w.total = std::max<size_t>(at, kWsAlign);
    return w;
}

// One matrix's geometry (offsets left at zero) and its contribution to the sums.
MatInfo mat_of(const muon_matrix_desc_t& d, int gemm_mode) {
    MatInfo m;
    std::memset(&m, 0, sizeof(m));
    m.R = int32_t(d.rows);
    m.C = int32_t(d.cols);
    m.numel = d.rows * d.cols;
    m.off = d.offset;
    m.poff = d.param_offset;
    m.pstride = d.n_shards > 1 ? d.shard_stride : 0;
    m.slice_len = m.numel / d.n_shards;
    m.tall = m.R > m.C;
    m.r = std::min(m.R, m.C);
    m.c = std::max(m.R, m.C);
    m.tile = choose_tile(m.r, m.c, gemm_mode);
    m.rp = int32_t(round_up(m.r, m.tile));
    m.cp = int32_t(round_up(m.c, m.tile));
    m.scale = float(std::sqrt(std::max(1.0, double(m.R) / double(m.C))));
    m.group = d.group;
    m.ns_f32 = gemm_mode == MUON_GEMM_F32 || m.tile == kF32NsTile;
    m.n_chunks = int32_t((m.numel + kEwChunk - 1) / kEwChunk);
    m.n_cast = (m.rp / kCastTile) * (m.cp / kCastTile);
    return m;
}

void add_to(Sums& s, const MatInfo& m) {
    const int64_t es = m.ns_f32 ? 4 : 2;
    // every region start stays 256-byte aligned: rp and cp are multiples of 64
    s.x_bytes += int64_t(m.rp) * m.cp * es;
    s.g_bytes += int64_t(m.rp) * m.rp * es;
    s.u_floats += round_up(m.numel, 64);
    s.chunks += m.n_chunks;
    s.casts += m.n_cast;
    s.n += 1;
}

struct Geometry {
    std::vector<MatInfo> mats;
    std::vector<int32_t> chunk_prefix, cast_prefix;
    int64_t state_extent = 0;
    WsLayout ws{};
};

Geometry build_geometry(const muon_matrix_desc_t* d, int64_t n, int gemm_mode) {
    Geometry g;
    g.mats.resize(size_t(n));
    g.chunk_prefix.assign(size_t(n) + 1, 0);
    g.cast_prefix.assign(size_t(n) + 1, 0);
    Sums s;
    for (int64_t i = 0; i < n; ++i) {
        MatInfo& m = g.mats[size_t(i)];
        m = mat_of(d[i], gemm_mode);
        const int64_t es = m.ns_f32 ? 4 : 2;
        // X, A and B offsets count elements of the matrix's own product type
        m.x_off = s.x_bytes / es;
        m.g_off = s.g_bytes / es;
        m.u_off = s.u_floats;
        m.chunk_begin = int32_t(s.chunks);
        m.cast_begin = int32_t(s.casts);
        add_to(s, m);
        g.chunk_prefix[size_t(i) + 1] = int32_t(s.chunks);
        g.cast_prefix[size_t(i) + 1] = int32_t(s.casts);
        g.state_extent = std::max<int64_t>(g.state_extent, m.off + m.numel);
    }
    g.ws = layout_of(s);
    return g;
}

// Waves: matrices in decreasing order of workspace need (then offset), each
// placed in the first wave that still fits the capacity (first fit
// decreasing).  capacity == 0: one wave with every matrix.  Every matrix must
// fit a wave on its own (checked by the caller against min_workspace_bytes_for).
std::vector<std::vector<int64_t>> partition_waves(const muon_matrix_desc_t* d, int64_t n,
                                                  int gemm_mode, size_t capacity) {
    std::vector<std::vector<int64_t>> waves;
    if (capacity == 0) {
        waves.emplace_back(static_cast<size_t>(n));
        std::iota(waves[0].begin(), waves[0].end(), int64_t(0));
        return waves;
    }
    std::vector<MatInfo> mats(static_cast<size_t>(n));
    std::vector<size_t> need(static_cast<size_t>(n));
    for (int64_t i = 0; i < n; ++i) {
        mats[size_t(i)] = mat_of(d[i], gemm_mode);
        Sums one;
        add_to(one, mats[size_t(i)]);
        need[size_t(i)] = layout_of(one).total;
    }
    std::vector<int64_t> order(static_cast<size_t>(n));
    std::iota(order.begin(), order.end(), int64_t(0));
    std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
        if (need[size_t(a)] != need[size_t(b)]) return need[size_t(a)] > need[size_t(b)];
        return d[a].offset < d[b].offset;
    });
    std::vector<Sums> sums;
    for (int64_t i : order) {
        size_t w = 0;
        for (; w < waves.size(); ++w) {
            Sums t = sums[w];
            add_to(t, mats[size_t(i)]);
            if (layout_of(t).total <= capacity) break;
        }
        if (w == waves.size()) {
            waves.emplace_back();
            sums.emplace_back();
        }
        waves[w].push_back(i);
        add_to(sums[w], mats[size_t(i)]);
    }
    for (auto& v : waves) std::sort(v.begin(), v.end());
    return waves;
}

// Orthogonalization cost of one matrix per iteration (padded, dense count of
// the three products): the quantity used to order work.
double ns_cost(const MatInfo& m) {
    const double r = m.rp, c = m.cp;
    return 3.0 * r * r * c + r * r * r;
}

// Tile table layout.  The hardware hands workgroup b to XCD b % 8, and each
// XCD (32 CUs) has its own L2.  Tiles are cut into chunks of 32 neighbours
// (tiles of one matrix that share operand panels, so the 32 tiles an XCD runs
// at once read few distinct panels), chunks are dealt to the XCD with the
// least work so far in decreasing order of cost (longest-processing-time
// first), and XCD x's k-th tile is placed at index 8 k + x.  Slots past an
// XCD's last tile hold mat = -1 (the workgroup exits at once).
struct Chunk {
    std::vector<GemmTile> tiles;
    double cost;
};

std::vector<GemmTile> balance_over_xcds(std::vector<Chunk> chunks) {
    std::stable_sort(chunks.begin(), chunks.end(),
                     [](const Chunk& a, const Chunk& b) { return a.cost > b.cost; });
    std::vector<std::vector<GemmTile>> per(kXcds);
    double load[kXcds] = {0};
    for (const Chunk& c : chunks) {
        int best = 0;
        for (int x = 1; x < kXcds; ++x)
            if (load[x] < load[best]) best = x;
        load[best] += c.cost;
        per[best].insert(per[best].end(), c.tiles.begin(), c.tiles.end());
    }
    size_t rows = 0;
    for (const auto& v : per) rows = std::max(rows, v.size());
    std::vector<GemmTile> out(rows * kXcds, GemmTile{-1, 0, 0, 0});
    for (int x = 0; x < kXcds; ++x)
        for (size_t k = 0; k < per[x].size(); ++k) out[k * kXcds + size_t(x)] = per[x][k];
    return out;
}

// Per-tile cost in K blocks of 64, plus a fixed share for the epilogue.
constexpr double kEpilogueBlocks = 8.0;
// Chunk size: up to 32 neighbours (one per CU of an XCD), but small enough
// that every XCD receives about eight chunks to balance.
size_t chunk_tiles(size_t total) {
    const size_t c = total / (kXcds * 8);
    return std::max<size_t>(4, std::min<size_t>(32, c / 4 * 4));
}

}  // namespace

size_t workspace_bytes_for(const muon_matrix_desc_t* d, int64_t n, int gemm_mode) {
    if (n == 0) return 0;
    return build_geometry(d, n, gemm_mode).ws.total;
}

size_t min_workspace_bytes_for(const muon_matrix_desc_t* d, int64_t n, int gemm_mode) {
    size_t most = 0;
    for (int64_t i = 0; i < n; ++i) {
        Sums one;
        add_to(one, mat_of(d[i], gemm_mode));
        most = std::max(most, layout_of(one).total);
    }
    return most;
}

// One wave's tables, built on the host: the device blob (mats | chunk prefix |
// cast prefix | tile tables) and where each part starts in it.
struct WaveTables {
    std::vector<MatInfo> mats;
    std::vector<int32_t> chunk_prefix, cast_prefix;
    std::vector<GemmTile> sym_a[3], sym_b[3], full[3];
    int64_t state_extent = 0;
    WsLayout ws{};
    size_t o_mats = 0, o_cp = 0, o_kp = 0, o_sym_a[3] = {}, o_sym_b[3] = {}, o_full[3] = {};
    size_t blob_bytes = 0;
};

namespace {

void build_tiles(WaveTables& p, int64_t n) {
    // Canonical matrix order (descending cost, then offset) so that the
    // schedule, like the results, does not depend on descriptor order.
    std::vector<int32_t> order(static_cast<size_t>(n));
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
        const double ca = ns_cost(p.mats[size_t(a)]), cb = ns_cost(p.mats[size_t(b)]);
        if (ca != cb) return ca > cb;
        return p.mats[size_t(a)].off < p.mats[size_t(b)].off;
    });
    // tiles of each matrix in locality order, with their cost in K blocks
    struct Run {
        std::vector<GemmTile> tiles;
        double tile_cost;
    };
    std::vector<Run> sym_a_runs[3], sym_b_runs[3], full_runs[3];
    auto chunk_all = [](const std::vector<Run>& runs) {
        size_t total = 0;
        for (const Run& r : runs) total += r.tiles.size();
        const size_t per = chunk_tiles(total);
        std::vector<Chunk> out;
        for (const Run& r : runs)
            for (size_t b = 0; b < r.tiles.size(); b += per) {
                Chunk c;
                c.tiles.assign(r.tiles.begin() + b, r.tiles.begin() + std::min(r.tiles.size(), b + per));
                c.cost = r.tile_cost * double(c.tiles.size());
                out.push_back(std::move(c));
            }
        return out;
    };
    for (int32_t mi : order) {
        const MatInfo& m = p.mats[size_t(mi)];
        const int cls = class_index(m.tile);
        const int nr = m.rp / m.tile, nc = m.cp / m.tile;
        // symmetric stages: bands of 8 tile rows walked column by column over the
        // upper triangle, so a chunk of 32 neighbours touches few row panels
        std::vector<GemmTile> sym;
        for (int t0 = 0; t0 < nr; t0 += 8)
            for (int tj = t0; tj < nr; ++tj)
                for (int ti = t0; ti < std::min(nr, t0 + 8); ++ti)
                    if (ti <= tj) sym.push_back({mi, ti, tj, 0});
        // full grid: bands of 8 tile rows walked column by column; a chunk of 32
        // covers 8 x 4 tiles (8 row panels of B and 4 row panels of X^T)
        std::vector<GemmTile> full;
        for (int t0 = 0; t0 < nr; t0 += 8)
            for (int tj = 0; tj < nc; ++tj)
                for (int ti = t0; ti < std::min(nr, t0 + 8); ++ti) full.push_back({mi, ti, tj, 0});
        // stage A contracts over cp, stages B and X over rp
        sym_a_runs[cls].push_back({sym, double(m.cp) / 64.0 + kEpilogueBlocks});
        sym_b_runs[cls].push_back({sym, double(m.rp) / 64.0 + kEpilogueBlocks});
        full_runs[cls].push_back({std::move(full), double(m.rp) / 64.0 + kEpilogueBlocks});
    }
    for (int c = 0; c < 3; ++c) {
        p.sym_a[c] = balance_over_xcds(chunk_all(sym_a_runs[c]));
        p.sym_b[c] = balance_over_xcds(chunk_all(sym_b_runs[c]));
        p.full[c] = balance_over_xcds(chunk_all(full_runs[c]));
    }
}

// The wave's tables and the offsets of its parts in the device blob.
std::unique_ptr<WaveTables> build_wave(const muon_matrix_desc_t* d, int64_t n, int gemm_mode) {
    auto p = std::make_unique<WaveTables>();
    Geometry g = build_geometry(d, n, gemm_mode);
    p->mats = std::move(g.mats);
    p->chunk_prefix = std::move(g.chunk_prefix);
    p->cast_prefix = std::move(g.cast_prefix);
    p->state_extent = g.state_extent;
    p->ws = g.ws;
    build_tiles(*p, n);
    size_t at = 0;
    auto reserve = [&](size_t bytes) {
        const size_t here = at;
        at = align_up(at + bytes, 256);
        return here;
    };
    p->o_mats = reserve(p->mats.size() * sizeof(MatInfo));
    p->o_cp = reserve(p->chunk_prefix.size() * 4);
    p->o_kp = reserve(p->cast_prefix.size() * 4);
    // each stage's class tables back to back (a mixed launch of the 128- and
    // 64-tile classes reads both as one table); every table holds a multiple of
    // 8 slots, so the XCD of each slot (slot % 8) is kept
    auto contiguous = [&](std::vector<GemmTile>* t, size_t* o) {
        size_t bytes = 0;
        for (int c = 0; c < 3; ++c) bytes += t[c].size() * sizeof(GemmTile);
        o[0] = reserve(bytes);
        for (int c = 1; c < 3; ++c) o[c] = o[c - 1] + t[c - 1].size() * sizeof(GemmTile);
    };
    contiguous(p->sym_a, p->o_sym_a);
    contiguous(p->sym_b, p->o_sym_b);
    contiguous(p->full, p->o_full);
    p->blob_bytes = std::max<size_t>(at, 256);
    return p;
}

// Writes the wave's tables into dst (blob_bytes bytes of host memory).
void write_blob(const WaveTables& p, unsigned char* dst) {
    std::memset(dst, 0, p.blob_bytes);
    auto put = [&](size_t off, const void* src, size_t bytes) {
        if (bytes) std::memcpy(dst + off, src, bytes);
    };
    put(p.o_mats, p.mats.data(), p.mats.size() * sizeof(MatInfo));
    put(p.o_cp, p.chunk_prefix.data(), p.chunk_prefix.size() * 4);
    put(p.o_kp, p.cast_prefix.data(), p.cast_prefix.size() * 4);
    for (int c = 0; c < 3; ++c) {
        put(p.o_sym_a[c], p.sym_a[c].data(), p.sym_a[c].size() * sizeof(GemmTile));
        put(p.o_sym_b[c], p.sym_b[c].data(), p.sym_b[c].size() * sizeof(GemmTile));
        put(p.o_full[c], p.full[c].data(), p.full[c].size() * sizeof(GemmTile));
    }
}

// The wave's launch view with its tables at dev (a device copy of the blob).
PlanView bind(const WaveTables& p, const void* dev) {
    const unsigned char* base = static_cast<const unsigned char*>(dev);
    PlanView v{};
    v.n = int(p.mats.size());
    v.gemm_mode = 0;
    v.state_extent = p.state_extent;
    v.total_chunks = p.chunk_prefix.back();
    v.total_cast = p.cast_prefix.back();
    v.ws = p.ws;
    v.mats_host = p.mats.data();
    v.mats = reinterpret_cast<const MatInfo*>(base + p.o_mats);
    v.chunk_prefix = reinterpret_cast<const int32_t*>(base + p.o_cp);
    v.cast_prefix = reinterpret_cast<const int32_t*>(base + p.o_kp);
    v.n_classes = 3;
    const int tiles[3] = {256, 128, 64};
    for (int c = 0; c < 3; ++c) {
        v.classes[c].tile = tiles[c];
        v.classes[c].n_sym_a = int(p.sym_a[c].size());
        v.classes[c].n_sym_b = int(p.sym_b[c].size());
        v.classes[c].n_full = int(p.full[c].size());
        v.classes[c].sym_a = reinterpret_cast<const GemmTile*>(base + p.o_sym_a[c]);
        v.classes[c].sym_b = reinterpret_cast<const GemmTile*>(base + p.o_sym_b[c]);
        v.classes[c].full = reinterpret_cast<const GemmTile*>(base + p.o_full[c]);
    }
    return v;
}

// The set's waves, each built from its own descriptors.
std::vector<std::unique_ptr<WaveTables>> build_waves(const muon_matrix_desc_t* d, int64_t n,
                                                     int gemm_mode, size_t capacity) {
    std::vector<std::unique_ptr<WaveTables>> out;
    for (const auto& idx : partition_waves(d, n, gemm_mode, capacity)) {
        std::vector<muon_matrix_desc_t> sub(idx.size());
        for (size_t k = 0; k < idx.size(); ++k) sub[k] = d[idx[k]];
        out.push_back(build_wave(sub.data(), int64_t(sub.size()), gemm_mode));
    }
    return out;
}

}  // namespace

// A cached plan: every wave's tables in one device allocation.
struct StepPlan {
    std::vector<std::unique_ptr<WaveTables>> waves;
    std::vector<PlanView> views;
    void* dev = nullptr;

    ~StepPlan() {
        if (dev != nullptr) {
            // Kernels of any stream may still read the tables.  Only reached
            // outside the cache's lock (plans are dropped after it is released).
            // If the device cannot be synchronized (another stream is being
            // captured in global mode), the tables are left allocated rather
            // than freed while a launch may still read them.
            if (hipDeviceSynchronize() == hipSuccess) (void)hipFree(dev);
            else (void)hipGetLastError();
        }
    }
};

int plan_waves(const StepPlan& p) { return int(p.views.size()); }
const PlanView& wave_view(const StepPlan& p, int wave) { return p.views[size_t(wave)]; }

struct HostPlan {
    std::vector<std::unique_ptr<WaveTables>> waves;
    std::vector<size_t> at;  // start of each wave's tables in the blob
    std::vector<unsigned char> blob;
    size_t ws_bytes = 0;
    int gemm_mode = 0;
};

namespace {

// Every wave's tables in one host blob (wave w at at[w]).
size_t pack_waves(const std::vector<std::unique_ptr<WaveTables>>& waves, std::vector<size_t>* at,
                  std::vector<unsigned char>* blob) {
    size_t total = 0;
    at->clear();
    for (const auto& w : waves) {
        at->push_back(total);
        total += align_up(w->blob_bytes, 256);
    }
    blob->assign(std::max<size_t>(total, 256), 0);
    for (size_t k = 0; k < waves.size(); ++k) write_blob(*waves[k], blob->data() + (*at)[k]);
    return blob->size();
}

std::shared_ptr<StepPlan> build_plan(const muon_matrix_desc_t* d, int64_t n, int gemm_mode,
                                     size_t capacity, hipStream_t stream, Status* st) {
    auto p = std::make_shared<StepPlan>();
    p->waves = build_waves(d, n, gemm_mode, capacity);
    std::vector<size_t> at;
    std::vector<unsigned char> blob;
    const size_t bytes = pack_waves(p->waves, &at, &blob);
    hipError_t e = hipMalloc(&p->dev, bytes);
    if (e != hipSuccess) {
        p->dev = nullptr;
        st->code = MUON_ERR_HIP;
        snprintf(st->msg, sizeof(st->msg), "hipMalloc of %zu plan bytes: %s", bytes,
                 hipGetErrorString(e));
        return nullptr;
    }
    e = hipMemcpyAsync(p->dev, blob.data(), bytes, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);  // first use only
    if (e != hipSuccess) {
        st->code = MUON_ERR_HIP;
        snprintf(st->msg, sizeof(st->msg), "upload of plan tables: %s", hipGetErrorString(e));
        return nullptr;
    }
    for (size_t k = 0; k < p->waves.size(); ++k) {
        PlanView v = bind(*p->waves[k], static_cast<unsigned char*>(p->dev) + at[k]);
        v.gemm_mode = gemm_mode;
        p->views.push_back(v);
    }
    return p;
}

std::mutex g_mutex;
// Plans are a few KB to a few MB of device tables each; 64 descriptor sets in
// use at once is plenty for an optimizer (one per parameter-group layout).
PlanCache<StepPlan> g_cache(64);

}  // namespace

int get_plan(const muon_matrix_desc_t* d, int64_t n, int gemm_mode, size_t capacity,
             hipStream_t stream, std::shared_ptr<const StepPlan>* out, Status* st) {
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) {
        st->code = MUON_ERR_HIP;
        snprintf(st->msg, sizeof(st->msg), "hipGetDevice: %s", hipGetErrorString(e));
        return st->code;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) {
        st->code = MUON_ERR_HIP;
        snprintf(st->msg, sizeof(st->msg), "hipStreamIsCapturing: %s", hipGetErrorString(e));
        return st->code;
    }
    const bool capturing = cs == hipStreamCaptureStatusActive;
    const uint64_t cap = capacity;
    std::string key;
    key.resize(sizeof(int) * 2 + sizeof(cap) + size_t(n) * sizeof(muon_matrix_desc_t));
    std::memcpy(&key[0], &device, sizeof(int));
    std::memcpy(&key[sizeof(int)], &gemm_mode, sizeof(int));
    std::memcpy(&key[sizeof(int) * 2], &cap, sizeof(cap));
    if (n) std::memcpy(&key[sizeof(int) * 2 + sizeof(cap)], d, size_t(n) * sizeof(muon_matrix_desc_t));

    std::vector<std::shared_ptr<StepPlan>> evicted;  // destroyed after the lock is released
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        if (std::shared_ptr<StepPlan> p = g_cache.find(key, capturing)) {
            *out = std::move(p);
            return MUON_OK;
        }
        if (capturing) {
            st->code = MUON_ERR_BAD_ARG;
            snprintf(st->msg, sizeof(st->msg),
                     "no launch plan exists yet for these descriptors (and workspace size): "
                     "make one call outside graph capture first (it allocates and synchronizes)");
            return st->code;
        }
        std::shared_ptr<StepPlan> p = build_plan(d, n, gemm_mode, capacity, stream, st);
        if (!p) return st->code;
        evicted = g_cache.insert(std::move(key), p, false);
        *out = std::move(p);
    }
    return MUON_OK;
}

int build_host_plan(const muon_matrix_desc_t* d, int64_t n, int gemm_mode, size_t capacity,
                    std::shared_ptr<HostPlan>* out, Status* st) {
    (void)st;
    auto p = std::make_shared<HostPlan>();
    p->gemm_mode = gemm_mode;
    p->waves = build_waves(d, n, gemm_mode, capacity);
    pack_waves(p->waves, &p->at, &p->blob);
    for (const auto& w : p->waves) p->ws_bytes = std::max(p->ws_bytes, w->ws.total);
    *out = std::move(p);
    return MUON_OK;
}

size_t host_plan_blob_bytes(const HostPlan& p) { return p.blob.size(); }
const void* host_plan_blob(const HostPlan& p) { return p.blob.data(); }
size_t host_plan_workspace_bytes(const HostPlan& p) { return p.ws_bytes; }
int host_plan_waves(const HostPlan& p) { return int(p.waves.size()); }
PlanView host_plan_view(const HostPlan& p, int wave, const void* dev_blob) {
    PlanView v = bind(*p.waves[size_t(wave)], static_cast<const unsigned char*>(dev_blob) +
                                                  p.at[size_t(wave)]);
    v.gemm_mode = p.gemm_mode;
    return v;
}

}  // namespace muon
