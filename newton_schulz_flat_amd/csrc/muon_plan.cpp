// Launch plans: per-matrix geometry, workspace carve-up, elementwise chunk
// prefixes and the grouped GEMM tile tables, cached per descriptor set.
//
// The plan is the single-device analogue of FsdpMuon's owner assignment,
// which is "computed during initialization" and balances orthogonalization
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
#include <list>
#include <mutex>
#include <numeric>
#include <string>
#include <unordered_map>
#include <vector>

#include <hip/hip_runtime.h>

#include "muon_internal.h"

namespace muon {

namespace {

constexpr int kXcds = 8;  // MI355X dispatches workgroup i to XCD i % 8

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// GEMM tile size for a matrix whose NS orientation is r x c.  Large tiles
// give the MFMA pipeline the operand reuse it needs; small matrices use small
// tiles so that zero padding stays a small fraction of the work.  float32
// products longer than kF32ChainK use at most 128-tiles: only those split
// their accumulation chains (the 256-tile has no registers to spare), and
// every contraction of a 256-tile is then at most c.
constexpr int64_t kF32ChainK = 32768;
int choose_tile(int64_t r, int64_t c, int gemm_mode) {
    if (r >= 768 && (gemm_mode != MUON_GEMM_F32 || c <= kF32ChainK)) return 256;
    if (r >= 160) return 128;
    return 64;
}

int class_index(int tile) { return tile == 256 ? 0 : tile == 128 ? 1 : 2; }

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
    // X, A and B regions in bytes; each matrix's offsets count elements of its
    // own product type (2 or 4 bytes)
    int64_t x_bytes = 0, g_bytes = 0, chunks = 0, casts = 0;
    for (int64_t i = 0; i < n; ++i) {
        MatInfo& m = g.mats[size_t(i)];
        std::memset(&m, 0, sizeof(m));
        m.R = int32_t(d[i].rows);
        m.C = int32_t(d[i].cols);
        m.numel = d[i].rows * d[i].cols;
        m.off = d[i].offset;
        m.poff = d[i].param_offset;
        m.pstride = d[i].n_shards > 1 ? d[i].shard_stride : 0;
        m.slice_len = m.numel / d[i].n_shards;
        m.tall = m.R > m.C;
        m.r = std::min(m.R, m.C);
        m.c = std::max(m.R, m.C);
        m.tile = choose_tile(m.r, m.c, gemm_mode);
        m.rp = int32_t(round_up(m.r, m.tile));
        m.cp = int32_t(round_up(m.c, m.tile));
        m.scale = float(std::sqrt(std::max(1.0, double(m.R) / double(m.C))));
        m.group = d[i].group;
        m.ns_f32 = gemm_mode == MUON_GEMM_F32 || m.tile == kF32NsTile;
        const int64_t es = m.ns_f32 ? 4 : 2;
        // Every region start stays 256-byte aligned: rp and cp are multiples of 64.
        m.x_off = x_bytes / es;
        x_bytes += int64_t(m.rp) * m.cp * es;
        m.g_off = g_bytes / es;
        g_bytes += int64_t(m.rp) * m.rp * es;
        m.n_chunks = int32_t((m.numel + kEwChunk - 1) / kEwChunk);
        m.chunk_begin = int32_t(chunks);
        chunks += m.n_chunks;
        m.n_cast = (m.rp / kCastTile) * (m.cp / kCastTile);
        m.cast_begin = int32_t(casts);
        casts += m.n_cast;
        g.chunk_prefix[size_t(i) + 1] = int32_t(chunks);
        g.cast_prefix[size_t(i) + 1] = int32_t(casts);
        g.state_extent = std::max<int64_t>(g.state_extent, m.off + m.numel);
    }
    WsLayout& w = g.ws;
    size_t at = 0;
    w.u = at;
    at = align_up(at + size_t(g.state_extent) * 4, kWsAlign);
    // The second X region starts 64 KiB past an alignment boundary so that the
    // two iterates never alias at a power-of-two distance.
    w.x[0] = at;
    at = align_up(at + size_t(x_bytes), kWsAlign) + (size_t(1) << 16);
    w.x[1] = at;
    at = align_up(at + size_t(x_bytes), kWsAlign);
    w.a = at;
    at = align_up(at + size_t(g_bytes), kWsAlign);
    w.b = at;
    at = align_up(at + size_t(g_bytes), kWsAlign);
    // partial sums: one per elementwise chunk or one per cast tile
    w.partial = at;
    at = align_up(at + size_t(std::max<int64_t>(chunks, casts)) * 4, kWsAlign);
    w.inv = at;
    at = align_up(at + size_t(n) * 4, kWsAlign);
    w.total = std::max<size_t>(at, kWsAlign);
    return g;
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

struct PlanStore {
    PlanView view{};
    std::vector<MatInfo> mats;
    std::vector<int32_t> chunk_prefix, cast_prefix;
    std::vector<GemmTile> sym_a[3], sym_b[3], full[3];
    std::vector<unsigned char> host_blob;  // staging copy of the device tables
    void* dev = nullptr;
    int device = -1;

    ~PlanStore() {
        if (dev != nullptr) {
            // Kernels of any stream may still read the tables.
            (void)hipDeviceSynchronize();
            (void)hipFree(dev);
        }
    }
};

const PlanView& view_of(const PlanStore& s) { return s.view; }

namespace {

std::shared_ptr<PlanStore> build_plan(const muon_matrix_desc_t* d, int64_t n, int gemm_mode,
                                      int device, hipStream_t stream, Status* st) {
    auto p = std::make_shared<PlanStore>();
    p->device = device;
    Geometry g = build_geometry(d, n, gemm_mode);
    p->mats = std::move(g.mats);
    p->chunk_prefix = std::move(g.chunk_prefix);
    p->cast_prefix = std::move(g.cast_prefix);

    // Canonical matrix order (descending cost, then offset) so that the
    // schedule, like the results, does not depend on descriptor order.
    std::vector<int32_t> order(static_cast<size_t>(n));
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
        const double ca = ns_cost(p->mats[size_t(a)]), cb = ns_cost(p->mats[size_t(b)]);
        if (ca != cb) return ca > cb;
        return p->mats[size_t(a)].off < p->mats[size_t(b)].off;
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
        const MatInfo& m = p->mats[size_t(mi)];
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
        p->sym_a[c] = balance_over_xcds(chunk_all(sym_a_runs[c]));
        p->sym_b[c] = balance_over_xcds(chunk_all(sym_b_runs[c]));
        p->full[c] = balance_over_xcds(chunk_all(full_runs[c]));
    }

    // One device blob: mats | chunk prefix | cast prefix | tile tables.
    size_t at = 0;
    auto reserve = [&](size_t bytes) {
        const size_t here = at;
        at = align_up(at + bytes, 256);
        return here;
    };
    const size_t o_mats = reserve(p->mats.size() * sizeof(MatInfo));
    const size_t o_cp = reserve(p->chunk_prefix.size() * 4);
    const size_t o_kp = reserve(p->cast_prefix.size() * 4);
    size_t o_sym_a[3], o_sym_b[3], o_full[3];
    for (int c = 0; c < 3; ++c) {
        o_sym_a[c] = reserve(p->sym_a[c].size() * sizeof(GemmTile));
        o_sym_b[c] = reserve(p->sym_b[c].size() * sizeof(GemmTile));
        o_full[c] = reserve(p->full[c].size() * sizeof(GemmTile));
    }
    const size_t blob = std::max<size_t>(at, 256);
    p->host_blob.assign(blob, 0);
    auto put = [&](size_t off, const void* src, size_t bytes) {
        if (bytes) std::memcpy(p->host_blob.data() + off, src, bytes);
    };
    put(o_mats, p->mats.data(), p->mats.size() * sizeof(MatInfo));
    put(o_cp, p->chunk_prefix.data(), p->chunk_prefix.size() * 4);
    put(o_kp, p->cast_prefix.data(), p->cast_prefix.size() * 4);
    for (int c = 0; c < 3; ++c) {
        put(o_sym_a[c], p->sym_a[c].data(), p->sym_a[c].size() * sizeof(GemmTile));
        put(o_sym_b[c], p->sym_b[c].data(), p->sym_b[c].size() * sizeof(GemmTile));
        put(o_full[c], p->full[c].data(), p->full[c].size() * sizeof(GemmTile));
    }
    hipError_t e = hipMalloc(&p->dev, blob);
    if (e != hipSuccess) {
        p->dev = nullptr;
        st->code = MUON_ERR_HIP;
        snprintf(st->msg, sizeof(st->msg), "hipMalloc of %zu plan bytes: %s", blob,
                 hipGetErrorString(e));
        return nullptr;
    }
    e = hipMemcpyAsync(p->dev, p->host_blob.data(), blob, hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);  // first use only
    if (e != hipSuccess) {
        st->code = MUON_ERR_HIP;
        snprintf(st->msg, sizeof(st->msg), "upload of plan tables: %s", hipGetErrorString(e));
        return nullptr;
    }
    unsigned char* base = static_cast<unsigned char*>(p->dev);
    PlanView& v = p->view;
    v.n = int(n);
    v.gemm_mode = gemm_mode;
    v.state_extent = g.state_extent;
    v.total_chunks = p->chunk_prefix.back();
    v.total_cast = p->cast_prefix.back();
    v.ws = g.ws;
    v.mats_host = p->mats.data();
    v.mats = reinterpret_cast<const MatInfo*>(base + o_mats);
    v.chunk_prefix = reinterpret_cast<const int32_t*>(base + o_cp);
    v.cast_prefix = reinterpret_cast<const int32_t*>(base + o_kp);
    v.n_classes = 3;
    const int tiles[3] = {256, 128, 64};
    for (int c = 0; c < 3; ++c) {
        v.classes[c].tile = tiles[c];
        v.classes[c].n_sym_a = int(p->sym_a[c].size());
        v.classes[c].n_sym_b = int(p->sym_b[c].size());
        v.classes[c].n_full = int(p->full[c].size());
        v.classes[c].sym_a = reinterpret_cast<const GemmTile*>(base + o_sym_a[c]);
        v.classes[c].sym_b = reinterpret_cast<const GemmTile*>(base + o_sym_b[c]);
        v.classes[c].full = reinterpret_cast<const GemmTile*>(base + o_full[c]);
    }
    return p;
}

struct CacheEntry {
    std::string key;
    std::shared_ptr<PlanStore> plan;
};

std::mutex g_mutex;
std::list<CacheEntry> g_lru;  // most recent first
constexpr size_t kMaxPlans = 32;

}  // namespace

int get_plan(const muon_matrix_desc_t* d, int64_t n, int gemm_mode, hipStream_t stream,
             std::shared_ptr<const PlanStore>* out, Status* st) {
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) {
        st->code = MUON_ERR_HIP;
        snprintf(st->msg, sizeof(st->msg), "hipGetDevice: %s", hipGetErrorString(e));
        return st->code;
    }
    std::string key;
    key.resize(sizeof(int) * 2 + size_t(n) * sizeof(muon_matrix_desc_t));
    std::memcpy(&key[0], &device, sizeof(int));
    std::memcpy(&key[sizeof(int)], &gemm_mode, sizeof(int));
    if (n) std::memcpy(&key[sizeof(int) * 2], d, size_t(n) * sizeof(muon_matrix_desc_t));

    std::lock_guard<std::mutex> lock(g_mutex);
    for (auto it = g_lru.begin(); it != g_lru.end(); ++it) {
        if (it->key == key) {
            g_lru.splice(g_lru.begin(), g_lru, it);
            *out = g_lru.front().plan;
            return MUON_OK;
        }
    }
    std::shared_ptr<PlanStore> p = build_plan(d, n, gemm_mode, device, stream, st);
    if (!p) return st->code;
    g_lru.push_front(CacheEntry{std::move(key), p});
    if (g_lru.size() > kMaxPlans) g_lru.pop_back();
    *out = p;
    return MUON_OK;
}

}  // namespace muon
