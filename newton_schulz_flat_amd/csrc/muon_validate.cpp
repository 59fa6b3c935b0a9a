// Host-side validation of the Muon step's arguments.  Makes no HIP call, so
// every check here also runs (and is tested) on a machine without a GPU.
//
// Loud validation follows FsdpMuon._validate_parameter_groups on the page
// "core.distributed.fsdp.src.megatron_fsdp.experimental.muon" (parameters and
// the buffers holding them are checked up front) and the error convention of
// PR #6873 (an inconsistent layout is an error, never a quiet wrong mapping of shards).
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <vector>

#include "muon_internal.h"

namespace muon {

static int fail(Status* st, int code, const char* fmt, ...) {
    st->code = code;
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(st->msg, sizeof(st->msg), fmt, ap);
    va_end(ap);
    return code;
}

int check_desc_shapes(const muon_matrix_desc_t* d, int64_t n, Status* st, int64_t n_groups) {
    if (n < 0) return fail(st, MUON_ERR_BAD_ARG, "descriptor count n = %lld < 0", (long long)n);
    if (n > 0 && d == nullptr) return fail(st, MUON_ERR_NULL_POINTER, "descs is NULL");
    if (n > (int64_t(1) << 24))
        return fail(st, MUON_ERR_BAD_ARG, "descriptor count n = %lld is too large", (long long)n);
    int64_t set_numel = 0;
    for (int64_t i = 0; i < n; ++i) {
        const muon_matrix_desc_t& m = d[i];
        if (m.rows < 1 || m.cols < 1)
            return fail(st, MUON_ERR_BAD_SHAPE, "descs[%lld]: shape %lld x %lld has a side < 1",
                        (long long)i, (long long)m.rows, (long long)m.cols);
        if (m.rows > kMaxSide || m.cols > kMaxSide || m.rows * m.cols > kMaxNumel)
            return fail(st, MUON_ERR_BAD_SHAPE, "descs[%lld]: shape %lld x %lld is too large",
                        (long long)i, (long long)m.rows, (long long)m.cols);
        set_numel += m.rows * m.cols;
        if (set_numel > kMaxSetNumel)
            return fail(st, MUON_ERR_BAD_SHAPE,
                        "descs[0..%lld] hold more than %lld elements in total", (long long)i,
                        (long long)kMaxSetNumel);
        if (m.group < 0 || m.group >= n_groups)
            return fail(st, MUON_ERR_BAD_ARG, "descs[%lld]: group %d outside [0, %lld)",
                        (long long)i, m.group, (long long)n_groups);
        if (m.n_shards < 1)
            return fail(st, MUON_ERR_BAD_SHAPE, "descs[%lld]: n_shards = %d < 1", (long long)i,
                        m.n_shards);
        const int64_t numel = m.rows * m.cols;
        if (numel % m.n_shards != 0)
            return fail(st, MUON_ERR_BAD_SHAPE,
                        "descs[%lld]: numel %lld is not a multiple of n_shards %d", (long long)i,
                        (long long)numel, m.n_shards);
        if (m.n_shards > 1) {
            const int64_t len = numel / m.n_shards;
            if (len % 8 != 0)
                return fail(st, MUON_ERR_BAD_SHAPE,
                            "descs[%lld]: slice length %lld is not a multiple of 8",
                            (long long)i, (long long)len);
            if (m.shard_stride < len)
                return fail(st, MUON_ERR_OVERLAP,
                            "descs[%lld]: shard_stride %lld < slice length %lld (slices overlap)",
                            (long long)i, (long long)m.shard_stride, (long long)len);
        }
    }
    return MUON_OK;
}

namespace {
struct Span {
    int64_t begin, end;
    int64_t desc;
};

// Sorted spans must be pairwise disjoint.
int check_disjoint(std::vector<Span>& spans, const char* what, Status* st) {
    std::sort(spans.begin(), spans.end(), [](const Span& a, const Span& b) {
        return a.begin < b.begin || (a.begin == b.begin && a.desc < b.desc);
    });
    for (size_t i = 1; i < spans.size(); ++i) {
        if (spans[i].begin < spans[i - 1].end)
            return fail(st, MUON_ERR_OVERLAP, "%s of descs[%lld] and descs[%lld] overlap", what,
                        (long long)spans[i - 1].desc, (long long)spans[i].desc);
    }
    return MUON_OK;
}
}  // namespace

int check_state_ranges(const muon_matrix_desc_t* d, int64_t n, int64_t n_elems, const char* what,
                       Status* st) {
    if (n_elems < 0) return fail(st, MUON_ERR_BAD_ARG, "%s element count < 0", what);
    std::vector<Span> spans;
    spans.reserve(size_t(n));
    for (int64_t i = 0; i < n; ++i) {
        const int64_t numel = d[i].rows * d[i].cols;
        if (d[i].offset < 0 || d[i].offset > n_elems - numel)
            return fail(st, MUON_ERR_OUT_OF_BOUNDS,
                        "descs[%lld]: [%lld, %lld) is outside the %s buffer of %lld elements",
                        (long long)i, (long long)d[i].offset, (long long)(d[i].offset + numel),
                        what, (long long)n_elems);
        if (d[i].offset % 4 != 0)
            return fail(st, MUON_ERR_MISALIGNED,
                        "descs[%lld]: offset %lld is not 16-byte aligned in the float32 %s buffer",
                        (long long)i, (long long)d[i].offset, what);
        spans.push_back({d[i].offset, d[i].offset + numel, i});
    }
    return check_disjoint(spans, "state ranges", st);
}

int check_param_ranges(const muon_matrix_desc_t* d, int64_t n, int64_t n_param_elems,
                       int param_dtype, Status* st) {
    if (param_dtype != MUON_DTYPE_F32 && param_dtype != MUON_DTYPE_BF16)
        return fail(st, MUON_ERR_BAD_ARG, "param_dtype %d is not MUON_DTYPE_F32 or _BF16",
                    param_dtype);
    if (n_param_elems < 0) return fail(st, MUON_ERR_BAD_ARG, "n_param_elems < 0");
    const int64_t align = param_dtype == MUON_DTYPE_F32 ? 4 : 8;  // 16 bytes
    std::vector<Span> spans;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t len = d[i].rows * d[i].cols / d[i].n_shards;
        for (int32_t k = 0; k < d[i].n_shards; ++k) {
            const int64_t start = d[i].param_offset + int64_t(k) * d[i].shard_stride;
            if (d[i].param_offset < 0 || start < 0 || start > n_param_elems - len)
                return fail(st, MUON_ERR_OUT_OF_BOUNDS,
                            "descs[%lld]: slice %d [%lld, %lld) is outside params (%lld elements)",
                            (long long)i, k, (long long)start, (long long)(start + len),
                            (long long)n_param_elems);
            if (start % align != 0)
                return fail(st, MUON_ERR_MISALIGNED,
                            "descs[%lld]: slice %d starts at element %lld, not 16-byte aligned",
                            (long long)i, k, (long long)start);
            spans.push_back({start, start + len, i});
            if (d[i].n_shards == 1) break;
        }
    }
    return check_disjoint(spans, "param slices", st);
}

int check_no_alias(const Range* r, int count, Status* st) {
    for (int i = 0; i < count; ++i) {
        if (r[i].bytes == 0) continue;
        const uintptr_t ai = reinterpret_cast<uintptr_t>(r[i].ptr);
        for (int j = i + 1; j < count; ++j) {
            if (r[j].bytes == 0) continue;
            const uintptr_t aj = reinterpret_cast<uintptr_t>(r[j].ptr);
            if (ai < aj + r[j].bytes && aj < ai + r[i].bytes)
                return fail(st, MUON_ERR_ALIAS, "buffers %s and %s overlap in memory", r[i].name,
                            r[j].name);
        }
    }
    return MUON_OK;
}

int check_scalar(float v, const char* name, Status* st) {
    if (!std::isfinite(v)) return fail(st, MUON_ERR_BAD_ARG, "%s = %g is not finite", name, v);
    return MUON_OK;
}

}  // namespace muon
