// C-ABI layer: argument validation (before any HIP call), error reporting,
// launch-shape tuning, and dispatch to the kernels. Nothing here allocates
// device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <new>
#include <vector>

#include "zr.h"
#include "zr_guard.hpp"
#include "zr_internal.hpp"

namespace zr {

namespace {

thread_local std::string g_err;

zr_status fail(zr_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

zr_status ok() { return ZR_OK; }

// Largest element count per rank buffer: keeps every tile index of the
// kernels within 32 bits.
constexpr int64_t kMaxElems = ZR_MAX_ELEMS;

zr_status hip_fail(hipError_t e, const char* what) {
    return fail(ZR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool dt_valid(int dt) { return dt == ZR_BF16 || dt == ZR_FP32; }
int64_t dt_bytes(zr_dtype dt) { return dt == ZR_BF16 ? 2 : 4; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
bool overlaps(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi && a.lo < a.hi && b.lo < b.hi; }
Range range_of(const void* p, int64_t elems, int64_t es) {
    return Range{(uintptr_t)p, (uintptr_t)p + (uintptr_t)(elems * es)};
}

int env_int(const char* name, int dflt, int lo, int hi) {
    const char* v = std::getenv(name);
    if (!v || !*v) return dflt;
    int x = std::atoi(v);
    return x < lo ? lo : (x > hi ? hi : x);
}

// ZR_FORCE_PATH: "element", "small" or "large"; unset, empty or "auto" leaves
// the choice to the kernels. Any other value is reported once on stderr and
// ignored.
int env_path(const char* name) {
    const char* v = std::getenv(name);
    if (!v || !*v || !std::strcmp(v, "auto")) return kPathAuto;
    if (!std::strcmp(v, "element")) return kPathElement;
    if (!std::strcmp(v, "small")) return kPathSmall;
    if (!std::strcmp(v, "large")) return kPathLarge;
    std::fprintf(stderr, "libzr: %s=%s is not one of element, small, large; ignored\n", name, v);
    return kPathAuto;
}

zr_status check_k(int K) {
    if (K < 1 || K > kMaxRanks) return fail(ZR_ERR_INVALID, "K=%d out of range [1, %d]", K, kMaxRanks);
    return ok();
}

// Non-null and aligned to the element size.
zr_status check_table(const void* const* t, int K, int64_t es, const char* name) {
    if (!t) return fail(ZR_ERR_INVALID, "%s table is NULL", name);
    for (int r = 0; r < K; ++r) {
        if (!t[r]) return fail(ZR_ERR_INVALID, "%s[%d] is NULL", name, r);
        if (((uintptr_t)t[r]) & (uintptr_t)(es - 1))  // element sizes are powers of two
            return fail(ZR_ERR_ALIGN, "%s[%d]=%p is not aligned to %lld bytes", name, r, t[r],
                        (long long)es);
    }
    return ok();
}

// The K ranges of one table must be pairwise disjoint.
zr_status check_distinct(const std::vector<Range>& rs, const char* name) {
    for (size_t a = 0; a < rs.size(); ++a)
        for (size_t b = a + 1; b < rs.size(); ++b)
            if (overlaps(rs[a], rs[b]))
                return fail(ZR_ERR_ALIAS, "%s[%zu] and %s[%zu] overlap", name, a, name, b);
    return ok();
}

// xs must already be pairwise disjoint (check_distinct). Sorted by start,
// their ends then increase too, so the only x that can overlap a range y is
// the first one ending after y starts: one binary search per y instead of a
// test against every x (the fragment tables hold up to K * F ranges).
zr_status check_disjoint(const std::vector<Range>& xs, const char* xn, const std::vector<Range>& ys,
                         const char* yn) {
    std::vector<size_t> ord;  // the non-empty xs, by start
    ord.reserve(xs.size());
    for (size_t a = 0; a < xs.size(); ++a)
        if (xs[a].lo < xs[a].hi) ord.push_back(a);
    std::sort(ord.begin(), ord.end(), [&](size_t p, size_t q) { return xs[p].lo < xs[q].lo; });
    for (size_t b = 0; b < ys.size(); ++b) {
        const Range& y = ys[b];
        if (!(y.lo < y.hi)) continue;
        const auto it = std::partition_point(ord.begin(), ord.end(), [&](size_t a) { return xs[a].hi <= y.lo; });
        if (it != ord.end() && overlaps(xs[*it], y))
            return fail(ZR_ERR_ALIAS, "%s[%zu] overlaps %s[%zu]", xn, *it, yn, b);
    }
    return ok();
}

// Fragment sizes: each in [0, kMaxElems], and so is their running total.
zr_status check_sizes(const int64_t* numels, int n, int64_t* total) {
    *total = 0;
    for (int p = 0; p < n; ++p) {
        if (numels[p] < 0 || numels[p] > kMaxElems)
            return fail(ZR_ERR_INVALID, "numels[%d]=%lld not in [0, 2^40]", p, (long long)numels[p]);
        *total += numels[p];
        if (*total > kMaxElems) return fail(ZR_ERR_INVALID, "fragments total more than 2^40 elements");
    }
    return ZR_OK;
}

#define ZR_TRY(expr)                       \
    do {                                   \
        zr_status st_ = (expr);            \
        if (st_ != ZR_OK) return st_;      \
    } while (0)

// A workspace argument: NULL (no staging), or an 8-byte-aligned device
// buffer of ws_bytes bytes.
zr_status check_workspace(const void* ws, size_t ws_bytes) {
    if (!ws) return ok();
    if (((uintptr_t)ws) & 7) return fail(ZR_ERR_ALIGN, "workspace %p is not 8-byte aligned", ws);
    if (ws_bytes == 0) return fail(ZR_ERR_WORKSPACE, "workspace of 0 bytes");
    return ok();
}

// A staged table of `need` bytes must fit the workspace and must not overlap
// any buffer the call reads or writes.
zr_status check_staging(const void* ws, size_t ws_bytes, size_t need, const std::vector<Range>& a,
                        const char* an, const std::vector<Range>& b, const char* bn) {
    if (need > ws_bytes)
        return fail(ZR_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu-byte table", ws_bytes,
                    need);
    const Range w{(uintptr_t)ws, (uintptr_t)ws + need};
    for (size_t i = 0; i < a.size(); ++i)
        if (overlaps(w, a[i])) return fail(ZR_ERR_ALIAS, "workspace overlaps %s[%zu]", an, i);
    for (size_t i = 0; i < b.size(); ++i)
        if (overlaps(w, b[i])) return fail(ZR_ERR_ALIAS, "workspace overlaps %s[%zu]", bn, i);
    return ok();
}

// Whether work enqueued on `s` would be recorded into a graph. A table staged
// by an asynchronous copy from a host buffer must not be recorded (a replay
// would read the buffer after the call freed it), so such calls go out as
// argument launches instead. A failing query counts as capturing.
bool capturing(hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) != hipSuccess) return true;
    return st != hipStreamCaptureStatusNone;
}

// The status of a call whose launches on `s` returned `e`. With ZR_DEBUG set
// (and `s` not capturing) the call first waits for `s`, so an error the
// kernels raise comes back from the call that launched them.
zr_status launched(hipError_t e, hipStream_t s, const char* what) {
    if (e == hipSuccess && tuning().debug && !capturing(s)) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, what);
    return ok();
}

}  // namespace

hipError_t stage_table(void* ws, const void* image, size_t bytes, hipStream_t stream, bool stream_order) {
    if (bytes == 0) return hipSuccess;
    if (stream_order) return hipMemcpyAsync(ws, image, bytes, hipMemcpyHostToDevice, stream);
    return hipMemcpy(ws, image, bytes, hipMemcpyHostToDevice);
}

zr_status set_error(zr_status st, const char* msg) {
    g_err = msg ? msg : "";
    return st;
}

const Tuning& tuning() {
    static const Tuning t = {
        env_int("ZR_AR_NONTEMPORAL", 1, 0, 1),
        env_int("ZR_AG_NONTEMPORAL", 1, 0, 1),
        env_int("ZR_MAX_GRID", 1 << 30, 1, 1 << 30),
        env_path("ZR_FORCE_PATH"),
        env_int("ZR_RS_PAIRS", 1, 0, 1),
        env_int("ZR_DEBUG", 0, 0, 1),
    };
    return t;
}

int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    if (dev < 64) {
        int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Validation of a reduce-scatter call; shared with the scheduler.
zr_status validate_rs(int K, const void* const* in, zr_dtype in_dt, int64_t N, void* const* out,
                      zr_dtype out_dt, int shift, int flags, zr_order order, bool* no_work) {
    ZR_TRY(check_k(K));
    if (flags & ~(ZR_AVERAGE | ZR_ACCUMULATE)) return fail(ZR_ERR_INVALID, "flags=%d has unknown bits", flags);
    if (N < 0) return fail(ZR_ERR_INVALID, "N=%lld is negative", (long long)N);
    if (!dt_valid(in_dt) || !dt_valid(out_dt))
        return fail(ZR_ERR_UNSUPPORTED, "dtype pair (%d, %d) not supported", (int)in_dt, (int)out_dt);
    if (shift < 0 || shift >= K) return fail(ZR_ERR_INVALID, "chunk_shift=%d not in [0, %d)", shift, K);
    if (order != ZR_ORDER_RING && order != ZR_ORDER_FREE && order != ZR_ORDER_RING_WIRE)
        return fail(ZR_ERR_INVALID, "order=%d is not a zr_order", (int)order);
    *no_work = (N == 0);
    if (N == 0) return ok();
    if (N > kMaxElems) return fail(ZR_ERR_INVALID, "N=%lld too large", (long long)N);
    const int64_t C = (N + K - 1) / K;
    ZR_TRY(check_table(in, K, dt_bytes(in_dt), "in"));
    ZR_TRY(check_table(const_cast<const void* const*>(out), K, dt_bytes(out_dt), "out"));
    std::vector<Range> ri(K), ro(K);
    for (int r = 0; r < K; ++r) {
        ri[r] = range_of(in[r], N, dt_bytes(in_dt));
        ro[r] = range_of(out[r], C, dt_bytes(out_dt));
    }
    ZR_TRY(check_distinct(ro, "out"));
    ZR_TRY(check_disjoint(ro, "out", ri, "in"));
    return ok();
}

zr_status run_rs(int K, const void* const* in, zr_dtype in_dt, int64_t N, void* const* out,
                 zr_dtype out_dt, int shift, int flags, zr_order order, hipStream_t stream) {
    ConstPtrs ip{};
    MutPtrs op{};
    for (int r = 0; r < K; ++r) {
        ip.p[r] = in[r];
        op.p[r] = out[r];
    }
    hipError_t e = launch_reduce_scatter(K, ip, in_dt, N, op, out_dt, shift, flags, order, stream);
    return launched(e, stream, "reduce-scatter launch");
}

zr_status validate_ag(int K, const void* const* shards, void* const* fulls, zr_dtype dt,
                      const zr_seg* segs, int n_segs, int shift, bool* no_work) {
    ZR_TRY(check_k(K));
    if (!dt_valid(dt)) return fail(ZR_ERR_UNSUPPORTED, "dtype %d not supported", (int)dt);
    if (shift < 0 || shift >= K) return fail(ZR_ERR_INVALID, "chunk_shift=%d not in [0, %d)", shift, K);
    if (n_segs < 0) return fail(ZR_ERR_INVALID, "n_segs=%d is negative", n_segs);
    if (n_segs > 0 && !segs) return fail(ZR_ERR_INVALID, "segs is NULL");
    int64_t full_lo = INT64_MAX, full_hi = 0, shard_lo = INT64_MAX, shard_hi = 0;
    std::vector<std::pair<int64_t, int64_t>> fr;
    for (int s = 0; s < n_segs; ++s) {
        if (segs[s].numel < 0 || segs[s].shard_off < 0 || segs[s].full_off < 0)
            return fail(ZR_ERR_INVALID, "segment %d has a negative field", s);
        if (segs[s].numel == 0) continue;
        if (segs[s].numel > kMaxElems || segs[s].shard_off > kMaxElems || segs[s].full_off > kMaxElems)
            return fail(ZR_ERR_INVALID, "segment %d has a field above 2^40", s);
        const int64_t C = (segs[s].numel + K - 1) / K;
        full_lo = std::min(full_lo, segs[s].full_off);
        full_hi = std::max(full_hi, segs[s].full_off + segs[s].numel);
        shard_lo = std::min(shard_lo, segs[s].shard_off);
        shard_hi = std::max(shard_hi, segs[s].shard_off + C);
        fr.push_back({segs[s].full_off, segs[s].full_off + segs[s].numel});
    }
    *no_work = fr.empty();
    if (fr.empty()) return ok();
    std::sort(fr.begin(), fr.end());
    for (size_t i = 1; i < fr.size(); ++i)
        if (fr[i].first < fr[i - 1].second)
            return fail(ZR_ERR_ALIAS, "two segments write overlapping full ranges");
    const int64_t es = dt_bytes(dt);
    ZR_TRY(check_table(shards, K, es, "shards"));
    ZR_TRY(check_table(const_cast<const void* const*>(fulls), K, es, "fulls"));
    std::vector<Range> rf(K), rsh(K);
    for (int r = 0; r < K; ++r) {
        rf[r] = Range{(uintptr_t)fulls[r] + (uintptr_t)(full_lo * es), (uintptr_t)fulls[r] + (uintptr_t)(full_hi * es)};
        rsh[r] = Range{(uintptr_t)shards[r] + (uintptr_t)(shard_lo * es), (uintptr_t)shards[r] + (uintptr_t)(shard_hi * es)};
    }
    ZR_TRY(check_distinct(rf, "fulls"));
    ZR_TRY(check_disjoint(rf, "fulls", rsh, "shards"));
    return ok();
}

// The prefetch coordinator's configuration; `buffers` also checks the shard
// and arena tables (zr_pf_plan needs only the sizes and the trace).
zr_status validate_pf(const zr_pf_config* c, bool buffers) {
    if (!c) return fail(ZR_ERR_INVALID, "config is NULL");
    ZR_TRY(check_k(c->K));
    if (!dt_valid(c->dtype)) return fail(ZR_ERR_UNSUPPORTED, "dtype %d not supported", (int)c->dtype);
    if (c->n_params < 1) return fail(ZR_ERR_INVALID, "n_params=%d < 1", c->n_params);
    if (!c->numels) return fail(ZR_ERR_INVALID, "numels is NULL");
    for (int p = 0; p < c->n_params; ++p)
        if (c->numels[p] < 1 || c->numels[p] > kMaxElems)
            return fail(ZR_ERR_INVALID, "numels[%d]=%lld not in [1, 2^40]", p, (long long)c->numels[p]);
    if (c->arena_numel < 1 || c->arena_numel > kMaxElems)
        return fail(ZR_ERR_INVALID, "arena_numel=%lld not in [1, 2^40]", (long long)c->arena_numel);
    if (c->chunk_shift < 0 || c->chunk_shift >= c->K)
        return fail(ZR_ERR_INVALID, "chunk_shift=%d not in [0, %d)", c->chunk_shift, c->K);
    if (c->n_steps < 1) return fail(ZR_ERR_INVALID, "n_steps=%d < 1", c->n_steps);
    if (!c->step_offsets) return fail(ZR_ERR_INVALID, "step_offsets is NULL");
    if (c->step_offsets[0] != 0) return fail(ZR_ERR_INVALID, "step_offsets[0] is not 0");
    for (int t = 0; t < c->n_steps; ++t)
        if (c->step_offsets[t + 1] < c->step_offsets[t])
            return fail(ZR_ERR_INVALID, "step_offsets decrease at step %d", t);
    const int total = c->step_offsets[c->n_steps];
    if (total > 0 && !c->step_params) return fail(ZR_ERR_INVALID, "step_params is NULL");
    for (int i = 0; i < total; ++i)
        if (c->step_params[i] < 0 || c->step_params[i] >= c->n_params)
            return fail(ZR_ERR_INVALID, "step_params[%d]=%d not a parameter id", i, c->step_params[i]);
    if (c->prefetch_bucket_numel < 1) return fail(ZR_ERR_INVALID, "prefetch_bucket_numel < 1");
    if (c->max_live_numel < 1) return fail(ZR_ERR_INVALID, "max_live_numel < 1");
    if (c->max_reuse_numel < 0) return fail(ZR_ERR_INVALID, "max_reuse_numel < 0");
    if (c->max_ongoing_fetches < 1 || c->max_ongoing_fetches > 64)
        return fail(ZR_ERR_INVALID, "max_ongoing_fetches=%d not in [1, 64]", c->max_ongoing_fetches);
    if (!buffers) return ok();
    const int K = c->K;
    const int64_t es = dt_bytes(c->dtype);
    if (!c->shard_offsets) return fail(ZR_ERR_INVALID, "shard_offsets is NULL");
    int64_t lo = INT64_MAX, hi = 0;
    for (int p = 0; p < c->n_params; ++p) {
        if (c->shard_offsets[p] < 0 || c->shard_offsets[p] > kMaxElems)
            return fail(ZR_ERR_INVALID, "shard_offsets[%d] out of range", p);
        lo = std::min(lo, c->shard_offsets[p]);
        hi = std::max(hi, c->shard_offsets[p] + (c->numels[p] + K - 1) / K);
    }
    ZR_TRY(check_table(c->shards, K, es, "shards"));
    ZR_TRY(check_table(const_cast<const void* const*>(c->arenas), K, es, "arenas"));
    std::vector<Range> ra(K), rs(K);
    for (int r = 0; r < K; ++r) {
        ra[r] = range_of(c->arenas[r], c->arena_numel, es);
        rs[r] = Range{(uintptr_t)c->shards[r] + (uintptr_t)(lo * es), (uintptr_t)c->shards[r] + (uintptr_t)(hi * es)};
    }
    ZR_TRY(check_distinct(ra, "arenas"));
    ZR_TRY(check_disjoint(ra, "arenas", rs, "shards"));
    return ok();
}

zr_status run_ag(int K, const void* const* shards, void* const* fulls, zr_dtype dt, const zr_seg* segs,
                 int n_segs, int shift, hipStream_t stream) {
    ConstPtrs sp{};
    MutPtrs fp{};
    for (int r = 0; r < K; ++r) {
        sp.p[r] = shards[r];
        fp.p[r] = fulls[r];
    }
    for (int s0 = 0; s0 < n_segs; s0 += kAgSegsPerLaunch) {
        const int n = std::min(kAgSegsPerLaunch, n_segs - s0);
        hipError_t e = launch_all_gather(K, sp, fp, dt, segs + s0, n, shift, stream);
        if (e != hipSuccess) return hip_fail(e, "all-gather launch");
    }
    return launched(hipSuccess, stream, "all-gather launch");
}

}  // namespace zr

using namespace zr;

extern "C" {

const char* zr_last_error(void) { return g_err.c_str(); }

int zr_version(void) { return 100; }  // 0.1.0

zr_status zr_reduce_scatter_avg(int K, const void* const* in, zr_dtype in_dt, int64_t N,
                                void* const* out, zr_dtype out_dt, int chunk_shift, int flags,
                                zr_order order, void* stream) {
    return zr::guarded([&]() -> zr_status {
        bool no_work = false;
        ZR_TRY(validate_rs(K, in, in_dt, N, out, out_dt, chunk_shift, flags, order, &no_work));
        if (no_work) return ok();
        return run_rs(K, in, in_dt, N, out, out_dt, chunk_shift, flags, order, (hipStream_t)stream);
    });
}

zr_status zr_all_gather(int K, const void* const* shards, void* const* fulls, zr_dtype dt,
                        const zr_seg* segs, int n_segs, int chunk_shift, void* workspace,
                        size_t ws_bytes, void* stream) {
    return zr::guarded([&]() -> zr_status {
        bool no_work = false;
        ZR_TRY(validate_ag(K, shards, fulls, dt, segs, n_segs, chunk_shift, &no_work));
        ZR_TRY(check_workspace(workspace, ws_bytes));
        if (no_work) return ok();
        hipStream_t s = (hipStream_t)stream;
        if (!workspace || n_segs <= kAgSegsPerLaunch)
            return run_ag(K, shards, fulls, dt, segs, n_segs, chunk_shift, s);
        // the staged table must not overlap the written full extents or the shards
        const int64_t es = dt_bytes(dt);
        int64_t full_lo = INT64_MAX, full_hi = 0, shard_lo = INT64_MAX, shard_hi = 0;
        for (int i = 0; i < n_segs; ++i) {
            if (segs[i].numel == 0) continue;
            full_lo = std::min(full_lo, segs[i].full_off);
            full_hi = std::max(full_hi, segs[i].full_off + segs[i].numel);
            shard_lo = std::min(shard_lo, segs[i].shard_off);
            shard_hi = std::max(shard_hi, segs[i].shard_off + (segs[i].numel + K - 1) / K);
        }
        std::vector<Range> rf(K), rsh(K);
        for (int r = 0; r < K; ++r) {
            rf[r] = Range{(uintptr_t)fulls[r] + (uintptr_t)(full_lo * es), (uintptr_t)fulls[r] + (uintptr_t)(full_hi * es)};
            rsh[r] = Range{(uintptr_t)shards[r] + (uintptr_t)(shard_lo * es), (uintptr_t)shards[r] + (uintptr_t)(shard_hi * es)};
        }
        ZR_TRY(check_staging(workspace, ws_bytes, ag_table_bytes(n_segs), rf, "fulls", rsh, "shards"));
        if (capturing(s)) return run_ag(K, shards, fulls, dt, segs, n_segs, chunk_shift, s);
        ConstPtrs sp{};
        MutPtrs fp{};
        for (int r = 0; r < K; ++r) {
            sp.p[r] = shards[r];
            fp.p[r] = fulls[r];
        }
        hipError_t e = launch_all_gather_ws(K, sp, fp, dt, segs, n_segs, chunk_shift, workspace, s);
        return launched(e, s, "all-gather launch");
    });
}

zr_status zr_allreduce(int K, const void* const* in, void* const* out, zr_dtype dt, int64_t N,
                       int average, zr_order order, int fused, void* scratch, void* stream) {
    return zr::guarded([&]() -> zr_status {
        ZR_TRY(check_k(K));
        if (N < 0) return fail(ZR_ERR_INVALID, "N=%lld is negative", (long long)N);
        if (!dt_valid(dt)) return fail(ZR_ERR_UNSUPPORTED, "dtype %d not supported", (int)dt);
        if (order != ZR_ORDER_RING && order != ZR_ORDER_FREE && order != ZR_ORDER_RING_WIRE)
            return fail(ZR_ERR_INVALID, "order=%d is not a zr_order", (int)order);
        if (N == 0) return ok();
        const int64_t es = dt_bytes(dt);
        const int64_t C = (N + K - 1) / K;
        if (N > kMaxElems) return fail(ZR_ERR_INVALID, "N=%lld too large", (long long)N);
        ZR_TRY(check_table(in, K, es, "in"));
        ZR_TRY(check_table(const_cast<const void* const*>(out), K, es, "out"));
        std::vector<Range> ri(K), ro(K);
        for (int r = 0; r < K; ++r) {
            ri[r] = range_of(in[r], N, es);
            ro[r] = range_of(out[r], N, es);
        }
        ZR_TRY(check_distinct(ro, "out"));
        for (int a = 0; a < K; ++a)
            for (int b = 0; b < K; ++b) {
                if (a == b && in[a] == out[a]) continue;
                if (overlaps(ro[a], ri[b]))
                    return fail(ZR_ERR_ALIAS, "out[%d] overlaps in[%d] (only out[r] == in[r] is allowed)", a, b);
            }
        hipStream_t s = (hipStream_t)stream;
        if (fused) {
            ConstPtrs ip{};
            MutPtrs op{};
            for (int r = 0; r < K; ++r) {
                ip.p[r] = in[r];
                op.p[r] = out[r];
            }
            hipError_t e = launch_allreduce_fused(K, ip, op, dt, N, average ? 1 : 0, order, s);
            return launched(e, s, "all-reduce launch");
        }
        if (!scratch) return fail(ZR_ERR_INVALID, "scratch is NULL (needed when fused == 0)");
        if (((uintptr_t)scratch) & (uintptr_t)(es - 1)) return fail(ZR_ERR_ALIGN, "scratch is not aligned");
        const Range rsc = range_of(scratch, K * C, es);
        for (int r = 0; r < K; ++r)
            if (overlaps(rsc, ri[r]) || overlaps(rsc, ro[r]))
                return fail(ZR_ERR_ALIAS, "scratch overlaps rank %d's buffers", r);
        std::vector<void*> sh(K);
        for (int q = 0; q < K; ++q) sh[q] = (char*)scratch + (size_t)(q * C * es);
        ZR_TRY(run_rs(K, in, dt, N, sh.data(), dt, 1 % K, average ? ZR_AVERAGE : 0, order, s));
        zr_seg seg{0, 0, N};
        return run_ag(K, const_cast<const void* const*>(sh.data()), out, dt, &seg, 1, 1 % K, s);
    });
}

}  // extern "C"

namespace zr {
namespace {

// Validates a bucket flatten and builds its launches (with `ws`: one launch
// over a table to be staged there, when more than one argument launch would
// be needed). *plan is NULL (with ZR_OK) when there is nothing to do. On
// success with a staged table, *rw holds the ranges the table must not
// overlap (buckets then fragments, split at *n_buckets).
zr_status make_flat_plan(int K, int n_frag, const void* const* frags, const int64_t* numels,
                         void* const* buckets, int64_t padded_numel, zr_dtype dt, void* ws,
                         size_t ws_bytes, FlatPlan** plan, std::vector<Range>* rb, std::vector<Range>* rf) {
    *plan = nullptr;
    ZR_TRY(check_k(K));
    if (n_frag < 0) return fail(ZR_ERR_INVALID, "n_frag=%d is negative", n_frag);
    if (!dt_valid(dt)) return fail(ZR_ERR_UNSUPPORTED, "dtype %d not supported", (int)dt);
    if (n_frag > 0 && (!frags || !numels)) return fail(ZR_ERR_INVALID, "frags or numels is NULL");
    ZR_TRY(check_workspace(ws, ws_bytes));
    const int64_t es = dt_bytes(dt);
    int64_t total = 0;
    ZR_TRY(check_sizes(numels, n_frag, &total));
    if (padded_numel > kMaxElems)
        return fail(ZR_ERR_INVALID, "padded_numel=%lld too large", (long long)padded_numel);
    if (padded_numel < total)
        return fail(ZR_ERR_INVALID, "padded_numel=%lld < total fragment size %lld", (long long)padded_numel,
                    (long long)total);
    if (padded_numel == 0) return ok();
    ZR_TRY(check_table(const_cast<const void* const*>(buckets), K, es, "buckets"));
    rb->assign(K, Range{});
    rf->clear();
    rf->reserve((size_t)K * n_frag);
    for (int r = 0; r < K; ++r) (*rb)[r] = range_of(buckets[r], padded_numel, es);
    ZR_TRY(check_distinct(*rb, "buckets"));
    for (int r = 0; r < K; ++r)
        for (int p = 0; p < n_frag; ++p) {
            const void* f = frags[(size_t)r * n_frag + p];
            if (numels[p] == 0) continue;
            if (!f) return fail(ZR_ERR_INVALID, "fragment %d of rank %d is NULL", p, r);
            if (((uintptr_t)f) & (uintptr_t)(es - 1))
                return fail(ZR_ERR_ALIGN, "fragment %d of rank %d is not aligned", p, r);
            rf->push_back(range_of(f, numels[p], es));
        }
    ZR_TRY(check_disjoint(*rb, "buckets", *rf, "fragment"));
    // one entry per non-empty fragment (every rank's copy of it), then the padding
    std::vector<FragEntry> entries;
    entries.reserve((size_t)n_frag + 1);
    int64_t off = 0;
    for (int p = 0; p < n_frag; ++p) {
        if (numels[p] > 0) {
            FragEntry f{};
            for (int r = 0; r < K; ++r) f.ptr[r] = frags[(size_t)r * n_frag + p];
            f.off = off;
            f.n = numels[p];
            entries.push_back(f);
        }
        off += numels[p];
    }
    if (padded_numel > off) {
        FragEntry f{};
        f.off = off;
        f.n = padded_numel - off;
        entries.push_back(f);
    }
    MutPtrs bp{};
    for (int r = 0; r < K; ++r) bp.p[r] = buckets[r];
    *plan = flat_plan_build(K, entries.data(), (int)entries.size(), bp, (int)es, ws);
    if (!*plan) return fail(ZR_ERR_NOMEM, "out of host memory");
    const size_t need = flat_plan_table_bytes(*plan);
    if (need > 0) {
        const zr_status st = check_staging(ws, ws_bytes, need, *rb, "buckets", *rf, "fragment");
        if (st != ZR_OK) {
            flat_plan_free(*plan);
            *plan = nullptr;
            return st;
        }
    }
    return ok();
}

// Validates a discrete reduce-scatter and builds its launches, as
// make_flat_plan does. *plan is NULL (with ZR_OK) when N == 0.
zr_status make_frags_plan(int K, int n_frag, const void* const* frags, const int64_t* numels,
                          int64_t N, zr_dtype in_dt, void* const* out, zr_dtype out_dt,
                          int chunk_shift, int flags, zr_order order, void* ws, size_t ws_bytes,
                          RsfPlan** plan) {
    *plan = nullptr;
    ZR_TRY(check_k(K));
    if (n_frag < 0) return fail(ZR_ERR_INVALID, "n_frag=%d is negative", n_frag);
    if (N < 0) return fail(ZR_ERR_INVALID, "N=%lld is negative", (long long)N);
    if (!dt_valid(in_dt) || !dt_valid(out_dt))
        return fail(ZR_ERR_UNSUPPORTED, "dtype pair (%d, %d) not supported", (int)in_dt, (int)out_dt);
    if (chunk_shift < 0 || chunk_shift >= K)
        return fail(ZR_ERR_INVALID, "chunk_shift=%d not in [0, %d)", chunk_shift, K);
    if (flags & ~(ZR_AVERAGE | ZR_ACCUMULATE)) return fail(ZR_ERR_INVALID, "flags=%d has unknown bits", flags);
    if (order != ZR_ORDER_RING && order != ZR_ORDER_FREE && order != ZR_ORDER_RING_WIRE)
        return fail(ZR_ERR_INVALID, "order=%d is not a zr_order", (int)order);
    if (n_frag > 0 && (!frags || !numels)) return fail(ZR_ERR_INVALID, "frags or numels is NULL");
    ZR_TRY(check_workspace(ws, ws_bytes));
    int64_t total = 0;
    ZR_TRY(check_sizes(numels, n_frag, &total));
    if (N < total)
        return fail(ZR_ERR_INVALID, "N=%lld < total fragment size %lld", (long long)N, (long long)total);
    if (N == 0) return ok();
    if (N > kMaxElems) return fail(ZR_ERR_INVALID, "N=%lld too large", (long long)N);
    const int64_t ies = dt_bytes(in_dt), oes = dt_bytes(out_dt);
    const int64_t C = (N + K - 1) / K;
    ZR_TRY(check_table(const_cast<const void* const*>(out), K, oes, "out"));
    std::vector<Range> ro(K), rf;
    for (int r = 0; r < K; ++r) ro[r] = range_of(out[r], C, oes);
    ZR_TRY(check_distinct(ro, "out"));
    for (int r = 0; r < K; ++r)
        for (int p = 0; p < n_frag; ++p) {
            if (numels[p] == 0) continue;
            const void* f = frags[(size_t)r * n_frag + p];
            if (!f) return fail(ZR_ERR_INVALID, "fragment %d of rank %d is NULL", p, r);
            if (((uintptr_t)f) & (uintptr_t)(ies - 1))
                return fail(ZR_ERR_ALIGN, "fragment %d of rank %d is not aligned", p, r);
            rf.push_back(range_of(f, numels[p], ies));
        }
    ZR_TRY(check_disjoint(ro, "out", rf, "fragment"));
    std::vector<FragEntry> entries;
    entries.reserve((size_t)n_frag + 1);
    int64_t off = 0;
    for (int p = 0; p < n_frag; ++p) {
        if (numels[p] > 0) {
            FragEntry e{};
            for (int r = 0; r < K; ++r) e.ptr[r] = frags[(size_t)r * n_frag + p];
            e.off = off;
            e.n = numels[p];
            entries.push_back(e);
        }
        off += numels[p];
    }
    // the zero padding: null pointers, up to the end of the last chunk (K*C),
    // where the contiguous reduce-scatter also writes +0 past N
    if (K * C > off) {
        FragEntry e{};
        e.off = off;
        e.n = K * C - off;
        entries.push_back(e);
    }
    MutPtrs op{};
    for (int r = 0; r < K; ++r) op.p[r] = out[r];
    *plan = rsf_plan_build(K, entries.data(), (int)entries.size(), N, in_dt, op, out_dt, chunk_shift,
                           flags, order, ws);
    if (!*plan) return fail(ZR_ERR_NOMEM, "out of host memory");
    const size_t need = rsf_plan_table_bytes(*plan);
    if (need > 0) {
        const zr_status st = check_staging(ws, ws_bytes, need, ro, "out", rf, "fragment");
        if (st != ZR_OK) {
            rsf_plan_free(*plan);
            *plan = nullptr;
            return st;
        }
    }
    return ok();
}

// A plan built for one call: launched once (after staging its table on the
// stream), then freed.
template <typename Plan, typename Build, typename Bytes, typename Image, typename Launch, typename Free>
zr_status run_once(Build build, Bytes bytes, Image image, Launch launch, Free free_plan, void* ws,
                   hipStream_t s, const char* what) {
    Plan* plan = nullptr;
    ZR_TRY(build(ws, &plan));
    if (!plan) return ok();
    if (bytes(plan) > 0 && capturing(s)) {
        // no asynchronous copy from a host buffer into a graph: argument launches
        free_plan(plan);
        plan = nullptr;
        ZR_TRY(build(nullptr, &plan));
        if (!plan) return ok();
    }
    hipError_t e = stage_table(ws, image(plan), bytes(plan), s, true);
    if (e == hipSuccess) e = launch(plan, s);
    free_plan(plan);
    return launched(e, s, what);
}

}  // namespace
}  // namespace zr

struct zr_rsf_plan {
    zr::RsfPlan* plan;  // NULL: nothing to launch
};

struct zr_flatten_plan {
    zr::FlatPlan* plan;  // NULL: nothing to launch
};

struct zr_rs_plan {
    zr::RsPlan* plan;  // NULL: nothing to launch (N == 0)
};

extern "C" {

size_t zr_workspace_bytes(int K, int n) {
    if (K < 1 || K > kMaxRanks || n < 0) return 0;
    // the flatten and the discrete reduce-scatter carry min(32, 256 / K)
    // fragments per argument block, the all-gather 32 segments
    const int fit = std::min(kRsfEntriesPerLaunch, kRsfPtrsPerLaunch / K);
    if (n <= fit) return 0;
    const int64_t nent = (int64_t)n + 1;  // the fragments and the padding
    const int64_t nseg = (int64_t)n + K;  // each of the K - 1 chunk boundaries splits one entry at most
    const size_t b = std::max({rsf_table_bytes(K, nent, nseg), flatten_table_bytes(K, nent), ag_table_bytes(n)});
    return (b + kWsAlign - 1) / kWsAlign * kWsAlign;
}

zr_status zr_flatten_bucket(int K, int n_frag, const void* const* frags, const int64_t* numels,
                            void* const* buckets, int64_t padded_numel, zr_dtype dt, void* workspace,
                            size_t ws_bytes, void* stream) {
    return zr::guarded([&]() -> zr_status {
        std::vector<Range> rb, rf;
        auto build = [&](void* ws, FlatPlan** p) {
            return make_flat_plan(K, n_frag, frags, numels, buckets, padded_numel, dt, ws, ws_bytes, p, &rb, &rf);
        };
        return run_once<FlatPlan>(build, flat_plan_table_bytes, flat_plan_table_image, flat_plan_launch,
                                  flat_plan_free, workspace, (hipStream_t)stream, "flatten launch");
    });
}

zr_status zr_flatten_plan_create(int K, int n_frag, const void* const* frags, const int64_t* numels,
                                 void* const* buckets, int64_t padded_numel, zr_dtype dt, void* workspace,
                                 size_t ws_bytes, zr_flatten_plan** plan) {
    return zr::guarded([&]() -> zr_status {
        if (!plan) return fail(ZR_ERR_INVALID, "plan is NULL");
        *plan = nullptr;
        FlatPlan* p = nullptr;
        std::vector<Range> rb, rf;
        ZR_TRY(make_flat_plan(K, n_frag, frags, numels, buckets, padded_numel, dt, workspace, ws_bytes, &p, &rb,
                              &rf));
        if (p && flat_plan_table_bytes(p) > 0) {
            const hipError_t e = stage_table(workspace, flat_plan_table_image(p), flat_plan_table_bytes(p), nullptr,
                                             false);
            if (e != hipSuccess) {
                flat_plan_free(p);
                return hip_fail(e, "staging the flatten table");
            }
        }
        zr_flatten_plan* h = new (std::nothrow) zr_flatten_plan{p};
        if (!h) {
            if (p) flat_plan_free(p);
            return fail(ZR_ERR_NOMEM, "out of host memory");
        }
        *plan = h;
        return ok();
    });
}

zr_status zr_flatten_plan_launch(const zr_flatten_plan* plan, void* stream) {
    if (!plan) return fail(ZR_ERR_INVALID, "plan is NULL");
    if (!plan->plan) return ok();
    const hipError_t e = flat_plan_launch(plan->plan, (hipStream_t)stream);
    return launched(e, (hipStream_t)stream, "flatten launch");
}

zr_status zr_flatten_plan_info(const zr_flatten_plan* plan, int* launches, size_t* table_bytes) {
    if (!plan) return fail(ZR_ERR_INVALID, "plan is NULL");
    if (launches) *launches = plan->plan ? flat_plan_launch_count(plan->plan) : 0;
    if (table_bytes) *table_bytes = plan->plan ? flat_plan_table_bytes(plan->plan) : 0;
    return ok();
}

zr_status zr_flatten_plan_destroy(zr_flatten_plan* plan) {
    if (!plan) return ok();
    if (plan->plan) flat_plan_free(plan->plan);
    delete plan;
    return ok();
}

zr_status zr_reduce_scatter_frags(int K, int n_frag, const void* const* frags,
                                  const int64_t* numels, int64_t N, zr_dtype in_dt,
                                  void* const* out, zr_dtype out_dt, int chunk_shift, int flags,
                                  zr_order order, void* workspace, size_t ws_bytes, void* stream) {
    return zr::guarded([&]() -> zr_status {
        auto build = [&](void* ws, RsfPlan** p) {
            return make_frags_plan(K, n_frag, frags, numels, N, in_dt, out, out_dt, chunk_shift, flags, order, ws,
                                   ws_bytes, p);
        };
        return run_once<RsfPlan>(build, rsf_plan_table_bytes, rsf_plan_table_image, rsf_plan_launch, rsf_plan_free,
                                 workspace, (hipStream_t)stream, "discrete reduce-scatter launch");
    });
}

zr_status zr_rs_plan_create(int K, const void* const* in, zr_dtype in_dt, int64_t N, void* const* out,
                            zr_dtype out_dt, int chunk_shift, int flags, zr_order order, zr_rs_plan** plan) {
    return zr::guarded([&]() -> zr_status {
        if (!plan) return fail(ZR_ERR_INVALID, "plan is NULL");
        *plan = nullptr;
        bool no_work = false;
        ZR_TRY(validate_rs(K, in, in_dt, N, out, out_dt, chunk_shift, flags, order, &no_work));
        RsPlan* p = nullptr;
        if (!no_work) {
            ConstPtrs ip{};
            MutPtrs op{};
            for (int r = 0; r < K; ++r) {
                ip.p[r] = in[r];
                op.p[r] = out[r];
            }
            p = rs_plan_build(K, ip, in_dt, N, op, out_dt, chunk_shift, flags, order);
            if (!p) return fail(ZR_ERR_NOMEM, "out of host memory");
        }
        zr_rs_plan* h = new (std::nothrow) zr_rs_plan{p};
        if (!h) {
            if (p) rs_plan_free(p);
            return fail(ZR_ERR_NOMEM, "out of host memory");
        }
        *plan = h;
        return ok();
    });
}

zr_status zr_rs_plan_launch(const zr_rs_plan* plan, void* stream) {
    if (!plan) return fail(ZR_ERR_INVALID, "plan is NULL");
    if (!plan->plan) return ok();
    const hipError_t e = rs_plan_launch(plan->plan, (hipStream_t)stream);
    return launched(e, (hipStream_t)stream, "reduce-scatter launch");
}

zr_status zr_rs_plan_destroy(zr_rs_plan* plan) {
    if (!plan) return ok();
    if (plan->plan) rs_plan_free(plan->plan);
    delete plan;
    return ok();
}

zr_status zr_reduce_scatter_frags_noalloc(int K, int n_frag, const void* const* frags,
                                          const int64_t* numels, int64_t N, zr_dtype in_dt,
                                          void* const* out, zr_dtype out_dt, int chunk_shift,
                                          int flags, zr_order order, void* stream) {
    return zr::guarded([&]() -> zr_status {
        // validation first: the same checks as the one-shot call, on the host
        RsfPlan* probe = nullptr;
        ZR_TRY(make_frags_plan(K, n_frag, frags, numels, N, in_dt, out, out_dt, chunk_shift, flags, order, nullptr,
                               0, &probe));
        if (!probe) return ok();
        const bool one_launch = rsf_plan_launch_count(probe) <= 1;
        rsf_plan_free(probe);
        void* ws = nullptr;
        if (!one_launch) {
            const hipError_t e = noalloc_scratch(&ws);
            if (e != hipSuccess) return hip_fail(e, "looking up the staging array");
        }
        auto build = [&](void* w, RsfPlan** p) {
            const zr_status st = make_frags_plan(K, n_frag, frags, numels, N, in_dt, out, out_dt, chunk_shift, flags,
                                                 order, w, ZR_NOALLOC_TABLE_BYTES, p);
            if (st == ZR_ERR_WORKSPACE)
                return fail(ZR_ERR_WORKSPACE,
                            "the table of %d fragments at K=%d needs more than the %d bytes this entry point "
                            "stages (zr_workspace_bytes(K, n_frag) <= %d is always accepted)",
                            n_frag, K, ZR_NOALLOC_TABLE_BYTES, ZR_NOALLOC_TABLE_BYTES);
            return st;
        };
        return run_once<RsfPlan>(build, rsf_plan_table_bytes, rsf_plan_table_image, rsf_plan_launch, rsf_plan_free,
                                 ws, (hipStream_t)stream, "discrete reduce-scatter launch");
    });
}

zr_status zr_rsf_plan_create(int K, int n_frag, const void* const* frags, const int64_t* numels,
                             int64_t N, zr_dtype in_dt, void* const* out, zr_dtype out_dt,
                             int chunk_shift, int flags, zr_order order, void* workspace,
                             size_t ws_bytes, zr_rsf_plan** plan) {
    return zr::guarded([&]() -> zr_status {
        if (!plan) return fail(ZR_ERR_INVALID, "plan is NULL");
        *plan = nullptr;
        RsfPlan* p = nullptr;
        ZR_TRY(make_frags_plan(K, n_frag, frags, numels, N, in_dt, out, out_dt, chunk_shift, flags, order,
                               workspace, ws_bytes, &p));
        if (p && rsf_plan_table_bytes(p) > 0) {
            const hipError_t e = stage_table(workspace, rsf_plan_table_image(p), rsf_plan_table_bytes(p), nullptr,
                                             false);
            if (e != hipSuccess) {
                rsf_plan_free(p);
                return hip_fail(e, "staging the discrete reduce-scatter table");
            }
        }
        zr_rsf_plan* h = new (std::nothrow) zr_rsf_plan{p};
        if (!h) {
            if (p) rsf_plan_free(p);
            return fail(ZR_ERR_NOMEM, "out of host memory");
        }
        *plan = h;
        return ok();
    });
}

zr_status zr_rsf_plan_launch(const zr_rsf_plan* plan, void* stream) {
    if (!plan) return fail(ZR_ERR_INVALID, "plan is NULL");
    if (!plan->plan) return ok();
    const hipError_t e = rsf_plan_launch(plan->plan, (hipStream_t)stream);
    return launched(e, (hipStream_t)stream, "discrete reduce-scatter launch");
}

zr_status zr_rsf_plan_info(const zr_rsf_plan* plan, int* launches, size_t* table_bytes) {
    if (!plan) return fail(ZR_ERR_INVALID, "plan is NULL");
    if (launches) *launches = plan->plan ? rsf_plan_launch_count(plan->plan) : 0;
    if (table_bytes) *table_bytes = plan->plan ? rsf_plan_table_bytes(plan->plan) : 0;
    return ok();
}

zr_status zr_rsf_plan_destroy(zr_rsf_plan* plan) {
    if (!plan) return ok();
    if (plan->plan) rsf_plan_free(plan->plan);
    delete plan;
    return ok();
}

zr_status zr_plan_buckets(int n, const int64_t* numels, int64_t cap, int32_t* bucket_of,
                          int32_t* n_buckets) {
    if (n < 0) return fail(ZR_ERR_INVALID, "n=%d is negative", n);
    if (cap < 1) return fail(ZR_ERR_INVALID, "cap=%lld < 1", (long long)cap);
    if (!n_buckets || (n > 0 && (!numels || !bucket_of)))
        return fail(ZR_ERR_INVALID, "NULL argument");
    int32_t b = -1;
    int64_t total = 0;
    for (int i = 0; i < n; ++i) {
        if (numels[i] < 0 || numels[i] > kMaxElems)
            return fail(ZR_ERR_INVALID, "numels[%d]=%lld not in [0, 2^40]", i, (long long)numels[i]);
        if (b < 0 || total >= cap) {
            ++b;
            total = 0;
        }
        bucket_of[i] = b;
        total += numels[i];
    }
    *n_buckets = b + 1;
    return ok();
}

}  // extern "C"
