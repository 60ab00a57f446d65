// Test harness: the prefetch coordinator core
// (gradient_sync_zr_amd/csrc/prefetch_core.hpp) driven by a backend that
// only logs what it is asked to do. Event queries are answered by a callback
// (the Python replay knows when each gather finishes). The Python tests
// replay the log on a discrete-event model of streams, events and host time.
// Test infrastructure only; built with g++, no HIP.
#include <cstddef>
#include <cstdint>
#include <new>
#include <vector>

#include "prefetch_core.hpp"

namespace {

enum Op { kCreate = 1, kDestroy = 2, kRecord = 3, kWait = 4, kSync = 5, kGather = 6 };

typedef int (*QueryFn)(int event);

// Log records: (op, a, b) triples; a gather is (kGather, stream, n) followed
// by n (param, offset) pairs.
struct LogBackend {
    using Stream = int;
    using Event = int;
    std::vector<int64_t> log;
    int next_event = 1;
    int fail_on_call = -1;  // make the n-th backend call fail (0-based)
    int calls = 0;
    QueryFn query_fn = nullptr;
    bool tick() { return fail_on_call >= 0 && calls++ == fail_on_call; }
    void put(int64_t op, int64_t a, int64_t b) {
        log.push_back(op);
        log.push_back(a);
        log.push_back(b);
    }
    int create(Event* e) {
        if (tick()) return 1;
        *e = next_event++;
        put(kCreate, *e, 0);
        return 0;
    }
    int destroy(Event e) {
        put(kDestroy, e, 0);
        return 0;
    }
    int record(Event e, Stream s) {
        if (tick()) return 1;
        put(kRecord, e, s);
        return 0;
    }
    int wait(Stream s, Event e) {
        if (tick()) return 1;
        put(kWait, s, e);
        return 0;
    }
    int query(Event e, bool* done) {
        if (tick()) return 1;
        *done = query_fn ? query_fn(e) != 0 : false;
        return 0;
    }
    int sync(Event e) {
        if (tick()) return 1;
        put(kSync, e, 0);
        return 0;
    }
    int gather(Stream s, const int* params, const int64_t* offs, int n) {
        if (tick()) return 1;
        put(kGather, s, n);
        for (int i = 0; i < n; ++i) {
            log.push_back(params[i]);
            log.push_back(offs[i]);
        }
        return 0;
    }
};

struct Sim {
    LogBackend be;
    zr::PrefetchCore<LogBackend> core;
    Sim() : core(be) {}
};

}  // namespace

extern "C" {

// cfg64: bucket, max_live, max_reuse, arena, align; cfg32: max_ongoing,
// gather stream, compute stream, fail_on_call.
void* pf_create(int n_params, const int64_t* numels, int n_steps, const int32_t* step_off,
                const int32_t* step_params, const int64_t* cfg64, const int32_t* cfg32,
                QueryFn query, int* err) {
    Sim* s = new (std::nothrow) Sim();
    if (!s) return nullptr;
    s->be.fail_on_call = cfg32[3];
    s->be.query_fn = query;
    zr::PrefetchCore<LogBackend>::Config c;
    c.n_params = n_params;
    c.numels = numels;
    c.n_steps = n_steps;
    c.step_off = step_off;
    c.step_params = step_params;
    c.bucket = cfg64[0];
    c.max_live = cfg64[1];
    c.max_reuse = cfg64[2];
    c.arena = cfg64[3];
    c.align = cfg64[4];
    c.max_ongoing = cfg32[0];
    c.gather = cfg32[1];
    c.compute = cfg32[2];
    *err = (int)s->core.init(c);
    return s;
}

int pf_fetch(void* h, int step) { return (int)static_cast<Sim*>(h)->core.fetch(step); }
int pf_release(void* h, int step) { return (int)static_cast<Sim*>(h)->core.release(step); }
int64_t pf_offset(void* h, int param) { return static_cast<Sim*>(h)->core.offset_of(param); }

// live, peak_live, gathers, immediate_gathers, host_syncs, retained, prefetch_trimmed
void pf_stats(void* h, int64_t* out) {
    const zr::PfStats& s = static_cast<Sim*>(h)->core.stats();
    out[0] = s.live;
    out[1] = s.peak_live;
    out[2] = s.gathers;
    out[3] = s.immediate_gathers;
    out[4] = s.host_syncs;
    out[5] = s.retained;
    out[6] = s.prefetch_trimmed;
}

int64_t pf_log_size(void* h) { return (int64_t)static_cast<Sim*>(h)->be.log.size(); }

void pf_log(void* h, int64_t* out) {
    Sim* s = static_cast<Sim*>(h);
    for (size_t i = 0; i < s->be.log.size(); ++i) out[i] = s->be.log[i];
}

// The core's destroy() alone (its log stays readable); pf_destroy frees.
void pf_shutdown(void* h) { static_cast<Sim*>(h)->core.destroy(); }

void pf_destroy(void* h) {
    Sim* s = static_cast<Sim*>(h);
    s->core.destroy();
    delete s;
}

}  // extern "C"
