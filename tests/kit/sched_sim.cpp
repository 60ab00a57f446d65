// Test harness: the scheduler core (gradient_sync_zr_amd/csrc/sched_core.hpp)
// driven by a backend that only logs what it is asked to do. The Python
// tests replay the log on a discrete-event model of streams and events.
// Test infrastructure only; built with g++, no HIP.
#include <cstddef>
#include <cstdint>
#include <new>
#include <vector>

#include "sched_core.hpp"

namespace {

enum Op { kCreate = 1, kDestroy = 2, kRecord = 3, kWait = 4, kLaunch = 5 };

struct LogBackend {
    using Stream = int;
    using Event = int;
    std::vector<int64_t> log;  // triples (op, a, b)
    int next_event = 1;
    int fail_on_call = -1;     // make the n-th backend call fail (0-based)
    int calls = 0;
    bool tick() { return fail_on_call >= 0 && calls++ == fail_on_call; }
    void put(int op, int64_t a, int64_t b) {
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
};

struct Sim {
    LogBackend be;
    zr::SchedCore<LogBackend> core;
    explicit Sim(int red) : core(be, red) {}
};

}  // namespace

extern "C" {

void* sim_create(int n_buffers, int max_producers, int reduction_stream, int fail_on_call, int* err) {
    Sim* s = new (std::nothrow) Sim(reduction_stream);
    if (!s) return nullptr;
    s->be.fail_on_call = fail_on_call;
    *err = (int)s->core.init(n_buffers, max_producers);
    return s;
}

int sim_acquire(void* h, int buf, int producer) {
    return (int)static_cast<Sim*>(h)->core.acquire(buf, producer);
}

// `launch_ok` = 0 makes the launch itself fail.
int sim_submit(void* h, int buf, const int* producers, int n_prod, int launch_ok) {
    Sim* s = static_cast<Sim*>(h);
    return (int)s->core.submit(buf, producers, n_prod, [&](int red) {
        if (!launch_ok) return false;
        s->be.put(kLaunch, buf, red);
        return true;
    });
}

int sim_flush(void* h, int caller) { return (int)static_cast<Sim*>(h)->core.flush(caller); }

int64_t sim_log_size(void* h) { return (int64_t)static_cast<Sim*>(h)->be.log.size(); }

void sim_log(void* h, int64_t* out) {
    Sim* s = static_cast<Sim*>(h);
    for (size_t i = 0; i < s->be.log.size(); ++i) out[i] = s->be.log[i];
}

void sim_destroy(void* h) {
    Sim* s = static_cast<Sim*>(h);
    s->core.release();
    delete s;
}

}  // extern "C"
