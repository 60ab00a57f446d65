// C-ABI of the bucket/stream scheduler: SchedCore driven by HIP events.
#include <hip/hip_runtime.h>

#include <memory>

#include "zr_guard.hpp"

#include "sched_core.hpp"
#include "zr.h"
#include "zr_internal.hpp"

namespace zr {
zr_status validate_rs(int K, const void* const* in, zr_dtype in_dt, int64_t N, void* const* out,
                      zr_dtype out_dt, int shift, int flags, zr_order order, bool* no_work);
zr_status run_rs(int K, const void* const* in, zr_dtype in_dt, int64_t N, void* const* out,
                 zr_dtype out_dt, int shift, int flags, zr_order order, hipStream_t stream);
zr_status set_error(zr_status st, const char* msg);

namespace {
struct HipBackend {
    using Stream = hipStream_t;
    using Event = hipEvent_t;
    hipError_t last = hipSuccess;
    int create(Event* e) { return (last = hipEventCreateWithFlags(e, hipEventDisableTiming)) != hipSuccess; }
    int destroy(Event e) { return (last = hipEventDestroy(e)) != hipSuccess; }
    int record(Event e, Stream s) { return (last = hipEventRecord(e, s)) != hipSuccess; }
    int wait(Stream s, Event e) { return (last = hipStreamWaitEvent(s, e, 0)) != hipSuccess; }
};
}  // namespace
}  // namespace zr

struct zr_sched {
    zr::HipBackend be;
    zr::SchedCore<zr::HipBackend> core;
    explicit zr_sched(hipStream_t red) : core(be, red) {}
};

namespace {

zr_status map_err(zr_sched* s, zr::SchedErr e, const char* what) {
    switch (e) {
        case zr::SchedErr::kOk: return ZR_OK;
        case zr::SchedErr::kBadBuf: return zr::set_error(ZR_ERR_INVALID, "buffer index out of range");
        case zr::SchedErr::kBadState:
            return zr::set_error(ZR_ERR_INVALID,
                                 "buffer state: acquire twice without submit, or submit without acquire");
        case zr::SchedErr::kTooManyProducers:
            return zr::set_error(ZR_ERR_INVALID, "more producer streams than max_producers");
        case zr::SchedErr::kBadArg: return zr::set_error(ZR_ERR_INVALID, what);
        case zr::SchedErr::kBackend:
        default: return zr::set_error(ZR_ERR_HIP, s ? hipGetErrorString(s->be.last) : what);
    }
}

}  // namespace

extern "C" {

zr_status zr_sched_create(zr_sched** out, int n_buffers, int max_producers, void* reduction_stream) {
    return zr::guarded([&]() -> zr_status {
        if (!out) return zr::set_error(ZR_ERR_INVALID, "out is NULL");
        *out = nullptr;
        if (n_buffers < 1 || n_buffers > 64) return zr::set_error(ZR_ERR_INVALID, "n_buffers not in [1, 64]");
        if (max_producers < 0 || max_producers > 64)
            return zr::set_error(ZR_ERR_INVALID, "max_producers not in [0, 64]");
        std::unique_ptr<zr_sched> s(new zr_sched((hipStream_t)reduction_stream));
        zr::SchedErr e = s->core.init(n_buffers, max_producers);
        if (e != zr::SchedErr::kOk) return map_err(s.get(), e, "init");
        *out = s.release();
        return ZR_OK;
    });
}

zr_status zr_sched_acquire(zr_sched* s, int buf, void* producer_stream) {
    return zr::guarded([&]() -> zr_status {
        if (!s) return zr::set_error(ZR_ERR_INVALID, "scheduler is NULL");
        return map_err(s, s->core.acquire(buf, (hipStream_t)producer_stream), "acquire");
    });
}

zr_status zr_sched_submit_rs(zr_sched* s, int buf, void* const* producer_streams, int n_prod, int K,
                             const void* const* in, zr_dtype in_dt, int64_t N, void* const* out,
                             zr_dtype out_dt, int chunk_shift, int flags, zr_order order) {
    return zr::guarded([&]() -> zr_status {
        if (!s) return zr::set_error(ZR_ERR_INVALID, "scheduler is NULL");
        bool no_work = false;
        zr_status st = zr::validate_rs(K, in, in_dt, N, out, out_dt, chunk_shift, flags, order, &no_work);
        if (st != ZR_OK) return st;
        zr_status launch_st = ZR_OK;
        auto launch = [&](hipStream_t red) {
            if (no_work) return true;
            launch_st = zr::run_rs(K, in, in_dt, N, out, out_dt, chunk_shift, flags, order, red);
            return launch_st == ZR_OK;
        };
        zr::SchedErr e = s->core.submit(buf, reinterpret_cast<const hipStream_t*>(producer_streams), n_prod, launch);
        if (e == zr::SchedErr::kBackend && launch_st != ZR_OK) return launch_st;
        return map_err(s, e, "submit");
    });
}

zr_status zr_sched_flush(zr_sched* s, void* caller_stream) {
    return zr::guarded([&]() -> zr_status {
        if (!s) return zr::set_error(ZR_ERR_INVALID, "scheduler is NULL");
        return map_err(s, s->core.flush((hipStream_t)caller_stream), "flush");
    });
}

zr_status zr_sched_destroy(zr_sched* s) {
    delete s;
    return ZR_OK;
}

}  // extern "C"
