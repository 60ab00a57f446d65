// C-ABI of the ZeRO-3 prefetch coordinator: PrefetchCore driven by HIP
// events and the all-gather kernel, or (zr_pf_plan) by a backend whose
// gathers finish at once, to size an arena on the host.
#include <hip/hip_runtime.h>

#include <memory>
#include <vector>

#include "prefetch_core.hpp"
#include "zr_guard.hpp"
#include "zr.h"
#include "zr_internal.hpp"

namespace zr {
zr_status validate_pf(const zr_pf_config* c, bool buffers);
zr_status run_ag(int K, const void* const* shards, void* const* fulls, zr_dtype dt, const zr_seg* segs,
                 int n_segs, int shift, hipStream_t stream);
zr_status set_error(zr_status st, const char* msg);

namespace {

// Gathers go to zr_all_gather's kernel: parameter p's shard at
// shard_offsets[p] of every rank's shard buffer, its full copy at the arena
// offset the coordinator chose.
struct PfHip {
    using Stream = hipStream_t;
    using Event = hipEvent_t;
    hipError_t last = hipSuccess;
    zr_status gather_st = ZR_OK;
    int K = 0, shift = 0;
    zr_dtype dt = ZR_BF16;
    std::vector<const void*> shards;
    std::vector<void*> arenas;
    std::vector<int64_t> numels, shard_off;
    std::vector<zr_seg> segs;

    int create(Event* e) { return (last = hipEventCreateWithFlags(e, hipEventDisableTiming)) != hipSuccess; }
    int destroy(Event e) { return (last = hipEventDestroy(e)) != hipSuccess; }
    int record(Event e, Stream s) { return (last = hipEventRecord(e, s)) != hipSuccess; }
    int wait(Stream s, Event e) { return (last = hipStreamWaitEvent(s, e, 0)) != hipSuccess; }
    int query(Event e, bool* done) {
        const hipError_t r = hipEventQuery(e);
        if (r == hipSuccess || r == hipErrorNotReady) {
            *done = r == hipSuccess;
            return 0;
        }
        last = r;
        return 1;
    }
    int sync(Event e) { return (last = hipEventSynchronize(e)) != hipSuccess; }
    int gather(Stream s, const int* params, const int64_t* offs, int n) {
        segs.resize(n);
        for (int i = 0; i < n; ++i) segs[i] = zr_seg{shard_off[params[i]], offs[i], numels[params[i]]};
        gather_st = run_ag(K, shards.data(), arenas.data(), dt, segs.data(), n, shift, s);
        return gather_st != ZR_OK;
    }
};

struct PfNull {
    using Stream = int;
    using Event = int;
    int create(Event* e) {
        *e = 0;
        return 0;
    }
    int destroy(Event) { return 0; }
    int record(Event, Stream) { return 0; }
    int wait(Stream, Event) { return 0; }
    int query(Event, bool* done) {
        *done = true;
        return 0;
    }
    int sync(Event) { return 0; }
    int gather(Stream, const int*, const int64_t*, int) { return 0; }
};

template <class Core>
typename Core::Config core_config(const zr_pf_config* c, typename Core::Stream g, typename Core::Stream s) {
    typename Core::Config k;
    k.n_params = c->n_params;
    k.numels = c->numels;
    k.n_steps = c->n_steps;
    k.step_off = c->step_offsets;
    k.step_params = c->step_params;
    k.bucket = c->prefetch_bucket_numel;
    k.max_live = c->max_live_numel;
    k.max_reuse = c->max_reuse_numel;
    k.arena = c->arena_numel;
    k.align = 256 / (c->dtype == ZR_BF16 ? 2 : 4);
    k.max_ongoing = c->max_ongoing_fetches;
    k.gather = g;
    k.compute = s;
    return k;
}

void copy_stats(const PfStats& s, zr_pf_stats* o) {
    o->gathers = s.gathers;
    o->immediate_gathers = s.immediate_gathers;
    o->immediate_numel = s.immediate_numel;
    o->prefetch_numel = s.prefetch_numel;
    o->host_syncs = s.host_syncs;
    o->stream_waits = s.stream_waits;
    o->live = s.live;
    o->peak_live = s.peak_live;
    o->peak_ongoing = s.peak_ongoing;
    o->arena_peak = s.arena_peak;
    o->prefetch_trimmed = s.prefetch_trimmed;
    o->retained = s.retained;
}

}  // namespace
}  // namespace zr

struct zr_pf {
    zr::PfHip be;
    zr::PrefetchCore<zr::PfHip> core;
    int64_t es = 2;
    zr_pf() : core(be) {}
};

namespace {

zr_status map_err(const zr::PfHip* be, zr::PfErr e, const char* what) {
    switch (e) {
        case zr::PfErr::kOk: return ZR_OK;
        case zr::PfErr::kBadArg: return zr::set_error(ZR_ERR_INVALID, what);
        case zr::PfErr::kBadState:
            return zr::set_error(ZR_ERR_INVALID, "steps must be fetched, then released, in trace order");
        case zr::PfErr::kNoMemory:
            return zr::set_error(ZR_ERR_NOMEM, "the arena cannot hold the parameters that must be live");
        case zr::PfErr::kBackend:
        default:
            if (be && be->gather_st != ZR_OK) return be->gather_st;
            return zr::set_error(ZR_ERR_HIP, be ? hipGetErrorString(be->last) : what);
    }
}

}  // namespace

extern "C" {

zr_status zr_pf_create(const zr_pf_config* cfg, zr_pf** out) {
    return zr::guarded([&]() -> zr_status {
        if (!out) return zr::set_error(ZR_ERR_INVALID, "out is NULL");
        *out = nullptr;
        zr_status st = zr::validate_pf(cfg, true);
        if (st != ZR_OK) return st;
        std::unique_ptr<zr_pf> pf(new zr_pf());
        zr::PfHip& be = pf->be;
        be.K = cfg->K;
        be.shift = cfg->chunk_shift;
        be.dt = cfg->dtype;
        be.shards.assign(cfg->shards, cfg->shards + cfg->K);
        be.arenas.assign(cfg->arenas, cfg->arenas + cfg->K);
        be.numels.assign(cfg->numels, cfg->numels + cfg->n_params);
        be.shard_off.assign(cfg->shard_offsets, cfg->shard_offsets + cfg->n_params);
        pf->es = cfg->dtype == ZR_BF16 ? 2 : 4;
        zr::PfErr e = pf->core.init(zr::core_config<zr::PrefetchCore<zr::PfHip>>(
            cfg, (hipStream_t)cfg->gather_stream, (hipStream_t)cfg->compute_stream));
        if (e != zr::PfErr::kOk) return map_err(&pf->be, e, "invalid trace");
        *out = pf.release();
        return ZR_OK;
    });
}

zr_status zr_pf_fetch(zr_pf* pf, int step) {
    return zr::guarded([&]() -> zr_status {
        if (!pf) return zr::set_error(ZR_ERR_INVALID, "coordinator is NULL");
        pf->be.gather_st = ZR_OK;
        return map_err(&pf->be, pf->core.fetch(step), "step out of range");
    });
}

zr_status zr_pf_release(zr_pf* pf, int step) {
    return zr::guarded([&]() -> zr_status {
        if (!pf) return zr::set_error(ZR_ERR_INVALID, "coordinator is NULL");
        return map_err(&pf->be, pf->core.release(step), "step out of range");
    });
}

zr_status zr_pf_full(const zr_pf* pf, int param, int rank, void** full) {
    if (!pf || !full) return zr::set_error(ZR_ERR_INVALID, "NULL argument");
    if (rank < 0 || rank >= pf->be.K) return zr::set_error(ZR_ERR_INVALID, "rank out of range");
    const int64_t off = pf->core.offset_of(param);
    if (off < 0) return zr::set_error(ZR_ERR_INVALID, "parameter is not live");
    *full = static_cast<char*>(pf->be.arenas[rank]) + off * pf->es;
    return ZR_OK;
}

zr_status zr_pf_get_stats(const zr_pf* pf, zr_pf_stats* out) {
    if (!pf || !out) return zr::set_error(ZR_ERR_INVALID, "NULL argument");
    zr::copy_stats(pf->core.stats(), out);
    return ZR_OK;
}

zr_status zr_pf_destroy(zr_pf* pf) {
    delete pf;
    return ZR_OK;
}

zr_status zr_pf_plan(const zr_pf_config* cfg, int iterations, zr_pf_stats* out) {
    return zr::guarded([&]() -> zr_status {
        if (!out) return zr::set_error(ZR_ERR_INVALID, "out is NULL");
        if (iterations < 1) return zr::set_error(ZR_ERR_INVALID, "iterations < 1");
        zr_status st = zr::validate_pf(cfg, false);
        if (st != ZR_OK) return st;
        zr::PfNull be;
        zr::PrefetchCore<zr::PfNull> core(be);
        zr::PfErr e = core.init(zr::core_config<zr::PrefetchCore<zr::PfNull>>(cfg, 0, 0));
        for (int it = 0; it < iterations && e == zr::PfErr::kOk; ++it)
            for (int t = 0; t < cfg->n_steps && e == zr::PfErr::kOk; ++t) {
                e = core.fetch(t);
                if (e == zr::PfErr::kOk) e = core.release(t);
            }
        zr::copy_stats(core.stats(), out);
        core.destroy();
        return map_err(nullptr, e, "invalid trace");
    });
}

}  // extern "C"
