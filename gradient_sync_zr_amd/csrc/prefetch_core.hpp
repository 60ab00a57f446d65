// ZeRO-3 parameter prefetch coordinator, independent of the runtime it drives.
//
// A trace is a fixed sequence of steps (module visits, forward then
// backward), each using a list of parameters. Full parameters exist only
// while "live"; they are gathered from the 1/K shards into an arena by
// all-gathers on their own stream and released when a step is done with
// them. fetch(step) follows the three parts of a module's fetch in
// "DeepSpeed ZeRO-3 源码解析" (2.1):
//   1. gather at once every parameter of the step that is not live;
//   2. make the compute stream wait for the gathers that produce the step's
//      parameters (no wait at all for gathers the host has already seen
//      finish);
//   3. prefetch: take the next parameters of the trace, in order, skipping
//      those already live, and gather them as one batch without waiting. The
//      batch stops once its size reaches the cap
//          min(max_live - live, prefetch_bucket)            (2.2)
//      so the parameter that crosses the cap is still in it (the greedy rule
//      of the prefetch buckets); no prefetch starts while live >= max_live.
// `live` counts the elements of every gathered or in-flight full parameter:
// it grows when a gather is issued and shrinks at release (2.2). At most
// `max_ongoing` gathers are outstanding: before issuing another, the host
// drops those it sees finished and then blocks on the oldest until fewer
// remain (2.2: two queued fetch events).
//
// release(step) keeps a parameter live when it is used again soon: the
// steps after this one are scanned in trace order, a step at a time, until
// the elements of the parameters seen reach `max_reuse`; a parameter of this
// step that appears there is not released (2.4, the conservative release;
// the scan stays within this pass of the trace). max_reuse = 0 releases
// every parameter of the step.
//
// Memory: every live parameter occupies a range of the arena (the same
// offsets on every rank), taken when its gather is issued and returned when
// it is released. A released range may still be read by the compute the
// caller queued for that step, so each release records an event on the
// compute stream (a ring of kReleaseEvents, one per release in turn) and its
// freed ranges carry that release's number. A gather that reuses memory waits
// for the newest release among the ranges it takes, and only when the host
// has not yet seen that release pass; a ring slot recorded again since then
// holds a later release, which is a safe (longer) wait.
//
// Backend requirements: types Stream and Event, and
//   int create(Event*), int destroy(Event), int record(Event, Stream),
//   int wait(Stream, Event), int query(Event, bool* done), int sync(Event),
//   int gather(Stream, const int* params, const int64_t* offsets, int n)
// returning 0 on success. wait() captures the event's most recent record.
#pragma once

#include <algorithm>
#include <cstdint>
#include <deque>
#include <map>
#include <vector>

namespace zr {

enum class PfErr { kOk = 0, kBadArg, kBadState, kNoMemory, kBackend };

// Allocator over [0, capacity) elements with sizes rounded up to `align`.
// Every free range remembers the epoch (release number) that freed it, -1
// for memory never used: a gather that takes a range must not write it before
// the compute stream has passed that release. alloc() prefers the range freed
// longest ago (then the lowest offset), so prefetches land in memory whose
// readers are long done; when no single range is large enough, adjacent free
// ranges are merged (the merged range takes the newest of their epochs).
class ArenaAlloc {
  public:
    void init(int64_t capacity, int64_t align) {
        align_ = align > 0 ? align : 1;
        cap_ = capacity / align_ * align_;
        free_.clear();
        if (cap_ > 0) free_[0] = Free{cap_, -1};
        peak_ = 0;
    }
    int64_t rounded(int64_t n) const { return (n + align_ - 1) / align_ * align_; }
    int64_t capacity() const { return cap_; }
    int64_t peak_extent() const { return peak_; }

    // On success *off is the range and *epoch the newest release it reuses.
    bool alloc(int64_t n, int64_t* off, int64_t* epoch) {
        const int64_t need = rounded(n);
        auto best = free_.end();
        for (auto it = free_.begin(); it != free_.end(); ++it)
            if (it->second.len >= need && (best == free_.end() || it->second.epoch < best->second.epoch))
                best = it;
        if (best == free_.end()) best = merge_run(need);
        if (best == free_.end()) return false;
        *off = best->first;
        *epoch = best->second.epoch;
        const Free f = best->second;
        free_.erase(best);
        if (f.len > need) free_[*off + need] = Free{f.len - need, f.epoch};
        peak_ = std::max(peak_, *off + need);
        return true;
    }

    void release(int64_t off, int64_t n, int64_t epoch) {
        Free f{rounded(n), epoch};
        // ranges freed by the same release merge at once
        auto next = free_.lower_bound(off);
        if (next != free_.end() && off + f.len == next->first && next->second.epoch == epoch) {
            f.len += next->second.len;
            free_.erase(next);
        }
        next = free_.lower_bound(off);
        if (next != free_.begin()) {
            auto prev = std::prev(next);
            if (prev->first + prev->second.len == off && prev->second.epoch == epoch) {
                prev->second.len += f.len;
                return;
            }
        }
        free_[off] = f;
    }

  private:
    struct Free {
        int64_t len, epoch;
    };
    // The run of adjacent free ranges, at least `need` long, whose newest
    // epoch is oldest; merged into one range. end() when there is none.
    std::map<int64_t, Free>::iterator merge_run(int64_t need) {
        auto best_lo = free_.end();
        int64_t best_epoch = 0;
        for (auto lo = free_.begin(); lo != free_.end(); ++lo) {
            int64_t len = 0, ep = -1;
            for (auto it = lo; it != free_.end(); ++it) {
                if (it != lo && std::prev(it)->first + std::prev(it)->second.len != it->first) break;
                len += it->second.len;
                ep = std::max(ep, it->second.epoch);
                if (len >= need) {
                    if (best_lo == free_.end() || ep < best_epoch) {
                        best_lo = lo;
                        best_epoch = ep;
                    }
                    break;
                }
            }
        }
        if (best_lo == free_.end()) return best_lo;
        Free m{0, -1};
        auto it = best_lo;
        const int64_t lo_off = best_lo->first;
        while (m.len < need) {
            m.len += it->second.len;
            m.epoch = std::max(m.epoch, it->second.epoch);
            it = free_.erase(it);
        }
        return free_.emplace(lo_off, m).first;
    }

    std::map<int64_t, Free> free_;  // offset -> free range
    int64_t cap_ = 0, align_ = 1, peak_ = 0;
};

struct PfStats {
    int64_t gathers = 0;           // gather batches issued
    int64_t immediate_gathers = 0; // part 1 batches (parameters that were not prefetched)
    int64_t immediate_numel = 0;
    int64_t prefetch_numel = 0;
    int64_t host_syncs = 0;        // host blocked on the oldest gather (event cap)
    int64_t stream_waits = 0;      // compute stream waits on a gather
    int64_t live = 0;              // elements of live full parameters now
    int64_t peak_live = 0;
    int64_t peak_ongoing = 0;
    int64_t arena_peak = 0;        // highest arena offset ever used (elements)
    int64_t prefetch_trimmed = 0;  // prefetches cut short because the arena was full
    int64_t retained = 0;          // releases skipped: the parameter is reused soon
};

template <class Backend>
class PrefetchCore {
  public:
    using Stream = typename Backend::Stream;
    using Event = typename Backend::Event;

    struct Config {
        int n_params = 0;
        const int64_t* numels = nullptr;
        int n_steps = 0;
        const int32_t* step_off = nullptr;     // n_steps + 1 offsets into step_params
        const int32_t* step_params = nullptr;  // parameters of each step, trace order
        int64_t bucket = 0;                    // prefetch bucket cap (elements)
        int64_t max_live = 0;                  // live full-parameter budget (elements)
        int64_t max_reuse = 0;                 // conservative-release window (elements)
        int64_t arena = 0;                     // arena capacity (elements)
        int64_t align = 1;                     // arena range alignment (elements)
        int max_ongoing = 2;                   // outstanding gathers
        Stream gather{}, compute{};
    };

    explicit PrefetchCore(Backend& be) : be_(be) {}
    ~PrefetchCore() { destroy(); }  // the backend must outlive the core
    PrefetchCore(const PrefetchCore&) = delete;
    PrefetchCore& operator=(const PrefetchCore&) = delete;

    PfErr init(const Config& c) {
        if (c.n_params < 1 || !c.numels || c.n_steps < 1 || !c.step_off || c.bucket < 1 ||
            c.max_live < 1 || c.max_reuse < 0 || c.arena < 1 || c.max_ongoing < 1)
            return PfErr::kBadArg;
        if (c.step_off[c.n_steps] > 0 && !c.step_params) return PfErr::kBadArg;
        cfg_ = c;
        params_.assign(c.n_params, Param{});
        for (int p = 0; p < c.n_params; ++p) {
            if (c.numels[p] < 1) return PfErr::kBadArg;
            params_[p].numel = c.numels[p];
        }
        if (c.step_off[0] != 0) return PfErr::kBadArg;
        for (int s = 0; s < c.n_steps; ++s)
            if (c.step_off[s + 1] < c.step_off[s]) return PfErr::kBadArg;
        if (c.step_off[c.n_steps] > 0) order_.assign(c.step_params, c.step_params + c.step_off[c.n_steps]);
        step_off_.assign(c.step_off, c.step_off + c.n_steps + 1);
        for (int p : order_)
            if (p < 0 || p >= c.n_params) return PfErr::kBadArg;
        arena_.init(c.arena, c.align);
        // every step's parameters are live together: they must fit the arena
        stamp_.assign(c.n_params, 0);
        for (int s = 0; s < c.n_steps; ++s) {
            ++tick_;
            int64_t need = 0;
            for (int i = step_off_[s]; i < step_off_[s + 1]; ++i) {
                const int p = order_[i];
                if (stamp_[p] == tick_) continue;
                stamp_[p] = tick_;
                need += arena_.rounded(params_[p].numel);
            }
            if (need > arena_.capacity()) return PfErr::kNoMemory;
        }
        // what each step releases, fixed with the trace: its parameters that
        // do not appear within the reuse window after it
        release_off_.assign(1, 0);
        release_.clear();
        retained_.assign(c.n_steps, 0);
        for (int st = 0; st < c.n_steps; ++st) {
            const uint32_t reused = ++tick_;
            int64_t seen = 0;
            for (int t = st + 1; t < c.n_steps && seen < c.max_reuse; ++t)
                for (int i = step_off_[t]; i < step_off_[t + 1]; ++i) {
                    stamp_[order_[i]] = reused;
                    seen += params_[order_[i]].numel;
                }
            const uint32_t listed = ++tick_;
            for (int i = step_off_[st]; i < step_off_[st + 1]; ++i) {
                const int p = order_[i];
                if (stamp_[p] == listed) continue;
                if (stamp_[p] == reused)
                    ++retained_[st];
                else
                    release_.push_back(p);
                stamp_[p] = listed;
            }
            release_off_.push_back((int32_t)release_.size());
        }
        slots_.assign(c.max_ongoing + 1, Slot{});
        for (Slot& s : slots_) {
            if (be_.create(&s.ev)) return PfErr::kBackend;
            s.created = true;
        }
        rel_.assign(kReleaseEvents, Rel{});
        for (Rel& r : rel_) {
            if (be_.create(&r.ev)) return PfErr::kBackend;
            r.created = true;
        }
        step_state_.assign(c.n_steps, 0);
        return PfErr::kOk;
    }

    // Blocks until the outstanding gathers have finished (they write the
    // arena), then frees the events. Errors are ignored: nothing is left to
    // report them to.
    void destroy() {
        while (!ongoing_.empty()) {
            be_.sync(slots_[ongoing_.front()].ev);
            retire_front();
        }
        for (Slot& s : slots_)
            if (s.created) be_.destroy(s.ev);
        slots_.clear();
        for (Rel& r : rel_)
            if (r.created) be_.destroy(r.ev);
        rel_.clear();
    }

    const PfStats& stats() const { return st_; }
    int n_steps() const { return cfg_.n_steps; }
    int n_params() const { return cfg_.n_params; }

    // Arena offset of a live parameter, -1 when it is not live.
    int64_t offset_of(int p) const {
        if (p < 0 || p >= (int)params_.size() || params_[p].st == kOff) return -1;
        return params_[p].off;
    }

    PfErr fetch(int step) {
        if (step < 0 || step >= cfg_.n_steps) return PfErr::kBadArg;
        if (step != next_ || step_state_[step] != 0) return PfErr::kBadState;
        // 1. what the step needs and nobody has gathered
        std::vector<int> now;
        ++tick_;
        for (int i = step_off_[step]; i < step_off_[step + 1]; ++i) {
            const int p = order_[i];
            if (stamp_[p] == tick_) continue;
            stamp_[p] = tick_;
            if (params_[p].st == kOff) now.push_back(p);
        }
        if (!now.empty()) {
            PfErr e = gather(now);
            if (e != PfErr::kOk) return e;
            ++st_.immediate_gathers;
            for (int p : now) st_.immediate_numel += params_[p].numel;
        }
        // 2. the compute stream waits for the gathers still outstanding
        std::vector<int> waited;
        for (int i = step_off_[step]; i < step_off_[step + 1]; ++i) {
            const Param& q = params_[order_[i]];
            if (q.st != kInflight) continue;
            if (std::find(waited.begin(), waited.end(), q.slot) != waited.end()) continue;
            waited.push_back(q.slot);
            if (be_.wait(cfg_.compute, slots_[q.slot].ev)) return PfErr::kBackend;
            ++st_.stream_waits;
        }
        step_state_[step] = 1;
        next_ = step + 1;
        // 3. prefetch what follows in the trace
        qpos_ = std::max(qpos_, step_off_[step + 1]);
        const int64_t cap = std::min(cfg_.max_live - st_.live, cfg_.bucket);
        if (cap <= 0) return PfErr::kOk;
        std::vector<int> batch, qidx;
        int64_t acc = 0;
        ++tick_;
        while (qpos_ < (int)order_.size() && acc < cap) {
            const int i = qpos_++;
            const int p = order_[i];
            if (params_[p].st != kOff || stamp_[p] == tick_) continue;
            stamp_[p] = tick_;
            batch.push_back(p);
            qidx.push_back(i);
            acc += params_[p].numel;
        }
        if (batch.empty()) return PfErr::kOk;
        // an arena too full for the whole batch prefetches the part that
        // fits; the rest stays in the queue for a later prefetch
        size_t used = 0;
        PfErr e = gather(batch, &used);
        if (e == PfErr::kNoMemory) e = PfErr::kOk;  // nothing fits now
        if (e != PfErr::kOk) return e;
        if (used < batch.size()) {
            ++st_.prefetch_trimmed;
            qpos_ = qidx[used];
        }
        for (size_t k = 0; k < used; ++k) st_.prefetch_numel += params_[batch[k]].numel;
        return PfErr::kOk;
    }

    // The step is done with its parameters. The caller has queued the
    // step's compute on the compute stream before this call.
    PfErr release(int step) {
        if (step < 0 || step >= cfg_.n_steps) return PfErr::kBadArg;
        if (step_state_[step] != 1) return PfErr::kBadState;
        Rel& r = rel_[epoch_ % kReleaseEvents];
        if (be_.record(r.ev, cfg_.compute)) return PfErr::kBackend;
        r.epoch = epoch_;
        st_.retained += retained_[step];
        for (int i = release_off_[step]; i < release_off_[step + 1]; ++i) {
            Param& q = params_[release_[i]];
            if (q.st == kOff) continue;
            arena_.release(q.off, q.numel, epoch_);
            q.st = kOff;
            q.off = -1;
            ++q.seq;  // a later retirement of its gather no longer refers to it
            st_.live -= q.numel;
        }
        ++epoch_;
        step_state_[step] = 2;
        if (step == cfg_.n_steps - 1) {  // the trace starts over
            std::fill(step_state_.begin(), step_state_.end(), 0);
            next_ = 0;
            qpos_ = 0;
        }
        return PfErr::kOk;
    }

  private:
    enum St : uint8_t { kOff, kInflight, kReady };
    struct Param {
        int64_t numel = 0, off = -1;
        St st = kOff;
        int slot = -1;
        uint32_t seq = 0;
    };
    struct Slot {
        Event ev{};
        bool created = false, busy = false;
        std::vector<std::pair<int, uint32_t>> params;  // (param, its seq at gather)
    };

    void retire_front() {
        Slot& s = slots_[ongoing_.front()];
        ongoing_.pop_front();
        for (auto& pr : s.params) {
            Param& q = params_[pr.first];
            if (q.seq == pr.second && q.st == kInflight) q.st = kReady;
        }
        s.params.clear();
        s.busy = false;
    }

    PfErr make_room() {
        while (!ongoing_.empty()) {
            bool done = false;
            if (be_.query(slots_[ongoing_.front()].ev, &done)) return PfErr::kBackend;
            if (!done) break;
            retire_front();
        }
        while ((int)ongoing_.size() >= cfg_.max_ongoing) {
            if (be_.sync(slots_[ongoing_.front()].ev)) return PfErr::kBackend;
            ++st_.host_syncs;
            retire_front();
        }
        return PfErr::kOk;
    }

    // Gathers `batch`, all of it or (prefix != nullptr) its longest prefix
    // that the arena can hold; *prefix receives the count gathered.
    // kNoMemory when not even the first parameter fits (or, without prefix,
    // when the batch does not fit whole); nothing is issued then.
    PfErr gather(const std::vector<int>& batch_in, size_t* prefix = nullptr) {
        std::vector<int> batch = batch_in;
        std::vector<int64_t> offs(batch.size()), eps(batch.size());
        auto undo = [&](size_t n) {
            for (size_t k = 0; k < n; ++k) arena_.release(offs[k], params_[batch[k]].numel, eps[k]);
        };
        for (size_t i = 0; i < batch.size(); ++i) {
            if (arena_.alloc(params_[batch[i]].numel, &offs[i], &eps[i])) continue;
            if (!prefix || i == 0) {
                undo(i);
                if (prefix) *prefix = 0;
                return PfErr::kNoMemory;
            }
            batch.resize(i);
            offs.resize(i);
            eps.resize(i);
            break;
        }
        if (prefix) *prefix = batch.size();
        const int64_t reuse = *std::max_element(eps.begin(), eps.end());
        PfErr e = make_room();
        if (e == PfErr::kOk && reuse > done_epoch_) {
            // reused memory: the compute stream must have passed release `reuse`
            Rel& r = rel_[reuse % kReleaseEvents];
            bool done = false;
            if (be_.query(r.ev, &done)) e = PfErr::kBackend;
            if (e == PfErr::kOk && done)
                done_epoch_ = std::max(done_epoch_, r.epoch);
            else if (e == PfErr::kOk && be_.wait(cfg_.gather, r.ev))
                e = PfErr::kBackend;
        }
        if (e == PfErr::kOk && be_.gather(cfg_.gather, batch.data(), offs.data(), (int)batch.size()))
            e = PfErr::kBackend;
        int slot = -1;
        for (int i = 0; i < (int)slots_.size() && e == PfErr::kOk; ++i)
            if (!slots_[i].busy) {
                slot = i;
                break;
            }
        if (e == PfErr::kOk && (slot < 0 || be_.record(slots_[slot].ev, cfg_.gather))) e = PfErr::kBackend;
        if (e != PfErr::kOk) {
            undo(batch.size());
            if (prefix) *prefix = 0;
            return e;
        }
        Slot& s = slots_[slot];
        s.busy = true;
        ongoing_.push_back(slot);
        for (size_t i = 0; i < batch.size(); ++i) {
            Param& q = params_[batch[i]];
            q.st = kInflight;
            q.off = offs[i];
            q.slot = slot;
            s.params.push_back({batch[i], q.seq});
            st_.live += q.numel;
        }
        ++st_.gathers;
        st_.peak_live = std::max(st_.peak_live, st_.live);
        st_.peak_ongoing = std::max(st_.peak_ongoing, (int64_t)ongoing_.size());
        st_.arena_peak = arena_.peak_extent();
        return PfErr::kOk;
    }

    Backend& be_;
    Config cfg_{};
    std::vector<Param> params_;
    std::vector<int32_t> order_, step_off_;
    std::vector<int32_t> release_, release_off_;  // what each step releases
    std::vector<int32_t> retained_;               // parameters each step keeps live
    std::vector<uint8_t> step_state_;  // 0 not fetched, 1 fetched, 2 released
    std::vector<uint32_t> stamp_;      // dedupe marks
    uint32_t tick_ = 0;
    std::vector<Slot> slots_;
    std::deque<int> ongoing_;          // slots of outstanding gathers, oldest first
    static constexpr int kReleaseEvents = 8;
    struct Rel {
        Event ev{};
        bool created = false;
        int64_t epoch = -1;  // the release last recorded on this event
    };
    std::vector<Rel> rel_;
    int64_t epoch_ = 0;        // releases so far
    int64_t done_epoch_ = -1;  // newest release the host has seen pass
    ArenaAlloc arena_;
    int next_ = 0, qpos_ = 0;
    PfStats st_;
};

}  // namespace zr
