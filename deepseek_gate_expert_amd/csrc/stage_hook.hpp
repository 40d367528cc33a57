// stage_hook.hpp - the measurement hook's state (moe_set_stage_events), host code only.
//
// One process-wide registry: a caller sets (stage, array of 2 * n_pairs event handles); every
// moe_forward call takes, once and at entry, the pair (2 i, 2 i + 1) with i = its rank among
// the calls since the hook was set, modulo n_pairs.  A mutex makes setting the hook and taking
// pairs safe from any number of threads; each taken pair belongs to one consistent setting.
// Event handles are opaque here (hipEvent_t is a pointer type), so this file needs no HIP header
// and its thread safety is tested on the host on its own.
#pragma once

#include <stdint.h>

#include <mutex>

namespace dsmoe {

struct HookPair {
    int32_t stage = -1;  // -1: record nothing
    void* start = nullptr;
    void* stop = nullptr;
};

class StageHookRegistry {
  public:
    // stage < 0 or n_pairs == 0 clears the hook; returns false for invalid arguments (then
    // nothing changes)
    bool set(int32_t stage, void* const* events, int32_t n_pairs, int32_t max_stage) {
        if (stage < -1 || stage > max_stage || n_pairs < 0 || (n_pairs > 0 && !events && stage >= 0)) return false;
        std::lock_guard<std::mutex> lk(mu_);
        stage_ = (stage < 0 || n_pairs == 0) ? -1 : stage;
        events_ = events;
        n_pairs_ = stage_ < 0 ? 0 : n_pairs;
        calls_ = 0;
        return true;
    }

    HookPair take() {
        std::lock_guard<std::mutex> lk(mu_);
        HookPair h;
        if (stage_ < 0 || n_pairs_ <= 0) return h;
        const int64_t i = calls_++ % n_pairs_;
        h.stage = stage_;
        h.start = events_[2 * i];
        h.stop = events_[2 * i + 1];
        return h;
    }

  private:
    std::mutex mu_;
    int32_t stage_ = -1;
    void* const* events_ = nullptr;
    int32_t n_pairs_ = 0;
    int64_t calls_ = 0;
};

}  // namespace dsmoe
