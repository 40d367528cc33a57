// Host-only stress of the measurement hook's registry (the moe_set_stage_events state): two
// threads keep re-setting the hook while six others take event pairs, as concurrent
// moe_forward calls would.  Every pair taken must come from one setting: its two handles are
// consecutive entries of the same event array, and the stage is the one set with that array.
// Built with -fsanitize=thread by tests/test_host_threads.py; exit status 0 = consistent.
#include <stdint.h>
#include <stdio.h>

#include <atomic>
#include <thread>
#include <vector>

#include "stage_hook.hpp"

namespace {
constexpr int NSET = 4, NPAIRS = 5, ROUNDS = 20000;
// event "handles": generation g owns handles tag(g, 0 .. 2*NPAIRS)
void* tag(int g, int k) { return (void*)(uintptr_t)(0x1000 + g * 0x100 + k); }
}  // namespace

int main() {
    static void* arrays[NSET][2 * NPAIRS];
    for (int g = 0; g < NSET; ++g)
        for (int k = 0; k < 2 * NPAIRS; ++k) arrays[g][k] = tag(g, k);
    dsmoe::StageHookRegistry reg;
    std::atomic<int> bad{0}, taken{0};
    std::vector<std::thread> th;
    for (int s = 0; s < 2; ++s)
        th.emplace_back([&, s] {
            for (int r = 0; r < ROUNDS; ++r) {
                const int g = (r + s) % NSET;
                if (r % 7 == 3) reg.set(-1, nullptr, 0, 5);
                else if (!reg.set(g, arrays[g], NPAIRS, 5)) bad++;
            }
        });
    for (int c = 0; c < 6; ++c)
        th.emplace_back([&] {
            for (int r = 0; r < ROUNDS; ++r) {
                const dsmoe::HookPair p = reg.take();
                if (p.stage < 0) {
                    if (p.start || p.stop) bad++;
                    continue;
                }
                taken++;
                const uintptr_t a = (uintptr_t)p.start - 0x1000, b = (uintptr_t)p.stop - 0x1000;
                const int g = (int)(a / 0x100), k = (int)(a % 0x100);
                if (g != p.stage || b != a + 1 || k % 2 != 0 || k >= 2 * NPAIRS) bad++;
            }
        });
    for (auto& t : th) t.join();
    // invalid settings leave the registry as it was
    reg.set(2, arrays[2], NPAIRS, 5);
    if (reg.set(6, arrays[0], 1, 5) || reg.set(1, nullptr, 3, 5) || reg.set(0, arrays[0], -1, 5)) bad++;
    dsmoe::HookPair p = reg.take();
    if (p.stage != 2 || p.start != tag(2, 0) || p.stop != tag(2, 1)) bad++;
    p = reg.take();
    if (p.start != tag(2, 2)) bad++;
    printf("pairs taken %d, inconsistent %d\n", taken.load(), bad.load());
    return bad.load() == 0 && taken.load() > 0 ? 0 : 1;
}
