// Host-only check of the slot arena's residency protocol (EStream, section
// 3.3: an expert cannot execute before its parameters are ready, and a slot
// is not overwritten while a queued invocation still references it).
//
// The library's ResidencyTable (routed_expert_ffn_top_amd/csrc/residency.h)
// runs here on a fake backend: each stream is a worker thread that executes
// its queue in order, an event is a counter of completed records, a wait
// blocks its worker until the event's record at the time of the wait has
// completed. Loads copy each expert's slices into its slot in chunks with
// random pauses; invocations read every slot their placement map names in
// chunks with random pauses and compare each byte with the expert's own
// pattern. The schedule is the paged layer's: the first B groups of G
// experts load into the B banks before "routing", then every group with
// routes loads into the bank released longest ago and runs, with random
// groups skipped, over many layer calls, on one or two compute streams.
//
//   residency_sim correct <calls> <seed>   exit 0 iff no invocation saw a
//                                          partly loaded or overwritten slot
//   residency_sim control <calls> <seed>   the same with every wait dropped:
//                                          exit 0 iff violations were seen
//                                          (the check can detect them)
#include <assert.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <chrono>
#include <condition_variable>
#include <deque>
#include <functional>
#include <mutex>
#include <random>
#include <thread>
#include <vector>

#include "residency.h"

namespace {

struct FakeStream {
    std::mutex m;
    std::condition_variable cv;
    std::deque<std::function<void()>> q;
    bool stop = false, busy = false;
    std::thread th;

    FakeStream() : th([this] { run(); }) {}
    ~FakeStream()
    {
        {
            std::lock_guard<std::mutex> lk(m);
            stop = true;
        }
        cv.notify_all();
        th.join();
    }
    void push(std::function<void()> f)
    {
        {
            std::lock_guard<std::mutex> lk(m);
            q.push_back(std::move(f));
        }
        cv.notify_all();
    }
    void run()
    {
        for (;;) {
            std::function<void()> f;
            {
                std::unique_lock<std::mutex> lk(m);
                cv.wait(lk, [&] { return stop || !q.empty(); });
                if (q.empty()) return;
                f = std::move(q.front());
                q.pop_front();
                busy = true;
            }
            f();
            {
                std::lock_guard<std::mutex> lk(m);
                busy = false;
            }
            cv.notify_all();
        }
    }
    void drain()
    {
        std::unique_lock<std::mutex> lk(m);
        cv.wait(lk, [&] { return q.empty() && !busy; });
    }
};

struct FakeEvent {
    std::mutex m;
    std::condition_variable cv;
    uint64_t issued = 0, done = 0;
};

struct FakeBackend {
    using Stream = FakeStream *;
    using Event = FakeEvent *;
    bool drop_waits = false;   // the control run: every wait does nothing
    std::atomic<int> live{0};

    int create(Event *e)
    {
        *e = new FakeEvent();
        live++;
        return 0;
    }
    void destroy(Event e)
    {
        delete e;
        live--;
    }
    int record(Event e, Stream s)
    {
        uint64_t g;
        {
            std::lock_guard<std::mutex> lk(e->m);
            g = ++e->issued;
        }
        s->push([e, g] {
            {
                std::lock_guard<std::mutex> lk(e->m);
                if (e->done < g) e->done = g;
            }
            e->cv.notify_all();
        });
        return 0;
    }
    int wait(Stream s, Event e)
    {
        if (drop_waits) return 0;
        uint64_t g;
        {
            std::lock_guard<std::mutex> lk(e->m);
            g = e->issued;   // the record at the time of the wait
        }
        if (g == 0) return 0;
        s->push([e, g] {
            std::unique_lock<std::mutex> lk(e->m);
            e->cv.wait(lk, [&] { return e->done >= g; });
        });
        return 0;
    }
    int sync(Event e)
    {
        std::unique_lock<std::mutex> lk(e->m);
        const uint64_t g = e->issued;
        e->cv.wait(lk, [&] { return e->done >= g; });
        return 0;
    }
};

constexpr int kSlotBytes = 2048, kChunks = 4;
// experts per group, banks, slots, experts, groups
constexpr int G = 4, Bk = 2, P = G * Bk, NE = 24, NG = NE / G;

uint8_t pattern(int expert, int i) { return (uint8_t)(expert * 37 + i * 11 + (i >> 8) * 5 + 1); }

void pause_us(std::mt19937 &rng, int max_us)
{
    std::this_thread::sleep_for(std::chrono::microseconds(rng() % (unsigned)(max_us + 1)));
}

}  // namespace

int main(int argc, char **argv)
{
    if (argc < 4) {
        fprintf(stderr, "usage: %s correct|control <calls> <seed>\n", argv[0]);
        return 2;
    }
    const bool control = strcmp(argv[1], "control") == 0;
    const int calls = atoi(argv[2]);
    const unsigned seed = (unsigned)atoi(argv[3]);

    FakeBackend bk;
    bk.drop_waits = control;
    std::vector<std::vector<uint8_t>> host(NE, std::vector<uint8_t>(kSlotBytes));
    for (int e = 0; e < NE; ++e)
        for (int i = 0; i < kSlotBytes; ++i) host[e][i] = pattern(e, i);
    std::vector<uint8_t> plane((size_t)P * kSlotBytes, 0);
    std::atomic<long> violations{0}, checked{0};
    std::mt19937 host_rng(seed);
    {
        moe::ResidencyTable<FakeBackend> res(bk, P, NE);
        FakeStream copy, compute0, compute1;
        FakeStream *compute[2] = {&compute0, &compute1};
        int invocation = 0;
        for (int call = 0; call < calls; ++call) {
            res.forget_mapping();
            // groups with routes this call (the rest are skipped after routing)
            std::vector<int> routed(NG);
            for (int g = 0; g < NG; ++g) routed[g] = (host_rng() % 4) != 0;
            auto load_group = [&](int g, int bank) {
                std::vector<int> sl, ex;
                for (int r = 0; r < G; ++r) {
                    sl.push_back(bank * G + r);
                    ex.push_back(g * G + r);
                }
                const unsigned cs = (unsigned)host_rng();
                auto write = [&](FakeStream *st) -> moe_status {
                    for (size_t i = 0; i < sl.size(); ++i) {
                        uint8_t *dst = plane.data() + (size_t)sl[i] * kSlotBytes;
                        const uint8_t *src = host[ex[i]].data();
                        st->push([dst, src, cs, i] {
                            std::mt19937 rng(cs + (unsigned)i);
                            for (int c = 0; c < kChunks; ++c) {
                                memcpy(dst + c * (kSlotBytes / kChunks), src + c * (kSlotBytes / kChunks),
                                       kSlotBytes / kChunks);
                                pause_us(rng, 150);
                            }
                        });
                    }
                    return MOE_OK;
                };
                const moe_status rc = res.load(sl.data(), ex.data(), (int)sl.size(), &copy, write);
                if (rc != MOE_OK) {
                    fprintf(stderr, "load failed: %s\n", res.msg());
                    exit(3);
                }
            };
            auto run_group = [&](int g, int bank) {
                std::vector<int32_t> phi(NE, -1);
                for (int r = 0; r < G; ++r) phi[g * G + r] = bank * G + r;
                FakeStream *st = compute[invocation++ % 2];
                if (res.acquire(phi.data(), st) != MOE_OK) {
                    fprintf(stderr, "acquire failed: %s\n", res.msg());
                    exit(3);
                }
                const unsigned ks = (unsigned)host_rng();
                st->push([&plane, &violations, &checked, phi, ks] {
                    std::mt19937 rng(ks);
                    for (int e = 0; e < NE; ++e) {
                        const int s = phi[e];
                        if (s < 0) continue;
                        const uint8_t *p = plane.data() + (size_t)s * kSlotBytes;
                        for (int c = 0; c < kChunks; ++c) {
                            for (int i = c * (kSlotBytes / kChunks); i < (c + 1) * (kSlotBytes / kChunks); ++i)
                                if (p[i] != pattern(e, i)) {
                                    violations++;
                                    break;
                                }
                            checked++;
                            pause_us(rng, 100);
                        }
                    }
                });
                if (res.release_after(phi.data(), st) != MOE_OK) {
                    fprintf(stderr, "release failed: %s\n", res.msg());
                    exit(3);
                }
            };
            // the first B groups load before routing is known
            for (int g = 0; g < Bk && g < NG; ++g) load_group(g, g);
            std::deque<int> banks;
            for (int g = 0; g < NG; ++g) {
                const bool pre = g < Bk;
                if (!routed[g]) {
                    if (pre) banks.push_front(g);
                    continue;
                }
                int bank;
                if (pre) {
                    bank = g;
                } else {
                    bank = banks.front();
                    banks.pop_front();
                    load_group(g, bank);
                }
                run_group(g, bank);
                banks.push_back(bank);
            }
            // state checks on the host: executed groups' slots are In-use
            for (int s = 0; s < P; ++s) {
                const int st = res.state(s);
                assert(st == MOE_SLOT_IN_USE || st == MOE_SLOT_READY || st == MOE_SLOT_AVAILABLE);
                (void)st;
            }
        }
        copy.drain();
        compute0.drain();
        compute1.drain();
    }
    const long v = violations.load(), n = checked.load();
    printf("%s: %d layer calls, %ld slot chunks checked, %ld violations, %d events left\n",
           control ? "control (waits dropped)" : "protocol", calls, n, v, bk.live.load());
    if (bk.live.load() != 0) return 4;
    if (n == 0) return 5;
    return control ? (v > 0 ? 0 : 1) : (v == 0 ? 0 : 1);
}
