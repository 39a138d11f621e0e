// Host-side check of the dynamic unit schedule (unit_sched.h), built for the host only.
//
// Simulates G persistent workgroups drawing tickets from the per-XCD and shared counters in random
// interleavings (a ticket is drawn a while before the claiming workgroup's unit ends, and resolved
// to a unit when it ends; other workgroups' draws and resolutions may fall in between), and checks
// that every unit [0, n_units) runs exactly once and nothing else runs.
//
// Usage: unit_sched_check <seed> <cases>; prints one line per failure and "ok <cases>" at the end.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../long_sequence_bidirectional_amd/csrc/unit_sched.h"

using namespace cpattn;

// Map as the launcher builds it for n_dp whole tiles and n_split tiles of split_s pieces on G
// resident workgroups.
static AttnTileMap make_map(int n_dp, int n_split, int split_s, int G) {
    AttnTileMap m{};
    m.n_dp = n_dp;
    m.n_split = n_split;
    m.split_s = n_split > 0 ? split_s : 1;
    m.per_xcd = sched_per_xcd(n_dp, G);
    return m;
}

struct Wg {
    int cur = -1;                    // unit in progress (-1: finished)
    bool drawn = false;              // ticket for the next unit drawn
    unsigned long long ticket = 0;
};

// One simulated launch; returns the number of errors found (and prints them).
static int run_case(int n_dp, int n_split, int split_s, int G, std::mt19937_64& rng) {
    const AttnTileMap m = make_map(n_dp, n_split, split_s, G);
    const int n_units = m.n_dp + m.n_split * m.split_s;
    std::vector<unsigned long long> counters(kNumXcd + 1, 0);
    std::vector<int> runs(n_units, 0);
    std::vector<Wg> wgs(G);
    int active = 0, errors = 0;
    for (int b = 0; b < G; ++b) {
        const int u = sched_first(m, b);
        if (u >= 0 && u < n_units) {
            wgs[b].cur = u;
            ++active;
        }
    }
    auto fail = [&](const char* what, int a, int c) {
        if (errors++ < 5)
            std::printf("FAIL n_dp=%d n_split=%d s=%d G=%d per_xcd=%d: %s (%d, %d)\n", n_dp, n_split, split_s, G,
                        m.per_xcd, what, a, c);
    };
    long long steps = 0;
    while (active > 0) {
        if (++steps > 100000000LL) {
            fail("no progress", active, 0);
            break;
        }
        const int b = (int)(rng() % (unsigned)G);
        Wg& w = wgs[b];
        if (w.cur < 0) continue;
        if (!w.drawn) {                       // draw the ticket some time before the unit ends
            w.ticket = counters[sched_counter(m, w.cur, b)]++;
            w.drawn = true;
            continue;
        }
        // the unit ends: it ran once; resolve the ticket (maybe drawing from the shared counter)
        if (w.cur >= n_units) fail("unit out of range", w.cur, n_units);
        else ++runs[w.cur];
        const int next = sched_unit(m, w.cur, b, G, w.ticket, [&]() { return counters[kNumXcd]++; });
        w.drawn = false;
        if (next >= 0 && next < n_units) {
            w.cur = next;
        } else {
            w.cur = -1;
            --active;
        }
    }
    for (int u = 0; u < n_units; ++u)
        if (runs[u] != 1) fail("unit ran a number of times other than one", u, runs[u]);
    return errors;
}

int main(int argc, char** argv) {
    const unsigned long long seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
    const int cases = argc > 2 ? std::atoi(argv[2]) : 2000;
    std::mt19937_64 rng(seed);
    int errors = 0, done = 0;
    // the bench's shapes at 256 workgroups first: video self-attention, cross-attention,
    // AllGather-KV rank, Ulysses rank, ring chunk
    const int fixed[][3] = {{4096, 56, 9}, {4096, 56, 4}, {512, 16, 16}, {512, 7, 36}, {512, 16, 10}};
    for (const auto& f : fixed) {
        errors += run_case(f[0], f[1], f[2], 256, rng);
        ++done;
    }
    for (; done < cases; ++done) {
        const int G = 8 * (1 + (int)(rng() % 64));                 // 8 .. 512 workgroups
        const int n_dp = (int)(rng() % 4600);
        const int n_split = (int)(rng() % 4) == 0 ? 0 : (int)(rng() % (unsigned)(G + 1));
        const int split_s = 2 + (int)(rng() % 20);
        if (n_dp + n_split == 0) continue;
        errors += run_case(n_dp, n_split, split_s, G, rng);
    }
    std::printf("%s %d cases, %d errors\n", errors ? "FAIL" : "ok", done, errors);
    return errors ? 1 : 0;
}
