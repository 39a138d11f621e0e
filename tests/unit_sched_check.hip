// Host-side check of the dynamic unit schedule (unit_sched.h), built for the host only.
//
// For the unit maps the launchers build (sched_plan), checks the static order (every workgroup
// walks its grid ids) and simulates the persistent workgroups drawing tickets from the per-XCD and
// shared counters in random interleavings (a ticket is drawn a while before the claiming
// workgroup's unit ends, and resolved to a unit when it ends; other workgroups' draws and
// resolutions may fall in between).  In both orders every unit [0, n_units) must run exactly once
// and nothing else may run.
//
// Usage: unit_sched_check <seed> <cases>; prints one line per failure and "ok <cases>" at the end.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../long_sequence_bidirectional_amd/csrc/unit_sched.h"

using namespace cpattn;

struct Wg {
    int cur = -1;                    // unit in progress (-1: finished)
    bool drawn = false;              // ticket for the next unit drawn
    unsigned long long ticket = 0;
};

// One launch over `total` tiles, the last `split_tiles` of them in `pieces` pieces each, with the
// unit map and grid the launchers build (sched_plan) for `slots` resident workgroups: the static
// order (each workgroup walks its grid ids), then the dynamic order under a random interleaving of
// the claims.  Returns the number of errors found (and prints them).
static int run_case(int total, int split_tiles, int pieces, int slots, std::mt19937_64& rng) {
    int errors = 0;
    const UnitGrid st = sched_plan(total, split_tiles, pieces, slots, false);
    const UnitGrid dy = sched_plan(total, split_tiles, pieces, slots, true);
    const int n_units = st.map.n_dp + st.map.n_split * st.map.split_s;
    auto fail = [&](const char* order, const char* what, int a, int c) {
        if (errors++ < 5)
            std::printf("FAIL %s total=%d split=%d s=%d slots=%d: %s (%d, %d)\n", order, total, split_tiles, pieces,
                        slots, what, a, c);
    };
    if (dy.map.n_dp + dy.map.n_split * dy.map.split_s != n_units || dy.grid != st.grid ||
        dy.launch_grid != st.launch_grid)
        fail("plan", "static and dynamic plans differ", st.grid, dy.grid);
    if (st.launch_grid % kNumXcd != 0 || st.launch_grid <= 0 || (slots >= kNumXcd && st.launch_grid > slots))
        fail("plan", "launch grid", st.launch_grid, slots);

    // static order: workgroup b runs the units of grid ids b, b + G, ... (padding ids skipped)
    {
        std::vector<int> runs(n_units, 0);
        const int G = st.launch_grid;
        for (int b = 0; b < G; ++b)
            for (long long bid = b; bid < st.grid; bid += G) {
                const int u = sched_static_unit(st.map, bid);
                if (u < 0) continue;
                if (u >= n_units) fail("static", "unit out of range", u, n_units);
                else ++runs[u];
            }
        for (int u = 0; u < n_units; ++u)
            if (runs[u] != 1) fail("static", "unit ran a number of times other than one", u, runs[u]);
    }

    // dynamic order
    const AttnTileMap& m = dy.map;
    const int G = dy.launch_grid;
    std::vector<unsigned long long> counters(kNumXcd + 1, 0);
    std::vector<int> runs(n_units, 0);
    std::vector<Wg> wgs(G);
    int active = 0;
    for (int b = 0; b < G; ++b) {
        const int u = sched_first(m, b);
        if (u >= 0 && u < n_units) {
            wgs[b].cur = u;
            ++active;
        }
    }
    long long steps = 0;
    while (active > 0) {
        if (++steps > 100000000LL) {
            fail("dynamic", "no progress", active, 0);
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
        if (w.cur >= n_units) fail("dynamic", "unit out of range", w.cur, n_units);
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
        if (runs[u] != 1) fail("dynamic", "unit ran a number of times other than one", u, runs[u]);
    return errors;
}

int main(int argc, char** argv) {
    const unsigned long long seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
    const int cases = argc > 2 ? std::atoi(argv[2]) : 2000;
    std::mt19937_64 rng(seed);
    int errors = 0, done = 0;
    // the bench's shapes at 256 resident workgroups first: video self-attention, cross-attention,
    // AllGather-KV rank, Ulysses rank, ring chunk
    const int fixed[][3] = {{4152, 56, 9}, {4152, 56, 4}, {528, 16, 16}, {519, 7, 36}, {528, 16, 10}};
    for (const auto& f : fixed) {
        errors += run_case(f[0], f[1], f[2], 256, rng);
        ++done;
    }
    for (; done < cases; ++done) {
        const int slots = 8 * (1 + (int)(rng() % 64));             // 8 .. 512 resident workgroups
        const int total = 1 + (int)(rng() % 4600);
        const int split = (int)(rng() % 4) == 0 ? 0 : (int)(rng() % (unsigned)(slots < total ? slots : total));
        const int pieces = 2 + (int)(rng() % 20);
        errors += run_case(total, split, split > 0 ? pieces : 1, (int)(rng() % 8) == 0 ? 0 : slots, rng);
    }
    std::printf("%s %d cases, %d errors\n", errors ? "FAIL" : "ok", done, errors);
    return errors ? 1 : 0;
}
