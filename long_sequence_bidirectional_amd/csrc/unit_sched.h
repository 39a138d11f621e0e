// The unit schedules of the persistent attention kernels.
//
// Units [0, n_units) are numbered as the kernels number them (whole query tiles in tile order,
// then split pieces).  The first kNumXcd * per_xcd units (whole tiles only, in whole rounds of
// the grid) form one contiguous range per XCD; the rest are a tail shared by all XCDs.  Workgroup b runs on XCD b % kNumXcd (ids are dealt
// round-robin over the XCDs) and starts on the unit at its own index in its XCD's range; after
// that it claims units from its XCD's counter until the range is used up, then from the shared
// counter.  So the workgroups resident on one XCD walk neighbouring tiles together and share
// the K/V stream of a head in that XCD's L2, while XCDs that run faster (their clocks differ
// under the power limit) take more of the tail.  Every ticket maps to a distinct unit and every
// workgroup claims until it draws one past the end, so each unit runs exactly once.
//
// The static order (no counters) and the unit map both launchers build are here too.  The
// mapping from grid ids and tickets to units is plain arithmetic, written for host and device
// alike (a CPU test drives it through random interleavings of the claims); only the counter
// increments are device atomics.
#pragma once

#include <climits>

#include "common.h"
#include "kernels.h"

namespace cpattn {

// Unit map of a launch over `total` query tiles whose last `split_tiles` are cut into `pieces`
// key-range pieces each (unit numbering: whole tiles, then pieces piece-major), on at most
// `slots` resident workgroups (0: unknown); `dynamic`: the counters are in use.  The static unit
// grid `grid` holds each XCD's contiguous range of whole tiles and then of pieces, padded to a
// multiple of the XCD count; the launch runs min(grid, slots rounded down to the XCD count)
// persistent workgroups.  The launcher fills in the workspace, accumulate and counter fields.
struct UnitGrid {
    AttnTileMap map;
    int grid;           // static unit grid ids [0, grid)
    int launch_grid;    // workgroups launched
};
inline UnitGrid sched_plan(int64_t total, int64_t split_tiles, int64_t pieces, int64_t slots, bool dynamic) {
    UnitGrid g{};
    AttnTileMap& m = g.map;
    m.n_dp = (int)(total - split_tiles);
    m.per_xcd_dp = (m.n_dp + kNumXcd - 1) / kNumXcd;
    m.grid_dp = m.per_xcd_dp * kNumXcd;
    m.n_split = (int)split_tiles;
    m.split_s = split_tiles > 0 ? (int)pieces : 1;
    m.per_xcd_sp = (m.n_split * m.split_s + kNumXcd - 1) / kNumXcd;
    g.grid = m.grid_dp + m.per_xcd_sp * kNumXcd;
    const int64_t cap = slots - slots % kNumXcd;
    g.launch_grid = (cap > 0 && g.grid > cap) ? (int)cap : g.grid;
    m.per_xcd = dynamic ? sched_per_xcd(m.n_dp, g.launch_grid) : 0;
    return g;
}

// Static schedule: the unit of static grid id `bid`, or -1 for the padding ids.  Ids are dealt
// round-robin over the XCDs (workgroup b runs ids b, b + G, ...) and mapped so that each XCD walks
// a contiguous range of whole tiles, then of pieces.
__host__ __device__ __forceinline__ int sched_static_unit(const AttnTileMap& m, int64_t bid) {
    if (bid < m.grid_dp) {
        const int u = (int)((bid % kNumXcd) * m.per_xcd_dp + bid / kNumXcd);
        return u < m.n_dp ? u : -1;
    }
    const int64_t w = bid - m.grid_dp;
    const int logical = (int)((w % kNumXcd) * m.per_xcd_sp + w / kNumXcd);
    return logical < m.n_split * m.split_s ? m.n_dp + logical : -1;
}

// First unit of workgroup b of a grid of G.
__host__ __device__ __forceinline__ int sched_first(const AttnTileMap& m, int b) {
    return m.per_xcd > 0 ? (b % kNumXcd) * m.per_xcd + b / kNumXcd : b;
}

// Counter that serves the claim after unit `cur` of workgroup b: its XCD's own while `cur` lies
// in the XCD ranges, else the shared one (index kNumXcd).
__host__ __device__ __forceinline__ int sched_counter(const AttnTileMap& m, int cur, int b) {
    return cur < kNumXcd * m.per_xcd ? b % kNumXcd : kNumXcd;
}

// The unit ticket t (drawn from sched_counter(m, cur, b)) stands for.  A ticket past the end of
// the XCD's range is replaced by one from the shared counter, which draw_shared() returns (called
// at most once).  Past the last unit the result is >= n_units (clamped to INT_MAX).
template <class DrawShared>
__host__ __device__ __forceinline__ int sched_unit(const AttnTileMap& m, int cur, int b, int G, unsigned long long t,
                                                   DrawShared&& draw_shared) {
    const unsigned long long n1 = (unsigned long long)kNumXcd * (unsigned)m.per_xcd;
    if ((unsigned long long)cur < n1) {
        const unsigned long long x = (unsigned)(b % kNumXcd);
        const unsigned long long u = x * (unsigned)m.per_xcd + (unsigned)(G / kNumXcd) + t;
        if (u < (x + 1) * (unsigned)m.per_xcd) return (int)u;
        t = draw_shared();
    }
    const unsigned long long u = n1 + (m.per_xcd > 0 ? 0ull : (unsigned long long)G) + t;
    return u < (unsigned long long)INT_MAX ? (int)u : INT_MAX;
}

// A ticket from the counter that serves the unit after `cur` (one lane; the result is read later,
// so the atomic's round trip overlaps other work).  A vector atomic with device scope.
__device__ __forceinline__ unsigned long long sched_ticket(const AttnTileMap& m, int cur, int b) {
    return __hip_atomic_fetch_add(m.sched + sched_counter(m, cur, b), 1ull, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
}

// The unit a ticket stands for (one lane); a ticket from the shared counter, when needed, is
// waited for here (once per workgroup).
__device__ __forceinline__ int sched_next(const AttnTileMap& m, int cur, int b, int G, unsigned long long t) {
    return sched_unit(m, cur, b, G, t, [&]() {
        return __hip_atomic_fetch_add(m.sched + kNumXcd, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    });
}

}  // namespace cpattn
