// The dynamic unit schedule of the persistent attention kernels.
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
// The mapping from tickets to units is plain arithmetic, written for host and device alike (a
// CPU test drives it through random interleavings of the claims); only the counter increments
// are device atomics.
#pragma once

#include <climits>

#include "common.h"
#include "kernels.h"

namespace cpattn {

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
