// Host-side launch arithmetic of the gfx950 decoders: how a persistent grid
// is shared between the streams of a batched launch, and how many work
// counters a stream's dynamic schedule uses.  Plain C++ (no HIP), so that a
// CPU test can build and check it on its own.
#ifndef DF11_LAUNCH_H
#define DF11_LAUNCH_H

#include <stdint.h>

#include <algorithm>
#include <numeric>

namespace df11 {

// Dynamic schedule: at most kPools counters per stream, each serving at most
// kMaxPerPool workgroups; streams with fewer than kDynamicMinRounds
// super-groups per workgroup keep the static schedule.
constexpr uint32_t kPools = 8;
constexpr uint64_t kDynamicMinRounds = 12;
constexpr uint32_t kMaxPerPool = 96;

// Workgroups per stream of a batch, from each stream's super-groups sup[i]
// (every sup[i] >= 1) and the resident workgroup count (resident >= n).  A
// batched launch ends with its slowest stream, so the shares minimise the
// largest number of super-groups per workgroup, sup[i] / want[i]: every
// stream starts with one workgroup, then each further workgroup goes to the
// stream with the largest sup[i] / want[i] that still has a super-group
// without a workgroup of its own (Adams' method of apportionment, which
// minimises that largest ratio).  The shares never add up to more than
// max(resident, n).
inline void split_grid(const uint64_t *sup, uint32_t n, uint64_t resident, uint64_t *want) {
    uint64_t given = 0;
    for (uint32_t i = 0; i < n; ++i) {
        want[i] = 1;
        ++given;
    }
    while (given < resident) {
        uint32_t best = n;
        for (uint32_t i = 0; i < n; ++i)
            if (want[i] < sup[i] && (best == n || sup[i] * want[best] > sup[best] * want[i])) best = i;
        if (best == n) break;
        ++want[best];
        ++given;
    }
}

// Workgroup count and pool count for the dynamic schedule of a stream with
// n_super super-groups given `want` workgroups.  The pools must divide the
// workgroup count (a pool's share of the work is fixed), and a pool balances
// only its own workgroups, so the fewest pools that keep every counter within
// kMaxPerPool workgroups are taken, dropping a few workgroups if no count of
// kPools or fewer divides theirs.  Beyond kPools * kMaxPerPool workgroups the
// count is rounded down to a multiple of kPools.  *dynamic is cleared when
// the schedule does not pay (fewer than kDynamicMinRounds rounds).  The
// result is at least 1 and at most max(1, min(want, n_super)).
inline uint32_t pool_shape(uint64_t n_super, uint64_t want, uint32_t *pools, bool *dynamic) {
    uint64_t n_wg = std::max<uint64_t>(1, std::min(want, n_super));
    uint32_t p_found = 0;
    if (n_wg > static_cast<uint64_t>(kPools) * kMaxPerPool) {
        n_wg -= n_wg % kPools;
        p_found = kPools;
    }
    while (!p_found) {  // ends by n_wg = kMaxPerPool at the latest (one pool)
        for (uint32_t p = 1; p <= kPools && !p_found; ++p)
            if (n_wg % p == 0 && n_wg / p <= kMaxPerPool) p_found = p;
        if (!p_found) --n_wg;
    }
    *pools = p_found;
    *dynamic = n_super >= kDynamicMinRounds * n_wg;
    return static_cast<uint32_t>(n_wg);
}

// A stride near 0.618 of the grid and coprime to it: id * stride mod grid
// then spreads each stream's range of a batch over every dispatch position.
inline uint32_t coprime_stride(uint32_t grid) {
    for (uint32_t c = std::max<uint32_t>(1, static_cast<uint32_t>(grid * 0.618)); c < 2 * grid + 2; ++c)
        if (std::gcd(c, grid) == 1) return c;
    return 1;
}

}  // namespace df11

#endif  // DF11_LAUNCH_H
