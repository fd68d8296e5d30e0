// Index arithmetic of the whole-line decompression of a matrix stored in
// MFMA tile order (merge_group_pairs in df11_decode.hip).  Plain constexpr
// C++ (no HIP), so that the gfx950 kernel calls it and a CPU test builds it
// on its own and checks it against the tile order's definition.
//
// The tile order (df11_tile_order): 512-element blocks of 64 chunks of 8
// elements; block b is n-tile b mod 4 of global k-step b / 4, and global
// k-step g is k-step g mod (C / 32) of the 64-row panel g / (C / 32); lane l
// of a block holds row 16 nt + (l mod 16), columns 32 ks + 8 (l / 16) .. + 7.
// With an even number of k-steps per panel, chunks [512 j, 512 j + 512) are
// two k-steps of one panel, 64 consecutive columns of its 64 rows: a
// pair-round.  Thread t (wave t / 64) of a group merges chunk
// pair_chunk(c0, p, h, t) of each half h of each pair-round p, puts it in its
// wave's stage at pair_unit(h, t mod 64), and in store s, lane L stores the
// stage's chunk of half pair_src_half(L), lane pair_src_lane(L, s) to row
// 8 s + L / 8 of the wave's n-tile, columns 8 (L mod 8) .. + 7 of the pair:
// eight lanes to a 128-byte line.
#ifndef DF11_PAIRS_H
#define DF11_PAIRS_H

#include <stdint.h>

namespace df11 {

// 16-byte units per stage half: 64 chunks and a pad after every 16, so that
// eight lanes of one row (stores) and eight consecutive lanes (merges) fall
// on distinct banks.
constexpr uint32_t kPairUnits = 68;

// First chunk of the pair-round that holds chunk c0.
constexpr uint32_t pair_base(uint32_t c0) { return c0 & ~511u; }

// Pair-rounds covering a group's chunks [c0, c0 + n).
constexpr uint32_t pair_rounds(uint32_t c0, uint32_t n) {
    return n ? (c0 + n - pair_base(c0) + 511u) / 512u : 0u;
}

// Chunk merged by thread t (0 .. 255) in half h of pair-round p.
constexpr uint32_t pair_chunk(uint32_t c0, uint32_t p, uint32_t h, uint32_t t) {
    return pair_base(c0) + 512u * p + 256u * h + t;
}

// Stage unit of lane l's chunk of half h.
constexpr uint32_t pair_unit(uint32_t h, uint32_t l) { return kPairUnits * h + l + (l >> 4); }

// The chunk lane L stores in store s: half and lane in the stage.
constexpr uint32_t pair_src_half(uint32_t lane) { return (lane & 7u) >> 2; }
constexpr uint32_t pair_src_lane(uint32_t lane, uint32_t s) { return (lane >> 3) + 8u * s + 16u * (lane & 3u); }

// Row-major element index of that store: the wave's part (panel, n-tile w,
// the pair's first k-step ks) plus the lane's part.
constexpr uint32_t pair_wave_dst(uint32_t panel, uint32_t ks, uint32_t cols, uint32_t w) {
    return (64u * panel + 16u * w) * cols + 32u * ks;
}
constexpr uint32_t pair_lane_dst(uint32_t lane, uint32_t s, uint32_t cols) {
    return ((lane >> 3) + 8u * s) * cols + 8u * (lane & 7u);
}

// Whether the line of the chunk at stage lane l_src (cb: the wave's chunk of
// lane 0, half 0) lies whole in [c0, c0 + n): its 8 chunks lie between its
// first (half 0, run 0) and its last (half 1, run 3) in the stream.
constexpr bool pair_line_whole(uint32_t cb, uint32_t l_src, uint32_t c0, uint32_t n) {
    return cb + (l_src & 15u) - c0 < n && cb + (l_src & 15u) + 304u - c0 < n;
}

}  // namespace df11

#endif  // DF11_PAIRS_H
