// Reads groups of a tile-ordered matrix from stdin and prints what the
// whole-line decompression's index arithmetic (csrc/df11_pairs.h), composed
// as merge_group_pairs composes it, makes of them, for
// tests/test_tile_pairs.py.
//   "Q cols c0 n"  ->  one line per merged chunk, "M p h w lane chunk unit",
//                      one per stored chunk, "S p s w lane chunk unit dst whole",
//                      then "E"
#include <stdint.h>
#include <stdio.h>

#include "df11_pairs.h"

int main() {
    char kind;
    while (scanf(" %c", &kind) == 1) {
        if (kind != 'Q') return 1;
        unsigned cols, c0, n;
        if (scanf("%u %u %u", &cols, &c0, &n) != 3 || cols % 64 || cols == 0) return 1;
        const uint32_t ks_per_panel = cols / 32;
        for (uint32_t p = 0; p < df11::pair_rounds(c0, n); ++p) {
            for (uint32_t w = 0; w < 4; ++w) {
                const uint32_t cb = df11::pair_chunk(c0, p, 0, 64 * w);
                for (uint32_t lane = 0; lane < 64; ++lane)
                    for (uint32_t h = 0; h < 2; ++h) {
                        const uint32_t c = df11::pair_chunk(c0, p, h, 64 * w + lane);
                        if (c - c0 < n) printf("M %u %u %u %u %u %u\n", p, h, w, lane, c, df11::pair_unit(h, lane));
                    }
                const uint32_t g = cb >> 8, panel = g / ks_per_panel;
                const uint32_t wave_dst = df11::pair_wave_dst(panel, g - panel * ks_per_panel, cols, w);
                for (uint32_t lane = 0; lane < 64; ++lane)
                    for (uint32_t s = 0; s < 2; ++s) {
                        const uint32_t h_src = df11::pair_src_half(lane), l_src = df11::pair_src_lane(lane, s);
                        const uint32_t c = cb + 256 * h_src + l_src;
                        if (c - c0 >= n) continue;
                        printf("S %u %u %u %u %u %u %u %d\n", p, s, w, lane, c, df11::pair_unit(h_src, l_src),
                               wave_dst + df11::pair_lane_dst(lane, s, cols),
                               df11::pair_line_whole(cb, l_src, c0, n) ? 1 : 0);
                    }
            }
        }
        printf("E\n");
    }
    return 0;
}
