// Reads launch-shape cases from stdin and prints what the library's host
// launch arithmetic (csrc/df11_launch.h) makes of them, for
// tests/test_launch_shape.py.
//   "S n resident sup_0 .. sup_{n-1}"  ->  "want_0 .. want_{n-1}"
//   "P n_super want"                   ->  "n_wg pools dynamic"
//   "C grid"                           ->  "stride"
#include <stdint.h>
#include <stdio.h>

#include "df11_launch.h"

int main() {
    char kind;
    while (scanf(" %c", &kind) == 1) {
        if (kind == 'S') {
            unsigned n;
            unsigned long long resident;
            if (scanf("%u %llu", &n, &resident) != 2 || n > 64) return 1;
            uint64_t sup[64], want[64];
            for (unsigned i = 0; i < n; ++i) {
                unsigned long long v;
                if (scanf("%llu", &v) != 1) return 1;
                sup[i] = v;
            }
            df11::split_grid(sup, n, resident, want);
            for (unsigned i = 0; i < n; ++i) printf("%llu%c", (unsigned long long)want[i], i + 1 < n ? ' ' : '\n');
        } else if (kind == 'P') {
            unsigned long long n_super, want;
            if (scanf("%llu %llu", &n_super, &want) != 2) return 1;
            uint32_t pools = 0;
            bool dynamic = false;
            const uint32_t n_wg = df11::pool_shape(n_super, want, &pools, &dynamic);
            printf("%u %u %d\n", n_wg, pools, dynamic ? 1 : 0);
        } else if (kind == 'C') {
            unsigned grid;
            if (scanf("%u", &grid) != 1) return 1;
            printf("%u\n", df11::coprime_stride(grid));
        } else {
            return 1;
        }
    }
    return 0;
}
