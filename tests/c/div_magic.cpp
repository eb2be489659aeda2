// Exhaustive host check of the kernels' division by a runtime divisor
// without a division (div_magic / fast_div in the library's launch.hpp):
// for every divisor d in 1..64 and every n in [0, 2^26), fast_div(n, d,
// div_magic(d)) must equal n / d.  Built with hipcc (the header includes the
// HIP runtime header) and run on the host only; prints "ok" and exits 0, or
// prints the first counterexample and exits 1.
#include <cstdio>

#include "launch.hpp"

int main() {
    for (int d = 1; d <= 64; ++d) {
        const uint32_t m = absk::div_magic(d);
        for (int n = 0; n < (1 << 26); ++n) {
            if (absk::fast_div(n, d, m) != n / d) {
                std::printf("fast_div(%d, %d) = %d, expected %d\n", n, d, absk::fast_div(n, d, m), n / d);
                return 1;
            }
        }
    }
    std::printf("ok\n");
    return 0;
}
