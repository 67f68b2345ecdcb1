// Host-side checks of the index helpers the kernels use (built with hipcc, run on the CPU).
//   fastdiv: FastDiv::div(n) == n / d for edge and random n, many d
//   xcd:     xcd_contiguous is a bijection on [0, total) for many totals
#include <stdio.h>
#include <stdint.h>
#include <stdlib.h>
#include <vector>

#include "common.h"
#include "fastdiv.h"

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint32_t next32() {  // xorshift64*
    rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
    return (uint32_t)((rng * 2685821657736338717ull) >> 32);
}

int main() {
    long bad = 0;
    std::vector<uint32_t> ds = {1, 2, 3, 5, 6, 7, 8, 12, 16, 24, 40, 48, 80, 96, 1152, 4608, 9450,
                                27280, 75600, 604800, 65535, 65536, 65537, 1u << 31, 0x7fffffffu,
                                0x80000001u, 0xffffffffu};
    for (int i = 0; i < 2000; ++i) ds.push_back(1 + next32() % 100000);
    for (int i = 0; i < 200; ++i) ds.push_back(1 + next32());
    for (uint32_t d : ds) {
        dtl::FastDiv f = dtl::FastDiv::make(d);
        uint32_t ns[] = {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 2 * d, 0x7fffffffu, 0x80000000u, 0xfffffffeu, 0xffffffffu};
        for (uint32_t n : ns)
            if (f.div(n) != n / d) { if (bad < 10) printf("fastdiv d=%u n=%u got %u\n", d, n, f.div(n)); ++bad; }
        for (int i = 0; i < 2000; ++i) {
            uint32_t n = next32();
            if (f.div(n) != n / d) { if (bad < 10) printf("fastdiv d=%u n=%u got %u\n", d, n, f.div(n)); ++bad; }
        }
    }
    for (int total = 1; total <= 6000; total += (total < 600 ? 1 : 37)) {
        std::vector<int> seen(total, 0);
        for (int pid = 0; pid < total; ++pid) {
            int l = dtl::xcd_contiguous(pid, total);
            if (l < 0 || l >= total || seen[l]++) { if (bad < 10) printf("xcd total=%d pid=%d -> %d\n", total, pid, l); ++bad; }
        }
    }
    printf("%s (%ld failures)\n", bad ? "FAIL" : "OK", bad);
    return bad ? 1 : 0;
}
