// Prints rocRAND's Philox4x32-10 block function on the (counter, key) lines read from stdin.
// Used only by the CPU test that cross-checks the oracle's own Philox implementation
// against an independent library implementation (rocRAND, open source).
// Input lines:  c0 c1 c2 c3 k0 k1   (hex);  output lines: x0 x1 x2 x3 (hex).
#include <cstdio>
#include <rocrand/rocrand_philox4x32_10.h>

struct Probe : rocrand_device::philox4x32_10_engine {
    uint4 block(uint4 c, uint2 k) { return this->ten_rounds(c, k); }
};

int main() {
    unsigned c0, c1, c2, c3, k0, k1;
    Probe p;
    while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        uint4 r = p.block(uint4{c0, c1, c2, c3}, uint2{k0, k1});
        std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
