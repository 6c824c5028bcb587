// Host-only helper for the oracle's Philox pin: evaluates rocRAND's
// Philox4x32-10 bijection (a library implementation of the SC'11 generator)
// on (counter, key) pairs read from stdin, one "c0 c1 c2 c3 k0 k1" per line,
// and prints the four output words.  Built with g++ by the test; never part
// of the library.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

struct PhiloxProbe : rocrand_device::philox4x32_10_engine {
    uint4 rounds(uint4 c, uint2 k) { return ten_rounds(c, k); }
};

int main()
{
    PhiloxProbe p;
    unsigned c0, c1, c2, c3, k0, k1;
    while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        uint4 c = {c0, c1, c2, c3};
        uint2 k = {k0, k1};
        uint4 r = p.rounds(c, k);
        std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
    }
    return 0;
}
