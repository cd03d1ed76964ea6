// Host-side driver that runs rocRAND's Philox4x32-10 engine (an independent
// library implementation of Salmon et al., SC'11) on counter/key pairs read
// from stdin ("c0 c1 c2 c3 k0 k1" in hex, one per line) and prints the four
// output words.  Used only to pin the CPU oracle's generator.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
    unsigned c0, c1, c2, c3, k0, k1;
    while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
        unsigned long long seed = (unsigned long long)k0 | ((unsigned long long)k1 << 32);
        unsigned long long subsequence = (unsigned long long)c2 | ((unsigned long long)c3 << 32);
        unsigned long long block = (unsigned long long)c0 | ((unsigned long long)c1 << 32);
        // The engine's counter is (block lo, block hi, subsequence lo,
        // subsequence hi); the offset counts 32-bit outputs, four per block.
        rocrand_device::philox4x32_10_engine e(seed, subsequence, 0);
        e.discard(block * 4ULL);
        unsigned r0 = e(), r1 = e(), r2 = e(), r3 = e();
        std::printf("%08x %08x %08x %08x\n", r0, r1, r2, r3);
    }
    return 0;
}
