// Test-only cross-check program: prints Philox4x32-10 words from rocRAND's open-source,
// host-callable engine (rocrand_philox4x32_10.h) so that the oracle's generator can be pinned to
// an implementation it shares nothing with. Input lines: "seed subsequence offset"; output lines:
// the four 32-bit words the engine yields from that position, in decimal.
// rocRAND's engine keys with (seed lo, seed hi) and counts with
// (offset/4 lo, offset/4 hi, subsequence lo, subsequence hi).
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
    unsigned long long seed, subsequence, offset;
    while (std::scanf("%llu %llu %llu", &seed, &subsequence, &offset) == 3) {
        rocrand_device::philox4x32_10_engine eng(seed, subsequence, offset);
        unsigned int w0 = eng.next(), w1 = eng.next(), w2 = eng.next(), w3 = eng.next();
        std::printf("%u %u %u %u\n", w0, w1, w2, w3);
    }
    return 0;
}
