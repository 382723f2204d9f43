// Host-side reference stream from rocRAND's Philox4x32-10 engine (source
// header, built with g++ for the CPU).  Used only to pin the oracle's own
// Philox implementation.  Reads lines "seed subsequence discard count" on
// stdin and prints `count` 32-bit outputs in hex, one line per request.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main() {
    unsigned long long seed, sub, skip, count;
    while (std::scanf("%llu %llu %llu %llu", &seed, &sub, &skip, &count) == 4) {
        rocrand_device::philox4x32_10_engine eng(seed, sub, skip);
        for (unsigned long long i = 0; i < count; ++i)
            std::printf("%08x%c", eng.next(), i + 1 == count ? '\n' : ' ');
    }
    return 0;
}
