// Test helper: prints rocRAND's Philox4x32-10 output for (seed, stream, row,
// col8) tuples read from stdin, as the independent reference that pins the
// oracle's Philox.  Engine (seed, subsequence = stream, offset =
// 4 * (row * 2^32 + col8)) puts counter = {col8, row, stream, 0} and
// key = {seed low, seed high}.  Host-only use of the header; runs on the CPU.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main()
{
    unsigned long long seed, stream, row, col8;
    while (std::scanf("%llu %llu %llu %llu", &seed, &stream, &row, &col8) == 4) {
        unsigned long long offset = 4ULL * ((row << 32) | col8);
        rocrand_device::philox4x32_10_engine e(seed, stream, offset);
        unsigned w0 = e.next(), w1 = e.next(), w2 = e.next(), w3 = e.next();
        std::printf("%u %u %u %u\n", w0, w1, w2, w3);
    }
    return 0;
}
