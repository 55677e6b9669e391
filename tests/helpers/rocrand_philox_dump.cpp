// Test helper: prints rocRAND's Philox4x32-10 output for (key, counter) lines read from
// stdin, through the engine's public API, so the oracle's Philox can be checked against an
// independent implementation.  Input lines: key c0 c1 c2 c3 (decimal); output: w0 w1 w2 w3.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

int main()
{
    unsigned long long key;
    unsigned int c[4];
    while (std::scanf("%llu %u %u %u %u", &key, &c[0], &c[1], &c[2], &c[3]) == 5) {
        // The engine keeps counter words 2,3 as the "subsequence" and words 0,1 as the
        // offset / 4; next4() at substate 0 returns the block for exactly that counter.
        unsigned long long subsequence = (unsigned long long)c[2] | ((unsigned long long)c[3] << 32);
        unsigned long long blocks = (unsigned long long)c[0] | ((unsigned long long)c[1] << 32);
        rocrand_device::philox4x32_10_engine eng(key, subsequence, 0);
        // discard() counts single 32-bit outputs (4 per block); advance in pieces of
        // 2^60 blocks so that the element count never overflows 64 bits.
        for (unsigned long long i = 0; i < (blocks >> 60); ++i) eng.discard(1ull << 62);
        eng.discard((blocks & ((1ull << 60) - 1)) * 4ull);
        uint4 w = eng.next4();
        std::printf("%u %u %u %u\n", w.x, w.y, w.z, w.w);
    }
    return 0;
}
