// Host-only reference stream from rocRAND's Philox4x32-10 engine, used by the
// CPU tests as an independent implementation of the published generator.
// Usage: rocrand_philox_ref <seed> <subsequence> <first_block> <nblocks>
// Prints nblocks lines of four hex words: the generator outputs for counter
// blocks first_block .. first_block+nblocks-1 of that subsequence.
#include <rocrand/rocrand_kernel.h>
#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv)
{
    if (argc != 5) return 2;
    unsigned long long seed = strtoull(argv[1], nullptr, 0);
    unsigned long long subseq = strtoull(argv[2], nullptr, 0);
    unsigned long long first = strtoull(argv[3], nullptr, 0);
    long n = strtol(argv[4], nullptr, 0);
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, subseq, 4ull * first, &st);
    for (long i = 0; i < n; ++i) {
        uint4 v = rocrand4(&st);
        printf("%08x %08x %08x %08x\n", v.x, v.y, v.z, v.w);
    }
    return 0;
}
