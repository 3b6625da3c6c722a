// rocrand_philox_ref.cpp - Philox-4x32-10 words from rocRAND, for pinning the
// oracle's generator against an implementation it shares nothing with.
//
// TEST INFRASTRUCTURE ONLY (host code; no GPU is touched).  rocRAND's
// philox4x32_10 engine implements the generator of Salmon, Moraes, Dror and
// Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC 2011).  Its state is
// a 128-bit counter and a 64-bit key (the seed, low word first); rocrand()
// returns the four words of each counter's block in order, then moves to the
// next counter (carrying across all four words).  rocrand_init(seed,
// subsequence, offset) starts at counter (offset / 4, low 64 bits) plus
// (subsequence << 64) and skips offset % 4 words of that block.
//
// stdin, one request per line (hex words):
//   B k0 k1 c0 c1 c2 c3   -> the block of counter (c0, c1, c2, c3) under key (k0, k1)
//   W s_lo s_hi o_lo o_hi n_lo n_hi
//                         -> the word at position n of the stream that starts at
//                            word 4 * offset of counter 0 under key seed, i.e.
//                            word (n mod 4) of counter offset + floor(n / 4)
// stdout: the four words (B) or the one word (W), hex, one line per request.
#include <cstdio>

#include <rocrand/rocrand_kernel.h>

typedef unsigned long long u64;

int main()
{
    char kind[4];
    unsigned a0, a1, a2, a3, a4, a5;
    while (std::scanf("%3s %x %x %x %x %x %x", kind, &a0, &a1, &a2, &a3, &a4, &a5) == 7) {
        rocrand_state_philox4x32_10 st;
        if (kind[0] == 'B') {
            const u64 seed = ((u64)a1 << 32) | a0;
            const u64 hi = ((u64)a5 << 32) | a4;  // counter words 2 and 3
            rocrand_init(seed, hi, 0ull, &st);
            // counter words 0 and 1: advance that many blocks, in steps that
            // keep the word count (4 per block) inside 64 bits
            u64 lo = ((u64)a3 << 32) | a2;
            while (lo != 0) {
                const u64 step = lo < (1ull << 61) ? lo : (1ull << 61);
                skipahead(4 * step, &st);
                lo -= step;
            }
            const unsigned w0 = rocrand(&st);
            const unsigned w1 = rocrand(&st);
            const unsigned w2 = rocrand(&st);
            const unsigned w3 = rocrand(&st);
            std::printf("%08x %08x %08x %08x\n", w0, w1, w2, w3);
        } else {
            const u64 seed = ((u64)a1 << 32) | a0;
            const u64 off = ((u64)a3 << 32) | a2;
            const u64 n = ((u64)a5 << 32) | a4;
            rocrand_init(seed, 0ull, 0ull, &st);
            // skip 4 * offset words (in steps), then n more
            u64 left = off;
            while (left != 0) {
                const u64 step = left < (1ull << 61) ? left : (1ull << 61);
                skipahead(4 * step, &st);
                left -= step;
            }
            skipahead(n, &st);
            std::printf("%08x\n", rocrand(&st));
        }
    }
    return 0;
}
