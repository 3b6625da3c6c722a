// asan_abi_driver.cpp - drives the host side of libfa_mi355x under
// AddressSanitizer (TEST INFRASTRUCTURE ONLY; host code, no GPU).
//
// Linked against a copy of the library whose host code was built with
// AddressSanitizer.  It calls every entry point with arguments that fail a
// check (so nothing reaches the GPU), walks the variant registry, reads every
// status string and error message, and exercises the stride, alignment and
// size arithmetic on large and odd values.  Any out-of-bounds access or leak
// in that host code makes the sanitizer fail the run.  Prints "ok <n>" with
// the number of rejected calls.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fa_mi355x.h"

namespace {

int g_checked = 0;
int g_failed = 0;

void expect(fa_status got, fa_status want, const char* what)
{
    ++g_checked;
    const char* msg = fa_last_error();
    // read the whole message: an unterminated or freed buffer shows up here
    const size_t n = std::strlen(msg);
    if (got != want || (want != FA_OK && n == 0)) {
        std::printf("FAIL %s: status %d (%s), message '%s'\n", what, (int)got, fa_status_string(got), msg);
        ++g_failed;
    }
}

}  // namespace

int main()
{
    char* const P = reinterpret_cast<char*>(uintptr_t(1) << 20);  // aligned stand-in, never dereferenced
    const fa_status E = FA_ERR_INVALID_ARGUMENT;

    // registry and strings
    const int nv = fa_variant_count();
    size_t total = 0;
    for (int i = -1; i <= nv; ++i) {
        const char* s = fa_variant_name(i);
        if (s) total += std::strlen(s);
    }
    for (int s = -1; s < 6; ++s) total += std::strlen(fa_status_string((fa_status)s));
    if (fa_abi_version() != FA_ABI_VERSION || nv <= 0 || total == 0) {
        std::printf("FAIL registry\n");
        return 1;
    }
    for (int dt = -1; dt < 3; ++dt)
        for (int D = 0; D <= 300; D += 4)
            for (int mk = -1; mk < 4; ++mk) {
                fa_supported((fa_dtype)dt, D, (fa_mask_kind)mk, D & 4);
                fa_bwd_supported((fa_dtype)dt, D, (fa_mask_kind)mk, D & 4);
            }

    // fa_fwd: one failing check at a time
    expect(fa_fwd(P, P, P, nullptr, P, (float*)P, 0, 4, 2, 16, 16, 64, 0.125f, 0, FA_DTYPE_BF16, FA_MASK_NONE, nullptr),
           E, "B = 0");
    expect(fa_fwd(P, P, P, nullptr, P, (float*)P, 1, 3, 2, 16, 16, 64, 0.125f, 0, FA_DTYPE_BF16, FA_MASK_NONE, nullptr),
           E, "H_q % H_kv");
    expect(fa_fwd(P, P, P, nullptr, P, (float*)P, 1, 4, 2, 16, 16, 72, 0.125f, 0, FA_DTYPE_BF16, FA_MASK_NONE, nullptr),
           E, "D = 72");
    expect(fa_fwd(P, P, P, P, P, (float*)P, 1, 4, 2, 16, 16, 64, 0.125f, 0, FA_DTYPE_BF16, FA_MASK_NONE, nullptr), E,
           "mask without kind");
    expect(fa_fwd(P + 8, P, P, nullptr, P, (float*)P, 1, 4, 2, 16, 16, 64, 0.125f, 0, FA_DTYPE_BF16, FA_MASK_NONE,
                  nullptr),
           E, "misaligned Q");
    expect(fa_fwd(P, P, P, nullptr, P, (float*)P, 0x7fffffff, 0x7fffffff, 1, 0x7fffffff, 0x7fffffff, 256, 1.f, 0,
                  FA_DTYPE_BF16, FA_MASK_NONE, nullptr),
           E, "too large");

    // strides: every tensor and axis, negative and misaligned values, huge values
    const int64_t bad_values[] = {-8, 3, 60, INT64_MIN, -1};
    for (int t = 0; t < 4; ++t)
        for (int a = 0; a < 3; ++a)
            for (int64_t v : bad_values) {
                fa_strides st;
                std::memset(&st, 0, sizeof(st));
                int64_t* tri = t == 0 ? st.q : t == 1 ? st.k : t == 2 ? st.v : st.o;
                tri[a] = v;
                tri[(a + 1) % 3] = 64;
                expect(fa_fwd_strided(P, P, P, nullptr, P, (float*)P, 1, 4, 2, 16, 16, 64, 0.125f, 0, FA_DTYPE_BF16,
                                      FA_MASK_NONE, &st, nullptr),
                       E, "bad stride");
                expect(fa_fwd_strided_noalloc(P, P, P, nullptr, P, (float*)P, 1, 4, 2, 16, 16, 64, 0.125f, 0,
                                              FA_DTYPE_BF16, FA_MASK_NONE, &st, nullptr),
                       E, "bad stride (noalloc)");
            }
    {
        fa_strides st;
        std::memset(&st, 0, sizeof(st));
        st.mask[2] = -5;
        expect(fa_fwd_strided(P, P, P, P, P, (float*)P, 1, 4, 2, 16, 16, 64, 0.125f, 0, FA_DTYPE_BF16, FA_MASK_BOOL,
                              &st, nullptr),
               E, "negative mask stride");
    }

    // dropout and window
    const float rates[] = {-0.01f, 1.5f, __builtin_nanf(""), __builtin_inff()};
    for (float r : rates)
        expect(fa_fwd_dropout(P, P, P, nullptr, P, (float*)P, 1, 4, 2, 16, 16, 64, 0.125f, 0, FA_DTYPE_BF16,
                              FA_MASK_NONE, r, ~0ull, 1ull << 63, nullptr, nullptr),
               E, "dropout rate");
    expect(fa_fwd_window(P, P, P, nullptr, P, (float*)P, 1, 4, 2, 16, 16, 64, 0.125f, 1, FA_DTYPE_BF16, FA_MASK_NONE, 0,
                         nullptr, nullptr),
           E, "window 0");
    expect(fa_fwd_window(P, P, P, nullptr, P, (float*)P, 1, 4, 2, 16, 16, 64, 0.125f, 0, FA_DTYPE_BF16, FA_MASK_NONE, 8,
                         nullptr, nullptr),
           E, "window without causal");

    // backward
    expect(fa_bwd(P, P, P, P, P, (float*)P, nullptr, (float*)P, P, P, P, 1, 4, 2, 16, 16, 64, 0.125f, 0, FA_DTYPE_F32,
                  FA_MASK_NONE, nullptr),
           FA_ERR_UNSUPPORTED, "bwd fp32");
    expect(fa_bwd(P, P, P, P, nullptr, (float*)P, nullptr, (float*)P, P, P, P, 1, 4, 2, 16, 16, 64, 0.125f, 0,
                  FA_DTYPE_BF16, FA_MASK_NONE, nullptr),
           E, "bwd dO null");
    expect(fa_bwd(P, P, P, P, P, (float*)(P + 2), nullptr, (float*)P, P, P, P, 1, 4, 2, 16, 16, 64, 0.125f, 0,
                  FA_DTYPE_BF16, FA_MASK_NONE, nullptr),
           E, "bwd L misaligned");

    if (g_failed) return 1;
    std::printf("ok %d\n", g_checked);
    return 0;
}
