// Calls the C ABI with rejected arguments (fake, never dereferenced device addresses) and checks
// the status codes and messages; built with -fsanitize=address,undefined against kda_api.cpp and
// the host-only stand-ins (tests/test_host_asan.py).
#include <cstdint>
#include <cstdio>
#include <cstring>
#include "kda.h"
static int fails = 0;
static void expect(kda_status got, kda_status want, const char* what) {
    if (got != want) { std::printf("FAIL %s: %d, expected %d (%s)\n", what, int(got), int(want), kda_last_error()); ++fails; }
    else if (want != KDA_OK && kda_last_error()[0] == 0) { std::printf("FAIL %s: no message\n", what); ++fails; }
}
static void* P(uintptr_t a) { return reinterpret_cast<void*>(a); }
int main() {
    struct F { uintptr_t q, k, v, la, b, cu, out, fs; int64_t T; int32_t N, H, dk, dv; int dt; kda_status want; const char* what; };
    const F base{0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000, 0x700000, 0x800000, 128, 1, 2, 128, 128, KDA_BF16, KDA_OK, ""};
    F cases[16];
    int n = 0;
    auto add = [&](F f, kda_status w, const char* what) { f.want = w; f.what = what; cases[n++] = f; };
    F f = base; f.dt = 7; add(f, KDA_E_DTYPE, "dtype");
    f = base; f.T = -1; add(f, KDA_E_SHAPE, "tokens");
    f = base; f.H = 0; add(f, KDA_E_SHAPE, "heads");
    f = base; f.dk = 96; add(f, KDA_E_UNSUPPORTED, "d_k");
    f = base; f.cu = 0; add(f, KDA_E_NULL, "cu_seqlens");
    f = base; f.q = 0; add(f, KDA_E_NULL, "q");
    f = base; f.v = 0x300008; add(f, KDA_E_ALIGN, "v alignment");
    f = base; f.out = 0x108000; add(f, KDA_E_SHAPE, "out inside q");
    f = base; f.fs = 0x708000; add(f, KDA_E_SHAPE, "final_state over out");
    f = base; f.T = int64_t(1) << 26; f.H = 64; add(f, KDA_E_UNSUPPORTED, "too large");
    for (int i = 0; i < n; ++i) {
        const F& c = cases[i];
        expect(kda_forward(P(c.q), P(c.k), P(c.v), P(c.la), P(c.b), static_cast<const int32_t*>(P(c.cu)), P(c.out),
                           static_cast<float*>(P(c.fs)), c.T, c.N, c.H, c.dk, c.dv, kda_dtype(c.dt), nullptr),
               c.want, c.what);
        expect(kda_forward_noalloc(P(c.q), P(c.k), P(c.v), P(c.la), P(c.b), static_cast<const int32_t*>(P(c.cu)),
                                   nullptr, P(c.out), static_cast<float*>(P(c.fs)), c.T, c.N, c.H, c.dk, c.dv,
                                   kda_dtype(c.dt), 0u, nullptr),
               c.want, c.what);
    }
    // empty batch: no launch, OK
    expect(kda_forward(P(0x100000), P(0x200000), P(0x300000), P(0x400000), P(0x500000),
                       static_cast<const int32_t*>(P(0x600000)), P(0x700000), nullptr, 0, 0, 2, 128, 128, KDA_BF16,
                       nullptr), KDA_OK, "empty");
    // backward: an aliasing gradient, unknown option bits, a null d_out
    auto bwd = [&](uintptr_t dq, uint32_t options, uintptr_t dout) {
        return kda_backward(P(0x100000), P(0x200000), P(0x300000), P(0x400000), P(0x500000),
                            static_cast<const int32_t*>(P(0x600000)), nullptr, P(dout), nullptr, P(dq), P(0x900000),
                            P(0xa00000), P(0xb00000), P(0xc00000), nullptr, 128, 1, 2, 128, 128, KDA_BF16, options,
                            nullptr);
    };
    expect(bwd(0x100000, 0u, 0x700000), KDA_E_SHAPE, "backward dq aliases q");
    expect(bwd(0x800000, 4u, 0x700000), KDA_E_UNSUPPORTED, "backward options");
    expect(bwd(0x800000, 0u, 0), KDA_E_NULL, "backward d_out");
    // short convolution: odd channels, a bad tap count, y over x
    auto conv = [&](int32_t channels, int32_t kt, uintptr_t y) {
        return kda_short_conv(P(0x100000), static_cast<const float*>(P(0x200000)), static_cast<const float*>(P(0x300000)),
                              static_cast<const int32_t*>(P(0x400000)), static_cast<const int32_t*>(P(0x500000)),
                              static_cast<const int32_t*>(P(0x600000)), P(y), 100, 1, channels, 4, kt, 3, 3, KDA_BF16,
                              nullptr);
    };
    expect(conv(60, 3, 0x700000), KDA_E_UNSUPPORTED, "conv channels");
    expect(conv(64, 5, 0x700000), KDA_E_UNSUPPORTED, "conv taps");
    expect(conv(64, 3, 0x100800), KDA_E_SHAPE, "conv y inside x");
    // status strings and pure size queries
    for (int s = -1; s < 12; ++s)
        if (!kda_status_str(kda_status(s)) || !kda_status_str(kda_status(s))[0]) { std::printf("FAIL status %d\n", s); ++fails; }
    if (kda_workspace_bytes(1000, 2, 2, 96, 128, KDA_BF16) != 0) { std::printf("FAIL workspace\n"); ++fails; }
    if (kda_workspace_bytes(1000, 2, 2, 128, 128, KDA_F32) != 0) { std::printf("FAIL workspace f32\n"); ++fails; }
    std::printf("done, %d failures\n", fails);
    return fails ? 1 : 0;
}
