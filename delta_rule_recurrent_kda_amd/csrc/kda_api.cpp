// kda_api.cpp -- C ABI of libkda: argument checks, error reporting, dispatch.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

thread_local std::string g_last_error;

kda_status fail(kda_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kda_status fail(kda_status s, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool validate_env()
{
    const char* e = std::getenv("KDA_VALIDATE");
    return e && e[0] == '1';
}

// KDA_SCAN_VARIANT=sequential selects the one-chunk-at-a-time kernel for bf16 data
// (the pipelined kernel is the default); fp32 data always uses the sequential one.
bool sequential_env()
{
    const char* e = std::getenv("KDA_SCAN_VARIANT");
    return e && std::strcmp(e, "sequential") == 0;
}

}  // namespace

extern "C" {

const char* kda_status_str(kda_status s)
{
    switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_E_NULL: return "KDA_E_NULL";
    case KDA_E_DTYPE: return "KDA_E_DTYPE";
    case KDA_E_SHAPE: return "KDA_E_SHAPE";
    case KDA_E_ALIGN: return "KDA_E_ALIGN";
    case KDA_E_UNSUPPORTED: return "KDA_E_UNSUPPORTED";
    case KDA_E_SEQLENS: return "KDA_E_SEQLENS";
    case KDA_E_HIP: return "KDA_E_HIP";
    }
    return "KDA_E_UNKNOWN";
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

int32_t kda_version(void) { return 100; }   // 0.1.0

kda_status kda_forward(const void* q, const void* k, const void* v, const void* log_alpha,
                       const void* beta, const int32_t* cu_seqlens, void* out, float* final_state,
                       int64_t total_tokens, int32_t num_seqs, int32_t num_heads, int32_t d_k,
                       int32_t d_v, kda_dtype dtype, hipStream_t stream)
{
    g_last_error.clear();
    if (dtype != KDA_F32 && dtype != KDA_BF16)
        return fail(KDA_E_DTYPE, "dtype %d is neither KDA_F32 nor KDA_BF16", int(dtype));
    if (total_tokens < 0 || num_seqs < 0 || num_heads < 1)
        return fail(KDA_E_SHAPE, "bad sizes: total_tokens=%lld num_seqs=%d num_heads=%d",
                    (long long)total_tokens, num_seqs, num_heads);
    if ((d_k != 64 && d_k != 128) || (d_v != 64 && d_v != 128))
        return fail(KDA_E_UNSUPPORTED, "d_k=%d d_v=%d: only 64 and 128 are supported", d_k, d_v);
    const int64_t dmax = d_k > d_v ? d_k : d_v;
    if (total_tokens * num_heads * dmax >= (int64_t(1) << 31) ||
        int64_t(num_seqs) * num_heads * d_k * d_v >= (int64_t(1) << 31))
        return fail(KDA_E_UNSUPPORTED, "problem too large for 32-bit element offsets");
    if (!cu_seqlens) return fail(KDA_E_NULL, "cu_seqlens is NULL");
    if (total_tokens > 0 && (!q || !k || !v || !log_alpha || !beta || !out))
        return fail(KDA_E_NULL, "a tensor pointer is NULL");
    const void* ptrs[] = {q, k, v, log_alpha, beta, cu_seqlens, out, final_state};
    const char* names[] = {"q", "k", "v", "log_alpha", "beta", "cu_seqlens", "out", "final_state"};
    for (int i = 0; i < 8; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(KDA_E_ALIGN, "%s is not 16-byte aligned", names[i]);
    if (out && (out == q || out == k || out == v || out == log_alpha || out == beta))
        return fail(KDA_E_SHAPE, "out aliases an input");
    if (num_seqs == 0) return KDA_OK;

    if (validate_env()) {
        std::vector<int32_t> h(size_t(num_seqs) + 1);
        hipError_t e = hipMemcpyAsync(h.data(), cu_seqlens, h.size() * sizeof(int32_t),
                                      hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess)
            return fail(KDA_E_HIP, "reading cu_seqlens: %s", hipGetErrorString(e));
        if (h[0] != 0) return fail(KDA_E_SEQLENS, "cu_seqlens[0] = %d, expected 0", h[0]);
        for (int32_t n = 0; n < num_seqs; ++n)
            if (h[n + 1] < h[n]) return fail(KDA_E_SEQLENS, "cu_seqlens decreases at %d", n);
        if (h[num_seqs] != total_tokens)
            return fail(KDA_E_SEQLENS, "cu_seqlens[N] = %d, expected total_tokens = %lld",
                        h[num_seqs], (long long)total_tokens);
    }

    kda::LaunchArgs a{q, k, v, log_alpha, beta, cu_seqlens, out, final_state, total_tokens,
                      num_seqs, num_heads, d_k, d_v, dtype == KDA_BF16 ? 1 : 0, stream};
    const hipError_t e = (a.dtype_bf16 && !sequential_env()) ? kda::launch_forward_pipe(a)
                                                              : kda::launch_forward_seq(a);
    if (e != hipSuccess) return fail(KDA_E_HIP, "launch failed: %s", hipGetErrorString(e));
    return KDA_OK;
}

}  // extern "C"
