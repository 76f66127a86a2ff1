// kda_api.cpp -- C ABI of libkda: argument checks, error reporting, dispatch.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
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

// A caller's array as a byte range; a NULL pointer or an empty range overlaps nothing.
struct Span {
    const void* p;
    int64_t bytes;
    const char* name;
};
bool overlap(const Span& a, const Span& b)
{
    if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a.p), y = reinterpret_cast<uintptr_t>(b.p);
    return x < y + uintptr_t(b.bytes) && y < x + uintptr_t(a.bytes);
}
// every output against every input and against the other outputs
kda_status check_overlaps(const Span* outs, int nout, const Span* ins, int nin)
{
    for (int o = 0; o < nout; ++o) {
        for (int i = 0; i < nin; ++i)
            if (overlap(outs[o], ins[i])) return fail(KDA_E_SHAPE, "%s overlaps %s", outs[o].name, ins[i].name);
        for (int j = o + 1; j < nout; ++j)
            if (overlap(outs[o], outs[j])) return fail(KDA_E_SHAPE, "%s overlaps %s", outs[o].name, outs[j].name);
    }
    return KDA_OK;
}

}  // namespace

namespace kda {

hipError_t aux_stream(int idx, AuxStream*& out)
{
    static thread_local AuxStream cache[16][4];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 16 || idx < 0 || idx >= 4) return hipErrorInvalidValue;
    AuxStream& s = cache[dev][idx];
    if (!s.stream) {
        AuxStream n;
        if ((e = hipStreamCreateWithFlags(&n.stream, hipStreamNonBlocking)) != hipSuccess) return e;
        if ((e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming)) != hipSuccess) return e;
        if ((e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming)) != hipSuccess) return e;
        s = n;
    }
    out = &s;
    return hipSuccess;
}

hipError_t aux_fork(hipStream_t main, AuxStream* aux)
{
    hipError_t e = hipEventRecord(aux->fork, main);
    return e != hipSuccess ? e : hipStreamWaitEvent(aux->stream, aux->fork, 0);
}

hipError_t aux_join(hipStream_t main, AuxStream* aux)
{
    hipError_t e = hipEventRecord(aux->join, aux->stream);
    return e != hipSuccess ? e : hipStreamWaitEvent(main, aux->join, 0);
}

}  // namespace kda

namespace {

bool validate_env()
{
    const char* e = std::getenv("KDA_VALIDATE");
    return e && e[0] == '1';
}

// KDA_SCAN_VARIANT selects the bf16 scan: "fused" (the default for d_k = d_v = 128: one
// kernel that computes every chunk's operands on the CU), "wy" (the default for other
// sizes: a prep kernel over all chunks and a chain kernel, with a workspace) or
// "sequential" (one chunk at a time). fp32 data always uses the sequential kernel.
enum class Variant { Wy, Fused, Sequential };
Variant variant_env()
{
    const char* e = std::getenv("KDA_SCAN_VARIANT");
    if (e && std::strcmp(e, "sequential") == 0) return Variant::Sequential;
    if (e && std::strcmp(e, "wy") == 0) return Variant::Wy;
    return Variant::Fused;
}

// ---- per-kernel event timing (diagnostics) ----
struct Timing : kda::TimingHook {
    std::mutex mu;
    bool on = false;
    std::vector<hipEvent_t> free_events;
    struct Rec { std::string name; hipEvent_t start, stop; };
    std::vector<Rec> recs;
    std::string cur;
    hipEvent_t cur_start = nullptr;

    hipEvent_t get() {
        if (!free_events.empty()) {
            hipEvent_t e = free_events.back();
            free_events.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        return e;
    }
    // a launch whose events cannot be recorded is left out of the records
    void begin(const char* kernel, hipStream_t stream) override {
        cur = kernel;
        cur_start = get();
        if (cur_start && hipEventRecord(cur_start, stream) != hipSuccess) {
            free_events.push_back(cur_start);
            cur_start = nullptr;
        }
    }
    void end(hipStream_t stream) override {
        if (!cur_start) return;
        hipEvent_t stop = get();
        if (!stop || hipEventRecord(stop, stream) != hipSuccess) {
            free_events.push_back(cur_start);
            if (stop) free_events.push_back(stop);
            cur_start = nullptr;
            return;
        }
        recs.push_back({cur, cur_start, stop});
        cur_start = nullptr;
    }
};
Timing g_timing;

// The device's default stream-ordered pool keeps freed workspace for reuse instead of
// returning it to the driver at every synchronisation.
std::mutex g_pool_mu;
std::vector<bool> g_pool_done;           // devices whose default pool the library has prepared

bool prepare_pool(int dev)
{
    std::lock_guard<std::mutex> lk(g_pool_mu);
    if (dev < 0) return false;
    if (size_t(dev) >= g_pool_done.size()) g_pool_done.resize(size_t(dev) + 1, false);
    if (g_pool_done[size_t(dev)]) return true;
    hipMemPool_t pool = nullptr;
    if (hipDeviceGetDefaultMemPool(&pool, dev) != hipSuccess) return false;
    uint64_t thr = UINT64_MAX;
    if (hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr) != hipSuccess) return false;
    g_pool_done[size_t(dev)] = true;
    return true;
}

kda_status check_args(const void* q, const void* k, const void* v, const void* log_alpha,
                      const void* beta, const int32_t* cu_seqlens, void* out, float* final_state,
                      const float* initial_state, int64_t total_tokens, int32_t num_seqs,
                      int32_t num_heads, int32_t d_k, int32_t d_v, kda_dtype dtype, uint32_t options,
                      hipStream_t stream, bool host_checks = true);
kda_status run(const kda::LaunchArgs& a);

bool debug_sync_env()
{
    const char* e = std::getenv("KDA_DEBUG_SYNC");
    return e && e[0] == '1';
}

// The end of every call that enqueued work: a launch error, or else, under KDA_DEBUG_SYNC=1
// and outside stream capture, the stream's completion, so that a failed kernel is reported by
// the call that enqueued it rather than by a later one.
kda_status finish(hipError_t e, hipStream_t stream)
{
    if (e != hipSuccess) return fail(KDA_E_HIP, "launch failed: %s", hipGetErrorString(e));
    if (!debug_sync_env()) return KDA_OK;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if ((e = hipStreamIsCapturing(stream, &cs)) != hipSuccess)
        return fail(KDA_E_HIP, "KDA_DEBUG_SYNC: stream capture status: %s", hipGetErrorString(e));
    if (cs != hipStreamCaptureStatusNone) return KDA_OK;
    if ((e = hipStreamSynchronize(stream)) != hipSuccess)
        return fail(KDA_E_HIP, "KDA_DEBUG_SYNC: the call's kernels failed: %s", hipGetErrorString(e));
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_release(void)
{
    std::lock_guard<std::mutex> lk(g_pool_mu);
    for (size_t d = 0; d < g_pool_done.size(); ++d) {
        if (!g_pool_done[d]) continue;
        hipMemPool_t pool = nullptr;
        hipError_t e = hipDeviceGetDefaultMemPool(&pool, int(d));
        if (e == hipSuccess) e = hipMemPoolTrimTo(pool, 0);
        if (e != hipSuccess) return fail(KDA_E_HIP, "kda_release, device %zu: %s", d, hipGetErrorString(e));
    }
    return KDA_OK;
}

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
    const kda_status st = check_args(q, k, v, log_alpha, beta, cu_seqlens, out, final_state, nullptr,
                                     total_tokens, num_seqs, num_heads, d_k, d_v, dtype, 0u, stream);
    if (st != KDA_OK || num_seqs == 0) return st;
    return run(kda::LaunchArgs{q, k, v, log_alpha, beta, cu_seqlens, out, final_state, nullptr,
                               total_tokens, num_seqs, num_heads, d_k, d_v, dtype == KDA_BF16 ? 1 : 0,
                               stream, 0});
}

kda_status kda_forward_from_state(const void* q, const void* k, const void* v, const void* log_alpha,
                                  const void* beta, const int32_t* cu_seqlens,
                                  const float* initial_state, void* out, float* final_state,
                                  int64_t total_tokens, int32_t num_seqs, int32_t num_heads,
                                  int32_t d_k, int32_t d_v, kda_dtype dtype, hipStream_t stream)
{
    g_last_error.clear();
    return kda_forward_ex(q, k, v, log_alpha, beta, cu_seqlens, initial_state, out, final_state,
                          total_tokens, num_seqs, num_heads, d_k, d_v, dtype, 0u, stream);
}

kda_status kda_forward_ex(const void* q, const void* k, const void* v, const void* log_alpha,
                          const void* beta, const int32_t* cu_seqlens, const float* initial_state,
                          void* out, float* final_state, int64_t total_tokens, int32_t num_seqs,
                          int32_t num_heads, int32_t d_k, int32_t d_v, kda_dtype dtype, uint32_t options,
                          hipStream_t stream)
{
    g_last_error.clear();
    const kda_status st = check_args(q, k, v, log_alpha, beta, cu_seqlens, out, final_state,
                                     initial_state, total_tokens, num_seqs, num_heads, d_k, d_v, dtype,
                                     options, stream);
    if (st != KDA_OK || num_seqs == 0) return st;
    return run(kda::LaunchArgs{q, k, v, log_alpha, beta, cu_seqlens, out, final_state, initial_state,
                               total_tokens, num_seqs, num_heads, d_k, d_v, dtype == KDA_BF16 ? 1 : 0,
                               stream, (options & KDA_OPT_QK_L2NORM) ? 1 : 0});
}

kda_status kda_forward_noalloc(const void* q, const void* k, const void* v, const void* log_alpha,
                               const void* beta, const int32_t* cu_seqlens, const float* initial_state,
                               void* out, float* final_state, int64_t total_tokens, int32_t num_seqs,
                               int32_t num_heads, int32_t d_k, int32_t d_v, kda_dtype dtype,
                               uint32_t options, hipStream_t stream)
{
    g_last_error.clear();
    const kda_status st = check_args(q, k, v, log_alpha, beta, cu_seqlens, out, final_state,
                                     initial_state, total_tokens, num_seqs, num_heads, d_k, d_v, dtype,
                                     options, stream, false);
    if (st != KDA_OK || num_seqs == 0) return st;
    const kda::LaunchArgs a{q, k, v, log_alpha, beta, cu_seqlens, out, final_state, initial_state,
                            total_tokens, num_seqs, num_heads, d_k, d_v, dtype == KDA_BF16 ? 1 : 0,
                            stream, (options & KDA_OPT_QK_L2NORM) ? 1 : 0};
    hipError_t e;
    if (kda::fused_supported(a)) {
        const size_t cap = kda::noalloc_scratch_bytes();
        const size_t bytes = kda::fused_workspace_bytes(total_tokens, num_seqs, num_heads, cap);
        if (bytes > cap)
            return fail(KDA_E_UNSUPPORTED, "the scan needs %zu bytes of scratch, more than the fixed %zu",
                        bytes, cap);
        void* ws = nullptr;
        if (bytes && (e = kda::noalloc_scratch(&ws)) != hipSuccess)
            return fail(KDA_E_HIP, "looking up the scratch buffer: %s", hipGetErrorString(e));
        e = kda::launch_forward_fused(a, ws, nullptr, cap);
    } else {
        e = kda::launch_forward_seq(a);
    }
    return finish(e, stream);
}

kda_status kda_backward(const void* q, const void* k, const void* v, const void* log_alpha,
                        const void* beta, const int32_t* cu_seqlens, const float* initial_state,
                        const void* d_out, const float* d_final_state, void* dq, void* dk, void* dv,
                        void* dlog_alpha, void* dbeta, float* d_initial_state, int64_t total_tokens,
                        int32_t num_seqs, int32_t num_heads, int32_t d_k, int32_t d_v, kda_dtype dtype,
                        uint32_t options, hipStream_t stream)
{
    g_last_error.clear();
    if (options & ~uint32_t(KDA_OPT_QK_L2NORM))
        return fail(KDA_E_UNSUPPORTED, "unknown option bits 0x%x", unsigned(options & ~uint32_t(KDA_OPT_QK_L2NORM)));
    // the forward-argument checks on the inputs (no output there: pass q as a stand-in
    // that aliases nothing of its own)
    kda_status st = check_args(q, k, v, log_alpha, beta, cu_seqlens, dq, nullptr, nullptr, total_tokens,
                               num_seqs, num_heads, d_k, d_v, dtype, 0u, stream);
    if (st != KDA_OK) return st;
    if (total_tokens > 0 && (!d_out || !dq || !dk || !dv || !dlog_alpha || !dbeta))
        return fail(KDA_E_NULL, "d_out or a gradient pointer is NULL");
    const void* ptrs[] = {d_out, dk, dv, dlog_alpha, dbeta, initial_state, d_final_state, d_initial_state};
    const char* names[] = {"d_out", "dk", "dv", "dlog_alpha", "dbeta", "initial_state", "d_final_state",
                           "d_initial_state"};
    for (int i = 0; i < 8; ++i)
        if (ptrs[i] && !aligned16(ptrs[i])) return fail(KDA_E_ALIGN, "%s is not 16-byte aligned", names[i]);
    {
        const int64_t es = dtype == KDA_BF16 ? 2 : 4, th = total_tokens * num_heads;
        const int64_t st_bytes = int64_t(num_seqs) * num_heads * d_k * d_v * 4;
        const Span ins[] = {{q, th * d_k * es, "q"}, {k, th * d_k * es, "k"}, {v, th * d_v * es, "v"},
                            {log_alpha, th * d_k * es, "log_alpha"}, {beta, th * es, "beta"},
                            {cu_seqlens, (int64_t(num_seqs) + 1) * 4, "cu_seqlens"},
                            {d_out, th * d_v * es, "d_out"}, {initial_state, st_bytes, "initial_state"},
                            {d_final_state, st_bytes, "d_final_state"}};
        const Span outs[] = {{dq, th * d_k * es, "dq"}, {dk, th * d_k * es, "dk"}, {dv, th * d_v * es, "dv"},
                             {dlog_alpha, th * d_k * es, "dlog_alpha"}, {dbeta, th * es, "dbeta"},
                             {d_initial_state, st_bytes, "d_initial_state"}};
        if ((st = check_overlaps(outs, 6, ins, 9)) != KDA_OK) return st;
    }
    if (num_seqs == 0) return KDA_OK;

    std::unique_lock<std::mutex> lk(g_timing.mu);
    kda::TimingHook* th = g_timing.on ? &g_timing : nullptr;
    if (!th) lk.unlock();
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || !prepare_pool(dev))
        return fail(KDA_E_HIP, "setting up the workspace pool: %s", hipGetErrorString(e));
    const size_t bytes = kda::bwd_workspace_bytes(total_tokens, num_seqs, num_heads, d_k, d_v);
    void* ws = nullptr;
    e = hipMallocAsync(&ws, bytes, stream);
    if (e != hipSuccess) return fail(KDA_E_HIP, "workspace of %zu bytes: %s", bytes, hipGetErrorString(e));
    const kda::BwdArgs a{q, k, v, log_alpha, beta, cu_seqlens, initial_state, d_out, d_final_state, dq, dk, dv,
                         dlog_alpha, dbeta, d_initial_state, total_tokens, num_seqs, num_heads, d_k, d_v,
                         dtype == KDA_BF16 ? 1 : 0, (options & KDA_OPT_QK_L2NORM) ? 1 : 0, stream};
    e = kda::launch_backward(a, ws, th);
    const hipError_t ef = hipFreeAsync(ws, stream);
    if (e == hipSuccess) e = ef;
    return finish(e, stream);
}

size_t kda_backward_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_heads, int32_t d_k,
                                    int32_t d_v)
{
    if (total_tokens < 0 || num_seqs <= 0 || num_heads < 1) return 0;
    if ((d_k != 64 && d_k != 128) || (d_v != 64 && d_v != 128)) return 0;
    return kda::bwd_workspace_bytes(total_tokens, num_seqs, num_heads, d_k, d_v);
}

namespace {

// Argument checks shared by the short convolution and its reverse mode; outs/ins are the
// byte ranges that must not overlap. Reads the sample tables back under KDA_VALIDATE=1.
kda_status conv_check(const void* x, const float* w_text, const float* w_vis, const int32_t* cu_seqlens,
                      const int32_t* text_len, const int32_t* grid, int64_t total_tokens, int32_t num_seqs,
                      int32_t channels, int32_t k_text, int32_t k_t, int32_t k_h, int32_t k_w, kda_dtype dtype,
                      const Span* outs, int nout, const void* const* tok_outs, int ntok_out, hipStream_t stream)
{
    if (dtype != KDA_F32 && dtype != KDA_BF16)
        return fail(KDA_E_DTYPE, "dtype %d is neither KDA_F32 nor KDA_BF16", int(dtype));
    if (total_tokens < 0 || num_seqs < 0 || channels < 1)
        return fail(KDA_E_SHAPE, "bad sizes: total_tokens=%lld num_seqs=%d channels=%d", (long long)total_tokens,
                    num_seqs, channels);
    if (channels % 8 != 0)
        return fail(KDA_E_UNSUPPORTED, "channels=%d: a multiple of 8 is required", channels);
    if (k_text < 1 || k_text > 8 || k_t < 1 || k_t > 4 || k_h < 1 || k_h > 5 || k_w < 1 || k_w > 5 ||
        k_h % 2 == 0 || k_w % 2 == 0)
        return fail(KDA_E_UNSUPPORTED, "kernel sizes text %d, visual %dx%dx%d: supported text 1..8, time 1..4, "
                    "height and width odd 1..5", k_text, k_t, k_h, k_w);
    if (total_tokens * channels >= (int64_t(1) << 31))
        return fail(KDA_E_UNSUPPORTED, "problem too large for 32-bit element offsets");
    if (!cu_seqlens || (num_seqs > 0 && (!text_len || !grid)))
        return fail(KDA_E_NULL, "cu_seqlens, text_len or grid is NULL");
    if (total_tokens > 0 && (!x || !w_text || !w_vis)) return fail(KDA_E_NULL, "a tensor pointer is NULL");
    for (int i = 0; i < nout; ++i)
        if (total_tokens > 0 && !outs[i].p) return fail(KDA_E_NULL, "%s is NULL", outs[i].name);
    if (x && !aligned16(x)) return fail(KDA_E_ALIGN, "x is not 16-byte aligned");
    for (int i = 0; i < ntok_out; ++i)
        if (tok_outs[i] && !aligned16(tok_outs[i])) return fail(KDA_E_ALIGN, "a token tensor is not 16-byte aligned");
    {
        const int64_t es = dtype == KDA_BF16 ? 2 : 4;
        const Span ins[] = {{x, total_tokens * channels * es, "x"},
                            {w_text, int64_t(k_text) * channels * 4, "w_text"},
                            {w_vis, int64_t(k_t) * k_h * k_w * channels * 4, "w_vis"},
                            {cu_seqlens, (int64_t(num_seqs) + 1) * 4, "cu_seqlens"},
                            {text_len, int64_t(num_seqs) * 4, "text_len"},
                            {grid, int64_t(num_seqs) * 12, "grid"}};
        const kda_status st = check_overlaps(outs, nout, ins, 6);
        if (st != KDA_OK) return st;
    }
    if (num_seqs == 0 || total_tokens == 0) return KDA_OK;
    if (validate_env()) {
        std::vector<int32_t> hc(size_t(num_seqs) + 1), ht(num_seqs), hg(size_t(num_seqs) * 3);
        hipError_t e = hipMemcpyAsync(hc.data(), cu_seqlens, hc.size() * 4, hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipMemcpyAsync(ht.data(), text_len, ht.size() * 4, hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipMemcpyAsync(hg.data(), grid, hg.size() * 4, hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return fail(KDA_E_HIP, "reading the sample tables: %s", hipGetErrorString(e));
        if (hc[0] != 0 || hc[num_seqs] != total_tokens) return fail(KDA_E_SEQLENS, "cu_seqlens does not span the tokens");
        for (int32_t n = 0; n < num_seqs; ++n) {
            const int64_t len = int64_t(hc[n + 1]) - hc[n];
            const int64_t vis = int64_t(hg[3 * n]) * hg[3 * n + 1] * hg[3 * n + 2];
            if (len < 0 || ht[n] < 0 || hg[3 * n] < 0 || hg[3 * n + 1] < 0 || hg[3 * n + 2] < 0 || ht[n] + vis != len)
                return fail(KDA_E_SEQLENS, "sample %d: text_len + T*H*W != its length", n);
        }
    }
    return KDA_OK;
}

}  // namespace

kda_status kda_short_conv(const void* x, const float* w_text, const float* w_vis, const int32_t* cu_seqlens,
                          const int32_t* text_len, const int32_t* grid, void* y, int64_t total_tokens,
                          int32_t num_seqs, int32_t channels, int32_t k_text, int32_t k_t, int32_t k_h, int32_t k_w,
                          kda_dtype dtype, hipStream_t stream)
{
    g_last_error.clear();
    const int64_t es = dtype == KDA_BF16 ? 2 : 4;
    const Span outs[] = {{y, total_tokens * channels * es, "y"}};
    const void* const tok_outs[] = {y};
    kda_status st = conv_check(x, w_text, w_vis, cu_seqlens, text_len, grid, total_tokens, num_seqs, channels,
                               k_text, k_t, k_h, k_w, dtype, outs, 1, tok_outs, 1, stream);
    if (st != KDA_OK || num_seqs == 0 || total_tokens == 0) return st;
    std::unique_lock<std::mutex> lk(g_timing.mu);
    kda::TimingHook* th = g_timing.on ? &g_timing : nullptr;
    if (!th) lk.unlock();
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || !prepare_pool(dev))
        return fail(KDA_E_HIP, "setting up the workspace pool: %s", hipGetErrorString(e));
    void* ws = nullptr;
    const size_t bytes = kda::conv_workspace_bytes(num_seqs);
    e = hipMallocAsync(&ws, bytes, stream);
    if (e != hipSuccess) return fail(KDA_E_HIP, "workspace of %zu bytes: %s", bytes, hipGetErrorString(e));
    const kda::ConvArgs a{x, w_text, w_vis, cu_seqlens, text_len, grid, y, total_tokens, num_seqs, channels,
                          k_text, k_t, k_h, k_w, dtype == KDA_BF16 ? 1 : 0, stream};
    e = kda::launch_short_conv(a, ws, th);
    const hipError_t ef = hipFreeAsync(ws, stream);
    if (e == hipSuccess) e = ef;
    return finish(e, stream);
}

kda_status kda_short_conv_backward(const void* x, const float* w_text, const float* w_vis,
                                   const int32_t* cu_seqlens, const int32_t* text_len, const int32_t* grid,
                                   const void* dy, void* dx, float* dw_text, float* dw_vis, int64_t total_tokens,
                                   int32_t num_seqs, int32_t channels, int32_t k_text, int32_t k_t, int32_t k_h,
                                   int32_t k_w, kda_dtype dtype, hipStream_t stream)
{
    g_last_error.clear();
    const int64_t es = dtype == KDA_BF16 ? 2 : 4;
    if (total_tokens > 0 && !dy) return fail(KDA_E_NULL, "dy is NULL");
    if (dy && !aligned16(dy)) return fail(KDA_E_ALIGN, "dy is not 16-byte aligned");
    const Span outs[] = {{dx, total_tokens * channels * es, "dx"},
                         {dw_text, int64_t(k_text) * channels * 4, "dw_text"},
                         {dw_vis, int64_t(k_t) * k_h * k_w * channels * 4, "dw_vis"}};
    const void* const tok_outs[] = {dx};
    kda_status st = conv_check(x, w_text, w_vis, cu_seqlens, text_len, grid, total_tokens, num_seqs, channels,
                               k_text, k_t, k_h, k_w, dtype, outs, 3, tok_outs, 1, stream);
    if (st != KDA_OK) return st;
    {
        const Span dys[] = {{dy, total_tokens * channels * es, "dy"}};
        st = check_overlaps(outs, 3, dys, 1);
        if (st != KDA_OK) return st;
    }
    std::unique_lock<std::mutex> lk(g_timing.mu);
    kda::TimingHook* th = g_timing.on ? &g_timing : nullptr;
    if (!th) lk.unlock();
    const kda::ConvBwdArgs a{{x, w_text, w_vis, cu_seqlens, text_len, grid, nullptr, total_tokens, num_seqs,
                              channels, k_text, k_t, k_h, k_w, dtype == KDA_BF16 ? 1 : 0, stream},
                             dy, dx, dw_text, dw_vis};
    if (num_seqs == 0 || total_tokens == 0) {
        // no tokens: the weight gradients are empty sums, written as zeros without a workspace
        if (!dw_text || !dw_vis) return fail(KDA_E_NULL, "dw_text or dw_vis is NULL");
        return finish(kda::launch_short_conv_backward(a, nullptr, th), stream);
    }
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || !prepare_pool(dev))
        return fail(KDA_E_HIP, "setting up the workspace pool: %s", hipGetErrorString(e));
    void* ws = nullptr;
    const size_t bytes = kda::conv_bwd_workspace_bytes(num_seqs, channels, k_text, k_t, k_h, k_w);
    e = hipMallocAsync(&ws, bytes, stream);
    if (e != hipSuccess) return fail(KDA_E_HIP, "workspace of %zu bytes: %s", bytes, hipGetErrorString(e));
    e = kda::launch_short_conv_backward(a, ws, th);
    const hipError_t ef = hipFreeAsync(ws, stream);
    if (e == hipSuccess) e = ef;
    return finish(e, stream);
}

kda_status kda_timing_enable(int32_t on)
{
    std::lock_guard<std::mutex> lk(g_timing.mu);
    g_timing.on = on != 0;
    return KDA_OK;
}

kda_status kda_timing_read(const char* kernel, int32_t* launches, double* total_ms)
{
    g_last_error.clear();
    if (!kernel || !launches || !total_ms) return fail(KDA_E_NULL, "kda_timing_read: NULL argument");
    std::lock_guard<std::mutex> lk(g_timing.mu);
    int32_t n = 0;
    double ms = 0.0;
    std::vector<Timing::Rec> keep;
    for (auto& rec : g_timing.recs) {
        if (rec.name != kernel) {
            keep.push_back(rec);
            continue;
        }
        hipError_t e = hipEventSynchronize(rec.stop);
        float t = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&t, rec.start, rec.stop);
        if (e != hipSuccess) {
            g_timing.recs.clear();
            return fail(KDA_E_HIP, "kda_timing_read: %s", hipGetErrorString(e));
        }
        ++n;
        ms += t;
        g_timing.free_events.push_back(rec.start);
        g_timing.free_events.push_back(rec.stop);
    }
    g_timing.recs.swap(keep);
    *launches = n;
    *total_ms = ms;
    return KDA_OK;
}

size_t kda_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_heads, int32_t d_k,
                           int32_t d_v, kda_dtype dtype)
{
    if (dtype != KDA_BF16 || total_tokens < 0 || num_seqs <= 0 || num_heads < 1) return 0;
    if ((d_k != 64 && d_k != 128) || (d_v != 64 && d_v != 128)) return 0;
    const Variant var = variant_env();
    if (var == Variant::Sequential) return 0;
    if (d_k == 128 && d_v == 128 && var == Variant::Fused)
        return kda::fused_workspace_bytes(total_tokens, num_seqs, num_heads);
    return kda::wy_workspace_bytes(total_tokens, num_seqs, num_heads, d_k, d_v);
}

}  // extern "C"

namespace {

kda_status check_args(const void* q, const void* k, const void* v, const void* log_alpha,
                      const void* beta, const int32_t* cu_seqlens, void* out, float* final_state,
                      const float* initial_state, int64_t total_tokens, int32_t num_seqs,
                      int32_t num_heads, int32_t d_k, int32_t d_v, kda_dtype dtype, uint32_t options,
                      hipStream_t stream, bool host_checks)
{
    if (options & ~uint32_t(KDA_OPT_QK_L2NORM))
        return fail(KDA_E_UNSUPPORTED, "unknown option bits 0x%x", unsigned(options & ~uint32_t(KDA_OPT_QK_L2NORM)));
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
    const void* ptrs[] = {q, k, v, log_alpha, beta, cu_seqlens, out, final_state, initial_state};
    const char* names[] = {"q", "k", "v", "log_alpha", "beta", "cu_seqlens", "out", "final_state",
                           "initial_state"};
    for (int i = 0; i < 9; ++i)
        if (ptrs[i] && !aligned16(ptrs[i]))
            return fail(KDA_E_ALIGN, "%s is not 16-byte aligned", names[i]);
    {
        const int64_t es = dtype == KDA_BF16 ? 2 : 4, th = total_tokens * num_heads;
        const int64_t st_bytes = int64_t(num_seqs) * num_heads * d_k * d_v * 4;
        const Span ins[] = {{q, th * d_k * es, "q"}, {k, th * d_k * es, "k"}, {v, th * d_v * es, "v"},
                            {log_alpha, th * d_k * es, "log_alpha"}, {beta, th * es, "beta"},
                            {cu_seqlens, (int64_t(num_seqs) + 1) * 4, "cu_seqlens"},
                            {initial_state, st_bytes, "initial_state"}};
        const Span outs[] = {{out, th * d_v * es, "out"}, {final_state, st_bytes, "final_state"}};
        const kda_status st = check_overlaps(outs, 2, ins, 7);
        if (st != KDA_OK) return st;
    }
    if (num_seqs == 0) return KDA_OK;

    if (host_checks && validate_env()) {
        std::vector<int32_t> h(size_t(num_seqs) + 1);
        hipError_t e = hipMemcpyAsync(h.data(), cu_seqlens, h.size() * sizeof(int32_t),
                                      hipMemcpyDeviceToHost, stream);
        if (e == hipSuccess) e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return fail(KDA_E_HIP, "reading cu_seqlens: %s", hipGetErrorString(e));
        if (h[0] != 0) return fail(KDA_E_SEQLENS, "cu_seqlens[0] = %d, expected 0", h[0]);
        for (int32_t n = 0; n < num_seqs; ++n)
            if (h[n + 1] < h[n]) return fail(KDA_E_SEQLENS, "cu_seqlens decreases at %d", n);
        if (h[num_seqs] != total_tokens)
            return fail(KDA_E_SEQLENS, "cu_seqlens[N] = %d, expected total_tokens = %lld",
                        h[num_seqs], (long long)total_tokens);
    }
    return KDA_OK;
}

kda_status run(const kda::LaunchArgs& a)
{
    std::unique_lock<std::mutex> lk(g_timing.mu);
    kda::TimingHook* th = g_timing.on ? &g_timing : nullptr;
    if (!th) lk.unlock();
    const Variant var = a.dtype_bf16 ? variant_env() : Variant::Sequential;
    hipError_t e = hipSuccess;
    if (var != Variant::Sequential) {
        const bool fused = var == Variant::Fused && kda::fused_supported(a);
        const size_t bytes = fused ? kda::fused_workspace_bytes(a.total_tokens, a.num_seqs, a.num_heads)
                                   : kda::wy_workspace_bytes(a.total_tokens, a.num_seqs, a.num_heads, a.d_k, a.d_v);
        void* ws = nullptr;
        if (bytes) {
            int dev = -1;
            e = hipGetDevice(&dev);
            if (e != hipSuccess || !prepare_pool(dev))
                return fail(KDA_E_HIP, "setting up the workspace pool: %s", hipGetErrorString(e));
            e = hipMallocAsync(&ws, bytes, a.stream);
            if (e != hipSuccess)
                return fail(KDA_E_HIP, "workspace of %zu bytes: %s", bytes, hipGetErrorString(e));
        }
        e = fused ? kda::launch_forward_fused(a, ws, th) : kda::launch_forward_wy(a, ws, th);
        if (ws) {
            const hipError_t ef = hipFreeAsync(ws, a.stream);
            if (e == hipSuccess) e = ef;
        }
    } else {
        if (th) th->begin("scan", a.stream);
        e = kda::launch_forward_seq(a);
        if (th) th->end(a.stream);
    }
    return finish(e, a.stream);
}

}  // namespace
