// kda_internal.h -- launch interface between the C ABI and the HIP kernels.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct LaunchArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* log_alpha;
    const void* beta;
    const int32_t* cu_seqlens;
    void* out;
    float* final_state;
    const float* init_state;        // [num_seqs][num_heads][d_k][d_v] fp32 or NULL (zero state)
    int64_t total_tokens;
    int32_t num_seqs;
    int32_t num_heads;
    int32_t d_k;
    int32_t d_v;
    int32_t dtype_bf16;
    hipStream_t stream;
    int32_t qk_l2norm;              // nonzero: q_t, k_t divided by their length on load
};

// Scan variants (arguments already validated).
// Sequential: 4 waves per (sample, head, 64-column tile), 64-token chunks for bf16
// and 32-token chunks for fp32, one chunk at a time.
hipError_t launch_forward_seq(const LaunchArgs& a);

// Records a pair of HIP events on the launch stream around each kernel launch
// (diagnostic per-kernel timing; NULL when off).
struct TimingHook {
    virtual void begin(const char* kernel, hipStream_t stream) = 0;
    virtual void end(hipStream_t stream) = 0;
    virtual ~TimingHook() = default;
};

// Fused path (bf16, d_k = d_v = 128): one workgroup per (sample segment, head) computes
// every chunk's operands on the CU and carries the state; samples are cut into segments
// (a summary pass, a combine and the output pass) when they give too few workgroups.
// `workspace` must hold fused_workspace_bytes(...) bytes (0 when no sample is cut),
// 256-byte aligned. `cap` bounds the workspace: the segment plan takes fewer, longer
// segments (or none) so that it fits; the same cap must be passed to both calls.
bool fused_supported(const LaunchArgs& a);
hipError_t launch_forward_fused(const LaunchArgs& a, void* workspace, TimingHook* th, size_t cap = SIZE_MAX);
size_t fused_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_heads, size_t cap = SIZE_MAX);

// The library's fixed device buffer of noalloc_scratch_bytes() bytes on the current device
// (its address there, looked up once per device); shared by every call on that device.
hipError_t noalloc_scratch(void** ptr);
size_t noalloc_scratch_bytes();

// Two-kernel path (bf16 only): a prep kernel over all (64-token chunk, head) pairs
// writes the chunk operands to `workspace`, a chain kernel carries the state.
// `workspace` must hold wy_workspace_bytes(...) bytes, 256-byte aligned.
hipError_t launch_forward_wy(const LaunchArgs& a, void* workspace, TimingHook* th);
size_t wy_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_heads, int d_k, int d_v);
// Bytes of one (64-token chunk, head) record of the workspace.
size_t wy_record_bytes(int d_k, int d_v);

// Backward (gradients of the scan): chunk table, prep, forward state chain, reverse
// state-gradient chain and a chunk-parallel gradient kernel; fp32 arithmetic.
struct BwdArgs {
    const void *q, *k, *v, *log_alpha, *beta;
    const int32_t* cu_seqlens;
    const float* init_state;        // [N][H][d_k][d_v] or NULL
    const void* d_out;              // [T][H][d_v] dtype
    const float* d_final_state;     // [N][H][d_k][d_v] or NULL
    void *dq, *dk, *dv, *dlog_alpha, *dbeta;
    float* d_init_state;            // [N][H][d_k][d_v] or NULL
    int64_t total_tokens;
    int32_t num_seqs, num_heads, d_k, d_v, dtype_bf16, qk_l2norm;
    hipStream_t stream;
};
hipError_t launch_backward(const BwdArgs& a, void* workspace, TimingHook* th);
size_t bwd_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_heads, int d_k, int d_v);

// Modality-aware short convolution over packed samples (workspace: the tile table).
struct ConvArgs {
    const void* x;
    const float *w_text, *w_vis;    // [k_text][C], [k_t][k_h][k_w][C]
    const int32_t *cu_seqlens, *text_len, *grid;   // [N+1], [N], [N][3]
    void* y;
    int64_t total_tokens;
    int32_t num_seqs, channels, k_text, k_t, k_h, k_w, dtype_bf16;
    hipStream_t stream;
};
hipError_t launch_short_conv(const ConvArgs& a, void* workspace, TimingHook* th);
size_t conv_workspace_bytes(int32_t num_seqs);

// Its reverse mode: f holds the forward's arguments (f.y unused); dy in, dx, dw_text, dw_vis out.
struct ConvBwdArgs {
    ConvArgs f;
    const void* dy;
    void* dx;
    float *dw_text, *dw_vis;
};
hipError_t launch_short_conv_backward(const ConvBwdArgs& a, void* workspace, TimingHook* th);
size_t conv_bwd_workspace_bytes(int32_t num_seqs, int32_t channels, int32_t k_text, int32_t k_t, int32_t k_h,
                                int32_t k_w);

// Auxiliary streams for work that runs beside the caller's stream inside one call: idx
// 0..3, one set per host thread and device, default priority, created on first use, each
// with a fork event (recorded on the caller's stream, waited on by the aux stream) and a
// join event (recorded on the aux stream, waited on by the caller's stream).
struct AuxStream {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
hipError_t aux_stream(int idx, AuxStream*& out);
// fork: `aux` starts after the work enqueued so far on `main`
hipError_t aux_fork(hipStream_t main, AuxStream* aux);
// join: work enqueued next on `main` waits for the work enqueued so far on `aux`
hipError_t aux_join(hipStream_t main, AuxStream* aux);

// LDS bytes one workgroup uses.
size_t smem_bytes(int dtype_bf16, int d_k);

}  // namespace kda
