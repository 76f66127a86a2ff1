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
    int64_t total_tokens;
    int32_t num_seqs;
    int32_t num_heads;
    int32_t d_k;
    int32_t d_v;
    int32_t dtype_bf16;
    hipStream_t stream;
};

// Scan variants (arguments already validated).
// Sequential: 4 waves per (sample, head, 64-column tile), 64-token chunks for bf16
// and 32-token chunks for fp32, one chunk at a time.
hipError_t launch_forward_seq(const LaunchArgs& a);
// Pipelined (bf16 only): 8 waves, 32-token chunks, the decayed operands of the
// next chunk computed while the current chunk's products run.
hipError_t launch_forward_pipe(const LaunchArgs& a);

// LDS bytes one workgroup uses.
size_t smem_bytes(int dtype_bf16, int d_k);
size_t smem_bytes_pipe(int d_k);

}  // namespace kda
