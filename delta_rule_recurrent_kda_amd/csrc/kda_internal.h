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

// Enqueue the scan. Arguments are already validated.
hipError_t launch_forward(const LaunchArgs& a);

// LDS bytes one workgroup of the scan kernel uses.
size_t smem_bytes(int dtype_bf16, int d_k);

}  // namespace kda
