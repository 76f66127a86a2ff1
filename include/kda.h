/*
 * kda.h -- C ABI of the MI355X (gfx950) KDA forward-scan library, libkda.so.
 *
 * The operation (Chimera: Designing and Chinchilla-Scaling Hybrid Visual
 * Diffusion Transformers, arXiv 2607.28611):
 *
 *   per packed sample n and head h, for t over the sample's tokens in storage
 *   order (the single causal scan order shared by all heads, paper Sec. 3 KDA
 *   paragraph; visual tokens already in temporal-major raster order
 *   m = iHW + jW + k, explainer page "One stream, three mechanisms, no positions"):
 *
 *     S_0 = 0                                      reset at every packed-sample
 *                                                  boundary (paper Sec. 3, Eq. 14 text)
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *                                                  (explainer page, same section)
 *     o_t = S_t^T q_t                              readout of the post-update state
 *
 *   with alpha_t = exp(log_alpha_t) in (0,1]^{d_k} a forget gate per key
 *   channel, beta_t a scalar write/erase strength, S_t in R^{d_k x d_v}. No query
 *   scale and no normalisation is applied inside the operation.
 *
 * The library evaluates this recurrence in a chunkwise form on bf16/fp32 MFMA
 * with fp32 accumulation and an fp32 state; results agree with the token
 * recurrence up to floating-point rounding.
 */
#ifndef KDA_H
#define KDA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v, log_alpha, beta and out. final_state is always fp32. */
typedef enum {
    KDA_F32 = 0,
    KDA_BF16 = 1
} kda_dtype;

typedef enum {
    KDA_OK = 0,
    KDA_E_NULL = 1,         /* a required pointer is NULL                          */
    KDA_E_DTYPE = 2,        /* dtype is not KDA_F32 or KDA_BF16                    */
    KDA_E_SHAPE = 3,        /* negative or inconsistent sizes                      */
    KDA_E_ALIGN = 4,        /* a tensor pointer is not 16-byte aligned             */
    KDA_E_UNSUPPORTED = 5,  /* d_k or d_v outside {64, 128}, or sizes too large    */
    KDA_E_SEQLENS = 6,      /* cu_seqlens content invalid (checked when KDA_VALIDATE=1) */
    KDA_E_HIP = 7           /* a HIP runtime call or kernel launch failed           */
} kda_status;

/*
 * kda_forward -- the KDA forward scan over a packed token batch.
 *
 * All tensor pointers are DEVICE pointers on the current HIP device, C-contiguous:
 *   q, k, log_alpha : [total_tokens][num_heads][d_k]   dtype
 *   v               : [total_tokens][num_heads][d_v]   dtype
 *   beta            : [total_tokens][num_heads]        dtype
 *   cu_seqlens      : [num_seqs + 1] int32, 0 = c_0 <= c_1 <= ... <= c_N = total_tokens;
 *                     sample n owns tokens [c_n, c_{n+1}); zero-length samples allowed.
 *                     A dense [B][L] batch passes {0, L, 2L, ..., B*L}.
 *   out             : [total_tokens][num_heads][d_v]   dtype (written; may not alias inputs)
 *   final_state     : [num_seqs][num_heads][d_k][d_v] fp32, rows = key channels, the state
 *                     after each sample's last token (zeros for an empty sample). May be NULL.
 *
 * Sizes: d_k, d_v in {64, 128}; num_heads >= 1; num_seqs >= 0; total_tokens >= 0 and
 * total_tokens * num_heads * max(d_k, d_v) < 2^31. Pointers must be 16-byte aligned.
 *
 * Numerics: inputs are used as stored; internally fp32 state and accumulation. For
 * bf16 inputs the chunk contractions run on bf16 MFMA; out is rounded to nearest-even.
 * Precondition: within any 64-token chunk (32 for fp32 with d_k = 128) the summed
 * log_alpha of each key channel is above -80; stronger decay overflows the factored
 * per-chunk decay and gives non-finite results. NaN/Inf inputs propagate only within
 * their own (sample, head).
 *
 * Execution: enqueued on `stream` (NULL = the null stream) and returns without
 * synchronising; buffers must stay valid until the stream reaches the work. The
 * library keeps no pointer after returning and allocates no device memory on this
 * path. Results are bitwise deterministic for identical inputs on the same device.
 * cu_seqlens is read on the device; its content is checked on the host only when the
 * environment variable KDA_VALIDATE=1 (one synchronous device-to-host copy).
 *
 * Errors: returns KDA_OK or an error code; argument checks run before any launch and
 * nothing is enqueued on error. kda_last_error() gives a message for the calling thread.
 */
kda_status kda_forward(const void *q, const void *k, const void *v, const void *log_alpha,
                       const void *beta, const int32_t *cu_seqlens, void *out,
                       float *final_state, int64_t total_tokens, int32_t num_seqs,
                       int32_t num_heads, int32_t d_k, int32_t d_v, kda_dtype dtype,
                       hipStream_t stream);

/* Static string naming a status code. */
const char *kda_status_str(kda_status status);

/* Detail of the last error raised on the calling thread ("" if none). */
const char *kda_last_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
