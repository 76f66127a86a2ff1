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
 *   scale is applied, and no normalisation unless kda_forward_ex asks for it.
 *
 * The library evaluates this recurrence in a chunkwise form on bf16/fp32 MFMA
 * with fp32 accumulation and an fp32 state; results agree with the token
 * recurrence up to floating-point rounding.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
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
 *   out             : [total_tokens][num_heads][d_v]   dtype (written; may not overlap an input)
 *   final_state     : [num_seqs][num_heads][d_k][d_v] fp32, rows = key channels, the state
 *                     after each sample's last token (zeros for an empty sample). May be NULL.
 *
 * Sizes: d_k, d_v in {64, 128}; num_heads >= 1; num_seqs >= 0; total_tokens >= 0 and
 * total_tokens * num_heads * max(d_k, d_v) < 2^31. Pointers must be 16-byte aligned.
 *
 * Numerics: inputs are used as stored; internally fp32 state and accumulation. For
 * bf16 inputs the chunk contractions run on bf16 MFMA; out is rounded to nearest-even.
 * Precondition: within any 64-token chunk (the longest chunk of any scan) the summed
 * log_alpha of each key channel is above -80; stronger decay overflows the factored
 * per-chunk decay and gives non-finite results. NaN/Inf inputs propagate only within
 * their own (sample, head).
 *
 * Execution: enqueued on `stream` (NULL = the null stream) and returns without
 * synchronising; buffers must stay valid until the stream reaches the work. The
 * library keeps no pointer after returning. Every entry point that enqueues work may be captured into a
 * HIP graph by stream capture on a non-null stream: workspaces are stream-ordered
 * allocations, other streams are forked and joined by events, and no call records a
 * memset. For bf16 data the default scan takes a
 * workspace of kda_workspace_bytes(...) bytes
 * from the device's default stream-ordered memory pool (hipMallocAsync on `stream`,
 * released with hipFreeAsync on `stream` after the kernels; the pool keeps the
 * memory for the next call, and kda_release gives it back to the driver). The environment
 * variable KDA_SCAN_VARIANT selects the bf16 scan: "fused" (the default for d_k = d_v = 128),
 * one kernel that forms every chunk's operands on the CU and whose workspace holds the
 * counters its persistent workgroups take (segment, head) units from (256 bytes) and, when a
 * few long samples are cut into segments, two 64 KB summaries per (segment, head);
 * "wy" (the default for other sizes), a prep kernel whose per-chunk records the workspace
 * holds and a chain kernel; "sequential", a single kernel that needs no workspace. fp32 data
 * always uses the sequential scan. Results are bitwise deterministic for identical inputs on
 * the same device and variant.
 * cu_seqlens is read on the device; its content is checked on the host only when the
 * environment variable KDA_VALIDATE=1 (one synchronous device-to-host copy).
 *
 * Errors: returns KDA_OK or an error code; argument checks run before any launch and
 * nothing is enqueued on error. kda_last_error() gives a message for the calling thread.
 * With the environment variable KDA_DEBUG_SYNC=1, every call that enqueues work (the
 * forward, backward and short-convolution entry points) waits for its stream before it
 * returns, outside stream capture, and reports a failure of its kernels as KDA_E_HIP.
 */
kda_status kda_forward(const void *q, const void *k, const void *v, const void *log_alpha,
                       const void *beta, const int32_t *cu_seqlens, void *out,
                       float *final_state, int64_t total_tokens, int32_t num_seqs,
                       int32_t num_heads, int32_t d_k, int32_t d_v, kda_dtype dtype,
                       hipStream_t stream);

/*
 * kda_forward_from_state -- kda_forward with a given state at the start of each sample.
 *
 * The recurrent state is the only thing a sample carries forward (fixed size per
 * head, independent of the number of tokens: explainer page "What O(N) buys in
 * memory and latency"; paper Sec. 5 hybrid-attention efficiency study, Fig. 18,
 * "roll-out cache" setting). This entry point continues a scan from a retained
 * state: S_0 = initial_state[n][h] instead of 0, every other step as kda_forward.
 * Running tokens [0, a) and then [a, L) of one sample, the second call starting from
 * the first call's final_state, gives the result of one call over [0, L) up to
 * floating-point rounding.
 *
 *   initial_state : [num_seqs][num_heads][d_k][d_v] fp32 DEVICE pointer, rows = key
 *                   channels, 16-byte aligned; read only; may not overlap final_state.
 *                   NULL means zero states (then identical to kda_forward).
 * All other arguments, errors and execution as kda_forward; supported for fp32 and
 * bf16 data on every scan variant.
 */
kda_status kda_forward_from_state(const void *q, const void *k, const void *v,
                                  const void *log_alpha, const void *beta,
                                  const int32_t *cu_seqlens, const float *initial_state,
                                  void *out, float *final_state, int64_t total_tokens,
                                  int32_t num_seqs, int32_t num_heads, int32_t d_k, int32_t d_v,
                                  kda_dtype dtype, hipStream_t stream);

/* Option bits of kda_forward_ex. */
#define KDA_OPT_QK_L2NORM 1u   /* normalise q_t and k_t to unit length on load */

/*
 * kda_forward_ex -- kda_forward with an optional initial state and option bits.
 *
 * KDA_OPT_QK_L2NORM: before the recurrence, q_t and k_t of every (token, head) are
 * divided by their Euclidean length (over the d_k channels; a zero vector stays
 * zero), in fp32 from the stored values, and the scan runs on the unit vectors. The
 * paper's training setup names chunked KDA kernels with the normalisation fused in
 * (paper, training setup paragraph on the custom kernels over the packed tokens); it
 * does not print the form, and this one, x / |x| per token and head, is the reading
 * taken. It spares the caller a separate pass over q and k in HBM. The stored q and
 * k are not modified.
 *
 *   initial_state : as kda_forward_from_state (NULL = zero states).
 *   options       : bitwise OR of KDA_OPT_* values; unknown bits give KDA_E_UNSUPPORTED.
 * All other arguments, errors and execution as kda_forward. KDA_OPT_QK_L2NORM is
 * supported for fp32 and bf16 data on every scan; initial_state as for
 * kda_forward_from_state.
 */
kda_status kda_forward_ex(const void *q, const void *k, const void *v, const void *log_alpha,
                          const void *beta, const int32_t *cu_seqlens, const float *initial_state,
                          void *out, float *final_state, int64_t total_tokens, int32_t num_seqs,
                          int32_t num_heads, int32_t d_k, int32_t d_v, kda_dtype dtype,
                          uint32_t options, hipStream_t stream);

/*
 * kda_forward_noalloc -- kda_forward_ex that allocates no memory, for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, hosts that forbid it.
 *
 * Arguments, layouts, ownership and results are those of kda_forward_ex. bf16 data with
 * d_k = d_v = 128 runs the fused scan ("fused" of KDA_SCAN_VARIANT) with its segment
 * summaries in a fixed 32 MiB device buffer that the library holds on every device it runs
 * on until the process ends; the segment plan is fitted to that buffer (fewer, longer
 * segments, or whole samples), so every size the arguments admit fits. Other sizes and
 * fp32 data run the sequential scan, which needs no buffer. No hipMalloc, hipFree or other
 * allocating call is made; KDA_SCAN_VARIANT, KDA_VALIDATE and the timing diagnostics are
 * not consulted. All calls on one device share the buffer: calls that overlap in time on
 * one device (different streams or threads without ordering between them) race and give
 * wrong results; order them on one stream. Nothing in the buffer needs to start at zero.
 * Returns KDA_E_UNSUPPORTED if a plan should ever need more than the buffer.
 */
kda_status kda_forward_noalloc(const void *q, const void *k, const void *v, const void *log_alpha,
                               const void *beta, const int32_t *cu_seqlens,
                               const float *initial_state, void *out, float *final_state,
                               int64_t total_tokens, int32_t num_seqs, int32_t num_heads,
                               int32_t d_k, int32_t d_v, kda_dtype dtype, uint32_t options,
                               hipStream_t stream);

/*
 * kda_backward -- gradients of the KDA scan.
 *
 * The paper trains its model through these kernels (paper, training setup paragraph
 * on the custom kernels over the packed tokens). For a scalar loss L whose gradient
 * with respect to out is d_out and with respect to final_state is d_final_state, this
 * returns dL/dq, dL/dk, dL/dv, dL/dlog_alpha, dL/dbeta and dL/dinitial_state of the
 * scan that kda_forward_ex computes from the same inputs, initial_state and options
 * (the reverse-mode derivative of the recurrence above; with KDA_OPT_QK_L2NORM the
 * gradients are those of the raw q and k, through the normalisation).
 *
 *   q, k, v, log_alpha, beta, cu_seqlens, initial_state, options : as kda_forward_ex
 *                     (initial_state may be NULL = zero states; supported for both dtypes)
 *   d_out           : [total_tokens][num_heads][d_v] dtype, read only
 *   d_final_state   : [num_seqs][num_heads][d_k][d_v] fp32 or NULL (= zero)
 *   dq, dk, dlog_alpha : [total_tokens][num_heads][d_k] dtype, written
 *   dv              : [total_tokens][num_heads][d_v] dtype, written
 *   dbeta           : [total_tokens][num_heads] dtype, written
 *   d_initial_state : [num_seqs][num_heads][d_k][d_v] fp32 or NULL (not written); the
 *                     gradient with respect to the initial states (equal to d_final_state
 *                     for an empty sample)
 * No output may overlap an input or another output (byte ranges; KDA_E_SHAPE).
 * Arithmetic is fp32 throughout (fp32 MFMA), over 32-token chunks; results in the data
 * dtype, rounded to nearest-even. Same size limits as kda_forward. For packs of few long
 * samples the chains run as two passes over segments of the samples (same results up to
 * rounding). Execution: enqueued on `stream`. The state chain runs on a second stream
 * that the library keeps per host thread and device (default priority): it waits for
 * `stream` after the prep, and `stream` waits for it before the gradient kernel, so the
 * call is ordered on `stream` as a whole. Takes a workspace of
 * kda_backward_workspace_bytes(...) bytes (chunk operands and the per-chunk state and
 * state gradient, about 6 KB per token and head at d = 128, plus per-segment summaries
 * when the chains are split) from the device's default stream-ordered pool, returned on
 * `stream` after the kernels. Results are bitwise reproducible for identical inputs, sizes
 * and device (partial sums are added in a fixed order, no atomics). Errors as kda_forward.
 */
kda_status kda_backward(const void *q, const void *k, const void *v, const void *log_alpha,
                        const void *beta, const int32_t *cu_seqlens, const float *initial_state,
                        const void *d_out, const float *d_final_state, void *dq, void *dk, void *dv,
                        void *dlog_alpha, void *dbeta, float *d_initial_state, int64_t total_tokens,
                        int32_t num_seqs, int32_t num_heads, int32_t d_k, int32_t d_v, kda_dtype dtype,
                        uint32_t options, hipStream_t stream);

/* Bytes of device workspace kda_backward takes for these sizes (0 for no samples or
 * unsupported sizes). Pure function of the sizes. */
size_t kda_backward_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_heads,
                                    int32_t d_k, int32_t d_v);

/*
 * kda_short_conv -- the modality-aware depthwise short convolution over packed samples.
 *
 * The layer's short convolution that supplies local structure next to the scan (paper
 * Sec. 3.4 and the NoPE discussion of position selection; explainer page "What RoPE was
 * actually doing"): a depthwise kernel per channel that mixes tokens at fixed index
 * offsets, text tokens along the token index (causal), visual tokens over their (T, H, W)
 * latent grid (causal in time), in one pass over the packed tokens. Sample n owns tokens
 * [cu_seqlens[n], cu_seqlens[n+1]): its first text_len[n] tokens are text, the rest its
 * grid (grid[3n], grid[3n+1], grid[3n+2]) = (T, H, W) in temporal-major raster order,
 * position (i, j, k) at index i*H*W + j*W + k after the text. For channel c:
 *   text    y[t][c] = sum_{i < k_text} w_text[i][c] x[t - i][c]                  (t - i >= 0)
 *   visual  y[i,j,k][c] = sum_{a < k_t, b < k_h, d < k_w} w_vis[a][b][d][c]
 *                         x[i - a, j + b - (k_h-1)/2, k + d - (k_w-1)/2][c]
 * with zeros outside the sample's text or grid: text and visual tokens never read each
 * other, and no sample reads another. The pages fix neither the kernel sizes nor a bias or
 * activation; there is none, and the sizes are arguments.
 *
 *   x, y        : [total_tokens][channels] dtype, DEVICE, 16-byte aligned; y may not overlap an input
 *   w_text      : [k_text][channels] fp32;  w_vis : [k_t][k_h][k_w][channels] fp32 (DEVICE)
 *   cu_seqlens  : [num_seqs + 1] int32; text_len : [num_seqs] int32; grid : [num_seqs][3] int32
 *                 (DEVICE; text_len and grid may be NULL when num_seqs is 0);
 *                 text_len[n] + T*H*W must equal the sample's length (checked on the
 *                 host only with KDA_VALIDATE=1). Otherwise the kernel still reads and writes
 *                 only inside the sample: grid positions past its last token read as zero,
 *                 and tokens past T*H*W (or after the text when T, H or W is 0) get zeros
 *   channels    : a multiple of 8; k_text 1..8, k_t 1..4, k_h and k_w odd in 1..5
 * Arithmetic is fp32; y is rounded to nearest-even for bf16. A workspace of the tile table
 * ((num_seqs + 1) int32, rounded up to 256 bytes) and eight tile counters (1 KiB) comes from
 * the stream-ordered pool as for kda_forward. Execution and errors as kda_forward; the
 * timing hook names the kernels "conv_plan" and "conv".
 */
kda_status kda_short_conv(const void *x, const float *w_text, const float *w_vis,
                          const int32_t *cu_seqlens, const int32_t *text_len, const int32_t *grid,
                          void *y, int64_t total_tokens, int32_t num_seqs, int32_t channels,
                          int32_t k_text, int32_t k_t, int32_t k_h, int32_t k_w, kda_dtype dtype,
                          hipStream_t stream);

/*
 * kda_short_conv_backward -- the reverse mode of kda_short_conv: for a loss whose gradient
 * with respect to y is dy, the gradients dx, dw_text and dw_vis.
 *
 * The convolution above is linear in x and, separately, in the weights, so each gradient is
 * the transpose of one of those linear maps applied to dy (same passages as kda_short_conv):
 *   dx[t][c]           = sum_{i < k_text, t + i < text_len} w_text[i][c] dy[t + i][c]
 *   dx[i,j,k][c]       = sum_{a,b,d} w_vis[a][b][d][c] dy[i + a, j - b + (k_h-1)/2, k - d + (k_w-1)/2][c]
 *   dw_text[i][c]      = sum over text tokens t with t - i >= 0 of x[t - i][c] dy[t][c]
 *   dw_vis[a][b][d][c] = sum over grid positions (i, j, k) of x[i - a, j + b - (k_h-1)/2, k + d - (k_w-1)/2][c] dy[i,j,k][c]
 * with terms outside the sample's text or grid zero; the weight sums run over every sample.
 *
 *   x, dy, dx   : [total_tokens][channels] dtype, DEVICE, 16-byte aligned
 *   dw_text     : [k_text][channels] fp32; dw_vis : [k_t][k_h][k_w][channels] fp32 (DEVICE),
 *                 overwritten (not accumulated into)
 *   the rest    : as kda_short_conv. No output may overlap an input or another output.
 * When a sample's grid does not match its length the calls read and write only inside the
 * sample, as kda_short_conv: grid positions past its last token hold zero in x and in dy, and
 * dx is zero for tokens past T*H*W. With no samples or no tokens dw_text and dw_vis are zero
 * and dx is not touched.
 * Arithmetic is fp32; dx is rounded to nearest-even for bf16. dx comes from the forward's
 * kernel with the taps mirrored and the time and text directions reversed; the weight sums
 * are formed per (channel block, part of the tile list: every parts-th tile) and the parts
 * then added in a fixed order, so the result is the same bit for bit from run to run. A
 * workspace of the forward's (table and counters) plus parts * (k_text + k_t*k_h*k_w) *
 * channels fp32 partial sums (parts is about 2048 / (ceil(channels / 64) * (k_t + 1)), at
 * least 1) comes from the stream-ordered pool as for kda_forward. Execution and errors as kda_forward; the timing
 * hook names the kernels "conv_bwd_plan", "conv_dx", "conv_dw" and "conv_dw_reduce".
 */
kda_status kda_short_conv_backward(const void *x, const float *w_text, const float *w_vis,
                                   const int32_t *cu_seqlens, const int32_t *text_len,
                                   const int32_t *grid, const void *dy, void *dx, float *dw_text,
                                   float *dw_vis, int64_t total_tokens, int32_t num_seqs,
                                   int32_t channels, int32_t k_text, int32_t k_t, int32_t k_h,
                                   int32_t k_w, kda_dtype dtype, hipStream_t stream);

/*
 * kda_workspace_bytes -- bytes of device workspace the bf16 scan selected by
 * KDA_SCAN_VARIANT takes for these sizes (0 when it takes none: fp32 data, no samples,
 * unsupported sizes, the sequential scan). Fused scan: 256 bytes of unit counters, plus per
 * (segment, head) state and transition when samples are cut into segments. WY scan: per (64-token
 * chunk, head) record of the chunk's decayed operands and WY factors (about 1.2 KB per token
 * and head), plus a chunk table.
 * Pure function of the sizes and the environment; no device access.
 */
size_t kda_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_heads,
                           int32_t d_k, int32_t d_v, kda_dtype dtype);

/*
 * Diagnostics: per-kernel timing with HIP events. While enabled (on != 0), each
 * kda_forward* call records a pair of events on its stream around every kernel it
 * launches, named "fused", "fused_sum" and "fused_combine" (fused bf16 scan: the output
 * pass, and for samples cut into segments the summary pass and the combine over segments),
 * "prep", "segments" and "chain" (WY bf16 scan; "segments" is the first pass of its
 * sequence split), "plan" (a table over the samples for packs of more than 64 samples; for
 * the fused scan it also clears the unit counters, on every call) or "scan" (single-kernel scans); kda_backward records "bwd_plan", "bwd_prep",
 * "bwd_state", "bwd_dstate" and "bwd_grad", plus "bwd_state_seg" and "bwd_dstate_seg" (the
 * first passes of the chains' sequence split, for packs of few long samples). kda_timing_read waits for the recorded events of `kernel`,
 * returns their count and summed duration in milliseconds, and drops them.
 * Process-wide state guarded by a mutex; returns KDA_E_NULL on NULL arguments and
 * KDA_E_HIP if an event cannot be read (all records are then dropped).
 */
kda_status kda_timing_enable(int32_t on);
kda_status kda_timing_read(const char *kernel, int32_t *launches, double *total_ms);

/*
 * kda_release -- give the workspace memory that earlier calls freed back to the driver.
 *
 * Every entry point takes its workspace from the default stream-ordered pool of the
 * device (hipMallocAsync on the caller's stream) and returns it there in stream order
 * (hipFreeAsync); the library raises that pool's release threshold so the memory is
 * kept for the next call. This call trims the default pool of every device the library
 * has used down to the memory still held (hipMemPoolTrimTo, nothing kept): memory that
 * pending work still uses stays allocated. It enqueues nothing and may be called from
 * any host thread. Returns KDA_OK, or KDA_E_HIP with the HIP message in kda_last_error().
 */
kda_status kda_release(void);

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
