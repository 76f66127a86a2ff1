/*
 * short_conv_oracle.c -- plain fp64 direct evaluation of the modality-aware short
 * convolution over packed samples.
 *
 * TEST INFRASTRUCTURE ONLY. This file is a correctness oracle that the HIP path is
 * checked against. Only the tests, the smoke check and the CPU baseline of the
 * benchmark may load it; the product path never does. It shares no code, header or
 * table with the HIP library.
 *
 * What it computes (Chimera, arXiv 2607.28611: paper Sec. 3.4 and the NoPE discussion
 * on position selection; explainer page "What RoPE was actually doing"): a depthwise
 * kernel per channel that mixes tokens at fixed index offsets; text tokens with a 1D
 * kernel along the token index, causal; visual tokens with a 3D kernel over the
 * (T, H, W) latent grid, causal in time. Visual tokens are stored in temporal-major
 * raster order, grid position (i, j, k) at index i*H*W + j*W + k after the sample's
 * text prefix (explainer page, "One stream, three mechanisms, no positions").
 *
 * Sample n owns tokens [cu[n], cu[n+1]): the first text_len[n] are text, the rest the
 * grid (grid[3n], grid[3n+1], grid[3n+2]) = (T, H, W). For channel c:
 *   text token t (0-based inside the text prefix):
 *     y[t][c] = sum_{i=0}^{kx-1} w_text[i][c] * x[t-i][c]          terms with t-i < 0 are 0
 *   visual token (i, j, k):
 *     y[i,j,k][c] = sum_{a<kt} sum_{b<kh} sum_{d<kw} w_vis[a][b][d][c] *
 *                   x[i-a, j+b-(kh-1)/2, k+d-(kw-1)/2][c]       terms outside the grid are 0
 * (kh, kw odd: centred in space; a >= 0 only: causal in time). Text and visual tokens
 * never read each other; no sample reads another. Weights are channel-last fp64 here
 * (the exact upcast of the stored fp32 weights). No bias, no activation: the pages
 * name neither. The kernel sizes are not on the pages and are parameters.
 */
#include <stdint.h>
#include <stdlib.h>

int kda_oracle_short_conv(const double *x, const double *w_text, const double *w_vis,
                          const int32_t *cu, const int32_t *text_len, const int32_t *grid,
                          int32_t n_seqs, int32_t C, int32_t kx, int32_t kt, int32_t kh, int32_t kw,
                          double *y)
{
    if (!cu || n_seqs < 0 || C <= 0 || kx < 1 || kt < 1 || kh < 1 || kw < 1 || kh % 2 == 0 || kw % 2 == 0)
        return -1;
    const int32_t ph = (kh - 1) / 2, pw = (kw - 1) / 2;
    for (int32_t n = 0; n < n_seqs; ++n) {
        const int64_t base = cu[n], len = (int64_t)cu[n + 1] - cu[n];
        const int64_t L = text_len[n];
        const int64_t T = grid[3 * n], H = grid[3 * n + 1], W = grid[3 * n + 2];
        if (L < 0 || T < 0 || H < 0 || W < 0 || L + T * H * W != len) return -1;
        /* text: causal 1D along the token index */
        for (int64_t t = 0; t < L; ++t)
            for (int32_t c = 0; c < C; ++c) {
                double acc = 0.0;
                for (int32_t i = 0; i < kx; ++i)
                    if (t - i >= 0) acc += w_text[(int64_t)i * C + c] * x[(base + t - i) * C + c];
                y[(base + t) * C + c] = acc;
            }
        /* visual: 3D, causal in time, centred in height and width */
        const int64_t v0 = base + L;
        for (int64_t i = 0; i < T; ++i)
            for (int64_t j = 0; j < H; ++j)
                for (int64_t k = 0; k < W; ++k)
                    for (int32_t c = 0; c < C; ++c) {
                        double acc = 0.0;
                        for (int32_t a = 0; a < kt; ++a)
                            for (int32_t b = 0; b < kh; ++b)
                                for (int32_t d = 0; d < kw; ++d) {
                                    const int64_t ii = i - a, jj = j + b - ph, kk = k + d - pw;
                                    if (ii < 0 || jj < 0 || jj >= H || kk < 0 || kk >= W) continue;
                                    acc += w_vis[(((int64_t)a * kh + b) * kw + d) * C + c] *
                                           x[(v0 + (ii * H + jj) * W + kk) * C + c];
                                }
                        y[(v0 + (i * H + j) * W + k) * C + c] = acc;
                    }
    }
    return 0;
}

/*
 * The reverse mode of the same convolution. For a loss whose gradient with respect to y
 * is dy, the gradients dx, dw_text and dw_vis. The convolution is linear in x and in the
 * weights: every term w * x[src] that makes up an output y[t] sends dy[t] * w back to
 * dx[src] and dy[t] * x[src] to the weight. This is that transpose, term by term, walked
 * in the forward's own order; dx, dw_text and dw_vis are overwritten.
 */
int kda_oracle_short_conv_backward(const double *x, const double *w_text, const double *w_vis,
                                   const int32_t *cu, const int32_t *text_len, const int32_t *grid,
                                   int32_t n_seqs, int32_t C, int32_t kx, int32_t kt, int32_t kh, int32_t kw,
                                   const double *dy, double *dx, double *dw_text, double *dw_vis)
{
    if (!cu || n_seqs < 0 || C <= 0 || kx < 1 || kt < 1 || kh < 1 || kw < 1 || kh % 2 == 0 || kw % 2 == 0)
        return -1;
    const int32_t ph = (kh - 1) / 2, pw = (kw - 1) / 2;
    const int64_t T_all = cu[n_seqs];
    for (int64_t e = 0; e < T_all * C; ++e) dx[e] = 0.0;
    for (int64_t e = 0; e < (int64_t)kx * C; ++e) dw_text[e] = 0.0;
    for (int64_t e = 0; e < (int64_t)kt * kh * kw * C; ++e) dw_vis[e] = 0.0;
    for (int32_t n = 0; n < n_seqs; ++n) {
        const int64_t base = cu[n], len = (int64_t)cu[n + 1] - cu[n];
        const int64_t L = text_len[n];
        const int64_t T = grid[3 * n], H = grid[3 * n + 1], W = grid[3 * n + 2];
        if (L < 0 || T < 0 || H < 0 || W < 0 || L + T * H * W != len) return -1;
        for (int64_t t = 0; t < L; ++t)
            for (int32_t c = 0; c < C; ++c) {
                const double g = dy[(base + t) * C + c];
                for (int32_t ti = 0; ti < kx; ++ti)
                    if (t - ti >= 0) {
                        dx[(base + t - ti) * C + c] += w_text[(int64_t)ti * C + c] * g;
                        dw_text[(int64_t)ti * C + c] += x[(base + t - ti) * C + c] * g;
                    }
            }
        const int64_t v0 = base + L;
        for (int64_t i = 0; i < T; ++i)
            for (int64_t j = 0; j < H; ++j)
                for (int64_t k = 0; k < W; ++k)
                    for (int32_t c = 0; c < C; ++c) {
                        const double g = dy[(v0 + (i * H + j) * W + k) * C + c];
                        for (int32_t ta = 0; ta < kt; ++ta)
                            for (int32_t tb = 0; tb < kh; ++tb)
                                for (int32_t td = 0; td < kw; ++td) {
                                    const int64_t si = i - ta, sj = j + tb - ph, sk = k + td - pw;
                                    if (si < 0 || sj < 0 || sj >= H || sk < 0 || sk >= W) continue;
                                    const int64_t src = (v0 + (si * H + sj) * W + sk) * C + c;
                                    const int64_t wi = (((int64_t)ta * kh + tb) * kw + td) * C + c;
                                    dx[src] += w_vis[wi] * g;
                                    dw_vis[wi] += x[src] * g;
                                }
                    }
    }
    return 0;
}

