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
