// kda_conv.hip -- modality-aware depthwise short convolution over packed samples (gfx950).
//
// The operation (Chimera, arXiv 2607.28611: paper Sec. 3.4 and the NoPE discussion of
// position selection; explainer page "What RoPE was actually doing"): a depthwise kernel
// per channel mixing tokens at fixed index offsets; text tokens causally along the token
// index, visual tokens over the (T, H, W) latent grid, causally in time. The paper runs it
// as one fused pass over the packed token representation instead of gather, convolve,
// scatter. Sample n owns tokens [cu[n], cu[n+1]): text_len[n] text tokens, then a grid of
// (T, H, W) tokens in temporal-major raster order (i*H*W + j*W + k):
//   text:   y[t][c] = sum_{i<kx} w_text[i][c] x[t-i][c]                        (t-i >= 0)
//   visual: y[i,j,k][c] = sum_{a<kt, b<kh, d<kw} w_vis[a][b][d][c] x[i-a, j+b-(kh-1)/2, k+d-(kw-1)/2][c]
// with zeros outside the sample's text or grid.
//
// The pass is bound by HBM (read x once, write y once). One thread computes 8 channels
// of a token from 16-byte loads of its taps. A workgroup covers 128 tokens x 64 channels,
// and the tiles are numbered so that each XCD walks a contiguous token range of one
// channel block: the rows above and the frames before a tile (128 bytes per token per
// channel block) were read shortly before by the same XCD and are still in its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {
using namespace dev;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCT = 256;            // threads per workgroup
constexpr int kCB = 64;             // channels per tile
constexpr int kTPT = 4;             // tokens per thread
constexpr int kTok = kCT / (kCB / 8) * kTPT;   // tokens per tile: 128
constexpr int kMaxTaps = 8 + 4 * 5 * 5;

template <typename E> struct Vec8;
template <> struct Vec8<uint16_t> {
    __device__ static void load(const uint16_t* p, float (&f)[8]) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[2 * j] = __uint_as_float(u[j] << 16);
            f[2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
        }
    }
    __device__ static void store(uint16_t* p, const float (&f)[8]) {
        *reinterpret_cast<u32x4*>(p) = u32x4{pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])};
    }
};
template <> struct Vec8<float> {
    __device__ static void load(const float* p, float (&f)[8]) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[j] = a[j];
            f[4 + j] = b[j];
        }
    }
    __device__ static void store(float* p, const float (&f)[8]) {
        *reinterpret_cast<f32x4*>(p) = f32x4{f[0], f[1], f[2], f[3]};
        *reinterpret_cast<f32x4*>(p + 4) = f32x4{f[4], f[5], f[6], f[7]};
    }
};

template <typename E>
__global__ __launch_bounds__(kCT) void kda_short_conv_kernel(
    const E* __restrict__ x, const float* __restrict__ w_text, const float* __restrict__ w_vis,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ text_len, const int32_t* __restrict__ grid,
    E* __restrict__ y, int64_t T, int num_seqs, int C, int kx, int kt, int kh, int kw, int ntb, int ncb)
{
    __shared__ float wl[kMaxTaps * kCB];     // [tap][channel of the tile]: text taps, then visual
    const int tid = threadIdx.x;
    // tiles of one XCD are consecutive: logical tile = xcd * per + slot
    const int nt = ntb * ncb, per = (nt + 7) / 8;
    const int lt = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (lt >= nt) return;
    const int cb = lt / ntb, tb = lt % ntb;
    const int ntaps = kx + kt * kh * kw;
    for (int i = tid; i < ntaps * kCB; i += kCT) {
        const int tap = i / kCB, c = kCB * cb + i % kCB;
        float w = 0.f;
        if (c < C) w = tap < kx ? w_text[int64_t(tap) * C + c] : w_vis[int64_t(tap - kx) * C + c];
        wl[i] = w;
    }
    __syncthreads();

    const int vec = tid & 7, c0 = kCB * cb + 8 * vec;
    if (c0 >= C) return;
    const float* wv = wl + 8 * vec;
    const int ph = (kh - 1) / 2, pw = (kw - 1) / 2;
#pragma unroll 1
    for (int u = 0; u < kTPT; ++u) {
        const int64_t tok = int64_t(tb) * kTok + (tid >> 3) + 32 * u;
        if (tok >= T) break;
        // owning sample: cu[n] <= tok < cu[n + 1]
        int lo = 0, hi = num_seqs;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (cu[mid] <= tok) lo = mid; else hi = mid;
        }
        // bounds clamped to the tokens, so malformed offsets never address outside x
        const int64_t base = min<int64_t>(max<int64_t>(cu[lo], 0), T);
        const int64_t end = min<int64_t>(max<int64_t>(cu[lo + 1], base), T);
        const int64_t L = min<int64_t>(max(text_len[lo], 0), end - base), rel = tok - base;
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        if (rel < L) {
            for (int i = 0; i < kx && rel - i >= 0; ++i) {
                float f[8];
                Vec8<E>::load(x + (tok - i) * C + c0, f);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += wv[i * kCB + e] * f[e];
            }
        } else {
            const int64_t Hn = grid[3 * lo + 1], Wn = grid[3 * lo + 2];
            const int64_t nv = end - base - L, m = rel - L;          // grid tokens present, this one's index
            if (Hn <= 0 || Wn <= 0 || m >= nv) {                     // grid inconsistent with the sample
                Vec8<E>::store(y + tok * C + c0, acc);
                continue;
            }
            const int64_t i = m / (Hn * Wn), j = (m / Wn) % Hn, k = m % Wn;
            for (int a = 0; a < kt && i - a >= 0; ++a)
                for (int b = 0; b < kh; ++b) {
                    const int64_t jj = j + b - ph;
                    if (jj < 0 || jj >= Hn) continue;
                    for (int d = 0; d < kw; ++d) {
                        const int64_t kk = k + d - pw;
                        const int64_t mm = ((i - a) * Hn + jj) * Wn + kk;
                        if (kk < 0 || kk >= Wn || mm >= nv) continue;
                        float f[8];
                        Vec8<E>::load(x + (base + L + mm) * C + c0, f);
                        const float* w = wv + (kx + (a * kh + b) * kw + d) * kCB;
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[e] += w[e] * f[e];
                    }
                }
        }
        Vec8<E>::store(y + tok * C + c0, acc);
    }
}

}  // namespace

hipError_t launch_short_conv(const ConvArgs& a)
{
    if (a.total_tokens == 0 || a.num_seqs == 0) return hipSuccess;
    const int64_t ntb = (a.total_tokens + kTok - 1) / kTok;
    const int ncb = (a.channels + kCB - 1) / kCB;
    if (ntb * ncb > 0x7FFFFFFF - 8) return hipErrorInvalidValue;
    const int nt = int(ntb * ncb);
    const int blocks = ((nt + 7) / 8) * 8;
    if (a.dtype_bf16)
        hipLaunchKernelGGL(kda_short_conv_kernel<uint16_t>, dim3(blocks), dim3(kCT), 0, a.stream,
                           static_cast<const uint16_t*>(a.x), a.w_text, a.w_vis, a.cu_seqlens, a.text_len, a.grid,
                           static_cast<uint16_t*>(a.y), a.total_tokens, a.num_seqs, a.channels, a.k_text, a.k_t,
                           a.k_h, a.k_w, int(ntb), ncb);
    else
        hipLaunchKernelGGL(kda_short_conv_kernel<float>, dim3(blocks), dim3(kCT), 0, a.stream,
                           static_cast<const float*>(a.x), a.w_text, a.w_vis, a.cu_seqlens, a.text_len, a.grid,
                           static_cast<float*>(a.y), a.total_tokens, a.num_seqs, a.channels, a.k_text, a.k_t, a.k_h,
                           a.k_w, int(ntb), ncb);
    return hipGetLastError();
}

}  // namespace kda
