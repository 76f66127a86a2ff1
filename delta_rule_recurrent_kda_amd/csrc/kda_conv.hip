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
// Every input feeds kt*kh*kw outputs, so the pass does 27 fp32 FMAs per output element for
// the 3x3x3 kernel; with packed fp32 arithmetic off, that vector work and the bf16 widening
// of the inputs, not HBM, bound it. The design therefore spends VALU on little else:
//   - Work is cut into tiles over 64 channels: a text tile is 128 text tokens of one sample;
//     a visual tile is 32 column strips, a strip being 4 adjacent columns of one row of one
//     frame (strips run frame-, row-, column-major through the sample's grid). A thread owns
//     one strip and 8 channels, so each loaded input column feeds the kw taps of up to 4
//     outputs and is widened from bf16 once.
//   - Inputs come straight from global memory: the kt*kh rows a strip reads are shared with
//     the strips of neighbouring rows and frames, which run at the same time on the same XCD
//     and find them in its L2. Each XCD owns a contiguous part of the tile list and its
//     workgroups take those tiles one at a time from the XCD's counter, so the tiles in
//     flight are always the latest ones started, a window that slides through the frames
//     (with tiles dealt out in turn the workgroups drift apart over a long sample and the
//     window spreads). A tile reads its time taps in the order of that walk: the frames the
//     tiles before it read last first, its newest frame last. Outputs are streaming stores.
//     Reads come to about 1.2-1.3x the input on the clip layouts (counters); reading the own
//     frame first, with tiles dealt out in turn, made them 1.9x.
//   - For whole-frame samples under 1 GiB the loads are buffer loads over the sample's grid
//     tokens: a position outside the grid gets an offset past the buffer's end and reads as
//     zero, so no lane spends arithmetic on padding.
//   - A plan kernel counts the tiles per sample and clears the counters; a fixed grid of
//     workgroups walks the tile list channel-block-major, with the weights of the current
//     channel block in LDS.
// The reverse mode (the gradients for a given dy) reuses the tiles: dx is the same kernel
// run on dy with the taps mirrored and time and text walked forward (REV); the weight
// gradients are sums over all tokens, formed per (channel block, part of the tile list,
// time offset) in fp32 and added in a fixed order by a reduce kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {
using namespace dev;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCT = 256;            // threads per workgroup
constexpr int kCB = 64;             // channels per tile
constexpr int kTextTok = 128;       // tokens per text tile
constexpr int kSW = 4;              // columns per thread strip
constexpr int kStrips = kCT / 8;    // column strips per visual tile
constexpr int kWgPerCu = 4;         // resident workgroups per CU of the persistent grid
constexpr int kQueueBytes = 8 * 128;        // a tile counter per XCD, each on its own 128-byte line
constexpr uint32_t kBufLimit = 1u << 30;    // bytes a buffer-load tile may span; also the "outside" offset
constexpr int kBufFlags = 0x00020000;       // raw buffer resource: 32-bit data format, no swizzle

template <typename E> struct Vec8;
template <> struct Vec8<uint16_t> {
    static constexpr int kBytes = 16;
    __device__ static void load(const uint16_t* p, float (&f)[8]) {
        const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[2 * j] = __uint_as_float(u[j] << 16);
            f[2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
        }
    }
    // outputs are written once and not read again here: streaming stores, so that they do not
    // push the inputs the neighbouring tiles still read out of the L2
    __device__ static void store(uint16_t* p, const float (&f)[8]) {
        __builtin_nontemporal_store(u32x4{pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7])},
                                    reinterpret_cast<u32x4*>(p));
    }
    // 8 channels as loaded (two bf16 per dword), widened one element at a time
    struct Raw { u32x4 u; };
    __device__ static Raw load_raw(const uint16_t* p, bool ok) {
        return Raw{ok ? *reinterpret_cast<const u32x4*>(p) : u32x4{0u, 0u, 0u, 0u}};
    }
    __device__ static float at(const Raw& r, int e) {
        return __uint_as_float((e & 1) ? (r.u[e >> 1] & 0xFFFF0000u) : (r.u[e >> 1] << 16));
    }
    // bytes at `off` of the buffer; zeros when off is past its end
    __device__ static Raw load_buf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return Raw{__builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0)};
    }
};
template <> struct Vec8<float> {
    static constexpr int kBytes = 32;
    __device__ static void load(const float* p, float (&f)[8]) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[j] = a[j];
            f[4 + j] = b[j];
        }
    }
    __device__ static void store(float* p, const float (&f)[8]) {
        __builtin_nontemporal_store(f32x4{f[0], f[1], f[2], f[3]}, reinterpret_cast<f32x4*>(p));
        __builtin_nontemporal_store(f32x4{f[4], f[5], f[6], f[7]}, reinterpret_cast<f32x4*>(p + 4));
    }
    struct Raw { f32x4 a, b; };
    __device__ static Raw load_raw(const float* p, bool ok) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        return Raw{ok ? *reinterpret_cast<const f32x4*>(p) : z, ok ? *reinterpret_cast<const f32x4*>(p + 4) : z};
    }
    __device__ static float at(const Raw& r, int e) { return e < 4 ? r.a[e] : r.b[e - 4]; }
    __device__ static Raw load_buf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0);
        return Raw{f32x4{__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[2]), __uint_as_float(a[3])},
                   f32x4{__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[2]), __uint_as_float(b[3])}};
    }
};

// Extent of sample n, with every value clamped so that the kernel reads and writes only
// inside the sample whatever the tables hold. Element offsets fit in 32 bits (the caller
// checks tokens x channels < 2^31). The grid is cut to the frames and rows that hold tokens:
// positions past the sample's last token read as zero either way, so this changes no output.
struct SampleGeom {
    int32_t base, L, nv;            // first token, text tokens, grid tokens present
    int32_t Tn, Hn, Wn;             // frames holding a token, rows, columns (0 frames: no grid)
    int32_t past;                   // first grid token past T*H*W (== nv when the grid fits)
};
__device__ __forceinline__ SampleGeom sample_geom(const int32_t* cu, const int32_t* text_len, const int32_t* grid,
                                                  int n, int64_t T) {
    SampleGeom g;
    const int64_t base = min<int64_t>(max<int64_t>(cu[n], 0), T);
    const int64_t end = min<int64_t>(max<int64_t>(cu[n + 1], base), T);
    const int64_t L = min<int64_t>(max(text_len[n], 0), end - base), nv = end - base - L;
    int64_t Tn = max(grid[3 * n], 0), Hn = max(grid[3 * n + 1], 0), Wn = max(grid[3 * n + 2], 0);
    int64_t past = 0;                           // no grid: every visual token past it
    if (Tn == 0 || Hn == 0 || Wn == 0 || nv == 0) {
        Tn = 0;
    } else {
        const int64_t hw = Hn * Wn;             // < 2^62
        past = Tn >= (nv + hw - 1) / hw ? nv : Tn * hw;
        // rows and frames past the last token hold none; the raster index of every
        // position that holds a token is unchanged by these cuts
        Wn = min(Wn, nv);
        Hn = min(Hn, (nv + Wn - 1) / Wn);
        Tn = min(Tn, (nv + Hn * Wn - 1) / (Hn * Wn));
    }
    g.base = int32_t(base); g.L = int32_t(L); g.nv = int32_t(nv);
    g.Tn = int32_t(Tn); g.Hn = int32_t(Hn); g.Wn = int32_t(Wn); g.past = int32_t(past);
    return g;
}

// Tiles of sample n per channel block: text tiles of 128 tokens, visual tiles of 32 column
// strips (a strip is 4 adjacent columns of one row of one frame; strips run frame, row,
// column-major), then tiles of 128 tokens past the grid, which get zeros.
struct SampleTiles {
    int32_t ntext, nvis, nzero, nsw;  // nsw: strips per row
};
__device__ __forceinline__ SampleTiles sample_tiles(const SampleGeom& g) {
    SampleTiles t;
    t.ntext = (g.L + kTextTok - 1) / kTextTok;
    t.nsw = (g.Wn + kSW - 1) / kSW;
    t.nvis = g.Tn > 0 ? int32_t((int64_t(g.Tn) * g.Hn * t.nsw + kStrips - 1) / kStrips) : 0;
    t.nzero = (g.nv - g.past + kTextTok - 1) / kTextTok;
    return t;
}

// tile_off[n] = tiles of samples 0..n-1 (per channel block), and the per-XCD tile counters
// cleared (queue may be null); one workgroup
__global__ __launch_bounds__(1024) void kda_conv_plan_kernel(const int32_t* __restrict__ cu,
                                                             const int32_t* __restrict__ text_len,
                                                             const int32_t* __restrict__ grid,
                                                             int32_t* __restrict__ tile_off, int* __restrict__ queue,
                                                             int num_seqs, int64_t T)
{
    __shared__ int32_t part[1024];
    const int tid = threadIdx.x;
    if (queue && tid < 8) queue[32 * tid] = 0;
    int32_t carry = 0;
    for (int b0 = 0; b0 < num_seqs; b0 += 1024) {
        const int n = b0 + tid;
        int32_t cnt = 0;
        if (n < num_seqs) {
            const SampleTiles t = sample_tiles(sample_geom(cu, text_len, grid, n, T));
            cnt = t.ntext + t.nvis + t.nzero;
        }
        part[tid] = cnt;
        __syncthreads();
        for (int d = 1; d < 1024; d <<= 1) {
            const int32_t add = tid >= d ? part[tid - d] : 0;
            __syncthreads();
            part[tid] += add;
            __syncthreads();
        }
        if (n < num_seqs) tile_off[n + 1] = carry + part[tid];
        carry += part[1023];
        __syncthreads();
    }
    if (tid == 0) tile_off[0] = 0;
}

// REV = false: y = conv(x). REV = true: the input gradient, dx = conv^T(dy), with dy passed as
// x and dx as y. The transpose of a causal-in-time, centred-in-space depthwise kernel is the
// same kind of kernel anti-causal in time with the taps mirrored in space:
//   dx[i,j,k] = sum_{a,b,d} w_vis[a][kh-1-b][kw-1-d] dy[i+a, j+b-(kh-1)/2, k+d-(kw-1)/2]
//   dx[t]     = sum_i w_text[i] dy[t+i]                                     (t+i < text_len)
// so REV mirrors the weights as it stages them and walks frames and text tokens forward.
// dy positions past the sample's grid tokens read as zero, like x positions in the forward.
template <typename E, int KW, bool REV>
__global__ __launch_bounds__(kCT) __attribute__((amdgpu_waves_per_eu(kWgPerCu))) void kda_short_conv_kernel(
    const E* __restrict__ x, const float* __restrict__ w_text, const float* __restrict__ w_vis,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ text_len, const int32_t* __restrict__ grid,
    const int32_t* __restrict__ tile_off, int* __restrict__ queue, E* __restrict__ y, int64_t T, int num_seqs, int C,
    int kx, int kt, int kh, int ncb)
{
    constexpr int kw = KW;
    extern __shared__ __align__(16) float wl[];                          // [tap][64]: text taps, then visual
    const int ntaps = kx + kt * kh * kw;
    const int tid = threadIdx.x, vec = tid & 7;
    const int ph = (kh - 1) / 2, pw = (kw - 1) / 2;

    const int per_cb = tile_off[num_seqs];
    const int64_t total = int64_t(per_cb) * ncb;
    // this XCD's contiguous range of the tile list (channel-block-major, so the tiles that
    // share inputs sit together), taken one tile at a time from the XCD's counter: the tiles
    // in flight are always the latest ones started, a window that slides through the frames
    // and finds the rows it shares with the tiles before it still in the XCD's L2
    const int xcd = blockIdx.x & 7;
    const int64_t per = (total + 7) / 8;
    const int64_t t_begin = xcd * per, t_end = min<int64_t>(total, (xcd + 1) * per);
    int* const ctr = queue + 32 * xcd;
    __shared__ int next_tile;
    int cb_loaded = -1;
    auto run_tile = [&](const int64_t tile) __attribute__((always_inline)) {
        const int cb = int(tile / per_cb), tp = int(tile % per_cb);
        if (cb != cb_loaded) {                      // weights of this channel block
            __syncthreads();
            for (int i = tid; i < ntaps * kCB; i += kCT) {
                const int tap = i / kCB, c = kCB * cb + i % kCB;
                float w = 0.f;
                if (c < C) {
                    int src = tap - kx;
                    if (REV && src >= 0) {          // mirror (b, d) within the time tap
                        const int hw = kh * kw, a = src / hw, b = (src - a * hw) / kw, d = src - a * hw - b * kw;
                        src = (a * kh + (kh - 1 - b)) * kw + (kw - 1 - d);
                    }
                    w = tap < kx ? w_text[tap * C + c] : w_vis[src * C + c];
                }
                wl[i] = w;
            }
            __syncthreads();
            cb_loaded = cb;
        }
        int n = 0, hi = num_seqs;                   // tile_off[n] <= tp < tile_off[n + 1]
        while (hi - n > 1) {
            const int mid = (n + hi) >> 1;
            if (tile_off[mid] <= tp) n = mid; else hi = mid;
        }
        const SampleGeom g = sample_geom(cu, text_len, grid, n, T);
        const SampleTiles st = sample_tiles(g);
        const int local = tp - tile_off[n];
        const int c0 = kCB * cb + 8 * vec;
        if (c0 >= C) return;
        const float* wv = wl + 8 * vec;

        if (local < st.ntext) {
            // ---- text tile: 128 tokens, a thread per token and 8 channels ----
            for (int r = tid >> 3; r < kTextTok; r += kCT / 8) {
                const int rel = local * kTextTok + r;
                if (rel >= g.L) break;
                const int tok = g.base + rel;
                float acc[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = 0.f;
                for (int i = 0; i < kx && (REV ? rel + i < g.L : rel - i >= 0); ++i) {
                    float f[8];
                    Vec8<E>::load(x + (REV ? tok + i : tok - i) * C + c0, f);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] += wv[i * kCB + e] * f[e];
                }
                Vec8<E>::store(y + tok * C + c0, acc);
            }
            return;
        }
        if (local >= st.ntext + st.nvis) {
            // ---- tokens past the grid: zeros ----
            const float zero[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            for (int r = tid >> 3; r < kTextTok; r += kCT / 8) {
                const int m = g.past + (local - st.ntext - st.nvis) * kTextTok + r;
                if (m < g.nv) Vec8<E>::store(y + (g.base + g.L + m) * C + c0, zero);
            }
            return;
        }

        // ---- visual tile: 32 strips; this thread's strip is 4 columns x 8 channels ----
        const int sidx = (local - st.ntext) * kStrips + (tid >> 3);
        const int per_frame = g.Hn * st.nsw;
        const int f = sidx / per_frame;
        if (f >= g.Tn) return;
        const int j = (sidx - f * per_frame) / st.nsw;
        const int kq = (sidx - f * per_frame - j * st.nsw) * kSW;
        const E* xs = x + (g.base + g.L) * C + c0;  // this sample's grid tokens, this thread's channels
        float acc[kSW][8];
#pragma unroll
        for (int q = 0; q < kSW; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[q][e] = 0.f;
        // the time taps whose frame exists, read in the order of the walk through the frames:
        // first the frames the tiles started before this one read last, the newest frame last
        const int na = REV ? min(kt, g.Tn - f) : min(kt, f + 1);
        const bool fast = g.past == g.nv && int64_t(g.Tn) * g.Hn * g.Wn == g.nv &&
                          int64_t(g.nv) * C * int64_t(sizeof(E)) <= kBufLimit;
        if (fast) {
            // Whole frames, sample under 1 GiB: buffer loads over the sample's grid tokens, so a
            // position outside the grid is an offset of at least kBufLimit and reads as zero.
            // Each position is widened once and feeds the KW taps of the strip that use it.
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<E*>(x + (g.base + g.L) * C), 0, int(int64_t(g.nv) * C * sizeof(E)), kBufFlags);
            const uint32_t rowb = uint32_t(g.Wn) * uint32_t(C) * sizeof(E);
            uint32_t colv[kSW + KW - 1];
#pragma unroll
            for (int p = 0; p < kSW + KW - 1; ++p) {
                const int kk = kq + p - pw;
                colv[p] = kk >= 0 && kk < g.Wn ? uint32_t(kk * C + c0) * sizeof(E) : kBufLimit;
            }
            for (int ai = 0; ai < na; ++ai)
                for (int b = 0, a = REV ? ai : na - 1 - ai; b < kh; ++b) {
                    const int jj = j + b - ph, fa = REV ? f + a : f - a;
                    const uint32_t roff = jj >= 0 && jj < g.Hn ? uint32_t(fa * g.Hn + jj) * rowb : kBufLimit;
                    typename Vec8<E>::Raw in[kSW + KW - 1];
#pragma unroll
                    for (int p = 0; p < kSW + KW - 1; ++p) in[p] = Vec8<E>::load_buf(rs, roff + colv[p]);
                    const float* wr = wv + (kx + (a * kh + b) * KW) * kCB;
                    float w[KW][8];
#pragma unroll
                    for (int d = 0; d < KW; ++d)
#pragma unroll
                        for (int e = 0; e < 8; ++e) w[d][e] = wr[d * kCB + e];
#pragma unroll
                    for (int p = 0; p < kSW + KW - 1; ++p) {
                        float xf[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) xf[e] = Vec8<E>::at(in[p], e);
#pragma unroll
                        for (int d = 0; d < KW; ++d) {
                            const int q = p - d;
                            if (q < 0 || q >= kSW) continue;
#pragma unroll
                            for (int e = 0; e < 8; ++e) acc[q][e] += w[d][e] * xf[e];
                        }
                    }
                }
        } else
        for (int ai = 0; ai < na; ++ai)
            for (int b = 0, a = REV ? ai : na - 1 - ai; b < kh; ++b) {
                const int jj = j + b - ph;
                if (jj < 0 || jj >= g.Hn) continue;
                const int row = ((REV ? f + a : f - a) * g.Hn + jj) * g.Wn;   // grid index of column 0
                // columns kq - pw .. kq + kSW - 1 + pw, zero outside the grid or the sample
                typename Vec8<E>::Raw in[kSW + KW - 1];
#pragma unroll
                for (int q = 0; q < kSW + KW - 1; ++q) {
                    const int kk = kq + q - pw;
                    const bool ok = kk >= 0 && kk < g.Wn && row + kk < (REV ? g.past : g.nv);
                    in[q] = Vec8<E>::load_raw(xs + (ok ? row + kk : 0) * C, ok);
                }
                const float* wr = wv + (kx + (a * kh + b) * kw) * kCB;
#pragma unroll
                for (int d = 0; d < KW; ++d) {
                    float w[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) w[e] = wr[d * kCB + e];
#pragma unroll
                    for (int q = 0; q < kSW; ++q)
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[q][e] += w[e] * Vec8<E>::at(in[q + d], e);
                }
            }
#pragma unroll
        for (int q = 0; q < kSW; ++q) {
            const int kk = kq + q, m = (f * g.Hn + j) * g.Wn + kk;
            if (kk < g.Wn && m < g.past) Vec8<E>::store(y + (g.base + g.L + m) * C + c0, acc[q]);
        }
    };
    if (tid == 0) next_tile = atomicAdd(ctr, 1);
    __syncthreads();
    for (int64_t tile = t_begin + next_tile; tile < t_end;) {
        int claim = 0;
        if (tid == 0) claim = atomicAdd(ctr, 1);            // the next tile, claimed while this one runs
        run_tile(tile);
        __syncthreads();                                    // every thread has read next_tile
        if (tid == 0) next_tile = claim;
        __syncthreads();
        tile = t_begin + next_tile;
    }
}

// ---- weight gradients ----
// dw_text[i][c]      = sum over text tokens t (t-i >= 0)   x[t-i][c] dy[t][c]
// dw_vis[a][b][d][c] = sum over grid outputs (i, j, k)     x[i-a, j+b-(kh-1)/2, k+d-(kw-1)/2][c] dy[i,j,k][c]
// with x zero outside the grid. A work unit is (channel block, part of the block's tile
// list, row group): row group a < kt sums the kh*kw visual taps of time offset a, row group
// kt the text taps. Part p holds every parts-th tile from tile p, so the units running
// together cover adjacent tiles: the row groups of a part read the same dy rows at the same
// time, and the x frame one row group reads is read by the next one a few tiles later, while
// it is still in the XCD's L2 (with contiguous parts each frame was fetched once per row
// group, 1.8x the input bytes; now about 1.1x). A thread holds 8 channels and every tap of its group for one strip lane
// (a visual tile's 32 strips, one per lane); per strip it widens the strip's 4 dy columns
// once and each x row's kw+3 columns once, then does kw*4*8 FMAs per row. The unit's 32
// strip lanes are added in LDS in a fixed order and written as one partial per (tap,
// channel); the reduce kernel adds the parts in order, so the result does not depend on
// scheduling. The unit's tile loop has one straight-line body per case (text, whole-frame
// buffer loads, checked loads), so the 8*kh*kw tap sums stay in their registers across
// iterations; like the forward, the pass is bound by vector instructions (FMAs plus the bf16
// widening), not by HBM.
constexpr int kDwUnitsTarget = 2048;

int dw_parts(int C, int kt)
{
    const int per_part = ((C + kCB - 1) / kCB) * (kt + 1);
    return std::max(1, std::min(1024, (kDwUnitsTarget + per_part - 1) / per_part));
}

template <typename E, int KH, int KW>
__global__ __launch_bounds__(kCT) void kda_short_conv_dw_kernel(
    const E* __restrict__ x, const E* __restrict__ dy, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ text_len, const int32_t* __restrict__ grid, const int32_t* __restrict__ tile_off,
    float* __restrict__ partial, int64_t T, int num_seqs, int C, int kx, int kt, int parts, int units)
{
    constexpr int kh = KH;
    constexpr int NACC = KH * KW > 8 ? KH * KW : 8;         // visual taps of one time offset, or text taps
    constexpr int es = int(sizeof(E));
    constexpr int kLanes = kCT / 8;                         // strip lanes (x 8 channel groups = 64 channels)
    static_assert(kLanes == kStrips, "one strip per lane per visual tile");
    __shared__ float red[kCT * 8];
    const int u = (blockIdx.x & 7) * int(gridDim.x >> 3) + int(blockIdx.x >> 3);
    if (u >= units) return;                                 // uniform over the workgroup
    const int tid = threadIdx.x, cv = tid & 7, sl = tid >> 3;
    const int rg = u % (kt + 1), p = (u / (kt + 1)) % parts, cb = u / ((kt + 1) * parts);
    const bool text = rg == kt;
    const int a = rg, ph = (kh - 1) / 2, pw = (KW - 1) / 2;
    const int per_cb = tile_off[num_seqs];
    // part p takes tiles p, p + parts, ... so that the parts running together cover adjacent tiles
    const int t0 = p, t1 = per_cb, S = parts;
    auto next_from = [&](int lo) { return lo + ((p - lo) % S + S) % S; };
    // lanes past the last channel read channels 0..7 of the same tokens and write nothing, so
    // every lane runs the same code
    const bool cok = kCB * cb + 8 * cv < C;                 // C is a multiple of 8: all 8 channels exist
    const int c0 = cok ? kCB * cb + 8 * cv : 0;
    float acc[NACC][8];
#pragma unroll
    for (int s = 0; s < NACC; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[s][e] = 0.f;

    int n0 = 0;
    if (t0 < t1) {                                          // tile_off[n0] <= t0 < tile_off[n0 + 1]
        int hi = num_seqs;
        while (hi - n0 > 1) {
            const int mid = (n0 + hi) >> 1;
            if (tile_off[mid] <= t0) n0 = mid; else hi = mid;
        }
    }
    // Three loops over the unit's tiles, each with its own straight-line body, so the tap sums
    // stay in place: text taps; visual taps when every sample the unit touches is whole frames
    // under the buffer limit (out-of-grid positions read as zero through the buffer bounds);
    // visual taps with per-position checks otherwise.
    bool all_fast = !text;
    for (int m = n0; all_fast && m < num_seqs && tile_off[m] < t1; ++m) {
        const SampleGeom g = sample_geom(cu, text_len, grid, m, T);
        if (g.Tn > 0 && !(g.past == g.nv && int64_t(g.Tn) * g.Hn * g.Wn == g.nv &&
                          int64_t(g.nv) * C * es <= kBufLimit))
            all_fast = false;
    }
    if (text) {
        int n = n0;
        for (int tp = t0; tp < t1; tp += S) {
            while (tile_off[n + 1] <= tp) ++n;              // next sample with tiles
            const SampleGeom g = sample_geom(cu, text_len, grid, n, T);
            const SampleTiles st = sample_tiles(g);
            const int local = tp - tile_off[n];
            if (local >= st.ntext) { tp = next_from(tile_off[n + 1]) - S; continue; }
            for (int r = sl; r < kTextTok; r += kLanes) {
                const int rel = local * kTextTok + r;
                if (rel >= g.L) break;
                const int tok = g.base + rel;
                const typename Vec8<E>::Raw gr = Vec8<E>::load_raw(dy + int64_t(tok) * C + c0, true);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (i >= kx || rel - i < 0) break;
                    const typename Vec8<E>::Raw xr = Vec8<E>::load_raw(x + int64_t(tok - i) * C + c0, true);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[i][e] += Vec8<E>::at(xr, e) * Vec8<E>::at(gr, e);
                }
            }
        }
    } else if (all_fast) {
        // samples in turn, then the sample's visual tiles inside [t0, t1): no branch in the
        // tile loop, so the tap sums keep their registers
        for (int n = n0; n < num_seqs && tile_off[n] < t1; ++n) {
            const SampleGeom g = sample_geom(cu, text_len, grid, n, T);
            const SampleTiles st = sample_tiles(g);
            const int v_lo = max(t0, tile_off[n] + st.ntext), v_hi = min(t1, tile_off[n] + st.ntext + st.nvis);
            for (int tp = next_from(v_lo); tp < v_hi; tp += S) {
                const int local = tp - tile_off[n];
                const int sidx = (local - st.ntext) * kStrips + sl;
                const int per_frame = g.Hn * st.nsw;
                const int f = sidx / per_frame;
                const int j = (sidx - f * per_frame) / st.nsw;
                const int kq = (sidx - f * per_frame - j * st.nsw) * kSW;
                const bool vo = f < g.Tn;                       // the strip's outputs exist
                const bool vx = vo && f - a >= 0;               // and so does its x frame
                const int64_t v0 = int64_t(g.base + g.L) * C;
                const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<E*>(x + v0), 0, int(int64_t(g.nv) * C * es), kBufFlags);
                const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<E*>(dy + v0), 0, int(int64_t(g.nv) * C * es), kBufFlags);
                const uint32_t rowb = uint32_t(g.Wn) * uint32_t(C) * es;
                const uint32_t doff = vo ? uint32_t(f * g.Hn + j) * rowb : kBufLimit;
                {
                    float gv[kSW][8];
#pragma unroll
                    for (int q = 0; q < kSW; ++q) {
                        const int kk = kq + q;
                        const typename Vec8<E>::Raw r =
                            Vec8<E>::load_buf(rd, doff + (kk < g.Wn ? uint32_t(kk * C + c0) * es : kBufLimit));
#pragma unroll
                        for (int e = 0; e < 8; ++e) gv[q][e] = Vec8<E>::at(r, e);
                    }
                    uint32_t colv[kSW + KW - 1];
#pragma unroll
                    for (int q = 0; q < kSW + KW - 1; ++q) {
                        const int kk = kq + q - pw;
                        colv[q] = kk >= 0 && kk < g.Wn ? uint32_t(kk * C + c0) * es : kBufLimit;
                    }
#pragma unroll
                    for (int b = 0; b < KH; ++b) {
                        const int jj = j + b - ph;
                        const uint32_t roff =
                            vx && jj >= 0 && jj < g.Hn ? uint32_t((f - a) * g.Hn + jj) * rowb : kBufLimit;
                        typename Vec8<E>::Raw in[kSW + KW - 1];
#pragma unroll
                        for (int q = 0; q < kSW + KW - 1; ++q) in[q] = Vec8<E>::load_buf(rx, roff + colv[q]);
#pragma unroll
                        for (int q = 0; q < kSW + KW - 1; ++q) {
                            float xf[8];
#pragma unroll
                            for (int e = 0; e < 8; ++e) xf[e] = Vec8<E>::at(in[q], e);
#pragma unroll
                            for (int d = 0; d < KW; ++d) {
                                const int o = q - d;            // output column fed by this tap
                                if (o < 0 || o >= kSW) continue;
#pragma unroll
                                for (int e = 0; e < 8; ++e) acc[b * KW + d][e] += xf[e] * gv[o][e];
                            }
                        }
                    }
                }
            }
        }
    } else {
        int n = n0;
        for (int tp = t0; tp < t1; tp += S) {
            while (tile_off[n + 1] <= tp) ++n;
            const SampleGeom g = sample_geom(cu, text_len, grid, n, T);
            const SampleTiles st = sample_tiles(g);
            const int local = tp - tile_off[n];
            if (local < st.ntext) { tp = next_from(tile_off[n] + st.ntext) - S; continue; }
            if (local >= st.ntext + st.nvis) { tp = next_from(tile_off[n + 1]) - S; continue; }
            const int sidx = (local - st.ntext) * kStrips + sl;
            const int per_frame = g.Hn * st.nsw;
            const int f = sidx / per_frame;
            if (f >= g.Tn || f - a < 0) continue;
            const int j = (sidx - f * per_frame) / st.nsw;
            const int kq = (sidx - f * per_frame - j * st.nsw) * kSW;
            const int64_t v0 = int64_t(g.base + g.L) * C;
            const E* xs = x + v0 + c0;
            const E* ds = dy + v0 + c0;
            const int orow = (f * g.Hn + j) * g.Wn;
            {
                float gv[kSW][8];
#pragma unroll
                for (int q = 0; q < kSW; ++q) {
                    const int kk = kq + q;
                    const bool ok = kk < g.Wn && orow + kk < g.past;
                    const typename Vec8<E>::Raw r = Vec8<E>::load_raw(ds + int64_t(ok ? orow + kk : 0) * C, ok);
#pragma unroll
                    for (int e = 0; e < 8; ++e) gv[q][e] = Vec8<E>::at(r, e);
                }
#pragma unroll
                for (int b = 0; b < KH; ++b) {
                    const int jj = j + b - ph;
                    if (jj < 0 || jj >= g.Hn) continue;
                    const int row = ((f - a) * g.Hn + jj) * g.Wn;
                    typename Vec8<E>::Raw in[kSW + KW - 1];
#pragma unroll
                    for (int q = 0; q < kSW + KW - 1; ++q) {
                        const int kk = kq + q - pw;
                        const bool ok = kk >= 0 && kk < g.Wn && row + kk < g.past;
                        in[q] = Vec8<E>::load_raw(xs + int64_t(ok ? row + kk : 0) * C, ok);
                    }
#pragma unroll
                    for (int q = 0; q < kSW + KW - 1; ++q)
#pragma unroll
                        for (int d = 0; d < KW; ++d) {
                            const int o = q - d;
                            if (o < 0 || o >= kSW) continue;
#pragma unroll
                            for (int e = 0; e < 8; ++e) acc[b * KW + d][e] += Vec8<E>::at(in[q], e) * gv[o][e];
                        }
                }
            }
        }
    }

    // the 32 strip lanes of each channel group, added in lane order; one tap at a time
    const int ntaps = kx + kt * kh * KW;
#pragma unroll
    for (int s = 0; s < NACC; ++s) {
        const bool live = text ? s < kx : s / KW < kh;      // uniform over the workgroup
        if (!live) continue;
#pragma unroll
        for (int e = 0; e < 8; ++e) red[tid * 8 + e] = acc[s][e];
        __syncthreads();
        if (tid < 64) {
            const int q = tid >> 3, e = tid & 7, c = kCB * cb + 8 * q + e;
            float sum = 0.f;
            for (int l = 0; l < kLanes; ++l) sum += red[(l * 8 + q) * 8 + e];
            const int tap = text ? s : kx + (a * kh + s / KW) * KW + s % KW;
            if (c < C) partial[(int64_t(p) * ntaps + tap) * C + c] = sum;   // lanes past C hold no channel
        }
        __syncthreads();
    }
}

// dw[tap][c] = sum over parts, in part order; taps < kx go to dw_text, the rest to dw_vis
__global__ __launch_bounds__(256) void kda_short_conv_dw_reduce_kernel(const float* __restrict__ partial,
                                                                       float* __restrict__ dw_text,
                                                                       float* __restrict__ dw_vis, int C, int kx,
                                                                       int ntaps, int parts)
{
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t nel = int64_t(ntaps) * C;
    if (i >= nel) return;
    float sum = 0.f;
    for (int q = 0; q < parts; ++q) sum += partial[q * nel + i];
    if (i < int64_t(kx) * C) dw_text[i] = sum; else dw_vis[i - int64_t(kx) * C] = sum;
}

template <typename E, int KW, bool REV>
void launch_conv_kw(const ConvArgs& a, const void* in, void* out, int32_t* tile_off, int* queue, size_t smem,
                    int blocks, int ncb)
{
    hipLaunchKernelGGL((kda_short_conv_kernel<E, KW, REV>), dim3(blocks), dim3(kCT), smem, a.stream,
                       static_cast<const E*>(in), a.w_text, a.w_vis, a.cu_seqlens, a.text_len, a.grid, tile_off,
                       queue, static_cast<E*>(out), a.total_tokens, a.num_seqs, a.channels, a.k_text, a.k_t, a.k_h, ncb);
}

// the kernel width is a template argument: it sizes the strip's input registers
template <typename E, bool REV>
void launch_conv(const ConvArgs& a, const void* in, void* out, int32_t* tile_off, int* queue, size_t smem, int blocks,
                 int ncb)
{
    switch (a.k_w) {
    case 1: launch_conv_kw<E, 1, REV>(a, in, out, tile_off, queue, smem, blocks, ncb); break;
    case 3: launch_conv_kw<E, 3, REV>(a, in, out, tile_off, queue, smem, blocks, ncb); break;
    default: launch_conv_kw<E, 5, REV>(a, in, out, tile_off, queue, smem, blocks, ncb); break;
    }
}

template <typename E, int KH, int KW>
void launch_dw_k(const ConvBwdArgs& a, int32_t* tile_off, float* partial, int blocks, int parts, int units)
{
    hipLaunchKernelGGL((kda_short_conv_dw_kernel<E, KH, KW>), dim3(blocks), dim3(kCT), 0, a.f.stream,
                       static_cast<const E*>(a.f.x), static_cast<const E*>(a.dy), a.f.cu_seqlens, a.f.text_len,
                       a.f.grid, tile_off, partial, a.f.total_tokens, a.f.num_seqs, a.f.channels, a.f.k_text,
                       a.f.k_t, parts, units);
}

// the kernel's height and width are template arguments: they size the per-thread tap sums
template <typename E, int KH>
void launch_dw_h(const ConvBwdArgs& a, int32_t* tile_off, float* partial, int blocks, int parts, int units)
{
    switch (a.f.k_w) {
    case 1: launch_dw_k<E, KH, 1>(a, tile_off, partial, blocks, parts, units); break;
    case 3: launch_dw_k<E, KH, 3>(a, tile_off, partial, blocks, parts, units); break;
    default: launch_dw_k<E, KH, 5>(a, tile_off, partial, blocks, parts, units); break;
    }
}

template <typename E>
void launch_dw(const ConvBwdArgs& a, int32_t* tile_off, float* partial, int blocks, int parts, int units)
{
    switch (a.f.k_h) {
    case 1: launch_dw_h<E, 1>(a, tile_off, partial, blocks, parts, units); break;
    case 3: launch_dw_h<E, 3>(a, tile_off, partial, blocks, parts, units); break;
    default: launch_dw_h<E, 5>(a, tile_off, partial, blocks, parts, units); break;
    }
}

}  // namespace

static size_t conv_table_bytes(int32_t num_seqs) { return ((size_t(num_seqs) + 1) * 4 + 255) & ~size_t(255); }
size_t conv_workspace_bytes(int32_t num_seqs) { return conv_table_bytes(num_seqs) + kQueueBytes; }

size_t conv_bwd_workspace_bytes(int32_t num_seqs, int32_t channels, int32_t k_text, int32_t k_t, int32_t k_h,
                                int32_t k_w)
{
    const size_t ntaps = size_t(k_text) + size_t(k_t) * k_h * k_w;
    return conv_workspace_bytes(num_seqs) + size_t(dw_parts(channels, k_t)) * ntaps * size_t(channels) * 4;
}

hipError_t launch_short_conv(const ConvArgs& a, void* workspace, TimingHook* th)
{
    if (a.total_tokens == 0 || a.num_seqs == 0) return hipSuccess;
    const size_t smem = size_t(a.k_text + a.k_t * a.k_h * a.k_w) * kCB * sizeof(float);
    const int ncb = (a.channels + kCB - 1) / kCB;
    int32_t* tile_off = static_cast<int32_t*>(workspace);
    if (th) th->begin("conv_plan", a.stream);
    int* queue = reinterpret_cast<int*>(static_cast<char*>(workspace) + conv_table_bytes(a.num_seqs));
    hipLaunchKernelGGL(kda_conv_plan_kernel, dim3(1), dim3(1024), 0, a.stream, a.cu_seqlens, a.text_len, a.grid,
                       tile_off, queue, a.num_seqs, a.total_tokens);
    if (th) th->end(a.stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int blocks = 256 * kWgPerCu;              // every CU, kWgPerCu resident workgroups each
    if (th) th->begin("conv", a.stream);
    if (a.dtype_bf16)
        launch_conv<uint16_t, false>(a, a.x, a.y, tile_off, queue, smem, blocks, ncb);
    else
        launch_conv<float, false>(a, a.x, a.y, tile_off, queue, smem, blocks, ncb);
    if (th) th->end(a.stream);
    return hipGetLastError();
}

hipError_t launch_short_conv_backward(const ConvBwdArgs& b, void* workspace, TimingHook* th)
{
    const ConvArgs& a = b.f;
    const int ntaps = a.k_text + a.k_t * a.k_h * a.k_w;
    const int64_t nel = int64_t(ntaps) * a.channels;
    if (a.total_tokens == 0 || a.num_seqs == 0) {         // empty sums: zeros, no workspace
        hipLaunchKernelGGL(kda_short_conv_dw_reduce_kernel, dim3(unsigned((nel + 255) / 256)), dim3(256), 0,
                           a.stream, static_cast<const float*>(nullptr), b.dw_text, b.dw_vis, a.channels, a.k_text,
                           ntaps, 0);
        return hipGetLastError();
    }
    const size_t smem = size_t(ntaps) * kCB * sizeof(float);
    const int ncb = (a.channels + kCB - 1) / kCB;
    int32_t* tile_off = static_cast<int32_t*>(workspace);
    float* partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + conv_workspace_bytes(a.num_seqs));
    if (th) th->begin("conv_bwd_plan", a.stream);
    int* queue = reinterpret_cast<int*>(static_cast<char*>(workspace) + conv_table_bytes(a.num_seqs));
    hipLaunchKernelGGL(kda_conv_plan_kernel, dim3(1), dim3(1024), 0, a.stream, a.cu_seqlens, a.text_len, a.grid,
                       tile_off, queue, a.num_seqs, a.total_tokens);
    if (th) th->end(a.stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (th) th->begin("conv_dx", a.stream);
    if (a.dtype_bf16)
        launch_conv<uint16_t, true>(a, b.dy, b.dx, tile_off, queue, smem, 256 * kWgPerCu, ncb);
    else
        launch_conv<float, true>(a, b.dy, b.dx, tile_off, queue, smem, 256 * kWgPerCu, ncb);
    if (th) th->end(a.stream);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int parts = dw_parts(a.channels, a.k_t);
    const int units = ncb * parts * (a.k_t + 1);
    const int blocks = (units + 7) / 8 * 8;
    if (th) th->begin("conv_dw", a.stream);
    if (a.dtype_bf16)
        launch_dw<uint16_t>(b, tile_off, partial, blocks, parts, units);
    else
        launch_dw<float>(b, tile_off, partial, blocks, parts, units);
    if (th) th->end(a.stream);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (th) th->begin("conv_dw_reduce", a.stream);
    hipLaunchKernelGGL(kda_short_conv_dw_reduce_kernel, dim3(unsigned((nel + 255) / 256)), dim3(256), 0, a.stream,
                       partial, b.dw_text, b.dw_vis, a.channels, a.k_text, ntaps, parts);
    if (th) th->end(a.stream);
    return hipGetLastError();
}

}  // namespace kda
