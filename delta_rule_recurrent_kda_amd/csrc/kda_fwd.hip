// kda_fwd.hip -- chunkwise KDA forward scan for gfx950 (CDNA4).
//
// Recurrence (Chimera, arXiv 2607.28611; update printed in the explainer page,
// "One stream, three mechanisms, no positions"; definitions and the reset rule in
// the paper's Sec. 3 KDA paragraph, Eq. 14):
//     S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,   o_t = S_t^T q_t,
//     S_0 = 0 at every packed-sample boundary.
//
// Chunkwise form used here (derived from that recurrence; the pages give no
// kernel). For a chunk of n <= C tokens with state S on entry, G = inclusive
// row-cumsum of log a (per key channel), gamma = exp(G[n-1]):
//     Qh = Q*exp(G)   Kh = K*exp(G)   Kc = K*exp(-G)   Kb = K*exp(G[n-1]-G)
//     A  = StrictLower(diag(b) Kh Kc^T),   T = (I + A)^{-1}        (UT transform)
//     X  = V - Kh S,   Vn = T diag(b) X   (rows are the delta-rule innovations)
//     O  = Qh S + LowerIncl(Qh Kc^T) Vn,   S <- diag(gamma) S + Kb^T Vn
// The diagonal of Qh Kc^T equals q_t . k_t exactly and is taken in fp32 from the
// stored inputs rather than from the rounded decayed operands.
//
// Mapping: one workgroup of 4 wave64s per (sample, head, 64-column value tile).
// Every wave owns 16 value columns of the state for the whole scan (S is fp32 in
// VGPRs, 128x16 per wave), so the only cross-wave traffic is the v-independent
// per-chunk operands staged in LDS. Value columns never mix in the recurrence,
// which is what makes this split exact.
//
// MFMA fragments: all contractions use 16x16 output tiles (v_mfma_f32_16x16x32_bf16
// for bf16 data, v_mfma_f32_16x16x4_f32 for fp32 data). A k-block of 32 is held by
// lane (r = lane%16, g = lane/16) as 8 elements: k = 16*t + 4*g + i (t in {0,1},
// i in 0..3). An MFMA accumulator holds rows 4*g + i, column r, so two stacked
// accumulator tiles are directly a B operand (k along their rows) and the A
// operand of their transpose; both operands of every product use the same k map.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // 4 wave64
constexpr int kBV = 64;         // value columns per workgroup (16 per wave)

__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }
__device__ __forceinline__ uint16_t f2bf(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }

// ---------------------------------------------------------------------------
// element-type traits: storage type E, MFMA fragment and product
// ---------------------------------------------------------------------------
template <typename E> struct Elt;

template <> struct Elt<uint16_t> {            // bf16 data
    struct Frag { uint4 u; };
    static constexpr int kPad = 4;            // row padding (elements) of LDS operand tiles
    __device__ static float to_f(uint16_t x) { return bf2f(x); }
    __device__ static uint16_t from_f(float x) { return f2bf(x); }
    // 8 elements of a row at k = 16t + 4g + i
    __device__ static Frag load(const uint16_t* row, int g) {
        const uint2 lo = *reinterpret_cast<const uint2*>(row + 4 * g);
        const uint2 hi = *reinterpret_cast<const uint2*>(row + 16 + 4 * g);
        return Frag{make_uint4(lo.x, lo.y, hi.x, hi.y)};
    }
    // same k map, elements taken down a column (B operand from a row-major matrix)
    __device__ static Frag load_col(const float* m, int ld, int k0, int col, int g, bool upper_half) {
        float v[8];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[4 * t + i] = (t == 0 || upper_half) ? m[(k0 + 16 * t + 4 * g + i) * ld + col] : 0.f;
        return pack(v);
    }
    __device__ static Frag load_f32row(const float* row, int g, bool upper_half) {
        float v[8];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[4 * t + i] = (t == 0 || upper_half) ? row[16 * t + 4 * g + i] : 0.f;
        return pack(v);
    }
    __device__ static Frag pack(const float* v) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            w[j] = uint32_t(f2bf(v[2 * j])) | (uint32_t(f2bf(v[2 * j + 1])) << 16);
        return Frag{make_uint4(w[0], w[1], w[2], w[3])};
    }
    // two accumulator tiles (rows 0..15 and 16..31 of a k-block), optional row scale
    __device__ static Frag from_acc(const f32x4& a0, const f32x4& a1) {
        float v[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        return pack(v);
    }
    __device__ static f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.u),
                                                       __builtin_bit_cast(bf16x8, b.u), c, 0, 0, 0);
    }
};

template <> struct Elt<float> {               // fp32 data
    struct Frag { float4 lo, hi; };
    static constexpr int kPad = 4;
    __device__ static float to_f(float x) { return x; }
    __device__ static float from_f(float x) { return x; }
    __device__ static Frag load(const float* row, int g) {
        return Frag{*reinterpret_cast<const float4*>(row + 4 * g),
                    *reinterpret_cast<const float4*>(row + 16 + 4 * g)};
    }
    __device__ static Frag load_col(const float* m, int ld, int k0, int col, int g, bool upper_half) {
        const float* p = m + (k0 + 4 * g) * ld + col;
        Frag f{make_float4(p[0], p[ld], p[2 * ld], p[3 * ld]), make_float4(0.f, 0.f, 0.f, 0.f)};
        if (upper_half) f.hi = make_float4(p[16 * ld], p[17 * ld], p[18 * ld], p[19 * ld]);
        return f;
    }
    // rows of the fp32 scratch have an odd stride: scalar reads only
    __device__ static Frag load_f32row(const float* row, int g, bool upper_half) {
        const float* p = row + 4 * g;
        Frag f{make_float4(p[0], p[1], p[2], p[3]), make_float4(0.f, 0.f, 0.f, 0.f)};
        if (upper_half) f.hi = make_float4(p[16], p[17], p[18], p[19]);
        return f;
    }
    __device__ static Frag from_acc(const f32x4& a0, const f32x4& a1) {
        return Frag{make_float4(a0[0], a0[1], a0[2], a0[3]), make_float4(a1[0], a1[1], a1[2], a1[3])};
    }
    __device__ static f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, c, 0, 0, 0);
        return c;
    }
};

// Raw per-lane chunk loads: CPL consecutive key channels of one row.
template <typename E, int CPL> struct Raw;
template <> struct Raw<uint16_t, 1> { using T = uint16_t;
    __device__ static float get(T x, int) { return bf2f(x); } };
template <> struct Raw<uint16_t, 2> { using T = uint32_t;
    __device__ static float get(T x, int c) { return bf2f(uint16_t(c ? (x >> 16) : (x & 0xFFFFu))); } };
template <> struct Raw<float, 1> { using T = float;
    __device__ static float get(T x, int) { return x; } };
template <> struct Raw<float, 2> { using T = float2;
    __device__ static float get(T x, int c) { return c ? x.y : x.x; } };

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// shared-memory layout
// ---------------------------------------------------------------------------
template <typename E, int DK, int C> struct Smem {
    static constexpr int LDK = DK + Elt<E>::kPad;     // row stride of [C][DK] tiles
    static constexpr int LDC = C + Elt<E>::kPad;      // row stride of [*][C] tiles
    static constexpr int LDV = kBV + 16 / sizeof(E);  // row stride of V / O staging (16B rows)
    static constexpr int LDA = C + 1;                 // fp32 [C][C] scratch
    E qh[C * LDK];        // Qh
    E kh[C * LDK];        // -Kh
    E kc[C * LDK];        // Kc
    E kbt[DK * LDC];      // Kb^T (key channel major)
    E p[C * LDC];         // LowerIncl(Qh Kc^T), row-major [i][j]
    E tb[C * LDC];        // T in the operand type
    E vs[C * LDV];        // V tile
    E os[C * LDV];        // O tile staging
    float a[C * LDA];     // A (strictly lower)
    float t32[C * LDA];   // T in fp32 while it is being built
    float gam[DK];
    float beta[C];
    float diag[C];
    float tot[4 * DK];
};

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <typename E, int DK, int C>
__global__ __launch_bounds__(kThreads) void kda_fwd_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ la, const E* __restrict__ beta, const int32_t* __restrict__ cu,
    E* __restrict__ out, float* __restrict__ final_state,
    int num_seqs, int H, int DV)
{
    using EL = Elt<E>;
    using Frag = typename EL::Frag;
    constexpr int CPL = DK / 64;          // key channels per lane in the elementwise phase
    constexpr int RPW = C / 4;            // chunk rows per wave in the elementwise phase
    constexpr int NRT = C / 16;           // 16-row tiles per chunk
    constexpr int NKC = C / 32;           // 32-wide k-blocks over chunk rows
    constexpr int NKD = DK / 32;          // 32-wide k-blocks over key channels
    constexpr int NCT = DK / 16;          // 16-row tiles over key channels
    constexpr int VPR = kBV * sizeof(E) / 16;                 // 16-byte pieces per V row
    constexpr int VLD = C * VPR / kThreads;                   // V pieces per thread
    static_assert(VLD >= 1 && (C * VPR) % kThreads == 0, "V tile split");
    using RT = Raw<E, CPL>;
    using RawT = typename RT::T;
    using S_ = Smem<E, DK, C>;
    constexpr int LDK = S_::LDK, LDC = S_::LDC, LDV = S_::LDV, LDA = S_::LDA;

    extern __shared__ __align__(16) unsigned char smem_raw[];
    S_& sm = *reinterpret_cast<S_*>(smem_raw);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;

    // XCD-aware block order: the value tiles of one (sample, head) are 8 blocks
    // apart so that they land on the same XCD and share its L2 for q, k, log a.
    const int nvt = DV / kBV;
    const int b = blockIdx.x;
    const int vt = (b >> 3) % nvt;
    const int unit = (b / (8 * nvt)) * 8 + (b & 7);
    if (unit >= num_seqs * H) return;
    const int n = unit / H, h = unit % H;
    const int64_t seq0 = cu[n];
    const int64_t len = int64_t(cu[n + 1]) - seq0;
    const int nchunks = int((len + C - 1) / C);
    const int col0 = vt * kBV;

    // blocks above the diagonal of T and P are never written: clear once
    for (int i = tid; i < C * LDA; i += kThreads) sm.t32[i] = 0.f;
    for (int i = tid; i < C * LDC; i += kThreads) { sm.tb[i] = E(0); sm.p[i] = E(0); }

    // state: wave owns value columns [16*wave, 16*wave+16) of the tile; NCT tiles of 16 key rows
    f32x4 S[NCT];
#pragma unroll
    for (int i = 0; i < NCT; ++i) S[i] = zero4();

    // ---- raw loads of one chunk into registers --------------------------------
    RawT rq[RPW], rk[RPW], rg[RPW];
    uint4 rv[VLD];
    E rb = E(0);
    auto load_chunk = [&](int c) {
        const int64_t t0 = seq0 + int64_t(c) * C;
        const int nrow = int(min<int64_t>(C, len - int64_t(c) * C));
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            const int row = wave * RPW + j;
            if (row < nrow) {
                const int64_t off = ((t0 + row) * H + h) * DK + lane * CPL;
                rq[j] = *reinterpret_cast<const RawT*>(q + off);
                rk[j] = *reinterpret_cast<const RawT*>(k + off);
                rg[j] = *reinterpret_cast<const RawT*>(la + off);
            } else {
                rq[j] = RawT{}; rk[j] = RawT{}; rg[j] = RawT{};
            }
        }
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int piece = tid + i * kThreads;
            const int row = piece / VPR, part = piece % VPR;
            if (row < nrow)
                rv[i] = *reinterpret_cast<const uint4*>(v + ((t0 + row) * H + h) * DV + col0 +
                                                        part * (16 / sizeof(E)));
            else
                rv[i] = make_uint4(0, 0, 0, 0);
        }
        if (tid < C) rb = (tid < nrow) ? beta[(t0 + tid) * H + h] : E(0);
    };

    if (nchunks > 0) load_chunk(0);

    for (int c = 0; c < nchunks; ++c) {
        const int64_t t0 = seq0 + int64_t(c) * C;
        const int nrow = int(min<int64_t>(C, len - int64_t(c) * C));

        // ---- phase 0a: local cumsum of log a over this wave's rows -------------
        float G[RPW][CPL];
        float diagp[RPW];
#pragma unroll
        for (int ch = 0; ch < CPL; ++ch) {
            float run = 0.f;
#pragma unroll
            for (int j = 0; j < RPW; ++j) { run += RT::get(rg[j], ch); G[j][ch] = run; }
            sm.tot[wave * DK + lane * CPL + ch] = run;
        }
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
            float s = 0.f;
#pragma unroll
            for (int ch = 0; ch < CPL; ++ch) s += RT::get(rq[j], ch) * RT::get(rk[j], ch);
            diagp[j] = s;
        }
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int piece = tid + i * kThreads;
            *reinterpret_cast<uint4*>(&sm.vs[(piece / VPR) * LDV + (piece % VPR) * (16 / sizeof(E))]) = rv[i];
        }
        if (tid < C) sm.beta[tid] = EL::to_f(rb);

        // exact diagonal q_t . k_t: reduce-scatter the RPW row partials over the wave
        {
            float vals[RPW];
#pragma unroll
            for (int j = 0; j < RPW; ++j) vals[j] = diagp[j];
            int cnt = RPW;
            int mask = 32;
#pragma unroll
            for (int step = 0; step < 6; ++step) {
                if (cnt > 1) {
                    const bool upper = (lane & mask) != 0;
                    const int half = cnt / 2;
#pragma unroll
                    for (int j = 0; j < RPW / 2; ++j) {
                        if (j < half) {
                            const float send = upper ? vals[j] : vals[j + half];
                            const float keep = upper ? vals[j + half] : vals[j];
                            vals[j] = keep + __shfl_xor(send, mask);
                        }
                    }
                    cnt = half;
                } else {
                    vals[0] += __shfl_xor(vals[0], mask);
                }
                mask >>= 1;
            }
            // lane holds the total for row index built from its upper lane bits
            int rowi = 0, m2 = 32, c2 = RPW;
#pragma unroll
            for (int step = 0; step < 6; ++step) {
                if (c2 > 1) { c2 >>= 1; if (lane & m2) rowi += c2; }
                m2 >>= 1;
            }
            constexpr int low_bits = 64 / RPW;       // lanes sharing one row total
            if ((lane & (low_bits - 1)) == 0) sm.diag[wave * RPW + rowi] = vals[0];
        }
        __syncthreads();                                             // B1

        // ---- phase 0b: decay factors, decayed operands --------------------------
        {
            float off[CPL], glast[CPL];
#pragma unroll
            for (int ch = 0; ch < CPL; ++ch) {
                float o = 0.f, a = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float t = sm.tot[w * DK + lane * CPL + ch];
                    a += t;
                    if (w < wave) o += t;
                }
                off[ch] = o; glast[ch] = a;
            }
            if (wave == 0) {
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch) sm.gam[lane * CPL + ch] = __expf(glast[ch]);
            }
#pragma unroll
            for (int j = 0; j < RPW; ++j) {
                const int row = wave * RPW + j;
#pragma unroll
                for (int ch = 0; ch < CPL; ++ch) {
                    const int col = lane * CPL + ch;
                    const float Gj = G[j][ch] + off[ch];
                    const float e = __expf(Gj), ei = __expf(-Gj), eb = __expf(glast[ch] - Gj);
                    const float qv = RT::get(rq[j], ch), kv = RT::get(rk[j], ch);
                    sm.qh[row * LDK + col] = EL::from_f(qv * e);
                    sm.kh[row * LDK + col] = EL::from_f(-(kv * e));
                    sm.kc[row * LDK + col] = EL::from_f(kv * ei);
                    sm.kbt[col * LDC + row] = EL::from_f(kv * eb);
                }
            }
        }
        // prefetch the next chunk while this one is processed
        if (c + 1 < nchunks) load_chunk(c + 1);
        __syncthreads();                                             // B2

        // ---- phase 1: A = StrictLower(diag(b) Kh Kc^T), P = LowerIncl(Qh Kc^T) ----
        // computed transposed (Kc rows as the A operand) so that every lane writes
        // four consecutive columns of a row-major result.
        {
            constexpr int NPAIR = NRT * (NRT + 1) / 2;
            for (int pi = wave; pi < NPAIR; pi += 4) {
                int it = 0, rem = pi;
                while (rem > it) { rem -= it + 1; ++it; }
                const int jt = rem;                                    // jt <= it
                f32x4 accP = zero4(), accA = zero4();
#pragma unroll
                for (int kb = 0; kb < NKD; ++kb) {
                    const Frag fa = EL::load(&sm.kc[(16 * jt + r) * LDK + 32 * kb], g);
                    const Frag fq = EL::load(&sm.qh[(16 * it + r) * LDK + 32 * kb], g);
                    const Frag fk = EL::load(&sm.kh[(16 * it + r) * LDK + 32 * kb], g);
                    accP = EL::mma(fa, fq, accP);
                    accA = EL::mma(fa, fk, accA);
                }
                // accumulator element (row 16jt+4g+i, col 16it+r) is entry [i_=16it+r][j_=16jt+4g+i]
                const int irow = 16 * it + r;
                const float bi = sm.beta[irow];
                float pv[4], av[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int jcol = 16 * jt + 4 * g + i;
                    pv[i] = (jcol < irow) ? accP[i] : (jcol == irow ? sm.diag[irow] : 0.f);
                    av[i] = (jcol < irow) ? -bi * accA[i] : 0.f;       // kh holds -Kh
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sm.p[irow * LDC + 16 * jt + 4 * g + i] = EL::from_f(pv[i]);
                    sm.a[irow * LDA + 16 * jt + 4 * g + i] = av[i];
                }
            }
        }
        __syncthreads();                                             // B3

        // ---- phase 2a: diagonal 16x16 blocks of T = (I + A)^{-1} ----------------
        if (wave < NRT && lane < 16) {
            const int bb = 16 * wave, j = lane;
            float t[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = (i == j) ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) s -= sm.a[(bb + i) * LDA + bb + m] * t[m];
                t[i] = s;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                sm.t32[(bb + i) * LDA + bb + j] = t[i];
                sm.tb[(bb + i) * LDC + bb + j] = EL::from_f(t[i]);
            }
        }
        __syncthreads();                                             // B4

        // ---- phase 2b: T[b1][b0] = -T[b1][b1] (A[b1][b0] T[b0][b0]) in each 32-row block
        if (wave < NRT / 2) {
            const int b0 = 32 * wave, b1 = b0 + 16;
            // Y = A[b1][b0] T[b0][b0] (k over 16 -> upper half of the k-block is zero)
            const Frag fa = EL::load_f32row(&sm.a[(b1 + r) * LDA + b0], g, false);
            const Frag fb = EL::load_col(sm.t32, LDA, b0, b0 + r, g, false);   // T[b0+k][b0+r]
            f32x4 y = EL::mma(fa, fb, zero4());
            // T[b1][b0] = -T[b1][b1] Y: A operand T[b1][b1] (k over 16), B operand Y (accumulator rows)
            const Frag ft = EL::load_f32row(&sm.t32[(b1 + r) * LDA + b1], g, false);
            const Frag fy = EL::from_acc(y, zero4());
            f32x4 tz = EL::mma(ft, fy, zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float tv = -tz[i];
                sm.t32[(b1 + 4 * g + i) * LDA + b0 + r] = tv;
                sm.tb[(b1 + 4 * g + i) * LDC + b0 + r] = EL::from_f(tv);
            }
        }
        __syncthreads();                                             // B5

        // ---- phase 2c (C = 64): T[32:64][0:32] = -T2 (A[32:64][0:32] T1) ---------
        if constexpr (NRT == 4) {
            if (wave < 2) {
                const int cj = 16 * wave;                               // column tile of the result
                f32x4 z[2];
#pragma unroll
                for (int zi = 0; zi < 2; ++zi) {
                    const Frag fa = EL::load_f32row(&sm.a[(32 + 16 * zi + r) * LDA + 0], g, true);
                    const Frag fb = EL::load_col(sm.t32, LDA, 0, cj + r, g, true);
                    z[zi] = EL::mma(fa, fb, zero4());
                }
                const Frag fz = EL::from_acc(z[0], z[1]);
#pragma unroll
                for (int ti = 0; ti < 2; ++ti) {
                    const Frag ft = EL::load_f32row(&sm.t32[(32 + 16 * ti + r) * LDA + 32], g, true);
                    const f32x4 tz = EL::mma(ft, fz, zero4());
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sm.tb[(32 + 16 * ti + 4 * g + i) * LDC + cj + r] = EL::from_f(-tz[i]);
                }
            }
            __syncthreads();                                         // B6
        }

        // ---- phase 3: the state pass for this wave's 16 value columns -----------
        {
            const int vc = 16 * wave + r;                               // column within the tile
            Frag sf[NKD];
#pragma unroll
            for (int kb = 0; kb < NKD; ++kb) sf[kb] = EL::from_acc(S[2 * kb], S[2 * kb + 1]);

            // X = V - Kh S, scaled by beta per row
            f32x4 X[NRT];
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                f32x4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = EL::to_f(sm.vs[(16 * rt + 4 * g + i) * LDV + vc]);
#pragma unroll
                for (int kb = 0; kb < NKD; ++kb)
                    acc = EL::mma(EL::load(&sm.kh[(16 * rt + r) * LDK + 32 * kb], g), sf[kb], acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] *= sm.beta[16 * rt + 4 * g + i];
                X[rt] = acc;
            }
            Frag xf[NKC];
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb) xf[kb] = EL::from_acc(X[2 * kb], X[2 * kb + 1]);

            // Vn = T (beta X)
            f32x4 Vn[NRT];
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb <= rt / 2; ++kb)
                    acc = EL::mma(EL::load(&sm.tb[(16 * rt + r) * LDC + 32 * kb], g), xf[kb], acc);
                Vn[rt] = acc;
            }
            Frag vf[NKC];
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb) vf[kb] = EL::from_acc(Vn[2 * kb], Vn[2 * kb + 1]);

            // O = Qh S + P Vn
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
                f32x4 acc = zero4();
#pragma unroll
                for (int kb = 0; kb < NKD; ++kb)
                    acc = EL::mma(EL::load(&sm.qh[(16 * rt + r) * LDK + 32 * kb], g), sf[kb], acc);
#pragma unroll
                for (int kb = 0; kb <= rt / 2; ++kb)
                    acc = EL::mma(EL::load(&sm.p[(16 * rt + r) * LDC + 32 * kb], g), vf[kb], acc);
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.os[(16 * rt + 4 * g + i) * LDV + vc] = EL::from_f(acc[i]);
            }

            // S <- diag(gamma) S + Kb^T Vn
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                f32x4 acc = S[ct];
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] *= sm.gam[16 * ct + 4 * g + i];
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb)
                    acc = EL::mma(EL::load(&sm.kbt[(16 * ct + r) * LDC + 32 * kb], g), vf[kb], acc);
                S[ct] = acc;
            }
        }
        __syncthreads();                                             // B7

        // ---- phase 4: coalesced store of the output tile ------------------------
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int piece = tid + i * kThreads;
            const int row = piece / VPR, part = piece % VPR;
            if (row < nrow)
                *reinterpret_cast<uint4*>(out + ((t0 + row) * H + h) * DV + col0 + part * (16 / sizeof(E))) =
                    *reinterpret_cast<const uint4*>(&sm.os[row * LDV + part * (16 / sizeof(E))]);
        }
    }

    // ---- final state: rows = key channels, this wave's 16 columns -----------------
    if (final_state) {
        float* fs = final_state + ((int64_t(n) * H + h) * DK) * DV + col0 + 16 * wave + r;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) fs[int64_t(16 * ct + 4 * g + i) * DV] = S[ct][i];
    }
}

template <typename E, int DK, int C>
hipError_t launch_t(const LaunchArgs& a)
{
    const int nvt = a.d_v / kBV;
    const int units = a.num_seqs * a.num_heads;
    const int groups = (units + 7) / 8;
    const dim3 grid(groups * 8 * nvt), block(kThreads);
    const size_t shmem = sizeof(Smem<E, DK, C>);
    auto kern = kda_fwd_kernel<E, DK, C>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(shmem));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, block, shmem, a.stream,
                       static_cast<const E*>(a.q), static_cast<const E*>(a.k), static_cast<const E*>(a.v),
                       static_cast<const E*>(a.log_alpha), static_cast<const E*>(a.beta), a.cu_seqlens,
                       static_cast<E*>(a.out), a.final_state, a.num_seqs, a.num_heads, a.d_v);
    return hipGetLastError();
}

}  // namespace

size_t smem_bytes(int dtype_bf16, int d_k)
{
    if (dtype_bf16) return d_k == 128 ? sizeof(Smem<uint16_t, 128, 64>) : sizeof(Smem<uint16_t, 64, 64>);
    return d_k == 128 ? sizeof(Smem<float, 128, 32>) : sizeof(Smem<float, 64, 32>);
}

hipError_t launch_forward(const LaunchArgs& a)
{
    if (a.dtype_bf16) {
        if (a.d_k == 128) return launch_t<uint16_t, 128, 64>(a);
        return launch_t<uint16_t, 64, 64>(a);
    }
    if (a.d_k == 128) return launch_t<float, 128, 32>(a);
    return launch_t<float, 64, 32>(a);
}

}  // namespace kda
