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
//     Qh = Q*exp(G)   Kh = K*exp(G)   Kc = K*exp(-G)   Kb = gamma*Kc
//     A  = StrictLower(diag(b) Kh Kc^T)                               (UT transform)
//     X  = V - Kh S,   (I + A) Vn = diag(b) X   (rows of Vn are the delta-rule innovations)
//     O  = Qh S + LowerIncl(Qh Kc^T) Vn,   S <- diag(gamma) S + Kb^T Vn
// (I + A) Vn = diag(b) X is solved by blocks of 16 rows: the 16x16 diagonal blocks
// of (I + A) are inverted by substitution in fp32, the off-diagonal blocks enter
// as products with the already solved rows.
// The diagonal of Qh Kc^T equals q_t . k_t exactly and is taken in fp32 from the
// stored inputs. With bf16 data Qh Kc^T is formed from hi/lo bf16 pairs
// (hi*hi + lo*hi + hi*lo): rows whose output is a near-cancelling sum of a few
// such products (the first tokens of a sample) would otherwise carry the full
// bf16 operand error relative to a small result.
//
// Mapping: one workgroup of 4 wave64s per (sample, head, 64-column value tile).
// Every wave owns 16 value columns of the state for the whole scan (S is fp32 in
// registers, DK x 16 per wave), so the only cross-wave traffic is the
// v-independent per-chunk operands staged in LDS. Value columns never mix in the
// recurrence, which is what makes this split exact.
//
// MFMA fragments: all contractions use 16x16 output tiles (v_mfma_f32_16x16x32_bf16
// and _16x16x16_bf16 for bf16 data, v_mfma_f32_16x16x4_f32 for fp32 data). A
// k-block of 32 is held by lane (r = lane%16, g = lane/16) as 8 elements:
// k = 16*t + 4*g + i (t in {0,1}, i in 0..3); a k-block of 16 is the t = 0 half.
// An accumulator tile holds rows 4*g + i, column r, so one or two stacked
// accumulator tiles are directly a B operand (k along their rows) and the A
// operand of their transpose; both operands of every product use the same k map.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_device.h"
#include "kda_internal.h"


namespace kda {
namespace {

using namespace dev;

constexpr int kThreads = 256;   // 4 wave64
constexpr int kBV = 64;         // value columns per workgroup (16 per wave)

// ---------------------------------------------------------------------------
// shared-memory layout
// ---------------------------------------------------------------------------
template <typename E, int DK, int C> struct Smem {
    static constexpr bool kSplit = sizeof(E) == 2;
    static constexpr int LDK = DK + 4;                         // row stride of [C][DK] tiles
    static constexpr int LDC = C + 4;                          // row stride of [*][C] tiles
    static constexpr int LDV = kBV + 16 / sizeof(E);           // V / O staging (16-byte rows)
    static constexpr int LDT = 16 + 4;                         // 16x16 blocks
    static constexpr int NRG = kThreads / (DK / Elt<E>::kVec); // row groups of the elementwise phase
    alignas(16) E qh[C * LDK];            // Qh (hi part for bf16)
    alignas(16) E kh[C * LDK];            // -Kh
    alignas(16) E kc[C * LDK];            // Kc (hi part for bf16)
    alignas(16) E qlo[kSplit ? C * LDK : 4];
    alignas(16) E kclo[kSplit ? C * LDK : 4];
    alignas(16) E kbt[DK * LDC];          // Kb^T (key channel major)
    alignas(16) E p[C * LDC];             // LowerIncl(Qh Kc^T), row-major [i][j]
    alignas(16) E ab[C * LDC];            // -A below the diagonal blocks, row-major
    alignas(16) E tbb[C * LDT];           // inverses of the diagonal 16x16 blocks of I + A
    alignas(16) E vo[C * LDV];            // V tile, then the O tile of the same chunk
    alignas(16) float a16[C * LDT];       // diagonal 16x16 blocks of A (fp32)
    alignas(16) float wtot[4 * DK];       // per-wave sums of log a
    alignas(16) float gam[DK];
    float beta[C];
    float diag[C];
    float qs[C], ks[C];                   // 1/|q_t|, 1/|k_t| when normalising on load
};

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
// NORM: q_t and k_t are divided by their Euclidean length on load (a zero vector
// stays zero), the normalisation fused into the scan kernels that the paper's
// training setup describes.
template <typename E, int DK, int C, bool NORM>
__global__ __launch_bounds__(kThreads) void kda_fwd_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v,
    const E* __restrict__ la, const E* __restrict__ beta, const int32_t* __restrict__ cu,
    E* __restrict__ out, float* __restrict__ final_state, const float* __restrict__ init_state,
    int num_seqs, int H, int DV)
{
    using EL = Elt<E>;
    using Frag = typename EL::Frag;
    using Frag16 = typename EL::Frag16;
    using Vec = typename EL::Vec;
    using S_ = Smem<E, DK, C>;
    constexpr int VE = EL::kVec;            // elements per 16-byte vector
    constexpr int NV = DK / VE;             // vectors per key row
    constexpr int NRG = S_::NRG;            // row groups (threads sharing a vector column)
    constexpr int RPT = C / NRG;            // consecutive chunk rows per thread
    constexpr int NRT = C / 16;             // 16-row tiles per chunk
    constexpr int NKC = C / 32;             // 32-wide k-blocks over chunk rows
    constexpr int NKD = DK / 32;            // 32-wide k-blocks over key channels
    constexpr int NCT = DK / 16;            // 16-row tiles over key channels
    constexpr int VPR = kBV * sizeof(E) / 16;       // 16-byte pieces per V row
    constexpr int VLD = C * VPR / kThreads;         // V pieces per thread
    constexpr int NPAIR = NRT * (NRT + 1) / 2;      // lower 16x16 tiles of a CxC matrix
    constexpr int LDK = S_::LDK, LDC = S_::LDC, LDV = S_::LDV, LDT = S_::LDT;
    static_assert(RPT == 2 || RPT == 4, "elementwise row split");
    static_assert(VLD >= 1 && (C * VPR) % kThreads == 0, "V tile split");
    static_assert(64 % NV == 0, "a row group must sit inside one wave");

    extern __shared__ __align__(16) unsigned char smem_raw[];
    S_& sm = *reinterpret_cast<S_*>(smem_raw);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const int vcol = tid % NV, rg = tid / NV;       // elementwise phase: vector column, row group

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
    const int64_t rstride = int64_t(H) * DK;       // elements between consecutive tokens

    // the blocks of P and -A above the diagonal are never written: clear once
    for (int i = tid; i < C * LDC; i += kThreads) { sm.p[i] = E(0); sm.ab[i] = E(0); }

    // state: wave owns value columns [16*wave, 16*wave+16) of the tile; NCT tiles of 16 key rows,
    // lane (r, g) element i of tile ct = S[16ct + 4g + i][col0 + 16 wave + r]; zero at the start
    // of the sample, or the given state
    f32x4 S[NCT];
    if (init_state) {
        const float* is = init_state + ((int64_t(n) * H + h) * DK) * DV + col0 + 16 * wave + r;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[ct][i] = is[int64_t(16 * ct + 4 * g + i) * DV];
    } else {
#pragma unroll
        for (int i = 0; i < NCT; ++i) S[i] = zero4();
    }

    // ---- raw loads of one chunk into registers --------------------------------
    Vec rq[RPT], rk[RPT], rla[RPT];
    uint4 rv[VLD];
    E rb = E(0);
    // loads are issued unconditionally from a clamped, valid address and masked
    // where they are consumed (a conditional load makes the compiler wait for the
    // data right away)
    auto load_chunk = [&](int c) {
        c = min(c, nchunks - 1);
        const int64_t t0 = seq0 + int64_t(c) * C;
        const int last = int(min<int64_t>(C, len - int64_t(c) * C)) - 1;
        const int64_t base = int64_t(h) * DK + vcol * VE;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int64_t off = (t0 + min(rg * RPT + i, last)) * rstride + base;
            rq[i] = *reinterpret_cast<const Vec*>(q + off);
            rk[i] = *reinterpret_cast<const Vec*>(k + off);
            rla[i] = *reinterpret_cast<const Vec*>(la + off);
        }
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int piece = tid + i * kThreads;
            const int row = min(piece / VPR, last), part = piece % VPR;
            rv[i] = *reinterpret_cast<const uint4*>(v + ((t0 + row) * H + h) * DV + col0 + part * (16 / sizeof(E)));
        }
        rb = beta[(t0 + min(tid % C, last)) * H + h];
    };
    if (nchunks > 0) load_chunk(0);

    for (int c = 0; c < nchunks; ++c) {
        const int64_t t0 = seq0 + int64_t(c) * C;
        const int nrow = int(min<int64_t>(C, len - int64_t(c) * C));

        // rows past the sample's end were loaded from a valid row: zero them
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            if (rg * RPT + i >= nrow) { rq[i] = Vec{}; rk[i] = Vec{}; rla[i] = Vec{}; }
#pragma unroll
        for (int i = 0; i < VLD; ++i)
            if ((tid + i * kThreads) / VPR >= nrow) rv[i] = make_uint4(0, 0, 0, 0);
        if (tid >= nrow) rb = E(0);

        // ---- phase A: sums of log a over row groups and their prefix inside the wave;
        //      exact diagonal q.k ----------------------------------------------------
        float excl[VE];                           // log a summed over earlier rows of this wave
        {
            float tl[VE], inc[VE];
#pragma unroll
            for (int e = 0; e < VE; ++e) tl[e] = 0.f;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                float gv[VE];
                EL::unpack(rla[i], gv);
#pragma unroll
                for (int e = 0; e < VE; ++e) tl[e] += gv[e];
            }
#pragma unroll
            for (int e = 0; e < VE; ++e) inc[e] = tl[e];
#pragma unroll
            for (int sft = NV; sft < 64; sft *= 2) {          // row groups of a wave are NV lanes apart
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    const float o = __shfl_up(inc[e], sft);
                    if (lane >= sft) inc[e] += o;
                }
            }
#pragma unroll
            for (int e = 0; e < VE; ++e) excl[e] = inc[e] - tl[e];
            if (lane >= 64 - NV) {
#pragma unroll
                for (int e = 0; e < VE; e += 4)
                    *reinterpret_cast<float4*>(&sm.wtot[wave * DK + vcol * VE + e]) =
                        make_float4(inc[e], inc[e + 1], inc[e + 2], inc[e + 3]);
            }
            float dp[RPT], qq[RPT], kk[RPT];
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                float qv[VE], kv[VE];
                EL::unpack(rq[i], qv);
                EL::unpack(rk[i], kv);
                float sum = 0.f, sq = 0.f, sk = 0.f;
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    sum += qv[e] * kv[e];
                    sq += qv[e] * qv[e];
                    sk += kv[e] * kv[e];
                }
                dp[i] = sum;
                qq[i] = sq;
                kk[i] = sk;
            }
            float tot = reduce_scatter<RPT, NV / 2>(dp, lane);
            const int drow = rg * RPT + reduce_index<RPT, NV>(lane);
            if constexpr (NORM) {
                const float tq = reduce_scatter<RPT, NV / 2>(qq, lane);
                const float tk = reduce_scatter<RPT, NV / 2>(kk, lane);
                const float qs = tq > 0.f ? 1.f / sqrtf(tq) : 0.f;
                const float ks = tk > 0.f ? 1.f / sqrtf(tk) : 0.f;
                tot *= qs * ks;
                if ((lane & (NV / RPT - 1)) == 0) {
                    sm.qs[drow] = qs;
                    sm.ks[drow] = ks;
                }
            }
            if ((lane & (NV / RPT - 1)) == 0) sm.diag[drow] = tot;
        }
        if (tid < C) sm.beta[tid] = EL::to_f(rb);
        lds_barrier();  // B1

        // ---- phase B: decay factors and decayed operands -------------------------
        // (the V tile goes in only now: the previous chunk's O store read this buffer)
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int piece = tid + i * kThreads;
            *reinterpret_cast<uint4*>(&sm.vo[(piece / VPR) * LDV + (piece % VPR) * (16 / sizeof(E))]) = rv[i];
        }
        {
            float run[VE], gam[VE];
#pragma unroll
            for (int e = 0; e < VE; ++e) { run[e] = excl[e]; gam[e] = 0.f; }
#pragma unroll
            for (int w = 0; w < 4; ++w) {
#pragma unroll
                for (int e = 0; e < VE; e += 4) {
                    const float4 t4 = *reinterpret_cast<const float4*>(&sm.wtot[w * DK + vcol * VE + e]);
                    const float tv[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        gam[e + u] += tv[u];
                        if (w < wave) run[e + u] += tv[u];
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < VE; ++e) gam[e] = fast_exp2(gam[e] * kLog2e);
            if (rg == 0) {
#pragma unroll
                for (int e = 0; e < VE; e += 4)
                    *reinterpret_cast<float4*>(&sm.gam[vcol * VE + e]) =
                        make_float4(gam[e], gam[e + 1], gam[e + 2], gam[e + 3]);
            }
#pragma unroll
            for (int i = 0; i < RPT; i += 2) {
                float kb[VE][2];
#pragma unroll
                for (int ii = 0; ii < 2; ++ii) {
                    const int row = rg * RPT + i + ii;
                    float gv[VE], qv[VE], kv[VE];
                    EL::unpack(rla[i + ii], gv);
                    EL::unpack(rq[i + ii], qv);
                    EL::unpack(rk[i + ii], kv);
                    if constexpr (NORM) {
                        const float qs = sm.qs[row], ks = sm.ks[row];
#pragma unroll
                        for (int e = 0; e < VE; ++e) {
                            qv[e] *= qs;
                            kv[e] *= ks;
                        }
                    }
                    float fq[VE], fkh[VE], fkc[VE];
#pragma unroll
                    for (int e = 0; e < VE; ++e) {
                        run[e] += gv[e];
                        const float G2 = run[e] * kLog2e;
                        const float ex = fast_exp2(G2), ei = fast_exp2(-G2);
                        fq[e] = qv[e] * ex;
                        fkh[e] = -(kv[e] * ex);
                        fkc[e] = kv[e] * ei;
                        kb[e][ii] = fkc[e] * gam[e];
                    }
                    EL::store_vec(&sm.qh[row * LDK + vcol * VE], fq);
                    EL::store_vec(&sm.kh[row * LDK + vcol * VE], fkh);
                    EL::store_vec(&sm.kc[row * LDK + vcol * VE], fkc);
                    if constexpr (S_::kSplit) {
                        float lq[VE], lk[VE];
#pragma unroll
                        for (int e = 0; e < VE; ++e) {
                            lq[e] = fq[e] - bf2f(f2bf(fq[e]));
                            lk[e] = fkc[e] - bf2f(f2bf(fkc[e]));
                        }
                        EL::store_vec(&sm.qlo[row * LDK + vcol * VE], lq);
                        EL::store_vec(&sm.kclo[row * LDK + vcol * VE], lk);
                    }
                }
#pragma unroll
                for (int e = 0; e < VE; ++e)
                    EL::template store_run<2>(&sm.kbt[(vcol * VE + e) * LDC + rg * RPT + i], kb[e]);
            }
        }
        lds_barrier();  // B2

        // ---- phase C: P and A tiles, inverse of this wave's diagonal block of I + A,
        //      and the S-dependent products that need neither -------------------------
        const int vc = 16 * wave + r;                               // column within the value tile
        f32x4 X[NRT], O[NRT];
        {
            // wave w computes the diagonal tile (w, w) and tiles below the diagonal;
            // tiles are computed transposed (Kc rows as the A operand) so that each
            // lane writes four consecutive columns of a row-major result
            int its[3], jts[3];
            bool ok[3];
#pragma unroll
            for (int u = 0; u < 3; ++u) { its[u] = jts[u] = 0; ok[u] = false; }
            if constexpr (NRT == 4) {
                its[0] = jts[0] = wave; ok[0] = true;
                const int t1i[4] = {1, 2, 2, 3}, t1j[4] = {0, 0, 1, 0};
                its[1] = t1i[wave]; jts[1] = t1j[wave]; ok[1] = true;
                its[2] = 3; jts[2] = 2 - wave; ok[2] = wave < 2;       // (3,2) and (3,1)
            } else {
                const int ti[4] = {0, 1, 1, 0}, tj[4] = {0, 1, 0, 0};
                its[0] = ti[wave]; jts[0] = tj[wave]; ok[0] = wave < 3;
            }
            f32x4 accP[3], accA[3];
#pragma unroll
            for (int u = 0; u < 3; ++u) { accP[u] = zero4(); accA[u] = zero4(); }
#pragma unroll
            for (int kb = 0; kb < NKD; ++kb) {
#pragma unroll
                for (int u = 0; u < 3; ++u) {
                    if (ok[u]) {
                        const int it = its[u], jt = jts[u];
                        const Frag fa = EL::load(&sm.kc[(16 * jt + r) * LDK + 32 * kb], g);
                        const Frag fq = EL::load(&sm.qh[(16 * it + r) * LDK + 32 * kb], g);
                        accP[u] = EL::mma(fa, fq, accP[u]);
                        accA[u] = EL::mma(fa, EL::load(&sm.kh[(16 * it + r) * LDK + 32 * kb], g), accA[u]);
                        if constexpr (S_::kSplit) {
                            accP[u] = EL::mma(EL::load(&sm.kclo[(16 * jt + r) * LDK + 32 * kb], g), fq, accP[u]);
                            accP[u] = EL::mma(fa, EL::load(&sm.qlo[(16 * it + r) * LDK + 32 * kb], g), accP[u]);
                        }
                    }
                }
            }
            // accumulator element i of tile (it, jt) is entry [16it + r][16jt + 4g + i]
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                if (ok[u]) {
                    const int it = its[u], jt = jts[u];
                    const int irow = 16 * it + r;
                    const float bi = sm.beta[irow];
                    f32x4 pv, av;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int jcol = 16 * jt + 4 * g + i;
                        pv[i] = (jcol < irow) ? accP[u][i] : (jcol == irow ? sm.diag[irow] : 0.f);
                        av[i] = bi * accA[u][i];            // kh holds -Kh: this is -A
                    }
                    EL::store4(&sm.p[irow * LDC + 16 * jt + 4 * g], pv);
                    if (jt < it) {
                        EL::store4(&sm.ab[irow * LDC + 16 * jt + 4 * g], av);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) av[i] = (4 * g + i < r) ? -av[i] : 0.f;
                        *reinterpret_cast<float4*>(&sm.a16[irow * LDT + 4 * g]) =
                            make_float4(av[0], av[1], av[2], av[3]);
                    }
                }
            }

            // X = V - Kh S and O = Qh S
            Frag sf[NKD];
#pragma unroll
            for (int kb = 0; kb < NKD; ++kb) sf[kb] = EL::from_acc(S[2 * kb], S[2 * kb + 1]);
#pragma unroll
            for (int kb = 0; kb < NKD; kb += 2) EL::ready(sf[kb], sf[kb + 1]);
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) X[rt][i] = EL::to_f(sm.vo[(16 * rt + 4 * g + i) * LDV + vc]);
                O[rt] = zero4();
            }
#pragma unroll
            for (int kb = 0; kb < NKD; ++kb) {
#pragma unroll
                for (int rt = 0; rt < NRT; ++rt) {
                    X[rt] = EL::mma(EL::load(&sm.kh[(16 * rt + r) * LDK + 32 * kb], g), sf[kb], X[rt]);
                    O[rt] = EL::mma(EL::load(&sm.qh[(16 * rt + r) * LDK + 32 * kb], g), sf[kb], O[rt]);
                }
            }

            // (I + A_ww)^{-1} for this wave's diagonal block by substitution: lane j%16
            // builds column j; every lane computes so the work can interleave with the
            // products above, lanes 0..15 store
            if (NRT == 4 || wave < NRT) {
                const float* ablk = &sm.a16[wave * 16 * LDT];
                const int j = lane & 15;
                float t[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float s0 = (i == j) ? 1.f : 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
                    for (int m = 0; m < i; m += 4) {
                        s0 -= ablk[i * LDT + m] * t[m];
                        if (m + 1 < i) s1 -= ablk[i * LDT + m + 1] * t[m + 1];
                        if (m + 2 < i) s2 -= ablk[i * LDT + m + 2] * t[m + 2];
                        if (m + 3 < i) s3 -= ablk[i * LDT + m + 3] * t[m + 3];
                    }
                    t[i] = (s0 + s1) + (s2 + s3);
                }
                if (lane < 16) {
                    E* dst = &sm.tbb[wave * 16 * LDT + j];
#pragma unroll
                    for (int i = 0; i < 16; ++i) dst[i * LDT] = EL::from_f(t[i]);
                }
            }
        }
        lds_barrier();  // B3

        // ---- phase E: innovations, output, state update ----------------------------
        // prefetch the next chunk while this one finishes
        load_chunk(c + 1);
        {
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) X[rt][i] *= sm.beta[16 * rt + 4 * g + i];
            // (I + A) Vn = diag(b) X by blocks of 16 rows
            f32x4 Vn[NRT];
#pragma unroll
            for (int bb = 0; bb < NRT; ++bb) {
                f32x4 acc = X[bb];
#pragma unroll
                for (int kb = 0; kb < bb / 2; ++kb) {
                    Frag vb = EL::from_acc(Vn[2 * kb], Vn[2 * kb + 1]);
                    EL::ready(vb);
                    acc = EL::mma(EL::load(&sm.ab[(16 * bb + r) * LDC + 32 * kb], g), vb, acc);
                }
                if (bb & 1) {
                    Frag16 vb = EL::from_acc16(Vn[bb - 1]);
                    EL::ready(vb);
                    acc = EL::mma16(EL::load16(&sm.ab[(16 * bb + r) * LDC + 16 * (bb - 1)], g), vb, acc);
                }
                Frag16 pa = EL::from_acc16(acc);
                EL::ready(pa);
                Vn[bb] = EL::mma16(EL::load16(&sm.tbb[(16 * bb + r) * LDT], g), pa, zero4());
            }
            Frag vf[NKC];
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb) vf[kb] = EL::from_acc(Vn[2 * kb], Vn[2 * kb + 1]);
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb) EL::ready(vf[kb]);

            // O += P Vn, to the staging tile
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb)
#pragma unroll
                for (int rt = 2 * kb; rt < NRT; ++rt)
                    O[rt] = EL::mma(EL::load(&sm.p[(16 * rt + r) * LDC + 32 * kb], g), vf[kb], O[rt]);
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.vo[(16 * rt + 4 * g + i) * LDV + vc] = EL::from_f(O[rt][i]);

            // S <- diag(gamma) S + Kb^T Vn
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[ct][i] *= sm.gam[16 * ct + 4 * g + i];
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb)
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct)
                    S[ct] = EL::mma(EL::load(&sm.kbt[(16 * ct + r) * LDC + 32 * kb], g), vf[kb], S[ct]);
        }
        lds_barrier();  // B4

        // ---- phase F: coalesced store of the output tile ---------------------------
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int piece = tid + i * kThreads;
            const int row = piece / VPR, part = piece % VPR;
            if (row < nrow)
                *reinterpret_cast<uint4*>(out + ((t0 + row) * H + h) * DV + col0 + part * (16 / sizeof(E))) =
                    *reinterpret_cast<const uint4*>(&sm.vo[row * LDV + part * (16 / sizeof(E))]);
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
    auto kern = a.qk_l2norm ? kda_fwd_kernel<E, DK, C, true> : kda_fwd_kernel<E, DK, C, false>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(shmem));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, block, shmem, a.stream,
                       static_cast<const E*>(a.q), static_cast<const E*>(a.k), static_cast<const E*>(a.v),
                       static_cast<const E*>(a.log_alpha), static_cast<const E*>(a.beta), a.cu_seqlens,
                       static_cast<E*>(a.out), a.final_state, a.init_state, a.num_seqs, a.num_heads, a.d_v);
    return hipGetLastError();
}

}  // namespace

size_t smem_bytes(int dtype_bf16, int d_k)
{
    if (dtype_bf16) return d_k == 128 ? sizeof(Smem<uint16_t, 128, 64>) : sizeof(Smem<uint16_t, 64, 64>);
    return d_k == 128 ? sizeof(Smem<float, 128, 32>) : sizeof(Smem<float, 64, 32>);
}

hipError_t launch_forward_seq(const LaunchArgs& a)
{
    if (a.dtype_bf16) {
        if (a.d_k == 128) return launch_t<uint16_t, 128, 64>(a);
        return launch_t<uint16_t, 64, 64>(a);
    }
    if (a.d_k == 128) return launch_t<float, 128, 32>(a);
    return launch_t<float, 64, 32>(a);
}

}  // namespace kda
