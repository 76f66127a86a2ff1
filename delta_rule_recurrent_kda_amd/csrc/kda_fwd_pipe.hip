// kda_fwd_pipe.hip -- software-pipelined chunkwise KDA forward scan for bf16 data (gfx950).
//
// Same recurrence and chunkwise form as the sequential kernel in kda_fwd.hip
// (Chimera, arXiv 2607.28611: update printed in the explainer page, "One stream,
// three mechanisms, no positions"; reset and definitions in the paper's Sec. 3
// KDA paragraph). Chunks are C = 32 tokens.
//
// Workgroup: 8 wave64s (two per SIMD) for one (sample, head, 64-column value tile).
// Iteration i overlaps three streams of work through two barrier-separated
// segments, with every per-chunk LDS operand double-buffered (slot i & 1):
//   waves 0-3 ("chain", 16 value columns each, fp32 state in registers):
//       segment 1: X = V - Kh S and O = Qh S for chunk i
//       segment 2: (I + A) Vn = diag(b) X, O += P Vn, S <- diag(gamma) S + Kb^T Vn
//   waves 4-6: segment 1: P and A tiles of chunk i on MFMA, the inverses of the
//       two diagonal 16x16 blocks of I + A
//   all waves: segment 1: raw q, k, log a of chunk i+1 to LDS, its exact q.k
//       diagonal, the output store of chunk i-1; segment 2: the cumulative log
//       decay of chunk i+1 as one MFMA product with a triangular ones matrix,
//       the decay factors and the decayed operands of chunk i+1.
// Global loads run one chunk ahead of the elementwise work.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_device.h"
#include "kda_internal.h"

#ifndef KDA_PHASE_DECL
#define KDA_PHASE_DECL
#define KDA_PHASE_MARK(i) ((void)0)
#define KDA_PHASE_FLUSH
#endif

namespace kda {
namespace {
using namespace dev;

constexpr int kPThreads = 512;   // 8 wave64
constexpr int kPC = 32;          // chunk rows
constexpr int kPBV = 64;         // value columns per workgroup
constexpr uint16_t kBf16One = 0x3F80;

// N bf16 values held as 2N bytes
template <int N> struct BfVec;
template <> struct BfVec<8> {
    using T = uint4;
    __device__ static void unpack(const T& v, float (&f)[8]) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[2 * j] = __uint_as_float(w[j] << 16);
            f[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
    }
    // raw bits to an LDS row that is 8-byte aligned
    __device__ static void put(uint16_t* dst, const T& v) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(v.x, v.y);
        *reinterpret_cast<uint2*>(dst + 4) = make_uint2(v.z, v.w);
    }
};
template <> struct BfVec<4> {
    using T = uint2;
    __device__ static void unpack(const T& v, float (&f)[4]) {
        f[0] = __uint_as_float(v.x << 16);
        f[1] = __uint_as_float(v.x & 0xFFFF0000u);
        f[2] = __uint_as_float(v.y << 16);
        f[3] = __uint_as_float(v.y & 0xFFFF0000u);
    }
    __device__ static void put(uint16_t* dst, const T& v) { *reinterpret_cast<uint2*>(dst) = v; }
};

template <int DK> struct PipeSlot {
    static constexpr int LDK = DK + 4;        // [C][DK] tiles, 8-byte aligned rows
    static constexpr int LDC = kPC + 4;       // [*][C] tiles
    static constexpr int LDV = kPBV + 8;      // V / O staging, 16-byte rows
    static constexpr int LDT = 16 + 4;        // 16-wide blocks
    alignas(16) uint16_t qh[kPC * LDK];       // Qh, hi part
    alignas(16) uint16_t kh[kPC * LDK];       // -Kh
    alignas(16) uint16_t kc[kPC * LDK];       // Kc, hi part
    alignas(16) uint16_t qlo[kPC * LDK];      // Qh, lo part
    alignas(16) uint16_t kclo[kPC * LDK];     // Kc, lo part
    alignas(16) uint16_t kbt[DK * LDC];       // Kb^T, key channel major
    alignas(16) uint16_t p[kPC * LDC];        // LowerIncl(Qh Kc^T)
    alignas(16) uint16_t ab[kPC * LDC];       // -A, block (1,0) only
    alignas(16) uint16_t tbb[kPC * LDT];      // inverses of the diagonal blocks of I + A
    alignas(16) uint16_t vo[kPC * LDV];       // V tile, then the O tile of the same chunk
    alignas(16) float gam[DK];
    alignas(16) float beta[kPC];
    alignas(16) float diag[kPC];
};

template <int DK> struct PipeSmem {
    static constexpr int LDR = DK + 4;        // raw rows, 8-byte aligned
    PipeSlot<DK> slot[2];
    alignas(16) uint16_t graw[kPC * LDR];     // raw log a of the chunk being prepared
    alignas(16) uint16_t qraw[kPC * LDR];
    alignas(16) uint16_t kraw[kPC * LDR];
    alignas(16) float a16[kPC * 20];          // diagonal blocks of A (fp32)
};

template <int DK>
__global__ __launch_bounds__(kPThreads) void kda_fwd_pipe_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ la, const uint16_t* __restrict__ beta, const int32_t* __restrict__ cu,
    uint16_t* __restrict__ out, float* __restrict__ final_state, const float* __restrict__ init_state,
    int num_seqs, int H, int DV)
{
    using EL = Elt<uint16_t>;
    using Frag = EL::Frag;
    using Slot = PipeSlot<DK>;
    constexpr int C = kPC;
    constexpr int NKD = DK / 32;                 // k-blocks over key channels
    constexpr int NCT = DK / 16;                 // 16-row tiles over key channels
    constexpr int VE = DK / 16;                  // channels per thread when loading a row
    constexpr int NV = DK / VE;                  // 16 threads per chunk row
    constexpr int LDK = Slot::LDK, LDC = Slot::LDC, LDV = Slot::LDV, LDT = Slot::LDT;
    constexpr int LDR = PipeSmem<DK>::LDR;
    constexpr int VPR = kPBV * 2 / 16;           // 16-byte pieces per V row
    constexpr int NVP = C * VPR;                 // V pieces per chunk
    constexpr int TPW = 2 * NCT / 8;             // cumsum output tiles per wave: 2 (d_k 128) or 1
    using BV = BfVec<VE>;
    using Vec = typename BV::T;
    static_assert(C * NV == kPThreads, "one chunk row vector per thread");
    static_assert(NVP <= kPThreads, "V tile split");
    static_assert(TPW == 1 || TPW == 2, "cumsum tile split");

    extern __shared__ __align__(16) unsigned char smem_raw[];
    PipeSmem<DK>& sm = *reinterpret_cast<PipeSmem<DK>*>(smem_raw);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const int vcol = tid % NV, row = tid / NV;   // row-vector mapping: one row, VE channels

    // the value tiles of one (sample, head) are 8 blocks apart: same XCD, shared L2
    const int nvt = DV / kPBV;
    const int b = blockIdx.x;
    const int vt = (b >> 3) % nvt;
    const int unit = (b / (8 * nvt)) * 8 + (b & 7);
    if (unit >= num_seqs * H) return;
    const int n = unit / H, h = unit % H;
    const int64_t seq0 = cu[n];
    const int64_t len = int64_t(cu[n + 1]) - seq0;
    const int nchunks = int((len + C - 1) / C);
    const int col0 = vt * kPBV;

    // tiles above the diagonal of P are never written
    for (int i = tid; i < C * LDC; i += kPThreads) {
        sm.slot[0].p[i] = 0; sm.slot[1].p[i] = 0;
        sm.slot[0].ab[i] = 0; sm.slot[1].ab[i] = 0;
    }

    // the state, in waves 0-3 (16 value columns each): zero at the start of the sample, or
    // the given state, in the layout of the final_state write below
    f32x4 S[NCT];
    if (init_state && wave < 4) {
        const float* is = init_state + ((int64_t(n) * H + h) * DK) * DV + col0 + 16 * wave + r;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[ct][i] = is[int64_t(16 * ct + 4 * g + i) * DV];
    } else {
#pragma unroll
        for (int i = 0; i < NCT; ++i) S[i] = zero4();
    }

    // ---- raw loads, one chunk ahead ---------------------------------------------
    // One register set: the rows of chunk c+1 are loaded at the end of the
    // iteration that used those of chunk c, so they are never copied (a copy of
    // registers with loads in flight waits for the data) and their latency hides
    // behind the next segment's MFMA work. Loads are issued unconditionally from a
    // clamped, valid address (rows past the sample's end and chunks past the last
    // one re-read a valid row) and masked where they are consumed.
    struct Raw { Vec q, k, g; uint4 v; uint16_t b; };
    Raw cur;
    auto load_chunk = [&](Raw& dst, int c) {
        c = min(c, nchunks - 1);
        const int64_t t0 = seq0 + int64_t(c) * C;
        const int last = int(min<int64_t>(C, len - int64_t(c) * C)) - 1;
        const int64_t off = ((t0 + min(row, last)) * H + h) * DK + vcol * VE;
        dst.q = *reinterpret_cast<const Vec*>(q + off);
        dst.k = *reinterpret_cast<const Vec*>(k + off);
        dst.g = *reinterpret_cast<const Vec*>(la + off);
        const int vr = min((tid % NVP) / VPR, last), part = tid % VPR;
        dst.v = *reinterpret_cast<const uint4*>(v + ((t0 + vr) * H + h) * DV + col0 + part * 8);
        dst.b = beta[(t0 + min(tid % C, last)) * H + h];
    };
    // rows of chunk c that exist
    auto rows_of = [&](int c) { return int(min<int64_t>(C, len - int64_t(c) * C)); };
    auto store_out = [&](int c) {                // O tile of chunk c from its slot
        const int64_t t0 = seq0 + int64_t(c) * C;
        const int nrow = int(min<int64_t>(C, len - int64_t(c) * C));
        if (tid < NVP) {
            const int vr = tid / VPR, part = tid % VPR;
            if (vr < nrow)
                *reinterpret_cast<uint4*>(out + ((t0 + vr) * H + h) * DV + col0 + part * 8) =
                    *reinterpret_cast<const uint4*>(&sm.slot[c & 1].vo[vr * LDV + part * 8]);
        }
    };

    if (nchunks > 0) load_chunk(cur, 0);
    KDA_PHASE_DECL

    // cumsum tiles of this wave (transposed: channels along the accumulator rows)
    const int cct = (TPW == 2) ? wave : (wave & 3);          // channel tile
    const int crt = (TPW == 2) ? 0 : (wave >> 2);            // first row tile
    // B operand of the cumsum: L^T[k][n] = (k <= n) for row tile rt, in the k map
    Frag lt[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        uint32_t e[8];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) e[4 * t + i] = (16 * t + 4 * g + i <= 16 * rt + r) ? kBf16One : 0u;
        lt[rt].u = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16));
    }

    f32x4 X[2], O[2];
    for (int it = -1; it < nchunks; ++it) {
        const int nx = it + 1;
        Slot& sc = sm.slot[it & 1];              // chunk it (valid when it >= 0)
        Slot& sn = sm.slot[nx & 1];              // chunk it + 1

        // =========================== segment 1 =====================================
        if (it >= 1) store_out(it - 1);          // slot (it-1)&1 == nx&1, refilled in segment 2
        KDA_PHASE_MARK(4);

        if (it >= 0) {
            if (wave >= 4) {
                const int wp = wave - 4;
                if (wp < 3) {
                    // ---- P and A tiles of chunk it, computed transposed (Kc rows as the A
                    //      operand) so that each lane writes four consecutive columns ----
                    const int ti = (wp == 0) ? 0 : 1, tj = (wp == 1) ? 1 : 0;   // (0,0) (1,1) (1,0)
                    f32x4 accP = zero4(), accL = zero4(), accA = zero4();
                    Frag f[2][5];
                    auto ld = [&](Frag (&d)[5], int kb) {
                        d[0] = EL::load(&sc.kc[(16 * tj + r) * LDK + 32 * kb], g);
                        d[1] = EL::load(&sc.qh[(16 * ti + r) * LDK + 32 * kb], g);
                        d[2] = EL::load(&sc.kh[(16 * ti + r) * LDK + 32 * kb], g);
                        d[3] = EL::load(&sc.kclo[(16 * tj + r) * LDK + 32 * kb], g);
                        d[4] = EL::load(&sc.qlo[(16 * ti + r) * LDK + 32 * kb], g);
                    };
                    ld(f[0], 0);
#pragma unroll
                    for (int kb = 0; kb < NKD; ++kb) {
                        if (kb + 1 < NKD) ld(f[(kb + 1) & 1], kb + 1);
                        const Frag (&c5)[5] = f[kb & 1];
                        accP = EL::mma(c5[0], c5[1], accP);
                        accA = EL::mma(c5[0], c5[2], accA);
                        accL = EL::mma(c5[3], c5[1], accL);
                        accL = EL::mma(c5[0], c5[4], accL);
                    }
                    // element i is entry [16ti + r][16tj + 4g + i]
                    const int irow = 16 * ti + r;
                    const float bi = sc.beta[irow];
                    f32x4 pv, av;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int jcol = 16 * tj + 4 * g + i;
                        pv[i] = (jcol < irow) ? accP[i] + accL[i] : (jcol == irow ? sc.diag[irow] : 0.f);
                        av[i] = bi * accA[i];                    // kh holds -Kh: this is -A
                    }
                    EL::store4(&sc.p[irow * LDC + 16 * tj + 4 * g], pv);
                    if (ti != tj) {
                        EL::store4(&sc.ab[irow * LDC + 16 * tj + 4 * g], av);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) av[i] = (4 * g + i < r) ? -av[i] : 0.f;
                        *reinterpret_cast<float4*>(&sm.a16[irow * LDT + 4 * g]) =
                            make_float4(av[0], av[1], av[2], av[3]);
                    }
                    KDA_PHASE_MARK(5);
                    if (wp < 2) {
                        // (I + A_bb)^{-1} by substitution; the strictly lower block is
                        // read into registers first, lane j%16 builds column j, lanes
                        // 0..15 store
                        const float* ablk = &sm.a16[wp * 16 * LDT];
                        float a[16][16];
#pragma unroll
                        for (int i = 1; i < 16; ++i)
#pragma unroll
                            for (int m = 0; m < i; m += 4) {
                                const float4 a4 = *reinterpret_cast<const float4*>(&ablk[i * LDT + m]);
                                a[i][m] = a4.x; a[i][m + 1] = a4.y; a[i][m + 2] = a4.z; a[i][m + 3] = a4.w;
                            }
                        const int j = lane & 15;
                        float t[16];
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            float s0 = (i == j) ? 1.f : 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
                            for (int m = 0; m < i; m += 4) {
                                s0 -= a[i][m] * t[m];
                                if (m + 1 < i) s1 -= a[i][m + 1] * t[m + 1];
                                if (m + 2 < i) s2 -= a[i][m + 2] * t[m + 2];
                                if (m + 3 < i) s3 -= a[i][m + 3] * t[m + 3];
                            }
                            t[i] = (s0 + s1) + (s2 + s3);
                        }
                        if (lane < 16) {
#pragma unroll
                            for (int i = 0; i < 16; ++i) sc.tbb[(16 * wp + i) * LDT + j] = f2bf(t[i]);
                        }
                    }
                }
            } else {
                // ---- chain part 1: X = V - Kh S and O = Qh S --------------------------
                const int vc = 16 * wave + r;
                Frag sf[NKD];
#pragma unroll
                for (int kb = 0; kb < NKD; ++kb) sf[kb] = EL::from_acc(S[2 * kb], S[2 * kb + 1]);
                Frag f[2][4];
                auto ld = [&](Frag (&d)[4], int kb) {
                    d[0] = EL::load(&sc.kh[r * LDK + 32 * kb], g);
                    d[1] = EL::load(&sc.kh[(16 + r) * LDK + 32 * kb], g);
                    d[2] = EL::load(&sc.qh[r * LDK + 32 * kb], g);
                    d[3] = EL::load(&sc.qh[(16 + r) * LDK + 32 * kb], g);
                };
                ld(f[0], 0);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) X[rt][i] = bf2f(sc.vo[(16 * rt + 4 * g + i) * LDV + vc]);
                    O[rt] = zero4();
                }
#pragma unroll
                for (int kb = 0; kb < NKD; ++kb) {
                    if (kb + 1 < NKD) ld(f[(kb + 1) & 1], kb + 1);
                    const Frag (&c4)[4] = f[kb & 1];
                    X[0] = EL::mma(c4[0], sf[kb], X[0]);
                    X[1] = EL::mma(c4[1], sf[kb], X[1]);
                    O[0] = EL::mma(c4[2], sf[kb], O[0]);
                    O[1] = EL::mma(c4[3], sf[kb], O[1]);
                }
            }
        }
        KDA_PHASE_MARK(6);

        if (nx < nchunks) {
            // ---- chunk it+1: raw rows to LDS; exact diagonal q.k ---------------------
            const int nrow = rows_of(nx);
            if (row >= nrow) { cur.q = Vec{}; cur.k = Vec{}; cur.g = Vec{}; }
            BV::put(&sm.graw[row * LDR + vcol * VE], cur.g);
            BV::put(&sm.qraw[row * LDR + vcol * VE], cur.q);
            BV::put(&sm.kraw[row * LDR + vcol * VE], cur.k);
            float qv[VE], kv[VE];
            BV::unpack(cur.q, qv);
            BV::unpack(cur.k, kv);
            float dp = 0.f;
#pragma unroll
            for (int e = 0; e < VE; ++e) dp += qv[e] * kv[e];
#pragma unroll
            for (int m = NV / 2; m >= 1; m >>= 1) dp += __shfl_xor(dp, m);
            if (vcol == 0) sn.diag[row] = dp;
            if (tid < C) sn.beta[tid] = (tid < nrow) ? bf2f(cur.b) : 0.f;
        }
        KDA_PHASE_MARK(0); lds_barrier(); KDA_PHASE_MARK(1);

        // =========================== segment 2 =====================================
        if (it >= 0 && wave < 4) {
            // ---- chain part 2 ---------------------------------------------------------
            const int vc = 16 * wave + r;
            const auto t0f = EL::load16(&sc.tbb[r * LDT], g);
            const auto t1f = EL::load16(&sc.tbb[(16 + r) * LDT], g);
            const auto a10 = EL::load16(&sc.ab[(16 + r) * LDC], g);
            const Frag p0 = EL::load(&sc.p[r * LDC], g);
            const Frag p1 = EL::load(&sc.p[(16 + r) * LDC], g);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const float4 b4 = *reinterpret_cast<const float4*>(&sc.beta[16 * rt + 4 * g]);
                X[rt][0] *= b4.x; X[rt][1] *= b4.y; X[rt][2] *= b4.z; X[rt][3] *= b4.w;
            }
            // (I + A) Vn = diag(b) X with the 16x16 blocks of I + A
            const f32x4 vn0 = EL::mma16(t0f, EL::from_acc16(X[0]), zero4());
            const f32x4 y1 = EL::mma16(a10, EL::from_acc16(vn0), X[1]);
            const f32x4 vn1 = EL::mma16(t1f, EL::from_acc16(y1), zero4());
            const Frag vf = EL::from_acc(vn0, vn1);
            O[0] = EL::mma(p0, vf, O[0]);
            O[1] = EL::mma(p1, vf, O[1]);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) sc.vo[(16 * rt + 4 * g + i) * LDV + vc] = f2bf(O[rt][i]);
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const float4 g4 = *reinterpret_cast<const float4*>(&sc.gam[16 * ct + 4 * g]);
                S[ct][0] *= g4.x; S[ct][1] *= g4.y; S[ct][2] *= g4.z; S[ct][3] *= g4.w;
                S[ct] = EL::mma(EL::load(&sc.kbt[(16 * ct + r) * LDC], g), vf, S[ct]);
            }
        }
        KDA_PHASE_MARK(8);

        if (nx < nchunks) {
            // ---- chunk it+1: cumulative log decay, decay factors, decayed operands -----
            if (tid < NVP)
                *reinterpret_cast<uint4*>(&sn.vo[(tid / VPR) * LDV + (tid % VPR) * 8]) =
                    (tid / VPR < rows_of(nx)) ? cur.v : make_uint4(0, 0, 0, 0);
            // G^T = g^T L^T: accumulator element i of row tile rt is G[16rt + r][16cct + 4g + i]
            uint32_t ge[8];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) ge[4 * t + i] = sm.graw[(16 * t + 4 * g + i) * LDR + 16 * cct + r];
            Frag fg;
            fg.u = make_uint4(ge[0] | (ge[1] << 16), ge[2] | (ge[3] << 16), ge[4] | (ge[5] << 16), ge[6] | (ge[7] << 16));
            f32x4 Gt[2];
            Gt[0] = EL::mma(fg, lt[0], zero4());
            Gt[1] = EL::mma(fg, lt[1], zero4());
            float gam[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) gam[i] = fast_exp2(__shfl(Gt[1][i], 15 + 16 * g) * kLog2e);
            const int c0 = 16 * cct + 4 * g;
            if (r == 0 && crt == 0)
                *reinterpret_cast<float4*>(&sn.gam[c0]) = make_float4(gam[0], gam[1], gam[2], gam[3]);
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int rt = crt + u;
                const int rw = 16 * rt + r;
                const uint2 q4 = *reinterpret_cast<const uint2*>(&sm.qraw[rw * LDR + c0]);
                const uint2 k4 = *reinterpret_cast<const uint2*>(&sm.kraw[rw * LDR + c0]);
                const float qv[4] = {__uint_as_float(q4.x << 16), __uint_as_float(q4.x & 0xFFFF0000u),
                                     __uint_as_float(q4.y << 16), __uint_as_float(q4.y & 0xFFFF0000u)};
                const float kv[4] = {__uint_as_float(k4.x << 16), __uint_as_float(k4.x & 0xFFFF0000u),
                                     __uint_as_float(k4.y << 16), __uint_as_float(k4.y & 0xFFFF0000u)};
                const f32x4 Gr = (TPW == 2) ? (u == 0 ? Gt[0] : Gt[1]) : (crt == 0 ? Gt[0] : Gt[1]);
                f32x4 fq, fkh, fkc, lq, lk;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float G2 = Gr[i] * kLog2e;
                    const float ex = fast_exp2(G2), ei = fast_exp2(-G2);
                    fq[i] = qv[i] * ex;
                    fkh[i] = -(kv[i] * ex);
                    fkc[i] = kv[i] * ei;
                    lq[i] = fq[i] - bf2f(f2bf(fq[i]));
                    lk[i] = fkc[i] - bf2f(f2bf(fkc[i]));
                    sn.kbt[(c0 + i) * LDC + rw] = f2bf(fkc[i] * gam[i]);
                }
                EL::store4(&sn.qh[rw * LDK + c0], fq);
                EL::store4(&sn.kh[rw * LDK + c0], fkh);
                EL::store4(&sn.kc[rw * LDK + c0], fkc);
                EL::store4(&sn.qlo[rw * LDK + c0], lq);
                EL::store4(&sn.kclo[rw * LDK + c0], lk);
            }
            KDA_PHASE_MARK(9);
            load_chunk(cur, nx + 1);
        }
        KDA_PHASE_MARK(2); lds_barrier(); KDA_PHASE_MARK(3);
    }
    if (nchunks > 0) store_out(nchunks - 1);
    KDA_PHASE_MARK(15);
    KDA_PHASE_FLUSH

    if (final_state && wave < 4) {
        float* fs = final_state + ((int64_t(n) * H + h) * DK) * DV + col0 + 16 * wave + r;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) fs[int64_t(16 * ct + 4 * g + i) * DV] = S[ct][i];
    }
}

template <int DK>
hipError_t launch_pipe(const LaunchArgs& a)
{
    const int nvt = a.d_v / kPBV;
    const int units = a.num_seqs * a.num_heads;
    const int groups = (units + 7) / 8;
    const dim3 grid(groups * 8 * nvt), block(kPThreads);
    const size_t shmem = sizeof(PipeSmem<DK>);
    auto kern = kda_fwd_pipe_kernel<DK>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(shmem));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, block, shmem, a.stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.log_alpha),
                       static_cast<const uint16_t*>(a.beta), a.cu_seqlens, static_cast<uint16_t*>(a.out),
                       a.final_state, a.init_state, a.num_seqs, a.num_heads, a.d_v);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_pipe(const LaunchArgs& a)
{
    return a.d_k == 128 ? launch_pipe<128>(a) : launch_pipe<64>(a);
}

size_t smem_bytes_pipe(int d_k)
{
    return d_k == 128 ? sizeof(PipeSmem<128>) : sizeof(PipeSmem<64>);
}

}  // namespace kda
