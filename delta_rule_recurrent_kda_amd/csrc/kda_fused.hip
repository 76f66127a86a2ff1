// kda_fused.hip -- single-pass chunkwise KDA forward for bf16 data, d_k = d_v = 128 (gfx950).
//
// Recurrence (Chimera, arXiv 2607.28611: update printed in the explainer page, "One
// stream, three mechanisms, no positions"; state reset at every packed sample, paper
// Sec. 3 KDA paragraph), per (sample, head):
//     S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,   o_t = S_t^T q_t.
// Chunkwise form over chunks of C = 32 tokens (G = inclusive cumsum of log a over the
// chunk's rows, per key channel; gamma = exp(G of the last row)):
//     Qh = Q e^G, Kh = K e^G, Kc = K e^-G, Kb = gamma Kc
//     A = StrictLower(diag(b) Kh Kc^T),  T = (I + A)^-1,  W = T diag(b) Kh,  U = T diag(b) V
//     Vn = U - W S,  O = Qh S + LowerIncl(Qh Kc^T) Vn,  S <- diag(gamma) S + Kb^T Vn
//
// One workgroup of 8 wave64s owns one (sample segment, head) and all 128 value columns,
// so every S-independent operand of a chunk is computed once, on the CU, from the raw
// inputs, and never leaves it: the kernel reads q, k, v, log a, beta once and writes the
// output once. Per chunk the eight waves run, between workgroup barriers:
//   E  wave w owns token tile w & 1 and channel slab w >> 1 (32 channels): the chunk-local
//      cumulative decay G as one product with a triangular ones matrix, e^{+-G}, Qh and Kc
//      as hi/lo bf16 pairs, Kh, partial q.k sums, gamma; all to LDS.
//   2  waves 0-2: the three 16x16 blocks of A, the two diagonal ones inverted exactly on
//      fp32 MFMA (nilpotent product); waves 3-5: the three blocks of P = LowerIncl(Qh Kc^T)
//      from the hi/lo pairs with the exact q.k diagonal; every wave w: the right-hand sides
//      diag(b) Kh of key tile w and diag(b) V of value tile w, and the Kb^T tile of key
//      channels 16w..16w+15.
//   3  every wave solves (I + A) X = Y by 16-row blocks for its key tile (-W, to LDS) and
//      its value tile (U, kept in registers for the chain).
//   C  wave w carries the 16 value columns 16w..16w+15 of S (fp32 in registers) through
//      the chunk: Vn = U - W S, O^T = S^T Qh^T + Vn^T P^T, S <- diag(gamma) S + Kb^T Vn.
// The next chunk's raw rows are loaded into registers while the current chunk runs. Two
// workgroups share a CU (57.5 KB of LDS each), so one's barriers and dependent products
// overlap the other's.
//
// Long samples (few (sample, head) units for the CUs): the sample is cut into segments.
//   pass 1  per segment that is not its sample's last: the state reached from zero
//           (S_loc) and the segment's transition Phi (the same chunk pass on a d_k-column
//           state started at the identity with U taken as zero), no output;
//   combine per (sample, head, 16 value columns): S_in(k+1) = Phi(k) S_in(k) + S_loc(k)
//           from the sample's initial state, with hi/lo bf16 operands;
//   pass 2  every segment from its S_in with outputs; the last one writes final_state.
//
// Fragment conventions are those of kda_device.h: an accumulator tile (rows 4g+i,
// column r) is the B operand of the same matrix and the A operand of its transpose, and a
// product with the identity as B operand transposes a bf16 tile exactly.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {
using namespace dev;

constexpr int kFC = 32;            // tokens per chunk
constexpr int kFD = 128;           // d_k = d_v
constexpr int kFThreads = 512;     // 8 wave64
constexpr int kLDK = kFD + 8;      // token-row stride of the LDS tiles (272 bytes)
constexpr uint16_t kOneBf = 0x3F80;
constexpr int kCombThreads = 256;  // combine: 4 wave64 per (sample, head, 16 value columns)

struct FusedSmem {
    alignas(16) uint16_t kh[kFC * kLDK];    // Kh (token rows); after the solve, -W
    alignas(16) uint16_t kch[kFC * kLDK];   // Kc, hi part
    alignas(16) uint16_t kcl[kFC * kLDK];   // Kc, lo part
    alignas(16) uint16_t qh[kFC * kLDK];    // Qh, hi part
    alignas(16) uint16_t ql[kFC * kLDK];    // Qh, lo part
    alignas(16) uint4 kbt[8 * 64];          // Kb^T A fragments [key tile][lane]
    alignas(16) uint4 pf[2 * 64];           // P^T B fragments [token tile][lane]
    alignas(16) uint2 tinv[2 * 64];         // (I + A_ii)^-1 as 16x16x16 A fragments
    alignas(16) uint2 na10[64];             // -A_10 as a 16x16x16 A fragment
    alignas(16) float gam[kFD];
    alignas(16) float beta[kFC];
    alignas(16) float dpp[4 * kFC];         // partial q.k per 32-channel slab
    alignas(16) float ssq[2 * 4 * kFC];     // partial sums of squares of q and k per slab
};

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
    return make_uint2(pack2(a, b), pack2(c, d));
}
__device__ __forceinline__ uint2 pack4(const f32x4& x) { return pack4(x[0], x[1], x[2], x[3]); }
__device__ __forceinline__ void unpack4(const uint2& u, float (&f)[4]) {
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xFFFF0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xFFFF0000u);
}
__device__ __forceinline__ uint2 ld8(const uint16_t* p) { return *reinterpret_cast<const uint2*>(p); }

// clamped sample bounds, so that malformed offsets never address outside the tokens
__device__ __forceinline__ void bounds(const int32_t* cu, int n, int64_t T, int64_t& s0, int64_t& s1) {
    s0 = min<int64_t>(max<int64_t>(cu[n], 0), T);
    s1 = min<int64_t>(max<int64_t>(cu[n + 1], s0), T);
}

// segments of sample n: ceil(chunks / lseg), at least one (one when lseg = 0)
__device__ __forceinline__ int seg_count(const int32_t* cu, int n, int64_t T, int lseg) {
    int64_t s0, s1;
    bounds(cu, n, T, s0, s1);
    const int nch = int((s1 - s0 + kFC - 1) / kFC);
    return lseg > 0 ? max(1, (nch + lseg - 1) / lseg) : 1;
}

// ---------------------------------------------------------------------------
// plan (one workgroup, packs of more than 64 samples): seg_off[n] = segments before n
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void kda_fused_plan_kernel(const int32_t* __restrict__ cu,
                                                              int32_t* __restrict__ seg_off, int num_seqs,
                                                              int64_t T, int lseg)
{
    __shared__ int32_t part[1024];
    const int tid = threadIdx.x;
    int32_t carry = 0;
    for (int base = 0; base < num_seqs; base += 1024) {
        const int n = base + tid;
        part[tid] = n < num_seqs ? seg_count(cu, n, T, lseg) : 0;
        __syncthreads();
        for (int d = 1; d < 1024; d <<= 1) {          // inclusive scan
            const int32_t add = tid >= d ? part[tid - d] : 0;
            __syncthreads();
            part[tid] += add;
            __syncthreads();
        }
        if (n < num_seqs) seg_off[n + 1] = carry + part[tid];
        carry += part[1023];
        __syncthreads();
    }
    if (tid == 0) seg_off[0] = 0;
}

// The (sample, segment) of global segment id `sid`; every lane of the wave takes part.
// With seg_off NULL (at most 64 samples) lane l scans the segment counts itself.
struct Seg {
    int n, seg, nseg;
};
__device__ __forceinline__ bool find_segment(int sid, const int32_t* cu, const int32_t* seg_off, int num_seqs,
                                             int64_t T, int lseg, int max_segs, int lane, Seg& s)
{
    if (lseg == 0) {
        if (sid >= num_seqs) return false;
        s = Seg{sid, 0, 1};
        return true;
    }
    if (!seg_off) {
        int cnt = lane < num_seqs ? seg_count(cu, lane, T, lseg) : 0;
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int t = __shfl_up(incl, d);
            if (lane >= d) incl += t;
        }
        if (sid >= min(__shfl(incl, 63), max_segs)) return false;
        const int n = __popcll(__ballot(incl <= sid));   // samples that end at or before sid
        const int base = n > 0 ? __shfl(incl, n - 1) : 0;
        s = Seg{n, sid - base, __shfl(cnt, n)};
        return true;
    }
    if (sid >= min(seg_off[num_seqs], max_segs)) return false;
    int lo = 0, hi = num_seqs;                  // seg_off[lo] <= sid < seg_off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (seg_off[mid] <= sid) lo = mid; else hi = mid;
    }
    s = Seg{lo, sid - seg_off[lo], seg_off[lo + 1] - seg_off[lo]};
    return true;
}

// raw rows of one chunk that wave (token tile tt, channel slab cs) and value tile w need
struct Raw {
    uint2 q[2], k[2], l[2], l0[2], v[2];
    uint32_t b;
};

// ---------------------------------------------------------------------------
// PASS 0: one segment per sample, outputs. PASS 1: segment summaries (S_loc, Phi), no
// output. PASS 2: segments from their entry state, outputs.
// ---------------------------------------------------------------------------
template <int PASS, bool NORM>
__global__ __launch_bounds__(kFThreads, 2) void kda_fused_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ la, const uint16_t* __restrict__ beta, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ seg_off, const float* __restrict__ init_state, const float* __restrict__ carry,
    uint16_t* __restrict__ out, float* __restrict__ final_state, float* __restrict__ sloc,
    uint16_t* __restrict__ phi, int num_seqs, int H, int64_t T, int lseg, int max_segs)
{
    using EL = Elt<uint16_t>;
    using Frag = EL::Frag;
    using Frag16 = EL::Frag16;
    constexpr bool kOut = PASS != 1;

    __shared__ FusedSmem sm;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const int tt = w & 1, cs = w >> 1;          // elementwise role: token tile, 32-channel slab

    // block -> (segment, head): consecutive ids on one XCD, so the heads of a segment
    // share their XCD's L2 for beta's rows
    const int nb = gridDim.x;                   // a multiple of 8
    const int lin = (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3);
    const int sid = lin / H, h = lin % H;
    Seg sg;
    if (!find_segment(sid, cu, seg_off, num_seqs, T, lseg, max_segs, lane, sg)) return;
    if (PASS == 1 && sg.seg == sg.nseg - 1) return;          // the last segment needs no summary
    int64_t s0, s1;
    bounds(cu, sg.n, T, s0, s1);
    const int nch = int((s1 - s0 + kFC - 1) / kFC);
    const int c0 = lseg > 0 ? min(sg.seg * lseg, nch) : 0;
    const int c1 = lseg > 0 ? min(c0 + lseg, nch) : nch;

    // state: value columns 16w..16w+15; tile ct holds S[16ct + 4g + i][16w + r]. PASS 1 also
    // carries columns 16w..16w+15 of Phi (identity start).
    f32x4 S[8], Ph[PASS == 1 ? 8 : 1];
    {
        const float* src = nullptr;
        if (PASS == 2 && sg.seg > 0) src = carry + (int64_t(sid - 1) * H + h) * kFD * kFD;
        else if (PASS != 1 && init_state) src = init_state + (int64_t(sg.n) * H + h) * kFD * kFD;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[ct][i] = src ? src[(16 * ct + 4 * g + i) * kFD + 16 * w + r] : 0.f;
        if constexpr (PASS == 1) {
#pragma unroll
            for (int ct = 0; ct < 8; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) Ph[ct][i] = (16 * ct + 4 * g + i == 16 * w + r) ? 1.f : 0.f;
        }
    }

    // constant fragments: identity, inclusive lower triangle (k <= column), all ones
    Frag16 ident, tri, ones;
    {
        uint32_t e[4], t[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            e[s] = (4 * g + s == r) ? kOneBf : 0u;
            t[s] = (4 * g + s <= r) ? kOneBf : 0u;
        }
        ident.u = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
        tri.u = make_uint2(t[0] | (t[1] << 16), t[2] | (t[3] << 16));
        ones.u = make_uint2(kOneBf | (uint32_t(kOneBf) << 16), kOneBf | (uint32_t(kOneBf) << 16));
    }

    // Raw rows of chunk c (clamped to the segment's last chunk: a load past the end is issued
    // all the same and never used). Every wave issues the same loads without conditions, so
    // that the waits for one chunk's rows never include the loads issued after them.
    auto load_raw = [&](Raw& x, int c) __attribute__((always_inline)) {
        const int64_t t0 = s0 + int64_t(min(c, c1 - 1)) * kFC;
        const int nrow = int(min<int64_t>(kFC, s1 - t0));
        const int64_t ob = ((t0 + min(16 * tt + r, nrow - 1)) * H + h) * kFD + 32 * cs + 4 * g;
        const int64_t o0 = ((t0 + min(r, nrow - 1)) * H + h) * kFD + 32 * cs + 4 * g;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if constexpr (kOut) x.q[j] = ld8(q + ob + 16 * j);
            x.k[j] = ld8(k + ob + 16 * j);
            x.l[j] = ld8(la + ob + 16 * j);
            x.l0[j] = ld8(la + o0 + 16 * j);
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
            x.v[rt] = ld8(v + ((t0 + min(16 * rt + r, nrow - 1)) * H + h) * kFD + 16 * w + 4 * g);
        x.b = beta[(t0 + min(lane & 31, nrow - 1)) * H + h];
    };

    // One chunk: `cur` holds its raw rows, the next chunk's rows are loaded into `nxt`. The
    // loop below alternates two register sets, so a chunk waits only for its own rows, which
    // were loaded during the previous chunk (a copy of nxt into cur would tie every chunk's
    // waits to the loads it has just issued).
    auto step = [&](const Raw& cur, Raw& nxt, int c) __attribute__((always_inline)) {
        const int64_t t0 = s0 + int64_t(c) * kFC;
        const int nrow = int(min<int64_t>(kFC, s1 - t0));
        load_raw(nxt, c + 1);

        // ===== E: decayed operands of token tile tt, channels 32cs..32cs+31 =====
        {
            const bool rowok = 16 * tt + r < nrow;
            const uint2 z2 = make_uint2(0u, 0u);
            // G^T(ct, tt) = sum_{rp <= tt} Lam^T(ct, rp) L^T(rp, tt): lane (r, g) then holds
            // G[16tt + r][16ct + 4g + i], the layout of the raw rows
            Frag16 lf[2], l0f[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                lf[j] = EL::from_acc16(EL::mma16(Frag16{rowok ? cur.l[j] : z2}, ident, zero4()));
                l0f[j] = tt ? EL::from_acc16(EL::mma16(Frag16{r < nrow ? cur.l0[j] : z2}, ident, zero4())) : Frag16{z2};
            }
            mfma_ready(lf[0].u, lf[1].u, l0f[0].u, l0f[1].u);
            f32x4 G[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                G[j] = EL::mma16(lf[j], tri, zero4());
                if (tt) G[j] = EL::mma16(l0f[j], ones, G[j]);
            }
            float qf[2][4], kf[2][4];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if constexpr (kOut) unpack4(rowok ? cur.q[j] : z2, qf[j]);
                unpack4(rowok ? cur.k[j] : z2, kf[j]);
            }
            if constexpr (NORM) {
                // each row's sums of squares over the 128 channels: four lanes of this wave
                // and the three waves of the row's other channel slabs
                float qq = 0.f, kk = 0.f;
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        if constexpr (kOut) qq += qf[j][s] * qf[j][s];
                        kk += kf[j][s] * kf[j][s];
                    }
                qq += __shfl_xor(qq, 16);
                qq += __shfl_xor(qq, 32);
                kk += __shfl_xor(kk, 16);
                kk += __shfl_xor(kk, 32);
                if (g == 0) {
                    sm.ssq[cs * kFC + 16 * tt + r] = qq;
                    sm.ssq[(4 + cs) * kFC + 16 * tt + r] = kk;
                }
                lds_barrier();
                float tq = 0.f, tk = 0.f;
#pragma unroll
                for (int x = 0; x < 4; ++x) {      // fixed order: the same sum in every wave
                    tq += sm.ssq[x * kFC + 16 * tt + r];
                    tk += sm.ssq[(4 + x) * kFC + 16 * tt + r];
                }
                const float qs = tq > 0.f ? 1.f / sqrtf(tq) : 0.f;
                const float ks = tk > 0.f ? 1.f / sqrtf(tk) : 0.f;
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        if constexpr (kOut) qf[j][s] *= qs;
                        kf[j][s] *= ks;
                    }
            }
            float dp = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int ct = 2 * cs + j;
                float ex[4], fkh[4], fkc[4], lkc[4], fq[4], lq[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float G2 = G[j][s] * kLog2e;
                    ex[s] = fast_exp2(G2);
                    const float ei = fast_exp2(-G2);
                    fkh[s] = kf[j][s] * ex[s];
                    fkc[s] = kf[j][s] * ei;
                    lkc[s] = fkc[s] - bf2f(f2bf(fkc[s]));
                    if constexpr (kOut) {
                        dp += qf[j][s] * kf[j][s];
                        fq[s] = qf[j][s] * ex[s];
                        lq[s] = fq[s] - bf2f(f2bf(fq[s]));
                    }
                }
                const int o = (16 * tt + r) * kLDK + 16 * ct + 4 * g;
                *reinterpret_cast<uint2*>(&sm.kh[o]) = pack4(fkh[0], fkh[1], fkh[2], fkh[3]);
                *reinterpret_cast<uint2*>(&sm.kch[o]) = pack4(fkc[0], fkc[1], fkc[2], fkc[3]);
                *reinterpret_cast<uint2*>(&sm.kcl[o]) = pack4(lkc[0], lkc[1], lkc[2], lkc[3]);
                if constexpr (kOut) {
                    *reinterpret_cast<uint2*>(&sm.qh[o]) = pack4(fq[0], fq[1], fq[2], fq[3]);
                    *reinterpret_cast<uint2*>(&sm.ql[o]) = pack4(lq[0], lq[1], lq[2], lq[3]);
                }
                // gamma = exp(G of row 31); rows past the sample's end add nothing to G
                if (tt == 1 && r == 15)
                    *reinterpret_cast<float4*>(&sm.gam[16 * ct + 4 * g]) = make_float4(ex[0], ex[1], ex[2], ex[3]);
            }
            if constexpr (kOut) {
                dp += __shfl_xor(dp, 16);
                dp += __shfl_xor(dp, 32);
                if (g == 0) sm.dpp[cs * kFC + 16 * tt + r] = dp;
            }
            if (w == 0 && lane < kFC) sm.beta[lane] = lane < nrow ? bf2f(uint16_t(cur.b)) : 0.f;
        }
        lds_barrier();

        // ===== 2: blocks of A (and its diagonal inverses) and of P; right-hand sides and
        //       Kb^T of key tile w / value tile w =====
        auto lds4 = [&](const uint16_t* arr, int row, int col) -> uint2 {
            return *reinterpret_cast<const uint2*>(&arr[row * kLDK + col]);
        };
        if (w < 3) {
            // A block (ti, tj): w0 (0, 0), w1 (1, 1), w2 (1, 0). With Kc rows as the A operand
            // and Kh rows as the B operand, lane (r, g) holds (Kh Kc^T)[16ti + r][16tj + 4g + s],
            // a row of the block: the A operand layout of a 16x16x16 product.
            const int ti = w == 0 ? 0 : 1, tj = w == 1 ? 1 : 0;
            f32x4 aa = zero4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                aa = EL::mma(EL::load(&sm.kch[(16 * tj + r) * kLDK + 32 * kb], g),
                             EL::load(&sm.kh[(16 * ti + r) * kLDK + 32 * kb], g), aa);
            const float bt = sm.beta[16 * ti + r];
            if (w == 2) {
                sm.na10[lane] = pack4(-bt * aa[0], -bt * aa[1], -bt * aa[2], -bt * aa[3]);
            } else {
                // A_ii strictly lower: (I + A)^-1 = (I - A)(I + A^2)(I + A^4)(I + A^8) exactly
                // (A^16 = 0), on fp32 MFMA. mm(xt, y) = X Y from the accumulator tiles of X^T and Y.
                f32x4 at, id;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    at[s] = (4 * g + s < r) ? bt * aa[s] : 0.f;     // tile of A^T: A[r][4g + s]
                    id[s] = (4 * g + s == r) ? 1.f : 0.f;
                }
                auto mm = [](const f32x4& xt, const f32x4& y) {
                    f32x4 c = zero4();
#pragma unroll
                    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(xt[s], y[s], c, 0, 0, 0);
                    return c;
                };
                const f32x4 ac = mm(at, id);                        // tile of A (exact transpose)
                const f32x4 b1 = mm(at, ac), b1t = mm(ac, at);      // A^2, (A^2)^T
                const f32x4 b2 = mm(b1t, b1), b2t = mm(b1, b1t);    // A^4, (A^4)^T
                const f32x4 b3 = mm(b2t, b2);                       // A^8
                const f32x4 x1t = id - at + b1t - mm(b1, at);       // ((I - A)(I + A^2))^T
                const f32x4 x2t = x1t + mm(b2, x1t);                // (X1 (I + A^4))^T
                const f32x4 tinv = x2t + mm(b3, x2t);               // T^T: lane holds T[r][4g + s]
                sm.tinv[w * 64 + lane] = pack4(tinv);
            }
        } else if (kOut && w < 6) {
            // P block (ti, tj): w3 (0, 0), w4 (1, 1), w5 (1, 0); hi*hi + lo*hi + hi*lo, and the
            // exact q.k on the diagonal
            const int ti = w == 3 ? 0 : 1, tj = w == 4 ? 1 : 0;
            f32x4 pp = zero4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const Frag kch = EL::load(&sm.kch[(16 * tj + r) * kLDK + 32 * kb], g);
                const Frag kcl = EL::load(&sm.kcl[(16 * tj + r) * kLDK + 32 * kb], g);
                const Frag qhh = EL::load(&sm.qh[(16 * ti + r) * kLDK + 32 * kb], g);
                const Frag qhl = EL::load(&sm.ql[(16 * ti + r) * kLDK + 32 * kb], g);
                pp = EL::mma(kch, qhh, pp);
                pp = EL::mma(kcl, qhh, pp);
                pp = EL::mma(kch, qhl, pp);
            }
            float pv[4];
            if (ti == tj) {
                const int row = 16 * ti + r;
                const float dg = sm.dpp[row] + sm.dpp[kFC + row] + sm.dpp[2 * kFC + row] + sm.dpp[3 * kFC + row];
#pragma unroll
                for (int s = 0; s < 4; ++s) pv[s] = 4 * g + s < r ? pp[s] : (4 * g + s == r ? dg : 0.f);
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) pv[s] = pp[s];
            }
            // the B fragment of P^T for output tile ti holds P[16ti + r][16t' + 4g + s], t' = tj
            uint2* dst = reinterpret_cast<uint2*>(&sm.pf[ti * 64 + lane]);
            dst[tj] = pack4(pv[0], pv[1], pv[2], pv[3]);
            if (w == 3) dst[1] = make_uint2(0u, 0u);               // P(0, 1) is above the diagonal
        }
        // right-hand sides of key tile w and value tile w, channel-row layout: tile rt holds
        // Y[16rt + 4g + s][16w + r] (the B operand over the chunk's tokens)
        f32x4 yk[2], yv[2];
        {
            float4 b4[2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) b4[rt] = *reinterpret_cast<const float4*>(&sm.beta[16 * rt + 4 * g]);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const f32x4 kt = EL::mma16(Frag16{lds4(sm.kh, 16 * rt + r, 16 * w + 4 * g)}, ident, zero4());
                const f32x4 vt = EL::mma16(Frag16{16 * rt + r < nrow ? cur.v[rt] : make_uint2(0u, 0u)}, ident, zero4());
                yk[rt] = f32x4{b4[rt].x * kt[0], b4[rt].y * kt[1], b4[rt].z * kt[2], b4[rt].w * kt[3]};
                yv[rt] = f32x4{b4[rt].x * vt[0], b4[rt].y * vt[1], b4[rt].z * vt[2], b4[rt].w * vt[3]};
            }
            // Kb^T tile of key channels 16w..16w+15 as the A operand over the chunk's tokens:
            // lane (r, g) holds gamma[16w + r] Kc[16t' + 4g + s][16w + r]
            const float gm = sm.gam[16 * w + r];
            uint2 kb2[2];
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) {
                f32x4 kc = EL::mma16(Frag16{lds4(sm.kch, 16 * t2 + r, 16 * w + 4 * g)}, ident, zero4());
                kc = EL::mma16(Frag16{lds4(sm.kcl, 16 * t2 + r, 16 * w + 4 * g)}, ident, kc);
                kb2[t2] = pack4(gm * kc[0], gm * kc[1], gm * kc[2], gm * kc[3]);
            }
            sm.kbt[w * 64 + lane] = make_uint4(kb2[0].x, kb2[0].y, kb2[1].x, kb2[1].y);
        }
        lds_barrier();

        // ===== 3: (I + A) X = Y by 16-row blocks: X0 = T00 Y0, X1 = T11 (Y1 - A10 X0) =====
        {
            const Frag16 t00{sm.tinv[lane]}, t11{sm.tinv[64 + lane]}, a10{sm.na10[lane]};
            // U of value tile w (stays in registers) and W of key tile w, side by side
            Frag16 pv = EL::from_acc16(yv[0]), pk = EL::from_acc16(yk[0]);
            mfma_ready(pv.u, pk.u);
            yv[0] = EL::mma16(t00, pv, zero4());
            yk[0] = EL::mma16(t00, pk, zero4());
            pv = EL::from_acc16(yv[0]);
            pk = EL::from_acc16(yk[0]);
            mfma_ready(pv.u, pk.u);
            const f32x4 av = EL::mma16(a10, pv, yv[1]);
            const f32x4 ak = EL::mma16(a10, pk, yk[1]);
            pv = EL::from_acc16(av);
            pk = EL::from_acc16(ak);
            mfma_ready(pv.u, pk.u);
            yv[1] = EL::mma16(t11, pv, zero4());
            yk[1] = EL::mma16(t11, pk, zero4());
            // -W in token rows (the A operand of W S): transpose with the identity product
            Frag16 nw[2] = {EL::from_acc16(-yk[0]), EL::from_acc16(-yk[1])};
            mfma_ready(nw[0].u, nw[1].u);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const f32x4 wt = EL::mma16(nw[rt], ident, zero4());
                *reinterpret_cast<uint2*>(&sm.kh[(16 * rt + r) * kLDK + 16 * w + 4 * g]) = pack4(wt);
            }
        }
        lds_barrier();

        // ===== C: the state pass over value columns 16w..16w+15 =====
        {
            Frag sf[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) sf[kb] = EL::from_acc(S[2 * kb], S[2 * kb + 1]);
            mfma_ready(sf[0].u, sf[1].u, sf[2].u, sf[3].u);
            f32x4 X[2] = {yv[0], yv[1]};                 // Vn = U - W S: rows 16rt + 4g + i, column r
            f32x4 XP[2] = {zero4(), zero4()};            // the transition's columns (U = 0)
            Frag pfr[4];
            if constexpr (PASS == 1) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) pfr[kb] = EL::from_acc(Ph[2 * kb], Ph[2 * kb + 1]);
                mfma_ready(pfr[0].u, pfr[1].u, pfr[2].u, pfr[3].u);
            }
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const Frag wf = EL::load(&sm.kh[(16 * rt + r) * kLDK + 32 * kb], g);
                    X[rt] = EL::mma(wf, sf[kb], X[rt]);
                    if constexpr (PASS == 1) XP[rt] = EL::mma(wf, pfr[kb], XP[rt]);
                }
            f32x4 O[2] = {zero4(), zero4()};             // O^T: O[16rt + r][16w + 4g + i]
            if constexpr (kOut) {
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt)
                        O[rt] = EL::mma(sf[kb], EL::load(&sm.qh[(16 * rt + r) * kLDK + 32 * kb], g), O[rt]);
            }
            Frag vf = EL::from_acc(X[0], X[1]);          // Vn over the chunk's tokens
            Frag vfp;
            if constexpr (PASS == 1) {
                vfp = EL::from_acc(XP[0], XP[1]);
                mfma_ready(vf.u, vfp.u);
            } else {
                mfma_ready(vf.u);
            }
            if constexpr (kOut) {
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) O[rt] = EL::mma(vf, Frag{sm.pf[rt * 64 + lane]}, O[rt]);
            }
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                const float4 g4 = *reinterpret_cast<const float4*>(&sm.gam[16 * ct + 4 * g]);
                const Frag kf = Frag{sm.kbt[ct * 64 + lane]};
                S[ct] = f32x4{S[ct][0] * g4.x, S[ct][1] * g4.y, S[ct][2] * g4.z, S[ct][3] * g4.w};
                S[ct] = EL::mma(kf, vf, S[ct]);
                if constexpr (PASS == 1) {
                    Ph[ct] = f32x4{Ph[ct][0] * g4.x, Ph[ct][1] * g4.y, Ph[ct][2] * g4.z, Ph[ct][3] * g4.w};
                    Ph[ct] = EL::mma(kf, vfp, Ph[ct]);
                }
            }
            if constexpr (kOut) {
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const int row = 16 * rt + r;
                    if (row < nrow)
                        *reinterpret_cast<uint2*>(out + ((t0 + row) * H + h) * kFD + 16 * w + 4 * g) = pack4(O[rt]);
                }
            }
        }
        lds_barrier();
    };
    Raw ra, rb;
    if (c0 < c1) load_raw(ra, c0);
    for (int c = c0; c < c1; c += 2) {
        step(ra, rb, c);
        if (c + 1 < c1) step(rb, ra, c + 1);
    }

    if constexpr (PASS == 1) {
        // S_loc (fp32, [d_k][d_v]) and Phi as hi/lo bf16 A fragments of the combine's products
        // (rows = output key channel, k = input key channel): fragment (ct, kb) half w & 1 of
        // kb = w >> 1 holds Phi[16ct + r][16w + 4g + s], the exact transpose of tile ct
        const int64_t unit = int64_t(sid) * H + h;
        float* sl = sloc + unit * kFD * kFD;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) sl[(16 * ct + 4 * g + i) * kFD + 16 * w + r] = S[ct][i];
        uint16_t* pb = phi + unit * (2 * 8 * 4 * 64 * 8);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            f32x4 lo;
#pragma unroll
            for (int i = 0; i < 4; ++i) lo[i] = Ph[ct][i] - bf2f(f2bf(Ph[ct][i]));
            Frag16 fh = EL::from_acc16(Ph[ct]), fl = EL::from_acc16(lo);
            mfma_ready(fh.u, fl.u);
            const f32x4 th = EL::mma16(fh, ident, zero4());
            const f32x4 tl = EL::mma16(fl, ident, zero4());
            const int o = ((ct * 4 + (w >> 1)) * 64 + lane) * 8 + (w & 1) * 4;
            *reinterpret_cast<uint2*>(pb + o) = pack4(th);
            *reinterpret_cast<uint2*>(pb + 8 * 4 * 64 * 8 + o) = pack4(tl);
        }
    } else if (final_state && sg.seg == sg.nseg - 1) {
        float* fs = final_state + (int64_t(sg.n) * H + h) * kFD * kFD;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) fs[(16 * ct + 4 * g + i) * kFD + 16 * w + r] = S[ct][i];
    }
}

// ---------------------------------------------------------------------------
// combine: per (sample, head, 16 value columns), the entry state of every segment,
// S_in(k + 1) = Phi(k) S_in(k) + S_loc(k), S_in(0) = the initial state; S_in(k + 1) is
// written over S_loc(k) (the slot of segment k), which no later step reads. Wave w
// computes output rows 32w..32w+31 (key tiles 2w, 2w + 1); the full S_in enters every
// wave's products as hi/lo bf16 B fragments through LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kCombThreads) void kda_fused_combine_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ seg_off, const float* __restrict__ init_state,
    float* __restrict__ sloc, const uint16_t* __restrict__ phi, int num_seqs, int H, int64_t T, int lseg,
    int max_segs)
{
    using EL = Elt<uint16_t>;
    using Frag = EL::Frag;
    __shared__ uint4 sb[2][4][64];              // S_in as B fragments: [hi/lo][k-block][lane]
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const int ct0 = blockIdx.x & 7;             // value tile: columns 16 ct0 + r
    const int unit = blockIdx.x >> 3;
    if (unit >= num_seqs * H) return;
    const int n = unit / H, h = unit % H;
    // first segment id of sample n and its segment count
    int first, nseg;
    if (!seg_off) {
        int cnt = lane < num_seqs ? seg_count(cu, lane, T, lseg) : 0;
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int t = __shfl_up(incl, d);
            if (lane >= d) incl += t;
        }
        first = n > 0 ? __shfl(incl, n - 1) : 0;
        nseg = __shfl(cnt, n);
    } else {
        first = seg_off[n];
        nseg = seg_off[n + 1] - seg_off[n];
    }
    if (first + nseg > max_segs) nseg = max(0, max_segs - first);
    if (nseg <= 1) return;

    const int col = 16 * ct0 + r;
    f32x4 S[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[j][i] = init_state ? init_state[((int64_t(n) * H + h) * kFD + 32 * w + 16 * j + 4 * g + i) * kFD + col]
                                 : 0.f;
    constexpr int kPhiHalf = 8 * 4 * 64 * 8;    // bf16 elements of the hi (or lo) fragments
    auto phi_frag = [&](int64_t u, int hl, int ct, int kb) -> Frag {
        return Frag{*reinterpret_cast<const uint4*>(phi + u * 2 * kPhiHalf + hl * kPhiHalf + ((ct * 4 + kb) * 64 + lane) * 8)};
    };
    for (int kseg = 0; kseg + 1 < nseg; ++kseg) {
        const int64_t u = int64_t(first + kseg) * H + h;
        // publish S_in(kseg): this wave's rows are k-block w of the products
        {
            f32x4 l0, l1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                l0[i] = S[0][i] - bf2f(f2bf(S[0][i]));
                l1[i] = S[1][i] - bf2f(f2bf(S[1][i]));
            }
            sb[0][w][lane] = EL::from_acc(S[0], S[1]).u;
            sb[1][w][lane] = EL::from_acc(l0, l1).u;
        }
        lds_barrier();
        float* sl = sloc + u * kFD * kFD;
        f32x4 acc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int ct = 2 * w + j;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[j][i] = sl[(16 * ct + 4 * g + i) * kFD + col];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const Frag ah = phi_frag(u, 0, ct, kb), al = phi_frag(u, 1, ct, kb);
                const Frag bh{sb[0][kb][lane]}, bl{sb[1][kb][lane]};
                acc[j] = EL::mma(ah, bh, acc[j]);
                acc[j] = EL::mma(ah, bl, acc[j]);
                acc[j] = EL::mma(al, bh, acc[j]);
            }
        }
        lds_barrier();
        // S_in(kseg + 1) over S_loc(kseg): the same lanes read and write these elements
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            S[j] = acc[j];
#pragma unroll
            for (int i = 0; i < 4; ++i) sl[(16 * (2 * w + j) + 4 * g + i) * kFD + col] = acc[j][i];
        }
    }
}

struct FusedPlan {
    int lseg;          // chunks (32 tokens) per segment; 0 = one segment per sample
    int max_segs;
    size_t table_bytes, sloc_bytes, phi_bytes;
};

FusedPlan plan_with(int64_t chunks, int32_t N, int32_t H, int64_t lseg)
{
    FusedPlan p{};
    p.lseg = lseg > 0 && lseg < chunks ? int(lseg) : 0;
    p.max_segs = p.lseg ? int((chunks + p.lseg - 1) / p.lseg + N) : N;
    p.table_bytes = (p.lseg && N > 64) ? ((size_t(N) + 1) * 4 + 255) & ~size_t(255) : 0;
    p.sloc_bytes = p.lseg ? size_t(p.max_segs) * H * kFD * kFD * 4 : 0;
    p.phi_bytes = p.lseg ? size_t(p.max_segs) * H * kFD * kFD * 4 : 0;   // hi + lo bf16
    return p;
}

// Cut samples into segments when the (sample, head) units alone would fill fewer than two
// workgroups per CU: about 512 segment-workgroups then run, of at least 16 chunks each.
// With a byte limit on the workspace, segments grow until their summaries fit (fewer,
// longer segments); when not even one cut per sample fits, samples stay whole.
FusedPlan fused_plan(int64_t T, int32_t N, int32_t H, size_t cap)
{
    const int64_t units = int64_t(N) * H;
    const int64_t chunks = (T + kFC - 1) / kFC + N;         // upper bound over all samples
    int64_t lseg = units < 512 ? std::max<int64_t>(16, (chunks * H + 511) / 512) : 0;
    FusedPlan p = plan_with(chunks, N, H, lseg);
    if (p.table_bytes + p.sloc_bytes + p.phi_bytes <= cap) return p;
    const size_t slot = size_t(2) * kFD * kFD * 4 * size_t(H);          // one segment's summaries, all heads
    const size_t avail = cap > p.table_bytes ? cap - p.table_bytes : 0;
    const int64_t max_segs = int64_t(avail / slot);
    lseg = max_segs > N ? std::max<int64_t>(lseg, (chunks + (max_segs - N) - 1) / (max_segs - N)) : 0;
    return plan_with(chunks, N, H, lseg);
}

template <int PASS, bool NORM>
hipError_t launch_pass(const LaunchArgs& a, const int32_t* seg_off, const FusedPlan& p, const float* carry,
                       float* sloc, uint16_t* phi)
{
    const int units = (p.lseg ? p.max_segs : a.num_seqs) * a.num_heads;
    const int blocks = ((units + 7) / 8) * 8;
    hipLaunchKernelGGL((kda_fused_kernel<PASS, NORM>), dim3(blocks), dim3(kFThreads), 0, a.stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.log_alpha),
                       static_cast<const uint16_t*>(a.beta), a.cu_seqlens, seg_off, a.init_state, carry,
                       static_cast<uint16_t*>(a.out), a.final_state, sloc, phi, a.num_seqs, a.num_heads,
                       a.total_tokens, p.lseg, p.max_segs);
    return hipGetLastError();
}

template <bool NORM>
hipError_t launch_fused_norm(const LaunchArgs& a, const int32_t* seg_off, const FusedPlan& p, float* sloc,
                             uint16_t* phi, TimingHook* th)
{
    hipError_t e;
    if (p.lseg == 0) {
        if (th) th->begin("fused", a.stream);
        e = launch_pass<0, NORM>(a, seg_off, p, nullptr, nullptr, nullptr);
        if (th) th->end(a.stream);
        return e;
    }
    if (th) th->begin("fused_sum", a.stream);
    e = launch_pass<1, NORM>(a, seg_off, p, nullptr, sloc, phi);
    if (th) th->end(a.stream);
    if (e != hipSuccess) return e;
    if (th) th->begin("fused_combine", a.stream);
    hipLaunchKernelGGL(kda_fused_combine_kernel, dim3(a.num_seqs * a.num_heads * 8), dim3(kCombThreads), 0,
                       a.stream, a.cu_seqlens, seg_off, a.init_state, sloc, phi, a.num_seqs, a.num_heads,
                       a.total_tokens, p.lseg, p.max_segs);
    if (th) th->end(a.stream);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (th) th->begin("fused", a.stream);
    e = launch_pass<2, NORM>(a, seg_off, p, sloc, nullptr, nullptr);
    if (th) th->end(a.stream);
    return e;
}

}  // namespace

bool fused_supported(const LaunchArgs& a)
{
    return a.dtype_bf16 && a.d_k == kFD && a.d_v == kFD;
}

size_t fused_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_heads, size_t cap)
{
    const FusedPlan p = fused_plan(total_tokens, num_seqs, num_heads, cap);
    return p.table_bytes + p.sloc_bytes + p.phi_bytes;
}

hipError_t launch_forward_fused(const LaunchArgs& a, void* workspace, TimingHook* th, size_t cap)
{
    const FusedPlan p = fused_plan(a.total_tokens, a.num_seqs, a.num_heads, cap);
    if (int64_t(p.max_segs) * a.num_heads > 0x7FFFFFFF / 8) return hipErrorInvalidValue;
    char* base = static_cast<char*>(workspace);
    int32_t* seg_off = p.table_bytes ? reinterpret_cast<int32_t*>(base) : nullptr;
    float* sloc = p.lseg ? reinterpret_cast<float*>(base + p.table_bytes) : nullptr;
    uint16_t* phi = p.lseg ? reinterpret_cast<uint16_t*>(base + p.table_bytes + p.sloc_bytes) : nullptr;
    if (seg_off) {
        if (th) th->begin("plan", a.stream);
        hipLaunchKernelGGL(kda_fused_plan_kernel, dim3(1), dim3(1024), 0, a.stream, a.cu_seqlens, seg_off,
                           a.num_seqs, a.total_tokens, p.lseg);
        if (th) th->end(a.stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return a.qk_l2norm ? launch_fused_norm<true>(a, seg_off, p, sloc, phi, th)
                       : launch_fused_norm<false>(a, seg_off, p, sloc, phi, th);
}

}  // namespace kda
