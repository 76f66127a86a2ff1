// kda_wy.hip -- two-kernel chunkwise KDA forward scan for bf16 data (gfx950).
//
// Recurrence (Chimera, arXiv 2607.28611: update printed in the explainer page,
// "One stream, three mechanisms, no positions"; state reset at every packed
// sample, paper Sec. 3 KDA paragraph), per (sample, head):
//     S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,   o_t = S_t^T q_t.
// Chunkwise form over chunks of C = 64 tokens (G = inclusive cumsum of log a over
// the chunk's rows, per key channel; gamma = exp(G of the last row)):
//     Qh = Q e^G, Kh = K e^G, Kc = K e^-G, Kb = K e^(G_last - G)
//     A = StrictLower(diag(b) Kh Kc^T),  (I + A) [W | U] = diag(b) [Kh | V]
//     Vn = U - W S,  O = Qh S + LowerIncl(Qh Kc^T) Vn,  S <- diag(gamma) S + Kb^T Vn
// Every term except the last three lines is independent of S, so it is computed
// for all (chunk, head) pairs at once by the prep kernel, which writes the chunk's
// operands to a workspace in the exact MFMA fragment order the chain kernel reads.
// The chain kernel carries S through the chunks of one sample: three groups of
// products per chunk and no solve on the serial path.
//
// Fragment conventions are those of kda_device.h. With the 16x16x16 product, an
// accumulator tile (rows 4g+s, column r) is the B operand of the same matrix and
// the A operand of its transpose; a product with the identity as B operand
// transposes a tile exactly (bf16 values times one, fp32 accumulation).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "kda_device.h"
#include "kda_internal.h"


namespace kda {
namespace {
using namespace dev;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 16 bytes as a native vector:
                                                               // copies stay in registers
constexpr int kWC = 64;            // chunk rows
constexpr int kWThreads = 256;     // 4 wave64
constexpr uint16_t kOne = 0x3F80;  // bf16 1.0

// Workspace record of one (chunk, head), in bf16 units.
template <int DK, int DV> struct WyLayout {
    static constexpr int NKB = DK / 32;    // k-blocks over key channels
    static constexpr int NCT = DK / 16;    // 16-wide key channel tiles
    static constexpr int NVT = DV / 16;    // 16-wide value column tiles
    static constexpr int W = 0;                        // -W: [rt 4][kb NKB][lane 64][8], token rows
    static constexpr int Q = W + 4 * NKB * 512;        // Qh: [rt 4][kb NKB][64][8], token rows
    static constexpr int K = Q + 4 * NKB * 512;        // Kb^T: [ct NCT][kb 2][64][8], key channel rows
    static constexpr int P = K + NCT * 2 * 512;        // P: [rt 4][kb 2][64][8], token rows
    static constexpr int G = P + 8 * 512;              // gamma: DK fp32
    static constexpr int SHARED = G + 2 * DK;          // operands every value tile reads
    static constexpr int U = SHARED;                   // U: [vt NVT][rt 4][64][4], accumulator layout
    static constexpr int UTILE = 4 * 1024;             // U of one 64-column value tile
    static constexpr int TOTAL = U + NVT * 1024;
    static_assert((SHARED * 2) % 16 == 0 && (TOTAL * 2) % 16 == 0, "16-byte sections");
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

// ---------------------------------------------------------------------------
// plan (one workgroup): chunk_off[n] = number of chunks of the samples before n;
// seg_off[n] = number of segments before n, where a sample of c chunks has
// ceil(c / lseg) segments of lseg chunks (at least one; one when lseg = 0)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void kda_wy_plan_kernel(const int32_t* __restrict__ cu,
                                                           int32_t* __restrict__ chunk_off,
                                                           int32_t* __restrict__ seg_off, int num_seqs,
                                                           int64_t total_tokens, int lseg)
{
    __shared__ int32_t part[1024], segp[1024];
    const int tid = threadIdx.x;
    int32_t carry = 0, scarry = 0;
    for (int base = 0; base < num_seqs; base += 1024) {
        const int n = base + tid;
        int32_t cnt = 0, nseg = 0;
        if (n < num_seqs) {
            const int64_t s0 = min<int64_t>(max<int64_t>(cu[n], 0), total_tokens);
            const int64_t s1 = min<int64_t>(max<int64_t>(cu[n + 1], s0), total_tokens);
            cnt = int32_t((s1 - s0 + kWC - 1) / kWC);
            nseg = lseg > 0 ? max(1, (cnt + lseg - 1) / lseg) : 1;
        }
        part[tid] = cnt;
        segp[tid] = nseg;
        __syncthreads();
        for (int d = 1; d < 1024; d <<= 1) {          // inclusive scans
            const int32_t add = tid >= d ? part[tid - d] : 0;
            const int32_t sadd = tid >= d ? segp[tid - d] : 0;
            __syncthreads();
            part[tid] += add;
            segp[tid] += sadd;
            __syncthreads();
        }
        if (n < num_seqs) {
            chunk_off[n + 1] = carry + part[tid];
            seg_off[n + 1] = scarry + segp[tid];
        }
        carry += part[1023];
        scarry += segp[1023];
        __syncthreads();
    }
    if (tid == 0) {
        chunk_off[0] = 0;
        seg_off[0] = 0;
    }
}

// clamped sample bounds, so that malformed offsets never address outside the tokens
__device__ __forceinline__ void sample_bounds(const int32_t* cu, int n, int64_t T, int64_t& s0, int64_t& s1) {
    s0 = min<int64_t>(max<int64_t>(cu[n], 0), T);
    s1 = min<int64_t>(max<int64_t>(cu[n + 1], s0), T);
}

// For a pack of at most 64 samples each wave forms the chunk table itself: lane l
// holds the number of chunks of samples 0..l (inclusive), and no plan kernel runs.
__device__ __forceinline__ int wave_chunk_scan(const int32_t* cu, int num_seqs, int64_t T, int lane) {
    int v = 0;
    if (lane < num_seqs) {
        int64_t s0, s1;
        sample_bounds(cu, lane, T, s0, s1);
        v = int((s1 - s0 + kWC - 1) / kWC);
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(v, d);
        if (lane >= d) v += t;
    }
    return v;
}

// ---------------------------------------------------------------------------
// prep: the S-independent operands of one (chunk, head)
// ---------------------------------------------------------------------------
template <int DK> struct PrepSmem {
    static constexpr int LDK = DK + 8;       // token rows, 16-byte aligned
    alignas(16) uint16_t qk[kWC * LDK];      // raw q; each wave then writes Kc hi over its own rows
    alignas(16) uint16_t kcl[kWC * LDK];     // Kc, lo part
    alignas(16) uint16_t kr[kWC * LDK];      // raw k; each wave then writes Kh over its own rows
    alignas(16) uint16_t lr[kWC * LDK];      // raw log a
    alignas(16) uint16_t aoff[6 * 256];      // -A blocks (i, j), j < i: 16x16x16 A fragments [blk][lane][4]
    alignas(16) float at[4 * 16 * 20];       // strictly lower diagonal blocks of A, rows; then
                                             // (I + A_ii)^-1 as 16x16x16 A fragments
    alignas(16) float beta[kWC];
    alignas(16) float gam[DK];               // exp(G) of the chunk's last row
};

// NORM: q_t and k_t are divided by their Euclidean length on load (per token and
// head; a zero vector stays zero), the normalisation fused into the scan kernels
// that the paper's training setup describes.
template <int DK, int DV, bool NORM>
__global__ __launch_bounds__(kWThreads, 2) void kda_wy_prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ la, const uint16_t* __restrict__ beta, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ chunk_off, uint16_t* __restrict__ ws, int num_seqs, int H,
    int64_t total_tokens, int max_chunks)
{
    using EL = Elt<uint16_t>;
    using Frag = EL::Frag;
    using Frag16 = EL::Frag16;
    using Lay = WyLayout<DK, DV>;
    using Sm = PrepSmem<DK>;
    constexpr int NKB = Lay::NKB, NCT = Lay::NCT, NVT = Lay::NVT;
    constexpr int CW = NCT / 4, VW = NVT / 4;   // key channel / value tiles per wave
    constexpr int LDK = Sm::LDK;
    static_assert(CW >= 1 && VW >= 1, "d_k and d_v must be multiples of 64");

    __shared__ Sm sm;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;

    const int c = blockIdx.x, h = blockIdx.y;
    int lo, cbase;                              // sample owning chunk c, its first chunk
    if (!chunk_off) {
        const int incl = wave_chunk_scan(cu, num_seqs, total_tokens, lane);
        if (c >= min(__shfl(incl, 63), max_chunks)) return;
        lo = __popcll(__ballot(incl <= c));     // samples that end at or before chunk c
        cbase = lo > 0 ? __shfl(incl, lo - 1) : 0;
    } else {
        const int ntot = min(chunk_off[num_seqs], max_chunks);
        if (c >= ntot) return;
        lo = 0;
        int hi = num_seqs;                      // chunk_off[lo] <= c < chunk_off[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (chunk_off[mid] <= c) lo = mid; else hi = mid;
        }
        cbase = chunk_off[lo];
    }
    int64_t s0, s1;
    sample_bounds(cu, lo, total_tokens, s0, s1);
    const int64_t t0 = s0 + int64_t(c - cbase) * kWC;
    const int nrow = int(min<int64_t>(kWC, s1 - t0));   // >= 1
    uint16_t* rec = ws + (int64_t(h) * max_chunks + c) * Lay::TOTAL;
    auto grow = [&](int row) { return (t0 + min(row, nrow - 1)) * H + h; };   // clamped token row

    // ===== stage: raw q, k, log a rows of the chunk to LDS (zero past the sample's
    //       end), this wave's value columns and the gates to registers; every load is
    //       issued before the first wait =====
    constexpr int PPR = DK / 8;                 // 16-byte pieces per row
    constexpr int NPC = kWC * PPR / kWThreads;  // pieces per thread and array
    static_assert(kWC * PPR % kWThreads == 0, "staging split");
    u32x4 rq[NPC], rk[NPC], rl[NPC];
#pragma unroll
    for (int j = 0; j < NPC; ++j) {
        const int p = tid + j * kWThreads, row = p / PPR, col = (p % PPR) * 8;
        const int64_t off = grow(row) * DK + col;
        rq[j] = *reinterpret_cast<const u32x4*>(q + off);
        rk[j] = *reinterpret_cast<const u32x4*>(k + off);
        rl[j] = *reinterpret_cast<const u32x4*>(la + off);
    }
    uint2 vraw[VW][4];
#pragma unroll
    for (int u = 0; u < VW; ++u)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
            vraw[u][rt] = *reinterpret_cast<const uint2*>(v + grow(16 * rt + r) * DV + 16 * (VW * wave + u) + 4 * g);
    const uint16_t braw = beta[grow(tid & 63)];
#pragma unroll
    for (int j = 0; j < NPC; ++j) {
        const int p = tid + j * kWThreads, row = p / PPR, col = (p % PPR) * 8;
        const u32x4 z = {0u, 0u, 0u, 0u};
        const bool ok = row < nrow;
        *reinterpret_cast<u32x4*>(&sm.qk[row * LDK + col]) = ok ? rq[j] : z;
        *reinterpret_cast<u32x4*>(&sm.kr[row * LDK + col]) = ok ? rk[j] : z;
        *reinterpret_cast<u32x4*>(&sm.lr[row * LDK + col]) = ok ? rl[j] : z;
    }
    if (tid < kWC) sm.beta[tid] = tid < nrow ? bf2f(braw) : 0.f;
#pragma unroll
    for (int u = 0; u < VW; ++u)
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
            if (16 * rt + r >= nrow) vraw[u][rt] = make_uint2(0, 0);
    lds_barrier();

    // 4 consecutive elements of an LDS row
    auto lds4 = [&](const uint16_t* arr, int row, int col) -> uint2 {
        return *reinterpret_cast<const uint2*>(&arr[row * LDK + col]);
    };
    // constant fragments: identity, all-ones, inclusive lower triangle (k <= row)
    Frag16 ident, ones, tri;
    {
        uint32_t e[4], t[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            e[s] = (4 * g + s == r) ? kOne : 0u;
            t[s] = (4 * g + s <= r) ? kOne : 0u;
        }
        ident.u = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
        tri.u = make_uint2(t[0] | (t[1] << 16), t[2] | (t[3] << 16));
        ones.u = make_uint2(kOne | (uint32_t(kOne) << 16), kOne | (uint32_t(kOne) << 16));
    }

    // ===== phase 1: token tile i = wave, all key channels (token-row layout) =====
    const int i = wave;
    uint2 khv[NCT], qhh[NCT], qhl[NCT];         // Kh, Qh hi, Qh lo of token tile i
    float dp = 0.f;                             // q.k of token 16i + r (partial over this lane's channels)
    {
        // G of token tile i: G^T(ct, i) = sum_{rp <= i} Lam^T(ct, rp) L^T(rp, i)
        f32x4 gt[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) gt[ct] = zero4();
        for (int rp = 0; rp <= i; ++rp) {
            const Frag16 lb = (rp < i) ? ones : tri;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                // transposed tile: Lam[16rp + 4g + s][16ct + r], the A operand of Lam^T
                Frag16 lamT = EL::from_acc16(EL::mma16(Frag16{lds4(sm.lr, 16 * rp + r, 16 * ct + 4 * g)}, ident, zero4()));
                EL::ready(lamT);
                gt[ct] = EL::mma16(lamT, lb, gt[ct]);
            }
        }
        // lane (r, g), tile ct: G[16i + r][16ct + 4g + s]; q, k in the same layout
        uint2 qv[NCT], kv[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            qv[ct] = lds4(sm.qk, 16 * i + r, 16 * ct + 4 * g);
            kv[ct] = lds4(sm.kr, 16 * i + r, 16 * ct + 4 * g);
        }
        // the four lanes r, r + 16, r + 32, r + 48 hold all channels of row 16i + r
        float qs = 1.f, ks = 1.f;
        if constexpr (NORM) {
            float qq = 0.f, kk = 0.f;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                float qf[4], kf[4];
                unpack4(qv[ct], qf);
                unpack4(kv[ct], kf);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    qq += qf[s] * qf[s];
                    kk += kf[s] * kf[s];
                }
            }
            qq += __shfl_xor(qq, 16);
            qq += __shfl_xor(qq, 32);
            kk += __shfl_xor(kk, 16);
            kk += __shfl_xor(kk, 32);
            qs = qq > 0.f ? 1.f / sqrtf(qq) : 0.f;
            ks = kk > 0.f ? 1.f / sqrtf(kk) : 0.f;
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            float qf[4], kf[4], fq[4], fkh[4], fkc[4], lq[4], lk[4];
            unpack4(qv[ct], qf);
            unpack4(kv[ct], kf);
            if constexpr (NORM) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    qf[s] *= qs;
                    kf[s] *= ks;
                }
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float G2 = gt[ct][s] * kLog2e;
                const float ex = fast_exp2(G2), ei = fast_exp2(-G2);
                dp += qf[s] * kf[s];
                fq[s] = qf[s] * ex;
                fkh[s] = kf[s] * ex;
                fkc[s] = kf[s] * ei;
                lq[s] = fq[s] - bf2f(f2bf(fq[s]));
                lk[s] = fkc[s] - bf2f(f2bf(fkc[s]));
            }
            qhh[ct] = pack4(fq[0], fq[1], fq[2], fq[3]);
            qhl[ct] = pack4(lq[0], lq[1], lq[2], lq[3]);
            khv[ct] = pack4(fkh[0], fkh[1], fkh[2], fkh[3]);
            // Kc hi over the raw q and Kh over the raw k of this wave's own rows (no
            // other wave reads them)
            *reinterpret_cast<uint2*>(&sm.qk[(16 * i + r) * LDK + 16 * ct + 4 * g]) = pack4(fkc[0], fkc[1], fkc[2], fkc[3]);
            *reinterpret_cast<uint2*>(&sm.kcl[(16 * i + r) * LDK + 16 * ct + 4 * g]) = pack4(lk[0], lk[1], lk[2], lk[3]);
            *reinterpret_cast<uint2*>(&sm.kr[(16 * i + r) * LDK + 16 * ct + 4 * g]) = khv[ct];
            // gamma = exp(G of row 63); rows past the sample's end add nothing to G
            if (i == 3 && r == 15)
                *reinterpret_cast<float4*>(&sm.gam[16 * ct + 4 * g]) =
                    make_float4(fast_exp2(gt[ct][0] * kLog2e), fast_exp2(gt[ct][1] * kLog2e),
                                fast_exp2(gt[ct][2] * kLog2e), fast_exp2(gt[ct][3] * kLog2e));
        }
        dp += __shfl_xor(dp, 16);
        dp += __shfl_xor(dp, 32);
        // Qh fragments of the chain kernel: (rt = i, kb) = [tile 2kb | tile 2kb + 1]
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
            *reinterpret_cast<uint4*>(rec + Lay::Q + ((i * NKB + kb) * 64 + lane) * 8) =
                make_uint4(qhh[2 * kb].x, qhh[2 * kb].y, qhh[2 * kb + 1].x, qhh[2 * kb + 1].y);
    }
    const float bt = sm.beta[16 * i + r];
    lds_barrier();

    // ===== phase 2: A and P tiles of token rows i (columns j <= i) =====
    for (int j = 0; j <= i; ++j) {
        f32x4 aa = zero4(), pp = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const Frag kh = EL::load(&sm.qk[(16 * j + r) * LDK + 32 * kb], g);
            const Frag kl = EL::load(&sm.kcl[(16 * j + r) * LDK + 32 * kb], g);
            const Frag khat{make_uint4(khv[2 * kb].x, khv[2 * kb].y, khv[2 * kb + 1].x, khv[2 * kb + 1].y)};
            const Frag qh{make_uint4(qhh[2 * kb].x, qhh[2 * kb].y, qhh[2 * kb + 1].x, qhh[2 * kb + 1].y)};
            const Frag ql{make_uint4(qhl[2 * kb].x, qhl[2 * kb].y, qhl[2 * kb + 1].x, qhl[2 * kb + 1].y)};
            aa = EL::mma(kh, khat, aa);      // (Kh Kc^T)[16i + r][16j + 4g + s]
            pp = EL::mma(kh, qh, pp);        // (Qh Kc^T)[16i + r][16j + 4g + s], hi/lo
            pp = EL::mma(kl, qh, pp);
            pp = EL::mma(kh, ql, pp);
        }
        if (j < i) {
            *reinterpret_cast<uint2*>(&sm.aoff[((i * (i - 1)) / 2 + j) * 256 + lane * 4]) =
                pack4(-bt * aa[0], -bt * aa[1], -bt * aa[2], -bt * aa[3]);
        } else {
            float4 x;
            x.x = (4 * g + 0 < r) ? bt * aa[0] : 0.f;
            x.y = (4 * g + 1 < r) ? bt * aa[1] : 0.f;
            x.z = (4 * g + 2 < r) ? bt * aa[2] : 0.f;
            x.w = (4 * g + 3 < r) ? bt * aa[3] : 0.f;
            *reinterpret_cast<float4*>(&sm.at[(i * 16 + r) * 20 + 4 * g]) = x;
        }
        float pv[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int col = 4 * g + s;
            pv[s] = (j < i || col < r) ? pp[s] : (col == r ? dp : 0.f);
        }
        *reinterpret_cast<uint2*>(rec + Lay::P + ((i * 2 + j / 2) * 64 + lane) * 8 + (j & 1) * 4) =
            pack4(pv[0], pv[1], pv[2], pv[3]);
    }
    if ((i & 1) == 0)   // the upper half of the last fragment of rows i lies above the diagonal
        *reinterpret_cast<uint2*>(rec + Lay::P + ((i * 2 + i / 2) * 64 + lane) * 8 + 4) = make_uint2(0, 0);
    lds_barrier();

    // ===== phase 3: inverse of diagonal block `wave`; key channel and value slabs =====
    {
        // A_ww is strictly lower triangular, so (A_ww)^16 = 0 and
        // (I + A)^-1 = sum_{k<16} (-A)^k = (I - A)(I + A^2)(I + A^4)(I + A^8), exactly.
        // Products run on fp32 MFMA straight from accumulator-layout registers: with
        // k = 4g + s in step s, element s of the accumulator tile of X^T is the A operand
        // of X and element s of the tile of Y is the B operand of Y.
        float* a = &sm.at[wave * 16 * 20];
        f32x4 ac, at, id;                       // A, A^T, I in accumulator layout
        {
            const float4 x = *reinterpret_cast<const float4*>(&a[r * 20 + 4 * g]);   // A[r][4g + s]
            at = f32x4{x.x, x.y, x.z, x.w};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                ac[s] = a[(4 * g + s) * 20 + r];
                id[s] = (4 * g + s == r) ? 1.f : 0.f;
            }
        }
        auto mm = [](const f32x4& xt, const f32x4& y) {   // X Y from tiles of X^T and Y
            f32x4 c = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(xt[s], y[s], c, 0, 0, 0);
            return c;
        };
        const f32x4 b1 = mm(at, ac), b1t = mm(ac, at);          // A^2, (A^2)^T
        const f32x4 b2 = mm(b1t, b1), b2t = mm(b1, b1t);        // A^4, (A^4)^T
        const f32x4 b3 = mm(b2t, b2);                           // A^8
        // X1 = (I - A)(I + A^2) = I - A + A^2 - A A^2, as X1^T
        const f32x4 x1t = id - at + b1t - mm(b1, at);
        // X2^T = ((X1 (I + A^4)))^T = X1^T + (A^4)^T X1^T
        const f32x4 x2t = x1t + mm(b2, x1t);
        // T^T = X2^T + (A^8)^T X2^T; lane (r, g) holds T[r][4g + s], the A operand of T
        const f32x4 tt = x2t + mm(b3, x2t);
        // T_ww over this wave's own block (no other wave reads it), as a 16x16x16 A fragment
        *reinterpret_cast<uint2*>(&a[lane * 2]) = pack4(tt);
    }
    // right-hand sides diag(b) Kh (key channel tiles) and diag(b) V (value tiles),
    // channel-row layout: lane (r, g) of tile (rt, x) holds row 16rt + 4g + s, column
    // 16x + r. Token-row tiles are transposed exactly by the identity product.
    f32x4 yw[CW][4], yu[VW][4];
    float4 b4[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) b4[rt] = *reinterpret_cast<const float4*>(&sm.beta[16 * rt + 4 * g]);
    float* gam_out = reinterpret_cast<float*>(rec + Lay::G);
#pragma unroll
    for (int u = 0; u < CW; ++u) {
        const int ct = CW * wave + u;
        const float gam = sm.gam[16 * ct + r];
        if (g == 0) gam_out[16 * ct + r] = gam;
        uint2 kbp[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const f32x4 kh = EL::mma16(Frag16{lds4(sm.kr, 16 * rt + r, 16 * ct + 4 * g)}, ident, zero4());
            f32x4 kc = EL::mma16(Frag16{lds4(sm.qk, 16 * rt + r, 16 * ct + 4 * g)}, ident, zero4());
            kc = EL::mma16(Frag16{lds4(sm.kcl, 16 * rt + r, 16 * ct + 4 * g)}, ident, kc);
            // Kb = K exp(G_last - G) = gamma Kc
            kbp[rt] = pack4(gam * kc[0], gam * kc[1], gam * kc[2], gam * kc[3]);
#pragma unroll
            for (int s = 0; s < 4; ++s) yw[u][rt][s] = b4[rt][s] * kh[s];
        }
        // Kb^T fragments (ct, kb): token tiles 2kb (t = 0) and 2kb + 1 (t = 1)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
            *reinterpret_cast<uint4*>(rec + Lay::K + ((ct * 2 + kb) * 64 + lane) * 8) =
                make_uint4(kbp[2 * kb].x, kbp[2 * kb].y, kbp[2 * kb + 1].x, kbp[2 * kb + 1].y);
    }
#pragma unroll
    for (int u = 0; u < VW; ++u) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            const f32x4 vv = EL::mma16(Frag16{vraw[u][rt]}, ident, zero4());   // V[16rt + 4g + s][16vt + r]
#pragma unroll
            for (int s = 0; s < 4; ++s) yu[u][rt][s] = b4[rt][s] * vv[s];
        }
    }
    lds_barrier();

    // ===== phase 4: (I + A) X = Y by 16-row blocks, for this wave's tiles =====
    Frag16 tf[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) tf[ii].u = *reinterpret_cast<const uint2*>(&sm.at[ii * 16 * 20 + lane * 2]);
    auto solve = [&](f32x4 (&y)[4]) {
        Frag16 py[4];
        py[0] = EL::from_acc16(y[0]);
        EL::ready(py[0]);
        y[0] = EL::mma16(tf[0], py[0], zero4());
        py[0] = EL::from_acc16(y[0]);
        EL::ready(py[0]);
#pragma unroll
        for (int ii = 1; ii < 4; ++ii) {
            f32x4 acc = y[ii];
#pragma unroll
            for (int jj = 0; jj < ii; ++jj)
                acc = EL::mma16(Frag16{*reinterpret_cast<const uint2*>(&sm.aoff[((ii * (ii - 1)) / 2 + jj) * 256 + lane * 4])},
                                py[jj], acc);
            Frag16 pa = EL::from_acc16(acc);
            EL::ready(pa);
            y[ii] = EL::mma16(tf[ii], pa, zero4());
            if (ii < 3) {
                py[ii] = EL::from_acc16(y[ii]);
                EL::ready(py[ii]);
            }
        }
    };
#pragma unroll
    for (int u = 0; u < VW; ++u) {
        solve(yu[u]);
        const int vt = VW * wave + u;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
            *reinterpret_cast<uint2*>(rec + Lay::U + ((vt * 4 + rt) * 64 + lane) * 4) = pack4(yu[u][rt]);
    }
#pragma unroll
    for (int u = 0; u < CW; ++u) {
        solve(yw[u]);
        const int ct = CW * wave + u;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            // -W tile (rt, ct) in token rows: transpose with the identity product
            const f32x4 nw = -yw[u][rt];
            Frag16 pw = EL::from_acc16(nw);
            EL::ready(pw);
            const f32x4 wt = EL::mma16(pw, ident, zero4());   // W[16rt + r][16ct + 4g + s]
            *reinterpret_cast<uint2*>(rec + Lay::W + ((rt * NKB + ct / 2) * 64 + lane) * 8 + (ct & 1) * 4) = pack4(wt);
        }
    }
}

// ---------------------------------------------------------------------------
// chain: the state pass of one (sample, head, 64-column value tile)
// ---------------------------------------------------------------------------
// Waves 0-3 carry the state (16 value columns each, fp32 in registers; the code
// also allows two waves of 32 columns, which measured slower) and read a chunk's
// operands only from LDS; waves 4-7 move the next chunk's operands from the
// workspace into the other of two LDS buffers with global-to-LDS transfers.
constexpr int kStateWaves = 4;
constexpr int kLoadWaves = 4;
constexpr int kCThreads = (kStateWaves + kLoadWaves) * 64;

// MODE 0: one workgroup walks a whole sample.
// MODE 1 (sequence split, first pass): per segment that is not the last of its
// sample, the state reached from zero (S_loc, value tiles) and the segment's
// transition Phi (d_k columns: identity start, U taken as zero), written to sloc / phi.
// MODE 2 (second pass): per segment, the state on entry from the prefix
// S_in(k) = Phi(k-1) S_in(k-1) + S_loc(k-1) starting at the sample's initial state,
// then the segment's chunks with outputs; the last segment writes final_state.
template <int DK, int DV, int MODE>
__global__ __launch_bounds__(kCThreads) void kda_wy_chain_kernel(
    const uint16_t* ws, const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_off,
    const float* __restrict__ init_state, uint16_t* __restrict__ out, float* __restrict__ final_state,
    int num_seqs, int H, int64_t total_tokens, int max_chunks, const int32_t* __restrict__ seg_off,
    int lseg, int max_segs, float* __restrict__ sloc, float* __restrict__ phi)
{
    using EL = Elt<uint16_t>;
    using Frag = EL::Frag;
    using Lay = WyLayout<DK, DV>;
    constexpr int NKB = Lay::NKB, NCT = Lay::NCT;
    constexpr int NVT64 = DV / 64;
    constexpr int CPW = 4 / kStateWaves;           // 16-column tiles per state wave
    constexpr int SH16 = Lay::SHARED * 2 / 16;     // 16-byte pieces of the shared operands
    constexpr int U16 = Lay::UTILE * 2 / 16;       // 16-byte pieces of this tile's U
    constexpr int NP = SH16 + U16;
    constexpr int LT = kLoadWaves * 64;            // loading threads
    constexpr int PER = (NP + LT - 1) / LT;        // pieces per loading thread
    constexpr int BUF = PER * LT;                  // pieces per LDS buffer (padded)

    extern __shared__ __align__(16) unsigned char smem_raw[];
    u32x4* lds = reinterpret_cast<u32x4*>(smem_raw);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    const bool loader = wave >= kStateWaves;
    const int ltid = tid - kStateWaves * 64;

    // the column tiles of one unit are 8 blocks apart: same XCD, shared L2
    constexpr int NT = MODE == 1 ? NVT64 + DK / 64 : NVT64;      // column tiles per unit
    const int b = blockIdx.x;
    const int tile = (b >> 3) % NT;
    const int unit = (b / (8 * NT)) * 8 + (b & 7);
    const bool trans = MODE == 1 && tile >= NVT64;               // a tile of Phi
    const int vt = trans ? 0 : tile;                             // value tile of U to load
    int n, h, seg = 0, nseg = 1, sid = 0;
    if constexpr (MODE == 0) {
        if (unit >= num_seqs * H) return;
        n = unit / H;
        h = unit % H;
    } else {
        const int ns = min(seg_off[num_seqs], max_segs);        // the workspace holds max_segs segments
        if (unit >= ns * H) return;
        sid = unit / H;
        h = unit % H;
        int lo = 0, hi = num_seqs;              // seg_off[lo] <= sid < seg_off[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (seg_off[mid] <= sid) lo = mid; else hi = mid;
        }
        n = lo;
        seg = sid - seg_off[n];
        nseg = seg_off[n + 1] - seg_off[n];
        if (MODE == 1 && seg == nseg - 1) return;                // the last segment needs no transition
    }
    int c0, c1;
    if (!chunk_off) {                           // small pack: the wave forms the chunk table
        const int incl = wave_chunk_scan(cu, num_seqs, total_tokens, lane);
        c0 = min(n > 0 ? __shfl(incl, n - 1) : 0, max_chunks);
        c1 = min(__shfl(incl, n), max_chunks);
    } else {
        c0 = min(chunk_off[n], max_chunks);
        c1 = min(chunk_off[n + 1], max_chunks);
    }
    if constexpr (MODE != 0) {
        c0 = min(c0 + seg * lseg, c1);
        c1 = min(c0 + lseg, c1);
    }
    const int nch = c1 - c0;
    int64_t s0, s1;
    sample_bounds(cu, n, total_tokens, s0, s1);
    if constexpr (MODE != 0) s0 += int64_t(seg) * lseg * kWC;    // first token of the segment
    // loading waves: piece j of a chunk goes straight from the workspace to LDS
    // (global_load_lds_dwordx4: each lane's 16 bytes land at the wave's LDS base + 16 *
    // lane); pieces past NP re-read the last piece into the buffer's padding
    const int lw = wave - kStateWaves;         // loading wave index
    int src[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int idx = min(ltid + j * LT, NP - 1);
        src[j] = idx + (idx >= SH16 ? vt * U16 : 0);
    }
    // 64-piece blocks a pass never reads are skipped: P fragments (rt, kb) = (0, 1) and
    // (1, 1) lie above the diagonal (never written, never read); the first pass of the
    // sequence split writes no output (no Qh, no P), and its transition tiles take U as zero
    static_assert(Lay::P % 512 == 0, "P fragments start on a 64-piece block");
    auto needed = [&](int b0) {
        const bool p_upper = b0 == Lay::P / 8 + 64 || b0 == Lay::P / 8 + 3 * 64;
        if constexpr (MODE != 1) return !p_upper;
        const bool in_q = b0 >= Lay::Q / 8 && b0 + 64 <= Lay::K / 8;
        const bool in_p = b0 >= Lay::P / 8 && b0 + 64 <= Lay::G / 8;
        const bool in_u = b0 >= SH16;
        return !(in_q || in_p || (trans && in_u));
    };
    auto dma = [&](int i, int bi) __attribute__((always_inline)) {
        const int cc = c0 + min(i, nch - 1);
        const u32x4* rec = reinterpret_cast<const u32x4*>(ws + (int64_t(h) * max_chunks + cc) * Lay::TOTAL);
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (needed(lw * 64 + j * LT))
                __builtin_amdgcn_global_load_lds(
                    (__attribute__((address_space(1))) void*)(rec + src[j]),
                    (__attribute__((address_space(3))) void*)(lds + bi * BUF + lw * 64 + j * LT), 16, 0, 0);
    };
    // wait for this wave's transfers to land in LDS, then hand the buffer over
    auto dma_barrier = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
    };

    // one chunk of products from LDS buffer bi, for this wave's CPW column tiles
    auto products = [&](f32x4 (&S)[CPW][NCT], int i, int bi) __attribute__((always_inline)) {
        const uint16_t* sl = reinterpret_cast<const uint16_t*>(lds + bi * BUF);
        Frag sf[CPW][NKB];                      // S as the B operand over key channels
#pragma unroll
        for (int j = 0; j < CPW; ++j)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) sf[j][kb] = EL::from_acc(S[j][2 * kb], S[j][2 * kb + 1]);
#pragma unroll
        for (int j = 0; j < CPW; ++j)
#pragma unroll
            for (int kb = 0; kb < NKB; kb += 2) EL::ready(sf[j][kb], sf[j][kb + 1]);
        // Vn = U - W S: tile (j, rt) holds Vn[16rt + 4g + s][16 vc_j + r]
        f32x4 X[CPW][4];
#pragma unroll
        for (int j = 0; j < CPW; ++j)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                float u4[4];
                unpack4(*reinterpret_cast<const uint2*>(sl + Lay::SHARED + (((CPW * wave + j) * 4 + rt) * 64 + lane) * 4), u4);
                X[j][rt] = trans ? zero4() : f32x4{u4[0], u4[1], u4[2], u4[3]};
            }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const Frag wf{*reinterpret_cast<const uint4*>(sl + Lay::W + ((rt * NKB + kb) * 64 + lane) * 8)};
#pragma unroll
                for (int j = 0; j < CPW; ++j) X[j][rt] = EL::mma(wf, sf[j][kb], X[j][rt]);
            }
        // O^T = S^T Qh^T + Vn^T P^T: tile (j, rt) holds O[16rt + r][16 vc_j + 4g + s]
        f32x4 O[CPW][4];
#pragma unroll
        for (int j = 0; j < CPW; ++j)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) O[j][rt] = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const Frag qf{*reinterpret_cast<const uint4*>(sl + Lay::Q + ((rt * NKB + kb) * 64 + lane) * 8)};
#pragma unroll
                for (int j = 0; j < CPW; ++j) O[j][rt] = EL::mma(sf[j][kb], qf, O[j][rt]);
            }
        Frag vf[CPW][2];
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
            vf[j][0] = EL::from_acc(X[j][0], X[j][1]);
            vf[j][1] = EL::from_acc(X[j][2], X[j][3]);
            EL::ready(vf[j][0], vf[j][1]);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int kb = 0; kb <= rt / 2; ++kb) {
                const Frag pf{*reinterpret_cast<const uint4*>(sl + Lay::P + ((rt * 2 + kb) * 64 + lane) * 8)};
#pragma unroll
                for (int j = 0; j < CPW; ++j) O[j][rt] = EL::mma(vf[j][kb], pf, O[j][rt]);
            }
        // S <- diag(gamma) S + Kb^T Vn
        const float* gam = reinterpret_cast<const float*>(sl + Lay::G);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            const float4 g4 = *reinterpret_cast<const float4*>(gam + 16 * ct + 4 * g);
#pragma unroll
            for (int j = 0; j < CPW; ++j) {
                S[j][ct][0] *= g4.x; S[j][ct][1] *= g4.y; S[j][ct][2] *= g4.z; S[j][ct][3] *= g4.w;
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const Frag kf{*reinterpret_cast<const uint4*>(sl + Lay::K + ((ct * 2 + kb) * 64 + lane) * 8)};
#pragma unroll
                for (int j = 0; j < CPW; ++j) S[j][ct] = EL::mma(kf, vf[j][kb], S[j][ct]);
            }
        }
        // output rows of this chunk
        if constexpr (MODE != 1) {
            const int64_t t0 = s0 + int64_t(i) * kWC;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int64_t t = t0 + 16 * rt + r;
                if (t < s1) {
#pragma unroll
                    for (int j = 0; j < CPW; ++j)
                        *reinterpret_cast<uint2*>(out + (t * H + h) * DV + 16 * (4 * vt + CPW * wave + j) + 4 * g) = pack4(O[j][rt]);
                }
            }
        }
    };

    // The two roles run separate loops with the same barrier sequence (one barrier
    // after the prologue and one per chunk). In iteration i the state waves read
    // buffer i & 1 while the loading waves fill buffer (i + 1) & 1, freed by chunk i - 1.
    if (loader) {
        if (nch > 0) dma(0, 0);
        dma_barrier();
       
        for (int i = 0; i < nch; ++i) {
            if (i + 1 < nch) dma(i + 1, (i + 1) & 1);
           
            dma_barrier();
           
        }
        return;
    }

    // column c of this wave's tile j: 16 * (4 * tile + CPW * wave + j) + r
    f32x4 S[CPW][NCT];
#pragma unroll
    for (int j = 0; j < CPW; ++j)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) S[j][ct] = zero4();
    if (trans) {                                // Phi starts at the identity
#pragma unroll
        for (int j = 0; j < CPW; ++j)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    S[j][ct][s] = (16 * ct + 4 * g + s == 16 * (4 * (tile - NVT64) + CPW * wave + j) + r) ? 1.f : 0.f;
    } else if (init_state && MODE != 1) {
#pragma unroll
        for (int j = 0; j < CPW; ++j)
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct) {
                const float* st = init_state + ((int64_t(n) * H + h) * DK + 16 * ct + 4 * g) * DV +
                                  16 * (4 * vt + CPW * wave + j) + r;
#pragma unroll
                for (int s = 0; s < 4; ++s) S[j][ct][s] = st[s * DV];
            }
    }
    if constexpr (MODE == 2) {
        // S_in(seg) = Phi(k) S_in(k) + S_loc(k) for k < seg, with hi/lo bf16 operands
        for (int kseg = 0; kseg < seg; ++kseg) {
            const int64_t ks = int64_t(seg_off[n] + kseg) * H + h;
            const float* ph = phi + ks * DK * DK;
            const float* sl0 = sloc + ks * DK * DV;
#pragma unroll
            for (int j = 0; j < CPW; ++j) {
                const int colj = 16 * (4 * vt + CPW * wave + j) + r;
                Frag shi[NKB], slo[NKB];
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    f32x4 l0, l1;
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        l0[s] = S[j][2 * kb][s] - bf2f(f2bf(S[j][2 * kb][s]));
                        l1[s] = S[j][2 * kb + 1][s] - bf2f(f2bf(S[j][2 * kb + 1][s]));
                    }
                    shi[kb] = EL::from_acc(S[j][2 * kb], S[j][2 * kb + 1]);
                    slo[kb] = EL::from_acc(l0, l1);
                    EL::ready(shi[kb], slo[kb]);
                }
#pragma unroll
                for (int ct = 0; ct < NCT; ++ct) {
                    f32x4 acc;
#pragma unroll
                    for (int s = 0; s < 4; ++s) acc[s] = sl0[int64_t(16 * ct + 4 * g + s) * DV + colj];
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) {
                        // Phi rows 16ct + r, k = 32kb + 16t + 4g + i, as hi and lo A operands
                        const float* pr = ph + int64_t(16 * ct + r) * DK + 32 * kb + 4 * g;
                        const float4 p0 = *reinterpret_cast<const float4*>(pr);
                        const float4 p1 = *reinterpret_cast<const float4*>(pr + 16);
                        const f32x4 a0{p0.x, p0.y, p0.z, p0.w}, a1{p1.x, p1.y, p1.z, p1.w};
                        f32x4 b0, b1;
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            b0[s] = a0[s] - bf2f(f2bf(a0[s]));
                            b1[s] = a1[s] - bf2f(f2bf(a1[s]));
                        }
                        Frag ahi = EL::from_acc(a0, a1), alo = EL::from_acc(b0, b1);
                        EL::ready(ahi, alo);
                        acc = EL::mma(ahi, shi[kb], acc);
                        acc = EL::mma(ahi, slo[kb], acc);
                        acc = EL::mma(alo, shi[kb], acc);
                    }
                    S[j][ct] = acc;     // safe: later ct read only shi / slo, taken before the loop
                }
            }
        }
    }
    lds_barrier();
   
    for (int i = 0; i < nch; ++i) {
        products(S, i, i & 1);
       
        lds_barrier();
       
    }
    if constexpr (MODE == 1) {
        // segment result: S_loc (value tiles) or Phi (transition tiles)
        const int64_t ks = int64_t(sid) * H + h;
        float* dst = trans ? phi + ks * DK * DK : sloc + ks * DK * DV;
        const int ld = trans ? DK : DV;
        const int tc = trans ? tile - NVT64 : vt;
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
            float* fs = dst + 16 * (4 * tc + CPW * wave + j) + r;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int s = 0; s < 4; ++s) fs[int64_t(16 * ct + 4 * g + s) * ld] = S[j][ct][s];
        }
    } else if (final_state && seg == nseg - 1) {
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
            float* fs = final_state + ((int64_t(n) * H + h) * DK) * DV + 16 * (4 * vt + CPW * wave + j) + r;
#pragma unroll
            for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
                for (int s = 0; s < 4; ++s) fs[int64_t(16 * ct + 4 * g + s) * DV] = S[j][ct][s];
        }
    }
}

// LDS of the chain kernel: two buffers of one chunk's operands, each padded to whole
// 16-byte pieces per loading thread
template <int DK, int DV>
constexpr size_t chain_smem() {
    constexpr int np = (WyLayout<DK, DV>::SHARED + WyLayout<DK, DV>::UTILE) * 2 / 16;
    constexpr int lt = kLoadWaves * 64;
    return 2 * size_t((np + lt - 1) / lt) * lt * 16;
}

struct WyPlan {
    int max_chunks;
    int lseg;          // chunks per segment of the sequence split; 0 = no split
    int max_segs;
    size_t table_bytes, rec_bytes, sloc_bytes, phi_bytes;
};

template <int DK, int DV, int MODE>
hipError_t launch_chain(const LaunchArgs& a, const uint16_t* ws, const int32_t* chunk_off, const int32_t* seg_off,
                        const WyPlan& p, float* sloc, float* phi)
{
    constexpr size_t smem = chain_smem<DK, DV>();
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda_wy_chain_kernel<DK, DV, MODE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
    const int nt = MODE == 1 ? (DV + DK) / 64 : DV / 64;
    const int units = (MODE == 0 ? a.num_seqs : p.max_segs) * a.num_heads;
    const int blocks = ((units + 7) / 8) * 8 * nt;
    hipLaunchKernelGGL((kda_wy_chain_kernel<DK, DV, MODE>), dim3(blocks), dim3(kCThreads), smem, a.stream,
                       ws, a.cu_seqlens, chunk_off, a.init_state, static_cast<uint16_t*>(a.out), a.final_state,
                       a.num_seqs, a.num_heads, a.total_tokens, p.max_chunks, seg_off, p.lseg, p.max_segs,
                       sloc, phi);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_dims(const LaunchArgs& a, uint16_t* ws, const int32_t* chunk_off, const int32_t* seg_off,
                       const WyPlan& p, float* sloc, float* phi, TimingHook* th)
{
    dim3 pgrid(p.max_chunks, a.num_heads);
    if (th) th->begin("prep", a.stream);
    auto prep = a.qk_l2norm ? kda_wy_prep_kernel<DK, DV, true> : kda_wy_prep_kernel<DK, DV, false>;
    hipLaunchKernelGGL(prep, pgrid, dim3(kWThreads), 0, a.stream,
                       static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                       static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.log_alpha),
                       static_cast<const uint16_t*>(a.beta), a.cu_seqlens, chunk_off, ws, a.num_seqs,
                       a.num_heads, a.total_tokens, p.max_chunks);
    if (th) th->end(a.stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.lseg == 0) {
        if (th) th->begin("chain", a.stream);
        e = launch_chain<DK, DV, 0>(a, ws, chunk_off, seg_off, p, sloc, phi);
        if (th) th->end(a.stream);
        return e;
    }
    if (th) th->begin("segments", a.stream);
    e = launch_chain<DK, DV, 1>(a, ws, chunk_off, seg_off, p, sloc, phi);
    if (th) th->end(a.stream);
    if (e != hipSuccess) return e;
    if (th) th->begin("chain", a.stream);
    e = launch_chain<DK, DV, 2>(a, ws, chunk_off, seg_off, p, sloc, phi);
    if (th) th->end(a.stream);
    return e;
}

// Sequence split: when the samples give at most 64 chain workgroups (a quarter of the
// CUs or less), each sample is cut into segments of lseg chunks so that about 256
// workgroups run the second pass.
WyPlan make_plan(int64_t total_tokens, int32_t num_seqs, int32_t num_heads, int d_k, int d_v)
{
    WyPlan p{};
    const int64_t chunks_bound = (total_tokens + kWC - 1) / kWC;
    p.max_chunks = int(chunks_bound + num_seqs);
    const int64_t chain_units = int64_t(num_seqs) * num_heads * (d_v / 64);
    p.lseg = 0;
    if (chain_units <= 64) {
        const int64_t segs = std::max<int64_t>(1, 256 / (int64_t(num_heads) * (d_v / 64)));
        const int64_t lseg = std::max<int64_t>(32, (chunks_bound + segs - 1) / segs);
        if (lseg < chunks_bound) p.lseg = int(lseg);
    }
    p.max_segs = p.lseg ? int((chunks_bound + num_seqs + p.lseg - 1) / p.lseg + num_seqs) : num_seqs;
    const size_t tab = 2 * (size_t(num_seqs) + 1) * sizeof(int32_t);
    p.table_bytes = (tab + 255) & ~size_t(255);
    p.rec_bytes = size_t(p.max_chunks) * size_t(num_heads) * wy_record_bytes(d_k, d_v);
    p.sloc_bytes = p.lseg ? size_t(p.max_segs) * num_heads * d_k * d_v * sizeof(float) : 0;
    p.phi_bytes = p.lseg ? size_t(p.max_segs) * num_heads * d_k * d_k * sizeof(float) : 0;
    return p;
}

}  // namespace

size_t wy_record_bytes(int d_k, int d_v)
{
    if (d_k == 128 && d_v == 128) return size_t(WyLayout<128, 128>::TOTAL) * 2;
    if (d_k == 128 && d_v == 64) return size_t(WyLayout<128, 64>::TOTAL) * 2;
    if (d_k == 64 && d_v == 128) return size_t(WyLayout<64, 128>::TOTAL) * 2;
    return size_t(WyLayout<64, 64>::TOTAL) * 2;
}

size_t wy_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_heads, int d_k, int d_v)
{
    const WyPlan p = make_plan(total_tokens, num_seqs, num_heads, d_k, d_v);
    return p.table_bytes + p.rec_bytes + p.sloc_bytes + p.phi_bytes;
}

hipError_t launch_forward_wy(const LaunchArgs& a, void* workspace, TimingHook* th)
{
    const WyPlan p = make_plan(a.total_tokens, a.num_seqs, a.num_heads, a.d_k, a.d_v);
    if (int64_t(p.max_chunks) * a.num_heads > 0x7FFFFFFF / 8) return hipErrorInvalidValue;
    char* base = static_cast<char*>(workspace);
    int32_t* chunk_off = reinterpret_cast<int32_t*>(base);
    int32_t* seg_off = chunk_off + (a.num_seqs + 1);
    uint16_t* ws = reinterpret_cast<uint16_t*>(base + p.table_bytes);
    float* sloc = p.lseg ? reinterpret_cast<float*>(base + p.table_bytes + p.rec_bytes) : nullptr;
    float* phi = p.lseg ? reinterpret_cast<float*>(base + p.table_bytes + p.rec_bytes + p.sloc_bytes) : nullptr;

    if (p.lseg == 0 && a.num_seqs <= 64) {
        chunk_off = nullptr;                    // the kernels form the chunk table per wave
    } else {
        if (th) th->begin("plan", a.stream);
        hipLaunchKernelGGL(kda_wy_plan_kernel, dim3(1), dim3(1024), 0, a.stream, a.cu_seqlens, chunk_off, seg_off,
                           a.num_seqs, a.total_tokens, p.lseg);
        if (th) th->end(a.stream);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }

    if (a.d_k == 128 && a.d_v == 128) return launch_dims<128, 128>(a, ws, chunk_off, seg_off, p, sloc, phi, th);
    if (a.d_k == 128 && a.d_v == 64) return launch_dims<128, 64>(a, ws, chunk_off, seg_off, p, sloc, phi, th);
    if (a.d_k == 64 && a.d_v == 128) return launch_dims<64, 128>(a, ws, chunk_off, seg_off, p, sloc, phi, th);
    return launch_dims<64, 64>(a, ws, chunk_off, seg_off, p, sloc, phi, th);
}

}  // namespace kda
