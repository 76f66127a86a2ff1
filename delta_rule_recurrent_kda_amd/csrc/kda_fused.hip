// kda_fused.hip -- single-pass chunkwise KDA forward for bf16 data, d_k = d_v = 128 (gfx950).
//
// Recurrence (Chimera, arXiv 2607.28611: update printed in the explainer page, "One
// stream, three mechanisms, no positions"; state reset at every packed sample, paper
// Sec. 3 KDA paragraph), per (sample, head):
//     S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,   o_t = S_t^T q_t.
// Chunkwise form over chunks of C = 32 tokens (G = inclusive cumsum of log a over the
// chunk's rows, per key channel; gamma = exp(G of the last row)):
//     Qh = Q e^G, Kh = K e^G, Kc = K e^-G, Kb = gamma Kc
//     A = StrictLower(diag(b) Kh Kc^T),  T = (I + A)^-1
//     X = T diag(b) (V - Kh S),  O = Qh S + LowerIncl(Qh Kc^T) X,  S <- diag(gamma) S + Kb^T X
// (X = U - W S of the WY form with W = T diag(b) Kh, U = T diag(b) V, taken the other way
// round: the residual V - Kh S is formed first and solved once, so W and U are never built).
//
// One workgroup of 8 wave64s owns one (sample segment, head); q, k, v, log a and beta are
// read once and the output written once. The waves split into two roles that work on
// consecutive chunks at the same time, handing operands over through double-buffered LDS,
// with two workgroup barriers per chunk:
//   producers (waves 4-7; wave 4 + p owns key channels and value columns 32p..32p+31)
//     before the first barrier: chunk c + 1's rows from 16-byte row loads (chunk c + 2's
//     loads go out as registers fall free): G by a product with a triangular ones matrix,
//     the decayed rows, -diag(b) Kh and Qh as fragments, Kb and diag(b) V transposed, the
//     slab's share of A and P (products over the slab's 32 channels) and of diag(P) = q.k
//     (the output pass forms only token tile 1 before it, and tile 0, the shares and the
//     transposes after it);
//     in the summary pass, after it: the sums of the shares and the inverses of the two
//     diagonal blocks of I + A (each block's columns split over two waves), -A10 (wave 6);
//   consumers (waves 0-3; wave j owns value columns 32j..32j+31) carry their columns of
//     S (fp32, registers) through chunk c: in the output pass they first sum the shares into
//     the inverses of the diagonal blocks (waves 0, 1), -A10 (wave 2) and P (wave 3); then
//     Z = diag(b) (V - Kh S) and Qh S before the first barrier, X = T Z by 16-row blocks
//     (X0 = T00 Z0, X1 = T11 (Z1 - A10 X0)), O += P X, the output, and the state update.
// Operand layouts are chosen so that every hand-over is a lane-ordered LDS store and load
// and every transpose is an exact product with the identity (bf16 values).
//
// The inverse of a diagonal block (16x16, I + A with A strictly lower) is formed in fp32 by
// elimination: lane (r, g) holds row r of A and T[r][4g..4g+3]; for k = 0..14 row k of T
// is final, is broadcast along the 16 lanes of each row by DPP, and every row r > k takes
// -A[r][k] T[k][.] (15 steps of 4 broadcasts and 4 FMAs).
//
// Long samples (few (sample, head) units for the CUs): the sample is cut into segments.
//   pass 1  per segment that is not its sample's last: the state reached from zero
//           (S_loc) and the segment's transition Phi (the same chunk pass on a d_k-column
//           state started at the identity with V taken as zero), no output;
//   combine per (sample, head, 32 value columns): S_in(k+1) = Phi(k) S_in(k) + S_loc(k)
//           from the sample's initial state, with hi/lo bf16 operands;
//   pass 2  every segment from its S_in with outputs; the last one writes final_state.
//
// Fragment conventions: see kda_device.h. Here an operand over 32 channels of one slab
// holds, in lane (r, g), the 8 contiguous channels 8g..8g+7 of row r (a 16-byte load),
// and both operands of a product use that order. Transposed (channel-row) tiles come out
// of products with the identity on half-slabs: virtual column c of half t is channel
// 8(c/4) + 4t + c%4 of the slab. The consumers' state uses the same orders: key tile
// kt = 2p + t, row m is key 32p + 8(m/4) + 4t + m%4; value half th of consumer j, column
// c is value column 32j + 8(c/4) + 4th + c%4.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <type_traits>
#include <utility>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {
using namespace dev;
using EL = Elt<uint16_t>;
using Frag = EL::Frag;
using Frag16 = EL::Frag16;

constexpr int kFC = 32;            // tokens per chunk
constexpr int kFD = 128;           // d_k = d_v
constexpr int kFThreads = 512;     // 4 consumer + 4 producer wave64
constexpr uint16_t kOneBf = 0x3F80;
constexpr int kFCounters = 4;      // unit counters of the persistent passes (one per pass)
constexpr int kCombThreads = 256;  // combine: 4 wave64 per (sample, head, kCombCT 16-column value tiles)
constexpr int kCombCT = 2;         // value tiles per combine workgroup (each Phi fragment serves all of them)

// one chunk's operands for the state pass, every array in lane order
struct Buf {
    uint4 qf[2][4][64];    // Qh B fragments [token tile][key slab][lane]
    uint4 yk[2][4][64];    // -Kh A fragments [token tile][key slab][lane]
    uint4 kf[8][64];       // Kc^T A fragments [key tile][lane]
    uint4 yv[4][2][64];    // V, tokens down the rows [value slab][half][lane]
    uint4 pf[2][64];       // P^T B fragments [token tile][lane]
    uint2 tf[3][64];       // (I + A_00)^-1, (I + A_11)^-1, -A_10 as 16x16x16 A fragments
    float gam[kFD];        // gamma per key channel
    float beta[kFC];       // beta per token (0 past the sample's end)
};
struct FusedSmem {
    Buf buf[2];
    f32x4 part[2][4][6][64];  // per chunk (two in flight) and producer slab: partial A and P^T blocks
    float ablk[4][16][20]; // the diagonal blocks of A (rows, fp32, padded) for the inverses, one per inverting wave
    float ssq[2][4][kFC];  // sums of squares of q and k per (slab, token)
    float dpp[2][4][kFC];  // per chunk (two in flight): q.k per (slab, token), the diagonal of P
};

__device__ __forceinline__ uint32_t bfbits_lo(uint32_t u) { return u << 16; }
__device__ __forceinline__ uint32_t bfbits_hi(uint32_t u) { return u & 0xFFFF0000u; }
__device__ __forceinline__ void unpack8(const uint4& u, float (&f)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = __uint_as_float(bfbits_lo(w[j]));
        f[2 * j + 1] = __uint_as_float(bfbits_hi(w[j]));
    }
}
__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
    return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
}
__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
    return make_uint2(pack2(a, b), pack2(c, d));
}
__device__ __forceinline__ uint2 half_of(const uint4& u, int t) {
    return t ? make_uint2(u.z, u.w) : make_uint2(u.x, u.y);
}
// the 8 values as hi and lo bf16 parts (x = hi + lo up to the rounding of lo)
__device__ __forceinline__ void split8(const float (&f)[8], uint4& hi, uint4& lo) {
    hi = pack8(f);
    const uint32_t w[4] = {hi.x, hi.y, hi.z, hi.w};
    float r[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        r[2 * j] = f[2 * j] - __uint_as_float(bfbits_lo(w[j]));
        r[2 * j + 1] = f[2 * j + 1] - __uint_as_float(bfbits_hi(w[j]));
    }
    lo = pack8(r);
}

// One elimination step of the block inverse: row KK of T (lanes KK of each 16-lane row,
// broadcast by DPP row_newbcast) leaves every row r > KK with -A[r][KK] T[KK][.].
template <int KK>
__device__ __forceinline__ void elim_step(float (&t)[4], const float (&ar)[16], int r) {
    const float a = r > KK ? -ar[KK] : 0.f;
    float tk[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        tk[m] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(t[m]), 0x150 + KK, 0xF, 0xF, false));
#pragma unroll
    for (int m = 0; m < 4; ++m) t[m] = fmaf(a, tk[m], t[m]);
}
template <int... KK>
__device__ __forceinline__ void elim_rows(float (&t)[4], const float (&ar)[16], int r, std::integer_sequence<int, KK...>) {
    (elim_step<KK>(t, ar, r), ...);
}
// The same on two columns per lane (half of the block's columns per wave)
template <int KK>
__device__ __forceinline__ void elim_step2(float (&t)[2], const float (&ar)[16], int r) {
    const float a = r > KK ? -ar[KK] : 0.f;
    float tk[2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
        tk[m] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(t[m]), 0x150 + KK, 0xF, 0xF, false));
#pragma unroll
    for (int m = 0; m < 2; ++m) t[m] = fmaf(a, tk[m], t[m]);
}
template <int... KK>
__device__ __forceinline__ void elim_rows2(float (&t)[2], const float (&ar)[16], int r, std::integer_sequence<int, KK...>) {
    (elim_step2<KK>(t, ar, r), ...);
}

// Orders one wave's LDS writes before its later reads of other lanes' data: the LDS
// executes a wave's instructions in order; the clobber keeps the compiler from moving them.
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

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
                                                              int64_t T, int lseg, int* __restrict__ counters)
{
    __shared__ int32_t part[1024];
    const int tid = threadIdx.x;
    if (tid < kFCounters) counters[tid] = 0;        // the passes' unit counters
    if (seg_off == nullptr) return;
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

// a value that is the same in every lane, moved to scalar registers
__device__ __forceinline__ int64_t uniform64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x) >> 32));
    return int64_t((uint64_t(hi) << 32) | lo);
}
// buffer resource word 3 for raw (untyped) loads on gfx9-family parts; loads past the
// resource's byte range return zeros
constexpr int kBufFlags = 0x00020000;

// key of row m of the consumers' key tile kt; value column c of half th of consumer j
__device__ __forceinline__ int key_of(int kt, int m) { return 32 * (kt >> 1) + 8 * (m >> 2) + 4 * (kt & 1) + (m & 3); }
__device__ __forceinline__ int col_of(int j, int th, int c) { return 32 * j + 8 * (c >> 2) + 4 * th + (c & 3); }

// raw rows of one chunk for producer slab p: token tiles 0 and 1, lane (r, g) = row r,
// channels 32p + 8g .. +7; b = beta of tokens r and 16 + r
struct Raw {
    uint4 q[2], k[2], l[2], v[2];
    uint16_t b[2];
};

// An empty asm that takes the rows as read-write operands: code that uses them cannot be
// scheduled before it (and it is ordered after the barriers before it).
__device__ __forceinline__ void pin_raw(Raw& x) {
    auto q0 = as_v(x.q[0]), q1 = as_v(x.q[1]), k0 = as_v(x.k[0]), k1 = as_v(x.k[1]);
    auto l0 = as_v(x.l[0]), l1 = as_v(x.l[1]), v0 = as_v(x.v[0]), v1 = as_v(x.v[1]);
    asm volatile("" : "+v"(q0), "+v"(q1), "+v"(k0), "+v"(k1), "+v"(l0), "+v"(l1), "+v"(v0), "+v"(v1),
                 "+v"(x.b[0]), "+v"(x.b[1]));
    from_v(x.q[0], q0); from_v(x.q[1], q1); from_v(x.k[0], k0); from_v(x.k[1], k1);
    from_v(x.l[0], l0); from_v(x.l[1], l1); from_v(x.v[0], v0); from_v(x.v[1], v1);
}

// ---------------------------------------------------------------------------
// PASS 0: one segment per sample, outputs. PASS 1: segment summaries (S_loc, Phi), no
// output. PASS 2: segments from their entry state, outputs.
// ---------------------------------------------------------------------------
template <int PASS, bool NORM, bool CONSUMER>
__device__ __forceinline__ void fused_unit(
    FusedSmem& sm, const int lin, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ la, const uint16_t* __restrict__ beta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ seg_off, const float* __restrict__ init_state,
    const float* __restrict__ carry, uint16_t* __restrict__ out, float* __restrict__ final_state,
    float* __restrict__ sloc, float* __restrict__ phi, int num_seqs, int H, int64_t T, int lseg, int max_segs)
{
    constexpr bool kOut = PASS != 1;
    // Who sums the partial products and inverts the diagonal blocks of I + A: with outputs,
    // the consumers, at the start of the chunk's own iteration (their first interval has room
    // next to the producers' decay work); without, the producers in their second interval
    // (the consumers' second interval then carries the state and the transition).
    constexpr bool kConsInv = PASS != 1;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: role and slab in SGPRs
    const int r = lane & 15, g = lane >> 4;

    // unit -> (segment, head): the heads of a segment are consecutive units
    const int sid = lin / H, h = lin % H;
    Seg sg;
    if (!find_segment(sid, cu, seg_off, num_seqs, T, lseg, max_segs, lane, sg)) return;
    if (PASS == 1 && sg.seg == sg.nseg - 1) return;          // the last segment needs no summary
    int64_t s0, s1;
    bounds(cu, sg.n, T, s0, s1);
    // the chunk range is the same on every lane: in scalar registers, the chunk's part of a
    // load's offset is a scalar operand (a per-lane one makes the compiler loop over lanes)
    const int nch = int((s1 - s0 + kFC - 1) / kFC);
    const int c0 = __builtin_amdgcn_readfirstlane(lseg > 0 ? min(sg.seg * lseg, nch) : 0);
    const int c1 = __builtin_amdgcn_readfirstlane(lseg > 0 ? min(c0 + lseg, nch) : nch);

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

    if constexpr (CONSUMER) {
        // ================= consumer: value columns of consumer j = w =================
        const int j = w;
        // S[kt][th]: rows key_of(kt, 4g + i), column col_of(j, th, r). PASS 1 also carries
        // Phi's columns (keys col_of(j, th, r)), from the identity.
        f32x4 S[8][2], Ph[PASS == 1 ? 8 : 1][PASS == 1 ? 2 : 1];
        {
            const float* src = nullptr;
            if (PASS == 2 && sg.seg > 0) src = carry + (int64_t(sid - 1) * H + h) * kFD * kFD;
            else if (PASS != 1 && init_state) src = init_state + (int64_t(sg.n) * H + h) * kFD * kFD;
#pragma unroll
            for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                for (int th = 0; th < 2; ++th)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = key_of(kt, 4 * g + i), col = col_of(j, th, r);
                        S[kt][th][i] = src ? src[key * kFD + col] : 0.f;
                        if constexpr (PASS == 1) Ph[kt][th][i] = key == col ? 1.f : 0.f;
                    }
        }
        // iteration it: chunk it of the segment (the producers form chunk it + 1)
        for (int it = c0 - 1; it < c1; ++it) {
            const bool run = it >= c0;
            const Buf& bf = sm.buf[it & 1];
            const int64_t t0 = s0 + int64_t(it) * kFC;
            f32x4 Z[2][2], ZP[PASS == 1 ? 2 : 1][PASS == 1 ? 2 : 1], O[2][2];
            if constexpr (NORM) lds_barrier();
            if (kConsInv && run) {
                // ---- chunk it's sums of the producers' partial products: the inverses of the two
                //      diagonal blocks of I + A (waves 0, 1), -A10 (wave 2), P (wave 3) ----
                Buf& bw = sm.buf[it & 1];
                const f32x4(*part)[6][64] = sm.part[it & 1];
                if (j < 2) {
                    // A_jj = StrictLower(diag(b) Kh Kc^T) of diagonal block j, rows to LDS
                    {
                        f32x4 n = zero4();
#pragma unroll
                        for (int x = 0; x < 4; ++x) n += part[x][j][lane];
                        const float4 b4 = *reinterpret_cast<const float4*>(&bw.beta[16 * j + 4 * g]);
                        const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                        for (int i = 0; i < 4; ++i) sm.ablk[j][4 * g + i][r] = 4 * g + i > r ? bb[i] * n[i] : 0.f;
                    }
                    lds_wait();
                    // T = (I + A_jj)^-1 in fp32 by elimination: lane (r, g) holds row r of A and
                    // T[r][4g..4g+3]; for k = 0..14 row k is final and every row below it takes
                    // -A[r][k] T[k][.], with T[k][.] broadcast along the lanes of the row (DPP)
                    float ar[16];
#pragma unroll
                    for (int k4 = 0; k4 < 4; ++k4) {
                        const float4 a4 = *reinterpret_cast<const float4*>(&sm.ablk[j][r][4 * k4]);
                        ar[4 * k4] = a4.x;
                        ar[4 * k4 + 1] = a4.y;
                        ar[4 * k4 + 2] = a4.z;
                        ar[4 * k4 + 3] = a4.w;
                    }
                    float t[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) t[m] = r == 4 * g + m ? 1.f : 0.f;
                    elim_rows(t, ar, r, std::make_integer_sequence<int, 15>{});
                    bw.tf[j][lane] = pack4(t[0], t[1], t[2], t[3]);     // A operand: T_jj[r][4g + i]
                } else if (j == 2) {
                    // A10 as the A operand: Acc((Kh1 Kc0^T)^T) holds (Kh1 Kc0^T)[r][4g + i], row r
                    // of block (1, 0), scaled by beta of token 16 + r; negated for the solve
                    f32x4 n = zero4();
#pragma unroll
                    for (int x = 0; x < 4; ++x) n += part[x][2][lane];
                    const float nbt = -bw.beta[16 + r];
                    bw.tf[2][lane] = pack4(nbt * n[0], nbt * n[1], nbt * n[2], nbt * n[3]);
                } else if (kOut) {
                    f32x4 p00 = zero4(), p11 = zero4(), p10 = zero4();
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        p00 += part[x][3][lane];
                        p11 += part[x][4][lane];
                        p10 += part[x][5][lane];
                    }
                    float dg[2] = {0.f, 0.f};                           // the exact diagonal, tokens r, 16 + r
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        dg[0] += sm.dpp[it & 1][x][r];
                        dg[1] += sm.dpp[it & 1][x][16 + r];
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {                       // P[r][4g + i], inclusive lower
                        if (4 * g + i > r) {
                            p00[i] = 0.f;
                            p11[i] = 0.f;
                        } else if (4 * g + i == r) {
                            p00[i] = dg[0];
                            p11[i] = dg[1];
                        }
                    }
                    bw.pf[0][lane] = EL::from_acc(p00, zero4()).u;
                    bw.pf[1][lane] = EL::from_acc(p10, p11).u;
                }
            }
            if (run) {
                // ---- Z = diag(b) (V - Kh S); O = Qh S ----
#pragma unroll
                for (int th = 0; th < 2; ++th) {
                    const uint4 yv = bf.yv[j][th][lane];         // slot (ja, i): token 16ja + 4g + i
                    Z[0][th] = f32x4{__uint_as_float(bfbits_lo(yv.x)), __uint_as_float(bfbits_hi(yv.x)),
                                     __uint_as_float(bfbits_lo(yv.y)), __uint_as_float(bfbits_hi(yv.y))};
                    Z[1][th] = f32x4{__uint_as_float(bfbits_lo(yv.z)), __uint_as_float(bfbits_hi(yv.z)),
                                     __uint_as_float(bfbits_lo(yv.w)), __uint_as_float(bfbits_hi(yv.w))};
                    if constexpr (PASS == 1) ZP[0][th] = ZP[1][th] = zero4();
                }
                Frag sf[4][2];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    Frag pf2[PASS == 1 ? 2 : 1];
#pragma unroll
                    for (int th = 0; th < 2; ++th) {
                        sf[kb][th] = EL::from_acc(S[2 * kb][th], S[2 * kb + 1][th]);
                        if constexpr (PASS == 1) pf2[th] = EL::from_acc(Ph[2 * kb][th], Ph[2 * kb + 1][th]);
                    }
                    if constexpr (PASS == 1) mfma_ready(sf[kb][0].u, sf[kb][1].u, pf2[0].u, pf2[1].u);
                    else mfma_ready(sf[kb][0].u, sf[kb][1].u);
#pragma unroll
                    for (int ja = 0; ja < 2; ++ja) {
                        const Frag ya{bf.yk[ja][kb][lane]};
#pragma unroll
                        for (int th = 0; th < 2; ++th) {
                            Z[ja][th] = EL::mma(ya, sf[kb][th], Z[ja][th]);
                            if constexpr (PASS == 1) ZP[ja][th] = EL::mma(ya, pf2[th], ZP[ja][th]);
                        }
                    }
                }
                if constexpr (kOut) {
#pragma unroll
                    for (int ja = 0; ja < 2; ++ja)
#pragma unroll
                        for (int th = 0; th < 2; ++th) O[ja][th] = zero4();
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                        for (int ja = 0; ja < 2; ++ja) {
                            const Frag qb{bf.qf[ja][kb][lane]};
#pragma unroll
                            for (int th = 0; th < 2; ++th) O[ja][th] = EL::mma(sf[kb][th], qb, O[ja][th]);
                        }
                }
                // rows scaled by beta of their tokens (16ja + 4g + i)
#pragma unroll
                for (int ja = 0; ja < 2; ++ja) {
                    const float4 b4 = *reinterpret_cast<const float4*>(&bf.beta[16 * ja + 4 * g]);
#pragma unroll
                    for (int th = 0; th < 2; ++th) {
                        Z[ja][th] = f32x4{Z[ja][th][0] * b4.x, Z[ja][th][1] * b4.y, Z[ja][th][2] * b4.z,
                                          Z[ja][th][3] * b4.w};
                        if constexpr (PASS == 1)
                            ZP[ja][th] = f32x4{ZP[ja][th][0] * b4.x, ZP[ja][th][1] * b4.y, ZP[ja][th][2] * b4.z,
                                               ZP[ja][th][3] * b4.w};
                    }
                }
            }
            // The summary pass's block inverses are ready when its chunk starts (the producers
            // formed them after the previous chunk's first barrier), so it solves before the first
            // barrier and updates S and Phi after it; the output pass forms its inverses here and
            // solves after the barrier.
            constexpr bool kEarly = PASS == 1;
            Frag xf[2], xpf[PASS == 1 ? 2 : 1];
            auto solve_out = [&]() __attribute__((always_inline)) {
                // ---- X = T Z by 16-row blocks: X0 = T00 Z0, X1 = T11 (Z1 - A10 X0) ----
                const Frag16 t00{bf.tf[0][lane]}, t11{bf.tf[1][lane]}, na10{bf.tf[2][lane]};
                auto solve = [&](const f32x4 (&z)[2][2], int th, f32x4& x0, f32x4& x1) __attribute__((always_inline)) {
                    Frag16 zf = EL::from_acc16(z[0][th]);
                    mfma_ready(zf.u);
                    x0 = EL::mma16(t00, zf, zero4());
                    Frag16 xf0 = EL::from_acc16(x0);
                    mfma_ready(xf0.u);
                    const f32x4 z1 = EL::mma16(na10, xf0, z[1][th]);
                    Frag16 zf1 = EL::from_acc16(z1);
                    mfma_ready(zf1.u);
                    x1 = EL::mma16(t11, zf1, zero4());
                };
#pragma unroll
                for (int th = 0; th < 2; ++th) {
                    f32x4 x0, x1;
                    solve(Z, th, x0, x1);
                    xf[th] = EL::from_acc(x0, x1);
                    if constexpr (PASS == 1) {
                        solve(ZP, th, x0, x1);
                        xpf[th] = EL::from_acc(x0, x1);
                    }
                }
                if constexpr (PASS == 1) mfma_ready(xf[0].u, xf[1].u, xpf[0].u, xpf[1].u);
                else mfma_ready(xf[0].u, xf[1].u);
                // ---- O += P X, store ----
                if constexpr (kOut) {
                    const int nrow = int(min<int64_t>(kFC, s1 - t0));
#pragma unroll
                    for (int ja = 0; ja < 2; ++ja) {
                        const Frag pb{bf.pf[ja][lane]};
#pragma unroll
                        for (int th = 0; th < 2; ++th) O[ja][th] = EL::mma(xf[th], pb, O[ja][th]);
                        // lane (token r, g): columns 32j + 8g + 4th + i of token 16ja + r
                        if (16 * ja + r < nrow)
                            *reinterpret_cast<uint4*>(out + ((t0 + 16 * ja + r) * H + h) * kFD + 32 * j + 8 * g) =
                                make_uint4(pack2(O[ja][0][0], O[ja][0][1]), pack2(O[ja][0][2], O[ja][0][3]),
                                           pack2(O[ja][1][0], O[ja][1][1]), pack2(O[ja][1][2], O[ja][1][3]));
                    }
                }
            };
            auto update_state = [&]() __attribute__((always_inline)) {
                // ---- S <- diag(gamma) S + Kb^T X = diag(gamma) (S + Kc^T X) ----
#pragma unroll
                for (int kt = 0; kt < 8; ++kt) {
                    const Frag ka{bf.kf[kt][lane]};
                    const float4 g4 = *reinterpret_cast<const float4*>(&bf.gam[key_of(kt, 4 * g)]);
#pragma unroll
                    for (int th = 0; th < 2; ++th) {
                        S[kt][th] = EL::mma(ka, xf[th], S[kt][th]);
                        S[kt][th] = f32x4{S[kt][th][0] * g4.x, S[kt][th][1] * g4.y, S[kt][th][2] * g4.z,
                                          S[kt][th][3] * g4.w};
                    }
                }
            };
            // ---- Phi <- diag(gamma) (Phi + Kc^T Xp), Xp the solve with Phi in place of V - Kh S ----
            auto update_phi = [&]() __attribute__((always_inline)) {
                if constexpr (PASS == 1) {
#pragma unroll
                    for (int kt = 0; kt < 8; ++kt) {
                        const Frag ka{bf.kf[kt][lane]};
                        const float4 g4 = *reinterpret_cast<const float4*>(&bf.gam[key_of(kt, 4 * g)]);
#pragma unroll
                        for (int th = 0; th < 2; ++th) {
                            Ph[kt][th] = EL::mma(ka, xpf[th], Ph[kt][th]);
                            Ph[kt][th] = f32x4{Ph[kt][th][0] * g4.x, Ph[kt][th][1] * g4.y, Ph[kt][th][2] * g4.z,
                                               Ph[kt][th][3] * g4.w};
                        }
                    }
                }
            };
            if constexpr (kEarly) {
                if (run) solve_out();
            }
            lds_barrier();                                      // B1
            if (run) {
                if constexpr (!kEarly) solve_out();
                update_state();
                update_phi();
            }
            lds_barrier();                                      // B2
        }
        // ---- the segment's results ----
        float* dst = nullptr;
        if constexpr (PASS == 1) {
            const int64_t unit = int64_t(sid) * H + h;
            dst = sloc + unit * kFD * kFD;
            float* pd = phi + unit * kFD * kFD;
#pragma unroll
            for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                for (int th = 0; th < 2; ++th)
#pragma unroll
                    for (int i = 0; i < 4; ++i) pd[key_of(kt, 4 * g + i) * kFD + col_of(j, th, r)] = Ph[kt][th][i];
        } else if (final_state && sg.seg == sg.nseg - 1) {
            dst = final_state + (int64_t(sg.n) * H + h) * kFD * kFD;
        }
        if (dst) {
#pragma unroll
            for (int kt = 0; kt < 8; ++kt)
#pragma unroll
                for (int th = 0; th < 2; ++th)
#pragma unroll
                    for (int i = 0; i < 4; ++i) dst[key_of(kt, 4 * g + i) * kFD + col_of(j, th, r)] = S[kt][th][i];
        }
        return;
    } else {

    // ================= producer: slab p = w - 4 =================
    const int p = w - 4;
    // The sample's rows through buffer resources whose range ends with the sample: a row past
    // its end (in the last chunk, or the prefetch after it) reads as zeros, so log a, k, q, v
    // and beta are 0 there and no row needs a mask. Offsets in bytes from the sample's first
    // token; the lane's part is fixed, the chunk's part (32 rows) is a scalar.
    const int64_t us0 = uniform64(s0), us1 = uniform64(s1);
    const uint32_t rowb = uint32_t(H) * kFD * 2;              // one token's row over all heads
    const int nbytes = int(uint32_t(us1 - us0) * rowb);
    const int64_t base = us0 * int64_t(H) * kFD;
    const auto rsq = __builtin_amdgcn_make_buffer_rsrc((void*)(q + base), 0, nbytes, kBufFlags);
    const auto rsk = __builtin_amdgcn_make_buffer_rsrc((void*)(k + base), 0, nbytes, kBufFlags);
    const auto rsv = __builtin_amdgcn_make_buffer_rsrc((void*)(v + base), 0, nbytes, kBufFlags);
    const auto rsl = __builtin_amdgcn_make_buffer_rsrc((void*)(la + base), 0, nbytes, kBufFlags);
    const auto rsb = __builtin_amdgcn_make_buffer_rsrc((void*)(beta + us0 * H), 0,
                                                       int(uint32_t(us1 - us0) * uint32_t(H) * 2), kBufFlags);
    uint32_t voff[2], boff[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        voff[tt] = uint32_t(16 * tt + r) * rowb + uint32_t(h) * kFD * 2 + 2 * (32 * p + 8 * g);
        boff[tt] = (uint32_t(16 * tt + r) * uint32_t(H) + uint32_t(h)) * 2;
    }
    auto ld16 = [&](__amdgpu_buffer_rsrc_t rs, uint32_t vo, int c) __attribute__((always_inline)) -> uint4 {
        const u32x4v x = __builtin_amdgcn_raw_buffer_load_b128(rs, vo, int(uint32_t(c) * kFC * rowb), 0);
        return make_uint4(x[0], x[1], x[2], x[3]);
    };
    // Every step issues its loads without conditions, so that the waits for one chunk's rows
    // never include the loads issued after them.
    auto load_l = [&](Raw& x, int c) __attribute__((always_inline)) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) x.l[tt] = ld16(rsl, voff[tt], c);
    };
    auto load_tile = [&](Raw& x, int c, int tt) __attribute__((always_inline)) {
        if constexpr (kOut) x.q[tt] = ld16(rsq, voff[tt], c);
        x.k[tt] = ld16(rsk, voff[tt], c);
        x.v[tt] = ld16(rsv, voff[tt], c);
    };
    // beta first in a step: the conversion of its 16 bits may be placed anywhere before the
    // next step, and then waits for these two loads only (the counter is in order)
    auto load_beta = [&](Raw& x, int c) __attribute__((always_inline)) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
            x.b[tt] = __builtin_amdgcn_raw_buffer_load_b16(rsb, boff[tt], int(uint32_t(c) * kFC * uint32_t(H) * 2), 0);
    };

    // Operands of chunk c from its raw rows `cur`; the rows of chunk c + 1 are loaded into
    // `nxt` piece by piece as `cur`'s registers fall free. Barriers as the consumers'.
    auto step = [&](const Raw& cur_in, Raw& nxt, int c) __attribute__((always_inline)) {
        Buf& bf = sm.buf[c & 1];
        // the rows become visible here, after the previous step's last barrier: no use of them
        // moves up into the previous step, where it would wait for the loads just issued
        Raw cur = cur_in;
        pin_raw(cur);
        load_beta(nxt, c + 1);
        load_l(nxt, c + 1);
        load_tile(nxt, c + 1, 1);
        load_tile(nxt, c + 1, 0);
        // ---- E: decayed rows; after the first barrier the partial products over the slab
        //      and the transposes ----
        float bt[2], qs[2] = {1.f, 1.f}, ks[2] = {1.f, 1.f};
        uint4 khF[2], kcH[2], qH[2];
        uint4 kcL[2], qL[2];      // the bf16 remainders of Kc and Qh for P (output passes)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) bt[tt] = bf2f(cur.b[tt]);
        if constexpr (NORM) {
            // each row's sums of squares over the 128 channels: four lanes here and the
            // three other slabs' waves, summed in a fixed order
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                float kf[8], qf[8], qq = 0.f, kk = 0.f;
                unpack8(cur.k[tt], kf);
                if constexpr (kOut) unpack8(cur.q[tt], qf);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if constexpr (kOut) qq += qf[e] * qf[e];
                    kk += kf[e] * kf[e];
                }
                qq += __shfl_xor(qq, 16);
                qq += __shfl_xor(qq, 32);
                kk += __shfl_xor(kk, 16);
                kk += __shfl_xor(kk, 32);
                if (g == 0) {
                    sm.ssq[0][p][16 * tt + r] = qq;
                    sm.ssq[1][p][16 * tt + r] = kk;
                }
            }
            lds_barrier();
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                float tq = 0.f, tk = 0.f;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    tq += sm.ssq[0][x][16 * tt + r];
                    tk += sm.ssq[1][x][16 * tt + r];
                }
                qs[tt] = tq > 0.f ? 1.f / sqrtf(tq) : 0.f;
                ks[tt] = tk > 0.f ? 1.f / sqrtf(tk) : 0.f;
            }
        }
        // G over the chunk: the half-slab tiles of log a transposed (product with the identity),
        // then a product with the inclusive triangle, tile 1 plus tile 0's sum; lane (r, g) gets
        // G[16tt + r][8g + 4t + i], the layout of its raw rows
        f32x4 G[2][2];
        {
            Frag16 lt[2][2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    lt[tt][t] = EL::from_acc16(EL::mma16(Frag16{half_of(cur.l[tt], t)}, ident, zero4()));
            mfma_ready(lt[0][0].u, lt[0][1].u, lt[1][0].u, lt[1][1].u);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                G[0][t] = EL::mma16(lt[0][t], tri, zero4());
                G[1][t] = EL::mma16(lt[0][t], ones, EL::mma16(lt[1][t], tri, zero4()));
            }
        }
        if (p == 0 && g == 0) {
            bf.beta[r] = bt[0];
            bf.beta[16 + r] = bt[1];
        }
        // decayed rows of token tile tt (rows past the sample's end are zeros: they reach no
        // valid row through A, P, X or the state, and G and gamma stop at the last valid row);
        // the tile's next rows are loaded as its registers fall free
        auto tile_pass = [&](const int tt) __attribute__((always_inline)) {
            float kf[8], qf[8];
            unpack8(cur.k[tt], kf);
            if constexpr (kOut) unpack8(cur.q[tt], qf);
            float ex[8], ei[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float G2 = G[tt][e >> 2][e & 3] * kLog2e;
                ex[e] = fast_exp2(G2);
                ei[e] = fast_exp2(-G2);
            }
            // gamma = e^G of token 31, held by the lanes of row 15 of tile 1
            if (tt == 1 && r == 15) {
                *reinterpret_cast<float4*>(&bf.gam[32 * p + 8 * g]) = make_float4(ex[0], ex[1], ex[2], ex[3]);
                *reinterpret_cast<float4*>(&bf.gam[32 * p + 8 * g + 4]) = make_float4(ex[4], ex[5], ex[6], ex[7]);
            }
            float fkh[8], fkc[8], fq[8];
            float dp = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float kx = NORM ? kf[e] * ks[tt] : kf[e];
                const float qx = kOut ? (NORM ? qf[e] * qs[tt] : qf[e]) : 0.f;
                fkh[e] = kx * ex[e];
                fkc[e] = kx * ei[e];
                fq[e] = qx * ex[e];
                dp += kx * qx;
            }
            khF[tt] = pack8(fkh);
            if constexpr (kOut) split8(fkc, kcH[tt], kcL[tt]);
            else kcH[tt] = pack8(fkc);
            bf.yk[tt][p][lane] = make_uint4(khF[tt].x ^ 0x80008000u, khF[tt].y ^ 0x80008000u,
                                            khF[tt].z ^ 0x80008000u, khF[tt].w ^ 0x80008000u);
            if constexpr (kOut) {
                // q.k of the row over the slab (e^G e^-G = 1 on the diagonal of P)
                dp += __shfl_xor(dp, 16);
                dp += __shfl_xor(dp, 32);
                if (g == 0) sm.dpp[c & 1][p][16 * tt + r] = dp;
                split8(fq, qH[tt], qL[tt]);
                bf.qf[tt][p][lane] = qH[tt];
            } else {
                qH[tt] = make_uint4(0u, 0u, 0u, 0u);
            }
        };
        auto partials = [&]() __attribute__((always_inline)) {
            mfma_ready(khF[0], khF[1], kcH[0], kcH[1]);
            mfma_ready(qH[0], qH[1]);
            if constexpr (kOut) mfma_ready(kcL[0], kcL[1], qL[0], qL[1]);
            // partial products over the slab: Acc(X) holds X[4g + i][r]
            f32x4* pp = &sm.part[c & 1][p][0][0];
            pp[0 * 64 + lane] = EL::mma(Frag{khF[0]}, Frag{kcH[0]}, zero4());   // Kh0 Kc0^T
            pp[1 * 64 + lane] = EL::mma(Frag{khF[1]}, Frag{kcH[1]}, zero4());   // Kh1 Kc1^T
            pp[2 * 64 + lane] = EL::mma(Frag{kcH[0]}, Frag{khF[1]}, zero4());   // (Kh1 Kc0^T)^T
            if constexpr (kOut) {
                // P^T blocks (Kc Qh^T): (0, 0), (1, 1), (1, 0), each from hi/lo bf16 parts of both
                // operands (lo*hi + hi*lo + hi*hi): a row whose output is mostly P X (a sample's
                // first chunk, where the state is zero) can be much shorter than |q| |k| |X|, and
                // single bf16 operands put an error of about 2^-9 |q| |k| on each of its terms
                auto p3 = [&](int a, int b) __attribute__((always_inline)) {
                    return EL::mma(Frag{kcH[a]}, Frag{qH[b]},
                                   EL::mma(Frag{kcH[a]}, Frag{qL[b]}, EL::mma(Frag{kcL[a]}, Frag{qH[b]}, zero4())));
                };
                pp[3 * 64 + lane] = p3(0, 0);
                pp[4 * 64 + lane] = p3(1, 1);
                pp[5 * 64 + lane] = p3(0, 1);
            }
            // transposes (channel rows over the chunk's tokens, exact): Kc^T and V to LDS
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const f32x4 a0 = EL::mma16(Frag16{half_of(kcH[0], t)}, ident, zero4());
                const f32x4 a1 = EL::mma16(Frag16{half_of(kcH[1], t)}, ident, zero4());
                bf.kf[2 * p + t][lane] = EL::from_acc(a0, a1).u;
                const f32x4 v0 = EL::mma16(Frag16{half_of(cur.v[0], t)}, ident, zero4());
                const f32x4 v1 = EL::mma16(Frag16{half_of(cur.v[1], t)}, ident, zero4());
                bf.yv[p][t][lane] = EL::from_acc(v0, v1).u;
            }
        };
        // The output pass splits its decay work at the first barrier (the consumers' second
        // interval is the longer one there); the summary pass does all of it first and its
        // inverses after the barrier.
        tile_pass(1);
        if constexpr (!kConsInv) {
            tile_pass(0);
            partials();
        }
        lds_barrier();                                          // B1
        if constexpr (kConsInv) {
            tile_pass(0);
            partials();
        } else {
            // ---- sums of the partial products and the inverses of the two diagonal blocks of
            //      I + A: wave 4 + p inverts block p & 1 on its columns 8 (p >> 1) .. + 7 (the
            //      columns of an inverse are independent, so two waves halve the chain of
            //      dependent steps); wave 6 also forms -A10 ----
            {
                const int ii = p & 1, hc = p >> 1;
                {
                    // A_ii = StrictLower(diag(b) Kh Kc^T) of diagonal block ii, rows to this wave's copy
                    f32x4 n = zero4();
#pragma unroll
                    for (int x = 0; x < 4; ++x) n += sm.part[c & 1][x][ii][lane];
                    const float4 b4 = *reinterpret_cast<const float4*>(&bf.beta[16 * ii + 4 * g]);
                    const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) sm.ablk[p][4 * g + i][r] = 4 * g + i > r ? bb[i] * n[i] : 0.f;
                }
                lds_wait();
                // T = (I + A_ii)^-1 in fp32 by elimination: lane (r, g) holds row r of A and T[r][j0],
                // T[r][j0 + 1] with j0 = 8 hc + 2 g; for k = 0..14 row k is final and every row below
                // it takes -A[r][k] T[k][.], T[k][.] broadcast along the lanes of the row (DPP)
                float ar[16];
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4) {
                    const float4 a4 = *reinterpret_cast<const float4*>(&sm.ablk[p][r][4 * k4]);
                    ar[4 * k4] = a4.x;
                    ar[4 * k4 + 1] = a4.y;
                    ar[4 * k4 + 2] = a4.z;
                    ar[4 * k4 + 3] = a4.w;
                }
                const int j0 = 8 * hc + 2 * g;
                float t[2];
#pragma unroll
                for (int m = 0; m < 2; ++m) t[m] = r == j0 + m ? 1.f : 0.f;
                elim_rows2(t, ar, r, std::make_integer_sequence<int, 15>{});
                // A operand of T_ii: lane (r, g') holds T[r][4g' .. 4g' + 3]; columns j0, j0 + 1 are
                // its elements 2 (g & 1), + 1 in lane (r, j0 / 4)
                reinterpret_cast<uint32_t*>(&bf.tf[ii][16 * (j0 >> 2) + r])[g & 1] = pack2(t[0], t[1]);
            }
            if (p == 2) {
                // A10 as the A operand: Acc((Kh1 Kc0^T)^T) holds (Kh1 Kc0^T)[r][4g + i], row r of block
                // (1, 0), scaled by beta of token 16 + r; negated for the solve
                f32x4 n = zero4();
#pragma unroll
                for (int x = 0; x < 4; ++x) n += sm.part[c & 1][x][2][lane];
                const float nbt = -bf.beta[16 + r];
                bf.tf[2][lane] = pack4(nbt * n[0], nbt * n[1], nbt * n[2], nbt * n[3]);
            }
        }
        lds_barrier();                                          // B2
    };

    if (c0 < c1) {
        // step c forms chunk c (the consumers' chunk c - 1); the loop alternates two
        // register sets for the raw rows
        Raw ra, rb;
        load_beta(ra, c0);
        load_l(ra, c0);
        load_tile(ra, c0, 1);
        load_tile(ra, c0, 0);
        int c = c0;
        for (; c + 1 < c1; c += 2) {
            step(ra, rb, c);
            step(rb, ra, c + 1);
        }
        if (c < c1) step(ra, rb, c);
    }
    // the consumers' last chunk: barriers only
    if constexpr (NORM) lds_barrier();
    lds_barrier();
    lds_barrier();
    }
}

struct FusedArgs {
    const uint16_t *q, *k, *v, *la, *beta;
    const int32_t *cu, *seg_off;
    const float *init_state, *carry;
    uint16_t* out;
    float *final_state, *sloc, *phi;
    int* counter;          // next unit; starts at zero
    int64_t T;
    int num_seqs, H, lseg, max_segs, units;
};
using KernArgs = const __attribute__((address_space(4))) FusedArgs*;

// A persistent grid, one workgroup per CU: each workgroup takes the next unit from a counter
// in memory until none is left, so units run wherever a CU is free (a grid of two or more
// workgroups per CU leaves some CUs idle while others run a third unit, since the dispatcher
// does not place workgroups on whichever CU finished first).
template <int PASS, bool NORM>
__global__ __launch_bounds__(kFThreads, 1) void kda_fused_kernel(const FusedArgs args)
{
    __shared__ FusedSmem sm;
    __shared__ int next_unit;
    // each role in a loop of its own (the same barriers per unit), so that neither keeps the
    // other's values live
    auto run = [&](auto role) __attribute__((always_inline)) {
        for (;;) {
            // the arguments are loaded again for every unit, through a pointer the compiler cannot
            // follow across iterations: kept in scalar registers over the loop they would crowd
            // out the unit's own
            uint64_t kp = reinterpret_cast<uint64_t>(__builtin_amdgcn_kernarg_segment_ptr());
            asm volatile("" : "+s"(kp));
            const KernArgs ap = reinterpret_cast<KernArgs>(kp);
            if (threadIdx.x == 0) next_unit = atomicAdd(ap->counter, 1);
            lds_barrier();
            const int lin = __builtin_amdgcn_readfirstlane(next_unit);
            lds_barrier();                              // every wave has read it before the next
            if (lin >= ap->units) break;
            fused_unit<PASS, NORM, decltype(role)::value>(sm, lin, ap->q, ap->k, ap->v, ap->la, ap->beta, ap->cu,
                                                          ap->seg_off, ap->init_state, ap->carry, ap->out,
                                                          ap->final_state, ap->sloc, ap->phi, ap->num_seqs, ap->H,
                                                          ap->T, ap->lseg, ap->max_segs);
        }
    };
    if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < 4) run(std::true_type{});   // waves 0-3
    else run(std::false_type{});
}

// ---------------------------------------------------------------------------
// combine: per (sample, head, kCombCT value tiles of 16 columns), the entry state of every segment,
// S_in(k + 1) = Phi(k) S_in(k) + S_loc(k), S_in(0) = the initial state; S_in(k + 1) is
// written over S_loc(k) (the slot of segment k), which no later step reads. Wave w
// computes output rows 32w..32w+31 (key tiles 2w, 2w + 1); Phi's rows (fp32) enter as
// hi/lo bf16 A fragments, the full S_in as hi/lo B fragments through LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kCombThreads) void kda_fused_combine_kernel(
    const int32_t* __restrict__ cu, const int32_t* __restrict__ seg_off, const float* __restrict__ init_state,
    float* __restrict__ sloc, const float* __restrict__ phi, int num_seqs, int H, int64_t T, int lseg,
    int max_segs)
{
    constexpr int CT = kCombCT;
    __shared__ uint4 sb[2][4][CT][64];          // S_in as B fragments: [hi/lo][k-block][value tile][lane]
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    constexpr int kGroups = 8 / CT;             // workgroups per (sample, head)
    const int ct0 = (blockIdx.x % kGroups) * CT;    // value tiles ct0 .. ct0 + CT - 1: columns 16 ct + r
    const int unit = blockIdx.x / kGroups;
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

    f32x4 S[CT][2];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[c][j][i] = init_state ? init_state[((int64_t(n) * H + h) * kFD + 32 * w + 16 * j + 4 * g + i) * kFD +
                                                     16 * (ct0 + c) + r]
                                        : 0.f;
    // Phi(k) and S_loc(k) do not depend on the chain: the next segment's are loaded while the
    // current product runs, so a step waits only for its own products. Each fragment of Phi
    // serves the workgroup's CT value tiles.
    struct Next {
        float a[2][4][8];       // Phi rows row + r, columns 32 kb + [4g, 4g + 4) and + 16
        f32x4 c[CT][2];         // S_loc rows row + 4g + i, columns 16 ct + r
    };
    auto load_next = [&](Next& x, int kseg) __attribute__((always_inline)) {
        const int64_t u = int64_t(first + kseg) * H + h;
        const float* sl = sloc + u * kFD * kFD;
        const float* ph = phi + u * kFD * kFD;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = 32 * w + 16 * j;            // output key rows row + 4g + i (acc), row + r (A)
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) x.c[c][j][i] = sl[(row + 4 * g + i) * kFD + 16 * (ct0 + c) + r];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const float4 a0 = *reinterpret_cast<const float4*>(ph + (row + r) * kFD + 32 * kb + 4 * g);
                const float4 a1 = *reinterpret_cast<const float4*>(ph + (row + r) * kFD + 32 * kb + 16 + 4 * g);
                x.a[j][kb][0] = a0.x; x.a[j][kb][1] = a0.y; x.a[j][kb][2] = a0.z; x.a[j][kb][3] = a0.w;
                x.a[j][kb][4] = a1.x; x.a[j][kb][5] = a1.y; x.a[j][kb][6] = a1.z; x.a[j][kb][7] = a1.w;
            }
        }
    };
    auto step = [&](const Next& cur, Next& nxt, int kseg) __attribute__((always_inline)) {
        // Phi(kseg) as hi/lo fragments before the chain's own wait
        Frag ah[2][4], al[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) split8(cur.a[j][kb], ah[j][kb].u, al[j][kb].u);
        if (kseg + 2 < nseg) load_next(nxt, kseg + 1);
        // publish S_in(kseg): this wave's rows are k-block w of the products
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            const float s8[8] = {S[c][0][0], S[c][0][1], S[c][0][2], S[c][0][3],
                                 S[c][1][0], S[c][1][1], S[c][1][2], S[c][1][3]};
            uint4 hi, lo;
            split8(s8, hi, lo);
            sb[0][w][c][lane] = hi;
            sb[1][w][c][lane] = lo;
        }
        lds_barrier();
        f32x4 acc[CT][2];
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[c][j] = cur.c[c][j];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int j = 0; j < 2; ++j) mfma_ready(ah[j][kb].u, al[j][kb].u);
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                const Frag bh{sb[0][kb][c][lane]}, bl{sb[1][kb][c][lane]};
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    acc[c][j] = EL::mma(al[j][kb], bh, acc[c][j]);
                    acc[c][j] = EL::mma(ah[j][kb], bl, acc[c][j]);
                    acc[c][j] = EL::mma(ah[j][kb], bh, acc[c][j]);
                }
            }
        }
        lds_barrier();
        // S_in(kseg + 1) over S_loc(kseg): the same lanes read and write these elements
        float* sl = sloc + (int64_t(first + kseg) * H + h) * kFD * kFD;
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                S[c][j] = acc[c][j];
#pragma unroll
                for (int i = 0; i < 4; ++i) sl[(32 * w + 16 * j + 4 * g + i) * kFD + 16 * (ct0 + c) + r] = acc[c][j][i];
            }
    };
    Next na, nb;
    load_next(na, 0);
    int kseg = 0;
    for (; kseg + 2 < nseg; kseg += 2) {
        step(na, nb, kseg);
        step(nb, na, kseg + 1);
    }
    if (kseg + 1 < nseg) step(na, nb, kseg);
}

struct FusedPlan {
    int lseg;          // chunks (32 tokens) per segment; 0 = one segment per sample
    int max_segs;
    size_t table_bytes, sloc_bytes, phi_bytes;
    size_t total() const { return kCounterBytes + table_bytes + sloc_bytes + phi_bytes; }
    static constexpr size_t kCounterBytes = 256;
};

FusedPlan plan_with(int64_t chunks, int32_t N, int32_t H, int64_t lseg)
{
    FusedPlan p{};
    p.lseg = lseg > 0 && lseg < chunks ? int(lseg) : 0;
    p.max_segs = p.lseg ? int((chunks + p.lseg - 1) / p.lseg + N) : N;
    p.table_bytes = (p.lseg && N > 64) ? ((size_t(N) + 1) * 4 + 255) & ~size_t(255) : 0;
    p.sloc_bytes = p.lseg ? size_t(p.max_segs) * H * kFD * kFD * 4 : 0;
    p.phi_bytes = p.lseg ? size_t(p.max_segs) * H * kFD * kFD * 4 : 0;
    return p;
}

// Cut samples into segments when the (sample, head) units alone would not give every CU one:
// about 256 segment units then run, one per CU, of at least 16 chunks each (two rounds of
// half-length segments take as long for the passes and double the combine's chain).
// With a byte limit on the workspace, segments grow until their summaries fit (fewer,
// longer segments); when not even one cut per sample fits, samples stay whole.
FusedPlan fused_plan(int64_t T, int32_t N, int32_t H, size_t cap)
{
    const int64_t units = int64_t(N) * H;
    const int64_t chunks = (T + kFC - 1) / kFC + N;         // upper bound over all samples
    int64_t lseg = units < 256 ? std::max<int64_t>(16, (chunks * H + 255) / 256) : 0;
    FusedPlan p = plan_with(chunks, N, H, lseg);
    if (p.total() <= cap) return p;
    const size_t slot = size_t(2) * kFD * kFD * 4 * size_t(H);          // one segment's summaries, all heads
    const size_t fixed = FusedPlan::kCounterBytes + p.table_bytes;
    const size_t avail = cap > fixed ? cap - fixed : 0;
    const int64_t max_segs = int64_t(avail / slot);
    lseg = max_segs > N ? std::max<int64_t>(lseg, (chunks + (max_segs - N) - 1) / (max_segs - N)) : 0;
    return plan_with(chunks, N, H, lseg);
}

// CUs of the current device (cached per device)
hipError_t device_cus(int& n)
{
    static std::atomic<int> cache[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64 && (n = cache[dev].load(std::memory_order_relaxed)) > 0) return hipSuccess;
    if ((e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if (n <= 0) return hipErrorInvalidDevice;
    if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
    return hipSuccess;
}

template <int PASS, bool NORM>
hipError_t launch_pass(const LaunchArgs& a, const int32_t* seg_off, const FusedPlan& p, const float* carry,
                       float* sloc, float* phi, int* counter)
{
    const int units = (p.lseg ? p.max_segs : a.num_seqs) * a.num_heads;
    int cus = 0;
    const hipError_t e = device_cus(cus);
    if (e != hipSuccess) return e;
    const int blocks = std::min(units, cus);
    FusedArgs fa{};
    fa.q = static_cast<const uint16_t*>(a.q);
    fa.k = static_cast<const uint16_t*>(a.k);
    fa.v = static_cast<const uint16_t*>(a.v);
    fa.la = static_cast<const uint16_t*>(a.log_alpha);
    fa.beta = static_cast<const uint16_t*>(a.beta);
    fa.cu = a.cu_seqlens;
    fa.seg_off = seg_off;
    fa.init_state = a.init_state;
    fa.carry = carry;
    fa.out = static_cast<uint16_t*>(a.out);
    fa.final_state = a.final_state;
    fa.sloc = sloc;
    fa.phi = phi;
    fa.counter = counter;
    fa.T = a.total_tokens;
    fa.num_seqs = a.num_seqs;
    fa.H = a.num_heads;
    fa.lseg = p.lseg;
    fa.max_segs = p.max_segs;
    fa.units = units;
    hipLaunchKernelGGL((kda_fused_kernel<PASS, NORM>), dim3(blocks), dim3(kFThreads), 0, a.stream, fa);
    return hipGetLastError();
}

template <bool NORM>
hipError_t launch_fused_norm(const LaunchArgs& a, const int32_t* seg_off, const FusedPlan& p, float* sloc,
                             float* phi, int* counters, TimingHook* th)
{
    hipError_t e;
    if (p.lseg == 0) {
        if (th) th->begin("fused", a.stream);
        e = launch_pass<0, NORM>(a, seg_off, p, nullptr, nullptr, nullptr, counters);
        if (th) th->end(a.stream);
        return e;
    }
    if (th) th->begin("fused_sum", a.stream);
    e = launch_pass<1, NORM>(a, seg_off, p, nullptr, sloc, phi, counters + 1);
    if (th) th->end(a.stream);
    if (e != hipSuccess) return e;
    if (th) th->begin("fused_combine", a.stream);
    hipLaunchKernelGGL(kda_fused_combine_kernel, dim3(a.num_seqs * a.num_heads * (8 / kCombCT)), dim3(kCombThreads), 0,
                       a.stream, a.cu_seqlens, seg_off, a.init_state, sloc, phi, a.num_seqs, a.num_heads,
                       a.total_tokens, p.lseg, p.max_segs);
    if (th) th->end(a.stream);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (th) th->begin("fused", a.stream);
    e = launch_pass<2, NORM>(a, seg_off, p, sloc, nullptr, nullptr, counters + 2);
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
    return fused_plan(total_tokens, num_seqs, num_heads, cap).total();
}

hipError_t launch_forward_fused(const LaunchArgs& a, void* workspace, TimingHook* th, size_t cap)
{
    const FusedPlan p = fused_plan(a.total_tokens, a.num_seqs, a.num_heads, cap);
    if (int64_t(p.max_segs) * a.num_heads > 0x7FFFFFFF / 8) return hipErrorInvalidValue;
    if (workspace == nullptr) return hipErrorInvalidValue;
    char* base = static_cast<char*>(workspace);
    int* counters = reinterpret_cast<int*>(base);
    base += FusedPlan::kCounterBytes;
    int32_t* seg_off = p.table_bytes ? reinterpret_cast<int32_t*>(base) : nullptr;
    float* sloc = p.lseg ? reinterpret_cast<float*>(base + p.table_bytes) : nullptr;
    float* phi = p.lseg ? reinterpret_cast<float*>(base + p.table_bytes + p.sloc_bytes) : nullptr;
    // the unit counters start at zero (and the segment table is built) in one small kernel
    if (th) th->begin("plan", a.stream);
    hipLaunchKernelGGL(kda_fused_plan_kernel, dim3(1), dim3(1024), 0, a.stream, a.cu_seqlens, seg_off,
                       a.num_seqs, a.total_tokens, p.lseg, counters);
    if (th) th->end(a.stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return a.qk_l2norm ? launch_fused_norm<true>(a, seg_off, p, sloc, phi, counters, th)
                       : launch_fused_norm<false>(a, seg_off, p, sloc, phi, counters, th);
}

}  // namespace kda
