// kda_bwd.hip -- gradients of the KDA scan (q, k, v, log alpha, beta and the initial
// state) for fp32 and bf16 data, fp32 arithmetic (gfx950): fp32 MFMA, except on bf16 data
// the two chains' products and the gradient kernel's products over value columns, which
// take hi/lo bf16 operands (three bf16 MFMA terms, two where one operand is bf16 data).
//
// The paper trains its model through these kernels (training setup paragraph on the
// custom kernels over the packed tokens). The recurrence, per (sample, head)
// (explainer page, "One stream, three mechanisms, no positions"; reset at each packed
// sample, paper Sec. 3 KDA paragraph):
//     S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,   o_t = S_t^T q_t.
// Chunkwise over C = 32 tokens (G = inclusive cumsum of log a over the chunk's rows
// per key channel, gamma = exp(G of the last row)):
//     Qh = Q e^G, Kh = K e^G, Kc = K e^-G, M = Kh Kc^T, A = StrictLower(diag(b) M),
//     T = (I + A)^-1, P = LowerIncl(Qh Kc^T),
//     X = V - Kh S,  Vn = T diag(b) X,  O = Qh S + P Vn,  S' = diag(gamma)(S + Kc^T Vn)
// (Vn = U - W S with the WY factors U = T diag(b) V, W = T diag(b) Kh multiplied out.)
// For a loss with gradients dO and dS' (the state leaving the chunk):
//     dVn = P^T dO + Kc diag(gamma) dS',   dX = diag(b) T^T dVn
//     dS  = diag(gamma) dS' + Qh^T dO - Kh^T dX              (state entering the chunk)
//     dP  = LowerIncl(dO Vn^T),  dT = dVn X^T diag(b),  dA = StrictLower(-T^T dT T^T)
//     dM  = diag(b) dA,  dV = dX,  db = rowsum((T^T dVn) X) + rowsum(dA M)
//     dQh = dO S^T + dP Kc,  dKh = -dX S^T + dM Kc,
//     dKc = dP^T Qh + (Vn dS'^T) diag(gamma) + dM^T Kh
//     dgamma = colsum((Vn dS'^T) Kc) + rowsum(dS' S)
// and through the decays: dQ = dQh e^G, dK = dKh e^G + dKc e^-G,
//     dG = dQh Qh + dKh Kh - dKc Kc (+ dgamma gamma on the last row), dlog a = the
//     reverse cumsum of dG over the chunk's rows.
//
// Kernels: a chunk table; a prep over all (chunk, head) pairs writing Kh, Kc, Qh, T, P,
// M, gamma, b (and the norms' reciprocals); a chain carrying S forwards that saves the
// state entering every chunk; a chain carrying dS backwards that saves the gradient of
// the state leaving every chunk; and a gradient kernel over all (chunk, head) pairs that
// reads the chunk's operands back from the prep's record and applies the formulas above. For packs of few long samples each chain
// runs as two passes over segments of the samples (the sequence split below).
//
// MFMA: v_mfma_f32_16x16x4f32; lane (r = lane%16, g = lane/16) supplies A(r, k) and
// B(k, r) for the four k of a step, and holds D(4g + v, r), v = 0..3. Supplying
// k = 16t + 4g + s in step s makes an accumulator tile (rows 4g + v) a B operand as it
// stands; every operand read from LDS takes any k order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "kda_device.h"
#include "kda_internal.h"

namespace kda {
namespace {
using namespace dev;

constexpr int kBC = 32;            // chunk rows
constexpr int kBT = 256;           // threads per workgroup: 4 wave64
constexpr int kLC = kBC + 4;       // row stride of [C][C] tiles in LDS

__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// bf16 products for bf16 data in the chains (v_mfma_f32_16x16x32_bf16, fp32 accumulate). A
// k-block of 32 is split over the lanes as elsewhere in these kernels: lane group g supplies
// k = 4g + s and 16 + 4g + s (s = 0..3), so two accumulator tiles (rows 4g + v of tiles t and
// t + 1) make one B fragment as they stand. Every fp32 operand enters as a hi + lo bf16 pair
// (16 bits of mantissa) and a product as the three terms hi*hi, hi*lo, lo*hi: the chains
// carry the state over the whole sequence, and db sums products of residuals (V - Kh S) that
// cancel, so single bf16 operands are not enough there. dO (bf16 data) is exact as one bf16.
struct BF {
    uint4 u;
};
struct BF2 {
    BF h, l;
};
__device__ __forceinline__ BF bf_pack(const float (&f)[8]) {
    return BF{make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]))};
}
__device__ __forceinline__ BF2 bf_split(const float (&f)[8]) {
    BF2 o;
    o.h = bf_pack(f);
    const uint32_t w[4] = {o.h.u.x, o.h.u.y, o.h.u.z, o.h.u.w};
    float r[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        r[2 * j] = f[2 * j] - __uint_as_float(w[j] << 16);
        r[2 * j + 1] = f[2 * j + 1] - __uint_as_float(w[j] & 0xFFFF0000u);
    }
    o.l = bf_pack(r);
    return o;
}
__device__ __forceinline__ BF2 bf_split(const f32x4& a, const f32x4& b) {
    const float f[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return bf_split(f);
}
__device__ __forceinline__ f32x4 mmab(const BF& a, const BF& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.u), __builtin_bit_cast(bf16x8, b.u),
                                                   c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mm3(const BF2& a, const BF2& b, f32x4 c) {
    return mmab(a.h, b.h, mmab(a.h, b.l, mmab(a.l, b.h, c)));
}
__device__ __forceinline__ f32x4 mm2(const BF2& a, const BF& b, f32x4 c) { return mmab(a.h, b, mmab(a.l, b, c)); }
__device__ __forceinline__ void ready(BF2& a) { mfma_ready(a.h.u, a.l.u); }
__device__ __forceinline__ void ready(BF2& a, BF2& b) { mfma_ready(a.h.u, a.l.u, b.h.u, b.l.u); }
// the 8 values a lane supplies from column `col` of a [32][ld] fp32 LDS array (k = row)
__device__ __forceinline__ void col8(const float* a, int ld, int col, int g, float (&f)[8]) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        f[s] = a[(4 * g + s) * ld + col];
        f[4 + s] = a[(16 + 4 * g + s) * ld + col];
    }
}
__device__ __forceinline__ BF2 bf_col(const float* a, int ld, int col, int g) {
    float f[8];
    col8(a, ld, col, g, f);
    return bf_split(f);
}
// ... and from row `row` (k = column k0 + ...), 16-byte aligned pieces
__device__ __forceinline__ BF2 bf_row(const float* a, int ld, int row, int k0, int g) {
    const float4 x = *reinterpret_cast<const float4*>(a + row * ld + k0 + 4 * g);
    const float4 y = *reinterpret_cast<const float4*>(a + row * ld + k0 + 16 + 4 * g);
    const float f[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
    return bf_split(f);
}

// ... one bf16 per value, for values that are bf16 already (dO of bf16 data: exact)
__device__ __forceinline__ BF bf_row1(const float* a, int ld, int row, int k0, int g) {
    const float4 x = *reinterpret_cast<const float4*>(a + row * ld + k0 + 4 * g);
    const float4 y = *reinterpret_cast<const float4*>(a + row * ld + k0 + 16 + 4 * g);
    const float f[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
    return bf_pack(f);
}
// acc + sum over the W columns j of a[ra][j] * b[rb][j] ([*][ld] fp32 LDS arrays, rows ra
// and rb as the lane's A row and B column): hi/lo bf16 products, three terms, or two when
// a holds bf16 values (EXACT_A)
template <int W, bool EXACT_A>
__device__ __forceinline__ f32x4 rowdot(const float* a, int ra, const float* b, int rb, int ld, int g, f32x4 acc) {
#pragma unroll
    for (int j0 = 0; j0 < W; j0 += 32) {
        BF2 y = bf_row(b, ld, rb, j0, g);
        if constexpr (EXACT_A) {
            BF x = bf_row1(a, ld, ra, j0, g);
            mfma_ready(x.u);
            ready(y);
            acc = mmab(x, y.h, mmab(x, y.l, acc));
        } else {
            BF2 x = bf_row(a, ld, ra, j0, g);
            ready(x, y);
            acc = mm3(x, y, acc);
        }
    }
    return acc;
}

template <typename E> __device__ __forceinline__ float ldf(const E* p);
template <> __device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p) { return bf2f(*p); }
template <typename E> __device__ __forceinline__ void stf(E* p, float x);
template <> __device__ __forceinline__ void stf<float>(float* p, float x) { *p = x; }
template <> __device__ __forceinline__ void stf<uint16_t>(uint16_t* p, float x) { *p = f2bf(x); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 16 raw bytes in registers

// 16 bytes of data dtype E as fp32 to LDS (8 bf16 or 4 fp32 values), zeros when !ok
template <typename E> __device__ __forceinline__ void put16(float* dst, const u32x4& raw, bool ok);
template <> __device__ __forceinline__ void put16<float>(float* dst, const u32x4& raw, bool ok) {
    const float4 f = ok ? make_float4(__uint_as_float(raw.x), __uint_as_float(raw.y), __uint_as_float(raw.z),
                                      __uint_as_float(raw.w))
                        : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(dst) = f;
}
template <> __device__ __forceinline__ void put16<uint16_t>(float* dst, const u32x4& raw, bool ok) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (ok) {
        a = make_float4(__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xFFFF0000u),
                        __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xFFFF0000u));
        b = make_float4(__uint_as_float(raw.z << 16), __uint_as_float(raw.z & 0xFFFF0000u),
                        __uint_as_float(raw.w << 16), __uint_as_float(raw.w & 0xFFFF0000u));
    }
    *reinterpret_cast<float4*>(dst) = a;
    *reinterpret_cast<float4*>(dst + 4) = b;
}

// A [C][W] block of rows t0.. of a [T][H][W] tensor of dtype E, as 16-byte pieces held
// by the workgroup's threads (rows past the chunk's end re-read its last row and are
// zeroed when written to LDS). Loads only: put() writes them to a [C][ld] LDS array.
template <typename E, int W> struct RowPieces {
    static constexpr int EPP = 16 / sizeof(E);       // elements per piece
    static constexpr int PPR = W / EPP;              // pieces per row
    static constexpr int NP = (kBC * PPR + kBT - 1) / kBT;
    u32x4 v[NP];
    __device__ __forceinline__ void load(const E* __restrict__ src, int64_t t0, int nrow, int H, int h, int col0,
                                         int rowlen) {
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int pc = min(int(threadIdx.x) + j * kBT, kBC * PPR - 1);
            const int row = min(pc / PPR, nrow - 1);
            v[j] = *reinterpret_cast<const u32x4*>(src + ((t0 + row) * H + h) * rowlen + col0 + (pc % PPR) * EPP);
        }
    }
    __device__ __forceinline__ void put(float* dst, int ld, int nrow) const {
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int pc = int(threadIdx.x) + j * kBT;
            if (pc < kBC * PPR) put16<E>(dst + (pc / PPR) * ld + (pc % PPR) * EPP, v[j], pc / PPR < nrow);
        }
    }
};

// Record of one (chunk, head) written by the prep: every chunk operand, for the two
// chains and the gradient kernel (floats).
template <int DK> struct BRec {
    static constexpr int KH = 0;                    // Kh [C][DK]
    static constexpr int KC = KH + kBC * DK;        // Kc [C][DK]
    static constexpr int QH = KC + kBC * DK;        // Qh [C][DK]
    static constexpr int T = QH + kBC * DK;         // T  [C][C]
    static constexpr int P = T + kBC * kBC;         // P  [C][C]
    static constexpr int GAM = P + kBC * kBC;       // gamma [DK]
    static constexpr int BETA = GAM + DK;           // b [C] (0 past the sample's end)
    static constexpr int M = BETA + kBC;            // M = Kh Kc^T [C][C]
    static constexpr int QINV = M + kBC * kBC;      // 1/|q_t| [C] (1 without normalisation)
    static constexpr int KINV = QINV + kBC;         // 1/|k_t| [C]
    static constexpr int TOTAL = KINV + kBC;
    static_assert(KC % 4 == 0 && QH % 4 == 0 && T % 4 == 0 && P % 4 == 0 && GAM % 4 == 0 && BETA % 4 == 0 &&
                  M % 4 == 0 && QINV % 4 == 0 && KINV % 4 == 0 && TOTAL % 4 == 0, "16-byte fields and records");
};

// ---------------------------------------------------------------------------
// chunk table: chunk_off[n] = number of 32-token chunks of samples 0..n-1; with the
// sequence split (lseg > 0 chunks per segment) also seg_off[n] = number of segments of
// samples 0..n-1, every sample having at least one (an empty sample has one, empty).
// order[r] = the sample with the r-th most chunks (ties by index) for packs of at most
// 1024 samples, else r: chain units walk samples longest first, so the chains that set
// the length of a pass start first when CUs free up.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void kda_bwd_plan_kernel(const int32_t* __restrict__ cu,
                                                            int32_t* __restrict__ chunk_off, int32_t* __restrict__ seg_off,
                                                            int32_t* __restrict__ order, int num_seqs,
                                                            int64_t total_tokens, int lseg)
{
    __shared__ int32_t part[1024], spart[1024], len[1024];
    const int tid = threadIdx.x;
    int32_t carry = 0, scarry = 0;
    for (int base = 0; base < num_seqs; base += 1024) {
        const int n = base + tid;
        int32_t cnt = 0, scnt = 0;
        if (n < num_seqs) {
            const int64_t s0 = min<int64_t>(max<int64_t>(cu[n], 0), total_tokens);
            const int64_t s1 = min<int64_t>(max<int64_t>(cu[n + 1], s0), total_tokens);
            cnt = int32_t((s1 - s0 + kBC - 1) / kBC);
            scnt = lseg > 0 ? max(1, (cnt + lseg - 1) / lseg) : 1;
        }
        part[tid] = cnt;
        spart[tid] = scnt;
        len[tid] = cnt;
        __syncthreads();
        if (num_seqs <= 1024 && n < num_seqs) {     // one block of samples: rank by length
            int rank = 0;
            for (int j = 0; j < num_seqs; ++j) rank += len[j] > cnt || (len[j] == cnt && j < n);
            order[rank] = n;
        } else if (n < num_seqs) {
            order[n] = n;
        }
        for (int d = 1; d < 1024; d <<= 1) {
            const int32_t add = tid >= d ? part[tid - d] : 0;
            const int32_t sadd = tid >= d ? spart[tid - d] : 0;
            __syncthreads();
            part[tid] += add;
            spart[tid] += sadd;
            __syncthreads();
        }
        if (n < num_seqs) {
            chunk_off[n + 1] = carry + part[tid];
            if (seg_off) seg_off[n + 1] = scarry + spart[tid];
        }
        carry += part[1023];
        scarry += spart[1023];
        __syncthreads();
    }
    if (tid == 0) {
        chunk_off[0] = 0;
        if (seg_off) seg_off[0] = 0;
    }
}

__device__ __forceinline__ void bounds(const int32_t* cu, int n, int64_t T, int64_t& s0, int64_t& s1) {
    s0 = min<int64_t>(max<int64_t>(cu[n], 0), T);
    s1 = min<int64_t>(max<int64_t>(cu[n + 1], s0), T);
}

// sample owning global chunk c (chunk_off[n] <= c < chunk_off[n + 1]), or -1 past the end
__device__ __forceinline__ int owner(const int32_t* chunk_off, int num_seqs, int c, int max_chunks) {
    const int ntot = min(chunk_off[num_seqs], max_chunks);
    if (c >= ntot) return -1;
    int lo = 0, hi = num_seqs;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (chunk_off[mid] <= c) lo = mid; else hi = mid;
    }
    return lo;
}

// The chunks a chain workgroup walks. Without the split (lseg == 0) a unit is a
// (sample, head) and walks the whole sample; with it a unit is a (segment, head):
// segment sid is segment `seg` of `nseg` of sample n (seg_off[n] <= sid < seg_off[n+1]),
// chunks [c0, c1) starting at token t0. Returns false past the last segment.
struct ChainSpan {
    int n, seg, nseg, c0, c1;
    int64_t t0, s1;                 // first token of the span, end of the sample
};
__device__ __forceinline__ bool chain_span(int sid, const int32_t* cu, const int32_t* chunk_off,
                                           const int32_t* seg_off, const int32_t* order, int num_seqs, int lseg,
                                           int max_chunks, int max_segs, int64_t T, ChainSpan& o) {
    int n = sid, seg = 0, nseg = 1;
    if (lseg > 0) {
        if (sid >= min(seg_off[num_seqs], max_segs)) return false;
        int lo = 0, hi = num_seqs;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (seg_off[mid] <= sid) lo = mid; else hi = mid;
        }
        n = lo;
        seg = sid - seg_off[n];
        nseg = seg_off[n + 1] - seg_off[n];
    } else if (sid >= num_seqs) {
        return false;
    } else {
        n = order[sid];                 // samples longest first
    }
    const int cs0 = min(chunk_off[n], max_chunks), cs1 = min(chunk_off[n + 1], max_chunks);
    o.n = n;
    o.seg = seg;
    o.nseg = nseg;
    o.c0 = lseg > 0 ? min(cs0 + seg * lseg, cs1) : cs0;
    o.c1 = lseg > 0 ? min(o.c0 + lseg, cs1) : cs1;
    int64_t s0;
    bounds(cu, n, T, s0, o.s1);
    o.t0 = s0 + int64_t(o.c0 - cs0) * kBC;
    return true;
}

// ---------------------------------------------------------------------------
// operands of one chunk in LDS: Qh, Kh, Kc (row stride LK), gamma, b, M, P, T
// ---------------------------------------------------------------------------
struct ChunkLds {
    float *qh, *kh, *kc;    // [C][LK]
    float *m, *t, *p;       // [C][kLC]
    float *gam, *beta;      // [DK], [C]
    float *qinv, *kinv;     // [C]: 1/|q_t|, 1/|k_t| (1 without normalisation)
};

// Cumulative sums down the C = 32 rows of a [C][ld] fp32 LDS array on fp32 MFMA, as a
// product with a triangular ones matrix: UPPER = false gives the inclusive prefix sum
// G[i] = sum_{k <= i} X[k], UPPER = true the suffix sum over the rows k >= i, k < nrow.
// Wave w takes the column tiles w * NCT / 4 ..; lane (r, g) receives the sums of rows
// 16 ti + 4 g + v, column 16 tj + r in out[ti][tj'][v] (tj' the wave's tile index).
template <int NCT, bool UPPER>
__device__ __forceinline__ void tri_cumsum(const float* __restrict__ x, int ld, int nrow, int wave, int r, int g,
                                           f32x4 (&out)[2][NCT / 4]) {
#pragma unroll
    for (int u = 0; u < NCT / 4; ++u) {
        const int tj = wave * (NCT / 4) + u;
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            f32x4 acc = zero4();
#pragma unroll
            for (int k0 = UPPER ? 16 * ti : 0; k0 < (UPPER ? kBC : 16 * ti + 16); k0 += 4) {
                const int i = 16 * ti + r, kk = k0 + g;
                const float a = UPPER ? ((kk >= i && kk < nrow) ? 1.f : 0.f) : (kk <= i ? 1.f : 0.f);
                acc = mma4(a, x[kk * ld + 16 * tj + r], acc);
            }
            out[ti][u] = acc;
        }
    }
}

// X Y from accumulator tiles of X^T and Y (16 x 16, fp32): with k = 4g + s in step s,
// element s of a tile is directly the operand
__device__ __forceinline__ f32x4 mm16(const f32x4& xt, const f32x4& y) {
    f32x4 c = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(xt[s], y[s], c, 0, 0, 0);
    return c;
}

template <typename E, int DK, bool NORM>
__device__ void chunk_operands(const ChunkLds& L, const E* __restrict__ q, const E* __restrict__ k,
                               const E* __restrict__ la, const E* __restrict__ beta, int64_t t0, int nrow,
                               int H, int h)
{
    constexpr int LK = DK + 4;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;
    // raw q, k, log a rows to LDS (zeros past the sample's end); log a goes where Kc
    // will be. Every load is issued before the first LDS write.
    RowPieces<E, DK> pq, pk, pl;
    pq.load(q, t0, nrow, H, h, 0, DK);
    pk.load(k, t0, nrow, H, h, 0, DK);
    pl.load(la, t0, nrow, H, h, 0, DK);
    const float bv = tid < nrow ? ldf(beta + (t0 + min(tid, nrow - 1)) * H + h) : 0.f;
    pq.put(L.qh, LK, nrow);
    pk.put(L.kh, LK, nrow);
    pl.put(L.kc, LK, nrow);
    if (tid < kBC) L.beta[tid] = bv;
    __syncthreads();
    if constexpr (NORM) {
        // 8 lanes per row, DK/8 channels each
        const int row = tid >> 3, part = tid & 7;
        float sq = 0.f, sk = 0.f;
        for (int c = part; c < DK; c += 8) {
            const float a = L.qh[row * LK + c], b = L.kh[row * LK + c];
            sq += a * a;
            sk += b * b;
        }
#pragma unroll
        for (int m = 1; m < 8; m <<= 1) {
            sq += __shfl_xor(sq, m);
            sk += __shfl_xor(sk, m);
        }
        if (part == 0) {
            L.qinv[row] = sq > 0.f ? 1.f / sqrtf(sq) : 0.f;
            L.kinv[row] = sk > 0.f ? 1.f / sqrtf(sk) : 0.f;
        }
        __syncthreads();
    } else {
        if (tid < kBC) {
            L.qinv[tid] = 1.f;
            L.kinv[tid] = 1.f;
        }
    }
    // cumulative log decay down each key channel (rows past the sample's end add 0), the
    // decayed operands and gamma; each wave reads and writes only its own column tiles
    {
        constexpr int NCT = DK / 16;
        f32x4 G[2][NCT / 4];
        tri_cumsum<NCT, false>(L.kc, LK, kBC, wave, r, g, G);
#pragma unroll
        for (int u = 0; u < NCT / 4; ++u) {
            const int c = 16 * (wave * (NCT / 4) + u) + r;
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int row = 16 * ti + 4 * g + v;
                    const float ex = expf(G[ti][u][v]);
                    const float qv = L.qh[row * LK + c] * (NORM ? L.qinv[row] : 1.f);
                    const float kv = L.kh[row * LK + c] * (NORM ? L.kinv[row] : 1.f);
                    L.qh[row * LK + c] = qv * ex;
                    L.kh[row * LK + c] = kv * ex;
                    L.kc[row * LK + c] = kv * expf(-G[ti][u][v]);
                    if (row == kBC - 1) L.gam[c] = ex;
                }
        }
    }
    __syncthreads();
    // M = Kh Kc^T and P = LowerIncl(Qh Kc^T): wave w computes tile (w >> 1, w & 1) of each
    {
        const int ti = wave >> 1, tj = wave & 1;
        f32x4 am = zero4(), ap = zero4();
#pragma unroll 8
        for (int k0 = 0; k0 < DK; k0 += 4) {
            const float bk = L.kc[(16 * tj + r) * LK + k0 + g];
            am = mma4(L.kh[(16 * ti + r) * LK + k0 + g], bk, am);
            ap = mma4(L.qh[(16 * ti + r) * LK + k0 + g], bk, ap);
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = 16 * ti + 4 * g + v, j = 16 * tj + r;
            L.m[i * kLC + j] = am[v];
            L.p[i * kLC + j] = i >= j ? ap[v] : 0.f;
        }
    }
    __syncthreads();
    // T = (I + A)^-1, A = StrictLower(diag(b) M), by 16-row blocks:
    //   T_bb = (I + A_bb)^-1 = (I - A)(I + A^2)(I + A^4)(I + A^8) exactly (A_bb^16 = 0),
    //   T_10 = -T_11 A_10 T_00,  T_01 = 0.
    if (wave < 2) {
        const int b = wave;
        f32x4 ac, at, id;                       // A_bb, A_bb^T, I as accumulator tiles
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int i = 16 * b + 4 * g + s, j = 16 * b + r;       // A_bb[4g + s][r]
            ac[s] = 4 * g + s > r ? L.beta[i] * L.m[i * kLC + j] : 0.f;
            const int i2 = 16 * b + r, j2 = 16 * b + 4 * g + s;     // A_bb[r][4g + s]
            at[s] = r > 4 * g + s ? L.beta[i2] * L.m[i2 * kLC + j2] : 0.f;
            id[s] = 4 * g + s == r ? 1.f : 0.f;
        }
        const f32x4 b1 = mm16(at, ac), b1t = mm16(ac, at);         // A^2, (A^2)^T
        const f32x4 b2 = mm16(b1t, b1), b2t = mm16(b1, b1t);       // A^4, (A^4)^T
        const f32x4 b3 = mm16(b2t, b2);                            // A^8
        const f32x4 x1t = id - at + b1t - mm16(b1, at);            // ((I - A)(I + A^2))^T
        const f32x4 x2t = x1t + mm16(b2, x1t);                     // (.. (I + A^4))^T
        const f32x4 tt = x2t + mm16(b3, x2t);                      // T_bb^T: T_bb[r][4g + s]
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            L.t[(16 * b + r) * kLC + 16 * b + 4 * g + s] = tt[s];
            if (b == 0) L.t[r * kLC + 16 + 4 * g + s] = 0.f;
        }
    }
    __syncthreads();
    if (wave == 2) {
        f32x4 a10t, t00, t11t;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            a10t[s] = L.beta[16 + r] * L.m[(16 + r) * kLC + 4 * g + s];   // A_10[r][4g + s]
            t00[s] = L.t[(4 * g + s) * kLC + r];                         // T_00[4g + s][r]
            t11t[s] = L.t[(16 + r) * kLC + 16 + 4 * g + s];              // T_11[r][4g + s]
        }
        const f32x4 z = mm16(a10t, t00);                                // A_10 T_00
        const f32x4 t10 = mm16(t11t, z);                                // T_11 A_10 T_00
#pragma unroll
        for (int v = 0; v < 4; ++v) L.t[(16 + 4 * g + v) * kLC + r] = -t10[v];
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// prep: the records the chains read
// ---------------------------------------------------------------------------
template <int DK> struct PrepLds {
    static constexpr int LK = DK + 4;
    float qh[kBC * LK], kh[kBC * LK], kc[kBC * LK];
    float m[kBC * kLC], t[kBC * kLC], p[kBC * kLC];
    float gam[DK], beta[kBC], qinv[kBC], kinv[kBC];
};

template <typename E, int DK, bool NORM>
__global__ __launch_bounds__(kBT) void kda_bwd_prep_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ la, const E* __restrict__ beta,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_off, float* __restrict__ rec_ws,
    int num_seqs, int H, int64_t total_tokens, int max_chunks)
{
    using R = BRec<DK>;
    constexpr int LK = DK + 4;
    extern __shared__ __align__(16) unsigned char smem_raw[];
    PrepLds<DK>& sm = *reinterpret_cast<PrepLds<DK>*>(smem_raw);
    const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    const int n = owner(chunk_off, num_seqs, c, max_chunks);
    if (n < 0) return;
    int64_t s0, s1;
    bounds(cu, n, total_tokens, s0, s1);
    const int64_t t0 = s0 + int64_t(c - chunk_off[n]) * kBC;
    const int nrow = int(min<int64_t>(kBC, s1 - t0));
    const ChunkLds L{sm.qh, sm.kh, sm.kc, sm.m, sm.t, sm.p, sm.gam, sm.beta, sm.qinv, sm.kinv};
    chunk_operands<E, DK, NORM>(L, q, k, la, beta, t0, nrow, H, h);
    float* rec = rec_ws + (int64_t(h) * max_chunks + c) * R::TOTAL;
    for (int i = tid; i < kBC * DK; i += kBT) {
        const int row = i / DK, cc = i % DK;
        rec[R::KH + i] = sm.kh[row * LK + cc];
        rec[R::KC + i] = sm.kc[row * LK + cc];
        rec[R::QH + i] = sm.qh[row * LK + cc];
    }
    for (int i = tid; i < kBC * kBC; i += kBT) {
        rec[R::T + i] = sm.t[(i / kBC) * kLC + i % kBC];
        rec[R::P + i] = sm.p[(i / kBC) * kLC + i % kBC];
        rec[R::M + i] = sm.m[(i / kBC) * kLC + i % kBC];
    }
    if (tid < DK) rec[R::GAM + tid] = sm.gam[tid];
    if (tid < kBC) {
        rec[R::BETA + tid] = sm.beta[tid];
        rec[R::QINV + tid] = sm.qinv[tid];
        rec[R::KINV + tid] = sm.kinv[tid];
    }
}

// The chunk operands of the gradient kernel, read back from the prep's record into the
// LDS layout chunk_operands() builds (the same values, so the same gradients). load()
// issues every 16-byte load into registers; put() writes them to LDS (the caller then
// takes a barrier), so that loads issued between the two stay in flight.
template <int DK> struct RecordRegs {
    using R = BRec<DK>;
    static constexpr int LK = DK + 4;
    static constexpr int NK = kBC * DK / 4 / kBT;   // f32x4 per thread per [C][DK] array
    static constexpr int NG = DK / 4, NB = kBC / 4;
    static_assert(kBC * kBC / 4 == kBT, "one f32x4 of each [C][C] array per thread");
    f32x4 kh[NK], kc[NK], qh[NK], t, p, m, small;   // small: gamma, b, 1/|q|, 1/|k|
    __device__ __forceinline__ void load(const float* __restrict__ rec) {
        const int tid = threadIdx.x;
        const f32x4* r4 = reinterpret_cast<const f32x4*>(rec);
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const int i = tid + j * kBT;
            kh[j] = r4[R::KH / 4 + i];
            kc[j] = r4[R::KC / 4 + i];
            qh[j] = r4[R::QH / 4 + i];
        }
        t = r4[R::T / 4 + tid];
        p = r4[R::P / 4 + tid];
        m = r4[R::M / 4 + tid];
        small = zero4();
        if (tid < NG) small = r4[R::GAM / 4 + tid];
        else if (tid < NG + NB) small = r4[R::BETA / 4 + tid - NG];
        else if (tid < NG + 2 * NB) small = r4[R::QINV / 4 + tid - NG - NB];
        else if (tid < NG + 3 * NB) small = r4[R::KINV / 4 + tid - NG - 2 * NB];
    }
    __device__ __forceinline__ void put(const ChunkLds& L) const {
        const int tid = threadIdx.x;
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            const int e = 4 * (tid + j * kBT), row = e / DK, col = e % DK;
            *reinterpret_cast<f32x4*>(L.kh + row * LK + col) = kh[j];
            *reinterpret_cast<f32x4*>(L.kc + row * LK + col) = kc[j];
            *reinterpret_cast<f32x4*>(L.qh + row * LK + col) = qh[j];
        }
        {
            const int e = 4 * tid, row = e / kBC, col = e % kBC;
            *reinterpret_cast<f32x4*>(L.t + row * kLC + col) = t;
            *reinterpret_cast<f32x4*>(L.p + row * kLC + col) = p;
            *reinterpret_cast<f32x4*>(L.m + row * kLC + col) = m;
        }
        if (tid < NG) *reinterpret_cast<f32x4*>(L.gam + 4 * tid) = small;
        else if (tid < NG + NB) *reinterpret_cast<f32x4*>(L.beta + 4 * (tid - NG)) = small;
        else if (tid < NG + 2 * NB) *reinterpret_cast<f32x4*>(L.qinv + 4 * (tid - NG - NB)) = small;
        else if (tid < NG + 3 * NB) *reinterpret_cast<f32x4*>(L.kinv + 4 * (tid - NG - 2 * NB)) = small;
    }
};

// ---------------------------------------------------------------------------
// chains: one workgroup per (sample, head, 64-column value tile); wave w holds columns
// 16w..16w+15 of the tile of S (or dS) as DK/16 accumulator tiles
// ---------------------------------------------------------------------------
template <int DK> struct ChainLds {
    static constexpr int LK = DK + 4, LV = 64 + 4;
    float qh[kBC * LK], kh[kBC * LK], kc[kBC * LK];
    float t[kBC * kLC], p[kBC * kLC];
    float vt[kBC * LV];                 // V (state chain) or dO (gradient chain) tile
    float gam[DK], beta[kBC];
};

// unit of block b: the value tiles of one (sample, head) are 8 blocks apart (same XCD)
__device__ __forceinline__ void chain_unit(int b, int nvt, int& unit, int& vt) {
    vt = (b >> 3) % nvt;
    unit = (b / (8 * nvt)) * 8 + (b & 7);
}

// The record of one chunk and a [C][64] tile of V or dO, held in registers: loaded one
// chunk ahead, written to LDS once the previous chunk's products are done.
template <typename E, int DK, bool GRAD> struct ChainFetch {
    using R = BRec<DK>;
    static constexpr int NKP = kBC * DK / 4 / kBT;      // f32x4 per thread per [C][DK] array
    static constexpr int NGB = (DK + kBC) / 4;          // f32x4 pieces of gamma and b
    static_assert(kBC * kBC / 4 == kBT, "one f32x4 of T and of P per thread");
    f32x4 kh[NKP], kc[NKP], qh[GRAD ? NKP : 1];
    f32x4 t, p, gb;
    RowPieces<E, 64> vt;
    int nrow;
    __device__ __forceinline__ void load(const float* __restrict__ rec, const E* __restrict__ src, int64_t t0,
                                         int nrow_, int H, int h, int DV, int col0) {
        const int tid = threadIdx.x;
        nrow = nrow_;
#pragma unroll
        for (int j = 0; j < NKP; ++j) {
            kh[j] = *reinterpret_cast<const f32x4*>(rec + R::KH + 4 * (tid + j * kBT));
            kc[j] = *reinterpret_cast<const f32x4*>(rec + R::KC + 4 * (tid + j * kBT));
            if constexpr (GRAD) qh[j] = *reinterpret_cast<const f32x4*>(rec + R::QH + 4 * (tid + j * kBT));
        }
        t = *reinterpret_cast<const f32x4*>(rec + R::T + 4 * tid);
        if constexpr (GRAD) p = *reinterpret_cast<const f32x4*>(rec + R::P + 4 * tid);
        gb = *reinterpret_cast<const f32x4*>(rec + R::GAM + 4 * min(tid, NGB - 1));
        vt.load(src, t0, nrow, H, h, col0, DV);
    }
    __device__ __forceinline__ void put(ChainLds<DK>& sm) const {
        constexpr int LK = DK + 4, LV = 64 + 4;
        const int tid = threadIdx.x;
#pragma unroll
        for (int j = 0; j < NKP; ++j) {
            const int i = 4 * (tid + j * kBT), row = i / DK, c = i % DK;
            *reinterpret_cast<f32x4*>(&sm.kh[row * LK + c]) = kh[j];
            *reinterpret_cast<f32x4*>(&sm.kc[row * LK + c]) = kc[j];
            if constexpr (GRAD) *reinterpret_cast<f32x4*>(&sm.qh[row * LK + c]) = qh[j];
        }
        const int i = 4 * tid, row = i / kBC, c = i % kBC;
        *reinterpret_cast<f32x4*>(&sm.t[row * kLC + c]) = t;
        if constexpr (GRAD) *reinterpret_cast<f32x4*>(&sm.p[row * kLC + c]) = p;
        if (tid < NGB) {
            if (4 * tid < DK) *reinterpret_cast<f32x4*>(&sm.gam[4 * tid]) = gb;
            else *reinterpret_cast<f32x4*>(&sm.beta[4 * tid - DK]) = gb;
        }
        vt.put(sm.vt, LV, nrow);
    }
};

// Sequence split of the chains (lseg > 0), for packs whose (sample, head) units are too
// few to fill the GPU. Each chunk maps the state affinely: S_out = M S_in + b, and the
// gradient back: dS_in = M^T dS_out + e. Over a segment of chunks the state pass gives
// both parts: started from zero it gives the segment's b (S_loc), started from the
// identity with V = 0 it gives the product of the M (Phi, d_k columns); the gradient
// pass started from zero gives the segment's e. So:
//   MODE 1 state:     per segment, S_loc (value tiles) and Phi (d_k / 64 more tiles);
//   MODE 2 state:     S_in(seg) = Phi(k) S_in(k) + S_loc(k) over the sample's earlier
//                     segments k (from the initial state), then the segment with the
//                     state entering each chunk saved, as MODE 0 does for a sample;
//   MODE 1 gradient:  per segment, e from dS = 0 at its end;
//   MODE 2 gradient:  dS at the segment's end = Phi(k)^T dS + e(k) over the later
//                     segments k, from d_final_state, then the segment as MODE 0.
// Samples of one segment skip MODE 1. The arithmetic stays fp32 throughout.
template <int DK, int DV>
__device__ __forceinline__ void seg_prefix_state(f32x4 (&S)[DK / 16], const float* __restrict__ phi,
                                                 const float* __restrict__ sloc, int sid0, int nk, int H, int h,
                                                 int col, int r, int g) {
    constexpr int NCT = DK / 16;
    for (int k = 0; k < nk; ++k) {
        const int64_t ks = int64_t(sid0 + k) * H + h;
        const float* ph = phi + ks * DK * DK;
        const float* sl = sloc + ks * DK * DV;
        f32x4 nS[NCT];
#pragma unroll
        for (int t2 = 0; t2 < NCT; ++t2) {
            f32x4 acc;
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) acc[v4] = sl[int64_t(16 * t2 + 4 * g + v4) * DV + col];
#pragma unroll
            for (int ti = 0; ti < NCT; ++ti) {
                const f32x4 a4 = *reinterpret_cast<const f32x4*>(ph + int64_t(16 * t2 + r) * DK + 16 * ti + 4 * g);
#pragma unroll
                for (int st = 0; st < 4; ++st) acc = mma4(a4[st], S[ti][st], acc);
            }
            nS[t2] = acc;
        }
#pragma unroll
        for (int t2 = 0; t2 < NCT; ++t2) S[t2] = nS[t2];
    }
}

// phi_t holds each Phi transposed, so that Phi^T is read like Phi above
template <int DK, int DV>
__device__ __forceinline__ void seg_prefix_grad(f32x4 (&dS)[DK / 16], const float* __restrict__ phi_t,
                                                const float* __restrict__ eseg, int sid_last, int sid_stop, int H,
                                                int h, int col, int r, int g) {
    constexpr int NCT = DK / 16;
    for (int sid = sid_last; sid > sid_stop; --sid) {
        const int64_t ks = int64_t(sid) * H + h;
        const float* pt = phi_t + ks * DK * DK;
        const float* es = eseg + ks * DK * DV;
        f32x4 nS[NCT];
#pragma unroll
        for (int t2 = 0; t2 < NCT; ++t2) {
            f32x4 acc;
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) acc[v4] = es[int64_t(16 * t2 + 4 * g + v4) * DV + col];
#pragma unroll
            for (int ti = 0; ti < NCT; ++ti) {
                const f32x4 a4 = *reinterpret_cast<const f32x4*>(pt + int64_t(16 * t2 + r) * DK + 16 * ti + 4 * g);
#pragma unroll
                for (int st = 0; st < 4; ++st) acc = mma4(a4[st], dS[ti][st], acc);
            }
            nS[t2] = acc;
        }
#pragma unroll
        for (int t2 = 0; t2 < NCT; ++t2) dS[t2] = nS[t2];
    }
}

template <typename E, int DK, int DV, int MODE>
__global__ __launch_bounds__(kBT) void kda_bwd_state_kernel(
    const E* __restrict__ v, const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_off,
    const int32_t* __restrict__ seg_off, const int32_t* __restrict__ order, const float* __restrict__ rec_ws,
    const float* __restrict__ init_state,
    float* __restrict__ s_in, float* __restrict__ sloc, float* __restrict__ phi, float* __restrict__ phi_t,
    int num_seqs, int H, int64_t total_tokens, int max_chunks, int lseg, int max_segs)
{
    using R = BRec<DK>;
    constexpr int NCT = DK / 16, LK = DK + 4, LV = 64 + 4;
    constexpr int NT = MODE == 1 ? DV / 64 + DK / 64 : DV / 64;     // column tiles per unit
    constexpr bool kBf = sizeof(E) == 2;                            // bf16 data: bf16 products
    extern __shared__ __align__(16) unsigned char smem_raw[];
    ChainLds<DK>& sm = *reinterpret_cast<ChainLds<DK>*>(smem_raw);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
    int unit, tile;
    chain_unit(blockIdx.x, NT, unit, tile);
    const int sid = unit / H, h = unit % H;
    ChainSpan sp;
    if (!chain_span(sid, cu, chunk_off, seg_off, order, num_seqs, MODE == 0 ? 0 : lseg, max_chunks, max_segs, total_tokens,
                    sp))
        return;
    if (MODE == 1 && sp.nseg == 1) return;
    const int n = sp.n;
    const bool trans = MODE == 1 && tile >= DV / 64;                 // a tile of Phi: identity start, V = 0
    const int vt = trans ? 0 : tile;
    const int col = 64 * (trans ? tile - DV / 64 : tile) + 16 * wave + r;   // this lane's column
    const int c0 = sp.c0, c1 = sp.c1;

    f32x4 S[NCT];
#pragma unroll
    for (int ti = 0; ti < NCT; ++ti) {
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const int row = 16 * ti + 4 * g + v4;
            S[ti][v4] = trans ? (row == col ? 1.f : 0.f)
                              : (init_state && MODE != 1 ? init_state[((int64_t(n) * H + h) * DK + row) * DV + col] : 0.f);
        }
    }
    if constexpr (MODE == 2) seg_prefix_state<DK, DV>(S, phi, sloc, sid - sp.seg, sp.seg, H, h, col, r, g);
    ChainFetch<E, DK, false> f;
    auto fetch = [&](int cc) __attribute__((always_inline)) {
        const int64_t t0 = sp.t0 + int64_t(cc - c0) * kBC;
        f.load(rec_ws + (int64_t(h) * max_chunks + cc) * R::TOTAL, v, t0, int(min<int64_t>(kBC, sp.s1 - t0)), H, h,
               DV, 64 * vt);
    };
    if (c0 < c1) fetch(c0);
    for (int cc = c0; cc < c1; ++cc) {
        f.put(sm);
        __syncthreads();
        if constexpr (MODE != 1) {
            float* so = s_in + (int64_t(h) * max_chunks + cc) * DK * DV;
#pragma unroll
            for (int ti = 0; ti < NCT; ++ti)
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) so[(16 * ti + 4 * g + v4) * DV + col] = S[ti][v4];
        }
        fetch(min(cc + 1, c1 - 1));                       // in flight during this chunk's products
        // X = V - Kh S, then Y = diag(b) X (rows 16xi + 4g + v)
        f32x4 Y[2], Vn[2];
        if constexpr (kBf) {
            BF2 sf[NCT / 2];
#pragma unroll
            for (int b = 0; b < NCT / 2; ++b) sf[b] = bf_split(S[2 * b], S[2 * b + 1]);
#pragma unroll
            for (int b = 0; b < NCT / 2; b += 2) ready(sf[b], sf[b + 1]);
#pragma unroll
            for (int xi = 0; xi < 2; ++xi) {
                BF2 a[NCT / 2];
#pragma unroll
                for (int b = 0; b < NCT / 2; ++b) a[b] = bf_row(sm.kh, LK, 16 * xi + r, 32 * b, g);
#pragma unroll
                for (int b = 0; b < NCT / 2; b += 2) ready(a[b], a[b + 1]);
                f32x4 acc = zero4();
#pragma unroll
                for (int b = 0; b < NCT / 2; ++b) acc = mm3(a[b], sf[b], acc);
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const int row = 16 * xi + 4 * g + v4;
                    const float vv = trans ? 0.f : sm.vt[row * LV + 16 * wave + r];
                    Y[xi][v4] = sm.beta[row] * (vv - acc[v4]);
                }
            }
            // Vn = T Y
            BF2 yf = bf_split(Y[0], Y[1]), ta[2];
#pragma unroll
            for (int vi = 0; vi < 2; ++vi) ta[vi] = bf_row(sm.t, kLC, 16 * vi + r, 0, g);
            ready(yf);
            ready(ta[0], ta[1]);
#pragma unroll
            for (int vi = 0; vi < 2; ++vi) Vn[vi] = mm3(ta[vi], yf, zero4());
            // S <- diag(gamma) (S + Kc^T Vn)
            BF2 vf = bf_split(Vn[0], Vn[1]);
            ready(vf);
#pragma unroll
            for (int ti = 0; ti < NCT; ti += 2) {
                BF2 ka = bf_col(sm.kc, LK, 16 * ti + r, g), kb = bf_col(sm.kc, LK, 16 * (ti + 1) + r, g);
                ready(ka, kb);
                const f32x4 a0 = mm3(ka, vf, zero4()), a1 = mm3(kb, vf, zero4());
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    S[ti][v4] = sm.gam[16 * ti + 4 * g + v4] * (S[ti][v4] + a0[v4]);
                    S[ti + 1][v4] = sm.gam[16 * (ti + 1) + 4 * g + v4] * (S[ti + 1][v4] + a1[v4]);
                }
            }
        } else {
#pragma unroll
            for (int xi = 0; xi < 2; ++xi) {
                f32x4 acc = zero4();
#pragma unroll
                for (int ti = 0; ti < NCT; ++ti)
#pragma unroll
                    for (int st = 0; st < 4; ++st) acc = mma4(sm.kh[(16 * xi + r) * LK + 16 * ti + 4 * g + st], S[ti][st], acc);
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) {
                    const int row = 16 * xi + 4 * g + v4;
                    const float vv = trans ? 0.f : sm.vt[row * LV + 16 * wave + r];
                    Y[xi][v4] = sm.beta[row] * (vv - acc[v4]);
                }
            }
            // Vn = T Y
#pragma unroll
            for (int vi = 0; vi < 2; ++vi) {
                f32x4 acc = zero4();
#pragma unroll
                for (int xi = 0; xi < 2; ++xi)
#pragma unroll
                    for (int st = 0; st < 4; ++st) acc = mma4(sm.t[(16 * vi + r) * kLC + 16 * xi + 4 * g + st], Y[xi][st], acc);
                Vn[vi] = acc;
            }
            // S <- diag(gamma) (S + Kc^T Vn)
#pragma unroll
            for (int ti = 0; ti < NCT; ++ti) {
                f32x4 acc = zero4();
#pragma unroll
                for (int vi = 0; vi < 2; ++vi)
#pragma unroll
                    for (int st = 0; st < 4; ++st) acc = mma4(sm.kc[(16 * vi + 4 * g + st) * LK + 16 * ti + r], Vn[vi][st], acc);
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) S[ti][v4] = sm.gam[16 * ti + 4 * g + v4] * (S[ti][v4] + acc[v4]);
            }
        }
        __syncthreads();
    }
    if constexpr (MODE == 1) {
        // the segment's S_loc (value tiles) or Phi (transition tiles)
        const int64_t ks = int64_t(sid) * H + h;
        float* dst = trans ? phi + ks * DK * DK : sloc + ks * DK * DV;
        const int ld = trans ? DK : DV;
#pragma unroll
        for (int ti = 0; ti < NCT; ++ti)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) dst[int64_t(16 * ti + 4 * g + v4) * ld + col] = S[ti][v4];
        if (trans) {                            // and Phi^T: column col of Phi is row col
            float* dt = phi_t + ks * DK * DK + int64_t(col) * DK;
#pragma unroll
            for (int ti = 0; ti < NCT; ++ti) *reinterpret_cast<f32x4*>(dt + 16 * ti + 4 * g) = S[ti];
        }
    }
}

template <typename E, int DK, int DV, int MODE>
__global__ __launch_bounds__(kBT) void kda_bwd_dstate_kernel(
    const E* __restrict__ d_out, const int32_t* __restrict__ cu, const int32_t* __restrict__ chunk_off,
    const int32_t* __restrict__ seg_off, const int32_t* __restrict__ order, const float* __restrict__ rec_ws,
    const float* __restrict__ d_final,
    float* __restrict__ ds_out, float* __restrict__ d_init, const float* __restrict__ phi_t, float* __restrict__ eseg,
    int num_seqs, int H, int64_t total_tokens, int max_chunks, int lseg, int max_segs)
{
    using R = BRec<DK>;
    constexpr int NCT = DK / 16, LK = DK + 4, LV = 64 + 4;
    constexpr bool kBf = sizeof(E) == 2;                            // bf16 data: bf16 products
    extern __shared__ __align__(16) unsigned char smem_raw[];
    ChainLds<DK>& sm = *reinterpret_cast<ChainLds<DK>*>(smem_raw);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
    int unit, vt;
    chain_unit(blockIdx.x, DV / 64, unit, vt);
    const int sid = unit / H, h = unit % H;
    ChainSpan sp;
    if (!chain_span(sid, cu, chunk_off, seg_off, order, num_seqs, MODE == 0 ? 0 : lseg, max_chunks, max_segs, total_tokens,
                    sp))
        return;
    if (MODE == 1 && sp.nseg == 1) return;
    const int n = sp.n;
    const int col = 64 * vt + 16 * wave + r;
    const int c0 = sp.c0, c1 = sp.c1;

    f32x4 dS[NCT];
#pragma unroll
    for (int ti = 0; ti < NCT; ++ti)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
            dS[ti][v4] = d_final && MODE != 1 ? d_final[((int64_t(n) * H + h) * DK + 16 * ti + 4 * g + v4) * DV + col] : 0.f;
    if constexpr (MODE == 2)
        seg_prefix_grad<DK, DV>(dS, phi_t, eseg, sid - sp.seg + sp.nseg - 1, sid, H, h, col, r, g);
    ChainFetch<E, DK, true> f;
    auto fetch = [&](int cc) __attribute__((always_inline)) {
        const int64_t t0 = sp.t0 + int64_t(cc - c0) * kBC;
        f.load(rec_ws + (int64_t(h) * max_chunks + cc) * R::TOTAL, d_out, t0, int(min<int64_t>(kBC, sp.s1 - t0)),
               H, h, DV, 64 * vt);
    };
    if (c0 < c1) fetch(c1 - 1);
    for (int cc = c1 - 1; cc >= c0; --cc) {
        f.put(sm);
        __syncthreads();
        if constexpr (MODE != 1) {
            float* so = ds_out + (int64_t(h) * max_chunks + cc) * DK * DV;
#pragma unroll
            for (int ti = 0; ti < NCT; ++ti)
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) so[(16 * ti + 4 * g + v4) * DV + col] = dS[ti][v4];
        }
        fetch(max(cc - 1, c0));                           // in flight during this chunk's products
        f32x4 dVn[2], dX[2];
        if constexpr (kBf) {
            // dVn = P^T dO + Kc diag(gamma) dS
            BF2 df[NCT / 2];
#pragma unroll
            for (int b = 0; b < NCT / 2; ++b) df[b] = bf_split(dS[2 * b], dS[2 * b + 1]);
#pragma unroll
            for (int b = 0; b < NCT / 2; b += 2) ready(df[b], df[b + 1]);
            BF dof;                                                         // dO as B (exact in bf16)
            {
                float f[8];
                col8(sm.vt, LV, 16 * wave + r, g, f);
                dof = bf_pack(f);
            }
#pragma unroll
            for (int vi = 0; vi < 2; ++vi) {
                BF2 pa = bf_col(sm.p, kLC, 16 * vi + r, g);
                BF2 a[NCT / 2];
#pragma unroll
                for (int b = 0; b < NCT / 2; ++b) {
                    const float* kr = sm.kc + (16 * vi + r) * LK + 32 * b + 4 * g;
                    const float* gr = sm.gam + 32 * b + 4 * g;
                    const float4 k0 = *reinterpret_cast<const float4*>(kr), k1 = *reinterpret_cast<const float4*>(kr + 16);
                    const float4 g0 = *reinterpret_cast<const float4*>(gr), g1 = *reinterpret_cast<const float4*>(gr + 16);
                    const float f[8] = {k0.x * g0.x, k0.y * g0.y, k0.z * g0.z, k0.w * g0.w,
                                        k1.x * g1.x, k1.y * g1.y, k1.z * g1.z, k1.w * g1.w};
                    a[b] = bf_split(f);
                }
                mfma_ready(pa.h.u, pa.l.u, dof.u, dof.u);
#pragma unroll
                for (int b = 0; b < NCT / 2; b += 2) ready(a[b], a[b + 1]);
                f32x4 acc = mm2(pa, dof, zero4());
#pragma unroll
                for (int b = 0; b < NCT / 2; ++b) acc = mm3(a[b], df[b], acc);
                dVn[vi] = acc;
            }
            // dX = diag(b) T^T dVn
            BF2 vf = bf_split(dVn[0], dVn[1]), ta[2];
#pragma unroll
            for (int zi = 0; zi < 2; ++zi) ta[zi] = bf_col(sm.t, kLC, 16 * zi + r, g);
            ready(vf);
            ready(ta[0], ta[1]);
#pragma unroll
            for (int zi = 0; zi < 2; ++zi) {
                const f32x4 acc = mm3(ta[zi], vf, zero4());
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) dX[zi][v4] = sm.beta[16 * zi + 4 * g + v4] * acc[v4];
            }
            // dS <- diag(gamma) dS + Qh^T dO - Kh^T dX
            BF2 xf = bf_split(-dX[0], -dX[1]);
            ready(xf);
#pragma unroll
            for (int ti = 0; ti < NCT; ++ti) {
                BF2 qa = bf_col(sm.qh, LK, 16 * ti + r, g), ka = bf_col(sm.kh, LK, 16 * ti + r, g);
                ready(qa, ka);
                const f32x4 acc = mm3(ka, xf, mm2(qa, dof, zero4()));
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) dS[ti][v4] = sm.gam[16 * ti + 4 * g + v4] * dS[ti][v4] + acc[v4];
            }
        } else {
            // dVn = P^T dO + Kc diag(gamma) dS
#pragma unroll
            for (int vi = 0; vi < 2; ++vi) {
                f32x4 acc = zero4();
#pragma unroll
                for (int k0 = 0; k0 < kBC; k0 += 4)
                    acc = mma4(sm.p[(k0 + g) * kLC + 16 * vi + r], sm.vt[(k0 + g) * LV + 16 * wave + r], acc);
#pragma unroll
                for (int ti = 0; ti < NCT; ++ti)
#pragma unroll
                    for (int st = 0; st < 4; ++st) {
                        const int c = 16 * ti + 4 * g + st;
                        acc = mma4(sm.kc[(16 * vi + r) * LK + c] * sm.gam[c], dS[ti][st], acc);
                    }
                dVn[vi] = acc;
            }
            // dX = diag(b) T^T dVn
#pragma unroll
            for (int zi = 0; zi < 2; ++zi) {
                f32x4 acc = zero4();
#pragma unroll
                for (int vi = 0; vi < 2; ++vi)
#pragma unroll
                    for (int st = 0; st < 4; ++st) acc = mma4(sm.t[(16 * vi + 4 * g + st) * kLC + 16 * zi + r], dVn[vi][st], acc);
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) dX[zi][v4] = sm.beta[16 * zi + 4 * g + v4] * acc[v4];
            }
            // dS <- diag(gamma) dS + Qh^T dO - Kh^T dX
#pragma unroll
            for (int ti = 0; ti < NCT; ++ti) {
                f32x4 acc = zero4();
#pragma unroll
                for (int k0 = 0; k0 < kBC; k0 += 4)
                    acc = mma4(sm.qh[(k0 + g) * LK + 16 * ti + r], sm.vt[(k0 + g) * LV + 16 * wave + r], acc);
#pragma unroll
                for (int zi = 0; zi < 2; ++zi)
#pragma unroll
                    for (int st = 0; st < 4; ++st) acc = mma4(-sm.kh[(16 * zi + 4 * g + st) * LK + 16 * ti + r], dX[zi][st], acc);
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) dS[ti][v4] = sm.gam[16 * ti + 4 * g + v4] * dS[ti][v4] + acc[v4];
            }
        }
        __syncthreads();
    }
    if constexpr (MODE == 1) {
        float* es = eseg + (int64_t(sid) * H + h) * DK * DV;
#pragma unroll
        for (int ti = 0; ti < NCT; ++ti)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) es[int64_t(16 * ti + 4 * g + v4) * DV + col] = dS[ti][v4];
    } else if (d_init && sp.seg == 0) {
#pragma unroll
        for (int ti = 0; ti < NCT; ++ti)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4)
                d_init[((int64_t(n) * H + h) * DK + 16 * ti + 4 * g + v4) * DV + col] = dS[ti][v4];
    }
}

// ---------------------------------------------------------------------------
// gradients of one (chunk, head)
// ---------------------------------------------------------------------------
template <int DK, int DV> struct GradLds {
    static constexpr int LK = DK + 4, LV = DV + 4;
    float qh[kBC * LK], kh[kBC * LK], kc[kBC * LK];
    // dead once the products are done; the last phase reuses them as one flat area
    float x[kBC * LV], dout[kBC * LV], vn[kBC * LV], dvn[kBC * LV], sblk[kBC * LV];
    float m[kBC * kLC], t[kBC * kLC], p[kBC * kLC], dp[kBC * kLC], dt[kBC * kLC];
    float gam[DK], dgam[DK], beta[kBC], dbeta[kBC], qinv[kBC], kinv[kBC];
    // partial sums of dgamma and db, one writer per slot, added in a fixed order (no
    // atomics, so the gradients are bitwise reproducible)
    float dgam_p[3][DK];                // dVn pass, token tiles 0 and 1; the state pass
    float dbeta_p[4][kBC];              // one per wave
    static_assert(5 * kBC * LV + 5 * kBC * kLC >= 3 * kBC * LK, "flat area holds three [C][DK] arrays");
};

// 32 rows (32 kb ..) of a [DK][DV] fp32 state matrix as float4 pieces in registers:
// piece j of thread i is row (i + 256 j) / (DV/4), columns 4 ((i + 256 j) % (DV/4)) ..
template <int DV> struct StateBlock {
    static constexpr int PR = DV / 4;                // f32x4 per row
    static constexpr int NP = kBC * PR / kBT;
    f32x4 v[NP];
    __device__ __forceinline__ void load(const float* __restrict__ src, int kb) {
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int pc = int(threadIdx.x) + j * kBT;
            v[j] = *reinterpret_cast<const f32x4*>(src + (32 * kb + pc / PR) * DV + 4 * (pc % PR));
        }
    }
    __device__ __forceinline__ void put(float* dst, int ld) const {
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int pc = int(threadIdx.x) + j * kBT;
            *reinterpret_cast<f32x4*>(dst + (pc / PR) * ld + 4 * (pc % PR)) = v[j];
        }
    }
};

// rows < nrow of a [C][W] fp32 LDS array (row stride ld) to rows t0.. of a [T][H][W]
// tensor of dtype E, 16 bytes per store
template <typename E, int W>
__device__ __forceinline__ void store_rows(E* __restrict__ dst, const float* src, int ld, int64_t t0, int nrow, int H,
                                           int h) {
    constexpr int EPP = 16 / sizeof(E), PPR = W / EPP;
    for (int pc = threadIdx.x; pc < kBC * PPR; pc += kBT) {
        const int row = pc / PPR, c = (pc % PPR) * EPP;
        if (row >= nrow) continue;
        E* d = dst + ((t0 + row) * H + h) * W + c;
        const float* s = src + row * ld + c;
        if constexpr (sizeof(E) == 4) {
            *reinterpret_cast<float4*>(d) = *reinterpret_cast<const float4*>(s);
        } else {
            const float4 a = *reinterpret_cast<const float4*>(s), b = *reinterpret_cast<const float4*>(s + 4);
            *reinterpret_cast<u32x4*>(d) = u32x4{pack2(a.x, a.y), pack2(a.z, a.w), pack2(b.x, b.y), pack2(b.z, b.w)};
        }
    }
}

// The [C][DK] gradients dQh, dKh, dKc live in registers. Wave w owns the 16x16 tiles
// (ti, tj) with tj = ((w - 2 ti) & 3) + 4 j', j' < DK/64, at index m = ti DK/64 + j';
// every block of 32 key channels then holds exactly one tile of each wave.
template <typename E, int DK, int DV, bool NORM>
__global__ __launch_bounds__(kBT) void kda_bwd_grad_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v, const E* __restrict__ la,
    const E* __restrict__ beta, const E* __restrict__ d_out, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ chunk_off, const float* __restrict__ rec_ws, const float* __restrict__ s_in,
    const float* __restrict__ ds_out, E* __restrict__ dq, E* __restrict__ dk, E* __restrict__ dv,
    E* __restrict__ dla, E* __restrict__ dbeta, int num_seqs, int H, int64_t total_tokens, int max_chunks)
{
    using S_ = GradLds<DK, DV>;
    constexpr int LK = S_::LK, LV = S_::LV;
    constexpr int NCT = DK / 16, NVT = DV / 16;
    constexpr int XPW = NVT / 2;            // [C][DV] tiles per wave
    constexpr int KPW = NCT / 2;            // [C][DK] tiles per wave
    constexpr int J4 = DK / 64;             // j' range of the owned tiles
    constexpr int NKB = DK / 32;            // 32-row blocks of a state matrix
    constexpr bool kBf = sizeof(E) == 2;    // bf16 data: the row-by-row products on hi/lo bf16 MFMA
    extern __shared__ __align__(16) unsigned char smem_raw[];
    S_& sm = *reinterpret_cast<S_*>(smem_raw);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;

    const int c = blockIdx.x, h = blockIdx.y;
    const int n = owner(chunk_off, num_seqs, c, max_chunks);
    if (n < 0) return;
    int64_t s0, s1;
    bounds(cu, n, total_tokens, s0, s1);
    const int64_t t0 = s0 + int64_t(c - chunk_off[n]) * kBC;
    const int nrow = int(min<int64_t>(kBC, s1 - t0));
    const float* Sg = s_in + (int64_t(h) * max_chunks + c) * DK * DV;
    const float* dSg = ds_out + (int64_t(h) * max_chunks + c) * DK * DV;

    // ---- operands, V and dO, S and dS' (every load issued before the first wait) ----
    RowPieces<E, DV> pv, pd;
    pv.load(v, t0, nrow, H, h, 0, DV);
    pd.load(d_out, t0, nrow, H, h, 0, DV);
    RecordRegs<DK> rr;
    rr.load(rec_ws + (int64_t(h) * max_chunks + c) * BRec<DK>::TOTAL);
    // the state entering the chunk and the gradient of the one leaving it stay in registers
    // from here to the last product that reads them, so each is read from memory once
    StateBlock<DV> sS[NKB], sD[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sS[kb].load(Sg, kb);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sD[kb].load(dSg, kb);
    const ChunkLds L{sm.qh, sm.kh, sm.kc, sm.m, sm.t, sm.p, sm.gam, sm.beta, sm.qinv, sm.kinv};
    rr.put(L);
    pv.put(sm.x, LV, nrow);
    pd.put(sm.dout, LV, nrow);      // the first barrier of the X pass orders these writes

    // a [C][DV]-shaped result: tile index wave + 4 mm
    auto xtile = [&](int mm, int& ti, int& tj) {
        const int tt = wave + 4 * mm;
        ti = tt / NVT;
        tj = tt % NVT;
    };
    // this wave's owned [C][DK] tile in the 32-channel block kb
    auto block_tile = [&](int kb, int& ti, int& tj) {
        ti = (((wave & 3) >> 1) == (kb & 1)) ? 0 : 1;
        tj = 4 * (kb >> 1) + ((wave - 2 * ti) & 3);
    };

    // On bf16 data the products over key channels with a state block take hi/lo bf16 MFMA
    // terms too: this wave's [C][DV] tiles mm are (mm / NTJ, wave + 4 (mm % NTJ)), so it needs
    // two row fragments (token tiles 0, 1) and NTJ column fragments of the block.
    constexpr int NTJ = NVT / 4;
    // ---- X = V - Kh S (S put into LDS one 32-row block at a time) ----
    {
        f32x4 ax[XPW];
#pragma unroll
        for (int mm = 0; mm < XPW; ++mm) ax[mm] = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            sS[kb].put(sm.sblk, LV);
            __syncthreads();
            if constexpr (kBf) {
                BF2 ka[2], sc[NTJ];
#pragma unroll
                for (int i = 0; i < 2; ++i) ka[i] = bf_row(sm.kh, LK, 16 * i + r, 32 * kb, g);
#pragma unroll
                for (int i = 0; i < NTJ; ++i) sc[i] = bf_col(sm.sblk, LV, 16 * (wave + 4 * i) + r, g);
                ready(ka[0], ka[1]);
#pragma unroll
                for (int i = 0; i < NTJ; ++i) ready(sc[i]);
#pragma unroll
                for (int mm = 0; mm < XPW; ++mm) ax[mm] = mm3(ka[mm / NTJ], sc[mm % NTJ], ax[mm]);
            } else {
#pragma unroll
                for (int mm = 0; mm < XPW; ++mm) {
                    int ti, tj;
                    xtile(mm, ti, tj);
#pragma unroll
                    for (int k0 = 0; k0 < 32; k0 += 4)
                        ax[mm] = mma4(sm.kh[(16 * ti + r) * LK + 32 * kb + k0 + g], sm.sblk[(k0 + g) * LV + 16 * tj + r],
                                      ax[mm]);
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int mm = 0; mm < XPW; ++mm) {
            int ti, tj;
            xtile(mm, ti, tj);
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) sm.x[(16 * ti + 4 * g + v4) * LV + 16 * tj + r] -= ax[mm][v4];
        }
    }
    __syncthreads();
    // ---- Vn = T diag(b) X ----
#pragma unroll
    for (int mm = 0; mm < XPW; ++mm) {
        int ti, tj;
        xtile(mm, ti, tj);
        f32x4 acc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < kBC; k0 += 4)
            acc = mma4(sm.t[(16 * ti + r) * kLC + k0 + g], sm.beta[k0 + g] * sm.x[(k0 + g) * LV + 16 * tj + r], acc);
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) sm.vn[(16 * ti + 4 * g + v4) * LV + 16 * tj + r] = acc[v4];
    }
    __syncthreads();

    f32x4 aQh[KPW], aKh[KPW], aKc[KPW];
#pragma unroll
    for (int mm = 0; mm < KPW; ++mm) {
        aQh[mm] = zero4();
        aKh[mm] = zero4();
        aKc[mm] = zero4();
    }

    // ---- dVn = P^T dO + Kc diag(gamma) dS';  dKbar = Vn dS'^T -> dKc, dgamma ----
    {
        f32x4 adv[XPW];
#pragma unroll
        for (int mm = 0; mm < XPW; ++mm) {
            int ti, tj;
            xtile(mm, ti, tj);
            f32x4 acc = zero4();
#pragma unroll
            for (int k0 = 0; k0 < kBC; k0 += 4)
                acc = mma4(sm.p[(k0 + g) * kLC + 16 * ti + r], sm.dout[(k0 + g) * LV + 16 * tj + r], acc);
            adv[mm] = acc;
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            sD[kb].put(sm.sblk, LV);
            __syncthreads();
            if constexpr (kBf) {
                BF2 ka[2], sc[NTJ];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    // Kc diag(gamma): row 16 i + r over channels 32 kb + ..
                    const float* kr = sm.kc + (16 * i + r) * LK + 32 * kb + 4 * g;
                    const float* gr = sm.gam + 32 * kb + 4 * g;
                    const float4 k0 = *reinterpret_cast<const float4*>(kr), k1 = *reinterpret_cast<const float4*>(kr + 16);
                    const float4 g0 = *reinterpret_cast<const float4*>(gr), g1 = *reinterpret_cast<const float4*>(gr + 16);
                    const float f[8] = {k0.x * g0.x, k0.y * g0.y, k0.z * g0.z, k0.w * g0.w,
                                        k1.x * g1.x, k1.y * g1.y, k1.z * g1.z, k1.w * g1.w};
                    ka[i] = bf_split(f);
                }
#pragma unroll
                for (int i = 0; i < NTJ; ++i) sc[i] = bf_col(sm.sblk, LV, 16 * (wave + 4 * i) + r, g);
                ready(ka[0], ka[1]);
#pragma unroll
                for (int i = 0; i < NTJ; ++i) ready(sc[i]);
#pragma unroll
                for (int mm = 0; mm < XPW; ++mm) adv[mm] = mm3(ka[mm / NTJ], sc[mm % NTJ], adv[mm]);
            } else {
#pragma unroll
                for (int mm = 0; mm < XPW; ++mm) {
                    int ti, tj;
                    xtile(mm, ti, tj);
#pragma unroll
                    for (int k0 = 0; k0 < 32; k0 += 4) {
                        const int cc = 32 * kb + k0 + g;
                        adv[mm] = mma4(sm.kc[(16 * ti + r) * LK + cc] * sm.gam[cc], sm.sblk[(k0 + g) * LV + 16 * tj + r],
                                       adv[mm]);
                    }
                }
            }
            int ti, tj;
            block_tile(kb, ti, tj);
            f32x4 acc = zero4();
            if constexpr (kBf) {
                acc = rowdot<DV, false>(sm.vn, 16 * ti + r, sm.sblk, 16 * (tj - 2 * kb) + r, LV, g, acc);
            } else {
#pragma unroll 8
                for (int j0 = 0; j0 < DV; j0 += 4)
                    acc = mma4(sm.vn[(16 * ti + r) * LV + j0 + g], sm.sblk[(16 * (tj - 2 * kb) + r) * LV + j0 + g], acc);
            }
            const int cc = 16 * tj + r;
            const float gm = sm.gam[cc];
            float part = 0.f;
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) part += acc[v4] * sm.kc[(16 * ti + 4 * g + v4) * LK + cc];
            part += __shfl_xor(part, 16);       // the tile's 16 rows, held by lanes r + 16 g'
            part += __shfl_xor(part, 32);
            if (g == 0) sm.dgam_p[ti][cc] = part;
            if (ti == 0) {
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) aKc[kb >> 1][v4] += acc[v4] * gm;
            } else {
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) aKc[J4 + (kb >> 1)][v4] += acc[v4] * gm;
            }
            __syncthreads();
        }
#pragma unroll
        for (int mm = 0; mm < XPW; ++mm) {
            int ti, tj;
            xtile(mm, ti, tj);
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) sm.dvn[(16 * ti + 4 * g + v4) * LV + 16 * tj + r] = adv[mm][v4];
        }
    }
    __syncthreads();

    // ---- dP = LowerIncl(dO Vn^T);  Z = T^T dVn, dX = diag(b) Z, db += rowsum(Z X) ----
    f32x4 adx[XPW];
    {
        const int ti = wave >> 1, tj = wave & 1;
        f32x4 acc = zero4();
        if constexpr (kBf) {
            acc = rowdot<DV, true>(sm.dout, 16 * ti + r, sm.vn, 16 * tj + r, LV, g, acc);
        } else {
#pragma unroll 8
            for (int j0 = 0; j0 < DV; j0 += 4)
                acc = mma4(sm.dout[(16 * ti + r) * LV + j0 + g], sm.vn[(16 * tj + r) * LV + j0 + g], acc);
        }
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const int i = 16 * ti + 4 * g + v4, j = 16 * tj + r;
            sm.dp[i * kLC + j] = i >= j ? acc[v4] : 0.f;
        }
    }
    float dbw[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};   // this wave's db, rows 16 ti + 4 g + v4
#pragma unroll
    for (int mm = 0; mm < XPW; ++mm) {
        int ti, tj;
        xtile(mm, ti, tj);
        f32x4 acc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < kBC; k0 += 4)
            acc = mma4(sm.t[(k0 + g) * kLC + 16 * ti + r], sm.dvn[(k0 + g) * LV + 16 * tj + r], acc);
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const int row = 16 * ti + 4 * g + v4;
            float part = acc[v4] * sm.x[row * LV + 16 * tj + r];
#pragma unroll
            for (int sh = 1; sh < 16; sh <<= 1) part += __shfl_xor(part, sh);
            dbw[4 * mm / NVT][v4] += part;     // = ti (the waves' tiles never straddle a row tile)
            adx[mm][v4] = sm.beta[row] * acc[v4];
        }
    }
    if (r == 0) {
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4) sm.dbeta_p[wave][16 * ti + 4 * g + v4] = dbw[ti][v4];
    }
    __syncthreads();
    // ---- dX over Vn (dead); dT = dVn X^T diag(b) ----
#pragma unroll
    for (int mm = 0; mm < XPW; ++mm) {
        int ti, tj;
        xtile(mm, ti, tj);
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) sm.vn[(16 * ti + 4 * g + v4) * LV + 16 * tj + r] = adx[mm][v4];
    }
    {
        const int ti = wave >> 1, tj = wave & 1;
        f32x4 acc = zero4();
        if constexpr (kBf) {
            acc = rowdot<DV, false>(sm.dvn, 16 * ti + r, sm.x, 16 * tj + r, LV, g, acc);
        } else {
#pragma unroll 8
            for (int j0 = 0; j0 < DV; j0 += 4)
                acc = mma4(sm.dvn[(16 * ti + r) * LV + j0 + g], sm.x[(16 * tj + r) * LV + j0 + g], acc);
        }
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const int i = 16 * ti + 4 * g + v4, s = 16 * tj + r;
            sm.dt[i * kLC + s] = acc[v4] * sm.beta[s];
        }
    }
    __syncthreads();
    // ---- R = dT T^T (over P, dead) ----
    {
        const int ti = wave >> 1, tj = wave & 1;
        f32x4 acc = zero4();
#pragma unroll
        for (int u0 = 0; u0 < kBC; u0 += 4)
            acc = mma4(sm.dt[(16 * ti + r) * kLC + u0 + g], sm.t[(16 * tj + r) * kLC + u0 + g], acc);
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) sm.p[(16 * ti + 4 * g + v4) * kLC + 16 * tj + r] = acc[v4];
    }
    __syncthreads();
    // ---- dA = StrictLower(-T^T R), dM = diag(b) dA (over dT), db += rowsum(dA M) ----
    {
        const int ti = wave >> 1, tj = wave & 1;
        f32x4 acc = zero4();
#pragma unroll
        for (int u0 = 0; u0 < kBC; u0 += 4)
            acc = mma4(sm.t[(u0 + g) * kLC + 16 * ti + r], sm.p[(u0 + g) * kLC + 16 * tj + r], acc);
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const int i = 16 * ti + 4 * g + v4, s = 16 * tj + r;
            const float da = i > s ? -acc[v4] : 0.f;
            sm.dt[i * kLC + s] = sm.beta[i] * da;
            float part = da * sm.m[i * kLC + s];
#pragma unroll
            for (int sh = 1; sh < 16; sh <<= 1) part += __shfl_xor(part, sh);
            if (r == 0) sm.dbeta_p[wave][i] += part;
        }
    }
    __syncthreads();

    // rows of log a (and of q, k) for the last phase, loaded now
    RowPieces<E, DK> pl, pq, pk;
    pl.load(la, t0, nrow, H, h, 0, DK);
    if constexpr (NORM) {
        pq.load(q, t0, nrow, H, h, 0, DK);
        pk.load(k, t0, nrow, H, h, 0, DK);
    }

    // ---- chunk-internal parts: dQh += dP Kc, dKh += dM Kc, dKc += dP^T Qh + dM^T Kh ----
#pragma unroll
    for (int mm = 0; mm < KPW; ++mm) {
        const int ti = mm / J4, tj = ((wave - 2 * ti) & 3) + 4 * (mm % J4);
#pragma unroll
        for (int u0 = 0; u0 < kBC; u0 += 4) {
            const int s = u0 + g;
            const float kcv = sm.kc[s * LK + 16 * tj + r];
            aQh[mm] = mma4(sm.dp[(16 * ti + r) * kLC + s], kcv, aQh[mm]);
            aKh[mm] = mma4(sm.dt[(16 * ti + r) * kLC + s], kcv, aKh[mm]);
            aKc[mm] = mma4(sm.dp[s * kLC + 16 * ti + r], sm.qh[s * LK + 16 * tj + r], aKc[mm]);
            aKc[mm] = mma4(sm.dt[s * kLC + 16 * ti + r], sm.kh[s * LK + 16 * tj + r], aKc[mm]);
        }
    }
    // ---- state parts: dQh += dO S^T, dKh -= dX S^T;  dgamma += rowsum(dS' S) ----
    {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            sS[kb].put(sm.sblk, LV);
            // dgamma: this thread's pieces of rows of S and dS' (the same positions)
#pragma unroll
            for (int j = 0; j < StateBlock<DV>::NP; ++j) {
                const f32x4 a = sS[kb].v[j], b = sD[kb].v[j];
                float part = a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
#pragma unroll
                for (int sh = 1; sh < StateBlock<DV>::PR; sh <<= 1) part += __shfl_xor(part, sh);
                const int pc = tid + j * kBT;
                if (pc % StateBlock<DV>::PR == 0) sm.dgam_p[2][32 * kb + pc / StateBlock<DV>::PR] = part;
            }
            __syncthreads();
            int ti, tj;
            block_tile(kb, ti, tj);
            f32x4 aq = zero4(), ak = zero4();
            if constexpr (kBf) {
#pragma unroll
                for (int j0 = 0; j0 < DV; j0 += 32) {
                    BF2 sv = bf_row(sm.sblk, LV, 16 * (tj - 2 * kb) + r, j0, g);
                    BF xo = bf_row1(sm.dout, LV, 16 * ti + r, j0, g);
                    BF2 xx = bf_row(sm.vn, LV, 16 * ti + r, j0, g);
                    ready(sv, xx);
                    mfma_ready(xo.u);
                    aq = mmab(xo, sv.h, mmab(xo, sv.l, aq));
                    ak = mm3(xx, sv, ak);
                }
            } else {
#pragma unroll 8
                for (int j0 = 0; j0 < DV; j0 += 4) {
                    const float sv = sm.sblk[(16 * (tj - 2 * kb) + r) * LV + j0 + g];
                    aq = mma4(sm.dout[(16 * ti + r) * LV + j0 + g], sv, aq);
                    ak = mma4(sm.vn[(16 * ti + r) * LV + j0 + g], sv, ak);
                }
            }
            if (ti == 0) {
                aQh[kb >> 1] += aq;
                aKh[kb >> 1] -= ak;
            } else {
                aQh[J4 + (kb >> 1)] += aq;
                aKh[J4 + (kb >> 1)] -= ak;
            }
            __syncthreads();
        }
    }
    // ---- dv = dX, db (the waves' parts in a fixed order); dgamma likewise ----
    store_rows<E, DV>(dv, sm.vn, LV, t0, nrow, H, h);
    if (tid < nrow)
        stf(dbeta + (t0 + tid) * H + h, ((sm.dbeta_p[0][tid] + sm.dbeta_p[1][tid]) + sm.dbeta_p[2][tid]) + sm.dbeta_p[3][tid]);
    if (tid < DK) sm.dgam[tid] = (sm.dgam_p[0][tid] + sm.dgam_p[1][tid]) + sm.dgam_p[2][tid];
    __syncthreads();

    // ---- through the decays: G again (flat area 0), then dQ, dK, dG ----
    float* F0 = sm.x;                       // log a, G, then dQ
    float* F1 = sm.x + kBC * LK;            // dK
    float* F2 = sm.x + 2 * kBC * LK;        // dG, then dlog a
    pl.put(F0, LK, nrow);
    __syncthreads();
    {
        f32x4 G[2][NCT / 4];
        tri_cumsum<NCT, false>(F0, LK, kBC, wave, r, g, G);
#pragma unroll
        for (int u = 0; u < NCT / 4; ++u)
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    F0[(16 * ti + 4 * g + v) * LK + 16 * (wave * (NCT / 4) + u) + r] = G[ti][u][v];
    }
    __syncthreads();
#pragma unroll
    for (int mm = 0; mm < KPW; ++mm) {
        const int ti = mm / J4, tj = ((wave - 2 * ti) & 3) + 4 * (mm % J4);
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
            const int row = 16 * ti + 4 * g + v4, cc = 16 * tj + r, o = row * LK + cc;
            const float G = F0[o], G2 = G * kLog2e, ex = fast_exp2(G2), ei = fast_exp2(-G2);
            const float a = aQh[mm][v4], b = aKh[mm][v4], e = aKc[mm][v4];
            F0[o] = a * ex;
            F1[o] = b * ex + e * ei;
            F2[o] = a * sm.qh[o] + b * sm.kh[o] - e * sm.kc[o];
        }
    }
    __syncthreads();
    // dlog a: reverse cumsum of dG over the valid rows, dgamma gamma entering at the last one
    {
        f32x4 R[2][NCT / 4];
        tri_cumsum<NCT, true>(F2, LK, nrow, wave, r, g, R);
#pragma unroll
        for (int u = 0; u < NCT / 4; ++u) {
            const int c = 16 * (wave * (NCT / 4) + u) + r;
            const float dg = sm.dgam[c] * sm.gam[c];
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int row = 16 * ti + 4 * g + v;
                    F2[row * LK + c] = row < nrow ? R[ti][u][v] + dg : 0.f;
                }
        }
    }
    if constexpr (NORM) {
        // dx = (dx^ - x^ (x^ . dx^)) / |x| for x^ = x / |x|, x = q, k of the row; the row's
        // pieces sit in consecutive threads
        using RP = RowPieces<E, DK>;
#pragma unroll
        for (int j = 0; j < RP::NP; ++j) {
            const int pc = tid + j * kBT, row = min(pc / RP::PPR, kBC - 1), c0 = (pc % RP::PPR) * RP::EPP;
            float xq[RP::EPP], xk[RP::EPP];
            put16<E>(xq, pq.v[j], true);
            put16<E>(xk, pk.v[j], true);
            float dotq = 0.f, dotk = 0.f;
#pragma unroll
            for (int e = 0; e < RP::EPP; ++e) {
                xq[e] *= sm.qinv[row];
                xk[e] *= sm.kinv[row];
                dotq += xq[e] * F0[row * LK + c0 + e];
                dotk += xk[e] * F1[row * LK + c0 + e];
            }
#pragma unroll
            for (int sh = 1; sh < RP::PPR; sh <<= 1) {
                dotq += __shfl_xor(dotq, sh);
                dotk += __shfl_xor(dotk, sh);
            }
            if (pc < kBC * RP::PPR) {
#pragma unroll
                for (int e = 0; e < RP::EPP; ++e) {
                    F0[row * LK + c0 + e] = (F0[row * LK + c0 + e] - xq[e] * dotq) * sm.qinv[row];
                    F1[row * LK + c0 + e] = (F1[row * LK + c0 + e] - xk[e] * dotk) * sm.kinv[row];
                }
            }
        }
    }
    __syncthreads();
    store_rows<E, DK>(dq, F0, LK, t0, nrow, H, h);
    store_rows<E, DK>(dk, F1, LK, t0, nrow, H, h);
    store_rows<E, DK>(dla, F2, LK, t0, nrow, H, h);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct BwdPlan {
    int max_chunks;
    int lseg;          // chunks per segment of the chains' sequence split; 0 = no split
    int max_segs;
    size_t table_bytes, rec_bytes, state_bytes, seg_bytes, phi_bytes;
};

// Sequence split: when the pack gives at most 64 chain workgroups (a quarter of the CUs
// or less), each sample is cut into segments of lseg chunks (at least 64, i.e. 2,048
// tokens) so that about 256 workgroups run the second passes.
BwdPlan bwd_plan(int64_t total_tokens, int32_t num_seqs, int32_t num_heads, int d_k, int d_v)
{
    BwdPlan p{};
    const int64_t chunks_bound = (total_tokens + kBC - 1) / kBC;
    p.max_chunks = int(chunks_bound + num_seqs);
    p.lseg = 0;
    const int64_t units = int64_t(num_seqs) * num_heads * (d_v / 64);
    if (units <= 64) {
        const int64_t segs = std::max<int64_t>(1, 256 / (int64_t(num_heads) * (d_v / 64)));
        const int64_t lseg = std::max<int64_t>(64, (chunks_bound + segs - 1) / segs);
        if (lseg < chunks_bound) p.lseg = int(lseg);
    }
    // every sample has at most ceil(chunks / lseg) <= chunks / lseg + 1 segments, and the
    // chunks of all samples number at most chunks_bound + num_seqs
    p.max_segs = p.lseg ? int((chunks_bound + num_seqs + p.lseg - 1) / p.lseg + num_seqs) : 0;
    p.table_bytes = ((3 * size_t(num_seqs) + 2) * sizeof(int32_t) + 255) & ~size_t(255);
    const size_t rec = d_k == 128 ? BRec<128>::TOTAL : BRec<64>::TOTAL;
    p.rec_bytes = size_t(p.max_chunks) * num_heads * rec * sizeof(float);
    p.state_bytes = size_t(p.max_chunks) * num_heads * d_k * d_v * sizeof(float);
    p.seg_bytes = size_t(p.max_segs) * num_heads * d_k * d_v * sizeof(float);
    p.phi_bytes = size_t(p.max_segs) * num_heads * d_k * d_k * sizeof(float);
    return p;
}

template <typename K> hipError_t set_smem(K kern, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                               int(bytes));
}

template <typename E, int DK, int DV, bool NORM>
hipError_t launch_bwd_t(const BwdArgs& a, void* workspace, TimingHook* th)
{
    const BwdPlan p = bwd_plan(a.total_tokens, a.num_seqs, a.num_heads, DK, DV);
    char* base = static_cast<char*>(workspace);
    int32_t* chunk_off = reinterpret_cast<int32_t*>(base);
    int32_t* seg_off = chunk_off + (a.num_seqs + 1);
    int32_t* order = seg_off + (a.num_seqs + 1);
    char* next = base + p.table_bytes;
    float* rec = reinterpret_cast<float*>(next);
    next += p.rec_bytes;
    float* s_in = reinterpret_cast<float*>(next);
    next += p.state_bytes;
    float* ds_out = reinterpret_cast<float*>(next);
    next += p.state_bytes;
    float* sloc = p.lseg ? reinterpret_cast<float*>(next) : nullptr;
    next += p.seg_bytes;
    float* eseg = p.lseg ? reinterpret_cast<float*>(next) : nullptr;
    next += p.seg_bytes;
    float* phi = p.lseg ? reinterpret_cast<float*>(next) : nullptr;
    next += p.phi_bytes;
    float* phi_t = p.lseg ? reinterpret_cast<float*>(next) : nullptr;
    const E* q = static_cast<const E*>(a.q);
    const E* k = static_cast<const E*>(a.k);
    const E* v = static_cast<const E*>(a.v);
    const E* la = static_cast<const E*>(a.log_alpha);
    const E* beta = static_cast<const E*>(a.beta);
    const E* dout = static_cast<const E*>(a.d_out);
    const int H = a.num_heads;
    hipError_t e;

    if (th) th->begin("bwd_plan", a.stream);
    hipLaunchKernelGGL(kda_bwd_plan_kernel, dim3(1), dim3(1024), 0, a.stream, a.cu_seqlens, chunk_off,
                       p.lseg ? seg_off : nullptr, order, a.num_seqs, a.total_tokens, p.lseg);
    if (th) th->end(a.stream);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    const size_t prep_smem = sizeof(PrepLds<DK>);
    auto prep = kda_bwd_prep_kernel<E, DK, NORM>;
    if ((e = set_smem(prep, prep_smem)) != hipSuccess) return e;
    if (th) th->begin("bwd_prep", a.stream);
    hipLaunchKernelGGL(prep, dim3(p.max_chunks, H), dim3(kBT), prep_smem, a.stream, q, k, la, beta, a.cu_seqlens,
                       chunk_off, rec, a.num_seqs, H, a.total_tokens, p.max_chunks);
    if (th) th->end(a.stream);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    // chain grids: units of (sample or segment, head), padded to 8, times the column tiles
    const int units = p.lseg ? p.max_segs * H : a.num_seqs * H;
    const int ublocks = ((units + 7) / 8) * 8;
    const size_t chain_smem = sizeof(ChainLds<DK>);
    auto launch_state = [&](auto kern, int ntiles, const char* name, hipStream_t st) -> hipError_t {
        hipError_t err = set_smem(kern, chain_smem);
        if (err != hipSuccess) return err;
        if (th) th->begin(name, st);
        hipLaunchKernelGGL(kern, dim3(ublocks * ntiles), dim3(kBT), chain_smem, st, v, a.cu_seqlens, chunk_off,
                           seg_off, order, rec, a.init_state, s_in, sloc, phi, phi_t, a.num_seqs, H, a.total_tokens,
                           p.max_chunks, p.lseg, p.max_segs);
        if (th) th->end(st);
        return hipGetLastError();
    };
    auto launch_dstate = [&](auto kern, const char* name, hipStream_t st) -> hipError_t {
        hipError_t err = set_smem(kern, chain_smem);
        if (err != hipSuccess) return err;
        if (th) th->begin(name, st);
        hipLaunchKernelGGL(kern, dim3(ublocks * (DV / 64)), dim3(kBT), chain_smem, st, dout, a.cu_seqlens,
                           chunk_off, seg_off, order, rec, a.d_final_state, ds_out, a.d_init_state, phi_t, eseg, a.num_seqs, H,
                           a.total_tokens, p.max_chunks, p.lseg, p.max_segs);
        if (th) th->end(st);
        return hipGetLastError();
    };
    // Without the sequence split the two chains are independent (the state-gradient chain
    // reads the records and dO, never S). Fork: the state chain on an auxiliary stream once
    // the prep is done; the state-gradient chain, the longer of the two, goes first on the
    // caller's stream so that it takes the CUs first, and the state chain gets the CUs its
    // shorter samples free. With the split, the state-gradient chain's second pass reads the
    // transposed segment transitions that the state chain's first pass writes: that pass is
    // launched first, and the caller's stream waits for it before the second pass.
    AuxStream* ss = nullptr;
    if ((e = aux_stream(0, ss)) != hipSuccess) return e;
    if ((e = aux_fork(a.stream, ss)) != hipSuccess) return e;
    // from here on every path joins the auxiliary stream back, so that nothing enqueued on
    // it outlives the call's stream order (the workspace is freed on the caller's stream);
    // the first error is kept
    auto chains = [&]() -> hipError_t {
        hipError_t err;
        if (p.lseg == 0) {
            if ((err = launch_dstate(kda_bwd_dstate_kernel<E, DK, DV, 0>, "bwd_dstate", a.stream)) != hipSuccess)
                return err;
            return launch_state(kda_bwd_state_kernel<E, DK, DV, 0>, DV / 64, "bwd_state", ss->stream);
        }
        if ((err = launch_state(kda_bwd_state_kernel<E, DK, DV, 1>, DV / 64 + DK / 64, "bwd_state_seg",
                                ss->stream)) != hipSuccess)
            return err;
        if ((err = launch_dstate(kda_bwd_dstate_kernel<E, DK, DV, 1>, "bwd_dstate_seg", a.stream)) != hipSuccess)
            return err;
        // Phi^T (phi_t) is complete once the state chain's first pass is
        if ((err = aux_join(a.stream, ss)) != hipSuccess) return err;
        if ((err = launch_dstate(kda_bwd_dstate_kernel<E, DK, DV, 2>, "bwd_dstate", a.stream)) != hipSuccess)
            return err;
        return launch_state(kda_bwd_state_kernel<E, DK, DV, 2>, DV / 64, "bwd_state", ss->stream);
    };
    e = chains();
    // join: the gradient kernel needs both chains
    const hipError_t ej = aux_join(a.stream, ss);
    if (e == hipSuccess) e = ej;
    if (e != hipSuccess) return e;

    const size_t grad_smem = sizeof(GradLds<DK, DV>);
    auto grad = kda_bwd_grad_kernel<E, DK, DV, NORM>;
    if ((e = set_smem(grad, grad_smem)) != hipSuccess) return e;
    if (th) th->begin("bwd_grad", a.stream);
    hipLaunchKernelGGL(grad, dim3(p.max_chunks, H), dim3(kBT), grad_smem, a.stream, q, k, v, la, beta, dout,
                       a.cu_seqlens, chunk_off, rec, s_in, ds_out, static_cast<E*>(a.dq), static_cast<E*>(a.dk),
                       static_cast<E*>(a.dv), static_cast<E*>(a.dlog_alpha), static_cast<E*>(a.dbeta), a.num_seqs,
                       H, a.total_tokens, p.max_chunks);
    if (th) th->end(a.stream);
    return hipGetLastError();
}

template <typename E, bool NORM>
hipError_t launch_bwd_n(const BwdArgs& a, void* ws, TimingHook* th)
{
    if (a.d_k == 128 && a.d_v == 128) return launch_bwd_t<E, 128, 128, NORM>(a, ws, th);
    if (a.d_k == 128 && a.d_v == 64) return launch_bwd_t<E, 128, 64, NORM>(a, ws, th);
    if (a.d_k == 64 && a.d_v == 128) return launch_bwd_t<E, 64, 128, NORM>(a, ws, th);
    return launch_bwd_t<E, 64, 64, NORM>(a, ws, th);
}

}  // namespace

size_t bwd_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_heads, int d_k, int d_v)
{
    const BwdPlan p = bwd_plan(total_tokens, num_seqs, num_heads, d_k, d_v);
    return p.table_bytes + p.rec_bytes + 2 * p.state_bytes + 2 * p.seg_bytes + 2 * p.phi_bytes;
}

hipError_t launch_backward(const BwdArgs& a, void* workspace, TimingHook* th)
{
    const BwdPlan p = bwd_plan(a.total_tokens, a.num_seqs, a.num_heads, a.d_k, a.d_v);
    if (int64_t(p.max_chunks) * a.num_heads > 0x7FFFFFFF / 64) return hipErrorInvalidValue;
    if (a.dtype_bf16)
        return a.qk_l2norm ? launch_bwd_n<uint16_t, true>(a, workspace, th) : launch_bwd_n<uint16_t, false>(a, workspace, th);
    return a.qk_l2norm ? launch_bwd_n<float, true>(a, workspace, th) : launch_bwd_n<float, false>(a, workspace, th);
}

}  // namespace kda
