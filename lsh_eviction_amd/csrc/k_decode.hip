// k_decode.hip -- the decode step of the HashEvict path on gfx950.
//
// Method: HashEvict summary page ("HashEvict: A Pre-Attention KV Cache
// Eviction Strategy using Locality-Sensitive Hashing", arXiv 2412.16187),
// "Technical framework" stages 1-5 and the abstract: encode the query, score
// every cached key code by Hamming distance, evict the farthest slot before
// any attention is computed, write the new token there, attend.
//
// Two schedules of the same step:
//
//   FUSED (one launch).  Every block owns a chunk of slots of one (sequence,
//   KV head).  It encodes the group's queries and the new key on the matrix
//   cores, finds its chunk's candidate (highest GQA score, lowest slot on
//   ties), folds it into the head's eviction key with a 64-bit atomic max,
//   and accumulates softmax partials over its chunk with that candidate held
//   out.  It then publishes its partial with write-through stores and takes a
//   ticket; the head's last block reads the winner from the eviction key
//   (the global argmax with lowest-index ties is always its own chunk's
//   candidate), adds back the held-out candidates of the other chunks and the
//   new token, merges the partials against one common maximum per head
//   (a running log-sum-exp when there are very many) and writes the new token into the
//   winner's slot.  The result equals "evict, write, then attend" with every
//   K/V byte read once and no grid-wide barrier or L2-wide fence.  The other
//   blocks run the same merge dry (empty record buffers, no stores), which
//   keeps its code in every compute unit's instruction cache.
//
//   SPLIT (five launches): lsh_encode, hamming_argmax, evict_write, split-K
//   attention, LSE merge.
//
// The step at token position t folds its candidates into ekey[t & 1]; the
// reader of that key (the head's last block, or evict_write) clears it, so
// the next step starts from a cleared key without a launch of its own.
#include <type_traits>

#include "hkv_consts.h"
#include "hkv_device.h"

namespace hkv {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
// Cache policy sc1 of a buffer load or store = the agent-scope policy (see
// the fused schedule).
constexpr int kCpolSC1 = 16;
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D>
__device__ __forceinline__ float qscale2()
{
    // base-2 softmax: logits (q.k / sqrt(d)) * log2(e)
    return kLog2e * (D == 64 ? 0.125f : 0.08838834764831845f);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }


// ---------------------------------------------------------------------------
// stages 1-2 on the matrix cores
// ---------------------------------------------------------------------------

// The calling wave computes bit columns [16 nt, 16 nt + 16) of the codes of
// rows v < nvec <= 16 of X (row stride D): Y = X R on a 16x16x4 fp32 MFMA
// (lane l feeds row l % 16 and the quarter l / 16 of the head dimension), one
// ballot of (y > 0) per accumulator register.  Lane i < nvec returns the
// 16-bit chunk of row i.
// Operands of one wave's share of the encoder (see encode16_mfma).
template <int D>
struct EncOps {
    float x[D / 4];    // the lane's quarter of its row of X
    float rv[D / 4];   // the matching entries of R's column
};

template <int D, int BITS, typename XT>
__device__ __forceinline__ void enc_load_x(EncOps<D>& op, const XT* __restrict__ X, int nvec)
{
    constexpr int DQ = D / 4;
    constexpr int EPL = Vec16<XT>::EPL;
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, qd = lane >> 4;
    const XT* src = X + (size_t)(m < nvec ? m : 0) * D + qd * DQ;
#pragma unroll
    for (int v = 0; v < DQ / EPL; ++v) {
        const uint4 raw = *reinterpret_cast<const uint4*>(src + v * EPL);
        float f[EPL];
        Vec16<XT>::cvt(raw, f);
#pragma unroll
        for (int e = 0; e < EPL; ++e) op.x[v * EPL + e] = m < nvec ? f[e] : 0.f;
    }
}

template <int D, int BITS>
__device__ __forceinline__ void enc_load_r(EncOps<D>& op, const float* __restrict__ R, int nt)
{
    constexpr int DQ = D / 4;
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, qd = lane >> 4;
    const float* rc = R + (size_t)(qd * DQ) * BITS + nt * 16 + m;
#pragma unroll
    for (int s = 0; s < DQ; ++s) op.rv[s] = rc[s * BITS];
}

// The calling wave computes bit columns [16 nt, 16 nt + 16) of the codes of
// up to 16 rows: Y = X R on a 16x16x4 fp32 MFMA (lane l feeds row l % 16 and
// the quarter l / 16 of the head dimension), one ballot of (y > 0) per
// accumulator register.  Lane i returns the 16-bit chunk of row i.
template <int D>
__device__ __forceinline__ uint32_t enc_compute(const EncOps<D>& op)
{
    constexpr int DQ = D / 4;
    const int lane = threadIdx.x & 63;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < DQ; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(op.x[s], op.rv[s], acc, 0, 0, 0);
    unsigned long long mk[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) mk[r] = __ballot(acc[r] > 0.f);
    // result row i = 4 a + r sits in register r of lanes 16 a + column
    const int a = (lane & 15) >> 2, r = lane & 3;
    const unsigned long long mm = r == 0 ? mk[0] : r == 1 ? mk[1] : r == 2 ? mk[2] : mk[3];
    return (uint32_t)((mm >> (16 * a)) & 0xFFFFull);
}

template <int D, int BITS, typename XT>
__device__ __forceinline__ uint32_t encode16_mfma(const XT* __restrict__ X, int nvec, const float* __restrict__ R,
                                                  int nt)
{
    EncOps<D> op;
    enc_load_x<D, BITS, XT>(op, X, nvec);
    enc_load_r<D, BITS>(op, R, nt);
    return enc_compute<D>(op);
}

// Codes of rows [0, nvec <= 16) of X into out16[nt][row] (LDS), waves 0 .. NT-1.
template <int D, int BITS, typename XT>
__device__ __forceinline__ void encode_block16(const XT* __restrict__ X, int nvec, const float* __restrict__ R,
                                               uint32_t (*out16)[16])
{
    constexpr int NT = BITS / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int nt = wave; nt < NT; nt += kWaves) {
        const uint32_t c16 = encode16_mfma<D, BITS, XT>(X, nvec, R, nt);
        if (lane < nvec) out16[nt][lane] = c16;
    }
}

// Wave-level encoder over operands staged in LDS: rows 0 .. nq-1 of X are
// the fp32 rows of Xq (row stride XS), row nq is the vector xk (stored as
// KT), rows above are zero; Rt is R transposed, b rows of d entries with row
// stride D + 4.  Lane i returns the 16-bit chunk nt of the code of row i (as
// encode16_mfma).  Lane (m, qd) = (l % 16, l / 16) feeds row m of X and
// column 16 nt + m of R over k = qd d/4 + s at product s; it reads both
// operands as 16-byte runs, and the row padding puts the 16 lanes of a
// quarter-wave on distinct banks.
template <int D, int BITS, typename KT, int XS>
__device__ __forceinline__ uint32_t enc_lds(const float* Xq, int nq, const KT* xk, const float* Rt, int nt)
{
    constexpr int DQ = D / 4;
    constexpr int EPL = Vec16<KT>::EPL;
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, qd = lane >> 4;
    const float* xr = Xq + (size_t)(m < nq ? m : 0) * XS + qd * DQ;
    const KT* kr = xk + qd * DQ;
    const float* rr = Rt + (size_t)(nt * 16 + m) * (D + 4) + qd * DQ;
    // Every operand is read from LDS before the first product, so the reads
    // overlap; a product that waits for its own read would make the encoder
    // a chain of LDS round trips.
    float xs[DQ], rs[DQ];
#pragma unroll
    for (int v = 0; v < DQ / EPL; ++v) {
        float kf[EPL];
        Vec16<KT>::cvt(*reinterpret_cast<const uint4*>(kr + v * EPL), kf);
#pragma unroll
        for (int e4 = 0; e4 < EPL / 4; ++e4) {
            const float4 q4 = *reinterpret_cast<const float4*>(xr + v * EPL + 4 * e4);
            const float qv[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                xs[v * EPL + 4 * e4 + e] = m < nq ? qv[e] : (m == nq ? kf[4 * e4 + e] : 0.f);
        }
    }
#pragma unroll
    for (int v = 0; v < DQ / 4; ++v) {
        const float4 r4 = *reinterpret_cast<const float4*>(rr + 4 * v);
        rs[4 * v] = r4.x;
        rs[4 * v + 1] = r4.y;
        rs[4 * v + 2] = r4.z;
        rs[4 * v + 3] = r4.w;
    }
    __builtin_amdgcn_sched_barrier(0);
    // four independent accumulation chains, added at the end (any fp32
    // summation order gives the exact sign outside the flagged band)
    f32x4 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < DQ; ++s) acc[s & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(xs[s], rs[s], acc[s & 3], 0, 0, 0);
    unsigned long long mk[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) mk[r] = __ballot((acc[0][r] + acc[1][r]) + (acc[2][r] + acc[3][r]) > 0.f);
    const int a = (lane & 15) >> 2, r = lane & 3;
    const unsigned long long mm = r == 0 ? mk[0] : r == 1 ? mk[1] : r == 2 ? mk[2] : mk[3];
    return (uint32_t)((mm >> (16 * a)) & 0xFFFFull);
}

template <int BITS>
__device__ __forceinline__ unsigned long long join16(const uint32_t (*c16)[16], int row)
{
    unsigned long long v = 0;
#pragma unroll
    for (int nt = 0; nt < BITS / 16; ++nt) v |= (unsigned long long)c16[nt][row] << (16 * nt);
    return v;
}

// ---------------------------------------------------------------------------
// Hamming candidate of a slot range
// ---------------------------------------------------------------------------
// Best (score, lowest slot) key of the thread's codes in [s0, s1): group j
// is the 16 bytes at slot s0 + (j * kThreads + tid) * VS.  The first NPRE
// groups were loaded by the caller before the tile ring (pre); later groups
// (chunks longer than NPRE * kThreads * VS slots) are loaded here, and a wait
// for one of those is a wait for every tile issued before it.
template <int BITS, int GM, int NPRE>
__device__ __forceinline__ unsigned long long thread_candidate(const typename CodeT<BITS>::T* __restrict__ code,
                                                               const typename CodeT<BITS>::T (&qc)[GM], int G,
                                                               int s0, int s1, const uint4 (&pre)[NPRE])
{
    using CT = typename CodeT<BITS>::T;
    constexpr int VS = 16 / sizeof(CT);
    unsigned long long best = 0;
    auto fold = [&](uint4 raw, int s) {
        CT cs[VS];
        __builtin_memcpy(cs, &raw, 16);
#pragma unroll
        for (int u = 0; u < VS; ++u) {
            int sc = 0;
#pragma unroll
            for (int g = 0; g < GM; ++g)
                if (g < G) sc += popc((CT)(cs[u] ^ qc[g]));
            const unsigned long long k = (s + u < s1) ? cand_key(sc, s + u) : 0ull;
            best = k > best ? k : best;
        }
    };
    // (a wave whose preloaded groups all lie past the range skips them: its
    // first lane holds the lowest slot)
#pragma unroll
    for (int j = 0; j < NPRE; ++j) {
        const int sj = s0 + (j * kThreads + (int)threadIdx.x) * VS;
        if (__builtin_amdgcn_readfirstlane(sj) < s1) fold(pre[j], sj);
    }
    for (int s = s0 + (NPRE * kThreads + (int)threadIdx.x) * VS; s < s1; s += kThreads * VS)
        fold(*reinterpret_cast<const uint4*>(code + s), s);
    return best;
}

__device__ __forceinline__ unsigned long long block_max_u64(unsigned long long v, unsigned long long* red)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_max_u64(v);
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) v = red[w] > v ? red[w] : v;
    return v;
}

// ---------------------------------------------------------------------------
// softmax partial over a slot range (VALU, 16-byte coalesced row loads)
// ---------------------------------------------------------------------------
template <int D, int GM>
struct AttnSmem {
    float m[kWaves][GM];
    float l[kWaves][GM];
    float acc[kWaves][GM][D];
};

template <int D, typename KT>
struct Tile {
    static constexpr int EPL = Vec16<KT>::EPL;   // elements per 16-byte load
    static constexpr int LPR = D / EPL;          // lanes per row
    static constexpr int RPW = 64 / LPR;         // rows per wave load
    static constexpr int UNR = 2;                // wave loads per tile and lane
    static constexpr int ROWS = RPW * UNR;       // rows of a wave's tile
    uint4 k[UNR], v[UNR];

    // tile `base` (row offset within the range of `len` rows, first row r0)
    __device__ __forceinline__ void load(const KT* __restrict__ Kh, const KT* __restrict__ Vh, int r0, int len,
                                         int base)
    {
        const int lane = threadIdx.x & 63;
        const int rg = lane / LPR, cc = lane % LPR;
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int row = base + u * RPW + rg;
            if (row < len) {
                const size_t off = (size_t)(r0 + row) * D + cc * EPL;
                k[u] = *reinterpret_cast<const uint4*>(Kh + off);
                v[u] = *reinterpret_cast<const uint4*>(Vh + off);
            } else {
                k[u] = make_uint4(0, 0, 0, 0);
                v[u] = make_uint4(0, 0, 0, 0);
            }
        }
    }
};

// Softmax partial of the G query heads of one KV head over rows [r0, r0+len)
// of Kh / Vh, leaving out row `skip` (-1: none), whose base-2 logits go to
// sm.candlg.  `first` is the wave's first tile, already in flight.  The next
// tile is loaded while the current one is computed.  On return (after a block
// barrier) sm.m, sm.l, sm.acc hold one (max, sum, acc) per wave.
template <int D, int GM, typename KT, int QS = D>
__device__ __forceinline__ void attend_rows(const KT* __restrict__ Kh, const KT* __restrict__ Vh,
                                            const float* __restrict__ qh, int G, int r0, int len, int skip,
                                            Tile<D, KT> cur, AttnSmem<D, GM>& sm, float* clg)
{
    using T = Tile<D, KT>;
    constexpr int EPL = T::EPL, LPR = T::LPR, RPW = T::RPW, UNR = T::UNR;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rg = lane / LPR, cc = lane % LPR;

    float qr[GM][EPL];
    const float qs = qscale2<D>();
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        if (g < G) {
            const float4* qp = reinterpret_cast<const float4*>(qh + g * QS + cc * EPL);
#pragma unroll
            for (int e4 = 0; e4 < EPL / 4; ++e4) {
                const float4 f = qp[e4];
                qr[g][4 * e4 + 0] = f.x * qs;
                qr[g][4 * e4 + 1] = f.y * qs;
                qr[g][4 * e4 + 2] = f.z * qs;
                qr[g][4 * e4 + 3] = f.w * qs;
            }
        } else {
#pragma unroll
            for (int e = 0; e < EPL; ++e) qr[g][e] = 0.f;
        }
    }

    float m[GM], l[GM], acc[GM][EPL];
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
    }

    for (int base = wave * T::ROWS; base < len; base += kWaves * T::ROWS) {
        T nxt;
        const int nb = base + kWaves * T::ROWS;
        if (nb < len) nxt.load(Kh, Vh, r0, len, nb);
        float lg[UNR][GM];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            float kf[EPL];
            Vec16<KT>::cvt(cur.k[u], kf);
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                float dot = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) dot = fmaf(qr[g][e], kf[e], dot);
                lg[u][g] = group_sum<LPR>(dot);
            }
            const int row = base + u * RPW + rg;
            const bool isc = (r0 + row) == skip;
            if (isc && cc == 0) {   // the held-out row's logits
#pragma unroll
                for (int g = 0; g < GM; ++g) clg[g] = lg[u][g];
            }
            if (row >= len || isc) {
#pragma unroll
                for (int g = 0; g < GM; ++g) lg[u][g] = -INFINITY;
            }
        }
        float p[UNR][GM];
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            float mx = m[g];
#pragma unroll
            for (int u = 0; u < UNR; ++u) mx = fmaxf(mx, lg[u][g]);
            const float ms = mx == -INFINITY ? 0.f : mx;
            const float alpha = exp2_fast(m[g] - ms);
            m[g] = mx;
            float ls = l[g] * alpha;
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                p[u][g] = exp2_fast(lg[u][g] - ms);
                ls += p[u][g];
            }
            l[g] = ls;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[g][e] *= alpha;
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            float vf[EPL];
            Vec16<KT>::cvt(cur.v[u], vf);
#pragma unroll
            for (int g = 0; g < GM; ++g)
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p[u][g], vf[e], acc[g][e]);
        }
        cur = nxt;
    }

    // combine the row groups of the wave
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            const float mo = __shfl_xor(m[g], off);
            const float lo = __shfl_xor(l[g], off);
            const float mx = fmaxf(m[g], mo);
            const float ms = mx == -INFINITY ? 0.f : mx;
            const float a = exp2_fast(m[g] - ms), bb = exp2_fast(mo - ms);
            l[g] = l[g] * a + lo * bb;
            m[g] = mx;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                const float ao = __shfl_xor(acc[g][e], off);
                acc[g][e] = acc[g][e] * a + ao * bb;
            }
        }
    }
    if (rg == 0) {
#pragma unroll
        for (int g = 0; g < GM; ++g) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) sm.acc[wave][g][cc * EPL + e] = acc[g][e];
            if (cc == 0) {
                sm.m[wave][g] = m[g];
                sm.l[wave][g] = l[g];
            }
        }
    }
    __syncthreads();
}

// The block's partial for query heads g < G: part[(hq, split)] = acc[D], m, l.
template <int D, int GM>
__device__ __forceinline__ void store_partial(const AttnSmem<D, GM>& sm, float* __restrict__ part, int hq0, int G,
                                              int nsplit, int split)
{
    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
        const int g = idx / D, i = idx % D;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm.m[w][g]);
        const float ms = mx == -INFINITY ? 0.f : mx;
        float a = 0.f, ls = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float sc = exp2_fast(sm.m[w][g] - ms);
            a += sm.acc[w][g][i] * sc;
            ls += sm.l[w][g] * sc;
        }
        float* rec = part + ((size_t)(hq0 + g) * nsplit + split) * (D + 4);
        rec[i] = a;
        if (i == 0) {
            rec[D] = mx;
            rec[D + 1] = ls;
        }
    }
}

// ---------------------------------------------------------------------------
// softmax partial over a slot range, bf16 K/V: QK^T on the matrix cores
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// One wave's tile of TR rows: K in the A-operand layout of the 16x16x32 bf16
// MFMA (lane l: row l % 16 of each 16-row half, the contiguous quarter
// (l / 16) of the head dimension, 16 bytes per k-step), V in coalesced
// 16-byte row segments (lane l: row group l / (D/8), segment l % (D/8)).
// Rows at or beyond `len` are not loaded and read as zero.
// P.V runs on the matrix cores for d = 128 (see mfma_tile_pv), with values
// as given or quantized; d = 64 accumulates P.V on the VALU.
// VQ: the width of the stored value codes, 0 (values as given), 8 or 4.
template <int D, int VQ>
constexpr bool pv_on_mfma()
{
    return D == 128;
}

template <int D, int TR, int VQ = 0>
struct MTile {
    static constexpr int H = TR / 16;          // 16-row halves
    static constexpr int KS = D / 32;          // k-steps of 32 per half
    static constexpr int LPR = D / 8;          // V lanes per row (8 values each)
    static constexpr int RPW = 64 / LPR;       // V rows per wave load
    static constexpr int VU = TR / RPW;        // V loads per lane
    // 8 bf16 values, 8 int8 codes or 8 4-bit codes
    using VW = typename std::conditional<VQ == 8, uint2, typename std::conditional<VQ == 4, uint32_t, uint4>::type>::type;
    uint4 k[H][KS];
    VW v[VU];
    float vs[VQ ? H : 1][4];   // quantized values: scales of rows 16h + 4(l/16) + r (MFMA layout)

    // Rows beyond the range are clamped to its last row (loaded, then masked by
    // the caller); len == 0 clamps to row 0 of the range, which is in bounds.
    // No load sits in a branch, so the wait counters stay exact and the tile
    // in flight is never waited for early.
    // Vh: bf16 rows, or code rows (VQ bits a code) with their scales at Vsh.
    __device__ __forceinline__ void load(const bf16_t* __restrict__ Kh, const void* __restrict__ Vh,
                                         const float* __restrict__ Vsh, int r0, int len, int base)
    {
        const int lane = threadIdx.x & 63;
        const int i = lane & 15, qd = lane >> 4;
        if constexpr (pv_on_mfma<D, VQ>()) {
            // MFMA row i of the block holds physical row i / 4 + 4 (i % 4) (see
            // mfma_tile_pv).  Buffer loads over the range's len rows: 32-bit
            // offsets, and rows at or beyond len read as zero (the caller masks
            // them).
            static_assert(H == 1, "one 16-row block per tile");
            const int nb = len * D * 2;
            const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(Kh + (size_t)r0 * D), 0, nb, kRsrcWord3);
            const auto rv = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<bf16_t*>(reinterpret_cast<const bf16_t*>(Vh) + (size_t)r0 * D), 0, nb, kRsrcWord3);
            const int ko = (base + (i >> 2) + 4 * (i & 3)) * (D * 2) + qd * (D / 2);
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const auto w = __builtin_amdgcn_raw_buffer_load_b128(rk, ko + 16 * s, 0, 0);
                __builtin_memcpy(&k[0][s], &w, 16);
            }
            const int rg = lane / LPR, cc = lane % LPR;
            if constexpr (VQ == 0) {
#pragma unroll
                for (int u = 0; u < VU; ++u) {
                    const auto w =
                        __builtin_amdgcn_raw_buffer_load_b128(rv, (base + u * RPW + rg) * (D * 2) + cc * 16, 0, 0);
                    __builtin_memcpy(&v[u], &w, 16);
                }
            } else {
                // the same rows and columns as codes (VB bytes a row), then
                // the scales of rows qd + 4 r: the rows of this lane's logits
                constexpr int VB = D * VQ / 8;
                const auto rq = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(Vh) + (size_t)r0 * VB), 0, len * VB,
                    kRsrcWord3);
#pragma unroll
                for (int u = 0; u < VU; ++u) {
                    const int off = (base + u * RPW + rg) * VB + cc * VQ;   // 8 codes of VQ bits
                    if constexpr (VQ == 8) {
                        const auto w = __builtin_amdgcn_raw_buffer_load_b64(rq, off, 0, 0);
                        __builtin_memcpy(&v[u], &w, 8);
                    } else {
                        v[u] = __builtin_amdgcn_raw_buffer_load_b32(rq, off, 0, 0);
                    }
                }
                const int last = len > 0 ? len - 1 : 0;
#pragma unroll
                for (int r = 0; r < 4; ++r) vs[0][r] = Vsh[r0 + min(base + qd + 4 * r, last)];
            }
            return;
        }
        const int last = len > 0 ? len - 1 : 0;
#pragma unroll
        for (int h = 0; h < H; ++h) {
            const int row = min(base + 16 * h + i, last);
            const uint4* p = reinterpret_cast<const uint4*>(Kh + (size_t)(r0 + row) * D + qd * (D / 4));
#pragma unroll
            for (int s = 0; s < KS; ++s) k[h][s] = p[s];
        }
        const int rg = lane / LPR, cc = lane % LPR;
#pragma unroll
        for (int u = 0; u < VU; ++u) {
            const int row = min(base + u * RPW + rg, last);
            if constexpr (VQ == 8)
                v[u] = *reinterpret_cast<const uint2*>(reinterpret_cast<const int8_t*>(Vh) + (size_t)(r0 + row) * D + cc * 8);
            else if constexpr (VQ == 4)
                v[u] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(Vh) + (size_t)(r0 + row) * (D / 2) +
                                                          cc * 4);
            else
                v[u] = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(Vh) + (size_t)(r0 + row) * D + cc * 8);
        }
        if constexpr (VQ) {
#pragma unroll
            for (int h = 0; h < H; ++h)
#pragma unroll
                for (int r = 0; r < 4; ++r) vs[h][r] = Vsh[r0 + min(base + 16 * h + 4 * qd + r, last)];
        }
    }
};

template <int GM>
constexpr int pad_g()
{
    return GM < 4 ? 4 : GM;
}

// LDS hand-off from the MFMA lanes (logits, one head per lane) to the value
// lanes (rows): probabilities and rescale factors of the wave's current tile.
template <int GM, int TR>
struct PSmem {
    float p[kWaves][TR][pad_g<GM>()];
    float alpha[kWaves][pad_g<GM>()];
};

// Sums over the four 16-lane rows of a wave of NV values per lane (NV a
// multiple of 4), transposed on the way: a 32-lane swap of the pair (v[2i],
// v[2i+1]) and an add leave value 2i summed over lanes l and l ^ 32 in rows
// 0-1 and value 2i+1 in rows 2-3; a 16-lane swap of two such results and an
// add complete four sums, one per row.  Afterwards register t[i] of every
// lane of row r holds the total of value 4 i + kRowOrder[r].
constexpr int kRowOrder[4] = {0, 2, 1, 3};

template <int NV>
__device__ __forceinline__ void rows_sum_transposed(const float (&v)[NV], float (&t)[NV / 4])
{
    float s[NV / 2];
#pragma unroll
    for (int i = 0; i < NV / 2; ++i) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[2 * i]), __float_as_uint(v[2 * i + 1]),
                                                        false, false);
        s[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
#pragma unroll
    for (int i = 0; i < NV / 4; ++i) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(s[2 * i]), __float_as_uint(s[2 * i + 1]),
                                                        false, false);
        t[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}

// Running state of one wave's softmax partial (GM heads, padded heads carry
// zero queries and are discarded by the caller).
template <int GM>
struct MState {
    float m, lsum;          // MFMA view: head (lane % 16)
    float acc[GM][8];       // value view: 8 elements of the lane's row segment
};

// The logits of the held-out row (skip) go to clg[head] as they are computed.
template <int D, int GM, int TR, int VQ>
__device__ __forceinline__ void mfma_tile(const MTile<D, TR, VQ>& tl, int base, int r0, int len, int skip,
                                          const bf16x8 (&qhi)[D / 32], const bf16x8 (&qlo)[D / 32],
                                          PSmem<GM, TR>& ps, MState<GM>& st, float* clg)
{
    using T = MTile<D, TR, VQ>;
    constexpr int H = T::H, KS = T::KS, LPR = T::LPR, RPW = T::RPW, VU = T::VU;
    constexpr int GP = pad_g<GM>();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, qd = lane >> 4;
    const int rg = lane / LPR;

    f32x4 C[H];
#pragma unroll
    for (int h = 0; h < H; ++h) {
        C[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, tl.k[h][s]);
            C[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qhi[s], C[h], 0, 0, 0);
            C[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qlo[s], C[h], 0, 0, 0);
        }
    }
    // logits of rows 16h + 4qd + r for head n; masked rows get -inf
    float lg[H][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = base + 16 * h + 4 * qd + r;
            const bool held = (r0 + row) == skip;
            const bool ok = row < len && !held;
            if (held && n < GM) clg[n] = C[h][r];
            lg[h][r] = ok ? C[h][r] : -INFINITY;
            tmax = fmaxf(tmax, lg[h][r]);
        }
    {
        float2 t2 = swap_pair<16>(tmax);
        tmax = fmaxf(t2.x, t2.y);
        t2 = swap_pair<32>(tmax);
        tmax = fmaxf(t2.x, t2.y);
    }
    const float mx = fmaxf(st.m, tmax);
    const float ms = mx == -INFINITY ? 0.f : mx;
    const float alpha = exp2_fast(st.m - ms);
    st.m = mx;
    float psum = 0.f;
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = exp2_fast(lg[h][r] - ms);
            psum += p;
            // quantized values: the row's scale rides on its probability
            const float pv = VQ ? p * tl.vs[VQ ? h : 0][r] : p;
            if (n < GM) ps.p[wave][16 * h + 4 * qd + r][n] = pv;
        }
    st.lsum = st.lsum * alpha + psum;
    if (qd == 0 && n < GM) ps.alpha[wave][n] = alpha;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // value lanes: rescale, then accumulate p * v
    float al[GP];
#pragma unroll
    for (int g4 = 0; g4 < GP / 4; ++g4) {
        const float4 a4 = reinterpret_cast<const float4*>(ps.alpha[wave])[g4];
        al[4 * g4] = a4.x;
        al[4 * g4 + 1] = a4.y;
        al[4 * g4 + 2] = a4.z;
        al[4 * g4 + 3] = a4.w;
    }
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) st.acc[g][e] *= al[g];
#pragma unroll
    for (int u = 0; u < VU; ++u) {
        const int trow = u * RPW + rg;
        float pg[GP];
#pragma unroll
        for (int g4 = 0; g4 < GP / 4; ++g4) {
            const float4 p4 = reinterpret_cast<const float4*>(ps.p[wave][trow])[g4];
            pg[4 * g4] = p4.x;
            pg[4 * g4 + 1] = p4.y;
            pg[4 * g4 + 2] = p4.z;
            pg[4 * g4 + 3] = p4.w;
        }
        float vf[8];
        if constexpr (VQ == 8) {
            const uint32_t w[2] = {tl.v[u].x, tl.v[u].y};
#pragma unroll
            for (int e = 0; e < 8; ++e) vf[e] = (float)(int8_t)((w[e >> 2] >> (8 * (e & 3))) & 0xFFu);
        } else if constexpr (VQ == 4) {
            // code e in bits 4e .. 4e + 3, sign-extended by an arithmetic shift
#pragma unroll
            for (int e = 0; e < 8; ++e) vf[e] = (float)((int32_t)(tl.v[u] << (28 - 4 * e)) >> 28);
        } else {
            Vec16<bf16_t>::cvt(tl.v[u], vf);
        }
#pragma unroll
        for (int g = 0; g < GM; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) st.acc[g][e] = fmaf(pg[g], vf[e], st.acc[g][e]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// A wave's running partial when P.V runs on the matrix cores: the running
// max and sum of head n = lane % 16 (the logits' layout; the sum over the
// wave's rows of quarter lane / 16), and in register r of acc[blk] the
// accumulator of head 4 (lane / 16) + r, column 8 (lane % 16) + blk.
struct MStatePV {
    float m, lsum;
    f32x4 acc[8];
};

// Rescale factor of head 4 (lane / 16) + r, from the lane of the logits
// layout that holds it (alpha: head lane % 16).  Heads beyond the group are
// padding whatever they get.
template <int GM>
__device__ __forceinline__ float head_alpha(float alpha, int qd, int r)
{
    const int ai = __float_as_int(alpha);
    if constexpr (GM <= 4) {
        return __int_as_float(__builtin_amdgcn_readlane(ai, r));
    } else if constexpr (GM <= 8) {
        const int a0 = __builtin_amdgcn_readlane(ai, r), a1 = __builtin_amdgcn_readlane(ai, 4 + r);
        return __int_as_float((qd & 1) ? a1 : a0);
    } else {
        return __int_as_float(__builtin_amdgcn_ds_bpermute((4 * qd + r) * 4, __float_as_int(alpha)));
    }
}

// One 16-row tile with both products on the matrix cores (d = 128).  The K
// tile's rows enter the logits MFMA in the order
// pi(i) = i / 4 + 4 (i % 4) (MTile::load), so register r of the lanes of
// quarter qd holds the logit of physical row qd + 4 r for head n = lane % 16.
// That is the A-operand layout of a 16 x 16 x 16 MFMA with the heads as its M
// dimension and the tile's rows, in the order pi, as its K dimension.  The
// coalesced value loads hold row qd + 4 u, columns 8 n .. 8 n + 7 in v[u]
// (lane n of quarter qd), so element blk of v[0..3] is that MFMA's B operand
// for output column 8 n + blk: P.V is eight MFMAs, one per column block, with
// no exchange between lanes.  The probabilities enter as a bf16 high part and
// a bf16 remainder (two MFMAs into one fp32 accumulator), as the queries do
// in the logits; the values are bf16, or integer codes converted exactly to
// bf16 with each row's scale folded into its probability, so every product
// is exact.
// Two small integers as a pair of bf16 (a in the low half): their fp32
// forms are exact in bf16 (|code| <= 127 needs 7 bits), i.e. the high halves.
__device__ __forceinline__ uint32_t bf16_pair_of_ints(int a, int b)
{
    return __builtin_amdgcn_perm(__float_as_uint((float)b), __float_as_uint((float)a), 0x07060302u);
}

template <int GM, int VQ = 0>
__device__ __forceinline__ void mfma_tile_pv(const MTile<128, 16, VQ>& tl, int base, int r0, int len, int skip,
                                             const bf16x8 (&qhi)[4], const bf16x8 (&qlo)[4], MStatePV& st,
                                             float* clg)
{
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, qd = lane >> 4;

    f32x4 C = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, tl.k[0][s]);
        C = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qhi[s], C, 0, 0, 0);
        C = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qlo[s], C, 0, 0, 0);
    }
    // logits of physical rows qd + 4 r for head n; masked rows get -inf
    float lg[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = base + qd + 4 * r;
        const bool held = (r0 + row) == skip;
        if (held && n < GM) clg[n] = C[r];
        lg[r] = (row < len && !held) ? C[r] : -INFINITY;
        tmax = fmaxf(tmax, lg[r]);
    }
    {
        float2 t2 = swap_pair<16>(tmax);
        tmax = fmaxf(t2.x, t2.y);
        t2 = swap_pair<32>(tmax);
        tmax = fmaxf(t2.x, t2.y);
    }
    const float mold = st.m;
    const float mx = fmaxf(mold, tmax);
    const float ms = mx == -INFINITY ? 0.f : mx;
    const float alpha = exp2_fast(mold - ms);
    st.m = mx;
    float p[4], psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        p[r] = exp2_fast(lg[r] - ms);
        psum += p[r];
    }
    st.lsum = st.lsum * alpha + psum;
    // the accumulators are rescaled only when some head's maximum moved
    // (a wave-uniform branch; alpha is exactly 1 for the others)
    if (__builtin_amdgcn_ballot_w64(mx != mold) != 0ull) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float ah = head_alpha<GM>(alpha, qd, r);
#pragma unroll
            for (int blk = 0; blk < 8; ++blk) st.acc[blk][r] *= ah;
        }
    }
    // quantized values: each row's scale rides on its probability in the A
    // operand (the sum above is of the unscaled ones), and P.V runs on the
    // raw codes, converted exactly to bf16
    bf16x4 ph, pl;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float pa = VQ ? p[r] * tl.vs[0][r] : p[r];
        ph[r] = (__bf16)pa;
        pl[r] = (__bf16)(pa - (float)ph[r]);
    }
    const s16x4 aph = __builtin_bit_cast(s16x4, ph), apl = __builtin_bit_cast(s16x4, pl);
    // Value rows at or past len read as zero (the buffer's range ends at
    // len), so masked rows add exactly 0 * 0.
    uint4 vr[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if constexpr (VQ == 8) {
            const uint32_t x = tl.v[u].x, y = tl.v[u].y;
            auto c8 = [](uint32_t w, int k) { return (int)(int8_t)(w >> (8 * k)); };
            vr[u] = make_uint4(bf16_pair_of_ints(c8(x, 0), c8(x, 1)), bf16_pair_of_ints(c8(x, 2), c8(x, 3)),
                               bf16_pair_of_ints(c8(y, 0), c8(y, 1)), bf16_pair_of_ints(c8(y, 2), c8(y, 3)));
        } else if constexpr (VQ == 4) {
            const uint32_t w = tl.v[u];
            auto c4 = [](uint32_t x, int e) { return (int32_t)(x << (28 - 4 * e)) >> 28; };
            vr[u] = make_uint4(bf16_pair_of_ints(c4(w, 0), c4(w, 1)), bf16_pair_of_ints(c4(w, 2), c4(w, 3)),
                               bf16_pair_of_ints(c4(w, 4), c4(w, 5)), bf16_pair_of_ints(c4(w, 6), c4(w, 7)));
        } else {
            vr[u] = tl.v[u];
        }
    }
#pragma unroll
    for (int blk = 0; blk < 8; ++blk) {
        const int w = blk >> 1;
        uint32_t x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint4 vv = vr[u];
            x[u] = w == 0 ? vv.x : w == 1 ? vv.y : w == 2 ? vv.z : vv.w;
        }
        // v_perm_b32: bytes 0-3 of the selection are the second operand's,
        // 4-7 the first's; take the low (even blk) or high (odd blk) halves
        const uint32_t sel = (blk & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t b0 = __builtin_amdgcn_perm(x[1], x[0], sel);
        const uint32_t b1 = __builtin_amdgcn_perm(x[3], x[2], sel);
        const s16x4 bv = __builtin_bit_cast(s16x4, make_uint2(b0, b1));
        st.acc[blk] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aph, bv, st.acc[blk], 0, 0, 0);
        st.acc[blk] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(apl, bv, st.acc[blk], 0, 0, 0);
    }
}

// Same contract as attend_rows, for bf16 K/V.  Logits come from MFMA: the
// query of head n is column n of the B operand, split into a bf16 high part
// and a bf16 remainder (two MFMAs into one fp32 accumulator), so the products
// keep fp32 accuracy while K stays exact.  Probabilities go through LDS to the
// lanes that hold the value rows; P.V is accumulated in fp32 on the VALU.
// Two tiles alternate: one is computed while the other is in flight.
template <int D, int GM, int TR, int NB, int VQ = 0, int QS = D>
__device__ __forceinline__ void attend_rows_mfma(const bf16_t* __restrict__ Kh, const void* __restrict__ Vh,
                                                 const float* __restrict__ Vsh, const float* __restrict__ qh, int G,
                                                 int r0, int len, int skip, MTile<D, TR, VQ> (&ring)[NB],
                                                 AttnSmem<D, GM>& sm, PSmem<GM, TR>& ps, float* clg)
{
    constexpr int KS = D / 32, LPR = D / 8;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, qd = lane >> 4;
    const int rg = lane / LPR, cc = lane % LPR;

    bf16x8 qhi[KS], qlo[KS];
    {
        const float qs = qscale2<D>();
        const float* qp = qh + (size_t)(n < G ? n : 0) * QS + qd * (D / 4);
#pragma unroll
        for (int s = 0; s < KS; ++s) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = n < G ? qp[8 * s + e] * qs : 0.f;
                const __bf16 hi = (__bf16)x;
                qhi[s][e] = hi;
                qlo[s][e] = (__bf16)(x - (float)hi);
            }
        }
    }

    const int step = kWaves * TR;
    const int b0 = wave * TR;
    const int ntile = len > b0 ? (len - b0 + step - 1) / step : 0;
    if constexpr (pv_on_mfma<D, VQ>()) {
        static_assert(TR == 16, "one 16-row block per tile");
        MStatePV st;
        st.m = -INFINITY;
        st.lsum = 0.f;
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) st.acc[blk] = f32x4{0.f, 0.f, 0.f, 0.f};
        // the ring as below
        int k = 0;
        for (; k + 2 * NB <= ntile; k += NB) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                mfma_tile_pv<GM, VQ>(ring[i], b0 + (k + i) * step, r0, len, skip, qhi, qlo, st, clg);
                ring[i].load(Kh, Vh, Vsh, r0, len, b0 + (k + i + NB) * step);
            }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (k + i < ntile) {
                mfma_tile_pv<GM, VQ>(ring[i], b0 + (k + i) * step, r0, len, skip, qhi, qlo, st, clg);
                if (k + i + NB < ntile) ring[i].load(Kh, Vh, Vsh, r0, len, b0 + (k + i + NB) * step);
            }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i)
            if (k + NB + i < ntile)
                mfma_tile_pv<GM, VQ>(ring[i], b0 + (k + NB + i) * step, r0, len, skip, qhi, qlo, st, clg);

        float lsum = st.lsum;
        {
            float2 t2 = swap_pair<16>(lsum);
            lsum = t2.x + t2.y;
            t2 = swap_pair<32>(lsum);
            lsum = t2.x + t2.y;
        }
        if (qd == 0 && n < GM) {
            sm.m[wave][n] = st.m;
            sm.l[wave][n] = lsum;
        }
        // head 4 qd + r, columns 8 n .. 8 n + 7: the eight blocks' register r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int g = 4 * qd + r;
            if (g < GM) {
                float4* dst = reinterpret_cast<float4*>(&sm.acc[wave][g < GM ? g : 0][8 * n]);
                dst[0] = make_float4(st.acc[0][r], st.acc[1][r], st.acc[2][r], st.acc[3][r]);
                dst[1] = make_float4(st.acc[4][r], st.acc[5][r], st.acc[6][r], st.acc[7][r]);
            }
        }
        __syncthreads();
        return;
    }

    MState<GM> st;
    st.m = -INFINITY;
    st.lsum = 0.f;
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) st.acc[g][e] = 0.f;

    // tiles of this wave: base = b0 + k * step, k < ntile.  Tiles 0 .. NB-1
    // are in flight on entry; every buffer is reloaded with the tile NB ahead
    // as soon as it has been computed.  In the main loop every reload is
    // valid, so no load sits in a branch there and the wait counters stay
    // exact; the last 2 NB tiles form the tail.
    int k = 0;
    for (; k + 2 * NB <= ntile; k += NB) {
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            mfma_tile<D, GM, TR>(ring[i], b0 + (k + i) * step, r0, len, skip, qhi, qlo, ps, st, clg);
            ring[i].load(Kh, Vh, Vsh, r0, len, b0 + (k + i + NB) * step);
        }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        if (k + i < ntile) {
            mfma_tile<D, GM, TR>(ring[i], b0 + (k + i) * step, r0, len, skip, qhi, qlo, ps, st, clg);
            if (k + i + NB < ntile) ring[i].load(Kh, Vh, Vsh, r0, len, b0 + (k + i + NB) * step);
        }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i)
        if (k + NB + i < ntile) mfma_tile<D, GM, TR>(ring[i], b0 + (k + NB + i) * step, r0, len, skip, qhi, qlo, ps, st, clg);

    // the wave's rows share one running max per head: sums combine directly
    float lsum = st.lsum;
    {
        float2 t2 = swap_pair<16>(lsum);
        lsum = t2.x + t2.y;
        t2 = swap_pair<32>(lsum);
        lsum = t2.x + t2.y;
    }
    if (qd == 0 && n < GM) {
        sm.m[wave][n] = st.m;
        sm.l[wave][n] = lsum;
    }
    // value view: the lanes of a 16-lane row hold 8 columns each of one row
    // group; with 8-lane groups (D = 64) the two groups of a row add first
    float v[GM * 8];
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) v[g * 8 + e] = st.acc[g][e];
    if constexpr (LPR == 8) {
#pragma unroll
        for (int i = 0; i < GM * 8; ++i) v[i] += dpp_f<kDppRor8>(v[i]);
    }
    float t[GM * 2];
    rows_sum_transposed<GM * 8>(v, t);
    if (LPR == 16 || (lane & 15) < 8) {
        const int ord = kRowOrder[qd];
#pragma unroll
        for (int i = 0; i < GM * 2; ++i) {
            const int idx = 4 * i + ord;
            sm.acc[wave][idx / 8][(lane % LPR) * 8 + idx % 8] = t[i];
        }
    }
    __syncthreads();
}


// ---------------------------------------------------------------------------
// LSE merge of the partials of one query head
// ---------------------------------------------------------------------------

// (m, l, a) <- log-sum-exp union with (mo, lo, ao); a holds 4 output elements.
__device__ __forceinline__ void lse_add4(float& m, float& l, float4& a, float mo, float lo, float4 ao)
{
    const float mx = fmaxf(m, mo);
    if (mx == -INFINITY) return;
    const float sa = exp2_fast(m - mx), sb = exp2_fast(mo - mx);
    l = l * sa + lo * sb;
    a.x = a.x * sa + ao.x * sb;
    a.y = a.y * sa + ao.y * sb;
    a.z = a.z * sa + ao.z * sb;
    a.w = a.w * sa + ao.w * sb;
    m = mx;
}

// The lane's (m, l, a) joined with those of lane ^ X (X = 16 or 32) through
// swap_pair; the join is symmetric, so it takes the two values as given.
template <int X>
__device__ __forceinline__ void lse_join_swap(float& m, float& l, float4& a)
{
    const float2 m2 = swap_pair<X>(m), l2 = swap_pair<X>(l);
    const float2 x2 = swap_pair<X>(a.x), y2 = swap_pair<X>(a.y), z2 = swap_pair<X>(a.z), w2 = swap_pair<X>(a.w);
    m = m2.x;
    l = l2.x;
    a = make_float4(x2.x, y2.x, z2.x, w2.x);
    lse_add4(m, l, a, m2.y, l2.y, make_float4(x2.y, y2.y, z2.y, w2.y));
}

// Sum over aligned groups of n adjacent lanes, n in {1, 2, 4, 8} and uniform
// over the block; every lane of a group ends with the group's sum.
__device__ __forceinline__ float lane_group_sum(float x, int n)
{
    if (n >= 2) x += dpp_f<kDppXor1>(x);
    if (n >= 4) x += dpp_f<kDppXor2>(x);
    if (n >= 8) x += dpp_f<kDppHalfMirror>(x);
    return x;
}

constexpr int kMergeThreads = 1024;

template <int D>
struct MergeSmem {
    static constexpr int TPR = D / 4;                 // threads per record (4 outputs each)
    static constexpr int RPI = kMergeThreads / TPR;   // records in flight per pass
    float m[RPI], l[RPI];
    float4 a[RPI][TPR];
    float nlg;
};

// One block merges the nsb partial records rec(j) of one query head, in
// hold-out mode also the candidate of every split j != js (base-2 logit and
// fp32 value row from cand(j)), and, if has_new, the new token (logit *nlg,
// value vnew4 of thread t: elements 4t .. 4t+3).  Every thread owns 4 output
// elements of a subset of the records, so all record loads are independent.
// Returns true in threads t < D/4, with outputs 4t .. 4t+3 in o.
// Records j < nbound are loaded (nbound needs no device load, so the loads
// are not held back by the ones that give nsb and js); those j >= nsb are
// ignored.
template <int D, typename RecF, typename CandF>
__device__ __forceinline__ bool merge_head(MergeSmem<D>& sm, int nbound, int nsb, RecF rec, bool holdout, int js,
                                           CandF cand, bool has_new, const float* nlg, float4 vnew4, float4& o)
{
    constexpr int TPR = MergeSmem<D>::TPR, RPI = MergeSmem<D>::RPI;
    const int tid = threadIdx.x, c4 = tid % TPR, jr = tid / TPR;
    float m = -INFINITY, l = 0.f;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
    for (int j = jr; j < nbound; j += RPI) {
        const float* r = rec(j);
        const float4 av = reinterpret_cast<const float4*>(r)[c4];
        const float mj = r[D], lj = r[D + 1];
        float cl = -INFINITY;
        float4 cv4 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (holdout) {
            const float* cv;
            cand(j, cl, cv);
            cv4 = reinterpret_cast<const float4*>(cv)[c4];
        }
        if (j < nsb) {
            if (lj > 0.f) lse_add4(m, l, a, mj, lj, av);
            if (holdout && j != js) lse_add4(m, l, a, cl, 1.f, cv4);
        }
    }
    if (c4 == 0) {
        sm.m[jr] = m;
        sm.l[jr] = l;
    }
    sm.a[jr][c4] = a;
    __syncthreads();
    if (tid >= TPR) return false;
    float M = -INFINITY, L = 0.f;
    float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
    if (has_new) {
        M = *nlg;
        L = 1.f;
        A = vnew4;
    }
#pragma unroll
    for (int k = 0; k < RPI; ++k) lse_add4(M, L, A, sm.m[k], sm.l[k], sm.a[k][tid]);
    const float inv = L > 0.f ? 1.f / L : 0.f;
    o = make_float4(A.x * inv, A.y * inv, A.z * inv, A.w * inv);
    return true;
}

template <typename KT>
__device__ __forceinline__ float4 load4_f32(const KT* p)
{
    return make_float4(to_f32(p[0]), to_f32(p[1]), to_f32(p[2]), to_f32(p[3]));
}

template <int GM>
constexpr int tile_rows()
{
    return 16;   // rows of a wave's tile in the bf16 path
}

// tiles of a wave in flight at once in the bf16 path
template <int GM, int D, int VQ>
constexpr int ring_depth()
{
    // with P.V on the VALU, 16 heads' accumulators take 128 registers a lane;
    // on the matrix cores they take 32 whatever the group size
    return pv_on_mfma<D, VQ>() || GM < 16 ? 2 : 1;
}

// ---------------------------------------------------------------------------
// FUSED schedule (one launch)
// ---------------------------------------------------------------------------

// Device-coherent accesses for data one block hands to another inside a
// launch.  Each XCD has its own L2 and those L2s are not coherent with each
// other; agent-scope atomic loads and stores (the sc1 cache policy) write
// through and re-fetch past them, so the data never sits stale in a writer's
// or a reader's L2, and no L2-wide writeback fence is needed.

// Every memory operation this thread issued has completed -- its write-through
// stores have reached the coherence point -- before anything after it is
// issued; the compiler may not move memory operations across either.
__device__ __forceinline__ void own_stores_complete()
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Loads of records other blocks wrote through to memory, with the cache
// policy of an agent-scope load (sc1: a line this XCD's L2 may hold stale is
// fetched again), 16 bytes at byte offset `off` of a buffer resource.
// Out-of-range offsets read zero.

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const float* base, size_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, (int)bytes, kRsrcWord3);
}

__device__ __forceinline__ float4 ld_sc1_16(__amdgpu_buffer_rsrc_t rs, int off)
{
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kCpolSC1);
    float4 f;
    __builtin_memcpy(&f, &v, 16);
    return f;
}

// Write-through stores with the same policy (the store side of the hand-off).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void st_sc1_16(__amdgpu_buffer_rsrc_t rs, int off, float4 v)
{
    u32x4 u;
    __builtin_memcpy(&u, &v, 16);
    __builtin_amdgcn_raw_buffer_store_b128(u, rs, off, 0, kCpolSC1);
}

__device__ __forceinline__ void st_sc1_8(__amdgpu_buffer_rsrc_t rs, int off, float2 v)
{
    u32x2 u;
    __builtin_memcpy(&u, &v, 8);
    __builtin_amdgcn_raw_buffer_store_b64(u, rs, off, 0, kCpolSC1);
}

// The block's partial of the fused step, write-through: acc [G][D] at `rec`
// and one (max, sum, candidate logit, 0) per head at `scal` (base 2; the
// candidate logit is 0 when the chunk has no candidate).
// One thread per output float4 (head g, columns i .. i + 3), summing the
// waves in order.  (Splitting an entry over several adjacent lanes joined by
// DPP measured slower: those lanes read rows of different waves that sit in
// the same LDS banks.)
template <int D, int GM>
__device__ __forceinline__ void publish_fused(const AttnSmem<D, GM>& sm, __amdgpu_buffer_rsrc_t rec,
                                              __amdgpu_buffer_rsrc_t scal, int G, const float* clg, bool has_cand)
{
    constexpr int D4 = D / 4;
    for (int idx = threadIdx.x; idx < G * D4; idx += kThreads) {
        const int g = idx / D4, i = (idx % D4) * 4;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm.m[w][g]);
        const float ms = mx == -INFINITY ? 0.f : mx;
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
        float ls = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float sc = exp2_fast(sm.m[w][g] - ms);
            const float4 x = *reinterpret_cast<const float4*>(&sm.acc[w][g][i]);
            a = make_float4(fmaf(x.x, sc, a.x), fmaf(x.y, sc, a.y), fmaf(x.z, sc, a.z), fmaf(x.w, sc, a.w));
            ls = fmaf(sm.l[w][g], sc, ls);
        }
        st_sc1_16(rec, (g * D + i) * 4, a);
        if (i == 0) st_sc1_16(scal, g * 16, make_float4(mx, ls, has_cand ? clg[g] : 0.f, 0.f));
    }
}

// The published records of the blocks of a head, as read by its last block:
// acc [nsplit][G][D], (max, sum, candidate logit, 0) [nsplit][G] and
// candidate value rows [nsplit][D].
struct MergeArgs {
    __amdgpu_buffer_rsrc_t rec, scal, cv;
    int G, nsb, r, c4;
    bool full;
    unsigned wkey0;   // low half of the head's eviction key (its slot), valid in lane 0 of each wave
    int chunk;
};

// Folds the records of splits j = j0 + r + RS * jj (jj < JB, all j0) into the
// thread's running (M, L, A) of its 4 output columns c4 for every head.  The
// loads of a batch are all issued before any is used (one round trip to
// memory per batch); the (max, sum, logit) records of a batch are fetched
// once, one per thread, and shared through s_sc.  Every split's held-out
// candidate is added back except the winner's (split js of the evicted
// slot).  Returns the evicted slot (`e` when the cache is not full).
template <int D, int GM, int JB>
__device__ __forceinline__ int merge_splits(const MergeArgs& a, int e, float4* s_sc, float (&Mt)[GM],
                                            float (&Lt)[GM], float4 (&At)[GM])
{
    constexpr int RS = kThreads / (D / 4);
    const int tid = threadIdx.x;
    const int nsc = RS * JB * a.G;   // (split, head) records of a batch, <= kThreads
    const int jl = tid / a.G, gl = tid - jl * a.G;
    int js = -1;
    for (int j0 = 0; j0 < a.nsb; j0 += RS * JB) {
        const float4 scv = ld_sc1_16(a.scal, (min(j0 + jl, a.nsb - 1) * a.G + gl) * 16);
        float4 av[JB][GM], cv[JB];
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            const int j = min(j0 + a.r + RS * jj, a.nsb - 1);
            cv[jj] = ld_sc1_16(a.cv, (j * D + 4 * a.c4) * 4);
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                const int gg = min(g, a.G - 1);
                av[jj][g] = ld_sc1_16(a.rec, ((j * a.G + gg) * D + 4 * a.c4) * 4);
            }
        }
        if (a.full) {
            e = cand_slot(__builtin_amdgcn_readlane(a.wkey0, 0));
            js = e / a.chunk;
        }
        __syncthreads();   // readers of the previous batch are done
        if (tid < nsc) s_sc[tid] = scv;
        __syncthreads();
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            const int j = j0 + a.r + RS * jj;
            if (j < a.nsb) {
                const bool hold = a.full && j != js;
#pragma unroll
                for (int g = 0; g < GM; ++g) {
                    const float4 sc = s_sc[(a.r + RS * jj) * a.G + min(g, a.G - 1)];
                    if (sc.y > 0.f) lse_add4(Mt[g], Lt[g], At[g], sc.x, sc.y, av[jj][g]);
                    if (hold) lse_add4(Mt[g], Lt[g], At[g], sc.z, 1.f, cv[jj]);
                }
            }
        }
    }
    return e;
}

// Shared memory of the last block's merge: one (max, sum) per head and wave
// and 4 outputs per wave, head and 4-element column, and the (max, sum, logit) records of the
// batch being folded; with one common maximum per head, the two weights of
// every record and per head the total weight and the new token's weight.
template <int D, int GM>
struct MergeBlockSmem {
    float m[GM][kWaves];
    float l[GM][kWaves];
    float4 a[kWaves][GM][D / 4];
    float4 sc[kThreads];
    float2 w[kThreads];
    float L[GM], sn[GM];
};

// Merge of a head's split records against one common maximum per head, for
// nsb * G <= kThreads records.  Thread t < nsb * G fetches record t = (split
// j = t / G, head g = t % G): (max m, sum l, candidate logit z).  M_g is the
// largest of the maxima of the non-empty partials, of the logits of the
// candidates that are added back (every split's but the winner's) and of the
// new token's logit, so every weight exp2(x - M_g) is at most 1.  One wave
// per head writes each record's weights (exp2(m - M_g) for the partial,
// exp2(z - M_g) for its candidate) to w, and the head's total weight (the
// new token's included) to L.  Each thread then folds the acc rows and
// candidate value rows of splits j = r + RS * jj into At[g] (its 4 columns
// c4) with plain multiply-adds; the batch's loads are all issued before any
// is used.  Returns the evicted slot (`e` when the cache is not full).
template <int D, int GM, int JB>
__device__ __forceinline__ int merge_scaled(const MergeArgs& a, int e, const float* nlg, MergeBlockSmem<D, GM>& mg,
                                            float4 (&At)[GM])
{
    constexpr int RS = kThreads / (D / 4);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = a.G, nrec = a.nsb * G;
    const float4 scv = ld_sc1_16(a.scal, min(tid, nrec - 1) * 16);
    float4 av[JB][GM], cv[JB];
    auto issue = [&](int j0) {
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            const int j = min(j0 + a.r + RS * jj, a.nsb - 1);
            // candidate rows exist only when the cache is full (every split
            // then writes one); otherwise their weight is 0 and the row is
            // taken as 0, never read
            cv[jj] = a.full ? ld_sc1_16(a.cv, (j * D + 4 * a.c4) * 4) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int g = 0; g < GM; ++g)
                av[jj][g] = ld_sc1_16(a.rec, ((j * G + min(g, G - 1)) * D + 4 * a.c4) * 4);
        }
    };
    issue(0);
    __builtin_amdgcn_sched_barrier(0);   // the key is read after the record loads are issued
    int js = -1;
    if (a.full) {
        e = cand_slot(__builtin_amdgcn_readlane(a.wkey0, 0));
        js = e / a.chunk;
    }
    if (tid < nrec) mg.sc[tid] = scv;
    __syncthreads();
    for (int g = wave; g < G; g += kWaves) {
        float mx = nlg[g];
        for (int j = lane; j < a.nsb; j += 64) {
            const float4 r = mg.sc[j * G + g];
            if (r.y > 0.f) mx = fmaxf(mx, r.x);
            if (a.full && j != js) mx = fmaxf(mx, r.z);
        }
        mx = wave_max_f(mx);
        float ls = 0.f;
        for (int j = lane; j < a.nsb; j += 64) {
            const float4 r = mg.sc[j * G + g];
            const float sp = r.y > 0.f ? exp2_fast(r.x - mx) : 0.f;
            const float sc = a.full && j != js ? exp2_fast(r.z - mx) : 0.f;
            ls = fmaf(r.y, sp, ls) + sc;
            mg.w[j * G + g] = make_float2(sp, sc);
        }
        ls = wave_sum_f(ls);
        if (lane == 0) {
            const float sn = exp2_fast(nlg[g] - mx);
            mg.sn[g] = sn;
            mg.L[g] = ls + sn;
        }
    }
    __syncthreads();
    for (int j0 = 0; j0 < a.nsb; j0 += RS * JB) {
        if (j0 > 0) issue(j0);
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            const int j = j0 + a.r + RS * jj;
            if (j < a.nsb) {
#pragma unroll
                for (int g = 0; g < GM; ++g) {
                    if (g < G) {
                        const float2 w = mg.w[j * G + g];
                        const float4 x = av[jj][g], y = cv[jj];
                        At[g] = make_float4(fmaf(y.x, w.y, fmaf(x.x, w.x, At[g].x)), fmaf(y.y, w.y, fmaf(x.y, w.x, At[g].y)),
                                            fmaf(y.z, w.y, fmaf(x.z, w.x, At[g].z)), fmaf(y.w, w.y, fmaf(x.w, w.x, At[g].w)));
                    }
                }
            }
        }
    }
    return e;
}

// Sum of v over the lane and its partner lane ^ X (X = 16 or 32); the sum is
// the same in both lanes.
template <int X>
__device__ __forceinline__ float4 pair_sum4(float4 v)
{
    const float2 x2 = swap_pair<X>(v.x), y2 = swap_pair<X>(v.y), z2 = swap_pair<X>(v.z), w2 = swap_pair<X>(v.w);
    return make_float4(x2.x + x2.y, y2.x + y2.y, z2.x + z2.y, w2.x + w2.y);
}

template <int D, int BITS, int GM>
union FusedSmem {
    float R[BITS * (D + 4)];    // encoder operand (R transposed, rows padded), dead once the codes are known
    AttnSmem<D, GM> at;
    MergeBlockSmem<D, GM> mg;
};

// 16-byte code groups per thread the fused step loads before its tiles
constexpr int kCodePre = 4;

// VQ: values are stored as codes of VQ bits (8 or 4) with a per-row scale
// (bf16 keys only), or as given (0).
template <int D, int BITS, int GM, typename KT, int VQ = 0>
__global__ __launch_bounds__(kThreads) void k_decode_fused(DevCache c, const float* __restrict__ q,
                                                           const KT* __restrict__ knew, const KT* __restrict__ vnew,
                                                           float* __restrict__ out, int* __restrict__ evicted)
{
    using CT = typename CodeT<BITS>::T;
    constexpr int VS = 16 / sizeof(CT);
    constexpr bool kMfma = std::is_same<KT, bf16_t>::value;
    constexpr int TR = tile_rows<GM>();
    // Workgroups go to the XCDs round-robin by number.  With equal budgets
    // the split is fastest, which spreads each head over all XCDs (measured
    // marginally faster there).  With ragged budgets the KV head is fastest
    // and the rest follows the block list (equal splits per sequence,
    // longest first): each XCD gets the same mix of work, and its compute
    // units that finish early take the short blocks.
    int split, h, b, chunk;
    if (c.ragged) {
        const int i = blockIdx.x / c.Hkv;
        h = blockIdx.x - i * c.Hkv;
        const uint2 e = c.blk[i];
        b = (int)(e.x & 0xFFFFu);
        split = (int)(e.x >> 16);
        chunk = (int)e.y;
    } else {
        split = blockIdx.x;
        h = blockIdx.y;
        b = blockIdx.z;
        chunk = c.chunk;
    }
    const int G = c.G;
    const int head = b * c.Hkv + h;
    const int s0 = split * chunk;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    __shared__ FusedSmem<D, BITS, GM> u;
    __shared__ PSmem<GM, TR> ps;
    constexpr int QS = D + 4;                      // row stride of s_q (padded: see enc_lds)
    __shared__ __align__(16) float s_q[GM][QS];    // the group's queries (fp32)
    __shared__ __align__(16) KT s_kn[D], s_vn[D];  // the new token's key and value
    __shared__ __align__(16) float s_vdq[VQ ? D : 1];   // quantized values: the new value as the cache holds it
    __shared__ uint16_t s_vq2[VQ ? D / 2 : 1];          // ... its codes, two per entry (in the low byte at 4 bits)
    __shared__ float s_vsc;                              // ... and its scale
    __shared__ uint32_t s_q16[BITS / 16][16];
    __shared__ uint32_t s_k16[BITS / 16];
    __shared__ unsigned long long s_red[kWaves];
    __shared__ float s_nlg[GM];
    __shared__ float s_clg[GM];
    __shared__ int s_last;
    __shared__ int s_state[3];   // budget, occupancy, step
    AttnSmem<D, GM>& sm = u.at;

    const int hq0 = b * c.Hq + h * G;
    const float* qh = q + (size_t)hq0 * D;
    const size_t rowbase = (size_t)head * c.Smax;
    KT* Kh = reinterpret_cast<KT*>(c.K) + rowbase * D;
    KT* Vh = reinterpret_cast<KT*>(c.V) + rowbase * D;
    constexpr int VROW = VQ ? D * VQ / 8 : 1;                      // bytes of a row of value codes
    uint8_t* Vq = reinterpret_cast<uint8_t*>(c.V) + rowbase * VROW;  // value codes (VQ)
    float* Vsh = VQ ? c.vs + rowbase : nullptr;
    const void* Vbase = VQ ? (const void*)Vq : (const void*)Vh;
    const CT* codeh = reinterpret_cast<const CT*>(c.code) + (size_t)head * c.code_slots;
    const size_t crec = (size_t)head * c.nsplit + split;
    const KT* kh = knew + (size_t)head * D;
    const KT* vh = vnew + (size_t)head * D;

    // The small operands (R, the group's queries, the new key and value) and
    // the chunk's codes are fetched first and waited for before any K/V tile
    // is requested: issued behind the tile prefetch of every block they would
    // queue behind ~all of it in the memory system, and the loop cannot start
    // before the codes are known.  They go through LDS.
    constexpr int NR4 = D * BITS / 4;
    constexpr int RPT = (NR4 + kThreads - 1) / kThreads;
    constexpr int NK4 = D * (int)sizeof(KT) / 16;
    static_assert(GM * D / 4 <= kThreads && NK4 <= 64, "staging shape");
    float4 rst[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) rst[j] = reinterpret_cast<const float4*>(c.R)[min(tid + j * kThreads, NR4 - 1)];
    const int NQ4 = G * D / 4;
    const float4 qst = reinterpret_cast<const float4*>(qh)[min(tid, NQ4 - 1)];
    const uint4 kvst = reinterpret_cast<const uint4*>(wave == 0 ? kh : vh)[min(lane, NK4 - 1)];
    // the chunk's codes, up to kCodePre 16-byte groups per thread (every
    // workload's chunk; longer chunks load the rest while scoring)
    // (groups past the chunk read its last group again, one cached line)
    const int clast = max(min(s0 + chunk, (int)c.code_slots) - VS, 0);
    uint4 craw[kCodePre];
#pragma unroll
    for (int j = 0; j < kCodePre; ++j)
        craw[j] = *reinterpret_cast<const uint4*>(codeh + min(s0 + (j * kThreads + tid) * VS, clast));
    // (threads past the end store the last element again, with the value
    // they loaded from it, so every store is unconditional)
    // R goes in transposed (b rows of d entries, padded), q with padded rows
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int i4 = min(tid + j * kThreads, NR4 - 1);
        const int k = i4 / (BITS / 4), c = 4 * (i4 % (BITS / 4));
        u.R[(c + 0) * (D + 4) + k] = rst[j].x;
        u.R[(c + 1) * (D + 4) + k] = rst[j].y;
        u.R[(c + 2) * (D + 4) + k] = rst[j].z;
        u.R[(c + 3) * (D + 4) + k] = rst[j].w;
    }
    {
        const int i4 = min(tid, NQ4 - 1);
        *reinterpret_cast<float4*>(&s_q[i4 / (D / 4)][4 * (i4 % (D / 4))]) = qst;
    }
    reinterpret_cast<uint4*>(wave == 0 ? s_kn : s_vn)[min(lane, NK4 - 1)] = kvst;
    // The cache state goes through LDS before the barrier, stored by every
    // thread (the same values), which keeps its loads next to the ones above:
    // left alone, the compiler issues them after the barrier, and the tile
    // loads below, which need the chunk's length, would wait for one more
    // round trip.
    {
        const int S0 = c.budget[b], n0 = c.state[2 * head], t0 = c.state[2 * head + 1];
        s_state[0] = S0;
        s_state[1] = n0;
        s_state[2] = t0;
    }
    __syncthreads();
    const int S = s_state[0], n = s_state[1], t = s_state[2];
    const int nsb = (S + chunk - 1) / chunk;
    const bool full = n >= S;
    const int len = max(min(s0 + chunk, n) - s0, 0);
    if (split >= nsb) return;   // (no block lies past its sequence's splits; kept as a guard)

    // The first tile of every wave is in flight while the codes are computed;
    // the rest of the ring is requested once the chunk's candidate is known.
    // (Requested all at once here, the ring fills the memory pipeline's queue,
    // and every wave waits at issue until most of it has drained, which holds
    // back the codes and the start of the loop.)
    constexpr int NB = ring_depth<GM, D, VQ>();
    MTile<D, TR, VQ> ring[kMfma ? NB : 1];
    Tile<D, KT> first;
    if constexpr (kMfma) {
        ring[0].load(Kh, Vbase, Vsh, s0, len, wave * TR);
    } else {
        first.load(Kh, Vh, s0, len, wave * Tile<D, KT>::ROWS);
    }

    // stages 1-2: codes of the group's queries (rows 0 .. G-1) and of the new
    // key (row G, or a pass of its own when the group fills all 16 rows)
    constexpr int NT = BITS / 16;
    if (wave < NT) {
        const uint32_t c16 = enc_lds<D, BITS, KT, QS>(&s_q[0][0], G, s_kn, u.R, wave);
        if (lane < G) s_q16[wave][lane] = c16;
        if (lane == G && G < 16) s_k16[wave] = c16;
    } else if (G == 16 && wave < 2 * NT) {
        const uint32_t c16 = enc_lds<D, BITS, KT, QS>(&s_q[0][0], 0, s_kn, u.R, wave - NT);
        if (lane == 0) s_k16[wave - NT] = c16;
    }
    // base-2 logit of the new token for each head (only the head's last block
    // uses them)
    {
        const float qs = qscale2<D>();
        const int i0 = 2 * lane;
        for (int g = wave; g < G; g += kWaves) {
            float dot = 0.f;
            if (i0 < D) dot = fmaf(s_q[g][i0] * qs, to_f32(s_kn[i0]), s_q[g][i0 + 1] * qs * to_f32(s_kn[i0 + 1]));
            dot = wave_sum_f(dot);
            if (lane == 0) s_nlg[g] = dot;
        }
    }
    __syncthreads();   // the codes are known; u.R is dead from here on
    if (split == 0) {
        if (tid < G) store_words(c.dbg_q + (size_t)(hq0 + tid) * c.W, c.W, join16<BITS>(s_q16, tid));
        if (tid == 0) {
            unsigned long long kc = 0;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) kc |= (unsigned long long)s_k16[nt] << (16 * nt);
            store_words(c.dbg_k + (size_t)head * c.W, c.W, kc);
        }
    }

    // stages 3-4 inside the chunk; the chunk's candidate joins the head's key
    int cand = -1;
    unsigned long long ckey = 0;
    if (full) {
        CT qc[GM];
#pragma unroll
        for (int g = 0; g < GM; ++g) qc[g] = g < G ? (CT)join16<BITS>(s_q16, g) : (CT)0;
        ckey = thread_candidate<BITS, GM, kCodePre>(codeh, qc, G, s0, s0 + len, craw);
        ckey = block_max_u64(ckey, s_red);
        cand = ckey ? cand_slot(ckey) : -1;
        if (tid == 0 && ckey) atomicMax(&c.ekey[2 * head + (t & 1)], ckey);
    }

    // The held-out candidate's value row: fetched now, converted and published
    // after the loop (the loop takes its logits as it passes its row).  The
    // load is unconditional (row 0 when there is no candidate) and its bits
    // stay raw until then: a conversion here would wait for the load, and so
    // for the whole tile ring issued before it, ahead of the loop.
    const size_t crow = (size_t)(cand >= 0 ? cand : 0);
    const int ce = 2 * (lane % (D / 2));
    using VRaw = typename std::conditional<VQ != 0, uint16_t, typename std::conditional<kMfma, uint32_t, float2>::type>::type;
    VRaw vraw;
    float vcsc = 0.f;
    if constexpr (VQ == 8) {
        vraw = *reinterpret_cast<const uint16_t*>(Vq + crow * VROW + ce);
        vcsc = Vsh[crow];
    } else if constexpr (VQ == 4) {
        vraw = Vq[crow * VROW + ce / 2];   // the two codes of elements ce, ce + 1
        vcsc = Vsh[crow];
    } else {
        vraw = *reinterpret_cast<const VRaw*>(Vh + crow * D + ce);
    }

    // the rest of the ring
    if constexpr (kMfma) {
#pragma unroll
        for (int i = 1; i < NB; ++i) ring[i].load(Kh, Vbase, Vsh, s0, len, (wave + i * kWaves) * TR);
    }
    // attention over the chunk with the candidate held out
    if constexpr (kMfma)
        attend_rows_mfma<D, GM, TR, NB, VQ, QS>(Kh, Vbase, Vsh, &s_q[0][0], G, s0, len, cand, ring, sm, ps, s_clg);
    else
        attend_rows<D, GM, KT, QS>(Kh, Vh, &s_q[0][0], G, s0, len, cand, first, sm, s_clg);

    // publish this chunk: partial softmax, candidate logits and value row
    // (the attention's closing barrier made its LDS results, the candidate's
    // logits included, visible to every wave)
    if (cand >= 0 && wave == 0 && 2 * lane < D) {
        float2 vc2;
        if constexpr (VQ == 8)
            vc2 = make_float2((float)(int8_t)(vraw & 0xFFu) * vcsc, (float)(int8_t)(vraw >> 8) * vcsc);
        else if constexpr (VQ == 4)
            vc2 = make_float2((float)((int32_t)((uint32_t)vraw << 28) >> 28) * vcsc,
                              (float)((int32_t)((uint32_t)vraw << 24) >> 28) * vcsc);
        else if constexpr (kMfma)
            vc2 = make_float2(__uint_as_float(vraw << 16), __uint_as_float(vraw & 0xFFFF0000u));
        else
            vc2 = vraw;
        st_sc1_8(dev_rsrc(c.cand_v + crec * D, (size_t)D * 4), 2 * lane * 4, vc2);
    }
    publish_fused<D, GM>(sm, dev_rsrc(c.frec + crec * G * D, (size_t)G * D * 4),
                         dev_rsrc(c.fscal + crec * G * 4, (size_t)G * 16), G, s_clg, cand >= 0);
    own_stores_complete();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&c.count[head * kCountStride], 1u) == (unsigned)(nsb - 1);
    __syncthreads();
    // The other blocks run the merge below dry: over empty record buffers
    // (their loads read zero and touch no memory) and with every global
    // store skipped.  Which compute unit merges a head changes from step to
    // step; without this, the merge's instructions reach the instruction
    // caches only as each unit happens to merge, and the first few hundred
    // steps of a run merge from cold caches.  Only the merge against one
    // common maximum (at most kThreads records, one batch of loads) is run
    // dry: the running log-sum-exp over very many splits would cost every
    // block a loop over all of them.
    const bool dry = !s_last;
    if (dry && nsb * G > kThreads) return;

    // ---- the last block of the head: winner, merge, write ----
    // Every thread owns 4 output columns (c4) of every head for the splits
    // j = r + RS * jj.  All loads of a batch of splits are issued before any
    // of them is used, so the merge costs one round trip to memory per batch.
    if (tid == 0 && !dry) c.count[head * kCountStride] = 0u;
    if constexpr (VQ) {
        // the new token's value row as the cache will hold it: codes of VQ
        // bits (v / scale rounded half to even, clamped to +-Q) with scale =
        // max|v| / Q, Q = 127 or 7, all in fp32; every later use of the value
        // is code * scale
        if (wave == 0) {
            constexpr float Q = VQ == 8 ? 127.0f : 7.0f;
            const int i0 = 2 * lane;
            const float f0 = i0 < D ? to_f32(s_vn[i0]) : 0.f, f1 = i0 < D ? to_f32(s_vn[i0 + 1]) : 0.f;
            const float sc = wave_max_f(fmaxf(fabsf(f0), fabsf(f1))) / Q;
            const float c0 = sc > 0.f ? fminf(fmaxf(rintf(f0 / sc), -Q), Q) : 0.f;
            const float c1 = sc > 0.f ? fminf(fmaxf(rintf(f1 / sc), -Q), Q) : 0.f;
            if (i0 < D) {
                constexpr uint32_t M = (1u << VQ) - 1u;
                s_vq2[lane] = (uint16_t)(((uint32_t)(int32_t)c0 & M) | (((uint32_t)(int32_t)c1 & M) << VQ));
                s_vdq[i0] = c0 * sc;
                s_vdq[i0 + 1] = c1 * sc;
            }
            if (lane == 0) s_vsc = sc;
        }
    }
    constexpr int TPR = D / 4;
    constexpr int RS = kThreads / TPR;
    constexpr int JBMAX = GM <= 4 ? 4 : (GM <= 8 ? 2 : 1);   // register budget
    const int c4 = tid % TPR, r = tid / TPR;
    // The winner's slot is the low half of the eviction key.  One lane per
    // wave loads it: a load by all lanes of this uniform address becomes a
    // scalar at once, and its wait would hold back the record loads issued
    // after it; the merge reads it (readlane) once those are on their way.
    unsigned wkey0 = 0u;
    if (lane == 0 && !dry)
        wkey0 = __hip_atomic_load(reinterpret_cast<unsigned*>(&c.ekey[2 * head + (t & 1)]), __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
    const size_t hrec = (size_t)head * c.nsplit;
    const size_t live = dry ? 0 : 1;
    MergeArgs ma{dev_rsrc(c.frec + hrec * G * D, live * c.nsplit * G * D * 4),
                 dev_rsrc(c.fscal + hrec * G * 4, live * c.nsplit * G * 16),
                 dev_rsrc(c.cand_v + hrec * D, live * c.nsplit * D * 4), G, nsb, r, c4, full, wkey0, chunk};
    const int per = (nsb + RS - 1) / RS;   // splits per thread
    MergeBlockSmem<D, GM>& mg = u.mg;
    static_assert(TPR == 16 || TPR == 32, "rows per wave");
    // Output float4 (head g, columns 4 cc .. 4 cc + 3) is summed by Q adjacent
    // lanes, lane k taking waves k, k + Q, ...
    const int nout = G * TPR;
    int qsh = 0;
    while ((2 << qsh) <= kWaves && (nout << (qsh + 1)) <= kThreads) ++qsh;
    const int Q = 1 << qsh, k = tid & (Q - 1);
    const int oi = min(tid >> qsh, nout - 1);
    const int og = oi / TPR, cc = oi % TPR;
    int e = n;
    float4 o;
    if (nsb * G <= kThreads) {
        // one common maximum per head: plain weighted sums from here on
        float4 At[GM];
#pragma unroll
        for (int g = 0; g < GM; ++g) At[g] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (per <= 1 || JBMAX == 1)
            e = merge_scaled<D, GM, 1>(ma, e, s_nlg, mg, At);
        else if (per <= 2 || JBMAX == 2)
            e = merge_scaled<D, GM, (JBMAX >= 2 ? 2 : 1)>(ma, e, s_nlg, mg, At);
        else
            e = merge_scaled<D, GM, JBMAX>(ma, e, s_nlg, mg, At);
        // the rows of a wave (its lanes that share c4) add up, then one entry
        // per wave; merge_scaled's barriers ordered the last reads of the
        // attention's memory before these writes
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            if (g < G) {
                if constexpr (TPR == 16) At[g] = pair_sum4<16>(At[g]);
                At[g] = pair_sum4<32>(At[g]);
                if (lane < TPR) mg.a[wave][g][c4] = At[g];
            }
        }
        __syncthreads();
        float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int w = k; w < kWaves; w += Q) {
            const float4 a = mg.a[w][og][cc];
            A = make_float4(A.x + a.x, A.y + a.y, A.z + a.z, A.w + a.w);
        }
        A = make_float4(lane_group_sum(A.x, Q), lane_group_sum(A.y, Q), lane_group_sum(A.z, Q),
                        lane_group_sum(A.w, Q));
        const float4 vn = VQ ? *reinterpret_cast<const float4*>(&s_vdq[VQ ? 4 * cc : 0]) : load4_f32(s_vn + 4 * cc);
        const float sn = mg.sn[og], inv = 1.f / mg.L[og];
        o = make_float4(fmaf(vn.x, sn, A.x) * inv, fmaf(vn.y, sn, A.y) * inv, fmaf(vn.z, sn, A.z) * inv,
                        fmaf(vn.w, sn, A.w) * inv);
    } else {
        // more records than threads: running log-sum-exp per thread
        float Mt[GM], Lt[GM];
        float4 At[GM];
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            Mt[g] = -INFINITY;
            Lt[g] = 0.f;
            At[g] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (per <= 1 || JBMAX == 1)
            e = merge_splits<D, GM, 1>(ma, e, u.mg.sc, Mt, Lt, At);
        else if (per <= 2 || JBMAX == 2)
            e = merge_splits<D, GM, (JBMAX >= 2 ? 2 : 1)>(ma, e, u.mg.sc, Mt, Lt, At);
        else
            e = merge_splits<D, GM, JBMAX>(ma, e, u.mg.sc, Mt, Lt, At);
        // the rows of a wave join, then one entry per wave
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            if (g < G) {
                if constexpr (TPR == 16) lse_join_swap<16>(Mt[g], Lt[g], At[g]);
                lse_join_swap<32>(Mt[g], Lt[g], At[g]);
            }
        }
        // merge_splits' barriers already ordered the attention's last use of
        // this memory before these writes, and its s_sc is a separate member
        if (lane < TPR) {
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                if (g < G) {
                    mg.a[wave][g][c4] = At[g];
                    if (c4 == 0) {
                        mg.m[g][wave] = Mt[g];
                        mg.l[g][wave] = Lt[g];
                    }
                }
            }
        }
        __syncthreads();
        // every wave entry scaled to the head's largest max M (the new
        // token's logit included), so each entry costs one exp2 and the
        // lanes' sums add plainly
        float M = s_nlg[og];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mg.m[og][w]);
        float L = 0.f;
        float4 A = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int w = k; w < kWaves; w += Q) {
            const float s = exp2_fast(mg.m[og][w] - M);   // 0 for a wave that holds no split
            const float4 a = mg.a[w][og][cc];
            L = fmaf(mg.l[og][w], s, L);
            A = make_float4(fmaf(a.x, s, A.x), fmaf(a.y, s, A.y), fmaf(a.z, s, A.z), fmaf(a.w, s, A.w));
        }
        L = lane_group_sum(L, Q);
        A = make_float4(lane_group_sum(A.x, Q), lane_group_sum(A.y, Q), lane_group_sum(A.z, Q),
                        lane_group_sum(A.w, Q));
        const float sn = exp2_fast(s_nlg[og] - M);
        const float4 vn = VQ ? *reinterpret_cast<const float4*>(&s_vdq[VQ ? 4 * cc : 0]) : load4_f32(s_vn + 4 * cc);
        L += sn;
        const float inv = 1.f / L;
        o = make_float4(fmaf(vn.x, sn, A.x) * inv, fmaf(vn.y, sn, A.y) * inv, fmaf(vn.z, sn, A.z) * inv,
                        fmaf(vn.w, sn, A.w) * inv);
    }
    if (dry) return;
    if (k == 0 && (tid >> qsh) < nout) reinterpret_cast<float4*>(out + (size_t)(hq0 + og) * D)[cc] = o;

    // a host tier keeps the token that leaves: its rows and position are
    // copied out before the overwrite below (the same thread reads and then
    // writes each element, so the rows need no barrier; the count does)
    if constexpr (!VQ) {
        if (c.tK != nullptr && full) {
            const int cnt = c.tcount[head];
            if (cnt < c.tcap) {
                const size_t dst = ((size_t)head * c.tcap + cnt) * D;
                for (int i = tid; i < D; i += kThreads) {
                    reinterpret_cast<KT*>(c.tK)[dst + i] = Kh[(size_t)e * D + i];
                    reinterpret_cast<KT*>(c.tV)[dst + i] = Vh[(size_t)e * D + i];
                }
                if (tid == 0) c.ttok[(size_t)head * c.tcap + cnt] = c.tok[rowbase + e];
            }
            __syncthreads();   // every thread has read the count before it moves
            if (tid == 0) c.tcount[head] = cnt + 1;
        }
    }
    // stage 5: the new token takes slot e
    for (int i = tid; i < D; i += kThreads) {
        Kh[(size_t)e * D + i] = s_kn[i];
        if constexpr (VQ == 8) {
            if (i < D / 2) reinterpret_cast<uint16_t*>(Vq + (size_t)e * VROW)[i] = s_vq2[i];
        } else if constexpr (VQ == 4) {
            if (i < D / 2) Vq[(size_t)e * VROW + i] = (uint8_t)s_vq2[i];
        } else {
            Vh[(size_t)e * D + i] = s_vn[i];
        }
    }
    if (VQ && tid == 0) Vsh[e] = s_vsc;
    if (tid == 0) {
        unsigned long long kc = 0;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) kc |= (unsigned long long)s_k16[nt] << (16 * nt);
        reinterpret_cast<CT*>(c.code)[(size_t)head * c.code_slots + e] = (CT)kc;
        c.tok[rowbase + e] = t;
        c.state[2 * head] = full ? n : n + 1;
        c.state[2 * head + 1] = t + 1;
        c.ekey[2 * head + (t & 1)] = 0ull;
        evicted[head] = e;
    }
}

// ---------------------------------------------------------------------------
// SPLIT schedule
// ---------------------------------------------------------------------------

// lsh_encode: 16 query heads or 16 new keys of sequence b per block.
template <int D, int BITS, typename KT>
__global__ __launch_bounds__(kThreads) void k_lsh_encode(DevCache c, const float* __restrict__ q,
                                                         const KT* __restrict__ knew)
{
    __shared__ uint32_t s16[BITS / 16][16];
    const int b = blockIdx.y;
    const int nqt = (c.Hq + 15) / 16;
    const int tile = blockIdx.x;
    const bool isq = tile < nqt;
    const int r0 = (isq ? tile : tile - nqt) * 16;
    const int nv = min(16, (isq ? c.Hq : c.Hkv) - r0);
    if (isq)
        encode_block16<D, BITS, float>(q + ((size_t)b * c.Hq + r0) * D, nv, c.R, s16);
    else
        encode_block16<D, BITS, KT>(knew + ((size_t)b * c.Hkv + r0) * D, nv, c.R, s16);
    __syncthreads();
    if ((int)threadIdx.x < nv) {
        uint32_t* dst = isq ? c.dbg_q + ((size_t)b * c.Hq + r0 + threadIdx.x) * c.W
                            : c.dbg_k + ((size_t)b * c.Hkv + r0 + threadIdx.x) * c.W;
        store_words(dst, c.W, join16<BITS>(s16, threadIdx.x));
    }
}

__device__ __forceinline__ unsigned long long load_code_words(const uint32_t* p, int W)
{
    unsigned long long v = p[0];
    if (W > 1) v |= (unsigned long long)p[1] << 32;
    return v;
}

// hamming_argmax: every block folds the best (score, lowest slot) of its
// kScoreChunk slots into the head's eviction key.
template <int BITS, int GM>
__global__ __launch_bounds__(kThreads) void k_hamming_argmax(DevCache c)
{
    using CT = typename CodeT<BITS>::T;
    constexpr int VS = 16 / sizeof(CT);
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int S = c.budget[b];
    const int head = b * c.Hkv + h;
    const int n = c.state[2 * head];
    if (n < S) return;                    // not full: nothing is evicted
    const int s0 = split * kScoreChunk;
    if (s0 >= n) return;
    const int s1 = min(s0 + kScoreChunk, n);
    const int G = c.G;
    __shared__ unsigned long long s_red[kWaves];
    CT qc[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g)
        qc[g] = g < G ? (CT)load_code_words(c.dbg_q + ((size_t)b * c.Hq + h * G + g) * c.W, c.W) : (CT)0;
    const CT* codeh = reinterpret_cast<const CT*>(c.code) + (size_t)head * c.code_slots;
    uint4 first[1] = {make_uint4(0, 0, 0, 0)};
    if (s0 + (int)threadIdx.x * VS < s1) first[0] = *reinterpret_cast<const uint4*>(codeh + s0 + threadIdx.x * VS);
    unsigned long long key = thread_candidate<BITS, GM, 1>(codeh, qc, G, s0, s1, first);
    key = block_max_u64(key, s_red);
    if (threadIdx.x == 0 && key) atomicMax(&c.ekey[2 * head], key);
}

// evict_write: the new token's K, V, code and position take the chosen slot.
template <int D, int BITS, typename KT>
__global__ void k_evict_write(DevCache c, const KT* __restrict__ knew, const KT* __restrict__ vnew,
                              int* __restrict__ evicted)
{
    using CT = typename CodeT<BITS>::T;
    const int h = blockIdx.x, b = blockIdx.y, head = b * c.Hkv + h;
    const int n = c.state[2 * head], t = c.state[2 * head + 1];
    const bool full = n >= c.budget[b];
    const int e = full ? cand_slot(c.ekey[2 * head]) : n;
    const size_t rowbase = (size_t)head * c.Smax;
    KT* Kh = reinterpret_cast<KT*>(c.K) + rowbase * D;
    KT* Vh = reinterpret_cast<KT*>(c.V) + rowbase * D;
    // the leaving token goes to the host tier first (same thread per element)
    if (c.tK != nullptr && full) {
        const int cnt = c.tcount[head];
        if (cnt < c.tcap) {
            const size_t dst = ((size_t)head * c.tcap + cnt) * D;
            for (int i = threadIdx.x; i < D; i += blockDim.x) {
                reinterpret_cast<KT*>(c.tK)[dst + i] = Kh[(size_t)e * D + i];
                reinterpret_cast<KT*>(c.tV)[dst + i] = Vh[(size_t)e * D + i];
            }
            if (threadIdx.x == 0) c.ttok[(size_t)head * c.tcap + cnt] = c.tok[rowbase + e];
        }
        __syncthreads();   // every thread has read the count before it moves
        if (threadIdx.x == 0) c.tcount[head] = cnt + 1;
    }
    for (int i = threadIdx.x; i < D; i += blockDim.x) {
        Kh[(size_t)e * D + i] = knew[(size_t)head * D + i];
        Vh[(size_t)e * D + i] = vnew[(size_t)head * D + i];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        reinterpret_cast<CT*>(c.code)[(size_t)head * c.code_slots + e] =
            (CT)load_code_words(c.dbg_k + (size_t)head * c.W, c.W);
        c.tok[rowbase + e] = t;
        c.state[2 * head] = full ? n : n + 1;
        c.state[2 * head + 1] = t + 1;
        c.ekey[2 * head] = 0ull;
        evicted[head] = e;
    }
}

// split-K attention: partial softmax of every chunk of the occupied slots.
template <int D, int GM, typename KT>
__global__ __launch_bounds__(kThreads) void k_attn_split(DevCache c, const float* __restrict__ q)
{
    constexpr bool kMfma = std::is_same<KT, bf16_t>::value;
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int head = b * c.Hkv + h;
    const int n = c.state[2 * head];
    const int nsb = max((n + c.chunk - 1) / c.chunk, 1);
    if (split >= nsb) return;
    __shared__ AttnSmem<D, GM> sm;
    __shared__ PSmem<GM, tile_rows<GM>()> ps;
    const int hq0 = b * c.Hq + h * c.G;
    const size_t rowbase = (size_t)head * c.Smax;
    const KT* Kh = reinterpret_cast<const KT*>(c.K) + rowbase * D;
    const KT* Vh = reinterpret_cast<const KT*>(c.V) + rowbase * D;
    const int s0 = split * c.chunk;
    const int len = max(min(s0 + c.chunk, n) - s0, 0);
    const int wave = threadIdx.x >> 6;
    if constexpr (kMfma) {
        constexpr int TR = tile_rows<GM>(), NB = ring_depth<GM, D, false>();
        MTile<D, TR> ring[NB];
        const int ntile = len > wave * TR ? (len - wave * TR + kWaves * TR - 1) / (kWaves * TR) : 0;
#pragma unroll
        for (int i = 0; i < NB; ++i)
            if (i < ntile) ring[i].load(Kh, Vh, nullptr, s0, len, (wave + i * kWaves) * TR);
        attend_rows_mfma<D, GM, TR, NB>(Kh, Vh, nullptr, q + (size_t)hq0 * D, c.G, s0, len, -1, ring, sm, ps, nullptr);
    } else {
        Tile<D, KT> first;
        first.load(Kh, Vh, s0, len, wave * Tile<D, KT>::ROWS);
        attend_rows<D, GM, KT>(Kh, Vh, q + (size_t)hq0 * D, c.G, s0, len, -1, first, sm, nullptr);
    }
    store_partial<D, GM>(sm, c.part, hq0, c.G, c.nsplit, split);
}

// LSE merge of the chunk partials of one query head into the output.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void k_attn_merge(DevCache c, float* __restrict__ out)
{
    const int hq = blockIdx.x, b = blockIdx.y;
    const int head = b * c.Hkv + hq / c.G;
    const int n = c.state[2 * head];
    const int nsb = max((n + c.chunk - 1) / c.chunk, 1);
    const size_t row = (size_t)b * c.Hq + hq;
    const float* part = c.part + row * c.nsplit * (D + 4);
    __shared__ MergeSmem<D> sm;
    auto rec = [&](int j) { return part + (size_t)j * (D + 4); };
    auto cand = [&](int, float& cl, const float*& cv) {
        cl = -INFINITY;
        cv = nullptr;
    };
    float4 o;
    if (merge_head<D>(sm, c.nsplit, nsb, rec, false, -1, cand, false, nullptr, make_float4(0.f, 0.f, 0.f, 0.f), o))
        reinterpret_cast<float4*>(out + row * D)[threadIdx.x] = o;
}

// Rows of one split of a head's host tier (at least 16, a multiple of 16).
__device__ __forceinline__ int tier_rows_per_split(int m, int tsplit)
{
    return (((m + tsplit - 1) / tsplit) + 15) & ~15;
}

// Split-K attention over the host tier: the stored entries of a head's tier
// are cut into c.tsplit splits and each block folds one into a partial
// (acc, m, l), like k_attn_split does over the cache.  The rows are read in
// place (pinned host memory over the host link, or device memory); every wave
// keeps its next tiles in flight while it computes on the current ones.
template <int D, int GM, typename KT>
__global__ __launch_bounds__(kThreads) void k_attn_tier(DevCache c, const float* __restrict__ q)
{
    constexpr bool kMfma = std::is_same<KT, bf16_t>::value;
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int head = b * c.Hkv + h;
    const int m = min(c.tcount[head], c.tcap);
    const int rps = tier_rows_per_split(m, c.tsplit);
    const int s0 = split * rps;
    if (s0 >= m) return;
    __shared__ AttnSmem<D, GM> sm;
    __shared__ PSmem<GM, tile_rows<GM>()> ps;
    const int hq0 = b * c.Hq + h * c.G;
    const size_t rowbase = (size_t)head * c.tcap;
    const KT* Kh = reinterpret_cast<const KT*>(c.tK) + rowbase * D;
    const KT* Vh = reinterpret_cast<const KT*>(c.tV) + rowbase * D;
    const int len = min(s0 + rps, m) - s0;
    const int wave = threadIdx.x >> 6;
    if constexpr (kMfma) {
        constexpr int TR = tile_rows<GM>(), NB = ring_depth<GM, D, false>();
        MTile<D, TR> ring[NB];
        const int ntile = len > wave * TR ? (len - wave * TR + kWaves * TR - 1) / (kWaves * TR) : 0;
#pragma unroll
        for (int i = 0; i < NB; ++i)
            if (i < ntile) ring[i].load(Kh, Vh, nullptr, s0, len, (wave + i * kWaves) * TR);
        attend_rows_mfma<D, GM, TR, NB>(Kh, Vh, nullptr, q + (size_t)hq0 * D, c.G, s0, len, -1, ring, sm, ps, nullptr);
    } else {
        Tile<D, KT> first;
        first.load(Kh, Vh, s0, len, wave * Tile<D, KT>::ROWS);
        attend_rows<D, GM, KT>(Kh, Vh, q + (size_t)hq0 * D, c.G, s0, len, -1, first, sm, nullptr);
    }
    store_partial<D, GM>(sm, c.tpart, hq0, c.G, c.tsplit, split);
}

// LSE merge of the cache's split partials and the tier's split partials of
// one query head into the output.
template <int D>
__global__ __launch_bounds__(kMergeThreads) void k_attn_merge_tiered(DevCache c, float* __restrict__ out)
{
    const int hq = blockIdx.x, b = blockIdx.y;
    const int head = b * c.Hkv + hq / c.G;
    const int n = c.state[2 * head];
    const int nsb = max((n + c.chunk - 1) / c.chunk, 1);
    const int m = min(c.tcount[head], c.tcap);
    const int rps = tier_rows_per_split(m, c.tsplit);
    const int nst = m > 0 ? (m + rps - 1) / rps : 0;
    const size_t row = (size_t)b * c.Hq + hq;
    const float* part = c.part + row * c.nsplit * (D + 4);
    const float* tpart = c.tpart + row * c.tsplit * (D + 4);
    __shared__ MergeSmem<D> sm;
    auto rec = [&](int j) { return j < nsb ? part + (size_t)j * (D + 4) : tpart + (size_t)(j - nsb) * (D + 4); };
    auto cand = [&](int, float& cl, const float*& cv) {
        cl = -INFINITY;
        cv = nullptr;
    };
    float4 o;
    if (merge_head<D>(sm, nsb + nst, nsb + nst, rec, false, -1, cand, false, nullptr,
                      make_float4(0.f, 0.f, 0.f, 0.f), o))
        reinterpret_cast<float4*>(out + row * D)[threadIdx.x] = o;
}

// GQA scores of every slot (introspection).
template <int BITS, int GM>
__global__ void k_scores(DevCache c, const uint32_t* __restrict__ qcodes, int* __restrict__ scores)
{
    using CT = typename CodeT<BITS>::T;
    const int h = blockIdx.y, b = blockIdx.z, head = b * c.Hkv + h;
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= c.Smax) return;
    const int n = c.state[2 * head];
    int sc = -1;
    if (s < n) {
        const CT cs = reinterpret_cast<const CT*>(c.code)[(size_t)head * c.code_slots + s];
        sc = 0;
        for (int g = 0; g < c.G; ++g)
            sc += popc((CT)(cs ^ (CT)load_code_words(qcodes + ((size_t)b * c.Hq + h * c.G + g) * c.W, c.W)));
    }
    scores[(size_t)head * c.Smax + s] = sc;
}

// stand-alone encoder: 16 rows per block
template <int D, int BITS, typename XT>
__global__ __launch_bounds__(kThreads) void k_encode_rows(DevCache c, const XT* __restrict__ X, int n,
                                                          uint32_t* __restrict__ codes)
{
    __shared__ uint32_t s16[BITS / 16][16];
    const int r0 = blockIdx.x * 16;
    const int nv = min(16, n - r0);
    encode_block16<D, BITS, XT>(X + (size_t)r0 * D, nv, c.R, s16);
    __syncthreads();
    if ((int)threadIdx.x < nv) store_words(codes + (size_t)(r0 + threadIdx.x) * c.W, c.W, join16<BITS>(s16, threadIdx.x));
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
template <typename F>
hipError_t with_kv(const DevCache& c, F&& f)
{
    if (c.kv_bf16) return f(bf16_t{});
    return f(float{});
}

template <typename F>
hipError_t with_d(const DevCache& c, F&& f)
{
    if (c.d == 64) return f(std::integral_constant<int, 64>{});
    return f(std::integral_constant<int, 128>{});
}

template <typename F>
hipError_t with_bits(const DevCache& c, F&& f)
{
    if (c.bits == 16) return f(std::integral_constant<int, 16>{});
    if (c.bits == 32) return f(std::integral_constant<int, 32>{});
    return f(std::integral_constant<int, 64>{});
}

template <typename F>
hipError_t with_gm(const DevCache& c, F&& f)
{
    if (c.G <= 1) return f(std::integral_constant<int, 1>{});
    if (c.G <= 2) return f(std::integral_constant<int, 2>{});
    if (c.G <= 4) return f(std::integral_constant<int, 4>{});
    if (c.G <= 8) return f(std::integral_constant<int, 8>{});
    return f(std::integral_constant<int, 16>{});
}

}  // namespace

static dim3 fused_grid(const DevCache& c)
{
    return c.ragged ? dim3(c.nblk * c.Hkv) : dim3(c.nsplit, c.Hkv, c.B);
}

hipError_t launch_decode_fused(const DevCache& c, const float* q, const void* k, const void* v, float* out,
                               int* evicted, hipStream_t st)
{
    return with_kv(c, [&](auto kt) {
        using KT = decltype(kt);
        return with_d(c, [&](auto dd) {
            return with_bits(c, [&](auto bb) {
                return with_gm(c, [&](auto gg) {
                    constexpr int D = decltype(dd)::value, BITS = decltype(bb)::value, GM = decltype(gg)::value;
                    if constexpr (std::is_same<KT, bf16_t>::value) {
                        if (c.vbits == 8) {
                            hipLaunchKernelGGL((k_decode_fused<D, BITS, GM, KT, 8>), fused_grid(c),
                                               dim3(kThreads), 0, st, c, q, (const KT*)k, (const KT*)v, out, evicted);
                            return hipGetLastError();
                        }
                        if (c.vbits == 4) {
                            hipLaunchKernelGGL((k_decode_fused<D, BITS, GM, KT, 4>), fused_grid(c),
                                               dim3(kThreads), 0, st, c, q, (const KT*)k, (const KT*)v, out, evicted);
                            return hipGetLastError();
                        }
                    }
                    hipLaunchKernelGGL((k_decode_fused<D, BITS, GM, KT>), fused_grid(c), dim3(kThreads),
                                       0, st, c, q, (const KT*)k, (const KT*)v, out, evicted);
                    return hipGetLastError();
                });
            });
        });
    });
}

hipError_t launch_attend_tiered(const DevCache& c, const float* q, float* out, hipStream_t st)
{
    return with_kv(c, [&](auto kt) {
        using KT = decltype(kt);
        return with_d(c, [&](auto dd) {
            constexpr int D = decltype(dd)::value;
            return with_gm(c, [&](auto gg) {
                constexpr int GM = decltype(gg)::value;
                hipLaunchKernelGGL((k_attn_split<D, GM, KT>), dim3(c.nsplit, c.Hkv, c.B), dim3(kThreads), 0, st, c, q);
                hipLaunchKernelGGL((k_attn_tier<D, GM, KT>), dim3(c.tsplit, c.Hkv, c.B), dim3(kThreads), 0, st, c, q);
                hipLaunchKernelGGL((k_attn_merge_tiered<D>), dim3(c.Hq, c.B), dim3(kMergeThreads), 0, st, c, out);
                return hipGetLastError();
            });
        });
    });
}

hipError_t launch_decode_split(const DevCache& c, const float* q, const void* k, const void* v, float* out,
                               int* evicted, hipStream_t st)
{
    return with_kv(c, [&](auto kt) {
        using KT = decltype(kt);
        return with_d(c, [&](auto dd) {
            return with_bits(c, [&](auto bb) {
                return with_gm(c, [&](auto gg) {
                    constexpr int D = decltype(dd)::value, BITS = decltype(bb)::value, GM = decltype(gg)::value;
                    const int ntiles = (c.Hq + 15) / 16 + (c.Hkv + 15) / 16;
                    hipLaunchKernelGGL((k_lsh_encode<D, BITS, KT>), dim3(ntiles, c.B), dim3(kThreads), 0, st, c, q,
                                       (const KT*)k);
                    const int nsh = (c.Smax + kScoreChunk - 1) / kScoreChunk;
                    hipLaunchKernelGGL((k_hamming_argmax<BITS, GM>), dim3(nsh, c.Hkv, c.B), dim3(kThreads), 0, st, c);
                    hipLaunchKernelGGL((k_evict_write<D, BITS, KT>), dim3(c.Hkv, c.B), dim3(128), 0, st, c,
                                       (const KT*)k, (const KT*)v, evicted);
                    hipLaunchKernelGGL((k_attn_split<D, GM, KT>), dim3(c.nsplit, c.Hkv, c.B), dim3(kThreads), 0, st, c,
                                       q);
                    hipLaunchKernelGGL((k_attn_merge<D>), dim3(c.Hq, c.B), dim3(kMergeThreads), 0, st, c, out);
                    return hipGetLastError();
                });
            });
        });
    });
}

hipError_t launch_scores(const DevCache& c, const uint32_t* qcodes, int* scores, hipStream_t st)
{
    return with_bits(c, [&](auto bb) {
        return with_gm(c, [&](auto gg) {
            dim3 grid((c.Smax + 255) / 256, c.Hkv, c.B);
            hipLaunchKernelGGL((k_scores<decltype(bb)::value, decltype(gg)::value>), grid, dim3(256), 0, st, c, qcodes,
                               scores);
            return hipGetLastError();
        });
    });
}

hipError_t launch_encode_rows(const DevCache& c, const void* X, int x_bf16, int n, uint32_t* codes, hipStream_t st)
{
    if (n <= 0) return hipSuccess;
    return with_d(c, [&](auto dd) {
        return with_bits(c, [&](auto bb) {
            constexpr int D = decltype(dd)::value, BITS = decltype(bb)::value;
            dim3 grid((n + 15) / 16);
            if (x_bf16)
                hipLaunchKernelGGL((k_encode_rows<D, BITS, bf16_t>), grid, dim3(kThreads), 0, st, c, (const bf16_t*)X,
                                   n, codes);
            else
                hipLaunchKernelGGL((k_encode_rows<D, BITS, float>), grid, dim3(kThreads), 0, st, c, (const float*)X, n,
                                   codes);
            return hipGetLastError();
        });
    });
}

}  // namespace hkv
