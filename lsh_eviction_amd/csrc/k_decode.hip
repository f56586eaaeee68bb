// k_decode.hip -- the decode step of the HashEvict path on gfx950.
//
// Method: HashEvict summary page ("HashEvict: A Pre-Attention KV Cache
// Eviction Strategy using Locality-Sensitive Hashing", arXiv 2412.16187),
// "Technical framework" stages 1-5 and the abstract: encode the query, score
// every cached key code by Hamming distance, evict the farthest slot before
// any attention is computed, write the new token there, attend.
//
// Two schedules of the same step:
//   FUSED (one launch).  Every block owns a chunk of slots of one (sequence,
//   KV head).  It encodes the group's queries, finds its chunk's candidate
//   (highest GQA score, lowest slot on ties), and accumulates softmax partials
//   over its chunk with that candidate held out.  The last block of the head
//   to finish picks the winner among the chunk candidates (the global argmax
//   with lowest-index ties is always its own chunk's candidate), adds back the
//   held-out candidates of the other chunks and the new token, merges by
//   log-sum-exp, and writes the new token into the winner's slot.  The result
//   equals "evict, write, then attend" with every K/V byte read once.
//   SPLIT (five launches): lsh_encode, hamming_argmax, evict_write, split-K
//   attention, merge.
#include <type_traits>

#include "hkv_consts.h"
#include "hkv_device.h"

namespace hkv {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

template <int D>
__device__ __forceinline__ float qscale2()
{
    // base-2 softmax: logits (q.k / sqrt(d)) * log2(e)
    return kLog2e * (D == 64 ? 0.125f : 0.08838834764831845f);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Shared memory of one attention block.
template <int D, int GM>
struct AttnSmem {
    float m[kWaves][GM];
    float l[kWaves][GM];
    float acc[kWaves][GM][D];
    float candlg[GM];
};

// Softmax partial of the G query heads of one KV head over rows [r0, r1) of
// Kh / Vh (row stride D), leaving out row `skip` (-1: none).  The base-2
// logits of the skipped row go to sm.candlg.  On return (after a block
// barrier) sm.m[0..3][g], sm.l, sm.acc hold one (max, sum, acc) per wave.
template <int D, int GM, typename KT>
__device__ __forceinline__ void attend_rows(const KT* __restrict__ Kh, const KT* __restrict__ Vh,
                                            const float* __restrict__ qh, int G, int r0, int r1,
                                            int skip, AttnSmem<D, GM>& sm)
{
    constexpr int EPL = Vec16<KT>::EPL;   // elements per 16-byte load
    constexpr int LPR = D / EPL;          // lanes per row
    constexpr int RPW = 64 / LPR;         // rows per wave load
    constexpr int UNR = 4;                // wave loads in flight per lane
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rg = lane / LPR, cc = lane % LPR;

    float qr[GM][EPL];
    const float qs = qscale2<D>();
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
        for (int e = 0; e < EPL; ++e) qr[g][e] = g < G ? qh[g * D + cc * EPL + e] * qs : 0.f;

    float m[GM], l[GM], acc[GM][EPL];
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
    }

    const int len = r1 - r0;
    for (int base = wave * UNR * RPW; base < len; base += kWaves * UNR * RPW) {
        uint4 kr[UNR], vr[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int row = base + u * RPW + rg;
            if (row < len) {
                const size_t off = (size_t)(r0 + row) * D + cc * EPL;
                kr[u] = *reinterpret_cast<const uint4*>(Kh + off);
                vr[u] = *reinterpret_cast<const uint4*>(Vh + off);
            } else {
                kr[u] = make_uint4(0, 0, 0, 0);
                vr[u] = make_uint4(0, 0, 0, 0);
            }
        }
        float lg[UNR][GM];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            float kf[EPL];
            Vec16<KT>::cvt(kr[u], kf);
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                float dot = 0.f;
#pragma unroll
                for (int e = 0; e < EPL; ++e) dot = fmaf(qr[g][e], kf[e], dot);
                lg[u][g] = group_sum<LPR>(dot);
            }
            const int row = base + u * RPW + rg;
            const bool isc = (r0 + row) == skip;
            if (isc && cc == 0) {
#pragma unroll
                for (int g = 0; g < GM; ++g) sm.candlg[g] = lg[u][g];
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
            Vec16<KT>::cvt(vr[u], vf);
#pragma unroll
            for (int g = 0; g < GM; ++g)
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p[u][g], vf[e], acc[g][e]);
        }
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

// Writes the block's partial for query heads g < G: part[(hq, split)] = acc[D], m, l.
template <int D, int GM>
__device__ __forceinline__ void store_partial(const AttnSmem<D, GM>& sm, float* __restrict__ part,
                                              int hq0, int G, int nsplit, int split)
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

// GQA Hamming scores of slots [s0, s1) against qc[0..G); returns the block's
// best candidate key (0 if the range is empty).  Uses red[kWaves].
template <int BITS, int GM>
__device__ __forceinline__ unsigned long long block_candidate(
    const typename CodeT<BITS>::T* __restrict__ code, const typename CodeT<BITS>::T (&qc)[GM], int G,
    int s0, int s1, unsigned long long* red)
{
    using CT = typename CodeT<BITS>::T;
    constexpr int VS = 16 / sizeof(CT);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    unsigned long long best = 0;
    for (int s = s0 + tid * VS; s < s1; s += kThreads * VS) {
        const uint4 raw = *reinterpret_cast<const uint4*>(code + s);
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
    }
    best = wave_max_u64(best);
    __syncthreads();
    if (lane == 0) red[wave] = best;
    __syncthreads();
    best = red[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) best = red[w] > best ? red[w] : best;
    return best;
}

// ---------------------------------------------------------------------------
// FUSED schedule
// ---------------------------------------------------------------------------
template <int D, int BITS, int GM, typename KT>
__global__ __launch_bounds__(kThreads) void k_decode_fused(DevCache c, const float* __restrict__ q,
                                                           const KT* __restrict__ knew,
                                                           const KT* __restrict__ vnew,
                                                           float* __restrict__ out,
                                                           int* __restrict__ evicted)
{
    using CT = typename CodeT<BITS>::T;
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int S = c.budget[b];
    const int nsb = (S + c.chunk - 1) / c.chunk;
    if (split >= nsb) return;
    const int G = c.G;
    const int head = b * c.Hkv + h;
    const int n = c.state[2 * head];
    const bool full = n >= S;
    const int s0 = split * c.chunk;
    const int s1 = min(s0 + c.chunk, n);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    __shared__ AttnSmem<D, GM> sm;
    __shared__ CT s_qc[GM];
    __shared__ CT s_kc;
    __shared__ unsigned long long s_red[kWaves];
    __shared__ float s_f[kWaves][GM];
    __shared__ float s_M[GM], s_L[GM], s_nlg[GM];
    __shared__ int s_last;

    const int hq0 = b * c.Hq + h * G;
    const float* qh = q + (size_t)hq0 * D;
    const size_t rowbase = (size_t)head * c.Smax;
    KT* Kh = reinterpret_cast<KT*>(c.K) + rowbase * D;
    KT* Vh = reinterpret_cast<KT*>(c.V) + rowbase * D;
    CT* codeh = reinterpret_cast<CT*>(c.code) + (size_t)head * c.code_slots;

    // stages 1-2: the group's query codes
    encode_rows<D, BITS>(qh, G, c.R, [&](int v, unsigned long long cd) { s_qc[v] = (CT)cd; });
    if (tid < GM) sm.candlg[tid] = -INFINITY;
    __syncthreads();
    if (split == 0 && tid < G) store_words(c.dbg_q + (size_t)(hq0 + tid) * c.W, c.W, s_qc[tid]);

    // stages 3-4 inside the chunk
    int cand = -1;
    unsigned long long ckey = 0;
    if (full) {
        CT qc[GM];
#pragma unroll
        for (int g = 0; g < GM; ++g) qc[g] = g < G ? s_qc[g] : (CT)0;
        ckey = block_candidate<BITS, GM>(codeh, qc, G, s0, s1, s_red);
        cand = ckey ? cand_slot(ckey) : -1;
    }

    // attention over the chunk with the candidate held out
    attend_rows<D, GM, KT>(Kh, Vh, qh, G, s0, max(s1, s0), cand, sm);
    store_partial<D, GM>(sm, c.part, hq0, G, c.nsplit, split);
    const size_t crec = (size_t)head * c.cstride + split;
    if (tid == 0) c.cand_key[crec] = ckey;
    if (tid < G) c.cand_lg[crec * G + tid] = sm.candlg[tid];

    // the last block of this head merges and writes
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&c.count[head], 1u) == (unsigned)(nsb - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (tid == 0) c.count[head] = 0;

    int e;
    if (full) {
        unsigned long long best = 0;
        for (int j = tid; j < nsb; j += kThreads) {
            const unsigned long long k = c.cand_key[(size_t)head * c.cstride + j];
            best = k > best ? k : best;
        }
        best = wave_max_u64(best);
        if (lane == 0) s_red[wave] = best;
        __syncthreads();
        best = s_red[0];
        for (int w = 1; w < kWaves; ++w) best = s_red[w] > best ? s_red[w] : best;
        e = cand_slot(best);
    } else {
        e = n;
    }
    const int js = full ? e / c.chunk : -1;

    // code of the new key; base-2 logits of the new token
    const KT* kh = knew + (size_t)head * D;
    const KT* vh = vnew + (size_t)head * D;
    encode_rows<D, BITS>(kh, 1, c.R, [&](int, unsigned long long cd) { s_kc = (CT)cd; });
    for (int g = wave; g < G; g += kWaves) {
        float dot = 0.f;
        for (int i = lane; i < D; i += 64) dot = fmaf(qh[g * D + i] * qscale2<D>(), to_f32(kh[i]), dot);
        dot = wave_sum_f(dot);
        if (lane == 0) s_nlg[g] = dot;
    }
    __syncthreads();

    // M[g] = max over chunk maxima, added-back candidates and the new token
    const float* part = c.part;
    const float* clg = c.cand_lg + (size_t)head * c.cstride * G;
    float mloc[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g) mloc[g] = -INFINITY;
    for (int j = tid; j < nsb; j += kThreads) {
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            if (g < G) {
                const float* rec = part + ((size_t)(hq0 + g) * c.nsplit + j) * (D + 4);
                if (rec[D + 1] > 0.f) mloc[g] = fmaxf(mloc[g], rec[D]);
                if (full && j != js) mloc[g] = fmaxf(mloc[g], clg[(size_t)j * G + g]);
            }
        }
    }
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        const float v = wave_max_f(mloc[g]);
        if (lane == 0) s_f[wave][g] = v;
    }
    __syncthreads();
    if (tid < G) {
        float mx = s_nlg[tid];
        for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, s_f[w][tid]);
        s_M[tid] = mx;
    }
    __syncthreads();
    float lloc[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g) lloc[g] = 0.f;
    for (int j = tid; j < nsb; j += kThreads) {
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            if (g < G) {
                const float* rec = part + ((size_t)(hq0 + g) * c.nsplit + j) * (D + 4);
                if (rec[D + 1] > 0.f) lloc[g] += rec[D + 1] * exp2_fast(rec[D] - s_M[g]);
                if (full && j != js) lloc[g] += exp2_fast(clg[(size_t)j * G + g] - s_M[g]);
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        const float v = wave_sum_f(lloc[g]);
        if (lane == 0) s_f[wave][g] = v;
    }
    __syncthreads();
    if (tid < G) {
        float ls = exp2_fast(s_nlg[tid] - s_M[tid]);
        for (int w = 0; w < kWaves; ++w) ls += s_f[w][tid];
        s_L[tid] = ls;
    }
    __syncthreads();

    for (int idx = tid; idx < G * D; idx += kThreads) {
        const int g = idx / D, i = idx % D;
        const float Mg = s_M[g];
        float a = 0.f;
        for (int j = 0; j < nsb; ++j) {
            const float* rec = part + ((size_t)(hq0 + g) * c.nsplit + j) * (D + 4);
            const float lj = rec[D + 1];
            if (lj > 0.f) a = fmaf(rec[i], exp2_fast(rec[D] - Mg), a);
            if (full && j != js) {
                const int cj = cand_slot(c.cand_key[(size_t)head * c.cstride + j]);
                a = fmaf(exp2_fast(clg[(size_t)j * G + g] - Mg), to_f32(Vh[(size_t)cj * D + i]), a);
            }
        }
        a = fmaf(exp2_fast(s_nlg[g] - Mg), to_f32(vh[i]), a);
        out[(size_t)(hq0 + g) * D + i] = a / s_L[g];
    }
    __syncthreads();

    // stage 5: the new token takes slot e
    for (int i = tid; i < D; i += kThreads) {
        Kh[(size_t)e * D + i] = kh[i];
        Vh[(size_t)e * D + i] = vh[i];
    }
    if (tid == 0) {
        const int t = c.state[2 * head + 1];
        codeh[e] = s_kc;
        c.tok[rowbase + e] = t;
        c.state[2 * head] = full ? n : n + 1;
        c.state[2 * head + 1] = t + 1;
        evicted[head] = e;
        store_words(c.dbg_k + (size_t)head * c.W, c.W, s_kc);
    }
}

// ---------------------------------------------------------------------------
// SPLIT schedule
// ---------------------------------------------------------------------------

// lsh_encode: codes of all query heads and new keys of sequence b.
template <int D, int BITS, typename KT>
__global__ __launch_bounds__(kThreads) void k_lsh_encode(DevCache c, const float* __restrict__ q,
                                                         const KT* __restrict__ knew)
{
    const int b = blockIdx.x;
    encode_rows<D, BITS>(q + (size_t)b * c.Hq * D, c.Hq, c.R, [&](int v, unsigned long long cd) {
        store_words(c.dbg_q + ((size_t)b * c.Hq + v) * c.W, c.W, cd);
    });
    encode_rows<D, BITS>(knew + (size_t)b * c.Hkv * D, c.Hkv, c.R, [&](int v, unsigned long long cd) {
        store_words(c.dbg_k + ((size_t)b * c.Hkv + v) * c.W, c.W, cd);
    });
}

__device__ __forceinline__ unsigned long long load_code_words(const uint32_t* p, int W)
{
    unsigned long long v = p[0];
    if (W > 1) v |= (unsigned long long)p[1] << 32;
    return v;
}

// hamming_argmax: block candidates over kScoreChunk slots, the last block of
// a head reduces them to the evicted slot.
template <int BITS, int GM>
__global__ __launch_bounds__(kThreads) void k_hamming_argmax(DevCache c, int* __restrict__ evicted)
{
    using CT = typename CodeT<BITS>::T;
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int S = c.budget[b];
    const int nsb = (S + kScoreChunk - 1) / kScoreChunk;
    if (split >= nsb) return;
    const int G = c.G, head = b * c.Hkv + h, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = c.state[2 * head];
    const bool full = n >= S;
    __shared__ unsigned long long s_red[kWaves];
    __shared__ int s_last;
    unsigned long long key = 0;
    if (full) {
        CT qc[GM];
#pragma unroll
        for (int g = 0; g < GM; ++g)
            qc[g] = g < G ? (CT)load_code_words(c.dbg_q + ((size_t)b * c.Hq + h * G + g) * c.W, c.W)
                          : (CT)0;
        const CT* codeh = reinterpret_cast<const CT*>(c.code) + (size_t)head * c.code_slots;
        const int s0 = split * kScoreChunk;
        key = block_candidate<BITS, GM>(codeh, qc, G, s0, min(s0 + kScoreChunk, n), s_red);
    }
    if (tid == 0) c.cand_key[(size_t)head * c.cstride + split] = key;
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = atomicAdd(&c.count[head], 1u) == (unsigned)(nsb - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    unsigned long long best = 0;
    for (int j = tid; j < nsb; j += kThreads) {
        const unsigned long long k = c.cand_key[(size_t)head * c.cstride + j];
        best = k > best ? k : best;
    }
    best = wave_max_u64(best);
    if (lane == 0) s_red[wave] = best;
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < kWaves; ++w) best = s_red[w] > best ? s_red[w] : best;
        best = s_red[0] > best ? s_red[0] : best;
        const int e = full ? cand_slot(best) : n;
        c.evict[head] = e;
        evicted[head] = e;
        c.count[head] = 0;
    }
}

// evict_write: the new token's K, V, code and position take the chosen slot.
template <int D, int BITS, typename KT>
__global__ void k_evict_write(DevCache c, const KT* __restrict__ knew, const KT* __restrict__ vnew)
{
    using CT = typename CodeT<BITS>::T;
    const int h = blockIdx.x, b = blockIdx.y, head = b * c.Hkv + h;
    const int e = c.evict[head];
    const size_t rowbase = (size_t)head * c.Smax;
    KT* Kh = reinterpret_cast<KT*>(c.K) + rowbase * D;
    KT* Vh = reinterpret_cast<KT*>(c.V) + rowbase * D;
    for (int i = threadIdx.x; i < D; i += blockDim.x) {
        Kh[(size_t)e * D + i] = knew[(size_t)head * D + i];
        Vh[(size_t)e * D + i] = vnew[(size_t)head * D + i];
    }
    if (threadIdx.x == 0) {
        const int n = c.state[2 * head], t = c.state[2 * head + 1];
        reinterpret_cast<CT*>(c.code)[(size_t)head * c.code_slots + e] =
            (CT)load_code_words(c.dbg_k + (size_t)head * c.W, c.W);
        c.tok[rowbase + e] = t;
        c.state[2 * head] = n < c.budget[b] ? n + 1 : n;
        c.state[2 * head + 1] = t + 1;
    }
}

// split-K attention: partial softmax of every chunk of the occupied slots.
template <int D, int GM, typename KT>
__global__ __launch_bounds__(kThreads) void k_attn_split(DevCache c, const float* __restrict__ q)
{
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int head = b * c.Hkv + h;
    const int n = c.state[2 * head];
    const int nsb = max((n + c.chunk - 1) / c.chunk, 1);
    if (split >= nsb) return;
    __shared__ AttnSmem<D, GM> sm;
    if (threadIdx.x < GM) sm.candlg[threadIdx.x] = -INFINITY;
    const int hq0 = b * c.Hq + h * c.G;
    const size_t rowbase = (size_t)head * c.Smax;
    const KT* Kh = reinterpret_cast<const KT*>(c.K) + rowbase * D;
    const KT* Vh = reinterpret_cast<const KT*>(c.V) + rowbase * D;
    const int s0 = split * c.chunk;
    attend_rows<D, GM, KT>(Kh, Vh, q + (size_t)hq0 * D, c.G, s0, max(min(s0 + c.chunk, n), s0), -1, sm);
    store_partial<D, GM>(sm, c.part, hq0, c.G, c.nsplit, split);
}

// LSE merge of the chunk partials into the output.
template <int D>
__global__ __launch_bounds__(kThreads) void k_attn_merge(DevCache c, float* __restrict__ out)
{
    const int hq = blockIdx.x, b = blockIdx.y;
    const int head = b * c.Hkv + hq / c.G;
    const int n = c.state[2 * head];
    const int nsb = max((n + c.chunk - 1) / c.chunk, 1);
    const size_t row = (size_t)b * c.Hq + hq;
    const float* part = c.part + row * c.nsplit * (D + 4);
    __shared__ float s_red[kWaves];
    __shared__ float s_M, s_L;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float mx = -INFINITY;
    for (int j = tid; j < nsb; j += kThreads)
        if (part[(size_t)j * (D + 4) + D + 1] > 0.f) mx = fmaxf(mx, part[(size_t)j * (D + 4) + D]);
    mx = wave_max_f(mx);
    if (lane == 0) s_red[wave] = mx;
    __syncthreads();
    if (tid == 0) {
        float v = s_red[0];
        for (int w = 1; w < kWaves; ++w) v = fmaxf(v, s_red[w]);
        s_M = v == -INFINITY ? 0.f : v;
    }
    __syncthreads();
    float ls = 0.f;
    for (int j = tid; j < nsb; j += kThreads) {
        const float* rec = part + (size_t)j * (D + 4);
        if (rec[D + 1] > 0.f) ls += rec[D + 1] * exp2_fast(rec[D] - s_M);
    }
    ls = wave_sum_f(ls);
    __syncthreads();
    if (lane == 0) s_red[wave] = ls;
    __syncthreads();
    if (tid == 0) {
        float v = 0.f;
        for (int w = 0; w < kWaves; ++w) v += s_red[w];
        s_L = v;
    }
    __syncthreads();
    for (int i = tid; i < D; i += kThreads) {
        float a = 0.f;
        for (int j = 0; j < nsb; ++j) {
            const float* rec = part + (size_t)j * (D + 4);
            if (rec[D + 1] > 0.f) a = fmaf(rec[i], exp2_fast(rec[D] - s_M), a);
        }
        out[row * D + i] = s_L > 0.f ? a / s_L : 0.f;
    }
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

template <int D, int BITS, typename XT>
__global__ __launch_bounds__(kThreads) void k_encode_rows(DevCache c, const XT* __restrict__ X, int n,
                                                          uint32_t* __restrict__ codes)
{
    constexpr int PER = 64;   // rows per block
    const int r0 = blockIdx.x * PER;
    encode_rows<D, BITS>(X + (size_t)r0 * D, min(PER, n - r0), c.R, [&](int v, unsigned long long cd) {
        store_words(codes + (size_t)(r0 + v) * c.W, c.W, cd);
    });
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

hipError_t launch_decode_fused(const DevCache& c, const float* q, const void* k, const void* v,
                               float* out, int* evicted, hipStream_t st)
{
    return with_kv(c, [&](auto kt) {
        using KT = decltype(kt);
        return with_d(c, [&](auto dd) {
            return with_bits(c, [&](auto bb) {
                return with_gm(c, [&](auto gg) {
                    dim3 grid(c.nsplit, c.Hkv, c.B);
                    hipLaunchKernelGGL((k_decode_fused<decltype(dd)::value, decltype(bb)::value, decltype(gg)::value, KT>), grid,
                                       dim3(kThreads), 0, st, c, q, (const KT*)k, (const KT*)v, out,
                                       evicted);
                    return hipGetLastError();
                });
            });
        });
    });
}

hipError_t launch_decode_split(const DevCache& c, const float* q, const void* k, const void* v,
                               float* out, int* evicted, hipStream_t st)
{
    return with_kv(c, [&](auto kt) {
        using KT = decltype(kt);
        return with_d(c, [&](auto dd) {
            return with_bits(c, [&](auto bb) {
                return with_gm(c, [&](auto gg) {
                    constexpr int D = decltype(dd)::value, BITS = decltype(bb)::value, GM = decltype(gg)::value;
                    hipLaunchKernelGGL((k_lsh_encode<D, BITS, KT>), dim3(c.B), dim3(kThreads), 0, st, c,
                                       q, (const KT*)k);
                    const int nsh = (c.Smax + kScoreChunk - 1) / kScoreChunk;
                    hipLaunchKernelGGL((k_hamming_argmax<BITS, GM>), dim3(nsh, c.Hkv, c.B),
                                       dim3(kThreads), 0, st, c, evicted);
                    hipLaunchKernelGGL((k_evict_write<D, BITS, KT>), dim3(c.Hkv, c.B), dim3(128), 0, st,
                                       c, (const KT*)k, (const KT*)v);
                    hipLaunchKernelGGL((k_attn_split<D, GM, KT>), dim3(c.nsplit, c.Hkv, c.B),
                                       dim3(kThreads), 0, st, c, q);
                    hipLaunchKernelGGL((k_attn_merge<D>), dim3(c.Hq, c.B), dim3(kThreads), 0, st, c,
                                       out);
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
            hipLaunchKernelGGL((k_scores<decltype(bb)::value, decltype(gg)::value>), grid, dim3(256), 0, st, c, qcodes, scores);
            return hipGetLastError();
        });
    });
}

hipError_t launch_encode_rows(const DevCache& c, const void* X, int x_bf16, int n, uint32_t* codes,
                              hipStream_t st)
{
    if (n <= 0) return hipSuccess;
    return with_d(c, [&](auto dd) {
        return with_bits(c, [&](auto bb) {
            dim3 grid((n + 63) / 64);
            if (x_bf16)
                hipLaunchKernelGGL((k_encode_rows<decltype(dd)::value, decltype(bb)::value, bf16_t>), grid, dim3(kThreads), 0,
                                   st, c, (const bf16_t*)X, n, codes);
            else
                hipLaunchKernelGGL((k_encode_rows<decltype(dd)::value, decltype(bb)::value, float>), grid, dim3(kThreads), 0, st,
                                   c, (const float*)X, n, codes);
            return hipGetLastError();
        });
    });
}

}  // namespace hkv
