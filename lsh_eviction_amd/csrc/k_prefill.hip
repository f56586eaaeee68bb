// k_prefill.hip -- prompt code build and prefill selection on gfx950.
//
// Method stages 1-2 (HashEvict summary page, "Technical framework"): every
// prompt key is projected through the Gaussian matrix R and sign-binarised.
// Projecting N keys is a dense N x d x b contraction, so it runs on the
// matrix cores (fp32 MFMA 16x16x4: fp32 semantics, so the signs agree with an
// fp64 reference outside the flagged band).
//
// bf16 keys take a second form of the same contraction on the bf16 matrix
// cores: R is split by truncation into three bf16 parts, hi + mid + lo == R
// exactly (the bf16x3 scheme of Henry, Tang and Heinecke, "Leveraging the
// bfloat16 artificial intelligence datatype for higher-precision
// computations", 2019), and each bf16 x bf16 product is exact in fp32, so
// only the fp32 summation order differs from the fp32 kernel.
//
// Prefill rule (the page does not describe prefill; reading used here): with
// the STREAM policy the prompt enters the cache one token at a time by the
// decode rule, each token scored against its own key code; TRUNCATE keeps
// the first `budget` tokens.  The sequential selection keeps the whole code
// table of one (sequence, KV head) in the registers of one workgroup.
//
// Chunk-granular prefill (a reading of the ChunkKV summary page: tokens kept
// or dropped in groups of consecutive tokens, kept indices reusable across
// layers): the prompt is cut into chunks of C tokens, every chunk is scored
// by its summed Hamming distance to the observation query codes, and the
// chunks are evicted in order of (score descending, index ascending) until
// floor(S / C) remain.  Scores are computed one thread per chunk over the
// whole grid; a histogram of their values gives the threshold, and one block
// per (sequence, KV head) places the kept chunks.
#include <type_traits>

#include "hkv.h"
#include "hkv_consts.h"
#include "hkv_device.h"

namespace hkv {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// slot -> token map and per-head state before a prefill
__global__ void k_prefill_init(DevCache c)
{
    const int h = blockIdx.y, b = blockIdx.z, head = b * c.Hkv + h;
    const int N = c.plen[b], S = c.budget[b];
    const int occ = min(N, S);
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s < c.Smax) c.tok[(size_t)head * c.Smax + s] = s < occ ? s : -1;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        c.state[2 * head] = occ;
        c.state[2 * head + 1] = N;
        c.ekey[2 * head] = 0ull;
        c.ekey[2 * head + 1] = 0ull;
        c.count[head * kCountStride] = 0u;
    }
}

// reset of an empty cache (create)
__global__ void k_reset(DevCache c)
{
    const int h = blockIdx.y, b = blockIdx.z, head = b * c.Hkv + h;
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s < c.Smax) c.tok[(size_t)head * c.Smax + s] = -1;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        c.state[2 * head] = 0;
        c.state[2 * head + 1] = 0;
        c.ekey[2 * head] = 0ull;
        c.ekey[2 * head + 1] = 0ull;
        c.count[head * kCountStride] = 0u;
    }
}

// Codes of prompt rows of one head on the matrix cores: X is
// [B][nh][n_max][D] (prompt keys with nh = Hkv, prompt queries with nh = Hq),
// codes go to dst[(b * nh + h) * pcode_slots + t].  A block stages R in LDS
// once and then takes the 64-row tiles blockIdx.x, blockIdx.x + gridDim.x,
// ... of its head.  Wave w takes 16 rows of a tile; lane l feeds row (l % 16)
// and the quarter (l / 16) of the head dimension: MFMA step s of the two
// accumulators contracts dimensions (l / 16) * D/4 + s and + s + D/8.  The
// 16 x 16 result tile of bit columns nt*16 .. +15 is sign-packed by a wave
// ballot per accumulator register.
constexpr int kProjMaxBlocks = 256;   // blocks per head of the projection grid

// Element s of a lane's row quarter held as raw 16-byte words.
template <typename KT, int NV>
__device__ __forceinline__ float raw_elem(const uint4 (&r)[NV], int s)
{
    constexpr int EPL = Vec16<KT>::EPL;
    const uint4 q = r[s / EPL];
    const int e = s % EPL;
    if constexpr (std::is_same<KT, bf16_t>::value) {
        const uint32_t w = (e >> 1) == 0 ? q.x : (e >> 1) == 1 ? q.y : (e >> 1) == 2 ? q.z : q.w;
        return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
    } else {
        return __uint_as_float(e == 0 ? q.x : e == 1 ? q.y : e == 2 ? q.z : q.w);
    }
}

template <int D, int BITS, typename KT>
__global__ __launch_bounds__(256) void k_project_mfma(DevCache c, const KT* __restrict__ Kp, int n_max, int nh,
                                                      void* __restrict__ dst)
{
    using CT = typename CodeT<BITS>::T;
    constexpr int DQ = D / 4;                    // dimensions fed by one lane
    constexpr int NT = BITS / 16;                // bit tiles
    constexpr int NV = DQ / Vec16<KT>::EPL;      // 16-byte words per lane and row
    // R in LDS with the rows of quarter q of the head dimension shifted by
    // 16 q floats: the four lane groups of an operand read then fall on
    // different banks
    __shared__ __align__(16) float sR[D * BITS + 64];
    const int h = blockIdx.y, b = blockIdx.z, head = b * nh + h;
    const int N = c.plen[b];
    if (blockIdx.x * 64 >= N) return;
    {
        // every load of R is issued before any is waited for
        constexpr int NR4 = D * BITS / 4, RPT = (NR4 + 255) / 256;
        float4 rr[RPT];
#pragma unroll
        for (int j = 0; j < RPT; ++j)
            rr[j] = reinterpret_cast<const float4*>(c.R)[min((int)threadIdx.x + j * 256, NR4 - 1)];
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int i = 4 * ((int)threadIdx.x + j * 256);
            if (i < D * BITS) *reinterpret_cast<float4*>(sR + i + (i / (DQ * BITS)) * 16) = rr[j];
        }
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int qd = lane >> 4;
    const int stride = gridDim.x * 64;

    // the raw words of a tile's rows; the next tile's are in flight while
    // the current one is computed
    auto load_tile = [&](int t0, uint4 (&r)[NV]) {
        const int row = t0 + wave * 16 + (lane & 15);
        if (row < N) {
            const uint4* src = reinterpret_cast<const uint4*>(Kp + ((size_t)head * n_max + row) * D + qd * DQ);
#pragma unroll
            for (int v = 0; v < NV; ++v) r[v] = src[v];
        } else {
#pragma unroll
            for (int v = 0; v < NV; ++v) r[v] = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    uint4 cur[NV], nxt[NV];
    load_tile(blockIdx.x * 64, cur);
    for (int t0 = blockIdx.x * 64; t0 < N; t0 += stride) {
        if (t0 + stride < N) load_tile(t0 + stride, nxt);

        // two accumulators per bit tile (the two halves of the lane's
        // dimensions), so twice as many independent MFMA chains are in
        // flight; any fp32 summation order gives the same unflagged bits
        unsigned long long mk[NT][4];
        f32x4 acc[NT][2];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt][0] = acc[nt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < DQ / 2; ++s) {
            const float x0 = raw_elem<KT>(cur, s), x1 = raw_elem<KT>(cur, s + DQ / 2);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float* rcol = sR + (size_t)(qd * DQ) * BITS + qd * 16 + nt * 16 + (lane & 15);
                acc[nt][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(x0, rcol[s * BITS], acc[nt][0], 0, 0, 0);
                acc[nt][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(x1, rcol[(s + DQ / 2) * BITS], acc[nt][1], 0, 0, 0);
            }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const f32x4 y = acc[nt][0] + acc[nt][1];
#pragma unroll
            for (int r = 0; r < 4; ++r) mk[nt][r] = __ballot(y[r] > 0.f);
        }
        // result row i = 4 * (lane / 16) + r sits in register r of lanes 16 * (i / 4) + col
        if (lane < 16) {
            const int a = lane >> 2, r = lane & 3;
            unsigned long long cde = 0;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                // the lane's ballot by masks (a select chain over the four
                // became a private array indexed at run time, i.e. scratch)
                unsigned long long m = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) m |= mk[nt][q] & (0ull - (unsigned long long)(r == q));
                cde |= ((m >> (16 * a)) & 0xFFFFull) << (16 * nt);
            }
            const int t = t0 + wave * 16 + lane;
            if (t < N) reinterpret_cast<CT*>(dst)[(size_t)head * c.pcode_slots + t] = (CT)cde;
        }
#pragma unroll
        for (int v = 0; v < NV; ++v) cur[v] = nxt[v];
    }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Codes of bf16 prompt rows on the bf16 matrix cores (MFMA 16x16x32): X is
// [B][nh][n_max][D] bf16, codes go to dst[(b * nh + h) * pcode_slots + t].
// R is split into bf16 parts hi + mid + lo == R (truncation: hi keeps the
// top 8 significant bits of R, mid the top 8 of R - hi, lo the rest, at
// most 8 bits), so x * part is exact in fp32.  The hi products and the
// mid + lo products go to separate accumulators: the first carries the
// rounding of an fp32 dot product of length D, the second is below 2^-7 of
// the projection's magnitude, so the result stays within the error of an
// fp32 dot product in any summation order, and its signs agree with an
// exact projection outside the flagged band.
//
// The work is a stream of key rows, so the kernel is built to keep memory
// busy: a persistent grid of as many blocks as the compute units hold, each
// wave holding all of R's parts in registers and a ring of NB tiles in
// flight.  Block k takes a contiguous run of the 64-row tiles of all heads
// (tiles_per_head per head); wave w takes rows 16 w .. 16 w + 15 of a tile.
// Lane l feeds row l % 16 and dimensions 32 s + 8 (l / 16) .. + 7 of MFMA
// step s, and holds the same dimensions of R's column (tile * 16 + l % 16).
// Rows past the prompt (and tiles past the last) read as zero through the
// buffer resource, so every load is issued and the ring's waits are exact.
template <int D, int BITS>
__global__ __launch_bounds__(256, 1) void k_project_bf16x3(DevCache c, const bf16_t* __restrict__ Kp, int n_max,
                                                           int nh, int tiles_per_head, int total_tiles,
                                                           void* __restrict__ dst)
{
    using CT = typename CodeT<BITS>::T;
    constexpr int NT = BITS / 16;            // bit tiles
    constexpr int KS = D / 32;               // MFMA steps over the head dimension
    constexpr int NB = BITS > 32 ? 4 : 6;    // tiles in flight per wave (register budget)
    constexpr int LDR = D + 8;               // R^T row in LDS, padded by 16 bytes
    constexpr int NR4 = D * BITS / 4, RPT = NR4 / 256;
    static_assert(NR4 % 256 == 0 && BITS % 4 == 0, "R staging shape");
    __shared__ __align__(16) uint16_t sRT[3][BITS][LDR];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int qd = lane >> 4, col = lane & 15;
    const int lane_off = (wave * 16 + col) * (D * 2) + qd * 16;   // byte offset in a tile

    // block k takes the contiguous tiles [t_begin, t_end) of the stream of
    // all heads' tiles, so each block reads one run of memory
    const int t_begin = (int)((long long)total_tiles * blockIdx.x / gridDim.x);
    const int t_end = (int)((long long)total_tiles * (blockIdx.x + 1) / gridDim.x);
    auto issue = [&](int tau, uint4 (&r)[KS]) {
        const bf16_t* base = Kp;
        int bytes = 0;
        if (tau < t_end) {
            const int head = tau / tiles_per_head, t0 = (tau - head * tiles_per_head) * 64;
            base = Kp + ((size_t)head * n_max + t0) * D;
            bytes = max(min(c.plen[head / nh] - t0, 64), 0) * D * 2;
        }
        // uniform, but computed by a vector instruction (v_med3): kept in a
        // scalar register so the resource is scalar and no load is waterfalled
        bytes = __builtin_amdgcn_readfirstlane(bytes);
        const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(base), 0, bytes, kRsrcWord3);
#pragma unroll
        for (int s = 0; s < KS; ++s)
            r[s] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, lane_off + 64 * s, 0, 0));
    };
    // R is requested first (waits are in order of issue: a wait for R issued
    // after the ring would drain the ring), then the first tiles, which are
    // in flight while R is split
    float4 rr[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) rr[j] = reinterpret_cast<const float4*>(c.R)[threadIdx.x + j * 256];
    uint4 ring[NB][KS];
#pragma unroll
    for (int k = 0; k < NB; ++k) issue(t_begin + k, ring[k]);
    {
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int i = 4 * ((int)threadIdx.x + j * 256), dim = i / BITS, bit0 = i % BITS;
            const float v[4] = {rr[j].x, rr[j].y, rr[j].z, rr[j].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t hb = __float_as_uint(v[e]) & 0xFFFF0000u;
                const float r1 = v[e] - __uint_as_float(hb);   // exact: the low 16 bits
                const uint32_t mb = __float_as_uint(r1) & 0xFFFF0000u;
                const float r2 = r1 - __uint_as_float(mb);     // exact, at most 8 significant bits
                sRT[0][bit0 + e][dim] = (uint16_t)(hb >> 16);
                sRT[1][bit0 + e][dim] = (uint16_t)(mb >> 16);
                sRT[2][bit0 + e][dim] = (uint16_t)(__float_as_uint(r2) >> 16);
            }
        }
    }
    __syncthreads();
    bf16x8 Rf[NT][KS][3];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int p = 0; p < 3; ++p)
                Rf[nt][s][p] = *reinterpret_cast<const bf16x8*>(&sRT[p][nt * 16 + col][32 * s + 8 * qd]);

    // Whole rounds of the ring: the block's tile count is rounded up to a
    // multiple of NB, and the tiles past the last read nothing (a resource
    // of size 0) and store nothing.  No exit inside a round: with one, the
    // compiler sinks each prefetch down to its use and the ring is lost.
    for (int i0 = t_begin; i0 < t_end; i0 += NB) {
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int tau = i0 + k;
            const bool valid = tau < t_end;
            const int head = valid ? tau / tiles_per_head : 0;
            const int t0 = valid ? (tau - head * tiles_per_head) * 64 : 0;
            const int N = valid ? c.plen[head / nh] : 0;
            f32x4 ah[NT], am[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) ah[nt] = am[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, ring[k][s]);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    ah[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, Rf[nt][s][0], ah[nt], 0, 0, 0);
                    am[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, Rf[nt][s][1], am[nt], 0, 0, 0);
                    am[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, Rf[nt][s][2], am[nt], 0, 0, 0);
                }
            }
            // the ring slot is free once the products have read it
            issue(tau + NB, ring[k]);
            unsigned long long mk[NT][4];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const f32x4 y = ah[nt] + am[nt];
#pragma unroll
                for (int r = 0; r < 4; ++r) mk[nt][r] = __ballot(y[r] > 0.f);
            }
            // result row i = 4 * (lane / 16) + r sits in register r of lanes 16 * (i / 4) + col
            if (lane < 16) {
                const int a = lane >> 2, r = lane & 3;
                unsigned long long cde = 0;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    unsigned long long m = 0;
#pragma unroll
                    for (int q = 0; q < 4; ++q) m |= mk[nt][q] & (0ull - (unsigned long long)(r == q));
                    cde |= ((m >> (16 * a)) & 0xFFFFull) << (16 * nt);
                }
                const int t = t0 + wave * 16 + lane;
                if (t < N) reinterpret_cast<CT*>(dst)[(size_t)head * c.pcode_slots + t] = (CT)cde;
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);   // the last round's prefetches (of nothing) land before the wave ends
}

// Resident workgroups of a 256-thread kernel on the current device (every
// compute unit times the blocks one holds), the size of a persistent grid.
static int resident_blocks(const void* kernel)
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 256;
    }
    return cus * (per_cu > 0 ? per_cu : 1);
}

// Blocks per head of the fp32 projection of n_max rows.
static int proj_blocks(int n_max)
{
    const int tiles = (n_max + 63) / 64;
    return tiles < kProjMaxBlocks ? tiles : kProjMaxBlocks;
}

// Prompt key codes: bf16 keys on the bf16 matrix cores (bf16x3), fp32 keys
// on the fp32 ones.
template <int D, int BITS, typename KT>
hipError_t launch_project_keys(const DevCache& c, const void* K, int n_max, hipStream_t st)
{
    if constexpr (std::is_same<KT, bf16_t>::value) {
        const int per_head = (n_max + 63) / 64;
        const long long total = (long long)per_head * c.B * c.Hkv;
        if (total <= 0) return hipSuccess;
        if (total > INT32_MAX) return hipErrorInvalidValue;
        static const int resident = resident_blocks((const void*)k_project_bf16x3<D, BITS>);
        const int grid = total < resident ? (int)total : resident;
        hipLaunchKernelGGL((k_project_bf16x3<D, BITS>), dim3(grid), dim3(256), 0, st, c, (const bf16_t*)K, n_max,
                           c.Hkv, per_head, (int)total, c.pcode);
    } else {
        hipLaunchKernelGGL((k_project_mfma<D, BITS, KT>), dim3(proj_blocks(n_max), c.Hkv, c.B), dim3(256), 0, st,
                           c, (const KT*)K, n_max, c.Hkv, c.pcode);
    }
    return hipGetLastError();
}

template <int CTRL>
__device__ __forceinline__ unsigned dpp_u(unsigned x)
{
    return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

// Maximum over the wave (all 64 lanes active), returned wave-uniform: DPP
// steps within each 16-lane row, then the four row maxima by readlane (no
// LDS traffic).
__device__ __forceinline__ unsigned wave_max_u32(unsigned v)
{
    v = max(v, dpp_u<kDppXor1>(v));
    v = max(v, dpp_u<kDppXor2>(v));
    v = max(v, dpp_u<kDppHalfMirror>(v));
    v = max(v, dpp_u<kDppMirror>(v));
    const unsigned a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
    const unsigned c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
    return max(max(a, b), max(c, d));
}

// Sequential prefill selection for one (sequence, KV head): prompt tokens
// t >= S, one after the other, evict the occupied slot farthest in summed
// Hamming distance from their query codes -- their own key code under
// STREAM, the codes of their G query rows under QUERY -- ties to the lowest
// slot, and take it.  The code table lives in registers: thread tid holds
// the 16-byte groups k * 1024 + tid (VS codes each) in treg[k], so a scan
// reads no memory; a window of the coming tokens' codes is staged in LDS.
// One barrier per token: the waves' (score, slot) maxima are double-buffered,
// every wave reduces them to the same winner, and the thread holding the
// winning slot updates its register copy (it is the entry's only reader).
constexpr int kSelTokens = 128;   // tokens whose codes are staged at a time
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
constexpr int kTableRegs = 8;     // 16-byte groups of the table per thread: 1024 x 8 x 16 B = 128 KiB

template <int BITS>
constexpr size_t select_lds_bytes(int, int nq)
{
    return (size_t)kSelTokens * (1 + nq) * (BITS / 8);
}

// GQ = 0: STREAM (the token's key code); GQ > 0: QUERY with G <= GQ query
// codes per token (GQ a power of two, so a group of G costs G popcounts).
template <int BITS, int GQ>
__global__ __launch_bounds__(1024) void k_prefill_select(DevCache c)
{
    using CT = typename CodeT<BITS>::T;
    constexpr int VS = 16 / sizeof(CT);
    constexpr int SLOT_BITS = 17;   // slot field of the 32-bit (score, slot) key
    constexpr unsigned SLOT_MASK = (1u << SLOT_BITS) - 1u;
    extern __shared__ uint4 dyn_lds[];
    __shared__ unsigned s_red[2][16];
    const int h = blockIdx.x, b = blockIdx.y, head = b * c.Hkv + h;
    const int N = c.plen[b], S = c.budget[b];
    if (N <= S) return;
    const int G = c.G;
    CT* skey = reinterpret_cast<CT*>(dyn_lds);   // [kSelTokens] key codes of the window
    CT* sq = skey + kSelTokens;                   // [kSelTokens][G] query codes of the window (QUERY)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const CT* pc = reinterpret_cast<const CT*>(c.pcode) + (size_t)head * c.pcode_slots;
    constexpr bool QRY = GQ > 0;
    const CT* qc = QRY ? reinterpret_cast<const CT*>(c.qcode) + (size_t)(b * c.Hq + h * G) * c.pcode_slots : nullptr;
    int* tok = c.tok + (size_t)head * c.Smax;
    // the table: group k of this thread holds slots (k * 1024 + tid) * VS + u
    uint4 treg[kTableRegs];
#pragma unroll
    for (int k = 0; k < kTableRegs; ++k) {
        const int s = (k * 1024 + tid) * VS;
        treg[k] = s < S ? *reinterpret_cast<const uint4*>(pc + s) : make_uint4(0u, 0u, 0u, 0u);
    }
    const int nfull = S / (VS * 1024);                        // groups with every slot occupied, uniform
    const bool partial = S % (VS * 1024) != 0;                // one more group, partly occupied
    // key of slot s: (score << SLOT_BITS) | (SLOT_MASK - s) = (score << SLOT_BITS) + cbase - (k * 1024 * VS + u)
    const unsigned cbase = SLOT_MASK - (unsigned)(tid * VS);
    // 16-bit keys of the full groups: local index k * VS + u in LB bits; the
    // score (at most GQ' * BITS, 1024) shifted by LB stays below 2^15
    constexpr int LB = VS == 8 ? 6 : (VS == 4 ? 5 : 4);
    constexpr unsigned LMAX = (1u << LB) - 1u;
    static_assert(kTableRegs * VS == (1 << LB) && ((16u * BITS) << LB) < 65536u, "16-bit slot keys");
    int par = 0;
    for (int t0 = S; t0 < N; t0 += kSelTokens) {
        const int cnt = min(kSelTokens, N - t0);
        __syncthreads();   // the previous window has been consumed
        for (int i = tid; i < cnt; i += blockDim.x) skey[i] = pc[t0 + i];
        if constexpr (QRY) {
            for (int i = tid; i < cnt * G; i += blockDim.x) {
                const int j = i / G, g = i - j * G;
                sq[i] = qc[(size_t)g * c.pcode_slots + t0 + j];
            }
        }
        __syncthreads();
        for (int j = 0; j < cnt; ++j) {
            CT qv[QRY ? GQ : 1];
            if constexpr (QRY) {
#pragma unroll
                for (int g = 0; g < GQ; ++g) qv[g] = g < G ? sq[j * G + g] : (CT)0;
            } else {
                qv[0] = skey[j];
            }
            auto score = [&](CT code) {
                int sc = 0;
                if constexpr (QRY) {
#pragma unroll
                    for (int g = 0; g < GQ; ++g)
                        if (g < G) sc += popc((CT)(qv[g] ^ code));
                } else {
                    sc = popc((CT)(qv[0] ^ code));
                }
                return (unsigned)sc;
            };
            // Full groups: a 16-bit key per slot, (score << LB) | (last local
            // index - local index), two slots per packed max; the largest key
            // is the largest score at the lowest local (hence global) slot.
            u16x2 best2 = {0, 0};
#pragma unroll
            for (int k = 0; k < kTableRegs; ++k) {
                CT cs[VS];
                __builtin_memcpy(cs, &treg[k], 16);
                if (k < nfull) {
#pragma unroll
                    for (int u = 0; u < VS; u += 2) {
                        const unsigned li = (unsigned)(k * VS + u);
                        const u16x2 kk = {(unsigned short)((score(cs[u]) << LB) | (LMAX - li)),
                                          (unsigned short)((score(cs[u + 1]) << LB) | (LMAX - li - 1))};
                        best2 = __builtin_elementwise_max(best2, kk);
                    }
                }
            }
            unsigned best = 0;
            if (nfull > 0) {
                const unsigned k16 = max((unsigned)best2.x, (unsigned)best2.y);
                const unsigned li = LMAX - (k16 & LMAX);
                const unsigned slot = (li / VS) * (1024u * VS) + (unsigned)(tid * VS) + li % VS;
                best = ((k16 >> LB) << SLOT_BITS) | (SLOT_MASK - slot);
            }
#pragma unroll
            for (int k = 0; k < kTableRegs; ++k) {
                CT cs[VS];
                __builtin_memcpy(cs, &treg[k], 16);
                if (k == nfull && partial) {
                    const int s0 = (k * 1024 + tid) * VS;
#pragma unroll
                    for (int u = 0; u < VS; ++u)
                        if (s0 + u < S)
                            best = max(best, (score(cs[u]) << SLOT_BITS) + (cbase - (unsigned)(k * 1024 * VS + u)));
                }
            }
            best = wave_max_u32(best);
            if (lane == 0) s_red[par][wave] = best;
            __syncthreads();
            unsigned v = lane < 16 ? s_red[par][lane] : 0u;
            v = wave_max_u32(v);
            const int e = (int)(SLOT_MASK - (v & SLOT_MASK));
            if (tid == (e / VS) % 1024) {
                const int ke = e / (VS * 1024), ue = e % VS;
                const CT code = skey[j];
#pragma unroll
                for (int k = 0; k < kTableRegs; ++k) {
                    if (k == ke) {
                        CT cs[VS];
                        __builtin_memcpy(cs, &treg[k], 16);
#pragma unroll
                        for (int u = 0; u < VS; ++u)
                            if (u == ue) cs[u] = code;
                        __builtin_memcpy(&treg[k], cs, 16);
                    }
                }
                tok[e] = t0 + j;
            }
            par ^= 1;
        }
    }
}

// K, V and codes of the kept tokens into their slots; 16 lanes per row.
template <int D, int BITS, typename KT>
__global__ __launch_bounds__(256) void k_prefill_gather(DevCache c, const KT* __restrict__ Kp,
                                                        const KT* __restrict__ Vp, int n_max)
{
    using CT = typename CodeT<BITS>::T;
    constexpr int CH = D * (int)sizeof(KT) / 16;   // 16-byte chunks per row
    const int h = blockIdx.y, b = blockIdx.z, head = b * c.Hkv + h;
    const int occ = c.state[2 * head];   // min(N, S), or the kept tokens of a CHUNK prefill
    const int s = blockIdx.x * 16 + threadIdx.x / 16;
    const int j = threadIdx.x % 16;
    if (s >= occ) return;
    const size_t rowbase = (size_t)head * c.Smax;
    const int t = c.tok[rowbase + s];
    const uint4* ks = reinterpret_cast<const uint4*>(Kp + ((size_t)head * n_max + t) * D);
    const uint4* vs = reinterpret_cast<const uint4*>(Vp + ((size_t)head * n_max + t) * D);
    uint4* kd = reinterpret_cast<uint4*>(reinterpret_cast<KT*>(c.K) + (rowbase + s) * D);
    uint4* vd = reinterpret_cast<uint4*>(reinterpret_cast<KT*>(c.V) + (rowbase + s) * D);
    for (int q = j; q < CH; q += 16) kd[q] = ks[q];
    bool quantized = false;
    if constexpr (std::is_same<KT, bf16_t>::value) {
        if (c.vbits) {
            // value row -> codes of vbits bits and one scale (Q = 127 or 7:
            // scale = max|v| / Q, code = v / scale rounded half to even,
            // clamped to +-Q, fp32); the 16 lanes of the row each take 8
            // values (D / 8 <= 16)
            float f[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            const int nchunk = D / 8;
            if (j < nchunk) Vec16<bf16_t>::cvt(vs[j], f);
            float amax = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(f[e]));
            amax = fmaxf(amax, dpp_f<kDppXor1>(amax));
            amax = fmaxf(amax, dpp_f<kDppXor2>(amax));
            amax = fmaxf(amax, dpp_f<kDppHalfMirror>(amax));
            amax = fmaxf(amax, dpp_f<kDppMirror>(amax));
            if (c.vbits == 8) {
                const float sc = amax / 127.0f;
                if (j < nchunk)
                    reinterpret_cast<uint2*>(reinterpret_cast<int8_t*>(c.V) + (rowbase + s) * D)[j] = quantize8(f, sc);
                if (j == 0) c.vs[rowbase + s] = sc;
            } else {
                const float sc = amax / 7.0f;
                if (j < nchunk)
                    reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(c.V) + (rowbase + s) * (D / 2))[j] =
                        quantize4(f, sc);
                if (j == 0) c.vs[rowbase + s] = sc;
            }
            quantized = true;
        }
    }
    if (!quantized)
        for (int q = j; q < CH; q += 16) vd[q] = vs[q];
    if (j == 0)
        reinterpret_cast<CT*>(c.code)[(size_t)head * c.code_slots + s] =
            reinterpret_cast<const CT*>(c.pcode)[(size_t)head * c.pcode_slots + t];
}

// Exclusive prefix count of `flag` over the block's threads in thread order,
// and the block's total.  All threads of the block must call it; it holds
// two barriers and uses s_w[kSelWaves].
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

__device__ __forceinline__ int block_prefix(bool flag, int* s_w, int& total)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const unsigned long long m = __ballot(flag);
    const int below = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
    if (lane == 0) s_w[wave] = __popcll(m);
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        const int x = s_w[w];
        before += w < wave ? x : 0;
        all += x;
    }
    __syncthreads();   // s_w is reused by the next call
    total = all;
    return before + below;
}

// Exclusive prefix sum of v over the block's threads in thread order, and
// the block's total.  All threads of the block must call it; two barriers,
// s_w[kSelWaves] of scratch.
__device__ __forceinline__ int block_exclusive_sum(int v, int* s_w, int& total)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) s_w[wave] = x;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
        const int t = s_w[w];
        before += w < wave ? t : 0;
        all += t;
    }
    __syncthreads();
    total = all;
    return before + x - v;
}

// Chunk-granular prefill selection (HKV_PREFILL_CHUNK), three launches:
//   k_chunk_obs    (one block per head) hashes the G observation queries
//                  (fp32 dot products against R; any summation order is exact
//                  outside the flagged band), writes their codes, and clears
//                  the head's histogram of chunk scores;
//   k_chunk_score  (one thread per chunk) sums the Hamming distances of the
//                  chunk's key codes to the G query codes into its score and
//                  counts the score in the head's histogram (per block in
//                  LDS, then one global add per bin);
//   k_chunk_select (one block per head): E = nch - k chunks go, in order of
//                  (score descending, index ascending).  A suffix sum over the
//                  histogram finds the score T of the last one and how many
//                  chunks scoring exactly T go (the lowest-indexed ones); a
//                  prefix count in chunk order then places the kept chunks
//                  in slots 0, 1, ... and writes the kept list.
// With a reuse list the kept chunks are flags set from the list instead;
// with N <= S every chunk is kept.
template <int D, int BITS>
__global__ __launch_bounds__(kSelThreads) void k_chunk_obs(DevCache c, const float* __restrict__ qobs)
{
    using CT = typename CodeT<BITS>::T;
    // R and the group's queries go to LDS first, every load in flight at once
    constexpr int NR4 = D * BITS / 4, RPT = (NR4 + kSelThreads - 1) / kSelThreads;
    constexpr int NQ4 = kMaxGroup * D / 4, QPT = (NQ4 + kSelThreads - 1) / kSelThreads;
    __shared__ __align__(16) float sR[D * BITS];
    __shared__ __align__(16) float sQ[kMaxGroup * D];
    const int h = blockIdx.x, b = blockIdx.y, head = b * c.Hkv + h;
    const int tid = threadIdx.x, lane = tid & 63;
    const int G = c.G;
    const int nq4 = G * D / 4;
    const float4* q4 = reinterpret_cast<const float4*>(qobs + ((size_t)b * c.Hq + (size_t)h * G) * D);
    float4 rr[RPT], qq[QPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) rr[k] = reinterpret_cast<const float4*>(c.R)[min(tid + k * kSelThreads, NR4 - 1)];
#pragma unroll
    for (int k = 0; k < QPT; ++k) qq[k] = q4[min(tid + k * kSelThreads, nq4 - 1)];
#pragma unroll
    for (int k = 0; k < RPT; ++k)
        if (tid + k * kSelThreads < NR4) reinterpret_cast<float4*>(sR)[tid + k * kSelThreads] = rr[k];
#pragma unroll
    for (int k = 0; k < QPT; ++k)
        if (tid + k * kSelThreads < nq4) reinterpret_cast<float4*>(sQ)[tid + k * kSelThreads] = qq[k];
    int* hist = c.chist + (size_t)head * c.chist_bins;
    for (int i = tid; i < c.chist_bins; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    const int g = tid / BITS, j = tid % BITS;
    float y = 0.f;
    if (g < G) {
#pragma unroll 8
        for (int i = 0; i < D; ++i) y = fmaf(sQ[g * D + i], sR[i * BITS + j], y);
    }
    const unsigned long long m = __ballot(y > 0.f);
    if (g < G && j == 0) {
        const CT code = (CT)(m >> (lane & ~(BITS - 1) & 63));
        store_words(c.dbg_q + ((size_t)b * c.Hq + (size_t)h * G + g) * c.W, c.W, (unsigned long long)code);
    }
}

constexpr int kScoreThreads = 256;

template <int BITS>
__global__ __launch_bounds__(kScoreThreads) void k_chunk_score(DevCache c)
{
    using CT = typename CodeT<BITS>::T;
    extern __shared__ unsigned s_bins[];   // c.chist_bins counters
    __shared__ CT s_qc[kMaxGroup];
    const int h = blockIdx.y, b = blockIdx.z, head = b * c.Hkv + h;
    const int tid = threadIdx.x;
    const int G = c.G, C = c.pchunk;
    const int N = c.plen[b], S = c.budget[b];
    const int nch = (N + C - 1) / C;
    const int i = blockIdx.x * kScoreThreads + tid;
    if (N <= S || blockIdx.x * kScoreThreads >= nch) return;   // uniform over the block
    if (tid < G) {
        const uint32_t* p = c.dbg_q + ((size_t)b * c.Hq + (size_t)h * G + tid) * c.W;
        unsigned long long v = p[0];
        if (c.W > 1) v |= (unsigned long long)p[1] << 32;
        s_qc[tid] = (CT)v;
    }
    for (int k = tid; k < c.chist_bins; k += kScoreThreads) s_bins[k] = 0u;
    __syncthreads();
    if (i < nch) {
        const CT* pc = reinterpret_cast<const CT*>(c.pcode) + (size_t)head * c.pcode_slots;
        const int t1 = min(N, (i + 1) * C);
        int sum = 0;
        for (int t = i * C; t < t1; ++t) {
            const CT kc = pc[t];
            for (int g = 0; g < G; ++g) sum += popc((CT)(kc ^ s_qc[g]));
        }
        c.csum[(size_t)head * c.nchunk_max + i] = sum;
        atomicAdd(&s_bins[sum], 1u);
    }
    __syncthreads();
    int* hist = c.chist + (size_t)head * c.chist_bins;
    for (int k = tid; k < c.chist_bins; k += kScoreThreads)
        if (s_bins[k]) atomicAdd(hist + k, (int)s_bins[k]);
}

template <int BITS>
__global__ __launch_bounds__(kSelThreads) void k_chunk_select(DevCache c, const int* __restrict__ reuse,
                                                             int* __restrict__ kept, int kmax)
{
    const int h = blockIdx.x, b = blockIdx.y, head = b * c.Hkv + h;
    const int tid = threadIdx.x;
    const int C = c.pchunk;
    const int N = c.plen[b], S = c.budget[b];
    const int nch = (N + C - 1) / C;
    const bool all = N <= S;
    const int k = all ? nch : S / C;
    int* score = c.csum + (size_t)head * c.nchunk_max;
    const size_t rowbase = (size_t)head * c.Smax;

    __shared__ int s_w[kSelWaves];
    __shared__ int s_T, s_evict_eq, s_short;
    if (tid == 0) {
        s_short = 0;
        s_T = 0;
        s_evict_eq = 0;
    }

    const bool scored = !all && !reuse;
    if (scored) {
        // the E-th largest score: thread tid owns a run of bins counted from
        // the top; a prefix sum over threads gives the chunks above its run
        const int E = nch - k;
        const int* hist = c.chist + (size_t)head * c.chist_bins;
        const int nb = c.chist_bins, per = (nb + kSelThreads - 1) / kSelThreads;
        const int hi = nb - 1 - tid * per, lo = max(hi - per + 1, 0);   // run [lo, hi], top down
        int local = 0;
        for (int v = hi; v >= lo; --v) local += hist[v];
        int total;
        const int above = block_exclusive_sum(hi >= 0 ? local : 0, s_w, total);
        if (hi >= 0 && above < E && above + local >= E) {
            int cum = above, v = hi;
            for (; v > lo; --v) {
                if (cum + hist[v] >= E) break;
                cum += hist[v];
            }
            s_T = v;
            s_evict_eq = E - cum;   // chunks scoring exactly T that go, lowest first
        }
    } else if (!all) {
        // reuse: flags from the list.  Other threads read these flags: the
        // stores are waited for (agent-scope fence) before each barrier and
        // read back with agent-scope loads from L2, so the hand-off does not
        // depend on how the CU's L1 treats stores of other waves.
        for (int i = tid; i < nch; i += kSelThreads) score[i] = 0;
        __threadfence();
        __syncthreads();
        for (int j = tid; j < k; j += kSelThreads) {
            const int i = reuse[(size_t)head * kmax + j];
            if (i >= 0 && i < nch) __hip_atomic_store(score + i, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __threadfence();
    }
    __syncthreads();
    const int T = scored ? s_T : 0, evict_eq = scored ? s_evict_eq : 0;

    // 4. kept chunks in chunk order -> slots
    // scores come from k_chunk_score (an earlier launch), flags from other
    // threads of this block (through L2); values two tiles ahead are in
    // flight while a tile is placed
    auto value = [&](int i) {
        if (all || i >= nch) return 0;
        return scored ? score[i] : __hip_atomic_load(score + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    // One block scan per tile counts, for every chunk, the chunks before it
    // that score below T ("lt") and exactly T ("eq").  Of the eq chunks the
    // first evict_eq (in chunk order, over the whole head) go, so the kept
    // eq chunks before a chunk are its eq count minus the evicted ones.
    auto evicted_eq = [&](int eq_seen) { return min(eq_seen, evict_eq); };
    int base = 0, base_eq = 0;
    int next1 = value(tid), next2 = value(tid + kSelThreads);
    for (int i0 = 0; i0 < nch; i0 += kSelThreads) {
        const int i = i0 + tid;
        const bool valid = i < nch;
        const int sc = next1;
        next1 = next2;
        next2 = value(i + 2 * kSelThreads);
        bool lt, eq;
        if (scored) {
            lt = valid && sc < T;
            eq = valid && sc == T;
        } else {
            lt = valid && (all || sc != 0);   // kept chunk
            eq = false;
        }
        int tot;
        const int ex = block_exclusive_sum((int)lt | ((int)eq << 16), s_w, tot);
        const int lt_before = ex & 0xFFFF, eq_before = ex >> 16;
        const bool keep = lt || (eq && base_eq + eq_before >= evict_eq);
        const int pos = base + lt_before + eq_before - (evicted_eq(base_eq + eq_before) - evicted_eq(base_eq));
        if (keep && pos < k) {   // exactly k are kept; the bound keeps every write inside the slots regardless
            if (kept) kept[(size_t)head * kmax + pos] = i;
            const int len = min(C, N - i * C);
            for (int r = 0; r < len; ++r) c.tok[rowbase + (size_t)pos * C + r] = i * C + r;
            if (len < C) s_short = C - len;   // only the last chunk can be short; it is placed last
        }
        const int tlt = tot & 0xFFFF, teq = tot >> 16;
        base += tlt + teq - (evicted_eq(base_eq + teq) - evicted_eq(base_eq));
        base_eq += teq;
    }
    __syncthreads();
    const int placed = min(base, k);
    const int n = placed * C - s_short;   // kept tokens
    for (int s = n + tid; s < min(N, S); s += kSelThreads) c.tok[rowbase + s] = -1;
    if (kept)
        for (int j = placed + tid; j < kmax; j += kSelThreads) kept[(size_t)head * kmax + j] = -1;
    if (tid == 0) c.state[2 * head] = n;
}

// Host tier at prefill: the prompt tokens the cache does not hold become the
// tier's entries, in position order.  One block per head marks the held
// tokens in a bitset (device atomics, read back through L2 after a fence) and
// writes the positions of the others to the tier's token array with block
// prefix counts; k_tier_copy_prompt then copies their rows.
__global__ __launch_bounds__(kSelThreads) void k_tier_list_dropped(DevCache c)
{
    const int h = blockIdx.x, b = blockIdx.y, head = b * c.Hkv + h;
    const int tid = threadIdx.x;
    const int N = c.plen[b], n = c.state[2 * head];
    const int words = (N + 31) / 32;
    unsigned* flags = c.tflag + (size_t)head * c.tflag_words;
    const size_t rowbase = (size_t)head * c.Smax;
    __shared__ int s_w[kSelWaves];
    for (int w = tid; w < words; w += kSelThreads) flags[w] = 0u;
    __threadfence();
    __syncthreads();
    for (int s = tid; s < n; s += kSelThreads) {
        const int t = c.tok[rowbase + s];
        if (t >= 0 && t < N) atomicOr(flags + (t >> 5), 1u << (t & 31));
    }
    __threadfence();
    __syncthreads();
    const int cnt0 = c.tcount[head];
    int base = 0;
    for (int t0 = 0; t0 < N; t0 += kSelThreads) {
        const int t = t0 + tid;
        bool drop = false;
        if (t < N) {
            const unsigned w = __hip_atomic_load(flags + (t >> 5), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            drop = !((w >> (t & 31)) & 1u);
        }
        int total;
        const int pos = cnt0 + base + block_prefix(drop, s_w, total);
        if (drop && pos < c.tcap) c.ttok[(size_t)head * c.tcap + pos] = t;
        base += total;
    }
    if (tid == 0) c.tcount[head] = cnt0 + base;   // every thread read cnt0 before the loop's barriers
}

// Rows of the listed prompt tokens into the tier: 16 rows per block, 16 lanes
// per row.
template <int D, typename KT>
__global__ __launch_bounds__(256) void k_tier_copy_prompt(DevCache c, const KT* __restrict__ Kp,
                                                          const KT* __restrict__ Vp, int n_max)
{
    constexpr int CH = D * (int)sizeof(KT) / 16;   // 16-byte pieces per row
    const int h = blockIdx.y, b = blockIdx.z, head = b * c.Hkv + h;
    const int m = min(c.tcount[head], c.tcap);
    const int j = blockIdx.x * 16 + threadIdx.x / 16, l = threadIdx.x % 16;
    if (j >= m) return;
    const int t = c.ttok[(size_t)head * c.tcap + j];
    const uint4* ks = reinterpret_cast<const uint4*>(Kp + ((size_t)head * n_max + t) * D);
    const uint4* vs = reinterpret_cast<const uint4*>(Vp + ((size_t)head * n_max + t) * D);
    uint4* kd = reinterpret_cast<uint4*>(reinterpret_cast<KT*>(c.tK) + ((size_t)head * c.tcap + j) * D);
    uint4* vd = reinterpret_cast<uint4*>(reinterpret_cast<KT*>(c.tV) + ((size_t)head * c.tcap + j) * D);
    for (int q = l; q < CH; q += 16) {
        kd[q] = ks[q];
        vd[q] = vs[q];
    }
}

template <int BITS>
__global__ void k_export_codes(DevCache c, uint32_t* __restrict__ out)
{
    using CT = typename CodeT<BITS>::T;
    const int h = blockIdx.y, b = blockIdx.z, head = b * c.Hkv + h;
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= c.Smax) return;
    const unsigned long long v = reinterpret_cast<const CT*>(c.code)[(size_t)head * c.code_slots + s];
    store_words(out + ((size_t)head * c.Smax + s) * c.W, c.W, v);
}

template <int BITS>
__global__ void k_import_codes(DevCache c, const uint32_t* __restrict__ in)
{
    using CT = typename CodeT<BITS>::T;
    const int h = blockIdx.y, b = blockIdx.z, head = b * c.Hkv + h;
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= c.Smax) return;
    const uint32_t* p = in + ((size_t)head * c.Smax + s) * c.W;
    unsigned long long v = p[0];
    if (c.W > 1) v |= (unsigned long long)p[1] << 32;
    reinterpret_cast<CT*>(c.code)[(size_t)head * c.code_slots + s] = (CT)v;
}

template <int BITS>
__global__ void k_export_pcodes(DevCache c, const void* __restrict__ src, int nh, uint32_t* __restrict__ out,
                                int n_max)
{
    using CT = typename CodeT<BITS>::T;
    const int h = blockIdx.y, b = blockIdx.z, head = b * nh + h;
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= n_max) return;
    const unsigned long long v = reinterpret_cast<const CT*>(src)[(size_t)head * c.pcode_slots + t];
    store_words(out + ((size_t)head * n_max + t) * c.W, c.W, v);
}

template <typename F>
hipError_t with_bits(const DevCache& c, F&& f)
{
    if (c.bits == 16) return f(std::integral_constant<int, 16>{});
    if (c.bits == 32) return f(std::integral_constant<int, 32>{});
    return f(std::integral_constant<int, 64>{});
}

template <typename F>
hipError_t with_d_kv(const DevCache& c, F&& f)
{
    if (c.d == 64) {
        if (c.kv_bf16) return f(std::integral_constant<int, 64>{}, bf16_t{});
        return f(std::integral_constant<int, 64>{}, float{});
    }
    if (c.kv_bf16) return f(std::integral_constant<int, 128>{}, bf16_t{});
    return f(std::integral_constant<int, 128>{}, float{});
}

}  // namespace

__global__ void k_clear_step_scratch(DevCache c)
{
    const int head = blockIdx.x * blockDim.x + threadIdx.x;
    if (head < c.B * c.Hkv) {
        c.ekey[2 * head] = 0ull;
        c.ekey[2 * head + 1] = 0ull;
        c.count[head * kCountStride] = 0u;
    }
}

hipError_t launch_clear_step_scratch(const DevCache& c, hipStream_t st)
{
    hipLaunchKernelGGL(k_clear_step_scratch, dim3((c.B * c.Hkv + 255) / 256), dim3(256), 0, st, c);
    return hipGetLastError();
}

// Fills n words with a quiet NaN (debug poisoning of per-step partial results).
__global__ void k_fill_nan(uint32_t* __restrict__ p, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0x7FC00000u;
}

static hipError_t fill_nan(float* p, size_t n, hipStream_t st)
{
    if (!p || n == 0) return hipSuccess;
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(k_fill_nan, dim3((unsigned)(blocks < 2048 ? blocks : 2048)), dim3(256), 0, st,
                       reinterpret_cast<uint32_t*>(p), n);
    return hipGetLastError();
}

hipError_t launch_poison_partials(const DevCache& c, hipStream_t st)
{
    const size_t heads = (size_t)c.B * c.Hkv, qheads = (size_t)c.B * c.Hq;
    hipError_t e = fill_nan(c.frec, heads * c.nsplit * c.G * c.d, st);
    if (e == hipSuccess) e = fill_nan(c.fscal, heads * c.nsplit * c.G * 4, st);
    if (e == hipSuccess) e = fill_nan(c.cand_v, heads * c.nsplit * c.d, st);
    if (e == hipSuccess) e = fill_nan(c.part, qheads * c.nsplit * (c.d + 4), st);
    if (e == hipSuccess && c.tpart) e = fill_nan(c.tpart, qheads * c.tsplit * (c.d + 4), st);
    return e;
}

hipError_t launch_reset(const DevCache& c, hipStream_t st)
{
    hipLaunchKernelGGL(k_reset, dim3((c.Smax + 255) / 256, c.Hkv, c.B), dim3(256), 0, st, c);
    return hipGetLastError();
}

template <int BITS, int GQ>
hipError_t launch_select(const DevCache& c, hipStream_t st)
{
    const size_t lds = select_lds_bytes<BITS>(c.Smax, GQ > 0 ? c.G : 0);
    hipError_t e = hipFuncSetAttribute((const void*)k_prefill_select<BITS, GQ>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_prefill_select<BITS, GQ>), dim3(c.Hkv, c.B), dim3(1024), lds, st, c);
    return hipGetLastError();
}

template <int BITS>
hipError_t launch_select_query(const DevCache& c, hipStream_t st)
{
    if (c.G <= 1) return launch_select<BITS, 1>(c, st);
    if (c.G <= 2) return launch_select<BITS, 2>(c, st);
    if (c.G <= 4) return launch_select<BITS, 4>(c, st);
    if (c.G <= 8) return launch_select<BITS, 8>(c, st);
    return launch_select<BITS, 16>(c, st);
}

hipError_t launch_prefill(const DevCache& c, const void* K, const void* V, const float* Q, int n_max, int policy,
                          hipStream_t st)
{
    hipLaunchKernelGGL(k_prefill_init, dim3((c.Smax + 255) / 256, c.Hkv, c.B), dim3(256), 0, st, c);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (n_max <= 0) return hipSuccess;
    err = with_bits(c, [&](auto bb) {
        constexpr int BITS = decltype(bb)::value;
        return with_d_kv(c, [&](auto dd, auto kt) {
            constexpr int D = decltype(dd)::value;
            using KT = decltype(kt);
            hipError_t e = launch_project_keys<D, BITS, KT>(c, K, n_max, st);
            if (e != hipSuccess) return e;
            if (policy == HKV_PREFILL_STREAM) {
                e = launch_select<BITS, 0>(c, st);
            } else if (policy == HKV_PREFILL_QUERY) {
                hipLaunchKernelGGL((k_project_mfma<D, BITS, float>), dim3(proj_blocks(n_max), c.Hq, c.B),
                                   dim3(256), 0, st, c, Q, n_max, c.Hq, c.qcode);
                e = hipGetLastError();
                if (e == hipSuccess) e = launch_select_query<BITS>(c, st);
            }
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((k_prefill_gather<D, BITS, KT>), dim3((c.Smax + 15) / 16, c.Hkv, c.B),
                               dim3(256), 0, st, c, (const KT*)K, (const KT*)V, n_max);
            return hipGetLastError();
        });
    });
    if (err == hipSuccess && c.tK) err = launch_tier_spill_prompt(c, K, V, n_max, st);
    return err;
}

hipError_t launch_prefill_chunks(const DevCache& c, const void* K, const void* V, const float* q_obs,
                                 const int* reuse, int* kept, int kmax, int n_max, hipStream_t st)
{
    hipLaunchKernelGGL(k_prefill_init, dim3((c.Smax + 255) / 256, c.Hkv, c.B), dim3(256), 0, st, c);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    err = with_bits(c, [&](auto bb) {
        constexpr int BITS = decltype(bb)::value;
        return with_d_kv(c, [&](auto dd, auto kt) {
            constexpr int D = decltype(dd)::value;
            using KT = decltype(kt);
            if (n_max > 0) {
                hipError_t e = launch_project_keys<D, BITS, KT>(c, K, n_max, st);
                if (e != hipSuccess) return e;
            }
            if (q_obs) {
                hipLaunchKernelGGL((k_chunk_obs<D, BITS>), dim3(c.Hkv, c.B), dim3(kSelThreads), 0, st, c, q_obs);
                if (!reuse && n_max > 0) {
                    const size_t lds = (size_t)c.chist_bins * 4;
                    hipError_t ea = hipFuncSetAttribute((const void*)k_chunk_score<BITS>,
                                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
                    if (ea != hipSuccess) return ea;
                    const int nch = (n_max + c.pchunk - 1) / c.pchunk;
                    hipLaunchKernelGGL((k_chunk_score<BITS>), dim3((nch + kScoreThreads - 1) / kScoreThreads, c.Hkv, c.B),
                                       dim3(kScoreThreads), lds, st, c);
                }
            }
            hipLaunchKernelGGL((k_chunk_select<BITS>), dim3(c.Hkv, c.B), dim3(kSelThreads), 0, st, c, reuse, kept,
                               kmax);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess || n_max <= 0) return e;
            hipLaunchKernelGGL((k_prefill_gather<D, BITS, KT>), dim3((c.Smax + 15) / 16, c.Hkv, c.B),
                               dim3(256), 0, st, c, (const KT*)K, (const KT*)V, n_max);
            return hipGetLastError();
        });
    });
    if (err == hipSuccess && c.tK) err = launch_tier_spill_prompt(c, K, V, n_max, st);
    return err;
}

hipError_t launch_tier_spill_prompt(const DevCache& c, const void* K, const void* V, int n_max, hipStream_t st)
{
    hipLaunchKernelGGL(k_tier_list_dropped, dim3(c.Hkv, c.B), dim3(kSelThreads), 0, st, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n_max <= 0) return e;
    return with_d_kv(c, [&](auto dd, auto kt) {
        constexpr int D = decltype(dd)::value;
        using KT = decltype(kt);
        hipLaunchKernelGGL((k_tier_copy_prompt<D, KT>), dim3((n_max + 15) / 16, c.Hkv, c.B), dim3(256), 0, st, c,
                           (const KT*)K, (const KT*)V, n_max);
        return hipGetLastError();
    });
}

hipError_t launch_export_codes(const DevCache& c, uint32_t* codes, hipStream_t st)
{
    return with_bits(c, [&](auto bb) {
        hipLaunchKernelGGL((k_export_codes<decltype(bb)::value>), dim3((c.Smax + 255) / 256, c.Hkv, c.B),
                           dim3(256), 0, st, c, codes);
        return hipGetLastError();
    });
}

hipError_t launch_import_codes(const DevCache& c, const uint32_t* codes, hipStream_t st)
{
    return with_bits(c, [&](auto bb) {
        hipLaunchKernelGGL((k_import_codes<decltype(bb)::value>), dim3((c.Smax + 255) / 256, c.Hkv, c.B),
                           dim3(256), 0, st, c, codes);
        return hipGetLastError();
    });
}

hipError_t launch_export_pcodes(const DevCache& c, uint32_t* codes, int n_max, bool queries, hipStream_t st)
{
    if (n_max <= 0) return hipSuccess;
    const int nh = queries ? c.Hq : c.Hkv;
    const void* src = queries ? c.qcode : c.pcode;
    return with_bits(c, [&](auto bb) {
        hipLaunchKernelGGL((k_export_pcodes<decltype(bb)::value>), dim3((n_max + 255) / 256, nh, c.B),
                           dim3(256), 0, st, c, src, nh, codes, n_max);
        return hipGetLastError();
    });
}

}  // namespace hkv
