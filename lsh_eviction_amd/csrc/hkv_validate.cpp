// hkv_validate.cpp -- host-only configuration checks and workspace layout.
#include <algorithm>
#include <climits>
#include <functional>
#include <cstdio>
#include <cstring>
#include <vector>

#include "hkv_layout.h"

namespace hkv {

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

hkv_status compute_layout(const hkv_config* cfg, Layout* L, char* err, size_t errlen)
{
#define FAIL(code, ...)                                  \
    do {                                                 \
        if (err && errlen) snprintf(err, errlen, __VA_ARGS__); \
        return code;                                     \
    } while (0)
    if (!cfg) FAIL(HKV_ERR_INVALID_ARG, "config is NULL");
    if (!cfg->budgets) FAIL(HKV_ERR_INVALID_ARG, "budgets is NULL");
    if (cfg->batch < 1 || cfg->batch > kMaxBatch)
        FAIL(HKV_ERR_UNSUPPORTED, "batch %d outside [1, %d]", cfg->batch, kMaxBatch);
    if (cfg->n_kv_heads < 1 || cfg->n_q_heads < 1)
        FAIL(HKV_ERR_INVALID_ARG, "head counts must be positive");
    if (cfg->n_q_heads % cfg->n_kv_heads != 0)
        FAIL(HKV_ERR_UNSUPPORTED, "n_q_heads %d not a multiple of n_kv_heads %d", cfg->n_q_heads,
             cfg->n_kv_heads);
    const int G = cfg->n_q_heads / cfg->n_kv_heads;
    if (G > kMaxGroup) FAIL(HKV_ERR_UNSUPPORTED, "group size %d > %d", G, kMaxGroup);
    if (cfg->head_dim != 64 && cfg->head_dim != 128)
        FAIL(HKV_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", cfg->head_dim);
    if (cfg->n_bits != 16 && cfg->n_bits != 32 && cfg->n_bits != 64)
        FAIL(HKV_ERR_UNSUPPORTED, "n_bits %d not in {16, 32, 64}", cfg->n_bits);
    if (cfg->kv_dtype != HKV_F32 && cfg->kv_dtype != HKV_BF16)
        FAIL(HKV_ERR_UNSUPPORTED, "kv_dtype %d unknown", cfg->kv_dtype);
    if (cfg->prefill_policy != HKV_PREFILL_STREAM && cfg->prefill_policy != HKV_PREFILL_TRUNCATE &&
        cfg->prefill_policy != HKV_PREFILL_QUERY && cfg->prefill_policy != HKV_PREFILL_CHUNK)
        FAIL(HKV_ERR_UNSUPPORTED, "prefill_policy %d unknown", cfg->prefill_policy);
    const bool chunked = cfg->prefill_policy == HKV_PREFILL_CHUNK;
    if (!chunked && cfg->prefill_chunk != 0)
        FAIL(HKV_ERR_UNSUPPORTED, "prefill_chunk %d set without HKV_PREFILL_CHUNK", cfg->prefill_chunk);
    if (chunked && (cfg->prefill_chunk < 0 || cfg->prefill_chunk > kMaxPrefillChunk))
        FAIL(HKV_ERR_UNSUPPORTED, "prefill_chunk %d outside [0, %d]", cfg->prefill_chunk, kMaxPrefillChunk);
    if (cfg->value_bits != 0 && cfg->value_bits != 8 && cfg->value_bits != 4)
        FAIL(HKV_ERR_UNSUPPORTED, "value_bits %d not in {0, 4, 8}", cfg->value_bits);
    if (cfg->value_bits != 0 && (cfg->kv_dtype != HKV_BF16 || cfg->decode_schedule != HKV_DECODE_FUSED))
        FAIL(HKV_ERR_UNSUPPORTED, "value_bits %d needs kv_dtype HKV_BF16 and HKV_DECODE_FUSED", cfg->value_bits);
    if (cfg->tier_capacity < 0 || cfg->tier_capacity > kMaxTierCapacity)
        FAIL(HKV_ERR_UNSUPPORTED, "tier_capacity %d outside [0, %d]", cfg->tier_capacity, kMaxTierCapacity);
    if (cfg->tier_capacity > 0 && cfg->value_bits != 0)
        FAIL(HKV_ERR_UNSUPPORTED, "a host tier needs value_bits 0");
    if (cfg->decode_schedule != HKV_DECODE_FUSED && cfg->decode_schedule != HKV_DECODE_SPLIT)
        FAIL(HKV_ERR_UNSUPPORTED, "decode_schedule %d unknown", cfg->decode_schedule);
    if (cfg->max_prompt < 0 || cfg->max_prompt > (1 << 24))
        FAIL(HKV_ERR_UNSUPPORTED, "max_prompt %d outside [0, 2^24]", cfg->max_prompt);
    if (cfg->chunk != 0 && (cfg->chunk < 64 || cfg->chunk > 65536 || cfg->chunk % 64 != 0))
        FAIL(HKV_ERR_UNSUPPORTED, "chunk %d must be 0 or a multiple of 64 in [64, 65536]",
             cfg->chunk);
    const int cb = cfg->n_bits / 8;
    int Smax = 0;
    for (int b = 0; b < cfg->batch; ++b) {
        const int s = cfg->budgets[b];
        if (s < 1 || s > kMaxBudget)
            FAIL(HKV_ERR_UNSUPPORTED, "budget[%d] = %d outside [1, %d]", b, s, kMaxBudget);
        if ((cfg->prefill_policy == HKV_PREFILL_STREAM || cfg->prefill_policy == HKV_PREFILL_QUERY) &&
            (size_t)s * cb > kLdsTableBytes)
            FAIL(HKV_ERR_UNSUPPORTED,
                 "budget[%d] = %d: its %d-byte code table exceeds the %zu-byte on-chip table of "
                 "the sequential prefill", b, s, s * cb, kLdsTableBytes);
        if (s > Smax) Smax = s;
    }

    Layout& l = *L;
    memset(&l, 0, sizeof(l));
    l.B = cfg->batch; l.Hq = cfg->n_q_heads; l.Hkv = cfg->n_kv_heads; l.G = G;
    l.d = cfg->head_dim; l.bits = cfg->n_bits; l.W = (cfg->n_bits + 31) / 32; l.cb = cb;
    l.es = cfg->kv_dtype == HKV_BF16 ? 2 : 4;
    l.kv_dtype = cfg->kv_dtype; l.prefill_policy = cfg->prefill_policy;
    l.schedule = cfg->decode_schedule;
    l.value_bits = cfg->value_bits;
    l.Smax = Smax;
    bool ragged = false;
    for (int b = 1; b < cfg->batch; ++b) ragged = ragged || cfg->budgets[b] != cfg->budgets[0];
    if (cfg->chunk) {
        l.chunk = cfg->chunk;
    } else {
        // about one block of the decode step per compute unit: the slots of
        // all eviction domains over kChunkTargetBlocks, a multiple of 64, and
        // at least kMinAutoChunk (below that the merge of more, shorter
        // blocks costs more than the compute units they add)
        long long slots = 0;
        for (int b = 0; b < cfg->batch; ++b) slots += cfg->budgets[b];
        slots *= cfg->n_kv_heads;
        long long ch = (slots + kChunkTargetBlocks - 1) / kChunkTargetBlocks;
        ch = (ch + 63) / 64 * 64;
        l.chunk = (int)(ch < kMinAutoChunk ? kMinAutoChunk : (ch > 65536 ? 65536 : ch));
        // ragged budgets: the chunk whose longest-first block list ends first
        if (ragged) l.chunk = ragged_auto_chunk(cfg->budgets, cfg->batch, cfg->n_kv_heads, l.chunk);
    }
    l.nsplit = (Smax + l.chunk - 1) / l.chunk;
    if (l.nsplit > 65535)
        FAIL(HKV_ERR_UNSUPPORTED, "chunk %d too small for a budget of %d slots (more than 65535 splits)", l.chunk, Smax);
    l.nblk = ragged ? fused_block_order(cfg->budgets, cfg->batch, l.chunk, nullptr) : 0;
    if ((long long)l.nblk * l.Hkv > INT_MAX)
        FAIL(HKV_ERR_UNSUPPORTED, "chunk %d too small: more than 2^31 - 1 decode blocks", l.chunk);
    l.max_prompt = cfg->max_prompt;
    l.code_slots = align_up((size_t)Smax, 64);
    l.pcode_slots = align_up((size_t)(cfg->max_prompt > 0 ? cfg->max_prompt : 1), 64);
    l.pchunk = chunked ? (cfg->prefill_chunk ? cfg->prefill_chunk : kDefaultPrefillChunk) : 0;
    l.nchunk_max = chunked ? align_up((size_t)((cfg->max_prompt + l.pchunk - 1) / l.pchunk) + 1, 64) : 0;
    l.chist_bins = chunked ? l.pchunk * G * cfg->n_bits + 1 : 0;
    l.tcap = cfg->tier_capacity;
    if (l.tcap > 0) {
        int ts = kTierBlocks / (l.B * l.Hkv);
        ts = ts < 1 ? 1 : (ts > 256 ? 256 : ts);
        const int rows16 = (l.tcap + 15) / 16;   // no split smaller than 16 rows
        l.tsplit = ts < rows16 ? ts : rows16;
        l.tflag_words = (size_t)(cfg->max_prompt + 31) / 32 + 1;
    }

    const size_t heads = (size_t)l.B * l.Hkv;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align_up(off + bytes, kAlign);
        return o;
    };
    l.off_R = take((size_t)l.d * l.bits * 4);
    l.off_budget = take((size_t)l.B * 4);
    l.off_plen = take((size_t)l.B * 4);
    l.off_state = take(heads * 2 * 4);
    l.off_K = take(heads * Smax * l.d * l.es);
    // value rows: d elements of the kv dtype, or d codes of value_bits bits
    l.v_bytes = l.value_bits ? heads * Smax * l.d * l.value_bits / 8 : heads * Smax * l.d * l.es;
    l.off_V = take(l.v_bytes);
    // value scales, padded by 16 entries: the attention tile reads 16 rows' scales at once
    l.off_vs = take(l.value_bits ? (heads * Smax + 16) * 4 : 0);
    l.off_code = take(heads * l.code_slots * cb);
    l.off_tok = take(heads * Smax * 4);
    l.off_dbg_q = take((size_t)l.B * l.Hq * l.W * 4);
    l.off_dbg_k = take(heads * l.W * 4);
    l.off_part = take((size_t)l.B * l.Hq * l.nsplit * (l.d + 4) * 4);
    l.off_frec = take(heads * l.nsplit * G * l.d * 4);
    l.off_fscal = take(heads * l.nsplit * G * 16);
    l.off_cand_v = take(heads * l.nsplit * l.d * 4);
    l.off_ekey = take(heads * 2 * 8);
    l.off_info = take(heads * 2 * 4);
    l.off_count = take(heads * kCountStride * 4);
    l.off_blk = take((size_t)l.nblk * 8);
    l.off_pcode = take(heads * l.pcode_slots * cb);
    l.off_qcode = take(cfg->prefill_policy == HKV_PREFILL_QUERY ? (size_t)l.B * l.Hq * l.pcode_slots * cb : 0);
    // per-chunk scores of the prompt (HKV_PREFILL_CHUNK)
    l.off_csum = take(heads * l.nchunk_max * 4);
    l.off_chist = take(heads * (size_t)l.chist_bins * 4);
    // host tier: counts, partials of the tiered attention, held-token bitset of the prompt
    l.off_tcount = take(l.tcap > 0 ? heads * 4 : 0);
    l.off_tpart = take(l.tcap > 0 ? (size_t)l.B * l.Hq * l.tsplit * (l.d + 4) * 4 : 0);
    l.off_tflag = take(l.tcap > 0 ? heads * l.tflag_words * 4 : 0);
    l.total = off;
    return HKV_OK;
#undef FAIL
}

int fused_block_order(const int32_t* budgets, int B, int chunk, uint32_t* out)
{
    struct Blk {
        int rows, b, split, len;   // rows: slots of this split, len: the sequence's split length
    };
    std::vector<Blk> v;
    for (int b = 0; b < B; ++b) {
        const int S = budgets[b];
        const int k0 = (S + chunk - 1) / chunk;
        const int len = (int)align_up((size_t)((S + k0 - 1) / k0), 64);
        const int k = (S + len - 1) / len;
        for (int j = 0; j < k; ++j) v.push_back({std::min(len, S - j * len), b, j, len});
    }
    if (out) {
        std::stable_sort(v.begin(), v.end(), [](const Blk& x, const Blk& y) { return x.rows > y.rows; });
        for (size_t i = 0; i < v.size(); ++i) {
            out[2 * i] = (uint32_t)v[i].b | (uint32_t)v[i].split << 16;
            out[2 * i + 1] = (uint32_t)v[i].len;
        }
    }
    return (int)v.size();
}

long long fused_makespan(const int32_t* budgets, int B, int Hkv, int chunk)
{
    const int n = fused_block_order(budgets, B, chunk, nullptr);
    std::vector<uint32_t> list((size_t)n * 2);
    fused_block_order(budgets, B, chunk, list.data());
    // per XCD, the time each of its compute units is next free (min-heaps)
    std::vector<std::vector<long long>> free(kXcds, std::vector<long long>(kCusPerXcd, 0));
    long long id = 0, end = 0;
    for (int i = 0; i < n; ++i) {
        const int b = (int)(list[2 * i] & 0xFFFFu), j = (int)(list[2 * i] >> 16), len = (int)list[2 * i + 1];
        const long long rows = std::min(len, budgets[b] - j * len);
        for (int h = 0; h < Hkv; ++h, ++id) {
            std::vector<long long>& x = free[id % kXcds];
            std::pop_heap(x.begin(), x.end(), std::greater<long long>());
            x.back() += rows + kBlockFixedSlots;
            end = std::max(end, x.back());
            std::push_heap(x.begin(), x.end(), std::greater<long long>());
        }
    }
    return end;
}

int ragged_auto_chunk(const int32_t* budgets, int B, int Hkv, int base)
{
    int Smax = 0;
    long long slots = 0;
    for (int b = 0; b < B; ++b) {
        Smax = std::max(Smax, (int)budgets[b]);
        slots += budgets[b];
    }
    const int lo = std::max(kMinAutoChunk, (int)align_up((size_t)(base / 4), 64));
    const int hi = std::min(65536, (int)align_up((size_t)Smax, 64));
    if (lo >= hi) return base;
    const int step = (int)align_up((size_t)((hi - lo) / kAutoChunkCandidates + 1), 64);
    int best = base;
    long long best_t = fused_makespan(budgets, B, Hkv, base);
    for (int T = hi; T >= lo; T -= step) {
        // blocks of this chunk: at most sum_b ceil(S_b / T) per head
        if ((slots / T + B) * Hkv > kAutoChunkMaxBlocks) continue;
        const long long t = fused_makespan(budgets, B, Hkv, T);
        if (t < best_t || (t == best_t && T > best)) {
            best = T;
            best_t = t;
        }
    }
    return best;
}

}  // namespace hkv

extern "C" hkv_status hkv_validate_config(const hkv_config* cfg)
{
    hkv::Layout l;
    return hkv::compute_layout(cfg, &l, nullptr, 0);
}

extern "C" hkv_status hkv_workspace_bytes(const hkv_config* cfg, size_t* bytes)
{
    if (!bytes) return HKV_ERR_INVALID_ARG;
    hkv::Layout l;
    hkv_status s = hkv::compute_layout(cfg, &l, nullptr, 0);
    if (s == HKV_OK) *bytes = l.total;
    return s;
}

extern "C" hkv_status hkv_config_chunk(const hkv_config* cfg, int32_t* chunk)
{
    if (!chunk) return HKV_ERR_INVALID_ARG;
    hkv::Layout l;
    hkv_status s = hkv::compute_layout(cfg, &l, nullptr, 0);
    if (s == HKV_OK) *chunk = l.chunk;
    return s;
}

extern "C" const char* hkv_status_str(hkv_status s)
{
    switch (s) {
    case HKV_OK: return "HKV_OK";
    case HKV_ERR_INVALID_ARG: return "HKV_ERR_INVALID_ARG";
    case HKV_ERR_UNSUPPORTED: return "HKV_ERR_UNSUPPORTED";
    case HKV_ERR_STATE: return "HKV_ERR_STATE";
    case HKV_ERR_DEVICE: return "HKV_ERR_DEVICE";
    }
    return "HKV_UNKNOWN_STATUS";
}
