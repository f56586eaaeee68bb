/*
 * hkv.h -- C ABI of libhkv.so: HashEvict LSH eviction and decode attention
 * over a fixed-budget KV cache, on one MI355X (gfx950).
 *
 * The method (HashEvict summary page, "HashEvict: A Pre-Attention KV Cache
 * Eviction Strategy using Locality-Sensitive Hashing", arXiv 2412.16187;
 * section "Technical framework" stages 1-5 and the abstract): at every decode
 * step, for every (sequence, KV head),
 *   1. project the current query through a fixed Gaussian matrix R (d x b),
 *   2. binarise the projection to a b-bit code,
 *   3. take the Hamming distance between that code and the code of every
 *      cached key (codes kept in a packed table in GPU memory),
 *   4. pick the cached token farthest from the query (cosine-dissimilar, so
 *      expected to get the lowest attention) -- before any attention score,
 *   5. overwrite that slot with the new token's key, value and key code,
 * and then attend over the cache, which therefore never grows past its budget.
 *
 * Readings taken where the page is silent (the GPU path and the CPU oracle
 * both follow them):
 *   - binarisation threshold 0: bit j is set iff (x . R[:, j]) > 0;
 *   - bit j of a code is bit (j % 32) of uint32 word j / 32 (LSB first);
 *   - grouped-query attention: the score of a slot is the SUM over the G query
 *     heads of the KV head of their Hamming distances; query head hq belongs
 *     to KV head hq / G;
 *   - ties go to the lowest slot index;
 *   - while the cache is not full a new token goes to the lowest empty slot
 *     and nothing is evicted;
 *   - the new token is not a candidate for eviction; attention runs over the
 *     cache after the write, with logits q.k / sqrt(d), no mask, no rotary;
 *   - prefill (HKV_PREFILL_STREAM, default): the prompt tokens enter one at a
 *     time by the decode rule, each scored against its own key code (prefill
 *     has no query); HKV_PREFILL_TRUNCATE keeps the first `budget` tokens;
 *     HKV_PREFILL_QUERY applies the decode rule itself to every prompt token
 *     past the budget, scored against the token's own group of query rows
 *     (the caller passes the prompt's queries to hkv_prefill_queries);
 *     HKV_PREFILL_CHUNK keeps or evicts whole chunks of consecutive prompt
 *     tokens (a reading of the ChunkKV summary page, with the method's
 *     Hamming score in place of attention; hkv_prefill_chunks).
 *
 * Conventions for every call:
 *   - all device pointers are HIP device memory of the current device; `stream`
 *     is a hipStream_t (NULL = the null stream).  Calls only enqueue work on
 *     `stream` and return; inputs and outputs must stay alive until the work
 *     has completed.  Introspection calls (hkv_get_state, hkv_debug_*) enqueue
 *     copies as well; synchronise the stream before reading their results.
 *   - the caller owns the workspace and every buffer it passes; the handle
 *     owns only host metadata.  R is copied into the workspace at create.
 *   - a handle is not safe for concurrent use from several host threads.
 *   - errors are returned, never thrown.  Arguments are validated before
 *     anything is enqueued, so a call that fails validation has no effect.  A
 *     launch failure poisons the handle: every later call returns
 *     HKV_ERR_STATE.  hkv_last_error() gives a one-line reason.
 *   - debugging (environment, read at hkv_create): HKV_DEBUG=1 synchronises
 *     the stream after every call and reports a device error there;
 *     HKV_DEBUG_NAN=1 fills the per-step partial results (split records,
 *     candidate rows, tier partials) with NaN before every decode step and
 *     tiered attention, so a read of one that the step did not write shows
 *     as NaN in its output.
 *   - host tier (tier_capacity > 0, a reading of the TTKV page's slow DRAM
 *     tier): every token that leaves the cache -- the prompt tokens a prefill
 *     rule does not keep, in position order, then the token each full decode
 *     step evicts, in step order -- is appended to caller-owned tier buffers
 *     (normally pinned host memory) instead of being dropped, and
 *     hkv_attend_tiered attends over the cache and the tier together.
 *   - values (value_bits = 8 or 4, a reading of the DASH-KV page's value
 *     compression): V rows are kept as int8 or 4-bit codes with a per-row
 *     fp32 scale; keys, codes and eviction are unchanged.  Inputs stay kv dtype; the
 *     library quantizes when it stores a row.
 *   - supported: n_bits in {16, 32, 64}; head_dim in {64, 128};
 *     n_q_heads % n_kv_heads == 0 with G = n_q_heads / n_kv_heads <= 16;
 *     kv dtype fp32 or bf16; 1 <= budget <= 2^22 per sequence (a prefill
 *     with HKV_PREFILL_STREAM or HKV_PREFILL_QUERY needs
 *     budget * ceil(b/8) <= 128 KiB: one workgroup holds the head's code
 *     table in its registers);
 *     1 <= batch <= 4096; 1 <= prefill chunk <= 32 tokens.
 */
#ifndef HKV_H
#define HKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    HKV_OK = 0,
    HKV_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misaligned buffer */
    HKV_ERR_UNSUPPORTED = 2,   /* a value outside the supported set above */
    HKV_ERR_STATE = 3,         /* wrong call order, or a poisoned handle */
    HKV_ERR_DEVICE = 4         /* a HIP runtime call failed */
} hkv_status;

enum { HKV_F32 = 0, HKV_BF16 = 1 };                        /* kv_dtype */
enum { HKV_PREFILL_STREAM = 0, HKV_PREFILL_TRUNCATE = 1, HKV_PREFILL_QUERY = 2, HKV_PREFILL_CHUNK = 3 };
/* (prefill_policy) */
/* decode_schedule: FUSED = one launch per step (score, hold-out attention,
 * merge, write); SPLIT = the separate kernels lsh_encode, hamming_argmax,
 * evict_write, split-K attention and LSE merge (five launches). */
enum { HKV_DECODE_FUSED = 0, HKV_DECODE_SPLIT = 1 };

typedef struct {
    int32_t batch;           /* B sequences */
    int32_t n_q_heads;       /* Hq */
    int32_t n_kv_heads;      /* Hkv, divides Hq */
    int32_t head_dim;        /* d */
    int32_t n_bits;          /* b, LSH code length */
    int32_t kv_dtype;        /* HKV_F32 or HKV_BF16: storage of K, V, k, v */
    int32_t prefill_policy;  /* HKV_PREFILL_* */
    int32_t decode_schedule; /* HKV_DECODE_* */
    int32_t max_prompt;      /* largest n_max a prefill will be given (>= 0) */
    int32_t chunk;           /* slots per attention split (one workgroup each);
                                a multiple of 64 in [64, 65536], or 0: about
                                one workgroup per compute unit, i.e.
                                ceil(sum_b S_b * Hkv / 256) rounded up to a
                                multiple of 64 and clamped to [256, 65536].
                                When budgets differ, the fused step cuts
                                sequence b into ceil(S_b / chunk) splits of
                                one length (a multiple of 64, at most chunk)
                                and runs them longest first, and chunk 0
                                picks, from a quarter of that value up to
                                the largest budget, the chunk whose blocks a
                                model of the dispatch (8 XCDs of 32 compute
                                units) finishes first */
    int32_t value_bits;      /* 0: values stored in kv_dtype; 8 or 4: each
                                value row stored as d signed codes of that
                                width and one fp32 scale (Q = 127 or 7:
                                scale = max|v| / Q, code = v / scale rounded
                                half to even, clamped to +-Q, in fp32; the
                                cache holds code * scale; 4-bit codes two a
                                byte, element 2i in the low half of byte i).
                                Needs kv_dtype HKV_BF16 and HKV_DECODE_FUSED */
    int32_t prefill_chunk;   /* tokens per chunk under HKV_PREFILL_CHUNK: 0
                                selects 10, else 1 .. 32; must be 0 under the
                                other policies */
    int32_t tier_capacity;   /* 0: no host tier; else the tokens per (sequence,
                                KV head) a host tier attached with
                                hkv_attach_tier keeps (at most 2^28; needs
                                value_bits 0) */
    const int32_t* budgets;  /* host [batch]: cache slots S_b of each sequence */
} hkv_config;

typedef struct hkv_cache hkv_cache;   /* opaque handle */

/* Host-only checks of a configuration (no GPU needed).  HKV_OK if supported. */
hkv_status hkv_validate_config(const hkv_config* cfg);

/* Device workspace bytes a cache with this configuration needs (host-only).
 * Sizes: K and V caches [B][Hkv][Smax][d] of kv dtype, code table, slot->token
 * map, per-split partial results and the prefill code buffer; Smax = max_b S_b. */
hkv_status hkv_workspace_bytes(const hkv_config* cfg, size_t* bytes);

/* Slots per attention split a cache with this configuration uses: cfg.chunk
 * when it is set, else the default the chunk field describes (host-only).
 * Same status as hkv_validate_config; *chunk is written on HKV_OK. */
hkv_status hkv_config_chunk(const hkv_config* cfg, int32_t* chunk);

/* Create a cache in `workspace` (device, 256-byte aligned, >= the bytes
 * hkv_workspace_bytes reported; owned by the caller and not touched by
 * anyone else while the handle lives).  R_host: host fp32 [head_dim][n_bits]
 * row-major, the Gaussian projection shared by queries and keys (method stage
 * 1); copied.  The cache starts empty.  Synchronises `stream` once. */
hkv_status hkv_create(const hkv_config* cfg, const float* R_host, void* workspace,
                      size_t ws_bytes, void* stream, hkv_cache** out);

/* Fill an empty cache from a prompt.  K, V: device [B][Hkv][n_max][d] kv dtype
 * (row t of sequence b is valid for t < prompt_lens[b]); prompt_lens: host [B],
 * 0 <= prompt_lens[b] <= n_max <= cfg.max_prompt.  Builds the b-bit code of
 * every prompt key (method stages 1-2; an MFMA projection), applies the
 * prefill policy, and leaves occupancy min(N_b, S_b) and next position N_b.
 * HKV_ERR_STATE if the cache is not empty; HKV_ERR_INVALID_ARG under
 * HKV_PREFILL_QUERY or HKV_PREFILL_CHUNK, which take their own entry points
 * (hkv_prefill_queries, hkv_prefill_chunks). */
hkv_status hkv_prefill(hkv_cache* c, const void* K, const void* V, const int32_t* prompt_lens,
                       int32_t n_max, void* stream);

/* Prefill under HKV_PREFILL_QUERY (a cache created with that policy; any
 * other policy gives HKV_ERR_INVALID_ARG).  K, V, prompt_lens, n_max as in
 * hkv_prefill; Q: device fp32 [B][Hq][n_max][d], the query rows of the prompt
 * tokens (16-byte aligned).  Tokens t < S_b take slots 0, 1, ...; every later
 * token t is placed by the decode rule (method stages 1-5): the codes of its
 * G query rows Q[b][h*G + g][t] are projected and sign-packed, the occupied
 * slot with the largest summed Hamming distance to them (ties to the lowest
 * slot) is evicted and token t's key, value and key code take it. */
hkv_status hkv_prefill_queries(hkv_cache* c, const void* K, const void* V, const float* Q,
                               const int32_t* prompt_lens, int32_t n_max, void* stream);

/* Prefill under HKV_PREFILL_CHUNK (a cache created with that policy; any other
 * policy gives HKV_ERR_INVALID_ARG).  Reading of the ChunkKV summary page:
 * prompt tokens are kept or dropped in chunks of C = prefill_chunk
 * consecutive tokens (the last chunk of a prompt may be shorter), and the
 * indices kept for one layer can be reused for other layers.  K, V,
 * prompt_lens, n_max as in hkv_prefill.  With N_b <= S_b every token is kept.
 * Otherwise k = floor(S_b / C) chunks stay.  Chunks are evicted one at a
 * time by the decode rule applied to chunks (method stages 3-4): the chunk
 * whose key codes have the largest summed Hamming distance to the G
 * observation query codes goes first, ties to the lowest chunk.  The kept
 * chunks then fill slots 0, 1, ... in token order.  Occupancy becomes the
 * number of kept tokens (possibly below S_b: decode fills the rest first);
 * next position N_b.
 *   q_obs: device fp32 [B][Hq][d], 16-byte aligned, the observation queries
 *          (normally those of each sequence's last prompt token).  They are
 *          hashed with R (stages 1-2).  Not read when `reuse` is given; may
 *          then be NULL.
 *   reuse: device int32 [B][Hkv][kmax] or NULL.  For a sequence with
 *          N_b > S_b, entries 0 .. floor(S_b / C) - 1 of a head are the chunks
 *          to keep instead of scoring; entries outside [0, ceil(N_b / C)) are
 *          ignored and repeats count once.  Not read for a sequence whose
 *          prompt fits its budget (every token is kept).  Normally
 *          the `kept` output of the same call on another layer's cache with
 *          the same budgets, chunk size and prompt lengths.
 *   kept:  device int32 [B][Hkv][kmax] or NULL; receives the kept chunk
 *          indices of each head in ascending order, then -1.
 * kmax = ceil(Smax / C), Smax the largest budget.  When q_obs is given,
 * hkv_debug_last_codes then returns its codes as qcodes (until the first
 * decode step; kcodes unspecified).  HKV_ERR_INVALID_ARG if both q_obs and
 * reuse are NULL while some prompt exceeds its budget. */
hkv_status hkv_prefill_chunks(hkv_cache* c, const void* K, const void* V, const float* q_obs,
                              const int32_t* reuse, int32_t* kept, const int32_t* prompt_lens,
                              int32_t n_max, void* stream);

/* One decode step for every sequence (method stages 1-5, then attention).
 * q: device fp32 [B][Hq][d]; k, v: device kv dtype [B][Hkv][d], the new token;
 * out: device fp32 [B][Hq][d] = softmax(q K^T / sqrt(d)) V over the cache
 * after the write; evicted_slot: device int32 [B][Hkv], the slot the new token
 * was written to (the evicted one once the cache is full).  State (occupancy,
 * next position) lives on the device, so a sequence of steps can be captured
 * in a HIP graph and replayed.  HKV_ERR_STATE before a prefill. */
hkv_status hkv_decode_step(hkv_cache* c, const float* q, const void* k, const void* v,
                           float* out, int32_t* evicted_slot, void* stream);

/* hkv_decode_step for callers that cannot allocate or pass scratch memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same step, with the same results, but its per-step
 * scratch -- the split records, held-out candidate rows, eviction keys and
 * ticket counters (fused schedule) or split partials (split schedule) --
 * lives in a static device array of the library, 8 MiB per GPU, held until
 * the process ends, instead of the cache's workspace.  Makes no allocation.
 * The array is shared by every call on a GPU and keeps the last call's
 * contents; each call first clears what must start at zero (with a kernel,
 * so the call can be captured in a graph).  Calls that overlap on one GPU
 * (other streams, other host threads, other caches) race on the array and
 * must be serialised by the caller.  HKV_ERR_UNSUPPORTED, with nothing
 * enqueued, when the step would need more than 8 MiB (about
 * B * Hkv * nsplit * (G * d * 4 + G * 16 + d * 4) + B * Hq * nsplit *
 * (d + 4) * 4 bytes, nsplit = ceil(Smax / chunk)).  Otherwise as
 * hkv_decode_step. */
hkv_status hkv_decode_step_static(hkv_cache* c, const float* q, const void* k, const void* v,
                                  float* out, int32_t* evicted_slot, void* stream);

/* Attach the host tier (a cache created with tier_capacity > 0, before its
 * prefill; HKV_ERR_STATE after it, HKV_ERR_INVALID_ARG without a capacity).
 * K, V: [B][Hkv][tier_capacity][d] kv dtype; tok: [B][Hkv][tier_capacity]
 * int32.  All three must be memory the GPU can address: pinned host memory
 * (hipHostMalloc; the GPU reads and writes it over the host link) or device
 * memory; owned by the caller and alive while the handle is used.  Entry j
 * of a (sequence, KV head) holds the j-th token that left its cache (its key
 * row, value row and position); entries past tier_capacity are not stored,
 * but counted.  Tier counts start at 0.  Stream-ordered. */
hkv_status hkv_attach_tier(hkv_cache* c, void* K, void* V, int32_t* tok, void* stream);

/* Tokens sent to the tier so far, per (sequence, KV head): counts [B][Hkv]
 * int32 (device or pinned host memory); may exceed tier_capacity (entries
 * past it were not stored).  HKV_ERR_STATE without an attached tier. */
hkv_status hkv_tier_counts(const hkv_cache* c, int32_t* counts, void* stream);

/* Attention over the cache and its host tier together: out [B][Hq][d] fp32 =
 * softmax(q K^T / sqrt(d)) V over the occupied slots and the stored tier
 * entries of the query head's KV head; q: device fp32 [B][Hq][d] (16-byte
 * aligned).  While no tier has overflowed this is attention over every token
 * seen.  Split-K over both tiers and one LSE merge; the tier is read in place
 * over the host link, every block streaming its rows while it computes.
 * HKV_ERR_STATE before a prefill or without an attached tier. */
hkv_status hkv_attend_tiered(hkv_cache* c, const float* q, float* out, void* stream);

/* Free the handle (host metadata only; the workspace stays the caller's). */
hkv_status hkv_destroy(hkv_cache* c);

const char* hkv_status_str(hkv_status s);
/* Last error detail of this handle ("" if none); c may be NULL (then the
 * detail of the last failed hkv_create / hkv_validate_config of this thread). */
const char* hkv_last_error(const hkv_cache* c);

/* Checkpoint export (device -> caller device buffers; any may be NULL):
 * K, V [B][Hkv][Smax][d] kv dtype; codes [B][Hkv][Smax][W] uint32 with
 * W = ceil(b/32) (unused high bits zero); slot_token [B][Hkv][Smax] int32
 * (-1 = empty slot); head_state [B][Hkv][2] int32 = (occupancy, next position).
 * With value_bits = 8 or 4, V is [B][Hkv][Smax][d * value_bits / 8] bytes of
 * codes (int8, or two 4-bit codes a byte as stored) followed by
 * [B][Hkv][Smax] fp32 scales (B*Hkv*Smax*(d * value_bits / 8 + 4) bytes). */
hkv_status hkv_get_state(const hkv_cache* c, void* K, void* V, uint32_t* codes,
                         int32_t* slot_token, int32_t* head_state, void* stream);
/* Checkpoint import, same layouts; all five buffers required.  Marks the
 * cache as prefilled.  head_state is read back first (the call synchronises
 * `stream` once): HKV_ERR_INVALID_ARG, with nothing enqueued, unless every
 * head has 0 <= occupancy <= its budget and occupancy <= next position.  A
 * host tier is not part of the checkpoint: its buffers are the caller's, and
 * its counts are left as they are. */
hkv_status hkv_set_state(hkv_cache* c, const void* K, const void* V, const uint32_t* codes,
                         const int32_t* slot_token, const int32_t* head_state, void* stream);

/* Codes the last decode step computed: qcodes [B][Hq][W], kcodes [B][Hkv][W]
 * (uint32 device buffers).  After hkv_prefill_chunks with q_obs and before
 * any decode step: the observation query codes, kcodes unspecified.
 * HKV_ERR_STATE before either. */
hkv_status hkv_debug_last_codes(const hkv_cache* c, uint32_t* qcodes, uint32_t* kcodes,
                                void* stream);
/* Codes the last prefill computed for every prompt key:
 * codes [B][Hkv][n_max][W] (uint32 device buffer; rows t >= prompt_lens[b] are
 * unspecified). */
hkv_status hkv_debug_prefill_codes(const hkv_cache* c, uint32_t* codes, void* stream);
/* Codes the last QUERY prefill computed for every prompt query row:
 * codes [B][Hq][n_max][W] (uint32 device buffer; rows t >= prompt_lens[b] are
 * unspecified).  HKV_ERR_STATE unless the last prefill ran with
 * HKV_PREFILL_QUERY. */
hkv_status hkv_debug_prefill_query_codes(const hkv_cache* c, uint32_t* codes, void* stream);
/* GQA Hamming score of every slot against the given query codes
 * qcodes [B][Hq][W] (device): scores [B][Hkv][Smax] int32 (device), -1 for
 * slots at or beyond the occupancy. */
hkv_status hkv_debug_scores(const hkv_cache* c, const uint32_t* qcodes, int32_t* scores,
                            void* stream);

/* Stand-alone encoder (method stages 1-2): codes [n][W] uint32 (device) of the
 * rows X [n][d] (device, fp32 if x_dtype == HKV_F32 else bf16) under the
 * cache's R. */
hkv_status hkv_encode(const hkv_cache* c, const void* X, int32_t x_dtype, int32_t n,
                      uint32_t* codes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* HKV_H */
