/*
 * hkv_oracle.h -- plain, slow, single-threaded CPU oracle of the HashEvict
 * decode path (test infrastructure).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and
 * the CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or helper with the GPU library and the GPU library never
 * calls it.
 *
 * Source of the method: "HashEvict: A Pre-Attention KV Cache Eviction
 * Strategy using Locality-Sensitive Hashing" (arXiv 2412.16187, summary page),
 * sections "Technical framework" (the five stages: Gaussian projection,
 * binarisation, Hamming distance, eviction decision, dynamic in-place update)
 * and the English abstract (query code against cached key codes, decision made
 * before attention, the current token replaces the evicted one at every decode
 * step, a binary code table kept in GPU memory).
 *
 * One handle is one eviction domain: the cache of one (sequence, KV head)
 * pair, attended by the `group` query heads that share that KV head.
 * All arithmetic is fp64; K/V are passed already widened to double (bf16 and
 * fp32 inputs are exactly representable).
 *
 * Codes: W = ceil(n_bits / 32) uint32 words per code, bit j of the code is bit
 * (j mod 32) of word j / 32 (LSB first).  Unused high bits are zero.
 */
#ifndef HKV_ORACLE_H
#define HKV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct orc_head orc_head;

enum { ORC_PREFILL_STREAM = 0, ORC_PREFILL_TRUNCATE = 1, ORC_PREFILL_QUERY = 2, ORC_PREFILL_CHUNK = 3 };

/* R: [d][n_bits] fp32 values widened to double; copied. NULL on bad args. */
orc_head* orc_create(int d, int n_bits, int budget, int group, const double* R);
void orc_destroy(orc_head* h);

/* E: project x (length d), sign-binarise, pack.  flag bit j is set when
 * |y_j| < 1e-5 * ||x|| * ||R[:, j]|| (a sign too close to call in fp32). */
void orc_encode(const orc_head* h, const double* x, uint32_t* code, uint32_t* flag);
/* E over n vectors X[n][d] -> codes[n][W], flags[n][W]. */
void orc_encode_many(const orc_head* h, int n, const double* X, uint32_t* codes, uint32_t* flags);

/* P: prefill from an empty cache with the prompt K[n][d], V[n][d].
 * inj_codes (may be NULL): [n][W] codes used instead of E(K[t]).
 * Returns 0 on success, -1 if the cache is not empty or n < 0. */
int orc_prefill(orc_head* h, int policy, int n, const double* K, const double* V,
                const uint32_t* inj_codes);

/* P with the QUERY rule: tokens past the budget evict by the decode rule,
 * scored against their own group's query rows.  Q: [n][group][d];
 * inj_codes [n][W] and inj_qcodes [n][group][W] (may be NULL) replace the
 * key and query codes.  Returns 0, or -1 if the cache is not empty or n < 0. */
int orc_prefill_query(orc_head* h, int n, const double* K, const double* V, const double* Q,
                      const uint32_t* inj_codes, const uint32_t* inj_qcodes);

/* P with chunk-granular eviction (a reading; see the .c file): the prompt
 * is cut into chunks of `chunk` consecutive tokens; with n > budget only
 * floor(budget / chunk) whole chunks stay, the others evicted one at a time
 * by the decode rule applied to chunks (summed Hamming distance of a chunk's
 * key codes to the observation query codes, ties to the lowest chunk); kept
 * chunks fill slots 0, 1, ... in token order.  qobs [group][d];
 * inj_codes [n][W], inj_qcodes [group][W], reuse [k] (kept chunks given
 * instead of scored when n > budget) may be NULL; kept (may be NULL) receives
 * [ceil(budget / chunk)] kept chunk indices, ascending, -1 after the last.
 * Returns the number of kept chunks, or -1 (cache not empty, n < 0,
 * chunk < 1). */
int orc_prefill_chunks(orc_head* h, int n, int chunk, const double* K, const double* V, const double* qobs,
                       const uint32_t* inj_codes, const uint32_t* inj_qcodes, const int32_t* reuse,
                       int32_t* kept);

/* Host tier (a reading; see the .c file): tokens leaving the cache -- the
 * prompt tokens a prefill does not keep, in ascending position, then each
 * token a full decode step evicts -- are kept in a tier of `capacity` tokens
 * instead of being dropped.  Only on an empty cache with values as given;
 * returns 0, or -1. */
int orc_set_tier(orc_head* h, int capacity);
/* Tier contents K, V [min(count, capacity)][d], tok [...] (any may be NULL);
 * returns the number of tokens sent to the tier, -1 without a tier. */
int64_t orc_get_tier(const orc_head* h, double* K, double* V, int64_t* tok);
/* Attention over the cache and the tier's kept tokens: out [group][d]. */
void orc_attend_tiered(const orc_head* h, const double* q, double* out);

/* Value compression (a reading; see the .c file): bits = 8 or 4 stores every
 * value row as signed codes of that width with one fp32 scale (fp32
 * arithmetic, Q = 127 or 7: scale = max|v| / Q, code = round-half-even(v /
 * scale) clamped to +-Q) and the cache then holds code * scale; bits = 0
 * stores values as given.  Only on an empty cache; returns 0, or -1. */
int orc_set_value_bits(orc_head* h, int bits);
/* The rule on one row at the given width: q [d] codes, *scale. */
void orc_quantize_row(const double* v, int d, int bits, int8_t* q, float* scale);
/* Codes [budget][d] (one int8 per element) and scales [budget] of a cache
 * with quantized values (export, import; import sets the held values to
 * code * scale). */
void orc_get_value_codes(const orc_head* h, int8_t* q, float* scale);
void orc_set_value_codes(orc_head* h, const int8_t* q, const float* scale);

/* D + A: one decode step.  q: [group][d], k, v: [d].
 * inj_qcodes [group][W] / inj_kcode [W] (may be NULL) replace E's output.
 * Outputs (may be NULL): out [group][d], evicted slot, the codes and flags used. */
int orc_decode_step(orc_head* h, const double* q, const double* k, const double* v,
                    const uint32_t* inj_qcodes, const uint32_t* inj_kcode,
                    double* out, int32_t* evicted,
                    uint32_t* qcodes, uint32_t* qflags, uint32_t* kcode, uint32_t* kflag);

/* GQA Hamming score of every occupied slot against qcodes [group][W];
 * scores[s] for s < occupancy, -1 beyond. */
void orc_scores(const orc_head* h, const uint32_t* qcodes, int32_t* scores);

/* A alone over the current cache: out [group][d] for q [group][d]. */
void orc_attend(const orc_head* h, const double* q, double* out);

/* state export / import (checkpoint).  K, V: [budget][d]; code [budget][W];
 * tok [budget] (-1 for an empty slot); occupancy; next token position. */
void orc_get_state(const orc_head* h, double* K, double* V, uint32_t* code, int64_t* tok,
                   int32_t* occupancy, int64_t* next_pos);
void orc_set_state(orc_head* h, const double* K, const double* V, const uint32_t* code,
                   const int64_t* tok, int32_t occupancy, int64_t next_pos);

int orc_words(const orc_head* h);

#ifdef __cplusplus
}
#endif
#endif
