/*
 * hkv_oracle.c -- plain, slow, single-threaded fp64 CPU oracle of the
 * HashEvict decode path.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test-suite, the package smoke check
 * and the CPU-baseline leg of the benchmark, never by the GPU library.
 *
 * Each function follows the HashEvict summary page ("HashEvict: A
 * Pre-Attention KV Cache Eviction Strategy using Locality-Sensitive Hashing",
 * arXiv 2412.16187): section "Technical framework", stages 1-5, and the
 * English abstract.  Readings of points the page leaves open are marked
 * READING below.  No blocking, fusion or reordering: every sum runs over its
 * index in ascending order.
 */
#include "hkv_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

struct orc_head {
    int d, nbits, words, budget, group;
    double* R;        /* [d][nbits] */
    double* rnorm;    /* [nbits]  Euclidean norm of column j of R */
    double* K;        /* [budget][d] */
    double* V;        /* [budget][d] */
    uint32_t* code;   /* [budget][words] */
    int64_t* tok;     /* [budget]  token position held by the slot, -1 if empty */
    int n;            /* occupancy: slots 0 .. n-1 hold tokens */
    int64_t t;        /* position of the next token */
    int vbits;        /* 0: values kept as given; 8 or 4: codes of that width with a per-row scale */
    int8_t* vq;       /* [budget][d] value codes, one per element (vbits != 0) */
    float* vs;        /* [budget]    value scales (vbits != 0) */
    int tcap;         /* host tier: capacity in tokens, -1 when there is no tier */
    int64_t tcount;   /* tokens sent to the tier (may exceed tcap; the excess is not kept) */
    double* tK;       /* [tcap][d] */
    double* tV;       /* [tcap][d] */
    int64_t* ttok;    /* [tcap] */
};

int orc_words(const orc_head* h) { return h->words; }

orc_head* orc_create(int d, int n_bits, int budget, int group, const double* R)
{
    if (d <= 0 || n_bits <= 0 || budget < 0 || group <= 0 || !R) return NULL;
    orc_head* h = (orc_head*)calloc(1, sizeof(orc_head));
    h->d = d;
    h->nbits = n_bits;
    h->words = (n_bits + 31) / 32;
    h->budget = budget;
    h->group = group;
    h->R = (double*)malloc(sizeof(double) * (size_t)d * n_bits);
    memcpy(h->R, R, sizeof(double) * (size_t)d * n_bits);
    h->rnorm = (double*)malloc(sizeof(double) * n_bits);
    for (int j = 0; j < n_bits; ++j) {
        double s = 0.0;
        for (int i = 0; i < d; ++i) s += R[(size_t)i * n_bits + j] * R[(size_t)i * n_bits + j];
        h->rnorm[j] = sqrt(s);
    }
    size_t slots = budget > 0 ? (size_t)budget : 1;
    h->K = (double*)calloc(slots * d, sizeof(double));
    h->V = (double*)calloc(slots * d, sizeof(double));
    h->code = (uint32_t*)calloc(slots * h->words, sizeof(uint32_t));
    h->tok = (int64_t*)malloc(slots * sizeof(int64_t));
    for (size_t s = 0; s < slots; ++s) h->tok[s] = -1;
    h->n = 0;
    h->t = 0;
    h->tcap = -1;
    return h;
}

void orc_destroy(orc_head* h)
{
    if (!h) return;
    free(h->R); free(h->rnorm); free(h->K); free(h->V); free(h->code); free(h->tok);
    free(h->vq); free(h->vs);
    free(h->tK); free(h->tV); free(h->ttok);
    free(h);
}

/* Stages 1-2 of the technical framework: Gaussian random projection of the
 * vector to n_bits coordinates, then binarisation.  READING: the
 * binarisation threshold is 0 (a bit is set when the projection is strictly
 * positive) -- the page names the threshold as a design knob without a value,
 * and the sign is the plain binarisation of a Gaussian projection. */
void orc_encode(const orc_head* h, const double* x, uint32_t* code, uint32_t* flag)
{
    double xn = 0.0;
    for (int i = 0; i < h->d; ++i) xn += x[i] * x[i];
    xn = sqrt(xn);
    for (int w = 0; w < h->words; ++w) { code[w] = 0u; flag[w] = 0u; }
    for (int j = 0; j < h->nbits; ++j) {
        double y = 0.0;
        for (int i = 0; i < h->d; ++i) y += x[i] * h->R[(size_t)i * h->nbits + j];
        if (y > 0.0) code[j >> 5] |= 1u << (j & 31);
        if (fabs(y) < 1e-5 * xn * h->rnorm[j]) flag[j >> 5] |= 1u << (j & 31);
    }
}

void orc_encode_many(const orc_head* h, int n, const double* X, uint32_t* codes, uint32_t* flags)
{
    for (int t = 0; t < n; ++t)
        orc_encode(h, X + (size_t)t * h->d, codes + (size_t)t * h->words, flags + (size_t)t * h->words);
}

static int popcount32(uint32_t v) { return __builtin_popcount(v); }

/* Stage 3: Hamming distance between two codes (number of differing bits). */
static int hamming(const uint32_t* a, const uint32_t* b, int words)
{
    int s = 0;
    for (int w = 0; w < words; ++w) s += popcount32(a[w] ^ b[w]);
    return s;
}

/* Stage 3 under grouped-query attention: the score of a slot is the sum of
 * its Hamming distances to the codes of the query heads that share the KV
 * head. */
static int gqa_score(const orc_head* h, const uint32_t* qcodes, int ngroup, int slot)
{
    int s = 0;
    for (int g = 0; g < ngroup; ++g)
        s += hamming(qcodes + (size_t)g * h->words, h->code + (size_t)slot * h->words, h->words);
    return s;
}

/* Stage 4: the slot to evict is the occupied slot whose code is farthest in
 * Hamming distance from the query code(s) -- the most cosine-dissimilar key,
 * hence the lowest expected attention.  READING: ties go to the lowest slot. */
static int pick_victim(const orc_head* h, const uint32_t* qcodes, int ngroup)
{
    int best = -1, e = -1;
    for (int s = 0; s < h->n; ++s) {
        int sc = gqa_score(h, qcodes, ngroup, s);
        if (sc > best) { best = sc; e = s; }
    }
    return e;
}

/* READING of the value compression (the DASH-KV summary page, "Value
 * compression strategy": values tolerate a coarser quantization than keys
 * because the output is their weighted average; it gives no rule, and its
 * introduction names INT8 "or lower").  One row of d values (exact fp32 /
 * bf16 numbers) becomes d signed codes of `bits` bits (8 or 4) and one fp32
 * scale, all in fp32 arithmetic, with Q = 2^(bits-1) - 1 (127 or 7):
 * scale = max_i |v_i| / Q; code_i = v_i / scale rounded to nearest, ties to
 * even, clamped to [-Q, Q]; a zero row has scale 0 and codes 0.  The value
 * the cache holds is code_i * scale. */
void orc_quantize_row(const double* v, int d, int bits, int8_t* q, float* scale)
{
    const float Q = (float)((1 << (bits - 1)) - 1);
    float amax = 0.0f;
    for (int i = 0; i < d; ++i) {
        const float a = fabsf((float)v[i]);
        if (a > amax) amax = a;
    }
    const float sc = amax / Q;
    for (int i = 0; i < d; ++i) {
        float c = 0.0f;
        if (sc > 0.0f) {
            const float x = (float)v[i] / sc;
            c = rintf(x);
            if (c > Q) c = Q;
            if (c < -Q) c = -Q;
        }
        q[i] = (int8_t)c;
    }
    *scale = sc;
}

/* Stage 5: the token's key, value and key code take the slot. */
static void write_slot(orc_head* h, int e, const double* k, const double* v, const uint32_t* kc,
                       int64_t pos)
{
    memcpy(h->K + (size_t)e * h->d, k, sizeof(double) * h->d);
    if (h->vbits != 0) {
        int8_t* q = h->vq + (size_t)e * h->d;
        orc_quantize_row(v, h->d, h->vbits, q, &h->vs[e]);
        for (int i = 0; i < h->d; ++i) h->V[(size_t)e * h->d + i] = (double)q[i] * (double)h->vs[e];
    } else {
        memcpy(h->V + (size_t)e * h->d, v, sizeof(double) * h->d);
    }
    memcpy(h->code + (size_t)e * h->words, kc, sizeof(uint32_t) * h->words);
    h->tok[e] = pos;
}

/* Slot a new token goes to: the lowest empty slot while the cache is not
 * full (READING: nothing is evicted then), else the stage-4 victim. */
static int place(orc_head* h, const uint32_t* qcodes, int ngroup)
{
    if (h->n < h->budget) return h->n++;
    return pick_victim(h, qcodes, ngroup);
}

/* READING of the tiered cache (the TTKV summary page: a fast tier in HBM and
 * a slow tier in host DRAM; recent and important tokens stay fast, older ones
 * go to the slow tier, and attention over the slow tier is streamed in small
 * pieces overlapped with compute).  Here the HBM cache is the fast tier, and
 * every token that leaves it goes to the slow tier instead of being dropped:
 * the prompt tokens a prefill rule does not keep (in ascending position, once
 * the prefill is done) and the token each full decode step evicts (in step
 * order).  An entry is the token's key row, value row and position.  Tokens
 * past the tier's capacity are counted but not kept. */
int orc_set_tier(orc_head* h, int capacity)
{
    if (h->n != 0 || h->t != 0 || capacity < 0 || h->vbits != 0 || h->tcap >= 0) return -1;
    size_t c = capacity > 0 ? (size_t)capacity : 1;
    h->tcap = capacity;
    h->tcount = 0;
    h->tK = (double*)calloc(c * h->d, sizeof(double));
    h->tV = (double*)calloc(c * h->d, sizeof(double));
    h->ttok = (int64_t*)malloc(c * sizeof(int64_t));
    for (size_t j = 0; j < c; ++j) h->ttok[j] = -1;
    return 0;
}

static void tier_push(orc_head* h, const double* k, const double* v, int64_t pos)
{
    if (h->tcap < 0) return;
    if (h->tcount < h->tcap) {
        memcpy(h->tK + (size_t)h->tcount * h->d, k, sizeof(double) * h->d);
        memcpy(h->tV + (size_t)h->tcount * h->d, v, sizeof(double) * h->d);
        h->ttok[h->tcount] = pos;
    }
    h->tcount += 1;
}

/* After a prefill of n prompt tokens: the ones the cache does not hold go to
 * the tier in ascending position. */
static void tier_spill_prompt(orc_head* h, int n, const double* K, const double* V)
{
    if (h->tcap < 0 || n <= 0) return;
    char* held = (char*)calloc((size_t)n, 1);
    for (int s = 0; s < h->n; ++s)
        if (h->tok[s] >= 0 && h->tok[s] < n) held[h->tok[s]] = 1;
    for (int t = 0; t < n; ++t)
        if (!held[t]) tier_push(h, K + (size_t)t * h->d, V + (size_t)t * h->d, (int64_t)t);
    free(held);
}

/* Tier contents: K, V [min(count, capacity)][d], tok [...]; returns the
 * number of tokens sent to the tier, or -1 without a tier. */
int64_t orc_get_tier(const orc_head* h, double* K, double* V, int64_t* tok)
{
    if (h->tcap < 0) return -1;
    const int64_t m = h->tcount < h->tcap ? h->tcount : h->tcap;
    if (K) memcpy(K, h->tK, sizeof(double) * (size_t)m * h->d);
    if (V) memcpy(V, h->tV, sizeof(double) * (size_t)m * h->d);
    if (tok) memcpy(tok, h->ttok, sizeof(int64_t) * (size_t)m);
    return h->tcount;
}

/* Attention over both tiers: softmax(q . k / sqrt(d)) v over the occupied
 * cache slots and the tier's kept entries, max logit subtracted first. */
void orc_attend_tiered(const orc_head* h, const double* q, double* out)
{
    const int64_t m = h->tcap < 0 ? 0 : (h->tcount < h->tcap ? h->tcount : h->tcap);
    const int64_t rows = h->n + m;
    double* lg = (double*)malloc(sizeof(double) * (rows > 0 ? (size_t)rows : 1));
    const double scale = 1.0 / sqrt((double)h->d);
    for (int g = 0; g < h->group; ++g) {
        const double* qg = q + (size_t)g * h->d;
        double* og = out + (size_t)g * h->d;
        double mx = -INFINITY;
        for (int64_t r = 0; r < rows; ++r) {
            const double* kr = r < h->n ? h->K + (size_t)r * h->d : h->tK + (size_t)(r - h->n) * h->d;
            double dot = 0.0;
            for (int i = 0; i < h->d; ++i) dot += qg[i] * kr[i];
            lg[r] = dot * scale;
            if (lg[r] > mx) mx = lg[r];
        }
        double den = 0.0;
        for (int i = 0; i < h->d; ++i) og[i] = 0.0;
        for (int64_t r = 0; r < rows; ++r) {
            const double* vr = r < h->n ? h->V + (size_t)r * h->d : h->tV + (size_t)(r - h->n) * h->d;
            const double p = exp(lg[r] - mx);
            den += p;
            for (int i = 0; i < h->d; ++i) og[i] += p * vr[i];
        }
        for (int i = 0; i < h->d; ++i) og[i] = rows > 0 ? og[i] / den : 0.0;
    }
    free(lg);
}

/* READING of the prefill rule (the page does not describe prefill): STREAM
 * feeds the prompt through the decode rule one token at a time, scoring the
 * cache against the token's own key code because no query accompanies a
 * prompt key; TRUNCATE keeps the first `budget` prompt tokens. */
int orc_prefill(orc_head* h, int policy, int n, const double* K, const double* V,
                const uint32_t* inj_codes)
{
    if (h->n != 0 || n < 0) return -1;
    uint32_t* c = (uint32_t*)malloc(sizeof(uint32_t) * h->words);
    uint32_t* f = (uint32_t*)malloc(sizeof(uint32_t) * h->words);
    for (int t = 0; t < n; ++t) {
        const double* kt = K + (size_t)t * h->d;
        const uint32_t* ct;
        if (inj_codes) {
            ct = inj_codes + (size_t)t * h->words;
        } else {
            orc_encode(h, kt, c, f);
            ct = c;
        }
        int e;
        if (policy == ORC_PREFILL_TRUNCATE) {
            if (h->n >= h->budget) break;
            e = h->n++;
        } else {
            e = place(h, ct, 1);
            if (e < 0) continue;
        }
        write_slot(h, e, kt, V + (size_t)t * h->d, ct, (int64_t)t);
    }
    free(c);
    free(f);
    h->t = n;
    tier_spill_prompt(h, n, K, V);
    return 0;
}

/* Query-driven prefill (READING: the pages do not describe prefill).  Every
 * prompt token past the budget is placed by the decode rule itself: its
 * group's query rows Q[t][g] are hashed (stages 1-2), the occupied slot with
 * the largest summed Hamming distance to them is evicted (stages 3-4, ties to
 * the lowest slot) and the token's key, value and key code take it (stage 5).
 * Tokens before the budget fill slots 0, 1, ... in order.
 * Q: [n][group][d]; inj_codes [n][W] replace E(K[t]); inj_qcodes
 * [n][group][W] replace E(Q[t][g]).  Returns 0, or -1 if the cache is not
 * empty or n < 0. */
int orc_prefill_query(orc_head* h, int n, const double* K, const double* V, const double* Q,
                      const uint32_t* inj_codes, const uint32_t* inj_qcodes)
{
    if (h->n != 0 || n < 0) return -1;
    uint32_t* c = (uint32_t*)malloc(sizeof(uint32_t) * h->words);
    uint32_t* f = (uint32_t*)malloc(sizeof(uint32_t) * h->words);
    uint32_t* qc = (uint32_t*)malloc(sizeof(uint32_t) * h->words * h->group);
    uint32_t* qf = (uint32_t*)malloc(sizeof(uint32_t) * h->words);
    for (int t = 0; t < n; ++t) {
        const double* kt = K + (size_t)t * h->d;
        const uint32_t* ct;
        if (inj_codes) {
            ct = inj_codes + (size_t)t * h->words;
        } else {
            orc_encode(h, kt, c, f);
            ct = c;
        }
        int e;
        if (h->n < h->budget) {
            e = h->n++;
        } else {
            const uint32_t* qcodes;
            if (inj_qcodes) {
                qcodes = inj_qcodes + (size_t)t * h->group * h->words;
            } else {
                for (int g = 0; g < h->group; ++g)
                    orc_encode(h, Q + ((size_t)t * h->group + g) * h->d, qc + (size_t)g * h->words, qf);
                qcodes = qc;
            }
            e = pick_victim(h, qcodes, h->group);
        }
        write_slot(h, e, kt, V + (size_t)t * h->d, ct, (int64_t)t);
    }
    free(c);
    free(f);
    free(qc);
    free(qf);
    h->t = n;
    tier_spill_prompt(h, n, K, V);
    return 0;
}

/* READING of chunk-granular eviction (the ChunkKV summary page: tokens are
 * kept or dropped in groups of consecutive tokens rather than one by one, a
 * chunk of about 10 tokens works best, and the indices kept at one layer can
 * be reused at other layers; the page scores chunks by attention, which the
 * method replaces by its Hamming proxy).  The prompt is cut into chunks of
 * `chunk` consecutive tokens, the last one possibly shorter.  With n <= budget
 * every chunk is kept.  Otherwise floor(budget / chunk) chunks are kept: the
 * decode rule is applied to chunks, evicting one at a time the remaining
 * chunk whose key codes are farthest in summed Hamming distance (over its
 * tokens and the group's observation query codes) from the observation
 * queries, ties to the lowest chunk, until that many remain.  The kept chunks
 * then fill slots 0, 1, ... in token order.
 *
 * qobs [group][d]: the observation queries (those of the token decoding
 * starts from).  inj_codes [n][W] and inj_qcodes [group][W] (may be NULL)
 * replace E's output.  reuse (may be NULL): when n > budget, its first k
 * entries are the chunk indices to keep instead of scoring (k = the count
 * above); entries outside [0, number of chunks) are ignored and repeats count
 * once.  A prompt that fits keeps every token whatever reuse says.  kept (may be
 * NULL): out, [ceil(budget / chunk)] kept chunk indices in ascending order,
 * -1 after the last.  Returns the number of kept chunks, or -1 if the cache
 * is not empty, n < 0 or chunk < 1. */
int orc_prefill_chunks(orc_head* h, int n, int chunk, const double* K, const double* V, const double* qobs,
                       const uint32_t* inj_codes, const uint32_t* inj_qcodes, const int32_t* reuse,
                       int32_t* kept)
{
    if (h->n != 0 || n < 0 || chunk < 1) return -1;
    const int W = h->words;
    const int nch = (n + chunk - 1) / chunk;
    const int k = n <= h->budget ? nch : h->budget / chunk;
    uint32_t* codes = (uint32_t*)malloc(sizeof(uint32_t) * W * (n > 0 ? n : 1));
    uint32_t* f = (uint32_t*)malloc(sizeof(uint32_t) * W);
    char* keep = (char*)calloc(nch > 0 ? nch : 1, 1);
    for (int t = 0; t < n; ++t) {
        if (inj_codes)
            memcpy(codes + (size_t)t * W, inj_codes + (size_t)t * W, sizeof(uint32_t) * W);
        else
            orc_encode(h, K + (size_t)t * h->d, codes + (size_t)t * W, f);
    }
    if (n <= h->budget) {
        for (int i = 0; i < nch; ++i) keep[i] = 1;
    } else if (reuse) {
        for (int j = 0; j < k; ++j)
            if (reuse[j] >= 0 && reuse[j] < nch) keep[reuse[j]] = 1;
    } else {
        uint32_t* qc = (uint32_t*)malloc(sizeof(uint32_t) * W * h->group);
        if (inj_qcodes)
            memcpy(qc, inj_qcodes, sizeof(uint32_t) * W * h->group);
        else
            for (int g = 0; g < h->group; ++g) orc_encode(h, qobs + (size_t)g * h->d, qc + (size_t)g * W, f);
        int* score = (int*)malloc(sizeof(int) * nch);
        for (int i = 0; i < nch; ++i) {
            score[i] = 0;
            for (int t = i * chunk; t < n && t < (i + 1) * chunk; ++t)
                for (int g = 0; g < h->group; ++g)
                    score[i] += hamming(qc + (size_t)g * W, codes + (size_t)t * W, W);
            keep[i] = 1;
        }
        /* stage 4 on chunks, repeated: the farthest remaining chunk goes,
         * the lowest of equals first */
        for (int left = nch; left > k; --left) {
            int best = -1, e = -1;
            for (int i = 0; i < nch; ++i)
                if (keep[i] && score[i] > best) { best = score[i]; e = i; }
            keep[e] = 0;
        }
        free(score);
        free(qc);
    }
    int slot = 0, j = 0;
    for (int i = 0; i < nch; ++i) {
        if (!keep[i]) continue;
        if (kept) kept[j] = i;
        ++j;
        for (int t = i * chunk; t < n && t < (i + 1) * chunk; ++t, ++slot)
            write_slot(h, slot, K + (size_t)t * h->d, V + (size_t)t * h->d, codes + (size_t)t * W, (int64_t)t);
    }
    if (kept)
        for (int r = j; r < (h->budget + chunk - 1) / chunk; ++r) kept[r] = -1;
    h->n = slot;
    h->t = n;
    tier_spill_prompt(h, n, K, V);
    free(codes);
    free(f);
    free(keep);
    return j;
}

/* Attention over the occupied slots: softmax(q . K^T / sqrt(d)) V, with the
 * maximum logit subtracted before exponentiation. */
void orc_attend(const orc_head* h, const double* q, double* out)
{
    double* lg = (double*)malloc(sizeof(double) * (h->n > 0 ? h->n : 1));
    const double scale = 1.0 / sqrt((double)h->d);
    for (int g = 0; g < h->group; ++g) {
        const double* qg = q + (size_t)g * h->d;
        double* og = out + (size_t)g * h->d;
        double m = -INFINITY;
        for (int s = 0; s < h->n; ++s) {
            double dot = 0.0;
            for (int i = 0; i < h->d; ++i) dot += qg[i] * h->K[(size_t)s * h->d + i];
            lg[s] = dot * scale;
            if (lg[s] > m) m = lg[s];
        }
        double den = 0.0;
        for (int i = 0; i < h->d; ++i) og[i] = 0.0;
        for (int s = 0; s < h->n; ++s) {
            double p = exp(lg[s] - m);
            den += p;
            for (int i = 0; i < h->d; ++i) og[i] += p * h->V[(size_t)s * h->d + i];
        }
        for (int i = 0; i < h->d; ++i) og[i] = h->n > 0 ? og[i] / den : 0.0;
    }
    free(lg);
}

/* One decode step: encode the query heads and the new key (stages 1-2),
 * choose the slot (stages 3-4) before any attention is computed, write the
 * new token there (stage 5), then attend over the updated cache. */
int orc_decode_step(orc_head* h, const double* q, const double* k, const double* v,
                    const uint32_t* inj_qcodes, const uint32_t* inj_kcode,
                    double* out, int32_t* evicted,
                    uint32_t* qcodes, uint32_t* qflags, uint32_t* kcode, uint32_t* kflag)
{
    const int W = h->words, G = h->group;
    uint32_t* qc = (uint32_t*)calloc((size_t)G * W, sizeof(uint32_t));
    uint32_t* qf = (uint32_t*)calloc((size_t)G * W, sizeof(uint32_t));
    uint32_t* kc = (uint32_t*)calloc((size_t)W, sizeof(uint32_t));
    uint32_t* kf = (uint32_t*)calloc((size_t)W, sizeof(uint32_t));
    for (int g = 0; g < G; ++g)
        orc_encode(h, q + (size_t)g * h->d, qc + (size_t)g * W, qf + (size_t)g * W);
    orc_encode(h, k, kc, kf);
    if (inj_qcodes) memcpy(qc, inj_qcodes, sizeof(uint32_t) * (size_t)G * W);
    if (inj_kcode) memcpy(kc, inj_kcode, sizeof(uint32_t) * (size_t)W);

    const int was_full = h->n >= h->budget;
    int e = place(h, qc, G);
    /* the evicted token leaves the cache for the tier, if there is one */
    if (e >= 0 && was_full) tier_push(h, h->K + (size_t)e * h->d, h->V + (size_t)e * h->d, h->tok[e]);
    if (e >= 0) write_slot(h, e, k, v, kc, h->t);
    h->t += 1;
    if (out) orc_attend(h, q, out);
    if (evicted) *evicted = e;
    if (qcodes) memcpy(qcodes, qc, sizeof(uint32_t) * (size_t)G * W);
    if (qflags) memcpy(qflags, qf, sizeof(uint32_t) * (size_t)G * W);
    if (kcode) memcpy(kcode, kc, sizeof(uint32_t) * (size_t)W);
    if (kflag) memcpy(kflag, kf, sizeof(uint32_t) * (size_t)W);
    free(qc); free(qf); free(kc); free(kf);
    return e >= 0 ? 0 : -1;
}

void orc_scores(const orc_head* h, const uint32_t* qcodes, int32_t* scores)
{
    for (int s = 0; s < h->budget; ++s)
        scores[s] = s < h->n ? gqa_score(h, qcodes, h->group, s) : -1;
}

/* Store values as 8- or 4-bit codes with a per-row scale (bits = 8 or 4)
 * or as given (bits = 0).  Only on an empty cache; returns 0, or -1. */
int orc_set_value_bits(orc_head* h, int bits)
{
    if (h->n != 0 || (bits != 0 && bits != 8 && bits != 4) || (bits != 0 && h->tcap >= 0)) return -1;
    h->vbits = bits;
    if (bits != 0 && !h->vq) {
        size_t slots = h->budget > 0 ? (size_t)h->budget : 1;
        h->vq = (int8_t*)calloc(slots * h->d, 1);
        h->vs = (float*)calloc(slots, sizeof(float));
    }
    return 0;
}

/* Value codes [budget][d] (one per element, whatever their width) and
 * scales [budget] of a cache with quantized values. */
void orc_get_value_codes(const orc_head* h, int8_t* q, float* scale)
{
    if (h->vbits == 0) return;
    size_t S = (size_t)h->budget;
    if (q) memcpy(q, h->vq, S * h->d);
    if (scale) memcpy(scale, h->vs, S * sizeof(float));
}

/* Restore value codes and scales (the held values become code * scale). */
void orc_set_value_codes(orc_head* h, const int8_t* q, const float* scale)
{
    if (h->vbits == 0) return;
    size_t S = (size_t)h->budget;
    memcpy(h->vq, q, S * h->d);
    memcpy(h->vs, scale, S * sizeof(float));
    for (size_t e = 0; e < S; ++e)
        for (int i = 0; i < h->d; ++i) h->V[e * h->d + i] = (double)h->vq[e * h->d + i] * (double)h->vs[e];
}

void orc_get_state(const orc_head* h, double* K, double* V, uint32_t* code, int64_t* tok,
                   int32_t* occupancy, int64_t* next_pos)
{
    size_t S = (size_t)h->budget;
    if (K) memcpy(K, h->K, sizeof(double) * S * h->d);
    if (V) memcpy(V, h->V, sizeof(double) * S * h->d);
    if (code) memcpy(code, h->code, sizeof(uint32_t) * S * h->words);
    if (tok) memcpy(tok, h->tok, sizeof(int64_t) * S);
    if (occupancy) *occupancy = h->n;
    if (next_pos) *next_pos = h->t;
}

void orc_set_state(orc_head* h, const double* K, const double* V, const uint32_t* code,
                   const int64_t* tok, int32_t occupancy, int64_t next_pos)
{
    size_t S = (size_t)h->budget;
    memcpy(h->K, K, sizeof(double) * S * h->d);
    memcpy(h->V, V, sizeof(double) * S * h->d);
    memcpy(h->code, code, sizeof(uint32_t) * S * h->words);
    memcpy(h->tok, tok, sizeof(int64_t) * S);
    h->n = occupancy;
    h->t = next_pos;
}
