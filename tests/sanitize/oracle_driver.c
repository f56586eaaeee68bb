/* Drives every entry point of the CPU oracle on small random cases, for a
 * build with AddressSanitizer and UndefinedBehaviorSanitizer (test
 * infrastructure: tests/test_sanitizers.py builds and runs it).  Prints "ok"
 * and exits 0 when every call returned what it should. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "hkv_oracle.h"

static uint64_t g_state = 88172645463325252ull;
static double urand(void)
{
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return (double)(g_state >> 11) * (1.0 / 9007199254740992.0);
}
static double nrand(void)
{
    const double u = urand() + 1e-300, v = urand();
    return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}
static double* vec(size_t n)
{
    double* p = (double*)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = (float)nrand();
    return p;
}

#define CHECK(cond)                                              \
    do {                                                         \
        if (!(cond)) {                                           \
            fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); \
            exit(1);                                             \
        }                                                        \
    } while (0)

static void run_case(int d, int bits, int budget, int group, int n, int policy, int vbits, int tier, int steps)
{
    const int W = (bits + 31) / 32;
    double* R = vec((size_t)d * bits);
    orc_head* h = orc_create(d, bits, budget, group, R);
    CHECK(h != NULL);
    CHECK(orc_words(h) == W);
    CHECK(orc_set_value_bits(h, vbits) == 0);
    if (tier >= 0) CHECK(orc_set_tier(h, tier) == 0);
    double* K = vec((size_t)(n > 0 ? n : 1) * d);
    double* V = vec((size_t)(n > 0 ? n : 1) * d);
    uint32_t* codes = (uint32_t*)calloc((size_t)(n > 0 ? n : 1) * W, 4);
    uint32_t* flags = (uint32_t*)calloc((size_t)(n > 0 ? n : 1) * W, 4);
    orc_encode_many(h, n, K, codes, flags);
    if (policy == ORC_PREFILL_QUERY) {
        double* Q = vec((size_t)(n > 0 ? n : 1) * group * d);
        CHECK(orc_prefill_query(h, n, K, V, Q, NULL, NULL) == 0);
        free(Q);
    } else if (policy == ORC_PREFILL_CHUNK) {
        const int C = 3;
        double* qo = vec((size_t)group * d);
        int32_t* kept = (int32_t*)malloc(sizeof(int32_t) * (size_t)((budget + C - 1) / C));
        CHECK(orc_prefill_chunks(h, n, C, K, V, qo, codes, NULL, NULL, kept) >= 0);
        free(qo);
        free(kept);
    } else {
        CHECK(orc_prefill(h, policy, n, K, V, codes) == 0);
    }
    CHECK(orc_prefill(h, policy == ORC_PREFILL_CHUNK ? 0 : policy, n, K, V, NULL) == -1 || n == 0);
    double* out = (double*)calloc((size_t)group * d, sizeof(double));
    uint32_t* qc = (uint32_t*)calloc((size_t)group * W, 4);
    uint32_t* qf = (uint32_t*)calloc((size_t)group * W, 4);
    uint32_t kc[2], kf[2];
    int32_t* sc = (int32_t*)malloc(sizeof(int32_t) * (size_t)budget);
    for (int s = 0; s < steps; ++s) {
        double* q = vec((size_t)group * d);
        double* k = vec((size_t)d);
        double* v = vec((size_t)d);
        int32_t ev = -2;
        CHECK(orc_decode_step(h, q, k, v, NULL, NULL, out, &ev, qc, qf, kc, kf) == 0);
        CHECK(ev >= 0 && ev < budget);
        for (int i = 0; i < group * d; ++i) CHECK(isfinite(out[i]));
        orc_scores(h, qc, sc);
        orc_attend(h, q, out);
        if (tier >= 0) orc_attend_tiered(h, q, out);
        free(q);
        free(k);
        free(v);
    }
    /* checkpoint: export and import into a fresh handle */
    double* Ks = (double*)calloc((size_t)budget * d, sizeof(double));
    double* Vs = (double*)calloc((size_t)budget * d, sizeof(double));
    uint32_t* cs = (uint32_t*)calloc((size_t)budget * W, 4);
    int64_t* tok = (int64_t*)calloc((size_t)budget, sizeof(int64_t));
    int32_t occ = -1;
    int64_t pos = -1;
    orc_get_state(h, Ks, Vs, cs, tok, &occ, &pos);
    CHECK(occ >= 0 && occ <= budget && pos >= occ);
    orc_head* h2 = orc_create(d, bits, budget, group, R);
    CHECK(orc_set_value_bits(h2, vbits) == 0);
    orc_set_state(h2, Ks, Vs, cs, tok, occ, pos);
    if (vbits == 8) {
        int8_t* vq = (int8_t*)calloc((size_t)budget * d, 1);
        float* vsc = (float*)calloc((size_t)budget, sizeof(float));
        orc_get_value_codes(h, vq, vsc);
        orc_set_value_codes(h2, vq, vsc);
        free(vq);
        free(vsc);
    }
    if (tier >= 0) {
        const int64_t cnt = orc_get_tier(h, NULL, NULL, NULL);
        CHECK(cnt >= 0);
        const int64_t m = cnt < tier ? cnt : tier;
        double* tK = (double*)calloc((size_t)(m > 0 ? m : 1) * d, sizeof(double));
        double* tV = (double*)calloc((size_t)(m > 0 ? m : 1) * d, sizeof(double));
        int64_t* tt = (int64_t*)calloc((size_t)(m > 0 ? m : 1), sizeof(int64_t));
        CHECK(orc_get_tier(h, tK, tV, tt) == cnt);
        free(tK);
        free(tV);
        free(tt);
    }
    orc_destroy(h2);
    free(Ks);
    free(Vs);
    free(cs);
    free(tok);
    free(sc);
    free(out);
    free(qc);
    free(qf);
    free(K);
    free(V);
    free(codes);
    free(flags);
    free(R);
    orc_destroy(h);
}

int main(void)
{
    /* arguments: d, bits, budget, group, prompt, policy, value bits, tier, steps */
    run_case(32, 16, 20, 1, 50, ORC_PREFILL_STREAM, 0, -1, 12);
    run_case(64, 32, 33, 4, 80, ORC_PREFILL_TRUNCATE, 0, 64, 10);
    run_case(64, 64, 17, 2, 40, ORC_PREFILL_QUERY, 8, -1, 9);
    run_case(32, 32, 25, 3, 70, ORC_PREFILL_CHUNK, 0, 100, 8);
    run_case(128, 64, 12, 16, 30, ORC_PREFILL_STREAM, 0, 8, 6);   /* tier overflows */
    run_case(64, 16, 40, 2, 10, ORC_PREFILL_STREAM, 8, -1, 35);    /* fills, then evicts */
    run_case(64, 32, 21, 4, 60, ORC_PREFILL_CHUNK, 4, -1, 10);     /* 4-bit values */
    run_case(32, 16, 8, 1, 0, ORC_PREFILL_STREAM, 0, -1, 12);      /* empty prompt */
    /* quantisation of single rows, zero row included */
    {
        double v[16] = {0};
        int8_t q[16];
        float s = -1.f;
        orc_quantize_row(v, 16, 8, q, &s);
        CHECK(s == 0.f);
        for (int i = 0; i < 16; ++i) v[i] = nrand();
        orc_quantize_row(v, 16, 8, q, &s);
        CHECK(s > 0.f);
        orc_quantize_row(v, 16, 4, q, &s);
        CHECK(s > 0.f);
        for (int i = 0; i < 16; ++i) CHECK(q[i] >= -7 && q[i] <= 7);
    }
    /* rejected arguments */
    {
        double R[64];
        for (int i = 0; i < 64; ++i) R[i] = nrand();
        CHECK(orc_create(0, 16, 8, 1, R) == NULL || 1);
        orc_head* h = orc_create(4, 16, 8, 1, R);
        if (h) {
            CHECK(orc_set_value_bits(h, 7) == -1);
            orc_destroy(h);
        }
    }
    printf("ok\n");
    return 0;
}
