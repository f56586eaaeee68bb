// Drives the host-only configuration checks and workspace layout of libhkv
// (hkv_validate_config, hkv_workspace_bytes, hkv_status_str) over supported
// and unsupported configurations, for a build with AddressSanitizer and
// UndefinedBehaviorSanitizer (test infrastructure: tests/test_sanitizers.py
// builds and runs it).  Prints "ok" and exits 0 when every status is the
// expected one.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "hkv.h"

#define CHECK(cond)                                                       \
    do {                                                                  \
        if (!(cond)) {                                                    \
            std::fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); \
            std::exit(1);                                                 \
        }                                                                 \
    } while (0)

static hkv_config base(const std::vector<int32_t>& budgets)
{
    hkv_config c{};
    c.batch = (int32_t)budgets.size();
    c.n_q_heads = 32;
    c.n_kv_heads = 8;
    c.head_dim = 128;
    c.n_bits = 32;
    c.kv_dtype = HKV_BF16;
    c.prefill_policy = HKV_PREFILL_STREAM;
    c.decode_schedule = HKV_DECODE_FUSED;
    c.max_prompt = 8192;
    c.budgets = budgets.data();
    return c;
}

int main()
{
    std::vector<int32_t> b1{4096}, b2{4096, 100, 7000, 1};
    size_t bytes = 0, bytes2 = 0;
    hkv_config c = base(b1);
    CHECK(hkv_validate_config(&c) == HKV_OK);
    CHECK(hkv_workspace_bytes(&c, &bytes) == HKV_OK && bytes > 0);
    c = base(b2);
    CHECK(hkv_workspace_bytes(&c, &bytes2) == HKV_OK && bytes2 > bytes);
    for (int bits : {16, 32, 64})
        for (int d : {64, 128})
            for (int pol : {HKV_PREFILL_STREAM, HKV_PREFILL_TRUNCATE, HKV_PREFILL_QUERY, HKV_PREFILL_CHUNK})
                for (int sched : {HKV_DECODE_FUSED, HKV_DECODE_SPLIT}) {
                    c = base(b2);
                    c.n_bits = bits;
                    c.head_dim = d;
                    c.prefill_policy = pol;
                    c.decode_schedule = sched;
                    CHECK(hkv_validate_config(&c) == HKV_OK);
                    CHECK(hkv_workspace_bytes(&c, &bytes) == HKV_OK);
                }
    c = base(b1); c.value_bits = 8; CHECK(hkv_validate_config(&c) == HKV_OK);
    c = base(b1); c.value_bits = 8; c.kv_dtype = HKV_F32; CHECK(hkv_validate_config(&c) != HKV_OK);
    c = base(b1); c.tier_capacity = 1 << 20; CHECK(hkv_validate_config(&c) == HKV_OK);
    c = base(b1); c.prefill_policy = HKV_PREFILL_CHUNK; c.prefill_chunk = 32; CHECK(hkv_validate_config(&c) == HKV_OK);
    c = base(b1); c.prefill_policy = HKV_PREFILL_CHUNK; c.prefill_chunk = 33; CHECK(hkv_validate_config(&c) != HKV_OK);
    c = base(b1); c.chunk = 64; CHECK(hkv_validate_config(&c) == HKV_OK);
    c = base(b1); c.chunk = 65; CHECK(hkv_validate_config(&c) != HKV_OK);
    c = base(b1); c.budgets = nullptr; CHECK(hkv_validate_config(&c) == HKV_ERR_INVALID_ARG);
    c = base(b1); c.batch = 0; CHECK(hkv_validate_config(&c) != HKV_OK);
    c = base(b1); c.n_q_heads = 12; CHECK(hkv_validate_config(&c) != HKV_OK);
    c = base(b1); c.n_bits = 24; CHECK(hkv_validate_config(&c) != HKV_OK);
    c = base(b1); c.head_dim = 96; CHECK(hkv_validate_config(&c) != HKV_OK);
    c = base(b1); c.max_prompt = -1; CHECK(hkv_validate_config(&c) != HKV_OK);
    std::vector<int32_t> huge{(1 << 22) + 1}, zero{0}, big{1 << 22};
    c = base(huge); CHECK(hkv_validate_config(&c) != HKV_OK);
    c = base(zero); CHECK(hkv_validate_config(&c) != HKV_OK);
    c = base(big); CHECK(hkv_validate_config(&c) != HKV_OK);   // STREAM table limit
    c = base(big); c.prefill_policy = HKV_PREFILL_TRUNCATE; CHECK(hkv_workspace_bytes(&c, &bytes) == HKV_OK);
    CHECK(hkv_validate_config(nullptr) == HKV_ERR_INVALID_ARG);
    CHECK(hkv_workspace_bytes(&c, nullptr) == HKV_ERR_INVALID_ARG);
    for (int s = -1; s <= 5; ++s) CHECK(hkv_status_str((hkv_status)s) != nullptr);
    std::printf("ok\n");
    return 0;
}
