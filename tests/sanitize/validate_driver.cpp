// Drives the host-only configuration checks and workspace layout of libhkv
// (hkv_validate_config, hkv_workspace_bytes, hkv_status_str) over supported
// and unsupported configurations, and the block list of the fused decode
// step for ragged budgets (hkv::fused_block_order), for a build with
// AddressSanitizer and UndefinedBehaviorSanitizer (test infrastructure:
// tests/test_sanitizers.py builds and runs it).  Prints "ok" and exits 0
// when every status is the expected one and every block list is valid.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "hkv.h"
#include "hkv_layout.h"

#define CHECK(cond)                                                       \
    do {                                                                  \
        if (!(cond)) {                                                    \
            std::fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); \
            std::exit(1);                                                 \
        }                                                                 \
    } while (0)

// Every split of every sequence exactly once, the splits of a sequence of
// one length (a multiple of 64, at most the chunk, no more of them than
// ceil(S_b / chunk) and covering S_b with less than one split to spare),
// listed by slots, most first.
static void check_block_list(const std::vector<int32_t>& budgets, int chunk)
{
    const int B = (int)budgets.size();
    const int n = hkv::fused_block_order(budgets.data(), B, chunk, nullptr);
    std::vector<uint32_t> out((size_t)n * 2 + 2, 0xDEADBEEFu);
    CHECK(hkv::fused_block_order(budgets.data(), B, chunk, out.data()) == n);
    CHECK(out[2 * n] == 0xDEADBEEFu && out[2 * n + 1] == 0xDEADBEEFu);
    std::vector<int> len(B, 0), seen_count(B, 0);
    std::vector<std::vector<int>> seen(B);
    int prev_rows = 1 << 30;
    for (int i = 0; i < n; ++i) {
        const int b = (int)(out[2 * i] & 0xFFFFu), j = (int)(out[2 * i] >> 16), l = (int)out[2 * i + 1];
        CHECK(b >= 0 && b < B);
        const int S = budgets[b];
        CHECK(l > 0 && l % 64 == 0 && l <= chunk);
        CHECK(len[b] == 0 || len[b] == l);
        len[b] = l;
        const int k = (S + l - 1) / l;
        CHECK(j >= 0 && j < k && k <= (S + chunk - 1) / chunk);
        if (seen[b].empty()) seen[b].assign(k, 0);
        CHECK(seen[b][j] == 0);
        seen[b][j] = 1;
        ++seen_count[b];
        const int rows = l < S - j * l ? l : S - j * l;
        CHECK(rows > 0 && rows <= prev_rows);
        prev_rows = rows;
        const int k0 = (S + chunk - 1) / chunk;
        CHECK(l - 64 < (S + k0 - 1) / k0 && (S + k0 - 1) / k0 <= l);
    }
    for (int b = 0; b < B; ++b) CHECK(seen_count[b] == (int)seen[b].size() && seen_count[b] > 0);
}

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
    // block lists: fixed cases, then seeded random batches
    check_block_list({4096, 100, 7000, 1}, 256);
    check_block_list({7854, 2092, 4800, 4801, 9600}, 4800);
    check_block_list({64, 65, 127, 128, 129}, 64);
    check_block_list({1 << 22, 3}, 65536);
    uint64_t st = 0x9E3779B97F4A7C15ull;
    auto next = [&st]() {
        st = st * 6364136223846793005ull + 1442695040888963407ull;
        return (uint32_t)(st >> 33);
    };
    for (int t = 0; t < 200; ++t) {
        std::vector<int32_t> bud(1 + next() % 40);
        for (auto& x : bud) x = 1 + (int32_t)(next() % 20000);
        check_block_list(bud, 64 * (1 + (int)(next() % 128)));
    }
    // dispatch model: closed forms, then the default chunk of a ragged batch
    std::vector<int32_t> two{640, 576}, many(33, 64);
    CHECK(hkv::fused_makespan(two.data(), 2, 8, 640) == 640 + hkv::kBlockFixedSlots);
    CHECK(hkv::fused_makespan(many.data(), 33, 8, 64) == 2 * (64 + hkv::kBlockFixedSlots));
    std::vector<int32_t> rag{7854, 2092, 4800, 4801, 9600, 3000, 6100, 2500};
    {
        c = base(rag);
        hkv::Layout L;
        char err[256];
        CHECK(hkv::compute_layout(&c, &L, err, sizeof(err)) == HKV_OK);
        long long slots = 0;
        for (int32_t x : rag) slots += x;
        const int plain = (int)((slots * 8 + 255) / 256 + 63) / 64 * 64;
        CHECK(L.chunk % 64 == 0 && L.chunk >= 256 && L.chunk <= 65536);
        CHECK(hkv::fused_makespan(rag.data(), (int)rag.size(), 8, L.chunk) <=
              hkv::fused_makespan(rag.data(), (int)rag.size(), 8, plain));
        CHECK(L.nblk == hkv::fused_block_order(rag.data(), (int)rag.size(), L.chunk, nullptr));
        c.chunk = 1024;   // an explicit chunk is kept
        CHECK(hkv::compute_layout(&c, &L, err, sizeof(err)) == HKV_OK && L.chunk == 1024);
    }
    // the layout reserves the list only when budgets differ
    std::vector<int32_t> eq{5000, 5000}, ne{5000, 5001};
    size_t beq = 0, bne = 0;
    c = base(eq); CHECK(hkv_workspace_bytes(&c, &beq) == HKV_OK);
    c = base(ne); CHECK(hkv_workspace_bytes(&c, &bne) == HKV_OK);
    CHECK(bne > beq);
    std::printf("ok\n");
    return 0;
}
