// hkv_layout.h -- host-side configuration checks and the workspace layout.
// Host-only: no HIP types, so the validation can be compiled and tested
// without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>

#include "hkv.h"
#include "hkv_consts.h"

namespace hkv {

constexpr int kMaxBudget = 1 << 22;
constexpr int kMaxBatch = 4096;
constexpr size_t kLdsTableBytes = 128 * 1024;   // code table of the sequential prefill selection (registers of one block)
constexpr int kChunkTargetBlocks = 256;   // default split: about one decode block per compute unit of the part
constexpr int kMinAutoChunk = 256;        // ... but at least this many slots per block
constexpr int kDefaultPrefillChunk = 10;   // tokens per prefill chunk (HKV_PREFILL_CHUNK)
constexpr int kMaxPrefillChunk = 32;
constexpr int kMaxTierCapacity = 1 << 28;
constexpr int kTierBlocks = 2048;   // tier attention: splits per head = this / heads, in [1, 256]
constexpr size_t kAlign = 256;

struct Layout {
    int B, Hq, Hkv, G, d, bits, W, cb, es;   // cb: code bytes, es: kv element bytes
    int kv_dtype, prefill_policy, schedule, value_bits;
    int Smax, chunk, nsplit, max_prompt;
    int pchunk;            // tokens per prefill chunk (HKV_PREFILL_CHUNK), else 0
    size_t nchunk_max;     // prompt chunks per head, padded (HKV_PREFILL_CHUNK)
    int chist_bins;        // possible chunk scores, C * G * b + 1 (HKV_PREFILL_CHUNK)
    int tcap;              // host tier capacity per head (0: none)
    int tsplit;            // splits per head of the tiered attention over the host tier
    size_t tflag_words;    // words per head of the prompt's held-token bitset
    size_t code_slots;     // slots per head in the code table (padded)
    size_t pcode_slots;    // prompt positions per head in the prefill code buffer (padded)
    // byte offsets into the workspace
    size_t off_R, off_budget, off_plen, off_state, off_K, off_V, off_code, off_tok;
    size_t off_dbg_q, off_dbg_k, off_part, off_frec, off_fscal, off_cand_v, off_ekey;
    size_t off_info, off_count, off_pcode, off_qcode, off_vs, off_csum;
    size_t off_tcount, off_tpart, off_tflag, off_chist;
    size_t v_bytes;        // bytes of the V region (kv dtype, or int8 codes)
    size_t total;
};

// Fills `lay` and returns HKV_OK, or an error code with a reason in `err`.
hkv_status compute_layout(const hkv_config* cfg, Layout* lay, char* err, size_t errlen);

}  // namespace hkv
