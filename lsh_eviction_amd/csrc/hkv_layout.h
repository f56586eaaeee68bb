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
// Dispatch model of the fused decode step with ragged budgets (default chunk):
// workgroups go to the XCDs round-robin by number and, within one, to the
// first compute unit that is free; a block costs its slots plus a fixed
// amount (prologue, publish, merge), fitted to measured steps.
constexpr int kXcds = 8;
constexpr int kCusPerXcd = 32;
constexpr int kBlockFixedSlots = 512;
constexpr int kAutoChunkCandidates = 128;   // chunks the model compares
constexpr long long kAutoChunkMaxBlocks = 16384;   // ... each with at most this many blocks
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
    int nblk;              // fused decode blocks per KV head when budgets differ (the block list), else 0
    size_t code_slots;     // slots per head in the code table (padded)
    size_t pcode_slots;    // prompt positions per head in the prefill code buffer (padded)
    // byte offsets into the workspace
    size_t off_R, off_budget, off_plen, off_state, off_K, off_V, off_code, off_tok;
    size_t off_dbg_q, off_dbg_k, off_part, off_frec, off_fscal, off_cand_v, off_ekey;
    size_t off_info, off_count, off_pcode, off_qcode, off_vs, off_csum;
    size_t off_tcount, off_tpart, off_tflag, off_chist, off_blk;
    size_t v_bytes;        // bytes of the V region (kv dtype, or codes of value_bits bits)
    size_t total;
};

// Fills `lay` and returns HKV_OK, or an error code with a reason in `err`.
hkv_status compute_layout(const hkv_config* cfg, Layout* lay, char* err, size_t errlen);

// The block list of the fused decode step when budgets differ.  Sequence b
// is cut into splits of one length, ceil(S_b / k) rounded up to a multiple
// of 64 with k = ceil(S_b / chunk), so none of its blocks outlives the
// others; every split of every sequence is one block, and the list runs
// from the split with the most slots to the one with the fewest (ties in
// sequence and split order), so the compute units that finish early pick
// up the short blocks.  Writes two words per block to `out` when it is not
// null, (b | split << 16, the sequence's split length; its last split may
// hold fewer slots), and returns the number of blocks (at most
// sum_b ceil(S_b / chunk)).
int fused_block_order(const int32_t* budgets, int B, int chunk, uint32_t* out);

// Finish time of that block list for Hkv heads under the dispatch model
// above, in slots' worth of one compute unit's streaming.
long long fused_makespan(const int32_t* budgets, int B, int Hkv, int chunk);

// Default chunk with ragged budgets: among multiples of 64 from a quarter
// of `base` (the one-block-per-compute-unit chunk) to the largest budget,
// at most kAutoChunkCandidates of them, the one whose block list the model
// finishes first (the largest of equals).
int ragged_auto_chunk(const int32_t* budgets, int B, int Hkv, int base);

}  // namespace hkv
