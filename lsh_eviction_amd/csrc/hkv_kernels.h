// hkv_kernels.h -- device-side view of a cache and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace hkv {

// Pointers into the caller's workspace plus the sizes every kernel needs.
struct DevCache {
    const float* R;                 // [d][bits] fp32
    const int* budget;              // [B]
    const int* plen;                // [B] prompt lengths of the last prefill
    int* state;                     // [B][Hkv][2]: occupancy, next position
    void* K;                        // [B][Hkv][Smax][d] kv dtype
    void* V;
    void* code;                     // [B][Hkv][code_slots] codes of cb bytes
    int* tok;                       // [B][Hkv][Smax] token held by a slot, -1 empty
    uint32_t* dbg_q;                // [B][Hq][W] query codes of the last step
    uint32_t* dbg_k;                // [B][Hkv][W] key codes of the last step
    float* part;                    // [B][Hq][nsplit][d + 4]: acc[d], m, l
    float* frec;                    // [B][Hkv][nsplit][G][d] fused-step partial acc of each split
    float* fscal;                   // [B][Hkv][nsplit][G][4] (max, sum, candidate logit, 0), base 2
    float* cand_v;                  // [B][Hkv][nsplit][d] value row of the split's candidate (fp32)
    unsigned long long* ekey;       // [B][Hkv][2] eviction key of the step, by parity of its position
    int* info;                      // [B][Hkv][2] occupancy and position at the start of the step
    unsigned* count;                // [B][Hkv][kCountStride] blocks of the current step that have published (entry 0)
    void* pcode;                    // [B][Hkv][pcode_slots] prompt key codes
    void* qcode;                    // [B][Hq][pcode_slots] prompt query codes (QUERY prefill)
    float* vs;                      // [B][Hkv][Smax] (+16) value scales when values are stored as codes
    int B, Hq, Hkv, G, d, bits, W, Smax, chunk, nsplit;
    int ragged;                     // budgets differ: the fused step runs the block list `blk`
    const uint2* blk;               // [nblk] (b | split << 16, split length) of each fused block, longest first
    int nblk;
    int vbits;                      // values stored as given (0), or as 8- or 4-bit codes + scales
    int kv_bf16;
    long long code_slots, pcode_slots;
    int* csum;                      // [B][Hkv][nchunk_max] per-chunk scores or flags (CHUNK prefill)
    int pchunk;                     // tokens per prefill chunk (CHUNK prefill)
    long long nchunk_max;
    int* chist;                     // [B][Hkv][chist_bins] histogram of chunk scores (CHUNK prefill)
    int chist_bins;                 // C * G * b + 1: every possible chunk score
    // host tier (null tK when none is attached)
    void* tK;                       // [B][Hkv][tcap][d] kv dtype, GPU-addressable (pinned host or device)
    void* tV;
    int* ttok;                      // [B][Hkv][tcap] token positions
    int* tcount;                    // [B][Hkv] tokens sent to the tier (device)
    float* tpart;                   // [B][Hq][tsplit][d + 4] partials of the tiered attention
    unsigned* tflag;                // [B][Hkv][tflag_words] prompt tokens the cache holds (prefill spill)
    int tcap, tsplit;
    long long tflag_words;
};

// decode, fused schedule: one launch
hipError_t launch_decode_fused(const DevCache& c, const float* q, const void* k, const void* v,
                               float* out, int* evicted, hipStream_t st);
// decode, split schedule: lsh_encode, hamming_argmax, evict_write, attention, merge
hipError_t launch_decode_split(const DevCache& c, const float* q, const void* k, const void* v,
                               float* out, int* evicted, hipStream_t st);
hipError_t launch_scores(const DevCache& c, const uint32_t* qcodes, int* scores, hipStream_t st);
hipError_t launch_encode_rows(const DevCache& c, const void* X, int x_bf16, int n,
                              uint32_t* codes, hipStream_t st);

// prefill
hipError_t launch_reset(const DevCache& c, hipStream_t st);
hipError_t launch_prefill(const DevCache& c, const void* K, const void* V, const float* Q, int n_max, int policy,
                          hipStream_t st);
// CHUNK prefill: q_obs [B][Hq][d] fp32 (may be null with reuse), reuse / kept [B][Hkv][kmax] (may be null)
hipError_t launch_prefill_chunks(const DevCache& c, const void* K, const void* V, const float* q_obs,
                                 const int* reuse, int* kept, int kmax, int n_max, hipStream_t st);
// host tier: prefill spill (after the gather) and attention over cache + tier
hipError_t launch_tier_spill_prompt(const DevCache& c, const void* K, const void* V, int n_max, hipStream_t st);
hipError_t launch_attend_tiered(const DevCache& c, const float* q, float* out, hipStream_t st);
// checkpoint
hipError_t launch_export_codes(const DevCache& c, uint32_t* codes, hipStream_t st);
hipError_t launch_import_codes(const DevCache& c, const uint32_t* codes, hipStream_t st);
hipError_t launch_export_pcodes(const DevCache& c, uint32_t* codes, int n_max, bool queries, hipStream_t st);
// clears the per-step scratch (eviction keys) after a state import
hipError_t launch_clear_step_scratch(const DevCache& c, hipStream_t st);
// debug: fills the per-step partial results (fused records, split and tier
// partials, candidate rows) with NaN, so a read of one not written by the
// step that follows shows in its output
hipError_t launch_poison_partials(const DevCache& c, hipStream_t st);

}  // namespace hkv
