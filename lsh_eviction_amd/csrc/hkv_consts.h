// hkv_consts.h -- constants shared by the host layout code and the kernels.
#pragma once

namespace hkv {
constexpr int kScoreChunk = 4096;   // slots per block of the stand-alone hamming_argmax
constexpr int kMaxGroup = 16;       // query heads per KV head
constexpr int kCountStride = 32;    // 4-byte entries per head's ticket counter: one 128-byte line each, so the
                                    // atomics of different heads never meet on one line
}  // namespace hkv
