// hkv_consts.h -- constants shared by the host layout code and the kernels.
#pragma once

namespace hkv {
constexpr int kScoreChunk = 4096;   // slots per block of the stand-alone hamming_argmax
constexpr int kMaxGroup = 16;       // query heads per KV head
}  // namespace hkv
