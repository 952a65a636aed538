// q8_format.h -- weight formats of a packed matrix (shared by host and device code).
//
// Q8_0: 16-byte chunks of 16 int8 quants, one fp16 scale per 32-quant block.
// Q4_0: 16-byte chunks holding one GGUF Q4_0 block's 32 4-bit values.
#pragma once

namespace q8 {

enum : int { kFmtQ8 = 0, kFmtQ4 = 1 };

// 16-byte chunks per row of K weights.
inline constexpr long long chunks_per_row(int fmt, long long K) {
  return fmt == kFmtQ4 ? K / 32 : K / 16;
}

}  // namespace q8
