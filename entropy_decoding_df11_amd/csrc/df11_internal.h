// Constants shared by the host encoder and the gfx950 decoder (product code only).
#ifndef DF11_INTERNAL_H
#define DF11_INTERNAL_H

#include <stdint.h>

namespace df11 {

// First-level decode table: indexed by the next `bits` bits of the stream.
// Entry x is two 32-bit words stored in two arrays (lo[x], then hi[x]):
//   lo: up to four exponents (byte j = j-th complete code of the window)
//   hi: bits 0..15  exponents 4 and 5,
//       bits 16..27 start mask (bit j set: a listed code starts at offset j),
//       bits 28..31 total length of the listed codes (0: the first code is
//                   longer than the window; bits 0..7 then hold the root LUT's
//                   pointer value for the window's first 8 bits).
// Exponents are stored rotated right by one bit, (e >> 1) | ((e & 1) << 7), so
// that the decoder's merge with the sign/mantissa byte is a single bitfield
// insert per BF16 pair.
constexpr uint32_t kDecodeTableMinBits = 10;
constexpr uint32_t kDecodeTableMaxBits = 12;
constexpr uint32_t kDecodeTableMaxSyms = 6;

inline constexpr uint32_t rotate_exponent(uint32_t e) { return ((e >> 1) | (e << 7)) & 0xFFu; }

// Layout supported by the GPU decoder.
constexpr uint32_t kBytesPerThread = 8;
constexpr uint32_t kThreadsPerGroup = 256;

}  // namespace df11

#endif  // DF11_INTERNAL_H
