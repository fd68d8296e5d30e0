// Constants shared by the host encoder and the gfx950 decoder (product code only).
#ifndef DF11_INTERNAL_H
#define DF11_INTERNAL_H

#include <stdint.h>

namespace df11 {

// First-level decode table: indexed by the next `bits` bits of the stream.
// Entry x is the pair of uint32 words 2x (lo) and 2x + 1 (aux), read by the
// decoder as one 64-bit word; the 2^bits pairs are followed by a uint16 array
// of 2^bits start masks:
//   lo:    exponents 0..3 of the complete codes at the start of the window
//          (byte j = j-th code; unused bytes are zero)
//   aux:   bits 0..15  increment (m << 11) + nb, where m (1..5) is the number
//                      of codes listed and nb their total length; for a
//                      window whose first code is longer than the window,
//                      kLongCodeIncrement (and lo = aux bits 16..31 = 0)
//          bits 16..23 exponent 4 (zero when unused), bits 24..31 zero, so
//                      that (aux >> 16):lo is the 5-byte run of exponents
//   start: bit j set when a listed code starts at offset j of the window (1
//          for a window whose first code is too long)
// The increment advances a decoder accumulator (x << 11) | p, p < 256, by m in
// x and nb in p with one add; x is a count of codes or an LDS byte address.
// kLongCodeIncrement adds 128 to p only: it pushes p past any segment end,
// which ends the table-driven loop, and the decoder then finishes that code
// through the LUT hierarchy.
// Exponents are stored rotated right by one bit, (e >> 1) | ((e & 1) << 7), so
// that each byte of a BF16 word is one bitfield insert of a rotated exponent
// byte and a sign/mantissa byte.
constexpr uint32_t kDecodeTableMinBits = 10;
constexpr uint32_t kDecodeTableMaxBits = 12;
constexpr uint32_t kDecodeTableMaxSyms = 5;
constexpr uint32_t kLongCodeIncrement = 0x80;

inline constexpr uint32_t rotate_exponent(uint32_t e) { return ((e >> 1) | (e << 7)) & 0xFFu; }

// Layout supported by the GPU decoder.
constexpr uint32_t kBytesPerThread = 8;
constexpr uint32_t kThreadsPerGroup = 256;

}  // namespace df11

#endif  // DF11_INTERNAL_H
