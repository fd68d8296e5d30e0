// Host side of the rANS exponent coder: frequency quantization, the encoder
// and the decoder's slot table.  The format (this library's reading of the
// rANS alternative that the discussion on "DFloat11: Kompresi inferensi GPU
// lossless yang mengecilkan LLM menjadi 70% ukurannya" (GeekNews), section
// "Opini Hacker News", mentions) is described in df11.h.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

#include "df11.h"

namespace {

constexpr uint32_t kProbBits = DF11_RANS_PROB_BITS;
constexpr uint32_t kM = 1u << kProbBits;
constexpr uint32_t kLanes = DF11_RANS_LANES;
constexpr uint32_t kSteps = DF11_RANS_STEPS;
constexpr uint64_t kSegment = static_cast<uint64_t>(kLanes) * kSteps;
constexpr uint32_t kStateLow = 1u << 16;  // states live in [2^16, 2^32)
constexpr uint32_t kFirstReserved = 240;  // exponents 240..255 are reserved (Inf/NaN or huge)

// Cumulative frequencies; false unless they sum to M.
bool cumulate(const uint32_t freq[256], uint32_t cum[257]) {
    uint64_t c = 0;
    for (int s = 0; s < 256; ++s) {
        cum[s] = static_cast<uint32_t>(c);
        c += freq[s];
    }
    cum[256] = static_cast<uint32_t>(c);
    return c == kM;
}

}  // namespace

extern "C" {

int df11_rans_quantize(const uint64_t hist[256], uint32_t freq[256]) {
    if (!hist || !freq) return DF11_E_INVALID_ARG;
    uint64_t total = 0;
    for (int s = 0; s < 256; ++s) {
        if (hist[s] && s >= static_cast<int>(kFirstReserved)) return DF11_E_RESERVED_EXPONENT;
        total += hist[s];
    }
    std::memset(freq, 0, 256 * sizeof(uint32_t));
    if (total == 0) return DF11_OK;
    uint64_t sum = 0;
    int most = -1;  // most frequent exponent, lowest value first
    for (int s = 0; s < 256; ++s) {
        if (!hist[s]) continue;
        const uint64_t q = static_cast<uint64_t>((static_cast<unsigned __int128>(hist[s]) * kM) / total);
        freq[s] = static_cast<uint32_t>(q > 0 ? q : 1);
        sum += freq[s];
        if (most < 0 || hist[s] > hist[most]) most = s;
    }
    if (sum < kM) freq[most] += static_cast<uint32_t>(kM - sum);
    // (at most 240 used exponents, so the sum exceeds M by less than 240)
    while (sum > kM) {
        int big = -1;
        for (int s = 0; s < 256; ++s)
            if (freq[s] > 1 && (big < 0 || freq[s] > freq[big])) big = s;
        --freq[big];
        --sum;
    }
    return DF11_OK;
}

int df11_rans_build_table(const uint32_t freq[256], uint32_t *table) {
    if (!freq || !table) return DF11_E_INVALID_ARG;
    uint32_t cum[257];
    if (!cumulate(freq, cum)) return DF11_E_INVALID_ARG;
    for (uint32_t s = 0; s < 256; ++s) {
        const uint32_t rotated = ((s >> 1) | ((s & 1u) << 7)) & 0xFFu;
        for (uint32_t k = cum[s]; k < cum[s + 1]; ++k) table[k] = rotated | ((freq[s] - 1u) << 8) | ((k - cum[s]) << 20);
    }
    return DF11_OK;
}

int df11_rans_encode(const uint32_t freq[256], const uint16_t *w, uint64_t n, uint32_t *states,
                     uint32_t *word_offsets, uint16_t *words, uint64_t words_cap, uint8_t *sm, df11_rans_header *h) {
    if (!freq || !h || !word_offsets || (n && (!w || !states || !sm || !words))) return DF11_E_INVALID_ARG;
    if (n > DF11_MAX_ELEMENTS) return DF11_E_TOO_LARGE;
    uint32_t cum[257];
    const bool ok = cumulate(freq, cum);
    if (n && !ok) return DF11_E_INVALID_ARG;
    const uint64_t n_seg = (n + kSegment - 1) / kSegment;
    std::vector<uint16_t> pending;  // one segment's words, in the order the encoder emits them
    pending.reserve(kSegment);
    uint32_t x[kLanes];
    uint64_t total = 0;
    for (uint64_t g = 0; g < n_seg; ++g) {
        const uint64_t base = g * kSegment;
        const uint64_t count = std::min<uint64_t>(kSegment, n - base);
        pending.clear();
        for (uint32_t l = 0; l < kLanes; ++l) x[l] = kStateLow;
        // The decoder runs step ascending, lane ascending; the encoder the reverse.
        for (uint64_t j = kSteps; j-- > 0;) {
            for (uint32_t l = kLanes; l-- > 0;) {
                const uint64_t q = j * kLanes + l;
                if (q >= count) continue;
                const uint32_t s = (w[base + q] >> 7) & 0xFFu;
                if (s >= kFirstReserved) return DF11_E_RESERVED_EXPONENT;
                const uint32_t f = freq[s];
                if (f == 0) return DF11_E_INVALID_ARG;
                const uint64_t limit = static_cast<uint64_t>(f) << (32 - kProbBits);
                uint32_t v = x[l];
                while (v >= limit) {
                    pending.push_back(static_cast<uint16_t>(v & 0xFFFFu));
                    v >>= 16;
                }
                x[l] = ((v / f) << kProbBits) + v % f + cum[s];
            }
        }
        if (total + pending.size() > words_cap) return DF11_E_BUFFER_TOO_SMALL;
        if (total + pending.size() >= (1ull << 32)) return DF11_E_TOO_LARGE;
        word_offsets[g] = static_cast<uint32_t>(total);
        for (size_t i = 0; i < pending.size(); ++i) words[total + i] = pending[pending.size() - 1 - i];
        total += pending.size();
        std::memcpy(states + g * kLanes, x, sizeof(x));
    }
    word_offsets[n_seg] = static_cast<uint32_t>(total);
    for (uint64_t i = 0; i < n; ++i) sm[i] = static_cast<uint8_t>(((w[i] >> 8) & 0x80u) | (w[i] & 0x7Fu));
    h->n_elements = n;
    h->n_segments = n_seg;
    h->n_words = total;
    h->prob_bits = kProbBits;
    h->lanes = kLanes;
    h->steps = kSteps;
    h->reserved = 0;
    return DF11_OK;
}

}  // extern "C"
