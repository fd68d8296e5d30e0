// Host side of the DF11 codec: histogram, codebook (Huffman lengths, canonical
// codes, CodeLengths, hierarchical LUTs), layout planning, encoding with the
// per-thread Gaps and per-group output positions, and the GPU decoder's
// first-level table.
//
// Method: "DFloat11: Kompresi inferensi GPU lossless yang mengecilkan LLM
// menjadi 70% ukurannya" (GeekNews), sections "Format DFloat11",
// "Decoding berbasis LUT hierarkis" and "Kernel GPU 2 tahap dan metadata bantu".
#include <algorithm>
#include <array>
#include <cstdint>
#include <cstring>
#include <queue>
#include <utility>
#include <vector>

#include "df11.h"
#include "df11_internal.h"

namespace {

constexpr int kFirstPointer = DF11_FIRST_POINTER;
constexpr int kMaxLen = DF11_MAX_CODE_LEN;
constexpr int kMaxLuts = DF11_MAX_LUTS;

uint64_t round_up(uint64_t x, uint64_t m) { return (x + m - 1) / m * m; }

// Huffman code lengths.  Min-heap keyed by (weight, id); leaves use their
// exponent as id, the k-th merged node uses 256 + k.
int huffman_lengths(const uint64_t hist[256], uint8_t lens[256]) {
    std::array<bool, 256> present{};
    int used = 0;
    for (int e = 0; e < 256; ++e) {
        if (hist[e] == 0) continue;
        if (e >= kFirstPointer) return DF11_E_RESERVED_EXPONENT;
        present[e] = true;
        ++used;
    }
    // Fewer than two symbols: pad with the smallest unused exponents (weight 0).
    for (int e = 0; e < kFirstPointer && used < 2; ++e) {
        if (!present[e]) {
            present[e] = true;
            ++used;
        }
    }
    using Node = std::pair<uint64_t, uint32_t>;  // (weight, id)
    std::priority_queue<Node, std::vector<Node>, std::greater<Node>> heap;
    std::vector<int32_t> parent(512, -1);
    for (int e = 0; e < 256; ++e)
        if (present[e]) heap.emplace(hist[e], static_cast<uint32_t>(e));
    uint32_t next_id = 256;
    while (heap.size() > 1) {
        Node a = heap.top();
        heap.pop();
        Node b = heap.top();
        heap.pop();
        parent[a.second] = static_cast<int32_t>(next_id);
        parent[b.second] = static_cast<int32_t>(next_id);
        heap.emplace(a.first + b.first, next_id);
        ++next_id;
    }
    // Depth of node id, memoised from the root down.
    std::vector<int> depth(512, -1);
    const uint32_t root = next_id - 1;
    depth[root] = 0;
    for (int id = static_cast<int>(root) - 1; id >= 0; --id) {
        if (parent[id] >= 0) depth[id] = depth[parent[id]] + 1;
    }
    for (int e = 0; e < 256; ++e) {
        lens[e] = 0;
        if (!present[e]) continue;
        if (depth[e] > kMaxLen) return DF11_E_CODE_TOO_LONG;
        lens[e] = static_cast<uint8_t>(depth[e]);
    }
    return DF11_OK;
}

// Canonical codes: per-length counts give each length's first code; within a
// length, codes ascend with the exponent.
int canonical_codes(const uint8_t lens[256], uint32_t codes[256]) {
    std::array<uint64_t, kMaxLen + 2> count{};
    for (int e = 0; e < 256; ++e) {
        if (lens[e] > kMaxLen) return DF11_E_CODE_TOO_LONG;
        if (lens[e]) ++count[lens[e]];
    }
    std::array<uint64_t, kMaxLen + 2> next{};
    uint64_t code = 0;
    for (int len = 1; len <= kMaxLen; ++len) {
        code = (code + count[len - 1]) << 1;
        next[len] = code;
    }
    // Kraft equality: the codes of the longest length end exactly at 2^len.
    int max_len = 0;
    for (int len = 1; len <= kMaxLen; ++len)
        if (count[len]) max_len = len;
    if (max_len == 0) return DF11_E_BAD_STREAM;
    if (next[max_len] + count[max_len] != (1ull << max_len)) return DF11_E_BAD_STREAM;
    for (int e = 0; e < 256; ++e) {
        codes[e] = 0;
        if (lens[e]) codes[e] = static_cast<uint32_t>(next[lens[e]]++);
    }
    return DF11_OK;
}

// Hierarchical LUTs.  A LUT belongs to a code-tree node at depth 0, 8, 16 or 24,
// named by (depth, prefix).  Lower LUTs are the internal nodes at depths 8/16/24
// (prefixes of longer codes), numbered 1.. in (depth, prefix) order.
int build_luts(const uint8_t lens[256], const uint32_t codes[256], uint8_t luts[kMaxLuts][256],
               uint32_t *n_luts) {
    std::vector<std::pair<int, uint32_t>> nodes;  // (depth, prefix)
    for (int e = 0; e < 256; ++e) {
        const int len = lens[e];
        for (int d = 8; d < len; d += 8) nodes.emplace_back(d, codes[e] >> (len - d));
    }
    std::sort(nodes.begin(), nodes.end());
    nodes.erase(std::unique(nodes.begin(), nodes.end()), nodes.end());
    if (nodes.size() + 1 > static_cast<size_t>(kMaxLuts)) return DF11_E_TOO_MANY_LUTS;
    auto lut_id = [&](int d, uint32_t prefix) -> int {
        auto it = std::lower_bound(nodes.begin(), nodes.end(), std::make_pair(d, prefix));
        return 1 + static_cast<int>(it - nodes.begin());
    };
    std::vector<std::array<int, 256>> fill(nodes.size() + 1);
    for (auto &f : fill) f.fill(-1);
    for (int e = 0; e < 256; ++e) {
        const int len = lens[e];
        if (!len) continue;
        for (int d = 0; d < len; d += 8) {
            const int id = d == 0 ? 0 : lut_id(d, codes[e] >> (len - d));
            const int rest = len - d;  // bits of the code below this LUT's node
            if (rest <= 8) {
                const uint32_t low = codes[e] & ((1u << rest) - 1u);
                const uint32_t first = low << (8 - rest);
                for (uint32_t x = first; x < first + (1u << (8 - rest)); ++x) fill[id][x] = e;
            } else {
                const uint32_t x = (codes[e] >> (rest - 8)) & 0xFFu;
                fill[id][x] = 256 - lut_id(d + 8, codes[e] >> (rest - 8));
            }
        }
    }
    for (size_t id = 0; id < fill.size(); ++id) {
        for (int x = 0; x < 256; ++x) {
            if (fill[id][x] < 0) return DF11_E_BAD_STREAM;  // incomplete code
            luts[id][x] = static_cast<uint8_t>(fill[id][x]);
        }
    }
    *n_luts = static_cast<uint32_t>(fill.size());
    return DF11_OK;
}

bool layout_ok(const df11_layout *lay) {
    return lay && lay->bytes_per_thread >= 4 && lay->threads_per_group >= 64 &&
           lay->threads_per_group % 64 == 0 && lay->bytes_per_thread <= (1u << 20) &&
           lay->threads_per_group <= 4096;
}

// Fill the size fields for a stream of n elements with total_bits payload bits.
void fill_sizes(df11_header *h, uint64_t n, uint64_t total_bits, const df11_layout *lay) {
    const uint64_t seg_bits = 8ull * lay->bytes_per_thread;
    h->n_elements = n;
    h->total_bits = total_bits;
    h->bytes_per_thread = lay->bytes_per_thread;
    h->threads_per_group = lay->threads_per_group;
    h->n_threads = (total_bits + seg_bits - 1) / seg_bits;
    h->n_groups = (h->n_threads + lay->threads_per_group - 1) / lay->threads_per_group;
    h->enc_bytes = round_up(h->n_threads * lay->bytes_per_thread, 16) + 16;
    h->sm_bytes = round_up(n, 64);
    h->gaps_bytes = 4 * ((5 * h->n_threads + 31) / 32 + 1);
    h->out_pos_bytes = 4 * (h->n_groups + 1);
}

// MSB-first bit sink with a 64-bit accumulator.
struct BitWriter {
    uint8_t *out;
    uint64_t acc = 0;   // pending bits, left-aligned
    int fill = 0;       // number of pending bits
    uint64_t bytes = 0; // bytes flushed
    void put(uint32_t code, int len) {
        acc |= static_cast<uint64_t>(code) << (64 - fill - len);
        fill += len;
        while (fill >= 8) {
            out[bytes++] = static_cast<uint8_t>(acc >> 56);
            acc <<= 8;
            fill -= 8;
        }
    }
    void finish() {
        if (fill > 0) out[bytes++] = static_cast<uint8_t>(acc >> 56);
        acc = 0;
        fill = 0;
    }
};

}  // namespace

extern "C" {

int df11_histogram(const uint16_t *bf16, uint64_t n, uint64_t hist[256]) {
    if (!hist || (n && !bf16)) return DF11_E_INVALID_ARG;
    std::array<uint64_t, 256> local{};
    for (uint64_t i = 0; i < n; ++i) ++local[(bf16[i] >> 7) & 0xFF];
    for (int e = kFirstPointer; e < 256; ++e)
        if (local[e]) return DF11_E_RESERVED_EXPONENT;
    for (int e = 0; e < 256; ++e) hist[e] += local[e];
    return DF11_OK;
}

int df11_build_codebook(const uint64_t hist[256], df11_codebook *cb) {
    if (!hist || !cb) return DF11_E_INVALID_ARG;
    df11_codebook tmp;
    std::memset(&tmp, 0, sizeof(tmp));
    int rc = huffman_lengths(hist, tmp.code_lengths);
    if (rc) return rc;
    rc = canonical_codes(tmp.code_lengths, tmp.codes);
    if (rc) return rc;
    rc = build_luts(tmp.code_lengths, tmp.codes, tmp.luts, &tmp.n_luts);
    if (rc) return rc;
    tmp.max_len = 0;
    for (int e = 0; e < 256; ++e) tmp.max_len = std::max<uint32_t>(tmp.max_len, tmp.code_lengths[e]);
    *cb = tmp;
    return DF11_OK;
}

int df11_plan(const df11_codebook *cb, const uint64_t hist[256], uint64_t n, const df11_layout *lay,
              df11_header *h) {
    if (!cb || !hist || !h || !layout_ok(lay)) return DF11_E_INVALID_ARG;
    if (n > DF11_MAX_ELEMENTS) return DF11_E_TOO_LARGE;
    uint64_t total = 0, count = 0;
    for (int e = 0; e < 256; ++e) {
        if (hist[e] && !cb->code_lengths[e]) return DF11_E_INVALID_ARG;
        total += hist[e] * cb->code_lengths[e];
        count += hist[e];
    }
    if (count != n) return DF11_E_INVALID_ARG;
    df11_header tmp;
    std::memset(&tmp, 0, sizeof(tmp));
    fill_sizes(&tmp, n, total, lay);
    tmp.n_luts = cb->n_luts;
    tmp.max_len = cb->max_len;
    const uint64_t bound = 8ull * lay->bytes_per_thread * lay->threads_per_group;
    tmp.max_group_elems = static_cast<uint32_t>(std::min<uint64_t>(bound, n));
    *h = tmp;
    return DF11_OK;
}

int df11_encode(const df11_codebook *cb, const uint16_t *bf16, uint64_t n, const df11_layout *lay,
                df11_header *h, uint8_t *enc, uint8_t *sm, uint8_t *gaps, uint32_t *out_pos) {
    if (!cb || !h || !enc || !sm || !gaps || !out_pos || !layout_ok(lay) || (n && !bf16))
        return DF11_E_INVALID_ARG;
    if (n > DF11_MAX_ELEMENTS) return DF11_E_TOO_LARGE;
    if (h->n_elements != n || h->bytes_per_thread != lay->bytes_per_thread ||
        h->threads_per_group != lay->threads_per_group)
        return DF11_E_INVALID_ARG;
    // Check the data against the planned sizes before writing anything.
    uint64_t total = 0;
    for (uint64_t i = 0; i < n; ++i) {
        const uint32_t e = (bf16[i] >> 7) & 0xFF;
        if (e >= static_cast<uint32_t>(kFirstPointer)) return DF11_E_RESERVED_EXPONENT;
        if (!cb->code_lengths[e]) return DF11_E_INVALID_ARG;
        total += cb->code_lengths[e];
    }
    df11_header planned;
    std::memset(&planned, 0, sizeof(planned));
    fill_sizes(&planned, n, total, lay);
    if (planned.total_bits != h->total_bits || planned.enc_bytes != h->enc_bytes ||
        planned.gaps_bytes != h->gaps_bytes || planned.sm_bytes != h->sm_bytes ||
        planned.out_pos_bytes != h->out_pos_bytes)
        return DF11_E_INVALID_ARG;

    const uint32_t n_bytes = lay->bytes_per_thread;
    const uint32_t G = lay->threads_per_group;
    const uint64_t seg_bits = 8ull * n_bytes;
    const uint64_t T = h->n_threads;
    std::memset(enc, 0, h->enc_bytes);
    std::memset(gaps, 0, h->gaps_bytes);
    std::memset(sm + n, 0, h->sm_bytes - n);

    BitWriter bits{enc};
    uint64_t pos = 0;        // start bit of the next code
    uint64_t next_thread = 0;
    uint64_t gap_acc = 0;    // 5-bit gaps packed MSB-first through a small accumulator
    int gap_fill = 0;
    uint64_t gap_byte = 0;
    auto emit_gap = [&](uint32_t gap) {
        gap_acc = (gap_acc << 5) | gap;
        gap_fill += 5;
        while (gap_fill >= 8) {
            gaps[gap_byte++] = static_cast<uint8_t>(gap_acc >> (gap_fill - 8));
            gap_fill -= 8;
        }
        gap_acc &= (1ull << gap_fill) - 1;
    };
    auto close_threads_upto = [&](uint64_t start, uint64_t index) {
        // Every thread whose segment begins at or before `start` (and after the
        // previous code start) has its first code start at `start`.
        while (next_thread < T && next_thread * seg_bits <= start) {
            emit_gap(static_cast<uint32_t>(start - next_thread * seg_bits));
            if (next_thread % G == 0) out_pos[next_thread / G] = static_cast<uint32_t>(index);
            ++next_thread;
        }
    };
    for (uint64_t i = 0; i < n; ++i) {
        const uint16_t w = bf16[i];
        const uint32_t e = (w >> 7) & 0xFF;
        sm[i] = static_cast<uint8_t>(((w >> 8) & 0x80) | (w & 0x7F));
        if (next_thread < T && next_thread * seg_bits <= pos) close_threads_upto(pos, i);
        const int len = cb->code_lengths[e];
        bits.put(cb->codes[e], len);
        pos += len;
    }
    bits.finish();
    close_threads_upto(pos, n);  // the stream end acts as the last code start
    if (gap_fill > 0) gaps[gap_byte++] = static_cast<uint8_t>(gap_acc << (8 - gap_fill));
    out_pos[h->n_groups] = static_cast<uint32_t>(n);

    uint32_t max_elems = 0;
    for (uint64_t g = 0; g < h->n_groups; ++g)
        max_elems = std::max(max_elems, out_pos[g + 1] - out_pos[g]);
    h->total_bits = pos;
    h->n_luts = cb->n_luts;
    h->max_len = cb->max_len;
    h->max_group_elems = max_elems;
    return DF11_OK;
}

uint64_t df11_decode_table_bytes(uint32_t bits) {
    if (bits < df11::kDecodeTableMinBits || bits > df11::kDecodeTableMaxBits) return 0;
    return 10ull << bits;  // lo and aux words and a 16-bit start mask per entry
}

int df11_build_decode_table(const df11_codebook *cb, uint32_t bits, void *table, uint64_t table_bytes) {
    if (!cb || !table) return DF11_E_INVALID_ARG;
    const uint64_t need = df11_decode_table_bytes(bits);
    if (!need) return DF11_E_INVALID_ARG;
    if (table_bytes < need) return DF11_E_BUFFER_TOO_SMALL;
    // Canonical decoding data: for each length, the first code and the
    // exponents of that length in ascending order.
    std::array<uint32_t, kMaxLen + 2> first{}, count{}, offset{};
    std::vector<uint8_t> by_len;
    for (int len = 1; len <= kMaxLen; ++len) {
        offset[len] = static_cast<uint32_t>(by_len.size());
        bool have = false;
        for (int e = 0; e < 256; ++e) {
            if (cb->code_lengths[e] != len) continue;
            if (!have) first[len] = cb->codes[e];
            have = true;
            by_len.push_back(static_cast<uint8_t>(e));
            ++count[len];
        }
    }
    const uint32_t size = 1u << bits;
    // Entry x: words 2x (exponent run) and 2x + 1 (aux), then the start masks.
    uint32_t *pairs = static_cast<uint32_t *>(table);
    uint16_t *starts = reinterpret_cast<uint16_t *>(pairs + 2 * size);
    for (uint32_t x = 0; x < size; ++x) {
        uint32_t used = 0, mask = 0, m = 0;
        uint8_t syms[df11::kDecodeTableMaxSyms] = {0};
        while (m < df11::kDecodeTableMaxSyms) {
            // Find the code at offset `used` among lengths that fit in the window.
            int sym = -1, len = 0;
            for (int l = 1; l <= static_cast<int>(bits - used); ++l) {
                const uint32_t v = (x >> (bits - used - l)) & ((1u << l) - 1u);
                if (count[l] && v >= first[l] && v - first[l] < count[l]) {
                    sym = by_len[offset[l] + (v - first[l])];
                    len = l;
                    break;
                }
            }
            if (sym < 0) break;
            syms[m++] = static_cast<uint8_t>(sym);
            mask |= 1u << used;
            used += static_cast<uint32_t>(len);
        }
        uint32_t lo_word = 0;
        for (uint32_t j = 0; j < 4 && j < m; ++j)
            lo_word |= static_cast<uint32_t>(df11::rotate_exponent(syms[j])) << (8 * j);
        pairs[2 * x] = lo_word;
        pairs[2 * x + 1] = m ? (((m << 11) + used) | ((m > 4 ? df11::rotate_exponent(syms[4]) : 0u) << 16))
                             : df11::kLongCodeIncrement;
        starts[x] = static_cast<uint16_t>(m ? mask : 1u);
    }
    return DF11_OK;
}

int df11_tile_order(const uint16_t *w, uint64_t rows, uint64_t cols, uint16_t *out) {
    if (!w || !out || rows % 64 || cols % 32) return DF11_E_INVALID_ARG;
    const uint64_t n = rows * cols;
    if (n && (w < out ? w + n > out : out + n > w)) return DF11_E_INVALID_ARG;
    // Walk the ordered sequence block by block: block b is n-tile b mod 4 of
    // global k-step b / 4 (k-step ks of panel p); lane l of a block takes 8
    // consecutive columns of one row.
    const uint64_t ks_per_panel = cols / 32;
    uint64_t s = 0;
    for (uint64_t p = 0; p < rows / 64; ++p)
        for (uint64_t ks = 0; ks < ks_per_panel; ++ks)
            for (uint64_t nt = 0; nt < 4; ++nt)
                for (uint64_t l = 0; l < 64; ++l, s += 8) {
                    const uint64_t r = 64 * p + 16 * nt + l % 16, c = 32 * ks + 8 * (l / 16);
                    memcpy(out + s, w + r * cols + c, 8 * sizeof(uint16_t));
                }
    return DF11_OK;
}

const char *df11_status_str(int status) {
    switch (status) {
    case DF11_OK: return "DF11_OK";
    case DF11_E_INVALID_ARG: return "DF11_E_INVALID_ARG";
    case DF11_E_RESERVED_EXPONENT: return "DF11_E_RESERVED_EXPONENT";
    case DF11_E_CODE_TOO_LONG: return "DF11_E_CODE_TOO_LONG";
    case DF11_E_TOO_MANY_LUTS: return "DF11_E_TOO_MANY_LUTS";
    case DF11_E_BUFFER_TOO_SMALL: return "DF11_E_BUFFER_TOO_SMALL";
    case DF11_E_BAD_STREAM: return "DF11_E_BAD_STREAM";
    case DF11_E_TOO_LARGE: return "DF11_E_TOO_LARGE";
    case DF11_E_HIP: return "DF11_E_HIP";
    default: return "DF11_E_UNKNOWN";
    }
}

}  // extern "C"
