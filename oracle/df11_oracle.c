/*
 * DF11 oracle: a plain, slow, obviously correct CPU encoder/decoder.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg may load this file's library.  It shares no code,
 * header, table or constant generator with the HIP path, and it includes
 * nothing from the product.
 *
 * Source of the method: the GeekNews summary "DFloat11: Kompresi inferensi GPU
 * lossless yang mengecilkan LLM menjadi 70% ukurannya" (id.news.hada.io topic
 * 20542).  Section names below are that page's headings:
 *   [Entropy]  "Ruang kompresi yang tersisa pada exponent BFloat16"
 *   [Format]   "Format DFloat11"
 *   [GPU]      "Dekompresi yang disesuaikan untuk inferensi GPU"
 *   [LUT]      "Decoding berbasis LUT hierarkis"
 *   [Kernel]   "Kernel GPU 2 tahap dan metadata bantu"
 *
 * Readings of points the page leaves open are fixed here and listed in the
 * repository's design notes: MSB-first bit order, min-heap (weight, id)
 * Huffman tie-break, canonical code assignment, phantom symbol for a single
 * used exponent, LUT ids in breadth-first (depth, prefix) order with
 * pointer value 256 - id, 5-bit MSB-first gaps, the end of the stream as the
 * sentinel code start, and the buffer paddings below.
 *
 * Every function returns 0 on success or a negative error code.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_E_INVALID_ARG (-1)
#define ORC_E_RESERVED_EXPONENT (-2)
#define ORC_E_CODE_TOO_LONG (-3)
#define ORC_E_TOO_MANY_LUTS (-4)
#define ORC_E_BUFFER_TOO_SMALL (-5)
#define ORC_E_BAD_STREAM (-6)
#define ORC_E_TOO_LARGE (-7)

/* [LUT]: exponent values 240..255 never occur in the weights and are reused
 * as pointers to lower LUTs, so 240 is the first value an input may not use. */
#define ORC_FIRST_POINTER 240
#define ORC_MAX_LUTS 17     /* the root plus one LUT per pointer value 240..255 */
#define ORC_MAX_LEN 32      /* [Kernel]: gaps lie in [0, 31] because codes are at most 32 bits */

/* ---------------------------------------------------------------------------
 * Step 1, [Entropy] + [Format]: a BF16 word is 1 sign bit, 8 exponent bits and
 * 7 mantissa bits.  The exponent goes to the entropy coder; sign and mantissa
 * are kept verbatim, one byte per weight, sign in bit 7, mantissa in bits 0-6.
 * ------------------------------------------------------------------------- */
int orc_split(const uint16_t *w, uint64_t n, uint8_t *exponent, uint8_t *sign_mantissa)
{
    for (uint64_t i = 0; i < n; i++) {
        uint32_t sign = (w[i] >> 15) & 1u;
        uint32_t e = (w[i] >> 7) & 0xFFu;
        uint32_t mant = w[i] & 0x7Fu;
        if (e >= ORC_FIRST_POINTER) return ORC_E_RESERVED_EXPONENT;
        exponent[i] = (uint8_t)e;
        sign_mantissa[i] = (uint8_t)((sign << 7) | mant);
    }
    return ORC_OK;
}

/* Inverse of orc_split: put the three fields back in their BF16 positions. */
int orc_merge(const uint8_t *exponent, const uint8_t *sign_mantissa, uint64_t n, uint16_t *w)
{
    for (uint64_t i = 0; i < n; i++) {
        uint32_t sign = (sign_mantissa[i] >> 7) & 1u;
        uint32_t mant = sign_mantissa[i] & 0x7Fu;
        w[i] = (uint16_t)((sign << 15) | ((uint32_t)exponent[i] << 7) | mant);
    }
    return ORC_OK;
}

/* Step 2, [Format]: the Huffman tree is built from the exponent histogram.
 * Accumulates into hist so several tensors can share one codebook. */
int orc_histogram(const uint16_t *w, uint64_t n, uint64_t hist[256])
{
    for (uint64_t i = 0; i < n; i++) {
        uint32_t e = (w[i] >> 7) & 0xFFu;
        if (e >= ORC_FIRST_POINTER) return ORC_E_RESERVED_EXPONENT;
        hist[e] += 1;
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Step 3, [Format]: Huffman code lengths.  Frequent exponents get short codes.
 * Nodes carry (weight, id); a leaf's id is its exponent, the k-th merged node
 * gets id 256 + k.  Each round removes the two smallest nodes in (weight, id)
 * order and adds their sum.  A symbol's code length is its depth.
 * With fewer than two used exponents, the smallest unused exponent(s) below
 * 240 join with weight 0 so that every code has at least one bit.
 * ------------------------------------------------------------------------- */
int orc_code_lengths(const uint64_t hist[256], uint8_t lens[256])
{
    uint64_t weight[512];
    int parent[512];
    int alive[512];
    int n_nodes = 0;
    int in_tree[256];
    int used = 0;

    for (int s = 0; s < 256; s++) {
        lens[s] = 0;
        in_tree[s] = 0;
    }
    for (int s = 0; s < 256; s++) {
        if (hist[s] > 0) {
            if (s >= ORC_FIRST_POINTER) return ORC_E_RESERVED_EXPONENT;
            in_tree[s] = 1;
            used++;
        }
    }
    for (int s = 0; s < ORC_FIRST_POINTER && used < 2; s++) {
        if (!in_tree[s]) {
            in_tree[s] = 1;
            used++;
        }
    }

    /* node index == id: leaves 0..255, merged nodes 256.. */
    for (int i = 0; i < 512; i++) {
        weight[i] = 0;
        parent[i] = -1;
        alive[i] = 0;
    }
    for (int s = 0; s < 256; s++) {
        if (in_tree[s]) {
            weight[s] = hist[s];
            alive[s] = 1;
        }
    }
    n_nodes = 256;
    for (int remaining = used; remaining > 1; remaining--) {
        int a = -1, b = -1;
        for (int i = 0; i < n_nodes; i++) {
            if (!alive[i]) continue;
            /* ascending id order, so "strictly smaller weight" breaks ties by id */
            if (a < 0 || weight[i] < weight[a]) {
                b = a;
                a = i;
            } else if (b < 0 || weight[i] < weight[b]) {
                b = i;
            }
        }
        int m = n_nodes++;
        weight[m] = weight[a] + weight[b];
        alive[m] = 1;
        alive[a] = 0;
        alive[b] = 0;
        parent[a] = m;
        parent[b] = m;
    }

    for (int s = 0; s < 256; s++) {
        if (!in_tree[s]) continue;
        int depth = 0;
        for (int v = s; parent[v] >= 0; v = parent[v]) depth++;
        if (depth > ORC_MAX_LEN) return ORC_E_CODE_TOO_LONG;
        lens[s] = (uint8_t)depth;
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Step 4: canonical codes from the lengths.  Symbols are taken in ascending
 * (length, symbol) order; each code is the previous code plus one, shifted
 * left by the length increase.
 * ------------------------------------------------------------------------- */
int orc_canonical_codes(const uint8_t lens[256], uint32_t codes[256])
{
    uint64_t code = 0;
    int prev_len = 0;
    int first = 1;
    for (int s = 0; s < 256; s++) {
        codes[s] = 0;
        if (lens[s] > ORC_MAX_LEN) return ORC_E_CODE_TOO_LONG;
    }
    for (int len = 1; len <= ORC_MAX_LEN; len++) {
        for (int s = 0; s < 256; s++) {
            if (lens[s] != len) continue;
            if (first) {
                code = 0;
                first = 0;
            } else {
                code <<= (len - prev_len);
            }
            codes[s] = (uint32_t)code;
            code += 1;
            prev_len = len;
        }
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * The code tree, built explicitly from the codes: every node has two children
 * (-1 when absent) and a symbol (-1 for internal nodes).  Node 0 is the root.
 * ------------------------------------------------------------------------- */
typedef struct {
    int child[2];
    int symbol;
    int depth;
    uint32_t prefix; /* the bits on the path from the root, MSB-first */
} orc_node;

#define ORC_TREE_CAP 1024

static int orc_build_tree(const uint8_t lens[256], const uint32_t codes[256], orc_node *tree, int *n_nodes)
{
    int count = 1;
    tree[0].child[0] = tree[0].child[1] = -1;
    tree[0].symbol = -1;
    tree[0].depth = 0;
    tree[0].prefix = 0;
    for (int s = 0; s < 256; s++) {
        int len = lens[s];
        if (len == 0) continue;
        int v = 0;
        for (int j = len - 1; j >= 0; j--) {
            int bit = (int)((codes[s] >> j) & 1u);
            if (tree[v].symbol >= 0) return ORC_E_BAD_STREAM; /* a code passes through a leaf */
            if (tree[v].child[bit] < 0) {
                if (count >= ORC_TREE_CAP) return ORC_E_BAD_STREAM;
                int c = count++;
                tree[c].child[0] = tree[c].child[1] = -1;
                tree[c].symbol = -1;
                tree[c].depth = tree[v].depth + 1;
                tree[c].prefix = (tree[v].prefix << 1) | (uint32_t)bit;
                tree[v].child[bit] = c;
            }
            v = tree[v].child[bit];
        }
        if (tree[v].symbol >= 0 || tree[v].child[0] >= 0 || tree[v].child[1] >= 0) return ORC_E_BAD_STREAM;
        tree[v].symbol = s;
    }
    *n_nodes = count;
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Step 8, [LUT]: the tree is cut into non-overlapping subtrees of height 8,
 * each a 256-entry LUT.  A LUT stands for a tree node u at depth 0, 8, 16 or
 * 24.  Entry x walks the 8 bits of x, MSB-first, from u: a leaf reached within
 * those bits gives its exponent; an internal node reached after all 8 bits
 * gives the pointer 256 - id of that node's own LUT.  The root LUT has id 0;
 * lower LUTs get ids 1, 2, ... in order of depth, then of prefix.
 * ------------------------------------------------------------------------- */
int orc_build_luts(const uint8_t lens[256], const uint32_t codes[256], uint8_t luts[ORC_MAX_LUTS][256],
                   uint32_t *n_luts)
{
    orc_node tree[ORC_TREE_CAP];
    int n_nodes = 0;
    int rc = orc_build_tree(lens, codes, tree, &n_nodes);
    if (rc) return rc;

    /* LUT roots: the root, then internal nodes at depths 8, 16, 24 in (depth, prefix) order */
    int lut_node[ORC_MAX_LUTS];
    int k = 0;
    lut_node[k++] = 0;
    for (int depth = 8; depth <= 24; depth += 8) {
        /* gather this depth's internal nodes, then order them by prefix (selection sort) */
        int list[ORC_TREE_CAP];
        int m = 0;
        for (int v = 0; v < n_nodes; v++)
            if (tree[v].depth == depth && tree[v].symbol < 0) list[m++] = v;
        for (int i = 0; i < m; i++) {
            int best = i;
            for (int j = i + 1; j < m; j++)
                if (tree[list[j]].prefix < tree[list[best]].prefix) best = j;
            int tmp = list[i];
            list[i] = list[best];
            list[best] = tmp;
        }
        for (int i = 0; i < m; i++) {
            if (k >= ORC_MAX_LUTS) return ORC_E_TOO_MANY_LUTS;
            lut_node[k++] = list[i];
        }
    }

    for (int id = 0; id < k; id++) {
        for (int x = 0; x < 256; x++) {
            int v = lut_node[id];
            int entry = -1;
            for (int j = 7; j >= 0; j--) {
                int bit = (x >> j) & 1;
                v = tree[v].child[bit];
                if (v < 0) return ORC_E_BAD_STREAM; /* incomplete code: some path has no node */
                if (tree[v].symbol >= 0) {
                    entry = tree[v].symbol;
                    break;
                }
            }
            if (entry < 0) {
                /* internal node after 8 bits: point to its own LUT */
                int target = -1;
                for (int t = 1; t < k; t++)
                    if (lut_node[t] == v) target = t;
                if (target < 0) return ORC_E_BAD_STREAM;
                entry = 256 - target;
            }
            luts[id][x] = (uint8_t)entry;
        }
    }
    *n_luts = (uint32_t)k;
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Layout sizes.  T = ceil(total_bits / (8 n)) threads, ceil(T / G) groups.
 * Paddings: EncodedExponent to round_up(T n, 16) + 16 bytes, PackedSignMantissa
 * to round_up(N, 64) bytes, Gaps to 4 (ceil(5 T / 32) + 1) bytes, all zero.
 * ------------------------------------------------------------------------- */
static uint64_t orc_round_up(uint64_t x, uint64_t m) { return (x + m - 1) / m * m; }

uint64_t orc_total_bits(const uint8_t lens[256], const uint64_t hist[256])
{
    uint64_t bits = 0;
    for (int s = 0; s < 256; s++) bits += (uint64_t)lens[s] * hist[s];
    return bits;
}

int orc_layout(uint64_t n_elements, uint64_t total_bits, uint32_t n, uint32_t G, uint64_t sizes[6])
{
    if (n < 4 || G == 0 || G % 64 != 0) return ORC_E_INVALID_ARG;
    if (n_elements >= (1ull << 32)) return ORC_E_TOO_LARGE;
    uint64_t seg_bits = 8ull * n;
    uint64_t T = (total_bits + seg_bits - 1) / seg_bits;
    uint64_t groups = (T + G - 1) / G;
    sizes[0] = T;
    sizes[1] = groups;
    sizes[2] = orc_round_up(T * n, 16) + 16;      /* EncodedExponent bytes */
    sizes[3] = orc_round_up(n_elements, 64);      /* PackedSignMantissa bytes */
    sizes[4] = 4 * ((5 * T + 31) / 32 + 1);       /* Gaps bytes */
    sizes[5] = 4 * (groups + 1);                  /* output positions bytes */
    return ORC_OK;
}

/* MSB-first bit writer: bit position p is bit (7 - p%8) of byte p/8. */
static void orc_put_bit(uint8_t *buf, uint64_t pos, int bit)
{
    if (bit) buf[pos >> 3] |= (uint8_t)(0x80u >> (pos & 7));
}

static int orc_get_bit(const uint8_t *buf, uint64_t pos)
{
    return (buf[pos >> 3] >> (7 - (pos & 7))) & 1;
}

/* ---------------------------------------------------------------------------
 * Steps 5-7, [Format] + [Kernel]: emit every exponent's code into
 * EncodedExponent, keep sign and mantissa in PackedSignMantissa, and write the
 * auxiliary metadata:
 *   gap_t   = (first code start at or after s_t) - s_t, with s_t = 8 n t and
 *             the end of the stream counting as a code start; 5 bits, MSB-first.
 *   out_pos[g] = number of codes that start before s_(g G); out_pos[groups] = N.
 * Buffers must be zeroed by the caller and sized by orc_layout.
 * ------------------------------------------------------------------------- */
int orc_encode(const uint16_t *w, uint64_t n_elements, const uint8_t lens[256], const uint32_t codes[256],
               uint32_t n, uint32_t G, uint8_t *enc, uint8_t *sm, uint8_t *gaps, uint32_t *out_pos,
               uint64_t *total_bits_out)
{
    uint64_t hist[256];
    uint64_t sizes[6];
    for (int s = 0; s < 256; s++) hist[s] = 0;
    int rc = orc_histogram(w, n_elements, hist);
    if (rc) return rc;
    for (int s = 0; s < 256; s++)
        if (hist[s] > 0 && lens[s] == 0) return ORC_E_INVALID_ARG;
    uint64_t total_bits = orc_total_bits(lens, hist);
    rc = orc_layout(n_elements, total_bits, n, G, sizes);
    if (rc) return rc;
    uint64_t T = sizes[0];
    uint64_t groups = sizes[1];
    uint64_t seg_bits = 8ull * n;

    uint64_t pos = 0;      /* next bit to write */
    uint64_t t_next = 0;   /* first thread whose gap is not yet known */
    for (uint64_t i = 0; i < n_elements; i++) {
        uint32_t sign = (w[i] >> 15) & 1u;
        uint32_t e = (w[i] >> 7) & 0xFFu;
        uint32_t mant = w[i] & 0x7Fu;
        sm[i] = (uint8_t)((sign << 7) | mant);
        /* code i starts at pos: it is the first code start at or after every s_t in (previous start, pos] */
        while (t_next < T && t_next * seg_bits <= pos) {
            uint64_t gap = pos - t_next * seg_bits;
            if (gap >= ORC_MAX_LEN) return ORC_E_BAD_STREAM;
            for (int b = 0; b < 5; b++) orc_put_bit(gaps, 5 * t_next + b, (int)((gap >> (4 - b)) & 1u));
            if (t_next % G == 0) out_pos[t_next / G] = (uint32_t)i;
            t_next++;
        }
        for (int j = lens[e] - 1; j >= 0; j--) orc_put_bit(enc, pos++, (int)((codes[e] >> j) & 1u));
    }
    while (t_next < T) { /* segments after the last code start: the stream end is the sentinel start */
        uint64_t gap = pos - t_next * seg_bits;
        if (gap >= ORC_MAX_LEN) return ORC_E_BAD_STREAM;
        for (int b = 0; b < 5; b++) orc_put_bit(gaps, 5 * t_next + b, (int)((gap >> (4 - b)) & 1u));
        if (t_next % G == 0) out_pos[t_next / G] = (uint32_t)n_elements;
        t_next++;
    }
    out_pos[groups] = (uint32_t)n_elements;
    *total_bits_out = pos;
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Step 9, [GPU]: the conventional Huffman decoder walks the tree one bit at a
 * time.  That sequential walk is the oracle's decoder; it reads N codes from
 * bit 0 and merges each exponent with its sign/mantissa byte.
 * ------------------------------------------------------------------------- */
int orc_decode_treewalk(const uint8_t lens[256], const uint32_t codes[256], const uint8_t *enc, uint64_t total_bits,
                        const uint8_t *sm, uint64_t n_elements, uint16_t *w)
{
    orc_node tree[ORC_TREE_CAP];
    int n_nodes = 0;
    int rc = orc_build_tree(lens, codes, tree, &n_nodes);
    if (rc) return rc;
    uint64_t pos = 0;
    for (uint64_t i = 0; i < n_elements; i++) {
        int v = 0;
        while (tree[v].symbol < 0) {
            if (pos >= total_bits) return ORC_E_BAD_STREAM;
            v = tree[v].child[orc_get_bit(enc, pos++)];
            if (v < 0) return ORC_E_BAD_STREAM;
        }
        uint32_t sign = (sm[i] >> 7) & 1u;
        uint32_t mant = sm[i] & 0x7Fu;
        w[i] = (uint16_t)((sign << 15) | ((uint32_t)tree[v].symbol << 7) | mant);
    }
    if (pos != total_bits) return ORC_E_BAD_STREAM;
    return ORC_OK;
}

/* Same decoder over the codes of groups [g0, g1) only, starting from the stored
 * gap of the group's first thread and its stored output position.  Groups are
 * independent, so callers may run disjoint ranges on different host threads. */
int orc_decode_groups_treewalk(const uint8_t lens[256], const uint32_t codes[256], const uint8_t *enc,
                               uint64_t total_bits, const uint8_t *gaps, const uint32_t *out_pos, const uint8_t *sm,
                               uint32_t n, uint32_t G, uint64_t n_threads, uint64_t g0, uint64_t g1, uint16_t *w)
{
    orc_node tree[ORC_TREE_CAP];
    int n_nodes = 0;
    int rc = orc_build_tree(lens, codes, tree, &n_nodes);
    if (rc) return rc;
    uint64_t seg_bits = 8ull * n;
    for (uint64_t g = g0; g < g1; g++) {
        uint64_t t0 = g * G;
        if (t0 >= n_threads) break;
        uint64_t gap = 0;
        for (int b = 0; b < 5; b++) gap = (gap << 1) | (uint64_t)orc_get_bit(gaps, 5 * t0 + b);
        uint64_t pos = t0 * seg_bits + gap;
        uint64_t end_thread = t0 + G < n_threads ? t0 + G : n_threads;
        uint64_t end_bit = end_thread * seg_bits < total_bits ? end_thread * seg_bits : total_bits;
        uint64_t i = out_pos[g];
        while (pos < end_bit) {
            int v = 0;
            while (tree[v].symbol < 0) {
                if (pos >= total_bits) return ORC_E_BAD_STREAM;
                v = tree[v].child[orc_get_bit(enc, pos++)];
                if (v < 0) return ORC_E_BAD_STREAM;
            }
            if (i >= out_pos[g + 1]) return ORC_E_BAD_STREAM;
            uint32_t sign = (sm[i] >> 7) & 1u;
            uint32_t mant = sm[i] & 0x7Fu;
            w[i] = (uint16_t)((sign << 15) | ((uint32_t)tree[v].symbol << 7) | mant);
            i++;
        }
        if (i != out_pos[g + 1]) return ORC_E_BAD_STREAM;
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Decode through the LUT hierarchy instead of the tree ([LUT]): the next 8
 * bits index the current LUT; a value of 240 or more is a pointer to LUT
 * 256 - value for the following 8 bits, any other value is the exponent, and
 * CodeLengths gives how many bits it used.
 * ------------------------------------------------------------------------- */
static uint32_t orc_get_bits8(const uint8_t *buf, uint64_t pos)
{
    uint32_t x = 0;
    for (int j = 0; j < 8; j++) x = (x << 1) | (uint32_t)orc_get_bit(buf, pos + (uint64_t)j);
    return x;
}

int orc_decode_lut(const uint8_t luts[ORC_MAX_LUTS][256], uint32_t n_luts, const uint8_t code_lengths[256],
                   const uint8_t *enc, uint64_t total_bits, const uint8_t *sm, uint64_t n_elements, uint16_t *w)
{
    uint64_t pos = 0;
    for (uint64_t i = 0; i < n_elements; i++) {
        uint32_t id = 0;
        uint64_t depth = 0;
        uint32_t v;
        for (;;) {
            v = luts[id][orc_get_bits8(enc, pos + depth)];
            if (v < ORC_FIRST_POINTER) break;
            id = 256 - v;
            depth += 8;
            if (id >= n_luts || depth > 24) return ORC_E_BAD_STREAM;
        }
        if (code_lengths[v] == 0) return ORC_E_BAD_STREAM;
        pos += code_lengths[v];
        uint32_t sign = (sm[i] >> 7) & 1u;
        uint32_t mant = sm[i] & 0x7Fu;
        w[i] = (uint16_t)((sign << 15) | (v << 7) | mant);
    }
    if (pos != total_bits) return ORC_E_BAD_STREAM;
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Step 10, [Kernel]: check the auxiliary metadata against the tree.  For every
 * thread t, walk the codes that start in [s_t + gap_t, min(s_(t+1), total_bits));
 * the walk must end exactly at the next thread's first code start (or at the
 * stream end), the counts' prefix sums over each group must reproduce out_pos,
 * and the first gap must be 0.
 * counts (optional, may be NULL) receives the per-thread code counts.
 * ------------------------------------------------------------------------- */
int orc_check_metadata(const uint8_t lens[256], const uint32_t codes[256], const uint8_t *enc, uint64_t total_bits,
                       const uint8_t *gaps, const uint32_t *out_pos, uint64_t n_elements, uint32_t n, uint32_t G,
                       uint64_t n_threads, uint32_t *counts)
{
    orc_node tree[ORC_TREE_CAP];
    int n_nodes = 0;
    int rc = orc_build_tree(lens, codes, tree, &n_nodes);
    if (rc) return rc;
    uint64_t seg_bits = 8ull * n;
    uint64_t running = 0;
    uint64_t groups = (n_threads + G - 1) / G;
    for (uint64_t t = 0; t < n_threads; t++) {
        uint64_t gap = 0;
        for (int b = 0; b < 5; b++) gap = (gap << 1) | (uint64_t)orc_get_bit(gaps, 5 * t + b);
        if (t == 0 && gap != 0) return ORC_E_BAD_STREAM;
        if (t % G == 0 && out_pos[t / G] != running) return ORC_E_BAD_STREAM;
        uint64_t pos = t * seg_bits + gap;
        uint64_t end = (t + 1) * seg_bits < total_bits ? (t + 1) * seg_bits : total_bits;
        uint32_t c = 0;
        while (pos < end) {
            int v = 0;
            while (tree[v].symbol < 0) {
                if (pos >= total_bits) return ORC_E_BAD_STREAM;
                v = tree[v].child[orc_get_bit(enc, pos++)];
                if (v < 0) return ORC_E_BAD_STREAM;
            }
            c++;
        }
        /* the walk must stop exactly where the next thread's first code starts */
        uint64_t next_start = total_bits;
        if (t + 1 < n_threads) {
            uint64_t next_gap = 0;
            for (int b = 0; b < 5; b++) next_gap = (next_gap << 1) | (uint64_t)orc_get_bit(gaps, 5 * (t + 1) + b);
            next_start = (t + 1) * seg_bits + next_gap;
        }
        if (pos != next_start) return ORC_E_BAD_STREAM;
        if (counts) counts[t] = c;
        running += c;
    }
    if (running != n_elements) return ORC_E_BAD_STREAM;
    if (out_pos[groups] != n_elements) return ORC_E_BAD_STREAM;
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * rANS exponent coder.  The page's discussion ("Opini Hacker News") names
 * rANS as an entropy coder that suits SIMD-style instruction sets better than
 * Huffman; the page gives no format, so the one below is this project's
 * reading: the plain static rANS of Duda's asymmetric numeral systems with
 * 16-bit renormalisation, laid out for 64-lane waves.
 *   - The exponent histogram is quantized to frequencies f[s] summing to
 *     M = 2^prob_bits (orc_rans_quantize); c[s] = f[0] + ... + f[s - 1].
 *   - A state x lives in [L, 2^32), L = 2^16.  Encoding s from x first
 *     emits the low 16 bits of x and shifts them out while x >= f[s] *
 *     2^(32 - prob_bits), then sets x = floor(x / f[s]) * M + (x mod f[s]) +
 *     c[s].  Decoding inverts it: slot = x mod M, s is the symbol with
 *     c[s] <= slot < c[s] + f[s], x = f[s] * floor(x / M) + slot - c[s], and
 *     if x < L, x = x * 2^16 + the next word (one word at most per symbol).
 *   - The exponents are cut into segments of lanes x steps symbols; in a
 *     segment, lane l codes the positions step * lanes + l (step = 0, 1, ...)
 *     with a state of its own, which starts at L in the encoder.  The
 *     decoder reads a segment's words in the order step ascending, lane
 *     ascending, one for each lane whose state fell below L; the encoder
 *     therefore runs step descending, lane descending, and its words are
 *     stored reversed.  Per segment the stream keeps the lanes' final encoder
 *     states (the decoder's start states) and the offset of its words.
 * Sign and mantissa bytes are stored as in DF11.
 * ------------------------------------------------------------------------- */
#define ORC_RANS_L 65536u

/* Frequencies: every used exponent gets max(1, floor(hist * M / N)); if the
 * sum is below M the difference goes to the most frequent exponent (lowest
 * value on ties); while it is above M the largest frequency above 1 (lowest
 * value on ties) drops by one. */
int orc_rans_quantize(const uint64_t hist[256], uint32_t prob_bits, uint32_t freq[256])
{
    if (prob_bits < 1 || prob_bits > 16) return ORC_E_INVALID_ARG;
    const uint64_t M = 1ull << prob_bits;
    uint64_t n = 0, used = 0;
    for (int s = 0; s < 256; s++) {
        n += hist[s];
        used += hist[s] > 0;
        freq[s] = 0;
    }
    if (n == 0) return ORC_OK;
    if (used > M) return ORC_E_INVALID_ARG;
    uint64_t sum = 0;
    int top = -1;
    for (int s = 0; s < 256; s++) {
        if (!hist[s]) continue;
        uint64_t f = (uint64_t)(((unsigned __int128)hist[s] * M) / n);
        freq[s] = (uint32_t)(f ? f : 1);
        sum += freq[s];
        if (top < 0 || hist[s] > hist[top]) top = s;
    }
    if (sum < M) freq[top] += (uint32_t)(M - sum);
    while (sum > M) {
        int big = -1;
        for (int s = 0; s < 256; s++)
            if (freq[s] > 1 && (big < 0 || freq[s] > freq[big])) big = s;
        freq[big]--;
        sum--;
    }
    return ORC_OK;
}

static void orc_rans_cum(const uint32_t freq[256], uint32_t cum[257])
{
    cum[0] = 0;
    for (int s = 0; s < 256; s++) cum[s + 1] = cum[s] + freq[s];
}

/* Encode n BF16 words.  states: n_segments * lanes; word_offsets:
 * n_segments + 1 (word_offsets[g] is segment g's first word); words: room for
 * words_cap (n suffices: at most one word per symbol); sm: n bytes.  Returns
 * the number of words in *n_words. */
int orc_rans_encode(const uint16_t *w, uint64_t n, uint32_t prob_bits, const uint32_t freq[256], uint32_t lanes,
                    uint32_t steps, uint32_t *states, uint64_t *word_offsets, uint16_t *words, uint64_t words_cap,
                    uint64_t *n_words, uint8_t *sm)
{
    if (prob_bits < 1 || prob_bits > 16 || lanes == 0 || steps == 0) return ORC_E_INVALID_ARG;
    uint32_t cum[257];
    orc_rans_cum(freq, cum);
    if (n && cum[256] != (1u << prob_bits)) return ORC_E_INVALID_ARG;
    const uint64_t seg = (uint64_t)lanes * steps;
    const uint64_t n_seg = (n + seg - 1) / seg;
    uint32_t *x = (uint32_t *)malloc(sizeof(uint32_t) * lanes);
    uint16_t *stack = (uint16_t *)malloc(sizeof(uint16_t) * (seg ? seg : 1));
    if (!x || !stack) {
        free(x);
        free(stack);
        return ORC_E_INVALID_ARG;
    }
    uint64_t total = 0;
    int rc = ORC_OK;
    for (uint64_t g = 0; g < n_seg && rc == ORC_OK; g++) {
        const uint64_t base = g * seg;
        const uint64_t count = n - base < seg ? n - base : seg;
        uint64_t top = 0;
        for (uint32_t l = 0; l < lanes; l++) x[l] = ORC_RANS_L;
        for (uint64_t j = steps; j-- > 0 && rc == ORC_OK;) {
            for (uint32_t l = lanes; l-- > 0;) {
                const uint64_t q = j * lanes + l;
                if (q >= count) continue;
                const uint32_t s = (w[base + q] >> 7) & 0xFFu;
                const uint32_t f = freq[s];
                if (s >= ORC_FIRST_POINTER) { rc = ORC_E_RESERVED_EXPONENT; break; }
                if (f == 0) { rc = ORC_E_INVALID_ARG; break; }
                const uint64_t x_max = (uint64_t)f << (32 - prob_bits);
                while (x[l] >= x_max) {
                    stack[top++] = (uint16_t)(x[l] & 0xFFFFu);
                    x[l] >>= 16;
                }
                x[l] = (x[l] / f << prob_bits) + x[l] % f + cum[s];
            }
        }
        if (rc != ORC_OK) break;
        if (total + top > words_cap) { rc = ORC_E_BUFFER_TOO_SMALL; break; }
        word_offsets[g] = total;
        for (uint64_t i = 0; i < top; i++) words[total + i] = stack[top - 1 - i];
        total += top;
        for (uint32_t l = 0; l < lanes; l++) states[g * lanes + l] = x[l];
    }
    free(x);
    free(stack);
    if (rc != ORC_OK) return rc;
    word_offsets[n_seg] = total;
    *n_words = total;
    for (uint64_t i = 0; i < n; i++) sm[i] = (uint8_t)(((w[i] >> 8) & 0x80u) | (w[i] & 0x7Fu));
    return ORC_OK;
}

/* Decode the stream above into n BF16 words.  Fails with ORC_E_BAD_STREAM if
 * a segment needs more words than it has, leaves some unread, or does not
 * return every state to L (the encoder's start). */
int orc_rans_decode(const uint32_t freq[256], uint32_t prob_bits, uint32_t lanes, uint32_t steps,
                    const uint32_t *states, const uint64_t *word_offsets, const uint16_t *words, const uint8_t *sm,
                    uint64_t n, uint16_t *w)
{
    if (prob_bits < 1 || prob_bits > 16 || lanes == 0 || steps == 0) return ORC_E_INVALID_ARG;
    if (n == 0) return ORC_OK;
    uint32_t cum[257];
    orc_rans_cum(freq, cum);
    const uint32_t M = 1u << prob_bits;
    if (cum[256] != M) return ORC_E_BAD_STREAM;
    uint8_t *sym = (uint8_t *)malloc(M);
    uint32_t *x = (uint32_t *)malloc(sizeof(uint32_t) * lanes);
    if (!sym || !x) {
        free(sym);
        free(x);
        return ORC_E_INVALID_ARG;
    }
    for (int s = 0; s < 256; s++)
        for (uint32_t k = cum[s]; k < cum[s + 1]; k++) sym[k] = (uint8_t)s;
    const uint64_t seg = (uint64_t)lanes * steps;
    const uint64_t n_seg = (n + seg - 1) / seg;
    int rc = ORC_OK;
    for (uint64_t g = 0; g < n_seg && rc == ORC_OK; g++) {
        const uint64_t base = g * seg;
        const uint64_t count = n - base < seg ? n - base : seg;
        uint64_t ptr = word_offsets[g];
        const uint64_t ptr_end = word_offsets[g + 1];
        for (uint32_t l = 0; l < lanes; l++) x[l] = states[g * lanes + l];
        for (uint64_t j = 0; j < steps && rc == ORC_OK; j++) {
            for (uint32_t l = 0; l < lanes; l++) {
                const uint64_t q = j * lanes + l;
                if (q >= count) continue;
                const uint32_t slot = x[l] & (M - 1);
                const uint32_t s = sym[slot];
                x[l] = freq[s] * (x[l] >> prob_bits) + slot - cum[s];
                if (x[l] < ORC_RANS_L) {
                    if (ptr >= ptr_end) { rc = ORC_E_BAD_STREAM; break; }
                    x[l] = (x[l] << 16) | words[ptr++];
                }
                const uint32_t b = sm[base + q];
                w[base + q] = (uint16_t)(((b & 0x80u) << 8) | (s << 7) | (b & 0x7Fu));
            }
        }
        if (rc != ORC_OK) break;
        if (ptr != ptr_end) rc = ORC_E_BAD_STREAM;
        for (uint32_t l = 0; l < lanes && rc == ORC_OK; l++)
            if (x[l] != ORC_RANS_L) rc = ORC_E_BAD_STREAM;
    }
    free(sym);
    free(x);
    return rc;
}
