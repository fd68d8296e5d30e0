// gfx950 DF11 decoder and the device entry points of the C ABI.
//
// Method: "DFloat11: Kompresi inferensi GPU lossless yang mengecilkan LLM
// menjadi 70% ukurannya" (GeekNews), sections "Decoding berbasis LUT
// hierarkis", "Kernel GPU 2 tahap dan metadata bantu" and "Dekompresi per
// transformer block".
//
// One workgroup of 256 threads (four wave64s) decodes one group of the stream
// at a time and loops over groups (persistent grid sized to the chip), so the
// decode tables are staged into LDS once per workgroup rather than once per
// group.  Per group:
//   1. each thread loads its 8-byte EncodedExponent segment plus the 4 bytes
//      after it, and its 5-bit gap (the first code start in the segment);
//      the group's PackedSignMantissa bytes are prefetched into registers;
//   2. phase 1: the thread walks its segment's codes and counts them, writing
//      nothing;
//   3. a wave64 DPP scan plus an LDS scan over the four waves turn the counts
//      into offsets within the group; the stored group offset out_pos[g] makes
//      them global;
//   4. phase 2: the thread decodes its segment again and writes the exponents
//      into an LDS buffer at its offset;
//   5. the workgroup merges exponents with sign/mantissa and writes BF16 with
//      16-byte coalesced stores.
//
// Decoding a code: the next K bits index a first-level LDS table that lists
// every complete code at the start of the window (up to five), so one lookup
// resolves several of the 2-3 bit codes that dominate LLM exponents.  A window
// whose first code is longer than K bits continues in the page's LUT hierarchy
// (256-entry LUTs, values 240..255 pointing to lower LUTs) and CodeLengths,
// which are also staged in LDS.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <numeric>
#include <vector>

#include <stdint.h>
#include <string.h>

#include "df11.h"
#include "df11_device.h"
#include "df11_internal.h"
#include "df11_launch.h"
#include "df11_pairs.h"

namespace {

using df11::kBytesPerThread;
using df11::kThreadsPerGroup;
constexpr uint32_t kWaves = kThreadsPerGroup / kWaveSize;
constexpr uint32_t kSegBits = 8 * kBytesPerThread;
constexpr int kPrefetchChunks = 4;  // 8-element sign/mantissa chunks held in registers per thread
constexpr uint32_t kDefaultGroupsPerWorkgroup = 2;
// Bytes of an exponent buffer that one thread's phase 2 can reach past its
// first output: at most 64 + 11 codes start in the bits it walks (every code
// is at least one bit), and the last OR touches the 8 aligned bytes around
// its address.  A thread's start offset is clamped this far below the end of
// the buffer, which no valid stream reaches (the buffer holds the largest
// group plus this much), so a corrupt one stays inside it.
constexpr uint32_t kDecodeReach = 96;
constexpr uint32_t kLongCode = df11::kLongCodeIncrement;
// Table lookups per 32-bit half segment whose entries phase 1 keeps in
// registers for phase 2 (LLM-like exponent streams need 3..5 at K = 11; a
// wave that needs more decodes phase 2 again from the stream).
constexpr int kSavedSteps = 5;

struct DecodeArgs {
    const uint8_t *enc;
    const uint8_t *sm;
    const uint8_t *gaps;
    const uint32_t *out_pos;
    const uint8_t *luts;
    const uint8_t *code_lengths;
    const uint32_t *dtab;
    uint16_t *out;
    uint64_t total_bits;
    uint32_t n_elements;
    uint32_t n_threads;
    uint32_t n_groups;
    uint32_t n_luts;
    uint32_t ebuf_cap;       // bytes of the LDS exponent buffer, a multiple of 16
    uint32_t last_seg_bits;  // payload bits in the last thread's segment (1..64)
    uint32_t sm_chunks;      // 8-byte chunks in the PackedSignMantissa buffer
    uint32_t tile_cols;      // 0, or the columns C of a matrix held in MFMA tile order
    uint32_t *sched;         // work counters (dynamic schedule) or null
    uint32_t pools;          // dynamic schedule: counters in use, dividing the workgroup count
    uint32_t tile_ks;        // C / 32: k-steps per 64-row panel of a tiled matrix
    uint64_t tile_magic;     // floor(2^64 / tile_ks) + 1: umulhi64(i, tile_magic) == i / tile_ks, i < 2^32
};

// MFMA tile order (df11_tile_order): 512-element blocks, each the operand
// of one 16 x 16 x 32 bf16 matrix instruction; block b is n-tile b mod 4 of
// global k-step b / 4, and global k-step g is k-step g mod (C / 32) of the
// 64-row panel g / (C / 32).  Lane l of a block holds the 8 elements of row
// 16 nt + (l mod 16), columns 32 ks + 8 (l / 16) .. + 7.  Element index in
// the row-major matrix of the first element of chunk c (8 elements):
__device__ __forceinline__ uint32_t tiled_chunk_origin(const DecodeArgs &a, uint32_t c) {
    const uint32_t l = c & 63u, nt = (c >> 6) & 3u, g = c >> 8;
    const uint32_t panel = static_cast<uint32_t>(__umul64hi(g, a.tile_magic));
    const uint32_t ks = g - panel * a.tile_ks;
    return (64u * panel + 16u * nt + (l & 15u)) * a.tile_cols + 32u * ks + 8u * (l >> 4);
}

// The fused decode + matmul: y = x W^T, W (out_features x in_features,
// row-major) being the decoded stream.
struct MatmulArgs {
    const uint16_t *x;     // n_tokens x in_features BF16, row-major, 16-byte aligned
    float *y;              // n_tokens x out_features, zero when the kernel starts
    uint64_t row_magic;    // floor(2^64 / in_features) + 1: row of element i = umulhi64(i, row_magic)
    uint32_t in_features;  // a multiple of 8, at least 512
    uint32_t out_features;
    uint32_t n_tokens;     // 1 .. the kernel's token slots (any count for the matrix-core product)
    uint32_t yacc_rows;    // rows of W that one group's outputs can touch
    uint32_t passes;       // matrix-core product: sweeps of the stream, 16 MT tokens each
    uint32_t fixed_len;    // matrix-core product with a dealt tail: super-groups of each fixed range
};

__device__ __forceinline__ uint32_t bswap32(uint32_t x) { return __builtin_amdgcn_perm(x, x, 0x00010203u); }

// Continue a code longer than the first-level window through the LUT
// hierarchy.  ptr is the root LUT's pointer value for the window's first byte.
// Returns the exponent and its code length (at least 1 even for a corrupt
// stream, so decoding always advances).
__device__ __forceinline__ uint32_t walk_luts(uint32_t win, uint32_t ptr, const uint8_t *s_luts,
                                              const uint8_t *s_clen, uint32_t n_luts, uint32_t &len) {
    uint32_t v = ptr;
    uint32_t shift = 16;
#pragma unroll
    for (int level = 0; level < 3; ++level) {
        if (v >= DF11_FIRST_POINTER) {
            const uint32_t id = min(256u - v, n_luts - 1u);
            v = s_luts[id * 256u + ((win >> shift) & 0xFFu)];
        }
        shift -= 8;
    }
    const uint32_t l = s_clen[v];
    len = l ? l : 32u;
    return v;
}

// Build the first-level decode table in LDS from the staged LUTs and
// CodeLengths, for a stream given without one, so that it holds exactly what
// df11_build_decode_table writes for the same codebook.  Two passes over the
// 2^K windows, with the bits past a window taken as zero (a code inside the
// window decodes the same either way, and one that does not cannot fit):
//   1. s_first[x]: the first code of window x, through the LUT hierarchy:
//      its rotated exponent and its length, or 0 if it is longer than K;
//   2. entry x: the code at offset u of window x is the first code of window
//      (x << u) mod 2^K when it fits in the K - u bits left, so the run of
//      complete codes is a chain of s_first reads.
// Each thread takes kPer windows at once, so that their chains of dependent
// LDS reads overlap.
template <int K, uint32_t kThreads>
__device__ __forceinline__ void derive_table(uint32_t *s_tab, uint16_t *s_first, const uint8_t *s_luts,
                                             const uint8_t *s_clen, uint32_t n_luts, uint32_t tid) {
    constexpr uint32_t kSize = 1u << K;
    constexpr uint32_t kPer = (kSize + kThreads - 1) / kThreads;
    constexpr uint32_t kBatch = kPer < 4 ? kPer : 4;  // windows in flight per thread
    // Both passes are branch-free (every lookup is made, selects pick the
    // result), so that the windows' chains of dependent LDS reads overlap.
    for (uint32_t j0 = 0; j0 < kPer; j0 += kBatch) {
        uint32_t v[kBatch];
#pragma unroll
        for (uint32_t j = 0; j < kBatch; ++j) v[j] = s_luts[min(tid + (j0 + j) * kThreads, kSize - 1u) >> (K - 8)];
#pragma unroll
        for (uint32_t level = 1; level < 4; ++level) {
#pragma unroll
            for (uint32_t j = 0; j < kBatch; ++j) {
                const uint32_t x = min(tid + (j0 + j) * kThreads, kSize - 1u);
                const uint32_t byte = ((x << (32 - K)) >> (24 - 8 * level)) & 0xFFu;
                const bool ptr = v[j] >= DF11_FIRST_POINTER;
                const uint32_t id = ptr ? min(256u - v[j], n_luts - 1u) : 0u;
                const uint32_t nv = s_luts[id * 256u + byte];
                v[j] = ptr ? nv : v[j];
            }
        }
#pragma unroll
        for (uint32_t j = 0; j < kBatch; ++j) {
            const uint32_t x = tid + (j0 + j) * kThreads;
            const uint32_t len = s_clen[v[j]];
            if (x < kSize)
                s_first[x] = static_cast<uint16_t>(len && len <= K ? df11::rotate_exponent(v[j]) | (len << 8) : 0u);
        }
    }
    __syncthreads();
    uint16_t *s_start = reinterpret_cast<uint16_t *>(s_tab + (2u << K));
    for (uint32_t j0 = 0; j0 < kPer; j0 += kBatch) {
        uint32_t used[kBatch], lo[kBatch], fifth[kBatch], mask[kBatch], m[kBatch];
        bool open[kBatch];
#pragma unroll
        for (uint32_t j = 0; j < kBatch; ++j) {
            used[j] = lo[j] = fifth[j] = mask[j] = m[j] = 0;
            open[j] = true;
        }
#pragma unroll
        for (uint32_t step = 0; step < df11::kDecodeTableMaxSyms; ++step) {
#pragma unroll
            for (uint32_t j = 0; j < kBatch; ++j) {
                const uint32_t x = min(tid + (j0 + j) * kThreads, kSize - 1u);
                const uint32_t f = s_first[(x << used[j]) & (kSize - 1u)];
                const uint32_t len = f >> 8;
                open[j] = open[j] && len != 0 && len <= K - used[j];
                const uint32_t r = open[j] ? f & 0xFFu : 0u;
                if (step < 4) {
                    lo[j] |= r << (8 * step);
                } else {
                    fifth[j] = r;
                }
                mask[j] |= open[j] ? 1u << used[j] : 0u;
                used[j] += open[j] ? len : 0u;
                m[j] += open[j] ? 1u : 0u;
            }
        }
#pragma unroll
        for (uint32_t j = 0; j < kBatch; ++j) {
            const uint32_t x = tid + (j0 + j) * kThreads;
            if (x < kSize) {
                s_tab[2 * x] = lo[j];
                s_tab[2 * x + 1] = m[j] ? ((m[j] << 11) + used[j]) | (fifth[j] << 16) : df11::kLongCodeIncrement;
                s_start[x] = static_cast<uint16_t>(m[j] ? mask[j] : 1u);
            }
        }
    }
}

__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    // Hillis-Steele within each row of 16 lanes, then across rows.
    x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
    return x;
}

// Sum of v over the wave, complete in lane 63 (the scan above on floats).
__device__ __forceinline__ float wave_total(float v) {
#define DF11_DPP_ADD(ctrl, rows)                                                                           \
    v += __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), ctrl, rows, 0xF, false))
    DF11_DPP_ADD(0x111, 0xF);
    DF11_DPP_ADD(0x112, 0xF);
    DF11_DPP_ADD(0x114, 0xF);
    DF11_DPP_ADD(0x118, 0xF);
    DF11_DPP_ADD(0x142, 0xA);
    DF11_DPP_ADD(0x143, 0xC);
#undef DF11_DPP_ADD
    return v;
}

using LdsU8 = __attribute__((address_space(3))) uint8_t;
using LdsU32 = __attribute__((address_space(3))) uint32_t;

// 32-bit LDS offset of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_offset(const uint8_t *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const LdsU8 *)p));
}

// OR the 5-byte exponent run x (byte 0 first; unused bytes zero) into LDS at
// the byte address held in acc = (address << 11) | p, p < 256.  LDS stores
// that are not naturally aligned are several times slower on gfx950, so x is
// shifted into the two aligned dwords it spans and combined with aligned
// atomic ORs; zero bytes leave their neighbours untouched.  Bits 8..10 of acc
// are zero, so bits 8..12 are (address & 3) * 8, the shift.
__device__ __forceinline__ void or_exponents(uint32_t acc, uint64_t x) {
    const uint64_t xs = x << __builtin_amdgcn_ubfe(acc, 8, 5);
    LdsU32 *d = (LdsU32 *)(uintptr_t)((acc >> 11) & ~3u);
    __hip_atomic_fetch_or(d, static_cast<uint32_t>(xs), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __hip_atomic_fetch_or(d + 1, static_cast<uint32_t>(xs >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// out_pos is read-only for the whole kernel and indexed by a wave-uniform
// group number: reading it through the constant address space gives scalar
// loads, which are counted apart from the vector-memory operations.

__device__ __forceinline__ uint32_t out_pos_at(const DecodeArgs &a, uint32_t g) {
    return ((const ConstU32 *)a.out_pos)[min(g, a.n_groups)];
}



// Number of 8-element chunks that hold the outputs [base, end).
__device__ __forceinline__ uint32_t group_chunks(uint32_t base, uint32_t end) {
    return end > base ? ((end + 7u) >> 3) - (base >> 3) : 0u;
}

// Per-thread inputs of one group, loaded one loop iteration before they are
// used.  On gfx9 one counter tracks loads and stores in issue order, so a
// group's inputs are loaded before the previous group's stores are issued:
// waiting for them then does not wait for those stores.
struct GroupLoad {
    uint32_t e0, e1, e2, e3;       // the thread's EncodedExponent words (bytes 8t .. 8t+15)
    uint32_t g0, g1;               // the two Gaps words that hold its 5 bits
};

// Issues the same loads for every group (addresses clamped into the buffers,
// values of out-of-range items unused) so that the number of operations in
// flight is the same on every path.
__device__ __forceinline__ GroupLoad load_group(const DecodeArgs &a, uint32_t g, uint32_t ltid) {
    GroupLoad r;
    const uint32_t t = min(g * kThreadsPerGroup + ltid, a.n_threads - 1u);
    const uint32_t *e32 = reinterpret_cast<const uint32_t *>(a.enc + 8ull * t);
    r.e0 = e32[0];
    r.e1 = e32[1];
    r.e2 = e32[2];
    r.e3 = e32[3];
    const uint64_t gbit = 5ull * t;
    const uint32_t *g32 = reinterpret_cast<const uint32_t *>(a.gaps) + (gbit >> 5);
    r.g0 = g32[0];
    r.g1 = g32[1];
    return r;
}

// Sign/mantissa chunks of the group with outputs [base, end) that this
// thread merges in its first kPrefetchChunks rounds, loaded (clamped like
// load_group) one iteration before the merge uses them: chunk ltid + 256 j
// for the store, or round j of the thread's wave run for the fused matmul
// (run_chunk).  Each byte is read once, so the loads are non-temporal (they
// do not displace the encoded words, which neighbouring threads share, from
// the caches); the block decode took 122-123 us with them against 126-127.
template <int TB>
__device__ __forceinline__ void load_sm(const DecodeArgs &a, uint32_t base, uint32_t end, uint32_t ltid,
                                        uint64_t (&sm)[kPrefetchChunks]);

// Byte offset of the first-level table entry (a pair of uint32: the
// exponent run, then the aux word) for the K-bit window at bit p = acc & 63
// of the 64-bit pair.  The entry's start mask is the uint16 at byte offset
// (offset >> 2) of the masks.
template <int K>
__device__ __forceinline__ uint32_t entry_offset(uint64_t pair, uint32_t acc) {
    return (static_cast<uint32_t>((pair << (acc & 63u)) >> 32) >> (29 - K)) & ~7u;
}

template <typename T>
__device__ __forceinline__ T lds_at(const void *base, uint32_t byte_offset) {
    return *reinterpret_cast<const T *>(reinterpret_cast<const uint8_t *>(base) + byte_offset);
}

// Bits [p, p + 32) of the thread's 96-bit window (w0 w1 w2, MSB-first), p < 64.
__device__ __forceinline__ uint32_t window_at(uint64_t pa, uint64_t pb, uint32_t p) {
    return static_cast<uint32_t>((p < 32u ? pa << p : pb << (p - 32u)) >> 32);
}

// Merge one decoded group's exponents with its sign/mantissa bytes and store
// BF16.  LDS byte 8k + i of the group's buffer holds element 8 (base/8 + k) + i;
// every chunk read is zeroed again for the next group that uses the buffer.
// skip_first: the previous group's workgroup wrote the chunk this group shares
// with it; whole_last: this group's buffer also holds the next group's
// elements of their shared chunk, which is written whole.
__device__ __forceinline__ void merge_group(const DecodeArgs &a, uint8_t *ebuf, const uint64_t (&sm)[kPrefetchChunks],
                                            uint32_t base, uint32_t end, uint32_t ltid, bool skip_first,
                                            bool whole_last) {
    const uint32_t c0 = base >> 3;
    const uint32_t n_chunks = min(group_chunks(base, end), a.ebuf_cap / 8u);
    const uint32_t store_base = skip_first ? (base + 7u) & ~7u : base;
    // A valid stream always has elements after a group whose last chunk is
    // written whole; the clamp keeps a corrupt one inside out.
    const uint32_t store_end = whole_last ? min((end + 7u) & ~7u, a.n_elements) : end;
    // A matrix in MFMA tile order goes back to row-major: each chunk is 8
    // consecutive elements of one row (tiled_chunk_origin), and a wave's 64
    // chunks are 16 rows x 64 bytes, half cache lines whose other halves
    // another wave writes.  Those stores go through the L2 (not
    // non-temporal), which joins the halves before they reach memory: the
    // per-weight block decoded in 214 us that way against 437 us with
    // non-temporal stores (and 134 us in row order).
    auto store = [&](uint32_t c, uint4 v) {
        if (a.tile_cols) {
            const uint32_t dst = tiled_chunk_origin(a, c), first = 8u * c;
            if (first >= store_base && first + 8u <= store_end) {
                *reinterpret_cast<uint4 *>(a.out + dst) = v;
            } else {
                store_chunk_at(a.out, dst, first, v, store_base, store_end);
            }
        } else {
            store_chunk(a.out, c, v, store_base, store_end);
        }
    };
#pragma unroll
    for (int j = 0; j < kPrefetchChunks; ++j) {
        const uint32_t k = ltid + j * kThreadsPerGroup;
        if (k < n_chunks) {
            uint64_t *cell = reinterpret_cast<uint64_t *>(ebuf + 8u * k);
            const uint64_t r8 = *cell;
            *cell = 0;
            store(c0 + k, merge8(sm[j], r8));
        }
    }
    for (uint32_t k = ltid + kPrefetchChunks * kThreadsPerGroup; k < n_chunks; k += kThreadsPerGroup) {
        const uint64_t s8 = __builtin_nontemporal_load(reinterpret_cast<const uint64_t *>(a.sm + 8ull * (c0 + k)));
        uint64_t *cell = reinterpret_cast<uint64_t *>(ebuf + 8u * k);
        const uint64_t r8 = *cell;
        *cell = 0;
        store(c0 + k, merge8(s8, r8));
    }
    // Codes past the group's last output reach at most 4 bytes into the next chunk.
    if (ltid == 0 && 8u * (n_chunks + 1u) <= a.ebuf_cap) *reinterpret_cast<uint64_t *>(ebuf + 8u * n_chunks) = 0;
}

// merge_group for a matrix in MFMA tile order whose panels hold an even
// number of k-steps: it goes back to row-major in whole 128-byte lines.  Two
// consecutive k-steps of a panel are 64 consecutive columns of its rows, so
// the group's chunks are taken in pair-rounds aligned to 512 chunks
// (df11_pairs.h): in pair-round p, wave w merges n-tile w of both k-steps,
// reading its LDS exponent cells in order as merge_group does, puts the
// merged chunks into a per-wave LDS stage, and stores them row by row, eight
// lanes to a line.  (Stored in the order merged, each 16-row, 32-column
// block left half lines: the per-weight block decoded in 211 us that way
// against 131 us in row order.)  Chunks outside the group are neither read
// nor stored.
using df11::kPairUnits;
constexpr uint32_t kPairStageBytes = 2u * kPairUnits * 16u;  // per wave

__device__ __forceinline__ void merge_group_pairs(const DecodeArgs &a, uint8_t *ebuf,
                                                  const uint64_t (&sm)[kPrefetchChunks], uint32_t base, uint32_t end,
                                                  uint32_t ltid, bool skip_first, bool whole_last, uint4 *stage) {
    const uint32_t c0 = base >> 3;
    const uint32_t n_chunks = min(group_chunks(base, end), a.ebuf_cap / 8u);
    const uint32_t store_base = skip_first ? (base + 7u) & ~7u : base;
    const uint32_t store_end = whole_last ? min((end + 7u) & ~7u, a.n_elements) : end;
    uint32_t lane = ltid & (kWaveSize - 1u);
    // (recomputed at every merge: the lane constants below, hoisted out of
    // the decoder's loop, would hold registers through the decode)
    asm volatile("" : "+v"(lane));
    const uint32_t wave = ltid / kWaveSize;
    const uint32_t h_src = df11::pair_src_half(lane), l_src0 = df11::pair_src_lane(lane, 0);
    const uint32_t lane_dst = df11::pair_lane_dst(lane, 0, a.tile_cols);
    const uint32_t n_pr = df11::pair_rounds(c0, n_chunks);
    auto pair_round = [&](uint32_t p, uint64_t s0, uint64_t s1) {
        const uint32_t cb = df11::pair_chunk(c0, p, 0, ltid - lane);  // the wave's lane 0, half 0
        const uint32_t g = cb >> 8;                                    // global k-step of half 0 (even)
        const uint32_t panel = static_cast<uint32_t>(__umul64hi(g, a.tile_magic));
        const uint32_t wave_dst = df11::pair_wave_dst(panel, g - panel * a.tile_ks, a.tile_cols, wave);
#pragma unroll
        for (uint32_t h = 0; h < 2; ++h) {
            const uint32_t k = cb + 256u * h + lane - c0;  // (wraps past n_chunks before c0)
            uint4 v = make_uint4(0, 0, 0, 0);
            if (k < n_chunks) {
                uint64_t *cell = reinterpret_cast<uint64_t *>(ebuf + 8u * k);
                const uint64_t r8 = *cell;
                *cell = 0;
                v = merge8(h ? s1 : s0, r8);
            }
            stage[df11::pair_unit(h, lane)] = v;
        }
        // The wave's own LDS operations complete in order; this keeps the
        // compiler from moving the reads of other lanes' values above the writes.
        __builtin_amdgcn_wave_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
        for (uint32_t s = 0; s < 2; ++s) {
            const uint32_t l_src = l_src0 + 8u * s;
            const uint32_t c = cb + 256u * h_src + l_src;
            if (c - c0 < n_chunks) {
                const uint4 v = stage[df11::pair_unit(h_src, l_src)];
                const uint32_t dst = wave_dst + lane_dst + 8u * s * a.tile_cols;
                // A line the group holds whole bypasses the caches; one whose
                // other part a neighbouring group writes goes through them
                // (partial lines written non-temporally from two workgroups
                // are several times slower).
                const bool whole = 8u * c >= store_base && 8u * c + 8u <= store_end;
                if (whole && df11::pair_line_whole(cb, l_src, c0, n_chunks)) {
                    u32x4 x = {v.x, v.y, v.z, v.w};
                    __builtin_nontemporal_store(x, reinterpret_cast<u32x4 *>(a.out + dst));
                } else if (whole) {
                    *reinterpret_cast<uint4 *>(a.out + dst) = v;
                } else {
                    store_chunk_at(a.out, dst, 8u * c, v, store_base, store_end);
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };
    if (n_pr > 0u) pair_round(0, sm[0], sm[1]);
    if (n_pr > 1u) pair_round(1, sm[2], sm[3]);
    for (uint32_t p = 2; p < n_pr; ++p) {  // (groups of more than 1024 chunks)
        const uint32_t c = df11::pair_chunk(c0, p, 0, ltid);
        pair_round(p, __builtin_nontemporal_load(reinterpret_cast<const uint64_t *>(a.sm + 8ull * min(c, a.sm_chunks - 1u))),
                   __builtin_nontemporal_load(
                       reinterpret_cast<const uint64_t *>(a.sm + 8ull * min(c + 256u, a.sm_chunks - 1u))));
    }
    // Codes past the group's last output reach at most 4 bytes into the next chunk.
    if (ltid == 0 && 8u * (n_chunks + 1u) <= a.ebuf_cap) *reinterpret_cast<uint64_t *>(ebuf + 8u * n_chunks) = 0;
}

// Fused matmul (y = x W^T) in place of the store.  A group's chunks are
// split into four contiguous runs, one per wave, taken 64 chunks (one per
// lane) per round; chunk k holds W's elements 8 (c0 + k) .. + 7, all in one
// row since in_features is a multiple of 8.  Each lane multiplies its chunk
// by the tokens' matching 8 columns of x (BF16 pairs straight into
// v_dot2c_f32_bf16, whose products are exact in float) and keeps a running
// sum per token for the wave's current row.  A round spans 512 elements, so
// at most two rows (in_features >= 512); when the row changes the wave adds
// its lanes' sums (DPP) and lane 63 adds them into the workgroup's LDS row
// sums yacc, which flush_rows later adds into y.  The rows of one wave's run
// only grow, so a wave reduces about once per row it touches.
__device__ __forceinline__ uint32_t wave_rounds(uint32_t n_chunks) {
    return (n_chunks + kThreadsPerGroup - 1u) / kThreadsPerGroup;
}

// Chunk of lane `lane` of wave `wave` in round j of a group with n_chunks
// chunks (the runs of merge_matmul; load_sm prefetches the same chunks).
__device__ __forceinline__ uint32_t run_chunk(uint32_t wave, uint32_t lane, uint32_t j, uint32_t n_chunks) {
    return (wave * wave_rounds(n_chunks) + j) * kWaveSize + lane;
}

template <int TB, bool kPairs = false>
__device__ __forceinline__ void load_sm(const DecodeArgs &a, uint32_t base, uint32_t end, uint32_t ltid,
                                        uint64_t (&sm)[kPrefetchChunks]) {
    const uint32_t c0 = base >> 3;
    const uint32_t nch = min(group_chunks(base, end), a.ebuf_cap / 8u);
#pragma unroll
    for (int j = 0; j < kPrefetchChunks; ++j) {
        // (the matrix-core product takes rounds aligned to 256 chunks: mfma_chunk; merge_group_pairs
        // pair-rounds aligned to 512, register j holding half j mod 2 of pair-round j / 2)
        const uint32_t k = kPairs   ? df11::pair_chunk(c0, j >> 1, j & 1, ltid) - c0
                           : TB == 0 ? ltid + j * kThreadsPerGroup
                           : TB > 0  ? run_chunk(ltid / kWaveSize, ltid & (kWaveSize - 1), j, nch)
                                     : ltid + j * kThreadsPerGroup - (c0 & 255u);
        const uint32_t c = min(c0 + (k < nch ? k : 0u), a.sm_chunks - 1u);
        sm[j] = __builtin_nontemporal_load(reinterpret_cast<const uint64_t *>(a.sm + 8ull * c));
    }
}

template <int TB>
struct RowSums {
    float acc[TB];    // this lane's sums for the wave's current row
    uint32_t row;     // the current row (wave-uniform)
    bool dirty;       // acc holds something (wave-uniform)
};

using bf16x2 = __bf16 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// Wave sums of the current row into yacc (lane 63), then start over.
template <int TB>
__device__ __forceinline__ void flush_wave(const MatmulArgs &m, RowSums<TB> &rs, uint32_t row0, float *yacc) {
    if (!rs.dirty) return;
    const bool last = (threadIdx.x & (kWaveSize - 1)) == kWaveSize - 1;
    float *ya = yacc + (rs.row - row0) * TB;
#pragma unroll
    for (int t = 0; t < TB; ++t) {
        if (t >= static_cast<int>(m.n_tokens)) break;
        const float v = wave_total(rs.acc[t]);
        if (last) __hip_atomic_fetch_add(ya + t, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        rs.acc[t] = 0.0f;
    }
    rs.dirty = false;
}

// merge_group's counterpart for the fused matmul: the group's elements [lo,
// hi) (the ones merge_group would store) go into the LDS row sums yacc, whose
// first row is row0 and which cover `rows` rows (both returned for
// flush_rows).  sm holds the chunks of rounds 0 .. kPrefetchChunks - 1 of
// this thread's run (load_sm).
//
// Wave `wave` takes the run of chunks k0 .. k0 + 64 R - 1 (k0 = 64 R wave,
// R = wave_rounds), 64 chunks per round; in a round lane l holds W's
// elements i0 .. i0 + 7, i0 = e0 + 8 l.  The run's elements only grow, so
// the row bookkeeping is one division per run and one scalar test per round:
// B is the first element of the row after the wave's current one, and a
// round spans 512 <= in_features elements, so it crosses at most B.  Lanes at
// or past B belong to the next row.  Each lane tracks the byte offset in x's
// rows of its element's column (one add and one min per round: a lane's next
// element is 512 further, at most one row on).  x is loaded a round ahead
// when the tokens' registers allow, with unconditional loads that the
// columns keep in bounds (lanes without weights multiply zeros; token slots
// past n_tokens read token 0 and are never flushed), so that each wait for x
// is an exact count; and the fused kernel runs the merge before issuing the
// next group's loads, so that those waits do not include them.
template <int TB>
__device__ __forceinline__ void load_x(const MatmulArgs &m, uint32_t colb, uint4 (&xv)[TB]) {
    const uint8_t *xb = reinterpret_cast<const uint8_t *>(m.x);
#pragma unroll
    for (int t = 0; t < TB; ++t) {
        const uint32_t tt = t < static_cast<int>(m.n_tokens) ? static_cast<uint32_t>(t) : 0u;
        xv[t] = *reinterpret_cast<const uint4 *>(xb + static_cast<size_t>(tt) * m.in_features * 2u + colb);
    }
}

template <int TB>
__device__ __forceinline__ void merge_matmul(const DecodeArgs &a, const MatmulArgs &m, uint8_t *ebuf,
                                             const uint64_t (&sm)[kPrefetchChunks], uint32_t base, uint32_t end,
                                             uint32_t ltid, bool skip_first, bool whole_last, float *yacc,
                                             uint32_t &row0, uint32_t &rows) {
    const uint32_t c0 = base >> 3;
    const uint32_t n_chunks = min(group_chunks(base, end), a.ebuf_cap / 8u);
    const uint32_t lo = skip_first ? (base + 7u) & ~7u : base;
    const uint32_t hi = whole_last ? min((end + 7u) & ~7u, a.n_elements) : end;  // (as in merge_group)
    row0 = static_cast<uint32_t>(__umul64hi(lo, m.row_magic));
    rows = lo < hi ? min(static_cast<uint32_t>(__umul64hi(hi - 1u, m.row_magic)) - row0 + 1u, m.yacc_rows) : 0u;
    const uint32_t lane = ltid & (kWaveSize - 1), wave = __builtin_amdgcn_readfirstlane(ltid / kWaveSize);
    const uint32_t n_rounds = wave_rounds(n_chunks);
    // Every chunk before n_chunks starts before hi (hi >= end), so
    // chunk_end bounds the elements that count as well as the LDS cells.
    const uint32_t chunk_end = 8u * (c0 + n_chunks);
    const uint32_t hi_eff = min(hi, chunk_end);
    const uint32_t k0 = run_chunk(wave, 0, 0, n_chunks);
    uint32_t e0 = 8u * (c0 + k0);
    const uint32_t run_end = min(e0 + 8u * kWaveSize * n_rounds, hi_eff);
    if (ltid == 0 && 8u * (n_chunks + 1u) <= a.ebuf_cap) *reinterpret_cast<uint64_t *>(ebuf + 8u * n_chunks) = 0;
    if (e0 >= run_end) return;  // (then no cell of this run is before n_chunks either)

    RowSums<TB> rs;
#pragma unroll
    for (int t = 0; t < TB; ++t) rs.acc[t] = 0.0f;
    rs.row = static_cast<uint32_t>(__umul64hi(max(e0, lo), m.row_magic));
    rs.dirty = true;
    uint32_t B = (rs.row + 1u) * m.in_features;
    // x of the first kPrefetchChunks rounds is loaded all at once (1-2
    // tokens: the decode's registers are free during the merge), one round
    // ahead (4 tokens), or in its round (8 tokens).
    constexpr bool kAll = TB <= 2;
    constexpr bool kAhead = TB <= 4;
    constexpr uint32_t kRound = 8u * kWaveSize;  // elements per round
    uint4 xv[TB], xn[TB];
    uint8_t *cell = ebuf + 8u * (k0 + lane);
    uint32_t i0 = e0 + 8u * lane;
    // Byte offset of i0's column, from i0's own row: a lane before lo can
    // lie two rows before B (lo is then the first element of the row before
    // B), so B alone does not place every lane.
    uint32_t colb = 2u * (i0 - static_cast<uint32_t>(__umul64hi(i0, m.row_magic)) * m.in_features);
    const uint32_t wrapb = 2u * kRound - 2u * m.in_features;  // modulo 2^32
    // The lane's column one round on: 512 further, less a row when that
    // passes the row's end.
    auto next_col = [wrapb](uint32_t c) { return min(c + 2u * kRound, c + wrapb); };
    uint4 xr[kAll ? kPrefetchChunks : 1][TB];
    if constexpr (kAll) {
        uint32_t c = colb;
#pragma unroll
        for (int j = 0; j < kPrefetchChunks; ++j) {
            load_x<TB>(m, c, xr[j]);
            c = next_col(c);
        }
    } else if constexpr (kAhead) {
        load_x<TB>(m, colb, xv);
    }

    // One round, with xc this round's x columns.
    auto step = [&](uint64_t s8, const uint4 (&xc)[TB]) {
        const bool in_chunks = i0 < chunk_end;
        uint64_t r8 = 0;
        if (in_chunks) {
            r8 = *reinterpret_cast<uint64_t *>(cell);
            *reinterpret_cast<uint64_t *>(cell) = 0;
        }
        // Does this round reach the next row?  (B only moves forward and
        // stays past e0.)
        const bool cross = B < hi_eff && B - e0 < kRound;
        // Chunks past the group's last one merge as zero.
        const uint4 v = merge8(in_chunks ? s8 : 0ull, r8);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
        // Only the rounds that hold the group's first or last output can be
        // cut by lo or hi (e0 < run_end <= hi).
        if (e0 < lo || hi - e0 < kRound) {
            if (i0 < lo || i0 + 8u > hi) {
#pragma unroll
                for (uint32_t e = 0; e < 8; ++e)
                    if (i0 + e < lo || i0 + e >= hi) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
            }
        }
        if (!cross) {
#pragma unroll
            for (int t = 0; t < TB; ++t)
                rs.acc[t] = dot2_bf16(w[3], xc[t].w,
                                      dot2_bf16(w[2], xc[t].z,
                                                dot2_bf16(w[1], xc[t].y, dot2_bf16(w[0], xc[t].x, rs.acc[t]))));
        } else {
            // Finish the current row with the lanes before B, carry on with the rest.
            float p[TB];
#pragma unroll
            for (int t = 0; t < TB; ++t)
                p[t] = dot2_bf16(w[3], xc[t].w,
                                 dot2_bf16(w[2], xc[t].z, dot2_bf16(w[1], xc[t].y, dot2_bf16(w[0], xc[t].x, 0.0f))));
            const bool in_b = i0 >= B;
#pragma unroll
            for (int t = 0; t < TB; ++t) rs.acc[t] += in_b ? 0.0f : p[t];
            flush_wave<TB>(m, rs, row0, yacc);
#pragma unroll
            for (int t = 0; t < TB; ++t) rs.acc[t] = in_b ? p[t] : 0.0f;
            rs.row += 1u;
            rs.dirty = true;
            B += m.in_features;
        }
        colb = next_col(colb);
        e0 += kRound;
        i0 += kRound;
        cell += kRound;
    };
#pragma unroll
    for (int j = 0; j < kPrefetchChunks; ++j) {
        if (e0 >= run_end) break;
        if constexpr (kAll) {
            step(sm[j], xr[j]);
        } else if constexpr (kAhead) {
            load_x<TB>(m, next_col(colb), xn);
            step(sm[j], xv);
#pragma unroll
            for (int t = 0; t < TB; ++t) xv[t] = xn[t];
        } else {
            load_x<TB>(m, colb, xv);
            step(sm[j], xv);
        }
    }
    // Rounds past the prefetched ones (groups of more than 1024 chunks).
    while (e0 < run_end) {
        load_x<TB>(m, colb, xv);
        step(*reinterpret_cast<const uint64_t *>(a.sm + 8ull * min(i0 >> 3, a.sm_chunks - 1u)), xv);
    }
    flush_wave<TB>(m, rs, row0, yacc);
}

// Add a group's LDS row sums into y (other workgroups add the other parts
// of rows that cross groups) and zero them for the next group.  Called by
// the group's threads after a barrier that follows merge_matmul.
template <int TB>
__device__ __forceinline__ void flush_rows(const MatmulArgs &m, float *yacc, uint32_t row0, uint32_t rows,
                                           uint32_t ltid) {
    for (uint32_t i = ltid; i < rows * TB; i += kThreadsPerGroup) {
        const float v = yacc[i];
        yacc[i] = 0.0f;
        const uint32_t t = i % TB;
        if (t < m.n_tokens) unsafeAtomicAdd(m.y + static_cast<size_t>(t) * m.out_features + row0 + i / TB, v);
    }
}

// The matrix-core product (y = x W^T, W stored in MFMA tile order; see
// tiled_chunk_origin).  A group's chunks are taken in rounds of 256 aligned
// to the blocks: round j holds the chunks 256 (c0 / 256 + j) .. + 255, one
// per thread, so that wave w, lane l holds lane l of n-tile w of one global
// k-step, exactly the B operand of a v_mfma_f32_16x16x32_bf16 for the 16
// rows of that n-tile; chunks outside the group, and elements of its edge
// chunks outside [base, end), merge as zero (the neighbouring group adds
// them).  Each wave keeps the running 16 x 16 sums of its n-tile for MT
// tiles of 16 tokens of the current pass, and adds them into y when its
// panel or pass changes, or at the end (float atomics: the groups of a panel
// lie in several workgroups).  x must hold finite values.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <int MT>
struct PanelSums {
    floatx4 d[MT];   // lane l, entry r: token 16 mt + 4 (l / 16) + r, row 16 wave + (l mod 16)
    uint32_t panel;  // 64-row panel of the sums (wave-uniform), ~0 when empty
    uint32_t pass;   // pass of the sums (wave-uniform)
};

template <int MT>
__device__ __forceinline__ void flush_panel(const MatmulArgs &m, PanelSums<MT> &ps, uint32_t wave, uint32_t lane) {
    if (ps.panel == ~0u) return;
    const uint32_t row = 64u * ps.panel + 16u * wave + (lane & 15u);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t t = (ps.pass * MT + mt) * 16u + 4u * (lane >> 4) + r;
            if (t < m.n_tokens) unsafeAtomicAdd(m.y + static_cast<size_t>(t) * m.out_features + row, ps.d[mt][r]);
            ps.d[mt][r] = 0.0f;
        }
    }
    ps.panel = ~0u;
}

// x operands of one round: token tiles mt of the pass, the 8 columns of the
// lane at global k-step g (tokens past n_tokens read as zero).
template <int MT>
__device__ __forceinline__ void load_xa(const DecodeArgs &a, const MatmulArgs &m, uint32_t g, uint32_t pass,
                                        uint32_t lane, uint4 (&xa)[MT]) {
    const uint32_t panel = static_cast<uint32_t>(__umul64hi(g, a.tile_magic));
    const uint32_t col = 32u * (g - panel * a.tile_ks) + 8u * (lane >> 4);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const uint32_t t = (pass * MT + mt) * 16u + (lane & 15u);
        const uint4 v = *reinterpret_cast<const uint4 *>(m.x + static_cast<size_t>(min(t, m.n_tokens - 1u)) *
                                                                   m.in_features + col);
        xa[mt] = t < m.n_tokens ? v : make_uint4(0, 0, 0, 0);
    }
}

// The x operands of a group's first kXTiles rounds are staged in LDS for
// the merge (one copy per group slot, read by its four waves, which would
// otherwise each load the same tiles): a 1 KB tile per (round, token tile),
// lane l's 16 bytes at 16 l.  The four waves load them straight from
// global memory into LDS (global_load_lds_dwordx4, no registers), each a
// quarter of the tiles, right after the scan barrier of the iteration that
// decodes the group: every wave has finished the previous merge's reads by
// then, so one buffer per slot suffices; the loads land during phase 2 and
// are waited for before the iteration's last barrier.  Rounds past
// kXTiles (groups of more than about 1000 chunks) load theirs in the round.
template <int MT>
constexpr int kXTiles = MT <= 2 ? 4 : 2;

template <int MT>
__device__ __forceinline__ void stage_x(const DecodeArgs &a, const MatmulArgs &m, uint32_t base, uint32_t pass,
                                        uint32_t wave, uint32_t lane, uint8_t *s_x) {
    // (global_load_lds writes lane l's 16 bytes at the wave-uniform LDS
    // address + 16 l)
    const uint32_t g0 = base >> 11;
    wave = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int q = 0; q < kXTiles<MT> * MT; q += 4) {
        const uint32_t tile = q + wave;  // (round tile / MT, token tile tile % MT)
        if (tile < static_cast<uint32_t>(kXTiles<MT> * MT)) {
            const uint32_t g = g0 + tile / MT, mt = tile % MT;
            const uint32_t panel = static_cast<uint32_t>(__umul64hi(g, a.tile_magic));
            const uint32_t col = 32u * (g - panel * a.tile_ks) + 8u * (lane >> 4);
            const uint32_t t = min((pass * MT + mt) * 16u + (lane & 15u), m.n_tokens - 1u);
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void *)(m.x + static_cast<size_t>(t) * m.in_features + col),
                (__attribute__((address_space(3))) void *)(s_x + 1024u * tile), 16, 0, 0);
        }
    }
}

template <int MT>
__device__ __forceinline__ void merge_mfma(const DecodeArgs &a, const MatmulArgs &m, uint8_t *ebuf,
                                           const uint64_t (&sm)[kPrefetchChunks], uint32_t base, uint32_t end,
                                           uint32_t pass, uint32_t ltid, PanelSums<MT> &ps, const uint8_t *s_x) {
    const uint32_t c0 = base >> 3;
    const uint32_t n_chunks = min(group_chunks(base, end), a.ebuf_cap / 8u);
    const uint32_t lead = c0 & 255u;
    const uint32_t rounds = (lead + n_chunks + 255u) >> 8;
    uint32_t lane = ltid & (kWaveSize - 1);
    // Two token tiles: the lane constants are recomputed at every merge (hoisted
    // out of the decoder's loop they held registers through the decode, and
    // the kernel spilled; 32 tokens 0.167 -> 0.155 ms per block).  At one and
    // four tiles the hoisted form measured faster.
    if constexpr (MT == 2) asm volatile("" : "+v"(lane));
    const uint32_t wave = __builtin_amdgcn_readfirstlane(ltid / kWaveSize);
    if (ltid == 0 && 8u * (n_chunks + 1u) <= a.ebuf_cap) *reinterpret_cast<uint64_t *>(ebuf + 8u * n_chunks) = 0;
    if (n_chunks == 0) return;
    const uint32_t g0 = c0 >> 8;
    auto round = [&](uint32_t j, const uint4 (&xa)[MT], uint64_t s8) {
        const uint32_t kk = ltid + 256u * j;
        const uint32_t k = kk - lead;
        const bool in = kk >= lead && k < n_chunks;
        uint64_t r8 = 0;
        if (in) {
            uint64_t *cell = reinterpret_cast<uint64_t *>(ebuf + 8u * k);
            r8 = *cell;
            *cell = 0;
        }
        const uint4 v = merge8(in ? s8 : 0ull, r8);
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
        const uint32_t e0 = 8u * (c0 + k);
        if (!in) {
            w[0] = w[1] = w[2] = w[3] = 0u;
        } else if (e0 < base || e0 + 8u > end) {
#pragma unroll
            for (uint32_t e = 0; e < 8; ++e)
                if (e0 + e < base || e0 + e >= end) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
        }
        const uint32_t g = g0 + j;
        const uint32_t panel = static_cast<uint32_t>(__umul64hi(g, a.tile_magic));
        if (panel != ps.panel || pass != ps.pass) {
            flush_panel<MT>(m, ps, wave, lane);
            ps.panel = panel;
            ps.pass = pass;
        }
        const bf16x8 b = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            ps.d[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[mt]), b, ps.d[mt], 0, 0, 0);
    };
    // (sm holds the chunks of rounds 0 .. kPrefetchChunks - 1, load_sm)
    static_assert(kXTiles<MT> <= kPrefetchChunks, "staged rounds must have their sign/mantissa chunks");
#pragma unroll
    for (int j = 0; j < kXTiles<MT>; ++j) {
        if (static_cast<uint32_t>(j) < rounds) {
            uint4 xa[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                // (tokens past n_tokens were staged from the last token: zero them)
                const uint4 v = *reinterpret_cast<const uint4 *>(s_x + 1024u * (j * MT + mt) + 16u * lane);
                xa[mt] = (pass * MT + mt) * 16u + (lane & 15u) < m.n_tokens ? v : make_uint4(0, 0, 0, 0);
            }
            round(j, xa, sm[j]);
        }
    }
    for (uint32_t j = kXTiles<MT>; j < rounds; ++j) {
        uint4 xa[MT];
        load_xa<MT>(a, m, g0 + j, pass, lane, xa);
        uint64_t s8 = 0;
        const uint32_t kk = ltid + 256u * j;
        if (j < static_cast<uint32_t>(kPrefetchChunks)) {
#pragma unroll
            for (int q = 0; q < kPrefetchChunks; ++q)
                if (j == static_cast<uint32_t>(q)) s8 = sm[q];
        } else if (kk >= lead && kk - lead < n_chunks) {
            s8 = __builtin_nontemporal_load(reinterpret_cast<const uint64_t *>(a.sm + 8ull * (c0 + kk - lead)));
        }
        round(j, xa, s8);
    }
}

// Group edges.  When a group's first element is not a multiple of 8, the
// group shares an 8-element output chunk with the previous group; stored
// separately, each half of it would be a partial write of one cache line from
// each of two workgroups.  Instead the previous group's workgroup writes the
// whole chunk, decoding the c codes that open the group (c = elements of the
// group in that chunk), when they can be decoded from the first 64 bits of the
// group's first segment: the c-th code ends at or before bit 64 - K (so every
// K-bit window used lies in those bits) and none of them is longer than K
// bits.  The previous group's last thread holds those 64 bits as its third and
// fourth words and the group's first thread as its first two; both evaluate
// the rule from the stream alone, so they agree without communicating.
//
// boundary_codes walks from bit q of the pair, a code start preceded by `cum`
// of the c codes, and returns whether the rule holds; with write set it also
// ORs each lookup's exponents at the LDS accumulator acc2.
template <int K>
__device__ __forceinline__ bool boundary_codes(uint64_t pair, uint32_t q, uint32_t cum, uint32_t c, uint32_t acc2,
                                               bool write, const uint32_t *s_lo, const uint32_t *s_aux,
                                               const uint16_t *s_start) {
    constexpr uint32_t kLastEnd = 64u - K;
    while (cum < c) {
        if (q > kLastEnd) return false;
        const uint32_t off = entry_offset<K>(pair, q);
        const uint32_t x = lds_at<uint32_t>(s_aux, off);
        if (x == kLongCode) return false;
        const uint32_t m = (x >> 11) & 7u;
        if (write) or_exponents(acc2, (static_cast<uint64_t>(x >> 16) << 32) | lds_at<uint32_t>(s_lo, off));
        if (cum + m >= c) {
            // End of the c-th code: the next listed code's start, or the end
            // of the listed run.
            const uint32_t j = c - cum;
            uint32_t code_end = q + (x & 0xFFu);
            if (j < m) {
                uint32_t starts = lds_at<uint16_t>(s_start, off >> 2);
                for (uint32_t i = 0; i < j; ++i) starts &= starts - 1u;
                code_end = q + __builtin_ctz(starts);
            }
            return code_end <= kLastEnd;
        }
        acc2 += m << 11;
        cum += m;
        q += x & 0xFFu;
    }
    return true;
}

// Dynamic schedule.  Workgroups run at different speeds (a CU favours its
// oldest waves), so after two static rounds (super-groups wg, wg + grid)
// each workgroup takes its next super-groups from one of P <= 8 pools: pool
// x hands out 2 grid + x + P v for v = 0, 1, ... from its own counter, so
// that the ticket fetches of the whole grid are spread over P addresses (one
// address would serialise them).  Thread 0 fetches a ticket at the top of
// every iteration and, after that iteration's scan barrier, hands it to the
// other waves through LDS; the next iteration issues its loads and the one
// after decodes it.  A workgroup thus commits to a super-group two
// iterations before it decodes it (three measured 1-2% slower on the block:
// at the end the workgroups finish further apart).  A workgroup's tickets
// increase, so it stops at its first ticket past the end having processed
// every earlier one.  On exit every workgroup counts itself in the done word;
// the last one zeroes every word for the next launch.  A pool's share of the
// work is fixed, so P divides the workgroup count (schedule_pools).
using df11::kPools;
constexpr uint32_t kPoolStride = DF11_SCHEDULE_WORDS / (kPools + 1);  // words: one cache line per counter

// The pool of workgroup wg.  Workgroup i runs on XCD i mod 8, so pools
// wg mod P would each sit on one XCD (for P = 8) and a slower XCD would end
// last with its fixed share; (wg + wg / 8) mod P gives every pool the same
// number of workgroups of every XCD when P divides 8 (and P divides the
// workgroup count, so each pool gets the same number).
__device__ __forceinline__ uint32_t pool_of(uint32_t wg, uint32_t pools) {
    return (wg + (8u % pools == 0u ? wg / 8u : 0u)) % pools;
}

__device__ __forceinline__ uint32_t take_ticket(uint32_t *sched, uint32_t pool) {
    return __hip_atomic_fetch_add(sched + pool * kPoolStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void finish_schedule(uint32_t *sched, uint32_t n_wg) {
    if (!sched || threadIdx.x != 0) return;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's ticket fetches are complete
    uint32_t *done_word = sched + kPools * kPoolStride;
    const uint32_t done = __hip_atomic_fetch_add(done_word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == n_wg - 1u) {
        for (uint32_t x = 0; x < kPools; ++x)
            __hip_atomic_store(sched + x * kPoolStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(done_word, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Phase 1 over one half of a segment: table lookups from bit p = acc & 0xFF
// of the 64-bit pair while p < end, advancing acc by each increment (inc keeps
// the last one).  The entries of the first kSavedSteps lookups go to
// slo/saux[first ..] (zero for lookups after the lane's last), with a window
// whose first code is too long replaced by that code alone (rotated exponent,
// increment (1 << 11) + length).  Further lookups are counted only, and set
// spill.
template <int K>
__device__ __forceinline__ void count_half(uint64_t pair, uint32_t end, uint32_t &acc, uint32_t &inc,
                                           uint32_t (&slo)[2 * kSavedSteps], uint32_t (&saux)[2 * kSavedSteps],
                                           int first, bool &spill, const uint32_t *s_lo, const uint32_t *s_aux,
                                           const uint8_t *s_luts, const uint8_t *s_clen, uint32_t n_luts) {
#pragma unroll
    for (int j = 0; j < kSavedSteps; ++j) {
        const uint32_t off = entry_offset<K>(pair, acc);
        uint32_t l = lds_at<uint32_t>(s_lo, off);
        uint32_t x = lds_at<uint32_t>(s_aux, off);
        const bool act = (acc & 0xFFu) < end;
        if (act && x == kLongCode) {
            const uint32_t win = static_cast<uint32_t>((pair << (acc & 63u)) >> 32);
            uint32_t len;
            l = df11::rotate_exponent(walk_luts(win, s_luts[win >> 24], s_luts, s_clen, n_luts, len));
            x = (1u << 11) + len;
        }
        slo[first + j] = act ? l : 0u;
        saux[first + j] = act ? x : 0u;
        inc = act ? (x & 0xFFFFu) : inc;
        acc += act ? (x & 0xFFFFu) : 0u;
    }
    if ((acc & 0xFFu) < end) {
        spill = true;
        for (;;) {
            while ((acc & 0xFFu) < end) {
                inc = lds_at<uint16_t>(s_aux, entry_offset<K>(pair, acc));
                acc += inc;
            }
            if (!(acc & kLongCode)) break;
            acc -= kLongCode;
            const uint32_t win = static_cast<uint32_t>((pair << (acc & 63u)) >> 32);
            uint32_t len;
            walk_luts(win, s_luts[win >> 24], s_luts, s_clen, n_luts, len);
            inc = (1u << 11) + len;
            acc += inc;
        }
    }
}

// Phase 2 over one half without kept entries: the same lookups as phase 1,
// each ORing its exponent run at the LDS address in acc2.
template <int K>
__device__ __forceinline__ void decode_half(uint64_t pair, uint32_t end, uint32_t &acc2, const uint32_t *s_lo,
                                            const uint32_t *s_aux, const uint8_t *s_luts, const uint8_t *s_clen,
                                            uint32_t n_luts) {
    for (;;) {
        while ((acc2 & 0xFFu) < end) {
            // lo and aux are one paired LDS read.
            const uint32_t off = entry_offset<K>(pair, acc2);
            const uint32_t w = lds_at<uint32_t>(s_aux, off);
            const uint32_t at = acc2;
            acc2 += w & 0xFFFFu;
            or_exponents(at, (static_cast<uint64_t>(w >> 16) << 32) | lds_at<uint32_t>(s_lo, off));
        }
        if (!(acc2 & kLongCode)) break;
        acc2 -= kLongCode;
        const uint32_t win = static_cast<uint32_t>((pair << (acc2 & 63u)) >> 32);
        uint32_t len;
        or_exponents(acc2, df11::rotate_exponent(walk_luts(win, s_luts[win >> 24], s_luts, s_clen, n_luts, len)));
        acc2 += (1u << 11) + len;
    }
}

// GPW groups of 256 threads share one workgroup (and one copy of the decode
// tables in LDS).  Super-groups (GPW consecutive groups) are dealt to the
// workgroups round-robin, so at any moment the whole grid reads and writes
// one compact window of each buffer rather than one region per workgroup,
// which HBM serves markedly faster.  (Neighbouring super-groups thus run on
// different XCDs, since workgroup i goes to XCD i mod 8; grouping them per
// XCD instead measured slower, as it splits the window into eight.)
// Iteration i first issues the loads of the super-group of iteration i + 1,
// then merges and stores the super-group decoded in iteration i - 1 (reading
// and re-zeroing its LDS exponent buffer) and loads its own sign/mantissa
// chunks for that merge in the next iteration, then decodes its own: phase 1,
// the scan (whose barrier also orders the merge's reads before this
// iteration's phase-2 writes, so one buffer per group suffices), phase 2 and a
// barrier.  Every wait for loaded data therefore comes a whole decode phase
// after the last stores were issued.  One buffer per group (rather than two)
// keeps the LDS of a 512-thread workgroup small enough for four per CU.
//
// TB > 0 turns the merge into the fused matmul with up to TB tokens
// (merge_matmul and flush_rows in place of merge_group).
//
// kTail (matrix-core product, one pass): workgroup wg first sweeps the fixed
// range [wg L, (wg + 1) L) of L = m.fixed_len super-groups, then takes the
// rest, [n_wg L, n_super), one super-group per ticket from the work
// counters, as the decoder does.
// kPairs (decompression of a tile-ordered stream with an even number of
// k-steps per panel): the merge writes whole row-major lines
// (merge_group_pairs) through a per-wave LDS stage after the dynamic LDS.
template <int K, int GPW, int TB, bool kTail = false, bool kPairs = false>
__device__ __forceinline__ void decode_stream(const DecodeArgs &a, const MatmulArgs &m, const uint32_t wg,
                                              const uint32_t n_wg) {
    // Static LDS: the first-level table (2^K (lo, aux) word pairs, then 2^K
    // start masks) at a fixed address, so a lookup's address is its index
    // times 8.  A pair is one 64-bit LDS read; lo and aux 8 KB apart (the
    // same bank for every lane) made random lookups take 1.8x as long.
    // Dynamic LDS: LUTs | CodeLengths | GPW exponent buffers | wave sums |
    // edge flags | ticket | (fused matmul) GPW row-sum arrays.
    __shared__ __align__(16) uint32_t s_tab[(10u << K) / 4u];
    extern __shared__ __align__(16) uint8_t smem[];
    const uint32_t *s_lo = s_tab;      // word 0 of each pair
    const uint32_t *s_aux = s_tab + 1;  // word 1
    const uint16_t *s_start = reinterpret_cast<const uint16_t *>(s_tab + (2u << K));
    uint8_t *s_luts = smem;
    uint8_t *s_clen = s_luts + a.n_luts * 256u;
    const uint32_t tid = threadIdx.x;
    const uint32_t slot = __builtin_amdgcn_readfirstlane(tid / kThreadsPerGroup);
    const uint32_t ltid = tid % kThreadsPerGroup;
    const uint32_t lane = tid & (kWaveSize - 1);
    const uint32_t wave = ltid / kWaveSize;
    uint8_t *s_ebuf = s_clen + 256u + slot * a.ebuf_cap;
    uint32_t *s_wsum = reinterpret_cast<uint32_t *>(s_clen + 256u + GPW * a.ebuf_cap) + slot * kWaves;
    // Per group: [0] the previous group wrote the shared first chunk, [1] this
    // group's last chunk is written whole (see boundary_codes).
    uint32_t *s_edge = reinterpret_cast<uint32_t *>(s_clen + 256u + GPW * a.ebuf_cap) + GPW * kWaves + slot * 2u;
    // The next super-group of the dynamic schedule, from thread 0.
    uint32_t *s_ticket = reinterpret_cast<uint32_t *>(s_clen + 256u + GPW * a.ebuf_cap) + GPW * (kWaves + 2u);
    // The fused matmul's row sums (yacc_rows x TB floats per group; none
    // for the matrix-core product, TB < 0, whose sums stay in registers).
    constexpr uint32_t kRowTB = TB > 0 ? TB : 0;
    float *s_yacc = reinterpret_cast<float *>(s_ticket + 4) + slot * m.yacc_rows * kRowTB;
    // Only for a stream without a decode table: the first code of each
    // window, while the table is derived (2^K uint16).
    constexpr uint32_t kXBytes = TB < 0 ? GPW * kXTiles<(TB < 0 ? -TB : 1)> * (TB < 0 ? -TB : 1) * 1024u : 0u;
    uint16_t *s_first = reinterpret_cast<uint16_t *>(reinterpret_cast<uint8_t *>(
                                                         reinterpret_cast<float *>(s_ticket + 4) + GPW * m.yacc_rows * kRowTB) +
                                                     kXBytes);
    uint32_t y_row0 = 0, y_rows = 0;  // rows of the merged group awaiting flush_rows
    static_assert(!kPairs || TB == 0, "whole-line stores only when decompressing");
    uint4 *s_pair = reinterpret_cast<uint4 *>(reinterpret_cast<uint8_t *>(s_first) + (a.dtab ? 0u : 2u << K) +
                                              (slot * kWaves + wave) * kPairStageBytes);

    const uint32_t n_super = (a.n_groups + GPW - 1) / GPW;
    uint32_t *const sched = a.sched;
    if (wg >= n_super) {  // whole workgroup
        finish_schedule(sched, n_wg);
        return;
    }
    // The matrix-core product (TB < 0, MT = -TB tiles of 16 tokens) gives
    // each workgroup a contiguous range of super-groups [r0, r0 + len),
    // swept m.passes times (16 MT tokens each), so that consecutive groups
    // of a workgroup mostly share a panel and its sums stay in registers
    // (dealing the super-groups out round-robin, with a flush of the sums
    // after every group, took twice as long at 16 tokens).  Its iterations
    // are numbered v = pass * len + (super-group - r0).
    constexpr bool kMfma = TB < 0;
    constexpr int MT = kMfma ? -TB : 1;
    static_assert(!kTail || TB == -1, "a dealt tail only for the one-tile matrix-core product");
    const uint32_t r0 = kTail   ? wg * m.fixed_len
                        : kMfma ? static_cast<uint32_t>(static_cast<uint64_t>(wg) * n_super / n_wg)
                                : 0u;
    const uint32_t len = kTail   ? m.fixed_len
                         : kMfma ? static_cast<uint32_t>(static_cast<uint64_t>(wg + 1) * n_super / n_wg) - r0
                                 : 1u;
    // (with kTail, iterations are numbered by super-group, as the decoder's)
    const uint32_t v_end = kMfma && !kTail ? len * m.passes : n_super;
    // Super-group of iteration v (n_super past the end).
    auto super_of = [&](uint32_t v) -> uint32_t {
        return kMfma && !kTail ? (v < v_end ? r0 + v % len : n_super) : v;
    };
    PanelSums<MT> ps;
    // matrix-core product: the next merge's staged x tiles (stage_x)
    uint8_t *s_x = reinterpret_cast<uint8_t *>(s_ticket + 4) + slot * kXTiles<MT> * MT * 1024u * (kMfma ? 1u : 0u);
    if constexpr (kMfma) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) ps.d[mt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
        ps.panel = ~0u;
        ps.pass = 0;
    }
    uint32_t prev_pass = 0;

    // Pipeline state: the group's output range (scalar) and thread inputs one
    // super-group ahead; the sign/mantissa chunks of the group waiting to be
    // merged.
    const uint32_t s_first_it = kTail ? r0 : kMfma ? 0u : wg;
    const uint32_t g_first = super_of(s_first_it) * GPW + slot;
    uint32_t cur_base = out_pos_at(a, g_first), cur_end = out_pos_at(a, g_first + 1);
    GroupLoad cur = load_group(a, g_first, ltid);
    uint64_t sm[kPrefetchChunks] = {};  // the previous group's, until the merge, then this group's
    uint32_t prev_base = 0, prev_end = 0;

    // Stage the first-level table, the LUT hierarchy and CodeLengths.  Every
    // load is issued before any of them is written to LDS, so staging costs
    // one memory round trip rather than one per loop pass (the whole grid
    // waits for it at the start of every launch).
    {
        constexpr uint32_t kThreads = kThreadsPerGroup * GPW;
        constexpr uint32_t kTabVecs = (10u << K) / 16u;
        constexpr uint32_t kTabPer = (kTabVecs + kThreads - 1) / kThreads;
        constexpr uint32_t kLutPer = (DF11_MAX_LUTS * 64u + kThreads - 1) / kThreads;
        // Without a table (derived below) every lane loads the first 16
        // bytes of EncodedExponent instead and stores them anywhere in the
        // table's place: the loads and stores stay unconditional.
        const bool have_tab = a.dtab != nullptr;
        const uint4 *src = reinterpret_cast<const uint4 *>(have_tab ? static_cast<const void *>(a.dtab)
                                                                    : static_cast<const void *>(a.enc));
        const uint32_t tab_last = have_tab ? kTabVecs - 1u : 0u;
        const uint32_t *l32 = reinterpret_cast<const uint32_t *>(a.luts);
        const uint32_t lut_words = a.n_luts * 64u;
        uint4 tv[kTabPer];
        uint32_t lv[kLutPer];
#pragma unroll
        for (uint32_t j = 0; j < kTabPer; ++j) tv[j] = src[min(tid + j * kThreads, tab_last)];
#pragma unroll
        for (uint32_t j = 0; j < kLutPer; ++j) lv[j] = l32[min(tid + j * kThreads, lut_words - 1u)];
        const uint32_t cv = reinterpret_cast<const uint32_t *>(a.code_lengths)[tid & 63u];
        // Phase 2 ORs exponents into the buffers, so they start out zero (and
        // the merge zeroes every chunk it consumes).
        uint4 *z = reinterpret_cast<uint4 *>(s_clen + 256u);
        for (uint32_t i = tid; i < GPW * a.ebuf_cap / 16u; i += kThreads) z[i] = make_uint4(0, 0, 0, 0);
        if constexpr (TB > 0) {
            float *y0 = reinterpret_cast<float *>(s_ticket + 4);
            for (uint32_t i = tid; i < GPW * m.yacc_rows * TB; i += kThreads) y0[i] = 0.0f;
        }
        // Unconditional stores (indices clamped like the loads: extra lanes
        // write the last element's value to it again), so the compiler cannot
        // sink each load into a branch next to its store.
        uint4 *dst = reinterpret_cast<uint4 *>(s_tab);
#pragma unroll
        for (uint32_t j = 0; j < kTabPer; ++j) dst[min(tid + j * kThreads, kTabVecs - 1u)] = tv[j];
        uint32_t *d32 = reinterpret_cast<uint32_t *>(s_luts);
#pragma unroll
        for (uint32_t j = 0; j < kLutPer; ++j) d32[min(tid + j * kThreads, lut_words - 1u)] = lv[j];
        reinterpret_cast<uint32_t *>(s_clen)[tid & 63u] = cv;
    }
    __syncthreads();
    if (!a.dtab) {  // a stream without a decode table: derive it from the LUTs and CodeLengths
        derive_table<K, kThreadsPerGroup * GPW>(s_tab, s_first, s_luts, s_clen, a.n_luts, tid);
        __syncthreads();
    }

    uint32_t s_cur = s_first_it;
    for (uint32_t it = 0; s_cur < v_end; ++it) {
        // Wave priorities by phase (the SIMD issues the higher one first
        // among ready waves): the next loads 2, the merge and its stores 0,
        // phase 1's chain of dependent lookups 3, phase 2 1.  A wave that
        // starts decoding runs its chain with fewer gaps while the waves in
        // their merge keep the memory busy.
        __builtin_amdgcn_s_setprio(2);
        const uint32_t g = super_of(s_cur) * GPW + slot;
        // Rounds 0 and 1 are static; the ticket for round it + 1 >= 2 was
        // fetched and written to LDS in iteration it - 1.
        // (kTail: the fixed range, then the tickets, the first fetched two
        // iterations before the range ends)
        const uint32_t s_nx = kTail                  ? (it + 1u < len ? s_cur + 1u
                                                                      : __builtin_amdgcn_readfirstlane(*s_ticket))
                              : kMfma                ? s_cur + 1u
                              : (sched && it >= 1u) ? __builtin_amdgcn_readfirstlane(*s_ticket)
                                                    : min(s_cur + n_wg, n_super);

        // 1. Loads of the next super-group's thread inputs and output range
        // (group numbers past the end are clamped inside the loads and never
        // decoded), issued first so that they are in flight longest.  The
        // output range is clamped so that a corrupt out_pos stays in bounds.
        const uint32_t end = min(cur_end, a.n_elements);
        const uint32_t base = min(cur_base, end);
        const uint32_t g_nx = min(super_of(s_nx) * GPW + slot, a.n_groups);
        const uint32_t nx_base = out_pos_at(a, g_nx), nx_end = out_pos_at(a, g_nx + 1);
        if constexpr (TB > 0) {
            // The fused merge waits for its own loads of x; issued before
            // the next group's loads, those waits do not include them.
            if (it > 0)
                merge_matmul<TB>(a, m, s_ebuf, sm, prev_base, prev_end, ltid, s_edge[0] != 0, s_edge[1] != 0, s_yacc,
                                 y_row0, y_rows);
        } else if constexpr (kMfma) {
            if (it > 0) merge_mfma<MT>(a, m, s_ebuf, sm, prev_base, prev_end, prev_pass, ltid, ps, s_x);
        }
        const GroupLoad nx = load_group(a, g_nx, ltid);
        uint32_t fetched = 0;
        if (sched && tid == 0 && (!kTail || it + 2u >= len))
            fetched = take_ticket(sched, pool_of(wg, a.pools));  // for round it + 2
        // (the whole-line merge, with its stage round trips, at the loads' priority:
        // per-weight block 162.4 -> 159.2 us hot; at 1 or 3, 163.4 and 160.6)
        __builtin_amdgcn_s_setprio(kPairs ? 2 : 0);

        // 2. Merge and store the super-group decoded in the previous
        // iteration (the fused matmul merged it before step 1's loads), then
        // load this group's sign/mantissa chunks (into the registers the
        // merge has just consumed) for the next one.
        if constexpr (TB == 0) {
            if constexpr (kPairs) {
                if (it > 0)
                    merge_group_pairs(a, s_ebuf, sm, prev_base, prev_end, ltid, s_edge[0] != 0, s_edge[1] != 0, s_pair);
            } else {
                if (it > 0) merge_group(a, s_ebuf, sm, prev_base, prev_end, ltid, s_edge[0] != 0, s_edge[1] != 0);
            }
        }
        load_sm<TB, kPairs>(a, base, end, ltid, sm);
        __builtin_amdgcn_s_setprio(3);

        // 3. Decode this super-group.
        const uint32_t lead = base & 7u;

        const uint32_t t = g * kThreadsPerGroup + ltid;
        uint32_t gap = 0, seg_end = 0;
        if (g < a.n_groups && t < a.n_threads) {
            const uint64_t gbit = 5ull * t;
            const uint64_t gw = (static_cast<uint64_t>(bswap32(cur.g0)) << 32) | bswap32(cur.g1);
            gap = static_cast<uint32_t>((gw << (gbit & 31)) >> 59);
            seg_end = t + 1 < a.n_threads ? kSegBits : a.last_seg_bits;
        }
        const uint32_t w0 = bswap32(cur.e0), w1 = bswap32(cur.e1), w2 = bswap32(cur.e2), w3 = bswap32(cur.e3);
        // Lookups that start in bits [0, 32) of the segment read the pair w0 w1
        // and those that start later read w1 w2, each with one 64-bit shift by
        // the start bit: a code read from bit p < 32 plus the K-bit window ends
        // before bit 64 of its pair.  Positions are kept in accumulators
        // (x << 11) | p; a table increment (m << 11) + nb adds m to x and nb to p.
        const uint64_t pa = (static_cast<uint64_t>(w0) << 32) | w1;
        const uint64_t pb = (static_cast<uint64_t>(w1) << 32) | w2;
        const uint32_t end_a = min(seg_end, 32u);
        const uint32_t end_b = seg_end > 32u ? seg_end - 32u : 0u;

        // Phase 1: walk the codes that start in [gap, seg_end) and count them.
        // The first kSavedSteps lookups of each half keep their table entries
        // (exponent run and increment) in registers, so that phase 2 only has
        // to OR them into place; a lookup whose window starts with a code
        // longer than K bits is finished through the LUT hierarchy and kept in
        // the same form.  A lane with more lookups in a half finishes counting
        // in a loop, and its wave then decodes phase 2 again from the stream.
        uint32_t slo[2 * kSavedSteps], saux[2 * kSavedSteps];
        uint32_t acc = gap, inc = 0;
        bool spill = false;
        count_half<K>(pa, end_a, acc, inc, slo, saux, 0, spill, s_lo, s_aux, s_luts, s_clen, a.n_luts);
        uint32_t shift_back = 0;
        if (end_b) {
            acc -= 32u;
            shift_back = 32u;
        }
        count_half<K>(pb, end_b, acc, inc, slo, saux, kSavedSteps, spill, s_lo, s_aux, s_luts, s_clen, a.n_luts);
        uint32_t cnt = acc >> 11, past = 0;
        if (cnt) {
            // The last lookup, at p_last, may list codes that start at or
            // after seg_end; its start mask says how many.
            const uint32_t p_last = (acc + shift_back - inc) & 0xFFu;
            const uint32_t mask = s_start[window_at(pa, pb, p_last) >> (32 - K)];
            past = __popc(mask >> min(seg_end - p_last, 31u));
            cnt -= past;
        }

        // Offsets within the group.
        const uint32_t incl = wave_inclusive_scan(cnt);
        if (lane == kWaveSize - 1) s_wsum[wave] = incl;
        __syncthreads();
        if constexpr (TB > 0) {
            // The barrier completed the merge's LDS sums; the one at the end
            // of the iteration orders the zeroing before the next merge.
            flush_rows<TB>(m, s_yacc, y_row0, y_rows, ltid);
            y_rows = 0;
        } else if constexpr (kMfma) {
            // Every wave's merge has read the staged tiles: stage this group's.
            stage_x<MT>(a, m, base, kTail ? 0u : s_cur / len, wave, lane, s_x);
        }
        __builtin_amdgcn_s_setprio(1);
        uint32_t wave_off = 0;
#pragma unroll
        for (uint32_t w = 0; w < kWaves - 1; ++w) wave_off += w < wave ? s_wsum[w] : 0u;
        const uint32_t o_start = min(lead + wave_off + incl - cnt, a.ebuf_cap - kDecodeReach);
        // Round it + 2's ticket (fetched at the top of this iteration) for
        // the other waves; they read it after the next barrier, at the top of
        // iteration it + 1.
        if constexpr (kTail) {
            if (tid == 0 && it + 2u >= len) *s_ticket = n_wg * len + pool_of(wg, a.pools) + a.pools * fetched;
        } else {
            if (sched && tid == 0) *s_ticket = 2u * n_wg + pool_of(wg, a.pools) + a.pools * fetched;
        }

        // Phase 2: OR the (rotated) exponents into the zeroed LDS buffer at
        // their output positions (accumulator x = LDS byte address).  A
        // thread's last lookup may list codes that start past its segment;
        // those are the next thread's first codes, decoded at the same code
        // boundaries, so they land on the next thread's first outputs with the
        // same values (or, after the group's last output, in the chunk the
        // merge zeroes).
        uint32_t acc2;
        if (!__builtin_amdgcn_ballot_w64(spill)) {
            acc2 = (lds_offset(s_ebuf) + o_start) << 11;
#pragma unroll
            for (int j = 0; j < 2 * kSavedSteps; ++j) {
                if (!__builtin_amdgcn_ballot_w64(saux[j] != 0u)) continue;
                or_exponents(acc2, (static_cast<uint64_t>(saux[j] >> 16) << 32) | slo[j]);
                acc2 += saux[j] & 0xFFFFu;
            }
        } else {
            // Some lane needed more lookups than were kept: decode again.
            acc2 = ((lds_offset(s_ebuf) + o_start) << 11) | gap;
            decode_half<K>(pa, end_a, acc2, s_lo, s_aux, s_luts, s_clen, a.n_luts);
            if (end_b) {
                acc2 -= 32u;
                decode_half<K>(pb, end_b, acc2, s_lo, s_aux, s_luts, s_clen, a.n_luts);
            }
        }

        // Group edges (see boundary_codes).  acc2 now addresses the byte after
        // the last code this thread listed, `past` of which opened the next
        // segment, which ends this thread's phase-1 walk at bit p_end.
        if (ltid == kThreadsPerGroup - 1u) {
            bool whole = false;
            const uint32_t c = (8u - (end & 7u)) & 7u;
            if (g + 2u < a.n_groups && c) {
                const uint32_t p_end = (acc & 0xFFu) + shift_back;
                whole = boundary_codes<K>((static_cast<uint64_t>(w2) << 32) | w3, p_end - kSegBits, past, c, acc2,
                                          true, s_lo, s_aux, s_start);
            }
            s_edge[1] = whole;
        }
        if (ltid == 0) {
            bool skip = false;
            const uint32_t c = (8u - (base & 7u)) & 7u;
            if (g >= 1u && g + 1u < a.n_groups && c)
                skip = boundary_codes<K>(pa, gap, 0, c, 0, false, s_lo, s_aux, s_start);
            s_edge[0] = skip;
        }
        if constexpr (kMfma) __builtin_amdgcn_s_waitcnt(0);  // (stage_x's loads have landed)
        __syncthreads();

        prev_base = base;
        prev_end = end;
        if constexpr (kMfma) prev_pass = kTail ? 0u : s_cur / len;
        cur = nx;
        cur_base = nx_base;
        cur_end = nx_end;
        s_cur = s_nx;
    }
    if constexpr (kPairs) {
        merge_group_pairs(a, s_ebuf, sm, prev_base, prev_end, ltid, s_edge[0] != 0, s_edge[1] != 0, s_pair);
    } else if constexpr (TB == 0) {
        merge_group(a, s_ebuf, sm, prev_base, prev_end, ltid, s_edge[0] != 0, s_edge[1] != 0);
    } else if constexpr (kMfma) {
        merge_mfma<MT>(a, m, s_ebuf, sm, prev_base, prev_end, prev_pass, ltid, ps, s_x);
        flush_panel<MT>(m, ps, wave, lane);
    } else {
        merge_matmul<TB>(a, m, s_ebuf, sm, prev_base, prev_end, ltid, s_edge[0] != 0, s_edge[1] != 0, s_yacc, y_row0,
                         y_rows);
        __syncthreads();
        flush_rows<TB>(m, s_yacc, y_row0, y_rows, ltid);
    }
    finish_schedule(sched, n_wg);
}

// One stream over the whole grid.
template <int K, int GPW>
__global__ __launch_bounds__(kThreadsPerGroup *GPW) void df11_decode_kernel(DecodeArgs a) {
    decode_stream<K, GPW, 0>(a, MatmulArgs{}, blockIdx.x, gridDim.x);
}

// The decoder for tile-ordered streams that go back to row-major in whole
// lines (merge_group_pairs), held to the plain decoder's six waves per SIMD.
template <int K, int GPW>
__global__ __launch_bounds__(kThreadsPerGroup *GPW) __attribute__((amdgpu_waves_per_eu(6))) void df11_decode_pairs_kernel(
    DecodeArgs a) {
    decode_stream<K, GPW, 0, false, true>(a, MatmulArgs{}, blockIdx.x, gridDim.x);
}

// Several independent streams (each with its own codebook and output) in one
// launch: the grid is split into ranges of workgroups, one range per stream,
// sized by the stream's work, so that every workgroup stages one stream's
// tables once.  The ranges are taken over a permutation of the workgroup ids
// (id * stride mod grid, stride coprime to the grid), so that each stream
// gets workgroups of every dispatch position; a CU favours its oldest waves,
// and a stream made only of late ids would run ~20% slower than the rest.
// The descriptors travel in the kernel arguments.
constexpr uint32_t kMaxBatch = DF11_MAX_BATCH;
constexpr uint32_t kZero = 0;

struct BatchArgs {
    DecodeArgs s[kMaxBatch];
    uint32_t wg_begin[kMaxBatch + 1];  // stream i owns permuted ids [wg_begin[i], wg_begin[i + 1])
    uint32_t n;
    uint32_t stride;  // coprime to the grid size
};

template <int K, int GPW>
__global__ __launch_bounds__(kThreadsPerGroup *GPW) void df11_decode_batch_kernel(BatchArgs b) {
    const uint32_t id = static_cast<uint32_t>((static_cast<uint64_t>(blockIdx.x) * b.stride) % gridDim.x);
    uint32_t i = 0;
    while (i + 1u < b.n && id >= b.wg_begin[i + 1]) ++i;
    decode_stream<K, GPW, 0>(b.s[i], MatmulArgs{}, id - b.wg_begin[i], b.wg_begin[i + 1] - b.wg_begin[i]);
}

template <int K, int GPW>
__global__ __launch_bounds__(kThreadsPerGroup *GPW) __attribute__((amdgpu_waves_per_eu(6))) void df11_decode_pairs_batch_kernel(
    BatchArgs b) {
    const uint32_t id = static_cast<uint32_t>((static_cast<uint64_t>(blockIdx.x) * b.stride) % gridDim.x);
    uint32_t i = 0;
    while (i + 1u < b.n && id >= b.wg_begin[i + 1]) ++i;
    decode_stream<K, GPW, 0, false, true>(b.s[i], MatmulArgs{}, id - b.wg_begin[i],
                                          b.wg_begin[i + 1] - b.wg_begin[i]);
}

// Decode fused with y = x W^T for up to TB tokens: W's BF16 never leaves the
// workgroup.  y must be zero at the start (df11_zero_kernel, launched first).
constexpr int kLinearGPW = 2;

template <int K, int TB>
__global__ __launch_bounds__(kThreadsPerGroup *kLinearGPW) void df11_linear_kernel(DecodeArgs a, MatmulArgs m) {
    decode_stream<K, kLinearGPW, TB>(a, m, blockIdx.x, gridDim.x);
}

__global__ __launch_bounds__(256) void df11_zero_kernel(float *y, uint32_t n) {
    for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u) y[i] = 0.0f;
}

// Decode fused with y = x W^T on the matrix cores, for any token count: W
// stored in MFMA tile order, 16 MT tokens per pass over the stream (see
// merge_mfma).  y must be zero at the start, or hold what the products add to.
constexpr int kGemmGPW = 2;

// Waves per SIMD the matrix-core kernels are built for (registers per lane:
// 80 at six waves, the decoder's occupancy).
template <int MT>
constexpr int kGemmWaves = MT == 1 ? 6 : MT == 2 ? 6 : 4;

template <int K, int MT, bool kTail = false>
__global__ __launch_bounds__(kThreadsPerGroup *kGemmGPW) __attribute__((amdgpu_waves_per_eu(kGemmWaves<MT>)))
void df11_gemm_kernel(DecodeArgs a, MatmulArgs m) {
    decode_stream<K, kGemmGPW, -MT, kTail>(a, m, blockIdx.x, gridDim.x);
}


// Several weight matrices multiplying the same x in one launch (a block's q,
// k and v, or gate and up): the grid is split between them as for
// df11_decode_batch_kernel.
struct LinearBatchArgs {
    DecodeArgs s[kMaxBatch];
    MatmulArgs m[kMaxBatch];
    uint32_t wg_begin[kMaxBatch + 1];  // stream i owns permuted ids [wg_begin[i], wg_begin[i + 1])
    uint32_t n;
    uint32_t stride;  // coprime to the grid size
};

template <int K, int TB>
__global__ __launch_bounds__(kThreadsPerGroup *kLinearGPW) void df11_linear_batch_kernel(LinearBatchArgs b) {
    const uint32_t id = static_cast<uint32_t>((static_cast<uint64_t>(blockIdx.x) * b.stride) % gridDim.x);
    uint32_t i = 0;
    while (i + 1u < b.n && id >= b.wg_begin[i + 1]) ++i;
    decode_stream<K, kLinearGPW, TB>(b.s[i], b.m[i], id - b.wg_begin[i], b.wg_begin[i + 1] - b.wg_begin[i]);
}

// Several matrix-core products in one launch, the grid split between them
// as for df11_decode_batch_kernel (LinearBatchArgs: each stream with its
// own x, y and shape).
template <int K, int MT, bool kTail = false>
__global__ __launch_bounds__(kThreadsPerGroup *kGemmGPW) __attribute__((amdgpu_waves_per_eu(kGemmWaves<MT>)))
void df11_gemm_batch_kernel(LinearBatchArgs b) {
    const uint32_t id = static_cast<uint32_t>((static_cast<uint64_t>(blockIdx.x) * b.stride) % gridDim.x);
    uint32_t i = 0;
    while (i + 1u < b.n && id >= b.wg_begin[i + 1]) ++i;
    decode_stream<K, kGemmGPW, -MT, kTail>(b.s[i], b.m[i], id - b.wg_begin[i], b.wg_begin[i + 1] - b.wg_begin[i]);
}

// Zero several outputs: y[i] has end[i] - end[i - 1] floats (end[-1] = 0).
struct ZeroArgs {
    float *y[kMaxBatch];
    uint32_t end[kMaxBatch];
    uint32_t n;
};

__global__ __launch_bounds__(256) void df11_zero_batch_kernel(ZeroArgs z) {
    const uint32_t total = z.end[z.n - 1];
    for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < total; i += gridDim.x * 256u) {
        uint32_t k = 0;
        while (i >= z.end[k]) ++k;
        z.y[k][i - (k ? z.end[k - 1] : 0u)] = 0.0f;
    }
}


// Index width of a stream's first-level decode table: decode_table_bits,
// which may be 0 (the default width) for a stream without a table, whose
// table the kernel derives in LDS.
constexpr uint32_t kDefaultTableBits = 11;

uint32_t table_bits(const df11_device_stream *s) {
    return !s->decode_table && s->decode_table_bits == 0 ? kDefaultTableBits : s->decode_table_bits;
}

int validate(const df11_device_stream *s) {
    if (!s) return DF11_E_INVALID_ARG;
    const df11_header &h = s->h;
    if (h.bytes_per_thread != kBytesPerThread || h.threads_per_group != kThreadsPerGroup) return DF11_E_INVALID_ARG;
    if (h.n_elements > DF11_MAX_ELEMENTS) return DF11_E_TOO_LARGE;
    if (h.n_elements == 0) return h.total_bits == 0 ? DF11_OK : DF11_E_BAD_STREAM;
    if (df11_decode_table_bytes(table_bits(s)) == 0) return DF11_E_INVALID_ARG;
    if (s->groups_per_workgroup != 0 && s->groups_per_workgroup != 1 && s->groups_per_workgroup != 2 &&
        s->groups_per_workgroup != 4)
        return DF11_E_INVALID_ARG;
    if (!s->enc || !s->sm || !s->gaps || !s->out_pos || !s->luts || !s->code_lengths)
        return DF11_E_INVALID_ARG;
    if (!aligned(s->enc, 16) || !aligned(s->sm, 16) || !aligned(s->gaps, 4) || !aligned(s->out_pos, 4) ||
        !aligned(s->luts, 4) || !aligned(s->code_lengths, 4) || !aligned(s->decode_table, 16) ||
        (s->schedule && !aligned(s->schedule, 4)))
        return DF11_E_INVALID_ARG;
    if (h.n_luts < 1 || h.n_luts > DF11_MAX_LUTS || h.max_len < 1 || h.max_len > DF11_MAX_CODE_LEN)
        return DF11_E_BAD_STREAM;
    if (h.total_bits < h.n_elements || h.total_bits > DF11_MAX_CODE_LEN * h.n_elements) return DF11_E_BAD_STREAM;
    const uint64_t seg_bits = 8ull * h.bytes_per_thread;
    const uint64_t T = (h.total_bits + seg_bits - 1) / seg_bits;
    const uint64_t groups = (T + h.threads_per_group - 1) / h.threads_per_group;
    if (h.n_threads != T || h.n_groups != groups || h.enc_bytes != round_up(T * h.bytes_per_thread, 16) + 16 ||
        h.sm_bytes != round_up(h.n_elements, 64) || h.gaps_bytes != 4 * ((5 * T + 31) / 32 + 1) ||
        h.out_pos_bytes != 4 * (groups + 1))
        return DF11_E_BAD_STREAM;
    if (h.max_group_elems == 0 || h.max_group_elems > seg_bits * h.threads_per_group) return DF11_E_BAD_STREAM;
    if (s->tile_cols && (s->tile_cols % 32 || h.n_elements % (64ull * s->tile_cols))) return DF11_E_INVALID_ARG;
    return DF11_OK;
}

// Workgroup count of a stream given `want` workgroups, with its pool count
// for the dynamic schedule (df11::pool_shape).  Sets a.sched to null when the
// schedule does not pay.
uint32_t schedule_pools(DecodeArgs &a, uint64_t n_super, uint64_t want) {
    bool dynamic = false;
    const uint32_t n_wg = df11::pool_shape(n_super, want, &a.pools, &dynamic);
    if (!dynamic) a.sched = nullptr;
    return n_wg;
}

// Dynamic LDS of one stream's workgroup (beyond the static decode table),
// with `extra` bytes of the fused product's row sums; a stream without a
// decode table adds the first-code array of its derivation.
template <int K, int GPW>
size_t dynamic_lds(const DecodeArgs &a, size_t extra = 0) {
    return a.n_luts * 256u + 256u + GPW * (a.ebuf_cap + 4u * kWaves + 8u) + 16u + extra + (a.dtab ? 0u : 2u << K);
}

// Whether a stream decompresses through merge_group_pairs: MFMA tile order
// with an even number of k-steps per panel.
bool pairs_layout(const DecodeArgs &a) { return a.tile_cols && a.tile_ks % 2u == 0u; }

// The instance (and its dynamic LDS) a decompression of these streams uses:
// the whole-line one when every stream is paired and its LDS stage leaves as
// many workgroups resident per CU.
template <int K, int GPW, typename Kernel>
const void *pick_pairs(const DecodeArgs *s, uint32_t n, Kernel plain, Kernel paired, int dev, size_t &lds) {
    bool pairs = n > 0;
    for (uint32_t i = 0; i < n; ++i) pairs = pairs && pairs_layout(s[i]);
    if (!pairs) return reinterpret_cast<const void *>(plain);
    size_t lds_p = 0;
    for (uint32_t i = 0; i < n; ++i)
        lds_p = std::max(lds_p, dynamic_lds<K, GPW>(s[i], GPW * kWaves * kPairStageBytes));
    const int plain_cu = resident_per_cu(reinterpret_cast<const void *>(plain), kThreadsPerGroup * GPW, dev, lds);
    const int pair_cu = resident_per_cu(reinterpret_cast<const void *>(paired), kThreadsPerGroup * GPW, dev, lds_p);
    if (pair_cu < plain_cu) return reinterpret_cast<const void *>(plain);
    lds = lds_p;
    return reinterpret_cast<const void *>(paired);
}

template <int K, int GPW>
int launch(const DecodeArgs &a, uint32_t max_wg, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    size_t lds = dynamic_lds<K, GPW>(a);
    int dev = 0, cus = 0;
    if (device_cus(dev, cus)) return DF11_E_HIP;
    const void *fn = pick_pairs<K, GPW>(&a, 1, &df11_decode_kernel<K, GPW>, &df11_decode_pairs_kernel<K, GPW>, dev,
                                        lds);
    const int per_cu = resident_per_cu(fn, kThreadsPerGroup * GPW, dev, lds);
    if (per_cu < 1) return DF11_E_HIP;
    const uint64_t n_super = (a.n_groups + GPW - 1) / GPW;
    uint64_t resident = static_cast<uint64_t>(per_cu) * static_cast<uint64_t>(cus);
    if (max_wg) resident = std::min<uint64_t>(resident, max_wg);
    (void)hipGetLastError();
    DecodeArgs args = a;
    // The dynamic schedule pays a few microseconds of ticket and exit
    // latency; it wins only when each workgroup has many rounds to balance.
    const uint32_t grid = schedule_pools(args, n_super, resident);
    void *params[] = {&args};
    // start / stop (when given) are recorded at the kernel's own start and
    // end, not around the launch.
    return launch_kernel(fn, dim3(grid), dim3(kThreadsPerGroup * GPW), params, lds, stream, start, stop);
}

template <int K>
int launch_k(const DecodeArgs &a, uint32_t gpw, uint32_t max_wg, hipStream_t stream, hipEvent_t start,
             hipEvent_t stop) {
    switch (gpw) {
    case 1: return launch<K, 1>(a, max_wg, stream, start, stop);
    case 4: return launch<K, 4>(a, max_wg, stream, start, stop);
    default: return launch<K, 2>(a, max_wg, stream, start, stop);
    }
}

// Split the resident grid between the streams of a batch (df11::split_grid) and
// launch once.
template <int K, int GPW>
int launch_batch(BatchArgs &b, uint32_t max_wg, hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    size_t lds = 0;
    for (uint32_t i = 0; i < b.n; ++i) lds = std::max(lds, dynamic_lds<K, GPW>(b.s[i]));
    int dev = 0, cus = 0;
    if (device_cus(dev, cus)) return DF11_E_HIP;
    const void *fn = pick_pairs<K, GPW>(b.s, b.n, &df11_decode_batch_kernel<K, GPW>,
                                        &df11_decode_pairs_batch_kernel<K, GPW>, dev, lds);
    const int per_cu = resident_per_cu(fn, kThreadsPerGroup * GPW, dev, lds);
    if (per_cu < 1) return DF11_E_HIP;
    uint64_t resident = static_cast<uint64_t>(per_cu) * static_cast<uint64_t>(cus);
    if (max_wg) resident = std::min<uint64_t>(resident, std::max<uint32_t>(max_wg, b.n));
    uint64_t sup[kMaxBatch], want[kMaxBatch];
    for (uint32_t i = 0; i < b.n; ++i) sup[i] = (b.s[i].n_groups + GPW - 1) / GPW;
    df11::split_grid(sup, b.n, resident, want);
    uint32_t next = 0;
    for (uint32_t i = 0; i < b.n; ++i) {
        const uint32_t share = schedule_pools(b.s[i], sup[i], want[i]);
        b.wg_begin[i] = next;
        next += share;
    }
    b.wg_begin[b.n] = next;
    b.stride = df11::coprime_stride(next);
    (void)hipGetLastError();
    void *params[] = {&b};
    return launch_kernel(fn, dim3(next), dim3(kThreadsPerGroup * GPW), params, lds, stream, start, stop);
}

void fill_args(const df11_device_stream *s, DecodeArgs &a);

// Whether stream i of a batch uses work counters that an earlier stream of
// the same launch also uses (the same tensor twice, say).  Its workgroups
// would take tickets from the other stream's counters, so it runs the static
// schedule instead.
bool shares_schedule(const df11_device_stream *streams, uint32_t i) {
    const uint32_t *sc = streams[i].schedule;
    if (!sc) return false;
    for (uint32_t j = 0; j < i; ++j)
        if (overlaps(sc, 4 * DF11_SCHEDULE_WORDS, streams[j].schedule, streams[j].schedule ? 4 * DF11_SCHEDULE_WORDS : 0))
            return true;
    return false;
}

// Checks s and out (no launch) and fills the kernel arguments of one stream.
int make_args(const df11_device_stream *s, uint16_t *out, DecodeArgs &a) {
    int rc = validate(s);
    if (rc) return rc;
    const df11_header &h = s->h;
    if (h.n_elements == 0) return DF11_OK;
    if (!out || !aligned(out, 16)) return DF11_E_INVALID_ARG;
    const uint64_t out_bytes = 2 * h.n_elements;
    const uint32_t bits = table_bits(s);
    if (overlaps(out, out_bytes, s->enc, h.enc_bytes) || overlaps(out, out_bytes, s->sm, h.sm_bytes) ||
        overlaps(out, out_bytes, s->gaps, h.gaps_bytes) || overlaps(out, out_bytes, s->out_pos, h.out_pos_bytes) ||
        overlaps(out, out_bytes, s->luts, 256ull * h.n_luts) || overlaps(out, out_bytes, s->code_lengths, 256) ||
        overlaps(out, out_bytes, s->decode_table, df11_decode_table_bytes(bits)) ||
        overlaps(out, out_bytes, s->schedule, s->schedule ? 4 * DF11_SCHEDULE_WORDS : 0))
        return DF11_E_INVALID_ARG;
    fill_args(s, a);
    a.out = out;
    return DF11_OK;
}

// Kernel arguments of a validated, non-empty stream (no output).
void fill_args(const df11_device_stream *s, DecodeArgs &a) {
    const df11_header &h = s->h;
    a = DecodeArgs{};
    a.enc = s->enc;
    a.sm = s->sm;
    a.gaps = s->gaps;
    a.out_pos = s->out_pos;
    a.luts = s->luts;
    a.code_lengths = s->code_lengths;
    a.dtab = static_cast<const uint32_t *>(s->decode_table);
    a.total_bits = h.total_bits;
    a.n_elements = static_cast<uint32_t>(h.n_elements);
    a.n_threads = static_cast<uint32_t>(h.n_threads);
    a.n_groups = static_cast<uint32_t>(h.n_groups);
    a.n_luts = h.n_luts;
    // lead (< 8) + the group's elements, rounded up to whole 8-byte chunks, plus
    // slack for the 8-byte LDS writes.
    a.ebuf_cap = static_cast<uint32_t>(round_up(static_cast<uint64_t>(h.max_group_elems) + 8 + kDecodeReach, 16));
    a.last_seg_bits = static_cast<uint32_t>(h.total_bits - kSegBits * (h.n_threads - 1));
    a.sm_chunks = static_cast<uint32_t>(h.sm_bytes / 8);
    a.sched = s->schedule;
    a.tile_cols = s->tile_cols;
    if (s->tile_cols) {
        a.tile_ks = s->tile_cols / 32u;
        a.tile_magic = ~0ull / a.tile_ks + 1ull;  // umulhi64(i, tile_magic) == i / tile_ks for all i < 2^32
    }
}

int decompress_impl(const df11_device_stream *s, uint16_t *out, hipStream_t stream, hipEvent_t start,
                    hipEvent_t stop) {
    DecodeArgs a;
    const int rc = make_args(s, out, a);
    if (rc || s->h.n_elements == 0) return rc;
    const uint32_t gpw = s->groups_per_workgroup ? s->groups_per_workgroup : kDefaultGroupsPerWorkgroup;
    switch (table_bits(s)) {
    case 10: return launch_k<10>(a, gpw, s->max_workgroups, stream, start, stop);
    case 11: return launch_k<11>(a, gpw, s->max_workgroups, stream, start, stop);
    case 12: return launch_k<12>(a, gpw, s->max_workgroups, stream, start, stop);
    default: return DF11_E_INVALID_ARG;
    }
}

__global__ __launch_bounds__(256) void df11_fill_u32_kernel(uint32_t *p, uint32_t n, uint32_t v) {
    for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u) p[i] = v;
}

// counters: when not null, stream i of the call takes its dynamic-schedule
// counters from counters + i * DF11_SCHEDULE_WORDS (zeroed by a fill kernel
// launched before the decode) instead of streams[i].schedule.
int decompress_batch_impl(const df11_device_stream *streams, uint32_t n, uint16_t *const *outs,
                          hipStream_t stream, hipEvent_t start, hipEvent_t stop, uint32_t *counters = nullptr) {
    if (n > kMaxBatch) return DF11_E_TOO_LARGE;
    if (n && (!streams || !outs)) return DF11_E_INVALID_ARG;
    BatchArgs b{};
    uint32_t bits = 0, gpw = 0, max_wg = 0;
    for (uint32_t i = 0; i < n; ++i) {
        DecodeArgs a;
        const int rc = make_args(&streams[i], outs[i], a);
        if (rc) return rc;
        // every output must also stay clear of the other streams' buffers and outputs
        const uint64_t out_bytes = 2 * streams[i].h.n_elements;
        for (uint32_t j = 0; j < n; ++j) {
            if (j == i) continue;
            const df11_device_stream &o = streams[j];
            if (overlaps(outs[i], out_bytes, outs[j], 2 * o.h.n_elements) ||
                overlaps(outs[i], out_bytes, o.enc, o.h.enc_bytes) || overlaps(outs[i], out_bytes, o.sm, o.h.sm_bytes) ||
                overlaps(outs[i], out_bytes, o.gaps, o.h.gaps_bytes) ||
                overlaps(outs[i], out_bytes, o.out_pos, o.h.out_pos_bytes) ||
                overlaps(outs[i], out_bytes, o.luts, 256ull * o.h.n_luts) ||
                overlaps(outs[i], out_bytes, o.code_lengths, 256) ||
                overlaps(outs[i], out_bytes, o.decode_table, df11_decode_table_bytes(table_bits(&o))) ||
                overlaps(outs[i], out_bytes, o.schedule, o.schedule ? 4 * DF11_SCHEDULE_WORDS : 0))
                return DF11_E_INVALID_ARG;
        }
        if (streams[i].h.n_elements == 0) continue;
        if (counters) {
            a.sched = counters + i * DF11_SCHEDULE_WORDS;
        } else if (shares_schedule(streams, i)) {
            a.sched = nullptr;
        }
        const uint32_t g = streams[i].groups_per_workgroup ? streams[i].groups_per_workgroup
                                                           : kDefaultGroupsPerWorkgroup;
        if (streams[i].max_workgroups) max_wg = max_wg ? std::min(max_wg, streams[i].max_workgroups)
                                                       : streams[i].max_workgroups;
        if (b.n == 0) {
            bits = table_bits(&streams[i]);
            gpw = g;
        } else if (table_bits(&streams[i]) != bits || g != gpw) {
            return DF11_E_INVALID_ARG;
        }
        b.s[b.n++] = a;
    }
    if (b.n == 0) return DF11_OK;
    if (counters) {
        const uint32_t words = n * DF11_SCHEDULE_WORDS;
        void *fparams[] = {&counters, const_cast<uint32_t *>(&words), const_cast<uint32_t *>(&kZero)};
        const int rc = launch_kernel(reinterpret_cast<const void *>(&df11_fill_u32_kernel), dim3(1), dim3(256),
                                     fparams, 0, stream, nullptr, nullptr);
        if (rc) return rc;
    }
    if (b.n == 1) {  // one non-empty stream: the single-stream kernel
        switch (bits) {
        case 10: return launch_k<10>(b.s[0], gpw, max_wg, stream, start, stop);
        case 11: return launch_k<11>(b.s[0], gpw, max_wg, stream, start, stop);
        case 12: return launch_k<12>(b.s[0], gpw, max_wg, stream, start, stop);
        default: return DF11_E_INVALID_ARG;
        }
    }
#define DF11_BATCH_CASE(KB)                                                  \
    case KB:                                                                 \
        switch (gpw) {                                                       \
        case 1: return launch_batch<KB, 1>(b, max_wg, stream, start, stop);  \
        case 4: return launch_batch<KB, 4>(b, max_wg, stream, start, stop);  \
        default: return launch_batch<KB, 2>(b, max_wg, stream, start, stop); \
        }
    switch (bits) {
        DF11_BATCH_CASE(10)
        DF11_BATCH_CASE(11)
        DF11_BATCH_CASE(12)
    default: return DF11_E_INVALID_ARG;
    }
#undef DF11_BATCH_CASE
}

// y = 0 (zero kernel, unless the caller accumulates into y), then the
// fused kernel over the persistent grid.
template <int K, int TB>
int launch_linear(const DecodeArgs &a, const MatmulArgs &m, uint32_t max_wg, hipStream_t stream,
                  hipEvent_t start, hipEvent_t stop, bool zero) {
    const size_t lds = dynamic_lds<K, kLinearGPW>(a, sizeof(float) * kLinearGPW * m.yacc_rows * TB);
    int dev = 0, cus = 0;
    if (device_cus(dev, cus)) return DF11_E_HIP;
    const void *fn = reinterpret_cast<const void *>(&df11_linear_kernel<K, TB>);
    const int per_cu = resident_per_cu(fn, kThreadsPerGroup * kLinearGPW, dev, lds);
    if (per_cu < 1) return DF11_E_HIP;
    const uint64_t n_super = (a.n_groups + kLinearGPW - 1) / kLinearGPW;
    uint64_t resident = static_cast<uint64_t>(per_cu) * static_cast<uint64_t>(cus);
    if (max_wg) resident = std::min<uint64_t>(resident, max_wg);
    (void)hipGetLastError();
    DecodeArgs args = a;
    MatmulArgs margs = m;
    const uint32_t grid = schedule_pools(args, n_super, resident);
    const uint32_t n_y = m.n_tokens * m.out_features;
    float *y = m.y;
    void *zparams[] = {&y, const_cast<uint32_t *>(&n_y)};
    const uint32_t zgrid = std::max<uint32_t>(1, std::min<uint32_t>((n_y + 255) / 256, 1024));
    if (zero) {
        const int rc = launch_kernel(reinterpret_cast<const void *>(&df11_zero_kernel), dim3(zgrid), dim3(256),
                                     zparams, 0, stream, nullptr, nullptr);
        if (rc) return rc;
    }
    void *params[] = {&args, &margs};
    return launch_kernel(fn, dim3(grid), dim3(kThreadsPerGroup * kLinearGPW), params, lds, stream, start, stop);
}

// Checks one product's arguments (no launch) and fills its kernel arguments;
// *empty is set for a stream with no rows (nothing to launch).
int linear_args(const df11_device_stream *s, const uint16_t *x, uint32_t n_tokens, uint32_t in_features,
                uint32_t out_features, float *y, DecodeArgs &a, MatmulArgs &m, bool &empty) {
    int rc = validate(s);
    if (rc) return rc;
    const df11_header &h = s->h;
    if (n_tokens < 1 || n_tokens > DF11_LINEAR_MAX_TOKENS || in_features < DF11_LINEAR_MIN_IN_FEATURES ||
        in_features % 8 || static_cast<uint64_t>(in_features) * out_features != h.n_elements || s->tile_cols)
        return DF11_E_INVALID_ARG;
    empty = h.n_elements == 0;
    if (empty) return DF11_OK;
    if (!x || !y || !aligned(x, 16) || !aligned(y, 4)) return DF11_E_INVALID_ARG;
    const uint64_t y_bytes = 4ull * n_tokens * out_features, x_bytes = 2ull * n_tokens * in_features;
    if (overlaps(y, y_bytes, x, x_bytes) || overlaps(y, y_bytes, s->enc, h.enc_bytes) ||
        overlaps(y, y_bytes, s->sm, h.sm_bytes) || overlaps(y, y_bytes, s->gaps, h.gaps_bytes) ||
        overlaps(y, y_bytes, s->out_pos, h.out_pos_bytes) || overlaps(y, y_bytes, s->luts, 256ull * h.n_luts) ||
        overlaps(y, y_bytes, s->code_lengths, 256) ||
        overlaps(y, y_bytes, s->decode_table, df11_decode_table_bytes(table_bits(s))) ||
        overlaps(y, y_bytes, s->schedule, s->schedule ? 4 * DF11_SCHEDULE_WORDS : 0))
        return DF11_E_INVALID_ARG;
    if (y_bytes / 4 >= (1ull << 32)) return DF11_E_TOO_LARGE;
    fill_args(s, a);
    m = MatmulArgs{};
    m.x = x;
    m.y = y;
    m.row_magic = ~0ull / in_features + 1ull;  // umulhi64(i, row_magic) == i / in_features for all i < 2^32
    m.in_features = in_features;
    m.out_features = out_features;
    m.n_tokens = n_tokens;
    m.yacc_rows = (a.ebuf_cap - 1u) / in_features + 2u;
    return DF11_OK;
}

uint32_t token_slots(uint32_t n_tokens) { return n_tokens <= 1 ? 1 : n_tokens <= 2 ? 2 : n_tokens <= 4 ? 4 : 8; }

int linear_impl(const df11_device_stream *s, const uint16_t *x, uint32_t n_tokens, uint32_t in_features,
                uint32_t out_features, float *y, hipStream_t stream, hipEvent_t start, hipEvent_t stop,
                bool zero) {
    DecodeArgs a;
    MatmulArgs m;
    bool empty = false;
    const int rc = linear_args(s, x, n_tokens, in_features, out_features, y, a, m, empty);
    if (rc || empty) return rc;
#define DF11_LINEAR_CASE(KB)                                                                      \
    case KB:                                                                                      \
        switch (token_slots(n_tokens)) {                                                          \
        case 1: return launch_linear<KB, 1>(a, m, s->max_workgroups, stream, start, stop, zero);  \
        case 2: return launch_linear<KB, 2>(a, m, s->max_workgroups, stream, start, stop, zero);  \
        case 4: return launch_linear<KB, 4>(a, m, s->max_workgroups, stream, start, stop, zero);  \
        default: return launch_linear<KB, 8>(a, m, s->max_workgroups, stream, start, stop, zero); \
        }
    switch (table_bits(s)) {
        DF11_LINEAR_CASE(10)
        DF11_LINEAR_CASE(11)
        DF11_LINEAR_CASE(12)
    default: return DF11_E_INVALID_ARG;
    }
#undef DF11_LINEAR_CASE
}

// Zero every output, then the batched fused kernel over the persistent grid
// split between the streams (df11::split_grid).
template <int K, int TB>
int launch_linear_batch(LinearBatchArgs &b, ZeroArgs &z, uint32_t max_wg, hipStream_t stream, hipEvent_t start,
                        hipEvent_t stop, bool zero) {
    size_t lds = 0;
    for (uint32_t i = 0; i < b.n; ++i)
        lds = std::max(lds, dynamic_lds<K, kLinearGPW>(b.s[i], sizeof(float) * kLinearGPW * b.m[i].yacc_rows * TB));
    int dev = 0, cus = 0;
    if (device_cus(dev, cus)) return DF11_E_HIP;
    const void *fn = reinterpret_cast<const void *>(&df11_linear_batch_kernel<K, TB>);
    const int per_cu = resident_per_cu(fn, kThreadsPerGroup * kLinearGPW, dev, lds);
    if (per_cu < 1) return DF11_E_HIP;
    uint64_t resident = static_cast<uint64_t>(per_cu) * static_cast<uint64_t>(cus);
    if (max_wg) resident = std::min<uint64_t>(resident, std::max<uint32_t>(max_wg, b.n));
    uint64_t sup[kMaxBatch], want[kMaxBatch];
    for (uint32_t i = 0; i < b.n; ++i) sup[i] = (b.s[i].n_groups + kLinearGPW - 1) / kLinearGPW;
    df11::split_grid(sup, b.n, resident, want);
    uint32_t next = 0;
    for (uint32_t i = 0; i < b.n; ++i) {
        const uint32_t share = schedule_pools(b.s[i], sup[i], want[i]);
        b.wg_begin[i] = next;
        next += share;
    }
    b.wg_begin[b.n] = next;
    b.stride = df11::coprime_stride(next);
    (void)hipGetLastError();
    const uint32_t total = z.end[z.n - 1];
    void *zparams[] = {&z};
    const uint32_t zgrid = std::max<uint32_t>(1, std::min<uint32_t>((total + 255) / 256, 1024));
    if (zero) {
        const int rc = launch_kernel(reinterpret_cast<const void *>(&df11_zero_batch_kernel), dim3(zgrid), dim3(256),
                                     zparams, 0, stream, nullptr, nullptr);
        if (rc) return rc;
    }
    void *params[] = {&b};
    return launch_kernel(fn, dim3(next), dim3(kThreadsPerGroup * kLinearGPW), params, lds, stream, start, stop);
}

int linear_batch_impl(const df11_device_stream *ws, uint32_t n, const uint16_t *x, uint32_t n_tokens,
                      uint32_t in_features, const uint32_t *out_features, float *const *ys, hipStream_t stream,
                      hipEvent_t start, hipEvent_t stop, bool zero) {
    if (n > kMaxBatch) return DF11_E_TOO_LARGE;
    if (n && (!ws || !out_features || !ys)) return DF11_E_INVALID_ARG;
    LinearBatchArgs b{};
    ZeroArgs z{};
    uint32_t bits = 0, max_wg = 0, total = 0;
    for (uint32_t i = 0; i < n; ++i) {
        DecodeArgs a;
        MatmulArgs m;
        bool empty = false;
        const int rc = linear_args(&ws[i], x, n_tokens, in_features, out_features[i], ys[i], a, m, empty);
        if (rc) return rc;
        // every output must also stay clear of the other outputs and the other streams' buffers
        const uint64_t y_bytes = 4ull * n_tokens * out_features[i];
        for (uint32_t j = 0; j < n && !empty; ++j) {
            if (j == i) continue;
            const df11_device_stream &o = ws[j];
            if (overlaps(ys[i], y_bytes, ys[j], 4ull * n_tokens * out_features[j]) ||
                overlaps(ys[i], y_bytes, o.enc, o.h.enc_bytes) || overlaps(ys[i], y_bytes, o.sm, o.h.sm_bytes) ||
                overlaps(ys[i], y_bytes, o.gaps, o.h.gaps_bytes) ||
                overlaps(ys[i], y_bytes, o.out_pos, o.h.out_pos_bytes) ||
                overlaps(ys[i], y_bytes, o.luts, 256ull * o.h.n_luts) ||
                overlaps(ys[i], y_bytes, o.code_lengths, 256) ||
                overlaps(ys[i], y_bytes, o.decode_table, df11_decode_table_bytes(table_bits(&o))) ||
                overlaps(ys[i], y_bytes, o.schedule, o.schedule ? 4 * DF11_SCHEDULE_WORDS : 0))
                return DF11_E_INVALID_ARG;
        }
        if (empty) continue;
        if (shares_schedule(ws, i)) a.sched = nullptr;
        if (b.n && table_bits(&ws[i]) != bits) return DF11_E_INVALID_ARG;
        bits = table_bits(&ws[i]);
        if (ws[i].max_workgroups) max_wg = max_wg ? std::min(max_wg, ws[i].max_workgroups) : ws[i].max_workgroups;
        if (static_cast<uint64_t>(total) + static_cast<uint64_t>(n_tokens) * out_features[i] >= (1ull << 32))
            return DF11_E_TOO_LARGE;
        total += n_tokens * out_features[i];
        z.y[b.n] = ys[i];
        z.end[b.n] = total;
        b.s[b.n] = a;
        b.m[b.n] = m;
        ++b.n;
    }
    if (b.n == 0) return DF11_OK;
    z.n = b.n;
#define DF11_LINEAR_BATCH_CASE(KB)                                                           \
    case KB:                                                                                 \
        switch (token_slots(n_tokens)) {                                                     \
        case 1: return launch_linear_batch<KB, 1>(b, z, max_wg, stream, start, stop, zero);  \
        case 2: return launch_linear_batch<KB, 2>(b, z, max_wg, stream, start, stop, zero);  \
        case 4: return launch_linear_batch<KB, 4>(b, z, max_wg, stream, start, stop, zero);  \
        default: return launch_linear_batch<KB, 8>(b, z, max_wg, stream, start, stop, zero); \
        }
    switch (bits) {
        DF11_LINEAR_BATCH_CASE(10)
        DF11_LINEAR_BATCH_CASE(11)
        DF11_LINEAR_BATCH_CASE(12)
    default: return DF11_E_INVALID_ARG;
    }
#undef DF11_LINEAR_BATCH_CASE
}

// The matrix-core product: y = 0 (unless accumulating), then the fused
// kernel over as many workgroups as fit at once (at most one per
// super-group), each with a contiguous range of the stream.
// LDS of the staged x tiles of a matrix-core workgroup (stage_x).
template <int MT>
constexpr size_t kGemmXBytes = kGemmGPW * kXTiles<MT> * MT * 1024u;

// The dealt tail of the one-tile matrix-core product (decode_stream with
// kTail): at up to kTailMaxTokens tokens (a flush of a wave's sums is then
// at most 128 atomics) a stream with work counters and at least
// kDynamicMinRounds super-groups per workgroup sweeps fixed ranges over
// kTailFixedPercent of its super-groups and deals the rest out by tickets.
// The fixed ranges keep a panel's sums in registers; the dealt rest absorbs
// the workgroups' different speeds (the three on a CU differ by ~3% each
// step, CUs by a few percent), which fixed ranges alone left as ~20 us
// between the first and the last workgroup to end.  On the block at one
// token: 125.5 us against 135.5 with fixed ranges alone (70% fixed 128,
// 80% 127, 90% 126, 95% and 97% 125.5); at 16 tokens, where a flush is 256
// atomics per wave, the dealt tail lost (140 against 137).
constexpr uint32_t kTailMaxTokens = 8;
constexpr uint64_t kTailFixedPercent = 95;

// Sets up the dealt tail for a stream given `want` workgroups: pools and
// m.fixed_len; returns the workgroup count, or 0 (a.sched cleared) when the
// stream does not qualify.
uint32_t tail_schedule(DecodeArgs &a, MatmulArgs &m, uint64_t n_super, uint64_t want) {
    m.fixed_len = 0;
    if (!a.sched || m.n_tokens > kTailMaxTokens) {
        a.sched = nullptr;
        return 0;
    }
    const uint32_t n_wg = schedule_pools(a, n_super, want);
    const uint64_t fixed = n_super * kTailFixedPercent / 100 / n_wg;
    if (!a.sched || fixed < 2) {
        a.sched = nullptr;
        return 0;
    }
    m.fixed_len = static_cast<uint32_t>(fixed);
    return n_wg;
}

template <int K, int MT>
int launch_gemm(const DecodeArgs &a, const MatmulArgs &m, uint32_t max_wg, hipStream_t stream, hipEvent_t start,
                hipEvent_t stop, bool zero) {
    const size_t lds = dynamic_lds<K, kGemmGPW>(a, kGemmXBytes<MT>);
    int dev = 0, cus = 0;
    if (device_cus(dev, cus)) return DF11_E_HIP;
    const void *fn = reinterpret_cast<const void *>(&df11_gemm_kernel<K, MT>);
    // (the persistent grid must fit whichever instance launches)
    int per_cu = resident_per_cu(fn, kThreadsPerGroup * kGemmGPW, dev, lds);
    if constexpr (MT == 1)
        per_cu = std::min(per_cu, resident_per_cu(reinterpret_cast<const void *>(&df11_gemm_kernel<K, 1, true>),
                                                  kThreadsPerGroup * kGemmGPW, dev, lds));
    if (per_cu < 1) return DF11_E_HIP;
    const uint64_t n_super = (a.n_groups + kGemmGPW - 1) / kGemmGPW;
    uint64_t resident = static_cast<uint64_t>(per_cu) * static_cast<uint64_t>(cus);
    if (max_wg) resident = std::min<uint64_t>(resident, max_wg);
    uint32_t grid = static_cast<uint32_t>(std::max<uint64_t>(1, std::min(resident, n_super)));
    (void)hipGetLastError();
    DecodeArgs args = a;
    MatmulArgs margs = m;
    margs.passes = (m.n_tokens + 16u * MT - 1u) / (16u * MT);
    if constexpr (MT == 1) {
        if (const uint32_t n_wg = tail_schedule(args, margs, n_super, resident)) {
            grid = n_wg;
            fn = reinterpret_cast<const void *>(&df11_gemm_kernel<K, 1, true>);
        }
    } else {
        args.sched = nullptr;  // (contiguous ranges: no dynamic schedule)
    }
    if (zero) {
        float *y = m.y;
        const uint32_t n_y = m.n_tokens * m.out_features;
        void *zparams[] = {&y, const_cast<uint32_t *>(&n_y)};
        const uint32_t zgrid = std::max<uint32_t>(1, std::min<uint32_t>((n_y + 255) / 256, 1024));
        const int rc = launch_kernel(reinterpret_cast<const void *>(&df11_zero_kernel), dim3(zgrid), dim3(256),
                                     zparams, 0, stream, nullptr, nullptr);
        if (rc) return rc;
    }
    void *params[] = {&args, &margs};
    return launch_kernel(fn, dim3(grid), dim3(kThreadsPerGroup * kGemmGPW), params, lds, stream, start, stop);
}

// Checks one matrix-core product's arguments (no launch) and fills its
// kernel arguments; *empty is set for a stream with no elements.
int gemm_args(const df11_device_stream *s, const uint16_t *x, uint32_t n_tokens, uint32_t in_features,
              uint32_t out_features, float *y, DecodeArgs &a, MatmulArgs &m, bool &empty) {
    int rc = validate(s);
    if (rc) return rc;
    const df11_header &h = s->h;
    if (n_tokens < 1 || in_features < 32 || in_features % 32 || out_features % 64 ||
        static_cast<uint64_t>(in_features) * out_features != h.n_elements ||
        (h.n_elements && s->tile_cols != in_features))
        return DF11_E_INVALID_ARG;
    empty = h.n_elements == 0;
    if (empty) return DF11_OK;
    if (!x || !y || !aligned(x, 16) || !aligned(y, 4)) return DF11_E_INVALID_ARG;
    const uint64_t y_elems = static_cast<uint64_t>(n_tokens) * out_features;
    const uint64_t y_bytes = 4 * y_elems, x_bytes = 2ull * n_tokens * in_features;
    // (the kernel numbers its iterations, passes x super-groups, with 32 bits)
    const uint64_t sweeps = (n_tokens + 15ull) / 16ull, n_super = (h.n_groups + kGemmGPW - 1) / kGemmGPW;
    if (y_elems >= (1ull << 32) || sweeps * n_super >= (1ull << 31)) return DF11_E_TOO_LARGE;
    if (overlaps(y, y_bytes, x, x_bytes) || overlaps(y, y_bytes, s->enc, h.enc_bytes) ||
        overlaps(y, y_bytes, s->sm, h.sm_bytes) || overlaps(y, y_bytes, s->gaps, h.gaps_bytes) ||
        overlaps(y, y_bytes, s->out_pos, h.out_pos_bytes) || overlaps(y, y_bytes, s->luts, 256ull * h.n_luts) ||
        overlaps(y, y_bytes, s->code_lengths, 256) ||
        overlaps(y, y_bytes, s->decode_table, df11_decode_table_bytes(table_bits(s))))
        return DF11_E_INVALID_ARG;
    fill_args(s, a);
    m = MatmulArgs{};
    m.x = x;
    m.y = y;
    m.in_features = in_features;
    m.out_features = out_features;
    m.n_tokens = n_tokens;
    return DF11_OK;
}

// Token tiles of 16 per pass: 1 up to 16 tokens, 2 up to 32, else 4.
uint32_t gemm_tiles(uint32_t n_tokens) { return n_tokens <= 16 ? 1 : n_tokens <= 32 ? 2 : 4; }

int gemm_impl(const df11_device_stream *s, const uint16_t *x, uint32_t n_tokens, uint32_t in_features,
              uint32_t out_features, float *y, hipStream_t stream, hipEvent_t start, hipEvent_t stop, bool zero) {
    DecodeArgs a;
    MatmulArgs m;
    bool empty = false;
    const int rc = gemm_args(s, x, n_tokens, in_features, out_features, y, a, m, empty);
    if (rc || empty) return rc;
#define DF11_GEMM_CASE(KB)                                                                   \
    case KB:                                                                                 \
        switch (gemm_tiles(n_tokens)) {                                                      \
        case 1: return launch_gemm<KB, 1>(a, m, s->max_workgroups, stream, start, stop, zero); \
        case 2: return launch_gemm<KB, 2>(a, m, s->max_workgroups, stream, start, stop, zero); \
        default: return launch_gemm<KB, 4>(a, m, s->max_workgroups, stream, start, stop, zero); \
        }
    switch (table_bits(s)) {
        DF11_GEMM_CASE(10)
        DF11_GEMM_CASE(11)
        DF11_GEMM_CASE(12)
    default: return DF11_E_INVALID_ARG;
    }
#undef DF11_GEMM_CASE
}

// Several matrix-core products in one launch: every output zeroed by one
// kernel (unless accumulating), then the batched fused kernel over the
// resident grid split between the streams in proportion to their
// super-groups (every stream sweeps its range the same number of times).
template <int K, int MT>
int launch_gemm_batch(LinearBatchArgs &b, ZeroArgs &z, uint32_t max_wg, hipStream_t stream, hipEvent_t start,
                      hipEvent_t stop, bool zero) {
    size_t lds = 0;
    for (uint32_t i = 0; i < b.n; ++i) lds = std::max(lds, dynamic_lds<K, kGemmGPW>(b.s[i], kGemmXBytes<MT>));
    int dev = 0, cus = 0;
    if (device_cus(dev, cus)) return DF11_E_HIP;
    const void *fn = reinterpret_cast<const void *>(&df11_gemm_batch_kernel<K, MT>);
    // (the persistent grid must fit whichever instance launches)
    int per_cu = resident_per_cu(fn, kThreadsPerGroup * kGemmGPW, dev, lds);
    if constexpr (MT == 1)
        per_cu = std::min(per_cu, resident_per_cu(reinterpret_cast<const void *>(&df11_gemm_batch_kernel<K, 1, true>),
                                                  kThreadsPerGroup * kGemmGPW, dev, lds));
    if (per_cu < 1) return DF11_E_HIP;
    uint64_t resident = static_cast<uint64_t>(per_cu) * static_cast<uint64_t>(cus);
    if (max_wg) resident = std::min<uint64_t>(resident, std::max<uint32_t>(max_wg, b.n));
    uint64_t sup[kMaxBatch], want[kMaxBatch];
    for (uint32_t i = 0; i < b.n; ++i) sup[i] = (b.s[i].n_groups + kGemmGPW - 1) / kGemmGPW;
    df11::split_grid(sup, b.n, resident, want);
    // The dealt tail when every stream qualifies (one kernel serves them all).
    bool tail = MT == 1;
    uint32_t share[kMaxBatch];
    for (uint32_t i = 0; i < b.n; ++i) {
        b.m[i].passes = (b.m[i].n_tokens + 16u * MT - 1u) / (16u * MT);
        DecodeArgs s = b.s[i];
        share[i] = tail ? tail_schedule(s, b.m[i], sup[i], want[i]) : 0u;
        tail = tail && share[i] != 0;
        if (share[i]) b.s[i].pools = s.pools;
    }
    uint32_t next = 0;
    for (uint32_t i = 0; i < b.n; ++i) {
        if (!tail) {
            b.s[i].sched = nullptr;  // (contiguous ranges: no dynamic schedule)
            b.m[i].fixed_len = 0;
        }
        b.wg_begin[i] = next;
        next += tail ? share[i] : static_cast<uint32_t>(want[i]);
    }
    if constexpr (MT == 1) {
        if (tail) fn = reinterpret_cast<const void *>(&df11_gemm_batch_kernel<K, 1, true>);
    }
    b.wg_begin[b.n] = next;
    b.stride = df11::coprime_stride(next);
    (void)hipGetLastError();
    if (zero) {
        const uint32_t total = z.end[z.n - 1];
        void *zparams[] = {&z};
        const uint32_t zgrid = std::max<uint32_t>(1, std::min<uint32_t>((total + 255) / 256, 1024));
        const int rc = launch_kernel(reinterpret_cast<const void *>(&df11_zero_batch_kernel), dim3(zgrid), dim3(256),
                                     zparams, 0, stream, nullptr, nullptr);
        if (rc) return rc;
    }
    void *params[] = {&b};
    return launch_kernel(fn, dim3(next), dim3(kThreadsPerGroup * kGemmGPW), params, lds, stream, start, stop);
}

int gemm_batch_impl(const df11_device_stream *ws, uint32_t n, const uint16_t *const *xs, uint32_t n_tokens,
                    const uint32_t *in_features, const uint32_t *out_features, float *const *ys, hipStream_t stream,
                    hipEvent_t start, hipEvent_t stop, bool zero) {
    if (n > kMaxBatch) return DF11_E_TOO_LARGE;
    if (n && (!ws || !xs || !in_features || !out_features || !ys)) return DF11_E_INVALID_ARG;
    LinearBatchArgs b{};
    ZeroArgs z{};
    uint32_t bits = 0, max_wg = 0, total = 0;
    for (uint32_t i = 0; i < n; ++i) {
        DecodeArgs a;
        MatmulArgs m;
        bool empty = false;
        const int rc = gemm_args(&ws[i], xs[i], n_tokens, in_features[i], out_features[i], ys[i], a, m, empty);
        if (rc) return rc;
        // every output must also stay clear of the other outputs, every x and the other streams' buffers
        const uint64_t y_bytes = 4ull * n_tokens * out_features[i];
        for (uint32_t j = 0; j < n && !empty; ++j) {
            if (overlaps(ys[i], y_bytes, xs[j], 2ull * n_tokens * in_features[j])) return DF11_E_INVALID_ARG;
            if (j == i) continue;
            const df11_device_stream &o = ws[j];
            if (overlaps(ys[i], y_bytes, ys[j], 4ull * n_tokens * out_features[j]) ||
                overlaps(ys[i], y_bytes, o.enc, o.h.enc_bytes) || overlaps(ys[i], y_bytes, o.sm, o.h.sm_bytes) ||
                overlaps(ys[i], y_bytes, o.gaps, o.h.gaps_bytes) ||
                overlaps(ys[i], y_bytes, o.out_pos, o.h.out_pos_bytes) ||
                overlaps(ys[i], y_bytes, o.luts, 256ull * o.h.n_luts) ||
                overlaps(ys[i], y_bytes, o.code_lengths, 256) ||
                overlaps(ys[i], y_bytes, o.decode_table, df11_decode_table_bytes(table_bits(&o))))
                return DF11_E_INVALID_ARG;
        }
        if (empty) continue;
        if (b.n && table_bits(&ws[i]) != bits) return DF11_E_INVALID_ARG;
        bits = table_bits(&ws[i]);
        if (ws[i].max_workgroups) max_wg = max_wg ? std::min(max_wg, ws[i].max_workgroups) : ws[i].max_workgroups;
        if (static_cast<uint64_t>(total) + static_cast<uint64_t>(n_tokens) * out_features[i] >= (1ull << 32))
            return DF11_E_TOO_LARGE;
        total += n_tokens * out_features[i];
        z.y[b.n] = ys[i];
        z.end[b.n] = total;
        if (shares_schedule(ws, i)) a.sched = nullptr;  // (the same tensor twice, say)
        b.s[b.n] = a;
        b.m[b.n] = m;
        ++b.n;
    }
    if (b.n == 0) return DF11_OK;
    if (b.n == 1) {
        // One product: the one-stream kernel, whose loop keeps the stream's
        // arguments in scalar registers instead of indexing the batch's.
#define DF11_GEMM_ONE_CASE(KB)                                                                         \
    case KB:                                                                                           \
        switch (gemm_tiles(n_tokens)) {                                                                \
        case 1: return launch_gemm<KB, 1>(b.s[0], b.m[0], max_wg, stream, start, stop, zero);          \
        case 2: return launch_gemm<KB, 2>(b.s[0], b.m[0], max_wg, stream, start, stop, zero);          \
        default: return launch_gemm<KB, 4>(b.s[0], b.m[0], max_wg, stream, start, stop, zero);         \
        }
        switch (bits) {
            DF11_GEMM_ONE_CASE(10)
            DF11_GEMM_ONE_CASE(11)
            DF11_GEMM_ONE_CASE(12)
        default: return DF11_E_INVALID_ARG;
        }
#undef DF11_GEMM_ONE_CASE
    }
    z.n = b.n;
#define DF11_GEMM_BATCH_CASE(KB)                                                                \
    case KB:                                                                                    \
        switch (gemm_tiles(n_tokens)) {                                                         \
        case 1: return launch_gemm_batch<KB, 1>(b, z, max_wg, stream, start, stop, zero);        \
        case 2: return launch_gemm_batch<KB, 2>(b, z, max_wg, stream, start, stop, zero);        \
        default: return launch_gemm_batch<KB, 4>(b, z, max_wg, stream, start, stop, zero);       \
        }
    switch (bits) {
        DF11_GEMM_BATCH_CASE(10)
        DF11_GEMM_BATCH_CASE(11)
        DF11_GEMM_BATCH_CASE(12)
    default: return DF11_E_INVALID_ARG;
    }
#undef DF11_GEMM_BATCH_CASE
}

// The allocation-free batched decode's work counters: one set of
// DF11_SCHEDULE_WORDS words per stream of a call, in a file-scope device
// array that every call on a GPU shares (each GPU holds its own copy until
// the process ends).  Host code never uses the array's name as an address:
// its device address comes from hipGetSymbolAddress, once per device.
constexpr uint32_t kNoAllocWords = DF11_MAX_BATCH * DF11_SCHEDULE_WORDS;
static __device__ __align__(256) uint32_t scratch[kNoAllocWords];
constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device (looked up on the
// first call on each device, with that device current).
int scratch_address(uint32_t **ptr) {
    static std::mutex mu;
    static uint32_t *per_device[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DF11_E_HIP;
    std::lock_guard<std::mutex> lock(mu);
    if (!per_device[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DF11_E_HIP;
        per_device[dev] = static_cast<uint32_t *>(p);
    }
    *ptr = per_device[dev];
    return DF11_OK;
}

}  // namespace

extern "C" {

int df11_decompress_batch_noalloc(const df11_device_stream *streams, uint32_t n_streams, uint16_t *const *outs,
                                  void *hip_stream) {
    // (the counters hold n_streams * DF11_SCHEDULE_WORDS words at most kNoAllocWords)
    if (n_streams > kNoAllocWords / DF11_SCHEDULE_WORDS) return DF11_E_TOO_LARGE;
    if (n_streams && (!streams || !outs)) return DF11_E_INVALID_ARG;
    uint32_t *counters = nullptr;
    const int rc = scratch_address(&counters);
    if (rc) return rc;
    return decompress_batch_impl(streams, n_streams, outs, static_cast<hipStream_t>(hip_stream), nullptr, nullptr,
                                 counters);
}

int df11_decompress(const df11_device_stream *s, uint16_t *out, void *hip_stream) {
    return decompress_impl(s, out, static_cast<hipStream_t>(hip_stream), nullptr, nullptr);
}

int df11_decompress_block(const df11_device_stream *s, uint16_t *block_out, uint64_t scratch_elems,
                          void *hip_stream) {
    if (!s) return DF11_E_INVALID_ARG;
    if (scratch_elems < s->h.n_elements) return DF11_E_BUFFER_TOO_SMALL;
    return decompress_impl(s, block_out, static_cast<hipStream_t>(hip_stream), nullptr, nullptr);
}

int df11_decompress_batch(const df11_device_stream *streams, uint32_t n_streams, uint16_t *const *outs,
                          void *hip_stream) {
    return decompress_batch_impl(streams, n_streams, outs, static_cast<hipStream_t>(hip_stream), nullptr, nullptr);
}

int df11_decompress_batch_timed(const df11_device_stream *streams, uint32_t n_streams, uint16_t *const *outs,
                                void *hip_stream, void *start_event, void *stop_event) {
    return decompress_batch_impl(streams, n_streams, outs, static_cast<hipStream_t>(hip_stream),
                                 static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event));
}

int df11_decompress_timed(const df11_device_stream *s, uint16_t *out, void *hip_stream, void *start_event,
                          void *stop_event) {
    return decompress_impl(s, out, static_cast<hipStream_t>(hip_stream), static_cast<hipEvent_t>(start_event),
                           static_cast<hipEvent_t>(stop_event));
}

int df11_matmul(const df11_device_stream *w, const uint16_t *x, uint32_t n_tokens, uint32_t in_features,
                uint32_t out_features, float *y, void *hip_stream) {
    return gemm_impl(w, x, n_tokens, in_features, out_features, y, static_cast<hipStream_t>(hip_stream), nullptr,
                     nullptr, true);
}

int df11_matmul_acc(const df11_device_stream *w, const uint16_t *x, uint32_t n_tokens, uint32_t in_features,
                    uint32_t out_features, float *y, void *hip_stream) {
    return gemm_impl(w, x, n_tokens, in_features, out_features, y, static_cast<hipStream_t>(hip_stream), nullptr,
                     nullptr, false);
}

int df11_matmul_batch(const df11_device_stream *ws, uint32_t n_streams, const uint16_t *const *xs, uint32_t n_tokens,
                      const uint32_t *in_features, const uint32_t *out_features, float *const *ys, int accumulate,
                      void *hip_stream, void *start_event, void *stop_event) {
    return gemm_batch_impl(ws, n_streams, xs, n_tokens, in_features, out_features, ys,
                           static_cast<hipStream_t>(hip_stream), static_cast<hipEvent_t>(start_event),
                           static_cast<hipEvent_t>(stop_event), accumulate == 0);
}

int df11_matmul_timed(const df11_device_stream *w, const uint16_t *x, uint32_t n_tokens, uint32_t in_features,
                      uint32_t out_features, float *y, void *hip_stream, void *start_event, void *stop_event) {
    return gemm_impl(w, x, n_tokens, in_features, out_features, y, static_cast<hipStream_t>(hip_stream),
                     static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event), true);
}

int df11_linear(const df11_device_stream *w, const uint16_t *x, uint32_t n_tokens, uint32_t in_features,
                uint32_t out_features, float *y, void *hip_stream) {
    return linear_impl(w, x, n_tokens, in_features, out_features, y, static_cast<hipStream_t>(hip_stream), nullptr,
                       nullptr, true);
}

int df11_linear_acc(const df11_device_stream *w, const uint16_t *x, uint32_t n_tokens, uint32_t in_features,
                    uint32_t out_features, float *y, void *hip_stream) {
    return linear_impl(w, x, n_tokens, in_features, out_features, y, static_cast<hipStream_t>(hip_stream), nullptr,
                       nullptr, false);
}

int df11_linear_timed(const df11_device_stream *w, const uint16_t *x, uint32_t n_tokens, uint32_t in_features,
                      uint32_t out_features, float *y, void *hip_stream, void *start_event, void *stop_event) {
    return linear_impl(w, x, n_tokens, in_features, out_features, y, static_cast<hipStream_t>(hip_stream),
                       static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event), true);
}

int df11_linear_batch(const df11_device_stream *ws, uint32_t n_streams, const uint16_t *x, uint32_t n_tokens,
                      uint32_t in_features, const uint32_t *out_features, float *const *ys, void *hip_stream,
                      void *start_event, void *stop_event) {
    return linear_batch_impl(ws, n_streams, x, n_tokens, in_features, out_features, ys,
                             static_cast<hipStream_t>(hip_stream), static_cast<hipEvent_t>(start_event),
                             static_cast<hipEvent_t>(stop_event), true);
}

int df11_linear_batch_acc(const df11_device_stream *ws, uint32_t n_streams, const uint16_t *x, uint32_t n_tokens,
                          uint32_t in_features, const uint32_t *out_features, float *const *ys, void *hip_stream,
                          void *start_event, void *stop_event) {
    return linear_batch_impl(ws, n_streams, x, n_tokens, in_features, out_features, ys,
                             static_cast<hipStream_t>(hip_stream), static_cast<hipEvent_t>(start_event),
                             static_cast<hipEvent_t>(stop_event), false);
}

}  // extern "C"
