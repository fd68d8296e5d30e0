// gfx950 decoder of the rANS exponent coder and its C ABI entry points.
//
// The format is this library's reading of the rANS alternative that the
// discussion on "DFloat11: Kompresi inferensi GPU lossless yang mengecilkan
// LLM menjadi 70% ukurannya" (GeekNews), section "Opini Hacker News",
// mentions; it is described in df11.h.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>

#include <stdint.h>

#include "df11.h"
#include "df11_device.h"

namespace {

// ---------------------------------------------------------------------------
// rANS exponent decoder (format in df11.h; this library's reading of the
// rANS alternative named in the section "Opini Hacker News").
//
// One wave decodes one segment at a time, lane l keeping the state of the
// segment's lane l, so the output positions are fixed by the layout and no
// count or scan phase is needed.  A step decodes 64 consecutive exponents:
// each lane looks its slot up in the LDS slot table, updates its state, and
// the lanes whose state fell below 2^16 take the next words in lane order
// (ballot + mbcnt).  Steps run in sub-blocks of 8 (512 exponents), whose
// exponents go into a per-wave LDS stage; at the end of the pass they are
// merged with the sign/mantissa bytes into 16-byte BF16 stores.
//
// Words reach the steps through a per-wave LDS ring of four 512-word chunks
// (chunk c = words 512 c .. 512 c + 511, in ring slot c mod 4).  A sub-block
// uses at most 512 words, so one that starts in chunk c needs chunks c and
// c + 1, and the next one needs chunks up to c + 2: a pass starts by loading
// chunk c + 2 (and the sub-block's sign/mantissa chunk) into registers and,
// after its steps, writes it into the ring (slot (c + 2) mod 4 held chunk
// c - 2, no longer needed) and merges.  A pass's loads come before its
// stores and are waited for after its steps, so the step loop never waits for
// global memory, no wait for a load includes a store, and only a segment's
// first two chunks are loaded on the spot.  (No register holding a load in
// flight is copied across passes: a copy would wait for every load before it.)
// ---------------------------------------------------------------------------
constexpr uint32_t kRansLanes = DF11_RANS_LANES;
static_assert(kRansLanes == kWaveSize, "a segment's lanes are a wave's lanes");
constexpr uint32_t kRansSegment = DF11_RANS_LANES * DF11_RANS_STEPS;
// Steps per sub-block.  8 leaves 4.5 KB of LDS per wave (plus the 16 KB
// table per workgroup); 4 would fit more segments per CU but measured 18%
// slower (the per-pass loads, waits and merge come twice as often).
constexpr uint32_t kRansSub = 8;
constexpr uint32_t kRansSubElems = kRansSub * kRansLanes;    // exponents (and most words) per sub-block
constexpr uint32_t kRansChunk = kRansSubElems;               // words per ring chunk (8 per lane)
constexpr uint32_t kRansRing = 4 * kRansChunk;               // staged words per wave
static_assert(kRansChunk >= kRansSubElems, "a sub-block spans at most two chunks");
constexpr uint32_t kRansStateLow = 1u << 16;

struct RansArgs {
    const uint32_t *table;
    const uint32_t *states;
    const uint32_t *word_offsets;
    const uint16_t *words;
    const uint8_t *sm;
    uint16_t *out;
    uint32_t n_elements;
    uint32_t n_segments;
    uint32_t word_slots;  // readable words: n_words rounded up to 8, plus 8
    uint32_t sm_chunks;   // 8-byte chunks of the sign/mantissa buffer
};

static_assert(kRansChunk == 8 * kRansLanes, "a lane moves 8 words of a chunk");

// This lane's 8 words of word chunk c (clamped into the buffer).
__device__ __forceinline__ uint4 rans_chunk8(const RansArgs &a, uint32_t c, uint32_t lane) {
    const uint32_t i = min(c * kRansChunk + 8u * lane, a.word_slots - 8u);
    return *reinterpret_cast<const uint4 *>(a.words + i);
}

__device__ __forceinline__ void rans_ring_put(uint16_t *ring, uint32_t c, uint32_t lane, uint4 v) {
    *reinterpret_cast<uint4 *>(ring + (c & 3u) * kRansChunk + 8u * lane) = v;
}

// Each sign/mantissa byte is read once: a non-temporal load (the block
// decode took 155-156 us with it against 166).  The same hint on the word
// chunks as well took the block to 173 us and the stress stream from 205 to
// 243 us.
__device__ __forceinline__ uint64_t rans_sm8(const RansArgs &a, uint32_t c) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint64_t *>(a.sm + 8ull * min(c, a.sm_chunks - 1u)));
}

// Merge a decoded sub-block (rotated exponents in stage) with its
// sign/mantissa chunk and store elements [p0, p0 + len); lane l takes chunk l.
__device__ __forceinline__ void rans_merge(const RansArgs &a, const uint8_t *stage, uint64_t sm8, uint32_t p0,
                                           uint32_t len, uint32_t lane) {
    if (8u * lane < len) {
        const uint64_t r8 = *reinterpret_cast<const uint64_t *>(stage + 8u * lane);
        store_chunk(a.out, p0 / 8u + lane, merge8(sm8, r8), p0, p0 + len);
    }
}

// kRansSub decoding steps of one wave (see df11_rans_decode_kernel); kFull:
// every lane has a symbol in every step.  The next word is read by every
// lane whether or not its state needs one (the empty asm keeps the read
// unconditional, so the step has no branch); lanes that need none discard it.
template <bool kFull>
__device__ __forceinline__ void rans_steps(const uint32_t *s_tab, const uint16_t *ring, uint8_t *stage, uint32_t &x,
                                           uint32_t &ptr, uint32_t q0, uint32_t count, uint32_t lane) {
#pragma unroll
    for (uint32_t jj = 0; jj < kRansSub; ++jj) {
        const bool active = kFull || q0 + jj * kRansLanes + lane < count;
        const uint32_t e = s_tab[x & (DF11_RANS_TABLE_ENTRIES - 1u)];
        const uint32_t xs = x >> DF11_RANS_PROB_BITS;
        const uint32_t xn = ((e >> 8) & 0xFFFu) * xs + xs + (e >> 20);  // f * floor(x / M) + slot - c
        const bool need = active && xn < kRansStateLow;
        const uint64_t m = __builtin_amdgcn_ballot_w64(need);
        // ptr + (lanes below this one that need a word)
        const uint32_t k = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), ptr));
        uint32_t word = ring[k & (kRansRing - 1u)];
        asm volatile("" : "+v"(word));
        const uint32_t xr = (xn << 16) | word;
        x = need ? xr : (active ? xn : x);
        stage[jj * kRansLanes + lane] = static_cast<uint8_t>(active ? e : 0u);
        ptr += static_cast<uint32_t>(__builtin_popcountll(m));
    }
}

// W waves (segments in flight) per workgroup; the host picks W per stream
// (rans_waves).
template <uint32_t W>
__global__ __launch_bounds__(kWaveSize *W) void df11_rans_decode_kernel(RansArgs a) {
    constexpr uint32_t kRansWaves = W;
    __shared__ __align__(16) uint32_t s_tab[DF11_RANS_TABLE_ENTRIES];
    __shared__ __align__(16) uint8_t s_stage[kRansWaves][kRansSubElems];
    __shared__ __align__(16) uint16_t s_ring[kRansWaves][kRansRing];
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWaveSize - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / kWaveSize);
    {
        // Every load first, then every store; indices clamped (extra lanes
        // copy the last vector again).
        constexpr uint32_t kThreads = kWaveSize * kRansWaves;
        constexpr uint32_t kVecs = DF11_RANS_TABLE_ENTRIES / 4;
        constexpr uint32_t kPer = (kVecs + kThreads - 1) / kThreads;
        const uint4 *src = reinterpret_cast<const uint4 *>(a.table);
        uint4 v[kPer];
#pragma unroll
        for (uint32_t j = 0; j < kPer; ++j) v[j] = src[min(tid + j * kThreads, kVecs - 1u)];
#pragma unroll
        for (uint32_t j = 0; j < kPer; ++j) reinterpret_cast<uint4 *>(s_tab)[min(tid + j * kThreads, kVecs - 1u)] = v[j];
    }
    __syncthreads();
    const uint32_t stride = gridDim.x * kRansWaves;
    uint8_t *stage = s_stage[wave];
    uint16_t *ring = s_ring[wave];
    const ConstU32 *offs = (const ConstU32 *)a.word_offsets;  // scalar loads (wave-uniform index)

    for (uint32_t g = blockIdx.x * kRansWaves + wave; g < a.n_segments; g += stride) {
        const uint32_t seg0 = g * kRansSegment;
        const uint32_t count = min(kRansSegment, a.n_elements - seg0);
        uint32_t ptr = offs[g];  // next word (absolute index)
        uint32_t x = a.states[g * kRansLanes + lane];
        // The segment's first two chunks now; later ones a pass ahead.
        const uint32_t c0 = ptr / kRansChunk;
        rans_ring_put(ring, c0, lane, rans_chunk8(a, c0, lane));
        rans_ring_put(ring, c0 + 1u, lane, rans_chunk8(a, c0 + 1u, lane));
        // Everything issued so far (these chunks, the states) is complete:
        // the waits inside the passes then count only the passes' own loads.
        __builtin_amdgcn_s_waitcnt(0);
        for (uint32_t q0 = 0; q0 < count; q0 += kRansSubElems) {
            const uint32_t pf_c = ptr / kRansChunk + 2u;
            const uint4 pf = rans_chunk8(a, pf_c, lane);
            const uint64_t smv = rans_sm8(a, (seg0 + q0) / 8u + lane);
            if (q0 + kRansSubElems <= count)
                rans_steps<true>(s_tab, ring, stage, x, ptr, q0, count, lane);
            else
                rans_steps<false>(s_tab, ring, stage, x, ptr, q0, count, lane);
            rans_ring_put(ring, pf_c, lane, pf);
            rans_merge(a, stage, smv, seg0 + q0, min(kRansSubElems, count - q0), lane);
        }
    }
}

// Launch shape.  A CU decodes its resident segments at a throughput of
// about one per 6.5 us (block workload), but no round of segments takes less
// than the ~50 us that one segment's chain of steps needs alone: a round with
// fewer than ~8 segments per CU costs as much as one with 8.  The cost of
// W-wave workgroups, in units of one segment's CU time, is therefore the sum
// over rounds of max(8, segments on the busiest CU).  LDS bounds the
// workgroups per CU: three of 8 waves, two of 10 to 14 (24 to 28 segments
// per CU); the cheapest shape wins, the one with more waves on a tie.
struct RansShape {
    const void *fn;
    uint32_t waves;
    uint32_t grid;
};

template <uint32_t W>
void consider_shape(uint64_t n_seg, int dev, int cus, RansShape &best, uint64_t &best_cost) {
    const void *fn = reinterpret_cast<const void *>(&df11_rans_decode_kernel<W>);
    const int per_cu = resident_per_cu(fn, kWaveSize * W, dev, 0);
    if (per_cu < 1) return;
    const uint64_t grid = std::min<uint64_t>((n_seg + W - 1) / W, static_cast<uint64_t>(per_cu) * cus);
    const uint64_t slots = grid * W;
    uint64_t cost = 0;
    for (uint64_t done = 0; done < n_seg; done += slots) {
        const uint64_t in_round = std::min(slots, n_seg - done);
        const uint64_t wgs = (in_round + W - 1) / W;
        const uint64_t busiest = std::min<uint64_t>((wgs + cus - 1) / cus * W, in_round);
        cost += std::max<uint64_t>(8, busiest);
    }
    if (!best.fn || cost <= best_cost) {
        best = RansShape{fn, W, static_cast<uint32_t>(grid)};
        best_cost = cost;
    }
}

RansShape rans_shape(uint64_t n_seg, int dev, int cus) {
    RansShape best{nullptr, 0, 0};
    uint64_t cost = 0;
    consider_shape<8>(n_seg, dev, cus, best, cost);
    consider_shape<10>(n_seg, dev, cus, best, cost);
    consider_shape<11>(n_seg, dev, cus, best, cost);
    consider_shape<12>(n_seg, dev, cus, best, cost);
    consider_shape<13>(n_seg, dev, cus, best, cost);
    consider_shape<14>(n_seg, dev, cus, best, cost);
    return best;
}

int rans_impl(const df11_rans_device_stream *s, uint16_t *out, hipStream_t stream, hipEvent_t start,
              hipEvent_t stop) {
    if (!s) return DF11_E_INVALID_ARG;
    const df11_rans_header &h = s->h;
    if (h.prob_bits != DF11_RANS_PROB_BITS || h.lanes != DF11_RANS_LANES || h.steps != DF11_RANS_STEPS)
        return DF11_E_INVALID_ARG;
    if (h.n_elements > DF11_MAX_ELEMENTS) return DF11_E_TOO_LARGE;
    if (h.n_segments != (h.n_elements + kRansSegment - 1) / kRansSegment || h.n_words > h.n_elements)
        return DF11_E_BAD_STREAM;
    if (h.n_elements == 0) return DF11_OK;
    if (!out || !s->table || !s->states || !s->word_offsets || !s->words || !s->sm) return DF11_E_INVALID_ARG;
    if (!aligned(out, 16) || !aligned(s->table, 16) || !aligned(s->states, 4) || !aligned(s->word_offsets, 4) ||
        !aligned(s->words, 16) || !aligned(s->sm, 16))
        return DF11_E_INVALID_ARG;
    const uint64_t slots = round_up(h.n_words, 8) + 8, sm_bytes = round_up(h.n_elements, 64);
    const uint64_t out_bytes = 2 * h.n_elements;
    if (overlaps(out, out_bytes, s->table, 4ull * DF11_RANS_TABLE_ENTRIES) ||
        overlaps(out, out_bytes, s->states, 4ull * kRansLanes * h.n_segments) ||
        overlaps(out, out_bytes, s->word_offsets, 4ull * (h.n_segments + 1)) ||
        overlaps(out, out_bytes, s->words, 2 * slots) || overlaps(out, out_bytes, s->sm, sm_bytes))
        return DF11_E_INVALID_ARG;
    RansArgs a{};
    a.table = s->table;
    a.states = s->states;
    a.word_offsets = s->word_offsets;
    a.words = s->words;
    a.sm = s->sm;
    a.out = out;
    a.n_elements = static_cast<uint32_t>(h.n_elements);
    a.n_segments = static_cast<uint32_t>(h.n_segments);
    a.word_slots = static_cast<uint32_t>(slots);
    a.sm_chunks = static_cast<uint32_t>(sm_bytes / 8);
    int dev = 0, cus = 0;
    if (device_cus(dev, cus)) return DF11_E_HIP;
    const RansShape shape = rans_shape(h.n_segments, dev, cus);
    if (!shape.fn) return DF11_E_HIP;
    (void)hipGetLastError();
    void *params[] = {&a};
    return launch_kernel(shape.fn, dim3(shape.grid), dim3(kWaveSize * shape.waves), params, 0, stream, start, stop);
}

}  // namespace

extern "C" {

int df11_rans_decompress(const df11_rans_device_stream *s, uint16_t *out, void *hip_stream) {
    return rans_impl(s, out, static_cast<hipStream_t>(hip_stream), nullptr, nullptr);
}

int df11_rans_decompress_timed(const df11_rans_device_stream *s, uint16_t *out, void *hip_stream, void *start_event,
                               void *stop_event) {
    return rans_impl(s, out, static_cast<hipStream_t>(hip_stream), static_cast<hipEvent_t>(start_event),
                     static_cast<hipEvent_t>(stop_event));
}

}  // extern "C"
