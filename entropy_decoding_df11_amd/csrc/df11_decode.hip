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
// every complete code at the start of the window (up to six), so one lookup
// resolves several of the 2-3 bit codes that dominate LLM exponents.  A window
// whose first code is longer than K bits continues in the page's LUT hierarchy
// (256-entry LUTs, values 240..255 pointing to lower LUTs) and CodeLengths,
// which are also staged in LDS.
#include <hip/hip_runtime.h>

#include <algorithm>

#include <stdint.h>
#include <string.h>

#include "df11.h"
#include "df11_internal.h"

namespace {

using df11::kBytesPerThread;
using df11::kThreadsPerGroup;
constexpr uint32_t kWaveSize = 64;
constexpr uint32_t kWaves = kThreadsPerGroup / kWaveSize;
constexpr uint32_t kSegBits = 8 * kBytesPerThread;
constexpr int kPrefetchChunks = 4;  // 8-element sign/mantissa chunks held in registers per thread

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
    uint32_t ebuf_cap;  // bytes of the LDS exponent buffer, a multiple of 16
    uint32_t pad;
};

__device__ __forceinline__ uint32_t bswap32(uint32_t x) { return __builtin_amdgcn_perm(x, x, 0x00010203u); }

// Bits [p, p + 32) of the thread's 96-bit window, p < 64.  v0..v2 hold the
// window shifted right by one bit, so the funnel shift amount 31 - p (taken
// mod 32 by v_alignbit) stays in range for every p, including p = 0 and 32.
__device__ __forceinline__ uint32_t window_bits(uint32_t v0, uint32_t v1, uint32_t v2, uint32_t p) {
    const bool low = p < 32;
    const uint32_t x = low ? v0 : v1;
    const uint32_t y = low ? v1 : v2;
    return __builtin_amdgcn_alignbit(x, y, ~p);
}

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

__device__ __forceinline__ uint32_t bitfield_insert(uint32_t mask, uint32_t a, uint32_t b) {
    return (mask & a) | (~mask & b);
}

// Merge 8 rotated exponents with 8 sign/mantissa bytes into 8 BF16 words.
// With r = exponent rotated right by one bit, a BF16 is
//   low byte  = (r & 0x80) | (sm & 0x7F),   high byte = (sm & 0x80) | (r & 0x7F).
__device__ __forceinline__ uint4 merge8(uint64_t sm8, uint64_t r8) {
    const uint32_t s0 = static_cast<uint32_t>(sm8), s1 = static_cast<uint32_t>(sm8 >> 32);
    const uint32_t r0 = static_cast<uint32_t>(r8), r1 = static_cast<uint32_t>(r8 >> 32);
    constexpr uint32_t kFromSm = 0x807F807Fu;
    uint4 o;
    o.x = bitfield_insert(kFromSm, __builtin_amdgcn_perm(s0, s0, 0x01010000u), __builtin_amdgcn_perm(r0, r0, 0x01010000u));
    o.y = bitfield_insert(kFromSm, __builtin_amdgcn_perm(s0, s0, 0x03030202u), __builtin_amdgcn_perm(r0, r0, 0x03030202u));
    o.z = bitfield_insert(kFromSm, __builtin_amdgcn_perm(s1, s1, 0x01010000u), __builtin_amdgcn_perm(r1, r1, 0x01010000u));
    o.w = bitfield_insert(kFromSm, __builtin_amdgcn_perm(s1, s1, 0x03030202u), __builtin_amdgcn_perm(r1, r1, 0x03030202u));
    return o;
}

// Store chunk c (elements 8c .. 8c+7) restricted to [base, end).
__device__ __forceinline__ void store_chunk(uint16_t *out, uint32_t c, uint4 v, uint32_t base, uint32_t end) {
    const uint32_t first = 8u * c;
    if (first >= base && first + 8u <= end) {
        *reinterpret_cast<uint4 *>(out + first) = v;
    } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (uint32_t i = 0; i < 8; ++i) {
            const uint32_t gi = first + i;
            if (gi >= base && gi < end) out[gi] = static_cast<uint16_t>(w[i >> 1] >> (16 * (i & 1)));
        }
    }
}

template <int K>
__global__ __launch_bounds__(kThreadsPerGroup) void df11_decode_kernel(DecodeArgs a) {
    // Dynamic LDS: lo table | hi table | LUTs | CodeLengths | exponent buffer | wave sums.
    // The tables start at LDS address 0 so lookups need no base add.
    extern __shared__ __align__(16) uint8_t smem[];
    uint32_t *s_lo = reinterpret_cast<uint32_t *>(smem);
    uint32_t *s_hi = s_lo + (1u << K);
    uint8_t *s_luts = smem + (8u << K);
    uint8_t *s_clen = s_luts + a.n_luts * 256u;
    uint8_t *s_ebuf = s_clen + 256u;
    uint32_t *s_wsum = reinterpret_cast<uint32_t *>(s_ebuf + a.ebuf_cap);
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & (kWaveSize - 1);
    const uint32_t wave = tid / kWaveSize;

    // Stage the first-level table, the LUT hierarchy and CodeLengths.
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(a.dtab);
        uint4 *dst = reinterpret_cast<uint4 *>(smem);
        for (uint32_t i = tid; i < (8u << K) / 16u; i += kThreadsPerGroup) dst[i] = src[i];
        const uint32_t *l32 = reinterpret_cast<const uint32_t *>(a.luts);
        uint32_t *d32 = reinterpret_cast<uint32_t *>(s_luts);
        for (uint32_t i = tid; i < a.n_luts * 64u; i += kThreadsPerGroup) d32[i] = l32[i];
        if (tid < 64) reinterpret_cast<uint32_t *>(s_clen)[tid] = reinterpret_cast<const uint32_t *>(a.code_lengths)[tid];
    }
    __syncthreads();

    for (uint32_t g = blockIdx.x; g < a.n_groups; g += gridDim.x) {
        const uint32_t t = g * kThreadsPerGroup + tid;

        // Output range of the group, clamped so a corrupt out_pos stays in bounds.
        uint32_t end = min(a.out_pos[g + 1], a.n_elements);
        uint32_t base = min(a.out_pos[g], end);
        const uint32_t lead = base & 7u;
        const uint32_t c0 = base >> 3;
        uint32_t n_chunks = end > base ? ((end + 7u) >> 3) - c0 : 0u;
        n_chunks = min(n_chunks, a.ebuf_cap / 8u);

        uint64_t smv[kPrefetchChunks];
#pragma unroll
        for (int j = 0; j < kPrefetchChunks; ++j) {
            const uint32_t k = tid + j * kThreadsPerGroup;
            smv[j] = k < n_chunks ? *reinterpret_cast<const uint64_t *>(a.sm + 8ull * (c0 + k)) : 0ull;
        }

        uint32_t w0 = 0, w1 = 0, w2 = 0, gap = 0, seg_end = 0;
        if (t < a.n_threads) {
            const uint32_t *e32 = reinterpret_cast<const uint32_t *>(a.enc + 8ull * t);
            w0 = bswap32(e32[0]);
            w1 = bswap32(e32[1]);
            w2 = bswap32(e32[2]);
            const uint64_t gbit = 5ull * t;
            const uint32_t *g32 = reinterpret_cast<const uint32_t *>(a.gaps) + (gbit >> 5);
            const uint64_t gw = (static_cast<uint64_t>(bswap32(g32[0])) << 32) | bswap32(g32[1]);
            gap = static_cast<uint32_t>((gw << (gbit & 31)) >> 59);
            const uint64_t rem = a.total_bits - static_cast<uint64_t>(kSegBits) * t;
            seg_end = rem < kSegBits ? static_cast<uint32_t>(rem) : kSegBits;
        }
        const uint32_t v0 = w0 >> 1;
        const uint32_t v1 = __builtin_amdgcn_alignbit(w0, w1, 1);
        const uint32_t v2 = __builtin_amdgcn_alignbit(w1, w2, 1);

        // Phase 1: count the codes that start in [gap, seg_end).
        uint32_t cnt = 0, last_p = 0, last_mask = 0;
        for (uint32_t p = gap; p < seg_end;) {
            const uint32_t win = window_bits(v0, v1, v2, p);
            const uint32_t hi = s_hi[win >> (32 - K)];
            uint32_t nb = hi >> 28;
            uint32_t mask = (hi >> 16) & 0xFFFu;
            if (nb == 0) {
                uint32_t len;
                walk_luts(win, hi & 0xFFu, s_luts, s_clen, a.n_luts, len);
                nb = len;
                mask = 1;
            }
            last_p = p;
            last_mask = mask;
            cnt += __popc(mask);
            p += nb;
        }
        // The last lookup may list codes that start at or after seg_end.
        cnt -= __popc(last_mask >> min(seg_end - last_p, 31u));

        // Offsets within the group.
        const uint32_t incl = wave_inclusive_scan(cnt);
        if (lane == kWaveSize - 1) s_wsum[wave] = incl;
        __syncthreads();
        uint32_t wave_off = 0;
#pragma unroll
        for (uint32_t w = 0; w < kWaves - 1; ++w) wave_off += w < wave ? s_wsum[w] : 0u;
        uint32_t o = lead + wave_off + incl - cnt;
        const uint32_t e_end = min(o + cnt, a.ebuf_cap);

        // Phase 2: decode again and write the (rotated) exponents into LDS.
        for (uint32_t p = gap; o < e_end && p < seg_end;) {
            const uint32_t win = window_bits(v0, v1, v2, p);
            const uint32_t idx = win >> (32 - K);
            uint32_t lo = s_lo[idx];
            uint32_t hi = s_hi[idx];
            uint32_t nb = hi >> 28;
            uint32_t m = __popc((hi >> 16) & 0xFFFu);
            if (nb == 0) {
                uint32_t len;
                const uint32_t e = walk_luts(win, hi & 0xFFu, s_luts, s_clen, a.n_luts, len);
                lo = df11::rotate_exponent(e);
                hi = 0;
                nb = len;
                m = 1;
            }
            const uint64_t syms = static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi & 0xFFFFu) << 32);
            if (o + 8u <= e_end) {
                __builtin_memcpy(s_ebuf + o, &syms, 8);
            } else {
                // Near the end of this thread's range: write exactly the bytes that belong to it.
                const uint32_t k = min(m, e_end - o);
                uint32_t q = o;
                uint64_t rest = syms;
                if (k & 4u) {
                    const uint32_t v = static_cast<uint32_t>(rest);
                    __builtin_memcpy(s_ebuf + q, &v, 4);
                    q += 4;
                    rest >>= 32;
                }
                if (k & 2u) {
                    const uint16_t v = static_cast<uint16_t>(rest);
                    __builtin_memcpy(s_ebuf + q, &v, 2);
                    q += 2;
                    rest >>= 16;
                }
                if (k & 1u) s_ebuf[q] = static_cast<uint8_t>(rest);
            }
            o += m;
            p += nb;
        }
        __syncthreads();

        // Merge and store.  LDS byte 8k + i holds element 8 (c0 + k) + i.
#pragma unroll
        for (int j = 0; j < kPrefetchChunks; ++j) {
            const uint32_t k = tid + j * kThreadsPerGroup;
            if (k < n_chunks) {
                const uint64_t r8 = *reinterpret_cast<const uint64_t *>(s_ebuf + 8u * k);
                store_chunk(a.out, c0 + k, merge8(smv[j], r8), base, end);
            }
        }
        for (uint32_t k = tid + kPrefetchChunks * kThreadsPerGroup; k < n_chunks; k += kThreadsPerGroup) {
            const uint64_t s8 = *reinterpret_cast<const uint64_t *>(a.sm + 8ull * (c0 + k));
            const uint64_t r8 = *reinterpret_cast<const uint64_t *>(s_ebuf + 8u * k);
            store_chunk(a.out, c0 + k, merge8(s8, r8), base, end);
        }
        // The next group's scan barrier orders these LDS reads before its phase-2 writes.
    }
}

uint64_t round_up(uint64_t x, uint64_t m) { return (x + m - 1) / m * m; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void *a, uint64_t an, const void *b, uint64_t bn) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return an && bn && a0 < b0 + bn && b0 < a0 + an;
}

int validate(const df11_device_stream *s) {
    if (!s) return DF11_E_INVALID_ARG;
    const df11_header &h = s->h;
    if (h.bytes_per_thread != kBytesPerThread || h.threads_per_group != kThreadsPerGroup) return DF11_E_INVALID_ARG;
    if (h.n_elements >= (1ull << 32)) return DF11_E_TOO_LARGE;
    if (h.n_elements == 0) return h.total_bits == 0 ? DF11_OK : DF11_E_BAD_STREAM;
    if (df11_decode_table_bytes(s->decode_table_bits) == 0) return DF11_E_INVALID_ARG;
    if (!s->enc || !s->sm || !s->gaps || !s->out_pos || !s->luts || !s->code_lengths || !s->decode_table)
        return DF11_E_INVALID_ARG;
    if (!aligned(s->enc, 16) || !aligned(s->sm, 16) || !aligned(s->gaps, 4) || !aligned(s->out_pos, 4) ||
        !aligned(s->luts, 4) || !aligned(s->code_lengths, 4) || !aligned(s->decode_table, 16))
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
    return DF11_OK;
}

template <int K>
int launch(const DecodeArgs &a, hipStream_t stream) {
    const size_t lds = (8u << K) + a.n_luts * 256u + 256u + a.ebuf_cap + 4u * kWaves;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DF11_E_HIP;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return DF11_E_HIP;
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, df11_decode_kernel<K>, kThreadsPerGroup, lds) !=
            hipSuccess ||
        per_cu < 1)
        return DF11_E_HIP;
    const uint64_t resident = static_cast<uint64_t>(per_cu) * static_cast<uint64_t>(cus);
    const uint32_t grid = static_cast<uint32_t>(std::min<uint64_t>(a.n_groups, resident));
    (void)hipGetLastError();
    hipLaunchKernelGGL(df11_decode_kernel<K>, dim3(grid), dim3(kThreadsPerGroup), lds, stream, a);
    return hipGetLastError() == hipSuccess ? DF11_OK : DF11_E_HIP;
}

int decompress_impl(const df11_device_stream *s, uint16_t *out, hipStream_t stream) {
    int rc = validate(s);
    if (rc) return rc;
    const df11_header &h = s->h;
    if (h.n_elements == 0) return DF11_OK;
    if (!out || !aligned(out, 16)) return DF11_E_INVALID_ARG;
    const uint64_t out_bytes = 2 * h.n_elements;
    const uint32_t bits = s->decode_table_bits;
    if (overlaps(out, out_bytes, s->enc, h.enc_bytes) || overlaps(out, out_bytes, s->sm, h.sm_bytes) ||
        overlaps(out, out_bytes, s->gaps, h.gaps_bytes) || overlaps(out, out_bytes, s->out_pos, h.out_pos_bytes) ||
        overlaps(out, out_bytes, s->luts, 256ull * h.n_luts) || overlaps(out, out_bytes, s->code_lengths, 256) ||
        overlaps(out, out_bytes, s->decode_table, df11_decode_table_bytes(bits)))
        return DF11_E_INVALID_ARG;

    DecodeArgs a{};
    a.enc = s->enc;
    a.sm = s->sm;
    a.gaps = s->gaps;
    a.out_pos = s->out_pos;
    a.luts = s->luts;
    a.code_lengths = s->code_lengths;
    a.dtab = static_cast<const uint32_t *>(s->decode_table);
    a.out = out;
    a.total_bits = h.total_bits;
    a.n_elements = static_cast<uint32_t>(h.n_elements);
    a.n_threads = static_cast<uint32_t>(h.n_threads);
    a.n_groups = static_cast<uint32_t>(h.n_groups);
    a.n_luts = h.n_luts;
    // lead (< 8) + the group's elements, rounded up to whole 8-byte chunks, plus
    // slack for the 8-byte LDS writes.
    a.ebuf_cap = static_cast<uint32_t>(round_up(static_cast<uint64_t>(h.max_group_elems) + 16, 16));
    switch (bits) {
    case 10: return launch<10>(a, stream);
    case 11: return launch<11>(a, stream);
    case 12: return launch<12>(a, stream);
    default: return DF11_E_INVALID_ARG;
    }
}

}  // namespace

extern "C" {

int df11_decompress(const df11_device_stream *s, uint16_t *out, void *hip_stream) {
    return decompress_impl(s, out, static_cast<hipStream_t>(hip_stream));
}

int df11_decompress_block(const df11_device_stream *s, uint16_t *scratch, uint64_t scratch_elems, void *hip_stream) {
    if (!s) return DF11_E_INVALID_ARG;
    if (scratch_elems < s->h.n_elements) return DF11_E_BUFFER_TOO_SMALL;
    return decompress_impl(s, scratch, static_cast<hipStream_t>(hip_stream));
}

}  // extern "C"
