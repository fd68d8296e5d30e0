// Device helpers and launch utilities shared by the gfx950 kernels (the
// DF11 decoder and fused product in df11_decode.hip, the rANS decoder in
// df11_rans_decode.hip).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include <stdint.h>

#include "df11.h"

namespace {

constexpr uint32_t kWaveSize = 64;

// A wave-uniform index into read-only memory through the constant address
// space gives scalar loads.
using ConstU32 = const __attribute__((address_space(4))) uint32_t;
using u32x4 = uint32_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t bitfield_insert(uint32_t mask, uint32_t a, uint32_t b) {
    return (mask & a) | (~mask & b);
}

// Merge 8 rotated exponents with 8 sign/mantissa bytes into 8 BF16 words.
// With r = exponent rotated right by one bit, a BF16 is
//   low byte  = (r & 0x80) | (sm & 0x7F),   high byte = (sm & 0x80) | (r & 0x7F),
// so two bitfield inserts give the low and high bytes of four outputs and two
// byte permutes interleave them.
__device__ __forceinline__ void merge4(uint32_t s4, uint32_t r4, uint32_t &out01, uint32_t &out23) {
    const uint32_t lo = bitfield_insert(0x7F7F7F7Fu, s4, r4);
    const uint32_t hi = bitfield_insert(0x80808080u, s4, r4);
    // v_perm byte selectors: 0..3 pick bytes of the second operand (lo), 4..7 of the first (hi).
    out01 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
    out23 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

__device__ __forceinline__ uint4 merge8(uint64_t sm8, uint64_t r8) {
    uint4 o;
    merge4(static_cast<uint32_t>(sm8), static_cast<uint32_t>(r8), o.x, o.y);
    merge4(static_cast<uint32_t>(sm8 >> 32), static_cast<uint32_t>(r8 >> 32), o.z, o.w);
    return o;
}

// Store chunk c (elements 8c .. 8c+7) restricted to [base, end).  Whole chunks
// are written with one 16-byte store that bypasses cache allocation: the BF16
// output is written once and read later by another kernel.
__device__ __forceinline__ void store_chunk(uint16_t *out, uint32_t c, uint4 v, uint32_t base, uint32_t end) {
    const uint32_t first = 8u * c;
    if (first >= base && first + 8u <= end) {
        u32x4 x = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(x, reinterpret_cast<u32x4 *>(out + first));
    } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (uint32_t i = 0; i < 8; ++i) {
            const uint32_t gi = first + i;
            if (gi >= base && gi < end) out[gi] = static_cast<uint16_t>(w[i >> 1] >> (16 * (i & 1)));
        }
    }
}

// store_chunk for a chunk whose 8 elements (stream positions first ..
// first + 7, kept where they lie in [base, end)) go to out[dst .. dst + 7]:
// a matrix stored in another order than the one it is written back in.
__device__ __forceinline__ void store_chunk_at(uint16_t *out, uint32_t dst, uint32_t first, uint4 v, uint32_t base,
                                               uint32_t end) {
    if (first >= base && first + 8u <= end) {
        u32x4 x = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(x, reinterpret_cast<u32x4 *>(out + dst));
    } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (uint32_t i = 0; i < 8; ++i) {
            const uint32_t gi = first + i;
            if (gi >= base && gi < end) out[dst + i] = static_cast<uint16_t>(w[i >> 1] >> (16 * (i & 1)));
        }
    }
}

uint64_t round_up(uint64_t x, uint64_t m) { return (x + m - 1) / m * m; }

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void *a, uint64_t an, const void *b, uint64_t bn) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return an && bn && a0 < b0 + bn && b0 < a0 + an;
}

// Workgroups of kernel fn (with `threads` threads and `lds` bytes of dynamic
// LDS) that fit on one CU of device dev, cached per (kernel, device, LDS).
int resident_per_cu(const void *fn, uint32_t threads, int dev, size_t lds) {
    struct Entry {
        const void *fn;
        int dev;
        size_t lds;
        int per_cu;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (const Entry &e : cache)
            if (e.fn == fn && e.dev == dev && e.lds == lds) return e.per_cu;
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (per_cu > 0 && cache.size() < 256) cache.push_back({fn, dev, lds, per_cu});
    return per_cu;
}

// Launch fn.  With both events null this is a plain hipLaunchKernel, which a
// caller may capture into a HIP graph; with either event given,
// hipExtLaunchKernel records it at the kernel's own start or end.
int launch_kernel(const void *fn, dim3 grid, dim3 block, void **params, size_t lds, hipStream_t stream,
                  hipEvent_t start, hipEvent_t stop) {
    const hipError_t e = (start || stop)
                             ? hipExtLaunchKernel(fn, grid, block, params, lds, stream, start, stop, 0)
                             : hipLaunchKernel(fn, grid, block, params, lds, stream);
    if (e != hipSuccess) return DF11_E_HIP;
    return hipGetLastError() == hipSuccess ? DF11_OK : DF11_E_HIP;
}

int device_cus(int &dev, int &cus) {
    if (hipGetDevice(&dev) != hipSuccess) return DF11_E_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return DF11_E_HIP;
    return DF11_OK;
}

}  // namespace
