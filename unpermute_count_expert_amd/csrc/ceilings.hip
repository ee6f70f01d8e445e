// ceilings.hip -- plain HBM streams on gfx950, timed beside the memory-bound
// kernels of the pipeline as their measured ceilings: a read of n bytes, a
// write of n bytes (non-temporal or ordinary 16-byte stores) and a copy.
// Every lane moves 16 bytes per access, eight accesses in flight, on a
// grid-stride walk over one 256-thread block per CU: a sweep of 1 to 32
// blocks per CU, 4 or 8 accesses in flight and contiguous per-block ranges
// put this shape at or near the top for all three streams (1 GiB: read
// ~7.2 TB/s, write ~6.6 TB/s, copy ~6.1 TB/s read + write).
#include "moe.h"
#include "moe_internal.hpp"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStreamThreads = 256;
constexpr int kUnroll = 8;

// MODE: 0 read, 1 non-temporal write, 2 copy, 3 ordinary write
template <int MODE>
__global__ __launch_bounds__(kStreamThreads) void k_stream(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                           int64_t n16, uint32_t* __restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
    int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    const u32x4 fill = {0x5A5A5A5Au, 0x5A5A5A5Au, 0x5A5A5A5Au, 0x5A5A5A5Au};
    for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
        u32x4 v[kUnroll];
        if constexpr (MODE == 0 || MODE == 2) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if constexpr (MODE == 0) acc ^= v[u];
            if constexpr (MODE == 1) __builtin_nontemporal_store(fill, dst + i + u * stride);
            if constexpr (MODE == 2) __builtin_nontemporal_store(v[u], dst + i + u * stride);
            if constexpr (MODE == 3) dst[i + u * stride] = fill;
        }
    }
    for (; i < n16; i += stride) {
        if constexpr (MODE == 0) acc ^= __builtin_nontemporal_load(src + i);
        if constexpr (MODE == 1) __builtin_nontemporal_store(fill, dst + i);
        if constexpr (MODE == 2) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
        if constexpr (MODE == 3) dst[i] = fill;
    }
    if constexpr (MODE == 0) {
        // keeps the loads live; the sink is written only if the xor of a
        // lane's data equals this constant
        const uint32_t h = acc.x ^ acc.y ^ acc.z ^ acc.w;
        if (h == 0x9E3779B9u) *sink = h;
    }
}

}  // namespace

hipError_t launch_stream(int mode, const void* src, void* dst, size_t bytes, uint32_t* sink, int num_cus,
                         hipStream_t s) {
    const int64_t n16 = (int64_t)(bytes / 16);
    const unsigned grid = (unsigned)num_cus;
    const u32x4* in = static_cast<const u32x4*>(src);
    u32x4* out = static_cast<u32x4*>(dst);
    switch (mode) {
        case MOE_STREAM_READ: k_stream<0><<<grid, kStreamThreads, 0, s>>>(in, out, n16, sink); break;
        case MOE_STREAM_WRITE_NT: k_stream<1><<<grid, kStreamThreads, 0, s>>>(in, out, n16, sink); break;
        case MOE_STREAM_COPY: k_stream<2><<<grid, kStreamThreads, 0, s>>>(in, out, n16, sink); break;
        default: k_stream<3><<<grid, kStreamThreads, 0, s>>>(in, out, n16, sink); break;
    }
    return hipGetLastError();
}

}  // namespace moe
