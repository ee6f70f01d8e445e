// count_permute.hip -- expert counting and the stable expert-contiguous permute
// (count_expert_num_tokens of vLLM PR #20392 and the ep_scatter permute of
// vLLM PR #20903), written for gfx950.
//
// Permute runs in three launches:
//   hist    one block per 256 (token, k) pairs: per-block expert histogram
//   scan    one block: counts, aligned offsets, per-block row bases, padding
//   scatter one block per 256 pairs: wave-ballot ranks (stable in flat pair
//           order), inverse indices, then each token row is read once and
//           written to each of its expert rows with 16-byte lanes.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kPermThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / kWave;

__global__ void k_fill_i32(int32_t* __restrict__ p, int64_t n, int32_t v) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

__global__ __launch_bounds__(256) void k_count(const int32_t* __restrict__ ids, int64_t num_pairs,
                                               const int32_t* __restrict__ emap, int Eg, int El,
                                               int32_t* __restrict__ counts,
                                               int32_t* __restrict__ invalid) {
    __shared__ int h[kMaxLocalExperts];
    __shared__ int bad;
    for (int e = threadIdx.x; e < El; e += blockDim.x) h[e] = 0;
    if (threadIdx.x == 0) bad = 0;
    __syncthreads();
    int my_bad = 0;
    for (int64_t f = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; f < num_pairs;
         f += (int64_t)gridDim.x * blockDim.x) {
        int id = ids[f];
        int e = local_expert(id, emap, Eg, El);
        if (e >= 0) atomicAdd(&h[e], 1);
        my_bad += (id < -1 || id >= Eg) ? 1 : 0;
    }
    if (my_bad) atomicAdd(&bad, my_bad);
    __syncthreads();
    for (int e = threadIdx.x; e < El; e += blockDim.x)
        if (h[e]) atomicAdd(&counts[e], h[e]);
    if (threadIdx.x == 0 && invalid && bad) atomicAdd(invalid, bad);
}

// Per-block histogram of local experts over the block's (token, k) pairs.
__global__ __launch_bounds__(kPermThreads) void k_permute_hist(const int32_t* __restrict__ ids,
                                                               int64_t Mc, int topk, int tpb,
                                                               const int32_t* __restrict__ emap,
                                                               int Eg, int El,
                                                               int32_t* __restrict__ hist) {
    __shared__ int h[kMaxLocalExperts];
    for (int e = threadIdx.x; e < El; e += blockDim.x) h[e] = 0;
    __syncthreads();
    const int64_t t0 = (int64_t)blockIdx.x * tpb;
    const int64_t ntok = (Mc - t0) < tpb ? (Mc - t0) : tpb;
    const int npairs = (int)ntok * topk;
    const int i = threadIdx.x;
    if (i < npairs) {
        int e = local_expert(ids[t0 * topk + i], emap, Eg, El);
        if (e >= 0) atomicAdd(&h[e], 1);
    }
    __syncthreads();
    int32_t* row = hist + (int64_t)blockIdx.x * El;
    for (int e = threadIdx.x; e < El; e += blockDim.x) row[e] = h[e];
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int u = __shfl_up(v, d, kWave);
        if (lane >= d) v += u;
    }
    return v;
}

// Column scan of hist [nblk, El]: counts, aligned offsets and, in place, the
// first row of each expert's segment that block b fills.  Also marks padding
// rows and rows past the last segment with row_src = -1.
__global__ __launch_bounds__(kScanThreads) void k_permute_scan(
    int32_t* __restrict__ hist, int nblk, int El, int align, int64_t cap_rows,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ row_src,
    int32_t* __restrict__ counts_copy) {
    __shared__ int band[kScanWaves][kWave];
    __shared__ int s_off[kMaxLocalExperts + 1];
    __shared__ int s_cnt[kMaxLocalExperts];
    __shared__ int running;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int per_band = (nblk + kScanWaves - 1) / kScanWaves;
    const int b_lo = wave * per_band;
    const int b_hi = min(nblk, b_lo + per_band);
    if (threadIdx.x == 0) running = 0;
    __syncthreads();
    for (int c0 = 0; c0 < El; c0 += kWave) {
        const int col = c0 + lane;
        const bool valid = col < El;
        int sum = 0;
        if (valid) {
            // independent loads, eight in flight per lane
#pragma unroll 8
            for (int b = b_lo; b < b_hi; ++b) sum += hist[(int64_t)b * El + col];
        }
        band[wave][lane] = sum;
        __syncthreads();
        if (wave == 0) {
            int acc = 0;
            for (int w = 0; w < kScanWaves; ++w) {
                int t = band[w][lane];
                band[w][lane] = acc;
                acc += t;
            }
            const int cnt = valid ? acc : 0;
            const int seg = ((cnt + align - 1) / align) * align;
            const int incl = wave_inclusive_scan(seg);
            const int base = running;
            const int off = base + incl - seg;
            if (valid) {
                s_off[col] = off;
                s_cnt[col] = cnt;
                counts[col] = cnt;
                offsets[col] = off;
                if (counts_copy) counts_copy[col] = cnt;
            }
            const int total = __shfl(incl, kWave - 1, kWave);
            if (lane == 0) running = base + total;
        }
        __syncthreads();
        if (valid) {
            int base = s_off[col] + band[wave][lane];
#pragma unroll 8
            for (int b = b_lo; b < b_hi; ++b) {
                int64_t idx = (int64_t)b * El + col;
                int t = hist[idx];
                hist[idx] = base;
                base += t;
            }
        }
        __syncthreads();
    }
    const int R = running;
    if (threadIdx.x == 0) offsets[El] = R;
    s_off[El] = R;  // every thread writes the same value; read after the barrier
    __syncthreads();
    for (int e = threadIdx.x; e < El; e += blockDim.x)
        for (int r = s_off[e] + s_cnt[e]; r < s_off[e + 1]; ++r) row_src[r] = -1;
    for (int64_t r = R + threadIdx.x; r < cap_rows; r += blockDim.x) row_src[r] = -1;
}

// Stable rank of every local pair, inverse indices, then the row copies.
__global__ __launch_bounds__(kPermThreads) void k_permute_scatter(
    const uint8_t* __restrict__ a_q, const float* __restrict__ a_s, const int32_t* __restrict__ ids,
    const float* __restrict__ topk_w, int apply_on_input, int64_t Mc, int K, int topk, int tpb,
    const int32_t* __restrict__ emap, int Eg, int El, int nbits, const int32_t* __restrict__ base,
    uint8_t* __restrict__ a_perm, float* __restrict__ a_perm_s, int32_t* __restrict__ inv_perm,
    int32_t* __restrict__ row_src) {
    constexpr int kWaves = kPermThreads / kWave;
    __shared__ int wcnt[kWaves][kMaxLocalExperts];
    __shared__ int rowmap[kPermThreads];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    for (int j = threadIdx.x; j < kWaves * El; j += blockDim.x) wcnt[j / El][j % El] = 0;

    const int64_t t0 = (int64_t)blockIdx.x * tpb;
    const int ntok = (int)((Mc - t0) < tpb ? (Mc - t0) : tpb);
    const int npairs = ntok * topk;
    const int i = threadIdx.x;
    const bool active = i < npairs;
    const int64_t f = t0 * topk + i;
    const int e = active ? local_expert(ids[f], emap, Eg, El) : -1;

    // lanes of this wave with the same expert (multisplit over the id bits)
    uint64_t peers = ballot(e >= 0);
    for (int bit = 0; bit < nbits; ++bit) {
        const bool b = (e >> bit) & 1;
        const uint64_t m = ballot(b);
        peers &= b ? m : ~m;
    }
    const int rank_w = __popcll(peers & lanemask_lt());
    __syncthreads();  // wcnt zeroed
    if (e >= 0 && rank_w == 0) wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    int row = -1;
    if (e >= 0) {
        int pre = 0;
        for (int w = 0; w < wave; ++w) pre += wcnt[w][e];
        row = base[(int64_t)blockIdx.x * El + e] + pre + rank_w;
    }
    if (active) {
        inv_perm[f] = row;
        rowmap[i] = row;
        if (row >= 0) row_src[row] = (int32_t)(t0 + i / topk);
    }
    __syncthreads();

    // copies: each wave takes every fourth token of the block; a lane reads
    // 16-byte chunks of the token rows, up to kBatch of them in flight at
    // once, and writes each to the token's expert rows
    constexpr int kBatch = 8;
    const int kg = K / kGroup;
    const int nchunk = K / 16;
    const int cpl = (nchunk + kWave - 1) / kWave;        // chunks per lane per token
    const int my_tokens = ntok > wave ? (ntok - wave + kWaves - 1) / kWaves : 0;
    const int items = my_tokens * cpl;
    for (int q0 = 0; q0 < items; q0 += kBatch) {
        uint4 v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int q = q0 + u;
            const int tl = wave + (q / cpl) * kWaves;
            const int c = lane + (q % cpl) * kWave;
            v[u] = uint4{0, 0, 0, 0};
            if (q < items && c < nchunk)
                v[u] = *reinterpret_cast<const uint4*>(a_q + (t0 + tl) * K + (int64_t)c * 16);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int q = q0 + u;
            const int tl = wave + (q / cpl) * kWaves;
            const int c = lane + (q % cpl) * kWave;
            if (q < items && c < nchunk) {
                const int* rm = rowmap + tl * topk;
                for (int k = 0; k < topk; ++k) {
                    const int r = rm[k];
                    if (r >= 0) *reinterpret_cast<uint4*>(a_perm + (int64_t)r * K + (int64_t)c * 16) = v[u];
                }
            }
        }
    }
    for (int tl = wave; tl < ntok; tl += kWaves) {
        const int64_t t = t0 + tl;
        const int* rm = rowmap + tl * topk;
        for (int g = lane; g < kg; g += kWave) {
            const float s = a_s[t * kg + g];
            for (int k = 0; k < topk; ++k) {
                const int r = rm[k];
                if (r >= 0) a_perm_s[(int64_t)r * kg + g] = apply_on_input ? s * topk_w[t * topk + k] : s;
            }
        }
    }
}

int bits_for(int El) {
    int b = 0;
    while ((1 << b) < El) ++b;
    return b;
}

}  // namespace

hipError_t launch_count(const int32_t* ids, int64_t num_pairs, const int32_t* emap, int Eg, int El,
                        int32_t* counts, int32_t* invalid, hipStream_t s) {
    k_fill_i32<<<1, 256, 0, s>>>(counts, El, 0);
    if (invalid) k_fill_i32<<<1, 64, 0, s>>>(invalid, 1, 0);
    if (num_pairs > 0) {
        int64_t blocks = (num_pairs + 256 * 8 - 1) / (256 * 8);
        if (blocks > 2048) blocks = 2048;
        k_count<<<(unsigned)blocks, 256, 0, s>>>(ids, num_pairs, emap, Eg, El, counts, invalid);
    }
    return hipGetLastError();
}

hipError_t launch_permute(const uint8_t* a_q, const float* a_s, const int32_t* ids,
                          const float* topk_w, int apply_on_input, int64_t Mc, int K, int topk,
                          const int32_t* emap, int Eg, int El, int align, int64_t cap_rows,
                          uint8_t* a_perm, float* a_perm_s, int32_t* counts, int32_t* offsets,
                          int32_t* inv_perm, int32_t* row_src, int32_t* hist,
                          int32_t* counts_copy, hipStream_t s) {
    const int tpb = permute_tokens_per_block(topk);
    const int64_t nblk = permute_num_blocks(Mc, topk);
    if (nblk > 0)
        k_permute_hist<<<(unsigned)nblk, kPermThreads, 0, s>>>(ids, Mc, topk, tpb, emap, Eg, El, hist);
    k_permute_scan<<<1, kScanThreads, 0, s>>>(hist, (int)nblk, El, align, cap_rows, counts, offsets,
                                              row_src, counts_copy);
    if (nblk > 0)
        k_permute_scatter<<<(unsigned)nblk, kPermThreads, 0, s>>>(
            a_q, a_s, ids, topk_w, apply_on_input, Mc, K, topk, tpb, emap, Eg, El, bits_for(El), hist,
            a_perm, a_perm_s, inv_perm, row_src);
    return hipGetLastError();
}

}  // namespace moe
