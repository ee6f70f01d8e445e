// unpermute.hip -- ep_gather unpermute with topk weight and reduce for gfx950
// (vLLM PR #20903 Purpose item 2 and bot Highlights; the weight-and-reduce
// inside the experts of vLLM PR #20725 Purpose), producing (M, K) directly.
//
// One wave per token (for few tokens, per token and slice of its columns).
// Each lane owns 8 consecutive columns (16 bytes) of a 512-column slab; for
// each slab the token's expert rows are gathered in k order and folded with
// one fmaf per element, exactly in the order
// acc = fmaf(w_k, y_k, acc), k = 0..topk-1, then rounded once to bf16.
// The row index of the token is wave-uniform, so indices and weights come
// through the scalar cache.  With topk <= 8 all the rows of a pass of four
// slabs (32 16-byte loads per lane) are issued before the first fold.  Every
// row of y is read exactly once and out is written once, so both go through
// non-temporal loads and stores that do not keep the lines in the caches
// (on the 16k-token layer: 0.126 -> 0.104 ms).
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTokensPerBlock = kThreads / kWave;
constexpr int kSlabs = 4;   // 512-column slabs per pass

// acc[0..7] = fmaf(w, each bf16 of v, acc) in column order
__device__ __forceinline__ void fold8(float (&acc)[8], float w, const uint4& v) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        acc[2 * i] = __builtin_fmaf(w, __uint_as_float(u[i] << 16), acc[2 * i]);
        acc[2 * i + 1] = __builtin_fmaf(w, __uint_as_float(u[i] & 0xffff0000u), acc[2 * i + 1]);
    }
}

__device__ __forceinline__ uint4 to_bf16x8(const float (&acc)[8]) {
    uint4 o;
    o.x = f32x2_to_bf16x2(acc[0], acc[1]);
    o.y = f32x2_to_bf16x2(acc[2], acc[3]);
    o.z = f32x2_to_bf16x2(acc[4], acc[5]);
    o.w = f32x2_to_bf16x2(acc[6], acc[7]);
    return o;
}

__global__ __launch_bounds__(kThreads) void k_unpermute(const uint16_t* __restrict__ y,
                                                        const int32_t* __restrict__ inv_perm,
                                                        const float* __restrict__ topk_w,
                                                        int64_t y_rows, int64_t Mc, int K,
                                                        int topk, int apply_on_input,
                                                        uint16_t* __restrict__ out) {
    const int lane = threadIdx.x & (kWave - 1);
    // wave-uniform token index, so its row indices and weights load through the scalar cache
    const int64_t t = (int64_t)blockIdx.x * kTokensPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (t >= Mc) return;
    const int32_t* rows = inv_perm + t * topk;
    const float* wts = topk_w + t * topk;
    // this wave's columns: slice blockIdx.y of the token's 512-column slabs
    const int nslab = (K + kWave * 8 - 1) / (kWave * 8);
    const int spw = (nslab + (int)gridDim.y - 1) / (int)gridDim.y;
    const int c_beg = min(K, (int)blockIdx.y * spw * kWave * 8);
    const int c_end = min(K, c_beg + spw * kWave * 8);
    if (y_rows <= 0) {   // nothing to gather: the token's output is +0
        for (int c0 = c_beg + lane * 8; c0 < c_end; c0 += kWave * 8)
            *reinterpret_cast<uint4*>(out + t * K + c0) = uint4{0, 0, 0, 0};
        return;
    }
    // With at most eight rows per token, their indices and weights are read
    // once per token, and each pass of four 512-column slabs loads all its
    // rows before folding them; beyond eight, each slab takes the rows eight
    // at a time.  Rows outside y are replaced by row 0 for the load and not
    // folded.
    const bool few = topk <= 8;
    int rr[8];
    float ww[8];
    if (few) {
        if (topk == 8) {   // 32 bytes at a 16-byte aligned address: two scalar loads each
            const int4 i0 = *reinterpret_cast<const int4*>(rows);
            const int4 i1 = *reinterpret_cast<const int4*>(rows + 4);
            rr[0] = i0.x; rr[1] = i0.y; rr[2] = i0.z; rr[3] = i0.w;
            rr[4] = i1.x; rr[5] = i1.y; rr[6] = i1.z; rr[7] = i1.w;
            if (!apply_on_input) {
                const float4 w0 = *reinterpret_cast<const float4*>(wts);
                const float4 w1 = *reinterpret_cast<const float4*>(wts + 4);
                ww[0] = w0.x; ww[1] = w0.y; ww[2] = w0.z; ww[3] = w0.w;
                ww[4] = w1.x; ww[5] = w1.y; ww[6] = w1.z; ww[7] = w1.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                rr[j] = j < topk ? rows[j] : -1;
                if (!apply_on_input) ww[j] = j < topk ? wts[j] : 0.0f;
            }
        }
        if (apply_on_input) {
#pragma unroll
            for (int j = 0; j < 8; ++j) ww[j] = 1.0f;
        }
    }
    if (few) {
        bool ok[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) ok[j] = rr[j] >= 0 && rr[j] < y_rows;
        for (int p0 = c_beg + lane * 8; p0 < c_end; p0 += kSlabs * kWave * 8) {
            // every row load of the pass first (rows outside y read row 0,
            // columns past K column 0, and are not folded)
            uint4 v[kSlabs][8];
#pragma unroll
            for (int sb = 0; sb < kSlabs; ++sb) {
                const int c0 = p0 + sb * kWave * 8;
                if (p0 - lane * 8 + sb * kWave * 8 < c_end) {   // the slab starts in the slice (wave-uniform)
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        v[sb][j] = load_once16(y + (int64_t)(ok[j] ? rr[j] : 0) * K + (c0 < c_end ? c0 : 0));
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) v[sb][j] = uint4{0, 0, 0, 0};
                }
            }
#pragma unroll
            for (int sb = 0; sb < kSlabs; ++sb) {
                const int c0 = p0 + sb * kWave * 8;
                float acc[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (ok[j]) fold8(acc, ww[j], v[sb][j]);
                if (c0 < c_end) store_once16(out + t * K + c0, to_bf16x8(acc));
            }
        }
        return;
    }
    // topk > 8: per slab, the rows eight at a time
    for (int c0 = c_beg + lane * 8; c0 < c_end; c0 += kWave * 8) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        for (int k0 = 0; k0 < topk; k0 += 8) {
            uint4 v[8];
            bool ok[8];
            float wk[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = k0 + j < topk ? rows[k0 + j] : -1;
                wk[j] = apply_on_input ? 1.0f : (k0 + j < topk ? wts[k0 + j] : 0.0f);
                ok[j] = r >= 0 && r < y_rows;
                v[j] = load_once16(y + (int64_t)(ok[j] ? r : 0) * K + c0);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (ok[j]) fold8(acc, wk[j], v[j]);
        }
        store_once16(out + t * K + c0, to_bf16x8(acc));
    }
}

// Before the down GEMM with the weight-and-reduce in its epilogue: one wave
// per token zeroes the token's (token, n-tile) counters and, when none of its
// topk rows is valid (no tile will complete it), writes its output row as +0.
__global__ __launch_bounds__(kThreads) void k_reduce_prep(const int32_t* __restrict__ inv_perm, int64_t Mc, int topk,
                                                          int64_t y_rows, int K, int32_t* __restrict__ cnt, int ntn,
                                                          uint16_t* __restrict__ out) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = (int64_t)blockIdx.x * kTokensPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (t >= Mc) return;
    for (int j = lane; j < ntn; j += kWave) cnt[t * ntn + j] = 0;
    bool any = false;
    for (int k = lane; k < topk; k += kWave) {
        const int r = inv_perm[t * topk + k];
        any |= r >= 0 && r < y_rows;
    }
    if (__ballot(any) == 0)
        for (int c0 = lane * 8; c0 < K; c0 += kWave * 8)
            *reinterpret_cast<uint4*>(out + t * K + c0) = uint4{0, 0, 0, 0};
}

}  // namespace

hipError_t launch_reduce_prep(const int32_t* inv_perm, int64_t Mc, int topk, int64_t y_rows, int K, int32_t* cnt,
                              uint16_t* out, hipStream_t s) {
    if (Mc <= 0) return hipSuccess;
    const int ntn = (K + 255) / 256;
    k_reduce_prep<<<(unsigned)((Mc + kTokensPerBlock - 1) / kTokensPerBlock), kThreads, 0, s>>>(
        inv_perm, Mc, topk, y_rows, K, cnt, ntn, out);
    return hipGetLastError();
}

hipError_t launch_unpermute(const uint16_t* y, int64_t y_rows, const int32_t* inv_perm,
                            const float* topk_w, int64_t Mc, int K, int topk, int apply_on_input, uint16_t* out,
                            hipStream_t s) {
    if (Mc <= 0) return hipSuccess;
    const int64_t blocks = (Mc + kTokensPerBlock - 1) / kTokensPerBlock;
    // few tokens: each token's 512-column slabs are split over up to four
    // waves (slices of grid.y), so that at least ~256 blocks take part
    const int64_t nslab = (K + kWave * 8 - 1) / (kWave * 8);
    int64_t ys = (256 + blocks - 1) / blocks;
    ys = ys < 1 ? 1 : (ys > 4 ? 4 : ys);
    ys = ys < nslab ? ys : nslab;
    const int64_t spw = (nslab + ys - 1) / ys;
    ys = (nslab + spw - 1) / spw;   // no empty slice
    k_unpermute<<<dim3((unsigned)blocks, (unsigned)ys), kThreads, 0, s>>>(y, inv_perm, topk_w, y_rows, Mc, K, topk,
                                                                        apply_on_input, out);
    return hipGetLastError();
}

}  // namespace moe
