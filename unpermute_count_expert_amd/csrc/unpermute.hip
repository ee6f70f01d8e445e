// unpermute.hip -- ep_gather unpermute with topk weight and reduce for gfx950
// (vLLM PR #20903 Purpose item 2 and bot Highlights; the weight-and-reduce
// inside the experts of vLLM PR #20725 Purpose), producing (M, K) directly.
//
// One wave per token.  Each lane owns 8 consecutive columns (16 bytes) of a
// 512-column slab; for each slab the token's expert rows are gathered in k
// order and folded with one fmaf per element, exactly in the order
// acc = fmaf(w_k, y_k, acc), k = 0..topk-1, then rounded once to bf16.
// The row index of the token is wave-uniform, so indices and weights come
// through the scalar cache and the row loads of a slab issue back to back.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTokensPerBlock = kThreads / kWave;

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
    if (y_rows <= 0) {   // nothing to gather: the token's output is +0
        for (int c0 = lane * 8; c0 < K; c0 += kWave * 8)
            *reinterpret_cast<uint4*>(out + t * K + c0) = uint4{0, 0, 0, 0};
        return;
    }
    // passes of up to four 512-column slabs; each slab folds the token's rows
    // eight at a time (all eight loads issued before the first use, rows
    // outside y replaced by row 0 and skipped), and the pass stores its
    // slabs at the end.  With at most eight rows per token their indices and
    // weights are read once per token.
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
    for (int p0 = lane * 8; p0 < K; p0 += 4 * kWave * 8) {
        uint4 o[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            const int c0 = p0 + sb * kWave * 8;
            float acc[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
            if (c0 < K) {
                for (int k0 = 0; k0 < topk; k0 += 8) {
                    uint4 v[8];
                    bool ok[8];
                    float wk[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int r = few ? rr[j] : (k0 + j < topk ? rows[k0 + j] : -1);
                        wk[j] = few ? ww[j] : (apply_on_input ? 1.0f : (k0 + j < topk ? wts[k0 + j] : 0.0f));
                        ok[j] = r >= 0 && r < y_rows;
                        v[j] = *reinterpret_cast<const uint4*>(y + (int64_t)(ok[j] ? r : 0) * K + c0);
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        if (!ok[j]) continue;
                        const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            acc[2 * i] = __builtin_fmaf(wk[j], __uint_as_float(u[i] << 16), acc[2 * i]);
                            acc[2 * i + 1] = __builtin_fmaf(wk[j], __uint_as_float(u[i] & 0xffff0000u), acc[2 * i + 1]);
                        }
                    }
                }
            }
            o[sb].x = f32x2_to_bf16x2(acc[0], acc[1]);
            o[sb].y = f32x2_to_bf16x2(acc[2], acc[3]);
            o[sb].z = f32x2_to_bf16x2(acc[4], acc[5]);
            o[sb].w = f32x2_to_bf16x2(acc[6], acc[7]);
        }
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            const int c0 = p0 + sb * kWave * 8;
            if (c0 < K) *reinterpret_cast<uint4*>(out + t * K + c0) = o[sb];
        }
    }
}

}  // namespace

hipError_t launch_unpermute(const uint16_t* y, int64_t y_rows, const int32_t* inv_perm,
                            const float* topk_w, int64_t Mc, int K, int topk, int apply_on_input, uint16_t* out,
                            hipStream_t s) {
    if (Mc <= 0) return hipSuccess;
    const int64_t blocks = (Mc + kTokensPerBlock - 1) / kTokensPerBlock;
    k_unpermute<<<(unsigned)blocks, kThreads, 0, s>>>(y, inv_perm, topk_w, y_rows, Mc, K, topk, apply_on_input,
                                                      out);
    return hipGetLastError();
}

}  // namespace moe
