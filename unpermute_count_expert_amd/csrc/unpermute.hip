// unpermute.hip -- ep_gather unpermute with topk weight and reduce for gfx950
// (vLLM PR #20903 Purpose item 2 and bot Highlights; the weight-and-reduce
// inside the experts of vLLM PR #20725 Purpose), producing (M, K) directly.
//
// One wave per token.  Each lane owns 8 consecutive columns (16 bytes) of a
// 512-column slab; for each slab the token's expert rows are gathered in k
// order and folded with one fmaf per element, exactly in the order
// acc = fmaf(w_k, y_k, acc), k = 0..topk-1, then rounded once to bf16.
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
    const int64_t t = (int64_t)blockIdx.x * kTokensPerBlock + threadIdx.x / kWave;
    if (t >= Mc) return;
    const int32_t* rows = inv_perm + t * topk;   // wave-uniform: scalar loads
    const float* wts = topk_w + t * topk;
    for (int c0 = lane * 8; c0 < K; c0 += kWave * 8) {
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
        // eight of the token's rows at a time: all eight loads are issued
        // before the first use, then folded strictly in k order
        for (int k0 = 0; k0 < topk; k0 += 8) {
            uint4 v[8];
            bool ok[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int r = k0 + j < topk ? rows[k0 + j] : -1;
                ok[j] = r >= 0 && r < y_rows;
                v[j] = ok[j] ? *reinterpret_cast<const uint4*>(y + (int64_t)r * K + c0) : uint4{0, 0, 0, 0};
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (!ok[j]) continue;
                const float wk = apply_on_input ? 1.0f : wts[k0 + j];
                const uint32_t u[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = __builtin_fmaf(wk, __uint_as_float(u[i] << 16), acc[2 * i]);
                    acc[2 * i + 1] = __builtin_fmaf(wk, __uint_as_float(u[i] & 0xffff0000u), acc[2 * i + 1]);
                }
            }
        }
        uint4 o;
        o.x = f32x2_to_bf16x2(acc[0], acc[1]);
        o.y = f32x2_to_bf16x2(acc[2], acc[3]);
        o.z = f32x2_to_bf16x2(acc[4], acc[5]);
        o.w = f32x2_to_bf16x2(acc[6], acc[7]);
        *reinterpret_cast<uint4*>(out + t * K + c0) = o;
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
