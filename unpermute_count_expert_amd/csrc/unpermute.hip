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

// The same gather, weight and reduce with y as the K-split down GEMM leaves
// it: S = min(info[0], smax) slabs of fp32 partial sums [part_rows, K],
// rows at their place in the valid-row sequence (experts in order).  Each
// gathered row is first summed over the slabs in slab order and rounded to
// bf16, the y value the whole-K GEMM would store, then folded as above, so
// the output bits follow from those y bits exactly as in k_unpermute.  Row r
// of expert e (offsets[e] <= r < offsets[e] + counts[e]) has place
// vpre[e] + r - offsets[e]; an index that is no expert's valid row is not
// folded.  Lane j finds the place of the token's pair k0 + j (a search of
// the experts' first rows in LDS), and the rows are then gathered four pairs
// at a time, every slab load of the four issued before the first add.
constexpr int kPartPairs = 4;

template <int S>
__device__ __forceinline__ void fold_part_rows(float (&acc)[8], const float* __restrict__ part, int64_t slab,
                                               int K, int c0, const int64_t (&vr)[kPartPairs],
                                               const float (&wk)[kPartPairs]) {
    uint4 v[kPartPairs][S][2];
#pragma unroll
    for (int j = 0; j < kPartPairs; ++j) {
        const float* p = part + (vr[j] >= 0 ? vr[j] : 0) * K + c0;   // row 0 stands in, unfolded
#pragma unroll
        for (int sg = 0; sg < S; ++sg) {
            v[j][sg][0] = load_once16(p + sg * slab);
            v[j][sg][1] = load_once16(p + sg * slab + 4);
        }
    }
#pragma unroll
    for (int j = 0; j < kPartPairs; ++j) {
        if (vr[j] < 0) continue;   // wave-uniform
        float ys[8];
#pragma unroll
        for (int sg = 0; sg < S; ++sg) {
            const uint32_t pv[8] = {v[j][sg][0].x, v[j][sg][0].y, v[j][sg][0].z, v[j][sg][0].w,
                                    v[j][sg][1].x, v[j][sg][1].y, v[j][sg][1].z, v[j][sg][1].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) ys[i] = sg == 0 ? __uint_as_float(pv[i]) : ys[i] + __uint_as_float(pv[i]);
        }
        fold8(acc, wk[j], to_bf16x8(ys));
    }
}

__global__ __launch_bounds__(kThreads) void k_unpermute_part(const float* __restrict__ part,
                                                             const int32_t* __restrict__ info, int64_t part_rows,
                                                             int smax, const int32_t* __restrict__ offsets,
                                                             const int32_t* __restrict__ counts, int El,
                                                             const int32_t* __restrict__ inv_perm,
                                                             const float* __restrict__ topk_w, int64_t y_rows,
                                                             int64_t Mc, int K, int topk, int apply_on_input,
                                                             uint16_t* __restrict__ out) {
    __shared__ int s_lo[kMaxLocalExperts];
    __shared__ int s_cnt[kMaxLocalExperts];
    __shared__ int64_t s_vpre[kMaxLocalExperts];
    __shared__ int64_t s_wsum[kThreads / kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    {
        // valid rows per expert (clamped as the GEMM clamps them) and their
        // exclusive scan; four experts per thread covers El <= 1024
        int64_t v[4], tsum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = threadIdx.x * 4 + j;
            v[j] = 0;
            if (e < El) {
                const int64_t lo = min((int64_t)max(offsets[e], 0), y_rows);
                const int64_t hi = min(lo + (int64_t)max(counts[e], 0), y_rows);
                s_lo[e] = (int)lo;
                s_cnt[e] = (int)(hi - lo);
                v[j] = hi - lo;
            }
            tsum += v[j];
        }
        const int64_t incl = wave_inclusive_scan(tsum);
        if (lane == kWave - 1) s_wsum[wave] = incl;
        __syncthreads();
        int64_t run = incl - tsum;
        for (int w = 0; w < wave; ++w) run += s_wsum[w];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = threadIdx.x * 4 + j;
            if (e < El) s_vpre[e] = run;
            run += v[j];
        }
        __syncthreads();
    }
    const int64_t t = (int64_t)blockIdx.x * kTokensPerBlock + __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    if (t >= Mc) return;
    int nseg = min(max(info[0], 1), smax);
    nseg = nseg > 8 ? 8 : nseg;
    const int nslab = (K + kWave * 8 - 1) / (kWave * 8);
    const int spw = (nslab + (int)gridDim.y - 1) / (int)gridDim.y;
    const int c_beg = min(K, (int)blockIdx.y * spw * kWave * 8);
    const int c_end = min(K, c_beg + spw * kWave * 8);
    const int64_t slab = part_rows * (int64_t)K;
    for (int cw = c_beg; cw < c_end; cw += kWave * 8) {   // wave-uniform column pass
        const int c0 = cw + lane * 8;
        const bool in_cols = c0 < c_end;
        const int c_ld = in_cols ? c0 : c_beg;   // lanes past the slice load in-slice columns, store nothing
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
        for (int k0 = 0; k0 < topk; k0 += kWave) {
            // lane j: the place of pair k0 + j (-1: not folded) and its weight
            int64_t my_vr = -1;
            float my_w = 0.0f;
            const int k = k0 + lane;
            if (k < topk) {
                const int r = inv_perm[t * topk + k];
                if (r >= 0 && r < y_rows) {
                    int lo = 0, hi = El - 1;   // the last e with s_lo[e] <= r
                    while (lo < hi) {
                        const int mid = (lo + hi + 1) >> 1;
                        if (s_lo[mid] <= r) lo = mid; else hi = mid - 1;
                    }
                    const int d = r - s_lo[lo];
                    const int64_t vrow = s_vpre[lo] + d;
                    if (d >= 0 && d < s_cnt[lo] && vrow < part_rows) my_vr = vrow;
                }
                my_w = apply_on_input ? 1.0f : topk_w[t * topk + k];
            }
            const int kn = min(kWave, topk - k0);
            for (int kb = 0; kb < kn; kb += kPartPairs) {
                int64_t vr[kPartPairs];
                float wk[kPartPairs];
#pragma unroll
                for (int j = 0; j < kPartPairs; ++j) {
                    const int src = kb + j < kn ? kb + j : 0;
                    const int64_t x = __shfl(my_vr, src, kWave);
                    vr[j] = kb + j < kn ? x : -1;
                    wk[j] = __shfl(my_w, src, kWave);
                }
                switch (nseg) {
                    case 1: fold_part_rows<1>(acc, part, slab, K, c_ld, vr, wk); break;
                    case 2: fold_part_rows<2>(acc, part, slab, K, c_ld, vr, wk); break;
                    case 3: fold_part_rows<3>(acc, part, slab, K, c_ld, vr, wk); break;
                    case 4: fold_part_rows<4>(acc, part, slab, K, c_ld, vr, wk); break;
                    case 5: fold_part_rows<5>(acc, part, slab, K, c_ld, vr, wk); break;
                    case 6: fold_part_rows<6>(acc, part, slab, K, c_ld, vr, wk); break;
                    case 7: fold_part_rows<7>(acc, part, slab, K, c_ld, vr, wk); break;
                    default: fold_part_rows<8>(acc, part, slab, K, c_ld, vr, wk); break;
                }
            }
        }
        if (in_cols) store_once16(out + t * K + c0, to_bf16x8(acc));
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

hipError_t launch_unpermute_part(const float* part, const int32_t* info, int64_t part_rows, int smax,
                                 const int32_t* offsets, const int32_t* counts, int El, int64_t y_rows,
                                 const int32_t* inv_perm, const float* topk_w, int64_t Mc, int K, int topk,
                                 int apply_on_input, uint16_t* out, hipStream_t s) {
    if (Mc <= 0) return hipSuccess;
    const int64_t blocks = (Mc + kTokensPerBlock - 1) / kTokensPerBlock;
    const int64_t nslab = (K + kWave * 8 - 1) / (kWave * 8);
    int64_t ys = (256 + blocks - 1) / blocks;
    ys = ys < 1 ? 1 : (ys > 4 ? 4 : ys);
    ys = ys < nslab ? ys : nslab;
    const int64_t spw = (nslab + ys - 1) / ys;
    ys = (nslab + spw - 1) / spw;
    k_unpermute_part<<<dim3((unsigned)blocks, (unsigned)ys), kThreads, 0, s>>>(
        part, info, part_rows, smax, offsets, counts, El, inv_perm, topk_w, y_rows, Mc, K, topk, apply_on_input, out);
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
