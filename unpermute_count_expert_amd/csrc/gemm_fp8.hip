// gemm_fp8.hip -- block-scaled fp8 (OCP E4M3FN) grouped GEMM for gfx950 (the
// DeepGEMM grouped GEMM role in vLLM PR #20903: e4m3 operands, one fp32
// scale per 1x128 activation group and per 128x128 weight block).
//
//   out[r, n] = bf16( sum_g a_s[r,g] * w_s[e,n/128,g] * sum_{k in g} a[r,k] w[e,n,k] )
//
// Design:
//  * 128x128 output tile per 256-thread block, 4 waves in 2x2, 64x64 per
//    wave = 4x4 MFMA 16x16x128 fp8 tiles.  One MFMA spans exactly one K
//    group, so each MFMA result is a whole group's partial sum: it is scaled
//    by a_s * w_s and folded into the fp32 accumulator with one FMA per
//    output (the group scales cannot be folded into the fp8 operands).
//  * K loop in 128-byte steps; A and B tiles staged through LDS with a
//    144-byte row pitch (conflict-free 16-byte fragment reads), the next step
//    prefetched into registers while the current one feeds the MFMAs.
//  * Tiles cover only valid rows of each expert segment (counts from the
//    device), so alignment padding is never multiplied.
//  * Persistent grid with an XCD-aware tile order: workgroups are dealt to
//    the 8 XCDs round-robin, so XCD x walks the contiguous x-th eighth of the
//    (expert, m-tile, n-tile) sequence and one expert's weights stay hot in
//    that XCD's L2.
//  * All row indices are clamped to [0, cap_rows) on the device, so even
//    inconsistent offsets/counts cannot move an access out of bounds.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 128;
constexpr int kThreads = 256;
constexpr int kPitch = BK + 16;  // LDS row pitch in bytes

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        int u = __shfl_up(v, d, kWave);
        if (lane >= d) v += u;
    }
    return v;
}

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b) {
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    // cbsz = blgp = 0: both operands E4M3; zero scale operands select the
    // unscaled 16x16x128 f8f6f4 MFMA.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

__global__ __launch_bounds__(kThreads, 2) void k_grouped_gemm(
    const uint8_t* __restrict__ a, const float* __restrict__ a_s, const uint8_t* __restrict__ w,
    const float* __restrict__ w_s, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ counts, int El, int64_t cap_rows, int n_out, int k_in,
    uint16_t* __restrict__ out) {
    __shared__ int s_tpre[kMaxLocalExperts + 1];
    __shared__ int s_lo[kMaxLocalExperts];
    __shared__ int s_hi[kMaxLocalExperts];
    __shared__ int s_wsum[kThreads / kWave];
    __shared__ __attribute__((aligned(16))) uint8_t sA[BM * kPitch];
    __shared__ __attribute__((aligned(16))) uint8_t sB[BN * kPitch];
    __shared__ __attribute__((aligned(16))) float sAs[BM];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;

    // ---- per-expert valid row ranges and the m-tile prefix --------------
    int ntl[4];
    int tsum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = tid * 4 + j;
        int nt = 0;
        if (e < El) {
            int64_t lo = offsets[e];
            lo = lo < 0 ? 0 : (lo > cap_rows ? cap_rows : lo);
            int64_t c = counts[e];
            c = c < 0 ? 0 : c;
            int64_t hi = lo + c;
            hi = hi > cap_rows ? cap_rows : hi;
            s_lo[e] = (int)lo;
            s_hi[e] = (int)hi;
            nt = (int)((hi - lo + BM - 1) / BM);
        }
        ntl[j] = nt;
        tsum += nt;
    }
    const int incl = wave_incl_scan(tsum);
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    int excl = incl - tsum;
    for (int w2 = 0; w2 < wave; ++w2) excl += s_wsum[w2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int e = tid * 4 + j;
        if (e < El) s_tpre[e] = excl;
        excl += ntl[j];
    }
    if (tid == kThreads - 1) s_tpre[El] = excl;
    __syncthreads();

    const int mtiles = s_tpre[El];
    const int ntn = n_out / BN;
    const int kg = k_in / BK;
    const int64_t total = (int64_t)mtiles * ntn;
    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    const int nslots = gridDim.x >> 3;
    const int64_t t_lo = total * xcd / 8;
    const int64_t t_hi = total * (xcd + 1) / 8;

    const int wm = wave >> 1;
    const int wn = wave & 1;
    // global -> register assignment: 4 x 16 bytes of A and of B per thread
    const int ld_row = tid >> 3;       // + 32 * q
    const int ld_col = (tid & 7) * 16;

    for (int64_t t = t_lo + slot; t < t_hi; t += nslots) {
        const int tm = (int)(t / ntn);
        const int tn = (int)(t - (int64_t)tm * ntn);
        int lo = 0, hi = El - 1;  // largest e < El with s_tpre[e] <= tm
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_tpre[mid] <= tm) lo = mid; else hi = mid - 1;
        }
        const int e = lo;
        const int m0 = s_lo[e] + (tm - s_tpre[e]) * BM;
        const int row_end = s_hi[e];
        const int n0 = tn * BN;
        const uint8_t* wbase = w + ((int64_t)e * n_out + n0) * k_in;
        const float* wsbase = w_s + ((int64_t)e * ntn + tn) * kg;

        v4i ra[4], rb[4];
        float ras = 0.0f;
        float sw_next = 0.0f;
        auto load_step = [&](int g) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = ld_row + 32 * q;
                const int ar = m0 + r;
                if (ar < row_end)
                    ra[q] = *reinterpret_cast<const v4i*>(a + (int64_t)ar * k_in + g * BK + ld_col);
                else
                    ra[q] = v4i{0, 0, 0, 0};
                rb[q] = *reinterpret_cast<const v4i*>(wbase + (int64_t)r * k_in + g * BK + ld_col);
            }
            if (tid < BM) {
                const int ar = m0 + tid;
                ras = ar < row_end ? a_s[(int64_t)ar * kg + g] : 0.0f;
            }
            sw_next = wsbase[g];
        };

        v4f acc[4][4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

        bool act[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) act[mi] = (m0 + wm * 64 + mi * 16) < row_end;

        load_step(0);
        for (int g = 0; g < kg; ++g) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = ld_row + 32 * q;
                *reinterpret_cast<v4i*>(sA + r * kPitch + ld_col) = ra[q];
                *reinterpret_cast<v4i*>(sB + r * kPitch + ld_col) = rb[q];
            }
            if (tid < BM) sAs[tid] = ras;
            const float sw = sw_next;
            __syncthreads();
            if (g + 1 < kg) load_step(g + 1);

            v8i bf[4];
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) {
                const uint8_t* p = sB + (wn * 64 + ni * 16 + (lane & 15)) * kPitch + (lane >> 4) * 32;
                const v4i lo4 = *reinterpret_cast<const v4i*>(p);
                const v4i hi4 = *reinterpret_cast<const v4i*>(p + 16);
                bf[ni] = v8i{lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
            }
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
                if (!act[mi]) continue;
                const uint8_t* p = sA + (wm * 64 + mi * 16 + (lane & 15)) * kPitch + (lane >> 4) * 32;
                const v4i lo4 = *reinterpret_cast<const v4i*>(p);
                const v4i hi4 = *reinterpret_cast<const v4i*>(p + 16);
                const v8i af = v8i{lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
                const v4f sa = *reinterpret_cast<const v4f*>(sAs + wm * 64 + mi * 16 + (lane >> 4) * 4);
                v4f sc;
                sc.x = sa.x * sw;
                sc.y = sa.y * sw;
                sc.z = sa.z * sw;
                sc.w = sa.w * sw;
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) {
                    const v4f pr = mfma_fp8(af, bf[ni]);
                    acc[mi][ni].x = __builtin_fmaf(sc.x, pr.x, acc[mi][ni].x);
                    acc[mi][ni].y = __builtin_fmaf(sc.y, pr.y, acc[mi][ni].y);
                    acc[mi][ni].z = __builtin_fmaf(sc.z, pr.z, acc[mi][ni].z);
                    acc[mi][ni].w = __builtin_fmaf(sc.w, pr.w, acc[mi][ni].w);
                }
            }
            __syncthreads();
        }

        // epilogue: lane holds rows 4*(lane/16)+v, column lane%16 of each 16x16 tile
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
            if (!act[mi]) continue;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = m0 + wm * 64 + mi * 16 + (lane >> 4) * 4 + v;
                if (row >= row_end) continue;
                uint16_t* orow = out + (int64_t)row * n_out + n0 + wn * 64 + (lane & 15);
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) orow[ni * 16] = f32_to_bf16(acc[mi][ni][v]);
            }
        }
    }
}

}  // namespace

hipError_t launch_grouped_gemm(const uint8_t* a, const float* a_s, const uint8_t* w,
                               const float* w_s, const int32_t* offsets, const int32_t* counts,
                               int El, int64_t cap_rows, int n_out, int k_in, uint16_t* out,
                               int num_cus, hipStream_t s) {
    const int64_t ntn = n_out / BN;
    const int64_t bound = ((cap_rows + BM - 1) / BM + El) * ntn;
    int64_t grid = (int64_t)num_cus * 2;
    if (bound < grid) grid = bound;
    grid = ((grid + 7) / 8) * 8;
    if (grid < 8) grid = 8;
    k_grouped_gemm<<<(unsigned)grid, kThreads, 0, s>>>(a, a_s, w, w_s, offsets, counts, El, cap_rows,
                                                        n_out, k_in, out);
    return hipGetLastError();
}

}  // namespace moe
