// gemm_fp8.hip -- block-scaled fp8 (OCP E4M3FN) grouped GEMM for gfx950 (the
// DeepGEMM grouped GEMM role in vLLM PR #20903: e4m3 operands, one fp32
// scale per 1x128 activation group and per 128x128 weight block).
//
//   out[r, n] = bf16( sum_g a_s[r,g] * w_s[e,n/128,g] * sum_{k in g} a[r,k] w[e,n,k] )
//
// Design:
//  * 128x256 output tile per 512-thread block: 8 waves in 2 (M) x 4 (N),
//    64x64 per wave = 4x4 MFMA 16x16x128 fp8 tiles, one block per CU.
//  * One MFMA spans exactly one K group, so each MFMA result is a whole
//    group's partial sum; it is scaled by a_s * w_s and folded into the fp32
//    accumulator with one FMA per output.  The group scales are arbitrary
//    fp32 values, so they cannot ride in the MFMA's power-of-two block-scale
//    operands; and the MFMA's own summation keeps only ~14 bits below the
//    largest product of each 8-wide K block, so promoting every 128 K to fp32
//    also bounds that error.  The per-row products a_s * w_s are formed once
//    per step when the scales are staged, and the MFMAs of row block i+1 are
//    issued before the promotion FMAs of row block i.
//  * K loop in 128-byte steps through a double-buffered LDS stage (48 KB):
//    the next step's A and B tiles (or the next tile's first step) are
//    fetched into registers while the MFMAs consume the current stage, then
//    written to the other stage; one barrier per step and no bubble between
//    tiles.
//  * LDS rows are 128 bytes, the 16-byte chunk c of row r stored at position
//    c ^ ((r ^ r/8) mod 8): the 16 lanes feeding one MFMA row block and the 16
//    lanes storing two global rows both touch 16 distinct bank groups
//    (measured on gfx950: no conflict cycles for either pattern).
//  * Weight rows are placed so that lane j of MFMA column block b holds output
//    column 4j + b: each lane owns 4 adjacent columns and the epilogue writes
//    8-byte bf16 quads straight from registers, 128 contiguous bytes per row.
//  * Rows past an expert's valid count are loaded as a copy of its last valid
//    row and never stored, so the K loop has no divergent branches; tiles
//    cover only valid rows, so alignment padding is never multiplied.
//  * Persistent grid with an XCD-aware tile order: workgroups are dealt to the
//    8 XCDs round-robin, so XCD x walks the contiguous x-th eighth of the
//    (expert, m-tile, n-tile) sequence and an expert's weights stay hot in
//    that XCD's L2.
//  * Row indices are clamped on the device, so even inconsistent
//    offsets/counts cannot move an access out of bounds.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int BM = 128;
constexpr int BN = 256;
constexpr int BK = 128;
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;   // 8: 2 along M, 4 along N
constexpr int kStageA = BM * BK;           // bytes
constexpr int kStage = kStageA + BN * BK;  // 48 KB

typedef int v2i __attribute__((ext_vector_type(2)));
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

// byte offset of 16-byte chunk c of LDS tile row r
__device__ __forceinline__ int swz(int c, int r) { return r * 128 + ((c ^ ((r ^ (r >> 3)) & 7)) << 4); }

// LDS row of weight row n of the tile: within each 64-row quarter, row 4j+b
// goes to 16b+j, so MFMA column j of column block b is weight row 4j+b
__device__ __forceinline__ int b_row(int n) { return (n & ~63) | ((n & 3) << 4) | ((n >> 2) & 15); }

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b) {
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    // cbsz = blgp = 0: both operands E4M3; zero scale operands select the
    // unscaled 16x16x128 f8f6f4 MFMA.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i frag(const uint8_t* p, int off_lo) {
    // the two 16-byte halves of a lane's 32 K-bytes: chunks 2h and 2h+1 sit
    // at positions x and x^1 of the same row
    const v4i lo = *reinterpret_cast<const v4i*>(p + off_lo);
    const v4i hi = *reinterpret_cast<const v4i*>(p + (off_lo ^ 16));
    return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

struct Tile {
    int e, m0, row_end, n0;
    bool valid;
};

__global__ __launch_bounds__(kThreads, 1) void k_grouped_gemm(
    const uint8_t* __restrict__ a, const float* __restrict__ a_s, const uint8_t* __restrict__ w,
    const float* __restrict__ w_s, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ counts, int El, int64_t cap_rows, int n_out, int k_in,
    uint16_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStage];
    __shared__ __attribute__((aligned(16))) float sSc[2][2][BM];   // [stage][128-col block][row]
    __shared__ int s_tpre[kMaxLocalExperts + 1];
    __shared__ int s_wsum[kWaves];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);

    // ---- m-tile prefix over the experts' valid row counts ------------------
    auto rows_of = [&](int e, int64_t& lo, int64_t& hi) {
        lo = offsets[e];
        lo = lo < 0 ? 0 : (lo > cap_rows ? cap_rows : lo);
        int64_t c = counts[e];
        c = c < 0 ? 0 : c;
        hi = lo + c > cap_rows ? cap_rows : lo + c;
    };
    int ntl[2];
    int tsum = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = tid * 2 + j;
        int nt = 0;
        if (e < El) {
            int64_t lo, hi;
            rows_of(e, lo, hi);
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
    for (int j = 0; j < 2; ++j) {
        const int e = tid * 2 + j;
        if (e < El) s_tpre[e] = excl;
        excl += ntl[j];
    }
    if (tid == kThreads - 1) s_tpre[El] = excl;
    __syncthreads();

    const int mtiles = s_tpre[El];
    const int ntn = (n_out + BN - 1) / BN;   // the last n-tile may hold only 128 columns
    const int nb128 = n_out / 128;
    const int kg = k_in / BK;
    const int64_t total = (int64_t)mtiles * ntn;
    const int xcd = blockIdx.x & 7;
    const int nslots = gridDim.x >> 3;
    const int64_t t_hi = total * (xcd + 1) / 8;
    int64_t t_cur = total * xcd / 8 + (blockIdx.x >> 3);

    auto tile_at = [&](int64_t t) {
        Tile T;
        T.valid = t < t_hi;
        if (!T.valid) {
            T.e = T.m0 = T.row_end = T.n0 = 0;
            return T;
        }
        const int tm = (int)(t / ntn);
        int lo = 0, hi = El - 1;  // largest e < El with s_tpre[e] <= tm
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_tpre[mid] <= tm) lo = mid; else hi = mid - 1;
        }
        T.e = __builtin_amdgcn_readfirstlane(lo);
        int64_t rlo, rhi;
        rows_of(T.e, rlo, rhi);
        T.m0 = __builtin_amdgcn_readfirstlane((int)rlo + (tm - s_tpre[T.e]) * BM);
        T.row_end = __builtin_amdgcn_readfirstlane((int)rhi);
        T.n0 = (int)(t - (int64_t)tm * ntn) * BN;
        return T;
    };

    const int wm = wave >> 2;   // 0..1
    const int wn = wave & 3;    // 0..3
    // global -> register assignment: chunk j = tid + 512*q, row j>>3, chunk j&7
    const int ld_r = tid >> 3;  // + 64*q
    const int ld_c = tid & 7;
    const int fr = lane & 15;
    const int fc = 2 * (lane >> 4);   // this lane's K chunk pair
    // per-lane LDS offsets (stage 0) of the fragments and of the stash slots
    int offA[4], offB[4], stA[2], stB[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        offA[i] = swz(fc, wm * 64 + i * 16 + fr);
        offB[i] = kStageA + swz(fc, wn * 64 + i * 16 + fr);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) stA[q] = swz(ld_c, ld_r + 64 * q);
#pragma unroll
    for (int q = 0; q < 4; ++q) stB[q] = kStageA + swz(ld_c, b_row(ld_r + 64 * q));
    const int sc_row = tid & (BM - 1);   // threads 0..255 stage one scale product
    const int sc_nb = (tid >> 7) & 1;

    v4i ra[2], rb[4];
    float ras = 0.0f, rws = 0.0f;
    auto fetch = [&](const Tile& T, int g) {
        const int last = T.row_end - 1 - T.m0;   // last valid row of the tile (>= 0)
        const int nlast = min(BN, n_out - T.n0) - 1;
        const uint8_t* abase = a + (int64_t)T.m0 * k_in + g * BK;
        const uint8_t* bbase = w + ((int64_t)T.e * n_out + T.n0) * k_in + g * BK;
#pragma unroll
        for (int q = 0; q < 2; ++q)
            ra[q] = *reinterpret_cast<const v4i*>(abase + (uint32_t)(min(ld_r + 64 * q, last) * k_in + ld_c * 16));
#pragma unroll
        for (int q = 0; q < 4; ++q)
            rb[q] = *reinterpret_cast<const v4i*>(bbase + (uint32_t)(min(ld_r + 64 * q, nlast) * k_in + ld_c * 16));
        // every thread loads (threads >= 256 duplicate 0..255 and never stash),
        // so there is no divergent branch, and the product is formed at stash
        // time: nothing in the compute waits on these loads
        ras = a_s[((int64_t)T.m0 + min(sc_row, last)) * kg + g];
        rws = w_s[((int64_t)T.e * nb128 + min(T.n0 / 128 + sc_nb, nb128 - 1)) * kg + g];
    };
    auto stash = [&](int stage) {
        uint8_t* base = smem + stage * kStage;
#pragma unroll
        for (int q = 0; q < 2; ++q) *reinterpret_cast<v4i*>(base + stA[q]) = ra[q];
#pragma unroll
        for (int q = 0; q < 4; ++q) *reinterpret_cast<v4i*>(base + stB[q]) = rb[q];
        if (tid < 2 * BM) sSc[stage][sc_nb][sc_row] = ras * rws;
    };

    Tile cur = tile_at(t_cur);
    if (cur.valid) {
        fetch(cur, 0);
        stash(0);
    }
    __syncthreads();
    int stage = 0;
    while (cur.valid) {
        const Tile nxt = tile_at(t_cur + nslots);
        const int n_valid = min(BN, n_out - cur.n0);
        const bool wave_has_rows = (cur.m0 + wm * 64) < cur.row_end && wn * 64 < n_valid;
        v4f acc[4][4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

        for (int g = 0; g < kg; ++g) {
            const bool more = (g + 1 < kg) || nxt.valid;
            if (g + 1 < kg) fetch(cur, g + 1);
            else if (nxt.valid) fetch(nxt, 0);
            if (wave_has_rows) {
                const uint8_t* base = smem + stage * kStage;
                const float* scs = &sSc[stage][wn >> 1][wm * 64 + (lane >> 4) * 4];
                v8i bf[4];
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) bf[ni] = frag(base, offB[ni]);
                // software-pipelined over the four row blocks: the MFMAs of
                // row block mi+1 are in flight while row block mi is promoted
                v4f p[2][4];
                {
                    const v8i af = frag(base, offA[0]);
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) p[0][ni] = mfma_fp8(af, bf[ni]);
                }
#pragma unroll
                for (int mi = 0; mi < 4; ++mi) {
                    if (mi + 1 < 4) {
                        const v8i af = frag(base, offA[mi + 1]);
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni) p[(mi + 1) & 1][ni] = mfma_fp8(af, bf[ni]);
                    }
                    const v4f sc = *reinterpret_cast<const v4f*>(scs + mi * 16);
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
                        const v4f pr = p[mi & 1][ni];
                        acc[mi][ni].x = __builtin_fmaf(sc.x, pr.x, acc[mi][ni].x);
                        acc[mi][ni].y = __builtin_fmaf(sc.y, pr.y, acc[mi][ni].y);
                        acc[mi][ni].z = __builtin_fmaf(sc.z, pr.z, acc[mi][ni].z);
                        acc[mi][ni].w = __builtin_fmaf(sc.w, pr.w, acc[mi][ni].w);
                    }
                }
            }
            if (more) stash(stage ^ 1);
            __syncthreads();
            stage ^= 1;
        }

        // ---- epilogue: each lane owns 4 adjacent columns of 16 rows --------
        if (wave_has_rows) {
            const int col = cur.n0 + wn * 64 + 4 * fr;
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int row = cur.m0 + wm * 64 + mi * 16 + (lane >> 4) * 4 + v;
                    if (row < cur.row_end) {
                        v2i q;
                        q.x = (int)((uint32_t)f32_to_bf16(acc[mi][0][v]) |
                                    ((uint32_t)f32_to_bf16(acc[mi][1][v]) << 16));
                        q.y = (int)((uint32_t)f32_to_bf16(acc[mi][2][v]) |
                                    ((uint32_t)f32_to_bf16(acc[mi][3][v]) << 16));
                        *reinterpret_cast<v2i*>(out + (int64_t)row * n_out + col) = q;
                    }
                }
        }
        cur = nxt;
        t_cur += nslots;
    }
}

}  // namespace

hipError_t launch_grouped_gemm(const uint8_t* a, const float* a_s, const uint8_t* w,
                               const float* w_s, const int32_t* offsets, const int32_t* counts,
                               int El, int64_t cap_rows, int n_out, int k_in, uint16_t* out,
                               int num_cus, hipStream_t s) {
    const int64_t ntn = (n_out + BN - 1) / BN;
    const int64_t bound = ((cap_rows + BM - 1) / BM + El) * ntn;
    int64_t grid = num_cus;            // one 8-wave block per CU (97 KB of LDS)
    if (bound < grid) grid = bound;
    grid = ((grid + 7) / 8) * 8;
    if (grid < 8) grid = 8;
    k_grouped_gemm<<<(unsigned)grid, kThreads, 0, s>>>(a, a_s, w, w_s, offsets, counts, El, cap_rows,
                                                        n_out, k_in, out);
    return hipGetLastError();
}

}  // namespace moe
