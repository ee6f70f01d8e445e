// act_quant.hip -- per-token 1x128-group fp8 (OCP E4M3FN) quantisation on
// gfx950: the input activations before the permute (fp8 block-128 tokens and
// scales of vLLM PR #20903, Optimizations) and SiLU-and-mul + requant between
// the two grouped GEMMs.
//
// Sixteen lanes own one group (8 bf16 = 16 bytes each, fully coalesced); the
// group amax is a DPP maximum over the 16 lanes; codes leave as one 8-byte
// store per lane.  Compiled without FMA contraction so each operation
// below is the IEEE operation written.
//
// SiLU of a bf16 gate value is a function of 16 bits, so each block first
// tabulates silu(g) = g / (1 + exp(-g)) in LDS, with the same pinned exp and
// IEEE division, for every g with 2^-12 <= |g| < 2^8 (5120 values, 20 KB),
// and then looks the gate values up; the few others (zeros, tiny and huge
// values, infinities, NaN) take the formula itself.  The table holds the
// formula's own results, so the codes are the same bit for bit, and the
// kernel no longer spends ~40 VALU instructions per element on it.
//
// The input rows are read once and the codes written once, with
// non-temporal loads and stores.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerGroup = 16;
constexpr int kGroupsPerBlock = kThreads / kLanesPerGroup;


struct Vals8 {
    float v[8];
};

__device__ __forceinline__ Vals8 unpack_bf16x8(uint4 u) {
    Vals8 r;
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r.v[2 * i] = __uint_as_float(w[i] << 16);
        r.v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
    return r;
}

// The gate/up input as the K-split GEMM leaves it: S = min(info[0], smax)
// slabs of fp32 partial sums [part_rows, 2n], rows at their place in the
// valid-row sequence; h is their sum in slab order, rounded to bf16.
struct PartIn {
    const float* part;
    const int32_t* info;
    int64_t part_rows;
    int smax;
};

// gs / us[0..7] = the sums, in slab order, of S slabs' 8 gate values at g and
// 8 up values at g + up; every load is issued before the first add
template <int S>
__device__ __forceinline__ void sum_slabs(const float* g, int64_t slab, int64_t up, float (&gs)[8], float (&us)[8]) {
    uint4 v[S][4];
#pragma unroll
    for (int sg = 0; sg < S; ++sg) {
        v[sg][0] = load_once16(g + sg * slab);
        v[sg][1] = load_once16(g + sg * slab + 4);
        v[sg][2] = load_once16(g + sg * slab + up);
        v[sg][3] = load_once16(g + sg * slab + up + 4);
    }
#pragma unroll
    for (int sg = 0; sg < S; ++sg) {
        const uint32_t gv[8] = {v[sg][0].x, v[sg][0].y, v[sg][0].z, v[sg][0].w,
                                v[sg][1].x, v[sg][1].y, v[sg][1].z, v[sg][1].w};
        const uint32_t uv[8] = {v[sg][2].x, v[sg][2].y, v[sg][2].z, v[sg][2].w,
                                v[sg][3].x, v[sg][3].y, v[sg][3].z, v[sg][3].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            gs[i] = sg == 0 ? __uint_as_float(gv[i]) : gs[i] + __uint_as_float(gv[i]);
            us[i] = sg == 0 ? __uint_as_float(uv[i]) : us[i] + __uint_as_float(uv[i]);
        }
    }
}

// MODE: identity or SiLU-mul; TABLE (SiLU-mul only): SiLU from the LDS table.
// With offsets (masked), the rows are expert slots: the valid rows of expert
// e are [offsets[e], offsets[e] + counts[e]), cut at the next slot and at
// rows; only those are read and written.  The work is the sequence of the
// valid rows' groups, so padding rows cost nothing.  PART (SiLU-mul, masked):
// the gate/up values come from the split GEMM's partial sums (pi) instead
// of in.
template <int MODE, bool TABLE, bool PART = false>
__global__ __launch_bounds__(kThreads) void k_act_quant(const uint16_t* __restrict__ in, int64_t rows,
                                                        int n, const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ counts, int El,
                                                        uint8_t* __restrict__ q,
                                                        float* __restrict__ q_s, PartIn pi) {
    static_assert(!PART || MODE == MOE_ACT_SILU_MUL_K, "partial sums feed the SiLU-mul only");
    __shared__ int s_off[kMaxLocalExperts];        // first row of each expert's slot
    // valid rows of the experts before e, in 64 bits: slots that overlap
    // (inconsistent offsets) may add up to more than 2^31 rows
    __shared__ int64_t s_vpre[kMaxLocalExperts + 1];
    __shared__ int64_t s_wsum[kThreads / kWave];
    __shared__ float s_silu[TABLE ? kSiluEntries : 1];
    const bool masked = offsets != nullptr;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    if (masked) {
        // valid rows per expert (clamped to the slot and to [0, rows)), then
        // their exclusive scan; four experts per thread covers El <= 1024
        int64_t v[4], tsum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = threadIdx.x * 4 + j;
            v[j] = 0;
            if (e < El) {
                const int64_t lo = min((int64_t)max(offsets[e], 0), rows);
                int64_t hi = min(lo + (int64_t)max(counts[e], 0), rows);
                hi = min(hi, max((int64_t)offsets[e + 1], lo));   // offsets has El + 1 entries
                s_off[e] = (int)lo;
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
        if (threadIdx.x == kThreads - 1) s_vpre[El] = run;
    }
    if (TABLE) silu_table_build(s_silu);
    __syncthreads();
    int nseg = 1;
    if constexpr (PART) {
        const int v = pi.info[0];
        nseg = v < 1 ? 1 : (v > pi.smax ? pi.smax : v);
        nseg = nseg > 8 ? 8 : nseg;
    }
    const int ng = n / kGroup;
    const int64_t nrows = masked ? s_vpre[El] : rows;   // rows of the work sequence
    const int64_t total = nrows * ng;
    const int sub = threadIdx.x & (kLanesPerGroup - 1);
    // each block takes a contiguous range of groups, 16 at a time, so a
    // thread's rows advance slowly and the expert found for one row is
    // reused for the next ones
    const int64_t per_block = ((total + gridDim.x - 1) / gridDim.x + kGroupsPerBlock - 1) / kGroupsPerBlock *
                              kGroupsPerBlock;
    const int64_t g_lo = (int64_t)blockIdx.x * per_block;
    const int64_t g_hi = g_lo + per_block < total ? g_lo + per_block : total;
    // masked: valid rows [seg_lo, seg_hi) of the sequence belong to one
    // expert, whose slot starts at row seg_lo + seg_shift
    int64_t seg_lo = 0, seg_hi = -1, seg_shift = 0;
    // (row, group in row) of this thread's group, advanced by 16 groups per
    // iteration without a division
    int64_t grp = g_lo + threadIdx.x / kLanesPerGroup;
    int64_t r = grp / ng;
    int gi = (int)(grp - r * ng);
    const int adv_r = kGroupsPerBlock / ng, adv_g = kGroupsPerBlock % ng;
    for (; grp < g_hi; grp += kGroupsPerBlock) {
        int64_t r_this = r;
        const int gi_this = gi;
        gi += adv_g;
        r += adv_r;
        if (gi >= ng) {
            gi -= ng;
            ++r;
        }
        const int64_t r_seq = r_this;   // place in the valid-row sequence
        if (masked) {
            if (r_this < seg_lo || r_this >= seg_hi) {
                // the expert of valid row r_this: largest e < El with s_vpre[e] <= r_this
                int lo = 0, hi = El - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (s_vpre[mid] <= r_this) lo = mid; else hi = mid - 1;
                }
                seg_lo = s_vpre[lo];
                seg_hi = s_vpre[lo + 1];
                seg_shift = (int64_t)s_off[lo] - seg_lo;
            }
            r_this += seg_shift;
        }
        Vals8 x;
        if (MODE == MOE_ACT_IDENTITY_K) {
            const uint4 u = load_once16(in + r_this * n + gi_this * kGroup + sub * 8);
            x = unpack_bf16x8(u);
        } else {
            uint4 gw;
            Vals8 u;
            if constexpr (PART) {
                // h = bf16(sum of the partials in slab order); a row past the
                // slabs (only with inconsistent counts) reads as zero
                float gs[8], us[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) gs[i] = us[i] = 0.0f;
                if (r_seq < pi.part_rows) {
                    const float* p0 = pi.part + r_seq * 2 * (int64_t)n + gi_this * kGroup + sub * 8;
                    const int64_t slab = pi.part_rows * 2 * (int64_t)n;
                    switch (nseg) {   // uniform; the partial buffer holds up to 8 slabs
                        case 1: sum_slabs<1>(p0, slab, n, gs, us); break;
                        case 2: sum_slabs<2>(p0, slab, n, gs, us); break;
                        case 3: sum_slabs<3>(p0, slab, n, gs, us); break;
                        case 4: sum_slabs<4>(p0, slab, n, gs, us); break;
                        case 5: sum_slabs<5>(p0, slab, n, gs, us); break;
                        case 6: sum_slabs<6>(p0, slab, n, gs, us); break;
                        case 7: sum_slabs<7>(p0, slab, n, gs, us); break;
                        default: sum_slabs<8>(p0, slab, n, gs, us); break;
                    }
                }
                gw.x = f32x2_to_bf16x2(gs[0], gs[1]);
                gw.y = f32x2_to_bf16x2(gs[2], gs[3]);
                gw.z = f32x2_to_bf16x2(gs[4], gs[5]);
                gw.w = f32x2_to_bf16x2(gs[6], gs[7]);
                u = unpack_bf16x8(uint4{f32x2_to_bf16x2(us[0], us[1]), f32x2_to_bf16x2(us[2], us[3]),
                                        f32x2_to_bf16x2(us[4], us[5]), f32x2_to_bf16x2(us[6], us[7])});
            } else {
                const uint16_t* base = in + r_this * 2 * (int64_t)n + gi_this * kGroup + sub * 8;
                gw = load_once16(base);
                u = unpack_bf16x8(load_once16(base + n));
            }
            const uint32_t gbits[4] = {gw.x, gw.y, gw.z, gw.w};
            float prod[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (TABLE) {
                    prod[2 * i] = silu_bf16(s_silu, gbits[i] & 0xffffu) * u.v[2 * i];
                    prod[2 * i + 1] = silu_bf16(s_silu, gbits[i] >> 16) * u.v[2 * i + 1];
                } else {
                    prod[2 * i] = silu_pinned(__uint_as_float(gbits[i] << 16)) * u.v[2 * i];
                    prod[2 * i + 1] = silu_pinned(__uint_as_float(gbits[i] & 0xffff0000u)) * u.v[2 * i + 1];
                }
            }
            // the activation is rounded to bf16 before it is quantised
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const uint32_t pk = f32x2_to_bf16x2(prod[i], prod[i + 1]);
                x.v[i] = __uint_as_float(pk << 16);
                x.v[i + 1] = __uint_as_float(pk & 0xffff0000u);
            }
        }
        uint2 codes;
        const float scale = quant_group16(x.v, codes);
        store_once8(q + r_this * n + gi_this * kGroup + sub * 8, codes);
        if (sub == 0) q_s[r_this * ng + gi_this] = scale;
    }
}

}  // namespace

hipError_t launch_act_quant(const uint16_t* in, int64_t rows, int n, int mode,
                            const int32_t* offsets, const int32_t* counts, int El, uint8_t* q,
                            float* q_s, int64_t rows_hint, hipStream_t s) {
    const int64_t groups = rows * (n / kGroup);
    if (groups <= 0) return hipSuccess;
    // masked, the kernel walks the valid rows only, of which there are at
    // most rows_hint
    const int64_t work_rows = offsets && rows_hint < rows ? (rows_hint > 1 ? rows_hint : 1) : rows;
    int64_t blocks = (work_rows * (n / kGroup) + kGroupsPerBlock - 1) / kGroupsPerBlock;
    if (mode == MOE_ACT_IDENTITY_K) {
        if (blocks > 8192) blocks = 8192;
        k_act_quant<MOE_ACT_IDENTITY_K, false><<<(unsigned)blocks, kThreads, 0, s>>>(in, rows, n, offsets, counts,
                                                                                    El, q, q_s, PartIn{});
    } else if ((rows_hint < rows ? rows_hint : rows) * (n / kGroup) >= (int64_t)1024 * 64) {
        // enough valid rows for 1024 blocks of >= 64 groups each: every block
        // builds the SiLU table (as costly as ~90 groups) and then looks up
        if (blocks > 1024) blocks = 1024;
        k_act_quant<MOE_ACT_SILU_MUL_K, true><<<(unsigned)blocks, kThreads, 0, s>>>(in, rows, n, offsets, counts,
                                                                                   El, q, q_s, PartIn{});
    } else {
        if (blocks > 8192) blocks = 8192;
        k_act_quant<MOE_ACT_SILU_MUL_K, false><<<(unsigned)blocks, kThreads, 0, s>>>(in, rows, n, offsets, counts,
                                                                                    El, q, q_s, PartIn{});
    }
    return hipGetLastError();
}

hipError_t launch_act_quant_part(const float* part, const int32_t* info, int64_t part_rows, int smax, int64_t rows,
                                 int n, const int32_t* offsets, const int32_t* counts, int El, uint8_t* q, float* q_s,
                                 int64_t rows_hint, hipStream_t s) {
    const int64_t work_rows = rows_hint < rows ? (rows_hint > 1 ? rows_hint : 1) : rows;
    int64_t blocks = (work_rows * (n / kGroup) + kGroupsPerBlock - 1) / kGroupsPerBlock;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 8192) blocks = 8192;
    k_act_quant<MOE_ACT_SILU_MUL_K, false, true><<<(unsigned)blocks, kThreads, 0, s>>>(
        nullptr, rows, n, offsets, counts, El, q, q_s, PartIn{part, info, part_rows, smax});
    return hipGetLastError();
}

}  // namespace moe
