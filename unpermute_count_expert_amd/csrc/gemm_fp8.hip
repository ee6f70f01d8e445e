// gemm_fp8.hip -- block-scaled fp8 (OCP E4M3FN) grouped GEMM for gfx950 (the
// DeepGEMM grouped GEMM role in vLLM PR #20903: e4m3 operands, one fp32
// scale per 1x128 activation group and per 128x128 weight block).
//
//   out[r, n] = bf16( sum_g a_s[r,g] * w_s[e,n/128,g] * sum_{k in g} a[r,k] w[e,n,k] )
//
// Design:
//  * 256x256 output tile per 512-thread block: 8 waves in 2 (M) x 4 (N),
//    128x64 per wave = 8x4 MFMA 16x16x128 fp8 tiles, one block per CU
//    (128x256 tiles, 64x64 per wave, when the experts hold few rows).  The
//    operand stream from L2 and HBM is what bounds this kernel on gfx950, so
//    the tile is as large as the 256 VGPRs of two waves per SIMD allow: a
//    step moves 64 KB for 16.8 MFLOP (128x256 tiles: 48 KB for 8.4), and
//    each expert's weights are re-read by half as many m-tiles.  The fused
//    gate/up + SiLU-mul requant variant keeps 128x256 tiles (its epilogue
//    needs the registers).
//  * One MFMA spans exactly one K group, so each MFMA result is a whole
//    group's partial sum; it is scaled by a_s * w_s and folded into the fp32
//    accumulator with one FMA per output.  The group scales are arbitrary
//    fp32 values, so they cannot ride in the MFMA's power-of-two block-scale
//    operands; and the MFMA's own summation keeps only ~14 bits below the
//    largest product of each 8-wide K block, so promoting every 128 K to fp32
//    also bounds that error.  The MFMAs of row block i+1 are issued before
//    the promotion FMAs of row block i.
//  * Operands move global -> LDS by LDS DMA (global_load_lds_dwordx4: each
//    lane's 16 bytes land at M0 + 16*lane) through a ring of two 64 KB
//    stages (three 48 KB stages for 128-row tiles), so the next step's loads
//    are in flight while the MFMAs consume step i, with no staging registers
//    and no LDS store instructions.  A wave waits only for its own DMAs of the step it is
//    about to read (loads retire in issue order), and one barrier per step
//    publishes every wave's.  The activation scales of a step ride in the same
//    ring (dword DMA); the weight block scale is wave-uniform and comes
//    through the scalar cache.
//  * LDS rows are 128 bytes, the 16-byte chunk c of row r stored at position
//    c ^ (r mod 8) ^ (r/8 mod 2), so the 16 lanes feeding one MFMA row block
//    read 16 distinct bank groups (measured on gfx950: no conflict cycles);
//    the pattern repeats every 16 rows, so a lane's fragment addresses in
//    the row blocks of a stage differ by constants.  A DMA
//    writes 8 whole LDS rows, so each lane fetches the global chunk that the
//    swizzle places at its LDS position.
//  * Weight rows are placed so that lane j of MFMA column block b holds output
//    column 4j + b: each lane owns 4 adjacent columns and the epilogue writes
//    8-byte bf16 quads straight from registers, 128 contiguous bytes per row.
//  * Rows past an expert's valid count are loaded as a copy of its last valid
//    row and never stored, so the K loop has no divergent branches; tiles
//    cover only valid rows, so alignment padding is never multiplied.
//  * Persistent grid with an XCD-aware tile order: workgroups are dealt to the
//    8 XCDs round-robin, so XCD x walks the contiguous x-th eighth of the
//    (expert, m-tile, n-tile) sequence and an expert's weights stay hot in
//    that XCD's L2.  Tiles are walked without divisions, and the DMA stream
//    runs one step (two for 128-row tiles) ahead across tile boundaries.
//  * Row indices are clamped on the device, so even inconsistent
//    offsets/counts cannot move an access out of bounds.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int BN = 256;
constexpr int BK = 128;
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;   // 8: 2 along M, 4 along N
// Tile shape by MI, the 16-row MFMA blocks per wave (the tile has 2 * 16 * MI
// rows): MI = 8 gives 256x256 tiles with two 64 KB LDS stages, MI = 4 gives
// 128x256 tiles with three 48 KB stages, MI = 2 (the K-split kernel for
// experts of a few rows) 64x256 tiles with three 40 KB stages.
template <int MI>
struct Shape {
    static constexpr int BM = 32 * MI;
    static constexpr int kStageA = BM * BK;              // bytes
    static constexpr int kStage = kStageA + BN * BK;
    static constexpr int kStages = MI == 8 ? 2 : 3;
    static constexpr int kADma = MI / 2;                  // 8-row A DMAs per wave and step
    static constexpr int kDmaPerStep = kADma + 4 + 1;     // + 4 B + 1 scale
    static constexpr int kScaleRows = 4 * MI;             // A scale rows per wave
};

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int wave_incl_scan(int v) { return wave_inclusive_scan(v); }

// position (0..7) of 16-byte chunk c in LDS tile row r, and its inverse
__device__ __forceinline__ int swz_pos(int c, int r) { return c ^ (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz(int c, int r) { return r * 128 + (swz_pos(c, r) << 4); }

// LDS row of weight row n of the tile: within each 64-row quarter, row 4j+b
// goes to 16b+j, so MFMA column j of column block b is weight row 4j+b
__device__ __forceinline__ int b_row(int n) { return (n & ~63) | ((n & 3) << 4) | ((n >> 2) & 15); }
__device__ __forceinline__ int b_row_inv(int R) { return (R & ~63) | ((R & 15) << 2) | ((R >> 4) & 3); }

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b) {
    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    // cbsz = blgp = 0: both operands E4M3; zero scale operands select the
    // unscaled 16x16x128 f8f6f4 MFMA.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// A lane's 32 K-bytes of one MFMA operand: the two 16-byte halves (chunks
// 2h and 2h+1 of the row, at swizzled positions x and x^1) at LDS byte
// offsets lo + imm and hi + imm
__device__ __forceinline__ v8i frag2(const uint8_t* lo, const uint8_t* hi, int imm) {
    const v4i l = *reinterpret_cast<const v4i*>(lo + imm);
    const v4i h = *reinterpret_cast<const v4i*>(hi + imm);
    return v8i{l.x, l.y, l.z, l.w, h.x, h.y, h.z, h.w};
}

// LDS DMA (global_load_lds_dwordx4 / _dword): lane l's 16 (4) bytes from
// sbase + voff land at LDS byte lds + 16*l (4*l).  The compiler owns M0,
// which carries the wave-uniform LDS base; sbase is wave-uniform and voff a
// 32-bit per-lane offset, so the load takes the scalar-base form.  The
// compiler does not wait for these writes before later LDS reads: the K loop
// does that itself (wait_loads_barrier_c).
typedef __attribute__((address_space(3))) void* lds_ptr;
__device__ __forceinline__ lds_ptr lds_at(uint32_t lds) { return (lds_ptr)(uintptr_t)lds; }
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t voff, const void* sbase) {
    __builtin_amdgcn_global_load_lds(static_cast<const uint8_t*>(sbase) + voff, lds_at(lds), 16, 0, 0);
}
__device__ __forceinline__ void dma4(uint32_t lds, uint32_t voff, const void* sbase) {
    __builtin_amdgcn_global_load_lds(static_cast<const uint8_t*>(sbase) + voff, lds_at(lds), 4, 0, 0);
}

// Wait until at most N of this wave's vector-memory loads issued after the
// one waited for are outstanding, then the workgroup barrier.  Loads retire
// in issue order, so a younger load can never be the reason the count is
// low; stores may retire in any order, which only makes the wait longer.
// N is a compile-time count: a count chosen at run time would need a
// dispatch over literal vmcnt values, which costs ~5% of the GEMM's time.
template <int N>
__device__ __forceinline__ void wait_loads_barrier_c() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// rows [lo, hi) of expert e, clamped to [0, cap_rows)
__device__ __forceinline__ void rows_of(const int32_t* __restrict__ offsets, const int32_t* __restrict__ counts,
                                        int64_t cap_rows, int e, int64_t& lo, int64_t& hi) {
    lo = offsets[e];
    lo = lo < 0 ? 0 : (lo > cap_rows ? cap_rows : lo);
    int64_t c = counts[e];
    c = c < 0 ? 0 : c;
    hi = lo + c > cap_rows ? cap_rows : lo + c;
}

// Walks one block's tiles t_lo, t_lo + nslots, ... of the (expert, m-tile,
// n-tile) sequence without divisions: the m-tile/n-tile pair advances by a
// precomputed quotient and remainder, and the expert by a forward scan of
// s_tpre (s_tpre[e] = first m-tile of expert e).  All fields are
// wave-uniform.
struct TileCursor {
    int64_t t;           // tile index
    int tm, tn;          // m-tile, n-tile (split: n-tile + nsplit-th of K, see TileWalk)
    int e;               // expert of m-tile tm
    int e_lo, e_hi;      // its rows [e_lo, e_hi)
    bool valid;
    int m0, row_end, n0; // the tile: rows [m0, min(m0 + bm, row_end)), columns n0..
    int seg, g0;         // K segment and its first K group (0 and 0 without a split)
};

// With a split of K into nsplit segments of kseg groups, the walk runs over
// ntn * nsplit "n-tiles" per m-tile: n-tile tn of segment seg is number
// seg * ntn_real + tn.
struct TileWalk {
    const int32_t* offsets;
    const int32_t* counts;
    int64_t cap_rows;
    const int* s_tpre;
    const int* s_lo;     // LDS copies of the experts' clamped rows, or null: read offsets/counts
    const int* s_hi;
    int El, ntn, step_q, step_r;   // nslots = step_q * ntn + step_r
    int bm;                        // tile rows
    int64_t t_hi, nslots;
    int ntn_real, kseg, nsplit;

    __device__ __forceinline__ void fill(TileCursor& c) const {
        if (s_lo != nullptr) {
            c.e_lo = __builtin_amdgcn_readfirstlane(s_lo[c.e]);
            c.e_hi = __builtin_amdgcn_readfirstlane(s_hi[c.e]);
            return;
        }
        int64_t lo, hi;
        rows_of(offsets, counts, cap_rows, c.e, lo, hi);
        c.e_lo = __builtin_amdgcn_readfirstlane((int)lo);
        c.e_hi = __builtin_amdgcn_readfirstlane((int)hi);
    }
    __device__ __forceinline__ void tile(TileCursor& c) const {
        // clamped so that every row this tile touches is in [0, cap_rows)
        int m0 = c.e_lo + (c.tm - s_tpre[c.e]) * bm;
        m0 = max(c.e_lo, min(m0, c.e_hi - 1));
        c.m0 = __builtin_amdgcn_readfirstlane(min(m0, (int)cap_rows - 1));
        c.row_end = c.e_hi;
        if (nsplit > 1) {
            const int seg = c.tn / ntn_real;
            c.seg = seg;
            c.g0 = seg * kseg;
            c.n0 = (c.tn - seg * ntn_real) * BN;
        } else {
            c.seg = c.g0 = 0;
            c.n0 = c.tn * BN;
        }
    }
    __device__ __forceinline__ void start(TileCursor& c, int64_t t) const {
        c.t = t;
        c.valid = t < t_hi;
        c.tm = c.tn = c.e = c.e_lo = c.e_hi = c.m0 = c.row_end = c.n0 = c.seg = c.g0 = 0;
        if (!c.valid) return;
        if (t < (int64_t)0x7fffffff) {   // a 32-bit division when it fits
            c.tm = (int)t / ntn;
            c.tn = (int)t - c.tm * ntn;
        } else {
            c.tm = (int)(t / ntn);
            c.tn = (int)(t - (int64_t)c.tm * ntn);
        }
        int lo = 0, hi = El - 1;  // largest e < El with s_tpre[e] <= tm
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_tpre[mid] <= c.tm) lo = mid; else hi = mid - 1;
        }
        c.e = __builtin_amdgcn_readfirstlane(lo);
        fill(c);
        tile(c);
    }
    __device__ __forceinline__ void next(TileCursor& c) const {
        c.t += nslots;
        c.valid = c.t < t_hi;
        if (!c.valid) return;
        c.tn += step_r;
        c.tm += step_q;
        if (c.tn >= ntn) {
            c.tn -= ntn;
            c.tm += 1;
        }
        bool moved = false;
        while (c.e + 1 < El && s_tpre[c.e + 1] <= c.tm) {
            ++c.e;
            moved = true;
        }
        c.e = __builtin_amdgcn_readfirstlane(c.e);
        if (moved) fill(c);
        tile(c);
    }
};

// KACT = false: out[r, n] = bf16(GEMM), n < n_out.
// KACT = true (the gate/up GEMM fused with SiLU-and-mul and requant): n_out =
// 2N, w rows [0, N) are the gate and [N, 2N) the up projection; for every
// valid row r and act column c < N,
//   h = bf16(GEMM(r, c)), h' = bf16(GEMM(r, N + c)),
//   act = bf16(silu(h) * h'), then per 1x128 group of act: amax, scale and
//   e4m3 codes exactly as the SiLU-mul requant of act_quant.hip,
// written to q [rows, N] and q_s [rows, N/128].  A tile then holds 128 gate
// and the matching 128 up columns, and each lane owns matched gate/up pairs,
// so no intermediate h is stored.
//
// RED (with KACT = false; the down GEMM with the unpermute's weight-and-reduce
// folded into its epilogue): out is y as above, and for every token t of the
// chunk and column n, red_out[t, n] = bf16(fmaf chain over k = 0..topk-1 with
// a valid row r = inv_perm[t, k] of w'_k * y[r, n]), w'_k = topk_w[t, k] or 1
// on input: the same bits as moe_unpermute_weight_reduce.  A tile that has
// stored its y rows makes them visible device-wide and counts, per row, its
// token's (token, n-tile) counter up; the tile that brings a counter to the
// token's number of valid rows folds that token's rows for its columns (the
// other rows were made visible before their counts) and sets the counter back
// to zero.  Nothing waits for another tile.  The counters must be zero on entry
// and are zero again on exit; tokens without a valid row are written by the
// launcher's preparation kernel.
struct ReduceArgs {
    const int32_t* row_src;   // [cap_rows] token of each row, -1 on padding
    const int32_t* inv_perm;  // [Mc, topk]
    const float* topk_w;      // [Mc, topk]
    int on_input;
    int topk;
    int64_t Mc;
    int32_t* cnt;             // [Mc, ceil(n_out / 256)]
    uint16_t* out;            // [Mc, n_out]
};

// SMALL (with KACT = false and RED = false, MI = 2): the kernel for chunks
// with few routed rows per expert.  Its 64-row tiles waste less of each
// A step on copies of an expert's last row, and its 140 KB of LDS leave room
// on a CU for the small kernels of the forward's other lane.  Its units are
// short and each starts on another weight block, so the weight block scales
// ride in the ring as well (one more dword DMA per step) instead of coming
// through the scalar cache, whose miss at every unit start stalls the step.
// Without part, the output is bf16 out as above.  With part, and when the
// tiles fill fewer than four rounds of the grid, K is cut into sp.nsplit
// equal segments (the launcher's nsplit divides k_in / 128) and the grid
// walks (tile, segment) units; unit (tile, seg) folds the promoted group
// terms of its segment in k order, as the whole-K loop does, and stores the
// fp32 sums (not bf16) at part[seg, v, n], where v is the row's place among
// the valid rows of all experts in expert order; info[0] receives the
// segment count used (1 when not cut) and out is not written.  The consumer
// adds the partials in segment order and rounds the sum to bf16.
struct SplitArgs {
    float* part;          // [nsplit, part_rows, n_out], or null: bf16 out
    int32_t* info;        // segments used
    int64_t part_rows;    // valid rows held per segment; rows past it are not stored
    int nsplit;
};

template <bool KACT, int MI, bool RED = false, bool SMALL = false>
__global__ __launch_bounds__(kThreads, 1) void k_grouped_gemm(
    const uint8_t* __restrict__ a, const float* __restrict__ a_s, const uint8_t* __restrict__ w,
    const float* __restrict__ w_s, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ counts, int El, int64_t cap_rows, int n_out, int k_in,
    uint16_t* __restrict__ out, uint8_t* __restrict__ q, float* __restrict__ q_s, ReduceArgs red,
    SplitArgs sp) {
    static_assert(!SMALL || (!KACT && !RED && MI == 2), "the small-chunk kernel is the plain one on 64-row tiles");
    using Sh = Shape<MI>;
    constexpr int BM = Sh::BM, kStageA = Sh::kStageA, kStage = Sh::kStage, kStages = Sh::kStages;
    constexpr int kADma = Sh::kADma, kScaleRows = Sh::kScaleRows;
    constexpr int kDmaPerStep = Sh::kDmaPerStep + (SMALL ? 1 : 0);   // + the weight scales
    // the 256-row fused kernel has room for the SiLU table next to its two
    // 64 KB stages; the 128-row one, with three 48 KB stages, computes SiLU
    constexpr bool kSiluLds = KACT && MI == 8;
    __shared__ __attribute__((aligned(16))) uint8_t smem[kStages * kStage];
    __shared__ float s_silu[kSiluLds ? kSiluEntries : 1];
    __shared__ __attribute__((aligned(16))) float sAs[kStages][BM];   // [stage][row]
    __shared__ float sWs[SMALL ? kStages : 1][2];                       // [stage][128-column block]
    __shared__ int s_tpre[kMaxLocalExperts + 1];
    __shared__ int s_wsum[kWaves];
    __shared__ float s_amax[KACT ? 4 : 1][KACT ? BM : 1];   // per-wave-column partial group maxima
    __shared__ __attribute__((aligned(16))) float s_inv[KACT ? BM : 1];   // 448 / d of each row
    __shared__ int s_fold[RED ? BM : 1];   // tokens this tile completes
    __shared__ int s_nfold;
    __shared__ int s_vpre[SMALL ? kMaxLocalExperts + 1 : 1];   // valid rows before expert e, capped (split)
    // every expert's clamped rows [lo, hi), read once here: the tile walk
    // then finds them in LDS rather than in global memory (the fused kernel
    // has no LDS left for them)
    constexpr bool kLdsRows = !KACT;
    __shared__ int s_lo[kLdsRows ? kMaxLocalExperts : 1];
    __shared__ int s_hi[kLdsRows ? kMaxLocalExperts : 1];
    __shared__ int64_t s_vwsum[SMALL ? kWaves : 1];
    const int n_half = n_out / 2;                 // N when KACT

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    if constexpr (kSiluLds) silu_table_build(s_silu);   // published by the barriers below

    // ---- m-tile prefix over the experts' valid row counts ------------------
    // (and, for the split, the valid-row prefix: the partials' row places)
    int ntl[2];
    int64_t vl[2];
    int tsum = 0;
    int64_t vsum = 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int e = tid * 2 + j;
        int nt = 0;
        vl[j] = 0;
        if (e < El) {
            int64_t lo, hi;
            rows_of(offsets, counts, cap_rows, e, lo, hi);
            nt = (int)((hi - lo + BM - 1) / BM);
            vl[j] = hi - lo;
            if constexpr (kLdsRows) {
                s_lo[e] = (int)lo;
                s_hi[e] = (int)hi;
            }
        }
        ntl[j] = nt;
        tsum += nt;
        vsum += vl[j];
    }
    const int incl = wave_incl_scan(tsum);
    if (lane == kWave - 1) s_wsum[wave] = incl;
    // rows are at most cap_rows < 2^31 per expert, so 64-bit sums; the stored
    // row prefix is capped at part_rows
    int64_t vin = 0;
    if constexpr (SMALL) {
        vin = wave_inclusive_scan(vsum);
        if (lane == kWave - 1) s_vwsum[wave] = vin;
    }
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
    if constexpr (SMALL) {
        int64_t vex = vin - vsum;
        for (int w2 = 0; w2 < wave; ++w2) vex += s_vwsum[w2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int e = tid * 2 + j;
            if (e < El) s_vpre[e] = (int)(vex < sp.part_rows ? vex : sp.part_rows);
            vex += vl[j];
        }
    }
    __syncthreads();

    const int mtiles = __builtin_amdgcn_readfirstlane(s_tpre[El]);
    const int ntn = (n_out + BN - 1) / BN;   // the last n-tile may hold only 128 columns
    const int nb128 = n_out / 128;
    const int kg = k_in / BK;
    const int xcd = blockIdx.x & 7;
    const int nslots = gridDim.x >> 3;
    int nsplit = 1;
    if constexpr (SMALL) {
        if (sp.part != nullptr) {
            const int64_t tiles = (int64_t)mtiles * ntn;
            const int ns = sp.nsplit;   // checked here too: a bad count never leaves K short
            nsplit = (tiles < 4 * (int64_t)gridDim.x && ns > 1 && ns <= 8 && kg % ns == 0) ? ns : 1;
            if (blockIdx.x == 0 && tid == 0) sp.info[0] = nsplit;
        }
    }
    const int kseg = kg / nsplit;   // K groups per unit
    const int64_t total = (int64_t)mtiles * ntn * nsplit;
    const int64_t t_lo = total * xcd / 8 + (blockIdx.x >> 3);
    const int64_t t_hi = total * (xcd + 1) / 8;

    TileWalk walk;
    walk.offsets = offsets;
    walk.counts = counts;
    walk.cap_rows = cap_rows;
    walk.s_tpre = s_tpre;
    walk.s_lo = kLdsRows ? s_lo : nullptr;
    walk.s_hi = kLdsRows ? s_hi : nullptr;
    walk.El = El;
    walk.ntn = ntn * nsplit;
    walk.step_q = nslots / walk.ntn;
    walk.step_r = nslots - walk.step_q * walk.ntn;
    walk.t_hi = t_hi;
    walk.nslots = nslots;
    walk.bm = BM;
    walk.ntn_real = ntn;
    walk.kseg = kseg;
    walk.nsplit = nsplit;

    const int wm = wave >> 2;   // 0..1
    const int wn = wave & 3;    // 0..3
    const int fr = lane & 15;
    const int fc = 2 * (lane >> 4);   // this lane's K chunk pair
    // per-lane LDS byte offsets (within a stage) of this lane's two fragment
    // halves in row block 0 of A and of B; row block j adds j * 2048
    const uint32_t fA_lo = (uint32_t)swz(fc, wm * 16 * MI + fr), fA_hi = fA_lo ^ 16u;
    const uint32_t fB_lo = (uint32_t)(kStageA + swz(fc, wn * 64 + fr)), fB_hi = fB_lo ^ 16u;

    // ---- DMA side: which global chunk this lane fetches ---------------------
    // Wave w fills LDS rows 4*MI*w .. 4*MI*w + 4*MI-1 of A (MI/2 8-row DMAs)
    // and 32w..32w+31 of B (four), and the scales of its A rows (lanes
    // 0..4*MI-1).
    int rA[kADma], cA[kADma];
#pragma unroll
    for (int j = 0; j < kADma; ++j) {
        rA[j] = (wave * kADma + j) * 8 + (lane >> 3);
        cA[j] = swz_pos(lane & 7, rA[j]);   // the swizzle is an involution
    }
    // B: LDS row R holds weight row nB of the tile.  Plain: within each
    // 64-row quarter, row 4j+b goes to 16b+j, so lane j of MFMA column block
    // b computes output column 4j+b.  KACT: in the quarter of wave column wn,
    // MFMA blocks 0/1 are gate columns 2j / 2j+1 and blocks 2/3 the up
    // columns 2j / 2j+1 of the same 32-column slice; waves with even index
    // fill gate rows and odd ones up rows, nB counted from their half.
    int nB[4], cB[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
        const int R = (wave * 4 + qq) * 8 + (lane >> 3);
        nB[qq] = KACT ? (R >> 6) * 32 + 2 * (R & 15) + ((R >> 4) & 1) : b_row_inv(R);
        cB[qq] = swz_pos(lane & 7, R);
    }
    const int rS = wave * kScaleRows + (lane & (kScaleRows - 1));
    const uint32_t lds_smem = (uint32_t)(uintptr_t)smem;
    const uint32_t lds_as = (uint32_t)(uintptr_t)&sAs[0][0];
    const uint32_t lds_ws = (uint32_t)(uintptr_t)&sWs[0][0];

    // Loads issued by this wave so far, and the count right after each
    // pending step's DMAs (by ring slot).
    int loads = 0;
    int d_end0 = 0, d_end1 = 0, d_end2 = 0;

    // DMA cursor: tile, K step, ring slot, and the per-lane offsets
    TileCursor dT;
    walk.start(dT, t_lo);
    int d_g = 0, d_slot = 0;
    uint32_t voA[kADma], voB0 = 0, voB1 = 0, voB2 = 0, voB3 = 0, voS = 0;
#pragma unroll
    for (int j = 0; j < kADma; ++j) voA[j] = 0;
    // the DMA cursor's tile: its A rows, weight rows and A scales at its
    // current K step, set per tile and advanced by one step per DMA step
    const uint8_t* dA = a;
    const uint8_t* dB = w;
    const float* dS = a_s;
    const float* dW = w_s;
    uint32_t voW = 0;
#define MOE_DMA_OFFSETS()                                                             \
    do {                                                                              \
        const int last_ = max(dT.row_end - 1 - dT.m0, 0);                             \
        const int nlast_ = KACT ? 127 : min(BN, n_out - dT.n0) - 1;                   \
        _Pragma("unroll") for (int j_ = 0; j_ < kADma; ++j_)                          \
            voA[j_] = (uint32_t)(min(rA[j_], last_) * k_in + cA[j_] * 16);           \
        voB0 = (uint32_t)(min(nB[0], nlast_) * k_in + cB[0] * 16);                    \
        voB1 = (uint32_t)(min(nB[1], nlast_) * k_in + cB[1] * 16);                    \
        voB2 = (uint32_t)(min(nB[2], nlast_) * k_in + cB[2] * 16);                    \
        voB3 = (uint32_t)(min(nB[3], nlast_) * k_in + cB[3] * 16);                    \
        voS = (uint32_t)(min(rS, last_) * kg * 4);                                    \
        const int64_t brow0_ = KACT ? (int64_t)((wave & 1) ? n_half : 0) + (dT.n0 >> 1) \
                                    : (int64_t)dT.n0;                                 \
        dA = a + (int64_t)dT.m0 * k_in + dT.g0 * BK;                                  \
        dB = w + ((int64_t)dT.e * n_out + brow0_) * k_in + dT.g0 * BK;                \
        dS = a_s + (int64_t)dT.m0 * kg + dT.g0;                                       \
        if (SMALL) {                                                                  \
            dW = w_s + (int64_t)dT.e * nb128 * kg + dT.g0;                            \
            voW = (uint32_t)(min(dT.n0 / 128 + (lane & 1), nb128 - 1) * kg * 4);      \
        }                                                                             \
    } while (0)
    // one step of DMAs into ring slot d_slot, then advance the cursor
#define MOE_DMA_NEXT()                                                                \
    do {                                                                              \
        const uint8_t* sa_ = dA;                                                      \
        const uint8_t* sb_ = dB;                                                      \
        const float* ss_ = dS;                                                        \
        const float* sw_ = dW;                                                        \
        dA += BK;                                                                     \
        dB += BK;                                                                     \
        dS += 1;                                                                      \
        dW += 1;                                                                      \
        const uint32_t base_ = lds_smem + d_slot * kStage;                            \
        _Pragma("unroll") for (int j_ = 0; j_ < kADma; ++j_)                          \
            dma16(base_ + (wave * kADma + j_) * 1024, voA[j_], sa_);                  \
        dma16(base_ + kStageA + (wave * 4) * 1024, voB0, sb_);                        \
        dma16(base_ + kStageA + (wave * 4 + 1) * 1024, voB1, sb_);                    \
        dma16(base_ + kStageA + (wave * 4 + 2) * 1024, voB2, sb_);                    \
        dma16(base_ + kStageA + (wave * 4 + 3) * 1024, voB3, sb_);                    \
        if (lane < kScaleRows)                                                        \
            dma4(lds_as + d_slot * (BM * 4) + wave * (kScaleRows * 4), voS, ss_);     \
        if (SMALL && lane < 2) /* every wave, the same two dwords */                  \
            dma4(lds_ws + d_slot * 8, voW, sw_);                                      \
        loads += kDmaPerStep;                                                         \
        if (d_slot == 0) d_end0 = loads;                                              \
        else if (d_slot == 1) d_end1 = loads;                                         \
        else d_end2 = loads;                                                          \
        d_slot = d_slot == kStages - 1 ? 0 : d_slot + 1;                              \
        if (++d_g == kseg) {                                                          \
            d_g = 0;                                                                  \
            walk.next(dT);                                                            \
            if (dT.valid) MOE_DMA_OFFSETS();                                          \
        }                                                                             \
    } while (0)
    if (dT.valid) MOE_DMA_OFFSETS();
    // the DMA stream runs kStages - 1 steps ahead
    if (dT.valid) MOE_DMA_NEXT();
    if (kStages > 2 && dT.valid) MOE_DMA_NEXT();

    int slot = 0;    // ring slot of the step being computed
    TileCursor cur;
    walk.start(cur, t_lo);
    while (cur.valid) {
        const int n_valid = KACT ? BN : min(BN, n_out - cur.n0);
        const bool wave_has_rows = (cur.m0 + wm * 16 * MI) < cur.row_end && wn * 64 < n_valid;
        // weight block-scale rows: plain, the 128-column block of this wave;
        // KACT, the gate block (MFMA blocks 0/1) and the up block (2/3)
        const int64_t ws_row = KACT ? ((int64_t)cur.e * nb128 + (cur.n0 >> 8)) * kg
                                    : ((int64_t)cur.e * nb128 + min(cur.n0 / 128 + (wn >> 1), nb128 - 1)) * kg +
                                          cur.g0;
        const int64_t ws_row_up = ws_row + (int64_t)(n_half / 128) * kg;
        v4f acc[MI][4];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

        for (int g = 0; g < kseg; ++g) {
            // this step's DMAs complete, in every wave.  The loads issued after
            // them are the next kStages - 2 steps' DMAs: none with two
            // stages, where vmcnt(0) is exact; with three, one step's or (at
            // the end of the stream) none.  Waiting for fewer outstanding
            // loads than issued after them is always safe, so two fixed
            // counts cover every case without a dispatch.
            if constexpr (kStages == 2) {
                wait_loads_barrier_c<0>();
            } else {
                const int n_after = __builtin_amdgcn_readfirstlane(
                    loads - (slot == 0 ? d_end0 : (slot == 1 ? d_end1 : d_end2)));
                if (n_after >= kDmaPerStep) wait_loads_barrier_c<kDmaPerStep>();
                else wait_loads_barrier_c<0>();
            }
            // into the slot the previous step has released, while the DMA
            // cursor (kStages - 1 steps ahead) has steps left: a flag of the
            // tile walk, so no step count is compared
            if (dT.valid) MOE_DMA_NEXT();
            if (wave_has_rows) {
                const uint32_t sb = (uint32_t)slot * kStage;
                const uint8_t* alo = smem + (sb + fA_lo);
                const uint8_t* ahi = smem + (sb + fA_hi);
                const uint8_t* blo = smem + (sb + fB_lo);
                const uint8_t* bhi = smem + (sb + fB_hi);
                const float* scs = &sAs[slot][wm * 16 * MI + (lane >> 4) * 4];
                const float ws = SMALL ? sWs[slot][wn >> 1] : w_s[ws_row + g];
                const float ws_up = KACT ? w_s[ws_row_up + g] : ws;
                v8i bf[4];
#pragma unroll
                for (int ni = 0; ni < 4; ++ni) bf[ni] = frag2(blo, bhi, ni * 2048);
                // software-pipelined over the four row blocks: the MFMAs of
                // row block mi+1 are in flight while row block mi is promoted
                v4f p[2][4];
                {
                    const v8i af = frag2(alo, ahi, 0);
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) p[0][ni] = mfma_fp8(af, bf[ni]);
                }
#pragma unroll
                for (int mi = 0; mi < MI; ++mi) {
                    if (mi + 1 < MI) {
                        const v8i af = frag2(alo, ahi, (mi + 1) * 2048);
#pragma unroll
                        for (int ni = 0; ni < 4; ++ni) p[(mi + 1) & 1][ni] = mfma_fp8(af, bf[ni]);
                    }
                    const v4f sa4 = *reinterpret_cast<const v4f*>(scs + mi * 16);
                    const v4f sc_lo = {sa4.x * ws, sa4.y * ws, sa4.z * ws, sa4.w * ws};
                    v4f sc_hi = sc_lo;
                    if (KACT) sc_hi = v4f{sa4.x * ws_up, sa4.y * ws_up, sa4.z * ws_up, sa4.w * ws_up};
#pragma unroll
                    for (int ni = 0; ni < 4; ++ni) {
                        const v4f sc = ni < 2 ? sc_lo : sc_hi;
                        const v4f pr = p[mi & 1][ni];
                        acc[mi][ni].x = __builtin_fmaf(sc.x, pr.x, acc[mi][ni].x);
                        acc[mi][ni].y = __builtin_fmaf(sc.y, pr.y, acc[mi][ni].y);
                        acc[mi][ni].z = __builtin_fmaf(sc.z, pr.z, acc[mi][ni].z);
                        acc[mi][ni].w = __builtin_fmaf(sc.w, pr.w, acc[mi][ni].w);
                    }
                }
            }
            slot = slot == kStages - 1 ? 0 : slot + 1;
        }

        if constexpr (!KACT) {
            // ---- epilogue: each lane owns 4 adjacent columns of 16 rows ----
            // Streaming stores: the output is read back from HBM by the next
            // kernel, so it need not take L2 lines from the operands.  Rows
            // are addressed from the lane's first row by 32-bit offsets; a
            // wave whose 16 * MI rows are all valid stores without row tests.
            if (SMALL && sp.part != nullptr && wave_has_rows) {
                // fp32 partial sums of the segment, at the rows' valid-row places
                const int row0 = cur.m0 + wm * 16 * MI + (lane >> 4) * 4;
                const int64_t v0 = (int64_t)s_vpre[cur.e] + (row0 - cur.e_lo);
                float* const pb = sp.part + ((int64_t)cur.seg * sp.part_rows + v0) * n_out +
                                  (cur.n0 + wn * 64 + 4 * fr);
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int dr = mi * 16 + v;
                        if (row0 + dr < cur.row_end && v0 + dr < sp.part_rows)
                            __builtin_nontemporal_store(v4f{acc[mi][0][v], acc[mi][1][v], acc[mi][2][v], acc[mi][3][v]},
                                                        reinterpret_cast<v4f*>(pb + (int64_t)dr * n_out));
                    }
            } else if (wave_has_rows) {
                const int row0 = cur.m0 + wm * 16 * MI + (lane >> 4) * 4;
                uint16_t* const base = out + (int64_t)row0 * n_out + (cur.n0 + wn * 64 + 4 * fr);
                auto store_row = [&](int mi, int v) __attribute__((always_inline)) {
                    v2i qv;
                    qv.x = (int)f32x2_to_bf16x2(acc[mi][0][v], acc[mi][1][v]);
                    qv.y = (int)f32x2_to_bf16x2(acc[mi][2][v], acc[mi][3][v]);
                    __builtin_nontemporal_store(qv, reinterpret_cast<v2i*>(base + (mi * 16 + v) * n_out));
                };
                if (cur.m0 + wm * 16 * MI + 16 * MI <= cur.row_end) {
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                        for (int v = 0; v < 4; ++v) store_row(mi, v);
                } else {
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            if (row0 + mi * 16 + v < cur.row_end) store_row(mi, v);
                }
            }
            if constexpr (RED) {
                // ---- weight-and-reduce of the tokens this tile completes ----
                // the y stores of every wave, visible device-wide before any
                // count of this tile
                if (tid == 0) s_nfold = 0;
                __threadfence();
                __syncthreads();
                const int ntn_ = (n_out + BN - 1) / BN;
                if (tid < BM) {
                    const int row = cur.m0 + tid;
                    const int64_t t = row < cur.row_end ? (int64_t)red.row_src[row] : -1;
                    if (t >= 0 && t < red.Mc) {
                        int need = 0;
                        for (int k = 0; k < red.topk; ++k) {
                            const int r = red.inv_perm[t * red.topk + k];
                            need += (r >= 0 && r < cap_rows) ? 1 : 0;
                        }
                        const int old = atomicAdd(&red.cnt[t * ntn_ + cur.tn], 1);
                        if (old + 1 == need) s_fold[atomicAdd(&s_nfold, 1)] = (int)t;
                    }
                }
                __syncthreads();
                const int nfold = s_nfold;
                if (nfold > 0) {
                    // the other tiles' y rows of these tokens: counted after
                    // they were made visible
                    __threadfence();
                    const int c = cur.n0 + 4 * lane;   // this lane's 4 columns
                    for (int f = wave; f < nfold; f += kWaves) {
                        const int64_t t = s_fold[f];
                        if (4 * lane < n_valid) {
                            float acc4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                            for (int k = 0; k < red.topk; ++k) {
                                const int r = red.inv_perm[t * red.topk + k];
                                if (r < 0 || r >= cap_rows) continue;
                                const float wk = red.on_input ? 1.0f : red.topk_w[t * red.topk + k];
                                const v2i yv = *reinterpret_cast<const v2i*>(out + (int64_t)r * n_out + c);
                                const uint32_t lo = (uint32_t)yv.x, hi = (uint32_t)yv.y;
                                acc4[0] = __builtin_fmaf(wk, __uint_as_float(lo << 16), acc4[0]);
                                acc4[1] = __builtin_fmaf(wk, __uint_as_float(lo & 0xffff0000u), acc4[1]);
                                acc4[2] = __builtin_fmaf(wk, __uint_as_float(hi << 16), acc4[2]);
                                acc4[3] = __builtin_fmaf(wk, __uint_as_float(hi & 0xffff0000u), acc4[3]);
                            }
                            v2i o;
                            o.x = (int)f32x2_to_bf16x2(acc4[0], acc4[1]);
                            o.y = (int)f32x2_to_bf16x2(acc4[2], acc4[3]);
                            __builtin_nontemporal_store(o, reinterpret_cast<v2i*>(red.out + t * n_out + c));
                        }
                        if (lane == 0) red.cnt[t * ntn_ + cur.tn] = 0;
                    }
                }
                // s_fold and s_nfold are reused by the next tile
                __syncthreads();
            }
        } else {
            // ---- epilogue: SiLU-and-mul and per-128 requant ----------------
            // This lane holds, for 4 * MI rows, act columns 2fr and 2fr+1 of
            // the wave's 32-column slice (gate in blocks 0/1, up in 2/3).
            // The group of a row is the tile's 128 act columns, spread over
            // the 16 lanes of a row quad and the 4 waves of the same wm.
            const int j = cur.n0 >> 8;   // act column block
            float act[MI][4][2];
            float amax[MI][4];
            if constexpr (kSiluLds) {
                // SiLU of the bf16 gates from the table, without branches;
                // gates outside it (rare) are redone below with the formula
                bool outside = false;
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const uint32_t hg = f32x2_to_bf16x2(acc[mi][0][v], acc[mi][1][v]);
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const uint32_t hb = h ? hg >> 16 : hg & 0xffffu;
                            const uint32_t t = (hb & 0x7fffu) - (uint32_t)(kSiluExpLo << 7);
                            const bool in = t < (uint32_t)kSiluHalf;
                            act[mi][v][h] = s_silu[in ? t + (hb >> 15) * kSiluHalf : 0u];
                            outside |= !in;
                        }
                    }
                if (__builtin_expect(__ballot(outside) != 0, 0)) {
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const uint32_t hg = f32x2_to_bf16x2(acc[mi][0][v], acc[mi][1][v]);
#pragma unroll
                            for (int h = 0; h < 2; ++h) {
                                const uint32_t hb = h ? hg >> 16 : hg & 0xffffu;
                                const uint32_t t = (hb & 0x7fffu) - (uint32_t)(kSiluExpLo << 7);
                                if (t >= (uint32_t)kSiluHalf) act[mi][v][h] = silu_pinned(__uint_as_float(hb << 16));
                            }
                        }
                }
            }
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const uint32_t hu = f32x2_to_bf16x2(acc[mi][2][v], acc[mi][3][v]);
                    const float u0 = __uint_as_float(hu << 16), u1 = __uint_as_float(hu & 0xffff0000u);
                    float s0, s1;
                    if constexpr (kSiluLds) {
                        s0 = act[mi][v][0];
                        s1 = act[mi][v][1];
                    } else {
                        const uint32_t hg = f32x2_to_bf16x2(acc[mi][0][v], acc[mi][1][v]);
                        s0 = silu_pinned(__uint_as_float(hg << 16));
                        s1 = silu_pinned(__uint_as_float(hg & 0xffff0000u));
                    }
                    const float p0 = s0 * u0;
                    const float p1 = s1 * u1;
                    const uint32_t pk = f32x2_to_bf16x2(p0, p1);   // act is rounded to bf16
                    act[mi][v][0] = __uint_as_float(pk << 16);
                    act[mi][v][1] = __uint_as_float(pk & 0xffff0000u);
                    // largest non-NaN magnitude (compare-select, so m is never
                    // NaN), then over the 16 lanes of the row quad
                    float m = 0.0f;
                    const float a0 = __builtin_fabsf(act[mi][v][0]), a1 = __builtin_fabsf(act[mi][v][1]);
                    m = a0 > m ? a0 : m;
                    m = a1 > m ? a1 : m;
                    amax[mi][v] = row16_max_nonnan(m);
                }
            if (fr == 0) {
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        s_amax[wn][wm * 16 * MI + mi * 16 + (lane >> 4) * 4 + v] = amax[mi][v];
            }
            // publish the partial maxima (LDS only: the DMAs in flight for
            // the next steps are not waited for)
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            const int ng = n_half / 128;
            // each row's d, scale and 448 / d once: the 4 waves of a wave row
            // take 4 * MI of its 16 * MI rows each, one per lane
            if (lane < 4 * MI) {
                const int rl = wm * 16 * MI + wn * 4 * MI + lane;
                float m = s_amax[0][rl];
#pragma unroll
                for (int ww = 1; ww < 4; ++ww) {
                    const float o = s_amax[ww][rl];
                    m = o > m ? o : m;
                }
                const float dd = __builtin_fmaxf(m, 1e-10f);
                s_inv[rl] = 448.0f / dd;
                const int row = cur.m0 + rl;
                if (row < cur.row_end) q_s[(int64_t)row * ng + j] = dd / 448.0f;
            }
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
                const v4f inv4 = *reinterpret_cast<const v4f*>(&s_inv[wm * 16 * MI + mi * 16 + (lane >> 4) * 4]);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int rl = wm * 16 * MI + mi * 16 + (lane >> 4) * 4 + v;
                    const float inv = inv4[v];
                    // |act * inv| <= 448 (1 + 2^-23) unless NaN: d >= every |act| of the group
                    const uint32_t codes =
                        f32x4_to_e4m3_bounded(act[mi][v][0] * inv, act[mi][v][1] * inv, 0.0f, 0.0f);
                    const int row = cur.m0 + rl;
                    if (wave_has_rows && row < cur.row_end)
                        *reinterpret_cast<uint16_t*>(q + (int64_t)row * n_half + j * 128 + wn * 32 + 2 * fr) =
                            (uint16_t)codes;
                }
            }
        }
        walk.next(cur);
    }
#undef MOE_DMA_OFFSETS
#undef MOE_DMA_NEXT
}

}  // namespace

namespace {

int64_t gemm_grid(int64_t cap_rows, int El, int n_out, int bm, int num_cus, int units_per_tile = 1) {
    const int64_t ntn = (n_out + BN - 1) / BN;
    const int64_t bound = ((cap_rows + bm - 1) / bm + El) * ntn * units_per_tile;
    int64_t grid = num_cus;            // one 8-wave block per CU (up to 150 KB of LDS)
    if (bound < grid) grid = bound;
    grid = ((grid + 7) / 8) * 8;
    if (grid < 8) grid = 8;
    return grid;
}

}  // namespace

// 256-row tiles move fewer bytes per flop, but every 16-row block of an
// active wave is computed, so experts of a few rows are cheaper on 128-row
// tiles.  Measured with hidden size 2048, intermediate size 768, 128 experts
// and top-8 routing (ms, 128-row vs 256-row tiles, gate/up GEMM): 80 routed
// rows per expert 0.081 vs 0.087, 96 rows 0.083 vs 0.090, 112 rows 0.103 vs
// 0.094, 128 rows 0.117 vs 0.101, 192 rows 0.133 vs 0.114, 256 rows 0.182
// vs 0.167, 384 rows 0.238 vs 0.199 (the down GEMM alike).
int gemm_tile_rows(int64_t rows_hint, int El) {
    return (El > 0 && rows_hint >= (int64_t)256 * El) ? 256 : 128;
}

int gemm_tile_rows_routed(int64_t pairs, int El) {
    return (El > 0 && pairs >= (int64_t)104 * El) ? 256 : 128;
}

hipError_t launch_grouped_gemm(const uint8_t* a, const float* a_s, const uint8_t* w,
                               const float* w_s, const int32_t* offsets, const int32_t* counts,
                               int El, int64_t cap_rows, int n_out, int k_in, uint16_t* out,
                               int tile_rows, int num_cus, hipStream_t s) {
    if (tile_rows == 256) {
        const int64_t grid = gemm_grid(cap_rows, El, n_out, Shape<8>::BM, num_cus);
        k_grouped_gemm<false, 8><<<(unsigned)grid, kThreads, 0, s>>>(a, a_s, w, w_s, offsets, counts, El,
                                                                      cap_rows, n_out, k_in, out, nullptr, nullptr, ReduceArgs{}, SplitArgs{});
    } else {
        const int64_t grid = gemm_grid(cap_rows, El, n_out, Shape<4>::BM, num_cus);
        k_grouped_gemm<false, 4><<<(unsigned)grid, kThreads, 0, s>>>(a, a_s, w, w_s, offsets, counts, El,
                                                                      cap_rows, n_out, k_in, out, nullptr, nullptr, ReduceArgs{}, SplitArgs{});
    }
    return hipGetLastError();
}

hipError_t launch_grouped_gemm_small(const uint8_t* a, const float* a_s, const uint8_t* w, const float* w_s,
                                     const int32_t* offsets, const int32_t* counts, int El, int64_t cap_rows,
                                     int n_out, int k_in, uint16_t* out, float* part, int64_t part_rows, int nsplit,
                                     int32_t* info, int num_cus, hipStream_t s) {
    const int64_t grid = gemm_grid(cap_rows, El, n_out, Shape<2>::BM, num_cus, part != nullptr ? nsplit : 1);
    k_grouped_gemm<false, 2, false, true><<<(unsigned)grid, kThreads, 0, s>>>(
        a, a_s, w, w_s, offsets, counts, El, cap_rows, n_out, k_in, part != nullptr ? nullptr : out, nullptr, nullptr,
        ReduceArgs{}, SplitArgs{part, info, part_rows, nsplit});
    return hipGetLastError();
}

hipError_t launch_grouped_gemm_reduce(const uint8_t* a, const float* a_s, const uint8_t* w, const float* w_s,
                                      const int32_t* offsets, const int32_t* counts, int El, int64_t cap_rows,
                                      int n_out, int k_in, uint16_t* y, const int32_t* row_src,
                                      const int32_t* inv_perm, const float* topk_w, int on_input, int64_t Mc,
                                      int topk, int32_t* cnt, uint16_t* out, int tile_rows, int num_cus,
                                      hipStream_t s) {
    const ReduceArgs red{row_src, inv_perm, topk_w, on_input, topk, Mc, cnt, out};
    if (tile_rows == 256) {
        const int64_t grid = gemm_grid(cap_rows, El, n_out, Shape<8>::BM, num_cus);
        k_grouped_gemm<false, 8, true><<<(unsigned)grid, kThreads, 0, s>>>(a, a_s, w, w_s, offsets, counts, El,
                                                                            cap_rows, n_out, k_in, y, nullptr,
                                                                            nullptr, red, SplitArgs{});
    } else {
        const int64_t grid = gemm_grid(cap_rows, El, n_out, Shape<4>::BM, num_cus);
        k_grouped_gemm<false, 4, true><<<(unsigned)grid, kThreads, 0, s>>>(a, a_s, w, w_s, offsets, counts, El,
                                                                            cap_rows, n_out, k_in, y, nullptr,
                                                                            nullptr, red, SplitArgs{});
    }
    return hipGetLastError();
}

hipError_t launch_grouped_gemm_act(const uint8_t* a, const float* a_s, const uint8_t* w13,
                                   const float* w13_s, const int32_t* offsets, const int32_t* counts,
                                   int El, int64_t cap_rows, int N, int k_in, uint8_t* q, float* q_s,
                                   int tile_rows, int num_cus, hipStream_t s) {
    if (tile_rows == 256) {
        const int64_t grid = gemm_grid(cap_rows, El, 2 * N, Shape<8>::BM, num_cus);
        k_grouped_gemm<true, 8><<<(unsigned)grid, kThreads, 0, s>>>(a, a_s, w13, w13_s, offsets, counts, El,
                                                                     cap_rows, 2 * N, k_in, nullptr, q, q_s, ReduceArgs{}, SplitArgs{});
    } else {
        const int64_t grid = gemm_grid(cap_rows, El, 2 * N, Shape<4>::BM, num_cus);
        k_grouped_gemm<true, 4><<<(unsigned)grid, kThreads, 0, s>>>(a, a_s, w13, w13_s, offsets, counts, El,
                                                                     cap_rows, 2 * N, k_in, nullptr, q, q_s, ReduceArgs{}, SplitArgs{});
    }
    return hipGetLastError();
}

}  // namespace moe
