// count_permute.hip -- expert counting and the stable expert-contiguous permute
// (count_expert_num_tokens of vLLM PR #20392 and the ep_scatter permute of
// vLLM PR #20903), written for gfx950.
//
// Permute runs in three launches:
//   hist    one block per 256 (token, k) pairs: per-block expert histogram
//   colscan one block per expert: exclusive scan of its column of the
//           histogram (the block's first row within the expert's segment)
//           and the expert's count
//   (chunks of at most 4096 pairs skip these two: each scatter block counts
//   all the pairs itself)
//   scatter one block per 256 pairs and slice of the K groups: aligned
//           offsets (every block scans the El counts itself; block (0, 0)
//           publishes them and all blocks share the padding marks),
//           wave-ballot ranks
//           (stable in flat pair order), inverse indices (written by the
//           blocks of slice 0), then each token row slice is read once and
//           written to each of its expert rows with 16-byte lanes.  The
//           rows are split along K so that about 1024 blocks share them
//           (chunks of few tokens have few pair blocks).  The token rows
//           are read with non-temporal loads; the stores of a_perm stay
//           ordinary (non-temporal ones move their cost into the GEMM
//           that reads a_perm next: both ways the step takes as long).
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kPermThreads = 256;
constexpr int kMapLds = 2048;   // expert maps of up to this many global experts are staged in LDS
constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / kWave;

// counts [El] and, when given, invalid [1] set to zero in one launch
__global__ void k_count_clear(int32_t* __restrict__ counts, int El, int32_t* __restrict__ invalid) {
    for (int e = threadIdx.x; e < El; e += blockDim.x) counts[e] = 0;
    if (invalid && threadIdx.x == 0) invalid[0] = 0;
}

// The batched, masked layout: slot e holds rows [e * max_tokens,
// (e + 1) * max_tokens), the first counts[e] of them valid.  offsets[e] =
// e * max_tokens, cut[e] = counts[e] clamped to [0, max_tokens].
__global__ void k_slot_offsets(const int32_t* __restrict__ counts, int El, int64_t max_tokens,
                               int32_t* __restrict__ offsets, int32_t* __restrict__ cut) {
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e <= El; e += gridDim.x * blockDim.x) {
        offsets[e] = (int32_t)(e * max_tokens);
        if (e < El) {
            const int64_t c = counts[e];
            cut[e] = (int32_t)(c < 0 ? 0 : (c > max_tokens ? max_tokens : c));
        }
    }
}

// Tokens per local expert over a flat list of (token, k) expert ids.
//
// A block of kCountThreads keeps one LDS table of El x S counters, S slots
// per expert (S a power of two, at most 64): lane l adds to slot l mod S of
// its expert, so the adds of one wave spread over the banks whatever the ids
// are (a plain El-word histogram makes lanes that draw nearby experts collide
// on one bank).  The ids stream through 16-byte non-temporal loads, eight per
// lane, the next eight in flight while the LDS adds count the last.  At the
// end each block folds the slots and adds its totals to counts: two experts
// per 64-bit atomic when the caller's counts are 8-byte aligned and no count
// can pass 2^31 (then no carry crosses into the neighbour's word), else one
// 32-bit atomic per expert.  Every block's adds meet on the same few cache
// lines, where the memory side takes them one block at a time (about 15 ns
// each, measured), so the launch uses at most one block per CU.
constexpr int kCountThreads = 1024;
constexpr int kCountLdsWords = 16384;   // the El x S table: 64 KiB

__host__ __device__ inline int count_slots_log2(int El) {
    int sl = 6;
    while (sl > 0 && (El << sl) > kCountLdsWords) --sl;
    return sl;
}

// MAP: kCountMapNone (local expert = id), kCountMapLds (the map staged in
// LDS) or kCountMapGlobal (a map too long for LDS, read where it is).  The
// first two keep global loads out of the counting, so the batch in flight is
// never waited for early.
enum { kCountMapNone = 0, kCountMapLds = 1, kCountMapGlobal = 2 };

template <int MAP>
__global__ __launch_bounds__(kCountThreads) void k_count(const int32_t* __restrict__ ids, int64_t num_pairs,
                                                         const int32_t* __restrict__ emap, int Eg, int El,
                                                         int slots_log2, int pack64,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ invalid) {
    // h[e * S + slot]; the kWave words past the table take the adds of ids
    // that are not local (one word per slot), so every id adds somewhere and
    // the counting has no branches
    __shared__ int h[kCountLdsWords + kWave];
    __shared__ int s_map[MAP == kCountMapLds ? kMapLds + 1 : 1];   // [Eg] = -1
    __shared__ int s_sum[kMaxLocalExperts];   // the block's total per expert
    __shared__ int bad;
    const int S = 1 << slots_log2;
    const int tid = threadIdx.x;
    const int table = El << slots_log2;
    for (int j = tid; j < table + S; j += kCountThreads) h[j] = 0;
    if constexpr (MAP == kCountMapLds)
        for (int j = tid; j <= Eg; j += kCountThreads) s_map[j] = j < Eg ? emap[j] : -1;
    if (tid == 0) bad = 0;
    __syncthreads();
    const int slot = tid & (S - 1);
    int my_bad = 0;
    // The local expert as an unsigned value: anything at or past El (ids
    // that are -1, not local or out of range) is clamped to El, the row of
    // the table's spare words.  Invalid ids (below -1 or at least Eg) are
    // counted apart.
    auto add = [&](int id) __attribute__((always_inline)) {
        my_bad += ((unsigned)id + 1u > (unsigned)Eg) ? 1 : 0;
        unsigned e;
        if constexpr (MAP == kCountMapNone)
            e = (unsigned)id;   // El <= Eg without a map: ids in [El, Eg) are not local
        else if constexpr (MAP == kCountMapLds)
            e = (unsigned)s_map[min((unsigned)id, (unsigned)Eg)];
        else
            e = (unsigned)id < (unsigned)Eg ? (unsigned)emap[id] : 0xffffffffu;
        atomicAdd(&h[(min(e, (unsigned)El) << slots_log2) | slot], 1);
    };
    // Full batches: kLoads vectors per lane, every one in bounds, so the
    // loads are unconditional and the wait before counting a batch leaves
    // the next batch in flight.  The rest (less than two batches of vectors,
    // then the last num_pairs mod 4 ids) is read with bounds checks.
    // (with a map read from global memory each count waits for its map
    // loads, and with them for every load before: few vectors per batch)
    constexpr int kLoads = MAP == kCountMapGlobal ? 2 : 8;
    typedef int v4i __attribute__((ext_vector_type(4)));
    const v4i* ids4 = reinterpret_cast<const v4i*>(ids);
    const int64_t nvec = num_pairs / 4;
    const int64_t stride = (int64_t)gridDim.x * kCountThreads;
    const int64_t batch = kLoads * stride;
    const int64_t lane_v = blockIdx.x * (int64_t)kCountThreads + tid;
    auto load = [&](v4i (&q)[kLoads], int64_t v0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kLoads; ++u) q[u] = __builtin_nontemporal_load(ids4 + v0 + u * stride);
    };
    auto count = [&](const v4i (&q)[kLoads]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            add(q[u].x);
            add(q[u].y);
            add(q[u].z);
            add(q[u].w);
        }
    };
    // batches go in pairs, A and B: B loads while A counts, then the next A
    // while B counts; the scheduling barriers keep each batch's loads ahead
    // of the counting they overlap
    const int64_t npair = nvec / (2 * batch);
    if (npair > 0) {
        v4i qa[kLoads], qb[kLoads];
        load(qa, lane_v);
        for (int64_t p = 0; p + 1 < npair; ++p) {
            load(qb, lane_v + (2 * p + 1) * batch);
            __builtin_amdgcn_sched_barrier(0);
            count(qa);
            __builtin_amdgcn_sched_barrier(0);
            load(qa, lane_v + (2 * p + 2) * batch);
            __builtin_amdgcn_sched_barrier(0);
            count(qb);
            __builtin_amdgcn_sched_barrier(0);
        }
        load(qb, lane_v + (2 * npair - 1) * batch);
        __builtin_amdgcn_sched_barrier(0);
        count(qa);
        count(qb);
    }
    for (int64_t v = 2 * npair * batch + lane_v; v < nvec; v += stride) {
        const v4i q = ids4[v];
        add(q.x);
        add(q.y);
        add(q.z);
        add(q.w);
    }
    for (int64_t f = nvec * 4 + lane_v; f < num_pairs; f += stride) add(ids[f]);
    if (my_bad) atomicAdd(&bad, my_bad);
    __syncthreads();
    // Fold: G consecutive lanes share expert e, each summing S / G of its
    // slots (rotated by e, so that one wave's reads fall in distinct banks),
    // then a shuffle reduction over the G lanes.
    int g_log2 = 0;
    while (g_log2 < slots_log2 && (El << (g_log2 + 1)) <= kCountThreads) ++g_log2;
    const int G = 1 << g_log2;
    const int e = tid >> g_log2;
    const int part = tid & (G - 1);
    const int per = S >> g_log2;
    int c = 0;
    if (e < El) {
        const int* he = h + (e << slots_log2);
        for (int j = 0; j < per; ++j) c += he[(part * per + j + e) & (S - 1)];
    }
    for (int o = 1; o < G; o <<= 1) c += __shfl_xor(c, o);
    if (e < El && part == 0) s_sum[e] = c;
    __syncthreads();
    // The block's totals leave from consecutive lanes over consecutive
    // words (two experts per lane with 64-bit adds), so that each wave's
    // atomics reach memory as few dense requests rather than many sparse
    // ones: the adds of every block meet on these few hundred bytes.
    if (pack64) {
        const int pairs = El >> 1;
        for (int q = tid; q < pairs; q += kCountThreads) {
            const unsigned long long both = (unsigned long long)(unsigned)s_sum[2 * q] |
                                            ((unsigned long long)(unsigned)s_sum[2 * q + 1] << 32);
            if (both) atomicAdd(reinterpret_cast<unsigned long long*>(counts + 2 * q), both);
        }
        if ((El & 1) && tid == 0 && s_sum[El - 1]) atomicAdd(&counts[El - 1], s_sum[El - 1]);
    } else {
        for (int q = tid; q < El; q += kCountThreads)
            if (s_sum[q]) atomicAdd(&counts[q], s_sum[q]);
    }
    if (tid == 0 && invalid && bad) atomicAdd(invalid, bad);
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

__device__ __forceinline__ int wave_exclusive_scan(int v) { return wave_inclusive_scan(v) - v; }

// Column e of hist [nblk, El] (one block per expert): replaced in place by
// its exclusive prefix (the first row of expert e's segment that block b
// fills, relative to the segment start); the column total is counts[e].
__global__ __launch_bounds__(kScanThreads) void k_permute_colscan(int32_t* __restrict__ hist, int nblk, int El,
                                                                  int32_t* __restrict__ counts,
                                                                  int32_t* __restrict__ counts_copy) {
    __shared__ int wsum[kScanWaves];
    const int e = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int per = (nblk + kScanThreads - 1) / kScanThreads;   // rows per thread, contiguous
    const int b_lo = min(nblk, (int)threadIdx.x * per);
    const int b_hi = min(nblk, b_lo + per);
    int sum = 0;
#pragma unroll 8
    for (int b = b_lo; b < b_hi; ++b) sum += hist[(int64_t)b * El + e];
    const int incl = wave_inclusive_scan(sum);
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int base = incl - sum;
    for (int w = 0; w < wave; ++w) base += wsum[w];
#pragma unroll 8
    for (int b = b_lo; b < b_hi; ++b) {
        const int64_t idx = (int64_t)b * El + e;
        const int t = hist[idx];
        hist[idx] = base;
        base += t;
    }
    if (threadIdx.x == kScanThreads - 1) {
        counts[e] = base;   // the last thread ends on the column total
        if (counts_copy) counts_copy[e] = base;
    }
}

// What the scatter's loads of items past the end read (never written; not
// const, so that they sit in the global address space with the kernel's
// pointers and a choice between the two is still a global load).
__device__ int32_t g_fill_neg1[1] = {-1};
__device__ int32_t g_fill_zero[1] = {0};
__device__ float g_fill_one[1] = {1.0f};
__device__ __attribute__((aligned(16))) uint32_t g_fill_zero16[4] = {0u, 0u, 0u, 0u};

// Stable rank of every local pair, inverse indices, then the row copies.
// QUANT: the rows come from bf16 x [Mc, K] and are quantised here (per
// 1x128 group, exactly as the identity act quant), so a_q / a_s are never
// written or read; otherwise they are copied from a_q / a_s.  GMAP: the
// expert map has too many entries for LDS and is read from global memory.
// SELF: few pairs, so every block counts all of the chunk's pairs itself
// (no histogram launches); otherwise the counts and this block's row bases
// come from the column scan.  Every global read is issued first (the block's ids and router weights, the
// chunk's ids or the block's counts and row bases, the expert map, the first
// batch of rows), and that batch is quantised as soon as it arrives, before
// the first store: a wait for a load issued after a store waits for the
// store as well, so the count, scan and rank that follow use LDS alone and
// every store leaves after them.
template <bool QUANT, bool GMAP, bool SELF>
__global__ __launch_bounds__(kPermThreads) void k_permute_scatter(
    const uint8_t* __restrict__ a_q, const float* __restrict__ a_s, const uint16_t* __restrict__ x,
    const int32_t* __restrict__ ids,
    const float* __restrict__ topk_w, int apply_on_input, int64_t Mc, int K, int topk, int tpb,
    const int32_t* __restrict__ emap, int Eg, int El, int nbits, const int32_t* __restrict__ base,
    int32_t* __restrict__ counts, int32_t* __restrict__ counts_copy, int align,
    int64_t cap_rows, int32_t* __restrict__ offsets,
    uint8_t* __restrict__ a_perm, float* __restrict__ a_perm_s, int32_t* __restrict__ inv_perm,
    int32_t* __restrict__ row_src) {
    constexpr int kWaves = kPermThreads / kWave;
    constexpr int kBatch = 8;
    constexpr int kSelfLoads = 16;                                  // SELF: at most 16 * 256 pairs
    constexpr int kExPerThread = kMaxLocalExperts / kPermThreads;   // experts 4 * tid + j
    constexpr int kMapPerThread = GMAP ? 1 : kMapLds / kPermThreads;
    __shared__ int wcnt[kWaves][kMaxLocalExperts];
    __shared__ int rowmap[kPermThreads];
    __shared__ float s_tw[kPermThreads];       // the block's router weights (apply_on_input)
    __shared__ int s_off[kMaxLocalExperts + 1];
    __shared__ int s_wsum[kWaves];
    __shared__ int s_cnt[kMaxLocalExperts];    // the counts
    __shared__ int s_base[kMaxLocalExperts];   // pairs of each expert before this block
    __shared__ int s_map[GMAP ? 1 : kMapLds + 1];   // expert_map, when there is one; [kMapLds] = -1
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    // every argument and grid size in SGPRs here, all loaded together: the
    // compiler would otherwise load each just before its first use, and at a
    // kernel's start each such load waits for a scalar-cache miss
    const unsigned grid_x = gridDim.x, grid_y = gridDim.y;
    asm volatile("" ::"s"(a_q), "s"(a_s), "s"(x), "s"(ids), "s"(topk_w), "s"(apply_on_input), "s"(Mc), "s"(K),
                 "s"(topk), "s"(tpb), "s"(emap), "s"(Eg), "s"(El), "s"(nbits), "s"(base));
    asm volatile("" ::"s"(counts), "s"(counts_copy), "s"(align), "s"(cap_rows), "s"(offsets), "s"(a_perm),
                 "s"(a_perm_s), "s"(inv_perm), "s"(row_src), "s"(grid_x), "s"(grid_y));
    // the fill constants at a per-lane offset the compiler cannot see is
    // zero: read with vector loads, which it counts with the others, rather
    // than as scalar loads of a uniform address
    int vzero = 0;
    asm volatile("" : "+v"(vzero));
    const int32_t* f_neg1 = g_fill_neg1 + vzero;
    const int32_t* f_zero = g_fill_zero + vzero;
    const float* f_one = g_fill_one + vzero;
    const void* f_zero16 = g_fill_zero16 + vzero;

    // ---- every global read, issued before the first wait and none of them
    // conditional (an item past the end reads one of the fill constants
    // instead), so that the compiler knows how many loads follow each one
    // and a wait covers only the loads it needs: the rows, loaded last, are
    // still in flight while the count, scan and rank run
    const int64_t t0 = (int64_t)blockIdx.x * tpb;
    const int ntok = (int)((Mc - t0) < tpb ? (Mc - t0) : tpb);
    const int npairs = ntok * topk;
    const int i = threadIdx.x;
    const bool active = i < npairs;
    const int64_t f = t0 * topk + i;
    const int own_id = *(active ? ids + f : f_neg1);
    const float own_w = *(active && apply_on_input ? topk_w + f : f_one);
    const int64_t np = Mc * topk;
    int sid[SELF ? kSelfLoads : 1];
    int cb[2][SELF ? 1 : kExPerThread];   // not SELF: counts and this block's row bases
    if constexpr (SELF) {
#pragma unroll
        for (int u = 0; u < kSelfLoads; ++u) {
            const int64_t f2 = threadIdx.x + (int64_t)u * kPermThreads;
            sid[u] = *(f2 < np ? ids + f2 : f_neg1);
        }
    } else {
#pragma unroll
        for (int j = 0; j < kExPerThread; ++j) {
            const int ex = threadIdx.x * kExPerThread + j;
            cb[0][j] = *(ex < El ? counts + ex : f_zero);
            cb[1][j] = *(ex < El ? base + (int64_t)blockIdx.x * El + ex : f_zero);
        }
    }
    int mv[kMapPerThread];
    if constexpr (!GMAP) {
#pragma unroll
        for (int m = 0; m < kMapPerThread; ++m) {
            const int j = threadIdx.x + m * kPermThreads;
            mv[m] = *(emap != nullptr && j < Eg ? emap + j : f_neg1);
        }
    }
    // this block's slice of the K groups: [g_lo, g_lo + ng)
    const int kg = K / kGroup;
    const int gps = (kg + (int)grid_y - 1) / (int)grid_y;
    const int g_lo = min(kg, (int)blockIdx.y * gps);
    const int ng = min(kg, g_lo + gps) - g_lo;
    const int my_tokens = ntok > wave ? (ntok - wave + kWaves - 1) / kWaves : 0;
    // QUANT: each wave takes every fourth token of the block; 16 lanes hold
    // one 128-group (8 bf16 each), so a wave-wide load covers 4 (token,
    // group) items of the wave's tokens and the block's groups.  Copies:
    // (token, 16-byte chunk) items over the wave's tokens and the block's
    // 8 * ng chunks, one per lane.  Up to kBatch loads per lane are in flight.
    const int sub = lane & 15;
    const int nch = ng * (kGroup / 16);
    const int c_lo = g_lo * (kGroup / 16);
    const int items = QUANT ? my_tokens * ng : my_tokens * nch;
    const int istep = QUANT ? 4 * kBatch : kWave * kBatch;
    auto item = [&](int q0, int u, int& tl, int& gc) __attribute__((always_inline)) {
        const int q = QUANT ? q0 + 4 * u + (lane >> 4) : q0 + u * kWave + lane;
        const int per = QUANT ? ng : nch;
        tl = wave + (q / per) * kWaves;
        gc = (QUANT ? g_lo : c_lo) + q % per;
        return q;
    };
    auto load_batch = [&](int q0, uint4 (&v)[kBatch]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            int tl, gc;
            const int q = item(q0, u, tl, gc);
            const void* src = f_zero16;
            if constexpr (QUANT) {
                if (q < items) src = x + (t0 + tl) * K + (int64_t)gc * kGroup + sub * 8;
            } else {
                if (q < items) src = a_q + (t0 + tl) * K + (int64_t)gc * 16;
            }
            v[u] = load_once16(src);
        }
    };
    // QUANT: codes and scales of a batch (every lane quantises, zeros past
    // the end, so the group max always runs on whole 16-lane groups)
    uint2 codes[kBatch];
    float scale[kBatch];
    auto quant_batch = [&](int q0, const uint4 (&v)[kBatch]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (q0 + 4 * u >= items) break;   // no item of this wave left (wave-uniform)
            float fv[8];
            bf16x8_to_f32(v[u], fv);
            scale[u] = quant_group16(fv, codes[u]);
        }
    };
    uint4 v[kBatch];
    load_batch(0, v);

    // ---- LDS set-up from what was read
    if constexpr (!GMAP) {
        if (emap != nullptr) {
#pragma unroll
            for (int m = 0; m < kMapPerThread; ++m) {
                const int j = threadIdx.x + m * kPermThreads;
                if (j < Eg) s_map[j] = mv[m];
            }
        }
        if (threadIdx.x == 0) s_map[kMapLds] = -1;
    }
    for (int j = threadIdx.x; j < kWaves * El; j += kPermThreads) wcnt[j / El][j % El] = 0;
#pragma unroll
    for (int j = 0; j < kExPerThread; ++j) {
        const int ex = threadIdx.x * kExPerThread + j;
        if (ex < El) {
            s_cnt[ex] = SELF ? 0 : cb[0][SELF ? 0 : j];
            s_base[ex] = SELF ? 0 : cb[1][SELF ? 0 : j];
        }
    }
    s_tw[i] = own_w;
    // local expert of a global id, -1 when out of range or not local; with
    // the map in LDS the read is unconditional (out-of-range ids read the
    // -1 past its end), so lookups do not wait on one another
    const bool has_map = emap != nullptr;
    auto loc = [&](int id) __attribute__((always_inline)) {
        const bool in = (unsigned)id < (unsigned)Eg;
        int ex;
        if constexpr (GMAP) {
            ex = in ? emap[id] : -1;
        } else {
            const int m = s_map[in && has_map ? id : kMapLds];
            ex = has_map ? m : (in ? id : -1);
        }
        return (unsigned)ex < (unsigned)El ? ex : -1;
    };
    __syncthreads();   // s_map, wcnt, s_cnt, s_base, s_tw ready
    if constexpr (SELF) {
        // few pairs: every block counts them all
        const int64_t mine = (int64_t)blockIdx.x * tpb * topk;   // this block's first pair
        int exu[kSelfLoads];   // every map lookup before the first add
#pragma unroll
        for (int u = 0; u < kSelfLoads; ++u) exu[u] = loc(sid[u]);
#pragma unroll
        for (int u = 0; u < kSelfLoads; ++u) {
            const int64_t f2 = threadIdx.x + (int64_t)u * kPermThreads;
            if (exu[u] >= 0) {
                atomicAdd(&s_cnt[exu[u]], 1);
                if (f2 < mine) atomicAdd(&s_base[exu[u]], 1);
            }
        }
        __syncthreads();
    }

    // aligned segment offsets: exclusive scan of align * ceil(counts / align)
    // over the experts, four experts per thread
    {
        int seg[kExPerThread], tsum = 0;
#pragma unroll
        for (int j = 0; j < kExPerThread; ++j) {
            const int ex = threadIdx.x * kExPerThread + j;
            const int c = ex < El ? s_cnt[ex] : 0;
            seg[j] = ((c + align - 1) / align) * align;
            tsum += seg[j];
        }
        const int incl = wave_inclusive_scan(tsum);
        if (lane == kWave - 1) s_wsum[wave] = incl;
        __syncthreads();
        int run = incl - tsum;
        for (int w = 0; w < wave; ++w) run += s_wsum[w];
#pragma unroll
        for (int j = 0; j < kExPerThread; ++j) {
            const int ex = threadIdx.x * kExPerThread + j;
            if (ex < El) s_off[ex] = run;
            run += seg[j];
        }
        if (threadIdx.x == kPermThreads - 1) s_off[El] = run;
    }
    // lanes of this wave with the same expert (multisplit over the id bits)
    const int e = active ? loc(own_id) : -1;
    uint64_t peers = ballot(e >= 0);
    for (int bit = 0; bit < nbits; ++bit) {
        const bool b = (e >> bit) & 1;
        const uint64_t m = ballot(b);
        peers &= b ? m : ~m;
    }
    const int rank_w = __popcll(peers & lanemask_lt());
    if (e >= 0 && rank_w == 0) wcnt[wave][e] = __popcll(peers);
    __syncthreads();   // s_off, wcnt ready
    int row = -1;
    if (e >= 0) {
        int pre = 0;
        for (int w = 0; w < wave; ++w) pre += wcnt[w][e];
        row = s_off[e] + s_base[e] + pre + rank_w;
    }
    if (active) rowmap[i] = row;
    if constexpr (QUANT) quant_batch(0, v);   // its loads flew during the count, scan and rank
    __syncthreads();   // rowmap ready

    // ---- the stores
    {   // block (0, 0) publishes the counts and offsets; all blocks share the
        // padding marks (one wave per expert, its lanes on consecutive
        // padding rows) and the rows past the last segment
        const int nblocks = (int)(grid_x * grid_y);
        const int bid = (int)(blockIdx.y * grid_x + blockIdx.x);
        if (bid == 0) {
            for (int ex = threadIdx.x; ex <= El; ex += kPermThreads) offsets[ex] = s_off[ex];
            if (SELF)
                for (int ex = threadIdx.x; ex < El; ex += kPermThreads) {
                    counts[ex] = s_cnt[ex];
                    if (counts_copy) counts_copy[ex] = s_cnt[ex];
                }
        }
        if (active && blockIdx.y == 0) {
            inv_perm[f] = row;
            if (row >= 0) row_src[row] = (int32_t)(t0 + i / topk);
        }
        for (int ex = bid * kWaves + wave; ex < El; ex += nblocks * kWaves) {
            const int pad_lo = s_off[ex] + s_cnt[ex];
            for (int r = pad_lo + lane; r < s_off[ex + 1]; r += kWave) row_src[r] = -1;
        }
        for (int64_t r = s_off[El] + (int64_t)bid * kPermThreads + threadIdx.x; r < cap_rows;
             r += (int64_t)nblocks * kPermThreads)
            row_src[r] = -1;
    }
    // the row copies, batch 0 already loaded (and quantised)
    for (int q0 = 0; q0 < items; q0 += istep) {
        if (q0 > 0) {
            load_batch(q0, v);
            if constexpr (QUANT) quant_batch(q0, v);
        }
        if constexpr (QUANT) {
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (q0 + 4 * u >= items) break;   // no item of this wave left (wave-uniform)
                int tl, g;
                const int q = item(q0, u, tl, g);
                if (q < items) {
                    const int* rm = rowmap + tl * topk;
                    for (int k = 0; k < topk; ++k) {
                        const int r = rm[k];
                        if (r >= 0) {
                            *reinterpret_cast<uint2*>(a_perm + (int64_t)r * K + (int64_t)g * kGroup + sub * 8) =
                                codes[u];
                            if (sub == 0)
                                a_perm_s[(int64_t)r * kg + g] =
                                    apply_on_input ? scale[u] * s_tw[tl * topk + k] : scale[u];
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (q0 + u * kWave >= items) break;   // no item of this wave left (wave-uniform)
                int tl, c;
                const int q = item(q0, u, tl, c);
                if (q < items) {
                    const int* rm = rowmap + tl * topk;
                    for (int k = 0; k < topk; ++k) {
                        const int r = rm[k];
                        if (r >= 0) *reinterpret_cast<uint4*>(a_perm + (int64_t)r * K + (int64_t)c * 16) = v[u];
                    }
                }
            }
        }
    }
    if constexpr (!QUANT) {
        for (int tl = wave; tl < ntok; tl += kWaves) {
            const int64_t t = t0 + tl;
            const int* rm = rowmap + tl * topk;
            for (int g = g_lo + lane; g < g_lo + ng; g += kWave) {
                const float s = a_s[t * kg + g];
                for (int k = 0; k < topk; ++k) {
                    const int r = rm[k];
                    if (r >= 0) a_perm_s[(int64_t)r * kg + g] = apply_on_input ? s * s_tw[tl * topk + k] : s;
                }
            }
        }
    }
}

// Up to 16 pair blocks (4096 pairs) every scatter block reads all the ids
// itself for the counts and its per-expert row bases, which saves the
// histogram and column-scan launches; beyond that the reads would grow with
// the square of the pair count.
int permute_self_count(int64_t nblk) { return nblk <= 16 ? 1 : 0; }

// (pair blocks, K slices): at least one block, so that the offsets and
// padding marks are written even for an empty chunk; the rows are split
// along K into about 1024 blocks in all, at least 4 slices (but at most
// 2048 blocks) and at most one slice per group.  Measured on 2048-wide
// tokens with topk 8: the best slice counts were 16 at 32 and 64 pair
// blocks, 8 at 128, 4 at 256 and 512 (16384 tokens: 0.095 ms with 1 slice,
// 0.089 with 4, 0.094 with 8).
dim3 scatter_grid(int64_t nblk, int K) {
    const int64_t bx = nblk > 0 ? nblk : 1;
    const int64_t kg = K / kGroup;
    int64_t lo = 2048 / bx;
    lo = lo < 1 ? 1 : (lo > 4 ? 4 : lo);
    int64_t by = 1024 / bx;
    by = by < lo ? lo : by;
    by = by > kg ? kg : by;
    const int64_t gps = (kg + by - 1) / by;   // groups per slice; no slice left empty
    return dim3((unsigned)bx, (unsigned)((kg + gps - 1) / gps), 1);
}

int bits_for(int El) {
    int b = 0;
    while ((1 << b) < El) ++b;
    return b;
}

template <bool QUANT>
auto scatter_kernel(bool gmap, int self) {
    if (gmap) return self ? k_permute_scatter<QUANT, true, true> : k_permute_scatter<QUANT, true, false>;
    return self ? k_permute_scatter<QUANT, false, true> : k_permute_scatter<QUANT, false, false>;
}

}  // namespace

hipError_t launch_slot_offsets(const int32_t* counts, int El, int64_t max_tokens, int32_t* offsets, int32_t* cut,
                               hipStream_t s) {
    k_slot_offsets<<<(unsigned)((El + 256) / 256), 256, 0, s>>>(counts, El, max_tokens, offsets, cut);
    return hipGetLastError();
}

hipError_t launch_count(const int32_t* ids, int64_t num_pairs, const int32_t* emap, int Eg, int El,
                        int32_t* counts, int32_t* invalid, int num_cus, hipStream_t s) {
    k_count_clear<<<1, 256, 0, s>>>(counts, El, invalid);
    if (num_pairs > 0) {
        // one 16-byte vector per lane until every CU has a block (small
        // counts are latency-bound: the more lanes load at once the better),
        // then at most one block per CU, each lane striding over the rest
        const int64_t nvec = num_pairs / 4;
        int64_t blocks = (nvec + kCountThreads - 1) / kCountThreads;
        if (blocks < 1) blocks = 1;
        if (blocks > num_cus) blocks = num_cus;
        const int pack64 = ((uintptr_t)counts & 7u) == 0 && num_pairs <= INT32_MAX;
        const int sl = count_slots_log2(El);
        if (emap == nullptr)
            k_count<kCountMapNone><<<(unsigned)blocks, kCountThreads, 0, s>>>(ids, num_pairs, emap, Eg, El, sl, pack64,
                                                                         counts, invalid);
        else if (Eg <= kMapLds)
            k_count<kCountMapLds><<<(unsigned)blocks, kCountThreads, 0, s>>>(ids, num_pairs, emap, Eg, El, sl, pack64,
                                                                        counts, invalid);
        else
            k_count<kCountMapGlobal><<<(unsigned)blocks, kCountThreads, 0, s>>>(ids, num_pairs, emap, Eg, El, sl, pack64,
                                                                           counts, invalid);
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
    const int self = permute_self_count(nblk);
    if (!self) {
        k_permute_hist<<<(unsigned)nblk, kPermThreads, 0, s>>>(ids, Mc, topk, tpb, emap, Eg, El, hist);
        k_permute_colscan<<<(unsigned)El, kScanThreads, 0, s>>>(hist, (int)nblk, El, counts, counts_copy);
    }
    auto* kern = scatter_kernel<false>(emap != nullptr && Eg > kMapLds, self);
    kern<<<scatter_grid(nblk, K), kPermThreads, 0, s>>>(
        a_q, a_s, nullptr, ids, topk_w, apply_on_input, Mc, K, topk, tpb, emap, Eg, El, bits_for(El), hist,
        counts, counts_copy, align, cap_rows, offsets, a_perm, a_perm_s, inv_perm, row_src);
    return hipGetLastError();
}

hipError_t launch_quant_permute(const uint16_t* x, const int32_t* ids, const float* topk_w, int apply_on_input,
                                int64_t Mc, int K, int topk, const int32_t* emap, int Eg, int El, int align,
                                int64_t cap_rows, uint8_t* a_perm, float* a_perm_s, int32_t* counts,
                                int32_t* offsets, int32_t* inv_perm, int32_t* row_src, int32_t* hist,
                                int32_t* counts_copy, hipStream_t s) {
    const int tpb = permute_tokens_per_block(topk);
    const int64_t nblk = permute_num_blocks(Mc, topk);
    const int self = permute_self_count(nblk);
    if (!self) {
        k_permute_hist<<<(unsigned)nblk, kPermThreads, 0, s>>>(ids, Mc, topk, tpb, emap, Eg, El, hist);
        k_permute_colscan<<<(unsigned)El, kScanThreads, 0, s>>>(hist, (int)nblk, El, counts, counts_copy);
    }
    auto* kern = scatter_kernel<true>(emap != nullptr && Eg > kMapLds, self);
    kern<<<scatter_grid(nblk, K), kPermThreads, 0, s>>>(
        nullptr, nullptr, x, ids, topk_w, apply_on_input, Mc, K, topk, tpb, emap, Eg, El, bits_for(El), hist,
        counts, counts_copy, align, cap_rows, offsets, a_perm, a_perm_s, inv_perm, row_src);
    return hipGetLastError();
}

}  // namespace moe
