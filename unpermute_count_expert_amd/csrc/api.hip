// api.hip -- the C ABI of include/moe.h: host-side validation, the workspace
// plan and the chunk loop of the MoE expert pipeline on gfx950.
//
// Every entry point validates its arguments before enqueuing anything, so a
// bad call leaves the stream untouched.  Nothing here allocates, frees or
// synchronises device memory.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "moe.h"
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_dev_cus[kMaxDevices];

// Confirms the current device is gfx950 (cached per device) and returns its
// compute-unit count through *cus.
int check_device(int* cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED_DEVICE, "device %d", dev);
    int st = g_dev_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return fail(MOE_ERR_HIP, "hipGetDeviceProperties failed");
        const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
        st = ok ? 1 : 2;
        g_dev_state[dev].store(st, std::memory_order_release);
    }
    if (st != 1) return fail(MOE_ERR_UNSUPPORTED_DEVICE, "device %d is not gfx950", dev);
    if (cus) *cus = g_dev_cus[dev].load(std::memory_order_relaxed);
    return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, status, ...) \
    do {                           \
        if (!(cond)) return fail(status, __VA_ARGS__); \
    } while (0)

#define REQUIRE_PTR(p) \
    REQUIRE((p) != nullptr && aligned16(p), MOE_ERR_INVALID_ARG, "%s must be a non-null 16-byte aligned device pointer", #p)

#define HIP_OK(expr)                                                                   \
    do {                                                                               \
        hipError_t e_ = (expr);                                                        \
        if (e_ != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

bool valid_align(int a) { return a == 16 || a == 32 || a == 64 || a == 128; }

int64_t max_rows(int64_t Mc, int32_t topk, int32_t El, int32_t align) {
    if (Mc < 0 || topk <= 0 || El <= 0 || !valid_align(align)) return -1;
    const int64_t p = Mc * topk;
    const int64_t ne = p < El ? p : El;
    return p + ne * (align - 1);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na && nb && x < y + nb && y < x + na;
}

size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

// The forward workspace, carved once for the largest chunk and reused by all.
//   bufA   a_perm [cap,K] then act_q [cap,N]          (e4m3)
//   bufAs  a_perm_s then act_s                         (fp32 scales)
//   bufB   h [cap,2N], then y [cap,K]                  (bf16)
//   small  counts, offsets, inv_perm, row_src, per-block histogram
//   part   fp32 partial sums of a GEMM with K split, [S, pairs, n]
//   info   the two split GEMMs' segment counts S
// The input quantisation is fused into the permute's scatter, so no a_q /
// a_s buffer exists.  Each buffer is dead before it is reused: GEMM w13
// reads bufA and writes bufB, the SiLU-mul requant reads bufB and writes
// bufA, GEMM w2 reads bufA and writes bufB, the unpermute reads bufB.  The
// output never aliases the workspace.  Every slice is followed by a guard
// band of kGuard bytes that no kernel touches, so a write past a slice's end
// is visible to a caller that fills the workspace with a pattern first.
//
// Small chunks (at most 64 routed rows per expert on average) take the
// GEMMs on 64-row tiles (launch_grouped_gemm_small).  Their tiles are too
// few to spread evenly over the CUs (64 tokens, topk 8: ~300 tiles of w13
// on 256 CUs, two rounds with the second a quarter full), so a GEMM whose K
// holds 16 groups or more also cuts K into segments of at least 8 groups:
// h (or y) then passes through part as fp32 partial sums, which the
// SiLU-mul requant (or the unpermute) adds up in a fixed order, and bufB is
// not used for it.  The cut is planned where the partials of the largest
// chunk fit in kPartBudget bytes; the GEMM keeps K whole when its tiles
// fill four rounds of the grid or more.
//
// Lanes: with two chunks or more, consecutive chunks alternate between two
// copies of these slices (lane c % 2, the second at offset `one`) and two
// library streams that fork from and join the caller's stream.  Chunk c + 1
// then runs its kernels beside chunk c's: its permute and its GEMM's first
// tiles fill the CUs that chunk c's last partial round of tiles, its
// SiLU-mul requant and its unpermute leave idle.  Every chunk computes
// exactly what it computes alone.
constexpr size_t kGuard = 256;
constexpr int kSlices = 10;
constexpr size_t kPartBudget = size_t(64) << 20;
// Chunk lanes: consecutive chunks go round-robin to this many library streams,
// each with its own copy of the workspace slices, so that one chunk's
// latency-bound kernels overlap the next chunks' work.  Three: HIP gives a
// process four hardware queues by default, one of them the caller's stream;
// with a fourth lane two streams share a queue and serialise.  Measured
// (ms; 2, 3, 4 lanes): 8192 tokens in chunks of 64, 6.06 / 4.82 / 6.07;
// 16384 tokens in chunks of 512, 4.23 / 3.94 / 4.17, of 2048, 1.670 / 1.657 /
// 1.684 (one lane: 4.85 and 1.85).
constexpr int kLanes = 3;

struct Plan {
    int64_t cs, cap, nblk;
    int lanes;               // 1, or min(chunks, kLanes) with two chunks or more
    size_t one;              // bytes of one lane's slices
    size_t bufA, bufAs, bufB, counts, offsets, inv, rsrc, hist, part, info, total;
    bool small;              // the GEMMs on 64-row tiles
    int64_t part_rows;       // pairs of the largest chunk, 0 without a split
    int smax13, smax2;       // K segments of GEMM w13 and w2 (1: not split)
    size_t off[kSlices], len[kSlices];   // the slices above, in this order
};

Plan make_plan(const moe_problem& p, bool allow_lanes = true) {
    Plan pl{};
    pl.cs = (p.chunk_size <= 0 || p.chunk_size >= p.M) ? p.M : p.chunk_size;
    if (pl.cs < 1) pl.cs = 1;
    pl.cap = max_rows(pl.cs, p.topk, p.num_local_experts, p.align);
    pl.nblk = moe::permute_num_blocks(pl.cs, p.topk);
    const int64_t K = p.K, N = p.N, El = p.num_local_experts;
    const int64_t wA = K > N ? K : N;
    const int64_t wB = (2 * N > K ? 2 * N : K) * 2;
    // the split: the segments of gemm_split_segments, fewer (still dividing
    // K / 128) where the budget holds fewer partials
    const int64_t pairs = pl.cs * p.topk;
    pl.small = moe::gemm_small_chunk(pairs, (int)El, p.num_global_experts, (int)(2 * N));
    auto segments = [&](int k_in, int64_t n) {
        if (!pl.small) return 1;
        const int64_t fit = (int64_t)(kPartBudget / ((size_t)pairs * (size_t)n * 4));
        int sm = moe::gemm_split_segments(k_in);
        while (sm > 1 && (sm > fit || (k_in / moe::kGroup) % sm != 0)) --sm;
        return sm;
    };
    pl.smax13 = segments((int)K, 2 * N);
    pl.smax2 = segments((int)N, K);
    pl.part_rows = (pl.smax13 > 1 || pl.smax2 > 1) ? pairs : 0;
    const int64_t part_w = (pl.smax13 * 2 * N > pl.smax2 * K) ? pl.smax13 * 2 * N : pl.smax2 * K;
    const size_t len[kSlices] = {
        (size_t)pl.cap * wA,                        // bufA
        (size_t)pl.cap * (wA / moe::kGroup) * 4,    // bufAs
        (size_t)pl.cap * wB,                        // bufB
        (size_t)El * 4,                             // counts
        (size_t)(El + 1) * 4,                       // offsets
        (size_t)pl.cs * p.topk * 4,                 // inv_perm
        (size_t)pl.cap * 4,                         // row_src
        (size_t)pl.nblk * El * 4,                   // histogram
        (size_t)pl.part_rows * part_w * 4,          // partial sums
        (size_t)2 * 4,                              // split counts
    };
    size_t off = 0;
    for (int i = 0; i < kSlices; ++i) {
        pl.off[i] = off;
        pl.len[i] = len[i];
        off += up256(len[i]) + kGuard;
    }
    pl.bufA = pl.off[0];
    pl.bufAs = pl.off[1];
    pl.bufB = pl.off[2];
    pl.counts = pl.off[3];
    pl.offsets = pl.off[4];
    pl.inv = pl.off[5];
    pl.rsrc = pl.off[6];
    pl.hist = pl.off[7];
    pl.part = pl.off[8];
    pl.info = pl.off[9];
    pl.one = off;
    const int64_t nchunks = (p.M + pl.cs - 1) / pl.cs;
    pl.lanes = (allow_lanes && nchunks > 1) ? (int)(nchunks < kLanes ? nchunks : kLanes) : 1;
    pl.total = off * pl.lanes;
    return pl;
}

int check_problem(const moe_problem* p) {
    REQUIRE(p != nullptr, MOE_ERR_INVALID_ARG, "problem is NULL");
    REQUIRE(p->M >= 0, MOE_ERR_SHAPE, "M=%lld < 0", (long long)p->M);
    REQUIRE(p->K > 0 && p->K % moe::kGroup == 0 && p->K <= 65536, MOE_ERR_SHAPE,
            "K=%d is not a positive multiple of 128 up to 65536", p->K);
    REQUIRE(p->N > 0 && p->N % moe::kGroup == 0 && p->N <= 32768, MOE_ERR_SHAPE,
            "N=%d is not a positive multiple of 128 up to 32768", p->N);
    REQUIRE(p->topk >= 1 && p->topk <= 256, MOE_ERR_SHAPE, "topk=%d outside [1,256]", p->topk);
    REQUIRE(p->num_global_experts >= 1, MOE_ERR_SHAPE, "Eg=%d", p->num_global_experts);
    REQUIRE(p->num_local_experts >= 1 && p->num_local_experts <= moe::kMaxLocalExperts, MOE_ERR_SHAPE,
            "El=%d outside [1,1024]", p->num_local_experts);
    REQUIRE(valid_align(p->align), MOE_ERR_SHAPE, "align=%d not in {16,32,64,128}", p->align);
    REQUIRE(p->apply_router_weight_on_input == 0 || p->apply_router_weight_on_input == 1,
            MOE_ERR_INVALID_ARG, "apply_router_weight_on_input=%d", p->apply_router_weight_on_input);
    const int64_t cs = (p->chunk_size <= 0 || p->chunk_size >= p->M) ? p->M : p->chunk_size;
    const int64_t cap = max_rows(cs > 0 ? cs : 1, p->topk, p->num_local_experts, p->align);
    REQUIRE(cs * p->topk < (int64_t(1) << 31) && cap < (int64_t(1) << 31), MOE_ERR_SHAPE,
            "chunk of %lld tokens x topk %d is too large", (long long)cs, p->topk);
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(int s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
        case MOE_ERR_UNSUPPORTED_DEVICE: return "MOE_ERR_UNSUPPORTED_DEVICE";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        default: return "MOE_ERR_UNKNOWN";
    }
}

const char* moe_last_error(void) { return g_err; }

int64_t moe_max_rows(int64_t Mc, int32_t topk, int32_t El, int32_t align) {
    return max_rows(Mc, topk, El, align);
}

int32_t moe_grouped_gemm_tile_rows(int64_t rows_hint, int32_t El) {
    return El < 1 ? -1 : moe::gemm_tile_rows(rows_hint, El);
}

int moe_forward_workspace_size(const moe_problem* p, size_t* bytes) {
    int st = check_problem(p);
    if (st) return st;
    REQUIRE(bytes != nullptr, MOE_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = make_plan(*p).total;
    return MOE_OK;
}

int moe_forward_workspace_slices(const moe_problem* p, size_t* offsets, size_t* bytes, int32_t max_slices,
                                 int32_t* num_slices) {
    int st = check_problem(p);
    if (st) return st;
    REQUIRE(num_slices != nullptr, MOE_ERR_INVALID_ARG, "num_slices is NULL");
    REQUIRE(max_slices >= 0 && (max_slices == 0 || (offsets != nullptr && bytes != nullptr)),
            MOE_ERR_INVALID_ARG, "offsets / bytes are NULL");
    const Plan pl = make_plan(*p);
    *num_slices = kSlices * pl.lanes;
    for (int i = 0; i < kSlices * pl.lanes && i < max_slices; ++i) {
        offsets[i] = (size_t)(i / kSlices) * pl.one + pl.off[i % kSlices];
        bytes[i] = pl.len[i % kSlices];
    }
    return MOE_OK;
}

int moe_permute_workspace_size(int64_t Mc, int32_t topk, int32_t El, size_t* bytes) {
    REQUIRE(bytes != nullptr, MOE_ERR_INVALID_ARG, "bytes is NULL");
    REQUIRE(Mc >= 0 && topk >= 1 && topk <= 256 && El >= 1 && El <= moe::kMaxLocalExperts, MOE_ERR_SHAPE,
            "Mc=%lld topk=%d El=%d", (long long)Mc, topk, El);
    *bytes = up256((size_t)moe::permute_num_blocks(Mc, topk) * El * 4);
    if (*bytes == 0) *bytes = 256;
    return MOE_OK;
}

int moe_count(const int32_t* topk_ids, int64_t num_pairs, const int32_t* expert_map, int32_t Eg,
              int32_t El, int32_t* counts, int32_t* invalid_ids, void* stream) {
    REQUIRE(num_pairs >= 0, MOE_ERR_SHAPE, "num_pairs < 0");
    REQUIRE(Eg >= 1 && El >= 1 && El <= moe::kMaxLocalExperts, MOE_ERR_SHAPE, "Eg=%d El=%d", Eg, El);
    REQUIRE(expert_map != nullptr || El <= Eg, MOE_ERR_SHAPE, "El > Eg without an expert map");
    if (num_pairs > 0) REQUIRE_PTR(topk_ids);
    REQUIRE(counts != nullptr && ((uintptr_t)counts & 3u) == 0, MOE_ERR_INVALID_ARG, "counts");
    REQUIRE(expert_map == nullptr || ((uintptr_t)expert_map & 3u) == 0, MOE_ERR_INVALID_ARG, "expert_map");
    REQUIRE(invalid_ids == nullptr || ((uintptr_t)invalid_ids & 3u) == 0, MOE_ERR_INVALID_ARG, "invalid_ids");
    int cus = 0;
    int st = check_device(&cus);
    if (st) return st;
    HIP_OK(moe::launch_count(topk_ids, num_pairs, expert_map, Eg, El, counts, invalid_ids, cus,
                             static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

}  // extern "C"

namespace {

// moe_permute (quant false: a_q / a_s given) and moe_quant_permute (quant
// true: x given): the same checks, then the launch
int permute_common(bool quant, const uint8_t* a_q, const float* a_s, const uint16_t* x, const int32_t* topk_ids,
                   const float* topk_weights, int32_t apply_on_input, int64_t Mc, int32_t K, int32_t topk,
                   const int32_t* expert_map, int32_t Eg, int32_t El, int32_t align, int64_t cap_rows,
                   uint8_t* a_perm, float* a_perm_s, int32_t* counts, int32_t* expert_offsets,
                   int32_t* inv_perm, int32_t* row_src, void* workspace, size_t workspace_bytes,
                   void* stream) {
    REQUIRE(Mc >= 0, MOE_ERR_SHAPE, "Mc < 0");
    REQUIRE(K > 0 && K % moe::kGroup == 0, MOE_ERR_SHAPE, "K=%d is not a positive multiple of 128", K);
    REQUIRE(topk >= 1 && topk <= 256, MOE_ERR_SHAPE, "topk=%d outside [1,256]", topk);
    REQUIRE(Eg >= 1 && El >= 1 && El <= moe::kMaxLocalExperts, MOE_ERR_SHAPE, "Eg=%d El=%d", Eg, El);
    REQUIRE(expert_map != nullptr || El <= Eg, MOE_ERR_SHAPE, "El > Eg without an expert map");
    REQUIRE(valid_align(align), MOE_ERR_SHAPE, "align=%d not in {16,32,64,128}", align);
    REQUIRE(apply_on_input == 0 || apply_on_input == 1, MOE_ERR_INVALID_ARG, "apply_on_input=%d", apply_on_input);
    REQUIRE(Mc * topk < (int64_t(1) << 31) && cap_rows < (int64_t(1) << 31), MOE_ERR_SHAPE, "too many rows");
    const int64_t need_rows = max_rows(Mc, topk, El, align);
    REQUIRE(cap_rows >= need_rows, MOE_ERR_WORKSPACE_TOO_SMALL, "cap_rows=%lld < %lld",
            (long long)cap_rows, (long long)need_rows);
    size_t need_ws = 0;
    moe_permute_workspace_size(Mc, topk, El, &need_ws);
    REQUIRE(workspace_bytes >= need_ws, MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes",
            workspace_bytes, need_ws);
    REQUIRE_PTR(workspace);
    REQUIRE_PTR(counts);
    REQUIRE_PTR(expert_offsets);
    if (cap_rows > 0) REQUIRE_PTR(row_src);
    if (Mc > 0) {
        if (quant) {
            REQUIRE_PTR(x);
            REQUIRE(aligned16(x), MOE_ERR_INVALID_ARG, "x is not 16-byte aligned");
        } else {
            REQUIRE_PTR(a_q);
            REQUIRE_PTR(a_s);
        }
        REQUIRE_PTR(topk_ids);
        REQUIRE_PTR(a_perm);
        REQUIRE_PTR(a_perm_s);
        REQUIRE_PTR(inv_perm);
        if (apply_on_input) REQUIRE_PTR(topk_weights);
    }
    REQUIRE(expert_map == nullptr || aligned16(expert_map), MOE_ERR_INVALID_ARG, "expert_map alignment");
    int st = check_device(nullptr);
    if (st) return st;
    if (quant)
        HIP_OK(moe::launch_quant_permute(x, topk_ids, topk_weights, apply_on_input, Mc, K, topk, expert_map, Eg,
                                         El, align, cap_rows, a_perm, a_perm_s, counts, expert_offsets, inv_perm,
                                         row_src, static_cast<int32_t*>(workspace), nullptr,
                                         static_cast<hipStream_t>(stream)));
    else
        HIP_OK(moe::launch_permute(a_q, a_s, topk_ids, topk_weights, apply_on_input, Mc, K, topk, expert_map,
                                   Eg, El, align, cap_rows, a_perm, a_perm_s, counts, expert_offsets, inv_perm,
                                   row_src, static_cast<int32_t*>(workspace), nullptr,
                                   static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_permute(const uint8_t* a_q, const float* a_s, const int32_t* topk_ids,
                const float* topk_weights, int32_t apply_on_input, int64_t Mc, int32_t K,
                int32_t topk, const int32_t* expert_map, int32_t Eg, int32_t El, int32_t align,
                int64_t cap_rows, uint8_t* a_perm, float* a_perm_s, int32_t* counts,
                int32_t* expert_offsets, int32_t* inv_perm, int32_t* row_src, void* workspace,
                size_t workspace_bytes, void* stream) {
    if (Mc > 0) {
        REQUIRE_PTR(a_q);
        REQUIRE_PTR(a_s);
    }
    return permute_common(false, a_q, a_s, nullptr, topk_ids, topk_weights, apply_on_input, Mc, K, topk, expert_map,
                          Eg, El, align, cap_rows, a_perm, a_perm_s, counts, expert_offsets, inv_perm, row_src,
                          workspace, workspace_bytes, stream);
}

int moe_quant_permute(const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                      int32_t apply_on_input, int64_t Mc, int32_t K, int32_t topk, const int32_t* expert_map,
                      int32_t Eg, int32_t El, int32_t align, int64_t cap_rows, uint8_t* a_perm,
                      float* a_perm_s, int32_t* counts, int32_t* expert_offsets, int32_t* inv_perm,
                      int32_t* row_src, void* workspace, size_t workspace_bytes, void* stream) {
    if (Mc > 0) REQUIRE_PTR(x);
    return permute_common(true, nullptr, nullptr, x, topk_ids, topk_weights, apply_on_input, Mc, K, topk, expert_map,
                          Eg, El, align, cap_rows, a_perm, a_perm_s, counts, expert_offsets, inv_perm, row_src,
                          workspace, workspace_bytes, stream);
}

int moe_grouped_gemm_fp8(const uint8_t* a, const float* a_s, const uint8_t* w, const float* w_s,
                         const int32_t* expert_offsets, const int32_t* counts, int32_t El,
                         int64_t cap_rows, int32_t n_out, int32_t k_in, uint16_t* out,
                         void* stream) {
    REQUIRE(El >= 1 && El <= moe::kMaxLocalExperts, MOE_ERR_SHAPE, "El=%d outside [1,1024]", El);
    REQUIRE(n_out > 0 && n_out % moe::kGroup == 0 && n_out <= 65536, MOE_ERR_SHAPE,
            "n_out=%d is not a positive multiple of 128 up to 65536", n_out);
    REQUIRE(k_in > 0 && k_in % moe::kGroup == 0 && k_in <= 65536, MOE_ERR_SHAPE,
            "k_in=%d is not a positive multiple of 128 up to 65536", k_in);
    REQUIRE(cap_rows >= 0 && cap_rows < (int64_t(1) << 31), MOE_ERR_SHAPE, "cap_rows=%lld", (long long)cap_rows);
    if (cap_rows == 0) return MOE_OK;
    REQUIRE_PTR(a);
    REQUIRE_PTR(a_s);
    REQUIRE_PTR(w);
    REQUIRE_PTR(w_s);
    REQUIRE_PTR(expert_offsets);
    REQUIRE_PTR(counts);
    REQUIRE_PTR(out);
    int cus = 0;
    int st = check_device(&cus);
    if (st) return st;
    HIP_OK(moe::launch_grouped_gemm(a, a_s, w, w_s, expert_offsets, counts, El, cap_rows, n_out, k_in, out,
                                    moe::gemm_tile_rows(cap_rows, El), cus, static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

int moe_grouped_gemm_fp8_weight_reduce(const uint8_t* a, const float* a_s, const uint8_t* w, const float* w_s,
                                       const int32_t* expert_offsets, const int32_t* counts, int32_t El,
                                       int64_t cap_rows, int32_t n_out, int32_t k_in, const int32_t* row_src,
                                       const int32_t* inv_perm, const float* topk_weights, int32_t apply_on_input,
                                       int64_t Mc, int32_t topk, uint16_t* y, int32_t* counters, uint16_t* out,
                                       void* stream) {
    REQUIRE(El >= 1 && El <= moe::kMaxLocalExperts, MOE_ERR_SHAPE, "El=%d outside [1,1024]", El);
    REQUIRE(n_out > 0 && n_out % moe::kGroup == 0 && n_out <= 65536, MOE_ERR_SHAPE,
            "n_out=%d is not a positive multiple of 128 up to 65536", n_out);
    REQUIRE(k_in > 0 && k_in % moe::kGroup == 0 && k_in <= 65536, MOE_ERR_SHAPE,
            "k_in=%d is not a positive multiple of 128 up to 65536", k_in);
    REQUIRE(cap_rows >= 0 && cap_rows < (int64_t(1) << 31), MOE_ERR_SHAPE, "cap_rows=%lld", (long long)cap_rows);
    REQUIRE(Mc >= 0 && topk >= 1 && topk <= 256, MOE_ERR_SHAPE, "Mc=%lld topk=%d", (long long)Mc, topk);
    REQUIRE(apply_on_input == 0 || apply_on_input == 1, MOE_ERR_INVALID_ARG, "apply_on_input=%d", apply_on_input);
    if (Mc == 0) return MOE_OK;
    REQUIRE_PTR(inv_perm);
    REQUIRE_PTR(counters);
    REQUIRE_PTR(out);
    if (!apply_on_input) REQUIRE_PTR(topk_weights);
    if (cap_rows > 0) {
        REQUIRE_PTR(a);
        REQUIRE_PTR(a_s);
        REQUIRE_PTR(w);
        REQUIRE_PTR(w_s);
        REQUIRE_PTR(expert_offsets);
        REQUIRE_PTR(counts);
        REQUIRE_PTR(row_src);
        REQUIRE_PTR(y);
    }
    const size_t out_bytes = (size_t)Mc * n_out * 2;
    REQUIRE(!overlaps(out, out_bytes, y, (size_t)cap_rows * n_out * 2), MOE_ERR_INVALID_ARG, "out overlaps y");
    REQUIRE(!overlaps(counters, (size_t)Mc * ((n_out + 255) / 256) * 4, y, (size_t)cap_rows * n_out * 2),
            MOE_ERR_INVALID_ARG, "counters overlap y");
    int cus = 0;
    int st = check_device(&cus);
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    HIP_OK(moe::launch_reduce_prep(inv_perm, Mc, topk, cap_rows, n_out, counters, out, s));
    if (cap_rows > 0)
        HIP_OK(moe::launch_grouped_gemm_reduce(a, a_s, w, w_s, expert_offsets, counts, El, cap_rows, n_out, k_in, y,
                                               row_src, inv_perm, topk_weights, apply_on_input, Mc, topk, counters,
                                               out, moe::gemm_tile_rows(cap_rows, El), cus, s));
    return MOE_OK;
}

int moe_grouped_gemm_fp8_act_quant(const uint8_t* a, const float* a_s, const uint8_t* w13,
                                   const float* w13_s, const int32_t* expert_offsets,
                                   const int32_t* counts, int32_t El, int64_t cap_rows, int32_t N,
                                   int32_t k_in, uint8_t* q, float* q_s, void* stream) {
    REQUIRE(El >= 1 && El <= moe::kMaxLocalExperts, MOE_ERR_SHAPE, "El=%d outside [1,1024]", El);
    REQUIRE(N > 0 && N % moe::kGroup == 0 && N <= 32768, MOE_ERR_SHAPE,
            "N=%d is not a positive multiple of 128 up to 32768", N);
    REQUIRE(k_in > 0 && k_in % moe::kGroup == 0 && k_in <= 65536, MOE_ERR_SHAPE,
            "k_in=%d is not a positive multiple of 128 up to 65536", k_in);
    REQUIRE(cap_rows >= 0 && cap_rows < (int64_t(1) << 31), MOE_ERR_SHAPE, "cap_rows=%lld", (long long)cap_rows);
    if (cap_rows == 0) return MOE_OK;
    REQUIRE_PTR(a);
    REQUIRE_PTR(a_s);
    REQUIRE_PTR(w13);
    REQUIRE_PTR(w13_s);
    REQUIRE_PTR(expert_offsets);
    REQUIRE_PTR(counts);
    REQUIRE_PTR(q);
    REQUIRE_PTR(q_s);
    int cus = 0;
    int st = check_device(&cus);
    if (st) return st;
    HIP_OK(moe::launch_grouped_gemm_act(a, a_s, w13, w13_s, expert_offsets, counts, El, cap_rows, N, k_in, q,
                                        q_s, moe::gemm_tile_rows(cap_rows, El), cus,
                                        static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

int moe_act_quant(const uint16_t* in, int64_t rows, int32_t n, int32_t mode,
                  const int32_t* expert_offsets, const int32_t* counts, int32_t El, uint8_t* q,
                  float* q_s, void* stream) {
    REQUIRE(rows >= 0, MOE_ERR_SHAPE, "rows < 0");
    REQUIRE(n > 0 && n % moe::kGroup == 0, MOE_ERR_SHAPE, "n=%d is not a positive multiple of 128", n);
    REQUIRE(mode == MOE_ACT_IDENTITY || mode == MOE_ACT_SILU_MUL, MOE_ERR_INVALID_ARG, "mode=%d", mode);
    REQUIRE((expert_offsets == nullptr) == (counts == nullptr), MOE_ERR_INVALID_ARG,
            "expert_offsets and counts must both be given or both be NULL");
    if (expert_offsets) {
        REQUIRE(El >= 1 && El <= moe::kMaxLocalExperts, MOE_ERR_SHAPE, "El=%d outside [1,1024]", El);
        REQUIRE_PTR(expert_offsets);
        REQUIRE_PTR(counts);
    }
    if (rows == 0) return MOE_OK;
    REQUIRE_PTR(in);
    REQUIRE_PTR(q);
    REQUIRE_PTR(q_s);
    int st = check_device(nullptr);
    if (st) return st;
    HIP_OK(moe::launch_act_quant(in, rows, n, mode, expert_offsets, counts, El, q, q_s, rows,
                                 static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

int moe_unpermute_weight_reduce(const uint16_t* y, int64_t y_rows, const int32_t* inv_perm,
                                const float* topk_weights, int64_t Mc, int32_t K, int32_t topk,
                                int32_t apply_on_input, uint16_t* out, void* stream) {
    REQUIRE(Mc >= 0 && y_rows >= 0, MOE_ERR_SHAPE, "Mc / y_rows < 0");
    REQUIRE(K > 0 && K % moe::kGroup == 0, MOE_ERR_SHAPE, "K=%d is not a positive multiple of 128", K);
    REQUIRE(topk >= 1 && topk <= 256, MOE_ERR_SHAPE, "topk=%d outside [1,256]", topk);
    REQUIRE(apply_on_input == 0 || apply_on_input == 1, MOE_ERR_INVALID_ARG, "apply_on_input=%d", apply_on_input);
    if (Mc == 0) return MOE_OK;
    REQUIRE_PTR(inv_perm);
    REQUIRE_PTR(out);
    if (y_rows > 0) REQUIRE_PTR(y);
    if (!apply_on_input) REQUIRE_PTR(topk_weights);
    REQUIRE(!overlaps(out, (size_t)Mc * K * 2, y, (size_t)y_rows * K * 2), MOE_ERR_INVALID_ARG,
            "out overlaps y");
    int st = check_device(nullptr);
    if (st) return st;
    HIP_OK(moe::launch_unpermute(y, y_rows, inv_perm, topk_weights, Mc, K, topk, apply_on_input, out,
                                 static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

int moe_grouped_gemm_fp8_small(const uint8_t* a, const float* a_s, const uint8_t* w, const float* w_s,
                               const int32_t* expert_offsets, const int32_t* counts, int32_t El, int64_t cap_rows,
                               int32_t n_out, int32_t k_in, uint16_t* out, float* part, int64_t part_rows,
                               int32_t nsplit, int32_t* info, void* stream) {
    REQUIRE(El >= 1 && El <= moe::kMaxLocalExperts, MOE_ERR_SHAPE, "El=%d outside [1,1024]", El);
    REQUIRE(n_out > 0 && n_out % moe::kGroup == 0 && n_out <= 65536, MOE_ERR_SHAPE,
            "n_out=%d is not a positive multiple of 128 up to 65536", n_out);
    REQUIRE(k_in > 0 && k_in % moe::kGroup == 0 && k_in <= 65536, MOE_ERR_SHAPE,
            "k_in=%d is not a positive multiple of 128 up to 65536", k_in);
    REQUIRE(cap_rows >= 0 && cap_rows < (int64_t(1) << 31), MOE_ERR_SHAPE, "cap_rows=%lld", (long long)cap_rows);
    if (part != nullptr) {
        REQUIRE(nsplit >= 1 && nsplit <= 8 && (k_in / moe::kGroup) % nsplit == 0, MOE_ERR_SHAPE,
                "nsplit=%d must be 1..8 and divide k_in/128=%d", nsplit, k_in / moe::kGroup);
        REQUIRE(part_rows >= 1 && part_rows < (int64_t(1) << 31), MOE_ERR_SHAPE, "part_rows=%lld",
                (long long)part_rows);
        REQUIRE_PTR(info);
    }
    if (cap_rows == 0) return MOE_OK;
    REQUIRE_PTR(a);
    REQUIRE_PTR(a_s);
    REQUIRE_PTR(w);
    REQUIRE_PTR(w_s);
    REQUIRE_PTR(expert_offsets);
    REQUIRE_PTR(counts);
    if (part == nullptr) REQUIRE_PTR(out);
    int cus = 0;
    int st = check_device(&cus);
    if (st) return st;
    HIP_OK(moe::launch_grouped_gemm_small(a, a_s, w, w_s, expert_offsets, counts, El, cap_rows, n_out, k_in, out,
                                          part, part_rows, nsplit, info, cus, static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

int moe_act_quant_partials(const float* part, const int32_t* info, int64_t part_rows, int32_t nsplit, int64_t rows,
                           int32_t n, const int32_t* expert_offsets, const int32_t* counts, int32_t El, uint8_t* q,
                           float* q_s, void* stream) {
    REQUIRE(rows >= 0, MOE_ERR_SHAPE, "rows < 0");
    REQUIRE(n > 0 && n % moe::kGroup == 0 && n <= 32768, MOE_ERR_SHAPE,
            "n=%d is not a positive multiple of 128 up to 32768", n);
    REQUIRE(El >= 1 && El <= moe::kMaxLocalExperts, MOE_ERR_SHAPE, "El=%d outside [1,1024]", El);
    REQUIRE(nsplit >= 1 && nsplit <= 8, MOE_ERR_SHAPE, "nsplit=%d outside [1,8]", nsplit);
    REQUIRE(part_rows >= 1 && part_rows < (int64_t(1) << 31), MOE_ERR_SHAPE, "part_rows=%lld", (long long)part_rows);
    if (rows == 0) return MOE_OK;
    REQUIRE_PTR(part);
    REQUIRE_PTR(info);
    REQUIRE_PTR(expert_offsets);
    REQUIRE_PTR(counts);
    REQUIRE_PTR(q);
    REQUIRE_PTR(q_s);
    int st = check_device(nullptr);
    if (st) return st;
    // the grid is sized for the slabs' rows (the kernel's blocks take more
    // groups each when there are more valid rows than that)
    HIP_OK(moe::launch_act_quant_part(part, info, part_rows, nsplit, rows, n, expert_offsets, counts, El, q, q_s,
                                      part_rows < rows ? part_rows : rows, static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

int moe_unpermute_partials(const float* part, const int32_t* info, int64_t part_rows, int32_t nsplit,
                           const int32_t* expert_offsets, const int32_t* counts, int32_t El, int64_t y_rows,
                           const int32_t* inv_perm, const float* topk_weights, int64_t Mc, int32_t K, int32_t topk,
                           int32_t apply_on_input, uint16_t* out, void* stream) {
    REQUIRE(Mc >= 0 && y_rows >= 0, MOE_ERR_SHAPE, "Mc / y_rows < 0");
    REQUIRE(K > 0 && K % moe::kGroup == 0, MOE_ERR_SHAPE, "K=%d is not a positive multiple of 128", K);
    REQUIRE(topk >= 1 && topk <= 256, MOE_ERR_SHAPE, "topk=%d outside [1,256]", topk);
    REQUIRE(apply_on_input == 0 || apply_on_input == 1, MOE_ERR_INVALID_ARG, "apply_on_input=%d", apply_on_input);
    REQUIRE(El >= 1 && El <= moe::kMaxLocalExperts, MOE_ERR_SHAPE, "El=%d outside [1,1024]", El);
    REQUIRE(nsplit >= 1 && nsplit <= 8, MOE_ERR_SHAPE, "nsplit=%d outside [1,8]", nsplit);
    REQUIRE(part_rows >= 1 && part_rows < (int64_t(1) << 31), MOE_ERR_SHAPE, "part_rows=%lld", (long long)part_rows);
    if (Mc == 0) return MOE_OK;
    REQUIRE_PTR(part);
    REQUIRE_PTR(info);
    REQUIRE_PTR(expert_offsets);
    REQUIRE_PTR(counts);
    REQUIRE_PTR(inv_perm);
    REQUIRE_PTR(out);
    if (!apply_on_input) REQUIRE_PTR(topk_weights);
    REQUIRE(!overlaps(out, (size_t)Mc * K * 2, part, (size_t)nsplit * part_rows * K * 4), MOE_ERR_INVALID_ARG,
            "out overlaps part");
    int st = check_device(nullptr);
    if (st) return st;
    HIP_OK(moe::launch_unpermute_part(part, info, part_rows, nsplit, expert_offsets, counts, El, y_rows, inv_perm,
                                      topk_weights, Mc, K, topk, apply_on_input, out,
                                      static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

int moe_forward_plan_info(const moe_problem* p, int32_t* small_tiles, int32_t* nsplit_w13, int32_t* nsplit_w2,
                          int64_t* part_rows, int32_t* lanes) {
    int st = check_problem(p);
    if (st) return st;
    const Plan pl = make_plan(*p);
    if (small_tiles) *small_tiles = pl.small ? 1 : 0;
    if (nsplit_w13) *nsplit_w13 = pl.part_rows > 0 ? pl.smax13 : 1;
    if (nsplit_w2) *nsplit_w2 = pl.part_rows > 0 ? pl.smax2 : 1;
    if (part_rows) *part_rows = pl.part_rows;
    if (lanes) *lanes = pl.lanes;
    return MOE_OK;
}

}  // extern "C"

namespace {

// The library's chunk-lane streams of a device and the events that fork them
// from and join them to the caller's stream; created on first use and kept.
// The mutex covers one call's enqueue: a wait on an event takes the event as
// last recorded before the wait, so the next call may record it again.
struct LaneStreams {
    std::mutex mu;
    bool ready = false;
    hipStream_t s[kLanes] = {};
    hipEvent_t fork = nullptr, join[kLanes] = {};
};
LaneStreams g_lanes[kMaxDevices];

int lane_streams(LaneStreams** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED_DEVICE, "device %d", dev);
    *out = &g_lanes[dev];
    return MOE_OK;
}

// Enqueues chunk c of the layer on stream s, with the slices of one lane at ws.
int forward_chunk(const moe_problem& P, const Plan& pl, int64_t c, const uint16_t* x, const int32_t* topk_ids,
                  const float* topk_weights, const int32_t* expert_map, const uint8_t* w13, const float* w13_s,
                  const uint8_t* w2, const float* w2_s, uint16_t* out, uint8_t* ws, int32_t* per_chunk_counts,
                  int cus, hipStream_t s) {
    uint8_t* bufA = ws + pl.bufA;
    float* bufAs = reinterpret_cast<float*>(ws + pl.bufAs);
    uint16_t* hy = reinterpret_cast<uint16_t*>(ws + pl.bufB);
    int32_t* counts = reinterpret_cast<int32_t*>(ws + pl.counts);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + pl.offsets);
    int32_t* inv = reinterpret_cast<int32_t*>(ws + pl.inv);
    int32_t* rsrc = reinterpret_cast<int32_t*>(ws + pl.rsrc);
    int32_t* hist = reinterpret_cast<int32_t*>(ws + pl.hist);
    float* part = reinterpret_cast<float*>(ws + pl.part);
    int32_t* info = reinterpret_cast<int32_t*>(ws + pl.info);
    const bool split13 = pl.part_rows > 0 && pl.smax13 > 1;
    const bool split2 = pl.part_rows > 0 && pl.smax2 > 1;

    const int64_t K = P.K, N = P.N, T = P.topk, El = P.num_local_experts;
    const int on_in = P.apply_router_weight_on_input;
    const int64_t t0 = c * pl.cs;
    const int64_t Mc = (t0 + pl.cs <= P.M) ? pl.cs : (P.M - t0);
    const int32_t* ids_c = topk_ids + t0 * T;
    const float* w_c = topk_weights + t0 * T;
    // input quant fused into the permute's scatter
    HIP_OK(moe::launch_quant_permute(x + t0 * K, ids_c, w_c, on_in, Mc, (int)K, (int)T, expert_map,
                                     P.num_global_experts, (int)El, P.align, pl.cap, bufA, bufAs, counts,
                                     offsets, inv, rsrc, hist,
                                     per_chunk_counts ? per_chunk_counts + c * El : nullptr, s));
    if (pl.small) {
        HIP_OK(moe::launch_grouped_gemm_small(bufA, bufAs, w13, w13_s, offsets, counts, (int)El, pl.cap,
                                              (int)(2 * N), (int)K, hy, split13 ? part : nullptr, pl.part_rows,
                                              pl.smax13, info, cus, s));
    } else {
        HIP_OK(moe::launch_grouped_gemm(bufA, bufAs, w13, w13_s, offsets, counts, (int)El, pl.cap,
                                        (int)(2 * N), (int)K, hy, moe::gemm_tile_rows_routed(Mc * T, (int)El), cus,
                                        s));
    }
    if (split13) {
        HIP_OK(moe::launch_act_quant_part(part, info, pl.part_rows, pl.smax13, pl.cap, (int)N, offsets, counts,
                                          (int)El, bufA, bufAs, Mc * T, s));
    } else {
        HIP_OK(moe::launch_act_quant(hy, pl.cap, (int)N, moe::MOE_ACT_SILU_MUL_K, offsets, counts, (int)El,
                                     bufA, bufAs, Mc * T, s));
    }
    if (pl.small) {
        HIP_OK(moe::launch_grouped_gemm_small(bufA, bufAs, w2, w2_s, offsets, counts, (int)El, pl.cap, (int)K,
                                              (int)N, hy, split2 ? part : nullptr, pl.part_rows, pl.smax2, info + 1,
                                              cus, s));
    } else {
        HIP_OK(moe::launch_grouped_gemm(bufA, bufAs, w2, w2_s, offsets, counts, (int)El, pl.cap, (int)K,
                                        (int)N, hy, moe::gemm_tile_rows_routed(Mc * T, (int)El), cus, s));
    }
    if (split2) {
        HIP_OK(moe::launch_unpermute_part(part, info + 1, pl.part_rows, pl.smax2, offsets, counts, (int)El,
                                          pl.cap, inv, w_c, Mc, (int)K, (int)T, on_in, out + t0 * K, s));
    } else {
        HIP_OK(moe::launch_unpermute(hy, pl.cap, inv, w_c, Mc, (int)K, (int)T, on_in, out + t0 * K, s));
    }
    return MOE_OK;
}

// The chunk loop of moe_forward_chunked over an already validated problem
// and a workspace of at least pl.total bytes.
int forward_impl(const moe_problem& P, const Plan& pl, const uint16_t* x, const int32_t* topk_ids,
                 const float* topk_weights, const int32_t* expert_map, const uint8_t* w13, const float* w13_s,
                 const uint8_t* w2, const float* w2_s, uint16_t* out, uint8_t* ws, int32_t* per_chunk_counts,
                 int cus, hipStream_t s) {
    const int64_t nchunks = (P.M + pl.cs - 1) / pl.cs;
    if (pl.lanes == 1 || nchunks < 2) {
        for (int64_t c = 0; c < nchunks; ++c) {
            const int st = forward_chunk(P, pl, c, x, topk_ids, topk_weights, expert_map, w13, w13_s, w2, w2_s, out,
                                         ws, per_chunk_counts, cus, s);
            if (st) return st;
        }
        return MOE_OK;
    }
    LaneStreams* L = nullptr;
    int st = lane_streams(&L);
    if (st) return st;
    std::lock_guard<std::mutex> lock(L->mu);
    if (!L->ready) {
        for (int i = 0; i < kLanes; ++i) {
            HIP_OK(hipStreamCreateWithFlags(&L->s[i], hipStreamNonBlocking));
            HIP_OK(hipEventCreateWithFlags(&L->join[i], hipEventDisableTiming));
        }
        HIP_OK(hipEventCreateWithFlags(&L->fork, hipEventDisableTiming));
        L->ready = true;
    }
    const int nl = pl.lanes;   // <= kLanes and <= nchunks
    HIP_OK(hipEventRecord(L->fork, s));
    for (int i = 0; i < nl; ++i) HIP_OK(hipStreamWaitEvent(L->s[i], L->fork, 0));
    // the lanes run free: holding chunk c + 1 until chunk c's gate/up GEMM is
    // done was measured slower (8192 tokens in chunks of 64: 6.7 against
    // 6.1 ms)
    for (int64_t c = 0; c < nchunks; ++c) {
        const int lane = (int)(c % nl);
        st = forward_chunk(P, pl, c, x, topk_ids, topk_weights, expert_map, w13, w13_s, w2, w2_s, out,
                           ws + lane * pl.one, per_chunk_counts, cus, L->s[lane]);
        if (st) break;
    }
    // joined even after a failed launch, so the caller's stream never runs
    // ahead of work already enqueued on the lanes
    for (int i = 0; i < nl; ++i) {
        HIP_OK(hipEventRecord(L->join[i], L->s[i]));
        HIP_OK(hipStreamWaitEvent(s, L->join[i], 0));
    }
    return st;
}

// Checks of moe_forward_chunked's arguments other than the workspace.
int check_forward(const moe_problem* p, const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                  const int32_t* expert_map, const uint8_t* w13, const float* w13_s, const uint8_t* w2,
                  const float* w2_s, uint16_t* out, int32_t* per_chunk_counts) {
    int st = check_problem(p);
    if (st) return st;
    const moe_problem& P = *p;
    REQUIRE(expert_map != nullptr || P.num_local_experts <= P.num_global_experts, MOE_ERR_SHAPE,
            "El > Eg without an expert map");
    if (P.M == 0) return MOE_OK;
    REQUIRE_PTR(x);
    REQUIRE_PTR(topk_ids);
    REQUIRE_PTR(topk_weights);
    REQUIRE_PTR(w13);
    REQUIRE_PTR(w13_s);
    REQUIRE_PTR(w2);
    REQUIRE_PTR(w2_s);
    REQUIRE_PTR(out);
    REQUIRE(expert_map == nullptr || aligned16(expert_map), MOE_ERR_INVALID_ARG, "expert_map alignment");
    REQUIRE(per_chunk_counts == nullptr || aligned16(per_chunk_counts), MOE_ERR_INVALID_ARG,
            "per_chunk_counts alignment");
    const size_t out_bytes = (size_t)P.M * P.K * 2;
    REQUIRE(!overlaps(out, out_bytes, x, out_bytes), MOE_ERR_INVALID_ARG, "out overlaps x");
    return MOE_OK;
}

// ---- the forward without allocation --------------------------------------
// The workspace of moe_forward_chunked_noalloc: one fixed device array per
// GPU, allocated with the code object when the library is loaded on a device
// and held until the process ends.  Host code never uses its name as an
// address (that is a host-side stand-in): each device's address is taken
// once with hipGetSymbolAddress and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = size_t(MOE_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::atomic<uint8_t*> g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (looked up on the first call on
// each device, with that device current).
int scratch_for_current_device(uint8_t** ptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice failed");
    if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED_DEVICE, "device %d", dev);
    uint8_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        void* q = nullptr;
        HIP_OK(hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)));
        REQUIRE(q != nullptr && aligned16(q), MOE_ERR_HIP, "hipGetSymbolAddress gave %p", q);
        p = static_cast<uint8_t*>(q);
        g_scratch_ptr[dev].store(p, std::memory_order_release);   // the same value if two threads race here
    }
    *ptr = p;
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward_chunked(const moe_problem* p, const uint16_t* x, const int32_t* topk_ids,
                        const float* topk_weights, const int32_t* expert_map, const uint8_t* w13,
                        const float* w13_s, const uint8_t* w2, const float* w2_s, uint16_t* out,
                        void* workspace, size_t workspace_bytes, int32_t* per_chunk_counts,
                        void* stream) {
    int st = check_forward(p, x, topk_ids, topk_weights, expert_map, w13, w13_s, w2, w2_s, out, per_chunk_counts);
    if (st) return st;
    if (p->M == 0) return MOE_OK;
    REQUIRE_PTR(workspace);
    const Plan pl = make_plan(*p);
    REQUIRE(workspace_bytes >= pl.total, MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes",
            workspace_bytes, pl.total);
    REQUIRE(!overlaps(out, (size_t)p->M * p->K * 2, workspace, pl.total), MOE_ERR_INVALID_ARG,
            "out overlaps the workspace");
    int cus = 0;
    st = check_device(&cus);
    if (st) return st;
    return forward_impl(*p, pl, x, topk_ids, topk_weights, expert_map, w13, w13_s, w2, w2_s, out,
                        static_cast<uint8_t*>(workspace), per_chunk_counts, cus, static_cast<hipStream_t>(stream));
}

namespace {

// The batched entry's workspace: offsets, cut counts, act codes and scales.
struct BatchedPlan {
    size_t offsets, cut, act_q, act_s, total;
};

BatchedPlan batched_plan(int32_t El, int64_t max_tokens, int32_t N) {
    BatchedPlan b{};
    const size_t rows = (size_t)El * (size_t)max_tokens;
    size_t off = 0;
    b.offsets = off; off += up256((size_t)(El + 1) * 4);
    b.cut = off;     off += up256((size_t)El * 4);
    b.act_q = off;   off += up256(rows * N);
    b.act_s = off;   off += up256(rows * (N / moe::kGroup) * 4);
    b.total = off;
    return b;
}

int check_batched_shape(int32_t El, int64_t max_tokens, int32_t K, int32_t N) {
    REQUIRE(El >= 1 && El <= moe::kMaxLocalExperts, MOE_ERR_SHAPE, "El=%d outside [1,1024]", El);
    REQUIRE(max_tokens >= 0 && (int64_t)El * max_tokens < (int64_t(1) << 31), MOE_ERR_SHAPE,
            "max_tokens=%lld", (long long)max_tokens);
    REQUIRE(K > 0 && K % moe::kGroup == 0 && K <= 65536, MOE_ERR_SHAPE,
            "K=%d is not a positive multiple of 128 up to 65536", K);
    REQUIRE(N > 0 && N % moe::kGroup == 0 && N <= 32768, MOE_ERR_SHAPE,
            "N=%d is not a positive multiple of 128 up to 32768", N);
    return MOE_OK;
}

}  // namespace

int moe_batched_workspace_size(int32_t El, int64_t max_tokens, int32_t N, size_t* bytes) {
    int st = check_batched_shape(El, max_tokens, 128, N);
    if (st) return st;
    REQUIRE(bytes != nullptr, MOE_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = batched_plan(El, max_tokens, N).total;
    return MOE_OK;
}

int moe_experts_batched_masked(const uint8_t* a_q, const float* a_s, const int32_t* counts, int32_t El,
                               int64_t max_tokens, int32_t K, int32_t N, const uint8_t* w13, const float* w13_s,
                               const uint8_t* w2, const float* w2_s, uint16_t* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
    int st = check_batched_shape(El, max_tokens, K, N);
    if (st) return st;
    if (max_tokens == 0) return MOE_OK;
    REQUIRE_PTR(a_q);
    REQUIRE_PTR(a_s);
    REQUIRE_PTR(counts);
    REQUIRE_PTR(w13);
    REQUIRE_PTR(w13_s);
    REQUIRE_PTR(w2);
    REQUIRE_PTR(w2_s);
    REQUIRE_PTR(out);
    REQUIRE_PTR(workspace);
    const BatchedPlan b = batched_plan(El, max_tokens, N);
    REQUIRE(workspace_bytes >= b.total, MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", workspace_bytes,
            b.total);
    const int64_t rows = (int64_t)El * max_tokens;
    const size_t out_bytes = (size_t)rows * K * 2;
    REQUIRE(!overlaps(out, out_bytes, workspace, b.total), MOE_ERR_INVALID_ARG, "out overlaps the workspace");
    REQUIRE(!overlaps(out, out_bytes, a_q, (size_t)rows * K), MOE_ERR_INVALID_ARG, "out overlaps a_q");
    int cus = 0;
    st = check_device(&cus);
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + b.offsets);
    int32_t* cut = reinterpret_cast<int32_t*>(ws + b.cut);
    uint8_t* act_q = ws + b.act_q;
    float* act_s = reinterpret_cast<float*>(ws + b.act_s);
    HIP_OK(moe::launch_slot_offsets(counts, El, max_tokens, offsets, cut, s));
    // gate/up GEMM with the SiLU-mul requant in its epilogue: h never
    // reaches memory
    HIP_OK(moe::launch_grouped_gemm_act(a_q, a_s, w13, w13_s, offsets, cut, El, rows, N, K, act_q, act_s,
                                        moe::gemm_tile_rows(rows, El), cus, s));
    HIP_OK(moe::launch_grouped_gemm(act_q, act_s, w2, w2_s, offsets, cut, El, rows, K, N, out,
                                    moe::gemm_tile_rows(rows, El), cus, s));
    return MOE_OK;
}

int moe_hbm_stream(int32_t mode, const void* src, void* dst, size_t bytes, void* stream) {
    REQUIRE(mode >= MOE_STREAM_READ && mode <= MOE_STREAM_WRITE, MOE_ERR_INVALID_ARG, "mode=%d", mode);
    REQUIRE(bytes % 16 == 0, MOE_ERR_SHAPE, "bytes=%zu is not a multiple of 16", bytes);
    REQUIRE_PTR(dst);
    if (mode == MOE_STREAM_READ || mode == MOE_STREAM_COPY) REQUIRE_PTR(src);
    if (mode == MOE_STREAM_COPY)
        REQUIRE(!overlaps(src, bytes, dst, bytes), MOE_ERR_INVALID_ARG, "src and dst overlap");
    if (bytes == 0) return MOE_OK;
    int cus = 0;
    int st = check_device(&cus);
    if (st) return st;
    HIP_OK(moe::launch_stream(mode, src, dst, bytes, static_cast<uint32_t*>(dst), cus,
                              static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

size_t moe_noalloc_scratch_bytes(void) { return kScratchBytes; }

int moe_forward_chunked_noalloc(const moe_problem* p, const uint16_t* x, const int32_t* topk_ids,
                                const float* topk_weights, const int32_t* expert_map, const uint8_t* w13,
                                const float* w13_s, const uint8_t* w2, const float* w2_s, uint16_t* out,
                                int32_t* per_chunk_counts, void* stream) {
    int st = check_forward(p, x, topk_ids, topk_weights, expert_map, w13, w13_s, w2, w2_s, out, per_chunk_counts);
    if (st) return st;
    if (p->M == 0) return MOE_OK;
    // one lane: the chunks run in order on the caller's stream alone, with no
    // library stream or event created for them
    const Plan pl = make_plan(*p, false);
    REQUIRE(pl.total <= kScratchBytes, MOE_ERR_WORKSPACE_TOO_SMALL,
            "the problem needs %zu workspace bytes, more than the %zu of the fixed scratch array: use a smaller "
            "chunk_size or moe_forward_chunked with a workspace", pl.total, kScratchBytes);
    int cus = 0;
    st = check_device(&cus);
    if (st) return st;
    uint8_t* ws = nullptr;
    st = scratch_for_current_device(&ws);
    if (st) return st;
    REQUIRE(!overlaps(out, (size_t)p->M * p->K * 2, ws, kScratchBytes), MOE_ERR_INVALID_ARG,
            "out overlaps the scratch array");
    return forward_impl(*p, pl, x, topk_ids, topk_weights, expert_map, w13, w13_s, w2, w2_s, out, ws,
                        per_chunk_counts, cus, static_cast<hipStream_t>(stream));
}

}  // extern "C"
