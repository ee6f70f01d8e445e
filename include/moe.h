/*
 * moe.h -- C ABI of the MI355X (gfx950) fused MoE expert pipeline.
 *
 * One layer call on one GPU's local experts:
 *   input fp8 quant -> count -> permute -> fp8 grouped GEMM (w13)
 *   -> SiLU-and-mul + fp8 requant -> fp8 grouped GEMM (w2)
 *   -> unpermute with topk weight and reduce to (M, K),
 * chunked over M with per-chunk expert counts and workspace shapes.
 *
 * The operations follow three vLLM pull-request pages:
 *  [P20903] "[Kernel] DeepGemm MoE : Integrate triton permute / unpermute
 *           kernels" -- Purpose (workspaces sized from local experts and
 *           expert counts; ep_scatter / ep_gather permute and unpermute),
 *           Optimizations (float8_e4m3fn, 128x128 block shape, topk 4
 *           profile), bot Highlights (weights applied and reduced inside the
 *           experts; finalize becomes a no-op).
 *  [P20725] "[Misc] ModularKernel : Perform WeightAndReduce inside
 *           TritonExperts & DeepGemmExperts" -- Purpose/Changes
 *           (topk_weights and apply_router_weight_on_input reach the
 *           experts; workspace reuse rules).
 *  [P20392] "[Bugfix] Fused MoE Modular Kernel chunking loop" -- Purpose
 *           Bug 1 (workspace shapes per chunk), Bug 2 (expert_num_tokens
 *           recounted per chunk by count_expert_num_tokens), review thread
 *           (count over topk ids, local expert count and expert map).
 *
 * Conventions for every entry point:
 *  - Tensors are DEVICE pointers, contiguous row-major, caller-owned, 16-byte
 *    aligned.  bf16 travels as uint16_t bits, e4m3 (OCP E4M3FN) as uint8_t.
 *    Nothing is retained after return.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *    asynchronously; the library never synchronises and never allocates or
 *    frees device memory.
 *  - Arguments are validated on the host before anything is enqueued; on an
 *    error nothing is launched and a status != MOE_OK is returned, with
 *    detail in moe_last_error() (thread-local).  Device faults surface at the
 *    caller's next synchronisation.
 *  - The library runs on gfx950 only (MOE_ERR_UNSUPPORTED_DEVICE otherwise).
 *  - A local expert id of a global id is: -1 if the id is -1 or outside
 *    [0, Eg); expert_map[id] if a map is given; else the id if < El, else -1.
 *    Pairs with local id -1 are dropped.  Limits: 1 <= El <= 1024,
 *    1 <= topk <= 256, K and N multiples of 128, Mc*topk < 2^31.
 */
#ifndef MOE_H
#define MOE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,        /* null / misaligned pointer, bad flag, overlap */
    MOE_ERR_SHAPE = 2,              /* size not supported (K%128, align, limits) */
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,
    MOE_ERR_UNSUPPORTED_DEVICE = 4, /* current device is not gfx950 */
    MOE_ERR_HIP = 5                 /* a HIP call or kernel launch failed */
} moe_status;

#define MOE_ACT_IDENTITY 0
#define MOE_ACT_SILU_MUL 1

typedef struct {
    int64_t M;                         /* tokens in the layer call */
    int32_t K;                         /* hidden size, multiple of 128, <= 65536 */
    int32_t N;                         /* expert intermediate size, multiple of 128, <= 32768 */
    int32_t topk;
    int32_t num_global_experts;        /* Eg */
    int32_t num_local_experts;         /* El */
    int32_t align;                     /* row padding per expert: 16, 32, 64 or 128 */
    int32_t apply_router_weight_on_input; /* 0 or 1 [P20725 Purpose/Changes] */
    int64_t chunk_size;                /* <= 0 or >= M: one chunk [P20392 Bug 1] */
} moe_problem;

const char* moe_status_string(int status);
const char* moe_last_error(void);

/* Rows a padded, expert-contiguous permuted buffer needs for Mc tokens, for
 * any routing: P + min(El, P) * (align - 1) with P = Mc * topk.  Returns -1 on
 * bad arguments.  Sync-free stand-in for sizing from host-side expert counts
 * [P20903 Purpose item 1]. */
int64_t moe_max_rows(int64_t Mc, int32_t topk, int32_t El, int32_t align);

/* Workspace bytes moe_forward_chunked needs for problem p (sized for the
 * largest chunk and reused by every chunk). */
int moe_forward_workspace_size(const moe_problem* p, size_t* bytes);

/* The slices moe_forward_chunked carves from its workspace for problem p:
 * *num_slices receives their number (10: permuted rows then act codes,
 * their scales, h then y, counts, offsets, inv_perm, row_src, the permute's
 * per-block histogram, the fp32 partial sums of the GEMMs with K split for
 * small chunks (empty when the plan splits neither GEMM) and the two
 * GEMMs' segment counts), times the lanes (min(chunks, 3) with two chunks
 * or more: each lane's ten slices follow the previous lane's, in the same
 * order); the
 * first min(max_slices, *num_slices) byte offsets
 * and lengths are written to offsets[] and bytes[].  Between the end of a
 * slice and the next slice's offset (and up to the workspace size after the
 * last) lies a guard band that no kernel reads or writes: a caller can fill
 * the workspace with a pattern and check the bands after a call. */
int moe_forward_workspace_slices(const moe_problem* p, size_t* offsets, size_t* bytes, int32_t max_slices,
                                 int32_t* num_slices);

/* Workspace bytes moe_permute needs for Mc tokens. */
int moe_permute_workspace_size(int64_t Mc, int32_t topk, int32_t El, size_t* bytes);

/* count_expert_num_tokens [P20392 Bug 2; review thread]:
 *   counts[e] = #{ f < num_pairs : local(topk_ids[f]) == e },  e < El.
 * topk_ids: [num_pairs] int32 global ids.  expert_map: [Eg] int32 or NULL
 * (identity, requires El <= Eg).  counts: [El] int32, overwritten.
 * invalid_ids: NULL or [1] int32, overwritten with the number of ids outside
 * [-1, Eg).  Exact integer counts.  topk_ids 16-byte aligned; counts and
 * invalid_ids 4-byte aligned (counts 8-byte aligned lets the kernel add two
 * experts' totals per atomic, which is faster on large inputs). */
int moe_count(const int32_t* topk_ids, int64_t num_pairs, const int32_t* expert_map, int32_t Eg,
              int32_t El, int32_t* counts, int32_t* invalid_ids, void* stream);

/* ep_scatter permute [P20903 Purpose item 2]:
 *   counts as moe_count; expert_offsets[0] = 0,
 *   expert_offsets[e+1] = expert_offsets[e] + align * ceil(counts[e] / align);
 *   pair f = t*topk + k with local expert e takes row
 *   expert_offsets[e] + #{ f' < f : local(f') == e }   (stable order);
 *   a_perm[row] = a_q[t];  a_perm_s[row] = a_s[t] (times topk_weights[f]
 *   when apply_on_input [P20725 Purpose/Changes]);
 *   inv_perm[f] = row or -1;  row_src[row] = t, -1 on padding rows and on
 *   rows in [expert_offsets[El], cap_rows).
 * a_q [Mc,K] e4m3, a_s [Mc,K/128] f32, topk_ids [Mc,topk], topk_weights
 * [Mc,topk] f32 (read only if apply_on_input), cap_rows >= moe_max_rows(),
 * a_perm [cap_rows,K], a_perm_s [cap_rows,K/128], counts [El],
 * expert_offsets [El+1], inv_perm [Mc,topk], row_src [cap_rows].
 * Padding rows of a_perm / a_perm_s are left unwritten.
 * workspace: >= moe_permute_workspace_size() bytes of device memory. */
int moe_permute(const uint8_t* a_q, const float* a_s, const int32_t* topk_ids,
                const float* topk_weights, int32_t apply_on_input, int64_t Mc, int32_t K,
                int32_t topk, const int32_t* expert_map, int32_t Eg, int32_t El, int32_t align,
                int64_t cap_rows, uint8_t* a_perm, float* a_perm_s, int32_t* counts,
                int32_t* expert_offsets, int32_t* inv_perm, int32_t* row_src, void* workspace,
                size_t workspace_bytes, void* stream);

/* ep_scatter permute [P20903 Purpose item 2] with the per-token 1x128 fp8
 * input quantisation [P20903 Optimizations] fused in, so the bf16 tokens are
 * read once: x [Mc,K] bf16; every group of
 * 128 values of a token is quantised as moe_act_quant in identity mode and
 * its codes and scale are written straight to the token's expert rows, so
 * a_perm, a_perm_s, counts, expert_offsets, inv_perm and row_src are exactly
 * those of moe_act_quant (identity) followed by moe_permute, and no a_q/a_s
 * buffer exists.  Other arguments, limits and errors as moe_permute; x must
 * be 16-byte aligned. */
int moe_quant_permute(const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                      int32_t apply_on_input, int64_t Mc, int32_t K, int32_t topk, const int32_t* expert_map,
                      int32_t Eg, int32_t El, int32_t align, int64_t cap_rows, uint8_t* a_perm,
                      float* a_perm_s, int32_t* counts, int32_t* expert_offsets, int32_t* inv_perm,
                      int32_t* row_src, void* workspace, size_t workspace_bytes, void* stream);

/* Output-tile rows (128 or 256) the grouped GEMM entry points use for a
 * row buffer of rows_hint rows over El local experts: 256 once it holds at
 * least 256 rows per expert, else 128.  moe_grouped_gemm_fp8 (and the fused
 * and reducing variants) pass cap_rows as the hint; for a buffer sized by
 * moe_max_rows with 128-row alignment that is 256 tiles once the routed rows
 * average about 129 per expert.  moe_forward_chunked knows its chunk's
 * token-expert pairs (Mc * topk) and takes 256-row tiles once they average
 * 104 per expert, the measured crossover.  The tile changes only speed:
 * outputs are identical either way.  Returns -1 when El < 1. */
int32_t moe_grouped_gemm_tile_rows(int64_t rows_hint, int32_t El);

/* Block-scaled fp8 grouped GEMM (the DeepGEMM grouped GEMM of [P20903],
 * Optimizations: e4m3, 128x128 blocks).  For every valid row r of expert e
 * (expert_offsets[e] <= r < expert_offsets[e] + counts[e]) and n < n_out:
 *   out[r,n] = bf16( sum_g a_s[r,g] * w_s[e, n/128, g] *
 *                    sum_{k in group g} a[r,k] * w[e,n,k] ),
 * fp32 accumulation.  a [cap_rows,k_in] e4m3, a_s [cap_rows,k_in/128] f32,
 * w [El,n_out,k_in] e4m3, w_s [El,n_out/128,k_in/128] f32,
 * out [cap_rows,n_out] bf16.  Rows that are not valid are not written.
 * n_out and k_in: positive multiples of 128, at most 65536 (MOE_ERR_SHAPE
 * otherwise). */
int moe_grouped_gemm_fp8(const uint8_t* a, const float* a_s, const uint8_t* w, const float* w_s,
                         const int32_t* expert_offsets, const int32_t* counts, int32_t El,
                         int64_t cap_rows, int32_t n_out, int32_t k_in, uint16_t* out,
                         void* stream);

/* The gate/up grouped GEMM fused with SiLU-and-mul and the per-token-group
 * requant: moe_grouped_gemm_fp8 on w13 followed by moe_act_quant in
 * MOE_ACT_SILU_MUL mode, with the same results bit for bit, but without
 * writing h [cap_rows, 2N] to memory.  For every valid row r (as in
 * moe_grouped_gemm_fp8) and group j of 128 columns of N:
 *   h   = bf16(GEMM(a, w13)) over the 2N outputs (gate = columns [0, N),
 *         up = [N, 2N)),
 *   act = bf16(silu(h[r, c]) * h[r, N + c]),
 *   q_s[r, j] = d/448, q[r, c] = e4m3(act * (448/d)), d = max(amax|act|, 1e-10).
 * a [cap_rows,k_in] e4m3, a_s [cap_rows,k_in/128] f32, w13 [El,2N,k_in]
 * e4m3, w13_s [El,2N/128,k_in/128] f32, q [cap_rows,N] e4m3,
 * q_s [cap_rows,N/128] f32; rows that are not valid are not written.
 * N: positive multiple of 128 up to 32768; k_in: positive multiple of 128
 * up to 65536 (MOE_ERR_SHAPE otherwise). */
int moe_grouped_gemm_fp8_act_quant(const uint8_t* a, const float* a_s, const uint8_t* w13,
                                   const float* w13_s, const int32_t* expert_offsets,
                                   const int32_t* counts, int32_t El, int64_t cap_rows, int32_t N,
                                   int32_t k_in, uint8_t* q, float* q_s, void* stream);

/* The down grouped GEMM with the unpermute's topk weight-and-reduce in its
 * epilogue (weight-and-reduce inside the experts, [P20725] Purpose/Changes;
 * output (M, K), [P20903] bot Highlights): y = moe_grouped_gemm_fp8(a, w) on
 * the valid rows, and out = moe_unpermute_weight_reduce(y, inv_perm,
 * topk_weights, apply_on_input), the same bits as those two calls.  Each tile
 * that has written its y rows counts, per row, that row's token up (row_src
 * gives the token of a row); the tile that completes a token's valid rows for
 * its 256 columns folds them in k order (fmaf from +0, one bf16 rounding), so
 * the result does not depend on which tile finishes last.  y [cap_rows,n_out]
 * bf16 (written), counters [Mc, ceil(n_out/256)] int32 device memory (any
 * contents on entry; zero on exit), out [Mc, n_out] bf16 (tokens without a
 * valid row get +0).  Other arguments as moe_grouped_gemm_fp8 and
 * moe_unpermute_weight_reduce; row_src and inv_perm as moe_permute writes
 * them (row_src [cap_rows]: token of a valid row). */
int moe_grouped_gemm_fp8_weight_reduce(const uint8_t* a, const float* a_s, const uint8_t* w, const float* w_s,
                                       const int32_t* expert_offsets, const int32_t* counts, int32_t El,
                                       int64_t cap_rows, int32_t n_out, int32_t k_in, const int32_t* row_src,
                                       const int32_t* inv_perm, const float* topk_weights, int32_t apply_on_input,
                                       int64_t Mc, int32_t topk, uint16_t* y, int32_t* counters, uint16_t* out,
                                       void* stream);

/* Per-token-group (1x128) fp8 quantisation.
 *   MOE_ACT_IDENTITY: v = in[r, :n]                        (in is [rows, n])
 *   MOE_ACT_SILU_MUL: v = bf16(silu(in[r, :n]) * in[r, n:2n]) (in is [rows, 2n])
 * then per group of 128: d = max(amax|v|, 1e-10), q_s = d/448,
 * q = e4m3(v * (448/d)) (saturating, nearest-even).
 * expert_offsets / counts: NULL = every row valid; otherwise only valid rows
 * (as in moe_grouped_gemm_fp8) are read and written: the rows of expert e are
 * [expert_offsets[e], expert_offsets[e] + counts[e]), cut at
 * expert_offsets[e+1] and at rows, so inconsistent offsets or counts never
 * move an access outside [0, rows).  q [rows,n], q_s [rows,n/128]. */
int moe_act_quant(const uint16_t* in, int64_t rows, int32_t n, int32_t mode,
                  const int32_t* expert_offsets, const int32_t* counts, int32_t El, uint8_t* q,
                  float* q_s, void* stream);

/* ep_gather unpermute with topk weight and reduce [P20903 Highlights;
 * P20725 Purpose]: for each token t and column c,
 *   acc = +0; for k = 0..topk-1 with 0 <= inv_perm[t,k] < y_rows:
 *       acc = fmaf(w', y[inv_perm[t,k], c], acc)
 *   out[t,c] = bf16(acc),  w' = topk_weights[t,k], or 1 when apply_on_input.
 * y [y_rows,K] bf16, inv_perm [Mc,topk], topk_weights [Mc,topk] f32 (unread
 * if apply_on_input), out [Mc,K] bf16 (must not overlap y).  Rows outside
 * [0, y_rows) are never read. */
int moe_unpermute_weight_reduce(const uint16_t* y, int64_t y_rows, const int32_t* inv_perm,
                                const float* topk_weights, int64_t Mc, int32_t K, int32_t topk,
                                int32_t apply_on_input, uint16_t* out, void* stream);

/* moe_grouped_gemm_fp8 for experts of few rows (the layer's small chunks,
 * e.g. the 64-token chunks of [P20392 Purpose]): 64-row output tiles, and
 * the option of cutting K so that a few tiles still spread over all CUs.
 *   part NULL: out exactly as moe_grouped_gemm_fp8 (the same bits).
 *   part set:  when the tiles fill fewer than four rounds of the CUs, K is cut
 *     into S = nsplit segments of k_in/nsplit (nsplit in 1..8 dividing
 *     k_in/128), else S = 1; info[0] receives S.  Slab s of part holds, for
 *     each valid row, the fp32 sum over the groups g of segment s of the
 *     terms a_s[r,g] * w_s[e,n/128,g] * sum_{k in g} a[r,k] w[e,n,k], folded
 *     in g order as the whole-K GEMM folds them: part[s, v, n], where v is
 *     the row's place in the valid rows of all experts in expert order
 *     (expert e's rows from sum_{e'<e} counts[e']).  bf16 of the slabs' sum
 *     in slab order is the GEMM's output (with S = 1, out's exact bits).
 *     part [nsplit, part_rows, n_out] f32; rows at places >= part_rows are
 *     not stored; out is not written.
 * Other arguments, limits and errors as moe_grouped_gemm_fp8. */
int moe_grouped_gemm_fp8_small(const uint8_t* a, const float* a_s, const uint8_t* w, const float* w_s,
                               const int32_t* expert_offsets, const int32_t* counts, int32_t El, int64_t cap_rows,
                               int32_t n_out, int32_t k_in, uint16_t* out, float* part, int64_t part_rows,
                               int32_t nsplit, int32_t* info, void* stream);

/* moe_act_quant in MOE_ACT_SILU_MUL mode, masked, whose input h is given as
 * moe_grouped_gemm_fp8_small's partial sums: h[r, c] = bf16 of the sum, in
 * slab order, of the first min(info[0], nsplit) slabs of part [nsplit,
 * part_rows, 2n] at row r's valid-row place (a place >= part_rows reads
 * as 0).  q, q_s and every other argument as moe_act_quant; the codes equal
 * moe_act_quant's on that h. */
int moe_act_quant_partials(const float* part, const int32_t* info, int64_t part_rows, int32_t nsplit, int64_t rows,
                           int32_t n, const int32_t* expert_offsets, const int32_t* counts, int32_t El, uint8_t* q,
                           float* q_s, void* stream);

/* moe_unpermute_weight_reduce whose y is given as moe_grouped_gemm_fp8_small's
 * partial sums: y[r, c] = bf16 of the sum, in slab order, of the first
 * min(info[0], nsplit) slabs of part [nsplit, part_rows, K] at row r's
 * valid-row place (expert_offsets / counts / El locate it; y_rows bounds r
 * as before).  An index that is no expert's valid row is not folded.  The
 * output equals moe_unpermute_weight_reduce's on that y. */
int moe_unpermute_partials(const float* part, const int32_t* info, int64_t part_rows, int32_t nsplit,
                           const int32_t* expert_offsets, const int32_t* counts, int32_t El, int64_t y_rows,
                           const int32_t* inv_perm, const float* topk_weights, int64_t Mc, int32_t K, int32_t topk,
                           int32_t apply_on_input, uint16_t* out, void* stream);

/* How moe_forward_chunked runs problem p: *small_tiles = 1 when its chunks
 * take moe_grouped_gemm_fp8_small (a chunk's token-expert pairs average at
 * most 48 per local expert, and the gate/up GEMM would have fewer than 512
 * tiles of 128 or 256 rows: the local experts that uniform routing over the
 * Eg experts would touch, times its 256-column tiles); *nsplit_w13 /
 * *nsplit_w2 the K segments those GEMMs are given (1: K whole, bf16 h / y),
 * *part_rows the rows of the partial slabs (0 without a cut), *lanes the
 * chunk lanes (min(chunks, 3) with two chunks or more).  Any output pointer
 * may be NULL. */
int moe_forward_plan_info(const moe_problem* p, int32_t* small_tiles, int32_t* nsplit_w13, int32_t* nsplit_w2,
                          int64_t* part_rows, int32_t* lanes);

/* The whole layer, chunked over M [P20392 Purpose]: for each chunk of
 * chunk_size tokens (the last one may be short) it runs input quant, count,
 * permute, GEMM(w13), SiLU-mul requant, GEMM(w2) and unpermute into the
 * chunk's rows of out.  Counts and shapes are per chunk; the workspace is
 * reused, laid out so that out never aliases it [P20725 author notes].
 * x [M,K] bf16, topk_ids [M,topk], topk_weights [M,topk] f32, expert_map
 * [Eg] or NULL, w13 [El,2N,K] e4m3, w13_s [El,2N/128,K/128] f32, w2 [El,K,N]
 * e4m3, w2_s [El,K/128,N/128] f32, out [M,K] bf16, workspace >=
 * moe_forward_workspace_size(p).  per_chunk_counts: NULL or device
 * [num_chunks, El] int32 receiving each chunk's counts.
 * Small chunks take the small-tile GEMMs (moe_forward_plan_info).  With
 * two chunks or more, consecutive chunks go round-robin to min(chunks, 3)
 * copies of the workspace slices and as many library streams (created on
 * the first such call on a device and kept), which wait for the work
 * enqueued on `stream` before the call, and on which `stream` waits after
 * it: every chunk computes what it computes alone, and work enqueued on
 * `stream` afterwards sees the whole output. */
int moe_forward_chunked(const moe_problem* p, const uint16_t* x, const int32_t* topk_ids,
                        const float* topk_weights, const int32_t* expert_map, const uint8_t* w13,
                        const float* w13_s, const uint8_t* w2, const float* w2_s, uint16_t* out,
                        void* workspace, size_t workspace_bytes, int32_t* per_chunk_counts,
                        void* stream);

/* The experts on the batched, masked layout (the batched DeepGEMM experts
 * variant named in [P20903] bot Highlights, for low-latency dispatch):
 * tokens already routed to slot e of a_q [El, max_tokens, K] e4m3 with
 * scales a_s [El, max_tokens, K/128] f32, the first counts[e] rows of slot e
 * valid (counts clamped to [0, max_tokens]).  For every valid row i of slot e
 *   act = SiLU-mul requant of bf16(GEMM(a_q[e,i], w13[e]))   (as
 *         moe_grouped_gemm_fp8_act_quant),
 *   out[e, i, :] = bf16(GEMM(act, w2[e]))                   (as
 *         moe_grouped_gemm_fp8),
 * the same bits as those two calls with expert_offsets[e] = e * max_tokens.
 * Rows past a slot's count are not written.  out [El, max_tokens, K] bf16;
 * the weighted reduce over a token's experts belongs to the combine that
 * follows and is not done here.  w13 [El,2N,K], w13_s [El,2N/128,K/128],
 * w2 [El,K,N], w2_s [El,K/128,N/128]; workspace >=
 * moe_batched_workspace_size(El, max_tokens, N) bytes. */
int moe_batched_workspace_size(int32_t El, int64_t max_tokens, int32_t N, size_t* bytes);
int moe_experts_batched_masked(const uint8_t* a_q, const float* a_s, const int32_t* counts, int32_t El,
                               int64_t max_tokens, int32_t K, int32_t N, const uint8_t* w13, const float* w13_s,
                               const uint8_t* w2, const float* w2_s, uint16_t* out, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Plain HBM streams, timed beside the memory-bound kernels as their measured
 * ceilings (not part of the layer): MOE_STREAM_READ reads `bytes` from src
 * (dst: >= 16 bytes of device memory, receives nothing unless the data hash
 * to one fixed value); MOE_STREAM_WRITE_NT / MOE_STREAM_WRITE write `bytes`
 * to dst with non-temporal / ordinary 16-byte stores; MOE_STREAM_COPY copies
 * `bytes` from src to dst (non-overlapping).  bytes: a multiple of 16. */
#define MOE_STREAM_READ 0
#define MOE_STREAM_WRITE_NT 1
#define MOE_STREAM_COPY 2
#define MOE_STREAM_WRITE 3
int moe_hbm_stream(int32_t mode, const void* src, void* dst, size_t bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation as moe_forward_chunked, bit for bit, with the workspace taken
 * from a fixed array of MOE_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on each GPU it runs on (allocated with the library's code object on
 * that device and kept until the process ends).  Nothing is allocated or
 * freed by the call.  The caller still passes every input and the output.
 * Problems whose workspace (moe_forward_workspace_size) exceeds the array
 * return MOE_ERR_WORKSPACE_TOO_SMALL before anything is enqueued: at the
 * K=2048, N=768, topk 8, align 128 shape that is chunks up to ~3300 tokens
 * with 128 local experts.  Every call on a GPU uses that GPU's one array,
 * which keeps the last call's contents (nothing in it needs to start at
 * zero): calls that overlap in time on one GPU (other streams, other host
 * threads) race, and the caller must order them. */
#define MOE_NOALLOC_SCRATCH_BYTES (256u << 20)
size_t moe_noalloc_scratch_bytes(void);
int moe_forward_chunked_noalloc(const moe_problem* p, const uint16_t* x, const int32_t* topk_ids,
                                const float* topk_weights, const int32_t* expert_map, const uint8_t* w13,
                                const float* w13_s, const uint8_t* w2, const float* w2_s, uint16_t* out,
                                int32_t* per_chunk_counts, void* stream);

#ifdef __cplusplus
}
#endif
#endif
