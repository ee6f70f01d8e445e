// moe_internal.hpp -- host-side launchers of the gfx950 kernels (internal to
// libmoe_hip.so; the public surface is include/moe.h).  Launchers assume
// arguments were validated by the C-ABI layer and return hipGetLastError().
#pragma once
#include <cmath>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int MOE_ACT_IDENTITY_K = 0;  // same values as MOE_ACT_* in moe.h
constexpr int MOE_ACT_SILU_MUL_K = 1;

// ---- count / permute -------------------------------------------------------
// Tokens handled by one permute block: a token's topk pairs never straddle
// blocks and a block holds at most 256 pairs.
inline int permute_tokens_per_block(int topk) { return topk >= 256 ? 1 : 256 / topk; }
inline int64_t permute_num_blocks(int64_t Mc, int topk) {
    int tb = permute_tokens_per_block(topk);
    return (Mc + tb - 1) / tb;
}

hipError_t launch_count(const int32_t* ids, int64_t num_pairs, const int32_t* emap, int Eg, int El,
                        int32_t* counts, int32_t* invalid, int num_cus, hipStream_t s);

// hist: [nblk, El] int32 scratch.  Writes counts, offsets, row_src padding,
// and per-block row bases into hist.
hipError_t launch_permute(const uint8_t* a_q, const float* a_s, const int32_t* ids,
                          const float* topk_w, int apply_on_input, int64_t Mc, int K, int topk,
                          const int32_t* emap, int Eg, int El, int align, int64_t cap_rows,
                          uint8_t* a_perm, float* a_perm_s, int32_t* counts, int32_t* offsets,
                          int32_t* inv_perm, int32_t* row_src, int32_t* hist,
                          int32_t* counts_copy, hipStream_t s);
// launch_permute with the input quantisation fused into the scatter: reads
// bf16 x [Mc, K] and writes a_perm / a_perm_s exactly as launch_act_quant
// (identity) followed by launch_permute would.
hipError_t launch_quant_permute(const uint16_t* x, const int32_t* ids, const float* topk_w, int apply_on_input,
                                int64_t Mc, int K, int topk, const int32_t* emap, int Eg, int El, int align,
                                int64_t cap_rows, uint8_t* a_perm, float* a_perm_s, int32_t* counts,
                                int32_t* offsets, int32_t* inv_perm, int32_t* row_src, int32_t* hist,
                                int32_t* counts_copy, hipStream_t s);

// The batched, masked layout [El, max_tokens, ...]: offsets [El+1] =
// e * max_tokens and the counts cut to [0, max_tokens].
hipError_t launch_slot_offsets(const int32_t* counts, int El, int64_t max_tokens, int32_t* offsets, int32_t* cut,
                               hipStream_t s);

// ---- activation quantisation ------------------------------------------------
// rows_hint: at most this many rows are valid (the chunk's routed pairs in
// the forward; rows otherwise).  It sizes the grid of a masked launch, which
// walks the valid rows only, and decides whether the SiLU table pays.
hipError_t launch_act_quant(const uint16_t* in, int64_t rows, int n, int mode,
                            const int32_t* offsets, const int32_t* counts, int El, uint8_t* q,
                            float* q_s, int64_t rows_hint, hipStream_t s);

// The SiLU-mul requant (masked) of the gate/up values that
// launch_grouped_gemm_small left as partial sums part [S, part_rows, 2n]:
// the same codes and scales as launch_act_quant of their bf16 sum.
hipError_t launch_act_quant_part(const float* part, const int32_t* info, int64_t part_rows, int smax, int64_t rows,
                                 int n, const int32_t* offsets, const int32_t* counts, int El, uint8_t* q, float* q_s,
                                 int64_t rows_hint, hipStream_t s);

// ---- grouped GEMM ------------------------------------------------------------
// Output-tile rows (128 or 256) of the plain, fused and reducing GEMMs.
// gemm_tile_rows: from a row-buffer bound (the GEMM entry points' cap_rows,
// which for a buffer sized by moe_max_rows with 128-row alignment holds up to
// 127 padding rows per expert): 256 once it reaches 256 rows per expert.
// gemm_tile_rows_routed: from the routed pairs themselves (the forward's
// Mc * topk): 256 once they average 104 rows per expert, the measured
// crossover.
int gemm_tile_rows(int64_t rows_hint, int El);
int gemm_tile_rows_routed(int64_t pairs, int El);
hipError_t launch_grouped_gemm(const uint8_t* a, const float* a_s, const uint8_t* w,
                               const float* w_s, const int32_t* offsets, const int32_t* counts,
                               int El, int64_t cap_rows, int n_out, int k_in, uint16_t* out,
                               int tile_rows, int num_cus, hipStream_t s);

// Whether a chunk of `pairs` token-expert pairs (routed over Eg experts, El
// of them local) runs its GEMMs on 64-row tiles with K cut into segments
// (launch_grouped_gemm_small) rather than on 128/256-row tiles: when the
// pairs average at most 48 per local expert and the gate/up GEMM (n13
// output columns) would have fewer than 512 tiles on the larger tiles (two
// rounds of the MI355X's 256 CUs), counting the local experts that uniform
// routing would touch, El (1 - (1 - 1/Eg)^pairs).  Measured on forward
// steps (hidden 2048, intermediate 768, top-8): with all 128 experts local
// the 128-row tiles are 3-13% faster from 64 tokens on (their 750+ tiles
// fill the chip without a cut); with 64 of 128 local the small tiles are
// 3-6% faster at 128-256 tokens, level at 384, 2% slower at 512.
inline bool gemm_small_chunk(int64_t pairs, int El, int Eg, int n13) {
    if (El <= 0 || Eg <= 0 || pairs > (int64_t)48 * El) return false;
    const double touched = El * (1.0 - std::pow(1.0 - 1.0 / Eg, (double)pairs));
    return touched * ((n13 + 255) / 256) < 512.0;
}
// The plain GEMM on 64-row tiles for such chunks (see gemm_fp8.hip).  part
// null: bf16 out [cap_rows, n_out].  part set: when the tiles fill fewer than
// four rounds of num_cus CUs, K is cut into nsplit segments (nsplit divides
// k_in / 128, at most 8) and the fp32 partial sums go to part [nsplit,
// part_rows, n_out], rows at their place among the valid rows (experts in
// order); info[0] receives the segments used (1: one slab of whole-K sums,
// whose bf16 rounding is the unsplit output).
hipError_t launch_grouped_gemm_small(const uint8_t* a, const float* a_s, const uint8_t* w, const float* w_s,
                                     const int32_t* offsets, const int32_t* counts, int El, int64_t cap_rows,
                                     int n_out, int k_in, uint16_t* out, float* part, int64_t part_rows, int nsplit,
                                     int32_t* info, int num_cus, hipStream_t s);
// The K segments of a small-chunk GEMM: the largest S <= 8 dividing
// k_in / 128 whose segments keep at least 8 groups (1024 of K); 1 below
// 16 groups.  A shorter unit costs more in its pipeline refill (~1 us per
// unit start, measured) than its finer spread over the grid saves.
inline int gemm_split_segments(int k_in) {
    const int kg = k_in / 128;
    for (int S = 8; S > 1; --S)
        if (kg % S == 0 && kg / S >= 8) return S;
    return 1;
}

// The gate/up GEMM (w13 [El, 2N, k_in]) fused with SiLU-and-mul and the
// per-128 requant: writes q [cap_rows, N] e4m3 and q_s [cap_rows, N/128].
hipError_t launch_grouped_gemm_act(const uint8_t* a, const float* a_s, const uint8_t* w13,
                                   const float* w13_s, const int32_t* offsets, const int32_t* counts,
                                   int El, int64_t cap_rows, int N, int k_in, uint8_t* q, float* q_s,
                                   int tile_rows, int num_cus, hipStream_t s);

// The down GEMM with the unpermute's weight-and-reduce in its epilogue: y
// [cap_rows, n_out] as launch_grouped_gemm, and out [Mc, n_out] as
// launch_unpermute of that y.  cnt [Mc, ceil(n_out / 256)] must be zero on
// entry (launch_reduce_prep) and is zero again on exit.
hipError_t launch_grouped_gemm_reduce(const uint8_t* a, const float* a_s, const uint8_t* w, const float* w_s,
                                      const int32_t* offsets, const int32_t* counts, int El, int64_t cap_rows,
                                      int n_out, int k_in, uint16_t* y, const int32_t* row_src,
                                      const int32_t* inv_perm, const float* topk_w, int on_input, int64_t Mc,
                                      int topk, int32_t* cnt, uint16_t* out, int tile_rows, int num_cus,
                                      hipStream_t s);
// Zeroes cnt [Mc, ceil(K / 256)] and writes +0 output rows for the tokens
// without a valid row.
hipError_t launch_reduce_prep(const int32_t* inv_perm, int64_t Mc, int topk, int64_t y_rows, int K, int32_t* cnt,
                              uint16_t* out, hipStream_t s);

// ---- unpermute ----------------------------------------------------------------
hipError_t launch_unpermute(const uint16_t* y, int64_t y_rows, const int32_t* inv_perm,
                            const float* topk_w, int64_t Mc, int K, int topk, int apply_on_input, uint16_t* out,
                            hipStream_t s);

// launch_unpermute of y given as launch_grouped_gemm_small's partial sums
// part [S, part_rows, K] (y_rows: the rows of the expert slots).
hipError_t launch_unpermute_part(const float* part, const int32_t* info, int64_t part_rows, int smax,
                                 const int32_t* offsets, const int32_t* counts, int El, int64_t y_rows,
                                 const int32_t* inv_perm, const float* topk_w, int64_t Mc, int K, int topk,
                                 int apply_on_input, uint16_t* out, hipStream_t s);

// ---- HBM streams (measured ceilings) -------------------------------------------
// mode: MOE_STREAM_* of moe.h; sink receives nothing in practice (read mode
// keeps its loads live through it).
hipError_t launch_stream(int mode, const void* src, void* dst, size_t bytes, uint32_t* sink, int num_cus,
                         hipStream_t s);

}  // namespace moe
