/*
 * moe_ref.h -- CPU oracle for the fused MoE expert layer (TEST INFRASTRUCTURE).
 *
 * This is the slow, plain definition the HIP library is checked against.  It
 * is used only by the tests, by the smoke check and by the bench's CPU
 * baseline; no product code links it.  It shares no source with the HIP
 * library: every conversion, quantiser and reduction below is written out
 * here on its own.
 *
 * Sources (vLLM pull-request pages):
 *  - PR #20903 "[Kernel] DeepGemm MoE : Integrate triton permute / unpermute
 *    kernels": Purpose (workspaces sized by local experts and expert counts;
 *    ep_scatter permute / ep_gather unpermute), Optimizations (fp8 e4m3 with
 *    128x128 blocks), bot Highlights (router weight applied and reduced
 *    inside the experts, output (M, K)).
 *  - PR #20725 "[Misc] ModularKernel : Perform WeightAndReduce inside
 *    TritonExperts & DeepGemmExperts": Purpose/Changes (topk_weights and
 *    apply_router_weight_on_input passed to the experts).
 *  - PR #20392 "[Bugfix] Fused MoE Modular Kernel chunking loop": Purpose
 *    (Bug 1: workspace shapes per chunk; Bug 2: expert_num_tokens recounted per
 *    chunk), review (count_expert_num_tokens over topk_ids, local_num_experts,
 *    expert_map).
 * Where the pages leave a step open, the reading taken is stated at that
 * function.
 *
 * Conventions: host pointers, row-major, caller-owned.  bf16 travels as its
 * uint16 bit pattern, e4m3 as its uint8 bit pattern.  Functions returning int
 * return 0 on success and a negative code on a bad argument.
 */
#ifndef MOE_REF_H
#define MOE_REF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_REF_OK 0
#define MOE_REF_ERR_ARG (-1)
#define MOE_REF_ERR_SHAPE (-2)
#define MOE_REF_ERR_CAPACITY (-3)

/* ---- numerics ---------------------------------------------------------- */
uint16_t moe_ref_bf16_from_f32(float v);        /* round to nearest even */
uint16_t moe_ref_bf16_from_f64(double v);       /* one rounding, nearest even */
float moe_ref_f32_from_bf16(uint16_t b);
uint8_t moe_ref_e4m3_from_f32(float v);         /* OCP E4M3FN, saturating */
double moe_ref_e4m3_value(uint8_t q);           /* exact value (NaN for 0x7F/0xFF) */
float moe_ref_exp_spec(float x);
void moe_ref_quant_group(const float* v, uint8_t* q, float* s); /* 128 values */

/* ---- single-op definitions --------------------------------------------- */
int moe_ref_loc(int32_t id, const int32_t* expert_map, int32_t Eg, int32_t El);

int moe_ref_count(const int32_t* topk_ids, int64_t num_pairs, const int32_t* expert_map,
                  int32_t Eg, int32_t El, int32_t* counts, int32_t* invalid_ids);

int64_t moe_ref_max_rows(int64_t Mc, int32_t topk, int32_t El, int32_t align);

int moe_ref_act_quant_identity(const uint16_t* x, int64_t rows, int32_t n, uint8_t* q, float* q_s);

int moe_ref_permute(const uint8_t* a_q, const float* a_s, const int32_t* topk_ids,
                    const float* topk_weights, int32_t apply_on_input, int64_t Mc, int32_t K,
                    int32_t topk, const int32_t* expert_map, int32_t Eg, int32_t El, int32_t align,
                    int64_t cap_rows, uint8_t* a_perm, float* a_perm_s, int32_t* counts,
                    int32_t* expert_offsets, int32_t* inv_perm, int32_t* row_src);

int moe_ref_gemm_rows(const uint8_t* a, const float* a_s, const int32_t* row_expert, int64_t rows,
                      const uint8_t* w, const float* w_s, int32_t El, int32_t n_out, int32_t k_in,
                      uint16_t* out);

int moe_ref_grouped_gemm(const uint8_t* a, const float* a_s, const uint8_t* w, const float* w_s,
                         const int32_t* expert_offsets, const int32_t* counts, int32_t El,
                         int64_t cap_rows, int32_t n_out, int32_t k_in, uint16_t* out);

int moe_ref_silu_mul_quant(const uint16_t* h, int64_t rows, int32_t n, const int32_t* expert_offsets,
                           const int32_t* counts, int32_t El, uint8_t* q, float* q_s);

int moe_ref_unpermute(const uint16_t* y, const int32_t* inv_perm, const float* topk_weights,
                      int64_t Mc, int32_t K, int32_t topk, int32_t apply_on_input, uint16_t* out);

/* ---- whole layer -------------------------------------------------------- */
int moe_ref_forward_chunked(int64_t M, int32_t K, int32_t N, int32_t topk, int32_t Eg, int32_t El,
                            int32_t align, int32_t apply_on_input, int64_t chunk_size,
                            const uint16_t* x, const int32_t* topk_ids, const float* topk_weights,
                            const int32_t* expert_map, const uint8_t* w13, const float* w13_s,
                            const uint8_t* w2, const float* w2_s, uint16_t* out,
                            int32_t* per_chunk_counts);

int moe_ref_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
