// Launchers of the row-wise DSpark loss kernels (see rowwise.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

typedef uint16_t bf16_t;

// Per-row state saved by the forward pass for the backward pass.
struct RowState {
  uint8_t* mask;   // supervised slot (prefix rule x block keep)
  float* w;        // decay weight exp(-k / gamma) on supervised slots, else 0
  float* lse_z;    // log-sum-exp of the corrected draft logits
  float* lse_t;    // log-sum-exp of the teacher logits
  float* l1;       // sum |p - q|
  float* S;        // sum p sign(p - q)
  float* ce;       // lse_z - z'_y
  float* accept;   // clamp(1 - l1 / 2, 0, 1); 1 on unsupervised slots
  float* conf;     // confidence logit
  float* bce;      // BCE(conf, accept)
  float* dcoef;    // sigmoid(conf) - accept
};

hipError_t launch_fill_u32(void* p, int64_t n, uint32_t v, hipStream_t s);
hipError_t launch_prep_rows(int64_t R, int K, const uint8_t* eval, const uint8_t* keep,
                            const int32_t* tid, const int32_t* prev, int64_t Vd, int64_t Vt,
                            int has_markov, float gamma, uint32_t set_bits, uint8_t* mask, float* w,
                            uint32_t* flags, hipStream_t s, int check_target = 1);
hipError_t launch_gather_embed(int dtype, int64_t R, int64_t rank, int64_t Vt, const int32_t* prev,
                               const uint8_t* mask, const void* W1, void* E, hipStream_t s);
// Loss rows of sampled anchors [B, N] over sequences [B, L] (labels, previous
// tokens, contiguous eval mask, block keep) and, if cand is not null, the
// anchor candidates [B, L].
hipError_t launch_build_blocks(int64_t B, int64_t L, int64_t N, int K, const int32_t* ids,
                               const uint8_t* lm, const int32_t* anchors, int32_t* target,
                               int32_t* prev, uint8_t* evalm, uint8_t* keep, uint8_t* cand,
                               hipStream_t s);
// c_r = W_c . [h_r ; e_r] + b on rows with mask[r] != 0 (every row if mask is
// null), 0 elsewhere (E unused unless with_markov_conf).
hipError_t launch_conf_logits(int dtype, int64_t R, int64_t Hd, int64_t rank, int with_markov_conf,
                              const void* hd, const void* E, const void* Wc, const void* bc,
                              const uint8_t* mask, float* out, hipStream_t s);
// Zeroes the rows r of out [R, N] (fp32) where mask[r] == 0.
hipError_t launch_zero_masked_rows(int64_t R, int64_t N, const uint8_t* mask, float* out,
                                   hipStream_t s);
hipError_t launch_l1_sweep(int64_t R, int64_t V, const float* Zp, const float* Tt,
                           const float2* sz, const float2* st, int64_t nstat, const uint8_t* mask,
                           const int32_t* tid, int has_teacher, RowState rs, hipStream_t s);
// lse_z, lse_t of supervised rows from tile statistics (0 on the others).
hipError_t launch_lse_rows(int64_t R, const float2* sz, const float2* st, int64_t nstat,
                           const uint8_t* mask, int has_teacher, RowState rs, hipStream_t s);
hipError_t launch_finalize_rows(int dtype, int64_t R, int64_t Hd, int64_t rank,
                                int with_markov_conf, int has_conf, const void* hd, const void* E,
                                const void* Wc, const void* bc, RowState rs, float* accept_out,
                                float* row_terms, uint32_t* flags, float ce_a, float l1_a,
                                float c_a, hipStream_t s);
hipError_t launch_reduce_fwd(int64_t R, int64_t nblk, int K, RowState rs, const uint8_t* eval,
                             const uint8_t* keep, float ce_a, float l1_a, float c_a, double* loss,
                             int64_t* num_tokens, double* pairs, hipStream_t s);
hipError_t launch_accept_report(int64_t nblk, int K, const float* accept, const uint8_t* eval,
                                const uint8_t* keep, double* out4, hipStream_t s);
hipError_t launch_grad_sweep(int grad_dtype, int64_t R, int64_t V, const float* Zp,
                             const float* Tt, const int32_t* tid, RowState rs, int has_teacher,
                             float g, float ce_a, float l1_a, void* dz, bf16_t* ghi, bf16_t* glo,
                             float* g32, hipStream_t s);
hipError_t launch_grad_sweep8(int grad_dtype, int64_t R, int64_t rgroups, int64_t V,
                              const float* Zp, const float* Tt, const int32_t* tid, RowState rs,
                              int has_teacher, float g, float ce_a, float l1_a, void* dz,
                              bf16_t* ghi_rm, bf16_t* glo_rm, bf16_t* blk_hi, bf16_t* blk_lo,
                              hipStream_t s);
hipError_t launch_transpose_bf16(int64_t rows, int64_t cols, const void* in, void* out,
                                 hipStream_t s);
hipError_t launch_embed_blocked(int64_t R, int64_t rgroups, int64_t rank, const void* E, void* out,
                                hipStream_t s);
hipError_t launch_add2(int64_t n, const float* a, const float* b, float* out, hipStream_t s);
// out = sum over k < parts of p[k * n .. k * n + n) (n % 4 == 0), in order of k.
hipError_t launch_sum_parts(int64_t n, int parts, const float* p, float* out, hipStream_t s);
hipError_t launch_de_reduce(int dtype, int64_t R, int64_t rank, int splits, const float* part,
                            RowState rs, int conf_markov, const void* Wc, int64_t Hd, float g,
                            float c_a, float* dE, hipStream_t s);
hipError_t launch_dw1_scatter(int64_t R, int64_t rank, int64_t Vt, const int32_t* prev,
                              const uint8_t* mask, const float* dE, float* dW1, hipStream_t s);
// Deterministic dW1 (fixed-point integer sums, see rowwise.hip): acc [Vt, r]
// 64-bit zeroed and dW1 zeroed by the caller; maxp: one float of scratch.
hipError_t launch_dw1_scatter_fixed(int64_t R, int64_t rank, int64_t Vt, const int32_t* prev,
                                    const uint8_t* mask, const float* dE, float* maxp,
                                    unsigned long long* acc, float* dW1, hipStream_t s);
hipError_t launch_conf_bwd(int dtype, int64_t R, int64_t Hd, int64_t rank, int conf_markov,
                           const void* hd, const void* E, const void* Wc, RowState rs, float g,
                           float c_a, float* part, int chunks, float* dWc, float* db, float* dh,
                           hipStream_t s);

// Vocabulary shards.  Per row, the shard's (lse_z, lse_t), -inf on unsupervised
// rows and for lse_t without a teacher.
hipError_t launch_shard_lse_out(int64_t R, int has_teacher, RowState rs, float2* out,
                                hipStream_t s);
// out [R, 2] = log-sum-exp over the G shards of parts [G, R, 2].
hipError_t launch_shard_merge_lse(int64_t G, int64_t R, const float* parts, float* out,
                                  hipStream_t s);
// rs.lse_z, rs.lse_t from merged log-sum-exps [R, 2] (0 on unsupervised rows).
hipError_t launch_shard_set_lse(int64_t R, int has_teacher, const float2* lse, RowState rs,
                                hipStream_t s);
// rs.l1, rs.S, rs.ce from the shard-summed (L1, S, z'_y, owners) [R, 4]
// (fp64); flag bit 1 where a supervised row's owner count is not 1.
hipError_t launch_shard_set_terms(int64_t R, const double* terms, RowState rs, uint32_t* flags,
                                  hipStream_t s);

}  // namespace dspark
