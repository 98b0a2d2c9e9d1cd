// Vocabulary sweeps over the corrected draft logits z' = z + E . W2^T that
// recompute the low-rank Markov bias tile by tile (bf16 MFMA) instead of
// reading a stored z' (NeMo-RL "DSpark Auxiliary Heads": the Markov head adds
// W2 . W1[prev] to the draft logits).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rowwise.h"

namespace dspark {

// Shapes the bias sweeps handle: vocabulary V (a multiple of 8, below 2^24)
// and rank in {0, 32, 64, 128, 256} (0 = no Markov head: z' = z).
bool bias_sweep_ok(int64_t V, int64_t rank);

// Row tiles of 256 rows x vocabulary splits of `vsplit` columns (a multiple of
// 64) each sweep launches.
struct BiasGrid {
  int64_t row_tiles, splits, vsplit;
};
BiasGrid bias_grid(int64_t R, int64_t V);

// Per (row, 64-column tile) maximum and fixed-point exp-sum of z' into sz
// [R, nstat], computed exactly as the logits GEMM epilogue computes them for T.
// z [R, V] bf16, E [R, rank] bf16 (zero rows on unsupervised slots), W2 [V, rank] bf16.
hipError_t launch_bias_stats(int64_t R, int64_t V, int64_t rank, const bf16_t* z, const bf16_t* E,
                             const bf16_t* W2, float2* sz, int64_t nstat, hipStream_t s);

// On supervised rows, per vocabulary split: sum |p - q| and sum p sign(p - q)
// (fp64 partials [splits, R] each), with p = exp(z' - lse_z), q = exp(T - lse_t);
// and sign(p - q) of every element as two bits (p > q, p < q) into `signs`
// (bias_signs_words() uint2 words) for the gradient pass.  Without a teacher
// (T == nullptr) there is nothing to sweep: no launch.
hipError_t launch_bias_l1(int64_t R, int64_t V, int64_t rank, const bf16_t* z, const bf16_t* E,
                          const bf16_t* W2, const float* T, const int32_t* tid, RowState rs,
                          double* part_l1, double* part_s, uint2* signs, hipStream_t s);

// uint2 words of the sign bits launch_bias_l1 writes.
int64_t bias_signs_words(int64_t R, int64_t V);

// Per row: L1 and S from the split partials (0 without a teacher) and
// CE = lse_z - z'_y with z'_y = z_y + E_row . W2_y (masked rows: 0).
hipError_t launch_bias_l1_finish(int64_t R, int64_t V, int64_t rank, int splits, int has_teacher,
                                 const double* part_l1, const double* part_s, const bf16_t* z,
                                 const bf16_t* E, const bf16_t* W2, const int32_t* tid,
                                 RowState rs, hipStream_t s);

// G = g w [ce_a (p - [v = y]) + l1_a p (sign(p - q) - S)] (0 on unsupervised rows):
// dz in the gradient dtype, and with fp32 dz (grad_dtype 0) ghi = bf16(G) and,
// if not null, glo = bf16(G - bf16(G)).  With bf16 dz (grad_dtype 1) dz is
// bf16(G) itself and ghi, glo must be null.
// With a teacher, sign(p - q) comes from the bits launch_bias_l1 wrote (T is
// not read again).
// shard: a target id outside [0, V) lives in another vocabulary shard (no
// target term here) instead of being clamped.
hipError_t launch_bias_grad(int grad_dtype, int64_t R, int64_t V, int64_t rank, const bf16_t* z,
                            const bf16_t* E, const bf16_t* W2, const uint2* signs,
                            const int32_t* tid, RowState rs, int has_teacher, float g, float ce_a,
                            float l1_a, void* dz, bf16_t* ghi, bf16_t* glo, hipStream_t s,
                            int shard = 0);

// z' = z + E . W2^T into out [R, V] (fp32), zero rows where valid[row] == 0
// (valid null: every row written): the Markov head op on the sweep path.
hipError_t launch_bias_store(int64_t R, int64_t V, int64_t rank, const bf16_t* z,
                             const bf16_t* E, const bf16_t* W2, const uint8_t* valid, float* out,
                             hipStream_t s);

// Vocabulary shard: part [R, 4] (fp64) = this shard's L1, S and, on the shard
// that owns the target, z'_y and 1 (0 and 0 on the others and on unsupervised
// rows).
hipError_t launch_bias_l1_shard(int64_t R, int64_t V, int64_t rank, int splits, int has_teacher,
                                const double* part_l1, const double* part_s, const bf16_t* z,
                                const bf16_t* E, const bf16_t* W2, const int32_t* tid,
                                RowState rs, double* part, hipStream_t s);

}  // namespace dspark
