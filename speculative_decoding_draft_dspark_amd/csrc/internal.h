// Internal launch interface between the C ABI (capi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

// One operand of C[M,N] = A[M,K] . B[N,K]^T, possibly made of two K segments.
// The K axis is padded: segment s covers k in [s*kpad, s*kpad + kseg), and
// k in [s*kpad + kseg, (s+1)*kpad) reads as zero.  kpad must be a multiple of
// the GEMM's BK (64 for bf16, 32 for fp32) and equal for A and B.
//   LAYOUT_KC: element (i, k) of segment s at seg[s][i * ld + k]   (row i K-contiguous)
//   LAYOUT_MC: element (i, k) of segment s at seg[s][k * ld + i]   (row i strided)
//   LAYOUT_KB: element (i, k) of segment s at
//              seg[s][(k / c) * c * ld + i * c + k % c]  (k-blocked: c = elements per
//              16-byte chunk, i.e. c consecutive k of one row are contiguous)
// Byte offsets i*ld + k (resp. k*ld + i) within one 256-row tile must stay below 2^31.
// KC: [rows][K] (K contiguous); MC: [K][rows] read element-wise; KB: k-blocked
// [K/c][rows][c]; MK: [K][rows] (rows contiguous) read with transposing LDS loads.
enum OperandLayout { LAYOUT_KC = 0, LAYOUT_MC = 1, LAYOUT_KB = 2, LAYOUT_MK = 3 };

struct Operand {
  const void* seg[2];
  int64_t kseg;
  int64_t kpad;
  int64_t ld;
  int layout;
  int nseg;
};

// Padded K extent of an operand segment for the GEMM of element size `esize`.
inline int64_t gemm_kpad(int64_t k, int esize) {
  const int64_t bk = esize == 2 ? 64 : 32;
  return (k + bk - 1) / bk * bk;
}

enum Epilogue { EPI_STATS = 0, EPI_STORE = 1, EPI_PARTIAL = 2 };

struct EpiParams {
  float* C;            // fp32 [M, ldc] (EPI_PARTIAL: [splits, M, ldc])
  int64_t ldc;
  const void* X;       // EPI_STATS: optional addend [M, ldx] of the operand dtype
  int64_t ldx;
  float2* stats;       // EPI_STATS: [M, nstat] (tile max, tile sum of exp(x - max))
  int64_t nstat;
};

// One GEMM of a multi-job launch: C = A . B^T with K = A.kseg * A.nseg (0 allowed).
struct GemmJob {
  Operand A, B;
  EpiParams ep;
  int64_t K;
};

// dtype: 0 = fp32, 1 = bf16.  splits > 1 only with EPI_PARTIAL.  tag (EPI_STATS):
// 0 = corrected draft logits, 1 = teacher logits (separate kernel symbols).
// EPI_STATS jobs sharing M and N (the corrected draft logits, then the teacher
// logits), fused into one launch where the DMA path applies.
hipError_t launch_logits(int dtype, int64_t M, int64_t N, const Operand* A, const Operand* B,
                         const EpiParams* ep, int njobs, hipStream_t s);

hipError_t launch_gemm(int dtype, int epi, int tag, int64_t M, int64_t N, const Operand& A,
                       const Operand& B, int splits, const EpiParams& ep, hipStream_t s);

// bf16 products of the backward pass on the 4-wave kernel: C[split] = A . B^T
// over K split in `splits` ranges (fp32 partials [splits, M, ldc]).  Each
// operand is KC or MK; every K segment a multiple of 32; MK operands need
// rows % 8 == 0.  tag names the kernel symbol (2 = dE, 3 = dW2).
bool w4p_ok(const Operand& A, const Operand& B, int64_t M, int64_t N);
hipError_t launch_gemm_w4p(int tag, int64_t M, int64_t N, const Operand& A, const Operand& B,
                           int splits, float* C, int64_t ldc, hipStream_t s);

}  // namespace dspark
