// Row-wise kernels of the DSpark loss (gfx950): masks, softmax/L1 sweeps,
// per-row terms, deterministic reductions and the backward helpers.
//
// Definitions (cited by page title and section):
//   Megatron-Bridge API page "bridge.training.post_training.dspark.loss":
//     module docstring (ce, raw L1 without 1/2, confidence BCE against the
//     label 1 - 0.5 L1, decay exp(-k / gamma), accept = 1 - 0.5 L1,
//     tau = sum_k cumprod(accept)_k + 1), `DSparkForwardOutput.eval_mask`
//     (contiguous supervised prefix), `_acceptance_report`, `_pair`.
//   Megatron-Bridge pull request #5241, merge note: masked rows are selected
//     away before any reduction and accept is clamped to [0, 1].
//   TorchSpec pull request #132, PR description: prefix mask as a cumprod.
//   NeMo-RL "DSpark Auxiliary Heads": Markov embedding W1[prev], confidence
//     logit = proj([hidden ; embedding]) + bias, zero on invalid slots.
#include "common.h"
#include "rowwise.h"

namespace dspark {

// ---------------------------------------------------------------- fill

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_u32(void* p, int64_t n, uint32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s,
                     static_cast<uint32_t*>(p), n, v);
  return hipGetLastError();
}

// ---------------------------------------------------------------- masks

// m_r = keep[b,n] * prod_{j<=k} [eval_j != 0]; w_r = m_r * exp(-k / gamma).
__device__ __forceinline__ bool slot_supervised(const uint8_t* eval, const uint8_t* keep, int64_t r,
                                                int K) {
  const int64_t blk = r / K;
  const int k = static_cast<int>(r - blk * K);
  if (keep && !keep[blk]) return false;
  for (int j = 0; j <= k; ++j)
    if (!eval[blk * K + j]) return false;
  return true;
}

__global__ void prep_rows_kernel(int64_t R, int K, const uint8_t* eval, const uint8_t* keep,
                                 const int32_t* tid, const int32_t* prev, int64_t Vd, int64_t Vt,
                                 int has_markov, float gamma, uint32_t set_bits, int check_target,
                                 uint8_t* mask, float* w, uint32_t* flags) {
  const int64_t r = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (r >= R) return;
  if (r == 0 && set_bits) atomicOr(flags, set_bits);
  const bool m = slot_supervised(eval, keep, r, K);
  const int k = static_cast<int>(r % K);
  mask[r] = m ? 1 : 0;
  w[r] = m ? (gamma > 0.f ? expf(-static_cast<float>(k) / gamma) : 1.f) : 0.f;
  if (m) {
    uint32_t f = 0;
    const int32_t y = tid[r];
    if (check_target && (y < 0 || y >= Vd)) f |= 1u;
    if (has_markov) {
      const int32_t pv = prev[r];
      if (pv < 0 || pv >= Vt) f |= 2u;
    }
    if (f) atomicOr(flags, f);
  }
}

hipError_t launch_prep_rows(int64_t R, int K, const uint8_t* eval, const uint8_t* keep,
                            const int32_t* tid, const int32_t* prev, int64_t Vd, int64_t Vt,
                            int has_markov, float gamma, uint32_t set_bits, uint8_t* mask, float* w,
                            uint32_t* flags, hipStream_t s, int check_target) {
  hipLaunchKernelGGL(prep_rows_kernel, dim3(static_cast<uint32_t>((R + 255) / 256)), dim3(256), 0,
                     s, R, K, eval, keep, tid, prev, Vd, Vt, has_markov, gamma, set_bits,
                     check_target, mask, w, flags);
  return hipGetLastError();
}

// E[r, :] = W1[prev_r, :] on supervised slots with an in-range id, else 0.
// One thread per 16-byte chunk.
template <typename T>
__global__ void gather_embed_kernel(int64_t R, int64_t rank, int64_t Vt, const int32_t* prev,
                                    const uint8_t* mask, const T* W1, T* E) {
  constexpr int KPC = Elem<T>::kPerChunk;
  const int64_t chunks = rank / KPC;
  const int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (i >= R * chunks) return;
  const int64_t r = i / chunks, c = i - r * chunks;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (mask[r]) {
    const int32_t pv = prev[r];
    if (pv >= 0 && pv < Vt) v = reinterpret_cast<const uint4*>(W1 + pv * rank)[c];
  }
  reinterpret_cast<uint4*>(E + r * rank)[c] = v;
}

hipError_t launch_gather_embed(int dtype, int64_t R, int64_t rank, int64_t Vt, const int32_t* prev,
                               const uint8_t* mask, const void* W1, void* E, hipStream_t s) {
  const int kpc = dtype == 1 ? 8 : 4;
  const int64_t n = R * (rank / kpc);
  if (n <= 0) return hipSuccess;
  dim3 grid(static_cast<uint32_t>((n + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(gather_embed_kernel<bf16_t>, grid, dim3(256), 0, s, R, rank, Vt, prev, mask,
                       static_cast<const bf16_t*>(W1), static_cast<bf16_t*>(E));
  else
    hipLaunchKernelGGL(gather_embed_kernel<float>, grid, dim3(256), 0, s, R, rank, Vt, prev, mask,
                       static_cast<const float*>(W1), static_cast<float*>(E));
  return hipGetLastError();
}

// ---------------------------------------------------------------- L1 sweep

constexpr int kSweepThreads = 256;

// log-sum-exp of a row from its per-tile (max, sum exp(x - max)) statistics.
// The same routine (same order) is used for the draft and the teacher row, so
// equal statistics give bitwise-equal results.
__device__ float merge_lse(const float2* st, int64_t n, float* fscr, double* dscr) {
  float m = -INFINITY;
  for (int64_t i = threadIdx.x; i < n; i += kSweepThreads) m = fmaxf(m, st[i].x);
  const float M = block_max<kSweepThreads>(m, fscr);
  double acc = 0.0;
  if (M != -INFINITY)
    for (int64_t i = threadIdx.x; i < n; i += kSweepThreads) {
      const float2 t = st[i];
      if (t.x != -INFINITY) acc += static_cast<double>(t.y) * static_cast<double>(dexp(t.x - M));
    }
  const double L = block_sum<kSweepThreads>(acc, dscr);
  return M + static_cast<float>(log(L));
}

// Per supervised row: lse of the corrected draft logits and of the teacher
// logits, then L1 = sum |p - q|, S = sum p sign(p - q) and CE = lse_z - z'_y.
__global__ __launch_bounds__(kSweepThreads) void l1_sweep_kernel(
    int64_t V, const float* Zp, const float* Tt, const float2* sz, const float2* st, int64_t nstat,
    const uint8_t* mask, const int32_t* tid, int has_teacher, float* lse_z, float* lse_t,
    float* l1, float* S, float* ce) {
  __shared__ float fscr[kSweepThreads / kWave];
  __shared__ double dscr[kSweepThreads / kWave];
  const int64_t r = blockIdx.x;
  if (!mask[r]) {
    if (threadIdx.x == 0) { lse_z[r] = 0.f; lse_t[r] = 0.f; l1[r] = 0.f; S[r] = 0.f; ce[r] = 0.f; }
    return;
  }
  const float lz = merge_lse(sz + r * nstat, nstat, fscr, dscr);
  float lt = 0.f;
  double sum_l1 = 0.0, sum_s = 0.0;
  if (has_teacher) {
    lt = merge_lse(st + r * nstat, nstat, fscr, dscr);
    const float4* z4 = reinterpret_cast<const float4*>(Zp + r * V);
    const float4* t4 = reinterpret_cast<const float4*>(Tt + r * V);
    const int64_t n4 = V / 4;
    float a1 = 0.f, a2 = 0.f;
#pragma unroll 4
    for (int64_t c = threadIdx.x; c < n4; c += kSweepThreads) {
      const float4 zz = z4[c], tt = t4[c];
      const float p0 = dexp(zz.x - lz), q0 = dexp(tt.x - lt);
      const float p1 = dexp(zz.y - lz), q1 = dexp(tt.y - lt);
      const float p2 = dexp(zz.z - lz), q2 = dexp(tt.z - lt);
      const float p3 = dexp(zz.w - lz), q3 = dexp(tt.w - lt);
      a1 += fabsf(p0 - q0) + fabsf(p1 - q1) + fabsf(p2 - q2) + fabsf(p3 - q3);
      a2 += p0 * sgnf(p0 - q0) + p1 * sgnf(p1 - q1) + p2 * sgnf(p2 - q2) + p3 * sgnf(p3 - q3);
    }
    sum_l1 = a1;
    sum_s = a2;
  }
  sum_l1 = block_sum<kSweepThreads>(sum_l1, dscr);
  sum_s = block_sum<kSweepThreads>(sum_s, dscr);
  if (threadIdx.x == 0) {
    int32_t y = tid[r];
    y = y < 0 ? 0 : (y >= V ? static_cast<int32_t>(V - 1) : y);
    lse_z[r] = lz;
    lse_t[r] = lt;
    l1[r] = static_cast<float>(sum_l1);
    S[r] = static_cast<float>(sum_s);
    ce[r] = lz - Zp[r * V + y];
  }
}

// The bias path's merge: one wave per row, both rows' tiles in one pass.
// Each lane folds its tiles (lane, lane + 64, ...) into a running (max m,
// fp64 sum l of 2^(tile sum) scaled to m); the lanes merge by an xor
// butterfly, whose pairwise merge is symmetric, so every lane ends with the
// same value.  The draft and the teacher row go through the same code, so
// equal statistics still give bitwise-equal log-sum-exps.
struct RunLse {
  float m;
  double l;
};
__device__ __forceinline__ void lse_fold(RunLse& a, float2 t) {
  if (t.x == -INFINITY) return;  // an empty tile
  const float mn = fmaxf(a.m, t.x);
  const double keep = a.m == -INFINITY ? 0.0 : a.l * static_cast<double>(dexp(a.m - mn));
  a.l = keep + static_cast<double>(t.y) * static_cast<double>(dexp(t.x - mn));
  a.m = mn;
}
__device__ __forceinline__ RunLse lse_wave_merge(RunLse a) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(a.m, o, kWave);
    const double l2 = __shfl_xor(a.l, o, kWave);
    const float mn = fmaxf(a.m, m2);
    const double x = a.m == -INFINITY ? 0.0 : a.l * static_cast<double>(dexp(a.m - mn));
    const double y = m2 == -INFINITY ? 0.0 : l2 * static_cast<double>(dexp(m2 - mn));
    a.l = x + y;
    a.m = mn;
  }
  return a;
}

constexpr int kLseWaves = 4;
__global__ __launch_bounds__(kLseWaves * kWave) void lse_rows_wave_kernel(
    int64_t R, const float2* sz, const float2* st, int64_t nstat, const uint8_t* mask,
    int has_teacher, float* lse_z, float* lse_t) {
  const int64_t r = blockIdx.x * static_cast<int64_t>(kLseWaves) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= R) return;
  if (!mask[r]) {
    if (lane == 0) { lse_z[r] = 0.f; lse_t[r] = 0.f; }
    return;
  }
  const float2* a = sz + r * nstat;
  const float2* b = st + r * nstat;
  RunLse za{-INFINITY, 0.0}, ta{-INFINITY, 0.0};
  constexpr int U = 4;
  for (int64_t i0 = lane; i0 < nstat; i0 += kWave * U) {
    float2 va[U], vb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = i0 + static_cast<int64_t>(u) * kWave;
      va[u] = i < nstat ? a[i] : make_float2(-INFINITY, 0.f);
      vb[u] = (has_teacher && i < nstat) ? b[i] : make_float2(-INFINITY, 0.f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      lse_fold(za, va[u]);
      lse_fold(ta, vb[u]);
    }
  }
  za = lse_wave_merge(za);
  ta = lse_wave_merge(ta);
  if (lane == 0) {
    lse_z[r] = za.m + static_cast<float>(log(za.l));
    lse_t[r] = has_teacher ? ta.m + static_cast<float>(log(ta.l)) : 0.f;
  }
}

hipError_t launch_lse_rows(int64_t R, const float2* sz, const float2* st, int64_t nstat,
                           const uint8_t* mask, int has_teacher, RowState rs, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(lse_rows_wave_kernel,
                     dim3(static_cast<uint32_t>((R + kLseWaves - 1) / kLseWaves)),
                     dim3(kLseWaves * kWave), 0, s, R, sz, st, nstat, mask, has_teacher, rs.lse_z,
                     rs.lse_t);
  return hipGetLastError();
}

hipError_t launch_l1_sweep(int64_t R, int64_t V, const float* Zp, const float* Tt,
                           const float2* sz, const float2* st, int64_t nstat, const uint8_t* mask,
                           const int32_t* tid, int has_teacher, RowState rs, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(l1_sweep_kernel, dim3(static_cast<uint32_t>(R)), dim3(kSweepThreads), 0, s, V,
                     Zp, Tt, sz, st, nstat, mask, tid, has_teacher, rs.lse_z, rs.lse_t, rs.l1, rs.S,
                     rs.ce);
  return hipGetLastError();
}

// ---------------------------------------------------------------- per-row finalize

// Confidence logit of row r, W_c . [h ; e] + b, by one wave (lane strides,
// then a fixed butterfly): the loss and the standalone head op share it, so
// both give the same value for a row.
// acc + sum over this lane's 8-element groups (lane, lane + 64, ...) of
// a . b, bf16 pairs widened to fp32, elements in order (n % 8 == 0, a and b
// 16-byte aligned).
__device__ __forceinline__ float dot8_lane(const bf16_t* a, const bf16_t* b, int64_t n, int lane,
                                           float acc) {
#pragma unroll 4
  for (int64_t i = static_cast<int64_t>(lane) * 8; i < n; i += 64 * 8) {
    const uint4 x = *reinterpret_cast<const uint4*>(a + i);
    const uint4 y = *reinterpret_cast<const uint4*>(b + i);
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc += __uint_as_float(xs[k] << 16) * __uint_as_float(ys[k] << 16);
      acc += __uint_as_float(xs[k] & 0xffff0000u) * __uint_as_float(ys[k] & 0xffff0000u);
    }
  }
  return acc;
}

template <typename T>
__device__ __forceinline__ float conf_logit_wave(int64_t r, int64_t Hd, int64_t rank,
                                                 int with_markov_conf, const T* hd, const T* E,
                                                 const T* Wc, const T* bc, int lane) {
  float acc = 0.f;
  const T* h = hd + r * Hd;
  if (sizeof(T) == 2 && Hd % 8 == 0) {
    // bf16: 8 consecutive elements per lane and load (16-byte aligned: the
    // rows and Wc start 16-byte aligned and Hd, rank are multiples of 8)
    acc = dot8_lane(reinterpret_cast<const bf16_t*>(h), reinterpret_cast<const bf16_t*>(Wc), Hd,
                    lane, acc);
    if (with_markov_conf)
      acc = dot8_lane(reinterpret_cast<const bf16_t*>(E + r * rank),
                      reinterpret_cast<const bf16_t*>(Wc + Hd), rank, lane, acc);
    return wave_sumf(acc) + Elem<T>::to_f32(bc[0]);
  }
  for (int64_t i = lane; i < Hd; i += 64) acc += Elem<T>::to_f32(h[i]) * Elem<T>::to_f32(Wc[i]);
  if (with_markov_conf) {
    const T* e = E + r * rank;
    for (int64_t j = lane; j < rank; j += 64)
      acc += Elem<T>::to_f32(e[j]) * Elem<T>::to_f32(Wc[Hd + j]);
  }
  return wave_sumf(acc) + Elem<T>::to_f32(bc[0]);
}

// One wave per row: confidence logit c = W_c . [h ; e] + b (0 on invalid
// slots), accept = clamp(1 - L1/2, 0, 1) (1 on invalid slots), BCE(c, accept)
// with the label held constant, and the outputs the caller asked for.
template <typename T>
__global__ __launch_bounds__(256) void finalize_rows_kernel(
    int64_t R, int64_t Hd, int64_t rank, int with_markov_conf, int has_conf, const T* hd,
    const T* E, const T* Wc, const T* bc, RowState rs, float* accept_out, float* row_terms,
    uint32_t* flags, float ce_a, float l1_a, float c_a) {
  const int lane = threadIdx.x & 63;
  const int64_t r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const bool m = rs.mask[r] != 0;
  float c = 0.f;
  if (m && has_conf) c = conf_logit_wave(r, Hd, rank, with_markov_conf, hd, E, Wc, bc, lane);
  if (lane != 0) return;
  float accept = 1.f, bce = 0.f, ce = 0.f, l1 = 0.f, dco = 0.f;
  if (m) {
    ce = rs.ce[r];
    l1 = rs.l1[r];
    accept = fminf(fmaxf(1.f - 0.5f * l1, 0.f), 1.f);
    if (has_conf) {
      bce = fmaxf(c, 0.f) - c * accept + log1pf(expf(-fabsf(c)));
      dco = 1.f / (1.f + expf(-c)) - accept;
    }
    const float lr = rs.w[r] * (ce_a * ce + l1_a * l1 + c_a * bce);
    if (!isfinite(lr)) atomicOr(flags, 4u);
  }
  rs.accept[r] = accept;
  rs.conf[r] = c;
  rs.bce[r] = bce;
  rs.dcoef[r] = dco;
  if (accept_out) accept_out[r] = accept;
  if (row_terms) {
    float4 t = make_float4(ce, l1, bce, c);
    reinterpret_cast<float4*>(row_terms)[r] = t;
  }
}

hipError_t launch_finalize_rows(int dtype, int64_t R, int64_t Hd, int64_t rank,
                                int with_markov_conf, int has_conf, const void* hd, const void* E,
                                const void* Wc, const void* bc, RowState rs, float* accept_out,
                                float* row_terms, uint32_t* flags, float ce_a, float l1_a,
                                float c_a, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  dim3 grid(static_cast<uint32_t>((R + 3) / 4));
  if (dtype == 1)
    hipLaunchKernelGGL(finalize_rows_kernel<bf16_t>, grid, dim3(256), 0, s, R, Hd, rank,
                       with_markov_conf, has_conf, static_cast<const bf16_t*>(hd),
                       static_cast<const bf16_t*>(E), static_cast<const bf16_t*>(Wc),
                       static_cast<const bf16_t*>(bc), rs, accept_out, row_terms, flags, ce_a,
                       l1_a, c_a);
  else
    hipLaunchKernelGGL(finalize_rows_kernel<float>, grid, dim3(256), 0, s, R, Hd, rank,
                       with_markov_conf, has_conf, static_cast<const float*>(hd),
                       static_cast<const float*>(E), static_cast<const float*>(Wc),
                       static_cast<const float*>(bc), rs, accept_out, row_terms, flags, ce_a, l1_a,
                       c_a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- reductions

constexpr int kRedThreads = 1024;

// accept pair (sum m*accept, sum m) and tau pair (sum over kept blocks of
// 1 + sum_k prod_{j<=k} m_j accept_j, number of kept blocks) for this thread's
// share, with m from the prefix rule.
__device__ void accept_tau_share(int64_t nblk, int K, const float* accept, const uint8_t* eval,
                                 const uint8_t* keep, double* acc_num, double* acc_den,
                                 double* tau_num, double* tau_den) {
  for (int64_t b = threadIdx.x; b < nblk; b += kRedThreads) {
    const bool kept = keep == nullptr || keep[b] != 0;
    double run = 1.0, tau = 1.0;
    bool alive = kept;
    for (int k = 0; k < K; ++k) {
      const int64_t r = b * K + k;
      alive = alive && eval[r] != 0;
      const double a = alive ? static_cast<double>(accept[r]) : 0.0;
      if (alive) { *acc_num += a; *acc_den += 1.0; }
      run *= a;
      tau += run;
    }
    if (kept) { *tau_num += tau; *tau_den += 1.0; }
  }
}

__device__ void block_sum_many(double* v, int n, double* scr) {
  // fixed-order reduction of n values per thread over the block
  for (int i = 0; i < n; ++i) v[i] = wave_sum(v[i]);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  constexpr int NW = kRedThreads / kWave;
  __syncthreads();
  if (l == 0)
    for (int i = 0; i < n; ++i) scr[i * NW + w] = v[i];
  __syncthreads();
  for (int i = 0; i < n; ++i) {
    double r = 0.0;
    for (int j = 0; j < NW; ++j) r += scr[i * NW + j];
    v[i] = r;
  }
}

__global__ __launch_bounds__(kRedThreads) void reduce_fwd_kernel(
    int64_t R, int64_t nblk, int K, RowState rs, const uint8_t* eval, const uint8_t* keep,
    float ce_a, float l1_a, float c_a, double* loss, int64_t* num_tokens, double* pairs) {
  __shared__ double scr[8 * (kRedThreads / kWave)];
  double v[8] = {0, 0, 0, 0, 0, 0, 0, 0};  // ce, l1, bce, tokens, acc_num, acc_den, tau_num, tau_den
  for (int64_t r = threadIdx.x; r < R; r += kRedThreads) {
    if (!rs.mask[r]) continue;
    const double w = rs.w[r];
    v[0] += w * static_cast<double>(rs.ce[r]);
    v[1] += w * static_cast<double>(rs.l1[r]);
    v[2] += w * static_cast<double>(rs.bce[r]);
    v[3] += 1.0;
  }
  accept_tau_share(nblk, K, rs.accept, eval, keep, &v[4], &v[5], &v[6], &v[7]);
  block_sum_many(v, 8, scr);
  if (threadIdx.x == 0) {
    *loss = static_cast<double>(ce_a) * v[0] + static_cast<double>(l1_a) * v[1] +
            static_cast<double>(c_a) * v[2];
    *num_tokens = static_cast<int64_t>(v[3]);
    pairs[0] = v[0]; pairs[1] = v[3];
    pairs[2] = v[1]; pairs[3] = v[3];
    pairs[4] = v[2]; pairs[5] = v[3];
    pairs[6] = v[4]; pairs[7] = v[5];
    pairs[8] = v[6]; pairs[9] = v[7];
  }
}

hipError_t launch_reduce_fwd(int64_t R, int64_t nblk, int K, RowState rs, const uint8_t* eval,
                             const uint8_t* keep, float ce_a, float l1_a, float c_a, double* loss,
                             int64_t* num_tokens, double* pairs, hipStream_t s) {
  hipLaunchKernelGGL(reduce_fwd_kernel, dim3(1), dim3(kRedThreads), 0, s, R, nblk, K, rs, eval,
                     keep, ce_a, l1_a, c_a, loss, num_tokens, pairs);
  return hipGetLastError();
}

__global__ __launch_bounds__(kRedThreads) void accept_report_kernel(int64_t nblk, int K,
                                                                    const float* accept,
                                                                    const uint8_t* eval,
                                                                    const uint8_t* keep,
                                                                    double* out4) {
  __shared__ double scr[4 * (kRedThreads / kWave)];
  double v[4] = {0, 0, 0, 0};
  accept_tau_share(nblk, K, accept, eval, keep, &v[0], &v[1], &v[2], &v[3]);
  block_sum_many(v, 4, scr);
  if (threadIdx.x == 0)
    for (int i = 0; i < 4; ++i) out4[i] = v[i];
}

hipError_t launch_accept_report(int64_t nblk, int K, const float* accept, const uint8_t* eval,
                                const uint8_t* keep, double* out4, hipStream_t s) {
  hipLaunchKernelGGL(accept_report_kernel, dim3(1), dim3(kRedThreads), 0, s, nblk, K, accept, eval,
                     keep, out4);
  return hipGetLastError();
}

// ---------------------------------------------------------------- gradient sweep

__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store4(bf16_t* p, float a, float b, float c, float d) {
  uint2 u;
  u.x = pack_bf16x2(a, b);
  u.y = pack_bf16x2(c, d);
  *reinterpret_cast<uint2*>(p) = u;
}
__device__ __forceinline__ float bf16_round(float x) { return bf16_to_f32(f32_to_bf16(x)); }

// G_v = g w [ce_a (p_v - [v = y]) + l1_a p_v (s_v - S)], s = sign(p - q).
// Writes dz (grad dtype); for bf16 operands also G as hi + lo bf16 parts (hi
// may alias dz) for the MFMA products dE = G W2 and dW2 = G^T E; for fp32
// operands G in fp32 (may alias dz).
template <typename GT>
__global__ __launch_bounds__(kSweepThreads) void grad_sweep_kernel(
    int64_t V, const float* Zp, const float* Tt, const int32_t* tid, RowState rs, int has_teacher,
    float g, float ce_a, float l1_a, GT* dz, bf16_t* ghi, bf16_t* glo, float* g32) {
  const int64_t r = blockIdx.x;
  const int64_t n4 = V / 4;
  const bool m = rs.mask[r] != 0;
  GT* dzr = dz + r * V;
  bf16_t* hir = ghi ? ghi + r * V : nullptr;
  bf16_t* lor = glo ? glo + r * V : nullptr;
  float* g32r = g32 ? g32 + r * V : nullptr;
  if (!m) {
    for (int64_t c = threadIdx.x; c < n4; c += kSweepThreads) {
      store4(dzr + 4 * c, 0.f, 0.f, 0.f, 0.f);
      if (hir) store4(hir + 4 * c, 0.f, 0.f, 0.f, 0.f);
      if (lor) store4(lor + 4 * c, 0.f, 0.f, 0.f, 0.f);
      if (g32r) store4(g32r + 4 * c, 0.f, 0.f, 0.f, 0.f);
    }
    return;
  }
  const float gw = g * rs.w[r];
  const float cc = gw * ce_a, cl = gw * l1_a;
  const float Sr = rs.S[r];
  const float lz = rs.lse_z[r], lt = rs.lse_t[r];
  int32_t y = tid[r];
  y = y < 0 ? 0 : (y >= V ? static_cast<int32_t>(V - 1) : y);
  const float4* z4 = reinterpret_cast<const float4*>(Zp + r * V);
  const float4* t4 = reinterpret_cast<const float4*>(Tt + r * V);
#pragma unroll 2
  for (int64_t c = threadIdx.x; c < n4; c += kSweepThreads) {
    const float4 zz = z4[c];
    float p[4] = {dexp(zz.x - lz), dexp(zz.y - lz), dexp(zz.z - lz), dexp(zz.w - lz)};
    float G[4];
    if (has_teacher) {
      const float4 tt = t4[c];
      const float q[4] = {dexp(tt.x - lt), dexp(tt.y - lt), dexp(tt.z - lt), dexp(tt.w - lt)};
#pragma unroll
      for (int e = 0; e < 4; ++e) G[e] = p[e] * (cc + cl * (sgnf(p[e] - q[e]) - Sr));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) G[e] = p[e] * cc;
    }
    const int64_t v0 = 4 * c;
    if (y >= v0 && y < v0 + 4) G[y - v0] -= cc;
    store4(dzr + v0, G[0], G[1], G[2], G[3]);
    if (hir) store4(hir + v0, G[0], G[1], G[2], G[3]);
    if (lor) {
      store4(lor + v0, G[0] - bf16_round(G[0]), G[1] - bf16_round(G[1]), G[2] - bf16_round(G[2]),
             G[3] - bf16_round(G[3]));
    }
    if (g32r) store4(g32r + v0, G[0], G[1], G[2], G[3]);
  }
}

hipError_t launch_grad_sweep(int grad_dtype, int64_t R, int64_t V, const float* Zp,
                             const float* Tt, const int32_t* tid, RowState rs, int has_teacher,
                             float g, float ce_a, float l1_a, void* dz, bf16_t* ghi, bf16_t* glo,
                             float* g32, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  dim3 grid(static_cast<uint32_t>(R));
  if (grad_dtype == 1)
    hipLaunchKernelGGL(grad_sweep_kernel<bf16_t>, grid, dim3(kSweepThreads), 0, s, V, Zp, Tt, tid,
                       rs, has_teacher, g, ce_a, l1_a, static_cast<bf16_t*>(dz), ghi, glo, g32);
  else
    hipLaunchKernelGGL(grad_sweep_kernel<float>, grid, dim3(kSweepThreads), 0, s, V, Zp, Tt, tid,
                       rs, has_teacher, g, ce_a, l1_a, static_cast<float*>(dz), ghi, glo, g32);
  return hipGetLastError();
}

// 8-row gradient sweep (bf16 operands).  One workgroup per group of 8 rows;
// thread t handles 4 consecutive vocabulary entries at a time for all 8 rows, so
// besides dz and the row-major low part of G it can write G in the k-blocked
// layout [rows/8][V][8] (8 consecutive rows of one entry in 16 bytes) that the
// row-contracting product dW2 = G^T E reads as K-contiguous chunks.
// hi = bf16(G) is dz itself when dz is bf16, else written to ghi_rm.
template <typename GT>
__global__ __launch_bounds__(kSweepThreads) void grad_sweep8_kernel(
    int64_t R, int64_t V, const float* Zp, const float* Tt, const int32_t* tid, RowState rs,
    int has_teacher, float g, float ce_a, float l1_a, GT* dz, bf16_t* ghi_rm, bf16_t* glo_rm,
    bf16_t* blk_hi, bf16_t* blk_lo) {
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * 8;
  bool mk[8];
  float lz[8], lt[8], cc[8], cl[8], Sr[8];
  int32_t yy[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t r = r0 + j;
    mk[j] = r < R && rs.mask[r] != 0;
    const float gw = mk[j] ? g * rs.w[r] : 0.f;
    lz[j] = mk[j] ? rs.lse_z[r] : 0.f;
    lt[j] = mk[j] ? rs.lse_t[r] : 0.f;
    Sr[j] = mk[j] ? rs.S[r] : 0.f;
    cc[j] = gw * ce_a;
    cl[j] = gw * l1_a;
    int32_t y = mk[j] ? tid[r] : -1;
    yy[j] = mk[j] ? (y < 0 ? 0 : (y >= V ? static_cast<int32_t>(V - 1) : y)) : -1;
  }
  const int64_t n4 = V / 4;
  for (int64_t c = threadIdx.x; c < n4; c += kSweepThreads) {
    const int64_t v0 = 4 * c;
    float G[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) G[j][e] = 0.f;
      if (!mk[j]) continue;
      const int64_t r = r0 + j;
      const float4 zz = reinterpret_cast<const float4*>(Zp + r * V)[c];
      const float p[4] = {dexp(zz.x - lz[j]), dexp(zz.y - lz[j]), dexp(zz.z - lz[j]),
                          dexp(zz.w - lz[j])};
      if (has_teacher) {
        const float4 tt = reinterpret_cast<const float4*>(Tt + r * V)[c];
        const float q[4] = {dexp(tt.x - lt[j]), dexp(tt.y - lt[j]), dexp(tt.z - lt[j]),
                            dexp(tt.w - lt[j])};
#pragma unroll
        for (int e = 0; e < 4; ++e) G[j][e] = p[e] * (cc[j] + cl[j] * (sgnf(p[e] - q[e]) - Sr[j]));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) G[j][e] = p[e] * cc[j];
      }
      if (yy[j] >= v0 && yy[j] < v0 + 4) G[j][yy[j] - v0] -= cc[j];
    }
    uint32_t hi[8][2], lo[8][2];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bf16_t h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[e] = f32_to_bf16(G[j][e]);
        l[e] = f32_to_bf16(G[j][e] - bf16_to_f32(h[e]));
      }
      hi[j][0] = h[0] | (static_cast<uint32_t>(h[1]) << 16);
      hi[j][1] = h[2] | (static_cast<uint32_t>(h[3]) << 16);
      lo[j][0] = l[0] | (static_cast<uint32_t>(l[1]) << 16);
      lo[j][1] = l[2] | (static_cast<uint32_t>(l[3]) << 16);
      const int64_t r = r0 + j;
      if (r < R) {
        if (sizeof(GT) == 2) {
          *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(dz) + r * V + v0) =
              make_uint2(hi[j][0], hi[j][1]);
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(dz) + r * V + v0) =
              make_float4(G[j][0], G[j][1], G[j][2], G[j][3]);
          *reinterpret_cast<uint2*>(ghi_rm + r * V + v0) = make_uint2(hi[j][0], hi[j][1]);
        }
        *reinterpret_cast<uint2*>(glo_rm + r * V + v0) = make_uint2(lo[j][0], lo[j][1]);
      }
    }
    // blocked: entry v0 + e of this row group = rows 0..7 packed in 16 bytes
    uint4* bh = reinterpret_cast<uint4*>(blk_hi + (static_cast<int64_t>(blockIdx.x) * V + v0) * 8);
    uint4* bl = reinterpret_cast<uint4*>(blk_lo + (static_cast<int64_t>(blockIdx.x) * V + v0) * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int w = e >> 1, sh = (e & 1) * 16;
      uint4 H, L;
      H.x = ((hi[0][w] >> sh) & 0xffffu) | (((hi[1][w] >> sh) & 0xffffu) << 16);
      H.y = ((hi[2][w] >> sh) & 0xffffu) | (((hi[3][w] >> sh) & 0xffffu) << 16);
      H.z = ((hi[4][w] >> sh) & 0xffffu) | (((hi[5][w] >> sh) & 0xffffu) << 16);
      H.w = ((hi[6][w] >> sh) & 0xffffu) | (((hi[7][w] >> sh) & 0xffffu) << 16);
      L.x = ((lo[0][w] >> sh) & 0xffffu) | (((lo[1][w] >> sh) & 0xffffu) << 16);
      L.y = ((lo[2][w] >> sh) & 0xffffu) | (((lo[3][w] >> sh) & 0xffffu) << 16);
      L.z = ((lo[4][w] >> sh) & 0xffffu) | (((lo[5][w] >> sh) & 0xffffu) << 16);
      L.w = ((lo[6][w] >> sh) & 0xffffu) | (((lo[7][w] >> sh) & 0xffffu) << 16);
      bh[e] = H;
      bl[e] = L;
    }
  }
}

hipError_t launch_grad_sweep8(int grad_dtype, int64_t R, int64_t rgroups, int64_t V,
                              const float* Zp, const float* Tt, const int32_t* tid, RowState rs,
                              int has_teacher, float g, float ce_a, float l1_a, void* dz,
                              bf16_t* ghi_rm, bf16_t* glo_rm, bf16_t* blk_hi, bf16_t* blk_lo,
                              hipStream_t s) {
  if (rgroups <= 0) return hipSuccess;
  dim3 grid(static_cast<uint32_t>(rgroups));
  if (grad_dtype == 1)
    hipLaunchKernelGGL(grad_sweep8_kernel<bf16_t>, grid, dim3(kSweepThreads), 0, s, R, V, Zp, Tt,
                       tid, rs, has_teacher, g, ce_a, l1_a, static_cast<bf16_t*>(dz), ghi_rm,
                       glo_rm, blk_hi, blk_lo);
  else
    hipLaunchKernelGGL(grad_sweep8_kernel<float>, grid, dim3(kSweepThreads), 0, s, R, V, Zp, Tt,
                       tid, rs, has_teacher, g, ce_a, l1_a, static_cast<float*>(dz), ghi_rm,
                       glo_rm, blk_hi, blk_lo);
  return hipGetLastError();
}

// out[c, r] = in[r, c] for a [rows, cols] bf16 matrix, through 64 x 64 LDS tiles.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(int64_t rows, int64_t cols,
                                                             const bf16_t* in, bf16_t* out) {
  __shared__ bf16_t t[64][66];
  const int64_t r0 = static_cast<int64_t>(blockIdx.y) * 64, c0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    t[i][tx] = (r < rows && c < cols) ? in[r * cols + c] : bf16_t(0);
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows) out[c * rows + r] = t[tx][i];
  }
}

hipError_t launch_transpose_bf16(int64_t rows, int64_t cols, const void* in, void* out,
                                 hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  dim3 grid(static_cast<uint32_t>((cols + 63) / 64), static_cast<uint32_t>((rows + 63) / 64));
  hipLaunchKernelGGL(transpose_bf16_kernel, grid, dim3(256), 0, s, rows, cols,
                     static_cast<const bf16_t*>(in), static_cast<bf16_t*>(out));
  return hipGetLastError();
}

// Eblk[rg, j, 0..7] = E[8 rg + 0..7, j] (zero past R), rg < rgroups.
__global__ void embed_blocked_kernel(int64_t R, int64_t rgroups, int64_t rank, const bf16_t* E,
                                     bf16_t* out) {
  const int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (i >= rgroups * rank) return;
  const int64_t rg = i / rank, j = i - rg * rank;
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t ra = rg * 8 + 2 * k, rb = ra + 1;
    const uint32_t a = ra < R ? E[ra * rank + j] : 0u;
    const uint32_t b = rb < R ? E[rb * rank + j] : 0u;
    w[k] = a | (b << 16);
  }
  reinterpret_cast<uint4*>(out)[i] = make_uint4(w[0], w[1], w[2], w[3]);
}

hipError_t launch_embed_blocked(int64_t R, int64_t rgroups, int64_t rank, const void* E, void* out,
                                hipStream_t s) {
  const int64_t n = rgroups * rank;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(embed_blocked_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256),
                     0, s, R, rgroups, rank, static_cast<const bf16_t*>(E),
                     static_cast<bf16_t*>(out));
  return hipGetLastError();
}

// out = a + b (fp32, n a multiple of 4).
__global__ void add2_kernel(int64_t n4, const float4* a, const float4* b, float4* out) {
  const int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (i >= n4) return;
  const float4 x = a[i], y = b[i];
  out[i] = make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
}

// out = sum of `parts` slices of n floats (split-K partials), in slice order.
__global__ void sum_parts_kernel(int64_t n4, int parts, const float4* p, float4* out) {
  const int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (i >= n4) return;
  float4 acc = p[i];
  for (int k = 1; k < parts; ++k) {
    const float4 x = p[k * n4 + i];
    acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
  }
  out[i] = acc;
}

hipError_t launch_sum_parts(int64_t n, int parts, const float* p, float* out, hipStream_t s) {
  const int64_t n4 = n / 4;
  if (n4 <= 0 || parts <= 0) return hipSuccess;
  hipLaunchKernelGGL(sum_parts_kernel, dim3(static_cast<uint32_t>((n4 + 255) / 256)), dim3(256), 0,
                     s, n4, parts, reinterpret_cast<const float4*>(p), reinterpret_cast<float4*>(out));
  return hipGetLastError();
}

hipError_t launch_add2(int64_t n, const float* a, const float* b, float* out, hipStream_t s) {
  const int64_t n4 = n / 4;
  if (n4 <= 0) return hipSuccess;
  hipLaunchKernelGGL(add2_kernel, dim3(static_cast<uint32_t>((n4 + 255) / 256)), dim3(256), 0, s,
                     n4, reinterpret_cast<const float4*>(a), reinterpret_cast<const float4*>(b),
                     reinterpret_cast<float4*>(out));
  return hipGetLastError();
}

// ---------------------------------------------------------------- backward helpers

// dE[r, j] = sum_s part[s, r, j] + dc_r W_c[Hd + j]  (dc_r = g w_r c_a (sigmoid(c_r) - accept_r)),
// zero on unsupervised rows.
template <typename T>
__global__ void de_reduce_kernel(int64_t R, int64_t rank, int splits, const float* part,
                                 RowState rs, int conf_markov, const T* Wc, int64_t Hd, float g,
                                 float c_a, float* dE) {
  const int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (i >= R * rank) return;
  const int64_t r = i / rank, j = i - r * rank;
  float v = 0.f;
  if (rs.mask[r]) {
    for (int s = 0; s < splits; ++s) v += part[s * R * rank + i];
    if (conf_markov) v += g * rs.w[r] * c_a * rs.dcoef[r] * Elem<T>::to_f32(Wc[Hd + j]);
  }
  dE[i] = v;
}

hipError_t launch_de_reduce(int dtype, int64_t R, int64_t rank, int splits, const float* part,
                            RowState rs, int conf_markov, const void* Wc, int64_t Hd, float g,
                            float c_a, float* dE, hipStream_t s) {
  const int64_t n = R * rank;
  if (n <= 0) return hipSuccess;
  dim3 grid(static_cast<uint32_t>((n + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(de_reduce_kernel<bf16_t>, grid, dim3(256), 0, s, R, rank, splits, part, rs,
                       conf_markov, static_cast<const bf16_t*>(Wc), Hd, g, c_a, dE);
  else
    hipLaunchKernelGGL(de_reduce_kernel<float>, grid, dim3(256), 0, s, R, rank, splits, part, rs,
                       conf_markov, static_cast<const float*>(Wc), Hd, g, c_a, dE);
  return hipGetLastError();
}

// dW1[prev_r, :] += dE[r, :] on supervised rows with an in-range id.
__global__ void dw1_scatter_kernel(int64_t R, int64_t rank, int64_t Vt, const int32_t* prev,
                                   const uint8_t* mask, const float* dE, float* dW1) {
  const int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (i >= R * rank) return;
  const int64_t r = i / rank, j = i - r * rank;
  if (!mask[r]) return;
  const int32_t pv = prev[r];
  if (pv < 0 || pv >= Vt) return;
  atomicAdd(dW1 + pv * rank + j, dE[i]);
}

hipError_t launch_dw1_scatter(int64_t R, int64_t rank, int64_t Vt, const int32_t* prev,
                              const uint8_t* mask, const float* dE, float* dW1, hipStream_t s) {
  const int64_t n = R * rank;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(dw1_scatter_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256),
                     0, s, R, rank, Vt, prev, mask, dE, dW1);
  return hipGetLastError();
}

// ---- deterministic dW1: fixed-point integer sums
// dW1[v, :] = sum of dE[r, :] over the supervised rows with prev_r = v, with
// the terms added as 64-bit fixed-point integers: integer addition is exact
// and associative, so the result does not depend on the order the atomics
// land in.  The fixed-point scale comes from the largest |dE| term M = 2^e m
// (m in [0.5, 1)): f = 62 - e - ceil(log2(R + 1)) fraction bits keep any sum of
// at most R terms below 2^62 in magnitude, and each term is rounded once, to
// a step of 2^-f, far below a float ulp of the sums.

// *out = max |dE| over supervised rows, as the bits of a non-negative float
// (zeroed by the caller).  Each workgroup's maximum is merged by an integer
// atomic maximum, which orders non-negative floats as their values; any order
// gives the same maximum.
__global__ __launch_bounds__(kRedThreads) void dw1_absmax_kernel(int64_t R, int64_t rank,
                                                                 const uint8_t* mask,
                                                                 const float* dE, unsigned* out) {
  __shared__ float scr[kRedThreads / kWave];
  float m = 0.f;
  const int64_t n = R * rank;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(kRedThreads) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kRedThreads) {
    const float a = fabsf(dE[i]);
    // NaN compares false: carry it as +inf so the caller sees a non-finite maximum
    const float v = a == a ? a : INFINITY;
    m = mask[i / rank] ? fmaxf(m, v) : m;
  }
  m = block_max<kRedThreads>(m, scr);
  if (threadIdx.x == 0) atomicMax(out, __float_as_uint(m));
}

__device__ __forceinline__ int dw1_fraction_bits(float maxabs, int64_t R) {
  int e = 0;
  frexpf(maxabs, &e);
  int lr = 0;
  while ((int64_t{1} << lr) < R + 1) ++lr;
  return 62 - e - lr;
}

// Each supervised row's terms as fixed-point integers added into acc [Vt, r]
// (zeroed by the caller).  A non-finite or zero maximum: plain float atomics
// into dW1 (zeroed by the caller) instead, so NaN / Inf propagate as without
// this mode.
__global__ void dw1_scatter_fixed_kernel(int64_t R, int64_t rank, int64_t Vt,
                                         const int32_t* prev, const uint8_t* mask,
                                         const float* dE, const float* maxp,
                                         unsigned long long* acc, float* dW1) {
  const int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (i >= R * rank) return;
  const int64_t r = i / rank, j = i - r * rank;
  if (!mask[r]) return;
  const int32_t pv = prev[r];
  if (pv < 0 || pv >= Vt) return;
  const float mx = *maxp;
  if (!(mx < INFINITY) || mx == 0.f) {
    atomicAdd(dW1 + pv * rank + j, dE[i]);
    return;
  }
  const int f = dw1_fraction_bits(mx, R);
  const long long q = __double2ll_rn(ldexp(static_cast<double>(dE[i]), f));
  atomicAdd(acc + pv * rank + j, static_cast<unsigned long long>(q));
}

// dW1 = acc 2^-f (rounded once to float), when the maximum was finite and
// nonzero; otherwise dW1 already holds the float sums.
__global__ void dw1_from_fixed_kernel(int64_t n, int64_t R, const unsigned long long* acc,
                                      const float* maxp, float* dW1) {
  const float mx = *maxp;
  if (!(mx < INFINITY) || mx == 0.f) return;
  const int f = dw1_fraction_bits(mx, R);
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    dW1[i] = static_cast<float>(ldexp(static_cast<double>(static_cast<long long>(acc[i])), -f));
}

hipError_t launch_dw1_scatter_fixed(int64_t R, int64_t rank, int64_t Vt, const int32_t* prev,
                                    const uint8_t* mask, const float* dE, float* maxp,
                                    unsigned long long* acc, float* dW1, hipStream_t s) {
  const int64_t n = R * rank;
  if (n <= 0) return hipSuccess;
  hipError_t e = launch_fill_u32(maxp, 1, 0u, s);
  if (e != hipSuccess) return e;
  int64_t mblocks = (n + kRedThreads - 1) / kRedThreads;
  if (mblocks > 512) mblocks = 512;
  hipLaunchKernelGGL(dw1_absmax_kernel, dim3(static_cast<uint32_t>(mblocks)), dim3(kRedThreads), 0,
                     s, R, rank, mask, dE, reinterpret_cast<unsigned*>(maxp));
  hipLaunchKernelGGL(dw1_scatter_fixed_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)),
                     dim3(256), 0, s, R, rank, Vt, prev, mask, dE, maxp, acc, dW1);
  const int64_t m = Vt * rank;
  int64_t blocks = (m + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(dw1_from_fixed_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s,
                     m, R, acc, maxp, dW1);
  return hipGetLastError();
}

// Confidence-head gradients.  Column f of the feature [h ; e] (f < F = Hd (+ r))
// and the bias (column F) are reduced over row chunks into part[chunk, F + 1];
// dh[r, i] = dc_r W_c[i].
template <typename T>
__global__ void conf_bwd_partial_kernel(int64_t R, int64_t Hd, int64_t rank, int64_t F,
                                        int64_t rows_per, const T* hd, const T* E, RowState rs,
                                        float g, float c_a, float* part) {
  const int64_t f = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  const int64_t r0 = blockIdx.y * rows_per;
  const int64_t r1 = (r0 + rows_per) < R ? (r0 + rows_per) : R;
  if (f > F) return;
  // rows unrolled with a select for unsupervised ones (no branch), so the
  // loads of several rows are in flight together; the select follows the
  // product, so whatever an unsupervised row holds contributes nothing
  const T* src = f < Hd ? hd + f : (f < F ? E + (f - Hd) : nullptr);
  const int64_t ld = f < Hd ? Hd : rank;
  float acc = 0.f;
#pragma unroll 8
  for (int64_t r = r0; r < r1; ++r) {
    const float x = src ? Elem<T>::to_f32(src[r * ld]) : 1.f;
    const float t = g * rs.w[r] * c_a * rs.dcoef[r] * x;
    acc += rs.mask[r] ? t : 0.f;
  }
  part[blockIdx.y * (F + 1) + f] = acc;
}

// bf16 inputs with Hd % 8 == 0: one thread per 8 consecutive features (one
// 16-byte load per row; a group never straddles h and e), plus one thread for
// the bias column.  Same per-feature sums, in the same row order.
__global__ void conf_bwd_partial8_kernel(int64_t R, int64_t Hd, int64_t rank, int64_t F,
                                         int64_t rows_per, const bf16_t* hd, const bf16_t* E,
                                         RowState rs, float g, float c_a, float* part) {
  const int64_t f0 = (blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x) * 8;
  const int64_t r0 = blockIdx.y * rows_per;
  const int64_t r1 = (r0 + rows_per) < R ? (r0 + rows_per) : R;
  if (f0 > F) return;
  float* out = part + blockIdx.y * (F + 1);
  if (f0 == F) {  // bias column: x = 1
    float acc = 0.f;
#pragma unroll 8
    for (int64_t r = r0; r < r1; ++r) {
      const float t = g * rs.w[r] * c_a * rs.dcoef[r];
      acc += rs.mask[r] ? t : 0.f;
    }
    out[F] = acc;
    return;
  }
  const bf16_t* src = f0 < Hd ? hd + f0 : E + (f0 - Hd);
  const int64_t ld = f0 < Hd ? Hd : rank;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int64_t r = r0; r < r1; ++r) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + r * ld);
    const float c = g * rs.w[r] * c_a * rs.dcoef[r];
    const bool m = rs.mask[r] != 0;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float t0 = c * __uint_as_float(w[i] << 16);
      const float t1 = c * __uint_as_float(w[i] & 0xffff0000u);
      acc[2 * i] += m ? t0 : 0.f;
      acc[2 * i + 1] += m ? t1 : 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) out[f0 + i] = acc[i];
}

__global__ void conf_bwd_final_kernel(int64_t F, int chunks, const float* part, float* dWc,
                                      float* db) {
  const int64_t f = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (f > F) return;
  double acc = 0.0;
#pragma unroll 8
  for (int c = 0; c < chunks; ++c) acc += part[c * (F + 1) + f];
  if (f < F) dWc[f] = static_cast<float>(acc);
  else *db = static_cast<float>(acc);
}

template <typename T>
__global__ void conf_dh_kernel(int64_t R, int64_t Hd, const T* Wc, RowState rs, float g, float c_a,
                               float* dh) {
  const int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (i >= R * Hd) return;
  const int64_t r = i / Hd, f = i - r * Hd;
  dh[i] = rs.mask[r] ? g * rs.w[r] * c_a * rs.dcoef[r] * Elem<T>::to_f32(Wc[f]) : 0.f;
}

hipError_t launch_conf_bwd(int dtype, int64_t R, int64_t Hd, int64_t rank, int conf_markov,
                           const void* hd, const void* E, const void* Wc, RowState rs, float g,
                           float c_a, float* part, int chunks, float* dWc, float* db, float* dh,
                           hipStream_t s) {
  const int64_t F = Hd + (conf_markov ? rank : 0);
  const int64_t rows_per = (R + chunks - 1) / chunks;
  dim3 grid(static_cast<uint32_t>((F + 1 + 255) / 256), static_cast<uint32_t>(chunks));
  if (dtype == 1 && Hd % 8 == 0) {
    dim3 grid8(static_cast<uint32_t>((F / 8 + 1 + 255) / 256), static_cast<uint32_t>(chunks));
    hipLaunchKernelGGL(conf_bwd_partial8_kernel, grid8, dim3(256), 0, s, R, Hd, rank, F, rows_per,
                       static_cast<const bf16_t*>(hd), static_cast<const bf16_t*>(E), rs, g, c_a,
                       part);
  } else if (dtype == 1)
    hipLaunchKernelGGL(conf_bwd_partial_kernel<bf16_t>, grid, dim3(256), 0, s, R, Hd, rank, F,
                       rows_per, static_cast<const bf16_t*>(hd), static_cast<const bf16_t*>(E), rs,
                       g, c_a, part);
  else
    hipLaunchKernelGGL(conf_bwd_partial_kernel<float>, grid, dim3(256), 0, s, R, Hd, rank, F,
                       rows_per, static_cast<const float*>(hd), static_cast<const float*>(E), rs, g,
                       c_a, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(conf_bwd_final_kernel, dim3(static_cast<uint32_t>((F + 1 + 255) / 256)),
                     dim3(256), 0, s, F, chunks, part, dWc, db);
  e = hipGetLastError();
  if (e != hipSuccess || dh == nullptr || R * Hd == 0) return e;
  dim3 g2(static_cast<uint32_t>((R * Hd + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(conf_dh_kernel<bf16_t>, g2, dim3(256), 0, s, R, Hd,
                       static_cast<const bf16_t*>(Wc), rs, g, c_a, dh);
  else
    hipLaunchKernelGGL(conf_dh_kernel<float>, g2, dim3(256), 0, s, R, Hd,
                       static_cast<const float*>(Wc), rs, g, c_a, dh);
  return hipGetLastError();
}

// ---------------------------------------------------------------- batch construction

// One thread per (sequence b, anchor n): the block's K rows.  Slot k is
// labelled by the token at a + k + 1 and its previous token is the one at
// a + k (slot 0: the anchor); the eval mask is the running product of the
// loss mask over the labels; a block whose anchor or first target is not in
// the loss mask (or out of range) is dropped and emits zeros.
__global__ void build_blocks_kernel(int64_t B, int64_t L, int64_t N, int K, const int32_t* ids,
                                    const uint8_t* lm, const int32_t* anchors, int32_t* target,
                                    int32_t* prev, uint8_t* evalm, uint8_t* keep) {
  const int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (i >= B * N) return;
  const int64_t b = i / N;
  const int64_t a = anchors[i];
  const int32_t* row = ids + b * L;
  const uint8_t* m = lm + b * L;
  const bool ok = a >= 0 && a + 1 < L && m[a] != 0 && m[a + 1] != 0;
  keep[i] = ok ? 1 : 0;
  int run = 1;
  for (int k = 0; k < K; ++k) {
    const int64_t r = i * K + k;
    int32_t t = 0, p = 0;
    uint8_t e = 0;
    if (ok) {
      const int64_t pos = a + k + 1;
      if (a + k < L) p = row[a + k];
      if (pos < L) {
        t = row[pos];
        run &= m[pos] != 0 ? 1 : 0;
      } else {
        run = 0;
      }
      e = static_cast<uint8_t>(run);
    }
    target[r] = t;
    prev[r] = p;
    evalm[r] = e;
  }
}

// Anchor candidates: position a of sequence b when a and a + 1 are both in
// the loss mask.
__global__ void anchor_candidates_kernel(int64_t B, int64_t L, const uint8_t* lm, uint8_t* out) {
  const int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (i >= B * L) return;
  const int64_t a = i % L;
  out[i] = (a + 1 < L && lm[i] != 0 && lm[i + 1] != 0) ? 1 : 0;
}

hipError_t launch_build_blocks(int64_t B, int64_t L, int64_t N, int K, const int32_t* ids,
                               const uint8_t* lm, const int32_t* anchors, int32_t* target,
                               int32_t* prev, uint8_t* evalm, uint8_t* keep, uint8_t* cand,
                               hipStream_t s) {
  if (B * N > 0) {
    hipLaunchKernelGGL(build_blocks_kernel, dim3(static_cast<uint32_t>((B * N + 255) / 256)),
                       dim3(256), 0, s, B, L, N, K, ids, lm, anchors, target, prev, evalm, keep);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (cand && B * L > 0)
    hipLaunchKernelGGL(anchor_candidates_kernel, dim3(static_cast<uint32_t>((B * L + 255) / 256)),
                       dim3(256), 0, s, B, L, lm, cand);
  return hipGetLastError();
}

// ---------------------------------------------------------------- head ops

// Standalone confidence head: c_r = W_c . [h_r ; e_r] + b on valid slots (e
// is the Markov embedding, when with_markov_conf), 0 on the others.
template <typename T>
__global__ __launch_bounds__(256) void conf_logits_kernel(int64_t R, int64_t Hd, int64_t rank,
                                                          int with_markov_conf, const T* hd,
                                                          const T* E, const T* Wc, const T* bc,
                                                          const uint8_t* mask, float* out) {
  const int lane = threadIdx.x & 63;
  const int64_t r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  if (mask && mask[r] == 0) {
    if (lane == 0) out[r] = 0.f;
    return;
  }
  const float c = conf_logit_wave(r, Hd, rank, with_markov_conf, hd, E, Wc, bc, lane);
  if (lane == 0) out[r] = c;
}

hipError_t launch_conf_logits(int dtype, int64_t R, int64_t Hd, int64_t rank, int with_markov_conf,
                              const void* hd, const void* E, const void* Wc, const void* bc,
                              const uint8_t* mask, float* out, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>((R + 3) / 4));
  if (dtype == 1)
    hipLaunchKernelGGL(conf_logits_kernel<bf16_t>, grid, dim3(256), 0, s, R, Hd, rank,
                       with_markov_conf, static_cast<const bf16_t*>(hd),
                       static_cast<const bf16_t*>(E), static_cast<const bf16_t*>(Wc),
                       static_cast<const bf16_t*>(bc), mask, out);
  else
    hipLaunchKernelGGL(conf_logits_kernel<float>, grid, dim3(256), 0, s, R, Hd, rank,
                       with_markov_conf, static_cast<const float*>(hd),
                       static_cast<const float*>(E), static_cast<const float*>(Wc),
                       static_cast<const float*>(bc), mask, out);
  return hipGetLastError();
}

// Rows r with mask[r] == 0 of an [R, N] fp32 array set to zero (one
// workgroup per row; valid rows untouched).
__global__ __launch_bounds__(256) void zero_masked_rows_kernel(int64_t N, const uint8_t* mask,
                                                               float* out) {
  const int64_t r = blockIdx.x;
  if (mask[r] != 0) return;
  float* row = out + r * N;
  for (int64_t i = threadIdx.x; i < N; i += blockDim.x) row[i] = 0.f;
}

hipError_t launch_zero_masked_rows(int64_t R, int64_t N, const uint8_t* mask, float* out,
                                   hipStream_t s) {
  if (R <= 0 || N <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_masked_rows_kernel, dim3(static_cast<uint32_t>(R)), dim3(256), 0, s, N,
                     mask, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- vocabulary shards

// A shard's log-sum-exp of z' and T per row: -inf on unsupervised rows (and for
// T without a teacher), the identity of the merge below.
__global__ void shard_lse_out_kernel(int64_t R, int has_teacher, RowState rs, float2* out) {
  const int64_t r = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (r >= R) return;
  const float ninf = -INFINITY;
  const bool m = rs.mask[r] != 0;
  out[r] = make_float2(m ? rs.lse_z[r] : ninf, m && has_teacher ? rs.lse_t[r] : ninf);
}

hipError_t launch_shard_lse_out(int64_t R, int has_teacher, RowState rs, float2* out,
                                hipStream_t s) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(shard_lse_out_kernel, dim3(static_cast<uint32_t>((R + 255) / 256)), dim3(256),
                     0, s, R, has_teacher, rs, out);
  return hipGetLastError();
}

// lse = M + log sum_g exp(lse_g - M), M = max_g lse_g, in fp64 over the shards
// in order; -inf when every shard gives -inf.
__global__ void shard_merge_lse_kernel(int64_t G, int64_t R, const float* parts, float* out) {
  const int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (i >= 2 * R) return;
  double M = -INFINITY;
  for (int64_t g = 0; g < G; ++g) M = fmax(M, static_cast<double>(parts[g * 2 * R + i]));
  double v = M;
  if (M > -INFINITY) {
    double l = 0.0;
    for (int64_t g = 0; g < G; ++g) l += exp(static_cast<double>(parts[g * 2 * R + i]) - M);
    v = M + log(l);
  }
  out[i] = static_cast<float>(v);
}

hipError_t launch_shard_merge_lse(int64_t G, int64_t R, const float* parts, float* out,
                                  hipStream_t s) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(shard_merge_lse_kernel, dim3(static_cast<uint32_t>((2 * R + 255) / 256)),
                     dim3(256), 0, s, G, R, parts, out);
  return hipGetLastError();
}

// Row state from the merged log-sum-exps (0 on unsupervised rows, lse_t 0
// without a teacher, as the unsplit forward leaves them).
__global__ void shard_set_lse_kernel(int64_t R, int has_teacher, const float2* lse, RowState rs) {
  const int64_t r = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (r >= R) return;
  const bool m = rs.mask[r] != 0;
  const float2 v = lse[r];
  rs.lse_z[r] = m ? v.x : 0.f;
  rs.lse_t[r] = m && has_teacher ? v.y : 0.f;
}

hipError_t launch_shard_set_lse(int64_t R, int has_teacher, const float2* lse, RowState rs,
                                hipStream_t s) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(shard_set_lse_kernel, dim3(static_cast<uint32_t>((R + 255) / 256)), dim3(256),
                     0, s, R, has_teacher, lse, rs);
  return hipGetLastError();
}

// Row state from the shard-summed terms [R, 4] (L1, S, z'_y, owners): CE =
// lse_z - z'_y on supervised rows, every term 0 on the others; a supervised
// row whose target no shard or several shards own sets flag bit 1.
__global__ void shard_set_terms_kernel(int64_t R, const double* terms, RowState rs,
                                       uint32_t* flags) {
  const int64_t r = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (r >= R) return;
  const bool m = rs.mask[r] != 0;
  rs.l1[r] = m ? static_cast<float>(terms[4 * r]) : 0.f;
  rs.S[r] = m ? static_cast<float>(terms[4 * r + 1]) : 0.f;
  rs.ce[r] = m ? rs.lse_z[r] - static_cast<float>(terms[4 * r + 2]) : 0.f;
  if (m && terms[4 * r + 3] != 1.0) atomicOr(flags, 1u);
}

hipError_t launch_shard_set_terms(int64_t R, const double* terms, RowState rs, uint32_t* flags,
                                  hipStream_t s) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(shard_set_terms_kernel, dim3(static_cast<uint32_t>((R + 255) / 256)),
                     dim3(256), 0, s, R, terms, rs, flags);
  return hipGetLastError();
}

}  // namespace dspark
