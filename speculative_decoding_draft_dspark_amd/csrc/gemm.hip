// MFMA GEMM C[M,N] = A[M,K] . B[N,K]^T for the DSpark loss (gfx950).
//
// Used for the dense contractions of the loss:
//   - the teacher lm_head projection T = H_t . LM^T (TorchSpec pull request
//     #132, PR description: teacher = target lm_head on the final hidden state),
//   - the Markov low-rank bias z' = z + E . W2^T with E = W1[prev] (NeMo-RL
//     "DSpark Auxiliary Heads", Inputs and Outputs),
//   - the backward products dE = G . W2 and dW2 = G^T . E.
//
// Design: BM x BN x BK tiles staged through LDS (double buffered, XOR-swizzled
// 16-byte chunks so MFMA operand reads are bank-conflict free), each wave
// computing a (BM/WM) x (BN/WN) sub-tile with 16x16 MFMAs
// (v_mfma_f32_16x16x32_bf16 for bf16, v_mfma_f32_16x16x4_f32 for fp32).  The
// tile order is XCD-aware (each of the 8 XCDs works a contiguous range of a
// grouped-M ordering so operand tiles are shared through its own L2).
// Operands may be K-contiguous or M-contiguous (the latter is transposed on its
// way into LDS) and may consist of two K segments (used for hi/lo splits).
#include "common.h"
#include "internal.h"

namespace dspark {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
  __device__ __forceinline__ static void run(f32x4_v& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a),
                                                  __builtin_bit_cast(bf16x8_v, b), acc, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  // A 16-byte chunk holds 4 consecutive k; the 4 MFMAs each take one of them.
  // A and B use the same k permutation, so the contraction is unchanged.
  __device__ __forceinline__ static void run(f32x4_v& acc, const u32x4& a, const u32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

// Buffer resource: raw (stride 0) buffer of kNumRecords bytes; word 3 holds the
// gfx9 data-format bits that make untyped dword loads valid.
constexpr int kNumRecords = 0x7fffffff;
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;

// LDS row of a tile = 8 chunks of 16 bytes; chunk c of row m sits at slot c ^ swz(m).
__device__ __forceinline__ int swz(int m) { return (m ^ (m >> 3)) & 7; }

// Per-lane 32-bit offsets (in elements, relative to the tile base) and row
// validity for one operand tile of ROWS rows x 8 chunks, fixed for the whole
// K loop.  kcontig: lane chunk (row, c) -> row*ld + c*KPC; mcontig: lane chunk
// (kr, mc) -> kr*ld + mc*KPC (KPC consecutive rows at one k).
template <typename T, int ROWS, int NT, bool MC>
struct TileLoader {
  static constexpr int KPC = Elem<T>::kPerChunk;
  static constexpr int PER = ROWS * 8 / NT;
  static constexpr int BK = 8 * KPC;
  static constexpr int MCH = ROWS / KPC;
  uint32_t off[PER];
  uint32_t rowok;   // bit p: row of chunk p is inside the operand
  int kofs[PER];    // k of chunk p within the K-tile

  __device__ __forceinline__ void init(const Operand& op, int64_t r0, int64_t rlim) {
    rowok = 0;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int idx = threadIdx.x + p * NT;
      int row, k;
      if (!MC) {
        row = idx >> 3;
        k = (idx & 7) * KPC;
        off[p] = static_cast<uint32_t>(row * op.ld + k);
      } else {
        const int mc = (idx & 7) + ((idx >> 3) / BK) * 8;
        k = (idx >> 3) % BK;
        row = mc * KPC;
        off[p] = static_cast<uint32_t>(k * op.ld + row);
      }
      kofs[p] = k;
      if (r0 + row < rlim) rowok |= 1u << p;
    }
  }

  // Load K-tile kt (global k range [kt*BK, kt*BK+BK) of the padded K axis)
  // with buffer loads: a uniform (SGPR) resource based at the tile origin and
  // a 32-bit byte offset per lane.  Chunks outside the operand get an offset
  // past num_records, for which the hardware returns zeros.
  __device__ __forceinline__ void load(const Operand& op, int64_t r0, int kt, int64_t kend,
                                       u32x4* reg) const {
    const int64_t kg = static_cast<int64_t>(kt) * BK;   // padded-K position (uniform)
    const int s = static_cast<int>(kg / op.kpad);
    const int64_t kk0 = kg - s * op.kpad;                  // k within segment s
    const int64_t kvalid = op.kseg - kk0;                 // chunks with k < kvalid are real
    const T* base = static_cast<const T*>(op.seg[s]) +
                    (MC ? kk0 * op.ld + r0 : r0 * op.ld + kk0);
    const int64_t klim = kend - kg;                        // split-K end
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), 0, kNumRecords, kRsrcWord3);
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const bool ok = ((rowok >> p) & 1u) && kofs[p] < kvalid && kofs[p] < klim;
      const uint32_t o = ok ? off[p] * static_cast<uint32_t>(sizeof(T)) : kOutOfRange;
      reg[p] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, o, 0, 0);
    }
  }
};

// Registers -> LDS (K-contiguous, swizzled) for the tile loaded by TileLoader.
template <typename T, int ROWS, int NT, bool MC>
__device__ __forceinline__ void store_tile(u32x4* lds, const u32x4* reg) {
  constexpr int KPC = Elem<T>::kPerChunk;
  constexpr int PER = ROWS * 8 / NT;
  constexpr int BK = 8 * KPC;
  if (!MC) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int idx = threadIdx.x + p * NT;
      const int row = idx >> 3, c = idx & 7;
      lds[row * 8 + (c ^ swz(row))] = reg[p];
    }
  } else {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int idx = threadIdx.x + p * NT;
      const int mc = (idx & 7) + ((idx >> 3) / BK) * 8;
      const int kr = (idx >> 3) % BK;
      const int kc = kr / KPC, ke = kr % KPC;
      T vals[KPC];
      __builtin_memcpy(vals, &reg[p], 16);
#pragma unroll
      for (int j = 0; j < KPC; ++j) {
        const int m = mc * KPC + j;
        reinterpret_cast<T*>(&lds[m * 8 + (kc ^ swz(m))])[ke] = vals[j];
      }
    }
  }
}

template <typename T, int BM, int BN, int WM, int WN, int EPI, bool AMC, bool BMC>
__global__ __launch_bounds__(WM* WN * 64, 1) void gemm_kernel(int64_t M, int64_t N, int64_t K,
                                                              int64_t kper, Operand A, Operand B,
                                                              EpiParams ep, int group_m) {
  constexpr int NT = WM * WN * 64;
  constexpr int KPC = Elem<T>::kPerChunk;
  constexpr int BK = 8 * KPC;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int A_CH = BM * 8, B_CH = BN * 8;
  constexpr int A_PER = A_CH / NT, B_PER = B_CH / NT;
  static_assert(A_CH % NT == 0 && B_CH % NT == 0, "tile / thread mismatch");
  static_assert(EPI != EPI_STATS || BN == kStatTile, "stats epilogue needs BN == stat tile");

  __shared__ u32x4 lds[2 * (A_CH + B_CH)];

  // ---- tile assignment: XCD-contiguous ranges of a grouped-M order
  const int64_t nM = (M + BM - 1) / BM, nN = (N + BN - 1) / BN;
  const int64_t tiles = nM * nN;
  int64_t b = blockIdx.x;
  const int64_t per_xcd = tiles / 8;
  if (b < per_xcd * 8) b = (b % 8) * per_xcd + b / 8;
  const int64_t gsz = static_cast<int64_t>(group_m) * nN;
  const int64_t fm = (b / gsz) * group_m;
  const int64_t gm = (nM - fm) < group_m ? (nM - fm) : group_m;
  const int64_t tm = fm + (b % gsz) % gm;
  const int64_t tn = (b % gsz) / gm;
  const int64_t m0 = tm * BM, n0 = tn * BN;

  const int64_t kbeg = static_cast<int64_t>(blockIdx.y) * kper;
  const int64_t kend = (kbeg + kper) < K ? (kbeg + kper) : K;
  const int nk = kend > kbeg ? static_cast<int>((kend - kbeg + BK - 1) / BK) : 0;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int g = lane >> 4, cl = lane & 15;

  f32x4_v acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};

  if (nk > 0) {
    TileLoader<T, BM, NT, AMC> la;
    TileLoader<T, BN, NT, BMC> lb;
    la.init(A, m0, M);
    lb.init(B, n0, N);
    const int kt0 = static_cast<int>(kbeg / BK);
    u32x4 ra[A_PER], rb[B_PER];
    la.load(A, m0, kt0, kend, ra);
    lb.load(B, n0, kt0, kend, rb);
    store_tile<T, BM, NT, AMC>(lds, ra);
    store_tile<T, BN, NT, BMC>(lds + A_CH, rb);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      u32x4* As = lds + (kt & 1) * (A_CH + B_CH);
      u32x4* Bs = As + A_CH;
      const bool more = kt + 1 < nk;
      if (more) {
        la.load(A, m0, kt0 + kt + 1, kend, ra);
        lb.load(B, n0, kt0 + kt + 1, kend, rb);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int c = s * 4 + g;
        u32x4 af[TM], bfr[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int m = wm * WTM + i * 16 + cl;
          af[i] = As[m * 8 + (c ^ swz(m))];
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = wn * WTN + j * 16 + cl;
          bfr[j] = Bs[n * 8 + (c ^ swz(n))];
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) Mfma<T>::run(acc[i][j], af[i], bfr[j]);
      }
      if (more) {
        u32x4* An = lds + ((kt + 1) & 1) * (A_CH + B_CH);
        store_tile<T, BM, NT, AMC>(An, ra);
        store_tile<T, BN, NT, BMC>(An + A_CH, rb);
      }
      __syncthreads();
    }
  }

  // ---- epilogue.  Lane (g, cl) of wave (wm, wn) holds, for sub-tile (i, j) and
  // element e, the output at row wm*WTM + 16 i + 4 g + e, column wn*WTN + 16 j + cl.
  if (EPI == EPI_STORE || EPI == EPI_PARTIAL) {
    float* C = ep.C;
    if (EPI == EPI_PARTIAL) C += static_cast<int64_t>(blockIdx.y) * M * ep.ldc;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t row = m0 + wm * WTM + i * 16 + g * 4 + e;
        if (row >= M) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int64_t col = n0 + wn * WTN + j * 16 + cl;
          if (col < N) C[row * ep.ldc + col] = acc[i][j][e];
        }
      }
    return;
  }

  // EPI_STATS: C = acc (+ X), plus per-(row, stat tile) max and fixed-point exp-sum.
  const T* X = static_cast<const T*>(ep.X);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t row = m0 + wm * WTM + i * 16 + g * 4 + e;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t col = n0 + wn * WTN + j * 16 + cl;
        float x = acc[i][j][e];
        if (row < M && col < N) {
          if (X) x += Elem<T>::to_f32(X[row * ep.ldx + col]);
          ep.C[row * ep.ldc + col] = x;
        }
        acc[i][j][e] = x;
      }
    }
  float* smax = reinterpret_cast<float*>(lds);           // [WN][BM]
  uint64_t* ssum = reinterpret_cast<uint64_t*>(smax + WN * BM);        // [WN][BM]
  // row maxima over this wave's columns, then across the WN waves of the row
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t col = n0 + wn * WTN + j * 16 + cl;
        if (col < N) mx = fmaxf(mx, acc[i][j][e]);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
      if (cl == 0) smax[wn * BM + wm * WTM + i * 16 + g * 4 + e] = mx;
    }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rl = wm * WTM + i * 16 + g * 4 + e;
      float mx = smax[rl];
#pragma unroll
      for (int w = 1; w < WN; ++w) mx = fmaxf(mx, smax[w * BM + rl]);
      uint64_t sum = 0;
      if (mx != -INFINITY) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int64_t col = n0 + wn * WTN + j * 16 + cl;
          if (col < N) sum += static_cast<uint64_t>(rintf(dexp(acc[i][j][e] - mx) * kFixScale));
        }
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const uint32_t lo = __shfl_xor(static_cast<uint32_t>(sum), o, kWave);
        const uint32_t hi = __shfl_xor(static_cast<uint32_t>(sum >> 32), o, kWave);
        sum += (static_cast<uint64_t>(hi) << 32) | lo;
      }
      if (cl == 0) ssum[wn * BM + rl] = sum;
    }
  __syncthreads();
  if (wn == 0 && cl == 0) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rl = wm * WTM + i * 16 + g * 4 + e;
        const int64_t row = m0 + rl;
        if (row >= M) continue;
        float mx = smax[rl];
        uint64_t sum = ssum[rl];
#pragma unroll
        for (int w = 1; w < WN; ++w) {
          mx = fmaxf(mx, smax[w * BM + rl]);
          sum += ssum[w * BM + rl];
        }
        const float l = static_cast<float>(static_cast<double>(sum) * (1.0 / 2147483648.0));
        ep.stats[row * ep.nstat + tn] = make_float2(mx, l);
      }
  }
}

namespace {
constexpr int kGroupM = 8;

template <typename T, int BM, int BN, int WM, int WN, int EPI, bool AMC, bool BMC>
hipError_t launch_cfg(int64_t M, int64_t N, const Operand& A, const Operand& B, int splits,
                      const EpiParams& ep, hipStream_t s) {
  constexpr int BK = 8 * Elem<T>::kPerChunk;
  const int64_t K = A.kpad * A.nseg;
  const int64_t nM = (M + BM - 1) / BM, nN = (N + BN - 1) / BN;
  int64_t kper = K;
  if (splits > 1) kper = ((K + splits - 1) / splits + BK - 1) / BK * BK;
  dim3 grid(static_cast<uint32_t>(nM * nN), static_cast<uint32_t>(splits), 1);
  if (A.mcontig != AMC || B.mcontig != BMC) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, EPI, AMC, BMC>), grid, dim3(WM * WN * 64), 0, s, M, N,
                     K, kper, A, B, ep, kGroupM);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(int epi, int64_t M, int64_t N, const Operand& A, const Operand& B, int splits,
                    const EpiParams& ep, hipStream_t s) {
  switch (epi) {
    // logits / teacher projections: both operands K-contiguous
    case EPI_STATS: return launch_cfg<T, 256, 256, 2, 4, EPI_STATS, false, false>(M, N, A, B, 1, ep, s);
    // dW2 = G^T . E: both operands row-strided along K
    case EPI_STORE: return launch_cfg<T, 256, 256, 2, 4, EPI_STORE, true, true>(M, N, A, B, 1, ep, s);
    // dE = G . W2 (split over the vocabulary): A K-contiguous, B row-strided
    case EPI_PARTIAL: return launch_cfg<T, 256, 256, 2, 4, EPI_PARTIAL, false, true>(M, N, A, B, splits, ep, s);
  }
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_gemm(int dtype, int epi, int64_t M, int64_t N, const Operand& A,
                       const Operand& B, int splits, const EpiParams& ep, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  return dtype == 1 ? launch_t<bf16_t>(epi, M, N, A, B, splits, ep, s)
                    : launch_t<float>(epi, M, N, A, B, splits, ep, s);
}

}  // namespace dspark
