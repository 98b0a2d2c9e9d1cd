// MFMA GEMM C[M,N] = A[M,K] . B[N,K]^T for the DSpark loss (gfx950).
//
// Used for the dense contractions of the loss:
//   - the teacher lm_head projection T = H_t . LM^T (TorchSpec pull request
//     #132, PR description: teacher = target lm_head on the final hidden state),
//   - the Markov low-rank bias z' = z + E . W2^T with E = W1[prev] (NeMo-RL
//     "DSpark Auxiliary Heads", Inputs and Outputs),
//   - the backward products dE = G . W2 and dW2 = G^T . E.
//
// Four kernels share the tile order (XCD-aware groups: each of the 8 XCDs
// works a contiguous range of 256 x 256 tiles, so operand slices are shared
// through its own L2) and XOR-swizzled LDS rows of 16-byte chunks:
//   * gemm_w4_kernel (bf16, K-contiguous operands, K a multiple of 32): the
//     logits projections, persistent, 4 waves of 128 x 128 built from
//     v_mfma_f32_32x32x16_bf16; operands go global -> LDS with
//     buffer_load_dwordx4 ... lds through a 4-stage ring of BK = 32 slices;
//     the epilogue stages the tile through two free ring stages and computes
//     the per-row softmax statistics of every 64-column tile.
//   * gemm_w4p_kernel (bf16): the same main loop for the backward products
//     that read G, W2 and E in place (K-contiguous or M-contiguous operands,
//     the latter transposed by ds_read_b64_tr_b16), split-K partial output.
//   * gemm_dma_kernel (bf16, both operands K-contiguous or k-blocked, K a
//     multiple of 32): 8 waves of 128 x 64 built from
//     v_mfma_f32_16x16x32_bf16 over an LDS-DMA ring; the split-K backward
//     products where G is not read in place (rows or draft vocabulary not
//     multiples of 32).
//   * gemm_kernel (fp32 or bf16, any operand layout): register-staged,
//     double-buffered LDS, 8 waves of 128 x 64 (v_mfma_f32_16x16x32_bf16 or
//     v_mfma_f32_16x16x4_f32); operands K-contiguous, M-contiguous
//     (transposed on the way into LDS) or k-blocked ([K/c][M][c] with c
//     elements per 16-byte chunk).  Everything the others do not take.
// Operands may consist of two K segments (used for hi/lo splits of a bf16
// gradient).
#include "common.h"
#include "internal.h"

namespace dspark {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((address_space(3))) void lds_void;

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
// gfx9 data-format bits that make untyped dword loads valid.  Offsets at or
// past num_records read as zero.
constexpr int kNumRecords = 0x7fffffff;
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;
// Cache policy of buffer accesses that stream data used once (the logits
// tiles): non-temporal, so they do not evict the operand panels other tiles
// re-read from L2 and the memory-side cache.
constexpr int kStreamPolicy = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, kNumRecords, kRsrcWord3);
}

// ------------------------------------------------------------------ tile order

struct TileCoord {
  int64_t m0, n0, tn;
};

// XCD-contiguous ranges of a grouped-M order: hardware hands consecutive
// workgroups to the 8 XCDs in turn, so block b is remapped to give each XCD a
// contiguous slice of the order; within it, group_m row tiles share each
// column tile.
__device__ __forceinline__ TileCoord tile_coord_of(int64_t b, int64_t M, int64_t N, int BM, int BN,
                                                   int group_m) {
  const int64_t nM = (M + BM - 1) / BM, nN = (N + BN - 1) / BN;
  const int64_t tiles = nM * nN;
  const int64_t per_xcd = tiles / 8;
  if (b < per_xcd * 8) b = (b % 8) * per_xcd + b / 8;
  const int64_t gsz = static_cast<int64_t>(group_m) * nN;
  const int64_t fm = (b / gsz) * group_m;
  const int64_t gm = (nM - fm) < group_m ? (nM - fm) : group_m;
  const int64_t tm = fm + (b % gsz) % gm;
  const int64_t tn = (b % gsz) / gm;
  return {tm * BM, tn * BN, tn};
}
__device__ __forceinline__ TileCoord tile_coord(int64_t M, int64_t N, int BM, int BN,
                                                int group_m) {
  return tile_coord_of(blockIdx.x, M, N, BM, BN, group_m);
}

// Workgroup barrier ordering LDS accesses only.  __syncthreads() also fences
// global memory, which makes every wave drain its in-flight global loads and
// stores (vmcnt(0)) at each barrier; here only LDS hazards need ordering, so
// the wave waits for its own LDS operations (lgkmcnt(0)) and meets the others.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
}

// exp(x - m) in the fixed point of the tile exp-sums, widened for summing.
__device__ __forceinline__ uint32_t fix_exp(float x, float m) { return fix_exp32(x, m); }

// ------------------------------------------------------------------ accumulators

typedef __attribute__((ext_vector_type(16))) float f32x16_v;

// A wave's accumulator tile built from 16x16 MFMA blocks.  Lane (g, cl) holds,
// for block (i, j) and element e, row 16 i + 4 g + e, column 16 j + cl.
template <int TM, int TN>
struct Acc16 {
  f32x4_v v[TM][TN];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) v[i][j] = f32x4_v{0.f, 0.f, 0.f, 0.f};
  }
  // Rows [r0, r0 + ROWS) of the workgroup tile into stage (row stride STRIDE);
  // (wr, wc) is this wave's tile origin.
  template <int ROWS, int STRIDE>
  __device__ __forceinline__ void scatter(float* stage, int wr, int wc, int r0) const {
    const int lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rl = wr + i * 16 + g * 4 + e - r0;
        if (rl < 0 || rl >= ROWS) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) stage[rl * STRIDE + wc + j * 16 + cl] = v[i][j][e];
      }
  }
};

// A wave's accumulator tile built from 32x32 MFMA blocks.  Lane (h, c) = (l / 32,
// l % 32) holds, for block (i, j) and element e, row 32 i + 8 (e / 4) + 4 h + e % 4,
// column 32 j + c.
template <int TM, int TN>
struct Acc32 {
  f32x16_v v[TM][TN];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) v[i][j][e] = 0.f;
  }
  template <int ROWS, int STRIDE>
  __device__ __forceinline__ void scatter(float* stage, int wr, int wc, int r0) const {
    const int lane = threadIdx.x & 63, h = lane >> 5, c = lane & 31;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rl = wr + i * 32 + 8 * (e >> 2) + 4 * h + (e & 3) - r0;
        if (rl < 0 || rl >= ROWS) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) stage[rl * STRIDE + wc + j * 32 + c] = v[i][j][e];
      }
  }
};

// ------------------------------------------------------------------ epilogue

// The accumulator tile goes through LDS in chunks of 64 rows; 8 consecutive
// lanes then own one 256-column row, lane sub handling columns 4 sub + 32 i
// (i = 0..7), so a chunk's 64 rows are finished in parallel with 16-byte
// stores, 8-byte addend loads and 3-step shuffle reductions per row.  (wr, wc)
// is the calling wave's tile origin within the workgroup tile.
template <typename T, int BM, int BN, int NT, int EPI, typename AccT>
__device__ __forceinline__ void row_epilogue(const AccT& acc, int wr, int wc, float* stage,
                                             int64_t M, int64_t N, int64_t m0, int64_t n0,
                                             int64_t tn, const EpiParams& ep) {
  static_assert(BN == 256, "row epilogue assumes 256 columns");
  constexpr int kChunkRows = 64;
  constexpr int kLanesPerRow = NT / kChunkRows;      // 8
  constexpr int kVecs = BN / 4 / kLanesPerRow;       // float4 column groups per lane (8)
  static_assert(kLanesPerRow == 8, "8 lanes per row");
  constexpr int kStride = BN + 4;  // floats; 4 * kStride = 16 (mod 32) banks: conflict-free writes
  const int rr = threadIdx.x >> 3, sub = threadIdx.x & 7;
  float* C = ep.C;
  if (EPI == EPI_PARTIAL) C += static_cast<int64_t>(blockIdx.y) * M * ep.ldc;
  const T* X = static_cast<const T*>(ep.X);
  // Addends are loaded one chunk ahead and before the previous chunk's stores:
  // vmcnt retires in issue order, so a load issued after a store cannot be
  // waited for without also waiting for that store.
  typedef typename Elem<T>::Raw4 Raw4;
  Raw4 xr[kVecs];
  auto load_x = [&](int q) {
    const int64_t row = m0 + q * kChunkRows + rr;
#pragma unroll
    for (int i = 0; i < kVecs; ++i) {
      const int64_t col = n0 + sub * 4 + 32 * i;
      xr[i] = (X && row < M && col < N) ? Elem<T>::load4raw(X + row * ep.ldx + col) : Raw4{};
    }
  };
  if (EPI == EPI_STATS) load_x(0);
  lds_barrier();  // main-loop LDS reads are done (no LDS-DMA is in flight here)
#pragma unroll 1
  for (int q = 0; q < BM / kChunkRows; ++q) {
    const int64_t row = m0 + q * kChunkRows + rr;
    const bool rowok = row < M;
    acc.template scatter<kChunkRows, kStride>(stage, wr, wc, q * kChunkRows);
    lds_barrier();
    float4 v[kVecs];
#pragma unroll
    for (int i = 0; i < kVecs; ++i)
      v[i] = *reinterpret_cast<const float4*>(&stage[rr * kStride + sub * 4 + 32 * i]);
    if (EPI == EPI_STATS) {
#pragma unroll
      for (int i = 0; i < kVecs; ++i) {
        const float4 x = Elem<T>::widen4(xr[i]);
        v[i].x += x.x; v[i].y += x.y; v[i].z += x.z; v[i].w += x.w;
      }
      if (q + 1 < BM / kChunkRows) load_x(q + 1);
#pragma unroll
      for (int i = 0; i < kVecs; ++i) {
        const int64_t col = n0 + sub * 4 + 32 * i;
        if (col < N && rowok) *reinterpret_cast<float4*>(C + row * ep.ldc + col) = v[i];
      }
      // statistics per 64-column tile: lane sub holds columns 4 sub + 32 i,
      // so tile s (i = 2 s, 2 s + 1) spans the row's 8 lanes
#pragma unroll
      for (int st = 0; st < BN / kStatTile; ++st) {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 2 * st; i < 2 * st + 2; ++i) {
          const int64_t col = n0 + sub * 4 + 32 * i;
          if (col < N)  // N % 4 == 0: the 4 columns are all in or all out
            mx = fmaxf(mx, fmaxf(fmaxf(v[i].x, v[i].y), fmaxf(v[i].z, v[i].w)));
        }
#pragma unroll
        for (int o = 1; o < kLanesPerRow; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
        // fixed-point sum of exp(x - max): exact integer adds, so the result
        // does not depend on the order in which the columns are visited
        uint32_t sum = 0;
        if (mx != -INFINITY) {
#pragma unroll
          for (int i = 2 * st; i < 2 * st + 2; ++i) {
            const int64_t col = n0 + sub * 4 + 32 * i;
            if (col < N) {
              sum += fix_exp(v[i].x, mx) + fix_exp(v[i].y, mx) + fix_exp(v[i].z, mx) +
                     fix_exp(v[i].w, mx);
            }
          }
        }
#pragma unroll
        for (int o = 1; o < kLanesPerRow; o <<= 1) sum += __shfl_xor(sum, o, kWave);
        if (sub == 0 && rowok && n0 + kStatTile * st < N)
          ep.stats[row * ep.nstat + tn * (BN / kStatTile) + st] = make_float2(mx, fix_to_float(sum));
      }
    } else if (rowok) {
#pragma unroll
      for (int i = 0; i < kVecs; ++i) {
        const int64_t col = n0 + sub * 4 + 32 * i;
        if (col < N) *reinterpret_cast<float4*>(C + row * ep.ldc + col) = v[i];
      }
    }
    lds_barrier();
  }
}

// ------------------------------------------------------------------ generic kernel

// LDS row of a generic tile = 8 chunks of 16 bytes; chunk c of row m sits at slot c ^ swz8(m).
__device__ __forceinline__ int swz8(int m) { return (m ^ (m >> 3)) & 7; }

// Which (row, k) of a ROWS x 8-chunk tile lane-chunk idx covers, by layout.
// K-contiguous: chunk-fastest so a row is one 128-byte run; k-blocked:
// row-fastest so consecutive rows of a block are one run; M-contiguous: KPC
// consecutive rows at one k (8 such chunks side by side per k-row).
template <int LAYOUT, int ROWS, int BK, int KPC>
__device__ __forceinline__ void chunk_of(int idx, int* row, int* kin) {
  if (LAYOUT == LAYOUT_KC) { *row = idx >> 3; *kin = (idx & 7) * KPC; }
  else if (LAYOUT == LAYOUT_KB) { *row = idx % ROWS; *kin = (idx / ROWS) * KPC; }
  else { *row = ((idx & 7) + ((idx >> 3) / BK) * 8) * KPC; *kin = (idx >> 3) % BK; }
}

template <typename T, int ROWS, int NT, int LAYOUT>
struct TileLoader {
  static constexpr int KPC = Elem<T>::kPerChunk;
  static constexpr int PER = ROWS * 8 / NT;
  static constexpr int BK = 8 * KPC;
  uint32_t off[PER];  // element offset of lane chunk p from the tile base
  uint32_t rowok;     // bit p: the row of chunk p is inside the operand
  int kofs[PER];      // k of chunk p within the K-tile

  __device__ __forceinline__ void init(const Operand& op, int64_t r0, int64_t rlim) {
    rowok = 0;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      int row, k;
      chunk_of<LAYOUT, ROWS, BK, KPC>(threadIdx.x + p * NT, &row, &k);
      if (LAYOUT == LAYOUT_KC) off[p] = static_cast<uint32_t>(row * op.ld + k);
      else if (LAYOUT == LAYOUT_KB) off[p] = static_cast<uint32_t>(k * op.ld + row * KPC);
      else off[p] = static_cast<uint32_t>(k * op.ld + row);
      kofs[p] = k;
      if (r0 + row < rlim) rowok |= 1u << p;
    }
  }

  // Load K-tile kt (padded-K positions [kt*BK, kt*BK+BK)) with buffer loads
  // based at the tile origin; chunks outside the operand read as zero.
  __device__ __forceinline__ void load(const Operand& op, int64_t r0, int kt, int64_t kend,
                                       u32x4* reg) const {
    const int64_t kg = static_cast<int64_t>(kt) * BK;
    const int s = static_cast<int>(kg / op.kpad);
    const int64_t kk0 = kg - s * op.kpad;
    const int64_t kvalid = op.kseg - kk0;
    const int64_t rofs = LAYOUT == LAYOUT_KC ? r0 * op.ld : (LAYOUT == LAYOUT_KB ? r0 * KPC : r0);
    const int64_t kofs0 = LAYOUT == LAYOUT_KC ? kk0 : kk0 * op.ld;
    const T* base = static_cast<const T*>(op.seg[s]) + rofs + kofs0;
    const int64_t klim = kend - kg;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(base);
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const bool ok = ((rowok >> p) & 1u) && kofs[p] < kvalid && kofs[p] < klim;
      const uint32_t o = ok ? off[p] * static_cast<uint32_t>(sizeof(T)) : kOutOfRange;
      reg[p] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, o, 0, 0);
    }
  }
};

// Registers -> LDS (K-contiguous, swizzled) for the tile loaded by TileLoader.
template <typename T, int ROWS, int NT, int LAYOUT>
__device__ __forceinline__ void store_tile(u32x4* lds, const u32x4* reg) {
  constexpr int KPC = Elem<T>::kPerChunk;
  constexpr int PER = ROWS * 8 / NT;
  constexpr int BK = 8 * KPC;
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    int row, k;
    chunk_of<LAYOUT, ROWS, BK, KPC>(threadIdx.x + p * NT, &row, &k);
    if (LAYOUT != LAYOUT_MC) {
      const int c = k / KPC;
      lds[row * 8 + (c ^ swz8(row))] = reg[p];
    } else {
      const int kc = k / KPC, ke = k % KPC;
      T vals[KPC];
      __builtin_memcpy(vals, &reg[p], 16);
#pragma unroll
      for (int j = 0; j < KPC; ++j) {
        const int m = row + j;
        reinterpret_cast<T*>(&lds[m * 8 + (kc ^ swz8(m))])[ke] = vals[j];
      }
    }
  }
}

// TAG only names the kernel symbol per role (draft logits / teacher / backward),
// so profilers report each role separately.
template <typename T, int BM, int BN, int WM, int WN, int EPI, int AL, int BL, int TAG>
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
  static_assert(EPI != EPI_STATS || BN == kGemmTileN, "stats epilogue needs BN == 256");

  __shared__ u32x4 lds[2 * (A_CH + B_CH)];
  const TileCoord tc = tile_coord(M, N, BM, BN, group_m);
  const int64_t m0 = tc.m0, n0 = tc.n0;
  const int64_t kbeg = static_cast<int64_t>(blockIdx.y) * kper;
  const int64_t kend = (kbeg + kper) < K ? (kbeg + kper) : K;
  const int nk = kend > kbeg ? static_cast<int>((kend - kbeg + BK - 1) / BK) : 0;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int g = lane >> 4, cl = lane & 15;

  Acc16<TM, TN> acc;
  acc.zero();

  if (nk > 0) {
    TileLoader<T, BM, NT, AL> la;
    TileLoader<T, BN, NT, BL> lb;
    la.init(A, m0, M);
    lb.init(B, n0, N);
    const int kt0 = static_cast<int>(kbeg / BK);
    u32x4 ra[A_PER], rb[B_PER];
    la.load(A, m0, kt0, kend, ra);
    lb.load(B, n0, kt0, kend, rb);
    store_tile<T, BM, NT, AL>(lds, ra);
    store_tile<T, BN, NT, BL>(lds + A_CH, rb);
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
          af[i] = As[m * 8 + (c ^ swz8(m))];
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = wn * WTN + j * 16 + cl;
          bfr[j] = Bs[n * 8 + (c ^ swz8(n))];
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) Mfma<T>::run(acc.v[i][j], af[i], bfr[j]);
      }
      if (more) {
        u32x4* An = lds + ((kt + 1) & 1) * (A_CH + B_CH);
        store_tile<T, BM, NT, AL>(An, ra);
        store_tile<T, BN, NT, BL>(An + A_CH, rb);
      }
      __syncthreads();
    }
  }
  row_epilogue<T, BM, BN, NT, EPI>(acc, wm * WTM, wn * WTN, reinterpret_cast<float*>(lds), M, N,
                                   m0, n0, tc.tn, ep);
}

// ------------------------------------------------------------------ LDS-DMA kernel

// bf16; each operand K-contiguous (LAYOUT_KC) or k-blocked by 8 (LAYOUT_KB);
// every K segment a multiple of 32.  LDS slice row = 32 bf16 = 4 chunks; chunk
// c of row m sits at slot c ^ swz4(m).
__device__ __forceinline__ int swz4(int m) { return (m >> 1) & 3; }

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt <= n only.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// Workgroup barrier of the DMA loop: lds_barrier(), after each wave waited for
// its own DMA slices explicitly (a fence would drain every in-flight slice).
__device__ __forceinline__ void dma_barrier() { lds_barrier(); }

// DMA slice t of a split into stage t % STAGES: the wave's p-th A load fills
// LDS chunks [(wave*A_LD + p) * 64, +64) of the stage (B after A_CH chunks).
// Element offset of chunk (row, c) of a 32-wide K slice, and of the slice base.
template <int LAYOUT>
__device__ __forceinline__ int64_t dma_chunk(int row, int c, int64_t ld) {
  return LAYOUT == LAYOUT_KB ? static_cast<int64_t>(c) * 8 * ld + row * 8 : row * ld + c * 8;
}
template <int LAYOUT>
__device__ __forceinline__ int64_t dma_base(int64_t r0, int64_t kk, int64_t ld) {
  return LAYOUT == LAYOUT_KB ? r0 * 8 + kk * ld : r0 * ld + kk;
}

template <int AL, int BL, int A_LD, int B_LD, int A_CH, int STAGE_CH, int STAGES>
__device__ __forceinline__ void dma_issue(const Operand& A, const Operand& B, int64_t kbeg, int t,
                                          int64_t m0, int64_t n0, int wave, const uint32_t* offA,
                                          const uint32_t* offB, u32x4* lds) {
  const int64_t kg = kbeg + static_cast<int64_t>(t) * 32;
  const bool s1 = kg >= A.kseg;  // at most two K segments
  const int64_t kk = s1 ? kg - A.kseg : kg;
  const bf16_t* abase = static_cast<const bf16_t*>(s1 ? A.seg[1] : A.seg[0]);
  const bf16_t* bbase = static_cast<const bf16_t*>(s1 ? B.seg[1] : B.seg[0]);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(abase + dma_base<AL>(m0, kk, A.ld));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(bbase + dma_base<BL>(n0, kk, B.ld));
  u32x4* st = lds + (t % STAGES) * STAGE_CH;
#pragma unroll
  for (int p = 0; p < A_LD; ++p)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(st + (wave * A_LD + p) * 64), 16,
                                             offA[p], 0, 0, 0);
#pragma unroll
  for (int p = 0; p < B_LD; ++p)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(st + A_CH + (wave * B_LD + p) * 64),
                                             16, offB[p], 0, 0, 0);
}

// One output tile's K loop on the DMA path: slices [kbeg, kbeg + 32 nk) of
// A (rows m0..) and B (rows n0..) accumulate into acc.
template <int BM, int BN, int WM, int WN, int AL, int BL>
__device__ __forceinline__ void dma_mainloop(Acc16<BM / WM / 16, BN / WN / 16>& acc,
                                             const Operand& A, const Operand& B, int64_t kbeg,
                                             int nk, int64_t M, int64_t N, int64_t m0, int64_t n0,
                                             u32x4* lds) {
  constexpr int NT = WM * WN * 64;
  constexpr int NW = NT / 64;
  constexpr int STAGES = 4;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 16, TN = WTN / 16;                 // 16x16 MFMA blocks per wave
  constexpr int A_CH = BM * 4, B_CH = BN * 4;                 // 16-byte chunks per slice
  constexpr int A_LD = A_CH / 64 / NW, B_LD = B_CH / 64 / NW;  // DMA loads per wave per slice
  constexpr int STAGE_CH = A_CH + B_CH;
  static_assert(A_CH % (64 * NW) == 0 && B_CH % (64 * NW) == 0, "tile / wave mismatch");
  static_assert(STAGES * STAGE_CH * 16 <= 160 * 1024, "LDS budget");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // Lane chunk of each DMA load: the wave's p-th load fills LDS chunks
  // [(wave*X_LD + p) * 64, +64) of the slice, lane l the one at +l, i.e. row
  // idx / 4, slot idx % 4, which holds global chunk slot ^ swz4(row).
  uint32_t offA[A_LD], offB[B_LD];
#pragma unroll
  for (int p = 0; p < A_LD; ++p) {
    const int idx = (wave * A_LD + p) * 64 + lane;
    const int row = idx >> 2, c = (idx & 3) ^ swz4(idx >> 2);
    offA[p] = (m0 + row < M) ? static_cast<uint32_t>(dma_chunk<AL>(row, c, A.ld) * 2) : kOutOfRange;
  }
#pragma unroll
  for (int p = 0; p < B_LD; ++p) {
    const int idx = (wave * B_LD + p) * 64 + lane;
    const int row = idx >> 2, c = (idx & 3) ^ swz4(idx >> 2);
    offB[p] = (n0 + row < N) ? static_cast<uint32_t>(dma_chunk<BL>(row, c, B.ld) * 2) : kOutOfRange;
  }

  constexpr int LPS = A_LD + B_LD;  // loads per wave per slice
#pragma unroll
  for (int t = 0; t < STAGES - 1; ++t)
    if (t < nk)
      dma_issue<AL, BL, A_LD, B_LD, A_CH, STAGE_CH, STAGES>(A, B, kbeg, t, m0, n0, wave, offA, offB,
                                                            lds);
  const int g = lane >> 4, cl = lane & 15;
  for (int kt = 0; kt < nk; ++kt) {
    // slice kt has landed once at most (slices issued after it) * LPS loads remain
    const int after = (nk - 1 - kt) < (STAGES - 2) ? (nk - 1 - kt) : (STAGES - 2);
    if (after >= 2) wait_vmcnt<2 * LPS>();
    else if (after == 1) wait_vmcnt<LPS>();
    else wait_vmcnt<0>();
    dma_barrier();  // every wave's slice-kt loads are in LDS; slice kt-1 is consumed
    if (kt + STAGES - 1 < nk)
      dma_issue<AL, BL, A_LD, B_LD, A_CH, STAGE_CH, STAGES>(A, B, kbeg, kt + STAGES - 1, m0, n0,
                                                            wave, offA, offB, lds);
    const u32x4* As = lds + (kt % STAGES) * STAGE_CH;
    const u32x4* Bs = As + A_CH;
    // v_mfma_f32_16x16x32_bf16: lane (g, cl) supplies row cl of a 16-row block at
    // k = 8 g .. 8 g + 7, i.e. chunk g of the 32-wide slice.
    u32x4 af[TM], bfr[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = wm * WTM + i * 16 + cl;
      af[i] = As[m * 4 + (g ^ swz4(m))];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = wn * WTN + j * 16 + cl;
      bfr[j] = Bs[n * 4 + (g ^ swz4(n))];
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) Mfma<bf16_t>::run(acc.v[i][j], af[i], bfr[j]);
  }
}

// One job of the DMA kernel on this workgroup's output tile.
template <int BM, int BN, int WM, int WN, int EPI, int AL, int BL>
__device__ __forceinline__ void dma_job(const GemmJob& J, int64_t M, int64_t N, int64_t kper,
                                        const TileCoord& tc, u32x4* lds) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t kbeg = static_cast<int64_t>(blockIdx.y) * kper;
  const int64_t kend = (kbeg + kper) < J.K ? (kbeg + kper) : J.K;
  const int nk = kend > kbeg ? static_cast<int>((kend - kbeg) / 32) : 0;
  Acc16<BM / WM / 16, BN / WN / 16> acc;
  acc.zero();
  dma_mainloop<BM, BN, WM, WN, AL, BL>(acc, J.A, J.B, kbeg, nk, M, N, tc.m0, tc.n0, lds);
  row_epilogue<bf16_t, BM, BN, NT, EPI>(acc, wm * WTM, wn * WTN, reinterpret_cast<float*>(lds), M,
                                        N, tc.m0, tc.n0, tc.tn, J.ep);
}

// Up to two GEMM jobs over the same output tile grid, run back to back per
// tile (launched here with one: the split-K backward partials).  A job with
// K = 0 is its epilogue alone (C = X).
template <int BM, int BN, int WM, int WN, int EPI, int AL, int BL, int TAG>
__global__ __launch_bounds__(WM* WN * 64, 1) void gemm_dma_kernel(int64_t M, int64_t N,
                                                                  int64_t kper, GemmJob j0,
                                                                  GemmJob j1, int njobs,
                                                                  int group_m) {
  static_assert(EPI != EPI_STATS || BN == kGemmTileN, "stats epilogue needs BN == 256");
  __shared__ u32x4 lds[4 * (BM * 4 + BN * 4)];
  const TileCoord tc = tile_coord(M, N, BM, BN, group_m);
  dma_job<BM, BN, WM, WN, EPI, AL, BL>(j0, M, N, kper, tc, lds);
  if (njobs > 1) dma_job<BM, BN, WM, WN, EPI, AL, BL>(j1, M, N, kper, tc, lds);
}

// ------------------------------------------------------------------ 4-wave logits kernel

// The logits projections (teacher T = H_t . LM^T, K = hidden; draft bias
// E . W2^T, K = markov rank, plus the logits addend) on 256 x 256 tiles with
// 4 waves of 128 x 128 built from v_mfma_f32_32x32x16_bf16: twice the MACs
// per LDS byte read of the 8-wave loop.  The MFMA takes the vocab (B)
// fragment as its first operand, so for block (j, i) lane (h, r) = (l / 32,
// l % 32) holds row 32 i + r of the wave tile at columns 32 j + 8 q + 4 h ..
// + 3 in elements 4 q .. 4 q + 3 (16-byte pieces of 4 columns; the logits
// epilogue regroups them by row through LDS, the backward partials store
// them as they are).  Operands stream
// through an LDS-DMA ring (4 stages of 32-wide K slices); each wave reads the
// next slice's fragments into a second register set while its MFMAs run,
// since with one wave per SIMD no other wave hides LDS latency.
namespace w4 {
constexpr int kNW = 4, kNT = 256, kStages = 4;
constexpr int kACh = 256 * 4, kBCh = 256 * 4, kStageCh = kACh + kBCh;  // 16-byte chunks per slice
constexpr int kALd = kACh / 64 / kNW, kBLd = kBCh / 64 / kNW;         // DMA loads per wave per slice
constexpr int kLps = kALd + kBLd;
}  // namespace w4

typedef __attribute__((ext_vector_type(4))) short s16x4_v;
typedef __attribute__((address_space(3))) s16x4_v lds_s16x4;

// Slot of 16-byte chunk c (0..3) of slice row m: rows 4 apart use different
// slots, so the 16 rows one ds_read_b128 phase touches hit distinct banks.
__device__ __forceinline__ int w4_slot(int m, int c) { return m * 4 + (c ^ ((m >> 2) & 3)); }

// One operand's 32-wide K slice of 256 rows in LDS (1024 chunks of 16 bytes),
// by global layout.
//   KC ([rows][K]): slice row m holds its 32 k in 4 chunks at w4_slot(m, c);
//      a lane's 8 consecutive k of one row are one ds_read_b128.
//   MK ([K][rows]): slice row k holds 256 rows in 32 chunks of 8; chunk c of
//      row k sits at k * 32 + (c ^ 4 (k & 3)).  A lane's 8 consecutive k of
//      one row come from two ds_read_b64_tr_b16: in each 16-lane group, lane
//      i loads 4 rows' worth at (k0 + i / 4, m0 + 4 (i % 4)) and lane j gets
//      the values of row m0 + j at k0 .. k0 + 3.  The XOR spreads the 4 k rows
//      (and the neighbouring group's 16 rows) of one such load over distinct
//      banks.
template <int L> struct W4Op;
template <> struct W4Op<LAYOUT_KC> {
  // (row, chunk) filled by LDS position idx of a slice
  __device__ static void chunk(int idx, int* row, int* c) {
    *row = idx >> 2;
    *c = (idx & 3) ^ ((*row >> 2) & 3);
  }
  __device__ static int64_t offset(int row, int c, int64_t ld) { return row * ld + 8 * c; }
  __device__ static int64_t base(int64_t r0, int64_t kk, int64_t ld) { return r0 * ld + kk; }
  __device__ static bool in_range(int64_t r0, int row, int c, int64_t rows) { return r0 + row < rows; }
  // fragment of rows rb .. rb + 31 (lane r = l % 32) at k = 16 ks + 8 (l / 32) .. + 7
  __device__ static u32x4 frag(const u32x4* s, int rb, int ks) {
    const int lane = threadIdx.x & 63;
    return s[w4_slot(rb + (lane & 31), 2 * ks + (lane >> 5))];
  }
};
template <> struct W4Op<LAYOUT_MK> {
  __device__ static int slot(int k, int c) { return k * 32 + (c ^ (4 * (k & 3))); }
  __device__ static void chunk(int idx, int* k, int* c) {
    *k = idx >> 5;
    *c = (idx & 31) ^ (4 * (*k & 3));
  }
  __device__ static int64_t offset(int k, int c, int64_t ld) { return k * ld + 8 * c; }
  __device__ static int64_t base(int64_t r0, int64_t kk, int64_t ld) { return kk * ld + r0; }
  __device__ static bool in_range(int64_t r0, int, int c, int64_t rows) { return r0 + 8 * c < rows; }
  __device__ static u32x4 frag(const u32x4* s, int rb, int ks) {
    const int lane = threadIdx.x & 63, gi = lane >> 4, i = lane & 15;
    const int m = rb + 16 * (gi & 1) + 4 * (i & 3);       // first of the lane's 4 loaded rows
    const int k = 16 * ks + 8 * (gi >> 1) + (i >> 2);
    const int half = (m & 7) >> 2;                           // 8-byte half of the chunk
    const char* base = reinterpret_cast<const char*>(s);
    const s16x4_v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(base + slot(k, m >> 3) * 16 + half * 8));
    const s16x4_v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(base + slot(k + 4, m >> 3) * 16 + half * 8));
    const uint2 a = __builtin_bit_cast(uint2, lo), b = __builtin_bit_cast(uint2, hi);
    return u32x4{a.x, a.y, b.x, b.y};
  }
};

// Fragments of one 32-wide K slice: [k step][block] for A (rows) and B (vocab).
struct W4Frags {
  u32x4 a[2][4], b[2][4];
};

template <int AL, int BL>
__device__ __forceinline__ void w4_read(W4Frags& f, const u32x4* st, int wm, int wn) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.a[ks][i] = W4Op<AL>::frag(st, wm * 128 + i * 32, ks);
      f.b[ks][i] = W4Op<BL>::frag(st + w4::kACh, wn * 128 + i * 32, ks);
    }
}

__device__ __forceinline__ void w4_mma(f32x16_v (&acc)[4][4], const W4Frags& f) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_v, f.b[ks][j]), __builtin_bit_cast(bf16x8_v, f.a[ks][i]),
            acc[j][i], 0, 0, 0);
}

// Lane chunk offsets (bytes from the slice base) of the wave's DMA loads.
struct W4Offsets {
  uint32_t a[w4::kALd], b[w4::kBLd];
};

template <int AL, int BL>
__device__ __forceinline__ void w4_offsets(W4Offsets& o, const Operand& A, const Operand& B,
                                           int64_t M, int64_t N, int64_t m0, int64_t n0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int p = 0; p < w4::kALd; ++p) {
    int row, c;
    W4Op<AL>::chunk((wave * w4::kALd + p) * 64 + lane, &row, &c);
    o.a[p] = W4Op<AL>::in_range(m0, row, c, M)
                 ? static_cast<uint32_t>(W4Op<AL>::offset(row, c, A.ld) * 2)
                 : kOutOfRange;
  }
#pragma unroll
  for (int p = 0; p < w4::kBLd; ++p) {
    int row, c;
    W4Op<BL>::chunk((wave * w4::kBLd + p) * 64 + lane, &row, &c);
    o.b[p] = W4Op<BL>::in_range(n0, row, c, N)
                 ? static_cast<uint32_t>(W4Op<BL>::offset(row, c, B.ld) * 2)
                 : kOutOfRange;
  }
}

// The ring's four stages are separate LDS arrays: with stage indices known
// at compile time, the compiler's own LDS-DMA hazard waits before a fragment
// read cover only the DMA into that stage (the one the loop waits for
// anyway), not every slice in flight.
struct W4Ring {
  u32x4* st[w4::kStages];
};

// Queue virtual slice t into stage S for a job whose K range starts at kbeg
// and holds nk real slices after `shift` leading zero slices.  A zero slice
// loads through a zero-length buffer: its stage fills with zeros and no
// memory is touched.
template <int S, int AL, int BL>
__device__ __forceinline__ void w4_issue(const Operand& A, const Operand& B, int64_t kbeg, int t,
                                         int nk, int shift, int64_t m0, int64_t n0,
                                         const W4Offsets& o, const W4Ring& ring) {
  const int r = t - shift;
  const bool real = r >= 0 && r < nk;
  const int64_t kg = kbeg + (real ? static_cast<int64_t>(r) * 32 : 0);
  const bool s1 = kg >= A.kseg;  // at most two K segments
  const int64_t kk = s1 ? kg - A.kseg : kg;
  const bf16_t* abase = static_cast<const bf16_t*>(s1 ? A.seg[1] : A.seg[0]);
  const bf16_t* bbase = static_cast<const bf16_t*>(s1 ? B.seg[1] : B.seg[0]);
  const int nrec = real ? kNumRecords : 0;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(abase + W4Op<AL>::base(m0, kk, A.ld)), 0, nrec, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(bbase + W4Op<BL>::base(n0, kk, B.ld)), 0, nrec, kRsrcWord3);
  u32x4* st = ring.st[S];
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int p = 0; p < w4::kALd; ++p)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(st + (wave * w4::kALd + p) * 64), 16,
                                             o.a[p], 0, 0, 0);
#pragma unroll
  for (int p = 0; p < w4::kBLd; ++p)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rb, (lds_void*)(st + w4::kACh + (wave * w4::kBLd + p) * 64), 16, o.b[p], 0, 0, 0);
}

// One step of the K loop for slice kt in stage S, whose fragments are in
// `cur`: wait until slice kt + 1 has landed (LATER slices were queued after
// it), queue slice kt + 3 (ISSUE), read slice kt + 1 into `nxt` (READ), run
// slice kt's MFMAs.  Scheduling fences keep each step's MFMAs between its
// own fragment reads and the next step's barrier.
template <int S, int LATER, bool ISSUE, bool READ, int AL, int BL>
__device__ __forceinline__ void w4_step(f32x16_v (&acc)[4][4], const W4Frags& cur, W4Frags& nxt,
                                        const Operand& A, const Operand& B, int64_t kbeg, int kt,
                                        int nk, int shift, int64_t m0, int64_t n0,
                                        const W4Offsets& o, const W4Ring& ring, int wm, int wn) {
  // LDS read instructions per slice: one per KC fragment, two per MK fragment
  constexpr int kReads = 8 * (AL == LAYOUT_MK ? 2 : 1) + 8 * (BL == LAYOUT_MK ? 2 : 1);
  __builtin_amdgcn_sched_barrier(0);
  if (READ) {
    if (LATER == 1) wait_vmcnt<w4::kLps>();
    else wait_vmcnt<0>();
    dma_barrier();
  }
  if (ISSUE)
    w4_issue<(S + 3) % w4::kStages, AL, BL>(A, B, kbeg, kt + 3, nk, shift, m0, n0, o, ring);
  if (READ) w4_read<AL, BL>(nxt, ring.st[(S + 1) % w4::kStages], wm, wn);
  w4_mma(acc, cur);
  // Interleave the fragment reads and DMA issues with the MFMAs so the matrix
  // pipe is not left idle while the wave issues its memory operations.
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                   // MFMA
    if (READ) __builtin_amdgcn_sched_group_barrier(0x100, kReads / 16, 0);  // DS read
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                   // MFMA
    if (READ) __builtin_amdgcn_sched_group_barrier(0x100, kReads / 16, 0);  // DS read
    if (ISSUE) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);         // VMEM read (LDS DMA)
  }
}

// First kStages - 1 virtual slices of a job's K loop (nothing when nk == 0,
// so no DMA is left in flight).
template <int AL, int BL>
__device__ __forceinline__ void w4_prologue(const Operand& A, const Operand& B, int64_t kbeg,
                                            int nk, int64_t m0, int64_t n0, const W4Offsets& o,
                                            const W4Ring& ring) {
  if (nk <= 0) return;
  const int shift = (4 - (nk & 3)) & 3;
  w4_issue<0, AL, BL>(A, B, kbeg, 0, nk, shift, m0, n0, o, ring);
  w4_issue<1, AL, BL>(A, B, kbeg, 1, nk, shift, m0, n0, o, ring);
  w4_issue<2, AL, BL>(A, B, kbeg, 2, nk, shift, m0, n0, o, ring);
}

// K loop of one job whose first slices w4_prologue already queued.  Runs
// over nv = nk rounded up to a multiple of 4 virtual slices (zero slices
// first), unrolled by the 4 ring stages; fragments alternate between two
// register sets so slice kt + 1 is read while slice kt's MFMAs run.  Every
// DMA has landed when it returns.
template <int AL, int BL>
__device__ __forceinline__ void w4_mainloop(f32x16_v (&acc)[4][4], const Operand& A,
                                            const Operand& B, int64_t kbeg, int nk, int64_t m0,
                                            int64_t n0, const W4Offsets& o, const W4Ring& ring) {
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][i][e] = 0.f;
  if (nk <= 0) return;
  const int shift = (4 - (nk & 3)) & 3, nv = nk + shift;
  wait_vmcnt<2 * w4::kLps>();  // slice 0 has landed (slices 1 and 2 follow it)
  dma_barrier();
  W4Frags f0, f1;
  w4_read<AL, BL>(f0, ring.st[0], wm, wn);
  int kt = 0;
  for (; kt + 4 < nv; kt += 4) {
    w4_step<0, 1, true, true, AL, BL>(acc, f0, f1, A, B, kbeg, kt, nk, shift, m0, n0, o, ring, wm, wn);
    w4_step<1, 1, true, true, AL, BL>(acc, f1, f0, A, B, kbeg, kt + 1, nk, shift, m0, n0, o, ring, wm, wn);
    w4_step<2, 1, true, true, AL, BL>(acc, f0, f1, A, B, kbeg, kt + 2, nk, shift, m0, n0, o, ring, wm, wn);
    w4_step<3, 1, true, true, AL, BL>(acc, f1, f0, A, B, kbeg, kt + 3, nk, shift, m0, n0, o, ring, wm, wn);
  }
  // last four slices: only slice nv - 1 remains to be queued
  w4_step<0, 1, true, true, AL, BL>(acc, f0, f1, A, B, kbeg, kt, nk, shift, m0, n0, o, ring, wm, wn);
  w4_step<1, 1, false, true, AL, BL>(acc, f1, f0, A, B, kbeg, kt + 1, nk, shift, m0, n0, o, ring, wm, wn);
  w4_step<2, 0, false, true, AL, BL>(acc, f0, f1, A, B, kbeg, kt + 2, nk, shift, m0, n0, o, ring, wm, wn);
  w4_step<3, 0, false, false, AL, BL>(acc, f1, f0, A, B, kbeg, kt + 3, nk, shift, m0, n0, o, ring, wm, wn);
  __builtin_amdgcn_sched_barrier(0);
}

// Partial-sum epilogue: the 256 x 256 fp32 tile straight from the
// accumulators (lane (h, r) of block (j, i): row 32 i + r, columns
// 32 j + 8 q + 4 h .. + 3) into C (rows < M, columns < N; N % 4 == 0).
__device__ __forceinline__ void w4_store(const f32x16_v (&acc)[4][4], int64_t M, int64_t N,
                                         int64_t m0, int64_t n0, float* C, int64_t ldc) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, r = lane & 31;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = m0 + wm * 128 + 32 * i + r;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = n0 + wn * 128 + 32 * j + 8 * q + 4 * h;
        if (col < N)
          *reinterpret_cast<float4*>(C + row * ldc + col) =
              make_float4(acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2],
                          acc[j][i][4 * q + 3]);
      }
  }
}

// C[blockIdx.y] = A . B^T over K range [blockIdx.y kper, + kper) on 256 x 256
// tiles (backward products; operands KC or MK).
template <int AL, int BL, int TAG>
__global__ __launch_bounds__(256, 1) void gemm_w4p_kernel(int64_t M, int64_t N, int64_t K,
                                                          int64_t kper, Operand A, Operand B,
                                                          float* C, int64_t ldc, int group_m) {
  __shared__ u32x4 st0[w4::kStageCh], st1[w4::kStageCh], st2[w4::kStageCh], st3[w4::kStageCh];
  const W4Ring ring{{st0, st1, st2, st3}};
  const TileCoord tc = tile_coord(M, N, 256, 256, group_m);
  const int64_t kbeg = static_cast<int64_t>(blockIdx.y) * kper;
  const int64_t kend = (kbeg + kper) < K ? (kbeg + kper) : K;
  const int nk = kend > kbeg ? static_cast<int>((kend - kbeg) / 32) : 0;
  W4Offsets o;
  w4_offsets<AL, BL>(o, A, B, M, N, tc.m0, tc.n0);
  w4_prologue<AL, BL>(A, B, kbeg, nk, tc.m0, tc.n0, o, ring);
  f32x16_v acc[4][4];
  w4_mainloop<AL, BL>(acc, A, B, kbeg, nk, tc.m0, tc.n0, o, ring);
  w4_store(acc, M, N, tc.m0, tc.n0, C + static_cast<int64_t>(blockIdx.y) * M * ldc, ldc);
}

// Stores the tile (plus the bf16 addend X when given) and, per row, the
// maximum and exp-sum of its 256 columns.  The accumulators go through two
// free ring stages (32 rows x 256 fp32 each, 16-byte slots XOR-swizzled by
// row so both the accumulator writes and the row reads are conflict-free),
// one 32-row block of each wave-row half at a time; then 16 lanes own a row:
// 256-byte coalesced stores and addend loads, and the row's maximum and
// fixed-point exp-sum reduce over 4 DPP steps.
__device__ __forceinline__ int w4_eslot(int row, int c4) { return row * 64 + (c4 ^ (row & 15)); }

// Maximum / sum over each row of 16 lanes with DPP row rotations (VALU
// only, no LDS round trips); every lane of the row receives the result, in
// an order that depends only on the lane.
template <int ROR>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + ROR, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, row_ror<8>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<2>(v));
  return fmaxf(v, row_ror<1>(v));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xf, 0xf, false));
}
// Sums of the four per-lane values p[0..3] over each row of 16 lanes,
// transposed: lane sub returns the row's total of p[sub >> 2].  Exchange with
// lane sub ^ 8 (row_ror:8), keeping values 2 b3, 2 b3 + 1 (b3 = bit 3 of sub);
// then with the mirror lane of the half row (row_half_mirror), keeping value
// 2 b3 + b2; then within the quad (quad_perm xor 1, xor 2).  The four partial
// sets of a quad's lanes tile the 16 lanes.  11 VALU operations where four
// separate 16-lane reductions take 16.
__device__ __forceinline__ uint32_t quad_tile_sums(const uint32_t (&p)[4], int sub) {
  const bool b3 = (sub & 8) != 0, b2 = (sub & 4) != 0;
  const uint32_t k0 = b3 ? p[2] : p[0], k1 = b3 ? p[3] : p[1];
  const uint32_t s0 = b3 ? p[0] : p[2], s1 = b3 ? p[1] : p[3];
  const uint32_t a0 = k0 + dpp_u32<0x128>(s0), a1 = k1 + dpp_u32<0x128>(s1);
  uint32_t c = (b2 ? a1 : a0) + dpp_u32<0x141>(b2 ? a0 : a1);
  c += dpp_u32<0xB1>(c);  // quad_perm [1, 0, 3, 2]
  return c + dpp_u32<0x4E>(c);  // quad_perm [2, 3, 0, 1]
}


// Rows of the row phase: wave w handles rows wrow(w, i) + 4 p + (lane >> 4),
// p = 0..3, of 32-row block i; every global access goes through a buffer
// resource based at the first of those rows, so offsets stay below 2^30 for
// any leading dimension below 2^26, and out-of-range lanes get an offset past
// the resource (loads read zero, stores are dropped) instead of a branch:
// with no branches the compiler's wait counts are exact and the addends of
// the next block stay in flight while this block is processed.
__device__ __forceinline__ int64_t w4_erow(int64_t m0, int i, int p) {
  // wave-uniform (scalar) so the buffer resources built from it are scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  return m0 + (wave >> 1) * 128 + 32 * i + 16 * (wave & 1) + 4 * p;
}

// Queue the bf16 addends of block i: lane (row, sub) reads columns
// 4 sub + 64 t .. + 3 of its row, t = 0..3.
__device__ __forceinline__ void w4_x_issue(uint2 (&xv)[4][4], const EpiParams& ep, int64_t M,
                                           int64_t N, int64_t m0, int64_t n0, int i) {
  const int lane = threadIdx.x & 63, sub = lane & 15, rl = lane >> 4;
  const bf16_t* X = static_cast<const bf16_t*>(ep.X);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int64_t r0 = w4_erow(m0, i, p);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X + r0 * ep.ldx + n0);
    const bool rok = r0 + rl < M;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = 4 * sub + 64 * t;
      const uint32_t off = (rok && n0 + c < N)
                               ? static_cast<uint32_t>((rl * ep.ldx + c) * 2)
                               : kOutOfRange;
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rx, off, 0, kStreamPolicy);
      xv[p][t] = make_uint2(v.x, v.y);
    }
  }
}

// Block i of the epilogue: stage the accumulators of the block's rows, then
// 16 lanes per row add the addends, store the row's 256 columns and reduce
// the row's maximum and fixed-point exp-sum.
template <bool HAS_X>
__device__ __forceinline__ void w4_eblock(const f32x16_v (&acc)[4][4], int i,
                                          const uint2 (&xv)[4][4], int64_t M, int64_t N,
                                          int64_t m0, int64_t n0, int64_t tn, const EpiParams& ep,
                                          float4* ea, float4* eb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5, r = lane & 31;
  const int sub = lane & 15, rl = lane >> 4;
  const int rbase = 16 * (wave & 1) + rl;  // + 4 p: row within the 32-row block
  float4* mine = wm == 0 ? ea : eb;
  const float4* src = (wave >> 1) == 0 ? ea : eb;
  lds_barrier();  // the stages are free (main-loop reads or the previous block's reads done)
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      mine[w4_eslot(r, wn * 32 + 8 * j + 2 * q + h)] =
          make_float4(acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2],
                      acc[j][i][4 * q + 3]);
  lds_barrier();
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int64_t r0 = w4_erow(m0, i, p);
    const bool rok = r0 + rl < M;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(ep.C + r0 * ep.ldc + n0);
    float4 v[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v[t] = src[w4_eslot(rbase + 4 * p, sub + 16 * t)];
      if (HAS_X) {
        v[t].x += __uint_as_float(xv[p][t].x << 16);
        v[t].y += __uint_as_float(xv[p][t].x & 0xffff0000u);
        v[t].z += __uint_as_float(xv[p][t].y << 16);
        v[t].w += __uint_as_float(xv[p][t].y & 0xffff0000u);
      }
      const int c = 4 * sub + 64 * t;
      const bool cok = n0 + c < N;  // N % 4 == 0: the lane's 4 columns are all in or all out
      const u32x4 w = {__float_as_uint(v[t].x), __float_as_uint(v[t].y), __float_as_uint(v[t].z),
                       __float_as_uint(v[t].w)};
      __builtin_amdgcn_raw_buffer_store_b128(
          w, rc, (rok && cok) ? static_cast<uint32_t>((rl * ep.ldc + c) * 4) : kOutOfRange, 0,
          kStreamPolicy);
    }
    // statistics of the 4 tiles of 64 columns (tile t = the lanes' t-th
    // vector): maximum (every lane gets all four) and fixed-point exp-sum
    // (the lanes of quad q get tile q's) over the row's 16 lanes; the columns
    // past N contribute nothing, and a tile with no column in range is not
    // stored
    float mx[4];
    uint32_t ps[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float m4 = fmaxf(fmaxf(v[t].x, v[t].y), fmaxf(v[t].z, v[t].w));
      mx[t] = row16_max(n0 + 4 * sub + 64 * t < N ? m4 : -INFINITY);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float off = fix_exp_offset(mx[t]);
      const uint32_t s4 = fix_exp32o(v[t].x, off) + fix_exp32o(v[t].y, off) +
                          fix_exp32o(v[t].z, off) + fix_exp32o(v[t].w, off);
      ps[t] = (n0 + 4 * sub + 64 * t < N) ? s4 : 0u;
    }
    const uint32_t tot = quad_tile_sums(ps, sub);
    // lane 4 q of the row stores tile q
    const int q = sub >> 2;
    const float ms = q == 0 ? mx[0] : (q == 1 ? mx[1] : (q == 2 ? mx[2] : mx[3]));
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(ep.stats + r0 * ep.nstat + 4 * tn);
    const u32x2 sv = {__float_as_uint(ms), __float_as_uint(fix_to_float(tot))};
    const bool sok = (sub & 3) == 0 && rok && n0 + kStatTile * q < N;
    __builtin_amdgcn_raw_buffer_store_b64(
        sv, rs, sok ? static_cast<uint32_t>((rl * ep.nstat + q) * 8) : kOutOfRange, 0, 0);
  }
}

template <bool HAS_X>
__device__ __forceinline__ void w4_epilogue(const f32x16_v (&acc)[4][4], int64_t M, int64_t N,
                                            int64_t m0, int64_t n0, int64_t tn,
                                            const EpiParams& ep, float4* ea, float4* eb) {
  // two named addend buffers, one block ahead (loop unrolled: static names)
  uint2 xa[4][4], xb[4][4];
  if (HAS_X) {
    w4_x_issue(xa, ep, M, N, m0, n0, 0);
    w4_x_issue(xb, ep, M, N, m0, n0, 1);
  }
  w4_eblock<HAS_X>(acc, 0, xa, M, N, m0, n0, tn, ep, ea, eb);
  if (HAS_X) w4_x_issue(xa, ep, M, N, m0, n0, 2);
  w4_eblock<HAS_X>(acc, 1, xb, M, N, m0, n0, tn, ep, ea, eb);
  if (HAS_X) w4_x_issue(xb, ep, M, N, m0, n0, 3);
  w4_eblock<HAS_X>(acc, 2, xa, M, N, m0, n0, tn, ep, ea, eb);
  w4_eblock<HAS_X>(acc, 3, xb, M, N, m0, n0, tn, ep, ea, eb);
}

// One logits job over the 256 x 256 output tile grid.  Persistent: one
// workgroup per CU walks tiles blockIdx.x, blockIdx.x + gridDim.x, ... of the
// XCD-aware order (gridDim.x a multiple of 8 keeps each workgroup on one
// XCD's range).  The next tile's first two slices are queued into stages 0
// and 1 before the current epilogue, which uses stages 2 and 3, and its third
// slice right after, so operand loads and the previous tile's stores overlap
// the epilogue and the next main loop.  K = 0 is the epilogue alone (C = X).
// Operands are bf16, K-contiguous, K a multiple of 32.
__device__ __forceinline__ void w4_queue(const GemmJob& J, const TileCoord& tc, int64_t M,
                                         int64_t N, W4Offsets& o, const W4Ring& ring) {
  const int nk = static_cast<int>(J.K / 32);
  const int shift = (4 - (nk & 3)) & 3;
  w4_offsets<LAYOUT_KC, LAYOUT_KC>(o, J.A, J.B, M, N, tc.m0, tc.n0);
  if (nk > 0) {
    w4_issue<0, LAYOUT_KC, LAYOUT_KC>(J.A, J.B, 0, 0, nk, shift, tc.m0, tc.n0, o, ring);
    w4_issue<1, LAYOUT_KC, LAYOUT_KC>(J.A, J.B, 0, 1, nk, shift, tc.m0, tc.n0, o, ring);
  }
}
__device__ __forceinline__ void w4_queue_third(const GemmJob& J, const TileCoord& tc,
                                               const W4Offsets& o, const W4Ring& ring) {
  const int nk = static_cast<int>(J.K / 32);
  const int shift = (4 - (nk & 3)) & 3;
  if (nk > 0) w4_issue<2, LAYOUT_KC, LAYOUT_KC>(J.A, J.B, 0, 2, nk, shift, tc.m0, tc.n0, o, ring);
}

template <int TAG>
__global__ __launch_bounds__(256, 1) void gemm_w4_kernel(int64_t M, int64_t N, GemmJob J,
                                                         int group_m) {
  __shared__ u32x4 st0[w4::kStageCh], st1[w4::kStageCh], st2[w4::kStageCh], st3[w4::kStageCh];
  const W4Ring ring{{st0, st1, st2, st3}};
  float4* ea = reinterpret_cast<float4*>(st2);
  float4* eb = reinterpret_cast<float4*>(st3);
  const int64_t ntiles = ((M + 255) / 256) * ((N + 255) / 256);
  const int nk = static_cast<int>(J.K / 32);
  int64_t v = blockIdx.x;
  TileCoord tc = tile_coord_of(v, M, N, 256, 256, group_m);
  f32x16_v acc[4][4];
  W4Offsets o;
  w4_queue(J, tc, M, N, o, ring);
  w4_queue_third(J, tc, o, ring);
  for (;;) {
    w4_mainloop<LAYOUT_KC, LAYOUT_KC>(acc, J.A, J.B, 0, nk, tc.m0, tc.n0, o, ring);
    const int64_t vn = v + gridDim.x;
    const bool more = vn < ntiles;
    const TileCoord tnext = tile_coord_of(more ? vn : v, M, N, 256, 256, group_m);
    lds_barrier();  // every wave has read its last fragments of this tile
    if (more) w4_queue(J, tnext, M, N, o, ring);
    w4_epilogue<TAG == 0>(acc, M, N, tc.m0, tc.n0, tc.tn, J.ep, ea, eb);
    if (!more) break;
    lds_barrier();  // stage 2 is read for the last time
    w4_queue_third(J, tnext, o, ring);
    v = vn;
    tc = tnext;
  }
}

// ------------------------------------------------------------------ launch

namespace {
constexpr int kGroupM = 8;

int64_t split_kper(int64_t K, int splits, int bk) {
  if (splits <= 1) return K;
  return ((K + splits - 1) / splits + bk - 1) / bk * bk;
}

template <typename T, int EPI, int AL, int BL, int TAG>
hipError_t launch_generic(int64_t M, int64_t N, const Operand& A, const Operand& B, int splits,
                          const EpiParams& ep, hipStream_t s) {
  constexpr int BK = 8 * Elem<T>::kPerChunk;
  const int64_t K = A.kpad * A.nseg;
  const int64_t nM = (M + 255) / 256, nN = (N + 255) / 256;
  dim3 grid(static_cast<uint32_t>(nM * nN), static_cast<uint32_t>(splits), 1);
  hipLaunchKernelGGL((gemm_kernel<T, 256, 256, 2, 4, EPI, AL, BL, TAG>), grid, dim3(512), 0, s, M,
                     N, K, split_kper(K, splits, BK), A, B, ep, kGroupM);
  return hipGetLastError();
}

template <int EPI, int AL, int BL, int TAG>
hipError_t launch_dma(int64_t M, int64_t N, const GemmJob& j0, const GemmJob& j1, int njobs,
                      int splits, hipStream_t s) {
  const int64_t nM = (M + 255) / 256, nN = (N + 255) / 256;
  dim3 grid(static_cast<uint32_t>(nM * nN), static_cast<uint32_t>(splits), 1);
  const int64_t kper = splits > 1 ? split_kper(j0.K, splits, 32) : (j0.K > j1.K ? j0.K : j1.K);
  hipLaunchKernelGGL((gemm_dma_kernel<256, 256, 2, 4, EPI, AL, BL, TAG>), grid, dim3(512), 0, s, M,
                     N, kper, j0, j1, njobs, kGroupM);
  return hipGetLastError();
}

// Workgroups of the persistent 4-wave kernel: one per CU (a multiple of 8,
// so each stays within one XCD's tile range), at most one per tile.
int64_t w4_grid(int64_t tiles) {
  static const int cus = [] {  // initialized once, thread-safe
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8)
      n = 256;
    return n / 8 * 8;
  }();
  return tiles < cus ? tiles : cus;
}

// Row tiles per group of the logits tile order.  When the row tiles split
// evenly over the 8 XCDs into shares of 4 to 16, a group is one XCD's share:
// each XCD walks its own row tiles across every column tile, no two XCDs read
// the same H_t panels, and its 32 concurrent tiles span those rows x about
// 5 columns.  At 56 row tiles (14336 rows) groups of 7 measured 6 % faster
// than groups of 8, whose XCD ranges straddle groups.
int w4_group_m(int64_t nM) {
  return (nM % 8 == 0 && nM / 8 >= 4 && nM / 8 <= 16) ? static_cast<int>(nM / 8) : kGroupM;
}

template <int TAG>
hipError_t launch_w4(int64_t M, int64_t N, const GemmJob& J, hipStream_t s) {
  const int64_t nM = (M + 255) / 256;
  const int64_t tiles = nM * ((N + 255) / 256);
  hipLaunchKernelGGL((gemm_w4_kernel<TAG>), dim3(static_cast<uint32_t>(w4_grid(tiles))),
                     dim3(w4::kNT), 0, s, M, N, J, w4_group_m(nM));
  return hipGetLastError();
}

template <int AL, int BL, int TAG>
hipError_t launch_w4p_t(int64_t M, int64_t N, const Operand& A, const Operand& B, int splits,
                        float* C, int64_t ldc, hipStream_t s) {
  const int64_t K = A.kseg * A.nseg;
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const dim3 grid(static_cast<uint32_t>(tiles), static_cast<uint32_t>(splits), 1);
  hipLaunchKernelGGL((gemm_w4p_kernel<AL, BL, TAG>), grid, dim3(w4::kNT), 0, s, M, N, K,
                     split_kper(K, splits, 32), A, B, C, ldc, kGroupM);
  return hipGetLastError();
}

GemmJob job_of(const Operand& A, const Operand& B, const EpiParams& ep) {
  GemmJob j;
  j.A = A; j.B = B; j.ep = ep; j.K = A.kseg * A.nseg;
  return j;
}

// The DMA path needs bf16, K-contiguous (or both k-blocked) operands and
// 32-aligned K segments.
bool dma_ok(const Operand& A, const Operand& B) {
  const bool kc = A.layout == LAYOUT_KC && B.layout == LAYOUT_KC;
  const bool kb = A.layout == LAYOUT_KB && B.layout == LAYOUT_KB;
  return (kc || kb) && A.kseg % 32 == 0 && A.kseg > 0 && A.kseg == B.kseg && A.nseg == B.nseg;
}

template <typename T>
hipError_t launch_t(int epi, int tag, int64_t M, int64_t N, const Operand& A, const Operand& B,
                    int splits, const EpiParams& ep, hipStream_t s) {
  const bool kc = A.layout == LAYOUT_KC && B.layout == LAYOUT_KC;
  if (epi == EPI_STATS) {
    if (!kc) return hipErrorInvalidValue;
    return tag == 1 ? launch_generic<T, EPI_STATS, LAYOUT_KC, LAYOUT_KC, 1>(M, N, A, B, 1, ep, s)
                    : launch_generic<T, EPI_STATS, LAYOUT_KC, LAYOUT_KC, 0>(M, N, A, B, 1, ep, s);
  }
  if (epi == EPI_PARTIAL && A.layout == LAYOUT_KC && B.layout == LAYOUT_MC)
    return launch_generic<T, EPI_PARTIAL, LAYOUT_KC, LAYOUT_MC, 2>(M, N, A, B, splits, ep, s);
  if (epi == EPI_PARTIAL && kc)
    return launch_generic<T, EPI_PARTIAL, LAYOUT_KC, LAYOUT_KC, 2>(M, N, A, B, splits, ep, s);
  if (epi == EPI_PARTIAL && A.layout == LAYOUT_KB && B.layout == LAYOUT_KB)
    return launch_generic<T, EPI_PARTIAL, LAYOUT_KB, LAYOUT_KB, 3>(M, N, A, B, splits, ep, s);
  if (epi == EPI_STORE && A.layout == LAYOUT_MC && B.layout == LAYOUT_MC)
    return launch_generic<T, EPI_STORE, LAYOUT_MC, LAYOUT_MC, 3>(M, N, A, B, 1, ep, s);
  return hipErrorInvalidValue;
}
}  // namespace

bool w4p_ok(const Operand& A, const Operand& B, int64_t M, int64_t N) {
  auto lay_ok = [](const Operand& X, int64_t rows) {
    if (X.layout == LAYOUT_KC) return X.ld % 8 == 0;
    if (X.layout == LAYOUT_MK) return X.ld % 8 == 0 && rows % 8 == 0;
    return false;
  };
  return A.kseg > 0 && A.kseg % 32 == 0 && A.kseg == B.kseg && A.nseg == B.nseg && N % 4 == 0 &&
         lay_ok(A, M) && lay_ok(B, N);
}

hipError_t launch_gemm_w4p(int tag, int64_t M, int64_t N, const Operand& A, const Operand& B,
                           int splits, float* C, int64_t ldc, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (!w4p_ok(A, B, M, N) || splits < 1) return hipErrorInvalidValue;
  if (A.layout == LAYOUT_KC && B.layout == LAYOUT_MK && tag == 2)
    return launch_w4p_t<LAYOUT_KC, LAYOUT_MK, 2>(M, N, A, B, splits, C, ldc, s);
  if (A.layout == LAYOUT_MK && B.layout == LAYOUT_MK && tag == 3)
    return launch_w4p_t<LAYOUT_MK, LAYOUT_MK, 3>(M, N, A, B, splits, C, ldc, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(int dtype, int epi, int tag, int64_t M, int64_t N, const Operand& A,
                       const Operand& B, int splits, const EpiParams& ep, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (dtype == 1 && dma_ok(A, B)) {
    const GemmJob j = job_of(A, B, ep);
    if (A.layout == LAYOUT_KB) {
      if (epi == EPI_PARTIAL)
        return launch_dma<EPI_PARTIAL, LAYOUT_KB, LAYOUT_KB, 3>(M, N, j, j, 1, splits, s);
    } else {
      if (epi == EPI_STATS)
        return tag == 1 ? launch_w4<1>(M, N, j, s) : launch_w4<0>(M, N, j, s);
      if (epi == EPI_PARTIAL)
        return launch_dma<EPI_PARTIAL, LAYOUT_KC, LAYOUT_KC, 2>(M, N, j, j, 1, splits, s);
    }
  }
  return dtype == 1 ? launch_t<bf16_t>(epi, tag, M, N, A, B, splits, ep, s)
                    : launch_t<float>(epi, tag, M, N, A, B, splits, ep, s);
}

// The logits projections of the stored-logits forward pass and of the
// Markov head op: the corrected draft logits (K = markov rank, z as the
// epilogue addend) and then the teacher logits (K = hidden), each a launch of
// the persistent 4-wave kernel.  Both epilogues compute the tile statistics
// the same way (maximum; fixed-point exp-sum), so equal rows give equal
// results.  Where the bf16 DMA paths do not apply, both jobs take the
// generic kernel.
hipError_t launch_logits(int dtype, int64_t M, int64_t N, const Operand* A, const Operand* B,
                         const EpiParams* ep, int njobs, hipStream_t s) {
  if (M <= 0 || N <= 0 || njobs <= 0) return hipSuccess;
  bool dma = dtype == 1 && njobs <= 2;
  GemmJob j[2];
  for (int i = 0; i < njobs; ++i) {
    j[i] = job_of(A[i], B[i], ep[i]);
    if (j[i].K > 0 && !dma_ok(A[i], B[i])) dma = false;
  }
  if (dma) {
    hipError_t e = launch_w4<0>(M, N, j[0], s);
    if (e == hipSuccess && njobs == 2) e = launch_w4<1>(M, N, j[1], s);
    return e;
  }
  for (int i = 0; i < njobs; ++i) {
    const hipError_t e = (dtype == 1)
        ? launch_t<bf16_t>(EPI_STATS, i == njobs - 1 ? 1 : 0, M, N, A[i], B[i], 1, ep[i], s)
        : launch_t<float>(EPI_STATS, i == njobs - 1 ? 1 : 0, M, N, A[i], B[i], 1, ep[i], s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dspark
