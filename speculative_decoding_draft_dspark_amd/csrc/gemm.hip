// MFMA GEMM C[M,N] = A[M,K] . B[N,K]^T for the DSpark loss (gfx950).
//
// Used for the dense contractions of the loss:
//   - the teacher lm_head projection T = H_t . LM^T (TorchSpec pull request
//     #132, PR description: teacher = target lm_head on the final hidden state),
//   - the Markov low-rank bias z' = z + E . W2^T with E = W1[prev] (NeMo-RL
//     "DSpark Auxiliary Heads", Inputs and Outputs),
//   - the backward products dE = G . W2 and dW2 = G^T . E.
//
// Two main loops share one tile order and one epilogue:
//   * gemm_dma_kernel (bf16, both operands K-contiguous, K a multiple of 32):
//     operand tiles go global -> LDS with buffer_load_dwordx4 ... lds (no VGPR
//     staging), through a 4-stage ring of BK = 32 slices prefetched 3 slices
//     ahead, one barrier per slice.  This is the lm_head / logits path.
//   * gemm_kernel (fp32 or bf16, any operand layout): register-staged,
//     double-buffered LDS; operands may be K-contiguous, M-contiguous
//     (transposed on the way into LDS) or k-blocked ([K/c][M][c] with c
//     elements per 16-byte chunk).
// Both: 256 x 256 output tiles, 8 waves of 128 x 64 each built from
// v_mfma_f32_16x16x32_bf16 (bf16) or v_mfma_f32_16x16x4_f32 (fp32; in this
// loss the 32x32x16 form measured slower in the full GEMM); LDS rows
// of 16-byte chunks XOR-swizzled so MFMA operand reads are conflict-free; an
// XCD-aware grouped tile order (each of the 8 XCDs works a contiguous range so
// operand slices are shared through its own L2).  Operands may consist of two
// K segments (used for hi/lo splits of a bf16 gradient).
#include "common.h"
#include "internal.h"

namespace dspark {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
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
__device__ __forceinline__ TileCoord tile_coord(int64_t M, int64_t N, int BM, int BN,
                                                int group_m) {
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
  return {tm * BM, tn * BN, tn};
}

// Workgroup barrier ordering LDS accesses only.  __syncthreads() also fences
// global memory, which makes every wave drain its in-flight global loads and
// stores (vmcnt(0)) at each barrier; here only LDS hazards need ordering, so
// the wave waits for its own LDS operations (lgkmcnt(0)) and meets the others.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
}

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
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < kVecs; ++i) {
        const int64_t col = n0 + sub * 4 + 32 * i;
        if (col < N) {  // N % 4 == 0: the 4 columns are all in or all out
          if (rowok) *reinterpret_cast<float4*>(C + row * ep.ldc + col) = v[i];
          mx = fmaxf(mx, fmaxf(fmaxf(v[i].x, v[i].y), fmaxf(v[i].z, v[i].w)));
        }
      }
#pragma unroll
      for (int o = 1; o < kLanesPerRow; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
      // fixed-point sum of exp(x - max): exact integer adds, so the result does
      // not depend on the order in which the columns are visited
      uint64_t sum = 0;
      if (mx != -INFINITY) {
#pragma unroll
        for (int i = 0; i < kVecs; ++i) {
          const int64_t col = n0 + sub * 4 + 32 * i;
          if (col < N) {
            sum += static_cast<uint64_t>(rintf(dexp(v[i].x - mx) * kFixScale)) +
                   static_cast<uint64_t>(rintf(dexp(v[i].y - mx) * kFixScale)) +
                   static_cast<uint64_t>(rintf(dexp(v[i].z - mx) * kFixScale)) +
                   static_cast<uint64_t>(rintf(dexp(v[i].w - mx) * kFixScale));
          }
        }
      }
#pragma unroll
      for (int o = 1; o < kLanesPerRow; o <<= 1) {
        const uint32_t lo = __shfl_xor(static_cast<uint32_t>(sum), o, kWave);
        const uint32_t hi = __shfl_xor(static_cast<uint32_t>(sum >> 32), o, kWave);
        sum += (static_cast<uint64_t>(hi) << 32) | lo;
      }
      if (sub == 0 && rowok) {
        const float l = static_cast<float>(static_cast<double>(sum) * (1.0 / 2147483648.0));
        ep.stats[row * ep.nstat + tn] = make_float2(mx, l);
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
  static_assert(EPI != EPI_STATS || BN == kStatTile, "stats epilogue needs BN == stat tile");

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
// tile (the corrected draft logits and the teacher logits share M and N, so a
// workgroup's memory-heavy draft epilogue overlaps other workgroups' MFMA
// phases).  A job with K = 0 is its epilogue alone (C = X).
template <int BM, int BN, int WM, int WN, int EPI, int AL, int BL, int TAG>
__global__ __launch_bounds__(WM* WN * 64, 1) void gemm_dma_kernel(int64_t M, int64_t N,
                                                                  int64_t kper, GemmJob j0,
                                                                  GemmJob j1, int njobs,
                                                                  int group_m) {
  static_assert(EPI != EPI_STATS || BN == kStatTile, "stats epilogue needs BN == stat tile");
  __shared__ u32x4 lds[4 * (BM * 4 + BN * 4)];
  const TileCoord tc = tile_coord(M, N, BM, BN, group_m);
  dma_job<BM, BN, WM, WN, EPI, AL, BL>(j0, M, N, kper, tc, lds);
  if (njobs > 1) dma_job<BM, BN, WM, WN, EPI, AL, BL>(j1, M, N, kper, tc, lds);
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
        return tag == 1 ? launch_dma<EPI_STATS, LAYOUT_KC, LAYOUT_KC, 1>(M, N, j, j, 1, 1, s)
                        : launch_dma<EPI_STATS, LAYOUT_KC, LAYOUT_KC, 0>(M, N, j, j, 1, 1, s);
      if (epi == EPI_PARTIAL)
        return launch_dma<EPI_PARTIAL, LAYOUT_KC, LAYOUT_KC, 2>(M, N, j, j, 1, splits, s);
    }
  }
  return dtype == 1 ? launch_t<bf16_t>(epi, tag, M, N, A, B, splits, ep, s)
                    : launch_t<float>(epi, tag, M, N, A, B, splits, ep, s);
}

// Both logits projections of the forward pass in one launch when both can use
// the DMA path (bf16, K-contiguous, K a multiple of 32 or K = 0); otherwise one
// launch each.
hipError_t launch_logits(int dtype, int64_t M, int64_t N, const Operand* A, const Operand* B,
                         const EpiParams* ep, int njobs, hipStream_t s) {
  if (M <= 0 || N <= 0 || njobs <= 0) return hipSuccess;
  bool fused = dtype == 1 && njobs <= 2;
  GemmJob j[2];
  for (int i = 0; i < njobs; ++i) {
    j[i] = job_of(A[i], B[i], ep[i]);
    if (j[i].K > 0 && !dma_ok(A[i], B[i])) fused = false;
  }
  if (fused)
    return launch_dma<EPI_STATS, LAYOUT_KC, LAYOUT_KC, 4>(M, N, j[0], j[njobs - 1], njobs, 1, s);
  for (int i = 0; i < njobs; ++i) {
    const hipError_t e = launch_gemm(dtype, EPI_STATS, i == njobs - 1 ? 1 : 0, M, N, A[i], B[i], 1,
                                     ep[i], s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dspark
