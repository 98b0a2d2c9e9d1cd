// Vocabulary sweeps that recompute the Markov bias of the corrected draft
// logits z' = z + E . W2^T (NeMo-RL "DSpark Auxiliary Heads", Inputs and
// Outputs) slice by slice, so the loss never writes z' to memory: the softmax
// statistics of z' (the first pass of the loss), the L1 / S / CE pass and the
// gradient pass (TorchSpec pull request #132, loss section: the fp32 log-softmax,
// the probability L1 and its gradient) each read z (bf16) and rebuild z'.  A
// fourth pass stores z' itself (fp32) for the standalone Markov head op.
//
// Work split: a workgroup of 8 waves owns 256 rows and one range of the
// vocabulary; each wave owns 32 rows (two MFMA row blocks of 16).  The wave
// keeps its rows of E as MFMA fragments in registers for the whole sweep; W2
// streams through a 4-stage LDS ring in slices of 64 vocabulary rows, filled
// by LDS-DMA three slices ahead and shared by the 8 waves.  Per slice and wave
// the bias is 4 vocabulary blocks x 2 row blocks of v_mfma_f32_16x16x32_bf16
// over the rank, with the W2 fragment as the first operand, so each fragment
// read from LDS feeds two MFMAs.  The W2 rows of a block are permuted so that
// lane (g, cl) ends up with the 8 consecutive columns 32 h + 8 g .. + 7 of
// its row for each block pair h: z (bf16) is one 16-byte chunk per
// (h, row block), loaded in whole lines and moved to its lane by a row
// rotation outside the L1 pass, and T (fp32) two.  z, widened to fp32, is the initial
// accumulator of the MFMA chains, so they end at z' itself.  Every sweep
// computes z' with the same instruction sequence, so all three see the same
// values.  A slice is one softmax-statistics tile (64 columns).
#include "bias_sweep.h"

#include "common.h"

namespace dspark {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// Buffer resource over `bytes` from base (untyped dword loads); offsets at or
// past the end read as zero and stores there are dropped, so every load and
// store is issued unconditionally and the compiler's wait counts stay exact.
constexpr uint32_t kOOB = 0xffffffffu;
// A lane offset past every buffer that stays so with the in-instruction
// offsets added (buffers here hold fewer than 2^31 bytes).
constexpr uint32_t kFar = 0x80000000u;
// Cache policy of the statistics sweep's z stream: non-temporal, so it does
// not evict the W2 slices every row tile re-reads (measured faster there; the
// L1 and gradient sweeps' streams measured faster with the default policy).
constexpr int kStream = 2;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

constexpr int kWaves = 8, kNT = kWaves * 64;
constexpr int kRowsPerWave = 32, kRowsPerWG = kWaves * kRowsPerWave;  // 256
constexpr int kSliceV = 64;  // vocabulary rows of W2 per slice (4 MFMA blocks of 16)
static_assert(kSliceV == kStatTile, "a slice is one statistics tile");
constexpr int kStages = 4;   // W2 slices in LDS: the one in use and three in flight

enum SweepMode { kStats = 0, kL1 = 1, kGrad = 2, kStore = 3 };

__device__ __forceinline__ void lds_sync() {
  // order LDS accesses only (no wait on outstanding global loads or stores)
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
}

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt <= n only.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// Reductions over the lanes l, l ^ 16, l ^ 32, l ^ 48 (a row's four lanes g)
// with the gfx950 lane swaps: with both operands x, permlane16_swap leaves
// {x[l], x[l ^ 16]} in its two results and permlane32_swap {x[l], x[l ^ 32]},
// so one swap and one operation per step, no LDS round trip.
__device__ __forceinline__ float max_g4(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ uint32_t sum_g4(uint32_t v) {
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = r[0] + r[1];
  r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return r[0] + r[1];
}

// Column within the slice of output m (0..15) of vocabulary block b (0..3):
// lane (g, cl) receives outputs 4 g .. 4 g + 3, i.e. columns
// 32 (b >> 1) + 8 g + 4 (b & 1) + 0..3.
__device__ __forceinline__ int vcol(int b, int m) {
  return 32 * (b >> 1) + 8 * (m >> 2) + 4 * (b & 1) + (m & 3);
}

// The bias of one wave's 32 rows over vocabulary slices: E fragments in
// registers, W2 slices in the LDS ring (rank RANK, a multiple of 32).
template <int RANK>
struct BiasEngine {
  static constexpr int KS = RANK > 0 ? RANK / 32 : 1;            // MFMA k steps over the rank
  static constexpr int CPR = RANK > 0 ? RANK / 8 : 1;             // 16-byte chunks per W2 row
  static constexpr int SWM = (CPR < 16 ? CPR : 16) - 1;           // chunk XOR against bank conflicts
  static constexpr int kChunks = RANK > 0 ? kSliceV * CPR : 0;    // chunks per slice
  static constexpr int kPer = kChunks > kNT ? kChunks / kNT : 1;  // DMA loads per thread per slice
  static constexpr int kStageCh = kPer * kNT;                     // u32x4 per ring stage

  u32x4 e[2][KS];  // [row block][k step]

  // LDS slot of chunk c of W2 row v: the chunk index is XORed with the MFMA
  // lane cl that reads row v (vcol(b, cl) = v), so the 16 rows one quarter
  // wave reads at the same k land in 16 distinct 16-byte bank groups.
  __device__ __forceinline__ static int lane_of(int v) { return (v & 3) | ((v >> 1) & 12); }
  __device__ __forceinline__ static int slot(int v, int c) { return v * CPR + (c ^ (lane_of(v) & SWM)); }

  // E fragments: lane (g, cl) holds row r0 + 16 rb + cl at rank 32 ks + 8 g .. + 7.
  __device__ __forceinline__ void load_e(const bf16_t* E, int64_t r0, int64_t R) {
    const int lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int64_t row = r0 + 16 * rb + cl;
      const int64_t rr = row < R ? row : R - 1;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (RANK == 0) { e[rb][ks] = u32x4{0u, 0u, 0u, 0u}; continue; }
        const u32x4 v = *reinterpret_cast<const u32x4*>(E + rr * RANK + 32 * ks + 8 * g);
        e[rb][ks] = row < R ? v : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  // Queue W2 rows [v0, v0 + 64) into a ring stage.  The buffer resource ends
  // at row vend, so rows past it read zero with no per-lane test; kPer loads
  // per thread, always issued.
  __device__ __forceinline__ void dma(const bf16_t* W2, int64_t v0, int64_t vend, u32x4* stage) const {
    if (RANK == 0) return;
    const int wave = threadIdx.x >> 6;
    const int64_t nv = vend - v0;
    const int64_t nrow = nv <= 0 ? int64_t{0} : (nv < int64_t{kSliceV} ? nv : int64_t{kSliceV});
    const __amdgpu_buffer_rsrc_t rs =
        rsrc_of(W2 + (nv > 0 ? v0 : int64_t{0}) * RANK, static_cast<uint32_t>(nrow * RANK * 2));
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      // lane l of the wave's p-th load fills chunk idx of the stage: row
      // idx / CPR, slot idx % CPR, which holds chunk slot ^ (lane_of(row) & SWM)
      const int idx = (wave * kPer + p) * 64 + lane;
      const int v = idx / CPR, c = (idx % CPR) ^ (lane_of(v) & SWM);
      const uint32_t off = idx < kChunks ? static_cast<uint32_t>((v * RANK + 8 * c) * 2) : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(stage + (wave * kPer + p) * 64), 16,
                                               off, 0, 0, 0);
    }
  }
  // Adds the bias of vocabulary blocks 2 h, 2 h + 1 of the slice in buf for
  // both row blocks to acc[bb][rb] (z on entry, so the chains end at z'); four
  // independent MFMA chains, the next k step's W2 fragments read while the
  // current step's MFMAs run.
  __device__ __forceinline__ void bias_pair(const u32x4* buf, int h, f32x4_v (&acc)[2][2]) const {
    if (RANK == 0) return;
    const int lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
    u32x4 w[KS][2];  // fully unrolled: registers, read one k step ahead of their MFMAs
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) w[0][bb] = buf[slot(vcol(2 * h + bb, cl), g)];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) {
#pragma unroll
        for (int bb = 0; bb < 2; ++bb)
          w[ks + 1][bb] = buf[slot(vcol(2 * h + bb, cl), 4 * (ks + 1) + g)];
      }
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          acc[bb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_v, w[ks][bb]), __builtin_bit_cast(bf16x8_v, e[rb][ks]),
              acc[bb][rb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads at most one k step ahead
    }
  }
};

// The lane's z (bf16), T (fp32, L1 pass) and sign bits (gradient pass) of
// one slice: per block pair h and row block rb, the 8 columns 32 h + 8 g .. + 7
// (z as loaded in whole lines until Sweep::fix() has run).
template <bool LOADT, bool LOADS>
struct SliceData {
  u32x4 z[2][2];
  u32x4 t[LOADT ? 2 : 1][2][2];  // [h][rb][half]
  u32x2 sg;  // sign(p - q) of block pair h in word h: bits 2 (8 rb + i), +1 / -1 / 0 as 01 / 11 / 00
};

// z of the lane's 8 columns (h, rb) as the accumulators of bias blocks 2 h
// (columns 0..3) and 2 h + 1 (columns 4..7).
__device__ __forceinline__ void z_acc(const u32x4& zz, f32x4_v& b0, f32x4_v& b1) {
  b0 = f32x4_v{__uint_as_float(zz.x << 16), __uint_as_float(zz.x & 0xffff0000u),
               __uint_as_float(zz.y << 16), __uint_as_float(zz.y & 0xffff0000u)};
  b1 = f32x4_v{__uint_as_float(zz.z << 16), __uint_as_float(zz.z & 0xffff0000u),
               __uint_as_float(zz.w << 16), __uint_as_float(zz.w & 0xffff0000u)};
}

struct SweepParams {
  int64_t R, V, nstat, vsplit;
  const bf16_t* z;
  const bf16_t* E;
  const bf16_t* W2;
  const float* T;
  const int32_t* tid;
  RowState rs;
  float2* sz;
  double* part_l1;
  double* part_s;
  u32x2* signs;  // [row tiles x 8 waves][nstat][64 lanes]
  void* dz;
  bf16_t* ghi;
  bf16_t* glo;
  float g, ce_a, l1_a;
  int shard;  // vocabulary shard: a target id outside [0, V) lives in another shard
  float* zout;           // store pass: z' [R, V] fp32
  const uint8_t* valid;  // store pass: rows to write (null: all); the others get zeros
};

// State of one sweep over a workgroup's 256 rows and vocabulary range.
// TEACHER: a teacher exists (the L1 pass reads T and writes the sign bits of
// p - q; the gradient pass reads those bits instead of T).
template <int RANK, int MODE, bool TEACHER, typename GT>
struct Sweep {
  using Eng = BiasEngine<RANK>;
  static constexpr bool kLoadT = TEACHER && MODE == kL1;
  static constexpr bool kLoadS = TEACHER && MODE == kGrad;
  using SD = SliceData<kLoadT, kLoadS>;
  static constexpr int kZT = 4 + (kLoadT ? 8 : 0) + (kLoadS ? 1 : 0);  // loads per lane per slice
  // stores issued unconditionally per slice: the statistics tile, the sign
  // words, or dz (bf16: one per (h, rb); fp32: two, plus G hi)
  static constexpr int kST = MODE == kStats || MODE == kL1 ? 1
                             : (MODE == kStore ? 8 : (sizeof(GT) == 2 ? 4 : 12));
  // slices of z / T in flight ahead of the one in use: 2 without T, 1 with T
  // (three register sets of z and T would not fit two waves per SIMD)
  static constexpr int kLead = kLoadT ? 1 : 2;
  static constexpr bool kWholeLines = MODE != kL1;  // z loads in whole lines
  const SweepParams& P;
  u32x4* ring;  // kStages x Eng::kStageCh
  Eng eng;
  int64_t r0;      // the wave's first row (wave-uniform)
  int64_t vb, ve;  // this workgroup's vocabulary range
  int nsl;         // slices in the range
  int g, cl;
  int vlen;        // columns in the range
  bool rowok[2], sup[2];
  float lz[2], lt[2], Sr[2], cc[2], cl1[2];  // lz, lt: lse_z, lse_t times log2 e
  int yl[2];          // target column within the range, -1 if outside
  // Per-lane element offset of (row r0 + 16 rb + cl, column 8 g) from a
  // slice's origin (row r0, its first column); rows past R: kFar, past every
  // buffer.  Each step builds its buffer resources at the slice's origin
  // (scalar arithmetic), so the lane offsets never change and no load needs
  // per-element address arithmetic; a resource ends at the end of the wave's
  // 32 rows, so no access leaves them.
  uint32_t eoff[2];
  // whole-line z loads: byte offset of load p of row block rb from a slice's
  // origin; hi = lane bit 3 (the second half of the lane's 16-lane row)
  uint32_t zoff[2][2];
  bool hi;
  uint32_t span;      // elements from row r0 to the end of the wave's rows below R
  uint32_t stoff;     // statistics pass: byte offset of the lane's tile store (lanes g = rb < 2)
  int64_t orig;       // element offset of the range's origin (row r0, column vb)
  double a_l1[2], a_s[2];  // L1 pass accumulators
  uint32_t wsg[2];         // L1 pass: sign words of the slice in progress
  float c0[2];             // gradient: g w (ce_a - l1_a S); + / - g w l1_a for sign +1 / -1
  u32x4 dzv[2][2];         // gradient, bf16 dz: the lane's chunk per (block pair, row block)

  __device__ __forceinline__ Sweep(const SweepParams& p, u32x4* rg) : P(p), ring(rg) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    g = lane >> 4;
    cl = lane & 15;
    hi = (lane & 8) != 0;
    // wave-uniform, so the buffer resources built from it are scalar and no
    // load or store needs a waterfall loop
    r0 = static_cast<int64_t>(blockIdx.x) * kRowsPerWG + wave * kRowsPerWave;
    vb = static_cast<int64_t>(blockIdx.y) * P.vsplit;
    ve = (vb + P.vsplit) < P.V ? (vb + P.vsplit) : P.V;
    nsl = vb < ve ? static_cast<int>((ve - vb + kSliceV - 1) / kSliceV) : 0;
    vlen = static_cast<int>(ve > vb ? ve - vb : 0);
    {
      const int64_t rows = P.R - r0 < kRowsPerWave ? P.R - r0 : kRowsPerWave;
      span = rows > 0 ? static_cast<uint32_t>(rows * P.V) : 0u;
    }
    orig = r0 * P.V + vb;
    stoff = g < 2 && r0 + 16 * g + cl < P.R
                ? static_cast<uint32_t>((16 * g + cl) * P.nstat * 8) : kOOB;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int64_t row = r0 + 16 * rb + cl;
      rowok[rb] = row < P.R;
      if (MODE == kStore)
        sup[rb] = rowok[rb] && (P.valid == nullptr || P.valid[row] != 0);
      else
        sup[rb] = MODE != kStats && rowok[rb] && P.rs.mask[row] != 0;
      lz[rb] = lt[rb] = Sr[rb] = cc[rb] = cl1[rb] = c0[rb] = 0.f;
      int64_t y = -1;
      if (MODE != kStats && MODE != kStore && sup[rb]) {
        // exp(x - lse) as exp2(x log2 e - lse log2 e): one fma per element
        lz[rb] = P.rs.lse_z[row] * kLog2e;
        lt[rb] = P.rs.lse_t[row] * kLog2e;
        if (MODE == kGrad) {
          const float gw = P.g * P.rs.w[row];
          cc[rb] = gw * P.ce_a;
          cl1[rb] = gw * P.l1_a;
          Sr[rb] = P.rs.S[row];
          c0[rb] = cc[rb] - cl1[rb] * Sr[rb];
        }
        const int64_t t = P.tid[row];
        if (P.shard) y = (t >= 0 && t < P.V) ? t : -1;  // another shard owns the target
        else y = t < 0 ? 0 : (t >= P.V ? P.V - 1 : t);
      }
      yl[rb] = (y >= vb && y < ve) ? static_cast<int>(y - vb) : -1;
      eoff[rb] = rowok[rb] ? static_cast<uint32_t>((16 * rb + cl) * P.V + 8 * g) : kFar;
      {
        // lane 16 g + 8 k + r: load 0 brings row r of the block, chunk
        // 4 k + g; load 1 row 8 + r, chunk 4 (1 - k) + g.  Rows past R lie
        // past the slice's buffer resource and read zero.
        const int r = lane & 7, k = (lane >> 3) & 1;
        zoff[0][rb] = static_cast<uint32_t>(((16 * rb + r) * P.V + 8 * (4 * k + g)) * 2);
        zoff[1][rb] = static_cast<uint32_t>(((16 * rb + 8 + r) * P.V + 8 * (4 * (1 - k) + g)) * 2);
      }
      a_l1[rb] = a_s[rb] = 0.0;
    }
  }

  __device__ __forceinline__ int64_t col0(int s) const { return vb + static_cast<int64_t>(s) * kSliceV; }
  __device__ __forceinline__ u32x4* stage(int t) const { return ring + (t % kStages) * Eng::kStageCh; }

  // Buffer resource over an [R, V] array from the origin of the slice at
  // column cs of the range to the end of the wave's rows (its last row below
  // R), so that no access leaves the array.
  template <typename E>
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const E* base, int cs) const {
    const uint32_t o = static_cast<uint32_t>(vb + cs);
    return rsrc_of(base + orig + cs, span > o ? (span - o) * static_cast<uint32_t>(sizeof(E)) : 0u);
  }
  // The lane's byte offset for element offset eo (kFar stays past the end).
  template <int ES>
  __device__ __forceinline__ static uint32_t bo(uint32_t eo) {
    return eo == kFar ? kFar : eo * ES;
  }

  // The lane's z and T of the slice at column cs of the range.  Rows past R
  // read zero; columns past the range read the neighbouring range's values
  // (or zero past the wave's rows), which the work on the slice masks out.
  __device__ __forceinline__ void load(SD& d, int cs) const {
    // Outside the L1 pass z comes in whole 128-byte lines (8 rows x 8
    // chunks of 16 bytes per load; load p of row block rb covers its rows
    // 8 p .. 8 p + 7) and fix() moves each chunk to the lane that computes on
    // it; the L1 pass, whose T loads dominate and whose registers are full,
    // loads each lane's own chunks (16 rows x 64 bytes per load).
    const __amdgpu_buffer_rsrc_t rzs = slice_rsrc(P.z, cs);
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        d.z[p][rb] = __builtin_amdgcn_raw_buffer_load_b128(
            rzs, kWholeLines ? zoff[p][rb] : bo<2>(eoff[rb]) + 64 * p, 0,
            MODE == kStats ? kStream : 0);
    if (kLoadT) {
      const __amdgpu_buffer_rsrc_t rts = slice_rsrc(P.T, cs);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int q = 0; q < 2; ++q)
            d.t[h][rb][q] = __builtin_amdgcn_raw_buffer_load_b128(
                rts, bo<4>(eoff[rb]) + 128 * h + 16 * q, 0, 0);
    }
    if (kLoadS) {
      // the wave's words of slice tn: slices past the range read zeros
      const int tn = (static_cast<int>(vb) + cs) / kSliceV;
      const int lane = threadIdx.x & 63;
      const __amdgpu_buffer_rsrc_t rs = sign_rsrc(tn);
      d.sg = __builtin_amdgcn_raw_buffer_load_b64(rs, cs < vlen ? lane * 8u : kOOB, 0, 0);
    }
  }
  // The wave's sign words from slice tn on.
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t sign_rsrc(int tn) const {
    const int64_t w = (r0 / kRowsPerWave) * P.nstat * 64 + static_cast<int64_t>(tn) * 64;
    return rsrc_of(P.signs + w, tn < P.nstat ? static_cast<uint32_t>((P.nstat - tn) * 64 * 8) : 0u);
  }

  // Slice s, whose z / T are in `cur`; queues W2 of slice s + 3 into the ring
  // (the stage slice s - 1 used) and z / T of slice s + kLead into `nxt` (the
  // buffer of slice s - 1, already consumed), so no register copies put a
  // wait on loads still in flight.  Loads past the range read zeros and are
  // always issued, and the per-element conditions are selects, so every wait
  // count is static.
  // The two whole-line loads of a row block into each lane's own chunks
  // (block pair 0 in a, 1 in b).  The low half of a 16-lane row holds its own
  // pair-0 chunk in a, the high half in b; each half's other load holds the
  // pair-1 chunk of the lane 8 away in the same row (row_ror:8).
  __device__ __forceinline__ void fix_pair(u32x4& a, u32x4& b) const {
    u32x4 own, other;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      own[j] = hi ? b[j] : a[j];
      const uint32_t x = hi ? a[j] : b[j];
      other[j] = static_cast<uint32_t>(
          __builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x128, 0xf, 0xf, false));
    }
    a = own;
    b = other;
  }
  // The inverse of fix_pair: the lanes' own chunks a (block pair 0) and b
  // (block pair 1) of a row block into the two whole-line stores (rows 0..7
  // and 8..15 of the block, as loaded).
  __device__ __forceinline__ void unfix_pair(const u32x4& a, const u32x4& b, u32x4& lo,
                                             u32x4& up) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t y = static_cast<uint32_t>(
          __builtin_amdgcn_update_dpp(0, static_cast<int>(b[j]), 0x128, 0xf, 0xf, false));
      lo[j] = hi ? y : a[j];
      up[j] = hi ? a[j] : y;
    }
  }
  // bf16 dz of the slice in whole 128-byte lines (the layout of the whole-line
  // z loads); a chunk whose columns lie past the range belongs to another
  // workgroup and is not written, rows past R lie past the buffer.
  __device__ __forceinline__ void store_dz(int cs) {
    const __amdgpu_buffer_rsrc_t rd = slice_rsrc(static_cast<bf16_t*>(P.dz), cs);
    const int k = hi ? 1 : 0;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      u32x4 v[2];
      unfix_pair(dzv[0][rb], dzv[1][rb], v[0], v[1]);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int c = p == 0 ? 4 * k + g : 4 * (1 - k) + g;  // the chunk this lane stores
        __builtin_amdgcn_raw_buffer_store_b128(v[p], rd, cs + 8 * c < vlen ? zoff[p][rb] : kFar,
                                               0, 0);
      }
    }
  }
  __device__ __forceinline__ void fix(SD& d) const {
    if (!kWholeLines) return;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) fix_pair(d.z[0][rb], d.z[1][rb]);
  }

  __device__ __forceinline__ void step(int s, SD& cur, SD& nxt) {
    // W2 of slice s landed: it was queued in step s - 3 (the prologue drains
    // its own), followed by that step's z / T loads and stores and two more
    // steps' DMA, loads and stores.  The vector memory counter retires loads
    // and stores in issue order, so counting the stores too leaves them in
    // flight instead of waiting for their writes every step (the G lo store
    // is conditional and not counted: the count stays a lower bound).
    static_assert(2 * Eng::kPer + 3 * kZT + 3 * kST < 64, "vmcnt range");
    wait_vm<2 * Eng::kPer + 3 * kZT + 3 * kST>();
    lds_sync();  // every wave's W2 slice s is in LDS; slice s - 1's stage is free
    eng.dma(P.W2, col0(s + 3), ve, stage(s + 3));
    // first column of the slice within the range, opaque to the optimizer:
    // otherwise loop strength reduction keeps one induction variable per
    // (slice of the unrolled loop, element) column test, far more registers
    // than recomputing the columns from cs each step
    int cs = __builtin_amdgcn_readfirstlane(s * kSliceV);
    asm volatile("" : "+s"(cs));
    load(nxt, cs + kLead * kSliceV);
    fix(cur);
    float zp[2][2][8];  // [h][rb][column]
    wsg[0] = wsg[1] = 0u;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4_v acc[2][2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) z_acc(cur.z[h][rb], acc[0][rb], acc[1][rb]);
      eng.bias_pair(stage(s), h, acc);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 8; ++i) zp[h][rb][i] = acc[i >> 2][rb][i & 3];
      if (MODE == kL1) l1_work(cs, h, cur, zp[h]);
      if (MODE == kGrad) grad_work(cs, h, cur, zp[h]);
      if (MODE == kStore) store_work(cs, h, zp[h]);
    }
    if (MODE == kStats) stats_work(cs, zp);
    if (MODE == kGrad && sizeof(GT) == 2) store_dz(cs);
    if (MODE == kL1) {  // every slice's words, stored unconditionally
      const int tn = (static_cast<int>(vb) + cs) / kSliceV;
      const int lane = threadIdx.x & 63;
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{wsg[0], wsg[1]}, sign_rsrc(tn), lane * 8u, 0,
                                            0);
    }
  }

  // Statistics of the slice (one 64-column tile) for both row blocks: the
  // maximum, then the fixed-point exp-sum, over the row's 4 lanes (g).
  __device__ __forceinline__ void stats_work(int cs, const float (&zp)[2][2][8]) {
    float2 out[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float mx = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool ok = cs + 32 * h + 8 * g < vlen;
        float m8 = zp[h][rb][0];
#pragma unroll
        for (int i = 1; i < 8; ++i) m8 = fmaxf(m8, zp[h][rb][i]);
        mx = ok ? fmaxf(mx, m8) : mx;
      }
      mx = max_g4(mx);
      const float off = fix_exp_offset(mx);
      uint32_t sum = 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool ok = cs + 32 * h + 8 * g < vlen;
        uint32_t s8 = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) s8 += fix_exp32o(zp[h][rb][i], off);
        sum += ok ? s8 : 0u;
      }
      sum = mx == -INFINITY ? 0u : sum;
      sum = sum_g4(sum);
      out[rb] = make_float2(mx, fix_to_float(sum));
    }
    // lane g = rb stores row block rb's tile (s < nsl: the tile has columns)
    const int rb = g & 1;
    const float2 o = rb == 0 ? out[0] : out[1];
    const int64_t tn = (vb + cs) / kSliceV;
    const __amdgpu_buffer_rsrc_t rs =
        rsrc_of(P.sz + r0 * P.nstat + tn,
                static_cast<uint32_t>((kRowsPerWave * P.nstat - tn) * 8));
    const u32x2 v = {__float_as_uint(o.x), __float_as_uint(o.y)};
    __builtin_amdgcn_raw_buffer_store_b64(v, rs, stoff, 0, 0);
  }

  // The lane's column i of 8 holding the row's target, or -1.
  __device__ __forceinline__ static int target_in(int yl_, int col) {
    const int d = yl_ - col;
    return static_cast<unsigned>(d) < 8u ? d : -1;
  }

  // L1 pass on block pair h: sum |p - q| and sum p sign(p - q), and the
  // signs as 2-bit two's-complement fields for the gradient pass.  sign(p - q)
  // is the sign bit of q - p minus that of p - q: a tie makes both +0, so
  // sign(0) = 0.
  __device__ __forceinline__ void l1_work(int cs, int h, const SD& cur, const float (&zh)[2][8]) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int col = cs + 32 * h + 8 * g;  // within the range
      const bool ok = sup[rb] && col < vlen;
      float s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float t = __uint_as_float(cur.t[h][rb][i >> 2][i & 3]);
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(zh[rb][i], kLog2e, -lz[rb]));
        const float q = __builtin_amdgcn_exp2f(__builtin_fmaf(t, kLog2e, -lt[rb]));
        const float d = p - q, e = q - p;
        const int sg = static_cast<int>(__float_as_uint(e) >> 31) -
                       static_cast<int>(__float_as_uint(d) >> 31);
        wsg[h] |= static_cast<uint32_t>(sg & 3) << (2 * (8 * rb + i));
        s1 += fabsf(d);
        s2 = __builtin_fmaf(p, static_cast<float>(sg), s2);
      }
      a_l1[rb] += ok ? s1 : 0.f;
      a_s[rb] += ok ? s2 : 0.f;
    }
  }

  // Gradient on block pair h: G = g w [ce_a (p - [v = y]) + l1_a p (sign(p - q) - S)].
  __device__ __forceinline__ void grad_work(int cs, int h, const SD& cur, const float (&zh)[2][8]) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int col = cs + 32 * h + 8 * g;  // within the range
      // unsupervised rows: G = 0 by select (their p may overflow: lse_z = 0)
      float G[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(zh[rb][i], kLog2e, -lz[rb]));
        float v;
        if (TEACHER) {  // g w p [ce_a + l1_a (sign(p - q) - S)], the sign from the L1 pass
          const uint32_t w = h == 0 ? cur.sg.x : cur.sg.y;
          const int sg = static_cast<int>(w << (30 - 2 * (8 * rb + i))) >> 30;
          v = p * __builtin_fmaf(cl1[rb], static_cast<float>(sg), c0[rb]);
        } else {
          v = p * cc[rb];
        }
        G[i] = sup[rb] ? v : 0.f;
      }
      // cc = 0 on unsupervised rows: G_y -= g w ce_a leaves their zeros
      const int ti = target_in(yl[rb], col);
      // one lane of the row, once per sweep: a wave-uniform branch, so the
      // other slices pay no per-element select
      if (__builtin_amdgcn_ballot_w64(ti >= 0) != 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) G[i] = i == ti ? G[i] - cc[rb] : G[i];
      }
      u32x4 hv;
#pragma unroll
      for (int j = 0; j < 4; ++j) hv[j] = pack_bf16x2(G[2 * j], G[2 * j + 1]);
      // columns past the range belong to another workgroup: never written
      const uint32_t eo = col < vlen ? eoff[rb] : kFar;
      if (sizeof(GT) == 2) {
        dzv[h][rb] = hv;  // stored in whole lines once both block pairs are done
      } else {
        const __amdgpu_buffer_rsrc_t rds = slice_rsrc(static_cast<GT*>(P.dz), cs);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const u32x4 gv = {__float_as_uint(G[4 * q]), __float_as_uint(G[4 * q + 1]),
                            __float_as_uint(G[4 * q + 2]), __float_as_uint(G[4 * q + 3])};
          __builtin_amdgcn_raw_buffer_store_b128(gv, rds, bo<4>(eo) + 128 * h + 16 * q, 0, 0);
        }
        __builtin_amdgcn_raw_buffer_store_b128(hv, slice_rsrc(P.ghi, cs), bo<2>(eo) + 64 * h, 0,
                                               0);
        if (P.glo) {  // G - hi, rounded: the second K segment of the weight products
          u32x4 lv;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            lv[j] = pack_bf16x2(G[2 * j] - __uint_as_float(hv[j] << 16),
                                G[2 * j + 1] - __uint_as_float(hv[j] & 0xffff0000u));
          __builtin_amdgcn_raw_buffer_store_b128(lv, slice_rsrc(P.glo, cs), bo<2>(eo) + 64 * h, 0,
                                                 0);
        }
      }
    }
  }

  // Store pass on block pair h: z' of the lane's 8 columns as fp32 (zeros on
  // rows the caller marks invalid), in whole 128-byte lines: the lane's two
  // 16-byte chunks go through the inverse row rotation, so each store covers
  // 8 rows x the pair's 32 columns.  A chunk whose columns lie past the range
  // belongs to another workgroup and is not written; rows past R lie past
  // the buffer.
  __device__ __forceinline__ void store_work(int cs, int h, const float (&zh)[2][8]) {
    const __amdgpu_buffer_rsrc_t ro = slice_rsrc(P.zout, cs);
    const int lane = threadIdx.x & 63, r = lane & 7, k = hi ? 1 : 0;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      u32x4 own[2];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) own[q][j] = sup[rb] ? __float_as_uint(zh[rb][4 * q + j]) : 0u;
      u32x4 v[2];
      unfix_pair(own[0], own[1], v[0], v[1]);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int c = p == 0 ? 2 * g + k : 2 * g + 1 - k;  // chunk of the pair's line
        const int row = 16 * rb + 8 * p + r;
        const uint32_t off = cs + 32 * h + 4 * c < vlen
                                 ? static_cast<uint32_t>((row * P.V + 32 * h + 4 * c) * 4)
                                 : kFar;
        __builtin_amdgcn_raw_buffer_store_b128(v[p], ro, off, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void finish() {
    if (MODE != kL1 || !TEACHER) return;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      double a = a_l1[rb], b = a_s[rb];
      a += __shfl_xor(a, 16, kWave);
      a += __shfl_xor(a, 32, kWave);
      b += __shfl_xor(b, 16, kWave);
      b += __shfl_xor(b, 32, kWave);
      const int64_t row = r0 + 16 * rb + cl;
      if (g == rb && rowok[rb]) {
        P.part_l1[blockIdx.y * P.R + row] = a;
        P.part_s[blockIdx.y * P.R + row] = b;
      }
    }
  }
};

// One sweep over this workgroup's 256 rows and vocabulary range; slices
// rotate through the z / T register sets by name (loop unrolled by kLead + 1).
template <int RANK, int MODE, bool TEACHER, typename GT>
__global__ __launch_bounds__(kNT, 1) void bias_sweep_kernel(SweepParams P) {
  using SW = Sweep<RANK, MODE, TEACHER, GT>;
  __shared__ u32x4 ring[kStages * SW::Eng::kStageCh];
  SW sw(P, ring);
  sw.eng.load_e(P.E, sw.r0, P.R);
  const int nsl = sw.nsl;
  if (nsl <= 0) {
    sw.finish();
    return;
  }
  // prologue: W2 of slices 0..2 and z / T of slices 0 .. kLead - 1, drained
  typename SW::SD A, B, C;
  sw.eng.dma(P.W2, sw.col0(0), sw.ve, sw.stage(0));
  sw.load(A, 0);
  sw.eng.dma(P.W2, sw.col0(1), sw.ve, sw.stage(1));
  if (SW::kLead == 2) sw.load(B, kSliceV);
  sw.eng.dma(P.W2, sw.col0(2), sw.ve, sw.stage(2));
  wait_vm<0>();
  int s = 0;
  if (SW::kLead == 2) {
    for (; s + 3 <= nsl; s += 3) {
      sw.step(s, A, C);
      sw.step(s + 1, B, A);
      sw.step(s + 2, C, B);
    }
    if (s < nsl) sw.step(s, A, C);
    if (s + 1 < nsl) sw.step(s + 1, B, A);
  } else {
    for (; s + 2 <= nsl; s += 2) {
      sw.step(s, A, B);
      sw.step(s + 1, B, A);
    }
    if (s < nsl) sw.step(s, A, B);
  }
  wait_vm<0>();  // no LDS-DMA in flight when the workgroup ends
  sw.finish();
}

// Finishing kernels: one wave per row (rows are few, each needs a short
// dot product and a sum over the vocabulary splits).
constexpr int kFinishWaves = 4;

// Per row, over the wave: (sum of the split partials of L1, of S) in fp64
// and, if y >= 0, z'_y = z_y + E_row . W2_y (fp32; lane k takes k, k + 64, ...).
struct RowFinish {
  double l1, S;
  float zy;
};
__device__ __forceinline__ RowFinish row_finish(int64_t r, int64_t R, int64_t y, int64_t V,
                                                int64_t rank, int splits, int has_teacher,
                                                const double* pl1, const double* ps,
                                                const bf16_t* z, const bf16_t* E,
                                                const bf16_t* W2, int lane) {
  double a = 0.0, b = 0.0;
  if (has_teacher)
    for (int k = lane; k < splits; k += kWave) {
      a += pl1[k * R + r];
      b += ps[k * R + r];
    }
  float bias = 0.f;
  if (y >= 0)
    for (int64_t k = lane; k < rank; k += kWave)
      bias = fmaf(bf16_to_f32(E[r * rank + k]), bf16_to_f32(W2[y * rank + k]), bias);
  RowFinish f;
  f.l1 = wave_sum(a);
  f.S = wave_sum(b);
  f.zy = y >= 0 ? bf16_to_f32(z[r * V + y]) + wave_sumf(bias) : 0.f;
  return f;
}

// Per supervised row: L1 and S from the split partials (0 without a
// teacher) and CE = lse_z - z'_y (target id clamped to the vocabulary);
// unsupervised rows: zeros.
__global__ void l1_finish_kernel(int64_t R, int64_t V, int64_t rank, int splits, int has_teacher,
                                 const double* pl1, const double* ps, const bf16_t* z,
                                 const bf16_t* E, const bf16_t* W2, const int32_t* tid,
                                 RowState rs) {
  const int64_t r = blockIdx.x * static_cast<int64_t>(kFinishWaves) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= R) return;
  if (!rs.mask[r]) {
    if (lane == 0) { rs.l1[r] = 0.f; rs.S[r] = 0.f; rs.ce[r] = 0.f; }
    return;
  }
  const int64_t t = tid[r];
  const int64_t y = t < 0 ? 0 : (t >= V ? V - 1 : t);
  const RowFinish f = row_finish(r, R, y, V, rank, splits, has_teacher, pl1, ps, z, E, W2, lane);
  if (lane == 0) {
    rs.l1[r] = static_cast<float>(f.l1);
    rs.S[r] = static_cast<float>(f.S);
    rs.ce[r] = rs.lse_z[r] - f.zy;
  }
}

// Vocabulary shard: per supervised row, this shard's L1 and S (its split
// partials summed), z'_y when the shard owns the target (else 0) and 1 when
// it owns it (else 0), for the caller to sum over the shards; unsupervised
// rows: zeros.
__global__ void l1_shard_kernel(int64_t R, int64_t V, int64_t rank, int splits, int has_teacher,
                                const double* pl1, const double* ps, const bf16_t* z,
                                const bf16_t* E, const bf16_t* W2, const int32_t* tid,
                                RowState rs, double* part) {
  const int64_t r = blockIdx.x * static_cast<int64_t>(kFinishWaves) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= R) return;
  RowFinish f{0.0, 0.0, 0.f};
  bool own = false;
  if (rs.mask[r]) {
    const int64_t t = tid[r];
    own = t >= 0 && t < V;
    f = row_finish(r, R, own ? t : -1, V, rank, splits, has_teacher, pl1, ps, z, E, W2, lane);
  }
  if (lane == 0) {
    part[4 * r] = f.l1;
    part[4 * r + 1] = f.S;
    part[4 * r + 2] = f.zy;
    part[4 * r + 3] = own ? 1.0 : 0.0;
  }
}

template <int MODE, bool TEACHER, typename GT>
hipError_t launch_mode(int64_t rank, const BiasGrid& gr, const SweepParams& P, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(gr.row_tiles), static_cast<uint32_t>(gr.splits), 1);
  switch (rank) {
    case 0: hipLaunchKernelGGL((bias_sweep_kernel<0, MODE, TEACHER, GT>), grid, dim3(kNT), 0, s, P); break;
    case 32: hipLaunchKernelGGL((bias_sweep_kernel<32, MODE, TEACHER, GT>), grid, dim3(kNT), 0, s, P); break;
    case 64: hipLaunchKernelGGL((bias_sweep_kernel<64, MODE, TEACHER, GT>), grid, dim3(kNT), 0, s, P); break;
    case 128: hipLaunchKernelGGL((bias_sweep_kernel<128, MODE, TEACHER, GT>), grid, dim3(kNT), 0, s, P); break;
    case 256: hipLaunchKernelGGL((bias_sweep_kernel<256, MODE, TEACHER, GT>), grid, dim3(kNT), 0, s, P); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

SweepParams base_params(int64_t R, int64_t V, const bf16_t* z, const bf16_t* E, const bf16_t* W2) {
  SweepParams P{};
  P.R = R; P.V = V; P.z = z; P.E = E; P.W2 = W2;
  P.vsplit = bias_grid(R, V).vsplit;
  return P;
}

}  // namespace

bool bias_sweep_ok(int64_t V, int64_t rank) {
  // 32 rows of fp32 T from one buffer resource: byte offsets below 2^31
  return (rank == 0 || rank == 32 || rank == 64 || rank == 128 || rank == 256) && V > 0 &&
         V % 8 == 0 && V < (int64_t{1} << 24);
}

int64_t bias_signs_words(int64_t R, int64_t V) {
  // one word per lane, slice and wave row of every launched row tile
  const int64_t waves = (R + kRowsPerWG - 1) / kRowsPerWG * kWaves;
  return waves * ((V + kSliceV - 1) / kSliceV) * 64;
}

BiasGrid bias_grid(int64_t R, int64_t V) {
  // Vocabulary ranges of whole 64-column slices, at least 8 of them.  A CU
  // runs one workgroup at a time (the W2 ring fills its LDS), so the
  // workgroups come in rounds of 256: among 1 .. 7 rounds per CU, the fewest
  // whose last round is within 2 % as full as the best.  Fewer, longer
  // workgroups pay the pipeline fill and drain less often (measured: 14 %
  // less sweep time at 1792 rows, 1 % at 14336 rows than 7 rounds).
  constexpr int64_t kCUs = 256;
  BiasGrid gr;
  gr.row_tiles = (R + kRowsPerWG - 1) / kRowsPerWG;
  const int64_t rt = gr.row_tiles > 0 ? gr.row_tiles : 1;  // callers launch nothing for R <= 0
  const int64_t slices = V > 0 ? (V + kSliceV - 1) / kSliceV : 1;
  const int64_t maxsp = slices / 8 > 1 ? slices / 8 : 1;
  int64_t per_n[8] = {}, splits_n[8] = {};
  double fill_n[8] = {}, best = 0.0;
  for (int64_t n = 1; n <= 7; ++n) {
    int64_t sp = n * kCUs / rt;
    if (sp > maxsp) sp = maxsp;
    if (sp < 1) sp = 1;
    per_n[n] = (slices + sp - 1) / sp;
    splits_n[n] = (slices + per_n[n] - 1) / per_n[n];
    const int64_t wg = rt * splits_n[n];
    fill_n[n] = static_cast<double>(wg) / static_cast<double>((wg + kCUs - 1) / kCUs * kCUs);
    if (fill_n[n] > best) best = fill_n[n];
  }
  int64_t n = 1;
  while (n < 7 && fill_n[n] < best - 0.02) ++n;
  gr.vsplit = per_n[n] * kSliceV;
  gr.splits = V > 0 ? (V + gr.vsplit - 1) / gr.vsplit : 0;
  return gr;
}

hipError_t launch_bias_stats(int64_t R, int64_t V, int64_t rank, const bf16_t* z, const bf16_t* E,
                             const bf16_t* W2, float2* sz, int64_t nstat, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  SweepParams P = base_params(R, V, z, E, W2);
  P.sz = sz;
  P.nstat = nstat;
  return launch_mode<kStats, false, bf16_t>(rank, bias_grid(R, V), P, s);
}

hipError_t launch_bias_l1(int64_t R, int64_t V, int64_t rank, const bf16_t* z, const bf16_t* E,
                          const bf16_t* W2, const float* T, const int32_t* tid, RowState rs,
                          double* part_l1, double* part_s, uint2* signs, hipStream_t s) {
  if (R <= 0 || T == nullptr) return hipSuccess;
  SweepParams P = base_params(R, V, z, E, W2);
  P.T = T; P.tid = tid; P.rs = rs; P.part_l1 = part_l1; P.part_s = part_s;
  P.signs = reinterpret_cast<u32x2*>(signs);
  P.nstat = (V + kSliceV - 1) / kSliceV;
  return launch_mode<kL1, true, bf16_t>(rank, bias_grid(R, V), P, s);
}

hipError_t launch_bias_l1_finish(int64_t R, int64_t V, int64_t rank, int splits, int has_teacher,
                                 const double* part_l1, const double* part_s, const bf16_t* z,
                                 const bf16_t* E, const bf16_t* W2, const int32_t* tid,
                                 RowState rs, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(l1_finish_kernel,
                     dim3(static_cast<uint32_t>((R + kFinishWaves - 1) / kFinishWaves)),
                     dim3(kFinishWaves * kWave), 0,
                     s, R, V, rank, splits, has_teacher, part_l1, part_s, z, E, W2, tid, rs);
  return hipGetLastError();
}

hipError_t launch_bias_l1_shard(int64_t R, int64_t V, int64_t rank, int splits, int has_teacher,
                                const double* part_l1, const double* part_s, const bf16_t* z,
                                const bf16_t* E, const bf16_t* W2, const int32_t* tid,
                                RowState rs, double* part, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(l1_shard_kernel,
                     dim3(static_cast<uint32_t>((R + kFinishWaves - 1) / kFinishWaves)),
                     dim3(kFinishWaves * kWave), 0,
                     s, R, V, rank, splits, has_teacher, part_l1, part_s, z, E, W2, tid, rs, part);
  return hipGetLastError();
}

hipError_t launch_bias_store(int64_t R, int64_t V, int64_t rank, const bf16_t* z,
                             const bf16_t* E, const bf16_t* W2, const uint8_t* valid, float* out,
                             hipStream_t s) {
  if (R <= 0) return hipSuccess;
  SweepParams P = base_params(R, V, z, E, W2);
  P.zout = out;
  P.valid = valid;
  return launch_mode<kStore, false, float>(rank, bias_grid(R, V), P, s);
}

hipError_t launch_bias_grad(int grad_dtype, int64_t R, int64_t V, int64_t rank, const bf16_t* z,
                            const bf16_t* E, const bf16_t* W2, const uint2* signs,
                            const int32_t* tid, RowState rs, int has_teacher, float g, float ce_a,
                            float l1_a, void* dz, bf16_t* ghi, bf16_t* glo, hipStream_t s,
                            int shard) {
  if (R <= 0) return hipSuccess;
  SweepParams P = base_params(R, V, z, E, W2);
  P.shard = shard;
  P.tid = tid; P.rs = rs; P.dz = dz; P.ghi = ghi; P.glo = glo;
  P.signs = reinterpret_cast<u32x2*>(const_cast<uint2*>(signs));
  P.nstat = (V + kSliceV - 1) / kSliceV;
  P.g = g; P.ce_a = ce_a; P.l1_a = l1_a;
  const BiasGrid gr = bias_grid(R, V);
  if (grad_dtype == 1 && (ghi || glo)) return hipErrorInvalidValue;  // bf16 dz is G itself
  if (grad_dtype == 1)
    return has_teacher ? launch_mode<kGrad, true, bf16_t>(rank, gr, P, s)
                       : launch_mode<kGrad, false, bf16_t>(rank, gr, P, s);
  return has_teacher ? launch_mode<kGrad, true, float>(rank, gr, P, s)
                     : launch_mode<kGrad, false, float>(rank, gr, P, s);
}

}  // namespace dspark
