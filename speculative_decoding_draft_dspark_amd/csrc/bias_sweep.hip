// Vocabulary sweeps that recompute the Markov bias of the corrected draft
// logits z' = z + E . W2^T (NeMo-RL "DSpark Auxiliary Heads", Inputs and
// Outputs) tile by tile, so z' is never written to memory: the softmax
// statistics of z' (the first pass of the loss), the L1 / S / CE pass and the
// gradient pass (TorchSpec pull request #132, loss section: the fp32 log-softmax,
// the probability L1 and its gradient) each read z (bf16) and rebuild z'.
//
// Work split: a workgroup of 8 waves owns 128 rows and one range of the
// vocabulary; each wave owns 16 rows.  The wave keeps its rows of E as MFMA
// fragments in registers for the whole sweep; W2 streams through LDS in
// slices of 64 vocabulary rows (register-staged, double-buffered, one barrier
// per slice) and is shared by the 8 waves.  Per slice and wave the bias is 4
// blocks of 16 x 16 from v_mfma_f32_16x16x32_bf16 over the rank, with the W2
// fragment as the first operand: lane (g, cl) holds row cl of the wave at the
// 4 consecutive columns 16 b + 4 g .. + 3 of block b, so z (bf16) and T (fp32)
// are read as 8- and 16-byte vectors at exactly the lane's positions.  Every
// sweep computes the bias with the same instruction sequence, so all three see
// the same z'.
#include "bias_sweep.h"

#include "common.h"

namespace dspark {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// Buffer resource over `bytes` from base (untyped dword loads); offsets at or
// past the end read as zero, so every load is issued unconditionally and the
// compiler's wait counts stay exact.
constexpr uint32_t kOOB = 0xffffffffu;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

constexpr int kWaves = 8, kNT = kWaves * 64;
constexpr int kRowsPerWave = 16, kRowsPerWG = kWaves * kRowsPerWave;  // 128
constexpr int kSliceV = 64;  // vocabulary rows of W2 per slice (4 MFMA blocks of 16)

enum SweepMode { kStats = 0, kL1 = 1, kGrad = 2 };

__device__ __forceinline__ void lds_sync() {
  // order LDS accesses only (no wait on outstanding global loads or stores)
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
  __builtin_amdgcn_s_barrier();
}


typedef __attribute__((address_space(3))) void lds_void;

constexpr int kStages = 4;  // W2 slices in LDS: the one in use and three in flight

// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt <= n only.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// The bias of one wave's 16 rows over vocabulary slices: E fragments in
// registers, W2 slices in a 4-stage LDS ring filled by LDS-DMA three slices
// ahead (rank RANK, a multiple of 32).
template <int RANK>
struct BiasEngine {
  static constexpr int KS = RANK > 0 ? RANK / 32 : 1;            // MFMA k steps over the rank
  static constexpr int CPR = RANK > 0 ? RANK / 8 : 1;             // 16-byte chunks per W2 row
  static constexpr int SWM = (CPR < 16 ? CPR : 16) - 1;           // chunk XOR against bank conflicts
  static constexpr int kChunks = RANK > 0 ? kSliceV * CPR : 0;    // chunks per slice
  static constexpr int kPer = kChunks > kNT ? kChunks / kNT : 1;  // DMA loads per thread per slice
  static constexpr int kStageCh = kPer * kNT;                     // u32x4 per ring stage

  u32x4 e[KS];

  __device__ static int slot(int v, int c) { return v * CPR + (c ^ (v & SWM)); }

  // E fragments: lane (g, cl) holds row cl of the wave at rank 32 ks + 8 g .. + 7.
  __device__ void load_e(const bf16_t* E, int64_t row, int64_t R) {
    const int lane = threadIdx.x & 63, g = lane >> 4;
    const int64_t rr = row < R ? row : R - 1;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (RANK == 0) { e[ks] = u32x4{0u, 0u, 0u, 0u}; continue; }
      const u32x4 v = *reinterpret_cast<const u32x4*>(E + rr * RANK + 32 * ks + 8 * g);
      e[ks] = row < R ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // Queue W2 rows [v0, v0 + 64) into a ring stage (rows past vend read zero):
  // the wave's p-th load fills chunks [(wave kPer + p) 64, + 64) of the stage,
  // lane l the one at + l, i.e. row idx / CPR, slot idx % CPR, which holds
  // chunk slot ^ (row & SWM).  kPer loads per thread, always issued.
  __device__ void dma(const bf16_t* W2, int64_t v0, int64_t vend, u32x4* stage) const {
    if (RANK == 0) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const __amdgpu_buffer_rsrc_t rs =
        rsrc_of(W2 + (v0 < vend ? v0 : 0) * RANK, kSliceV * RANK * 2);
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int idx = (wave * kPer + p) * 64 + lane;
      const int v = idx / CPR, c = (idx % CPR) ^ (v & SWM);
      const uint32_t off = (idx < kChunks && v0 + v < vend)
                               ? static_cast<uint32_t>((v * RANK + 8 * c) * 2)
                               : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(stage + (wave * kPer + p) * 64), 16,
                                               off, 0, 0, 0);
    }
  }
  // Bias blocks b0 and b0 + 1 of the slice in buf (block b: 16 vocabulary
  // rows); lane (g, cl) gets row cl, columns 16 b + 4 g .. + 3.  Two
  // independent MFMA chains, with the next k step's W2 fragments read while
  // the current step's MFMAs run.
  __device__ void bias2(const u32x4* buf, int b0, f32x4_v (&acc)[2]) const {
    acc[0] = acc[1] = f32x4_v{0.f, 0.f, 0.f, 0.f};
    if (RANK == 0) return;
    const int lane = threadIdx.x & 63, g = lane >> 4, cl = lane & 15;
    u32x4 w[KS][2];  // fully unrolled: registers, read one k step ahead of their MFMAs
#pragma unroll
    for (int b = 0; b < 2; ++b) w[0][b] = buf[slot(16 * (b0 + b) + cl, g)];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) {
#pragma unroll
        for (int b = 0; b < 2; ++b) w[ks + 1][b] = buf[slot(16 * (b0 + b) + cl, 4 * (ks + 1) + g)];
      }
#pragma unroll
      for (int b = 0; b < 2; ++b)
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, w[ks][b]),
                                                         __builtin_bit_cast(bf16x8_v, e[ks]), acc[b],
                                                         0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads at most one k step ahead
    }
  }
};

// The lane's z (bf16) and T (fp32) of one slice: 4 blocks x 4 consecutive columns.
struct SliceData {
  uint2 z[4];
  float4 t[4];
};

// The lane's z and T of one slice through buffer resources based at the
// wave's first row (16 rows: offsets below 2^32 bytes); rows and columns out
// of range read zeros.
template <bool TEACHER>
__device__ __forceinline__ void load_slice(SliceData& d, const __amdgpu_buffer_rsrc_t& rz,
                                           const __amdgpu_buffer_rsrc_t& rt, bool rowok,
                                           uint32_t ebase, int vlen, int cl0) {
  const int lane = threadIdx.x & 63, g = lane >> 4;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int col = cl0 + 16 * b + 4 * g;  // within the range; V % 4 == 0: all 4 in or all out
    const bool ok = rowok && col < vlen;
    const uint32_t e = ebase + static_cast<uint32_t>(col);
    const u32x2 zz = __builtin_amdgcn_raw_buffer_load_b64(rz, ok ? e * 2 : kOOB, 0, 0);
    d.z[b] = make_uint2(zz.x, zz.y);
    if (TEACHER) {
      const u32x4 tt = __builtin_amdgcn_raw_buffer_load_b128(rt, ok ? e * 4 : kOOB, 0, 0);
      d.t[b] = make_float4(__uint_as_float(tt.x), __uint_as_float(tt.y), __uint_as_float(tt.z),
                           __uint_as_float(tt.w));
    }
  }
}

__device__ __forceinline__ float4 zprime(const uint2& zz, const f32x4_v& bias) {
  return make_float4(__uint_as_float(zz.x << 16) + bias[0],
                     __uint_as_float(zz.x & 0xffff0000u) + bias[1],
                     __uint_as_float(zz.y << 16) + bias[2],
                     __uint_as_float(zz.y & 0xffff0000u) + bias[3]);
}

__device__ __forceinline__ float f4(const float4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
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
  float* zy;
  void* dz;
  bf16_t* ghi;
  bf16_t* glo;
  float g, ce_a, l1_a;
};

// One sweep over this workgroup's 128 rows and vocabulary range.
// State of one sweep over a workgroup's 128 rows and vocabulary range.
template <int RANK, int MODE, bool TEACHER, typename GT>
struct Sweep {
  using Eng = BiasEngine<RANK>;
  static constexpr int kZT = TEACHER ? 8 : 4;  // z / T loads per lane per slice
  // slices of z / T in flight ahead of the one in use: 2 without T, 1 with T
  // (three register sets of z and T would not fit two waves per SIMD)
  static constexpr int kLead = TEACHER ? 1 : 2;
  const SweepParams& P;
  u32x4* ring;  // kStages x Eng::kStageCh
  Eng eng;
  int64_t row, vb;
  int nsl;
  int g;
  bool rowok, sup;
  float lz, lt, Sr, cc, cl1;
  int64_t y;
  __amdgpu_buffer_rsrc_t rz, rt;      // z and T from the wave's first row
  __amdgpu_buffer_rsrc_t rd, rh, rl;  // dz, G hi, G lo from the wave's first row
  int64_t ve, r0;
  int vlen;        // columns in this workgroup's range
  int yl;          // target column within the range, -1 if outside
  uint32_t ebase;  // element offset of (this lane's row, column vb) from the wave's row 0
  float4 tile[4][4];   // statistics: the 4 slices of a 256-column tile
  double a_l1, a_s;    // L1 pass accumulators
  float zyv;
  bool has_y;

  __device__ Sweep(const SweepParams& p, u32x4* rg) : P(p), ring(rg) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    g = lane >> 4;
    row = static_cast<int64_t>(blockIdx.x) * kRowsPerWG + wave * kRowsPerWave + (lane & 15);
    vb = static_cast<int64_t>(blockIdx.y) * P.vsplit;
    ve = (vb + P.vsplit) < P.V ? (vb + P.vsplit) : P.V;
    nsl = vb < ve ? static_cast<int>((ve - vb + kSliceV - 1) / kSliceV) : 0;
    rowok = row < P.R;
    sup = MODE != kStats && rowok && P.rs.mask[row] != 0;
    r0 = row - (lane & 15);
    const uint32_t span = static_cast<uint32_t>(kRowsPerWave * P.V);  // elements
    rz = rsrc_of(P.z + r0 * P.V, span * 2);
    rt = rsrc_of(TEACHER ? P.T + r0 * P.V : P.T, TEACHER ? span * 4 : 0);
    if (MODE == kGrad) {
      rd = rsrc_of(static_cast<char*>(P.dz) + r0 * P.V * sizeof(GT), span * sizeof(GT));
      rh = rsrc_of(P.ghi ? P.ghi + r0 * P.V : P.ghi, P.ghi ? span * 2 : 0);
      rl = rsrc_of(P.glo ? P.glo + r0 * P.V : P.glo, P.glo ? span * 2 : 0);
    }
    lz = lt = Sr = cc = cl1 = 0.f;
    y = -1;
    if (MODE != kStats && sup) {
      lz = P.rs.lse_z[row];
      lt = P.rs.lse_t[row];
      if (MODE == kGrad) {
        const float gw = P.g * P.rs.w[row];
        cc = gw * P.ce_a;
        cl1 = gw * P.l1_a;
        Sr = P.rs.S[row];
      }
      const int64_t t = P.tid[row];
      y = t < 0 ? 0 : (t >= P.V ? P.V - 1 : t);
    }
    vlen = static_cast<int>(ve > vb ? ve - vb : 0);
    yl = (y >= vb && y < ve) ? static_cast<int>(y - vb) : -1;
    ebase = static_cast<uint32_t>((lane & 15) * P.V + vb);
    a_l1 = a_s = 0.0;
    zyv = 0.f;
    has_y = false;
  }

  __device__ int64_t col0(int s) const { return vb + static_cast<int64_t>(s) * kSliceV; }

  __device__ u32x4* stage(int t) const { return ring + (t % kStages) * Eng::kStageCh; }

  // Slice s, whose z / T are in `cur`; queues W2 of slice s + 3 into the ring
  // (the stage slice s - 1 used) and z / T of slice s + kLead into `nxt` (the
  // buffer of slice s - 1, already consumed), so no register copies put a
  // wait on loads still in flight.  Loads of slices past the range read zeros
  // and are always issued, and the per-element conditions are selects, so
  // every wait count is static.
  __device__ void step(int s, const SliceData& cur, SliceData& nxt) {
    // W2 of slice s landed: it was queued three steps ago (the prologue
    // drains its own), and the loads of two later steps (DMA and z / T each)
    // were issued after it
    wait_vm<2 * (Eng::kPer + kZT)>();
    lds_sync();  // every wave's W2 slice s is in LDS; slice s - 1's stage is free
    eng.dma(P.W2, col0(s + 3), ve, stage(s + 3));
    load_slice<TEACHER>(nxt, rz, rt, rowok, ebase, vlen, (s + kLead) * kSliceV);
    const int64_t c0 = col0(s);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      f32x4_v bias2[2];
      eng.bias2(stage(s), 2 * hb, bias2);
      work(s, c0, cur, hb, bias2);
    }
  }

  // The mode's work on blocks 2 hb, 2 hb + 1 of slice s.
  __device__ void work(int s, int64_t c0, const SliceData& cur, int hb, const f32x4_v (&bias2)[2]) {
    if (MODE == kStats) {
      const int j = s & 3;  // slice within the 256-column tile (vsplit % 256 == 0)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const int b = 2 * hb + bb;
        const float4 zp = zprime(cur.z[b], bias2[bb]);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (jj == j) tile[jj][b] = zp;
      }
      if (hb == 1 && (j == 3 || s == nsl - 1)) finish_tile(s, j);
    } else if (MODE == kL1) {
      float s1 = 0.f, s2 = 0.f;
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const int b = 2 * hb + bb;
        const float4 zp = zprime(cur.z[b], bias2[bb]);
        const int col = s * kSliceV + 16 * b + 4 * g;  // within the range
        const bool ok = sup && col < vlen;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (TEACHER) {
            const float p = dexp(f4(zp, i) - lz), q = dexp(f4(cur.t[b], i) - lt);
            s1 += ok ? fabsf(p - q) : 0.f;
            s2 += ok ? p * sgnf(p - q) : 0.f;
          }
          const bool hit = ok && col + i == yl;
          zyv = hit ? f4(zp, i) : zyv;
          has_y = has_y || hit;
        }
      }
      a_l1 += s1;
      a_s += s2;
    } else {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const int b = 2 * hb + bb;
        const float4 zp = zprime(cur.z[b], bias2[bb]);
        const int col = s * kSliceV + 16 * b + 4 * g;  // within the range
        float G[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = dexp(f4(zp, i) - lz);
          float v;
          if (TEACHER) {
            const float q = dexp(f4(cur.t[b], i) - lt);
            v = p * (cc + cl1 * (sgnf(p - q) - Sr));
          } else {
            v = p * cc;
          }
          v = col + i == yl ? v - cc : v;
          G[i] = sup ? v : 0.f;
        }
        uint32_t h[4], l[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h[i] = f32_to_bf16(G[i]);
          l[i] = f32_to_bf16(G[i] - bf16_to_f32(static_cast<bf16_t>(h[i])));
        }
        const u32x2 hv = {h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        const u32x2 lv = {l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
        const bool ok = rowok && col < vlen;
        const uint32_t e = ebase + static_cast<uint32_t>(col);
        if (sizeof(GT) == 2) {
          __builtin_amdgcn_raw_buffer_store_b64(hv, rd, ok ? e * 2 : kOOB, 0, 0);
        } else {
          const u32x4 gv = {__float_as_uint(G[0]), __float_as_uint(G[1]), __float_as_uint(G[2]),
                            __float_as_uint(G[3])};
          __builtin_amdgcn_raw_buffer_store_b128(gv, rd, ok ? e * 4 : kOOB, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b64(hv, rh, ok ? e * 2 : kOOB, 0, 0);
        }
        if (P.glo) __builtin_amdgcn_raw_buffer_store_b64(lv, rl, ok ? e * 2 : kOOB, 0, 0);
      }
    }
  }

  // Statistics of the 256-column tile whose slice j (0..3) is slice s:
  // maximum, then fixed-point exp-sum, over the row's 4 lanes.
  __device__ void finish_tile(int s, int j) {
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int col = (s - j + jj) * kSliceV + 16 * b + 4 * g;  // within the range
        const float4 v = tile[jj][b];
        const float m4 = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
        mx = (jj <= j && col < vlen) ? fmaxf(mx, m4) : mx;
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    uint64_t sum = 0;
    if (mx != -INFINITY) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int col = (s - j + jj) * kSliceV + 16 * b + 4 * g;
          const float4 v = tile[jj][b];
          const uint32_t a = fix_exp32(v.x, mx), c = fix_exp32(v.y, mx);
          const uint32_t d = fix_exp32(v.z, mx), f = fix_exp32(v.w, mx);
          const uint64_t t4 = static_cast<uint64_t>(a) + c + static_cast<uint64_t>(d) + f;
          sum += (jj <= j && col < vlen) ? t4 : 0ull;
        }
    }
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
      const uint32_t lo = __shfl_xor(static_cast<uint32_t>(sum), o, kWave);
      const uint32_t hi = __shfl_xor(static_cast<uint32_t>(sum >> 32), o, kWave);
      sum += (static_cast<uint64_t>(hi) << 32) | lo;
    }
    if (g == 0 && rowok) {
      const int64_t tn = vb / 256 + (s - j) / 4;
      const float l = static_cast<float>(static_cast<double>(sum) * (1.0 / 2147483648.0));
      P.sz[row * P.nstat + tn] = make_float2(mx, l);
    }
  }

  __device__ void finish() {
    if (MODE != kL1) return;
    a_l1 += __shfl_xor(a_l1, 16, kWave);
    a_l1 += __shfl_xor(a_l1, 32, kWave);
    a_s += __shfl_xor(a_s, 16, kWave);
    a_s += __shfl_xor(a_s, 32, kWave);
    if (g == 0 && rowok) {
      P.part_l1[blockIdx.y * P.R + row] = a_l1;
      P.part_s[blockIdx.y * P.R + row] = a_s;
    }
    if (has_y) P.zy[row] = zyv;
  }
};

// One sweep over this workgroup's 128 rows and vocabulary range; slices
// rotate through three z / T register sets by name (loop unrolled by 3).
template <int RANK, int MODE, bool TEACHER, typename GT>
__global__ __launch_bounds__(kNT, 1) void bias_sweep_kernel(SweepParams P) {
  using SW = Sweep<RANK, MODE, TEACHER, GT>;
  __shared__ u32x4 ring[kStages * SW::Eng::kStageCh];
  SW sw(P, ring);
  sw.eng.load_e(P.E, sw.row, P.R);
  const int nsl = sw.nsl;
  if (nsl <= 0) {
    sw.finish();
    return;
  }
  // prologue: W2 of slices 0..2 and z / T of slices 0 .. kLead - 1, drained
  SliceData A, B, C;
  sw.eng.dma(P.W2, sw.col0(0), sw.ve, sw.stage(0));
  load_slice<TEACHER>(A, sw.rz, sw.rt, sw.rowok, sw.ebase, sw.vlen, 0);
  sw.eng.dma(P.W2, sw.col0(1), sw.ve, sw.stage(1));
  if (SW::kLead == 2) load_slice<TEACHER>(B, sw.rz, sw.rt, sw.rowok, sw.ebase, sw.vlen, kSliceV);
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

__global__ void l1_finish_kernel(int64_t R, int splits, const double* pl1, const double* ps,
                                 const float* zy, RowState rs) {
  const int64_t r = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (r >= R) return;
  if (!rs.mask[r]) {
    rs.l1[r] = 0.f; rs.S[r] = 0.f; rs.ce[r] = 0.f;
    return;
  }
  double a = 0.0, b = 0.0;
  for (int k = 0; k < splits; ++k) {
    a += pl1[k * R + r];
    b += ps[k * R + r];
  }
  rs.l1[r] = static_cast<float>(a);
  rs.S[r] = static_cast<float>(b);
  rs.ce[r] = rs.lse_z[r] - zy[r];
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

bool bias_sweep_rank_ok(int64_t rank) {
  return rank == 0 || rank == 32 || rank == 64 || rank == 128 || rank == 256;
}

BiasGrid bias_grid(int64_t R, int64_t V) {
  // about 7 waves of workgroups over the 256 CUs, each range a multiple of 256
  // columns and at least 8 of them
  BiasGrid gr;
  gr.row_tiles = (R + kRowsPerWG - 1) / kRowsPerWG;
  const int64_t tiles = (V + 255) / 256;
  int64_t sp = (1792 + gr.row_tiles - 1) / gr.row_tiles;
  if (sp > tiles / 8) sp = tiles / 8;
  if (sp < 1) sp = 1;
  const int64_t per = (tiles + sp - 1) / sp;
  gr.vsplit = per * 256;
  gr.splits = (V + gr.vsplit - 1) / gr.vsplit;
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
                          double* part_l1, double* part_s, float* zy, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  SweepParams P = base_params(R, V, z, E, W2);
  P.T = T; P.tid = tid; P.rs = rs; P.part_l1 = part_l1; P.part_s = part_s; P.zy = zy;
  return T ? launch_mode<kL1, true, bf16_t>(rank, bias_grid(R, V), P, s)
           : launch_mode<kL1, false, bf16_t>(rank, bias_grid(R, V), P, s);
}

hipError_t launch_bias_l1_finish(int64_t R, int64_t V, int splits, const double* part_l1,
                                 const double* part_s, const float* zy, RowState rs,
                                 hipStream_t s) {
  (void)V;
  if (R <= 0) return hipSuccess;
  hipLaunchKernelGGL(l1_finish_kernel, dim3(static_cast<uint32_t>((R + 255) / 256)), dim3(256), 0,
                     s, R, splits, part_l1, part_s, zy, rs);
  return hipGetLastError();
}

hipError_t launch_bias_grad(int grad_dtype, int64_t R, int64_t V, int64_t rank, const bf16_t* z,
                            const bf16_t* E, const bf16_t* W2, const float* T, const int32_t* tid,
                            RowState rs, int has_teacher, float g, float ce_a, float l1_a, void* dz,
                            bf16_t* ghi, bf16_t* glo, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  SweepParams P = base_params(R, V, z, E, W2);
  P.T = T; P.tid = tid; P.rs = rs; P.dz = dz; P.ghi = ghi; P.glo = glo;
  P.g = g; P.ce_a = ce_a; P.l1_a = l1_a;
  const BiasGrid gr = bias_grid(R, V);
  if (grad_dtype == 1)
    return has_teacher ? launch_mode<kGrad, true, bf16_t>(rank, gr, P, s)
                       : launch_mode<kGrad, false, bf16_t>(rank, gr, P, s);
  return has_teacher ? launch_mode<kGrad, true, float>(rank, gr, P, s)
                     : launch_mode<kGrad, false, float>(rank, gr, P, s);
}

}  // namespace dspark
