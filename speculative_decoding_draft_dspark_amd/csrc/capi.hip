// C ABI of the DSpark loss library: host-side validation, workspace layout and
// the launch sequences of the forward, backward and acceptance report.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/dspark.h"
#include "common.h"
#include "internal.h"
#include "bias_sweep.h"
#include "rowwise.h"

namespace dspark {
namespace {

thread_local char g_hip_err[256] = "";

constexpr size_t kAlign = 256;
inline size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Dims {
  int64_t B, N, K, R, Vd, Vt, H, Hd, r, nstat, splits, conf_chunks, F;
  int64_t R32;  // R rounded up to a multiple of 32 (k-blocked row operands)
  int64_t dw2_splits;  // K splits of the in-place dW2 product: 1, or 2 (hi and lo, or row halves)
  int dtype, gdtype, esize;
  bool markov, conf, conf_markov;
  // bf16 backward products read G, W2 and E in place (row counts and the
  // vocabulary multiples of 32); otherwise through transposed / k-blocked copies
  bool direct_bwd;
  // The Markov weight products take G as bf16 hi + bf16 lo (two K segments).
  // Not with bf16 draft-logit gradients on the in-place backward: there the
  // products take the bf16 dz itself, as a bf16 autograd does (their error is
  // then that of dz's own rounding, about 2^-10 normwise).
  bool g_lo;
  // bf16 corrected draft logits never stored: every vocabulary sweep rebuilds
  // z' = z + E W2^T (ranks the bias sweeps support, with the in-place backward)
  bool bias_path;
  int64_t bsplits;  // vocabulary splits of the bias sweeps
  bool det;         // dW1 as fixed-point integer sums (order-independent)
};

struct Layout {
  size_t Zp, T, sz, st, E, mask, rowf, ghi, glo, g32, dEpart, dE, confpart;
  size_t pl1, ps;  // bias path: L1 / S split partials
  size_t sg;       // bias path: sign bits of p - q (L1 pass -> gradient pass)
  size_t w2t, eblk, blkhi, blklo, dw2part;  // bf16 backward operands
  size_t dw1acc, dw1max;  // deterministic dW1: fixed-point sums, the term maximum
  size_t total;
};

constexpr int kRowArrays = 10;  // float row arrays of RowState (w .. dcoef)
constexpr int64_t kCUs = 256;   // compute units of an MI355X (sizes the dE split count)

int make_dims(const dspark_shape* sh, Dims* d) {
  if (!sh) return DSPARK_ERR_NULL;
  if (sh->dtype != DSPARK_F32 && sh->dtype != DSPARK_BF16) return DSPARK_ERR_DTYPE;
  if (sh->grad_dtype != DSPARK_F32 && sh->grad_dtype != DSPARK_BF16) return DSPARK_ERR_DTYPE;
  if (sh->batch <= 0 || sh->num_blocks <= 0 || sh->block_size <= 0) return DSPARK_ERR_SHAPE;
  if (sh->draft_vocab <= 0 || sh->draft_vocab % 8) return DSPARK_ERR_SHAPE;
  if (sh->markov_rank < 0 || sh->markov_rank % 8) return DSPARK_ERR_SHAPE;
  if (sh->hidden < 0 || sh->hidden % 8) return DSPARK_ERR_SHAPE;
  if (sh->conf_hidden < 0) return DSPARK_ERR_SHAPE;
  if (sh->options & ~static_cast<int32_t>(DSPARK_OPT_STORE_DRAFT_LOGITS | DSPARK_OPT_DETERMINISTIC))
    return DSPARK_ERR_SHAPE;
  if (sh->markov_rank > 0 && sh->target_vocab <= 0) return DSPARK_ERR_SHAPE;
  if (sh->draft_vocab > (int64_t{1} << 26) || sh->hidden > (int64_t{1} << 20) ||
      sh->markov_rank > 4096)
    return DSPARK_ERR_SHAPE;  // keeps every tile's byte offsets below 2^31
  d->B = sh->batch; d->N = sh->num_blocks; d->K = sh->block_size;
  d->R = d->B * d->N * d->K;
  if (d->R > (int64_t{1} << 31) - 1) return DSPARK_ERR_SHAPE;
  d->Vd = sh->draft_vocab; d->Vt = sh->target_vocab; d->H = sh->hidden;
  d->Hd = sh->conf_hidden; d->r = sh->markov_rank;
  d->dtype = sh->dtype; d->gdtype = sh->grad_dtype;
  d->esize = d->dtype == DSPARK_BF16 ? 2 : 4;
  d->markov = d->r > 0;
  d->conf = d->Hd > 0;
  d->conf_markov = d->conf && d->markov && sh->with_markov_conf != 0;
  d->nstat = (d->Vd + kStatTile - 1) / kStatTile;
  const int64_t nM = (d->R + 255) / 256;
  int64_t sp = 640 / nM;
  const int64_t kmax = 2 * gemm_kpad(d->Vd, d->esize) / (8 * 64);  // at least 8 K-tiles per split
  if (sp > kmax) sp = kmax;
  if (sp > 32) sp = 32;
  if (sp < 1) sp = 1;
  d->direct_bwd = d->dtype == DSPARK_BF16 && d->markov && d->R % 32 == 0 && d->Vd % 32 == 0;
  d->dw2_splits = 2;
  d->g_lo = d->markov && !(d->direct_bwd && d->gdtype == DSPARK_BF16);
  if (d->direct_bwd) {
    // Split counts of the in-place products: the smallest whose tiles x
    // splits workgroups fill whole waves of the 256 CUs within 2 %, each
    // split at least 8 slices of 32 of its (hi, lo) contraction.
    auto pick = [](int64_t tiles, int64_t slices) {
      int64_t best = 1;
      double best_eff = 0.0;
      for (int64_t ds = 1; ds <= 64 && ds * 8 <= slices; ++ds) {
        const int64_t wg = tiles * ds, waves = (wg + kCUs - 1) / kCUs;
        const double eff = static_cast<double>(wg) / static_cast<double>(waves * kCUs);
        if (eff > best_eff + 0.02) { best = ds; best_eff = eff; }
      }
      return best;
    };
    sp = pick(nM, (d->g_lo ? 2 : 1) * d->Vd / 32);
    // dW2: Vd / 256 tiles of 256 x r.  Two K splits (the hi and lo halves, or
    // two halves of the rows) fill the waves better but add one fp32 Vd x r
    // partial to write and sum; that pays once each half is at least 2048
    // long (14336 rows: 1.12 ms against 1.17 ms with one; 1792 rows: 0.25 ms
    // with one against 0.29 ms with two; three or four splits were slower).
    const int64_t dw2_k = (d->g_lo ? 2 : 1) * d->R;
    d->dw2_splits = dw2_k >= 4096 ? 2 : 1;
  }
  d->splits = d->markov ? sp : 0;
  // Sweeps that rebuild z' from z instead of reading a stored fp32 z': always
  // without a Markov head (z' = z); with one unless the caller asks for the
  // stored logits (the bias is recomputed in each of the three sweeps, which
  // measures faster than writing and twice reading the R x Vd fp32 buffer).
  d->bias_path = d->dtype == DSPARK_BF16 && bias_sweep_ok(d->Vd, d->r) &&
                 (!d->markov ||
                  (d->direct_bwd && (sh->options & DSPARK_OPT_STORE_DRAFT_LOGITS) == 0));
  d->bsplits = d->bias_path ? bias_grid(d->R, d->Vd).splits : 0;
  d->det = d->markov && (sh->options & DSPARK_OPT_DETERMINISTIC) != 0;
  d->conf_chunks = d->R < 256 ? static_cast<int>(d->R) : 256;
  d->F = d->Hd + (d->conf_markov ? d->r : 0);
  d->R32 = (d->R + 31) / 32 * 32;
  return DSPARK_OK;
}

Layout make_layout(const Dims& d) {
  Layout L{};
  size_t o = 0;
  const size_t RV = static_cast<size_t>(d.R) * d.Vd;
  L.Zp = o;
  if (!d.bias_path) o = up(o + RV * 4);
  L.pl1 = L.ps = L.sg = o;
  if (d.bias_path) {
    L.pl1 = o; o = up(o + static_cast<size_t>(d.bsplits) * d.R * 8);
    L.ps = o; o = up(o + static_cast<size_t>(d.bsplits) * d.R * 8);
    L.sg = o; o = up(o + static_cast<size_t>(bias_signs_words(d.R, d.Vd)) * 8);
  }
  L.T = o; o = up(o + RV * 4);
  L.sz = o; o = up(o + static_cast<size_t>(d.R) * d.nstat * 8);
  L.st = o; o = up(o + static_cast<size_t>(d.R) * d.nstat * 8);
  L.E = o; o = up(o + static_cast<size_t>(d.R) * d.r * d.esize);
  L.mask = o; o = up(o + d.R);
  L.rowf = o; o = up(o + static_cast<size_t>(d.R) * 4 * kRowArrays);
  L.ghi = L.glo = L.g32 = L.w2t = L.eblk = L.blkhi = L.blklo = L.dw2part = 0;
  if (d.dtype == DSPARK_BF16) {
    if (d.gdtype != DSPARK_BF16) { L.ghi = o; o = up(o + RV * 2); }
    if (d.g_lo) { L.glo = o; o = up(o + RV * 2); }
    if (d.markov && d.direct_bwd) {
      if (d.dw2_splits > 1) {  // one split writes dW2 itself
        L.dw2part = o; o = up(o + static_cast<size_t>(d.dw2_splits) * d.Vd * d.r * 4);
      }
    } else if (d.markov) {
      const size_t R32V = static_cast<size_t>(d.R32) * d.Vd;
      L.w2t = o; o = up(o + static_cast<size_t>(d.Vd) * d.r * 2);
      L.eblk = o; o = up(o + static_cast<size_t>(d.R32) * d.r * 2);
      L.blkhi = o; o = up(o + R32V * 2);
      L.blklo = o; o = up(o + R32V * 2);
      L.dw2part = o; o = up(o + static_cast<size_t>(2) * d.Vd * d.r * 4);
    }
  } else if (d.gdtype != DSPARK_F32) {
    L.g32 = o; o = up(o + RV * 4);
  }
  L.dEpart = o; o = up(o + static_cast<size_t>(d.splits) * d.R * d.r * 4);
  L.dE = o; o = up(o + static_cast<size_t>(d.R) * d.r * 4);
  L.confpart = o; o = up(o + static_cast<size_t>(d.conf_chunks) * (d.F + 1) * 4);
  L.dw1acc = L.dw1max = o;
  if (d.det) {
    L.dw1acc = o; o = up(o + static_cast<size_t>(d.Vt) * d.r * 8);
    L.dw1max = o; o = up(o + 4);
  }
  L.total = o;
  return L;
}

RowState row_state(char* ws, const Layout& L, const Dims& d) {
  RowState s;
  float* f = reinterpret_cast<float*>(ws + L.rowf);
  s.mask = reinterpret_cast<uint8_t*>(ws + L.mask);
  s.w = f + 0 * d.R; s.lse_z = f + 1 * d.R; s.lse_t = f + 2 * d.R; s.l1 = f + 3 * d.R;
  s.S = f + 4 * d.R; s.ce = f + 5 * d.R; s.accept = f + 6 * d.R; s.conf = f + 7 * d.R;
  s.bce = f + 8 * d.R; s.dcoef = f + 9 * d.R;
  return s;
}

inline bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return DSPARK_OK;
  std::snprintf(g_hip_err, sizeof(g_hip_err), "%s", hipGetErrorString(e));
  return DSPARK_ERR_HIP;
}

#define DSPARK_TRY(expr)                          \
  do {                                            \
    const hipError_t e_ = (expr);                 \
    if (e_ != hipSuccess) return hip_status(e_);  \
  } while (0)

enum Teacher { kNone = 0, kHidden = 1, kAligned = 2 };

// ---- standalone head ops
// Shape checks shared by the two head ops (the loss's own limits).
int head_dims(int64_t rows, int64_t vocab, int64_t target_vocab, int64_t rank, int32_t dtype) {
  if (dtype != DSPARK_F32 && dtype != DSPARK_BF16) return DSPARK_ERR_DTYPE;
  if (rows < 0 || rows > (int64_t{1} << 31) - 1) return DSPARK_ERR_SHAPE;
  if (vocab < 0 || vocab % 8 || vocab > (int64_t{1} << 26)) return DSPARK_ERR_SHAPE;
  if (rank < 0 || rank % 8 || rank > 4096) return DSPARK_ERR_SHAPE;
  if (rank > 0 && target_vocab <= 0) return DSPARK_ERR_SHAPE;
  return DSPARK_OK;
}
struct HeadLayout {
  size_t E, st, total;
};
HeadLayout head_layout(int64_t rows, int64_t vocab, int64_t rank, int32_t dtype) {
  const size_t esize = dtype == DSPARK_BF16 ? 2 : 4;
  HeadLayout L{};
  size_t o = 0;
  L.E = o; o = up(o + static_cast<size_t>(rows) * rank * esize);
  L.st = o; o = up(o + static_cast<size_t>(rows) * ((vocab + kStatTile - 1) / kStatTile) * 8);
  L.total = o;
  return L;
}

// ---- per-stage timers (tracing aid)
enum Stage {
  kPrep, kGather, kLogitsGemm, kBiasStats, kL1Sweep, kFinalize, kReduce, kGradSweep, kOperandPrep,
  kDeGemm, kDeReduce, kDw1, kDw2Gemm, kConfBwd, kStages
};
const char* const kStageNames[kStages] = {
    "prep_rows", "gather_embed", "logits_gemm", "bias_stats", "l1_sweep",
    "finalize_rows", "reduce_fwd", "grad_sweep", "operand_prep", "dE_gemm", "dE_reduce",
    "dW1_scatter",
    "dW2_gemm", "conf_bwd"};

struct Profiler {
  std::mutex mu;
  std::atomic<bool> on{false};
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending[kStages];
  std::vector<hipEvent_t> pool;
  double ms[kStages] = {};
  int64_t count[kStages] = {};
};
Profiler g_prof;

hipEvent_t take_event() {
  if (!g_prof.pool.empty()) {
    hipEvent_t e = g_prof.pool.back();
    g_prof.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <class F>
hipError_t staged(int id, hipStream_t s, F&& launch) {
  if (!g_prof.on.load(std::memory_order_relaxed)) return launch();
  hipEvent_t a, b;
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    a = take_event();
    b = take_event();
  }
  if (a && hipEventRecord(a, s) != hipSuccess) a = nullptr;
  const hipError_t e = launch();
  if (b && hipEventRecord(b, s) != hipSuccess) b = nullptr;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (a && b) {
    g_prof.pending[id].emplace_back(a, b);
  } else {
    if (a) g_prof.pool.push_back(a);
    if (b) g_prof.pool.push_back(b);
  }
  return e;
}

#define DSPARK_STAGE(id, expr) DSPARK_TRY(staged((id), s, [&] { return (expr); }))

int check_inputs(const Dims& d, const dspark_hparams* hp, const dspark_inputs* in, Teacher* t) {
  if (!hp || !in) return DSPARK_ERR_NULL;
  if (!in->draft_logits || !in->target_ids || !in->eval_mask) return DSPARK_ERR_NULL;
  if (d.markov && (!in->prev_ids || !in->markov_w1 || !in->markov_w2)) return DSPARK_ERR_NULL;
  if (d.conf && (!in->conf_hidden || !in->conf_w || !in->conf_b)) return DSPARK_ERR_NULL;
  if (in->aligned_target_logits) *t = kAligned;
  else if (in->target_hidden && in->lm_head && d.H > 0) *t = kHidden;
  else *t = kNone;
  if (*t == kNone && (hp->l1_alpha != 0.f || d.conf)) return DSPARK_ERR_NO_TARGET;
  const void* ptrs[] = {in->draft_logits, in->target_ids, in->eval_mask, in->block_keep_mask,
                        in->prev_ids, in->markov_w1, in->markov_w2, in->target_hidden,
                        in->lm_head, in->aligned_target_logits, in->conf_hidden, in->conf_w,
                        in->conf_b};
  for (const void* p : ptrs)
    if (p && misaligned(p)) return DSPARK_ERR_ALIGN;
  return DSPARK_OK;
}

// dW1 = scatter of dE over the previous-token ids (zeroed first): fp32
// atomics, or with the deterministic option fixed-point integer sums.
hipError_t dw1_stage(const Dims& d, const Layout& L, char* ws, const int32_t* prev,
                     const uint8_t* mask, const float* dE, float* dW1, hipStream_t s) {
  hipError_t e = launch_fill_u32(dW1, d.Vt * d.r, 0u, s);
  if (e != hipSuccess) return e;
  if (!d.det) return launch_dw1_scatter(d.R, d.r, d.Vt, prev, mask, dE, dW1, s);
  e = launch_fill_u32(ws + L.dw1acc, 2 * d.Vt * d.r, 0u, s);
  if (e != hipSuccess) return e;
  return launch_dw1_scatter_fixed(d.R, d.r, d.Vt, prev, mask, dE,
                                  reinterpret_cast<float*>(ws + L.dw1max),
                                  reinterpret_cast<unsigned long long*>(ws + L.dw1acc), dW1, s);
}

// In-place bf16 backward products (R and Vd multiples of 32).  dE partials =
// [G hi | G lo] . [W2 | W2] (or G . W2) over vocabulary splits.
hipError_t de_parts_direct(const Dims& d, const void* gA, const void* glo, const void* W2,
                           float* dEpart, hipStream_t s) {
  Operand A{}, B{};
  const int gseg = glo ? 2 : 1;
  A.seg[0] = gA; A.seg[1] = glo ? glo : gA;
  A.kseg = d.Vd; A.kpad = d.Vd;
  A.ld = d.Vd; A.layout = LAYOUT_KC; A.nseg = gseg;
  B.seg[0] = B.seg[1] = W2; B.kseg = d.Vd; B.kpad = d.Vd; B.ld = d.r;
  B.layout = LAYOUT_MK; B.nseg = gseg;
  return launch_gemm_w4p(2, d.R, d.r, A, B, static_cast<int>(d.splits), dEpart, d.r, s);
}

// dW2 = [G hi ; G lo]^T . [E ; E] (or G^T . E) over row splits into `part`.
hipError_t dw2_parts_direct(const Dims& d, const void* gA, const void* glo, const void* E,
                            float* part, hipStream_t s) {
  Operand A{}, B{};
  const int gseg = glo ? 2 : 1;
  A.seg[0] = gA; A.seg[1] = glo ? glo : gA;
  A.kseg = d.R; A.kpad = d.R;
  A.ld = d.Vd; A.layout = LAYOUT_MK; A.nseg = gseg;
  B.seg[0] = B.seg[1] = E; B.kseg = d.R; B.kpad = d.R; B.ld = d.r;
  B.layout = LAYOUT_MK; B.nseg = gseg;
  return launch_gemm_w4p(3, d.Vd, d.r, A, B, static_cast<int>(d.dw2_splits), part, d.r, s);
}

// Where the in-place dW2 product writes: one split writes the fp32 gradient
// itself; two write their partials to the workspace, summed into it after.
float* dw2_target(const Dims& d, const Layout& L, char* ws, float* dW2) {
  return d.dw2_splits > 1 ? reinterpret_cast<float*>(ws + L.dw2part) : dW2;
}

// Common checks of the vocabulary-shard entry points: the shape must take the
// bias sweeps (bf16, rank in {0, 32, 64, 128, 256}, R and the shard width
// multiples of 32 with a Markov head) and not ask for stored logits.
int shard_setup(const dspark_shape* shape, const dspark_hparams* hp, const dspark_inputs* in,
                void* ws, size_t wsb, Dims* d, Layout* L, Teacher* t) {
  int st = make_dims(shape, d);
  if (st) return st;
  if (!d->bias_path) return DSPARK_ERR_SHAPE;
  st = check_inputs(*d, hp, in, t);
  if (st) return st;
  if (misaligned(ws)) return DSPARK_ERR_ALIGN;
  *L = make_layout(*d);
  if (!ws || wsb < L->total) return DSPARK_ERR_WORKSPACE;
  return DSPARK_OK;
}

// Argument checks of the confidence-head op (both entry points).
int conf_head_check(int64_t rows, int64_t draft_hidden, int64_t target_vocab, int64_t markov_rank,
                    int32_t with_markov_conf, int32_t dtype, const void* hidden,
                    const int32_t* prev_ids, const void* markov_w1, const void* conf_w,
                    const void* conf_b, const float* out) {
  const bool wm = with_markov_conf != 0 && markov_rank > 0;
  int st = head_dims(rows, 0, target_vocab, wm ? markov_rank : 0, dtype);
  if (st) return st;
  if (draft_hidden < 1 || draft_hidden > (int64_t{1} << 20)) return DSPARK_ERR_SHAPE;
  if (!hidden || !conf_w || !conf_b || !out) return DSPARK_ERR_NULL;
  if (wm && (!prev_ids || !markov_w1)) return DSPARK_ERR_NULL;
  if (misaligned(hidden) || misaligned(out) || misaligned(prev_ids) || misaligned(markov_w1) ||
      misaligned(conf_w))
    return DSPARK_ERR_ALIGN;
  return DSPARK_OK;
}

// The confidence-head launches on a checked call; `workspace` holds the
// gathered embeddings and, when the caller passes no mask, a ones mask.
int conf_head_launch(int64_t rows, int64_t draft_hidden, int64_t target_vocab,
                     int64_t markov_rank, int32_t with_markov_conf, int32_t dtype,
                     const void* hidden, const int32_t* prev_ids, const uint8_t* valid_mask,
                     const void* markov_w1, const void* conf_w, const void* conf_b, float* out,
                     void* workspace, hipStream_t s) {
  const bool wm = with_markov_conf != 0 && markov_rank > 0;
  if (rows == 0) return DSPARK_OK;
  const size_t esize = dtype == DSPARK_BF16 ? 2 : 4;
  const size_t eb = up(static_cast<size_t>(rows) * markov_rank * esize);
  if (wm) {
    // valid_mask NULL: every slot valid (a ones mask after the embeddings)
    const uint8_t* mask = valid_mask;
    if (!mask) {
      char* mz = static_cast<char*>(workspace) + eb;
      DSPARK_TRY(launch_fill_u32(mz, (rows + 3) / 4, 0x01010101u, s));
      mask = reinterpret_cast<const uint8_t*>(mz);
    }
    DSPARK_TRY(launch_gather_embed(dtype, rows, markov_rank, target_vocab, prev_ids, mask,
                                   markov_w1, workspace, s));
  }
  DSPARK_TRY(launch_conf_logits(dtype, rows, draft_hidden, wm ? markov_rank : 0, wm ? 1 : 0, hidden,
                                workspace, conf_w, conf_b, valid_mask, out, s));
  return DSPARK_OK;
}

// ---- the no-allocation entry point's scratch
// Device memory of dspark_confidence_logits_noalloc: one array per GPU the
// library runs on, held until the process ends.  Host code uses the address
// hipGetSymbolAddress returns for the current device, never the array's
// name (on the host that name is a stand-in, not a device address).
__device__ __align__(256) unsigned char scratch[DSPARK_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device.
int scratch_address(void** out) {
  int dev = 0;
  DSPARK_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return DSPARK_ERR_SHAPE;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    DSPARK_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return DSPARK_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSPARK_OK;
}

}  // namespace
}  // namespace dspark

using namespace dspark;

extern "C" {

size_t dspark_workspace_size(const dspark_shape* shape) {
  Dims d;
  if (make_dims(shape, &d) != DSPARK_OK) return 0;
  return make_layout(d).total;
}

const char* dspark_status_string(int status) {
  switch (status) {
    case DSPARK_OK: return "ok";
    case DSPARK_ERR_NULL: return "a required pointer is NULL";
    case DSPARK_ERR_SHAPE: return "invalid or inconsistent dimensions";
    case DSPARK_ERR_DTYPE: return "dtype must be DSPARK_F32 or DSPARK_BF16";
    case DSPARK_ERR_NO_TARGET: return "L1 term or confidence head requested without a teacher";
    case DSPARK_ERR_WORKSPACE: return "workspace NULL or smaller than dspark_workspace_size()";
    case DSPARK_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case DSPARK_ERR_HIP: return "HIP launch failure (see dspark_last_hip_error)";
    case DSPARK_ERR_SCRATCH:
      return "problem larger than the no-allocation entry point's scratch (DSPARK_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown status";
}

const char* dspark_last_hip_error(void) { return g_hip_err; }

int dspark_loss_fwd(const dspark_shape* shape, const dspark_hparams* hp, const dspark_inputs* in,
                    void* workspace, size_t workspace_bytes, dspark_fwd_out* out,
                    dspark_stream_t stream) {
  Dims d;
  int st = make_dims(shape, &d);
  if (st) return st;
  Teacher teacher;
  st = check_inputs(d, hp, in, &teacher);
  if (st) return st;
  if (!out || !out->loss || !out->num_tokens || !out->pairs || !out->flags) return DSPARK_ERR_NULL;
  if (misaligned(workspace) || misaligned(out->accept_rate) || misaligned(out->row_terms))
    return DSPARK_ERR_ALIGN;
  const Layout L = make_layout(d);
  if (!workspace || workspace_bytes < L.total) return DSPARK_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const RowState rs = row_state(ws, L, d);
  float* Zp = reinterpret_cast<float*>(ws + L.Zp);
  float* T = reinterpret_cast<float*>(ws + L.T);
  float2* sz = reinterpret_cast<float2*>(ws + L.sz);
  float2* stt = reinterpret_cast<float2*>(ws + L.st);
  void* E = ws + L.E;

  DSPARK_STAGE(kPrep, launch_prep_rows(d.R, static_cast<int>(d.K), in->eval_mask, in->block_keep_mask,
                              in->target_ids, in->prev_ids, d.Vd, d.Vt, d.markov,
                              hp->loss_decay_gamma, teacher == kNone ? DSPARK_FLAG_NO_TEACHER : 0u,
                              rs.mask, rs.w, out->flags, s));
  if (d.markov)
    DSPARK_STAGE(kGather, launch_gather_embed(d.dtype, d.R, d.r, d.Vt, in->prev_ids, rs.mask, in->markov_w1,
                                   E, s));

  if (d.bias_path) {
    // Teacher logits T (fp32) with per-tile statistics; the corrected draft
    // logits are rebuilt inside each sweep and never stored.
    if (teacher != kNone) {
      Operand A{}, B{};
      EpiParams ep{};
      A.nseg = B.nseg = 1;
      A.layout = B.layout = LAYOUT_KC;
      ep.C = T; ep.ldc = d.Vd; ep.stats = stt; ep.nstat = d.nstat;
      if (teacher == kHidden) {
        A.seg[0] = A.seg[1] = in->target_hidden; A.kseg = d.H; A.kpad = gemm_kpad(d.H, d.esize);
        A.ld = d.H;
        B.seg[0] = B.seg[1] = in->lm_head; B.kseg = d.H; B.kpad = A.kpad; B.ld = d.H;
      } else {  // K = 0: T = aligned logits
        ep.X = in->aligned_target_logits; ep.ldx = d.Vd;
      }
      DSPARK_STAGE(kLogitsGemm, launch_gemm(d.dtype, EPI_STATS, 1, d.R, d.Vd, A, B, 1, ep, s));
    }
    const bf16_t* z = static_cast<const bf16_t*>(in->draft_logits);
    const bf16_t* Eb = d.markov ? static_cast<const bf16_t*>(E) : nullptr;
    const bf16_t* W2 = d.markov ? static_cast<const bf16_t*>(in->markov_w2) : nullptr;
    double* pl1 = reinterpret_cast<double*>(ws + L.pl1);
    double* ps = reinterpret_cast<double*>(ws + L.ps);
    DSPARK_STAGE(kBiasStats, launch_bias_stats(d.R, d.Vd, d.r, z, Eb, W2, sz, d.nstat, s));
    DSPARK_STAGE(kL1Sweep, launch_lse_rows(d.R, sz, stt, d.nstat, rs.mask, teacher != kNone, rs, s));
    DSPARK_STAGE(kL1Sweep, launch_bias_l1(d.R, d.Vd, d.r, z, Eb, W2, teacher != kNone ? T : nullptr,
                                          in->target_ids, rs, pl1, ps,
                                          reinterpret_cast<uint2*>(ws + L.sg), s));
    DSPARK_STAGE(kL1Sweep, launch_bias_l1_finish(d.R, d.Vd, d.r, static_cast<int>(d.bsplits),
                                                 teacher != kNone, pl1, ps, z, Eb, W2,
                                                 in->target_ids, rs, s));
  } else {
  // Corrected draft logits z' = z + E W2^T and teacher logits T (both fp32),
  // each with per-tile softmax statistics, over the same [R, Vd] tile grid.
  {
    Operand A[2] = {}, B[2] = {};
    EpiParams ep[2] = {};
    A[0].seg[0] = A[0].seg[1] = E; A[0].kseg = d.r; A[0].kpad = gemm_kpad(d.r, d.esize);
    A[0].ld = d.r; A[0].layout = LAYOUT_KC; A[0].nseg = 1;
    B[0].seg[0] = B[0].seg[1] = in->markov_w2; B[0].kseg = d.r; B[0].kpad = A[0].kpad;
    B[0].ld = d.r; B[0].layout = LAYOUT_KC; B[0].nseg = 1;
    ep[0].C = Zp; ep[0].ldc = d.Vd; ep[0].X = in->draft_logits; ep[0].ldx = d.Vd;
    ep[0].stats = sz; ep[0].nstat = d.nstat;
    int njobs = 1;
    if (teacher != kNone) {
      njobs = 2;
      ep[1].C = T; ep[1].ldc = d.Vd; ep[1].stats = stt; ep[1].nstat = d.nstat;
      A[1].nseg = B[1].nseg = 1;
      A[1].layout = B[1].layout = LAYOUT_KC;
      if (teacher == kHidden) {
        A[1].seg[0] = A[1].seg[1] = in->target_hidden; A[1].kseg = d.H;
        A[1].kpad = gemm_kpad(d.H, d.esize); A[1].ld = d.H;
        B[1].seg[0] = B[1].seg[1] = in->lm_head; B[1].kseg = d.H; B[1].kpad = A[1].kpad;
        B[1].ld = d.H;
      } else {  // K = 0: T = aligned logits
        ep[1].X = in->aligned_target_logits; ep[1].ldx = d.Vd;
      }
    }
    DSPARK_STAGE(kLogitsGemm, launch_logits(d.dtype, d.R, d.Vd, A, B, ep, njobs, s));
  }
  DSPARK_STAGE(kL1Sweep, launch_l1_sweep(d.R, d.Vd, Zp, T, sz, stt, d.nstat, rs.mask, in->target_ids,
                             teacher != kNone, rs, s));
  }
  DSPARK_STAGE(kFinalize, launch_finalize_rows(d.dtype, d.R, d.Hd, d.r, d.conf_markov, d.conf,
                                  in->conf_hidden, E, in->conf_w, in->conf_b, rs,
                                  out->accept_rate, out->row_terms, out->flags, hp->ce_alpha,
                                  hp->l1_alpha, hp->confidence_alpha, s));
  DSPARK_STAGE(kReduce, launch_reduce_fwd(d.R, d.B * d.N, static_cast<int>(d.K), rs, in->eval_mask,
                               in->block_keep_mask, hp->ce_alpha, hp->l1_alpha,
                               d.conf ? hp->confidence_alpha : 0.f, out->loss, out->num_tokens,
                               out->pairs, s));
  return DSPARK_OK;
}

int dspark_loss_bwd(const dspark_shape* shape, const dspark_hparams* hp, const dspark_inputs* in,
                    void* workspace, size_t workspace_bytes, float grad_scale,
                    dspark_bwd_out* out, dspark_stream_t stream) {
  Dims d;
  int st = make_dims(shape, &d);
  if (st) return st;
  Teacher teacher;
  st = check_inputs(d, hp, in, &teacher);
  if (st) return st;
  if (!out || !out->d_draft_logits) return DSPARK_ERR_NULL;
  if (d.markov && (!out->d_markov_w1 || !out->d_markov_w2)) return DSPARK_ERR_NULL;
  if (d.conf && (!out->d_conf_w || !out->d_conf_b)) return DSPARK_ERR_NULL;
  if (misaligned(workspace) || misaligned(out->d_draft_logits) || misaligned(out->d_markov_w1) ||
      misaligned(out->d_markov_w2) || misaligned(out->d_conf_hidden))
    return DSPARK_ERR_ALIGN;
  const Layout L = make_layout(d);
  if (!workspace || workspace_bytes < L.total) return DSPARK_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const RowState rs = row_state(ws, L, d);
  const float* Zp = reinterpret_cast<const float*>(ws + L.Zp);
  const float* T = reinterpret_cast<const float*>(ws + L.T);
  void* E = ws + L.E;
  const float g = grad_scale;
  const float c_a = d.conf ? hp->confidence_alpha : 0.f;

  float* dEpart = reinterpret_cast<float*>(ws + L.dEpart);
  float* dE = reinterpret_cast<float*>(ws + L.dE);
  if (d.dtype == DSPARK_BF16) {
    // G = dloss/dz' (= dloss/dz) as dz plus bf16 hi/lo parts: row-major for
    // dE = G . W2 (contraction over the vocabulary) and k-blocked by 8 rows for
    // dW2 = G^T . E (contraction over rows).
    bf16_t* ghi = d.gdtype == DSPARK_BF16 ? nullptr : reinterpret_cast<bf16_t*>(ws + L.ghi);
    bf16_t* glo = d.g_lo ? reinterpret_cast<bf16_t*>(ws + L.glo) : nullptr;
    const void* gA = ghi ? static_cast<const void*>(ghi) : out->d_draft_logits;
    bf16_t* bhi = reinterpret_cast<bf16_t*>(ws + L.blkhi);
    bf16_t* blo = reinterpret_cast<bf16_t*>(ws + L.blklo);
    const int64_t rgroups = d.R32 / 8;
    if (d.bias_path) {
      // G (z' rebuilt from z, E and W2) as dz (hi) and its bf16 remainder (lo)
      DSPARK_STAGE(kGradSweep, launch_bias_grad(
                                   d.gdtype, d.R, d.Vd, d.r,
                                   static_cast<const bf16_t*>(in->draft_logits),
                                   d.markov ? static_cast<const bf16_t*>(E) : nullptr,
                                   d.markov ? static_cast<const bf16_t*>(in->markov_w2) : nullptr,
                                   reinterpret_cast<const uint2*>(ws + L.sg), in->target_ids, rs,
                                   teacher != kNone, g, hp->ce_alpha, hp->l1_alpha,
                                   out->d_draft_logits, ghi, glo, s));
    }
    if (d.direct_bwd) {
      // G as dz (hi) and, with fp32 dz, its bf16 remainder (lo), row-major;
      // both products read G, W2 and E in place.
      if (!d.bias_path)
        DSPARK_STAGE(kGradSweep, launch_grad_sweep(d.gdtype, d.R, d.Vd, Zp, T, in->target_ids, rs,
                                                   teacher != kNone, g, hp->ce_alpha, hp->l1_alpha,
                                                   out->d_draft_logits, ghi, glo, nullptr, s));
      DSPARK_STAGE(kDeGemm, de_parts_direct(d, gA, glo, in->markov_w2, dEpart, s));
      DSPARK_STAGE(kDeReduce, launch_de_reduce(d.dtype, d.R, d.r, static_cast<int>(d.splits),
                                               dEpart, rs, d.conf_markov, in->conf_w, d.Hd, g,
                                               c_a, dE, s));
      DSPARK_STAGE(kDw1, dw1_stage(d, L, ws, in->prev_ids, rs.mask, dE, out->d_markov_w1, s));
      {  // dW2 over row splits (summed when there are two)
        float* part = dw2_target(d, L, ws, out->d_markov_w2);
        DSPARK_STAGE(kDw2Gemm, dw2_parts_direct(d, gA, glo, E, part, s));
        if (d.dw2_splits > 1)
          DSPARK_STAGE(kDw2Gemm, launch_sum_parts(d.Vd * d.r, static_cast<int>(d.dw2_splits),
                                                  part, out->d_markov_w2, s));
      }
    } else if (d.markov) {
      DSPARK_STAGE(kGradSweep, launch_grad_sweep8(d.gdtype, d.R, rgroups, d.Vd, Zp, T,
                                                  in->target_ids, rs, teacher != kNone, g,
                                                  hp->ce_alpha, hp->l1_alpha, out->d_draft_logits,
                                                  ghi, glo, bhi, blo, s));
    } else if (!d.bias_path) {
      DSPARK_STAGE(kGradSweep, launch_grad_sweep(d.gdtype, d.R, d.Vd, Zp, T, in->target_ids, rs,
                                                 teacher != kNone, g, hp->ce_alpha, hp->l1_alpha,
                                                 out->d_draft_logits, nullptr, nullptr, nullptr,
                                                 s));
    }
    if (d.markov && !d.direct_bwd) {
      void* w2t = ws + L.w2t;
      void* eblk = ws + L.eblk;
      DSPARK_STAGE(kOperandPrep, launch_transpose_bf16(d.Vd, d.r, in->markov_w2, w2t, s));
      {  // dE partials = G . W2 over vocabulary splits (both operands K-contiguous)
        Operand A{}, B{};
        A.seg[0] = gA; A.seg[1] = glo; A.kseg = d.Vd; A.kpad = gemm_kpad(d.Vd, 2);
        A.ld = d.Vd; A.layout = LAYOUT_KC; A.nseg = 2;
        B.seg[0] = B.seg[1] = w2t; B.kseg = d.Vd; B.kpad = A.kpad; B.ld = d.Vd;
        B.layout = LAYOUT_KC; B.nseg = 2;
        EpiParams ep{};
        ep.C = dEpart; ep.ldc = d.r;
        DSPARK_STAGE(kDeGemm, launch_gemm(d.dtype, EPI_PARTIAL, 2, d.R, d.r, A, B,
                                          static_cast<int>(d.splits), ep, s));
      }
      DSPARK_STAGE(kDeReduce, launch_de_reduce(d.dtype, d.R, d.r, static_cast<int>(d.splits),
                                               dEpart, rs, d.conf_markov, in->conf_w, d.Hd, g,
                                               c_a, dE, s));
      DSPARK_STAGE(kDw1, dw1_stage(d, L, ws, in->prev_ids, rs.mask, dE, out->d_markov_w1, s));
      DSPARK_STAGE(kOperandPrep, launch_embed_blocked(d.R, rgroups, d.r, E, eblk, s));
      {  // dW2 = G^T . E: hi and lo segments as two splits, then summed
        float* part = reinterpret_cast<float*>(ws + L.dw2part);
        Operand A{}, B{};
        A.seg[0] = bhi; A.seg[1] = blo; A.kseg = d.R32; A.kpad = gemm_kpad(d.R32, 2);
        A.ld = d.Vd; A.layout = LAYOUT_KB; A.nseg = 2;
        B.seg[0] = B.seg[1] = eblk; B.kseg = d.R32; B.kpad = A.kpad; B.ld = d.r;
        B.layout = LAYOUT_KB; B.nseg = 2;
        EpiParams ep{};
        ep.C = part; ep.ldc = d.r;
        DSPARK_STAGE(kDw2Gemm, launch_gemm(d.dtype, EPI_PARTIAL, 3, d.Vd, d.r, A, B, 2, ep, s));
        DSPARK_STAGE(kDw2Gemm, launch_add2(d.Vd * d.r, part, part + d.Vd * d.r,
                                           out->d_markov_w2, s));
      }
    }
  } else {
    // fp32 operands: G in fp32, products on the fp32 MFMA with strided operands
    float* g32 = d.gdtype == DSPARK_F32 ? nullptr : reinterpret_cast<float*>(ws + L.g32);
    const void* gA = g32 ? static_cast<const void*>(g32) : out->d_draft_logits;
    DSPARK_STAGE(kGradSweep, launch_grad_sweep(d.gdtype, d.R, d.Vd, Zp, T, in->target_ids, rs,
                                               teacher != kNone, g, hp->ce_alpha, hp->l1_alpha,
                                               out->d_draft_logits, nullptr, nullptr, g32, s));
    if (d.markov) {
      {  // dE partials = G . W2 over vocabulary splits
        Operand A{}, B{};
        A.seg[0] = A.seg[1] = gA; A.kseg = d.Vd; A.kpad = gemm_kpad(d.Vd, 4);
        A.ld = d.Vd; A.layout = LAYOUT_KC; A.nseg = 1;
        B.seg[0] = B.seg[1] = in->markov_w2; B.kseg = d.Vd; B.kpad = A.kpad; B.ld = d.r;
        B.layout = LAYOUT_MC; B.nseg = 1;
        EpiParams ep{};
        ep.C = dEpart; ep.ldc = d.r;
        DSPARK_STAGE(kDeGemm, launch_gemm(d.dtype, EPI_PARTIAL, 2, d.R, d.r, A, B,
                                          static_cast<int>(d.splits), ep, s));
      }
      DSPARK_STAGE(kDeReduce, launch_de_reduce(d.dtype, d.R, d.r, static_cast<int>(d.splits),
                                               dEpart, rs, d.conf_markov, in->conf_w, d.Hd, g,
                                               c_a, dE, s));
      DSPARK_STAGE(kDw1, dw1_stage(d, L, ws, in->prev_ids, rs.mask, dE, out->d_markov_w1, s));
      {  // dW2 = G^T . E (reduction over rows)
        Operand A{}, B{};
        A.seg[0] = A.seg[1] = gA; A.kseg = d.R; A.kpad = gemm_kpad(d.R, 4);
        A.ld = d.Vd; A.layout = LAYOUT_MC; A.nseg = 1;
        B.seg[0] = B.seg[1] = E; B.kseg = d.R; B.kpad = A.kpad; B.ld = d.r;
        B.layout = LAYOUT_MC; B.nseg = 1;
        EpiParams ep{};
        ep.C = out->d_markov_w2; ep.ldc = d.r;
        DSPARK_STAGE(kDw2Gemm, launch_gemm(d.dtype, EPI_STORE, 3, d.Vd, d.r, A, B, 1, ep, s));
      }
    }
  }
  if (d.conf) {
    float* part = reinterpret_cast<float*>(ws + L.confpart);
    DSPARK_STAGE(kConfBwd, launch_conf_bwd(d.dtype, d.R, d.Hd, d.r, d.conf_markov, in->conf_hidden, E,
                               in->conf_w, rs, g, c_a, part, d.conf_chunks, out->d_conf_w,
                               out->d_conf_b, out->d_conf_hidden, s));
  }
  return DSPARK_OK;
}

int dspark_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (int i = 0; i < kStages; ++i) {
    for (auto& pr : g_prof.pending[i]) {
      (void)hipEventSynchronize(pr.second);
      g_prof.pool.push_back(pr.first);
      g_prof.pool.push_back(pr.second);
    }
    g_prof.pending[i].clear();
    g_prof.ms[i] = 0.0;
    g_prof.count[i] = 0;
  }
  g_prof.on.store(on != 0);
  return DSPARK_OK;
}

int dspark_profile_read(double* ms, int64_t* counts, int n) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  for (int i = 0; i < kStages; ++i) {
    for (auto& pr : g_prof.pending[i]) {
      float t = 0.f;
      if (hipEventSynchronize(pr.second) == hipSuccess &&
          hipEventElapsedTime(&t, pr.first, pr.second) == hipSuccess) {
        g_prof.ms[i] += t;
        g_prof.count[i] += 1;
      }
      g_prof.pool.push_back(pr.first);
      g_prof.pool.push_back(pr.second);
    }
    g_prof.pending[i].clear();
  }
  for (int i = 0; i < n && i < kStages; ++i) {
    if (ms) ms[i] = g_prof.ms[i];
    if (counts) counts[i] = g_prof.count[i];
  }
  return kStages;
}

const char* dspark_stage_name(int stage) {
  return (stage >= 0 && stage < kStages) ? kStageNames[stage] : "";
}

size_t dspark_markov_logits_workspace_size(int64_t rows, int64_t draft_vocab,
                                           int64_t markov_rank, int32_t dtype) {
  if (head_dims(rows, draft_vocab, markov_rank > 0 ? 1 : 0, markov_rank, dtype) != DSPARK_OK ||
      draft_vocab == 0)
    return 0;
  return head_layout(rows, draft_vocab, markov_rank, dtype).total;
}

int dspark_markov_logits(int64_t rows, int64_t draft_vocab, int64_t target_vocab,
                         int64_t markov_rank, int32_t dtype, const void* draft_logits,
                         const int32_t* prev_ids, const uint8_t* valid_mask,
                         const void* markov_w1, const void* markov_w2, float* out,
                         void* workspace, size_t workspace_bytes, dspark_stream_t stream) {
  int st = head_dims(rows, draft_vocab, target_vocab, markov_rank, dtype);
  if (st) return st;
  if (draft_vocab == 0) return DSPARK_ERR_SHAPE;
  if (!draft_logits || !out || !workspace) return DSPARK_ERR_NULL;
  if (markov_rank > 0 && (!prev_ids || !markov_w1 || !markov_w2)) return DSPARK_ERR_NULL;
  if (misaligned(draft_logits) || misaligned(out) || misaligned(workspace) ||
      misaligned(prev_ids) || misaligned(markov_w1) || misaligned(markov_w2))
    return DSPARK_ERR_ALIGN;
  const HeadLayout L = head_layout(rows, draft_vocab, markov_rank, dtype);
  if (workspace_bytes < L.total) return DSPARK_ERR_WORKSPACE;
  if (rows == 0) return DSPARK_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int esize = dtype == DSPARK_BF16 ? 2 : 4;
  // valid_mask NULL: every slot valid (a ones mask in the statistics area,
  // which the projection overwrites afterwards)
  const uint8_t* mask = valid_mask;
  if (markov_rank > 0) {
    if (!mask) {
      DSPARK_TRY(launch_fill_u32(ws + L.st, (rows + 3) / 4, 0x01010101u, s));
      mask = reinterpret_cast<const uint8_t*>(ws + L.st);
    }
    DSPARK_TRY(launch_gather_embed(dtype, rows, markov_rank, target_vocab, prev_ids, mask,
                                   markov_w1, ws + L.E, s));
  }
  if (dtype == DSPARK_BF16 && bias_sweep_ok(draft_vocab, markov_rank)) {
    // the loss's sweep engine in its store pass: the bias rebuilt slice by
    // slice on the rows' E, z' written in fp32 and invalid rows as zeros
    DSPARK_TRY(launch_bias_store(rows, draft_vocab, markov_rank,
                                 static_cast<const bf16_t*>(draft_logits),
                                 markov_rank > 0 ? reinterpret_cast<const bf16_t*>(ws + L.E)
                                                 : nullptr,
                                 static_cast<const bf16_t*>(markov_w2), valid_mask, out, s));
    return DSPARK_OK;
  }
  // elsewhere z' = z + E W2^T is the loss's logits projection with z as the
  // epilogue addend (K = 0 without a Markov head: z' = z)
  Operand A{}, B{};
  A.seg[0] = A.seg[1] = ws + L.E; A.kseg = markov_rank;
  A.kpad = gemm_kpad(markov_rank, esize); A.ld = markov_rank; A.layout = LAYOUT_KC; A.nseg = 1;
  B.seg[0] = B.seg[1] = markov_w2; B.kseg = markov_rank; B.kpad = A.kpad; B.ld = markov_rank;
  B.layout = LAYOUT_KC; B.nseg = 1;
  EpiParams ep{};
  ep.C = out; ep.ldc = draft_vocab; ep.X = draft_logits; ep.ldx = draft_vocab;
  ep.stats = reinterpret_cast<float2*>(ws + L.st);
  ep.nstat = (draft_vocab + kStatTile - 1) / kStatTile;
  DSPARK_TRY(launch_logits(dtype, rows, draft_vocab, &A, &B, &ep, 1, s));
  // the head returns zero on invalid slots
  if (valid_mask) DSPARK_TRY(launch_zero_masked_rows(rows, draft_vocab, valid_mask, out, s));
  return DSPARK_OK;
}

size_t dspark_confidence_logits_workspace_size(int64_t rows, int64_t markov_rank,
                                               int32_t with_markov_conf, int32_t dtype) {
  if (head_dims(rows, 0, markov_rank > 0 ? 1 : 0, markov_rank, dtype) != DSPARK_OK) return 0;
  if (with_markov_conf == 0 || markov_rank == 0) return 0;
  const size_t esize = dtype == DSPARK_BF16 ? 2 : 4;
  // embeddings, then room for a ones mask when the caller passes none
  return up(static_cast<size_t>(rows) * markov_rank * esize) + up(static_cast<size_t>(rows) + 3);
}

int dspark_confidence_logits(int64_t rows, int64_t draft_hidden, int64_t target_vocab,
                             int64_t markov_rank, int32_t with_markov_conf, int32_t dtype,
                             const void* hidden, const int32_t* prev_ids,
                             const uint8_t* valid_mask, const void* markov_w1,
                             const void* conf_w, const void* conf_b, float* out,
                             void* workspace, size_t workspace_bytes, dspark_stream_t stream) {
  const bool wm = with_markov_conf != 0 && markov_rank > 0;
  int st = conf_head_check(rows, draft_hidden, target_vocab, markov_rank, with_markov_conf, dtype,
                           hidden, prev_ids, markov_w1, conf_w, conf_b, out);
  if (st) return st;
  if (wm && !workspace) return DSPARK_ERR_NULL;
  if (misaligned(workspace)) return DSPARK_ERR_ALIGN;
  if (workspace_bytes < dspark_confidence_logits_workspace_size(rows, markov_rank,
                                                                with_markov_conf, dtype))
    return DSPARK_ERR_WORKSPACE;
  return conf_head_launch(rows, draft_hidden, target_vocab, markov_rank, with_markov_conf, dtype,
                          hidden, prev_ids, valid_mask, markov_w1, conf_w, conf_b, out,
                          workspace, static_cast<hipStream_t>(stream));
}

int dspark_confidence_logits_noalloc(int64_t rows, int64_t draft_hidden, int64_t target_vocab,
                                     int64_t markov_rank, int32_t with_markov_conf, int32_t dtype,
                                     const void* hidden, const int32_t* prev_ids,
                                     const uint8_t* valid_mask, const void* markov_w1,
                                     const void* conf_w, const void* conf_b, float* out,
                                     dspark_stream_t stream) {
  int st = conf_head_check(rows, draft_hidden, target_vocab, markov_rank, with_markov_conf, dtype,
                           hidden, prev_ids, markov_w1, conf_w, conf_b, out);
  if (st) return st;
  const size_t need = dspark_confidence_logits_workspace_size(rows, markov_rank, with_markov_conf,
                                                              dtype);
  if (need > DSPARK_NOALLOC_SCRATCH_BYTES) return DSPARK_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address(&ws);
    if (st) return st;
  }
  return conf_head_launch(rows, draft_hidden, target_vocab, markov_rank, with_markov_conf, dtype,
                          hidden, prev_ids, valid_mask, markov_w1, conf_w, conf_b, out, ws,
                          static_cast<hipStream_t>(stream));
}


int dspark_build_blocks(int64_t batch, int64_t seq_len, int64_t num_blocks, int64_t block_size,
                        const int32_t* input_ids, const uint8_t* loss_mask,
                        const int32_t* anchors, int32_t* target_ids, int32_t* prev_ids,
                        uint8_t* eval_mask, uint8_t* block_keep, uint8_t* anchor_ok,
                        dspark_stream_t stream) {
  if (!input_ids || !loss_mask || !anchors || !target_ids || !prev_ids || !eval_mask ||
      !block_keep)
    return DSPARK_ERR_NULL;
  if (batch < 1 || seq_len < 1 || num_blocks < 1 || block_size < 1 || block_size > 4096)
    return DSPARK_ERR_SHAPE;
  if (batch * num_blocks > (int64_t{1} << 31) / block_size || batch > (int64_t{1} << 40) / seq_len)
    return DSPARK_ERR_SHAPE;
  return hip_status(launch_build_blocks(batch, seq_len, num_blocks, static_cast<int>(block_size),
                                        input_ids, loss_mask, anchors, target_ids, prev_ids,
                                        eval_mask, block_keep, anchor_ok,
                                        static_cast<hipStream_t>(stream)));
}

int dspark_accept_report(int64_t batch, int64_t num_blocks, int64_t block_size,
                         const float* accept_rate, const uint8_t* eval_mask,
                         const uint8_t* block_keep_mask, double* out4, dspark_stream_t stream) {
  if (!accept_rate || !eval_mask || !out4) return DSPARK_ERR_NULL;
  if (batch <= 0 || num_blocks <= 0 || block_size <= 0) return DSPARK_ERR_SHAPE;
  if (misaligned(accept_rate) || misaligned(eval_mask) || misaligned(out4) ||
      misaligned(block_keep_mask))
    return DSPARK_ERR_ALIGN;
  return hip_status(launch_accept_report(batch * num_blocks, static_cast<int>(block_size),
                                         accept_rate, eval_mask, block_keep_mask, out4,
                                         static_cast<hipStream_t>(stream)));
}

// ---- vocabulary shards: each caller holds draft_vocab columns of the draft
// logits, teacher and W2; the (lse, L1, S, z'_y) row partials merge exactly.

int dspark_shard_fwd_stats(const dspark_shape* shape, const dspark_hparams* hp,
                           const dspark_inputs* in, void* workspace, size_t workspace_bytes,
                           float* lse_part, uint32_t* flags, dspark_stream_t stream) {
  Dims d;
  Layout L;
  Teacher teacher;
  int st = shard_setup(shape, hp, in, workspace, workspace_bytes, &d, &L, &teacher);
  if (st) return st;
  if (!lse_part || !flags) return DSPARK_ERR_NULL;
  if (misaligned(lse_part)) return DSPARK_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const RowState rs = row_state(ws, L, d);
  float* T = reinterpret_cast<float*>(ws + L.T);
  float2* sz = reinterpret_cast<float2*>(ws + L.sz);
  float2* stt = reinterpret_cast<float2*>(ws + L.st);
  void* E = ws + L.E;
  // target ids are shard-local: out of [0, Vd) means another shard owns them
  DSPARK_STAGE(kPrep, launch_prep_rows(d.R, static_cast<int>(d.K), in->eval_mask,
                                       in->block_keep_mask, in->target_ids, in->prev_ids, d.Vd,
                                       d.Vt, d.markov, hp->loss_decay_gamma,
                                       teacher == kNone ? DSPARK_FLAG_NO_TEACHER : 0u, rs.mask,
                                       rs.w, flags, s, 0));
  if (d.markov)
    DSPARK_STAGE(kGather, launch_gather_embed(d.dtype, d.R, d.r, d.Vt, in->prev_ids, rs.mask,
                                              in->markov_w1, E, s));
  if (teacher != kNone) {
    Operand A{}, B{};
    EpiParams ep{};
    A.nseg = B.nseg = 1;
    A.layout = B.layout = LAYOUT_KC;
    ep.C = T; ep.ldc = d.Vd; ep.stats = stt; ep.nstat = d.nstat;
    if (teacher == kHidden) {
      A.seg[0] = A.seg[1] = in->target_hidden; A.kseg = d.H; A.kpad = gemm_kpad(d.H, d.esize);
      A.ld = d.H;
      B.seg[0] = B.seg[1] = in->lm_head; B.kseg = d.H; B.kpad = A.kpad; B.ld = d.H;
    } else {
      ep.X = in->aligned_target_logits; ep.ldx = d.Vd;
    }
    DSPARK_STAGE(kLogitsGemm, launch_gemm(d.dtype, EPI_STATS, 1, d.R, d.Vd, A, B, 1, ep, s));
  }
  const bf16_t* z = static_cast<const bf16_t*>(in->draft_logits);
  DSPARK_STAGE(kBiasStats, launch_bias_stats(d.R, d.Vd, d.r, z,
                                             d.markov ? static_cast<const bf16_t*>(E) : nullptr,
                                             d.markov ? static_cast<const bf16_t*>(in->markov_w2)
                                                      : nullptr,
                                             sz, d.nstat, s));
  DSPARK_STAGE(kL1Sweep, launch_lse_rows(d.R, sz, stt, d.nstat, rs.mask, teacher != kNone, rs, s));
  DSPARK_STAGE(kL1Sweep, launch_shard_lse_out(d.R, teacher != kNone, rs,
                                              reinterpret_cast<float2*>(lse_part), s));
  return DSPARK_OK;
}

int dspark_shard_merge_lse(int64_t shards, int64_t rows, const float* lse_parts, float* lse,
                           dspark_stream_t stream) {
  if (shards < 1 || rows < 0 || rows > (int64_t{1} << 31) - 1 || shards > (int64_t{1} << 16))
    return DSPARK_ERR_SHAPE;
  if (rows == 0) return DSPARK_OK;
  if (!lse_parts || !lse) return DSPARK_ERR_NULL;
  if (misaligned(lse_parts) || misaligned(lse)) return DSPARK_ERR_ALIGN;
  return hip_status(launch_shard_merge_lse(shards, rows, lse_parts, lse,
                                           static_cast<hipStream_t>(stream)));
}

int dspark_shard_fwd_terms(const dspark_shape* shape, const dspark_hparams* hp,
                           const dspark_inputs* in, void* workspace, size_t workspace_bytes,
                           const float* lse, double* terms, dspark_stream_t stream) {
  Dims d;
  Layout L;
  Teacher teacher;
  int st = shard_setup(shape, hp, in, workspace, workspace_bytes, &d, &L, &teacher);
  if (st) return st;
  if (!lse || !terms) return DSPARK_ERR_NULL;
  if (misaligned(lse) || misaligned(terms)) return DSPARK_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const RowState rs = row_state(ws, L, d);
  const bf16_t* z = static_cast<const bf16_t*>(in->draft_logits);
  const bf16_t* Eb = d.markov ? reinterpret_cast<const bf16_t*>(ws + L.E) : nullptr;
  const bf16_t* W2 = d.markov ? static_cast<const bf16_t*>(in->markov_w2) : nullptr;
  double* pl1 = reinterpret_cast<double*>(ws + L.pl1);
  double* ps = reinterpret_cast<double*>(ws + L.ps);
  DSPARK_STAGE(kL1Sweep, launch_shard_set_lse(d.R, teacher != kNone,
                                              reinterpret_cast<const float2*>(lse), rs, s));
  DSPARK_STAGE(kL1Sweep, launch_bias_l1(d.R, d.Vd, d.r, z, Eb, W2,
                                        teacher != kNone ? reinterpret_cast<const float*>(ws + L.T)
                                                         : nullptr,
                                        in->target_ids, rs, pl1, ps,
                                        reinterpret_cast<uint2*>(ws + L.sg), s));
  DSPARK_STAGE(kL1Sweep, launch_bias_l1_shard(d.R, d.Vd, d.r, static_cast<int>(d.bsplits),
                                              teacher != kNone, pl1, ps, z, Eb, W2,
                                              in->target_ids, rs, terms, s));
  return DSPARK_OK;
}

int dspark_shard_fwd_finish(const dspark_shape* shape, const dspark_hparams* hp,
                            const dspark_inputs* in, void* workspace, size_t workspace_bytes,
                            const double* terms, dspark_fwd_out* out, dspark_stream_t stream) {
  Dims d;
  Layout L;
  Teacher teacher;
  int st = shard_setup(shape, hp, in, workspace, workspace_bytes, &d, &L, &teacher);
  if (st) return st;
  if (!terms) return DSPARK_ERR_NULL;
  if (!out || !out->loss || !out->num_tokens || !out->pairs || !out->flags) return DSPARK_ERR_NULL;
  if (misaligned(terms) || misaligned(out->accept_rate) || misaligned(out->row_terms))
    return DSPARK_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const RowState rs = row_state(ws, L, d);
  DSPARK_STAGE(kFinalize, launch_shard_set_terms(d.R, terms, rs, out->flags, s));
  DSPARK_STAGE(kFinalize, launch_finalize_rows(d.dtype, d.R, d.Hd, d.r, d.conf_markov, d.conf,
                                               in->conf_hidden, ws + L.E, in->conf_w, in->conf_b,
                                               rs, out->accept_rate, out->row_terms, out->flags,
                                               hp->ce_alpha, hp->l1_alpha, hp->confidence_alpha,
                                               s));
  DSPARK_STAGE(kReduce, launch_reduce_fwd(d.R, d.B * d.N, static_cast<int>(d.K), rs,
                                          in->eval_mask, in->block_keep_mask, hp->ce_alpha,
                                          hp->l1_alpha, d.conf ? hp->confidence_alpha : 0.f,
                                          out->loss, out->num_tokens, out->pairs, s));
  return DSPARK_OK;
}

int dspark_shard_bwd(const dspark_shape* shape, const dspark_hparams* hp, const dspark_inputs* in,
                     void* workspace, size_t workspace_bytes, float grad_scale,
                     void* d_draft_logits, float* d_markov_w2, float* d_embed,
                     dspark_stream_t stream) {
  Dims d;
  Layout L;
  Teacher teacher;
  int st = shard_setup(shape, hp, in, workspace, workspace_bytes, &d, &L, &teacher);
  if (st) return st;
  if (!d_draft_logits) return DSPARK_ERR_NULL;
  if (d.markov && (!d_markov_w2 || !d_embed)) return DSPARK_ERR_NULL;
  if (misaligned(d_draft_logits) || misaligned(d_markov_w2) || misaligned(d_embed))
    return DSPARK_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const RowState rs = row_state(ws, L, d);
  void* E = ws + L.E;
  bf16_t* ghi = d.gdtype == DSPARK_BF16 ? nullptr : reinterpret_cast<bf16_t*>(ws + L.ghi);
  bf16_t* glo = d.g_lo ? reinterpret_cast<bf16_t*>(ws + L.glo) : nullptr;
  const void* gA = ghi ? static_cast<const void*>(ghi) : d_draft_logits;
  DSPARK_STAGE(kGradSweep,
               launch_bias_grad(d.gdtype, d.R, d.Vd, d.r,
                                static_cast<const bf16_t*>(in->draft_logits),
                                d.markov ? static_cast<const bf16_t*>(E) : nullptr,
                                d.markov ? static_cast<const bf16_t*>(in->markov_w2) : nullptr,
                                reinterpret_cast<const uint2*>(ws + L.sg), in->target_ids, rs,
                                teacher != kNone, grad_scale, hp->ce_alpha, hp->l1_alpha,
                                d_draft_logits, ghi, glo, s, 1));
  if (d.markov) {
    float* dEpart = reinterpret_cast<float*>(ws + L.dEpart);
    DSPARK_STAGE(kDeGemm, de_parts_direct(d, gA, glo, in->markov_w2, dEpart, s));
    DSPARK_STAGE(kDeReduce, launch_de_reduce(d.dtype, d.R, d.r, static_cast<int>(d.splits),
                                             dEpart, rs, 0, nullptr, d.Hd, grad_scale, 0.f,
                                             d_embed, s));
    float* part = dw2_target(d, L, ws, d_markov_w2);
    DSPARK_STAGE(kDw2Gemm, dw2_parts_direct(d, gA, glo, E, part, s));
    if (d.dw2_splits > 1)
      DSPARK_STAGE(kDw2Gemm, launch_sum_parts(d.Vd * d.r, static_cast<int>(d.dw2_splits), part,
                                              d_markov_w2, s));
  }
  return DSPARK_OK;
}

int dspark_shard_bwd_finish(const dspark_shape* shape, const dspark_hparams* hp,
                            const dspark_inputs* in, void* workspace, size_t workspace_bytes,
                            float grad_scale, const float* d_embed, dspark_bwd_out* out,
                            dspark_stream_t stream) {
  Dims d;
  Layout L;
  Teacher teacher;
  int st = shard_setup(shape, hp, in, workspace, workspace_bytes, &d, &L, &teacher);
  if (st) return st;
  if (!out) return DSPARK_ERR_NULL;
  if (d.markov && (!d_embed || !out->d_markov_w1)) return DSPARK_ERR_NULL;
  if (d.conf && (!out->d_conf_w || !out->d_conf_b)) return DSPARK_ERR_NULL;
  if (misaligned(d_embed) || misaligned(out->d_markov_w1) || misaligned(out->d_conf_hidden))
    return DSPARK_ERR_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const RowState rs = row_state(ws, L, d);
  void* E = ws + L.E;
  const float c_a = d.conf ? hp->confidence_alpha : 0.f;
  if (d.markov) {
    float* dE = reinterpret_cast<float*>(ws + L.dE);
    // the confidence term of dE once, on the shard-summed vocabulary term
    DSPARK_STAGE(kDeReduce, launch_de_reduce(d.dtype, d.R, d.r, 1, d_embed, rs, d.conf_markov,
                                             in->conf_w, d.Hd, grad_scale, c_a, dE, s));
    DSPARK_STAGE(kDw1, dw1_stage(d, L, ws, in->prev_ids, rs.mask, dE, out->d_markov_w1, s));
  }
  if (d.conf) {
    float* part = reinterpret_cast<float*>(ws + L.confpart);
    DSPARK_STAGE(kConfBwd, launch_conf_bwd(d.dtype, d.R, d.Hd, d.r, d.conf_markov,
                                           in->conf_hidden, E, in->conf_w, rs, grad_scale, c_a,
                                           part, d.conf_chunks, out->d_conf_w, out->d_conf_b,
                                           out->d_conf_hidden, s));
  }
  return DSPARK_OK;
}

}  // extern "C"
