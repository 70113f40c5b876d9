// Host side of the C ABI declared in include/flce.h: chunk policy, workspace
// layout, argument checks, and the chunk loop that enqueues the kernels.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "flce.h"
#include "flce_internal.h"

namespace {

using namespace flce;

// ------------------------------------------------------------ chunk policy
int64_t floor_pow2(int64_t x) {
  int64_t p = 1;
  while (p <= x / 2) p <<= 1;
  return p;
}
int64_t next_pow2(int64_t x) {
  int64_t p = 1;
  while (p < x) p <<= 1;
  return p;
}
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

int64_t chunk_rows(int64_t BT, int64_t H, int64_t V, int64_t chunk_size, int32_t C) {
  if (BT < 0 || H < 1 || V < 1) return FLCE_E_ARG;
  int64_t c;
  if (chunk_size > 0) {
    // PR #1439: an explicit size is floored to a power of two and clamped to BT.
    c = floor_pow2(chunk_size);
  } else {
    // v0.8.3 commit bad6c3ec42: memory budget of about C * BT * H elements
    // for the [chunk, V] slab.  inc = ceil(V / (C * H)) chunks, each of
    // next_pow2(ceil(BT / inc)) rows.
    if (C < 1) return FLCE_E_ARG;
    const int64_t inc = ceil_div(V, (int64_t)C * H);
    c = next_pow2(ceil_div(BT, inc));
  }
  if (c > BT) c = BT;
  if (c < 1) c = 1;
  return c;
}

// ---------------------------------------------------------- workspace layout
constexpr int64_t kAlign = 256;
constexpr uint64_t kMaxOperandBytes = 0x7fff0000ull;  // 2 GiB - 64 KiB
constexpr uint64_t kMaxRangeBytes = 0x7ffffff0ull;    // largest range of one buffer descriptor
constexpr int kDxCUs = 256;  // split k until every resident workgroup slot of 256 CUs is busy
constexpr int64_t kDxMinKPerSplit = 1024;
constexpr int kDxMaxSplits = 32;

// MI355X chunk policy model (see flce_chunk_size_mi355x in flce.h).
constexpr double kMfma16 = 2516.6e12;           // dense bf16/fp16 MFMA peak, FLOP/s
constexpr double kMfmaF32 = 157.3e12;           // dense fp32 MFMA peak, FLOP/s
constexpr double kGemmEfficiency = 0.40;        // measured fraction of peak of the GEMMs
constexpr double kHbmBytesPerSecond = 5.1e12;   // measured device-copy rate
constexpr double kSlabPasses = 5.0;             // slab: write, read+write, read by dX and dW
constexpr double kPolicyTolerance = 1.10;       // accept 10 % above the large-chunk cost
constexpr size_t kDefaultSlabBudget = 2ull << 30;  // 2 GiB logits slab

struct Layout {
  int64_t c = 0, ldz = 0, ldx = 0, stats_ld = 0;
  bool x_gather = false;  // X exceeds one 32-bit range: logits read rows gathered into Xc
  int64_t xc_rows = 0;    // rows gathered (and multiplied) at a time in that case
  int splits = 1;
  int64_t k_per_split = 0;
  size_t off_slab = 0, off_xct = 0, off_stats = 0, off_ztgt = 0, off_partial = 0, off_idx = 0,
         off_lossrow = 0, off_flags = 0, off_amax = 0, off_bias = 0, off_zrow = 0,
         off_accrow = 0, off_xc = 0, total = 0;
};

// What the options add to a call.
struct Extras {
  bool forward_only = false, amax = false, bias_grad = false, zrow = false, accrow = false;
};
Extras extras_of(const flce_options_t* o) {
  Extras e;
  if (!o) return e;
  e.forward_only = o->forward_only != 0;
  e.amax = o->predicted || o->accuracy;
  e.bias_grad = o->grad_bias && !e.forward_only;
  e.zrow = o->z_loss != nullptr;
  e.accrow = o->accuracy != nullptr;
  return e;
}

size_t itemsize(int dt) { return dt == FLCE_F32 ? 4 : 2; }

Layout make_layout(int64_t BT, int64_t H, int64_t V, int dtype, int64_t c, const Extras& x) {
  Layout L;
  L.c = c;
  L.ldz = round_up(V, 8);
  L.ldx = round_up(c, 8);
  L.stats_ld = ceil_div(V, stats_cols());
  const DxTile dt = dx_tile(dtype, (int)c, H);
  // grad_input split over V: s splits make tiles x s workgroups, each with
  // 1/s of the work, run in ceil(tiles x s / slots) rounds.  Take the s that
  // minimises rounds / s (the time in units of one unsplit workgroup), moving
  // to a larger s only for a gain above 3 %: every split adds c x H fp32
  // partials to write and reduce.  (Rounding s up to cover the chip, as
  // tiles x s >= slots, can leave a nearly empty last round: 21 tiles x 13
  // splits = 273 workgroups on 256 CUs take two rounds.)
  const int64_t tiles = ceil_div(c, dt.bm) * ceil_div(H, dt.bn);
  const int64_t slots = (int64_t)kDxCUs * dt.wgs;
  int64_t smax = L.ldz / kDxMinKPerSplit;
  if (smax > kDxMaxSplits) smax = kDxMaxSplits;
  int64_t splits = 1;
  double best = (double)ceil_div(tiles, slots);
  for (int64_t sp = 2; sp <= smax; ++sp) {
    const double t = (double)ceil_div(tiles * sp, slots) / (double)sp;
    if (t < best * 0.97) {
      best = t;
      splits = sp;
    }
  }
  L.k_per_split = round_up(ceil_div(L.ldz, splits), 64);
  L.splits = (int)ceil_div(L.ldz, L.k_per_split);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (size_t)round_up((int64_t)bytes, kAlign);
    return o;
  };
  const bool grads = !x.forward_only;  // a loss-only call never stores logits
  const size_t nrow = (size_t)(BT > 0 ? BT : 1);
  L.off_slab = take(grads ? (size_t)c * L.ldz * itemsize(dtype) : 0);
  L.off_xct = take(grads ? (size_t)H * L.ldx * itemsize(dtype) : 0);
  L.off_stats = take((size_t)c * L.stats_ld * 8);
  L.off_ztgt = take((size_t)c * 4);
  L.off_partial = take(grads && L.splits > 1 ? (size_t)L.splits * c * H * 4 : 0);
  L.off_idx = take(nrow * 4);
  L.off_lossrow = take(nrow * 4);
  L.off_flags = take(sizeof(ScanFlags));
  L.off_amax = take(x.amax ? (size_t)c * L.stats_ld * 4 : 0);
  L.off_bias = take(x.bias_grad ? (size_t)ceil_div(c, kBiasRows) * L.ldz * 4 : 0);
  L.off_zrow = take(x.zrow ? nrow * 4 : 0);
  L.off_accrow = take(x.accrow ? nrow * 4 : 0);
  L.x_gather = (uint64_t)BT * (uint64_t)H * itemsize(dtype) > kMaxOperandBytes;
  if (L.x_gather) {
    // whole 256-row tiles whose gathered rows fit one range (H <= 2^20: >= 256 rows)
    const int64_t fit = (int64_t)(kMaxOperandBytes / ((uint64_t)H * itemsize(dtype))) / 256 * 256;
    L.xc_rows = c < fit ? c : fit;
  }
  L.off_xc = take(L.x_gather ? (size_t)L.xc_rows * H * itemsize(dtype) : 0);
  L.total = off;
  return L;
}

// ------------------------------------------------------------------ errors
thread_local char g_last_error[512] = "";

int fail_hip(hipError_t e, const char* what) {
  std::snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", what, hipGetErrorString(e),
                (int)e);
  return FLCE_E_HIP;
}

// --------------------------------------------------------------- profiling
struct ProfRec {
  int kind;
  hipEvent_t a, b;
};
struct Profiler {
  bool open = false;
  uint32_t kinds = 0;  // bit k set: kernels of kind k are bracketed
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
thread_local Profiler g_prof;

struct ProfScope {
  hipStream_t st;
  bool on = false;
  ProfRec rec{};
  ProfScope(int kind, hipStream_t s) : st(s) {
    if (!g_prof.open || !((g_prof.kinds >> kind) & 1u)) return;
    rec.kind = kind;
    rec.a = g_prof.get();
    rec.b = g_prof.get();
    if (rec.a && rec.b) {
      on = true;
      (void)hipEventRecord(rec.a, st);
    }
  }
  ~ProfScope() {
    if (!on) return;
    (void)hipEventRecord(rec.b, st);
    g_prof.recs.push_back(rec);
  }
};

#define FLCE_LAUNCH(kind, expr)                       \
  do {                                                \
    hipError_t e_;                                    \
    {                                                 \
      ProfScope ps_(kind, st);                        \
      e_ = (expr);                                    \
    }                                                 \
    if (e_ != hipSuccess) return fail_hip(e_, #expr); \
  } while (0)

// Pinned host word pair for the single device-to-host read, and a plain one
// for the entry point that allocates nothing.
thread_local ScanFlags* g_host_flags = nullptr;
thread_local ScanFlags g_pageable_flags;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// A buffer's byte range as the call uses it (empty when absent).
struct Span {
  const void* p;
  uint64_t n;
};
bool overlap(const Span& a, const Span& b) {
  if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

}  // namespace

extern "C" {

int64_t flce_chunk_size(int64_t BT, int64_t H, int64_t V, int64_t chunk_size,
                        int32_t chunk_mem_const) {
  return chunk_rows(BT, H, V, chunk_size, chunk_mem_const);
}

int64_t flce_chunk_size_mi355x(int64_t BT, int64_t H, int64_t V, flce_dtype_t dtype,
                               flce_dtype_t accum_dtype, int32_t frozen_weight,
                               size_t slab_budget_bytes) {
  if (BT < 0 || H < 1 || V < 1) return FLCE_E_ARG;
  if (dtype < FLCE_F32 || dtype > FLCE_BF16) return FLCE_E_ARG;
  if (accum_dtype != dtype && accum_dtype != FLCE_F32) return FLCE_E_ARG;
  if (BT == 0) return 1;
  const double s = (double)itemsize(dtype), a = (double)itemsize(accum_dtype);
  const double Hd = (double)H, Vd = (double)V;
  const double rate = (dtype == FLCE_F32 ? kMfmaF32 : kMfma16) * kGemmEfficiency;
  const double k = frozen_weight ? 4.0 : 6.0;
  // Time of one chunk of c rows: the larger of its GEMM time and its HBM time.
  auto chunk_time = [&](double c) {
    // the row-tiled GEMMs (logits, grad_input) compute whole 256-row tiles
    const double c_tiles = std::ceil(c / 256.0) * 256.0;
    const double flops = (k - 2.0) * c_tiles * Hd * Vd + 2.0 * c * Hd * Vd;
    double bytes = 2.0 * Vd * Hd * s + kSlabPasses * c * Vd * s;
    if (!frozen_weight) bytes += 2.0 * a * Vd * Hd;
    return flops / rate + bytes / kHbmBytesPerSecond;
  };
  // Per-row cost as c grows without bound.
  const double floor_row = k * Hd * Vd / rate + kSlabPasses * Vd * s / kHbmBytesPerSecond;
  const size_t budget = slab_budget_bytes ? slab_budget_bytes : kDefaultSlabBudget;
  int64_t cap = (int64_t)(budget / (size_t)((double)V * s));
  if (cap < 1) cap = 1;
  int64_t c = 1;
  while (c * 2 <= cap && c < BT && chunk_time((double)c) / (double)c > kPolicyTolerance * floor_row)
    c *= 2;
  return chunk_rows(BT, H, V, c, 1);
}

size_t flce_workspace_bytes_ex(int64_t BT, int64_t H, int64_t V, flce_dtype_t dtype,
                               int64_t chunk_size, int32_t chunk_mem_const,
                               const flce_options_t* opt) {
  if (dtype < FLCE_F32 || dtype > FLCE_BF16) return 0;
  const int64_t c = chunk_rows(BT, H, V, chunk_size, chunk_mem_const);
  if (c < 1) return 0;
  return make_layout(BT, H, V, dtype, c, extras_of(opt)).total;
}

size_t flce_workspace_row_index_offset(int64_t BT, int64_t H, int64_t V, flce_dtype_t dtype,
                                       int64_t chunk_size, int32_t chunk_mem_const,
                                       const flce_options_t* opt) {
  if (dtype < FLCE_F32 || dtype > FLCE_BF16) return (size_t)-1;
  const int64_t c = chunk_rows(BT, H, V, chunk_size, chunk_mem_const);
  if (c < 1) return (size_t)-1;
  return make_layout(BT, H, V, dtype, c, extras_of(opt)).off_idx;
}

size_t flce_workspace_bytes(int64_t BT, int64_t H, int64_t V, flce_dtype_t dtype,
                            int64_t chunk_size, int32_t chunk_mem_const) {
  return flce_workspace_bytes_ex(BT, H, V, dtype, chunk_size, chunk_mem_const, nullptr);
}

const char* flce_status_string(int status) {
  switch (status) {
    case FLCE_OK: return "FLCE_OK";
    case FLCE_E_ARG: return "FLCE_E_ARG: invalid argument";
    case FLCE_E_DTYPE: return "FLCE_E_DTYPE: unsupported dtype combination";
    case FLCE_E_TARGET: return "FLCE_E_TARGET: labelled target outside [0, V)";
    case FLCE_E_WORKSPACE: return "FLCE_E_WORKSPACE: workspace too small";
    case FLCE_E_HIP: return "FLCE_E_HIP: HIP runtime error";
    default: return "unknown status";
  }
}

const char* flce_last_error(void) { return g_last_error; }

const char* flce_kernel_name(int kind) {
  static const char* names[FLCE_K_COUNT] = {
      "mask_scan", "zero_ignored_rows", "logits_gemm", "softmax_grad", "dx_gemm",
      "dx_reduce", "dw_gemm",           "loss_finalize", "fill_cast",  "gather_rows",
      "bias_grad"};
  return (kind >= 0 && kind < FLCE_K_COUNT) ? names[kind] : "unknown";
}

int flce_profile_begin_kinds(uint32_t kind_mask) {
  if (kind_mask == 0 || (kind_mask >> FLCE_K_COUNT) != 0) return FLCE_E_ARG;
  for (auto& r : g_prof.recs) {
    g_prof.pool.push_back(r.a);
    g_prof.pool.push_back(r.b);
  }
  g_prof.recs.clear();
  g_prof.kinds = kind_mask;
  g_prof.open = true;
  return FLCE_OK;
}

int flce_profile_begin(void) { return flce_profile_begin_kinds((1u << FLCE_K_COUNT) - 1u); }

int flce_profile_end(flce_profile_t* out) {
  if (!g_prof.open) return FLCE_E_ARG;
  g_prof.open = false;
  flce_profile_t p;
  std::memset(&p, 0, sizeof p);
  int rc = FLCE_OK;
  for (auto& r : g_prof.recs) {
    hipError_t e = hipEventSynchronize(r.b);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) {
      rc = fail_hip(e, "flce_profile_end");
      continue;
    }
    p.launches[r.kind] += 1;
    p.total_ms[r.kind] += ms;
    g_prof.pool.push_back(r.a);
    g_prof.pool.push_back(r.b);
  }
  g_prof.recs.clear();
  if (out) *out = p;
  return rc;
}

int flce_scale_cast(const void* src, flce_dtype_t src_dtype, void* dst, flce_dtype_t dst_dtype,
                    int64_t n, const float* scale, void* stream) {
  if (n < 0 || (n > 0 && (!src || !dst))) return FLCE_E_ARG;
  if (src_dtype < FLCE_F32 || src_dtype > FLCE_BF16) return FLCE_E_DTYPE;
  if (dst_dtype < FLCE_F32 || dst_dtype > FLCE_BF16) return FLCE_E_DTYPE;
  if (n > 0 && src == dst && src_dtype != dst_dtype) return FLCE_E_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  FLCE_LAUNCH(FLCE_K_FILL, launch_scale_cast(src, (int)src_dtype, dst, (int)dst_dtype, n, scale,
                                             st));
  return FLCE_OK;
}

}  // extern "C"

namespace {

// The whole call.  `pageable_flags`: read the labelled-row count and the
// range flag at the single sync into plain host memory instead of the
// thread's pinned pair (which is allocated on its first use), so that the
// call allocates nothing.
int fwd_bwd(const void* X, const void* W, const int64_t* targets, int64_t BT, int64_t H,
            int64_t V, flce_dtype_t dtype, int64_t ignore_index, flce_reduction_t reduction,
            int64_t chunk_size, int32_t chunk_mem_const, flce_dtype_t accum_dtype,
            int32_t frozen_weight, int32_t accumulate_dw, const float* grad_output, float* loss,
            void* dX, void* dW, void* workspace, size_t workspace_bytes, void* stream,
            flce_stats_t* stats, const flce_options_t* opt, bool pageable_flags) {
  // ---- host-side checks: nothing is launched or written on failure
  if (dtype < FLCE_F32 || dtype > FLCE_BF16) return FLCE_E_DTYPE;
  if (accum_dtype != dtype && accum_dtype != FLCE_F32) return FLCE_E_DTYPE;
  if (reduction < FLCE_MEAN || reduction > FLCE_NONE) return FLCE_E_ARG;
  // H <= 2^20 keeps a 256-row tile of dW (fp32) within one 32-bit buffer range
  if (BT < 0 || BT > 0x7ffffffe || V < 1 || V > 0x7ffffffe || H < 8 || H % 8 != 0 ||
      H > (1 << 20))
    return FLCE_E_ARG;
  if (frozen_weight != 0 && frozen_weight != 1) return FLCE_E_ARG;
  if (accumulate_dw != 0 && accumulate_dw != 1) return FLCE_E_ARG;
  // (reduction none over zero rows has an empty loss vector, which may be NULL)
  if (!loss && !(reduction == FLCE_NONE && BT == 0)) return FLCE_E_ARG;
  flce_options_t o;
  std::memset(&o, 0, sizeof o);
  if (opt) o = *opt;
  if (o.forward_only != 0 && o.forward_only != 1) return FLCE_E_ARG;
  if (!(o.z_loss_scale >= 0.f) || !std::isfinite(o.z_loss_scale)) return FLCE_E_ARG;
  if ((o.bias && !aligned(o.bias, 16)) || (o.grad_bias && !aligned(o.grad_bias, 16)) ||
      (o.predicted && !aligned(o.predicted, 8)) || (o.z_loss && !aligned(o.z_loss, 4)) ||
      (o.accuracy && !aligned(o.accuracy, 4)))
    return FLCE_E_ARG;
  const bool grads = !o.forward_only;
  const bool want_dw = grads && !frozen_weight;
  if (want_dw && (!dW || !aligned(dW, 16))) return FLCE_E_ARG;
  if (BT > 0 && (!X || !W || !targets || (grads && !dX))) return FLCE_E_ARG;
  if (BT > 0 && (!aligned(X, 16) || !aligned(W, 16) || (grads && !aligned(dX, 16))))
    return FLCE_E_ARG;
  const int64_t c = chunk_rows(BT, H, V, chunk_size, chunk_mem_const);
  if (c < 1) return FLCE_E_ARG;
  // The GEMMs address their operands through 32-bit buffer ranges of one
  // tile: 256 rows of the logits slab (grad_input) and 256 hidden units of
  // the transposed chunk rows (grad_weight).  X of any size: when it exceeds
  // one range, the logits GEMM reads the chunk's rows gathered into the
  // workspace, a range-sized block of rows at a time.
  {
    const uint64_t s = itemsize(dtype);
    if (grads && 256ull * (uint64_t)round_up(V, 8) * s > kMaxRangeBytes) return FLCE_E_ARG;
    if (want_dw && 256ull * (uint64_t)round_up(c, 8) * s > kMaxRangeBytes) return FLCE_E_ARG;
  }
  const Extras ext = extras_of(&o);
  const Layout L = make_layout(BT, H, V, dtype, c, ext);
  if (!workspace || !aligned(workspace, kAlign)) return FLCE_E_ARG;
  {
    // Every buffer the call writes must be disjoint from every other buffer it
    // reads or writes (the kernels read inputs while outputs are being written).
    const bool none_red = reduction == FLCE_NONE;
    const uint64_t s = itemsize(dtype), a = itemsize(accum_dtype);
    const uint64_t per_tok = none_red ? 4ull * (uint64_t)BT : 4ull;
    const Span written[] = {
        {loss, per_tok},
        {grads ? dX : nullptr, (uint64_t)BT * H * s},
        {want_dw ? dW : nullptr, (uint64_t)V * H * a},
        {workspace, L.total},
        {grads ? o.grad_bias : nullptr, (uint64_t)V * a},
        {o.z_loss, per_tok},
        {o.accuracy, per_tok},
        {o.predicted, 8ull * (uint64_t)BT}};
    const Span read[] = {{X, (uint64_t)BT * H * s},
                         {W, (uint64_t)V * H * s},
                         {targets, 8ull * (uint64_t)BT},
                         {grad_output, per_tok},
                         {o.bias, (uint64_t)V * s}};
    const int nw = (int)(sizeof written / sizeof written[0]);
    for (int i = 0; i < nw; ++i) {
      for (int j = i + 1; j < nw; ++j)
        if (overlap(written[i], written[j])) return FLCE_E_ARG;
      for (const Span& r : read)
        if (overlap(written[i], r)) return FLCE_E_ARG;
    }
  }
  if (workspace_bytes < L.total) return FLCE_E_WORKSPACE;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const int dt = (int)dtype;
  const int red = (int)reduction;
  const int dw_dt = (int)accum_dtype;
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  void* slab = ws + L.off_slab;
  void* xct = ws + L.off_xct;
  float* stats_buf = reinterpret_cast<float*>(ws + L.off_stats);
  float* ztgt = reinterpret_cast<float*>(ws + L.off_ztgt);
  float* partial = reinterpret_cast<float*>(ws + L.off_partial);
  int32_t* idx = reinterpret_cast<int32_t*>(ws + L.off_idx);
  float* lossrow = reinterpret_cast<float*>(ws + L.off_lossrow);
  ScanFlags* dflags = reinterpret_cast<ScanFlags*>(ws + L.off_flags);
  int32_t* amax = ext.amax ? reinterpret_cast<int32_t*>(ws + L.off_amax) : nullptr;
  float* bias_partial = reinterpret_cast<float*>(ws + L.off_bias);
  float* zrow = ext.zrow ? reinterpret_cast<float*>(ws + L.off_zrow) : nullptr;
  float* accrow = ext.accrow ? reinterpret_cast<float*>(ws + L.off_accrow) : nullptr;
  void* xc = ws + L.off_xc;
  const bool none = reduction == FLCE_NONE;

  if (stats) {
    std::memset(stats, 0, sizeof *stats);
    stats->chunk_size = c;
    stats->chunks_total = ceil_div(BT, c);
    stats->dx_splits = L.splits;
  }

  // ---- row compaction and the single host sync
  int64_t N = 0;
  if (BT > 0) {
    FLCE_LAUNCH(FLCE_K_MASK_SCAN,
                launch_mask_scan(targets, BT, V, ignore_index, idx, dflags, st));
    IgnoredOut io;
    io.dX = grads ? dX : nullptr;
    io.dx_dtype = dt;
    io.loss_none = none ? loss : nullptr;
    io.z_none = none ? o.z_loss : nullptr;
    io.acc_none = none ? o.accuracy : nullptr;
    io.pred = o.predicted;
    FLCE_LAUNCH(FLCE_K_ZERO_ROWS, launch_zero_ignored(targets, BT, H, ignore_index, io, st));
    ScanFlags* hf = &g_pageable_flags;
    if (!pageable_flags) {
      if (!g_host_flags) {
        hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&g_host_flags), 64,
                                     hipHostMallocDefault);
        if (e != hipSuccess) {
          g_host_flags = nullptr;
          return fail_hip(e, "hipHostMalloc");
        }
      }
      hf = g_host_flags;
    }
    hipError_t e = hipMemcpyAsync(hf, dflags, sizeof(ScanFlags), hipMemcpyDeviceToHost, st);
    if (e != hipSuccess) return fail_hip(e, "hipMemcpyAsync(flags)");
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail_hip(e, "hipStreamSynchronize");
    if (hf->bad_target) return FLCE_E_TARGET;
    N = hf->n_valid;
  }
  const int64_t chunks = ceil_div(N, c);
  if (stats) {
    stats->n_valid = N;
    stats->chunks_run = chunks;
    stats->compacted = chunks < ceil_div(BT, c) ? 1 : 0;
  }

  if (want_dw && !accumulate_dw && chunks == 0)
    FLCE_LAUNCH(FLCE_K_FILL, launch_fill_zero(dW, V * H * (int64_t)itemsize(dw_dt), st));
  if (ext.bias_grad && !accumulate_dw && chunks == 0)
    FLCE_LAUNCH(FLCE_K_FILL, launch_fill_zero(o.grad_bias, V * (int64_t)itemsize(dw_dt), st));

  const float inv_n = N > 0 ? 1.0f / (float)N : 0.f;

  // softmax pass geometry: enough workgroups to cover the chip, >= 2048 columns each
  int parts = (int)ceil_div(2048, c);
  const int64_t max_parts = ceil_div(L.ldz, 2048);
  if (parts > max_parts) parts = (int)max_parts;
  if (parts < 1 || !grads) parts = 1;
  const int64_t cols_per_part = round_up(ceil_div(L.ldz, parts), 8);

  // ---- the chunk loop: logits -> softmax-gradient -> dX -> dW per chunk
  for (int64_t k = 0; k < chunks; ++k) {
    const int64_t base = k * c;
    const int rows = (int)((N - base) < c ? (N - base) : c);
    const int32_t* cidx = idx + base;

    LogitsArgs la;
    la.X = X;
    la.x_gathered = 0;
    la.W = W;
    la.idx = cidx;
    la.targets = targets;
    la.rows = rows;
    la.BT = BT;
    la.H = H;
    la.V = V;
    la.slab = slab;
    la.ldz = L.ldz;
    la.stats = stats_buf;
    la.stats_ld = L.stats_ld;
    la.ztgt = ztgt;
    la.bias = o.bias;
    la.amax = amax;
    la.store_slab = grads ? 1 : 0;
    if (!L.x_gather) {
      FLCE_LAUNCH(FLCE_K_LOGITS, launch_logits(dt, la, st));
    } else {
      // X beyond one 32-bit range: gather a block of the chunk's rows, then
      // multiply that block into its rows of the slab and statistics.
      for (int64_t r0 = 0; r0 < rows; r0 += L.xc_rows) {
        const int nr = (int)((rows - r0) < L.xc_rows ? (rows - r0) : L.xc_rows);
        FLCE_LAUNCH(FLCE_K_GATHER, launch_gather_rows(dt, X, cidx + r0, nr, H, xc, st));
        LogitsArgs lb = la;
        lb.X = xc;
        lb.x_gathered = 1;
        lb.idx = cidx + r0;
        lb.rows = nr;
        lb.slab = static_cast<unsigned char*>(slab) + (size_t)r0 * L.ldz * itemsize(dt);
        lb.stats = stats_buf + (size_t)r0 * L.stats_ld * 2;
        lb.ztgt = ztgt + r0;
        lb.amax = amax ? amax + (size_t)r0 * L.stats_ld : nullptr;
        FLCE_LAUNCH(FLCE_K_LOGITS, launch_logits(dt, lb, st));
      }
    }

    SoftmaxArgs sa;
    sa.slab = slab;
    sa.ldz = L.ldz;
    sa.V = V;
    sa.rows = rows;
    sa.stats = stats_buf;
    sa.stats_ld = L.stats_ld;
    sa.stats_n = L.stats_ld;
    sa.ztgt = ztgt;
    sa.idx = cidx;
    sa.targets = targets;
    sa.grad_output = grad_output;
    sa.reduction = red;
    sa.lossrow = lossrow + base;
    sa.loss_out = loss;
    sa.parts = parts;
    sa.cols_per_part = cols_per_part;
    sa.write_grad = grads ? 1 : 0;
    sa.z_scale = o.z_loss_scale;
    sa.amax = amax;
    sa.pred_out = o.predicted;
    sa.zrow = zrow ? zrow + base : nullptr;
    sa.accrow = accrow ? accrow + base : nullptr;
    sa.z_out = none ? o.z_loss : nullptr;
    sa.acc_out = none ? o.accuracy : nullptr;
    FLCE_LAUNCH(FLCE_K_SOFTMAX, launch_softmax(dt, sa, st));
    if (!grads) continue;

    if (ext.bias_grad) {
      BiasGradArgs ba;
      ba.slab = slab;
      ba.rows = rows;
      ba.V = V;
      ba.ldz = L.ldz;
      ba.partial = bias_partial;
      ba.grad_bias = o.grad_bias;
      ba.db_dtype = dw_dt;
      ba.accumulate = (accumulate_dw || k > 0) ? 1 : 0;
      ba.grad_output = grad_output;
      ba.inv_n = inv_n;
      ba.reduction = red;
      FLCE_LAUNCH(FLCE_K_BIAS_GRAD, launch_bias_grad(dt, ba, st));
    }

    DxArgs xa;
    xa.slab = slab;
    xa.W = W;
    xa.idx = cidx;
    xa.rows = rows;
    xa.rows_cap = (int)c;
    xa.H = H;
    xa.V = V;
    xa.ldz = L.ldz;
    xa.splits = L.splits;
    xa.k_per_split = L.k_per_split;
    xa.dX = dX;
    xa.partial = partial;
    xa.grad_output = grad_output;
    xa.inv_n = inv_n;
    xa.reduction = red;
    FLCE_LAUNCH(FLCE_K_DX, launch_dx(dt, xa, st));
    if (L.splits > 1) {
      DxReduceArgs ra;
      ra.partial = partial;
      ra.splits = L.splits;
      ra.rows = rows;
      ra.rows_cap = (int)c;
      ra.H = H;
      ra.idx = cidx;
      ra.dX = dX;
      ra.grad_output = grad_output;
      ra.inv_n = inv_n;
      ra.reduction = red;
      FLCE_LAUNCH(FLCE_K_DX_REDUCE, launch_dx_reduce(dt, ra, st));
    }

    if (want_dw) {
      FLCE_LAUNCH(FLCE_K_GATHER, launch_gather_t(dt, X, cidx, rows, H, xct, L.ldx, st));
      DwArgs wa;
      wa.slab = slab;
      wa.XcT = xct;
      wa.rows = rows;
      wa.H = H;
      wa.V = V;
      wa.ldz = L.ldz;
      wa.ldx = L.ldx;
      wa.dW = dW;
      wa.dw_dtype = dw_dt;
      wa.accumulate = (accumulate_dw || k > 0) ? 1 : 0;
      wa.grad_output = grad_output;
      wa.inv_n = inv_n;
      wa.reduction = red;
      FLCE_LAUNCH(FLCE_K_DW, launch_dw(dt, wa, st));
    }
  }

  if (!none) {
    const int mean = red == FLCE_MEAN;
    FLCE_LAUNCH(FLCE_K_FINALIZE, launch_finalize(lossrow, (int)N, mean, loss, st));
    if (o.z_loss) FLCE_LAUNCH(FLCE_K_FINALIZE, launch_finalize(zrow, (int)N, mean, o.z_loss, st));
    if (o.accuracy)
      FLCE_LAUNCH(FLCE_K_FINALIZE, launch_finalize(accrow, (int)N, mean, o.accuracy, st));
  }
  return FLCE_OK;
}

}  // namespace

// ------------------------------------------------------------ static scratch
// Device memory of flce_fwd_bwd_ex_noalloc: the workspace of callers that
// cannot allocate.  One copy per GPU, at its own address, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device memory: kernels and copies get the address from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[FLCE_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's scratch; the stream must run on
// that device.
int scratch_for(hipStream_t st, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
  if (st) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(st, &sdev);
    if (e != hipSuccess) return fail_hip(e, "hipStreamGetDevice");
    if ((int)sdev != dev) {
      std::snprintf(g_last_error, sizeof g_last_error,
                    "flce_fwd_bwd_ex_noalloc: the stream runs on device %d, the current device "
                    "is %d",
                    (int)sdev, dev);
      return FLCE_E_ARG;
    }
  }
  if (dev < 0 || dev >= kMaxScratchDevices) {
    std::snprintf(g_last_error, sizeof g_last_error,
                  "flce_fwd_bwd_ex_noalloc: device ordinal %d beyond %d", dev,
                  kMaxScratchDevices - 1);
    return FLCE_E_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FLCE_OK;
}

}  // namespace

extern "C" {

int flce_fwd_bwd_ex(const void* X, const void* W, const int64_t* targets, int64_t BT, int64_t H,
                    int64_t V, flce_dtype_t dtype, int64_t ignore_index,
                    flce_reduction_t reduction, int64_t chunk_size, int32_t chunk_mem_const,
                    flce_dtype_t accum_dtype, int32_t frozen_weight, int32_t accumulate_dw,
                    const float* grad_output, float* loss, void* dX, void* dW, void* workspace,
                    size_t workspace_bytes, void* stream, flce_stats_t* stats,
                    const flce_options_t* opt) {
  return fwd_bwd(X, W, targets, BT, H, V, dtype, ignore_index, reduction, chunk_size,
                 chunk_mem_const, accum_dtype, frozen_weight, accumulate_dw, grad_output, loss, dX,
                 dW, workspace, workspace_bytes, stream, stats, opt, false);
}

int flce_fwd_bwd_ex_noalloc(const void* X, const void* W, const int64_t* targets, int64_t BT,
                            int64_t H, int64_t V, flce_dtype_t dtype, int64_t ignore_index,
                            flce_reduction_t reduction, int64_t chunk_size,
                            int32_t chunk_mem_const, flce_dtype_t accum_dtype,
                            int32_t frozen_weight, int32_t accumulate_dw,
                            const float* grad_output, float* loss, void* dX, void* dW,
                            void* stream, flce_stats_t* stats, const flce_options_t* opt) {
  if (dtype < FLCE_F32 || dtype > FLCE_BF16) return FLCE_E_DTYPE;
  const size_t need =
      flce_workspace_bytes_ex(BT, H, V, dtype, chunk_size, chunk_mem_const, opt);
  if (need == 0) return FLCE_E_ARG;
  if (need > (size_t)FLCE_SCRATCH_BYTES) {
    std::snprintf(g_last_error, sizeof g_last_error,
                  "flce_fwd_bwd_ex_noalloc: this call needs %zu bytes of workspace, the static "
                  "scratch holds %zu; use a smaller chunk_size or flce_fwd_bwd_ex",
                  need, (size_t)FLCE_SCRATCH_BYTES);
    return FLCE_E_WORKSPACE;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  const int rc = scratch_for(st, &ws);
  if (rc != FLCE_OK) return rc;
  return fwd_bwd(X, W, targets, BT, H, V, dtype, ignore_index, reduction, chunk_size,
                 chunk_mem_const, accum_dtype, frozen_weight, accumulate_dw, grad_output, loss, dX,
                 dW, ws, (size_t)FLCE_SCRATCH_BYTES, stream, stats, opt, true);
}

int flce_fwd_bwd(const void* X, const void* W, const int64_t* targets, int64_t BT, int64_t H,
                 int64_t V, flce_dtype_t dtype, int64_t ignore_index, flce_reduction_t reduction,
                 int64_t chunk_size, int32_t chunk_mem_const, flce_dtype_t accum_dtype,
                 int32_t frozen_weight, int32_t accumulate_dw, const float* grad_output,
                 float* loss, void* dX, void* dW, void* workspace, size_t workspace_bytes,
                 void* stream, flce_stats_t* stats) {
  return fwd_bwd(X, W, targets, BT, H, V, dtype, ignore_index, reduction, chunk_size,
                 chunk_mem_const, accum_dtype, frozen_weight, accumulate_dw, grad_output, loss, dX,
                 dW, workspace, workspace_bytes, stream, stats, nullptr, false);
}

}  // extern "C"
