// Bandwidth-bound kernels around the projections: ignored-row compaction,
// zeroing of ignored outputs, the in-place softmax-gradient pass over the
// logits slab, the fixed-order reduction of split grad_input partials, the
// loss reduction, and fill / cast helpers.
#include "flce_device.hpp"
#include "flce_internal.h"

namespace flce {

// ---------------------------------------------------------------------------
// Row compaction (PR #1554, Summary: the projections run only on rows whose
// target is not ignore_index; nonzero() gives the row index and costs the one
// host sync).  One workgroup: mask, exclusive prefix sum of the mask, and the
// ascending list of labelled rows as int32; also flags labelled targets
// outside [0, V).
// ---------------------------------------------------------------------------
constexpr int SCAN_T = 1024;
constexpr int SCAN_PER = 8;

__global__ __launch_bounds__(SCAN_T) void mask_scan_kernel(const int64_t* __restrict__ t,
                                                           int64_t BT, int64_t V, int64_t ign,
                                                           int32_t* __restrict__ idx,
                                                           ScanFlags* flags) {
  __shared__ int wave_tot[SCAN_T / kWave];
  __shared__ int bad_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) bad_s = 0;
  int base = 0;
  int bad = 0;
  for (int64_t s0 = 0; s0 < BT; s0 += (int64_t)SCAN_T * SCAN_PER) {
    const int64_t e0 = s0 + (int64_t)tid * SCAN_PER;
    unsigned mask = 0;
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < SCAN_PER; ++q) {
      const int64_t e = e0 + q;
      if (e < BT) {
        const int64_t tv = t[e];
        if (tv != ign) {
          if (tv < 0 || tv >= V) bad = 1;
          mask |= 1u << q;
          ++cnt;
        }
      }
    }
    int x = cnt;  // inclusive scan within the wave
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int y = __shfl_up(x, d, kWave);
      if (lane >= d) x += y;
    }
    if (lane == kWave - 1) wave_tot[wave] = x;
    __syncthreads();
    int wave_off = 0, total = 0;
#pragma unroll
    for (int w = 0; w < SCAN_T / kWave; ++w) {
      const int c = wave_tot[w];
      if (w < wave) wave_off += c;
      total += c;
    }
    int pos = base + wave_off + x - cnt;
#pragma unroll
    for (int q = 0; q < SCAN_PER; ++q)
      if (mask & (1u << q)) idx[pos++] = (int32_t)(e0 + q);
    base += total;
    __syncthreads();  // wave_tot is rewritten by the next tile
  }
  if (bad) atomicOr(&bad_s, 1);
  __syncthreads();
  if (tid == 0) {
    flags->n_valid = base;
    flags->bad_target = bad_s;
  }
}

hipError_t launch_mask_scan(const int64_t* targets, int64_t BT, int64_t V, int64_t ignore_index,
                            int32_t* idx, ScanFlags* flags, hipStream_t st) {
  hipLaunchKernelGGL(mask_scan_kernel, dim3(1), dim3(SCAN_T), 0, st, targets, BT, V,
                     ignore_index, idx, flags);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row gather of the chunk's labelled X rows, written transposed:
// XcT[h, r] = X[idx[r], h] for r < rows, 0 for rows <= r < ldx (PR #1554,
// Details item 3: the compacted rows of a chunk are gathered into one reused
// chunk buffer).  The transposed layout makes the chunk's rows the contiguous
// k dimension of the grad_weight GEMM.  64 x 64 tiles through LDS.
// ---------------------------------------------------------------------------
template <class S>
__global__ __launch_bounds__(256) void gather_t_kernel(const S* __restrict__ X,
                                                       const int32_t* __restrict__ idx, int rows,
                                                       int64_t H, S* __restrict__ XcT,
                                                       int64_t ldx) {
  // 16-byte vectors both ways: VE elements of one row along h on the way in,
  // VE rows of one h on the way out.  H is a multiple of 8, so a vector along
  // h lies wholly inside or outside [0, H).
  constexpr int VE = 16 / (int)sizeof(S);
  constexpr int VPR = 64 / VE;             // vectors per 64-element tile row
  constexpr int PER = 64 * VPR / 256;      // vectors per thread each way
  __shared__ S tile[64][64 + 2];           // [row][h]; the pad spreads a column over banks
  __shared__ int32_t ridx[64];
  const int r0 = blockIdx.x * 64;
  const int64_t h0 = (int64_t)blockIdx.y * 64;
  const int tid = threadIdx.x;
  if (tid < 64) ridx[tid] = (r0 + tid < rows) ? idx[r0 + tid] : -1;
  __syncthreads();
  u32x4_t in[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int q = tid + e * 256;
    const int r = q / VPR, hv = (q % VPR) * VE;
    const int32_t src = ridx[r];
    in[e] = u32x4_t{0u, 0u, 0u, 0u};
    if (src >= 0 && h0 + hv < H)
      in[e] = *reinterpret_cast<const u32x4_t*>(X + (int64_t)src * H + h0 + hv);
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int q = tid + e * 256;
    const int r = q / VPR, hv = (q % VPR) * VE;
    const S* v = reinterpret_cast<const S*>(&in[e]);
#pragma unroll
    for (int k = 0; k < VE; ++k) tile[r][hv + k] = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int q = tid + e * 256;
    const int h = q / VPR, rv = (q % VPR) * VE;
    u32x4_t out;
    S* o = reinterpret_cast<S*>(&out);
#pragma unroll
    for (int k = 0; k < VE; ++k) o[k] = tile[rv + k][h];
    // ldx is a multiple of 8 (and so of VE): a vector lies wholly below or past it
    if (h0 + h < H && r0 + rv < ldx)
      *reinterpret_cast<u32x4_t*>(XcT + (h0 + h) * ldx + r0 + rv) = out;
  }
}

hipError_t launch_gather_t(int dtype, const void* X, const int32_t* idx, int rows, int64_t H,
                           void* XcT, int64_t ldx, hipStream_t st) {
  const dim3 grid((unsigned)((ldx + 63) / 64), (unsigned)((H + 63) / 64));
  if (dtype == 0)
    hipLaunchKernelGGL(gather_t_kernel<float>, grid, dim3(256), 0, st,
                       static_cast<const float*>(X), idx, rows, H, static_cast<float*>(XcT), ldx);
  else
    hipLaunchKernelGGL(gather_t_kernel<u16>, grid, dim3(256), 0, st, static_cast<const u16*>(X),
                       idx, rows, H, static_cast<u16*>(XcT), ldx);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row gather, row-major: Xc[r, :] = X[idx[r], :] for r < rows.  Used when X
// is larger than one 32-bit buffer range, so that the logits GEMM can read
// the chunk's rows with small offsets.  One 16-byte vector per thread and
// step; a workgroup walks a row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gather_rows_kernel(const u32x4_t* __restrict__ X,
                                                          const int32_t* __restrict__ idx,
                                                          int64_t row_vecs,
                                                          u32x4_t* __restrict__ Xc) {
  const int r = blockIdx.x;
  const u32x4_t* src = X + (int64_t)idx[r] * row_vecs;
  u32x4_t* dst = Xc + (int64_t)r * row_vecs;
  for (int64_t v = threadIdx.x; v < row_vecs; v += blockDim.x) dst[v] = src[v];
}

hipError_t launch_gather_rows(int dtype, const void* X, const int32_t* idx, int rows, int64_t H,
                              void* Xc, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const int64_t row_vecs = H * (dtype == 0 ? 4 : 2) / 16;  // H % 8 == 0
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)rows), dim3(256), 0, st,
                     static_cast<const u32x4_t*>(X), idx, row_vecs, static_cast<u32x4_t*>(Xc));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Ignored rows get a +0.0 grad_input row and +0.0 per-token loss (PR #1554,
// Details item 1).  Labelled rows are left alone: the projections write them.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void zero_ignored_kernel(const int64_t* __restrict__ t,
                                                           int64_t BT, int64_t row_vecs,
                                                           int64_t ign, IgnoredOut o) {
  for (int64_t row = blockIdx.x; row < BT; row += gridDim.x) {
    if (t[row] != ign) continue;
    if (o.dX) {
      u32x4_t* p = static_cast<u32x4_t*>(o.dX) + row * row_vecs;
      for (int64_t v = threadIdx.x; v < row_vecs; v += blockDim.x)
        p[v] = u32x4_t{0u, 0u, 0u, 0u};
    }
    if (threadIdx.x == 0) {
      if (o.loss_none) o.loss_none[row] = 0.f;
      if (o.z_none) o.z_none[row] = 0.f;
      if (o.acc_none) o.acc_none[row] = 0.f;
      if (o.pred) o.pred[row] = -1;
    }
  }
}

hipError_t launch_zero_ignored(const int64_t* targets, int64_t BT, int64_t H,
                               int64_t ignore_index, const IgnoredOut& o, hipStream_t st) {
  if (BT <= 0) return hipSuccess;
  const int64_t row_bytes = H * (o.dx_dtype == 0 ? 4 : 2);
  const int grid = (int)(BT < 2048 ? BT : 2048);
  hipLaunchKernelGGL(zero_ignored_kernel, dim3(grid), dim3(256), 0, st, targets, BT,
                     row_bytes / 16, ignore_index, o);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Softmax-gradient pass (v0.8.3 commit bad6c3ec42, Summary: the Triton fused
// cross-entropy step; here one read and one write of the slab).  For row m of
// the chunk:
//   lse  = log sum_v exp(z_v), combined from the per-64-column (max, sum exp)
//          pairs the logits GEMM left behind (fixed-order tree, fp32)
//   loss = lse - z_t + lam * lse^2 (z_t kept in fp32 by the logits GEMM; lam
//          is the optional z-loss coefficient, 0 by default)
//   G_v  = gamma * ((1 + 2 lam lse) exp(z_v - lse) - [v == t]),
//          gamma = g_i for none, else 1
// The slab holds z_v - M_b, with M_b the maximum of v's 64-column block (fp32
// difference rounded to the slab dtype), so exp(z_v - lse) is taken as
// exp((z_v - M_b) + (M_b - lse)): its rounding error grows with the distance
// from the block maximum, not with the size of the logits.  G is
// written over the slab in the operand dtype (round to nearest even); the
// slab's padding columns [V, ldz) become 0.  The mean/sum scale g/N or g is
// applied later, in fp32, by the gradient GEMMs: folding 1/N into a 16-bit
// slab would flush small fp16 probabilities to zero.
// Per-token outputs (PR #1554, Details item 1 and Tests: per-token loss,
// z-loss, accuracy and predicted token): the predicted token is the lowest
// column holding the row maximum (the first 64-column block whose maximum is
// the row's, then that block's first maximum, found by the logits GEMM from
// the same fp32 values); accuracy is predicted == target; the z-loss output
// is lse^2.
// ---------------------------------------------------------------------------
constexpr int SM_T = 256;

// (max, sum exp rescaled to max, first index of max) of two parts: the sums
// are rescaled to the larger maximum; of equal maxima the lower index wins.
// A part with no entries has (-inf, 0, INT_MAX) and leaves the other as is.
__device__ __forceinline__ void merge_max_sum_first(float& m, float& s, int& f, float m2, float s2,
                                                    int f2) {
  const float M = fmaxf(m, m2);
  const float a = m == M ? s : s * __expf(m - M);
  const float b = m2 == M ? s2 : s2 * __expf(m2 - M);
  const int fa = m == M ? f : 0x7fffffff, fb = m2 == M ? f2 : 0x7fffffff;
  s = a + b;
  f = fa < fb ? fa : fb;
  m = M;
}
// The same over the 64 lanes of a wave (butterfly: every lane ends with the
// wave's triple).
__device__ __forceinline__ void combine_max_sum_first(float& m, float& s, int& f) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const float m2 = __shfl_xor(m, o, kWave), s2 = __shfl_xor(s, o, kWave);
    const int f2 = __shfl_xor(f, o, kWave);
    merge_max_sum_first(m, s, f, m2, s2, f2);
  }
}

template <class T>
__global__ __launch_bounds__(SM_T) void softmax_kernel(SoftmaxArgs a) {
  typedef typename T::storage S;
  __shared__ float red[SM_T / kWave], red2[SM_T / kWave];
  __shared__ int ired[SM_T / kWave];
  __shared__ float bcast, bcast2;
  __shared__ int ibcast;
  const int m = blockIdx.x / a.parts;
  const int part = blockIdx.x % a.parts;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  const float2* st = reinterpret_cast<const float2*>(a.stats) + (int64_t)m * a.stats_ld;
  // One pass over the row's (block max, block sum exp) pairs: each thread
  // keeps a running maximum, the sum rescaled to it, and the first block
  // holding it; the threads' triples are then combined in a fixed tree.
  float mx = -INFINITY, s = 0.f;
  int first = 0x7fffffff;  // lowest block holding the row maximum
  for (int64_t j = tid; j < a.stats_n; j += SM_T) {
    const float2 p = st[j];
    if (p.x > mx) {
      s = s * __expf(mx - p.x) + p.y;
      mx = p.x;
      first = (int)j;
    } else {
      s += p.y * __expf(p.x - mx);
    }
  }
  combine_max_sum_first(mx, s, first);
  if (lane == 0) {
    red[wave] = mx;
    red2[wave] = s;
    ired[wave] = first;
  }
  __syncthreads();
  if (tid == 0) {
    float v = red[0], t = red2[0];
    int f = ired[0];
    for (int w = 1; w < SM_T / kWave; ++w) merge_max_sum_first(v, t, f, red[w], red2[w], ired[w]);
    bcast = v;
    bcast2 = t;
    ibcast = f;
  }
  __syncthreads();
  const float M = bcast;
  const float lse = M + logf(bcast2);

  const int64_t row = a.idx[m];
  const int64_t tgt = a.targets[row];
  if (part == 0 && tid == 0) {
    const float l = lse - a.ztgt[m] + a.z_scale * lse * lse;
    const float z2 = lse * lse;
    int64_t pred = -1;
    if (a.amax && ibcast != 0x7fffffff) pred = a.amax[(int64_t)m * a.stats_ld + ibcast];
    const float acc = (pred == tgt) ? 1.f : 0.f;
    if (a.pred_out) a.pred_out[row] = pred;
    if (a.reduction == 2) {
      a.loss_out[row] = l;
      if (a.z_out) a.z_out[row] = z2;
      if (a.acc_out) a.acc_out[row] = acc;
    } else {
      a.lossrow[m] = l;
      if (a.zrow) a.zrow[m] = z2;
      if (a.accrow) a.accrow[m] = acc;
    }
  }
  if (!a.write_grad) return;
  const float gamma = (a.reduction == 2 && a.grad_output) ? a.grad_output[row] : 1.f;
  const float pscale = gamma * (1.f + 2.f * a.z_scale * lse);

  S* z = static_cast<S*>(a.slab) + (int64_t)m * a.ldz;
  const int64_t c_beg = (int64_t)part * a.cols_per_part;
  int64_t c_end = c_beg + a.cols_per_part;
  if (c_end > a.ldz) c_end = a.ldz;
  constexpr int VE = T::vec;
  for (int64_t c = c_beg + (int64_t)tid * VE; c < c_end; c += (int64_t)SM_T * VE) {
    u32x4_t raw = *reinterpret_cast<const u32x4_t*>(z + c);
    S* e = reinterpret_cast<S*>(&raw);
    // the slab holds z - (block maximum); the VE columns share one 64-column block
    const float off = st[c >> 6].x - lse;
#pragma unroll
    for (int q = 0; q < VE; ++q) {
      const int64_t col = c + q;
      float g = 0.f;
      if (col < a.V) {
        const float p = __expf(T::to_f32(e[q]) + off);
        g = col == tgt ? pscale * p - gamma : pscale * p;
      }
      e[q] = T::from_f32(g);
    }
    *reinterpret_cast<u32x4_t*>(z + c) = raw;
  }
}

hipError_t launch_softmax(int dtype, const SoftmaxArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)(a.rows * a.parts));
  if (dtype == 0)
    hipLaunchKernelGGL(softmax_kernel<F32>, grid, dim3(SM_T), 0, st, a);
  else if (dtype == 1)
    hipLaunchKernelGGL(softmax_kernel<F16>, grid, dim3(SM_T), 0, st, a);
  else
    hipLaunchKernelGGL(softmax_kernel<BF16>, grid, dim3(SM_T), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split grad_input: dX[idx[m], n] = s * sum_split part[split][m][n], splits
// summed in ascending order (deterministic), then scattered to the row.
// ---------------------------------------------------------------------------
template <class T>
__global__ __launch_bounds__(256) void dx_reduce_kernel(DxReduceArgs a) {
  typedef typename T::storage S;
  const int64_t total4 = (int64_t)a.rows * a.H / 4;
  const float g = a.reduction == 2 ? 1.f : (a.grad_output ? a.grad_output[0] : 1.f);
  const float s = a.reduction == 0 ? g * a.inv_n : g;
  const int64_t plane = (int64_t)a.rows_cap * a.H;
  S* dX = static_cast<S*>(a.dX);
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total4;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int64_t f = e * 4;
    const int64_t m = f / a.H, n = f % a.H;
    // Splits summed in order 0, 1, 2, ...; eight loads in flight at a time.
    f32x4_t acc = *reinterpret_cast<const f32x4_t*>(a.partial + f);
    int sp = 1;
    for (; sp + 8 <= a.splits; sp += 8) {
      f32x4_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = *reinterpret_cast<const f32x4_t*>(a.partial + (sp + u) * plane + f);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; sp < a.splits; ++sp) acc += *reinterpret_cast<const f32x4_t*>(a.partial + sp * plane + f);
    S* o = dX + (int64_t)a.idx[m] * a.H + n;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = T::from_f32(s * acc[q]);
  }
}

hipError_t launch_dx_reduce(int dtype, const DxReduceArgs& a, hipStream_t st) {
  const int64_t total4 = (int64_t)a.rows * a.H / 4;
  int64_t blocks = (total4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  if (dtype == 0)
    hipLaunchKernelGGL(dx_reduce_kernel<F32>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  else if (dtype == 1)
    hipLaunchKernelGGL(dx_reduce_kernel<F16>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(dx_reduce_kernel<BF16>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Loss reduction: sum of the per-row losses of the labelled rows, in a fixed
// order (fp64 partial sums), divided by N for mean; 0 when N == 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void finalize_kernel(const float* __restrict__ lossrow, int n,
                                                        int mean, float* loss) {
  __shared__ double red[1024 / kWave];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double s = 0.0;
  for (int i = tid; i < n; i += 1024) s += (double)lossrow[i];
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) s += __shfl_xor(s, m, kWave);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  if (tid == 0) {
    double v = 0.0;
    for (int w = 0; w < 1024 / kWave; ++w) v += red[w];
    if (mean) v = n > 0 ? v / (double)n : 0.0;
    loss[0] = (float)v;
  }
}

hipError_t launch_finalize(const float* lossrow, int n, int mean, float* loss, hipStream_t st) {
  hipLaunchKernelGGL(finalize_kernel, dim3(1), dim3(1024), 0, st, lossrow, n, mean, loss);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// grad_bias of one chunk (PR #1554, Tests: bias on and off): the bias enters
// every labelled row's logits, so its gradient is the column sum of G,
// scaled like the other gradients (g/N for mean, g for sum; none carries g_i
// inside G).  Two deterministic passes: partial sums over blocks of
// kBiasRows rows in row order, then the blocks in order per column, added to
// grad_bias (accumulate) or written over it.
// ---------------------------------------------------------------------------
template <class T>
__global__ __launch_bounds__(256) void bias_partial_kernel(BiasGradArgs a) {
  typedef typename T::storage S;
  constexpr int VE = T::vec;
  const int64_t c = ((int64_t)blockIdx.y * 256 + threadIdx.x) * VE;
  if (c >= a.ldz) return;
  const int r0 = blockIdx.x * kBiasRows;
  const int r1 = r0 + kBiasRows < a.rows ? r0 + kBiasRows : a.rows;
  float acc[VE];
#pragma unroll
  for (int q = 0; q < VE; ++q) acc[q] = 0.f;
  const S* g = static_cast<const S*>(a.slab);
  for (int r = r0; r < r1; ++r) {
    u32x4_t raw = *reinterpret_cast<const u32x4_t*>(g + (int64_t)r * a.ldz + c);
    const S* e = reinterpret_cast<const S*>(&raw);
#pragma unroll
    for (int q = 0; q < VE; ++q) acc[q] += T::to_f32(e[q]);
  }
  float* out = a.partial + (int64_t)blockIdx.x * a.ldz + c;
#pragma unroll
  for (int q = 0; q < VE; ++q) out[q] = acc[q];
}

__global__ __launch_bounds__(256) void bias_reduce_kernel(BiasGradArgs a, int nblocks) {
  const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (v >= a.V) return;
  float s = 0.f;
  for (int b = 0; b < nblocks; ++b) s += a.partial[(int64_t)b * a.ldz + v];
  const float g = a.reduction == 2 ? 1.f : (a.grad_output ? a.grad_output[0] : 1.f);
  s *= a.reduction == 0 ? g * a.inv_n : g;
  if (a.db_dtype == 0) {
    float* d = static_cast<float*>(a.grad_bias);
    d[v] = a.accumulate ? d[v] + s : s;
  } else if (a.db_dtype == 1) {
    u16* d = static_cast<u16*>(a.grad_bias);
    d[v] = F16::from_f32(a.accumulate ? F16::to_f32(d[v]) + s : s);
  } else {
    u16* d = static_cast<u16*>(a.grad_bias);
    d[v] = BF16::from_f32(a.accumulate ? BF16::to_f32(d[v]) + s : s);
  }
}

hipError_t launch_bias_grad(int dtype, const BiasGradArgs& a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  const int nblocks = (a.rows + kBiasRows - 1) / kBiasRows;
  const int ve = dtype == 0 ? 4 : 8;
  const int64_t col_groups = (a.ldz / ve + 255) / 256;
  const dim3 grid((unsigned)nblocks, (unsigned)col_groups);
  if (dtype == 0)
    hipLaunchKernelGGL(bias_partial_kernel<F32>, grid, dim3(256), 0, st, a);
  else if (dtype == 1)
    hipLaunchKernelGGL(bias_partial_kernel<F16>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(bias_partial_kernel<BF16>, grid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bias_reduce_kernel, dim3((unsigned)((a.V + 255) / 256)), dim3(256), 0, st,
                     a, nblocks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fill / cast helpers.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_zero_kernel(u32x4_t* p, int64_t nvec,
                                                        unsigned char* tail, int tail_bytes) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = u32x4_t{0u, 0u, 0u, 0u};
  if (blockIdx.x == 0 && (int)threadIdx.x < tail_bytes) tail[threadIdx.x] = 0;
}

hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t st) {
  if (bytes <= 0) return hipSuccess;
  const int64_t nvec = bytes / 16;
  int64_t blocks = (nvec + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<u32x4_t*>(p), nvec,
                     static_cast<unsigned char*>(p) + nvec * 16, (int)(bytes - nvec * 16));
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void scale_cast_kernel(const void* src, int sdt, void* dst,
                                                         int ddt, int64_t n,
                                                         const float* scale) {
  const float s = scale ? scale[0] : 1.f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    store_as(dst, i, s * load_as(src, i, sdt), ddt);
}

// Eight elements per thread and iteration, moved as 16-byte vectors (two for
// fp32): the cast of a [V, H] fp32 dW to 16 bits is a pure streaming pass.
// Same arithmetic and rounding as scale_cast_kernel, element by element.
template <class TS, class TD>
__device__ __forceinline__ void load8(const typename TS::storage* p, float (&v)[8]) {
  if constexpr (sizeof(typename TS::storage) == 4) {
    const f32x4_t lo = reinterpret_cast<const f32x4_t*>(p)[0];
    const f32x4_t hi = reinterpret_cast<const f32x4_t*>(p)[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = lo[e], v[4 + e] = hi[e];
  } else {
    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = TS::to_f32((u16)(x[e] & 0xffffu));
      v[2 * e + 1] = TS::to_f32((u16)(x[e] >> 16));
    }
  }
}
template <class TS, class TD>
__global__ __launch_bounds__(256) void scale_cast8_kernel(const typename TS::storage* src,
                                                          typename TD::storage* dst,
                                                          int64_t n8, const float* scale) {
  const float s = scale ? scale[0] : 1.f;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    float v[8];
    load8<TS, TD>(src + i * 8, v);
    // scale * x is rounded to fp32 and then to the destination dtype, as in
    // the element-wise kernel.  The empty asm keeps the compiler from folding
    // product and conversion into one v_fma_mix (a single rounding to f16).
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] *= s;
      asm volatile("" : "+v"(v[e]));
    }
    if constexpr (sizeof(typename TD::storage) == 4) {
      f32x4_t* d = reinterpret_cast<f32x4_t*>(dst + i * 8);
      d[0] = f32x4_t{v[0], v[1], v[2], v[3]};
      d[1] = f32x4_t{v[4], v[5], v[6], v[7]};
    } else {
      u32x4_t o;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = (uint32_t)TD::from_f32(v[2 * e]) | ((uint32_t)TD::from_f32(v[2 * e + 1]) << 16);
      *reinterpret_cast<u32x4_t*>(dst + i * 8) = o;
    }
  }
}

template <class TS, class TD>
static void launch_cast8(const void* src, void* dst, int64_t n8, const float* scale,
                         hipStream_t st) {
  int64_t blocks = (n8 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL((scale_cast8_kernel<TS, TD>), dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const typename TS::storage*>(src),
                     static_cast<typename TD::storage*>(dst), n8, scale);
}
template <class TS>
static void launch_cast8_to(int ddt, const void* src, void* dst, int64_t n8, const float* scale,
                            hipStream_t st) {
  if (ddt == 0)
    launch_cast8<TS, F32>(src, dst, n8, scale, st);
  else if (ddt == 1)
    launch_cast8<TS, F16>(src, dst, n8, scale, st);
  else
    launch_cast8<TS, BF16>(src, dst, n8, scale, st);
}

hipError_t launch_scale_cast(const void* src, int src_dtype, void* dst, int dst_dtype,
                             int64_t n, const float* scale, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  // the 16-byte-vector body when both ends are 16-byte aligned, then the
  // remaining elements one by one
  int64_t done = 0;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 == 0) {
    const int64_t n8 = n / 8;
    if (n8 > 0) {
      if (src_dtype == 0)
        launch_cast8_to<F32>(dst_dtype, src, dst, n8, scale, st);
      else if (src_dtype == 1)
        launch_cast8_to<F16>(dst_dtype, src, dst, n8, scale, st);
      else
        launch_cast8_to<BF16>(dst_dtype, src, dst, n8, scale, st);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      done = n8 * 8;
    }
  }
  if (done == n) return hipSuccess;
  const int64_t rest = n - done;
  int64_t blocks = (rest + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  const size_t ss = src_dtype == 0 ? 4 : 2, ds = dst_dtype == 0 ? 4 : 2;
  hipLaunchKernelGGL(scale_cast_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const unsigned char*>(src) + done * ss, src_dtype,
                     static_cast<unsigned char*>(dst) + done * ds, dst_dtype, rest, scale);
  return hipGetLastError();
}

}  // namespace flce
