// The three per-chunk projections of fused linear cross-entropy as MFMA GEMMs
// for gfx950 (v0.8.3 commit bad6c3ec42, Summary: reusable logits, direct dX,
// direct dW; PR #1554, Summary: logits, grad_input and grad_weight GEMMs):
//
//   logits  Z[m, n]  = sum_k X[idx[m], k] * W[n, k]        (A K-contiguous, B K-contiguous)
//   dX      dX[idx[m], n] = s * sum_k G[m, k] * W[k, n]    (A K-contiguous, B N-contiguous)
//   dW      dW[m, n] (+)= s * sum_k G[k, m] * X[idx[k], n] (A M-contiguous, B N-contiguous)
//
// All three share one main loop: 128x128 block tiles, four waves of 64x64,
// 32x32 MFMA tiles, both operands staged through LDS in a k-contiguous layout
// so that each lane reads its MFMA fragment with one 16-byte LDS read.
// Operands that are contiguous along M or N in memory are transposed in
// registers (4 k-rows x one 16-byte vector) on their way into LDS.  Two LDS
// buffers: the next k-tile's global loads are in flight while the current
// tile is multiplied.
#include "flce_device.hpp"
#include "flce_internal.h"

namespace flce {

constexpr int BM = 128, BN = 128;
constexpr int WAVES_M = 2, WAVES_N = 2;
constexpr int NT = 64 * WAVES_M * WAVES_N;
constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // 64 x 64 per wave
constexpr int FM = WTM / 32, FN = WTN / 32;            // 2 x 2 MFMA tiles per wave

template <class T>
struct Tile {
  typedef typename T::storage S;
  static constexpr int BK = (sizeof(S) == 2) ? 64 : 32;
  static constexpr int LDK = BK + ((sizeof(S) == 2) ? 8 : 4);  // padded LDS row (elements)
  static constexpr int A_ELEMS = BM * LDK;
  static constexpr int B_ELEMS = BN * LDK;
  static constexpr size_t LDS_BYTES = 2 * (A_ELEMS + B_ELEMS) * sizeof(S);
};

// ---------------------------------------------------------------------------
// Operand tile loaders.  Each fills an R x BK tile of LDS laid out [R][LDK]
// (k contiguous).
// ---------------------------------------------------------------------------

// Source already k-contiguous: row r of the tile starts at rowp(r) (nullptr:
// a zero row).  Vectors whose first k is >= kend read as zero; callers keep
// kend a multiple of the vector width, and any element between the logical
// K and kend is zero in memory.
template <class T, int R>
struct KRowsLoader {
  typedef typename T::storage S;
  static constexpr int BK = Tile<T>::BK;
  static constexpr int VPR = BK / T::vec;
  static constexpr int NV = R * VPR / NT;
  static_assert((R * VPR) % NT == 0, "tile not divisible among threads");
  u32x4_t reg[NV];
  const S* ptr[NV];
  int kofs[NV];
  int lrow[NV];

  template <class RowFn>
  __device__ void init(int tid, RowFn rowp) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + i * NT;
      lrow[i] = v / VPR;
      kofs[i] = (v % VPR) * T::vec;
      ptr[i] = rowp(lrow[i]);
    }
  }
  __device__ void load(int k0, int kend) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int k = k0 + kofs[i];
      if (ptr[i] != nullptr && k < kend)
        reg[i] = *reinterpret_cast<const u32x4_t*>(ptr[i] + k);
      else
        reg[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  __device__ void store(S* lds) const {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      *reinterpret_cast<u32x4_t*>(lds + lrow[i] * Tile<T>::LDK + kofs[i]) = reg[i];
  }
};

// Source contiguous along the tile's row index: element (r, k) of the tile is
// kptr(k)[c0 + r], with kptr(k) == nullptr for a zero k-row and columns at or
// past cend reading as zero (vector granularity, as above).  Each thread moves
// 4 k-rows x one 16-byte vector and transposes them in registers.
template <class T, int R>
struct KColsLoader {
  typedef typename T::storage S;
  static constexpr int BK = Tile<T>::BK;
  static constexpr int CB = R / T::vec;   // column blocks
  static constexpr int KB = BK / 4;       // k blocks of 4 rows
  static constexpr int NB = CB * KB / NT; // blocks per thread
  static_assert((CB * KB) % NT == 0, "tile not divisible among threads");
  u32x4_t reg[NB][4];
  int cb[NB], kb[NB];

  __device__ void init(int tid) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int b = tid + i * NT;
      cb[i] = b % CB;
      kb[i] = b / CB;
    }
  }
  template <class KFn>
  __device__ void load(int k0, KFn kptr, int c0, int cend) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int c = c0 + cb[i] * T::vec;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const S* p = kptr(k0 + kb[i] * 4 + q);
        if (p != nullptr && c < cend)
          reg[i][q] = *reinterpret_cast<const u32x4_t*>(p + c);
        else
          reg[i][q] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ void store(S* lds) const {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      S* base = lds + (cb[i] * T::vec) * Tile<T>::LDK + kb[i] * 4;
      if constexpr (sizeof(S) == 2) {
        // reg[i][q] holds 8 columns of k-row q as 4 dwords (2 columns each).
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t r0 = reg[i][0][d], r1 = reg[i][1][d], r2 = reg[i][2][d], r3 = reg[i][3][d];
          // column 2d: low halves; column 2d+1: high halves
          u32x2_t lo, hi;
          lo[0] = (r0 & 0xffffu) | (r1 << 16);
          lo[1] = (r2 & 0xffffu) | (r3 << 16);
          hi[0] = (r0 >> 16) | (r1 & 0xffff0000u);
          hi[1] = (r2 >> 16) | (r3 & 0xffff0000u);
          *reinterpret_cast<u32x2_t*>(base + (2 * d) * Tile<T>::LDK) = lo;
          *reinterpret_cast<u32x2_t*>(base + (2 * d + 1) * Tile<T>::LDK) = hi;
        }
      } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          u32x4_t col;
          col[0] = reg[i][0][d];
          col[1] = reg[i][1][d];
          col[2] = reg[i][2][d];
          col[3] = reg[i][3][d];
          *reinterpret_cast<u32x4_t*>(base + d * Tile<T>::LDK) = col;
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// One BK-deep step of the wave's 64x64 tile from LDS.
// ---------------------------------------------------------------------------
template <class T>
__device__ __forceinline__ void mma_tile(const typename T::storage* As,
                                         const typename T::storage* Bs, int wm, int wn,
                                         int lane, f32x16_t (&acc)[FM][FN]) {
  constexpr int BK = Tile<T>::BK, LDK = Tile<T>::LDK;
  const int r32 = lane & 31, hk = lane >> 5;
#pragma unroll
  for (int s = 0; s < BK / T::kstep; ++s) {
    if constexpr (sizeof(typename T::storage) == 2) {
      u32x4_t fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        fa[i] = *reinterpret_cast<const u32x4_t*>(As + (wm * WTM + i * 32 + r32) * LDK +
                                                   s * 16 + hk * 8);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[j] = *reinterpret_cast<const u32x4_t*>(Bs + (wn * WTN + j * 32 + r32) * LDK +
                                                   s * 16 + hk * 8);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) T::mma(fa[i], fb[j], acc[i][j]);
    } else {
      float fa[FM], fb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[i] = As[(wm * WTM + i * 32 + r32) * LDK + s * 2 + hk];
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = Bs[(wn * WTN + j * 32 + r32) * LDK + s * 2 + hk];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) T::mma(fa[i], fb[j], acc[i][j]);
    }
  }
}

// Row / column of accumulator element r of MFMA tile (i, j) in the block tile
// (32x32 MFMA output layout: column = lane % 32; row = 8*(r/4) + 4*(lane/32) + r%4).
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) {
  return wn * WTN + j * 32 + (lane & 31);
}

__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[FM][FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// Upstream scale s for mean / sum (grad_output may be NULL = 1).
__device__ __forceinline__ float upstream_scale(const float* grad_output, float inv_n,
                                                int reduction) {
  if (reduction == 2) return 1.f;  // none: g_i is already inside G
  const float g = grad_output ? grad_output[0] : 1.f;
  return reduction == 0 ? g * inv_n : g;
}

// ---------------------------------------------------------------------------
// Logits: slab[m, n] = X[idx[m], :] . W[n, :], plus per-(row, 64-column block)
// running max and sum of exp, and the target logit in fp32.
// ---------------------------------------------------------------------------
template <class T>
__global__ __launch_bounds__(NT) void logits_kernel(LogitsArgs a) {
  typedef typename T::storage S;
  constexpr int BK = Tile<T>::BK;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  S* As = reinterpret_cast<S*>(smem_raw);
  S* Bs = As + 2 * Tile<T>::A_ELEMS;
  __shared__ int64_t tgt_s[BM];

  const int tiles_m = (a.rows + BM - 1) / BM;
  const int tiles_n = (int)((a.V + BN - 1) / BN);
  const int lin = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  const int tm = lin % tiles_m, tn = lin / tiles_m;  // M fastest: blocks sharing a W tile are adjacent
  const int m0 = tm * BM;
  const int64_t n0 = (int64_t)tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  const S* X = static_cast<const S*>(a.X);
  const S* W = static_cast<const S*>(a.W);
  for (int m = tid; m < BM; m += NT) {
    const int gm = m0 + m;
    tgt_s[m] = gm < a.rows ? a.targets[a.idx[gm]] : -1;
  }

  KRowsLoader<T, BM> la;
  KRowsLoader<T, BN> lb;
  la.init(tid, [&](int r) -> const S* {
    const int gm = m0 + r;
    return gm < a.rows ? X + (int64_t)a.idx[gm] * a.H : nullptr;
  });
  lb.init(tid, [&](int r) -> const S* {
    const int64_t gn = n0 + r;
    return gn < a.V ? W + gn * a.H : nullptr;
  });

  f32x16_t acc[FM][FN];
  zero_acc(acc);
  const int K = (int)a.H;
  const int nk = (K + BK - 1) / BK;
  la.load(0, K);
  lb.load(0, K);
  la.store(As);
  lb.store(Bs);
  __syncthreads();
  for (int t = 0; t < nk; ++t) {
    const int cur = t & 1;
    if (t + 1 < nk) {
      la.load((t + 1) * BK, K);
      lb.load((t + 1) * BK, K);
    }
    mma_tile<T>(As + cur * Tile<T>::A_ELEMS, Bs + cur * Tile<T>::B_ELEMS, wm, wn, lane, acc);
    if (t + 1 < nk) {
      la.store(As + (cur ^ 1) * Tile<T>::A_ELEMS);
      lb.store(Bs + (cur ^ 1) * Tile<T>::B_ELEMS);
    }
    __syncthreads();
  }

  // Epilogue.
  S* slab = static_cast<S*>(a.slab);
  const int64_t nblk0 = n0 + wn * WTN;  // first column of this wave's 64-column block
  const bool blk_live = nblk0 < a.V;
  const int64_t sidx = nblk0 / WTN;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = acc_row(wm, i, r, lane);
      const int gm = m0 + m;
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t gn = n0 + acc_col(wn, j, lane);
        if (gn < a.V) mx = fmaxf(mx, acc[i][j][r]);
      }
      mx = half_wave_max(mx);
      float se = 0.f;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t gn = n0 + acc_col(wn, j, lane);
        if (gn < a.V) se += __expf(acc[i][j][r] - mx);
      }
      se = half_wave_sum(se);
      if (gm < a.rows) {
        if ((lane & 31) == 0 && blk_live) {
          float2 st;
          st.x = mx;
          st.y = se;
          reinterpret_cast<float2*>(a.stats)[(int64_t)gm * a.stats_ld + sidx] = st;
        }
        const int64_t tg = tgt_s[m];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int64_t gn = n0 + acc_col(wn, j, lane);
          if (gn < a.V) {
            slab[(int64_t)gm * a.ldz + gn] = T::from_f32(acc[i][j][r]);
            if (gn == tg) a.ztgt[gm] = acc[i][j][r];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// grad_input: dX[idx[m], n] = s * sum_k G[m, k] W[k, n] over one split of k,
// or, with splits > 1, fp32 partials part[split][m][n] reduced afterwards.
// ---------------------------------------------------------------------------
template <class T>
__global__ __launch_bounds__(NT) void dx_kernel(DxArgs a) {
  typedef typename T::storage S;
  constexpr int BK = Tile<T>::BK;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  S* As = reinterpret_cast<S*>(smem_raw);
  S* Bs = As + 2 * Tile<T>::A_ELEMS;

  const int tiles_m = (a.rows + BM - 1) / BM;
  const int tiles_n = (int)((a.H + BN - 1) / BN);
  const int per_split = tiles_m * tiles_n;
  const int lin = xcd_remap(blockIdx.x, per_split * a.splits);
  const int split = lin / per_split;
  const int rem = lin % per_split;
  const int tm = rem % tiles_m, tn = rem / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  const int64_t kbeg = (int64_t)split * a.k_per_split;
  const int64_t kend = kbeg + a.k_per_split < a.ldz ? kbeg + a.k_per_split : a.ldz;
  const int64_t kend_w = kend < a.V ? kend : a.V;
  const S* G = static_cast<const S*>(a.slab);
  const S* W = static_cast<const S*>(a.W);
  const int H = (int)a.H;

  KRowsLoader<T, BM> la;
  KColsLoader<T, BN> lb;
  la.init(tid, [&](int r) -> const S* {
    const int gm = m0 + r;
    return gm < a.rows ? G + (int64_t)gm * a.ldz + kbeg : nullptr;
  });
  lb.init(tid);
  auto wrow = [&](int k) -> const S* {
    const int64_t gk = kbeg + k;
    return gk < kend_w ? W + gk * H : nullptr;
  };

  f32x16_t acc[FM][FN];
  zero_acc(acc);
  const int K = (int)(kend - kbeg);
  const int nk = (K + BK - 1) / BK;
  if (nk > 0) {
    la.load(0, K);
    lb.load(0, wrow, n0, H);
    la.store(As);
    lb.store(Bs);
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
      const int cur = t & 1;
      if (t + 1 < nk) {
        la.load((t + 1) * BK, K);
        lb.load((t + 1) * BK, wrow, n0, H);
      }
      mma_tile<T>(As + cur * Tile<T>::A_ELEMS, Bs + cur * Tile<T>::B_ELEMS, wm, wn, lane, acc);
      if (t + 1 < nk) {
        la.store(As + (cur ^ 1) * Tile<T>::A_ELEMS);
        lb.store(Bs + (cur ^ 1) * Tile<T>::B_ELEMS);
      }
      __syncthreads();
    }
  }

  if (a.splits == 1) {
    const float s = upstream_scale(a.grad_output, a.inv_n, a.reduction);
    S* dX = static_cast<S*>(a.dX);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gm = m0 + acc_row(wm, i, r, lane);
        if (gm >= a.rows) continue;
        const int64_t orow = (int64_t)a.idx[gm] * H;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int gn = n0 + acc_col(wn, j, lane);
          if (gn < H) dX[orow + gn] = T::from_f32(s * acc[i][j][r]);
        }
      }
  } else {
    float* part = a.partial + (int64_t)split * a.rows_cap * H;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gm = m0 + acc_row(wm, i, r, lane);
        if (gm >= a.rows) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int gn = n0 + acc_col(wn, j, lane);
          if (gn < H) part[(int64_t)gm * H + gn] = acc[i][j][r];
        }
      }
  }
}

// ---------------------------------------------------------------------------
// grad_weight: dW[m, n] = (dW[m, n] if accumulate) + s * sum_k G[k, m] X[idx[k], n]
// The accumulator starts at zero and the destination is read only in the
// epilogue, so no [V, H] temporary exists.
// ---------------------------------------------------------------------------
template <class T>
__global__ __launch_bounds__(NT) void dw_kernel(DwArgs a) {
  typedef typename T::storage S;
  constexpr int BK = Tile<T>::BK;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  S* As = reinterpret_cast<S*>(smem_raw);
  S* Bs = As + 2 * Tile<T>::A_ELEMS;

  const int tiles_m = (int)((a.V + BM - 1) / BM);
  const int tiles_n = (int)((a.H + BN - 1) / BN);
  const int lin = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  const int tn = lin % tiles_n, tm = lin / tiles_n;  // N fastest: blocks sharing a G tile are adjacent
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int H = (int)a.H;

  const S* G = static_cast<const S*>(a.slab);
  const S* X = static_cast<const S*>(a.X);
  KColsLoader<T, BM> la;
  KColsLoader<T, BN> lb;
  la.init(tid);
  lb.init(tid);
  auto grow = [&](int k) -> const S* { return k < a.rows ? G + (int64_t)k * a.ldz : nullptr; };
  auto xrow = [&](int k) -> const S* {
    return k < a.rows ? X + (int64_t)a.idx[k] * H : nullptr;
  };
  const int ldz_cols = (int)a.ldz;

  f32x16_t acc[FM][FN];
  zero_acc(acc);
  const int nk = (a.rows + BK - 1) / BK;
  la.load(0, grow, (int)m0, ldz_cols);
  lb.load(0, xrow, n0, H);
  la.store(As);
  lb.store(Bs);
  __syncthreads();
  for (int t = 0; t < nk; ++t) {
    const int cur = t & 1;
    if (t + 1 < nk) {
      la.load((t + 1) * BK, grow, (int)m0, ldz_cols);
      lb.load((t + 1) * BK, xrow, n0, H);
    }
    mma_tile<T>(As + cur * Tile<T>::A_ELEMS, Bs + cur * Tile<T>::B_ELEMS, wm, wn, lane, acc);
    if (t + 1 < nk) {
      la.store(As + (cur ^ 1) * Tile<T>::A_ELEMS);
      lb.store(Bs + (cur ^ 1) * Tile<T>::B_ELEMS);
    }
    __syncthreads();
  }

  const float s = upstream_scale(a.grad_output, a.inv_n, a.reduction);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t gm = m0 + acc_row(wm, i, r, lane);
      if (gm >= a.V) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int gn = n0 + acc_col(wn, j, lane);
        if (gn >= H) continue;
        const int64_t o = gm * H + gn;
        float v = s * acc[i][j][r];
        if (a.accumulate) v += load_as(a.dW, o, a.dw_dtype);
        store_as(a.dW, o, v, a.dw_dtype);
      }
    }
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
// The 72 KiB of LDS per workgroup is above the default dynamic limit; raise
// the limit once per kernel (gfx950 has 160 KiB of LDS per CU).
template <class K>
static hipError_t allow_lds(K kernel, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <class T>
static hipError_t launch_logits_t(const LogitsArgs& a, hipStream_t st) {
  static const hipError_t prep = allow_lds(logits_kernel<T>, Tile<T>::LDS_BYTES);
  if (prep != hipSuccess) return prep;
  const int tiles = ((a.rows + BM - 1) / BM) * (int)((a.V + BN - 1) / BN);
  hipLaunchKernelGGL(logits_kernel<T>, dim3(tiles), dim3(NT), Tile<T>::LDS_BYTES, st, a);
  return hipGetLastError();
}
template <class T>
static hipError_t launch_dx_t(const DxArgs& a, hipStream_t st) {
  static const hipError_t prep = allow_lds(dx_kernel<T>, Tile<T>::LDS_BYTES);
  if (prep != hipSuccess) return prep;
  const int tiles = ((a.rows + BM - 1) / BM) * (int)((a.H + BN - 1) / BN) * a.splits;
  hipLaunchKernelGGL(dx_kernel<T>, dim3(tiles), dim3(NT), Tile<T>::LDS_BYTES, st, a);
  return hipGetLastError();
}
template <class T>
static hipError_t launch_dw_t(const DwArgs& a, hipStream_t st) {
  static const hipError_t prep = allow_lds(dw_kernel<T>, Tile<T>::LDS_BYTES);
  if (prep != hipSuccess) return prep;
  const int tiles = (int)((a.V + BM - 1) / BM) * (int)((a.H + BN - 1) / BN);
  hipLaunchKernelGGL(dw_kernel<T>, dim3(tiles), dim3(NT), Tile<T>::LDS_BYTES, st, a);
  return hipGetLastError();
}

hipError_t launch_logits(int dtype, const LogitsArgs& a, hipStream_t st) {
  if (dtype == 0) return launch_logits_t<F32>(a, st);
  if (dtype == 1) return launch_logits_t<F16>(a, st);
  return launch_logits_t<BF16>(a, st);
}
hipError_t launch_dx(int dtype, const DxArgs& a, hipStream_t st) {
  if (dtype == 0) return launch_dx_t<F32>(a, st);
  if (dtype == 1) return launch_dx_t<F16>(a, st);
  return launch_dx_t<BF16>(a, st);
}
hipError_t launch_dw(int dtype, const DwArgs& a, hipStream_t st) {
  if (dtype == 0) return launch_dw_t<F32>(a, st);
  if (dtype == 1) return launch_dw_t<F16>(a, st);
  return launch_dw_t<BF16>(a, st);
}

int gemm_bk(int dtype) { return dtype == 0 ? Tile<F32>::BK : Tile<BF16>::BK; }
int stats_cols_per_block() { return WTN; }
int gemm_block_m() { return BM; }
int gemm_block_n() { return BN; }

}  // namespace flce
