// The three per-chunk projections of fused linear cross-entropy as MFMA GEMMs
// for gfx950 (v0.8.3 commit bad6c3ec42, Summary: reusable logits, direct dX,
// direct dW; PR #1554, Summary: logits, grad_input and grad_weight GEMMs):
//
//   logits  Z[m, n]  = sum_k X[idx[m], k] * W[n, k]        (A k-contiguous, B k-contiguous)
//   dX      dX[idx[m], n] = s * sum_k G[m, k] * W[k, n]    (A k-contiguous, B n-contiguous)
//   dW      dW[m, n] (+)= s * sum_k G[k, m] * Xc[k, n]     (A m-contiguous, B k-contiguous)
//
// One main loop serves all three.  Every operand tile goes from global memory
// straight into LDS (buffer_load ... lds, 16 bytes per lane), in the layout it
// has in memory: k-contiguous tiles as rows of k, m/n-contiguous tiles as
// rows of m/n, both with an XOR swizzle of their 16-byte chunks.  MFMA
// fragments are read with 16-byte LDS reads (k-contiguous tiles) or with two
// transposing 8-byte reads (m/n-contiguous tiles); the swizzles keep both
// kinds free of bank conflicts on gfx950's 64-bank LDS.  Two or three LDS
// stages per operand: later k-tiles stream in while the current one is
// multiplied, their loads spread over its MFMA k-steps.
//
// Tile shapes: 256x256 blocks (one workgroup per CU) of four 128x128 waves
// for fp32 operands and of eight 64x128 or 128x64 waves (two per SIMD) for
// 16-bit operands; for chunks of at most 128 rows with 16-bit operands,
// 128x128 logits blocks of eight 64x32 waves (two workgroups per CU),
// 128x256 grad_input blocks of eight 64x64 waves (one per CU) and 256x128
// grad_weight blocks of eight 64x64 waves (two per CU); 128x128 blocks of
// four 64x64 waves (two workgroups per CU) for the other small problems
// (fp32 with few rows, or fewer than 256 hidden units).
#include <type_traits>

#include "flce_device.hpp"
#include "flce_internal.h"

namespace flce {

// A tile shape: BM x BN outputs per workgroup of WAVES_M x WAVES_N waves,
// KBYTES bytes of k per LDS row of a k-contiguous operand tile (BK = KBYTES
// / element size), sized for WGS resident workgroups per CU.  A CU's four
// SIMDs then hold WAVES_PER_SIMD waves each, which caps a wave at 512 /
// WAVES_PER_SIMD registers.
template <int BM_, int BN_, int KBYTES_, int WGS_, int WAVES_M_ = 2, int WAVES_N_ = 2>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int KBYTES = KBYTES_, WGS = WGS_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int WAVES_PER_SIMD = WGS * WAVES_M * WAVES_N / 4;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  // Rows of waves whose accumulators one epilogue pass stages in LDS: two for
  // the 64-row waves of the eight-wave tiles (half the passes, so half the
  // load round trips of grad_weight's read-modify-write; with bf16 dW at chunk
  // 256 that is 1.69 -> 1.53 ms).
  static constexpr int EPI_WROWS = WAVES_M >= 4 ? 2 : 1;
  static constexpr int EPI_ROWS = EPI_WROWS * WTM;
};
typedef Cfg<256, 256, 128, 1> Big;         // 4 waves of 128 x 128 (fp32 operands)
typedef Cfg<256, 256, 128, 1, 4, 2> Big8M;  // 8 waves of 64 x 128 (16-bit logits, grad_weight)
typedef Cfg<256, 256, 128, 1, 2, 4> Big8N;  // 8 waves of 128 x 64 (16-bit grad_input)
typedef Cfg<128, 128, 128, 2> Small;        // 4 waves of 64 x 64, 2 workgroups per CU
typedef Cfg<128, 128, 128, 2, 2, 4> Small8; // 8 waves of 64 x 32, 2 workgroups per CU (16-bit logits, <= 128 rows)
typedef Cfg<128, 256, 128, 1, 2, 4> Mid8N;  // 8 waves of 64 x 64 (16-bit grad_input, <= 128 rows)
typedef Cfg<256, 128, 64, 2, 4, 2> Twin8M;  // 8 waves of 64 x 64, 2 workgroups per CU (16-bit grad_weight, <= 128 rows)

// LDS stages per operand (SA, SB) and the parts P each k-tile's loads are
// split into, per kernel and tile shape (measured on MI355X).  A tile is
// needed S - 1 iterations after its loads are issued, so a third stage
// doubles the time that operand's loads have to arrive; the parts spread a
// tile's loads over the k-steps of the previous tile's MFMA work.
template <class C> struct LogitsPipe { static constexpr int SA = 2, SB = 3, P = 2; };
template <> struct LogitsPipe<Big8M> { static constexpr int SA = 2, SB = 3, P = 1; };
template <> struct LogitsPipe<Small8> { static constexpr int SA = 2, SB = 3, P = 1; };
template <class C> struct DxPipe { static constexpr int SA = 3, SB = 2, P = 2; };
// grad_input with the eight-wave tile (chunks of more than 128 rows): three
// stages of G, two of W.  Measured interleaved against two of G and three of
// W: Llama shape chunk 2048 1.75 -> 1.68 ms per launch, chunk 256 247 -> 238
// us, H 5376 / V 262144 chunk 256 644 -> 627 us.
struct DxPipeG3 { static constexpr int SA = 3, SB = 2, P = 1; };
// grad_input of chunks of at most 128 rows: a 128-row tile, whose G stages
// are half the size, leaves room for four stages of the W stream.
template <> struct DxPipe<Mid8N> { static constexpr int SA = 2, SB = 4, P = 1; };
template <class C> struct DwPipe { static constexpr int SA = 2, SB = 3, P = 4; };
template <> struct DwPipe<Big8M> { static constexpr int SA = 3, SB = 2, P = 1; };
// grad_weight of chunks of at most 128 rows (16-bit operands): the k loop is
// a few k-tiles and the dW read-modify-write is the kernel; two workgroups
// per CU, each 72 KB of LDS (64-byte k rows, three stages of each operand),
// so that one's read-modify-write overlaps the other's loads and MFMAs.
// Masked SFT at chunk 128 (bf16 dW): 257 -> 242 us per launch, step 38.9 ->
// 38.0 ms; at chunk 256 no gain (fp32 dW) or a loss (bf16 dW, 1430 -> 1463 us),
// at chunk 2048 14 % slower.
template <> struct DwPipe<Twin8M> { static constexpr int SA = 3, SB = 3, P = 1; };

template <class T, class C>
struct KT {
  typedef typename T::storage S;
  static constexpr int BK = C::KBYTES / (int)sizeof(S);
  static constexpr int RB = C::KBYTES;
  static constexpr int STEPS = BK / T::kstep;  // MFMA k-steps per k-tile
};

// ---------------------------------------------------------------------------
// Global memory access.  Raw buffer loads: a wave-uniform descriptor (base,
// byte range) plus a 32-bit per-lane byte offset; any offset at or past the
// range reads as zero, which is how rows and columns outside the problem are
// masked (an out-of-range lane gets kOOB).
// ---------------------------------------------------------------------------
constexpr uint32_t kOOB = 0xfffffff0u;

// Buffer descriptor (V#) in four wave-uniform words: base address, stride 0,
// size in bytes (reads at or past it return zero), raw-buffer format flags.
typedef int32_t desc_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ desc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0x7ffffff0ull ? 0x7ffffff0u : (uint32_t)bytes;
  const uint64_t b = (uint64_t)(uintptr_t)base;
  desc_t d;
  d[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)b);
  d[1] = __builtin_amdgcn_readfirstlane((int32_t)((uint32_t)(b >> 32) & 0xffffu));
  d[2] = __builtin_amdgcn_readfirstlane((int32_t)n);
  d[3] = 0x00020000;
  return d;
}
// 16 bytes per lane straight into LDS: lane i of the wave writes lds + 16 i
// (M0 holds the wave's LDS base).  Issued from inline assembly on purpose:
// the compiler cannot tell these LDS writes apart from the fragment reads of
// the stage being multiplied, and would wait for every load in flight before
// those reads, serialising the pipeline.  The k loop's own wait (vmcnt, then
// a barrier) orders each stage's loads before its reads.
__device__ __forceinline__ void buf_load16_lds(desc_t r, uint32_t off, unsigned char* lds) {
  // A generic pointer into LDS is the LDS aperture base plus the LDS offset,
  // so its low 32 bits are the offset M0 wants.
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
               :
               : "v"(off), "s"(base), "s"(r)
               : "memory");
}

// Wait until at most `VM` vector-memory loads of this wave are outstanding
// and all its LDS operations are done, then meet the other waves.  A plain
// s_barrier: the workgroup fence of __syncthreads would also wait for the
// loads still streaming into the other LDS buffers.
template <int VM>
__device__ __forceinline__ void wait_and_barrier() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  constexpr int imm = (VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(imm);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// LDS layouts of an operand tile, both filled straight from global memory in
// 16-byte chunks and both read as MFMA fragments without bank conflicts.
//
// RowSwz: R rows x BK (k contiguous), rows of RB bytes, unpadded; the 16-byte
//   chunk index is XORed with a function of the row so that the 16 lanes
//   reading one k-chunk of 16 consecutive rows hit 16 distinct 16-byte slots.
// ColSwz: BK k-rows x R (m or n contiguous, as in memory), rows of R * s
//   bytes, chunk index XORed with a function of k.  A 16-bit
//   fragment (8 consecutive k of one column per lane) is gathered with two
//   transposing reads (ds_read_b64_tr_b16): within each group of 16 lanes,
//   lane q points at 4 elements of row k0 + q / 4, columns c0 + 4 (q % 4), and
//   lane l then receives rows k0..k0+3 of column c0 + l.  The XOR puts the 4
//   rows' 64-byte pieces (two lane groups) in distinct bank groups.  fp32
//   fragments are single elements and need no transpose.
// frag16(b, c, s, lane): the 16-bit fragment of tile row/column c for k-step
//   s; frag4(b, c, k): the fp32 element (c, k).
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(4))) short v4i16_t;

template <class T, int RB_>
struct RowSwz {
  typedef typename T::storage S;
  static constexpr int RB = RB_;
  static_assert(RB == 64 || RB == 128, "row swizzle assumes 64- or 128-byte rows");
  static constexpr size_t bytes(int R) { return (size_t)R * RB; }
  // LDS serves 256 bytes per cycle (64 banks): the 16 rows read by 16
  // consecutive lanes must land in 16 distinct 16-byte slots of that window.
  // 128-byte rows: chunk ^= (r / 2) % 8; 64-byte rows: chunk ^= (r / 4) % 4.
  __device__ __forceinline__ static int swz(int r) { return RB == 128 ? ((r >> 1) & 7) : ((r >> 2) & 3); }
  // Rows per 16-bit fragment read: 32 for 32x32x16 MFMAs, 16 for 16x16x32.
  static constexpr int FRAG_ROWS = T::sub16 ? 16 : 32;
  // 16-bit fragment of row r for k-step s: lane l takes the 16-byte chunk
  // 2 s + l / 32 (32x32x16) or 4 s + l / 16 (16x16x32), 8 consecutive k.
  __device__ __forceinline__ static u32x4_t frag16(const unsigned char* b, int r, int s, int lane) {
    const int kc = T::sub16 ? 4 * s + (lane >> 4) : 2 * s + (lane >> 5);
    return *reinterpret_cast<const u32x4_t*>(b + r * RB + ((kc ^ swz(r)) << 4));
  }
  __device__ __forceinline__ static float frag4(const unsigned char* b, int r, int k) {
    return reinterpret_cast<const float*>(b + r * RB + (((k >> 2) ^ swz(r)) << 4))[k & 3];
  }
};

template <class T, int R, int BK>
struct ColSwz {
  typedef typename T::storage S;
  static constexpr int RBT = R * (int)sizeof(S);  // bytes per k-row
  static constexpr int EPC = 16 / (int)sizeof(S); // elements per 16-byte chunk
  static constexpr size_t bytes(int) { return (size_t)BK * RBT; }
  // 16-bit: the 4 k-rows of one transposing read move by 64 bytes each
  // (chunk ^= 4 (k % 4)); for 16x16x32 fragments, whose second lane group
  // reads k-rows 8 further on in the same pass, those move by another 32
  // bytes (chunk ^= 2 ((k / 8) % 2)).  fp32: odd k-rows move by 128 bytes
  // (chunk ^= 8 (k % 2)).
  static_assert(RBT >= 256, "column swizzle needs 16 chunks per k-row");
  __device__ __forceinline__ static int swz(int k) {
    if constexpr (sizeof(S) == 4) return 8 * (k & 1);
    return T::sub16 ? (4 * (k & 3)) ^ (2 * ((k >> 3) & 1)) : 4 * (k & 3);
  }
  __device__ __forceinline__ static const unsigned char* at(const unsigned char* b, int k, int c) {
    return b + k * RBT + (((c / EPC) ^ swz(k)) << 4) + (c % EPC) * (int)sizeof(S);
  }
  // c: first column of the MFMA block (32 columns for 32x32x16, 16 for
  // 16x16x32).  32x32x16: lanes 16-31 take the block's second 16 columns and
  // lanes 32-63 k-rows 8 further on; 16x16x32: lane group g = l / 16 gathers
  // k-rows 32 s + 8 g + 0..7.
  __device__ __forceinline__ static u32x4_t frag16(const unsigned char* b, int c, int s, int lane) {
    const int q = lane & 15;
    const int col = T::sub16 ? c + 4 * (q & 3) : c + 16 * ((lane >> 4) & 1) + 4 * (q & 3);
    const int k1 = T::sub16 ? 32 * s + 8 * (lane >> 4) + (q >> 2) : 16 * s + 8 * (lane >> 5) + (q >> 2);
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16_t*)at(b, k1, col));
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16_t*)at(b, k1 + 4, col));
    const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
    return u32x4_t{l2[0], l2[1], h2[0], h2[1]};
  }
  __device__ __forceinline__ static float frag4(const unsigned char* b, int c, int k) {
    return *reinterpret_cast<const float*>(at(b, k, c));
  }
};

// ---------------------------------------------------------------------------
// Operand tile loaders: each wave instruction moves 1 KiB (64 lanes x 16
// bytes) from global memory into consecutive LDS bytes.
// ---------------------------------------------------------------------------

// k-contiguous source into a RowSwz tile.  Tile row r starts at byte offset
// rowoff(r) (kOOB: zero row) of the descriptor.  An instruction fills RPI =
// 1024 / RB rows: lane L takes row L / CPR of its group and physical chunk
// L % CPR, i.e. k-chunk (L % CPR) ^ swz(row).  Chunks whose first k is >=
// kend read as zero; callers keep kend a multiple of the chunk width, and
// elements between the logical K and kend are zero in memory.
template <class T, class C, int R>
struct DmaRows {
  typedef RowSwz<T, C::KBYTES> Layout;
  typedef typename T::storage S;
  static constexpr int NWAVES = C::NT / 64;
  static constexpr int CPR = C::KBYTES / 16;
  static constexpr int RPI = 1024 / C::KBYTES;
  static constexpr int NI = R / RPI / NWAVES;  // instructions per wave per k-tile
  static_assert(R % (RPI * NWAVES) == 0, "tile rows not divisible among waves");
  static constexpr size_t TILE_BYTES = Layout::bytes(R);
  uint32_t roff[NI];
  int kc_el[NI];  // first k (elements) of this lane's chunk in each instruction
  int wave;

  template <class RowFn>
  __device__ __forceinline__ void init(int tid, RowFn rowoff) {
    const int lane = tid & 63;
    wave = tid >> 6;
    const int rin = lane / CPR;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = (wave + i * NWAVES) * RPI + rin;
      roff[i] = rowoff(row);
      kc_el[i] = ((lane % CPR) ^ Layout::swz(row)) * T::vec;
    }
  }
  // Rows found through a table: read(row) reads the table entry of every
  // row this lane loads, all reads in flight together, then off(row, entry)
  // turns each entry into the row's byte offset.
  template <class ReadFn, class OffFn>
  __device__ __forceinline__ void init_indexed(int tid, ReadFn read, OffFn off) {
    const int lane = tid & 63;
    wave = tid >> 6;
    const int rin = lane / CPR;
    uint32_t e[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) e[i] = read((wave + i * NWAVES) * RPI + rin);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      asm volatile("" : "+v"(e[i]));  // the reads stay unconditional and together
      const int row = (wave + i * NWAVES) * RPI + rin;
      roff[i] = off(row, e[i]);
      kc_el[i] = ((lane % CPR) ^ Layout::swz(row)) * T::vec;
    }
  }
  // Part `part` of P: the instructions i with i * P / NI == part (P parts
  // spread the tile's loads over the P k-steps of the previous tile).
  template <int P>
  __device__ __forceinline__ void issue(desc_t rs, unsigned char* tile, int k0, int kend,
                                        int part) const {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i * P / NI != part) continue;
      const int k = k0 + kc_el[i];
      buf_load16_lds(rs,
                     (k < kend && roff[i] != kOOB) ? roff[i] + (uint32_t)k * (uint32_t)sizeof(S)
                                                   : kOOB,
                     tile + (wave + i * NWAVES) * 1024);
    }
  }
};

// Source contiguous along the tile's columns into a ColSwz tile: tile element
// (k, c) sits at byte offset rowoff(k) + (c0 + c) * sizeof(S) of the
// descriptor, rowoff(k) == kOOB for a zero k-row; columns at or past cend
// read as zero (chunk granularity).  An instruction fills RPI = 1024 / (R *
// s) k-rows; lane L takes k-row L / CPRT of its group and physical chunk
// L % CPRT.
template <class T, class C, int R>
struct DmaCols {
  typedef ColSwz<T, R, KT<T, C>::BK> Layout;
  typedef typename T::storage S;
  static constexpr int NWAVES = C::NT / 64;
  static constexpr int BK = KT<T, C>::BK;
  static constexpr int RBT = Layout::RBT;
  static_assert(RBT <= 1024 && 1024 % RBT == 0, "k-row must divide 1 KiB");
  static constexpr int CPRT = RBT / 16;
  static constexpr int RPI = 1024 / RBT;
  static constexpr int NI = BK / RPI / NWAVES;
  static_assert(BK % (RPI * NWAVES) == 0, "k-rows not divisible among waves");
  static constexpr size_t TILE_BYTES = Layout::bytes(R);
  int krow[NI];      // k-row within the tile of each instruction
  uint32_t cofs[NI]; // byte offset of this lane's column chunk (kOOB: outside)
  int wave;

  __device__ __forceinline__ void init(int tid, int c0, int cend) {
    const int lane = tid & 63;
    wave = tid >> 6;
    const int rin = lane / CPRT, p = lane % CPRT;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      krow[i] = (wave + i * NWAVES) * RPI + rin;
      const int c = c0 + (p ^ Layout::swz(krow[i])) * Layout::EPC;
      cofs[i] = c < cend ? (uint32_t)c * (uint32_t)sizeof(S) : kOOB;
    }
  }
  template <int P, class KFn>
  __device__ __forceinline__ void issue(desc_t rs, unsigned char* tile, int k0, KFn rowoff,
                                        int part) const {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i * P / NI != part) continue;
      const uint32_t ro = rowoff(k0 + krow[i]);
      buf_load16_lds(rs, (ro != kOOB && cofs[i] != kOOB) ? ro + cofs[i] : kOOB,
                     tile + (wave + i * NWAVES) * 1024);
    }
  }
};

// Dynamic LDS of a kernel: SA stages of the A tile and SB of the B tile,
// or, after the main loop, the epilogue's staging area (EPI_ROWS x (BN + 4)
// fp32) plus EXTRA bytes, whichever is larger.
template <class C, class OA, class OB, int SA, int SB, size_t EXTRA = 0>
struct Smem {
  static_assert(SA >= 2 && SB >= 2, "at least two stages per operand");
  static constexpr size_t B_OFS = (size_t)SA * OA::TILE_BYTES;
  static constexpr size_t OPERANDS = B_OFS + (size_t)SB * OB::TILE_BYTES;
  static constexpr size_t EPI = (size_t)C::EPI_ROWS * (C::BN + 4) * sizeof(float);
  static constexpr size_t EPI_ALL = EPI + EXTRA;
  static constexpr size_t BYTES = OPERANDS > EPI_ALL ? OPERANDS : EPI_ALL;
  static_assert(BYTES * C::WGS <= 160 * 1024, "gfx950 LDS per CU");
};

// Fragment address helpers: a RowSwz operand is addressed by its row, a
// ColSwz operand by the first column of the MFMA block (32 or 16 wide).
template <class L> struct IsCol { static constexpr bool value = false; };
template <class T, int R, int BK> struct IsCol<ColSwz<T, R, BK>> { static constexpr bool value = true; };

template <class L>
__device__ __forceinline__ u32x4_t frag16_of(const unsigned char* b, int blk, int s, int lane) {
  if constexpr (IsCol<L>::value)
    return L::frag16(b, blk, s, lane);
  else
    return L::frag16(b, blk + (lane & (L::FRAG_ROWS - 1)), s, lane);
}
template <class L>
__device__ __forceinline__ float frag4_of(const unsigned char* b, int blk, int s, int lane) {
  return L::frag4(b, blk + (lane & 31), 2 * s + (lane >> 5));
}

// ---------------------------------------------------------------------------
// One k-tile of the wave's tile from LDS.  With 32x32 MFMAs fragments are
// double buffered across the k-steps: the LDS reads of step s+1 are issued
// before the MFMAs of step s, and the interleave is pinned for the
// scheduler.  With 16x16x32 MFMAs (Mfma16) each step reads its own
// fragments first.
// Consecutive MFMAs share an operand fragment where they can: the blocks of
// a wave row run in serpentine order, and 16x16 sub-blocks alternate their
// order, so the multipliers' inputs change on one side only.  Under the
// power limit that is worth a little clock: interleaved on MI355X, the Llama
// shape at chunk 2048 23.21 -> 23.13 and 23.22 -> 23.11 ms per step, logits
// and grad_input 0.5-1.6 % faster, grad_weight unchanged.
// ---------------------------------------------------------------------------
// Scheduling groups: NR LDS reads (mask 0x100) spread evenly between NM
// MFMAs (mask 0x008), read q followed by its share of MFMAs.
template <int NR, int NM, int Q = 0>
struct PinInterleave {
  __device__ __forceinline__ static void run() {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    constexpr int m = (NM * (Q + 1)) / NR - (NM * Q) / NR;
    if constexpr (m > 0) __builtin_amdgcn_sched_group_barrier(0x008, m, 0);
    PinInterleave<NR, NM, Q + 1>::run();
  }
};
template <int NR, int NM>
struct PinInterleave<NR, NM, NR> {
  __device__ __forceinline__ static void run() {}
};

template <class T, class C, class LA, class LB, class DMA>
__device__ __forceinline__ void mma_tile(const unsigned char* Ab, const unsigned char* Bb,
                                         int wm, int wn, int lane,
                                         f32x16_t (&acc)[C::FM][C::FN], DMA dma) {
  constexpr int STEPS = KT<T, C>::STEPS;
  if constexpr (T::sub16) {
    // 16x16x32 MFMAs: each 32x32 accumulator block is four 16x16 sub-blocks
    // and a k-step covers 32 k.  A step's fragments (one 16-byte read per 16
    // rows of a RowSwz operand, two transposing reads per 16 columns of a
    // ColSwz one) are read at its start: double buffering them across steps
    // needs twice the registers, and with the reads and MFMAs interleaved by
    // the same pinning as below it was 7 % slower (grad_input at chunk 2048,
    // 1632 -> 1861 us per launch); double buffering one operand and reading
    // the other in halves, pinned, was 8 % slower (1622 -> 1750 us).
    u32x4_t fa[C::FM][2], fb[C::FN][2];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) fa[i][h] = frag16_of<LA>(Ab, wm * C::WTM + i * 32 + h * 16, s, lane);
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) fb[j][h] = frag16_of<LB>(Bb, wn * C::WTN + j * 32 + h * 16, s, lane);
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < C::FN; ++jj) {
          const int j = (i & 1) ? C::FN - 1 - jj : jj;
          if (((i * C::FN + jj) & 1) == 0) {
            T::template mma16<0>(fa[i][0], fb[j][0], acc[i][j]);
            T::template mma16<1>(fa[i][0], fb[j][1], acc[i][j]);
            T::template mma16<3>(fa[i][1], fb[j][1], acc[i][j]);
            T::template mma16<2>(fa[i][1], fb[j][0], acc[i][j]);
          } else {
            T::template mma16<2>(fa[i][1], fb[j][0], acc[i][j]);
            T::template mma16<3>(fa[i][1], fb[j][1], acc[i][j]);
            T::template mma16<1>(fa[i][0], fb[j][1], acc[i][j]);
            T::template mma16<0>(fa[i][0], fb[j][0], acc[i][j]);
          }
        }
      dma(s);
    }
  } else if constexpr (sizeof(typename T::storage) == 2) {
    u32x4_t fa[2][C::FM], fb[2][C::FN];
    auto fetch = [&](int buf, int s) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i) fa[buf][i] = frag16_of<LA>(Ab, wm * C::WTM + i * 32, s, lane);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) fb[buf][j] = frag16_of<LB>(Bb, wn * C::WTN + j * 32, s, lane);
    };
    fetch(0, 0);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      if (s + 1 < STEPS) fetch((s + 1) & 1, s + 1);
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int jj = 0; jj < C::FN; ++jj) {
          const int j = (i & 1) ? C::FN - 1 - jj : jj;
          T::mma(fa[s & 1][i], fb[s & 1][j], acc[i][j]);
        }
      dma(s);
    }
    // reads per step: one per RowSwz fragment, two per ColSwz fragment
    constexpr int NR = C::FM * (IsCol<LA>::value ? 2 : 1) + C::FN * (IsCol<LB>::value ? 2 : 1);
    constexpr int NM = C::FM * C::FN;
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
    for (int s = 0; s + 1 < STEPS; ++s) PinInterleave<NR, NM>::run();
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
  } else {
    float fa[2][C::FM], fb[2][C::FN];
    auto fetch = [&](int buf, int s) {
#pragma unroll
      for (int i = 0; i < C::FM; ++i) fa[buf][i] = frag4_of<LA>(Ab, wm * C::WTM + i * 32, s, lane);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) fb[buf][j] = frag4_of<LB>(Bb, wn * C::WTN + j * 32, s, lane);
    };
    fetch(0, 0);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      if (s + 1 < STEPS) fetch((s + 1) & 1, s + 1);
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) T::mma(fa[s & 1][i], fb[s & 1][j], acc[i][j]);
      dma(s);
    }
  }
}

// The k loop shared by the three kernels.  Operand X's k-tile j lives in
// its stage j % SX and is loaded LX = SX - 1 iterations before it is
// multiplied: iteration i issues A's tile i + LA and B's tile i + LB, into
// the stages of tile i - 1, the operand with the shorter lead first.  The
// loads are spread over the k-steps of the MFMA work (part s after step s;
// with one part, the near operand's after the first step and the far one's
// after the middle one), so that no wave stalls on a burst of loads queued
// behind the other waves' before its first MFMA.  Tiles past the end are
// issued too, as loads that read zeros into a free stage, which keeps the
// loop body branch-free.  Each iteration first waits until this wave's
// loads of tile t are done (vector loads complete in issue order, so it
// waits until no more than the loads issued after them are outstanding) and
// meets the other waves, so that every wave's loads of tile t have landed
// and every wave has finished tile t - 1.
//   ia(tile, k0, part) / ib(tile, k0, part): issue part `part` (of the
//   k-steps per tile) of operand A's / B's k-tile at k0 into `tile`; a k0 at
//   or past the end reads zeros.
template <class T, class C, class OA, class OB, int SA, int SB, int P, class IA, class IB>
__device__ __forceinline__ void main_loop(IA ia, IB ib, int nk, unsigned char* smem, int wm, int wn,
                                          int lane, f32x16_t (&acc)[C::FM][C::FN]) {
  typedef typename OA::Layout LA_;
  typedef typename OB::Layout LB_;
  typedef Smem<C, OA, OB, SA, SB> SM;
  constexpr int BK = KT<T, C>::BK;
  constexpr int STEPS = KT<T, C>::STEPS;
  static_assert(P >= 1 && STEPS % P == 0, "parts must divide the k-steps");
  constexpr int LA = SA - 1, LB = SB - 1;
  constexpr int LEAD = LA > LB ? LA : LB;
  constexpr int PER_IT = OA::NI + OB::NI;
  // Loads issued after the later of A's and B's tile t.  Each iteration
  // issues its loads in P parts, each part the near operand's share and then
  // the far operand's, so after the near operand's last part only the far
  // operand's last part follows within that iteration.
  // instructions in part P - 1: i with i * P / NI == P - 1, i.e. i >= ceil((P - 1) NI / P)
  constexpr int LAST_A = OA::NI - ((P - 1) * OA::NI + P - 1) / P;
  constexpr int LAST_B = OB::NI - ((P - 1) * OB::NI + P - 1) / P;
  constexpr int AFTER = LA == LB ? (LA - 1) * PER_IT
                        : LA > LB ? LAST_A + (LB - 1) * PER_IT
                                  : LAST_B + (LA - 1) * PER_IT;
  static_assert(AFTER < 64, "vmcnt range");
  auto tile_a = [&](int j) { return smem + (j % SA) * OA::TILE_BYTES; };
  auto tile_b = [&](int j) { return smem + SM::B_OFS + (j % SB) * OB::TILE_BYTES; };
  // part `part` of iteration i's loads of the near (shorter-lead) operand
  // (far = 0) or of the far one (far = 1)
  auto issue_op = [&](int i, int part, int far) {
    const int ja = i + LA, jb = i + LB;
    if ((LA <= LB) == (far == 0)) {
      if (ja >= 0) ia(tile_a(ja), ja * BK, part);
    } else {
      if (jb >= 0) ib(tile_b(jb), jb * BK, part);
    }
  };
  auto issue = [&](int i, int part) {  // part of the loads of iteration i, near operand first
    issue_op(i, part, 0);
    issue_op(i, part, 1);
  };
  if (nk <= 0) return;
#pragma unroll
  for (int i = -LEAD; i < 0; ++i)
#pragma unroll
    for (int p = 0; p < P; ++p) issue(i, p);
  for (int t = 0; t < nk; ++t) {
    if (AFTER > 0 && t - 1 + LEAD < nk)
      wait_and_barrier<AFTER>();
    else
      wait_and_barrier<0>();
    mma_tile<T, C, LA_, LB_>(tile_a(t), tile_b(t), wm, wn, lane, acc, [&](int s) {
      if constexpr (P == 1 && LA != LB) {
        // One part per tile (the eight-wave tiles): the near operand's loads,
        // which have one iteration to land, after the first k-step; the far
        // operand's, which have two, after the middle one.  Splitting the burst
        // keeps both waves of a SIMD from stalling on it together (Llama shape,
        // chunk 2048: step 24.75 -> 24.16 ms, grad_weight 2.30 -> 2.17 ms).
        if (s == 0) issue_op(t, 0, 0);
        if (s == STEPS / 2) issue_op(t, 0, 1);
      } else if (s % (STEPS / P) == 0) {
        issue(t, s / (STEPS / P));
      }
    });
  }
  wait_and_barrier<0>();
}

// Row and column, within its 32x32 accumulator block, of element r of this
// lane's accumulators: four 16x16 sub-blocks for 16x16x32 MFMAs (SUB16),
// the 32x32 layout otherwise.
template <bool SUB16>
__device__ __forceinline__ int acc_row(int r, int lane) {
  return SUB16 ? 16 * (r >> 3) + 4 * ((lane >> 4) & 3) + (r & 3) : 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
template <bool SUB16>
__device__ __forceinline__ int acc_col(int r, int lane) {
  return SUB16 ? 16 * ((r >> 2) & 1) + (lane & 15) : (lane & 31);
}

template <class C>
__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[C::FM][C::FN]) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// Epilogue through LDS.  After the main loop the operand buffers are free;
// each pass writes the accumulators of EPI_WROWS rows of waves (EPI_ROWS x BN
// fp32) there in fully unrolled code (32x32 MFMA output layout: element r of
// a lane sits at column lane % 32, row 8*(r/4) + 4*(lane/32) + r%4 of its
// 32x32 tile), then every thread walks 8-column pieces of those rows:
// fn(block_row, block_col, v[8]).  Consecutive lanes take consecutive pieces
// of a row, so 8 aligned lanes cover one 64-column block and global accesses
// are 16-byte vectors.  Every lane of every wave runs the same number of
// pieces, so fn may use cross-lane operations within groups of 8 lanes.
template <class C>
struct Stage {
  static constexpr int LS = C::BN + 4;  // staged row stride in floats (16-byte pad)
  static constexpr int SUBS = C::BN / 8;
  static constexpr int WR = C::EPI_WROWS, ROWS = C::EPI_ROWS, PASSES = C::WAVES_M / WR;
  static constexpr int NQ = ROWS * SUBS / C::NT;  // pieces per thread per pass
  static_assert(C::WAVES_M % WR == 0, "whole passes");
  static_assert((ROWS * SUBS) % C::NT == 0, "uniform piece count per lane");
};

template <class C, bool SUB16, class Fn>
__device__ __forceinline__ void staged_epilogue(float* stage, const f32x16_t (&acc)[C::FM][C::FN],
                                                int wm, int wn, int lane, int tid, Fn fn) {
  typedef Stage<C> ST;
  constexpr int LS = ST::LS, SUBS = ST::SUBS;
  for (int p = 0; p < ST::PASSES; ++p) {
    __syncthreads();
    if (wm / ST::WR == p) {
      const int r0 = (wm % ST::WR) * C::WTM;
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = r0 + i * 32 + acc_row<SUB16>(r, lane);
            const int col = wn * C::WTN + j * 32 + acc_col<SUB16>(r, lane);
            stage[row * LS + col] = acc[i][j][r];
          }
    }
    __syncthreads();
    // Fully unrolled, so that the pieces' cross-lane reductions and stores
    // overlap instead of running as one dependent chain per piece.
    constexpr int NQ = ST::NQ;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int q = tid + i * C::NT;
      const int lrow = q / SUBS, piece = q % SUBS;
      const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(stage + lrow * LS + piece * 8);
      const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(stage + lrow * LS + piece * 8 + 4);
      float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      fn(p * ST::ROWS + lrow, piece * 8, v);
    }
  }
}

// Pack 8 floats into one 16-byte vector of the storage type.
template <class T>
__device__ __forceinline__ u32x4_t pack8(const float (&v)[8]) {
  u32x4_t o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (std::is_same<typename T::base, BF16>::value)
      o[e] = f32x2_to_bf16x2(v[2 * e], v[2 * e + 1]);
    else
      o[e] = (uint32_t)T::from_f32(v[2 * e]) | ((uint32_t)T::from_f32(v[2 * e + 1]) << 16);
  }
  return o;
}
template <class T>
__device__ __forceinline__ void unpack8(const u32x4_t& x, float (&v)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = T::to_f32((u16)(x[e] & 0xffffu));
    v[2 * e + 1] = T::to_f32((u16)(x[e] >> 16));
  }
}

// Store 8 consecutive values (16-bit: one 16-byte store; fp32: two).
template <class T>
__device__ __forceinline__ void store8(typename T::storage* p, const float (&v)[8]) {
  if constexpr (sizeof(typename T::storage) == 2) {
    *reinterpret_cast<u32x4_t*>(p) = pack8<T>(v);
  } else {
    *reinterpret_cast<f32x4_t*>(p) = f32x4_t{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4_t*>(p + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
  }
}

// Reductions over 8 aligned lanes with DPP moves (no LDS traffic): swap
// neighbours (quad_perm [1,0,3,2]), swap pairs (quad_perm [2,3,0,1]), then
// mirror within each half-row of 8 lanes (row_half_mirror), which pairs
// every lane of one quad with a lane of the other.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
constexpr int kDppSwap1 = 0xb1, kDppSwap2 = 0x4e, kDppHalfMirror = 0x141;

__device__ __forceinline__ float group8_max(float v) {
  v = fmaxf(v, dpp_f<kDppSwap1>(v));
  v = fmaxf(v, dpp_f<kDppSwap2>(v));
  return fmaxf(v, dpp_f<kDppHalfMirror>(v));
}
// Maximum over 8 aligned lanes with the lowest column holding it; a lane
// whose columns are all outside the matrix carries (-inf, INT_MAX).
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& col) {
  const float ov = dpp_f<CTRL>(v);
  const int oc = dpp_i<CTRL>(col);
  if (ov > v || (ov == v && oc < col)) {
    v = ov;
    col = oc;
  }
}
__device__ __forceinline__ void group8_argmax(float& v, int& col) {
  argmax_step<kDppSwap1>(v, col);
  argmax_step<kDppSwap2>(v, col);
  argmax_step<kDppHalfMirror>(v, col);
}
__device__ __forceinline__ float group8_sum(float v) {
  v += dpp_f<kDppSwap1>(v);
  v += dpp_f<kDppSwap2>(v);
  return v + dpp_f<kDppHalfMirror>(v);
}

// Upstream scale s for mean / sum (grad_output may be NULL = 1).
__device__ __forceinline__ float upstream_scale(const float* grad_output, float inv_n,
                                                int reduction) {
  if (reduction == 2) return 1.f;  // none: g_i is already inside G
  const float g = grad_output ? grad_output[0] : 1.f;
  return reduction == 0 ? g * inv_n : g;
}

// Tile coordinates of linear block id `lin` in a grid of `nr` x `nc` tiles,
// walked in groups of `g` tile rows: within a group the row index varies
// fastest, so consecutive blocks (which run together on one XCD) share
// column tiles, and a group covers every column before the next begins.
__device__ __forceinline__ void grouped_tile(int lin, int nr, int nc, int g, int& tr, int& tc) {
  const int per_group = g * nc;
  const int grp = lin / per_group;
  const int first = grp * g;
  const int gsz = nr - first < g ? nr - first : g;
  const int r = lin - grp * per_group;
  tr = first + r % gsz;
  tc = r / gsz;
}
constexpr int kLogitsGroupM = 4, kDxGroupM = 4, kDwGroupN = 8;

// ---------------------------------------------------------------------------
// Logits: slab[m, n] = X[idx[m], :] . W[n, :], plus per-(row, wave column
// block) running max and sum of exp, and the target logit in fp32.
// ---------------------------------------------------------------------------
template <class T, class C>
__global__ __launch_bounds__(C::NT, C::WAVES_PER_SIMD) void logits_kernel(LogitsArgs a) {
  typedef typename T::storage S;
  typedef DmaRows<T, C, C::BM> OA;
  typedef DmaRows<T, C, C::BN> OB;
  typedef LogitsPipe<C> PI;
  typedef Smem<C, OA, OB, PI::SA, PI::SB, C::BM * sizeof(int64_t)> SM;
  extern __shared__ __align__(16) unsigned char smem_raw[];

  const int tiles_m = (a.rows + C::BM - 1) / C::BM;
  const int tiles_n = (int)((a.V + C::BN - 1) / C::BN);
  const int lin = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  int tm, tn;  // M fastest within a group: blocks sharing a W tile are adjacent
  grouped_tile(lin, tiles_m, tiles_n, kLogitsGroupM, tm, tn);
  const int m0 = tm * C::BM;
  const int64_t n0 = (int64_t)tn * C::BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

  const S* X = static_cast<const S*>(a.X);
  const S* W = static_cast<const S*>(a.W);

  // X: gathered rows anywhere in [BT, H] (one 32-bit range over all of X),
  // or, when X is larger than that, the chunk's rows gathered beforehand
  // into [rows, H]; W: this tile's rows [n0, n0 + BN).
  const uint32_t row_bytes = (uint32_t)a.H * (uint32_t)sizeof(S);
  const desc_t xr =
      make_rsrc(X, (uint64_t)(a.x_gathered ? (int64_t)a.rows : a.BT) * a.H * sizeof(S));
  const int64_t nrows_w = a.V - n0 < C::BN ? a.V - n0 : C::BN;
  const desc_t wr = make_rsrc(W + n0 * a.H, (uint64_t)nrows_w * a.H * sizeof(S));
  OA la;
  OB lb;
  // The block's target columns are read now, so that the two dependent
  // global reads complete under the k loop, and staged in LDS for the
  // epilogue afterwards.  Table entries are read unconditionally (row 0 of
  // the chunk stands in for rows past its end), so that no read waits in a
  // branch of its own.
  constexpr int TPT = (C::BM + C::NT - 1) / C::NT;  // target rows per thread
  int tix[TPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int m = tid + i * C::NT, gm = m0 + m;
    tix[i] = a.idx[m < C::BM && gm < a.rows ? gm : 0];
  }
  if (a.x_gathered)
    la.init(tid, [&](int r) -> uint32_t {
      return m0 + r < a.rows ? (uint32_t)(m0 + r) * row_bytes : kOOB;
    });
  else
    la.init_indexed(
        tid, [&](int r) -> uint32_t { return (uint32_t)a.idx[m0 + r < a.rows ? m0 + r : 0]; },
        [&](int r, uint32_t e) -> uint32_t { return m0 + r < a.rows ? e * row_bytes : kOOB; });
  lb.init(tid, [&](int r) -> uint32_t { return r < nrows_w ? (uint32_t)r * row_bytes : kOOB; });
  int64_t tgt[TPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    asm volatile("" : "+v"(tix[i]));
    tgt[i] = a.targets[tix[i]];
  }

  f32x16_t acc[C::FM][C::FN];
  zero_acc<C>(acc);
  const int K = (int)a.H;
  constexpr int P = PI::P;
  main_loop<T, C, OA, OB, PI::SA, PI::SB, P>(
      [&](unsigned char* tile, int k0, int p) { la.template issue<P>(xr, tile, k0, K, p); },
      [&](unsigned char* tile, int k0, int p) { lb.template issue<P>(wr, tile, k0, K, p); },
      (K + KT<T, C>::BK - 1) / KT<T, C>::BK, smem_raw, wm, wn, lane, acc);

  // Epilogue: add the bias (when given; PR #1554, Tests: bias on and off),
  // store the logits relative to their 64-column block maximum (z - max, in
  // the slab dtype), and per (row, 64-column block) the max and the sum of
  // exp(z - max) in fp32, plus, when predictions are wanted, the first column
  // holding that max.  Both tile shapes reduce a 64-column block the same way
  // (8 lanes x 8 values), so a row's log-sum-exp does not depend on the
  // chunking.
  // The block's target columns go after the staging area (the operand
  // stages are free once the main loop is done; the epilogue's first barrier
  // publishes them).
  int64_t* tgt_s = reinterpret_cast<int64_t*>(smem_raw + SM::EPI);
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int m = tid + i * C::NT;
    if (m < C::BM) tgt_s[m] = m0 + m < a.rows ? tgt[i] : -1;
  }
  S* slab = static_cast<S*>(a.slab);
  float2* stats = reinterpret_cast<float2*>(a.stats);
  const S* bias = static_cast<const S*>(a.bias);
  staged_epilogue<C, T::sub16>(reinterpret_cast<float*>(smem_raw), acc, wm, wn, lane, tid,
                     [&](int brow, int bcol, float (&v)[8]) __attribute__((always_inline)) {
    // Branch-free except where a piece straddles the end of the vocabulary:
    // columns past V are masked to -inf for the statistics by selects.
    const int gm = m0 + brow;
    const int64_t gn = n0 + bcol;
    const int64_t left = a.V - gn;
    const int nv = left >= 8 ? 8 : (left > 0 ? (int)left : 0);  // valid columns here
    if (bias) {
      if (nv == 8) {
        float b8[8];
        if constexpr (sizeof(S) == 2) {
          unpack8<T>(*reinterpret_cast<const u32x4_t*>(bias + gn), b8);
        } else {
          const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(bias + gn);
          const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(bias + gn + 4);
          b8[0] = lo[0], b8[1] = lo[1], b8[2] = lo[2], b8[3] = lo[3];
          b8[4] = hi[0], b8[5] = hi[1], b8[6] = hi[2], b8[7] = hi[3];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += b8[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e < nv) v[e] += T::to_f32(bias[gn + e]);
      }
    }
    float w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = e < nv ? v[e] : -INFINITY;
    float mx = -INFINITY;
    int am = 0x7fffffff;  // first column of the block maximum (with a.amax)
    if (a.amax) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bool gt = w[e] > mx;
        am = gt ? (int)(gn + e) : am;
        mx = gt ? w[e] : mx;
      }
      group8_argmax(mx, am);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, w[e]);
      mx = group8_max(mx);
    }
    // exp(-inf - mx) = 0 for masked columns; a group whose 64 columns all lie
    // past V gets NaN here but is never stored.
    float se = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) se += __expf(w[e] - mx);
    se = group8_sum(se);
    if (gm >= a.rows || nv == 0) return;
    if ((bcol & 63) == 0) {
      stats[(int64_t)gm * a.stats_ld + gn / 64] = float2{mx, se};
      if (a.amax) a.amax[(int64_t)gm * a.stats_ld + gn / 64] = am;
    }
    if (a.store_slab) {
      // The slab keeps each logit minus its block maximum: the entries that
      // dominate the softmax are then small numbers, whose rounding to the
      // slab dtype is small in absolute terms whatever the logits' scale.
      float d8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) d8[e] = v[e] - mx;
      store8<T>(slab + (int64_t)gm * a.ldz + gn, d8);
    }
    const int64_t d = tgt_s[brow] - gn;  // target column within this piece, if any
    float zt = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) zt = d == e ? v[e] : zt;
    if (d >= 0 && d < 8) a.ztgt[gm] = zt;
  });
}

// ---------------------------------------------------------------------------
// grad_input: dX[idx[m], n] = s * sum_k G[m, k] W[k, n] over one split of k,
// or, with splits > 1, fp32 partials part[split][m][n] reduced afterwards.
// ---------------------------------------------------------------------------
template <class T, class C, class PI>
__global__ __launch_bounds__(C::NT, C::WAVES_PER_SIMD) void dx_kernel(DxArgs a) {
  typedef typename T::storage S;
  typedef DmaRows<T, C, C::BM> OA;
  typedef DmaCols<T, C, C::BN> OB;
  extern __shared__ __align__(16) unsigned char smem_raw[];

  const int tiles_m = (a.rows + C::BM - 1) / C::BM;
  const int tiles_n = (int)((a.H + C::BN - 1) / C::BN);
  const int per_split = tiles_m * tiles_n;
  const int lin = xcd_remap(blockIdx.x, per_split * a.splits);
  const int split = lin / per_split;
  const int rem = lin % per_split;
  int tm, tn;
  grouped_tile(rem, tiles_m, tiles_n, kDxGroupM, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

  const int64_t kbeg = (int64_t)split * a.k_per_split;
  const int64_t kend = kbeg + a.k_per_split < a.ldz ? kbeg + a.k_per_split : a.ldz;
  const int64_t kend_w = kend < a.V ? kend : a.V;
  const S* G = static_cast<const S*>(a.slab);
  const S* W = static_cast<const S*>(a.W);
  const int H = (int)a.H;

  // G: this tile's rows [m0, m0 + BM) of the slab from column kbeg on;
  // W: rows [kbeg, kend_w), one descriptor per k-tile.
  const uint32_t gz_bytes = (uint32_t)a.ldz * (uint32_t)sizeof(S);
  const int g_rows = a.rows - m0 < C::BM ? a.rows - m0 : C::BM;
  const desc_t gr = make_rsrc(
      G + (int64_t)m0 * a.ldz + kbeg, ((uint64_t)g_rows * a.ldz - kbeg) * sizeof(S));
  const uint32_t w_row_bytes = (uint32_t)H * (uint32_t)sizeof(S);
  OA la;
  OB lb;
  la.init(tid, [&](int r) -> uint32_t { return r < g_rows ? (uint32_t)r * gz_bytes : kOOB; });
  lb.init(tid, n0, H);

  f32x16_t acc[C::FM][C::FN];
  zero_acc<C>(acc);
  const int K = (int)(kend - kbeg);
  constexpr int BK = KT<T, C>::BK;
  constexpr int P = PI::P < KT<T, C>::STEPS ? PI::P : KT<T, C>::STEPS;
  main_loop<T, C, OA, OB, PI::SA, PI::SB, P>(
      [&](unsigned char* tile, int k0, int p) { la.template issue<P>(gr, tile, k0, K, p); },
      [&](unsigned char* tile, int k0, int p) {
        // W rows of this k-tile: one descriptor per tile keeps offsets small.
        // (branch-free: a tile past the end gets an empty descriptor)
        const int64_t r0 = kbeg + k0;
        const int64_t left = kend_w - r0;
        const int nr = left <= 0 ? 0 : (left < BK ? (int)left : BK);
        const desc_t wr =
            make_rsrc(W + (left > 0 ? r0 : 0) * H, (uint32_t)nr * w_row_bytes);
        lb.template issue<P>(
            wr, tile, 0, [&](int k) -> uint32_t { return k < nr ? (uint32_t)k * w_row_bytes : kOOB; },
            p);
      },
      K > 0 ? (K + BK - 1) / BK : 0, smem_raw, wm, wn, lane, acc);

  const float sc = upstream_scale(a.grad_output, a.inv_n, a.reduction);
  S* dX = static_cast<S*>(a.dX);
  float* part = a.partial + (int64_t)split * a.rows_cap * H;
  const bool direct = a.splits == 1;
  staged_epilogue<C, T::sub16>(reinterpret_cast<float*>(smem_raw), acc, wm, wn, lane, tid,
                     [&](int brow, int bcol, float (&v)[8]) __attribute__((always_inline)) {
    const int gm = m0 + brow;
    const int gn = n0 + bcol;
    if (gm >= a.rows || gn >= H) return;
    if (direct) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= sc;
      store8<T>(dX + (int64_t)a.idx[gm] * H + gn, v);
    } else {
      float* p = part + (int64_t)gm * H + gn;
      *reinterpret_cast<f32x4_t*>(p) = f32x4_t{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4_t*>(p + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
    }
  });
}

// ---------------------------------------------------------------------------
// grad_weight: dW[m, n] = (dW[m, n] if accumulate) + s * sum_k G[k, m] X[idx[k], n]
// The accumulator starts at zero and the destination is read only in the
// epilogue, so no [V, H] temporary exists.
// ---------------------------------------------------------------------------
// The grad_weight epilogue: staged like staged_epilogue, but every value a
// thread will add to is loaded before the pass's accumulators are staged,
// so those loads' latency overlaps the staging instead of serialising with
// the stores (the compiler cannot move a load of one piece above the store
// of another).
// Cache policy of a buffer load or store: non-temporal (gfx950's nt bit).
constexpr int kNonTemporal = 2;

// Under 16-bit operands dW is read and written non-temporally (NT).  Its
// read-modify-write is the chunk's largest stream at small chunks (2 V H a
// bytes), and kept out of the caches it no longer evicts the weight rows
// that grad_input has just read: the next chunk's logits GEMM then finds
// part of W in the 256 MB memory-side cache.  Measured on MI355X (loads and
// stores both non-temporal; either alone gained nothing):
//   16-bit dW: masked SFT (V 151936, H 2048, chunk 128) 42.8 -> 39.7 ms per
//     step, logits 220 -> 179 us per chunk; long sequences (V 262144,
//     H 5376, chunk 256) 95.7 -> 93.4 ms;
//   fp32 dW, Llama shape: chunk 256 42.96 -> 40.15 ms per step (grad_weight
//     792 -> 733 us, logits 283 -> 256 us); chunk 2048 grad_weight 2016 ->
//     1997 us.
// With fp32 operands (a k loop 16 times as long) the hint made grad_weight
// 1 % slower, and dW stays cached there.
template <class C, class D, bool NT, bool SUB16>
__device__ __forceinline__ void dw_epilogue(float* stage, const f32x16_t (&acc)[C::FM][C::FN],
                                            int wm, int wn, int lane, int tid, void* dW,
                                            int64_t m0, int n0, int64_t V, int H, float sc,
                                            bool accumulate) {
  typedef Stage<C> ST;
  constexpr int LS = ST::LS;
  constexpr bool F32 = std::is_same<D, float>::value;
  constexpr uint64_t ES = F32 ? 4 : 2;
  // The destination values are read and written through buffer descriptors
  // over this tile's rows of dW: a piece outside the matrix takes an offset
  // past the range, so its load reads zeros and its store is dropped, and
  // when not accumulating the load descriptor is empty.  The loads and
  // stores then need no branches, and the compiler can wait for the loads
  // one piece at a time.  (The library limits H to 2^20, so a tile's rows
  // span at most 1 GiB.)
  const int64_t trows = V - m0 < C::BM ? V - m0 : C::BM;
  const uint64_t span = (uint64_t)trows * (uint64_t)H * ES;
  unsigned char* const base = static_cast<unsigned char*>(dW) + (uint64_t)m0 * (uint64_t)H * ES;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)span, 0x00020000);
  const __amdgpu_buffer_rsrc_t rl =
      __builtin_amdgcn_make_buffer_rsrc(base, 0, accumulate ? (int)span : 0, 0x00020000);
  // A piece is PC columns of one staged row, one 16-byte vector of dW: 4
  // columns of an fp32 dW under the eight-wave tiles, 8 of a 16-bit one.
  // Consecutive lanes then read and write consecutive 16-byte chunks of a
  // row (chunk 2048: grad_weight 2.14 -> 2.07 ms against 8-column pieces of
  // two vectors each, which the four-wave fp32 tiles keep: 4 % faster there).
  constexpr bool ONE = !F32 || C::NT == 512;
  constexpr int PC = F32 ? (ONE ? 4 : 8) : 8;
  constexpr int NV = ONE ? 1 : 2;           // 16-byte vectors per piece
  constexpr int SUBSP = C::BN / PC;         // pieces per staged row
  constexpr int NQP = ST::ROWS * SUBSP / C::NT;
  static_assert((ST::ROWS * SUBSP) % C::NT == 0 && C::NT % SUBSP == 0, "uniform pieces per lane");
  // With one workgroup per CU, pass p stages BAND rows of every wave (its
  // accumulator blocks [p IPB, (p + 1) IPB)) rather than all rows of half
  // the waves, so every wave writes half as much per staging step.
  // Interleaved on MI355X: grad_weight at chunk 2048 2.107 -> 2.068 ms, at
  // chunk 256 857 -> 788 us, bf16 dW at H 5376 / V 262144 1436 -> 1375 us.
  // The tiles that share a CU between two workgroups keep rows of waves
  // (masked SFT at chunk 128: 242 against 245 us).  Each pass's destination
  // values are loaded at its start, before the barrier, and overlap the
  // staging; loading the next pass's values before this pass's stores was
  // no faster.
  constexpr bool SPLIT = C::WGS == 1;
  constexpr int PASSES = ST::PASSES, BAND = SPLIT ? ST::ROWS / C::WAVES_M : C::WTM, IPB = BAND / 32;
  static_assert(BAND % 32 == 0 && (!SPLIT || PASSES * BAND == C::WTM), "whole blocks per pass");
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    // Byte offset of piece i of this thread, or kOOB for a piece past column
    // H (a row past V lies past the descriptor's range by itself; a thread's
    // pieces all have the same columns, since SUBSP divides NT).  Staged row
    // s is tile row (s / BAND) WTM + p BAND + s % BAND when split, else
    // p ROWS + s.
    auto piece_off = [&](int i) -> uint32_t {
      const int s = (tid + i * C::NT) / SUBSP, gn = n0 + (tid % SUBSP) * PC;
      const int tr = SPLIT ? (s / BAND) * C::WTM + p * BAND + s % BAND : p * ST::ROWS + s;
      return gn < H ? (uint32_t)(((uint64_t)tr * (uint64_t)H + (uint64_t)gn) * ES) : kOOB;
    };
    u32x4_t old[NQP * NV];
#pragma unroll
    for (int i = 0; i < NQP; ++i) {
      const uint32_t off = piece_off(i);
#pragma unroll
      for (int h = 0; h < NV; ++h)
        old[i * NV + h] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rl, (int)(off == kOOB ? kOOB : off + 16u * h),
                                                           0, NT ? kNonTemporal : 0));
    }
    __syncthreads();
    if (SPLIT || wm / ST::WR == p) {
      const int r0 = SPLIT ? wm * BAND : (wm % ST::WR) * C::WTM;
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
        if (!SPLIT || i / IPB == p)
#pragma unroll
          for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = r0 + (i % IPB) * 32 + acc_row<SUB16>(r, lane);
              const int col = wn * C::WTN + j * 32 + acc_col<SUB16>(r, lane);
              stage[row * LS + col] = acc[i][j][r];
            }
    }
    __syncthreads();
    // Stores go through the tile's descriptor (rs, never empty), so a piece
    // outside the matrix is dropped by the hardware and the loop has no
    // branch.
#pragma unroll
    for (int i = 0; i < NQP; ++i) {
      const int q = tid + i * C::NT, lrow = q / SUBSP, piece = q % SUBSP;
      const uint32_t off = piece_off(i);
      if constexpr (F32) {
#pragma unroll
        for (int h = 0; h < NV; ++h) {
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(stage + lrow * LS + piece * PC + 4 * h);
          const f32x4_t o = __builtin_bit_cast(f32x4_t, old[i * NV + h]);
          const f32x4_t w = {v[0] * sc + o[0], v[1] * sc + o[1], v[2] * sc + o[2], v[3] * sc + o[3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, w), rs,
                                                 (int)(off == kOOB ? kOOB : off + 16u * h), 0,
                                                 NT ? kNonTemporal : 0);
        }
      } else {
        const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(stage + lrow * LS + piece * 8);
        const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(stage + lrow * LS + piece * 8 + 4);
        float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        float o[8];
        unpack8<D>(old[i], o);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = v[e] * sc + o[e];
        __builtin_amdgcn_raw_buffer_store_b128(pack8<D>(v), rs, (int)off, 0, NT ? kNonTemporal : 0);
      }
    }
  }
}

template <class T, class C, class D>
__global__ __launch_bounds__(C::NT, C::WAVES_PER_SIMD) void dw_kernel(DwArgs a) {
  typedef typename T::storage S;
  typedef DmaCols<T, C, C::BM> OA;
  typedef DmaRows<T, C, C::BN> OB;
  typedef DwPipe<C> PI;
  extern __shared__ __align__(16) unsigned char smem_raw[];

  const int tiles_m = (int)((a.V + C::BM - 1) / C::BM);
  const int tiles_n = (int)((a.H + C::BN - 1) / C::BN);
  const int lin = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  int tm, tn;  // N fastest within a group: blocks sharing a G tile are adjacent
  grouped_tile(lin, tiles_n, tiles_m, kDwGroupN, tn, tm);
  const int64_t m0 = (int64_t)tm * C::BM;
  const int n0 = tn * C::BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int H = (int)a.H;

  const S* G = static_cast<const S*>(a.slab);
  const S* XcT = static_cast<const S*>(a.XcT);
  // G: the chunk's rows (k) of the slab, one descriptor per k-tile; XcT:
  // hidden units [n0, n0 + BN) of the gathered chunk, k contiguous.
  const uint32_t gz_bytes = (uint32_t)a.ldz * (uint32_t)sizeof(S);
  const uint32_t xt_row_bytes = (uint32_t)a.ldx * (uint32_t)sizeof(S);
  const int xt_rows = H - n0 < C::BN ? H - n0 : C::BN;
  const desc_t xr =
      make_rsrc(XcT + (int64_t)n0 * a.ldx, (uint64_t)xt_rows * a.ldx * sizeof(S));
  OA la;
  OB lb;
  la.init(tid, (int)m0, (int)a.ldz);
  lb.init(tid, [&](int r) -> uint32_t { return r < xt_rows ? (uint32_t)r * xt_row_bytes : kOOB; });

  f32x16_t acc[C::FM][C::FN];
  zero_acc<C>(acc);
  constexpr int BK = KT<T, C>::BK;
  constexpr int P = PI::P < KT<T, C>::STEPS ? PI::P : KT<T, C>::STEPS;
  main_loop<T, C, OA, OB, PI::SA, PI::SB, P>(
      [&](unsigned char* tile, int k0, int p) {
        // (branch-free: a tile past the end gets an empty descriptor)
        const int left = a.rows - k0;
        const int nr = left <= 0 ? 0 : (left < BK ? left : BK);
        const desc_t gr =
            make_rsrc(G + (int64_t)(left > 0 ? k0 : 0) * a.ldz, (uint32_t)nr * gz_bytes);
        la.template issue<P>(
            gr, tile, 0, [&](int k) -> uint32_t { return k < nr ? (uint32_t)k * gz_bytes : kOOB; },
            p);
      },
      [&](unsigned char* tile, int k0, int p) { lb.template issue<P>(xr, tile, k0, a.rows, p); },
      (a.rows + BK - 1) / BK, smem_raw, wm, wn, lane, acc);

  const float sc = upstream_scale(a.grad_output, a.inv_n, a.reduction);
  const bool accumulate = a.accumulate != 0;
  dw_epilogue<C, D, sizeof(S) == 2, T::sub16>(reinterpret_cast<float*>(smem_raw), acc, wm, wn, lane, tid, a.dW,
                                    m0, n0, a.V, H, sc, accumulate);
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
// Workgroups above 64 KiB of LDS need the per-kernel limit raised (gfx950 has
// 160 KiB per CU).  Done once per kernel instantiation.
template <class K>
static hipError_t allow_lds(K kernel, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <class T, class C>
struct LogitsSmem : Smem<C, DmaRows<T, C, C::BM>, DmaRows<T, C, C::BN>, LogitsPipe<C>::SA,
                         LogitsPipe<C>::SB, C::BM * sizeof(int64_t)> {};
template <class T, class C, class PI>
struct DxSmem : Smem<C, DmaRows<T, C, C::BM>, DmaCols<T, C, C::BN>, PI::SA, PI::SB> {};
template <class T, class C>
struct DwSmem : Smem<C, DmaCols<T, C, C::BM>, DmaRows<T, C, C::BN>, DwPipe<C>::SA,
                     DwPipe<C>::SB> {};

template <class T, class C>
static hipError_t launch_logits_t(const LogitsArgs& a, hipStream_t st) {
  static const hipError_t prep = allow_lds(logits_kernel<T, C>, LogitsSmem<T, C>::BYTES);
  if (prep != hipSuccess) return prep;
  const int tiles = ((a.rows + C::BM - 1) / C::BM) * (int)((a.V + C::BN - 1) / C::BN);
  logits_kernel<T, C><<<dim3(tiles), dim3(C::NT), LogitsSmem<T, C>::BYTES, st>>>(a);
  return hipGetLastError();
}
template <class T, class C, class PI = DxPipe<C>>
static hipError_t launch_dx_t(const DxArgs& a, hipStream_t st) {
  static const hipError_t prep = allow_lds(dx_kernel<T, C, PI>, DxSmem<T, C, PI>::BYTES);
  if (prep != hipSuccess) return prep;
  const int tiles = ((a.rows + C::BM - 1) / C::BM) * (int)((a.H + C::BN - 1) / C::BN) * a.splits;
  dx_kernel<T, C, PI><<<dim3(tiles), dim3(C::NT), DxSmem<T, C, PI>::BYTES, st>>>(a);
  return hipGetLastError();
}
template <class T, class C, class D>
static hipError_t launch_dw_t(const DwArgs& a, hipStream_t st) {
  static const hipError_t prep = allow_lds(dw_kernel<T, C, D>, DwSmem<T, C>::BYTES);
  if (prep != hipSuccess) return prep;
  const int tiles = (int)((a.V + C::BM - 1) / C::BM) * (int)((a.H + C::BN - 1) / C::BN);
  dw_kernel<T, C, D><<<dim3(tiles), dim3(C::NT), DwSmem<T, C>::BYTES, st>>>(a);
  return hipGetLastError();
}

// Tile choice.  The 256-row tiles need enough rows and columns to fill
// them.  With 16-bit operands the three GEMMs take eight waves on the
// 256 x 256 tile, two per SIMD, so that one wave's waits for LDS, loads and
// barriers and the epilogue's memory traffic overlap the other wave's MFMA
// work.  Measured on MI355X at chunk 2048 (interleaved runs of the
// alternatives): logits 2.23 -> 1.86 ms (64 x 128 wave tiles, loads issued
// in one part), grad_input 1.92 -> 1.73 ms (128 x 64 wave tiles), grad_weight
// 2.60 -> 2.32 ms (64 x 128, three stages of G).  256 x 128 tiles with two
// workgroups per CU reached 2.40 ms for grad_weight but were 15-25 % slower
// for logits and grad_input, whose k loops then load twice the operand bytes
// per MFMA (half the operand reuse per workgroup).  fp32 keeps the four-wave
// tile.
// For 16-bit operands grad_input and grad_weight take the eight-wave tile at
// any chunk size ("wide"): with few rows per chunk, where the dW
// read-modify-write bounds grad_weight, a 256 x 256 tile moves four times the
// bytes per load round trip of a 128 x 128 one (grad_weight at chunk 256:
// 0.95 -> 0.89 ms with fp32 dW, 2.24 -> 1.72 ms with bf16 dW at H 5376,
// V 262144; at chunk 128 both GEMMs 9-12 % faster).  Logits keep a
// 128 x 128 tile for chunks of at most 128 rows (7-11 % faster there than
// 256 x 256); with 16-bit operands it is eight waves, two workgroups per CU,
// so that one workgroup's first loads and epilogue overlap the other's k
// loop.  Interleaved against one workgroup per CU over 256-byte k rows
// (longer runs per W row, but each tile's pipeline fill exposed): masked SFT
// (H 2048) at chunk 128 175 -> 169 us trained, 162 -> 161 us frozen; the
// Llama shape at chunk 128 227 -> 219 us.  Splitting each k-tile's loads in
// two parts was slower (176 us).
enum class Shape { Small, Big };
Shape logits_shape(int rows, int64_t V) { return rows > 128 && V >= 1024 ? Shape::Big : Shape::Small; }
Shape dx_shape(int rows, int64_t H, bool wide) {
  return (wide || rows > 128) && H >= 256 ? Shape::Big : Shape::Small;
}
Shape dw_shape(int rows, int64_t H, bool wide) {
  return (wide || rows > 256) && H >= 256 ? Shape::Big : Shape::Small;
}

template <class T>
static hipError_t logits_t(const LogitsArgs& a, hipStream_t st) {
  constexpr bool k16 = sizeof(typename T::storage) == 2;
  typedef typename std::conditional<k16, Big8M, Big>::type L;
  typedef typename std::conditional<k16, Small8, Small>::type LS;
  if constexpr (k16)
    if (logits_shape(a.rows, a.V) == Shape::Big) return launch_logits_t<Mfma16<T>, L>(a, st);
  return logits_shape(a.rows, a.V) == Shape::Big ? launch_logits_t<T, L>(a, st)
                                                 : launch_logits_t<T, LS>(a, st);
}
// MFMA shape of the 16-bit GEMMs on the large tiles.  16x16x32 MFMAs draw
// less power than 32x32x16 for the same flops, so under the chip's power
// limit they run at a higher clock, but their loop leaves more fragment-read
// latency exposed (two k-steps per k-tile instead of four).  Which wins
// depends on the kernel and on what else the step runs (the clock follows
// the power of the whole step).  Measured interleaved on MI355X:
// - grad_input from kDxSub16Rows rows per chunk: Llama shape chunk 2048
//   1738 -> 1691 us per launch, 4096 3438 -> 3226 us; H 4096 / V 32000 with
//   16384 rows 451 -> 425 us (bf16), 476 -> 433 us (fp16); 512 and 1024 rows
//   equal, 256 rows 258 -> 262 us (there the kernel streams W).
// - logits and grad_weight on the large tiles, with the MFMA order that
//   shares operands (mma_tile): with a 16-bit dW or none, steps 0.8-3.2 %
//   faster (fp16 sweep 11.65 -> 11.28 ms, bf16 sweep 11.28 -> 11.07 ms,
//   H 5376 / V 262144 with 32768 rows 247.8 -> 244.5 ms and at chunk 256
//   88.1 -> 86.7 ms, masked SFT at chunk 2048 14.27 -> 14.11 ms trained and
//   9.67 -> 9.59 ms frozen).  With an fp32 dW grad_weight is 3.5 % slower per
//   launch on 16x16x32, but it then leaves logits and grad_input more of the
//   power budget: the Llama shape at chunk 2048 23.03 -> 22.85 and 23.16 ->
//   22.94 ms per step (logits -4 %, grad_input -3.7 %), chunks 256 and 4096
//   0.1 % faster.
// - the small tiles (chunks of at most 128 rows) keep 32x32x16: those chunks
//   stream W from HBM, and 16x16x32 there was 0.2-0.3 % slower.
constexpr int kDxSub16Rows = 1024;
template <class T>
static hipError_t dx_t(const DxArgs& a, hipStream_t st) {
  constexpr bool k16 = sizeof(typename T::storage) == 2;
  typedef typename std::conditional<k16, Big8N, Big>::type L;
  if (dx_shape(a.rows, a.H, k16) != Shape::Big) return launch_dx_t<T, Small>(a, st);
  if constexpr (k16) {
    if (a.rows <= 128) return launch_dx_t<T, Mid8N>(a, st);
    return a.rows >= kDxSub16Rows ? launch_dx_t<Mfma16<T>, L, DxPipeG3>(a, st)
                                  : launch_dx_t<T, L, DxPipeG3>(a, st);
  } else {
    return launch_dx_t<T, L>(a, st);
  }
}
template <class T, class D>
static hipError_t dw_t(const DwArgs& a, hipStream_t st) {
  constexpr bool k16 = sizeof(typename T::storage) == 2;
  typedef typename std::conditional<k16, Big8M, Big>::type L;
  if (dw_shape(a.rows, a.H, k16) != Shape::Big) return launch_dw_t<T, Small, D>(a, st);
  if constexpr (k16)
    if (a.rows <= 128) return launch_dw_t<T, Twin8M, D>(a, st);
  if constexpr (k16) return launch_dw_t<Mfma16<T>, L, D>(a, st);
  return launch_dw_t<T, L, D>(a, st);
}

hipError_t launch_logits(int dtype, const LogitsArgs& a, hipStream_t st) {
  if (dtype == 0) return logits_t<F32>(a, st);
  if (dtype == 1) return logits_t<F16>(a, st);
  return logits_t<BF16>(a, st);
}
hipError_t launch_dx(int dtype, const DxArgs& a, hipStream_t st) {
  if (dtype == 0) return dx_t<F32>(a, st);
  if (dtype == 1) return dx_t<F16>(a, st);
  return dx_t<BF16>(a, st);
}
hipError_t launch_dw(int dtype, const DwArgs& a, hipStream_t st) {
  // dW is fp32 or the operand dtype.
  if (dtype == 0) return dw_t<F32, float>(a, st);
  if (dtype == 1) return a.dw_dtype == 0 ? dw_t<F16, float>(a, st) : dw_t<F16, F16>(a, st);
  return a.dw_dtype == 0 ? dw_t<BF16, float>(a, st) : dw_t<BF16, BF16>(a, st);
}

DxTile dx_tile(int dtype, int rows, int64_t H) {
  static_assert(Big::BM == Big8N::BM && Big::BN == Big8N::BN && Big::WGS == Big8N::WGS,
                "both large grad_input tiles split k alike");
  if (dx_shape(rows, H, dtype != 0) != Shape::Big) return DxTile{Small::BM, Small::BN, Small::WGS};
  if (dtype != 0 && rows <= 128) return DxTile{Mid8N::BM, Mid8N::BN, Mid8N::WGS};
  return DxTile{Big::BM, Big::BN, Big::WGS};
}
// Column width of one (max, sum exp) entry written by the logits GEMM.
int stats_cols() {
  static_assert(Big::BN % 64 == 0 && Big8M::BN % 64 == 0 && Small::BN % 64 == 0 &&
                    Small8::BN % 64 == 0,
                "64-column stats blocks");
  return 64;
}

}  // namespace flce
