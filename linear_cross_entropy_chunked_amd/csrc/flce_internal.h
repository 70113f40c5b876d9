// Internal interface between the host orchestrator and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

// Logits GEMM of one chunk (rows = labelled rows in this chunk).
struct LogitsArgs {
  const void* X;           // [BT, H] operand dtype, or with x_gathered the chunk's rows [rows, H]
  const void* W;           // [V, H]
  const int32_t* idx;      // [rows] labelled row ids of this chunk
  int x_gathered;          // 1: row r of the chunk is row r of X (already gathered)
  const int64_t* targets;  // [BT]
  int rows;
  int64_t BT, H, V;
  void* slab;              // [rows_cap, ldz] operand dtype
  int64_t ldz;
  float* stats;            // [rows_cap, stats_ld] float2 (max, sum exp) per 64-column block
  int64_t stats_ld;        // in float2 units
  float* ztgt;             // [rows_cap] fp32 target logit
  const void* bias;        // [V] operand dtype, added to every row's logits; NULL = none
  int32_t* amax;           // [rows_cap, stats_ld] column of each block's maximum; NULL = not needed
  int store_slab;          // 0: logits are not stored (loss-only call)
};

// Softmax-gradient pass of one chunk.
struct SoftmaxArgs {
  void* slab;
  int64_t ldz, V;
  int rows;
  const float* stats;
  int64_t stats_ld, stats_n;  // float2 row stride, live blocks per row
  const float* ztgt;
  const int32_t* idx;         // chunk's labelled row ids
  const int64_t* targets;
  const float* grad_output;   // none: [BT] per-row upstream gradient (NULL = 1)
  int reduction;              // 0 mean, 1 sum, 2 none
  float* lossrow;             // mean/sum: [rows] per-row loss of this chunk
  float* loss_out;            // none: [BT] output
  int parts;                  // workgroups per row
  int64_t cols_per_part;      // multiple of 8
  int write_grad;             // 0: loss and per-token outputs only, the slab is not touched
  float z_scale;              // coefficient of lse^2 in the loss (0: none)
  const int32_t* amax;        // block argmax from the logits GEMM; NULL = no predictions
  int64_t* pred_out;          // [BT] predicted token, or NULL
  float* zrow;                // mean/sum: [rows] lse^2 of this chunk, or NULL
  float* accrow;              // mean/sum: [rows] accuracy of this chunk, or NULL
  float* z_out;               // none: [BT] lse^2 output, or NULL
  float* acc_out;             // none: [BT] accuracy output, or NULL
};
// grad_bias of one chunk: column sums of G over the chunk's rows, first per
// block of kBiasRows rows (partials), then in row-block order per column.
struct BiasGradArgs {
  const void* slab;  // G [rows, ldz]
  int rows;
  int64_t V, ldz;
  float* partial;    // [ceil(rows_cap / kBiasRows), ldz] fp32
  void* grad_bias;   // [V] db_dtype
  int db_dtype;      // 0 f32, 1 f16, 2 bf16
  int accumulate;    // 1: add to grad_bias
  const float* grad_output;
  float inv_n;
  int reduction;
};
constexpr int kBiasRows = 32;

// grad_input GEMM of one chunk.
struct DxArgs {
  const void* slab;  // G [rows, ldz]
  const void* W;     // [V, H]
  const int32_t* idx;
  int rows, rows_cap;
  int64_t H, V, ldz;
  int splits;
  int64_t k_per_split;  // multiple of the GEMM k-tile
  void* dX;             // [BT, H] (splits == 1)
  float* partial;       // [splits, rows_cap, H] (splits > 1)
  const float* grad_output;
  float inv_n;
  int reduction;
};

struct DxReduceArgs {
  const float* partial;
  int splits, rows, rows_cap;
  int64_t H;
  const int32_t* idx;
  void* dX;
  const float* grad_output;
  float inv_n;
  int reduction;
};

// grad_weight GEMM of one chunk.
struct DwArgs {
  const void* slab;  // G [rows, ldz]
  const void* XcT;   // [H, ldx] the chunk's gathered rows, transposed
  int rows;
  int64_t H, V, ldz, ldx;
  void* dW;          // [V, H] dw_dtype
  int dw_dtype;      // 0 f32, 1 f16, 2 bf16
  int accumulate;    // 1: add to dW
  const float* grad_output;
  float inv_n;
  int reduction;
};

// Device flags written by the mask/scan kernel and read by the host once.
struct ScanFlags {
  int32_t n_valid;
  int32_t bad_target;
};

hipError_t launch_logits(int dtype, const LogitsArgs& a, hipStream_t st);
hipError_t launch_dx(int dtype, const DxArgs& a, hipStream_t st);
hipError_t launch_dw(int dtype, const DwArgs& a, hipStream_t st);
hipError_t launch_softmax(int dtype, const SoftmaxArgs& a, hipStream_t st);
hipError_t launch_dx_reduce(int dtype, const DxReduceArgs& a, hipStream_t st);
hipError_t launch_mask_scan(const int64_t* targets, int64_t BT, int64_t V, int64_t ignore_index,
                            int32_t* idx, ScanFlags* flags, hipStream_t st);
hipError_t launch_gather_t(int dtype, const void* X, const int32_t* idx, int rows, int64_t H,
                           void* XcT, int64_t ldx, hipStream_t st);
// Xc[r, :] = X[idx[r], :] for r < rows (row-major, H elements per row).
hipError_t launch_gather_rows(int dtype, const void* X, const int32_t* idx, int rows, int64_t H,
                              void* Xc, hipStream_t st);
// Outputs of an ignored row: zero dX row (dX may be NULL), and, where given,
// zero per-token loss / z-loss / accuracy and -1 as predicted token.
struct IgnoredOut {
  void* dX;
  int dx_dtype;
  float* loss_none;
  float* z_none;
  float* acc_none;
  int64_t* pred;
};
hipError_t launch_zero_ignored(const int64_t* targets, int64_t BT, int64_t H,
                               int64_t ignore_index, const IgnoredOut& o, hipStream_t st);
hipError_t launch_bias_grad(int dtype, const BiasGradArgs& a, hipStream_t st);
hipError_t launch_finalize(const float* lossrow, int n, int mean, float* loss, hipStream_t st);
hipError_t launch_fill_zero(void* p, int64_t bytes, hipStream_t st);
hipError_t launch_scale_cast(const void* src, int src_dtype, void* dst, int dst_dtype,
                             int64_t n, const float* scale, hipStream_t st);

// grad_input tile shape for a chunk of `rows` rows: bm x bn outputs per
// workgroup, wgs workgroups resident per CU.
struct DxTile {
  int bm, bn, wgs;
};
DxTile dx_tile(int dtype, int rows, int64_t H);
int stats_cols();

}  // namespace flce
