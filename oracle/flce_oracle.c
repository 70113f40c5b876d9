/*
 * Fused linear cross-entropy: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or constant with the GPU
 * library.
 *
 * What it computes is the plain, unchunked definition of the method:
 *   logits z[i,v] = sum_k X[i,k] * W[v,k]                       (lm_head projection)
 *   lse_i         = log sum_v exp(z[i,v])                       (log-softmax normaliser)
 *   loss_i        = lse_i - z[i, t_i]                           (negative log-likelihood)
 *   dX[i,:]       = s_i * sum_v (softmax(z_i)_v - [v == t_i]) * W[v,:]
 *   dW[v,:]       = sum_i s_i * (softmax(z_i)_v - [v == t_i]) * X[i,:]
 * Sources: issue #1323 "Reduce FLCE weight-gradient allocation overhead
 * across FP16, BF16, and FP32", Background and motivation (the loss is the
 * linear projection followed by cross-entropy; chunking only avoids holding
 * all logits at once); PR #1554 (ignored-row skipping), Summary (the three
 * projections logits, grad_input, grad_weight; an ignored row contributes
 * zero to the loss and to every gradient) and Details item 1 (an ignored
 * row's grad_input row and per-token loss are zero).
 *
 * Chunking, row compaction and direct accumulation only reorder this exact
 * arithmetic (PR #1554, Details item 4: results agree up to rounding order),
 * so the oracle has no chunk size at all.
 *
 * Row scale s_i (reading of the pages, which name mean, sum and none with a
 * per-token upstream gradient in PR #1554, Tests):
 *   mean: s_i = g / N   (N = number of labelled rows in the whole call)
 *   sum : s_i = g
 *   none: s_i = g_i
 * g defaults to 1 when no upstream gradient is given.  With N = 0 the mean
 * loss is 0 and every gradient is 0.
 *
 * Inputs are already widened, exactly, to double.  Loops run in ascending
 * index order inside each output element, so results do not depend on the
 * number of OpenMP threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_MEAN = 0, ORACLE_SUM = 1, ORACLE_NONE = 2 };
enum { ORACLE_OK = 0, ORACLE_E_ARG = -1, ORACLE_E_TARGET = -3, ORACLE_E_MEM = -6 };

/* Threads the oracle's parallel loops will use. */
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Labelled-row list.  A row is labelled when its target differs from
 * ignore_index (PR #1554, Summary); labelled targets must index the
 * vocabulary.  The list is ascending, the order nonzero() gives
 * (PR #1554, Summary: nonzero() supplies the row index). */
int oracle_compact(const int64_t* t, int64_t BT, int64_t V, int64_t ignore_index,
                   int64_t* idx, int64_t* n_valid) {
  int64_t n = 0;
  for (int64_t i = 0; i < BT; ++i) {
    if (t[i] == ignore_index) continue;
    if (t[i] < 0 || t[i] >= V) return ORACLE_E_TARGET;
    idx[n++] = i;
  }
  *n_valid = n;
  return ORACLE_OK;
}

static double row_scale(int reduction, const double* g, int64_t i, int64_t n_valid) {
  if (reduction == ORACLE_NONE) return g ? g[i] : 1.0;
  double gs = g ? g[0] : 1.0;
  if (reduction == ORACLE_MEAN) return gs / (double)n_valid;
  return gs;
}

/* z[v] = sum_k W[v,k] * X[i,k], k ascending. */
static void logits_row(const double* X, const double* W, int64_t H, int64_t V, int64_t i,
                       double* z) {
  const double* x = X + i * H;
  for (int64_t v = 0; v < V; ++v) {
    const double* w = W + v * H;
    double acc = 0.0;
    for (int64_t k = 0; k < H; ++k) acc += w[k] * x[k];
    z[v] = acc;
  }
}

/* log sum_v exp(z[v]), with the row maximum taken out first so that exp()
 * cannot overflow; mathematically the same value. */
static double logsumexp_row(const double* z, int64_t V) {
  double m = z[0];
  for (int64_t v = 1; v < V; ++v)
    if (z[v] > m) m = z[v];
  double s = 0.0;
  for (int64_t v = 0; v < V; ++v) s += exp(z[v] - m);
  return m + log(s);
}

/* Per-row log-sum-exp for every labelled row (lse[i]; unlabelled rows get NaN). */
int oracle_lse(const double* X, const double* W, const int64_t* t, int64_t BT, int64_t H,
               int64_t V, int64_t ignore_index, double* lse) {
  if (BT < 0 || H < 1 || V < 1) return ORACLE_E_ARG;
  int err = 0;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)V);
    if (!z) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < BT; ++i) {
      if (!z) continue;
      if (t[i] == ignore_index) {
        lse[i] = NAN;
        continue;
      }
      logits_row(X, W, H, V, i, z);
      lse[i] = logsumexp_row(z, V);
    }
    free(z);
  }
  return err ? ORACLE_E_MEM : ORACLE_OK;
}

/*
 * Full oracle.  Outputs:
 *   loss : mean/sum -> loss[0]; none -> loss[BT] with ignored rows 0
 *   dX   : [BT,H]; ignored rows are +0.0 and never computed from X
 *   dW   : [V,H] (skipped when frozen != 0 or dW == NULL); overwritten, or
 *          added to when accumulate != 0
 *   lse  : optional [BT] (NaN for ignored rows)
 *   n_valid_out : optional, number of labelled rows
 * Returns 0, or ORACLE_E_TARGET when a labelled target lies outside [0, V).
 */
int oracle_flce(const double* X, const double* W, const int64_t* t, int64_t BT, int64_t H,
                int64_t V, int64_t ignore_index, int reduction, const double* grad_output,
                int frozen, int accumulate, double* loss, double* dX, double* dW, double* lse_out,
                int64_t* n_valid_out) {
  if (BT < 0 || H < 1 || V < 1) return ORACLE_E_ARG;
  if (reduction < ORACLE_MEAN || reduction > ORACLE_NONE) return ORACLE_E_ARG;
  int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)(BT > 0 ? BT : 1));
  double* lse = (double*)malloc(sizeof(double) * (size_t)(BT > 0 ? BT : 1));
  double* lrow = (double*)malloc(sizeof(double) * (size_t)(BT > 0 ? BT : 1));
  if (!idx || !lse || !lrow) {
    free(idx); free(lse); free(lrow);
    return ORACLE_E_MEM;
  }
  int64_t N = 0;
  int rc = oracle_compact(t, BT, V, ignore_index, idx, &N);
  if (rc != ORACLE_OK) {
    free(idx); free(lse); free(lrow);
    return rc;
  }
  if (n_valid_out) *n_valid_out = N;

  /* Ignored rows: zero grad_input row, zero per-token loss, NaN lse. */
  for (int64_t i = 0; i < BT; ++i) {
    lse[i] = NAN;
    lrow[i] = 0.0;
    if (dX && t[i] == ignore_index)
      for (int64_t k = 0; k < H; ++k) dX[i * H + k] = 0.0;
  }

  /* Row phase: logits, log-sum-exp, per-row loss and grad_input of each labelled row. */
  int err = 0;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)V);
    double* acc = (double*)malloc(sizeof(double) * (size_t)H);
    if (!z || !acc) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t n = 0; n < N; ++n) {
      if (!z || !acc) continue;
      const int64_t i = idx[n];
      const int64_t ti = t[i];
      logits_row(X, W, H, V, i, z);
      const double l = logsumexp_row(z, V);
      lse[i] = l;
      lrow[i] = l - z[ti];
      if (!dX) continue;
      const double s = row_scale(reduction, grad_output, i, N);
      for (int64_t k = 0; k < H; ++k) acc[k] = 0.0;
      for (int64_t v = 0; v < V; ++v) {
        const double gv = s * (exp(z[v] - l) - (v == ti ? 1.0 : 0.0));
        const double* w = W + v * H;
        for (int64_t k = 0; k < H; ++k) acc[k] += gv * w[k];
      }
      for (int64_t k = 0; k < H; ++k) dX[i * H + k] = acc[k];
    }
    free(z);
    free(acc);
  }
  if (err) {
    free(idx); free(lse); free(lrow);
    return ORACLE_E_MEM;
  }

  /* Loss reduction, rows in ascending order. */
  if (reduction == ORACLE_NONE) {
    for (int64_t i = 0; i < BT; ++i) loss[i] = lrow[i];
  } else {
    double s = 0.0;
    for (int64_t n = 0; n < N; ++n) s += lrow[idx[n]];
    loss[0] = (reduction == ORACLE_MEAN) ? (N > 0 ? s / (double)N : 0.0) : s;
  }

  /* Vocabulary phase: grad_weight row v sums over labelled rows i in
   * ascending order; z[i,v] is recomputed with the same loop as above. */
  if (!frozen && dW) {
#pragma omp parallel
    {
      double* acc = (double*)malloc(sizeof(double) * (size_t)H);
      if (!acc) {
#pragma omp atomic write
        err = 1;
      }
#pragma omp for schedule(dynamic, 16)
      for (int64_t v = 0; v < V; ++v) {
        if (!acc) continue;
        const double* w = W + v * H;
        for (int64_t k = 0; k < H; ++k) acc[k] = 0.0;
        for (int64_t n = 0; n < N; ++n) {
          const int64_t i = idx[n];
          const double* x = X + i * H;
          double z = 0.0;
          for (int64_t k = 0; k < H; ++k) z += w[k] * x[k];
          const double s = row_scale(reduction, grad_output, i, N);
          const double gv = s * (exp(z - lse[i]) - (v == t[i] ? 1.0 : 0.0));
          for (int64_t k = 0; k < H; ++k) acc[k] += gv * x[k];
        }
        double* d = dW + v * H;
        if (accumulate)
          for (int64_t k = 0; k < H; ++k) d[k] += acc[k];
        else
          for (int64_t k = 0; k < H; ++k) d[k] = acc[k];
      }
      free(acc);
    }
  }
  if (lse_out)
    for (int64_t i = 0; i < BT; ++i) lse_out[i] = lse[i];
  free(idx);
  free(lse);
  free(lrow);
  return err ? ORACLE_E_MEM : ORACLE_OK;
}

/*
 * Per-row loss, lse and grad_input for a list of rows only (used where the
 * full oracle is too slow).  dX_rows is [n_rows, H]; an ignored row gives
 * +0.0 everywhere and NaN lse.  n_valid is the labelled count of the whole
 * call (for mean).  loss_rows and lse_rows are [n_rows] and may be NULL.
 */
int oracle_dx_rows(const double* X, const double* W, const int64_t* t, int64_t H, int64_t V,
                   int64_t ignore_index, int reduction, const double* grad_output,
                   int64_t n_valid, const int64_t* rows, int64_t n_rows, double* dX_rows,
                   double* loss_rows, double* lse_rows) {
  int err = 0;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)V);
    double* acc = (double*)malloc(sizeof(double) * (size_t)H);
    if (!z || !acc) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (!z || !acc) continue;
      const int64_t i = rows[r];
      double* out = dX_rows + r * H;
      if (t[i] == ignore_index) {
        for (int64_t k = 0; k < H; ++k) out[k] = 0.0;
        if (loss_rows) loss_rows[r] = 0.0;
        if (lse_rows) lse_rows[r] = NAN;
        continue;
      }
      logits_row(X, W, H, V, i, z);
      const double l = logsumexp_row(z, V);
      if (loss_rows) loss_rows[r] = l - z[t[i]];
      if (lse_rows) lse_rows[r] = l;
      const double s = row_scale(reduction, grad_output, i, n_valid);
      for (int64_t k = 0; k < H; ++k) acc[k] = 0.0;
      for (int64_t v = 0; v < V; ++v) {
        const double gv = s * (exp(z[v] - l) - (v == t[i] ? 1.0 : 0.0));
        const double* w = W + v * H;
        for (int64_t k = 0; k < H; ++k) acc[k] += gv * w[k];
      }
      for (int64_t k = 0; k < H; ++k) out[k] = acc[k];
    }
    free(z);
    free(acc);
  }
  return err ? ORACLE_E_MEM : ORACLE_OK;
}

/*
 * grad_weight rows for a list of vocabulary rows only, given lse of every
 * row (lse[i], read for labelled rows only).  dW_rows is [n_rows, H].
 */
int oracle_dw_rows(const double* X, const double* W, const int64_t* t, int64_t BT, int64_t H,
                   int64_t ignore_index, int reduction, const double* grad_output,
                   int64_t n_valid, const int64_t* vrows, int64_t n_rows, const double* lse,
                   double* dW_rows) {
  int err = 0;
#pragma omp parallel
  {
    double* acc = (double*)malloc(sizeof(double) * (size_t)H);
    if (!acc) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
      if (!acc) continue;
      const int64_t v = vrows[r];
      const double* w = W + v * H;
      for (int64_t k = 0; k < H; ++k) acc[k] = 0.0;
      for (int64_t i = 0; i < BT; ++i) {
        if (t[i] == ignore_index) continue;
        const double* x = X + i * H;
        double z = 0.0;
        for (int64_t k = 0; k < H; ++k) z += w[k] * x[k];
        const double s = row_scale(reduction, grad_output, i, n_valid);
        const double gv = s * (exp(z - lse[i]) - (v == t[i] ? 1.0 : 0.0));
        for (int64_t k = 0; k < H; ++k) acc[k] += gv * x[k];
      }
      for (int64_t k = 0; k < H; ++k) dW_rows[r * H + k] = acc[k];
    }
    free(acc);
  }
  return err ? ORACLE_E_MEM : ORACLE_OK;
}

/*
 * The method with its optional parts, for small cases (the whole gradient
 * matrix G [BT, V] is held in memory).
 *
 *   bias (PR #1554, Tests: the ignored-row cases run with bias on and off):
 *       z[i,v] = sum_k X[i,k] W[v,k] + b[v];  grad_bias[v] = sum_i G[i,v].
 *   per-token outputs (PR #1554, Details item 1 and Tests: per-token loss,
 *   z-loss, accuracy and predicted token; ignored rows get 0, 0, 0 and -1).
 *   The pages do not define them; the readings used here are:
 *       predicted_i = argmax_v z[i,v], the lowest such v on ties;
 *       accuracy_i  = 1 if predicted_i == t_i else 0;
 *       z-loss_i    = lse_i^2, the squared log-partition function.
 *   z-loss coefficient lam >= 0 (reading: when non-zero the term lam*lse_i^2
 *   joins the per-row loss and the gradient follows it):
 *       loss_i = lse_i - z[i,t_i] + lam * lse_i^2
 *       G[i,v] = s_i * ((1 + 2 lam lse_i) softmax(z_i)_v - [v == t_i])
 *   Reduced per-token outputs (mean / sum) follow the loss: the sum over
 *   labelled rows, divided by N for mean (0 when N == 0).
 *
 * Arguments as oracle_flce, plus:
 *   bias [V] or NULL; lam; grad_bias [V] or NULL (overwritten, or added to
 *   when accumulate != 0); zl, acc: NULL or [1] (mean/sum) / [BT] (none);
 *   pred: NULL or [BT].  dX, dW may be NULL (not computed).
 */
int oracle_flce_ex(const double* X, const double* W, const double* bias, const int64_t* t,
                   int64_t BT, int64_t H, int64_t V, int64_t ignore_index, int reduction,
                   const double* grad_output, double lam, int accumulate, double* loss,
                   double* dX, double* dW, double* grad_bias, double* zl, double* acc,
                   int64_t* pred) {
  if (BT < 0 || H < 1 || V < 1 || lam < 0.0) return ORACLE_E_ARG;
  if (reduction < ORACLE_MEAN || reduction > ORACLE_NONE) return ORACLE_E_ARG;
  const size_t nb = (size_t)(BT > 0 ? BT : 1);
  int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * nb);
  double* G = (double*)calloc(nb * (size_t)V, sizeof(double));
  double* z = (double*)malloc(sizeof(double) * (size_t)V);
  double* lrow = (double*)calloc(nb, sizeof(double));
  double* zrow = (double*)calloc(nb, sizeof(double));
  double* arow = (double*)calloc(nb, sizeof(double));
  int rc = ORACLE_OK;
  int64_t N = 0;
  if (!idx || !G || !z || !lrow || !zrow || !arow) rc = ORACLE_E_MEM;
  if (rc == ORACLE_OK) rc = oracle_compact(t, BT, V, ignore_index, idx, &N);
  if (rc != ORACLE_OK) {
    free(idx); free(G); free(z); free(lrow); free(zrow); free(arow);
    return rc;
  }
  if (pred)
    for (int64_t i = 0; i < BT; ++i) pred[i] = -1;

  /* Rows: logits with bias, log-sum-exp, per-token outputs, G. */
  for (int64_t n = 0; n < N; ++n) {
    const int64_t i = idx[n];
    logits_row(X, W, H, V, i, z);
    if (bias)
      for (int64_t v = 0; v < V; ++v) z[v] += bias[v];
    const double l = logsumexp_row(z, V);
    int64_t am = 0;
    for (int64_t v = 1; v < V; ++v)
      if (z[v] > z[am]) am = v;
    lrow[i] = l - z[t[i]] + lam * l * l;
    zrow[i] = l * l;
    arow[i] = (am == t[i]) ? 1.0 : 0.0;
    if (pred) pred[i] = am;
    const double s = row_scale(reduction, grad_output, i, N);
    for (int64_t v = 0; v < V; ++v)
      G[i * V + v] = s * ((1.0 + 2.0 * lam * l) * exp(z[v] - l) - (v == t[i] ? 1.0 : 0.0));
  }

  /* Loss and per-token outputs: per row (none), or reduced over labelled rows. */
  if (reduction == ORACLE_NONE) {
    for (int64_t i = 0; i < BT; ++i) {
      loss[i] = lrow[i];
      if (zl) zl[i] = zrow[i];
      if (acc) acc[i] = arow[i];
    }
  } else {
    double sl = 0.0, sz = 0.0, sa = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      sl += lrow[idx[n]];
      sz += zrow[idx[n]];
      sa += arow[idx[n]];
    }
    const double d = (reduction == ORACLE_MEAN) ? (N > 0 ? (double)N : 0.0) : 1.0;
    loss[0] = d > 0.0 ? sl / d : 0.0;
    if (zl) zl[0] = d > 0.0 ? sz / d : 0.0;
    if (acc) acc[0] = d > 0.0 ? sa / d : 0.0;
  }

  /* grad_input = G W, grad_weight = G^T X, grad_bias = column sums of G,
   * each summed over the labelled rows only (ascending).  An ignored row is
   * never read: its X row may hold NaN or Inf, and 0 * NaN is NaN, so a sum
   * over every row would let it into dW (PR #1554, Tests: NaN in ignored rows
   * must reach neither the loss nor the gradients).  Its dX row is +0.0. */
  if (dX) {
    for (int64_t i = 0; i < BT; ++i)
      for (int64_t k = 0; k < H; ++k) dX[i * H + k] = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const int64_t i = idx[n];
      for (int64_t k = 0; k < H; ++k) {
        double a = 0.0;
        for (int64_t v = 0; v < V; ++v) a += G[i * V + v] * W[v * H + k];
        dX[i * H + k] = a;
      }
    }
  }
  if (dW)
    for (int64_t v = 0; v < V; ++v)
      for (int64_t k = 0; k < H; ++k) {
        double a = 0.0;
        for (int64_t n = 0; n < N; ++n) a += G[idx[n] * V + v] * X[idx[n] * H + k];
        dW[v * H + k] = accumulate ? dW[v * H + k] + a : a;
      }
  if (grad_bias)
    for (int64_t v = 0; v < V; ++v) {
      double a = 0.0;
      for (int64_t n = 0; n < N; ++n) a += G[idx[n] * V + v];
      grad_bias[v] = accumulate ? grad_bias[v] + a : a;
    }
  free(idx); free(G); free(z); free(lrow); free(zrow); free(arow);
  return ORACLE_OK;
}
