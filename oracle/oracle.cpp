// CPU fp64 oracle for the activation-sparse ReLU FFN in TwELL form.
//
// TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls this
// file: only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
// shares no code, header, table or constant with the HIP library.
//
// Plain loops, fp64 everywhere, OpenMP across independent rows.  Each function names
// the passage of the pages it follows.  Pages cited:
//   Page A = upppp.jp TwELL article of 2026-05-11 (sections "What is the waste in LLM
//            FFN layers", "What TwELL and the custom CUDA kernels solve")
//   Page B = innovatopia.jp TwELL news article (section "Editor's commentary")
// Readings where the pages are silent are the ones listed in the design notes
// (plain ReLU FFN with an up bias; contiguous column tiles; ascending-column slots;
// padding (0, 0); true counts; per-tile-row dense remainder as the backup).
//
// Layouts (row-major):
//   x [T, D], W_up [F, D], b [F], W_down [F, D], h/z [T, F], y [T, D]
//   TwELL tile-major: counts [n_t, T] (uint16), vals [n_t, T, W], cols [n_t, T, W]
//   (uint8 local column), backup entries in ascending (tile, token) order, each a
//   dense K-wide slice holding the nonzeros of rank >= W.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

// fp64 -> fp32 (nearest) -> bf16 (nearest, ties to even), returned as its fp64 value.
static double round_to_bf16_value(double v) {
  float f = (float)v;
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  u &= 0xFFFF0000u;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

extern "C" {

// O1 + O2.  Up-projection, bias, ReLU (Page A, "What is the waste in LLM FFN layers":
// the FFN expands each token to the hidden width, applies the nonlinearity, and
// projects back).  One fp64 accumulator per output, inputs in ascending order, bias
// added after the sum.  h = z where z > 0, else +0.0.  z may be null.
void oracle_up_relu(const double* x, const double* W_up, const double* b,
                    int64_t T, int64_t D, int64_t F, double* z, double* h) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t j = 0; j < F; ++j) {
      double acc = 0.0;
      for (int64_t i = 0; i < D; ++i) acc += x[t * D + i] * W_up[j * D + i];
      acc += b[j];
      if (z) z[t * F + j] = acc;
      h[t * F + j] = (acc > 0.0) ? acc : 0.0;
    }
  }
}

// O3.  TwELL pack (Page A, "What TwELL and the custom CUDA kernels solve": the hidden
// columns are split into tiles and each tile keeps an ELL layout, so every token row
// stores its nonzero values and their column positions inside each tile; Page A,
// same section: a sparse main part plus a few dense backups).
//
// A value is nonzero iff h != 0 (IEEE: -0.0 is zero).  For tile k and token t the
// nonzeros in ascending local column form the list L.  counts = |L| (may exceed W);
// slot s < min(|L|, W) holds L[s]; other slots are (0, 0).  If |L| > W, one backup
// entry (k, t) is appended whose K-wide slice is zero except the entries of rank >= W.
// Entries come out in ascending (k, t).  At most `cap` entries are written; the number
// needed is returned through n_backup.  Returns 0, or 1 if cap was too small.
int oracle_pack(const double* h, int64_t T, int64_t F, int64_t K, int64_t W,
                uint16_t* counts, double* vals, uint8_t* cols,
                int64_t cap, int32_t* bk_tile, int32_t* bk_tok, double* bk_vals,
                int64_t* n_backup) {
  const int64_t nt = F / K;
  int64_t nb = 0;
  for (int64_t k = 0; k < nt; ++k) {
    for (int64_t t = 0; t < T; ++t) {
      const double* row = h + t * F + k * K;
      double* v = vals + (k * T + t) * W;
      uint8_t* c = cols + (k * T + t) * W;
      for (int64_t s = 0; s < W; ++s) { v[s] = 0.0; c[s] = 0; }
      int64_t n = 0;
      double* slice = nullptr;
      for (int64_t col = 0; col < K; ++col) {
        if (row[col] != 0.0) {
          if (n < W) {
            v[n] = row[col];
            c[n] = (uint8_t)col;
          } else {
            if (n == W) {  // first overflow element of this tile-row: open an entry
              if (nb < cap) {
                bk_tile[nb] = (int32_t)k;
                bk_tok[nb] = (int32_t)t;
                slice = bk_vals + nb * K;
                for (int64_t q = 0; q < K; ++q) slice[q] = 0.0;
              }
              ++nb;
            }
            if (slice) slice[col] = row[col];
          }
          ++n;
        }
      }
      counts[k * T + t] = (uint16_t)n;
    }
  }
  *n_backup = nb;
  return nb > cap ? 1 : 0;
}

// O4.  Unpack: main slots s < min(count, W) plus the backup slices, scattered into a
// zeroed dense [T, F].  Inverse of O3 up to the sign of zero.
void oracle_unpack(const uint16_t* counts, const double* vals, const uint8_t* cols,
                   int64_t n_bk, const int32_t* bk_tile, const int32_t* bk_tok,
                   const double* bk_vals, int64_t T, int64_t F, int64_t K, int64_t W,
                   double* h) {
  const int64_t nt = F / K;
  std::memset(h, 0, sizeof(double) * (size_t)(T * F));
  for (int64_t k = 0; k < nt; ++k)
    for (int64_t t = 0; t < T; ++t) {
      int64_t c = counts[k * T + t];
      int64_t m = c < W ? c : W;
      for (int64_t s = 0; s < m; ++s)
        h[t * F + k * K + cols[(k * T + t) * W + s]] = vals[(k * T + t) * W + s];
    }
  for (int64_t e = 0; e < n_bk; ++e)
    for (int64_t q = 0; q < K; ++q) {
      double v = bk_vals[e * K + q];
      if (v != 0.0) h[(int64_t)bk_tok[e] * F + (int64_t)bk_tile[e] * K + q] = v;
    }
}

// O5.  Dense down-projection y[t,:] = sum_j h[t,j] * W_down[j,:], j ascending
// (Page A, "What is the waste in LLM FFN layers").
void oracle_down_dense(const double* h, const double* W_down, int64_t T, int64_t D,
                       int64_t F, double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* yr = y + t * D;
    for (int64_t d = 0; d < D; ++d) yr[d] = 0.0;
    for (int64_t j = 0; j < F; ++j) {
      double a = h[t * F + j];
      const double* w = W_down + j * D;
      for (int64_t d = 0; d < D; ++d) yr[d] += a * w[d];
    }
  }
}

// O6.  Sparse down-projection over the stored entries only (Page A, "What is the waste
// in LLM FFN layers": products with zero activations are the wasted work).  Tiles in
// ascending order; inside a tile the main slots (ascending column) are followed by the
// backup remainder (ranks >= W, also ascending column), i.e. the same order as O5.
// The backup entry of (k, t) is found through a (k, t) -> entry map of the entry list.
void oracle_down_sparse(const uint16_t* counts, const double* vals, const uint8_t* cols,
                        int64_t n_bk, const int32_t* bk_tile, const int32_t* bk_tok,
                        const double* bk_vals, const double* W_down, int64_t T, int64_t D,
                        int64_t F, int64_t K, int64_t W, double* y) {
  const int64_t nt = F / K;
  // entry index per (k, t), or -1
  std::vector<int64_t> ent((size_t)(nt * T), -1);
  for (int64_t e = 0; e < n_bk; ++e) ent[(size_t)((int64_t)bk_tile[e] * T + bk_tok[e])] = e;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* yr = y + t * D;
    for (int64_t d = 0; d < D; ++d) yr[d] = 0.0;
    for (int64_t k = 0; k < nt; ++k) {
      int64_t c = counts[k * T + t];
      int64_t m = c < W ? c : W;
      for (int64_t s = 0; s < m; ++s) {
        double a = vals[(k * T + t) * W + s];
        const double* w = W_down + (k * K + cols[(k * T + t) * W + s]) * D;
        for (int64_t d = 0; d < D; ++d) yr[d] += a * w[d];
      }
      int64_t e = ent[(size_t)(k * T + t)];
      if (e >= 0) {
        for (int64_t q = 0; q < K; ++q) {
          double a = bk_vals[e * K + q];
          if (a == 0.0) continue;
          const double* w = W_down + (k * K + q) * D;
          for (int64_t d = 0; d < D; ++d) yr[d] += a * w[d];
        }
      }
    }
  }
}

// O9.  Backward of y = relu(x W_up^T + b) W_down with loss sum(y * g), from the stored
// activations h (Page A, "What TwELL and the custom CUDA kernels solve": training runs
// the whole backward pass from the hybrid sparse-main + dense-backup representation).
// The ReLU mask is the set of stored positions (h != 0).
//   dW_down[j,:] = sum_t h[t,j] g[t,:]
//   dh[t,j]      = [h[t,j] != 0] * sum_d g[t,d] W_down[j,d]
//   db[j]        = sum_t dh[t,j]
//   dW_up[j,:]   = sum_t dh[t,j] x[t,:]
//   dx[t,:]      = sum_j dh[t,j] W_up[j,:]
// Sums run in ascending index order.  dh may be null.  With round_dh, dh is stored in bf16
// (nearest-even, the O8 model) before it is used, as a bf16 TwELL of dh holds it; dh_out
// then returns the rounded values.
void oracle_backward(const double* x, const double* h, const double* g,
                     const double* W_up, const double* W_down, int64_t T, int64_t D,
                     int64_t F, int32_t round_dh, double* dx, double* dW_up, double* dW_down,
                     double* db, double* dh_out) {
  std::vector<double> dh((size_t)(T * F), 0.0);
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < F; ++j) {
      if (h[t * F + j] == 0.0) continue;
      double acc = 0.0;
      for (int64_t d = 0; d < D; ++d) acc += g[t * D + d] * W_down[j * D + d];
      dh[(size_t)(t * F + j)] = round_dh ? round_to_bf16_value(acc) : acc;
    }
  if (dh_out) std::memcpy(dh_out, dh.data(), sizeof(double) * (size_t)(T * F));
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < F; ++j) {
    double* a = dW_down + j * D;
    double* u = dW_up + j * D;
    for (int64_t d = 0; d < D; ++d) { a[d] = 0.0; u[d] = 0.0; }
    double bsum = 0.0;
    for (int64_t t = 0; t < T; ++t) {
      double hv = h[t * F + j];
      double gv = dh[(size_t)(t * F + j)];
      for (int64_t d = 0; d < D; ++d) a[d] += hv * g[t * D + d];
      for (int64_t d = 0; d < D; ++d) u[d] += gv * x[t * D + d];
      bsum += gv;
    }
    db[j] = bsum;
  }
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* r = dx + t * D;
    for (int64_t d = 0; d < D; ++d) r[d] = 0.0;
    for (int64_t j = 0; j < F; ++j) {
      double gv = dh[(size_t)(t * F + j)];
      const double* w = W_up + j * D;
      for (int64_t d = 0; d < D; ++d) r[d] += gv * w[d];
    }
  }
}

// O9's per-token half for many tokens at once, without the weight gradients: dh and dx of
// every given row (Page A, "What TwELL and the custom CUDA kernels solve": the backward runs
// from the stored hybrid form; the ReLU mask is the set of stored positions h != 0).
//   dh[t,j] = [h[t,j] != 0] * sum_d g[t,d] W_down[j,d]   (bf16-rounded with round_dh)
// Both sums run in ascending index order, as in oracle_backward; only the products with a
// zero dh (which add nothing) are skipped, so the work follows the stored nonzeros.
void oracle_dh_rows(const double* h, const double* g, const double* W_down, int64_t T,
                    int64_t D, int64_t F, int32_t round_dh, double* dh) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < F; ++j) {
      double v = 0.0;
      if (h[t * F + j] != 0.0) {
        double acc = 0.0;
        for (int64_t d = 0; d < D; ++d) acc += g[t * D + d] * W_down[j * D + d];
        v = round_dh ? round_to_bf16_value(acc) : acc;
      }
      dh[(size_t)(t * F + j)] = v;
    }
}

//   dx[t,:] = sum_j dh[t,j] W_up[j,:]   (rows of a given dh [T, F])
void oracle_dx_rows(const double* dh, const double* W_up, int64_t T, int64_t D, int64_t F,
                    double* dx) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < T; ++t) {
    double* r = dx + t * D;
    for (int64_t d = 0; d < D; ++d) r[d] = 0.0;
    for (int64_t j = 0; j < F; ++j) {
      const double gv = dh[(size_t)(t * F + j)];
      if (gv == 0.0) continue;
      const double* w = W_up + j * D;
      for (int64_t d = 0; d < D; ++d) r[d] += gv * w[d];
    }
  }
}

// O9's weight gradients as sums over the tokens of the stored activations:
//   dW[j,:] = sum_t a[t,j] b[t,:]   and   colsum[j] = sum_t a[t,j]   (ascending t)
// with (a, b) = (h, g) for dW_down and (dh, x) for dW_up and db (Page A, "What TwELL and
// the custom CUDA kernels solve": training from the hybrid form).  Tokens with a[t,j] == 0
// add nothing and are skipped, so the work follows the stored nonzeros.  colsum may be null.
void oracle_dw(const double* a, const double* b, int64_t T, int64_t D, int64_t F, double* dW,
               double* colsum) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t j = 0; j < F; ++j) {
    double* u = dW + j * D;
    for (int64_t d = 0; d < D; ++d) u[d] = 0.0;
    double s = 0.0;
    for (int64_t t = 0; t < T; ++t) {
      const double av = a[(size_t)(t * F + j)];
      if (av == 0.0) continue;
      for (int64_t d = 0; d < D; ++d) u[d] += av * b[t * D + d];
      s += av;
    }
    if (colsum) colsum[j] = s;
  }
}

// The dh-consuming half of O9 for a given dh [T, F] (as a layer stores it): dW_up, db and
// dx exactly as oracle_backward computes them from its own dh.
//   dW_up[j,:] = sum_t dh[t,j] x[t,:];  db[j] = sum_t dh[t,j];  dx[t,:] = sum_j dh[t,j] W_up[j,:]
void oracle_backward_from_dh(const double* x, const double* dh, const double* W_up, int64_t T,
                             int64_t D, int64_t F, double* dx, double* dW_up, double* db) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < F; ++j) {
    double* u = dW_up + j * D;
    for (int64_t d = 0; d < D; ++d) u[d] = 0.0;
    double bsum = 0.0;
    for (int64_t t = 0; t < T; ++t) {
      const double gv = dh[t * F + j];
      for (int64_t d = 0; d < D; ++d) u[d] += gv * x[t * D + d];
      bsum += gv;
    }
    db[j] = bsum;
  }
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double* r = dx + t * D;
    for (int64_t d = 0; d < D; ++d) r[d] = 0.0;
    for (int64_t j = 0; j < F; ++j) {
      const double gv = dh[t * F + j];
      const double* w = W_up + j * D;
      for (int64_t d = 0; d < D; ++d) r[d] += gv * w[d];
    }
  }
}

// O1..O3 + O6 for a chosen set of token rows (the FFN acts on each token on its own:
// Page A, "What is the waste in LLM FFN layers"), without materialising [T, F].
// Outputs per selected row r: y_rows[r, D], counts_rows[r, n_t] (true counts) and, if
// z_rows is not null, the pre-activations.  With round_h the stored activation values
// follow the O8 rounding model (bf16, nearest-even) before the down-projection, as a
// bf16 TwELL stores them.  Used for sampled checks at full layer sizes.
void oracle_ffn_rows(const double* x, const double* W_up, const double* b,
                     const double* W_down, const int64_t* rows, int64_t n_rows, int64_t D,
                     int64_t F, int64_t K, int64_t W, int32_t round_h, double* y_rows,
                     uint16_t* counts_rows, double* z_rows) {
  const int64_t nt = F / K;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n_rows; ++r) {
    const double* xr = x + rows[r] * D;
    std::vector<double> h((size_t)F);
    for (int64_t j = 0; j < F; ++j) {
      double acc = 0.0;
      for (int64_t i = 0; i < D; ++i) acc += xr[i] * W_up[j * D + i];
      acc += b[j];
      if (z_rows) z_rows[r * F + j] = acc;
      double hv = acc > 0.0 ? acc : 0.0;
      if (round_h && hv != 0.0) hv = round_to_bf16_value(hv);
      h[(size_t)j] = hv;
    }
    double* yr = y_rows + r * D;
    for (int64_t d = 0; d < D; ++d) yr[d] = 0.0;
    for (int64_t k = 0; k < nt; ++k) {
      // main slots then remainder, both ascending: the column order within the tile
      int64_t n = 0;
      for (int64_t col = 0; col < K; ++col) {
        double a = h[(size_t)(k * K + col)];
        if (a == 0.0) continue;
        const double* w = W_down + (k * K + col) * D;
        for (int64_t d = 0; d < D; ++d) yr[d] += a * w[d];
        ++n;
      }
      counts_rows[r * nt + k] = (uint16_t)n;
    }
  }
}

// O8.  Rounding model for comparisons: fp64 -> fp32 (nearest) -> bfloat16 (nearest,
// ties to even), returned as bit patterns.  NaN is outside the contract.
void oracle_round_bf16(const double* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    float f = (float)in[i];
    uint32_t u;
    std::memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    out[i] = (uint16_t)(u >> 16);
  }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

}  // extern "C"
