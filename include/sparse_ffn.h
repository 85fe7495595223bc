/* sparse_ffn.h -- C ABI of the activation-sparse ReLU FFN layer in TwELL form (MI355X / gfx950).
 *
 * The layer (upppp.jp TwELL article of 2026-05-11, section "What is the waste in LLM FFN
 * layers"): y = ReLU(x W_up^T + b) W_down, applied to each token on its own.  Most hidden
 * activations are zero, so the library packs them into TwELL (same article, section "What
 * TwELL and the custom CUDA kernels solve": hidden columns split into tiles, an ELL layout
 * inside each tile, plus a few dense backups for what does not fit).  The down-projection
 * reads only that packed form: its vector kernels multiply the stored nonzeros only, its
 * matrix-core kernels rebuild each tile in on-chip memory and contract it there.  On the
 * forward path of more than 128 tokens the dense hidden tensor never reaches device memory;
 * a batch of at most 128 tokens keeps its fp32 hidden rows (T x d_ff) in the workspace
 * between the small-batch up-projection and the pack.
 *
 * Conventions
 *   - Pointers are DEVICE pointers unless marked (host).  Row-major layouts.
 *     x [T, d_model], W_up [d_ff, d_model], b_up [d_ff], W_down [d_ff, d_model],
 *     y [T, d_model]; row j of W_down is neuron j's output weights.
 *   - Element type of x, weights, bias, y and TwELL values: sffn_config_t.dtype.  All
 *     accumulation is fp32; results are rounded to nearest-even into dtype.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are asynchronous on it
 *     unless marked (sync).  The caller keeps every buffer alive until the work finishes.
 *   - Errors are status codes; no call aborts or throws.  Arguments are validated on the
 *     host before anything is launched.  A HIP failure gives SFFN_ERR_DEVICE and the HIP
 *     message in sffn_last_error().  Device-side overflow of the backup capacity is
 *     reported through the buffers' status word: outputs of that call are then undefined,
 *     and twell_stats / sparse_ffn_check return SFFN_ERR_BACKUP_OVERFLOW.
 *   - The library allocates no device memory.  Every device buffer is the caller's.  (A
 *     handle under the auto down policy keeps one word of pinned host memory: see
 *     sparse_ffn_set_down_policy.)
 *
 * TwELL layout written by twell_pack and sparse_ffn_forward (n_t = d_ff / tile tiles,
 * "tile-row (k, t)" = token t restricted to the tile's columns [k*tile, (k+1)*tile)):
 *   counts [n_t, T]    uint16  true number of nonzeros of tile-row (k, t) (may exceed W)
 *   vals   [n_t, T, W] dtype   first min(count, W) nonzeros in ascending column; then 0
 *   cols   [n_t, T, W] uint8   their local column in 0..tile-1; then 0
 *   backup, one entry per tile-row with count > W, in ascending (tile, token) order:
 *   bk_tile[e], bk_tok[e] int32, bk_vals[e, tile] dtype = the nonzeros of rank >= W at
 *   their local column, zero elsewhere (the "dense backup" of the hybrid form).
 */
#ifndef SPARSE_FFN_H_
#define SPARSE_FFN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SFFN_OK = 0,
  SFFN_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, T out of range, ... */
  SFFN_ERR_UNSUPPORTED = 2,      /* valid but not implemented (shape constraint, dtype) */
  SFFN_ERR_BACKUP_OVERFLOW = 3,  /* more overflowing tile-rows than backup_capacity */
  SFFN_ERR_DEVICE = 4            /* a HIP call failed; see sffn_last_error() */
} sffn_status_t;

typedef enum { SFFN_F32 = 0, SFFN_BF16 = 1 } sffn_dtype_t;

/* Largest number of tiles (d_ff / tile) a configuration may have (SFFN_ERR_UNSUPPORTED
 * beyond it): the ordering pass keeps one offset per tile in workgroup-local memory. */
#define SFFN_MAX_TILES 4096

typedef struct {
  int32_t d_model;         /* D: multiple of 64 (layers in bf16: of 128) */
  int32_t d_ff;            /* F: multiple of tile (layers in bf16: also of 256), F / tile <= SFFN_MAX_TILES */
  int32_t tile;            /* K: hidden columns per tile, one of 64, 128, 256 */
  int32_t ell_width;       /* W: ELL slots per tile-row, 1 <= W <= tile */
  int32_t max_tokens;      /* largest T any call may pass (1 <= T <= max_tokens <= 2^24) */
  int32_t backup_capacity; /* backup entries the buffers hold (0 allowed) */
  sffn_dtype_t dtype;      /* SFFN_BF16 (MFMA up-projection) or SFFN_F32 */
} sffn_config_t;

/* Caller-owned device buffers for one packed activation of T tokens.  Sizes come from
 * twell_buffer_sizes().  The same struct holds the forward pass's packed activations
 * (the saved activations of a training step). */
typedef struct {
  uint16_t *counts;      /* [n_t, T] */
  void *vals;            /* [n_t, T, W] dtype */
  uint8_t *cols;         /* [n_t, T, W] */
  int32_t *bk_tile;      /* [backup_capacity] */
  int32_t *bk_tok;       /* [backup_capacity] */
  void *bk_vals;         /* [backup_capacity, tile] dtype */
  int32_t *bk_tile_ptr;  /* [n_t + 1] entries of tile k are e in [ptr[k], ptr[k+1]) */
  int32_t *bk_n;         /* [1] backup entries needed (may exceed the capacity) */
  int32_t *status;       /* [1] device status word: 0, or SFFN_ERR_BACKUP_OVERFLOW */
  void *workspace;       /* scratch: unordered backup staging, per-group, per-tile and per-block
                            counters, the first canonical backup entry of every (tile, group)
                            (read by sparse_ffn_down and sparse_ffn_backward: keep it with its
                            TwELL), and fp32 partial sums of the small-batch paths */
} twell_buffers_t;

/* Byte sizes of each field of twell_buffers_t for T tokens.  Each buffer must be at
 * least this large and 256-byte aligned (torch allocations are).  counts, vals and cols
 * hold 32 tile-rows of padding after [n_t, T(, W)] (read by whole-group and whole-word
 * loads, never used).  Buffers sized for T serve any call with fewer tokens. */
typedef struct {
  size_t counts, vals, cols, bk_tile, bk_tok, bk_vals, bk_tile_ptr, bk_n, status, workspace;
} twell_buffer_sizes_t;

/* Counters of one packed activation, computed on the device from the counts. */
typedef struct {
  int64_t nnz;                /* stored nonzeros, main + backup */
  int64_t slots_used;         /* sum over tile-rows of min(count, W) */
  int64_t overflow_tile_rows; /* tile-rows with count > W (= backup entries needed) */
  int64_t backup_nonzeros;    /* sum of max(count - W, 0) */
  int64_t backup_needed;      /* entries the pass asked for (bk_n) */
  int32_t max_count;          /* largest count of any tile-row */
  int32_t backup_overflowed;  /* 1 if backup_needed > backup_capacity */
  double density;             /* nnz / (T * d_ff) */
  double ell_fill;            /* slots_used / (n_t * T * W) */
  int64_t bytes_main;         /* counts + vals + cols bytes */
  int64_t bytes_backup;       /* bytes of the backup entries in use */
  int64_t bytes_dense_equiv;  /* T * d_ff * sizeof(dtype): the dense hidden tensor */
} twell_stats_t;

typedef struct sparse_ffn *sparse_ffn_t;

/* Status name ("SFFN_OK", ...) for a code; never NULL.  Interface of the library (the
 * pages define no API): error reporting by status codes only. */
const char *sffn_status_string(sffn_status_t s);

/* Message of the last failing call on this host thread ("" if none).  Interface of the
 * library; the string is owned by the library and valid until the next failing call on
 * the same thread. */
const char *sffn_last_error(void);

/* (host only) Sizes of the twell_buffers_t fields for T tokens: the storage of the
 * TwELL main part (counts, values, local column indices) and of the dense backup
 * (upppp.jp TwELL article of 2026-05-11, section "What TwELL and the custom CUDA kernels
 * solve": per-tile ELL rows plus a few dense backups), and the scratch workspace.
 * Validates cfg and T; *out is written only on SFFN_OK. */
sffn_status_t twell_buffer_sizes(const sffn_config_t *cfg, int32_t T, twell_buffer_sizes_t *out);

/* Number of buffers of twell_buffers_t, in its field order. */
#define SFFN_N_BUFFERS 10

/* (host only) The same sizes as twell_buffer_sizes, as an array in the field order of
 * twell_buffers_t: counts, vals, cols, bk_tile, bk_tok, bk_vals, bk_tile_ptr, bk_n,
 * status, workspace.  out_bytes (host) must hold SFFN_N_BUFFERS entries; it is written
 * only on SFFN_OK. */
sffn_status_t twell_buffer_bytes(const sffn_config_t *cfg, int32_t T,
                                 size_t out_bytes[SFFN_N_BUFFERS]);

/* (host only, no device work) Create a handle for one ReLU FFN layer
 * y = ReLU(x W_up^T + b) W_down (upppp.jp TwELL article of 2026-05-11, section "What is
 * the waste in LLM FFN layers": an up-projection that widens each token, an activation,
 * a down-projection back).  Beyond the checks every call makes, a bf16 layer needs
 * d_model % 128 == 0 and d_ff % 256 == 0 (SFFN_ERR_UNSUPPORTED otherwise).  The weights
 * are borrowed device pointers: they must stay valid while the handle is used and may be
 * updated in place between calls; nothing derived from their values is kept (the auto
 * down policy keeps one word about the last call's density, see sparse_ffn_set_down_policy).
 * b_up may not be NULL (pass zeros for a bias-free layer).  *out is written only on SFFN_OK. */
sffn_status_t sparse_ffn_create(const sffn_config_t *cfg, const void *W_up, const void *b_up,
                                const void *W_down, sparse_ffn_t *out);

/* (host only) Release a handle created by sparse_ffn_create; NULL is accepted.
 * Interface of the library: no device memory is owned, so nothing on the device is
 * released or waited for (the auto down policy's word of pinned host memory stays with the
 * library and is never given to another handle, so work of the handle still running, or a
 * recorded graph replayed later, writes only that word). */
sffn_status_t sparse_ffn_destroy(sparse_ffn_t h);

/* Pack a dense fp32 hidden tensor h [T, d_ff] into TwELL (same article, section "What
 * TwELL and the custom CUDA kernels solve").  A value is nonzero iff h != 0 (-0.0 is
 * zero).  Values are stored in cfg->dtype (rounded to nearest-even for bf16).  Writes
 * every field of `buf`, including the backup in canonical order and the status word. */
sffn_status_t twell_pack(const sffn_config_t *cfg, const float *h, int32_t T,
                         const twell_buffers_t *buf, void *stream);

/* Forward pass y = ReLU(x W_up^T + b) W_down for T tokens (upppp.jp TwELL article of
 * 2026-05-11, sections "What is the waste in LLM FFN layers" and "What TwELL and the
 * custom CUDA kernels solve": the activations are packed into TwELL by the up-projection
 * kernel itself and the down-projection runs over the stored nonzeros; innovatopia.jp
 * TwELL article, "Editor's commentary": no extra memory traffic for the format).  The
 * up-projection kernel applies bias and ReLU in fp32 (nonzero iff the fp32
 * pre-activation is > 0) and packs the result into `act` on the fly; the down-projection
 * then reads only the stored entries (main slots and backup).  x [T, d_model] and y
 * [T, d_model] are device buffers in the layer dtype; `act` (sized for at least T tokens)
 * doubles as the saved activations.  Host-side argument errors return before any launch;
 * a backup overflow is reported through act->status (outputs then undefined). */
sffn_status_t sparse_ffn_forward(sparse_ffn_t h, const void *x, int32_t T, void *y,
                                 const twell_buffers_t *act, void *stream);

/* Down-projection only, y = unpack(act) W_down, from a TwELL that twell_pack or
 * sparse_ffn_forward wrote for the same T.  Same arithmetic as the forward's second half.
 * act->workspace must be given (the per-block kernel choice is staged there). */
sffn_status_t sparse_ffn_down(sparse_ffn_t h, const twell_buffers_t *act, int32_t T, void *y,
                              void *stream);

/* Backward pass of sparse_ffn_forward (same article, section "What TwELL and the custom
 * CUDA kernels solve": training works on the same hybrid representation, with no dense
 * hidden tensor).  Inputs: the forward's x [T, d_model] and act (its packed activations h,
 * workspace included, unchanged since that forward), and dy = dL/dy [T, d_model], all in the
 * layer dtype.  With g = dy and the ReLU mask taken as the stored positions of act:
 *   dh[t, j]      = sum_d g[t, d] W_down[j, d]   at every stored position of h
 *   dW_down[j, :] = sum_t h[t, j] g[t, :]
 *   dW_up[j, :]   = sum_t dh[t, j] x[t, :]
 *   db_up[j]      = sum_t dh[t, j]
 *   dx[t, :]      = sum_j dh[t, j] W_up[j, :]
 * Outputs (device, overwritten): dh_vals [n_t, T, W] and dh_bk_vals [backup_capacity, tile]
 * (dtype; dh in the TwELL structure of act: act's counts, cols and backup entries index it;
 * values rounded to nearest-even), dx [T, d_model] dtype, dW_up and dW_down [d_ff, d_model]
 * fp32, db_up [d_ff] fp32 (may be NULL: then not computed).  Accumulation is fp32.
 * Needs a bf16 layer with tile 128 or 256, ell_width in {16, 32, 48, 64} and d_model % 256
 * == 0 (SFFN_ERR_UNSUPPORTED otherwise).  If act's status word reports a backup overflow the
 * outputs are undefined. */
sffn_status_t sparse_ffn_backward(sparse_ffn_t h, const void *x, const void *dy, int32_t T,
                                  const twell_buffers_t *act, void *dh_vals, void *dh_bk_vals,
                                  void *dx, float *dW_up, float *dW_down, float *db_up,
                                  void *stream);

/* Which kernel runs the down-projection (inside sparse_ffn_forward and sparse_ffn_down).
 * The TwELL tiles line up with tiled matrix-multiply execution (same article, section "What
 * TwELL and the custom CUDA kernels solve"), so the layer can gather the W_down rows its
 * stored nonzeros select on the vector ALUs (work grows with the nonzeros) or rebuild its
 * hidden tiles in on-chip memory and run them through the matrix cores (work independent of
 * the density, at ~16x the vector rate).  Three kernels:
 *   gather: one token at a time, W_down rows read straight from memory (cheapest when very
 *           few rows are used);
 *   tiles:  256 tokens share each W_down tile staged in LDS, two nonzeros per bf16
 *           dot-product instruction (bf16 layers with an even ell_width <= 128);
 *   mfma:   hidden tiles rebuilt in LDS, matrix-core contraction (bf16 layers with
 *           ell_width in {16, 32, 48, 64});
 *   union:  the matrix-core contraction of each 64-token block over only the columns where
 *           one of its tokens has a stored nonzero (the block's column union, per 64-column
 *           step; a step whose union leaves no 16-column k-step to skip runs densely), so
 *           the matrix-core work falls with the density (same shapes as mfma);
 *   sparse: the 2:4 structured-sparse matrix-core instruction: each stored nonzero goes to
 *           its rank within its four-column group, ranks 0-1 in one compressed plane and
 *           2-3 in a second that is contracted only where it holds a value, so a step costs
 *           half a dense one where no group has three nonzeros (same shapes as mfma).
 * Policies:
 *   SFFN_DOWN_AUTO:   by the layer's stored density (stored nonzeros / (T d_ff)): gather up to
 *                     gather_density, tiles up to mfma_density, mfma above; the count is taken
 *                     on the device, so the choice costs no host synchronisation (the default,
 *                     with the *_DEFAULT thresholds).  A kernel the layer does not support
 *                     hands its range to the next one down (mfma -> tiles -> gather), and so
 *                     do tiles below SFFN_DOWN_TILES_MIN_T tokens (its 256-token workgroups
 *                     walk every tile in turn and need many tokens to fill the GPU) and mfma
 *                     below SFFN_DOWN_MFMA_MIN_T (a handful of tokens: it contracts whole
 *                     256-token blocks and reads all of W_down, where the gather reads only
 *                     the rows in use).  With few tokens the mfma kernel splits the tiles
 *                     over more workgroups and adds the parts' fp32 sums in a fixed order.
 *                     Every candidate is correct at any density, so the choice is one of
 *                     speed: the first auto call on a handle (and the first after any
 *                     sparse_ffn_set_down_policy) launches every candidate and the count
 *                     decides on the device; the kernel that runs also writes which kernel its
 *                     count selects into a 4-byte word of pinned host memory that the handle
 *                     takes from pages the library keeps until the process ends (by the first
 *                     auto forward or down call, never by sparse_ffn_forward_noalloc or under
 *                     stream capture), and each later call launches that kernel alone.  A
 *                     change of density thus changes the kernel one call later; the result is
 *                     the kernel's that ran.
 *   SFFN_DOWN_GATHER, SFFN_DOWN_TILES, SFFN_DOWN_MFMA, SFFN_DOWN_UNION, SFFN_DOWN_SPARSE:
 *                     always that kernel (tiles, mfma, union and sparse fall back as above
 *                     when the layer does not support them).
 * All accumulate in fp32; they differ only in summation order.  Host only; the setting
 * belongs to the handle.  SFFN_ERR_INVALID_ARGUMENT for an unknown policy or thresholds
 * outside 0 <= gather_density <= mfma_density <= 1. */
#define SFFN_DOWN_AUTO 0
#define SFFN_DOWN_GATHER 1
#define SFFN_DOWN_MFMA 2
#define SFFN_DOWN_TILES 3
#define SFFN_DOWN_UNION 4
#define SFFN_DOWN_SPARSE 5
#define SFFN_DOWN_GATHER_DENSITY_DEFAULT 0.0005f
#define SFFN_DOWN_MFMA_DENSITY_DEFAULT 0.005f
#define SFFN_DOWN_TILES_MIN_T 4096
#define SFFN_DOWN_MFMA_MIN_T 64
/* Set the handle's down-projection policy and the auto policy's two density thresholds
 * (host only; the policies and their kernels are described above). */
sffn_status_t sparse_ffn_set_down_policy(sparse_ffn_t h, int32_t policy, float gather_density,
                                         float mfma_density);

/* (sync) Counters of `buf` for T tokens (the quantities the TwELL format is built from:
 * upppp.jp TwELL article of 2026-05-11, section "What TwELL and the custom CUDA kernels
 * solve" - per-tile nonzero counts, the ELL part's fill and the few dense backups);
 * synchronises `stream`.  *out (host) is filled; returns SFFN_ERR_BACKUP_OVERFLOW (with
 * *out filled) if the status word reports an overflow. */
sffn_status_t twell_stats(const sffn_config_t *cfg, const twell_buffers_t *buf, int32_t T,
                          twell_stats_t *out, void *stream);

/* Bins of a count histogram: counts 0 .. tile, tile <= 256. */
#define SFFN_HIST_BINS 257

/* (sync) Histogram of the tile-row counts of `buf` for T tokens: hist[c] = the number of
 * tile-rows (k, t) that hold c nonzeros, c = 0 .. cfg->tile (host array of cfg->tile + 1
 * entries, written on SFFN_OK).  The per-tile nonzero counts are what the TwELL format is
 * laid out from (upppp.jp TwELL article of 2026-05-11, section "What TwELL and the custom
 * CUDA kernels solve": per-tile ELL rows sized to the nonzeros, with a few dense backups for
 * the rows that do not fit); twell_choose_ell_width picks a width from it.  Computed on the
 * device; synchronises `stream`. */
sffn_status_t twell_count_histogram(const sffn_config_t *cfg, const twell_buffers_t *buf,
                                    int32_t T, int64_t *hist, void *stream);

/* (host only) The ELL width W that stores a packed activation with count histogram `hist`
 * (cfg->tile + 1 host entries, as twell_count_histogram writes it) in the fewest bytes
 * (same section: the hybrid form keeps memory overhead minimal): with R = sum_c hist[c]
 * tile-rows and O(W) = sum_{c > W} hist[c] of them overflowing,
 *   bytes(W) = R (2 + W (esz + 1)) + O(W) (esz tile + 8)
 * (a tile-row's count, its W value and column slots; an overflowing row's dense backup slice
 * and its tile and token indices; esz = bytes per value of cfg->dtype), the same accounting
 * as twell_stats' bytes_main and bytes_backup.  The minimum is taken over the n_candidates
 * widths in `candidates` (host; each in [1, tile]; NULL: every W in [1, tile]); ties go to
 * the smaller W.  cfg->ell_width is not used.  *W_out and *bytes_out (host; bytes_out may be
 * NULL) are written on SFFN_OK; SFFN_ERR_INVALID_ARGUMENT for NULL pointers, negative bins,
 * an empty or out-of-range candidate list. */
sffn_status_t twell_choose_ell_width(const sffn_config_t *cfg, const int64_t *hist,
                                     const int32_t *candidates, int32_t n_candidates,
                                     int32_t *W_out, int64_t *bytes_out);

/* (sync) Synchronise `stream` and return the status word of `buf`: SFFN_OK, or
 * SFFN_ERR_BACKUP_OVERFLOW when more tile-rows overflowed their W slots than the dense
 * backup holds (upppp.jp TwELL article of 2026-05-11, section "What TwELL and the custom
 * CUDA kernels solve": the backup holds only a few rows). */
sffn_status_t sparse_ffn_check(const twell_buffers_t *buf, void *stream);

/* Size of the fixed device scratch of sparse_ffn_forward_noalloc (bytes, per device). */
#define SFFN_NOALLOC_SCRATCH_BYTES (128u << 20)

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): sparse_ffn_forward with its workspace
 * taken from a fixed scratch array inside the library instead of act->workspace, which is
 * ignored (may be NULL).  Same kernels and results as sparse_ffn_forward; no device memory
 * is allocated or freed.  Every device the library runs on holds one such array of
 * SFFN_NOALLOC_SCRATCH_BYTES until the process ends; calls on one device share it and keep
 * the last call's contents, so calls that overlap on one device (other streams, other host
 * threads) race, and the workspace-dependent state of a call (the per-group backup offsets
 * that sparse_ffn_down and sparse_ffn_backward read) does not outlive the next call: the
 * TwELL and backup written into act stay complete and canonical.  Returns
 * SFFN_ERR_UNSUPPORTED, before any launch, when the call's workspace (twell_buffer_sizes'
 * workspace for exactly these T tokens) exceeds the scratch. */
sffn_status_t sparse_ffn_forward_noalloc(sparse_ffn_t h, const void *x, int32_t T, void *y,
                                         const twell_buffers_t *act, void *stream);

/* Test hook: sparse_ffn_forward that also writes the fp32 pre-activation
 * z = x W_up^T + b [T, d_ff] (before ReLU) exactly as the up-projection kernel computed
 * it, so its TwELL can be checked against a pack of the same z. */
sffn_status_t sparse_ffn_forward_dump(sparse_ffn_t h, const void *x, int32_t T, void *y,
                                      const twell_buffers_t *act, float *z, void *stream);

/* Per-kernel timing (measurement interface of the library, not part of the layer): while
 * enabled, every launch of this library on the calling thread is bracketed by HIP events
 * on its stream.  Host only; the event records live in a thread-local host list. */
sffn_status_t sffn_profile_enable(int32_t enable);

/* Restrict the timing to the kernels named in `names` (host string, comma-separated, e.g.
 * "up_pack,down"); NULL or "" times every launch again.  Fewer events perturb the timed
 * stream less. */
sffn_status_t sffn_profile_only(const char *names);

/* Drop every recorded event pair of the calling thread. */
sffn_status_t sffn_profile_reset(void);

/* (sync on the recorded events) For a kernel name ("up_pack", "down", "pack", "order",
 * ...), the summed duration in ms and the number of launches since the last reset
 * (host outputs; SFFN_ERR_INVALID_ARGUMENT for NULL pointers). */
sffn_status_t sffn_profile_read(const char *kernel, double *total_ms, int64_t *launches);

/* Measurement probe (interface of the library, for the benchmark's ceilings):
 *   y[t, :] = sum_j vals[t, j] W[rows[t, j], :]   for t < T, j < n
 * in fp32, rounded to nearest-even into bf16 y.  This is the gather-multiply-add a vector
 * down-projection performs for each stored nonzero - only the W_down rows that a token's
 * nonzero activations select contribute (upppp.jp TwELL article of 2026-05-11, section
 * "What is the waste in LLM FFN layers") - with the row lists given instead of decoded from
 * TwELL, so its rate bounds the vector down kernels on the same rows.  W [F, d] bf16
 * (d = d_model), rows [T, n] int32 (a row outside [0, F) reads row 0 or F-1), vals [T, n]
 * bf16, y [T, d] bf16, all device.  F >= 1, d >= 8 with d % 8 == 0, T >= 1, n >= 0 (n = 0:
 * y = 0, rows and vals may be NULL); SFFN_ERR_INVALID_ARGUMENT otherwise (and for NULL
 * pointers).  Async on `stream`; timed as
 * "probe_gather_fma" by the profiling calls. */
sffn_status_t sffn_probe_gather_fma(const void *W, int32_t F, int32_t d, const int32_t *rows,
                                    const void *vals, int32_t T, int32_t n, void *y,
                                    void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_FFN_H_ */
