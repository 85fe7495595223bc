// Host side of the C ABI declared in include/sparse_ffn.h: argument validation (always
// before any HIP call), buffer sizing, launch sequencing on the caller's stream, status
// reporting and the optional per-kernel event timing.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "sffn_common.hpp"

using namespace sffn;

struct sparse_ffn {
  sffn_config_t cfg;
  const void* W_up;
  const void* b_up;
  const void* W_down;
  int32_t down_policy = SFFN_DOWN_AUTO;
  float down_gather_density = SFFN_DOWN_GATHER_DENSITY_DEFAULT;
  float down_mfma_density = SFFN_DOWN_MFMA_DENSITY_DEFAULT;
  // Auto policy: the kernel the last running down kernel found the layer's count to select
  // (0 gather, 1 tiles, 2 matrix cores, -1 none yet), in one word of pinned host memory that
  // the kernels write; taken by the first auto call that may allocate, reset by a policy
  // change.
  int* hint_host = nullptr;
  int* hint_dev = nullptr;
  bool hint_failed = false;
  std::mutex hint_mu;
};

namespace {

#define SFFN_TRY_INNER(expr)                 \
  do {                                       \
    const sffn_status_t s__ = (expr);        \
    if (s__ != SFFN_OK) return s__;          \
  } while (0)

thread_local std::string g_last_error;

sffn_status_t fail(sffn_status_t s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

sffn_status_t dev_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return SFFN_ERR_DEVICE;
}

// ------------------------------------------------------------------ profiling
struct ProfRec {
  std::string name;
  hipEvent_t e0, e1;
};
struct Prof {
  bool enabled = false;
  std::vector<std::string> only;  // names to time (empty: all)
  std::vector<ProfRec> recs;
  bool times(const char* name) const {
    if (!enabled) return false;
    if (only.empty()) return true;
    for (auto& n : only)
      if (n == name) return true;
    return false;
  }
  ~Prof() { clear(); }
  void clear() {
    for (auto& r : recs) {
      (void)hipEventDestroy(r.e0);
      (void)hipEventDestroy(r.e1);
    }
    recs.clear();
  }
};
thread_local Prof g_prof;

// Launch `f` (returns hipError_t) under the kernel name `name`.
template <typename Fn>
sffn_status_t run(const char* name, hipStream_t s, Fn&& f) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  const bool timed = g_prof.times(name);
  if (timed) {
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess ||
        hipEventRecord(e0, s) != hipSuccess)
      return dev_fail(hipGetLastError(), "profiling event");
  }
  const hipError_t err = f();
  if (timed) {
    (void)hipEventRecord(e1, s);
    g_prof.recs.push_back({name, e0, e1});
  }
  if (err != hipSuccess) return dev_fail(err, name);
  return SFFN_OK;
}

// ------------------------------------------------------------------ validation
sffn_status_t check_cfg(const sffn_config_t* c) {
  if (!c) return fail(SFFN_ERR_INVALID_ARGUMENT, "config is NULL");
  if (c->dtype != SFFN_F32 && c->dtype != SFFN_BF16)
    return fail(SFFN_ERR_INVALID_ARGUMENT, "dtype must be SFFN_F32 or SFFN_BF16");
  if (c->tile != 64 && c->tile != 128 && c->tile != 256)
    return fail(SFFN_ERR_UNSUPPORTED, "tile must be 64, 128 or 256");
  if (c->ell_width < 1 || c->ell_width > c->tile)
    return fail(SFFN_ERR_INVALID_ARGUMENT, "ell_width must be in [1, tile]");
  if (c->d_model <= 0 || c->d_ff <= 0)
    return fail(SFFN_ERR_INVALID_ARGUMENT, "d_model and d_ff must be positive");
  if (c->d_ff % c->tile != 0)
    return fail(SFFN_ERR_INVALID_ARGUMENT, "d_ff must be a multiple of tile");
  if (c->d_model % 64 != 0) return fail(SFFN_ERR_UNSUPPORTED, "d_model must be a multiple of 64");
  if (c->max_tokens < 1 || c->max_tokens > (1 << 24))
    return fail(SFFN_ERR_INVALID_ARGUMENT, "max_tokens must be in [1, 2^24]");
  if (c->backup_capacity < 0) return fail(SFFN_ERR_INVALID_ARGUMENT, "backup_capacity < 0");
  const long long nt = c->d_ff / c->tile;
  if (nt > SFFN_MAX_TILES)
    return fail(SFFN_ERR_UNSUPPORTED, "d_ff / tile must be at most SFFN_MAX_TILES (4096)");
  if ((long long)c->backup_capacity > nt * (long long)c->max_tokens)
    return fail(SFFN_ERR_INVALID_ARGUMENT, "backup_capacity exceeds the number of tile-rows");
  const long long esz = c->dtype == SFFN_BF16 ? 2 : 4;
  if (nt * (long long)c->max_tokens * c->ell_width * esz >= (1LL << 31) ||
      (long long)c->backup_capacity * c->tile * esz >= (1LL << 31))
    return fail(SFFN_ERR_UNSUPPORTED, "TwELL and backup arrays must each stay below 2 GiB");
  return SFFN_OK;
}

// Extra shape constraints of the layer kernels (up-projection and down-projection).
sffn_status_t check_layer_cfg(const sffn_config_t* c) {
  SFFN_TRY_INNER(check_cfg(c));
  if (c->dtype == SFFN_BF16 && c->d_model % 128 != 0)
    return fail(SFFN_ERR_UNSUPPORTED, "bf16 layers need d_model to be a multiple of 128");
  if (c->dtype == SFFN_BF16 && c->d_ff % 256 != 0)
    return fail(SFFN_ERR_UNSUPPORTED, "bf16 layers need d_ff to be a multiple of 256");
  return SFFN_OK;
}

sffn_status_t check_T(const sffn_config_t* c, int32_t T) {
  if (T < 1 || T > c->max_tokens)
    return fail(SFFN_ERR_INVALID_ARGUMENT, "T must be in [1, max_tokens]");
  return SFFN_OK;
}

Dims make_dims(const sffn_config_t* c, int32_t T) {
  Dims d;
  d.D = c->d_model;
  d.F = c->d_ff;
  d.K = c->tile;
  d.W = c->ell_width;
  d.T = T;
  d.nt = c->d_ff / c->tile;
  d.ng = (T + GROUP - 1) / GROUP;
  d.cap = c->backup_capacity;
  d.bf16 = c->dtype == SFFN_BF16;
  d.esz = d.bf16 ? 2 : 4;
  return d;
}

sffn_status_t check_bufs(const twell_buffers_t* b, bool need_all) {
  if (!b) return fail(SFFN_ERR_INVALID_ARGUMENT, "buffers struct is NULL");
  if (!b->counts || !b->vals || !b->cols || !b->bk_tile_ptr || !b->bk_n || !b->status)
    return fail(SFFN_ERR_INVALID_ARGUMENT, "a TwELL buffer pointer is NULL");
  if (!b->bk_tile || !b->bk_tok || !b->bk_vals)
    return fail(SFFN_ERR_INVALID_ARGUMENT, "a backup buffer pointer is NULL");
  if (need_all && !b->workspace) return fail(SFFN_ERR_INVALID_ARGUMENT, "workspace is NULL");
  return SFFN_OK;
}

#define SFFN_TRY(expr)                       \
  do {                                       \
    const sffn_status_t s__ = (expr);        \
    if (s__ != SFFN_OK) return s__;          \
  } while (0)

}  // namespace

extern "C" {

const char* sffn_status_string(sffn_status_t s) {
  switch (s) {
    case SFFN_OK: return "SFFN_OK";
    case SFFN_ERR_INVALID_ARGUMENT: return "SFFN_ERR_INVALID_ARGUMENT";
    case SFFN_ERR_UNSUPPORTED: return "SFFN_ERR_UNSUPPORTED";
    case SFFN_ERR_BACKUP_OVERFLOW: return "SFFN_ERR_BACKUP_OVERFLOW";
    case SFFN_ERR_DEVICE: return "SFFN_ERR_DEVICE";
  }
  return "SFFN_UNKNOWN_STATUS";
}

const char* sffn_last_error(void) { return g_last_error.c_str(); }

sffn_status_t twell_buffer_sizes(const sffn_config_t* cfg, int32_t T, twell_buffer_sizes_t* out) {
  SFFN_TRY(check_cfg(cfg));
  SFFN_TRY(check_T(cfg, T));
  if (!out) return fail(SFFN_ERR_INVALID_ARGUMENT, "out is NULL");
  const Dims d = make_dims(cfg, T);
  // GROUP rows of padding after the last tile-row: kernels load the slot pairs of a whole
  // 32-token group at a time and may read (never use) rows past the last token
  const size_t slots = ((size_t)d.nt * T + GROUP) * d.W;
  const size_t cap = d.cap > 0 ? d.cap : 1;
  out->counts = sizeof(uint16_t) * ((size_t)d.nt * T + GROUP);  // + padding, as vals/cols
  out->vals = (size_t)d.esz * slots;
  out->cols = slots;
  out->bk_tile = sizeof(int32_t) * cap;
  out->bk_tok = sizeof(int32_t) * cap;
  out->bk_vals = (size_t)d.esz * cap * d.K;
  out->bk_tile_ptr = sizeof(int32_t) * (size_t)(d.nt + 1);
  out->bk_n = sizeof(int32_t);
  out->status = sizeof(int32_t);
  out->workspace = workspace_bytes(d);
  return SFFN_OK;
}

sffn_status_t twell_buffer_bytes(const sffn_config_t* cfg, int32_t T,
                                 size_t out_bytes[SFFN_N_BUFFERS]) {
  if (!out_bytes) return fail(SFFN_ERR_INVALID_ARGUMENT, "out_bytes is NULL");
  twell_buffer_sizes_t z;
  SFFN_TRY(twell_buffer_sizes(cfg, T, &z));
  const size_t v[SFFN_N_BUFFERS] = {z.counts, z.vals, z.cols, z.bk_tile, z.bk_tok,
                                    z.bk_vals, z.bk_tile_ptr, z.bk_n, z.status, z.workspace};
  for (int i = 0; i < SFFN_N_BUFFERS; ++i) out_bytes[i] = v[i];
  return SFFN_OK;
}

sffn_status_t sparse_ffn_create(const sffn_config_t* cfg, const void* W_up, const void* b_up,
                                const void* W_down, sparse_ffn_t* out) {
  SFFN_TRY(check_layer_cfg(cfg));
  if (!W_up || !b_up || !W_down || !out)
    return fail(SFFN_ERR_INVALID_ARGUMENT, "NULL weight or output pointer");
  sparse_ffn* h = new (std::nothrow) sparse_ffn;
  if (!h) return fail(SFFN_ERR_DEVICE, "host allocation failed");
  h->cfg = *cfg;
  h->W_up = W_up;
  h->b_up = b_up;
  h->W_down = W_down;
  *out = h;
  return SFFN_OK;
}

sffn_status_t sparse_ffn_destroy(sparse_ffn_t h) {
  delete h;  // its hint word, if any, stays with the library (never reused)
  return SFFN_OK;
}

sffn_status_t twell_pack(const sffn_config_t* cfg, const float* h, int32_t T,
                         const twell_buffers_t* buf, void* stream) {
  SFFN_TRY(check_cfg(cfg));
  SFFN_TRY(check_T(cfg, T));
  if (!h) return fail(SFFN_ERR_INVALID_ARGUMENT, "h is NULL");
  SFFN_TRY(check_bufs(buf, true));
  const Dims d = make_dims(cfg, T);
  const Workspace ws = carve(buf->workspace, d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  SFFN_TRY(run("pack", s, [&] { return launch_pack(d, h, *buf, ws, s); }));
  SFFN_TRY(run("order", s, [&] { return launch_order(d, *buf, ws, s); }));
  return SFFN_OK;
}

// The down-projection's kernel choice.  Forced policies name one kernel (an unsupported one
// falls back to the next one down).  Under the auto policy the layer's stored nonzeros n
// decide: gather for n <= thr_g, tiles for thr_g < n <= thr_m, mfma for n > thr_m; an
// unsupported kernel's range goes to the next one down, and with a single candidate no count
// is needed.
struct DownPlan {
  int32_t policy;
  long long thr_g, thr_m, all;
  bool needs_count;  // auto with several candidates: the per-block counts are read
};

static DownPlan plan_down(const sparse_ffn* hd, const Dims& d) {
  DownPlan p{hd->down_policy, 0, 0, 0, false};
  if ((p.policy == SFFN_DOWN_MFMA || p.policy == SFFN_DOWN_UNION ||
       p.policy == SFFN_DOWN_SPARSE) && !down_mfma_supported(d))
    p.policy = SFFN_DOWN_TILES;
  if (p.policy == SFFN_DOWN_TILES && !down_lds_supported(d)) p.policy = SFFN_DOWN_GATHER;
  if (p.policy != SFFN_DOWN_AUTO) return p;
  const double cells = (double)d.T * (double)d.F;
  p.thr_g = (long long)((double)hd->down_gather_density * cells);
  p.thr_m = (long long)((double)hd->down_mfma_density * cells);
  p.all = (long long)cells + 1;  // above any count
  if (!down_mfma_supported(d) || d.T < SFFN_DOWN_MFMA_MIN_T) p.thr_m = p.all;
  if (!down_lds_supported(d) || d.T < SFFN_DOWN_TILES_MIN_T) p.thr_g = p.thr_m;
  p.needs_count = p.thr_g < p.all;
  return p;
}

// Down-projection of a packed activation.  The gather kernel is the per-token row gather
// for bf16 layers (the staged-tile gather for fp32 layers and d_model > 4096); under the auto
// policy the kernel is chosen by the layer's stored nonzeros, counted and compared on the
// device: every candidate is launched with its range and all but one return at once.
// blk_ready: ws.blk_nnz already holds this TwELL's per-block counts (written by the ordering
// pass of the same call).
// Hint words come from pages of pinned host memory that the library keeps until the process
// ends; a word is never given to a second handle, so a kernel still writing one (or a graph
// recorded with it and replayed later) never writes memory that was freed or reused.
namespace {
constexpr int HINT_PAGE_WORDS = 1024;
std::mutex g_hint_mu;
int* g_hint_page = nullptr;      // host address of the current page
int* g_hint_page_dev = nullptr;  // its device address
int g_hint_used = HINT_PAGE_WORDS;
}  // namespace

static bool new_hint_word(int** host, int** dev) {
  std::lock_guard<std::mutex> lock(g_hint_mu);
  if (g_hint_used == HINT_PAGE_WORDS) {
    void* hp = nullptr;
    void* dp = nullptr;
    if (hipHostMalloc(&hp, sizeof(int) * HINT_PAGE_WORDS, hipHostMallocDefault) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    if (hipHostGetDevicePointer(&dp, hp, 0) != hipSuccess) {
      (void)hipGetLastError();
      (void)hipHostFree(hp);  // nothing has used it yet
      return false;
    }
    g_hint_page = static_cast<int*>(hp);
    g_hint_page_dev = static_cast<int*>(dp);
    g_hint_used = 0;
  }
  *host = g_hint_page + g_hint_used;
  *dev = g_hint_page_dev + g_hint_used;
  ++g_hint_used;
  return true;
}

// The hint word of a handle, set up on first use by a call that may allocate (not one that
// promised not to, and not while the stream is being captured): device address or null.
static int* hint_word(sparse_ffn* hd, hipStream_t s, bool may_alloc) {
  std::lock_guard<std::mutex> lock(hd->hint_mu);
  if (hd->hint_dev || hd->hint_failed || !may_alloc) return hd->hint_dev;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
    return nullptr;
  int* hp = nullptr;
  int* dp = nullptr;
  if (!new_hint_word(&hp, &dp)) {
    hd->hint_failed = true;
    return nullptr;
  }
  __atomic_store_n(hp, -1, __ATOMIC_RELAXED);
  hd->hint_host = hp;
  hd->hint_dev = dp;
  return hd->hint_dev;
}

static sffn_status_t down_impl(sparse_ffn* hd, const Dims& d, const twell_buffers_t& act,
                               const Workspace& ws, void* y, hipStream_t s, bool blk_ready,
                               bool may_alloc) {
  const bool rows_ok = down_rows_supported(d);
  DownHint hint;  // where the kernel that runs records its choice (auto policy only)
  auto gather = [&](const int32_t* blk, long long thr) {
    if (rows_ok)
      return run("down", s, [&] { return launch_down_rows(d, act, ws, hd->W_down, y, blk, thr, s, hint); });
    if (down_rows_f32_supported(d) && blk == nullptr)
      return run("down", s, [&] { return launch_down_rows_f32(d, act, ws, hd->W_down, y, s); });
    return run("down", s, [&] { return launch_down(d, act, hd->W_down, y, blk, thr, s); });
  };
  auto tiles = [&](const int32_t* blk, long long lo, long long hi) {
    return run("down_tiles", s,
               [&] { return launch_down_lds(d, act, ws, hd->W_down, y, blk, lo, hi, s, hint); });
  };
  auto mfma = [&](const int32_t* blk, long long thr) {
    return run("down_mfma", s,
               [&] { return launch_down_mfma(d, act, ws, hd->W_down, y, blk, thr, s, hint); });
  };
  auto unionk = [&](const int32_t* blk, long long thr) {
    return run("down_union", s,
               [&] { return launch_down_union(d, act, ws, hd->W_down, y, blk, thr, s); });
  };
  auto sparse = [&](const int32_t* blk, long long thr) {
    return run("down_sparse", s,
               [&] { return launch_down_sparse(d, act, ws, hd->W_down, y, blk, thr, s); });
  };
  const DownPlan p = plan_down(hd, d);
  if (p.policy == SFFN_DOWN_SPARSE) return sparse(nullptr, 0);
  if (p.policy == SFFN_DOWN_UNION) return unionk(nullptr, 0);
  if (p.policy == SFFN_DOWN_GATHER) return gather(nullptr, 0);
  if (p.policy == SFFN_DOWN_TILES) return tiles(nullptr, 0, 0);
  if (p.policy == SFFN_DOWN_MFMA) return mfma(nullptr, 0);
  if (!p.needs_count) return gather(nullptr, 0);
  if (!blk_ready)
    SFFN_TRY_INNER(run("block_nnz", s, [&] { return launch_block_nnz(d, act, ws.blk_nnz, s); }));
  // Every candidate gives the layer's result at any density (the choice is speed only), so
  // once a call has recorded the kernel its count selects, the next call launches that one
  // alone (and records its own count's choice for the call after it).  The first call, a
  // recorded kernel that is no candidate for this call's shape, or no hint word: every
  // candidate is launched and the count decides on the device.
  int* hw = rows_ok ? hint_word(hd, s, may_alloc) : nullptr;
  if (hw) {
    hint = DownHint{hw, ws.blk_nnz, p.thr_g, p.thr_m};
    const int h = __atomic_load_n(hd->hint_host, __ATOMIC_RELAXED);
    if (h == 0) return gather(nullptr, 0);
    if (h == 1 && p.thr_m > p.thr_g) return tiles(nullptr, 0, 0);
    if (h == 2 && p.thr_m < p.all) return mfma(nullptr, 0);
  }
  SFFN_TRY_INNER(gather(ws.blk_nnz, p.thr_g));
  if (p.thr_m > p.thr_g) SFFN_TRY_INNER(tiles(ws.blk_nnz, p.thr_g, p.thr_m));
  if (p.thr_m < p.all) SFFN_TRY_INNER(mfma(ws.blk_nnz, p.thr_m));
  return SFFN_OK;
}

static sffn_status_t forward_impl(sparse_ffn_t hd, const void* x, int32_t T, void* y,
                                  const twell_buffers_t* act, float* z, void* stream,
                                  bool may_alloc = true) {
  if (!hd) return fail(SFFN_ERR_INVALID_ARGUMENT, "handle is NULL");
  SFFN_TRY(check_T(&hd->cfg, T));
  if (!x || !y) return fail(SFFN_ERR_INVALID_ARGUMENT, "x or y is NULL");
  SFFN_TRY(check_bufs(act, true));
  const Dims d = make_dims(&hd->cfg, T);
  const Workspace ws = carve(act->workspace, d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (up_small_supported(d)) {
    // decode-shaped batch: up-projection over many small workgroups, then the pack kernel
    SFFN_TRY(run("up_small", s, [&] {
      return launch_up_small(d, static_cast<const uint16_t*>(x),
                             static_cast<const uint16_t*>(hd->W_up),
                             static_cast<const uint16_t*>(hd->b_up), ws.hsmall, z, s);
    }));
    SFFN_TRY(run("pack", s, [&] { return launch_pack(d, ws.hsmall, *act, ws, s); }));
  } else if (up_small_f32_supported(d)) {
    // the same for fp32 layers
    SFFN_TRY(run("up_small", s, [&] {
      return launch_up_small_f32(d, static_cast<const float*>(x),
                                 static_cast<const float*>(hd->W_up),
                                 static_cast<const float*>(hd->b_up), ws.hsmall, z, s);
    }));
    SFFN_TRY(run("pack", s, [&] { return launch_pack(d, ws.hsmall, *act, ws, s); }));
  } else if (d.bf16) {
    SFFN_TRY(run("up_pack", s, [&] {
      return launch_up_pack_bf16(d, static_cast<const uint16_t*>(x),
                                 static_cast<const uint16_t*>(hd->W_up),
                                 static_cast<const uint16_t*>(hd->b_up), *act, ws, z, s);
    }));
  } else {
    SFFN_TRY(run("up_pack", s, [&] {
      return launch_up_pack_f32(d, static_cast<const float*>(x),
                                static_cast<const float*>(hd->W_up),
                                static_cast<const float*>(hd->b_up), *act, ws, z, s);
    }));
  }
  // the ordering pass also writes the counts the kernel choice reads
  const bool blk = plan_down(hd, d).needs_count;
  SFFN_TRY(run("order", s, [&] { return launch_order(d, *act, ws, s, blk); }));
  return down_impl(hd, d, *act, ws, y, s, blk, may_alloc);
}

sffn_status_t sparse_ffn_forward(sparse_ffn_t hd, const void* x, int32_t T, void* y,
                                 const twell_buffers_t* act, void* stream) {
  return forward_impl(hd, x, T, y, act, nullptr, stream);
}

sffn_status_t sparse_ffn_forward_noalloc(sparse_ffn_t hd, const void* x, int32_t T, void* y,
                                         const twell_buffers_t* act, void* stream) {
  if (!hd) return fail(SFFN_ERR_INVALID_ARGUMENT, "handle is NULL");
  SFFN_TRY(check_T(&hd->cfg, T));
  if (!x || !y) return fail(SFFN_ERR_INVALID_ARGUMENT, "x or y is NULL");
  SFFN_TRY(check_bufs(act, false));
  const Dims d = make_dims(&hd->cfg, T);
  const size_t need = workspace_bytes(d, true);
  if (need > (size_t)SFFN_NOALLOC_SCRATCH_BYTES)
    return fail(SFFN_ERR_UNSUPPORTED,
                "this call needs " + std::to_string(need) +
                    " bytes of workspace, more than the no-allocation scratch holds (" +
                    std::to_string((size_t)SFFN_NOALLOC_SCRATCH_BYTES) + ")");
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* scratch = nullptr;
  const hipError_t e = noalloc_scratch(s, &scratch);
  if (e != hipSuccess) return dev_fail(e, "no-allocation scratch lookup");
  twell_buffers_t a = *act;
  a.workspace = scratch;
  return forward_impl(hd, x, T, y, &a, nullptr, stream, false);
}

sffn_status_t sparse_ffn_forward_dump(sparse_ffn_t hd, const void* x, int32_t T, void* y,
                                      const twell_buffers_t* act, float* z, void* stream) {
  if (!z) return fail(SFFN_ERR_INVALID_ARGUMENT, "z is NULL");
  return forward_impl(hd, x, T, y, act, z, stream);
}

sffn_status_t sparse_ffn_down(sparse_ffn_t hd, const twell_buffers_t* act, int32_t T, void* y,
                              void* stream) {
  if (!hd) return fail(SFFN_ERR_INVALID_ARGUMENT, "handle is NULL");
  SFFN_TRY(check_T(&hd->cfg, T));
  if (!y) return fail(SFFN_ERR_INVALID_ARGUMENT, "y is NULL");
  SFFN_TRY(check_bufs(act, true));
  const Dims d = make_dims(&hd->cfg, T);
  const Workspace ws = carve(act->workspace, d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  return down_impl(hd, d, *act, ws, y, s, false, true);
}

sffn_status_t sparse_ffn_backward(sparse_ffn_t hd, const void* x, const void* dy, int32_t T,
                                  const twell_buffers_t* act, void* dh_vals, void* dh_bk_vals,
                                  void* dx, float* dW_up, float* dW_down, float* db_up,
                                  void* stream) {
  if (!hd) return fail(SFFN_ERR_INVALID_ARGUMENT, "handle is NULL");
  SFFN_TRY(check_T(&hd->cfg, T));
  if (!x || !dy || !dx || !dW_up || !dW_down || !dh_vals || !dh_bk_vals)
    return fail(SFFN_ERR_INVALID_ARGUMENT, "NULL input, output or dh buffer");
  SFFN_TRY(check_bufs(act, true));
  const Dims d = make_dims(&hd->cfg, T);
  if (!backward_supported(d))
    return fail(SFFN_ERR_UNSUPPORTED,
                "backward needs a bf16 layer, tile 128 or 256, ell_width 16/32/48/64 and "
                "d_model % 256 == 0");
  const Workspace ws = carve(act->workspace, d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  static const char* const names[3] = {"bwd_dh", "bwd_dw_down", "bwd_dw_up"};
  for (int which = 0; which < 3; ++which)
    SFFN_TRY(run(names[which], s, [&] {
      return launch_backward_part(which, d, *act, ws, x, dy, hd->W_down, dh_vals, dh_bk_vals,
                                  dW_up, dW_down, db_up, s);
    }));
  // dx = dh W_up: the down-projection kernel over dh's TwELL (the structure of act)
  twell_buffers_t dact = *act;
  dact.vals = dh_vals;
  dact.bk_vals = dh_bk_vals;
  return run("bwd_dx", s,
             [&] { return launch_down_mfma(d, dact, ws, hd->W_up, dx, nullptr, 0, s); });
}

sffn_status_t sparse_ffn_set_down_policy(sparse_ffn_t hd, int32_t policy, float gather_density,
                                         float mfma_density) {
  if (!hd) return fail(SFFN_ERR_INVALID_ARGUMENT, "handle is NULL");
  if (policy != SFFN_DOWN_AUTO && policy != SFFN_DOWN_GATHER && policy != SFFN_DOWN_MFMA &&
      policy != SFFN_DOWN_TILES && policy != SFFN_DOWN_UNION && policy != SFFN_DOWN_SPARSE)
    return fail(SFFN_ERR_INVALID_ARGUMENT, "unknown down-projection policy");
  if (!(gather_density >= 0.0f && gather_density <= mfma_density && mfma_density <= 1.0f))
    return fail(SFFN_ERR_INVALID_ARGUMENT,
                "down-projection thresholds must satisfy 0 <= gather_density <= mfma_density <= 1");
  hd->down_policy = policy;
  hd->down_gather_density = gather_density;
  hd->down_mfma_density = mfma_density;
  {
    std::lock_guard<std::mutex> lock(hd->hint_mu);
    if (hd->hint_host) __atomic_store_n(hd->hint_host, -1, __ATOMIC_RELAXED);
  }
  return SFFN_OK;
}

sffn_status_t twell_stats(const sffn_config_t* cfg, const twell_buffers_t* buf, int32_t T,
                          twell_stats_t* out, void* stream) {
  SFFN_TRY(check_cfg(cfg));
  SFFN_TRY(check_T(cfg, T));
  SFFN_TRY(check_bufs(buf, true));
  if (!out) return fail(SFFN_ERR_INVALID_ARGUMENT, "out is NULL");
  const Dims d = make_dims(cfg, T);
  const Workspace ws = carve(buf->workspace, d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  SFFN_TRY(run("stats", s, [&] { return launch_stats(d, *buf, ws, s); }));
  long long host[8];
  hipError_t e = hipMemcpyAsync(host, ws.stats, sizeof(host), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return dev_fail(e, "stats copy");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return dev_fail(e, "stats sync");
  std::memset(out, 0, sizeof(*out));
  out->nnz = host[0];
  out->slots_used = host[1];
  out->overflow_tile_rows = host[2];
  out->backup_nonzeros = host[3];
  out->max_count = (int32_t)host[4];
  out->backup_needed = host[5];
  out->backup_overflowed = host[6] != 0 ? 1 : 0;
  const double cells = (double)T * d.F;
  out->density = cells > 0 ? (double)out->nnz / cells : 0.0;
  const double slots = (double)d.nt * T * d.W;
  out->ell_fill = slots > 0 ? (double)out->slots_used / slots : 0.0;
  out->bytes_main = (int64_t)d.nt * T * (2 + (int64_t)d.W * (d.esz + 1));
  const long long used = host[5] < d.cap ? host[5] : d.cap;
  out->bytes_backup = used * ((int64_t)d.K * d.esz + 8);
  out->bytes_dense_equiv = (int64_t)T * d.F * d.esz;
  if (out->backup_overflowed)
    return fail(SFFN_ERR_BACKUP_OVERFLOW, "backup capacity exceeded: outputs are undefined");
  return SFFN_OK;
}

sffn_status_t twell_count_histogram(const sffn_config_t* cfg, const twell_buffers_t* buf,
                                    int32_t T, int64_t* hist, void* stream) {
  SFFN_TRY(check_cfg(cfg));
  SFFN_TRY(check_T(cfg, T));
  SFFN_TRY(check_bufs(buf, true));
  if (!hist) return fail(SFFN_ERR_INVALID_ARGUMENT, "hist is NULL");
  const Dims d = make_dims(cfg, T);
  const Workspace ws = carve(buf->workspace, d);
  hipStream_t s = static_cast<hipStream_t>(stream);
  SFFN_TRY(run("hist", s, [&] { return launch_hist(d, *buf, ws, s); }));
  long long host[SFFN_HIST_BINS];
  hipError_t e = hipMemcpyAsync(host, ws.hist, sizeof(long long) * (d.K + 1),
                                hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return dev_fail(e, "histogram copy");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return dev_fail(e, "histogram sync");
  for (int c = 0; c <= d.K; ++c) hist[c] = host[c];
  return SFFN_OK;
}

sffn_status_t twell_choose_ell_width(const sffn_config_t* cfg, const int64_t* hist,
                                     const int32_t* candidates, int32_t n_candidates,
                                     int32_t* W_out, int64_t* bytes_out) {
  SFFN_TRY(check_cfg(cfg));
  if (!hist || !W_out) return fail(SFFN_ERR_INVALID_ARGUMENT, "hist or W_out is NULL");
  const int K = cfg->tile;
  const int64_t esz = cfg->dtype == SFFN_BF16 ? 2 : 4;
  if (candidates != nullptr && n_candidates < 1)
    return fail(SFFN_ERR_INVALID_ARGUMENT, "empty candidate list");
  int64_t R = 0;
  for (int c = 0; c <= K; ++c) {
    if (hist[c] < 0) return fail(SFFN_ERR_INVALID_ARGUMENT, "negative histogram bin");
    R += hist[c];
  }
  // over[W] = tile-rows with count > W
  std::vector<int64_t> over(K + 1, 0);
  for (int w = K - 1; w >= 0; --w) over[w] = over[w + 1] + hist[w + 1];
  const int n = candidates ? n_candidates : K;
  int best_w = 0;
  int64_t best = 0;
  for (int i = 0; i < n; ++i) {
    const int w = candidates ? candidates[i] : i + 1;
    if (w < 1 || w > K) return fail(SFFN_ERR_INVALID_ARGUMENT, "candidate width outside [1, tile]");
    const int64_t bytes = R * (2 + (int64_t)w * (esz + 1)) + over[w] * (esz * K + 8);
    if (best_w == 0 || bytes < best || (bytes == best && w < best_w)) {
      best = bytes;
      best_w = w;
    }
  }
  *W_out = best_w;
  if (bytes_out) *bytes_out = best;
  return SFFN_OK;
}

sffn_status_t sparse_ffn_check(const twell_buffers_t* buf, void* stream) {
  if (!buf || !buf->status) return fail(SFFN_ERR_INVALID_ARGUMENT, "status buffer is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t st = 0;
  hipError_t e = hipMemcpyAsync(&st, buf->status, sizeof(st), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return dev_fail(e, "status copy");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return dev_fail(e, "status sync");
  if (st == SFFN_ERR_BACKUP_OVERFLOW)
    return fail(SFFN_ERR_BACKUP_OVERFLOW, "backup capacity exceeded: outputs are undefined");
  if (st != 0) return fail(SFFN_ERR_DEVICE, "unexpected device status word");
  return SFFN_OK;
}

sffn_status_t sffn_profile_enable(int32_t enable) {
  g_prof.enabled = enable != 0;
  return SFFN_OK;
}

sffn_status_t sffn_profile_only(const char* names) {
  g_prof.only.clear();
  if (!names) return SFFN_OK;
  std::string cur;
  for (const char* p = names;; ++p) {
    if (*p == ',' || *p == '\0') {
      if (!cur.empty()) g_prof.only.push_back(cur);
      cur.clear();
      if (*p == '\0') break;
    } else {
      cur += *p;
    }
  }
  return SFFN_OK;
}

sffn_status_t sffn_profile_reset(void) {
  g_prof.clear();
  return SFFN_OK;
}

sffn_status_t sffn_profile_read(const char* kernel, double* total_ms, int64_t* launches) {
  if (!kernel || !total_ms || !launches) return fail(SFFN_ERR_INVALID_ARGUMENT, "NULL argument");
  double sum = 0.0;
  int64_t n = 0;
  for (auto& r : g_prof.recs) {
    if (r.name != kernel) continue;
    hipError_t e = hipEventSynchronize(r.e1);
    if (e != hipSuccess) return dev_fail(e, "profile sync");
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, r.e0, r.e1);
    if (e != hipSuccess) return dev_fail(e, "profile elapsed");
    sum += ms;
    ++n;
  }
  *total_ms = sum;
  *launches = n;
  return SFFN_OK;
}

sffn_status_t sffn_probe_gather_fma(const void* W, int32_t F, int32_t d, const int32_t* rows,
                                    const void* vals, int32_t T, int32_t n, void* y,
                                    void* stream) {
  if (!W || !y || (n > 0 && (!rows || !vals)))
    return fail(SFFN_ERR_INVALID_ARGUMENT, "probe: NULL pointer");
  if (F < 1 || d < 8 || d % 8 != 0 || T < 1 || n < 0)
    return fail(SFFN_ERR_INVALID_ARGUMENT, "probe: need F >= 1, d >= 8, d % 8 == 0, T >= 1, n >= 0");
  if ((long long)T * n >= (1ll << 31) || (long long)F * d >= (1ll << 40))
    return fail(SFFN_ERR_INVALID_ARGUMENT, "probe: sizes out of range");
  hipStream_t s = static_cast<hipStream_t>(stream);
  return run("probe_gather_fma", s,
             [&] { return sffn::launch_gather_fma_probe(W, F, d, rows, vals, T, n, y, s); });
}

}  // extern "C"
