// Internal definitions shared by the HIP kernels and the host launch code of the TwELL
// sparse FFN library (gfx950).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sparse_ffn.h"

namespace sffn {

// Token group of the per-(tile, group) overflow counters.  Every kernel that writes a
// TwELL also writes, for each tile k and each group of GROUP consecutive tokens, how many
// of the group's tile-rows overflow (count > W), and tags each staged backup entry with
// its rank inside the group.  An exclusive scan over (k, group) then gives every entry
// its canonical position in ascending (tile, token) order, independent of the order in
// which entries were staged.
constexpr int GROUP = 32;

struct Dims {
  int32_t D, F, K, W, T;
  int32_t nt;   // F / K tiles
  int32_t ng;   // ceil(T / GROUP) token groups
  int32_t cap;  // backup capacity (entries)
  int32_t esz;  // bytes per TwELL value (2 bf16, 4 fp32)
  bool bf16;
};

// Workspace carving.  Regions are 256-byte aligned.
struct Workspace {
  int32_t* claim;       // [1]      staging claim counter (any start value, see stage_slot)
  int32_t* ov_grp;      // [nt*ng]  overflowing tile-rows per (tile, group)
  int32_t* stage_key;   // [2*cap]  (tile, token | rank_in_group << 24)
  void* stage_vals;     // [cap*K]  dtype
  long long* stats;     // [8]      stats reduction output
  long long* hist;      // [SFFN_HIST_BINS] count histogram (twell_count_histogram)
  int32_t* blk_nnz;     // [nblk]   stored nonzeros per 256-token block (down-path choice)
  int32_t* grp_first;   // [nt*ng+1] first backup entry of each (tile, group), canonical order
  int32_t* tile_tot;    // [nt]     overflowing tile-rows per tile (ordering pass)
  uint32_t* umask;      // [nt*ng*K/32] per (tile, group): columns with a nonzero in any token
  float* hsmall;        // [min(T, UP_SMALL_T), F] ReLU output of the decode-shaped up path
  float* dpart;         // [S, T, D] fp32 partial sums of the split matrix-core down kernel
};

// Batches of at most this many tokens take the decode-shaped up-projection (one workgroup
// per 32 neurons, then the TwELL pack kernel) instead of the fused up + pack kernel.
constexpr int UP_SMALL_T = 128;

inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Column unions of the packed activation: for every tile k and token group g, K bits
// (K/32 words, bit b of word w = local column 32 w + b) telling which columns of the tile
// hold a nonzero in at least one token of the group (main slots and backup alike).  Every
// kernel that writes a TwELL writes them; the matrix-core down-projection contracts each
// token block only over the union of its groups' columns.
inline size_t umask_bytes(const Dims& d) {
  return sizeof(uint32_t) * (size_t)d.nt * d.ng * (d.K / 32);
}

// Split of the matrix-core down-projection over its tiles: when its workgroups of (256
// tokens, 256 columns) would fill at most half of the 256 CUs, the tile range is cut into S
// parts (at most DM_MAX_SPLIT, each at least two tiles), each part's fp32 sums go to dpart
// and a second kernel adds them in order.  S parts of `base` workgroups stay within the 256
// CUs (one workgroup per CU fits in LDS): one more part would start a second round of
// workgroups, each with fewer tiles, and take longer than S parts of more tiles.
constexpr int DM_MAX_SPLIT = 16;
inline int down_split_for(int T, int D, int nt) {
  const long long base = (long long)((T + 255) / 256) * ((D + 255) / 256);
  if (base > 128) return 1;
  int S = (int)(256 / base);
  S = S < DM_MAX_SPLIT ? S : DM_MAX_SPLIT;
  S = S < nt / 2 ? S : nt / 2;
  return S > 1 ? S : 1;
}
inline int down_split(const Dims& d) { return d.bf16 ? down_split_for(d.T, d.D, d.nt) : 1; }
// dpart floats for a call of T tokens and for every smaller T' (buffers sized for T serve
// calls with fewer tokens): the largest S(T') T' D over T' <= T
inline size_t down_part_floats(const Dims& d) {
  if (!d.bf16) return 0;
  size_t best = 0;
  for (long long t1 = 256; t1 - 255 <= d.T; t1 += 256) {  // S is constant on each 256-token block
    const long long t = t1 < d.T ? t1 : d.T;
    const int S = down_split_for((int)t, d.D, d.nt);
    if (S > 1 && (size_t)S * (size_t)t * (size_t)d.D > best) best = (size_t)S * (size_t)t * (size_t)d.D;
  }
  return best;
}

// this_call_only: size the split partial sums for a call of exactly d.T tokens (the
// workspace is used by that call alone) instead of for every T' <= d.T.
inline size_t workspace_bytes(const Dims& d, bool this_call_only = false) {
  size_t n = 0;
  n += align256(sizeof(int32_t));
  n += align256(sizeof(int32_t) * (size_t)d.nt * d.ng);
  n += align256(sizeof(int32_t) * 2 * (size_t)(d.cap > 0 ? d.cap : 1));
  n += align256((size_t)d.esz * (size_t)(d.cap > 0 ? d.cap : 1) * d.K);
  n += align256(sizeof(long long) * 8);
  n += align256(sizeof(long long) * SFFN_HIST_BINS);
  n += align256(sizeof(int32_t) * (size_t)((d.T + 255) / 256));
  n += align256(sizeof(int32_t) * ((size_t)d.nt * d.ng + 1));
  n += align256(sizeof(int32_t) * (size_t)d.nt);
  n += align256(umask_bytes(d));
  n += align256(sizeof(float) * (size_t)(d.T < UP_SMALL_T ? d.T : UP_SMALL_T) * d.F);
  const int S = down_split(d);
  n += align256(sizeof(float) * (this_call_only ? (S > 1 ? (size_t)S * d.T * d.D : 0)
                                                : down_part_floats(d)));
  return n;
}

// Callers that cannot allocate device memory: the forward variant that takes its
// workspace from a fixed array inside the library (one per device).  Returns the device
// address of the calling stream's device's array (looked up once per device).
hipError_t noalloc_scratch(hipStream_t s, void** out);

inline Workspace carve(void* base, const Dims& d) {
  char* p = static_cast<char*>(base);
  Workspace w;
  w.claim = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t));
  w.ov_grp = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * (size_t)d.nt * d.ng);
  w.stage_key = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * 2 * (size_t)(d.cap > 0 ? d.cap : 1));
  w.stage_vals = p;
  p += align256((size_t)d.esz * (size_t)(d.cap > 0 ? d.cap : 1) * d.K);
  w.stats = reinterpret_cast<long long*>(p);
  p += align256(sizeof(long long) * 8);
  w.hist = reinterpret_cast<long long*>(p);
  p += align256(sizeof(long long) * SFFN_HIST_BINS);
  w.blk_nnz = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * (size_t)((d.T + 255) / 256));
  w.grp_first = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * ((size_t)d.nt * d.ng + 1));
  w.tile_tot = reinterpret_cast<int32_t*>(p);
  p += align256(sizeof(int32_t) * (size_t)d.nt);
  w.umask = reinterpret_cast<uint32_t*>(p);
  p += align256(umask_bytes(d));
  w.hsmall = reinterpret_cast<float*>(p);
  p += align256(sizeof(float) * (size_t)(d.T < UP_SMALL_T ? d.T : UP_SMALL_T) * d.F);
  w.dpart = reinterpret_cast<float*>(p);
  return w;
}

// ---------------------------------------------------------------- device helpers
#if defined(__HIPCC__)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// Round to nearest, ties to even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }
// Number of set bits of `m` in lanes below this one.
__device__ __forceinline__ int mbcnt64(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}
template <typename T>
__device__ __forceinline__ T uniform(T v) {
  return __builtin_amdgcn_readfirstlane(v);
}
// Load through the constant address space: for a wave-uniform address of memory that no
// kernel of the launch writes, this becomes a scalar (SMEM) load into SGPRs.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T* p) {
  typedef const __attribute__((address_space(4))) T* cptr;
  return *(cptr)(uintptr_t)p;
}
// Staging slot of claimed position p.  Producers claim consecutive positions from
// ws.claim with atomicAdd; the counter is never cleared (it starts wherever the previous
// call left it), so slots run modulo the staging capacity, and the ordering pass recovers
// the first position as the final counter minus the total it scans.  cap > 0.
__device__ __forceinline__ int stage_slot(uint32_t p, int cap) { return (int)(p % (uint32_t)cap); }
// Sum of the n per-block counts (the layer's stored nonzeros), the same in every lane.
__device__ __forceinline__ long long layer_nnz(const int32_t* blk_nnz, int n) {
  long long s = 0;
  for (int q = (int)(threadIdx.x & 63); q < n; q += 64) s += blk_nnz[q];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  return s;
}
#endif

// Where a down kernel records the kernel the layer's count selects for the next call of the
// auto policy: dst (a word of pinned host memory, or null) gets 0 (gather, count <= thr_g),
// 1 (tiles, count <= thr_m) or 2 (matrix cores) from the per-block counts blk.
struct DownHint {
  int* dst = nullptr;
  const int32_t* blk = nullptr;
  long long thr_g = 0, thr_m = 0;
};
#if defined(__HIPCC__)
// Called by every thread of a kernel that runs; wave 0 of the workgroup for which `first`
// holds (wave-uniform) reads the counts and one lane stores the choice (system scope: the
// host reads it).
__device__ __forceinline__ void note_choice(const DownHint& h, int n_blocks, bool first) {
  if (h.dst == nullptr || !first || threadIdx.x >= 64) return;
  const long long n = layer_nnz(h.blk, n_blocks);
  if (threadIdx.x == 0)
    __hip_atomic_store(h.dst, n <= h.thr_g ? 0 : (n <= h.thr_m ? 1 : 2), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_SYSTEM);
}
#endif

// ---------------------------------------------------------------- launchers
// Each returns the launch's hipError_t (hipGetLastError after the launch).
hipError_t launch_pack(const Dims& d, const float* h, const twell_buffers_t& b,
                       const Workspace& ws, hipStream_t s);
// with_blk: also write ws.blk_nnz (the per-256-token-block stored nonzeros).
hipError_t launch_order(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                        hipStream_t s, bool with_blk = false);
hipError_t launch_stats(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                        hipStream_t s);
hipError_t launch_up_pack_f32(const Dims& d, const float* x, const float* Wu, const float* bu,
                              const twell_buffers_t& b, const Workspace& ws, float* zdump,
                              hipStream_t s);
// Decode-shaped up-projection: h = max(x W_up^T + b, 0) as fp32 [T, F] (T <= UP_SMALL_T),
// and z = x W_up^T + b into zdump if it is not null.
bool up_small_supported(const Dims& d);
hipError_t launch_up_small(const Dims& d, const uint16_t* x, const uint16_t* Wu,
                           const uint16_t* bu, float* h, float* zdump,
                           hipStream_t s);
// The same for fp32 layers (fp32 x, W_up, b).
bool up_small_f32_supported(const Dims& d);
hipError_t launch_up_small_f32(const Dims& d, const float* x, const float* Wu, const float* bu,
                               float* h, float* zdump, hipStream_t s);
hipError_t launch_up_pack_bf16(const Dims& d, const uint16_t* x, const uint16_t* Wu,
                               const uint16_t* bu, const twell_buffers_t& b,
                               const Workspace& ws, float* zdump, hipStream_t s);
// Down-projection.  Three kernels: the per-token gather, the LDS-tile vector kernel and the
// matrix-core kernel.  With blk_nnz (per-256-token-block stored-nonzero counts from
// launch_block_nnz) each is launched with its range of the layer's total and reads the
// total at entry: the one whose range holds it runs, the others return at once.
// blk_nnz == nullptr runs the kernel launched.  The kernel that runs records, through `hint`,
// the kernel the count selects (the next auto call launches only that one).
hipError_t launch_block_nnz(const Dims& d, const twell_buffers_t& b, int32_t* blk_nnz,
                            hipStream_t s);
hipError_t launch_down(const Dims& d, const twell_buffers_t& b, const void* Wd, void* y,
                       const int32_t* blk_nnz, long long thr, hipStream_t s);
bool down_mfma_supported(const Dims& d);
// One wave per token over the W_down rows its nonzeros select (bf16, d_model <= 4096).
bool down_rows_supported(const Dims& d);
hipError_t launch_down_rows(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                            const void* Wd, void* y, const int32_t* blk_nnz, long long thr,
                            hipStream_t s, const DownHint& hint = DownHint());
// One workgroup per (token, 256 output columns) over the W_down rows its nonzeros select
// (fp32 layers, T <= UP_SMALL_T).
bool down_rows_f32_supported(const Dims& d);
hipError_t launch_down_rows_f32(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                                const void* Wd, void* y, hipStream_t s);
// 256 tokens per workgroup over W_down tiles staged in LDS, bf16 dot products (bf16, even
// W <= 128).  With blk_nnz it runs only when the layer's stored nonzeros are in (lo, hi].
bool down_lds_supported(const Dims& d);
hipError_t launch_down_lds(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                           const void* Wd, void* y, const int32_t* blk_nnz, long long lo,
                           long long hi, hipStream_t s, const DownHint& hint = DownHint());
bool backward_supported(const Dims& d);
// One part of the backward weights pass: which = 0: dh at the stored positions of `act`
// (into dh_vals / dh_bk); 1: dW_down = H^T g; 2: dW_up = dH^T x and, if db is not null,
// db = column sums of dH.
hipError_t launch_backward_part(int which, const Dims& d, const twell_buffers_t& act,
                                const Workspace& ws, const void* x, const void* g,
                                const void* Wd, void* dh_vals, void* dh_bk, float* dW_up,
                                float* dW_down, float* db, hipStream_t s);
hipError_t launch_down_mfma(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                            const void* Wd, void* y, const int32_t* blk_nnz, long long thr,
                            hipStream_t s, const DownHint& hint = DownHint());
// The matrix-core down-projection over the column unions of 64-token blocks (the same
// shapes as launch_down_mfma; reads ws.umask, written by the kernel that produced the TwELL).
hipError_t launch_down_union(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                             const void* Wd, void* y, const int32_t* blk_nnz, long long thr,
                             hipStream_t s);
// The down-projection on the 2:4 structured-sparse matrix cores (the same shapes as
// launch_down_mfma): each stored nonzero at its rank within its four-column group.
hipError_t launch_down_sparse(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                              const void* Wd, void* y, const int32_t* blk_nnz, long long thr,
                              hipStream_t s);
// y[t] = sum_j vals[t, j] W[rows[t, j]] (bf16 W, vals, y; fp32 sums): the measurement probe.
hipError_t launch_gather_fma_probe(const void* W, int F, int D, const int32_t* rows,
                                   const void* vals, int T, int n, void* y, hipStream_t s);
// hist[c] = number of tile-rows with count c (c = 0 .. K), into ws.hist (cleared first).
hipError_t launch_hist(const Dims& d, const twell_buffers_t& b, const Workspace& ws, hipStream_t s);
// y = bf16 of the sum of the S fp32 parts in ws.dpart (split matrix-core kernels).
hipError_t launch_down_reduce(const Dims& d, const Workspace& ws, void* y, int S,
                              const int32_t* blk_nnz, long long thr, hipStream_t s);

}  // namespace sffn
