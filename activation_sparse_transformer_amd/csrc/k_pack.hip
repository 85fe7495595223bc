// TwELL packing kernels for gfx950: the standalone pack of a dense fp32 hidden tensor,
// the fp32 fused up-projection + ReLU + pack (small fp32 layers), the canonical ordering
// of backup entries, and the statistics reduction.
//
// Format (upppp.jp TwELL article of 2026-05-11, section "What TwELL and the custom CUDA
// kernels solve"): the hidden columns are split into tiles of K columns; inside a tile
// every token row keeps its nonzeros ELL-style (values plus local column indices, W slots);
// the nonzeros that do not fit the W slots go to a small dense backup (the "sparse main
// plus a few dense backups" hybrid of the same section), one K-wide slice per
// overflowing tile-row.
//
// Work decomposition: one wave64 owns one (tile, 32-token group).  Each lane holds K/64
// columns of every token of the group in registers; a token's tile-row is compacted with
// ballot + mbcnt: the rank of a nonzero is the number of nonzeros at lower columns, so
// slots come out in ascending column order with no shared-memory traffic.
#include <algorithm>

#include "sffn_common.hpp"

namespace sffn {


// Store one value of the TwELL value array in the layer dtype.
template <bool BF16>
__device__ __forceinline__ void store_val(void* base, size_t idx, float v) {
  if constexpr (BF16) {
    static_cast<uint16_t*>(base)[idx] = f32_to_bf16(v);
  } else {
    static_cast<float*>(base)[idx] = v;
  }
}

// Values source of the pack: MODE_H reads a dense fp32 hidden tensor (pack_kernel); MODE_UP
// computes h = ReLU(x W_up^T + b) in fp32 on the fly (up_pack_f32_kernel, the fused forward
// of fp32 layers).
enum { MODE_H = 0, MODE_UP = 1 };

// The pack of one (tile k, token group g) by one wave, from the group's values v: lane l
// holds column c*64 + l of token t0 + i in v[i][c] (0 for tokens past T).  Writes the main
// slots, their padding, the counts, the group's column union and overflow count, and stages
// the remainder of overflowing tile-rows under one claim.
template <int K, bool BF16>
__device__ __forceinline__ void pack_pair(const Dims& d, int k, int g, const float (&v)[GROUP][K / 64],
                                          const twell_buffers_t& b, const Workspace& ws) {
  constexpr int C = K / 64;
  const int lane = threadIdx.x & 63;
  const int t0 = g * GROUP;
  const int T = d.T, W = d.W;
  // Phase 1: true count of every tile-row of the group; lane i keeps token i's count.
  int cnt_lane = 0;
#pragma unroll
  for (int i = 0; i < GROUP; ++i) {
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) cnt += __popcll(ballot64(v[i][c] != 0.0f));
    if (lane == i) cnt_lane = cnt;
  }
  // Column union of the group: lane = column c*64 + lane, any token nonzero there.
#pragma unroll
  for (int c = 0; c < C; ++c) {
    bool any = false;
#pragma unroll
    for (int i = 0; i < GROUP; ++i) any |= v[i][c] != 0.0f;
    const uint64_t um = ballot64(any);
    if (lane == 0) {
      uint32_t* dst = ws.umask + ((int64_t)k * d.ng + g) * (K / 32) + 2 * c;
      dst[0] = (uint32_t)um;
      dst[1] = (uint32_t)(um >> 32);
    }
  }
  // One staging claim for all of the group's overflowing tile-rows.
  const uint64_t om = ballot64(lane < GROUP && cnt_lane > W);
  const int n_ov = __popcll(om);
  int base = 0;
  if (n_ov > 0) {
    if (lane == 0) base = atomicAdd(ws.claim, n_ov);
    base = __shfl(base, 0);
  }
  if (lane == 0) ws.ov_grp[(int64_t)k * d.ng + g] = n_ov;

  // Phase 2: write slots, padding, counts and the staged remainder.
  int lr = 0;  // rank of the next overflowing tile-row inside the group
#pragma unroll
  for (int i = 0; i < GROUP; ++i) {
    const int t = t0 + i;
    if (t >= T) break;
    const int cnt = __builtin_amdgcn_readlane(cnt_lane, i);
    const bool over = cnt > W;
    const bool stage = over && d.cap > 0;
    const int slot = stage ? stage_slot((uint32_t)base + (uint32_t)lr, d.cap) : 0;
    const size_t row = ((size_t)k * T + t) * (size_t)W;
    int prefix = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const bool nz = v[i][c] != 0.0f;
      const uint64_t m = ballot64(nz);
      const int r = prefix + mbcnt64(m);
      prefix += __popcll(m);
      const int col = c * 64 + lane;
      if (nz && r < W) {
        store_val<BF16>(b.vals, row + r, v[i][c]);
        b.cols[row + r] = (uint8_t)col;
      }
      if (stage) store_val<BF16>(ws.stage_vals, (size_t)slot * K + col, (nz && r >= W) ? v[i][c] : 0.0f);
    }
    const int used = cnt < W ? cnt : W;
    for (int s = used + lane; s < W; s += 64) {
      store_val<BF16>(b.vals, row + s, 0.0f);
      b.cols[row + s] = 0;
    }
    if (lane == 0) {
      b.counts[(size_t)k * T + t] = (uint16_t)cnt;
      if (stage) {
        ws.stage_key[2 * slot] = k;
        ws.stage_key[2 * slot + 1] = t | (lr << 24);
      }
    }
    if (over) ++lr;
  }
}


// One wave per (tile k, token group g).  4 waves per workgroup.  The values come from a
// dense fp32 hidden tensor h [T, F].
template <int K, bool BF16>
__global__ __launch_bounds__(256) void pack_kernel(Dims d, const float* __restrict__ h,
                                                   twell_buffers_t b, Workspace ws) {
  constexpr int C = K / 64;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= d.nt * d.ng) return;  // uniform per wave
  const int k = wave / d.ng;
  const int g = wave - k * d.ng;
  const int t0 = g * GROUP;
  float v[GROUP][C];
#pragma unroll
  for (int i = 0; i < GROUP; ++i) {
    const int t = t0 + i;
#pragma unroll
    for (int c = 0; c < C; ++c)
      v[i][c] = t < d.T ? h[(int64_t)t * d.F + (int64_t)k * K + c * 64 + lane] : 0.0f;
  }
  pack_pair<K, BF16>(d, k, g, v, b, ws);
}

// Fused up-projection + ReLU + pack of fp32 layers (small test-sized layers): one workgroup
// of 4 waves per (tile k, token group g).  Wave w sums the d_model quarter
// [w D/4, (w+1) D/4) of z[t, n] = x[t, :] . W_up[n, :] for the group's 32 tokens and the
// tile's K neurons: slices of DCH columns of the tile's W_up rows and of the group's x rows
// are copied into the wave's own LDS region with 16-byte loads (rows padded to DCH + 4
// floats, so the lanes' 16-byte reads of 16 consecutive rows fall in distinct banks), and
// every lane keeps its K/64 neurons x 32 tokens of sums in registers (x values are LDS
// broadcasts).  The four partial sums meet in LDS and are added in wave order; wave 0 adds
// the bias, applies ReLU and packs.
template <int K, bool BF16>
__global__ __launch_bounds__(256) void up_pack_f32_kernel(Dims d, const float* __restrict__ x,
                                                          const float* __restrict__ Wu,
                                                          const float* __restrict__ bu,
                                                          twell_buffers_t b, Workspace ws,
                                                          float* __restrict__ zdump) {
  constexpr int C = K / 64;
  constexpr int DCH = K >= 256 ? 16 : 32;        // d_model columns per staged slice
  constexpr int SWS = DCH + 4;                   // padded row stride (floats)
  constexpr int WREG = (K + GROUP) * SWS;        // one wave's staging (floats)
  constexpr int PART = 3 * GROUP * K;            // waves 1-3's partial sums (floats)
  constexpr int SBUF = 4 * WREG > PART ? 4 * WREG : PART;
  __shared__ __attribute__((aligned(16))) float sbuf[SBUF];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int k = blockIdx.x / d.ng;
  const int g = blockIdx.x - k * d.ng;
  const int t0 = g * GROUP;
  const int T = d.T, D = d.D;
  float* sW = sbuf + wave * WREG;
  float* sX = sW + K * SWS;
  const int dq = D / 4;  // D % 64 == 0
  const int dlo = wave * dq, dhi = dlo + dq;

  float acc[GROUP][C];
#pragma unroll
  for (int i = 0; i < GROUP; ++i)
#pragma unroll
    for (int c = 0; c < C; ++c) acc[i][c] = 0.0f;
  for (int dc = dlo; dc < dhi; dc += DCH) {
    // this wave's slice: K rows of W_up and 32 rows of x, columns dc .. dc+DCH-1 (16-byte
    // pieces; columns past the quarter and rows past T are zero)
    for (int p = lane; p < K * DCH / 4; p += 64) {
      const int r = p / (DCH / 4), q = p - r * (DCH / 4);
      const int c0 = dc + 4 * q;
      const float4 w = c0 < dhi ? *reinterpret_cast<const float4*>(Wu + ((int64_t)k * K + r) * D + c0)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(sW + r * SWS + 4 * q) = w;
    }
    for (int p = lane; p < GROUP * DCH / 4; p += 64) {
      const int i = p / (DCH / 4), q = p - i * (DCH / 4);
      const int c0 = dc + 4 * q, t = t0 + i;
      const float4 xv = (c0 < dhi && t < T) ? *reinterpret_cast<const float4*>(x + (int64_t)t * D + c0)
                                            : make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(sX + i * SWS + 4 * q) = xv;
    }
    // (one wave writes and reads its own region: program order suffices)
#pragma unroll
    for (int dd = 0; dd < DCH; dd += 4) {
      float4 w[C];
#pragma unroll
      for (int c = 0; c < C; ++c) w[c] = *reinterpret_cast<const float4*>(sW + (c * 64 + lane) * SWS + dd);
#pragma unroll
      for (int i = 0; i < GROUP; ++i) {
        const float4 xv = *reinterpret_cast<const float4*>(sX + i * SWS + dd);
#pragma unroll
        for (int c = 0; c < C; ++c) {
          float a = acc[i][c];
          a = fmaf(xv.x, w[c].x, a);
          a = fmaf(xv.y, w[c].y, a);
          a = fmaf(xv.z, w[c].z, a);
          a = fmaf(xv.w, w[c].w, a);
          acc[i][c] = a;
        }
      }
    }
  }
  // partial sums of waves 1-3 into LDS (over the staging), then wave 0 adds them in order
  __syncthreads();
  if (wave > 0) {
    float* pw = sbuf + (wave - 1) * GROUP * K;
#pragma unroll
    for (int i = 0; i < GROUP; ++i)
#pragma unroll
      for (int c = 0; c < C; ++c) pw[i * K + c * 64 + lane] = acc[i][c];
  }
  __syncthreads();
  if (wave > 0) return;
  float v[GROUP][C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int64_t n = (int64_t)k * K + c * 64 + lane;
    const float bias = bu[n];
#pragma unroll
    for (int i = 0; i < GROUP; ++i) {
      float z = acc[i][c];
#pragma unroll
      for (int w2 = 0; w2 < 3; ++w2) z += sbuf[w2 * GROUP * K + i * K + c * 64 + lane];
      z += bias;
      const int t = t0 + i;
      if (zdump && t < T) zdump[(int64_t)t * d.F + n] = z;
      v[i][c] = (t < T && z > 0.0f) ? z : 0.0f;
    }
  }
  pack_pair<K, BF16>(d, k, g, v, b, ws);
}

template <int K, bool BF16, int MODE>
static hipError_t launch_pack_t(const Dims& d, const float* h, const float* x, const float* Wu,
                                const float* bu, const twell_buffers_t& b, const Workspace& ws,
                                float* zdump, hipStream_t s) {
  if constexpr (MODE == MODE_UP) {
    hipLaunchKernelGGL((up_pack_f32_kernel<K, BF16>), dim3(d.nt * d.ng), dim3(256), 0, s, d, x,
                       Wu, bu, b, ws, zdump);
  } else {
    const int waves = d.nt * d.ng;
    const int blocks = (waves + 3) / 4;
    hipLaunchKernelGGL((pack_kernel<K, BF16>), dim3(blocks), dim3(256), 0, s, d, h, b, ws);
  }
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_pack_dispatch(const Dims& d, const float* h, const float* x,
                                       const float* Wu, const float* bu,
                                       const twell_buffers_t& b, const Workspace& ws,
                                       float* zdump, hipStream_t s) {
  if (d.bf16) {
    switch (d.K) {
      case 64: return launch_pack_t<64, true, MODE>(d, h, x, Wu, bu, b, ws, zdump, s);
      case 128: return launch_pack_t<128, true, MODE>(d, h, x, Wu, bu, b, ws, zdump, s);
      case 256: return launch_pack_t<256, true, MODE>(d, h, x, Wu, bu, b, ws, zdump, s);
    }
  } else {
    switch (d.K) {
      case 64: return launch_pack_t<64, false, MODE>(d, h, x, Wu, bu, b, ws, zdump, s);
      case 128: return launch_pack_t<128, false, MODE>(d, h, x, Wu, bu, b, ws, zdump, s);
      case 256: return launch_pack_t<256, false, MODE>(d, h, x, Wu, bu, b, ws, zdump, s);
    }
  }
  return hipErrorInvalidValue;
}

// Few (tile, group) pairs (decode-shaped batches): pack_kernel would leave most CUs idle and
// walk 32 tokens one after another.  Here a workgroup of 8 waves owns one (tile, group),
// each wave 4 of its tokens; the 32 counts meet in LDS, so every wave knows which rows of
// the group overflow and its rows' ranks among them, and one staging claim serves the
// group.  The output is the one pack_kernel writes.
constexpr int PS_WAVES = 8;
constexpr int PS_TPW = GROUP / PS_WAVES;  // tokens per wave
constexpr int PS_MAX_PAIRS = 2048;         // (tile, group) pairs below which it is used

template <int K, bool BF16>
__global__ __launch_bounds__(512) void pack_small_kernel(Dims d, const float* __restrict__ h,
                                                         twell_buffers_t b, Workspace ws) {
  constexpr int C = K / 64;
  __shared__ int cnt_s[GROUP];
  __shared__ int base_s;
  __shared__ uint32_t um_s[K / 32];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int k = blockIdx.x / d.ng;
  const int g = blockIdx.x - k * d.ng;
  if (threadIdx.x < K / 32) um_s[threadIdx.x] = 0u;
  const int i0 = wv * PS_TPW;  // first row of the group this wave owns
  const int t0 = g * GROUP + i0;
  const int T = d.T, W = d.W;

  float v[PS_TPW][C];
#pragma unroll
  for (int i = 0; i < PS_TPW; ++i) {
    const int t = t0 + i;
#pragma unroll
    for (int c = 0; c < C; ++c)
      v[i][c] = t < T ? h[(int64_t)t * d.F + (int64_t)k * K + c * 64 + lane] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < PS_TPW; ++i) {
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) cnt += __popcll(ballot64(v[i][c] != 0.0f));
    if (lane == 0) cnt_s[i0 + i] = cnt;  // rows past T hold zeros: count 0
  }
  __syncthreads();
  // column union of the group: each wave ORs in its 4 tokens
#pragma unroll
  for (int c = 0; c < C; ++c) {
    bool any = false;
#pragma unroll
    for (int i = 0; i < PS_TPW; ++i) any |= v[i][c] != 0.0f;
    const uint64_t um = ballot64(any);
    if (lane == 0) {
      if ((uint32_t)um) atomicOr(&um_s[2 * c], (uint32_t)um);
      if ((uint32_t)(um >> 32)) atomicOr(&um_s[2 * c + 1], (uint32_t)(um >> 32));
    }
  }
  const int cnt_lane = lane < GROUP ? cnt_s[lane] : 0;
  const uint64_t om = ballot64(lane < GROUP && cnt_lane > W);
  const int n_ov = __popcll(om);
  if (threadIdx.x == 0) {
    base_s = n_ov > 0 ? atomicAdd(ws.claim, n_ov) : 0;
    ws.ov_grp[(int64_t)k * d.ng + g] = n_ov;
  }
  __syncthreads();
  if (threadIdx.x < K / 32) ws.umask[((int64_t)k * d.ng + g) * (K / 32) + threadIdx.x] = um_s[threadIdx.x];
  const int base = base_s;

#pragma unroll
  for (int i = 0; i < PS_TPW; ++i) {
    const int t = t0 + i;
    if (t >= T) break;
    const int cnt = __builtin_amdgcn_readlane(cnt_lane, i0 + i);
    const bool over = cnt > W;
    const int lr = __popcll(om & ((1ull << (i0 + i)) - 1));  // rank among the group's overflows
    const bool stage = over && d.cap > 0;
    const int slot = stage ? stage_slot((uint32_t)base + (uint32_t)lr, d.cap) : 0;
    const size_t row = ((size_t)k * T + t) * (size_t)W;
    int prefix = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const bool nz = v[i][c] != 0.0f;
      const uint64_t m = ballot64(nz);
      const int r = prefix + mbcnt64(m);
      prefix += __popcll(m);
      const int col = c * 64 + lane;
      if (nz && r < W) {
        store_val<BF16>(b.vals, row + r, v[i][c]);
        b.cols[row + r] = (uint8_t)col;
      }
      if (stage) store_val<BF16>(ws.stage_vals, (size_t)slot * K + col, (nz && r >= W) ? v[i][c] : 0.0f);
    }
    const int used = cnt < W ? cnt : W;
    for (int s = used + lane; s < W; s += 64) {
      store_val<BF16>(b.vals, row + s, 0.0f);
      b.cols[row + s] = 0;
    }
    if (lane == 0) {
      b.counts[(size_t)k * T + t] = (uint16_t)cnt;
      if (stage) {
        ws.stage_key[2 * slot] = k;
        ws.stage_key[2 * slot + 1] = t | (lr << 24);
      }
    }
  }
}

template <int K, bool BF16>
static hipError_t launch_pack_small_t(const Dims& d, const float* h, const twell_buffers_t& b,
                                      const Workspace& ws, hipStream_t s) {
  hipLaunchKernelGGL((pack_small_kernel<K, BF16>), dim3(d.nt * d.ng), dim3(64 * PS_WAVES), 0, s,
                     d, h, b, ws);
  return hipGetLastError();
}

hipError_t launch_pack(const Dims& d, const float* h, const twell_buffers_t& b,
                       const Workspace& ws, hipStream_t s) {
  if (d.nt * d.ng < PS_MAX_PAIRS) {
    if (d.bf16) {
      switch (d.K) {
        case 64: return launch_pack_small_t<64, true>(d, h, b, ws, s);
        case 128: return launch_pack_small_t<128, true>(d, h, b, ws, s);
        case 256: return launch_pack_small_t<256, true>(d, h, b, ws, s);
      }
    } else {
      switch (d.K) {
        case 64: return launch_pack_small_t<64, false>(d, h, b, ws, s);
        case 128: return launch_pack_small_t<128, false>(d, h, b, ws, s);
        case 256: return launch_pack_small_t<256, false>(d, h, b, ws, s);
      }
    }
    return hipErrorInvalidValue;
  }
  return launch_pack_dispatch<MODE_H>(d, h, nullptr, nullptr, nullptr, b, ws, nullptr, s);
}

hipError_t launch_up_pack_f32(const Dims& d, const float* x, const float* Wu, const float* bu,
                              const twell_buffers_t& b, const Workspace& ws, float* zdump,
                              hipStream_t s) {
  return launch_pack_dispatch<MODE_UP>(d, nullptr, x, Wu, bu, b, ws, zdump, s);
}

// ---------------------------------------------------------------------------------------
// Canonical backup order.  Producers stage overflowing tile-rows in claim order and
// record, per (tile, group), how many overflowed and each entry's rank in its group.  The
// final position of an entry of (k, t) is the exclusive prefix over (k, group) of those
// counts, plus its rank: ascending (tile, token), the same for every run.


__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

// Two launches.  order_tile_kernel (one workgroup per tile): exclusive scan of the tile's
// per-group overflow counts, in place in ov_grp, and the tile's total.  order_copy_kernel:
// every workgroup scans the tile totals into tile offsets in LDS; together they write
// grp_first (tile offset + group offset: the first canonical entry of every (tile, group)),
// the first one bk_tile_ptr, bk_n and the status word, and every staged entry goes to
// grp_first[tile, group] + its rank inside the group.  With with_blk, workgroup i also
// writes the stored nonzeros of 256-token blocks i, i + gridDim.x, ... (blk_nnz, read by the
// down-projection's kernel choice), which saves the forward pass that launch.
constexpr int ORDER_COPY_MAX_NT = SFFN_MAX_TILES;  // tile offsets the copy kernel's LDS holds

__global__ __launch_bounds__(1024) void order_tile_kernel(Dims d, Workspace ws) {
  __shared__ int wsum[16];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  int32_t* grp = ws.ov_grp + (size_t)blockIdx.x * d.ng;
  int carry = 0;
  for (int base = 0; base < d.ng; base += 1024) {
    const int i = base + tid;
    const int v = i < d.ng ? grp[i] : 0;
    const int incl = wave_incl_scan(v);
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int sw = wsum[w];
      woff += w < wv ? sw : 0;
      tot += sw;
    }
    if (i < d.ng) grp[i] = carry + woff + incl - v;
    carry += tot;
    __syncthreads();  // wsum is rewritten by the next round
  }
  if (tid == 0) ws.tile_tot[blockIdx.x] = carry;
}

template <int K, bool BF16>
__global__ __launch_bounds__(256) void order_copy_kernel(Dims d, twell_buffers_t b, Workspace ws,
                                                         int with_blk) {
  __shared__ int toff[ORDER_COPY_MAX_NT + 1];
  __shared__ int wsum[4];
  __shared__ int bsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // tile offsets: exclusive scan of the tile totals, 256 at a time
  int carry = 0;
  for (int base = 0; base < d.nt; base += 256) {
    const int k = base + tid;
    const int v = k < d.nt ? ws.tile_tot[k] : 0;
    const int incl = wave_incl_scan(v);
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int sw = wsum[w];
      woff += w < wv ? sw : 0;
      tot += sw;
    }
    if (k < d.nt) toff[k] = carry + woff + incl - v;
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) toff[d.nt] = carry;
  __syncthreads();
  const int total = carry;
  const int N = d.nt * d.ng;
  if (blockIdx.x == 0) {
    for (int k = tid; k <= d.nt; k += 256) b.bk_tile_ptr[k] = toff[k];
    if (tid == 0) {
      ws.grp_first[N] = total;
      *b.bk_n = total;
      *b.status = total > d.cap ? (int)SFFN_ERR_BACKUP_OVERFLOW : 0;
    }
  }
  for (int q = blockIdx.x * 256 + tid; q < N; q += gridDim.x * 256)
    ws.grp_first[q] = toff[q / d.ng] + ws.ov_grp[q];
  if (with_blk) {
    // thread i sums every tile's count of token i of the block (coalesced rows of counts)
    for (int tb = blockIdx.x; tb * 256 < d.T; tb += gridDim.x) {
      const int t = tb * 256 + tid;
      int sum = 0;
      if (t < d.T) {
#pragma unroll 16
        for (int k = 0; k < d.nt; ++k) sum += b.counts[(size_t)k * d.T + t];
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
      __syncthreads();  // bsum's previous readers are done
      if (lane == 0) bsum[wv] = sum;
      __syncthreads();
      if (tid == 0) ws.blk_nnz[tb] = bsum[0] + bsum[1] + bsum[2] + bsum[3];
    }
  }
  // the copy: the producers claimed positions first .. first + total - 1 (slots modulo cap)
  const int n_staged = min(total, d.cap);
  const uint32_t first_pos = (uint32_t)*ws.claim - (uint32_t)total;
  const int gw = blockIdx.x * 4 + wv;
  const int nw = gridDim.x * 4;
  constexpr int WORDS = K * (BF16 ? 2 : 4) / 4;  // 32-bit words per slice
  for (int i = gw; i < n_staged; i += nw) {
    const int e = stage_slot(first_pos + (uint32_t)i, d.cap);
    const int kk = ws.stage_key[2 * e];
    const int tw = ws.stage_key[2 * e + 1];
    const int t = tw & 0xFFFFFF, lr = tw >> 24;
    const int fin = toff[kk] + ws.ov_grp[kk * d.ng + t / GROUP] + lr;
    if (fin >= d.cap) continue;  // capacity exceeded: the status word reports it
    const uint32_t* src = static_cast<const uint32_t*>(ws.stage_vals) + (size_t)e * WORDS;
    uint32_t* dst = static_cast<uint32_t*>(b.bk_vals) + (size_t)fin * WORDS;
    for (int q = lane; q < WORDS; q += 64) dst[q] = src[q];
    if (lane == 0) {
      b.bk_tile[fin] = kk;
      b.bk_tok[fin] = t;
    }
  }
}

// Few (tile, group) pairs (decode-shaped batches): one launch instead of two.  Every
// workgroup scans the counts (one per thread, at most 1024) into LDS, the first one also
// writes the scan's outputs, and the workgroups then share the moves of the staged entries.
// With with_blk the last workgroup also writes the stored nonzeros of every 256-token block
// (blk_nnz, read by the down-projection's kernel choice), which saves the forward pass that
// launch.
constexpr int ORDER_SMALL_N = 1024;
constexpr int ORDER_SMALL_MAX_WG = 128;

template <int K, bool BF16>
__global__ __launch_bounds__(1024) void order_small_kernel(Dims d, twell_buffers_t b, Workspace ws,
                                                           int with_blk) {
  __shared__ int wsum[16];
  __shared__ int first_s[ORDER_SMALL_N];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int N = d.nt * d.ng;
  const int v = tid < N ? ws.ov_grp[tid] : 0;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int woff = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int sw = wsum[w];
    woff += w < wv ? sw : 0;
    tot += sw;
  }
  const int first = woff + incl - v;
  if (tid < N) first_s[tid] = first;
  if (blockIdx.x == 0) {
    if (tid < N) {
      ws.grp_first[tid] = first;
      if (tid % d.ng == 0) b.bk_tile_ptr[tid / d.ng] = first;
    }
    if (tid == 0) {
      ws.grp_first[N] = tot;
      b.bk_tile_ptr[d.nt] = tot;
      *b.bk_n = tot;
      *b.status = tot > d.cap ? (int)SFFN_ERR_BACKUP_OVERFLOW : 0;
    }
  }
  if (with_blk && blockIdx.x == gridDim.x - 1) {
    // thread i sums tiles i/256, i/256 + 4, ... of token i%256 of each block
    for (int tb = 0; tb * 256 < d.T; ++tb) {
      const int t = tb * 256 + (tid & 255);
      int sum = 0;
      if (t < d.T) {
#pragma unroll 16
        for (int k = tid >> 8; k < d.nt; k += 4) sum += b.counts[(size_t)k * d.T + t];
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
      __syncthreads();  // wsum's previous readers are done
      if (lane == 0) wsum[wv] = sum;
      __syncthreads();
      if (tid == 0) {
        int v = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) v += wsum[w];
        ws.blk_nnz[tb] = v;
      }
    }
  }
  __syncthreads();
  // the copy: entry e of the staging goes to first(tile, group) + its rank in the group.
  // A slice is LPE 16-byte pieces (slices start 16-byte aligned), so a wave moves EPW
  // entries at once and the grid 16 EPW per workgroup.
  // the producers claimed positions first .. first + tot - 1 (slots modulo cap)
  const int n_staged = min(tot, d.cap);
  const uint32_t first_pos = (uint32_t)*ws.claim - (uint32_t)tot;
  constexpr int LPE = K * (BF16 ? 2 : 4) / 16;  // lanes per entry: 8 .. 64
  constexpr int EPW = 64 / LPE;
  const int sub = lane / LPE, q = lane - sub * LPE;
  for (int e0 = (blockIdx.x * 16 + wv) * EPW; e0 < n_staged; e0 += gridDim.x * 16 * EPW) {
    const int i = e0 + sub;
    if (i < n_staged) {
      const int e = stage_slot(first_pos + (uint32_t)i, d.cap);
      const int kk = ws.stage_key[2 * e];
      const int tw = ws.stage_key[2 * e + 1];
      const int t = tw & 0xFFFFFF, lr = tw >> 24;
      const int fin = first_s[kk * d.ng + t / GROUP] + lr;
      if (fin < d.cap) {  // capacity exceeded: the status word reports it
        const uint4* src = static_cast<const uint4*>(ws.stage_vals) + (size_t)e * LPE;
        uint4* dst = static_cast<uint4*>(b.bk_vals) + (size_t)fin * LPE;
        dst[q] = src[q];
        if (q == 0) {
          b.bk_tile[fin] = kk;
          b.bk_tok[fin] = t;
        }
      }
    }
  }
}

hipError_t launch_order(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                        hipStream_t s, bool with_blk) {
  if (d.nt * d.ng <= ORDER_SMALL_N) {
    // workgroups for the copy: 64 staged entries each, of at most min(cap, n_t T)
    const long long most = std::min<long long>((long long)d.cap, (long long)d.nt * d.T);
    const int nwg = (int)std::min<long long>(ORDER_SMALL_MAX_WG, std::max<long long>(1, (most + 63) / 64));
#define SFFN_ORDER_SMALL(KK, BB) \
  hipLaunchKernelGGL((order_small_kernel<KK, BB>), dim3(nwg), dim3(1024), 0, s, d, b, ws, \
                     with_blk ? 1 : 0)
    if (d.bf16) {
      if (d.K == 64) SFFN_ORDER_SMALL(64, true);
      else if (d.K == 128) SFFN_ORDER_SMALL(128, true);
      else SFFN_ORDER_SMALL(256, true);
    } else {
      if (d.K == 64) SFFN_ORDER_SMALL(64, false);
      else if (d.K == 128) SFFN_ORDER_SMALL(128, false);
      else SFFN_ORDER_SMALL(256, false);
    }
#undef SFFN_ORDER_SMALL
    return hipGetLastError();
  }
  if (d.nt > ORDER_COPY_MAX_NT) return hipErrorInvalidValue;
  hipLaunchKernelGGL(order_tile_kernel, dim3(d.nt), dim3(1024), 0, s, d, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 4 waves per workgroup, about one staged entry per wave at full capacity
  int blocks = (d.cap + 3) / 4;
  blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
#define SFFN_ORDER(KK, BB) \
  hipLaunchKernelGGL((order_copy_kernel<KK, BB>), dim3(blocks), dim3(256), 0, s, d, b, ws, \
                     with_blk ? 1 : 0)
  if (d.bf16) {
    if (d.K == 64) SFFN_ORDER(64, true);
    else if (d.K == 128) SFFN_ORDER(128, true);
    else SFFN_ORDER(256, true);
  } else {
    if (d.K == 64) SFFN_ORDER(64, false);
    else if (d.K == 128) SFFN_ORDER(128, false);
    else SFFN_ORDER(256, false);
  }
#undef SFFN_ORDER
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Statistics: a grid of workgroups reduces the counts array into ws.stats (cleared by the
// launcher first); integer sums and a maximum, so the order of the atomic updates does not
// change the result.
constexpr int STATS_WG = 256;

__global__ __launch_bounds__(256) void stats_kernel(Dims d, twell_buffers_t b, Workspace ws) {
  __shared__ unsigned long long red[5][4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const size_t n = (size_t)d.nt * d.T;
  const int W = d.W;
  unsigned long long nnz = 0, slots = 0, over = 0, bnz = 0, mx = 0;
  // eight counts (16 bytes) per load where the run is aligned; the tail one by one
  const size_t n8 = n / 8;
  const uint4* c8 = reinterpret_cast<const uint4*>(b.counts);
  for (size_t q = (size_t)blockIdx.x * 256 + tid; q < n8; q += (size_t)gridDim.x * 256) {
    const uint4 v = c8[q];
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const unsigned long long c = (w4[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      nnz += c;
      slots += c < (unsigned)W ? c : (unsigned)W;
      over += c > (unsigned)W ? 1 : 0;
      bnz += c > (unsigned)W ? c - W : 0;
      mx = c > mx ? c : mx;
    }
  }
  for (size_t q = n8 * 8 + (size_t)blockIdx.x * 256 + tid; q < n; q += (size_t)gridDim.x * 256) {
    const unsigned long long c = b.counts[q];
    nnz += c;
    slots += c < (unsigned)W ? c : (unsigned)W;
    over += c > (unsigned)W ? 1 : 0;
    bnz += c > (unsigned)W ? c - W : 0;
    mx = c > mx ? c : mx;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    nnz += __shfl_xor(nnz, o);
    slots += __shfl_xor(slots, o);
    over += __shfl_xor(over, o);
    bnz += __shfl_xor(bnz, o);
    const unsigned long long m2 = __shfl_xor(mx, o);
    mx = m2 > mx ? m2 : mx;
  }
  if (lane == 0) {
    red[0][wv] = nnz; red[1][wv] = slots; red[2][wv] = over; red[3][wv] = bnz; red[4][wv] = mx;
  }
  __syncthreads();
  if (tid == 0) {
    unsigned long long a[5] = {0, 0, 0, 0, 0};
    for (int w = 0; w < 4; ++w) {
      for (int j = 0; j < 4; ++j) a[j] += red[j][w];
      a[4] = red[4][w] > a[4] ? red[4][w] : a[4];
    }
    unsigned long long* st = reinterpret_cast<unsigned long long*>(ws.stats);
    for (int j = 0; j < 4; ++j)
      if (a[j]) atomicAdd(st + j, a[j]);
    if (a[4]) atomicMax(st + 4, a[4]);
    if (blockIdx.x == 0) {
      ws.stats[5] = *b.bk_n;
      ws.stats[6] = *b.status;
    }
  }
}

hipError_t launch_stats(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                        hipStream_t s) {
  hipError_t e = hipMemsetAsync(ws.stats, 0, 8 * sizeof(long long), s);
  if (e != hipSuccess) return e;
  const size_t n8 = ((size_t)d.nt * d.T) / 8;
  const int grid = (int)std::max<size_t>(1, std::min<size_t>(STATS_WG, (n8 + 255) / 256));
  hipLaunchKernelGGL(stats_kernel, dim3(grid), dim3(256), 0, s, d, b, ws);
  return hipGetLastError();
}

// Count histogram: each workgroup bins its share of the counts in LDS (32-bit), then adds
// its bins into the cleared 64-bit global bins.
__global__ __launch_bounds__(256) void hist_kernel(Dims d, const uint16_t* __restrict__ counts,
                                                   unsigned long long* __restrict__ hist) {
  __shared__ uint32_t bins[SFFN_HIST_BINS];
  for (int i = threadIdx.x; i < d.K + 1; i += 256) bins[i] = 0;
  __syncthreads();
  const size_t n = (size_t)d.nt * d.T;
  for (size_t q = (size_t)blockIdx.x * 256 + threadIdx.x; q < n; q += (size_t)gridDim.x * 256) {
    const int c = counts[q];
    atomicAdd(&bins[c <= d.K ? c : d.K], 1u);  // (a count never exceeds the tile width)
  }
  __syncthreads();
  for (int i = threadIdx.x; i < d.K + 1; i += 256)
    if (bins[i] != 0) atomicAdd(&hist[i], (unsigned long long)bins[i]);
}

hipError_t launch_hist(const Dims& d, const twell_buffers_t& b, const Workspace& ws, hipStream_t s) {
  hipError_t e = hipMemsetAsync(ws.hist, 0, sizeof(long long) * SFFN_HIST_BINS, s);
  if (e != hipSuccess) return e;
  const size_t n = (size_t)d.nt * d.T;
  const int grid = (int)std::max<size_t>(1, std::min<size_t>(STATS_WG, (n + 255) / 256));
  hipLaunchKernelGGL(hist_kernel, dim3(grid), dim3(256), 0, s, d, b.counts,
                     reinterpret_cast<unsigned long long*>(ws.hist));
  return hipGetLastError();
}

}  // namespace sffn
