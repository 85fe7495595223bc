// Decode-shaped forward of fp32 layers (at most UP_SMALL_T tokens).
//
// With few tokens the fused fp32 kernel (one workgroup per (tile, 32-token group)) and the
// staged-tile down kernel (one workgroup per 256 tokens x 64 columns) run on a handful of
// CUs: 16 and 4 workgroups for 64 tokens at d_model 256, d_ff 1024.  Here the work is
// spread over many small workgroups instead, as the bf16 small-batch path does:
//
//  * up_small_f32_kernel: h = max(x W_up^T + b, 0) as fp32 [T, F] in the workspace (the
//    nonzero predicate is the fp32 pre-activation z > 0, as in the fused kernels), which the
//    pack kernel then turns into TwELL (upppp.jp TwELL article of 2026-05-11, section "What
//    TwELL and the custom CUDA kernels solve": the hidden activations are packed per tile).
//    A workgroup owns 8 neurons and every token; d_model is walked in slices of 64 columns
//    staged in LDS (rows padded so that the 8 rows one wave reads at a column hit distinct
//    banks); thread (neuron n = tid % 8, token slot tid / 8) keeps the sums of tokens
//    tid / 8 + 32 i, added over d_model in ascending order, then the bias.
//  * down_rows_f32_kernel: y[t, :] = sum over the stored (tile k, column c, value v) of
//    token t of v W_down[kK + c, :] plus the backup slices of its overflowing tile-rows (same
//    article and section: the down-projection over the stored nonzeros only).  A workgroup
//    owns one token and 256 output columns (4 per lane); its 4 waves take every fourth
//    tile; a wave's slots sit one per lane and are broadcast with readlane into batches of
//    16 (row, value) pairs whose W_down row loads are all issued before the FMAs.  The
//    waves' partial rows are added in LDS in wave order.
#include "sffn_common.hpp"

namespace sffn {

constexpr int UF_NN = 8;            // neurons per workgroup
constexpr int UF_DC = 64;           // d_model columns per staged slice
constexpr int UF_RS = UF_DC + 4;    // padded LDS row stride (floats)
constexpr int UF_TS = 256 / UF_NN;  // token slots (threads per neuron)
constexpr int UF_TPT = UP_SMALL_T / UF_TS;  // tokens per thread
static_assert(UF_TPT * UF_TS == UP_SMALL_T, "token slots cover UP_SMALL_T tokens");

__global__ __launch_bounds__(256) void up_small_f32_kernel(Dims d, const float* __restrict__ x,
                                                           const float* __restrict__ Wu,
                                                           const float* __restrict__ bu,
                                                           float* __restrict__ h,
                                                           float* __restrict__ zdump) {
  __shared__ __attribute__((aligned(16))) float sX[UP_SMALL_T * UF_RS];
  __shared__ __attribute__((aligned(16))) float sW[UF_NN * UF_RS];
  const int tid = threadIdx.x;
  const int T = d.T, D = d.D;
  const int n0 = blockIdx.x * UF_NN;
  const int nl = tid % UF_NN, ts = tid / UF_NN;
  float acc[UF_TPT];
#pragma unroll
  for (int i = 0; i < UF_TPT; ++i) acc[i] = 0.0f;
  constexpr int PPR = UF_DC / 4;  // 16-byte pieces per staged row
  for (int dc = 0; dc < D; dc += UF_DC) {  // D % 64 == 0
    __syncthreads();  // the previous slice has been read
    for (int p = tid; p < T * PPR; p += 256) {
      const int r = p / PPR, q = p - r * PPR;
      *reinterpret_cast<float4*>(sX + r * UF_RS + 4 * q) =
          *reinterpret_cast<const float4*>(x + (size_t)r * D + dc + 4 * q);
    }
    for (int p = tid; p < UF_NN * PPR; p += 256) {
      const int r = p / PPR, q = p - r * PPR;
      *reinterpret_cast<float4*>(sW + r * UF_RS + 4 * q) =
          *reinterpret_cast<const float4*>(Wu + (size_t)(n0 + r) * D + dc + 4 * q);
    }
    __syncthreads();
#pragma unroll 4
    for (int c = 0; c < UF_DC; c += 4) {
      const float4 w = *reinterpret_cast<const float4*>(sW + nl * UF_RS + c);
#pragma unroll
      for (int i = 0; i < UF_TPT; ++i) {
        const int t = ts + UF_TS * i;
        if (UF_TS * i < T) {  // workgroup-uniform: token slot block i holds a token
          const float4 xv = *reinterpret_cast<const float4*>(sX + (t < T ? t : 0) * UF_RS + c);
          float a = acc[i];
          a = fmaf(xv.x, w.x, a);
          a = fmaf(xv.y, w.y, a);
          a = fmaf(xv.z, w.z, a);
          a = fmaf(xv.w, w.w, a);
          acc[i] = a;
        }
      }
    }
  }
  const int n = n0 + nl;
  const float bias = bu[n];
#pragma unroll
  for (int i = 0; i < UF_TPT; ++i) {
    const int t = ts + UF_TS * i;
    if (t < T) {
      const float z = acc[i] + bias;
      if (zdump) zdump[(size_t)t * d.F + n] = z;
      h[(size_t)t * d.F + n] = z > 0.0f ? z : 0.0f;
    }
  }
}

bool up_small_f32_supported(const Dims& d) {
  return !d.bf16 && d.T <= UP_SMALL_T && d.D % UF_DC == 0 && d.F % UF_NN == 0;
}

hipError_t launch_up_small_f32(const Dims& d, const float* x, const float* Wu, const float* bu,
                               float* h, float* zdump, hipStream_t s) {
  if (!up_small_f32_supported(d)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(up_small_f32_kernel, dim3(d.F / UF_NN), dim3(256), 0, s, d, x, Wu, bu, h,
                     zdump);
  return hipGetLastError();
}

constexpr int DRF_NW = 4;     // waves per workgroup
constexpr int DRF_CW = 256;   // output columns per workgroup (4 per lane)
constexpr int DRF_BATCH = 16; // (row, value) pairs whose row loads are in flight together

__global__ __launch_bounds__(64 * DRF_NW) void down_rows_f32_kernel(
    Dims d, const uint16_t* __restrict__ counts, const float* __restrict__ vals,
    const uint8_t* __restrict__ cols, const float* __restrict__ bk_vals,
    const int32_t* __restrict__ grp_first, const float* __restrict__ Wd, float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) float part[DRF_NW - 1][DRF_CW];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int T = d.T, D = d.D, K = d.K, W = d.W;
  const int t = blockIdx.x;
  const int c0 = blockIdx.y * DRF_CW + 4 * lane;  // this lane's first output column
  const bool col_ok = c0 < D;                      // D % 64 == 0: whole float4 or none
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);

  // pending (row, value) pairs, pair i in lane i
  int bj = 0;
  float bv = 0.0f;
  int nb = 0;
  auto flush = [&]() __attribute__((always_inline)) {
    float4 w[DRF_BATCH];
    float v[DRF_BATCH];
#pragma unroll
    for (int i = 0; i < DRF_BATCH; ++i) {
      w[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      v[i] = 0.0f;
      if (i < nb) {  // wave-uniform
        const int r = __builtin_amdgcn_readlane(bj, i);
        v[i] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), i));
        if (col_ok) w[i] = *reinterpret_cast<const float4*>(Wd + (size_t)r * D + c0);
      }
    }
#pragma unroll
    for (int i = 0; i < DRF_BATCH; ++i) {
      acc.x = fmaf(v[i], w[i].x, acc.x);
      acc.y = fmaf(v[i], w[i].y, acc.y);
      acc.z = fmaf(v[i], w[i].z, acc.z);
      acc.w = fmaf(v[i], w[i].w, acc.w);
    }
    nb = 0;
  };
  // queue the pairs (jl, vl) of the lanes in `act`, in lane order
  auto add_lanes = [&](uint64_t act, int jl, float vl) __attribute__((always_inline)) {
    while (act != 0) {
      const int b = __builtin_ctzll(act);
      act &= act - 1;
      const int j = __builtin_amdgcn_readlane(jl, b);
      const float v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, vl), b));
      bj = lane == nb ? j : bj;
      bv = lane == nb ? v : bv;
      if (++nb == DRF_BATCH) flush();
    }
  };

  for (int k = wave; k < d.nt; k += DRF_NW) {
    const uint32_t cnt = ld_uniform(counts + (size_t)k * T + t);
    const int m = (int)(cnt < (uint32_t)W ? cnt : (uint32_t)W);
    const size_t row = ((size_t)k * T + t) * W;
    for (int s0 = 0; s0 < m; s0 += 64) {
      const int s = s0 + lane;
      const bool in = s < m;
      const float v = in ? vals[row + s] : 0.0f;
      const int c = in ? (int)cols[row + s] : 0;
      add_lanes(ballot64(in), k * K + c, v);
    }
    if (cnt > (uint32_t)W) {
      // backup slice of (k, t): the first entry of its 32-token group plus the number of the
      // group's earlier tokens that overflow in tile k
      const int g = t / GROUP;
      const int tl = g * GROUP + (lane & 31);
      const uint32_t cg = (lane < 32 && tl < T) ? counts[(size_t)k * T + tl] : 0u;
      const uint64_t ov = ballot64(cg > (uint32_t)W);
      const int rank = __builtin_popcountll(ov & ((1ull << (t - g * GROUP)) - 1ull));
      const int e = ld_uniform(grp_first + k * d.ng + g) + rank;
      if (e < d.cap) {  // capacity exceeded: the status word reports it
        const float* sl = bk_vals + (size_t)e * K;
        for (int q = 0; q < K; q += 64) {
          const float sv = sl[q + lane];
          add_lanes(ballot64(sv != 0.0f), k * K + q + lane, sv);
        }
      }
    }
  }
  if (nb > 0) flush();

  if (wave > 0) *reinterpret_cast<float4*>(&part[wave - 1][4 * lane]) = acc;
  __syncthreads();
  if (wave == 0 && col_ok) {
#pragma unroll
    for (int w2 = 0; w2 < DRF_NW - 1; ++w2) {
      const float4 p = *reinterpret_cast<const float4*>(&part[w2][4 * lane]);
      acc.x += p.x;
      acc.y += p.y;
      acc.z += p.z;
      acc.w += p.w;
    }
    *reinterpret_cast<float4*>(y + (size_t)t * D + c0) = acc;
  }
}

bool down_rows_f32_supported(const Dims& d) { return !d.bf16 && d.T <= UP_SMALL_T && d.D % 64 == 0; }

hipError_t launch_down_rows_f32(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                                const void* Wd, void* y, hipStream_t s) {
  if (!down_rows_f32_supported(d)) return hipErrorInvalidValue;
  const dim3 grid(d.T, (d.D + DRF_CW - 1) / DRF_CW), block(64 * DRF_NW);
  hipLaunchKernelGGL(down_rows_f32_kernel, grid, block, 0, s, d, b.counts,
                     static_cast<const float*>(b.vals), b.cols,
                     static_cast<const float*>(b.bk_vals), ws.grp_first,
                     static_cast<const float*>(Wd), static_cast<float*>(y));
  return hipGetLastError();
}

}  // namespace sffn
