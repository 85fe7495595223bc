// Measurement probe: the gather-multiply-add of a vector down-projection without TwELL.
//
//   y[t, :] = sum_j vals[t, j] W[rows[t, j], :]    (fp32 sums, bf16 result)
//
// Only the rows of W_down that a token's nonzero activations select contribute to its output
// (upppp.jp TwELL article of 2026-05-11, section "What is the waste in LLM FFN layers"); the
// vector down kernels multiply exactly those rows, plus the work of decoding TwELL.  This
// kernel does the multiply-adds alone, with the row lists given, so its rate on the device
// bounds what a vector down kernel can reach on the same rows.
//
// One wave per (token, 512-column chunk): lane l owns columns 8l .. 8l+7 of the chunk (one
// 16-byte load per row, 1 KB per wave and row), the token's row indices and values are
// wave-uniform scalar loads, and U rows are loaded before any is used.
#include "sffn_common.hpp"

namespace sffn {

constexpr int PR_WAVES = 4;
constexpr int PR_CHUNK = 512;  // columns per wave

template <int U>
__global__ __launch_bounds__(64 * PR_WAVES) void gather_fma_probe_kernel(
    const uint16_t* __restrict__ W, int F, int D, const int32_t* __restrict__ rows,
    const uint16_t* __restrict__ vals, int T, int n, uint16_t* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int nch = (D + PR_CHUNK - 1) / PR_CHUNK;
  const int gw = blockIdx.x * PR_WAVES + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int t = gw / nch;
  if (t >= T) return;
  const int c0 = (gw - t * nch) * PR_CHUNK + 8 * lane;
  const bool ok = c0 < D;  // D % 8 == 0: a lane's 8 columns are all in or all out
  const int32_t* r = rows + (size_t)t * n;
  const uint16_t* v = vals + (size_t)t * n;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  for (int j = 0; j < n; j += U) {
    uint4 w[U];
    float vv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = j + u < n;
      int idx = ld_uniform(r + (in ? j + u : j));
      idx = idx < 0 ? 0 : (idx >= F ? F - 1 : idx);  // rows outside W read its first/last row
      vv[u] = in ? bf16_to_f32(ld_uniform(v + j + u)) : 0.0f;
      w[u] = ok ? *reinterpret_cast<const uint4*>(W + (size_t)idx * D + c0) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t ww[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(vv[u], __uint_as_float(ww[q] << 16), acc[2 * q]);
        acc[2 * q + 1] = fmaf(vv[u], __uint_as_float(ww[q] & 0xFFFF0000u), acc[2 * q + 1]);
      }
    }
  }
  if (ok) {
    uint4 o;
    o.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
    o.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
    o.z = (uint32_t)f32_to_bf16(acc[4]) | ((uint32_t)f32_to_bf16(acc[5]) << 16);
    o.w = (uint32_t)f32_to_bf16(acc[6]) | ((uint32_t)f32_to_bf16(acc[7]) << 16);
    *reinterpret_cast<uint4*>(y + (size_t)t * D + c0) = o;
  }
}

hipError_t launch_gather_fma_probe(const void* W, int F, int D, const int32_t* rows,
                                   const void* vals, int T, int n, void* y, hipStream_t s) {
  const long long waves = (long long)T * ((D + PR_CHUNK - 1) / PR_CHUNK);
  const dim3 grid((unsigned)((waves + PR_WAVES - 1) / PR_WAVES));
  hipLaunchKernelGGL((gather_fma_probe_kernel<8>), grid, dim3(64 * PR_WAVES), 0, s,
                     static_cast<const uint16_t*>(W), F, D, rows,
                     static_cast<const uint16_t*>(vals), T, n, static_cast<uint16_t*>(y));
  return hipGetLastError();
}

}  // namespace sffn
