// Up-projection + bias + ReLU for decode-shaped batches (at most 128 tokens), bf16 layers.
//
// With a handful of tokens the layer is bound by reading W_up (upppp.jp TwELL article of
// 2026-05-11, section "What TwELL and the custom CUDA kernels solve": inference throughput
// of the sparse FFN), and the 256-neuron workgroups of the fused kernel would leave most
// CUs idle.  Here a workgroup owns 32 neurons (F/32 workgroups: 256 at d_ff 8192) and all
// tokens, as NTB blocks of 32; its 4 waves split d_model into quarters and each runs
// v_mfma_f32_32x32x16_bf16 with A = its 32 W_up rows (loaded once per step, used for every
// token block) and B = the token rows, both loaded straight from memory as 16-byte pieces
// (lane l: row l % 32, columns 8 (l / 32) .. + 7 of each 16-column step).  Per token block
// the four partial 32 x 32 sums are added in LDS in a fixed order, the bias is added and
// h = max(z, 0) is written as fp32 [T, F] for the TwELL pack kernel (the same packing the
// standalone twell_pack performs); tokens past T are computed from a repeated row and not
// written.
#include "sffn_common.hpp"

namespace sffn {

typedef __bf16 bf16x8_s __attribute__((ext_vector_type(8)));
typedef float floatx16_s __attribute__((ext_vector_type(16)));

constexpr int US_NB = 32;  // neurons per workgroup

template <int NTB>
__global__ __launch_bounds__(256) void up_small_kernel(Dims d, const uint16_t* __restrict__ x,
                                                       const uint16_t* __restrict__ Wu,
                                                       const uint16_t* __restrict__ bu,
                                                       float* __restrict__ h,
                                                       float* __restrict__ zdump,
                                                       int32_t* __restrict__ claim) {
  __shared__ __attribute__((aligned(16))) float red[4][16][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int D = d.D, T = d.T, F = d.F;
  const int n0 = blockIdx.x * US_NB;
  // the backup staging counter the pack kernel (the next launch) claims from
  if (blockIdx.x == 0 && threadIdx.x == 0) *claim = 0;
  const int r = lane & 31, hh = lane >> 5;
  const int nks = D / 16;                          // 16-column steps (D % 16 == 0)
  const int ks0 = wave * nks / 4, ks1 = (wave + 1) * nks / 4;
  const uint16_t* wrow = Wu + (size_t)(n0 + r) * D + 8 * hh;
  const uint16_t* xrow[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const int t = 32 * tb + r;
    xrow[tb] = x + (size_t)(t < T ? t : T - 1) * D + 8 * hh;
  }

  floatx16_s acc[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[tb][e] = 0.0f;
  constexpr int ST = NTB == 1 ? 8 : 4;  // steps whose loads are in flight together
  int ks = ks0;
  for (; ks + ST <= ks1; ks += ST) {
    bf16x8_s a[ST], b[ST][NTB];
#pragma unroll
    for (int u = 0; u < ST; ++u) {
      a[u] = *reinterpret_cast<const bf16x8_s*>(wrow + (ks + u) * 16);
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
        b[u][tb] = *reinterpret_cast<const bf16x8_s*>(xrow[tb] + (ks + u) * 16);
    }
#pragma unroll
    for (int u = 0; u < ST; ++u)
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
        acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b[u][tb], acc[tb], 0, 0, 0);
  }
  for (; ks < ks1; ++ks) {
    const bf16x8_s a = *reinterpret_cast<const bf16x8_s*>(wrow + ks * 16);
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const bf16x8_s b = *reinterpret_cast<const bf16x8_s*>(xrow[tb] + ks * 16);
      acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[tb], 0, 0, 0);
    }
  }

  // per token block: sum the four quarters in a fixed order; element e of lane l is neuron
  // 8(e/4) + 4(l/32) + e%4 of the block and token l % 32 of the token block
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    if (tb > 0) __syncthreads();  // wave 0 has read the previous block's sums
#pragma unroll
    for (int e = 0; e < 16; ++e) red[wave][e][lane] = acc[tb][e];
    __syncthreads();
    if (wave != 0) continue;
    const int t = 32 * tb + r;
    float z[16];
#pragma unroll
    for (int e = 0; e < 16; ++e)
      z[e] = ((red[0][e][lane] + red[1][e][lane]) + red[2][e][lane]) + red[3][e][lane];
    if (t < T) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + 8 * q + 4 * hh;
        const uint2 bw = *reinterpret_cast<const uint2*>(bu + n);
        const float bias[4] = {__uint_as_float(bw.x << 16), __uint_as_float(bw.x & 0xFFFF0000u),
                               __uint_as_float(bw.y << 16), __uint_as_float(bw.y & 0xFFFF0000u)};
        float4 zz, hv;
        zz.x = z[4 * q] + bias[0];
        zz.y = z[4 * q + 1] + bias[1];
        zz.z = z[4 * q + 2] + bias[2];
        zz.w = z[4 * q + 3] + bias[3];
        hv.x = zz.x > 0.0f ? zz.x : 0.0f;
        hv.y = zz.y > 0.0f ? zz.y : 0.0f;
        hv.z = zz.z > 0.0f ? zz.z : 0.0f;
        hv.w = zz.w > 0.0f ? zz.w : 0.0f;
        *reinterpret_cast<float4*>(h + (size_t)t * F + n) = hv;
        if (zdump) *reinterpret_cast<float4*>(zdump + (size_t)t * F + n) = zz;
      }
    }
  }
}

bool up_small_supported(const Dims& d) {
  return d.bf16 && d.T <= UP_SMALL_T && d.D % 16 == 0 && d.F % US_NB == 0;
}
static_assert(UP_SMALL_T <= 128, "at most four 32-token blocks per workgroup");

hipError_t launch_up_small(const Dims& d, const uint16_t* x, const uint16_t* Wu,
                           const uint16_t* bu, float* h, float* zdump, int32_t* claim,
                           hipStream_t s) {
  if (!up_small_supported(d)) return hipErrorInvalidValue;
  const dim3 grid(d.F / US_NB), block(256);
  if (d.T <= 32)
    hipLaunchKernelGGL(up_small_kernel<1>, grid, block, 0, s, d, x, Wu, bu, h, zdump, claim);
  else if (d.T <= 64)
    hipLaunchKernelGGL(up_small_kernel<2>, grid, block, 0, s, d, x, Wu, bu, h, zdump, claim);
  else
    hipLaunchKernelGGL(up_small_kernel<4>, grid, block, 0, s, d, x, Wu, bu, h, zdump, claim);
  return hipGetLastError();
}

}  // namespace sffn
