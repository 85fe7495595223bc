// Up-projection + bias + ReLU for decode-shaped batches (at most 128 tokens), bf16 layers.
//
// With a handful of tokens the layer is bound by reading W_up (upppp.jp TwELL article of
// 2026-05-11, section "What TwELL and the custom CUDA kernels solve": inference throughput
// of the sparse FFN), and the 256-neuron workgroups of the fused kernel would leave most
// CUs idle.  Here a workgroup owns 32 neurons (F/32 workgroups: 256 at d_ff 8192) and all
// tokens, as NTB blocks of 32, and runs v_mfma_f32_32x32x16_bf16 with A = its 32 W_up rows
// and B = the token rows, both loaded straight from memory as 16-byte pieces (lane l: row
// l % 32, columns 8 (l / 32) .. + 7 of each 16-column step).  Its waves split d_model; the
// partial 32 x 32 sums of every token block are added in LDS in a fixed order, the bias is
// added and h = max(z, 0) is written as fp32 [T, F] for the TwELL pack kernel (the same
// packing the standalone twell_pack performs); tokens past T are computed from a repeated
// row and not written.
//
// Two forms, by measurement on MI355X at d_model 2048:
//  * up to 64 tokens (one or two token blocks): 4 waves, each over a quarter of d_model in
//    batches of 8 (4) steps whose loads are in flight together;
//  * 65 to 128 tokens (four token blocks, four times the token-row loads per W_up piece):
//    8 waves, each over an eighth of d_model, with all W_up pieces of a chunk of steps in
//    flight at once (16 KB per wave) and the token rows loaded one line of four steps ahead.
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

constexpr int US8_NW = 8;  // waves of the 8-wave form

// Steps c .. c + n - 1 (1 <= n <= CH) of one wave of the 8-wave form: all CH W_up pieces
// are loaded first.  A token row's 128-byte line holds four steps, so its pieces are loaded
// four steps at a time (the four loads of a line together), one group ahead of the MFMAs
// (all at once for one token block).
template <int NTB, int CH>
__device__ __forceinline__ void up_small_chunk(floatx16_s (&acc)[NTB], const uint16_t* wrow,
                                               const uint16_t* const (&xrow)[NTB], int c,
                                               int n) {
  static_assert(CH % 4 == 0, "whole groups of four steps");
  constexpr int NG = CH / 4;
  constexpr int GA = NTB == 1 ? NG : 1;  // groups loaded ahead of the one in the MFMAs
  bf16x8_s a[CH], b[CH][NTB];
  auto ldb = [&](int g) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int sl = 4 * g + j;
        b[sl][tb] =
            *reinterpret_cast<const bf16x8_s*>(xrow[tb] + (c + (sl < n ? sl : n - 1)) * 16);
      }
  };
#pragma unroll
  for (int s = 0; s < CH; ++s)
    a[s] = *reinterpret_cast<const bf16x8_s*>(wrow + (c + (s < n ? s : n - 1)) * 16);
#pragma unroll
  for (int g = 0; g < (GA < NG ? GA : NG); ++g) ldb(g);
  // keep the scheduler from sinking these loads back next to their MFMAs
  __builtin_amdgcn_sched_barrier(0);
  const bf16x8_s zero = {};
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (g + GA < NG) {
      ldb(g + GA);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s = 4 * g + j;
      const bf16x8_s av = s < n ? a[s] : zero;
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
        acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b[s][tb], acc[tb], 0, 0, 0);
    }
  }
}

template <int NTB>
__global__ __launch_bounds__(US8_NW * 64) void up_small8_kernel(
    Dims d, const uint16_t* __restrict__ x, const uint16_t* __restrict__ Wu,
    const uint16_t* __restrict__ bu, float* __restrict__ h, float* __restrict__ zdump,
    int32_t* __restrict__ claim) {
  constexpr int US_NW = US8_NW;
  // partial sums: [wave][token block][element][lane]
  __shared__ __attribute__((aligned(16))) float red[US_NW * NTB * 16 * 64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int D = d.D, T = d.T, F = d.F;
  const int n0 = blockIdx.x * US_NB;
  // the backup staging counter the pack kernel (the next launch) claims from
  if (blockIdx.x == 0 && threadIdx.x == 0) *claim = 0;
  const int r = lane & 31, hh = lane >> 5;
  const int nks = D / 16;                          // 16-column steps (D % 16 == 0)
  const int ks0 = wave * nks / US_NW, ks1 = (wave + 1) * nks / US_NW;
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
  // chunks of CH steps (W_up pieces in flight per wave: 16 KB at CH 16), the last one
  // partly filled
  constexpr int CH = NTB == 4 ? 8 : 16;
  int c = ks0;
  for (; c + CH <= ks1; c += CH) up_small_chunk<NTB, CH>(acc, wrow, xrow, c, CH);
  const int rest = ks1 - c;
  if (rest > 8)
    up_small_chunk<NTB, 16>(acc, wrow, xrow, c, rest);
  else if (rest > 4)
    up_small_chunk<NTB, 8>(acc, wrow, xrow, c, rest);
  else if (rest > 0)
    up_small_chunk<NTB, 4>(acc, wrow, xrow, c, rest);

  // element e of lane l is neuron 8(e/4) + 4(l/32) + e%4 of the block and token l % 32 of
  // the token block
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
    for (int e = 0; e < 16; ++e) red[((wave * NTB + tb) * 16 + e) * 64 + lane] = acc[tb][e];
  __syncthreads();
  // unit u = (token block u / 4, neurons 8 (u % 4) .. + 7): the eight partial sums in wave
  // order, then bias and ReLU
  for (int u = wave; u < NTB * 4; u += US_NW) {
    const int tb = u >> 2, q = u & 3;
    const int t = 32 * tb + r;
    if (t >= T) continue;
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * q + i;
      float sum = red[(tb * 16 + e) * 64 + lane];
#pragma unroll
      for (int w = 1; w < US_NW; ++w) sum += red[((w * NTB + tb) * 16 + e) * 64 + lane];
      z[i] = sum;
    }
    const int n = n0 + 8 * q + 4 * hh;
    const uint2 bw = *reinterpret_cast<const uint2*>(bu + n);
    float4 zz, hv;
    zz.x = z[0] + __uint_as_float(bw.x << 16);
    zz.y = z[1] + __uint_as_float(bw.x & 0xFFFF0000u);
    zz.z = z[2] + __uint_as_float(bw.y << 16);
    zz.w = z[3] + __uint_as_float(bw.y & 0xFFFF0000u);
    hv.x = zz.x > 0.0f ? zz.x : 0.0f;
    hv.y = zz.y > 0.0f ? zz.y : 0.0f;
    hv.z = zz.z > 0.0f ? zz.z : 0.0f;
    hv.w = zz.w > 0.0f ? zz.w : 0.0f;
    *reinterpret_cast<float4*>(h + (size_t)t * F + n) = hv;
    if (zdump) *reinterpret_cast<float4*>(zdump + (size_t)t * F + n) = zz;
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
  const dim3 grid(d.F / US_NB);
  if (d.T <= 32)
    hipLaunchKernelGGL(up_small_kernel<1>, grid, dim3(256), 0, s, d, x, Wu, bu, h, zdump, claim);
  else if (d.T <= 64)
    hipLaunchKernelGGL(up_small_kernel<2>, grid, dim3(256), 0, s, d, x, Wu, bu, h, zdump, claim);
  else
    hipLaunchKernelGGL(up_small8_kernel<4>, grid, dim3(US8_NW * 64), 0, s, d, x, Wu, bu, h,
                       zdump, claim);
  return hipGetLastError();
}

}  // namespace sffn
