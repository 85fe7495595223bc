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
//  * fewer than 8 tokens (one token block) where W_up's quarters fit LDS (d_model <= 2048, a
//    multiple of 512): 4 waves, each over a quarter of d_model in batches of 8 steps whose
//    loads are in flight together.  Each wave first copies its 32 W_up rows x D/4
//    columns into its own LDS region with contiguous 1 KB direct loads (16-byte piece s of row
//    rr at slot s ^ (rr % 16), so the fragment reads of 16 rows hit distinct banks): read in
//    the MFMA layout straight from memory, each load used 32 bytes of 32 lines, and W_up
//    streamed at 6.3 TB/s against 11.3 TB/s for whole-row loads (a probe over the 1.5B-like
//    layer's W_up, cache-resident as in the forward);
//  * otherwise, for d_model a multiple of 64 (one, two or four token blocks): 8 waves, each
//    over an eighth of d_model in groups of four steps, with the W_up pieces of four groups
//    (two for four token blocks, whose token rows take the registers) in flight at once and
//    the token rows of the next group loaded as whole 128-byte lines and staged through the
//    wave's own LDS (a token row's 32 bytes per step, loaded straight into the MFMA layout,
//    cost a line fetch from L2 each: the 4-wave form took 17.8 us at 64 tokens against
//    10.5 us at 32, and this form 12-13 us).
// Other shapes run the 4-wave form with W_up and the token rows loaded straight from memory.
#include "sffn_common.hpp"

namespace sffn {

typedef __bf16 bf16x8_s __attribute__((ext_vector_type(8)));
typedef float floatx16_s __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_s __attribute__((ext_vector_type(4)));

constexpr int US_NB = 32;  // neurons per workgroup

constexpr int US_STG_MAXQ = 512;  // d_model columns of a wave's quarter when W_up is staged

template <int NTB, bool STG>
__global__ __launch_bounds__(256) void up_small_kernel(Dims d, const uint16_t* __restrict__ x,
                                                       const uint16_t* __restrict__ Wu,
                                                       const uint16_t* __restrict__ bu,
                                                       float* __restrict__ h,
                                                       float* __restrict__ zdump) {
  __shared__ __attribute__((aligned(16))) float red[4][16][64];
  // STG: each wave's 32 W_up rows x D/4 columns (16-byte pieces, swizzled by row)
  __shared__ __attribute__((aligned(16))) uint4 sw[STG ? 4 : 1][STG ? 32 * US_STG_MAXQ / 8 : 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int D = d.D, T = d.T, F = d.F;
  const int n0 = blockIdx.x * US_NB;
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
  if constexpr (STG) {
    // D % 512 == 0 and D <= 2048: the quarter is q = D/4 columns, ppr = q/8 pieces per row
    // (a multiple of 16), q/16 steps (a multiple of 8)
    const int q = D / 4, ppr = q / 8, c0 = wave * q;
    uint4* my = sw[wave];
    typedef __attribute__((address_space(3))) void* lds_ptr_s;
    // slot p = 64 i + lane of the region: row p / ppr, logical piece (p % ppr) ^ (row % 16)
    for (int i = 0; i < 32 * ppr / 64; ++i) {
      const int p = i * 64 + lane;
      const int rr = p / ppr, sl = p - rr * ppr;
      __builtin_amdgcn_global_load_lds(Wu + (size_t)(n0 + rr) * D + c0 + 8 * (sl ^ (rr & 15)),
                                       (lds_ptr_s)(my + i * 64), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the wave's own region is in
    for (int k2 = 0; k2 < q / 16; k2 += ST) {
      bf16x8_s a[ST], b[ST][NTB];
#pragma unroll
      for (int u = 0; u < ST; ++u) {
        const int sp = 2 * (k2 + u) + hh;  // logical piece of this lane's 8 columns
        a[u] = __builtin_bit_cast(bf16x8_s, my[r * ppr + (sp ^ (r & 15))]);
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
          b[u][tb] = *reinterpret_cast<const bf16x8_s*>(xrow[tb] + c0 + (k2 + u) * 16);
      }
#pragma unroll
      for (int u = 0; u < ST; ++u)
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
          acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u], b[u][tb], acc[tb], 0, 0, 0);
    }
  }
  int ks = STG ? ks1 : ks0;
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

// groups of four steps per chunk for four token blocks (two: the 8 W_up pieces, two sets of
// token-row lines and the accumulators fill the 256 registers of a wave at two waves per SIMD)
constexpr int US8_NGC = 2;
// the same for one and two token blocks (fewer token-row registers: more W_up pieces in flight)
constexpr int US8_NGC12 = 4;

// Groups g0 .. g0 + n - 1 (1 <= n <= NGC) of one wave of the 8-wave form.  A group is
// four 16-column steps: 64 columns, one 128-byte line of every token row.  The W_up pieces of
// the whole chunk are loaded first.  The 32 NTB token rows of a group are loaded as whole
// lines (8 lanes per row, 8 rows per load), one group ahead of the MFMAs, and written to the
// wave's own 4 NTB KB of LDS (row t at t * 128 bytes, 16-byte piece p at (p ^ (t & 7)) * 16),
// from which each step reads its MFMA operand (lane l: row 32 tb + l % 32, piece 2 j + l / 32).
// Groups past n repeat a valid address and multiply a zero A.
template <int NGC, int NTB>
__device__ __forceinline__ void up_small8_chunk(floatx16_s (&acc)[NTB], const uint16_t* wrow,
                                                const uint16_t* xl, const int* toff, char* xs,
                                                int g0, int n, int lane) {
  bf16x8_s a[4 * NGC];
#pragma unroll
  for (int st = 0; st < 4 * NGC; ++st) {
    const int g = st >> 2, gc = g < n ? g : n - 1;
    a[st] = *reinterpret_cast<const bf16x8_s*>(wrow + ((g0 + gc) * 4 + (st & 3)) * 16);
  }
  constexpr int NL = 4 * NTB;  // token-row loads per group
  u32x4_s xr0[NL], xr1[NL];    // token-row lines of even and odd groups
#pragma unroll
  for (int i = 0; i < NL; ++i) xr0[i] = *reinterpret_cast<const u32x4_s*>(xl + toff[i] + g0 * 64);
  // keep the scheduler from sinking these loads back next to their uses
  __builtin_amdgcn_sched_barrier(0);
  const bf16x8_s zero = {};
  const int wp = lane & 7;
#pragma unroll
  for (int g = 0; g < NGC; ++g) {
    u32x4_s(&cur)[NL] = (g & 1) ? xr1 : xr0;
    u32x4_s(&nxt)[NL] = (g & 1) ? xr0 : xr1;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int t = 8 * i + (lane >> 3);
      *reinterpret_cast<u32x4_s*>(xs + t * 128 + ((wp ^ (t & 7)) << 4)) = cur[i];
    }
    if (g + 1 < NGC) {
      const int gc = g + 1 < n ? g + 1 : n - 1;
#pragma unroll
      for (int i = 0; i < NL; ++i)
        nxt[i] = *reinterpret_cast<const u32x4_s*>(xl + toff[i] + (g0 + gc) * 64);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8_s av = g < n ? a[4 * g + j] : zero;
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) {
        const int R = 32 * tb + (lane & 31), P = 2 * j + (lane >> 5);
        const bf16x8_s b =
            *reinterpret_cast<const bf16x8_s*>(xs + R * 128 + ((P ^ (R & 7)) << 4));
        acc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b, acc[tb], 0, 0, 0);
      }
    }
  }
}

template <int NTB, int NGC>
__global__ __launch_bounds__(US8_NW * 64) void up_small8_kernel(
    Dims d, const uint16_t* __restrict__ x, const uint16_t* __restrict__ Wu,
    const uint16_t* __restrict__ bu, float* __restrict__ h, float* __restrict__ zdump) {
  static_assert(NTB == 1 || NTB == 2 || NTB == 4, "the 8-wave form stages 32, 64 or 128 token rows");
  constexpr int US_NW = US8_NW;
  // wave w's 4 NTB KB: first its staged token rows, then its partial sums
  // [wave][token block][element][lane] (the same bytes, after its last MFMA)
  __shared__ __attribute__((aligned(16))) float red[US_NW * NTB * 16 * 64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int D = d.D, T = d.T, F = d.F;
  const int n0 = blockIdx.x * US_NB;
  const int r = lane & 31, hh = lane >> 5;
  const int ngr = D / 64;                          // groups of four steps (D % 64 == 0)
  const int g0 = wave * ngr / US_NW, g1 = (wave + 1) * ngr / US_NW;
  const uint16_t* wrow = Wu + (size_t)(n0 + r) * D + 8 * hh;
  // token-row loads: load i of lane l reads row 8 i + l / 8 (rows past T repeat row T - 1),
  // 16-byte piece l % 8 of the group's line
  const uint16_t* xl = x + 8 * (lane & 7);
  int toff[4 * NTB];
#pragma unroll
  for (int i = 0; i < 4 * NTB; ++i) {
    const int t = 8 * i + (lane >> 3);
    toff[i] = (t < T ? t : T - 1) * D;
  }
  char* xs = reinterpret_cast<char*>(red) + wave * NTB * 4096;

  floatx16_s acc[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[tb][e] = 0.0f;
  int g = g0;
  for (; g + NGC <= g1; g += NGC) up_small8_chunk<NGC, NTB>(acc, wrow, xl, toff, xs, g, NGC, lane);
  if (g < g1) up_small8_chunk<NGC, NTB>(acc, wrow, xl, toff, xs, g, g1 - g, lane);

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

// W_up staged through LDS: the four quarters of d_model fit the 32 KB regions
static bool up_small_staged(const Dims& d) { return d.D % 512 == 0 && d.D / 4 <= US_STG_MAXQ; }

bool up_small_supported(const Dims& d) {
  return d.bf16 && d.T <= UP_SMALL_T && d.D % 16 == 0 && d.F % US_NB == 0;
}
static_assert(UP_SMALL_T <= 128, "at most four 32-token blocks per workgroup");

hipError_t launch_up_small(const Dims& d, const uint16_t* x, const uint16_t* Wu,
                           const uint16_t* bu, float* h, float* zdump,
                           hipStream_t s) {
  if (!up_small_supported(d)) return hipErrorInvalidValue;
  const dim3 grid(d.F / US_NB), g8(US8_NW * 64);
  if (d.T < 8 && up_small_staged(d))
    hipLaunchKernelGGL((up_small_kernel<1, true>), grid, dim3(256), 0, s, d, x, Wu, bu, h, zdump);
  else if (d.D % 64 == 0 && d.T <= 32)
    hipLaunchKernelGGL((up_small8_kernel<1, US8_NGC12>), grid, g8, 0, s, d, x, Wu, bu, h, zdump);
  else if (d.D % 64 == 0 && d.T <= 64)
    hipLaunchKernelGGL((up_small8_kernel<2, US8_NGC12>), grid, g8, 0, s, d, x, Wu, bu, h, zdump);
  else if (d.D % 64 == 0)
    hipLaunchKernelGGL((up_small8_kernel<4, US8_NGC>), grid, g8, 0, s, d, x, Wu, bu, h, zdump);
  else if (d.T <= 32)
    hipLaunchKernelGGL((up_small_kernel<1, false>), grid, dim3(256), 0, s, d, x, Wu, bu, h, zdump);
  else if (d.T <= 64)
    hipLaunchKernelGGL((up_small_kernel<2, false>), grid, dim3(256), 0, s, d, x, Wu, bu, h, zdump);
  else
    hipLaunchKernelGGL((up_small_kernel<4, false>), grid, dim3(256), 0, s, d, x, Wu, bu, h, zdump);
  return hipGetLastError();
}

}  // namespace sffn
