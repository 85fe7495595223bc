// Down-projection of very sparse bf16 layers: each token reads only the W_down rows that its
// stored nonzeros select (upppp.jp TwELL article of 2026-05-11, section "What TwELL and the
// custom CUDA kernels solve": the down-projection runs over the stored nonzeros only, and
// W_down rows are the natural coalesced gather unit).
//
//   y[t, :] = sum over the stored (tile k, column c, value v) of token t of  v W_down[kK + c, :]
//
// The work and the W_down bytes read grow with the nonzeros (4 KB of W_down per nonzero for
// d_model 2048), so this kernel wins when few rows are used; the matrix-core kernel (whose
// work does not depend on the density) takes dense layers.
//
// One workgroup per token at a time (NW waves; for few tokens, when the gather is the call's
// only down kernel, NW = 16 and the workgroups of a token also split its columns into 256-wide
// chunks, 128-wide for a handful of tokens, so a short batch still spreads over many CUs);
// wave w takes a contiguous 1/NW of the
// tiles, lane l of it tile k = k0 + l: its count, then its slots 8 at a time (16 B values +
// 8 B columns).  The (row, value) pairs of the lanes are gathered with readlane into batches
// (slot i in lane i;
// 32 pairs for the 256- and 128-column chunks, 8 up to d_model 2048 and 4 above otherwise) whose
// W_down row loads are all issued before any is used, so a token with many nonzeros (heavy
// tokens run at 10-20x the mean density) is not a chain of single-row latencies.  Lane L owns
// the EPL output columns c0 + 64 EPL q + EPL L (q < NQ; c0 = the workgroup's column chunk;
// EPL = 8, or 4 / 2 for the 256- / 128-column chunks): every row is read as NQ coalesced wave loads of
// 128 EPL bytes.  The waves' partial rows are summed in LDS and y is written as 4 EPL-byte
// stores.
#include "sffn_common.hpp"

namespace sffn {

template <int NQ, int ROWS_WAVES, int EPL = 8>
__global__ __launch_bounds__(64 * ROWS_WAVES) void down_rows_kernel(
    Dims d, const uint16_t* __restrict__ counts, const uint16_t* __restrict__ vals,
    const uint8_t* __restrict__ cols, const uint16_t* __restrict__ bk_vals,
    const int32_t* __restrict__ grp_first, const uint16_t* __restrict__ Wd,
    uint16_t* __restrict__ y, const int32_t* __restrict__ blk_nnz, long long thr, DownHint hint) {
  static_assert(EPL == 8 || EPL == 4 || EPL == 2, "8, 4 or 2 output columns per lane");
  constexpr int CW = 64 * EPL;                 // columns of one wave load of a row
  // rows in flight per wave (registers: NQ EPL / 2 each; at most 64, one lane per slot)
  constexpr int ROWS_BATCH = (NQ == 1 && EPL <= 4) ? 32 : (NQ <= 4 ? 8 : 4);
  __shared__ __attribute__((aligned(16))) float part[ROWS_WAVES - 1][NQ * CW];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int T = d.T, D = d.D, K = d.K, W = d.W;
  const int cb = blockIdx.y * NQ * CW;  // first output column of this workgroup
  // the layer goes to this kernel only when its stored-nonzero count is at most thr
  if (blk_nnz != nullptr && layer_nnz(blk_nnz, (T + 255) / 256) > thr) return;
  note_choice(hint, (T + 255) / 256, blockIdx.x == 0 && blockIdx.y == 0);
  for (int t = blockIdx.x; t < T; t += gridDim.x) {  // workgroup-uniform token loop
  float acc[NQ][EPL];
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[q][e] = 0.0f;

  // a batch of up to ROWS_BATCH (row, value) pairs, slot i in lane i of bjl and bvl: the row
  // loads first, then the FMAs
  int bjl = 0;
  uint32_t bvl = 0u;
  int nb = 0;
  auto flush = [&]() __attribute__((always_inline)) {
    uint32_t w[ROWS_BATCH][NQ][EPL / 2];  // EPL bf16 of the row per lane and chunk
#pragma unroll
    for (int i = 0; i < ROWS_BATCH; ++i) {
#pragma unroll
      for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int e = 0; e < EPL / 2; ++e) w[i][q][e] = 0u;
      if (i < nb) {  // wave-uniform
        const uint16_t* wr = Wd + (size_t)__builtin_amdgcn_readlane(bjl, i) * D;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int c0 = cb + CW * q + EPL * lane;
          if (c0 < D) {
            if constexpr (EPL == 8) {
              const uint4 u = *reinterpret_cast<const uint4*>(wr + c0);
              w[i][q][0] = u.x, w[i][q][1] = u.y, w[i][q][2] = u.z, w[i][q][3] = u.w;
            } else if constexpr (EPL == 4) {
              const uint2 u = *reinterpret_cast<const uint2*>(wr + c0);
              w[i][q][0] = u.x, w[i][q][1] = u.y;
            } else {
              w[i][q][0] = *reinterpret_cast<const uint32_t*>(wr + c0);
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < ROWS_BATCH; ++i) {
      const float v = i < nb ? __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)bvl, i) << 16)
                             : 0.0f;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const uint32_t* ww = w[i][q];
#pragma unroll
        for (int e = 0; e < EPL / 2; ++e) {
          acc[q][2 * e] = fmaf(v, __uint_as_float(ww[e] << 16), acc[q][2 * e]);
          acc[q][2 * e + 1] = fmaf(v, __uint_as_float(ww[e] & 0xFFFF0000u), acc[q][2 * e + 1]);
        }
      }
    }
    nb = 0;
  };
  // add the pairs (jl, vl) of the lanes in `act` (lane-varying values, broadcast one by one)
  auto add_lanes = [&](uint64_t act, int jl, uint32_t vl) __attribute__((always_inline)) {
    while (act != 0) {
      const int b = __builtin_ctzll(act);
      act &= act - 1;
      const int j = __builtin_amdgcn_readlane(jl, b);
      const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)vl, b);
      bjl = lane == nb ? j : bjl;
      bvl = lane == nb ? v : bvl;
      if (++nb == ROWS_BATCH) flush();
    }
  };

  const int per = (d.nt + ROWS_WAVES - 1) / ROWS_WAVES;  // tiles per wave (<= 64 checked)
  const int k0 = wave * per;
  const int k = k0 + lane;
  const bool own = lane < per && k < d.nt;
  const uint32_t cnt = own ? counts[(size_t)k * T + t] : 0u;
  const uint32_t m = cnt < (uint32_t)W ? cnt : (uint32_t)W;
  int mx = (int)m;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o));
  const int mmax = __builtin_amdgcn_readfirstlane(mx);
  const size_t row = ((size_t)(own ? k : 0) * T + t) * W;
  // slots s0 .. s0+7 of this lane's tile-row (rows are W bytes / 2W bytes, W % 8 == 0), the
  // next eight loaded while these are added
  uint4 v4n = make_uint4(0, 0, 0, 0);
  uint2 c2n = make_uint2(0, 0);
  if (0u < m) {
    v4n = *reinterpret_cast<const uint4*>(vals + row);
    c2n = *reinterpret_cast<const uint2*>(cols + row);
  }
  for (int s0 = 0; s0 < mmax; s0 += 8) {
    const uint4 v4 = v4n;
    const uint2 c2 = c2n;
    if ((uint32_t)(s0 + 8) < m) {
      v4n = *reinterpret_cast<const uint4*>(vals + row + s0 + 8);
      c2n = *reinterpret_cast<const uint2*>(cols + row + s0 + 8);
    }
    const uint32_t vv[4] = {v4.x, v4.y, v4.z, v4.w};
    const uint32_t cc[2] = {c2.x, c2.y};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t col = (cc[e >> 2] >> (8 * (e & 3))) & 0xFFu;
      const uint32_t val = (e & 1) ? (vv[e >> 1] >> 16) : (vv[e >> 1] & 0xFFFFu);
      add_lanes(ballot64((uint32_t)(s0 + e) < m), k * K + (int)col, val);
    }
  }
  // backup slices of this wave's overflowing tiles: the entry of (k, t) is the first of its
  // 32-token group plus the number of the group's earlier tokens that overflow in tile k
  uint64_t ovt = ballot64(cnt > (uint32_t)W);
  while (ovt != 0) {
    const int b = __builtin_ctzll(ovt);
    ovt &= ovt - 1;
    const int kb = k0 + b;
    const int g = t / GROUP;
    const int tl = g * GROUP + (lane & 31);
    const uint32_t cg = (lane < 32 && tl < T) ? counts[(size_t)kb * T + tl] : 0u;
    const uint64_t ov = ballot64(cg > (uint32_t)W);
    const int rank = __builtin_popcountll(ov & ((1ull << (t - g * GROUP)) - 1ull));
    const int e = ld_uniform(grp_first + kb * d.ng + g) + rank;
    if (e >= d.cap) continue;  // capacity exceeded: the status word reports it
    // the slice's K <= 256 values, all loaded before any is added
    const uint16_t* sl = bk_vals + (size_t)e * K;
    uint32_t sv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) sv[q] = 64 * q < K ? (uint32_t)sl[64 * q + lane] : 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (64 * q < K) add_lanes(ballot64(sv[q] != 0u), kb * K + 64 * q + lane, sv[q]);
  }
  if (nb > 0) flush();

  // ---- sum the waves' partial rows in LDS; wave 0 writes y
  if (wave > 0) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      float* p = &part[wave - 1][CW * q + EPL * lane];
#pragma unroll
      for (int e = 0; e < EPL; ++e) p[e] = acc[q][e];
    }
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int c0 = cb + CW * q + EPL * lane;
      if (c0 < D) {
#pragma unroll
        for (int w2 = 0; w2 < ROWS_WAVES - 1; ++w2) {
          const float* p = &part[w2][CW * q + EPL * lane];
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[q][e] += p[e];
        }
        uint32_t o[EPL / 2];
#pragma unroll
        for (int e = 0; e < EPL / 2; ++e)
          o[e] = (uint32_t)f32_to_bf16(acc[q][2 * e]) |
                 ((uint32_t)f32_to_bf16(acc[q][2 * e + 1]) << 16);
        uint16_t* yo = y + (size_t)t * D + c0;
        if constexpr (EPL == 8)
          *reinterpret_cast<uint4*>(yo) = make_uint4(o[0], o[1], o[2], o[3]);
        else if constexpr (EPL == 4)
          *reinterpret_cast<uint2*>(yo) = make_uint2(o[0], o[1]);
        else
          *reinterpret_cast<uint32_t*>(yo) = o[0];
      }
    }
  }
  __syncthreads();  // part[] is rewritten for the next token
  }
}

// Few tokens, gather alone: 16 waves per workgroup and one 256-column chunk per workgroup.
constexpr int ROWS_FEW_T = 1024;

bool down_rows_supported(const Dims& d) {
  return d.bf16 && d.D <= 4096 && d.D % 8 == 0 && d.W % 8 == 0 && (d.nt + 3) / 4 <= 64;
}

hipError_t launch_down_rows(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                            const void* Wd, void* y, const int32_t* blk_nnz, long long thr,
                            hipStream_t s, const DownHint& hint) {
  if (!down_rows_supported(d)) return hipErrorInvalidValue;
  // from ROWS_FEW_T tokens at most 2048 workgroups (x), each looping over tokens: a skipped
  // launch (the layer went to the matrix cores) then costs little
  auto* c = b.counts;
  auto* v = static_cast<const uint16_t*>(b.vals);
  auto* bk = static_cast<const uint16_t*>(b.bk_vals);
  auto* w = static_cast<const uint16_t*>(Wd);
  auto* yy = static_cast<uint16_t*>(y);
  if (d.T < ROWS_FEW_T) {
    // few tokens: 16-wave workgroups over 256-column chunks, also as a candidate of the kernel
    // choice (the auto policy launches the candidates only until a call has recorded the
    // kernel its count selects), so that the gather's sums do not depend on how it was
    // launched
    if ((long long)d.T * ((d.D + 255) / 256) < 128) {
      // a handful of tokens: 128-column chunks, twice the workgroups (each CU's share of the
      // gathered rows bounds these)
      const dim3 grid(d.T, (d.D + 127) / 128), block(64 * 16);
      hipLaunchKernelGGL((down_rows_kernel<1, 16, 2>), grid, block, 0, s, d, c, v, b.cols, bk,
                         ws.grp_first, w, yy, blk_nnz, thr, hint);
      return hipGetLastError();
    }
    const dim3 grid(d.T, (d.D + 255) / 256), block(64 * 16);
    hipLaunchKernelGGL((down_rows_kernel<1, 16, 4>), grid, block, 0, s, d, c, v, b.cols, bk,
                       ws.grp_first, w, yy, blk_nnz, thr, hint);
    return hipGetLastError();
  }
  // many tokens: 4-wave workgroups over whole tokens
  const dim3 grid(d.T < 2048 ? d.T : 2048), block(64 * 4);
  switch ((d.D + 511) / 512) {
#define SFFN_ROWS(NQ)                                                                      \
  case NQ:                                                                                 \
    hipLaunchKernelGGL((down_rows_kernel<NQ, 4>), grid, block, 0, s, d, c, v, b.cols, bk,   \
                       ws.grp_first, w, yy, blk_nnz, thr, hint);                           \
    break;
    SFFN_ROWS(1) SFFN_ROWS(2) SFFN_ROWS(3) SFFN_ROWS(4)
    SFFN_ROWS(5) SFFN_ROWS(6) SFFN_ROWS(7) SFFN_ROWS(8)
#undef SFFN_ROWS
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sffn
