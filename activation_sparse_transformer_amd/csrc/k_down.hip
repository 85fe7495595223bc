// Sparse down-projection over a TwELL activation (gfx950, VALU gather path).
//
// y[t, :] = sum_k ( sum_{s < min(count, W)} vals[k,t,s] * W_down[k*K + cols[k,t,s], :]
//                   + sum_{c : backup(k,t)[c] != 0} backup(k,t)[c] * W_down[k*K + c, :] )
//
// Only stored nonzeros are multiplied (upppp.jp TwELL article of 2026-05-11, section "What
// is the waste in LLM FFN layers": with ReLU most hidden activations are zero and their
// products are wasted work); the dense remainder slices of the hybrid form (same article,
// section "What TwELL and the custom CUDA kernels solve") are folded in per tile.
//
// Design for MI355X
//   * A workgroup owns a block of NW*TPW tokens x DC output columns; its fp32 accumulators
//     stay in registers for the whole pass over the n_t tiles (TPW tokens per wave, DCL
//     consecutive columns per lane).
//   * For each tile k the workgroup stages W_down[kK : kK+K, d0 : d0+DC] in LDS (256 B per
//     row, double-buffered; the next tile's global loads are in flight while the current
//     one is consumed).  Each row is then reused by every token of the block that has
//     that hidden column active.
//   * A token's TwELL row is wave-uniform: values and columns arrive through scalar loads
//     and every lane gathers its DCL columns of the selected W_down row from LDS
//     (conflict-free: 64 lanes read one contiguous 256-byte row).
//   * bf16: two slots are consumed at once: the two gathered rows are interleaved into
//     bf16 pairs and fed to v_dot2_f32_bf16 together with the slot pair (fp32 accumulate).
//   * Workgroups are mapped so that all token blocks of one column chunk run on the same
//     XCD (blocks are dispatched to the 8 XCDs round-robin), keeping that chunk of W_down
//     in the XCD's L2.
#include "sffn_common.hpp"

namespace sffn {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int DOWN_NW = 8;  // waves per workgroup

template <int K, int TPW, bool BF16>
__global__ __launch_bounds__(DOWN_NW * 64) void down_kernel(
    Dims d, const uint16_t* __restrict__ counts, const void* __restrict__ vals_,
    const uint8_t* __restrict__ cols, const int32_t* __restrict__ bk_tile_ptr,
    const int32_t* __restrict__ bk_tok, const void* __restrict__ bk_vals,
    const void* __restrict__ Wd_, void* __restrict__ y_) {
  constexpr int DCL = BF16 ? 2 : 1;          // output columns per lane
  constexpr int DC = 64 * DCL;               // output columns per workgroup
  constexpr int ROWW = 64;                   // 32-bit words per staged row (256 bytes)
  constexpr int NTHR = DOWN_NW * 64;
  constexpr int LOADS = K * ROWW / 4 / NTHR;  // 16-byte loads per thread per tile
  static_assert(LOADS >= 1, "tile too small for the workgroup");
  __shared__ uint4 wl4[2][K * ROWW / 4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int T = d.T, W = d.W;
  const int nd = d.D / DC;
  const int BT = DOWN_NW * TPW;
  const int ntb = (T + BT - 1) / BT;
  // XCD-aware mapping: consecutive (chunk, token-block) pairs share an XCD.
  const int total = nd * ntb;
  const int per_xcd = (total + 7) / 8;
  const int P = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (P >= total) return;
  const int dchunk = P / ntb;
  const int tb = P - dchunk * ntb;
  const int d0 = dchunk * DC;
  const int tw0 = tb * BT + wv * TPW;  // first token of this wave

  const uint4* __restrict__ Wd4 = static_cast<const uint4*>(Wd_);
  const size_t row_u4 = (size_t)d.D * (BF16 ? 2 : 4) / 16;  // uint4 per W_down row
  const size_t col_u4 = (size_t)d0 * (BF16 ? 2 : 4) / 16;

  // Thread's share of a staged tile: LOADS 16-byte pieces (row = r, piece = tid % 16).
  uint4 pre[LOADS];
  auto load_tile = [&](int k) {
#pragma unroll
    for (int q = 0; q < LOADS; ++q) {
      const int idx = q * NTHR + tid;
      const int r = idx >> 4, pc = idx & 15;
      pre[q] = Wd4[((size_t)k * K + r) * row_u4 + col_u4 + pc];
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int q = 0; q < LOADS; ++q) wl4[buf][q * NTHR + tid] = pre[q];
  };

  float acc[TPW][DCL];
#pragma unroll
  for (int i = 0; i < TPW; ++i)
#pragma unroll
    for (int j = 0; j < DCL; ++j) acc[i][j] = 0.0f;

  const uint16_t* __restrict__ vals16 = static_cast<const uint16_t*>(vals_);
  const float* __restrict__ vals32 = static_cast<const float*>(vals_);

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int k = 0; k < d.nt; ++k) {
    const int buf = k & 1;
    if (k + 1 < d.nt) load_tile(k + 1);
    const uint32_t* wl = reinterpret_cast<const uint32_t*>(wl4[buf]);

    // counts of this wave's tokens for tile k (lane i <-> token tw0 + i)
    int cnt_lane = 0;
    if (lane < TPW && tw0 + lane < T) cnt_lane = counts[(size_t)k * T + tw0 + lane];
    // backup entries of tile k: first entry with token >= tw0 (binary search)
    int e_lo = 0, e_hi = 0;
    if (__ballot(cnt_lane > W) != 0ull) {
      e_lo = ld_uniform(bk_tile_ptr + k);
      e_hi = ld_uniform(bk_tile_ptr + k + 1);
      e_hi = e_hi < d.cap ? e_hi : d.cap;
      e_lo = e_lo < e_hi ? e_lo : e_hi;
      int lo = e_lo, hi = e_hi;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (ld_uniform(bk_tok + mid) < tw0) lo = mid + 1; else hi = mid;
      }
      e_lo = lo;
    }
    int cursor = e_lo;

#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = tw0 + i;
      const int cnt = __builtin_amdgcn_readlane(cnt_lane, i);
      if (cnt == 0) continue;
      const int m = cnt < W ? cnt : W;
      // 32-bit index: the host keeps every TwELL array below 2 GiB
      const uint32_t row = ((uint32_t)k * (uint32_t)T + (uint32_t)t) * (uint32_t)W;
      if constexpr (BF16) {
        if ((W & 3) == 0) {
          // Slot quads: two bf16 value pairs and four 8-bit columns per step, read as
          // whole dwords (scalar loads).  Slots past the count are padding (0, 0) and add
          // exact zeros, so a quad may run past m up to W.
          const uint32_t* __restrict__ vrow =
              reinterpret_cast<const uint32_t*>(vals16 + row);
          const uint32_t* __restrict__ crow = reinterpret_cast<const uint32_t*>(cols + row);
          for (int s = 0; s < m; s += 4) {
            const uint32_t vq0 = ld_uniform(vrow + (s >> 1)), vq1 = ld_uniform(vrow + (s >> 1) + 1);
            const uint32_t cq = ld_uniform(crow + (s >> 2));
            const uint32_t w0 = wl[(cq & 0xFFu) * ROWW + lane];
            const uint32_t w1 = wl[((cq >> 8) & 0xFFu) * ROWW + lane];
            const uint32_t w2 = wl[((cq >> 16) & 0xFFu) * ROWW + lane];
            const uint32_t w3 = wl[(cq >> 24) * ROWW + lane];
            // (row c0 col d, row c1 col d) and (row c0 col d+1, row c1 col d+1)
            const uint32_t p0 = __builtin_amdgcn_perm(w1, w0, 0x05040100u);
            const uint32_t p1 = __builtin_amdgcn_perm(w1, w0, 0x07060302u);
            const uint32_t p2 = __builtin_amdgcn_perm(w3, w2, 0x05040100u);
            const uint32_t p3 = __builtin_amdgcn_perm(w3, w2, 0x07060302u);
            acc[i][0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p0),
                                                        __builtin_bit_cast(bf16x2_t, vq0),
                                                        acc[i][0], false);
            acc[i][1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p1),
                                                        __builtin_bit_cast(bf16x2_t, vq0),
                                                        acc[i][1], false);
            acc[i][0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p2),
                                                        __builtin_bit_cast(bf16x2_t, vq1),
                                                        acc[i][0], false);
            acc[i][1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p3),
                                                        __builtin_bit_cast(bf16x2_t, vq1),
                                                        acc[i][1], false);
          }
        } else {
          for (int s = 0; s < m; s += 2) {
            const uint32_t v1 = ld_uniform(vals16 + row + s);
            const bool two = s + 1 < m;
            const uint32_t v2 = two ? (uint32_t)ld_uniform(vals16 + row + s + 1) : 0u;
            const int c1 = ld_uniform(cols + row + s);
            const int c2 = two ? (int)ld_uniform(cols + row + s + 1) : c1;
            const uint32_t w1 = wl[c1 * ROWW + lane];
            const uint32_t w2 = wl[c2 * ROWW + lane];
            const uint32_t a_lo = __builtin_amdgcn_perm(w2, w1, 0x05040100u);
            const uint32_t a_hi = __builtin_amdgcn_perm(w2, w1, 0x07060302u);
            const uint32_t vv = v1 | (v2 << 16);
            acc[i][0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a_lo),
                                                        __builtin_bit_cast(bf16x2_t, vv),
                                                        acc[i][0], false);
            acc[i][1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a_hi),
                                                        __builtin_bit_cast(bf16x2_t, vv),
                                                        acc[i][1], false);
          }
        }
      } else {
        for (int s = 0; s < m; ++s) {
          const float v = ld_uniform(vals32 + row + s);
          const int c = ld_uniform(cols + row + s);
          acc[i][0] = fmaf(v, __uint_as_float(wl[c * ROWW + lane]), acc[i][0]);
        }
      }
      if (cnt > W) {
        // this tile-row's dense remainder: the next entry of tile k in token order
        const int e = cursor;
        if (e < e_hi && ld_uniform(bk_tok + e) == t) {
          ++cursor;
          constexpr int WORDS = K * (BF16 ? 2 : 4) / 4;
          const uint32_t* sl = static_cast<const uint32_t*>(bk_vals) + (size_t)e * WORDS;
#pragma unroll
          for (int q0 = 0; q0 < WORDS; q0 += 64) {
            const uint32_t dw = (q0 + lane < WORDS) ? sl[q0 + lane] : 0u;
            if constexpr (BF16) {
              uint64_t mlo = __ballot((dw & 0xFFFFu) != 0u);
              uint64_t mhi = __ballot((dw >> 16) != 0u);
              uint64_t mm = mlo | mhi;
              while (mm) {
                const int l = __builtin_ctzll(mm);
                mm &= mm - 1;
                const uint32_t wsrc = __builtin_amdgcn_readlane(dw, l);
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                  const uint32_t bits = half ? (wsrc >> 16) : (wsrc & 0xFFFFu);
                  if (bits == 0u) continue;
                  const float v = __uint_as_float(bits << 16);
                  const int c = 2 * (q0 + l) + half;
                  const uint32_t w = wl[c * ROWW + lane];
                  acc[i][0] = fmaf(v, __uint_as_float(w << 16), acc[i][0]);
                  acc[i][1] = fmaf(v, __uint_as_float(w & 0xFFFF0000u), acc[i][1]);
                }
              }
            } else {
              uint64_t mm = __ballot(dw != 0u);
              while (mm) {
                const int l = __builtin_ctzll(mm);
                mm &= mm - 1;
                const float v = __uint_as_float(__builtin_amdgcn_readlane(dw, l));
                const int c = q0 + l;
                acc[i][0] = fmaf(v, __uint_as_float(wl[c * ROWW + lane]), acc[i][0]);
              }
            }
          }
        }
      }
    }
    if (k + 1 < d.nt) store_tile(buf ^ 1);
    __syncthreads();
  }

  // write y (rounded to the layer dtype)
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = tw0 + i;
    if (t >= T) break;
    if constexpr (BF16) {
      const uint32_t packed = (uint32_t)f32_to_bf16(acc[i][0]) | ((uint32_t)f32_to_bf16(acc[i][1]) << 16);
      static_cast<uint32_t*>(y_)[((size_t)t * d.D + d0) / 2 + lane] = packed;
    } else {
      static_cast<float*>(y_)[(size_t)t * d.D + d0 + lane] = acc[i][0];
    }
  }
}

template <int K, int TPW, bool BF16>
static hipError_t launch_down_t(const Dims& d, const twell_buffers_t& b, const void* Wd, void* y,
                                hipStream_t s) {
  constexpr int DC = BF16 ? 128 : 64;
  const int nd = d.D / DC;
  const int ntb = (d.T + DOWN_NW * TPW - 1) / (DOWN_NW * TPW);
  const int total = nd * ntb;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL((down_kernel<K, TPW, BF16>), dim3(8 * per_xcd), dim3(DOWN_NW * 64), 0, s,
                     d, b.counts, b.vals, b.cols, b.bk_tile_ptr, b.bk_tok, b.bk_vals, Wd, y);
  return hipGetLastError();
}

template <int K, bool BF16>
static hipError_t launch_down_k(const Dims& d, const twell_buffers_t& b, const void* Wd, void* y,
                                hipStream_t s) {
  // Tokens per wave: as many as keep >= ~2 workgroups per CU on 256 CUs.
  constexpr int DC = BF16 ? 128 : 64;
  const long long units = (long long)(d.D / DC) * d.T;  // (chunk, token) pairs
  if (units >= 512LL * DOWN_NW * 32) return launch_down_t<K, 32, BF16>(d, b, Wd, y, s);
  if (units >= 512LL * DOWN_NW * 16) return launch_down_t<K, 16, BF16>(d, b, Wd, y, s);
  return launch_down_t<K, 8, BF16>(d, b, Wd, y, s);
}

hipError_t launch_down(const Dims& d, const twell_buffers_t& b, const void* Wd, void* y,
                       hipStream_t s) {
  if (d.bf16) {
    if (d.K == 64) return launch_down_k<64, true>(d, b, Wd, y, s);
    if (d.K == 128) return launch_down_k<128, true>(d, b, Wd, y, s);
    return launch_down_k<256, true>(d, b, Wd, y, s);
  }
  if (d.K == 64) return launch_down_k<64, false>(d, b, Wd, y, s);
  if (d.K == 128) return launch_down_k<128, false>(d, b, Wd, y, s);
  return launch_down_k<256, false>(d, b, Wd, y, s);
}

}  // namespace sffn
