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
//   * A workgroup (16 waves) owns NW*TPW tokens x 128 output columns (bf16; 64 for fp32):
//     each lane accumulates 2 consecutive columns (1 for fp32) of TPW tokens in fp32
//     registers for the whole pass over the n_t tiles.
//   * Per tile k, W_down[kK : kK+K, d0 : d0+DC] (256 bytes per row) and each wave's TwELL
//     block (its TPW tokens' W-slot rows of values and columns, contiguous in the
//     tile-major layout) are copied global -> LDS with direct loads, double-buffered: tile
//     k+1 is in flight while tile k is consumed.
//   * A token's slots are wave-uniform: they are read from LDS by broadcast and used
//     directly as VALU operands.  The LDS address of W_down row c for this lane is
//     (c << 8) | (lane * 4), built by one v_perm from the byte holding c.  Slots are
//     consumed in pairs: the two gathered rows are interleaved into bf16 pairs and fed to
//     v_dot2_f32_bf16 together with the slot value pair (fp32 accumulate).
//   * Workgroups are numbered token-block-major per XCD (blocks go to the 8 XCDs
//     round-robin): the workgroups an XCD runs at once share their token blocks' TwELL
//     through that XCD's L2 and together read W_down tiles across all memory channels.
#include <type_traits>

#include "sffn_common.hpp"

namespace sffn {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int DOWN_NW = 16;   // waves per workgroup
constexpr int DOWN_TPW = 16;  // tokens per wave
constexpr int DOWN_BT = DOWN_NW * DOWN_TPW;
constexpr int DOWN_LDS = 160 * 1024;  // the whole LDS of a CU: one workgroup per CU

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Fold the backup slice of tile-row (k, t) into acc (rare: only overflowing tile-rows).
template <int K, bool BF16>
__device__ __forceinline__ void add_backup(const void* __restrict__ bk_vals, int e,
                                           const uint32_t* wl, int lane, float& a0, float& a1) {
  constexpr int WORDS = K * (BF16 ? 2 : 4) / 4;
  const uint32_t* sl = static_cast<const uint32_t*>(bk_vals) + (size_t)e * WORDS;
#pragma unroll
  for (int q0 = 0; q0 < WORDS; q0 += 64) {
    const uint32_t dw = (q0 + lane < WORDS) ? sl[q0 + lane] : 0u;
    if constexpr (BF16) {
      uint64_t mm = __ballot((dw & 0xFFFFu) != 0u) | __ballot((dw >> 16) != 0u);
      while (mm) {
        const int l = __builtin_ctzll(mm);
        mm &= mm - 1;
        const uint32_t wsrc = __builtin_amdgcn_readlane(dw, l);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const uint32_t bits = half ? (wsrc >> 16) : (wsrc & 0xFFFFu);
          if (bits == 0u) continue;
          const float v = __uint_as_float(bits << 16);
          const uint32_t w = wl[(2 * (q0 + l) + half) * 64 + lane];
          a0 = fmaf(v, __uint_as_float(w << 16), a0);
          a1 = fmaf(v, __uint_as_float(w & 0xFFFF0000u), a1);
        }
      }
    } else {
      uint64_t mm = __ballot(dw != 0u);
      while (mm) {
        const int l = __builtin_ctzll(mm);
        mm &= mm - 1;
        const float v = __uint_as_float(__builtin_amdgcn_readlane(dw, l));
        a0 = fmaf(v, __uint_as_float(wl[(q0 + l) * 64 + lane]), a0);
      }
    }
  }
}

template <int K, bool BF16, bool FAST>
__global__ __launch_bounds__(DOWN_NW * 64) void down_kernel(
    Dims d, const uint16_t* __restrict__ counts, const void* __restrict__ vals_,
    const uint8_t* __restrict__ cols, const int32_t* __restrict__ bk_tile_ptr,
    const int32_t* __restrict__ bk_tok, const void* __restrict__ bk_vals,
    const void* __restrict__ Wd_, void* __restrict__ y_, int tv_bytes, int tc_bytes,
    const int32_t* __restrict__ blk_nnz, long long thr) {
  constexpr int DCL = BF16 ? 2 : 1;   // output columns per lane
  constexpr int DC = 64 * DCL;        // output columns per workgroup
  constexpr int ESZ = BF16 ? 2 : 4;
  constexpr int WROW = 256;           // bytes of one staged W_down row
  constexpr int WTILE = K * WROW;     // bytes of one staged W_down tile
  // LDS: [W tile 0][W tile 1][TwELL stage 0][TwELL stage 1]; a TwELL stage holds DOWN_NW
  // blocks of (values tv_bytes, columns tc_bytes).  A static array, so that every LDS
  // offset is a compile-time immediate (the launcher checks the layout fits).
  __shared__ __attribute__((aligned(16))) unsigned char smem[DOWN_LDS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = d.T, W = d.W;
  const int nd = d.D / DC;
  const int ntb = (T + DOWN_BT - 1) / DOWN_BT;
  const int total = nd * ntb;
  const int per_xcd = (total + 7) / 8;
  const int P = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (P >= total) return;
  // token-block-major: the workgroups an XCD runs at once cover all column chunks of a few
  // token blocks, so each TwELL block is fetched once into that XCD's L2 and the W_down
  // tile loads spread over every memory channel
  const int tb = P / nd;
  if (blk_nnz != nullptr && layer_nnz(blk_nnz, ntb) > thr) return;  // the matrix cores' layer
  const int dchunk = P - tb * nd;
  const int d0 = dchunk * DC;
  const int tw0 = tb * DOWN_BT + wv * DOWN_TPW;  // first token of this wave
  const int ntok = max(0, min(DOWN_TPW, T - tw0));  // valid tokens of this wave

  const int stage_bytes = DOWN_NW * (tv_bytes + tc_bytes);
  auto wt_lds = [&](int buf) { return smem + buf * WTILE; };
  auto tw_lds = [&](int buf) { return smem + 2 * WTILE + buf * stage_bytes; };

  const unsigned char* Wd = static_cast<const unsigned char*>(Wd_);
  const size_t wrow_g = (size_t)d.D * ESZ;  // bytes per W_down row in memory
  const unsigned char* vals_b = static_cast<const unsigned char*>(vals_);

  // ---- async staging of tile k into buffer `buf`
  auto issue = [&](int k, int buf) {
    // W_down tile: K rows x 256 B = K*16 pieces of 16 B, loaded by 64-lane instructions of
    // 4 rows each, spread over the waves.
    constexpr int INSTR = K * 16 / 64;
#pragma unroll
    for (int j = 0; j < INSTR / DOWN_NW; ++j) {
      const int ins = j * DOWN_NW + wv;
      const int piece = ins * 64 + lane;
      const int r = piece >> 4, pc = piece & 15;
      __builtin_amdgcn_global_load_lds(
          Wd + ((size_t)k * K + r) * wrow_g + (size_t)d0 * ESZ + pc * 16,
          (lds_void_ptr)(wt_lds(buf) + ins * 1024), 16, 0, 0);
    }
    if constexpr (FAST) {
      // this wave's TwELL block: ntok rows of W values and W columns
      unsigned char* tv = tw_lds(buf) + wv * (tv_bytes + tc_bytes);
      const size_t row0 = (size_t)k * T + tw0;
      const int vb = ntok * W * ESZ, cb = ntok * W;
      for (int off = 0; off < vb; off += 1024) {
        if (off + lane * 16 < vb)
          __builtin_amdgcn_global_load_lds(vals_b + row0 * W * ESZ + off + lane * 16,
                                           (lds_void_ptr)(tv + off), 16, 0, 0);
      }
      for (int off = 0; off < cb; off += 1024) {
        if (off + lane * 16 < cb)
          __builtin_amdgcn_global_load_lds(cols + row0 * W + off + lane * 16,
                                           (lds_void_ptr)(tv + tv_bytes + off), 16, 0, 0);
      }
    }
  };

  float acc[DOWN_TPW][DCL];
#pragma unroll
  for (int i = 0; i < DOWN_TPW; ++i)
#pragma unroll
    for (int j = 0; j < DCL; ++j) acc[i][j] = 0.0f;

  auto load_counts = [&](int k) -> int {
    return (lane < ntok) ? (int)counts[(size_t)k * T + tw0 + lane] : 0;
  };

  issue(0, 0);
  int cnt_next = load_counts(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  const uint32_t lane4 = (uint32_t)lane * 4u;
  // One tile step; BUF is a compile-time buffer index so LDS offsets fold into immediates.
  auto step = [&](int k, auto buf_c) {
    constexpr int buf = decltype(buf_c)::value;
    const int cnt_lane = cnt_next;
    if (k + 1 < d.nt) {
      issue(k + 1, buf ^ 1);
      cnt_next = load_counts(k + 1);
    }
    const uint32_t* wl = reinterpret_cast<const uint32_t*>(wt_lds(buf));
    const unsigned char* tv = tw_lds(buf) + wv * (tv_bytes + tc_bytes);
    const unsigned char* tc = tv + tv_bytes;

    // backup entries of tile k: first entry with token >= tw0 (binary search)
    int e_hi = 0, cursor = 0;
    if (__ballot(cnt_lane > W) != 0ull) {
      int e_lo = ld_uniform(bk_tile_ptr + k);
      e_hi = ld_uniform(bk_tile_ptr + k + 1);
      e_hi = e_hi < d.cap ? e_hi : d.cap;
      e_lo = e_lo < e_hi ? e_lo : e_hi;
      int lo = e_lo, hi = e_hi;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (ld_uniform(bk_tok + mid) < tw0) lo = mid + 1; else hi = mid;
      }
      cursor = lo;
    }

#pragma unroll
    for (int i = 0; i < DOWN_TPW; ++i) {
      const int cnt = __builtin_amdgcn_readlane(cnt_lane, i);
      if (cnt == 0) continue;
      const int m = cnt < W ? cnt : W;
      if constexpr (FAST && BF16) {
        // Slot quads (W % 16 == 0 here): slots past m are padding (0, 0) and add exact
        // zeros; the second pair of a quad is skipped when m ends inside the first.
        for (int s = 0; s < m; s += 4) {
          const uint2 vq = *reinterpret_cast<const uint2*>(tv + (i * W + s) * 2);
          const uint32_t cq = *reinterpret_cast<const uint32_t*>(tc + i * W + s);
          {
            const uint32_t a0 = __builtin_amdgcn_perm(cq, lane4, 0x0C0C0400u);  // (c0<<8)|4*lane
            const uint32_t a1 = __builtin_amdgcn_perm(cq, lane4, 0x0C0C0500u);  // (c1<<8)|4*lane
            const uint32_t w0 = *reinterpret_cast<const uint32_t*>(
                reinterpret_cast<const unsigned char*>(wl) + a0);
            const uint32_t w1 = *reinterpret_cast<const uint32_t*>(
                reinterpret_cast<const unsigned char*>(wl) + a1);
            acc[i][0] = dot2_bf16(__builtin_amdgcn_perm(w1, w0, 0x05040100u), vq.x, acc[i][0]);
            acc[i][1] = dot2_bf16(__builtin_amdgcn_perm(w1, w0, 0x07060302u), vq.x, acc[i][1]);
          }
          if (s + 2 < m) {
            const uint32_t a2 = __builtin_amdgcn_perm(cq, lane4, 0x0C0C0600u);
            const uint32_t a3 = __builtin_amdgcn_perm(cq, lane4, 0x0C0C0700u);
            const uint32_t w2 = *reinterpret_cast<const uint32_t*>(
                reinterpret_cast<const unsigned char*>(wl) + a2);
            const uint32_t w3 = *reinterpret_cast<const uint32_t*>(
                reinterpret_cast<const unsigned char*>(wl) + a3);
            acc[i][0] = dot2_bf16(__builtin_amdgcn_perm(w3, w2, 0x05040100u), vq.y, acc[i][0]);
            acc[i][1] = dot2_bf16(__builtin_amdgcn_perm(w3, w2, 0x07060302u), vq.y, acc[i][1]);
          }
        }
      } else if constexpr (FAST && !BF16) {
        // Slot quads, as above: one 16-byte read of four values and one of four columns,
        // then the four W_down reads together (slots past m add exact zeros)
        const float* vrow = reinterpret_cast<const float*>(tv + i * W * 4);
        const uint8_t* crow = tc + i * W;
        for (int s = 0; s < m; s += 4) {
          const float4 vq = *reinterpret_cast<const float4*>(vrow + s);
          const uint32_t cq = *reinterpret_cast<const uint32_t*>(crow + s);
          const float w0 = __uint_as_float(wl[(cq & 0xFFu) * 64 + lane]);
          const float w1 = __uint_as_float(wl[((cq >> 8) & 0xFFu) * 64 + lane]);
          const float w2 = __uint_as_float(wl[((cq >> 16) & 0xFFu) * 64 + lane]);
          const float w3 = __uint_as_float(wl[(cq >> 24) * 64 + lane]);
          float a = acc[i][0];
          a = fmaf(vq.x, w0, a);
          a = fmaf(vq.y, w1, a);
          a = fmaf(vq.z, w2, a);
          a = fmaf(vq.w, w3, a);
          acc[i][0] = a;
        }
      } else {
        // generic slot layout (any W): scalar reads straight from the TwELL arrays
        const uint32_t row = ((uint32_t)k * (uint32_t)T + (uint32_t)(tw0 + i)) * (uint32_t)W;
        for (int s = 0; s < m; ++s) {
          const uint32_t c = ld_uniform(cols + row + s);
          const uint32_t w = wl[c * 64 + lane];
          if constexpr (BF16) {
            const float v = __uint_as_float(
                (uint32_t)static_cast<const uint16_t*>(vals_)[row + s] << 16);
            acc[i][0] = fmaf(v, __uint_as_float(w << 16), acc[i][0]);
            acc[i][DCL - 1] = fmaf(v, __uint_as_float(w & 0xFFFF0000u), acc[i][DCL - 1]);
          } else {
            const float v = static_cast<const float*>(vals_)[row + s];
            acc[i][0] = fmaf(v, __uint_as_float(w), acc[i][0]);
          }
        }
      }
      if (cnt > W) {
        const int t = tw0 + i;
        if (cursor < e_hi && ld_uniform(bk_tok + cursor) == t) {
          add_backup<K, BF16>(bk_vals, cursor, wl, lane, acc[i][0], acc[i][DCL - 1]);
          ++cursor;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // tile k+1 landed in LDS
    __syncthreads();
  };
  for (int k = 0; k < d.nt; k += 2) {
    step(k, std::integral_constant<int, 0>());
    if (k + 1 < d.nt) step(k + 1, std::integral_constant<int, 1>());
  }

  // write y (rounded to the layer dtype)
#pragma unroll
  for (int i = 0; i < DOWN_TPW; ++i) {
    if (i >= ntok) break;
    const int t = tw0 + i;
    if constexpr (BF16) {
      const uint32_t packed =
          (uint32_t)f32_to_bf16(acc[i][0]) | ((uint32_t)f32_to_bf16(acc[i][1]) << 16);
      static_cast<uint32_t*>(y_)[((size_t)t * d.D + d0) / 2 + lane] = packed;
    } else {
      static_cast<float*>(y_)[(size_t)t * d.D + d0 + lane] = acc[i][0];
    }
  }
}

template <int K, bool BF16, bool FAST>
static hipError_t launch_down_t(const Dims& d, const twell_buffers_t& b, const void* Wd, void* y,
                                const int32_t* blk_nnz, long long thr, hipStream_t s) {
  constexpr int DC = BF16 ? 128 : 64;
  const int esz = BF16 ? 2 : 4;
  const int nd = d.D / DC;
  const int ntb = (d.T + DOWN_BT - 1) / DOWN_BT;
  const int total = nd * ntb;
  const int per_xcd = (total + 7) / 8;
  const int tv = FAST ? ((DOWN_TPW * d.W * esz + 15) & ~15) : 0;
  const int tc = FAST ? ((DOWN_TPW * d.W + 15) & ~15) : 0;
  const size_t lds = 2 * (size_t)K * 256 + 2 * (size_t)DOWN_NW * (tv + tc);
  if (lds > DOWN_LDS) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((down_kernel<K, BF16, FAST>), dim3(8 * per_xcd), dim3(DOWN_NW * 64), 0, s, d,
                     b.counts, b.vals, b.cols, b.bk_tile_ptr, b.bk_tok, b.bk_vals, Wd, y, tv, tc,
                     blk_nnz, thr);
  return hipGetLastError();
}

template <int K, bool BF16>
static hipError_t launch_down_k(const Dims& d, const twell_buffers_t& b, const void* Wd, void* y,
                                const int32_t* blk_nnz, long long thr, hipStream_t s) {
  // The LDS fast path needs 16-byte aligned TwELL rows and room for two stages.
  const int esz = BF16 ? 2 : 4;
  const size_t lds_fast = 2 * (size_t)K * 256 +
                          2 * (size_t)DOWN_NW * (((DOWN_TPW * d.W * esz + 15) & ~15) +
                                                 ((DOWN_TPW * d.W + 15) & ~15));
  if (d.W % 16 == 0 && lds_fast <= DOWN_LDS) return launch_down_t<K, BF16, true>(d, b, Wd, y, blk_nnz, thr, s);
  return launch_down_t<K, BF16, false>(d, b, Wd, y, blk_nnz, thr, s);
}

hipError_t launch_down(const Dims& d, const twell_buffers_t& b, const void* Wd, void* y,
                       const int32_t* blk_nnz, long long thr, hipStream_t s) {
  if (d.bf16) {
    if (d.K == 64) return launch_down_k<64, true>(d, b, Wd, y, blk_nnz, thr, s);
    if (d.K == 128) return launch_down_k<128, true>(d, b, Wd, y, blk_nnz, thr, s);
    return launch_down_k<256, true>(d, b, Wd, y, blk_nnz, thr, s);
  }
  if (d.K == 64) return launch_down_k<64, false>(d, b, Wd, y, blk_nnz, thr, s);
  if (d.K == 128) return launch_down_k<128, false>(d, b, Wd, y, blk_nnz, thr, s);
  return launch_down_k<256, false>(d, b, Wd, y, blk_nnz, thr, s);
}

// Stored nonzeros (true tile-row counts) of every 256-token block: 1024 threads per block;
// thread i sums tiles i/256, i/256 + 4, ... of token i%256 (coalesced 512-byte rows).
__global__ __launch_bounds__(1024) void block_nnz_kernel(Dims d,
                                                         const uint16_t* __restrict__ counts,
                                                         int32_t* __restrict__ blk_nnz) {
  __shared__ int part[16];
  const int tb = blockIdx.x;
  const int t = tb * 256 + (threadIdx.x & 255);
  int sum = 0;
  if (t < d.T) {
#pragma unroll 8
    for (int k = threadIdx.x >> 8; k < d.nt; k += 4) sum += counts[(size_t)k * d.T + t];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = sum;
  __syncthreads();
  if (threadIdx.x < 64) {
    int v = threadIdx.x < 16 ? part[threadIdx.x] : 0;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (threadIdx.x == 0) blk_nnz[tb] = v;
  }
}

hipError_t launch_block_nnz(const Dims& d, const twell_buffers_t& b, int32_t* blk_nnz,
                            hipStream_t s) {
  hipLaunchKernelGGL(block_nnz_kernel, dim3((d.T + 255) / 256), dim3(1024), 0, s, d, b.counts,
                     blk_nnz);
  return hipGetLastError();
}

}  // namespace sffn
