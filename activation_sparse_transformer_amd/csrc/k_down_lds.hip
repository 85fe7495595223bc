// Down-projection of sparse bf16 layers on the vector ALUs, with W_down tiles staged in LDS
// and shared by the 256 tokens of a workgroup (upppp.jp TwELL article of 2026-05-11, section
// "What TwELL and the custom CUDA kernels solve": the down-projection runs over the stored
// nonzeros only, and the TwELL tiles line up with tiled matrix-multiply execution).
//
//   y[t, d] = sum over tiles k, stored (column c, value v) of token t in tile k: v W_down[kK + c, d]
//
// Work and LDS reads grow with the stored nonzeros: for each pair of stored nonzeros of a
// token, every lane reads its CPL columns of the two W_down rows from LDS, packs them into
// bf16 pairs with v_perm and accumulates with the two-term bf16 dot product of gfx950
// (v_dot2c_f32_bf16, fp32 accumulation: one instruction for two multiply-adds, no bf16 ->
// fp32 conversions).  The slot pairs (2p, 2p+1) of a tile-row are stored next to each other,
// so a value pair is one 32-bit word and its two columns one 16-bit word.
//
// Workgroup: 256 tokens x DC = 64*CPL output columns, 16 waves of 16 tokens (two waves per
// 32-token group, whose backup entries are found from the group's first entry and a ballot);
// lane l owns columns d0 + CPL*l .. +CPL-1 and the 16 x CPL fp32 accumulators stay in
// registers for the whole tile loop.  Per tile k the K x DC slice of W_down is loaded into
// LDS by direct global->LDS loads, double-buffered, and so are the wave's slot pairs and the
// group's counts, in registers: the tile-rows of consecutive tokens are contiguous, so NR
// coalesced loads give lane (j % (64/HP))*HP + p of register j / (64/HP) the pair p of token
// j (HP = W/2 rounded up to a power of two).  Once a tile's data has arrived, its column
// pairs are turned into LDS row offsets and its counts into pair counts, all in vector
// form, so the loop over a token's nonzeros is readlane broadcasts, address adds, LDS reads,
// v_perm and dot products, two pairs per step (an unused second pair is zero padding).
// Workgroups are ordered so that the ones on one XCD share a column chunk: that chunk of
// W_down (F x DC bf16, 4 MB at d_ff 8192, DC 256) is read from HBM about once per XCD and
// then served by its L2.
#include "sffn_common.hpp"

namespace sffn {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int DL_WAVES = 16;
constexpr int DL_TPW = 16;                 // tokens per wave: half a 32-token group
constexpr int DL_BM = DL_WAVES * DL_TPW;   // 256 tokens per workgroup

// a * b + c for a, b < 2^24 and a result below 2^32, as a 24-bit multiply-add: a 32-bit
// multiply-add is selected as v_mad_u64_u32, whose unused high addend register can be one a
// load is still writing, and the wait for it would stall the next tile's loads
__device__ __forceinline__ uint32_t mad24(int a, int b, int c) {
  return __umul24((uint32_t)a, (uint32_t)b) + (uint32_t)c;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

template <int K, int CPL, int HP>
__global__ __launch_bounds__(64 * DL_WAVES) void down_lds_kernel(
    Dims d, const uint16_t* __restrict__ counts, const uint32_t* __restrict__ vals2,
    const uint32_t* __restrict__ cols4, const uint16_t* __restrict__ bk_vals,
    const int32_t* __restrict__ grp_first, const uint16_t* __restrict__ Wd,
    uint16_t* __restrict__ y, const int32_t* __restrict__ blk_nnz, long long lo, long long hi,
    DownHint hint) {
  constexpr int DC = 64 * CPL;              // output columns per workgroup
  constexpr int ROWB = DC * 2;              // bytes per staged W_down row
  constexpr int STAGE = K * DC;             // bf16 elements of one staged W_down slice
  constexpr int PPR = DC / 8;               // 16-byte pieces per staged row
  constexpr int LPW = STAGE / 8 / 64 / DL_WAVES;  // direct loads per wave per slice
  static_assert(LPW * 64 * DL_WAVES * 8 == STAGE, "slice must split evenly over the waves");
  constexpr int TPR = 64 / HP;              // tokens per slot register
  constexpr int NR = DL_TPW / TPR;          // slot registers per wave
  // two stages as separate objects: reads of one are known not to alias loads into the other
  __shared__ __attribute__((aligned(16))) uint16_t sW0[STAGE];
  __shared__ __attribute__((aligned(16))) uint16_t sW1[STAGE];

  const int T = d.T, D = d.D, W = d.W, nt = d.nt;
  // the layer goes to this kernel only when its stored-nonzero count is in (lo, hi]
  if (blk_nnz != nullptr) {
    const long long n = layer_nnz(blk_nnz, (T + 255) / 256);
    if (n <= lo || n > hi) return;
  }
  note_choice(hint, (T + 255) / 256, blockIdx.x == 0);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));

  // ---- workgroup -> (column chunk, token block); consecutive positions P run over the token
  // blocks of one chunk and each XCD (blockIdx % 8) takes a contiguous range of P
  const int nTB = (T + DL_BM - 1) / DL_BM;
  const int nDC = (D + DC - 1) / DC;
  const int total = nTB * nDC;
  const int per_xcd = (total + 7) / 8;
  const int P = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (P >= total) return;
  const int chunk = P / nTB, tb = P - chunk * nTB;
  const int d0 = chunk * DC;
  const int tg = tb * DL_BM + (wave >> 1) * GROUP;  // first token of this wave's group
  const int half = (wave & 1) * DL_TPW;              // this wave's tokens: tg + half + j
  const int tw = tg + half;
  const int g = tg / GROUP;
  const int hw = W >> 1;                             // slot pairs per tile-row (even, <= HP)

  typedef __attribute__((address_space(3))) void* lds_ptr;
  auto issue_w = [&](int k, uint16_t* sW) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
      const int blk = wave * LPW + q;  // 64 pieces = 1 KB per direct load
      const int piece = blk * 64 + lane;
      const int r = piece / PPR;
      int col = d0 + (piece - r * PPR) * 8;
      col = col < D ? col : D - 8;  // columns past d_model: any in-range source
      __builtin_amdgcn_global_load_lds(Wd + mad24(k * K + r, D, col),
                                       (lds_ptr)(sW + blk * 512), 16, 0, 0);
    }
  };
  // slot pairs of the wave's tile-rows and counts of the group's, in tile k, as raw 32-bit
  // words.  The rows of tokens past T are in range (the buffers end with a group of padding
  // rows).  Lanes past a row's pairs load pair 0 again (never read).  The 16-bit column
  // pairs and counts are cut out of their words, and counts of lanes past the group or
  // past T masked to 0, only once the tile is used: an operation on a loaded value right
  // after the load would make the loads of the next tile wait for their data.
  const int lp = lane % HP;
  const int loff = (lane / HP) * hw + (lp < hw ? lp : 0);
  const uint32_t cmask = (lane < GROUP && tg + lane < T) ? 0xFFFFFFFFu : 0u;
  const int ctok = tg + (lane < GROUP ? lane : 0) < T ? tg + (lane < GROUP ? lane : 0) : T - 1;
  const uint32_t csh = (uint32_t)(lp & 1) * 16u;  // (hw even: pair lp sits in half lp % 2)
  const uint32_t* counts2 = reinterpret_cast<const uint32_t*>(counts);
  auto load_slots = [&](int k, uint32_t (&sv)[NR], uint32_t (&sc)[NR], uint32_t& cnt)
      __attribute__((always_inline)) {
    const uint32_t row0 = (uint32_t)((k * T + tw) * hw + loff);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      sv[r] = vals2[row0 + (uint32_t)(r * TPR * hw)];
      sc[r] = cols4[(row0 + (uint32_t)(r * TPR * hw)) >> 1];  // word holding pair lp
    }
    cnt = counts2[(uint32_t)(k * T + ctok) >> 1];  // word holding the count
  };

  float acc[DL_TPW][CPL];
#pragma unroll
  for (int i = 0; i < DL_TPW; ++i)
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[i][e] = 0.0f;

  const uint32_t lbase = (uint32_t)(lane * CPL * 2);  // this lane's byte offset in a row
  // add v0.lo W[r0a] + v0.hi W[r0b] + v1.lo W[r1a] + v1.hi W[r1b] (rows given as LDS byte
  // offsets) to token i's columns; all four rows are read before any is used
  auto pairs_fma = [&](const uint16_t* sW, int i, uint32_t v0, uint32_t r0a, uint32_t r0b,
                       uint32_t v1, uint32_t r1a, uint32_t r1b) __attribute__((always_inline)) {
    const char* base = reinterpret_cast<const char*>(sW);
    if constexpr (CPL == 4) {
      const uint2 a0 = *reinterpret_cast<const uint2*>(base + (lbase + r0a));
      const uint2 a1 = *reinterpret_cast<const uint2*>(base + (lbase + r0b));
      const uint2 b0 = *reinterpret_cast<const uint2*>(base + (lbase + r1a));
      const uint2 b1 = *reinterpret_cast<const uint2*>(base + (lbase + r1b));
      acc[i][0] = dot2_bf16(__builtin_amdgcn_perm(a1.x, a0.x, 0x05040100u), v0, acc[i][0]);
      acc[i][1] = dot2_bf16(__builtin_amdgcn_perm(a1.x, a0.x, 0x07060302u), v0, acc[i][1]);
      acc[i][2] = dot2_bf16(__builtin_amdgcn_perm(a1.y, a0.y, 0x05040100u), v0, acc[i][2]);
      acc[i][3] = dot2_bf16(__builtin_amdgcn_perm(a1.y, a0.y, 0x07060302u), v0, acc[i][3]);
      acc[i][0] = dot2_bf16(__builtin_amdgcn_perm(b1.x, b0.x, 0x05040100u), v1, acc[i][0]);
      acc[i][1] = dot2_bf16(__builtin_amdgcn_perm(b1.x, b0.x, 0x07060302u), v1, acc[i][1]);
      acc[i][2] = dot2_bf16(__builtin_amdgcn_perm(b1.y, b0.y, 0x05040100u), v1, acc[i][2]);
      acc[i][3] = dot2_bf16(__builtin_amdgcn_perm(b1.y, b0.y, 0x07060302u), v1, acc[i][3]);
    } else {
      const uint32_t a0 = *reinterpret_cast<const uint32_t*>(base + (lbase + r0a));
      const uint32_t a1 = *reinterpret_cast<const uint32_t*>(base + (lbase + r0b));
      const uint32_t b0 = *reinterpret_cast<const uint32_t*>(base + (lbase + r1a));
      const uint32_t b1 = *reinterpret_cast<const uint32_t*>(base + (lbase + r1b));
      acc[i][0] = dot2_bf16(__builtin_amdgcn_perm(a1, a0, 0x05040100u), v0, acc[i][0]);
      acc[i][1] = dot2_bf16(__builtin_amdgcn_perm(a1, a0, 0x07060302u), v0, acc[i][1]);
      acc[i][0] = dot2_bf16(__builtin_amdgcn_perm(b1, b0, 0x05040100u), v1, acc[i][0]);
      acc[i][1] = dot2_bf16(__builtin_amdgcn_perm(b1, b0, 0x07060302u), v1, acc[i][1]);
    }
  };

  auto pair_fma = [&](const uint16_t* sW, int i, uint32_t v0, uint32_t r0a, uint32_t r0b)
      __attribute__((always_inline)) {
    const char* base = reinterpret_cast<const char*>(sW);
    if constexpr (CPL == 4) {
      const uint2 a0 = *reinterpret_cast<const uint2*>(base + (lbase + r0a));
      const uint2 a1 = *reinterpret_cast<const uint2*>(base + (lbase + r0b));
      acc[i][0] = dot2_bf16(__builtin_amdgcn_perm(a1.x, a0.x, 0x05040100u), v0, acc[i][0]);
      acc[i][1] = dot2_bf16(__builtin_amdgcn_perm(a1.x, a0.x, 0x07060302u), v0, acc[i][1]);
      acc[i][2] = dot2_bf16(__builtin_amdgcn_perm(a1.y, a0.y, 0x05040100u), v0, acc[i][2]);
      acc[i][3] = dot2_bf16(__builtin_amdgcn_perm(a1.y, a0.y, 0x07060302u), v0, acc[i][3]);
    } else {
      const uint32_t a0 = *reinterpret_cast<const uint32_t*>(base + (lbase + r0a));
      const uint32_t a1 = *reinterpret_cast<const uint32_t*>(base + (lbase + r0b));
      acc[i][0] = dot2_bf16(__builtin_amdgcn_perm(a1, a0, 0x05040100u), v0, acc[i][0]);
      acc[i][1] = dot2_bf16(__builtin_amdgcn_perm(a1, a0, 0x07060302u), v0, acc[i][1]);
    }
  };

  uint32_t svA[NR], scA[NR], cntA, svB[NR], scB[NR], cntB;
  // Every tile step issues the same loads (past the last tile they repeat it), so the
  // compiler sees one path through the step and its waits.
  issue_w(0, sW0);
  load_slots(0, svA, scA, cntA);

  auto tile = [&](int k, const uint16_t* sW, uint16_t* sWn, const uint32_t (&sv)[NR],
                  const uint32_t (&sc)[NR], uint32_t cnt_raw, uint32_t (&svn)[NR],
                  uint32_t (&scn)[NR], uint32_t& cntn) __attribute__((always_inline)) {
    // this wave's slice k and slots are in ...
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    // ... and every wave's, and slice k-1 is no longer read.  A plain s_barrier (the
    // memory clobber keeps the compiler from moving memory accesses across it).
    __asm__ volatile("s_barrier" ::: "memory");
    // this tile's data, in the forms the loops use
    const uint32_t craw = cnt_raw;
    const uint32_t (&svl)[NR] = sv;
    const uint32_t (&scl)[NR] = sc;
    const uint32_t cnt = ((craw >> ((uint32_t)((k * T + ctok) & 1) * 16u)) & 0xFFFFu) & cmask;
    const uint32_t npv = ((cnt < (uint32_t)W ? cnt : (uint32_t)W) + 1u) >> 1;  // pairs in use
    uint32_t ra[NR], rb[NR];  // LDS byte offsets of the two rows of each pair
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint32_t cp = scl[r] >> csh;
      ra[r] = (cp & 0xFFu) * ROWB;
      rb[r] = ((cp >> 8) & 0xFFu) * ROWB;
    }
    {
      const int kn = k + 1 < nt ? k + 1 : k;
      issue_w(kn, sWn);
      load_slots(kn, svn, scn, cntn);
    }
    // overflowing tile-rows of the group: entry = first entry of (k, g) + rank in the group
    const uint64_t ovm = ballot64(cnt > (uint32_t)W);  // lanes < 32 only (cmask)
    const int e0 = ovm != 0ull ? ld_uniform(grp_first + (uint32_t)(k * d.ng + g)) : 0;
    // this wave's tokens with any stored nonzero in tile k: bit i for token half + i
    const uint32_t busy = (uint32_t)(ballot64(cnt != 0u) >> half) & 0xFFFFu;
#pragma unroll
    for (int i = 0; i < DL_TPW; ++i) {
      if (!((busy >> i) & 1u)) continue;
      const int np = __builtin_amdgcn_readlane((int)npv, half + i);
      const int vr = (int)svl[i / TPR];
      const int rar = (int)ra[i / TPR], rbr = (int)rb[i / TPR];
      const int lb = (i % TPR) * HP;
      // pairs p and p+1 per step; p+1 < hw always (np <= hw, hw even), and a pair at or
      // past np is the row's zero padding
      int p = 0;
      for (; p + 2 <= np; p += 2) {
        const int l0 = lb + p;
        pairs_fma(sW, i, (uint32_t)__builtin_amdgcn_readlane(vr, l0),
                  (uint32_t)__builtin_amdgcn_readlane(rar, l0),
                  (uint32_t)__builtin_amdgcn_readlane(rbr, l0),
                  (uint32_t)__builtin_amdgcn_readlane(vr, l0 + 1),
                  (uint32_t)__builtin_amdgcn_readlane(rar, l0 + 1),
                  (uint32_t)__builtin_amdgcn_readlane(rbr, l0 + 1));
      }
      if (p < np) {  // a last single pair
        const int l0 = lb + p;
        pair_fma(sW, i, (uint32_t)__builtin_amdgcn_readlane(vr, l0),
                 (uint32_t)__builtin_amdgcn_readlane(rar, l0),
                 (uint32_t)__builtin_amdgcn_readlane(rbr, l0));
      }
      if ((ovm >> (half + i)) & 1ull) {
        // remainder nonzeros in the backup slice: adjacent columns (2q, 2q+1) form a pair
        const int e = e0 + __builtin_popcountll(ovm & ((1ull << (half + i)) - 1ull));
        if (e < d.cap) {
          const uint32_t* sl = reinterpret_cast<const uint32_t*>(bk_vals + (uint32_t)(e * K));
#pragma unroll
          for (int h = 0; h < (K + 127) / 128; ++h) {
            const int q = h * 64 + lane;
            const uint32_t bv = q < K / 2 ? sl[q] : 0u;
            uint64_t nzm = ballot64(bv != 0u);
            while (nzm != 0ull) {
              const int b0 = __builtin_ctzll(nzm);
              nzm &= nzm - 1ull;
              const bool two = nzm != 0ull;
              const int b1 = two ? __builtin_ctzll(nzm) : b0;
              nzm &= nzm - 1ull;  // (no-op when empty)
              const uint32_t v0 = (uint32_t)__builtin_amdgcn_readlane((int)bv, b0);
              const uint32_t v1 =
                  (uint32_t)__builtin_amdgcn_readlane((int)bv, b1) & (two ? 0xFFFFFFFFu : 0u);
              const uint32_t q0 = (uint32_t)(2 * (h * 64 + b0)), q1 = (uint32_t)(2 * (h * 64 + b1));
              pairs_fma(sW, i, v0, q0 * ROWB, (q0 + 1) * ROWB, v1, q1 * ROWB, (q1 + 1) * ROWB);
            }
          }
        }
      }
    }
  };
  for (int k = 0; k < nt; k += 2) {
    tile(k, sW0, sW1, svA, scA, cntA, svB, scB, cntB);
    if (k + 1 < nt) tile(k + 1, sW1, sW0, svB, scB, cntB, svA, scA, cntA);
  }

  // the last step's loads (repeats of the last tile) must land before the LDS goes away
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  // ---- y: CPL bf16 per lane per token
  const int c0 = d0 + lane * CPL;
  if (c0 < D) {
#pragma unroll
    for (int i = 0; i < DL_TPW; ++i) {
      const int t = tw + i;
      if (t < T) {
        uint16_t* yp = y + (uint32_t)(t * D + c0);
        if constexpr (CPL == 4) {
          const uint32_t o0 = (uint32_t)f32_to_bf16(acc[i][0]) | ((uint32_t)f32_to_bf16(acc[i][1]) << 16);
          const uint32_t o1 = (uint32_t)f32_to_bf16(acc[i][2]) | ((uint32_t)f32_to_bf16(acc[i][3]) << 16);
          *reinterpret_cast<uint2*>(yp) = make_uint2(o0, o1);
        } else {
          *reinterpret_cast<uint32_t*>(yp) =
              (uint32_t)f32_to_bf16(acc[i][0]) | ((uint32_t)f32_to_bf16(acc[i][1]) << 16);
        }
      }
    }
  }
}

bool down_lds_supported(const Dims& d) {
  // 32-bit element offsets inside the kernel: every buffer it indexes stays below 2^31
  const long long lim = 1ll << 31;
  const bool fits = (long long)d.F * d.D < lim && ((long long)d.nt * d.T + GROUP) * d.W < lim &&
                    d.F < (1 << 24) && d.D < (1 << 24) &&
                    (long long)d.T * d.D < lim && (long long)d.cap * d.K < lim &&
                    (long long)d.nt * d.ng < lim;
  return d.bf16 && d.W % 4 == 0 && d.W <= 64 && d.D >= 8 && fits &&
         (d.K == 64 || d.K == 128 || d.K == 256);
}

template <int K, int CPL>
static void launch_lds_k(const Dims& d, dim3 grid, dim3 block, hipStream_t s,
                         const uint16_t* c, const uint32_t* v, const uint32_t* cl,
                         const uint16_t* bk, const int32_t* gf, const uint16_t* w, uint16_t* yy,
                         const int32_t* blk_nnz, long long lo, long long hi, const DownHint& hint) {
  const int hw = d.W / 2;
  if (hw <= 8)
    hipLaunchKernelGGL((down_lds_kernel<K, CPL, 8>), grid, block, 0, s, d, c, v, cl, bk, gf, w,
                       yy, blk_nnz, lo, hi, hint);
  else if (hw <= 16)
    hipLaunchKernelGGL((down_lds_kernel<K, CPL, 16>), grid, block, 0, s, d, c, v, cl, bk, gf, w,
                       yy, blk_nnz, lo, hi, hint);
  else
    hipLaunchKernelGGL((down_lds_kernel<K, CPL, 32>), grid, block, 0, s, d, c, v, cl, bk, gf, w,
                       yy, blk_nnz, lo, hi, hint);
}

hipError_t launch_down_lds(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                           const void* Wd, void* y, const int32_t* blk_nnz, long long lo,
                           long long hi, hipStream_t s, const DownHint& hint) {
  if (!down_lds_supported(d)) return hipErrorInvalidValue;
  auto* c = b.counts;
  auto* v = static_cast<const uint32_t*>(b.vals);
  auto* cl = reinterpret_cast<const uint32_t*>(b.cols);
  auto* bk = static_cast<const uint16_t*>(b.bk_vals);
  auto* w = static_cast<const uint16_t*>(Wd);
  auto* yy = static_cast<uint16_t*>(y);
  const int cpl = d.K == 256 ? 2 : 4;
  const int nTB = (d.T + DL_BM - 1) / DL_BM;
  const int nDC = (d.D + 64 * cpl - 1) / (64 * cpl);
  const int per_xcd = (nTB * nDC + 7) / 8;
  const dim3 grid(8 * per_xcd), block(64 * DL_WAVES);
  switch (d.K) {
    case 64: launch_lds_k<64, 4>(d, grid, block, s, c, v, cl, bk, ws.grp_first, w, yy, blk_nnz, lo, hi, hint); break;
    case 128: launch_lds_k<128, 4>(d, grid, block, s, c, v, cl, bk, ws.grp_first, w, yy, blk_nnz, lo, hi, hint); break;
    case 256: launch_lds_k<256, 2>(d, grid, block, s, c, v, cl, bk, ws.grp_first, w, yy, blk_nnz, lo, hi, hint); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sffn
