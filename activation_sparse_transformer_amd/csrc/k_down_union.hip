// Down-projection over a TwELL activation on the matrix cores, contracting each 64-token
// block only over the union of its tokens' nonzero columns (gfx950).
//
//   y[t, :] = sum_k  H_k[t, :] W_down[k*K : (k+1)*K, :]
//
// The stored nonzeros are what the down-projection has to multiply (upppp.jp TwELL
// article of 2026-05-11, section "What is the waste in LLM FFN layers": the zeros of the
// activation make most of a dense down-projection wasted work; section "What TwELL and the
// custom CUDA kernels solve": tiles aligned with tiled matrix-multiply execution, sparse
// main part plus a few dense backups).  A matrix-core contraction needs a dense operand,
// so per 64-token block and 64-column step the kernel builds a compacted one:
//
//   * U = the columns of the step where at least one of the block's 64 tokens has a stored
//     nonzero (main slot or backup), read from the per-(tile, 32-token group) column unions
//     the TwELL producers write;
//   * A = the block's rows restricted to U, in ascending column order (a stored value goes
//     to position rank_U(column)), B = the W_down rows of U; the MFMA runs ceil(|U| / 16)
//     k-steps instead of 4.  When |U| > 48 (no k-step to save) the step is contracted
//     densely (U = every column), exactly as a dense tile.
//
// Workgroup = 256 tokens x 256 output columns, 8 waves in a 2 x 4 grid, each computing 128
// tokens x 64 columns with v_mfma_f32_32x32x16_bf16 (A = hidden rows, B = W_down): its
// rows are two 64-token blocks, each with its own U and k-step count.  Per step of 64
// hidden columns:
//   * B step = W_down[64 rows, 256 columns], copied global -> LDS with direct loads one step
//     ahead (double buffer), the rows of every block's U gathered from it by the transposing
//     LDS read (ds_read_b64_tr_b16 takes one row address per lane);
//   * A step = 256 x 64 hidden values, double-buffered: each wave clears its 32 token rows
//     of the next step's buffer and writes the next step's stored values at their positions
//     (a per-(block, step) column -> position table in LDS: the identity when dense);
//     padding slots go to one dummy word.  Backup slices are written the same way.
//   * Per (block, step) tables (column -> position, position -> W_down row, k-step count)
//     are built two steps ahead by one wave of the block from the column unions, in a ring
//     of three; the barrier at the top of each step publishes them with A and B.
//   * Waves 0-3 write the next A step before their MFMAs, waves 4-7 after, so that the two
//     waves sharing a SIMD alternate between the vector/LDS work and the matrix core; the
//     writes skip the slot positions that are padding in every row of the wave.
// With few workgroups (small T) the tile range is split into S parts, one per workgroup
// group; each part's fp32 sums go to the workspace and down_reduce_kernel adds the parts in
// order into y.  When the layer's stored-nonzero count (the sum of the per-block counts) is
// at most `thr` another kernel takes the layer and every workgroup here returns at once
// (blk_nnz == nullptr: this kernel runs).
#include <algorithm>

#include "sffn_common.hpp"

namespace sffn {

typedef __bf16 bf16x8_u __attribute__((ext_vector_type(8)));
typedef short short4_u __attribute__((ext_vector_type(4)));
typedef short short8_u __attribute__((ext_vector_type(8)));
typedef float floatx16_u __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_vptr_u;
typedef __attribute__((address_space(3))) short4_u* lds_s4ptr_u;

constexpr int DU_BM = 256;  // tokens per workgroup
constexpr int DU_BN = 256;  // output columns per workgroup
constexpr int DU_KC = 64;   // hidden columns per contraction step
constexpr int DU_NW = 8;    // waves per workgroup: 2 along the tokens x 4 along the columns
constexpr int DU_DENSE = 0x80;  // k-step-count flag: the step is contracted densely

template <int K, int W>
__global__ __launch_bounds__(64 * DU_NW) __attribute__((amdgpu_waves_per_eu(DU_NW / 4, DU_NW / 4))) void
down_union_kernel(Dims d, const uint16_t* __restrict__ counts, const uint16_t* __restrict__ vals,
                  const uint8_t* __restrict__ cols, const uint16_t* __restrict__ bk_vals,
                  const int32_t* __restrict__ grp_first, const uint32_t* __restrict__ umask,
                  const uint16_t* __restrict__ Wd, uint16_t* __restrict__ y,
                  float* __restrict__ dpart, int S, const int32_t* __restrict__ blk_nnz,
                  long long thr) {
  constexpr int KC = DU_KC;
  constexpr int NCH = K / KC;          // steps per tile
  constexpr int KW = K / 32;           // column-union words per (tile, group)
  constexpr int U = W / 8;             // 8-slot units per tile-row
  constexpr int AROW = KC * 2;         // 128 B: one A row
  constexpr int ABUF = DU_BM * AROW;   // 32 KB: one A buffer
  constexpr int BROW = DU_BN * 2;      // 512 B: one B row
  constexpr int BBUF = KC * BROW;      // 32 KB: one B buffer
  constexpr int NW = DU_NW;
  constexpr int RW = DU_BM / NW;       // A rows each wave writes (one 32-token group)
  constexpr int NWC = NW / 2;          // waves along the columns
  constexpr int WN = DU_BN / NWC;      // output columns per wave
  constexpr int NJ = WN / 32;          // 32-column MFMA blocks per wave
  constexpr int UL = RW * U / 64;      // 8-slot units per lane
  constexpr int NB = DU_BM / 64;       // 64-token blocks per workgroup
  static_assert(RW == 32 && U % 2 == 0, "a lane owns one row's slot groups l/32, l/32 + 2, ..");
  __shared__ __attribute__((aligned(16))) unsigned char sA[2 * ABUF + 256];
  __shared__ __attribute__((aligned(16))) unsigned char sB0[BBUF];
  __shared__ __attribute__((aligned(16))) unsigned char sB1[BBUF];
  __shared__ __attribute__((aligned(16))) uint8_t sPos[NW][64];     // overflowing rows per wave
  __shared__ __attribute__((aligned(16))) uint8_t sColPos[3][NB][64];  // column -> position
  __shared__ __attribute__((aligned(16))) uint8_t sRowOf[3][NB][64];   // position -> row (permuted)
  __shared__ int sNks[3][NB];  // k-steps of (ring slot, block), | DU_DENSE when dense

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = wave / NWC, wc = wave % NWC;  // MFMA tile: tokens 128wt.., columns WN wc..
  const int T = d.T;
  const int nd = (d.D + DU_BN - 1) / DU_BN;
  const int ntb = (T + DU_BM - 1) / DU_BM;
  const int total = nd * ntb * S;
  const int per_xcd = (total + 7) / 8;
  const int P = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (P >= total) return;
  const int split = P / (nd * ntb);
  const int Pl = P - split * nd * ntb;
  const int tb = Pl / nd;
  if (blk_nnz != nullptr && layer_nnz(blk_nnz, ntb) <= thr) return;  // another kernel's layer
  const int dchunk = Pl - tb * nd;
  constexpr int TQ = NCH == 1 ? 2 : 1;
  const int nunits = d.nt / TQ;
  const int k_lo = split * nunits / S * TQ;
  const int k_hi = split + 1 == S ? d.nt : (split + 1) * nunits / S * TQ;
  const int d0 = dchunk * DU_BN;
  const bool active = d0 + WN * wc < d.D;
  const int t0 = tb * DU_BM;
  const int tw = t0 + wave * RW;  // first token of the rows this wave writes into A
  const int ugw = wave / 2;       // 64-token block of the rows this wave writes
  const uint32_t trash = 2 * ABUF;
  uint8_t* const pos = sPos[wave];
  const int c_lo = k_lo * NCH, c_hi = k_hi * NCH;  // this part's steps
  auto ring = [&](int ci) __attribute__((always_inline)) -> int { return (ci - c_lo) % 3; };

  // ---- per-(block, step) tables from the column unions.  Wave 2b builds block b's tables of
  // step ci: lane = column of the step.  Positions of the compacted form are stored permuted
  // so that the eight rows one lane needs in a step (positions 16 kk + 8 h + 4 q + l, kk <
  // 4, q < 2, for its fixed h, l) are eight consecutive bytes: index (4 h + l) * 8 + 2 kk + q.
  auto perm_idx = [](int p) __attribute__((always_inline)) -> int {
    const int kk = p >> 4, rem = p & 15;
    return ((((rem >> 3) << 2) | (rem & 3)) << 3) + 2 * kk + ((rem >> 2) & 1);
  };
  auto build_tables = [&](int ci) __attribute__((always_inline)) {
    if ((wave & 1) != 0 || ci >= c_hi) return;
    const int b = wave / 2;
    const int k = ci / NCH, c = ci % NCH;
    const int g0 = (t0 + 64 * b) / GROUP;
    uint64_t m = 0;
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const int g = g0 + gg;
      if (g < d.ng) {
        const uint32_t* u = umask + ((size_t)k * d.ng + g) * KW + 2 * c;
        m |= (uint64_t)ld_uniform(u) | ((uint64_t)ld_uniform(u + 1) << 32);
      }
    }
    const int cnt = __builtin_popcountll(m);
    const int r = ring(ci);
    if (cnt > 48) {
      sColPos[r][b][lane] = (uint8_t)lane;
      sRowOf[r][b][perm_idx(lane)] = (uint8_t)lane;
      if (lane == 0) sNks[r][b] = 4 | DU_DENSE;
    } else {
      const int rk = mbcnt64(m);
      sColPos[r][b][lane] = (uint8_t)rk;
      if (lane >= cnt) sRowOf[r][b][perm_idx(lane)] = 0;  // padding positions: any finite row
      if ((m >> lane) & 1) sRowOf[r][b][perm_idx(rk)] = (uint8_t)lane;
      if (lane == 0) sNks[r][b] = (cnt + 15) >> 4;
    }
  };

  // ---- B step -> LDS (dense: all 64 rows of the step; the blocks gather their rows at the
  // fragment reads).  Row r (512 B) keeps 16-byte piece c at c ^ (4*(r&3)).
  const int b_hl = lane >> 5;
  int b_col = d0 + ((lane & 31) ^ (4 * (2 * (wave & 1) + b_hl))) * 8;
  b_col = b_col < d.D ? b_col : d0;  // columns past D (half-wide chunk) are never read
  const uint32_t b_off = (uint32_t)(b_hl * d.D + b_col);
  auto issue_B = [&](int ci, unsigned char* sB) __attribute__((always_inline)) {
    const int row0 = ci * KC;
#pragma unroll
    for (int q = 0; q < BBUF / 1024 / NW; ++q) {
      const int ins = q * NW + wave;
      const uint16_t* src = Wd + (size_t)(row0 + 2 * ins) * d.D;
      __builtin_amdgcn_global_load_lds(src + b_off, (lds_vptr_u)(sB + ins * 1024), 16, 0, 0);
    }
  };

  // ---- TwELL units of tile k for this wave's rows (as the dense matrix-core kernel)
  uint4 uv[UL];
  uint2 uc[UL];
  uint32_t cnt = 0;
  auto load_units = [&](int k) __attribute__((always_inline)) {
    const size_t row_base = (size_t)k * T;
#pragma unroll
    for (int j = 0; j < UL; ++j) {
      const int tok = tw + (lane & 31);
      const int tk = tok < T ? tok : T - 1;
      const uint32_t m = tok < T ? 0xFFFFFFFFu : 0u;
      const size_t e0 = (row_base + tk) * W + 8 * ((lane >> 5) + 2 * j);
      const uint4 v = *reinterpret_cast<const uint4*>(vals + e0);
      uv[j] = make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
      uc[j] = *reinterpret_cast<const uint2*>(cols + e0);
    }
    const int t = tw + lane;
    const uint32_t m = (t < T && lane < RW) ? 0xFFFFu : 0u;
    cnt = (uint32_t)counts[row_base + (t < T ? t : T - 1)] & m;
  };

  // A rows are 128 B; 16-byte piece p of block row R sits at p ^ ((R >> 1) & 7).
  auto a_addr = [&](int buf, uint32_t r, uint32_t cc) __attribute__((always_inline)) -> uint32_t {
    return buf * ABUF + (wave * RW + r) * AROW + ((cc ^ (((r >> 1) & 7) << 3)) << 1);
  };

  // ---- write step c (of the tile) of the units into A buffer `buf` at the positions of
  // table `tab` (the identity when dense).  Slot 8 (h + 2 j) + e of a row is in unit j of the
  // lanes of half h; slots at or above the largest main count of the wave's rows (mmax) are
  // padding in every row and are skipped (a wave-uniform test), so the work follows the
  // stored nonzeros rather than the ELL width.
  auto build = [&](int c, int buf, const uint8_t* tab, int mmax) __attribute__((always_inline)) {
    const uint32_t r = (uint32_t)(lane & 31);
#pragma unroll
    for (int j = 0; j < UL; ++j) {
      if (16 * j >= mmax) break;
      const uint32_t vv[4] = {uv[j].x, uv[j].y, uv[j].z, uv[j].w};
      const uint32_t cw[2] = {uc[j].x, uc[j].y};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (16 * j + e >= mmax) break;
        const uint32_t col = (cw[e >> 2] >> (8 * (e & 3))) & 0xFFu;
        const uint32_t word = vv[e >> 1];
        const bool nz = (e & 1) ? (word > 0xFFFFu) : ((word & 0xFFFFu) != 0u);
        bool in = true;
        if constexpr (NCH > 1) in = (col >> 6) == (uint32_t)c;
        const uint32_t p = tab[col & (KC - 1)];
        const uint32_t addr = (nz && in) ? a_addr(buf, r, p) : trash;
        const uint16_t h = (e & 1) ? (uint16_t)(word >> 16) : (uint16_t)word;
        *reinterpret_cast<uint16_t*>(sA + addr) = h;
      }
    }
  };
  // largest main-slot count min(count, W) of the wave's rows (the loaded tile's counts)
  auto max_main = [&]() __attribute__((always_inline)) -> int {
    int m = (int)(cnt < (uint32_t)W ? cnt : (uint32_t)W);
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
      const int v = __shfl_xor(m, o);
      m = v > m ? v : m;
    }
    return __builtin_amdgcn_readfirstlane(m);
  };

  // ---- backup slices of the wave's overflowing rows (as the dense matrix-core kernel: only
  // the 4-row groups that hold one of the wave's rows)
  uint2 bkv[4];
  uint32_t bkr[4];
  int bk_e0 = 0, bk_n = 0;
  auto bk_load = [&](int k, int c, int first) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = first + 4 * q + (lane >> 4);
      bkv[q] = make_uint2(0, 0);
      bkr[q] = 0;
      if (first + 4 * q >= bk_n) continue;  // wave-uniform
      if (rr < bk_n && bk_e0 + rr < d.cap) {
        bkr[q] = pos[rr];
        bkv[q] = *reinterpret_cast<const uint2*>(bk_vals + (size_t)(bk_e0 + rr) * K + c * KC +
                                                 4 * (lane & 15));
      }
    }
  };
  auto bk_write = [&](int buf, const uint8_t* tab, int first) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (first + 4 * q >= bk_n) continue;  // wave-uniform
      const uint32_t w2[2] = {bkv[q].x, bkv[q].y};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t word = w2[e >> 1];
        const uint16_t h = (e & 1) ? (uint16_t)(word >> 16) : (uint16_t)word;
        const uint32_t cc = 4 * (lane & 15) + e;
        const uint32_t addr = h != 0 ? a_addr(buf, bkr[q], tab[cc]) : trash;
        *reinterpret_cast<uint16_t*>(sA + addr) = h;
      }
    }
  };
  auto bk_begin = [&](uint64_t ov, int e0, int k, int c) __attribute__((always_inline)) {
    bk_n = __builtin_popcountll(ov);
    if (bk_n == 0) return;
    if ((ov >> lane) & 1) pos[mbcnt64(ov)] = (uint8_t)lane;
    bk_e0 = e0;
    bk_load(k, c, 0);
  };
  auto first_entry = [&](int k) __attribute__((always_inline)) -> int {
    return ld_uniform(grp_first + (k < d.nt ? k : d.nt - 1) * d.ng + tw / GROUP);
  };
  // writes the backup rows of step ci (positions from the table of this wave's block)
  auto bk_finish = [&](int ci, int buf) __attribute__((always_inline)) {
    if (bk_n == 0) return;
    const uint8_t* tab = sColPos[ring(ci)][ugw];
    const int k = ci / NCH, c = ci % NCH;
    bk_write(buf, tab, 0);
    for (int first = 16; first < bk_n; first += 16) {
      bk_load(k, c, first);
      bk_write(buf, tab, first);
    }
  };

  auto clear_a = [&](int buf) __attribute__((always_inline)) {
    uint4* p = reinterpret_cast<uint4*>(sA + buf * ABUF + wave * RW * AROW);
#pragma unroll
    for (int q = 0; q < RW * AROW / 1024; ++q) p[q * 64 + lane] = make_uint4(0, 0, 0, 0);
  };

  // ---- fragments
  const int l32 = lane & 31, lh = lane >> 5;
  const int g16 = lane >> 4, li = lane & 15;
  auto a_frag = [&](int buf, int i, int kk) __attribute__((always_inline)) -> bf16x8_u {
    const int R = 128 * wt + 32 * i + l32;
    const int ch = kk * 2 + lh;
    return __builtin_bit_cast(bf16x8_u, *reinterpret_cast<const uint4*>(
                                            sA + buf * ABUF + R * AROW + ((ch ^ ((R >> 1) & 7)) << 4)));
  };
  // B fragment of k-step kk: lane L of a 16-lane group reads the row of position
  // 16 kk + 8 (g16 >> 1) + 4 q + L/4 (byte 2 kk + q of `rows8`), columns c0 + 4(L%4) .. +3
  auto b_frag = [&](const unsigned char* sB, int j, int kk, uint64_t rows8) __attribute__((always_inline)) -> bf16x8_u {
    const int c0 = WN * wc + 32 * j + 16 * (g16 & 1);
    const int col = c0 + 4 * (li & 3);
    short4_u h[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = (int)((rows8 >> (8 * (2 * kk + q))) & 0xFFu);
      const int off = r * BROW + ((((col >> 3) ^ (4 * (r & 3))) << 4) | ((col & 7) << 1));
      h[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4ptr_u)(sB + off));
    }
    const short8_u v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
    return __builtin_bit_cast(bf16x8_u, v);
  };

  floatx16_u acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // the lane's (h, l) in the permuted position order: byte 2 kk + q of its 8 row bytes is
  // the W_down row of position 16 kk + 8 h + 4 q + l
  const int lkey = ((g16 >> 1) << 2) | (li >> 2);

  // MFMAs of step ci for the wave's two 64-token blocks (row blocks 2g, 2g + 1), each over
  // its own k-step count
  auto mfma_step = [&](int ci, int cb, const unsigned char* sBc) __attribute__((always_inline)) {
    const int r = ring(ci);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int b = 2 * wt + g;
      const int nks = __builtin_amdgcn_readfirstlane(sNks[r][b]) & 7;
      const uint64_t rows8 = *reinterpret_cast<const uint64_t*>(&sRowOf[r][b][lkey * 8]);
      for (int kk = 0; kk < nks; ++kk) {
        bf16x8_u fa[2], fb[NJ];
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) fa[ii] = a_frag(cb, 2 * g + ii, kk);
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) fb[jj] = b_frag(sBc, jj, kk, rows8);
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
          for (int jj = 0; jj < NJ; ++jj)
            acc[2 * g + ii][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ii], fb[jj],
                                                                          acc[2 * g + ii][jj], 0, 0, 0);
      }
    }
  };

  // ---- prologue: tables of the first two steps, then A(c_lo) written, B(c_lo) in flight
  build_tables(c_lo);
  build_tables(c_lo + 1);
  issue_B(c_lo, sB0);
  load_units(k_lo);
  clear_a(0);
  int mmax = max_main();
  __syncthreads();  // tables of c_lo, c_lo + 1
  build(0, 0, sColPos[ring(c_lo)][ugw], mmax);
  {
    const uint64_t ov = ballot64(cnt > (uint32_t)W);
    if (NCH == 1) load_units(k_lo + 1 < d.nt ? k_lo + 1 : k_lo);
    bk_begin(ov, first_entry(k_lo), k_lo, 0);
    bk_finish(c_lo, 0);
  }
  int e0_next = first_entry((c_lo + 1) / NCH);

  // step ci: MFMAs of step ci (A and B buffers ci&1) and the A rows of step ci+1 written
  // into the other A buffer (the last step rebuilds a step nobody reads).  Waves 0-3 write
  // before their MFMAs and waves 4-7 after, so the two waves sharing a SIMD alternate
  // between the vector/LDS work and the matrix core.
  auto step = [&](int ci, int cb, unsigned char* sBc, unsigned char* sBn, bool load_next)
      __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): B(ci), the units, backup rows landed
    if (ci > c_lo) bk_finish(ci, cb);     // backup rows of step ci (loaded last step)
    mmax = max_main();                    // of the units the writes of this step use
    __syncthreads();                      // A(ci), B(ci), tables of ci+1 complete
    const int cn = ci + 1 < c_hi ? ci + 1 : c_hi - 1;
    const int c_next = cn % NCH;
    const uint64_t ov = ballot64(cnt > (uint32_t)W);
    const int e0 = e0_next;
    e0_next = first_entry((ci + 2) / NCH);
    bk_begin(ov, e0, cn / NCH, c_next);
    build_tables(ci + 2);
#pragma nounroll
    for (int ph = 0; ph < 2; ++ph) {
      if ((ph == 0) == (wave < 4)) {
        issue_B(cn, sBn);
        clear_a(cb ^ 1);
        build(c_next, cb ^ 1, sColPos[ring(cn)][ugw], mmax);
        if (load_next) {
          const int kt = (cn + 1) / NCH;
          load_units(kt < d.nt ? kt : d.nt - 1);
        }
      } else {
        mfma_step(ci, cb, sBc);
      }
    }
  };
  constexpr int UF = NCH < 2 ? 2 : NCH;  // steps per unrolled iteration ((c_hi - c_lo) % UF == 0)
  for (int base = c_lo; base < c_hi; base += UF) {
#pragma unroll
    for (int s2 = 0; s2 < UF; ++s2)
      step(base + s2, s2 & 1, (s2 & 1) ? sB1 : sB0, (s2 & 1) ? sB0 : sB1, (s2 + 2) % NCH == 0);
  }

  // ---- y (bf16), or this part's fp32 sums: C[m = token][n = column]; lane: column l32,
  // rows 8(r/4) + 4lh + r%4
  if (!active) return;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = t0 + 128 * wt + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
        const size_t o = (size_t)t * d.D + d0 + WN * wc + 32 * j + l32;
        if (t < T) {
          if (S == 1)
            y[o] = f32_to_bf16(acc[i][j][r]);
          else
            dpart[(size_t)split * T * d.D + o] = acc[i][j][r];
        }
      }
}

template <int K, int W>
static hipError_t launch_du_t(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                              const void* Wd, void* y, const int32_t* blk_nnz, long long thr,
                              hipStream_t s) {
  const int nd = (d.D + DU_BN - 1) / DU_BN;
  const int ntb = (d.T + DU_BM - 1) / DU_BM;
  const int S = down_split(d);
  const int total = nd * ntb * S;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL((down_union_kernel<K, W>), dim3(8 * per_xcd), dim3(64 * DU_NW), 0, s, d,
                     b.counts, static_cast<const uint16_t*>(b.vals), b.cols,
                     static_cast<const uint16_t*>(b.bk_vals), ws.grp_first, ws.umask,
                     static_cast<const uint16_t*>(Wd), static_cast<uint16_t*>(y), ws.dpart, S,
                     blk_nnz, thr);
  if (S > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_down_reduce(d, ws, y, S, blk_nnz, thr, s);
  }
  return hipGetLastError();
}

template <int K>
static hipError_t launch_du_k(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                              const void* Wd, void* y, const int32_t* blk_nnz, long long thr,
                              hipStream_t s) {
  switch (d.W) {
    case 16: return launch_du_t<K, 16>(d, b, ws, Wd, y, blk_nnz, thr, s);
    case 32: return launch_du_t<K, 32>(d, b, ws, Wd, y, blk_nnz, thr, s);
    case 48: return launch_du_t<K, 48>(d, b, ws, Wd, y, blk_nnz, thr, s);
    case 64: return launch_du_t<K, 64>(d, b, ws, Wd, y, blk_nnz, thr, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_down_union(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                             const void* Wd, void* y, const int32_t* blk_nnz, long long thr,
                             hipStream_t s) {
  if (!down_mfma_supported(d)) return hipErrorInvalidValue;
  if (d.K == 64) return launch_du_k<64>(d, b, ws, Wd, y, blk_nnz, thr, s);
  if (d.K == 128) return launch_du_k<128>(d, b, ws, Wd, y, blk_nnz, thr, s);
  return launch_du_k<256>(d, b, ws, Wd, y, blk_nnz, thr, s);
}

}  // namespace sffn
