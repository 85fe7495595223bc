// Down-projection over a TwELL activation on the matrix cores (gfx950), for token blocks
// dense enough that a dense contraction of the rebuilt tiles beats the vector gather (the
// bf16 MFMA rate is ~16x the vector rate, so the crossover sits well below 1% density).
//
//   y[t, :] = sum_k  H_k[t, :] W_down[k*K : (k+1)*K, :]
//
// where H_k, tile k of the activations, is rebuilt in LDS from its TwELL rows: the main
// slots (value, local column) plus, for overflowing tile-rows, the dense backup slice
// (upppp.jp TwELL article of 2026-05-11, section "What TwELL and the custom CUDA kernels
// solve": tiles aligned with tiled matrix-multiply execution, sparse main part plus a few
// dense backups).
//
// Workgroup = 256 tokens x 256 output columns, 8 waves in a 2 x 4 grid (two per SIMD, so
// one wave's A writes run while the other's MFMAs keep the matrix core busy); each wave
// computes 128 tokens x 64 columns with v_mfma_f32_32x32x16_bf16 (A = hidden rows,
// B = W_down; 128 fp32 accumulators per lane).  The contraction runs in steps of 64 hidden
// columns:
//   * B step = W_down[64 rows, 256 columns], copied global -> LDS with direct loads one
//     step ahead (double buffer); B fragments come straight out of its row-major layout
//     through ds_read_b64_tr_b16.
//   * A step = 256 x 64 hidden values, double-buffered: while the MFMAs of step c read one
//     buffer, each wave clears its 32 token rows of the other and writes step c+1's
//     nonzeros there, from TwELL data prefetched into registers as 8-slot units (coalesced
//     16 B value + 8 B column loads).  Padding slots hold value 0 and go to a dummy word,
//     so these writes need no branch, and the step body between barriers is one basic
//     block in which the A writes are interleaved with the MFMAs (one MFMA, then a few
//     vector and LDS instructions in its shadow).  Backup slices of a wave's overflowing
//     rows are loaded (up to 16 rows, 4 rows per load) at the start of the step and written
//     at the start of the next, before its barrier; their first entry comes from the
//     per-(tile, 32-token group) offsets of the ordering pass.  The barrier at the top of
//     each step publishes the A and B buffers.
// With few workgroups (small T) the tile range is split into S parts, one per workgroup
// group; each part's fp32 sums go to the workspace and down_reduce_kernel adds the parts in
// order into y.
// When the layer's stored-nonzero count (the sum of the per-block counts) is at most `thr`
// the gather kernel takes the layer and every workgroup here (and the reduce) returns at
// once (blk_nnz == nullptr: this kernel runs).  Workgroup 0 of a running launch records the
// kernel the count selects through `hint`.
#include <algorithm>

#include "sffn_common.hpp"

namespace sffn {

typedef __bf16 bf16x8_m __attribute__((ext_vector_type(8)));
typedef short short4_m __attribute__((ext_vector_type(4)));
typedef short short8_m __attribute__((ext_vector_type(8)));
typedef float floatx16_m __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_vptr;
typedef __attribute__((address_space(3))) short4_m* lds_s4ptr;

constexpr int DM_BM = 256;  // tokens per workgroup
constexpr int DM_BN = 256;  // output columns per workgroup
constexpr int DM_KC = 64;   // hidden columns per contraction step
constexpr int DM_NW = 8;    // waves per workgroup: 2 along the tokens x DM_NW / 2 along the columns

template <int K, int W>
__global__ __launch_bounds__(64 * DM_NW) __attribute__((amdgpu_waves_per_eu(DM_NW / 4, DM_NW / 4))) void down_mfma_kernel(
    Dims d, const uint16_t* __restrict__ counts, const uint16_t* __restrict__ vals,
    const uint8_t* __restrict__ cols, const uint16_t* __restrict__ bk_vals,
    const int32_t* __restrict__ grp_first, const uint16_t* __restrict__ Wd,
    uint16_t* __restrict__ y, float* __restrict__ dpart, int S, const int32_t* __restrict__ blk_nnz,
    long long thr, DownHint hint) {
  constexpr int KC = DM_KC;
  constexpr int NCH = K / KC;          // steps per tile
  constexpr int U = W / 8;             // 8-slot units per tile-row
  constexpr int NKK = KC / 16;         // MFMA k-steps per step
  constexpr int AROW = KC * 2;         // 128 B: one A row
  constexpr int ABUF = DM_BM * AROW;   // 32 KB: one A buffer
  constexpr int BROW = DM_BN * 2;      // 512 B: one B row
  constexpr int BBUF = KC * BROW;      // 32 KB: one B buffer
  constexpr int NW = DM_NW;
  constexpr int RW = DM_BM / NW;       // A rows each wave writes
  constexpr int NWC = NW / 2;          // waves along the columns
  constexpr int WN = DM_BN / NWC;      // output columns per wave
  constexpr int NJ = WN / 32;          // 32-column MFMA blocks per wave
  constexpr int UL = RW * U / 64;      // 8-slot units per lane
  static_assert(RW == 32 && U % 2 == 0, "a lane owns one row's slot groups l/32, l/32 + 2, ..");
  // A buffers, then 256 B holding the dummy word that padding writes go to; all A writes
  // address this one array, so the compiler sees they never touch the B buffers filled by
  // direct loads (and need not wait for those)
  __shared__ __attribute__((aligned(16))) unsigned char sA[2 * ABUF + 256];
  __shared__ __attribute__((aligned(16))) unsigned char sB0[BBUF];
  __shared__ __attribute__((aligned(16))) unsigned char sB1[BBUF];
  __shared__ __attribute__((aligned(16))) uint8_t sPos[NW][64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = wave / NWC, wc = wave % NWC;  // MFMA tile: tokens 128wt.., columns WN wc..
  const int T = d.T;
  const int nd = (d.D + DM_BN - 1) / DM_BN;
  const int ntb = (T + DM_BM - 1) / DM_BM;
  const int total = nd * ntb * S;
  const int per_xcd = (total + 7) / 8;
  const int P = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (P >= total) return;
  // split-major, then token-block-major: the workgroups an XCD runs together share a tile
  // range, token blocks (TwELL reads) and column chunks (W_down reads) in its L2
  const int split = P / (nd * ntb);
  const int Pl = P - split * nd * ntb;
  const int tb = Pl / nd;
  if (blk_nnz != nullptr && layer_nnz(blk_nnz, ntb) <= thr) return;  // the gather kernel's layer
  note_choice(hint, ntb, blockIdx.x == 0);
  const int dchunk = Pl - tb * nd;
  // tiles [k_lo, k_hi) of this part (in pairs for 64-column tiles, whose one-step tiles run
  // two per unrolled iteration)
  constexpr int TQ = NCH == 1 ? 2 : 1;
  const int nunits = d.nt / TQ;
  const int k_lo = split * nunits / S * TQ;
  const int k_hi = split + 1 == S ? d.nt : (split + 1) * nunits / S * TQ;
  const int d0 = dchunk * DM_BN;
  const bool active = d0 + WN * wc < d.D;  // D % 256 == 128: the last chunk is half wide
  const int t0 = tb * DM_BM;
  const int tw = t0 + wave * RW;  // first token of the rows this wave writes into A
  // byte offset in sA of the dummy word every discarded write goes to (one word for all
  // lanes: writes to one address do not add bank conflicts to the real writes beside them)
  const uint32_t trash = 2 * ABUF;
  uint8_t* const pos = sPos[wave];

  // ---- B step -> LDS.  Row r (512 B) keeps 16-byte piece c at c ^ (4*(r&3)), so the four
  // rows (4 pieces each) that one half-wave of a transposed read touches land on 16
  // different 4-bank groups, i.e. all 64 banks.  Load q of a wave is
  // 1 KB (two rows: 2 ins + lane/32, ins = NW q + wave), so r & 3 = 2 (wave & 1) + lane/32
  // for every load and the lane's part of the offset is the same each time.
  const int b_hl = lane >> 5;
  int b_col = d0 + ((lane & 31) ^ (4 * (2 * (wave & 1) + b_hl))) * 8;
  b_col = b_col < d.D ? b_col : d0;  // columns past D (half-wide chunk) are never read
  const uint32_t b_off = (uint32_t)(b_hl * d.D + b_col);
  auto issue_B = [&](int ci, unsigned char* sB) __attribute__((always_inline)) {
    const int row0 = ci * KC;  // step ci = rows [ci*KC, +KC) of W_down
#pragma unroll
    for (int q = 0; q < BBUF / 1024 / NW; ++q) {
      const int ins = q * NW + wave;
      const uint16_t* src = Wd + (size_t)(row0 + 2 * ins) * d.D;
      __builtin_amdgcn_global_load_lds(src + b_off, (lds_vptr)(sB + ins * 1024), 16, 0, 0);
    }
  };

  // ---- TwELL units of tile k for this wave's rows: unit j of lane l holds slots 8 g .. +7,
  // g = l / 32 + 2 j, of token tw + l % 32 (a lane's row is the same for all its units; the
  // wider ELL widths then need no register spills).  cnt = count of token tw + lane (lanes
  // < RW).
  uint4 uv[UL];
  uint2 uc[UL];
  uint32_t cnt = 0;
  auto load_units = [&](int k) __attribute__((always_inline)) {
    // addresses are clamped into the buffers and rows past T masked to zero with an AND
    // (a select on a loaded value would be turned into a branch around the load)
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

  // A rows are 128 B; 16-byte piece p of block row R sits at p ^ ((R >> 1) & 7), so the
  // 16 consecutive rows of one fragment read (alternating bank halves) hit distinct banks.
  // Byte offset in sA of (this wave's row r, hidden column cc) in A buffer `buf`:
  auto a_addr = [&](int buf, uint32_t r, uint32_t cc) __attribute__((always_inline)) -> uint32_t {
    return buf * ABUF + (wave * RW + r) * AROW + ((cc ^ (((r >> 1) & 7) << 3)) << 1);
  };

  // ---- write step c (of the tile) of the units into A buffer `buf`; the 8 UL slots of a
  // lane are split evenly into four parts (slot q = 8j + e in part 4q / (8 UL)) so the
  // writes spread over the four MFMA k-steps
  auto build_part = [&](int part, int c, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < UL; ++j) {
      const uint32_t r = (uint32_t)(lane & 31);
      const uint32_t vv[4] = {uv[j].x, uv[j].y, uv[j].z, uv[j].w};
      const uint32_t cw[2] = {uc[j].x, uc[j].y};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if ((4 * (8 * j + e)) / (8 * UL) != part) continue;
        const uint32_t col = (cw[e >> 2] >> (8 * (e & 3))) & 0xFFu;
        const uint32_t word = vv[e >> 1];
        const bool nz = (e & 1) ? (word > 0xFFFFu) : ((word & 0xFFFFu) != 0u);
        bool in = true;
        if constexpr (NCH > 1) in = (col >> 6) == (uint32_t)c;
        const uint32_t addr = (nz && in) ? a_addr(buf, r, col & (KC - 1)) : trash;
        const uint16_t h = (e & 1) ? (uint16_t)(word >> 16) : (uint16_t)word;
        *reinterpret_cast<uint16_t*>(sA + addr) = h;
      }
    }
  };

  // ---- backup slices of the wave's overflowing rows (bit b of ov = token tw + b); they are
  // consecutive entries from the first entry of the wave's first 32-token group on.
  // Batches of 16 rows: lane reads 4 columns (8 B) of row 4q + lane/16 of the batch.
  uint2 bkv[4];
  uint32_t bkr[4];
  int bk_e0 = 0, bk_n = 0;
  // only the 4-row groups that hold one of the wave's bk_n rows are loaded and written (a
  // wave usually has one to three: the rest of a batch of 16 would only delay the barrier)
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
  auto bk_write = [&](int buf, int first) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (first + 4 * q >= bk_n) continue;  // wave-uniform
      const uint32_t w2[2] = {bkv[q].x, bkv[q].y};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t word = w2[e >> 1];
        const uint16_t h = (e & 1) ? (uint16_t)(word >> 16) : (uint16_t)word;
        const uint32_t cc = 4 * (lane & 15) + e;
        const uint32_t addr = h != 0 ? a_addr(buf, bkr[q], cc) : trash;
        *reinterpret_cast<uint16_t*>(sA + addr) = h;
      }
    }
  };
  // positions of the overflowing rows, entry of the first; loads the first batch
  auto bk_begin = [&](uint64_t ov, int e0, int k, int c) __attribute__((always_inline)) {
    bk_n = __builtin_popcountll(ov);
    if (bk_n == 0) return;
    if ((ov >> lane) & 1) pos[mbcnt64(ov)] = (uint8_t)lane;
    bk_e0 = e0;
    bk_load(k, c, 0);
  };
  // first backup entry of this wave's rows in tile k (scalar load, issued a step ahead)
  auto first_entry = [&](int k) __attribute__((always_inline)) -> int {
    return ld_uniform(grp_first + (k < d.nt ? k : d.nt - 1) * d.ng + tw / GROUP);
  };
  // writes the first batch, then any further batches
  auto bk_finish = [&](int k, int c, int buf) __attribute__((always_inline)) {
    if (bk_n == 0) return;
    bk_write(buf, 0);
    for (int first = 16; first < bk_n; first += 16) {
      bk_load(k, c, first);
      bk_write(buf, first);
    }
  };

  // ---- clear this wave's RW rows of A buffer `buf` (16 B per lane per store)
  auto clear_a = [&](int buf) __attribute__((always_inline)) {
    uint4* p = reinterpret_cast<uint4*>(sA + buf * ABUF + wave * RW * AROW);
#pragma unroll
    for (int q = 0; q < RW * AROW / 1024; ++q) p[q * 64 + lane] = make_uint4(0, 0, 0, 0);
  };

  // ---- fragments
  const int l32 = lane & 31, lh = lane >> 5;
  const int g16 = lane >> 4, li = lane & 15;
  auto a_frag = [&](int buf, int i, int kk) __attribute__((always_inline)) -> bf16x8_m {
    const int R = 128 * wt + 32 * i + l32;  // block row; k = 16kk + 8lh ..
    const int ch = kk * 2 + lh;
    return __builtin_bit_cast(bf16x8_m, *reinterpret_cast<const uint4*>(
                                            sA + buf * ABUF + R * AROW + ((ch ^ ((R >> 1) & 7)) << 4)));
  };
  auto b_frag = [&](const unsigned char* sB, int j, int kk) __attribute__((always_inline)) -> bf16x8_m {
    // lane L of a 16-lane group reads row r0 + L/4, columns c0 + 4(L%4) .. +3; lane i then
    // holds column c0 + i of rows r0 .. r0+3
    const int c0 = WN * wc + 32 * j + 16 * (g16 & 1);
    const int col = c0 + 4 * (li & 3);
    short4_m h[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = kk * 16 + 8 * (g16 >> 1) + 4 * q + (li >> 2);
      const int off = r * BROW + ((((col >> 3) ^ (4 * (r & 3))) << 4) | ((col & 7) << 1));
      h[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4ptr)(sB + off));
    }
    const short8_m v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
    return __builtin_bit_cast(bf16x8_m, v);
  };

  floatx16_m acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // ---- prologue: A(0) written, B(0) in flight, units of the step after it loaded
  const int c_lo = k_lo * NCH, c_hi = k_hi * NCH;  // this part's steps
  issue_B(c_lo, sB0);
  load_units(k_lo);
  clear_a(0);
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) build_part(pt, 0, 0);
  {
    const uint64_t ov = ballot64(cnt > (uint32_t)W);
    if (NCH == 1) load_units(k_lo + 1 < d.nt ? k_lo + 1 : k_lo);
    bk_begin(ov, first_entry(k_lo), k_lo, 0);
    bk_finish(k_lo, 0, 0);
  }
  int e0_next = first_entry((c_lo + 1) / NCH);  // first backup entry for the chunk the first step prepares

  // step ci: MFMAs of step ci (A and B buffers ci&1) while the A rows of step ci+1 are
  // written into the other A buffer.  The last step rebuilds a chunk nobody reads instead
  // of branching, so the whole body between the backup handling is one block: the A writes
  // (VALU + LDS) interleave with the MFMAs (sched_group_barrier below).  load_next: the
  // units of the tile after chunk ci+1 are fetched in this step (a compile-time pattern).
  auto step = [&](int ci, int cb, unsigned char* sBc, unsigned char* sBn, bool load_next)
      __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): B(ci), the units, backup rows landed
    if (ci > c_lo) bk_finish(ci / NCH, ci % NCH, cb);  // backup rows of chunk ci (loaded last step)
    __syncthreads();                     // A(ci), B(ci) complete; step ci-1's buffers free
    const int cn = ci + 1 < c_hi ? ci + 1 : c_hi - 1;
    const int c_next = cn % NCH;
    const uint64_t ov = ballot64(cnt > (uint32_t)W);
    const int e0 = e0_next;
    e0_next = first_entry((ci + 2) / NCH);  // for the next step, ready by then
    bk_begin(ov, e0, cn / NCH, c_next);  // overflowing rows of chunk cn: loads in flight until
                                     // the top of the next step writes them
    bf16x8_m fa[2][4], fb[2][NJ];
    auto load_frags = [&](int kk, bf16x8_m* a, bf16x8_m* b) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = a_frag(cb, i, kk);
#pragma unroll
      for (int j = 0; j < NJ; ++j) b[j] = b_frag(sBc, j, kk);
    };
    load_frags(0, fa[0], fb[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (kk + 1 < NKK) load_frags(kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
      if (kk == 0) {
        issue_B(cn, sBn);
        clear_a(cb ^ 1);
      }
      build_part(kk, c_next, cb ^ 1);
      if (kk == NKK - 1 && load_next) {
        const int kt = (cn + 1) / NCH;
        load_units(kt < d.nt ? kt : d.nt - 1);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][i], fb[kk & 1][j],
                                                              acc[i][j], 0, 0, 0);
      // one MFMA, then a few vector and LDS instructions in its shadow
#pragma unroll
      for (int m = 0; m < 4 * NJ; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x080, 2, 0);  // LDS
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM
      }
      __builtin_amdgcn_sched_barrier(0);
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

// y = bf16(sum over the S parts of the split kernel), parts added in order (deterministic).
__global__ __launch_bounds__(256) void down_reduce_kernel(Dims d, const float* __restrict__ part,
                                                          int S, uint16_t* __restrict__ y,
                                                          const int32_t* __restrict__ blk_nnz,
                                                          long long thr) {
  const int ntb = (d.T + DM_BM - 1) / DM_BM;
  if (blk_nnz != nullptr && layer_nnz(blk_nnz, ntb) <= thr) return;  // the gather kernel's layer
  const size_t n4 = (size_t)d.T * d.D / 4;
  const float4* p4 = reinterpret_cast<const float4*>(part);
  for (size_t q = (size_t)blockIdx.x * 256 + threadIdx.x; q < n4; q += (size_t)gridDim.x * 256) {
    // every part's load in flight before the first add (S <= DM_MAX_SPLIT)
    float4 v[DM_MAX_SPLIT];
#pragma unroll
    for (int sp = 0; sp < DM_MAX_SPLIT; ++sp)
      v[sp] = sp < S ? p4[(size_t)sp * n4 + q] : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 a = v[0];
#pragma unroll
    for (int sp = 1; sp < DM_MAX_SPLIT; ++sp) {
      if (sp < S) {
        a.x += v[sp].x;
        a.y += v[sp].y;
        a.z += v[sp].z;
        a.w += v[sp].w;
      }
    }
    const uint32_t lo = (uint32_t)f32_to_bf16(a.x) | ((uint32_t)f32_to_bf16(a.y) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(a.z) | ((uint32_t)f32_to_bf16(a.w) << 16);
    reinterpret_cast<uint2*>(y)[q] = make_uint2(lo, hi);
  }
}

template <int K, int W>
static hipError_t launch_dm_t(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                              const void* Wd, void* y, const int32_t* blk_nnz, long long thr,
                              hipStream_t s, const DownHint& hint) {
  const int nd = (d.D + DM_BN - 1) / DM_BN;
  const int ntb = (d.T + DM_BM - 1) / DM_BM;
  const int S = down_split(d);
  const int total = nd * ntb * S;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL((down_mfma_kernel<K, W>), dim3(8 * per_xcd), dim3(64 * DM_NW), 0, s, d, b.counts,
                     static_cast<const uint16_t*>(b.vals), b.cols,
                     static_cast<const uint16_t*>(b.bk_vals), ws.grp_first,
                     static_cast<const uint16_t*>(Wd), static_cast<uint16_t*>(y), ws.dpart, S,
                     blk_nnz, thr, hint);
  if (S > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_down_reduce(d, ws, y, S, blk_nnz, thr, s);
  }
  return hipGetLastError();
}

hipError_t launch_down_reduce(const Dims& d, const Workspace& ws, void* y, int S,
                              const int32_t* blk_nnz, long long thr, hipStream_t s) {
  if (S < 1 || S > DM_MAX_SPLIT) return hipErrorInvalidValue;  // down_split keeps S in range
  const size_t n4 = (size_t)d.T * d.D / 4;
  const int blocks = (int)std::min<size_t>((n4 + 255) / 256, 2048);
  hipLaunchKernelGGL(down_reduce_kernel, dim3(blocks), dim3(256), 0, s, d, ws.dpart, S,
                     static_cast<uint16_t*>(y), blk_nnz, thr);
  return hipGetLastError();
}

template <int K>
static hipError_t launch_dm_k(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                              const void* Wd, void* y, const int32_t* blk_nnz, long long thr,
                              hipStream_t s, const DownHint& hint) {
  switch (d.W) {
    case 16: return launch_dm_t<K, 16>(d, b, ws, Wd, y, blk_nnz, thr, s, hint);
    case 32: return launch_dm_t<K, 32>(d, b, ws, Wd, y, blk_nnz, thr, s, hint);
    case 48: return launch_dm_t<K, 48>(d, b, ws, Wd, y, blk_nnz, thr, s, hint);
    case 64: return launch_dm_t<K, 64>(d, b, ws, Wd, y, blk_nnz, thr, s, hint);
  }
  return hipErrorInvalidValue;
}

bool down_mfma_supported(const Dims& d) {
  return d.bf16 && (d.W == 16 || d.W == 32 || d.W == 48 || d.W == 64) && d.D % 128 == 0;
}

hipError_t launch_down_mfma(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                            const void* Wd, void* y, const int32_t* blk_nnz, long long thr,
                            hipStream_t s, const DownHint& hint) {
  if (!down_mfma_supported(d)) return hipErrorInvalidValue;
  if (d.K == 64) return launch_dm_k<64>(d, b, ws, Wd, y, blk_nnz, thr, s, hint);
  if (d.K == 128) return launch_dm_k<128>(d, b, ws, Wd, y, blk_nnz, thr, s, hint);
  return launch_dm_k<256>(d, b, ws, Wd, y, blk_nnz, thr, s, hint);
}

}  // namespace sffn
