// Down-projection over a TwELL activation on the 2:4 structured-sparse matrix cores of gfx950
// (v_smfmac_f32_32x32x32_bf16).
//
//   y[t, :] = sum_k  H_k[t, :] W_down[k*K : (k+1)*K, :]
//
// Only the stored nonzeros of H multiply W_down rows (upppp.jp TwELL article of 2026-05-11,
// section "What is the waste in LLM FFN layers"), and TwELL keeps each tile's nonzeros in
// column order (section "What TwELL and the custom CUDA kernels solve").  The sparse matrix
// instruction takes an A operand in which every group of four consecutive columns holds at
// most two values, stored as those two values plus a 2-bit column index each, and covers
// 32 columns in the time the dense instruction takes for 16.  A stored nonzero's place in
// that form follows from its rank among the stored nonzeros of its four-column group, which
// the column-ordered slots give directly: it is the number of the three preceding slots of
// its row that fall in the same group.  Ranks 0 and 1 go to plane 0, ranks 2 and 3 (a group
// with three or four nonzeros) to plane 1, so the two planes together hold any pattern; plane
// 1 is contracted only for the (32-token, 32-column) blocks where one of its values landed.
// So each hidden column costs half a dense k-step where a group holds at most two nonzeros,
// and one k-step where it holds more.
//
// Layout and pipeline follow the dense-rebuild kernel: workgroup = 256 tokens x 256 output
// columns, 8 waves in a 2 x 4 grid, each wave 128 tokens x 64 columns (4 x 2 blocks of
// 32 x 32 accumulators).  The contraction runs in steps of 64 hidden columns (two 32-column
// sparse k-steps):
//   * B step = W_down[64 rows, 256 columns], copied global -> LDS with direct loads one step
//     ahead (double buffer); the 16 bf16 of a sparse B fragment are two dense-layout
//     fragments read with ds_read_b64_tr_b16.
//   * A step, double-buffered: per token row 128 B (plane 0: four 16-byte pieces, one per
//     (32-column block, 16-column half); plane 1 likewise), the 16-byte pieces swizzled by
//     row, and 16 B of index words (plane, 32-column block), each holding the two halves'
//     16 index bits.  While the sparse MFMAs of step c read one buffer, each wave clears its
//     32 rows of the other and writes step c+1's nonzeros there: one 2-byte value store and
//     one LDS OR of its index bits per slot, to a dummy word (and zero bits) for padding or
//     slots of another step, so the writes need no branch.
//   * The slots' ranks, places and index-bit shifts are computed once per tile, four slots at
//     a time in byte lanes of 32-bit words (each slot compared with the three before it; the
//     slot before a lane's first comes from the lane that holds the previous 8-slot unit).
//   * Backup slices of overflowing tile-rows hold the nonzeros of rank >= W, all at columns
//     after the main slots', so only the group of the last main slot can hold both; their
//     ranks start after that group's main count, which the lane holding the last main slot
//     leaves in LDS.
// With few workgroups (small T) the tile range is split into S parts whose fp32 sums
// down_reduce_kernel adds in order, as for the dense-rebuild kernel.
#include <algorithm>

#include "sffn_common.hpp"

namespace sffn {

typedef __bf16 bf16x8_p __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16_p __attribute__((ext_vector_type(16)));
typedef short short4_p __attribute__((ext_vector_type(4)));
typedef short short16_p __attribute__((ext_vector_type(16)));
typedef float floatx16_p __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_vptr_p;
typedef __attribute__((address_space(3))) short4_p* lds_s4ptr_p;
struct s4pair_p {
  short4_p a, b;
};

constexpr int SP_BM = 256;  // tokens per workgroup
constexpr int SP_BN = 256;  // output columns per workgroup
constexpr int SP_KC = 64;   // hidden columns per contraction step
constexpr int SP_NW = 8;    // waves per workgroup: 2 along the tokens x 4 along the columns

// byte lanes of a and b equal (a, b < 0x80 per byte): bit 7 of each equal byte
__device__ __forceinline__ uint32_t bytes_eq(uint32_t a, uint32_t b) {
  return (0x80808080u - (a ^ b)) & 0x80808080u;
}

template <int K, int W>
__global__ __launch_bounds__(64 * SP_NW) __attribute__((amdgpu_waves_per_eu(SP_NW / 4, SP_NW / 4))) void down_sparse_kernel(
    Dims d, const uint16_t* __restrict__ counts, const uint16_t* __restrict__ vals,
    const uint8_t* __restrict__ cols, const uint16_t* __restrict__ bk_vals,
    const int32_t* __restrict__ grp_first, const uint16_t* __restrict__ Wd,
    uint16_t* __restrict__ y, float* __restrict__ dpart, int S, const int32_t* __restrict__ blk_nnz,
    long long thr) {
  constexpr int KC = SP_KC;
  constexpr int NCH = K / KC;          // steps per tile
  constexpr int U = W / 8;             // 8-slot units per tile-row
  constexpr int NKB = KC / 32;         // sparse k-steps per step
  constexpr int AROW = 128;            // bytes per A row: plane 0 then plane 1, 64 B each
  constexpr int MROW = 16;             // index bytes per A row: words (plane, 32-column block)
  constexpr int AVAL = SP_BM * AROW;   // 32 KB of values per buffer
  constexpr int ABUF = AVAL + SP_BM * MROW;  // 36 KB: one A buffer
  constexpr int BROW = SP_BN * 2;      // 512 B: one B row
  constexpr int BBUF = KC * BROW;      // 32 KB: one B buffer
  constexpr int NW = SP_NW;
  constexpr int RW = SP_BM / NW;       // A rows each wave writes
  constexpr int NWC = NW / 2;          // waves along the columns
  constexpr int WN = SP_BN / NWC;      // output columns per wave
  constexpr int NJ = WN / 32;          // 32-column MFMA blocks per wave
  constexpr int UL = RW * U / 64;      // 8-slot units per lane
  static_assert(RW == 32 && U % 2 == 0, "a lane owns one row's slot groups l/32, l/32 + 2, ..");
  static_assert(NKB == 2, "two sparse k-steps per step");
  // A buffers, then 256 B holding the dummy word that discarded value writes go to
  __shared__ __attribute__((aligned(16))) unsigned char sA[2 * ABUF + 256];
  __shared__ __attribute__((aligned(16))) unsigned char sB0[BBUF];
  __shared__ __attribute__((aligned(16))) unsigned char sB1[BBUF];
  __shared__ __attribute__((aligned(16))) uint8_t sPos[NW][64];
  // per wave and row (index 32 + row): group of the last main slot | its count there << 8
  __shared__ __attribute__((aligned(16))) uint16_t sBnd[NW][64];
  // per A buffer and writing wave: bit b set if plane 1 holds a value in 32-column block b
  __shared__ __attribute__((aligned(16))) uint32_t sFlag[2][NW];
  // per wave: 16 backup rows (one step's 64 columns each), filled by direct loads
  __shared__ __attribute__((aligned(16))) unsigned char sBk[NW][16 * 128];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = wave / NWC, wc = wave % NWC;  // MFMA tile: tokens 128wt.., columns WN wc..
  const int T = d.T;
  const int nd = (d.D + SP_BN - 1) / SP_BN;
  const int ntb = (T + SP_BM - 1) / SP_BM;
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
  const int dchunk = Pl - tb * nd;
  constexpr int TQ = NCH == 1 ? 2 : 1;
  const int nunits = d.nt / TQ;
  const int k_lo = split * nunits / S * TQ;
  const int k_hi = split + 1 == S ? d.nt : (split + 1) * nunits / S * TQ;
  const int d0 = dchunk * SP_BN;
  const bool active = d0 + WN * wc < d.D;  // D % 256 == 128: the last chunk is half wide
  const int t0 = tb * SP_BM;
  const int tw = t0 + wave * RW;  // first token of the rows this wave writes into A
  const uint32_t trash = 2 * ABUF;
  uint8_t* const pos = sPos[wave];
  const int l32 = lane & 31, lh = lane >> 5;
  // piece swizzle of this lane's A row (wave * 32 + l32): 16-byte piece q sits at q ^ swz
  const uint32_t swz = (uint32_t)(l32 >> 1) & 7u;
  // OR into the 32-bit word at byte offset off of sA (an LDS atomic: lanes may share a word)
  auto lds_or = [&](uint32_t off, uint32_t bits) __attribute__((always_inline)) {
    uint32_t* w = static_cast<uint32_t*>(__builtin_assume_aligned(sA + off, 4));
    __hip_atomic_fetch_or(w, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };

  // ---- B step -> LDS (as in the dense-rebuild kernel: row r keeps 16-byte piece c at
  // c ^ (4 (r & 3)))
  int b_col = d0 + ((lane & 31) ^ (4 * (2 * (wave & 1) + lh))) * 8;
  b_col = b_col < d.D ? b_col : d0;  // columns past D (half-wide chunk) are never read
  const uint32_t b_off = (uint32_t)(lh * d.D + b_col);
  auto issue_B = [&](int ci, unsigned char* sB) __attribute__((always_inline)) {
    const int row0 = ci * KC;
#pragma unroll
    for (int q = 0; q < BBUF / 1024 / NW; ++q) {
      const int ins = q * NW + wave;
      const uint16_t* src = Wd + (size_t)(row0 + 2 * ins) * d.D;
      __builtin_amdgcn_global_load_lds(src + b_off, (lds_vptr_p)(sB + ins * 1024), 16, 0, 0);
    }
  };

  // ---- TwELL units of tile k for this wave's rows: unit j of lane l holds slots 8 u .. +7,
  // u = l / 32 + 2 j, of token tw + l % 32.  cnt = count of token tw + lane (lanes < RW).
  uint4 uv[UL];
  uint2 uc[UL];
  uint2 ucode[UL];  // per slot: column % 4 << 6 | (piece ^ swz) << 3 | place in the piece
  uint2 umeta[UL];  // per slot: padding << 7 | index word << 5 | half << 4 | step in the tile
  uint32_t cnt = 0;
  auto load_units = [&](int k) __attribute__((always_inline)) {
    const size_t row_base = (size_t)k * T;
#pragma unroll
    for (int j = 0; j < UL; ++j) {
      const int tok = tw + l32;
      const int tk = tok < T ? tok : T - 1;
      const uint32_t m = tok < T ? 0xFFFFFFFFu : 0u;
      const size_t e0 = (row_base + tk) * W + 8 * (lh + 2 * j);
      const uint4 v = *reinterpret_cast<const uint4*>(vals + e0);
      uv[j] = make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
      uc[j] = *reinterpret_cast<const uint2*>(cols + e0);
    }
    const int t = tw + lane;
    const uint32_t m = (t < T && lane < RW) ? 0xFFFFu : 0u;
    cnt = (uint32_t)counts[row_base + (t < T ? t : T - 1)] & m;
  };

  // ---- ranks and places of the units' slots (once per tile)
  auto prep_units = [&]() __attribute__((always_inline)) {
    const uint32_t crow = (uint32_t)__shfl_xor((int)cnt, 32);
    const int cnt_row = (int)(lh ? crow : cnt);  // lanes >= 32 take their row's count from l - 32
    uint32_t X[UL];
#pragma unroll
    for (int j = 0; j < UL; ++j) X[j] = (uint32_t)__shfl_xor((int)uc[j].y, 32);
    uint32_t last_r = 0;
#pragma unroll
    for (int j = 0; j < UL; ++j) {
      // the 4 slots before this unit: unit u - 1 is lane l - 32's unit j (odd u) or lane
      // l + 32's unit j - 1 (even u); unit 0 has none (group 0x40 never matches)
      uint32_t GP;
      if (j == 0)
        GP = lh ? ((X[0] >> 2) & 0x3F3F3F3Fu) : 0x40404040u;
      else
        GP = ((lh ? X[j] : X[j - 1]) >> 2) & 0x3F3F3F3Fu;
      const uint32_t C0 = uc[j].x, C1 = uc[j].y;
      const uint32_t G0 = (C0 >> 2) & 0x3F3F3F3Fu, G1 = (C1 >> 2) & 0x3F3F3F3Fu;
      const uint32_t R0 = (bytes_eq(G0, __builtin_amdgcn_alignbyte(G0, GP, 3)) >> 7) +
                          (bytes_eq(G0, __builtin_amdgcn_alignbyte(G0, GP, 2)) >> 7) +
                          (bytes_eq(G0, __builtin_amdgcn_alignbyte(G0, GP, 1)) >> 7);
      const uint32_t R1 = (bytes_eq(G1, __builtin_amdgcn_alignbyte(G1, G0, 3)) >> 7) +
                          (bytes_eq(G1, __builtin_amdgcn_alignbyte(G1, G0, 2)) >> 7) +
                          (bytes_eq(G1, __builtin_amdgcn_alignbyte(G1, G0, 1)) >> 7);
      // padding slots (index >= count): bit 7 of their byte
      const int nreal = min(max(cnt_row - 8 * (lh + 2 * j), 0), 8);
      const uint32_t pad0 = nreal >= 4 ? 0u : (0x80808080u << (8 * nreal));
      const uint32_t pad1 = nreal >= 8 ? 0u : nreal <= 4 ? 0x80808080u : (0x80808080u << (8 * (nreal - 4)));
      const uint32_t Cw[2] = {C0, C1}, Rw[2] = {R0, R1}, pad[2] = {pad0, pad1};
      uint32_t code[2], meta[2];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint32_t C = Cw[w], R = Rw[w];
        const uint32_t pl = (R >> 1) & 0x01010101u;                         // plane
        const uint32_t pc = (C >> 4) & 0x03030303u;                         // piece in the plane
        const uint32_t s = ((C >> 1) & 0x06060606u) | (R & 0x01010101u);    // place in the piece
        const uint32_t q = ((pl << 2) | pc) ^ (swz * 0x01010101u);
        code[w] = ((C & 0x03030303u) << 6) | (q << 3) | s;                  // index | place
        const uint32_t mw = (pl << 1) | ((C >> 5) & 0x01010101u);           // index word
        meta[w] = pad[w] | (mw << 5) | (C & 0x10101010u) | ((C >> 6) & 0x03030303u);
      }
      ucode[j] = make_uint2(code[0], code[1]);
      umeta[j] = make_uint2(meta[0], meta[1]);
      last_r = R1;
    }
    // the last main slot W - 1 is slot 7 of unit U - 1 = lane l32 + 32's unit UL - 1: its group
    // and rank + 1 (read by the backup slices of an overflowing row)
    sBnd[wave][lane] = (uint16_t)((uc[UL - 1].y >> 26) | (((last_r >> 24) + 1) << 8));
  };

  // ---- write step c (of the tile) of the units into A buffer `buf`; the lane's 8 UL slots
  // are split evenly into NKB parts so the writes spread over the sparse k-steps.  Returns
  // the plane-1 block bits of the part's slots (part 0 computes them for the whole step).
  auto build_part = [&](int part, int c, int buf) __attribute__((always_inline)) -> uint32_t {
    const uint32_t rowA = (uint32_t)(buf * ABUF + (wave * RW + l32) * AROW);
    const uint32_t rowM = (uint32_t)(buf * ABUF + AVAL + (wave * RW + l32) * MROW);
    uint32_t f0 = 0, f1 = 0;
#pragma unroll
    for (int j = 0; j < UL; ++j) {
      const uint32_t vv[4] = {uv[j].x, uv[j].y, uv[j].z, uv[j].w};
      const uint32_t kw[2] = {ucode[j].x, ucode[j].y};
      const uint32_t mw[2] = {umeta[j].x, umeta[j].y};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if ((NKB * (8 * j + e)) / (8 * UL) != part) continue;
        const uint32_t code = (kw[e >> 2] >> (8 * (e & 3))) & 0xFFu;
        const uint32_t mb = (mw[e >> 2] >> (8 * (e & 3))) & 0xFFu;
        bool sel = mb < 0x80u;
        if constexpr (NCH > 1) sel = sel && (mb & 3u) == (uint32_t)c;
        const uint32_t addr = sel ? rowA + 2 * (code & 63u) : trash;
        const uint32_t word = vv[e >> 1];
        const uint16_t h = (e & 1) ? (uint16_t)(word >> 16) : (uint16_t)word;
        *reinterpret_cast<uint16_t*>(sA + addr) = h;
        const uint32_t sh = (mb & 0x10u) | ((code & 7u) << 1);  // 16 half + 2 place
        const uint32_t bits = sel ? (code >> 6) << sh : 0u;
        lds_or(rowM + 4 * ((mb >> 5) & 3u), bits);
      }
      if (part == 0) {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          uint32_t a1 = (mw[w] << 1) & ~mw[w] & 0x80808080u;  // plane 1, not padding
          if constexpr (NCH > 1) a1 &= bytes_eq(mw[w] & 0x03030303u, (uint32_t)c * 0x01010101u);
          const uint32_t kb1 = (mw[w] << 2) & 0x80808080u;     // 32-column block 1
          f0 |= a1 & ~kb1;
          f1 |= a1 & kb1;
        }
      }
    }
    if (part != 0) return 0u;
    return (ballot64(f0 != 0u) ? 1u : 0u) | (ballot64(f1 != 0u) ? 2u : 0u);
  };

  // ---- backup slices of the wave's overflowing rows (bit b of ov = token tw + b); they are
  // consecutive entries from the first entry of the wave's first 32-token group on.
  // Batches of 16 rows: lane reads the 4 columns (one group) 4 (lane % 16) .. of row
  // 4q + lane/16 of the batch.
  int bk_e0 = 0, bk_n = 0;
  // 16 rows from overflowing row `first` on, staged into this wave's LDS rows by direct loads
  // (16 B per lane: row first + 8q + lane/8, columns 8 (lane % 8) .. of step c); rows past
  // the capacity read the last entry and are never used
  auto bk_load = [&](int c, int first) __attribute__((always_inline)) {
    if (d.cap <= 0) return;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      int e = bk_e0 + first + 8 * q + (lane >> 3);
      e = e < d.cap ? e : d.cap - 1;
      const uint16_t* src = bk_vals + (size_t)e * K + c * KC + 8 * (lane & 7);
      __builtin_amdgcn_global_load_lds(src, (lds_vptr_p)(sBk[wave] + q * 1024), 16, 0, 0);
    }
  };
  // lane: the 4 columns (one group) 4 (lane % 16) .. of staged row 4q + lane/16
  auto bk_write = [&](int c, int buf, int first) __attribute__((always_inline)) -> uint32_t {
    const uint32_t g = (uint32_t)(lane & 15);  // group within the step
    const uint32_t pc = g >> 2;                // piece in the plane (32-column block, half)
    uint32_t f0 = 0, f1 = 0;
#pragma unroll 1
    for (int q = 0; q < 4; ++q) {
      if (first + 4 * q >= bk_n) break;  // wave-uniform: the 4-row groups in use
      const int rr = first + 4 * q + (lane >> 4);
      const bool ok = rr < bk_n && bk_e0 + rr < d.cap;
      const uint32_t row = ok ? pos[rr] : 0u;
      uint2 v = *reinterpret_cast<const uint2*>(sBk[wave] + (4 * q + (lane >> 4)) * 128 + 8 * g);
      if (!ok) v = make_uint2(0, 0);
      const uint32_t bnd = sBnd[wave][32 + row];
      // ranks after the main slots of the group the main part ends in
      uint32_t r = (bnd & 0xFFu) == (uint32_t)c * 16u + g ? (bnd >> 8) : 0u;
      const uint32_t rA = (uint32_t)(buf * ABUF) + (wave * RW + row) * AROW;
      const uint32_t rM = (uint32_t)(buf * ABUF + AVAL) + (wave * RW + row) * MROW;
      const uint32_t sw = (row >> 1) & 7u;
      const uint32_t w2[2] = {v.x, v.y};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t word = w2[e >> 1];
        const uint16_t h = (e & 1) ? (uint16_t)(word >> 16) : (uint16_t)word;
        const bool nz = h != 0;
        const uint32_t pl = (r >> 1) & 1u, s = 2 * (g & 3u) + (r & 1u);
        const uint32_t addr = nz ? rA + ((((pl << 2) | pc) ^ sw) << 4) + 2 * s : trash;
        *reinterpret_cast<uint16_t*>(sA + addr) = h;
        const uint32_t bits = nz ? (uint32_t)e << (16 * (pc & 1u) + 2 * s) : 0u;
        lds_or(rM + 4 * (2 * pl + (pc >> 1)), bits);
        const bool a1 = nz && pl != 0u;
        f0 |= (a1 && (pc >> 1) == 0u) ? 1u : 0u;
        f1 |= (a1 && (pc >> 1) != 0u) ? 1u : 0u;
        r += nz ? 1u : 0u;
      }
    }
    return (ballot64(f0 != 0u) ? 1u : 0u) | (ballot64(f1 != 0u) ? 2u : 0u);
  };
  auto bk_begin = [&](uint64_t ov, int e0, int k, int c) __attribute__((always_inline)) {
    bk_n = __builtin_popcountll(ov);
    if (bk_n == 0) return;
    if (cnt > (uint32_t)W) pos[mbcnt64(ov)] = (uint8_t)lane;  // ov = ballot of this predicate
    bk_e0 = e0;
    bk_load(c, 0);
  };
  auto first_entry = [&](int k) __attribute__((always_inline)) -> int {
    return ld_uniform(grp_first + (k < d.nt ? k : d.nt - 1) * d.ng + tw / GROUP);
  };
  // writes the rows staged by bk_begin (their loads are waited for here), then any further
  // batches of 16
  auto bk_finish = [&](int c, int buf) __attribute__((always_inline)) -> uint32_t {
    if (bk_n == 0) return 0u;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    uint32_t f = bk_write(c, buf, 0);
    for (int first = 16; first < bk_n; first += 16) {
      bk_load(c, first);
      __builtin_amdgcn_s_waitcnt(0x0F70);
      f |= bk_write(c, buf, first);
    }
    return f;
  };

  // ---- clear this wave's RW rows of A buffer `buf`: values (16 B per lane per store) and
  // index words (8 B)
  auto clear_a = [&](int buf) __attribute__((always_inline)) {
    uint4* p = reinterpret_cast<uint4*>(sA + buf * ABUF + wave * RW * AROW);
#pragma unroll
    for (int q = 0; q < RW * AROW / 1024; ++q) p[q * 64 + lane] = make_uint4(0, 0, 0, 0);
    reinterpret_cast<uint2*>(sA + buf * ABUF + AVAL + wave * RW * MROW)[lane] = make_uint2(0, 0);
  };

  // ---- fragments
  const int g16 = lane >> 4, li = lane & 15;
  auto a_frag = [&](int buf, int pl, int i, int kb) __attribute__((always_inline)) -> bf16x8_p {
    const int R = 128 * wt + 32 * i + l32;  // block row; 16 logical columns 32 kb + 16 lh ..
    const int q = pl * 4 + kb * 2 + lh;
    return __builtin_bit_cast(bf16x8_p, *reinterpret_cast<const uint4*>(
                                            sA + buf * ABUF + R * AROW + ((q ^ ((R >> 1) & 7)) << 4)));
  };
  auto a_idx = [&](int buf, int pl, int i, int kb) __attribute__((always_inline)) -> int {
    const int R = 128 * wt + 32 * i + l32;
    return (int)*reinterpret_cast<const uint16_t*>(sA + buf * ABUF + AVAL + R * MROW +
                                                   4 * (2 * pl + kb) + 2 * lh);
  };
  auto b_half = [&](const unsigned char* sB, int j, int kk) __attribute__((always_inline)) -> s4pair_p {
    const int c0 = WN * wc + 32 * j + 16 * (g16 & 1);
    const int col = c0 + 4 * (li & 3);
    short4_p h[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = kk * 16 + 8 * (g16 >> 1) + 4 * q + (li >> 2);
      const int off = r * BROW + ((((col >> 3) ^ (4 * (r & 3))) << 4) | ((col & 7) << 1));
      h[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4ptr_p)(sB + off));
    }
    return s4pair_p{h[0], h[1]};
  };
  auto b_frag = [&](const unsigned char* sB, int j, int kb) __attribute__((always_inline)) -> bf16x16_p {
    const s4pair_p lo = b_half(sB, j, 2 * kb), hi = b_half(sB, j, 2 * kb + 1);
    const short16_p v = {lo.a[0], lo.a[1], lo.a[2], lo.a[3], lo.b[0], lo.b[1], lo.b[2], lo.b[3],
                         hi.a[0], hi.a[1], hi.a[2], hi.a[3], hi.b[0], hi.b[1], hi.b[2], hi.b[3]};
    return __builtin_bit_cast(bf16x16_p, v);
  };

  floatx16_p acc[4][NJ];
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
  prep_units();
  clear_a(0);
  uint32_t flags = 0;  // plane-1 blocks of the A buffer being written (wave-uniform)
#pragma unroll
  for (int pt = 0; pt < NKB; ++pt) flags |= build_part(pt, 0, 0);
  {
    const uint64_t ov = ballot64(cnt > (uint32_t)W);
    if (NCH == 1) load_units(k_lo + 1 < d.nt ? k_lo + 1 : k_lo);
    bk_begin(ov, first_entry(k_lo), k_lo, 0);
    flags |= bk_finish(0, 0);
  }
  int e0_next = first_entry((c_lo + 1) / NCH);

  // step ci: sparse MFMAs of step ci (A and B buffers ci&1) while the A rows of step ci+1
  // are written into the other A buffer; plane 1 after, for its flagged blocks only.
  // new_tile: step ci+1 starts a tile (its units were loaded in the step before);
  // load_next: the units of the tile after chunk ci+1 are fetched in this step.
  auto step = [&](int ci, int cb, unsigned char* sBc, unsigned char* sBn, bool new_tile, bool load_next)
      __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): B(ci), the units, backup rows landed
    if (ci > c_lo) flags |= bk_finish(ci % NCH, cb);
    sFlag[cb][wave] = flags;
    flags = 0;
    __syncthreads();                     // A(ci), B(ci) complete; step ci-1's buffers free
    const uint4 fl4 = *reinterpret_cast<const uint4*>(&sFlag[cb][4 * wt]);
    const uint32_t fl[4] = {(uint32_t)__builtin_amdgcn_readfirstlane((int)fl4.x),
                            (uint32_t)__builtin_amdgcn_readfirstlane((int)fl4.y),
                            (uint32_t)__builtin_amdgcn_readfirstlane((int)fl4.z),
                            (uint32_t)__builtin_amdgcn_readfirstlane((int)fl4.w)};
    const int cn = ci + 1 < c_hi ? ci + 1 : c_hi - 1;
    const int c_next = cn % NCH;
    if (new_tile) prep_units();
    const uint64_t ov = ballot64(cnt > (uint32_t)W);
    const int e0 = e0_next;
    e0_next = first_entry((ci + 2) / NCH);
    bk_begin(ov, e0, cn / NCH, c_next);
    bf16x8_p fa[NKB][4];
    int fx[NKB][4];
    bf16x16_p fb[NKB][NJ];
    auto load_a = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa[kb][i] = a_frag(cb, 0, i, kb);
        fx[kb][i] = a_idx(cb, 0, i, kb);
      }
    };
    auto load_b = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) fb[kb][j] = b_frag(sBc, j, kb);
    };
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      load_a(kb);
      if (kb == 0) {
        issue_B(cn, sBn);
        clear_a(cb ^ 1);
      }
      flags |= build_part(kb, c_next, cb ^ 1);
      if (kb == NKB - 1 && load_next) {
        const int kt = (cn + 1) / NCH;
        load_units(kt < d.nt ? kt : d.nt - 1);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        fb[kb][j] = b_frag(sBc, j, kb);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(fa[kb][i], fb[kb][j], acc[i][j],
                                                                fx[kb][i], 0, 0);
      }
#pragma unroll
      for (int m = 0; m < 4 * NJ; ++m) {

      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // plane 1 of the step, when one of the wave's blocks holds a value there
    if ((fl[0] | fl[1] | fl[2] | fl[3]) != 0u) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        bf16x8_p a1[4];
        int x1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a1[i] = a_frag(cb, 1, i, kb);
          x1[i] = a_idx(cb, 1, i, kb);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const bf16x16_p b = b_frag(sBc, j, kb);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[i][j] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a1[i], b, acc[i][j], x1[i], 0, 0);
        }
      }
    }
  };
  constexpr int UF = NCH < 2 ? 2 : NCH;  // steps per unrolled iteration ((c_hi - c_lo) % UF == 0)
  for (int base = c_lo; base < c_hi; base += UF) {
#pragma unroll
    for (int s2 = 0; s2 < UF; ++s2)
      step(base + s2, s2 & 1, (s2 & 1) ? sB1 : sB0, (s2 & 1) ? sB0 : sB1, (s2 + 1) % NCH == 0,
           (s2 + 2) % NCH == 0);
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
static hipError_t launch_ds_t(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                              const void* Wd, void* y, const int32_t* blk_nnz, long long thr,
                              hipStream_t s) {
  const int nd = (d.D + SP_BN - 1) / SP_BN;
  const int ntb = (d.T + SP_BM - 1) / SP_BM;
  const int S = down_split(d);
  const int total = nd * ntb * S;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL((down_sparse_kernel<K, W>), dim3(8 * per_xcd), dim3(64 * SP_NW), 0, s, d,
                     b.counts, static_cast<const uint16_t*>(b.vals), b.cols,
                     static_cast<const uint16_t*>(b.bk_vals), ws.grp_first,
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
static hipError_t launch_ds_k(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                              const void* Wd, void* y, const int32_t* blk_nnz, long long thr,
                              hipStream_t s) {
  switch (d.W) {
    case 16: return launch_ds_t<K, 16>(d, b, ws, Wd, y, blk_nnz, thr, s);
    case 32: return launch_ds_t<K, 32>(d, b, ws, Wd, y, blk_nnz, thr, s);
    case 48: return launch_ds_t<K, 48>(d, b, ws, Wd, y, blk_nnz, thr, s);
    case 64: return launch_ds_t<K, 64>(d, b, ws, Wd, y, blk_nnz, thr, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_down_sparse(const Dims& d, const twell_buffers_t& b, const Workspace& ws,
                              const void* Wd, void* y, const int32_t* blk_nnz, long long thr,
                              hipStream_t s) {
  if (!down_mfma_supported(d)) return hipErrorInvalidValue;
  if (d.K == 64) return launch_ds_k<64>(d, b, ws, Wd, y, blk_nnz, thr, s);
  if (d.K == 128) return launch_ds_k<128>(d, b, ws, Wd, y, blk_nnz, thr, s);
  return launch_ds_k<256>(d, b, ws, Wd, y, blk_nnz, thr, s);
}

}  // namespace sffn
