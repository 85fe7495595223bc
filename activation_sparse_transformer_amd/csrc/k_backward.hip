// Backward pass of the activation-sparse ReLU FFN layer over its packed activations (gfx950).
//
// The layer is y = h W_down with h = ReLU(x W_up^T + b) (upppp.jp TwELL article of
// 2026-05-11, section "What is the waste in LLM FFN layers").  Its training kernel works on
// the same hybrid representation as the forward pass, without a dense hidden tensor (same
// article, section "What TwELL and the custom CUDA kernels solve").  With g = dL/dy:
//
//   dh[t, j]      = sum_d g[t, d] W_down[j, d]   at the stored positions of h (ReLU mask)
//   dW_down[j, :] = sum_t h[t, j]  g[t, :]        = H^T g
//   dW_up[j, :]   = sum_t dh[t, j] x[t, :]        = dH^T x
//   db[j]         = sum_t dh[t, j]
//   dx[t, :]      = sum_j dh[t, j] W_up[j, :]     (the forward's matrix-core down kernel)
//
// dh is written in the TwELL structure of h (same counts, columns and backup entries; its own
// values), rounded to bf16 like the forward's stored activations.
//
// sddmm_kernel: one workgroup per (256-token block, 128 hidden columns).  C = g_blk W_blk^T
// on v_mfma_f32_32x32x16_bf16 (both operands contiguous along d, loaded global -> LDS with
// direct loads, double-buffered, 64 columns of d per step); C goes through LDS as bf16 and
// each token row picks the values of its stored slots (and its backup slice's nonzero
// positions).
//
// tmm_kernel: one workgroup per (256 hidden columns, 256 columns of d): dW = H^T M summed
// over 64-token steps.  Each step rebuilds the 64 x 256 block of H in LDS from TwELL rows
// (as the forward's down kernel does) and loads M (g or x) rows with direct loads; both MFMA
// operands come out of the token-major tiles through ds_read_b64_tr_b16.  With DB the same
// kernel also sums the A fragments into db.
#include "sffn_common.hpp"

namespace sffn {

typedef __bf16 bf16x8_b __attribute__((ext_vector_type(8)));
typedef short short4_b __attribute__((ext_vector_type(4)));
typedef short short8_b __attribute__((ext_vector_type(8)));
typedef float floatx16_b __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_b __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_vptr_b;
typedef __attribute__((address_space(3))) short4_b* lds_s4ptr_b;

constexpr int BW_JB = 128;  // hidden columns per sddmm workgroup

// ============================================================================ SDDMM
template <int K, int W>
__global__ __launch_bounds__(256) void sddmm_kernel(
    Dims d, const uint16_t* __restrict__ g, const uint16_t* __restrict__ Wd,
    const uint16_t* __restrict__ counts, const uint8_t* __restrict__ cols,
    const uint16_t* __restrict__ h_bk, const int32_t* __restrict__ grp_first,
    uint16_t* __restrict__ dh_vals, uint16_t* __restrict__ dh_bk) {
  constexpr int HALVES = K / BW_JB;  // workgroups per tile along the hidden columns
  constexpr int ROW = 128;           // bytes of one 64-column bf16 row of a step tile
  // step tiles: g rows of 256 tokens (A) and W_down rows of 128 hidden columns (B), both
  // 64 values of d; 16-byte piece p of row r at p ^ ((r >> 1) & 7)
  // three stages (separate objects: loads into one and reads of the others never alias)
  __shared__ __attribute__((aligned(16))) unsigned char sA0[256 * ROW];
  __shared__ __attribute__((aligned(16))) unsigned char sA1[256 * ROW];
  __shared__ __attribute__((aligned(16))) unsigned char sA2[256 * ROW];
  __shared__ __attribute__((aligned(16))) unsigned char sB0[128 * ROW];
  __shared__ __attribute__((aligned(16))) unsigned char sB1[128 * ROW];
  __shared__ __attribute__((aligned(16))) unsigned char sB2[128 * ROW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = wave >> 1, wj = wave & 1;  // MFMA tile: tokens 128wt.., columns 64wj..
  const int T = d.T, D = d.D;
  const int nj = d.F / BW_JB;
  const int ntb = (T + 255) / 256;
  const int total = nj * ntb;
  const int per_xcd = (total + 7) / 8;
  const int P = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (P >= total) return;
  const int tb = P / nj;
  const int jb = P - tb * nj;
  const int t0 = tb * 256;
  const int j0 = jb * BW_JB;
  const int k = j0 / K, hf = (j0 % K) / BW_JB;

  auto issue = [&](int s, unsigned char* sA, unsigned char* sB) __attribute__((always_inline)) {
    const int dcol = s * 64;
#pragma unroll
    for (int q = 0; q < 8; ++q) {  // A: 32 loads of 1 KB (8 rows), 8 per wave
      const int ins = q * 4 + wave;
      const int r = ins * 8 + (lane >> 3), pc = lane & 7;
      const int lc = pc ^ ((r >> 1) & 7);
      int t = t0 + r;
      t = t < T ? t : T - 1;  // rows past T: never written out
      __builtin_amdgcn_global_load_lds(g + (size_t)t * D + dcol + lc * 8,
                                       (lds_vptr_b)(sA + ins * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // B: 16 loads, 4 per wave
      const int ins = q * 4 + wave;
      const int r = ins * 8 + (lane >> 3), pc = lane & 7;
      const int lc = pc ^ ((r >> 1) & 7);
      __builtin_amdgcn_global_load_lds(Wd + (size_t)(j0 + r) * D + dcol + lc * 8,
                                       (lds_vptr_b)(sB + ins * 1024), 16, 0, 0);
    }
  };
  const int l32 = lane & 31, lh = lane >> 5;
  auto frag = [&](const unsigned char* s, int row, int kk) __attribute__((always_inline)) -> bf16x8_b {
    const int ch = kk * 2 + lh;
    return __builtin_bit_cast(
        bf16x8_b, *reinterpret_cast<const uint4*>(s + row * ROW + ((ch ^ ((row >> 1) & 7)) << 4)));
  };

  floatx16_b acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // The d-loop is a ring of three LDS stages of 64 columns (4 MFMA k-steps each); a stage's
  // loads are issued two stages ahead, the next k-step's fragments are read while the current
  // one's MFMAs run, and at a stage's last k-step the next stage is waited for (its loads and
  // every wave's reads of this stage: one barrier), the freed buffer refilled and the next
  // stage's first fragments read before that k-step's MFMAs.  Every stage runs the same
  // instructions (past the end the last stage is loaded again into a buffer nothing reads)
  // and the loop runs over whole rings, so the compiler adds no load waits of its own.
  constexpr int NS = 3;
  constexpr int LPS = 12;  // direct loads per wave per stage (8 of g, 4 of W_down)
  constexpr int VM_NEXT = LPS * (NS - 2), VM_FIRST = LPS * (NS - 1);
  static_assert(VM_FIRST <= 63, "vmcnt immediate");
  const int nsteps = D / 64;
  bf16x8_b fa[2][4], fb[2][2];
  auto load_frags = [&](const unsigned char* sA, const unsigned char* sB, int kk, bf16x8_b (&a)[4],
                        bf16x8_b (&b)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = frag(sA, 128 * wt + 32 * i + l32, kk);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = frag(sB, 64 * wj + 32 * j + l32, kk);
  };
  auto mfmas = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][i], fb[c][j], acc[i][j], 0, 0, 0);
  };
  auto stage = [&](int st, unsigned char* A, unsigned char* B, const unsigned char* An,
                   const unsigned char* Bn) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = kk & 1;
      if (kk < 3) {
        __builtin_amdgcn_sched_barrier(0);
        load_frags(A, B, kk + 1, fa[c ^ 1], fb[c ^ 1]);
        mfmas(c);
#pragma unroll
        for (int i = 0; i < 6; ++i) {  // one fragment read after each of the first MFMAs
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_barrier(0);
      } else {
        // the next stage is in once only the stage after it may still be loading
        __builtin_amdgcn_s_waitcnt(0x0F70 | (VM_NEXT & 15) | ((VM_NEXT >> 4) << 14));
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this stage's reads are done
        // a plain barrier: the fence of __syncthreads would also wait for the loads in
        // flight (they write LDS); the clobber keeps memory accesses in place
        __asm__ volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        issue(st + NS < nsteps ? st + NS : nsteps - 1, A, B);
        load_frags(An, Bn, 0, fa[c ^ 1], fb[c ^ 1]);
        mfmas(c);
#pragma unroll
        for (int i = 0; i < 6; ++i) {  // the refill loads between the MFMAs
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
          __builtin_amdgcn_sched_group_barrier(0x010, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  issue(0, sA0, sB0);
  issue(1 < nsteps ? 1 : 0, sA1, sB1);
  issue(2 < nsteps ? 2 : nsteps - 1, sA2, sB2);
  __builtin_amdgcn_s_waitcnt(0x0F70 | (VM_FIRST & 15) | ((VM_FIRST >> 4) << 14));  // stage 0
  __asm__ volatile("s_barrier" ::: "memory");
  load_frags(sA0, sB0, 0, fa[0], fb[0]);
  const int nring = nsteps / NS * NS;
  for (int st = 0; st < nring; st += NS) {
    stage(st, sA0, sB0, sA1, sB1);
    stage(st + 1, sA1, sB1, sA2, sB2);
    stage(st + 2, sA2, sB2, sA0, sB0);
  }
  // the last nsteps % 3 stages (the ring position is back at buffer 0)
  if (nring < nsteps) stage(nring, sA0, sB0, sA1, sB1);
  if (nring + 1 < nsteps) stage(nring + 1, sA1, sB1, sA2, sB2);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the repeated loads land before LDS is reused
  __syncthreads();  // every wave is done with the step tiles

  // ---- C (bf16) -> LDS: token row t (0..255) of 256 B at (t < 128 ? sA0 : sA1) + (t & 127) * 256
  auto crow = [&](int t) __attribute__((always_inline)) -> unsigned char* {
    return (t < 128 ? sA0 : sA1) + (t & 127) * 256;
  };
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = 128 * wt + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
        const int c = 64 * wj + 32 * j + l32;
        *reinterpret_cast<uint16_t*>(crow(t) + 2 * c) = f32_to_bf16(acc[i][j][r]);
      }
  __syncthreads();

  // ---- main slots: thread tid <-> token t0 + tid
  const int t = t0 + tid;
  uint32_t cnt = 0;
  if (t < T) {
    cnt = counts[(size_t)k * T + t];
    const unsigned char* cr = crow(tid);
    const size_t e0 = ((size_t)k * T + t) * W;
    const uint32_t m = cnt < (uint32_t)W ? cnt : (uint32_t)W;
#pragma unroll
    for (int q = 0; q < W / 8; ++q) {
      const uint2 cw = *reinterpret_cast<const uint2*>(cols + e0 + 8 * q);
      const uint32_t cc[2] = {cw.x, cw.y};
      if constexpr (HALVES == 1) {
        uint32_t o[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const uint32_t c0 = (cc[e >> 2] >> (8 * (e & 3))) & 0xFFu;
          const uint32_t c1 = (cc[(e + 1) >> 2] >> (8 * ((e + 1) & 3))) & 0xFFu;
          const uint32_t v0 = (uint32_t)(8 * q + e) < m ? *reinterpret_cast<const uint16_t*>(cr + 2 * c0) : 0u;
          const uint32_t v1 = (uint32_t)(8 * q + e + 1) < m ? *reinterpret_cast<const uint16_t*>(cr + 2 * c1) : 0u;
          o[e >> 1] = v0 | (v1 << 16);
        }
        *reinterpret_cast<uint4*>(dh_vals + e0 + 8 * q) = make_uint4(o[0], o[1], o[2], o[3]);
      } else {
        // two workgroups share the row: each writes the slots in its half; the first also
        // writes the padding
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t s = 8 * q + e;
          const uint32_t c = (cc[e >> 2] >> (8 * (e & 3))) & 0xFFu;
          if (s < m) {
            if ((int)(c >> 7) == hf)
              dh_vals[e0 + s] = *reinterpret_cast<const uint16_t*>(cr + 2 * (c & 127));
          } else if (hf == 0) {
            dh_vals[e0 + s] = 0;
          }
        }
      }
    }
  }

  // ---- backup slices: wave w covers tokens 64w..64w+63 of the block (two 32-token groups);
  // the entries of a group's overflowing rows are consecutive, in token order
  {
    const int tw = t0 + 64 * wave;
    const int tl = tw + lane;
    uint32_t cl = 0;
    if (tl < T) cl = counts[(size_t)k * T + tl];
    const uint64_t ov_all = ballot64(cl > (uint32_t)W);
    uint64_t ov = ov_all;
    while (ov != 0) {
      const int b = __builtin_ctzll(ov);
      ov &= ov - 1;
      const uint64_t below =
          ov_all & ((1ull << b) - 1ull) & (b >= 32 ? 0xFFFFFFFF00000000ull : 0xFFFFFFFFull);
      const int e = ld_uniform(grp_first + k * d.ng + tw / GROUP + (b >> 5)) + __builtin_popcountll(below);
      if (e >= d.cap) continue;  // capacity exceeded: the status word reports it
      const unsigned char* cr = crow(64 * wave + b);
      const size_t base = (size_t)e * K + hf * BW_JB + 2 * lane;
      const uint32_t hv = *reinterpret_cast<const uint32_t*>(h_bk + base);
      const uint32_t cv = *reinterpret_cast<const uint32_t*>(cr + 4 * lane);
      const uint32_t lo = (hv & 0xFFFFu) ? (cv & 0xFFFFu) : 0u;
      const uint32_t hi = (hv >> 16) ? (cv & 0xFFFF0000u) : 0u;
      *reinterpret_cast<uint32_t*>(dh_bk + base) = lo | hi;
    }
  }
}

// ============================================================================ H^T M
// tmm_kernel: dW = H^T M with 8 waves (two per SIMD) per workgroup of (256 hidden columns,
// 256 columns of d), 64-token steps; wave (wj, wd) computes hidden 64 wj.. x d 128 wd...  The H step tile is 64 tokens x 256 hidden columns.  Each wave owns whole row
// segments of it (one token x one tile: 16 segments of 128 columns or 8 of 256): it clears
// them, writes their slots and their backup slices, so no other wave touches them within the
// step.  Fragments of the next k-step are read while the current one's MFMAs run.
constexpr int TMM_JB = 256;  // hidden columns per workgroup
constexpr int TMM_TS = 64;   // tokens per step

template <int K, int W, bool DB>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void tmm_kernel(
    Dims d, const uint16_t* __restrict__ Hv, const uint16_t* __restrict__ Hbk,
    const uint16_t* __restrict__ counts, const uint8_t* __restrict__ cols,
    const int32_t* __restrict__ grp_first, const uint16_t* __restrict__ M,
    float* __restrict__ dW, float* __restrict__ db) {
  constexpr int TS = TMM_TS;
  constexpr int NTL = TMM_JB / K;           // tiles per workgroup (2 or 1)
  constexpr int U = W / 8;                  // 8-slot units per tile-row
  constexpr int SPW = TS * NTL / 8;         // row segments per wave (16 or 8)
  constexpr int NU = (SPW * U + 63) / 64;   // units per lane
  constexpr int SEGB = K * 2;               // bytes of one segment
  constexpr int HROW = TMM_JB * 2;          // 512 B: one token row of the H step tile
  constexpr int HBUF = TS * HROW;           // 32 KB
  constexpr int MROW = 512;                 // M step tile: TS tokens x 256 columns
  constexpr int MBUF = TS * MROW;           // 32 KB
  constexpr int NKK = TS / 16;              // MFMA k-steps per step
  constexpr int VPL = K / 64;               // backup values per lane (2 or 4)
  static_assert(SPW * SEGB == 4096, "a wave clears 4 KB per step");
  __shared__ __attribute__((aligned(16))) unsigned char sH[2 * HBUF + 256];
  __shared__ __attribute__((aligned(16))) unsigned char sM0[MBUF];
  __shared__ __attribute__((aligned(16))) unsigned char sM1[MBUF];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wj = wave >> 1, wd = wave & 1;  // MFMA tile: hidden 64 wj.., d 128 wd..
  const int T = d.T, D = d.D;
  const int nj = d.F / TMM_JB;
  const int nd = D / 256;
  const int total = nj * nd;
  const int per_xcd = (total + 7) / 8;
  const int P = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (P >= total) return;
  // column-chunk-major: the workgroups an XCD runs together read the same M columns
  const int dchunk = P / nj;
  const int jb = P - dchunk * nj;
  const int d0 = dchunk * 256;
  const int j0 = jb * TMM_JB;
  const int k0 = j0 / K;  // first tile of the workgroup
  const uint32_t trash = 2 * HBUF;  // one dummy word for every discarded write
  // this wave's segments: s = wave * SPW + i, tile s / TS, token s % TS of the step
  const int seg_tl = (wave * SPW) / TS;
  const int seg_t0 = (wave * SPW) % TS;

  auto issue_M = [&](int ts, unsigned char* sM) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < MBUF / 1024 / 8; ++q) {  // loads of 1 KB (two rows), 4 per wave
      const int ins = q * 8 + wave;
      const int slot = ins * 64 + lane;
      const int r = slot >> 5, pc = slot & 31;
      const int lc = pc ^ (4 * (r & 3));
      int t = ts * TS + r;
      t = t < T ? t : T - 1;  // rows past T meet zero rows of H
      __builtin_amdgcn_global_load_lds(M + (size_t)t * D + d0 + lc * 8,
                                       (lds_vptr_b)(sM + ins * 1024), 16, 0, 0);
    }
  };

  // ---- TwELL units of this wave's segments: unit v = lane + 64 q (v < SPW U) holds slots
  // 8 (v % U) .. +7 of segment v / U (token seg_t0 + v / U of tile k0 + seg_tl)
  uint4 uv[NU];
  uint2 uc[NU];
  uint32_t cnt = 0;  // count of token TS ts + lane in tile k0 + seg_tl (the backup rows)
  auto load_units = [&](int ts) __attribute__((always_inline)) {
    const size_t row_base = (size_t)(k0 + seg_tl) * T;
#pragma unroll
    for (int q = 0; q < NU; ++q) {
      const int v = lane + 64 * q;
      const int vv = v < SPW * U ? v : 0;
      int tok = ts * TS + seg_t0 + vv / U;
      tok = tok < T ? tok : T - 1;
      const size_t e0 = (row_base + tok) * W + 8 * (vv % U);
      uv[q] = *reinterpret_cast<const uint4*>(Hv + e0);
      uc[q] = *reinterpret_cast<const uint2*>(cols + e0);
    }
    const int tl = ts * TS + lane;
    const uint32_t m = tl < T ? 0xFFFFu : 0u;
    cnt = (uint32_t)counts[row_base + (tl < T ? tl : T - 1)] & m;
  };
  // byte offset of (token row r, hidden column hc of the workgroup) in H buffer `buf`; piece
  // p of a row sits at p ^ (4 (r & 3)), which keeps a segment's pieces inside the segment
  auto h_off = [&](int buf, uint32_t r, uint32_t hc) __attribute__((always_inline)) -> uint32_t {
    return buf * HBUF + r * HROW + ((((hc >> 3) ^ (4 * (r & 3))) << 4) | ((hc & 7) << 1));
  };
  // the H block of step ts is built in three pieces spread over the MFMAs of the step before:
  // clear_h (this wave's segments), build_part (its slots, split evenly over the k-steps:
  // slot q = 8 unit + e in part 4q / (8 NU)) and build_bk (its backup slices)
  auto clear_h = [&](int buf) __attribute__((always_inline)) {
    // this wave's segments (4 KB): piece i of the wave is piece i % (SEGB/16) of segment
    // i / (SEGB/16)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pi = lane + 64 * q;
      const int sg = pi / (SEGB / 16), pc = pi % (SEGB / 16);
      uint4* p = reinterpret_cast<uint4*>(sH + buf * HBUF + (seg_t0 + sg) * HROW + seg_tl * SEGB +
                                          pc * 16);
      *p = make_uint4(0, 0, 0, 0);
    }
  };
  auto build_part = [&](int part, int ts, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < NU; ++q) {
      const int v = lane + 64 * q;
      const uint32_t r = (uint32_t)(seg_t0 + (v < SPW * U ? v : 0) / U);  // token row of the step
      const bool ok = v < SPW * U && ts * TS + (int)r < T;
      const uint32_t vv[4] = {uv[q].x, uv[q].y, uv[q].z, uv[q].w};
      const uint32_t cw[2] = {uc[q].x, uc[q].y};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if ((4 * (8 * q + e)) / (8 * NU) != part) continue;
        const uint32_t col = (cw[e >> 2] >> (8 * (e & 3))) & 0xFFu;
        const uint32_t word = vv[e >> 1];
        const bool nz = (e & 1) ? (word > 0xFFFFu) : ((word & 0xFFFFu) != 0u);
        const uint32_t a = (ok && nz) ? h_off(buf, r, seg_tl * K + col) : trash;
        *reinterpret_cast<uint16_t*>(sH + a) = (e & 1) ? (uint16_t)(word >> 16) : (uint16_t)word;
      }
    }
  };
  // backup slices of the overflowing rows among this wave's segments; entry = first entry of
  // the row's (tile, 32-token group) + its rank among the group's overflowing rows.  The
  // slices of the first BKP such rows of the next step are loaded when the step starts (so
  // they land during its MFMAs) and written at its end; further rows are loaded there.
  constexpr int BKP = 2;
  uint32_t bkw[BKP][VPL / 2];
  int bkt[BKP];
  uint64_t bk_ovall = 0, bk_rest = 0;
  auto bk_entry = [&](int ts, int tt) __attribute__((always_inline)) -> int {
    const int gb = tt & ~(GROUP - 1);
    const uint64_t below = bk_ovall & ((1ull << tt) - 1ull) & ~((1ull << gb) - 1ull);
    return ld_uniform(grp_first + (k0 + seg_tl) * d.ng + (ts * TS + gb) / GROUP) +
           __builtin_popcountll(below);
  };
  auto bk_prefetch = [&](int ts) __attribute__((always_inline)) {
    bk_ovall = ballot64(cnt > (uint32_t)W);  // token TS ts + lane
    uint64_t ov = (bk_ovall >> seg_t0) & ((1ull << SPW) - 1ull);
#pragma unroll
    for (int j = 0; j < BKP; ++j) {
#pragma unroll
      for (int v = 0; v < VPL / 2; ++v) bkw[j][v] = 0u;
      bkt[j] = -1;
      if (ov == 0) continue;  // wave-uniform
      const int tt = seg_t0 + __builtin_ctzll(ov);
      ov &= ov - 1;
      const int e = bk_entry(ts, tt);
      if (e >= d.cap) continue;  // capacity exceeded: the status word reports it
      bkt[j] = tt;
      const uint32_t* src = reinterpret_cast<const uint32_t*>(Hbk + (size_t)e * K + VPL * lane);
#pragma unroll
      for (int v = 0; v < VPL / 2; ++v) bkw[j][v] = src[v];
    }
    bk_rest = ov;
  };
  auto build_bk = [&](int ts, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < BKP; ++j) {
      if (bkt[j] < 0) continue;  // wave-uniform
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const uint16_t hv = (uint16_t)(bkw[j][v >> 1] >> (16 * (v & 1)));
        const uint32_t a = hv ? h_off(buf, bkt[j], seg_tl * K + VPL * lane + v) : trash;
        *reinterpret_cast<uint16_t*>(sH + a) = hv;
      }
    }
    uint64_t ov = bk_rest;
    while (ov != 0) {
      const int i = __builtin_ctzll(ov);
      ov &= ov - 1;
      const int tt = seg_t0 + i;  // token row of the step
      const int e = bk_entry(ts, tt);
      if (e >= d.cap) continue;  // capacity exceeded: the status word reports it
      const uint16_t* src = Hbk + (size_t)e * K + VPL * lane;
      uint16_t hv[VPL];
      if constexpr (VPL == 2) {
        const uint32_t w2 = *reinterpret_cast<const uint32_t*>(src);
        hv[0] = (uint16_t)w2;
        hv[1] = (uint16_t)(w2 >> 16);
      } else {
        const uint2 w4 = *reinterpret_cast<const uint2*>(src);
        hv[0] = (uint16_t)w4.x;
        hv[1] = (uint16_t)(w4.x >> 16);
        hv[2] = (uint16_t)w4.y;
        hv[3] = (uint16_t)(w4.y >> 16);
      }
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const uint32_t a = hv[v] ? h_off(buf, tt, seg_tl * K + VPL * lane + v) : trash;
        *reinterpret_cast<uint16_t*>(sH + a) = hv[v];
      }
    }
  };

  const int g16 = lane >> 4, li = lane & 15;
  const int l32 = lane & 31, lh = lane >> 5;
  // transposed read: lane L of a 16-lane group reads row r0 + L/4, columns c0 + 4(L%4)..;
  // lane i then holds column c0 + i of rows r0..r0+3
  auto tr_frag = [&](const unsigned char* base, int rowb, int c0, int kk) __attribute__((always_inline)) -> bf16x8_b {
    const int col = c0 + 16 * (g16 & 1) + 4 * (li & 3);
    short4_b h[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int r = kk * 16 + 8 * (g16 >> 1) + 4 * q + (li >> 2);
      const int off = r * rowb + ((((col >> 3) ^ (4 * (r & 3))) << 4) | ((col & 7) << 1));
      h[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4ptr_b)(base + off));
    }
    const short8_b v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
    return __builtin_bit_cast(bf16x8_b, v);
  };

  floatx16_b acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  float dbacc[2] = {0.0f, 0.0f};
  const bool do_db = DB && dchunk == 0 && wd == 0;

  const int nts = (T + TS - 1) / TS;
  issue_M(0, sM0);
  load_units(0);
  clear_h(0);
#pragma unroll
  for (int pt = 0; pt < 4; ++pt) build_part(pt, 0, 0);
  bk_prefetch(0);
  build_bk(0, 0);
  load_units(nts > 1 ? 1 : 0);
  auto step = [&](int ts, int cb, unsigned char* sMc, unsigned char* sMn) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): M(ts) and the units have landed
    __syncthreads();                     // H(ts), M(ts) complete; step ts-1's buffers free
    const unsigned char* hb = sH + cb * HBUF;
    bf16x8_b fa[2][2], fb[2][4];
    auto load_frags = [&](int kk, bf16x8_b (&a)[2], bf16x8_b (&b)[4]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = tr_frag(hb, HROW, 64 * wj + 32 * i, kk);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = tr_frag(sMc, MROW, 128 * wd + 32 * j, kk);
    };
    // the next step's tiles while these MFMAs run; the last step rebuilds its own tiles into
    // the other buffers, which nothing reads any more, instead of branching, so each k-step's
    // MFMAs and build share one basic block
    const int tn = ts + 1 < nts ? ts + 1 : nts - 1;
    bk_prefetch(tn);  // the units of step tn are in
    load_frags(0, fa[0], fb[0]);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (kk + 1 < NKK) load_frags(kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
      if (kk == 0) {
        issue_M(tn, sMn);
        clear_h(cb ^ 1);
      }
      build_part(kk, tn, cb ^ 1);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][i], fb[kk & 1][j],
                                                              acc[i][j], 0, 0, 0);
      if constexpr (DB) {  // every wave sums; only the db waves store (no branch here)
        // the fragment's 8 values in pairs against (1, 1): four dot2 instructions (fp32
        // accumulation) instead of eight conversions and eight adds
        const bf16x2_b ones = __builtin_bit_cast(bf16x2_b, 0x3F803F80u);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint4 u = __builtin_bit_cast(uint4, fa[kk & 1][i]);
          const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            dbacc[i] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_b, w[q]), ones,
                                                       dbacc[i], false);
        }
      }
      // one MFMA, then a few vector and LDS instructions in its shadow
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x080, 2, 0);  // LDS
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    build_bk(tn, cb ^ 1);
    load_units(ts + 2 < nts ? ts + 2 : nts - 1);
  };
  for (int ts = 0; ts < nts; ts += 2) {
    step(ts, 0, sM0, sM1);
    if (ts + 1 < nts) step(ts + 1, 1, sM1, sM0);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the last step's repeated loads land before LDS goes away

  // ---- dW (fp32): C[m = j][n = d]; lane: column l32, rows 8(r/4) + 4lh + r%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int jr = j0 + 64 * wj + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
        dW[(size_t)jr * D + d0 + 128 * wd + 32 * j + l32] = acc[i][j][r];
      }
  if (do_db) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float s = dbacc[i] + __shfl_xor(dbacc[i], 32);
      if (lh == 0) db[j0 + 64 * wj + 32 * i + l32] = s;
    }
  }
}

// ============================================================================ launchers
bool backward_supported(const Dims& d) {
  return d.bf16 && (d.K == 128 || d.K == 256) && d.D % 256 == 0 &&
         (d.W == 16 || d.W == 32 || d.W == 48 || d.W == 64);
}

// which: 0 = dh (sddmm), 1 = dW_down (H^T g), 2 = dW_up (+ db if not null) (dH^T x)
template <int K, int W>
static hipError_t launch_bwd_t(int which, const Dims& d, const twell_buffers_t& act,
                               const Workspace& ws, const uint16_t* x, const uint16_t* g,
                               const uint16_t* Wd, uint16_t* dh_vals, uint16_t* dh_bk,
                               float* dW_up, float* dW_down, float* db, hipStream_t s) {
  const int nj = d.F / BW_JB;
  if (which == 0) {
    const int total = nj * ((d.T + 255) / 256);
    hipLaunchKernelGGL((sddmm_kernel<K, W>), dim3(8 * ((total + 7) / 8)), dim3(256), 0, s, d, g,
                       Wd, act.counts, act.cols, static_cast<const uint16_t*>(act.bk_vals),
                       ws.grp_first, dh_vals, dh_bk);
    return hipGetLastError();
  }
  const int total = (d.F / TMM_JB) * (d.D / 256);
  const dim3 grid(8 * ((total + 7) / 8));
  if (which == 1) {
    hipLaunchKernelGGL((tmm_kernel<K, W, false>), grid, dim3(512), 0, s, d,
                       static_cast<const uint16_t*>(act.vals),
                       static_cast<const uint16_t*>(act.bk_vals), act.counts, act.cols,
                       ws.grp_first, g, dW_down, nullptr);
  } else if (db) {
    hipLaunchKernelGGL((tmm_kernel<K, W, true>), grid, dim3(512), 0, s, d, dh_vals, dh_bk,
                       act.counts, act.cols, ws.grp_first, x, dW_up, db);
  } else {
    hipLaunchKernelGGL((tmm_kernel<K, W, false>), grid, dim3(512), 0, s, d, dh_vals, dh_bk,
                       act.counts, act.cols, ws.grp_first, x, dW_up, nullptr);
  }
  return hipGetLastError();
}

template <int K>
static hipError_t launch_bwd_k(int which, const Dims& d, const twell_buffers_t& act,
                               const Workspace& ws, const uint16_t* x, const uint16_t* g,
                               const uint16_t* Wd, uint16_t* dh_vals, uint16_t* dh_bk,
                               float* dW_up, float* dW_down, float* db, hipStream_t s) {
  switch (d.W) {
    case 16: return launch_bwd_t<K, 16>(which, d, act, ws, x, g, Wd, dh_vals, dh_bk, dW_up, dW_down, db, s);
    case 32: return launch_bwd_t<K, 32>(which, d, act, ws, x, g, Wd, dh_vals, dh_bk, dW_up, dW_down, db, s);
    case 48: return launch_bwd_t<K, 48>(which, d, act, ws, x, g, Wd, dh_vals, dh_bk, dW_up, dW_down, db, s);
    case 64: return launch_bwd_t<K, 64>(which, d, act, ws, x, g, Wd, dh_vals, dh_bk, dW_up, dW_down, db, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_backward_part(int which, const Dims& d, const twell_buffers_t& act,
                                const Workspace& ws, const void* x, const void* g,
                                const void* Wd, void* dh_vals, void* dh_bk, float* dW_up,
                                float* dW_down, float* db, hipStream_t s) {
  if (!backward_supported(d)) return hipErrorInvalidValue;
  auto* xx = static_cast<const uint16_t*>(x);
  auto* gg = static_cast<const uint16_t*>(g);
  auto* ww = static_cast<const uint16_t*>(Wd);
  auto* hv = static_cast<uint16_t*>(dh_vals);
  auto* hb = static_cast<uint16_t*>(dh_bk);
  if (d.K == 128)
    return launch_bwd_k<128>(which, d, act, ws, xx, gg, ww, hv, hb, dW_up, dW_down, db, s);
  return launch_bwd_k<256>(which, d, act, ws, xx, gg, ww, hv, hb, dW_up, dW_down, db, s);
}

}  // namespace sffn
