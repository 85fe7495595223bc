// Fused up-projection + bias + ReLU + TwELL pack, bf16 MFMA on gfx950.
//
// z = x W_up^T + b (fp32 accumulation), h = z if z > 0 else 0, and h goes straight into
// TwELL: the dense hidden tensor is never written to device memory (upppp.jp TwELL article
// of 2026-05-11, section "What TwELL and the custom CUDA kernels solve": the inference
// kernel builds the TwELL form on the fly; innovatopia.jp article, "Editor's commentary":
// no extra memory traffic or kernel launches for the sparse format).
//
// Main loop (dense contraction, MFMA-bound):
//   * workgroup tile 256 neurons x BM tokens (BM = 64*NB), 4 waves; wave (wn, wt) owns
//     neurons [128*wn, 128*wn+128) x tokens [wt*BM/2, (wt+1)*BM/2) of the tile.
//   * v_mfma_f32_32x32x16_bf16 with A = W_up rows (neurons) and B = x rows (tokens): both
//     operands are contiguous along d_model, so both are read from LDS as 16-byte rows.
//   * d_model is consumed in slices of BK columns (32 for 128- and 256-column tiles, 64 for
//     64-column tiles) through a ring of NS LDS stages filled by direct global -> LDS loads
//     issued NS - 1 stages ahead; 16-byte chunks XOR-swizzled by row so the rows a wave
//     reads at one column land in distinct banks.
//   * workgroups are ordered in groups of 8 token blocks and dispatched so that the
//     workgroups sharing an XCD's L2 cover a compact patch of the output.
//
// Epilogue (the TwELL pack, done on the accumulator registers):
//   The 32x32 accumulator layout puts token n = lane%32 of a block in lanes n and n+32,
//   each holding 16 of the block's 32 neurons (lane half h holds the neurons 8q+4h+i).
//   Over the wave's 4 neuron blocks the lane pair holds all 128 neurons of the token,
//   i.e. a whole 128-column tile-row.  Each lane builds a 64-bit mask of its positive
//   pre-activations, swaps masks with its partner (lane ^ 32), and gets the rank of every
//   nonzero - the number of nonzeros at lower columns - from popcounts.  No transpose of
//   the hidden tile through LDS is needed.  Ranks < W are scattered into an LDS staging
//   block that is then written out as contiguous TwELL rows; ranks >= W go to the staged
//   backup slice of the tile-row.  Tiles of 64 columns are handled as two tiles per wave,
//   tiles of 256 columns span the two waves with the same tokens (counts exchanged in LDS).
#include "sffn_common.hpp"

namespace sffn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int UP_BN = 256;  // neurons per workgroup
constexpr int UP_GM = 8;    // token blocks per ordering group

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// s_waitcnt immediate waiting for at most n vector-memory operations in flight (gfx9
// encoding: vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt left at their no-wait values).
constexpr int vmcnt_enc(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// BK: d_model slice per LDS stage.  WPE: waves per SIMD the kernel is built for; with 2
// (BK = 32, 128 tokens, 48 KB of LDS, at most 256 registers), two workgroups share a CU and
// one's pack epilogue runs while the other's MFMA loop keeps the matrix cores busy.
// NS: LDS stages in the ring (the loads of a stage are issued NS - 1 stages ahead).
template <int K, int NB, bool DUMP, int BK, int WPE, int NS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void
up_pack_bf16_kernel(Dims d, const uint16_t* __restrict__ x, const uint16_t* __restrict__ Wu,
                    const uint16_t* __restrict__ bu, twell_buffers_t b, Workspace ws,
                    float* __restrict__ zdump) {
  constexpr int BM = 64 * NB;            // tokens per workgroup
  constexpr int HM = BM / 2;             // tokens per wave
  constexpr int CH = BK / 8;             // 16-byte pieces per LDS row (8 or 4)
  constexpr int RPI = 64 / CH;           // rows filled by one 64-lane direct load
  constexpr int ALD = UP_BN / RPI / 4;   // direct loads of A per wave per stage
  constexpr int BLD = BM / RPI / 4;      // direct loads of B per wave per stage
  constexpr int TPW = (K == 64) ? 2 : 1; // tile parts per wave
  constexpr int NTWG = UP_BN / K;        // tiles per workgroup (4, 2, 1)

  // LDS: NS stages, each a separate object so that loads into one stage and reads of the
  // others are known not to alias; after the loop the A stages hold the TwELL staging.
  __shared__ __attribute__((aligned(16))) uint4 sA0[UP_BN * CH];
  __shared__ __attribute__((aligned(16))) uint4 sA1[UP_BN * CH];
  __shared__ __attribute__((aligned(16))) uint4 sA2[NS > 2 ? UP_BN * CH : 1];
  __shared__ __attribute__((aligned(16))) uint4 sB0[BM * CH];
  __shared__ __attribute__((aligned(16))) uint4 sB1[BM * CH];
  __shared__ __attribute__((aligned(16))) uint4 sB2[NS > 2 ? BM * CH : 1];
  __shared__ int part_cnt[2][32][2];   // K=256: per (wt, token) count of each wave half
  __shared__ int claim_base[NTWG][2];  // staged-backup base per (tile, wt)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 1, wt = wave >> 1;
  const int T = d.T, D = d.D, W = d.W;

  // ---- tile ordering (XCD-aware, grouped along tokens)
  const int nN = d.F / UP_BN;
  const int nM = (T + BM - 1) / BM;
  const int total = nN * nM;
  const int per_xcd = (total + 7) / 8;
  const int P = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (P >= total) return;
  const int grp = P / (UP_GM * nN);
  const int first_m = grp * UP_GM;
  const int gsz = min(nM - first_m, UP_GM);
  const int pin = P - grp * UP_GM * nN;
  const int mb = first_m + pin % gsz;
  const int nb = pin / gsz;
  const int n0 = nb * UP_BN, m0 = mb * BM;

  // ---- main loop
  // A k-slice stage is 256 rows x 2*BK bytes (CH chunks of 16 B); chunk c of row r sits at
  // position c ^ swz(r), swz(r) = r & 7 for CH = 8 and (r >> 2) & 3 for CH = 4, so the 16
  // consecutive rows one fragment read touches land in distinct banks.  Direct
  // global->LDS loads write 64 consecutive 16-byte slots per instruction (RPI rows); lane
  // i fills slot i, so it fetches the logical chunk (i % CH) ^ swz of row i / CH.
  auto swz = [](int r) { return CH == 8 ? (r & 7) : ((r >> 2) & 3); };
  const int lrow = lane / CH;
  const int lchunk = (lane % CH) ^ swz(lrow);
  typedef __attribute__((address_space(3))) void* lds_ptr;
  auto issue = [&](int kt, uint4* sA, uint4* sB) {
    const int k0 = kt * BK + lchunk * 8;
#pragma unroll
    for (int q = 0; q < ALD; ++q) {
      const int blk = wave * ALD + q;
      const int r = blk * RPI + lrow;
      __builtin_amdgcn_global_load_lds(Wu + (size_t)(n0 + r) * D + k0, (lds_ptr)(sA + blk * 64),
                                       16, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < BLD; ++q) {
      const int blk = wave * BLD + q;
      int tok = m0 + blk * RPI + lrow;
      tok = tok < T ? tok : T - 1;
      __builtin_amdgcn_global_load_lds(x + (size_t)tok * D + k0, (lds_ptr)(sB + blk * 64), 16, 0,
                                       0);
    }
  };

  floatx16 acc[4][NB];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][bb][r] = 0.0f;

  const int l32 = lane & 31, lh = lane >> 5;
  // Fragments are double-buffered in registers: the LDS reads of k-step kk+1 are in
  // flight while the MFMAs of step kk run (one wave per SIMD: nothing else hides them).
  auto load_frags = [&](const uint4* A, const uint4* B, int kk, bf16x8_t (&fa)[4],
                        bf16x8_t (&fb)[NB]) {
    const int ch = kk * 2 + lh;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int r = wn * 128 + a * 32 + l32;
      fa[a] = __builtin_bit_cast(bf16x8_t, A[r * CH + (ch ^ swz(r))]);
    }
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const int r = wt * HM + bb * 32 + l32;
      fb[bb] = __builtin_bit_cast(bf16x8_t, B[r * CH + (ch ^ swz(r))]);
    }
  };
  // The k-loop is a ring of NS LDS stages of BK columns, each stage KS = BK/16 MFMA k-steps;
  // the fragments of the next k-step are read while the current one's MFMAs run.  At the
  // last k-step of a stage the next stage is waited for (its loads, and every wave's reads
  // of this stage done: one barrier), the freed buffer is refilled with the stage NS ahead,
  // and the next stage's first fragments are read, all before that k-step's MFMAs.
  constexpr int KS = BK / 16;
  constexpr int LPS = ALD + BLD;  // direct loads per wave per stage
  static_assert(LPS * (NS - 1) <= 63, "vmcnt immediate");
  const int nk = D / BK;          // D % 128 == 0
  bf16x8_t fa[2][4], fb[2][NB];
  auto mfmas = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
        acc[a][bb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][a], fb[c][bb], acc[a][bb], 0, 0, 0);
  };
  // Instruction order of a k-step: its 4*NB MFMAs with the next fragments' LDS reads (and,
  // at a stage's end, the direct loads of the freed buffer and their address arithmetic)
  // placed between them, so the matrix pipe is fed while those issue.
  constexpr int NFR = 4 + NB;  // fragment reads per k-step
  constexpr int NM = 4 * NB;   // MFMAs per k-step
  // (64-token workgroups have fewer MFMAs than reads or loads to place between them: the
  // rest follow without one)
  constexpr int NPR = NFR < NM ? NFR : NM;            // (MFMA, read) pairs
  constexpr int NPL = LPS < NM - 1 ? LPS : NM - 1;    // (MFMA, direct load) pairs
  auto order_step = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NPR; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
    }
    if constexpr (NM > NPR) __builtin_amdgcn_sched_group_barrier(0x008, NM - NPR, 0);
    if constexpr (NFR > NPR) __builtin_amdgcn_sched_group_barrier(0x100, NFR - NPR, 0);
  };
  auto order_boundary = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      if (i < NPL) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU (load addresses)
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM (direct load)
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NFR, 0);  // the next stage's first reads
    if constexpr (NM - NPL - 1 > 0) __builtin_amdgcn_sched_group_barrier(0x008, NM - NPL - 1, 0);
  };
  // Every stage runs the same instructions: the last one also waits, reloads (the last
  // stage again, into a buffer nothing reads) and reads fragments it does not use.  With
  // one path through each stage, and a loop over whole rings of NS stages, the compiler
  // knows at every fragment read which buffers the loads in flight fill, and adds no waits.
  auto stage = [&](int st, uint4* A, uint4* B, const uint4* An, const uint4* Bn)
      __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int c = kk & 1;
      if (kk + 1 < KS) {
        __builtin_amdgcn_sched_barrier(0);
        load_frags(A, B, kk + 1, fa[c ^ 1], fb[c ^ 1]);
        mfmas(c);
        order_step();
        __builtin_amdgcn_sched_barrier(0);
      } else {
        // the next stage is in once only the NS - 2 stages after it may still be loading
        __builtin_amdgcn_s_waitcnt(vmcnt_enc(LPS * (NS - 2)));
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this stage's reads are done
        // a plain barrier: the workgroup fence of __syncthreads would also wait for the
        // loads still in flight (they write LDS); the clobber keeps memory accesses in place
        __asm__ volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        issue(st + NS < nk ? st + NS : nk - 1, A, B);
        load_frags(An, Bn, 0, fa[c ^ 1], fb[c ^ 1]);
        mfmas(c);
        order_boundary();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  issue(0, sA0, sB0);
  issue(1 < nk ? 1 : 0, sA1, sB1);
  if constexpr (NS > 2) issue(2 < nk ? 2 : nk - 1, sA2, sB2);
  __builtin_amdgcn_s_waitcnt(vmcnt_enc(LPS * (NS - 1)));  // stage 0 is in
  __asm__ volatile("s_barrier" ::: "memory");
  load_frags(sA0, sB0, 0, fa[0], fb[0]);
  const int nring = nk / NS * NS;
  for (int st = 0; st < nring; st += NS) {
    stage(st, sA0, sB0, sA1, sB1);
    if constexpr (NS == 2) {
      stage(st + 1, sA1, sB1, sA0, sB0);
    } else {
      stage(st + 1, sA1, sB1, sA2, sB2);
      stage(st + 2, sA2, sB2, sA0, sB0);
    }
  }
  // the last nk % NS stages (the ring position is back at buffer 0)
  if (nring < nk) stage(nring, sA0, sB0, sA1, sB1);
  if constexpr (NS > 2) {
    if (nring + 1 < nk) stage(nring + 1, sA1, sB1, sA2, sB2);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // the repeated loads land before the staging reuses LDS

  // ---- epilogue
  // Own element e = a*16 + r holds wave-local neuron nl = a*32 + 8*(r>>2) + 4*lh + (r&3);
  // e ascending <=> nl ascending among this lane's elements.  The bias is added into the
  // accumulators once (z = acc + b in fp32).
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nl = a * 32 + 8 * q + 4 * lh;
      const uint2 bw = *reinterpret_cast<const uint2*>(bu + n0 + wn * 128 + nl);
      const float bv[4] = {__uint_as_float(bw.x << 16), __uint_as_float(bw.x & 0xFFFF0000u),
                           __uint_as_float(bw.y << 16), __uint_as_float(bw.y & 0xFFFF0000u)};
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[a][bb][4 * q + i] += bv[i];
    }

  // Staging of one 32-token block: region r = (tile slot js, token half w2), r = 2 js + w2,
  // holds [32 tok][W] values (bf16) and [32 tok][W] columns (u8), W <= K.  Columns: all
  // regions in sA1.  Values: with three ring stages (16 KB stages) the regions of w2 = 0 go
  // to sA0 and those of w2 = 1 to sA2, NTWG * 32 * W * 2 bytes each; with two stages (32 KB)
  // all regions fit in sA0.
  static_assert(NS > 2 ? (NTWG * 32 * K * 2 <= (int)sizeof(sA0) && NTWG * 32 * K * 2 <= (int)sizeof(sA2))
                       : (NTWG * 2 * 32 * K * 2 <= (int)sizeof(sA0)),
                "TwELL value staging exceeds its LDS stage at W = K");
  static_assert(NTWG * 2 * 32 * K <= (int)sizeof(sA1), "TwELL column staging exceeds sA1 at W = K");
  uint8_t* st_cols = reinterpret_cast<uint8_t*>(sA1);
  auto st_vals = [&](int js, int w2) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (NS > 2)
      return reinterpret_cast<uint16_t*>(w2 ? sA2 : sA0) + js * 32 * W;
    else
      return reinterpret_cast<uint16_t*>(sA0) + (js * 2 + w2) * 32 * W;
  };
  const int st_cwords = NTWG * 2 * 32 * W / 4;  // 32-bit words of st_cols in use

#pragma unroll
  for (int bb = 0; bb < NB; ++bb) {
    const int tokblk = m0 + wt * HM + bb * 32;  // first token of this 32-token block
    const int tok = tokblk + l32;
    const bool valid = tok < T;
    const int g = tokblk / GROUP;

    // (1) clear the staging block
    __syncthreads();
    if constexpr (NS > 2) {
      for (int q = tid; q < NTWG * 32 * W / 2; q += 256) {
        reinterpret_cast<uint32_t*>(sA0)[q] = 0u;
        reinterpret_cast<uint32_t*>(sA2)[q] = 0u;
      }
    } else {
      for (int q = tid; q < NTWG * 2 * 32 * W / 2; q += 256) reinterpret_cast<uint32_t*>(sA0)[q] = 0u;
    }
    for (int q = tid; q < st_cwords; q += 256) reinterpret_cast<uint32_t*>(st_cols)[q] = 0u;

    // (2) positive mask of this lane's 64 elements
    uint64_t own = 0;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float z = acc[a][bb][r];
        if (DUMP && valid)
          zdump[(size_t)tok * d.F + n0 + wn * 128 + a * 32 + 8 * (r >> 2) + 4 * lh + (r & 3)] = z;
        own |= (uint64_t)(valid && z > 0.0f) << (a * 16 + r);
      }
    const uint32_t pm_lo = __shfl_xor((uint32_t)own, 32);
    const uint32_t pm_hi = __shfl_xor((uint32_t)(own >> 32), 32);
    const uint64_t pm = ((uint64_t)pm_hi << 32) | pm_lo;

    // column union of the block's 32 tokens (one token group): element e = 16 a + 4 q + i
    // of this lane is wave-local neuron 32 a + 8 q + 4 lh + i, so nibble q of the a-th
    // 16 bits of `own` goes to bits 8 q + 4 lh of column word a; OR over all 64 lanes
    {
      uint32_t cw[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const uint32_t f = (uint32_t)(own >> (16 * a)) & 0xFFFFu;
        const uint32_t sp = (f & 0xFu) | ((f & 0xF0u) << 4) | ((f & 0xF00u) << 8) | ((f & 0xF000u) << 12);
        cw[a] = sp << (4 * lh);
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1)
#pragma unroll
        for (int a = 0; a < 4; ++a) cw[a] |= __shfl_xor(cw[a], o);
      if (lane == 0 && tokblk < T) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int n = n0 + wn * 128 + 32 * a;  // first neuron of word a
          ws.umask[((size_t)(n / K) * d.ng + g) * (K / 32) + (n % K) / 32] = cw[a];
        }
      }
    }

    // (3) per tile part: count, rank base, overflow
    // tile part j of this wave covers own/partner bits tmask[j]
    uint64_t tmask[TPW];
    if constexpr (TPW == 2) {
      tmask[0] = 0x00000000FFFFFFFFull;
      tmask[1] = 0xFFFFFFFF00000000ull;
    } else {
      tmask[0] = ~0ull;
    }
    int part[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) part[j] = popc64(own & tmask[j]) + popc64(pm & tmask[j]);
    if constexpr (K == 256) {
      if (lh == 0) part_cnt[wt][l32][wn] = part[0];
    }
    __syncthreads();
    int tot[TPW], rbase[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      if constexpr (K == 256) {
        const int c0 = part_cnt[wt][l32][0], c1 = part_cnt[wt][l32][1];
        tot[j] = c0 + c1;
        rbase[j] = wn ? c0 : 0;
      } else {
        tot[j] = part[j];
        rbase[j] = 0;
      }
    }
    // global tile index and in-workgroup tile slot of part j
    int ktile[TPW], jslot[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      if constexpr (K == 64) jslot[j] = 2 * wn + j;
      else if constexpr (K == 128) jslot[j] = wn;
      else jslot[j] = 0;
      ktile[j] = n0 / K + jslot[j];
    }
    const bool owner = (K != 256) || (wn == 0);
    int lrank[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      const uint64_t om = __ballot(lane < 32 && tot[j] > W);
      lrank[j] = popc64(om & ((1ull << l32) - 1ull));
      const int n_ov = popc64(om);
      if (owner && lane == 0) {
        claim_base[jslot[j]][wt] = n_ov > 0 ? atomicAdd(ws.claim, n_ov) : 0;
        if (tokblk < T) ws.ov_grp[(size_t)ktile[j] * d.ng + g] = n_ov;  // g < ng
      }
    }
    __syncthreads();

    // (4) scatter: main slots into the staging block, remainder into the staged backup
    int slot[TPW];
    bool stage[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      stage[j] = tot[j] > W && d.cap > 0;
      slot[j] = stage[j] ? stage_slot((uint32_t)claim_base[jslot[j]][wt] + (uint32_t)lrank[j], d.cap) : 0;
    }
    int run[TPW];
#pragma unroll
    for (int j = 0; j < TPW; ++j) run[j] = 0;
#pragma unroll
    for (int gi = 0; gi < 16; ++gi) {
      const int j = (TPW == 2) ? (gi >> 3) : 0;
      // partner nonzeros in this tile part at lower columns than this group
      const int shiftp = 4 * (gi + lh);
      const uint64_t pbelow = (shiftp >= 64 ? ~0ull : ((1ull << shiftp) - 1ull)) & tmask[j];
      const int pb = popc64(pm & pbelow);
      uint16_t stbuf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = gi * 4 + i;
        const int a = e >> 4, r = e & 15;
        const float z = acc[a][bb][r];
        const bool nz = (own >> e) & 1ull;
        const int rank = rbase[j] + run[j] + pb;
        run[j] += nz ? 1 : 0;
        const int nl = a * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        int col;
        if constexpr (K == 64) col = nl - 64 * j;
        else if constexpr (K == 128) col = nl;
        else col = wn * 128 + nl;
        const uint16_t zb = f32_to_bf16(z);
        if (nz && rank < W) {
          st_vals(jslot[j], wt)[l32 * W + rank] = zb;
          st_cols[((jslot[j] * 2 + wt) * 32 + l32) * W + rank] = (uint8_t)col;
        }
        stbuf[i] = (nz && rank >= W) ? zb : (uint16_t)0;
      }
      if (stage[j]) {
        // 4 consecutive columns: col of i=0 .. i=3
        const int nl0 = (gi >> 2) * 32 + 8 * (gi & 3) + 4 * lh;
        int col0;
        if constexpr (K == 64) col0 = nl0 - 64 * j;
        else if constexpr (K == 128) col0 = nl0;
        else col0 = wn * 128 + nl0;
        uint2 pk;
        pk.x = (uint32_t)stbuf[0] | ((uint32_t)stbuf[1] << 16);
        pk.y = (uint32_t)stbuf[2] | ((uint32_t)stbuf[3] << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(ws.stage_vals) + (size_t)slot[j] * K + col0) = pk;
      }
    }
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
      if (valid && lh == 0 && owner) {
        b.counts[(size_t)ktile[j] * T + tok] = (uint16_t)tot[j];
        if (stage[j]) {
          ws.stage_key[2 * slot[j]] = ktile[j];
          ws.stage_key[2 * slot[j] + 1] = tok | (lrank[j] << 24);
        }
      }
    }
    __syncthreads();

    // (5) copy the staging block out: for each (tile slot, wt) a contiguous run of
    // nvalid*W values and columns.
#pragma unroll
    for (int js = 0; js < NTWG; ++js)
#pragma unroll
      for (int w2 = 0; w2 < 2; ++w2) {
        const int tb0 = m0 + w2 * HM + bb * 32;
        int nv = T - tb0;
        nv = nv < 0 ? 0 : (nv > 32 ? 32 : nv);
        if (nv == 0) continue;
        const int kt_g = n0 / K + js;
        const size_t gbase = ((size_t)kt_g * T + tb0) * (size_t)W;
        const int sbase = (js * 2 + w2) * 32 * W;  // region of st_cols
        const uint16_t* sv = st_vals(js, w2);
        const int n_el = nv * W;
        uint16_t* gv = static_cast<uint16_t*>(b.vals) + gbase;
        uint8_t* gc = b.cols + gbase;
        if ((W & 7) == 0) {
          for (int q = tid; q < n_el / 8; q += 256)
            reinterpret_cast<uint4*>(gv)[q] = reinterpret_cast<const uint4*>(sv)[q];
        } else {
          for (int q = tid; q < n_el; q += 256) gv[q] = sv[q];
        }
        if ((W & 15) == 0) {
          for (int q = tid; q < n_el / 16; q += 256)
            reinterpret_cast<uint4*>(gc)[q] = reinterpret_cast<const uint4*>(st_cols + sbase)[q];
        } else {
          for (int q = tid; q < n_el; q += 256) gc[q] = st_cols[sbase + q];
        }
      }
  }
}

template <int K, int NB, int BK = 64, int WPE = 1, int NS = 2>
static hipError_t launch_up_t(const Dims& d, const uint16_t* x, const uint16_t* Wu,
                              const uint16_t* bu, const twell_buffers_t& b, const Workspace& ws,
                              float* zdump, hipStream_t s) {
  constexpr int BM = 64 * NB;
  const int nN = d.F / UP_BN;
  const int nM = (d.T + BM - 1) / BM;
  const int total = nN * nM;
  const int per_xcd = (total + 7) / 8;
  if (zdump)
    hipLaunchKernelGGL((up_pack_bf16_kernel<K, NB, true, BK, WPE, NS>), dim3(8 * per_xcd), dim3(256), 0, s, d,
                       x, Wu, bu, b, ws, zdump);
  else
    hipLaunchKernelGGL((up_pack_bf16_kernel<K, NB, false, BK, WPE, NS>), dim3(8 * per_xcd), dim3(256), 0, s,
                       d, x, Wu, bu, b, ws, zdump);
  return hipGetLastError();
}

hipError_t launch_up_pack_bf16(const Dims& d, const uint16_t* x, const uint16_t* Wu,
                               const uint16_t* bu, const twell_buffers_t& b,
                               const Workspace& ws, float* zdump, hipStream_t s) {
  // 128-token workgroups, two per CU (BK = 32); K = 64 keeps one per CU (its staging of
  // four tiles needs the larger LDS stages).  When the 128-token workgroups would not cover
  // the CUs (a few hundred tokens), 64-token ones: twice the workgroups, each with half the
  // MFMAs for the same W_up slice.
  const bool few = (long long)(d.F / UP_BN) * ((d.T + 127) / 128) < 256;
  switch (d.K) {
    case 64: return launch_up_t<64, 2>(d, x, Wu, bu, b, ws, zdump, s);
    case 128:
      return few ? launch_up_t<128, 1, 32, 2, 3>(d, x, Wu, bu, b, ws, zdump, s)
                 : launch_up_t<128, 2, 32, 2, 3>(d, x, Wu, bu, b, ws, zdump, s);
    case 256:
      return few ? launch_up_t<256, 1, 32, 2, 3>(d, x, Wu, bu, b, ws, zdump, s)
                 : launch_up_t<256, 2, 32, 2, 3>(d, x, Wu, bu, b, ws, zdump, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sffn
