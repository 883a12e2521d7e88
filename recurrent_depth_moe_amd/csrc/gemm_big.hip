// Large-tile bf16 GEMM for the prefill products (QKV, O, shared and routed
// experts) on gfx950.
//
// Block tile 256 x 256, four wave64s in 2x2, each wave owns 128 x 128 of
// the output (16 accumulators of v_mfma_f32_32x32x16_bf16; measured on
// MI355X the 32x32x16 form sustains about 2.06 PFLOP/s even at one wave per
// SIMD, where 16x16x32 needs many more independent chains).  Tiles reach
// LDS with global_load_lds_dwordx4 (no register staging): lane i of a load
// fills 16-byte LDS slot i of its 1 KB window, so the XOR swizzle of the
// 16-byte chunks inside a row (chunk ^ ((row >> 1) & 7)) is applied on the
// source side by choosing which global chunk each lane fetches.
//
// The k loop runs over 64-deep stages, so every load takes whole 128-byte
// lines of A and B (a 32-deep stage would touch each line twice, and the
// measured L2->LDS throughput halves); two stages of 64 KB alternate.  A
// stage is consumed in two 32-deep halves from registers: while the MFMAs
// of one half run, the fragments of the next half are read from LDS, and
// the load of stage k+2 is issued once every wave has finished reading
// stage k (one barrier per stage).  Loads and fragment reads are spread
// between the MFMAs (sched_group_barrier), since with one wave per SIMD no
// other wave fills the issue slots.
//
// For the fused gate|up product the B tile holds 128 gate rows and the same
// 128 up rows, interleaved per wave column (gate 0-63, up 0-63, gate 64-127,
// up 64-127) so a wave holds the gate and up values of the same outputs.
//
// Ragged routed tiles compute all 256 rows (rows past the group's end are
// loaded from a valid row and never stored): a data-dependent skip of row
// fragments inside the stage makes the register allocator spill the
// accumulators.
#include "gemm_device.h"

#include <type_traits>

namespace {

// Issue order of the first half of a stage: a fragment read of the second
// half after each of the first MFMAs (NM MFMAs, ND fragment reads).
template <int NM, int ND>
__device__ __forceinline__ void interleave_first_half() {
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NM - ND, 0);
}
// Second half: the NV global->LDS loads of the next stages first (their
// latency is what the pipeline must hide), then the reads of the next
// stage's first half, one after each MFMA.
template <int NM, int ND, int NV>
__device__ __forceinline__ void interleave_second_half() {
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // VMEM
  }
#pragma unroll
  for (int i = 0; i < ND; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
  }
  if constexpr (NM > NV + ND) __builtin_amdgcn_sched_group_barrier(0x008, NM - NV - ND, 0);
}

constexpr int BK = 64;                               // k depth of one LDS stage
constexpr int NSTAGE = 2;                            // LDS stages
constexpr int LDS_BYTES = 160 * 1024;                // two 64 KB stages; short tiles use it all
constexpr int EP_LD = 128 + 4;                      // epilogue patch row stride (floats)
static_assert(4 * 32 * EP_LD * 4 <= LDS_BYTES, "epilogue patches fit in the tile LDS");

// One 32x32 accumulator into columns 32 j .. 32 j + 31 of a wave's
// row-major fp32 patch.  The MFMAs take their operands in (B, A) order, so
// lane l holds output row l % 32 and, in elements 4g .. 4g+3, the four
// consecutive columns 8g + 4 (l / 32) .. +3: one 16-byte LDS write each
// (rows 528 bytes apart, so sixteen lanes cover all 64 banks once).
__device__ __forceinline__ void patch_write(float* ep, int lane, int j, const floatx16_t& a) {
  float* row = ep + (lane & 31) * EP_LD + j * 32 + 4 * (lane >> 5);
#pragma unroll
  for (int g = 0; g < 4; ++g) *(float4*)(row + 8 * g) = make_float4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
}

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void g2lds(const void* src, uint4* lds_slot0) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds_slot0, 16, 0, 0);
}

// Fragments of one 32-deep half (hh = 0, 1) of a 64-deep stage for this
// wave, for v_mfma_f32_32x32x16_bf16 (two 16-deep k-steps): FMW A fragments
// (32 rows each) and WNF B fragments (32 columns each) per k-step; lane l
// holds row/column l % 32 and k values 8 * (l / 32) .. +7 of the k-step.
// Rows hold 8 chunks of 8 k (128 bytes); chunk c of row r sits at position
// c ^ ((r >> 1) & 7), so the 8 rows a quarter-wave reads land in distinct
// banks.
template <int WNF, int FMW>
__device__ __forceinline__ void read_frags(const uint4* sA, const uint4* sB, int wm, int wn, int lane, int hh,
                                           bf16x8_t (&af)[2 * FMW], bf16x8_t (&bf)[2 * WNF]) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int c = 4 * hh + 2 * s + (lane >> 5);
#pragma unroll
    for (int j = 0; j < WNF; ++j) {
      const int r = wn * (32 * WNF) + j * 32 + (lane & 31);
      bf[s * WNF + j] = __builtin_bit_cast(bf16x8_t, sB[r * 8 + (c ^ ((r >> 1) & 7))]);
    }
#pragma unroll
    for (int i = 0; i < FMW; ++i) {
      const int r = wm * (32 * FMW) + i * 32 + (lane & 31);
      af[s * FMW + i] = __builtin_bit_cast(bf16x8_t, sA[r * 8 + (c ^ ((r >> 1) & 7))]);
    }
  }
}

template <int WNF, int FMW>
__device__ __forceinline__ void mfma_stage(const bf16x8_t (&af)[2 * FMW], const bf16x8_t (&bf)[2 * WNF],
                                           floatx16_t (&acc)[FMW][WNF]) {
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < FMW; ++i)
#pragma unroll
      for (int j = 0; j < WNF; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[s * WNF + j], af[s * FMW + i], acc[i][j], 0, 0, 0);
}

// wait until at most `n` direct-to-LDS loads of this wave are in flight
__device__ __forceinline__ void wait_vm(int n) {
  // s_waitcnt: vmcnt in bits [3:0] and [15:14], expcnt and lgkmcnt left at max
  if (n >= 16) __builtin_amdgcn_s_waitcnt(0x4F70);
  else if (n >= 8) __builtin_amdgcn_s_waitcnt(0x0F78);
  else __builtin_amdgcn_s_waitcnt(0x0F70);
}

// s_waitcnt lgkmcnt(0) with vmcnt and expcnt left at max: the epilogues
// pass accumulators between lanes through LDS and wait for those LDS
// accesses only, so the global stores of one 32-row pass stay in flight
// while the next pass runs
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left at max
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// A tile with at most SR (64 or 128) valid rows: the tail of a routed
// expert's rows, or the last rows of a dense product.  Only A rows 0..SR-1
// are loaded and each wave computes those rows for 64 of the columns (for
// gate|up: 32 gate and the matching 32 up columns), so the tile costs
// SR/256 of a full tile's MFMAs.  192-column tiles (WNF = 3) give waves 0-2
// 64 columns each; wave 3 repeats wave 2's columns and stores nothing, so
// every wave issues the same instructions.  With so little math per stage
// the loads set the pace, so the smaller stages (A 8 or 16 KB + B 24 or 32
// KB) run in a deeper ring: 4 stages for 64 rows, 3 for 128.
template <int SR, bool DUAL, int EPI, typename TO, int WNF>
__device__ __forceinline__ void small_tile(const GemmParams& p, uint4* smem, const bf16_t* const* asrc,
                                           const bf16_t* const (&bsrc)[2 * WNF], int w, int lane, int rows,
                                           int row0, int n0, int KT) {
  static_assert(WNF == 4 || (WNF == 3 && !DUAL), "gate|up tiles are 256 columns wide");
  constexpr int FM = SR / 32;                  // 32-row fragments
  constexpr int SA_IT = SR / 32;               // A rows 0..SR-1 sit in LDS slots 0..SR*8-1
  constexpr int B_IT = 2 * WNF;                // B rows 64 WNF: 512 WNF chunks over 256 threads
  constexpr int IT = SA_IT + B_IT;             // loads per thread and stage
  constexpr int SA_CH = SR * 8, STG = SA_CH + 512 * WNF;
  constexpr int NS = SR == 64 ? 4 : 3;
  static_assert(NS * STG * 16 <= LDS_BYTES, "stages fit in LDS");
  auto issue = [&](int stage, int k0) {
    uint4* base = smem + stage * STG;
#pragma unroll
    for (int j = 0; j < SA_IT; ++j) g2lds(asrc[j] + k0, base + (j * 4 + w) * 64);
#pragma unroll
    for (int j = 0; j < B_IT; ++j) g2lds(bsrc[j] + k0, base + SA_CH + (j * 4 + w) * 64);
  };
  const int wc = WNF == 3 ? min(w, 2) : w;    // this wave's 64-column group
  const bool wstore = WNF == 4 || w < 3;
  const int brow0 = DUAL ? (w >> 1) * 128 + (w & 1) * 32 : 64 * wc;
  const int brow1 = DUAL ? brow0 + 64 : brow0 + 32;
  auto read = [&](int stage, int hh, bf16x8_t (&af)[2 * FM], bf16x8_t (&bf)[4]) {
    const uint4* sA = smem + stage * STG;
    const uint4* sB = sA + SA_CH;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int c = 4 * hh + 2 * s + (lane >> 5);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = i * 32 + (lane & 31);
        af[s * FM + i] = __builtin_bit_cast(bf16x8_t, sA[r * 8 + (c ^ ((r >> 1) & 7))]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int rb = (j ? brow1 : brow0) + (lane & 31);
        bf[s * 2 + j] = __builtin_bit_cast(bf16x8_t, sB[rb * 8 + (c ^ ((rb >> 1) & 7))]);
      }
    }
  };
  floatx16_t acc[FM][2];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  auto mfma = [&](const bf16x8_t (&af)[2 * FM], const bf16x8_t (&bf)[4]) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[s * 2 + j], af[s * FM + i], acc[i][j], 0, 0, 0);
  };
  // every buffer loading (past the end of K: repeats of the last stage)
#pragma unroll
  for (int st = 0; st < NS; ++st) issue(st, min(st, KT - 1) * BK);
  bf16x8_t a0[2 * FM], b0[4], a1[2 * FM], b1[4];
  wait_vmcnt<(NS - 1) * IT>();
  __syncthreads();
  read(0, 0, a0, b0);
  for (int kt = 0; kt < KT; ++kt) {
    read(kt % NS, 1, a1, b1);
    mfma(a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    // stage kt+1 landed; every wave is done with stage kt, whose buffer
    // takes stage kt+NS
    wait_vmcnt<(NS - 2) * IT>();
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    issue(kt % NS, min(kt + NS, KT - 1) * BK);
    read((kt + 1) % NS, 0, a0, b0);
    mfma(a1, b1);
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vmcnt<0>();
  __syncthreads();
  // epilogue: FM passes of 32 rows through a 32 x 64 patch per wave
  float* ep = (float*)smem + w * (32 * EP_LD);
#pragma unroll
  for (int pass = 0; pass < FM; ++pass) {
    if (pass * 32 < rows) {
#pragma unroll
      for (int j = 0; j < 2; ++j) patch_write(ep, lane, j, acc[pass][j]);
      wait_lgkm0();
      __builtin_amdgcn_wave_barrier();
      if constexpr (DUAL) {
        // 32 output columns: gate at patch columns 0..31, up at 32..63
#pragma unroll 1
        for (int it = 0; it < 2; ++it) {
          const int rl = it * 16 + (lane >> 2), c8 = (lane & 3) * 8;
          const int ml = pass * 32 + rl;
          float g[8], u[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            g[x] = ep[rl * EP_LD + c8 + x];
            u[x] = ep[rl * EP_LD + 32 + c8 + x];
          }
          if (ml < rows) epi_store8<EPI, TO>(p.epi, p.N, row0 + ml, n0 + 32 * w + c8, g, u);
        }
      } else {
#pragma unroll 1
        for (int it = 0; it < 4; ++it) {
          const int rl = it * 8 + (lane >> 3), c8 = (lane & 7) * 8;
          const int ml = pass * 32 + rl;
          float val[8];
#pragma unroll
          for (int x = 0; x < 8; ++x) val[x] = ep[rl * EP_LD + c8 + x];
          if (ml < rows && wstore) epi_store8<EPI, TO>(p.epi, p.N, row0 + ml, n0 + 64 * wc + c8, val, val);
        }
      }
      wait_lgkm0();
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();   // the next tile's loads reuse this LDS
}

// WNF = 32-column fragments per wave: 4 (256-column tiles) or 3 (192, for
// dense products whose 256-column tile count leaves the last round of CUs
// half idle)
template <bool DUAL, int EPI, typename TO, int WNF>
__global__ __launch_bounds__(256, 1) void gemm_bf16_big_kernel(GemmParams p) {
  static_assert(WNF == 4 || (WNF == 3 && !DUAL), "gate|up tiles are 256 columns wide");
  RDT_SKIP_IF_ALL_HALTED(p.live);
  constexpr int BM = 256, BN = 64 * WNF;
  constexpr int WTM = 128, WTN = 32 * WNF;
  constexpr int A_CH = BM * (BK / 8), B_CH = BN * (BK / 8);   // 16-byte chunks per stage
  constexpr int A_IT = A_CH / 256, B_IT = B_CH / 256;
  // 192-column single-B tiles also take up to two 32-row strips past the
  // 256 rows (the remainder of a routed expert's rows in a merged
  // schedule): their A rows follow the tile's in each A stage, and they
  // reuse the B fragments the waves already hold, so the expert's weights
  // stream once
  constexpr bool HAS_STRIP = WNF == 3 && !DUAL;
  constexpr int SROWS = HAS_STRIP ? 64 : 0;
  constexpr int A_CHS = (BM + SROWS) * (BK / 8), A_ITS = A_CHS / 256;   // A stage stride / loads with the strip
  static_assert((2 * A_CHS + 3 * B_CH) * 16 <= LDS_BYTES, "stages fit in LDS");
  constexpr int NCOL = DUAL ? BN / 2 : BN;       // output columns per tile
  extern __shared__ uint4 smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int ntn = (p.N + NCOL - 1) / NCOL;
  const int n_mt = p.mt_start ? p.mt_start[p.n_groups] : (p.M + BM - 1) / BM;
  const int total = n_mt * ntn;
  const int per_xcd = gridDim.x / RDT_NUM_XCD;
  const int xcd = blockIdx.x % RDT_NUM_XCD, slot = blockIdx.x / RDT_NUM_XCD;
  const int chunk = (total + RDT_NUM_XCD - 1) / RDT_NUM_XCD;
  const int t_end = min(total, (xcd + 1) * chunk);
  const bf16_t* Abase = (const bf16_t*)p.A;
  const int KT = p.K / BK;

  // XCD x owns tiles [x * chunk, (x + 1) * chunk), so tiles that share an
  // A or B panel meet in one L2.  Static order: slot s of the XCD takes
  // every per_xcd-th work unit of its share, a unit being a whole tile or,
  // when the share's last round would leave at least half of the XCD's
  // blocks idle (e.g. 640 QKV tiles on 256 CUs), one 128-row half of each
  // of the share's last tiles: every block then ends with a half-cost unit
  // instead of half the blocks with a whole one.  Claimed order (tile_ctr): blocks
  // take their XCD's tiles one at a time from its counter, then help the
  // other XCDs in turn, so tiles of unequal cost (the short tail tiles of
  // routed experts) level out over the CUs.  The claimed tile index passes
  // through LDS word 0, which no tile uses between its closing barrier and
  // the next tile's first load.
  const int c0 = xcd * chunk, cnt = max(0, t_end - c0);
  const int rem = cnt % per_xcd;
  const int n_split = (p.tile_ctr == nullptr && p.mt_start == nullptr && rem > 0 && 2 * rem <= per_xcd) ? rem : 0;
  const int n_whole = cnt - n_split, n_units = n_whole + 2 * n_split;
  int src = xcd;   // claimed order: the share thread 0 currently draws from
  auto next_tile = [&](int L) -> int {
    if (p.tile_ctr == nullptr) {
      L = L < 0 ? slot : L + per_xcd;   // a unit of this XCD's share
      return L < n_units ? L : -1;
    }
    int* const bc = (int*)smem;
    if (tid == 0) {
      int got = -1;
      for (int tries = 0; tries < RDT_NUM_XCD && got < 0; ++tries) {
        const int c0 = src * chunk, c1 = min(total, c0 + chunk);
        if (c0 < c1) {
          const int i = atomicAdd(p.tile_ctr + src, 1);
          if (c0 + i < c1) got = c0 + i;
        }
        if (got < 0) src = src + 1 == RDT_NUM_XCD ? 0 : src + 1;
      }
      *bc = got;
    }
    __syncthreads();
    const int got = __builtin_amdgcn_readfirstlane(*(volatile int*)bc);
    __syncthreads();
    return got;
  };

  for (int U = next_tile(-1); U >= 0; U = next_tile(U)) {
    // unit -> tile (and half: -1 for a whole tile)
    int L = U, half = -1;
    if (p.tile_ctr == nullptr) {
      L = c0 + (U < n_whole ? U : n_whole + ((U - n_whole) >> 1));
      if (U >= n_whole) half = (U - n_whole) & 1;
    }
    int mt, nt, row0, rows, grp;
    tile_coords(p, L, ntn, n_mt, mt, nt);
    tile_rows(p, mt, BM, row0, rows, grp);
    if (half >= 0) {
      row0 += 128 * half;
      rows = min(rows - 128 * half, 128);
      if (rows <= 0) continue;   // (uniform: a tile of at most 128 rows has no second half)
    }
    const int n0 = nt * NCOL;
    const bf16_t* W0 = (const bf16_t*)p.W0 + (int64_t)grp * p.w_stride;
    const bf16_t* W1 = DUAL ? (const bf16_t*)p.W1 + (int64_t)grp * p.w_stride : W0;

    // source pointers of this thread's chunks (k offset added per stage):
    // LDS slot s = (j*4 + w)*64 + lane holds row s/8, logical chunk
    // (s%8) ^ ((row >> 1) & 7)
    const bf16_t* asrc[A_ITS];
#pragma unroll
    for (int j = 0; j < A_ITS; ++j) {
      const int s = (j * 4 + w) * 64 + lane, r = s >> 3, c = (s & 7) ^ ((r >> 1) & 7);
      const int m = row0 + (r < rows ? r : 0);
      const int arow = p.a_rows ? p.a_rows[m] : m;
      asrc[j] = Abase + (int64_t)arow * p.lda + c * 8;
    }
    const bf16_t* bsrc[B_IT];
#pragma unroll
    for (int j = 0; j < B_IT; ++j) {
      const int s = (j * 4 + w) * 64 + lane, r = s >> 3, c = (s & 7) ^ ((r >> 1) & 7);
      const bf16_t* Wsel = W0;
      int col;
      if constexpr (DUAL) {
        // row r: wave column r/128, gate (r%128 < 64) or up, column within 64
        Wsel = ((r & 127) < 64) ? W0 : W1;
        col = (r >> 7) * 64 + (r & 63);
      } else {
        col = r;
      }
      const int n = n0 + col < p.N ? n0 + col : 0;
      bsrc[j] = Wsel + (int64_t)n * p.K + c * 8;
    }

    // LDS: A stages in a ring of 2 (A rows are shared by every n-tile of
    // the rows, so they come from L2), B stages in a ring of 3 (a routed
    // expert's weights stream from HBM, so they are requested one stage
    // earlier)
    uint4* const sAbuf = smem;
    uint4* const sBbuf = smem + 2 * A_CHS;
    auto issueA = [&](int buf, int k0, auto n_c) {
      constexpr int n = decltype(n_c)::value;   // A_IT (+ one per 32-row strip), or fewer for a 192-row tile
#pragma unroll
      for (int j = 0; j < n; ++j) g2lds(asrc[j] + k0, sAbuf + buf * A_CHS + (j * 4 + w) * 64);
    };
    auto issueB = [&](int buf, int k0) {
#pragma unroll
      for (int j = 0; j < B_IT; ++j) g2lds(bsrc[j] + k0, sBbuf + buf * B_CH + (j * 4 + w) * 64);
    };

    if constexpr (EPI != EPI_QKV) {   // (QKV rows come in full tiles but the last; its epilogue is the heaviest)
      if (rows <= 64) {
        small_tile<64, DUAL, EPI, TO, WNF>(p, smem, asrc, bsrc, w, lane, rows, row0, n0, KT);
        continue;
      }
      if (rows <= 128) {
        small_tile<128, DUAL, EPI, TO, WNF>(p, smem, asrc, bsrc, w, lane, rows, row0, n0, KT);
        continue;
      }
    }

    auto full_tile = [&](auto strip_c, auto fmw_c) {
      constexpr int NSTR = decltype(strip_c)::value;   // 32-row strips (0, 1, 2)
      constexpr int FMW = decltype(fmw_c)::value;      // 32-row fragments per wave: 4 (256-row tile) or 3 (192)
      constexpr int WTMF = 32 * FMW;                   // rows per wave
      constexpr int A_ITF = 2 * FMW;                   // A loads per thread and stage (rows 0 .. 64 FMW - 1)
      static_assert(FMW == 4 || NSTR == 0, "strips follow 256-row tiles");
      constexpr std::integral_constant<int, A_ITF + NSTR> na_c{};
      constexpr bool S = NSTR > 0;
      constexpr int NMS = 4 * NSTR, NDS = 2 * NSTR;   // strip MFMAs / fragment reads per half stage
      constexpr int NSA = NSTR > 0 ? NSTR : 1;        // array extents
      floatx16_t acc[FMW][WNF];
#pragma unroll
      for (int i = 0; i < FMW; ++i)
#pragma unroll
        for (int j = 0; j < WNF; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
      // strip st: 32 rows x this wave's B fragments 0 and 1 (wm = 0) or 2
      // (wm = 1; its second accumulator repeats fragment 2 and is never
      // stored, so every wave issues the same MFMAs)
      floatx16_t accs[NSA][2];
#pragma unroll
      for (int st = 0; st < NSA; ++st)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) accs[st][j][e] = 0.f;
      auto read_strip = [&](const uint4* sA, int hh, bf16x8_t (&fs)[NSA][2]) {
#pragma unroll
        for (int st = 0; st < NSTR; ++st)
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const int c = 4 * hh + 2 * x + (lane >> 5), r = BM + 32 * st + (lane & 31);
            fs[st][x] = __builtin_bit_cast(bf16x8_t, sA[r * 8 + (c ^ ((r >> 1) & 7))]);
          }
      };
      auto strip_mfma = [&](const bf16x8_t (&fs)[NSA][2], const bf16x8_t (&fb)[2 * WNF]) {
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const bf16x8_t b0 = wm ? fb[x * WNF + 2] : fb[x * WNF + 0];
          const bf16x8_t b1 = wm ? fb[x * WNF + 2] : fb[x * WNF + 1];
#pragma unroll
          for (int st = 0; st < NSTR; ++st) {
            accs[st][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0, fs[st][x], accs[st][0], 0, 0, 0);
            accs[st][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1, fs[st][x], accs[st][1], 0, 0, 0);
          }
        }
      };
      // 32-row fragments of this wave that hold at least one valid row
      const int fm_valid = max(0, min(FMW, (rows - wm * WTMF + 31) / 32));

      // prologue: A stages 0, 1 and B stages 0, 1, 2 in flight, first half
      // of stage 0 read (past the end of K, loads repeat the last stage into
      // a buffer nobody reads)
      issueA(0, 0, na_c);
      issueB(0, 0);
      issueA(1, min(1, KT - 1) * BK, na_c);
      issueB(1, min(1, KT - 1) * BK);
      issueB(2, min(2, KT - 1) * BK);
      bf16x8_t fa0[2 * FMW], fb0[2 * WNF], fa1[2 * FMW], fb1[2 * WNF], fs0[NSA][2], fs1[NSA][2];
      wait_vmcnt<A_ITF + NSTR + 2 * B_IT>();
      __syncthreads();
      read_frags<WNF, FMW>(sAbuf, sBbuf, wm, wn, lane, 0, fa0, fb0);
      if constexpr (S) read_strip(sAbuf, 0, fs0);
      int b3 = 0;   // kt % 3
      for (int kt = 0; kt < KT; ++kt) {
        const int b3n = b3 == 2 ? 0 : b3 + 1;
        {
          // first half of stage kt (registers fa0/fb0); read its second half
          read_frags<WNF, FMW>(sAbuf + (kt & 1) * A_CHS, sBbuf + b3 * B_CH, wm, wn, lane, 1, fa1, fb1);
          if constexpr (S) read_strip(sAbuf + (kt & 1) * A_CHS, 1, fs1);
          mfma_stage<WNF, FMW>(fa0, fb0, acc);
          if constexpr (S) strip_mfma(fs0, fb0);
          interleave_first_half<2 * FMW * WNF + NMS, 2 * FMW + 2 * WNF + NDS>();
          __builtin_amdgcn_sched_barrier(0);
        }
        {
          // second half: stage kt+1 landed (only B of stage kt+2 may still be
          // in flight) and every wave is done reading stage kt, so its
          // buffers take A of stage kt+2 and B of stage kt+3; read stage
          // kt+1's first half (past the end: unused)
          wait_vmcnt<B_IT>();
          __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
          __syncthreads();
          __builtin_amdgcn_sched_barrier(0);
          issueA(kt & 1, min(kt + 2, KT - 1) * BK, na_c);
          issueB(b3, min(kt + 3, KT - 1) * BK);
          read_frags<WNF, FMW>(sAbuf + ((kt + 1) & 1) * A_CHS, sBbuf + b3n * B_CH, wm, wn, lane, 0, fa0, fb0);
          if constexpr (S) read_strip(sAbuf + ((kt + 1) & 1) * A_CHS, 0, fs0);
          mfma_stage<WNF, FMW>(fa1, fb1, acc);
          if constexpr (S) strip_mfma(fs1, fb1);
          interleave_second_half<2 * FMW * WNF + NMS, 2 * FMW + 2 * WNF + NDS, A_ITF + NSTR + B_IT>();
          __builtin_amdgcn_sched_barrier(0);
        }
        b3 = b3n;
      }
      wait_vm(0);   // the trailing reloads land before the epilogue reuses LDS
      __syncthreads();   // every wave done with the stages before the epilogue reuses LDS

      // Epilogue through LDS, one pass of 32 rows per wave fragment row:
      // the accumulators go to a row-major 32 x 128 fp32 patch of the
      // wave's own LDS region with 16-byte writes straight from the
      // accumulator registers (patch_write), then each lane takes 8
      // consecutive columns of one row, so stores are 16-byte vectors and
      // RoPE pairs sit in one lane.
      {
        float* ep = (float*)smem + w * (32 * EP_LD);
#pragma unroll
        for (int pass = 0; pass < FMW; ++pass) {
          if (pass < fm_valid) {
#pragma unroll
            for (int j = 0; j < WNF; ++j) patch_write(ep, lane, j, acc[pass][j]);
            wait_lgkm0();
            __builtin_amdgcn_wave_barrier();
            if constexpr (DUAL) {
              // 64 output columns: gate at patch columns 0..63, up at 64..127
#pragma unroll 1
              for (int it = 0; it < 4; ++it) {
                const int rl = it * 8 + (lane >> 3), c8 = (lane & 7) * 8;
                const int ml = wm * WTMF + pass * 32 + rl;
                float g[8], u[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) {
                  g[x] = ep[rl * EP_LD + c8 + x];
                  u[x] = ep[rl * EP_LD + 64 + c8 + x];
                }
                if (ml < rows) epi_store8<EPI, TO>(p.epi, p.N, row0 + ml, n0 + wn * 64 + c8, g, u);
              }
            } else if (EPI == EPI_QKV && n0 + wn * WTN >= p.epi.H * p.epi.dq + p.epi.G * p.epi.dq) {
              // every column of this wave is a V channel, stored transposed
              // (V^T [b][g][d][position]): a lane takes 8 consecutive rows of
              // one column and stores them as one 16-byte run of positions
              const EpiParams& e = p.epi;
              const int hqk = e.H * e.dq + e.G * e.dq;
#pragma unroll 1
              for (int it = 0; it < 32 * WTN / (8 * 64); ++it) {
                const int idx = it * 64 + lane, c = idx % WTN, rg = idx / WTN;
                const int ml = wm * WTMF + pass * 32 + rg * 8;
                const int n = n0 + wn * WTN + c;
                if (ml >= rows || n >= p.N) continue;
                const int m = row0 + ml, mp = e.tok ? e.tok[m] : m, b = mp / e.T, i = mp - b * e.T;
                const int nn = n - hqk, g = nn / e.dv, d = nn - g * e.dv;
                TO* col = (TO*)e.vt + ((int64_t)(b * e.G + g) * e.dv + d) * e.cap + e.kbase + i;
                float v[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) v[x] = ep[(rg * 8 + x) * EP_LD + c];
                if (!e.tok && ml + 8 <= rows && i + 8 <= e.T && ((e.kbase + i) & 7) == 0) {
                  store8<EPI, TO>(col, v);
                } else {
                  // rows past the tile, a sequence boundary, an unaligned run
                  // or positions from a map
                  for (int x = 0; x < 8 && ml + x < rows; ++x) {
                    const int mx = e.tok ? e.tok[m + x] : m + x, bx = mx / e.T, ix = mx - bx * e.T;
                    St<TO>::st((TO*)e.vt + ((int64_t)(bx * e.G + g) * e.dv + d) * e.cap + e.kbase + ix, v[x]);
                  }
                }
              }
            } else {
              // 32 rows x WTN columns in groups of 8 columns, one group per lane
              constexpr int CG = WTN / 8, NIT = 32 * CG / 64;
              if constexpr (EPI == EPI_RESID) {
                // the residual rows of PG groups are requested before their
                // stores, so the load latencies overlap instead of each store
                // waiting on its own
                const EpiParams& e = p.epi;
                constexpr int PG = NIT % 4 == 0 ? 4 : 3;   // 8 groups per pass (256 columns) or 6 (192)
                static_assert(NIT % PG == 0, "whole load batches per pass");
#pragma unroll 1
                for (int g0 = 0; g0 < NIT; g0 += PG) {
                  float4 r[PG][2];
#pragma unroll
                  for (int u = 0; u < PG; ++u) {
                    const int idx = (g0 + u) * 64 + lane, rl = idx / CG, c8 = (idx - rl * CG) * 8;
                    const int ml = wm * WTMF + pass * 32 + rl, n = n0 + wn * WTN + c8;
                    r[u][0] = r[u][1] = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (ml < rows && n + 8 <= p.N) {
                      const float* src = e.resid + (int64_t)(row0 + ml) * e.ldo + n;
                      r[u][0] = *(const float4*)src;
                      r[u][1] = *(const float4*)(src + 4);
                    }
                  }
#pragma unroll
                  for (int u = 0; u < PG; ++u) {
                    const int idx = (g0 + u) * 64 + lane, rl = idx / CG, c8 = (idx - rl * CG) * 8;
                    const int ml = wm * WTMF + pass * 32 + rl, n = n0 + wn * WTN + c8;
                    if (ml >= rows) continue;
                    float v[8];
#pragma unroll
                    for (int x = 0; x < 8; ++x) v[x] = ep[rl * EP_LD + c8 + x];
                    if (n + 8 > p.N) {
                      epi_store8<EPI, TO>(e, p.N, row0 + ml, n, v, v);   // ragged column end
                    } else {
                      const float o[8] = {r[u][0].x + v[0], r[u][0].y + v[1], r[u][0].z + v[2], r[u][0].w + v[3],
                                          r[u][1].x + v[4], r[u][1].y + v[5], r[u][1].z + v[6], r[u][1].w + v[7]};
                      store8<EPI, float>((float*)e.out + (int64_t)(row0 + ml) * e.ldo + n, o);
                    }
                  }
                }
              } else {
#pragma unroll 1
                for (int it = 0; it < NIT; ++it) {
                  const int idx = it * 64 + lane, rl = idx / CG, c8 = (idx - rl * CG) * 8;
                  const int ml = wm * WTMF + pass * 32 + rl;
                  float v[8];
#pragma unroll
                  for (int x = 0; x < 8; ++x) v[x] = ep[rl * EP_LD + c8 + x];
                  if (ml < rows) epi_store8<EPI, TO>(p.epi, p.N, row0 + ml, n0 + wn * WTN + c8, v, v);
                }
              }
            }
            wait_lgkm0();
            __builtin_amdgcn_wave_barrier();
          }
        }
        if constexpr (S) {
          // strip rows 256 .. rows-1: per strip 32 x 64 (wm = 0) or 32 x 32
          // (wm = 1) columns
          const int cg = wm ? 4 : 8, ncol0 = n0 + wn * WTN + (wm ? 64 : 0);
#pragma unroll
          for (int st = 0; st < NSTR; ++st) {
#pragma unroll
            for (int j = 0; j < 2; ++j) patch_write(ep, lane, j, accs[st][j]);
            wait_lgkm0();
            __builtin_amdgcn_wave_barrier();
#pragma unroll 1
            for (int it = 0; it < 4; ++it) {
              const int idx = it * 64 + lane, rl = idx / cg, c8 = (idx - rl * cg) * 8;
              const int ml = BM + 32 * st + rl;
              if (rl < 32 && ml < rows) {
                float v[8];
#pragma unroll
                for (int x = 0; x < 8; ++x) v[x] = ep[rl * EP_LD + c8 + x];
                epi_store8<EPI, TO>(p.epi, p.N, row0 + ml, ncol0 + c8, v, v);
              }
            }
            wait_lgkm0();
            __builtin_amdgcn_wave_barrier();
          }
        }
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using F4 = std::integral_constant<int, 4>;
    constexpr bool ROUTED = EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE || EPI == EPI_STORE;   // the routed expert products
    if (ROUTED && rows <= 192) {
      // 129-192 rows (the last tile of a routed expert): three 32-row
      // fragments per wave, so the tile costs 3/4 of a full one
      if constexpr (ROUTED) full_tile(I0{}, std::integral_constant<int, 3>{});
    } else if (EPI == EPI_QKV && rows <= 128) {
      // a half unit or the short last m-tile of the QKV product (which has
      // no short-tile path): two 32-row fragments per wave
      if constexpr (EPI == EPI_QKV) full_tile(I0{}, std::integral_constant<int, 2>{});
    } else if constexpr (HAS_STRIP) {
      if (rows > BM + 32) full_tile(std::integral_constant<int, 2>{}, F4{});
      else if (rows > BM) full_tile(std::integral_constant<int, 1>{}, F4{});
      else full_tile(I0{}, F4{});
    } else {
      full_tile(I0{}, F4{});
    }
    __syncthreads();   // the next tile's loads reuse this LDS
  }
}

template <bool DUAL, int EPI, typename TO, int WNF = 4>
void launch_big(const GemmParams& p, int n_cu, hipStream_t s) {
  // the 128 KB of dynamic LDS must be allowed once per kernel and device
  static bool configured[64] = {false};
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev < 0 || dev >= 64 || !configured[dev]) {
    (void)hipFuncSetAttribute((const void*)gemm_bf16_big_kernel<DUAL, EPI, TO, WNF>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (dev >= 0 && dev < 64) configured[dev] = true;
  }
  const int grid = ((n_cu + RDT_NUM_XCD - 1) / RDT_NUM_XCD) * RDT_NUM_XCD;
  gemm_bf16_big_kernel<DUAL, EPI, TO, WNF><<<grid, 256, LDS_BYTES, s>>>(p);
}

}  // namespace

void launch_gemm_bf16_big(const GemmParams& p, int epi, bool dual, int out_is_bf16, int n_cu, hipStream_t s,
                          int bn) {
  if (dual) {
    if (epi == EPI_SWIGLU_SAVE && out_is_bf16) launch_big<true, EPI_SWIGLU_SAVE, bf16_t>(p, n_cu, s);
    else if (out_is_bf16) launch_big<true, EPI_SWIGLU, bf16_t>(p, n_cu, s);
    else launch_big<true, EPI_SWIGLU, float>(p, n_cu, s);
    return;
  }
  if (bn == 192 && (epi == EPI_STORE || epi == EPI_RESID)) {
    if (epi == EPI_RESID) launch_big<false, EPI_RESID, float, 3>(p, n_cu, s);
    else if (out_is_bf16) launch_big<false, EPI_STORE, bf16_t, 3>(p, n_cu, s);
    else launch_big<false, EPI_STORE, float, 3>(p, n_cu, s);
    return;
  }
  switch (epi) {
    case EPI_STORE:
      if (out_is_bf16) launch_big<false, EPI_STORE, bf16_t>(p, n_cu, s);
      else launch_big<false, EPI_STORE, float>(p, n_cu, s);
      break;
    case EPI_RESID: launch_big<false, EPI_RESID, float>(p, n_cu, s); break;
    case EPI_QKV: launch_big<false, EPI_QKV, bf16_t>(p, n_cu, s); break;
    default: break;
  }
}
