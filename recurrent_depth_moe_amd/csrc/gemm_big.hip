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

namespace {

// Issue order of the first half of a stage: a fragment read of the second
// half after each of the first 16 MFMAs.
__device__ __forceinline__ void interleave_first_half() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
}
// Second half: the 16 global->LDS loads of stage k+2 first (their latency
// is what the pipeline must hide), then the reads of the next stage's first
// half, one after each MFMA.
__device__ __forceinline__ void interleave_second_half() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);   // VMEM
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
  }
}

constexpr int BK = 64;                               // k depth of one LDS stage
constexpr int NSTAGE = 2;                            // LDS stages
constexpr int LDS_BYTES = NSTAGE * (256 + 256) * BK * 2;
constexpr int EP_LD = 128 + 4;                      // epilogue patch row stride (floats)
static_assert(4 * 32 * EP_LD * 4 <= LDS_BYTES, "epilogue patches fit in the tile LDS");

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void g2lds(const void* src, uint4* lds_slot0) {
  __builtin_amdgcn_global_load_lds(src, (lds_void_t*)lds_slot0, 16, 0, 0);
}

// Fragments of one 32-deep half (hh = 0, 1) of a 64-deep stage for this
// wave, for v_mfma_f32_32x32x16_bf16 (two 16-deep k-steps): 4 A fragments
// (32 rows each) and 4 B fragments (32 columns each) per k-step; lane l
// holds row/column l % 32 and k values 8 * (l / 32) .. +7 of the k-step.
// Rows hold 8 chunks of 8 k (128 bytes); chunk c of row r sits at position
// c ^ ((r >> 1) & 7), so the 8 rows a quarter-wave reads land in distinct
// banks.
__device__ __forceinline__ void read_frags(const uint4* sA, const uint4* sB, int wm, int wn, int lane, int hh,
                                           bf16x8_t (&af)[8], bf16x8_t (&bf)[8]) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int c = 4 * hh + 2 * s + (lane >> 5);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn * 128 + j * 32 + (lane & 31);
      bf[s * 4 + j] = __builtin_bit_cast(bf16x8_t, sB[r * 8 + (c ^ ((r >> 1) & 7))]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 128 + i * 32 + (lane & 31);
      af[s * 4 + i] = __builtin_bit_cast(bf16x8_t, sA[r * 8 + (c ^ ((r >> 1) & 7))]);
    }
  }
}

__device__ __forceinline__ void mfma_stage(const bf16x8_t (&af)[8], const bf16x8_t (&bf)[8],
                                           floatx16_t (&acc)[4][4]) {
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s * 4 + i], bf[s * 4 + j], acc[i][j], 0, 0, 0);
}

// wait until at most `n` direct-to-LDS loads of this wave are in flight
__device__ __forceinline__ void wait_vm(int n) {
  // s_waitcnt: vmcnt in bits [3:0] and [15:14], expcnt and lgkmcnt left at max
  if (n >= 16) __builtin_amdgcn_s_waitcnt(0x4F70);
  else if (n >= 8) __builtin_amdgcn_s_waitcnt(0x0F78);
  else __builtin_amdgcn_s_waitcnt(0x0F70);
}

template <bool DUAL, int EPI, typename TO>
__global__ __launch_bounds__(256, 1) void gemm_bf16_big_kernel(GemmParams p) {
  constexpr int BM = 256, BN = 256;
  constexpr int WTM = 128, WTN = 128;
  constexpr int A_CH = BM * (BK / 8), B_CH = BN * (BK / 8);   // 16-byte chunks per stage
  constexpr int A_IT = A_CH / 256, B_IT = B_CH / 256;
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

  for (int L = xcd * chunk + slot; L < t_end; L += per_xcd) {
    int mt, nt, row0, rows, grp;
    tile_coords(p, L, ntn, n_mt, mt, nt);
    tile_rows(p, mt, BM, row0, rows, grp);
    const int n0 = nt * NCOL;
    const bf16_t* W0 = (const bf16_t*)p.W0 + (int64_t)grp * p.w_stride;
    const bf16_t* W1 = DUAL ? (const bf16_t*)p.W1 + (int64_t)grp * p.w_stride : W0;

    // source pointers of this thread's chunks (k offset added per stage):
    // LDS slot s = (j*4 + w)*64 + lane holds row s/8, logical chunk
    // (s%8) ^ ((row >> 1) & 7)
    const bf16_t* asrc[A_IT];
#pragma unroll
    for (int j = 0; j < A_IT; ++j) {
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

    auto issue = [&](int stage, int k0) {
      uint4* base = smem + stage * (A_CH + B_CH);
#pragma unroll
      for (int j = 0; j < A_IT; ++j) g2lds(asrc[j] + k0, base + (j * 4 + w) * 64);
#pragma unroll
      for (int j = 0; j < B_IT; ++j) g2lds(bsrc[j] + k0, base + A_CH + (j * 4 + w) * 64);
    };

    floatx16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    // 32-row fragments of this wave that hold at least one valid row
    const int fm_valid = max(0, min(4, (rows - wm * WTM + 31) / 32));

    // prologue: stages 0 and 1 in flight, first half of stage 0 read (past
    // the end of K, loads repeat the last stage into a buffer nobody reads)
    issue(0, 0);
    issue(1, min(1, KT - 1) * BK);
    bf16x8_t fa0[8], fb0[8], fa1[8], fb1[8];
    wait_vm(A_IT + B_IT);
    __syncthreads();
    read_frags(smem, smem + A_CH, wm, wn, lane, 0, fa0, fb0);
    for (int kt = 0; kt < KT; ++kt) {
      {
        // first half of stage kt (registers fa0/fb0); read its second half
        const uint4* sb = smem + (kt & 1) * (A_CH + B_CH);
        read_frags(sb, sb + A_CH, wm, wn, lane, 1, fa1, fb1);
        mfma_stage(fa0, fb0, acc);
        interleave_first_half();
        __builtin_amdgcn_sched_barrier(0);
      }
      {
        // second half: stage kt+1 landed and every wave is done reading
        // stage kt, so its buffer takes stage kt+2; read stage kt+1's
        // first half (past the end: unused)
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
        issue(kt & 1, min(kt + 2, KT - 1) * BK);
        const uint4* sb = smem + ((kt + 1) & 1) * (A_CH + B_CH);
        read_frags(sb, sb + A_CH, wm, wn, lane, 0, fa0, fb0);
        mfma_stage(fa1, fb1, acc);
        interleave_second_half();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_vm(0);   // the trailing reloads land before the epilogue reuses LDS
    __syncthreads();   // every wave done with the stages before the epilogue reuses LDS

    // Epilogue through LDS, four passes of 32 rows per wave (one fragment
    // row each): a 32x32 accumulator holds, in lane l and element e, row
    // 8*(e/4) + 4*(l/32) + e%4 and column l%32.  The values go to a
    // row-major 32 x 128 fp32 patch of the wave's own LDS region, then each
    // lane takes 8 consecutive columns of one row, so stores are 16-byte
    // vectors and RoPE pairs sit in one lane.
    {
      float* ep = (float*)smem + w * (32 * EP_LD);
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
        if (pass < fm_valid) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
              ep[(8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * EP_LD + j * 32 + (lane & 31)] = acc[pass][j][e];
          __builtin_amdgcn_s_waitcnt(0);
          __builtin_amdgcn_wave_barrier();
          if constexpr (DUAL) {
            // 64 output columns: gate at patch columns 0..63, up at 64..127
#pragma unroll 1
            for (int it = 0; it < 4; ++it) {
              const int rl = it * 8 + (lane >> 3), c8 = (lane & 7) * 8;
              const int ml = wm * WTM + pass * 32 + rl;
              float g[8], u[8];
#pragma unroll
              for (int x = 0; x < 8; ++x) {
                g[x] = ep[rl * EP_LD + c8 + x];
                u[x] = ep[rl * EP_LD + 64 + c8 + x];
              }
              if (ml < rows) epi_store8<EPI, TO>(p.epi, p.N, row0 + ml, n0 + wn * 64 + c8, g, u);
            }
          } else {
#pragma unroll 1
            for (int it = 0; it < 8; ++it) {
              const int rl = it * 4 + (lane >> 4), c8 = (lane & 15) * 8;
              const int ml = wm * WTM + pass * 32 + rl;
              float v[8];
#pragma unroll
              for (int x = 0; x < 8; ++x) v[x] = ep[rl * EP_LD + c8 + x];
              if (ml < rows) epi_store8<EPI, TO>(p.epi, p.N, row0 + ml, n0 + wn * WTN + c8, v, v);
            }
          }
          __builtin_amdgcn_s_waitcnt(0);
          __builtin_amdgcn_wave_barrier();
        }
      }
    }
    __syncthreads();   // the next tile's loads reuse this LDS
  }
}

template <bool DUAL, int EPI, typename TO>
void launch_big(const GemmParams& p, int n_cu, hipStream_t s) {
  // the 128 KB of dynamic LDS must be allowed once per kernel and device
  static bool configured[64] = {false};
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev < 0 || dev >= 64 || !configured[dev]) {
    (void)hipFuncSetAttribute((const void*)gemm_bf16_big_kernel<DUAL, EPI, TO>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
    if (dev >= 0 && dev < 64) configured[dev] = true;
  }
  const int grid = ((n_cu + RDT_NUM_XCD - 1) / RDT_NUM_XCD) * RDT_NUM_XCD;
  gemm_bf16_big_kernel<DUAL, EPI, TO><<<grid, 256, LDS_BYTES, s>>>(p);
}

}  // namespace

void launch_gemm_bf16_big(const GemmParams& p, int epi, bool dual, int out_is_bf16, int n_cu, hipStream_t s) {
  if (dual) {
    if (out_is_bf16) launch_big<true, EPI_SWIGLU, bf16_t>(p, n_cu, s);
    else launch_big<true, EPI_SWIGLU, float>(p, n_cu, s);
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
