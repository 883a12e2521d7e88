// Skinny bf16 GEMM for products whose m-tiles hold at most 32 rows: the
// router logits (32 tokens x all experts per block) and every matrix
// product of a decode step (32 sequences, or the 1-2 rows an expert gets).
//
// Block = NW wave64s over one 32-row x NC-column tile (x2 for the fused
// gate|up product).  The K range is split NW ways; each wave runs
// v_mfma_f32_32x32x16_bf16 over its share with both operands streamed
// straight from global memory (lane l reads 16 bytes of row / column l % 32
// at k offset 8 * (l / 32)), the next U k-steps loading while the current U
// multiply.  Partial accumulators meet in LDS, are summed in a fixed order
// (deterministic) and go through the same epilogues as the large kernels.
// These products are bound by weight streaming, not by MFMA.
#include "gemm_device.h"

namespace {

template <int NC, bool DUAL, int EPI, typename TO, int NW, int U>
__global__ __launch_bounds__(64 * NW) void gemm_skinny_kernel(GemmParams p) {
  RDT_SKIP_IF_ALL_HALTED(p.live);
  constexpr int NF = NC / 32, NB = DUAL ? 2 : 1, NA = NB * NF;
  __shared__ float red[NW][NA][16 * 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ntn = (p.N + NC - 1) / NC;
  const int n_mt = p.mt_start ? p.mt_start[p.n_groups] : (p.M + 31) / 32;
  const int nt = blockIdx.x % ntn, mt = blockIdx.x / ntn;
  if (mt >= n_mt || nt >= ntn) return;   // grouped grids are sized for the worst case
  int row0, rows, grp;
  tile_rows(p, mt, 32, row0, rows, grp);
  const int n0 = nt * NC;
  const bf16_t* Wb[NB];
  Wb[0] = (const bf16_t*)p.W0 + (int64_t)grp * p.w_stride;
  if constexpr (DUAL) Wb[NB - 1] = (const bf16_t*)p.W1 + (int64_t)grp * p.w_stride;

  const int kq = p.K / NW, kbeg = w * kq, kk = 8 * (lane >> 5);
  const int r = lane & 31;
  const int m = row0 + (r < rows ? r : 0);
  const int arow = p.a_rows ? p.a_rows[m] : m;
  const bf16_t* ap = (const bf16_t*)p.A + (int64_t)arow * p.lda + kbeg + kk;
  const bf16_t* bp[NA];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int n = n0 + f * 32 + r;
      bp[b * NF + f] = Wb[b] + (int64_t)(n < p.N ? n : 0) * p.K + kbeg + kk;
    }
  floatx16_t acc[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;

  const int steps = kq / 16;
  int s = 0;
  auto load = [&](int s0, uint4 (&av)[U], uint4 (&bv)[U][NA]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      av[u] = *(const uint4*)(ap + (s0 + u) * 16);
#pragma unroll
      for (int i = 0; i < NA; ++i) bv[u][i] = *(const uint4*)(bp[i] + (s0 + u) * 16);
    }
  };
  auto mma = [&](const uint4 (&av)[U], const uint4 (&bv)[U][NA]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < NA; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av[u]),
                                                         __builtin_bit_cast(bf16x8_t, bv[u][i]), acc[i], 0, 0, 0);
  };
  // two register buffers: the loads of the next U steps are in flight while
  // the MFMAs of the current ones run.  The scheduling barriers keep the
  // compiler from sinking loads between the MFMAs (it would otherwise trade
  // the loads in flight for registers, which halves the streaming rate).
  {
    uint4 a0[U], b0[U][NA], a1[U], b1[U][NA];
    if (U <= steps) load(0, a0, b0);
    for (; s + 2 * U <= steps; s += 2 * U) {
      load(s + U, a1, b1);
      __builtin_amdgcn_sched_barrier(0);
      mma(a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      if (s + 3 * U <= steps) load(s + 2 * U, a0, b0);
      __builtin_amdgcn_sched_barrier(0);
      mma(a1, b1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (s + U <= steps) {
      mma(a0, b0);
      s += U;
    }
  }
  for (; s < steps; ++s) {
    const uint4 a1 = *(const uint4*)(ap + s * 16);
#pragma unroll
    for (int i = 0; i < NA; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a1),
                                                       __builtin_bit_cast(bf16x8_t, *(const uint4*)(bp[i] + s * 16)),
                                                       acc[i], 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < NA; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) red[w][i][e * 64 + lane] = acc[i][e];
  __syncthreads();
  // accumulator element e of lane l: row 8*(e/4) + 4*(l/32) + e%4, column l%32
  for (int idx = threadIdx.x; idx < NF * 16 * 64; idx += 64 * NW) {
    const int f = idx / (16 * 64), rem = idx - f * 16 * 64, e = rem >> 6, l = rem & 63;
    const int row = 8 * (e >> 2) + 4 * (l >> 5) + (e & 3);
    const int n = n0 + f * 32 + (l & 31);
    float v = 0.f, v2 = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      v += red[ww][f][e * 64 + l];
      v2 += DUAL ? red[ww][NF + f][e * 64 + l] : red[ww][f][e * 64 + (l ^ 1)];
    }
    if (row < rows && n < p.N) epi_store<EPI, TO>(p.epi, row0 + row, n, v, v2);
  }
}

}  // namespace

// grid = (m-tiles the grid is sized for) x (n-tiles), n-tile fastest, so the
// live m-tiles come first in dispatch order; grouped products size the grid
// for the worst case and the surplus blocks at its end exit at once
template <int NC, bool DUAL, int EPI, typename TO, int NW = 4, int U = 4>
static void launch_skinny_t(const GemmParams& p, int mt_cap, hipStream_t s) {
  const int ntn = (p.N + NC - 1) / NC;
  gemm_skinny_kernel<NC, DUAL, EPI, TO, NW, U><<<mt_cap * ntn, 64 * NW, 0, s>>>(p);
}

void launch_gemm_bf16_skinny(const GemmParams& p0, int epi, bool dual, int out_is_bf16, int mt_cap, int nc,
                             hipStream_t s, int nw) {
  const GemmParams& p = p0;
  // eight waves, eight k-steps per buffer: fp32 products with few blocks
  // (router logits), where the waves' sequential load round trips set the time
  if (nw == 8 && !dual && epi == EPI_STORE && !out_is_bf16 && p.K % (8 * 16) == 0) {
    if (nc == 64) launch_skinny_t<64, false, EPI_STORE, float, 8, 8>(p, mt_cap, s);
    else launch_skinny_t<32, false, EPI_STORE, float, 8, 8>(p, mt_cap, s);
    return;
  }
  if (dual) {
    if (out_is_bf16) launch_skinny_t<32, true, EPI_SWIGLU, bf16_t>(p, mt_cap, s);
    else launch_skinny_t<32, true, EPI_SWIGLU, float>(p, mt_cap, s);
    return;
  }
  if (nc == 64) {
    switch (epi) {
      case EPI_STORE:
        if (out_is_bf16) launch_skinny_t<64, false, EPI_STORE, bf16_t>(p, mt_cap, s);
        else launch_skinny_t<64, false, EPI_STORE, float>(p, mt_cap, s);
        return;
      default: break;
    }
  }
  switch (epi) {
    case EPI_STORE:
      if (out_is_bf16) launch_skinny_t<32, false, EPI_STORE, bf16_t>(p, mt_cap, s);
      else launch_skinny_t<32, false, EPI_STORE, float>(p, mt_cap, s);
      break;
    case EPI_RESID: launch_skinny_t<32, false, EPI_RESID, float>(p, mt_cap, s); break;
    case EPI_QKV: launch_skinny_t<32, false, EPI_QKV, bf16_t>(p, mt_cap, s); break;
    default: break;
  }
}
