// Skinny bf16 GEMM for products whose m-tiles hold at most 32 rows: the
// router logits (32 tokens x all experts per block) and every matrix
// product of a decode step (32 sequences, or the 1-2 rows an expert gets).
//
// Block = 4 wave64s over one 32-row x NC-column tile (x2 for the fused
// gate|up product).  The K range is split in four; each wave runs
// v_mfma_f32_32x32x16_bf16 over its quarter with both operands streamed
// straight from global memory (lane l reads 16 bytes of row / column l % 32
// at k offset 8 * (l / 32)), four k-steps in flight.  Partial accumulators
// meet in LDS, are summed in a fixed order (deterministic) and go through
// the same epilogues as the large kernels.  These products are bound by
// weight streaming, not by MFMA.
#include "gemm_device.h"

namespace {

template <int NC, bool DUAL, int EPI, typename TO>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(GemmParams p) {
  RDT_SKIP_IF_ALL_HALTED(p.live);
  constexpr int NF = NC / 32, NB = DUAL ? 2 : 1, NA = NB * NF;
  __shared__ float red[4][NA][16 * 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ntn = (p.N + NC - 1) / NC;
  const int n_mt = p.mt_start ? p.mt_start[p.n_groups] : (p.M + 31) / 32;
  const int mt = blockIdx.x % p.skinny_mt_cap, nt = blockIdx.x / p.skinny_mt_cap;
  if (mt >= n_mt || nt >= ntn) return;   // grouped grids are sized for the worst case
  int row0, rows, grp;
  tile_rows(p, mt, 32, row0, rows, grp);
  const int n0 = nt * NC;
  const bf16_t* Wb[NB];
  Wb[0] = (const bf16_t*)p.W0 + (int64_t)grp * p.w_stride;
  if constexpr (DUAL) Wb[NB - 1] = (const bf16_t*)p.W1 + (int64_t)grp * p.w_stride;

  const int kq = p.K / 4, kbeg = w * kq, kk = 8 * (lane >> 5);
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
  for (; s + 4 <= steps; s += 4) {
    uint4 av[4], bv[4][NA];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      av[u] = *(const uint4*)(ap + (s + u) * 16);
#pragma unroll
      for (int i = 0; i < NA; ++i) bv[u][i] = *(const uint4*)(bp[i] + (s + u) * 16);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < NA; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, av[u]),
                                                         __builtin_bit_cast(bf16x8_t, bv[u][i]), acc[i], 0, 0, 0);
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
  for (int idx = threadIdx.x; idx < NF * 16 * 64; idx += 256) {
    const int f = idx / (16 * 64), rem = idx - f * 16 * 64, e = rem >> 6, l = rem & 63;
    const int row = 8 * (e >> 2) + 4 * (l >> 5) + (e & 3);
    const int n = n0 + f * 32 + (l & 31);
    float v = 0.f, v2 = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      v += red[ww][f][e * 64 + l];
      v2 += DUAL ? red[ww][NF + f][e * 64 + l] : red[ww][f][e * 64 + (l ^ 1)];
    }
    if (row < rows && n < p.N) epi_store<EPI, TO>(p.epi, row0 + row, n, v, v2);
  }
}

}  // namespace

// grid = (m-tiles the grid is sized for) x (n-tiles); grouped products size
// it for the worst case and surplus blocks exit at once
template <int NC, bool DUAL, int EPI, typename TO>
static void launch_skinny_t(const GemmParams& p, int mt_cap, hipStream_t s) {
  const int ntn = (p.N + NC - 1) / NC;
  gemm_skinny_kernel<NC, DUAL, EPI, TO><<<mt_cap * ntn, 256, 0, s>>>(p);
}

void launch_gemm_bf16_skinny(const GemmParams& p0, int epi, bool dual, int out_is_bf16, int mt_cap, int nc,
                             hipStream_t s) {
  GemmParams p = p0;
  p.skinny_mt_cap = mt_cap;
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
