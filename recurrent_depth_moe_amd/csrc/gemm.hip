// fp32 matrix products (fp32 configs) on gfx950: 64x64x16 tiles, four
// waves in 2x2, each wave one 32x32 output block on v_mfma_f32_32x32x2_f32
// (full fp32 products and sums), the same epilogues and the same persistent,
// XCD-aware tile loop as the bf16 kernels (the tile list is cut into eight
// contiguous chunks, one per XCD, since workgroup i runs on XCD i % 8).
//
// The bf16 products live in gemm_big.hip (prefill) and gemm_skinny.hip
// (single-token steps, router logits).
#include "gemm_device.h"

namespace {

// ------------------------------------------------------------ fp32 MFMA

template <bool DUAL, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p) {
  RDT_SKIP_IF_ALL_HALTED(p.live);
  constexpr int BM = 64, BN = 64, BK = 16, NB = DUAL ? 2 : 1;
  // rows of a k are 96 floats apart, so the two 32-lane halves of a
  // fragment read (k and k + 1) fall in different banks
  __shared__ float sA[BK][BM + 32];
  __shared__ float sB[NB][BK][BN + 32];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, wm = w >> 1, wn = w & 1;
  const int ntn = (p.N + BN - 1) / BN;
  const int n_mt = p.mt_start ? p.mt_start[p.n_groups] : (p.M + BM - 1) / BM;
  const int total = n_mt * ntn;
  const int per_xcd = gridDim.x / RDT_NUM_XCD;
  const int xcd = blockIdx.x % RDT_NUM_XCD, slot = blockIdx.x / RDT_NUM_XCD;
  const int chunk = (total + RDT_NUM_XCD - 1) / RDT_NUM_XCD;
  const int t_end = min(total, (xcd + 1) * chunk);
  const float* Abase = (const float*)p.A;

  for (int L = xcd * chunk + slot; L < t_end; L += per_xcd) {
    int mt, nt, row0, rows, grp;
    tile_coords(p, L, ntn, n_mt, mt, nt);
    tile_rows(p, mt, BM, row0, rows, grp);
    const int n0 = nt * BN;
    const float* Wb[NB];
    Wb[0] = (const float*)p.W0 + (int64_t)grp * p.w_stride;
    if constexpr (DUAL) Wb[NB - 1] = (const float*)p.W1 + (int64_t)grp * p.w_stride;

    // loader: 64 rows x 16 k = 256 float4; thread -> row tid/4, k (tid%4)*4
    const int lr = tid >> 2, lk = (tid & 3) * 4;
    const bool aok = lr < rows;
    const int arow_l = row0 + (aok ? lr : 0);
    const int arow = p.a_rows ? p.a_rows[arow_l] : arow_l;
    const float* ap = Abase + (int64_t)arow * p.lda + lk;
    const bool bok = n0 + lr < p.N;
    const int bn = bok ? n0 + lr : 0;

    floatx16_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;

    for (int k0 = 0; k0 < p.K; k0 += BK) {
      const bool kin = k0 + lk < p.K;
      float4 av = (aok && kin) ? *(const float4*)(ap + k0) : make_float4(0.f, 0.f, 0.f, 0.f);
      sA[lk + 0][lr] = av.x;
      sA[lk + 1][lr] = av.y;
      sA[lk + 2][lr] = av.z;
      sA[lk + 3][lr] = av.w;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float4 bv = (bok && kin) ? *(const float4*)(Wb[b] + (int64_t)bn * p.K + k0 + lk) : make_float4(0.f, 0.f, 0.f, 0.f);
        sB[b][lk + 0][lr] = bv.x;
        sB[b][lk + 1][lr] = bv.y;
        sB[b][lk + 2][lr] = bv.z;
        sB[b][lk + 3][lr] = bv.w;
      }
      __syncthreads();
      // k pair kk: lane l supplies A[row l % 32][k] and B[k][column l % 32]
      // for k = 2 kk + l / 32
#pragma unroll
      for (int kk = 0; kk < BK / 2; ++kk) {
        const int k = 2 * kk + (lane >> 5);
        const float a = sA[k][wm * 32 + (lane & 31)];
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, sB[b][k][wn * 32 + (lane & 31)], acc[b], 0, 0, 0);
      }
      __syncthreads();
    }
    // lane l, element e: row 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32 of
    // the wave's block; the pair partner of a column (n ^ 1, for the RoPE
    // epilogues) sits in lane l ^ 1
    const int n = n0 + wn * 32 + (lane & 31);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int ml = wm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      const float v = acc[0][e];
      const float v2 = DUAL ? acc[NB - 1][e] : __shfl_xor(v, 1, 64);
      if (ml < rows && n < p.N) epi_store<EPI, float>(p.epi, row0 + ml, n, v, v2);
    }
  }
}

int grid_for(int n_cu, int blocks_per_cu) {
  int g = n_cu * blocks_per_cu;
  return ((g + RDT_NUM_XCD - 1) / RDT_NUM_XCD) * RDT_NUM_XCD;
}

}  // namespace

void launch_gemm_f32(const GemmParams& p, int epi, bool dual, int n_cu, hipStream_t s) {
  const dim3 grid(grid_for(n_cu, 4)), block(256);
  if (dual) {
    gemm_f32_kernel<true, EPI_SWIGLU><<<grid, block, 0, s>>>(p);
    return;
  }
  switch (epi) {
    case EPI_STORE: gemm_f32_kernel<false, EPI_STORE><<<grid, block, 0, s>>>(p); break;
    case EPI_RESID: gemm_f32_kernel<false, EPI_RESID><<<grid, block, 0, s>>>(p); break;
    case EPI_QKV: gemm_f32_kernel<false, EPI_QKV><<<grid, block, 0, s>>>(p); break;
    case EPI_MLA_Q: gemm_f32_kernel<false, EPI_MLA_Q><<<grid, block, 0, s>>>(p); break;
    case EPI_MLA_KV: gemm_f32_kernel<false, EPI_MLA_KV><<<grid, block, 0, s>>>(p); break;
    default: break;
  }
}
