// Matrix products of the recurrent block on gfx950.
//
// bf16 path: 128x128x64 block tiles (or 128x64 per matrix for the fused
// gate|up product), four wave64s in 2x2, v_mfma_f32_16x16x32_bf16 with fp32
// accumulation, double-buffered LDS with an XOR swizzle of the 16-byte
// chunks of each 128-byte row (chunk ^ ((row >> 1) & 7)) so the fragment
// reads of 16 consecutive rows land in distinct banks.
// fp32 path (fp32 configs): 64x64x16 tiles, 4x4 fp32 FMA micro-tiles.
//
// Both run a persistent, XCD-aware tile loop: the tile list is cut into
// eight contiguous chunks, one per XCD (workgroup i runs on XCD i % 8), so
// the m-tiles that share an expert's weight panel, and the n-tiles that
// share a group's activation rows, meet in the same L2.
#include "gemm_device.h"

namespace {

// ------------------------------------------------------------ bf16 MFMA

template <int BM, int BN, bool DUAL, int EPI, typename TO>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(GemmParams p) {
  constexpr int BK = 64;
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 16, FN = WN / 16;
  constexpr int A_LD = BM * 8 / 256, B_LD = BN * 8 / 256;
  __shared__ uint4 sA[2][BM * 8];
  __shared__ uint4 sB[2][NB][BN * 8];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int ntn = (p.N + BN - 1) / BN;
  const int n_mt = p.mt_start ? p.mt_start[p.n_groups] : (p.M + BM - 1) / BM;
  const int total = n_mt * ntn;
  const int per_xcd = gridDim.x / RDT_NUM_XCD;
  const int xcd = blockIdx.x % RDT_NUM_XCD, slot = blockIdx.x / RDT_NUM_XCD;
  const int chunk = (total + RDT_NUM_XCD - 1) / RDT_NUM_XCD;
  const int t_end = min(total, (xcd + 1) * chunk);
  const bf16_t* Abase = (const bf16_t*)p.A;

  for (int L = xcd * chunk + slot; L < t_end; L += per_xcd) {
    int mt, nt, row0, rows, grp;
    tile_coords(p, L, ntn, n_mt, mt, nt);
    tile_rows(p, mt, BM, row0, rows, grp);
    const int n0 = nt * BN;
    const bf16_t* Wb[NB];
    Wb[0] = (const bf16_t*)p.W0 + (int64_t)grp * p.w_stride;
    if constexpr (DUAL) Wb[NB - 1] = (const bf16_t*)p.W1 + (int64_t)grp * p.w_stride;

    const bf16_t* ap[A_LD];
    bool aok[A_LD];
#pragma unroll
    for (int j = 0; j < A_LD; ++j) {
      const int idx = tid + j * 256, r = idx >> 3, c = idx & 7;
      aok[j] = r < rows;
      const int m = row0 + (aok[j] ? r : 0);
      const int arow = p.a_rows ? p.a_rows[m] : m;
      ap[j] = Abase + (int64_t)arow * p.lda + c * 8;
    }
    const bf16_t* bp[NB][B_LD];
    bool bok[B_LD];
#pragma unroll
    for (int j = 0; j < B_LD; ++j) {
      const int idx = tid + j * 256, r = idx >> 3, c = idx & 7;
      bok[j] = n0 + r < p.N;
      const int n = bok[j] ? n0 + r : 0;
#pragma unroll
      for (int b = 0; b < NB; ++b) bp[b][j] = Wb[b] + (int64_t)n * p.K + c * 8;
    }

    floatx4_t acc[NB][FM][FN];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[b][i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    uint4 ra[A_LD], rb[NB][B_LD];
    const uint4 zero = {0u, 0u, 0u, 0u};
    auto gload = [&](int k0) {
#pragma unroll
      for (int j = 0; j < A_LD; ++j) {
        const int c = (tid + j * 256) & 7;
        ra[j] = (aok[j] && k0 + c * 8 < p.K) ? *(const uint4*)(ap[j] + k0) : zero;
      }
#pragma unroll
      for (int j = 0; j < B_LD; ++j) {
        const int c = (tid + j * 256) & 7;
        const bool ok = bok[j] && k0 + c * 8 < p.K;
#pragma unroll
        for (int b = 0; b < NB; ++b) rb[b][j] = ok ? *(const uint4*)(bp[b][j] + k0) : zero;
      }
    };
    auto sstore = [&](int buf) {
#pragma unroll
      for (int j = 0; j < A_LD; ++j) {
        const int idx = tid + j * 256, r = idx >> 3, c = idx & 7;
        sA[buf][r * 8 + (c ^ ((r >> 1) & 7))] = ra[j];
      }
#pragma unroll
      for (int j = 0; j < B_LD; ++j) {
        const int idx = tid + j * 256, r = idx >> 3, c = idx & 7;
#pragma unroll
        for (int b = 0; b < NB; ++b) sB[buf][b][r * 8 + (c ^ ((r >> 1) & 7))] = rb[b][j];
      }
    };

    const int KT = (p.K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < KT) gload((kt + 1) * BK);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int c = s * 4 + (lane >> 4);
        bf16x8_t af[FM], bfr[NB][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = wm * WM + i * 16 + (lane & 15);
          af[i] = __builtin_bit_cast(bf16x8_t, sA[buf][r * 8 + (c ^ ((r >> 1) & 7))]);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const int r = wn * WN + j * 16 + (lane & 15);
            bfr[b][j] = __builtin_bit_cast(bf16x8_t, sB[buf][b][r * 8 + (c ^ ((r >> 1) & 7))]);
          }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
              acc[b][i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[b][j], acc[b][i][j], 0, 0, 0);
      }
      if (kt + 1 < KT) sstore(buf ^ 1);
      __syncthreads();
    }

    // accumulator layout: lane holds rows 4*(lane/16)+r, column lane%16
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ml = wm * WM + i * 16 + 4 * (lane >> 4) + r;
          const int n = n0 + wn * WN + j * 16 + (lane & 15);
          const float v = acc[0][i][j][r];
          const float v2 = DUAL ? acc[NB - 1][i][j][r] : __shfl_xor(v, 1, 64);
          if (ml < rows && n < p.N) epi_store<EPI, TO>(p.epi, row0 + ml, n, v, v2);
        }
  }
}

// ------------------------------------------------------------ fp32 FMA

template <bool DUAL, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p) {
  constexpr int BM = 64, BN = 64, BK = 16, NB = DUAL ? 2 : 1;
  __shared__ float sA[BK][BM + 4];
  __shared__ float sB[NB][BK][BN + 4];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
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

    float acc[NB][4][4];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[b][i][j] = 0.f;

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
#pragma unroll
      for (int k = 0; k < BK; ++k) {
        const float4 a4 = *(const float4*)&sA[k][ty * 4];
        const float a[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float4 b4 = *(const float4*)&sB[b][k][tx * 4];
          const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[b][i][j] = fmaf(a[i], bb[j], acc[b][i][j]);
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ml = ty * 4 + i, n = n0 + tx * 4 + j;
        const float v = acc[0][i][j];
        const float v2 = DUAL ? acc[NB - 1][i][j] : acc[0][i][j ^ 1];
        if (ml < rows && n < p.N) epi_store<EPI, float>(p.epi, row0 + ml, n, v, v2);
      }
  }
}

int grid_for(int n_cu, int blocks_per_cu) {
  int g = n_cu * blocks_per_cu;
  return ((g + RDT_NUM_XCD - 1) / RDT_NUM_XCD) * RDT_NUM_XCD;
}

}  // namespace

void launch_gemm_bf16(const GemmParams& p, int epi, bool dual, int bm, int out_is_bf16, int n_cu, hipStream_t s) {
  (void)bm;
  const dim3 grid(grid_for(n_cu, 2)), block(256);
  if (dual) {
    if (out_is_bf16) gemm_bf16_kernel<128, 64, true, EPI_SWIGLU, bf16_t><<<grid, block, 0, s>>>(p);
    else gemm_bf16_kernel<128, 64, true, EPI_SWIGLU, float><<<grid, block, 0, s>>>(p);
    return;
  }
  switch (epi) {
    case EPI_STORE:
      if (out_is_bf16) gemm_bf16_kernel<128, 128, false, EPI_STORE, bf16_t><<<grid, block, 0, s>>>(p);
      else gemm_bf16_kernel<128, 128, false, EPI_STORE, float><<<grid, block, 0, s>>>(p);
      break;
    case EPI_RESID: gemm_bf16_kernel<128, 128, false, EPI_RESID, float><<<grid, block, 0, s>>>(p); break;
    case EPI_QKV: gemm_bf16_kernel<128, 128, false, EPI_QKV, bf16_t><<<grid, block, 0, s>>>(p); break;
    case EPI_MLA_Q: gemm_bf16_kernel<128, 128, false, EPI_MLA_Q, bf16_t><<<grid, block, 0, s>>>(p); break;
    case EPI_MLA_KV: gemm_bf16_kernel<128, 128, false, EPI_MLA_KV, bf16_t><<<grid, block, 0, s>>>(p); break;
    default: break;
  }
}

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
