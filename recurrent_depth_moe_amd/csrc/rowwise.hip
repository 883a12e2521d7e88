// Row-wise kernels of the recurrent block: tables, loop head (loop-index
// embedding + re-injection + two RMSNorms), RMSNorm, router top-k, dropless
// dispatch, loop tail (combine + depth-wise LoRA + LTI injection + ACT) and
// the MLA latent glue.  All are HBM-bound: one block streams one row with
// 16-byte accesses and keeps it in registers between its passes.
//
// Pages: [ZS] "OpenMythos 분석: …의 계산 모델링" (zero.shotlearni.ng);
//        [RC] "OpenMythos" (runchr.com).
#include "rowwise.h"

namespace {

constexpr int RB = 256;   // threads per row block
constexpr int MAXV4 = 8;  // float4 per thread: D <= 8192

__device__ __forceinline__ float4 ld4(const float* p) { return *(const float4*)p; }
__device__ __forceinline__ float4 ld4(const bf16_t* p) {
  const uint2 u = *(const uint2*)p;
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}
__device__ __forceinline__ void st4(float* p, float4 v) { *(float4*)p = v; }
__device__ __forceinline__ void st4(bf16_t* p, float4 v) {
  const uint2 u = {pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
  *(uint2*)p = u;
}
__device__ __forceinline__ float dot4(float4 a, float4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }
__device__ __forceinline__ float4 fma4(float s, float4 a, float4 b) {
  return make_float4(fmaf(s, a.x, b.x), fmaf(s, a.y, b.y), fmaf(s, a.z, b.z), fmaf(s, a.w, b.w));
}

// ------------------------------------------------------------ tables

__global__ void make_rope_kernel(float* c, float* s, int max_seq, int half, int rot, double theta) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= max_seq * half) return;
  const int p = idx / half, i = idx - p * half;
  const double ang = (double)p * pow(theta, -2.0 * i / rot);
  c[idx] = (float)cos(ang);
  s[idx] = (float)sin(ang);
}

// loop-index signal: sin(t w_j) on channel j, cos(t w_j) on channel half + j,
// w_j = theta^(-2j/loop_dim) ([ZS §Repeating the parameter reduces
// expressiveness]: sin and cos halves on the leading channels)
__global__ void make_loop_kernel(float* emb, int n_loops, int loop_dim, double theta) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_loops * loop_dim) return;
  const int t = idx / loop_dim, d = idx - t * loop_dim, half = loop_dim / 2;
  const int j = d < half ? d : d - half;
  const double ang = (double)t * pow(theta, -2.0 * j / loop_dim);
  emb[idx] = (float)(d < half ? sin(ang) : cos(ang));
}

// A = exp(-exp(clamp(log_dt + log_A, -20, 20))) ([ZS §latent reasoning])
__global__ void make_A_kernel(const float* log_A, const float* log_dt, float* A, int D) {
  const int d = blockIdx.x * blockDim.x + threadIdx.x;
  if (d >= D) return;
  double x = (double)log_dt[0] + (double)log_A[d];
  x = x < -20.0 ? -20.0 : (x > 20.0 ? 20.0 : x);
  A[d] = (float)exp(-exp(x));
}

// ------------------------------------------------------------ loop head

// NJ > 0: D = 4 RB NJ, every thread owns NJ whole float4 columns and all
// loads are unconditional (issued together); NJ = 0: any D <= 4 RB MAXV4.
template <typename TA, int NJ>
__global__ __launch_bounds__(RB) void loop_head_kernel(const float* __restrict__ h, const float* __restrict__ e,
                                                       const float* __restrict__ emb, int loop_dim,
                                                       const float* __restrict__ g_rec,
                                                       const float* __restrict__ g_attn, float eps,
                                                       float* __restrict__ c, TA* __restrict__ a, int D,
                                                       const int32_t* live_prev, int32_t* live_cur,
                                                       const int32_t* __restrict__ tok) {
  // this loop's running count starts at 0 (the tail adds to it), also when
  // the loop itself is skipped, so a skip carries on to every later loop
  if (live_cur && blockIdx.x == 0 && threadIdx.x == 0) *live_cur = 0;
  RDT_SKIP_IF_ALL_HALTED(live_prev);
  __shared__ float red[RB / 64];
  const int64_t base = (int64_t)blockIdx.x * D;                                   // rows of c, a
  const int64_t pbase = (int64_t)(tok ? tok[blockIdx.x] : (int)blockIdx.x) * D;   // position of h, e
  const int D4 = D >> 2;
  float4 v[MAXV4], y[MAXV4], m[MAXV4];
  // every load first (the loop embedding from a clamped, always valid
  // address, added only on its channels), then the arithmetic
#pragma unroll
  for (int j = 0; j < (NJ ? NJ : MAXV4); ++j) {
    const int i4 = threadIdx.x + j * RB;
    if (NJ || i4 < D4) {
      const int d = i4 * 4;
      v[j] = ld4(h + pbase + d);
      y[j] = ld4(e + pbase + d);
      if (loop_dim > 0) m[j] = ld4(emb + min(d, loop_dim - 4));
    }
  }
  __builtin_amdgcn_sched_barrier(0);   // every load issued before the first use
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < (NJ ? NJ : MAXV4); ++j) {
    const int i4 = threadIdx.x + j * RB;
    if (NJ || i4 < D4) {
      const int d = i4 * 4;
      float4 x = v[j];
      if (d < loop_dim) {
        x.x += m[j].x; x.y += m[j].y; x.z += m[j].z; x.w += m[j].w;
      }
      x.x += y[j].x; x.y += y[j].y; x.z += y[j].z; x.w += y[j].w;
      v[j] = x;
      ss += dot4(x, x);
    }
  }
  const float r1 = 1.0f / sqrtf(block_sum_dpp(ss, red) / D + eps);
  ss = 0.f;
#pragma unroll
  for (int j = 0; j < (NJ ? NJ : MAXV4); ++j) {
    const int i4 = threadIdx.x + j * RB;
    if (NJ || i4 < D4) {
      const int d = i4 * 4;
      const float4 g = ld4(g_rec + d);
      float4 x = v[j];
      x = make_float4(x.x * r1 * g.x, x.y * r1 * g.y, x.z * r1 * g.z, x.w * r1 * g.w);
      st4(c + base + d, x);
      v[j] = x;
      ss += dot4(x, x);
    }
  }
  const float r2 = 1.0f / sqrtf(block_sum_dpp(ss, red) / D + eps);
#pragma unroll
  for (int j = 0; j < (NJ ? NJ : MAXV4); ++j) {
    const int i4 = threadIdx.x + j * RB;
    if (NJ || i4 < D4) {
      const int d = i4 * 4;
      const float4 g = ld4(g_attn + d);
      const float4 x = v[j];
      st4(a + base + d, make_float4(x.x * r2 * g.x, x.y * r2 * g.y, x.z * r2 * g.z, x.w * r2 * g.w));
    }
  }
}

template <typename TO, int NJ>
__global__ __launch_bounds__(RB) void rmsnorm_kernel(const float* __restrict__ x, int64_t ldx,
                                                     const float* __restrict__ g, float eps, TO* __restrict__ out,
                                                     int64_t ldo, int D, const int32_t* live) {
  RDT_SKIP_IF_ALL_HALTED(live);
  __shared__ float red[RB / 64];
  const float* xr = x + (int64_t)blockIdx.x * ldx;
  TO* orow = out + (int64_t)blockIdx.x * ldo;
  const int D4 = D >> 2;
  float4 v[MAXV4];
#pragma unroll
  for (int j = 0; j < (NJ ? NJ : MAXV4); ++j) {
    const int i4 = threadIdx.x + j * RB;
    if (NJ || i4 < D4) v[j] = ld4(xr + i4 * 4);
  }
  __builtin_amdgcn_sched_barrier(0);   // every load issued before the first use
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < (NJ ? NJ : MAXV4); ++j) {
    const int i4 = threadIdx.x + j * RB;
    if (NJ || i4 < D4) ss += dot4(v[j], v[j]);
  }
  const float r = 1.0f / sqrtf(block_sum_dpp(ss, red) / D + eps);
#pragma unroll
  for (int j = 0; j < (NJ ? NJ : MAXV4); ++j) {
    const int i4 = threadIdx.x + j * RB;
    if (NJ || i4 < D4) {
      const float4 gg = ld4(g + i4 * 4);
      const float4 y = v[j];
      st4(orow + i4 * 4, make_float4(y.x * r * gg.x, y.y * r * gg.y, y.z * r * gg.z, y.w * r * gg.w));
    }
  }
}

// ------------------------------------------------------------ router
// Sixteen lanes (one DPP row) per token, lane j holding experts j, j + 16,
// ...  [ZS §MoE]: softmax scores over all experts; top-k taken on
// logits + router_bias (ties to the lower expert index); gates = chosen
// scores renormalised.  Every reduction stays inside the 16-lane row
// (quad_perm / row mirror DPP moves), so no LDS round trips.
template <int CTRL>
__device__ __forceinline__ int dpp_row_mov(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& best, int& bi, float& bz) {
  const float ob = __builtin_bit_cast(float, dpp_row_mov<CTRL>(__builtin_bit_cast(int, best)));
  const int oi = dpp_row_mov<CTRL>(bi);
  const float oz = __builtin_bit_cast(float, dpp_row_mov<CTRL>(__builtin_bit_cast(int, bz)));
  if (ob > best || (ob == best && oi < bi)) {
    best = ob;
    bi = oi;
    bz = oz;
  }
}
template <int CTRL>
__device__ __forceinline__ float max_step(float m) {
  return fmaxf(m, __builtin_bit_cast(float, dpp_row_mov<CTRL>(__builtin_bit_cast(int, m))));
}

template <int EPL>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits,
                                                          const float* __restrict__ bias, int N, int E, int k,
                                                          int32_t* __restrict__ sel, float* __restrict__ gate,
                                                          int32_t* __restrict__ cap_sel, const int32_t* live,
                                                          const int32_t* __restrict__ tok) {
  RDT_SKIP_IF_ALL_HALTED(live);
  const int l16 = threadIdx.x & 15;
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  if (row >= N) return;   // whole 16-lane rows leave together
  const float* z = logits + (int64_t)row * E;
  float zv[EPL], bv[EPL];
  unsigned taken = 0;
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int ex = l16 + 16 * j;
    if (ex < E) {
      zv[j] = z[ex];
      const float b = zv[j] + bias[ex];
      bv[j] = (b != b) ? -INFINITY : b;
      m = fmaxf(m, zv[j]);
    } else {
      zv[j] = 0.f;
      bv[j] = -INFINITY;
      taken |= 1u << j;
    }
  }
  m = max_step<0xB1>(m);    // quad_perm [1, 0, 3, 2]
  m = max_step<0x4E>(m);    // quad_perm [2, 3, 0, 1]
  m = max_step<0x141>(m);   // row_half_mirror
  m = max_step<0x140>(m);   // row_mirror
  float num[8];
  int idx[8];
  float den = 0.f;
  for (int kk = 0; kk < k; ++kk) {
    float best = -INFINITY, bz = 0.f;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int ex = l16 + 16 * j;
      if (!((taken >> j) & 1u) && (bv[j] > best || (bv[j] == best && ex < bi))) {
        best = bv[j];
        bi = ex;
        bz = zv[j];
      }
    }
    argmax_step<0xB1>(best, bi, bz);
    argmax_step<0x4E>(best, bi, bz);
    argmax_step<0x141>(best, bi, bz);
    argmax_step<0x140>(best, bi, bz);
    if ((bi & 15) == l16) taken |= 1u << (bi >> 4);
    num[kk] = expf(bz - m);
    idx[kk] = bi;
    den += num[kk];
  }
  if (l16 == 0) {
    for (int kk = 0; kk < k; ++kk) {
      sel[(int64_t)row * k + kk] = idx[kk];
      gate[(int64_t)row * k + kk] = num[kk] / den;
      if (cap_sel) cap_sel[(int64_t)(tok ? tok[row] : row) * k + kk] = idx[kk];
    }
  }
}

// ------------------------------------------------------------ dispatch
// counts per expert for each tile of 256 (token, slot) assignments
__global__ __launch_bounds__(RDT_DISP_TILE) void dispatch_count_kernel(const int32_t* __restrict__ sel, int NK,
                                                                       int E, int32_t* __restrict__ tile_counts,
                                                                       const int32_t* live) {
  RDT_SKIP_IF_ALL_HALTED(live);
  __shared__ int cnt[RDT_MAX_EXPERTS];
  for (int i = threadIdx.x; i < E; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  const int a = blockIdx.x * RDT_DISP_TILE + threadIdx.x;
  if (a < NK) atomicAdd(&cnt[sel[a]], 1);
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += blockDim.x) tile_counts[(int64_t)blockIdx.x * E + i] = cnt[i];
}

// per expert: exclusive scan over tiles (tile base), totals -> offsets,
// m-tile schedule of height bm.  Thread ex owns expert ex; the scans over
// experts are wave scans plus the totals of the earlier waves.
constexpr int RDT_SCAN_BATCH = 64;   // tile counts one thread holds in registers
__global__ __launch_bounds__(RDT_MAX_EXPERTS) void dispatch_scan_kernel(int32_t* __restrict__ tile_counts,
                                                                        int ntiles, int E, int bm,
                                                                        int32_t* __restrict__ offsets,
                                                                        int32_t* __restrict__ mt_start,
                                                                        int32_t* __restrict__ tile_row0,
                                                                        int32_t* __restrict__ tile_grp,
                                                                        int32_t* __restrict__ tile_claim,
                                                                        int n_claim, int merge_extra,
                                                                        int32_t* __restrict__ mt_start_m,
                                                                        int32_t* __restrict__ tile_row0_m,
                                                                        int32_t* __restrict__ tile_grp_m,
                                                                        const int32_t* live, int even_split) {
  RDT_SKIP_IF_ALL_HALTED(live);
  if ((int)threadIdx.x < n_claim) tile_claim[threadIdx.x] = 0;
  __shared__ int wsum[RDT_MAX_EXPERTS / 64][3];
  const int ex = threadIdx.x, lane = ex & 63, wv = ex >> 6;
  const bool own = ex < E;
  // exclusive scan down the tiles; with at most RDT_SCAN_BATCH tiles every
  // count is loaded before any is used and the prefixes stay in registers
  const bool one_batch = ntiles <= RDT_SCAN_BATCH;
  int pre[RDT_SCAN_BATCH];
  int run = 0;
  if (own) {
    if (one_batch) {
#pragma unroll
      for (int u = 0; u < RDT_SCAN_BATCH; ++u) pre[u] = u < ntiles ? tile_counts[(int64_t)u * E + ex] : 0;
#pragma unroll
      for (int u = 0; u < RDT_SCAN_BATCH; ++u) {
        const int c = pre[u];
        pre[u] = run;
        run += c;
      }
    } else {
      for (int t0 = 0; t0 < ntiles; t0 += 16) {
        int c[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) c[u] = t0 + u < ntiles ? tile_counts[(int64_t)(t0 + u) * E + ex] : 0;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if (t0 + u < ntiles) tile_counts[(int64_t)(t0 + u) * E + ex] = run;
          run += c[u];
        }
      }
    }
  }
  // exclusive scans over experts of the row totals and of the m-tile counts
  // (plain and merged schedule)
  const int tot = own ? run : 0, nmt = own ? (run + bm - 1) / bm : 0;
  const int rem = tot - (tot / bm) * bm;
  const int nmm = (merge_extra > 0 && tot > bm && rem > 0 && rem <= merge_extra) ? tot / bm : nmt;
  int it = tot, im = nmt, imm = nmm;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int a = __shfl_up(it, o, 64), b = __shfl_up(im, o, 64), c = __shfl_up(imm, o, 64);
    if (lane >= o) {
      it += a;
      im += b;
      imm += c;
    }
  }
  if (lane == 63) {
    wsum[wv][0] = it;
    wsum[wv][1] = im;
    wsum[wv][2] = imm;
  }
  __syncthreads();
  int off = it - tot, mts = im - nmt, mtm = imm - nmm;
  for (int w = 0; w < wv; ++w) {
    off += wsum[w][0];
    mts += wsum[w][1];
    mtm += wsum[w][2];
  }
  if (ex <= E) {   // thread E writes the totals
    offsets[ex] = off;
    mt_start[ex] = mts;
    if (merge_extra > 0) mt_start_m[ex] = mtm;
  }
  if (own) {
    if (one_batch) {
#pragma unroll
      for (int u = 0; u < RDT_SCAN_BATCH; ++u)
        if (u < ntiles) tile_counts[(int64_t)u * E + ex] = pre[u] + off;
    } else {
      for (int t0 = 0; t0 < ntiles; t0 += 16) {
        int c[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) c[u] = t0 + u < ntiles ? tile_counts[(int64_t)(t0 + u) * E + ex] : 0;
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (t0 + u < ntiles) tile_counts[(int64_t)(t0 + u) * E + ex] = c[u] + off;
      }
    }
    // even split: the expert's m-tiles take equal shares of its rows (within
    // one), so they run the same tile path at the same pace and stream the
    // expert's weight panels together
    for (int i = 0; i < nmt; ++i) {
      tile_grp[mts + i] = ex;
      tile_row0[mts + i] = off + (even_split ? (int)(((int64_t)i * tot) / nmt) : i * bm);
    }
    if (merge_extra > 0) {
      for (int i = 0; i < nmm; ++i) {
        tile_grp_m[mtm + i] = ex;
        tile_row0_m[mtm + i] = off + i * bm;
      }
    }
  }
}

// rank of each assignment among equal experts inside its tile, in
// (token, slot) order; destination = tile base + rank
__global__ __launch_bounds__(RDT_DISP_TILE) void dispatch_scatter_kernel(const int32_t* __restrict__ sel, int NK,
                                                                         int k, int E,
                                                                         const int32_t* __restrict__ tile_base,
                                                                         int32_t* __restrict__ perm_src,
                                                                         int32_t* __restrict__ inv,
                                                                         const int32_t* live) {
  RDT_SKIP_IF_ALL_HALTED(live);
  __shared__ int wcnt[RDT_DISP_TILE / 64][RDT_MAX_EXPERTS];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < (RDT_DISP_TILE / 64) * RDT_MAX_EXPERTS; i += blockDim.x) (&wcnt[0][0])[i] = 0;
  const int a = blockIdx.x * RDT_DISP_TILE + threadIdx.x;
  const bool valid = a < NK;
  const int ex = valid ? sel[a] : 0;
  uint64_t same = __ballot(valid);
  for (int bit = 0; (1 << bit) < E; ++bit) {
    const bool on = (ex >> bit) & 1;
    const uint64_t bal = __ballot(on);
    same &= on ? bal : ~bal;
  }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(same & lt);
  __syncthreads();
  if (valid && (same >> lane) == 1ull) wcnt[w][ex] = __popcll(same);
  __syncthreads();
  if (valid) {
    int r = rank;
    for (int ww = 0; ww < w; ++ww) r += wcnt[ww][ex];
    const int dest = tile_base[(int64_t)blockIdx.x * E + ex] + r;
    perm_src[dest] = a / k;
    inv[a] = dest;
  }
}

// ------------------------------------------------------------ loop tail
// tau = x1 + sum_j gate_j y_j + sum_s y_s; tau += ((tau Wd^T) * scale_t) B;
// h = A h + B e + tau ([RC §아키텍처]); p = sigmoid(h . w + b) and the ACT
// update ([ZS §ACT], [ZS §Recurrent Block]).
template <typename TW>
__global__ __launch_bounds__(RB) void loop_tail_kernel(TailArgs a) {
  RDT_SKIP_IF_ALL_HALTED(a.live_prev);
  __shared__ float red[RDT_MAX_LORA + 1][RB / 64];
  const int n = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int D = a.D, D4 = D >> 2;
  const int64_t base = (int64_t)n * D;                    // per-row tensors
  const int np = a.tok ? a.tok[n] : n;                    // this row's position
  const int64_t pbase = (int64_t)np * D;                  // per-position tensors
  const TW* Wd = (const TW*)a.lora_down;
  const TW* Wb = (const TW*)a.lora_B;

  int drow[8];
  float gw[8];
  for (int j = 0; j < a.k; ++j) {
    drow[j] = a.inv[(int64_t)n * a.k + j];
    gw[j] = a.gate[(int64_t)n * a.k + j];
  }
  float4 tau[MAXV4];
  float part[RDT_MAX_LORA];
#pragma unroll
  for (int r = 0; r < RDT_MAX_LORA; ++r) part[r] = 0.f;
#pragma unroll
  for (int j = 0; j < MAXV4; ++j) {
    const int i4 = threadIdx.x + j * RB;
    if (i4 < D4) {
      const int d = i4 * 4;
      float4 x = ld4(a.x1 + base + d);
      for (int s = 0; s < a.k; ++s) x = fma4(gw[s], ld4((const TW*)a.y + (int64_t)drow[s] * D + d), x);
      for (int s = 0; s < a.S; ++s) {
        const float4 ys = ld4((const TW*)a.y_s + (int64_t)s * a.N * D + base + d);
        x.x += ys.x; x.y += ys.y; x.z += ys.z; x.w += ys.w;
      }
      tau[j] = x;
#pragma unroll
      for (int r = 0; r < RDT_MAX_LORA; ++r)
        if (r < a.r) part[r] += dot4(x, ld4(Wd + (int64_t)r * D + d));
    }
  }
#pragma unroll
  for (int r = 0; r < RDT_MAX_LORA; ++r)
    if (r < a.r) {
      const float v = wave_sum(part[r]);
      if (lane == 0) red[r][w] = v;
    }
  __syncthreads();
  float lo[RDT_MAX_LORA];
#pragma unroll
  for (int r = 0; r < RDT_MAX_LORA; ++r) {
    lo[r] = 0.f;
    if (r < a.r) {
      float v = 0.f;
      for (int ww = 0; ww < RB / 64; ++ww) v += red[r][ww];
      lo[r] = v * a.lora_scale_row[r];
    }
  }
  float zs = 0.f;
#pragma unroll
  for (int j = 0; j < MAXV4; ++j) {
    const int i4 = threadIdx.x + j * RB;
    if (i4 < D4) {
      const int d = i4 * 4;
      float4 x = tau[j];
#pragma unroll
      for (int r = 0; r < RDT_MAX_LORA; ++r)
        if (r < a.r) x = fma4(lo[r], ld4(Wb + (int64_t)r * D + d), x);
      const float4 A = ld4(a.A + d), Bv = ld4(a.Bv + d), hp = ld4(a.h_prev + pbase + d), ee = ld4(a.e + pbase + d);
      float4 hn;
      hn.x = A.x * hp.x + Bv.x * ee.x + x.x;
      hn.y = A.y * hp.y + Bv.y * ee.y + x.y;
      hn.z = A.z * hp.z + Bv.z * ee.z + x.z;
      hn.w = A.w * hp.w + Bv.w * ee.w + x.w;
      tau[j] = hn;
      st4(a.h_next + pbase + d, hn);
      if (a.cap_h) st4(a.cap_h + pbase + d, hn);
      zs += dot4(hn, ld4(a.halt_w + d));
    }
  }
  const bool act = a.act_threshold > 0.f;
  const bool last = a.t == a.n_loops - 1;
  if (!act) {
    if (last) {
#pragma unroll
      for (int j = 0; j < MAXV4; ++j) {
        const int i4 = threadIdx.x + j * RB;
        if (i4 < D4) st4(a.h_out + pbase + i4 * 4, tau[j]);
      }
    }
    if (threadIdx.x == 0) a.halt_counts[np] = a.t + 1;
    return;
  }
  const float z = block_sum(zs, &red[RDT_MAX_LORA][0]) + a.halt_b[0];
  const float p = sigmoid_f(z);
  const float cum = a.t == 0 ? 0.f : a.cum[np];
  const int hc = a.t == 0 ? 0 : a.halt_counts[np];
  const bool running = hc == 0;
  float wgt = 0.f;
  bool halt_now = false;
  if (running) {
    const float s = cum + p;
    halt_now = (s >= a.act_threshold) || last;
    wgt = halt_now ? fmaxf(1.0f - cum, 0.f) : p;
  }
  if (a.t == 0 || running) {
#pragma unroll
    for (int j = 0; j < MAXV4; ++j) {
      const int i4 = threadIdx.x + j * RB;
      if (i4 < D4) {
        const int d = i4 * 4;
        const float4 prev = a.t == 0 ? make_float4(0.f, 0.f, 0.f, 0.f) : ld4(a.h_out + pbase + d);
        st4(a.h_out + pbase + d, fma4(wgt, tau[j], prev));
      }
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a.cum[np] = running ? cum + p : cum;
    a.halt_counts[np] = halt_now ? a.t + 1 : hc;
    if (a.cap_p) a.cap_p[np] = p;
    if (a.live_cur && running && !halt_now) atomicAdd(a.live_cur, 1);
  }
}

// Same step for R rows per block: the LoRA matrices (r x D each) are read
// once per block instead of once per row, which is what bounds the one-row
// form (2 r D bytes of L2 traffic per row).  Thread t owns float4 column t
// (+256 j) of every row.
template <typename TW, int R, int NJ, int LR>
__global__ __launch_bounds__(RB) void loop_tail_rows_kernel(TailArgs a) {
  RDT_SKIP_IF_ALL_HALTED(a.live_prev);
  __shared__ float red[RB / 64][LR * R + R];
  const int n0 = blockIdx.x * R, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int D = a.D, D4 = D >> 2;
  const TW* Wd = (const TW*)a.lora_down;
  const TW* Wb = (const TW*)a.lora_B;
  float4 tau[R][NJ];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int n = n0 + i;
    int drow[8];
    float gw[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s < a.k) {
        drow[s] = a.inv[(int64_t)n * a.k + s];
        gw[s] = a.gate[(int64_t)n * a.k + s];
      }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int i4 = threadIdx.x + j * RB;
      if (i4 < D4) {
        const int d = i4 * 4;
        float4 x = ld4(a.x1 + (int64_t)n * D + d);
#pragma unroll
        for (int s = 0; s < 8; ++s)
          if (s < a.k) x = fma4(gw[s], ld4((const TW*)a.y + (int64_t)drow[s] * D + d), x);
        for (int s = 0; s < a.S; ++s) {
          const float4 ys = ld4((const TW*)a.y_s + ((int64_t)s * a.N + n) * D + d);
          x.x += ys.x; x.y += ys.y; x.z += ys.z; x.w += ys.w;
        }
        tau[i][j] = x;
      }
    }
  }
  // LoRA down-projection, one rank at a time (few live partial sums)
#pragma unroll
  for (int r = 0; r < LR; ++r) {
    if (r < a.r) {
      float pr[R];
#pragma unroll
      for (int i = 0; i < R; ++i) pr[i] = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int i4 = threadIdx.x + j * RB;
        if (i4 < D4) {
          const float4 wv = ld4(Wd + (int64_t)r * D + i4 * 4);
#pragma unroll
          for (int i = 0; i < R; ++i) pr[i] += dot4(tau[i][j], wv);
        }
      }
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const float s = wave_sum(pr[i]);
        if (lane == 0) red[w][r * R + i] = s;
      }
    }
  }
  __syncthreads();
  // LoRA up-projection, one rank at a time (same per-element order over r)
#pragma unroll
  for (int r = 0; r < LR; ++r) {
    if (r < a.r) {
      float lo[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        float v = 0.f;
        for (int ww = 0; ww < RB / 64; ++ww) v += red[ww][r * R + i];
        lo[i] = v * a.lora_scale_row[r];
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int i4 = threadIdx.x + j * RB;
        if (i4 < D4) {
          const float4 bv = ld4(Wb + (int64_t)r * D + i4 * 4);
#pragma unroll
          for (int i = 0; i < R; ++i) tau[i][j] = fma4(lo[i], bv, tau[i][j]);
        }
      }
    }
  }
  float zs[R];
#pragma unroll
  for (int i = 0; i < R; ++i) zs[i] = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int i4 = threadIdx.x + j * RB;
    if (i4 < D4) {
      const int d = i4 * 4;
      const float4 A = ld4(a.A + d), Bv = ld4(a.Bv + d), hw = ld4(a.halt_w + d);
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int64_t off = (int64_t)(a.tok ? a.tok[n0 + i] : n0 + i) * D + d;   // position
        const float4 hp = ld4(a.h_prev + off), ee = ld4(a.e + off), x = tau[i][j];
        float4 hn;
        hn.x = A.x * hp.x + Bv.x * ee.x + x.x;
        hn.y = A.y * hp.y + Bv.y * ee.y + x.y;
        hn.z = A.z * hp.z + Bv.z * ee.z + x.z;
        hn.w = A.w * hp.w + Bv.w * ee.w + x.w;
        tau[i][j] = hn;
        st4(a.h_next + off, hn);
        if (a.cap_h) st4(a.cap_h + off, hn);
        zs[i] += dot4(hn, hw);
      }
    }
  }
  const bool act = a.act_threshold > 0.f;
  const bool last = a.t == a.n_loops - 1;
  if (!act) {
    if (last) {
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int i4 = threadIdx.x + j * RB;
          if (i4 < D4) st4(a.h_out + (int64_t)(a.tok ? a.tok[n0 + i] : n0 + i) * D + i4 * 4, tau[i][j]);
        }
    }
    if (threadIdx.x < R) a.halt_counts[a.tok ? a.tok[n0 + threadIdx.x] : n0 + threadIdx.x] = a.t + 1;
    return;
  }
  __syncthreads();   // red reused
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const float v = wave_sum(zs[i]);
    if (lane == 0) red[w][LR * R + i] = v;
  }
  __syncthreads();
  int still = 0;   // rows of this block still running after this loop
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int n = a.tok ? a.tok[n0 + i] : n0 + i;   // position of row n0 + i
    float z = a.halt_b[0];
    for (int ww = 0; ww < RB / 64; ++ww) z += red[ww][LR * R + i];
    const float p = sigmoid_f(z);
    const float cum = a.t == 0 ? 0.f : a.cum[n];
    const int hc = a.t == 0 ? 0 : a.halt_counts[n];
    const bool running = hc == 0;
    float wgt = 0.f;
    bool halt_now = false;
    if (running) {
      const float sum = cum + p;
      halt_now = (sum >= a.act_threshold) || last;
      wgt = halt_now ? fmaxf(1.0f - cum, 0.f) : p;
    }
    if (a.t == 0 || running) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int i4 = threadIdx.x + j * RB;
        if (i4 < D4) {
          const int64_t off = (int64_t)n * D + i4 * 4;
          const float4 prev = a.t == 0 ? make_float4(0.f, 0.f, 0.f, 0.f) : ld4(a.h_out + off);
          st4(a.h_out + off, fma4(wgt, tau[i][j], prev));
        }
      }
    }
    __syncthreads();   // every thread has read cum / halt_counts of row n
    if (threadIdx.x == 0) {
      a.cum[n] = running ? cum + p : cum;
      a.halt_counts[n] = halt_now ? a.t + 1 : hc;
      if (a.cap_p) a.cap_p[n] = p;
    }
    still += (running && !halt_now) ? 1 : 0;
  }
  if (a.live_cur && threadIdx.x == 0 && still > 0) atomicAdd(a.live_cur, still);
}

// Same step, bf16 LoRA weights, for the shapes the large configurations
// have: D a multiple of 4 * RB (every thread owns NJ whole float4 columns
// of every row), NS = k + S summed rows per output row, rank a multiple of
// four.  Every memory access is unconditional and batched so loads overlap:
// a row's x1 and NS source rows are all requested before they are summed,
// the LoRA rows four ranks at a time, a row's h_prev and e before its state
// update; wave sums use DPP (no LDS round trips).  Same
// per-element order as the generic form: x1, routed slots in slot order,
// shared experts in order; ranks in order.
template <int R, int NJ, int NS>
__global__ __launch_bounds__(RB) void loop_tail_fast_kernel(TailArgs a) {
  RDT_SKIP_IF_ALL_HALTED(a.live_prev);
  constexpr int RG = 4;   // ranks per LoRA group
  __shared__ float red[RB / 64][RDT_MAX_LORA * R + R];
  const int n0 = blockIdx.x * R, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int D = a.D, k = a.k;
  const bf16_t* Wd = (const bf16_t*)a.lora_down;
  const bf16_t* Wb = (const bf16_t*)a.lora_B;
  // row n0 + i (rows past N, in a last block of a row count that is not a
  // multiple of R, load row N - 1 and store nothing) and its position
  int nr[R], np[R];
  bool valid[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    valid[i] = n0 + i < a.N;
    nr[i] = valid[i] ? n0 + i : a.N - 1;
    np[i] = a.tok ? a.tok[nr[i]] : nr[i];
  }
  // source rows: the k routed slots (gate-weighted), then the S shared experts
  const bf16_t* src[R][NS];
  float wt[R][NS];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int n = nr[i];
#pragma unroll
    for (int q = 0; q < NS; ++q) {
      if (q < k) {
        src[i][q] = (const bf16_t*)a.y + (int64_t)a.inv[(int64_t)n * k + q] * D;
        wt[i][q] = a.gate[(int64_t)n * k + q];
      } else {
        src[i][q] = (const bf16_t*)a.y_s + ((int64_t)(q - k) * a.N + n) * D;
        wt[i][q] = 1.f;
      }
    }
  }
  float4 tau[R][NJ];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    float4 v[NJ][NS + 1];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int d = (threadIdx.x + j * RB) * 4;
      v[j][0] = ld4(a.x1 + (int64_t)nr[i] * D + d);
#pragma unroll
      for (int q = 0; q < NS; ++q) v[j][q + 1] = ld4(src[i][q] + d);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      float4 x = v[j][0];
#pragma unroll
      for (int q = 0; q < NS; ++q) x = fma4(wt[i][q], v[j][q + 1], x);
      tau[i][j] = x;
    }
  }
  // LoRA down-projection, RG ranks per group
  const int ng = a.r / RG;
#pragma unroll 1
  for (int g = 0; g < ng; ++g) {
    float4 wv[RG][NJ];
#pragma unroll
    for (int rr = 0; rr < RG; ++rr)
#pragma unroll
      for (int j = 0; j < NJ; ++j) wv[rr][j] = ld4(Wd + (int64_t)(g * RG + rr) * D + (threadIdx.x + j * RB) * 4);
#pragma unroll
    for (int rr = 0; rr < RG; ++rr)
#pragma unroll
      for (int i = 0; i < R; ++i) {
        float pr = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) pr += dot4(tau[i][j], wv[rr][j]);
        const float s = wave_sum_dpp(pr);
        if (lane == 0) red[w][(g * RG + rr) * R + i] = s;
      }
  }
  __syncthreads();
  // LoRA up-projection, ranks in order
#pragma unroll 1
  for (int g = 0; g < ng; ++g) {
    float4 bv[RG][NJ];
#pragma unroll
    for (int rr = 0; rr < RG; ++rr)
#pragma unroll
      for (int j = 0; j < NJ; ++j) bv[rr][j] = ld4(Wb + (int64_t)(g * RG + rr) * D + (threadIdx.x + j * RB) * 4);
#pragma unroll
    for (int rr = 0; rr < RG; ++rr) {
      const float sc = a.lora_scale_row[g * RG + rr];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        float v = 0.f;
#pragma unroll
        for (int ww = 0; ww < RB / 64; ++ww) v += red[ww][(g * RG + rr) * R + i];
        const float lo = v * sc;
#pragma unroll
        for (int j = 0; j < NJ; ++j) tau[i][j] = fma4(lo, bv[rr][j], tau[i][j]);
      }
    }
  }
  // state update h_{t+1} = A h_t + B e + tau
  float zs[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    zs[i] = 0.f;
    float4 hp[NJ], ee[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int64_t off = (int64_t)np[i] * D + (threadIdx.x + j * RB) * 4;
      hp[j] = ld4(a.h_prev + off);
      ee[j] = ld4(a.e + off);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int d = (threadIdx.x + j * RB) * 4;
      const int64_t off = (int64_t)np[i] * D + d;
      const float4 A = ld4(a.A + d), Bv = ld4(a.Bv + d), x = tau[i][j];
      float4 hn;
      hn.x = A.x * hp[j].x + Bv.x * ee[j].x + x.x;
      hn.y = A.y * hp[j].y + Bv.y * ee[j].y + x.y;
      hn.z = A.z * hp[j].z + Bv.z * ee[j].z + x.z;
      hn.w = A.w * hp[j].w + Bv.w * ee[j].w + x.w;
      tau[i][j] = hn;
      if (valid[i]) {
        st4(a.h_next + off, hn);
        if (a.cap_h) st4(a.cap_h + off, hn);
      }
      zs[i] += dot4(hn, ld4(a.halt_w + d));
    }
  }
  const bool act = a.act_threshold > 0.f;
  const bool last = a.t == a.n_loops - 1;
  if (!act) {
    if (last) {
#pragma unroll
      for (int i = 0; i < R; ++i)
        if (valid[i])
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            st4(a.h_out + (int64_t)np[i] * D + (threadIdx.x + j * RB) * 4, tau[i][j]);
    }
#pragma unroll
    for (int i = 0; i < R; ++i)
      if (threadIdx.x == i && valid[i]) a.halt_counts[np[i]] = a.t + 1;
    return;
  }
  // ACT: halting logit of every row (block sum), then the decisions
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const float v = wave_sum_dpp(zs[i]);
    if (lane == 0) red[w][RDT_MAX_LORA * R + i] = v;
  }
  __syncthreads();
  float pv[R], cumv[R];
  int hcv[R];
  bool run[R], halt[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int n = np[i];
    float z = a.halt_b[0];
#pragma unroll
    for (int ww = 0; ww < RB / 64; ++ww) z += red[ww][RDT_MAX_LORA * R + i];
    pv[i] = sigmoid_f(z);
    cumv[i] = a.t == 0 ? 0.f : a.cum[n];
    hcv[i] = a.t == 0 ? 0 : a.halt_counts[n];
    run[i] = hcv[i] == 0 && valid[i];
    halt[i] = false;
    float wgt = 0.f;
    if (run[i]) {
      halt[i] = (cumv[i] + pv[i] >= a.act_threshold) || last;
      wgt = halt[i] ? fmaxf(1.0f - cumv[i], 0.f) : pv[i];
    }
    if (run[i]) {
      float4 prev[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        prev[j] = a.t == 0 ? make_float4(0.f, 0.f, 0.f, 0.f)
                           : ld4(a.h_out + (int64_t)n * D + (threadIdx.x + j * RB) * 4);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        st4(a.h_out + (int64_t)n * D + (threadIdx.x + j * RB) * 4, fma4(wgt, tau[i][j], prev[j]));
    }
  }
  __syncthreads();   // every thread has read cum / halt_counts before they change
  int still = 0;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    if (threadIdx.x == i && valid[i]) {
      const int n = np[i];
      a.cum[n] = run[i] ? cumv[i] + pv[i] : cumv[i];
      a.halt_counts[n] = halt[i] ? a.t + 1 : hcv[i];
      if (a.cap_p) a.cap_p[n] = pv[i];
    }
    still += (run[i] && !halt[i]) ? 1 : 0;
  }
  if (a.live_cur && threadIdx.x == 0 && still > 0) atomicAdd(a.live_cur, still);
}

// ------------------------------------------------------------ embedding, argmax
template <typename TT>
__global__ __launch_bounds__(RB) void embed_kernel(const int32_t* __restrict__ ids, int64_t ids_ld, int T,
                                                    const TT* __restrict__ table, int V, int D,
                                                    float* __restrict__ x) {
  const int n = blockIdx.x, b = n / T, i = n - b * T;
  const int id = ids[(int64_t)b * ids_ld + i];
  float* xr = x + (int64_t)n * D;
  if (id < 0 || id >= V) {
    for (int d = threadIdx.x; d < D; d += RB) xr[d] = __builtin_nanf("");
    return;
  }
  const TT* tr = table + (int64_t)id * D;
  for (int d4 = threadIdx.x; d4 < (D >> 2); d4 += RB) st4(xr + 4 * d4, ld4(tr + 4 * d4));
}

// one block per row: each thread scans a strided share, then a block
// reduction keeps the larger value and, on equal values, the lower column
__global__ __launch_bounds__(RB) void argmax_rows_kernel(const float* __restrict__ logits, int V,
                                                         int32_t* __restrict__ out, int64_t out_ld) {
  __shared__ float bv[RB];
  __shared__ int bi[RB];
  const float* row = logits + (int64_t)blockIdx.x * V;
  float best = -INFINITY;
  int besti = 0x7fffffff;
  for (int j = threadIdx.x; j < V; j += RB) {
    const float v = row[j];
    if (v > best) {   // NaN compares false: never taken; ascending j keeps the first maximum
      best = v;
      besti = j;
    }
  }
  bv[threadIdx.x] = best;
  bi[threadIdx.x] = besti;
  __syncthreads();
  for (int w = RB / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      const float ov = bv[threadIdx.x + w];
      const int oi = bi[threadIdx.x + w];
      if (ov > bv[threadIdx.x] || (ov == bv[threadIdx.x] && oi < bi[threadIdx.x])) {
        bv[threadIdx.x] = ov;
        bi[threadIdx.x] = oi;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) out[(int64_t)blockIdx.x * out_ld] = bi[0] == 0x7fffffff ? 0 : bi[0];
}

// ------------------------------------------------------------ compaction
// ACT compute skipping: the positions still running (halt count 0) in
// ascending order, by one block: each wave ballots its 64 positions, the
// wave totals are scanned in LDS, and the block walks N in 1024-position
// chunks carrying the running offset.
__global__ __launch_bounds__(1024) void compact_running_kernel(const int32_t* __restrict__ halt_counts, int N,
                                                               int32_t* __restrict__ tok, int32_t* __restrict__ count) {
  __shared__ int wtot[16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int base = 0;
  for (int c0 = 0; c0 < N; c0 += 1024) {
    const int n = c0 + threadIdx.x;
    const bool run = n < N && halt_counts[n] == 0;
    const uint64_t m = __ballot(run);
    const int before = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wtot[w] = __popcll(m);
    __syncthreads();
    int off = base;
    int total = 0;
    for (int j = 0; j < 16; ++j) {
      if (j < w) off += wtot[j];
      total += wtot[j];
    }
    if (run) tok[off + before] = n;
    base += total;
    __syncthreads();   // wtot is rewritten by the next chunk
  }
  if (threadIdx.x == 0) *count = base;
}

// ------------------------------------------------------------ MLA glue
// [ZS §MLA]: the kv down-projection splits into the latent c_kv and one
// shared k_rope, which is rotated; both are what the cache holds.  The q
// latent and the kv latent are RMS-normalised (DeepSeek-V2 form).
template <typename TA>
__global__ __launch_bounds__(64) void mla_latent_kernel(const float* __restrict__ kv_raw,
                                                        const float* __restrict__ cq_raw,
                                                        const float* __restrict__ gq, float eps, int T, int ql,
                                                        int kvl, int rope, int start_pos,
                                                        const float* __restrict__ rcos,
                                                        const float* __restrict__ rsin, TA* __restrict__ cq_norm,
                                                        TA* __restrict__ lat_ckv, TA* __restrict__ lat_krope,
                                                        int lat_cap, int kbase, const int32_t* live) {
  RDT_SKIP_IF_ALL_HALTED(live);
  const int n = blockIdx.x, b = n / T, i = n - b * T, lane = threadIdx.x;
  const float* cq = cq_raw + (int64_t)n * ql;
  float ss = 0.f;
  for (int d = lane; d < ql; d += 64) ss += cq[d] * cq[d];
  const float r = 1.0f / sqrtf(wave_sum(ss) / ql + eps);
  for (int d = lane; d < ql; d += 64) St<TA>::st(cq_norm + (int64_t)n * ql + d, cq[d] * r * gq[d]);
  const float* kv = kv_raw + (int64_t)n * (kvl + rope);
  const int64_t slot = (int64_t)b * lat_cap + kbase + i;
  for (int d = lane; d < kvl; d += 64) St<TA>::st(lat_ckv + slot * kvl + d, kv[d]);
  const int half = rope / 2, pos = start_pos + i;
  for (int j = lane; j < half; j += 64) {
    const float x0 = kv[kvl + 2 * j], x1 = kv[kvl + 2 * j + 1];
    const float c = rcos[(int64_t)pos * half + j], s = rsin[(int64_t)pos * half + j];
    St<TA>::st(lat_krope + slot * rope + 2 * j, x0 * c - x1 * s);
    St<TA>::st(lat_krope + slot * rope + 2 * j + 1, x0 * s + x1 * c);
  }
}

template <typename TA>
__global__ __launch_bounds__(64) void mla_kv_prep_kernel(const TA* __restrict__ lat_ckv,
                                                         const TA* __restrict__ lat_krope, int lat_cap,
                                                         const float* __restrict__ gkv, float eps, int kvlen,
                                                         int kvl, int rope, int H, int dq,
                                                         TA* __restrict__ ckv_norm, TA* __restrict__ K,
                                                         const int32_t* live) {
  RDT_SKIP_IF_ALL_HALTED(live);
  const int m = blockIdx.x, b = m / kvlen, j = m - b * kvlen, lane = threadIdx.x;
  const TA* c = lat_ckv + ((int64_t)b * lat_cap + j) * kvl;
  float ss = 0.f;
  for (int d = lane; d < kvl; d += 64) {
    const float x = St<TA>::ld(c + d);
    ss += x * x;
  }
  const float r = 1.0f / sqrtf(wave_sum(ss) / kvl + eps);
  for (int d = lane; d < kvl; d += 64) St<TA>::st(ckv_norm + (int64_t)m * kvl + d, St<TA>::ld(c + d) * r * gkv[d]);
  const TA* kr = lat_krope + ((int64_t)b * lat_cap + j) * rope;
  const int nope = dq - rope;
  for (int x = lane; x < H * rope; x += 64) {
    const int h = x / rope, d = x - h * rope;
    K[(((int64_t)(b * H + h)) * kvlen + j) * dq + nope + d] = kr[d];
  }
}

// MLA decode step with the up-projections absorbed ([ZS §MLA] rebuilds
// k_nope and v from the cached latent; the products are regrouped here, an
// exact identity in real arithmetic): with W_k,h / W_v,h the k_nope / v rows
// of head h in W_ukv and n_j = RMSNorm(c_kv,j) * g_kv,
//   q_nope,h . (W_k,h n_j) = (W_k,h^T q_nope,h) . n_j     and
//   sum_j p_j (W_v,h n_j)  = W_v,h (sum_j p_j n_j),
// so attention runs once over the latent keys [n_j | k_rope,j] and values
// n_j (one key head shared by all query heads), without rebuilding
// per-head K / V for every cached position.

// latent keys [B][kvlen][kvl + rope] and values transposed [B][kvl][kvlen]
template <typename TA>
__global__ __launch_bounds__(64) void mla_latent_kv_kernel(const TA* __restrict__ lat_ckv,
                                                           const TA* __restrict__ lat_krope, int lat_cap,
                                                           const float* __restrict__ gkv, float eps, int kvlen,
                                                           int kvl, int rope, TA* __restrict__ k_lat,
                                                           TA* __restrict__ vt_lat, const int32_t* live) {
  RDT_SKIP_IF_ALL_HALTED(live);
  const int m = blockIdx.x, b = m / kvlen, j = m - b * kvlen, lane = threadIdx.x, dl = kvl + rope;
  const TA* c = lat_ckv + ((int64_t)b * lat_cap + j) * kvl;
  float ss = 0.f;
  for (int d = lane; d < kvl; d += 64) {
    const float x = St<TA>::ld(c + d);
    ss += x * x;
  }
  const float r = 1.0f / sqrtf(wave_sum(ss) / kvl + eps);
  for (int d = lane; d < kvl; d += 64) {
    const float x = St<TA>::ld(c + d) * r * gkv[d];
    St<TA>::st(k_lat + (int64_t)m * dl + d, x);
    St<TA>::st(vt_lat + ((int64_t)b * kvl + d) * kvlen + j, x);
  }
  const TA* kr = lat_krope + ((int64_t)b * lat_cap + j) * rope;
  for (int d = lane; d < rope; d += 64) k_lat[(int64_t)m * dl + kvl + d] = kr[d];
}

// q_lat[b][h] = [W_k,h^T q_nope,h | q_rope,h] (one query per sequence)
template <typename TA>
__global__ __launch_bounds__(64) void mla_absorb_q_kernel(const TA* __restrict__ q, const TA* __restrict__ wukv,
                                                          int H, int nope, int rope, int vd, int kvl,
                                                          TA* __restrict__ q_lat, const int32_t* live) {
  RDT_SKIP_IF_ALL_HALTED(live);
  const int bh = blockIdx.x, h = bh % H, lane = threadIdx.x;
  const TA* qr = q + (int64_t)bh * (nope + rope);
  TA* out = q_lat + (int64_t)bh * (kvl + rope);
  const TA* wk = wukv + (int64_t)h * (nope + vd) * kvl;
  for (int c = lane; c < kvl; c += 64) {
    float acc = 0.f;
    for (int d = 0; d < nope; ++d) acc = fmaf(St<TA>::ld(qr + d), St<TA>::ld(wk + (int64_t)d * kvl + c), acc);
    St<TA>::st(out + c, acc);
  }
  for (int r = lane; r < rope; r += 64) St<TA>::st(out + kvl + r, St<TA>::ld(qr + nope + r));
}

// o[b][h] = W_v,h o_lat[b][h]  (the O-projection input [B][H * vd])
template <typename TA>
__global__ __launch_bounds__(64) void mla_absorb_o_kernel(const TA* __restrict__ o_lat, const TA* __restrict__ wukv,
                                                          int H, int nope, int vd, int kvl, TA* __restrict__ o,
                                                          const int32_t* live) {
  RDT_SKIP_IF_ALL_HALTED(live);
  const int bh = blockIdx.x, h = bh % H, lane = threadIdx.x;
  const TA* ol = o_lat + (int64_t)bh * kvl;
  const TA* wv = wukv + ((int64_t)h * (nope + vd) + nope) * kvl;
  for (int e = lane; e < vd; e += 64) {
    float acc = 0.f;
    for (int c = 0; c < kvl; ++c) acc = fmaf(St<TA>::ld(ol + c), St<TA>::ld(wv + (int64_t)e * kvl + c), acc);
    St<TA>::st(o + (int64_t)bh * vd + e, acc);
  }
}

}  // namespace

void launch_mla_absorbed_decode_prep(const float* lat_ckv, const float* lat_krope, int lat_cap, const float* gkv,
                                     float eps, int B, int kvlen, int kvl, int rope, const float* q,
                                     const float* wukv, int H, int nope, int vd, float* k_lat, float* vt_lat,
                                     float* q_lat, hipStream_t s, const int32_t* live) {
  mla_latent_kv_kernel<float><<<B * kvlen, 64, 0, s>>>(lat_ckv, lat_krope, lat_cap, gkv, eps, kvlen, kvl, rope,
                                                       k_lat, vt_lat, live);
  mla_absorb_q_kernel<float><<<B * H, 64, 0, s>>>(q, wukv, H, nope, rope, vd, kvl, q_lat, live);
}

void launch_mla_absorb_o(const float* o_lat, const float* wukv, int B, int H, int nope, int vd, int kvl, float* o,
                         hipStream_t s, const int32_t* live) {
  mla_absorb_o_kernel<float><<<B * H, 64, 0, s>>>(o_lat, wukv, H, nope, vd, kvl, o, live);
}

void launch_make_tables(float* rope_cos, float* rope_sin, int max_seq, int rot_dim, double theta, hipStream_t s) {
  const int n = max_seq * (rot_dim / 2);
  make_rope_kernel<<<(n + 255) / 256, 256, 0, s>>>(rope_cos, rope_sin, max_seq, rot_dim / 2, rot_dim, theta);
}
void launch_make_loop_table(float* emb, int n_loops_max, int loop_dim, double theta, hipStream_t s) {
  const int n = n_loops_max * loop_dim;
  make_loop_kernel<<<(n + 255) / 256, 256, 0, s>>>(emb, n_loops_max, loop_dim, theta);
}
void launch_make_A(const float* log_A, const float* log_dt, float* A, int D, hipStream_t s) {
  make_A_kernel<<<(D + 255) / 256, 256, 0, s>>>(log_A, log_dt, A, D);
}

void launch_loop_head(int act_bf16, const float* h, const float* e, const float* emb_t, int loop_dim,
                      const float* g_rec, const float* g_attn, float eps, float* c, void* a, int N, int D,
                      hipStream_t s, const int32_t* live_prev, int32_t* live_cur, const int32_t* tok) {
#define RDT_LOOP_HEAD(TA, NJ) \
  loop_head_kernel<TA, NJ><<<N, RB, 0, s>>>(h, e, emb_t, loop_dim, g_rec, g_attn, eps, c, (TA*)a, D, live_prev, \
                                            live_cur, tok)
  const int nj = D % (4 * RB) == 0 ? D / (4 * RB) : 0;
  if (act_bf16) {
    switch (nj) {
      case 1: RDT_LOOP_HEAD(bf16_t, 1); break;
      case 2: RDT_LOOP_HEAD(bf16_t, 2); break;
      case 3: RDT_LOOP_HEAD(bf16_t, 3); break;
      case 4: RDT_LOOP_HEAD(bf16_t, 4); break;
      default: RDT_LOOP_HEAD(bf16_t, 0); break;
    }
  } else {
    RDT_LOOP_HEAD(float, 0);
  }
#undef RDT_LOOP_HEAD
}

void launch_rmsnorm(int out_bf16, const float* x, int64_t ldx, const float* g, float eps, void* out, int64_t ldo,
                    int rows, int D, hipStream_t s, const int32_t* live) {
  if (rows <= 0) return;
  const int nj = D % (4 * RB) == 0 ? D / (4 * RB) : 0;
  if (out_bf16) {
    switch (nj) {
      case 1: rmsnorm_kernel<bf16_t, 1><<<rows, RB, 0, s>>>(x, ldx, g, eps, (bf16_t*)out, ldo, D, live); break;
      case 2: rmsnorm_kernel<bf16_t, 2><<<rows, RB, 0, s>>>(x, ldx, g, eps, (bf16_t*)out, ldo, D, live); break;
      case 3: rmsnorm_kernel<bf16_t, 3><<<rows, RB, 0, s>>>(x, ldx, g, eps, (bf16_t*)out, ldo, D, live); break;
      case 4: rmsnorm_kernel<bf16_t, 4><<<rows, RB, 0, s>>>(x, ldx, g, eps, (bf16_t*)out, ldo, D, live); break;
      default: rmsnorm_kernel<bf16_t, 0><<<rows, RB, 0, s>>>(x, ldx, g, eps, (bf16_t*)out, ldo, D, live); break;
    }
  } else {
    rmsnorm_kernel<float, 0><<<rows, RB, 0, s>>>(x, ldx, g, eps, (float*)out, ldo, D, live);
  }
}

void launch_router_topk(const float* logits, const float* bias, int N, int E, int k, int32_t* sel, float* gate,
                        int32_t* cap_sel, hipStream_t s, const int32_t* live, const int32_t* tok) {
  const dim3 grid((N + 15) / 16);
  if (E <= 16) router_topk_kernel<1><<<grid, 256, 0, s>>>(logits, bias, N, E, k, sel, gate, cap_sel, live, tok);
  else if (E <= 32) router_topk_kernel<2><<<grid, 256, 0, s>>>(logits, bias, N, E, k, sel, gate, cap_sel, live, tok);
  else if (E <= 64) router_topk_kernel<4><<<grid, 256, 0, s>>>(logits, bias, N, E, k, sel, gate, cap_sel, live, tok);
  else if (E <= 128) router_topk_kernel<8><<<grid, 256, 0, s>>>(logits, bias, N, E, k, sel, gate, cap_sel, live, tok);
  else router_topk_kernel<16><<<grid, 256, 0, s>>>(logits, bias, N, E, k, sel, gate, cap_sel, live, tok);
}

void launch_dispatch(const int32_t* sel, int NK, int k, int E, int bm, int32_t* tile_counts, int32_t* offsets,
                     int32_t* mt_start, int32_t* tile_row0, int32_t* tile_grp, int32_t* perm_src, int32_t* inv,
                     int32_t* tile_claim, int n_claim, hipStream_t s, const int32_t* live, int merge_extra,
                     int32_t* mt_start_m, int32_t* tile_row0_m, int32_t* tile_grp_m) {
  const int ntiles = (NK + RDT_DISP_TILE - 1) / RDT_DISP_TILE;
  dispatch_count_kernel<<<ntiles, RDT_DISP_TILE, 0, s>>>(sel, NK, E, tile_counts, live);
  if (!(mt_start_m && tile_row0_m && tile_grp_m)) merge_extra = 0;
  dispatch_scan_kernel<<<1, RDT_MAX_EXPERTS, 0, s>>>(tile_counts, ntiles, E, bm, offsets, mt_start, tile_row0,
                                                     tile_grp, tile_claim, n_claim, merge_extra, mt_start_m,
                                                     tile_row0_m, tile_grp_m, live, bm >= 128 ? 1 : 0);
  dispatch_scatter_kernel<<<ntiles, RDT_DISP_TILE, 0, s>>>(sel, NK, k, E, tile_counts, perm_src, inv, live);
}

template <typename TW, int LR>
static void launch_tail_rows(const TailArgs& a, int nj, hipStream_t s) {
  constexpr int R = 4;
  const int grid = a.N / R;
  switch (nj) {
    case 1: loop_tail_rows_kernel<TW, R, 1, LR><<<grid, RB, 0, s>>>(a); break;
    case 2: loop_tail_rows_kernel<TW, R, 2, LR><<<grid, RB, 0, s>>>(a); break;
    case 3: loop_tail_rows_kernel<TW, R, 3, LR><<<grid, RB, 0, s>>>(a); break;
    default: loop_tail_rows_kernel<TW, R, 4, LR><<<grid, RB, 0, s>>>(a); break;
  }
}

template <int NJ, int R>
static bool launch_tail_fast_nj(const TailArgs& a, int ns, hipStream_t s) {
  const int grid = (a.N + R - 1) / R;
  switch (ns) {
    case 1: loop_tail_fast_kernel<R, NJ, 1><<<grid, RB, 0, s>>>(a); return true;
    case 2: loop_tail_fast_kernel<R, NJ, 2><<<grid, RB, 0, s>>>(a); return true;
    case 3: loop_tail_fast_kernel<R, NJ, 3><<<grid, RB, 0, s>>>(a); return true;
    case 4: loop_tail_fast_kernel<R, NJ, 4><<<grid, RB, 0, s>>>(a); return true;
    default: return false;
  }
}

void launch_loop_tail(const TailArgs& a, hipStream_t s) {
  // batched form: bf16 LoRA, whole float4 columns per thread (D a multiple
  // of 4 RB, at most 4 of them), 4-row blocks (1-row ones below 1024 rows;
  // a ragged last block masks its extra rows), k + S <= 4, rank a multiple
  // of 4 up to 16
  if (a.w_bf16 && a.D % (4 * RB) == 0 && a.D <= 16 * RB && a.r % 4 == 0 && a.r <= 16 && a.r > 0) {
    const int ns = a.k + a.S;
    bool ok = false;
    // one row per block when four-row blocks would leave most CUs idle
    // (single-token steps): the LoRA weights are re-read per row from L2,
    // but the block count, not bandwidth, sets the time there
    if (a.N < 1024) {
      switch (a.D / (4 * RB)) {
        case 1: ok = launch_tail_fast_nj<1, 1>(a, ns, s); break;
        case 2: ok = launch_tail_fast_nj<2, 1>(a, ns, s); break;
        case 3: ok = launch_tail_fast_nj<3, 1>(a, ns, s); break;
        default: ok = launch_tail_fast_nj<4, 1>(a, ns, s); break;
      }
    } else {
      switch (a.D / (4 * RB)) {
        case 1: ok = launch_tail_fast_nj<1, 4>(a, ns, s); break;
        case 2: ok = launch_tail_fast_nj<2, 4>(a, ns, s); break;
        case 3: ok = launch_tail_fast_nj<3, 4>(a, ns, s); break;
        default: ok = launch_tail_fast_nj<4, 4>(a, ns, s); break;
      }
    }
    if (ok) return;
  }
  // R-row blocks when the rows split evenly, D <= 4096 and rank <= 16
  const int nj = (a.D / 4 + RB - 1) / RB;
  if (a.N % 4 == 0 && nj <= 4 && a.r <= 16) {
    if (a.w_bf16) launch_tail_rows<bf16_t, 16>(a, nj, s);
    else launch_tail_rows<float, 16>(a, nj, s);
    return;
  }
  if (a.w_bf16) loop_tail_kernel<bf16_t><<<a.N, RB, 0, s>>>(a);
  else loop_tail_kernel<float><<<a.N, RB, 0, s>>>(a);
}

void launch_mla_latent(int act_bf16, const float* kv_raw, const float* cq_raw, const float* gq, float eps, int N,
                       int T, int ql, int kvl, int rope, int start_pos, const float* rcos, const float* rsin,
                       void* cq_norm, void* lat_ckv, void* lat_krope, int lat_cap, int kbase, hipStream_t s,
                       const int32_t* live) {
  if (act_bf16)
    mla_latent_kernel<bf16_t><<<N, 64, 0, s>>>(kv_raw, cq_raw, gq, eps, T, ql, kvl, rope, start_pos, rcos, rsin,
                                               (bf16_t*)cq_norm, (bf16_t*)lat_ckv, (bf16_t*)lat_krope, lat_cap,
                                               kbase, live);
  else
    mla_latent_kernel<float><<<N, 64, 0, s>>>(kv_raw, cq_raw, gq, eps, T, ql, kvl, rope, start_pos, rcos, rsin,
                                              (float*)cq_norm, (float*)lat_ckv, (float*)lat_krope, lat_cap, kbase,
                                              live);
}

void launch_mla_kv_prep(int act_bf16, const void* lat_ckv, const void* lat_krope, int lat_cap, const float* gkv,
                        float eps, int B, int kvlen, int kvl, int rope, int H, int dq, void* ckv_norm, void* K,
                        hipStream_t s, const int32_t* live) {
  if (act_bf16)
    mla_kv_prep_kernel<bf16_t><<<B * kvlen, 64, 0, s>>>((const bf16_t*)lat_ckv, (const bf16_t*)lat_krope, lat_cap,
                                                        gkv, eps, kvlen, kvl, rope, H, dq, (bf16_t*)ckv_norm,
                                                        (bf16_t*)K, live);
  else
    mla_kv_prep_kernel<float><<<B * kvlen, 64, 0, s>>>((const float*)lat_ckv, (const float*)lat_krope, lat_cap,
                                                       gkv, eps, kvlen, kvl, rope, H, dq, (float*)ckv_norm,
                                                       (float*)K, live);
}

void launch_compact_running(const int32_t* halt_counts, int N, int32_t* tok, int32_t* count, hipStream_t s) {
  compact_running_kernel<<<1, 1024, 0, s>>>(halt_counts, N, tok, count);
}

void launch_embed(int table_bf16, const int32_t* ids, int64_t ids_ld, int B, int T, const void* table, int V, int D,
                  float* x, hipStream_t s) {
  if (table_bf16)
    embed_kernel<bf16_t><<<B * T, RB, 0, s>>>(ids, ids_ld, T, (const bf16_t*)table, V, D, x);
  else
    embed_kernel<float><<<B * T, RB, 0, s>>>(ids, ids_ld, T, (const float*)table, V, D, x);
}

void launch_argmax_rows(const float* logits, int rows, int V, int32_t* out, int64_t out_ld, hipStream_t s) {
  argmax_rows_kernel<<<rows, RB, 0, s>>>(logits, V, out, out_ld);
}
