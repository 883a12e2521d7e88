// Backward pass of the recurrent block ([ZS §Recurrent Block] forward,
// differentiated with the expert choices and halting loops held fixed).
//
// Pages: [ZS] "OpenMythos 분석: …의 계산 모델링" (zero.shotlearni.ng).
//
// MFMA v_mfma_f32_32x32x16_bf16 layout used throughout: with operands
// (a, b), lane l supplies a row A[l % 32][8 (l / 32) .. +7] and a column
// B[8 (l / 32) .. +7][l % 32]; the result lane l holds column l % 32 of rows
// 8 (r / 4) + 4 (l / 32) + r % 4, r = 0 .. 15.  Any permutation of the 16
// contraction slots works as long as both operands use it: the products
// that contract over queries or keys use the order in which a lane already
// holds its scores (slot 8 h + x <-> index 8 (x / 4) + 4 h + x % 4).
#include "backward.h"

#include <type_traits>

#include <algorithm>

namespace {

__device__ __forceinline__ floatx16_t mfma32(const bf16x8_t& a, const bf16x8_t& b, const floatx16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf_elem(const uint4& v, int j) {
  const uint32_t d = j < 2 ? v.x : j < 4 ? v.y : j < 6 ? v.z : v.w;
  return (j & 1) ? (d >> 16) : (d & 0xffffu);
}

// 8 bf16 from p, the first `nvalid` of them (the rest zero)
__device__ __forceinline__ uint4 load8(const bf16_t* p, int nvalid) {
  if (nvalid >= 8) return *(const uint4*)p;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  for (int i = 0; i < nvalid; ++i) w[i >> 1] |= (uint32_t)p[i] << (16 * (i & 1));
  return uint4{w[0], w[1], w[2], w[3]};
}

__device__ __forceinline__ bf16x8_t as_frag(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

// eight fp32 scores -> one bf16 fragment
__device__ __forceinline__ bf16x8_t pack8(const float* p) {
  const uint4 v = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                   pack_bf16x2(p[6], p[7])};
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ float4 ld4(const float* p) { return *(const float4*)p; }
__device__ __forceinline__ void st4(float* p, float4 v) { *(float4*)p = v; }
__device__ __forceinline__ float4 ldbf4(const bf16_t* p) {
  const uint2 u = *(const uint2*)p;
  return float4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                __uint_as_float(u.y & 0xffff0000u)};
}
__device__ __forceinline__ void stbf4(bf16_t* p, float4 v) {
  *(uint2*)p = uint2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
}
__device__ __forceinline__ float dot4(float4 a, float4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }
__device__ __forceinline__ float4 fma4(float s, float4 a, float4 b) {
  return float4{fmaf(s, a.x, b.x), fmaf(s, a.y, b.y), fmaf(s, a.z, b.z), fmaf(s, a.w, b.w)};
}
__device__ __forceinline__ float4 add4(float4 a, float4 b) { return float4{a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w}; }
__device__ __forceinline__ float4 mul4(float4 a, float4 b) { return float4{a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w}; }
__device__ __forceinline__ float4 scl4(float s, float4 a) { return float4{s * a.x, s * a.y, s * a.z, s * a.w}; }

// ------------------------------------------------------------ transpose
// 64 x 64 tile per block; 16-byte global reads and writes where the tile
// lies inside the matrix and the strides allow, element-wise at the edges
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const bf16_t* __restrict__ in, int64_t isb1,
                                                             int64_t isb2, int nb2, int64_t ldi,
                                                             bf16_t* __restrict__ out, int64_t osb, int64_t ldo,
                                                             int R, int Rp, int C, int Cv, int vec) {
  __shared__ bf16_t tile[64][72];
  const int bi = blockIdx.z, b1 = bi / nb2, b2 = bi - b1 * nb2;
  const bf16_t* src = in + b1 * isb1 + b2 * isb2;
  bf16_t* dst = out + bi * osb;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const bool inside = vec && r0 + 64 <= R && c0 + 64 <= Cv && c0 + 64 <= C && r0 + 64 <= Rp;
  if (inside) {
    // thread: row i = tid / 8 (+ 32), columns 8 (tid % 8) .. +7
    const int i = threadIdx.x >> 3, cc = (threadIdx.x & 7) * 8;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 v = *(const uint4*)(src + (int64_t)(r0 + i + 32 * h) * ldi + c0 + cc);
      *(uint4*)&tile[i + 32 * h][cc] = v;
    }
    __syncthreads();
    // thread: output row (column c0 + i), rows r0 + rr .. +7 of the input
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = i + 32 * h;
      uint32_t w[4];
#pragma unroll
      for (int x = 0; x < 4; ++x)
        w[x] = (uint32_t)tile[cc + 2 * x][c] | ((uint32_t)tile[cc + 2 * x + 1][c] << 16);
      *(uint4*)(dst + (int64_t)(c0 + c) * ldo + r0 + cc) = uint4{w[0], w[1], w[2], w[3]};
    }
    return;
  }
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < Cv && c < C) ? src[(int64_t)r * ldi + c] : (bf16_t)0;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < C && r < Rp) dst[(int64_t)c * ldo + r] = tile[tx][i];
  }
}

// ------------------------------------------------------------ weight gradients
// Block tile 64 WF x 64 WF of the output (four waves in 2 x 2, each
// 32 WF x 32 WF: WF x WF MFMA blocks), 64 stacked rows per step.  Each
// thread loads 4 rows x 8 columns of each operand per 128 columns of the
// tile, turns them into 8 columns x 4 rows in registers and writes them to
// LDS as [column][row] (rows contiguous), so the MFMA fragments (8
// consecutive rows of one column) are single 16-byte LDS reads.  The next
// step's global loads are in flight while the current step computes.  With
// WF = 4 each fragment feeds four MFMAs, which keeps the LDS reads under the
// MFMA time; WF = 2 serves narrow products.
constexpr int WG_LD = 72;   // 64 rows + 8 pad (bf16) per LDS column

__device__ __forceinline__ void wg_store_t(bf16_t* s, const uint4* v, int col0, int rg) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint2 u = {bf_elem(v[0], j) | (bf_elem(v[1], j) << 16), bf_elem(v[2], j) | (bf_elem(v[3], j) << 16)};
    *(uint2*)&s[(col0 + j) * WG_LD + 4 * rg] = u;
  }
}

template <int WF>
__global__ __launch_bounds__(256, WF == 4 ? 1 : 2) void wgrad_kernel(WgradArgs a) {
  constexpr int TILE = 64 * WF, NP = TILE / 128;
  __shared__ __attribute__((aligned(16))) bf16_t sA[TILE * WG_LD];
  __shared__ __attribute__((aligned(16))) bf16_t sX[TILE * WG_LD];
  const int tilesN = (a.Nc + TILE - 1) / TILE, tilesK = (a.Kc + TILE - 1) / TILE, nt = tilesN * tilesK;
  // blocks go to the XCDs round-robin by linear index; a single product
  // gives each XCD a rectangle of tiles (its blocks share row slabs in its
  // L2); grouped products take the tiles of one group after another
  int g, tn, tk;
  {
    // the tiles of one group (one expert, or the whole dense matrix) are
    // dealt to the XCDs (workgroup i runs on XCD i % 8) as px x py blocks of
    // neighbouring (n, k) tiles, so an XCD's L2 serves each dY / X slab to
    // several of its tiles
    const int bid = blockIdx.x, L = bid % nt, xcd = L % RDT_NUM_XCD, j = L / RDT_NUM_XCD;
    int px = 0;
    if (nt % RDT_NUM_XCD == 0) {
      if (tilesN % 4 == 0 && tilesK % 2 == 0) px = 4;
      else if (tilesN % 2 == 0 && tilesK % 4 == 0) px = 2;
      else if (tilesN % 8 == 0) px = 8;
      else if (tilesK % 8 == 0) px = 1;
    }
    if (px) {
      const int py = RDT_NUM_XCD / px, wn_ = tilesN / px, wk_ = tilesK / py;
      g = bid / nt;
      tn = (xcd % px) * wn_ + j % wn_;
      tk = (xcd / px) * wk_ + j / wn_;
    } else {
      g = bid / nt;
      tn = (bid % nt) % tilesN;
      tk = (bid % nt) / tilesN;
    }
  }
  const int z = blockIdx.z;
  const int n0 = tn * TILE, k0 = tk * TILE;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5;
  const int wn = w >> 1, wk = w & 1;
  const int rg = tid & 15, cc = tid >> 4;
  floatx16_t acc[WF][WF];
#pragma unroll
  for (int i = 0; i < WF; ++i)
#pragma unroll
    for (int j = 0; j < WF; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const int t_lo = (int)((int64_t)z * a.n_loops / a.splits), t_hi = (int)((int64_t)(z + 1) * a.n_loops / a.splits);
  // chunk iterator over (loop, 64-row step) of this group
  // this group's row range in every loop, read once (a global read at each
  // segment change would stall the load stream)
  __shared__ int s_lo[RDT_MAX_WGRAD_LOOPS], s_hi[RDT_MAX_WGRAD_LOOPS];
  for (int i = tid; i < t_hi - t_lo; i += blockDim.x) {
    const int32_t* o = a.off ? a.off + (int64_t)(t_lo + i) * (a.G + 1) + g : nullptr;
    s_lo[i] = o ? o[0] : 0;
    s_hi[i] = o ? o[1] : a.rows;
  }
  __syncthreads();
  const bf16_t* Ab = (const bf16_t*)a.A + n0 + 8 * cc;
  const bf16_t* Xb = (const bf16_t*)a.X + k0 + 8 * cc;
  const bf16_t *Abt = Ab, *Xbt = Xb;   // this loop's rows
  int t = t_lo - 1;
  int64_t m0 = 0, r1 = 0;
  auto advance = [&]() -> bool {
    m0 += 64;
    while (m0 >= r1) {
      if (++t >= t_hi) return false;
      m0 = s_lo[t - t_lo];
      r1 = s_hi[t - t_lo];
      Abt = Ab + (int64_t)t * a.a_loop_stride;
      Xbt = Xb + (int64_t)t * a.x_loop_stride;
    }
    return true;
  };
  uint4 va[NP][4], vx[NP][4];
  // tiles wholly inside the output take plain 16-byte loads
  const bool full = n0 + TILE <= a.Nc && k0 + TILE <= a.Kc;
  auto load = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + 4 * rg + i;
      const bool ok = m < r1;
      const int64_t mm = ok ? m : r1 - 1;   // a row of the chunk; zeroed below when past its end
      const bf16_t* ar = Abt + mm * a.lda;
      const bf16_t* xr = Xbt + mm * a.ldx;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        if (full) {
          va[p][i] = *(const uint4*)(ar + 128 * p);
          vx[p][i] = *(const uint4*)(xr + 128 * p);
        } else {
          va[p][i] = load8(ar + 128 * p, a.Nc - (n0 + 8 * cc + 128 * p));
          vx[p][i] = load8(xr + 128 * p, a.Kc - (k0 + 8 * cc + 128 * p));
        }
        if (!ok) va[p][i] = vx[p][i] = uint4{0u, 0u, 0u, 0u};
      }
    }
  };
  m0 = -64;
  bool more = advance();
  if (more) load();
  while (more) {
    __syncthreads();
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      wg_store_t(sA, va[p], 8 * cc + 128 * p, rg);
      wg_store_t(sX, vx[p], 8 * cc + 128 * p, rg);
    }
    __syncthreads();
    more = advance();
    if (more) load();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t af[WF], xf[WF];
#pragma unroll
      for (int i = 0; i < WF; ++i)
        af[i] = *(const bf16x8_t*)&sA[(wn * 32 * WF + i * 32 + (lane & 31)) * WG_LD + 16 * ks + 8 * half];
#pragma unroll
      for (int j = 0; j < WF; ++j)
        xf[j] = *(const bf16x8_t*)&sX[(wk * 32 * WF + j * 32 + (lane & 31)) * WG_LD + 16 * ks + 8 * half];
#pragma unroll
      for (int i = 0; i < WF; ++i)
#pragma unroll
        for (int j = 0; j < WF; ++j) acc[i][j] = mfma32(af[i], xf[j], acc[i][j]);
      // one k-step's fragments live at a time (the 4 x 4 accumulators fill
      // the AGPRs)
      if constexpr (WF == 4) __builtin_amdgcn_sched_barrier(0);
    }
  }
  float* Cb = a.C + (int64_t)g * a.c_gstride + (int64_t)z * a.c_split_stride;
#pragma unroll
  for (int i = 0; i < WF; ++i)
#pragma unroll
    for (int j = 0; j < WF; ++j) {
      const int k = k0 + wk * 32 * WF + j * 32 + (lane & 31);
      if (k >= a.Kc) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = n0 + wn * 32 * WF + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (n < a.Nc) {
          float* p = Cb + (int64_t)n * a.ldc + k;
          *p = a.accumulate ? *p + acc[i][j][r] : acc[i][j][r];
        }
      }
    }
}

// Large products: 256 x 256 output tile, eight waves (2 along n x 4 along
// k, each 128 x 64: 4 x 2 MFMA blocks), two per SIMD.  LDS is
// double-buffered: step i computes from one buffer while the rows of step
// i + 1 (already in registers) are transposed into the other and those of
// step i + 2 are loaded from memory, with one barrier per step; the
// transposition's VALU and LDS writes run under the MFMAs queued before it.
__global__ __launch_bounds__(512, 1) void wgrad8_kernel(WgradArgs a) {
  constexpr int TILE = 256;
  __shared__ __attribute__((aligned(16))) bf16_t sA[2][TILE * WG_LD];
  __shared__ __attribute__((aligned(16))) bf16_t sX[2][TILE * WG_LD];
  const int tilesN = (a.Nc + TILE - 1) / TILE, tilesK = (a.Kc + TILE - 1) / TILE, nt = tilesN * tilesK;
  int g, tn, tk;
  {
    // the tiles of one group (one expert, or the whole dense matrix) are
    // dealt to the XCDs (workgroup i runs on XCD i % 8) as px x py blocks of
    // neighbouring (n, k) tiles, so an XCD's L2 serves each dY / X slab to
    // several of its tiles
    const int bid = blockIdx.x, L = bid % nt, xcd = L % RDT_NUM_XCD, j = L / RDT_NUM_XCD;
    int px = 0;
    if (nt % RDT_NUM_XCD == 0) {
      if (tilesN % 4 == 0 && tilesK % 2 == 0) px = 4;
      else if (tilesN % 2 == 0 && tilesK % 4 == 0) px = 2;
      else if (tilesN % 8 == 0) px = 8;
      else if (tilesK % 8 == 0) px = 1;
    }
    if (px) {
      const int py = RDT_NUM_XCD / px, wn_ = tilesN / px, wk_ = tilesK / py;
      g = bid / nt;
      tn = (xcd % px) * wn_ + j % wn_;
      tk = (xcd / px) * wk_ + j / wn_;
    } else {
      g = bid / nt;
      tn = (bid % nt) % tilesN;
      tk = (bid % nt) / tilesN;
    }
  }
  const int z = blockIdx.z;
  const int n0 = tn * TILE, k0 = tk * TILE;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5;
  const int wn = w >> 2, wk = w & 3;
  const int rg = tid & 15, cc = tid >> 4;   // rows 4 rg .. +3, columns 8 cc .. +7
  floatx16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const int t_lo = (int)((int64_t)z * a.n_loops / a.splits), t_hi = (int)((int64_t)(z + 1) * a.n_loops / a.splits);
  __shared__ int s_lo[RDT_MAX_WGRAD_LOOPS], s_hi[RDT_MAX_WGRAD_LOOPS];
  for (int i = tid; i < t_hi - t_lo; i += blockDim.x) {
    const int32_t* o = a.off ? a.off + (int64_t)(t_lo + i) * (a.G + 1) + g : nullptr;
    s_lo[i] = o ? o[0] : 0;
    s_hi[i] = o ? o[1] : a.rows;
  }
  __syncthreads();
  const bf16_t* Ab = (const bf16_t*)a.A + n0 + 8 * cc;
  const bf16_t* Xb = (const bf16_t*)a.X + k0 + 8 * cc;
  // The rows of loops t_lo .. t_hi-1 (loop t: rows s_lo .. s_hi-1 at its own
  // base) are taken as one sequence, 64 per step, so a step may end one
  // loop's rows and start the next loop's; only the last step has rows past
  // the end (zero).  A position in the sequence is (loop t, row m); `norm`
  // moves a position that lies past its loop's end into the next loops.
  auto norm = [&](int& t, int64_t& m) {
    while (t < t_hi && m >= s_hi[t - t_lo]) {
      const int64_t over = m - s_hi[t - t_lo];
      if (++t < t_hi) m = s_lo[t - t_lo] + over;
    }
  };
  int t = t_lo;                                   // first row of the next step to load
  int64_t m0 = t_lo < t_hi ? s_lo[0] : 0;
  norm(t, m0);
  const bool full = n0 + TILE <= a.Nc && k0 + TILE <= a.Kc;
  const int na = a.Nc - (n0 + 8 * cc), nx = a.Kc - (k0 + 8 * cc);
  uint4 va[4], vx[4];
  // loads the thread's 4 rows (4 rg .. 4 rg + 3 of the step starting at
  // (t, m0)) and moves (t, m0) to the next step; false when no rows are left
  auto load_step = [&]() -> bool {
    if (t >= t_hi) return false;
    int tr = t;
    int64_t mr = m0 + 4 * rg;
    norm(tr, mr);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = tr < t_hi;
      const int tc = ok ? tr : t;
      const int64_t mc = ok ? mr : m0;   // a valid row; zeroed below
      const bf16_t* ar = Ab + (int64_t)tc * a.a_loop_stride + mc * a.lda;
      const bf16_t* xr = Xb + (int64_t)tc * a.x_loop_stride + mc * a.ldx;
      if (full) {
        va[i] = *(const uint4*)ar;
        vx[i] = *(const uint4*)xr;
      } else {
        va[i] = load8(ar, na);
        vx[i] = load8(xr, nx);
      }
      if (!ok) va[i] = vx[i] = uint4{0u, 0u, 0u, 0u};
      if (i < 3) {
        ++mr;
        norm(tr, mr);
      }
    }
    m0 += 64;
    norm(t, m0);
    return true;
  };
  bool have = load_step();
  if (have) {
    wg_store_t(sA[0], va, 8 * cc, rg);
    wg_store_t(sX[0], vx, 8 * cc, rg);
  }
  bool more = have && load_step();
  __syncthreads();
  int cur = 0;
  while (have) {
    bool more2 = false;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t af[4], xf[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *(const bf16x8_t*)&sA[cur][(wn * 128 + i * 32 + (lane & 31)) * WG_LD + 16 * ks + 8 * half];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        xf[j] = *(const bf16x8_t*)&sX[cur][(wk * 64 + j * 32 + (lane & 31)) * WG_LD + 16 * ks + 8 * half];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], xf[j], acc[i][j]);
      if (ks == 0) {
        // the rows of step i + 1 go to the other buffer, then the loads of
        // step i + 2 are issued at once, a whole step ahead of their use
        __builtin_amdgcn_sched_barrier(0);
        if (more) {
          wg_store_t(sA[cur ^ 1], va, 8 * cc, rg);
          wg_store_t(sX[cur ^ 1], vx, 8 * cc, rg);
        }
        more2 = more && load_step();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
    have = more;
    more = more2;
    cur ^= 1;
  }
  float* Cb = a.C + (int64_t)g * a.c_gstride + (int64_t)z * a.c_split_stride;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int k = k0 + wk * 64 + j * 32 + (lane & 31);
      if (k >= a.Kc) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = n0 + wn * 128 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (n < a.Nc) {
          float* p = Cb + (int64_t)n * a.ldc + k;
          *p = a.accumulate ? *p + acc[i][j][r] : acc[i][j][r];
        }
      }
    }
}

// dWr[e][c] partial sums: block (256 columns, expert e, row slice z) takes
// rows z, z + RW_SLICES, ... of each loop's rows of e; the slices are added
// afterwards in order
#define RW_SLICES 16
__global__ __launch_bounds__(256) void router_wgrad_kernel(const float* __restrict__ dz,
                                                           const bf16_t* __restrict__ fperm,
                                                           const int32_t* __restrict__ off, int n_loops, int NK,
                                                           int E, int D, float* __restrict__ part) {
  const int e = blockIdx.y, z = blockIdx.z, c = blockIdx.x * 256 + threadIdx.x;
  if (c >= D) return;
  float acc0 = 0.f, acc1 = 0.f;
  for (int t = 0; t < n_loops; ++t) {
    const int32_t* o = off + (int64_t)t * (E + 1);
    const int m1 = o[e + 1];
    int m = o[e] + z;
    for (; m + RW_SLICES < m1; m += 2 * RW_SLICES) {
      const int64_t row = (int64_t)t * NK + m;
      acc0 = fmaf(dz[row], bf2f(fperm[row * D + c]), acc0);
      acc1 = fmaf(dz[row + RW_SLICES], bf2f(fperm[(row + RW_SLICES) * D + c]), acc1);
    }
    if (m < m1) {
      const int64_t row = (int64_t)t * NK + m;
      acc0 = fmaf(dz[row], bf2f(fperm[row * D + c]), acc0);
    }
  }
  part[((int64_t)z * E + e) * D + c] = acc0 + acc1;
}

// dst[m] = src[perm[m]] (bf16 rows of D)
__global__ __launch_bounds__(256) void gather_rows_kernel(const bf16_t* __restrict__ src,
                                                          const int32_t* __restrict__ perm, int M, int D,
                                                          bf16_t* __restrict__ dst) {
  const int64_t idx = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (idx >= (int64_t)M * D) return;
  const int64_t m = idx / D;
  const int c = (int)(idx - m * D);
  *(uint4*)(dst + idx) = *(const uint4*)(src + (int64_t)perm[m] * D + c);
}

// ------------------------------------------------------------ attention backward
constexpr int AQ = 64;      // queries per tile (dK / dV kernel), keys per tile (dQ kernel)
constexpr int LQ = 136;     // row stride of [row][128 d] LDS tiles (bf16)
constexpr int LT = 72;      // row stride of [d][64] transposed LDS tiles (bf16)

__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(const bf16_t* __restrict__ o,
                                                            const bf16_t* __restrict__ dO, int N, int H, int T,
                                                            float* __restrict__ Dq) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= N * H) return;
  const int n = idx / H, h = idx - n * H;
  const bf16_t* po = o + (int64_t)n * H * 128 + h * 128;
  const bf16_t* pd = dO + (int64_t)n * H * 128 + h * 128;
  float s = 0.f;
  for (int d = 0; d < 128; d += 4) s += dot4(ldbf4(po + d), ldbf4(pd + d));
  const int b = n / T, i = n - b * T;
  Dq[((int64_t)b * H + h) * T + i] = s;
}

// global -> LDS copy of 16 bytes per lane into the 1 KB window at lds (lane
// i fills bytes 16 i .. 16 i + 15), as asm so the compiler adds no wait of
// its own before later LDS reads: the kernels wait explicitly before the
// barrier that publishes a buffer.
__device__ __forceinline__ void dma16(const void* src, const void* lds) {
  typedef __attribute__((address_space(3))) void lds_void_t;
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void_t*)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src), "s"(m) : "memory", "m0");
}

// Row tiles [row][16 chunks of 8 d] keep chunk c at c ^ rswz(row): the
// lanes of a quarter-wave read rows in the permuted order of kperm, which
// this sends to 16 distinct positions.  Transposed tiles [d][8 chunks of 8]
// keep chunk c at c ^ tswz(d).
__device__ __forceinline__ int rswz(int r) { return (r & 7) | (((r >> 4) & 1) << 3); }
__device__ __forceinline__ int tswz(int d) { return (d >> 1) & 7; }
// score row read by lane i of a 32-row block: lane half h of the result
// then holds rows 16 h .. 16 h + 15 in order
__device__ __forceinline__ int kperm(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

// one block per (key tile of 128 keys, b, kv head g); wave w owns keys
// 32 w .. 32 w + 31 of the tile with dK and dV for all 128 d in registers
// and walks the 64-query tiles at and after its keys for every query head
// of the group.  The next query tile streams into the other LDS buffer
// while the current one is used.
struct alignas(16) DkdvBuf {
  uint4 q[AQ * 16], dO[AQ * 16], qt[128 * 8], dOt[128 * 8];
  float L[AQ], Dl[AQ];
};

__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dO, const bf16_t* __restrict__ qt, const bf16_t* __restrict__ dOt,
    const float* __restrict__ lse2, const float* __restrict__ Dq, float* __restrict__ dK, float* __restrict__ dV,
    int B, int H, int G, int T, int Tp, int cap, float scale_log2, float scale) {
  __shared__ DkdvBuf buf[2];
  const int BG = B * G, kt = blockIdx.x / BG, bg = blockIdx.x - kt * BG;
  const int b = bg / G, g = bg - b * G, rep = H / G;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5;
  const int kw0 = kt * 128 + w * 32, kl = kw0 + (lane & 31);
  bf16x8_t kf[8], vf[8];
  {
    const bf16_t* kr = k + ((int64_t)bg * cap + kl) * 128;
    const bf16_t* vr = v + ((int64_t)bg * cap + kl) * 128;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      uint4 a = uint4{0u, 0u, 0u, 0u}, c = a;
      if (kl < T) {
        a = *(const uint4*)(kr + 16 * ds + 8 * half);
        c = *(const uint4*)(vr + 16 * ds + 8 * half);
      }
      kf[ds] = as_frag(a);
      vf[ds] = as_frag(c);
    }
  }
  floatx16_t accK[4], accV[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) accK[i][e] = accV[i][e] = 0.f;
  const int nqt = (T + AQ - 1) / AQ, qt0 = (kt * 128) / AQ, nq = nqt - qt0, ntile = rep * nq;
  float Lr = 0.f, Dr = 0.f;
  // issue tile i (query head g rep + i / nq, query tile qt0 + i % nq) into buffer bb
  auto issue = [&](int i, int bb) {
    const int h = g * rep + i / nq, q0 = (qt0 + i % nq) * AQ;
    const bf16_t* qh = q + (int64_t)(b * H + h) * T * 128;
    const bf16_t* qth = qt + (int64_t)(b * H + h) * 128 * Tp;
    const bf16_t* dOth = dOt + (int64_t)(b * H + h) * 128 * Tp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sl = (j * 4 + w) * 64 + lane;
      const int row = sl >> 4, lc = (sl & 15) ^ rswz(row), qq = min(q0 + row, T - 1);
      dma16(qh + (int64_t)qq * 128 + lc * 8, &buf[bb].q[(j * 4 + w) * 64]);
      dma16(dO + ((int64_t)(b * T + qq) * H + h) * 128 + lc * 8, &buf[bb].dO[(j * 4 + w) * 64]);
      const int d = sl >> 3, tc = (sl & 7) ^ tswz(d);
      dma16(qth + (int64_t)d * Tp + q0 + tc * 8, &buf[bb].qt[(j * 4 + w) * 64]);
      dma16(dOth + (int64_t)d * Tp + q0 + tc * 8, &buf[bb].dOt[(j * 4 + w) * 64]);
    }
    if (tid < AQ) {
      const int qq = q0 + tid;
      const int64_t o = (int64_t)(b * H + h) * T + qq;
      Lr = qq < T ? lse2[o] : 0.f;
      Dr = qq < T ? Dq[o] : 0.f;
    }
  };
  if (ntile > 0) issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  if (tid < AQ) {
    buf[0].L[tid] = Lr;
    buf[0].Dl[tid] = Dr;
  }
  __syncthreads();
  const int myrow = kperm(lane & 31);
  for (int i = 0; i < ntile; ++i) {
    const int bb = i & 1;
    if (i + 1 < ntile) issue(i + 1, bb ^ 1);
    const int q0 = (qt0 + i % nq) * AQ;
    const DkdvBuf& cb = buf[bb];
    // the scores of one query tile against this wave's keys; tiles whose
    // queries all follow the wave's keys and end before T need no mask
    auto tile = [&](auto masked) {
      // S and dP of both 32-query blocks first, so the exponentials of the
      // first block can issue while the second block's products run
      floatx16_t Sq[2], dPq[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) Sq[qb][e] = dPq[qb][e] = 0.f;
        const int qrow = qb * 32 + myrow;
#pragma unroll
        for (int ds = 0; ds < 8; ++ds) {
          const int pc = (2 * ds + half) ^ rswz(qrow);
          Sq[qb] = mfma32(as_frag(cb.q[qrow * 16 + pc]), kf[ds], Sq[qb]);
          dPq[qb] = mfma32(as_frag(cb.dO[qrow * 16 + pc]), vf[ds], dPq[qb]);
        }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const floatx16_t& S = Sq[qb];
        const floatx16_t& dP = dPq[qb];
        // this lane: key kl, queries q0 + 32 qb + 16 half + r
        const int qbase = qb * 32 + 16 * half;
        float p[16], dsv[16];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const float4 L4 = *(const float4*)&cb.L[qbase + 4 * r4];
          const float4 D4 = *(const float4*)&cb.Dl[qbase + 4 * r4];
          const float Ls[4] = {L4.x, L4.y, L4.z, L4.w}, Ds[4] = {D4.x, D4.y, D4.z, D4.w};
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int r = 4 * r4 + x, qq = q0 + qbase + r;
            const bool ok = !decltype(masked)::value || (qq < T && kl <= qq && kl < T);
            const float pr = ok ? __builtin_amdgcn_exp2f(S[r] * scale_log2 - Ls[x]) : 0.f;
            p[r] = pr;
            dsv[r] = pr * (dP[r] - Ds[x]);
          }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8_t pa = pack8(p + 8 * ks), sa = pack8(dsv + 8 * ks);
          const int lc = 4 * qb + 2 * half + ks;
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const int d = db * 32 + (lane & 31), pc = lc ^ tswz(d);
            accV[db] = mfma32(pa, as_frag(cb.dOt[d * 8 + pc]), accV[db]);
            accK[db] = mfma32(sa, as_frag(cb.qt[d * 8 + pc]), accK[db]);
          }
        }
      }
    };
    if (kw0 <= q0 + AQ - 1) {   // else every query of the tile precedes this wave's keys
      if (kw0 + 31 <= q0 && q0 + AQ <= T) tile(std::false_type{});
      else tile(std::true_type{});
    }
    __builtin_amdgcn_s_waitcnt(0);
    if (i + 1 < ntile && tid < AQ) {
      buf[bb ^ 1].L[tid] = Lr;
      buf[bb ^ 1].Dl[tid] = Dr;
    }
    __syncthreads();
  }
  float* dKb = dK + (int64_t)bg * T * 128;
  float* dVb = dV + (int64_t)bg * T * 128;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (key < T) {
        const int64_t i = (int64_t)key * 128 + db * 32 + (lane & 31);
        dKb[i] = accK[db][r] * scale;
        dVb[i] = accV[db][r];
      }
    }
}

// one block per (query tile of 128, b, head h); wave w owns queries
// 32 w .. 32 w + 31 and walks the 64-key tiles up to its diagonal, the
// next tile streaming into the other LDS buffer
struct alignas(16) DqBuf {
  uint4 k[AQ * 16], v[AQ * 16], kt[128 * 8];
};

__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dO, const bf16_t* __restrict__ kt, const float* __restrict__ lse2,
    const float* __restrict__ Dq, float* __restrict__ dQ, int B, int H, int G, int T, int cap, float scale_log2,
    float scale) {
  __shared__ DqBuf buf[1];
  const int BH = B * H, nqt = (T + 127) / 128;
  const int qti = nqt - 1 - (int)(blockIdx.x / BH), bh = blockIdx.x % BH;
  const int b = bh / H, h = bh - b * H, g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5;
  const int qw0 = qti * 128 + w * 32, ql = qw0 + (lane & 31);
  bf16x8_t qf[8], df[8];
  {
    const bf16_t* qr = q + ((int64_t)bh * T + min(ql, T - 1)) * 128;
    const bf16_t* dr = dO + ((int64_t)(b * T + min(ql, T - 1)) * H + h) * 128;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      uint4 a = *(const uint4*)(qr + 16 * ds + 8 * half), c = *(const uint4*)(dr + 16 * ds + 8 * half);
      if (ql >= T) a = c = uint4{0u, 0u, 0u, 0u};
      qf[ds] = as_frag(a);
      df[ds] = as_frag(c);
    }
  }
  const int qlim = ql < T ? ql : -1;   // last key this lane's query sees (none past T)
  const float Lq = ql < T ? lse2[(int64_t)bh * T + ql] : 0.f;
  const float Dqq = ql < T ? Dq[(int64_t)bh * T + ql] : 0.f;
  floatx16_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  const int bg = b * G + g;
  const bf16_t* kb = k + (int64_t)bg * cap * 128;
  const bf16_t* vb = v + (int64_t)bg * cap * 128;
  const bf16_t* ktb = kt + (int64_t)bg * 128 * cap;
  const int kend = min(T, qti * 128 + 128);
  const int nkt = (kend + AQ - 1) / AQ;
  auto issue = [&](int i, int bb) {
    const int k0 = i * AQ;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sl = (j * 4 + w) * 64 + lane;
      const int row = sl >> 4, lc = (sl & 15) ^ rswz(row);
      dma16(kb + (int64_t)(k0 + row) * 128 + lc * 8, &buf[bb].k[(j * 4 + w) * 64]);
      dma16(vb + (int64_t)(k0 + row) * 128 + lc * 8, &buf[bb].v[(j * 4 + w) * 64]);
      const int d = sl >> 3, tc = (sl & 7) ^ tswz(d);
      dma16(ktb + (int64_t)d * cap + k0 + tc * 8, &buf[bb].kt[(j * 4 + w) * 64]);
    }
  };
  const int myrow = kperm(lane & 31);
  for (int i = 0; i < nkt; ++i) {
    issue(i, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int k0 = i * AQ;
    const DqBuf& cb = buf[0];
    if (k0 <= qw0 + 31) {   // else every key of the tile follows this wave's queries
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        floatx16_t S, dP;
#pragma unroll
        for (int e = 0; e < 16; ++e) S[e] = dP[e] = 0.f;
        const int krow = kb2 * 32 + myrow;
#pragma unroll
        for (int ds = 0; ds < 8; ++ds) {
          const int pc = (2 * ds + half) ^ rswz(krow);
          S = mfma32(as_frag(cb.k[krow * 16 + pc]), qf[ds], S);
          dP = mfma32(as_frag(cb.v[krow * 16 + pc]), df[ds], dP);
        }
        // this lane: query ql, keys k0 + 32 kb2 + 16 half + r
        float dsv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb2 * 32 + 16 * half + r;
          const bool ok = key <= qlim;
          const float pr = ok ? __builtin_amdgcn_exp2f(S[r] * scale_log2 - Lq) : 0.f;
          dsv[r] = pr * (dP[r] - Dqq);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8_t sa = pack8(dsv + 8 * ks);
          const int lc = 4 * kb2 + 2 * half + ks;
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            const int d = db * 32 + (lane & 31), pc = lc ^ tswz(d);
            acc[db] = mfma32(sa, as_frag(cb.kt[d * 8 + pc]), acc[db]);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  float* dQb = dQ + (int64_t)bh * T * 128;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qq = qw0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (qq < T) dQb[(int64_t)qq * 128 + db * 32 + (lane & 31)] = acc[db][r] * scale;
    }
}

// dqkv row n = b T + i: [dq heads | dk heads | dv heads], RoPE taken back
// on the q and k parts (pairs rotated by minus the angle)
__global__ __launch_bounds__(256) void qkv_bwd_kernel(const float* __restrict__ dQ, const float* __restrict__ dK,
                                                      const float* __restrict__ dV, const float* __restrict__ rcos,
                                                      const float* __restrict__ rsin, int B, int T, int H, int G,
                                                      bf16_t* __restrict__ dqkv) {
  const int W = (H + 2 * G) * 128, pairs = W / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)B * T * pairs) return;
  const int n = (int)(idx / pairs), col = 2 * (int)(idx - (int64_t)n * pairs);
  const int b = n / T, i = n - b * T;
  const int hd = col >> 7, d = col & 127;
  float x0, x1;
  bool rot = true;
  if (hd < H) {
    const float* p = dQ + (((int64_t)b * H + hd) * T + i) * 128 + d;
    x0 = p[0];
    x1 = p[1];
  } else if (hd < H + G) {
    const float* p = dK + (((int64_t)b * G + (hd - H)) * T + i) * 128 + d;
    x0 = p[0];
    x1 = p[1];
  } else {
    const float* p = dV + (((int64_t)b * G + (hd - H - G)) * T + i) * 128 + d;
    x0 = p[0];
    x1 = p[1];
    rot = false;
  }
  if (rot) {
    const float c = rcos[(int64_t)i * 64 + (d >> 1)], s = rsin[(int64_t)i * 64 + (d >> 1)];
    const float y0 = x0 * c + x1 * s, y1 = x1 * c - x0 * s;
    x0 = y0;
    x1 = y1;
  }
  *(uint32_t*)(dqkv + (int64_t)n * W + col) = pack_bf16x2(x0, x1);
}

// ------------------------------------------------------------ SwiGLU
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const bf16_t* __restrict__ gu, int M, int F,
                                                         bf16_t* __restrict__ act) {
  const int64_t idx = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (idx >= (int64_t)M * F) return;
  const int64_t m = idx / F;
  const int f = (int)(idx - m * F);
  const float4 G = ldbf4(gu + m * 2 * F + f), U = ldbf4(gu + m * 2 * F + F + f);
  stbf4(act + m * F + f, float4{silu_f(G.x) * U.x, silu_f(G.y) * U.y, silu_f(G.z) * U.z, silu_f(G.w) * U.w});
}

__device__ __forceinline__ void swiglu_grad(float g, float u, float da, float& dg, float& du) {
  const float sg = 1.0f / (1.0f + __expf(-g));
  du = da * g * sg;
  dg = da * u * sg * (1.0f + g * (1.0f - sg));
}

__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const bf16_t* __restrict__ gu, const float* __restrict__ dact,
                                                         int M, int F, bf16_t* __restrict__ dgu) {
  const int64_t idx = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (idx >= (int64_t)M * F) return;
  const int64_t m = idx / F;
  const int f = (int)(idx - m * F);
  const float4 G = ldbf4(gu + m * 2 * F + f), U = ldbf4(gu + m * 2 * F + F + f), dA = ld4(dact + m * F + f);
  float4 dG, dU;
  swiglu_grad(G.x, U.x, dA.x, dG.x, dU.x);
  swiglu_grad(G.y, U.y, dA.y, dG.y, dU.y);
  swiglu_grad(G.z, U.z, dA.z, dG.z, dU.z);
  swiglu_grad(G.w, U.w, dA.w, dG.w, dU.w);
  stbf4(dgu + m * 2 * F + f, dG);
  stbf4(dgu + m * 2 * F + F + f, dU);
}

// ------------------------------------------------------------ row-wise passes
// One wave per row (rows n = wave, wave + RDT_BWD_WAVES, ...); lane l owns
// the float4 columns 4 l + 256 j.

#define ROW_LOOP_BEGIN                                                  \
  const int lane = threadIdx.x & 63;                                   \
  const int wg = blockIdx.x * 4 + (threadIdx.x >> 6);                  \
  for (int n = wg; n < N; n += RDT_BWD_WAVES) {
#define ROW_LOOP_END }

__global__ __launch_bounds__(256) void act_prep_kernel(const float* __restrict__ states, int64_t sstride,
                                                       const float* __restrict__ dy,
                                                       const float* __restrict__ hw, const float* __restrict__ hb,
                                                       const int32_t* __restrict__ hc, int L, int N, int D,
                                                       float* __restrict__ w_act, float* __restrict__ z_act,
                                                       float* __restrict__ part_hw, float* __restrict__ part_hb) {
  ROW_LOOP_BEGIN
  // lane t keeps p_t and G_t = <dy, h_{t+1}>
  float my_p = 0.f, my_G = 0.f;
  const float* dyr = dy + (int64_t)n * D;
  for (int t = 0; t < L; ++t) {
    const float* sr = states + (int64_t)t * sstride + (int64_t)n * D;
    float zp = 0.f, gp = 0.f;
    for (int c = 4 * lane; c < D; c += 256) {
      const float4 x = ld4(sr + c);
      zp += dot4(x, ld4(hw + c));
      gp += dot4(x, ld4(dyr + c));
    }
    zp = wave_sum(zp);
    gp = wave_sum(gp);
    if (lane == t) {
      my_p = 1.0f / (1.0f + expf(-(zp + hb[0])));
      my_G = gp;
    }
  }
  const int th = hc[n] - 1;   // halting loop
  float cum_th = 0.f, G_th = 0.f;
  for (int t = 0; t < L; ++t) {
    const float pt = __shfl(my_p, t, 64), Gt = __shfl(my_G, t, 64);
    if (t < th) cum_th += pt;
    if (t == th) G_th = Gt;
  }
  const float rem = 1.0f - cum_th;
  if (lane < L) {
    const int t = lane;
    float wv = 0.f, zv = 0.f;
    if (t < th) {
      wv = my_p;
      const float dp = my_G - (rem > 0.f ? G_th : 0.f);
      zv = dp * my_p * (1.0f - my_p);
    } else if (t == th) {
      wv = rem > 0.f ? rem : 0.f;
    }
    w_act[(int64_t)t * N + n] = wv;
    z_act[(int64_t)t * N + n] = zv;
  }
  // d halt_w += sum_t z_t h_{t+1}; d halt_b += sum_t z_t
  float zsum = 0.f;
  float* ph = part_hw + (int64_t)wg * D;
  for (int t = 0; t < L && t < th; ++t) {
    const float zt = __shfl(my_p, t, 64) * (1.0f - __shfl(my_p, t, 64)) *
                     (__shfl(my_G, t, 64) - (rem > 0.f ? G_th : 0.f));
    zsum += zt;
    const float* sr = states + (int64_t)t * sstride + (int64_t)n * D;
    for (int c = 4 * lane; c < D; c += 256) st4(ph + c, fma4(zt, ld4(sr + c), ld4(ph + c)));
  }
  if (lane == 0) part_hb[wg] += zsum;
  ROW_LOOP_END
}

// Tail backward, first pass (no reductions): the state gradient with this
// loop's ACT terms, g_full = g + w dy + z halt_w; tau recomputed from its
// parts; dtau = g_full (the LoRA term is added by a product afterwards);
// the carry A g_full, de += B g_full and the partial sums of g_full h_prev
// (dA) and g_full e (dB).
__global__ __launch_bounds__(256) void tail_bwd_rows_kernel(TailBwdArgs a) {
  const int N = a.N, D = a.D, k = a.k;
  ROW_LOOP_BEGIN
  const int64_t ro = (int64_t)n * D;
  const float wa = a.w_act ? a.w_act[n] : 0.f, za = a.z_act ? a.z_act[n] : 0.f;
  const bf16_t* yb = (const bf16_t*)a.y;
  const bf16_t* ysb = (const bf16_t*)a.ys;
  int rows_j[8];
  float gates[8];
  for (int j = 0; j < k; ++j) {
    rows_j[j] = a.inv[(int64_t)n * k + j];
    gates[j] = a.gate[(int64_t)n * k + j];
  }
  float* pA = a.part_A + (int64_t)wg * D;
  float* pB = a.part_B + (int64_t)wg * D;
  for (int c = 4 * lane; c < D; c += 256) {
    float4 gf = ld4(a.g + ro + c);
    if (a.w_act) gf = fma4(wa, ld4(a.dy + ro + c), gf);
    if (a.z_act) gf = fma4(za, ld4(a.halt_w + c), gf);
    float4 tv = ld4(a.x1 + ro + c);
    for (int j = 0; j < k; ++j) tv = fma4(gates[j], ldbf4(yb + (int64_t)rows_j[j] * D + c), tv);
    for (int s2 = 0; s2 < a.S; ++s2) tv = add4(tv, ldbf4(ysb + ((int64_t)s2 * N + n) * D + c));
    stbf4((bf16_t*)a.sv_g + ro + c, gf);
    stbf4((bf16_t*)a.sv_tau + ro + c, tv);
    st4(a.dtau + ro + c, gf);
    const float4 hp = ld4(a.h_prev + ro + c), ev = ld4(a.e + ro + c);
    st4(a.de + ro + c, add4(ld4(a.de + ro + c), mul4(ld4(a.Bv + c), gf)));
    st4(pA + c, add4(ld4(pA + c), mul4(gf, hp)));
    st4(pB + c, add4(ld4(pB + c), mul4(gf, ev)));
    st4(a.g_next + ro + c, mul4(ld4(a.A + c), gf));
  }
  ROW_LOOP_END
}

// LoRA backward per row from v = tau Ld^T and dw = g_full LB^T ([N][r]
// fp32): dv = dw * scale (saved, and zero-padded to 64 columns for the
// product dtau += dv Ld), the saved (tau Ld^T) * scale, and the partial
// sums of dw * v (d scale of this loop)
__global__ __launch_bounds__(256) void lora_bwd_kernel(int N, int r, const float* __restrict__ v,
                                                       const float* __restrict__ dw,
                                                       const float* __restrict__ scale, bf16_t* __restrict__ sv_wl,
                                                       bf16_t* __restrict__ sv_dv, bf16_t* __restrict__ dv_pad,
                                                       float* __restrict__ part_s) {
  ROW_LOOP_BEGIN
  const int i = lane;
  const bool in = i < r;
  const float vi = in ? v[(int64_t)n * r + i] : 0.f, dwi = in ? dw[(int64_t)n * r + i] : 0.f;
  const float si = in ? scale[i] : 0.f, dvi = dwi * si;
  if (i < RDT_LORA_LD) {
    sv_wl[(int64_t)n * RDT_LORA_LD + i] = f2bf(vi * si);
    sv_dv[(int64_t)n * RDT_LORA_LD + i] = f2bf(dvi);
  }
  dv_pad[(int64_t)n * 64 + i] = f2bf(dvi);
  if (in) part_s[(int64_t)wg * RDT_LORA_LD + i] += dwi * vi;
  ROW_LOOP_END
}

// Tail backward, last pass: with dtau complete, the gate gradients
// dgate_j = <dtau, y_j>, the routed outputs' gradient dY[inv j] = gate_j
// dtau, bf16 dtau, and the router: the gates are the softmax of the chosen
// logits, so d z_j = gate_j (dgate_j - sum_i gate_i dgate_i), 0 elsewhere.
__global__ __launch_bounds__(256) void tail_bwd_gates_kernel(TailBwdArgs a) {
  const int N = a.N, D = a.D, k = a.k;
  ROW_LOOP_BEGIN
  const int64_t ro = (int64_t)n * D;
  const bf16_t* yb = (const bf16_t*)a.y;
  int rows_j[8];
  float gates[8], dg[8];
  for (int j = 0; j < k; ++j) {
    rows_j[j] = a.inv[(int64_t)n * k + j];
    gates[j] = a.gate[(int64_t)n * k + j];
    dg[j] = 0.f;
  }
  for (int c = 4 * lane; c < D; c += 256) {
    const float4 dt = ld4(a.dtau + ro + c);
    for (int j = 0; j < k; ++j) {
      dg[j] += dot4(dt, ldbf4(yb + (int64_t)rows_j[j] * D + c));
      stbf4((bf16_t*)a.dY + (int64_t)rows_j[j] * D + c, scl4(gates[j], dt));
    }
    stbf4((bf16_t*)a.dtau_bf + ro + c, dt);
  }
  float gd = 0.f;
  for (int j = 0; j < k; ++j) {
    dg[j] = wave_sum(dg[j]);
    gd += gates[j] * dg[j];
  }
  if (lane == 0)
    for (int j = 0; j < k; ++j) {
      const float dz = gates[j] * (dg[j] - gd);
      a.dz[(int64_t)n * k + j] = dz;
      a.dz_perm[rows_j[j]] = dz;
    }
  ROW_LOOP_END
}

// The same with the row's slices of x1 and of the summed gradient of f held
// in registers (NC float4 per lane, D <= 256 NC), so the second pass reads
// none of x1, df, dfp or the router rows again; same arithmetic, same order.
template <int NC>
__global__ __launch_bounds__(256) void ffn_norm_bwd_reg_kernel(int N, int D, int k, float eps,
                                                               const float* __restrict__ df,
                                                               const float* __restrict__ dfp,
                                                               const int32_t* __restrict__ inv,
                                                               const int32_t* __restrict__ sel,
                                                               const float* __restrict__ dz,
                                                               const bf16_t* __restrict__ Wr,
                                                               const float* __restrict__ x1,
                                                               const float* __restrict__ gf, float* __restrict__ dx1,
                                                               bf16_t* __restrict__ dx1_bf, float* __restrict__ part_g) {
  ROW_LOOP_BEGIN
  const int64_t ro = (int64_t)n * D;
  int rj[8], sj[8];
  float zj[8];
  for (int j = 0; j < k; ++j) {
    rj[j] = inv[(int64_t)n * k + j];
    sj[j] = sel[(int64_t)n * k + j];
    zj[j] = dz[(int64_t)n * k + j];
  }
  const float4 z4 = float4{0.f, 0.f, 0.f, 0.f};
  float4 xv[NC], dfv[NC];
  float ss = 0.f, dd = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = 4 * lane + 256 * i;
    xv[i] = dfv[i] = z4;
    if (c < D) {
      float4 v = df ? ld4(df + ro + c) : z4;
      for (int j = 0; j < k; ++j) {
        v = add4(v, ld4(dfp + (int64_t)rj[j] * D + c));
        v = fma4(zj[j], ldbf4(Wr + (int64_t)sj[j] * D + c), v);
      }
      dfv[i] = v;
      xv[i] = ld4(x1 + ro + c);
      ss += dot4(xv[i], xv[i]);
      dd += dot4(mul4(v, ld4(gf + c)), xv[i]);
    }
  }
  ss = wave_sum(ss);
  dd = wave_sum(dd);
  const float rstd = rsqrtf(ss / D + eps), m = dd * rstd * rstd / D;
  float* pg = part_g + (int64_t)wg * D;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = 4 * lane + 256 * i;
    if (c < D) {
      const float4 x = xv[i], dft = dfv[i], g4 = ld4(gf + c);
      const float4 xh = scl4(rstd, x);
      const float4 dx = scl4(rstd, float4{dft.x * g4.x - x.x * m, dft.y * g4.y - x.y * m, dft.z * g4.z - x.z * m,
                                          dft.w * g4.w - x.w * m});
      const float4 o = add4(ld4(dx1 + ro + c), dx);
      st4(dx1 + ro + c, o);
      stbf4(dx1_bf + ro + c, o);
      st4(pg + c, add4(ld4(pg + c), mul4(dft, xh)));
    }
  }
  ROW_LOOP_END
}

__global__ __launch_bounds__(256) void ffn_norm_bwd_kernel(int N, int D, int k, float eps, const float* __restrict__ df,
                                                           const float* __restrict__ dfp,
                                                           const int32_t* __restrict__ inv,
                                                           const int32_t* __restrict__ sel,
                                                           const float* __restrict__ dz, const bf16_t* __restrict__ Wr,
                                                           const float* __restrict__ x1,
                                                           const float* __restrict__ gf, float* __restrict__ dx1,
                                                           bf16_t* __restrict__ dx1_bf, float* __restrict__ part_g) {
  ROW_LOOP_BEGIN
  const int64_t ro = (int64_t)n * D;
  int rj[8], sj[8];
  float zj[8];
  for (int j = 0; j < k; ++j) {
    rj[j] = inv[(int64_t)n * k + j];
    sj[j] = sel[(int64_t)n * k + j];
    zj[j] = dz[(int64_t)n * k + j];
  }
  auto dft_at = [&](int c) {
    float4 v = df ? ld4(df + ro + c) : float4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      v = add4(v, ld4(dfp + (int64_t)rj[j] * D + c));
      v = fma4(zj[j], ldbf4(Wr + (int64_t)sj[j] * D + c), v);
    }
    return v;
  };
  float ss = 0.f, dd = 0.f;
  for (int c = 4 * lane; c < D; c += 256) {
    const float4 x = ld4(x1 + ro + c);
    ss += dot4(x, x);
    dd += dot4(mul4(dft_at(c), ld4(gf + c)), x);
  }
  ss = wave_sum(ss);
  dd = wave_sum(dd);
  const float rstd = rsqrtf(ss / D + eps), m = dd * rstd * rstd / D;
  float* pg = part_g + (int64_t)wg * D;
  for (int c = 4 * lane; c < D; c += 256) {
    const float4 x = ld4(x1 + ro + c), dft = dft_at(c), g4 = ld4(gf + c);
    const float4 xh = scl4(rstd, x);
    const float4 dx = scl4(rstd, float4{dft.x * g4.x - x.x * m, dft.y * g4.y - x.y * m, dft.z * g4.z - x.z * m,
                                        dft.w * g4.w - x.w * m});
    const float4 o = add4(ld4(dx1 + ro + c), dx);
    st4(dx1 + ro + c, o);
    stbf4(dx1_bf + ro + c, o);
    st4(pg + c, add4(ld4(pg + c), mul4(dft, xh)));
  }
  ROW_LOOP_END
}

__global__ __launch_bounds__(256) void head_bwd_kernel(int N, int D, float eps, const float* __restrict__ dx1,
                                                       const float* __restrict__ da, const float* __restrict__ c_,
                                                       const float* __restrict__ ga, const float* __restrict__ gr,
                                                       const float* __restrict__ hp, const float* __restrict__ e,
                                                       const float* __restrict__ emb, int loop_dim,
                                                       float* __restrict__ gcarry, float* __restrict__ de,
                                                       float* __restrict__ part_ga, float* __restrict__ part_gr) {
  ROW_LOOP_BEGIN
  const int64_t ro = (int64_t)n * D;
  auto r_at = [&](int c) {
    float4 v = add4(ld4(hp + ro + c), ld4(e + ro + c));
    if (c < loop_dim) v = add4(v, ld4(emb + c));
    return v;
  };
  float sc = 0.f, sac = 0.f, sr = 0.f;
  for (int c = 4 * lane; c < D; c += 256) {
    const float4 cv = ld4(c_ + ro + c), rv = r_at(c);
    sc += dot4(cv, cv);
    sac += dot4(mul4(ld4(da + ro + c), ld4(ga + c)), cv);
    sr += dot4(rv, rv);
  }
  sc = wave_sum(sc);
  sac = wave_sum(sac);
  sr = wave_sum(sr);
  const float rc = rsqrtf(sc / D + eps), mc = sac * rc * rc / D;
  const float rr = rsqrtf(sr / D + eps);
  auto dc_at = [&](int c) {
    const float4 cv = ld4(c_ + ro + c), dav = mul4(ld4(da + ro + c), ld4(ga + c));
    const float4 t = float4{dav.x - cv.x * mc, dav.y - cv.y * mc, dav.z - cv.z * mc, dav.w - cv.w * mc};
    return fma4(rc, t, ld4(dx1 + ro + c));
  };
  float scr = 0.f;
  for (int c = 4 * lane; c < D; c += 256) scr += dot4(mul4(dc_at(c), ld4(gr + c)), r_at(c));
  scr = wave_sum(scr);
  const float mr = scr * rr * rr / D;
  float* pa = part_ga + (int64_t)wg * D;
  float* pr = part_gr + (int64_t)wg * D;
  for (int c = 4 * lane; c < D; c += 256) {
    const float4 dc = dc_at(c), rv = r_at(c), g4 = ld4(gr + c);
    const float4 t = float4{dc.x * g4.x - rv.x * mr, dc.y * g4.y - rv.y * mr, dc.z * g4.z - rv.z * mr,
                            dc.w * g4.w - rv.w * mr};
    const float4 dr = scl4(rr, t);
    st4(gcarry + ro + c, add4(ld4(gcarry + ro + c), dr));
    st4(de + ro + c, add4(ld4(de + ro + c), dr));
    st4(pa + c, add4(ld4(pa + c), mul4(ld4(da + ro + c), scl4(rc, ld4(c_ + ro + c)))));
    st4(pr + c, add4(ld4(pr + c), mul4(dc, scl4(rr, rv))));
  }
  ROW_LOOP_END
}

// The same with the row's slices of c and da held in registers (NC float4
// per lane, D <= 256 NC), so the later passes read neither again; h_prev +
// e is re-read per pass (holding it too would leave one wave per SIMD).
// Same arithmetic, same order.
template <int NC>
__global__ __launch_bounds__(256) void head_bwd_reg_kernel(int N, int D, float eps, const float* __restrict__ dx1,
                                                           const float* __restrict__ da, const float* __restrict__ c_,
                                                           const float* __restrict__ ga, const float* __restrict__ gr,
                                                           const float* __restrict__ hp, const float* __restrict__ e,
                                                           const float* __restrict__ emb, int loop_dim,
                                                           float* __restrict__ gcarry, float* __restrict__ de,
                                                           float* __restrict__ part_ga, float* __restrict__ part_gr) {
  ROW_LOOP_BEGIN
  const int64_t ro = (int64_t)n * D;
  auto r_at = [&](int c) {
    float4 v = add4(ld4(hp + ro + c), ld4(e + ro + c));
    if (c < loop_dim) v = add4(v, ld4(emb + c));
    return v;
  };
  const float4 z4 = float4{0.f, 0.f, 0.f, 0.f};
  float4 cv[NC], dav[NC];
  float sc = 0.f, sac = 0.f, sr = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = 4 * lane + 256 * i;
    cv[i] = dav[i] = z4;
    if (c < D) {
      cv[i] = ld4(c_ + ro + c);
      dav[i] = ld4(da + ro + c);
      const float4 rv = r_at(c);
      sc += dot4(cv[i], cv[i]);
      sac += dot4(mul4(dav[i], ld4(ga + c)), cv[i]);
      sr += dot4(rv, rv);
    }
  }
  sc = wave_sum(sc);
  sac = wave_sum(sac);
  sr = wave_sum(sr);
  const float rc = rsqrtf(sc / D + eps), mc = sac * rc * rc / D;
  const float rr = rsqrtf(sr / D + eps);
  auto dc_at = [&](int i, int c) {
    const float4 dg = mul4(dav[i], ld4(ga + c));
    const float4 t = float4{dg.x - cv[i].x * mc, dg.y - cv[i].y * mc, dg.z - cv[i].z * mc, dg.w - cv[i].w * mc};
    return fma4(rc, t, ld4(dx1 + ro + c));
  };
  float scr = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = 4 * lane + 256 * i;
    if (c < D) scr += dot4(mul4(dc_at(i, c), ld4(gr + c)), r_at(c));
  }
  scr = wave_sum(scr);
  const float mr = scr * rr * rr / D;
  float* pa = part_ga + (int64_t)wg * D;
  float* pr = part_gr + (int64_t)wg * D;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = 4 * lane + 256 * i;
    if (c < D) {
      const float4 dc = dc_at(i, c), rv = r_at(c), g4 = ld4(gr + c);
      const float4 t = float4{dc.x * g4.x - rv.x * mr, dc.y * g4.y - rv.y * mr, dc.z * g4.z - rv.z * mr,
                              dc.w * g4.w - rv.w * mr};
      const float4 dr = scl4(rr, t);
      st4(gcarry + ro + c, add4(ld4(gcarry + ro + c), dr));
      st4(de + ro + c, add4(ld4(de + ro + c), dr));
      st4(pa + c, add4(ld4(pa + c), mul4(dav[i], scl4(rc, cv[i]))));
      st4(pr + c, add4(ld4(pr + c), mul4(dc, scl4(rr, rv))));
    }
  }
  ROW_LOOP_END
}

__global__ __launch_bounds__(256) void loop_index_kernel(const int32_t* __restrict__ perm,
                                                         const int32_t* __restrict__ off, int t, int NK, int N, int E,
                                                         int32_t* __restrict__ gidx, int32_t* __restrict__ load) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (gidx && i < NK) gidx[(int64_t)t * NK + i] = t * N + perm[i];
  if (blockIdx.x == 0 && threadIdx.x < E) load[threadIdx.x] += off[threadIdx.x + 1] - off[threadIdx.x];
}

// CW columns per block (64, or fewer for narrow sums); the 256 / CW row
// slices of each column are summed by their threads, then added in a
// fixed order
__global__ __launch_bounds__(256) void col_reduce_kernel(const float* __restrict__ part, int rows, int64_t ld, int len,
                                                         float* __restrict__ out, int accumulate, int CW) {
  __shared__ float red[256];
  const int cl = threadIdx.x % CW, rs = threadIdx.x / CW, RS = 256 / CW, c = blockIdx.x * CW + cl;
  float s0 = 0.f, s1 = 0.f;
  if (c < len) {
    int w = rs;
    for (; w + RS < rows; w += 2 * RS) {
      s0 += part[(int64_t)w * ld + c];
      s1 += part[(int64_t)(w + RS) * ld + c];
    }
    if (w < rows) s0 += part[(int64_t)w * ld + c];
  }
  red[threadIdx.x] = s0 + s1;
  __syncthreads();
  if (rs == 0 && c < len) {
    float t = 0.f;
    for (int i = 0; i < RS; ++i) t += red[i * CW + cl];
    out[c] = accumulate ? out[c] + t : t;
  }
}

// block (column chunk, slice z, batch b): CW columns of rows [z rows / S,
// (z + 1) rows / S), the 256 / CW row lanes of each column added in order
__global__ __launch_bounds__(256) void col_slices_kernel(const float* __restrict__ part, int rows, int64_t ld, int len,
                                                         int64_t pstride, float* __restrict__ slices, int CW) {
  __shared__ float red[256];
  const int cl = threadIdx.x % CW, rs = threadIdx.x / CW, RS = 256 / CW, c = blockIdx.x * CW + cl;
  const int z = blockIdx.y, b = blockIdx.z;
  const int r0 = (int)((int64_t)z * rows / RDT_COL_SLICES), r1 = (int)((int64_t)(z + 1) * rows / RDT_COL_SLICES);
  const float* p = part + (int64_t)b * pstride;
  float s0 = 0.f, s1 = 0.f;
  if (c < len) {
    int w = r0 + rs;
    for (; w + RS < r1; w += 2 * RS) {
      s0 += p[(int64_t)w * ld + c];
      s1 += p[(int64_t)(w + RS) * ld + c];
    }
    if (w < r1) s0 += p[(int64_t)w * ld + c];
  }
  red[threadIdx.x] = s0 + s1;
  __syncthreads();
  if (rs == 0 && c < len) {
    float t = 0.f;
    for (int i = 0; i < RS; ++i) t += red[i * CW + cl];
    slices[((int64_t)b * RDT_COL_SLICES + z) * len + c] = t;
  }
}

__global__ __launch_bounds__(256) void lti_param_grad_kernel(const float* __restrict__ dA, const float* __restrict__ A,
                                                             const float* __restrict__ log_A,
                                                             const float* __restrict__ log_dt, int D,
                                                             float* __restrict__ dlog_A, float* __restrict__ dlog_dt) {
  __shared__ float red[4];
  float s = 0.f;
  for (int i = threadIdx.x; i < D; i += 256) {
    const float x = log_dt[0] + log_A[i];
    // A = exp(-exp(x)): dA/dx = -A exp(x); no gradient outside the clamp
    const float g = (x >= -20.f && x <= 20.f) ? dA[i] * A[i] * -expf(x) : 0.f;
    dlog_A[i] = g;
    s += g;
  }
  s = block_sum(s, red);
  if (threadIdx.x == 0) dlog_dt[0] = s;
}

__global__ __launch_bounds__(256) void router_bias_update_kernel(float* __restrict__ bias,
                                                                 const int32_t* __restrict__ load, int E,
                                                                 float gamma) {
  __shared__ int tot[256];
  const int e = threadIdx.x;
  tot[e] = e < E ? load[e] : 0;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (e < o) tot[e] += tot[e + o];
    __syncthreads();
  }
  if (e < E) {
    const long long d = (long long)tot[0] - (long long)E * load[e];
    bias[e] += gamma * (float)((d > 0) - (d < 0));
  }
}

}  // namespace

// ------------------------------------------------------------ launchers

void launch_transpose_bf16(const void* in, int64_t isb1, int64_t isb2, int nb2, int64_t ldi, void* out, int64_t osb,
                           int64_t ldo, int nbatch, int R, int Rp, int C, int Cv, hipStream_t s) {
  const dim3 grid((C + 63) / 64, (Rp + 63) / 64, nbatch);
  // 16-byte accesses need 8-element aligned bases and strides
  const int vec = ((uintptr_t)in % 16 == 0) && ((uintptr_t)out % 16 == 0) && isb1 % 8 == 0 && isb2 % 8 == 0 &&
                  ldi % 8 == 0 && osb % 8 == 0 && ldo % 8 == 0;
  transpose_bf16_kernel<<<grid, 256, 0, s>>>((const bf16_t*)in, isb1, isb2, nb2, ldi, (bf16_t*)out, osb, ldo, R, Rp,
                                             C, Cv, vec);
}

void launch_wgrad(const WgradArgs& a, hipStream_t s) {
  // 256-wide tiles unless the product is narrow (LoRA rank, small shapes)
  if (a.Nc >= 256 && a.Kc >= 256) {
    const dim3 grid(((a.Nc + 255) / 256) * ((a.Kc + 255) / 256) * a.G, 1, a.splits);
    wgrad8_kernel<<<grid, 512, 0, s>>>(a);
  } else {
    const dim3 grid(((a.Nc + 127) / 128) * ((a.Kc + 127) / 128) * a.G, 1, a.splits);
    wgrad_kernel<2><<<grid, 256, 0, s>>>(a);
  }
}

void launch_router_wgrad(const float* dz, const void* fperm, const int32_t* off, int n_loops, int NK, int E, int D,
                         float* part, float* dWr, hipStream_t s) {
  router_wgrad_kernel<<<dim3((D + 255) / 256, E, RW_SLICES), 256, 0, s>>>(dz, (const bf16_t*)fperm, off, n_loops, NK,
                                                                           E, D, part);
  launch_col_reduce(part, RW_SLICES, (int64_t)E * D, E * D, dWr, 0, s);
}

void launch_gather_rows_bf16(const void* src, const int32_t* perm, int M, int D, void* dst, hipStream_t s) {
  const int64_t n = (int64_t)M * D / 8;
  gather_rows_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>((const bf16_t*)src, perm, M, D, (bf16_t*)dst);
}

void launch_attn_bwd_prep(const void* o, const void* dO, int N, int H, int T, float* Dq, hipStream_t s) {
  attn_bwd_prep_kernel<<<(N * H + 255) / 256, 256, 0, s>>>((const bf16_t*)o, (const bf16_t*)dO, N, H, T, Dq);
}

void launch_attn_bwd(const void* q, const void* k, const void* v, const void* dO, const void* qt, const void* dOt,
                     const void* kt, const float* lse2, const float* Dq, float* dQ, float* dK, float* dV, int B,
                     int H, int G, int T, int Tp, int cap, float scale, hipStream_t s) {
  const float sl2 = scale * 1.4426950408889634f;
  const int nkt = (T + 127) / 128;
  attn_bwd_dkdv_kernel<<<nkt * B * G, 256, 0, s>>>((const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v,
                                                   (const bf16_t*)dO, (const bf16_t*)qt, (const bf16_t*)dOt, lse2, Dq,
                                                   dK, dV, B, H, G, T, Tp, cap, sl2, scale);
  attn_bwd_dq_kernel<<<nkt * B * H, 256, 0, s>>>((const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v,
                                                 (const bf16_t*)dO, (const bf16_t*)kt, lse2, Dq, dQ, B, H, G, T, cap,
                                                 sl2, scale);
}

void launch_qkv_bwd(const float* dQ, const float* dK, const float* dV, const float* rcos, const float* rsin, int B,
                    int T, int H, int G, void* dqkv, hipStream_t s) {
  const int64_t n = (int64_t)B * T * (H + 2 * G) * 64;
  qkv_bwd_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(dQ, dK, dV, rcos, rsin, B, T, H, G, (bf16_t*)dqkv);
}

void launch_swiglu_fwd(const void* gu, int M, int F, void* act, hipStream_t s) {
  const int64_t n = (int64_t)M * F / 4;
  swiglu_fwd_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>((const bf16_t*)gu, M, F, (bf16_t*)act);
}

void launch_swiglu_bwd(const void* gu, const float* dact, int M, int F, void* dgu, hipStream_t s) {
  const int64_t n = (int64_t)M * F / 4;
  swiglu_bwd_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>((const bf16_t*)gu, dact, M, F, (bf16_t*)dgu);
}

void launch_act_prep(const float* states, int64_t state_stride, const float* dy, const float* halt_w,
                     const float* halt_b, const int32_t* halt_counts, int L, int N, int D, float* w_act, float* z_act,
                     float* part_hw, float* part_hb, hipStream_t s) {
  act_prep_kernel<<<RDT_BWD_BLOCKS, 256, 0, s>>>(states, state_stride, dy, halt_w, halt_b, halt_counts, L, N, D,
                                                 w_act, z_act, part_hw, part_hb);
}

void launch_tail_bwd_rows(const TailBwdArgs& a, hipStream_t s) {
  tail_bwd_rows_kernel<<<RDT_BWD_BLOCKS, 256, 0, s>>>(a);
}

void launch_lora_bwd(int N, int r, const float* v, const float* dw, const float* scale, void* sv_wl, void* sv_dv,
                     void* dv_pad, float* part_s, hipStream_t s) {
  lora_bwd_kernel<<<RDT_BWD_BLOCKS, 256, 0, s>>>(N, r, v, dw, scale, (bf16_t*)sv_wl, (bf16_t*)sv_dv, (bf16_t*)dv_pad,
                                                 part_s);
}

void launch_tail_bwd_gates(const TailBwdArgs& a, hipStream_t s) {
  tail_bwd_gates_kernel<<<RDT_BWD_BLOCKS, 256, 0, s>>>(a);
}

void launch_ffn_norm_bwd(int N, int D, int k, float eps, const float* df, const float* dfp, const int32_t* inv,
                         const int32_t* sel, const float* dz, const void* Wr, const float* x1, const float* g_ffn,
                         float* dx1, void* dx1_bf, float* part_g, hipStream_t s) {
  const int nc = (D + 255) / 256;
  if (nc <= 4)
    ffn_norm_bwd_reg_kernel<4><<<RDT_BWD_BLOCKS, 256, 0, s>>>(N, D, k, eps, df, dfp, inv, sel, dz, (const bf16_t*)Wr,
                                                              x1, g_ffn, dx1, (bf16_t*)dx1_bf, part_g);
  else if (nc <= 8)
    ffn_norm_bwd_reg_kernel<8><<<RDT_BWD_BLOCKS, 256, 0, s>>>(N, D, k, eps, df, dfp, inv, sel, dz, (const bf16_t*)Wr,
                                                              x1, g_ffn, dx1, (bf16_t*)dx1_bf, part_g);
  else if (nc <= 12)
    ffn_norm_bwd_reg_kernel<12><<<RDT_BWD_BLOCKS, 256, 0, s>>>(N, D, k, eps, df, dfp, inv, sel, dz, (const bf16_t*)Wr,
                                                               x1, g_ffn, dx1, (bf16_t*)dx1_bf, part_g);
  else
    ffn_norm_bwd_kernel<<<RDT_BWD_BLOCKS, 256, 0, s>>>(N, D, k, eps, df, dfp, inv, sel, dz, (const bf16_t*)Wr, x1,
                                                       g_ffn, dx1, (bf16_t*)dx1_bf, part_g);
}

void launch_head_bwd(int N, int D, float eps, const float* dx1, const float* da, const float* c,
                     const float* g_attn, const float* g_rec, const float* h_prev, const float* e, const float* emb_t,
                     int loop_dim, float* g_carry, float* de, float* part_ga, float* part_gr, hipStream_t s) {
  const int nc = (D + 255) / 256;
  if (nc <= 4)
    head_bwd_reg_kernel<4><<<RDT_BWD_BLOCKS, 256, 0, s>>>(N, D, eps, dx1, da, c, g_attn, g_rec, h_prev, e, emb_t,
                                                          loop_dim, g_carry, de, part_ga, part_gr);
  else if (nc <= 8)
    head_bwd_reg_kernel<8><<<RDT_BWD_BLOCKS, 256, 0, s>>>(N, D, eps, dx1, da, c, g_attn, g_rec, h_prev, e, emb_t,
                                                          loop_dim, g_carry, de, part_ga, part_gr);
  else if (nc <= 12)
    head_bwd_reg_kernel<12><<<RDT_BWD_BLOCKS, 256, 0, s>>>(N, D, eps, dx1, da, c, g_attn, g_rec, h_prev, e, emb_t,
                                                           loop_dim, g_carry, de, part_ga, part_gr);
  else
    head_bwd_kernel<<<RDT_BWD_BLOCKS, 256, 0, s>>>(N, D, eps, dx1, da, c, g_attn, g_rec, h_prev, e, emb_t, loop_dim,
                                                   g_carry, de, part_ga, part_gr);
}

void launch_loop_index(const int32_t* perm, const int32_t* off, int t, int NK, int N, int E, int32_t* gidx,
                       int32_t* load, hipStream_t s) {
  loop_index_kernel<<<(NK + 255) / 256, 256, 0, s>>>(perm, off, t, NK, N, E, gidx, load);
}

void launch_col_reduce(const float* part, int rows, int64_t ld, int len, float* out, int accumulate, hipStream_t s) {
  const int CW = len >= 64 ? 64 : len >= 16 ? 16 : 4;
  col_reduce_kernel<<<(len + CW - 1) / CW, 256, 0, s>>>(part, rows, ld, len, out, accumulate, CW);
}

void launch_col_slices(const float* part, int rows, int64_t ld, int len, int nb, int64_t pstride, float* slices,
                       hipStream_t s) {
  const int CW = len >= 64 ? 64 : len >= 16 ? 16 : 4;
  col_slices_kernel<<<dim3((len + CW - 1) / CW, RDT_COL_SLICES, nb), 256, 0, s>>>(part, rows, ld, len, pstride, slices,
                                                                                    CW);
}

void launch_lti_param_grad(const float* dA, const float* A, const float* log_A, const float* log_dt, int D,
                           float* dlog_A, float* dlog_dt, hipStream_t s) {
  lti_param_grad_kernel<<<1, 256, 0, s>>>(dA, A, log_A, log_dt, D, dlog_A, dlog_dt);
}

void launch_router_bias_update(float* bias, const int32_t* load, int E, float gamma, hipStream_t s) {
  router_bias_update_kernel<<<1, 256, 0, s>>>(bias, load, E, gamma);
}

namespace {
// n4 16-byte words from p (16-byte aligned), then n1 4-byte words
__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* __restrict__ p, size_t n4, size_t n1) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) p[i] = uint4{0u, 0u, 0u, 0u};
  uint32_t* t = (uint32_t*)(p + n4);
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n1; i += stride) t[i] = 0u;
}
}  // namespace

void launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  // a 4-byte aligned start that is not 16-byte aligned goes word by word
  const size_t n = bytes / 4;
  if (n == 0) return;
  const bool a16 = ((uintptr_t)p & 15) == 0;
  const size_t n4 = a16 ? n / 4 : 0, n1 = n - 4 * n4;
  const size_t work = std::max(n4, n1);
  const size_t blocks = std::min<size_t>((work + 255) / 256, 2048);
  fill_zero_kernel<<<(unsigned)blocks, 256, 0, s>>>((uint4*)p, n4, n1);
}
