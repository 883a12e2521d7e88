// Device helpers shared by the GEMM kernels: fused epilogues and the
// XCD-aware tile order.
#pragma once

#include "gemm.h"

template <int EPI, typename TO>
static __device__ __forceinline__ void epi_store(const EpiParams& e, int m, int n, float v, float v2) {
  if constexpr (EPI == EPI_STORE) {
    St<TO>::st((TO*)e.out + (int64_t)m * e.ldo + n, v);
  } else if constexpr (EPI == EPI_RESID) {
    const int64_t i = (int64_t)m * e.ldo + n;
    ((float*)e.out)[i] = e.resid[i] + v;
  } else if constexpr (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE) {
    St<TO>::st((TO*)e.out + (int64_t)m * e.ldo + n, silu_f(v) * v2);
    if constexpr (EPI == EPI_SWIGLU_SAVE) {
      TO* gu = (TO*)e.gu + (int64_t)m * e.ldgu + n;
      St<TO>::st(gu, v);
      St<TO>::st(gu + e.gu_up, v2);
    }
  } else if constexpr (EPI == EPI_QKV) {
    const int mp = e.tok ? e.tok[m] : m;
    const int b = mp / e.T, i = mp - b * e.T;
    const int hq = e.H * e.dq, hk = e.G * e.dq;
    if (n < hq + hk) {
      // adjacent channels (2j, 2j+1) are one complex number; v2 holds the
      // other member of the pair
      const int d = n % e.dq;
      const int64_t ti = (int64_t)(e.start_pos + i) * e.rot_half + (d >> 1);
      const float c = e.rcos[ti], s = e.rsin[ti];
      const float r = (d & 1) ? (v2 * s + v * c) : (v * c - v2 * s);
      if (n < hq) {
        const int h = n / e.dq;
        St<TO>::st((TO*)e.q + (((int64_t)(b * e.H + h) * e.T + i) * e.dq + d), r);
      } else {
        const int g = (n - hq) / e.dq;
        St<TO>::st((TO*)e.k + (((int64_t)(b * e.G + g) * e.cap + e.kbase + i) * e.dq + d), r);
      }
    } else {
      const int nn = n - hq - hk, g = nn / e.dv, d = nn - g * e.dv;
      St<TO>::st((TO*)e.vt + (((int64_t)(b * e.G + g) * e.dv + d) * e.cap + e.kbase + i), v);
    }
  } else if constexpr (EPI == EPI_MLA_Q) {
    const int b = m / e.T, i = m - b * e.T;
    const int h = n / e.dq, d = n - h * e.dq;
    float r = v;
    if (d >= e.nope) {
      const int64_t ti = (int64_t)(e.start_pos + i) * e.rot_half + ((d - e.nope) >> 1);
      const float c = e.rcos[ti], s = e.rsin[ti];
      r = ((d - e.nope) & 1) ? (v2 * s + v * c) : (v * c - v2 * s);
    }
    St<TO>::st((TO*)e.q + (((int64_t)(b * e.H + h) * e.T + i) * e.dq + d), r);
  } else if constexpr (EPI == EPI_MLA_KV) {
    const int b = m / e.T, j = m - b * e.T;
    const int w = e.nope + e.dv, h = n / w, d = n - h * w;
    if (d < e.nope)
      St<TO>::st((TO*)e.k + (((int64_t)(b * e.H + h) * e.cap + j) * e.dq + d), v);
    else
      St<TO>::st((TO*)e.vt + (((int64_t)(b * e.H + h) * e.dv + (d - e.nope)) * e.cap + j), v);
  }
}

// Tile index -> (m-tile, n-tile).  Grouped: groups in order, inside a group
// the n-tile is the slow index, so the m-tiles that share a weight panel are
// consecutive.  Dense: raster groups of `dense_gm` m-tiles.
static __device__ __forceinline__ void tile_coords(const GemmParams& p, int L, int ntn, int n_mt, int& mt, int& nt) {
  if (p.mt_start) {
    int lo = 0, hi = p.n_groups - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.mt_start[mid] * ntn <= L) lo = mid; else hi = mid - 1;
    }
    const int s0 = p.mt_start[lo], ne = p.mt_start[lo + 1] - s0;
    const int local = L - s0 * ntn;
    nt = local / ne;
    mt = s0 + (local - nt * ne);
  } else {
    const int GM = p.dense_gm;
    const int mt0 = (L / (GM * ntn)) * GM;
    const int gm = min(GM, n_mt - mt0);
    const int local = L - mt0 * ntn;
    nt = local / gm;
    mt = mt0 + (local - nt * gm);
  }
}

static __device__ __forceinline__ void tile_rows(const GemmParams& p, int mt, int bm, int& row0, int& rows, int& grp) {
  if (p.mt_start) {
    grp = p.tile_grp[mt];
    row0 = p.tile_row0[mt];
    // an m-tile ends where the next one of its group starts, the group's
    // last at the group's end (a merged schedule's last m-tile may hold more
    // than bm rows: its strip rows)
    rows = (mt + 1 < p.mt_start[grp + 1] ? p.tile_row0[mt + 1] : p.grp_end[grp + 1]) - row0;
  } else {
    grp = 0;
    row0 = mt * bm;
    rows = min(bm, p.M - row0);
  }
}


// Eight consecutive outputs (m, n..n+7), n a multiple of 8, from the
// LDS-staged epilogue.  v2 carries the up-projection values for
// EPI_SWIGLU; RoPE pairs are inside the eight.
template <int EPI, typename TO>
static __device__ __forceinline__ void store8(TO* p, const float* v) {
  if constexpr (sizeof(TO) == 2) {
    const uint4 u = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                     pack_bf16x2(v[6], v[7])};
    *(uint4*)p = u;
  } else {
    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

template <int EPI, typename TO>
static __device__ __forceinline__ void epi_store8(const EpiParams& e, int N, int m, int n, const float* v,
                                                  const float* v2) {
  if (n + 8 > N) {
#pragma unroll
    for (int x = 0; x < 8; ++x)
      if (n + x < N)
        epi_store<EPI, TO>(e, m, n + x, v[x], (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE) ? v2[x] : v[x ^ 1]);
    return;
  }
  if constexpr (EPI == EPI_STORE) {
    store8<EPI, TO>((TO*)e.out + (int64_t)m * e.ldo + n, v);
  } else if constexpr (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE) {
    float o[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) o[x] = silu_f(v[x]) * v2[x];
    store8<EPI, TO>((TO*)e.out + (int64_t)m * e.ldo + n, o);
    if constexpr (EPI == EPI_SWIGLU_SAVE) {
      TO* gu = (TO*)e.gu + (int64_t)m * e.ldgu + n;
      store8<EPI, TO>(gu, v);
      store8<EPI, TO>(gu + e.gu_up, v2);
    }
  } else if constexpr (EPI == EPI_RESID) {
    const int64_t i = (int64_t)m * e.ldo + n;
    const float4 r0 = *(const float4*)(e.resid + i), r1 = *(const float4*)(e.resid + i + 4);
    const float o[8] = {r0.x + v[0], r0.y + v[1], r0.z + v[2], r0.w + v[3],
                        r1.x + v[4], r1.y + v[5], r1.z + v[6], r1.w + v[7]};
    store8<EPI, float>((float*)e.out + i, o);
  } else if constexpr (EPI == EPI_QKV) {
    const int mp = e.tok ? e.tok[m] : m;
    const int b = mp / e.T, i = mp - b * e.T;
    const int hq = e.H * e.dq, hk = e.G * e.dq;
    if (n < hq + hk) {
      const int d = n % e.dq;
      const float* cs = e.rcos + (int64_t)(e.start_pos + i) * e.rot_half + (d >> 1);
      const float* sn = e.rsin + (int64_t)(e.start_pos + i) * e.rot_half + (d >> 1);
      float o[8];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float c = cs[x], s = sn[x];
        o[2 * x] = v[2 * x] * c - v[2 * x + 1] * s;
        o[2 * x + 1] = v[2 * x] * s + v[2 * x + 1] * c;
      }
      if (n < hq) {
        const int h = n / e.dq;
        store8<EPI, TO>((TO*)e.q + (((int64_t)(b * e.H + h) * e.T + i) * e.dq + d), o);
      } else {
        const int g = (n - hq) / e.dq;
        store8<EPI, TO>((TO*)e.k + (((int64_t)(b * e.G + g) * e.cap + e.kbase + i) * e.dq + d), o);
      }
    } else {
      const int nn = n - hq - hk, g = nn / e.dv, d = nn - g * e.dv;
      TO* col = (TO*)e.vt + (((int64_t)(b * e.G + g) * e.dv + d) * e.cap + e.kbase + i);
#pragma unroll
      for (int x = 0; x < 8; ++x) St<TO>::st(col + (int64_t)x * e.cap, v[x]);
    }
  }
}
