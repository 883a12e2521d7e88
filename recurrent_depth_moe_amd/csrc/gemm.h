// Grouped GEMM C[m, n] = sum_k A[row(m), k] * W[group(m)][n, k] with fused
// epilogues, for every matrix product of the recurrent block.
#pragma once

#include "common.h"

enum EpiKind {
  EPI_STORE = 0,   // out[m, n] = acc                         (type TO)
  EPI_RESID = 1,   // out[m, n] = resid[m, n] + acc           (fp32)
  EPI_QKV = 2,     // RoPE on q and k, scatter to q / K / V^T (type TO)
  EPI_SWIGLU = 3,  // dual B: out[m, n] = silu(acc0) * acc1   (type TO)
  EPI_MLA_Q = 4,   // MLA query: RoPE on the rope part of each head
  EPI_MLA_KV = 5,  // MLA kv up-projection: k_nope -> K, v -> V^T
  EPI_SWIGLU_SAVE = 6,  // EPI_SWIGLU that also stores acc0 and acc1 (type TO):
                        // gu[m, n] = acc0, gu[m, gu_up + n] = acc1
};

struct EpiParams {
  void* out;
  int64_t ldo;
  const float* resid;
  void* q;
  void* k;
  void* vt;
  int T;      // rows per sequence (query rows, or key rows for EPI_MLA_KV)
  int H, G;   // query heads, kv heads
  int dq;     // q/k head width (GQA: head_dim; MLA: nope + rope)
  int dv;     // v head width
  int nope;   // MLA: width of the no-RoPE part
  int cap;    // K / V^T buffer capacity (positions per (b, head))
  int kbase;  // buffer index of this call's first position
  int start_pos;
  const float* rcos;  // RoPE tables [position][rot_half]
  const float* rsin;
  int rot_half;
  // EPI_QKV with ACT compute skipping: output row m is sequence position
  // tok[m] (b = tok[m] / T, i = tok[m] % T); null: row m is position m
  const int32_t* tok;
  // EPI_SWIGLU_SAVE: the gate / up pre-activations, row stride ldgu, the
  // up half gu_up elements after the gate half
  void* gu;
  int64_t ldgu, gu_up;
};

struct GemmParams {
  const void* A;
  int64_t lda;
  const int32_t* a_rows;   // logical row -> row of A (null: identity)
  const void* W0;
  const void* W1;          // second B matrix for EPI_SWIGLU
  int64_t w_stride;        // elements between consecutive groups of W
  int M, N, K;
  // grouped schedule (routed experts), all device arrays; null = one group
  const int32_t* mt_start;   // [E+1] first m-tile of each group
  const int32_t* tile_row0;  // [m-tiles] first logical row of the m-tile
  const int32_t* tile_grp;   // [m-tiles] group of the m-tile
  const int32_t* grp_end;    // [E+1] offsets: rows of group e are [grp_end[e], grp_end[e+1])
  int n_groups;
  int dense_gm;              // dense raster: m-tiles per group of the tile order
  const int32_t* live;       // running positions after the previous loop (null: always run)
  // big kernel, grouped products: RDT_NUM_XCD tile-claim counters, zero at
  // launch (null: static round-robin over each XCD's share of the tiles)
  int32_t* tile_ctr;
  EpiParams epi;
};

// Launch helpers (stream-ordered, no sync).
// 256x256 tiles, direct-to-LDS loads; K must be a multiple of 64 and a
// grouped schedule must be built with m-tile height RDT_BM_BIG
// bn = 256, or 192 for single-B products (EPI_STORE, EPI_RESID) whose
// 256-wide tiles would leave part of the last round of CUs idle
void launch_gemm_bf16_big(const GemmParams& p, int epi, bool dual, int out_is_bf16, int n_cu, hipStream_t s,
                          int bn = 256);
// at most 32 rows per m-tile (grouped schedules built with RDT_BM_SKINNY),
// nc = 32 or 64 output columns per block; mt_cap bounds the m-tile count;
// nw = 8 splits K over eight waves instead of four (fp32 EPI_STORE
// products with K a multiple of 128; others ignore it)
void launch_gemm_bf16_skinny(const GemmParams& p, int epi, bool dual, int out_is_bf16, int mt_cap, int nc,
                             hipStream_t s, int nw = 4);
void launch_gemm_f32(const GemmParams& p, int epi, bool dual, int n_cu, hipStream_t s);

// m-tile heights the kernels are built with (the dispatch builds schedules
// for exactly these)
#define RDT_BM_BIG 256
#define RDT_BM_SKINNY 32
#define RDT_BM_F32 64
