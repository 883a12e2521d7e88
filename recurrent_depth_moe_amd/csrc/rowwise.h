// Row-wise (HBM-bound) kernels of the recurrent block and the router/dispatch.
#pragma once

#include "common.h"

#define RDT_DISP_TILE 256
#define RDT_MAX_EXPERTS 512
#define RDT_MAX_LORA 32

// tables: RoPE cos/sin [max_seq][rot/2] for each rotary width, loop-index
// embedding [n_loops_max][loop_dim], A [D]
void launch_make_tables(float* rope_cos, float* rope_sin, int max_seq, int rot_dim, double theta, hipStream_t s);
void launch_make_loop_table(float* emb, int n_loops_max, int loop_dim, double theta, hipStream_t s);
void launch_make_A(const float* log_A, const float* log_dt, float* A, int D, hipStream_t s);

// c = RMSNorm(h + emb_t + e) * g_rec (fp32); a = RMSNorm(c) * g_attn (bf16 or fp32)
// Row n of c and a reads position tok[n] of h and e (tok null: position n).
void launch_loop_head(int act_bf16, const float* h, const float* e, const float* emb_t, int loop_dim,
                      const float* g_rec, const float* g_attn, float eps, float* c, void* a, int N, int D,
                      hipStream_t s, const int32_t* live_prev = nullptr, int32_t* live_cur = nullptr,
                      const int32_t* tok = nullptr);
// Token embedding ([ZS §Core Structure], the model's first step): row
// n = b T + i of x (fp32 [B T, D]) is row ids[b ids_ld + i] of the table
// ([V, D], bf16 or fp32); an id outside [0, V) gives a row of NaN.
void launch_embed(int table_bf16, const int32_t* ids, int64_t ids_ld, int B, int T, const void* table, int V, int D,
                  float* x, hipStream_t s);
// Greedy choice: out[r * out_ld] = the column of the largest logit of row r
// (fp32 [rows, V]), the lowest column among equal maxima; NaN never wins
// (a row of NaN gives 0).
void launch_argmax_rows(const float* logits, int rows, int V, int32_t* out, int64_t out_ld, hipStream_t s);
// ACT compute skipping: tok[0 .. count) = the positions whose halt count is
// still 0 (running), in ascending order; *count written on the device.
void launch_compact_running(const int32_t* halt_counts, int N, int32_t* tok, int32_t* count, hipStream_t s);
// out[r] = RMSNorm(x[r]) * g for rows r < rows; x fp32 with row stride ldx,
// out (bf16 or fp32) with stride ldo
void launch_rmsnorm(int out_bf16, const float* x, int64_t ldx, const float* g, float eps, void* out, int64_t ldo,
                    int rows, int D, hipStream_t s, const int32_t* live = nullptr);

// softmax over E logits, top-k of logits + bias (descending, ties to the
// lower index), gates renormalised over the chosen experts
// (cap_sel, when set, receives row n's choice at position tok[n]; tok null:
// position n)
void launch_router_topk(const float* logits, const float* bias, int N, int E, int k, int32_t* sel, float* gate,
                        int32_t* cap_sel, hipStream_t s, const int32_t* live = nullptr,
                        const int32_t* tok = nullptr);
// dropless dispatch: stable order (token, slot) inside each expert
// (also zeroes the n_claim tile-claim counters the grouped products of the
// same loop draw from, n_claim <= RDT_MAX_EXPERTS).  With merge_extra > 0 a
// second m-tile schedule (mt_start_m, tile_row0_m, tile_grp_m) is built in
// which an expert's last m-tile also takes a remainder of at most
// merge_extra rows instead of leaving it to a tile of its own.
void launch_dispatch(const int32_t* sel, int NK, int k, int E, int bm, int32_t* tile_counts, int32_t* offsets,
                     int32_t* mt_start, int32_t* tile_row0, int32_t* tile_grp, int32_t* perm_src, int32_t* inv,
                     int32_t* tile_claim, int n_claim, hipStream_t s, const int32_t* live = nullptr,
                     int merge_extra = 0, int32_t* mt_start_m = nullptr, int32_t* tile_row0_m = nullptr,
                     int32_t* tile_grp_m = nullptr);

struct TailArgs {
  const float* x1;        // [N][D]
  const void* y;          // routed expert outputs in dispatch order [NK][D], weight dtype
  const int32_t* inv;     // [N*k] slot -> dispatch row
  const float* gate;      // [N*k]
  const void* y_s;        // shared expert outputs [S][N][D], weight dtype
  int S;
  const void* lora_down;  // [r][D] weight dtype
  const void* lora_B;     // [r][D]
  const float* lora_scale_row;  // [r] row min(t, L-1)
  int r;
  const float* A;         // [D]
  const float* Bv;        // [D]
  const float* e;         // [N][D]
  const float* h_prev;    // [N][D]
  float* h_next;          // [N][D]
  const float* halt_w;    // [D]
  const float* halt_b;    // [1]
  float act_threshold;    // 0 = off
  float* h_out;           // [N][D]
  float* cum;             // [N]
  int32_t* halt_counts;   // [N]
  int t, n_loops, N, D, k;
  float* cap_h;           // [N][D] slice of loop t, or null
  float* cap_p;           // [N] slice of loop t, or null
  int w_bf16;
  const int32_t* live_prev;  // running positions after loop t-1, or null (never skip)
  int32_t* live_cur;         // running positions after this loop are added here, or null
  // ACT compute skipping: the N rows are the running positions only, row n
  // is position tok[n] (null: row n is position n).  x1, y, inv, gate and
  // y_s are per row; e, h_prev, h_next, h_out, cum, halt_counts, cap_h and
  // cap_p are per position.
  const int32_t* tok;
};
void launch_loop_tail(const TailArgs& a, hipStream_t s);

// MLA glue (see attention.hip for buffer layouts)
void launch_mla_latent(int act_bf16, const float* kv_raw, const float* cq_raw, const float* gq, float eps, int N,
                       int T, int ql, int kvl, int rope, int start_pos, const float* rcos, const float* rsin,
                       void* cq_norm, void* lat_ckv, void* lat_krope, int lat_cap, int kbase, hipStream_t s,
                       const int32_t* live = nullptr);
// MLA decode step (one query per sequence, fp32) with absorbed
// up-projections: latent keys k_lat [B][kvlen][kvl + rope] and values
// vt_lat [B][kvl][kvlen] from the cached latent, queries q_lat
// [B][H][kvl + rope] from q [B][H][nope + rope]; after attention over the
// latent (one key head), o [B][H * vd] = W_v,h o_lat [B][H][kvl].
void launch_mla_absorbed_decode_prep(const float* lat_ckv, const float* lat_krope, int lat_cap, const float* gkv,
                                     float eps, int B, int kvlen, int kvl, int rope, const float* q,
                                     const float* wukv, int H, int nope, int vd, float* k_lat, float* vt_lat,
                                     float* q_lat, hipStream_t s, const int32_t* live = nullptr);
void launch_mla_absorb_o(const float* o_lat, const float* wukv, int B, int H, int nope, int vd, int kvl, float* o,
                         hipStream_t s, const int32_t* live = nullptr);
void launch_mla_kv_prep(int act_bf16, const void* lat_ckv, const void* lat_krope, int lat_cap, const float* gkv,
                        float eps, int B, int kvlen, int kvl, int rope, int H, int dq, void* ckv_norm, void* K,
                        hipStream_t s, const int32_t* live = nullptr);
