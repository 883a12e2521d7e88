// Kernels of the backward pass of the recurrent block (bf16 GQA, head
// width 128): weight-gradient products, flash-attention backward and the
// row-wise backward passes of the norms, SwiGLU, the tail and ACT.
#pragma once

#include "common.h"

// Per-wave partial rows of column sums: the row-wise backward kernels run
// RDT_BWD_BLOCKS blocks of four waves; wave w of block b owns partial row
// 4 b + w and adds its rows' contributions there, so every sum is formed in
// a fixed order.
#define RDT_BWD_BLOCKS 1024
#define RDT_BWD_WAVES (RDT_BWD_BLOCKS * 4)
// row stride of the saved LoRA vectors (lora_rank <= 32)
#define RDT_LORA_LD 32
// loops a weight-gradient product may stack (the training loop limit)
#define RDT_MAX_WGRAD_LOOPS 64

// out[bi][c][r] = in(bi)[r][c] for r < R and c < Cv, 0 for R <= r < Rp or
// Cv <= c < C, where bi = b1 * nb2 + b2 and in(bi) = in + b1 * isb1 + b2 * isb2
// (row stride ldi); out(bi) = out + bi * osb, row stride ldo.  bf16.
void launch_transpose_bf16(const void* in, int64_t isb1, int64_t isb2, int nb2, int64_t ldi, void* out, int64_t osb,
                           int64_t ldo, int nbatch, int R, int Rp, int C, int Cv, hipStream_t s);

// Weight gradient C_g[n][k] (+)= sum over loops t and rows m of group g
// of A_t[m][n] X_t[m][k] (bf16 operands, fp32 result), A_t = A + t a_loop_stride
// (elements), row m at A_t + m lda, likewise X; group g of loop t holds
// rows off[t][g] .. off[t][g+1] (off null: one group of `rows` rows).
// Loops split over `splits` slices along grid z, slice z writing
// C + z * c_split_stride.
struct WgradArgs {
  const void* A;
  int64_t lda;
  int64_t a_loop_stride;
  const void* X;
  int64_t ldx;
  int64_t x_loop_stride;
  const int32_t* off;    // nullable: [n_loops][G + 1]
  int n_loops;
  int rows;
  int G;
  int Nc, Kc;
  float* C;
  int64_t ldc;
  int64_t c_gstride;
  int splits;
  int64_t c_split_stride;
  int accumulate;
};
void launch_wgrad(const WgradArgs& a, hipStream_t s);

// dWr[e][c] = sum over loops t and dispatch rows m of expert e of
// dz[t][m] * fperm[t][m][c]   (f in dispatch order, bf16, stacked over loops);
// part: fp32 scratch of 16 E D floats (row-slice partial sums)
#define RDT_ROUTER_WGRAD_PART(E, D) ((size_t)16 * (E) * (D))
void launch_router_wgrad(const float* dz, const void* fperm, const int32_t* off, int n_loops, int NK, int E, int D,
                         float* part, float* dWr, hipStream_t s);
// dst[m] = src[perm[m]] for m < M (bf16 rows of D, D a multiple of 8)
void launch_gather_rows_bf16(const void* src, const int32_t* perm, int M, int D, void* dst, hipStream_t s);

// Flash-attention backward (bf16, head width 128, causal, GQA).
// Dq[b][h][i] = sum_d dO[b i][h d] o[b i][h d]
void launch_attn_bwd_prep(const void* o, const void* dO, int N, int H, int T, float* Dq, hipStream_t s);
// q [B][H][T][128]; k, v [B][G][cap][128] (v not transposed); dO [B T][H 128];
// qt, dOt [B H][128][Tp] and kt [B G][128][cap] transposed, zero past T;
// lse2, Dq [B][H][T]; outputs dK, dV [B][G][T][128], dQ [B][H][T][128] fp32
void launch_attn_bwd(const void* q, const void* k, const void* v, const void* dO, const void* qt, const void* dOt,
                     const void* kt, const float* lse2, const float* Dq, float* dQ, float* dK, float* dV, int B,
                     int H, int G, int T, int Tp, int cap, float scale, hipStream_t s);
// dqkv [B T][(H + 2G) 128] bf16 from dQ, dK, dV with the RoPE rotation
// taken back (positions 0 .. T-1)
void launch_qkv_bwd(const float* dQ, const float* dK, const float* dV, const float* rcos, const float* rsin, int B,
                    int T, int H, int G, void* dqkv, hipStream_t s);

// act[m][f] = silu(GU[m][f]) * GU[m][F + f]          (bf16 in, bf16 out)
void launch_swiglu_fwd(const void* gu, int M, int F, void* act, hipStream_t s);
// dGU[m][f] = dact * U * silu'(G), dGU[m][F + f] = dact * silu(G)
void launch_swiglu_bwd(const void* gu, const float* dact, int M, int F, void* dgu, hipStream_t s);

// ACT: per position n and loop t < L, w[t][n] = weight of h_{t+1} in the
// output and z[t][n] = d loss / d halting logit, from the recorded states
// (h_{t+1} = states + t state_stride, [N][D] fp32), dy and the halting
// loops; partial sums of z * h_{t+1} (d halt_w) and of z (d halt_b) per wave.
void launch_act_prep(const float* states, int64_t state_stride, const float* dy, const float* halt_w,
                     const float* halt_b, const int32_t* halt_counts, int L, int N, int D, float* w_act, float* z_act,
                     float* part_hw, float* part_hb, hipStream_t s);

struct TailBwdArgs {
  int N, D, k, S, r;
  const float* g;          // dL/dh_{t+1} without this loop's ACT terms [N][D]
  const float* dy;         // [N][D]
  const float* w_act;      // [N] or null (ACT off)
  const float* z_act;      // [N] or null
  const float* halt_w;     // [D]
  const float* x1;         // [N][D]
  const void* y;           // routed outputs, dispatch order [NK][D] bf16
  const int32_t* inv;      // [N k]
  const float* gate;       // [N k]
  const void* ys;          // [S][N][D] bf16
  const void* lora_down;   // [r][D] bf16
  const void* lora_B;      // [r][D] bf16
  const float* scale_row;  // [r]
  const float* A;          // [D]
  const float* Bv;         // [D]
  const float* h_prev;     // [N][D]
  const float* e;          // [N][D]
  float* g_next;           // A * g_full (may alias g)
  float* de;               // += B * g_full
  float* dtau;             // fp32 [N][D]: g_full after the rows pass, dtau after the LoRA product
  void* dtau_bf;           // bf16 [N][D]
  void* dY;                // bf16 [NK][D], row inv[n k + j] = gate_j dtau
  float* dz;               // [N][k] d loss / d router logit of each chosen expert
  float* dz_perm;          // [NK] the same in dispatch order
  void* sv_g;              // bf16 [N][D] g_full
  void* sv_tau;            // bf16 [N][D] tau
  void* sv_wl;             // bf16 [N][RDT_LORA_LD] (tau Ld^T) * scale
  void* sv_dv;             // bf16 [N][RDT_LORA_LD] d(tau Ld^T)
  float* part_A;           // [waves][D] += g_full * h_prev
  float* part_B;           // [waves][D] += g_full * e
};
// Three passes: rows (g_full, tau, carry, de, dA / dB partials; dtau =
// g_full), then after v = tau Ld^T and dw = g_full LB^T (products)
// launch_lora_bwd, then after dtau += dv Ld (product) the gates pass (dY,
// dz, bf16 dtau).  sv_wl, sv_dv and part_s are written by launch_lora_bwd.
void launch_tail_bwd_rows(const TailBwdArgs& a, hipStream_t s);
// dv = dw * scale, saved (tau Ld^T) * scale and dv ([N][RDT_LORA_LD] bf16),
// dv_pad [N][64] bf16 (zero past r), part_s [waves][RDT_LORA_LD] += dw * v
void launch_lora_bwd(int N, int r, const float* v, const float* dw, const float* scale, void* sv_wl, void* sv_dv,
                     void* dv_pad, float* part_s, hipStream_t s);
void launch_tail_bwd_gates(const TailBwdArgs& a, hipStream_t s);

// dx1 += RMSNorm backward of f = RMSNorm(x1) g_ffn at df_total = df (null:
// 0) + sum_j dfp[inv j] + sum_j dz_j Wr[sel_j]; dx1_bf = bf16(dx1);
// part_g += df_total * x1 / rms
void launch_ffn_norm_bwd(int N, int D, int k, float eps, const float* df, const float* dfp, const int32_t* inv,
                         const int32_t* sel, const float* dz, const void* Wr, const float* x1, const float* g_ffn,
                         float* dx1, void* dx1_bf, float* part_g, hipStream_t s);

// Backward of a = RMSNorm(c) g_attn and c = RMSNorm(h + emb + e) g_rec:
// dc = dx1 + (norm backward at da); dr = (norm backward at dc);
// g_carry += dr, de += dr; partial sums of the two gains' gradients.
void launch_head_bwd(int N, int D, float eps, const float* dx1, const float* da, const float* c,
                     const float* g_attn, const float* g_rec, const float* h_prev, const float* e, const float* emb_t,
                     int loop_dim, float* g_carry, float* de, float* part_ga, float* part_gr, hipStream_t s);

// gidx[t NK + m] = t N + perm[m] (gidx nullable); load[e] += off[e+1] - off[e]
void launch_loop_index(const int32_t* perm, const int32_t* off, int t, int NK, int N, int E, int32_t* gidx,
                       int32_t* load, hipStream_t s);
// out[c] (+)= sum_w part[w][c] for c < len, w < rows
void launch_col_reduce(const float* part, int rows, int64_t ld, int len, float* out, int accumulate, hipStream_t s);
// first stage of a long column sum, for nb batches (batch b at part + b
// pstride): slices[b][z][c] = sum of part rows [z rows / RDT_COL_SLICES,
// (z + 1) rows / RDT_COL_SLICES) of column c (len <= ld); the slices are
// then summed in order by launch_col_reduce
#define RDT_COL_SLICES 32
void launch_col_slices(const float* part, int rows, int64_t ld, int len, int nb, int64_t pstride, float* slices,
                       hipStream_t s);
// d log_A and d log_dt from dA (A = exp(-exp(clamp(log_dt + log_A, -20, 20))))
void launch_lti_param_grad(const float* dA, const float* A, const float* log_A, const float* log_dt, int D,
                           float* dlog_A, float* dlog_dt, hipStream_t s);
// bias[e] += gamma * sign(sum(load) - E load[e])
void launch_router_bias_update(float* bias, const int32_t* load, int E, float gamma, hipStream_t s);
// p[0 .. bytes) = 0 (bytes a multiple of 4)
void launch_fill_zero(void* p, size_t bytes, hipStream_t s);
