/*
 * rdt.h — C ABI of the looped Recurrent-Block forward (Recurrent-Depth
 * Transformer) on one MI355X (gfx950).
 *
 * Pages cited (title, then section):
 *   [ZS] "OpenMythos 분석: Mythos Preview의 장기 추론 성능과 OpenMythos의 계산 모델링"
 *        (zero.shotlearni.ng)
 *   [RC] "OpenMythos" (runchr.com, Korean copy of the project README)
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers, caller-owned, row-major,
 *     contiguous, 16-byte aligned.  Sizes are element counts.
 *   - Calls enqueue work on `stream` (a hipStream_t passed as void*) and
 *     return without waiting; outputs are valid after the stream syncs.
 *   - Every argument and shape check runs on the host before any HIP call;
 *     a failed check returns a status and enqueues nothing.  No exception
 *     crosses the ABI.  rdt_last_error() gives a thread-local message.
 *   - A handle must not be used from two threads at once.  Results are
 *     bitwise reproducible run to run (no floating-point atomics).
 *   - Only rdt_block_create allocates device memory (the handle's own copy
 *     of the weights and tables) or creates HIP objects (for bf16 configs
 *     with shared experts, a side stream of default priority and two
 *     events).  Forward and decode allocate nothing: the caller passes the
 *     workspace.
 *   - Single-token bf16 calls run the shared-expert products on the
 *     handle's side stream, forked from `stream` after the FFN norm and
 *     joined back before the loop tail with events, so the call stays
 *     ordered on `stream`; calls of one handle on different streams then
 *     share (and serialise on) that side stream.
 */
#ifndef RDT_H
#define RDT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RDT_ABI_VERSION 1
/* Loop-index embedding table size: n_loops may not exceed this. */
#define RDT_MAX_LOOPS 4096

typedef enum {
  RDT_OK = 0,
  RDT_E_INVALID_ARG = 1,        /* null pointer, bad shape or value        */
  RDT_E_UNSUPPORTED = 2,        /* valid but not built (e.g. head_dim)     */
  RDT_E_OUT_OF_MEMORY = 3,      /* device allocation in create failed      */
  RDT_E_HIP = 4,                /* a HIP runtime call failed               */
  RDT_E_BAD_STATE = 5,          /* decode without a usable cache           */
  RDT_E_WORKSPACE_TOO_SMALL = 6 /* ws_bytes below rdt_workspace_bytes()    */
} rdt_status;

typedef enum { RDT_F32 = 0, RDT_BF16 = 1 } rdt_dtype;
typedef enum { RDT_ATTN_GQA = 0, RDT_ATTN_MLA = 1 } rdt_attn;

/* Block shape ([RC §사용법] config fields; [RC §모델 변형] variants).
 * head_dim = dim / n_heads for GQA.  loop_dim (even, <= dim) is the number
 * of leading channels that carry the loop-index signal.  weight_dtype is the
 * storage type of every matrix and of the activations fed to matrix
 * products; state, residual stream, norms and softmax stay fp32. */
typedef struct {
  int32_t dim, n_heads, n_kv_heads, head_dim;
  int32_t attn; /* rdt_attn */
  int32_t q_lora_rank, kv_lora_rank, qk_rope_head_dim, qk_nope_head_dim, v_head_dim;
  int32_t n_experts, n_shared_experts, top_k, expert_dim;
  int32_t lora_rank, max_loop_iters, loop_dim, max_seq_len;
  float rope_theta, loop_theta, norm_eps;
  int32_t weight_dtype; /* rdt_dtype */
} rdt_config;

/* Index of each tensor in the `weights` array of rdt_block_create.
 * Shapes (D dim, H heads, G kv heads, dh head_dim, E experts, F expert_dim,
 * S shared experts, r lora_rank, L max_loop_iters); "M" = weight_dtype,
 * "f32" = float.  Matrices follow the [out, in] convention of a linear map.
 *   G_REC, G_ATTN, G_FFN  f32 [D]      RMSNorm gains (recurrent, attn, ffn)
 *   WQ M [H*dh, D]  WK, WV M [G*dh, D]  WO M [D, H*dh]            (GQA)
 *   WDQ M [ql, D]  GQ f32 [ql]  WUQ M [H*(nope+rope), ql]
 *   WDKV M [kvl+rope, D]  GKV f32 [kvl]  WUKV M [H*(nope+v), kvl]
 *   WO M [D, H*v]                                                  (MLA)
 *   ROUTER M [E, D]   ROUTER_BIAS f32 [E]
 *   GATE, UP M [E, F, D]   DOWN M [E, D, F]
 *   S_GATE, S_UP M [S, F, D]   S_DOWN M [S, D, F]
 *   LORA_DOWN M [r, D]  LORA_B M [r, D]  LORA_SCALE f32 [L, r]
 *   LOG_A f32 [D]  LOG_DT f32 [1]  B f32 [D]  HALT_W f32 [D]  HALT_B f32 [1]
 * Entries not used by the chosen attention type may be NULL. */
enum rdt_weight_id {
  RDT_W_G_REC = 0, RDT_W_G_ATTN, RDT_W_G_FFN,
  RDT_W_WQ, RDT_W_WK, RDT_W_WV, RDT_W_WO,
  RDT_W_WDQ, RDT_W_GQ, RDT_W_WUQ, RDT_W_WDKV, RDT_W_GKV, RDT_W_WUKV,
  RDT_W_ROUTER, RDT_W_ROUTER_BIAS,
  RDT_W_GATE, RDT_W_UP, RDT_W_DOWN, RDT_W_S_GATE, RDT_W_S_UP, RDT_W_S_DOWN,
  RDT_W_LORA_DOWN, RDT_W_LORA_B, RDT_W_LORA_SCALE,
  RDT_W_LOG_A, RDT_W_LOG_DT, RDT_W_B, RDT_W_HALT_W, RDT_W_HALT_B,
  RDT_W_COUNT
};

typedef struct rdt_block rdt_block; /* opaque */

int32_t rdt_abi_version(void);
const char* rdt_status_string(rdt_status s);
/* Detail of the last failure on this thread ("" if none). */
const char* rdt_last_error(void);

/* Build a block: the model object of [RC §사용법].  Validates `cfg`, copies
 * the device tensors of `weights` (RDT_W_COUNT pointers, see above) into
 * handle-owned memory (query/key/value matrices concatenated), and builds
 * the RoPE, loop-index and A = exp(-exp(clamp(log_dt + log_A, -20, 20)))
 * tables on the device ([ZS §latent reasoning]).  The caller's weights may
 * be freed once `stream` has synced.  On failure *out is NULL. */
rdt_status rdt_block_create(const rdt_config* cfg, const void* const* weights, void* stream,
                            rdt_block** out);
/* Frees the handle (waits for its device work).  NULL is a no-op. */
rdt_status rdt_block_destroy(rdt_block* blk);

/* Number of block parameters (sum of the tensor sizes above). */
rdt_status rdt_param_count(const rdt_block* blk, int64_t* count);

/* Workspace bytes needed for a call on B sequences of T tokens. */
rdt_status rdt_workspace_bytes(const rdt_block* blk, int32_t B, int32_t T, size_t* bytes);

/* Bytes of a per-loop KV cache for B sequences, `capacity` positions and
 * n_loops loop slots.  Layout (element type = weight_dtype), loop slot t at
 * byte offset t * slot_bytes, slot_bytes = bytes / n_loops, and
 * P = capacity rounded up to a multiple of 64 (the position stride):
 *   GQA: K [B][G][P][dh] (after RoPE) then V transposed [B][G][dh][P];
 *        RoPE is applied before caching as [RC §Attention 구현] describes.
 *   MLA: c_kv [B][P][kv_lora_rank] (before its RMSNorm) then
 *        k_rope [B][P][qk_rope_head_dim] (after RoPE), [ZS §MLA]. */
rdt_status rdt_kv_cache_bytes(const rdt_block* blk, int32_t B, int32_t capacity, int32_t n_loops,
                              size_t* bytes);

/* The looped Recurrent Block ([ZS §Recurrent Block]; update rule of
 * [RC §아키텍처]): for t = 0 .. n_loops-1, every position runs
 *   loop-index embedding, re-injection of e and RMSNorm; a pre-norm
 *   Transformer block (causal attention with RoPE, top-k MoE with shared
 *   experts); depth-wise LoRA; h <- A*h + B*e + block output; ACT.
 * e, h0:      [B, T, D] fp32 (anchor and initial state).
 * start_pos:  absolute position of token 0 (RoPE and causal mask).
 * act_threshold: 0 = ACT off (h_out = final h, halt_counts = n_loops);
 *             in (0, 1] = ACT on (h_out = sum_t weight_t * h_t, halt_counts
 *             = 1-based loop of each position's remainder step).  With ACT
 *             on and no cache, the loops after every position has halted
 *             are skipped on the device (nothing returned can change; the
 *             per-loop capture slots of skipped loops are left untouched).
 * kv_cache:   NULL, or a cache of kv_bytes bytes with `kv_capacity`
 *             positions per slot; positions [start_pos, start_pos+T) of the
 *             first n_loops slots are written and attention reads [0, pos].
 *             Without a cache attention sees only this call's T tokens.
 * workspace:  >= rdt_workspace_bytes(B, T), 256-byte aligned.
 * h_out [B, T, D] fp32, halt_counts [B, T] int32 (outputs).
 * Errors: INVALID_ARG (nulls, B/T/n_loops < 1, n_loops > RDT_MAX_LOOPS,
 * threshold outside {0} U (0, 1], start_pos + T > max_seq_len or >
 * kv_capacity, kv_bytes too small for n_loops slots), WORKSPACE_TOO_SMALL. */
rdt_status rdt_recurrent_forward(rdt_block* blk, const float* e, const float* h0, int32_t B, int32_t T,
                                 int32_t start_pos, int32_t n_loops, float act_threshold,
                                 void* kv_cache, int32_t kv_capacity, size_t kv_bytes,
                                 void* workspace, size_t ws_bytes,
                                 float* h_out, int32_t* halt_counts, void* stream);

/* One generation step of the recurrent stage ([ZS §RoPE & generation
 * cache]): each of B sequences brings one new token at absolute position
 * start_pos; in every loop slot its K/V are appended at start_pos and
 * attention reads positions [0, start_pos].  Same outputs as
 * rdt_recurrent_forward with T = 1 (with MLA both attend over the cached
 * latent c_kv | k_rope with the k_nope / v up-projections folded into the
 * query and the output instead of rebuilding per-head K / V, [ZS §MLA];
 * equal in exact arithmetic).  BAD_STATE if kv_cache is NULL or holds
 * fewer than n_loops slots. */
rdt_status rdt_decode_step(rdt_block* blk, const float* e_new, const float* h0_new, int32_t B,
                           int32_t start_pos, int32_t n_loops, float act_threshold,
                           void* kv_cache, int32_t kv_capacity, size_t kv_bytes,
                           void* workspace, size_t ws_bytes,
                           float* h_out, int32_t* halt_counts, void* stream);

/* Copies A (fp32, [D]) to host memory, for the rho(A) < 1 check of
 * [RC §사용법] (A is diagonal, so rho(A) = max A_i).  Synchronous. */
rdt_status rdt_get_A(const rdt_block* blk, float* A_host);

/* Debug capture (off when all NULL): later forward/decode calls also write,
 * per loop t < max_loops, the state after the injection h_loops[t][N][D]
 * (fp32), the chosen experts sel_loops[t][N][top_k] (int32) and the halting
 * probability p_loops[t][N] (fp32, ACT on only).  n_loops > max_loops is
 * then INVALID_ARG.  Device pointers, caller-owned. */
rdt_status rdt_set_capture(rdt_block* blk, float* h_loops, int32_t* sel_loops, float* p_loops,
                           int32_t max_loops);

/* Byte offset and size inside the workspace of a named intermediate of the
 * last loop run (for stage-level tests).  Names: "c", "a", "q", "k", "vt",
 * "o", "x1", "f", "logits", "sel", "gate", "tile_counts", "offsets",
 * "mt_start", "tile_row0", "tile_grp", "perm", "inv", "act", "y", "act_s",
 * "y_s", "h", "cum", "live" (running-position counts of the last two loops
 * when ACT is on without a cache), "attn_part" (split-KV partials of a bf16
 * decode step; 0 bytes otherwise), "tile_claim" (tile-claim counters of the
 * routed products, zeroed by each loop's dispatch) and for MLA "kv_raw",
 * "cq_raw", "cq_norm", "lat_ckv", "lat_krope", "ckv_norm", plus for MLA
 * decode steps (T = 1, attention over the latent with absorbed
 * up-projections) "q_lat", "k_lat", "vt_lat", "o_lat" (0 bytes otherwise).
 * Matrix-product inputs and outputs ("a", "f", "q", "k", "vt", "o", "act",
 * "act_s", "y", "y_s") are stored in the weight dtype; "c", "x1", "logits",
 * "gate", "h", "cum" are fp32.  INVALID_ARG for other names. */
rdt_status rdt_workspace_offset(const rdt_block* blk, int32_t B, int32_t T, const char* name,
                                size_t* offset, size_t* bytes);

/* Per-stage kernel timing with HIP events recorded on the call's stream
 * around each stage's launches (for benchmarks; off by default; each timed
 * launch costs two event records on the stream and some host time).
 * rdt_set_timing(1) times every stage, rdt_set_timing_stages(mask) only the
 * stages whose bit (1 << rdt_stage) is set, 0 turns timing off; both clear
 * the totals.  rdt_read_timing waits for the recorded events and returns,
 * per stage, the summed milliseconds and the number of timed launches since
 * then (RDT_STAGE_COUNT entries each). */
enum rdt_stage {
  RDT_STAGE_LOOP_HEAD = 0, RDT_STAGE_QKV, RDT_STAGE_ATTN, RDT_STAGE_OPROJ, RDT_STAGE_FFN_NORM,
  RDT_STAGE_ROUTER, RDT_STAGE_DISPATCH, RDT_STAGE_EXPERT_GATEUP, RDT_STAGE_EXPERT_DOWN,
  RDT_STAGE_SHARED_GATEUP, RDT_STAGE_SHARED_DOWN, RDT_STAGE_TAIL, RDT_STAGE_COUNT
};
rdt_status rdt_set_timing(rdt_block* blk, int32_t enable);
rdt_status rdt_set_timing_stages(rdt_block* blk, uint32_t stage_mask);
rdt_status rdt_read_timing(rdt_block* blk, double* total_ms, int64_t* launches);

/* Host-only variants that take the configuration instead of a handle, so a
 * caller can size buffers (and tests can check arguments) before any device
 * work.  rdt_check_config validates a configuration; rdt_check_call returns
 * the status rdt_recurrent_forward (decode = 0) or rdt_decode_step
 * (decode = 1) would return for these sizes with non-NULL pointers. */
rdt_status rdt_check_config(const rdt_config* cfg);
rdt_status rdt_workspace_bytes_cfg(const rdt_config* cfg, int32_t B, int32_t T, size_t* bytes);
rdt_status rdt_kv_cache_bytes_cfg(const rdt_config* cfg, int32_t B, int32_t capacity, int32_t n_loops,
                                  size_t* bytes);
rdt_status rdt_workspace_offset_cfg(const rdt_config* cfg, int32_t B, int32_t T, const char* name,
                                    size_t* offset, size_t* bytes);
rdt_status rdt_check_call(const rdt_config* cfg, int32_t B, int32_t T, int32_t start_pos, int32_t n_loops,
                          float act_threshold, int32_t has_kv, int32_t kv_capacity, size_t kv_bytes,
                          size_t ws_bytes, int32_t decode);

#ifdef __cplusplus
}
#endif
#endif /* RDT_H */
