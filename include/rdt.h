/*
 * rdt.h — C ABI of the looped Recurrent-Block forward (Recurrent-Depth
 * Transformer) on one MI355X (gfx950).
 *
 * Pages cited (title, then section):
 *   [ZS] "OpenMythos 분석: Mythos Preview의 장기 추론 성능과 OpenMythos의 계산 모델링"
 *        (zero.shotlearni.ng)
 *   [RC] "OpenMythos" (runchr.com, Korean copy of the project README)
 *   [GN] "[GeekNews 요약] OpenMythos: Claude Mythos 아키텍처를 역설계한 오픈소스
 *        Recurrent-Depth Transformer 구현" (aisleshub.com)
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
 *     workspace.  The one exception is opt-in stage timing
 *     (rdt_set_timing*): while it is on, forward and decode create the HIP
 *     events they record on demand; rdt_read_timing returns them to a pool
 *     of the handle that later calls reuse, and rdt_block_destroy frees
 *     them.
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

/* ACT with compute skipping ([GN §6]: continuous depth-wise batching, a
 * halted position leaves the batch).  Same arguments and outputs as
 * rdt_recurrent_forward without a cache, ACT on (act_threshold in (0, 1]),
 * GQA attention.  Loop t runs the block only on the positions that have not
 * halted before it; a halted position's state freezes, and in later loops
 * the running positions attend to the keys and values it had in the last
 * loop it ran (the reading these pages leave open: its K/V freeze with it).
 * With nothing halting before the last loop the result equals
 * rdt_recurrent_forward's.  The loop stops once no position runs.
 * The call synchronises `stream` once per loop after the first (the host
 * reads the running count to size that loop's launches), so it returns
 * after the last loop's kernels are enqueued.  The capture buffers, when
 * set, receive loop t's values only at the positions that ran it.
 * Errors: those of rdt_recurrent_forward; INVALID_ARG if act_threshold is
 * 0; UNSUPPORTED for MLA attention.
 * Source: [GN] "[GeekNews 요약] OpenMythos: …" (aisleshub.com), section 6
 * (deployment: depth-wise batching); ACT rule of [ZS §Recurrent Block]. */
rdt_status rdt_recurrent_forward_act_skip(rdt_block* blk, const float* e, const float* h0, int32_t B, int32_t T,
                                          int32_t start_pos, int32_t n_loops, float act_threshold,
                                          void* workspace, size_t ws_bytes, float* h_out, int32_t* halt_counts,
                                          void* stream);

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

/* rdt_decode_step for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same step, arguments and outputs without the workspace,
 * which comes from a static device array of RDT_NOALLOC_MAX_WORKSPACE bytes
 * that the library holds on each device until the process ends (its
 * address is looked up once per device, in rdt_block_create).  The call
 * allocates nothing and calls no allocating routine.  Every call on one
 * device shares that array: calls that overlap on one device (on several
 * streams, or from several threads or handles) race and must be ordered by
 * the caller.  Nothing in it has to start at zero: each call writes every
 * part of it it reads.  Errors: those of rdt_decode_step;
 * WORKSPACE_TOO_SMALL when rdt_workspace_bytes(B, 1) exceeds the array
 * (32 MiB holds a 4096-wide, 128-expert block at 32 sequences);
 * BAD_STATE while stage timing is on (timing creates events). */
#define RDT_NOALLOC_MAX_WORKSPACE ((size_t)32 << 20)
rdt_status rdt_decode_step_noalloc(rdt_block* blk, const float* e_new, const float* h0_new, int32_t B,
                                   int32_t start_pos, int32_t n_loops, float act_threshold, void* kv_cache,
                                   int32_t kv_capacity, size_t kv_bytes, float* h_out, int32_t* halt_counts,
                                   void* stream);

/* ------------------------------------------------------------------------
 * The whole model around the recurrent stage ([ZS §Core Structure]): token
 * embedding, prelude layers, e = x frozen as the anchor and initial state
 * of the recurrent stage, coda layers, final RMSNorm, LM head; greedy
 * generation with per-layer caches ([ZS §RoPE & generation cache]).
 * Prelude and coda layers are pre-norm blocks with the block's attention
 * type and shapes and a dense SwiGLU feed-forward of width dim * 4 / 3
 * (integer division, [ZS §MoE]): x1 = x + Attn(RMSNorm(x)), out = x1 +
 * W2 (silu(W1 f) * (W3 f)), f = RMSNorm(x1).  No biases.
 * ------------------------------------------------------------------------ */
typedef struct {
  rdt_config block;        /* the recurrent block; its attention shape is every layer's */
  int32_t vocab_size;
  int32_t prelude_layers;  /* 0 .. 64 */
  int32_t coda_layers;     /* 0 .. 64 */
} rdt_model_config;

/* Model-level tensors (device pointers, "M" = block.weight_dtype):
 *   EMBED M [V, D]   FINAL_NORM f32 [D]   HEAD M [V, D] */
enum rdt_model_weight_id { RDT_MW_EMBED = 0, RDT_MW_FINAL_NORM, RDT_MW_HEAD, RDT_MW_COUNT };
/* Tensors of one prelude / coda layer (Fd = dim * 4 / 3):
 *   ATTN_NORM, FFN_NORM f32 [D]; attention as the block's (GQA: WQ WK WV
 *   WO; MLA: WDQ GQ WUQ WDKV GKV WUKV WO, shapes as RDT_W_*);
 *   W1 (gate), W3 (up) M [Fd, D]; W2 (down) M [D, Fd].
 * Entries of the other attention type may be NULL. */
enum rdt_layer_weight_id {
  RDT_LW_ATTN_NORM = 0, RDT_LW_WQ, RDT_LW_WK, RDT_LW_WV, RDT_LW_WO,
  RDT_LW_WDQ, RDT_LW_GQ, RDT_LW_WUQ, RDT_LW_WDKV, RDT_LW_GKV, RDT_LW_WUKV,
  RDT_LW_FFN_NORM, RDT_LW_W1, RDT_LW_W3, RDT_LW_W2, RDT_LW_COUNT
};

typedef struct rdt_model rdt_model; /* opaque */

/* Build a model: the recurrent block from `block_weights` (as
 * rdt_block_create), the model tensors from `model_weights` (RDT_MW_COUNT
 * pointers) and the layers from `layer_weights` ((prelude_layers +
 * coda_layers) * RDT_LW_COUNT pointers, prelude layers first, layer l's
 * tensor id at l * RDT_LW_COUNT + id).  Weights are copied into
 * handle-owned memory (the dense hidden width padded with zero rows /
 * columns to the matrix-product granularity, which changes no value).
 * Errors: those of rdt_block_create; INVALID_ARG for vocab_size < 1 or a
 * layer count outside [0, 64]. */
rdt_status rdt_model_create(const rdt_model_config* cfg, const void* const* block_weights,
                            const void* const* model_weights, const void* const* layer_weights, void* stream,
                            rdt_model** out);
rdt_status rdt_model_destroy(rdt_model* m);
/* The model's recurrent-stage handle (owned by the model), e.g. for
 * rdt_set_capture or stage timing of the recurrent stage. */
rdt_status rdt_model_block(const rdt_model* m, rdt_block** blk);
/* Workspace bytes of a model call on B sequences of T tokens. */
rdt_status rdt_model_workspace_bytes(const rdt_model* m, int32_t B, int32_t T, size_t* bytes);
/* Bytes of the model's cache: prelude_layers + n_loops + coda_layers slots
 * of rdt_kv_cache_bytes' layout, in that order (prelude layer i in slot i,
 * loop t in slot prelude_layers + t, coda layer j after the loops). */
rdt_status rdt_model_kv_cache_bytes(const rdt_model* m, int32_t B, int32_t capacity, int32_t n_loops,
                                    size_t* bytes);
/* The model forward ([ZS §Core Structure]).  ids: device int32, token i of
 * sequence b at ids[b * ids_ld + i]; logits: fp32 [B, T, vocab_size].
 * start_pos, n_loops, act_threshold, the cache and the workspace as for
 * rdt_recurrent_forward (a single-token call with a cache runs the decode
 * kernels).  An id outside [0, vocab_size) makes its rows' logits NaN.
 * Errors: those of rdt_recurrent_forward. */
rdt_status rdt_model_forward(rdt_model* m, const int32_t* ids, int64_t ids_ld, int32_t B, int32_t T,
                             int32_t start_pos, int32_t n_loops, float act_threshold, void* kv_cache,
                             int32_t kv_capacity, size_t kv_bytes, void* workspace, size_t ws_bytes,
                             float* logits, void* stream);
/* Greedy generation ([ZS §RoPE & generation cache]): out_ids [B, T0 +
 * max_new] (device int32) receives the prompt [B, T0] then max_new tokens;
 * step 0 runs the prompt at start_pos 0, step s > 0 the last token at
 * start_pos T0 + s - 1, each token the argmax of the last position's
 * logits (lowest id on ties).  The cache needs capacity >= T0 + max_new and
 * the workspace rdt_model_workspace_bytes(B, T0).  Stream-ordered: the
 * chosen ids never leave the device.  Errors: those of rdt_model_forward;
 * INVALID_ARG for max_new < 1. */
rdt_status rdt_model_generate(rdt_model* m, const int32_t* prompt, int32_t B, int32_t T0, int32_t max_new,
                              int32_t n_loops, float act_threshold, void* kv_cache, int32_t kv_capacity,
                              size_t kv_bytes, void* workspace, size_t ws_bytes, int32_t* out_ids,
                              void* stream);

/* ------------------------------------------------------------------------
 * Training of the recurrent stage: its backward pass and the router-bias
 * balancing step ([ZS §Tokenizer & training script] trains with AdamW in
 * bf16; [ZS §MoE] notes the selection-only router bias that no step
 * updates).  Built for bf16 GQA blocks (head_dim 128) on sequences of
 * T >= 2 tokens without a cache.
 *
 * The gradient is that of the stage's output with the discrete decisions
 * of the forward held fixed (the expert choice of every loop and position,
 * the halting loop of every position): the derivative of the piece of the
 * output map the forward took.  The router bias only enters the choice and
 * gets no gradient.  Matrix products take bf16 operands (activations,
 * their gradients and the weights) with fp32 accumulation; states, norms,
 * the residual stream and every reduction stay fp32.
 * ------------------------------------------------------------------------ */
#define RDT_MAX_TRAIN_LOOPS 64

/* Bytes of the tape a training forward records (every loop's forward
 * intermediates: one forward workspace per loop, plus the attention's
 * softmax normalisers and the experts' gate / up pre-activations) and of the backward workspace for B x T and n_loops
 * (every loop's saved gradient operands, the working buffers of one loop
 * and transposed copies of the weights). */
rdt_status rdt_train_tape_bytes(const rdt_block* blk, int32_t B, int32_t T, int32_t n_loops, size_t* bytes);
rdt_status rdt_train_workspace_bytes(const rdt_block* blk, int32_t B, int32_t T, int32_t n_loops, size_t* bytes);

/* Layout of the gradient buffer (fp32): tensor `id` (RDT_W_*, shapes as in
 * the weights table) starts at element *offset and holds *numel elements
 * (0 for tensors the block does not use).  WQ, WK, WV are back to back.
 * rdt_grad_numel gives the buffer's total element count. */
rdt_status rdt_grad_layout(const rdt_block* blk, int32_t id, int64_t* offset, int64_t* numel);
rdt_status rdt_grad_numel(const rdt_block* blk, int64_t* numel);

/* Training forward: rdt_recurrent_forward without a cache (same outputs,
 * same stop once every position has halted), each loop running in its own
 * frame of `tape` (>= rdt_train_tape_bytes, 256-byte aligned), which then
 * holds what the backward pass reads; no other workspace is needed. */
rdt_status rdt_train_forward(rdt_block* blk, const float* e, const float* h0, int32_t B, int32_t T, int32_t n_loops,
                             float act_threshold, void* tape, size_t tape_bytes, float* h_out, int32_t* halt_counts,
                             void* stream);

/* Backward pass ([ZS §Recurrent Block] forward): given dy = dL/dh_out
 * (fp32 [B, T, D]) for the output of the rdt_train_forward call that wrote
 * `tape` and `halt_counts` with the same e, h0, n_loops and act_threshold,
 * writes the gradient of every trained tensor into `grad` (fp32, layout of
 * rdt_grad_layout; the router bias's entry is 0; the padding between
 * tensors is not written), dL/de and dL/dh0 (fp32
 * [B, T, D]), and expert_load (int32 [n_experts]): the (position, slot)
 * assignments of each expert summed over the loops run.  The loops are
 * taken in reverse order from their frames of the tape (nothing of the
 * forward is recomputed); weight gradients are
 * formed over all loops' rows at the end.  The handle's
 * weights (router bias included) must not change between the two calls.
 * The call synchronises `stream` once (to read the number of loops run).
 * Errors: INVALID_ARG (nulls, sizes, n_loops > RDT_MAX_TRAIN_LOOPS),
 * UNSUPPORTED (not bf16 GQA with head_dim 128, T < 2),
 * WORKSPACE_TOO_SMALL (tape, workspace or gradient buffer). */
rdt_status rdt_train_backward(rdt_block* blk, const float* e, const float* h0, int32_t B, int32_t T,
                              int32_t n_loops, float act_threshold, const void* tape, size_t tape_bytes,
                              const int32_t* halt_counts, const float* dy, float* grad, int64_t grad_numel,
                              float* de, float* dh0, int32_t* expert_load, void* workspace, size_t ws_bytes,
                              void* stream);

/* Router-bias balancing step on the handle's bias (aux-loss-free routing,
 * the rule [ZS §MoE] finds missing): bias_i += gamma * sign(mean load -
 * load_i), with load = expert_load of rdt_train_backward (device int32
 * [n_experts]); an expert at the mean load keeps its bias. */
rdt_status rdt_router_bias_update(rdt_block* blk, const int32_t* expert_load, float gamma, void* stream);
/* Copies the handle's router bias (fp32, [n_experts]) to host memory.
 * Synchronous. */
rdt_status rdt_get_router_bias(const rdt_block* blk, float* bias_host);

/* AdamW on the handle's trained tensors ([ZS §Tokenizer & training script]
 * trains with AdamW; the rule is decoupled weight decay with bias-corrected
 * moments).  The optimizer state is three fp32 buffers in the gradient
 * layout, back to back in `state` (device, >= rdt_adamw_state_bytes,
 * 16-byte aligned, caller-owned): the master weights, the first moments m
 * and the second moments v.  rdt_adamw_init sets the masters to the
 * handle's weights (bf16 widened exactly) and the moments to 0; the router
 * bias's master keeps that initial value.
 * rdt_adamw_step, for step = 1, 2, ... (the count of steps including this
 * one), takes grad (device fp32, rdt_grad_layout, 16-byte aligned) and, for
 * every trained tensor except the router bias (which only the balancing
 * step moves):  m = beta1 m + (1 - beta1) g,  v = beta2 v + (1 - beta2) g^2,
 * master -= lr (m / (1 - beta1^step) / (sqrt(v / (1 - beta2^step)) + eps)
 * + weight_decay master);  then writes the masters into the handle's
 * weights (matrices rounded to bf16, nearest even) and recomputes A.  fp32
 * arithmetic throughout.  Stream-ordered, no synchronisation.
 * Errors: INVALID_ARG (nulls, misalignment, step < 1, lr or weight_decay
 * negative or not finite, a beta outside [0, 1), eps <= 0 or not finite),
 * UNSUPPORTED (not a bf16 GQA block), WORKSPACE_TOO_SMALL (state or
 * gradient buffer). */
rdt_status rdt_adamw_state_bytes(const rdt_block* blk, size_t* bytes);
rdt_status rdt_adamw_init(rdt_block* blk, void* state, size_t state_bytes, void* stream);
rdt_status rdt_adamw_step(rdt_block* blk, const float* grad, int64_t grad_numel, void* state, size_t state_bytes,
                          int32_t step, float lr, float beta1, float beta2, float eps, float weight_decay,
                          void* stream);
/* Size in bytes of the handle's tensor `id` (RDT_W_*, shape of the weights
 * table; bf16 for matrices of a bf16 block, else fp32), 0 for a tensor the
 * block does not use; rdt_get_weight copies it to host memory `dst` of
 * `bytes` >= that size (INVALID_ARG otherwise, or for an unused tensor).
 * Synchronous. */
rdt_status rdt_weight_bytes(const rdt_block* blk, int32_t id, size_t* bytes);
rdt_status rdt_get_weight(const rdt_block* blk, int32_t id, void* dst, size_t bytes);

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
  RDT_STAGE_SHARED_GATEUP, RDT_STAGE_SHARED_DOWN, RDT_STAGE_TAIL,
  /* rdt_train_backward: the routed experts' weight-gradient products (three
   * launches: gate, up, down) and the attention backward (per loop);
   * rdt_adamw_step's update launch */
  RDT_STAGE_TRAIN_EXPERT_WGRAD, RDT_STAGE_TRAIN_ATTN_BWD, RDT_STAGE_TRAIN_OPTIMIZER,
  RDT_STAGE_COUNT
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
