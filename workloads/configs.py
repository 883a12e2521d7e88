"""Block shapes and run settings of the recurrent-block workloads.

Pure data: no arithmetic of the method lives here.  Both the oracle tests and
the HIP path read these dictionaries; the seeded tensors come from
``workloads.generate``.

Sources of the shapes (cited by page title and section):
  [ZS]  "OpenMythos 분석: Mythos Preview의 장기 추론 성능과 OpenMythos의 계산 모델링"
        (zero.shotlearni.ng blog)
  [RC]  "OpenMythos" (runchr.com, Korean copy of the project README)

* tiny_gqa / tiny_mla: the toy configuration of the usage example on [RC]
  (section "사용법": dim 256, 8 heads, 8 experts of width 64, top-2, one
  shared expert, LoRA rank 8, max_loop_iters 4; GQA with 2 KV heads, or MLA
  with kv_lora 32 / q_lora 64 / rope 16 / nope 16 / v 16; ids of shape (2, 16)).
* mythos_1b / mythos_3b / mythos_10b_decode: rows of the variants table on
  [RC] (section "모델 변형": dim, expert count, expert width, loop iterations).
  Head counts, KV-head counts, LoRA rank and batch shapes are workload
  choices stated here, not values the pages print.
* small_*: extra parity shapes (several MFMA tiles plus ragged tails) that
  the fp64 oracle finishes in seconds.

Readings that the pages leave open (loop_dim = dim/8, eps 1e-6, rope/loop
base 10000, fp32 state with bf16 matrices) are recorded per config so both
sides read the same constants.
"""

import copy

_COMMON = dict(
    rope_theta=10000.0,
    loop_theta=10000.0,
    norm_eps=1e-6,
    router_bias=0.0,
    start_pos=0,
    halt_b=0.0,
    q_lora_rank=0,
    kv_lora_rank=0,
    qk_rope_head_dim=0,
    qk_nope_head_dim=0,
    v_head_dim=0,
    use_cache=False,
    # the model around the recurrent stage (token embedding, prelude and
    # coda layers, final norm, LM head); the block-only workloads have none
    prelude_layers=0,
    coda_layers=0,
    # how e is made: "embed" = lookup of uniform token ids in an N(0, 0.02)
    # table (toy example); "rmsnorm_normal" = N(0,1) rows, RMS-normalised.
    e_kind="rmsnorm_normal",
    vocab=1000,
)


def _cfg(**kw):
    c = dict(_COMMON)
    c.update(kw)
    if c["attn"] == "gqa":
        c.setdefault("head_dim", c["dim"] // c["n_heads"])
    else:
        c.setdefault("head_dim", c["qk_nope_head_dim"] + c["qk_rope_head_dim"])
    c.setdefault("loop_dim", c["dim"] // 8)
    c.setdefault("max_seq_len", max(c["start_pos"] + c["seq"], 16))
    return c


CONFIGS = {
    # toy example, GQA, fp32 (usage section of [RC])
    "tiny_gqa": _cfg(
        dim=256, n_heads=8, n_kv_heads=2, attn="gqa",
        n_experts=8, n_shared_experts=1, top_k=2, expert_dim=64,
        lora_rank=8, max_loop_iters=4, max_seq_len=128,
        dtype="f32", batch=2, seq=16, n_loops=4, act_threshold=0.99,
        seed=1, e_kind="embed"),
    # toy example, MLA, fp32; 8 loops > max_loop_iters 4 exercises the LoRA clamp
    "tiny_mla": _cfg(
        dim=256, n_heads=8, n_kv_heads=8, attn="mla",
        q_lora_rank=64, kv_lora_rank=32, qk_rope_head_dim=16,
        qk_nope_head_dim=16, v_head_dim=16,
        n_experts=8, n_shared_experts=1, top_k=2, expert_dim=64,
        lora_rank=8, max_loop_iters=4, max_seq_len=128,
        dtype="f32", batch=2, seq=16, n_loops=8, act_threshold=0.99,
        seed=2, e_kind="embed"),
    # 1b row of the variants table: bf16 prefill, fixed 16 loops (ACT off)
    "mythos_1b": _cfg(
        dim=2048, n_heads=16, n_kv_heads=4, attn="gqa",
        n_experts=64, n_shared_experts=1, top_k=2, expert_dim=2048,
        lora_rank=16, max_loop_iters=16, max_seq_len=4096,
        dtype="bf16", batch=1, seq=4096, n_loops=16, act_threshold=0.0,
        seed=3),
    # 3b row: bf16 prefill with ACT at 0.99; halt_b set by the calibration
    # script (workloads/calibrate_halt.py) and read from calibration.json
    "mythos_3b": _cfg(
        dim=3072, n_heads=24, n_kv_heads=8, attn="gqa",
        n_experts=64, n_shared_experts=1, top_k=2, expert_dim=4096,
        lora_rank=16, max_loop_iters=16, max_seq_len=4096,
        dtype="bf16", batch=2, seq=4096, n_loops=16, act_threshold=0.99,
        seed=4),
    # 10b row: bf16 decode, 32 sequences x 1 new token against 8192 cached
    # positions in every loop's cache, 24 loops, ACT off
    "mythos_10b_decode": _cfg(
        dim=4096, n_heads=32, n_kv_heads=8, attn="gqa",
        n_experts=128, n_shared_experts=1, top_k=2, expert_dim=5632,
        lora_rank=16, max_loop_iters=24, max_seq_len=8193,
        dtype="bf16", batch=32, seq=1, start_pos=8192, n_loops=24,
        act_threshold=0.0, seed=5, use_cache=True),

    # ---- parity shapes the oracle finishes in seconds ----
    # bf16, head_dim 128 like the large configs, ragged T, ACT on
    "small_bf16": _cfg(
        dim=512, n_heads=4, n_kv_heads=2, attn="gqa",
        n_experts=8, n_shared_experts=1, top_k=2, expert_dim=384,
        lora_rank=8, max_loop_iters=4, max_seq_len=512,
        dtype="bf16", batch=2, seq=200, n_loops=3, act_threshold=0.99,
        seed=11),
    # bf16, odd sizes: top-3 of 12 experts, two shared experts, T not a
    # multiple of any tile, ACT off
    "small_bf16_k3": _cfg(
        dim=384, n_heads=3, n_kv_heads=1, attn="gqa",
        n_experts=12, n_shared_experts=2, top_k=3, expert_dim=320,
        lora_rank=4, max_loop_iters=2, max_seq_len=512,
        dtype="bf16", batch=3, seq=77, n_loops=3, act_threshold=0.0,
        seed=12),
    # bf16, dim a multiple of 192 with ~270 routed rows per expert: the
    # routed down product's 192-column tiles and merged m-tile schedule
    # (experts 1-64 rows past 256 computed as strips of the same tile)
    "small_bf16_strip": _cfg(
        dim=768, n_heads=6, n_kv_heads=2, attn="gqa",
        n_experts=8, n_shared_experts=1, top_k=2, expert_dim=384,
        lora_rank=8, max_loop_iters=4, max_seq_len=1088,
        dtype="bf16", batch=2, seq=540, n_loops=2, act_threshold=0.0,
        seed=15),
    # bf16 decode against a cache: 4 sequences, 1 token at position 300
    "small_bf16_decode": _cfg(
        dim=512, n_heads=4, n_kv_heads=2, attn="gqa",
        n_experts=16, n_shared_experts=1, top_k=2, expert_dim=256,
        lora_rank=8, max_loop_iters=4, max_seq_len=512,
        dtype="bf16", batch=4, seq=1, start_pos=300, n_loops=3,
        act_threshold=0.0, seed=13, use_cache=True),
    # fp32 GQA with a longer ragged sequence (several attention tiles)
    "small_f32": _cfg(
        dim=256, n_heads=8, n_kv_heads=4, attn="gqa",
        n_experts=8, n_shared_experts=1, top_k=2, expert_dim=96,
        lora_rank=8, max_loop_iters=4, max_seq_len=256,
        dtype="f32", batch=2, seq=150, n_loops=3, act_threshold=0.99,
        seed=14),

    # ---- whole model: the usage example of [RC] (vocabulary 1000, one
    # prelude and one coda layer, prompt of 2 x 16 token ids, 4 loops; 8 new
    # tokens generated with 8 loops) ----
    "tiny_model_gqa": _cfg(
        dim=256, n_heads=8, n_kv_heads=2, attn="gqa",
        n_experts=8, n_shared_experts=1, top_k=2, expert_dim=64,
        lora_rank=8, max_loop_iters=4, max_seq_len=128,
        dtype="f32", batch=2, seq=16, n_loops=4, act_threshold=0.99,
        seed=21, vocab=1000, prelude_layers=1, coda_layers=1),
    "tiny_model_mla": _cfg(
        dim=256, n_heads=8, n_kv_heads=8, attn="mla",
        q_lora_rank=64, kv_lora_rank=32, qk_rope_head_dim=16,
        qk_nope_head_dim=16, v_head_dim=16,
        n_experts=8, n_shared_experts=1, top_k=2, expert_dim=64,
        lora_rank=8, max_loop_iters=4, max_seq_len=128,
        dtype="f32", batch=2, seq=16, n_loops=4, act_threshold=0.99,
        seed=22, vocab=1000, prelude_layers=1, coda_layers=1),
    # bf16 model shape with head_dim 128 (large-tile GEMMs, flash and split-KV
    # attention in every layer), two prelude layers, ragged prompt
    "small_model_bf16": _cfg(
        dim=512, n_heads=4, n_kv_heads=2, attn="gqa",
        n_experts=8, n_shared_experts=1, top_k=2, expert_dim=384,
        lora_rank=8, max_loop_iters=4, max_seq_len=256,
        dtype="bf16", batch=2, seq=70, n_loops=3, act_threshold=0.99,
        seed=23, vocab=3000, prelude_layers=2, coda_layers=1),
}


def get(name, **overrides):
    """A copy of a named config, with optional field overrides."""
    c = copy.deepcopy(CONFIGS[name])
    c.update(overrides)
    c["name"] = name
    return c


def tokens_x_loops(cfg):
    return cfg["batch"] * cfg["seq"] * cfg["n_loops"]


def _apply_calibration():
    """mythos_3b's halting-head bias comes from workloads/calibrate_halt.py
    (an oracle run), stored in calibration.json beside this file."""
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "calibration.json")
    if os.path.exists(path):
        cal = json.load(open(path))
        for name, vals in cal.items():
            if name in CONFIGS:
                CONFIGS[name]["halt_b"] = float(vals["halt_b"])


_apply_calibration()
