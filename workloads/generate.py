"""Seeded synthetic inputs for the recurrent-block workloads.

This module only draws random numbers and lays them out; it holds none of
the block's arithmetic.  The oracle tests, the GPU parity tests and the bench
all take their inputs from here, so both sides see the same bytes.

Recipe (one seed per config, one independent stream per tensor chunk):
  * every tensor is drawn in chunks of ``CHUNK`` elements of its flattened
    array; chunk i of tensor ``name`` uses
    ``numpy.random.default_rng(SeedSequence([seed, crc32(name), i]))``,
    so any slice can be regenerated alone and the chunks can be drawn in
    parallel threads without changing a value;
  * matrices ~ N(0, 0.02), drawn in fp32; bf16 configs keep them as bf16
    bit patterns (uint16) rounded to nearest-even from the fp32 draw;
  * norm gains = 1, router_bias = config constant (0), log_dt = 0,
    log_A ~ N(0, 1), B ~ U(0, 1), lora_scale ~ N(0, 0.02),
    halt_w ~ N(0, 0.02), halt_b = config constant;
  * e: either a lookup of uniform token ids in an N(0, 0.02) table (toy
    example) or N(0, 1) rows scaled to unit root-mean-square; h0 = e;
  * decode caches: N(0, 1) values, stored bf16, in a logical
    [B, n_kv_heads, position, head_dim] layout for both K and V.
"""

import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22

MATRICES = ("wq", "wk", "wv", "wo", "wdq", "wuq", "wdkv", "wukv",
            "router_w", "w_gate", "w_up", "w_down", "s_gate", "s_up",
            "s_down", "lora_down", "lora_B")


def _threads():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return max(1, min(16, n or 1))


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest-even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b):
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def tensor_specs(cfg):
    """name -> (shape, kind, param, stored_as_bf16)."""
    D, E, F, S, k = cfg["dim"], cfg["n_experts"], cfg["expert_dim"], cfg["n_shared_experts"], cfg["top_k"]
    H, Hkv, dh = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    r, L = cfg["lora_rank"], cfg["max_loop_iters"]
    bf = cfg["dtype"] == "bf16"
    N02 = ("normal", 0.02)
    sp = {}

    def mat(name, shape):
        sp[name] = (tuple(shape), N02[0], N02[1], bf)

    def vec(name, shape, kind, param):
        sp[name] = (tuple(shape), kind, param, False)

    vec("g_rec", [D], "const", 1.0)
    vec("g_attn", [D], "const", 1.0)
    vec("g_ffn", [D], "const", 1.0)
    if cfg["attn"] == "gqa":
        mat("wq", [H * dh, D])
        mat("wk", [Hkv * dh, D])
        mat("wv", [Hkv * dh, D])
        mat("wo", [D, H * dh])
    else:
        ql, kvl = cfg["q_lora_rank"], cfg["kv_lora_rank"]
        rope, nope, vd = cfg["qk_rope_head_dim"], cfg["qk_nope_head_dim"], cfg["v_head_dim"]
        mat("wdq", [ql, D])
        vec("gq", [ql], "const", 1.0)
        mat("wuq", [H * (nope + rope), ql])
        mat("wdkv", [kvl + rope, D])
        vec("gkv", [kvl], "const", 1.0)
        mat("wukv", [H * (nope + vd), kvl])
        mat("wo", [D, H * vd])
    mat("router_w", [E, D])
    vec("router_bias", [E], "const", cfg["router_bias"])
    mat("w_gate", [E, F, D])
    mat("w_up", [E, F, D])
    mat("w_down", [E, D, F])
    mat("s_gate", [S, F, D])
    mat("s_up", [S, F, D])
    mat("s_down", [S, D, F])
    mat("lora_down", [r, D])
    mat("lora_B", [r, D])
    vec("lora_scale", [L, r], "normal", 0.02)
    vec("log_A", [D], "normal", 1.0)
    vec("log_dt", [1], "const", 0.0)
    vec("B", [D], "uniform", 1.0)
    vec("halt_w", [D], "normal", 0.02)
    vec("halt_b", [1], "const", cfg["halt_b"])
    # the model around the recurrent stage: token embedding, prelude and
    # coda layers (pre-norm attention + dense SwiGLU of width dim * 4 // 3),
    # final norm, LM head
    if cfg.get("prelude_layers", 0) or cfg.get("coda_layers", 0):
        V, Fd = cfg["vocab"], D * 4 // 3
        mat("embed", [V, D])
        for pre, n in (("prelude", cfg["prelude_layers"]), ("coda", cfg["coda_layers"])):
            for i in range(n):
                p = f"{pre}_{i}."
                vec(p + "attn_norm", [D], "const", 1.0)
                if cfg["attn"] == "gqa":
                    mat(p + "wq", [H * dh, D])
                    mat(p + "wk", [Hkv * dh, D])
                    mat(p + "wv", [Hkv * dh, D])
                    mat(p + "wo", [D, H * dh])
                else:
                    ql, kvl = cfg["q_lora_rank"], cfg["kv_lora_rank"]
                    rope, nope, vd = cfg["qk_rope_head_dim"], cfg["qk_nope_head_dim"], cfg["v_head_dim"]
                    mat(p + "wdq", [ql, D])
                    vec(p + "gq", [ql], "const", 1.0)
                    mat(p + "wuq", [H * (nope + rope), ql])
                    mat(p + "wdkv", [kvl + rope, D])
                    vec(p + "gkv", [kvl], "const", 1.0)
                    mat(p + "wukv", [H * (nope + vd), kvl])
                    mat(p + "wo", [D, H * vd])
                vec(p + "ffn_norm", [D], "const", 1.0)
                mat(p + "w1", [Fd, D])
                mat(p + "w3", [Fd, D])
                mat(p + "w2", [D, Fd])
        vec("final_norm", [D], "const", 1.0)
        mat("head", [V, D])
    return sp


def _chunk(seed, name, i, n, kind, param):
    if kind == "const":
        return np.full(n, param, dtype=np.float32)
    rng = np.random.default_rng(np.random.SeedSequence([seed, zlib.crc32(name.encode()), i]))
    if kind == "normal":
        x = rng.standard_normal(n, dtype=np.float32)
        if param != 1.0:
            x *= np.float32(param)
        return x
    if kind == "uniform":
        return rng.random(n, dtype=np.float32) * np.float32(param)
    if kind == "int":
        return rng.integers(0, int(param), size=n, dtype=np.int64)
    raise ValueError(kind)


def draw(seed, name, shape, kind, param, as_bf16=False, start=0, stop=None, pool=None):
    """Draw elements [start, stop) of the flattened tensor ``name``."""
    total = int(np.prod(shape)) if len(shape) else 1
    stop = total if stop is None else stop
    out_dtype = np.uint16 if as_bf16 else (np.int64 if kind == "int" else np.float32)
    out = np.empty(stop - start, dtype=out_dtype)
    c0, c1 = start // CHUNK, (stop + CHUNK - 1) // CHUNK

    def job(i):
        lo, hi = i * CHUNK, min(total, (i + 1) * CHUNK)
        x = _chunk(seed, name, i, hi - lo, kind, param)
        a, b = max(lo, start), min(hi, stop)
        x = x[a - lo:b - lo]
        out[a - start:b - start] = f32_to_bf16_bits(x) if as_bf16 else x

    if c1 - c0 > 1:
        if pool is None:
            with ThreadPoolExecutor(_threads()) as ex:
                list(ex.map(job, range(c0, c1)))
        else:
            list(pool.map(job, range(c0, c1)))
    else:
        for i in range(c0, c1):
            job(i)
    return out


def make_weights(cfg, scales=None, names=None):
    """All block parameters as numpy arrays.

    ``scales`` maps a tensor name to a replacement standard deviation (or
    constant) so stage tests can use O(1) magnitudes where the default init
    would hide a term below the tolerance.
    """
    scales = scales or {}
    W = {}
    with ThreadPoolExecutor(_threads()) as pool:
        for name, (shape, kind, param, bf) in tensor_specs(cfg).items():
            if names is not None and name not in names:
                continue
            p = scales.get(name, param)
            W[name] = draw(cfg["seed"], name, shape, kind, p, bf, pool=pool).reshape(shape)
    return W


def expert_slice(cfg, name, e, scales=None):
    """One expert's matrix of a stacked [E, ...] tensor, drawn on its own."""
    shape, kind, param, bf = tensor_specs(cfg)[name]
    per = int(np.prod(shape[1:]))
    p = (scales or {}).get(name, param)
    return draw(cfg["seed"], name, shape, kind, p, bf, start=e * per, stop=(e + 1) * per).reshape(shape[1:])


def make_inputs(cfg):
    """e [B, T, D] fp32 and h0 (= e), as in the pages' wiring where the
    recurrent stage receives the prelude output both as state and anchor."""
    B, T, D = cfg["batch"], cfg["seq"], cfg["dim"]
    seed = cfg["seed"]
    if cfg["e_kind"] == "embed":
        ids = draw(seed, "ids", (B, T), "int", cfg["vocab"]).reshape(B, T)
        table = draw(seed, "embed", (cfg["vocab"], D), "normal", 0.02).reshape(cfg["vocab"], D)
        e = table[ids]
    else:
        x = draw(seed, "e_raw", (B, T, D), "normal", 1.0).reshape(B, T, D).astype(np.float64)
        e = (x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True))).astype(np.float32)
    e = np.ascontiguousarray(e, dtype=np.float32)
    return e, e.copy()


def make_ids(cfg):
    """Prompt token ids [B, T], uniform in [0, vocab) (the usage example of
    the pages draws them the same way)."""
    B, T = cfg["batch"], cfg["seq"]
    return draw(cfg["seed"], "ids", (B, T), "int", cfg["vocab"]).reshape(B, T).astype(np.int32)


def make_cache_loop(cfg, t, which, b_range=None):
    """Prior K or V values of loop ``t``'s cache, logical layout
    [B, n_kv_heads, start_pos, head_dim], bf16 bits, N(0, 1)."""
    B, G, P, dh = cfg["batch"], cfg["n_kv_heads"], cfg["start_pos"], cfg["head_dim"]
    shape = (B, G, P, dh)
    per_b = G * P * dh
    b0, b1 = (0, B) if b_range is None else b_range
    x = draw(cfg["seed"], f"cache_{which}_{t}", shape, "normal", 1.0, True, start=b0 * per_b, stop=b1 * per_b)
    return x.reshape(b1 - b0, G, P, dh)
