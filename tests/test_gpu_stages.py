"""Stage-level parity: each kernel against the oracle's step fed the GPU's own
inputs of that step (read from the workspace after a one-loop forward), so
an error is pinned to the kernel that makes it.

Tolerances: outputs stored in bf16 may differ by their own rounding (2^-8
relative) plus fp32 accumulation; fp32 outputs by accumulation only.
"""

import math

import numpy as np
import pytest

from oracle import rdt_oracle as O
from workloads import configs, generate

from gpu_support import DeviceRun

pytestmark = pytest.mark.gpu


def _max_rel(got, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / (np.sqrt(np.mean(ref * ref)) + 1e-30))


def _elem_bf16_ok(got, ref, rel=2 ** -7, abs_=1e-6):
    """Element-wise: |got - ref| <= rel * |ref| + abs_ * rms(ref)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.sqrt(np.mean(ref * ref))
    bad = np.abs(got - ref) > rel * np.abs(ref) + abs_ * scale + 1e-3 * scale
    return int(bad.sum()), np.argwhere(bad)[:5]


@pytest.fixture(scope="module", params=["small_bf16", "small_bf16_k3", "small_f32", "small_bf16_strip"])
def stage_run(request):
    name = request.param
    cfg = configs.get(name, n_loops=1, act_threshold=0.0)
    W = generate.make_weights(cfg)
    e, h0 = generate.make_inputs(cfg)
    print(f"[stages] {name}", flush=True)
    run = DeviceRun(cfg, W, e, h0)
    return cfg, W, e, h0, run


def _get(run, cfg, name, shape, kind="act"):
    import torch
    if kind == "act":
        dt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    elif kind == "f32":
        dt = torch.float32
    else:
        dt = torch.int32
    x = run.ws_np(name, dt, shape)
    return O.as_f64(x) if kind != "i32" else x


def test_stage_loop_head(stage_run):
    cfg, W, e, h0, run = stage_run
    P = O.Params(W)
    B, T, D = e.shape
    N = B * T
    u = h0.astype(np.float64) + O.loop_index_embedding(0, cfg["loop_dim"], D, cfg["loop_theta"])
    c = O.rms_norm(u + e, P["g_rec"], cfg["norm_eps"]).reshape(N, D)
    gc = _get(run, cfg, "c", (N, D), "f32")
    assert _max_rel(gc, c) < 1e-5
    a = O.rms_norm(gc, P["g_attn"], cfg["norm_eps"])
    ga = _get(run, cfg, "a", (N, D))
    nbad, where = _elem_bf16_ok(ga, a)
    assert nbad == 0, where


def test_stage_qkv_rope(stage_run):
    cfg, W, e, h0, run = stage_run
    P = O.Params(W)
    B, T, D = e.shape
    N, H, G, dh = B * T, cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    a = _get(run, cfg, "a", (N, D)).reshape(B, T, D)
    cos, sin = O.rope_cos_sin(np.arange(T), dh, cfg["rope_theta"])
    q = O.apply_rope((a @ P["wq"].T).reshape(B, T, H, dh).transpose(0, 2, 1, 3), cos, sin)
    k = O.apply_rope((a @ P["wk"].T).reshape(B, T, G, dh).transpose(0, 2, 1, 3), cos, sin)
    v = (a @ P["wv"].T).reshape(B, T, G, dh).transpose(0, 2, 1, 3)
    cap = (T + 63) // 64 * 64
    gq = _get(run, cfg, "q", (B, H, T, dh))
    gk = _get(run, cfg, "k", (B, G, cap, dh))[:, :, :T]
    gv = _get(run, cfg, "vt", (B, G, dh, cap))[:, :, :, :T].transpose(0, 1, 3, 2)
    for name, g_, r_ in (("q", gq, q), ("k", gk, k), ("v", gv, v)):
        nbad, where = _elem_bf16_ok(g_, r_)
        assert nbad == 0, (name, where)


def test_stage_attention(stage_run):
    cfg, W, e, h0, run = stage_run
    B, T, D = e.shape
    N, H, G, dh = B * T, cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    cap = (T + 63) // 64 * 64
    q = _get(run, cfg, "q", (B, H, T, dh))
    k = _get(run, cfg, "k", (B, G, cap, dh))[:, :, :T]
    v = _get(run, cfg, "vt", (B, G, dh, cap))[:, :, :, :T].transpose(0, 1, 3, 2)
    pos = np.arange(T)
    o = np.zeros((B, T, H, dh))
    for b in range(B):
        for h in range(H):
            g = h // (H // G)
            o[b, :, h] = O.attend(q[b, h], k[b, g], v[b, g], pos, pos, 1 / math.sqrt(dh))
    go = _get(run, cfg, "o", (B, T, H, dh))
    # o is a convex combination of v rows; with P and o rounded to bf16 the
    # error is a few 2^-9 of the largest |v| (rows with few keys have |o|
    # near |v|, far above rms(o), so rms(o) is not the scale here)
    err = float(np.max(np.abs(go - o)) / np.max(np.abs(v)))
    print(f"  attention max|d|/max|v| = {err:.2e}")
    assert err < (1e-2 if cfg["dtype"] == "bf16" else 1e-6)


def test_stage_oproj_ffn_norm_router(stage_run):
    cfg, W, e, h0, run = stage_run
    P = O.Params(W)
    B, T, D = e.shape
    N, H, dh, E = B * T, cfg["n_heads"], cfg["head_dim"], cfg["n_experts"]
    o = _get(run, cfg, "o", (N, H * dh))
    c = _get(run, cfg, "c", (N, D), "f32")
    x1 = c + o @ P["wo"].T
    gx1 = _get(run, cfg, "x1", (N, D), "f32")
    assert _max_rel(gx1, x1) < 1e-5
    f = O.rms_norm(gx1, P["g_ffn"], cfg["norm_eps"])
    gf = _get(run, cfg, "f", (N, D))
    nbad, where = _elem_bf16_ok(gf, f)
    assert nbad == 0, where
    z = gf @ P["router_w"].T
    gz = _get(run, cfg, "logits", (N, E), "f32")
    assert np.max(np.abs(gz - z)) < 1e-5 * np.max(np.abs(z)) + 1e-6


def test_stage_experts(stage_run):
    cfg, W, e, h0, run = stage_run
    P = O.Params(W)
    B, T, D = e.shape
    N, k, F, S = B * T, cfg["top_k"], cfg["expert_dim"], cfg["n_shared_experts"]
    f = _get(run, cfg, "f", (N, D))
    sel = _get(run, cfg, "sel", (N, k), "i32")
    perm = _get(run, cfg, "perm", (N * k,), "i32")
    inv = _get(run, cfg, "inv", (N * k,), "i32")
    act = _get(run, cfg, "act", (N * k, F))
    y = _get(run, cfg, "y", (N * k, D))
    for a in range(N * k):
        assert perm[inv[a]] == a // k
    # per dispatch row: expert of the slot, token row
    slot_of_row = np.argsort(inv)
    ex_of_row = sel.ravel()[slot_of_row]
    ref_act = np.zeros((N * k, F))
    for ex in np.unique(ex_of_row):
        rows = np.nonzero(ex_of_row == ex)[0]
        x = f[perm[rows]]
        ref_act[rows] = O.silu(x @ P.expert("w_gate", ex).T) * (x @ P.expert("w_up", ex).T)
    nbad, where = _elem_bf16_ok(act, ref_act, abs_=1e-4)
    assert nbad == 0, where
    ref_y = np.zeros((N * k, D))
    for ex in np.unique(ex_of_row):
        rows = np.nonzero(ex_of_row == ex)[0]
        ref_y[rows] = act[rows] @ P.expert("w_down", ex).T
    # y is stored in the activation dtype (bf16 configs: its own rounding)
    if cfg["dtype"] == "bf16":
        nbad, where = _elem_bf16_ok(y, ref_y, abs_=1e-4)
        assert nbad == 0, where
    else:
        assert _max_rel(y, ref_y) < 1e-5
    acts = _get(run, cfg, "act_s", (N, F))
    ys = _get(run, cfg, "y_s", (S, N, D))
    ref_as = O.silu(f @ P.expert("s_gate", S - 1).T) * (f @ P.expert("s_up", S - 1).T)
    nbad, where = _elem_bf16_ok(acts, ref_as, abs_=1e-4)
    assert nbad == 0, where
    ref_ys = acts @ P.expert("s_down", S - 1).T
    if cfg["dtype"] == "bf16":
        nbad, where = _elem_bf16_ok(ys[S - 1], ref_ys, abs_=1e-4)
        assert nbad == 0, where
    else:
        assert _max_rel(ys[S - 1], ref_ys) < 1e-5


def test_stage_tail(stage_run):
    cfg, W, e, h0, run = stage_run
    P = O.Params(W)
    B, T, D = e.shape
    N, k, S = B * T, cfg["top_k"], cfg["n_shared_experts"]
    x1 = _get(run, cfg, "x1", (N, D), "f32")
    y = _get(run, cfg, "y", (N * k, D))
    ys = _get(run, cfg, "y_s", (S, N, D))
    inv = _get(run, cfg, "inv", (N * k,), "i32")
    gate = _get(run, cfg, "gate", (N * k,), "f32")
    tau = x1 + (gate[:, None] * y[inv]).reshape(N, k, D).sum(1) + ys.sum(0)
    tau = tau + O.depthwise_lora(cfg, P, tau, 0)
    h = O.lti_injection(P, h0.reshape(N, D).astype(np.float64), e.reshape(N, D).astype(np.float64), tau)
    gh = run.np()["out"].reshape(N, D)
    assert _max_rel(gh, h) < 1e-5
