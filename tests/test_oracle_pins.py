"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each test ties one oracle function to a closed form, an invariant the pages
state, brute force on tiny inputs, or an independent library routine
(PyTorch CPU: rms_norm, complex multiplication, scaled_dot_product_attention),
so that a dropped term, a wrong sign or index, or a transposed operand in the
oracle fails at least one of them.

Pages: [ZS] "OpenMythos 분석: …의 계산 모델링" (zero.shotlearni.ng);
[RC] "OpenMythos" (runchr.com).
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import rdt_oracle as O
from workloads import configs, generate

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _setup(name, scales=None, **over):
    cfg = configs.get(name, **over)
    W = generate.make_weights(cfg, scales=scales)
    e, h0 = generate.make_inputs(cfg)
    return cfg, W, O.Params(W), e, h0


def _t64(a):
    """float64 torch tensor of a weight array, decoded by torch itself:
    uint16 arrays are bfloat16 bit patterns (reinterpreted as torch.bfloat16),
    so this path shares no decoding with the oracle's as_f64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).double()
    return torch.from_numpy(a.astype(np.float64))


# ---------------------------------------------------------------- injection

def test_A_matches_zoh_discretisation_and_clamp():
    """[RC §해결책]: A = exp(dt * A_c) with A_c = -exp(log_A), dt = exp(log_dt)
    (zero-order hold of a negative diagonal); [ZS §latent reasoning] clamps
    log_dt + log_A to [-20, 20].  Values from tests/golden/lti_A.json."""
    gold = json.load(open(os.path.join(GOLDEN, "lti_A.json")))
    for case in gold["cases"]:
        P = O.Params({"log_A": np.array(case["log_A"]), "log_dt": np.array([case["log_dt"]])})
        A = O.lti_A(P)
        # inside the clamp: the ZOH form, written independently
        for la, a in zip(case["log_A"], A):
            s = case["log_dt"] + la
            if -20 <= s <= 20:
                ref = math.exp(math.exp(case["log_dt"]) * -math.exp(la))
                assert a == pytest.approx(ref, rel=1e-14, abs=0)
        np.testing.assert_allclose(A, case["expected"], rtol=1e-12, atol=0)


def test_transformer_term_zero_gives_closed_form_lti():
    """With the recurrent norm gain at 0 the block input is 0, so attention,
    experts and LoRA all return 0 and the loop is the pure LTI recurrence
    h_t = A^t h0 + (1 - A^t)/(1 - A) * B * e ([RC §동적 시스템 관점])."""
    cfg, W, P, e, h0 = _setup("tiny_gqa")
    W = dict(W)
    W["g_rec"] = np.zeros_like(W["g_rec"])
    P = O.Params(W)
    A = O.lti_A(P)
    Bv = O.as_f64(W["B"])
    e64, h64 = e.astype(np.float64), h0.astype(np.float64) * 0.5 + 0.3   # h0 != e on purpose
    for n in (1, 3, 6):
        r = O.recurrent_forward(cfg, P, e64, h64, n, 0.0)
        ref = A ** n * h64 + (1 - A ** n) / (1 - A) * Bv * e64
        np.testing.assert_allclose(r["out"], ref, rtol=1e-12, atol=1e-13)


def test_lti_fixed_point_after_5000_loops():
    """rho(A) < 1 makes h converge to (I - A)^-1 B e for any start."""
    cfg, W, P, e, h0 = _setup("tiny_gqa")
    e64 = e.astype(np.float64)
    h = np.full_like(e64, 7.0)
    for _ in range(5000):
        h = O.lti_injection(P, h, e64, 0.0)
    fixed = O.as_f64(W["B"]) * e64 / (1.0 - O.lti_A(P))
    np.testing.assert_allclose(h, fixed, rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", ["tiny_gqa", "tiny_mla", "small_bf16", "mythos_1b", "mythos_3b", "mythos_10b_decode"])
def test_spectral_radius_below_one(name):
    """[RC §사용법] checks rho(A) < 1; A diagonal so rho = max A_i.  Also in
    fp32, where exp(-exp(x)) rounds to 1 for x below about -17."""
    cfg = configs.get(name)
    W = generate.make_weights(cfg, names={"log_A", "log_dt"})
    A = O.lti_A(O.Params(W))
    assert A.max() < 1.0 and A.min() > 0.0
    assert np.float32(A.max()) <= np.float32(1.0 - 2.0 ** -24)


# ---------------------------------------------------------------- loop index

def test_loop_index_embedding_closed_form():
    """[ZS §Repeating the parameter reduces expressiveness]: sin then cos of
    t * freq on the leading channels, zero elsewhere."""
    emb0 = O.loop_index_embedding(0, 8, 16, 10000.0)
    np.testing.assert_array_equal(emb0, [0, 0, 0, 0, 1, 1, 1, 1] + [0] * 8)
    emb = O.loop_index_embedding(3, 8, 16, 10000.0)
    freqs = [1.0, 0.1, 0.01, 0.001]          # 10000^(-2j/8)
    np.testing.assert_allclose(emb[:4], [math.sin(3 * f) for f in freqs], rtol=1e-15, atol=1e-16)
    np.testing.assert_allclose(emb[4:8], [math.cos(3 * f) for f in freqs], rtol=1e-15)
    assert np.all(emb[8:] == 0)
    pairs = emb[:4] ** 2 + emb[4:8] ** 2
    np.testing.assert_allclose(pairs, 1.0, rtol=1e-15)


# ---------------------------------------------------------------- norms, rope

def test_rms_norm_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64))
    g = rng.standard_normal(64)
    ref = F.rms_norm(torch.from_numpy(x), (64,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(O.rms_norm(x, g, 1e-6), ref, rtol=1e-13, atol=1e-14)


def test_rope_matches_complex_rotation_and_is_relative():
    """[ZS §RoPE & generation cache]: adjacent pairs are complex numbers
    rotated by position.  Checked against torch complex arithmetic, norm
    preservation, and q_m . k_n depending only on m - n."""
    rng = np.random.default_rng(1)
    d, theta = 16, 10000.0
    x = rng.standard_normal((7, d))
    pos = np.arange(3, 10)
    cos, sin = O.rope_cos_sin(pos, d, theta)
    got = O.apply_rope(x, cos, sin)
    xc = torch.view_as_complex(torch.from_numpy(x).reshape(7, d // 2, 2).contiguous())
    inv = theta ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    ph = torch.polar(torch.ones(7, d // 2, dtype=torch.float64), torch.from_numpy(pos).double()[:, None] * inv)
    ref = torch.view_as_real(xc * ph).reshape(7, d).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(np.linalg.norm(got, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    def score(m, n):
        cm, sm = O.rope_cos_sin([m], d, theta)
        cn, sn = O.rope_cos_sin([n], d, theta)
        return O.apply_rope(q[None], cm, sm)[0] @ O.apply_rope(k[None], cn, sn)[0]
    assert score(9, 4) == pytest.approx(score(105, 100), rel=1e-10)
    assert score(9, 4) != pytest.approx(score(9, 5), rel=1e-3)


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("H,G", [(8, 2), (4, 4), (6, 3)])
def test_attention_matches_sdpa(H, G):
    """Oracle causal attention with GQA head mapping == torch SDPA
    (enable_gqa); H == G is plain multi-head attention."""
    rng = np.random.default_rng(H * 10 + G)
    T, d = 11, 16
    q = rng.standard_normal((H, T, d))
    k = rng.standard_normal((G, T, d))
    v = rng.standard_normal((G, T, d))
    pos = np.arange(T)
    got = np.stack([O.attend(q[h], k[h // (H // G)], v[h // (H // G)], pos, pos, 1 / math.sqrt(d)) for h in range(H)])
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None], torch.from_numpy(k)[None],
                                         torch.from_numpy(v)[None], is_causal=True, enable_gqa=True)[0].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- router / MoE

def test_topk_matches_brute_force_sort():
    rng = np.random.default_rng(2)
    v = rng.integers(0, 4, size=(50, 9)).astype(np.float32)   # many exact ties
    got = O.topk_desc_lowest_index(v, 3)
    for n in range(50):
        ref = sorted(range(9), key=lambda j: (-v[n, j], j))[:3]
        assert list(got[n]) == ref


def test_router_gates_use_unbiased_scores():
    """[ZS §MoE]: the bias steers selection only; gates come from the
    unbiased softmax renormalised over the chosen experts."""
    cfg, W, P, e, h0 = _setup("tiny_gqa")
    rng = np.random.default_rng(3)
    f = rng.standard_normal((20, cfg["dim"]))
    W2 = dict(W)
    bias = np.zeros(cfg["n_experts"], dtype=np.float32)
    bias[5] = 1e3
    W2["router_bias"] = bias
    z, sel, gate, _ = O.router(cfg, O.Params(W2), f)
    assert np.all(sel[:, 0] == 5)
    s = np.exp(z) / np.exp(z).sum(1, keepdims=True)
    np.testing.assert_allclose(s.sum(1), 1.0, rtol=1e-14)
    for n in range(20):
        ref = s[n, sel[n]] / s[n, sel[n]].sum()
        np.testing.assert_allclose(gate[n], ref, rtol=1e-14)
    np.testing.assert_allclose(gate.sum(1), 1.0, rtol=1e-14)


def test_moe_equals_dense_masked_sum():
    """Top-k MoE == every expert on every row, weighted by a gate matrix that
    is zero outside the chosen set (brute force), plus the shared expert."""
    cfg, W, P, e, h0 = _setup("tiny_gqa", n_shared_experts=2)
    rng = np.random.default_rng(4)
    f = rng.standard_normal((24, cfg["dim"]))
    z, sel, gate, _ = O.router(cfg, P, f)
    got = O.moe_ffn(cfg, P, f, sel, gate)
    ft = torch.from_numpy(f)
    def expert(wg, wu, wd):
        return F.linear(F.silu(F.linear(ft, _t64(wg))) * F.linear(ft, _t64(wu)), _t64(wd))
    dense = torch.stack([expert(W["w_gate"][x], W["w_up"][x], W["w_down"][x]) for x in range(cfg["n_experts"])], 1)
    mask = torch.zeros(24, cfg["n_experts"], dtype=torch.float64)
    for n in range(24):
        for j in range(cfg["top_k"]):
            mask[n, sel[n, j]] += gate[n, j]
    ref = (dense * mask[:, :, None]).sum(1)
    for s_ in range(2):
        ref = ref + expert(W["s_gate"][s_], W["s_up"][s_], W["s_down"][s_])
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-11, atol=1e-14)


# ---------------------------------------------------------------- LoRA

def test_depthwise_lora_closed_form_and_clamp():
    """With basis-vector down/B rows the LoRA term is x_j * scale[t', j] on the
    first r channels; t' = min(t, L - 1) ([ZS §Repeating the parameter
    reduces expressiveness]); scale 0 is a no-op."""
    D, r, L = 12, 3, 4
    cfg = dict(max_loop_iters=L)
    eye = np.eye(r, D)
    scale = np.arange(1, L * r + 1, dtype=np.float64).reshape(L, r)
    P = O.Params({"lora_down": eye, "lora_B": eye * 2.0, "lora_scale": scale})
    x = np.random.default_rng(5).standard_normal((4, D))
    for t in range(7):
        ti = min(t, L - 1)
        ref = np.zeros_like(x)
        ref[:, :r] = x[:, :r] * scale[ti] * 2.0
        np.testing.assert_allclose(O.depthwise_lora(cfg, P, x, t), ref, rtol=1e-15)
    P0 = O.Params({"lora_down": eye, "lora_B": eye, "lora_scale": np.zeros((L, r))})
    assert np.all(O.depthwise_lora(cfg, P0, x, 2) == 0)


# ---------------------------------------------------------------- ACT

def test_stop_once_all_halted_changes_nothing():
    """With every position halted by loop 2, stopping there returns the same
    output and halt counts as running all loops (the later loops only move
    h, which the ACT output no longer weights)."""
    scales = {"halt_w": 0.02, "halt_b": 1.0}
    cfg, W, P, e, h0 = _setup("tiny_gqa", scales=scales)
    n = 4
    stop = O.recurrent_forward(cfg, P, e, h0, n, cfg["act_threshold"])
    full = O.recurrent_forward(cfg, P, e, h0, n, cfg["act_threshold"], stop_when_halted=False)
    assert stop["loops_run"] < n and full["loops_run"] == n
    np.testing.assert_array_equal(stop["out"], full["out"])
    np.testing.assert_array_equal(stop["halt_counts"], full["halt_counts"])
    assert stop["halt_counts"].max() == stop["loops_run"]
    # with a cache being filled every loop runs
    cache = O.new_cache(cfg, cfg["batch"], cfg["seq"], n)
    assert O.recurrent_forward(cfg, P, e, h0, n, cfg["act_threshold"], cache=cache)["loops_run"] == n


@pytest.mark.parametrize("name", ["tiny_gqa", "tiny_mla", "small_f32"])
def test_act_weights_sum_to_one_and_first_crossing(name):
    """Halting weights sum to 1 per position; the halt count is the first
    loop where the float32 running sum of p reaches the threshold (or the
    last loop), recomputed by brute force from the recorded p; and halting
    leaves the h trajectory unchanged (it only weights the output)."""
    scales = {"halt_w": 0.05, "halt_b": -0.8}
    cfg, W, P, e, h0 = _setup(name, scales=scales)
    n = cfg["n_loops"]
    on = O.recurrent_forward(cfg, P, e, h0, n, cfg["act_threshold"], record=True, stop_when_halted=False)
    off = O.recurrent_forward(cfg, P, e, h0, n, 0.0, record=True)
    wsum = np.sum(on["record"]["weight"], axis=0)
    np.testing.assert_allclose(wsum, 1.0, rtol=0, atol=1e-12)
    for a, b in zip(on["record"]["h"], off["record"]["h"]):
        np.testing.assert_array_equal(a, b)
    ps = np.array(on["record"]["p"])              # [loops, N]
    thr = np.float32(cfg["act_threshold"])
    counts = on["halt_counts"].ravel()
    for pos in range(ps.shape[1]):
        cum = np.float32(0)
        want = n
        for t in range(n):
            if np.float32(cum + np.float32(ps[t, pos])) >= thr:
                want = t + 1
                break
            cum = np.float32(cum + np.float32(ps[t, pos]))
        assert counts[pos] == want
    assert len(np.unique(counts)) > 1, "halting is not spread; the pin would be weak"
    # the output is the weighted sum of the recorded states
    ref = sum(w.reshape(e.shape[0], e.shape[1], 1) * h for w, h in zip(on["record"]["weight"], on["record"]["h"]))
    np.testing.assert_allclose(on["out"], ref, rtol=1e-13)


def test_halting_probability_matches_torch_and_closed_form():
    """[ZS §ACT]: the halting head is a linear map of h to one logit followed
    by a sigmoid, p = sigmoid(h . w + b).  Checked against torch's
    sigmoid(F.linear(h, w) + b) on random states, and against the closed
    form sigmoid(b) = 1 / (1 + exp(-b)) for states orthogonal to w (b = 0
    gives exactly 1/2), so a flipped sign, a dropped bias or a transposed
    product fails."""
    rng = np.random.default_rng(11)
    D = 48
    w = rng.standard_normal(D) * 0.3
    for b in (0.0, -1.7, 2.3):
        P = O.Params({"halt_w": w, "halt_b": np.array([b])})
        h = rng.standard_normal((37, D))
        got = O.halting_probability(P, h)
        ref = torch.sigmoid(F.linear(torch.from_numpy(h), torch.from_numpy(w)[None, :]) + b)[:, 0].numpy()
        np.testing.assert_allclose(got, ref, rtol=1e-14, atol=0)
        # states orthogonal to w: the logit is the bias alone
        hp = h - np.outer(h @ w / (w @ w), w)
        np.testing.assert_allclose(O.halting_probability(P, hp), 1.0 / (1.0 + math.exp(-b)), rtol=1e-13)
    P0 = O.Params({"halt_w": w, "halt_b": np.array([0.0])})
    assert O.halting_probability(P0, np.zeros((3, D))).tolist() == [0.5, 0.5, 0.5]
    # monotone in the logit and in (0, 1)
    ramp = np.outer(np.linspace(-30, 30, 61), w / (w @ w))
    p = O.halting_probability(P0, ramp)
    assert np.all(np.diff(p) > 0) and p[0] > 0 and p[-1] < 1


def test_bf16_decode_matches_torch_on_every_bit_pattern():
    """as_f64 reads uint16 arrays as bfloat16 bit patterns.  All 65536
    patterns decode to what torch's own bfloat16 gives (NaN patterns to NaN),
    so a wrong shift, byte order or sign bit fails."""
    u16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):      # NaN patterns widen with a warning
        got = O.as_f64(u16)
    ref = torch.from_numpy(u16.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))     # -0.0 included
    # a few values fixed by the format itself: 1.0 = 0x3F80, -2.0 = 0xC000,
    # the smallest subnormal 2^-133 = 0x0001, +inf = 0x7F80
    assert O.as_f64(np.array([0x3F80, 0xC000, 0x0001, 0x7F80], dtype=np.uint16)).tolist() == \
        [1.0, -2.0, 2.0 ** -133, math.inf]


# ---------------------------------------------------------------- whole block

def _torch_attn(cfg, W, a, start_pos=0, frozen=None, running=None):
    """Causal attention of one layer with torch routines (complex-number
    RoPE, SDPA): GQA or MLA by cfg["attn"]; returns o [B, heads, T, dv].
    ``frozen`` / ``running``: see _torch_one_loop."""
    T64 = _t64
    B, T, D = a.shape
    eps = cfg["norm_eps"]

    def rot(x, d):                                 # x [B, T, heads, d]
        inv = cfg["rope_theta"] ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
        ang = (start_pos + torch.arange(T, dtype=torch.float64))[:, None] * inv
        xc = torch.view_as_complex(x.reshape(*x.shape[:-1], d // 2, 2).contiguous())
        return torch.view_as_real(xc * torch.polar(torch.ones_like(ang), ang)[None, :, None]).reshape(x.shape)

    H = cfg["n_heads"]
    if cfg["attn"] == "gqa":
        G, dh = cfg["n_kv_heads"], cfg["head_dim"]
        q = rot(F.linear(a, T64(W["wq"])).reshape(B, T, H, dh), dh).transpose(1, 2)
        k = rot(F.linear(a, T64(W["wk"])).reshape(B, T, G, dh), dh).transpose(1, 2)
        v = F.linear(a, T64(W["wv"])).reshape(B, T, G, dh).transpose(1, 2)
        if frozen is not None:
            keep = torch.from_numpy(np.asarray(running))[:, None, :, None]
            k = torch.where(keep, k, torch.from_numpy(frozen["k"]))
            v = torch.where(keep, v, torch.from_numpy(frozen["v"]))
            frozen["k"], frozen["v"] = k.numpy().copy(), v.numpy().copy()
        o = F.scaled_dot_product_attention(q, k, v, is_causal=True, enable_gqa=True)
    else:
        kvl, rp, nope, vd = cfg["kv_lora_rank"], cfg["qk_rope_head_dim"], cfg["qk_nope_head_dim"], cfg["v_head_dim"]
        cq = F.rms_norm(F.linear(a, T64(W["wdq"])), (cfg["q_lora_rank"],), T64(W["gq"]), eps)
        q = F.linear(cq, T64(W["wuq"])).reshape(B, T, H, nope + rp)
        q = torch.cat([q[..., :nope], rot(q[..., nope:], rp)], -1)
        raw = F.linear(a, T64(W["wdkv"]))
        kr = rot(raw[..., kvl:].reshape(B, T, 1, rp), rp).expand(B, T, H, rp)
        kv = F.linear(F.rms_norm(raw[..., :kvl], (kvl,), T64(W["gkv"]), eps), T64(W["wukv"])).reshape(B, T, H, nope + vd)
        k = torch.cat([kv[..., :nope], kr], -1)
        v = kv[..., nope:]
        o = F.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), is_causal=True)
    return o


def _torch_one_loop(cfg, W, h, e, t, start_pos=0, frozen=None, running=None):
    """One loop written independently with torch CPU library routines:
    F.rms_norm, complex-number RoPE, SDPA with GQA, a dense masked MoE.

    With ``frozen`` (dict of k, v [B, G, T, dh] float64 arrays) and
    ``running`` (bool [B, T]): keys and values are computed for every
    position and then replaced by the frozen ones where a position is not
    running (a dense masked form of ACT compute skipping); the keys and
    values used are returned in ``frozen``."""
    T64 = _t64
    h, e = torch.from_numpy(h), torch.from_numpy(e)
    B, T, D = h.shape
    eps = cfg["norm_eps"]
    half = cfg["loop_dim"] // 2
    fr = cfg["loop_theta"] ** (-torch.arange(0, cfg["loop_dim"], 2, dtype=torch.float64) / cfg["loop_dim"])
    emb = torch.zeros(D, dtype=torch.float64)
    emb[:half], emb[half:2 * half] = torch.sin(t * fr), torch.cos(t * fr)
    c = F.rms_norm(h + emb + e, (D,), T64(W["g_rec"]), eps)
    a = F.rms_norm(c, (D,), T64(W["g_attn"]), eps)

    o = _torch_attn(cfg, W, a, start_pos, frozen, running)
    x1 = c + F.linear(o.transpose(1, 2).reshape(B, T, -1), T64(W["wo"]))
    f = F.rms_norm(x1, (D,), T64(W["g_ffn"]), eps).reshape(B * T, D)
    z = F.linear(f, T64(W["router_w"]))
    s = torch.softmax(z, -1)
    sel = torch.topk(z + T64(W["router_bias"]), cfg["top_k"], -1).indices
    g = torch.gather(s, 1, sel)
    g = g / g.sum(-1, keepdim=True)
    mask = torch.zeros_like(s).scatter_add_(1, sel, g)

    def ex(wg, wu, wd, x):
        return F.linear(F.silu(F.linear(x, T64(wg))) * F.linear(x, T64(wu)), T64(wd))
    y = sum(mask[:, x_:x_ + 1] * ex(W["w_gate"][x_], W["w_up"][x_], W["w_down"][x_], f) for x_ in range(cfg["n_experts"]))
    y = y + sum(ex(W["s_gate"][s_], W["s_up"][s_], W["s_down"][s_], f) for s_ in range(cfg["n_shared_experts"]))
    tau = x1.reshape(B * T, D) + y
    ti = min(t, cfg["max_loop_iters"] - 1)
    tau = tau + (F.linear(tau, T64(W["lora_down"])) * T64(W["lora_scale"])[ti]) @ T64(W["lora_B"])
    A = torch.exp(-torch.exp(torch.clamp(T64(W["log_dt"]) + T64(W["log_A"]), -20, 20)))
    return (A * h.reshape(B * T, D) + T64(W["B"]) * e.reshape(B * T, D) + tau).reshape(B, T, D).numpy()


BIG = {"lora_scale": 1.0, "lora_B": 0.3, "wo": 0.1, "w_down": 0.1, "s_down": 0.1}


@pytest.mark.parametrize("name", ["tiny_gqa", "tiny_mla", "small_f32", "small_bf16_k3"])
def test_single_loop_matches_independent_torch_block(name):
    """n_loops = 1 equals one application of the block, written independently
    with library routines (the single-loop special case).  Larger LoRA /
    output scales keep every term visible above the tolerance."""
    cfg, W, P, e, h0 = _setup(name, scales=BIG)
    e64 = e.astype(np.float64)
    h = e64 * 0.7 + 0.1
    got = O.recurrent_forward(cfg, P, e64, h, 1, 0.0)["out"]
    ref = _torch_one_loop(cfg, W, h, e64, 0)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11)
    # a later loop index exercises the loop embedding and LoRA clamp
    t = cfg["max_loop_iters"] + 1
    got5 = O.run_loop(cfg, P, h, e64, t)["h"].reshape(h.shape)
    np.testing.assert_allclose(got5, _torch_one_loop(cfg, W, h, e64, t), rtol=1e-10, atol=1e-11)


def test_n_loops_is_repeated_single_loop():
    cfg, W, P, e, h0 = _setup("tiny_gqa")
    e64 = e.astype(np.float64)
    h = e64.copy()
    for t in range(3):
        h = O.run_loop(cfg, P, h, e64, t)["h"].reshape(h.shape)
    np.testing.assert_array_equal(O.recurrent_forward(cfg, P, e64, e64, 3, 0.0)["out"], h)


@pytest.mark.parametrize("name", ["tiny_gqa", "tiny_mla"])
def test_decode_equals_last_row_of_prefill(name):
    """[ZS §RoPE & generation cache]: with the per-loop caches of a prefill of
    positions 0..P-1, a one-token step at start_pos P gives the row P of a
    prefill of 0..P, in every loop (attention is causal in every loop)."""
    cfg, W, P, e, h0 = _setup(name, scales=BIG)
    B, T = e.shape[:2]
    n = 3
    full = O.recurrent_forward(cfg, P, e, h0, n, 0.0)["out"]
    cache = O.new_cache(cfg, B, T, n)
    O.recurrent_forward(cfg, P, e[:, :T - 1], h0[:, :T - 1], n, 0.0, start_pos=0, cache=cache)
    step = O.recurrent_forward(cfg, P, e[:, T - 1:], h0[:, T - 1:], n, 0.0, start_pos=T - 1, cache=cache)["out"]
    np.testing.assert_allclose(step[:, 0], full[:, T - 1], rtol=1e-11, atol=1e-12)


def test_row_subset_equals_full_loop():
    """The sampled-row mode used at full sizes returns exactly the rows of
    the all-rows pass (attention still reads every earlier position)."""
    cfg, W, P, e, h0 = _setup("small_f32")
    e64 = e.astype(np.float64)
    full = O.run_loop(cfg, P, e64, e64, 2)
    rows = [(0, 0), (0, 149), (1, 77), (1, 3)]
    part = O.run_loop(cfg, P, e64, e64, 2, rows=rows)
    T = e.shape[1]
    idx = [b * T + i for b, i in rows]
    np.testing.assert_allclose(part["h"], full["h"][idx], rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(part["sel"], full["sel"][idx])


# ---------------------------------------------------------------- ACT compute skipping

def test_act_skip_loop_matches_dense_masked_torch():
    """One loop of the compute-skipping mode (only the running positions are
    computed, halted positions keep their keys and values) equals a dense
    masked form written with torch: K/V for every position, replaced by the
    frozen ones where a position is not running, attention and the rest of
    the block for every position, read on the running rows."""
    cfg, W, P, e, h0 = _setup("small_f32", scales=BIG)
    B, T, D = e.shape
    G, dh = cfg["n_kv_heads"], cfg["head_dim"]
    rng = np.random.default_rng(21)
    e64 = e.astype(np.float64)
    h = e64 * 0.6 + 0.05 * rng.standard_normal(e.shape)
    running = rng.random((B, T)) < 0.55
    running[0, 0] = False
    frozen = dict(k=rng.standard_normal((B, G, T, dh)), v=rng.standard_normal((B, G, T, dh)))
    kv = dict(k=frozen["k"].copy(), v=frozen["v"].copy())
    rows = [(b, i) for b in range(B) for i in range(T) if running[b, i]]
    t = 2
    got = O.run_loop(cfg, P, h, e64, t, rows=rows, kv_state=kv)["h"]
    tf = dict(frozen)
    ref = _torch_one_loop(cfg, W, h, e64, t, frozen=tf, running=running)
    bi = np.array(rows)
    np.testing.assert_allclose(got, ref[bi[:, 0], bi[:, 1]], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(kv["k"], tf["k"], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(kv["v"], tf["v"], rtol=1e-12, atol=1e-13)


def test_act_skip_equals_full_path_when_nothing_halts_early():
    """With the halting head far negative no position halts before the last
    loop, so nothing is ever skipped and the mode reduces to the plain path."""
    cfg, W, P, e, h0 = _setup("small_f32", scales={"halt_w": 0.0, "halt_b": -30.0})
    n = cfg["n_loops"]
    a = O.recurrent_forward(cfg, P, e, h0, n, cfg["act_threshold"])
    b = O.recurrent_forward_act_skip(cfg, P, e, h0, n, cfg["act_threshold"])
    assert np.all(a["halt_counts"] == n)
    np.testing.assert_array_equal(a["halt_counts"], b["halt_counts"])
    np.testing.assert_allclose(b["out"], a["out"], rtol=1e-11, atol=1e-12)


def test_act_skip_equals_full_path_on_single_token_sequences():
    """Sequences of one token attend only to themselves, so skipping a halted
    position changes nothing it returns: output and halt counts equal the
    plain path even with halting spread over the loops."""
    cfg, W, P, e, h0 = _setup("tiny_gqa", scales={"halt_w": 0.05, "halt_b": -0.8}, batch=12, seq=1)
    n = cfg["n_loops"]
    a = O.recurrent_forward(cfg, P, e, h0, n, cfg["act_threshold"])
    b = O.recurrent_forward_act_skip(cfg, P, e, h0, n, cfg["act_threshold"])
    assert len(np.unique(a["halt_counts"])) > 1
    np.testing.assert_array_equal(a["halt_counts"], b["halt_counts"])
    np.testing.assert_allclose(b["out"], a["out"], rtol=1e-11, atol=1e-12)


def test_act_skip_weights_sum_to_one_and_halted_rows_stop():
    """In the skipping mode too the ACT weights of a position sum to 1, its
    halt count is the first loop where the float32 running sum of its p
    reaches the threshold, and a halted position is never computed again."""
    cfg, W, P, e, h0 = _setup("small_f32", scales={"halt_w": 0.05, "halt_b": -0.8})
    n = cfg["n_loops"]
    r = O.recurrent_forward_act_skip(cfg, P, e, h0, n, cfg["act_threshold"], record=True)
    N = e.shape[0] * e.shape[1]
    counts = r["halt_counts"].ravel()
    assert len(np.unique(counts)) > 1
    ps = {}
    for t, (idx, p) in enumerate(r["record"]["p"]):
        assert np.all(counts[idx] > t)                 # only running positions run
        for m, nn in enumerate(idx):
            ps.setdefault(int(nn), []).append(p[m])
    thr = np.float32(cfg["act_threshold"])
    for nn in range(N):
        seq = ps[nn]
        assert len(seq) == counts[nn]
        cum = np.float32(0)
        want = n
        for t, pv in enumerate(seq):
            if np.float32(cum + np.float32(pv)) >= thr:
                want = t + 1
                break
            cum = np.float32(cum + np.float32(pv))
        assert counts[nn] == want
        wsum = sum(seq[:-1]) + max(1.0 - sum(seq[:-1]), 0.0)
        assert abs(wsum - 1.0) < 1e-12


# ---------------------------------------------------------------- the whole model

def _layer_weights(W, prefix):
    return {k[len(prefix):]: v for k, v in W.items() if k.startswith(prefix)}


def _torch_dense_layer(cfg, LW, x):
    """A prelude / coda layer with torch routines: x1 = x + Attn(rms_norm(x)),
    out = x1 + silu(f W1^T) * (f W3^T) W2^T with f = rms_norm(x1)."""
    B, T, D = x.shape
    eps = cfg["norm_eps"]
    a = F.rms_norm(x, (D,), _t64(LW["attn_norm"]), eps)
    o = _torch_attn(cfg, LW, a)
    x1 = x + F.linear(o.transpose(1, 2).reshape(B, T, -1), _t64(LW["wo"]))
    f = F.rms_norm(x1, (D,), _t64(LW["ffn_norm"]), eps)
    return x1 + F.linear(F.silu(F.linear(f, _t64(LW["w1"]))) * F.linear(f, _t64(LW["w3"])), _t64(LW["w2"]))


@pytest.mark.parametrize("name", ["tiny_model_gqa", "tiny_model_mla"])
def test_dense_layer_matches_torch(name):
    """[ZS §MoE]: prelude and coda layers are the pre-norm block with a dense
    SwiGLU feed-forward of width dim * 4 // 3 (341 at dim 256)."""
    cfg = configs.get(name)
    W = generate.make_weights(cfg, scales={"prelude_0.wo": 0.1, "prelude_0.w2": 0.1})
    P = O.Params(W)
    assert W["prelude_0.w1"].shape == (O.dense_hidden(cfg), cfg["dim"]) == (341, 256)
    x = np.random.default_rng(31).standard_normal((cfg["batch"], cfg["seq"], cfg["dim"]))
    got = O.dense_layer(cfg, O.LayerParams(P, "prelude_0."), x)
    ref = _torch_dense_layer(cfg, _layer_weights(W, "prelude_0."), torch.from_numpy(x)).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("name", ["tiny_model_gqa", "tiny_model_mla"])
def test_model_forward_wiring(name):
    """[ZS §Core Structure]: embed, prelude, e = x as both anchor and initial
    state of the recurrent stage, coda, final norm, head -- written here with
    torch for every part but the recurrent stage (pinned on its own above).
    The usage example prints logits of shape (2, 16, vocab 1000)."""
    cfg = configs.get(name)
    W = generate.make_weights(cfg, scales={"prelude_0.wo": 0.1, "coda_0.wo": 0.1})
    P = O.Params(W)
    ids = generate.make_ids(cfg)
    logits, r = O.model_forward(cfg, P, ids, cfg["n_loops"], cfg["act_threshold"])
    assert logits.shape == (2, 16, 1000)
    x = _t64(W["embed"])[torch.from_numpy(ids.astype(np.int64))]
    x = _torch_dense_layer(cfg, _layer_weights(W, "prelude_0."), x)
    rr = O.recurrent_forward(cfg, P, x.numpy(), x.numpy(), cfg["n_loops"], cfg["act_threshold"])
    y = _torch_dense_layer(cfg, _layer_weights(W, "coda_0."), torch.from_numpy(rr["out"]))
    y = F.rms_norm(y, (cfg["dim"],), _t64(W["final_norm"]), cfg["norm_eps"])
    ref = F.linear(y, _t64(W["head"])).numpy()
    np.testing.assert_array_equal(r["halt_counts"], rr["halt_counts"])
    np.testing.assert_allclose(logits, ref, rtol=1e-9, atol=1e-11)


def test_argmax_lowest_index_brute_force():
    rng = np.random.default_rng(32)
    v = rng.integers(0, 4, size=(50, 9)).astype(np.float64)      # many exact ties
    idx, margin = O.argmax_lowest(v)
    for r in range(50):
        best = max(v[r])
        assert idx[r] == min(j for j in range(9) if v[r, j] == best)
        others = sorted(v[r], reverse=True)
        assert margin[r] == others[0] - others[1]


@pytest.mark.parametrize("name", ["tiny_model_gqa", "tiny_model_mla"])
def test_generate_with_caches_equals_full_recompute(name):
    """[ZS §RoPE & generation cache]: greedy generation that feeds the prompt
    once and then one token per step at start_pos = prompt_len + step - 1
    against the per-layer caches gives the tokens of recomputing the whole
    growing sequence every step (no cache).  The usage example generates 8
    tokens with 8 loops: output shape (2, 24)."""
    cfg = configs.get(name, seq=6)
    W = generate.make_weights(cfg)
    P = O.Params(W)
    ids = generate.make_ids(cfg)
    n_new, L = 4, 8
    out = O.generate(cfg, P, ids, n_new, L, cfg["act_threshold"])
    assert out.shape == (2, 6 + n_new)
    np.testing.assert_array_equal(out[:, :6], ids)
    seq = ids.copy()
    for _ in range(n_new):
        logits, _ = O.model_forward(cfg, P, seq, L, cfg["act_threshold"])
        nxt, margin = O.argmax_lowest(logits[:, -1])
        assert np.all(margin > 1e-9)
        seq = np.concatenate([seq, nxt[:, None]], axis=1)
    np.testing.assert_array_equal(out, seq)
    full = O.generate(configs.get(name), P, generate.make_ids(configs.get(name)), 8, 8, 0.99)
    assert full.shape == (2, 24)
