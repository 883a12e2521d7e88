"""Pins of the gradient oracle (oracle/rdt_backward.py).

* Its forward, with the decisions the numpy oracle took, reproduces the numpy
  oracle's output (so the PyTorch re-statement drops or flips no term).
* Its gradients agree with central finite differences of that forward along
  random directions, for every trained tensor and for e and h0 (so nothing in
  it blocks or bends autograd).
* With the Transformer term zeroed the stage is the pure LTI recurrence, whose
  gradients have a closed form ([RC §동적 시스템 관점]).
* The router-bias balancing rule on a hand-worked example.

Pages: [ZS] "OpenMythos 분석: …의 계산 모델링" (zero.shotlearni.ng);
[RC] "OpenMythos" (runchr.com).
"""

import numpy as np
import pytest
import torch

from oracle import rdt_backward as OB
from oracle import rdt_oracle as O
from workloads import configs, generate


def _setup(name, scales=None, **over):
    cfg = configs.get(name, **over)
    W = generate.make_weights(cfg, scales=scales)
    e, h0 = generate.make_inputs(cfg)
    return cfg, W, e, h0


def _decisions(cfg, P, e, h0):
    r = O.recurrent_forward(cfg, P, e, h0, cfg["n_loops"], cfg["act_threshold"], record=True)
    return r, np.stack(r["record"]["sel"]), r["halt_counts"]


@pytest.mark.parametrize("name", ["tiny_gqa", "small_bf16_k3"])
def test_fixed_forward_equals_numpy_oracle(name):
    cfg, W, e, h0 = _setup(name)
    P = O.Params(W)
    r, sel, hc = _decisions(cfg, P, e, h0)
    out, _ = OB.forward_fixed(cfg, P, e, h0, cfg["n_loops"], cfg["act_threshold"], sel, hc)
    ref = r["out"]
    np.testing.assert_allclose(out.detach().numpy(), ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_gradients_match_central_differences():
    """Directional derivatives <grad, v> against (L(x + eps v) - L(x - eps v))
    / (2 eps) in float64, one random direction per tensor, ACT on (positions
    halting at loop 3 or 4 of 4, so the remainder weights and the positions
    that keep running after others halted are both exercised)."""
    cfg, W, e, h0 = _setup("tiny_gqa", scales={"halt_w": 0.1}, seq=8, halt_b=-3.0)
    P = O.Params(W)
    _, sel, hc = _decisions(cfg, P, e, h0)
    assert len(set(hc.reshape(-1).tolist())) > 1, "want several halting loops"
    L, thr = cfg["n_loops"], cfg["act_threshold"]
    rng = np.random.default_rng(7)
    dy = rng.standard_normal(e.shape)
    g = OB.recurrent_grad(cfg, P, e, h0, L, thr, sel, hc, dy)
    dy_t = torch.from_numpy(dy)
    base = {n: torch.from_numpy(np.asarray(P[n], dtype=np.float64)) for n in OB.GRAD_NAMES}
    e64, h64 = torch.from_numpy(e.astype(np.float64)), torch.from_numpy(h0.astype(np.float64))

    def loss(W_, e_, h_):
        out, _ = OB.forward_fixed(cfg, P, e_, h_, L, thr, sel, hc, W=W_)
        return float((out * dy_t).sum())

    eps = 1e-6
    for name in list(OB.GRAD_NAMES) + ["e", "h0"]:
        ref_x = e64 if name == "e" else h64 if name == "h0" else base[name]
        v = torch.from_numpy(rng.standard_normal(tuple(ref_x.shape)))
        if name in ("g_rec", "g_attn", "g_ffn"):
            v = v * 0.1
        vals = []
        for sgn in (1.0, -1.0):
            W_ = dict(base)
            e_, h_ = e64, h64
            if name == "e":
                e_ = e64 + sgn * eps * v
            elif name == "h0":
                h_ = h64 + sgn * eps * v
            else:
                W_[name] = base[name] + sgn * eps * v
            vals.append(loss(W_, e_, h_))
        fd = (vals[0] - vals[1]) / (2 * eps)
        an = float((torch.from_numpy(g[name]) * v).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_closed_form_gradient_of_pure_lti_recurrence():
    """g_rec = 0 makes the block input 0, so attention, experts and LoRA
    return 0 and (ACT off) out = A^L h0 + (1 - A^L) / (1 - A) B e.  Then
    d/dh0 = A^L dy, d/de = (1 - A^L)/(1 - A) B dy, d/dB = sum dy (1 - A^L)/(1 - A) e,
    and d/dlog_A_i = dA_i * A_i * (-exp(log_dt + log_A_i)) with
    dA = sum dy (L A^(L-1) h0 + B e sum_{j<L} j A^(j-1))."""
    cfg, W, e, h0 = _setup("tiny_gqa", act_threshold=0.0)
    W = dict(W)
    W["g_rec"] = np.zeros_like(W["g_rec"])
    P = O.Params(W)
    L = 3
    h0 = h0 * 0.5 + 0.3
    N = e.shape[0] * e.shape[1]
    sel = np.zeros((L, N, cfg["top_k"]), dtype=np.int64)
    sel[..., 1] = 1
    rng = np.random.default_rng(3)
    dy = rng.standard_normal(e.shape)
    g = OB.recurrent_grad(cfg, P, e, h0, L, 0.0, sel, None, dy)
    A = O.lti_A(P)
    Bv = np.asarray(W["B"], dtype=np.float64)
    e64, h64 = e.astype(np.float64), h0.astype(np.float64)
    geo = (1 - A ** L) / (1 - A)
    np.testing.assert_allclose(g["h0"], A ** L * dy, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g["e"], geo * Bv * dy, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(g["B"], (dy * geo * e64).sum((0, 1)), rtol=1e-10, atol=1e-12)
    dgeo = sum(j * A ** (j - 1) for j in range(1, L))
    dA = (dy * (L * A ** (L - 1) * h64 + Bv * e64 * dgeo)).sum((0, 1))
    s = np.asarray(W["log_dt"], dtype=np.float64)[0] + np.asarray(W["log_A"], dtype=np.float64)
    np.testing.assert_allclose(g["log_A"], dA * A * -np.exp(s), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["log_dt"][0], np.sum(dA * A * -np.exp(s)), rtol=1e-10)
    for name in ("wq", "wo", "w_gate", "router_w", "lora_B", "halt_w"):
        assert np.all(g[name] == 0), name


def test_router_bias_balancing_rule():
    """Loads [5, 3, 0, 4] (mean 3): the over-loaded experts 0 and 3 go down by
    gamma, the idle expert 2 goes up, expert 1 at the mean stays."""
    bias = np.array([0.5, -0.25, 0.0, 1.0], dtype=np.float32)
    new = OB.router_bias_update(bias, [5, 3, 0, 4], 0.125)
    np.testing.assert_array_equal(new, np.array([0.375, -0.25, 0.125, 0.875], dtype=np.float32))
    assert OB.expert_load(np.array([[[0, 1], [1, 3]], [[3, 3], [0, 1]]]), 5).tolist() == [2, 3, 0, 3, 0]


def test_adamw_matches_torch_over_several_steps():
    """AdamW against torch.optim.AdamW (float64), three steps with weight
    decay on random parameters and gradients."""
    rng = np.random.default_rng(11)
    p0 = rng.standard_normal((7, 5))
    grads = [rng.standard_normal((7, 5)) * s for s in (1.0, 0.1, 3.0)]
    hp = dict(lr=1e-2, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([tp], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"])
    p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    for step, g in enumerate(grads, start=1):
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
        p, m, v = OB.adamw_step(p, g, m, v, step, **hp)
        np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-15)


def test_adamw_first_step_closed_form():
    """Step 1: m_hat = g and v_hat = g^2, so the update is lr g / (|g| + eps)
    plus lr * weight_decay * p."""
    g = np.array([2.0, -0.5, 1e-3, 0.0])
    p = np.array([1.0, -2.0, 0.5, 3.0])
    new, m, v = OB.adamw_step(p, g, 0 * g, 0 * g, 1, 0.1, 0.9, 0.999, 1e-8, 0.01)
    np.testing.assert_allclose(new, p - 0.1 * (g / (np.abs(g) + 1e-8) + 0.01 * p), rtol=1e-12)
    np.testing.assert_allclose(m, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v, 0.001 * g * g, rtol=1e-12)


def test_bf16_rounding_nearest_even():
    """round_bf16 against torch's own float32 -> bfloat16 conversion on
    random values, exact halfway cases (ties to even) and specials."""
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10 ** rng.uniform(-5, 5, 10000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0, np.inf, -np.inf],
                                 dtype=np.float32)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(OB.round_bf16(x), ref)
