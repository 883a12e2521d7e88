"""AdamW on the GPU (rdt_adamw_init / rdt_adamw_step) against the oracle's
AdamW rule (oracle/rdt_backward.adamw_step, pinned against torch.optim.AdamW
and the first step's closed form).

Protocol: seeded gradients (per-tensor scales from 1e-3 to 10, about 5 % of
entries exactly zero) drive three steps; the GPU's masters and moments are
compared with the oracle's float64 run from the same start, and the
handle's weights must be the GPU's own masters rounded (bf16, nearest even:
the rounding decision is taken on the GPU's fp32 value on both sides) or
copied (fp32 vectors) -- bit for bit.  A fresh handle built from the updated
weights must then give the same A table and the same forward output, bit
for bit, which checks that the step recomputed A.

Tolerance: the GPU runs the update in fp32.  Each of m, v and the update
term takes a handful of roundings (relative 2^-24 each), so one step's
master differs from the float64 step by a few 2^-24 of |p| plus a few 2^-24
of lr |u| (|u| <= about 1 / sqrt(1 - beta2) + weight_decay |p|); three
steps add those.  The bound used is 2^-20 (|p| + 10 lr) on the masters and
2^-20 of the magnitudes that form m and v.

Pages: [ZS] "OpenMythos 분석: …의 계산 모델링" (zero.shotlearni.ng),
§Tokenizer & training script (the training script uses AdamW).
"""

import numpy as np
import pytest

from oracle import rdt_backward as OB
from oracle import rdt_oracle as O
from workloads import configs, generate

from gpu_support import to_np

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-2, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def _grads(layout, total, rng):
    g = np.zeros(total, dtype=np.float32)
    for name, (o, m) in layout.items():
        if name == "router_bias":
            continue
        x = rng.standard_normal(m) * 10 ** rng.uniform(-3, 1)
        x[rng.random(m) < 0.05] = 0.0
        g[o:o + m] = x
    return g


def _state(state, total):
    s = to_np(state)
    return s[:total], s[total:2 * total], s[2 * total:3 * total]


@pytest.mark.parametrize("name", ["small_bf16", "small_bf16_k3"])
def test_adamw_steps_match_oracle(name):
    import torch
    from recurrent_depth_moe_amd import binding
    cfg = configs.get(name)
    W = generate.make_weights(cfg)
    print(f"[adamw] {name} D={cfg['dim']} E={cfg['n_experts']} S={cfg['n_shared_experts']}", flush=True)
    blk = binding.Block(cfg, binding.weights_to_device(W))
    layout, total = blk.grad_layout(), blk.grad_numel()
    state = blk.adamw_init()
    torch.cuda.synchronize()
    master, m_, v_ = _state(state, total)
    ref = {}
    for n, (o, m) in layout.items():
        w0 = O.as_f64(W[n]).reshape(-1)
        np.testing.assert_array_equal(master[o:o + m], w0.astype(np.float32), err_msg=n)
        assert not m_[o:o + m].any() and not v_[o:o + m].any(), n
        ref[n] = (w0, np.zeros(m), np.zeros(m))
    rng = np.random.default_rng(21)
    for step in (1, 2, 3):
        g = _grads(layout, total, rng)
        blk.adamw_step(torch.from_numpy(g).cuda(), state, step, **HP)
        for n, (o, m) in layout.items():
            if n != "router_bias":
                p, mo, vo = ref[n]
                ref[n] = OB.adamw_step(p, g[o:o + m], mo, vo, step, **HP)
    torch.cuda.synchronize()
    master, m_, v_ = _state(state, total)
    lr = HP["lr"]
    for n, (o, m) in layout.items():
        p_ref, m_ref, v_ref = ref[n]
        got = master[o:o + m].astype(np.float64)
        if n == "router_bias":
            np.testing.assert_array_equal(got, p_ref)
        else:
            err = np.abs(got - p_ref)
            bound = 2.0 ** -20 * (np.abs(p_ref) + 10 * lr)
            assert np.all(err <= bound), (n, float((err / bound).max()))
            np.testing.assert_allclose(m_[o:o + m], m_ref, rtol=0, atol=2.0 ** -20 * np.abs(m_ref).max() + 1e-30,
                                       err_msg=n)
            np.testing.assert_allclose(v_[o:o + m], v_ref, rtol=0, atol=2.0 ** -20 * np.abs(v_ref).max() + 1e-30,
                                       err_msg=n)
        w = blk.get_weight(n)
        if w.dtype == np.uint16:
            np.testing.assert_array_equal(w, OB.round_bf16(master[o:o + m]), err_msg=n)
        else:
            np.testing.assert_array_equal(w, master[o:o + m], err_msg=n)
    # the updated handle against a fresh handle built from its weights
    W2 = {n: blk.get_weight(n).reshape(np.shape(W[n])) for n in layout}
    for n in W:
        W2.setdefault(n, W[n])
    fresh = binding.Block(cfg, binding.weights_to_device(W2))
    np.testing.assert_array_equal(blk.get_A().numpy(), fresh.get_A().numpy())
    assert not np.array_equal(blk.get_A().numpy(), O.lti_A(O.Params(W)).astype(np.float32))
    e, h0 = generate.make_inputs(cfg)
    e_d = torch.from_numpy(np.ascontiguousarray(e)).cuda()
    h_d = torch.from_numpy(np.ascontiguousarray(h0)).cuda()
    out1, hc1 = blk.forward(e_d, h_d, cfg["n_loops"], cfg["act_threshold"])
    out2, hc2 = fresh.forward(e_d, h_d, cfg["n_loops"], cfg["act_threshold"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(out1), to_np(out2))
    np.testing.assert_array_equal(to_np(hc1), to_np(hc2))


def test_adamw_rejects_bad_arguments():
    import torch
    from recurrent_depth_moe_amd import binding
    cfg = configs.get("small_bf16")
    blk = binding.Block(cfg, binding.weights_to_device(generate.make_weights(cfg)))
    state = blk.adamw_init()
    g = torch.zeros(blk.grad_numel(), dtype=torch.float32, device="cuda")
    for kw in (dict(step=0), dict(lr=-1.0), dict(beta1=1.0), dict(beta2=-0.1), dict(eps=0.0),
               dict(weight_decay=float("nan"))):
        args = dict(step=1, lr=1e-3)
        args.update(kw)
        with pytest.raises(binding.RdtError, match="INVALID_ARG"):
            blk.adamw_step(g, state, **args)
    with pytest.raises(binding.RdtError, match="WORKSPACE_TOO_SMALL"):
        blk.adamw_step(g[:-64], state, 1, 1e-3)
    with pytest.raises(binding.RdtError, match="WORKSPACE_TOO_SMALL"):
        blk.adamw_step(g, state[:-1], 1, 1e-3)
