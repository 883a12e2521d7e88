"""Backward pass of the recurrent stage on the GPU (rdt_train_forward +
rdt_train_backward) against the gradient oracle (oracle/rdt_backward.py),
and the router-bias balancing step against its rule.

Protocol: the GPU forward records its expert choices and halt counts; the
numpy oracle replays the forward, taking a GPU choice only within rounding
of a tie (no other disagreement allowed); the gradient oracle then
differentiates the stage with those decisions held fixed.  Every gradient
(each trained tensor, e and h0) is compared by ||g - ref|| / ||ref||.

Tolerance (bf16 operands, fp32 accumulation): every matrix product of the
backward rounds both operands to bf16 (relative 2^-9), and a gradient
passes through a handful of such products per loop plus the forward's own
bf16 roundings that it differentiates; independent roundings add in
quadrature, so a norm-relative error of a few 1e-3 per loop, growing like
the square root of the loops, is expected.  The bound is
2e-2 * sqrt(loops) (the free-running forward's 3e-2 * sqrt(loops) scaled by
the ratio of norm-wise to max-wise error), checked on every tensor; the
scalar d log_dt, a sum of the D log_A gradients, against the sum of their
magnitudes.

Pages: [ZS] "OpenMythos 분석: …의 계산 모델링" (zero.shotlearni.ng),
§Recurrent Block, §ACT, §MoE.
"""

import numpy as np
import pytest

from oracle import rdt_backward as OB
from oracle import rdt_oracle as O
from workloads import configs, generate

from gpu_support import EPS_HALT, EPS_ROUTE, to_np

pytestmark = pytest.mark.gpu

SPREAD = {"halt_w": 0.05, "halt_b": -0.8}
# O(1) LoRA and output scales, so the LoRA and residual terms of every
# input gradient are far above the tolerance
BIG = {"lora_scale": 1.0, "lora_B": 0.3, "wo": 0.1, "w_down": 0.1, "s_down": 0.1, "halt_w": 0.05, "halt_b": -0.8}


def _grad_tol(n_loops):
    return 2e-2 * float(np.sqrt(n_loops))


def _run(cfg, W, e, h0, seed=5):
    import torch
    from recurrent_depth_moe_amd import binding
    B, T, D = e.shape
    N, L, k, thr = B * T, cfg["n_loops"], cfg["top_k"], cfg["act_threshold"]
    print(f"[train] {cfg['name']} B={B} T={T} D={D} loops={L} thr={thr}", flush=True)
    blk = binding.Block(cfg, binding.weights_to_device(W))
    cap_sel = torch.full((L, N, k), -1, dtype=torch.int32, device="cuda")
    blk.set_capture(None, cap_sel, None, L)
    e_d = torch.from_numpy(np.ascontiguousarray(e)).cuda()
    h_d = torch.from_numpy(np.ascontiguousarray(h0)).cuda()
    tape = blk.new_tape(B, T, L)
    out, halt = blk.train_forward(e_d, h_d, L, thr, tape)
    dy = np.random.default_rng(seed).standard_normal(e.shape).astype(np.float32)
    dy_d = torch.from_numpy(dy).cuda()
    ws = torch.empty(blk.train_workspace_bytes(B, T, L), dtype=torch.uint8, device="cuda")
    # NaN everywhere first: every tensor of the layout must be written
    grad0 = torch.full((blk.grad_numel(),), float("nan"), dtype=torch.float32, device="cuda")
    grad, de, dh0, load = blk.train_backward(e_d, h_d, L, thr, tape, halt, dy_d, ws, grad=grad0)
    torch.cuda.synchronize()
    layout = blk.grad_layout()
    g = to_np(grad)
    for n, (o, m) in layout.items():
        assert np.all(np.isfinite(g[o:o + m])), f"gradient of {n} not fully written"
    res = dict(out=to_np(out), halt=to_np(halt), sel=to_np(cap_sel), dy=dy, de=to_np(de), dh0=to_np(dh0),
               load=to_np(load), blk=blk)
    res["grads"] = {n: g[o:o + m] for n, (o, m) in layout.items()}
    return res


def _check(cfg, W, e, h0):
    g = _run(cfg, W, e, h0)
    L, thr, dt = cfg["n_loops"], cfg["act_threshold"], cfg["dtype"]
    P = O.Params(W)
    adopt = O.Adoption(sel=g["sel"], halt_counts=g["halt"], eps_route=EPS_ROUTE[dt], eps_halt=EPS_HALT[dt])
    ref_f = O.recurrent_forward(cfg, P, e, h0, L, thr, adopt=adopt, record=True)
    print(f"  adopted route={adopt.route_adopted} halt={adopt.halt_adopted}; "
          f"disagree route={adopt.route_disagree} halt={adopt.halt_disagree}", flush=True)
    assert adopt.route_disagree == 0 and adopt.halt_disagree == 0
    np.testing.assert_array_equal(ref_f["halt_counts"], g["halt"])
    loops = ref_f["loops_run"]
    sel = g["sel"][:loops]
    ref = OB.recurrent_grad(cfg, P, e, h0, L, thr, sel, g["halt"], g["dy"])
    # expert load: (position, slot) assignments summed over the loops run
    np.testing.assert_array_equal(g["load"], OB.expert_load(sel, cfg["n_experts"]))
    tol = _grad_tol(loops)
    worst = 0.0
    names = [n for n in OB.GRAD_NAMES if n in ref] + ["e", "h0"]
    if cfg["top_k"] == 1:
        # every gate is 1: the router's gradient is 0 up to the oracle's
        # rounding (checked exactly by the caller)
        names.remove("router_w")
    for name in names:
        got = g["de"] if name == "e" else g["dh0"] if name == "h0" else g["grads"][name]
        want = np.asarray(ref[name], dtype=np.float64).reshape(-1)
        got = np.asarray(got, dtype=np.float64).reshape(-1)
        nrm = np.linalg.norm(want)
        if name == "log_dt":
            # the sum of the log_A gradients: with each term off by a
            # relative e, the sum is off by at most e * sum |terms|
            nrm = np.abs(np.asarray(ref["log_A"], dtype=np.float64)).sum()
        err = np.linalg.norm(got - want) / nrm if nrm > 0 else np.linalg.norm(got)
        print(f"  {name:11s} |ref| {nrm:.3e}  rel err {err:.3e}", flush=True)
        worst = max(worst, err)
        assert err <= tol, (name, err, tol)
    assert np.all(g["grads"]["router_bias"] == 0)
    print(f"  worst {worst:.3e} (tol {tol:.3g})", flush=True)
    return g


@pytest.mark.parametrize("name, scales, over", [
    ("small_bf16", SPREAD, dict(n_loops=4)),
    ("small_bf16_k3", None, dict()),
    ("small_bf16", BIG, dict(n_loops=3)),
    ("small_bf16_strip", None, dict()),
    ("small_bf16", None, dict(n_shared_experts=0, top_k=1, n_loops=2)),
    ("small_bf16", SPREAD, dict(n_loops=1, seq=130)),
], ids=["small_bf16_act", "small_bf16_k3", "large_terms", "strip_540_tokens", "top1_no_shared",
        "one_loop_act"])
def test_backward_matches_gradient_oracle(name, scales, over):
    """small_bf16: ACT on with halting spread over the loops (remainder
    weights, positions running on after others halted), 200 tokens (ragged
    attention tiles); small_bf16_k3: ACT off, top-3 of 12 experts, two
    shared experts, 77 tokens; large_terms: O(1) LoRA and projections;
    strip_540_tokens: dim 768, 1080 rows (several 128-row attention and
    weight-gradient tiles, ~270 routed rows per expert); top1_no_shared: one
    routed expert per position (every gate is 1, so the router's gradient
    is 0) and no shared expert; one_loop_act: a single loop with ACT on
    (every position halts there with weight 1), 130 tokens (a 128-key tile
    plus two)."""
    cfg = configs.get(name, **over)
    W = generate.make_weights(cfg, scales=scales)
    e, h0 = generate.make_inputs(cfg)
    g = _check(cfg, W, e, h0)
    if scales is SPREAD and cfg["n_loops"] > 1:
        assert len(np.unique(g["halt"])) > 1   # halting spread over the loops, as intended
    if cfg["top_k"] == 1:
        assert np.all(g["grads"]["router_w"] == 0)


def test_backward_deterministic_bitwise():
    """Two training steps' backward passes on the same inputs (fresh handles,
    so the grouped products claim their tiles in whatever order the blocks
    arrive) give bitwise equal gradients, e / h0 gradients and expert loads:
    every sum runs in a fixed order, with no floating-point atomics."""
    cfg = configs.get("small_bf16")
    W = generate.make_weights(cfg)
    e, h0 = generate.make_inputs(cfg)
    a = _run(cfg, W, e, h0)
    b = _run(cfg, W, e, h0)
    for name in a["grads"]:
        assert np.array_equal(a["grads"][name].view(np.uint32), b["grads"][name].view(np.uint32)), name
    for key in ("de", "dh0", "out"):
        assert np.array_equal(a[key].view(np.uint32), b[key].view(np.uint32)), key
    np.testing.assert_array_equal(a["load"], b["load"])
    np.testing.assert_array_equal(a["halt"], b["halt"])


def test_router_bias_balancing_step():
    """After a backward pass, the handle's router bias moves by gamma
    towards balance (rule in oracle/rdt_backward.py), bit for bit."""
    cfg = configs.get("small_bf16_k3")
    W = generate.make_weights(cfg)
    e, h0 = generate.make_inputs(cfg)
    g = _run(cfg, W, e, h0)
    import torch
    load = torch.from_numpy(g["load"]).cuda()
    blk = g["blk"]
    before = blk.get_router_bias().numpy()
    blk.router_bias_update(load, 0.03125)
    torch.cuda.synchronize()
    after = blk.get_router_bias().numpy()
    np.testing.assert_array_equal(after, OB.router_bias_update(before, g["load"], 0.03125))
    assert np.any(after != before)


@pytest.mark.timeout(900)
def test_backward_full_size_mythos_1b_one_loop():
    """mythos_1b at full size (dim 2048, 16 heads, 64 experts of 2048,
    4096 tokens), one loop: every kernel at the shapes the training bench
    runs (many tiles, real routing skew, 32 attention tiles per head)."""
    cfg = configs.get("mythos_1b", n_loops=1)
    W = generate.make_weights(cfg)
    e, h0 = generate.make_inputs(cfg)
    _check(cfg, W, e, h0)
