"""ACT compute skipping on the GPU (rdt_recurrent_forward_act_skip) against
the oracle's skipping mode: a halted position leaves the batch, its state
and its keys/values freeze ([GN §6] continuous depth-wise batching; the
frozen-K/V reading is stated in the oracle).

Same protocol as the plain path: the oracle takes the GPU's router or
halting choice only within rounding of a tie; expert choices (at the
positions that ran each loop) and halt counts must then match exactly and
the output within max|d| / RMS <= 1e-4 (fp32) or 3e-2 (bf16).

Pages: [GN] "[GeekNews 요약] OpenMythos: …" (aisleshub.com), section 6;
[ZS] "OpenMythos 분석: …의 계산 모델링" (zero.shotlearni.ng), §ACT.
"""

import numpy as np
import pytest

from oracle import rdt_oracle as O
from workloads import configs, generate

from gpu_support import EPS_HALT, EPS_ROUTE, DeviceRun, loop_tol, rel_err

pytestmark = pytest.mark.gpu

SPREAD = {"halt_w": 0.05, "halt_b": -0.8}
BIG = {"lora_scale": 1.0, "lora_B": 0.3, "wo": 0.1, "w_down": 0.1, "s_down": 0.1, "halt_w": 0.05, "halt_b": -0.8}


def _inputs(name, scales=None, **over):
    cfg = configs.get(name, **over)
    W = generate.make_weights(cfg, scales=scales)
    e, h0 = generate.make_inputs(cfg)
    return cfg, W, e, h0


def _skip_e2e(cfg, W, e, h0):
    B, T, D = e.shape
    N, L, dt = B * T, cfg["n_loops"], cfg["dtype"]
    print(f"[act skip] {cfg['name']} B={B} T={T} D={D} loops={L} thr={cfg['act_threshold']}", flush=True)
    g = DeviceRun(cfg, W, e, h0, act_skip=True).np()
    adopt = O.Adoption(sel=g["sel"], halt_counts=g["halt"], eps_route=EPS_ROUTE[dt], eps_halt=EPS_HALT[dt])
    ref = O.recurrent_forward_act_skip(cfg, O.Params(W), e, h0, L, cfg["act_threshold"], adopt=adopt, record=True)
    print(f"  adopted route={adopt.route_adopted} halt={adopt.halt_adopted}; "
          f"disagree route={adopt.route_disagree} halt={adopt.halt_disagree}", flush=True)
    assert adopt.route_disagree == 0 and adopt.halt_disagree == 0
    np.testing.assert_array_equal(ref["halt_counts"], g["halt"])
    counts = g["halt"].ravel()
    rows_per_loop = []
    for t in range(L):
        sel = g["sel"][t].reshape(N, -1)
        ran = counts > t                       # positions that ran loop t
        rows_per_loop.append(int(ran.sum()))
        assert np.all(sel[~ran] == -1), f"loop {t}: a halted position was computed"
        if t < ref["loops_run"]:
            idx, osel = ref["record"]["sel"][t]
            np.testing.assert_array_equal(idx, np.nonzero(ran)[0])
            np.testing.assert_array_equal(osel, sel[idx])
    err, tol = rel_err(g["out"], ref["out"]), loop_tol(dt, L)
    print(f"  rows per loop {rows_per_loop}; max|d|/rms = {err:.3e} (tol {tol:.3g})", flush=True)
    assert err <= tol
    return g, ref, rows_per_loop


@pytest.mark.parametrize("name, scales, over", [
    ("tiny_gqa", SPREAD, dict(n_loops=6)),
    ("small_f32", BIG, dict(n_loops=5)),
    ("small_bf16", BIG, dict(n_loops=6)),
    ("small_bf16_k3", SPREAD, dict(n_loops=5, act_threshold=0.99)),
    ("small_bf16", BIG, dict(dim=1024, n_heads=8, n_kv_heads=2, loop_dim=128, lora_rank=16, seq=97, n_loops=4)),
], ids=["tiny_gqa", "small_f32", "small_bf16", "small_bf16_k3", "wide_rows_ragged"])
def test_act_skip_end_to_end(name, scales, over):
    """Halting spread over the loops: every later loop runs fewer rows (a
    ragged row count on the batched tail, the QKV epilogue placing rows by
    position, the O-projection gathering attention rows by position)."""
    cfg, W, e, h0 = _inputs(name, scales=scales, **over)
    g, ref, rows = _skip_e2e(cfg, W, e, h0)
    assert len(np.unique(g["halt"])) > 1
    assert rows[-1] < rows[0]


def test_act_skip_equals_plain_path_when_nothing_halts_early():
    """With no position halting before the last loop nothing is skipped:
    the skipping entry point gives the plain forward's output and halt
    counts bit for bit (same kernels, rows in the same order)."""
    cfg, W, e, h0 = _inputs("small_bf16", scales={"halt_w": 0.0, "halt_b": -30.0}, n_loops=4)
    skip = DeviceRun(cfg, W, e, h0, act_skip=True).np()
    plain = DeviceRun(cfg, W, e, h0).np()
    assert np.all(plain["halt"] == cfg["n_loops"])
    np.testing.assert_array_equal(skip["halt"], plain["halt"])
    np.testing.assert_array_equal(skip["out"], plain["out"])


def test_act_skip_single_token_sequences_match_plain_path():
    """Sequences of one token attend only to themselves, so skipping halted
    positions changes nothing returned: the skipping call matches the plain
    forward (halt counts exactly; outputs to fp32 rounding, since the two
    calls launch some kernels in other shapes for their other row counts,
    e.g. the router logits in 32- or 64-column blocks) while running fewer
    rows in later loops."""
    cfg, W, e, h0 = _inputs("small_bf16", scales=BIG, batch=40, seq=1, n_loops=6)
    skip = DeviceRun(cfg, W, e, h0, act_skip=True).np()
    plain = DeviceRun(cfg, W, e, h0).np()
    assert len(np.unique(plain["halt"])) > 1
    np.testing.assert_array_equal(skip["halt"], plain["halt"])
    assert rel_err(skip["out"], plain["out"]) <= 1e-5


def test_act_skip_refuses_act_off_and_mla():
    import torch
    from recurrent_depth_moe_amd import binding
    cfg, W, e, h0 = _inputs("small_bf16")
    blk = binding.Block(cfg, binding.weights_to_device(W))
    et = torch.from_numpy(e).cuda()
    with pytest.raises(binding.RdtError) as ex:
        blk.forward_act_skip(et, et, 3, 0.0)
    assert ex.value.status == 1
    cfg, W, e, h0 = _inputs("tiny_mla")
    blk = binding.Block(cfg, binding.weights_to_device(W))
    et = torch.from_numpy(e).cuda()
    with pytest.raises(binding.RdtError) as ex:
        blk.forward_act_skip(et, et, 3, 0.99)
    assert ex.value.status == 2
