"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

End to end: same seeded inputs, oracle free-running with the tie-adoption
protocol (the oracle takes the GPU's router / halting choice only where its
own decision is within rounding of a tie, and counts every other
disagreement as a failure); expert choices and halt counts must then match
bit for bit, and the output within max|d| / RMS <= 1e-4 (fp32 configs) or
3e-2 (bf16 configs).

Stage level: the oracle router fed the GPU's own f must give the GPU's
choices bit for bit; the dispatch tables must equal a brute-force stable
sort of the GPU's choices.
"""

import numpy as np
import pytest

from oracle import rdt_oracle as O
from workloads import configs, generate

from gpu_support import EPS_HALT, EPS_ROUTE, TOL, DeviceRun, fill_cache, kv_capacity, read_cache, rel_err

pytestmark = pytest.mark.gpu

SMALL = ["tiny_gqa", "tiny_mla", "small_f32", "small_bf16", "small_bf16_k3"]


def _inputs(name, scales=None, **over):
    cfg = configs.get(name, **over)
    W = generate.make_weights(cfg, scales=scales)
    e, h0 = generate.make_inputs(cfg)
    return cfg, W, e, h0


def _e2e(cfg, W, e, h0, **kw):
    print(f"[e2e] {cfg['name']} B={cfg['batch']} T={cfg['seq']} loops={cfg['n_loops']} thr={cfg['act_threshold']}",
          flush=True)
    g = DeviceRun(cfg, W, e, h0, **kw).np()
    N = e.shape[0] * e.shape[1]
    dt = cfg["dtype"]
    adopt = O.Adoption(sel=g["sel"], halt_counts=g["halt"], eps_route=EPS_ROUTE[dt], eps_halt=EPS_HALT[dt])
    ref = O.recurrent_forward(cfg, O.Params(W), e, h0, cfg["n_loops"], cfg["act_threshold"],
                              adopt=adopt, record=True)
    print(f"  adopted route={adopt.route_adopted} halt={adopt.halt_adopted}; "
          f"disagree route={adopt.route_disagree} halt={adopt.halt_disagree}", flush=True)
    if adopt.disagree_rows:
        T = e.shape[1]
        for (t, n, m) in adopt.disagree_rows[:10]:
            print(f"  disagree loop {t} row {n} (b={n // T}, i={n % T}) margin {m:.3e}: "
                  f"gpu {g['sel'][t].reshape(N, -1)[n]}", flush=True)
    assert adopt.route_disagree == 0
    assert adopt.halt_disagree == 0
    N = e.shape[0] * e.shape[1]
    for t in range(ref["loops_run"]):
        np.testing.assert_array_equal(ref["record"]["sel"][t], g["sel"][t].reshape(N, -1))
    # loops after every position halted are skipped on both sides: their capture slots stay untouched
    for t in range(ref["loops_run"], cfg["n_loops"]):
        assert np.all(g["sel"][t] == -1)
    np.testing.assert_array_equal(ref["halt_counts"], g["halt"])
    err = rel_err(g["out"], ref["out"])
    print(f"  max|d|/rms = {err:.3e} (tol {TOL[dt]})", flush=True)
    assert err <= TOL[dt]
    return g, ref


@pytest.mark.parametrize("name", SMALL)
def test_end_to_end(name):
    cfg, W, e, h0 = _inputs(name)
    _e2e(cfg, W, e, h0)


@pytest.mark.parametrize("name", ["tiny_gqa", "small_f32", "small_bf16"])
def test_end_to_end_large_terms(name):
    """O(1) LoRA / output / halting scales so every term of the loop is far
    above the tolerance (at the default init LoRA is ~1e-3 of the state)."""
    scales = {"lora_scale": 1.0, "lora_B": 0.3, "wo": 0.1, "w_down": 0.1, "s_down": 0.1,
              "halt_w": 0.05, "halt_b": -0.8}
    cfg, W, e, h0 = _inputs(name, scales=scales)
    g, ref = _e2e(cfg, W, e, h0)
    if cfg["act_threshold"] > 0:
        assert len(np.unique(g["halt"])) > 1


def test_end_to_end_f32_products_with_ragged_k():
    """fp32 products on the MFMA tile kernel with an expert width of 100:
    the routed and shared down products reduce over K = 100 (the last
    16-deep k stage is a quarter full) and the gate | up outputs end inside
    a 64-column tile; 300 rows end inside a 64-row tile."""
    cfg, W, e, h0 = _inputs("small_f32", expert_dim=100)
    assert cfg["expert_dim"] % 16 != 0
    _e2e(cfg, W, e, h0)


def test_end_to_end_groups_split_over_xcds():
    """batch 4 x 2 kv heads = 8 (batch, kv head) groups: flash attention
    gives each XCD its own group (the ordering the large prefill takes),
    with a ragged sequence."""
    cfg, W, e, h0 = _inputs("small_bf16", batch=4, seq=150)
    assert cfg["batch"] * cfg["n_kv_heads"] % 8 == 0
    _e2e(cfg, W, e, h0)


def test_end_to_end_merged_expert_tails():
    """dim 768 (a multiple of 192, so the routed down product runs on
    192-column tiles) with about 270 routed rows per expert: an expert with
    257-320 rows is one m-tile of the down product's merged schedule (its
    last rows one or two 32-row strips of that tile), the others keep a tile
    of their own for the rows past 256."""
    import torch
    scales = {"w_down": 0.1, "s_down": 0.1}
    cfg, W, e, h0 = _inputs("small_bf16_strip", scales=scales)
    run = DeviceRun(cfg, W, e, h0)
    E = cfg["n_experts"]
    counts = np.diff(run.ws_np("offsets", torch.int32, (E + 1,)))
    mts = run.ws_np("mt_start", torch.int32, (E + 1,))
    mtm = run.ws_np("mt_start_merged", torch.int32, (E + 1,))
    print(f"  rows per expert {counts.tolist()}; m-tiles {mts[-1]} plain, {mtm[-1]} merged", flush=True)
    merged = (counts > 256) & (counts <= 320)
    assert merged.any(), counts
    assert mtm[-1] == mts[-1] - int(merged.sum())
    _e2e(cfg, W, e, h0)


def test_end_to_end_short_tiles_of_192_column_products():
    """dim 768 with 24 experts (about 60 routed rows each): every expert's
    rows fit one short tile (<= 64 or <= 128 rows) of the routed down
    product's 192-column tiles, which then loads and multiplies only those
    rows (three waves store 64 columns each)."""
    import torch
    scales = {"w_down": 0.1, "s_down": 0.1}
    cfg, W, e, h0 = _inputs("small_bf16_strip", scales=scales, n_experts=24, seq=360)
    run = DeviceRun(cfg, W, e, h0)
    E = cfg["n_experts"]
    counts = np.diff(run.ws_np("offsets", torch.int32, (E + 1,)))
    print(f"  rows per expert {counts.tolist()}", flush=True)
    assert np.sum(counts <= 64) > 0 and np.sum((counts > 64) & (counts <= 128)) > 0
    _e2e(cfg, W, e, h0)


@pytest.mark.parametrize("over, where", [
    (dict(seq=300), "only"),                  # 112-212 rows per expert
    (dict(seq=420, n_experts=4), "second"),   # 371-465 rows: a 256-row tile, then 115-209
], ids=["only-tile", "second-tile"])
def test_end_to_end_192_row_tiles(over, where):
    """Routed tiles of 129-192 rows run with three 32-row fragments per wave
    (gate|up on 256-column tiles, down on 192-column ones): as an expert's
    only tile, and as the tile after a full 256-row one (the down product's
    merged schedule; the gate|up schedule splits an expert's rows evenly
    over its m-tiles, 186-233 rows each here).  Both schedules are checked
    exactly against their definitions from the dispatch offsets."""
    import torch
    scales = {"w_down": 0.1, "s_down": 0.1}
    cfg, W, e, h0 = _inputs("small_bf16_strip", scales=scales, **over)
    run = DeviceRun(cfg, W, e, h0)
    E = cfg["n_experts"]
    counts = np.diff(run.ws_np("offsets", torch.int32, (E + 1,)))
    print(f"  rows per expert {counts.tolist()}", flush=True)
    tail = counts % 256 if where == "second" else counts
    hit = (tail > 128) & (tail <= 192) & ((counts > 256) if where == "second" else (counts <= 256))
    assert hit.any(), counts
    # plain schedule: ceil(rows / 256) m-tiles per expert starting at
    # off + floor(i rows / n); merged: tiles of 256 rows, the last taking a
    # remainder of at most 64 rows
    off = run.ws_np("offsets", torch.int32, (E + 1,))
    mts = run.ws_np("mt_start", torch.int32, (E + 1,))
    mtm = run.ws_np("mt_start_merged", torch.int32, (E + 1,))
    tr0 = run.ws_np("tile_row0", torch.int32, (int(mts[-1]),))
    trm = run.ws_np("tile_row0_merged", torch.int32, (int(mtm[-1]),))
    for x in range(E):
        n = -(-int(counts[x]) // 256)
        assert mts[x + 1] - mts[x] == n
        np.testing.assert_array_equal(tr0[mts[x]:mts[x + 1]], off[x] + (np.arange(n) * int(counts[x])) // max(n, 1))
        nm = n - 1 if counts[x] > 256 and 0 < counts[x] % 256 <= 64 else n
        assert mtm[x + 1] - mtm[x] == nm
        np.testing.assert_array_equal(trm[mtm[x]:mtm[x + 1]], off[x] + 256 * np.arange(nm))
    _e2e(cfg, W, e, h0)


@pytest.mark.parametrize("name, over", [
    ("small_bf16", dict(batch=3, seq=1, n_loops=2)),                         # single-token prefill, no cache
    ("small_bf16", dict(batch=1, seq=5)),                                    # one short sequence
    ("small_bf16", dict(n_experts=2, top_k=2)),                              # every token to every expert
    ("small_bf16", dict(n_experts=1, top_k=1, n_shared_experts=0)),          # one expert, no shared expert
    ("small_f32", dict(act_threshold=1.0)),                                  # halting only by the last-loop rule
], ids=["T1-no-cache", "B1-T5", "top2-of-2", "one-expert", "thr-1.0"])
def test_end_to_end_degenerate_shapes(name, over):
    """Degenerate shapes and routing: every step of the path against the
    oracle where tiles are mostly padding, routing has no choice, or the
    shared expert is absent."""
    cfg, W, e, h0 = _inputs(name, **over)
    _e2e(cfg, W, e, h0)


@pytest.mark.parametrize("act", [0.99, 0.0])
def test_end_to_end_wide_rows(act):
    """dim 1024 with rank-16 LoRA, top-2 plus one shared expert: the batched
    loop-tail form the large configurations run, end to end, with O(1)
    LoRA / output / halting terms."""
    scales = {"lora_scale": 1.0, "lora_B": 0.3, "wo": 0.1, "w_down": 0.1, "s_down": 0.1,
              "halt_w": 0.05, "halt_b": -0.8}
    cfg, W, e, h0 = _inputs("small_bf16", scales=scales, dim=1024, n_heads=8, n_kv_heads=2, loop_dim=128,
                            lora_rank=16, seq=96, act_threshold=act)
    g, ref = _e2e(cfg, W, e, h0)
    if act > 0:
        assert len(np.unique(g["halt"])) > 1


@pytest.mark.parametrize("name", ["tiny_gqa", "tiny_mla", "small_bf16"])
def test_end_to_end_stops_once_all_halted(name):
    """Every position halts by loop 2: the remaining loops are skipped on the
    GPU (their capture slots stay untouched) and on the oracle, with the
    same output and halt counts."""
    cfg, W, e, h0 = _inputs(name, scales={"halt_w": 0.005, "halt_b": 3.0})
    g, ref = _e2e(cfg, W, e, h0)
    assert ref["loops_run"] < cfg["n_loops"]
    assert g["halt"].max() == ref["loops_run"]


@pytest.mark.parametrize("name", ["tiny_gqa", "small_bf16"])
def test_act_off_and_single_loop(name):
    cfg, W, e, h0 = _inputs(name, n_loops=1, act_threshold=0.0)
    g, _ = _e2e(cfg, W, e, h0)
    assert np.all(g["halt"] == 1)


@pytest.mark.parametrize("name", ["tiny_gqa", "small_bf16_k3"])
def test_router_and_dispatch_stage(name):
    """Oracle router on the GPU's own f: bit-identical choices; dispatch
    tables equal a brute-force stable sort of the choices."""
    cfg, W, e, h0 = _inputs(name, n_loops=1, act_threshold=0.0)
    run = DeviceRun(cfg, W, e, h0)
    import torch
    B, T, D = e.shape
    N, k, E = B * T, cfg["top_k"], cfg["n_experts"]
    fdt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    f = run.ws_np("f", fdt, (N, D))
    sel = run.ws_np("sel", torch.int32, (N, k))
    gate = run.ws_np("gate", torch.float32, (N, k))
    z, osel, ogate, margin = O.router(cfg, O.Params(W), O.as_f64(f))
    close = margin < 1e-6 * np.abs(z).max()
    assert np.array_equal(osel[~close], sel[~close])
    print(f"  near-tie rows excluded: {int(close.sum())}")
    np.testing.assert_allclose(gate, ogate, rtol=2e-6 if cfg["dtype"] == "f32" else 2e-5, atol=1e-7)
    counts = np.bincount(sel.ravel(), minlength=E)
    offsets = run.ws_np("offsets", torch.int32, (E + 1,))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    perm = run.ws_np("perm", torch.int32, (N * k,))
    inv = run.ws_np("inv", torch.int32, (N * k,))
    slots = sorted(range(N * k), key=lambda a: (sel.ravel()[a], a))   # stable by (expert, token, slot)
    np.testing.assert_array_equal(perm, np.array(slots) // k)
    np.testing.assert_array_equal(inv[np.array(slots)], np.arange(N * k))


def test_router_ties_go_to_lower_index():
    """Duplicate router rows give bitwise-equal logits; the lower expert
    index must win every such tie."""
    cfg, W, e, h0 = _inputs("small_bf16", n_loops=1, act_threshold=0.0)
    W = dict(W)
    rw = W["router_w"].copy()
    rw[5] = rw[2]
    rw[7] = rw[0]
    W["router_w"] = rw
    g = DeviceRun(cfg, W, e, h0).np()
    sel = g["sel"][0]
    for row in sel:
        row = list(row)
        if 5 in row:
            assert 2 in row and row.index(2) < row.index(5)
        if 7 in row:
            assert 0 in row and row.index(0) < row.index(7)
    assert any(2 in r or 5 in r for r in sel)


def test_deterministic_bitwise():
    cfg, W, e, h0 = _inputs("small_bf16")
    a = DeviceRun(cfg, W, e, h0).np()
    b = DeviceRun(cfg, W, e, h0).np()
    for key in ("out", "halt", "h", "sel", "p"):
        np.testing.assert_array_equal(a[key], b[key])


def test_spectral_radius_from_block():
    import torch
    from recurrent_depth_moe_amd import binding
    cfg, W, e, h0 = _inputs("tiny_gqa")
    blk = binding.Block(cfg, binding.weights_to_device(W))
    A = blk.get_A().numpy()
    ref = O.lti_A(O.Params(W))
    np.testing.assert_allclose(A, ref, rtol=1e-7)
    assert A.max() < 1.0
    assert blk.param_count() == sum(v.size for v in W.values())


# ---------------------------------------------------------------- decode

def _oracle_cache(cfg, n_loops, B, cap):
    return O.new_cache(cfg, B, cap, n_loops)


@pytest.mark.parametrize("start_pos", [1, 100])
def test_mla_decode_against_random_latent_cache(start_pos):
    """MLA decode step (attention over the cached latent with absorbed
    up-projections) of 3 sequences at ``start_pos`` against caches holding
    N(0,1) latents c_kv / k_rope at positions 0..start_pos-1 in every loop
    slot and NaN past them; the oracle rebuilds per-head K / V from the same
    latents."""
    import torch
    from recurrent_depth_moe_amd import binding
    cfg, W, e, h0 = _inputs("tiny_mla", batch=3, seq=1, start_pos=start_pos, n_loops=5, use_cache=True)
    B, P, n = cfg["batch"], cfg["start_pos"], cfg["n_loops"]
    kvl, rope = cfg["kv_lora_rank"], cfg["qk_rope_head_dim"]
    cap = kv_capacity(cfg)
    Pp = (cap + 63) // 64 * 64
    kv = torch.full((binding.kv_cache_bytes(cfg, B, cap, n),), 0xFF, dtype=torch.uint8, device="cuda")
    slot = kv.numel() // n
    oc = O.new_cache(cfg, B, cap, n)
    for t in range(n):
        ckv = generate.draw(cfg["seed"], f"cache_ckv_{t}", (B, P, kvl), "normal", 1.0)
        kr = generate.draw(cfg["seed"], f"cache_krope_{t}", (B, P, rope), "normal", 1.0)
        ckv, kr = ckv.reshape(B, P, kvl), kr.reshape(B, P, rope)
        base = kv[t * slot:(t + 1) * slot].view(torch.float32)
        base[:B * Pp * kvl].view(B, Pp, kvl)[:, :P] = torch.from_numpy(ckv).cuda()
        base[B * Pp * kvl:B * Pp * (kvl + rope)].view(B, Pp, rope)[:, :P] = torch.from_numpy(kr).cuda()
        oc[t]["c_kv"][:, :P] = ckv
        oc[t]["k_rope"][:, :P] = kr
    print(f"[mla decode] B={B} pos={P} loops={n}", flush=True)
    g = DeviceRun(cfg, W, e, h0, kv=kv, decode=True).np()
    assert np.all(np.isfinite(g["out"]))
    thr = cfg["act_threshold"]
    adopt = O.Adoption(sel=g["sel"], halt_counts=g["halt"], eps_route=EPS_ROUTE["f32"], eps_halt=EPS_HALT["f32"])
    ref = O.recurrent_forward(cfg, O.Params(W), e, h0, n, thr, start_pos=P, cache=oc, adopt=adopt, record=True)
    assert adopt.route_disagree == 0 and adopt.halt_disagree == 0
    np.testing.assert_array_equal(ref["halt_counts"], g["halt"])
    err = rel_err(g["out"], ref["out"])
    print(f"  max|d|/rms = {err:.3e}", flush=True)
    assert err <= TOL["f32"]


@pytest.mark.parametrize("start_pos,kv_heads,nan_past_end", [
    (300, 2, False),      # one key block, ragged
    (511, 1, True),       # exactly one full block of 512 keys; cache past the end holds NaN
    (512, 2, True),       # a second block holding one key
    (1100, 1, True),      # three blocks, four query heads per kv head
])
def test_decode_against_random_cache(start_pos, kv_heads, nan_past_end):
    """One decode step of 4 sequences at ``start_pos`` against caches holding
    N(0,1) bf16 K/V at positions 0..start_pos-1 in every loop slot.  With
    ``nan_past_end`` every cache byte past the new position is NaN, which
    must not reach the output."""
    import torch
    from recurrent_depth_moe_amd import binding
    cfg, W, e, h0 = _inputs("small_bf16_decode", start_pos=start_pos, n_kv_heads=kv_heads,
                            max_seq_len=max(512, start_pos + 1))
    B, P, n = cfg["batch"], cfg["start_pos"], cfg["n_loops"]
    cap = kv_capacity(cfg)
    fill = 0xFF if nan_past_end else 0
    kv = torch.full((binding.kv_cache_bytes(cfg, B, cap, n),), fill, dtype=torch.uint8, device="cuda")
    oc = _oracle_cache(cfg, n, B, cap)
    for t in range(n):
        K = generate.make_cache_loop(cfg, t, "k")
        V = generate.make_cache_loop(cfg, t, "v")
        fill_cache(cfg, None, kv, t, K, V)
        oc[t]["k"][:, :, :P] = O.as_f64(K)
        oc[t]["v"][:, :, :P] = O.as_f64(V)
    print(f"[decode] {cfg['name']} B={B} pos={P} kv_heads={kv_heads} loops={n} nan_past_end={nan_past_end}",
          flush=True)
    g = DeviceRun(cfg, W, e, h0, kv=kv, decode=True).np()
    assert np.all(np.isfinite(g["out"]))
    adopt = O.Adoption(sel=g["sel"], halt_counts=g["halt"], eps_route=EPS_ROUTE["bf16"], eps_halt=EPS_HALT["bf16"])
    ref = O.recurrent_forward(cfg, O.Params(W), e, h0, n, 0.0, start_pos=P, cache=oc, adopt=adopt, record=True)
    assert adopt.route_disagree == 0
    err = rel_err(g["out"], ref["out"])
    print(f"  max|d|/rms = {err:.3e}", flush=True)
    assert err <= TOL["bf16"]
    # the step appended its K/V at position P of every slot
    for t in range(n):
        k_gpu, v_gpu = read_cache(cfg, kv, t, B)
        np.testing.assert_array_equal(k_gpu[:, :, :P], O.as_f64(generate.make_cache_loop(cfg, t, "k")))
        assert rel_err(k_gpu[:, :, P], oc[t]["k"][:, :, P]) < TOL["bf16"]
        assert rel_err(v_gpu[:, :, P], oc[t]["v"][:, :, P]) < TOL["bf16"]


def test_decode_on_a_non_default_stream():
    """A bf16 decode step with a shared expert, enqueued on a fresh stream
    (its shared-expert products fork to the handle's side stream and join
    back before the loop tail), gives bitwise the outputs and cache writes
    of the same step on the default stream, twice in a row."""
    import torch
    from recurrent_depth_moe_amd import binding
    cfg, W, e, h0 = _inputs("small_bf16_decode")
    assert cfg["n_shared_experts"] > 0
    B, n = cfg["batch"], cfg["n_loops"]
    cap = kv_capacity(cfg)

    def cache():
        kv = torch.zeros((binding.kv_cache_bytes(cfg, B, cap, n),), dtype=torch.uint8, device="cuda")
        for t in range(n):
            fill_cache(cfg, None, kv, t, generate.make_cache_loop(cfg, t, "k"), generate.make_cache_loop(cfg, t, "v"))
        return kv

    print(f"[decode stream] {cfg['name']} B={B} pos={cfg['start_pos']} loops={n}", flush=True)
    kv0 = cache()
    ref = DeviceRun(cfg, W, e, h0, kv=kv0, decode=True).np()
    side = torch.cuda.Stream()
    for _ in range(2):
        kv1 = cache()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            got = DeviceRun(cfg, W, e, h0, kv=kv1, decode=True).np()
        np.testing.assert_array_equal(got["out"], ref["out"])
        np.testing.assert_array_equal(got["sel"], ref["sel"])
        assert torch.equal(kv1, kv0)


@pytest.mark.parametrize("name", ["tiny_gqa", "tiny_mla", "small_bf16"])
def test_prefill_then_decode_matches_full_prefill(name):
    """Prefill of positions 0..T-2 into the per-loop caches, then a decode
    step at T-1, gives row T-1 of a full prefill (GPU vs GPU, and vs the
    oracle) in every loop ([ZS §RoPE & generation cache])."""
    import torch
    from recurrent_depth_moe_amd import binding
    cfg, W, e, h0 = _inputs(name, act_threshold=0.0)
    B, T, n = cfg["batch"], cfg["seq"], cfg["n_loops"]
    cfgc = dict(cfg, start_pos=0)
    kv = torch.zeros(binding.kv_cache_bytes(cfg, B, T, n), dtype=torch.uint8, device="cuda")
    full = DeviceRun(cfg, W, e, h0).np()
    pre_cfg = dict(cfgc, seq=T - 1)
    DeviceRun(pre_cfg, W, e[:, :T - 1].copy(), h0[:, :T - 1].copy(), kv=kv, start_pos=0, capture=False, kv_cap=T)
    step_cfg = dict(cfgc, seq=1, start_pos=T - 1)
    g = DeviceRun(step_cfg, W, e[:, T - 1:].copy(), h0[:, T - 1:].copy(), kv=kv, decode=True, kv_cap=T).np()
    tol = TOL[cfg["dtype"]]
    assert rel_err(g["out"][:, 0], full["out"][:, T - 1]) < tol
    ref = O.recurrent_forward(cfg, O.Params(W), e, h0, n, 0.0)["out"]
    assert rel_err(g["out"][:, 0], ref[:, T - 1]) < tol


@pytest.mark.parametrize("name,act", [("tiny_gqa", True), ("tiny_mla", True), ("small_bf16", False)])
def test_chained_decode_steps_match_full_prefill(name, act):
    """Prefill of positions 0..T-5, then four chained decode steps at
    T-4 .. T-1, each appending to the same per-loop caches, reproduce the
    last four rows of a full prefill, ACT output and halt counts included
    ([ZS §RoPE & generation cache]); each step is also compared with the
    oracle's full prefill at that position."""
    import torch
    from recurrent_depth_moe_amd import binding
    over = {} if act else {"act_threshold": 0.0}
    cfg, W, e, h0 = _inputs(name, **over)
    B, T, n = cfg["batch"], cfg["seq"], cfg["n_loops"]
    steps = 4
    cfgc = dict(cfg, start_pos=0)
    kv = torch.zeros(binding.kv_cache_bytes(cfg, B, T, n), dtype=torch.uint8, device="cuda")
    full = DeviceRun(cfg, W, e, h0).np()
    # the oracle's full prefill, decisions within the tie margins taken
    # from the GPU's full prefill
    dt = cfg["dtype"]
    adopt = O.Adoption(sel=full["sel"], halt_counts=full["halt"], eps_route=EPS_ROUTE[dt], eps_halt=EPS_HALT[dt])
    ref = O.recurrent_forward(cfg, O.Params(W), e, h0, n, cfg["act_threshold"], adopt=adopt)
    assert adopt.route_disagree == 0 and adopt.halt_disagree == 0
    P0 = T - steps
    DeviceRun(dict(cfgc, seq=P0), W, e[:, :P0].copy(), h0[:, :P0].copy(), kv=kv, start_pos=0, capture=False, kv_cap=T)
    tol = TOL[dt]
    for i in range(P0, T):
        g = DeviceRun(dict(cfgc, seq=1, start_pos=i), W, e[:, i:i + 1].copy(), h0[:, i:i + 1].copy(), kv=kv,
                   decode=True, kv_cap=T).np()
        print(f"[chained decode] {name} position {i}: max|d|/rms {rel_err(g['out'][:, 0], full['out'][:, i]):.2e} "
              f"vs the GPU prefill, {rel_err(g['out'][:, 0], ref['out'][:, i]):.2e} vs the oracle", flush=True)
        assert rel_err(g["out"][:, 0], full["out"][:, i]) < tol
        np.testing.assert_array_equal(g["halt"][:, 0], full["halt"][:, i])
        assert rel_err(g["out"][:, 0], ref["out"][:, i]) < tol
        np.testing.assert_array_equal(g["halt"][:, 0], ref["halt_counts"][:, i])
