"""Parity at the full workload sizes, in the launch configuration the
benchmark times (same shapes, same entry point, same kernels), on sampled
outputs.

The fp64 oracle cannot run every loop at these sizes in seconds, so the
loop itself is checked teacher-forced: the GPU's captured state h_t enters
the oracle, which computes loop t for 512 sampled rows (K and V for every
position, everything else only for the sampled rows, first and last row of
each sequence included) and must reproduce the GPU's h_{t+1} there within
max|d| / RMS <= 3e-2 (bf16), with expert choices equal outside the router's
tie margin.  Properties that hold at any size are checked on every row:
the router on the GPU's own f, the dispatch tables against a brute-force
stable sort, the halt counts against the first crossing recomputed from
the captured halting probabilities, and the ACT output as the weighted sum
of the captured states.
"""

import numpy as np
import pytest

from oracle import rdt_oracle as O
from workloads import configs, generate

from gpu_support import EPS_HALT, EPS_ROUTE, TOL, DeviceRun, fill_cache, free_running_tol, kv_capacity, rel_err

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

N_SAMPLE = 512


def _sample_rows(B, T, n, seed):
    rng = np.random.default_rng(seed)
    rows = {(b, 0) for b in range(B)} | {(b, T - 1) for b in range(B)}
    while len(rows) < min(n, B * T):
        rows.add((int(rng.integers(B)), int(rng.integers(T))))
    return sorted(rows)


def _teacher_forced(cfg, P, g, e, t, rows, cache=None):
    """Oracle loop t from the GPU's state before it, compared on ``rows``
    with the GPU's state after it.  Router choices within the bf16 tie
    margin are taken from the GPU; any other difference fails."""
    B, T, D = e.shape
    N = B * T
    h_in = O.as_f64(g["h0"]) if t == 0 else O.as_f64(g["h"][t - 1]).reshape(B, T, D)
    gpu_sel = g["sel"][t].reshape(N, -1)
    idx = np.array([b * T + i for (b, i) in rows])
    stats = dict(adopted=0, disagree=0)

    def hook(sel, margin, rr):
        out = sel.copy()
        for n in range(len(rr)):
            want = gpu_sel[idx[n]]
            if not np.array_equal(sel[n], want):
                if margin[n] < EPS_ROUTE["bf16"]:
                    out[n] = want
                    stats["adopted"] += 1
                else:
                    stats["disagree"] += 1
                    print(f"  loop {t} row {rr[n]} margin {margin[n]:.3e}: oracle {sel[n]} gpu {want}", flush=True)
        return out

    step = O.run_loop(cfg, P, h_in, O.as_f64(e), t, cfg["start_pos"], cache, rows=rows, route_hook=hook)
    got = g["h"][t].reshape(N, D)[idx]
    err = rel_err(got, step["h"])
    print(f"[{cfg['name']}] loop {t}: {len(rows)} rows, max|d|/rms = {err:.3e}, "
          f"routes adopted {stats['adopted']}, disagree {stats['disagree']}", flush=True)
    assert stats["disagree"] == 0
    assert err <= TOL["bf16"]


def _dispatch_and_router(cfg, P, run):
    """Every row of the last loop: oracle router on the GPU's f, dispatch
    tables against a stable sort of the GPU's choices."""
    import torch
    B, T = cfg["batch"], cfg["seq"]
    N, D, k, E = B * T, cfg["dim"], cfg["top_k"], cfg["n_experts"]
    f = run.ws_np("f", torch.bfloat16, (N, D))
    sel = run.ws_np("sel", torch.int32, (N, k))
    z, osel, _, margin = O.router(cfg, P, O.as_f64(f))
    close = margin < 1e-6 * np.abs(z).max()
    print(f"[{cfg['name']}] router on GPU f: {N} rows, near-tie rows excluded {int(close.sum())}", flush=True)
    np.testing.assert_array_equal(osel[~close], sel[~close])
    counts = np.bincount(sel.ravel(), minlength=E)
    assert counts.sum() == N * k
    offsets = run.ws_np("offsets", torch.int32, (E + 1,))
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    order = np.argsort(sel.ravel(), kind="stable")        # by expert, then (token, slot)
    perm = run.ws_np("perm", torch.int32, (N * k,))
    inv = run.ws_np("inv", torch.int32, (N * k,))
    np.testing.assert_array_equal(perm, order // k)
    np.testing.assert_array_equal(inv[order], np.arange(N * k))


def _free_running(cfg, W, e, h0, r, seqs=None, cache=None, state_tol=None):
    """The oracle runs every loop from the same e and h0 as the GPU (no
    teacher forcing), on whole sequences (``seqs``: all when None; each
    sequence is independent of the others, so a subset is exact).  Router
    and halting decisions within the bf16 tie margins are taken from the
    GPU; any other difference fails.  Checks, on every row of those
    sequences: halt counts equal, expert choices equal outside the margins,
    and the final state within ``state_tol`` (max|d| / RMS); prints the
    per-loop state error and the output error.  With ACT on the output is
    the halting-weighted sum of states that differ by O(RMS) from loop to
    loop, and the weights p = sigmoid(h . w + b) sum the state error over all
    D channels, so its error is reported, not held to the state bound."""
    import time
    B, T, D = e.shape
    seqs = list(range(B)) if seqs is None else list(seqs)
    Bs, N, L = len(seqs), len(seqs) * T, cfg["n_loops"]
    sub = dict(cfg, batch=Bs)
    rows = np.concatenate([np.arange(b * T, (b + 1) * T) for b in seqs])
    sel = r["sel"].reshape(L, B * T, -1)[:, rows]
    halt = r["halt"].reshape(B, T)[seqs]
    adopt = O.Adoption(sel=sel, halt_counts=halt, eps_route=EPS_ROUTE["bf16"], eps_halt=EPS_HALT["bf16"])
    gh = r["h"].reshape(L, B * T, D)
    curve = []
    t0 = time.time()

    def on_loop(t, h):
        err = rel_err(gh[t][rows], h.reshape(N, D))
        curve.append(err)
        print(f"[{cfg['name']}] free-running loop {t}: state max|d|/rms = {err:.3e} "
              f"(routes adopted {adopt.route_adopted}, disagree {adopt.route_disagree}; "
              f"{time.time() - t0:.0f} s)", flush=True)

    ref = O.recurrent_forward(sub, O.Params(W), e[seqs], h0[seqs], L, cfg["act_threshold"],
                              start_pos=cfg["start_pos"], cache=cache, adopt=adopt, on_loop=on_loop)
    err = rel_err(r["out"].reshape(B, T, D)[seqs], ref["out"])
    print(f"[{cfg['name']}] free-running over {L} loops on {N} rows: output max|d|/rms = {err:.3e}; "
          f"per-loop state error {[round(x, 5) for x in curve]}; routes adopted {adopt.route_adopted}, "
          f"halts adopted {adopt.halt_adopted}", flush=True)
    for (lp, n, m) in adopt.disagree_rows[:10]:
        print(f"  route disagreement: loop {lp} row {n} margin {m:.3e}", flush=True)
    assert adopt.route_disagree == 0 and adopt.halt_disagree == 0
    np.testing.assert_array_equal(halt, ref["halt_counts"])
    tol = TOL["bf16"] if state_tol is None else state_tol
    print(f"[{cfg['name']}] final state max|d|/rms = {curve[-1]:.3e} (tol {tol:.3e})", flush=True)
    assert curve[-1] <= tol
    if cfg["act_threshold"] == 0:
        assert err <= tol


def _gpu(cfg, W, e, h0, **kw):
    g = DeviceRun(cfg, W, e, h0, **kw)
    r = g.np()
    r["h0"] = h0
    return g, r


# ------------------------------------------------------------------ mythos_3b

@pytest.fixture(scope="module")
def run_3b():
    cfg = configs.get("mythos_3b")
    W = generate.make_weights(cfg)
    e, h0 = generate.make_inputs(cfg)
    print(f"[mythos_3b] B={cfg['batch']} T={cfg['seq']} loops={cfg['n_loops']} thr={cfg['act_threshold']}",
          flush=True)
    g, r = _gpu(cfg, W, e, h0)
    return cfg, W, e, h0, g, r


def test_3b_router_and_dispatch(run_3b):
    cfg, W, e, h0, g, r = run_3b
    _dispatch_and_router(cfg, O.Params(W), g)


def test_3b_act_on_every_row(run_3b):
    """Halting probabilities from the captured states (sampled rows), halt
    counts from the captured probabilities (every row, same float32
    decision), output as the ACT-weighted sum of the captured states."""
    cfg, W, e, h0, g, r = run_3b
    B, T, D = e.shape
    N, L, thr = B * T, cfg["n_loops"], cfg["act_threshold"]
    P = O.Params(W)
    rows = _sample_rows(B, T, N_SAMPLE, 11)
    idx = np.array([b * T + i for (b, i) in rows])
    for t in range(L):
        p_ref = O.halting_probability(P, O.as_f64(r["h"][t].reshape(N, D)[idx]))
        assert np.max(np.abs(r["p"][t][idx] - p_ref)) < 1e-5
    cum = np.zeros(N)
    cum32 = np.zeros(N, dtype=np.float32)
    halted = np.zeros(N, dtype=bool)
    counts = np.full(N, L)
    out = np.zeros((len(idx), D))
    for t in range(L):
        p = r["p"][t].astype(np.float64)
        running = ~halted
        now = O.act_halts(cum32, running, p, t, L, thr)
        w = O.act_weights(cum, running, p, now)
        out += w[idx, None] * r["h"][t].reshape(N, D)[idx]
        cum = cum + p * running
        cum32 = np.where(running, (cum32 + p.astype(np.float32)).astype(np.float32), cum32)
        counts[now] = t + 1
        halted |= now
    np.testing.assert_array_equal(r["halt"].ravel(), counts)
    hist = np.bincount(counts, minlength=L + 1)[1:]
    print(f"[mythos_3b] halt histogram {hist.tolist()}", flush=True)
    assert len(np.unique(counts)) > 4
    err = rel_err(r["out"].reshape(N, D)[idx], out)
    print(f"[mythos_3b] ACT output on {len(idx)} rows: max|d|/rms = {err:.3e}", flush=True)
    assert err <= TOL["f32"]


def test_3b_free_running_all_loops(run_3b):
    """Every loop of the full mythos_3b workload (both sequences, all 4096
    positions, ACT at 0.99) against the oracle run free from the same
    inputs: decisions exact (tie adoption), the final state within the
    free-running bf16 bound."""
    cfg, W, e, h0, g, r = run_3b
    _free_running(cfg, W, e, h0, r, state_tol=free_running_tol(cfg["n_loops"]))


@pytest.mark.parametrize("t", [0, 15])
def test_3b_teacher_forced_loop(run_3b, t):
    cfg, W, e, h0, g, r = run_3b
    _teacher_forced(cfg, O.Params(W), r, e, t, _sample_rows(cfg["batch"], cfg["seq"], N_SAMPLE, 100 + t))


# ------------------------------------------------------------------ mythos_1b

def test_1b_full_size():
    """ACT off: the output is the last captured state; loops 0 and 15
    teacher-forced on sampled rows; router and dispatch on every row; all
    16 loops free-running against the oracle on every row."""
    cfg = configs.get("mythos_1b")
    W = generate.make_weights(cfg)
    e, h0 = generate.make_inputs(cfg)
    print(f"[mythos_1b] B={cfg['batch']} T={cfg['seq']} loops={cfg['n_loops']}", flush=True)
    g, r = _gpu(cfg, W, e, h0)
    np.testing.assert_array_equal(r["out"].reshape(-1), r["h"][-1].reshape(-1))
    assert np.all(r["halt"] == cfg["n_loops"])
    P = O.Params(W)
    _dispatch_and_router(cfg, P, g)
    for t in (0, cfg["n_loops"] - 1):
        _teacher_forced(cfg, P, r, e, t, _sample_rows(cfg["batch"], cfg["seq"], N_SAMPLE, 200 + t))
    _free_running(cfg, W, e, h0, r)


# ---------------------------------------------------------- mythos_10b decode

FREE_SEQS_10B = (0, 11, 22, 31)


def test_10b_decode_full_size():
    """One decode step of 32 sequences at position 8192 against 8192 cached
    N(0,1) positions in every one of the 24 loop slots (seeded, the same
    values the oracle reads).  Loops 0 and 23 are teacher-forced on every
    sequence; four whole sequences run free through all 24 loops against
    the oracle (sequences are independent, so the subset is exact)."""
    import torch
    from recurrent_depth_moe_amd import binding
    cfg = configs.get("mythos_10b_decode")
    W = generate.make_weights(cfg)
    e, h0 = generate.make_inputs(cfg)
    B, P, L = cfg["batch"], cfg["start_pos"], cfg["n_loops"]
    G, dh = cfg["n_kv_heads"], cfg["head_dim"]
    cap = kv_capacity(cfg)
    kv = torch.zeros(binding.kv_cache_bytes(cfg, B, cap, L), dtype=torch.uint8, device="cuda")
    checked = (0, L - 1)
    free = list(FREE_SEQS_10B)
    oc, ocf = {}, []
    for t in range(L):
        K = generate.make_cache_loop(cfg, t, "k")
        V = generate.make_cache_loop(cfg, t, "v")
        fill_cache(cfg, None, kv, t, K, V)
        fk = np.zeros((len(free), G, cap, dh))
        fv = np.zeros((len(free), G, cap, dh))
        fk[:, :, :P] = O.as_f64(K[free])
        fv[:, :, :P] = O.as_f64(V[free])
        ocf.append(dict(k=fk, v=fv))
        if t in checked:
            oc[t] = dict(k=np.zeros((B, G, cap, dh)), v=np.zeros((B, G, cap, dh)))
            oc[t]["k"][:, :, :P] = O.as_f64(K)
            oc[t]["v"][:, :, :P] = O.as_f64(V)
        del K, V
    torch.cuda.synchronize()
    print(f"[mythos_10b_decode] B={B} pos={P} loops={L}; every cache slot seeded", flush=True)
    g, r = _gpu(cfg, W, e, h0, kv=kv)
    np.testing.assert_array_equal(r["out"].reshape(-1), r["h"][-1].reshape(-1))
    Pm = O.Params(W)
    rows = [(b, 0) for b in range(B)]
    for t in checked:
        _teacher_forced(cfg, Pm, r, e, t, rows, cache=oc[t])
        del oc[t]
    _free_running(cfg, W, e, h0, r, seqs=free, cache=ocf, state_tol=free_running_tol(L))
