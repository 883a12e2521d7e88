"""Plain fp64 CPU oracle of the looped Recurrent Block forward.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It
shares no code with the HIP path and the HIP path never calls it.

It computes the block step by step in the order the pages give, in float64,
with NumPy's matmul as the only library primitive and explicit decisions.
Where floating point decides an integer (the router's top-k, the ACT halting
test) the decision is taken in float32, the precision the kernels decide in.

Pages cited (title, then section):
  [ZS] "OpenMythos 분석: Mythos Preview의 장기 추론 성능과 OpenMythos의 계산 모델링"
       (zero.shotlearni.ng)
  [RC] "OpenMythos" (runchr.com, Korean copy of the project README)

Readings of what the pages leave open:
  * h0 = e: the recurrent stage receives the prelude output both as its state
    and as the frozen anchor ([ZS §Core Structure]).
  * loop-index embedding: frequencies theta^(-2j/loop_dim) for
    j < loop_dim/2, sin half then cos half, added to the first loop_dim
    channels of h only; t counts from 0 ([ZS §Repeating the parameter
    reduces expressiveness]).
  * pre-norm block: x1 = c + Attn(RMSNorm(c)), tau = x1 + MoE(RMSNorm(x1)).
  * RMSNorm y = x / sqrt(mean(x^2) + eps) * g.
  * RoPE: adjacent channel pairs rotated as complex numbers by p * theta_i,
    theta_i = base^(-2i/rot_dim), p = start_pos + i ([ZS §RoPE & generation
    cache]).
  * attention: no biases; scale 1/sqrt(d_qk); query head h reads KV head
    floor(h / (H / Hkv)); causal on absolute positions.
  * MLA (DeepSeek-V2 form): RMSNorm on the q and kv latents, per-head
    [nope | rope] for q and k, [nope | v] for the kv up-projection, one
    shared rotated k_rope for all heads; cache = (c_kv before its norm,
    k_rope after RoPE).
  * router: no bias on the linear map; softmax over all experts; top-k on
    logits + router_bias, descending, ties to the lower expert index; gates
    from the unbiased softmax renormalised over the k chosen ([ZS §MoE]).
  * dropless routing; SwiGLU experts without biases; shared experts have the
    routed experts' width and are added with weight 1.
  * depth-wise LoRA acts on the block output with scale row min(t, L-1).
  * A and B are diagonal; rho(A) = max_i A_i.
  * ACT: cum starts at 0; a running position halts at the first loop where
    cum + p >= threshold, or at the last loop, and takes the remainder
    1 - cum as its weight there; every position keeps running the block
    after it halts (halting only zeroes its weight); threshold 0 = ACT off,
    output = final h.
"""

import math

import numpy as np


# --------------------------------------------------------------------------
# dtype helpers
# --------------------------------------------------------------------------

def as_f64(x):
    """Exact upcast: uint16 arrays are bfloat16 bit patterns."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


class Params:
    """Block parameters as float64, upcast on first use.

    ``arrays`` maps names to numpy arrays (bf16 bit patterns or floats).
    Stacked expert tensors may instead come from ``expert_loader(name, e)``,
    so the largest configs never hold every expert in float64 at once.
    """

    def __init__(self, arrays, expert_loader=None):
        self.arrays = arrays
        self.expert_loader = expert_loader
        self._cache = {}

    def __getitem__(self, name):
        if name not in self._cache:
            self._cache[name] = as_f64(self.arrays[name])
        return self._cache[name]

    def expert(self, name, e):
        if name in self.arrays:
            return as_f64(self.arrays[name][e])
        return as_f64(self.expert_loader(name, e))


# --------------------------------------------------------------------------
# single steps
# --------------------------------------------------------------------------

def loop_index_embedding(t, loop_dim, dim, theta):
    """Signal of the loop index t on the first ``loop_dim`` channels.

    [ZS §Repeating the parameter reduces expressiveness]: angles t*freq, the
    sines then the cosines, written into the leading channels and zero
    elsewhere.  Frequencies follow the sinusoidal rule of RoPE, as the
    loop-index hypothesis of [RC] calls it RoPE-like.
    """
    half = loop_dim // 2
    freqs = np.array([theta ** (-2.0 * j / loop_dim) for j in range(half)], dtype=np.float64)
    angles = float(t) * freqs
    emb = np.zeros(dim, dtype=np.float64)
    emb[:half] = np.sin(angles)
    emb[half:loop_dim] = np.cos(angles)
    return emb


def rms_norm(x, g, eps):
    """Root-mean-square normalisation over the last axis, then the gain."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope_cos_sin(positions, rot_dim, theta):
    """cos/sin of p * theta^(-2i/rot_dim) for each position p and pair i."""
    i = np.arange(rot_dim // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / rot_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def apply_rope(x, cos, sin):
    """Rotate adjacent channel pairs (2i, 2i+1) as the complex number
    x[2i] + j x[2i+1] times exp(j * angle) ([ZS §RoPE & generation cache]).

    x: [..., P, rot_dim]; cos, sin: [P, rot_dim/2].
    """
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * cos - x1 * sin
    out[..., 1::2] = x0 * sin + x1 * cos
    return out


def attend(q, k, v, q_pos, k_pos, scale):
    """Explicit causal softmax attention for one head.

    q [Tq, d], k [Tk, d], v [Tk, dv]; key j is visible to query i when
    k_pos[j] <= q_pos[i].
    """
    s = (q @ k.T) * scale
    visible = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]
    s = np.where(visible, s, -np.inf)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return p @ v


def gqa_attention(cfg, P, a, start_pos, cache, rows, kv_state=None):
    """Grouped-query attention with RoPE, output projection included.

    [RC §Attention 구현]: fewer KV heads than query heads, RoPE applied to q
    and k before they are cached.  ``a`` is [B, T, D]; ``rows`` lists the
    (b, i) query rows to produce.  ``cache`` (or None) is a dict with 'k',
    'v' arrays [B, Hkv, capacity, dh] that this call fills at positions
    start_pos .. start_pos+T-1 and then reads from position 0.

    ``kv_state`` (ACT compute skipping, no cache): a dict with 'k', 'v'
    arrays [B, Hkv, T, dh] that persists over the loops of one call.  Only
    the ``rows`` (the positions still running) get new keys and values,
    written into it; every other position keeps the keys and values of the
    last loop it ran.  Attention reads all T positions of it, causally.
    """
    B, T, D = a.shape
    H, G, dh = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    pos = start_pos + np.arange(T)
    cos, sin = rope_cos_sin(pos, dh, cfg["rope_theta"])
    if kv_state is not None:
        bi = np.array(rows)
        ar = a[bi[:, 0], bi[:, 1]]                                  # [M, D]
        kr = (ar @ P["wk"].T).reshape(len(rows), G, dh)
        vr = (ar @ P["wv"].T).reshape(len(rows), G, dh)
        kr = apply_rope(kr.transpose(1, 0, 2), cos[bi[:, 1]], sin[bi[:, 1]]).transpose(1, 0, 2)
        for n, (b, i) in enumerate(rows):
            kv_state["k"][b, :, i] = kr[n]
            kv_state["v"][b, :, i] = vr[n]
        k, v = kv_state["k"], kv_state["v"]
    else:
        k = (a @ P["wk"].T).reshape(B, T, G, dh).transpose(0, 2, 1, 3)
        v = (a @ P["wv"].T).reshape(B, T, G, dh).transpose(0, 2, 1, 3)
        k = apply_rope(k, cos, sin)
    if cache is not None:
        cache["k"][:, :, start_pos:start_pos + T] = k
        cache["v"][:, :, start_pos:start_pos + T] = v
        kk, vv = cache["k"], cache["v"]
        k_pos = np.arange(start_pos + T)
    else:
        kk, vv = k, v
        k_pos = pos
    rep = H // G
    out = {}
    by_b = {}
    for (b, i) in rows:
        by_b.setdefault(b, []).append(i)
    for b, idx in by_b.items():
        idx = np.asarray(idx)
        q = (a[b, idx] @ P["wq"].T).reshape(len(idx), H, dh)
        q = np.stack([apply_rope(q[:, h], cos[idx], sin[idx]) for h in range(H)], axis=1)
        o = np.empty((len(idx), H, dh))
        for h in range(H):
            g = h // rep
            o[:, h] = attend(q[:, h], as_f64(kk[b, g, :len(k_pos)]), as_f64(vv[b, g, :len(k_pos)]),
                             pos[idx], k_pos, 1.0 / math.sqrt(dh))
        y = o.reshape(len(idx), H * dh) @ P["wo"].T
        for n, i in enumerate(idx):
            out[(b, i)] = y[n]
    return out


def mla_attention(cfg, P, a, start_pos, cache, rows):
    """Multi-latent attention (DeepSeek-V2 form) with RoPE on the rope part.

    [ZS §MLA]: the kv down-projection splits into the latent c_kv
    (kv_lora_rank wide) and one k_rope shared by all heads, which is
    rotated; c_kv and k_rope are what the cache holds; k_nope and v are
    rebuilt from c_kv.  Queries go through the q latent (q_lora_rank).
    """
    B, T, D = a.shape
    H = cfg["n_heads"]
    kvl, rope, nope, vd = cfg["kv_lora_rank"], cfg["qk_rope_head_dim"], cfg["qk_nope_head_dim"], cfg["v_head_dim"]
    eps = cfg["norm_eps"]
    pos = start_pos + np.arange(T)
    cos, sin = rope_cos_sin(pos, rope, cfg["rope_theta"])
    kv_raw = a @ P["wdkv"].T                       # [B, T, kvl + rope]
    c_kv = kv_raw[..., :kvl]
    k_rope = apply_rope(kv_raw[..., kvl:], cos, sin)
    if cache is not None:
        cache["c_kv"][:, start_pos:start_pos + T] = c_kv
        cache["k_rope"][:, start_pos:start_pos + T] = k_rope
        all_ckv = as_f64(cache["c_kv"][:, :start_pos + T])
        all_kr = as_f64(cache["k_rope"][:, :start_pos + T])
        k_pos = np.arange(start_pos + T)
    else:
        all_ckv, all_kr, k_pos = c_kv, k_rope, pos
    kv = (rms_norm(all_ckv, P["gkv"], eps) @ P["wukv"].T).reshape(B, len(k_pos), H, nope + vd)
    out = {}
    by_b = {}
    for (b, i) in rows:
        by_b.setdefault(b, []).append(i)
    for b, idx in by_b.items():
        idx = np.asarray(idx)
        c_q = rms_norm(a[b, idx] @ P["wdq"].T, P["gq"], eps)
        q = (c_q @ P["wuq"].T).reshape(len(idx), H, nope + rope)
        o = np.empty((len(idx), H, vd))
        for h in range(H):
            qh = np.concatenate([q[:, h, :nope], apply_rope(q[:, h, nope:], cos[idx], sin[idx])], axis=-1)
            kh = np.concatenate([kv[b, :, h, :nope], all_kr[b]], axis=-1)
            o[:, h] = attend(qh, kh, kv[b, :, h, nope:], pos[idx], k_pos, 1.0 / math.sqrt(nope + rope))
        y = o.reshape(len(idx), H * vd) @ P["wo"].T
        for n, i in enumerate(idx):
            out[(b, i)] = y[n]
    return out


def topk_desc_lowest_index(values, k):
    """Indices of the k largest entries per row, largest first, equal values
    ordered by ascending index (a stable sort of the negated values)."""
    return np.argsort(-values, axis=-1, kind="stable")[:, :k]


def router(cfg, P, f):
    """Top-k softmax router with a selection-only bias ([ZS §MoE]).

    Returns logits z (float64), the chosen experts (an ordered list,
    largest first), their renormalised gates, and the float64 decision
    margin: the smallest gap between consecutive values among the k+1
    largest biased logits, since a near-tie anywhere there (inside the
    top-k order or at its edge) makes two answers correct.  The choice
    itself is made on float32 logits + float32 bias, as the kernel makes it.
    """
    k = cfg["top_k"]
    z = f @ P["router_w"].T                                   # [n, E]
    s = np.exp(z - z.max(axis=-1, keepdims=True))
    s = s / s.sum(axis=-1, keepdims=True)
    bias32 = np.asarray(P.arrays["router_bias"], dtype=np.float32)
    biased32 = (z.astype(np.float32) + bias32).astype(np.float32)
    sel = topk_desc_lowest_index(biased32, k)
    gate = np.take_along_axis(s, sel, axis=-1)
    gate = gate / gate.sum(axis=-1, keepdims=True)
    b64 = z + bias32.astype(np.float64)
    srt = -np.sort(-b64, axis=-1)
    top = srt[:, :min(k + 1, b64.shape[1])]
    margin = np.min(top[:, :-1] - top[:, 1:], axis=-1) if top.shape[1] > 1 else np.full(len(z), np.inf)
    return z, sel, gate, margin


def silu(x):
    return x / (1.0 + np.exp(-x))


def swiglu(x, wg, wu, wd):
    """Expert feed-forward: down( silu(gate x) * (up x) ), no biases."""
    return (silu(x @ wg.T) * (x @ wu.T)) @ wd.T


def moe_ffn(cfg, P, f, sel, gate):
    """Routed experts weighted by their gates, plus the shared experts.

    f [n, D]; sel, gate [n, k].  Each routed expert runs on exactly the rows
    that chose it (dropless); shared experts run on every row.
    """
    n, D = f.shape
    y = np.zeros((n, D))
    for e in range(cfg["n_experts"]):
        hit = np.nonzero(sel == e)
        if len(hit[0]) == 0:
            continue
        r, j = hit
        out = swiglu(f[r], P.expert("w_gate", e), P.expert("w_up", e), P.expert("w_down", e))
        y[r] += gate[r, j][:, None] * out
    for s in range(cfg["n_shared_experts"]):
        y += swiglu(f, P.expert("s_gate", s), P.expert("s_up", s), P.expert("s_down", s))
    return y


def depthwise_lora(cfg, P, x, t):
    """Loop-dependent low-rank term: (down(x) * scale[t']) @ B_lora, with the
    scale row t' = min(t, max_loop_iters-1) ([ZS §Repeating the parameter
    reduces expressiveness])."""
    ti = min(t, cfg["max_loop_iters"] - 1)
    return ((x @ P["lora_down"].T) * P["lora_scale"][ti]) @ P["lora_B"]


def lti_A(P):
    """Diagonal of A = exp(-exp(clamp(log_dt + log_A, -20, 20))), every entry
    in (0, 1) ([ZS §latent reasoning]; [RC §해결책])."""
    return np.exp(-np.exp(np.clip(P["log_dt"][0] + P["log_A"], -20.0, 20.0)))


def lti_injection(P, h, e, trans_out):
    """h_next = A*h + B*e + Transformer(h, e) ([RC §아키텍처])."""
    return lti_A(P) * h + P["B"] * e + trans_out


def halting_probability(P, h):
    """p = sigmoid(h . w_halt + b_halt) per position ([ZS §ACT])."""
    z = h @ P["halt_w"] + P["halt_b"][0]
    return 1.0 / (1.0 + np.exp(-z))


# --------------------------------------------------------------------------
# one loop and the full loop
# --------------------------------------------------------------------------

def act_halts(cum32, running, p, t, n_loops, threshold):
    """Positions that halt at loop t ([ZS §ACT]): running ones whose
    cumulative halting probability reaches the threshold (the running sum
    and the comparison in float32, as the kernel keeps them), and every
    running one at the last loop."""
    p32 = np.asarray(p).astype(np.float32)
    reach = (cum32 + p32).astype(np.float32) >= np.float32(threshold)
    return running & (reach | (t == n_loops - 1))


def act_weights(cum, running, p, halt_now):
    """Weight of this loop's state in the output: the remainder 1 - cum on
    the halting loop, p on earlier loops, 0 once halted."""
    return np.where(halt_now, np.maximum(1.0 - cum, 0.0), p) * running


def run_loop(cfg, P, h, e, t, start_pos=0, cache=None, rows=None, route_hook=None, kv_state=None):
    """One pass of the recurrent block at loop index t ([ZS §Recurrent Block]).

    h, e: [B, T, D] float64.  Returns the new state for ``rows`` (all rows
    when None) and the intermediates callers check.  ``route_hook(sel,
    margin, rows)`` may return a replacement expert choice (used by the
    tie-adoption protocol); the gates are then taken for that choice.
    ``kv_state``: see gqa_attention (ACT compute skipping).
    """
    B, T, D = h.shape
    eps = cfg["norm_eps"]
    if rows is None:
        rows = [(b, i) for b in range(B) for i in range(T)]
    u = h + loop_index_embedding(t, cfg["loop_dim"], D, cfg["loop_theta"])
    c = rms_norm(u + e, P["g_rec"], eps)
    a = rms_norm(c, P["g_attn"], eps)
    attn = gqa_attention if cfg["attn"] == "gqa" else mla_attention
    if kv_state is not None:
        if cfg["attn"] != "gqa" or cache is not None:
            raise NotImplementedError("ACT compute skipping is defined for GQA without a cache")
        o = gqa_attention(cfg, P, a, start_pos, None, rows, kv_state=kv_state)
    else:
        o = attn(cfg, P, a, start_pos, cache, rows)
    ridx = tuple(np.array(rows).T)
    x1 = c[ridx] + np.stack([o[r] for r in rows])
    f = rms_norm(x1, P["g_ffn"], eps)
    z, sel, gate, margin = router(cfg, P, f)
    if route_hook is not None:
        new_sel = route_hook(sel, margin, rows)
        if new_sel is not None and not np.array_equal(new_sel, sel):
            sel = np.asarray(new_sel)
            s = np.exp(z - z.max(axis=-1, keepdims=True))
            s = s / s.sum(axis=-1, keepdims=True)
            gate = np.take_along_axis(s, sel, axis=-1)
            gate = gate / gate.sum(axis=-1, keepdims=True)
    tau = x1 + moe_ffn(cfg, P, f, sel, gate)
    tau = tau + depthwise_lora(cfg, P, tau, t)
    h_new = lti_injection(P, h[ridx], e[ridx], tau)
    return dict(h=h_new, rows=rows, sel=sel, gate=gate, margin=margin, z=z, f=f, x1=x1, c=c, a=a)


def new_cache(cfg, batch, capacity, n_loops):
    """Empty per-loop caches (float64), one per loop index."""
    if cfg["attn"] == "gqa":
        G, dh = cfg["n_kv_heads"], cfg["head_dim"]
        return [dict(k=np.zeros((batch, G, capacity, dh)), v=np.zeros((batch, G, capacity, dh)))
                for _ in range(n_loops)]
    return [dict(c_kv=np.zeros((batch, capacity, cfg["kv_lora_rank"])),
                 k_rope=np.zeros((batch, capacity, cfg["qk_rope_head_dim"])))
            for _ in range(n_loops)]


class Adoption:
    """Decisions recorded by another implementation, taken where the
    oracle's own decision is within rounding of a tie.

    sel: [n_loops, N, k] chosen experts; halt_counts: [N] 1-based halting
    loop.  A router choice is adopted where the oracle's top-k margin is
    below eps_route; a halting decision where |cum + p - threshold| is
    below eps_halt.  Everything else must agree, and is counted when not.
    """

    def __init__(self, sel=None, halt_counts=None, eps_route=0.0, eps_halt=0.0):
        self.sel = sel
        self.halt_counts = halt_counts
        self.eps_route = eps_route
        self.eps_halt = eps_halt
        self.route_adopted = 0
        self.route_disagree = 0
        self.halt_adopted = 0
        self.halt_disagree = 0
        self.disagree_rows = []     # (loop, row, oracle margin) of route disagreements


def recurrent_forward(cfg, P, e, h0, n_loops, act_threshold, start_pos=0, cache=None,
                      adopt=None, record=False, stop_when_halted=True, on_loop=None):
    """The looped Recurrent Block ([ZS §Recurrent Block]; [RC §아키텍처]).

    e, h0: [B, T, D].  Returns dict(out=[B, T, D] float64, halt_counts=[B, T]
    int, loops_run, and per-loop records when ``record``).  With
    act_threshold == 0 the output is the final state; otherwise the
    ACT-weighted sum of the states, and the loop stops once every position
    has halted (nothing returned can change after that) unless a cache is
    being filled or ``stop_when_halted`` is False.  ``on_loop(t, state)``,
    when given, is called after each loop with the new state (progress
    reports of long runs; it cannot change anything).
    """
    e = as_f64(e)
    h = as_f64(h0)
    B, T, D = h.shape
    N = B * T
    act = act_threshold > 0
    thr32 = np.float32(act_threshold)
    h_out = np.zeros_like(h)
    cum = np.zeros(N)
    cum32 = np.zeros(N, dtype=np.float32)
    halted = np.zeros(N, dtype=bool)
    counts = np.full(N, n_loops, dtype=np.int64)
    rec = dict(h=[], sel=[], margin=[], p=[], weight=[])
    for t in range(n_loops):
        hook = None
        if adopt is not None and adopt.sel is not None:
            gpu = np.asarray(adopt.sel[t]).reshape(N, -1)

            def hook(sel, margin, rows, gpu=gpu, t=t):
                out = sel.copy()
                for n in range(len(rows)):
                    if not np.array_equal(sel[n], gpu[n]):
                        if margin[n] < adopt.eps_route:
                            out[n] = gpu[n]
                            adopt.route_adopted += 1
                        else:
                            adopt.route_disagree += 1
                            adopt.disagree_rows.append((t, n, float(margin[n])))
                return out
        step = run_loop(cfg, P, h, e, t, start_pos, None if cache is None else cache[t], route_hook=hook)
        h = step["h"].reshape(B, T, D)
        if act:
            p = halting_probability(P, h.reshape(N, D))
            p32 = p.astype(np.float32)
            running = ~halted
            halt_now = act_halts(cum32, running, p, t, n_loops, act_threshold)
            if adopt is not None and adopt.halt_counts is not None:
                gpu_halt = np.asarray(adopt.halt_counts).reshape(N) == t + 1
                near = running & (np.abs((cum32 + p32).astype(np.float64) - float(thr32)) < adopt.eps_halt) \
                    & (t != n_loops - 1)
                diff = running & (gpu_halt != halt_now)
                adopt.halt_adopted += int(np.sum(diff & near))
                adopt.halt_disagree += int(np.sum(diff & ~near))
                halt_now = np.where(near, gpu_halt & running, halt_now)
            weight = act_weights(cum, running, p, halt_now)
            h_out += weight.reshape(B, T, 1) * h
            cum = cum + p * running
            cum32 = np.where(running, (cum32 + p32).astype(np.float32), cum32)
            counts[halt_now] = t + 1
            halted |= halt_now
            if record:
                rec["p"].append(p)
                rec["weight"].append(weight)
        if record:
            rec["h"].append(h.copy())
            rec["sel"].append(step["sel"].copy())
            rec["margin"].append(step["margin"].copy())
        loops_run = t + 1
        if on_loop is not None:
            on_loop(t, h)
        if act and stop_when_halted and cache is None and halted.all():
            break
    out = h_out if act else h
    res = dict(out=out, halt_counts=counts.reshape(B, T), state=h, loops_run=loops_run)
    if record:
        res["record"] = rec
    return res


def recurrent_forward_act_skip(cfg, P, e, h0, n_loops, act_threshold, adopt=None, record=False, on_loop=None):
    """ACT with compute skipping: a position that has halted leaves the
    batch ([GN §6], continuous depth-wise batching: halted tokens stop
    taking compute).

    Reading of what the pages leave open: a halted position's state is
    frozen (its output is already complete), it is not run again, and in
    later loops the other positions attend to the keys and values it had in
    the last loop it ran (its K/V freeze with it).  Everything else is the
    rule of ``recurrent_forward``: the same block, the same ACT weights and
    halt counts, threshold in (0, 1], GQA, no cache.

    ``adopt`` (an Adoption with per-loop expert choices [n_loops, N, k]
    indexed by position and halt counts [N]) takes another implementation's
    decisions where the oracle's own are within its tie margins.  Returns
    dict(out, halt_counts, loops_run[, record]).
    """
    if act_threshold <= 0:
        raise ValueError("compute skipping needs ACT on")
    e = as_f64(e)
    h = as_f64(h0).copy()
    B, T, D = h.shape
    N = B * T
    G, dh = cfg["n_kv_heads"], cfg["head_dim"]
    kv = dict(k=np.zeros((B, G, T, dh)), v=np.zeros((B, G, T, dh)))
    thr32 = np.float32(act_threshold)
    hf = h.reshape(N, D)
    h_out = np.zeros((N, D))
    cum = np.zeros(N)
    cum32 = np.zeros(N, dtype=np.float32)
    halted = np.zeros(N, dtype=bool)
    counts = np.full(N, n_loops, dtype=np.int64)
    rec = dict(sel=[], p=[], running=[])
    loops_run = 0
    for t in range(n_loops):
        run_idx = np.nonzero(~halted)[0]
        if len(run_idx) == 0:
            break
        rows = [(int(n) // T, int(n) % T) for n in run_idx]
        hook = None
        if adopt is not None and adopt.sel is not None:
            gpu = np.asarray(adopt.sel[t]).reshape(N, -1)

            def hook(sel, margin, rr, gpu=gpu, t=t, run_idx=run_idx):
                out = sel.copy()
                for m in range(len(rr)):
                    want = gpu[run_idx[m]]
                    if not np.array_equal(sel[m], want):
                        if margin[m] < adopt.eps_route:
                            out[m] = want
                            adopt.route_adopted += 1
                        else:
                            adopt.route_disagree += 1
                            adopt.disagree_rows.append((t, int(run_idx[m]), float(margin[m])))
                return out
        step = run_loop(cfg, P, hf.reshape(B, T, D), e, t, rows=rows, route_hook=hook, kv_state=kv)
        hr = step["h"]
        hf[run_idx] = hr
        p = halting_probability(P, hr)
        p32 = p.astype(np.float32)
        sub_cum32 = cum32[run_idx]
        running = np.ones(len(run_idx), dtype=bool)
        halt_now = act_halts(sub_cum32, running, p, t, n_loops, act_threshold)
        if adopt is not None and adopt.halt_counts is not None:
            gpu_halt = np.asarray(adopt.halt_counts).reshape(N)[run_idx] == t + 1
            near = (np.abs((sub_cum32 + p32).astype(np.float64) - float(thr32)) < adopt.eps_halt) & \
                (t != n_loops - 1)
            diff = gpu_halt != halt_now
            adopt.halt_adopted += int(np.sum(diff & near))
            adopt.halt_disagree += int(np.sum(diff & ~near))
            halt_now = np.where(near, gpu_halt, halt_now)
        weight = act_weights(cum[run_idx], running, p, halt_now)
        h_out[run_idx] += weight[:, None] * hr
        cum[run_idx] += p
        cum32[run_idx] = (sub_cum32 + p32).astype(np.float32)
        counts[run_idx[halt_now]] = t + 1
        halted[run_idx[halt_now]] = True
        loops_run = t + 1
        if record:
            rec["sel"].append((run_idx.copy(), step["sel"].copy()))
            rec["p"].append((run_idx.copy(), p))
            rec["running"].append(run_idx.copy())
        if on_loop is not None:
            on_loop(t, hf.reshape(B, T, D))
    res = dict(out=h_out.reshape(B, T, D), halt_counts=counts.reshape(B, T), state=hf.reshape(B, T, D),
               loops_run=loops_run)
    if record:
        res["record"] = rec
    return res


# --------------------------------------------------------------------------
# the whole model around the recurrent stage
# --------------------------------------------------------------------------

def dense_hidden(cfg):
    """Hidden width of the prelude / coda feed-forward: the dense SwiGLU
    expert of width dim * 4 // 3 ([ZS §MoE]: only the recurrent block's FFN
    is a MoE)."""
    return cfg["dim"] * 4 // 3


class LayerParams:
    """The weights of one prelude or coda layer under the names the
    attention functions read ("wq", "wk", ...), stored as ``prefix + name``."""

    def __init__(self, P, prefix):
        self.P = P
        self.prefix = prefix
        self.arrays = {k[len(prefix):]: v for k, v in P.arrays.items() if k.startswith(prefix)}

    def __getitem__(self, name):
        return self.P[self.prefix + name]


def dense_layer(cfg, LP, x, start_pos=0, cache=None):
    """One prelude / coda layer: the pre-norm Transformer block with a dense
    SwiGLU feed-forward ([ZS §MoE]), x1 = x + Attn(RMSNorm(x)),
    out = x1 + FFN(RMSNorm(x1)).  x: [B, T, D]; ``cache`` is this layer's
    cache (or None) as in recurrent_forward."""
    B, T, D = x.shape
    eps = cfg["norm_eps"]
    rows = [(b, i) for b in range(B) for i in range(T)]
    a = rms_norm(x, LP["attn_norm"], eps)
    attn = gqa_attention if cfg["attn"] == "gqa" else mla_attention
    o = attn(cfg, LP, a, start_pos, cache, rows)
    x1 = x.reshape(B * T, D) + np.stack([o[r] for r in rows])
    f = rms_norm(x1, LP["ffn_norm"], eps)
    return (x1 + swiglu(f, LP["w1"], LP["w3"], LP["w2"])).reshape(B, T, D)


def new_model_cache(cfg, batch, capacity, n_loops):
    """Caches of every layer of the model: one per prelude layer, one per
    loop of the recurrent stage, one per coda layer ([ZS §Core Structure]:
    each layer and loop has its own cache key)."""
    one = lambda: new_cache(cfg, batch, capacity, 1)[0]
    return dict(prelude=[one() for _ in range(cfg["prelude_layers"])],
                loops=new_cache(cfg, batch, capacity, n_loops),
                coda=[one() for _ in range(cfg["coda_layers"])])


def model_forward(cfg, P, ids, n_loops, act_threshold, start_pos=0, cache=None, adopt=None):
    """The model forward of [ZS §Core Structure]: token embedding, the
    prelude layers, e = x frozen as the anchor, the recurrent stage with
    h0 = e, the coda layers, the final RMSNorm and the LM head.

    ids: [B, T] ints.  ``adopt`` is passed to the recurrent stage (see
    recurrent_forward).  Returns (logits [B, T, vocab] float64, the
    recurrent stage's result dict)."""
    x = P["embed"][np.asarray(ids)]
    for i in range(cfg["prelude_layers"]):
        x = dense_layer(cfg, LayerParams(P, f"prelude_{i}."), x, start_pos,
                        None if cache is None else cache["prelude"][i])
    e = x
    r = recurrent_forward(cfg, P, e, e, n_loops, act_threshold, start_pos=start_pos,
                          cache=None if cache is None else cache["loops"], adopt=adopt)
    x = r["out"]
    for i in range(cfg["coda_layers"]):
        x = dense_layer(cfg, LayerParams(P, f"coda_{i}."), x, start_pos,
                        None if cache is None else cache["coda"][i])
    x = rms_norm(x, P["final_norm"], cfg["norm_eps"])
    return x @ P["head"].T, r


def argmax_lowest(v):
    """Index of the largest entry of each row, the lowest index on ties, and
    the gap to the runner-up (the decision margin)."""
    v = np.asarray(v, dtype=np.float64)
    idx = np.argmax(v, axis=-1)                      # first maximum
    top = np.take_along_axis(v, idx[..., None], -1)[..., 0]
    rest = v.copy()
    np.put_along_axis(rest, idx[..., None], -np.inf, -1)
    return idx, top - rest.max(axis=-1)


def generate(cfg, P, ids, max_new, n_loops, act_threshold, choose=None):
    """Greedy decoding with per-layer caches ([ZS §RoPE & generation cache]):
    step 0 feeds the whole prompt at start_pos 0, every later step only the
    last token at start_pos = prompt_len + step - 1; the next token is the
    argmax of the last position's logits (lowest index on ties; the pages
    show no sampling rule).  ``choose(step, idx, margin)``, when given, may
    replace the choice (the tie-adoption protocol of the tests).  Returns the
    [B, prompt_len + max_new] token array."""
    ids = np.asarray(ids)
    B, T0 = ids.shape
    cache = new_model_cache(cfg, B, T0 + max_new, n_loops)
    out = ids.copy()
    for step in range(max_new):
        cur, sp = (ids, 0) if step == 0 else (out[:, -1:], T0 + step - 1)
        logits, _ = model_forward(cfg, P, cur, n_loops, act_threshold, start_pos=sp, cache=cache)
        idx, margin = argmax_lowest(logits[:, -1])
        if choose is not None:
            idx = choose(step, idx, margin)
        out = np.concatenate([out, np.asarray(idx).reshape(B, 1)], axis=1)
    return out
