"""fp64 CPU oracle of the gradient of the looped Recurrent Block (GQA).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It
shares no code with the HIP path and the HIP path never calls it.

What it computes: for a seeded upstream gradient dy of the recurrent
stage's output, the vector-Jacobian product of ``rdt_oracle.recurrent_forward``
with respect to every trained tensor of the block, the anchor e and the
initial state h0.  The forward is written a second time here in PyTorch
float64 (the same steps as ``rdt_oracle.run_loop`` and its callers) so that
autograd, the library primitive this module leans on, can differentiate it.

Pages cited (title, then section):
  [ZS] "OpenMythos 분석: Mythos Preview의 장기 추론 성능과 OpenMythos의 계산 모델링"
       (zero.shotlearni.ng)

Readings of what the pages leave open:
  * The block has discrete decisions: the router's top-k and the ACT halting
    loop.  The gradient is that of the smooth piece of the output the forward
    took, with the expert choice of every (loop, position) and the halting
    loop of every position held at the forward's values (the router bias,
    which only enters the choice, gets no gradient -- which is why the pages
    speak of a separate balancing rule for it, [ZS §MoE]).
  * ACT: the weight of the halting loop is max(1 - cum, 0) with cum the
    float64 sum of the earlier p, so its gradient flows into every earlier p
    of that position; the loops after the last halt are not run.
  * Router-bias balancing ([ZS §MoE] notes the selection-only bias and that
    nothing updates it; the rule of aux-loss-free balancing is taken): after
    a step, each expert's bias moves by gamma towards balance,
    b_i <- b_i + gamma * sign(mean_load - load_i), with load_i the number of
    (position, slot) assignments to expert i summed over the step's loops
    and sign(0) = 0; the sum is formed in float32, the bias's storage type.
  * Optimizer ([ZS §Tokenizer & training script]: the training script uses
    AdamW): decoupled weight decay (Loshchilov & Hutter) with bias-corrected
    moments, applied to every trained tensor with the same hyper-parameters,
    on float32 master weights; the block's matrices are the masters rounded
    to bfloat16 (nearest, ties to even).
"""

import numpy as np
import torch

from . import rdt_oracle as O

# trained tensors of the GQA block, in the order gradients are reported
GRAD_NAMES = ("g_rec", "g_attn", "g_ffn", "wq", "wk", "wv", "wo", "router_w", "w_gate", "w_up", "w_down",
              "s_gate", "s_up", "s_down", "lora_down", "lora_B", "lora_scale", "log_A", "log_dt", "B",
              "halt_w", "halt_b")


def _leaves(cfg, P):
    """Every trained tensor as a float64 leaf that records its gradient."""
    out = {}
    for name in GRAD_NAMES:
        if name.startswith("s_") and cfg["n_shared_experts"] == 0:
            continue
        out[name] = torch.from_numpy(np.ascontiguousarray(P[name], dtype=np.float64)).requires_grad_(True)
    return out


def _rms(x, g, eps):
    return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + eps) * g


def _rope(x, cos, sin):
    """Adjacent pairs (2i, 2i+1) rotated as complex numbers ([ZS §RoPE &
    generation cache]); x [..., T, d], cos/sin [T, d/2]."""
    x0, x1 = x[..., 0::2], x[..., 1::2]
    return torch.stack([x0 * cos - x1 * sin, x0 * sin + x1 * cos], dim=-1).flatten(-2)


def _swiglu(x, wg, wu, wd):
    g = x @ wg.T
    return (g * torch.sigmoid(g) * (x @ wu.T)) @ wd.T


def _loop(cfg, W, h, e, t, sel, cos, sin):
    """One pass of the block at loop t with the expert choice ``sel`` [N, k]
    fixed; h, e [B, T, D].  Same steps as rdt_oracle.run_loop (GQA, every
    position, no cache)."""
    B, T, D = h.shape
    N = B * T
    eps = cfg["norm_eps"]
    H, G, dh = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    emb = torch.from_numpy(O.loop_index_embedding(t, cfg["loop_dim"], D, cfg["loop_theta"]))
    c = _rms(h + emb + e, W["g_rec"], eps)
    a = _rms(c, W["g_attn"], eps)
    q = _rope((a @ W["wq"].T).reshape(B, T, H, dh).transpose(1, 2), cos, sin)      # [B, H, T, dh]
    k = _rope((a @ W["wk"].T).reshape(B, T, G, dh).transpose(1, 2), cos, sin)      # [B, G, T, dh]
    v = (a @ W["wv"].T).reshape(B, T, G, dh).transpose(1, 2)
    rep = H // G
    k = k.repeat_interleave(rep, dim=1)
    v = v.repeat_interleave(rep, dim=1)
    s = (q @ k.transpose(-1, -2)) / np.sqrt(dh)
    causal = torch.ones(T, T, dtype=torch.bool).tril()
    s = s.masked_fill(~causal, float("-inf"))
    o = torch.softmax(s, dim=-1) @ v                                                 # [B, H, T, dh]
    x1 = c.reshape(N, D) + o.transpose(1, 2).reshape(N, H * dh) @ W["wo"].T
    f = _rms(x1, W["g_ffn"], eps)
    scores = torch.softmax(f @ W["router_w"].T, dim=-1)
    sel_t = torch.from_numpy(np.asarray(sel, dtype=np.int64))
    gate = scores.gather(1, sel_t)
    gate = gate / gate.sum(-1, keepdim=True)
    y = torch.zeros(N, D, dtype=torch.float64)
    for ex in range(cfg["n_experts"]):
        r, j = np.nonzero(np.asarray(sel) == ex)
        if len(r) == 0:
            continue
        r_t = torch.from_numpy(r)
        out = _swiglu(f[r_t], W["w_gate"][ex], W["w_up"][ex], W["w_down"][ex])
        y = y.index_add(0, r_t, gate[r_t, torch.from_numpy(j)][:, None] * out)
    for si in range(cfg["n_shared_experts"]):
        y = y + _swiglu(f, W["s_gate"][si], W["s_up"][si], W["s_down"][si])
    tau = x1 + y
    ti = min(t, cfg["max_loop_iters"] - 1)
    tau = tau + ((tau @ W["lora_down"].T) * W["lora_scale"][ti]) @ W["lora_B"]
    A = torch.exp(-torch.exp(torch.clamp(W["log_dt"][0] + W["log_A"], -20.0, 20.0)))
    return (A * h.reshape(N, D) + W["B"] * e.reshape(N, D) + tau).reshape(B, T, D)


def forward_fixed(cfg, P, e, h0, n_loops, act_threshold, sel_loops, halt_counts, W=None):
    """The recurrent stage's output with every decision given.

    sel_loops [>= loops run, N, k] expert choices; halt_counts [N] the
    1-based halting loop (ignored with ACT off).  Returns (out [B, T, D]
    torch float64, the leaves dict)."""
    if cfg["attn"] != "gqa":
        raise NotImplementedError("the gradient oracle covers GQA attention")
    W = _leaves(cfg, P) if W is None else W
    e_t = e if torch.is_tensor(e) else torch.from_numpy(O.as_f64(e))
    h = h0 if torch.is_tensor(h0) else torch.from_numpy(O.as_f64(h0))
    B, T, D = h.shape
    N = B * T
    cos, sin = (torch.from_numpy(x) for x in O.rope_cos_sin(np.arange(T), cfg["head_dim"], cfg["rope_theta"]))
    act = act_threshold > 0
    hc = np.asarray(halt_counts).reshape(N) if act else None
    loops = int(hc.max()) if act else n_loops
    out = torch.zeros(N, D, dtype=torch.float64)
    cum = torch.zeros(N, dtype=torch.float64)
    for t in range(loops):
        h = _loop(cfg, W, h, e_t, t, np.asarray(sel_loops[t]).reshape(N, -1), cos, sin)
        if act:
            hf = h.reshape(N, D)
            p = torch.sigmoid(hf @ W["halt_w"] + W["halt_b"][0])
            running = torch.from_numpy(hc > t)
            now = torch.from_numpy(hc == t + 1)
            w = torch.where(now, torch.clamp(1.0 - cum, min=0.0), p)
            w = torch.where(running, w, torch.zeros_like(w))
            out = out + w[:, None] * hf
            cum = cum + torch.where(running, p, torch.zeros_like(p))
    if not act:
        out = h.reshape(N, D)
    return out.reshape(B, T, D), W


def recurrent_grad(cfg, P, e, h0, n_loops, act_threshold, sel_loops, halt_counts, dy):
    """Gradients of sum(dy * out) ([ZS §Recurrent Block] forward, decisions
    fixed).  Returns dict name -> float64 array (every trained tensor, plus
    "e" and "h0"), and "out"."""
    e_t = torch.from_numpy(O.as_f64(e)).requires_grad_(True)
    h_t = torch.from_numpy(O.as_f64(h0)).requires_grad_(True)
    out, W = forward_fixed(cfg, P, e_t, h_t, n_loops, act_threshold, sel_loops, halt_counts)
    loss = (out * torch.from_numpy(np.asarray(dy, dtype=np.float64))).sum()
    loss.backward()
    g = {name: (leaf.grad.numpy().copy() if leaf.grad is not None else np.zeros(leaf.shape))
         for name, leaf in W.items()}
    g["e"] = e_t.grad.numpy().copy()
    g["h0"] = h_t.grad.numpy().copy()
    g["out"] = out.detach().numpy().copy()
    return g


def expert_load(sel_loops, n_experts):
    """(position, slot) assignments per expert, summed over the loops."""
    return np.bincount(np.asarray(sel_loops).reshape(-1), minlength=n_experts).astype(np.int64)


def router_bias_update(bias, load, gamma):
    """Aux-loss-free balancing step: each expert's selection bias moves by
    gamma up when its load is below the mean, down when above, not at all
    when equal; float32 arithmetic, as the bias is stored."""
    load = np.asarray(load, dtype=np.int64)
    E = len(load)
    direction = np.sign(load.sum() - E * load)          # sign(mean - load_i), exact in integers
    return (np.asarray(bias, dtype=np.float32) + np.float32(gamma) * direction.astype(np.float32)).astype(np.float32)


def adamw_step(param, grad, m, v, step, lr, beta1, beta2, eps, weight_decay):
    """One AdamW step (1-based step count): moments m, v updated with grad,
    bias-corrected, and param <- param - lr (m_hat / (sqrt(v_hat) + eps) +
    weight_decay param), the decay on the value before the step.  Returns
    (param, m, v) as float64."""
    param, grad = np.asarray(param, dtype=np.float64), np.asarray(grad, dtype=np.float64)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * grad
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * grad * grad
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    return param - lr * (m_hat / (np.sqrt(v_hat) + eps) + weight_decay * param), m, v


def round_bf16(x):
    """float32 values rounded to bfloat16 bit patterns (nearest, ties to
    even; NaN stays NaN)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    return np.where(nan, np.uint16(0x7FC0), r)
