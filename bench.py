"""Benchmark of the looped Recurrent-Block forward on one MI355X.

Workload (default): the mythos_3b-shaped block, bf16 prefill, batch 2 x
4096 tokens, 16 loops, ACT at 0.99, synthetic seeded weights and inputs
(workloads.generate).  A step is one rdt_recurrent_forward call: every loop
of the whole block over the batch.  Inputs are resident in HBM before the
timed region.

Prints ONE JSON line: token*loops/s, the roofline of the dominant kernel
(routed expert gate|up grouped GEMM, timed live with HIP events recorded by
the library on the launch stream) and the fp64 CPU oracle timed on a bounded
sample of the same workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config mythos_3b]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "recurrent-block token·loops/sec (1 GPU) + % bf16 MFMA peak / % HBM peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
# the training step's optimizer: AdamW hyper-parameters and the router-bias
# balancing rate
OPT_HP = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
OPT_BIAS_GAMMA = 1e-3
# token-loops/s each workload would reach at the spec peaks: per loop the
# larger of its MFMA time (algorithmic flops) and its HBM time (touched
# expert weights once + the other tensors once per fused kernel)
ROOFLINE_TOKEN_LOOPS = {"mythos_1b": 10.9e6, "mythos_3b": 6.26e6, "mythos_10b_decode": 30.8e3}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def stage_work(cfg, touched=None):
    """Algorithmic flops and bytes of one launch of each stage (per loop).
    Expert weight bytes count the experts that received rows (``touched``,
    all of them when None)."""
    B, T, D = cfg["batch"], cfg["seq"], cfg["dim"]
    N = B * T
    H, G, dh, E, F, k, S = (cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["n_experts"],
                            cfg["expert_dim"], cfg["top_k"], cfg["n_shared_experts"])
    sp = cfg["start_pos"]
    NK = N * k
    es = 2.0 if cfg["dtype"] == "bf16" else 4.0   # stored width of matrix-product outputs
    Et = E if touched is None else touched
    w = {}
    w["qkv"] = dict(flops=2.0 * N * D * (H + 2 * G) * dh)
    w["attention"] = dict(flops=4.0 * B * H * dh * sum(sp + i + 1 for i in range(T)))
    w["o_proj"] = dict(flops=2.0 * N * D * H * dh)
    w["router"] = dict(flops=2.0 * N * D * E)
    w["expert_gate_up"] = dict(flops=2.0 * NK * 2 * F * D, bytes=2.0 * Et * 2 * F * D + 2.0 * NK * D + 2.0 * NK * F)
    w["expert_down"] = dict(flops=2.0 * NK * F * D, bytes=2.0 * Et * F * D + 2.0 * NK * F + es * NK * D)
    w["shared_gate_up"] = dict(flops=2.0 * N * 2 * F * D * S)
    w["shared_down"] = dict(flops=2.0 * N * F * D * S)
    # row-wise kernels: each tensor read / written once at its stored width
    w["loop_head"] = dict(bytes=N * D * (4 + 4 + 4 + 2))             # h, e in; c fp32, a bf16 out
    w["ffn_norm"] = dict(bytes=N * D * (4 + 2))                       # x1 in, f out
    w["tail"] = dict(bytes=N * D * (4 + es * k + es * S + 4 + 4 + 4 + 4))   # x1, y (k rows), y_s, h, e in; h, h_out
    return w


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic_per_kernel_{}_prefill.md")
MFMA_PROFILE = os.path.join(ROOT, "profiles", "mfma_counters_{}_prefill.md")
# The 256 MB MALL is not flushed between timed steps: one step streams tens
# of GB of weights and activations (every loop's expert weights alone pass
# 4.8 GB through it at mythos_3b), so a step starts with whatever its
# predecessor's last loop left there, as a step in a serving loop would.
MALL_STATE = "warm (not flushed between steps; each step streams far more than the 256 MB MALL)"

GEMM_SOURCES = ["gemm_big.hip", "gemm_device.h", "gemm.h", "common.h"]


def gemm_source_hash():
    import hashlib
    hsh = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "recurrent_depth_moe_amd", "csrc", name), "rb") as f:
            hsh.update(f.read())
    return hsh.hexdigest()


def profile_value(path, key):
    """A machine-readable `key: value` line of a committed rocprofv3 counter
    summary, or None when the file is absent or was taken on a different
    GEMM kernel source (its kernel_source_sha256 line)."""
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.split(":", 1)[0].strip() in (key, "kernel_source_sha256"):
                k, val = line.split(":", 1)
                fields[k.strip()] = val.strip().strip("`")
    if fields.get("kernel_source_sha256") != gemm_source_hash():
        return None
    try:
        return float(fields[key])
    except (KeyError, ValueError):
        return None


def measured_traffic(config):
    """HBM bytes per launch of the routed gate|up kernel (FETCH_SIZE and
    WRITE_SIZE passes, copy-calibrated) for this workload, or None."""
    return profile_value(TRAFFIC_PROFILE.format(config), "traffic_bytes_per_launch")


def counter_mfma_frac(config):
    """Executed bf16 MFMA flops of the routed gate|up launch
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) / (its duration x 2.5 PF), or None."""
    return profile_value(MFMA_PROFILE.format(config), "mfma_frac_counter_expert_gate_up")


def sample_sclk(stop, out):
    """GPU core clock (MHz) read with rocm-smi every ~0.2 s until `stop` is
    set (the sustained clock under load; MFMA-heavy phases run below the
    2.4 GHz peak clock)."""
    import re
    import subprocess
    while not stop.is_set():
        try:
            r = subprocess.run(["rocm-smi", "--showclocks"], stdout=subprocess.PIPE, stderr=subprocess.DEVNULL,
                               text=True, timeout=10)
            m = re.search(r"sclk clock level:\s*\S+:?\s*\((\d+)Mhz\)", r.stdout)
            if m:
                out.append(int(m.group(1)))
        except (OSError, subprocess.SubprocessError):
            return
        stop.wait(0.2)


def cpu_baseline(cfg, W, e, h0, prefix):
    """The fp64 oracle as it stands, on the first `prefix` tokens of each
    sequence for one loop (causal attention and per-token routing make this
    exactly the first rows of the full workload's first loop)."""
    import numpy as np
    from oracle import rdt_oracle as O
    cores = len(os.sched_getaffinity(0))
    P = O.Params(W)
    sub = dict(cfg, seq=prefix)
    t0 = time.perf_counter()
    O.recurrent_forward(sub, P, e[:, :prefix], h0[:, :prefix], 1, cfg["act_threshold"])
    dt = time.perf_counter() - t0
    return dict(value=round(cfg["batch"] * prefix / dt, 3), unit="token·loops/s", cores=cores, kind="oracle",
                sample=f"1 loop over the first {prefix} tokens of each of the {cfg['batch']} sequences "
                       f"({cfg['batch'] * prefix} token-loops, {dt:.1f} s)")


TRAIN_PROFILE = os.path.join(ROOT, "profiles", "counters_{}_train_step.md")
BACKWARD_SOURCES = ["backward.hip", "backward.h", "common.h"]


def train_traffic(config):
    """HBM bytes per launch of the experts' weight-gradient product
    (FETCH_SIZE and WRITE_SIZE passes, copy-calibrated) from the committed
    counter summary, or None when it was taken on other backward sources."""
    import hashlib
    path = TRAIN_PROFILE.format(config)
    if not os.path.exists(path):
        return None
    hsh = hashlib.sha256()
    for name in BACKWARD_SOURCES:
        with open(os.path.join(ROOT, "recurrent_depth_moe_amd", "csrc", name), "rb") as f:
            hsh.update(f.read())
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                k, val = line.split(":", 1)
                fields[k.strip()] = val.strip().strip("`")
    if fields.get("kernel_source_sha256") != hsh.hexdigest():
        return None
    try:
        return float(fields["traffic_bytes_per_launch_expert_wgrad"])
    except (KeyError, ValueError):
        return None


def train_flops(cfg, loops):
    """Algorithmic flops of one training step: the forward, then per loop the
    input-gradient and weight-gradient products (each the forward product's
    flops) and the attention backward (dV, dP, dQ, dK: twice the forward's
    two products)."""
    w = stage_work(cfg)
    fwd = sum(v["flops"] for v in w.values() if "flops" in v)
    att = w["attention"]["flops"]
    return loops * (fwd + 2 * (fwd - att) + 2 * att)


def train_cpu_baseline(cfg, W, e, h0, prefix):
    """The gradient oracle as it stands (fp64 autograd, the forward's
    decisions taken by the numpy oracle) on the first `prefix` tokens of the
    first sequence for one loop: a bounded sample of the training step."""
    import numpy as np
    from oracle import rdt_backward as OB
    from oracle import rdt_oracle as O
    cores = len(os.sched_getaffinity(0))
    sub = dict(cfg, batch=1, seq=prefix)
    P = O.Params(W)
    t0 = time.perf_counter()
    r = O.recurrent_forward(sub, P, e[:1, :prefix], h0[:1, :prefix], 1, cfg["act_threshold"], record=True)
    dy = np.random.default_rng(5).standard_normal((1, prefix, cfg["dim"]))
    OB.recurrent_grad(sub, P, e[:1, :prefix], h0[:1, :prefix], 1, cfg["act_threshold"],
                      np.stack(r["record"]["sel"]), r["halt_counts"], dy)
    dt = time.perf_counter() - t0
    return dict(value=round(prefix / dt, 3), unit="trained token·loops/s", cores=cores, kind="oracle",
                sample=f"forward and gradient of 1 loop over the first {prefix} tokens of sequence 0 "
                       f"({prefix} token-loops, {dt:.1f} s, every block weight in fp64 with its gradient)")


def train_bench(args, cfg):
    import threading

    import numpy as np
    import torch

    from recurrent_depth_moe_amd import binding
    from workloads import generate
    B, T, D, L, thr = cfg["batch"], cfg["seq"], cfg["dim"], cfg["n_loops"], cfg["act_threshold"]
    t0 = time.time()
    W = generate.make_weights(cfg)
    e, h0 = generate.make_inputs(cfg)
    log(f"[bench] {args.config} training step: inputs generated in {time.time() - t0:.1f}s")
    blk = binding.Block(cfg, binding.weights_to_device(W))
    et = torch.from_numpy(e).cuda()
    ht = torch.from_numpy(h0).cuda()
    dy = torch.from_numpy(np.random.default_rng(5).standard_normal(e.shape).astype(np.float32)).cuda()
    tape = blk.new_tape(B, T, L)
    bws = torch.empty(blk.train_workspace_bytes(B, T, L), dtype=torch.uint8, device="cuda")
    grad = torch.empty(blk.grad_numel(), dtype=torch.float32, device="cuda")
    de, dh0 = torch.empty_like(et), torch.empty_like(et)
    load = torch.empty(cfg["n_experts"], dtype=torch.int32, device="cuda")
    h_out = torch.empty_like(et)
    hc = torch.empty((B, T), dtype=torch.int32, device="cuda")
    opt = blk.adamw_init()
    log(f"[bench] training workspace {bws.numel() / 2**30:.1f} GiB, tape {tape.numel() / 2**30:.2f} GiB, "
        f"optimizer state {opt.numel() * 4 / 2**30:.1f} GiB")
    stream = torch.cuda.current_stream()
    n_steps = [0]
    # loops each step ran (the weights move, so the halting loops may too)
    loops_run = torch.zeros(args.warmup + args.steps, dtype=torch.int32, device="cuda")

    def step():
        blk.train_forward(et, ht, L, thr, tape, h_out, hc)
        blk.train_backward(et, ht, L, thr, tape, hc, dy, bws, grad, de, dh0, load)
        n_steps[0] += 1
        blk.adamw_step(grad, opt, n_steps[0], **OPT_HP)
        blk.router_bias_update(load, OPT_BIAS_GAMMA)
        if thr > 0:
            torch.amax(hc.view(-1), 0, out=loops_run[n_steps[0] - 1])

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup {i + 1}/{args.warmup} done")
    clocks, stop = [], threading.Event()
    sampler = threading.Thread(target=sample_sclk, args=(stop, clocks), daemon=True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    # the dominant kernel (the routed experts' weight-gradient launches) is
    # bracketed with HIP events by the library on the launch stream
    dom = "train_expert_wgrad"
    blk.set_timing_stages([dom, "train_attn_bwd", "train_optimizer"])
    torch.cuda.synchronize()
    if not args.no_clock:
        sampler.start()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
        log(f"[bench] step {i + 1}/{args.steps} enqueued")
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stop.set()
    if not args.no_clock:
        sampler.join(timeout=15)
    step_ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    tm = blk.read_timing()
    blk.set_timing(False)
    per_step = loops_run[args.warmup:].tolist() if thr > 0 else [L] * args.steps
    loops = max(per_step)
    value = B * T * sum(per_step) / elapsed
    fl = sum(train_flops(cfg, x) for x in per_step) / args.steps
    ms_step = elapsed / args.steps * 1e3
    # roofline of the dominant kernel: one launch is the weight gradient of
    # one routed matrix (gate, up or down) over every loop's rows,
    # 2 * (loops * N * k) * F * D flops
    N, k, F = B * T, cfg["top_k"], cfg["expert_dim"]
    wg_flops = 2.0 * loops * N * k * F * D
    wg_ms, wg_n = tm[dom]
    wg_avg = wg_ms / max(wg_n, 1)
    at_ms, at_n = tm["train_attn_bwd"]
    at_flops = 2 * stage_work(cfg)["attention"]["flops"]
    roof = dict(bound="mfma", achieved=round(wg_flops / (wg_avg * 1e-3) / 1e12, 2), peak=PEAK_BF16_TFLOPS,
                unit="TFLOP/s", traffic=train_traffic(args.config),
                kernel="routed experts' weight-gradient product (wgrad8_kernel, one routed matrix over every loop's rows)",
                per_launch_flops=wg_flops, avg_launch_ms=round(wg_avg, 4), launches=wg_n)
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    attn = dict(avg_launch_ms=round(at_ms / max(at_n, 1), 4), launches=at_n,
                tflops=round(at_flops / (at_ms / max(at_n, 1) * 1e-3) / 1e12, 1))
    # the AdamW launch: per trained element it reads the gradient, master,
    # m and v (16 B) and writes master, m, v (12 B) and the weight (bf16
    # matrices 2 B, fp32 vectors 4 B)
    opt_bytes = 0
    for name, (_, m) in blk.grad_layout().items():
        if name != "router_bias":
            opt_bytes += m * (28 + (2 if W[name].dtype == np.uint16 else 4))
    op_ms, op_n = tm["train_optimizer"]
    op_avg = op_ms / max(op_n, 1)
    optimizer = dict(bound="hbm", avg_launch_ms=round(op_avg, 4), launches=op_n, bytes_per_launch=opt_bytes,
                     achieved=round(opt_bytes / (op_avg * 1e-3) / 1e9, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                     lr=OPT_HP["lr"], betas=[OPT_HP["beta1"], OPT_HP["beta2"]], weight_decay=OPT_HP["weight_decay"],
                     router_bias_gamma=OPT_BIAS_GAMMA)
    optimizer["frac"] = round(optimizer["achieved"] / PEAK_HBM_GBS, 4)
    log(f"[bench] expert wgrad {wg_avg:.3f} ms/launch ({roof['achieved']} TFLOP/s), attention backward "
        f"{attn['avg_launch_ms']} ms/loop ({attn['tflops']} TFLOP/s), AdamW {op_avg:.3f} ms "
        f"({optimizer['achieved']} GB/s)")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = train_cpu_baseline(cfg, W, e, h0, min(args.cpu_prefix, 256))
        log(f"[bench] cpu baseline: {cpu}")
    out = {
        "metric": "recurrent-block training token·loops/sec (1 GPU; forward + backward + AdamW)", "value": round(value, 1),
        "unit": "token·loops/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3), "ms_per_step_median": round(step_ms[len(step_ms) // 2], 3),
        "ms_per_step_min": round(step_ms[0], 3), "sclk_mhz_samples": clocks, "mall": MALL_STATE, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg["dtype"],
        "data": "synthetic (seeded N(0,0.02) weights, RMS-normalised N(0,1) inputs, N(0,1) upstream gradient)",
        "config": {"workload": f"{args.config}-shaped recurrent block, training step (forward, backward, "
                               f"AdamW and router-bias step), "
                               f"{cfg['dtype']}, batch {B} x seq {T}, {L} loops, ACT {'off' if thr == 0 else thr}",
                   "loops_executed": loops, "loops_per_step": per_step},
        "algorithmic_tflops_per_step": round(fl / 1e12, 1),
        "achieved_tflops": round(fl / (ms_step * 1e-3) / 1e12, 1),
        "mfma_frac_of_step": round(fl / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "roofline": roof,
        "attention_backward": attn,
        "optimizer": optimizer,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="mythos_3b")
    ap.add_argument("--cpu-prefix", type=int, default=4096)   # 3b: one whole loop of the workload
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--act-skip", action="store_true",
                    help="ACT with compute skipping (halted positions leave the batch; "
                         "rdt_recurrent_forward_act_skip); value = token-loops actually run per second")
    ap.add_argument("--train", action="store_true",
                    help="training step: rdt_train_forward + rdt_train_backward (gradients of every trained "
                         "tensor, e and h0 for a seeded upstream gradient); value = token-loops trained per second")
    ap.add_argument("--no-clock", action="store_true",
                    help="do not sample the core clock with rocm-smi (for runs under a profiler)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run plain device copies of this many MiB (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.copy_probe_mib:
        import torch
        n = args.copy_probe_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 4}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the single-GPU recurrent-block forward; it does not run on more than one GPU "
              "(the block shards over independent sequences, or over experts with an all-to-all per loop, "
              "neither of which is built).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from recurrent_depth_moe_amd import binding
    from workloads import configs, generate

    cfg = configs.get(args.config)
    if args.train:
        train_bench(args, cfg)
        return
    B, T, D, n_loops, thr = cfg["batch"], cfg["seq"], cfg["dim"], cfg["n_loops"], cfg["act_threshold"]
    t0 = time.time()
    W = generate.make_weights(cfg)
    e, h0 = generate.make_inputs(cfg)
    log(f"[bench] {args.config}: inputs generated in {time.time() - t0:.1f}s")
    blk = binding.Block(cfg, binding.weights_to_device(W))
    et = torch.from_numpy(e).cuda()
    ht = torch.from_numpy(h0).cuda()
    ws = blk.new_workspace(B, T)
    h_out = torch.empty_like(et)
    hc = torch.empty((B, T), dtype=torch.int32, device="cuda")
    kv = None
    cap = 0
    if cfg["use_cache"]:
        cap = cfg["start_pos"] + T
        kv = torch.zeros(blk.kv_cache_bytes(B, cap, n_loops), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    if args.act_skip and (thr <= 0 or cfg["use_cache"]):
        print("--act-skip needs a prefill workload with ACT on", file=sys.stderr)
        sys.exit(2)

    def step():
        if args.act_skip:
            blk.forward_act_skip(et, ht, n_loops, thr, cfg["start_pos"], ws, h_out, hc)
        else:
            blk.forward(et, ht, n_loops, thr, cfg["start_pos"], kv, cap, ws, h_out, hc)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup {i + 1}/{args.warmup} done")
    # timed region: only the dominant kernel is bracketed with HIP events (two
    # event records per launch on the stream; timing every stage costs ~2.5%)
    dom = "expert_gate_up"
    blk.set_timing_stages([dom])
    import threading
    clocks, stop = [], threading.Event()
    sampler = threading.Thread(target=sample_sclk, args=(stop, clocks), daemon=True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    if not args.no_clock:
        sampler.start()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stop.set()
    if not args.no_clock:
        sampler.join(timeout=15)
    step_ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    dom_timing = blk.read_timing()[dom]
    # per-stage breakdown from one more step with every stage timed
    blk.set_timing(True)
    step()
    torch.cuda.synchronize()
    stages = blk.read_timing()
    blk.set_timing(False)
    stages[dom] = dom_timing
    log(f"[bench] {args.steps} timed steps in {elapsed:.3f}s")

    halt = hc.cpu().numpy()
    # loops actually run: with ACT on and no cache the block stops once every
    # position has halted, i.e. after max(halt_counts) loops
    loops_exec = int(halt.max()) if (thr > 0 and not cfg["use_cache"]) else n_loops
    ms_step = elapsed / args.steps * 1e3
    if args.act_skip:
        # every position runs exactly its halt count of loops
        value = float(halt.sum()) * args.steps / elapsed
    else:
        value = B * T * loops_exec * args.steps / elapsed

    E = cfg["n_experts"]
    offs = blk.workspace_view(ws, B, T, "offsets", torch.int32, (E + 1,)).cpu().numpy()
    counts = np.diff(offs)
    touched = int(np.sum(counts > 0))
    work = stage_work(cfg, touched)
    if args.act_skip:
        # per-launch work averaged over the loops: loop t runs the positions
        # whose halt count exceeds t
        rows_t = [int(np.sum(halt > t)) for t in range(loops_exec)]
        frac_rows = float(np.mean(rows_t)) / (B * T)
        work = stage_work(dict(cfg, seq=max(1, int(round(T * frac_rows)))), touched)
        log(f"[bench] act-skip rows per loop: {rows_t}")
    kernels = {}
    # milliseconds per step of each stage (the dominant one was timed over
    # args.steps steps, the others over one)
    per_step = {name: ms / (args.steps if name == dom else 1) for name, (ms, n) in stages.items()}
    step_total = max(1e-9, sum(per_step.values()))
    for name, (ms, n) in stages.items():
        if n == 0:
            continue
        avg = ms / n
        ent = dict(avg_ms=round(avg, 4), launches=n, share=round(per_step[name] / step_total, 4))
        wk = work.get(name, {})
        if "flops" in wk:
            ent["tflops"] = round(wk["flops"] / (avg * 1e-3) / 1e12, 2)
            ent["mfma_frac"] = round(ent["tflops"] / PEAK_BF16_TFLOPS, 4)
        if "bytes" in wk:
            ent["gbs"] = round(wk["bytes"] / (avg * 1e-3) / 1e9, 1)
            ent["hbm_frac"] = round(ent["gbs"] / PEAK_HBM_GBS, 4)
        kernels[name] = ent
    for name, ent in kernels.items():
        log(f"  {name:16s} {ent}")
    # roofline of the dominant kernel (timed over the timed region):
    # whichever of MFMA time and HBM time of its algorithmic work is longer
    # bounds it
    d = kernels.get(dom, {})
    wk = work[dom]
    t_mfma = wk["flops"] / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = wk["bytes"] / (PEAK_HBM_GBS * 1e9)
    avg_s = d["avg_ms"] * 1e-3 if d else None
    if t_hbm >= t_mfma:
        roof = dict(bound="hbm", achieved=round(wk["bytes"] / avg_s / 1e9, 1) if avg_s else None,
                    peak=PEAK_HBM_GBS, unit="GB/s")
    else:
        roof = dict(bound="mfma", achieved=round(wk["flops"] / avg_s / 1e12, 2) if avg_s else None,
                    peak=PEAK_BF16_TFLOPS, unit="TFLOP/s")
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4) if roof["achieved"] else None
    roof["traffic"] = None if args.act_skip else measured_traffic(args.config)
    roof.update(kernel="routed expert gate|up grouped GEMM (SwiGLU epilogue)",
                per_launch_flops=wk["flops"], per_launch_bytes=wk["bytes"], avg_launch_ms=d.get("avg_ms"),
                mfma_frac=d.get("mfma_frac"),
                mfma_frac_counter=None if args.act_skip else counter_mfma_frac(args.config))
    tiles = int(np.sum((counts + 255) // 256)) if T > 1 else int(np.sum((counts + 31) // 32))
    log(f"[bench] routed rows per expert (last loop): min {counts.min()} mean {counts.mean():.1f} "
        f"max {counts.max()}, experts touched {int(np.sum(counts > 0))}, m-tiles {tiles}, "
        f"tails <= 64 rows {int(np.sum((counts % 256 > 0) & (counts % 256 <= 64)))}")
    if thr > 0:
        hist = np.bincount(halt.ravel(), minlength=n_loops + 1)[1:]
        log(f"[bench] halt-count histogram (loops 1..{n_loops}): {hist.tolist()}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, W, e, h0, min(args.cpu_prefix, T))
        log(f"[bench] cpu baseline: {cpu}")

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "token·loops/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "ms_per_step_median": round(step_ms[len(step_ms) // 2], 3), "ms_per_step_min": round(step_ms[0], 3),
        "sclk_mhz_samples": clocks, "mall": MALL_STATE,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg["dtype"],
        "data": "synthetic (seeded N(0,0.02) weights, RMS-normalised N(0,1) inputs)",
        "config": {"workload": f"{args.config}-shaped recurrent block, {cfg['dtype']} "
                               f"{'decode' if cfg['use_cache'] else 'prefill'}, batch {B} x seq {T}, "
                               f"{n_loops} loops, ACT {'off' if thr == 0 else thr}"
                               f"{' with compute skipping' if args.act_skip else ''}",
                   "dim": D, "heads": cfg["n_heads"], "kv_heads": cfg["n_kv_heads"], "experts": cfg["n_experts"],
                   "expert_dim": cfg["expert_dim"], "top_k": cfg["top_k"], "loops_executed": loops_exec},
        "useful_token_loops_per_s": round(float(halt.sum()) * args.steps / elapsed, 1),
        "frac_of_workload_roofline": (round(value / ROOFLINE_TOKEN_LOOPS[args.config], 4)
                                      if args.config in ROOFLINE_TOKEN_LOOPS else None),
        "roofline": roof,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
