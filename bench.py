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


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "hbm_traffic_expert_gate_up_mythos_3b.md")
GEMM_SOURCES = ["gemm_big.hip", "gemm_device.h", "gemm.h", "common.h"]


def gemm_source_hash():
    import hashlib
    hsh = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "recurrent_depth_moe_amd", "csrc", name), "rb") as f:
            hsh.update(f.read())
    return hsh.hexdigest()


def measured_traffic(config):
    """HBM bytes per launch of the routed gate|up kernel from the committed
    rocprofv3 counter summary, or None when that summary was taken on
    another workload or on a different kernel source."""
    if config != "mythos_3b" or not os.path.exists(TRAFFIC_PROFILE):
        return None
    fields = {}
    with open(TRAFFIC_PROFILE) as f:
        for line in f:
            if ":" in line and line.split(":", 1)[0].strip() in ("traffic_bytes_per_launch", "kernel_source_sha256"):
                key, val = line.split(":", 1)
                fields[key.strip()] = val.strip().strip("`")
    if fields.get("kernel_source_sha256") != gemm_source_hash():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="mythos_3b")
    ap.add_argument("--cpu-prefix", type=int, default=4096)   # 3b: one whole loop of the workload
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    def step():
        blk.forward(et, ht, n_loops, thr, cfg["start_pos"], kv, cap, ws, h_out, hc)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup {i + 1}/{args.warmup} done")
    # timed region: only the dominant kernel is bracketed with HIP events (two
    # event records per launch on the stream; timing every stage costs ~2.5%)
    dom = "expert_gate_up"
    blk.set_timing_stages([dom])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
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
    value = B * T * loops_exec * args.steps / elapsed

    E = cfg["n_experts"]
    offs = blk.workspace_view(ws, B, T, "offsets", torch.int32, (E + 1,)).cpu().numpy()
    counts = np.diff(offs)
    touched = int(np.sum(counts > 0))
    work = stage_work(cfg, touched)
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
    roof["traffic"] = measured_traffic(args.config)
    roof.update(kernel="routed expert gate|up grouped GEMM (SwiGLU epilogue)",
                per_launch_flops=wk["flops"], per_launch_bytes=wk["bytes"], avg_launch_ms=d.get("avg_ms"),
                mfma_frac=d.get("mfma_frac"))
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
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg["dtype"],
        "data": "synthetic (seeded N(0,0.02) weights, RMS-normalised N(0,1) inputs)",
        "config": {"workload": f"{args.config}-shaped recurrent block, {cfg['dtype']} "
                               f"{'decode' if cfg['use_cache'] else 'prefill'}, batch {B} x seq {T}, "
                               f"{n_loops} loops, ACT {'off' if thr == 0 else thr}",
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
