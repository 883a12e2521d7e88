"""Choose the halting-head bias of the mythos_3b workload with the oracle.

The workload asks for positions that halt spread over loops 4..16.  Halting
only weights the output (every position keeps running the block), so the
state trajectory does not depend on the bias: one oracle run over the whole
workload (both sequences, every position) records z_t(n) = h_t(n) . w_halt
for every loop and position, and the halt counts under threshold 0.99 are
then a cheap function of the bias b.

A scalar bias moves every position's halting the same way, so it cannot
shape the spread, only place it: the largest b (the earliest halting) for
which at least 90% of positions halt at loop 4 or later is chosen, and the
share that halts by the threshold rule inside 4..15 (rather than at the
last loop, where halting is forced) is reported with the histogram.

The result goes to calibration.json next to this file; both the HIP path and
the oracle read it through workloads.configs.

Usage: python -m workloads.calibrate_halt [prefix_len]   (default: all 4096)
"""

import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

from oracle import rdt_oracle as O  # noqa: E402
from workloads import configs, generate  # noqa: E402


def halt_counts(zs, b, thr, n_loops):
    """First loop (1-based) where the float32 running sum of sigmoid(z + b)
    reaches thr, else n_loops."""
    p = (1.0 / (1.0 + np.exp(-(zs + b)))).astype(np.float32)   # [loops, N]
    cum = np.zeros(p.shape[1], dtype=np.float32)
    out = np.full(p.shape[1], n_loops)
    done = np.zeros(p.shape[1], dtype=bool)
    for t in range(n_loops):
        reach = (cum + p[t]).astype(np.float32) >= np.float32(thr)
        newly = reach & ~done
        out[newly] = t + 1
        done |= newly
        cum = np.where(done, cum, (cum + p[t]).astype(np.float32))
    return out


def main(prefix=None):
    cfg = configs.get("mythos_3b", halt_b=0.0)
    prefix = prefix or cfg["seq"]
    cfg_p = dict(cfg, seq=prefix)
    t0 = time.time()
    W = generate.make_weights(cfg)
    e, h0 = generate.make_inputs(cfg)
    e, h0 = e[:, :prefix].copy(), h0[:, :prefix].copy()
    print(f"generated in {time.time() - t0:.1f}s", flush=True)
    P = O.Params(W)
    n = cfg["n_loops"]
    wh = O.as_f64(W["halt_w"])
    zs = []
    t0 = time.time()

    def on_loop(t, h):
        zs.append(h.reshape(-1, cfg["dim"]) @ wh)
        print(f"loop {t} done at {time.time() - t0:.0f}s", flush=True)

    O.recurrent_forward(cfg_p, P, e, h0, n, 0.0, on_loop=on_loop)
    zs = np.stack(zs)                                   # [loops, N]
    thr = cfg["act_threshold"]
    lo, hi = -30.0, 10.0                                # share(>= 4) falls as b grows
    for _ in range(80):
        mid = 0.5 * (lo + hi)
        if np.mean(halt_counts(zs, mid, thr, n) >= 4) >= 0.9:
            lo = mid
        else:
            hi = mid
    b = float(np.float32(lo))
    hc = halt_counts(zs, b, thr, n)
    hist = np.bincount(hc, minlength=n + 1)[1:]
    frac = float(np.mean((hc >= 4) & (hc <= 16)))
    by_rule = float(np.mean((hc >= 4) & (hc <= 15)))
    print(f"halt_b = {b:.6f}; median {np.median(hc)}; in [4,16]: {frac:.3f}; halting by the threshold in "
          f"[4,15]: {by_rule:.3f}; hist {hist.tolist()}")
    out = dict(mythos_3b=dict(halt_b=b, prefix=prefix, median=float(np.median(hc)), frac_4_16=frac,
                              frac_4_15=by_rule, hist=hist.tolist(),
                              note="bias of the halting head: the largest bias with >= 90% of positions "
                                   "halting at loop 4 or later; chosen with the fp64 oracle on the "
                                   "whole workload"))
    json.dump(out, open(os.path.join(HERE, "calibration.json"), "w"), indent=1)


if __name__ == "__main__":
    main(int(sys.argv[1]) if len(sys.argv) > 1 else None)
