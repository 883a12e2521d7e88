"""Choose the halting-head bias of the mythos_3b workload with the oracle.

The workload asks for positions that halt spread over loops 4..16.  Halting
only weights the output (every position keeps running the block), so the
state trajectory does not depend on the bias: one oracle run records
z_t(n) = h_t(n) . w_halt for every loop and position, and the bias b is then
found by bisection so that the median halt count under threshold 0.99 is 10.

Causal attention and per-token routing make the first T' positions of each
sequence exactly those of the full-length run, so the oracle runs on a
prefix of both sequences.  The result goes to calibration.json next to this
file; both the HIP path and the oracle read it through workloads.configs.

Usage: python -m workloads.calibrate_halt [prefix_len]
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


def main(prefix=512):
    cfg = configs.get("mythos_3b", halt_b=0.0)
    cfg_p = dict(cfg, seq=prefix)
    t0 = time.time()
    W = generate.make_weights(cfg)
    e, h0 = generate.make_inputs(cfg)
    e, h0 = e[:, :prefix].copy(), h0[:, :prefix].copy()
    print(f"generated in {time.time() - t0:.1f}s", flush=True)
    P = O.Params(W)
    n = cfg["n_loops"]
    t0 = time.time()
    r = O.recurrent_forward(cfg_p, P, e, h0, n, 0.0, record=True)
    print(f"oracle {n} loops on 2x{prefix} in {time.time() - t0:.1f}s", flush=True)
    wh = O.as_f64(W["halt_w"])
    zs = np.stack([h.reshape(-1, cfg["dim"]) @ wh for h in r["record"]["h"]])   # [loops, N]
    lo, hi = -20.0, 20.0
    for _ in range(80):
        mid = 0.5 * (lo + hi)
        med = np.median(halt_counts(zs, mid, cfg["act_threshold"], n))
        if med > 10:
            lo = mid
        else:
            hi = mid
    b = hi
    hc = halt_counts(zs, b, cfg["act_threshold"], n)
    hist = np.bincount(hc, minlength=n + 1)[1:]
    frac = float(np.mean((hc >= 4) & (hc <= 16)))
    print(f"halt_b = {b:.6f}; median {np.median(hc)}; in [4,16]: {frac:.3f}; hist {hist.tolist()}")
    out = dict(mythos_3b=dict(halt_b=float(np.float32(b)), prefix=prefix, median=float(np.median(hc)),
                              frac_4_16=frac, hist=hist.tolist(),
                              note="bias of the halting head; chosen with the fp64 oracle on a causal prefix"))
    json.dump(out, open(os.path.join(HERE, "calibration.json"), "w"), indent=1)


if __name__ == "__main__":
    main(int(sys.argv[1]) if len(sys.argv) > 1 else 512)
