"""Write tests/golden/zipf_bias_e256.txt: the per-expert selection bias of the
16384-token prefill workload, fitted so that expert popularity follows a
Zipf(s=1.1) law over the 256 experts.

The bias is an input of that workload (a selection-only correction bias, as the
"Auxiliary-loss-free load balancing" row of the DeepSeek-V4-Flash techniques
map describes); parity never depends on how well it fits.  The fit uses only
the CPU oracle's router, on a calibration batch drawn separately from the
workload's own activations:

1. a seeded permutation gives every expert a popularity rank r (1 = hottest);
2. target slot shares q_r proportional to r^-1.1, capped at 1/6 by
   water-filling (a token cannot pick an expert twice, so no expert can hold
   more than one slot in six);
3. 200 steps of b_e += 0.1 * (ln target_e - ln(count_e + 1)) on the
   calibration batch's sqrt-softplus scores.

Run from the repository root:  python tests/golden/make_zipf_bias.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import moe_oracle as O  # noqa: E402
from mxfp4_routed_expert_moe_amd import workloads as WL  # noqa: E402

S = 1.1
STEPS = 200
LR = 0.1
T_CAL = 16384


def water_fill(q: np.ndarray, cap: float) -> np.ndarray:
    q = q / q.sum()
    for _ in range(len(q)):
        over = q > cap
        if not over.any():
            break
        excess = (q[over] - cap).sum()
        q[over] = cap
        free = q < cap
        q[free] += excess * q[free] / q[free].sum()
    return q


def main():
    w = WL.WORKLOADS[4]
    E, k = WL.N_EXPERTS, WL.TOP_K
    router = WL.make_router(w.seed, WL.HIDDEN, E)
    x_cal = WL.make_x(w.seed ^ 0xCA1B, T_CAL, WL.HIDDEN)       # a batch apart from the workload's x
    s = O.sqrt_softplus(O.router_logits(x_cal, router))
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 5])))
    rank = np.empty(E, dtype=np.int64)
    rank[g.permutation(E)] = np.arange(1, E + 1)
    q = water_fill(rank.astype(np.float64) ** -S, 1.0 / k)
    target = q * k * T_CAL
    b = np.zeros(E, dtype=np.float64)
    for _ in range(STEPS):
        ids = O.select_top_k(s + b.astype(np.float32).astype(np.float64)[None, :], k)
        cnt = np.bincount(ids.reshape(-1), minlength=E)
        b += LR * (np.log(target) - np.log(cnt + 1.0))
    b32 = b.astype(np.float32)
    ids = O.select_top_k(s + b32.astype(np.float64)[None, :], k)
    cnt = np.bincount(ids.reshape(-1), minlength=E)
    by_rank = cnt[np.argsort(rank)]
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_bias_e256.txt")
    with open(out, "w") as f:
        f.write("# Selection bias of the 16384-token Zipf(s=1.1) prefill workload, float32, one per expert.\n")
        f.write("# Written by tests/golden/make_zipf_bias.py with the CPU oracle's router.\n")
        f.write(f"# Calibration counts by popularity rank (first 8): {by_rank[:8].tolist()}\n")
        f.write(f"# median {int(np.median(cnt))}, min {int(cnt.min())}, total {int(cnt.sum())} slots\n")
        for v in b32:
            f.write(f"{float(v):.9g}\n")
    print("wrote", out, "counts by rank:", by_rank[:8].tolist(), "median", np.median(cnt), "min", cnt.min())


if __name__ == "__main__":
    main()
