"""Bisect the draft-noise standard deviation that gives a target acceptance.

Writes tests/golden/noise_sigma.json. It calls only the oracle (softmax) and
the seeded generators, never the HIP library. The per-draft acceptance
probability of the min(1, p/q) test is sum_x min(p(x), q(x)) (the standard
rejection-sampling identity behind the guarantee stated in I-DLM,
fr.news.hada.io, "Documentation et ressources > Inference & ISD"), and the
acceptance rate p of the closed form in "Speedup Factor Explorer" is that
quantity.

Run:  python -m oracle.calibrate_noise
"""

import json
import os
import sys

import numpy as np
import torch

from oracle.accept import softmax

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import workload  # noqa: E402


def mean_acceptance(sigma, V=151936, sigma_l=3.0, rows=96, seed=11):
    T = workload.normal((rows, V), sigma_l, torch.bfloat16, "cpu", seed, "cal-T")
    Z = workload.normal((rows, V), 1.0, torch.float32, "cpu", seed, "cal-Z")
    Q = (T.float() + sigma * Z).to(torch.bfloat16)
    acc = []
    for r in range(rows):
        p = softmax(T[r].double().numpy())
        q = softmax(Q[r].double().numpy())
        acc.append(np.minimum(p, q).sum())
    return float(np.mean(acc))


def bisect(target, lo=0.01, hi=4.0, iters=22):
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if mean_acceptance(mid) > target:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def main():
    out = {"V": 151936, "sigma_l": 3.0, "dtype": "bf16", "sigma_q": {}, "check": {}}
    for target in (0.5, 0.7, 0.9):
        s = round(bisect(target), 4)
        out["sigma_q"][str(target)] = s
        out["check"][str(target)] = round(mean_acceptance(s, seed=12), 4)
        print(target, s, out["check"][str(target)], flush=True)
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "tests", "golden", "noise_sigma.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
