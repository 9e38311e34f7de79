"""Find the bias strength alpha that makes each skewed level hit its maxvio target.

Writes synth/alpha_table.json.  Run:  python -m synth.tune [config ...]
Bisection on alpha in [0, 16]: maxvio grows with alpha; the target is met when
the realised maxvio is within 2 % of it.
"""
import json
import sys
import time

import numpy as np

import synth


def tune(config, level, tol=0.02):
    c = dict(synth.WORKLOADS[config])
    target = synth.LEVELS[config][level]
    seed = synth.seed_of(config, level)
    base = synth.base_logits(c, seed)

    def mv(alpha):
        topk, _ = synth.route_from_logits(c, seed, base, alpha)
        return synth.maxvio(topk, c["E"])

    lo, hi = 0.0, 16.0
    best = None
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        v = mv(mid)
        if best is None or abs(v - target) < abs(best[1] - target):
            best = (mid, v)
        if abs(v - target) <= tol * target:
            break
        if v < target:
            lo = mid
        else:
            hi = mid
    return {"alpha": best[0], "maxvio": best[1], "target": target, "seed": seed}


def main(argv):
    configs = [int(a) for a in argv] or [4, 5]
    tab = synth.load_alpha_table()
    for config in configs:
        for level, target in enumerate(synth.LEVELS[config]):
            if target is None:
                continue
            t0 = time.time()
            res = tune(config, level)
            tab[f"{config}:{level}"] = res
            print(config, level, res, f"{time.time() - t0:.1f}s", flush=True)
            with open(synth._ALPHA_FILE, "w") as f:
                json.dump(tab, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:])
