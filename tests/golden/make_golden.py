"""Writes the stored values under tests/golden/ from the oracle only.

c5_zipf.json: the Zipf exponent s of the prefill-chunk workload (4096 tokens,
hidden 4096, 256 routed experts, top-6): the smallest multiple of 0.1 for
which the seed-1 routing computed by the oracle sends more than 500 tokens to
one expert (the workload asks for a Zipf skew in which some experts receive
more than 500 tokens; about 96 tokens per expert on average).

Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import moe_inputs as mi  # noqa: E402
import oracle  # noqa: E402


def c5_zipf():
    T, H, E, k = 4096, 4096, 256, 6
    x = mi.gen_x(1, 0, T, H)
    W = mi.gen_router(1, 0, E, H)
    prev_max = 0
    for tenth in range(1, 31):
        s = round(tenth * 0.1, 1)
        b = mi.gen_bias(1, 0, E, mi.BIAS_ZIPF, s)
        ids, _ = oracle.select_topk(oracle.router_logits(x, W, b), k)
        hist = np.bincount(ids.ravel(), minlength=E)
        print(f"s={s}: max {hist.max()} median {np.median(hist)} empty {(hist == 0).sum()}")
        if hist.max() > 500:
            return {"s": s, "seed": 1, "max_tokens_per_expert": int(hist.max()),
                    "median_tokens_per_expert": float(np.median(hist)), "empty_experts": int((hist == 0).sum()),
                    "previous_s_max": int(prev_max), "histogram": hist.tolist()}
        prev_max = int(hist.max())
    raise RuntimeError("no s up to 3.0 reaches 500 tokens on one expert")


if __name__ == "__main__":
    rec = c5_zipf()
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "c5_zipf.json"), "w") as f:
        json.dump(rec, f)
    print(rec["s"])
