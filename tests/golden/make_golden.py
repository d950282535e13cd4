"""Writes tests/golden/tiny_streams.json from the CPU oracle alone.

The tiny decoder (2 layers, d 64, 4/2 heads of 16, FFN 256, vocab 256, MASK
255, float32 weights N(0, 0.02^2), seed 0), a 16-id prompt (seed 0), 64
tokens in each mode: AR greedy, block diffusion (block 8, threshold 0.9, no
step cap), self-speculation (block 8), and self-speculation with a forced
accept schedule.  Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import workloads as W  # noqa: E402


def main():
    s = W.SHAPES["tiny"]
    m = O.OracleModel(s, W.make_weights(s, seed=0), row_independent=True)
    p = W.prompt_ids(s, 16, seed=0)
    ar = O.generate_ar(m, p, 64)
    ss = O.generate_selfspec(m, p, 64, 8)
    sched = W.forced_accept_schedule(64, 8, seed=0)
    fs = O.generate_selfspec(m, p, 64, 8, forced=sched)
    df = O.generate_diffusion(m, p, 64, 8, 0.9)
    out = {
        "config": "tiny seed 0, prompt 16 ids seed 0, 64 tokens, block 8, tau 0.9",
        "prompt": [int(t) for t in p],
        "ar": ar.tokens, "ar_min_margin": min(ar.margins),
        "selfspec": ss.tokens, "selfspec_accept": ss.accept_lengths,
        "forced_schedule": [int(x) for x in sched], "forced": fs.tokens, "forced_accept": fs.accept_lengths,
        "diffusion": df.tokens, "diffusion_steps": df.steps_per_block,
    }
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_streams.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
