"""The oracle's own float32-vs-float64 logit gap: how far an exact
implementation of the same decoder, computing in fp32 instead of float64,
lands from the float64 oracle.  It is the floor under any fp32 GPU path's
logit deviation, measured from the oracle alone (no GPU).

Default inputs: those of the 14B full-depth lockstep test (40 layers, d 5120,
prompts of 257 and 600 tokens, each prefilled, then one diffusion step over an
all-MASK 32-token block): the prefills' last rows and every row of the steps.
Holds both widened models in turn (about 112 GB of float64, then 56 GB of
float32, on top of the 28 GB of bf16 draws): run it on a large-memory host,

    python tests/oracle_fp32_floor.py [shape] [prompt lengths ...]

Not collected by pytest (no test_ prefix).
"""
import gc
import os
import sys
import time

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import numpy as np  # noqa: E402

import oracle as O  # noqa: E402
import workloads as W  # noqa: E402


def main(argv):
    name = argv[1] if len(argv) > 1 else "14b"
    lens = [int(v) for v in argv[2:]] or [257, 600]
    s = W.SHAPES[name]
    w = W.make_weights(s, seed=0, threads=min(16, len(os.sched_getaffinity(0))))
    prompts = [W.prompt_ids(s, n, seed=0, index=i) for i, n in enumerate(lens)]
    out = {}
    for dt in (np.float64, np.float32):
        t0 = time.time()
        om = O.OracleModel(s, w, dtype=dt)
        rows = []
        for i, p in enumerate(prompts):
            ss = O.OracleSession(om)
            rows.append(ss.prefill(0, p).logits.astype(np.float64))
            _, _, _, sel = ss.diffuse_step(0, np.full(32, s.mask_id, dtype=np.int32), 0.9, False)
            rows.append(sel.logits.astype(np.float64))
            print(f"{dt.__name__}: sequence {i} done, {time.time() - t0:.0f}s", flush=True)
        out[dt.__name__] = rows
        del om, ss
        gc.collect()
    worst = 0.0
    for i, (a, b) in enumerate(zip(out["float64"], out["float32"])):
        d = np.abs(a - b)
        worst = max(worst, float(d.max()))
        kind = "prefill last row" if i % 2 == 0 else "diffusion step, 32 rows"
        print(f"sequence {i // 2} {kind}: max|d| {d.max():.3e}, mean {d.mean():.3e}", flush=True)
    print(f"{name} ({s.n_layers} layers), prompts {lens}: oracle float32 vs float64 max|dlogit| {worst:.3e}",
          flush=True)


if __name__ == "__main__":
    main(sys.argv)
