#!/usr/bin/env python3
"""Benchmark: decoded tokens/s of self-speculative block decoding on one GPU,
8B-shaped random-init decoder (36 layers, d 4096, 32 q / 8 KV heads of 128,
SwiGLU 12288, vocab 151936, bf16), single query, prompt 1024, block 32,
2048 generated tokens, accept length per cycle drawn from a seeded uniform
schedule over {1..32} (random weights accept ~1 token naturally, the schedule
exercises long accepts).  A step is one whole generation: the cycles (a
bidirectional draft forward, a causal verify forward and the KV commit) that
take the sequence from its 1024-token prompt to 2048 emitted tokens.  Each
timed step runs on its own sequence, prefilled before the timed region.

Prints one JSON line (rank 0, N = 1).  Also reported: the roofline of the
dominant kernel (the gate/up GEMM, measured with HIP events on the model's
stream), per-kernel and per-forward latencies, AR and natural-accept
self-speculation rates, the 3B and 14B-batch workloads, the 4-bit weight and
quadratic variants, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix peak
METRIC = "decoded tokens/s at 1 GPU, 8B-shape self-spec block 32; forward % of HBM roofline"


def layer_weight_bytes(s) -> dict:
    d, F = s.d_model, s.ffn_dim
    return {"qkv": s.qkv_dim * d * 2, "o": d * s.q_dim * 2, "gate_up": 2 * F * d * 2, "down": d * F * 2}


def forward_bytes(s, n: int, T: int, w4: bool = False) -> int:
    """Algorithmic HBM bytes of one T-row forward at committed length n:
    every weight once, the KV prefix read, the block's K/V written, the
    gathered embedding rows."""
    lw = layer_weight_bytes_w4(s) if w4 else layer_weight_bytes(s)
    w = sum(lw.values()) * s.n_layers + s.vocab * s.d_model * 2
    kv_tok = s.n_layers * 2 * s.n_kv_heads * s.head_dim * 2
    return w + (n + T) * kv_tok + T * kv_tok + T * s.d_model * 2


def layer_weight_bytes_w4(s) -> dict:
    """4-bit decoder matrices: half a byte per weight plus a bf16 scale per
    128 inputs."""
    d, F = s.d_model, s.ffn_dim
    nk = {"qkv": (s.qkv_dim, d), "o": (d, s.q_dim), "gate_up": (2 * F, d), "down": (d, F)}
    return {k: n * k_ // 2 + n * (k_ // 128) * 2 for k, (n, k_) in nk.items()}


def kernel_bytes(s, cls: str, M: int, w4: bool = False) -> int:
    """Algorithmic bytes of one launch of a GEMM class at M rows: weights +
    activations in + activations out.  Activations handed between kernels are
    two bf16 planes (4 bytes an element); k/v go to the cache as bf16; the O
    and down projections' result is one fp32 residual update per element."""
    d, F = s.d_model, s.ffn_dim
    lw = layer_weight_bytes_w4(s) if w4 else layer_weight_bytes(s)
    io = {"qkv": M * d * 4 + M * s.q_dim * 4 + M * 2 * s.kv_dim * 2,
          "o": M * s.q_dim * 4 + M * d * 4,
          "gate_up": M * d * 4 + M * F * 4,
          "down": M * F * 4 + M * d * 4}
    return lw[cls] + io[cls]


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "gate_up_gemm_8b_selfspec_hbm_traffic.txt")
KERNEL_SOURCE = os.path.join(ROOT, "self_speculative_amd", "csrc", "sdm_kernels.hip")
BUILD_SCRIPT = os.path.join(ROOT, "self_speculative_amd", "build.py")


def kernel_build_sha256() -> str:
    """sha256 of the kernel source followed by the build script (its compiler flags)."""
    import hashlib
    h = hashlib.sha256()
    for path in (KERNEL_SOURCE, BUILD_SCRIPT):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the gate/up GEMM from the committed rocprofv3
    --pmc record, or None if the kernel source or its build flags changed
    since it was taken."""
    try:
        kv = dict(l.strip().split("=", 1) for l in open(TRAFFIC_RECORD) if "=" in l and not l.startswith("#"))
        sha = kernel_build_sha256()
    except OSError:
        return None
    if kv.get("kernel_build_sha256") != sha:
        return None
    return int(float(kv["traffic_bytes_per_launch"]))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps, each one whole generation of --gen-tokens tokens on its own sequence (default 3)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--gen-tokens", type=int, default=2048)
    ap.add_argument("--prompt", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="headline pass only (for profilers)")
    ap.add_argument("--attention-op-only", action="store_true",
                    help="run only the standalone attention op measurement (for profilers) and print it")
    ap.add_argument("--no-batch14b", action="store_true",
                    help="skip the 14B-shaped 16-sequence batched diffusion pass (draws ~30 GB of weights)")
    ap.add_argument("--batch14b-only", action="store_true", help="only the 14B batched diffusion pass (for profilers)")
    ap.add_argument("--batch14b-tokens", type=int, default=1024, help="generated tokens per sequence of the 14B pass")
    ap.add_argument("--no-3b", action="store_true", help="skip the 3B-shaped decoder pass")
    ap.add_argument("--no-w4", action="store_true", help="skip the 4-bit weight (w4a16) pass of the extras")
    ap.add_argument("--no-quadratic", action="store_true", help="skip the quadratic self-speculation pass")
    ap.add_argument("--quadratic-only", action="store_true",
                    help="only the quadratic self-speculation pass (for profilers)")
    ap.add_argument("--w4-only", action="store_true", help="only the 4-bit weight (w4a16) pass (for profilers)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration under rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: runs on exactly one GPU; multi-GPU runs are not supported (the path's sharding across "
              "GPUs is a design, not an implementation)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import workloads as W
    from self_speculative_amd.decode import SelfSpecRun, prefill
    from self_speculative_amd.model import Model

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    log = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)
    if args.attention_op_only:
        print(json.dumps({"attention_op": attention_op_bench(log)}), flush=True)
        return 0
    if args.batch14b_only:
        print(json.dumps({"batch_14b": batch14b_bench(log, n_gen=args.batch14b_tokens)}), flush=True)
        return 0
    s = W.SHAPES["8b"]
    B = 32
    sched = W.forced_accept_schedule(8192, B, seed=0)
    # one step = one whole generation: y1 comes from the prefill, then forced
    # cycles until gen_tokens tokens have been emitted (the last cycle's
    # overshoot is discarded)
    gen_cyc, tot = 0, 1
    while tot < args.gen_tokens:
        tot += int(sched[gen_cyc])
        gen_cyc += 1
    if args.w4_only:
        print(json.dumps({"w4a16": w4a16_bench(log, s, W.prompt_ids(s, args.prompt, seed=0), sched, gen_cyc,
                                                args.warmup, 4096)}), flush=True)
        return 0
    t0 = time.time()
    weights = W.make_weights(s, seed=0, threads=min(16, len(os.sched_getaffinity(0))))
    log(f"weights drawn in {time.time() - t0:.1f}s")
    prompt = W.prompt_ids(s, args.prompt, seed=0)
    if args.quadratic_only:
        q = quadratic_bench(log, s, weights, prompt, sched, args.warmup, 4096, n_cyc=args.steps or 40)
        torch.cuda.empty_cache()
        print(json.dumps({"quadratic": q, "vendor_gemm_bf16": vendor_gemm_rate(log)}), flush=True)
        return 0
    K = args.steps if args.steps is not None else 3
    if K < 1:
        print("bench.py: --steps must be at least 1", file=sys.stderr)
        return 2
    max_ctx = 4096 if args.prompt + args.gen_tokens + 2 * B <= 4096 else args.prompt + args.gen_tokens + 1024
    t0 = time.time()
    # sequences 0..K-1 hold the timed generations; sequence K the warm-up
    model = Model(s, weights, max_seqs=K + 1, max_block=B, max_context=max_ctx, max_rows=1024)
    torch.cuda.synchronize()
    log(f"model uploaded + packed in {time.time() - t0:.1f}s ({model.weight_bytes / 1e9:.2f} GB)")
    dev = model.device

    def run_cycles(seq, n, sched_vals, first):
        run = SelfSpecRun(model, B, seq)
        blocks = torch.empty((n, B), dtype=torch.int32, device=dev)
        ars = torch.empty((n, B), dtype=torch.int32, device=dev)
        anchor = first.data_ptr()
        Ls = []
        for c in range(n):
            run.block, run.ar = blocks[c], ars[c]
            L = run.cycle(anchor, None if sched_vals is None else int(sched_vals[c]))
            Ls.append(L)
            anchor = ars[c].data_ptr() + 4 * (L - 1)
        return Ls, anchor

    # warm-up: whole generations on sequence K
    for _ in range(args.warmup):
        model.seq_reset(K)
        first = prefill(model, K, prompt)
        run_cycles(K, gen_cyc, sched, first)
    torch.cuda.synchronize()
    model.seq_reset(K)

    # headline: K whole generations, each on its own sequence prefilled before the timed region
    firsts = [prefill(model, q, prompt) for q in range(K)]
    gen_ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    gen_ev[0].record()
    for q in range(K):
        Ls, _ = run_cycles(q, gen_cyc, sched, firsts[q])
        gen_ev[q + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    gen_ms = [gen_ev[q].elapsed_time(gen_ev[q + 1]) for q in range(K)]
    log("generation ms (GPU events): " + " ".join(f"{v:.1f}" for v in gen_ms))
    assert sum(Ls) == tot - 1
    decoded = K * (args.gen_tokens - 1)        # tokens 2..N of every generation (y1 is the prefill's)
    value = decoded / wall
    log(f"self-spec forced: {K} generations x {gen_cyc} cycles, {decoded} decoded tokens in {wall * 1e3:.1f} ms "
        f"-> {value:.1f} tok/s")
    for q in range(K):
        model.seq_reset(q)
    cyc_tokens = tot - 1                       # tokens committed by one generation's cycles (before truncation)

    out = {"metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1, "steps": K,
           "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / K, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (random-init N(0,0.02^2) bf16 weights, uniform random prompt ids, seed 0)",
           "config": {"workload": f"8B-shape decoder (36 layers, d 4096, 32/8 heads x 128, FFN 12288, vocab 151936), "
                                  f"single query, prompt {args.prompt}, self-speculation block 32, forced accept "
                                  f"L~U{{1..32}} seed 0; one step = one whole {args.gen_tokens}-token generation "
                                  f"({gen_cyc} draft+verify cycles, committed length {args.prompt} -> "
                                  f"{args.prompt + tot - 1}), its prompt prefilled before the timed region",
                      "prompt_len": args.prompt, "generated_tokens": args.gen_tokens,
                      "decoded_tokens_per_step": args.gen_tokens - 1, "cycles_per_step": gen_cyc,
                      "block": B, "accept_schedule": "forced uniform {1..32}, seed 0"}}

    if not args.no_extras:
        # per-kernel-class timing passes (HIP events on the model's stream)
        ctx_n = args.prompt
        model.seq_reset(1)
        first = prefill(model, 1, prompt)
        anchor_t = first
        per = {}
        n_cyc = 6
        classes = ["gate_up", "down", "qkv", "o", "attn", "attn_combine", "norm", "lm_head", "finish", "forward"]
        extra_sched = W.forced_accept_schedule(n_cyc * len(classes), B, seed=2)
        pos = 0
        anchor_addr = first.data_ptr()
        run = SelfSpecRun(model, B, 1)
        ring_b = torch.empty((n_cyc * len(classes), B), dtype=torch.int32, device=dev)
        ring_a = torch.empty((n_cyc * len(classes), B), dtype=torch.int32, device=dev)
        fwd_ns = []
        for cls in classes:
            torch.cuda.synchronize()
            model.timing_start(cls, 4096)
            for c in range(n_cyc):
                run.block, run.ar = ring_b[pos], ring_a[pos]
                fwd_ns.append(model.seq_length(1))
                L = run.cycle(anchor_addr, int(extra_sched[pos]))
                anchor_addr = ring_a[pos].data_ptr() + 4 * (L - 1)
                pos += 1
            n, tot_ms, mn, mx = model.timing_stop()
            per[cls] = {"launches": n, "avg_us": round(tot_ms / max(1, n) * 1e3, 2), "min_us": round(mn * 1e3, 2),
                        "max_us": round(mx * 1e3, 2)}
            log(f"{cls:>12}: {n} launches, avg {per[cls]['avg_us']} us")
        # roofline of the dominant kernel (gate/up GEMM: 47% of a forward's weight bytes)
        gu = per["gate_up"]
        gu_bytes = kernel_bytes(s, "gate_up", B)
        achieved = gu_bytes / (gu["avg_us"] * 1e-6) / 1e9
        out["roofline"] = {"bound": "hbm", "kernel": "k_gemm_bf16<EPI_SWIGLU> (gate/up + SwiGLU), M=32",
                           "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                           "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                           "bytes_per_launch": gu_bytes, "avg_launch_us": gu["avg_us"]}
        # whole forward vs roofline
        f_us = per["forward"]["avg_us"]
        mean_n = statistics.mean(fwd_ns[-n_cyc:])
        fb = forward_bytes(s, int(mean_n), B)
        out["forward"] = {"avg_us": f_us, "algorithmic_bytes": fb, "hbm_frac": round(fb / (f_us * 1e-6) / 8e12, 4),
                          "mean_committed_len": round(mean_n, 1)}
        kern = {}
        for cls in ("qkv", "o", "gate_up", "down"):
            b = kernel_bytes(s, cls, B)
            kern[cls] = dict(per[cls], GBps=round(b / (per[cls]["avg_us"] * 1e-6) / 1e9, 1))
        for cls in ("attn", "attn_combine", "norm", "lm_head", "finish"):
            kern[cls] = per[cls]
        kern["lm_head"]["GBps"] = round(s.vocab * s.d_model * 2 / (per["lm_head"]["avg_us"] * 1e-6) / 1e9, 1)
        out["kernels"] = kern
        # per-forward latency by kind (HIP events around each call on the model's stream)
        model.seq_reset(1)
        first = prefill(model, 1, prompt)
        run = SelfSpecRun(model, B, 1)
        lat_sched = W.forced_accept_schedule(24, B, seed=3)
        t_draft, t_verify = [], []
        anchor_addr = first.data_ptr()
        lb = torch.empty((24, B), dtype=torch.int32, device=dev)
        la = torch.empty((24, B), dtype=torch.int32, device=dev)
        acc = torch.empty(1, dtype=torch.int32, device=dev)
        evs = []
        for c in range(24):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            model.draft_block(1, anchor_addr, B, lb[c])
            e[1].record()
            model.verify_block([1], lb[c], B, la[c], acc)
            e[2].record()
            model.commit_kv(1, int(lat_sched[c]))
            anchor_addr = la[c].data_ptr() + 4 * (int(lat_sched[c]) - 1)
            evs.append(e)
        ar_buf = torch.empty(33, dtype=torch.int32, device=dev)
        ar_buf[0:1].copy_(la[23, int(lat_sched[23]) - 1:int(lat_sched[23])])
        ar_ev = []
        for t in range(1, 33):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record()
            model.decode_ar(1, ar_buf.data_ptr() + 4 * (t - 1), ar_buf.data_ptr() + 4 * t)
            e[1].record()
            ar_ev.append(e)
        torch.cuda.synchronize()
        out["forward_latency"] = {
            "bidir_M32": _pct([e[0].elapsed_time(e[1]) * 1e3 for e in evs]),
            "causal_M32": _pct([e[1].elapsed_time(e[2]) * 1e3 for e in evs]),
            "ar_M1": _pct([e[0].elapsed_time(e[1]) * 1e3 for e in ar_ev]),
            "committed_len_range": [args.prompt, model.seq_length(1)]}
        out["attention_op"] = attention_op_bench(log)
        # natural-accept self-spec and AR rates (short windows)
        model.seq_reset(1)
        first = prefill(model, 1, prompt)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        Ln, _ = run_cycles(1, 16, None, first)
        torch.cuda.synchronize()
        t_nat = time.perf_counter() - t0
        model.seq_reset(1)
        first = prefill(model, 1, prompt)
        ar_out = torch.empty(65, dtype=torch.int32, device=dev)
        ar_out[0:1].copy_(first)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        base = ar_out.data_ptr()
        for t in range(1, 65):
            model.decode_ar(1, base + 4 * (t - 1), base + 4 * t)
        torch.cuda.synchronize()
        t_ar = time.perf_counter() - t0
        # prefill latency
        model.seq_reset(1)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        prefill(model, 1, prompt)
        torch.cuda.synchronize()
        t_pf = time.perf_counter() - t0
        # block diffusion: step budget sweep (random weights never clear tau = 0.9, so a block takes exactly
        # S bidirectional steps -- one position each, all of the rest on the last -- plus the causal commit)
        diff = {}
        nm = torch.empty(1, dtype=torch.int32, device=dev)
        blk = torch.empty((1, B), dtype=torch.int32, device=dev)
        ar = torch.empty(B, dtype=torch.int32, device=dev)
        acc1 = torch.empty(1, dtype=torch.int32, device=dev)
        for S, taur in [(1, None), (2, None), (4, None), (8, None), (16, None), (32, None), (8, 0.9)]:
            model.seq_reset(1)
            prefill(model, 1, prompt)
            n_blocks = 3
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(n_blocks):
                blk.fill_(s.mask_id)
                for st in range(S):
                    if taur is None:
                        model.diffuse_step([1], blk, B, 0.9, st == S - 1, nm)
                    else:
                        model.diffuse_step_revise([1], blk, B, 0.9, taur, st == S - 1, nm)
                model.verify_block([1], blk, B, ar, acc1)
                model.commit_kv(1, B)
            torch.cuda.synchronize()
            dt = time.perf_counter() - t0
            key = f"S{S}" + ("_revise" if taur is not None else "")
            diff[key] = {"steps": S, "tau": 0.9, "tau_revise": taur, "ms_per_block": round(dt / n_blocks * 1e3, 3),
                         "tok_per_s": round(n_blocks * B / dt, 1), "tpf": round(B / (S + 1), 3)}
            log(f"diffusion S={S}{' revise' if taur is not None else ''}: {diff[key]['ms_per_block']} ms per block, "
                f"{diff[key]['tok_per_s']} tok/s")
        out["diffusion_step_budget"] = diff
        # sampling at temperature 1: rejection-sampling self-spec (natural accepts; random weights give
        # near-uniform rows, so most drafts are accepted) and AR sampling, cycles timed after the prefill
        V = s.vocab
        model.seq_reset(1)
        nxt = torch.empty(1, dtype=torch.int32, device=dev)
        model.prefill_sample(1, torch.as_tensor(prompt, device=dev), 1.0, 7, nxt)
        sblk = torch.empty(B, dtype=torch.int32, device=dev)
        dlog = torch.empty((B, V), dtype=torch.float32, device=dev)
        dstat = torch.empty((2, B), dtype=torch.float32, device=dev)
        sacc = torch.empty(1, dtype=torch.int32, device=dev)
        n_cyc, toks_s, Ls_s, ev_d, ev_v = 24, 0, [], [], []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for c in range(n_cyc):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            model.draft_block_sample(1, nxt, B, 1.0, 7, sblk, dlog, dstat)
            e[1].record()
            model.verify_block_sample(1, sblk, B, 1.0, 7, dlog, dstat, sacc, nxt)
            e[2].record()
            L = int(sacc.item())
            model.commit_kv(1, L)
            Ls_s.append(L)
            toks_s += L
            ev_d.append(e)
        torch.cuda.synchronize()
        t_ss = time.perf_counter() - t0
        model.seq_reset(1)
        abuf = torch.empty(65, dtype=torch.int32, device=dev)
        model.prefill_sample(1, torch.as_tensor(prompt, device=dev), 1.0, 7, abuf[0:1])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(1, 65):
            model.decode_ar_sample(1, abuf.data_ptr() + 4 * (t - 1), 1.0, 7, abuf.data_ptr() + 4 * t)
        torch.cuda.synchronize()
        t_as = time.perf_counter() - t0
        out["sampling_T1"] = {
            "selfspec": {"cycles": n_cyc, "tokens": toks_s, "mean_accept": round(float(np.mean(Ls_s)), 3),
                         "tok_per_s": round(toks_s / t_ss, 1),
                         "draft_sample_us": _pct([e[0].elapsed_time(e[1]) * 1e3 for e in ev_d]),
                         "verify_sample_us": _pct([e[1].elapsed_time(e[2]) * 1e3 for e in ev_d])},
            "ar": {"tokens": 64, "tok_per_s": round(64 / t_as, 1), "ms_per_token": round(t_as / 64 * 1e3, 3)},
            "note": "one 4-byte read of L per self-spec cycle (natural accepts); prefill outside the timed region"}
        log(f"sampling T=1: self-spec {out['sampling_T1']['selfspec']['tok_per_s']} tok/s "
            f"(mean L {out['sampling_T1']['selfspec']['mean_accept']}), AR {out['sampling_T1']['ar']['tok_per_s']} tok/s")
        out["modes"] = {"selfspec_natural": {"cycles": 16, "tokens": int(sum(Ln)), "tok_per_s": round(sum(Ln) / t_nat, 1),
                                             "mean_accept": round(float(np.mean(Ln)), 3)},
                        "ar": {"tokens": 64, "tok_per_s": round(64 / t_ar, 1), "ms_per_token": round(t_ar / 64 * 1e3, 3)},
                        "selfspec_forced": {"tok_per_s": round(value, 1), "mean_accept": round(cyc_tokens / gen_cyc, 3),
                                            "tpf": round(cyc_tokens / (2 * gen_cyc), 3)},
                        "prefill_1024_ms": round(t_pf * 1e3, 2)}

    # the memory-bound 4-bit decode pass runs before the compute-bound quadratic one
    if not args.no_extras and not args.no_w4:
        model.close()
        model = None
        torch.cuda.empty_cache()
        out["w4a16"] = w4a16_bench(log, s, prompt, sched, gen_cyc, args.warmup, max_ctx, args.gen_tokens - 1)
    if not args.no_extras and not args.no_quadratic:
        if model is not None:
            model.close()
            model = None
        torch.cuda.empty_cache()
        out["quadratic"] = quadratic_bench(log, s, weights, prompt, sched, args.warmup, max_ctx,
                                           linear_tpf=cyc_tokens / (2 * gen_cyc))
        torch.cuda.empty_cache()
        out["vendor_gemm_bf16"] = vendor_gemm_rate(log)

    if args.calib_copy:
        # a plain copy of known size: 1 GiB read + 1 GiB written per launch
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["calib_copy_bytes"] = 1 << 30
        del src, dst
    if model is not None:
        model.close()
        model = None
    torch.cuda.empty_cache()
    if not args.no_extras and not args.no_3b:
        out["model_3b"] = bench_3b(log)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(s, weights, prompt, sched, log)
    if not args.no_extras and not args.no_batch14b:
        del weights
        import gc
        gc.collect()
        out["batch_14b"] = batch14b_bench(log, n_gen=args.batch14b_tokens)
    print(json.dumps(out), flush=True)
    return 0


def w4a16_bench(log, s, prompt, sched, K, warmup, max_ctx, decoded=None) -> dict:
    """The headline workload with the decoder's matrices in 4 bits (group-wise
    int4 + bf16 scales; embedding and LM head bf16): forced self-spec rate,
    per-class kernel times and the 4-bit gate/up GEMM against HBM."""
    import torch

    import workloads as W
    from self_speculative_amd.decode import SelfSpecRun, prefill
    from self_speculative_amd.model import Model
    B = 32
    t0 = time.time()
    w = W.make_w4_weights(s, seed=0, threads=min(16, len(os.sched_getaffinity(0))))
    log(f"w4a16: weights drawn in {time.time() - t0:.1f}s")
    model = Model(s, w, max_seqs=2, max_block=B, max_context=max_ctx, max_rows=128, free_host=True)
    del w
    torch.cuda.synchronize()
    log(f"w4a16: model uploaded + packed ({model.weight_bytes / 1e9:.2f} GB)")
    dev = model.device

    def run_cycles(seq, n_cyc, sched_vals, first):
        run = SelfSpecRun(model, B, seq)
        blocks = torch.empty((n_cyc, B), dtype=torch.int32, device=dev)
        ars = torch.empty((n_cyc, B), dtype=torch.int32, device=dev)
        anchor = first.data_ptr()
        Ls = []
        for c in range(n_cyc):
            run.block, run.ar = blocks[c], ars[c]
            L = run.cycle(anchor, int(sched_vals[c]))
            Ls.append(L)
            anchor = ars[c].data_ptr() + 4 * (L - 1)
        return Ls

    first = prefill(model, 1, prompt)
    run_cycles(1, warmup, W.forced_accept_schedule(warmup, B, seed=1), first)
    torch.cuda.synchronize()
    model.seq_reset(1)
    first = prefill(model, 0, prompt)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    Ls = run_cycles(0, K, sched[:K], first)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tokens = int(sum(Ls)) if decoded is None else int(decoded)   # a whole generation: its truncated length
    log(f"w4a16 self-spec forced: {K} cycles, {tokens} tokens in {wall * 1e3:.1f} ms -> {tokens / wall:.1f} tok/s")
    # per-class timing on sequence 1
    model.seq_reset(0)
    first = prefill(model, 1, prompt)
    classes = ["gate_up", "down", "qkv", "o", "forward"]
    n_cyc = 6
    ex = W.forced_accept_schedule(n_cyc * len(classes), B, seed=2)
    per, ns, pos = {}, [], 0
    run = SelfSpecRun(model, B, 1)
    rb = torch.empty((n_cyc * len(classes), B), dtype=torch.int32, device=dev)
    ra = torch.empty((n_cyc * len(classes), B), dtype=torch.int32, device=dev)
    anchor = first.data_ptr()
    for cls in classes:
        torch.cuda.synchronize()
        model.timing_start(cls, 4096)
        for c in range(n_cyc):
            run.block, run.ar = rb[pos], ra[pos]
            ns.append(model.seq_length(1))
            L = run.cycle(anchor, int(ex[pos]))
            anchor = ra[pos].data_ptr() + 4 * (L - 1)
            pos += 1
        n, tot_ms, mn, mx = model.timing_stop()
        per[cls] = {"launches": n, "avg_us": round(tot_ms / max(1, n) * 1e3, 2), "min_us": round(mn * 1e3, 2),
                    "max_us": round(mx * 1e3, 2)}
        if cls != "forward":
            b = kernel_bytes(s, cls, B, w4=True)
            per[cls]["bytes"] = b
            per[cls]["GBps"] = round(b / (per[cls]["avg_us"] * 1e-6) / 1e9, 1)
        log(f"w4a16 {cls:>8}: {n} launches, avg {per[cls]['avg_us']} us")
    model.close()
    gu = per["gate_up"]
    f_us = per["forward"]["avg_us"]
    fb = forward_bytes(s, int(statistics.mean(ns[-n_cyc:])), B, w4=True)
    ach = gu["bytes"] / (gu["avg_us"] * 1e-6) / 1e9
    return {"workload": "the headline workload (8B shape, prompt 1024, block 32, forced accept U{1..32} seed 0; "
                        f"one whole generation of {K} cycles, {tokens} decoded tokens) with QKV, O, gate/up and "
                        "down as group-wise int4 + bf16 scales (group 128)",
            "tok_per_s": round(tokens / wall, 1), "ms_per_cycle": round(wall * 1e3 / K, 4), "cycles": K,
            "decoded_tokens": tokens,
            "kernels": per,
            "forward": {"avg_us": f_us, "algorithmic_bytes": fb, "hbm_frac": round(fb / (f_us * 1e-6) / 8e12, 4)},
            "roofline_gate_up": {"bound": "hbm", "kernel": "k_gemm_w4<EPI_SWIGLU>, M=32", "achieved": round(ach, 1),
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                                 "bytes_per_launch": gu["bytes"], "avg_launch_us": gu["avg_us"]}}


def gemm_flops(s, cls: str, M: int) -> int:
    """Flops of one GEMM launch of a class at M rows (2 per multiply-add)."""
    d, F = s.d_model, s.ffn_dim
    nk = {"qkv": (s.qkv_dim, d), "o": (d, s.q_dim), "gate_up": (2 * F, d), "down": (d, F), "lm_head": (s.vocab, d)}
    n, k = nk[cls]
    return 2 * M * n * k


def vendor_gemm_rate(log, n: int = 8192, reps: int = 20) -> dict:
    """A practical reference for the MFMA-bound passes: the vendor library's bf16 GEMM (torch.matmul,
    hipBLASLt) on an n x n x n product of random N(0, 1) operands, which load the matrix units as real
    data does (all-zero operands run faster, at lower power)."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(n, n, device="cuda", dtype=torch.float32, generator=g).to(torch.bfloat16).contiguous()
    b = torch.randn(n, n, device="cuda", dtype=torch.float32, generator=g).to(torch.bfloat16).contiguous()
    for _ in range(3):
        c = torch.matmul(a, b)
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        c = torch.matmul(a, b)
    e1.record(st)
    e1.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    tflops = 2.0 * n ** 3 / (us * 1e-6) / 1e12
    del a, b, c
    log(f"vendor bf16 GEMM {n}^3: {us:.1f} us, {tflops:.1f} TFLOP/s")
    return {"kernel": f"torch.matmul bf16 {n}x{n}x{n} (hipBLASLt), random N(0,1) operands", "avg_us": round(us, 1),
            "TFLOPs": round(tflops, 1), "frac_of_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}


def quadratic_bench(log, s, weights, prompt, sched, warmup, max_ctx, n_cyc=40, linear_tpf=None) -> dict:
    """Quadratic self-speculation on the headline's 8B shape: after one draft
    forward, every cycle is a single forward of B + B^2 = 1056 rows (the
    causal verify and a candidate next block per accept length) and a commit.
    The headline's forced accept schedule (U{1..32}, seed 0) over n_cyc
    cycles: tokens/s and tokens per forward; per-class kernel times from HIP
    events; the gate/up GEMM and the whole forward against the dense bf16
    MFMA peak (the work is compute-bound: ~16 TFLOP per forward)."""
    import numpy as np
    import torch

    import workloads as W
    from self_speculative_amd.decode import QuadSpecRun, prefill
    from self_speculative_amd.model import Model
    B = 32
    M = B * (B + 1)
    model = Model(s, weights, max_seqs=2, max_block=B, max_context=max_ctx, max_rows=M)
    torch.cuda.synchronize()
    first = prefill(model, 1, prompt)
    run = QuadSpecRun(model, B, 1, max(1, warmup))
    run.draft_first(first.data_ptr())
    wsched = W.forced_accept_schedule(max(1, warmup), B, seed=1)
    for c in range(warmup):
        run.cycle(c, int(wsched[c]))
    torch.cuda.synchronize()
    model.seq_reset(1)
    # timed: the first draft forward and n_cyc quadratic cycles on sequence 0
    first = prefill(model, 0, prompt)
    run = QuadSpecRun(model, B, 0, n_cyc)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run.draft_first(first.data_ptr())
    Ls = [run.cycle(c, int(sched[c])) for c in range(n_cyc)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tokens = int(sum(Ls))
    log(f"quadratic forced: {n_cyc} cycles, {tokens} tokens in {wall * 1e3:.1f} ms -> {tokens / wall:.1f} tok/s")
    # per-class kernel times (HIP events on the model's stream), sequence 1
    first = prefill(model, 1, prompt)
    classes = ["gate_up", "down", "qkv", "o", "attn", "attn_combine", "norm", "lm_head", "finish", "forward"]
    per_cls = 2
    ex = W.forced_accept_schedule(per_cls * len(classes), B, seed=2)
    run = QuadSpecRun(model, B, 1, per_cls * len(classes))
    run.draft_first(first.data_ptr())
    per, ns, pos = {}, [], 0
    for cls in classes:
        torch.cuda.synchronize()
        model.timing_start(cls, 4096)
        for _ in range(per_cls):
            ns.append(model.seq_length(1))
            run.cycle(pos, int(ex[pos]))
            pos += 1
        n, tot_ms, mn, mx = model.timing_stop()
        per[cls] = {"launches": n, "avg_us": round(tot_ms / max(1, n) * 1e3, 2), "min_us": round(mn * 1e3, 2),
                    "max_us": round(mx * 1e3, 2)}
        if cls in ("gate_up", "down", "qkv", "o", "lm_head"):
            f = gemm_flops(s, cls, M)
            per[cls]["flops"] = f
            per[cls]["TFLOPs"] = round(f / (per[cls]["avg_us"] * 1e-6) / 1e12, 1)
        log(f"quadratic {cls:>12}: {n} launches, avg {per[cls]['avg_us']} us")
    # natural accept lengths (random weights: short accepts), 8 cycles
    model.seq_reset(1)
    first = prefill(model, 1, prompt)
    run = QuadSpecRun(model, B, 1, 8)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run.draft_first(first.data_ptr())
    Ln = [run.cycle(c, None) for c in range(8)]
    torch.cuda.synchronize()
    t_nat = time.perf_counter() - t0
    model.close()
    # one forward's work at the mean committed length of the timed classes
    n = float(np.mean(ns))
    params = sum(layer_weight_bytes(s).values()) // 2 * s.n_layers + s.vocab * s.d_model
    keys = B * n + B * (B + 1) / 2 + B * B * n + B * B * (B + 1) / 2 + B ** 3   # (row, visible key) pairs
    attn_flops = 4 * keys * s.n_q_heads * s.head_dim * s.n_layers
    fwd_flops = 2 * M * params + attn_flops
    f_us = per["forward"]["avg_us"]
    gu = per["gate_up"]
    ach = gu["flops"] / (gu["avg_us"] * 1e-6) / 1e12
    return {"workload": "8B shape, prompt 1024, block 32: one draft forward, then per cycle one forward of "
                        "B + B^2 = 1056 rows (causal verify + a candidate next block per accept length); "
                        "forced accept U{1..32} seed 0 (the headline schedule)",
            "cycles": n_cyc, "tokens": tokens, "tok_per_s": round(tokens / wall, 1),
            "ms_per_cycle": round(wall * 1e3 / n_cyc, 3),
            "tpf": round(tokens / (n_cyc + 1), 3), "linear_tpf": None if linear_tpf is None else round(linear_tpf, 3),
            "natural": {"cycles": 8, "tokens": int(sum(Ln)), "mean_accept": round(float(np.mean(Ln)), 3),
                        "tok_per_s": round(sum(Ln) / t_nat, 1)},
            "kernels": per,
            "forward": {"avg_us": f_us, "rows": M, "flops": int(fwd_flops),
                        "mfma_frac": round(fwd_flops / (f_us * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
                        "mean_committed_len": round(n, 1)},
            "roofline_gate_up": {"bound": "mfma", "kernel": f"k_gemm_bf16<EPI_SWIGLU> (gate/up + SwiGLU), M={M}",
                                 "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "flops_per_launch": gu["flops"],
                                 "avg_launch_us": gu["avg_us"],
                                 "note": "algorithmic flops; the two-term bf16 activations issue two MFMA products "
                                         "per weight tile, so the matrix units do twice this work"}}


def _pct(vals):
    import numpy as np
    a = np.asarray(vals, dtype=np.float64)
    return {"median_us": round(float(np.median(a)), 2), "p10_us": round(float(np.percentile(a, 10)), 2),
            "p90_us": round(float(np.percentile(a, 90)), 2), "n": int(a.size)}


def attention_op_bench(log) -> dict:
    """The standalone block attention op (32 block rows, 32 q / 8 KV heads of
    128, bf16, 64-token pages) over prefixes of 512, 4096 and 32768 keys in both
    block masks: per-call latency from HIP events over 100 calls, and GB/s of
    the algorithmic bytes (the K/V read once, q and the output)."""
    import torch
    import workloads as W
    from self_speculative_amd import _lib as L
    lib = L.lib()
    dev = "cuda"
    HQ, HKV, HD, T = 32, 8, 128, 32
    st = torch.cuda.current_stream()
    out = {}
    for P in (512, 4096, 32768):
        q, k, v = W.attention_op_inputs(P, T, HQ, HKV, HD, seed=0)
        nkeys = P + T
        n_pages = (nkeys + 63) // 64
        pool = torch.zeros(lib.sdm_attn_pool_bytes(HKV, HD, n_pages), dtype=torch.uint8, device=dev)
        pages = torch.arange(n_pages, dtype=torch.int32, device=dev)
        tq, tk, tv = (torch.from_numpy(a.view("int16")).to(dev) for a in (q, k, v))
        L.check(lib.sdm_attn_pack_kv(HKV, HD, tk.data_ptr(), tv.data_ptr(), nkeys, pages.data_ptr(), pool.data_ptr(),
                                     st.cuda_stream))
        wsb = lib.sdm_attn_workspace_bytes(HQ, HKV, HD, T, nkeys)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        o = torch.empty((T, HQ, HD), dtype=torch.int16, device=dev)
        nbytes = nkeys * HKV * HD * 2 * 2 + 2 * T * HQ * HD * 2
        for mode, name in ((1, "bidir"), (0, "causal")):
            call = lambda: L.check(lib.sdm_attention(HQ, HKV, HD, tq.data_ptr(), pool.data_ptr(), pages.data_ptr(), P,
                                                     T, mode, o.data_ptr(), ws.data_ptr(), wsb, st.cuda_stream))
            for _ in range(10):
                call()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(100)]
            for e0, e1 in ev:
                e0.record(st)
                call()
                e1.record(st)
            torch.cuda.synchronize()
            r = _pct([e0.elapsed_time(e1) * 1e3 for e0, e1 in ev])
            r["GBps"] = round(nbytes / (r["median_us"] * 1e-6) / 1e9, 1)
            r["hbm_frac"] = round(r["GBps"] / HBM_PEAK_GBS, 4)
            r["bytes"] = nbytes
            out[f"P{P}_{name}"] = r
            log(f"attention op P={P} {name}: median {r['median_us']} us, {r['GBps']} GB/s")
        del pool, ws, tk, tv, tq
    return out


def batch14b_bench(log, n_gen: int = 1024) -> dict:
    """The 14B-shaped batched diffusion workload: 16 sequences, prompt lengths
    uniform over {1024..8192} (seed 0), 64-token pages, block 32, tau 0.9 and at
    most 8 denoising steps, n_gen generated tokens per sequence (every
    sequence's blocks in lockstep: up to 8 batched 512-row bidirectional
    forwards, then one batched causal commit forward per block).  The whole
    generation is timed from the end of the prefill; the first block's
    forwards are also timed one by one with HIP events, each against its
    algorithmic HBM bytes (weights + KV read + KV written) and its GEMM +
    attention flops (8 TB/s and 2.5 PF/s dense bf16 peaks)."""
    import numpy as np
    import torch
    import workloads as W
    from self_speculative_amd import decode as D
    from self_speculative_amd.decode import prefill
    from self_speculative_amd.model import Model
    s = W.SHAPES["14b"]
    B, S_MAX, TAU, NSEQ = 32, 8, 0.9, 16
    t0 = time.time()
    w = W.make_weights(s, seed=0, threads=min(16, len(os.sched_getaffinity(0))))
    lens = W.prompt_lengths(NSEQ, 1024, 8192, seed=0)
    prompts = [W.prompt_ids(s, int(n), seed=0, index=i) for i, n in enumerate(lens)]
    model = Model(s, w, max_seqs=NSEQ, max_block=B, max_context=8192 + n_gen + 2 * B, max_rows=NSEQ * B,
                  free_host=True)
    del w
    torch.cuda.synchronize()
    log(f"14b batch: weights drawn and uploaded in {time.time() - t0:.1f}s")
    dev = model.device
    t0 = time.perf_counter()
    for i, p in enumerate(prompts):
        prefill(model, i, p)
    torch.cuda.synchronize()
    t_pf = time.perf_counter() - t0
    seqs = list(range(NSEQ))
    # the first block, forward by forward (HIP events)
    blk = torch.full((NSEQ, B), s.mask_id, dtype=torch.int32, device=dev)
    nm = torch.empty(NSEQ, dtype=torch.int32, device=dev)
    ar = torch.empty((NSEQ, B), dtype=torch.int32, device=dev)
    acc = torch.empty(NSEQ, dtype=torch.int32, device=dev)
    ev = []
    t0 = time.perf_counter()
    for step in range(S_MAX):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record()
        model.diffuse_step(seqs, blk, B, TAU, step == S_MAX - 1, nm)
        e[1].record()
        ev.append(e)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record()
    model.verify_block(seqs, blk, B, ar, acc)
    e[1].record()
    ev.append(e)
    for q in seqs:
        model.commit_kv(q, B)
    torch.cuda.synchronize()
    t_blk = time.perf_counter() - t0
    assert int((blk == s.mask_id).sum().item()) == 0
    fwd_us = [a.elapsed_time(b) * 1e3 for a, b in ev]
    # the rest of the generation: whole blocks in lockstep, timed together
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    gens = D.generate_diffusion_batch(model, prompts, n_gen - B, B, TAU, S_MAX, seqs, prefilled=True)
    torch.cuda.synchronize()
    t_rest = time.perf_counter() - t0
    t_gen = t_blk + t_rest
    n_fwd = len(fwd_us) + gens[0].forwards
    wbytes = sum(layer_weight_bytes(s).values()) * s.n_layers + s.vocab * s.d_model * 2
    kv_tok = s.n_layers * 2 * s.n_kv_heads * s.head_dim * 2
    M = NSEQ * B
    kv_read = int(sum(int(n) + B for n in lens)) * kv_tok
    nbytes = wbytes + kv_read + M * kv_tok
    params = wbytes // 2
    attn_flops = 4 * sum(int(n) + B for n in lens) * B * s.n_q_heads * s.head_dim * s.n_layers
    flops = 2 * M * params + attn_flops
    med = float(np.median(fwd_us))
    tokens = NSEQ * n_gen
    out = {"workload": "14B-shape decoder (40 layers, d 5120, 40/8 heads x 128, FFN 17408, vocab 151936), 16 sequences, "
                       f"prompt lengths U{{1024..8192}} seed 0, block 32, tau 0.9, at most 8 steps, {n_gen} generated "
                       "tokens per sequence; decode timed from the end of the prefill",
           "prompt_tokens": int(lens.sum()), "prefill_s": round(t_pf, 3),
           "prefill_tok_per_s": round(float(lens.sum()) / t_pf, 1),
           "generated_tokens": tokens, "forwards": n_fwd, "decode_s": round(t_gen, 3),
           "tokens_per_s": round(tokens / t_gen, 1), "ms_per_forward": round(t_gen / n_fwd * 1e3, 2),
           "first_block_forward_us": {"median": round(med, 1), "min": round(min(fwd_us), 1),
                                      "max": round(max(fwd_us), 1), "n": len(fwd_us)},
           "forward_bytes_first_block": nbytes, "forward_flops_first_block": flops,
           "hbm_frac": round(nbytes / (med * 1e-6) / 8e12, 4),
           "mfma_frac": round(flops / (med * 1e-6) / 2.5e15, 4)}
    log(f"14b batch: forward median {med:.0f} us, HBM {out['hbm_frac']:.3f}, MFMA {out['mfma_frac']:.3f}; "
        f"{tokens} tokens in {t_gen:.2f}s -> {out['tokens_per_s']} tok/s, prefill {out['prefill_tok_per_s']} tok/s")
    model.close()
    return out


def bench_3b(log, n_gen: int = 512, prompt_len: int = 512) -> dict:
    """The 3B-shaped decoder (28 layers, d 3072, 24/8 heads x 128, FFN 8192,
    vocab 151936), single query, a 512-token prompt and 512 generated tokens
    with block 32: block diffusion (tau 0.9, no step cap: a block takes steps
    until no MASK is left, then the causal commit forward), self-speculation
    with the natural accept lengths, and AR.  Each mode's decode is timed from
    the end of its prefill; forwards are also timed one by one with HIP events
    (32-row bidirectional, 32-row causal) against the 3B forward's bytes."""
    import numpy as np
    import torch

    import workloads as W
    from self_speculative_amd import decode as D
    from self_speculative_amd.model import Model
    s = W.SHAPES["3b"]
    B = 32
    t0 = time.time()
    w = W.make_weights(s, seed=0, threads=min(16, len(os.sched_getaffinity(0))))
    prompt = W.prompt_ids(s, prompt_len, seed=0)
    model = Model(s, w, max_seqs=3, max_block=B, max_context=prompt_len + n_gen + 2 * B, max_rows=512,
                  free_host=True)
    del w
    torch.cuda.synchronize()
    log(f"3b: weights drawn and uploaded in {time.time() - t0:.1f}s")
    dev = model.device
    out = {"workload": f"3B-shape decoder (28 layers, d 3072, 24/8 heads x 128, FFN 8192, vocab 151936), single "
                       f"query, prompt {prompt_len}, {n_gen} generated tokens, block 32; decode timed from the end of "
                       f"the prefill"}
    # warm-up
    D.generate_ar(model, prompt, 8, seq=2)
    model.seq_reset(2)
    # block diffusion: tau 0.9 and no cap; the generation's forwards are timed one by one as well
    first = D.prefill(model, 0, prompt)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g = D.generate_diffusion_batch(model, [prompt], n_gen, B, 0.9, None, [0], prefilled=True)[0]
    torch.cuda.synchronize()
    t_diff = time.perf_counter() - t0
    out["diffusion"] = {"tau": 0.9, "step_cap": None, "tokens": len(g.tokens), "forwards": g.forwards,
                        "tpf": round(g.tpf, 3), "mean_steps_per_block": round(float(np.mean(g.steps_per_block)), 2),
                        "tok_per_s": round(len(g.tokens) / t_diff, 1), "s": round(t_diff, 3)}
    log(f"3b diffusion: {len(g.tokens)} tokens, {g.forwards} forwards in {t_diff:.2f}s -> "
        f"{out['diffusion']['tok_per_s']} tok/s")
    # self-speculation, natural accept lengths (one 4-byte read of L per cycle)
    first = D.prefill(model, 1, prompt)
    run = D.SelfSpecRun(model, B, 1)
    blocks = torch.empty((n_gen, B), dtype=torch.int32, device=dev)
    ars = torch.empty((n_gen, B), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    Ls, emitted, anchor = [], 1, first.data_ptr()
    while emitted < n_gen:
        run.block, run.ar = blocks[len(Ls)], ars[len(Ls)]
        L = run.cycle(anchor, None)
        anchor = ars[len(Ls)].data_ptr() + 4 * (L - 1)
        Ls.append(L)
        emitted += L
    torch.cuda.synchronize()
    t_ss = time.perf_counter() - t0
    out["selfspec_natural"] = {"cycles": len(Ls), "decoded_tokens": n_gen - 1,
                               "mean_accept": round(float(np.mean(Ls)), 3), "tpf": round((n_gen - 1) / (2 * len(Ls)), 3),
                               "tok_per_s": round((n_gen - 1) / t_ss, 1), "s": round(t_ss, 3)}
    log(f"3b self-spec: {len(Ls)} cycles (mean L {out['selfspec_natural']['mean_accept']}) in {t_ss:.2f}s -> "
        f"{out['selfspec_natural']['tok_per_s']} tok/s")
    # AR
    model.seq_reset(0)
    ar_out = torch.empty(n_gen, dtype=torch.int32, device=dev)
    model.prefill(0, torch.as_tensor(prompt, device=dev), ar_out[0:1])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    base = ar_out.data_ptr()
    for t in range(1, n_gen):
        model.decode_ar(0, base + 4 * (t - 1), base + 4 * t)
    torch.cuda.synchronize()
    t_ar = time.perf_counter() - t0
    out["ar"] = {"decoded_tokens": n_gen - 1, "tok_per_s": round((n_gen - 1) / t_ar, 1),
                 "ms_per_token": round(t_ar / (n_gen - 1) * 1e3, 3)}
    log(f"3b AR: {out['ar']['tok_per_s']} tok/s")
    # per-forward latency at the end of the self-spec run (committed length ~ prompt + n_gen)
    blk = torch.empty(B, dtype=torch.int32, device=dev)
    ar = torch.empty(B, dtype=torch.int32, device=dev)
    acc = torch.empty(1, dtype=torch.int32, device=dev)
    ev = []
    for c in range(8):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        model.draft_block(1, anchor, B, blk)
        e[1].record()
        model.verify_block([1], blk, B, ar, acc)
        e[2].record()
        ev.append(e)
    torch.cuda.synchronize()
    n = model.seq_length(1)
    fb = forward_bytes(s, n, B)
    bid = _pct([e[0].elapsed_time(e[1]) * 1e3 for e in ev])
    cau = _pct([e[1].elapsed_time(e[2]) * 1e3 for e in ev])
    out["forward"] = {"committed_len": n, "algorithmic_bytes": fb, "bidir_M32": bid, "causal_M32": cau,
                      "hbm_frac": round(fb / (cau["median_us"] * 1e-6) / 8e12, 4)}
    log(f"3b forward at n={n}: {cau['median_us']} us, HBM {out['forward']['hbm_frac']:.3f}")
    model.close()
    return out


def cpu_baseline(s, weights, prompt, sched, log, n_cycles: int = 2) -> dict:
    """The CPU oracle (as it stands) on a bounded sample of the headline job:
    the same 1024-token prompt prefilled (setup, untimed), then the first
    ``n_cycles`` cycles of the same forced schedule (a bidirectional draft and
    a causal verify of 32 rows each, then the commit) timed at the headline's
    committed length; the rate is those cycles' tokens over their time."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 0) for i in threadpool_info()), default=0)
    except Exception:  # pragma: no cover
        blas_threads = 0
    cores = len(os.sched_getaffinity(0))
    om = O.OracleModel(s, weights)
    sess = O.OracleSession(om, keep_logits=False)
    t0 = time.time()
    first = sess.prefill(0, prompt)
    t_setup = time.time() - t0
    n0 = len(prompt)
    log(f"oracle setup (weight widening, prefill {n0}) {t_setup:.1f}s")
    g = int(first.tok[0])
    toks = 0
    t0 = time.perf_counter()
    for c in range(n_cycles):
        L = int(sched[c])
        blk, _ = sess.draft_block(0, g, 32)
        a, _, _ = sess.verify_block(0, blk)
        sess.commit_kv(0, L)
        g = int(a[L - 1])
        toks += L
    dt = time.perf_counter() - t0
    log(f"oracle {n_cycles} cycles ({toks} tokens) {dt:.1f}s")
    return {"value": round(toks / dt, 4), "unit": "tokens/s", "cores": int(blas_threads or cores),
            "kind": "oracle",
            "sample": f"the headline job's first {n_cycles} forced self-spec cycles (L = "
                      f"{', '.join(str(int(v)) for v in sched[:n_cycles])}: {toks} tokens; each a 32-row "
                      f"bidirectional draft + 32-row causal verify of the 36-layer 8B shape in float64 NumPy, then "
                      f"the commit) at committed length {n0} -> {n0 + toks}, {dt:.1f}s; the {n0}-token prompt "
                      f"prefilled first ({t_setup:.1f}s with the weight widening, untimed); host has {cores} cores"}


if __name__ == "__main__":
    sys.exit(main())
