"""The three decoding modes driven from the host over the library's calls.

* ``generate_ar``: prefill, then one ``decode_ar`` per token.  Tokens stay on
  the device; no host synchronisation inside the loop.
* ``generate_selfspec``: per cycle ``draft_block`` (bidirectional forward over
  [anchor, MASK x (B-1)]), ``verify_block`` (causal forward), ``commit_kv(L)``.
  With a forced accept-length schedule the host knows L in advance and the
  loop never synchronises; with the natural L one 4-byte read per cycle.
* ``generate_selfspec_quadratic``: one ``draft_block`` for the first block,
  then per cycle one ``verify_block_quadratic`` (the verify plus a candidate
  next block for every accept length) and ``commit_kv(L)``; the next block is
  row L-1 of the cycle's output, passed by address.
* ``generate_diffusion``: per block, ``diffuse_step`` until no MASK is left
  (step ``max_steps``-1 unmasks everything), then ``verify_block`` +
  ``commit_kv(B)`` commit the block's causal K/V.  Several sequences step in
  lockstep; a finished sequence leaves the later step forwards.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

from .model import Model


@dataclass
class GpuGen:
    tokens: List[int]
    forwards: int
    accept_lengths: List[int] = field(default_factory=list)
    steps_per_block: List[int] = field(default_factory=list)

    @property
    def tpf(self) -> float:
        return len(self.tokens) / max(1, self.forwards)


def _ids(x, dev) -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=dev)


def prefill(model: Model, seq: int, prompt) -> torch.Tensor:
    dev = model.device
    nxt = torch.empty(1, dtype=torch.int32, device=dev)
    model.prefill(seq, _ids(prompt, dev), nxt)
    return nxt


def generate_ar(model: Model, prompt, n_tokens: int, seq: int = 0) -> GpuGen:
    dev = model.device
    out = torch.empty(n_tokens, dtype=torch.int32, device=dev)
    model.prefill(seq, _ids(prompt, dev), out[0:1])
    base = out.data_ptr()
    for t in range(1, n_tokens):
        model.decode_ar(seq, base + 4 * (t - 1), base + 4 * t)
    return GpuGen(out.cpu().tolist(), n_tokens - 1)


class SelfSpecRun:
    """Self-speculation with per-cycle device buffers (reused ring)."""

    def __init__(self, model: Model, B: int, seq: int = 0):
        self.m, self.B, self.seq = model, B, seq
        dev = model.device
        self.block = torch.empty(B, dtype=torch.int32, device=dev)
        self.ar = torch.empty(B, dtype=torch.int32, device=dev)
        self.acc = torch.empty(1, dtype=torch.int32, device=dev)
        self.acc_host = torch.empty(1, dtype=torch.int32, pin_memory=True)

    def cycle(self, anchor_addr: int, forced_L: Optional[int]) -> int:
        """One draft + verify + commit.  Returns L (host value); for natural L
        this synchronises on a 4-byte copy."""
        m = self.m
        m.draft_block(self.seq, anchor_addr, self.B, self.block)
        m.verify_block([self.seq], self.block, self.B, self.ar, self.acc)
        if forced_L is None:
            self.acc_host.copy_(self.acc, non_blocking=True)
            m.stream.synchronize()
            L = int(self.acc_host[0])
        else:
            L = int(forced_L)
        m.commit_kv(self.seq, L)
        return L


def generate_selfspec(model: Model, prompt, n_tokens: int, B: int, forced: Optional[Sequence[int]] = None,
                      seq: int = 0) -> GpuGen:
    dev = model.device
    first = prefill(model, seq, prompt)
    run = SelfSpecRun(model, B, seq)
    n_cyc_max = n_tokens  # L >= 1 per cycle
    blocks = torch.empty((n_cyc_max, B), dtype=torch.int32, device=dev)
    ars = torch.empty((n_cyc_max, B), dtype=torch.int32, device=dev)
    Ls: List[int] = []
    emitted = 1
    anchor = first.data_ptr()
    while emitted < n_tokens:
        c = len(Ls)
        run.block, run.ar = blocks[c], ars[c]
        L = run.cycle(anchor, None if forced is None else forced[c])
        Ls.append(L)
        emitted += L
        anchor = ars[c].data_ptr() + 4 * (L - 1)
    bl, ar = blocks[: len(Ls)].cpu().numpy(), ars[: len(Ls)].cpu().numpy()
    toks = [int(first.item())]
    for c, L in enumerate(Ls):
        toks += [int(t) for t in bl[c, 1:L]] + [int(ar[c, L - 1])]
    return GpuGen(toks[:n_tokens], 2 * len(Ls), accept_lengths=Ls)


class QuadSpecRun:
    """Quadratic self-speculation with per-cycle device outputs: cycle c
    writes ar[c], the accept length and nexts[c] [B][B]; the block of cycle
    c + 1 is row L - 1 of nexts[c]."""

    def __init__(self, model: Model, B: int, seq: int, n_cycles: int):
        self.m, self.B, self.seq = model, B, seq
        dev = model.device
        self.first_block = torch.empty(B, dtype=torch.int32, device=dev)
        self.ars = torch.empty((n_cycles, B), dtype=torch.int32, device=dev)
        self.nexts = torch.empty((n_cycles, B, B), dtype=torch.int32, device=dev)
        self.acc = torch.empty(1, dtype=torch.int32, device=dev)
        self.acc_host = torch.empty(1, dtype=torch.int32, pin_memory=True)
        self.block_addr = self.first_block.data_ptr()

    def draft_first(self, anchor_addr: int):
        self.m.draft_block(self.seq, anchor_addr, self.B, self.first_block)
        self.block_addr = self.first_block.data_ptr()

    def cycle(self, c: int, forced_L: Optional[int]) -> int:
        """One quadratic forward + commit.  Returns L (host value); for natural
        L this synchronises on a 4-byte copy."""
        m = self.m
        m.verify_block_quadratic(self.seq, self.block_addr, self.B, self.ars[c], self.acc, self.nexts[c])
        if forced_L is None:
            self.acc_host.copy_(self.acc, non_blocking=True)
            m.stream.synchronize()
            L = int(self.acc_host[0])
        else:
            L = int(forced_L)
        m.commit_kv(self.seq, L)
        self.block_addr = self.nexts[c].data_ptr() + 4 * self.B * (L - 1)
        return L


def generate_selfspec_quadratic(model: Model, prompt, n_tokens: int, B: int,
                                forced: Optional[Sequence[int]] = None, seq: int = 0) -> GpuGen:
    first = prefill(model, seq, prompt)
    run = QuadSpecRun(model, B, seq, n_tokens)
    run.draft_first(first.data_ptr())
    Ls: List[int] = []
    emitted = 1
    while emitted < n_tokens:
        L = run.cycle(len(Ls), None if forced is None else forced[len(Ls)])
        Ls.append(L)
        emitted += L
    ar = run.ars[: len(Ls)].cpu().numpy()
    nx = run.nexts[: len(Ls)].cpu().numpy()
    blk = run.first_block.cpu().numpy()
    toks = [int(first.item())]
    for c, L in enumerate(Ls):
        toks += [int(t) for t in blk[1:L]] + [int(ar[c, L - 1])]
        blk = nx[c, L - 1]
    return GpuGen(toks[:n_tokens], 1 + len(Ls), accept_lengths=Ls)


def generate_diffusion_batch(model: Model, prompts: Sequence, n_tokens: int, B: int, tau: float,
                             max_steps: Optional[int] = None, seqs: Optional[Sequence[int]] = None,
                             tau_revise: Optional[float] = None, prefilled: bool = False) -> List[GpuGen]:
    """Block diffusion for several sequences in lockstep per block; with
    ``tau_revise`` each step also rewrites written positions
    (``sdm_diffuse_step_revise``).  ``prefilled``: the sequences already hold
    their prompts (the prefill is not repeated)."""
    dev = model.device
    seqs = list(seqs) if seqs is not None else list(range(len(prompts)))
    if not prefilled:
        for s, p in zip(seqs, prompts):
            prefill(model, s, p)
    mask = model.shape.mask_id
    n = len(seqs)
    out = [GpuGen([], 0) for _ in seqs]
    blk = torch.empty((n, B), dtype=torch.int32, device=dev)
    nm = torch.empty(n, dtype=torch.int32, device=dev)
    nm_host = torch.empty(n, dtype=torch.int32, pin_memory=True)
    ar = torch.empty((n, B), dtype=torch.int32, device=dev)
    acc = torch.empty(n, dtype=torch.int32, device=dev)
    while len(out[0].tokens) < n_tokens:
        blk.fill_(mask)
        active = list(range(n))
        steps = [0] * n
        s = 0
        while active:
            force = max_steps is not None and s == max_steps - 1
            idx = torch.as_tensor(active, device=dev)
            sub = blk[idx].contiguous()
            subn = nm[: len(active)]
            if tau_revise is None:
                model.diffuse_step([seqs[i] for i in active], sub, B, tau, force, subn)
            else:
                model.diffuse_step_revise([seqs[i] for i in active], sub, B, tau, tau_revise, force, subn)
            blk[idx] = sub
            nm_host[: len(active)].copy_(subn, non_blocking=True)
            model.stream.synchronize()
            left = nm_host[: len(active)].tolist()
            for i in active:
                steps[i] += 1
                out[i].forwards += 1
            active = [i for i, k in zip(active, left) if k > 0]
            s += 1
        model.verify_block(seqs, blk, B, ar, acc)
        for s_ in seqs:
            model.commit_kv(s_, B)
        host = blk.cpu().numpy()
        for i in range(n):
            out[i].tokens += [int(t) for t in host[i]]
            out[i].steps_per_block.append(steps[i])
            out[i].forwards += 1
    for g in out:
        g.tokens = g.tokens[:n_tokens]
    return out


def generate_diffusion(model: Model, prompt, n_tokens: int, B: int, tau: float, max_steps: Optional[int] = None,
                       seq: int = 0, tau_revise: Optional[float] = None) -> GpuGen:
    return generate_diffusion_batch(model, [prompt], n_tokens, B, tau, max_steps, [seq], tau_revise)[0]


def generate_ar_sample(model: Model, prompt, n_tokens: int, T: float, seed: int, seq: int = 0) -> GpuGen:
    """AR sampling at temperature T: ``prefill_sample`` then one
    ``decode_ar_sample`` per token, tokens kept on the device."""
    dev = model.device
    out = torch.empty(n_tokens, dtype=torch.int32, device=dev)
    model.prefill_sample(seq, _ids(prompt, dev), T, seed, out[0:1])
    base = out.data_ptr()
    for t in range(1, n_tokens):
        model.decode_ar_sample(seq, base + 4 * (t - 1), T, seed, base + 4 * t)
    return GpuGen([int(v) for v in out.cpu().tolist()], n_tokens - 1)


def generate_selfspec_sample(model: Model, prompt, n_tokens: int, B: int, T: float, seed: int,
                             seq: int = 0) -> GpuGen:
    """Self-speculation at temperature T: ``draft_block_sample`` +
    ``verify_block_sample`` (rejection-sampling verify) + ``commit_kv(L)``;
    one 4-byte read of L per cycle."""
    dev = model.device
    V = model.shape.vocab
    nxt = torch.empty(1, dtype=torch.int32, device=dev)
    model.prefill_sample(seq, _ids(prompt, dev), T, seed, nxt)
    blk = torch.empty(B, dtype=torch.int32, device=dev)
    dlog = torch.empty((B, V), dtype=torch.float32, device=dev)
    dstat = torch.empty((2, B), dtype=torch.float32, device=dev)
    acc = torch.empty(1, dtype=torch.int32, device=dev)
    acc_host = torch.empty(1, dtype=torch.int32, pin_memory=True)
    toks = [int(nxt.item())]
    Ls: List[int] = []
    fw = 0
    while len(toks) < n_tokens:
        model.draft_block_sample(seq, nxt, B, T, seed, blk, dlog, dstat)
        model.verify_block_sample(seq, blk, B, T, seed, dlog, dstat, acc, nxt)
        acc_host.copy_(acc, non_blocking=True)
        model.stream.synchronize()
        L = int(acc_host.item())
        model.commit_kv(seq, L)
        toks += blk[1:L].cpu().tolist() + [int(nxt.item())]
        Ls.append(L)
        fw += 2
    return GpuGen(toks[:n_tokens], fw, accept_lengths=Ls)
