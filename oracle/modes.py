"""The three decoding modes on the CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only tests, the package's ``smoke()`` check and the benchmark's CPU-baseline
leg may use this module.

``OracleSession`` mirrors the library's calls (prefill, diffuse_step,
draft_block, verify_block, commit_kv, decode_ar) one for one, so a test can run
the GPU and the oracle in lockstep.  The generation loops below it are the
modes as the pages state them:

* AR: one token per forward, left to right (ai-feeds "inference: three
  modes", item 1; fintech-frontier-insights "three generation modes",
  autoregressive bullet).
* Block diffusion: a 32-token block is denoised in parallel over several
  rounds (fintech-frontier-insights, diffusion bullet; ai-feeds item 2).  Each
  round unmasks the masked positions whose confidence clears a threshold,
  and always at least the most confident one; a step budget caps the rounds
  (aimodeling English text: fewer refinement steps cut the inference budget).
  Optionally a round also revises positions already written (the pages: the
  model can go back and modify generated content; the rule is a reading).
* Self-speculation: diffusion drafts a block in parallel and AR verifies it in
  one forward (ai-feeds item 3; hotpaper abstract point (2)).  The draft is
  kept up to the first token the AR argmax disagrees with; the AR token at
  that point is emitted in its place (gsyq.cn explainer, section 2.3, the
  classic verify rule).  At temperature 0 the output equals greedy AR
  (fintech-frontier-insights, self-speculation bullet and accuracy list).

* Quadratic self-speculation (a variant the pages name, with a higher
  tokens-per-forward figure than the linear one: ai-feeds item 3;
  fintech-frontier-insights, the release summary and its TPF table; no
  algorithm is given, so this is a reading): one forward verifies the block
  causally and, in the same pass, drafts the next block for every possible
  accept length, so no separate draft forward is needed.  The candidate for
  accept length L = k + 1 is a [MASK x B] block at positions n+k+1..n+k+B
  that sees the committed prefix, block rows 0..k and, bidirectionally, its
  own rows; its row 0 sits where the bonus token will go, rows 1..B-1 become
  the next cycle's drafts behind the AR token a_k.  B + B^2 rows per forward.

Readings of open points (listed in the design notes): the row at a MASK
position predicts that position in a bidirectional forward, while causal rows
predict the next position; a self-spec draft is one bidirectional forward over
[anchor, MASK x (B-1)]; confidence is the max softmax probability over the
non-MASK vocabulary, compared with a strict ">"; confidence ties go to the
lowest position; a finished diffusion block is committed through a causal
forward, so the cache holds causal K/V in every mode.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

from .model import BIDIR, CAUSAL, KVCache, OracleModel, select_rows
from . import sampling as SP


@dataclass
class RowSel:
    tok: np.ndarray
    conf: np.ndarray
    margin: np.ndarray
    logits: Optional[np.ndarray] = None


def unmask_rule(block: np.ndarray, tok: np.ndarray, conf: np.ndarray, tau: float,
                force_all: bool, mask_id: int):
    """One denoising step's selection on one block.

    Masked set Mk = positions still holding MASK.  U = {i in Mk: conf_i > tau}
    plus the most confident i in Mk (lowest i on ties); on the last allowed
    step U = Mk.  Returns (new block, U as a sorted index array, |Mk \\ U|).
    """
    block = np.array(block, dtype=np.int32, copy=True)
    masked = np.nonzero(block == mask_id)[0]
    if masked.size == 0:
        return block, masked, 0
    if force_all:
        U = masked
    else:
        c = conf[masked]
        best = masked[int(np.argmax(c))]            # argmax: first (lowest i) on ties
        U = np.union1d(masked[c > tau], [best]).astype(np.int64)
    block[U] = tok[U]
    return block, U, int(masked.size - U.size)


def revise_rule(block: np.ndarray, tok: np.ndarray, conf: np.ndarray, tau_revise: float, mask_id: int):
    """Revision of positions already written (the pages: in diffusion mode the
    model can go back and modify content it has already generated --
    fintech-frontier-insights, three generation modes, diffusion bullet; the
    aimodeling text.  The rule is a reading: the pages give none).

    R = {i : block_i is not MASK, tok_i != block_i, conf_i > tau_revise}; the
    positions in R take tok_i.  conf <= 1, so tau_revise >= 1 revises nothing.
    Returns (new block, R as a sorted index array)."""
    block = np.array(block, dtype=np.int32, copy=True)
    R = np.nonzero((block != mask_id) & (np.asarray(tok) != block) & (np.asarray(conf) > tau_revise))[0]
    block[R] = np.asarray(tok)[R]
    return block, R


def accept_length(block: np.ndarray, ar_tok: np.ndarray) -> int:
    """L = k + 1, k = largest k <= B-1 with block[j] == ar_tok[j-1] for all 1 <= j <= k."""
    B = len(block)
    k = 0
    while k + 1 <= B - 1 and block[k + 1] == ar_tok[k]:
        k += 1
    return k + 1


class OracleSession:
    """Per-sequence caches plus the library's call surface."""

    def __init__(self, model: OracleModel, keep_logits: bool = True):
        self.model = model
        self.mask_id = model.shape.mask_id
        self.caches: Dict[int, KVCache] = {}
        self.keep_logits = keep_logits
        self.forwards = 0

    def _cache(self, seq: int) -> KVCache:
        if seq not in self.caches:
            self.caches[seq] = self.model.new_cache()
        return self.caches[seq]

    def _sel(self, logits: np.ndarray) -> RowSel:
        tok, conf, margin = select_rows(logits, self.mask_id)
        return RowSel(tok, conf, margin, logits if self.keep_logits else None)

    def committed(self, seq: int) -> int:
        return self._cache(seq).n

    # -- calls -------------------------------------------------------------
    def prefill(self, seq: int, tokens: Sequence[int]) -> RowSel:
        """Causal forward over the prompt; commits it; row P-1 gives y1."""
        c = self._cache(seq)
        assert c.n == 0
        logits = self.model.forward(c, tokens, CAUSAL, logits_rows=[len(tokens) - 1])
        c.n = len(tokens)
        self.forwards += 1
        return self._sel(logits)

    def decode_ar(self, seq: int, token: int) -> RowSel:
        """Causal forward over one token at position n; commits it."""
        c = self._cache(seq)
        logits = self.model.forward(c, [token], CAUSAL)
        c.n += 1
        self.forwards += 1
        return self._sel(logits)

    def draft_block(self, seq: int, anchor: int, B: int):
        """Bidirectional forward over [anchor, MASK x (B-1)] -> (block, rows)."""
        c = self._cache(seq)
        blk = np.full(B, self.mask_id, dtype=np.int32)
        blk[0] = anchor
        sel = self._sel(self.model.forward(c, blk, BIDIR))
        self.forwards += 1
        blk[1:] = sel.tok[1:]
        return blk, sel

    def verify_block(self, seq: int, block: Sequence[int]):
        """Causal forward over the block -> (AR argmax per row, L, rows)."""
        c = self._cache(seq)
        block = np.asarray(block, dtype=np.int32)
        sel = self._sel(self.model.forward(c, block, CAUSAL))
        self.forwards += 1
        return sel.tok.copy(), accept_length(block, sel.tok), sel

    def commit_kv(self, seq: int, n_accept: int):
        self._cache(seq).n += int(n_accept)

    def diffuse_step(self, seq: int, block: Sequence[int], tau: float, force_all: bool):
        """Bidirectional forward over the block, then the unmask rule."""
        c = self._cache(seq)
        sel = self._sel(self.model.forward(c, block, BIDIR))
        self.forwards += 1
        new, U, n_left = unmask_rule(np.asarray(block), sel.tok, sel.conf, tau, force_all, self.mask_id)
        return new, U, n_left, sel

    def diffuse_step_revise(self, seq: int, block: Sequence[int], tau: float, tau_revise: float, force_all: bool):
        """A denoising step with revision: from the same forward, the masked
        positions follow the unmask rule and the written ones the revise rule,
        both decided on the block as it was before the step.  Returns
        (new block, U, R, |Mk \\ U|, row selections)."""
        c = self._cache(seq)
        before = np.asarray(block, dtype=np.int32)
        sel = self._sel(self.model.forward(c, before, BIDIR))
        self.forwards += 1
        new, U, n_left = unmask_rule(before, sel.tok, sel.conf, tau, force_all, self.mask_id)
        revised, R = revise_rule(before, sel.tok, sel.conf, tau_revise, self.mask_id)
        new[R] = revised[R]
        return new, U, R, n_left, sel


    def verify_block_quadratic(self, seq: int, block: Sequence[int], candidates: Optional[Sequence[int]] = None):
        """One forward over the block (causal: the verify) and the candidate
        next blocks.  Candidate k (default: every k in 0..B-1, else the listed
        ones) is [MASK x B] at positions n+k+1..n+k+B; it sees the committed
        prefix, block rows 0..k and all of its own rows.  The block's causal
        K/V go to the pending rows as in ``verify_block``.

        Returns (a, L, nxt, verify rows, {k: candidate rows}): a and L as
        ``verify_block``; nxt[k] = [a_k, argmax of candidate k's rows 1..B-1],
        the next cycle's block should L be k + 1 (-1 for candidates left out).
        """
        c = self._cache(seq)
        n = c.n
        block = np.asarray(block, dtype=np.int32)
        B = len(block)
        ks = list(range(B)) if candidates is None else sorted({int(k) for k in candidates})
        T = B * (1 + len(ks))
        tokens = np.concatenate([block, np.full(T - B, self.mask_id, dtype=np.int32)])
        pos = np.concatenate([n + np.arange(B)] + [n + k + 1 + np.arange(B) for k in ks])
        vis = np.zeros((T, n + T), dtype=bool)
        vis[:, :n] = True                                        # the committed prefix
        vis[:B, n:n + B] = np.tril(np.ones((B, B), dtype=bool))  # the verify rows: causal
        for ci, k in enumerate(ks):
            r0 = B * (1 + ci)
            vis[r0:r0 + B, n:n + k + 1] = True                   # block rows 0..k
            vis[r0:r0 + B, n + r0:n + r0 + B] = True             # its own rows
        logits = self.model.forward_masked(c, tokens, pos, vis, n_write=B)
        self.forwards += 1
        sel = self._sel(logits[:B])
        a = sel.tok.copy()
        nxt = np.full((B, B), -1, dtype=np.int32)
        cands = {}
        for ci, k in enumerate(ks):
            cs = self._sel(logits[B * (1 + ci):B * (2 + ci)])
            cands[k] = cs
            nxt[k, 0] = a[k]
            nxt[k, 1:] = cs.tok[1:]
        return a, accept_length(block, a), nxt, sel, cands

    # -- sampling at temperature T > 0 (see oracle/sampling.py) ---------------
    # A sampled token's position is the absolute position it will occupy:
    # prefill of P tokens -> P; an AR step on the token at position n -> n + 1;
    # draft row j -> n + j; verify row j -> n + j + 1.
    def prefill_sample(self, seq: int, tokens: Sequence[int], T: float, seed: int) -> SP.Sample:
        c = self._cache(seq)
        assert c.n == 0
        logits = self.model.forward(c, tokens, CAUSAL, logits_rows=[len(tokens) - 1])
        c.n = len(tokens)
        self.forwards += 1
        return SP.sample_row(logits[0], T, seed, seq, len(tokens), SP.PURPOSE_SAMPLE, self.mask_id)

    def decode_ar_sample(self, seq: int, token: int, T: float, seed: int):
        c = self._cache(seq)
        n = c.n
        logits = self.model.forward(c, [token], CAUSAL)
        c.n += 1
        self.forwards += 1
        return SP.sample_row(logits[0], T, seed, seq, n + 1, SP.PURPOSE_SAMPLE, self.mask_id), logits

    def draft_block_sample(self, seq: int, anchor: int, B: int, T: float, seed: int):
        """Bidirectional forward over [anchor, MASK x (B-1)]; row j >= 1 draws
        d_j (purpose DRAFT, position n + j).  -> (block, logits, samples)."""
        c = self._cache(seq)
        n = c.n
        blk = np.full(B, self.mask_id, dtype=np.int32)
        blk[0] = anchor
        logits = self.model.forward(c, blk, BIDIR)
        self.forwards += 1
        smp = [None] + [SP.sample_row(logits[j], T, seed, seq, n + j, SP.PURPOSE_DRAFT, self.mask_id)
                        for j in range(1, B)]
        for j in range(1, B):
            blk[j] = smp[j].tok
        return blk, logits, smp

    def verify_block_sample(self, seq: int, block: Sequence[int], draft_logits: np.ndarray, T: float, seed: int):
        """Causal forward over the drafted block; rejection-sampling verify.
        -> (L, emitted token, verify logits, details): L - 1 drafts accepted,
        the emitted token follows them (a residual draw at the first
        rejection, else the bonus from the last row)."""
        c = self._cache(seq)
        n = c.n
        block = np.asarray(block, dtype=np.int32)
        B = len(block)
        logits = self.model.forward(c, block, CAUSAL)
        self.forwards += 1
        k = 0
        margins = []
        for j in range(1, B):
            logp = float(SP.log_softmax_T(logits[j - 1], T, self.mask_id)[block[j]])
            logq = float(SP.log_softmax_T(draft_logits[j], T, self.mask_id)[block[j]])
            ok, d = SP.accept_draft(logp, logq, seed, seq, n + j)
            margins.append(d)
            if not ok:
                break
            k += 1
        if k < B - 1:
            out = SP.residual_sample(logits[k], draft_logits[k + 1], T, seed, seq, n + k + 1, self.mask_id)
        else:
            out = SP.sample_row(logits[B - 1], T, seed, seq, n + B, SP.PURPOSE_SAMPLE, self.mask_id)
        return k + 1, out.tok, logits, {"accept_margins": margins, "emitted": out}


# -- generation loops -----------------------------------------------------------
@dataclass
class GenResult:
    tokens: List[int]
    forwards: int
    accept_lengths: List[int] = field(default_factory=list)
    steps_per_block: List[int] = field(default_factory=list)
    margins: List[float] = field(default_factory=list)
    revisions: List[int] = field(default_factory=list)

    @property
    def tpf(self) -> float:
        return len(self.tokens) / max(1, self.forwards)


def generate_ar(model: OracleModel, prompt: Sequence[int], n_tokens: int, seq: int = 0) -> GenResult:
    sess = OracleSession(model, keep_logits=False)
    first = sess.prefill(seq, prompt)
    toks, margins = [int(first.tok[0])], [float(first.margin[0])]
    while len(toks) < n_tokens:
        r = sess.decode_ar(seq, toks[-1])
        toks.append(int(r.tok[0]))
        margins.append(float(r.margin[0]))
    return GenResult(toks, sess.forwards - 1, margins=margins)


def generate_selfspec(model: OracleModel, prompt: Sequence[int], n_tokens: int, B: int,
                      forced: Optional[Sequence[int]] = None, seq: int = 0) -> GenResult:
    """Linear self-speculation.  ``forced`` replaces the natural accept length
    cycle by cycle (a throughput schedule; the output is then not AR's)."""
    sess = OracleSession(model, keep_logits=False)
    first = sess.prefill(seq, prompt)
    toks = [int(first.tok[0])]
    Ls: List[int] = []
    cyc = 0
    while len(toks) < n_tokens:
        blk, _ = sess.draft_block(seq, toks[-1], B)
        a, L, _ = sess.verify_block(seq, blk)
        if forced is not None:
            L = int(forced[cyc])
        sess.commit_kv(seq, L)
        toks += [int(t) for t in blk[1:L]] + [int(a[L - 1])]
        Ls.append(L)
        cyc += 1
    return GenResult(toks[:n_tokens], sess.forwards - 1, accept_lengths=Ls)


def generate_selfspec_quadratic(model: OracleModel, prompt: Sequence[int], n_tokens: int, B: int,
                                forced: Optional[Sequence[int]] = None, seq: int = 0) -> GenResult:
    """Quadratic self-speculation: a plain draft forward drafts the first
    block; after that every cycle is one forward that verifies the block and
    holds the next block for each accept length.  ``forced`` as in
    ``generate_selfspec``."""
    sess = OracleSession(model, keep_logits=False)
    first = sess.prefill(seq, prompt)
    toks = [int(first.tok[0])]
    blk, _ = sess.draft_block(seq, toks[-1], B)
    Ls: List[int] = []
    cyc = 0
    while len(toks) < n_tokens:
        a, L, nxt, _, _ = sess.verify_block_quadratic(seq, blk)
        if forced is not None:
            L = int(forced[cyc])
        sess.commit_kv(seq, L)
        toks += [int(t) for t in blk[1:L]] + [int(a[L - 1])]
        Ls.append(L)
        blk = nxt[L - 1]
        cyc += 1
    return GenResult(toks[:n_tokens], sess.forwards - 1, accept_lengths=Ls)


def generate_diffusion(model: OracleModel, prompt: Sequence[int], n_tokens: int, B: int,
                       tau: float, max_steps: Optional[int] = None, seq: int = 0,
                       tau_revise: Optional[float] = None) -> GenResult:
    """Block diffusion: each block starts all-MASK; steps until none is left
    (step ``max_steps``-1 unmasks everything); then a causal commit forward.
    With ``tau_revise`` every step also applies the revise rule to the
    positions already written (the steps still end when no MASK is left)."""
    sess = OracleSession(model, keep_logits=False)
    sess.prefill(seq, prompt)
    mask = model.shape.mask_id
    toks: List[int] = []
    steps: List[int] = []
    revs: List[int] = []
    while len(toks) < n_tokens:
        blk = np.full(B, mask, dtype=np.int32)
        s = nrev = 0
        while True:
            force = max_steps is not None and s == max_steps - 1
            if tau_revise is None:
                blk, _, left, _ = sess.diffuse_step(seq, blk, tau, force)
            else:
                blk, _, R, left, _ = sess.diffuse_step_revise(seq, blk, tau, tau_revise, force)
                nrev += len(R)
            s += 1
            if left == 0:
                break
        sess.verify_block(seq, blk)
        sess.commit_kv(seq, B)
        toks += [int(t) for t in blk]
        steps.append(s)
        revs.append(nrev)
    return GenResult(toks[:n_tokens], sess.forwards - 1, steps_per_block=steps, revisions=revs)


def generate_diffusion_batch(model: OracleModel, prompts: Sequence[Sequence[int]], n_tokens: int,
                             B: int, tau: float, max_steps: Optional[int] = None,
                             tau_revise: Optional[float] = None):
    """Several sequences in lockstep per block.  In the oracle the sequences
    never interact, so this is each sequence decoded on its own."""
    return [generate_diffusion(model, p, n_tokens, B, tau, max_steps, seq=i, tau_revise=tau_revise)
            for i, p in enumerate(prompts)]


def generate_ar_sample(model: OracleModel, prompt: Sequence[int], n_tokens: int, T: float, seed: int,
                       seq: int = 0) -> GenResult:
    """AR sampling at temperature T (purpose SAMPLE at every position)."""
    sess = OracleSession(model, keep_logits=False)
    first = sess.prefill_sample(seq, prompt, T, seed)
    toks, gaps = [first.tok], [first.gap]
    while len(toks) < n_tokens:
        smp, _ = sess.decode_ar_sample(seq, toks[-1], T, seed)
        toks.append(smp.tok)
        gaps.append(smp.gap)
    return GenResult(toks, sess.forwards - 1, margins=gaps)


def generate_selfspec_sample(model: OracleModel, prompt: Sequence[int], n_tokens: int, B: int, T: float,
                             seed: int, seq: int = 0) -> GenResult:
    """Self-speculation at temperature T with the rejection-sampling verify."""
    sess = OracleSession(model, keep_logits=False)
    first = sess.prefill_sample(seq, prompt, T, seed)
    toks = [first.tok]
    Ls: List[int] = []
    margins = [first.gap]       # every decision's distance from flipping (Gumbel gaps, |ln u - ln p/q|)
    while len(toks) < n_tokens:
        blk, dlog, smp = sess.draft_block_sample(seq, toks[-1], B, T, seed)
        L, nxt, _, det = sess.verify_block_sample(seq, blk, dlog, T, seed)
        margins += [x.gap for x in smp[1:]] + [abs(d) for d in det["accept_margins"]] + [det["emitted"].gap]
        sess.commit_kv(seq, L)
        toks += [int(t) for t in blk[1:L]] + [int(nxt)]
        Ls.append(L)
    return GenResult(toks[:n_tokens], sess.forwards - 1, accept_lengths=Ls, margins=margins)
