"""Sampling at temperature > 0 on the CPU oracle -- TEST INFRASTRUCTURE ONLY.

The pages establish the self-speculation identity only at temperature 0 and
leave temperature > 0 open (fintech-frontier-insights, self-speculation
bullet and closing questions).  This module is the reading used here: the
standard lossless rejection-sampling verify, under which self-speculation
emits tokens distributed exactly as AR sampling at the same temperature.

Random numbers.  Every draw comes from Philox4x64-10 (Salmon, Moraes, Dror,
Shaw: "Parallel random numbers: as easy as 1, 2, 3", SC 2011), a counter-based
generator, so both implementations can produce the same numbers from the same
(key, counter) without sharing state:
    key     = (seed, 0)
    counter = (vocab id // 4, target position, sequence, purpose)
and word (vocab id % 4) of the output block; decisions that are not per
vocabulary id use counter word 0 = 0 and output word 0.  A 64-bit word x
becomes the uniform u = ((x >> 40) + 1/2) * 2^-24, in (0, 1) and exact in
float32 and float64.

Sampling a row at temperature T: tok = argmax over non-MASK ids v of
l_v / T + g_v with Gumbel noise g_v = -ln(-ln u_v) (purpose PURPOSE_*; ties to
the lowest id) -- an exact draw from softmax(l / T) (the Gumbel-max trick).

Self-speculation at T: the draft samples d_j from its row j (q_j, purpose
DRAFT, position n + j); the verify forward's row j - 1 gives p_j.  Draft j is
accepted iff ln u_j < ln p_j(d_j) - ln q_j(d_j) (purpose ACCEPT); at the first
rejection j the emitted token is a Gumbel-max draw from the weights
max(0, p_j - q_j) (purpose RESIDUAL, position n + j; should rounding leave no
id with p > q, the p row's own draw, purpose SAMPLE), otherwise the bonus is a
draw from the verify's last row (purpose SAMPLE, position n + B).  AR sampling
draws each token from its row with purpose SAMPLE.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

PURPOSE_DRAFT, PURPOSE_ACCEPT, PURPOSE_RESIDUAL, PURPOSE_SAMPLE = 1, 2, 3, 4

_M0, _M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157   # Philox4x64 multipliers
_W0, _W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B   # Weyl key increments
_MASK64 = (1 << 64) - 1


def philox4x64_10(counter: Sequence[int], key: Sequence[int]) -> List[int]:
    """Ten Philox rounds on a 4 x 64-bit counter block under a 2 x 64-bit key:
    each round takes the two 128-bit products M0 * c0 and M1 * c2, mixes their
    high halves with c1, c3 and the key, and bumps the key by the Weyl
    constants."""
    c0, c1, c2, c3 = (int(x) & _MASK64 for x in counter)
    k0, k1 = (int(x) & _MASK64 for x in key)
    for _ in range(10):
        p0, p1 = _M0 * c0, _M1 * c2
        c0, c1, c2, c3 = (p1 >> 64) ^ c1 ^ k0, p1 & _MASK64, (p0 >> 64) ^ c3 ^ k1, p0 & _MASK64
        k0, k1 = (k0 + _W0) & _MASK64, (k1 + _W1) & _MASK64
    return [c0, c1, c2, c3]


def philox_block_array(chunks: np.ndarray, position: int, seq: int, purpose: int, seed: int) -> np.ndarray:
    """Philox4x64-10 output words [len(chunks), 4] for counters
    (chunk, position, seq, purpose), vectorised with exact uint64 arithmetic
    (the 128-bit products are formed from 32-bit halves)."""
    c0 = np.asarray(chunks, dtype=np.uint64)
    c1 = np.full_like(c0, np.uint64(position))
    c2 = np.full_like(c0, np.uint64(seq))
    c3 = np.full_like(c0, np.uint64(purpose))
    k0, k1 = np.uint64(seed & _MASK64), np.uint64(0)
    lo32 = np.uint64(0xFFFFFFFF)

    def mulhilo(m: int, x: np.ndarray):
        a_lo, a_hi = np.uint64(m & 0xFFFFFFFF), np.uint64(m >> 32)
        b_lo, b_hi = x & lo32, x >> np.uint64(32)
        ll, lh, hl, hh = a_lo * b_lo, a_lo * b_hi, a_hi * b_lo, a_hi * b_hi
        mid = (ll >> np.uint64(32)) + (lh & lo32) + (hl & lo32)
        hi = hh + (lh >> np.uint64(32)) + (hl >> np.uint64(32)) + (mid >> np.uint64(32))
        lo = (mid << np.uint64(32)) | (ll & lo32)
        return hi, lo

    with np.errstate(over="ignore"):
        for _ in range(10):
            h0, l0 = mulhilo(_M0, c0)
            h1, l1 = mulhilo(_M1, c2)
            c0, c1, c2, c3 = h1 ^ c1 ^ k0, l1, h0 ^ c3 ^ k1, l0
            k0, k1 = k0 + np.uint64(_W0), k1 + np.uint64(_W1)
    return np.stack([c0, c1, c2, c3], axis=1)


def uniform24(x) -> np.ndarray:
    """((x >> 40) + 1/2) * 2^-24 for uint64 words x: a uniform in (0, 1)."""
    return ((np.asarray(x, dtype=np.uint64) >> np.uint64(40)).astype(np.float64) + 0.5) * 2.0 ** -24


def gumbel_noise(V: int, position: int, seq: int, purpose: int, seed: int) -> np.ndarray:
    """g_v = -ln(-ln u_v) for v < V."""
    words = philox_block_array(np.arange((V + 3) // 4), position, seq, purpose, seed).reshape(-1)[:V]
    return -np.log(-np.log(uniform24(words)))


def uniform_at(position: int, seq: int, purpose: int, seed: int) -> float:
    return float(uniform24(philox4x64_10((0, position, seq, purpose), (seed, 0))[0]))


def log_softmax_T(logits: np.ndarray, T: float, mask_id: int) -> np.ndarray:
    """ln softmax(l / T) over the non-MASK ids (MASK gets -inf)."""
    z = np.asarray(logits, dtype=np.float64) / T
    z = z.copy()
    z[mask_id] = -np.inf
    m = z.max()
    return z - (m + np.log(np.exp(z - m).sum()))


@dataclass
class Sample:
    tok: int
    logp: float      # ln p(tok) under softmax(l / T)
    gap: float       # best minus second-best perturbed score (a near-tie measure)


def gumbel_argmax(scores: np.ndarray, noise: np.ndarray) -> Sample:
    s = scores + noise
    order = np.argsort(-s, kind="stable")     # stable: lowest id first among equal scores
    tok = int(order[0])
    gap = float(s[order[0]] - s[order[1]]) if len(order) > 1 else math.inf
    return Sample(tok, float("nan"), gap)


def sample_row(logits: np.ndarray, T: float, seed: int, seq: int, position: int, purpose: int,
               mask_id: int) -> Sample:
    """A draw from softmax(l / T) over non-MASK ids by the Gumbel-max trick."""
    lp = log_softmax_T(logits, T, mask_id)
    s = gumbel_argmax(lp, gumbel_noise(len(lp), position, seq, purpose, seed))
    s.logp = float(lp[s.tok])
    return s


def residual_sample(p_logits: np.ndarray, q_logits: np.ndarray, T: float, seed: int, seq: int, position: int,
                    mask_id: int) -> Sample:
    """A draw from the weights max(0, p - q) (p, q = softmax(l / T) of the two
    rows) by the Gumbel-max trick on ln(p - q) where p > q."""
    p = np.exp(log_softmax_T(p_logits, T, mask_id))
    q = np.exp(log_softmax_T(q_logits, T, mask_id))
    w = p - q
    if not (w > 0).any():   # p == q to rounding: the p row's own sample at this position
        return sample_row(p_logits, T, seed, seq, position, PURPOSE_SAMPLE, mask_id)
    with np.errstate(divide="ignore"):
        lw = np.where(w > 0, np.log(np.where(w > 0, w, 1.0)), -np.inf)
    s = gumbel_argmax(lw, gumbel_noise(len(lw), position, seq, PURPOSE_RESIDUAL, seed))
    s.logp = float(np.log(w[s.tok] / w[w > 0].sum()))
    return s


def accept_draft(logp: float, logq: float, seed: int, seq: int, position: int):
    """(accepted, ln u - (ln p - ln q)): accept iff ln u < ln p - ln q."""
    u = uniform_at(position, seq, PURPOSE_ACCEPT, seed)
    d = math.log(u) - (logp - logq)
    return d < 0, d
