"""Lockstep parity helpers: drive the GPU model and the CPU oracle through the
same sequence of calls and compare after every call.

The bar (the near-tie reading of the parity rule, R16): token ids, accept
lengths and unmask sets must agree exactly, except where the oracle's decision
sits on a near-tie --
  * a token whose oracle top-2 logit margin is below 1e-3;
  * a threshold decision whose oracle log-confidence is within 1e-3 of ln tau;
  * a most-confident-position choice whose two best oracle log-confidences are
    within 1e-3 of each other.
On such an exempt disagreement the GPU's inputs are overwritten with the
oracle's decision and the run continues (a resync).  Any other disagreement is
a failure, and every resync must follow an exempt decision.

The row's measured logit deviation eps = max_v |gpu - oracle| is reported as a
diagnostic only: ``near_ties`` counts the compared decisions whose oracle
margin lies between 1e-3 and 2 eps -- decisions that a deviation of that size
could in principle flip, and which nevertheless had to agree.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle as O

MARGIN_EXEMPT = 1e-3


@dataclass
class Report:
    max_logit_err: float = 0.0
    compared_tokens: int = 0
    exempt: int = 0
    resyncs: int = 0
    near_ties: int = 0
    notes: list = field(default_factory=list)

    def logits(self, gpu: torch.Tensor, ref: np.ndarray) -> np.ndarray:
        """Record the comparison; returns the per-row max |gpu - oracle|."""
        d = np.abs(gpu.detach().cpu().numpy().astype(np.float64) - ref)
        row_err = d.reshape(d.shape[0], -1).max(axis=1) if d.ndim > 1 else d
        self.max_logit_err = max(self.max_logit_err, float(row_err.max()))
        return row_err

    def resync(self):
        """Count a resync; it must follow an exempt (near-tie) decision."""
        self.resyncs += 1
        assert self.resyncs <= self.exempt, f"resync {self.resyncs} without an exempt decision: {self.notes}"

    def summary(self) -> str:
        return (f"max|dlogit| {self.max_logit_err:.3e}, tokens {self.compared_tokens}, exempt {self.exempt}, "
                f"resyncs {self.resyncs}, near-ties within 2 eps (agreed) {self.near_ties}")

    def assert_strict(self):
        """Every disagreement was a near-tie of the oracle (margin < 1e-3) and
        every resync followed one."""
        assert self.resyncs <= self.exempt, self.summary()
        assert not self.notes, self.notes


def tokens_agree(gpu_tok, sel: O.RowSel, rows, rep: Report, eps=None) -> bool:
    """True if every listed row agrees or is a near-tie (oracle margin < 1e-3);
    exempt rows are counted.  eps: optional per-row logit deviation (indexed
    like sel's rows), used only for the near-tie diagnostic."""
    ok = True
    for r in rows:
        rep.compared_tokens += 1
        m = float(sel.margin[r])
        if int(gpu_tok[r]) != int(sel.tok[r]):
            if m < MARGIN_EXEMPT:
                rep.exempt += 1
            else:
                ok = False
                rep.notes.append(f"row {r}: gpu {int(gpu_tok[r])} oracle {int(sel.tok[r])} margin {m:.3g}"
                                 + ("" if eps is None else f" (row eps {float(eps[r]):.3g})"))
        elif eps is not None and MARGIN_EXEMPT <= m < 2 * float(eps[r]):
            rep.near_ties += 1
    return ok


def accept_exempt(vsel: O.RowSel, gL: int, oL: int, rep: Report) -> bool:
    """Accept lengths differ: allowed only through a near-tie argmax at the
    first position where they part (the verify row min(L) - 1)."""
    k = min(gL, oL) - 1
    if vsel.margin[k] < MARGIN_EXEMPT:
        rep.exempt += 1
        return True
    rep.notes.append(f"accept length gpu {gL} oracle {oL}: verify row {k} margin {float(vsel.margin[k]):.3g}")
    return False


def unmask_exempt(block_before, sel: O.RowSel, tau: float, mask_id: int, eps=None) -> bool:
    """Whether a diffusion step's selection sits on a near-tie (R16): a masked
    position's log-confidence within 1e-3 of ln tau, the two most confident
    masked positions within 1e-3 of each other, or a masked position's token
    margin below 1e-3.  eps is accepted for call compatibility and unused."""
    masked = np.nonzero(np.asarray(block_before) == mask_id)[0]
    if masked.size == 0:
        return False
    lc = np.log(sel.conf[masked])
    if tau > 0 and np.any(np.abs(lc - math.log(tau)) < MARGIN_EXEMPT):
        return True
    if masked.size > 1:
        order = np.argsort(lc)
        if lc[order[-1]] - lc[order[-2]] < MARGIN_EXEMPT:
            return True
    return bool(np.any(sel.margin[masked] < MARGIN_EXEMPT))


def revise_exempt(block_before, sel: O.RowSel, tau_revise: float, mask_id: int, eps, positions) -> bool:
    """Whether differing revise decisions at ``positions`` (written, not MASK)
    sit on a near-tie: the token's top-2 margin below 1e-3, or its
    log-confidence within 1e-3 of ln tau_revise."""
    for i in positions:
        if sel.margin[i] < MARGIN_EXEMPT:
            continue
        if tau_revise > 0 and abs(math.log(sel.conf[i]) - math.log(tau_revise)) < MARGIN_EXEMPT:
            continue
        return False
    return True
