"""Lockstep parity helpers: drive the GPU model and the CPU oracle through the
same sequence of calls and compare after every call.

Token decisions must agree exactly, except where the oracle's top-2 logit
margin is below 1e-3 (a near-tie that summation order may flip); confidence
threshold and most-confident-position decisions are exempt when the oracle's
log-confidences are within 1e-3 of the threshold / of each other.  On an
exempt disagreement the GPU's inputs are overwritten with the oracle's
decision and the run continues (counted as a resync).

With the row's measured logit deviation eps = max_v |gpu - oracle| passed in,
the exemption widens to what that deviation can flip: an argmax can change
only if the oracle's margin is below 2 eps; a log-confidence
ln conf = -ln sum_v exp(l_v - max) moves by at most 2 eps, so a threshold
decision can change only within 2 eps of ln tau and a most-confident choice
only within 4 eps.  The floor stays 1e-3.  Deep bf16 models need this: fp32
summation alone moves 36-layer logits by about 1e-2 against float64.
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
    notes: list = field(default_factory=list)

    def logits(self, gpu: torch.Tensor, ref: np.ndarray) -> np.ndarray:
        """Record the comparison; returns the per-row max |gpu - oracle|."""
        d = np.abs(gpu.detach().cpu().numpy().astype(np.float64) - ref)
        row_err = d.reshape(d.shape[0], -1).max(axis=1) if d.ndim > 1 else d
        self.max_logit_err = max(self.max_logit_err, float(row_err.max()))
        return row_err


def _margin_bar(eps, r, k=2.0) -> float:
    return MARGIN_EXEMPT if eps is None else max(MARGIN_EXEMPT, k * float(eps[r]))


def tokens_agree(gpu_tok, sel: O.RowSel, rows, rep: Report, eps=None) -> bool:
    """True if every listed row agrees or is exempt; exempt rows are counted.
    eps: optional per-row logit deviation (indexed like sel's rows)."""
    ok = True
    for r in rows:
        rep.compared_tokens += 1
        if int(gpu_tok[r]) != int(sel.tok[r]):
            if sel.margin[r] < _margin_bar(eps, r):
                rep.exempt += 1
            else:
                ok = False
                rep.notes.append(f"row {r}: gpu {int(gpu_tok[r])} oracle {int(sel.tok[r])} margin {sel.margin[r]:.3g}")
    return ok


def unmask_exempt(block_before, sel: O.RowSel, tau: float, mask_id: int, eps=None) -> bool:
    """Whether a diffusion step's selection sits on a near-tie (R16 reading),
    widened by the per-row logit deviation eps when given."""
    masked = np.nonzero(np.asarray(block_before) == mask_id)[0]
    if masked.size == 0:
        return False
    e = np.zeros(len(sel.tok)) if eps is None else np.asarray(eps, dtype=np.float64)
    lc = np.log(sel.conf[masked])
    if tau > 0:
        bar = np.maximum(MARGIN_EXEMPT, 2 * e[masked])
        if np.any(np.abs(lc - math.log(tau)) < bar):
            return True
    if masked.size > 1:
        order = np.argsort(lc)
        i1, i0 = order[-1], order[-2]
        if lc[i1] - lc[i0] < max(MARGIN_EXEMPT, 2 * (e[masked][i1] + e[masked][i0])):
            return True
    return bool(np.any(sel.margin[masked] < np.maximum(MARGIN_EXEMPT, 2 * e[masked])))


def revise_exempt(block_before, sel: O.RowSel, tau_revise: float, mask_id: int, eps, positions) -> bool:
    """Whether differing revise decisions at ``positions`` (written, not MASK)
    sit on a near-tie: the token decision (top-2 margin within 2 eps) or the
    confidence within 2 eps of ln tau_revise (log scale, as for unmasking)."""
    e = np.asarray(eps, dtype=np.float64)
    for i in positions:
        bar = max(MARGIN_EXEMPT, 2 * float(e[i]))
        if sel.margin[i] < bar:
            continue
        if tau_revise > 0 and abs(math.log(sel.conf[i]) - math.log(tau_revise)) < bar:
            continue
        return False
    return True
