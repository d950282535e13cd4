"""Lockstep parity helpers: drive the GPU model and the CPU oracle through the
same sequence of calls and compare after every call.

Token decisions must agree exactly, except where the oracle's top-2 logit
margin is below 1e-3 (a near-tie that summation order may flip); confidence
threshold and most-confident-position decisions are exempt when the oracle's
log-confidences are within 1e-3 of the threshold / of each other.  On an
exempt disagreement the GPU's inputs are overwritten with the oracle's
decision and the run continues (counted as a resync).
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

    def logits(self, gpu: torch.Tensor, ref: np.ndarray):
        err = float(np.abs(gpu.detach().cpu().numpy().astype(np.float64) - ref).max())
        self.max_logit_err = max(self.max_logit_err, err)
        return err


def tokens_agree(gpu_tok, sel: O.RowSel, rows, rep: Report) -> bool:
    """True if every listed row agrees or is exempt; exempt rows are counted."""
    ok = True
    for r in rows:
        rep.compared_tokens += 1
        if int(gpu_tok[r]) != int(sel.tok[r]):
            if sel.margin[r] < MARGIN_EXEMPT:
                rep.exempt += 1
            else:
                ok = False
                rep.notes.append(f"row {r}: gpu {int(gpu_tok[r])} oracle {int(sel.tok[r])} margin {sel.margin[r]:.3g}")
    return ok


def unmask_exempt(block_before, sel: O.RowSel, tau: float, mask_id: int) -> bool:
    """Whether a diffusion step's selection sits on a near-tie (R16 reading)."""
    masked = np.nonzero(np.asarray(block_before) == mask_id)[0]
    if masked.size == 0:
        return False
    lc = np.log(sel.conf[masked])
    if np.any(np.abs(lc - math.log(max(tau, 1e-300))) < MARGIN_EXEMPT) if tau > 0 else False:
        return True
    if masked.size > 1:
        top2 = np.sort(lc)[-2:]
        if top2[1] - top2[0] < MARGIN_EXEMPT:
            return True
    return bool(np.any(sel.margin[masked] < MARGIN_EXEMPT))
