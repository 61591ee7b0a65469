"""Hyperparameter screening by cosine.

The explainer ("The real work: suppressing interference") tunes Dust in two ways: a grid search
on a small token budget that keeps the setting whose loss fell most (reliable, expensive), or,
far cheaper, ranking candidate settings by the cosine between the estimate and the
backpropagation gradient on one batch, with no training at all. A high cosine on one batch does
not always mean a lower loss after training, so the cosine narrows the candidates and training
chooses among the survivors. This module is the cheap half: the estimate comes from the
library's chain, the cosine from dust_cosine_terms; the caller supplies the candidates, the
chain run per candidate and the reference gradient (its model's backward pass).
"""
from __future__ import annotations

import math
from typing import Callable, Iterable, List, Tuple

from . import dust_cosine_terms


def cosine(a, b, stream=None) -> float:
    """cos(a, b) of two fp32 device tensors of equal size (fp64 sums on the device)."""
    import torch
    if a.numel() != b.numel():
        raise ValueError("cosine: sizes differ (%d, %d)" % (a.numel(), b.numel()))
    terms = torch.empty(3, dtype=torch.float64, device=a.device)
    dust_cosine_terms(a, b, a.numel(), terms, stream)
    ab, aa, bb = terms.tolist()   # synchronises with the stream
    return ab / math.sqrt(aa * bb) if aa > 0.0 and bb > 0.0 else 0.0


def screen(candidates: Iterable, estimate: Callable, reference, keep: int | None = None,
           stream=None) -> List[Tuple[float, object]]:
    """Rank candidates by cos(estimate(candidate), reference), best first.

    estimate(candidate) returns the weight-gradient estimate (an fp32 device tensor) that the
    chain produces under that setting on the screening batch; reference is the backpropagation
    gradient of the same batch. keep limits the list to the best few, the ones to train.
    """
    ranked = sorted(((cosine(estimate(c), reference, stream), c) for c in candidates),
                    key=lambda x: -x[0])
    return ranked if keep is None else ranked[:keep]
