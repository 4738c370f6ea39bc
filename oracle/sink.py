"""Adaptive sink refresh decision, float64.  Test infrastructure only.

[WT] "自適應的sink和RoPE刷新": the new chunk embedding is compared with the sink set by cosine
similarity and the least similar sink is refreshed when the similarity is below a threshold
(which the page says should be set high).  Readings: the similarity of the set is the minimum
over sinks; ties go to the lowest sink index; the test is strict (alpha < tau); a zero-norm
vector has similarity 0.
"""
from __future__ import annotations

import numpy as np


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    na, nb = np.sqrt(a @ a), np.sqrt(b @ b)
    if na == 0.0 or nb == 0.0:
        return 0.0
    return float((a @ b) / (na * nb))


def decide(h, sink_embeds, tau: float):
    """(j*, alpha_j*, replace) for embedding h against the sinks' embeddings."""
    alphas = [cosine(h, e) for e in sink_embeds]
    j = int(np.argmin(alphas))            # first minimum = lowest index on ties
    return j, alphas[j], bool(alphas[j] < tau)
