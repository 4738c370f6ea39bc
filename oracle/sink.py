"""Adaptive sink refresh decision, float64.  Test infrastructure only.

[WT] "自適應的sink和RoPE刷新": the new chunk embedding is compared with the sink set by cosine
similarity and the least similar sink is refreshed when the similarity is below a threshold
(which the page says should be set high).  Readings: the similarity of the set is the minimum
over sinks; ties go to the lowest sink index; the test is strict (alpha < tau); a zero-norm
vector has similarity 0.
"""
from __future__ import annotations

import numpy as np


def similarity_terms(h, sink_embeds) -> dict:
    """The sums a cosine decision is made from, float64: h.h, e_j.e_j and h.e_j for every sink,
    and alpha_j = h.e_j / (|h| |e_j|), 0 when a norm is 0."""
    h = np.asarray(h, np.float64)
    es = [np.asarray(e, np.float64) for e in sink_embeds]
    hh = float(h @ h)
    ee = [float(e @ e) for e in es]
    he = [float(h @ e) for e in es]
    alphas = [0.0 if hh == 0.0 or e2 == 0.0 else d / (np.sqrt(hh) * np.sqrt(e2)) for e2, d in zip(ee, he)]
    return {"hh": hh, "ee": ee, "he": he, "alphas": alphas}


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    return similarity_terms(a, [b])["alphas"][0]


def decide(h, sink_embeds, tau: float):
    """(j*, alpha_j*, replace) for embedding h against the sinks' embeddings."""
    alphas = similarity_terms(h, sink_embeds)["alphas"]
    j = int(np.argmin(alphas))            # first minimum = lowest index on ties
    return j, alphas[j], bool(alphas[j] < tau)
