"""Brute-force policy search for tiny heads (n <= 16).

TEST INFRASTRUCTURE ONLY.  An independent, enumeration-based restatement of the
policy choice in the hyper.ai summary of "Model Tells You What to Discard"
(Method, constraint equation and shortlist equation), used to pin the oracle:

* the frequent set is found by enumerating every k_f-subset of the prompt keys
  and keeping the one with the largest total cumulative score (lexicographically
  smallest index tuple on ties) instead of sorting;
* each shortlist entry is built as an explicit union of base key sets, not as a
  level threshold;
* the constraint is evaluated literally: per query row, the full softmax row A_i
  is compared with softmax(q_i K_C^T) over the kept keys alone (zero elsewhere)
  by half the L1 distance; rows and query heads are averaged;
* CacheMemoryCost is the explicit count of prompt keys the first generated token
  keeps, and the argmin over feasible entries is taken with ties to the lower index.
"""
from __future__ import annotations

import itertools
import math
from typing import Dict

import numpy as np

SPECIAL, PUNCT = 1, 2


def _full_rows(q: np.ndarray, K: np.ndarray) -> np.ndarray:
    n, d = q.shape[0], q.shape[1]
    A = np.zeros((n, K.shape[0]))
    for i in range(n):
        s = np.array([float(np.dot(q[i], K[j])) / math.sqrt(d) for j in range(i + 1)])
        e = np.exp(s - s.max())
        A[i, : i + 1] = e / e.sum()
    return A


def _restricted_row(qi: np.ndarray, K: np.ndarray, keep: list) -> np.ndarray:
    d = qi.shape[0]
    out = np.zeros(K.shape[0])
    if not keep:
        return out
    s = np.array([float(np.dot(qi, K[j])) / math.sqrt(d) for j in keep])
    e = np.exp(s - s.max())
    out[keep] = e / e.sum()
    return out


def brute_force_head(Qg: np.ndarray, K: np.ndarray, cls: np.ndarray, k_f: int, w_l: int, T: float) -> Dict:
    Qg = np.asarray(Qg, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    G, n, _ = Qg.shape
    assert n <= 16, "enumeration is meant for tiny heads"
    rows = [_full_rows(Qg[g], K) for g in range(G)]
    cum = sum(A.sum(axis=0) for A in rows)
    best, best_sum = None, -np.inf
    for sub in itertools.combinations(range(n), k_f):      # lexicographic order
        tot = float(sum(cum[j] for j in sub))
        if tot > best_sum:                                   # strict: first (smallest) tuple wins ties
            best, best_sum = sub, tot
    F = set(best) if best is not None else set()
    specials = {j for j in range(n) if cls[j] == SPECIAL}
    puncts = {j for j in range(n) if cls[j] == PUNCT}

    def kept_for_row(entry: int, i: int) -> list:
        if entry == 4:
            return list(range(i + 1))
        keep = set(specials)
        if entry >= 1:
            keep |= puncts
        if entry >= 2:
            keep |= F
        if entry >= 3:
            keep |= {j for j in range(i + 1) if i - j < w_l}
        return sorted(j for j in keep if j <= i)

    distance = np.zeros(5)
    worst = np.zeros(5)                                     # the largest per-row distance of each entry
    for entry in range(5):
        tot = 0.0
        for g in range(G):
            for i in range(n):
                approx = _restricted_row(Qg[g, i], K, kept_for_row(entry, i))
                dist_i = 0.5 * np.abs(rows[g][i] - approx).sum()
                tot += dist_i
                worst[entry] = max(worst[entry], dist_i)
        distance[entry] = tot / (G * n)
    cost = np.array([len([j for j in kept_for_row(e, n) if j < n]) for e in range(5)])
    feasible = [e for e in range(5) if distance[e] <= 1.0 - T]
    if not feasible:
        feasible = [4]
    policy = min(feasible, key=lambda e: (cost[e], e))
    return {
        "cum": cum,
        "F": np.array([j in F for j in range(n)]),
        "distance": distance,
        "recovery": 1.0 - distance,
        "worst_row_recovery": 1.0 - worst,
        "cost": cost,
        "policy": int(policy),
        "kept": np.array([j for j in kept_for_row(policy, n) if j < n], dtype=np.int64),
    }
