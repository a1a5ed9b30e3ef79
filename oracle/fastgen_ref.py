"""Plain fp64 CPU oracle of FastGen's per-head profiling, compaction and decode.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py``; never by the product path.

Source: the hyper.ai summary pages of "Model Tells You What to Discard:
Adaptive KV Cache Compression for LLMs" (Ge et al., ICLR 2024), section
Method (the English text on the Korean page; the Chinese page says the same):

* two-phase inference -- profile every head while the prompt is encoded, then
  keep head-specific caches while generating (Method, first paragraph);
* the attention map A = softmax(Q K^T), the compressed cache
  K_C, V_C = f(K, V, C), and the policy choice C* = argmin CacheMemoryCost(C)
  subject to |A - softmax(Q K_C^T)| <= 1 - T with T the recover ratio
  (Method, second paragraph and its constraint equation);
* the base policies: special tokens, punctuation tokens, a local window set
  by a ratio r_l, the tokens with the largest cumulative attention set by a
  ratio r_f, and the full cache (Method, policy paragraph);
* the greedy shortlist of nested unions special, +punct, +frequent, +local,
  full (Method, shortlist equation);
* the policy picked on the prompt is reused for every generated token
  (Method, stability paragraph).

Readings taken where the pages are silent or garbled (each is listed with its
reason in the design notes of the repository):

* scores are scaled by 1/sqrt(d) and causally masked (Llama attention);
* the constraint's norm is, per query row, half the L1 distance between the
  full attention row and the softmax restricted to the kept keys, which equals
  one minus the attention mass the kept keys receive; rows (and the query
  heads sharing one KV head) are averaged.  So recovery R_k is the retained
  share of all attention mass, and the policy is the first shortlist entry
  with R_k >= T (nested entries have non-decreasing cost);
* k_f = floor(r_f n), w_l = floor(r_l n) computed in fp64;
* the cumulative attention score of key j is sum_{i >= j} A_ij over the
  prompt rows (diagonal included) and over the query heads of the group;
* the frequent set F is the k_f keys with the largest score, ties to the lower
  index, fixed after the prompt;
* row i keeps key j (j <= i) under the local base iff i - j < w_l;
* a key that several bases keep counts once, at the first level of the list
  (0 special, 1 punct, 2 frequent, 3 local, 4 full);
* CacheMemoryCost(C) is the number of prompt keys the first generated token
  (row n) keeps;
* during decode, position p attends to {j <= p : level(p, j) <= policy} and the
  cache afterwards holds {j <= p : level(p + 1, j) <= policy}.

Everything here is fp64 numpy, one KV head (with its G query heads) at a time.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

TOKEN_NORMAL, TOKEN_SPECIAL, TOKEN_PUNCT = 0, 1, 2
LEVEL_SPECIAL, LEVEL_PUNCT, LEVEL_FREQUENT, LEVEL_LOCAL, LEVEL_FULL = 0, 1, 2, 3, 4
N_LEVELS = 5

NEAR_T_WINDOW = 1e-4          # a head whose R_k lies this close to T is flagged
TIE_TAU_DEFAULT = 3e-5        # relative gap at the k-th score below which top-k is flagged
UNDERFLOW_FLOOR = 2.0 ** -100 # k-th score below this is flagged as well
ROW_BLOCK = 512


def budgets(n: int, r_l: float, r_f: float) -> tuple:
    """k_f = floor(r_f * n) frequent keys, w_l = floor(r_l * n) local window (policy paragraph)."""
    k_f = int(math.floor(float(r_f) * float(n)))
    w_l = int(math.floor(float(r_l) * float(n)))
    return k_f, w_l


def _causal_scores(q: np.ndarray, K: np.ndarray, row0: int) -> np.ndarray:
    """S_ij = q_i . k_j / sqrt(d) for query rows row0.., with -inf above the diagonal."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    m, d = q.shape
    S = (q @ K.T) / math.sqrt(d)
    i = row0 + np.arange(m)[:, None]
    j = np.arange(K.shape[0])[None, :]
    return np.where(j <= i, S, -np.inf)


def causal_attention_rows(q: np.ndarray, K: np.ndarray, row0: int) -> np.ndarray:
    """Rows row0 .. row0+m-1 of A = softmax(q K^T / sqrt(d)) under the causal mask.

    q: [m, d] query rows at positions row0.., K: [n, d].  Returns [m, n] fp64 with
    zeros above the diagonal.  (Method, second paragraph: the attention map.)
    """
    S = _causal_scores(q, K, row0)
    mx = S.max(axis=1, keepdims=True)
    E = np.exp(S - mx)
    return E / E.sum(axis=1, keepdims=True)


def _blocks(G: int, n: int):
    return [(g, r0, min(n, r0 + ROW_BLOCK)) for g in range(G) for r0 in range(0, n, ROW_BLOCK)]


def _map(fn, items, executor):
    return list(executor.map(fn, items)) if executor is not None else [fn(x) for x in items]


def column_scores(Qg: np.ndarray, K: np.ndarray, w_l: int, executor=None) -> Dict[str, np.ndarray]:
    """Per-key cumulative attention of one KV head and the per-row logsumexp.

    cum[j]  = sum_g sum_{i >= j} A^g_ij    (the cumulative attention score that
              ranks keys for the frequent policy, policy paragraph);
    band[j] = sum_g sum_{j <= i < j + w_l} A^g_ij, the part of cum that rows
              inside the local window contribute (a checked intermediate of
              the profiling kernels, not part of the method's definition);
    lse[g, i] = log sum_{j <= i} exp(q^g_i . k_j / sqrt(d)).
    Row blocks are independent; ``executor`` (e.g. a thread pool) may run them
    concurrently, their contributions are summed in block order.  A block of
    rows r0..r1-1 sees only the keys j < r1 (causal), so only those are scored.
    """
    G, n, _ = Qg.shape

    def block(item):
        g, r0, r1 = item
        S = _causal_scores(Qg[g, r0:r1], K[:r1], r0)
        mx = S.max(axis=1, keepdims=True)
        E = np.exp(S - mx)
        Z = E.sum(axis=1, keepdims=True)
        A = E / Z
        i = np.arange(r0, r1)[:, None]
        j = np.arange(r1)[None, :]
        return (mx + np.log(Z))[:, 0], A.sum(axis=0), np.where((i - j >= 0) & (i - j < w_l), A, 0.0).sum(axis=0)

    items = _blocks(G, n)
    cum = np.zeros(n, dtype=np.float64)
    band = np.zeros(n, dtype=np.float64)
    lse = np.zeros((G, n), dtype=np.float64)
    for (g, r0, r1), (l_blk, c_blk, b_blk) in zip(items, _map(block, items, executor)):
        lse[g, r0:r1] = l_blk
        cum[:r1] += c_blk
        band[:r1] += b_blk
    return {"cum": cum, "band": band, "lse": lse}


def attention_output(Qg: np.ndarray, K: np.ndarray, V: np.ndarray, executor=None) -> np.ndarray:
    """Prompt-phase attention output O^g = A^g V of one KV head's G query heads.

    This is the ordinary causal attention the model computes while it encodes
    the prompt, the pass the profiling rides on (Method, first paragraph: the
    heads are profiled during prompt encoding).  Qg: [G, n, d], K: [n, d],
    V: [n, d_v].  Returns [G, n, d_v] fp64; row blocks are independent.
    """
    Qg = np.asarray(Qg, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    G, n, _ = Qg.shape

    def block(item):
        g, r0, r1 = item
        return causal_attention_rows(Qg[g, r0:r1], K[:r1], r0) @ V[:r1]

    items = _blocks(G, n)
    out = np.zeros((G, n, V.shape[1]), dtype=np.float64)
    for (g, r0, r1), o in zip(items, _map(block, items, executor)):
        out[g, r0:r1] = o
    return out


def frequent_set(cum: np.ndarray, k_f: int) -> np.ndarray:
    """F: the k_f keys with the largest cumulative score, ties to the lower index."""
    n = cum.shape[0]
    order = sorted(range(n), key=lambda j: (-float(cum[j]), j))
    F = np.zeros(n, dtype=bool)
    F[order[:k_f]] = True
    return F


def key_levels(cls: np.ndarray, F: np.ndarray, rows: np.ndarray, w_l: int) -> np.ndarray:
    """level(i, j) for query rows ``rows`` and every key j < len(cls).

    First shortlist entry whose union keeps (i, j): 0 special, 1 punct, 2 frequent,
    3 local (i - j < w_l), 4 full only.  F may be shorter than cls (decode positions
    are never frequent).  Entries with j > i are returned as 5 (not attended).
    """
    m = len(rows)
    nk = len(cls)
    Fx = np.zeros(nk, dtype=bool)
    Fx[: len(F)] = F[: nk]
    i = np.asarray(rows)[:, None]
    j = np.arange(nk)[None, :]
    lev = np.full((m, nk), LEVEL_FULL, dtype=np.int8)
    lev = np.where(i - j < w_l, LEVEL_LOCAL, lev)
    lev = np.where(Fx[None, :], LEVEL_FREQUENT, lev)
    lev = np.where((cls == TOKEN_PUNCT)[None, :], LEVEL_PUNCT, lev)
    lev = np.where((cls == TOKEN_SPECIAL)[None, :], LEVEL_SPECIAL, lev)
    return np.where(j <= i, lev, N_LEVELS)


def row_bins(Qg: np.ndarray, K: np.ndarray, cls: np.ndarray, F: np.ndarray, w_l: int,
             executor=None) -> np.ndarray:
    """bins[g, i, l] = attention mass row i of query head g puts on keys of level l."""
    G, n, _ = Qg.shape

    def block(item):
        g, r0, r1 = item
        A = causal_attention_rows(Qg[g, r0:r1], K[:r1], r0)              # keys j < r1 (causal)
        lev = key_levels(cls[:r1], F[:r1], np.arange(r0, r1), w_l)
        return np.stack([np.where(lev == lv, A, 0.0).sum(axis=1) for lv in range(N_LEVELS)], axis=1)

    items = _blocks(G, n)
    bins = np.zeros((G, n, N_LEVELS), dtype=np.float64)
    for (g, r0, r1), b_blk in zip(items, _map(block, items, executor)):
        bins[g, r0:r1] = b_blk
    return bins


def recovery_from_bins(bins: np.ndarray) -> np.ndarray:
    """R_k = share of all attention mass kept by shortlist entry k (rows and heads averaged).

    The pages' constraint reads per row as half the L1 distance between A_i and
    the renormalised restriction to the kept keys, which is 1 - kept mass; the
    rows of the head (and of the G query heads of a KV head) are averaged.
    R_4 (full cache) is 1 by definition; the computed value is checked.
    """
    G, n, _ = bins.shape
    per_level = bins.sum(axis=(0, 1)) / float(G * n)
    R = np.cumsum(per_level)
    if abs(R[LEVEL_FULL] - 1.0) > 1e-12:
        raise AssertionError(f"full-cache recovery {R[LEVEL_FULL]!r} is not 1")
    R[LEVEL_FULL] = 1.0
    return R


def row_min_share(bins: np.ndarray) -> np.ndarray:
    """The least kept share of any row under each shortlist entry: for entry k, the minimum
    over the query heads g and rows i of sum_{l <= k} bins[g, i, l] -- the constraint of the
    Method section (second paragraph) read per row and taken at its worst row instead of
    averaged.  Entry 4 is the least row total (1 up to rounding).  A diagnostic beside R_k."""
    cum = np.cumsum(np.asarray(bins, dtype=np.float64), axis=-1)
    return cum.reshape(-1, N_LEVELS).min(axis=0)


def select_policy(R: np.ndarray, T: float) -> int:
    """Cheapest shortlist entry meeting R_k >= T (costs are non-decreasing along the list)."""
    for k in range(N_LEVELS):
        if R[k] >= T:
            return k
    return LEVEL_FULL


def head_type_map(R: np.ndarray, policies: np.ndarray, T: float) -> Dict[str, np.ndarray]:
    """Offline multi-prompt head map: one policy per KV head from many sample prompts.

    The jisaku.com glossary entry "FastGen" (section Profiling phase) profiles
    a set of representative prompts once, assigns every head a type from its
    attention over them, saves that map and applies it at inference.  Read
    here as: R [P, H, 5] holds each prompt's recovery per KV head; the map
    takes the recovery averaged over the P prompts and picks the first
    shortlist entry whose mean reaches T (the per-prompt rule applied to the
    mean); ``count`` [H, 5] tallies the per-prompt policies ``policies``
    [P, H] as the spread of that choice.
    """
    R = np.asarray(R, dtype=np.float64)
    policies = np.asarray(policies, dtype=np.int64)
    P, H, _ = R.shape
    mean = R.sum(axis=0) / float(P)
    policy = np.array([select_policy(mean[h], T) for h in range(H)], dtype=np.int64)
    count = np.zeros((H, N_LEVELS), dtype=np.int64)
    for p in range(P):
        for h in range(H):
            count[h, policies[p, h]] += 1
    return {"mean": mean, "policy": policy, "count": count}


def kept_positions(cls: np.ndarray, F: np.ndarray, w_l: int, policy: int) -> np.ndarray:
    """Prompt keys kept in the compressed cache: {j < n : level(n, j) <= policy}.

    Row n is the first generated token, so this is the cache that
    K_C, V_C = f(K, V, C) hands to generation.
    """
    n = len(cls)
    lev = key_levels(cls, F, np.array([n]), w_l)[0]          # row n never sees key n: no key n here
    return np.flatnonzero(lev <= policy).astype(np.int64)


def compact_head(K: np.ndarray, V: np.ndarray, kept: np.ndarray):
    """K_C, V_C = K[kept], V[kept] (rows in ascending position)."""
    return K[kept], V[kept]


@dataclass
class HeadProfile:
    k_f: int
    w_l: int
    lse: np.ndarray               # [G, n]
    cum: np.ndarray               # [n]
    band: np.ndarray              # [n]
    F: np.ndarray                 # [n] bool
    bins: np.ndarray              # [G, n, 5]
    R: np.ndarray                 # [5]
    policy: int
    kept: np.ndarray              # positions kept for generation
    near_T: bool
    topk_tie: bool
    kth_gap: float = field(default=float("nan"))


def topk_tie_flag(cum: np.ndarray, k_f: int, tau: float) -> tuple:
    """(flag, relative gap) of the frequent set's boundary.

    With the scores sorted in descending order, s_(k) is the k-th largest (the
    weakest key of F) and s_(k+1) the largest key left out.  The choice of F is
    fragile under rounding when s_(k) - s_(k+1) <= tau * s_(k), or when s_(k)
    has underflowed below 2^-100 (every score of the boundary is then a rounding
    residue).  With no boundary (k_f <= 0 or k_f >= n) F is every key or none
    and nothing is flagged.
    """
    n = len(cum)
    if k_f <= 0 or k_f >= n:
        return False, float("inf")
    s = np.sort(cum)[::-1]
    sk, sk1 = s[k_f - 1], s[k_f]
    gap = (sk - sk1) / sk if sk > 0 else 0.0
    return bool(sk - sk1 <= tau * sk or sk < UNDERFLOW_FLOOR), float(gap)


def near_t_flag(R: np.ndarray, T: float) -> bool:
    """A policy choice that rounding could change: some R_k of the four partial
    shortlist entries (k = 0..3) lies within NEAR_T_WINDOW of T.  R_4 = 1 by
    definition and never decides, so it is not tested."""
    R = np.asarray(R, dtype=np.float64)
    return bool(np.any(np.abs(R[:LEVEL_FULL] - T) <= NEAR_T_WINDOW))


def profile_head(Qg: np.ndarray, K: np.ndarray, cls: np.ndarray, r_l: float, r_f: float, T: float,
                 tau: float = TIE_TAU_DEFAULT, executor=None) -> HeadProfile:
    """Profile one KV head from its G query heads' prompt rows and pick its policy."""
    Qg = np.asarray(Qg, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    G, n, _ = Qg.shape
    k_f, w_l = budgets(n, r_l, r_f)
    cs = column_scores(Qg, K, w_l, executor)
    F = frequent_set(cs["cum"], k_f)
    bins = row_bins(Qg, K, cls, F, w_l, executor)
    R = recovery_from_bins(bins)
    policy = select_policy(R, T)
    kept = kept_positions(cls, F, w_l, policy)
    near = near_t_flag(R, T)
    tie, gap = topk_tie_flag(cs["cum"], k_f, tau)
    return HeadProfile(k_f, w_l, cs["lse"], cs["cum"], cs["band"], F, bins, R, policy, kept, near, tie, gap)


def profile_layer(Q: np.ndarray, K: np.ndarray, cls: np.ndarray, r_l: float, r_f: float, T: float,
                  tau: float = TIE_TAU_DEFAULT) -> List[List[HeadProfile]]:
    """profile_head over every (batch entry, KV head) of one layer.  Q: [B,Hq,n,d], K: [B,Hkv,n,d]."""
    B, Hq = Q.shape[:2]
    Hkv = K.shape[1]
    G = Hq // Hkv
    return [[profile_head(Q[b, h * G:(h + 1) * G], K[b, h], cls[b], r_l, r_f, T, tau)
             for h in range(Hkv)] for b in range(B)]


def _masked_softmax_out(qg: np.ndarray, Ks: np.ndarray, Vs: np.ndarray) -> np.ndarray:
    """softmax(q K^T / sqrt(d)) V for each of G query rows; zeros when no key is kept."""
    G, d = qg.shape
    if Ks.shape[0] == 0:
        return np.zeros((G, Vs.shape[1] if Vs.ndim == 2 else d), dtype=np.float64)
    S = (qg @ Ks.T) / math.sqrt(d)
    S = S - S.max(axis=1, keepdims=True)
    E = np.exp(S)
    return (E / E.sum(axis=1, keepdims=True)) @ Vs


def decode_incremental(K: np.ndarray, V: np.ndarray, cls: np.ndarray, F: np.ndarray, w_l: int, policy: int,
                       q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, new_cls: np.ndarray):
    """Generation with a head-specific cache, step by step.

    The cache starts as the compacted prompt keys {j < n : level(n, j) <= policy}.
    At position p = n + t the new token attends to the cache plus itself when
    level(p, p) <= policy; afterwards the cache keeps {j <= p : level(p + 1, j) <= policy},
    obtained by re-testing every cached key and the new one against row p + 1.

    q: [steps, G, d]; k_new, v_new: [steps, d]; new_cls: [steps].
    Returns (out [steps, G, d], caches: list of kept position arrays after each step).
    """
    n = len(cls)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    steps = q.shape[0]
    cls_all = np.concatenate([cls, np.asarray(new_cls, dtype=cls.dtype)])
    rows = {int(j): (K[j], V[j]) for j in kept_positions(cls, F, w_l, policy)}
    outs = np.zeros((steps, q.shape[1], q.shape[2]), dtype=np.float64)
    caches = []
    for t in range(steps):
        p = n + t
        cand = dict(rows)
        cand[p] = (np.asarray(k_new[t], dtype=np.float64), np.asarray(v_new[t], dtype=np.float64))
        lev_p = key_levels(cls_all[: p + 1], F, np.array([p]), w_l)[0]
        att = sorted(j for j in cand if lev_p[j] <= policy)
        Ks = np.stack([cand[j][0] for j in att]) if att else np.zeros((0, K.shape[1]))
        Vs = np.stack([cand[j][1] for j in att]) if att else np.zeros((0, V.shape[1]))
        outs[t] = _masked_softmax_out(np.asarray(q[t], dtype=np.float64), Ks, Vs)
        lev_next = key_levels(cls_all[: p + 1], F, np.array([p + 1]), w_l)[0]
        rows = {j: cand[j] for j in cand if lev_next[j] <= policy}
        caches.append(np.array(sorted(rows), dtype=np.int64))
    return outs, caches


def decode_tracking(K_all: np.ndarray, cls_all: np.ndarray, F: np.ndarray, w_l: int, n: int,
                    caches: Sequence[np.ndarray], q: np.ndarray, cum0: np.ndarray):
    """Attention of each generated token over its head's cache, split by level, and
    the cumulative attention score of every cached key carried through generation.

    The method reuses the prompt's policy because the accumulated attention of a
    head keeps its shape from prompt encoding into decoding (hyper.ai summary,
    Method, last paragraph, which checks accumulated scores at the prompt step and
    later decode steps).  Step t (position p = n + t) takes the cache after that
    step (``caches[t]``: kept positions, e.g. from ``decode_incremental``; with the
    full policy these are 0..p) and the step's queries q[t] [G, d]:

      a_gj    = softmax_j(q_g . k_j / sqrt(d)) over the cached positions j;
      bins[t] = (1/G) sum_g sum_{j : level(p, j) = k} a_gj    for k = 0..4;
      score_j += sum_g a_gj, where a position entering the cache starts at 0 and
              the prompt positions start at cum0 (the prompt's cumulative score).

    Returns (bins [steps, 5], score: {position: score} of the final cache).
    """
    K_all = np.asarray(K_all, dtype=np.float64)
    steps, G, d = q.shape
    score: Dict[int, float] = {}
    for j in (caches[0] if steps else []):
        if j < n:
            score[int(j)] = float(cum0[j])
    bins = np.zeros((steps, N_LEVELS), dtype=np.float64)
    for t in range(steps):
        p = n + t
        rows = np.asarray(caches[t], dtype=np.int64)
        score = {int(j): (score.get(int(j), 0.0) if j != p else 0.0) for j in rows}
        if len(rows) == 0:
            continue
        s = (np.asarray(q[t], dtype=np.float64) @ K_all[rows].T) / math.sqrt(d)
        a = np.exp(s - s.max(axis=1, keepdims=True))
        a /= a.sum(axis=1, keepdims=True)
        lev = key_levels(cls_all[: p + 1], F, np.array([p]), w_l)[0][rows]
        for k in range(N_LEVELS):
            bins[t, k] = a[:, lev == k].sum() / G
        col = a.sum(axis=0)
        for idx, j in enumerate(rows):
            score[int(j)] += col[idx]
    return bins, score


class DynamicFrequentHead:
    """Generation of one KV head under the local + frequent policy (level 3) with a
    frequent set that changes during decoding: a key leaving the local window stays
    if its cumulative attention beats the weakest frequent key, which is evicted
    in its place.

    The pages rank the frequent set by cumulative attention on the prompt and keep
    the policy fixed while generating (hyper.ai summary, Method, policy and last
    paragraphs).  This variant keeps ranking by the same score during generation,
    reading the budget k_f as fixed: at step p (position p), after the attention
    output, the key j_out = p + 1 - w_l that the window drops (a cached key of
    class normal outside the frequent set) is compared with the frequent key of
    the lowest score (ties: the larger position); j_out replaces it when its score
    is strictly larger, else j_out is dropped.  Scores: the prompt's cumulative
    score for prompt keys, 0 for a generated key when it enters, plus
    sum_g softmax(q_g K^T / sqrt(d)) over the cache after each step (as
    decode_tracking), so the decision at step p uses the scores through step p - 1.
    Frequent keys are the cached keys of class normal outside the window's ring.
    """

    def __init__(self, K: np.ndarray, V: np.ndarray, cls: np.ndarray, F: np.ndarray, w_l: int, cum0: np.ndarray):
        self.n = len(cls)
        self.w_l = int(w_l)
        self.cls = [int(c) for c in cls]
        kept = kept_positions(cls, F, w_l, LEVEL_LOCAL)
        self.kv = {int(j): (np.asarray(K[j], np.float64), np.asarray(V[j], np.float64)) for j in kept}
        self.freq = {int(j) for j in kept if F[j] and cls[j] == TOKEN_NORMAL}
        self.score = {int(j): float(cum0[j]) for j in kept}
        self.t = 0

    def _level_self(self, c: int) -> int:
        return LEVEL_SPECIAL if c == TOKEN_SPECIAL else LEVEL_PUNCT if c == TOKEN_PUNCT else \
            (LEVEL_LOCAL if self.w_l >= 1 else LEVEL_FULL)

    def step(self, q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, c_new: int, force: Optional[bool] = None,
             weakest: Optional[int] = None):
        """One generated token.  q [G, d].  ``force`` overrides the replacement decision and
        ``weakest`` the frequent key it evicts (None: the rule above; tests use them to follow
        a decision that rounding could take either way).  Returns (out [G, d], kept positions
        after the step, info {candidate, weakest, margin, replaced, runner_up_gap})."""
        p = self.n + self.t
        q = np.asarray(q, np.float64)
        new = (np.asarray(k_new, np.float64), np.asarray(v_new, np.float64))
        att = sorted(self.kv)
        Ks = [self.kv[j][0] for j in att]
        Vs = [self.kv[j][1] for j in att]
        if self._level_self(c_new) <= LEVEL_LOCAL:
            Ks.append(new[0])
            Vs.append(new[1])
        d = q.shape[1]
        out = _masked_softmax_out(q, np.array(Ks).reshape(-1, d), np.array(Vs).reshape(-1, d))
        info = {"candidate": None, "weakest": None, "margin": None, "replaced": False, "runner_up_gap": None}
        j_out = p + 1 - self.w_l
        if self.w_l >= 2 and j_out in self.kv and j_out not in self.freq and self.cls[j_out] == TOKEN_NORMAL:
            info["candidate"] = j_out
            if self.freq:
                ranked = sorted(self.freq, key=lambda j: (self.score[j], -j))
                if len(ranked) > 1:
                    info["runner_up_gap"] = self.score[ranked[1]] - self.score[ranked[0]]
                weakest = ranked[0] if weakest is None else int(weakest)
                margin = self.score[j_out] - self.score[weakest]
                replace = margin > 0.0 if force is None else bool(force)
                info.update(weakest=weakest, margin=margin, replaced=replace)
                if replace:
                    self.freq.discard(weakest)
                    del self.kv[weakest], self.score[weakest]
                    self.freq.add(j_out)
            if not info["replaced"]:
                del self.kv[j_out], self.score[j_out]
        if c_new in (TOKEN_SPECIAL, TOKEN_PUNCT) or self.w_l >= 2:
            self.kv[p] = new
            self.score[p] = 0.0
        self.cls.append(int(c_new))
        rows = sorted(self.kv)
        if rows:
            sc = (q @ np.array([self.kv[j][0] for j in rows]).T) / math.sqrt(d)
            a = np.exp(sc - sc.max(axis=1, keepdims=True))
            a /= a.sum(axis=1, keepdims=True)
            for j, w in zip(rows, a.sum(axis=0)):
                self.score[j] += float(w)
        self.t += 1
        return out, np.array(rows, dtype=np.int64), info


def decode_masked(K: np.ndarray, V: np.ndarray, cls: np.ndarray, F: np.ndarray, w_l: int, policy: int,
                  q: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, new_cls: np.ndarray,
                  steps_subset: Optional[Sequence[int]] = None):
    """The same generation computed in one shot: row p of the level-masked attention
    over the concatenated prompt + generated sequence.  Returns (out, caches) like
    ``decode_incremental``; caches[t] = {j <= p : level(p + 1, j) <= policy}.
    With ``steps_subset`` only those steps are computed (outputs and caches in that order)."""
    n = len(cls)
    steps = q.shape[0]
    ts = list(range(steps)) if steps_subset is None else [int(t) for t in steps_subset]
    K_all = np.concatenate([np.asarray(K, np.float64), np.asarray(k_new, np.float64)])
    V_all = np.concatenate([np.asarray(V, np.float64), np.asarray(v_new, np.float64)])
    cls_all = np.concatenate([cls, np.asarray(new_cls, dtype=cls.dtype)])
    outs = np.zeros((len(ts), q.shape[1], q.shape[2]), dtype=np.float64)
    caches = []
    for idx, t in enumerate(ts):
        p = n + t
        lev = key_levels(cls_all[: p + 1], F, np.array([p, p + 1]), w_l)
        att = np.flatnonzero(lev[0] <= policy)
        outs[idx] = _masked_softmax_out(np.asarray(q[t], np.float64), K_all[att], V_all[att])
        caches.append(np.flatnonzero(lev[1] <= policy).astype(np.int64))
    return outs, caches


def decode_head_from_profile(prof: HeadProfile, K, V, cls, q, k_new, v_new, new_cls,
                             policy: Optional[int] = None, F: Optional[np.ndarray] = None):
    """Incremental decode of one KV head, optionally forcing the policy / frequent set."""
    pol = prof.policy if policy is None else int(policy)
    Fs = prof.F if F is None else np.asarray(F, dtype=bool)
    return decode_incremental(K, V, cls, Fs, prof.w_l, pol, q, k_new, v_new, new_cls)


def forced_kept(cls: np.ndarray, F: np.ndarray, w_l: int, policy: int) -> np.ndarray:
    """kept_positions under a policy / frequent set given from outside (flagged heads)."""
    return kept_positions(cls, np.asarray(F, dtype=bool), w_l, int(policy))


def pairs_causal(n: int) -> int:
    return n * (n + 1) // 2


__all__: Sequence[str] = [
    "budgets", "causal_attention_rows", "attention_output", "column_scores", "frequent_set", "key_levels", "row_bins",
    "recovery_from_bins", "row_min_share", "select_policy", "kept_positions", "compact_head", "profile_head",
    "profile_layer", "decode_incremental", "decode_masked", "HeadProfile", "head_type_map",
    "decode_tracking", "DynamicFrequentHead",
]
