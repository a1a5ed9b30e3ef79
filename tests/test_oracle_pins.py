"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test ties the oracle to something other than itself: exact closed forms
(uniform attention), an enumeration-based restatement of the policy choice
(brute force over frequent subsets, literal half-L1 constraint, explicit memory
cost), library routines (torch SDPA in float64 on the CPU, scipy logsumexp, a
stable argsort), invariants of nested unions, planted synthetic heads, and two
independent decode routes.  A last group plants mistakes in the oracle and
checks that a pin catches each of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import fastgen_ref as ref
from oracle.brute import brute_force_head
from synth import inputs as syn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "uniform_closed_form.json")


def _ratio_for(k, n):
    """A ratio r with floor(r * n) == k."""
    return (k + 0.5) / n


def _random_head(rng, n, d, G, scale=1.0):
    Qg = rng.standard_normal((G, n, d)) * scale
    K = rng.standard_normal((n, d)) * scale
    V = rng.standard_normal((n, d))
    cls = np.zeros(n, dtype=np.uint8)
    cls[0] = ref.TOKEN_SPECIAL
    if n > 1:
        m = rng.random(n - 1)
        cls[1:][m < 0.1] = ref.TOKEN_SPECIAL
        cls[1:][(m >= 0.1) & (m < 0.3)] = ref.TOKEN_PUNCT
    return Qg, K, V, cls


def _planted_head(rng, n, d, G, kind):
    """Tiny head whose attention concentrates on one key type (so every level is exercised)."""
    Qg, K, V, cls = _random_head(rng, n, d, G, scale=0.5)
    u = rng.standard_normal(d)
    u *= math.sqrt(d) / np.linalg.norm(u)
    if kind == "special":
        Qg = Qg + u
        K[cls == ref.TOKEN_SPECIAL] += 3 * u
    elif kind == "punct":
        Qg = Qg + u
        K[cls == ref.TOKEN_PUNCT] += 3 * u
    elif kind == "heavy":
        Qg = Qg + u
        K[rng.choice(n, size=max(1, n // 4), replace=False)] += 3 * u
    return Qg, K, V, cls


# ---------------------------------------------------------------- closed form (uniform attention)

def _check_uniform(case):
    n, k_f, w_l = case["n"], case["k_f"], case["w_l"]
    rng = np.random.default_rng(n)
    Qg = np.zeros((1, n, 8))
    K = rng.standard_normal((n, 8))
    cls = np.zeros(n, dtype=np.uint8)
    cls[0] = ref.TOKEN_SPECIAL
    prof = ref.profile_head(Qg, K, cls, _ratio_for(w_l, n), _ratio_for(k_f, n), 0.5)
    assert (prof.k_f, prof.w_l) == (k_f, w_l)
    np.testing.assert_allclose(prof.lse[0], case["lse"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(prof.cum, case["cum"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(prof.band, case["band"], rtol=0, atol=1e-12)
    assert np.array_equal(np.flatnonzero(prof.F), np.arange(k_f))
    np.testing.assert_allclose(prof.R, case["R"], rtol=0, atol=1e-12)


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_uniform_closed_form(idx):
    case = json.load(open(GOLDEN))["cases"][idx]
    _check_uniform(case)


def test_uniform_policy_thresholds():
    case = json.load(open(GOLDEN))["cases"][0]
    n, k_f, w_l = case["n"], case["k_f"], case["w_l"]
    R = case["R"]
    Qg = np.zeros((1, n, 8))
    K = np.random.default_rng(0).standard_normal((n, 8))
    cls = np.zeros(n, dtype=np.uint8)
    cls[0] = ref.TOKEN_SPECIAL
    for T, want in [(R[0] - 1e-6, 0), (R[0] + 1e-6, 2), (R[2] + 1e-6, 3), (R[3] + 1e-6, 4), (1.0, 4)]:
        prof = ref.profile_head(Qg, K, cls, _ratio_for(w_l, n), _ratio_for(k_f, n), T)
        assert prof.policy == want, (T, prof.R)


def test_budgets_floor():
    assert ref.budgets(2048, 0.3, 0.3) == (614, 614)
    assert ref.budgets(32768, 0.05, 0.1) == (3276, 1638)
    assert ref.budgets(256, 0.3, 0.3) == (76, 76)
    assert ref.budgets(10, 0.3, 0.7) == (7, 3)
    assert ref.budgets(1, 0.3, 0.3) == (0, 0)


# ---------------------------------------------------------------- brute force + literal half-L1 constraint

def _brute_cases():
    rng = np.random.default_rng(1234)
    cases = []
    for t in range(120):
        n = int(rng.integers(1, 13))
        d = int(rng.choice([4, 8]))
        G = int(rng.choice([1, 2]))
        kind = ["none", "special", "punct", "heavy"][t % 4]
        Qg, K, V, cls = _planted_head(rng, n, d, G, kind)
        k_f = int(rng.integers(0, n + 1))
        w_l = int(rng.integers(0, n + 2))
        T = float(rng.choice([0.5, 0.8, 0.9, 0.95, 0.99, 1.0]))
        cases.append((Qg, K, cls, k_f, w_l, T))
    return cases


def test_brute_force_matches_oracle():
    levels_seen = set()
    for Qg, K, cls, k_f, w_l, T in _brute_cases():
        n = K.shape[0]
        bf = brute_force_head(Qg, K, cls, k_f, w_l, T)
        r_l, r_f = _ratio_for(w_l, n), _ratio_for(k_f, n)
        prof = ref.profile_head(Qg, K, cls, r_l, r_f, T)
        assert (prof.k_f, prof.w_l) == (k_f, w_l)
        np.testing.assert_allclose(prof.cum, bf["cum"], rtol=0, atol=1e-12)
        # the literal constraint: 1 - mean half-L1 distance == retained mass
        np.testing.assert_allclose(prof.R, bf["recovery"], rtol=0, atol=1e-12)
        # the worst row: the least kept share equals one minus the largest per-row half-L1 distance
        if not prof.topk_tie:
            np.testing.assert_allclose(ref.row_min_share(prof.bins), bf["worst_row_recovery"], rtol=0, atol=1e-12)
        if not prof.topk_tie:
            assert np.array_equal(prof.F, bf["F"])
        if not prof.near_T and not prof.topk_tie:
            assert prof.policy == bf["policy"], (prof.R, bf["recovery"], T)
            assert np.array_equal(prof.kept, bf["kept"])
            assert len(prof.kept) == bf["cost"][prof.policy]
        levels_seen.add(prof.policy)
    assert levels_seen == {0, 1, 2, 3, 4}


def test_frequent_ties_go_to_lower_index():
    cum = np.array([1.0, 3.0, 2.0, 3.0, 2.0, 2.0, 0.5])
    F = ref.frequent_set(cum, 4)
    assert np.flatnonzero(F).tolist() == [1, 2, 3, 4]
    # same answer as a stable argsort of -cum
    order = np.argsort(-cum, kind="stable")
    assert sorted(order[:4].tolist()) == [1, 2, 3, 4]


def test_frequent_matches_stable_argsort_random():
    rng = np.random.default_rng(5)
    for _ in range(50):
        n = int(rng.integers(1, 300))
        cum = np.round(rng.random(n) * 20) / 4.0          # many exact ties
        k = int(rng.integers(0, n + 1))
        F = ref.frequent_set(cum, k)
        order = np.argsort(-cum, kind="stable")[:k]
        assert np.array_equal(np.flatnonzero(F), np.sort(order))


# ---------------------------------------------------------------- column identity (what the GPU computes)

def _recovery_from_columns(cum, band, F, cls, G, n):
    """R_k from per-key column sums only: the identity the profiling kernels use."""
    s = cls == ref.TOKEN_SPECIAL
    p = cls == ref.TOKEN_PUNCT
    f = F & ~s & ~p
    rest = ~(s | p | F)
    m0 = cum[s].sum()
    m1 = m0 + cum[p].sum()
    m2 = m1 + cum[f].sum()
    m3 = m2 + band[rest].sum()
    return np.array([m0, m1, m2, m3, G * n]) / (G * n)


def test_column_identity():
    rng = np.random.default_rng(7)
    for t in range(30):
        n = int(rng.integers(1, 200))
        G = int(rng.choice([1, 2, 4]))
        Qg, K, V, cls = _planted_head(rng, n, 16, G, ["none", "special", "punct", "heavy"][t % 4])
        r_l, r_f = float(rng.random()), float(rng.random())
        prof = ref.profile_head(Qg, K, cls, r_l, r_f, 0.9)
        R = _recovery_from_columns(prof.cum, prof.band, prof.F, cls, G, n)
        np.testing.assert_allclose(R, prof.R, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- invariants

def test_invariants():
    rng = np.random.default_rng(11)
    for t in range(25):
        n = int(rng.integers(1, 150))
        G = int(rng.choice([1, 2, 4]))
        Qg, K, V, cls = _planted_head(rng, n, 16, G, ["none", "special", "punct", "heavy"][t % 4])
        prof = ref.profile_head(Qg, K, cls, 0.3, 0.3, 0.95)
        assert abs(prof.cum.sum() - G * n) < 1e-9
        last = sum(ref.causal_attention_rows(Qg[g, n - 1:n], K, n - 1)[0, n - 1] for g in range(G))
        assert abs(prof.cum[n - 1] - last) < 1e-12
        assert prof.cum[0] >= G - 1e-12
        assert np.all(np.diff(prof.R) >= -1e-15)
        assert prof.R[4] == 1.0
        np.testing.assert_allclose(prof.bins.sum(axis=2), 1.0, atol=1e-12)
        kept_sets = [set(ref.kept_positions(cls, prof.F, prof.w_l, k)) for k in range(5)]
        for a, b in zip(kept_sets, kept_sets[1:]):
            assert a <= b
        assert kept_sets[4] == set(range(n))


def test_band_special_cases():
    rng = np.random.default_rng(3)
    Qg, K, V, cls = _random_head(rng, 40, 8, 2)
    full = ref.column_scores(Qg, K, 40)
    np.testing.assert_allclose(full["band"], full["cum"], atol=1e-12)
    diag = ref.column_scores(Qg, K, 1)
    want = sum(np.diag(ref.causal_attention_rows(Qg[g], K, 0)) for g in range(2))
    np.testing.assert_allclose(diag["band"], want, atol=1e-12)
    zero = ref.column_scores(Qg, K, 0)
    assert np.all(zero["band"] == 0)


# ---------------------------------------------------------------- decode-time tracking

def _tracking_case(rng, n, d, G, steps, policy, zero_q=False):
    Qg, K, V, cls = _random_head(rng, n, d, G)
    cls = cls.copy()
    cls[0] = ref.TOKEN_SPECIAL
    cls[rng.random(n) < 0.1] = ref.TOKEN_PUNCT
    w_l, k_f = 5, 6
    prof = ref.profile_head(Qg, K, cls, 0.1, 0.1, 0.9)
    F = ref.frequent_set(prof.cum, k_f)
    q = np.zeros((steps, G, d)) if zero_q else rng.standard_normal((steps, G, d))
    kn = rng.standard_normal((steps, d))
    vn = rng.standard_normal((steps, d))
    nc = np.where(rng.random(steps) < 0.3, ref.TOKEN_PUNCT, ref.TOKEN_NORMAL).astype(np.uint8)
    _, caches = ref.decode_incremental(K, V, cls, F, w_l, policy, q, kn, vn, nc)
    K_all = np.concatenate([K, kn])
    cls_all = np.concatenate([cls, nc])
    return dict(Qg=Qg, K_all=K_all, cls_all=cls_all, F=F, w_l=w_l, n=n, caches=caches, q=q, cum0=prof.cum, G=G)


def test_tracking_uniform_attention_closed_form():
    rng = np.random.default_rng(41)
    n, G, steps = 40, 2, 9
    c = _tracking_case(rng, n, 8, G, steps, ref.LEVEL_FULL, zero_q=True)
    bins, score = ref.decode_tracking(c["K_all"], c["cls_all"], c["F"], c["w_l"], n, c["caches"], c["q"], c["cum0"])
    cls_all, F, w_l = c["cls_all"], c["F"], c["w_l"]
    for t in range(steps):
        p = n + t
        js = np.arange(p + 1)
        sp = cls_all[js] == ref.TOKEN_SPECIAL
        pu = cls_all[js] == ref.TOKEN_PUNCT
        fr = np.zeros(p + 1, dtype=bool)
        fr[:n] = F
        fr &= ~sp & ~pu
        lo = (p - js < w_l) & ~sp & ~pu & ~fr
        counts = [sp.sum(), pu.sum(), fr.sum(), lo.sum()]
        counts.append(p + 1 - sum(counts))
        np.testing.assert_allclose(bins[t], np.array(counts) / (p + 1), atol=1e-13)
    harm = [G * sum(1.0 / (n + u + 1) for u in range(t0, steps)) for t0 in range(steps)]
    for j, v in score.items():
        want = c["cum0"][j] + harm[0] if j < n else harm[j - n]
        assert abs(v - want) < 1e-12, (j, v, want)


def test_tracking_full_cache_equals_row_bins_and_conserves_mass():
    rng = np.random.default_rng(42)
    n, d, G, steps = 30, 8, 3, 7
    c = _tracking_case(rng, n, d, G, steps, ref.LEVEL_FULL)
    bins, score = ref.decode_tracking(c["K_all"], c["cls_all"], c["F"], c["w_l"], n, c["caches"], c["q"], c["cum0"])
    for t in range(steps):
        p = n + t
        Qx = rng.standard_normal((G, p + 1, d))
        Qx[:, p] = c["q"][t]
        rb = ref.row_bins(Qx, c["K_all"][: p + 1], c["cls_all"][: p + 1], c["F"], c["w_l"])
        np.testing.assert_allclose(bins[t], rb[:, p].mean(axis=0), atol=1e-13)
        assert abs(bins[t].sum() - 1.0) < 1e-13
    assert sorted(score) == list(range(n + steps))
    assert abs(sum(score.values()) - (c["cum0"].sum() + G * steps)) < 1e-10


@pytest.mark.parametrize("policy", [0, 1, 2, 3])
def test_tracking_compressed_cache_has_no_mass_above_its_policy(policy):
    rng = np.random.default_rng(43 + policy)
    n, G, steps = 35, 2, 8
    c = _tracking_case(rng, n, 8, G, steps, policy)
    bins, score = ref.decode_tracking(c["K_all"], c["cls_all"], c["F"], c["w_l"], n, c["caches"], c["q"], c["cum0"])
    for t in range(steps):
        if len(c["caches"][t]):
            assert abs(bins[t].sum() - 1.0) < 1e-13
            assert np.all(bins[t, policy + 1:] == 0.0)
    assert sorted(score) == sorted(int(j) for j in c["caches"][-1])


def test_dynamic_frequent_without_replacement_is_the_static_policy():
    rng = np.random.default_rng(51)
    for w_l in (0, 1, 2, 5):
        n, d, G, steps = 40, 8, 2, 12
        Qg, K, V, cls = _random_head(rng, n, d, G)
        prof = ref.profile_head(Qg, K, cls, 0.1, 0.2, 0.9)
        F = prof.F
        q = rng.standard_normal((steps, G, d))
        kn, vn = rng.standard_normal((steps, d)), rng.standard_normal((steps, d))
        nc = np.where(rng.random(steps) < 0.3, ref.TOKEN_PUNCT, ref.TOKEN_NORMAL).astype(np.uint8)
        outs, caches = ref.decode_incremental(K, V, cls, F, w_l, ref.LEVEL_LOCAL, q, kn, vn, nc)
        dyn = ref.DynamicFrequentHead(K, V, cls, F, w_l, prof.cum)
        for t in range(steps):
            o, kept, info = dyn.step(q[t], kn[t], vn[t], int(nc[t]), force=False)
            np.testing.assert_allclose(o, outs[t], atol=1e-12)
            assert np.array_equal(kept, caches[t]), (w_l, t)


def test_dynamic_frequent_replaces_the_weakest_key():
    # keys: 0 special; 3, 5, 7 frequent; the window (w_l = 4) holds the last three positions.
    # Key 17 carries a large prompt score, so when it leaves the window it replaces the weakest
    # frequent key: 5 and 7 tie at the lowest score, the larger position (7) goes.
    n, d, w_l = 20, 4, 4
    rng = np.random.default_rng(52)
    K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    cls = np.zeros(n, dtype=np.uint8)
    cls[0] = ref.TOKEN_SPECIAL
    F = np.zeros(n, dtype=bool)
    F[[3, 5, 7]] = True
    cum0 = np.full(n, 0.5)
    cum0[3], cum0[5], cum0[7], cum0[17] = 2.0, 0.25, 0.25, 9.0
    dyn = ref.DynamicFrequentHead(K, V, cls, F, w_l, cum0)
    assert sorted(dyn.kv) == [0, 3, 5, 7, 17, 18, 19] and dyn.freq == {3, 5, 7}
    q = np.zeros((1, d))                               # uniform attention: each cached key gains 1/|cache|
    o, kept, info = dyn.step(q, rng.standard_normal(d), rng.standard_normal(d), ref.TOKEN_NORMAL)   # p = 20
    assert (info["candidate"], info["weakest"], info["replaced"]) == (17, 7, True)
    assert abs(info["margin"] - (9.0 - 0.25)) < 1e-12                 # scores through the previous step
    assert kept.tolist() == [0, 3, 5, 17, 18, 19, 20] and dyn.freq == {3, 5, 17}
    # step p = 21: key 18 leaves with score 0.5 + 1/7 (+ the step-20 share), below the weakest (5: 0.25 + 1/7)? no:
    # 18 has 0.5 + 1/7 > 0.25 + 1/7, so it replaces 5
    o, kept, info = dyn.step(q, rng.standard_normal(d), rng.standard_normal(d), ref.TOKEN_PUNCT)     # p = 21
    assert (info["candidate"], info["weakest"], info["replaced"]) == (18, 5, True)
    assert kept.tolist() == [0, 3, 17, 18, 19, 20, 21] and dyn.freq == {3, 17, 18}
    assert len(dyn.freq) == 3


def test_dynamic_frequent_keeps_its_budget_and_evicts_only_weaker_keys():
    rng = np.random.default_rng(53)
    n, d, G, steps, w_l = 60, 8, 2, 30, 6
    Qg, K, V, cls = _random_head(rng, n, d, G)
    prof = ref.profile_head(Qg, K, cls, 0.1, 0.2, 0.9)
    # prompt scores scaled down so that keys leaving the window can beat frequent keys
    dyn = ref.DynamicFrequentHead(K, V, cls, prof.F, w_l, prof.cum * 0.02)
    budget = len(dyn.freq)
    replaced = 0
    for t in range(steps):
        before = {j: dyn.score[j] for j in dyn.freq}
        q = rng.standard_normal((G, d)) * 2
        o, kept, info = dyn.step(q, rng.standard_normal(d), rng.standard_normal(d), ref.TOKEN_NORMAL)
        assert len(dyn.freq) == budget
        if info["replaced"]:
            replaced += 1
            w = info["weakest"]
            assert all((s, -j) >= (before[w], -w) for j, s in before.items())   # the weakest went
            assert info["margin"] > 0 and info["candidate"] in dyn.freq and w not in dyn.kv
        elif info["candidate"] is not None:
            assert info["candidate"] not in dyn.kv
    assert replaced > 0


# ---------------------------------------------------------------- multi-prompt head map

def test_head_map_of_identical_prompts_is_the_single_prompt_policy():
    rng = np.random.default_rng(31)
    for _ in range(20):
        H = 6
        R1 = np.sort(rng.random((H, 5)), axis=1)
        R1[:, 4] = 1.0
        T = float(rng.choice([0.5, 0.9, 0.95]))
        pol1 = np.array([ref.select_policy(R1[h], T) for h in range(H)])
        P = int(rng.integers(1, 9))
        m = ref.head_type_map(np.broadcast_to(R1, (P, H, 5)), np.broadcast_to(pol1, (P, H)), T)
        assert np.array_equal(m["policy"], pol1)
        np.testing.assert_allclose(m["mean"], R1, rtol=0, atol=1e-15)
        assert np.array_equal(m["count"][np.arange(H), pol1], np.full(H, P))
        assert np.all(m["count"].sum(axis=1) == P)


def test_head_map_decides_on_the_mean_not_the_majority():
    # two prompts: R_0 = 0.96 and 0.90 at T = 0.92 -> mean 0.93 keeps the special-only
    # policy although one prompt alone needed more; three prompts with R_0 = 0.95, 0.95, 0.80
    # at T = 0.92 -> mean 0.90 falls to the next entry although most prompts chose policy 0
    R = np.array([[[0.96, 0.97, 0.98, 0.99, 1.0]], [[0.90, 0.97, 0.98, 0.99, 1.0]]])
    m = ref.head_type_map(R, [[0], [1]], 0.92)
    assert m["policy"].tolist() == [0] and m["count"].tolist() == [[1, 1, 0, 0, 0]]
    np.testing.assert_allclose(m["mean"][0, 0], 0.93, atol=1e-15)
    R = np.array([[[0.95, 0.96, 0.97, 0.98, 1.0]], [[0.95, 0.96, 0.97, 0.98, 1.0]], [[0.80, 0.90, 0.95, 0.97, 1.0]]])
    m = ref.head_type_map(R, [[0], [0], [2]], 0.92)
    assert m["policy"].tolist() == [1] and m["count"].tolist() == [[2, 0, 1, 0, 0]]


def test_head_map_recovers_planted_types_over_prompts():
    # eight independent tiny prompts of one planted layer: the map lands on the planted policy
    spec = syn.CONFIGS[0]
    li = syn.make_layer(spec, batch=[0], seed=101)
    types = li.types
    Rs, pols = [], []
    for seed in range(101, 109):
        li = syn.make_layer(spec, batch=[0], seed=seed)
        assert li.types == types
        prof = ref.profile_layer(li.Q, li.K, li.token_class, spec.r_l, spec.r_f, spec.T[0])[0]
        Rs.append([p.R for p in prof])
        pols.append([p.policy for p in prof])
    m = ref.head_type_map(np.array(Rs), np.array(pols), spec.T[0])
    want = {"special": 0, "punct": 1, "local": 3, "none": 4}
    assert [int(x) for x in m["policy"]] == [want[t] for t in types]


# ---------------------------------------------------------------- library routines

def test_attention_rows_match_torch_sdpa():
    rng = np.random.default_rng(21)
    for n, d in [(1, 8), (7, 16), (130, 64)]:
        q = rng.standard_normal((n, d))
        K = rng.standard_normal((n, d))
        A = ref.causal_attention_rows(q, K, 0)
        out = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None, None], torch.from_numpy(K)[None, None],
            torch.eye(n, dtype=torch.float64)[None, None], is_causal=True)
        np.testing.assert_allclose(A, out[0, 0].numpy(), atol=1e-13)


def test_attention_output_matches_torch_sdpa():
    rng = np.random.default_rng(25)
    for G, n, d, dv in [(1, 1, 8, 8), (2, 9, 16, 5), (3, 600, 32, 32)]:
        Qg = rng.standard_normal((G, n, d)) * 2
        K = rng.standard_normal((n, d)) * 2
        V = rng.standard_normal((n, dv))
        O = ref.attention_output(Qg, K, V)
        want = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Qg)[None], torch.from_numpy(K)[None, None].expand(1, G, -1, -1),
            torch.from_numpy(V)[None, None].expand(1, G, -1, -1), is_causal=True)[0]
        np.testing.assert_allclose(O, want.numpy(), atol=1e-12)


def test_attention_output_closed_forms():
    rng = np.random.default_rng(26)
    G, n, d = 2, 700, 16
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, 4))
    # zero queries attend uniformly: row i is the mean of V[0..i]
    O = ref.attention_output(np.zeros((G, n, d)), K, V)
    prefix_mean = np.cumsum(V, axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(O[0], prefix_mean, atol=1e-12)
    np.testing.assert_allclose(O[1], prefix_mean, atol=1e-12)
    # row 0 sees only key 0; a constant value column passes through unchanged
    Qg = rng.standard_normal((G, n, d)) * 3
    V[:, 2] = 1.75
    O = ref.attention_output(Qg, K, V)
    np.testing.assert_allclose(O[:, 0], np.broadcast_to(V[0], (G, 4)), atol=1e-12)
    np.testing.assert_allclose(O[:, :, 2], 1.75, atol=1e-12)
    # a query far along k_j picks out v_j when k_j is the unique maximiser
    K2 = np.eye(n, d) if n <= d else np.vstack([np.eye(d), np.zeros((n - d, d))])
    q = np.zeros((1, n, d))
    q[0, d - 1:, d - 1] = 200.0
    O2 = ref.attention_output(q, K2, V)
    np.testing.assert_allclose(O2[0, n - 1], V[d - 1], atol=1e-12)


def test_lse_matches_scipy():
    from scipy.special import logsumexp
    rng = np.random.default_rng(22)
    n, d = 50, 16
    Qg = rng.standard_normal((1, n, d)) * 3
    K = rng.standard_normal((n, d)) * 3
    lse = ref.column_scores(Qg, K, 5)["lse"][0]
    want = [logsumexp((Qg[0, i] @ K[: i + 1].T) / math.sqrt(d)) for i in range(n)]
    np.testing.assert_allclose(lse, want, atol=1e-12)


def test_decode_matches_torch_sdpa_with_level_mask():
    rng = np.random.default_rng(23)
    n, d, G, steps = 60, 16, 2, 12
    for kind, policy in [("special", 0), ("punct", 1), ("heavy", 2), ("none", 3), ("none", 4)]:
        Qg, K, V, cls = _planted_head(rng, n, d, G, kind)
        prof = ref.profile_head(Qg, K, cls, 0.2, 0.2, 0.9)
        q = rng.standard_normal((steps, G, d))
        kn = rng.standard_normal((steps, d))
        vn = rng.standard_normal((steps, d))
        nc = np.where(rng.random(steps) < 0.3, ref.TOKEN_PUNCT, ref.TOKEN_NORMAL).astype(np.uint8)
        out, _ = ref.decode_incremental(K, V, cls, prof.F, prof.w_l, policy, q, kn, vn, nc)
        K_all = np.concatenate([K, kn])
        V_all = np.concatenate([V, vn])
        cls_all = np.concatenate([cls, nc])
        lev = ref.key_levels(cls_all, prof.F, n + np.arange(steps), prof.w_l)
        for t in range(steps):
            mask = torch.from_numpy(lev[t] <= policy)
            if not mask.any():
                assert np.all(out[t] == 0)
                continue
            o = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[t])[None, :, None, :],
                torch.from_numpy(K_all)[None, None].expand(1, G, -1, -1),
                torch.from_numpy(V_all)[None, None].expand(1, G, -1, -1),
                attn_mask=mask[None, None, None, :])
            np.testing.assert_allclose(out[t], o[0, :, 0].numpy(), atol=1e-12)


def test_full_policy_decode_is_causal_attention():
    rng = np.random.default_rng(24)
    n, d, steps = 20, 8, 6
    Qg, K, V, cls = _random_head(rng, n, d, 1)
    F = np.zeros(n, dtype=bool)
    q = rng.standard_normal((steps, 1, d))
    kn = rng.standard_normal((steps, d))
    vn = rng.standard_normal((steps, d))
    nc = np.zeros(steps, dtype=np.uint8)
    out, caches = ref.decode_incremental(K, V, cls, F, 3, 4, q, kn, vn, nc)
    K_all, V_all = np.concatenate([K, kn]), np.concatenate([V, vn])
    for t in range(steps):
        p = n + t
        s = K_all[: p + 1] @ q[t, 0] / math.sqrt(d)
        a = np.exp(s - s.max())
        a /= a.sum()
        np.testing.assert_allclose(out[t, 0], a @ V_all[: p + 1], atol=1e-12)
        assert caches[t].tolist() == list(range(p + 1))


# ---------------------------------------------------------------- decode routes and compaction

@pytest.mark.parametrize("w_l", [0, 1, 2, 5, 30])
def test_incremental_equals_one_shot(w_l):
    rng = np.random.default_rng(31 + w_l)
    n, d, G, steps = 40, 8, 2, 25
    Qg, K, V, cls = _random_head(rng, n, d, G)
    F = np.zeros(n, dtype=bool)
    F[rng.choice(n, 6, replace=False)] = True
    q = rng.standard_normal((steps, G, d))
    kn = rng.standard_normal((steps, d))
    vn = rng.standard_normal((steps, d))
    nc = rng.choice([0, 0, 0, 2, 1], size=steps).astype(np.uint8)
    for policy in range(5):
        o1, c1 = ref.decode_incremental(K, V, cls, F, w_l, policy, q, kn, vn, nc)
        o2, c2 = ref.decode_masked(K, V, cls, F, w_l, policy, q, kn, vn, nc)
        np.testing.assert_allclose(o1, o2, atol=1e-12)
        for a, b in zip(c1, c2):
            assert np.array_equal(a, b)


def test_compaction_bytes_exact():
    spec = syn.custom_spec(syn.CONFIGS[1], seq_len=128, n_q_heads=4, n_kv_heads=4)
    li = syn.make_layer(spec, 0)
    for h in range(4):
        prof = ref.profile_head(li.Q[0, h:h + 1], li.K[0, h], li.token_class[0], 0.3, 0.3, 0.95)
        Kc, Vc = ref.compact_head(li.K[0, h], li.V[0, h], prof.kept)
        assert Kc.dtype == np.float32
        assert np.array_equal(Kc.view(np.uint32), li.K[0, h][prof.kept].view(np.uint32))
        assert np.array_equal(Vc.view(np.uint32), li.V[0, h][prof.kept].view(np.uint32))
        assert np.all(np.diff(prof.kept) > 0)


def test_empty_kept_set_decodes_to_zero():
    n, d = 6, 4
    rng = np.random.default_rng(2)
    K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    cls = np.zeros(n, dtype=np.uint8)                 # no special token at all
    F = np.zeros(n, dtype=bool)
    assert len(ref.kept_positions(cls, F, 0, 0)) == 0
    out, caches = ref.decode_incremental(K, V, cls, F, 0, 0, rng.standard_normal((2, 1, d)),
                                         rng.standard_normal((2, d)), rng.standard_normal((2, d)),
                                         np.zeros(2, dtype=np.uint8))
    assert np.all(out == 0) and all(len(c) == 0 for c in caches)


# ---------------------------------------------------------------- planted heads land in their policy

def _landing(spec, seed):
    li = syn.make_layer(spec, 0, seed=seed)
    G = spec.group
    res = []
    for h, kind in enumerate(li.types):
        prof = ref.profile_head(li.Q[0, h * G:(h + 1) * G], li.K[0, h], li.token_class[0],
                                spec.r_l, spec.r_f, spec.T[0])
        margin = float(np.min(np.abs(prof.R[:4] - spec.T[0])))
        res.append((kind, prof.policy, margin, prof.R))
    return res


WANT = {"special": 0, "punct": 1, "heavy": 2, "local": 3, "none": 4}


def test_planted_config0_canonical_seed():
    spec = syn.CONFIGS[0]
    cls = syn.token_classes(spec, 0)
    assert int(np.flatnonzero(cls == syn.TOKEN_PUNCT)[0]) <= 12
    for kind, policy, margin, R in _landing(spec, None):
        assert margin >= 0.01, (kind, R)
        assert policy == WANT[kind], (kind, R)


@pytest.mark.slow
def test_planted_config0_many_seeds():
    spec = syn.custom_spec(syn.CONFIGS[0], fixed_types=("special", "punct", "heavy", "local", "none"),
                           n_q_heads=5, n_kv_heads=5)
    landed = total = 0
    for seed in range(1, 9):
        for kind, policy, margin, R in _landing(spec, seed):
            if margin >= 0.01:
                total += 1
                if kind == "punct" and policy == 2:
                    continue      # punct head whose first punct token came late spreads mass
                assert policy == WANT[kind], (seed, kind, R)
                landed += 1
    assert landed >= 0.85 * total


# ---------------------------------------------------------------- shapes and indexing

def test_batch_gqa_and_permutation():
    spec = syn.custom_spec(syn.CONFIGS[4], seq_len=96, batch=2, n_q_heads=8, n_kv_heads=2,
                           fixed_types=("special", "local"))
    li = syn.make_layer(spec, 0)
    full = ref.profile_layer(li.Q, li.K, li.token_class, spec.r_l, spec.r_f, 0.95)
    for b in range(2):
        one = ref.profile_layer(li.Q[b:b + 1], li.K[b:b + 1], li.token_class[b:b + 1], spec.r_l, spec.r_f, 0.95)
        for h in range(2):
            np.testing.assert_array_equal(one[0][h].cum, full[b][h].cum)
    # the sub-batch generator equals the slice of the full batch
    li1 = syn.make_layer(spec, 0, batch=[1])
    assert np.array_equal(li1.Q[0], li.Q[1]) and np.array_equal(li1.K[0], li.K[1])
    # GQA with G = 1 is plain multi-head profiling of each query head
    g1 = ref.profile_layer(li.Q[:, :4], np.repeat(li.K[:, :1], 4, axis=1), li.token_class,
                           spec.r_l, spec.r_f, 0.95)
    cum_sum = sum(g1[0][h].cum for h in range(4))
    np.testing.assert_allclose(cum_sum, full[0][0].cum, atol=1e-10)
    # permuting KV heads permutes results
    Qp = li.Q.reshape(2, 2, 4, 96, -1)[:, ::-1].reshape(2, 8, 96, -1)
    perm = ref.profile_layer(Qp, li.K[:, ::-1], li.token_class, spec.r_l, spec.r_f, 0.95)
    for b in range(2):
        for h in range(2):
            np.testing.assert_allclose(perm[b][h].cum, full[b][1 - h].cum, atol=1e-12)
            assert perm[b][h].policy == full[b][1 - h].policy


# ---------------------------------------------------------------- planted mistakes are caught

def _golden_case(i=0):
    return json.load(open(GOLDEN))["cases"][i]


def test_mistake_strict_causal_mask_is_caught(monkeypatch):
    orig = ref.causal_attention_rows

    def strict(q, K, row0):                       # plants: drops the diagonal
        q = np.asarray(q, np.float64)
        K = np.asarray(K, np.float64)
        m, d = q.shape
        S = (q @ K.T) / math.sqrt(d)
        i = row0 + np.arange(m)[:, None]
        j = np.arange(K.shape[0])[None, :]
        S = np.where((j < i) | ((i == 0) & (j == 0)), S, -np.inf)
        E = np.exp(S - S.max(axis=1, keepdims=True))
        return E / E.sum(axis=1, keepdims=True)

    monkeypatch.setattr(ref, "causal_attention_rows", strict)
    with pytest.raises(AssertionError):
        _check_uniform(_golden_case())
    monkeypatch.setattr(ref, "causal_attention_rows", orig)
    _check_uniform(_golden_case())


def test_mistake_local_off_by_one_is_caught(monkeypatch):
    orig = ref.key_levels

    def loose(cls, F, rows, w_l):                 # plants: i - j <= w_l
        return orig(cls, F, rows, w_l + 1)

    monkeypatch.setattr(ref, "key_levels", loose)
    with pytest.raises(AssertionError):
        _check_uniform(_golden_case())


def test_mistake_ties_to_higher_index_is_caught(monkeypatch):
    def high(cum, k_f):                           # plants: ties broken toward the higher index
        n = len(cum)
        order = sorted(range(n), key=lambda j: (-float(cum[j]), -j))
        F = np.zeros(n, dtype=bool)
        F[order[:k_f]] = True
        return F

    monkeypatch.setattr(ref, "frequent_set", high)
    with pytest.raises(AssertionError):
        test_frequent_ties_go_to_lower_index()


def test_mistake_missing_scale_is_caught(monkeypatch):
    def unscaled(q, K, row0):                     # plants: no 1/sqrt(d)
        q = np.asarray(q, np.float64)
        K = np.asarray(K, np.float64)
        S = q @ K.T
        i = row0 + np.arange(q.shape[0])[:, None]
        j = np.arange(K.shape[0])[None, :]
        S = np.where(j <= i, S, -np.inf)
        E = np.exp(S - S.max(axis=1, keepdims=True))
        return E / E.sum(axis=1, keepdims=True)

    monkeypatch.setattr(ref, "causal_attention_rows", unscaled)
    with pytest.raises(AssertionError):
        test_attention_rows_match_torch_sdpa()


def test_mistake_wrong_precedence_is_caught(monkeypatch):
    orig = ref.key_levels

    def swapped(cls, F, rows, w_l):               # plants: frequent checked before punct
        lev = orig(cls, F, rows, w_l)
        Fx = np.zeros(len(cls), dtype=bool)
        Fx[: len(F)] = F[: len(cls)]
        both = Fx[None, :] & (np.asarray(cls) == ref.TOKEN_PUNCT)[None, :] & (lev < 5)
        return np.where(both, ref.LEVEL_FREQUENT, lev)

    monkeypatch.setattr(ref, "key_levels", swapped)
    with pytest.raises(AssertionError):
        test_brute_force_matches_oracle()


@pytest.mark.parametrize("n,k_f,w_l", [(64, 19, 19), (50, 5, 12), (33, 0, 7), (40, 10, 0), (17, 16, 16)])
def test_row_min_share_uniform_closed_form(n, k_f, w_l):
    """Zero queries: row i spreads 1/(i+1) over keys 0..i, so cum_j = H_n - H_j is strictly
    decreasing and F = {0 .. k_f-1}.  With the special set {0} and no punctuation, row i keeps
    1/(i+1) under entries 0 and 1, |{0} u F u window| / (i+1) under entries 2 and 3; the kept
    counts stop growing once the row passes them, so the least share of each entry is at the
    last row: 1/n, 1/n, max(k_f, 1)/n, |{0} u F u (n - w_l, n - 1]|/n, and 1."""
    d = 8
    Qg = np.zeros((1, n, d))
    K = np.random.default_rng(n).standard_normal((n, d))
    cls = np.zeros(n, dtype=np.uint8)
    cls[0] = ref.TOKEN_SPECIAL
    F = np.zeros(n, dtype=bool)
    F[:k_f] = True
    bins = ref.row_bins(Qg, K, cls, F, w_l)
    got = ref.row_min_share(bins)
    # the kept count of the last row under entry 3: the union of {0}, F and the window (n - w_l, n - 1]
    kept3 = len({0} | set(range(k_f)) | set(range(max(0, n - w_l), n)))
    want = np.array([1.0 / n, 1.0 / n, max(k_f, 1) / n, kept3 / n, 1.0])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
