"""Pins of the oracle's two flags, the cases where rounding may decide.

* top-k tie: the frequent set (the k_f keys with the largest cumulative
  attention, ties to the lower index -- hyper.ai summary of "Model Tells You
  What to Discard", Method, policy paragraph) is fragile when the weakest chosen
  score s_(k) and the strongest rejected one s_(k+1) lie within a relative
  window tau of each other, or when s_(k) has underflowed below 2^-100;
* near-T: the policy (the first shortlist entry whose recovery reaches T, Method,
  constraint equation) is fragile when some R_k, k <= 3, lies within 1e-4 of T.

Each pin is a hand-built input whose flag follows from the definitions by
inspection.  Planted mistakes (an off-by-one in the sorted index, a window ten
times too wide, the comparison on one side only, R_4 included, R_3 left out) each
break at least one pin.
"""
import numpy as np
import pytest

from oracle import fastgen_ref as ref

TAU = 3e-5


def _tie_pins():
    """(cum, k_f, tau, flag) tuples."""
    rng = np.random.default_rng(11)
    pins = []

    def add(vals, k_f, flag, tau=TAU):
        vals = np.asarray(vals, dtype=np.float64)
        pins.append((vals, k_f, tau, flag))
        pins.append((vals[rng.permutation(len(vals))], k_f, tau, flag))   # positions do not matter

    # the relative gap at the boundary just inside and just outside the window
    add([5.0, 4.0, 3.0, 3.0 * (1.0 - 2.9e-5), 1.0], 3, True)
    add([5.0, 4.0, 3.0, 3.0 * (1.0 - 3.1e-5), 1.0], 3, False)
    add([5.0, 4.0, 3.0, 3.0 * (1.0 - 2.9e-6), 1.0], 3, True, tau=3e-6)
    add([5.0, 4.0, 3.0, 3.0 * (1.0 - 3.1e-6), 1.0], 3, False, tau=3e-6)
    # exact ties away from the boundary do not flag; at the boundary they do
    add([5.0, 4.0, 3.0, 3.0, 1.0], 2, False)
    add([5.0, 4.0, 3.0, 3.0, 1.0], 3, True)
    add([5.0, 4.0, 4.0, 3.0, 1.0], 3, False)
    # no boundary: F is every key or none
    add([2.0, 2.0, 2.0, 2.0], 0, False)
    add([2.0, 2.0, 2.0, 2.0], 4, False)
    add([2.0, 2.0, 2.0, 2.0], 5, False)
    # k_f = 1 and k_f = n - 1
    add([2.0, 2.0, 1.0], 1, True)
    add([2.0, 1.0, 1.0], 1, False)
    add([3.0, 2.0, 1.0, 1.0], 3, True)
    add([3.0, 2.0, 1.0, 0.5], 3, False)
    # the underflow floor: s_(k) below 2^-100 flags whatever the relative gap
    add([1.0, 2.0 ** -101, 0.0], 2, True)
    add([1.0, 2.0 ** -99, 2.0 ** -101], 2, False)
    add([1.0, 2.0 ** -100 * 0.75, 0.0], 2, True)
    add([0.0, 0.0, 0.0], 1, True)
    return pins


def _check_tie(fn):
    bad = []
    for i, (cum, k_f, tau, flag) in enumerate(_tie_pins()):
        got, _ = fn(cum, k_f, tau)
        if got != flag:
            bad.append(i)
    return bad


def test_topk_tie_flag_pins():
    assert _check_tie(ref.topk_tie_flag) == []


def test_topk_tie_gap_value():
    flag, gap = ref.topk_tie_flag(np.array([1.0, 4.0, 3.0, 5.0]), 2, TAU)
    assert not flag and gap == pytest.approx(0.25, abs=0)                # (4 - 3) / 4
    flag, gap = ref.topk_tie_flag(np.array([1.0, 4.0, 3.0, 5.0]), 4, TAU)
    assert not flag and gap == float("inf")


def _mutant(kind):
    def fn(cum, k_f, tau):
        n = len(cum)
        if k_f <= 0 or k_f >= n:
            return False, float("inf")
        s = np.sort(cum)[::-1]
        if kind == "next_pair":             # s_(k+1) against s_(k+2)
            a, b = s[min(k_f, n - 1)], s[min(k_f + 1, n - 1)]
        elif kind == "prev_pair":           # s_(k-1) against s_(k)
            a, b = s[max(k_f - 2, 0)], s[k_f - 1]
        else:
            a, b = s[k_f - 1], s[k_f]
        t = tau * (10.0 if kind == "wide" else 1.0)
        floor = 0.0 if kind == "no_floor" else ref.UNDERFLOW_FLOOR
        flag = a - b <= t * a or a < floor
        if kind == "absolute":              # the window read as absolute instead of relative
            flag = a - b <= t or a < floor
        return bool(flag), 0.0
    return fn


@pytest.mark.parametrize("kind", ["next_pair", "prev_pair", "wide", "no_floor", "absolute"])
def test_topk_tie_mistakes_are_caught(kind):
    assert _check_tie(_mutant(kind)) != [], kind


def _near_pins():
    """(R, T, flag) tuples; the offsets 2^-14 (6.1e-5) and 2^-13 (1.22e-4) bracket the 1e-4
    window and are exact in binary."""
    inside, outside = 2.0 ** -14, 2.0 ** -13
    pins = []
    for T in (0.95, 0.5, 0.9):
        base = np.array([0.1, 0.2, 0.3, 0.4, 1.0])
        pins.append((base, T, False))
        for k in range(4):
            for off, flag in ((inside, True), (-inside, True), (outside, False), (-outside, False)):
                R = np.array([0.01, 0.02, 0.03, 0.04, 1.0])      # every other entry far from T
                R[k] = T + off
                pins.append((R, T, flag))
    # R_4 never decides: T just below 1 with every partial entry far away
    pins.append((np.array([0.1, 0.2, 0.3, 0.4, 1.0]), 1.0 - inside, False))
    pins.append((np.array([0.1, 0.2, 0.3, 0.4, 1.0]), 1.0, False))
    pins.append((np.array([0.1, 0.2, 0.3, 1.0 - inside, 1.0]), 1.0, True))
    return pins


def _check_near(fn):
    return [i for i, (R, T, flag) in enumerate(_near_pins()) if fn(R, T) != flag]


def test_near_t_flag_pins():
    assert _check_near(ref.near_t_flag) == []


@pytest.mark.parametrize("kind", ["with_R4", "without_R3", "one_sided", "wide"])
def test_near_t_mistakes_are_caught(kind):
    def fn(R, T):
        R = np.asarray(R, dtype=np.float64)
        if kind == "with_R4":
            return bool(np.any(np.abs(R[:5] - T) <= ref.NEAR_T_WINDOW))
        if kind == "without_R3":
            return bool(np.any(np.abs(R[:3] - T) <= ref.NEAR_T_WINDOW))
        if kind == "one_sided":
            return bool(np.any(R[:4] - T <= ref.NEAR_T_WINDOW))
        return bool(np.any(np.abs(R[:4] - T) <= 10 * ref.NEAR_T_WINDOW))
    assert _check_near(fn) != [], kind


def test_profile_head_uses_the_flags():
    # zero queries: row i spreads 1/(i+1) over keys 0..i, so cum_j = H_n - H_j is strictly
    # decreasing with relative gaps far above tau; T placed on R_2 flags the head
    n, d = 16, 8
    Qg = np.zeros((1, n, d))
    K = np.random.default_rng(0).standard_normal((n, d))
    cls = np.zeros(n, dtype=np.uint8)
    cls[0] = ref.TOKEN_SPECIAL
    prof = ref.profile_head(Qg, K, cls, 0.25, 0.25, 0.7)
    assert prof.near_T == ref.near_t_flag(prof.R, 0.7)
    assert prof.topk_tie == ref.topk_tie_flag(prof.cum, prof.k_f, ref.TIE_TAU_DEFAULT)[0]
    assert not prof.topk_tie                          # harmonic differences are far above tau
    # T placed on R_2 exactly: flagged
    prof2 = ref.profile_head(Qg, K, cls, 0.25, 0.25, float(prof.R[2]))
    assert prof2.near_T
