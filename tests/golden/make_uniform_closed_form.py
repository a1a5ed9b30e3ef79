"""Write uniform_closed_form.json: exact values for a head whose queries are all zero.

With q_i = 0 every causal score is 0, so A_ij = 1/(i+1) for j <= i.  Then (exact
rationals, from the definitions in the hyper.ai summary of "Model Tells You What
to Discard", Method section):

* cum_j = sum_{i=j}^{n-1} 1/(i+1) = H_n - H_j (harmonic numbers), strictly
  decreasing, so the frequent set is {0 .. k_f-1};
* with only position 0 special and no punctuation:
    R_0 = R_1 = cum_0 / n = H_n / n,
    R_2 = (1/n) sum_i min(i+1, k_f)/(i+1),
    R_3 = (1/n) sum_i min(i+1, k_f + w_l)/(i+1)   (a prefix and a suffix of [0, i]),
    R_4 = 1;
* band_j = sum_{i=j}^{min(n, j+w_l)-1} 1/(i+1) = H_{min(n, j+w_l)} - H_j;
* lse_i = log(i+1).

Only ``fractions`` is used; nothing here calls the oracle.
"""
import json
import math
from fractions import Fraction
from pathlib import Path


def harmonic(k):
    return sum((Fraction(1, t) for t in range(1, k + 1)), Fraction(0))


def case(n, k_f, w_l):
    H = [harmonic(k) for k in range(n + 1)]
    cum = [H[n] - H[j] for j in range(n)]
    band = [H[min(n, j + w_l)] - H[j] for j in range(n)]
    R0 = H[n] / n
    R2 = sum((Fraction(min(i + 1, k_f), i + 1) for i in range(n)), Fraction(0)) / n
    R3 = sum((Fraction(min(i + 1, k_f + w_l), i + 1) for i in range(n)), Fraction(0)) / n
    return {
        "n": n, "k_f": k_f, "w_l": w_l,
        "cum": [float(c) for c in cum],
        "band": [float(b) for b in band],
        "lse": [math.log(i + 1) for i in range(n)],
        "R": [float(R0), float(R0), float(R2), float(R3), 1.0],
        "R_exact": [str(R0), str(R0), str(R2), str(R3), "1"],
    }


if __name__ == "__main__":
    # r_l = r_f = 0.3 at n = 64 gives k_f = w_l = 19; n = 37 with r = 0.25 gives 9.
    out = {"source": "closed form of uniform causal attention (zero queries)",
           "cases": [case(64, 19, 19), case(37, 9, 9), case(16, 4, 1)]}
    Path(__file__).with_name("uniform_closed_form.json").write_text(json.dumps(out, indent=1))
