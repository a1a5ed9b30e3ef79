"""GPU parity of the multi-prompt head map (fg_head_map_accumulate / fg_head_map_finish)
against the oracle's head_type_map, and of compaction under a map's policies."""
import numpy as np
import pytest
import torch

from adaptive_kv_cache_fg_amd import fastgen as fg
from oracle import fastgen_ref as ref
from synth import inputs as syn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpl():
    import gpu_parity_lib
    return gpu_parity_lib


def _profile_prompts(gpl, spec, T):
    li = syn.make_layer(spec)
    Qd, Kd = gpl.upload(li.Q, spec.dtype), gpl.upload(li.K, spec.dtype)
    Vd = gpl.upload(li.V, spec.dtype)
    cls = torch.from_numpy(li.token_class).cuda()
    prof = fg.profile(Qd, Kd, cls, spec.r_l, spec.r_f, T)
    return li, (Qd, Kd, Vd, cls), prof


def _oracle_map(li, spec, T):
    B, Hq = li.Q.shape[:2]
    Hkv = li.K.shape[1]
    G = Hq // Hkv
    profs = [[ref.profile_head(li.Q[b, h * G:(h + 1) * G], li.K[b, h], li.token_class[b], spec.r_l, spec.r_f, T)
              for h in range(Hkv)] for b in range(B)]
    R = np.array([[p.R for p in row] for row in profs])
    pol = np.array([[p.policy for p in row] for row in profs])
    return profs, ref.head_type_map(R, pol, T)


@pytest.mark.parametrize("spec_kw", [
    dict(base=0, batch=8),                                                       # tiny planted fp32, 8 prompts
    dict(base=1, batch=6, seq_len=700, n_q_heads=8, n_kv_heads=4, mix="fixed",
         fixed_types=("special", "punct", "local", "none")),                     # bf16 GQA, 6 prompts
])
def test_head_map_matches_oracle(gpl, spec_kw):
    kw = dict(spec_kw)
    spec = syn.custom_spec(syn.CONFIGS[kw.pop("base")], **kw)
    T = spec.T[0]
    li, (Qd, Kd, Vd, cls), prof = _profile_prompts(gpl, spec, T)
    hm = fg.HeadMap(spec.n_kv_heads)
    hm.add(prof)
    mean, policy = hm.finish(T)
    torch.cuda.synchronize()
    mean_g = mean.cpu().numpy().astype(np.float64)
    pol_g = policy.cpu().numpy().astype(np.int64)
    count_g = hm.policy_count.cpu().numpy()
    R_g = prof.recovery.cpu().numpy().astype(np.float64)
    ppol_g = prof.policy.cpu().numpy().astype(np.int64)
    # the map's arithmetic on the GPU's own per-prompt outputs: exact
    own = ref.head_type_map(R_g, ppol_g, T)
    assert np.array_equal(pol_g, own["policy"])
    assert np.array_equal(count_g, own["count"])
    np.testing.assert_allclose(mean_g, own["mean"], rtol=2.0 ** -23, atol=0)
    # against the oracle's own profiles
    _, want = _oracle_map(li, spec, T)
    assert np.max(np.abs(mean_g - want["mean"])) <= gpl.REC_TOL
    for h in range(spec.n_kv_heads):
        if not np.any(np.abs(want["mean"][h, :4] - T) <= ref.NEAR_T_WINDOW):
            assert pol_g[h] == want["policy"][h], (h, mean_g[h], want["mean"][h])
    if spec.cfg_id == 0:                   # the planted special / local / unplanted heads are unambiguous
        kinds = {"special": 0, "local": 3, "none": 4}
        assert all(int(p) == kinds[t] for p, t in zip(pol_g, li.types) if t in kinds)
    # applying the map: every prompt compacted under the map's policies with its own frequent set
    cache = fg.compact(Kd, Vd, cls, fg.apply_head_map(prof, policy), spec.n_q_heads, max_new_tokens=4,
                       max_new_kept=4)
    kept = cache.kept_positions()
    F = prof.frequent()
    k_f, w_l = ref.budgets(spec.seq_len, spec.r_l, spec.r_f)
    for b in range(spec.batch):
        for h in range(spec.n_kv_heads):
            assert np.array_equal(kept[b * spec.n_kv_heads + h],
                                  ref.kept_positions(li.token_class[b], F[b, h], w_l, int(pol_g[h])))


def test_head_map_accumulates_over_calls(gpl):
    spec = syn.custom_spec(syn.CONFIGS[0], batch=8)
    T = spec.T[0]
    li, (Qd, Kd, Vd, cls), prof = _profile_prompts(gpl, spec, T)
    one = fg.HeadMap(spec.n_kv_heads)
    one.add(prof)
    split = fg.HeadMap(spec.n_kv_heads)
    for lo, hi in ((0, 3), (3, 8)):
        part = fg.Profile(prof.policy[lo:hi].contiguous(), prof.cum[lo:hi].contiguous(),
                          prof.recovery[lo:hi].contiguous(), prof.freq_mask[lo:hi].contiguous(), None, None,
                          prof.r_l, prof.r_f, prof.T)
        split.add(part)
    assert split.n_prompts == one.n_prompts == 8
    m1, p1 = one.finish(T)
    m2, p2 = split.finish(T)
    torch.cuda.synchronize()
    assert torch.equal(one.policy_count, split.policy_count)
    assert torch.equal(one.rec_sum, split.rec_sum)      # prompt-by-prompt order in both
    assert torch.equal(m1, m2) and torch.equal(p1, p2)


def test_headmap_cli_and_sensitivity(gpl, capsys):
    from adaptive_kv_cache_fg_amd import headmap
    import json
    assert headmap.main(["--config", "0", "--prompts", "6", "--r", "0.2", "0.3", "--T", "0.9", "0.95", "0.99"]) == 0
    out = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    m = out["layers"]["0"]
    assert m["n_prompts"] == 6 and sum(m["policy_histogram"]) == 4
    assert 0.0 < m["agreement"] <= 1.0
    assert 0.0 < m["kept_share_map_policies"] <= 1.0
    rows = out["sensitivity"]
    assert len(rows) == 6
    for row in rows:
        assert row["retained_min"] >= row["T"] - 1e-6          # the chosen policy meets T (or is full)
    for r in (0.2, 0.3):                                        # a higher T never keeps fewer keys
        shares = [row["kept_share"] for row in rows if row["r"] == r]
        assert shares == sorted(shares)
