"""GPU parity of decode-time tracking (fg_decode_track) against the oracle's
decode_tracking: per-step level shares of the generated tokens' attention and
the cumulative scores of cached keys, over full caches (the stability
measurement) and over the adaptive caches, at ragged shapes with GQA, fp32 and
bf16.  Tolerances: level shares 1e-4 absolute (as recovery); scores
2e-4 relative plus 1e-6 * G * steps absolute (as the prompt's cumulative
scores).  The oracle takes the GPU's frequent set, policies and prompt scores
as inputs, so the comparison isolates the tracking itself."""
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


def _run(gpl, spec, T, steps, heads=None, full=False):
    gpl.log(f"[track] n={spec.seq_len} d={spec.head_dim} {spec.dtype} Hq={spec.n_q_heads} Hkv={spec.n_kv_heads} "
            f"B={spec.batch} T={T} steps={steps}")
    li = syn.make_layer(spec)
    ds = syn.make_decode_stream(spec, steps=steps)
    B, Hq, n, d = li.Q.shape
    Hkv = li.K.shape[1]
    G = Hq // Hkv
    Qd, Kd, Vd = (gpl.upload(x, spec.dtype) for x in (li.Q, li.K, li.V))
    cls = torch.from_numpy(li.token_class).cuda()
    cls_all_h = np.concatenate([li.token_class, ds.new_class.T], axis=1)          # [B, n + steps]
    cls_all = torch.from_numpy(np.ascontiguousarray(cls_all_h)).cuda()
    prof = fg.profile(Qd, Kd, cls, spec.r_l, spec.r_f, T)
    if full:                                                  # every head keeps every key
        prof = fg.apply_head_map(prof, torch.full((Hkv,), 4, dtype=torch.uint8, device="cuda"))
    cache = fg.compact(Kd, Vd, cls, prof, Hq, max_new_tokens=steps, max_new_kept=steps)
    score = cache.track_init(prof)
    qs, ks, vs = (gpl.upload(x, spec.dtype) for x in (ds.q, ds.k, ds.v))
    ncs = torch.from_numpy(np.ascontiguousarray(ds.new_class)).cuda()
    bins, caches = [], []
    for t in range(steps):
        cache.decode_step(qs[t], ks[t], vs[t], ncs[t])
        bins.append(cache.track(qs[t], cls_all, prof.freq_mask, score).cpu().numpy().astype(np.float64))
        caches.append(cache.kept_positions())
    torch.cuda.synchronize()
    F = prof.frequent()
    pol = prof.policy.cpu().numpy()
    cum = prof.cum.cpu().numpy().astype(np.float64)
    w_l = ref.budgets(n, spec.r_l, spec.r_f)[1]
    sc = score.cpu().numpy().astype(np.float64)
    ro = cache.t["row_offset"].cpu().numpy()
    ln = cache.t["len"].cpu().numpy()
    pos = cache.t["pos"].cpu().numpy()
    heads = [(b, h) for b in range(B) for h in range(Hkv)] if heads is None else heads
    worst_bin = 0.0
    for b, h in heads:
        hd = b * Hkv + h
        K_all = np.concatenate([li.K[b, h], ds.k[:, b, h]]).astype(np.float64)
        q = ds.q[:, b, h * G:(h + 1) * G].astype(np.float64)
        want_bins, want_score = ref.decode_tracking(K_all, cls_all_h[b], F[b, h], w_l, n,
                                                    [c[hd] for c in caches], q, cum[b, h])
        got_bins = np.array([x[b, h] for x in bins])
        err = float(np.max(np.abs(got_bins - want_bins)))
        worst_bin = max(worst_bin, err)
        assert err <= 1e-4, (b, h, int(pol[b, h]), err)
        rows = slice(ro[hd], ro[hd] + ln[hd])
        got_score = {int(j): float(v) for j, v in zip(pos[rows], sc[rows]) if j >= 0}
        assert sorted(got_score) == sorted(want_score), (b, h)
        for j, v in want_score.items():
            assert abs(got_score[j] - v) <= 2e-4 * abs(v) + 1e-6 * G * steps, (b, h, j, got_score[j], v)
    return pol, bins, worst_bin


@pytest.mark.parametrize("n,d,dtype,hq,hkv,batch", [
    (300, 128, "bf16", 8, 4, 2),
    (129, 64, "f32", 4, 4, 1),
    (700, 128, "bf16", 16, 2, 1),
])
def test_track_full_cache(gpl, n, d, dtype, hq, hkv, batch):
    types = ("special", "punct", "heavy", "local")[:hkv]
    spec = syn.custom_spec(syn.CONFIGS[1], seq_len=n, head_dim=d, dtype=dtype, n_q_heads=hq, n_kv_heads=hkv,
                           batch=batch, mix="fixed", fixed_types=types)
    pol, bins, _ = _run(gpl, spec, 0.95, 12, full=True)
    assert np.all(pol == 4)
    for x in bins:
        np.testing.assert_allclose(x.sum(axis=-1), 1.0, atol=1e-5)


@pytest.mark.parametrize("T", [0.9, 0.95])
def test_track_adaptive_caches(gpl, T):
    spec = syn.custom_spec(syn.CONFIGS[1], seq_len=400, head_dim=128, n_q_heads=8, n_kv_heads=8, batch=2,
                           mix="fixed", fixed_types=("special", "punct", "heavy", "local", "none", "special",
                                                     "punct", "local"))
    pol, bins, _ = _run(gpl, spec, T, 10)
    for x in bins:                                            # no mass above a head's policy
        for b in range(spec.batch):
            for h in range(spec.n_kv_heads):
                assert np.all(x[b, h, pol[b, h] + 1:] == 0.0)


def test_track_config0_tiny_planted(gpl):
    spec = syn.CONFIGS[0]
    _run(gpl, spec, spec.T[0], spec.decode_steps, full=True)


def test_track_llama7b_layer_sampled_heads(gpl):
    spec = syn.CONFIGS[1]                                     # 32 heads, n 2048, bf16, full caches
    types = syn.head_types(spec, 0)
    picks = sorted({h for kind in ("special", "punct", "local", "none")
                    for h in [i for i, t in enumerate(types) if t == kind][:1]})
    _run(gpl, spec, spec.T[0], 6, heads=[(0, h) for h in picks], full=True)
