"""GPU parity of the prompt attention output (fg_attention, fg_profile_attention)
against the oracle's O = A V, on seeded synthetic layers: ragged shapes across
several key tiles and row blocks, GQA groups, batch > 1, sharp score
distributions (the lazy-rescale path), full Llama-1-7B layer size, and sampled
rows at the 32k-token GQA size.  The small and the Llama-1-7B shapes run the
launch with two key groups per workgroup, the 32k shape the one with one.
Tolerances are derived in gpu_parity_lib."""
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


TYPES = ("special", "punct", "heavy", "local", "none", "none", "none", "none")


def _spec(n, d, hq, hkv, batch):
    return syn.custom_spec(syn.CONFIGS[1], seq_len=n, head_dim=d, dtype="bf16", n_q_heads=hq, n_kv_heads=hkv,
                           batch=batch, mix="fixed", fixed_types=TYPES[:hkv], decode_steps=8)


def _upload_layer(gpl, li):
    return gpl.upload(li.Q, "bf16"), gpl.upload(li.K, "bf16"), gpl.upload(li.V, "bf16")


def _check_layer(gpl, li, O_g, lse_g=None, heads=None):
    B, Hq, n, _ = li.Q.shape
    Hkv = li.K.shape[1]
    G = Hq // Hkv
    heads = [(b, h) for b in range(B) for h in range(Hkv)] if heads is None else heads
    for b, h in heads:
        Qg = li.Q[b, h * G:(h + 1) * G].astype(np.float64)
        K = li.K[b, h].astype(np.float64)
        gpl.check_attention_head(O_g[b, h * G:(h + 1) * G], Qg, K, li.V[b, h].astype(np.float64))
        if lse_g is not None:
            want = ref.column_scores(Qg, K, 0)["lse"]
            assert np.max(np.abs(lse_g[b, h * G:(h + 1) * G] - want)) <= 2e-4 + 2e-6 * np.max(np.abs(want))


@pytest.mark.parametrize("n,d,hq,hkv,batch", [
    (1, 128, 2, 2, 1),
    (33, 64, 4, 2, 2),
    (200, 128, 8, 2, 2),
    (517, 128, 8, 1, 1),
    (1000, 64, 4, 4, 1),
])
def test_attention_matches_oracle(gpl, n, d, hq, hkv, batch):
    gpl.log(f"[attention] n={n} d={d} Hq={hq} Hkv={hkv} B={batch}")
    li = syn.make_layer(_spec(n, d, hq, hkv, batch))
    Qd, Kd, Vd = _upload_layer(gpl, li)
    O, lse = fg.attention(Qd, Kd, Vd, want_lse=True)
    torch.cuda.synchronize()
    _check_layer(gpl, li, gpl.download(O), lse.cpu().numpy().astype(np.float64))


def test_sharp_scores_take_the_rescale_path(gpl):
    # queries scaled by 4 (exact in bf16): row maxima grow by far more than the
    # lazy-rescale threshold along the keys
    li = syn.make_layer(_spec(700, 128, 4, 4, 1))
    li.Q *= 4.0
    s = li.Q[0, 0].astype(np.float64) @ li.K[0, 0].T / np.sqrt(128) * np.log2(np.e)
    s = np.where(np.tril(np.ones(s.shape, dtype=bool)), s, -np.inf)
    assert np.max(s.max(axis=1) - s[:, :32].max(axis=1)) > 8.0   # some row's max grows past the first unit's
    Qd, Kd, Vd = _upload_layer(gpl, li)
    O, lse = fg.attention(Qd, Kd, Vd, want_lse=True)
    torch.cuda.synchronize()
    _check_layer(gpl, li, gpl.download(O), lse.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("n,d,hq,hkv,batch", [(300, 128, 4, 4, 1), (777, 64, 8, 2, 2)])
def test_profile_attention_matches_oracle(gpl, n, d, hq, hkv, batch):
    # the whole path with the fused prompt pass: profile checks, O, compaction, decode
    gpl.run_case(_spec(n, d, hq, hkv, batch), fused=True)


def test_fused_output_equals_attention_call(gpl):
    spec = _spec(640, 128, 8, 4, 1)
    li = syn.make_layer(spec)
    Qd, Kd, Vd = _upload_layer(gpl, li)
    cls_d = torch.from_numpy(li.token_class).cuda()
    O, lse = fg.attention(Qd, Kd, Vd, want_lse=True)
    fused = fg.profile(Qd, Kd, cls_d, spec.r_l, spec.r_f, 0.95, want_lse=True, V=Vd)
    plain = fg.profile(Qd, Kd, cls_d, spec.r_l, spec.r_f, 0.95, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(fused.out, O) and torch.equal(fused.lse, lse)
    assert torch.equal(fused.policy, plain.policy)
    assert torch.equal(fused.freq_mask, plain.freq_mask)
    torch.testing.assert_close(fused.cum, plain.cum, rtol=2e-4, atol=1e-6)
    torch.testing.assert_close(fused.lse, plain.lse, rtol=0, atol=2e-4)


def test_attention_rejects_fp32(gpl):
    x = torch.zeros((1, 2, 16, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(fg.FastGenError) as e:
        fg.attention(x, x.clone(), x.clone())
    assert e.value.status == 2


def test_attention_llama7b_layer_full_size(gpl):
    spec = syn.CONFIGS[1]                              # 32 heads, d 128, n 2048, bf16
    li = syn.make_layer(spec)
    Qd, Kd, Vd = _upload_layer(gpl, li)
    O, lse = fg.attention(Qd, Kd, Vd, want_lse=True)
    torch.cuda.synchronize()
    O_g = gpl.download(O)
    assert np.all(np.isfinite(O_g))
    picks = []
    for kind in ("special", "punct", "heavy", "local", "none"):
        picks += [h for h, t in enumerate(li.types) if t == kind][:2]
    _check_layer(gpl, li, O_g, lse.cpu().numpy().astype(np.float64), heads=[(0, h) for h in sorted(set(picks))])


def test_attention_long_gqa_sampled_rows(gpl):
    spec = syn.CONFIGS[4]                              # 32 query / 8 KV heads, n 32768
    li = syn.make_layer(spec)
    Qd, Kd, Vd = _upload_layer(gpl, li)
    O, _ = fg.attention(Qd, Kd, Vd)
    torch.cuda.synchronize()
    n = spec.seq_len
    rows = np.array([0, 1, 31, 32, 127, 128, 4095, 16384, n - 2, n - 1])
    G = spec.group
    for h in (0, 4):
        O_rows = O[0, h * G:(h + 1) * G, torch.as_tensor(rows, device=O.device)].float().cpu().numpy().astype(np.float64)
        gpl.check_attention_head(O_rows, li.Q[0, h * G:(h + 1) * G].astype(np.float64),
                                 li.K[0, h].astype(np.float64), li.V[0, h].astype(np.float64), rows=rows)
