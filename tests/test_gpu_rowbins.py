"""GPU parity of fg_profile_row_bins: the attention mass of every query row on
the special, punct, frequent, local and remaining keys, against the oracle's
row_bins (fp64, levels by the shortlist definition) on the same seeded inputs.

Tolerance: 5e-5 absolute per bin.  A bin is a sum of at most n row-softmax
entries whose total is 1; each entry carries the fp32 error of its score
(products of bf16-exact operands accumulated in fp32 over d terms) and of the
exp2 and row log-sum-exp, a few 1e-6 relative, so the sum is off by a few 1e-6
of the row's mass; 5e-5 leaves a margin of ten.  Heads whose frequent set the
oracle flags as a top-k tie (the k-th and next cumulative scores within the
relative window the parity tests use) may legitimately differ in F; for them
only the special and punct bins and the row totals are compared.

Also checked on the GPU's own output: every row's bins sum to 1, and summed
over rows and the group's query heads they give fg_profile's recovery."""
import numpy as np
import pytest
import torch

from adaptive_kv_cache_fg_amd import fastgen as fg
from oracle import fastgen_ref as ref
from synth import inputs as syn

pytestmark = pytest.mark.gpu

BIN_TOL = 5e-5
TIE_TAU = 3e-5


def _upload(x, dtype):
    if dtype == "bf16":
        return torch.from_numpy(syn.bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def _run(spec, heads=None):
    li = syn.make_layer(spec)
    Q, K = _upload(li.Q, spec.dtype), _upload(li.K, spec.dtype)
    cls = torch.from_numpy(li.token_class).cuda()
    T = spec.T[0]
    prof = fg.profile(Q, K, cls, spec.r_l, spec.r_f, T, want_lse=True)
    bins = fg.row_bins(Q, K, cls, prof).cpu().numpy().astype(np.float64)
    rec = prof.recovery.cpu().numpy()
    F_gpu = prof.frequent()
    B, Hq, n, _ = bins.shape
    Hkv = spec.n_kv_heads
    G = Hq // Hkv
    # properties of the GPU's output at any size
    np.testing.assert_allclose(bins.sum(axis=-1), 1.0, atol=BIN_TOL)
    assert bins.min() >= 0.0
    per_head = bins.reshape(B, Hkv, G * n, 5).sum(axis=2) / (G * n)
    np.testing.assert_allclose(np.cumsum(per_head, axis=-1)[..., :4], rec[..., :4], atol=1e-4)
    # oracle parity on the chosen heads
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hkv)]
    for b, h in heads:
        hp = ref.profile_head(li.Q[b, h * G:(h + 1) * G], li.K[b, h], li.token_class[b], spec.r_l, spec.r_f, T,
                              tau=TIE_TAU)
        got = bins[b, h * G:(h + 1) * G]
        if hp.topk_tie:
            np.testing.assert_allclose(got[..., :2], hp.bins[..., :2], atol=BIN_TOL, err_msg=f"head {(b, h)}")
            continue
        assert np.array_equal(F_gpu[b, h], hp.F), (b, h)
        err = np.abs(got - hp.bins).max()
        assert err <= BIN_TOL, (b, h, err)


@pytest.mark.parametrize("n,d,dtype,hq,hkv,batch", [
    (1, 128, "bf16", 2, 2, 1),
    (33, 64, "bf16", 4, 2, 2),          # one partial row block, GQA
    (300, 128, "bf16", 4, 4, 1),        # two row blocks, ragged tail
    (300, 64, "f32", 4, 4, 1),
    (600, 128, "f32", 2, 2, 1),
    (1100, 128, "bf16", 8, 2, 1),       # five row blocks, groups of four query heads
])
def test_row_bins_match_oracle(n, d, dtype, hq, hkv, batch):
    print(f"[rowbins] n={n} d={d} {dtype} Hq={hq} Hkv={hkv} B={batch}", flush=True)
    types = ("special", "punct", "heavy", "local", "none", "none", "none", "none")[:hkv]
    spec = syn.custom_spec(syn.CONFIGS[1], seq_len=n, head_dim=d, dtype=dtype, n_q_heads=hq, n_kv_heads=hkv,
                           batch=batch, mix="fixed", fixed_types=types)
    _run(spec)


def test_row_bins_planted_heads_fp32():
    print("[rowbins] tiny planted fp32", flush=True)
    _run(syn.CONFIGS[0])


def test_row_bins_llama7b_layer_sampled_heads():
    """The one-layer shape (32 heads, n = 2048): properties on every row, the
    oracle on three heads."""
    print("[rowbins] llama7b layer n=2048", flush=True)
    _run(syn.CONFIGS[1], heads=[(0, 0), (0, 13), (0, 31)])


def test_row_bins_needs_lse():
    spec = syn.custom_spec(syn.CONFIGS[1], seq_len=64, n_q_heads=2, n_kv_heads=2, mix="fixed",
                           fixed_types=("punct", "local"))
    li = syn.make_layer(spec)
    Q, K = _upload(li.Q, "bf16"), _upload(li.K, "bf16")
    cls = torch.from_numpy(li.token_class).cuda()
    prof = fg.profile(Q, K, cls, spec.r_l, spec.r_f, spec.T[0])
    with pytest.raises(ValueError):
        fg.row_bins(Q, K, cls, prof)


def test_row_bins_long_gqa_sampled_rows():
    """The 32k GQA shape (32 query heads on 8 KV heads, n = 32768): rows sum to 1 and
    reproduce fg_profile's recovery on every head; on sampled rows of three query heads the
    special and punct bins (which do not depend on the frequent set) match the oracle's
    attention row restricted to those classes."""
    print("[rowbins] long GQA n=32768, sampled rows", flush=True)
    spec = syn.CONFIGS[4]
    li = syn.make_layer(spec)
    Q, K = _upload(li.Q, spec.dtype), _upload(li.K, spec.dtype)
    cls = torch.from_numpy(li.token_class).cuda()
    prof = fg.profile(Q, K, cls, spec.r_l, spec.r_f, spec.T[0], want_lse=True)
    bins_d = fg.row_bins(Q, K, cls, prof)
    rec = prof.recovery.cpu().numpy()
    bins = bins_d.cpu().numpy().astype(np.float64)
    del bins_d
    B, Hq, n, _ = bins.shape
    G = Hq // spec.n_kv_heads
    np.testing.assert_allclose(bins.sum(axis=-1), 1.0, atol=BIN_TOL)
    per_head = bins.reshape(B, spec.n_kv_heads, G * n, 5).sum(axis=2) / (G * n)
    np.testing.assert_allclose(np.cumsum(per_head, axis=-1)[..., :4], rec[..., :4], atol=1e-4)
    rng = np.random.default_rng(44)
    c = li.token_class[0]
    for hq in (0, 13, 31):
        h = hq // G
        for i in sorted(set(rng.integers(0, n, size=6).tolist()) | {0, n - 1}):
            A = ref.causal_attention_rows(li.Q[0, hq, i:i + 1].astype(np.float64), li.K[0, h].astype(np.float64), i)[0]
            want0 = A[c == ref.TOKEN_SPECIAL].sum()
            want1 = A[c == ref.TOKEN_PUNCT].sum()
            assert abs(bins[0, hq, i, 0] - want0) <= BIN_TOL, (hq, i)
            assert abs(bins[0, hq, i, 1] - want1) <= BIN_TOL, (hq, i)


@pytest.mark.parametrize("r_l,r_f", [(0.0, 0.0), (1.0, 1.0), (0.004, 0.3), (0.3, 0.0)])
def test_row_bins_degenerate_budgets(r_l, r_f):
    """No local window (w_l = 0), a window covering every pair (w_l = n), a one-key window,
    an empty frequent set."""
    print(f"[rowbins] budgets r_l={r_l} r_f={r_f}", flush=True)
    spec = syn.custom_spec(syn.CONFIGS[1], seq_len=260, n_q_heads=4, n_kv_heads=4, mix="fixed",
                           fixed_types=("special", "punct", "local", "none"), r_l=r_l, r_f=r_f)
    _run(spec)
