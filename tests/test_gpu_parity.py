"""GPU parity of the whole path (profile -> compact -> decode) against the oracle.

Every case runs the HIP kernels through the C ABI on seeded synthetic inputs
and compares, head by head, with the fp64 oracle on the same inputs (see
gpu_parity_lib for the tolerances).  Shapes span several MFMA / LDS tiles with
ragged tails, GQA groups, batch > 1 and the degenerate budgets.
"""
import pytest

from synth import inputs as syn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib_mod():
    import gpu_parity_lib as gpl
    return gpl


def test_config0_tiny_planted_fp32(lib_mod):
    rep = lib_mod.run_case(syn.CONFIGS[0])
    want = {"special": 0, "punct": 1, "local": 3, "none": 4}
    for hr in rep.heads:
        assert hr.policy_gpu == want[hr.kind], hr


@pytest.mark.parametrize("n,d,dtype,hq,hkv,batch", [
    (1, 128, "bf16", 2, 2, 1),
    (33, 64, "bf16", 4, 2, 2),
    (200, 128, "bf16", 8, 2, 2),
    (300, 64, "f32", 4, 4, 1),
    (517, 128, "bf16", 8, 1, 1),
    (2600, 128, "bf16", 2, 2, 1),      # split sweep 1 with 11 key chunks per row: merge past the prefetched 8
    (1100, 128, "f32", 4, 2, 1),       # fp32 operands at d = 128 (two waves per SIMD), GQA, ragged tiles
    (2600, 64, "f32", 2, 1, 1),        # fp32, both sweeps split
])
def test_ragged_shapes(lib_mod, n, d, dtype, hq, hkv, batch):
    types = ("special", "punct", "heavy", "local", "none", "none", "none", "none")[:hkv]
    spec = syn.custom_spec(syn.CONFIGS[1], seq_len=n, head_dim=d, dtype=dtype, n_q_heads=hq, n_kv_heads=hkv,
                           batch=batch, mix="fixed", fixed_types=types, decode_steps=20)
    lib_mod.run_case(spec)


@pytest.mark.parametrize("r_l,r_f,T", [(0.0, 0.0, 0.95), (0.004, 0.3, 0.9), (1.0, 1.0, 0.99), (0.3, 0.3, 1.0)])
def test_degenerate_budgets(lib_mod, r_l, r_f, T):
    spec = syn.custom_spec(syn.CONFIGS[1], seq_len=260, n_q_heads=4, n_kv_heads=4, mix="fixed",
                           fixed_types=("special", "punct", "local", "none"), r_l=r_l, r_f=r_f, T=(T,),
                           decode_steps=12)
    lib_mod.run_case(spec)


def test_config1_llama7b_layer(lib_mod):
    rep = lib_mod.run_case(syn.CONFIGS[1])
    assert len(rep.heads) == 32
