"""GPU parity at the full per-layer sizes of the Llama-1-7B stack, the Llama-1-65B
stack and the 32k-token GQA workload, on sampled heads (the oracle is fp64 and
O(n^2) per head), plus properties and forced-mode kept lists for every head."""
import numpy as np
import pytest

from synth import inputs as syn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpl():
    import gpu_parity_lib
    return gpu_parity_lib


def _sample(spec, layer, batch_entries, per_type=2, seed=0):
    """A few KV heads of every planted type (and unplanted) for the given batch entries."""
    types = syn.head_types(spec, layer)
    picks = []
    for kind in ("special", "punct", "heavy", "local", "none"):
        hs = [h for h, t in enumerate(types) if t == kind][:per_type]
        picks += hs
    return [(b, h) for b in batch_entries for h in sorted(set(picks))]


@pytest.mark.parametrize("layer", [0, 16])
def test_llama7b_stack_layer(gpl, layer):
    spec = syn.CONFIGS[2]                              # B=8, 32 heads, n=4096, T in {0.90, 0.95, 0.99}
    sample = _sample(spec, layer, [0, 7])
    rep = gpl.run_fullsize(spec, layer, sample, decode_sample=sample[:6])
    assert rep["checked"] == 3 * len(sample)


@pytest.mark.parametrize("layer", [0, 40])
def test_llama65b_stack_layer(gpl, layer):
    spec = syn.CONFIGS[3]                              # B=16, 64 heads, n=2048
    sample = _sample(spec, layer, [0, 15])
    gpl.run_fullsize(spec, layer, sample, decode_sample=sample[:6])


def test_long_gqa_32k(gpl):
    spec = syn.CONFIGS[4]                              # 32 query / 8 KV heads, n=32768
    sample = [(0, 0), (0, 4)]                          # one planted (special) and one unplanted KV head
    gpl.run_fullsize(spec, 0, sample, decode_sample=sample)
