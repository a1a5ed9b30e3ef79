"""GPU parity at the full per-layer sizes of the Llama-1-7B stack, the Llama-1-65B
stack and the 32k-token GQA workload, with inputs drawn on the device (the same
generator the benchmark uses), against the fp64 oracle:

* Llama-1-7B stack (B=8, 32 heads, n=4096): layers 0, 3, 4, 15, 16, 27, 28, 31 --
  the outer four and the middle of the depth mix -- every head of every batch
  entry against the oracle at T = 0.90, 0.95 and 0.99, each T with its own
  compaction and 512 decode steps, decode outputs of two heads of every planted
  type in batch entries 0 and 7;
* Llama-1-65B stack (B=16, 64 heads, n=2048): layers 0, 3, 4, 40, 75, 76, 79, every
  KV head of batch entries 0 and 15 against the oracle; decode outputs at every one
  of the 1024 steps for all of them in layers 0 and 40, for one head of every
  planted type per entry in the others;
* 32k GQA (32 query / 8 KV heads): every KV head against the oracle, decode
  outputs of every head at every one of the 1024 steps.

In every case every head's kept list and final cache are checked exactly, and
the decode outputs of the decode-sampled heads at every listed step."""
import numpy as np
import pytest

from synth import inputs as syn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpl():
    import gpu_parity_lib
    return gpu_parity_lib


def _by_type(spec, layer, per_type):
    """Up to per_type KV heads of each planted type (and unplanted) of one layer."""
    types = syn.head_types(spec, layer)
    picks = []
    for kind in ("special", "punct", "heavy", "local", "none"):
        picks += [h for h, t in enumerate(types) if t == kind][:per_type]
    return sorted(set(picks))


@pytest.mark.parametrize("layer", [0, 3, 4, 15, 16, 27, 28, 31])
def test_llama7b_stack_layer(gpl, layer):
    spec = syn.CONFIGS[2]                              # B=8, 32 heads, n=4096, T in {0.90, 0.95, 0.99}
    sample = [(b, h) for b in range(spec.batch) for h in range(spec.n_kv_heads)]
    decode_sample = [(b, h) for b in (0, 7) for h in _by_type(spec, layer, 2)]
    rep = gpl.run_fullsize(spec, layer, sample, decode_sample)
    assert rep["checked"] == 3 * len(sample)


@pytest.mark.parametrize("layer", [0, 3, 4, 40, 75, 76, 79])
def test_llama65b_stack_layer(gpl, layer):
    spec = syn.CONFIGS[3]                              # B=16, 64 heads, n=2048
    sample = [(b, h) for b in (0, 15) for h in range(spec.n_kv_heads)]
    # decode outputs at every step: every sampled head in an outer and a middle layer, else two heads
    # of every planted type
    decode_sample = sample if layer in (0, 40) else [(b, h) for b in (0, 15) for h in _by_type(spec, layer, 1)]
    rep = gpl.run_fullsize(spec, layer, sample, decode_sample)
    assert rep["checked"] == len(sample)


def test_long_gqa_32k(gpl):
    spec = syn.CONFIGS[4]                              # 32 query / 8 KV heads, n=32768
    heads = [(0, h) for h in range(spec.n_kv_heads)]
    rep = gpl.run_fullsize(spec, 0, heads, heads)     # decode outputs of every head at every step
    assert rep["checked"] == spec.n_kv_heads
