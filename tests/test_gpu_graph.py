"""Decode steps captured in a HIP graph replay exactly like eager launches.

The decode loop is launch-bound at small shapes, so callers capture it; this
checks that replays (each after an eager re-compaction into the same buffers,
with synchronisations in between) reproduce the eager outputs bit for bit and
leave the same cache."""
import numpy as np
import pytest
import torch

from adaptive_kv_cache_fg_amd import fastgen as fg
from synth import inputs as syn

pytestmark = pytest.mark.gpu


def _upload(x, dtype):
    if dtype == "bf16":
        return torch.from_numpy(syn.bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


@pytest.mark.parametrize("hq,hkv", [(8, 8), (8, 2)])
def test_decode_graph_replay_matches_eager(hq, hkv):
    types = ("special", "punct", "heavy", "local", "none", "none", "none", "none")[:hkv]
    spec = syn.custom_spec(syn.CONFIGS[1], seq_len=700, n_q_heads=hq, n_kv_heads=hkv, mix="fixed",
                           fixed_types=types, batch=2)
    steps = 24
    print(f"[graph] hq={hq} hkv={hkv} n={spec.seq_len} steps={steps}", flush=True)
    li = syn.make_layer(spec, 0)
    ds = syn.make_decode_stream(spec, 0, steps)
    Q, K, V = (_upload(x, spec.dtype) for x in (li.Q, li.K, li.V))
    cls = torch.from_numpy(li.token_class).cuda()
    qs, ks, vs = (_upload(x, spec.dtype) for x in (ds.q, ds.k, ds.v))
    ncs = torch.from_numpy(ds.new_class).cuda()
    outs = torch.empty((steps, 2, hq, spec.head_dim), dtype=torch.float32, device="cuda")

    prof = fg.profile(Q, K, cls, spec.r_l, spec.r_f, spec.T[0])
    cache = fg.compact(K, V, cls, prof, hq, max_new_tokens=steps)
    for t in range(steps):
        cache.decode_step(qs[t], ks[t], vs[t], ncs[t], out=outs[t])
    torch.cuda.synchronize()
    eager = outs.clone()
    eager_kept = cache.kept_positions()

    fg.compact(K, V, cls, prof, hq, max_new_tokens=steps, reuse=cache)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(steps):
            cache.decode_step(qs[t], ks[t], vs[t], ncs[t], out=outs[t])
    torch.cuda.synchronize()
    for rep in range(3):
        outs.zero_()
        fg.compact(K, V, cls, prof, hq, max_new_tokens=steps, reuse=cache)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs, eager), rep
        kept = cache.kept_positions()
        assert all(np.array_equal(a, b) for a, b in zip(kept, eager_kept)), rep


def test_decode_partials_leaves_the_cache_unchanged():
    """fg_decode_partials (the split-K launch alone) neither changes the cache nor next_pos, and
    the following steps give the same outputs as a cache that never ran it."""
    spec = syn.custom_spec(syn.CONFIGS[1], seq_len=300, n_q_heads=4, n_kv_heads=2, mix="fixed",
                           fixed_types=("punct", "local"), batch=1)
    steps = 6
    print(f"[partials] n={spec.seq_len} steps={steps}", flush=True)
    li = syn.make_layer(spec, 0)
    ds = syn.make_decode_stream(spec, 0, steps)
    Q, K, V = (_upload(x, spec.dtype) for x in (li.Q, li.K, li.V))
    cls = torch.from_numpy(li.token_class).cuda()
    qs, ks, vs = (_upload(x, spec.dtype) for x in (ds.q, ds.k, ds.v))
    ncs = torch.from_numpy(ds.new_class).cuda()
    prof = fg.profile(Q, K, cls, spec.r_l, spec.r_f, spec.T[0])
    ref = fg.compact(K, V, cls, prof, 4, max_new_tokens=steps)
    ref_out = [ref.decode_step(qs[t], ks[t], vs[t], ncs[t]).clone() for t in range(steps)]
    cache = fg.compact(K, V, cls, prof, 4, max_new_tokens=steps)
    kept0, pos0 = cache.kept_positions(), cache.next_pos
    for t in range(steps):
        cache.decode_partials(qs[t])
    torch.cuda.synchronize()
    assert cache.next_pos == pos0
    assert all(np.array_equal(a, b) for a, b in zip(cache.kept_positions(), kept0))
    for t in range(steps):
        cache.decode_partials(qs[t])                  # repeated: still no effect
        assert torch.equal(cache.decode_step(qs[t], ks[t], vs[t], ncs[t]), ref_out[t]), t


def test_prompt_graph_with_policies_written_into_the_cache():
    """The prompt phase captured as a graph, with the profile writing its policies straight
    into the cache's policy buffer (no copy): every replay, after eager profiles that overwrite
    that buffer with other policies, restores the policies and kept sets of the eager run."""
    hq = hkv = 4
    spec = syn.custom_spec(syn.CONFIGS[1], seq_len=900, n_q_heads=hq, n_kv_heads=hkv, mix="fixed",
                           fixed_types=("special", "punct", "local", "none"), batch=2)
    steps = 8
    print(f"[graph] prompt phase, policies in place, n={spec.seq_len}", flush=True)
    li = syn.make_layer(spec, 0)
    Q, K, V = (_upload(x, spec.dtype) for x in (li.Q, li.K, li.V))
    cls = torch.from_numpy(li.token_class).cuda()
    T = spec.T[0]
    prof = fg.profile(Q, K, cls, spec.r_l, spec.r_f, T)
    cache = fg.compact(K, V, cls, prof, hq, max_new_tokens=steps)
    torch.cuda.synchronize()
    pol0 = prof.policy.reshape(-1).clone()
    kept0 = cache.kept_positions()
    assert torch.equal(cache.t["policy"], pol0)

    def prompt():
        p = fg.profile(Q, K, cls, spec.r_l, spec.r_f, T, policy_out=cache.t["policy"])
        fg.compact(K, V, cls, p, hq, max_new_tokens=steps, reuse=cache, check=False)

    prompt()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        prompt()
    torch.cuda.synchronize()
    Qx = torch.flip(Q, dims=[2]).contiguous()                 # other scores, other policies
    for rep in range(3):
        other = fg.profile(Qx, K, cls, spec.r_l, spec.r_f, 0.01, policy_out=cache.t["policy"])
        torch.cuda.synchronize()
        assert other.policy.data_ptr() == cache.t["policy"].data_ptr()
        assert not torch.equal(cache.t["policy"], pol0), "the eager profile should change the policies"
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(cache.t["policy"], pol0), rep
        kept = cache.kept_positions()
        assert all(np.array_equal(a, b) for a, b in zip(kept, kept0)), rep
