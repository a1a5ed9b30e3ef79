"""fg_decode_step_noalloc (the decode step with the library's static scratch, for callers that
cannot allocate) against fg_decode_step with a caller workspace: bit-identical outputs and caches,
over two calls in a row, the second on a smaller cache, and a cache too large for the scratch is
refused with FG_ERR_WORKSPACE before any launch."""
import ctypes

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


def _pair(spec, steps):
    """Two caches of the same prompt: one decoded with a workspace, one without."""
    li = syn.make_layer(spec, 0)
    ds = syn.make_decode_stream(spec, 0, steps)
    Q, K, V = (_upload(x, spec.dtype) for x in (li.Q, li.K, li.V))
    cls = torch.from_numpy(li.token_class).cuda()
    prof = fg.profile(Q, K, cls, spec.r_l, spec.r_f, spec.T[0])
    a = fg.compact(K, V, cls, prof, spec.n_q_heads, max_new_tokens=steps)
    b = fg.compact(K, V, cls, prof, spec.n_q_heads, max_new_tokens=steps)
    return a, b, ds


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_noalloc_matches_workspace_decode(dtype, d):
    big = syn.custom_spec(syn.CONFIGS[1], seq_len=1500, head_dim=d, dtype=dtype, n_q_heads=16, n_kv_heads=4,
                          batch=2, mix="fixed", fixed_types=("special", "punct", "local", "none"))
    small = syn.custom_spec(big, seq_len=300, n_q_heads=4, n_kv_heads=2, batch=1, fixed_types=("none", "local"))
    steps = 12
    for spec in (big, small):                       # the second call runs on a smaller cache
        print(f"[noalloc] {dtype} d={d} n={spec.seq_len} B={spec.batch} Hq={spec.n_q_heads} "
              f"Hkv={spec.n_kv_heads}", flush=True)
        a, b, ds = _pair(spec, steps)
        assert fg.lib().fg_decode_workspace_size(ctypes.byref(b.c)) <= fg.lib().fg_decode_noalloc_max_bytes()
        out = torch.empty((spec.batch, spec.n_q_heads, spec.head_dim), dtype=torch.float32, device="cuda")
        for t in range(steps):
            q, k, v = (_upload(x[t], spec.dtype) for x in (ds.q, ds.k, ds.v))
            nc = torch.from_numpy(ds.new_class[t].copy()).cuda()
            want = a.decode_step(q, k, v, nc)
            got = b.decode_step_noalloc(q, k, v, nc, out)
            assert torch.equal(got, want), (spec.seq_len, t)
        torch.cuda.synchronize()
        assert b.next_pos == a.next_pos
        assert all(np.array_equal(x, y) for x, y in zip(a.kept_positions(), b.kept_positions()))
        assert b.error_bits() == 0


def test_noalloc_refuses_a_cache_beyond_its_scratch():
    spec = syn.custom_spec(syn.CONFIGS[1], seq_len=64, n_q_heads=2, n_kv_heads=2, batch=1, mix="fixed",
                           fixed_types=("none", "none"))
    a, b, ds = _pair(spec, 4)
    fake = fg.FgCache.from_buffer_copy(b.c)
    cap = fg.lib().fg_decode_noalloc_max_bytes()
    per_slot = spec.group * (spec.head_dim + 2) * 4
    fake.items_per_head = cap // (spec.batch * spec.n_kv_heads * per_slot) + 1   # state beyond the scratch
    assert fg.lib().fg_decode_workspace_size(ctypes.byref(fake)) > cap
    q, k, v = (_upload(x[0], spec.dtype) for x in (ds.q, ds.k, ds.v))
    out = torch.empty((1, 2, spec.head_dim), dtype=torch.float32, device="cuda")
    st = fg.lib().fg_decode_step_noalloc(ctypes.byref(fake), q.data_ptr(), k.data_ptr(), v.data_ptr(), None,
                                         out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 3 and b"static scratch" in fg.lib().fg_last_error()
    assert fake.next_pos == b.c.next_pos                 # refused before anything ran
