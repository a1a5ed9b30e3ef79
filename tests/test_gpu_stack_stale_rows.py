"""Decode through a deep stack of the Llama-1-65B-shaped workload never reads a cache row
that the compaction or a decode step should have written and did not.

Two sets of caches are compacted from the same profiles; before the refill one set's K/V
buffers are zeroed and the other's filled with NaN.  Every generated token is then decoded
through every layer of both sets with the same inputs: the outputs must be finite and equal
bit for bit at every token, so any row left unwritten (a lost or misplaced append, a ring
slot not refilled) shows up at once.  Regression test of a race in the decode merge launch:
every thread of a workgroup read the head's row count while thread 0 of the same workgroup
was storing the incremented count, so a late wave could write its half of the appended row
one row too far."""
import numpy as np
import pytest
import torch

from adaptive_kv_cache_fg_amd import fastgen as fg
from synth import device as sdev
from synth import inputs as syn

pytestmark = pytest.mark.gpu


def test_stack_decode_reads_only_written_rows():
    spec = syn.CONFIGS[3]                             # B=16, 64 heads, n=2048, 1024 decode steps
    L, steps, T = 24, spec.decode_steps, spec.T[0]
    torch.cuda.empty_cache()
    dev = torch.device("cuda")
    print(f"[stale] llama1-65b-stack, {L} layers (outer and middle), {steps} tokens", flush=True)
    layers = list(range(4)) + list(range(38, 54)) + list(range(76, 80))
    lay = [sdev.make_layer_device(spec, l, dev) for l in layers]
    cls = lay[0].token_class
    B, Hq = spec.batch, spec.n_q_heads
    ncls_h = np.ascontiguousarray(np.stack([syn.new_token_classes(spec, b, steps) for b in range(B)], axis=1))
    ncls = torch.from_numpy(ncls_h).to(dev)
    pools = [sdev.make_decode_stream_device(spec, l, 16, dev, classes=ncls_h[:16]) for l in layers]
    mk = int(max(np.count_nonzero(ncls_h[:, b]) for b in range(B)))
    sets = []
    for fill in (0.0, float("nan")):
        caches = []
        for i in range(L):
            prof = fg.profile(lay[i].Q, lay[i].K, cls, spec.r_l, spec.r_f, T)
            c = fg.compact(lay[i].K, lay[i].V, cls, prof, Hq, max_new_tokens=steps, max_new_kept=mk)
            c.t["k"].fill_(fill)
            c.t["v"].fill_(fill)
            fg.compact(lay[i].K, lay[i].V, cls, prof, Hq, max_new_tokens=steps, max_new_kept=mk, reuse=c)
            caches.append(c)
        sets.append((caches, torch.empty((L, B, Hq, spec.head_dim), dtype=torch.float32, device=dev)))
    for t in range(steps):
        i = t % 16
        for caches, outs in sets:
            for l in range(L):
                caches[l].decode_step(pools[l].q[i], pools[l].k[i], pools[l].v[i], ncls[t], out=outs[l])
        if t % 64 == 63 or t == steps - 1:
            a, b = sets[0][1], sets[1][1]
            assert torch.isfinite(b).all(), t
            assert torch.equal(a, b), (t, [l for l in range(L) if not torch.equal(a[l], b[l])])
            print(f"[stale] token {t + 1}: outputs equal and finite", flush=True)
    # the caches themselves: every row in use holds the same bytes
    for l in range(L):
        ca, cb = sets[0][0][l], sets[1][0][l]
        assert torch.equal(ca.t["len"], cb.t["len"])
        ro = ca.t["row_offset"].cpu().numpy()
        ln = ca.t["len"].cpu().numpy()
        rows = torch.from_numpy(np.concatenate([np.arange(ro[h], ro[h] + ln[h]) for h in range(len(ln))])).cuda()
        assert torch.equal(ca.t["pos"][rows], cb.t["pos"][rows]), l
        assert torch.equal(ca.t["k"][rows], cb.t["k"][rows]) and torch.equal(ca.t["v"][rows], cb.t["v"][rows]), l
        assert ca.error_bits() == 0 and cb.error_bits() == 0
