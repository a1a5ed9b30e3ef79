"""Exact ties at the frequent-set threshold: the selection takes the keys above
the k-th largest cumulative score and, among keys equal to it, the lowest
positions.  The oracle cannot pin this case (its fp64 scores of these keys are
tiny but distinct, so it flags the head), so the check is a property of the
GPU's own output: the frequent set equals the top k_f of the GPU's cum with
ties broken by position, bit for bit.

Inputs: a shared direction u; queries 30u + noise; a sink key at position 0
and ~10 % of the other keys at +30u (live), the rest at -30u (dead).  Every row
sees the sink, so each dead key's attention underflows to exactly 0 in fp32
and the ~90 % dead keys tie at cum = 0, below the 30 % frequent budget."""
import numpy as np
import pytest
import torch

from adaptive_kv_cache_fg_amd import fastgen as fg
from synth import inputs as syn

pytestmark = pytest.mark.gpu


def _layer(B, Hq, Hkv, n, d, dtype, seed):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    Q = 30.0 * u + 0.1 * rng.standard_normal((B, Hq, n, d))
    live = rng.random((B, Hkv, n)) < 0.1
    live[:, :, 0] = True
    K = np.where(live[..., None], 30.0, -30.0) * u + 0.1 * rng.standard_normal((B, Hkv, n, d))
    Q, K = Q.astype(np.float32), K.astype(np.float32)
    if dtype == "bf16":
        Q, K = syn.round_to_bf16(Q), syn.round_to_bf16(K)
    return Q, K


def _upload(x, dtype):
    if dtype == "bf16":
        return torch.from_numpy(syn.bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


@pytest.mark.parametrize("B,Hq,Hkv,n,dtype", [
    (1, 2, 2, 700, "bf16"),       # one score per thread
    (2, 4, 2, 2500, "bf16"),      # several scores per thread, GQA
    (1, 2, 1, 1500, "f32"),
    (1, 1, 1, 33000, "bf16"),     # scores read from memory on every pass
])
def test_threshold_ties_take_the_lowest_positions(B, Hq, Hkv, n, dtype):
    print(f"[ties] B={B} Hq={Hq} Hkv={Hkv} n={n} {dtype}", flush=True)
    r_l, r_f, T = 0.3, 0.3, 0.95
    Q, K = _layer(B, Hq, Hkv, n, 128, dtype, seed=n)
    cls = torch.zeros((B, n), dtype=torch.uint8, device="cuda")
    prof = fg.profile(_upload(Q, dtype), _upload(K, dtype), cls, r_l, r_f, T)
    cum = prof.cum.cpu().numpy()
    F = prof.frequent()
    k_f = int(np.floor(r_f * n))
    for b in range(B):
        for h in range(Hkv):
            c = cum[b, h]
            order = np.lexsort((np.arange(n), -c))          # by score descending, then position
            want = np.zeros(n, bool)
            want[order[:k_f]] = True
            kth = c[order[k_f - 1]]
            assert kth == 0.0 and np.count_nonzero(c == kth) > np.count_nonzero(want & (c == kth)), \
                "the case does not exercise a partial tie"
            assert np.array_equal(F[b, h], want), (b, h)


def test_selection_at_every_workgroup_width():
    """The selection runs one workgroup per head, 1024 threads wide while every head fits on the chip at
    two per CU, 512 up to four per CU and 256 beyond: at head counts in each range (sized from the
    device's CU count) the frequent set is the top k_f of the GPU's cum with ties by position, and the
    recovery is the fp64 identity over the GPU's own cum, band, classes and frequent set."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n, H, r_l, r_f, T = 300, 32, 0.3, 0.3, 0.95
    k_f, w_l = int(np.floor(r_f * n)), int(np.floor(r_l * n))
    for per_cu in (2, 3, 5):
        B = max(1, per_cu * cus // H)
        print(f"[ties] width case: B={B} heads={B * H} ({B * H / cus:.1f} per CU)", flush=True)
        Q, K = _layer(B, H, H, n, 128, "bf16", seed=per_cu)
        rng = np.random.default_rng(100 + per_cu)
        cls_h = np.where(rng.random((B, n)) < 0.05, 1, np.where(rng.random((B, n)) < 0.1, 2, 0)).astype(np.uint8)
        prof = fg.profile(_upload(Q, "bf16"), _upload(K, "bf16"), torch.from_numpy(cls_h).cuda(), r_l, r_f, T,
                          want_band=True)
        cum = prof.cum.cpu().numpy().astype(np.float64)
        band = prof.band.cpu().numpy().astype(np.float64)
        rec = prof.recovery.cpu().numpy().astype(np.float64)
        pol = prof.policy.cpu().numpy()
        F = prof.frequent()
        assert w_l > 0
        for b in range(B):
            spec, punct = cls_h[b] == 1, cls_h[b] == 2
            for h in range(H):
                c = cum[b, h]
                order = np.lexsort((np.arange(n), -c))
                want = np.zeros(n, bool)
                want[order[:k_f]] = True
                assert np.array_equal(F[b, h], want), (B, b, h)
                rest = ~(spec | punct | want)
                m = np.array([c[spec].sum(), c[punct].sum(), c[want & ~spec & ~punct].sum(), band[b, h][rest].sum()])
                R = np.cumsum(m) / n                                   # G = 1
                np.testing.assert_allclose(rec[b, h, :4], R, rtol=0, atol=2e-6)
                assert rec[b, h, 4] == 1.0
                if not np.any(np.abs(rec[b, h, :4] - T) < 1e-6):
                    assert int(pol[b, h]) == next((k for k in range(4) if rec[b, h, k] >= T), 4), (b, h)
