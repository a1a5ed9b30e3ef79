"""GPU parity of fg_compact_plan on seeded policies, frequent masks and token
classes (no profile needed): kept counts, ring sizes and capacities against the
oracle's kept sets (kept_positions, the level definition) and the budget
arithmetic, and the row / work-item offsets and totals against their prefix-sum
definitions.  Bit-exact integers.  The shapes cover the one-workgroup plan (with
an unaligned class row and a ragged 32-position tail) and the per-head plan plus
separate scan (more class words than one workgroup takes, and more heads)."""
import ctypes

import numpy as np
import pytest
import torch

from adaptive_kv_cache_fg_amd import fastgen as fg
from oracle import fastgen_ref as ref

pytestmark = pytest.mark.gpu


def _inputs(B, Hkv, n, seed):
    rng = np.random.default_rng(seed)
    u = rng.random((B, n))
    cls = np.where(u < 0.01, 1, np.where(u < 0.07, 2, 0)).astype(np.uint8)
    policy = rng.integers(0, 5, size=B * Hkv).astype(np.uint8)
    nw = (n + 31) // 32
    bits = rng.random((B * Hkv, nw * 32)) < 0.3
    bits[:, n:] = False                                      # no frequent bit past the prompt
    fmask = np.packbits(bits.reshape(B * Hkv, nw, 32)[:, :, ::-1], axis=-1, bitorder="big")
    fmask = fmask.reshape(B * Hkv, nw, 4)[:, :, ::-1].copy().view(np.uint32).reshape(B * Hkv, nw)
    return cls, policy, bits[:, :n], fmask


def _expected(cls, policy, bits, Hkv, w_l, max_new, max_new_kept, chunk):
    H = len(policy)
    kept = np.zeros(H, np.int64)
    ring = np.zeros(H, np.int64)
    cap = np.zeros(H, np.int64)
    for hd in range(H):
        b, pol = hd // Hkv, int(policy[hd])
        c = cls[b]
        kept[hd] = len(ref.kept_positions(c, bits[hd], w_l, pol))     # frequent set as a mask
        perm = (c == 1) | ((c == 2) & (pol >= 1)) | (bits[hd] & (pol >= 2)) | (pol == 4)
        ring[hd] = w_l - 1 if (pol == 3 and w_l >= 2) else 0
        cap[hd] = ring[hd] + int(perm.sum()) + (max_new if pol == 4 else max_new_kept)
    items = np.maximum(1, (cap + chunk - 1) // chunk)
    row_offset = np.concatenate([[0], np.cumsum(cap)])
    work_offset = np.concatenate([[0], np.cumsum(items)])
    totals = np.array([cap.sum(), items.sum(), items.max()], np.int64)
    return kept, ring, cap, row_offset, work_offset, totals


@pytest.mark.parametrize("B,Hkv,n,seed", [
    (1, 1, 5, 7),           # one head, no whole 32-position word
    (3, 1, 33, 8),          # one word and a one-position tail per head, unaligned class rows
    (2, 4, 1000, 1),        # one workgroup; n % 32 != 0 and the second class row unaligned
    (1, 3, 257, 2),
    (2, 8, 4096, 3),        # 16 heads x 128 class words: still one workgroup
    (2, 16, 4096, 4),       # 32 heads x 128 class words: per-head plan and a separate scan
    (4, 40, 27001, 5),
    (3, 700, 64, 6),        # 2100 heads
])
def test_plan_matches_definitions(B, Hkv, n, seed):
    print(f"[plan] B={B} Hkv={Hkv} n={n}", flush=True)
    r_l, r_f, T = 0.3, 0.3, 0.95
    max_new, max_new_kept = 37, 11
    cls, policy, bits, fmask = _inputs(B, Hkv, n, seed)
    H = B * Hkv
    dev = "cuda"
    cls_d = torch.from_numpy(cls).to(dev)
    pol_d = torch.from_numpy(policy).to(dev)
    fm_d = torch.from_numpy(fmask).to(dev)
    kept_d, ring_d, cap_d = (torch.full((H,), -7, dtype=torch.int32, device=dev) for _ in range(3))
    ro_d, wo_d = (torch.full((H + 1,), -7, dtype=torch.int64, device=dev) for _ in range(2))
    tot_d = torch.full((3,), -7, dtype=torch.int64, device=dev)
    shape = fg.FgShape(B, Hkv, Hkv, n, 128, 0)
    params = fg.FgParams(r_l, r_f, T)
    L = fg.lib()
    assert L.fg_compact_plan(ctypes.byref(shape), ctypes.byref(params), fg._ptr(cls_d), fg._ptr(pol_d),
                             fg._ptr(fm_d), max_new, max_new_kept, fg._ptr(kept_d), fg._ptr(ring_d),
                             fg._ptr(cap_d), fg._ptr(ro_d), fg._ptr(wo_d), fg._ptr(tot_d), fg._stream()) == 0
    torch.cuda.synchronize()
    chunk = int(L.fg_decode_chunk_rows(ctypes.byref(shape)))
    w_l = ref.budgets(n, r_l, r_f)[1]
    kept, ring, cap, row_offset, work_offset, totals = _expected(cls, policy, bits, Hkv, w_l, max_new,
                                                                 max_new_kept, chunk)
    np.testing.assert_array_equal(kept_d.cpu().numpy(), kept)
    np.testing.assert_array_equal(ring_d.cpu().numpy(), ring)
    np.testing.assert_array_equal(cap_d.cpu().numpy(), cap)
    np.testing.assert_array_equal(ro_d.cpu().numpy(), row_offset)
    np.testing.assert_array_equal(wo_d.cpu().numpy(), work_offset)
    np.testing.assert_array_equal(tot_d.cpu().numpy(), totals)
