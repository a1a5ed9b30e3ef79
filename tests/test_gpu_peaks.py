"""The chip-ceiling micro-benchmarks (fg_peak_*) compute what their headers say, so the
ceilings bench.py reports come from the work it counts:

* MFMA loops on all-ones bf16 operands: each of the 4 chains adds 16 (a 16-long dot product
  of ones) to each of a lane's 16 accumulators per iteration, so a lane's sum is 1024 * iters;
* the MFMA + softmax kernel: the same for waves 0-3; waves 4-7 sum iters values of a chain
  x <- 2^(0.18 x - 0.5) per lane and chain, which stays in (0.7, 0.9);
* the exp loop: every chain settles at the fixed point of x = 2^(-x) (0.641186);
* the copy moves the bytes unchanged; the read stream's per-thread XORs fold to the XOR of
  every 32-bit word of the buffer (each word is read by exactly one thread)."""
import numpy as np
import pytest
import torch

from adaptive_kv_cache_fg_amd import fastgen as fg

pytestmark = pytest.mark.gpu


def test_mfma_and_mix_loops_count_their_work():
    ones = torch.ones(8192, dtype=torch.bfloat16, device="cuda")
    iters, blocks = 10, 6
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    flops = fg.peak_mfma_bf16(ones, out, iters, blocks)
    torch.cuda.synchronize()
    assert flops == blocks * 4 * 4 * 32768 * iters
    assert torch.all(out == 1024.0 * iters)
    mix = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    fg.peak_mfma_softmax(ones, mix, iters, blocks)
    torch.cuda.synchronize()
    m = mix.view(blocks, 512).cpu().numpy()
    assert np.all(m[:, :256] == 1024.0 * iters)
    assert np.all((m[:, 256:] > 8 * iters * 0.7) & (m[:, 256:] < 8 * iters * 0.9))


def test_exp_loop_settles_at_the_fixed_point():
    blocks = 4
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    fg.peak_exp(out, 2000, blocks)
    torch.cuda.synchronize()
    np.testing.assert_allclose(out.cpu().numpy(), 8 * 0.6411857, rtol=0, atol=1e-4)


@pytest.mark.parametrize("nontemporal", [False, True])
def test_copy_and_read_streams(nontemporal):
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    n = (1 << 18) + 4 * 37                                   # a ragged grid-stride tail
    src = torch.randint(-2**31, 2**31 - 1, (n,), dtype=torch.int32, device="cuda", generator=g)
    dst = torch.zeros_like(src)
    assert fg.peak_copy(src, dst, nontemporal, 8) == 8 * n
    blocks = 16
    words = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    assert fg.peak_read(src, words, nontemporal, blocks) == 4 * n
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    host = src.cpu().numpy().view(np.uint32)
    assert np.bitwise_xor.reduce(words.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(host)
