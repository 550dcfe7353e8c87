"""rmm_linear_noalloc (the reduced product without a caller workspace) against
rmm_linear with one, through the C ABI.  Two calls in a row share the library's
device scratch array, the second with a smaller input; each must equal
rmm_linear's result bit for bit (same kernels, same summation order).  A product
whose scratch would not fit the array is refused before anything is enqueued."""
import pytest
import torch

import input_adaptive_reduced_score_amd as rmm
import workloads as W
from _util import dev, dev_padded

pytestmark = pytest.mark.gpu


def _both(cs, r):
    x, wt, c = dev_padded(cs.x), dev_padded(cs.wt), dev(cs.c)
    idx = rmm.select(x, c, cs.tile, r)
    ref = rmm.linear(x, wt, idx, cs.tile)
    got = rmm.linear_noalloc(x, wt, idx, cs.tile)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_equals_linear_twice_second_smaller():
    cases = ((W.linear_decode(), 0.5),                              # 1 x 14336 x 4096: split-K partials
             (W.linear_random(3, 3000, 1000, 1, "bf16", seed=5), 0.3))  # smaller, three tokens
    for cs, r in cases:
        print(f"[case] no-alloc {cs.name} r={r}", flush=True)
        ref, got = _both(cs, r)
        assert torch.equal(ref, got), f"{cs.name} r={r}: no-alloc result differs from rmm_linear"


def test_noalloc_mfma_path_then_smaller():
    # tiles of 64 tokens run the MFMA path, whose packed activations live in the array
    for T, K, M, tile in ((256, 2048, 1024, 64), (64, 512, 264, 64)):
        cs = W.linear_random(T, K, M, tile, "bf16", seed=T)
        print(f"[case] no-alloc {cs.name} r=0.5", flush=True)
        ref, got = _both(cs, 0.5)
        assert torch.equal(ref, got), f"{cs.name}: no-alloc result differs from rmm_linear"


def test_noalloc_refuses_products_beyond_the_array():
    # 4096 tokens in one tile, 4096 kept slices: the MFMA path would pack 32 MiB of activations
    T = K = M = 4096
    x = torch.zeros((T, K), dtype=torch.bfloat16, device="cuda:0")
    wt = torch.zeros((K, M), dtype=torch.bfloat16, device="cuda:0")
    idx = torch.arange(K, dtype=torch.int32, device="cuda:0").reshape(1, K)
    with pytest.raises(rmm.RmmError) as e:
        rmm.linear_noalloc(x, wt, idx, T)
    assert e.value.status == 2 and "scratch" in e.value.detail
