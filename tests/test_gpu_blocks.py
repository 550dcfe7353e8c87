"""GPU parity of the block-granular variant (rmm_select_blocks, then rmm_linear on
the expanded list) against the oracle, through the C ABI.

Bar: kept index lists bit-exact (block scores are summed in the same order and
precision on both sides); the product within rel-L2 1e-5, as for the slice path.
"""
import numpy as np
import pytest
import torch

import input_adaptive_reduced_score_amd as rmm
import oracle
import workloads as W
from _util import dev, dev_padded, rel_l2

pytestmark = pytest.mark.gpu
TOL = 1e-5


def check(x_np, tile, block, keep, wt_np=None):
    print(f"[case] T={x_np.shape[0]} K={x_np.shape[1]} tile={tile} block={block} keep={keep}", flush=True)
    x = dev_padded(x_np)
    idx = rmm.select_blocks(x, tile, block, keep)
    torch.cuda.synchronize()
    ref = oracle.select_blocks(x_np, tile, block, keep)
    assert np.array_equal(idx.cpu().numpy(), ref), (tile, block, keep)
    if wt_np is not None:
        y = rmm.linear(x, dev_padded(wt_np), idx, tile)
        torch.cuda.synchronize()
        yr = oracle.linear(x_np, wt_np, ref, tile)
        assert rel_l2(y.cpu().numpy(), yr) <= TOL
    return idx


def test_ffn_block_demo():
    # the blog's demo shape: 64 blocks of 64 intermediate neurons, keep half
    cs = W.ffn_block_demo()
    idx = check(cs.x, 1, 64, 0.5, cs.wt)
    assert idx.shape == (1, 32 * 64)


@pytest.mark.parametrize("keep", [1 / 64, 0.25, 0.75, 1.0, 0.29])
def test_ffn_block_demo_keeps(keep):
    cs = W.ffn_block_demo()
    check(cs.x, 1, 64, keep, cs.wt)


@pytest.mark.parametrize("T,K,tile,block,dtype", [
    (1, 1024, 1, 1, "bf16"),      # block 1: one block per slice (1024 blocks, the limit)
    (3, 768, 3, 12, "f32"),       # direct tile of 3 rows, fp32
    (7, 640, 2, 64, "bf16"),      # several tiles, ragged last tile
    (1, 4096, 1, 4096, "bf16"),   # one block
    (300, 2048, 128, 64, "bf16"), # column-max partials path (tiles of > 16 rows), ragged
    (5, 32768, 5, 32, "bf16"),    # maximum K
])
def test_block_shapes(T, K, tile, block, dtype):
    cs = W.linear_random(T, K, 16, tile, dtype, seed=T + K + block)
    for keep in (0.5, 0.1, 1.0):
        check(cs.x, tile, block, keep)


def test_block_ties_lowest_blocks():
    # integer activations: many equal block means; the lower block must win
    rng = np.random.default_rng(7)
    x = W.f32_to_bf16_bits(rng.integers(-2, 3, size=(2, 2048)).astype(np.float32))
    for keep in (0.1, 0.5, 0.9):
        check(x, 2, 16, keep)
    z = np.zeros((1, 1024), np.float32)
    idx = check(z, 1, 64, 0.25)
    assert list(idx.cpu().numpy()[0]) == list(range(4 * 64))


def test_block1_equals_slice_selector_unit_weights():
    cs = W.linear_random(2, 1024, 16, 2, "bf16", seed=11)
    x = dev(cs.x)
    a = rmm.select_blocks(x, 2, 1, 0.25)
    b = rmm.select(x, dev(np.ones(1024, np.float32)), 2, 0.25)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
