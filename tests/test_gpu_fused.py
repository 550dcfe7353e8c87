"""GPU parity of the one-launch decode step rmm_select_linear (selection and
reduced product of one token) against the oracle and against rmm_select +
rmm_linear, through the C ABI.

Bars: the kept index list bit-exact (the oracle's and rmm_select's); y within
rel-L2 1e-5 of the oracle (fp32 accumulation of exact products: the fused
kernel adds each split's rows kept for certain before the others, a different
fixed order than rmm_linear's); repeated calls bit-identical (the launch's
flags return to zero after every call)."""
import numpy as np
import pytest
import torch

import input_adaptive_reduced_score_amd as rmm
import oracle
import workloads as W
from _util import dev, dev_padded, rel_l2

pytestmark = pytest.mark.gpu
TOL = 1e-5


def run_fused(cs, r, want_idx=True, both=False):
    """The fused step against the oracle; both=True also runs it without the index list (the
    selector then publishes the threshold and skips its compaction) and checks that y is the same."""
    assert cs.T == 1
    x, wt, c = dev_padded(cs.x), dev_padded(cs.wt), dev(cs.c)
    print(f"[case] fused {cs.name} r={r}", flush=True)
    y, idx = rmm.select_linear(x, c, r, wt, want_idx=want_idx)
    torch.cuda.synchronize()
    idx_ref = oracle.select(cs.x, cs.c, 1, r)
    if want_idx:
        assert np.array_equal(idx.cpu().numpy(), idx_ref), f"{cs.name} r={r}: kept slice lists differ"
    yr = oracle.linear(cs.x, cs.wt, idx_ref, 1)
    err = rel_l2(y.cpu().numpy(), yr)
    assert err <= TOL, f"{cs.name} r={r}: rel-L2 {err:.3e}"
    if both:
        y2, _ = rmm.select_linear(x, c, r, wt, want_idx=not want_idx)
        torch.cuda.synchronize()
        assert torch.equal(y, y2), f"{cs.name} r={r}: y depends on whether the index list is asked for"
    return y, idx


@pytest.mark.parametrize("r", [0.25, 0.5, 0.75, 1.0])
def test_decode_down_proj_full_size(r):
    run_fused(W.linear_decode(), r)


@pytest.mark.parametrize("r", [0.25, 0.5, 0.75, 1.0])
def test_decode_down_proj_without_index_list(r):
    # the benchmark's call: no kept list asked for (the threshold goes out before the selector's
    # compaction, which then does not run)
    cs = W.linear_decode()
    x, wt, c = dev_padded(cs.x), dev_padded(cs.wt), dev(cs.c)
    print(f"[case] fused {cs.name} r={r} no index list", flush=True)
    y, idx = rmm.select_linear(x, c, r, wt, want_idx=False)
    torch.cuda.synchronize()
    assert idx is None
    yr = oracle.linear(cs.x, cs.wt, oracle.select(cs.x, cs.c, 1, r), 1)
    err = rel_l2(y.cpu().numpy(), yr)
    assert err <= TOL, f"r={r}: rel-L2 {err:.3e}"


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_decode_down_proj_other_seeds(seed):
    run_fused(W.linear_decode(seed=seed), 0.5)


def test_equals_select_then_linear():
    cs = W.linear_decode(seed=5)
    x, wt, c = dev(cs.x), dev(cs.wt), dev(cs.c)
    for r in (0.3, 0.5, 0.9):
        y, idx = rmm.select_linear(x, c, r, wt)
        idx2 = rmm.select(x, c, 1, r)
        y2 = rmm.linear(x, wt, idx2, 1)
        torch.cuda.synchronize()
        assert torch.equal(idx, idx2)
        assert rel_l2(y.cpu().numpy(), y2.cpu().numpy()) <= 1e-6


def test_tiny_fp32():
    cs = W.linear_random(1, 512, 1024, 1, "f32", seed=0, xsigma=1.0, wsigma=0.05)
    for r in (0.5, 0.25, 1.0, 1 / 3, 0.001):
        run_fused(cs, r)


@pytest.mark.parametrize("K,M,dtype", [
    (1, 8, "bf16"), (7, 520, "bf16"), (100, 64, "f32"), (1003, 4100, "bf16"), (4096, 1024, "f32"),
    (16385, 512, "bf16"), (32768, 4096, "bf16"), (14336, 16384, "bf16"), (3000, 8, "f32"),
    (4096, 6144, "bf16"), (4096, 4096, "bf16"),  # the decode layer's QKV (12 column slices) and o_proj
])
def test_ragged_and_edge_shapes(K, M, dtype):
    cs = W.linear_random(1, K, M, 1, dtype, seed=K + M)
    for r in (0.3, 1.0, 1.0 / K):
        run_fused(cs, r, both=True)


def test_ties_lowest_indices_win():
    # integer-valued activations and unit slice weights: many equal scores, the lower index wins
    cs = W.linear_random(1, 14336, 4096, 1, "bf16", seed=9)
    rng = np.random.default_rng(9)
    cs.x[:] = W.f32_to_bf16_bits(rng.integers(-3, 4, size=cs.x.shape).astype(np.float32))
    cs.c[:] = 1.0
    for r in (0.25, 0.5, 0.8):
        run_fused(cs, r, both=True)


def test_all_equal_scores():
    cs = W.linear_random(1, 5000, 1000, 1, "bf16", seed=10)
    cs.x[:] = W.f32_to_bf16_bits(np.ones(cs.x.shape, np.float32))
    cs.c[:] = 2.0
    _, idx = run_fused(cs, 0.5, both=True)
    assert np.array_equal(idx.cpu().numpy()[0], np.arange(2500))


@pytest.mark.parametrize("scale", [1.0 / 64, 64.0])
def test_early_estimate_misled_by_its_sample(scale):
    # each workgroup estimates the threshold from its own slices' keys; here the first 4096
    # slices score far below (above) the rest, so the workgroups holding them (the others)
    # stream rows early that the selection drops, and take them back
    cs = W.linear_random(1, 14336, 4096, 1, "bf16", seed=12)
    cs.c[:4096] *= np.float32(scale)
    for r in (0.25, 0.5, 0.75):
        run_fused(cs, r)


def test_without_index_list_and_repeated_calls():
    # the benchmark's call: no index list; repeated calls and calls of other shapes in between give
    # bit-identical results (the launch's flags are cleared after every call)
    cs = W.linear_decode(seed=6)
    x, wt, c = dev(cs.x), dev(cs.wt), dev(cs.c)
    y0, _ = rmm.select_linear(x, c, 0.5, wt, want_idx=False)
    y0 = y0.clone()
    small = W.linear_random(1, 300, 72, 1, "bf16", seed=11)
    for i in range(5):
        y1, i1 = rmm.select_linear(x, c, 0.5, wt)
        run_fused(small, 0.4)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1), f"call {i} differs"
    run_fused(cs, 0.5)


def test_graph_replays_match_eager():
    cs = W.linear_decode(seed=7)
    x, wt, c = dev(cs.x), dev(cs.wt), dev(cs.c)
    y, idx = rmm.select_linear(x, c, 0.5, wt)   # warm: workspace allocated
    torch.cuda.synchronize()
    ref_y, ref_i = y.clone(), idx.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rmm.select_linear(x, c, 0.5, wt, out=y, idx=idx)
    for _ in range(4):
        y.zero_()
        idx.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref_y) and torch.equal(idx, ref_i)
        rmm.select_linear(x, c, 0.25, wt)  # eager work on the same workspace between replays
        torch.cuda.synchronize()
