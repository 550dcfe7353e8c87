"""The hot path captured in a HIP graph (as a serving loop or the benchmark
runs it) replays the eager results exactly, replay after replay, with eager
work and synchronizations in between.  The kernels enqueue no memset and the
workspace counters return to zero after every call, so replays are independent."""
import numpy as np
import pytest
import torch

import input_adaptive_reduced_score_amd as rmm
import workloads as W
from _util import dev

pytestmark = pytest.mark.gpu


def _capture(fn):
    fn()  # warm: workspace allocated, one-time attributes set
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def test_decode_select_linear_graph_replays_match_eager():
    cs = W.linear_decode()
    x, wt, c = dev(cs.x), dev(cs.wt), dev(cs.c)
    k = rmm.keep_count(cs.K, 0.25)
    idx = torch.empty((1, k), dtype=torch.int32, device="cuda:0")
    y = torch.empty((1, cs.M), dtype=torch.float32, device="cuda:0")

    def step():
        rmm.select(x, c, 1, 0.25, idx=idx)
        rmm.linear(x, wt, idx, 1, out=y)

    step()
    torch.cuda.synchronize()
    ref_idx, ref_y = idx.clone(), y.clone()
    g = _capture(step)
    for rep in range(4):
        idx.fill_(-1)
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx) and torch.equal(y, ref_y), f"replay {rep}"
        # eager work between replays, on the same workspace
        rmm.linear_dense(x[:, :4096], wt[:4096], out=torch.empty((1, cs.M), device="cuda:0"))
        torch.cuda.synchronize()


def test_prefill_graph_replays_match_eager():
    cs = W.linear_random(512, 4096, 1024, 256, "bf16", seed=2)
    x, wt, c = dev(cs.x), dev(cs.wt), dev(cs.c)
    k = rmm.keep_count(cs.K, 0.5)
    idx = torch.empty((2, k), dtype=torch.int32, device="cuda:0")
    y = torch.empty((512, cs.M), dtype=torch.float32, device="cuda:0")

    def step():
        rmm.select(x, c, 256, 0.5, idx=idx)
        rmm.linear(x, wt, idx, 256, out=y)

    step()
    torch.cuda.synchronize()
    ref = y.clone()
    g = _capture(step)
    for rep in range(3):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {rep}"


def test_attention_graph_replays_match_eager():
    cs = W.attn_case(1, 32768, seed=3)
    q, kt, v, kn = dev(cs.q), dev(cs.kt), dev(cs.v), dev(cs.kn)
    out = torch.empty((1, 32, 128), dtype=torch.float32, device="cuda:0")
    pos = torch.empty((1, 8, rmm.keep_count(32768, 0.25)), dtype=torch.int32, device="cuda:0")
    dims = torch.empty((1, 8, 32), dtype=torch.int32, device="cuda:0")
    lse = torch.empty((1, 32), dtype=torch.float32, device="cuda:0")

    def step():
        rmm.attn_decode(q, kt, v, kn, 0.25, 0.25, scale=cs.scale, out=out, dim_idx=dims, pos_idx=pos, lse=lse)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, dims, pos, lse)]
    g = _capture(step)
    for rep in range(3):
        for t in (out, lse):
            t.fill_(float("nan"))
        pos.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((out, dims, pos, lse), ref):
            assert torch.equal(a, b), f"replay {rep}"
        rmm.attn_decode_dense(q, kt, v, scale=cs.scale)
        torch.cuda.synchronize()
    assert np.isfinite(out.cpu().numpy()).all()


def test_decode_ffn_chain_graph_replays_match_eager():
    # gated producer -> selection on its tile maxima -> reduced down projection
    cs = W.ffn_case(1, 4096, 14336, 1, seed=4)
    x, wg, wu, wd, c = dev(cs.x), dev(cs.wg), dev(cs.wu), dev(cs.wd), dev(cs.c)
    h = torch.empty((1, 14336), dtype=torch.bfloat16, device="cuda:0")
    pm = torch.empty((1, 14336), dtype=torch.float32, device="cuda:0")
    idx = torch.empty((1, rmm.keep_count(14336, 0.5)), dtype=torch.int32, device="cuda:0")
    y = torch.empty((1, 4096), dtype=torch.float32, device="cuda:0")

    def step():
        rmm.gate_up(x, wg, wu, 1, h=h, pmax=pm)
        rmm.select(pm, c, 1, 0.5, idx=idx)
        rmm.linear(h, wd, idx, 1, out=y)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (h, pm, idx, y)]
    g = _capture(step)
    for rep in range(3):
        for t in (pm, y):
            t.fill_(float("nan"))
        idx.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((h, pm, idx, y), ref):
            assert torch.equal(a, b), f"replay {rep}"
        rmm.gate_up(x[:, :1024], wg[:1024], wu[:1024], 1)  # eager work on the same workspace
        torch.cuda.synchronize()


def test_paged_attention_graph_replays_match_eager():
    pc = W.attn_paged([3000, 17, 9000], page=128, Hq=8, Hkv=2, seed=5, n_hot=4)
    args = (dev(pc.q), dev(pc.k_pages), dev(pc.v_pages), dev(pc.kn), dev(pc.block_table), dev(pc.seqlens))
    out = torch.empty((3, 8, 128), dtype=torch.float32, device="cuda:0")

    def step():
        rmm.attn_decode_paged(*args, 0.5, 0.25, scale=pc.scale, S=pc.S, out=out, want_idx=False)

    step()
    torch.cuda.synchronize()
    ref = out.clone()
    g = _capture(step)
    for rep in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}"
        rmm.attn_decode_dense_paged(*args[:3], *args[4:], scale=pc.scale, S=pc.S)
        torch.cuda.synchronize()
