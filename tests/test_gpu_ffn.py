"""GPU parity of the gated FFN producer (rmm_gate_up) and of the decode FFN
chain it feeds (rmm_gate_up -> rmm_select on the producer's tile maxima ->
rmm_linear over the down projection), against the oracle, through the C ABI.

The producer accumulates in fp32 and the oracle in double, and both round
silu(g)*u to bfloat16, so h may differ where the exact value lies within the
fp32 error of a rounding boundary.  Bars, all derived from the arithmetic:
 - h: every element within E + half a bfloat16 ulp of the oracle's exact
   silu(g)*u, where E is the first-order fp32 bound of the accumulations
   (H*2^-24 times the sums of |x*w|) carried through silu (|silu'| <= 1.1)
   and the product, plus a few fp32 roundings; at least 99% of h bit-exact;
 - pmax: exactly the tile maxima of |h| the GPU wrote, and within the h bound
   of the oracle's;
 - kept slices: may differ from the oracle's only at slices whose oracle score
   lies within twice the largest score perturbation of the k-th score;
 - y: every element within the bound the h differences, the differing slices
   and fp32 accumulation give.
"""
import numpy as np
import pytest
import torch

import input_adaptive_reduced_score_amd as rmm
import oracle
import workloads as W
from _util import dev

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def f64(a):
    return W.bf16_bits_to_f32(a).astype(np.float64)


def bf16_ulp(a):
    a = np.abs(a)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(int)
    return np.ldexp(1.0, np.maximum(e - 7, -133))


def h_bound(x, wg, wu, hd):
    """Per-element bound on |h_gpu - exact silu(g)*u| (see module docstring)."""
    xf, gf, uf = f64(x), f64(wg), f64(wu)
    H = xf.shape[1]
    g, u = xf @ gf, xf @ uf
    eg = 1.01 * H * U32 * (np.abs(xf) @ np.abs(gf))
    eu = 1.01 * H * U32 * (np.abs(xf) @ np.abs(uf))
    sil = g / (1.0 + np.exp(-g))
    ev = 1.1 * eg * (np.abs(u) + eu) + (np.abs(sil) + 1.1 * eg) * eu + 8 * U32 * np.abs(hd) + 1e-37
    return ev + 0.5 * bf16_ulp(np.abs(hd) + ev)


def gpu_gate_up(cs, tile, ldx=None, ldw=None, ldh=None):
    T, H, Mi = cs.T, cs.H, cs.Mi
    print(f"[case] gate_up T={T} H={H} Mi={Mi} tile={tile} ldx={ldx} ldw={ldw} ldh={ldh}", flush=True)

    def padded(a, ld, fill=0x7FC0):
        if ld is None:
            ld = -(-a.shape[1] // 8) * 8  # the library's layout rule: pitch a multiple of 8 elements
        if ld == a.shape[1]:
            return dev(a)
        buf = np.full((a.shape[0], ld), fill, np.uint16)  # NaN padding must never be read
        buf[:, :a.shape[1]] = a
        return dev(buf)[:, :a.shape[1]]

    x = padded(cs.x, ldx)
    wg = padded(cs.wg, ldw)
    wu = padded(cs.wu, ldw)
    h = None
    if ldh is not None:
        h = torch.full((T, ldh), float("nan"), dtype=torch.bfloat16, device="cuda:0")[:, :Mi]
    h, pmax = rmm.gate_up(x, wg, wu, tile=tile, h=h)
    torch.cuda.synchronize()
    return h.contiguous().view(torch.int16).cpu().numpy().view(np.uint16), pmax.cpu().numpy()


def check_gate_up(cs, tile, **kw):
    hg, pg = gpu_gate_up(cs, tile, **kw)
    ho, po, hd = oracle.gate_up(cs.x, cs.wg, cs.wu, tile)
    bound = h_bound(cs.x, cs.wg, cs.wu, hd)
    err = np.abs(f64(hg) - hd)
    assert np.all(err <= bound), f"h outside the bound at {np.argwhere(err > bound)[:4]}"
    exact = float(np.mean(hg == ho))
    assert exact >= 0.99, f"only {exact:.4f} of h bit-exact"
    # pmax: the GPU's tile maxima of its own |h|, and close to the oracle's
    T = cs.T
    want = np.stack([np.abs(W.bf16_bits_to_f32(hg[t0:t0 + tile])).max(axis=0) for t0 in range(0, T, tile)])
    assert np.array_equal(pg, want)
    pb = np.stack([bound[t0:t0 + tile].max(axis=0) for t0 in range(0, T, tile)])
    assert np.all(np.abs(pg.astype(np.float64) - po) <= pb)
    return hg, pg, ho, po, hd, exact


@pytest.mark.parametrize("T,H,Mi,tile", [(1, 64, 40, 1), (3, 200, 1000, 2), (8, 512, 520, 8), (13, 1000, 777, 4),
                                         (20, 96, 513, 16), (5, 64, 64, 64), (2, 8, 8, 1)])
def test_gate_up_shapes(T, H, Mi, tile):
    cs = W.ffn_case(T, H, Mi, tile, seed=T + H, wsigma=0.1)
    check_gate_up(cs, tile)


def test_gate_up_strided():
    cs = W.ffn_case(4, 256, 600, 2, seed=3, wsigma=0.1)
    check_gate_up(cs, 2, ldx=264, ldw=616, ldh=611)


def test_gate_up_decode_full_size():
    cs = W.ffn_case()
    _, _, _, _, _, exact = check_gate_up(cs, 1)
    print(f"h bit-exact fraction {exact:.5f}")


def test_gate_up_deterministic():
    cs = W.ffn_case(2, 1024, 2048, 2, seed=9)
    a = gpu_gate_up(cs, 2)
    b = gpu_gate_up(cs, 2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_select_on_tile_maxima_equals_select_on_h():
    # the producer's maxima stand in for h in the scorer: the same slices are kept
    cs = W.ffn_case(16, 512, 3000, 8, seed=4, wsigma=0.05)
    x, wg, wu, c = dev(cs.x), dev(cs.wg), dev(cs.wu), dev(cs.c)
    h, pmax = rmm.gate_up(x, wg, wu, tile=8)
    for r in (0.1, 0.5, 0.9):
        a = rmm.select(h, c, 8, r)
        b = rmm.select(pmax, c, 1, r)
        torch.cuda.synchronize()
        assert torch.equal(a, b), r


@pytest.mark.parametrize("r", [0.25, 0.5])
def test_ffn_decode_chain_full_size(r):
    cs = W.ffn_case()
    hg, pg, ho, po, hd, _ = check_gate_up(cs, 1)
    x, wg, wu, wd, c = dev(cs.x), dev(cs.wg), dev(cs.wu), dev(cs.wd), dev(cs.c)
    h, pmax = rmm.gate_up(x, wg, wu, tile=1)
    idx = rmm.select(pmax, c, 1, r)
    y = rmm.linear(h, wd, idx, 1)
    torch.cuda.synchronize()
    ig = idx.cpu().numpy()[0]
    io = oracle.select(ho, cs.c, 1, r)[0]
    yo = oracle.linear(ho, cs.wd, io[None], 1)
    # kept slices: differences only within twice the largest score perturbation of the k-th score
    so = oracle.scores(ho, cs.c, 1)[0].astype(np.float64)
    sg = (np.abs(W.bf16_bits_to_f32(hg[0])) * cs.c).astype(np.float32).astype(np.float64)
    D = np.max(np.abs(sg - so))
    kth = so[io].min()
    diff = np.setxor1d(ig, io)
    assert np.all(np.abs(so[diff] - kth) <= 2 * D * (1 + 1e-6)), diff[:8]
    # y: elementwise bound from the h differences, the differing slices and fp32 accumulation
    hgf, hof, wdf = f64(hg[0]), f64(ho[0]), f64(cs.wd)
    both = np.intersect1d(ig, io)
    only_g, only_o = np.setdiff1d(ig, io), np.setdiff1d(io, ig)
    aw = np.abs(wdf)
    bound = (np.abs(hgf[both] - hof[both]) @ aw[both] + np.abs(hgf[only_g]) @ aw[only_g]
             + np.abs(hof[only_o]) @ aw[only_o] + 1.01 * len(ig) * U32 * (np.abs(hgf[ig]) @ aw[ig])
             + U32 * np.abs(yo[0]))
    yg = y.cpu().numpy()[0].astype(np.float64)
    assert np.all(np.abs(yg - yo[0]) <= bound)
    print(f"r={r}: {len(diff)} differing slices, y rel-L2 "
          f"{np.linalg.norm(yg - yo[0]) / np.linalg.norm(yo[0]):.2e}")
