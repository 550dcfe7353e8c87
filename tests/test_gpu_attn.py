"""GPU parity of the reduced attention decode (rmm_attn_decode) and the dense
baseline (rmm_attn_decode_dense) against the oracle, through the C ABI.

Bars: head_dim index sets bit-exact; key-position sets may differ from the
oracle's only at positions whose oracle score is within 1e-6 relative of the
k-th score; out within rel-L2 2e-2 (bf16 inputs), and within 1e-5 whenever the
position sets agree exactly (fp32 accumulation of exact products); lse within
1e-6 relative.
"""
import numpy as np
import pytest
import torch

import input_adaptive_reduced_score_amd as rmm
import oracle
import workloads as W
from _util import check_near_tie_sets, dev, rel_l2

pytestmark = pytest.mark.gpu


def padded_keys(kt):
    """Keys in a cache whose row pitch ldk is a multiple of 8 positions (the
    library's layout rule); the tail holds +inf, which must never be read."""
    S = kt.shape[3]
    ldk = -(-S // 8) * 8
    if ldk == S:
        return kt
    out = np.full(kt.shape[:3] + (ldk,), 0x7f80, np.uint16)
    out[..., :S] = kt
    return out


def run_attn(cs, r_dim, r_pos, mode=0, kt=None, v=None, S=None, vn=None):
    kt = cs.kt if kt is None else kt
    v = cs.v if v is None else v
    if S is None:
        S = cs.S
    kt = padded_keys(kt)
    print(f"[case] {cs.name} r_dim={r_dim} r_pos={r_pos} mode={mode} vn={vn is not None}", flush=True)
    out, dim_idx, pos_idx, lse = rmm.attn_decode(dev(cs.q), dev(kt), dev(v), dev(cs.kn), r_dim, r_pos,
                                                 scale=cs.scale, mode=mode, S=S,
                                                 vn=None if vn is None else dev(vn))
    torch.cuda.synchronize()
    ref = oracle.attn_decode(cs.q, kt, v, cs.kn, cs.scale, r_dim, r_pos, mode, S=S, want=("pi",), vn=vn)
    assert np.array_equal(dim_idx.cpu().numpy(), ref["dim_idx"]), "head_dim selections differ"
    B, Hsel = ref["pos_idx"].shape[:2]
    gi = pos_idx.cpu().numpy().reshape(B * Hsel, -1)
    oi = ref["pos_idx"].reshape(B * Hsel, -1)
    ndiff = check_near_tie_sets(gi, oi, ref["pi"].reshape(B * Hsel, -1))
    err = rel_l2(out.cpu().numpy(), ref["out"])
    assert err <= 2e-2, f"out rel-L2 {err:.3e}"
    if ndiff == 0:
        assert err <= 1e-5, f"out rel-L2 {err:.3e} with identical position sets"
    lg, lr = lse.cpu().numpy(), ref["lse"]
    assert np.max(np.abs(lg - lr) / np.abs(lr)) <= 1e-6
    run_attn.last_out = out
    return ndiff, err


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("r_dim,r_pos", [(0.5, 0.5), (0.25, 0.25), (1.0, 1.0), (0.75, 0.1), (1 / 128, 1e-3)])
def test_small_gqa(mode, r_dim, r_pos):
    cs = W.attn_case(2, 1000, Hq=8, Hkv=2, seed=1, n_hot=8)
    run_attn(cs, r_dim, r_pos, mode)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 2), (4, 2)])
def test_group_sizes(Hq, Hkv):
    cs = W.attn_case(1, 777, Hq=Hq, Hkv=Hkv, seed=2, n_hot=4)
    run_attn(cs, 0.5, 0.25, 0)
    run_attn(cs, 0.5, 0.25, 1)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("S", [1, 7, 8, 513, 4095, 9999])
def test_ragged_lengths(S, mode):
    cs = W.attn_case(1, S, Hq=4, Hkv=1, seed=S, n_hot=min(4, S))
    run_attn(cs, 0.5, 0.3, mode)


@pytest.mark.parametrize("mode", [0, 1])
def test_cache_with_spare_capacity(mode):
    # ldk/ldv larger than S: the kernels must read positions < S only
    cs = W.attn_case(1, 1000, Hq=8, Hkv=2, seed=3, n_hot=4)
    kt = np.full((1, 2, 128, 1032), 0x7f80, np.uint16)  # +inf beyond S
    kt[..., :1000] = cs.kt
    v = np.full((1, 2, 1100, 128), 0x7f80, np.uint16)
    v[:, :, :1000] = cs.v
    run_attn(cs, 0.5, 0.5, mode, kt=kt, v=v, S=1000)


def test_all_equal_logits_take_lowest_positions():
    # zero keys: every logit is 0 and every position ties; more ties than the
    # candidate buffer holds, so the selector's generic radix path runs
    cs = W.attn_case(1, 20000, Hq=4, Hkv=1, seed=4, n_hot=1)
    kt = np.zeros_like(cs.kt)
    cs.kn[:] = 0.0
    ndiff, _ = run_attn(cs, 0.5, 0.25, 0, kt=kt)
    assert ndiff == 0


@pytest.mark.parametrize("r", [0.25, 0.5])
def test_gqa_32k_full_size(r):
    cs = W.attn_32k()
    run_attn(cs, r, r, 0)


@pytest.mark.parametrize("seed", [1, 2])
def test_gqa_32k_other_seeds(seed):
    run_attn(W.attn_32k(seed=seed), 0.25, 0.25, 0)


def test_gqa_128k_batch4_full_size():
    cs = W.attn_128k()
    run_attn(cs, 0.5, 0.25, 0)


@pytest.mark.parametrize("S", [8192, 65536, 262144])
def test_one_sequence_context_lengths(S):
    # the lengths of the benchmark's context sweep beyond 32K (one sequence, 8 groups; up to 256K
    # positions the launches are split as at 128K x 4)
    run_attn(W.attn_case(1, S, seed=21), 0.25, 0.25, 0)


def test_gqa_32k_per_query_head():
    # mode 1 at the full 32K shape: 32 selection groups of one query head
    run_attn(W.attn_32k(), 0.25, 0.25, 1)


def test_gqa_128k_batch4_per_query_head():
    # mode 1 at 128K x 4: 128 selection groups over 131072 positions each
    run_attn(W.attn_128k(), 0.5, 0.25, 1)


@pytest.mark.parametrize("r", [0.25, 0.5])
def test_gqa_32k_without_optional_outputs(r):
    # the call as the benchmark times it: dim_idx, pos_idx and lse not requested (NULL).  Its
    # output must equal, bit for bit, the output of the same call with every output requested,
    # and that one is checked against the oracle (position sets, out, lse)
    cs = W.attn_32k()
    print(f"[case] {cs.name} r={r} NULL optional outputs", flush=True)
    out0, d0, p0, l0 = rmm.attn_decode(dev(cs.q), dev(cs.kt), dev(cs.v), dev(cs.kn), r, r, scale=cs.scale,
                                       want_idx=False)
    torch.cuda.synchronize()
    assert d0 is None and p0 is None and l0 is None
    ndiff, err = run_attn(cs, r, r, 0)
    assert torch.equal(out0, run_attn.last_out)
    ref = oracle.attn_decode(cs.q, cs.kt, cs.v, cs.kn, cs.scale, r, r, 0)
    e0 = rel_l2(out0.cpu().numpy(), ref["out"])
    assert e0 <= (1e-5 if ndiff == 0 else 2e-2), f"NULL-output call: out rel-L2 {e0:.3e}"


@pytest.mark.parametrize("B,S,Hq,Hkv", [(1, 32768, 32, 8), (2, 1000, 8, 2), (1, 77, 8, 1)])
def test_dense_attention(B, S, Hq, Hkv):
    cs = W.attn_case(B, S, Hq=Hq, Hkv=Hkv, seed=6, n_hot=min(8, S))
    out, lse = rmm.attn_decode_dense(dev(cs.q), dev(padded_keys(cs.kt)), dev(cs.v), scale=cs.scale, S=S,
                                     lse=torch.empty((B, Hq), device="cuda:0"))
    torch.cuda.synchronize()
    ref = oracle.dense_attn(cs.q, cs.kt, cs.v, cs.scale)
    assert rel_l2(out.cpu().numpy(), ref) <= 1e-5


def test_deterministic_repeat():
    cs = W.attn_case(1, 32768, seed=7)
    args = (dev(cs.q), dev(cs.kt), dev(cs.v), dev(cs.kn), 0.25, 0.25)
    a = [t.clone() for t in rmm.attn_decode(*args, scale=cs.scale)]
    b = rmm.attn_decode(*args, scale=cs.scale)
    torch.cuda.synchronize()
    for u, w in zip(a, b):
        assert torch.equal(u, w)


# ---- position score weighted by the value-row norm (p * ||V_s||)

@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("r_dim,r_pos", [(0.5, 0.5), (0.25, 0.1), (1.0, 1.0), (1 / 128, 1e-3)])
def test_value_norm_small_gqa(mode, r_dim, r_pos):
    cs = W.attn_case(2, 1000, Hq=8, Hkv=2, seed=11, n_hot=8)
    run_attn(cs, r_dim, r_pos, mode, vn=W.value_row_norms(cs.v))


def test_value_norm_changes_the_selection():
    # norms spread over four decades: the weighted set must follow the oracle's
    # weighted scores, and differ from the probability-only set
    cs = W.attn_case(1, 4000, Hq=8, Hkv=2, seed=12, n_hot=4)
    rng = np.random.default_rng(12)
    vn = (W.value_row_norms(cs.v) * 10.0 ** rng.uniform(-2, 2, size=(1, 2, 4000))).astype(np.float32)
    run_attn(cs, 0.5, 0.25, 0, vn=vn)
    _, _, plain, _ = rmm.attn_decode(dev(cs.q), dev(cs.kt), dev(cs.v), dev(cs.kn), 0.5, 0.25, scale=cs.scale)
    _, _, weighted, _ = rmm.attn_decode(dev(cs.q), dev(cs.kt), dev(cs.v), dev(cs.kn), 0.5, 0.25, scale=cs.scale,
                                        vn=dev(vn))
    torch.cuda.synchronize()
    assert not torch.equal(plain, weighted)


def test_value_norm_ones_is_probability_score():
    cs = W.attn_case(1, 3000, Hq=8, Hkv=2, seed=13, n_hot=4)
    ndiff, _ = run_attn(cs, 0.5, 0.3, 1, vn=np.ones((1, 2, 3000), np.float32))
    assert ndiff == 0


@pytest.mark.parametrize("S", [7, 513, 9999])
def test_value_norm_ragged_spare_capacity(S):
    # ldv > S; the norms beyond S hold NaN and must not influence anything
    cs = W.attn_case(1, S, Hq=4, Hkv=1, seed=S + 1, n_hot=min(4, S))
    ldv = -(-S // 8) * 8 + 8
    v = np.zeros((1, 1, ldv, 128), np.uint16)
    v[:, :, :S] = cs.v
    vn = np.full((1, 1, ldv), np.nan, np.float32)
    vn[..., :S] = W.value_row_norms(cs.v)
    run_attn(cs, 0.5, 0.3, 0, v=v, S=S, vn=vn)


def test_value_norm_32k_full_size():
    cs = W.attn_32k()
    run_attn(cs, 0.25, 0.25, 0, vn=W.value_row_norms(cs.v))


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("scale,r_pos", [(4.0, 0.9), (8.0, 0.5), (8.0, 0.9), (16.0, 0.5), (16.0, 0.9)])
def test_sharp_softmax_threshold_far_below(mode, scale, r_pos):
    # sharp softmaxes: the k-th log-probability lies between -96 and -680 nats (measured with the
    # oracle), and at scale 16 in mode 1 with r_pos 0.9 the k-th probability underflows to 0 in
    # double, where every zero ties and the lowest positions win.  Positions are still ranked by
    # their scores wherever the oracle's scores differ.
    cs = W.attn_case(1, 4000, Hq=4, Hkv=1, seed=21, n_hot=4)
    cs.scale = scale
    run_attn(cs, 0.5, r_pos, mode)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("factor", [1e7, 1e-8])
def test_value_norm_far_outside_the_fine_bins(mode, factor):
    # value norms scaled so that log(p * ||V_s||) at the k-th position lies far above (x1e7: about
    # +11) or far below (x1e-8) the 1/128-nat bins of the score histogram; a half-nat bin then
    # holds hundreds of positions, ranked exactly in LDS
    cs = W.attn_case(1, 4000, Hq=8, Hkv=2, seed=23, n_hot=4)
    vn = (W.value_row_norms(cs.v) * factor).astype(np.float32)
    run_attn(cs, 0.5, 0.25, mode, vn=vn)
    run_attn(cs, 0.5, 0.9, mode, vn=vn)


@pytest.mark.parametrize("mode", [0, 1])
def test_threshold_below_histogram_window(mode):
    # a sharp softmax (scale 2): the k-th log-probability lies near -80, below the key
    # histogram's [-32, 0) window, so the selector resolves all 32 key bits by radix passes
    cs = W.attn_case(1, 4000, Hq=4, Hkv=1, seed=21, n_hot=4)
    cs.scale = 2.0
    run_attn(cs, 0.5, 0.5, mode)
    run_attn(cs, 0.25, 0.9, mode)
