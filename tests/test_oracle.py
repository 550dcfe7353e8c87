"""Pins of the CPU oracle against facts other than itself (no GPU).

Each test names the passage it follows.  Pins used: exact rational closed
forms, brute force over every subset, float64 BLAS / torch float64 library
routines for the special cases that reduce to plain products and textbook
attention, and identities that must hold exactly.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W


# --------------------------------------------------------------------------- keep count
# Paper abstract: a single retention ratio r; kept count ceil(r*K).

def _exact_keep(K, r: Fraction):
    p = r * K
    n = math.floor(p + Fraction(1, 2))
    if abs(p - n) <= Fraction(1, 10**9) * max(1, p):
        k = n
    else:
        k = math.ceil(p)
    return max(1, min(K, k))


@pytest.mark.parametrize("K", list(range(1, 21)) + [127, 128, 4096, 14336, 131072])
def test_keep_count_closed_form(K):
    decimals = ["0.07", "0.1", "0.3", "0.25", "0.5", "0.75", "1", "0.001", "0.999"]
    for s in decimals:
        assert oracle.keep_count(K, float(s)) == _exact_keep(K, Fraction(s)), (K, s)
        # away from the snap band the closed form is the plain ceiling
        if (Fraction(s) * K).denominator == 1 or abs(Fraction(s) * K - round(Fraction(s) * K)) > Fraction(1, 1000):
            assert oracle.keep_count(K, float(s)) == max(1, min(K, math.ceil(Fraction(s) * K)))
    assert oracle.keep_count(K, 1.0 / 3.0) == _exact_keep(K, Fraction(1, 3))
    if K <= 20:
        for k in range(1, K + 1):
            assert oracle.keep_count(K, k / K) == k
    for bad in (0.0, -0.25, 1.5, float("nan"), float("inf")):
        assert oracle.keep_count(K, bad) == -1


def test_keep_count_configs():
    # the decode shapes keep 3584/7168/10752/14336 of 14336; head_dim 32/64 of 128
    assert [oracle.keep_count(14336, r) for r in (0.25, 0.5, 0.75, 1.0)] == [3584, 7168, 10752, 14336]
    assert [oracle.keep_count(128, r) for r in (0.25, 0.5)] == [32, 64]
    assert oracle.keep_count(32768, 0.25) == 8192 and oracle.keep_count(131072, 0.25) == 32768
    assert oracle.keep_count(100, 0.07) == 7  # 0.07*100 is 7.000000000000001 in binary


# --------------------------------------------------------------------------- scorer
# Blog section 5.1: a cheap score per slice from the current input.

def test_scorer_tile1_unit_weight_is_abs():
    cs = W.linear_random(6, 300, 8, 1, "f32", seed=3)
    s = oracle.scores(cs.x, np.ones(300, np.float32), 1)
    assert np.array_equal(s, np.abs(cs.x))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scorer_max_then_scale_equals_scale_then_max(dtype):
    # rounding is monotone and c >= 0, so fl(max|x| * c) == max fl(|x| * c) (numpy float32 ops)
    cs = W.linear_random(10, 257, 8, 4, dtype, seed=5)
    s = oracle.scores(cs.x, cs.c, 4)
    xf = W.bf16_bits_to_f32(cs.x) if dtype == "bf16" else cs.x
    for tau in range(3):
        blk = np.abs(xf[4 * tau:4 * tau + 4]) * cs.c[None, :]
        assert np.array_equal(s[tau], blk.max(axis=0))


def test_scorer_is_token_order_independent():
    cs = W.linear_random(8, 100, 8, 8, "bf16", seed=7)
    perm = np.random.default_rng(1).permutation(8)
    assert np.array_equal(oracle.scores(cs.x, cs.c, 8), oracle.scores(cs.x[perm], cs.c, 8))


def test_scorer_single_token_column():
    # only one token of the tile is non-zero in column j: the score is exactly |x|*c
    x = np.zeros((4, 5), np.float32)
    x[2, 0], x[0, 1], x[3, 2], x[1, 4] = -3.0, 0.5, 1e-30, 7.25
    c = np.array([2.0, 0.1, 3.0, 5.0, 0.0], np.float32)
    s = oracle.scores(x, c, 4)[0]
    exp = np.array([6.0, np.float32(0.5) * np.float32(0.1), np.float32(1e-30) * np.float32(3.0), 0.0, 0.0],
                   np.float32)
    assert np.array_equal(s, exp)


# --------------------------------------------------------------------------- selector
# Blog sections 5.2 / 6.1: top-k, kept indices sorted ascending.  Brute force:
# the kept set maximises the score sum; among maximisers, the lexicographically
# smallest ascending index list (ties go to the lower index).

def _exact_ints(vals):
    fr = [Fraction(float(v)) for v in vals]
    den = math.lcm(*[f.denominator for f in fr])
    return [int(f * den) for f in fr]


def _brute_topk(scores, k):
    ints = _exact_ints(scores)
    best, best_set = None, None
    for comb in itertools.combinations(range(len(scores)), k):  # lexicographic order
        tot = sum(ints[i] for i in comb)
        if best is None or tot > best:
            best, best_set = tot, comb
    return list(best_set)


def _tie_case(seed, T=4, K=12):
    rng = np.random.default_rng(seed)
    x = rng.integers(-3, 4, size=(T, K)).astype(np.float32)
    return x, np.ones(K, np.float32)


@pytest.mark.parametrize("tile", [4, 2, 3])
def test_select_brute_force_random(tile):
    for seed in range(40):
        cs = W.linear_random(4, 12, 8, tile, "f32", seed=seed, wsigma=0.05)
        s = oracle.scores(cs.x, cs.c, tile)
        for k in range(1, 13):
            idx = oracle.select(cs.x, cs.c, tile, k / 12)
            assert idx.shape == (s.shape[0], k)
            for tau in range(s.shape[0]):
                assert list(idx[tau]) == _brute_topk(s[tau], k), (seed, k, tau)


def test_select_brute_force_ties():
    for seed in range(120):
        x, c = _tie_case(seed)
        s = oracle.scores(x, c, 4)
        for k in range(1, 13):
            idx = oracle.select(x, c, 4, k / 12)
            assert list(idx[0]) == _brute_topk(s[0], k), (seed, k)


def test_select_all_equal_keeps_lowest():
    x = np.ones((1, 50), np.float32)
    c = np.ones(50, np.float32)
    assert list(oracle.select(x, c, 1, 0.2)[0]) == list(range(10))
    # negative zero ranks with +0: zero scores keep the lowest indices
    x = np.zeros((1, 8), np.float32)
    c = np.array([0, 0, 0, 0, 1, 1, 1, 1], np.float32)
    x[0, 4:] = 1.0
    x[0, 0] = -0.0
    assert list(oracle.select(x, c, 1, 6 / 8)[0]) == [0, 1, 4, 5, 6, 7]


@pytest.mark.parametrize("case", ["tiny", "ragged"])
def test_select_count_and_order(case):
    cs = W.linear_tiny() if case == "tiny" else W.linear_random(37, 300, 16, 8, "bf16", seed=2)
    for r in (0.1, 0.25, 0.5, 1 / 3, 0.75, 1.0):
        idx = oracle.select(cs.x, cs.c, cs.tile, r)
        k = oracle.keep_count(cs.K, r)
        assert idx.shape == (-(-cs.T // cs.tile), k)
        assert np.all(np.diff(idx, axis=1) > 0) and idx.min() >= 0 and idx.max() < cs.K


# --------------------------------------------------------------------------- products
# Blog section 2 (Y = X @ W^T) and 6.1 (keep ratio 1.0 equals the full result).

def _f64(a, dtype):
    return (W.bf16_bits_to_f32(a) if dtype == "bf16" else a).astype(np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_linear_r1_equals_dense(dtype):
    cs = W.linear_random(5, 96, 40, 2, dtype, seed=11)
    idx = oracle.select(cs.x, cs.c, 2, 1.0)
    y, yd = oracle.linear(cs.x, cs.wt, idx, 2, want_double=True)
    yf, yfd = oracle.dense_linear(cs.x, cs.wt, want_double=True)
    assert np.array_equal(y, yf) and np.array_equal(yd, yfd)  # same order, bitwise
    ref = _f64(cs.x, dtype) @ _f64(cs.wt, dtype)  # float64 BLAS (different summation order)
    assert np.max(np.abs(yfd - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("dtype,tile", [("f32", 4), ("f32", 2), ("bf16", 3)])
def test_linear_dropped_slice_identity(dtype, tile):
    # Y_full - Y_red = X[:, dropped] @ W^T[dropped, :]   (per tile's own dropped set)
    cs = W.linear_random(7, 64, 24, tile, dtype, seed=13)
    xd, wd = _f64(cs.x, dtype), _f64(cs.wt, dtype)
    _, yfull = oracle.dense_linear(cs.x, cs.wt, want_double=True)
    for r in (0.25, 0.5, 0.75):
        idx = oracle.select(cs.x, cs.c, tile, r)
        _, yred = oracle.linear(cs.x, cs.wt, idx, tile, want_double=True)
        for t in range(cs.T):
            keep = set(idx[t // tile].tolist())
            drop = [j for j in range(cs.K) if j not in keep]
            rhs = xd[t, drop] @ wd[drop, :]
            assert np.max(np.abs((yfull[t] - yred[t]) - rhs)) <= 1e-12 * np.max(np.abs(yfull)), (r, t)


def test_linear_row_subset_matches_full():
    cs = W.linear_random(9, 80, 30, 4, "bf16", seed=17)
    idx = oracle.select(cs.x, cs.c, 4, 0.5)
    full = oracle.linear(cs.x, cs.wt, idx, 4)
    part = oracle.linear(cs.x, cs.wt, idx, 4, rows=(3, 7))
    assert np.array_equal(full[3:7], part[3:7]) and not part[:3].any() and not part[7:].any()


# --------------------------------------------------------------------------- attention
# Blog sections 3.1 / 3.3; GEMM notes section 1 (scores = Q K^T, softmax, @ V).

def _qkv_f64(cs):
    q = W.bf16_bits_to_f32(cs.q).astype(np.float64)
    kt = W.bf16_bits_to_f32(cs.kt).astype(np.float64)
    v = W.bf16_bits_to_f32(cs.v).astype(np.float64)
    return q, kt, v


def _sdpa64(q, k, v, scale):
    # q [Hq, d], k [S, d], v [S, D] float64 -> torch's float64 SDPA
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(np.ascontiguousarray(k))[None, None].expand(1, q.shape[0], *k.shape),
        torch.from_numpy(np.ascontiguousarray(v))[None, None].expand(1, q.shape[0], *v.shape), scale=scale)
    return out[0, :, 0, :].numpy()


@pytest.mark.parametrize("mode", [0, 1])
def test_attn_full_ratios_equal_textbook(mode):
    cs = W.attn_case(2, 40, Hq=4, Hkv=2, D=16, seed=1, n_hot=3)
    res = oracle.attn_decode(cs.q, cs.kt, cs.v, cs.kn, cs.scale, 1.0, 1.0, mode, want=("out_d", "p"))
    dense = oracle.dense_attn(cs.q, cs.kt, cs.v, cs.scale)
    q, kt, v = _qkv_f64(cs)
    for b in range(2):
        for g in range(2):
            ref = _sdpa64(q[b, 2 * g:2 * g + 2], kt[b, g].T, v[b, g], cs.scale)
            assert np.max(np.abs(res["out_d"][b, 2 * g:2 * g + 2] - ref)) <= 1e-12 * np.max(np.abs(ref))
            assert np.max(np.abs(dense[b, 2 * g:2 * g + 2] - ref)) <= 1e-12 * np.max(np.abs(ref))
    assert np.max(np.abs(res["p"].sum(axis=2) - 1.0)) <= 1e-12


@pytest.mark.parametrize("mode", [0, 1])
def test_attn_reduced_dims_equal_sliced_textbook(mode):
    # with every position kept, the result is textbook attention over the kept head_dim slices
    # (scale stays 1/sqrt(full D)); lse matches torch.logsumexp of the sliced logits
    cs = W.attn_case(1, 64, Hq=4, Hkv=1, D=32, seed=2, n_hot=4)
    res = oracle.attn_decode(cs.q, cs.kt, cs.v, cs.kn, cs.scale, 0.25, 1.0, mode, want=("out_d",))
    q, kt, v = _qkv_f64(cs)
    for h in range(4):
        sel = res["dim_idx"][0, 0 if mode == 0 else h]
        ref = _sdpa64(q[0][h:h + 1][:, sel], kt[0, 0][sel].T, v[0, 0], cs.scale)
        assert np.max(np.abs(res["out_d"][0, h] - ref[0])) <= 1e-12 * np.max(np.abs(ref))
        logits = torch.from_numpy(cs.scale * (q[0, h, sel] @ kt[0, 0][sel]))
        assert abs(float(torch.logsumexp(logits, 0)) - float(res["lse"][0, h])) <= 2e-6 * abs(float(res["lse"][0, h]))


@pytest.mark.parametrize("mode", [0, 1])
def test_attn_dropped_position_identity(mode):
    cs = W.attn_case(2, 50, Hq=8, Hkv=2, D=16, seed=3, n_hot=5)
    _, _, v = _qkv_f64(cs)
    full = oracle.attn_decode(cs.q, cs.kt, cs.v, cs.kn, cs.scale, 0.5, 1.0, mode, want=("out_d", "p"))
    for r_pos in (0.1, 0.25, 0.5, 0.9):
        red = oracle.attn_decode(cs.q, cs.kt, cs.v, cs.kn, cs.scale, 0.5, r_pos, mode, want=("out_d", "p"))
        assert np.array_equal(red["dim_idx"], full["dim_idx"])
        G = 4
        for b in range(2):
            for h in range(8):
                sg = h // G if mode == 0 else h
                keep = set(red["pos_idx"][b, sg].tolist())
                drop = [s for s in range(50) if s not in keep]
                rhs = full["p"][b, h, drop] @ v[b, h // G][drop]
                lhs = full["out_d"][b, h] - red["out_d"][b, h]
                assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(full["out_d"][b, h]))
                assert full["p"][b, h, sorted(keep)].sum() <= 1.0 + 1e-12


def _dim_scores(cs, b, heads, g):
    qa = np.abs(W.bf16_bits_to_f32(cs.q[b, heads])).max(axis=0)
    return qa * cs.kn[b, g]  # float32 multiply, as the definition


@pytest.mark.parametrize("mode", [0, 1])
def test_attn_selections_brute_force(mode):
    for seed in range(12):
        cs = W.attn_case(1, 12, Hq=4, Hkv=1, D=12, seed=seed, n_hot=2)
        for kd in range(1, 13, 3):
            for ks in range(1, 13):
                res = oracle.attn_decode(cs.q, cs.kt, cs.v, cs.kn, cs.scale, kd / 12, ks / 12, mode,
                                         want=("pi", "p"))
                groups = [[0, 1, 2, 3]] if mode == 0 else [[h] for h in range(4)]
                for sg, heads in enumerate(groups):
                    sig = _dim_scores(cs, 0, heads, 0)
                    assert list(res["dim_idx"][0, sg]) == _brute_topk(sig, kd)
                    pi = res["pi"][0, sg]
                    assert np.array_equal(pi, res["p"][0, heads].max(axis=0))
                    assert list(res["pos_idx"][0, sg]) == _brute_topk(pi, ks)


def test_attn_mode1_equals_mode0_without_grouping():
    cs = W.attn_case(1, 30, Hq=2, Hkv=2, D=16, seed=4, n_hot=2)
    a = oracle.attn_decode(cs.q, cs.kt, cs.v, cs.kn, cs.scale, 0.5, 0.5, 0)
    b = oracle.attn_decode(cs.q, cs.kt, cs.v, cs.kn, cs.scale, 0.5, 0.5, 1)
    for key in ("out", "dim_idx", "pos_idx", "lse"):
        assert np.array_equal(a[key], b[key])


def test_attn_strided_cache_equals_packed():
    # ldk/ldv larger than S (a cache with spare capacity) gives the same result as packed buffers
    cs = W.attn_case(1, 40, Hq=4, Hkv=2, D=16, seed=6, n_hot=3)
    ktp = np.zeros((1, 2, 16, 64), np.uint16)
    ktp[..., :40] = cs.kt
    vp = np.zeros((1, 2, 56, 16), np.uint16)
    vp[:, :, :40] = cs.v
    a = oracle.attn_decode(cs.q, cs.kt, cs.v, cs.kn, cs.scale, 0.5, 0.25, 0)
    b = oracle.attn_decode(cs.q, ktp, vp, cs.kn, cs.scale, 0.5, 0.25, 0, S=40)
    for key in ("out", "dim_idx", "pos_idx", "lse"):
        assert np.array_equal(a[key], b[key])


# ---------------------------------------------------------------- block-granular variant
# Blog section 6.1 demo (ffn_block_reduce): block-mean |h| scores, keep_num =
# max(1, int(num_blocks * keep_ratio)), top blocks re-sorted ascending, expanded.

def test_block_select_hand_example():
    # block means (1+3)/2 = 2, 0, 2, (5+0)/2 = 2.5; keep 2 of 4: block 3, then the
    # lower of the tied blocks 0 and 2
    x = np.array([[1, -3, 0, 0, 2, 2, -5, 0]], np.float32)
    assert list(oracle.select_blocks(x, 1, 2, 0.5)[0]) == [0, 1, 6, 7]


@pytest.mark.parametrize("nb,keep,want", [(64, 0.5, 32), (10, 0.01, 1), (100, 0.29, 28), (7, 1.0, 7),
                                          (3, 0.5, 1), (4, 0.75, 3)])
def test_block_keep_count_truncates(nb, keep, want):
    # int() of the double product, as the demo code writes it (100 * 0.29 = 28.999999999999996)
    assert oracle.block_keep_count(nb, keep) == want


def test_block_keep_count_rejects_bad_ratio():
    assert oracle.block_keep_count(8, 0.0) == -1
    assert oracle.block_keep_count(8, 1.5) == -1


def _brute_blocks(m, block, nk):
    """Exact rational block means; the lexicographically first maximising set."""
    nb = len(m) // block
    fr = [Fraction(float(v)) for v in m]
    means = [sum(fr[b * block:(b + 1) * block]) / block for b in range(nb)]
    best, best_set = None, None
    for comb in itertools.combinations(range(nb), nk):
        tot = sum(means[b] for b in comb)
        if best is None or tot > best:
            best, best_set = tot, comb
    return [b * block + e for b in best_set for e in range(block)]


@pytest.mark.parametrize("block", [1, 2, 3, 4, 6])
def test_block_select_brute_force(block):
    K = 12
    nb = K // block
    for seed in range(25):
        rng = np.random.default_rng(seed)
        T, tile = (3, 3) if seed % 2 else (4, 2)
        if seed % 3 == 0:
            x = rng.integers(-2, 3, size=(T, K)).astype(np.float32)  # many tied block means
        else:
            x = rng.standard_normal((T, K)).astype(np.float32)
        colmax = [np.abs(x[t0:t0 + tile]).max(axis=0) for t0 in range(0, T, tile)]
        for nk in range(1, nb + 1):
            keep = nk / nb
            assert oracle.block_keep_count(nb, keep) == nk
            idx = oracle.select_blocks(x, tile, block, keep)
            for tau, m in enumerate(colmax):
                assert list(idx[tau]) == _brute_blocks(m, block, nk), (block, seed, nk, tau)


def test_block1_equals_slice_selector_with_unit_weights():
    # block = 1 scores |x| exactly as the slice scorer with c = 1; with r*K an exact
    # integer both counts agree, so the index sets must be identical
    K = 64
    for seed in range(10):
        rng = np.random.default_rng(100 + seed)
        x = rng.standard_normal((2, K)).astype(np.float32)
        for k in (1, 16, 32, 63, 64):
            a = oracle.select_blocks(x, 2, 1, k / K)
            b = oracle.select(x, np.ones(K, np.float32), 2, k / K)
            assert np.array_equal(a, b), (seed, k)


# ---------------------------------------------------------------- value-norm-weighted position score
# The analogue of the linear scorer for positions: p_h[s] * ||V[s,:]|| (max over the group's heads).

@pytest.mark.parametrize("mode", [0, 1])
def test_attn_vn_ones_equals_probability_score(mode):
    cs = W.attn_case(1, 50, Hq=4, Hkv=2, D=16, seed=8, n_hot=3)
    ones = np.ones((1, 2, 50), np.float32)
    a = oracle.attn_decode(cs.q, cs.kt, cs.v, cs.kn, cs.scale, 0.5, 0.3, mode)
    b = oracle.attn_decode(cs.q, cs.kt, cs.v, cs.kn, cs.scale, 0.5, 0.3, mode, vn=ones)
    for key in ("out", "dim_idx", "pos_idx", "lse"):
        assert np.array_equal(a[key], b[key])


@pytest.mark.parametrize("mode", [0, 1])
def test_attn_vn_brute_force(mode):
    for seed in range(10):
        cs = W.attn_case(1, 12, Hq=4, Hkv=1, D=12, seed=seed, n_hot=2)
        vn = W.value_row_norms(cs.v)
        for ks in range(1, 13):
            res = oracle.attn_decode(cs.q, cs.kt, cs.v, cs.kn, cs.scale, 0.5, ks / 12, mode, want=("pi", "p"),
                                     vn=vn)
            groups = [[0, 1, 2, 3]] if mode == 0 else [[h] for h in range(4)]
            for sg, heads in enumerate(groups):
                want = res["p"][0, heads].max(axis=0) * vn[0, 0].astype(np.float64)
                assert np.array_equal(res["pi"][0, sg], want)
                assert list(res["pos_idx"][0, sg]) == _brute_topk(want, ks)


def test_attn_vn_scale_invariant():
    cs = W.attn_case(1, 64, Hq=4, Hkv=2, D=16, seed=9, n_hot=4)
    vn = W.value_row_norms(cs.v)
    a = oracle.attn_decode(cs.q, cs.kt, cs.v, cs.kn, cs.scale, 0.5, 0.25, 0, vn=vn)
    b = oracle.attn_decode(cs.q, cs.kt, cs.v, cs.kn, cs.scale, 0.5, 0.25, 0, vn=vn * np.float32(8.0))
    assert np.array_equal(a["pos_idx"], b["pos_idx"]) and np.array_equal(a["out"], b["out"])


def test_attn_vn_strided_equals_packed():
    cs = W.attn_case(1, 40, Hq=4, Hkv=2, D=16, seed=6, n_hot=3)
    rng = np.random.default_rng(1)
    vn = rng.uniform(0.5, 2.0, size=(1, 2, 40)).astype(np.float32)
    ktp = np.zeros((1, 2, 16, 64), np.uint16)
    ktp[..., :40] = cs.kt
    vp = np.zeros((1, 2, 56, 16), np.uint16)
    vp[:, :, :40] = cs.v
    vnp = np.full((1, 2, 56), 100.0, np.float32)  # spare capacity: must never be read
    vnp[:, :, :40] = vn
    a = oracle.attn_decode(cs.q, cs.kt, cs.v, cs.kn, cs.scale, 0.5, 0.25, 0, vn=vn)
    b = oracle.attn_decode(cs.q, ktp, vp, cs.kn, cs.scale, 0.5, 0.25, 0, S=40, vn=vnp)
    for key in ("out", "dim_idx", "pos_idx", "lse"):
        assert np.array_equal(a[key], b[key])


# --------------------------------------------------------------------------- gated FFN producer
# Blog section 6.1 demo code (ffn_full): gate = x W_gate^T, up = x W_up^T,
# h = silu(gate) * up; section 5.1 scores the down projection from h.

def _bf16_bits(vals):
    """float values that are exactly bfloat16 -> uint16 bit patterns."""
    u = np.asarray(vals, dtype=np.float32).view(np.uint32)
    assert np.all(u & 0xFFFF == 0), "value not representable in bfloat16"
    return (u >> 16).astype(np.uint16)


def test_gate_up_hand_example():
    # g = 64 x_t, u = x_t * wu: silu(64) is 64 in double (1 + e^-64 rounds to 1) and
    # silu(128) is 128, so tokens with x > 0 give h = g*u exactly; x = -1 gives the
    # negative branch, -64 / (1 + e^64) = -1.03e-26, times u
    x = _bf16_bits([[1.0], [-1.0], [1.0], [2.0]])
    wg = _bf16_bits([[64.0, 64.0, 64.0]])
    wu = _bf16_bits([[0.5, -2.0, 3.0]])
    h, pmax, hd = oracle.gate_up(x, wg, wu, tile=2)
    hv = W.bf16_bits_to_f32(h)
    assert np.array_equal(hv[0], [32.0, -128.0, 192.0])
    assert np.array_equal(hv[2], [32.0, -128.0, 192.0])
    assert np.array_equal(hv[3], [128.0, -512.0, 768.0])
    neg = 64.0 * math.exp(-64.0) * np.array([0.5, -2.0, 3.0])  # -silu(-64) ~ 64 e^-64 to 1e-27 relative
    assert np.all(np.sign(hv[1]) == np.sign(neg))
    assert np.allclose(hv[1], neg, rtol=2 ** -8, atol=0)
    assert np.allclose(hd[1], neg, rtol=1e-12, atol=0)
    assert np.array_equal(pmax, [[32.0, 128.0, 192.0], [128.0, 512.0, 768.0]])


def test_gate_up_rounding_ties_and_subnormals():
    # g = 64 for both tokens, so h = 64 u exactly in double.  Token 0 lands on the
    # bfloat16 ties 1 + 2^-8 (-> 1, even) and 1 + 3*2^-8 (-> 1 + 2^-6, even); token 1
    # lands on 8.5 and 9.5 subnormal quanta 2^-133 (-> 8 and 10 quanta).
    e = math.ldexp
    x = _bf16_bits([[1.0, 1.0, 0.0, 0.0], [0.0, 0.0, e(1, -8), e(1, -8)]])
    wg = _bf16_bits([[64.0, 64.0], [0.0, 0.0], [e(1, 14), e(1, 14)], [0.0, 0.0]])
    wu = _bf16_bits([[e(1, -6), e(1, -6)], [e(1, -14), 3 * e(1, -14)], [e(1, -128), e(1, -128)],
                     [e(1, -132), 3 * e(1, -132)]])
    h, _, hd = oracle.gate_up(x, wg, wu)
    assert hd[0, 0] == 1 + e(1, -8) and hd[0, 1] == 1 + 3 * e(1, -8)
    assert hd[1, 0] == 8.5 * e(1, -133) and hd[1, 1] == 9.5 * e(1, -133)
    assert [int(v) for v in h[0]] == [0x3F80, 0x3F82]
    assert [int(v) for v in h[1]] == [0x0008, 0x000A]


def test_gate_up_equals_library_products():
    # float64 library matmul of the exact bf16 values and scipy's logistic function;
    # the oracle's h must be the bfloat16 nearest to silu(g) * u
    from scipy.special import expit
    T, H, Mi = 3, 64, 40
    x = W.normal_bf16(5, W.S_X, T * H).reshape(T, H)
    wg = W.normal_bf16(5, W.S_WG, H * Mi, 0.2).reshape(H, Mi)
    wu = W.normal_bf16(5, W.S_WU, H * Mi, 0.2).reshape(H, Mi)
    h, pmax, hd = oracle.gate_up(x, wg, wu, tile=2)
    f = lambda a: W.bf16_bits_to_f32(a).astype(np.float64)
    g, u = f(x) @ f(wg), f(x) @ f(wu)
    want = g * expit(g) * u
    assert np.allclose(hd, want, rtol=1e-12, atol=1e-300)
    hv = f(h)
    # nearest: no other bfloat16 is closer than the chosen one (one ulp above and below)
    mag = np.abs(want)  # the spacing at the exact value: below a power of two it is the finer one
    ulp = np.ldexp(1.0, np.maximum(np.floor(np.log2(np.where(mag > 0, mag, 1.0))).astype(int) - 7, -133))
    assert np.all(np.abs(hv - want) <= 0.5 * ulp * (1 + 1e-9))
    assert np.array_equal(pmax[0], np.abs(hv[:2]).max(axis=0)) and np.array_equal(pmax[1], np.abs(hv[2]))
