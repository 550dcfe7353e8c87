"""GPU parity of decode attention over paged caches and ragged batches
(rmm_attn_decode_paged, rmm_attn_decode_dense_paged) against the oracle,
through the C ABI.

A ragged batch is B independent decodes: sequence b is checked against the
oracle run on its own contiguous cache of S_b positions, with the bars of the
contiguous path (head_dim sets bit-exact; position sets equal up to the
near-tie rule; out within rel-L2 2e-2, 1e-5 when the position sets agree; lse
within 1e-6 relative).  Positions past a sequence's end, spare pages and the
block-table entries past a sequence's pages hold +inf keys and values (and huge
value norms): any read of them would show in the results.
"""
import numpy as np
import pytest
import torch

import input_adaptive_reduced_score_amd as rmm
import oracle
import workloads as W
from _util import check_near_tie_sets, dev, rel_l2

pytestmark = pytest.mark.gpu


def gpu_paged(pc, r_dim, r_pos, mode, use_vn=False, S=None):
    print(f"[case] {pc.name} lengths={list(pc.seqlens)} r=({r_dim},{r_pos}) mode={mode} vn={use_vn}", flush=True)
    out, dim_idx, pos_idx, lse = rmm.attn_decode_paged(
        dev(pc.q), dev(pc.k_pages), dev(pc.v_pages), dev(pc.kn), dev(pc.block_table), dev(pc.seqlens),
        r_dim, r_pos, scale=pc.scale, mode=mode, S=S if S is not None else pc.S,
        vn_pages=dev(pc.vn_pages) if use_vn else None)
    torch.cuda.synchronize()
    return out.cpu().numpy(), dim_idx.cpu().numpy(), pos_idx.cpu().numpy(), lse.cpu().numpy()


def check_paged(pc, r_dim, r_pos, mode=0, use_vn=False, S=None):
    out, dim_idx, pos_idx, lse = gpu_paged(pc, r_dim, r_pos, mode, use_vn, S)
    ndiff = 0
    for b, cs in enumerate(pc.seqs):
        vn = W.value_row_norms(cs.v) if use_vn else None
        ref = oracle.attn_decode(cs.q, cs.kt, cs.v, cs.kn, cs.scale, r_dim, r_pos, mode, want=("pi",), vn=vn)
        assert np.array_equal(dim_idx[b], ref["dim_idx"][0]), f"sequence {b}: head_dim selections differ"
        kb = ref["pos_idx"].shape[2]
        assert kb == oracle.keep_count(int(pc.seqlens[b]), r_pos)
        assert np.all(pos_idx[b][:, kb:] == -1), f"sequence {b}: index row not closed with -1"
        Hsel = ref["pos_idx"].shape[1]
        nd = check_near_tie_sets(pos_idx[b][:, :kb].reshape(Hsel, kb), ref["pos_idx"][0],
                                 ref["pi"].reshape(Hsel, -1))
        ndiff += nd
        err = rel_l2(out[b], ref["out"][0])
        assert err <= 2e-2, f"sequence {b}: out rel-L2 {err:.3e}"
        if nd == 0:
            assert err <= 1e-5, f"sequence {b}: out rel-L2 {err:.3e} with identical position sets"
        assert np.max(np.abs(lse[b] - ref["lse"][0]) / np.abs(ref["lse"][0])) <= 1e-6
    return ndiff


@pytest.mark.parametrize("mode", [0, 1])
def test_ragged_small_pages(mode):
    pc = W.attn_paged([1, 7, 300, 1000], page=64, Hq=8, Hkv=2, seed=1, n_hot=4)
    check_paged(pc, 0.5, 0.5, mode)
    check_paged(pc, 0.25, 0.1, mode)


@pytest.mark.parametrize("page", [8, 24, 512])
def test_page_sizes(page):
    pc = W.attn_paged([513, 100, 2049], page=page, Hq=8, Hkv=2, seed=page, n_hot=4)
    check_paged(pc, 0.5, 0.25, 0)


def test_ratios_one_equal_full_attention_per_sequence():
    pc = W.attn_paged([77, 600], page=32, Hq=4, Hkv=1, seed=3, n_hot=2)
    check_paged(pc, 1.0, 1.0, 0)


def test_bound_above_every_length():
    # S is only a bound: a larger S than any sequence gives the same per-sequence results
    pc = W.attn_paged([300, 1000], page=64, Hq=8, Hkv=2, seed=4, n_hot=4)
    check_paged(pc, 0.5, 0.5, 0, S=pc.block_table.shape[1] * pc.page)


def test_value_norm_weighted_paged():
    pc = W.attn_paged([999, 64, 2500], page=128, Hq=8, Hkv=2, seed=5, n_hot=4)
    check_paged(pc, 0.5, 0.25, 0, use_vn=True)
    check_paged(pc, 0.5, 0.25, 1, use_vn=True)


@pytest.mark.parametrize("mode", [0, 1])
def test_long_mixed_batch_gqa(mode):
    # (mode 0: more workgroups than stay resident, so the key role runs alone and the split PV kernel follows)
    pc = W.attn_paged([40000, 9000, 1, 16384], page=256, Hq=32, Hkv=8, seed=6, n_hot=16)
    check_paged(pc, 0.25, 0.25, mode)


def test_long_mixed_batch_value_norms():
    # the split PV kernel with the value-norm weighted score
    pc = W.attn_paged([40000, 9000, 1, 16384], page=256, Hq=32, Hkv=8, seed=7, n_hot=16)
    check_paged(pc, 0.5, 0.25, 0, use_vn=True)


def test_one_page_per_sequence_equals_contiguous_cache():
    # a contiguous cache is the paged layout with one page per sequence: results bit-identical
    cs = W.attn_case(1, 4096, Hq=8, Hkv=2, seed=8, n_hot=4)
    k_pages = np.ascontiguousarray(cs.kt[0][None])          # [1, Hkv, D, page=S]
    v_pages = np.ascontiguousarray(cs.v[0][None])           # [1, Hkv, page, D]
    bt, sl = np.zeros((1, 1), np.int32), np.array([4096], np.int32)
    a = rmm.attn_decode_paged(dev(cs.q), dev(k_pages), dev(v_pages), dev(cs.kn), dev(bt), dev(sl), 0.5, 0.25,
                              scale=cs.scale)
    b = rmm.attn_decode(dev(cs.q), dev(cs.kt), dev(cs.v), dev(cs.kn), 0.5, 0.25, scale=cs.scale)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("lengths,page", [([1, 7, 300, 1000], 64), ([40000, 9000, 1, 16384], 256)])
def test_dense_paged(lengths, page):
    pc = W.attn_paged(lengths, page=page, Hq=8, Hkv=2, seed=9, n_hot=4)
    print(f"[case] dense paged {lengths} page={page}", flush=True)
    out, lse = rmm.attn_decode_dense_paged(dev(pc.q), dev(pc.k_pages), dev(pc.v_pages), dev(pc.block_table),
                                           dev(pc.seqlens), scale=pc.scale, S=pc.S,
                                           lse=torch.empty((pc.B, 8), device="cuda:0"))
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for b, cs in enumerate(pc.seqs):
        ref = oracle.dense_attn(cs.q, cs.kt, cs.v, cs.scale)
        assert rel_l2(out[b], ref[0]) <= 1e-5, b
        lref = oracle.attn_decode(cs.q, cs.kt, cs.v, cs.kn, cs.scale, 1.0, 1.0, 0)["lse"][0]
        assert np.max(np.abs(lse[b] - lref) / np.abs(lref)) <= 1e-5, b
