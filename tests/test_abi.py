"""C ABI checks that need no GPU: the library loads, exports every function
include/rmm.h declares, its host-only keep count agrees with the oracle's, and
argument errors are reported before anything touches a device."""
import ctypes as C
import os
import re

import pytest

import input_adaptive_reduced_score_amd as rmm
import oracle

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "rmm.h")


def declared():
    txt = open(HDR).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(rmm_[a-z_]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    L = rmm.lib()
    names = declared()
    assert len(names) >= 13
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert sorted(rmm.EXPORTS) == names


@pytest.mark.parametrize("n", [1, 2, 7, 12, 128, 4096, 14336, 131072])
def test_keep_count_matches_oracle(n):
    for r in (1e-6, 0.001, 0.07, 0.1, 1 / 3, 0.25, 0.3, 0.5, 0.75, 0.999, 1.0, 0.0, -1.0, 1.5, float("nan")):
        assert rmm.keep_count(n, r) == oracle.keep_count(n, r), (n, r)


def _call_select(**kw):
    L = rmm.lib()
    a = dict(x=C.c_void_p(16), xt=1, T=1, K=64, ldx=64, c=C.c_void_p(16), tile=1, r=0.5, idx=C.c_void_p(16),
             ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return L.rmm_select(*a.values())


def test_select_argument_errors_host_only():
    L = rmm.lib()
    assert _call_select(x=None) == 1
    assert _call_select(r=0.0) == 1
    assert _call_select(r=1.01) == 1
    assert _call_select(T=0) == 1
    assert _call_select(ldx=8) == 1
    assert _call_select(xt=7) == 1
    assert _call_select(K=40000, ldx=40000) == 2          # above the selector's K limit
    assert _call_select(x=C.c_void_p(18)) == 2            # misaligned
    assert _call_select() == 3                            # no workspace
    assert b"workspace" in L.rmm_last_error()


def test_linear_and_attn_argument_errors_host_only():
    L = rmm.lib()
    p = C.c_void_p(256)
    # dtype mismatch
    assert L.rmm_linear(p, 1, 1, 64, 64, p, 0, 64, 64, p, 8, 1, p, 64, None, 0, None) == 1
    # k > K
    assert L.rmm_linear(p, 1, 1, 64, 64, p, 1, 64, 64, p, 65, 1, p, 64, None, 0, None) == 1
    # ldw not a multiple of 8 bf16 elements
    assert L.rmm_linear(p, 1, 1, 64, 64, p, 1, 60, 60, p, 8, 1, p, 64, None, 0, None) == 2
    # no workspace
    assert L.rmm_linear(p, 1, 1, 64, 64, p, 1, 64, 64, p, 8, 1, p, 64, None, 0, None) == 3
    args = [p, p, p, p, 1, 32, 8, 128, 1000, 1000, 1000, 0.088, 0.5, 0.5, 0, p, None, None, None, None, 0, None]
    bad = list(args)
    bad[5] = 30      # Hq not a multiple of Hkv
    assert L.rmm_attn_decode(*bad) == 1
    bad = list(args)
    bad[7] = 64      # head_dim without a kernel
    assert L.rmm_attn_decode(*bad) == 2
    bad = list(args)
    bad[12] = 0.0    # r_dim
    assert L.rmm_attn_decode(*bad) == 1
    assert L.rmm_attn_decode(*args) == 3  # no workspace
    bad = list(args)
    bad[4] = 65      # B * Hsel = 520 selection groups, above the 512 the entry points take
    assert L.rmm_attn_decode(*bad) == 2
    bad[4] = 64      # 512 groups: accepted (fails only for the missing workspace)
    assert L.rmm_attn_decode(*bad) == 3
    # the value-norm variant: vn inserted after kn, NULL allowed, 16-byte alignment checked
    ex = args[:4] + [None] + args[4:]
    assert L.rmm_attn_decode_ex(*ex) == 3
    ex[4] = p
    assert L.rmm_attn_decode_ex(*ex) == 3
    ex[4] = C.c_void_p(260)
    assert L.rmm_attn_decode_ex(*ex) == 2
    ex[4], ex[0] = p, None
    assert L.rmm_attn_decode_ex(*ex) == 1
    assert L.rmm_attn_decode_workspace_size(1, 32, 8, 128, 32768, 0.25, 0.25, 0) > 0
    # lengths that are not a multiple of 8 still get a size (it grows with S)
    a = L.rmm_attn_decode_workspace_size(2, 8, 2, 128, 2500, 0.5, 0.25, 1)
    assert a >= L.rmm_attn_decode_workspace_size(2, 8, 2, 128, 2496, 0.5, 0.25, 1) > 0
    assert L.rmm_attn_decode_dense_workspace_size(1, 8, 2, 128, 9999) > 0
    assert L.rmm_status_string(3).startswith(b"RMM_EWORKSPACE")


@pytest.mark.parametrize("nb", [1, 3, 7, 64, 100, 1024])
def test_block_keep_count_matches_oracle(nb):
    for keep in (1e-6, 0.01, 0.29, 1 / 3, 0.5, 0.75, 0.999, 1.0, 0.0, -0.5, 1.5, float("nan")):
        assert rmm.block_keep_count(nb, keep) == oracle.block_keep_count(nb, keep), (nb, keep)


def _call_select_blocks(**kw):
    L = rmm.lib()
    a = dict(x=C.c_void_p(16), xt=1, T=1, K=4096, ldx=4096, tile=1, block=64, keep=0.5, idx=C.c_void_p(16),
             ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return L.rmm_select_blocks(*a.values())


def test_select_blocks_argument_errors_host_only():
    L = rmm.lib()
    assert _call_select_blocks(x=None) == 1
    assert _call_select_blocks(block=0) == 1
    assert _call_select_blocks(block=100) == 1               # K not a multiple of the block size
    assert b"multiple" in L.rmm_last_error()
    assert _call_select_blocks(keep=0.0) == 1
    assert _call_select_blocks(keep=2.0) == 1
    assert _call_select_blocks(block=2) == 2                 # 2048 blocks: above the block-count limit
    assert _call_select_blocks(K=40960, ldx=40960) == 2      # above the selector's K limit
    assert _call_select_blocks(x=C.c_void_p(18)) == 2        # misaligned
    assert _call_select_blocks() == 3                        # no workspace


def test_gate_up_argument_errors_host_only():
    L = rmm.lib()
    p = C.c_void_p(256)
    ok = dict(x=p, T=1, H=64, ldx=64, wg=p, wu=p, ldw=128, Mi=128, tile=1, h=p, ldh=128, pmax=None, ws=None,
              ws_bytes=0, stream=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.rmm_gate_up(*a.values())

    assert call(x=None) == 1
    assert call(h=None) == 1
    assert call(T=0) == 1
    assert call(tile=0) == 1
    assert call(ldx=32) == 1               # ldx < H
    assert call(ldw=120) == 1              # ldw < Mi
    assert call(ldh=100) == 1              # ldh < Mi
    assert call(ldw=132) == 2              # pitch not a multiple of 8
    assert call(wu=C.c_void_p(264)) == 2   # misaligned
    assert call(h=C.c_void_p(257)) == 2    # h not 2-byte aligned
    assert call() == 3                     # no workspace
    assert L.rmm_gate_up_workspace_size(1, 4096, 14336, 1) > 0
    assert L.rmm_gate_up_workspace_size(0, 4096, 14336, 1) == 0


def test_paged_attention_argument_errors_host_only():
    L = rmm.lib()
    p = C.c_void_p(256)
    ok = dict(q=p, kp=p, vp=p, kn=p, vn=None, bt=p, maxp=4, page=256, sl=p, B=2, Hq=32, Hkv=8, D=128, S=1000,
              scale=0.088, r_dim=0.5, r_pos=0.5, mode=0, out=p, dim_idx=None, pos_idx=None, lse=None, ws=None,
              ws_bytes=0, stream=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.rmm_attn_decode_paged(*a.values())

    assert call(bt=None) == 1              # no block table
    assert call(sl=None) == 1              # no lengths
    assert call(S=1025) == 1               # S above max_pages * page
    assert call(page=12) == 2              # page not a multiple of 8
    assert call(page=4) == 2
    assert call(kp=C.c_void_p(264)) == 2   # misaligned pool
    assert call(vn=C.c_void_p(260)) == 2   # misaligned value norms
    assert call(D=64) == 2                 # head_dim without a kernel
    assert call(r_pos=0.0) == 1
    assert call() == 3                     # no workspace
    d = [p, p, p, p, 4, 256, p, 2, 32, 8, 128, 1000, 0.088, p, None, None, 0, None]
    assert L.rmm_attn_decode_dense_paged(*d) == 3
    d[4] = 3                               # 3 pages of 256 < S
    assert L.rmm_attn_decode_dense_paged(*d) == 1
