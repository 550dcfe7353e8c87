"""RMM oracle -- TEST INFRASTRUCTURE ONLY.

ctypes wrapper over the plain single-threaded C oracle in ``rmm_oracle.c``.
Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the product library never does.  It shares no code with
the HIP path (it has its own keep count, scorer, top-k and products).

Functions whose result has no pin other than the pages' definitions are
marked "parity unpinned" in their docstring; at present there are none: see
``tests/test_oracle.py`` for the pin of every function.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "rmm_oracle.c")

F32, BF16 = 0, 1

CFLAGS = ["-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build(force=True)
        L = C.CDLL(LIB)
        i64, dbl, vp, i32 = C.c_int64, C.c_double, C.c_void_p, C.c_int
        L.ora_keep_count.restype = i64
        L.ora_keep_count.argtypes = [i64, dbl]
        L.ora_scores.restype = i32
        L.ora_scores.argtypes = [vp, i32, i64, i64, i64, vp, i64, vp]
        L.ora_select.restype = i32
        L.ora_select.argtypes = [vp, i32, i64, i64, i64, vp, i64, dbl, vp]
        L.ora_block_keep_count.restype = i64
        L.ora_block_keep_count.argtypes = [i64, dbl]
        L.ora_select_blocks.restype = i32
        L.ora_select_blocks.argtypes = [vp, i32, i64, i64, i64, i64, i64, dbl, vp]
        L.ora_linear.restype = i32
        L.ora_linear.argtypes = [vp, i32, i64, i64, i64, vp, i32, i64, i64, vp, i64, i64, i64, i64,
                                 vp, i64, vp]
        L.ora_dense_linear.restype = i32
        L.ora_dense_linear.argtypes = [vp, i32, i64, i64, i64, vp, i32, i64, i64, i64, i64, vp, i64, vp]
        L.ora_attn_decode.restype = i32
        L.ora_attn_decode.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, C.c_float,
                                      dbl, dbl, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.ora_gate_up.restype = i32
        L.ora_gate_up.argtypes = [vp, i64, i64, i64, vp, vp, i64, i64, i64, vp, i64, vp, vp]
        L.ora_dense_attn.restype = i32
        L.ora_dense_attn.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, C.c_float, vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _dt(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or uint16 (bf16 bits), got {a.dtype}")


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def keep_count(n: int, r: float) -> int:
    return int(lib().ora_keep_count(int(n), float(r)))


def scores(x, c, tile):
    x = np.ascontiguousarray(x)
    c = np.ascontiguousarray(c, dtype=np.float32)
    T, K = x.shape
    nt = -(-T // tile)
    s = np.empty((nt, K), dtype=np.float32)
    _check(lib().ora_scores(_p(x), _dt(x), T, K, K, _p(c), tile, _p(s)), "scores")
    return s


def select(x, c, tile, r):
    """idx [n_tiles, k] int32, ascending per tile."""
    x = np.ascontiguousarray(x)
    c = np.ascontiguousarray(c, dtype=np.float32)
    T, K = x.shape
    k = keep_count(K, r)
    if k < 0:
        raise ValueError("r must be in (0, 1]")
    nt = -(-T // tile)
    idx = np.empty((nt, k), dtype=np.int32)
    _check(lib().ora_select(_p(x), _dt(x), T, K, K, _p(c), tile, float(r), _p(idx)), "select")
    return idx


def block_keep_count(nb, keep):
    return int(lib().ora_block_keep_count(int(nb), float(keep)))


def select_blocks(x, tile, block, keep):
    """Block-granular selection: idx [n_tiles, nk*block] int32 (kept blocks ascending, expanded)."""
    x = np.ascontiguousarray(x)
    T, K = x.shape
    if block < 1 or K % block:
        raise ValueError("K must be a multiple of block")
    nk = block_keep_count(K // block, keep)
    if nk < 0:
        raise ValueError("keep must be in (0, 1]")
    nt = -(-T // tile)
    idx = np.empty((nt, nk * block), dtype=np.int32)
    _check(lib().ora_select_blocks(_p(x), _dt(x), T, K, K, tile, block, float(keep), _p(idx)), "select_blocks")
    return idx


def linear(x, wt, idx, tile, rows=None, want_double=False):
    """Reduced product y [T, M] float32 (rows outside ``rows`` (t0, t1) are left 0)."""
    x = np.ascontiguousarray(x)
    wt = np.ascontiguousarray(wt)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, K = x.shape
    M = wt.shape[1]
    k = idx.shape[1]
    t0, t1 = rows if rows is not None else (0, T)
    y = np.zeros((T, M), dtype=np.float32)
    yd = np.zeros((T, M), dtype=np.float64) if want_double else None
    _check(lib().ora_linear(_p(x), _dt(x), T, K, K, _p(wt), _dt(wt), M, M, _p(idx), k, tile, t0, t1,
                            _p(y), M, _p(yd)), "linear")
    return (y, yd) if want_double else y


def dense_linear(x, wt, rows=None, want_double=False):
    x = np.ascontiguousarray(x)
    wt = np.ascontiguousarray(wt)
    T, K = x.shape
    M = wt.shape[1]
    t0, t1 = rows if rows is not None else (0, T)
    y = np.zeros((T, M), dtype=np.float32)
    yd = np.zeros((T, M), dtype=np.float64) if want_double else None
    _check(lib().ora_dense_linear(_p(x), _dt(x), T, K, K, _p(wt), _dt(wt), M, M, t0, t1, _p(y), M, _p(yd)),
           "dense_linear")
    return (y, yd) if want_double else y


def gate_up(x, wg, wu, tile=1):
    """Gated FFN producer (blog section 6.1 demo code, ffn_full; sections 5.1, 6.2).
    x [T,H] uint16 (bf16); wg, wu [H,Mi] uint16 (W_gate^T, W_up^T, K-major).
    Returns (h [T,Mi] uint16 bf16, pmax [ceil(T/tile),Mi] float32, hd [T,Mi] float64):
    h = bf16(silu(g)*u) with g, u summed in double, pmax = tile maxima of |h|,
    hd = silu(g)*u before the rounding."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    wg = np.ascontiguousarray(wg, dtype=np.uint16)
    wu = np.ascontiguousarray(wu, dtype=np.uint16)
    T, H = x.shape
    if wg.shape != wu.shape or wg.shape[0] != H:
        raise ValueError("wg and wu must both be [H, Mi]")
    Mi = wg.shape[1]
    h = np.zeros((T, Mi), dtype=np.uint16)
    pmax = np.zeros((-(-T // tile), Mi), dtype=np.float32)
    hd = np.zeros((T, Mi), dtype=np.float64)
    _check(lib().ora_gate_up(_p(x), T, H, H, _p(wg), _p(wu), Mi, Mi, tile, _p(h), Mi, _p(pmax), _p(hd)), "gate_up")
    return h, pmax, hd


def attn_decode(q, kt, v, kn, scale, r_dim, r_pos, mode=0, S=None, want=("out",), vn=None):
    """Reduced GQA decode attention. q [B,Hq,D], kt [B,Hkv,D,ldk], v [B,Hkv,ldv,D] uint16 (bf16),
    kn [B,Hkv,D] float32; vn [B,Hkv,ldv] float32 (optional: weights the position score by the
    value-row norm).  Returns a dict with the requested entries among
    out, dim_idx, pos_idx, lse, pi, p, out_d."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    kt = np.ascontiguousarray(kt, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    kn = np.ascontiguousarray(kn, dtype=np.float32)
    vn = None if vn is None else np.ascontiguousarray(vn, dtype=np.float32)
    B, Hq, D = q.shape
    Hkv, ldk = kt.shape[1], kt.shape[3]
    ldv = v.shape[2]
    if vn is not None and vn.shape != (B, Hkv, ldv):
        raise ValueError("vn must be [B, Hkv, ldv]")
    S = ldk if S is None else S
    Hsel = Hkv if mode == 0 else Hq
    kd, ks = keep_count(D, r_dim), keep_count(S, r_pos)
    if kd < 0 or ks < 0:
        raise ValueError("ratios must be in (0, 1]")
    res = {}
    res["out"] = np.zeros((B, Hq, D), dtype=np.float32)
    res["dim_idx"] = np.zeros((B, Hsel, kd), dtype=np.int32)
    res["pos_idx"] = np.zeros((B, Hsel, ks), dtype=np.int32)
    res["lse"] = np.zeros((B, Hq), dtype=np.float32)
    res["pi"] = np.zeros((B, Hsel, S), dtype=np.float64) if "pi" in want else None
    res["p"] = np.zeros((B, Hq, S), dtype=np.float64) if "p" in want else None
    res["out_d"] = np.zeros((B, Hq, D), dtype=np.float64) if "out_d" in want else None
    _check(lib().ora_attn_decode(_p(q), _p(kt), _p(v), _p(kn), B, Hq, Hkv, D, S, ldk, ldv, float(scale),
                                 float(r_dim), float(r_pos), int(mode), _p(res["out"]), _p(res["dim_idx"]),
                                 _p(res["pos_idx"]), _p(res["lse"]), _p(res["pi"]), _p(res["p"]),
                                 _p(res["out_d"]), _p(vn)), "attn_decode")
    return res


def dense_attn(q, kt, v, scale, S=None):
    q = np.ascontiguousarray(q, dtype=np.uint16)
    kt = np.ascontiguousarray(kt, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    B, Hq, D = q.shape
    Hkv, ldk = kt.shape[1], kt.shape[3]
    ldv = v.shape[2]
    S = ldk if S is None else S
    out = np.zeros((B, Hq, D), dtype=np.float64)
    _check(lib().ora_dense_attn(_p(q), _p(kt), _p(v), B, Hq, Hkv, D, S, ldk, ldv, float(scale), _p(out)),
           "dense_attn")
    return out
