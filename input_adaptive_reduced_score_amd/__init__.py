"""Python binding of librmm.so, the MI355X (gfx950) hot path of Reduced Matrix
Multiplication (RMM).

Argument marshalling only: every step of the path runs in the HIP kernels of
``librmm.so`` (see ``include/rmm.h`` for the semantics of each call).  PyTorch
provides device memory and the current stream.  There is no CPU or PyTorch
fallback: if the library is missing or the device is not a GPU, calls raise.

Names follow the C ABI: ``keep_count``, ``select``, ``linear``,
``linear_dense``, ``attn_decode``, ``attn_decode_dense``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "librmm.so")
SOURCES = ["select.hip", "gemv.hip", "linear.hip", "ffn.hip", "attn.hip", "api.hip"]
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

RMM_F32, RMM_BF16 = 0, 1
PER_KV_GROUP, PER_Q_HEAD = 0, 1
STATUS = {0: "RMM_OK", 1: "RMM_EINVAL", 2: "RMM_EUNSUPPORTED", 3: "RMM_EWORKSPACE", 4: "RMM_EHIP"}
WS_HEADER_BYTES = 4096


class RmmError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


def build(out: str = LIB_PATH, extra_flags=(), jobs: int = 4) -> str:
    """Compile every HIP source for gfx950 and link librmm.so (in-tree)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = os.path.join(ROOT, "include")
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [hipcc, *HIPCC_FLAGS, *extra_flags, f"-I{inc}", "-c", os.path.join(HERE, "csrc", src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    for p in procs:
        _wait(p)
    tmp = out + ".tmp"
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], check=True,
                   stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    os.replace(tmp, out)
    return out


def _wait(item):
    cmd, p = item
    txt, _ = p.communicate()
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed ({p.returncode}): {' '.join(cmd)}\n{txt.decode(errors='replace')}")


_lib = None
_lock = threading.Lock()


def lib():
    """Load librmm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() (hipcc, gfx950) first")
            L = C.CDLL(LIB_PATH)
            vp, i64, i32, dbl, sz, flt = C.c_void_p, C.c_int64, C.c_int, C.c_double, C.c_size_t, C.c_float
            sig = {
                "rmm_keep_count": (i64, [i64, dbl]),
                "rmm_select_workspace_size": (sz, [i64, i64, i64, i32]),
                "rmm_select": (i32, [vp, i32, i64, i64, i64, vp, i64, dbl, vp, vp, sz, vp]),
                "rmm_select_linear_workspace_size": (sz, [i64, i64, i32]),
                "rmm_select_linear": (i32, [vp, i32, i64, vp, dbl, vp, i32, i64, i64, vp, vp, vp, sz, vp]),
                "rmm_block_keep_count": (i64, [i64, dbl]),
                "rmm_select_blocks_workspace_size": (sz, [i64, i64, i64, i64, i32]),
                "rmm_select_blocks": (i32, [vp, i32, i64, i64, i64, i64, i64, dbl, vp, vp, sz, vp]),
                "rmm_linear_workspace_size": (sz, [i64, i64, i64, i64, i64, i32]),
                "rmm_linear": (i32, [vp, i32, i64, i64, i64, vp, i32, i64, i64, vp, i64, i64, vp, i64, vp, sz, vp]),
                "rmm_linear_noalloc": (i32, [vp, i32, i64, i64, i64, vp, i32, i64, i64, vp, i64, i64, vp, i64,
                                             vp]),
                "rmm_linear_dense_workspace_size": (sz, [i64, i64, i64, i32]),
                "rmm_linear_dense": (i32, [vp, i32, i64, i64, i64, vp, i32, i64, i64, vp, i64, vp, sz, vp]),
                "rmm_attn_decode_workspace_size": (sz, [i64, i64, i64, i64, i64, dbl, dbl, i32]),
                "rmm_attn_decode": (i32, [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, flt, dbl, dbl, i32,
                                          vp, vp, vp, vp, vp, sz, vp]),
                "rmm_attn_decode_ex": (i32, [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, flt, dbl, dbl,
                                             i32, vp, vp, vp, vp, vp, sz, vp]),
                "rmm_gate_up_workspace_size": (sz, [i64, i64, i64, i64]),
                "rmm_gate_up": (i32, [vp, i64, i64, i64, vp, vp, i64, i64, i64, vp, i64, vp, vp, sz, vp]),
                "rmm_attn_decode_paged": (i32, [vp, vp, vp, vp, vp, vp, i64, i64, vp, i64, i64, i64, i64, i64, flt,
                                                dbl, dbl, i32, vp, vp, vp, vp, vp, sz, vp]),
                "rmm_attn_decode_dense_paged": (i32, [vp, vp, vp, vp, i64, i64, vp, i64, i64, i64, i64, i64, flt,
                                                      vp, vp, vp, sz, vp]),
                "rmm_attn_decode_dense_workspace_size": (sz, [i64, i64, i64, i64, i64]),
                "rmm_attn_decode_dense": (i32, [vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, flt, vp, vp, vp, sz,
                                                vp]),
                "rmm_status_string": (C.c_char_p, [i32]),
                "rmm_last_error": (C.c_char_p, []),
            }
            for name, (res, args) in sig.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
    return _lib


EXPORTS = ("rmm_keep_count", "rmm_select_workspace_size", "rmm_select", "rmm_select_linear_workspace_size",
           "rmm_select_linear", "rmm_block_keep_count",
           "rmm_select_blocks_workspace_size", "rmm_select_blocks", "rmm_linear_workspace_size", "rmm_linear",
           "rmm_linear_noalloc", "rmm_linear_dense_workspace_size", "rmm_linear_dense", "rmm_attn_decode_workspace_size",
           "rmm_gate_up_workspace_size", "rmm_gate_up",
           "rmm_attn_decode", "rmm_attn_decode_ex", "rmm_attn_decode_paged", "rmm_attn_decode_dense_paged", "rmm_attn_decode_dense_workspace_size", "rmm_attn_decode_dense", "rmm_status_string",
           "rmm_last_error")


def _check(st: int):
    if st != 0:
        raise RmmError(st, lib().rmm_last_error().decode(errors="replace"))


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return RMM_F32
    if t.dtype == torch.bfloat16:
        return RMM_BF16
    raise TypeError(f"tensors must be float32 or bfloat16, got {t.dtype}")


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise RuntimeError(f"{name} must be a GPU tensor (the RMM path has no CPU fallback)")


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("matrices must be 2-D with unit column stride")
    return t.stride(0)


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


class Workspace:
    """A zero-initialised device workspace, grown on demand (per device)."""

    def __init__(self):
        self._bufs = {}

    def get(self, nbytes: int, device) -> torch.Tensor:
        if nbytes <= 0:
            raise RmmError(1, "workspace size query rejected the arguments: " +
                           lib().rmm_last_error().decode(errors="replace"))
        key = torch.device(device).index
        buf = self._bufs.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(nbytes, 1 << 16), dtype=torch.uint8, device=device)
            self._bufs[key] = buf
        return buf


_WS = Workspace()


def keep_count(n: int, r: float) -> int:
    return int(lib().rmm_keep_count(int(n), float(r)))


def select(x: torch.Tensor, c: torch.Tensor, tile: int, r: float, idx: torch.Tensor | None = None, ws=None):
    """Scorer + top-k: returns idx int32 [ceil(T/tile), keep_count(K, r)], ascending per tile."""
    L = lib()
    _dev(x, "x")
    T, K = x.shape
    k = keep_count(K, r)
    if k < 0:
        raise RmmError(1, f"retention ratio {r} not in (0, 1]")
    nt = -(-T // tile)
    if idx is None:
        idx = torch.empty((nt, k), dtype=torch.int32, device=x.device)
    need = L.rmm_select_workspace_size(T, K, tile, _dtype(x))
    w = ws if ws is not None else _WS.get(need, x.device)
    _check(L.rmm_select(_ptr(x), _dtype(x), T, K, _ld(x), _ptr(c), tile, float(r), _ptr(idx), _ptr(w),
                        w.numel() * w.element_size(), _stream()))
    return idx


def select_linear(x: torch.Tensor, c: torch.Tensor, r: float, wt: torch.Tensor, out: torch.Tensor | None = None,
                  idx: torch.Tensor | None = None, want_idx: bool = True, ws=None):
    """One-token decode step in one launch: selection + reduced product.  x [1,K] or [K];
    returns (y [1,M] fp32, idx [1,k] int32 or None).  The workspace's first WS_HEADER_BYTES
    bytes must be zero before first use (the default workspaces are zero-filled)."""
    L = lib()
    _dev(x, "x")
    K = x.shape[-1]
    if x.dim() == 2 and x.shape[0] != 1:
        raise ValueError("select_linear takes one token")
    M = wt.shape[1]
    k = keep_count(K, r)
    if k < 0:
        raise RmmError(1, "ratio must be in (0, 1]")
    if out is None:
        out = torch.empty((1, M), dtype=torch.float32, device=x.device)
    if want_idx and idx is None:
        idx = torch.empty((1, k), dtype=torch.int32, device=x.device)
    need = L.rmm_select_linear_workspace_size(K, M, _dtype(x))
    w = ws if ws is not None else _WS.get(need, x.device)
    _check(L.rmm_select_linear(_ptr(x), _dtype(x), K, _ptr(c), float(r), _ptr(wt), _dtype(wt), M, _ld(wt),
                               _ptr(idx if want_idx else None), _ptr(out), _ptr(w), w.numel() * w.element_size(),
                               _stream()))
    return out, (idx if want_idx else None)


def block_keep_count(nb: int, keep: float) -> int:
    """max(1, floor(nb * keep)) clamped to nb; -1 if keep is not in (0, 1]."""
    return int(lib().rmm_block_keep_count(int(nb), float(keep)))


def select_blocks(x: torch.Tensor, tile: int, block: int, keep: float, idx: torch.Tensor | None = None, ws=None):
    """Block-granular selection: idx int32 [ceil(T/tile), nk*block], kept blocks ascending, expanded to slices."""
    L = lib()
    _dev(x, "x")
    T, K = x.shape
    if block < 1 or K % block:
        raise RmmError(1, f"K = {K} is not a multiple of the block size {block}")
    nk = block_keep_count(K // block, keep)
    if nk < 0:
        raise RmmError(1, f"keep ratio {keep} not in (0, 1]")
    nt = -(-T // tile)
    if idx is None:
        idx = torch.empty((nt, nk * block), dtype=torch.int32, device=x.device)
    need = L.rmm_select_blocks_workspace_size(T, K, tile, block, _dtype(x))
    w = ws if ws is not None else _WS.get(need, x.device)
    _check(L.rmm_select_blocks(_ptr(x), _dtype(x), T, K, _ld(x), tile, block, float(keep), _ptr(idx), _ptr(w),
                               w.numel() * w.element_size(), _stream()))
    return idx


def linear(x: torch.Tensor, wt: torch.Tensor, idx: torch.Tensor, tile: int, out: torch.Tensor | None = None,
           ws=None):
    """Reduced product y = sum over kept slices of x[t, j] * wt[j, :]  (fp32 [T, M])."""
    L = lib()
    _dev(x, "x")
    T, K = x.shape
    M = wt.shape[1]
    k = idx.shape[1]
    if out is None:
        out = torch.empty((T, M), dtype=torch.float32, device=x.device)
    need = L.rmm_linear_workspace_size(T, K, M, k, tile, _dtype(x))
    w = ws if ws is not None else _WS.get(need, x.device)
    _check(L.rmm_linear(_ptr(x), _dtype(x), T, K, _ld(x), _ptr(wt), _dtype(wt), M, _ld(wt), _ptr(idx), k, tile,
                        _ptr(out), _ld(out), _ptr(w), w.numel() * w.element_size(), _stream()))
    return out


def linear_noalloc(x: torch.Tensor, wt: torch.Tensor, idx: torch.Tensor, tile: int,
                   out: torch.Tensor | None = None):
    """rmm_linear without a workspace: the library's own device scratch array is used (calls on one
    GPU must not overlap).  Same arguments and results as linear()."""
    L = lib()
    _dev(x, "x")
    T, K = x.shape
    k = idx.shape[1]
    M = wt.shape[1]
    if out is None:
        out = torch.empty((T, M), dtype=torch.float32, device=x.device)
    _check(L.rmm_linear_noalloc(_ptr(x), _dtype(x), T, K, _ld(x), _ptr(wt), _dtype(wt), M, _ld(wt), _ptr(idx), k,
                                tile, _ptr(out), _ld(out), _stream()))
    return out


def linear_dense(x: torch.Tensor, wt: torch.Tensor, out: torch.Tensor | None = None, ws=None):
    """Dense product y = x @ wt over all slices by the same kernels (r = 1 baseline)."""
    L = lib()
    _dev(x, "x")
    T, K = x.shape
    M = wt.shape[1]
    if out is None:
        out = torch.empty((T, M), dtype=torch.float32, device=x.device)
    need = L.rmm_linear_dense_workspace_size(T, K, M, _dtype(x))
    w = ws if ws is not None else _WS.get(need, x.device)
    _check(L.rmm_linear_dense(_ptr(x), _dtype(x), T, K, _ld(x), _ptr(wt), _dtype(wt), M, _ld(wt), _ptr(out),
                              _ld(out), _ptr(w), w.numel() * w.element_size(), _stream()))
    return out


def gate_up(x, wg, wu, tile: int = 1, h=None, pmax=None, want_pmax: bool = True, ws=None):
    """Gated FFN producer: h = bf16(silu(x W_gate^T) * (x W_up^T)) and the tile maxima of |h|.
    x [T,H] bf16; wg, wu [H,Mi] bf16 (W_gate^T, W_up^T, K-major, same pitch).
    Returns (h [T,Mi] bf16, pmax [ceil(T/tile),Mi] fp32 or None)."""
    L = lib()
    _dev(x, "x")
    if x.dtype != torch.bfloat16 or wg.dtype != torch.bfloat16 or wu.dtype != torch.bfloat16:
        raise ValueError("x, wg and wu must be bfloat16")
    T, H = x.shape
    Mi = wg.shape[1]
    if wg.shape[0] != H or tuple(wu.shape) != tuple(wg.shape) or _ld(wg) != _ld(wu):
        raise ValueError("wg and wu must both be [H, Mi] with the same row pitch")
    dev = x.device
    if h is None:
        h = torch.empty((T, Mi), dtype=torch.bfloat16, device=dev)
    if pmax is None and want_pmax:
        pmax = torch.empty((-(-T // tile), Mi), dtype=torch.float32, device=dev)
    need = L.rmm_gate_up_workspace_size(T, H, Mi, tile)
    w = ws if ws is not None else _WS.get(need, dev)
    _check(L.rmm_gate_up(_ptr(x), T, H, _ld(x), _ptr(wg), _ptr(wu), _ld(wg), Mi, tile, _ptr(h), _ld(h), _ptr(pmax),
                         _ptr(w), w.numel() * w.element_size(), _stream()))
    return h, pmax


def attn_decode(q, kt, v, kn, r_dim: float, r_pos: float, scale: float | None = None, mode: int = PER_KV_GROUP,
                S: int | None = None, out=None, dim_idx=None, pos_idx=None, lse=None, want_idx: bool = True,
                ws=None, vn=None):
    """Reduced GQA decode attention.  q [B,Hq,D] bf16; kt [B,Hkv,D,ldk] bf16 (dim-major keys);
    v [B,Hkv,ldv,D] bf16; kn [B,Hkv,D] fp32; vn None or [B,Hkv,ldv] fp32 value-row norms, which
    weight the position score (p * ||V_s||).  Returns (out, dim_idx, pos_idx, lse)."""
    L = lib()
    _dev(q, "q")
    B, Hq, D = q.shape
    Hkv, ldk = kt.shape[1], kt.shape[3]
    ldv = v.shape[2]
    S = ldk if S is None else S
    for t, n in ((q, "q"), (kt, "kt"), (v, "v"), (kn, "kn")):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if vn is not None:
        _dev(vn, "vn")
        if vn.dtype != torch.float32 or tuple(vn.shape) != (B, Hkv, ldv) or not vn.is_contiguous():
            raise ValueError(f"vn must be a contiguous float32 tensor of shape {(B, Hkv, ldv)}")
    scale = float(D) ** -0.5 if scale is None else float(scale)
    Hsel = Hkv if mode == PER_KV_GROUP else Hq
    kd, ks = keep_count(D, r_dim), keep_count(S, r_pos)
    if kd < 0 or ks < 0:
        raise RmmError(1, "ratios must be in (0, 1]")
    dev = q.device
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    if want_idx:
        if dim_idx is None:
            dim_idx = torch.empty((B, Hsel, kd), dtype=torch.int32, device=dev)
        if pos_idx is None:
            pos_idx = torch.empty((B, Hsel, ks), dtype=torch.int32, device=dev)
        if lse is None:
            lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    need = L.rmm_attn_decode_workspace_size(B, Hq, Hkv, D, S, float(r_dim), float(r_pos), mode)
    w = ws if ws is not None else _WS.get(need, dev)
    if vn is None:
        _check(L.rmm_attn_decode(_ptr(q), _ptr(kt), _ptr(v), _ptr(kn), B, Hq, Hkv, D, S, ldk, ldv, scale,
                                 float(r_dim), float(r_pos), mode, _ptr(out), _ptr(dim_idx), _ptr(pos_idx),
                                 _ptr(lse), _ptr(w), w.numel() * w.element_size(), _stream()))
    else:
        _check(L.rmm_attn_decode_ex(_ptr(q), _ptr(kt), _ptr(v), _ptr(kn), _ptr(vn), B, Hq, Hkv, D, S, ldk, ldv,
                                    scale, float(r_dim), float(r_pos), mode, _ptr(out), _ptr(dim_idx),
                                    _ptr(pos_idx), _ptr(lse), _ptr(w), w.numel() * w.element_size(), _stream()))
    return out, dim_idx, pos_idx, lse


def _paged_args(q, k_pages, v_pages, block_table, seqlens, S):
    _dev(q, "q")
    for t, n in ((q, "q"), (k_pages, "k_pages"), (v_pages, "v_pages"), (block_table, "block_table"),
                 (seqlens, "seqlens")):
        _dev(t, n)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    if block_table.dtype != torch.int32 or seqlens.dtype != torch.int32:
        raise ValueError("block_table and seqlens must be int32")
    B, Hq, D = q.shape
    npages, Hkv, Dk, page = k_pages.shape
    if Dk != D or tuple(v_pages.shape) != (npages, Hkv, page, D):
        raise ValueError("k_pages must be [num_pages, Hkv, D, page] and v_pages [num_pages, Hkv, page, D]")
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(seqlens.shape) != (B,):
        raise ValueError("block_table must be [B, max_pages] and seqlens [B]")
    maxp = block_table.shape[1]
    S = maxp * page if S is None else int(S)
    return B, Hq, Hkv, D, page, maxp, S


def attn_decode_paged(q, k_pages, v_pages, kn, block_table, seqlens, r_dim: float, r_pos: float,
                      scale: float | None = None, mode: int = PER_KV_GROUP, S: int | None = None, vn_pages=None,
                      out=None, want_idx: bool = True, ws=None):
    """Reduced GQA decode over paged, ragged caches.  k_pages [P,Hkv,D,page], v_pages [P,Hkv,page,D] bf16;
    block_table [B,max_pages], seqlens [B] int32 (device); kn [B,Hkv,D] fp32; vn_pages None or
    [P,Hkv,page] fp32; S bounds every sequence length (default max_pages*page).
    Returns (out, dim_idx, pos_idx, lse); pos_idx rows end in -1 past each sequence's kept count."""
    L = lib()
    B, Hq, Hkv, D, page, maxp, S = _paged_args(q, k_pages, v_pages, block_table, seqlens, S)
    if vn_pages is not None:
        _dev(vn_pages, "vn_pages")
        if vn_pages.dtype != torch.float32 or tuple(vn_pages.shape) != tuple(k_pages.shape[:2]) + (page,):
            raise ValueError("vn_pages must be float32 [num_pages, Hkv, page]")
    scale = float(D) ** -0.5 if scale is None else float(scale)
    Hsel = Hkv if mode == PER_KV_GROUP else Hq
    kd, ks = keep_count(D, r_dim), keep_count(S, r_pos)
    if kd < 0 or ks < 0:
        raise RmmError(1, "ratios must be in (0, 1]")
    dev = q.device
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev) if out is None else out
    dim_idx = pos_idx = lse = None
    if want_idx:
        dim_idx = torch.empty((B, Hsel, kd), dtype=torch.int32, device=dev)
        pos_idx = torch.empty((B, Hsel, ks), dtype=torch.int32, device=dev)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    need = L.rmm_attn_decode_workspace_size(B, Hq, Hkv, D, S, float(r_dim), float(r_pos), mode)
    w = ws if ws is not None else _WS.get(need, dev)
    _check(L.rmm_attn_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(kn), _ptr(vn_pages),
                                   _ptr(block_table), maxp, page, _ptr(seqlens), B, Hq, Hkv, D, S, scale,
                                   float(r_dim), float(r_pos), mode, _ptr(out), _ptr(dim_idx), _ptr(pos_idx),
                                   _ptr(lse), _ptr(w), w.numel() * w.element_size(), _stream()))
    return out, dim_idx, pos_idx, lse


def attn_decode_dense_paged(q, k_pages, v_pages, block_table, seqlens, scale: float | None = None,
                            S: int | None = None, out=None, lse=None, ws=None):
    """Dense decode attention over paged, ragged caches (r = 1 baseline).  Returns (out, lse)."""
    L = lib()
    B, Hq, Hkv, D, page, maxp, S = _paged_args(q, k_pages, v_pages, block_table, seqlens, S)
    scale = float(D) ** -0.5 if scale is None else float(scale)
    dev = q.device
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev) if out is None else out
    need = L.rmm_attn_decode_dense_workspace_size(B, Hq, Hkv, D, S)
    w = ws if ws is not None else _WS.get(need, dev)
    _check(L.rmm_attn_decode_dense_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), maxp, page,
                                         _ptr(seqlens), B, Hq, Hkv, D, S, scale, _ptr(out), _ptr(lse), _ptr(w),
                                         w.numel() * w.element_size(), _stream()))
    return out, lse


def attn_decode_dense(q, kt, v, scale: float | None = None, S: int | None = None, out=None, lse=None, ws=None):
    """Dense decode attention over all dims and positions (r = 1 baseline).  Returns (out, lse)."""
    L = lib()
    _dev(q, "q")
    B, Hq, D = q.shape
    Hkv, ldk = kt.shape[1], kt.shape[3]
    ldv = v.shape[2]
    S = ldk if S is None else S
    scale = float(D) ** -0.5 if scale is None else float(scale)
    dev = q.device
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    need = L.rmm_attn_decode_dense_workspace_size(B, Hq, Hkv, D, S)
    w = ws if ws is not None else _WS.get(need, dev)
    _check(L.rmm_attn_decode_dense(_ptr(q), _ptr(kt), _ptr(v), B, Hq, Hkv, D, S, ldk, ldv, scale, _ptr(out),
                                   _ptr(lse), _ptr(w), w.numel() * w.element_size(), _stream()))
    return out, lse
