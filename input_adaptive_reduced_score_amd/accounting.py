"""Algorithmic work of the RMM hot path: the bytes and FLOPs the method itself
must move or compute (retained work only), used for the roofline figures.

FLOP convention: a product of an [m, k] and a [k, n] matrix costs 2*m*n*k
(GEMM notes, section 6 worked example: 2*8*11008*4096 ~ 721 M); the blog's
section 6.2 puts the reduced down projection at 2*H*active_M per token.
"""
from __future__ import annotations

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s


def gemm_flops(m: int, n: int, k: int) -> int:
    return 2 * m * n * k


def linear_flops(T: int, k: int, M: int) -> int:
    """Reduced product of T tokens over k kept slices into M outputs."""
    return gemm_flops(T, M, k)


def decode_step_bytes(K: int, M: int, k: int, xbytes: int = 2, wbytes: int = 2, kept_list: bool = True) -> int:
    """select + reduced GEMV for one token: read x and c (scorer), write and read
    the k indices (kept_list: the two-call step, or the kept list asked for),
    read the k kept W^T rows, write y (fp32)."""
    return K * (xbytes + 4) + (8 * k if kept_list else 0) + wbytes * k * M + 4 * M


def gemv_launch_bytes(k: int, M: int, T: int = 1, xbytes: int = 2, wbytes: int = 2) -> int:
    """The reduced GEMV kernel alone: kept W^T rows, the kept x values, idx, y."""
    return wbytes * k * M + T * xbytes * k + 4 * k + 4 * T * M


def attn_step_bytes(B: int, Hq: int, Hkv: int, D: int, S: int, kd: int, ks: int, mode: int = 0) -> int:
    """Reduced decode attention (mode 0): kept K^T rows (kd dims x S positions,
    bf16), kept V rows (ks positions x D, bf16), the fp32 logits written and
    read back, the ks kept position indices written and read, plus q, kn, out."""
    groups = B * Hkv
    kept_k = groups * kd * S * 2
    kept_v = groups * ks * D * 2
    logits = 2 * B * Hq * S * 4
    idx = 2 * groups * ks * 4
    small = B * Hq * D * 2 + B * Hkv * D * 4 + B * Hq * D * 4
    return kept_k + kept_v + logits + idx + small


def attn_union_step_bytes(B: int, Hq: int, Hkv: int, D: int, S: int, dims_union: int, pos_union: int) -> int:
    """Reduced decode attention with per-query-head selection, read as the union
    over each KV head's query heads: dims_union and pos_union are the sizes of the
    union of the heads' kept dims and kept positions, summed over the B*Hkv KV
    heads.  Each union K^T row (S positions) and V row (D dims) is read once;
    plus the fp32 logits written and read back, q, kn and out."""
    small = B * Hq * D * 2 + B * Hkv * D * 4 + B * Hq * D * 4
    return dims_union * S * 2 + pos_union * D * 2 + 2 * B * Hq * S * 4 + small


def attn_dense_bytes(B: int, Hq: int, Hkv: int, D: int, S: int) -> int:
    return B * Hkv * S * D * 2 * 2 + B * Hq * D * (2 + 4)


def gateup_bytes(T: int, H: int, Mi: int, tile: int = 1) -> int:
    """Gated FFN producer: W_gate^T and W_up^T read once (bf16), x read, h written
    (bf16) and the tile maxima written (fp32)."""
    ntiles = -(-T // tile)
    return 2 * 2 * H * Mi + 2 * T * H + 2 * T * Mi + 4 * ntiles * Mi
