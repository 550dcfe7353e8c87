"""Seeded synthetic inputs for the RMM (Reduced Matrix Multiplication) hot path.

This module only draws random tensors and prepares the side inputs the method
takes from its caller (per-slice weight-row norms c_j, per-dim key norms).  It
holds none of the method's arithmetic: no scoring, no selection, no reduced
product, no softmax.  Both the oracle under ``oracle/`` and the HIP path receive
the very same host buffers built here.

Workloads follow the shapes of a Llama-3-8B-style decoder layer (the model
family the RMM paper's results table names); the data are Gaussian, not
trained weights.  Recipe (all draws float32, seeded per tensor "stream"):

* bf16 tensors are formed in float32 first and rounded once to bf16 with
  round-to-nearest-even; bf16 values travel as ``uint16`` bit patterns.
* ``N(mu, sigma)`` means standard deviation ``sigma`` (the blog's demo scales
  ``torch.randn`` by 0.02 for weights).
* Large tensors are drawn in slabs, each slab from its own
  ``SeedSequence([seed, stream, slab])`` generator, so the result does not
  depend on the thread count.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# tensor stream ids: one independent random stream per role
S_X, S_W, S_A, S_B, S_OUTLIER, S_Q, S_K, S_V, S_HOT = 1, 2, 3, 4, 5, 6, 7, 8, 9
S_WG, S_WU = 10, 11

SLAB = 1 << 24  # elements per independently seeded slab


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _gen(seed: int, stream: int, slab: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, slab])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    t = u >> 16
    t &= 1
    t += 0x7FFF
    t += u
    t >>= 16
    return t.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_f32(seed: int, stream: int, n: int, sigma: float = 1.0) -> np.ndarray:
    """n float32 draws of N(0, sigma), slab-seeded, filled in parallel."""
    out = np.empty(n, dtype=np.float32)
    nslab = max(1, -(-n // SLAB))

    def fill(i):
        lo, hi = i * SLAB, min(n, (i + 1) * SLAB)
        seg = out[lo:hi]
        _gen(seed, stream, i).standard_normal(hi - lo, dtype=np.float32, out=seg)
        if sigma != 1.0:
            seg *= np.float32(sigma)

    if nslab == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nslab)))
    return out


def normal_bf16(seed: int, stream: int, n: int, sigma: float = 1.0) -> np.ndarray:
    """n bf16 draws of N(0, sigma) as uint16 bits (float32 draw, one RNE rounding)."""
    out = np.empty(n, dtype=np.uint16)
    nslab = max(1, -(-n // SLAB))

    def fill(i):
        lo, hi = i * SLAB, min(n, (i + 1) * SLAB)
        a = _gen(seed, stream, i).standard_normal(hi - lo, dtype=np.float32)
        if sigma != 1.0:
            a *= np.float32(sigma)
        out[lo:hi] = f32_to_bf16_bits(a)

    if nslab == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nslab)))
    return out


def row_l2_f32(w: np.ndarray, is_bf16: bool) -> np.ndarray:
    """L2 norm of every row of a [rows, cols] matrix, summed in float64, rounded to float32.

    This is the per-slice weight c_j the linear scorer receives as an input
    (the norm of row j of W^T, i.e. of the weights slice j multiplies)."""
    rows = w.shape[0]
    out = np.empty(rows, dtype=np.float32)
    step = 1024
    for lo in range(0, rows, step):
        blk = w[lo:lo + step]
        f = bf16_bits_to_f32(blk) if is_bf16 else blk.astype(np.float32)
        f = f.astype(np.float64)
        out[lo:lo + step] = np.sqrt(np.einsum("ij,ij->i", f, f)).astype(np.float32)
    return out


# ----------------------------------------------------------------------------
# linear workloads
# ----------------------------------------------------------------------------

@dataclass
class LinearCase:
    name: str
    x: np.ndarray        # [T, K]  float32 or uint16 (bf16 bits)
    wt: np.ndarray       # [K, M]  W^T, K-major: row j is slice j
    c: np.ndarray        # [K] float32 row norms of wt
    tile: int
    dtype: str           # "f32" or "bf16"
    rs: tuple = field(default_factory=tuple)

    @property
    def T(self):
        return self.x.shape[0]

    @property
    def K(self):
        return self.x.shape[1]

    @property
    def M(self):
        return self.wt.shape[1]


def linear_random(T: int, K: int, M: int, tile: int, dtype: str, seed: int = 0,
                  xsigma: float = 1.0, wsigma: float = 0.05, name: str = "random") -> LinearCase:
    """Plain Gaussian linear case of any shape (tests: ragged tiles, odd sizes)."""
    if dtype == "f32":
        x = normal_f32(seed, S_X, T * K, xsigma).reshape(T, K)
        wt = normal_f32(seed, S_W, K * M, wsigma).reshape(K, M)
        c = row_l2_f32(wt, False)
    else:
        x = normal_bf16(seed, S_X, T * K, xsigma).reshape(T, K)
        wt = normal_bf16(seed, S_W, K * M, wsigma).reshape(K, M)
        c = row_l2_f32(wt, True)
    return LinearCase(name, x, wt, c, tile, dtype)


def linear_tiny(seed: int = 0) -> LinearCase:
    """X[4,512] f32 ~N(0,1), W^T[512,1024] f32 ~N(0,0.05), one tile of 4 tokens, r = 0.5."""
    cs = linear_random(4, 512, 1024, 4, "f32", seed, 1.0, 0.05, "tiny_linear_f32_T4_K512_M1024")
    cs.rs = (0.5,)
    return cs


def silu_times_b_bf16(seed: int, n: int) -> np.ndarray:
    """bf16(silu(a) * b), a, b ~ N(0,1): the gated activation feeding an MLP down projection.

    silu is evaluated in float64 and rounded to float32 before the product so
    the result does not depend on the host's vector exp."""
    a = normal_f32(seed, S_A, n).astype(np.float64)
    b = normal_f32(seed, S_B, n)
    s = (a / (1.0 + np.exp(-a))).astype(np.float32)
    return f32_to_bf16_bits(s * b)


def linear_decode(seed: int = 0, K: int = 14336, M: int = 4096) -> LinearCase:
    """MLP down_proj decode: X[1,14336] bf16 = silu(a)*b; W^T[14336,4096] bf16 ~N(0,0.02)."""
    x = silu_times_b_bf16(seed, K).reshape(1, K)
    wt = normal_bf16(seed, S_W, K * M, 0.02).reshape(K, M)
    c = row_l2_f32(wt, True)
    return LinearCase(f"decode_down_proj_bf16_K{K}_M{M}", x, wt, c, 1, "bf16",
                      (0.25, 0.5, 0.75, 1.0))


def linear_qkv_decode(seed: int = 6, H: int = 4096, Hq: int = 32, Hkv: int = 8, D: int = 128) -> LinearCase:
    """One decode token into the fused Q, K, V projections of a GQA layer: x[1,H] ~N(0,1) bf16,
    W_qkv^T [H, (Hq+2*Hkv)*D] bf16 ~N(0,0.02) (the three K-major matrices side by side).  A single
    selection over H is shared by the three products: c_j is the norm of the whole row j."""
    cs = linear_random(1, H, (Hq + 2 * Hkv) * D, 1, "bf16", seed, 1.0, 0.02,
                       f"decode_qkv_proj_bf16_K{H}_M{(Hq + 2 * Hkv) * D}")
    cs.rs = (0.25, 0.5)
    return cs


def linear_o_decode(seed: int = 7, H: int = 4096) -> LinearCase:
    """One decode token into the attention output projection: x[1,H] ~N(0,1), W_o^T [H,H] ~N(0,0.02)."""
    cs = linear_random(1, H, H, 1, "bf16", seed, 1.0, 0.02, f"decode_o_proj_bf16_K{H}_M{H}")
    cs.rs = (0.25, 0.5)
    return cs


def linear_prefill(seed: int = 0, T: int = 2048, K: int = 4096, M: int = 4096,
                   tile: int = 256, outlier_frac: float = 0.01, outlier_scale: float = 20.0) -> LinearCase:
    """Prefill: X[2048,4096] bf16 ~N(0,1) with ceil(1%) outlier columns x20; W^T[4096,4096] bf16 ~N(0,0.02)."""
    x = normal_f32(seed, S_X, T * K).reshape(T, K)
    nout = int(math.ceil(outlier_frac * K))
    cols = _gen(seed, S_OUTLIER).choice(K, size=nout, replace=False)
    x[:, cols] *= np.float32(outlier_scale)
    xb = f32_to_bf16_bits(x)
    wt = normal_bf16(seed, S_W, K * M, 0.02).reshape(K, M)
    c = row_l2_f32(wt, True)
    return LinearCase(f"prefill_bf16_T{T}_K{K}_M{M}_tile{tile}", xb, wt, c, tile, "bf16",
                      (0.25, 0.5, 0.75, 1.0))


def ffn_block_demo(seed: int = 42, H: int = 1024, Mi: int = 4096) -> LinearCase:
    """The blog's block demo shape (section 6.1 run_demo): one token x[1,H] ~N(0,1),
    W_gate, W_up [Mi,H] ~N(0,0.02); the down projection's input h = silu(W_gate x) *
    (W_up x) [1,Mi] (float64 products, rounded to bf16) is the activation; W^T =
    W_down^T [Mi,H] bf16 ~N(0,0.02).  Synthetic stand-in for the demo's torch draws."""
    x_in = normal_f32(seed, S_X, H).astype(np.float64)
    wg = normal_f32(seed, S_WG, Mi * H, 0.02).reshape(Mi, H).astype(np.float64)
    wu = normal_f32(seed, S_WU, Mi * H, 0.02).reshape(Mi, H).astype(np.float64)
    g, u = wg @ x_in, wu @ x_in
    h = (g / (1.0 + np.exp(-g))) * u
    xb = f32_to_bf16_bits(h.astype(np.float32)).reshape(1, Mi)
    wt = normal_bf16(seed, S_W, Mi * H, 0.02).reshape(Mi, H)
    c = row_l2_f32(wt, True)
    return LinearCase(f"ffn_block_demo_bf16_Mi{Mi}_H{H}", xb, wt, c, 1, "bf16", (0.5,))


@dataclass
class FfnCase:
    """Gated FFN of one decoder layer: x [T,H] -> h = silu(x Wg^T)*(x Wu^T) [T,Mi] -> h W_down^T."""
    name: str
    x: np.ndarray        # [T, H] uint16 (bf16): the FFN input
    wg: np.ndarray       # [H, Mi] uint16: W_gate^T, K-major
    wu: np.ndarray       # [H, Mi] uint16: W_up^T, K-major
    wd: np.ndarray       # [Mi, H] uint16: W_down^T, K-major (row j = slice j of the down projection)
    c: np.ndarray        # [Mi] float32 row norms of wd (the down projection's scorer weights)
    tile: int

    @property
    def T(self):
        return self.x.shape[0]

    @property
    def H(self):
        return self.x.shape[1]

    @property
    def Mi(self):
        return self.wg.shape[1]


def ffn_case(T: int = 1, H: int = 4096, Mi: int = 14336, tile: int = 1, seed: int = 0,
             xsigma: float = 1.0, wsigma: float = 0.02, name: str | None = None) -> FfnCase:
    """x ~N(0, xsigma) (a normalised hidden state), all three weight matrices ~N(0, wsigma), bf16.
    The default is the decode FFN of the down-projection shape (H 4096, Mi 14336, one token)."""
    x = normal_bf16(seed, S_X, T * H, xsigma).reshape(T, H)
    wg = normal_bf16(seed, S_WG, H * Mi, wsigma).reshape(H, Mi)
    wu = normal_bf16(seed, S_WU, H * Mi, wsigma).reshape(H, Mi)
    wd = normal_bf16(seed, S_W, Mi * H, wsigma).reshape(Mi, H)
    c = row_l2_f32(wd, True)
    return FfnCase(name or f"ffn_decode_bf16_T{T}_H{H}_Mi{Mi}", x, wg, wu, wd, c, tile)


# ----------------------------------------------------------------------------
# attention decode workloads
# ----------------------------------------------------------------------------

@dataclass
class AttnCase:
    name: str
    q: np.ndarray      # [B, Hq, D] uint16 (bf16)
    kt: np.ndarray     # [B, Hkv, D, S] uint16: keys stored dim-major (row j = dim j over positions)
    v: np.ndarray      # [B, Hkv, S, D] uint16: values position-major
    kn: np.ndarray     # [B, Hkv, D] float32 = ||K[b,g,0:S,j]||_2
    scale: float
    hot: np.ndarray    # [B, n_hot] int64 hot positions (for reporting)
    r_pairs: tuple = field(default_factory=tuple)   # (r_dim, r_pos) sweeps

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def Hq(self):
        return self.q.shape[1]

    @property
    def Hkv(self):
        return self.kt.shape[1]

    @property
    def D(self):
        return self.q.shape[2]

    @property
    def S(self):
        return self.kt.shape[3]


def attn_case(B: int, S: int, Hq: int = 32, Hkv: int = 8, D: int = 128, seed: int = 0,
              n_hot: int = 64, hot_gain: float = 2.0, name: str | None = None) -> AttnCase:
    """GQA decode inputs: q, K, V bf16 ~N(0,1); n_hot random key positions per batch element
    get K[b,g,s,:] += sum over the group's query heads of hot_gain * q_h / ||q_h|| (float32,
    before the bf16 rounding); kn = column norms of the stored bf16 keys (float64 sum)."""
    G = Hq // Hkv
    q = normal_bf16(seed, S_Q, B * Hq * D).reshape(B, Hq, D)
    qf = bf16_bits_to_f32(q).astype(np.float64)
    qdir = qf / np.linalg.norm(qf, axis=2, keepdims=True)          # [B,Hq,D]
    shift = (hot_gain * qdir).reshape(B, Hkv, G, D).sum(axis=2)     # [B,Hkv,D]
    hr = _gen(seed, S_HOT)
    hot = np.stack([np.sort(hr.choice(S, size=min(n_hot, S), replace=False)) for _ in range(B)])

    kt = np.empty((B, Hkv, D, S), dtype=np.uint16)
    v = normal_bf16(seed, S_V, B * Hkv * S * D).reshape(B, Hkv, S, D)
    kn = np.empty((B, Hkv, D), dtype=np.float32)

    def slab(bg):
        b, g = divmod(bg, Hkv)
        a = _gen(seed, S_K, bg).standard_normal(D * S, dtype=np.float32).reshape(D, S)
        a[:, hot[b]] += shift[b, g][:, None].astype(np.float32)
        kb = f32_to_bf16_bits(a)
        kt[b, g] = kb
        f = bf16_bits_to_f32(kb).astype(np.float64)
        kn[b, g] = np.sqrt(np.einsum("ds,ds->d", f, f)).astype(np.float32)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(slab, range(B * Hkv)))
    nm = name or f"attn_decode_gqa_B{B}_Hq{Hq}_Hkv{Hkv}_D{D}_S{S}"
    return AttnCase(nm, q, kt, v, kn, float(np.float32(1.0 / math.sqrt(D))), hot)


def value_row_norms(v: np.ndarray) -> np.ndarray:
    """vn [B,Hkv,ldv] float32: L2 norm of every stored bf16 value row (float64 sum, rounded once),
    the per-position side input a cache owner keeps next to V."""
    vf = bf16_bits_to_f32(v).astype(np.float64)
    return np.sqrt((vf * vf).sum(axis=-1)).astype(np.float32)


def attn_32k(seed: int = 0) -> AttnCase:
    cs = attn_case(1, 32768, seed=seed)
    cs.r_pairs = ((0.25, 0.25), (0.5, 0.5))
    return cs


def attn_128k(seed: int = 0) -> AttnCase:
    cs = attn_case(4, 131072, seed=seed)
    cs.r_pairs = ((0.5, 0.25),)
    return cs


def attn_small(B: int = 1, S: int = 1000, Hq: int = 8, Hkv: int = 2, D: int = 128, seed: int = 0,
               n_hot: int = 8) -> AttnCase:
    return attn_case(B, S, Hq, Hkv, D, seed, n_hot)


# ----------------------------------------------------------------------------
# paged, ragged decode batches
# ----------------------------------------------------------------------------

BF16_INF = 0x7F80


@dataclass
class PagedAttnCase:
    """A decode batch of sequences of different lengths whose caches live in a shared page pool.
    seqs[b] holds sequence b as a contiguous one-sequence AttnCase (its own q, keys, values, kn);
    the pool holds the same keys and values scattered over pages in a shuffled order."""
    name: str
    seqs: list               # AttnCase per sequence (B = 1, S = its length)
    q: np.ndarray            # [B, Hq, D] uint16
    kn: np.ndarray           # [B, Hkv, D] float32
    k_pages: np.ndarray      # [P, Hkv, D, page] uint16 (dim-major keys per page)
    v_pages: np.ndarray      # [P, Hkv, page, D] uint16
    vn_pages: np.ndarray     # [P, Hkv, page] float32 value-row norms
    block_table: np.ndarray  # [B, max_pages] int32
    seqlens: np.ndarray      # [B] int32
    page: int
    scale: float

    @property
    def B(self):
        return len(self.seqs)

    @property
    def S(self):
        return int(self.seqlens.max())


def attn_paged(lengths, page: int = 256, Hq: int = 32, Hkv: int = 8, D: int = 128, seed: int = 0,
               n_hot: int = 8, spare_pages: int = 3, name: str | None = None) -> PagedAttnCase:
    """Sequence b is attn_case(1, lengths[b], seed = seed*1000 + b) (so q and kn are per sequence).
    Pages are assigned to sequences in a seeded random order from a pool with `spare_pages` extra
    pages; positions past a sequence's end inside its last page, the spare pages and the
    block-table entries past a sequence's pages (which name a spare page) hold +inf keys and
    values and huge norms, so any read of them would show in the results."""
    lengths = [int(n) for n in lengths]
    seqs = [attn_case(1, n, Hq, Hkv, D, seed * 1000 + b, min(n_hot, n)) for b, n in enumerate(lengths)]
    npg = [-(-n // page) for n in lengths]
    P = sum(npg) + spare_pages
    perm = _gen(seed, S_HOT, 7).permutation(P).astype(np.int32)
    k_pages = np.full((P, Hkv, D, page), BF16_INF, np.uint16)
    v_pages = np.full((P, Hkv, page, D), BF16_INF, np.uint16)
    vn_pages = np.full((P, Hkv, page), 1e30, np.float32)
    maxp = max(npg)
    poison = perm[-1]  # a spare page
    bt = np.full((len(lengths), maxp), poison, np.int32)
    nxt = 0
    for b, cs in enumerate(seqs):
        n = lengths[b]
        vn = value_row_norms(cs.v)[0]                      # [Hkv, n]
        for i in range(npg[b]):
            pg = perm[nxt]
            nxt += 1
            bt[b, i] = pg
            lo, hi = i * page, min(n, (i + 1) * page)
            k_pages[pg, :, :, :hi - lo] = cs.kt[0, :, :, lo:hi]
            v_pages[pg, :, :hi - lo, :] = cs.v[0, :, lo:hi, :]
            vn_pages[pg, :, :hi - lo] = vn[:, lo:hi]
    q = np.concatenate([cs.q for cs in seqs], axis=0)
    kn = np.concatenate([cs.kn for cs in seqs], axis=0)
    nm = name or f"attn_paged_B{len(lengths)}_Hq{Hq}_Hkv{Hkv}_page{page}_S{max(lengths)}"
    return PagedAttnCase(nm, seqs, q, kn, k_pages, v_pages, vn_pages, bt, np.array(lengths, np.int32), page,
                         seqs[0].scale)
