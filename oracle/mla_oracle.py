"""Float64 CPU oracle for Multi-Head Latent Attention decode over a latent KV cache.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline leg of
the benchmark may import this module; the product path never does.  It shares
no code with the HIP library: it reads the logical (unpaged) arrays, or unpacks
a paged pool with its own reader, and computes everything in float64 numpy.

What it computes, and where the pages fix it:

* MLA caches one latent vector c per token plus a narrow RoPE key k_rope; the
  latent is up-projected into per-head keys and values when decoding
  (RAQ-MLA abstract, searcharxiv "Linchuan Xie" author page).  The RoPE key
  only enters the attention score, the latent supplies the values (same
  abstract).
* Two decoding paths over the same weights are algebraically equivalent: the
  unabsorbed one that materialises K and V per head, and the absorbed MQA one
  where W_UK is folded into the query (GQLA abstract, thelatestinai.com paper
  cards page).  ``decode_unabsorbed`` is the plain definition; ``decode_absorbed``
  is its twin; the P1 pin checks they agree.
* The low-bit cache is dequantised inside attention with no full-precision
  copy of the history (QuantMLA English abstract, arxivdaily QuantMLA page, and
  the cache-layout part of the QuantMLA podcast page).  The oracle dequantises
  element by element: RNE_bf16((code - z) * s), integer zero-point z and fp16
  scale s per (token, group); the product is exact, the bf16 rounding is the
  only rounding (a reading: the pages give no formula).

* The cache writer (``write_tokens``) fills a paged pool with new tokens: float
  caches take the values (float32) or their bf16 rounding; quantised caches take
  the round-to-nearest asymmetric quantiser per token and group (``quantise_rtn``;
  the pages pair an INT4 or INT2 latent with an INT4 RoPE key and name
  round-to-nearest as the plain quantiser: QuantMLA abstract and podcast page).

* GQLA's second decode path (``group_weights``, ``expand_groups``, ``attend_groups``): with
  head groups sharing their key/value up-projections, the latent is expanded once per group
  and decoded as grouped-query attention (GQLA abstract, thelatestinai.com paper-cards page).

* A fixed orthogonal rotation of the latent (``hadamard``, ``rotate``,
  ``fold_rotation``) folded into W_UK and W_UV leaves every full-precision result
  unchanged and spreads outlier channels before quantisation (fixed rotations
  adapted to MLA with the same quantiser: QuantMLA podcast page).

Conventions (readings where the pages are silent): W_UK[h] is [d_n, d_c] with
k_nope = W_UK[h] c; W_UV[h] is [d_c, d_v] with v = c W_UV[h]; query i of s_q
attends cached tokens 0 .. L - s_q + i; lse is the natural log of the softmax
denominator of the scaled scores.

Every function here is pinned by tests against closed forms, invariants, brute
force or library routines; none is "parity unpinned".
"""
from __future__ import annotations

from fractions import Fraction
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 64


# --------------------------------------------------------------------------- bf16 / codes

def bf16_round(x) -> np.ndarray:
    """Round to the nearest bfloat16 value, ties to even, for values exact in float32.

    Input float64 values must be exactly representable in float32 (true for the
    dequant products below); the float32 bit pattern is rounded at bit 16.
    Returns float64.
    """
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    if not np.array_equal(f.astype(np.float64), x, equal_nan=True):
        raise ValueError("bf16_round expects float32-exact inputs")
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isnan(x), np.nan, out)


def unpack_codes(packed: np.ndarray, bits: int, n: int) -> np.ndarray:
    """Codes from packed bytes: element e lives in byte e*bits//8 at bit (e*bits) % 8."""
    packed = np.asarray(packed, dtype=np.uint8)
    e = np.arange(n)
    byte = packed[..., (e * bits) // 8].astype(np.int64)
    return ((byte >> ((e * bits) % 8)) & ((1 << bits) - 1)).astype(np.uint8)


def dequant(codes: np.ndarray, sz: np.ndarray, group: int) -> np.ndarray:
    """x_hat = RNE_bf16((code - z) * s) per element; sz[..., g, :] = (s, z) as fp16.

    codes [..., d] uint8, sz [..., d/group, 2] float16.  Float64 result.
    """
    codes = np.asarray(codes).astype(np.float64)
    s = np.asarray(sz[..., 0], dtype=np.float16).astype(np.float64)
    z = np.asarray(sz[..., 1], dtype=np.float16).astype(np.float64)
    s_e = np.repeat(s, group, axis=-1)
    z_e = np.repeat(z, group, axis=-1)
    return bf16_round((codes - z_e) * s_e)


def quantise_rtn(x: np.ndarray, group: int, bits: int):
    """Round-to-nearest asymmetric quantiser (independent of the input generator's).

    Per group: s = fp16((max-min)/(2^b-1)) (1 if 0); z = clamp(rint(-min/s), 0, 2^b-1), an
    integer (stored as +0 when it is zero); code = clamp(rint(x/s) + z, 0, 2^b-1).
    """
    qmax = 2 ** bits - 1
    x = np.asarray(x, dtype=np.float64)
    lead = x.shape[:-1]
    ng = x.shape[-1] // group
    codes = np.empty(x.shape, dtype=np.uint8)
    sz = np.empty(lead + (ng, 2), dtype=np.float16)
    for g in range(ng):
        seg = x[..., g * group:(g + 1) * group]
        lo = seg.min(axis=-1)
        hi = seg.max(axis=-1)
        s = ((hi - lo) / qmax).astype(np.float16)
        s[s == 0] = np.float16(1)
        sd = s.astype(np.float64)
        z = np.minimum(np.maximum(np.rint(-lo / sd), 0), qmax) + 0.0   # an integer: a zero is +0
        q = np.rint(seg / sd[..., None]) + z[..., None]
        codes[..., g * group:(g + 1) * group] = np.minimum(np.maximum(q, 0), qmax).astype(np.uint8)
        sz[..., g, 0] = s
        sz[..., g, 1] = z.astype(np.float16)
    return codes, sz


# --------------------------------------------------------------------------- cache layout

FMT_BITS = {"int4": 4, "int2": 2}
FMT_BYTES = {"f32": 4, "bf16": 2}


def token_bytes(latent_fmt: str, rope_fmt: str, d_c: int, d_r: int,
                g_c: int = 0, g_r: int = 0) -> int:
    """Bytes one cached token occupies: values, or codes plus an fp16 (s, z) pair per group."""
    if latent_fmt in FMT_BYTES:
        return (d_c + d_r) * FMT_BYTES[latent_fmt]
    lat = d_c * FMT_BITS[latent_fmt] // 8 + (d_c // g_c) * 4
    rope = d_r * FMT_BITS[rope_fmt] // 8 + (d_r // g_r) * 4
    return lat + rope


def block_planes(latent_fmt: str, rope_fmt: str, d_c: int, d_r: int, g_c: int = 0, g_r: int = 0):
    """Plane byte offsets inside one 64-token block; each plane starts 16-byte aligned."""
    if latent_fmt in FMT_BYTES:
        return {"row": 0}, BLOCK * token_bytes(latent_fmt, rope_fmt, d_c, d_r)
    sizes = [("lc", BLOCK * d_c * FMT_BITS[latent_fmt] // 8), ("ls", BLOCK * (d_c // g_c) * 4),
             ("rc", BLOCK * d_r * FMT_BITS[rope_fmt] // 8), ("rs", BLOCK * (d_r // g_r) * 4)]
    off, pos = {}, 0
    for name, size in sizes:
        off[name] = pos
        pos += -(-size // 16) * 16
    return off, pos


def read_pool(pool: np.ndarray, block_table: np.ndarray, seq_lens: np.ndarray, latent_fmt: str,
              rope_fmt: str, d_c: int, d_r: int, g_c: int = 0, g_r: int = 0) -> Dict[str, List[np.ndarray]]:
    """Gather the logical per-sequence cache out of a paged pool (own reader).

    Returns lists over sequences of: 'c', 'k_rope' (float formats, float64) or
    'c_codes', 'c_sz', 'r_codes', 'r_sz' (quantised formats).
    """
    off, bb = block_planes(latent_fmt, rope_fmt, d_c, d_r, g_c, g_r)
    pool = np.asarray(pool, dtype=np.uint8).reshape(-1, bb)
    out: Dict[str, List[np.ndarray]] = {}
    for b, L in enumerate(np.asarray(seq_lens)):
        L = int(L)
        nb = -(-L // BLOCK)
        blocks = pool[np.asarray(block_table[b][:nb], dtype=np.int64)]
        if latent_fmt in FMT_BYTES:
            dt = np.float32 if latent_fmt == "f32" else np.uint16
            rows = blocks.view(dt).reshape(nb * BLOCK, d_c + d_r)[:L]
            if latent_fmt == "bf16":
                rows = (rows.astype(np.uint32) << 16).view(np.float32)
            rows = rows.astype(np.float64)
            out.setdefault("c", []).append(rows[:, :d_c])
            out.setdefault("k_rope", []).append(rows[:, d_c:])
        else:
            lb, rb = FMT_BITS[latent_fmt], FMT_BITS[rope_fmt]

            def plane(name, per_tok):
                p = blocks[:, off[name]: off[name] + BLOCK * per_tok]
                return p.reshape(nb * BLOCK, per_tok)[:L]

            out.setdefault("c_codes", []).append(unpack_codes(plane("lc", d_c * lb // 8), lb, d_c))
            out.setdefault("c_sz", []).append(
                np.ascontiguousarray(plane("ls", (d_c // g_c) * 4)).view(np.float16).reshape(L, d_c // g_c, 2))
            out.setdefault("r_codes", []).append(unpack_codes(plane("rc", d_r * rb // 8), rb, d_r))
            out.setdefault("r_sz", []).append(
                np.ascontiguousarray(plane("rs", (d_r // g_r) * 4)).view(np.float16).reshape(L, d_r // g_r, 2))
    return out


def pack_codes_bytes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Packed bytes from codes, the inverse of unpack_codes: element e goes to byte
    e*bits//8 at bit (e*bits) % 8."""
    codes = np.asarray(codes, dtype=np.uint8)
    n = codes.shape[-1]
    out = np.zeros(codes.shape[:-1] + (n * bits // 8,), dtype=np.uint8)
    for e in range(n):
        out[..., (e * bits) // 8] |= (codes[..., e] << ((e * bits) % 8)).astype(np.uint8)
    return out


def write_tokens(pool: np.ndarray, slots: Sequence[int], c_new: np.ndarray, k_new: np.ndarray, latent_fmt: str,
                 rope_fmt: str, d_c: int, d_r: int, g_c: int = 0, g_r: int = 0) -> np.ndarray:
    """The pool after writing token i (latent c_new[i], RoPE key k_new[i]) into slot slots[i] =
    block * 64 + position; slots outside the pool are skipped.  A float cache stores the row
    [c | k_rope] as float32 or rounded to bf16; a quantised cache stores the codes and fp16
    (s, z) pairs of quantise_rtn, per token and group, in its four planes.  The latent at INT4
    or INT2 with an INT4 RoPE key is the pairing the QuantMLA abstract reports; round-to-nearest
    is the plain quantiser of the QuantMLA podcast page's comparison.  Inputs must be exact in
    float32 for float caches.  Returns a new array shaped like pool.
    """
    off, bb = block_planes(latent_fmt, rope_fmt, d_c, d_r, g_c, g_r)
    shape = np.asarray(pool).shape
    out = np.array(pool, dtype=np.uint8, copy=True).reshape(-1, bb)
    nblk = out.shape[0]
    for i, slot in enumerate(np.asarray(slots, dtype=np.int64).tolist()):
        if slot < 0 or slot >= nblk * BLOCK:
            continue
        blk, pos = divmod(slot, BLOCK)
        c = np.asarray(c_new[i], dtype=np.float64)
        k = np.asarray(k_new[i], dtype=np.float64)
        if latent_fmt in FMT_BYTES:
            row = np.concatenate([c, k])
            if latent_fmt == "f32":
                f = row.astype(np.float32)
                if not np.array_equal(f.astype(np.float64), row):
                    raise ValueError("float32 cache rows must be float32-exact")
                raw = f.view(np.uint8)
            else:
                raw = (bf16_round(row).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16).view(np.uint8)
            out[blk, pos * raw.size:(pos + 1) * raw.size] = raw
            continue
        for vec, g, fmt, pc, ps in ((c, g_c, latent_fmt, "lc", "ls"), (k, g_r, rope_fmt, "rc", "rs")):
            bits = FMT_BITS[fmt]
            codes, sz = quantise_rtn(vec[None, :], g, bits)
            packed = pack_codes_bytes(codes[0], bits)
            sz_bytes = np.ascontiguousarray(sz[0], dtype=np.float16).view(np.uint8).reshape(-1)
            out[blk, off[pc] + pos * packed.size: off[pc] + (pos + 1) * packed.size] = packed
            out[blk, off[ps] + pos * sz_bytes.size: off[ps] + (pos + 1) * sz_bytes.size] = sz_bytes
    return out.reshape(shape)


# --------------------------------------------------------------------------- fixed rotations

def hadamard(d: int) -> np.ndarray:
    """The normalised Walsh-Hadamard matrix H_d / sqrt(d) in Sylvester order (d a power of
    two), built by doubling: H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]].  Orthogonal and
    symmetric, so it is its own inverse: a data-free rotation that can be folded into the
    weights around the cached latent (fixed rotations adapted to MLA with the same
    quantiser: QuantMLA podcast page, comparison part)."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(d)


def rotate(x: np.ndarray, d_axis: int = -1) -> np.ndarray:
    """x . H_d / sqrt(d) along d_axis (a library matrix product as the one step)."""
    x = np.moveaxis(np.asarray(x, dtype=np.float64), d_axis, -1)
    return np.moveaxis(x @ hadamard(x.shape[-1]), -1, d_axis)


def fold_rotation(w_uk: np.ndarray, w_uv: np.ndarray):
    """Weights that absorb a latent rotation c -> c R, R = H / sqrt(d_c): W_UK[h] -> W_UK[h] R
    (so that q_lat . c is unchanged) and W_UV[h] -> R^T W_UV[h] = R W_UV[h] (so that
    o_lat W_UV is unchanged)."""
    return rotate(w_uk, -1), rotate(w_uv, -2)


# --------------------------------------------------------------------------- attention

def _softmax_attend(s: np.ndarray, values: np.ndarray):
    """Numerically exact-ish float64 softmax of scores s [T] applied to values [T, d]."""
    m = s.max()
    e = np.exp(s - m)
    den = e.sum()
    return (e / den) @ values, m + np.log(den)


def absorb_q(q_nope: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """q_lat[..., h, :] = q_nope[..., h, :] @ W_UK[h]  (W_UK folded into the query)."""
    return np.einsum("...hn,hnc->...hc", np.asarray(q_nope, np.float64), np.asarray(w_uk, np.float64))


def out_proj(o_lat: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """out[..., h, :] = o_lat[..., h, :] @ W_UV[h]  (latent output up-projected to values)."""
    return np.einsum("...hc,hcv->...hv", np.asarray(o_lat, np.float64), np.asarray(w_uv, np.float64))


def attend_latent(q_lat, q_rope, c, k_rope, seq_lens, s_q: int, sm_scale: float,
                  rows: Optional[Iterable[Tuple[int, int, int]]] = None):
    """Absorbed-form attention over the shared latent (the decode stage).

    s_t = sm_scale * (q_lat . c_t + q_rope . k_rope_t) for t <= L - s_q + i;
    o_lat = softmax(s) @ c; lse = log-sum-exp of s.
    q_lat [B, s_q, H, d_c], q_rope [B, s_q, H, d_r]; c / k_rope indexable per
    sequence as [L, d].  ``rows`` restricts to (b, i, h) triples (others NaN).
    Returns o_lat [B, s_q, H, d_c], lse [B, s_q, H].
    """
    q_lat = np.asarray(q_lat, np.float64)
    q_rope = np.asarray(q_rope, np.float64)
    B, S, H, d_c = q_lat.shape
    o = np.full((B, S, H, d_c), np.nan)
    lse = np.full((B, S, H), np.nan)
    want = None if rows is None else {}
    if rows is not None:
        for (b, i, h) in rows:
            want.setdefault(b, set()).add((i, h))
    for b in range(B):
        if want is not None and b not in want:
            continue
        L = int(seq_lens[b])
        cb = np.asarray(c[b][:L], np.float64)
        kb = np.asarray(k_rope[b][:L], np.float64)
        for i in range(S):
            n = L - s_q + i + 1
            for h in range(H):
                if want is not None and (i, h) not in want[b]:
                    continue
                s = sm_scale * (cb[:n] @ q_lat[b, i, h] + kb[:n] @ q_rope[b, i, h])
                o[b, i, h], lse[b, i, h] = _softmax_attend(s, cb[:n])
    return o, lse


def decode_unabsorbed(q_nope, q_rope, w_uk, w_uv, c, k_rope, seq_lens, s_q: int, sm_scale: float,
                      rows: Optional[Iterable[Tuple[int, int, int]]] = None):
    """The plain MLA decode: per head, K = [c W_UK[h]^T | k_rope], V = c W_UV[h], softmax attention.

    Returns out [B, s_q, H, d_v], lse [B, s_q, H] (NaN outside ``rows`` if given).
    """
    q_nope = np.asarray(q_nope, np.float64)
    q_rope = np.asarray(q_rope, np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    B, S, H, _ = q_nope.shape
    d_v = w_uv.shape[-1]
    out = np.full((B, S, H, d_v), np.nan)
    lse = np.full((B, S, H), np.nan)
    sel = None if rows is None else set(rows)
    for b in range(B):
        L = int(seq_lens[b])
        cb = np.asarray(c[b][:L], np.float64)
        kb = np.asarray(k_rope[b][:L], np.float64)
        for h in range(H):
            if sel is not None and not any((b, i, h) in sel for i in range(S)):
                continue
            k_nope = cb @ w_uk[h].T          # [L, d_n]
            v = cb @ w_uv[h]                 # [L, d_v]
            for i in range(S):
                if sel is not None and (b, i, h) not in sel:
                    continue
                n = L - s_q + i + 1
                s = sm_scale * (k_nope[:n] @ q_nope[b, i, h] + kb[:n] @ q_rope[b, i, h])
                out[b, i, h], lse[b, i, h] = _softmax_attend(s, v[:n])
    return out, lse


def decode_absorbed(q_nope, q_rope, w_uk, w_uv, c, k_rope, seq_lens, s_q: int, sm_scale: float,
                    rows=None):
    """The absorbed twin: q_lat = q_nope W_UK, attend the latent, then up-project by W_UV."""
    q_lat = absorb_q(q_nope, w_uk)
    o_lat, lse = attend_latent(q_lat, q_rope, c, k_rope, seq_lens, s_q, sm_scale, rows)
    return {"q_lat": q_lat, "o_lat": o_lat, "lse": lse, "out": out_proj(o_lat, w_uv)}


# --------------------------------------------------------------------------- GQLA per-group path
#
# GQLA (GQLA abstract, thelatestinai.com paper-cards page) modifies MLA so that the same
# weights expose two algebraically equivalent decode paths: the absorbed MQA path above and a
# GQA path over a per-group expanded cache.  Reading (the abstract gives no formula): the H heads
# form G groups of H/G consecutive heads, and the heads of a group share their key and value
# up-projections, W_UK[h] = W_UK^g and W_UV[h] = W_UV^g for g = h // (H/G).  The GQA path then
# expands the cached latent once per group, k_nope_g = W_UK^g c and v_g = c W_UV^g, next to the
# shared RoPE key, and decodes as grouped-query attention with G key/value heads.

def group_weights(w_g: np.ndarray, H: int) -> np.ndarray:
    """Per-head weights of a model whose G groups of H/G consecutive heads share one matrix:
    W[h] = W_g[h // (H/G)].  w_g [G, ...] -> [H, ...]."""
    w_g = np.asarray(w_g)
    G = w_g.shape[0]
    if H % G:
        raise ValueError("the head count must be a multiple of the group count")
    return np.repeat(w_g, H // G, axis=0)


def expand_groups(c: np.ndarray, w_uk_g: np.ndarray, w_uv_g: np.ndarray):
    """The per-group expanded cache of one sequence's latent c [L, d_c]: keys k_nope[g] =
    c W_UK^g^T [L, d_n] and values v[g] = c W_UV^g [L, d_v] for every group (float64).
    w_uk_g [G, d_n, d_c], w_uv_g [G, d_c, d_v].  Returns (k_nope [G, L, d_n], v [G, L, d_v])."""
    c = np.asarray(c, np.float64)
    w_uk_g = np.asarray(w_uk_g, np.float64)
    w_uv_g = np.asarray(w_uv_g, np.float64)
    k = np.stack([c @ w_uk_g[g].T for g in range(w_uk_g.shape[0])])
    v = np.stack([c @ w_uv_g[g] for g in range(w_uv_g.shape[0])])
    return k, v


def attend_groups(q_nope, q_rope, k_nope, k_rope, v, seq_lens, s_q: int, sm_scale: float,
                  rows: Optional[Iterable[Tuple[int, int, int]]] = None):
    """Grouped-query attention over per-group caches (the GQLA GQA decode).

    Head h belongs to group g = h // (H/G) and, for query i of sequence b, attends tokens
    t <= L - s_q + i with s_t = sm_scale (q_nope[b,i,h] . k_nope[b][g, t] + q_rope[b,i,h] .
    k_rope[b][t]); out = softmax(s) @ v[b][g], lse = log-sum-exp of s.
    q_nope [B, s_q, H, d_n], q_rope [B, s_q, H, d_r]; per sequence k_nope[b] [G, L, d_n],
    k_rope[b] [L, d_r], v[b] [G, L, d_v].  Returns out [B, s_q, H, d_v], lse [B, s_q, H].
    """
    q_nope = np.asarray(q_nope, np.float64)
    q_rope = np.asarray(q_rope, np.float64)
    B, S, H, _ = q_nope.shape
    G = np.asarray(k_nope[0]).shape[0]
    d_v = np.asarray(v[0]).shape[-1]
    out = np.full((B, S, H, d_v), np.nan)
    lse = np.full((B, S, H), np.nan)
    sel = None if rows is None else set(rows)
    for b in range(B):
        L = int(seq_lens[b])
        kn = np.asarray(k_nope[b], np.float64)[:, :L]
        kr = np.asarray(k_rope[b], np.float64)[:L]
        vb = np.asarray(v[b], np.float64)[:, :L]
        for h in range(H):
            g = h // (H // G)
            for i in range(S):
                if sel is not None and (b, i, h) not in sel:
                    continue
                n = L - s_q + i + 1
                s = sm_scale * (kn[g, :n] @ q_nope[b, i, h] + kr[:n] @ q_rope[b, i, h])
                out[b, i, h], lse[b, i, h] = _softmax_attend(s, vb[g, :n])
    return out, lse


def merge_partials(o_parts: Sequence[np.ndarray], lse_parts: Sequence[np.ndarray]):
    """Combine attention results over disjoint token subsets: lse = log sum exp(lse_u),
    o = sum_u exp(lse_u - lse) o_u.  Parts with lse = -inf contribute nothing."""
    lse_parts = [np.asarray(x, np.float64) for x in lse_parts]
    m = np.max(np.stack(lse_parts), axis=0)
    w = [np.exp(l - m) for l in lse_parts]
    tot = sum(w)
    lse = m + np.log(tot)
    o = sum(wi[..., None] * np.asarray(oi, np.float64) for wi, oi in zip(w, o_parts)) / tot[..., None]
    return o, lse


def dequant_cache(c_codes, c_sz, r_codes, r_sz, g_c: int, g_r: int):
    """Per-sequence float64 latent and RoPE key from codes (brute force, element by element)."""
    c = [dequant(cc, cs, g_c) for cc, cs in zip(c_codes, c_sz)]
    k = [dequant(rc, rs, g_r) for rc, rs in zip(r_codes, r_sz)]
    return c, k


def exact_dequant_value(code: int, z: float, s: float) -> float:
    """RNE_bf16 of the exact rational (code - z) * s, computed with Fractions (a second,
    independent route to the same number, used by the pins)."""
    v = (Fraction(int(code)) - Fraction(z)) * Fraction(s)
    if v == 0:
        return 0.0
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    # bf16: 8 significant bits (1 implicit + 7 stored); normal range only
    scaled = a * 128
    lo = scaled.numerator // scaled.denominator
    rem = scaled - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return float(sign * Fraction(lo, 128) * (Fraction(2) ** e))


__all__ = ["bf16_round", "unpack_codes", "pack_codes_bytes", "write_tokens", "hadamard", "rotate", "fold_rotation",
           "dequant", "quantise_rtn",
           "token_bytes", "block_planes",
           "read_pool", "absorb_q", "out_proj", "attend_latent", "decode_unabsorbed", "decode_absorbed",
           "merge_partials", "dequant_cache", "exact_dequant_value", "group_weights", "expand_groups",
           "attend_groups"]
