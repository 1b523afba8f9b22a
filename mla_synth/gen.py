"""Seeded synthetic inputs for MLA decode over a paged latent cache.

Everything here is input preparation shared by the float64 oracle and the GPU
path: random draws, rounding the draws to the storage dtype, the round-to-
nearest quantiser that turns latent values into stored codes (the cache
producer, not the decode), packing into paged blocks with a shuffled block
table, and NaN poison in every byte the decode must not use.  It contains no
attention arithmetic.

Draw order (numpy PCG64, seed = workload number unless given):
  seq_lens, q_nope, q_rope, W_UK, W_UV, c_KV, k_rope, outlier channels,
  block permutation.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import numpy as np

from .configs import BLOCK_TOKENS, FMT_BITS, POISON_BLOCKS, MlaConfig, block_layout

BF16_NAN = np.uint16(0x7FC0)
F16_NAN_BITS = np.uint16(0x7E00)


def to_bf16_exact(x: np.ndarray) -> np.ndarray:
    """Round float32 draws to the nearest bfloat16 value (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x_bf16_exact: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns of float32 values that are already bf16-exact."""
    return (np.ascontiguousarray(x_bf16_exact, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def quantise_rtn(x: np.ndarray, group: int, bits: int):
    """Asymmetric round-to-nearest quantiser, per token and per group of channels.

    s = fp16((max - min) / (2^b - 1)), s := 1 if it is 0; integer zero-point
    z = clamp(rint(-min / s), 0, 2^b - 1) stored as fp16;
    code = clamp(rint(x / s) + z, 0, 2^b - 1), rint ties to even.
    Returns (codes uint8 [..., d], scale_zero float16 [..., d/group, 2]).
    """
    qmax = (1 << bits) - 1
    d = x.shape[-1]
    xg = x.reshape(x.shape[:-1] + (d // group, group)).astype(np.float64)
    mn = xg.min(axis=-1)
    mx = xg.max(axis=-1)
    s16 = ((mx - mn) / qmax).astype(np.float16)
    s16 = np.where(s16 == 0, np.float16(1.0), s16)
    s = s16.astype(np.float64)
    z = np.clip(np.rint(-mn / s), 0, qmax) + 0.0   # an integer: a zero is stored as +0
    codes = np.clip(np.rint(xg / s[..., None]) + z[..., None], 0, qmax).astype(np.uint8)
    sz = np.stack([s16, z.astype(np.float16)], axis=-1)
    return codes.reshape(x.shape), sz


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack codes little-end first: INT4 element 2j -> low nibble of byte j,
    INT2 element 4j+k -> bits 2k..2k+1 of byte j."""
    per = 8 // bits
    c = codes.reshape(codes.shape[:-1] + (codes.shape[-1] // per, per)).astype(np.uint8)
    out = np.zeros(c.shape[:-1], dtype=np.uint8)
    for k in range(per):
        out |= (c[..., k] << np.uint8(bits * k)).astype(np.uint8)
    return out


def append_rows(cfg: MlaConfig, n: int, seed: int):
    """Seeded new-token rows for the cache writer: c [n, d_c] and k_rope [n, d_r] float32,
    drawn like the workload's cache (N(0,1), the workload's outlier channels scaled), with edge
    rows mixed in: a constant row, an all-negative row, rows of tiny (fp16-subnormal scale) and
    of large magnitude, and rows whose values lie exactly half a quantisation step between two
    INT4 codes (groups [0, 3.75], step 0.25) or two INT2 codes (groups [0, 0.75], step 0.25)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    c = rng.standard_normal((n, cfg.d_c), dtype=np.float32)
    k = rng.standard_normal((n, cfg.d_r), dtype=np.float32)
    if cfg.outliers:
        ch = np.sort(rng.choice(cfg.d_c, cfg.outliers, replace=False))
        c[:, ch] *= np.float32(cfg.outlier_scale)
    edges = []
    for d in (cfg.d_c, cfg.d_r):
        j = np.arange(d)
        tie4 = ((j % 15) + 0.5) * 0.25
        tie4[j % 64 == 0], tie4[j % 64 == 1] = 0.0, 3.75
        tie2 = ((j % 3) + 0.5) * 0.25
        tie2[j % 32 == 0], tie2[j % 32 == 1] = 0.0, 0.75
        edges.append([np.full(d, 0.7), -np.abs(rng.standard_normal(d)) - 0.5, rng.standard_normal(d) * 1e-6,
                      rng.standard_normal(d) * 3e3, tie4, tie2])
    for r, (ec, ek) in enumerate(zip(*edges)):
        if r < n:
            c[r], k[r] = ec, ek
    return c, k


def append_slots(num_blocks: int, n: int, seed: int) -> np.ndarray:
    """n distinct cache slots (block * 64 + position) of a pool of num_blocks blocks, seeded,
    with about one in twenty replaced by -1 or by a slot past the pool (both to be skipped)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    slots = rng.choice(num_blocks * BLOCK_TOKENS, n, replace=False).astype(np.int64)
    bad = rng.random(n) < 0.05
    slots[bad] = np.where(rng.random(int(bad.sum())) < 0.5, -1, num_blocks * BLOCK_TOKENS + 7)
    return slots.astype(np.int32)


def rope_rotate(x: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate interleaved pairs (2i, 2i+1) of x [..., d] by angle pos * base^(-2i/d)."""
    d = x.shape[-1]
    inv = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    ang = pos.astype(np.float64)[..., None] * inv
    cs, sn = np.cos(ang), np.sin(ang)
    x0 = x[..., 0::2].astype(np.float64)
    x1 = x[..., 1::2].astype(np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    out[..., 0::2] = x0 * cs - x1 * sn
    out[..., 1::2] = x0 * sn + x1 * cs
    return out.astype(np.float32)


@dataclass
class MlaInputs:
    cfg: MlaConfig
    seq_lens: np.ndarray            # int32 [B], counts the s_q new tokens too
    q_nope: np.ndarray              # float32 [B, s_q, H, d_n] (bf16-exact for bf16 workloads)
    q_rope: np.ndarray              # float32 [B, s_q, H, d_r] (already rotated)
    w_uk: np.ndarray                # float32 [H, d_n, d_c]
    w_uv: np.ndarray                # float32 [H, d_c, d_v]
    # float caches (logical, unpaged; rows past a sequence's length are 0)
    c: Optional[np.ndarray] = None          # float32 [B, Lmax, d_c]
    k_rope: Optional[np.ndarray] = None     # float32 [B, Lmax, d_r]
    # quantised caches (logical, unpaged)
    c_codes: Optional[np.ndarray] = None    # uint8 [B, Lmax, d_c]
    c_sz: Optional[np.ndarray] = None       # float16 [B, Lmax, d_c/g, 2]  (scale, zero)
    r_codes: Optional[np.ndarray] = None    # uint8 [B, Lmax, d_r]
    r_sz: Optional[np.ndarray] = None       # float16 [B, Lmax, d_r/g_r, 2]
    # paged pool
    pool: Optional[np.ndarray] = None       # uint8 [num_blocks, block_bytes]
    block_table: Optional[np.ndarray] = None  # int32 [B, max_blocks]
    plane_offsets: Optional[Dict[str, int]] = None
    outlier_channels: Optional[np.ndarray] = None

    @property
    def sm_scale(self) -> float:
        return self.cfg.sm_scale

    @property
    def max_len(self) -> int:
        return int(self.seq_lens.max())


def _draw_lens(cfg: MlaConfig, rng, B: int) -> np.ndarray:
    kind = cfg.lens[0]
    if kind == "fixed":
        return np.full(B, cfg.lens[1], dtype=np.int32)
    if kind == "uniform":
        return rng.integers(cfg.lens[1], cfg.lens[2] + 1, size=B).astype(np.int32)
    raise ValueError(kind)


def make_inputs(cfg: MlaConfig, seed: int, B: Optional[int] = None,
                lens: Optional[Sequence[int]] = None, H: Optional[int] = None,
                poison: bool = True, build_pool: bool = True) -> MlaInputs:
    """Draw one workload.  ``B``/``lens``/``H`` override the recipe (smaller test sizes)."""
    if H is not None:
        cfg = cfg.with_(H=H)
    if lens is not None:
        B = len(lens)
    B = cfg.B if B is None else B
    rng = np.random.Generator(np.random.PCG64(seed))
    seq_lens = _draw_lens(cfg, rng, B)
    if lens is not None:
        seq_lens = np.asarray(lens, dtype=np.int32)
    if np.any(seq_lens < cfg.s_q):
        raise ValueError("every sequence must hold at least s_q tokens")
    Lmax = int(seq_lens.max())
    H_, s_q = cfg.H, cfg.s_q
    rnd = to_bf16_exact if cfg.dtype == "bf16" else (lambda a: a.astype(np.float32))

    q_nope = rnd(rng.standard_normal((B, s_q, H_, cfg.d_n), dtype=np.float32))
    q_rope_raw = rng.standard_normal((B, s_q, H_, cfg.d_r), dtype=np.float32)
    w_uk = rnd(rng.standard_normal((H_, cfg.d_n, cfg.d_c), dtype=np.float32) * np.float32(cfg.w_std))
    w_uv = rnd(rng.standard_normal((H_, cfg.d_c, cfg.d_v), dtype=np.float32) * np.float32(cfg.w_std))
    c = rng.standard_normal((B, Lmax, cfg.d_c), dtype=np.float32)
    k_raw = rng.standard_normal((B, Lmax, cfg.d_r), dtype=np.float32)
    outl = None
    if cfg.outliers:
        outl = np.sort(rng.choice(cfg.d_c, cfg.outliers, replace=False))
        c[:, :, outl] *= np.float32(cfg.outlier_scale)
    if cfg.rope_base is not None:
        k_raw = rope_rotate(k_raw, np.arange(Lmax)[None, :].repeat(B, 0), cfg.rope_base)
        qpos = (seq_lens[:, None] - s_q + np.arange(s_q)[None, :])[:, :, None].repeat(H_, 2)
        q_rope_raw = rope_rotate(q_rope_raw, qpos, cfg.rope_base)
    q_rope = rnd(q_rope_raw)
    valid = (np.arange(Lmax)[None, :] < seq_lens[:, None])  # [B, Lmax]

    inp = MlaInputs(cfg=cfg, seq_lens=seq_lens, q_nope=q_nope, q_rope=q_rope, w_uk=w_uk,
                    w_uv=w_uv, outlier_channels=outl)
    if cfg.quantised:
        lb, rb = FMT_BITS[cfg.latent_fmt], FMT_BITS[cfg.rope_fmt]
        parts = [quantise_rtn(c[b], cfg.latent_group, lb) for b in range(B)]
        cc = np.stack([p[0] for p in parts]); csz = np.stack([p[1] for p in parts])
        parts = [quantise_rtn(k_raw[b], cfg.rope_group, rb) for b in range(B)]
        rc = np.stack([p[0] for p in parts]); rsz = np.stack([p[1] for p in parts])
        del parts
        cc[~valid] = 0
        rc[~valid] = 0
        csz[~valid] = 0
        rsz[~valid] = 0
        inp.c_codes, inp.c_sz, inp.r_codes, inp.r_sz = cc, csz, rc, rsz
    else:
        cf = rnd(c)
        kf = rnd(k_raw)
        cf[~valid] = 0
        kf[~valid] = 0
        inp.c, inp.k_rope = cf, kf
    del c, k_raw

    nblk = (seq_lens + BLOCK_TOKENS - 1) // BLOCK_TOKENS
    n_used = int(nblk.sum())
    num_blocks = n_used + POISON_BLOCKS
    perm = rng.permutation(num_blocks).astype(np.int32)
    if not build_pool:
        return inp
    max_blocks = int(nblk.max())
    block_bytes, off = block_layout(cfg)
    poison_id = int(perm[n_used])
    table = np.full((B, max_blocks), poison_id, dtype=np.int32)
    cur = 0
    for b in range(B):
        table[b, : nblk[b]] = perm[cur: cur + nblk[b]]
        cur += nblk[b]
    pool = np.zeros((num_blocks, block_bytes), dtype=np.uint8)
    T = BLOCK_TOKENS

    if not cfg.quantised:
        if cfg.latent_fmt == "bf16":
            row = np.concatenate([bf16_bits(inp.c), bf16_bits(inp.k_rope)], axis=-1)
            nan_row = BF16_NAN
        else:
            row = np.concatenate([inp.c, inp.k_rope], axis=-1).astype(np.float32)
            nan_row = np.float32(np.nan)
        if poison:
            row[~valid] = nan_row
            pool.view(row.dtype)[...] = nan_row
        for b in range(B):
            nb = int(nblk[b])
            pad = np.full((nb * T, row.shape[-1]), nan_row if poison else 0, dtype=row.dtype)
            L = min(nb * T, Lmax)
            pad[:L] = row[b, :L]
            pool[table[b, :nb]] = pad.reshape(nb, -1).view(np.uint8)
    else:
        lb, rb = FMT_BITS[cfg.latent_fmt], FMT_BITS[cfg.rope_fmt]
        planes = {
            "lc": pack_codes(inp.c_codes, lb),
            "ls": np.ascontiguousarray(inp.c_sz).copy().view(np.uint8).reshape(B, Lmax, -1),
            "rc": pack_codes(inp.r_codes, rb),
            "rs": np.ascontiguousarray(inp.r_sz).copy().view(np.uint8).reshape(B, Lmax, -1),
        }
        if poison:
            pool[:] = 0xFF
            for name in ("ls", "rs"):
                planes[name].view(np.uint16)[~valid] = F16_NAN_BITS
            planes["lc"][~valid] = 0xFF
            planes["rc"][~valid] = 0xFF
        for b in range(B):
            nb = int(nblk[b])
            ids = table[b, :nb]
            L = min(nb * T, Lmax)
            for name, arr in planes.items():
                per_tok = arr.shape[-1]
                fill = 0xFF if poison else 0
                pad = np.full((nb * T, per_tok), fill, dtype=np.uint8)
                if poison and name in ("ls", "rs"):
                    pad.view(np.uint16)[...] = F16_NAN_BITS
                pad[:L] = arr[b, :L]
                pool[ids, off[name]: off[name] + T * per_tok] = pad.reshape(nb, T * per_tok)
    inp.pool, inp.block_table, inp.plane_offsets = pool, table, off
    return inp


def workload(name: str, seed: Optional[int] = None, **kw) -> MlaInputs:
    """Inputs of a named workload ('1', '2', '3', '3b', '4', '5') with its default seed."""
    from .configs import CONFIGS, SEEDS
    cfg = CONFIGS[name]
    return make_inputs(cfg, SEEDS[name] if seed is None else seed, **kw)


def attended_pairs(seq_lens: np.ndarray, s_q: int) -> int:
    """Number of (query, cached token) pairs one decode step attends, summed over the batch."""
    L = seq_lens.astype(np.int64)
    return int(sum(int((L - s_q + i + 1).sum()) for i in range(s_q)))


__all__ = ["MlaInputs", "make_inputs", "workload", "quantise_rtn", "pack_codes", "to_bf16_exact", "append_rows",
           "append_slots",
           "bf16_bits", "rope_rotate", "attended_pairs"]
