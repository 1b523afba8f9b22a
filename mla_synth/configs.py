"""Synthetic MLA-decode workloads (shapes, value distributions, cache formats).

Each workload stands in for a model/context setting the pages talk about
(DeepSeek-V2-Lite and DeepSeek-V3 shapes, 32K and 128K contexts, INT4 and
INT2 latent caches).  No model weights or datasets are involved: every tensor
is drawn from a seeded numpy PCG64 generator by ``mla_synth.gen``.

This module holds only shapes and recipes; it computes nothing of the method.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional, Tuple

BLOCK_TOKENS = 64          # tokens per paged cache block
POISON_BLOCKS = 16         # extra NaN-filled blocks appended to every pool


@dataclass(frozen=True)
class MlaConfig:
    name: str
    B: int                 # sequences in the batch
    H: int                 # attention heads
    d_c: int               # latent width (c_KV)
    d_r: int               # decoupled RoPE key width
    d_n: int               # no-RoPE query/key width (nope)
    d_v: int               # value width per head
    s_q: int               # query tokens per sequence (1, or 2 for MTP-style decode)
    dtype: str             # 'f32' or 'bf16': dtype of q, weights and float caches
    latent_fmt: str        # 'f32' | 'bf16' | 'int4' | 'int2'
    rope_fmt: str          # 'f32' | 'bf16' | 'int4'
    latent_group: int = 0  # channels per quantisation group of the latent (quantised formats)
    rope_group: int = 0    # channels per quantisation group of the RoPE key
    lens: Tuple = ("fixed", 256)   # ('fixed', L) or ('uniform', lo, hi) inclusive
    outliers: int = 0      # latent channels multiplied by outlier_scale
    outlier_scale: float = 20.0
    rope_base: Optional[float] = None   # rotate k_rope / q_rope by position with this base
    weight_std: Optional[float] = None  # std of W_UK / W_UV entries (default 1/sqrt(d_c))

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_n + self.d_r)

    @property
    def w_std(self) -> float:
        return self.weight_std if self.weight_std is not None else 1.0 / math.sqrt(self.d_c)

    @property
    def quantised(self) -> bool:
        return self.latent_fmt in ("int4", "int2")

    def with_(self, **kw) -> "MlaConfig":
        return replace(self, **kw)


# The five workloads.  Seeds default to the workload number (3 and 3b share 3).
CONFIGS = {
    # Tiny fp32 case: the absorbed and unabsorbed forms are compared directly.
    "1": MlaConfig("tiny-f32", B=1, H=8, d_c=64, d_r=16, d_n=32, d_v=32, s_q=1,
                   dtype="f32", latent_fmt="f32", rope_fmt="f32", lens=("fixed", 256),
                   weight_std=1.0 / math.sqrt(64)),
    # DeepSeek-V2-Lite-shaped bf16 decode, every sequence 4096 tokens.
    "2": MlaConfig("v2lite-bf16", B=32, H=16, d_c=512, d_r=64, d_n=128, d_v=128, s_q=1,
                   dtype="bf16", latent_fmt="bf16", rope_fmt="bf16", lens=("fixed", 4096)),
    # DeepSeek-V3-shaped bf16 decode, lengths uniform in [1024, 8192]; s_q = 1 and 2.
    "3": MlaConfig("v3-bf16-sq1", B=64, H=128, d_c=512, d_r=64, d_n=128, d_v=128, s_q=1,
                   dtype="bf16", latent_fmt="bf16", rope_fmt="bf16", lens=("uniform", 1024, 8192)),
    "3b": MlaConfig("v3-bf16-sq2", B=64, H=128, d_c=512, d_r=64, d_n=128, d_v=128, s_q=2,
                    dtype="bf16", latent_fmt="bf16", rope_fmt="bf16", lens=("uniform", 1024, 8192)),
    # Joint INT4 cache (latent and RoPE key), V2-Lite heads, 32K context, 8 outlier channels.
    "4": MlaConfig("v2lite-int4-32k", B=16, H=16, d_c=512, d_r=64, d_n=128, d_v=128, s_q=1,
                   dtype="bf16", latent_fmt="int4", rope_fmt="int4", latent_group=64,
                   rope_group=64, lens=("fixed", 32768), outliers=8),
    # INT2 latent + INT4 RoPE key, V3 heads, 128K context, 16 outlier channels, RoPE base 1e4.
    "5": MlaConfig("v3-int2-128k", B=4, H=128, d_c=512, d_r=64, d_n=128, d_v=128, s_q=1,
                   dtype="bf16", latent_fmt="int2", rope_fmt="int4", latent_group=32,
                   rope_group=64, lens=("fixed", 131072), outliers=16, rope_base=10000.0),
}

SEEDS = {"1": 1, "2": 2, "3": 3, "3b": 3, "4": 4, "5": 5}

FMT_BITS = {"int4": 4, "int2": 2}
FMT_ELEM_BYTES = {"f32": 4, "bf16": 2}


def _align16(n: int) -> int:
    return (n + 15) // 16 * 16


def block_layout(cfg: MlaConfig):
    """Byte layout of one paged block: returns (block_bytes, plane offsets dict).

    Float caches: one plane, rows of [latent | rope] per token.
    Quantised caches: four 16-byte-aligned planes per block,
      'lc' latent codes      [64][d_c*bits/8] (element 2j in the low nibble of byte j;
                                             INT2 element 4j+k in bits 2k..2k+1),
      'ls' latent scale/zero [64][d_c/g][2] fp16,
      'rc' rope codes        [64][d_r*bits/8],
      'rs' rope scale/zero   [64][d_r/g_r][2] fp16.
    """
    T = BLOCK_TOKENS
    if not cfg.quantised:
        eb = FMT_ELEM_BYTES[cfg.latent_fmt]
        return T * (cfg.d_c + cfg.d_r) * eb, {"row": 0}
    lb = FMT_BITS[cfg.latent_fmt]
    rb = FMT_BITS[cfg.rope_fmt]
    lc = T * cfg.d_c * lb // 8
    ls = T * (cfg.d_c // cfg.latent_group) * 4
    rc = T * cfg.d_r * rb // 8
    rs = T * (cfg.d_r // cfg.rope_group) * 4
    off = {}
    pos = 0
    for name, size in (("lc", lc), ("ls", ls), ("rc", rc), ("rs", rs)):
        off[name] = pos
        pos += _align16(size)
    return pos, off
