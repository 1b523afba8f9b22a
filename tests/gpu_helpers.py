"""Shared helpers of the GPU tests: move generated inputs to the device, build oracle references.

The oracle side only ever sees numpy arrays made by mla_synth or by the oracle itself;
nothing the GPU computed is used as an expected value, except where a stage's oracle
is deliberately fed that stage's actual bf16 input (stage-wise parity).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import mla_latent_kv_02_amd as mla
from mla_synth import MlaInputs


def dev():
    return torch.device("cuda:0")


def desc_of(cfg):
    return mla.cache_desc(cfg.d_c, cfg.d_r, cfg.latent_fmt, cfg.rope_fmt, cfg.latent_group, cfg.rope_group)


def tdtype(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def to_device(x: MlaInputs):
    d = dev()
    dt = tdtype(x.cfg)
    return {
        "pool": torch.from_numpy(x.pool).to(d),
        "block_table": torch.from_numpy(x.block_table).to(d),
        "seq_lens": torch.from_numpy(x.seq_lens).to(d),
        "q_nope": torch.from_numpy(x.q_nope).to(dt).to(d),
        "q_rope": torch.from_numpy(x.q_rope).to(dt).to(d),
        "w_uk": torch.from_numpy(x.w_uk).to(dt).to(d),
        "w_uv": torch.from_numpy(x.w_uv).to(dt).to(d),
    }


def logical_cache(x: MlaInputs):
    """Per-sequence float64 latent and RoPE key as the oracle sees them (dequantised if needed)."""
    cfg = x.cfg
    B = len(x.seq_lens)
    if cfg.quantised:
        cc = [x.c_codes[b, :L] for b, L in enumerate(x.seq_lens)]
        cs = [x.c_sz[b, :L] for b, L in enumerate(x.seq_lens)]
        rc = [x.r_codes[b, :L] for b, L in enumerate(x.seq_lens)]
        rs = [x.r_sz[b, :L] for b, L in enumerate(x.seq_lens)]
        return oracle.dequant_cache(cc, cs, rc, rs, cfg.latent_group, cfg.rope_group)
    return ([x.c[b, :L].astype(np.float64) for b, L in enumerate(x.seq_lens)],
            [x.k_rope[b, :L].astype(np.float64) for b, L in enumerate(x.seq_lens)])


def norm_err(got, ref) -> float:
    """max |got - ref| / max |ref| over finite reference entries."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    m = np.isfinite(ref)
    den = np.max(np.abs(ref[m])) if m.any() else 1.0
    return float(np.max(np.abs(got[m] - ref[m])) / max(den, 1e-30))


def bf16_exact(a: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 through torch (input preparation for a bf16 stage)."""
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
