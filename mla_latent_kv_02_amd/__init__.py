"""libmla for MI355X: MLA decode over a paged latent KV cache (bf16 / INT4 / INT2).

Thin Python binding over the C ABI in include/libmla.h.  Every step of the
decode runs in the library's HIP kernels; this module only checks tensors and
passes pointers and the current HIP stream.  PyTorch provides device memory
and streams.  Importing works without a GPU; calling needs the built
libmla.so (``python -m mla_latent_kv_02_amd.build``) and an MI355X.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from . import _lib
from ._lib import (MLA_BF16, MLA_F32, MLA_FMT_BF16, MLA_FMT_F32, MLA_FMT_INT2, MLA_FMT_INT4,  # noqa: F401
                   CacheDesc, DecodeArgs, FMT_BY_NAME)

__all__ = ["MlaError", "cache_desc", "block_bytes", "plane_offsets", "absorb_q", "decode_paged", "out_proj",
           "decode_mixed", "dequant_blocks", "append_kv", "hadamard_rotate", "decode_workspace_size",
           "decode_plan", "DecodeStep", "gqa_block_bytes", "gqa_expand", "gqa_decode_paged", "lib"]


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.load().mla_status_string(status).decode()
        super().__init__(f"{where}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    return _lib.load()


def _check(status: int, where: str) -> None:
    if status != _lib.MLA_OK:
        raise MlaError(status, where)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MLA_F32
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_cuda(*ts: torch.Tensor) -> None:
    for t in ts:
        if not t.is_cuda:
            raise ValueError("libmla operates on GPU tensors")


def cache_desc(d_c: int = 512, d_r: int = 64, latent_fmt="bf16", rope_fmt=None, latent_group: int = 0,
               rope_group: int = 0) -> CacheDesc:
    lf = FMT_BY_NAME[latent_fmt] if isinstance(latent_fmt, str) else int(latent_fmt)
    rf = lf if rope_fmt is None else (FMT_BY_NAME[rope_fmt] if isinstance(rope_fmt, str) else int(rope_fmt))
    return CacheDesc(d_c, d_r, 64, lf, rf, latent_group, rope_group)


def block_bytes(desc: CacheDesc) -> int:
    return int(_lib.load().mla_cache_block_bytes(ctypes.byref(desc)))


def plane_offsets(desc: CacheDesc):
    off = (ctypes.c_int64 * 4)()
    _check(_lib.load().mla_cache_plane_offsets(ctypes.byref(desc), off), "mla_cache_plane_offsets")
    return list(off)


def _proj(fn, name, x, w, out_dtype, out):
    # x [N, H, K] (strided rows allowed, unit stride along K), w [H, K, M] dense
    _need_cuda(x, w)
    if x.dim() != 3 or w.dim() != 3 or x.shape[1] != w.shape[0] or x.shape[2] != w.shape[1]:
        raise ValueError(f"{name}: shapes {tuple(x.shape)} x {tuple(w.shape)} do not match")
    if x.stride(2) != 1:
        x = x.contiguous()
    w = w.contiguous()
    N, H, K = x.shape
    M = w.shape[2]
    if out is None:
        out = torch.empty((N, H, M), dtype=out_dtype, device=x.device)
    if not out.is_contiguous() or out.shape != (N, H, M):
        raise ValueError(f"{name}: out must be a dense [N, H, M] tensor")
    st = fn(ctypes.c_void_p(x.data_ptr()), x.stride(0), x.stride(1), _dt(x), ctypes.c_void_p(w.data_ptr()),
            _dt(w), ctypes.c_void_p(out.data_ptr()), _dt(out), N, H, K, M, _stream(x.device))
    _check(st, name)
    return out


def absorb_q(q_nope: torch.Tensor, w_uk: torch.Tensor, out_dtype=torch.bfloat16,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """q_lat[n, h, :] = q_nope[n, h, :] @ W_UK[h]; q_nope [N, H, d_n], w_uk [H, d_n, d_c]."""
    return _proj(_lib.load().mla_absorb_q, "mla_absorb_q", q_nope, w_uk, out_dtype, out)


def out_proj(o_lat: torch.Tensor, w_uv: torch.Tensor, out_dtype=torch.float32,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[n, h, :] = o_lat[n, h, :] @ W_UV[h]; o_lat [N, H, d_c], w_uv [H, d_c, d_v]."""
    return _proj(_lib.load().mla_out_proj, "mla_out_proj", o_lat, w_uv, out_dtype, out)


def _decode_args(q_lat, q_rope, pool, desc, block_table, seq_lens, max_seq_len, sm_scale, num_splits,
                 o_lat, lse, workspace, total_seq_len=0) -> DecodeArgs:
    B, s_q, H, d_c = q_lat.shape
    a = DecodeArgs()
    a.q_lat = q_lat.data_ptr()
    a.q_rope = q_rope.data_ptr()
    a.q_dtype = _dt(q_lat)
    a.cache_pool = pool.data_ptr()
    a.num_blocks = pool.shape[0]
    a.cache = desc
    a.block_table = block_table.data_ptr()
    a.block_table_stride = block_table.shape[1]
    a.seq_lens = seq_lens.data_ptr()
    a.max_seq_len = int(max_seq_len)
    a.total_seq_len = int(total_seq_len)
    a.batch, a.s_q, a.num_heads = B, s_q, H
    a.sm_scale = float(sm_scale)
    a.num_splits = int(num_splits)
    a.o_lat = o_lat.data_ptr() if o_lat is not None else 1 << 12
    a.o_dtype = _dt(o_lat) if o_lat is not None else MLA_F32
    a.lse = lse.data_ptr() if lse is not None else None
    a.workspace = workspace.data_ptr() if workspace is not None else None
    a.workspace_bytes = workspace.numel() if workspace is not None else 0
    return a


def _check_out(t, shape, dtypes, device, name):
    """An output the kernels write densely: exact shape, dtype, dense, on the inputs' device."""
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if tuple(t.shape) != tuple(shape) or t.dtype not in dtypes or not t.is_contiguous():
        raise ValueError(f"{name} must be a dense {list(shape)} tensor of {[str(d) for d in dtypes]}, "
                         f"got {list(t.shape)} {t.dtype}")


def _check_pool(pool, desc, name):
    if pool.dtype != torch.uint8 or pool.dim() != 2 or not pool.is_contiguous() or pool.shape[1] != block_bytes(desc):
        raise ValueError(f"{name}: pool must be a dense uint8 [num_blocks, {block_bytes(desc)}] tensor")


def _check_decode_tensors(q_lat, q_rope, pool, desc, block_table, seq_lens):
    _need_cuda(q_lat, q_rope, pool, block_table, seq_lens)
    if q_lat.dim() != 4 or q_rope.dim() != 4 or q_lat.shape[:3] != q_rope.shape[:3]:
        raise ValueError("q_lat [B, s_q, H, d_c] and q_rope [B, s_q, H, d_r] expected")
    if q_lat.shape[3] != desc.d_c or q_rope.shape[3] != desc.d_r:
        raise ValueError("q widths do not match the cache descriptor")
    if q_lat.dtype != q_rope.dtype or not q_lat.is_contiguous() or not q_rope.is_contiguous():
        raise ValueError("q_lat and q_rope must be dense and of one dtype")
    if pool.dtype != torch.uint8 or pool.dim() != 2 or not pool.is_contiguous() or pool.shape[1] != block_bytes(desc):
        raise ValueError("pool must be a dense uint8 [num_blocks, block_bytes] tensor")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be dense int32 [B, max_blocks]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (q_lat.shape[0],):
        raise ValueError("seq_lens must be int32 [B]")


def decode_workspace_size(q_lat, q_rope, pool, desc, block_table, seq_lens, max_seq_len, sm_scale,
                          num_splits: int = 0, total_seq_len: int = 0) -> int:
    a = _decode_args(q_lat, q_rope, pool, desc, block_table, seq_lens, max_seq_len, sm_scale, num_splits,
                     None, None, None, total_seq_len)
    n = ctypes.c_size_t()
    _check(_lib.load().mla_decode_workspace_size(ctypes.byref(a), ctypes.byref(n)), "mla_decode_workspace_size")
    return int(n.value)


def decode_plan(q_lat, q_rope, pool, desc, block_table, seq_lens, max_seq_len, sm_scale, num_splits: int = 0,
                num_cus: int = 0, total_seq_len: int = 0) -> Tuple[int, int]:
    a = _decode_args(q_lat, q_rope, pool, desc, block_table, seq_lens, max_seq_len, sm_scale, num_splits,
                     None, None, None, total_seq_len)
    s, t = ctypes.c_int32(), ctypes.c_int32()
    _check(_lib.load().mla_decode_plan(ctypes.byref(a), num_cus, ctypes.byref(s), ctypes.byref(t)), "mla_decode_plan")
    return s.value, t.value


def decode_paged(q_lat: torch.Tensor, q_rope: torch.Tensor, pool: torch.Tensor, desc: CacheDesc,
                 block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, sm_scale: float,
                 num_splits: int = 0, o_dtype=torch.float32, out: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                 want_lse: bool = True, total_seq_len: int = 0):
    """Absorbed-form attention over the paged latent cache.  Returns (o_lat, lse)."""
    _check_decode_tensors(q_lat, q_rope, pool, desc, block_table, seq_lens)
    B, s_q, H, d_c = q_lat.shape
    if out is None:
        out = torch.empty((B, s_q, H, d_c), dtype=o_dtype, device=q_lat.device)
    if lse is None and want_lse:
        lse = torch.empty((B, s_q, H), dtype=torch.float32, device=q_lat.device)
    _check_out(out, (B, s_q, H, d_c), (torch.float32, torch.bfloat16), q_lat.device, "o_lat")
    if lse is not None:
        _check_out(lse, (B, s_q, H), (torch.float32,), q_lat.device, "lse")
    if workspace is None:
        n = decode_workspace_size(q_lat, q_rope, pool, desc, block_table, seq_lens, max_seq_len, sm_scale,
                                  num_splits, total_seq_len)
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=q_lat.device)
    a = _decode_args(q_lat, q_rope, pool, desc, block_table, seq_lens, max_seq_len, sm_scale, num_splits,
                     out, lse, workspace, total_seq_len)
    _check(_lib.load().mla_decode_paged(ctypes.byref(a), _stream(q_lat.device)), "mla_decode_paged")
    return out, lse


def decode_mixed(q_lat: torch.Tensor, q_rope: torch.Tensor, sink, middle, recent, sm_scale: float,
                 o_dtype=torch.float32, num_splits: int = 0):
    """One decode over a history kept in up to three caches: sink ++ middle ++ recent per
    sequence (e.g. bf16 sink and recent window, low-bit middle).  Each part is None or
    (pool, desc, block_table, seq_lens, max_seq_len) for that part's tokens; the recent part
    ends with the s_q new tokens and carries the causal mask.  Returns (o_lat, lse)."""
    parts = []
    for part in (sink, middle, recent):
        if part is None:
            parts.append(None)
            continue
        pool, desc, bt, sl, mx = part
        _check_decode_tensors(q_lat, q_rope, pool, desc, bt, sl)
        parts.append(_decode_args(q_lat, q_rope, pool, desc, bt, sl, mx, sm_scale, num_splits, None, None, None))
    refs = [ctypes.byref(a) if a is not None else None for a in parts]
    L = _lib.load()
    n = ctypes.c_size_t()
    _check(L.mla_decode_mixed_workspace_size(*refs, ctypes.byref(n)), "mla_decode_mixed_workspace_size")
    B, s_q, H, d_c = q_lat.shape
    out = torch.empty((B, s_q, H, d_c), dtype=o_dtype, device=q_lat.device)
    lse = torch.empty((B, s_q, H), dtype=torch.float32, device=q_lat.device)
    ws = torch.empty(max(n.value, 256), dtype=torch.uint8, device=q_lat.device)
    _check(L.mla_decode_mixed(*refs, ctypes.c_void_p(out.data_ptr()), _dt(out), ctypes.c_void_p(lse.data_ptr()),
                              ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(q_lat.device)), "mla_decode_mixed")
    return out, lse


def dequant_blocks(pool: torch.Tensor, desc: CacheDesc, block_ids: torch.Tensor, family: str = "partition") -> torch.Tensor:
    """bf16 [n, 64, d_c + d_r] view of cache blocks as a decode kernel family ('partition' or
    'rows') dequantises them in its attention loop (its own DMA and dequant routine)."""
    _need_cuda(pool, block_ids)
    _check_pool(pool, desc, "dequant_blocks")
    if block_ids.dtype != torch.int32 or not block_ids.is_contiguous():
        raise ValueError("block_ids must be dense int32")
    n = block_ids.numel()
    out = torch.empty((n, 64, desc.d_c + desc.d_r), dtype=torch.bfloat16, device=pool.device)
    st = _lib.load().mla_dequant_blocks(ctypes.c_void_p(pool.data_ptr()), pool.shape[0], ctypes.byref(desc),
                                        ctypes.c_void_p(block_ids.data_ptr()), n, _lib.DEQUANT_FAMILY[family],
                                        ctypes.c_void_p(out.data_ptr()), _stream(pool.device))
    _check(st, "mla_dequant_blocks")
    return out


def append_kv(c_new: torch.Tensor, k_rope_new: torch.Tensor, pool: torch.Tensor, desc: CacheDesc,
              slots: torch.Tensor) -> None:
    """Write n new tokens into their cache slots (block * 64 + position), quantising for
    INT4/INT2 caches: c_new [n, d_c] and k_rope_new [n, d_r] of one dtype (bf16 or fp32,
    rows may be strided), slots int32 [n] (negative = skip).  pool [num_blocks, block_bytes]
    uint8 is updated in place on the current stream."""
    _need_cuda(c_new, k_rope_new, pool, slots)
    _check_pool(pool, desc, "append_kv")
    if c_new.dim() != 2 or k_rope_new.dim() != 2 or c_new.shape[0] != k_rope_new.shape[0]:
        raise ValueError("c_new and k_rope_new must be [n, d] with the same n")
    if c_new.shape[1] != desc.d_c or k_rope_new.shape[1] != desc.d_r:
        raise ValueError(f"c_new [n, {desc.d_c}] and k_rope_new [n, {desc.d_r}] expected by the descriptor")
    if c_new.dtype != k_rope_new.dtype:
        raise ValueError("c_new and k_rope_new must share a dtype")
    if c_new.stride(1) != 1 or k_rope_new.stride(1) != 1:
        raise ValueError("rows must be dense")
    if slots.dtype != torch.int32 or not slots.is_contiguous() or slots.numel() != c_new.shape[0]:
        raise ValueError("slots must be dense int32 [n]")
    n = c_new.shape[0]
    st = _lib.load().mla_append_kv(ctypes.c_void_p(c_new.data_ptr()), c_new.stride(0) if n > 1 else c_new.shape[1],
                                   ctypes.c_void_p(k_rope_new.data_ptr()),
                                   k_rope_new.stride(0) if n > 1 else k_rope_new.shape[1], _dt(c_new),
                                   ctypes.c_void_p(slots.data_ptr()), n, ctypes.c_void_p(pool.data_ptr()),
                                   pool.shape[0], ctypes.byref(desc), _stream(pool.device))
    _check(st, "mla_append_kv")


def gqa_block_bytes(num_groups: int, d_n: int = 128, d_v: int = 128, d_r: int = 64) -> int:
    """Bytes of one 64-token block of the GQLA per-group expanded cache."""
    return int(_lib.load().mla_gqa_block_bytes(num_groups, d_n, d_v, d_r))


def gqa_expand(c_new: torch.Tensor, k_rope_new: torch.Tensor, w_uk_g: torch.Tensor, w_uv_g: torch.Tensor,
               pool: torch.Tensor, slots: torch.Tensor) -> None:
    """Write n new tokens into the per-group expanded cache: c_new [n, d_c] and k_rope_new [n, d_r]
    bf16 (rows may be strided), w_uk_g [G, d_n, d_c], w_uv_g [G, d_c, d_v] bf16, slots int32 [n]
    (block * 64 + position; outside the pool = skip).  pool [num_blocks, block_bytes] uint8."""
    _need_cuda(c_new, k_rope_new, w_uk_g, w_uv_g, pool, slots)
    G, d_n, d_c = w_uk_g.shape
    d_v = w_uv_g.shape[2]
    d_r = k_rope_new.shape[1]
    if w_uv_g.shape[:2] != (G, d_c) or c_new.dim() != 2 or c_new.shape[1] != d_c:
        raise ValueError("gqa_expand: c_new [n, d_c], w_uk_g [G, d_n, d_c] and w_uv_g [G, d_c, d_v] expected")
    if c_new.shape[0] != k_rope_new.shape[0] or slots.numel() != c_new.shape[0]:
        raise ValueError("gqa_expand: one slot and one RoPE key per token")
    for t in (c_new, k_rope_new, w_uk_g, w_uv_g):
        if t.dtype != torch.bfloat16:
            raise ValueError("gqa_expand: bf16 inputs")
    if c_new.stride(1) != 1 or k_rope_new.stride(1) != 1 or not w_uk_g.is_contiguous() or not w_uv_g.is_contiguous():
        raise ValueError("gqa_expand: rows and weights must be dense")
    if slots.dtype != torch.int32 or not slots.is_contiguous():
        raise ValueError("gqa_expand: slots must be dense int32")
    bb = gqa_block_bytes(G, d_n, d_v, d_r)
    if pool.dtype != torch.uint8 or pool.dim() != 2 or not pool.is_contiguous() or pool.shape[1] != bb:
        raise ValueError(f"gqa_expand: pool must be a dense uint8 [num_blocks, {bb}] tensor")
    n = c_new.shape[0]
    st = _lib.load().mla_gqa_expand(ctypes.c_void_p(c_new.data_ptr()), c_new.stride(0) if n > 1 else d_c,
                                    ctypes.c_void_p(k_rope_new.data_ptr()), k_rope_new.stride(0) if n > 1 else d_r,
                                    ctypes.c_void_p(w_uk_g.data_ptr()), ctypes.c_void_p(w_uv_g.data_ptr()), G, d_c,
                                    d_n, d_v, d_r, ctypes.c_void_p(slots.data_ptr()), n,
                                    ctypes.c_void_p(pool.data_ptr()), pool.shape[0], _stream(pool.device))
    _check(st, "mla_gqa_expand")


def _gqa_args(q_nope, q_rope, pool, num_groups, block_table, seq_lens, max_seq_len, sm_scale, num_splits, out, lse,
              workspace, total_seq_len, d_v=128):
    B, s_q, H, d_n = q_nope.shape
    a = _lib.GqaArgs()
    a.q_nope, a.q_rope, a.cache_pool = q_nope.data_ptr(), q_rope.data_ptr(), pool.data_ptr()
    a.num_blocks = pool.shape[0]
    a.num_groups, a.d_n, a.d_v, a.d_r = num_groups, d_n, d_v, q_rope.shape[3]
    a.block_table, a.block_table_stride = block_table.data_ptr(), block_table.shape[1]
    a.seq_lens, a.max_seq_len, a.total_seq_len = seq_lens.data_ptr(), int(max_seq_len), int(total_seq_len)
    a.batch, a.s_q, a.num_heads = B, s_q, H
    a.sm_scale, a.num_splits = float(sm_scale), int(num_splits)
    a.out = out.data_ptr() if out is not None else 1 << 12
    a.lse = lse.data_ptr() if lse is not None else None
    a.workspace = workspace.data_ptr() if workspace is not None else None
    a.workspace_bytes = workspace.numel() if workspace is not None else 0
    return a


def gqa_decode_paged(q_nope: torch.Tensor, q_rope: torch.Tensor, pool: torch.Tensor, num_groups: int,
                     block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, sm_scale: float,
                     num_splits: int = 0, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, total_seq_len: int = 0, d_v: int = 128):
    """GQLA's GQA decode over the per-group expanded cache: q_nope [B, s_q, H, d_n], q_rope
    [B, s_q, H, d_r] bf16; returns (out [B, s_q, H, d_v] fp32, lse [B, s_q, H])."""
    _need_cuda(q_nope, q_rope, pool, block_table, seq_lens)
    if q_nope.dim() != 4 or q_rope.dim() != 4 or q_nope.shape[:3] != q_rope.shape[:3]:
        raise ValueError("q_nope [B, s_q, H, d_n] and q_rope [B, s_q, H, d_r] expected")
    if q_nope.dtype != torch.bfloat16 or q_rope.dtype != torch.bfloat16:
        raise ValueError("bf16 queries expected")
    if not q_nope.is_contiguous() or not q_rope.is_contiguous():
        raise ValueError("queries must be dense")
    bb = gqa_block_bytes(num_groups, q_nope.shape[3], d_v, q_rope.shape[3])
    if pool.dtype != torch.uint8 or pool.dim() != 2 or not pool.is_contiguous() or pool.shape[1] != bb:
        raise ValueError(f"pool must be a dense uint8 [num_blocks, {bb}] tensor")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be dense int32 [B, max_blocks]")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (q_nope.shape[0],):
        raise ValueError("seq_lens must be int32 [B]")
    B, s_q, H, _ = q_nope.shape
    if out is None:
        out = torch.empty((B, s_q, H, d_v), dtype=torch.float32, device=q_nope.device)
    if lse is None:
        lse = torch.empty((B, s_q, H), dtype=torch.float32, device=q_nope.device)
    _check_out(out, (B, s_q, H, d_v), (torch.float32,), q_nope.device, "out")
    _check_out(lse, (B, s_q, H), (torch.float32,), q_nope.device, "lse")
    L = _lib.load()
    if workspace is None:
        a = _gqa_args(q_nope, q_rope, pool, num_groups, block_table, seq_lens, max_seq_len, sm_scale, num_splits,
                      out, lse, None, total_seq_len, d_v)
        n = ctypes.c_size_t()
        _check(L.mla_gqa_workspace_size(ctypes.byref(a), ctypes.byref(n)), "mla_gqa_workspace_size")
        workspace = torch.empty(max(n.value, 256), dtype=torch.uint8, device=q_nope.device)
    a = _gqa_args(q_nope, q_rope, pool, num_groups, block_table, seq_lens, max_seq_len, sm_scale, num_splits,
                  out, lse, workspace, total_seq_len, d_v)
    _check(L.mla_gqa_decode_paged(ctypes.byref(a), _stream(q_nope.device)), "mla_gqa_decode_paged")
    return out, lse


def hadamard_rotate(x: torch.Tensor, dim: int = -1) -> torch.Tensor:
    """In place, x <- x . H_d / sqrt(d) along axis dim (d = x.shape[dim], a power of two):
    the Walsh-Hadamard rotation, its own inverse.  x is bf16 or fp32; every other axis is
    flattened into the vector index, so x must be a strided view whose other axes can be
    traversed as (outer, inner) pairs: the axes before dim with one stride, those after it
    with another (true of any contiguous tensor).  Returns x."""
    _need_cuda(x)
    dim = dim % x.dim()
    d = x.shape[dim]
    before, after = x.shape[:dim], x.shape[dim + 1:]
    n_outer = 1
    for v in before:
        n_outer *= v
    n_inner = 1
    for v in after:
        n_inner *= v
    # the axes before dim must collapse to one stride, and so must those after it
    def collapsed_stride(axes):
        st = None
        for a in range(len(axes) - 1, -1, -1):
            if x.shape[axes[a]] == 1:
                continue
            s_a = x.stride(axes[a])
            if st is None:
                st, span = s_a, x.shape[axes[a]] * s_a
            elif s_a != span:
                raise ValueError("axes around dim do not collapse to one stride; make x contiguous")
            else:
                span = x.shape[axes[a]] * s_a
        return 0 if st is None else st
    outer_stride = collapsed_stride(list(range(dim)))
    inner_stride = collapsed_stride(list(range(dim + 1, x.dim())))
    st = _lib.load().mla_hadamard_rotate(ctypes.c_void_p(x.data_ptr()), _dt(x), d, x.stride(dim), n_outer,
                                         outer_stride, max(n_inner, 1), inner_stride, _stream(x.device))
    _check(st, "mla_hadamard_rotate")
    return x


@dataclass
class DecodeStep:
    """One MLA decode step with preallocated buffers: absorb -> paged decode -> out_proj.

    q_nope [B, s_q, H, d_n], q_rope [B, s_q, H, d_r] (bf16 or fp32), w_uk [H, d_n, d_c],
    w_uv [H, d_c, d_v].  ``run`` enqueues the three library calls on the current stream
    and returns out [B, s_q, H, d_v] (fp32).
    """
    w_uk: torch.Tensor
    w_uv: torch.Tensor
    desc: CacheDesc
    batch: int
    s_q: int
    max_seq_len: int
    sm_scale: float
    num_splits: int = 0
    q_lat_dtype: torch.dtype = torch.bfloat16
    total_seq_len: int = 0

    def __post_init__(self):
        H, d_n, d_c = self.w_uk.shape
        d_v = self.w_uv.shape[2]
        dev = self.w_uk.device
        N = self.batch * self.s_q
        self.H, self.d_n, self.d_c, self.d_v = H, d_n, d_c, d_v
        self.q_lat = torch.empty((N, H, d_c), dtype=self.q_lat_dtype, device=dev)
        self.o_lat = torch.empty((self.batch, self.s_q, H, d_c), dtype=torch.float32, device=dev)
        self.lse = torch.empty((self.batch, self.s_q, H), dtype=torch.float32, device=dev)
        self.out = torch.empty((N, H, d_v), dtype=torch.float32, device=dev)
        self.workspace = None

    def run(self, q_nope, q_rope, pool, block_table, seq_lens):
        B, s_q, H = self.batch, self.s_q, self.H
        absorb_q(q_nope.view(B * s_q, H, self.d_n), self.w_uk, out=self.q_lat)
        ql = self.q_lat.view(B, s_q, H, self.d_c)
        if self.workspace is None:
            n = decode_workspace_size(ql, q_rope, pool, self.desc, block_table, seq_lens, self.max_seq_len,
                                      self.sm_scale, self.num_splits, self.total_seq_len)
            self.workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=pool.device)
        decode_paged(ql, q_rope, pool, self.desc, block_table, seq_lens, self.max_seq_len, self.sm_scale,
                     self.num_splits, out=self.o_lat, lse=self.lse, workspace=self.workspace,
                     total_seq_len=self.total_seq_len)
        out_proj(self.o_lat.view(B * s_q, H, self.d_c), self.w_uv, out=self.out)
        return self.out.view(B, s_q, H, self.d_v)

    def capture(self, q_nope, q_rope, pool, block_table, seq_lens) -> "torch.cuda.CUDAGraph":
        """Record one step on these tensors into a HIP graph; ``graph.replay()`` re-runs it.

        The three library calls only launch kernels (no allocation, no memset), so the
        captured step is the same work as ``run``.  Buffers are the step's own and must
        not be freed while the graph is alive.
        """
        self.run(q_nope, q_rope, pool, block_table, seq_lens)  # sizes the workspace outside capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run(q_nope, q_rope, pool, block_table, seq_lens)
        return g
