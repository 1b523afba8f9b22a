"""Every quantised cache layout the decode accepts, for both decode kernel families (marked gpu).

mla_decode_paged accepts an INT4 or INT2 latent with groups of 32 .. 512 channels and an INT4
RoPE key with groups of 32 or 64.  For each of these 20 layouts:
  * mla_dequant_blocks, running each family's own in-loop DMA and dequantisation, equals the
    oracle's RNE_bf16((code - z) * s) bit for bit (block ids outside the pool: zero rows);
  * the decode (16 heads: the pipelined kernel, or the split kernel for INT4 latent groups of
    32; 64 heads: the 4-tile partition kernel; 128 heads: the row-owner kernel) matches the
    oracle's attention over the dequantised cache within 2e-3;
  * a sequence of one token attends exactly that token (P = 1), so its o_lat must equal the
    dequantised latent row bit for bit, through the whole decode and combine.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mla_synth import CONFIGS, make_inputs  # noqa: E402
from tests.gpu_helpers import desc_of, dev, logical_cache, to_device  # noqa: E402
from tests.test_gpu_parity import _decode_stage  # noqa: E402
from tests.test_gpu_precision import _check  # noqa: E402

pytestmark = pytest.mark.gpu

LAYOUTS = [(fmt, lg, rg) for fmt in ("int4", "int2") for lg in (32, 64, 128, 256, 512) for rg in (32, 64)]


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_02_amd as m
    m.lib()
    return m


def _cfg(fmt, lg, rg):
    return CONFIGS["5"].with_(latent_fmt=fmt, latent_group=lg, rope_group=rg, rope_base=None)


def _bits(a):
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("fmt,lg,rg", LAYOUTS)
def test_dequant_every_layout(mla, fmt, lg, rg):
    cfg = _cfg(fmt, lg, rg)
    x = make_inputs(cfg, 81, lens=[1, 64, 65, 130], H=2)
    t = to_device(x)
    nb = x.block_table.shape[1]
    ids = x.block_table.reshape(-1).copy()
    ids = np.concatenate([ids, np.array([-1, x.pool.shape[0]], np.int32)])   # two ids outside the pool
    c, k = logical_cache(x)
    for family in ("partition", "rows"):
        print(f"[case] dequant layout {fmt} g{lg} rope g{rg} {family}", flush=True)
        got = mla.dequant_blocks(t["pool"], desc_of(cfg), torch.from_numpy(ids).to(dev()), family)
        got = got.view(torch.int16).cpu().numpy().view(np.uint16)
        for b, L in enumerate(x.seq_lens):
            blk = got[b * nb:(b + 1) * nb].reshape(-1, cfg.d_c + cfg.d_r)[:L]
            np.testing.assert_array_equal(blk, _bits(np.concatenate([c[b], k[b]], axis=1)))
        assert np.all(got[-2:] == 0)


@pytest.mark.parametrize("fmt,lg,rg", LAYOUTS)
def test_decode_every_layout(mla, fmt, lg, rg):
    cfg = _cfg(fmt, lg, rg)
    for H in (16, 64, 128):
        if H == 64 and (lg, rg) not in ((32, 32), (512, 64)):
            continue
        x = make_inputs(cfg, 82, lens=[1, 70, 333], H=H)
        o, lse, ref_o, ref_lse = _decode_stage(mla, x)
        _check(f"decode layout {fmt} g{lg} rope g{rg} H={H}", o, lse, ref_o, ref_lse)


@pytest.mark.parametrize("fmt,lg,rg", LAYOUTS)
def test_single_token_decode_returns_the_dequantised_row(mla, fmt, lg, rg):
    """L = 1: the softmax is one weight P = exp2(0) = 1 (hi term 1, lo term 0), so o_lat is the
    token's dequantised latent row exactly, for every head, in both families."""
    cfg = _cfg(fmt, lg, rg)
    for H in (16, 128):
        x = make_inputs(cfg, 83, lens=[1] * 6, H=H)
        t = to_device(x)
        q = torch.from_numpy(np.random.default_rng(1).standard_normal((6, 1, H, cfg.d_c), dtype=np.float32))
        q = q.to(torch.bfloat16).to(dev())
        o, _ = mla.decode_paged(q, t["q_rope"], t["pool"], desc_of(cfg), t["block_table"], t["seq_lens"], 1,
                                cfg.sm_scale)
        o = o.cpu().numpy()
        c, _k = logical_cache(x)
        print(f"[case] single token {fmt} g{lg} rope g{rg} H={H}", flush=True)
        for b in range(6):
            want = c[b][0].astype(np.float32)
            np.testing.assert_array_equal(o[b, 0], np.broadcast_to(want, o[b, 0].shape))
