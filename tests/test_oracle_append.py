"""Pins of the oracle's cache writer (CPU).

write_tokens is checked against the input generator's own, independently written pieces
(its quantiser, its code packer, its bf16 rounding and its block layout), against its own
reader (round trip), against the closed form of ties-to-even rounding, and for slots it
must skip.
"""
import numpy as np
import pytest

import oracle
from mla_synth import CONFIGS, append_rows, append_slots, bf16_bits, block_layout, pack_codes, quantise_rtn, \
    to_bf16_exact

N_BLOCKS = 6


def _fmt_args(cfg):
    return (cfg.latent_fmt, cfg.rope_fmt, cfg.d_c, cfg.d_r, cfg.latent_group, cfg.rope_group)


def _generator_pool(cfg, slots, c, k):
    """The same writes assembled from the input generator's pieces."""
    bb, off = block_layout(cfg)
    pool = np.zeros((N_BLOCKS, bb), dtype=np.uint8)
    for i, slot in enumerate(slots.tolist()):
        if slot < 0 or slot >= N_BLOCKS * 64:
            continue
        blk, pos = divmod(slot, 64)
        if not cfg.quantised:
            row = np.concatenate([c[i], k[i]]).astype(np.float32)
            raw = (bf16_bits(to_bf16_exact(row)) if cfg.latent_fmt == "bf16" else row).view(np.uint8)
            pool[blk, pos * raw.size:(pos + 1) * raw.size] = raw
            continue
        bits = {"int4": 4, "int2": 2}
        for vec, g, fmt, pc, ps in ((c[i], cfg.latent_group, cfg.latent_fmt, "lc", "ls"),
                                    (k[i], cfg.rope_group, cfg.rope_fmt, "rc", "rs")):
            codes, sz = quantise_rtn(vec[None].astype(np.float64), g, bits[fmt])
            packed = pack_codes(codes[0], bits[fmt])
            szb = np.ascontiguousarray(sz[0]).view(np.uint8).reshape(-1)
            pool[blk, off[pc] + pos * packed.size: off[pc] + (pos + 1) * packed.size] = packed
            pool[blk, off[ps] + pos * szb.size: off[ps] + (pos + 1) * szb.size] = szb
    return pool


@pytest.mark.parametrize("name", ["1", "2", "4", "5"])
def test_writer_matches_generator_pieces(name):
    """Every format: the oracle's pool equals the one built from the generator's quantiser,
    packer and layout, over workload-like rows, the edge rows and skipped slots."""
    cfg = CONFIGS[name]
    c, k = append_rows(cfg, 60, 11)
    slots = append_slots(N_BLOCKS, 60, 12)
    assert (slots < 0).any() or (slots >= N_BLOCKS * 64).any()
    bb, _ = block_layout(cfg)
    got = oracle.write_tokens(np.zeros((N_BLOCKS, bb), np.uint8), slots, c, k, *_fmt_args(cfg))
    np.testing.assert_array_equal(got, _generator_pool(cfg, slots, c, k))


@pytest.mark.parametrize("name", ["4", "5"])
def test_writer_round_trip(name):
    """Reading the written tokens back (the oracle's own pool reader) gives the quantiser's
    codes and (s, z) pairs, and every dequantised value lies within s/2 of its input."""
    cfg = CONFIGS[name]
    n = 130
    c, k = append_rows(cfg, n, 21)
    slots = np.arange(n, dtype=np.int32)[::-1].copy()   # token t of one sequence in slot n-1-t
    bb, _ = block_layout(cfg)
    pool = oracle.write_tokens(np.zeros((3, bb), np.uint8), slots, c, k, *_fmt_args(cfg))
    # a "sequence" reading slots 0 .. n-1 in order sees the tokens reversed
    back = oracle.read_pool(pool, np.array([[0, 1, 2]], np.int32), np.array([n]), *_fmt_args(cfg))
    cc, csz = oracle.quantise_rtn(c[::-1].astype(np.float64), cfg.latent_group, 4 if cfg.latent_fmt == "int4" else 2)
    rc, rsz = oracle.quantise_rtn(k[::-1].astype(np.float64), cfg.rope_group, 4)
    np.testing.assert_array_equal(back["c_codes"][0], cc)
    np.testing.assert_array_equal(back["c_sz"][0], csz)
    np.testing.assert_array_equal(back["r_codes"][0], rc)
    np.testing.assert_array_equal(back["r_sz"][0], rsz)
    # the error bound of round-to-nearest where nothing is clamped (neither the zero-point nor
    # the code: a group's range that misses 0, or an fp16 scale rounded down, e.g. a subnormal
    # one, can push codes past 2^b - 1); the bf16 rounding of the dequantised value adds up
    # to half a bf16 unit, at most 2^-8 of its magnitude
    g, qmax = cfg.latent_group, (15 if cfg.latent_fmt == "int4" else 3)
    x = c[::-1].astype(np.float64)
    s = np.repeat(csz[..., 0].astype(np.float64), g, axis=-1)
    lo = np.repeat(x.reshape(n, -1, g).min(-1), g, axis=-1)
    zr, qr = np.rint(-lo / s), np.rint(x / s) + np.rint(-lo / s)
    fits = (zr >= 0) & (zr <= qmax) & (qr >= 0) & (qr <= qmax)
    assert fits.mean() > 0.9
    xh = oracle.dequant(cc, csz, g)
    err = np.abs(xh - x)
    assert np.all(err[fits] <= (s / 2 + 2.0 ** -8 * np.abs(xh))[fits] * (1 + 1e-12))


def test_ties_round_to_even():
    """Values exactly half a step between two codes take the even one: an INT4 group over
    [0, 3.75] has s = 0.25, z = 0 and x = (j + 1/2) s, so code = j for even j, j + 1 for odd."""
    cfg = CONFIGS["4"]
    c, k = append_rows(cfg, 8, 3)
    row = c[4]                                   # the INT4 tie row of append_rows
    codes, sz = oracle.quantise_rtn(row[None].astype(np.float64), 64, 4)
    assert np.all(sz[0, :, 0] == np.float16(0.25)) and np.all(sz[0, :, 1] == 0)
    j = np.arange(512) % 15
    expect = np.where(j % 2 == 0, j, j + 1)
    expect[np.arange(512) % 64 == 0] = 0
    expect[np.arange(512) % 64 == 1] = 15
    np.testing.assert_array_equal(codes[0], expect)


def test_constant_group_takes_scale_one():
    """A constant group has max - min = 0: s = 1 and z = rint(-x), clamped."""
    codes, sz = oracle.quantise_rtn(np.full((1, 64), 0.7), 64, 4)
    assert sz[0, 0, 0] == np.float16(1) and sz[0, 0, 1] == 0
    assert np.all(codes == 1)                    # rint(0.7 / 1) + 0


def test_writer_skips_slots_outside_the_pool():
    """Slots below 0 or past the pool change nothing; a valid one changes only its token."""
    cfg = CONFIGS["5"]
    bb, off = block_layout(cfg)
    rng = np.random.default_rng(5)
    pool = rng.integers(0, 256, (N_BLOCKS, bb), dtype=np.uint8)
    c, k = append_rows(cfg, 3, 6)
    same = oracle.write_tokens(pool, np.array([-1, N_BLOCKS * 64, -7]), c, k, *_fmt_args(cfg))
    np.testing.assert_array_equal(same, pool)
    one = oracle.write_tokens(pool, np.array([-1, 2 * 64 + 5, -7]), c, k, *_fmt_args(cfg))
    changed = np.argwhere(one != pool)
    assert np.all(changed[:, 0] == 2)
    per_tok = {"lc": 512 // 4, "ls": (512 // 32) * 4, "rc": 64 // 2, "rs": 4}
    for name, width in per_tok.items():
        lo = off[name] + 5 * width
        inside = (changed[:, 1] >= lo) & (changed[:, 1] < lo + width)
        outside_plane = (changed[:, 1] >= off[name]) & (changed[:, 1] < off[name] + 64 * width) & ~inside
        assert not outside_plane.any()
