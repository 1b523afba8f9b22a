"""Pins of the float64 oracle against things other than itself.

Closed forms and hand-worked cases (tests/golden/tiny_cases.json), invariants
the method must satisfy, reductions to library routines (torch SDPA, torch's
bf16 conversion), brute force over every code, and the exact rational value of
each dequantised code.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from mla_synth import CONFIGS, SEEDS, block_layout, make_inputs, pack_codes
from mla_synth.gen import quantise_rtn as gen_quantise

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_cases.json")))


def _ev(expr):
    return float(eval(str(expr), {"__builtins__": {}}, {"log": math.log}))


def _evs(a):
    return np.array([[_ev(x) for x in row] for row in a]) if isinstance(a[0], list) else np.array([_ev(x) for x in a])


def _rng(seed=0):
    return np.random.default_rng(seed)


def _rand_case(rng, B=2, S=1, H=3, d_c=16, d_r=4, d_n=8, d_v=6, L=(20, 33)):
    q_nope = rng.standard_normal((B, S, H, d_n))
    q_rope = rng.standard_normal((B, S, H, d_r))
    w_uk = rng.standard_normal((H, d_n, d_c)) / math.sqrt(d_c)
    w_uv = rng.standard_normal((H, d_c, d_v)) / math.sqrt(d_c)
    c = [rng.standard_normal((l, d_c)) for l in L]
    k = [rng.standard_normal((l, d_r)) for l in L]
    return q_nope, q_rope, w_uk, w_uv, c, k, np.array(L)


# ----------------------------------------------------------------- hand-worked fixtures

def test_golden_latent_attention():
    g = GOLD["latent_attention"]
    c = [_evs(g["c"])]
    k = [_evs(g["k_rope"])]
    q_lat = np.array(g["q_lat"])[None, None, None]
    q_rope = np.array(g["q_rope"])[None, None, None]
    o, lse = oracle.attend_latent(q_lat, q_rope, c, k, [3], 1, g["sm_scale"])
    np.testing.assert_allclose(o[0, 0, 0], _evs(g["expect_o_lat"]), rtol=0, atol=1e-14)
    assert abs(lse[0, 0, 0] - _ev(g["expect_lse"])) < 1e-14


def test_golden_unabsorbed_and_absorbed():
    g, base = GOLD["unabsorbed"], GOLD["latent_attention"]
    c = [_evs(base["c"])]
    k = [_evs(base["k_rope"])]
    qn = np.array(g["q_nope"])[None, None, None]
    qr = np.array(g["q_rope"])[None, None, None]
    wuk = np.array(g["w_uk"])[None]
    wuv = np.array(g["w_uv"])[None]
    out, lse = oracle.decode_unabsorbed(qn, qr, wuk, wuv, c, k, [3], 1, g["sm_scale"])
    assert abs(out[0, 0, 0, 0] - _ev(g["expect_out"])) < 1e-13
    assert abs(lse[0, 0, 0] - _ev(g["expect_lse"])) < 1e-14
    ab = oracle.decode_absorbed(qn, qr, wuk, wuv, c, k, [3], 1, g["sm_scale"])
    assert abs(ab["out"][0, 0, 0, 0] - _ev(g["expect_out"])) < 1e-13


def test_golden_two_query_tokens():
    g, base = GOLD["two_query_tokens"], GOLD["latent_attention"]
    c = [_evs(base["c"])]
    k = [_evs(base["k_rope"])]
    q_lat = np.tile(np.array(base["q_lat"]), (1, 2, 1, 1))
    q_rope = np.tile(np.array(base["q_rope"]), (1, 2, 1, 1))
    o, lse = oracle.attend_latent(q_lat, q_rope, c, k, [3], 2, 1.0)
    np.testing.assert_allclose(o[0, :, 0], _evs(g["expect_o_lat"]), atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse[0, :, 0], _evs(g["expect_lse"]), atol=1e-14, rtol=0)


def test_golden_dequant_cases():
    for code, z, s, want in GOLD["dequant"]["cases"]:
        sz = np.array([[s, z]], dtype=np.float16)
        assert float(np.float16(s)) == s
        got = oracle.dequant(np.array([code], dtype=np.uint8), sz, 1)[0]
        assert got == want, (code, z, s, got, want)
        assert oracle.exact_dequant_value(code, z, s) == want


def test_golden_bytes_per_token():
    for lf, rf, dc, dr, gc, gr, want in GOLD["bytes_per_token"]["cases"]:
        assert oracle.token_bytes(lf, rf, dc, dr, gc, gr) == want
        _, bb = oracle.block_planes(lf, rf, dc, dr, gc, gr)
        assert bb >= 64 * want and bb % 16 == 0


# ----------------------------------------------------------------- P1: absorbed == unabsorbed

@pytest.mark.parametrize("s_q", [1, 2])
def test_p1_absorbed_equals_unabsorbed_random(s_q):
    qn, qr, wuk, wuv, c, k, L = _rand_case(_rng(1), S=s_q)
    out, lse = oracle.decode_unabsorbed(qn, qr, wuk, wuv, c, k, L, s_q, 0.3)
    ab = oracle.decode_absorbed(qn, qr, wuk, wuv, c, k, L, s_q, 0.3)
    assert np.max(np.abs(out - ab["out"])) <= 1e-10 * np.max(np.abs(out))
    np.testing.assert_allclose(lse, ab["lse"], rtol=0, atol=1e-10)


def test_p1_tiny_fp32_workload():
    """The tiny fp32 workload (8 heads, d_c 64, 256 tokens): the two forms agree."""
    x = make_inputs(CONFIGS["1"], SEEDS["1"])
    c = [x.c[b] for b in range(x.c.shape[0])]
    k = [x.k_rope[b] for b in range(x.c.shape[0])]
    out, lse = oracle.decode_unabsorbed(x.q_nope, x.q_rope, x.w_uk, x.w_uv, c, k, x.seq_lens, 1, x.sm_scale)
    ab = oracle.decode_absorbed(x.q_nope, x.q_rope, x.w_uk, x.w_uv, c, k, x.seq_lens, 1, x.sm_scale)
    assert np.max(np.abs(out - ab["out"])) <= 1e-10 * np.max(np.abs(out))
    assert np.all(np.isfinite(out))


def test_p1_detects_planted_mistakes():
    """A transposed W_UK or a dropped RoPE term breaks the equivalence check."""
    qn, qr, wuk, wuv, c, k, L = _rand_case(_rng(2), H=2, d_n=16, d_c=16)
    out, _ = oracle.decode_unabsorbed(qn, qr, wuk, wuv, c, k, L, 1, 0.3)
    bad = oracle.decode_absorbed(qn, qr, np.swapaxes(wuk, 1, 2), wuv, c, k, L, 1, 0.3)
    assert np.max(np.abs(out - bad["out"])) > 1e-3
    bad2 = oracle.decode_absorbed(qn, np.zeros_like(qr), wuk, wuv, c, k, L, 1, 0.3)
    assert np.max(np.abs(out - bad2["out"])) > 1e-3


# ----------------------------------------------------------------- P2, P3, P4, P5

def test_p2_ones_channel_and_weights_sum_to_one():
    qn, qr, wuk, wuv, c, k, L = _rand_case(_rng(3), S=2)
    c = [x.copy() for x in c]
    for x in c:
        x[:, 5] = 1.0
    q_lat = oracle.absorb_q(qn, wuk)
    o, _ = oracle.attend_latent(q_lat, qr, c, k, L, 2, 0.4)
    np.testing.assert_allclose(o[..., 5], 1.0, rtol=0, atol=1e-13)


def test_p3_rope_shift_invariance():
    qn, qr, wuk, wuv, c, k, L = _rand_case(_rng(4))
    q_lat = oracle.absorb_q(qn, wuk)
    o, lse = oracle.attend_latent(q_lat, qr, c, k, L, 1, 0.5)
    u = _rng(5).standard_normal(k[0].shape[1])
    o2, lse2 = oracle.attend_latent(q_lat, qr, c, [x + u for x in k], L, 1, 0.5)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse2 - lse, 0.5 * np.einsum("bshr,r->bsh", qr, u), atol=1e-10)


def test_p4_token_order_and_block_permutation():
    qn, qr, wuk, wuv, c, k, L = _rand_case(_rng(6))
    q_lat = oracle.absorb_q(qn, wuk)
    o, lse = oracle.attend_latent(q_lat, qr, c, k, L, 1, 0.5)
    perm = [_rng(7 + i).permutation(len(x)) for i, x in enumerate(c)]
    o2, lse2 = oracle.attend_latent(q_lat, qr, [x[p] for x, p in zip(c, perm)],
                                    [x[p] for x, p in zip(k, perm)], L, 1, 0.5)
    np.testing.assert_allclose(o2, o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse2, lse, atol=1e-12, rtol=0)
    # physical block renumbering leaves the logical cache unchanged
    x = make_inputs(CONFIGS["2"], 11, lens=[130, 64, 1], H=2)
    ref = oracle.read_pool(x.pool, x.block_table, x.seq_lens, "bf16", "bf16", 512, 64)
    pp = _rng(8).permutation(x.pool.shape[0])
    inv = np.argsort(pp)
    got = oracle.read_pool(x.pool[pp], inv[x.block_table], x.seq_lens, "bf16", "bf16", 512, 64)
    for a, b in zip(ref["c"], got["c"]):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("L", [1, 63, 64, 65, 130])
def test_p5_closed_forms_lengths(L):
    rng = _rng(L)
    c = [rng.standard_normal((L, 12))]
    k = [rng.standard_normal((L, 4))]
    q_lat = rng.standard_normal((1, 1, 2, 12))
    q_rope = rng.standard_normal((1, 1, 2, 4))
    o, lse = oracle.attend_latent(q_lat, q_rope, c, k, [L], 1, 0.7)
    if L == 1:
        np.testing.assert_array_equal(o[0, 0, 0], c[0][0])
        assert abs(lse[0, 0, 0] - 0.7 * (q_lat[0, 0, 0] @ c[0][0] + q_rope[0, 0, 0] @ k[0][0])) < 1e-12
    o0, lse0 = oracle.attend_latent(np.zeros_like(q_lat), np.zeros_like(q_rope), c, k, [L], 1, 0.7)
    np.testing.assert_allclose(o0[0, 0, 0], c[0].mean(axis=0), atol=1e-13, rtol=0)
    assert abs(lse0[0, 0, 0] - math.log(L)) < 1e-12


def test_p6_matches_torch_sdpa():
    torch = pytest.importorskip("torch")
    rng = _rng(9)
    L, d = 77, 24
    c = rng.standard_normal((L, d))
    q = rng.standard_normal((1, 1, 1, d))
    o, _ = oracle.attend_latent(q, np.zeros((1, 1, 1, 3)), [c], [np.zeros((L, 3))], [L], 1, 0.3)
    t = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q[0, 0][None, None]), torch.tensor(c[None, None]), torch.tensor(c[None, None]), scale=0.3)
    np.testing.assert_allclose(o[0, 0, 0], t.numpy()[0, 0, 0], atol=1e-13, rtol=0)


def test_p7_two_query_tokens_reduce_to_one():
    qn, qr, wuk, wuv, c, k, L = _rand_case(_rng(10), S=2)
    q_lat = oracle.absorb_q(qn, wuk)
    o2, l2 = oracle.attend_latent(q_lat, qr, c, k, L, 2, 0.5)
    o_last, l_last = oracle.attend_latent(q_lat[:, 1:], qr[:, 1:], c, k, L, 1, 0.5)
    o_prev, l_prev = oracle.attend_latent(q_lat[:, :1], qr[:, :1], c, k, L - 1, 1, 0.5)
    np.testing.assert_allclose(o2[:, 1], o_last[:, 0], atol=1e-13, rtol=0)
    np.testing.assert_allclose(o2[:, 0], o_prev[:, 0], atol=1e-13, rtol=0)
    np.testing.assert_allclose(l2[:, 0], l_prev[:, 0], atol=1e-13, rtol=0)


def test_p8_merging_partials_equals_one_pass():
    rng = _rng(11)
    L = 300
    c = rng.standard_normal((L, 10))
    k = rng.standard_normal((L, 2))
    q = rng.standard_normal((1, 1, 3, 10))
    qr = rng.standard_normal((1, 1, 3, 2))
    o, lse = oracle.attend_latent(q, qr, [c], [k], [L], 1, 0.6)
    cuts = sorted(set([0, L] + list(rng.integers(1, L, 5))))
    parts = [oracle.attend_latent(q, qr, [c[a:b]], [k[a:b]], [b - a], 1, 0.6) for a, b in zip(cuts, cuts[1:])]
    om, lm = oracle.merge_partials([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(om, o, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lm, lse, atol=1e-12, rtol=0)
    # a part that saw no tokens (lse = -inf, o = 0) changes nothing
    om2, lm2 = oracle.merge_partials([p[0] for p in parts] + [np.zeros_like(o)],
                                     [p[1] for p in parts] + [np.full_like(lse, -np.inf)])
    np.testing.assert_allclose(om2, o, atol=1e-13, rtol=0)


def test_p9_offline_fusible_transforms_change_nothing():
    """Orthogonal latent rotation folded into W_UK/W_UV; RoPE pair rotation and reciprocal
    pair scaling applied to q and k: the full-precision output is unchanged."""
    qn, qr, wuk, wuv, c, k, L = _rand_case(_rng(12), H=2, d_r=6)
    out, lse = oracle.decode_unabsorbed(qn, qr, wuk, wuv, c, k, L, 1, 0.5)
    R, _ = np.linalg.qr(_rng(13).standard_normal((16, 16)))
    out2, lse2 = oracle.decode_unabsorbed(qn, qr, wuk @ R, np.swapaxes(R, 0, 1) @ wuv,
                                          [x @ R for x in c], k, L, 1, 0.5)
    np.testing.assert_allclose(out2, out, atol=1e-12, rtol=0)
    th = 0.7
    rot = np.array([[math.cos(th), -math.sin(th)], [math.sin(th), math.cos(th)]])

    def pairwise(x, m):
        y = x.copy()
        y[..., 0:2] = x[..., 0:2] @ m.T
        return y
    out3, _ = oracle.decode_unabsorbed(qn, pairwise(qr, rot), wuk, wuv, c, [pairwise(x, rot) for x in k], L, 1, 0.5)
    np.testing.assert_allclose(out3, out, atol=1e-12, rtol=0)
    a = 3.0
    qs, ks = qr.copy(), [x.copy() for x in k]
    qs[..., 2:4] /= a
    for x in ks:
        x[:, 2:4] *= a
    out4, _ = oracle.decode_unabsorbed(qn, qs, wuk, wuv, c, ks, L, 1, 0.5)
    np.testing.assert_allclose(out4, out, atol=1e-12, rtol=0)


# ----------------------------------------------------------------- P10: dequant brute force

def _fp16_samples():
    rng = _rng(14)
    bits = np.concatenate([np.array([0x0001, 0x0003, 0x03FF, 0x0400, 0x3C00, 0x3C01, 0x7BFF, 0x2E66], np.uint16),
                           rng.integers(0x0001, 0x7BFF, 200).astype(np.uint16)])
    return bits.view(np.float16)


@pytest.mark.parametrize("bits", [4, 2])
def test_p10_dequant_every_code_matches_exact_rational(bits):
    qmax = 2 ** bits - 1
    svals = _fp16_samples()
    codes = np.arange(qmax + 1, dtype=np.uint8)
    for z in range(qmax + 1):
        sz = np.zeros((len(svals), 1, 2), np.float16)
        sz[:, 0, 0] = svals
        sz[:, 0, 1] = z
        got = oracle.dequant(np.broadcast_to(codes, (len(svals), qmax + 1)), sz, qmax + 1)
        for i, s in enumerate(svals[:40]):
            for code in range(qmax + 1):
                assert got[i, code] == oracle.exact_dequant_value(code, z, float(s))
        # every sample against torch's float32 -> bfloat16 rounding of the exact product
        torch = pytest.importorskip("torch")
        prod = ((codes[None, :].astype(np.float64) - z) * svals[:, None].astype(np.float64)).astype(np.float32)
        ref = torch.from_numpy(prod).to(torch.bfloat16).to(torch.float64).numpy()
        np.testing.assert_array_equal(got, ref)


def test_bf16_round_matches_torch_on_ties_and_randoms():
    torch = pytest.importorskip("torch")
    rng = _rng(15)
    u = np.concatenate([rng.integers(0, 2 ** 31, 100000, dtype=np.uint32),
                        (rng.integers(0, 2 ** 15, 1000, dtype=np.uint32) << 16) | 0x8000,
                        (rng.integers(0, 2 ** 15, 1000, dtype=np.uint32) << 16) | 0x7FFF])
    u = u[(u & 0x7F800000) != 0x7F800000]
    x = u.view(np.float32)
    got = oracle.bf16_round(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(got, ref)


def test_unpack_inverts_generator_packing():
    rng = _rng(16)
    for bits in (4, 2):
        codes = rng.integers(0, 2 ** bits, (5, 128)).astype(np.uint8)
        packed = pack_codes(codes, bits)
        assert packed.shape[-1] == 128 * bits // 8
        np.testing.assert_array_equal(oracle.unpack_codes(packed, bits, 128), codes)
    # explicit nibble order: element 0 is the low nibble of byte 0
    assert pack_codes(np.array([[1, 2]], np.uint8), 4)[0, 0] == 0x21
    assert pack_codes(np.array([[1, 2, 3, 0]], np.uint8), 2)[0, 0] == 0b00111001


# ----------------------------------------------------------------- P11: quantiser

@pytest.mark.parametrize("bits,group", [(4, 64), (2, 32), (4, 32)])
def test_p11_quantiser_bound_and_generator_agreement(bits, group):
    rng = _rng(17)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    x[:, 7] *= 20
    codes, sz = oracle.quantise_rtn(x, group, bits)
    gcodes, gsz = gen_quantise(x, group, bits)
    np.testing.assert_array_equal(codes, gcodes)
    np.testing.assert_array_equal(sz.view(np.uint16), gsz.view(np.uint16))
    assert codes.max() <= 2 ** bits - 1
    xhat = oracle.dequant(codes, sz, group)
    s = np.repeat(sz[..., 0].astype(np.float64), group, axis=-1)
    # RTN error at most s/2 where rint(x/s)+z was not clamped, at most s where it was
    # (the zero point is itself rounded), plus the final bf16 rounding of x_hat
    zz = np.repeat(sz[..., 1].astype(np.float64), group, -1)
    q = np.rint(x.astype(np.float64) / s) + zz
    inside = (q >= 0) & (q <= 2 ** bits - 1)
    err = np.abs(x - xhat)
    tol_b = np.abs(xhat) * 2.0 ** -8
    assert np.all(err[inside] <= s[inside] / 2 * (1 + 1e-6) + tol_b[inside])
    assert np.all(err <= s * (1 + 1e-6) + tol_b)
    assert inside.mean() > 0.7


# ----------------------------------------------------------------- P12: layout and pool

def test_p12_layouts_agree_with_generator():
    for name in ("1", "2", "4", "5"):
        cfg = CONFIGS[name]
        gb, goff = block_layout(cfg)
        off, bb = oracle.block_planes(cfg.latent_fmt, cfg.rope_fmt, cfg.d_c, cfg.d_r,
                                      cfg.latent_group, cfg.rope_group)
        assert gb == bb and goff == off
    assert oracle.token_bytes("bf16", "bf16", 512, 64) == 1152


@pytest.mark.parametrize("name", ["2", "4", "5"])
def test_p12_pool_round_trip(name):
    cfg = CONFIGS[name]
    x = make_inputs(cfg, 21, lens=[1, 64, 65, 190], H=2)
    got = oracle.read_pool(x.pool, x.block_table, x.seq_lens, cfg.latent_fmt, cfg.rope_fmt, cfg.d_c,
                           cfg.d_r, cfg.latent_group, cfg.rope_group)
    for b, L in enumerate(x.seq_lens):
        if cfg.quantised:
            np.testing.assert_array_equal(got["c_codes"][b], x.c_codes[b, :L])
            np.testing.assert_array_equal(got["c_sz"][b].view(np.uint16), x.c_sz[b, :L].view(np.uint16))
            np.testing.assert_array_equal(got["r_codes"][b], x.r_codes[b, :L])
            np.testing.assert_array_equal(got["r_sz"][b].view(np.uint16), x.r_sz[b, :L].view(np.uint16))
        else:
            np.testing.assert_array_equal(got["c"][b], x.c[b, :L])
            np.testing.assert_array_equal(got["k_rope"][b], x.k_rope[b, :L])


def test_generator_quantised_codes_match_oracle_quantiser():
    """Codes stored by the workload generator equal the oracle's own RTN quantiser."""
    cfg = CONFIGS["4"]
    x = make_inputs(cfg, 22, lens=[70], H=2, poison=False)
    # regenerate the float latent by the recorded draw order to requantise independently
    rng = np.random.Generator(np.random.PCG64(22))
    B, Lm = 1, 70
    rng.standard_normal((B, 1, 2, cfg.d_n), dtype=np.float32)
    rng.standard_normal((B, 1, 2, cfg.d_r), dtype=np.float32)
    rng.standard_normal((2, cfg.d_n, cfg.d_c), dtype=np.float32)
    rng.standard_normal((2, cfg.d_c, cfg.d_v), dtype=np.float32)
    c = rng.standard_normal((B, Lm, cfg.d_c), dtype=np.float32)
    kr = rng.standard_normal((B, Lm, cfg.d_r), dtype=np.float32)
    outl = np.sort(rng.choice(cfg.d_c, cfg.outliers, replace=False))
    c[:, :, outl] *= np.float32(20)
    codes, sz = oracle.quantise_rtn(c[0], 64, 4)
    np.testing.assert_array_equal(codes, x.c_codes[0])
    np.testing.assert_array_equal(sz.view(np.uint16), x.c_sz[0].view(np.uint16))
    rcodes, rsz = oracle.quantise_rtn(kr[0], 64, 4)
    np.testing.assert_array_equal(rcodes, x.r_codes[0])


def test_oracle_is_independent_of_the_product():
    src = open(os.path.join(os.path.dirname(oracle.__file__), "mla_oracle.py")).read()
    assert "mla_latent_kv_02_amd" not in src and "mla_synth" not in src and "ctypes" not in src
