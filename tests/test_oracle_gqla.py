"""Pins of the oracle's GQLA per-group path (CPU).

GQLA exposes two algebraically equivalent decode paths over the same weights (GQLA abstract,
thelatestinai.com paper-cards page).  With head groups sharing their key/value up-projections,
the oracle's GQA path (expand the latent per group, grouped-query attention) must equal:
  * the plain unabsorbed MLA definition with those shared weights (decode_unabsorbed, itself
    pinned to hand-derived values), and the absorbed twin, to 1e-10 of the output scale;
  * torch's scaled_dot_product_attention for a single group (MQA) with no RoPE term;
  * the value row itself for a one-token sequence.
Planted mistakes (a transposed key projection, heads assigned to the wrong group) move the
result far beyond 1e-10, so the agreement is not vacuous.
"""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def _inputs(seed, B, H, G, d_c, d_n, d_v, d_r, lens, s_q):
    rng = np.random.default_rng(seed)
    q_nope = rng.standard_normal((B, s_q, H, d_n))
    q_rope = rng.standard_normal((B, s_q, H, d_r))
    w_uk_g = rng.standard_normal((G, d_n, d_c)) / np.sqrt(d_c)
    w_uv_g = rng.standard_normal((G, d_c, d_v)) / np.sqrt(d_c)
    c = [rng.standard_normal((L, d_c)) for L in lens]
    k = [rng.standard_normal((L, d_r)) for L in lens]
    return q_nope, q_rope, w_uk_g, w_uv_g, c, k, np.asarray(lens)


def _gqa(q_nope, q_rope, w_uk_g, w_uv_g, c, k, lens, s_q, scale):
    kn, v = zip(*[oracle.expand_groups(cb, w_uk_g, w_uv_g) for cb in c])
    return oracle.attend_groups(q_nope, q_rope, list(kn), k, list(v), lens, s_q, scale)


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("s_q", [1, 2])
def test_group_path_equals_the_mla_definition(G, s_q):
    H, d_c, d_n, d_v, d_r = 8, 32, 16, 12, 8
    args = _inputs(100 + G + s_q, 3, H, G, d_c, d_n, d_v, d_r, [2, 37, 70], s_q)
    q_nope, q_rope, w_uk_g, w_uv_g, c, k, lens = args
    scale = 1.0 / np.sqrt(d_n + d_r)
    out, lse = _gqa(*args, s_q, scale)
    w_uk, w_uv = oracle.group_weights(w_uk_g, H), oracle.group_weights(w_uv_g, H)
    ref, ref_lse = oracle.decode_unabsorbed(q_nope, q_rope, w_uk, w_uv, c, k, lens, s_q, scale)
    assert _rel(out, ref) <= 1e-10 and float(np.max(np.abs(lse - ref_lse))) <= 1e-10
    ab = oracle.decode_absorbed(q_nope, q_rope, w_uk, w_uv, c, k, lens, s_q, scale)
    assert _rel(out, ab["out"]) <= 1e-10 and float(np.max(np.abs(lse - ab["lse"]))) <= 1e-10


def test_group_weights_layout():
    w = np.arange(3 * 2 * 2).reshape(3, 2, 2)
    r = oracle.group_weights(w, 6)
    assert r.shape == (6, 2, 2)
    for h in range(6):
        assert np.array_equal(r[h], w[h // 2])
    with pytest.raises(ValueError):
        oracle.group_weights(w, 7)


def test_planted_mistakes_are_caught():
    """A transposed key projection (square, so it still runs) and heads mapped to the next
    group both leave the definition far behind."""
    H, G, d = 8, 4, 24
    q_nope, q_rope, w_uk_g, w_uv_g, c, k, lens = _inputs(7, 2, H, G, d, d, d, 8, [40, 9], 1)
    scale = 0.2
    ref, _ = oracle.decode_unabsorbed(q_nope, q_rope, oracle.group_weights(w_uk_g, H),
                                      oracle.group_weights(w_uv_g, H), c, k, lens, 1, scale)
    wrong_t = _gqa(q_nope, q_rope, np.transpose(w_uk_g, (0, 2, 1)), w_uv_g, c, k, lens, 1, scale)[0]
    assert _rel(wrong_t, ref) > 1e-3
    shifted = np.roll(np.arange(G), 1)
    wrong_g = _gqa(q_nope, q_rope, w_uk_g[shifted], w_uv_g[shifted], c, k, lens, 1, scale)[0]
    assert _rel(wrong_g, ref) > 1e-3
    good = _gqa(q_nope, q_rope, w_uk_g, w_uv_g, c, k, lens, 1, scale)[0]
    assert _rel(good, ref) <= 1e-10


def test_one_token_attends_its_value_row():
    H, G = 6, 3
    q_nope, q_rope, w_uk_g, w_uv_g, c, k, lens = _inputs(8, 2, H, G, 16, 8, 8, 4, [1, 1], 1)
    out, lse = _gqa(q_nope, q_rope, w_uk_g, w_uv_g, c, k, lens, 1, 0.3)
    for b in range(2):
        for h in range(H):
            g = h // (H // G)
            np.testing.assert_allclose(out[b, 0, h], c[b][0] @ w_uv_g[g], rtol=0, atol=1e-14)
            s = 0.3 * ((w_uk_g[g] @ c[b][0]) @ q_nope[b, 0, h] + k[b][0] @ q_rope[b, 0, h])
            assert abs(lse[b, 0, h] - s) <= 1e-12


def test_single_group_is_torch_sdpa():
    """G = 1 (every head shares one key/value head) with no RoPE term: torch's
    scaled_dot_product_attention in float64 on the expanded key and value."""
    H, d_c, d_n, d_v = 4, 20, 10, 6
    q_nope, q_rope, w_uk_g, w_uv_g, c, k, lens = _inputs(9, 1, H, 1, d_c, d_n, d_v, 4, [33], 1)
    q_rope[:] = 0.0
    out, _ = _gqa(q_nope, q_rope, w_uk_g, w_uv_g, c, k, lens, 1, 0.25)
    kn, v = oracle.expand_groups(c[0], w_uk_g, w_uv_g)
    q = torch.from_numpy(q_nope[0, 0])[:, None, :]                   # [H, 1, d_n]
    kk = torch.from_numpy(kn[0])[None].expand(H, -1, -1)             # [H, L, d_n]
    vv = torch.from_numpy(v[0])[None].expand(H, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(q, kk, vv, scale=0.25)[:, 0].numpy()
    np.testing.assert_allclose(out[0, 0], ref, rtol=0, atol=1e-12)
