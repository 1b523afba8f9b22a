"""Pins of the oracle's fixed rotation (CPU): the Walsh-Hadamard matrix against its
closed form, orthogonality, and the invariance of the full MLA decode when the rotation is
folded into the weights and the cached latent."""
import numpy as np
import pytest

import oracle
from mla_synth import CONFIGS, make_inputs


@pytest.mark.parametrize("d", [1, 2, 4, 8, 64, 512])
def test_hadamard_closed_form(d):
    """H_d[i][j] = (-1)^popcount(i & j) / sqrt(d), entry by entry."""
    i, j = np.meshgrid(np.arange(d), np.arange(d), indexing="ij")
    pop = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    np.testing.assert_array_equal(oracle.hadamard(d) * np.sqrt(d), (-1.0) ** pop)


@pytest.mark.parametrize("d", [2, 64, 512, 4096])
def test_hadamard_is_an_orthogonal_involution(d):
    h = oracle.hadamard(d)
    np.testing.assert_allclose(h @ h.T, np.eye(d), atol=1e-12)
    np.testing.assert_array_equal(h, h.T)
    x = np.random.default_rng(d).standard_normal((3, d))
    np.testing.assert_allclose(oracle.rotate(oracle.rotate(x)), x, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(oracle.rotate(x), axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)


def test_rotate_along_an_inner_axis():
    """rotate(x, axis) equals rotating the moved axis: W_UV [H][d_c][d_v] along d_c is R^T W."""
    w = np.random.default_rng(1).standard_normal((3, 8, 5))
    got = oracle.rotate(w, -2)
    ref = np.stack([oracle.hadamard(8).T @ w[h] for h in range(3)])
    np.testing.assert_allclose(got, ref, atol=1e-13)


@pytest.mark.parametrize("name", ["1", "2"])
def test_folded_rotation_leaves_decode_unchanged(name):
    """Unabsorbed MLA (explicit K and V) over c R with W_UK R and R^T W_UV equals MLA over c
    with the original weights, to float64 rounding; the RoPE path is untouched."""
    x = make_inputs(CONFIGS[name], 3, B=2, lens=[70, 130], H=4)
    wuk_r, wuv_r = oracle.fold_rotation(x.w_uk, x.w_uv)
    c = [x.c[b, :x.seq_lens[b]].astype(np.float64) for b in range(2)]
    k = [x.k_rope[b, :x.seq_lens[b]].astype(np.float64) for b in range(2)]
    cr = [oracle.rotate(cb) for cb in c]
    ref = oracle.decode_unabsorbed(x.q_nope, x.q_rope, x.w_uk, x.w_uv, c, k, x.seq_lens, x.cfg.s_q, x.cfg.sm_scale)
    got = oracle.decode_unabsorbed(x.q_nope, x.q_rope, wuk_r, wuv_r, cr, k, x.seq_lens, x.cfg.s_q, x.cfg.sm_scale)
    for a, b in zip(got, ref):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)
    # a fold that forgets W_UV (the values then come out rotated) is caught
    bad = oracle.decode_unabsorbed(x.q_nope, x.q_rope, wuk_r, x.w_uv, cr, k, x.seq_lens, x.cfg.s_q, x.cfg.sm_scale)
    assert not np.allclose(bad[0], ref[0], atol=1e-6)
    np.testing.assert_allclose(bad[1], ref[1], rtol=1e-10)   # the scores, hence lse, are still right
