"""GPU parity of mla_hadamard_rotate and of the rotation folded into a decode (marked gpu).

1. The rotation against the oracle (x . H_d / sqrt(d) in float64) along rows, along the
   middle axis of a [H][d][v] tensor (W_UV's d_c), over the RoPE key's pairs and over
   strided rows, fp32 and bf16, d from 2 to 4096, vector counts that leave a ragged last
   workgroup.  Bar: the fp32 evaluation's own error bound, (log2 d + 2) 2^-24 ||x||_1 /
   sqrt(d) per vector, plus one bf16 unit (2^-8 relative) for bf16 vectors.
2. The whole fp32 step (absorb, decode, out_proj) with the rotation folded into W_UK, W_UV
   and the cached latent (rotated inside the pool) equals the unrotated step within the
   fp32 tolerance 1e-5: the full-precision invariance of the fold, on the GPU.
3. The purpose of the fold: with 16 outlier channels x20 in the latent, an INT2 cache of the
   rotated latent gives a smaller decode error than an INT2 cache of the latent itself
   (both the max-normalised and the RMS-relative error; the figures are printed).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from mla_synth import CONFIGS, append_rows, make_inputs, to_bf16_exact  # noqa: E402
from tests.gpu_helpers import desc_of, dev, norm_err, to_device  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_02_amd as m
    m.lib()
    return m


def _bound(x_vecs, d, bf16, ref):
    """Per-element bound; x_vecs [..., d] are the input vectors matching ref [..., d]."""
    fp32 = (np.log2(d) + 2) * 2.0 ** -24 * np.abs(x_vecs).sum(-1, keepdims=True) / np.sqrt(d)
    return fp32 + (2.0 ** -8 * np.abs(ref) if bf16 else 0.0) + 1e-30


LAYOUTS = [("rows", 2048, (37,)), ("rows", 4096, (3,)), ("rows", 512, (300,)), ("rows", 64, (70,)),
           ("cols", 512, (3, 40)), ("pairs", 2, (45, 32)), ("strided", 512, (33,))]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("layout,d,shape", LAYOUTS)
def test_rotation_matches_oracle(mla, layout, d, shape, dtype):
    print(f"[case] rotate {layout} d={d} {shape} {dtype}", flush=True)
    rng = np.random.default_rng(d + len(shape))
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    if layout == "cols":                                   # [H][d][v], rotate along d
        x = rng.standard_normal((shape[0], d, shape[1])).astype(np.float32)
        axis = 1
    elif layout == "pairs":                                # [n][pairs][2], rotate each pair
        x = rng.standard_normal(shape + (2,)).astype(np.float32)
        axis = 2
    else:
        x = rng.standard_normal(shape + (d,)).astype(np.float32)
        x[:, :4] *= 20.0                                   # a few large channels
        axis = 1
    if dtype == "bf16":
        x = to_bf16_exact(x)
    if layout == "strided":
        wide = torch.zeros((shape[0], d + 40), dtype=tdt)
        wide[:, 8:8 + d] = torch.from_numpy(x).to(tdt)
        wide = wide.to(dev())
        t = wide[:, 8:8 + d]
    else:
        t = torch.from_numpy(x).to(tdt).to(dev())
    mla.hadamard_rotate(t, dim=axis)
    torch.cuda.synchronize()
    got = t.float().cpu().numpy()
    ref = oracle.rotate(x.astype(np.float64), axis)
    xm = np.moveaxis(x.astype(np.float64), axis, -1)
    bound = np.moveaxis(_bound(xm, d, dtype == "bf16", np.moveaxis(ref, axis, -1)), -1, axis)
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"max err/bound {float(np.max(err / bound)):.3f}"
    if layout == "strided":                                # the bytes around the rows are untouched
        w = wide.float().cpu().numpy()
        assert not w[:, :8].any() and not w[:, 8 + d:].any()


def _step(mla, t, wuk, wuv, pool, x):
    B, s_q, H = len(x.seq_lens), x.cfg.s_q, x.cfg.H
    ql = mla.absorb_q(t["q_nope"].view(B * s_q, H, -1), wuk, out_dtype=t["q_nope"].dtype)
    o, _ = mla.decode_paged(ql.view(B, s_q, H, -1), t["q_rope"], pool, desc_of(x.cfg), t["block_table"],
                            t["seq_lens"], int(x.seq_lens.max()), x.cfg.sm_scale)
    return mla.out_proj(o.view(B * s_q, H, -1), wuv).view(B, s_q, H, -1)


def test_folded_rotation_fp32_step(mla):
    """fp32 workload shape (d_c = 64, d_r = 16), 8 heads, ragged lengths."""
    x = make_inputs(CONFIGS["1"], 31, B=3, lens=[256, 100, 7])
    t = to_device(x)
    print("[case] folded rotation, fp32 step", flush=True)
    base = _step(mla, t, t["w_uk"], t["w_uv"], t["pool"], x).cpu().numpy()
    wuk = mla.hadamard_rotate(t["w_uk"].clone(), dim=2)          # W_UK[h] R
    wuv = mla.hadamard_rotate(t["w_uv"].clone(), dim=1)          # R^T W_UV[h]
    pool = t["pool"].clone()
    rows = pool.view(torch.float32).view(pool.shape[0], 64, x.cfg.d_c + x.cfg.d_r)
    mla.hadamard_rotate(rows[:, :, :x.cfg.d_c], dim=2)           # cached latent c R, in place
    rot = _step(mla, t, wuk, wuv, pool, x).cpu().numpy()
    ref, _ = oracle.decode_unabsorbed(x.q_nope, x.q_rope, x.w_uk, x.w_uv,
                                      [x.c[b, :x.seq_lens[b]] for b in range(3)],
                                      [x.k_rope[b, :x.seq_lens[b]] for b in range(3)], x.seq_lens, 1, x.cfg.sm_scale)
    e_fold, e_base = norm_err(rot, base), norm_err(rot, ref)
    print(f"  rotated vs unrotated step {e_fold:.2e}, rotated vs oracle {e_base:.2e}", flush=True)
    assert e_fold <= 1e-5 and e_base <= 1e-5


def test_rotation_reduces_int2_error(mla):
    """INT2 latent (g32) + INT4 RoPE key, 16 heads, 16 outlier channels x20: decode of the
    quantised latent against float64 attention over the float latent, without and with the
    rotation (the rotated run's o_lat is rotated back, R being its own inverse)."""
    cfg = CONFIGS["5"].with_(H=16)
    lens = np.array([1500, 700], dtype=np.int32)
    T = int(lens.sum())
    c, k = append_rows(cfg, T + 6, 17)
    c, k = to_bf16_exact(c[6:]), to_bf16_exact(k[6:])     # the workload-like rows only
    print("[case] rotation against INT2 error", flush=True)
    rng = np.random.default_rng(18)
    q_lat = to_bf16_exact(rng.standard_normal((2, 1, 16, 512)).astype(np.float32) * 0.1)
    q_rope = to_bf16_exact(rng.standard_normal((2, 1, 16, 64)).astype(np.float32) * 0.1)
    starts = np.concatenate([[0], np.cumsum(lens)])
    ref, _ = oracle.attend_latent(q_lat.astype(np.float64), q_rope.astype(np.float64),
                                  [c[starts[b]:starts[b + 1]].astype(np.float64) for b in range(2)],
                                  [k[starts[b]:starts[b + 1]].astype(np.float64) for b in range(2)], lens, 1,
                                  cfg.sm_scale)
    nblk = -(-lens // 64)
    table = np.zeros((2, int(nblk.max())), dtype=np.int32)
    table[0, :nblk[0]] = np.arange(nblk[0])
    table[1, :nblk[1]] = nblk[0] + np.arange(nblk[1])
    slots = np.concatenate([table[b, np.arange(lens[b]) // 64] * 64 + np.arange(lens[b]) % 64 for b in range(2)])
    bb = mla.block_bytes(desc_of(cfg))
    errs = {}
    for rot in (False, True):
        ct = torch.from_numpy(c).to(torch.bfloat16).to(dev())
        qt = torch.from_numpy(q_lat).to(torch.bfloat16).to(dev())
        if rot:
            ct = mla.hadamard_rotate(ct.float(), dim=1).to(torch.bfloat16)
            qt = mla.hadamard_rotate(qt.float(), dim=3).to(torch.bfloat16)
        pool = torch.zeros((int(nblk.sum()), bb), dtype=torch.uint8, device=dev())
        mla.append_kv(ct, torch.from_numpy(k).to(torch.bfloat16).to(dev()), pool, desc_of(cfg),
                      torch.from_numpy(slots.astype(np.int32)).to(dev()))
        o, _ = mla.decode_paged(qt, torch.from_numpy(q_rope).to(torch.bfloat16).to(dev()), pool, desc_of(cfg),
                                torch.from_numpy(table).to(dev()), torch.from_numpy(lens).to(dev()), int(lens.max()),
                                cfg.sm_scale)
        if rot:
            o = mla.hadamard_rotate(o.float().contiguous(), dim=3)
        torch.cuda.synchronize()
        got = o.float().cpu().numpy()
        errs[rot] = (norm_err(got, ref), float(np.sqrt(np.mean((got - ref) ** 2)) / np.sqrt(np.mean(ref ** 2))))
    print(f"  INT2 o_lat error (max-normalised, RMS-relative): plain {errs[False][0]:.3e}, {errs[False][1]:.3e}; "
          f"rotated {errs[True][0]:.3e}, {errs[True][1]:.3e}", flush=True)
    assert errs[True][0] < errs[False][0] and errs[True][1] < errs[False][1]
