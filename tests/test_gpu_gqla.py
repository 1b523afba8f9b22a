"""GPU parity of GQLA's per-group GQA decode path (marked gpu).

* mla_gqa_expand: every group's k_nope = W_UK^g c and v = c W_UV^g against the float64 oracle
  (one RNE bf16 rounding of an fp32-accumulated value), the shared RoPE key copied bit for bit,
  skipped slots and every other byte of the pool untouched.
* mla_gqa_decode_paged, stage-wise: over an expanded pool packed on the host from the oracle's
  expansion rounded to bf16, against the oracle's grouped-query attention fed those same
  values: max|out - ref| / max|ref| and |lse - ref| within 2e-3; 1 .. 16 groups, one and two
  query tokens, several split counts, empty sequences and block ids outside the pool.
* End to end on the same (group-shared) weights, against the unabsorbed float64 definition: the
  absorbed MQA path (absorb, paged latent decode, up-projection) within the pipeline bound of
  4e-3, and the GQA path (expand, then decode) within the error its bf16 expanded cache has by
  itself (the oracle's attention over the bf16-rounded expansion) plus the 2e-3 stage
  tolerance; the two paths agree within the sum of their bounds.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from mla_synth import CONFIGS, make_inputs  # noqa: E402
from tests.gpu_helpers import bf16_exact, desc_of, dev, norm_err, to_device  # noqa: E402

pytestmark = pytest.mark.gpu
TOL_STAGE = 2e-3
TOL_PIPE = 4e-3
DN = DV = 128
DR = 64


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_02_amd as m
    m.lib()
    return m


def _bits(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _pool_planes(pool, G):
    """(planes [nb, G, 64, 256], rope [nb, 64, 64]) uint16 views of an expanded pool."""
    nb = pool.shape[0]
    u = pool.view(np.uint16).reshape(nb, -1)
    planes = u[:, :G * 64 * (DN + DV)].reshape(nb, G, 64, DN + DV)
    rope = u[:, G * 64 * (DN + DV):].reshape(nb, 64, DR)
    return planes, rope


def _pack_pool(k_nope, v, k_rope, lens, block_table, n_blocks, G):
    """Host-packed expanded pool from per-sequence bf16-exact values (k_nope[b] [G, L, 128],
    v[b] [G, L, 128], k_rope[b] [L, 64]); unused rows hold NaN so any stray read shows."""
    pool = np.full((n_blocks, G * 64 * (DN + DV) + 64 * DR), 0x7FC0, np.uint16)
    planes = pool[:, :G * 64 * (DN + DV)].reshape(n_blocks, G, 64, DN + DV)
    rope = pool[:, G * 64 * (DN + DV):].reshape(n_blocks, 64, DR)
    for b, L in enumerate(lens):
        for t in range(L):
            blk, pos = block_table[b, t // 64], t % 64
            planes[blk, :, pos, :DN] = _bits(k_nope[b][:, t])
            planes[blk, :, pos, DN:] = _bits(v[b][:, t])
            rope[blk, pos] = _bits(k_rope[b][t])
    return pool.view(np.uint8)


def _group_weights(x, G):
    """Group-shared weights from a drawn workload: group g takes head g's matrices."""
    return x.w_uk[:G].copy(), x.w_uv[:G].copy()


def test_expand_matches_oracle(mla):
    x = make_inputs(CONFIGS["3"], 91, lens=[100, 37], H=8)
    G = 4
    w_uk_g, w_uv_g = _group_weights(x, G)
    c = np.concatenate([x.c[0, :100], x.c[1, :37]])
    k = np.concatenate([x.k_rope[0, :100], x.k_rope[1, :37]])
    n, nb = c.shape[0], 4
    rng = np.random.default_rng(5)
    slots = rng.permutation(nb * 64)[:n].astype(np.int32)
    slots[[3, 50]] = -1                                   # skipped
    slots[7] = nb * 64 + 9                                # outside the pool: skipped
    bb = mla.gqa_block_bytes(G)
    pool0 = rng.integers(0, 256, (nb, bb), dtype=np.uint8)
    pool_t = torch.from_numpy(pool0).to(dev())
    bf = lambda a: torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).to(dev())  # noqa: E731
    # strided latent rows: a view into a wider buffer
    cw = torch.zeros((n, 512 + 32), dtype=torch.bfloat16, device=dev())
    cw[:, :512] = bf(c)
    print("[case] gqa expand G=4", flush=True)
    mla.gqa_expand(cw[:, :512], bf(k), bf(w_uk_g), bf(w_uv_g), pool_t, torch.from_numpy(slots).to(dev()))
    torch.cuda.synchronize()
    got = pool_t.cpu().numpy()
    kn, vv = oracle.expand_groups(c, w_uk_g, w_uv_g)          # [G, n, 128] float64
    planes, rope = _pool_planes(got, G)
    planes0, rope0 = _pool_planes(pool0, G)
    written = np.zeros((nb, 64), bool)
    worst = 0.0
    for i in range(n):
        s = int(slots[i])
        if s < 0 or s >= nb * 64:
            continue
        blk, pos = divmod(s, 64)
        written[blk, pos] = True
        gk = (planes[blk, :, pos, :DN].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        gv = (planes[blk, :, pos, DN:].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        for gg, ref in ((gk, kn[:, i]), (gv, vv[:, i])):
            mx = np.max(np.abs(ref))
            err = np.abs(gg - ref) - 2.0 ** -8 * np.abs(ref) - 1e-5 * mx
            worst = max(worst, float(np.max(err)))
        np.testing.assert_array_equal(rope[blk, pos], _bits(k[i]))
    assert worst <= 0.0, worst
    np.testing.assert_array_equal(planes.transpose(0, 2, 1, 3)[~written], planes0.transpose(0, 2, 1, 3)[~written])
    np.testing.assert_array_equal(rope[~written], rope0[~written])


def _stage_case(mla, H, G, s_q, lens, seed, splits=0, empty=(), bad_block=None):
    name = "3" if s_q == 1 else "3b"
    x = make_inputs(CONFIGS[name], seed, lens=lens, H=H)
    w_uk_g, w_uv_g = _group_weights(x, G)
    ks, vs = [], []
    for b, L in enumerate(x.seq_lens):
        kn, vv = oracle.expand_groups(x.c[b, :L].astype(np.float64), w_uk_g, w_uv_g)
        ks.append(bf16_exact(kn))
        vs.append(bf16_exact(vv))
    kr = [x.k_rope[b, :L].astype(np.float64) for b, L in enumerate(x.seq_lens)]
    nb = x.pool.shape[0]
    pool = _pack_pool(ks, vs, kr, x.seq_lens, x.block_table, nb, G)
    lens_run = x.seq_lens.copy()
    for b in empty:
        lens_run[b] = 0
    bt = x.block_table.copy()
    keep_tok = [np.arange(L) for L in x.seq_lens]
    if bad_block is not None:
        b, j = bad_block
        bt[b, j] = -5
        keep_tok[b] = np.setdiff1d(keep_tok[b], np.arange(64 * j, 64 * j + 64))
    t = lambda a: torch.from_numpy(a).to(dev())  # noqa: E731
    qn = torch.from_numpy(x.q_nope).to(torch.bfloat16).to(dev())
    qr = torch.from_numpy(x.q_rope).to(torch.bfloat16).to(dev())
    out, lse = mla.gqa_decode_paged(qn, qr, t(pool), G, t(bt), t(lens_run), int(x.seq_lens.max()), x.cfg.sm_scale,
                                    num_splits=splits)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    live = [b for b in range(len(lens)) if b not in empty]
    for b in empty:
        assert np.all(out[b] == 0.0) and np.all(lse[b] == -np.inf)
    sel = [b for b in live]
    kk = [ks[b][:, keep_tok[b]] for b in sel]
    vv = [vs[b][:, keep_tok[b]] for b in sel]
    rr = [kr[b][keep_tok[b]] for b in sel]
    ref, ref_lse = oracle.attend_groups(x.q_nope[sel], x.q_rope[sel], kk, rr, vv,
                                        np.array([len(keep_tok[b]) for b in sel]), s_q, x.cfg.sm_scale)
    e = norm_err(out[sel], ref)
    el = float(np.max(np.abs(lse[sel] - ref_lse)))
    print(f"[case] gqa decode H={H} G={G} s_q={s_q} lens={list(lens)} splits={splits}: out err {e:.3e} "
          f"lse err {el:.3e}", flush=True)
    assert e <= TOL_STAGE and el <= TOL_STAGE


@pytest.mark.parametrize("H,G,s_q", [(128, 8, 2), (128, 8, 1), (128, 16, 2), (128, 4, 2), (16, 1, 2), (16, 2, 1)])
def test_gqa_decode_stage(mla, H, G, s_q):
    for splits in (0, 3):
        _stage_case(mla, H, G, s_q, [2, 70, 333, 1100], 92, splits)


def test_gqa_decode_edges(mla):
    """An empty sequence (out = 0, lse = -inf) and a block-table entry outside the pool (its
    tokens take no part), in one batch."""
    _stage_case(mla, 128, 8, 2, [300, 5, 200, 90], 93, splits=2, empty=(1,), bad_block=(2, 1))


@pytest.mark.parametrize("s_q", [2, 1])
def test_gqa_and_absorbed_paths_agree(mla, s_q):
    """The two decode paths GQLA exposes, on the same group-shared weights and the same bf16
    latent cache: both against the unabsorbed definition, and against each other."""
    H, G = 128, 8
    name = "3" if s_q == 1 else "3b"
    x = make_inputs(CONFIGS[name], 94, lens=[64, 700, 1500], H=H)
    w_uk_g, w_uv_g = _group_weights(x, G)
    w_uk, w_uv = oracle.group_weights(w_uk_g, H), oracle.group_weights(w_uv_g, H)
    B, L = len(x.seq_lens), x.seq_lens
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).to(dev())  # noqa: E731
    t = to_device(x)
    # the absorbed MQA path on the MLA cache
    q_lat = mla.absorb_q(bf(x.q_nope).view(B * s_q, H, DN), bf(w_uk))
    o_lat, _ = mla.decode_paged(q_lat.view(B, s_q, H, 512), t["q_rope"], t["pool"], desc_of(x.cfg), t["block_table"],
                                t["seq_lens"], int(L.max()), x.cfg.sm_scale)
    out_abs = mla.out_proj(o_lat.view(B * s_q, H, 512), bf(w_uv)).view(B, s_q, H, DV)
    # the GQA path: expand every cached token into the per-group pool, then decode
    nb = x.pool.shape[0]
    gpool = torch.zeros((nb, mla.gqa_block_bytes(G)), dtype=torch.uint8, device=dev())
    rows = np.concatenate([x.c[b, :Lb] for b, Lb in enumerate(L)])
    krows = np.concatenate([x.k_rope[b, :Lb] for b, Lb in enumerate(L)])
    slots = np.concatenate([x.block_table[b, np.arange(Lb) // 64] * 64 + np.arange(Lb) % 64
                            for b, Lb in enumerate(L)]).astype(np.int32)
    mla.gqa_expand(bf(rows), bf(krows), bf(w_uk_g), bf(w_uv_g), gpool, torch.from_numpy(slots).to(dev()))
    out_gqa, _ = mla.gqa_decode_paged(bf(x.q_nope), bf(x.q_rope), gpool, G, t["block_table"], t["seq_lens"],
                                      int(L.max()), x.cfg.sm_scale)
    torch.cuda.synchronize()
    ref, _ = oracle.decode_unabsorbed(x.q_nope, x.q_rope, w_uk, w_uv, [x.c[b, :Lb] for b, Lb in enumerate(L)],
                                      [x.k_rope[b, :Lb] for b, Lb in enumerate(L)], L, s_q, x.cfg.sm_scale)
    # the error the bf16 expanded cache carries by itself (no kernel involved)
    kx, vx = zip(*[oracle.expand_groups(x.c[b, :Lb].astype(np.float64), w_uk_g, w_uv_g) for b, Lb in enumerate(L)])
    fmt, _ = oracle.attend_groups(x.q_nope, x.q_rope, [bf16_exact(k) for k in kx],
                                  [x.k_rope[b, :Lb] for b, Lb in enumerate(L)], [bf16_exact(v) for v in vx], L, s_q,
                                  x.cfg.sm_scale)
    e_fmt = norm_err(fmt, ref)
    a, g = out_abs.cpu().numpy(), out_gqa.cpu().numpy()
    ea, eg, eag = norm_err(a, ref), norm_err(g, ref), norm_err(g, a)
    print(f"[case] paths s_q={s_q}: absorbed {ea:.3e}  gqa {eg:.3e} (bf16 expanded cache alone {e_fmt:.3e})  "
          f"gqa vs absorbed {eag:.3e}", flush=True)
    assert ea <= TOL_PIPE
    assert eg <= e_fmt + TOL_STAGE
    assert eag <= TOL_PIPE + e_fmt + TOL_STAGE
