"""GPU parity of mla_decode_mixed: one decode over a history kept at two precisions (marked gpu).

Sequence b's history is sink_b ++ middle_b ++ recent_b.  The sink (earliest tokens) and the
recent window (ending with the s_q new tokens) are bf16 caches; the middle is INT4 or INT2
(+ INT4 RoPE key).  Every part is filled through mla_append_kv into paged blocks of its own.
The oracle attends over the concatenated logical history (bf16 rows, and for the middle the
dequantised output of the oracle's own quantiser), with the causal mask on the last s_q
tokens.  Cases: both decode families (16 and 128 heads), s_q = 1 and 2, ragged parts, a
sequence with no middle, an absent sink part.  Bar: the decode tolerance 2e-3.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from mla_synth import CONFIGS, append_rows, to_bf16_exact  # noqa: E402
from tests.gpu_helpers import desc_of, dev, norm_err  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_02_amd as m
    m.lib()
    return m


def _part(mla, cfg, cs, ks, rng):
    """A paged cache holding the token rows cs[b], ks[b] of every sequence b, written with
    mla_append_kv through a shuffled block table."""
    B = len(cs)
    lens = np.array([len(c) for c in cs], dtype=np.int32)
    nblk = -(-lens // 64)
    width = max(1, int(nblk.max()))
    perm = rng.permutation(int(nblk.sum()) + 2).astype(np.int32)
    table = np.full((B, width), perm[-1], dtype=np.int32)
    slots, cur = [], 0
    for b in range(B):
        table[b, :nblk[b]] = perm[cur:cur + nblk[b]]
        cur += nblk[b]
        slots += [int(table[b, t // 64]) * 64 + t % 64 for t in range(lens[b])]
    desc = desc_of(cfg)
    pool = torch.zeros((len(perm), mla.block_bytes(desc)), dtype=torch.uint8, device=dev())
    if slots:
        mla.append_kv(torch.from_numpy(np.concatenate(cs)).to(torch.bfloat16).to(dev()),
                      torch.from_numpy(np.concatenate(ks)).to(torch.bfloat16).to(dev()), pool, desc,
                      torch.tensor(slots, dtype=torch.int32, device=dev()))
    return (pool, desc, torch.from_numpy(table).to(dev()), torch.from_numpy(lens).to(dev()), max(1, int(lens.max())))


def _logical(cfg, c, k):
    """What the decode sees of rows written to a cache of cfg's format (float64)."""
    if not cfg.quantised:
        return c.astype(np.float64), k.astype(np.float64)
    cc, csz = oracle.quantise_rtn(c.astype(np.float64), cfg.latent_group, 4 if cfg.latent_fmt == "int4" else 2)
    rc, rsz = oracle.quantise_rtn(k.astype(np.float64), cfg.rope_group, 4)
    cd, kd = oracle.dequant_cache([cc], [csz], [rc], [rsz], cfg.latent_group, cfg.rope_group)
    return cd[0], kd[0]


@pytest.mark.parametrize("low", ["4", "5"])
@pytest.mark.parametrize("s_q", [1, 2])
@pytest.mark.parametrize("H", [16, 128])
def test_mixed_history_matches_oracle(mla, H, s_q, low):
    lo_cfg = CONFIGS[low].with_(H=H)
    hi_cfg = CONFIGS["2"].with_(H=H)
    sink = [64, 64, 5]
    middle = [1000, 0, 333]
    recent = [200, 130, 2]
    B = 3
    print(f"[case] mixed history H={H} s_q={s_q} middle {lo_cfg.latent_fmt}", flush=True)
    rng = np.random.default_rng(100 + H + s_q)
    T = [sink[b] + middle[b] + recent[b] for b in range(B)]
    rows = [append_rows(lo_cfg, t + 6, 200 + b) for b, t in enumerate(T)]
    c_all = [to_bf16_exact(r[0][6:]) for r in rows]          # workload-like rows (no edge rows)
    k_all = [to_bf16_exact(r[1][6:]) for r in rows]
    cut = lambda x, b: (x[:sink[b]], x[sink[b]:sink[b] + middle[b]], x[sink[b] + middle[b]:])  # noqa: E731
    parts_c = [cut(c_all[b], b) for b in range(B)]
    parts_k = [cut(k_all[b], b) for b in range(B)]
    p_sink = _part(mla, hi_cfg, [parts_c[b][0] for b in range(B)], [parts_k[b][0] for b in range(B)], rng)
    p_mid = _part(mla, lo_cfg, [parts_c[b][1] for b in range(B)], [parts_k[b][1] for b in range(B)], rng)
    p_rec = _part(mla, hi_cfg, [parts_c[b][2] for b in range(B)], [parts_k[b][2] for b in range(B)], rng)
    q_lat = to_bf16_exact(rng.standard_normal((B, s_q, H, 512)).astype(np.float32) * 0.1)
    q_rope = to_bf16_exact(rng.standard_normal((B, s_q, H, 64)).astype(np.float32) * 0.1)
    qt = torch.from_numpy(q_lat).to(torch.bfloat16).to(dev())
    rt = torch.from_numpy(q_rope).to(torch.bfloat16).to(dev())
    o, lse = mla.decode_mixed(qt, rt, p_sink, p_mid, p_rec, lo_cfg.sm_scale)
    torch.cuda.synchronize()
    cs, ks = [], []
    for b in range(B):
        sc, sk = _logical(hi_cfg, parts_c[b][0], parts_k[b][0])
        mc, mk = _logical(lo_cfg, parts_c[b][1], parts_k[b][1])
        rc, rk = _logical(hi_cfg, parts_c[b][2], parts_k[b][2])
        cs.append(np.concatenate([sc, mc, rc]))
        ks.append(np.concatenate([sk, mk, rk]))
    ref_o, ref_lse = oracle.attend_latent(q_lat.astype(np.float64), q_rope.astype(np.float64), cs, ks,
                                          np.array(T), s_q, lo_cfg.sm_scale)
    e = norm_err(o.cpu().numpy(), ref_o)
    el = float(np.max(np.abs(lse.cpu().numpy() - ref_lse)))
    print(f"  o_lat err {e:.3e}  lse abs err {el:.3e}", flush=True)
    assert e <= 2e-3 and el <= 2e-3
    # no sink part: the history is middle ++ recent
    o2, lse2 = mla.decode_mixed(qt, rt, None, p_mid, p_rec, lo_cfg.sm_scale)
    ref2_o, ref2_lse = oracle.attend_latent(q_lat.astype(np.float64), q_rope.astype(np.float64),
                                            [c[sink[b]:] for b, c in enumerate(cs)],
                                            [k[sink[b]:] for b, k in enumerate(ks)],
                                            np.array([T[b] - sink[b] for b in range(B)]), s_q, lo_cfg.sm_scale)
    torch.cuda.synchronize()
    assert norm_err(o2.cpu().numpy(), ref2_o) <= 2e-3
    assert float(np.max(np.abs(lse2.cpu().numpy() - ref2_lse))) <= 2e-3


@pytest.mark.parametrize("H", [16, 128])
def test_sink_and_window_in_one_cache(mla, H):
    """The sink and the recent window stored as one bf16 cache (sink ++ window, ending with the
    new tokens) and passed as the recent part, with no sink part: the result equals the
    attention over sink ++ middle ++ window, since only the causal mask depends on order."""
    s_q = 2
    lo_cfg = CONFIGS["5"].with_(H=H)
    hi_cfg = CONFIGS["2"].with_(H=H)
    sink, middle, recent = [64, 3], [700, 90], [130, 66]
    B = 2
    print(f"[case] sink and window in one cache H={H}", flush=True)
    rng = np.random.default_rng(300 + H)
    T = [sink[b] + middle[b] + recent[b] for b in range(B)]
    rows = [append_rows(lo_cfg, t + 6, 400 + b) for b, t in enumerate(T)]
    c_all = [to_bf16_exact(r[0][6:]) for r in rows]
    k_all = [to_bf16_exact(r[1][6:]) for r in rows]
    hi_c = [np.concatenate([c_all[b][:sink[b]], c_all[b][sink[b] + middle[b]:]]) for b in range(B)]
    hi_k = [np.concatenate([k_all[b][:sink[b]], k_all[b][sink[b] + middle[b]:]]) for b in range(B)]
    p_hi = _part(mla, hi_cfg, hi_c, hi_k, rng)
    p_mid = _part(mla, lo_cfg, [c_all[b][sink[b]:sink[b] + middle[b]] for b in range(B)],
                  [k_all[b][sink[b]:sink[b] + middle[b]] for b in range(B)], rng)
    q_lat = to_bf16_exact(rng.standard_normal((B, s_q, H, 512)).astype(np.float32) * 0.1)
    q_rope = to_bf16_exact(rng.standard_normal((B, s_q, H, 64)).astype(np.float32) * 0.1)
    o, lse = mla.decode_mixed(torch.from_numpy(q_lat).to(torch.bfloat16).to(dev()),
                              torch.from_numpy(q_rope).to(torch.bfloat16).to(dev()), None, p_mid, p_hi,
                              lo_cfg.sm_scale)
    torch.cuda.synchronize()
    cs, ks = [], []
    for b in range(B):
        mc, mk = _logical(lo_cfg, c_all[b][sink[b]:sink[b] + middle[b]], k_all[b][sink[b]:sink[b] + middle[b]])
        cs.append(np.concatenate([c_all[b][:sink[b]].astype(np.float64), mc,
                                  c_all[b][sink[b] + middle[b]:].astype(np.float64)]))
        ks.append(np.concatenate([k_all[b][:sink[b]].astype(np.float64), mk,
                                  k_all[b][sink[b] + middle[b]:].astype(np.float64)]))
    ref_o, ref_lse = oracle.attend_latent(q_lat.astype(np.float64), q_rope.astype(np.float64), cs, ks,
                                          np.array(T), s_q, lo_cfg.sm_scale)
    e = norm_err(o.cpu().numpy(), ref_o)
    el = float(np.max(np.abs(lse.cpu().numpy() - ref_lse)))
    print(f"  o_lat err {e:.3e}  lse abs err {el:.3e}", flush=True)
    assert e <= 2e-3 and el <= 2e-3
