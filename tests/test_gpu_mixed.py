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


@pytest.mark.parametrize("s_q", [1, 2])
@pytest.mark.parametrize("H", [16, 128])
def test_mixed_bf16_parts_merged_per_part(mla, H, s_q):
    """A history whose middle is bf16 too is not decoded as one loop: each part is its own
    decode (16 heads: split partitions; 128 heads: the row-owner kernel, whose ranges' last
    pieces are fp16) and one merge reads every part's partials in place."""
    cfg = CONFIGS["2"].with_(H=H)
    sink, middle, recent = [64, 3, 128], [900, 0, 2100], [130, 77, 5]
    B = 3
    print(f"[case] bf16 parts merged per part H={H} s_q={s_q}", flush=True)
    rng = np.random.default_rng(300 + H + s_q)
    T = [sink[b] + middle[b] + recent[b] for b in range(B)]
    rows = [append_rows(cfg, t + 6, 400 + b) for b, t in enumerate(T)]
    c_all = [to_bf16_exact(r[0][6:]) for r in rows]
    k_all = [to_bf16_exact(r[1][6:]) for r in rows]
    cut = lambda x, b: (x[:sink[b]], x[sink[b]:sink[b] + middle[b]], x[sink[b] + middle[b]:])  # noqa: E731
    parts_c = [cut(c_all[b], b) for b in range(B)]
    parts_k = [cut(k_all[b], b) for b in range(B)]
    p = [_part(mla, cfg, [parts_c[b][i] for b in range(B)], [parts_k[b][i] for b in range(B)], rng) for i in range(3)]
    q_lat = to_bf16_exact(rng.standard_normal((B, s_q, H, 512)).astype(np.float32) * 0.1)
    q_rope = to_bf16_exact(rng.standard_normal((B, s_q, H, 64)).astype(np.float32) * 0.1)
    qt = torch.from_numpy(q_lat).to(torch.bfloat16).to(dev())
    rt = torch.from_numpy(q_rope).to(torch.bfloat16).to(dev())
    o, lse = mla.decode_mixed(qt, rt, p[0], p[1], p[2], cfg.sm_scale)
    torch.cuda.synchronize()
    cs = [np.concatenate([x.astype(np.float64) for x in parts_c[b]]) for b in range(B)]
    ks = [np.concatenate([x.astype(np.float64) for x in parts_k[b]]) for b in range(B)]
    ref_o, ref_lse = oracle.attend_latent(q_lat.astype(np.float64), q_rope.astype(np.float64), cs, ks,
                                          np.array(T), s_q, cfg.sm_scale)
    e = norm_err(o.cpu().numpy(), ref_o)
    el = float(np.max(np.abs(lse.cpu().numpy() - ref_lse)))
    print(f"  o_lat err {e:.3e}  lse abs err {el:.3e}", flush=True)
    assert e <= 2e-3 and el <= 2e-3


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


def _mixed_case(mla, H, s_q, low, sink, middle, recent, seed, o_dtype=None):
    """Decode sink ++ middle ++ recent (token counts per sequence) with mla_decode_mixed and
    return (o, lse, ref_o, ref_lse); a part whose counts are all zero is passed as absent."""
    lo_cfg = CONFIGS[low].with_(H=H)
    hi_cfg = CONFIGS["2"].with_(H=H)
    B = len(sink)
    rng = np.random.default_rng(seed)
    T = [sink[b] + middle[b] + recent[b] for b in range(B)]
    rows = [append_rows(lo_cfg, t + 6, seed + b) for b, t in enumerate(T)]
    c_all = [to_bf16_exact(r[0][6:]) for r in rows]
    k_all = [to_bf16_exact(r[1][6:]) for r in rows]
    cuts = [(c_all[b][:sink[b]], c_all[b][sink[b]:sink[b] + middle[b]], c_all[b][sink[b] + middle[b]:]) for b in range(B)]
    kuts = [(k_all[b][:sink[b]], k_all[b][sink[b]:sink[b] + middle[b]], k_all[b][sink[b] + middle[b]:]) for b in range(B)]
    parts = []
    for i, (cfg, n) in enumerate(((hi_cfg, sink), (lo_cfg, middle), (hi_cfg, recent))):
        parts.append(_part(mla, cfg, [cuts[b][i] for b in range(B)], [kuts[b][i] for b in range(B)], rng)
                     if max(n) > 0 else None)
    q_lat = to_bf16_exact(rng.standard_normal((B, s_q, H, 512)).astype(np.float32) * 0.1)
    q_rope = to_bf16_exact(rng.standard_normal((B, s_q, H, 64)).astype(np.float32) * 0.1)
    kw = {} if o_dtype is None else {"o_dtype": o_dtype}
    o, lse = mla.decode_mixed(torch.from_numpy(q_lat).to(torch.bfloat16).to(dev()),
                              torch.from_numpy(q_rope).to(torch.bfloat16).to(dev()), *parts, lo_cfg.sm_scale, **kw)
    torch.cuda.synchronize()
    cs, ks = [], []
    for b in range(B):
        sc, sk = _logical(hi_cfg, cuts[b][0], kuts[b][0])
        mc, mk = _logical(lo_cfg, cuts[b][1], kuts[b][1])
        rc, rk = _logical(hi_cfg, cuts[b][2], kuts[b][2])
        cs.append(np.concatenate([sc, mc, rc]).reshape(-1, 512))
        ks.append(np.concatenate([sk, mk, rk]).reshape(-1, 64))
    # the oracle over the non-empty histories (an empty one has no attention to compare)
    idx = [b for b in range(B) if T[b] > 0]
    ro, rl = oracle.attend_latent(q_lat[idx].astype(np.float64), q_rope[idx].astype(np.float64),
                                  [cs[b] for b in idx], [ks[b] for b in idx], np.array([T[b] for b in idx]), s_q,
                                  lo_cfg.sm_scale)
    ref_o = np.full((B, s_q, H, 512), np.nan)
    ref_lse = np.full((B, s_q, H), np.nan)
    ref_o[idx], ref_lse[idx] = ro, rl
    return o.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_lse


@pytest.mark.parametrize("low", ["4", "5"])
@pytest.mark.parametrize("H", [16, 128])
def test_mixed_one_loop_edge_sequences(mla, H, low):
    """One decode over the joint history (16 heads: the pipelined partition kernel, 128: the
    row-owner kernel): sequences with only a sink, only a recent window, nothing at all, a
    partial sink block and no middle, and a long middle, in one batch; the empty one gets
    o = 0 and lse = -inf."""
    sink = [64, 40, 0, 0, 5, 64]
    middle = [900, 0, 0, 0, 0, 2500]
    recent = [70, 0, 130, 0, 66, 512]
    print(f"[case] mixed edge sequences H={H} middle {CONFIGS[low].latent_fmt}", flush=True)
    o, lse, ref_o, ref_lse = _mixed_case(mla, H, 1, low, sink, middle, recent, 700 + H + int(low))
    e = norm_err(o[[0, 1, 2, 4, 5]], ref_o[[0, 1, 2, 4, 5]])
    el = float(np.max(np.abs(lse[[0, 1, 2, 4, 5]] - ref_lse[[0, 1, 2, 4, 5]])))
    print(f"  o_lat err {e:.3e}  lse abs err {el:.3e}", flush=True)
    assert e <= 2e-3 and el <= 2e-3
    assert np.all(o[3] == 0) and np.all(np.isneginf(lse[3]))


@pytest.mark.parametrize("H,s_q", [(16, 1), (128, 1), (128, 2)])
def test_mixed_one_loop_many_ranges(mla, H, s_q):
    """INT2 middle: a batch of ragged histories whose blocks are cut into ranges (128 heads) or
    partitions (16 heads) that straddle the part boundaries of several sequences, with bf16
    output."""
    rng = np.random.default_rng(800 + s_q + H)
    B = 10
    sink = [int(v) for v in rng.choice([0, 17, 64, 64], B)]
    middle = [int(v) for v in rng.integers(0, 3000, B)]
    recent = [int(v) for v in rng.integers(2, 600, B)]
    print(f"[case] mixed many ranges H={H} s_q={s_q} B={B}", flush=True)
    o, lse, ref_o, ref_lse = _mixed_case(mla, H, s_q, "5", sink, middle, recent, 900 + s_q + H, o_dtype=torch.bfloat16)
    e = norm_err(o, ref_o)
    el = float(np.max(np.abs(lse - ref_lse)))
    print(f"  o_lat err {e:.3e}  lse abs err {el:.3e}", flush=True)
    assert e <= 4e-3 and el <= 2e-3   # bf16 output: its own rounding (2^-9 relative) on top


@pytest.mark.parametrize("seed", range(8))
def test_mixed_random_sweep(mla, seed):
    """Seeded random mixed histories: 16 or 128 heads, s_q 1 or 2, INT4 or INT2 middle, 1-7
    sequences with random sink (0-130), middle (0-2000) and window (s_q-700) token counts,
    an absent sink part now and then, fp32 or bf16 output.  Against the oracle at the decode
    bar (4e-3 with bf16 output); empty histories give o = 0 and lse = -inf."""
    rng = np.random.default_rng(5000 + seed)
    H = int(rng.choice([16, 128]))
    s_q = int(rng.choice([1, 2]))
    low = str(rng.choice(["4", "5"]))
    B = int(rng.integers(1, 8))
    no_sink = rng.random() < 0.25
    sink = [0 if no_sink else int(v) for v in rng.integers(0, 131, B)]
    middle = [int(v) for v in rng.integers(0, 2001, B)]
    recent = [int(v) for v in rng.integers(s_q, 701, B)]
    if no_sink:
        sink[0] = 0
    bf16_out = bool(rng.random() < 0.5)
    print(f"[case] mixed sweep seed={seed} H={H} s_q={s_q} low={low} B={B} sink={sink} middle={middle} "
          f"recent={recent} bf16_out={bf16_out}", flush=True)
    o, lse, ref_o, ref_lse = _mixed_case(mla, H, s_q, low, sink, middle, recent, 6000 + seed,
                                         o_dtype=torch.bfloat16 if bf16_out else None)
    T = [sink[b] + middle[b] + recent[b] for b in range(B)]
    full = [b for b in range(B) if T[b] > 0]
    e = norm_err(o[full], ref_o[full])
    el = float(np.max(np.abs(lse[full] - ref_lse[full])))
    print(f"  o_lat err {e:.3e}  lse abs err {el:.3e}", flush=True)
    assert e <= (4e-3 if bf16_out else 2e-3) and el <= 2e-3


@pytest.mark.parametrize("H", [16, 128])
def test_mixed_out_of_range_block_ids(mla, H):
    """Block ids outside their part's pool (a negative id in the sink table, one past the pool
    in the middle's, a huge one in the window's) take no part in the softmax: the result is
    the oracle's attention over the remaining tokens (each part checks ids against its own
    pool)."""
    lo_cfg = CONFIGS["4"].with_(H=H)
    hi_cfg = CONFIGS["2"].with_(H=H)
    sink, middle, recent = [64, 100], [300, 700], [130, 70]
    B = 2
    print(f"[case] mixed out-of-range block ids H={H}", flush=True)
    rng = np.random.default_rng(1200 + H)
    T = [sink[b] + middle[b] + recent[b] for b in range(B)]
    rows = [append_rows(lo_cfg, t + 6, 1300 + b) for b, t in enumerate(T)]
    c_all = [to_bf16_exact(r[0][6:]) for r in rows]
    k_all = [to_bf16_exact(r[1][6:]) for r in rows]
    cut = lambda x, b: (x[:sink[b]], x[sink[b]:sink[b] + middle[b]], x[sink[b] + middle[b]:])  # noqa: E731
    pc = [cut(c_all[b], b) for b in range(B)]
    pk = [cut(k_all[b], b) for b in range(B)]
    parts = [_part(mla, cfg, [pc[b][i] for b in range(B)], [pk[b][i] for b in range(B)], rng)
             for i, cfg in enumerate((hi_cfg, lo_cfg, hi_cfg))]
    # knock out: sequence 0's sink block 0, sequence 1's middle block 2, sequence 1's window block 1
    dropped = {(0, 0, 0), (1, 1, 2), (1, 2, 1)}
    for (b, i, blk) in dropped:
        pool, desc, bt, sl, mx = parts[i]
        bt[b, blk] = {0: -1, 1: pool.shape[0], 2: 1 << 30}[i]
    q_lat = to_bf16_exact(rng.standard_normal((B, 1, H, 512)).astype(np.float32) * 0.1)
    q_rope = to_bf16_exact(rng.standard_normal((B, 1, H, 64)).astype(np.float32) * 0.1)
    o, lse = mla.decode_mixed(torch.from_numpy(q_lat).to(torch.bfloat16).to(dev()),
                              torch.from_numpy(q_rope).to(torch.bfloat16).to(dev()), *parts, lo_cfg.sm_scale)
    torch.cuda.synchronize()
    cs, ks, Ts = [], [], []
    for b in range(B):
        keep_c, keep_k = [], []
        for i, cfg in enumerate((hi_cfg, lo_cfg, hi_cfg)):
            lc, lk = _logical(cfg, pc[b][i], pk[b][i])
            lc, lk = lc.reshape(-1, 512), lk.reshape(-1, 64)
            for blk in range(-(-len(lc) // 64)):
                if (b, i, blk) not in dropped:
                    keep_c.append(lc[64 * blk:64 * blk + 64])
                    keep_k.append(lk[64 * blk:64 * blk + 64])
        cs.append(np.concatenate(keep_c))
        ks.append(np.concatenate(keep_k))
        Ts.append(len(cs[-1]))
    ref_o, ref_lse = oracle.attend_latent(q_lat.astype(np.float64), q_rope.astype(np.float64), cs, ks,
                                          np.array(Ts), 1, lo_cfg.sm_scale)
    e = norm_err(o.cpu().numpy(), ref_o)
    el = float(np.max(np.abs(lse.cpu().numpy() - ref_lse)))
    print(f"  o_lat err {e:.3e}  lse abs err {el:.3e}", flush=True)
    assert e <= 2e-3 and el <= 2e-3
