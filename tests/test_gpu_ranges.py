"""GPU parity of the many-rows decode path (96 or more query rows per sequence, e.g. 128 heads)
and of batch edge cases shared by both decode paths, against the float64 oracle.

The many-rows path cuts the batch's cache blocks into equal ranges that may cover several
sequences or a part of one; these cases vary the range count (num_splits), mix sequence
lengths, and cover empty sequences and block-table entries outside the pool.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from mla_synth import CONFIGS, make_inputs  # noqa: E402
from tests.gpu_helpers import bf16_exact, desc_of, dev, logical_cache, norm_err, to_device  # noqa: E402
from tests.test_gpu_parity import TOL_BF16, TOL_F32, _decode_stage, assert_bf16_output  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_02_amd as m
    m.lib()
    return m


def _say(*a):
    print("[case]", *a, flush=True)


def _check(o, lse, ref_o, ref_lse, tol=TOL_BF16):
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    e = norm_err(o, ref_o)
    el = float(np.max(np.abs(lse - ref_lse)))
    print(f"  o_lat err {e:.3e}  lse abs err {el:.3e}", flush=True)
    assert e <= tol and el <= tol


@pytest.mark.parametrize("splits", [0, 1, 2, 3, 7])
def test_range_count_invariance(mla, splits):
    """Ranges of every size: whole sequences, pieces, several sequences per range."""
    x = make_inputs(CONFIGS["3"], 47, lens=[1, 64, 200, 900, 65, 3], H=128)
    _say("ranges", splits)
    _check(*_decode_stage(mla, x, num_splits=splits))


@pytest.mark.parametrize("splits", [40, 100])
def test_range_many_pieces_per_sequence(mla, splits):
    """More than 16 ranges per sequence (the combine's wide load batches).  95 blocks over two
    sequences: num_splits = 40 asks for 80 ranges (two blocks each, ~24 partials per row: one
    ragged batch of 32), 100 is capped at one block per range (~48 partials per row: a full
    batch of 32 and a ragged one)."""
    x = make_inputs(CONFIGS["3"], 49, lens=[2900, 3100], H=128)
    _say("many pieces", splits)
    _check(*_decode_stage(mla, x, num_splits=splits))


def test_range_many_sequences_two_queries(mla):
    """s_q = 2 with 128 heads: 256 rows, two row groups over the same ranges."""
    rng = np.random.default_rng(5)
    lens = [int(v) for v in rng.integers(2, 700, size=20)]
    x = make_inputs(CONFIGS["3b"], 48, lens=lens, H=128)
    _say("many sequences s_q=2", lens)
    _check(*_decode_stage(mla, x))


@pytest.mark.parametrize("name,lens", [("4", [64, 333, 1030]), ("5", [1, 65, 700])])
def test_range_quantised(mla, name, lens):
    x = make_inputs(CONFIGS[name], 49, lens=lens, H=128)
    _say("quantised ranges", name, lens)
    _check(*_decode_stage(mla, x))


def test_range_bf16_output(mla):
    x = make_inputs(CONFIGS["3"], 50, lens=[100, 333, 7], H=128)
    _say("bf16 o_lat ranges")
    for splits in (0, 1, 3):
        o, lse, ref_o, ref_lse = _decode_stage(mla, x, num_splits=splits, o_dtype=torch.bfloat16)
        assert_bf16_output(o, ref_o, TOL_BF16)


def test_range_deterministic(mla):
    cfg = CONFIGS["3"]
    x = make_inputs(cfg, 51, lens=[300, 1000, 17], H=128)
    t = to_device(x)
    q = torch.from_numpy(bf16_exact(oracle.absorb_q(x.q_nope, x.w_uk))).to(torch.bfloat16).to(dev())
    _say("range determinism")
    outs = []
    for _ in range(2):
        o, l = mla.decode_paged(q, t["q_rope"], t["pool"], desc_of(cfg), t["block_table"], t["seq_lens"],
                                1000, cfg.sm_scale)
        outs.append((o.cpu().numpy().copy(), l.cpu().numpy().copy()))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("name,H", [("3", 128), ("3b", 112)])
def test_range_workspace_reuse(mla, name, H):
    """The workspace carries nothing from one call to the next: one holding stale bytes (all
    0x7F) and the same workspace reused call after call give the bits of a zeroed one, with or
    without lse.  112 heads x 2 queries leave a second row group of 96 rows; 30 ranges over these
    lengths give sequences of one piece and of several, and ranges that hold several sequences."""
    x = make_inputs(CONFIGS[name], 53, lens=[2, 700, 2900, 64, 3, 450], H=H)
    t = to_device(x)
    q_lat64 = bf16_exact(oracle.absorb_q(x.q_nope, x.w_uk))
    q = torch.from_numpy(q_lat64).to(torch.bfloat16).to(dev())
    args = (q, t["q_rope"], t["pool"], desc_of(x.cfg), t["block_table"], t["seq_lens"], int(x.seq_lens.max()),
            x.cfg.sm_scale)
    n = mla.decode_workspace_size(*args, num_splits=30)
    ws = torch.zeros(max(n, 256), dtype=torch.uint8, device=dev())
    _say("workspace reuse", name, H)
    runs = []
    for fill, want_lse in ((0, True), (0x7F, True), (None, True), (None, False), (None, True)):
        if fill is not None:
            ws.fill_(fill)
        o, l = mla.decode_paged(*args, num_splits=30, workspace=ws, want_lse=want_lse)
        torch.cuda.synchronize()
        runs.append((o.cpu().numpy(), None if l is None else l.cpu().numpy()))
    for o, l in runs[1:]:
        np.testing.assert_array_equal(o, runs[0][0])
        if l is not None:
            np.testing.assert_array_equal(l, runs[0][1])
    c, k = logical_cache(x)
    ref_o, ref_lse = oracle.attend_latent(q_lat64, x.q_rope.astype(np.float64), c, k, x.seq_lens, x.cfg.s_q,
                                          x.cfg.sm_scale)
    _check(runs[0][0], runs[0][1], ref_o, ref_lse)


@pytest.mark.parametrize("name,splits", [("2", 3), ("2", 12), ("4", 12)])
def test_partition_workspace_stale_bytes(mla, name, splits):
    """Partition mode (16 heads): the merge reads a partition slot only when the sequence has
    that partition.  A workspace full of NaN (0xFF) or of huge finite values (0x7F), and one
    reused call after call, give the bits of a zeroed one.  Twelve partitions take the merge's
    second batch of eight, and the short sequences leave most of their partition slots
    unwritten by the decode (bf16 cache: the partition kernel; INT4: the pipelined kernel)."""
    x = make_inputs(CONFIGS[name], 61, lens=[1, 64, 200, 2900, 1500, 5], H=16)
    t = to_device(x)
    q_lat64 = bf16_exact(oracle.absorb_q(x.q_nope, x.w_uk))
    q = torch.from_numpy(q_lat64).to(torch.bfloat16).to(dev())
    args = (q, t["q_rope"], t["pool"], desc_of(x.cfg), t["block_table"], t["seq_lens"], int(x.seq_lens.max()),
            x.cfg.sm_scale)
    plan = mla.decode_plan(*args, num_splits=splits)
    assert plan[0] == splits, plan
    n = mla.decode_workspace_size(*args, num_splits=splits)
    ws = torch.zeros(max(n, 256), dtype=torch.uint8, device=dev())
    _say("partition workspace", name, splits)
    runs = []
    for fill in (0, 0xFF, 0x7F, None):
        if fill is not None:
            ws.fill_(fill)
        o, l = mla.decode_paged(*args, num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        runs.append((o.cpu().numpy(), l.cpu().numpy()))
    for o, l in runs[1:]:
        np.testing.assert_array_equal(o, runs[0][0])
        np.testing.assert_array_equal(l, runs[0][1])
    c, k = logical_cache(x)
    ref_o, ref_lse = oracle.attend_latent(q_lat64, x.q_rope.astype(np.float64), c, k, x.seq_lens, x.cfg.s_q,
                                          x.cfg.sm_scale)
    _check(runs[0][0], runs[0][1], ref_o, ref_lse)


def _run(mla, x, seq_lens, block_table, splits=0):
    cfg = x.cfg
    t = to_device(x)
    if cfg.dtype == "f32":
        q_lat64 = oracle.absorb_q(x.q_nope, x.w_uk).astype(np.float32).astype(np.float64)
        q = torch.from_numpy(q_lat64.astype(np.float32)).to(dev())
    else:
        q_lat64 = bf16_exact(oracle.absorb_q(x.q_nope, x.w_uk))
        q = torch.from_numpy(q_lat64).to(torch.bfloat16).to(dev())
    o, l = mla.decode_paged(q, t["q_rope"], t["pool"], desc_of(cfg), torch.from_numpy(block_table).to(dev()),
                            torch.from_numpy(seq_lens).to(dev()), int(x.seq_lens.max()), cfg.sm_scale,
                            num_splits=splits)
    torch.cuda.synchronize()
    return q_lat64, o.float().cpu().numpy(), l.cpu().numpy()


@pytest.mark.parametrize("name,H", [("1", 8), ("2", 16), ("3", 128)])
def test_empty_sequences(mla, name, H):
    """A sequence of length 0 attends to nothing: o = 0, lse = -inf; the others are unaffected
    (fp32 cache kernel, partition kernel, row-owner kernel)."""
    x = make_inputs(CONFIGS[name], 52, lens=[100, 1, 300, 1, 65], H=H)
    lens = x.seq_lens.copy()
    lens[[1, 3]] = 0
    _say("empty sequences", name, H)
    for splits in (0, 2):
        q_lat64, o, lse = _run(mla, x, lens, x.block_table, splits)
        assert np.all(o[[1, 3]] == 0.0) and np.all(lse[[1, 3]] == -np.inf)
        keep = [0, 2, 4]
        c, k = logical_cache(x)
        ref_o, ref_lse = oracle.attend_latent(q_lat64[keep], x.q_rope[keep].astype(np.float64),
                                              [c[b] for b in keep], [k[b] for b in keep], x.seq_lens[keep],
                                              x.cfg.s_q, x.cfg.sm_scale)
        _check(o[keep], lse[keep], ref_o, ref_lse, _tol(x))


def _tol(x):
    return TOL_F32 if x.cfg.dtype == "f32" else TOL_BF16


@pytest.mark.parametrize("name,H", [("1", 8), ("2", 16), ("3", 128)])
def test_out_of_range_block_ids_are_skipped(mla, name, H):
    """Tokens of a block-table entry outside [0, num_blocks) take no part in the softmax:
    the result equals attention over the sequence with that block's tokens removed."""
    x = make_inputs(CONFIGS[name], 53, lens=[300, 200], H=H)
    bt = x.block_table.copy()
    nblocks = x.pool.shape[0]
    bt[0, 1] = -1
    bt[1, 2] = nblocks + 5
    _say("out-of-range ids", name, H)
    q_lat64, o, lse = _run(mla, x, x.seq_lens, bt)
    c, k = logical_cache(x)
    keep0 = np.r_[0:64, 128:300]
    keep1 = np.r_[0:128, 192:200]
    c2 = [c[0][keep0], c[1][keep1]]
    k2 = [k[0][keep0], k[1][keep1]]
    ref_o, ref_lse = oracle.attend_latent(q_lat64, x.q_rope.astype(np.float64), c2, k2,
                                          np.array([len(keep0), len(keep1)]), x.cfg.s_q, x.cfg.sm_scale)
    _check(o, lse, ref_o, ref_lse, _tol(x))


def test_range_start_charge(mla):
    """Ranges cut a block space in which each non-empty sequence's start counts 3 extra
    positions (the sequence starts here are off the plain range boundaries).  Lengths within
    the V3 workload's [1024, 8192].  [2000, 2000] with 24 ranges of 3 positions: the first range
    holds only start positions and does no work, one range ends with the second sequence's
    start positions and the next begins with them.  [1100, 0, 2000, 1300] with 28 ranges adds
    an empty sequence (written by the range holding its position), a range in the middle that
    holds only start positions, and a last range with no position at all."""
    x = make_inputs(CONFIGS["3"], 53, lens=[2000, 2000], H=128)
    _say("start charge", [2000, 2000], 12)
    _check(*_decode_stage(mla, x, num_splits=12))
    x = make_inputs(CONFIGS["3"], 54, lens=[1100, 1, 2000, 1300], H=128)
    lens = x.seq_lens.copy()
    lens[1] = 0
    _say("start charge", [int(v) for v in lens], 7)
    q_lat64, o, lse = _run(mla, x, lens, x.block_table, 7)
    assert np.all(o[1] == 0.0) and np.all(lse[1] == -np.inf)
    keep = [0, 2, 3]
    c, k = logical_cache(x)
    ref_o, ref_lse = oracle.attend_latent(q_lat64[keep], x.q_rope[keep].astype(np.float64),
                                          [c[b] for b in keep], [k[b] for b in keep], x.seq_lens[keep],
                                          x.cfg.s_q, x.cfg.sm_scale)
    _check(o[keep], lse[keep], ref_o, ref_lse)


def test_range_max_batch(mla):
    """The row-owner path at its largest batch, 8192 sequences (its sequence table is three LDS
    arrays of 8193 entries), 96 heads, lengths 0..64 (one block each, some empty).  Seeded
    bf16 rows, queries and a shuffled block table; a sample of sequences (the empty ones,
    the longest, random others) against the oracle, which sees only those."""
    B, H, d_c, d_r = 8192, 96, 512, 64
    rng = np.random.default_rng(91)
    lens = rng.integers(0, 65, size=B).astype(np.int32)
    lens[[5, 4000]] = 0
    lens[[17, 8191]] = 64
    perm = rng.permutation(B + 3).astype(np.int32)
    table = perm[:B].reshape(B, 1).copy()
    _say("max batch", B, H)
    rows = rng.standard_normal((B + 3, 64, d_c + d_r), dtype=np.float32)
    rows_b = (rows.view(np.uint32) + 0x7FFF + ((rows.view(np.uint32) >> 16) & 1)) >> 16   # bf16 bits, RNE
    pool = rows_b.astype(np.uint16).view(np.uint8).reshape(B + 3, -1)
    del rows
    q = rng.standard_normal((B, 1, H, d_c + d_r), dtype=np.float32) * 0.05
    qb = ((q.view(np.uint32) + 0x7FFF + ((q.view(np.uint32) >> 16) & 1)) >> 16).astype(np.uint16)
    del q
    q_t = torch.from_numpy(qb.view(np.int16)).to(dev()).view(torch.bfloat16)
    cfg = CONFIGS["3"].with_(H=H)
    o, lse = mla.decode_paged(q_t[..., :d_c].contiguous(), q_t[..., d_c:].contiguous(), torch.from_numpy(pool).to(dev()),
                              desc_of(cfg), torch.from_numpy(table).to(dev()), torch.from_numpy(lens).to(dev()), 64,
                              cfg.sm_scale)
    torch.cuda.synchronize()
    sel = sorted({5, 4000, 17, 8191, 0, 1} | {int(v) for v in rng.integers(0, B, 10)})
    o = o[sel].float().cpu().numpy()
    lse = lse[sel].cpu().numpy()
    bf = lambda u: (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)   # noqa: E731
    live = [i for i, b in enumerate(sel) if lens[b] > 0]
    for i, b in enumerate(sel):
        if lens[b] == 0:
            assert np.all(o[i] == 0.0) and np.all(lse[i] == -np.inf)
    c = [bf(rows_b[table[sel[i], 0], :lens[sel[i]], :d_c]) for i in live]
    k = [bf(rows_b[table[sel[i], 0], :lens[sel[i]], d_c:]) for i in live]
    qs = bf(qb[[sel[i] for i in live]])
    ref_o, ref_lse = oracle.attend_latent(qs[..., :d_c], qs[..., d_c:], c, k, lens[[sel[i] for i in live]], 1,
                                          cfg.sm_scale)
    _check(o[live], lse[live], ref_o, ref_lse)


@pytest.mark.parametrize("H", [128, 16])
def test_all_sequences_empty(mla, H):
    """Every sequence of length 0 (both decode paths): o_lat = 0 and lse = -inf everywhere."""
    cfg = CONFIGS["3"].with_(H=H)
    B = 5
    _say("all empty", H)
    q = torch.randn((B, 1, H, 512), device=dev()).to(torch.bfloat16)
    r = torch.randn((B, 1, H, 64), device=dev()).to(torch.bfloat16)
    pool = torch.zeros((2, mla.block_bytes(desc_of(cfg))), dtype=torch.uint8, device=dev())
    table = torch.zeros((B, 1), dtype=torch.int32, device=dev())
    lens = torch.zeros(B, dtype=torch.int32, device=dev())
    o, lse = mla.decode_paged(q, r, pool, desc_of(cfg), table, lens, 1, cfg.sm_scale)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isinf(lse) & (lse < 0))
