"""Parity at the full workload sizes, in the launch configuration bench.py times (marked gpu).

Each case builds a workload exactly as bench.py does (same configuration, same seed), runs
mla_decode_paged over the whole batch with the library's own partition plan and the
total-length hint, and checks sampled (sequence, query, head) rows against the float64
oracle, which evaluates those rows one by one (only the sampled sequences are dequantised).
The decode's q_lat input is the oracle's absorbed query rounded to bf16, the same value on
both sides.  Bar: max|gpu - ref| / max|ref| <= 2e-3 over the sampled o_lat rows, lse within
2e-3.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from mla_synth import CONFIGS, SEEDS, make_inputs  # noqa: E402
from tests.gpu_helpers import bf16_exact, desc_of, dev, norm_err, tdtype, to_device  # noqa: E402

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-3


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_02_amd as m
    m.lib()
    return m


def _sampled_rows(seq_lens, s_q, H, rng):
    """The longest and the shortest sequence, the first and last head and query, and a few
    random (b, i, h) triples."""
    B = len(seq_lens)
    bl, bs = int(np.argmax(seq_lens)), int(np.argmin(seq_lens))
    rows = {(bl, 0, 0), (bl, s_q - 1, H - 1), (bs, s_q - 1, 0), (bs, 0, H - 1)}
    for _ in range(4):
        rows.add((int(rng.integers(B)), int(rng.integers(s_q)), int(rng.integers(H))))
    return sorted(rows)


def _logical_rows(x, bs):
    """Float64 latent and RoPE key of the sequences in bs (others None), dequantised if needed."""
    cfg = x.cfg
    c, k = [None] * len(x.seq_lens), [None] * len(x.seq_lens)
    for b in bs:
        L = int(x.seq_lens[b])
        if cfg.quantised:
            cc, kk = oracle.dequant_cache([x.c_codes[b, :L]], [x.c_sz[b, :L]], [x.r_codes[b, :L]], [x.r_sz[b, :L]],
                                          cfg.latent_group, cfg.rope_group)
            c[b], k[b] = cc[0], kk[0]
        else:
            c[b], k[b] = x.c[b, :L].astype(np.float64), x.k_rope[b, :L].astype(np.float64)
    return c, k


@pytest.mark.parametrize("name", ["2", "3", "3b", "4", "5"])
def test_full_size_sampled_rows(mla, name):
    cfg = CONFIGS[name]
    print("[case] full size", cfg.name, flush=True)
    x = make_inputs(cfg, SEEDS[name])
    t = to_device(x)
    B, s_q, H = len(x.seq_lens), cfg.s_q, cfg.H
    q_lat64 = oracle.absorb_q(x.q_nope, x.w_uk)
    if cfg.dtype == "bf16":
        q_lat64 = bf16_exact(q_lat64)
    q_lat = torch.from_numpy(q_lat64).to(tdtype(cfg)).to(dev())
    total = int(x.seq_lens.astype(np.int64).sum())
    out, lse = mla.decode_paged(q_lat, t["q_rope"], t["pool"], desc_of(cfg), t["block_table"], t["seq_lens"],
                                int(x.seq_lens.max()), cfg.sm_scale, num_splits=0, total_seq_len=total)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    lse = lse.cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    rows = _sampled_rows(x.seq_lens, s_q, H, np.random.default_rng(SEEDS[name]))
    c, k = _logical_rows(x, sorted({b for b, _, _ in rows}))
    ref_o, ref_lse = oracle.attend_latent(q_lat64, x.q_rope.astype(np.float64), c, k, x.seq_lens, s_q,
                                          cfg.sm_scale, rows=rows)
    got = np.stack([o[b, i, h] for b, i, h in rows])
    ref = np.stack([ref_o[b, i, h] for b, i, h in rows])
    e = norm_err(got, ref)
    el = max(abs(float(lse[b, i, h]) - float(ref_lse[b, i, h])) for b, i, h in rows)
    print(f"  {len(rows)} rows, o_lat err {e:.3e}, lse abs err {el:.3e}", flush=True)
    assert e <= TOL_BF16
    assert el <= TOL_BF16
