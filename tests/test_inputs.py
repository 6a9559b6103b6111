"""The seeded input generator: determinism, value recipe, memory layout."""

import numpy as np

from mla_inputs import BLOCK_TOKENS, CONFIGS, MLAInputs, scaled


def test_same_seed_same_bytes():
    cfg = scaled(CONFIGS["dsv3_b64_ragged_paged"], batch=3, len_lo=70, len_hi=200, heads=32)
    a, b = MLAInputs(cfg), MLAInputs(cfg)
    for name in ("seq_lens", "positions", "q_nope", "q_rope", "w_uk", "w_uv"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    pa, pb = a.pool(), b.pool()
    assert np.array_equal(pa.rows.view(np.uint16), pb.rows.view(np.uint16))
    assert np.array_equal(pa.block_table, pb.block_table)
    c = MLAInputs(cfg, seed=cfg.seed + 1)
    assert not np.array_equal(a.q_nope, c.q_nope)


def test_ragged_lengths_and_positions():
    inp = MLAInputs(CONFIGS["dsv3_b64_ragged_paged"])
    assert inp.seq_lens.min() >= 1024 and inp.seq_lens.max() <= 8192
    assert np.array_equal(inp.positions[:, 0], inp.seq_lens)
    fp8 = MLAInputs(scaled(CONFIGS["fp8_b128_l16k_q2"], batch=2, seq_len=100, heads=32))
    assert np.array_equal(fp8.positions, np.array([[98, 99], [98, 99]]))
    tiny = MLAInputs(CONFIGS["tiny_f32"])
    assert tiny.positions[0, 0] == 64 and tiny.seq_lens[0] == 64


def test_paged_pool_layout_and_poison():
    cfg = scaled(CONFIGS["dsv3_b64_ragged_paged"], batch=4, len_lo=1, len_hi=300, heads=32)
    inp = MLAInputs(cfg)
    pool = inp.pool()
    nblk = [-(-int(n) // BLOCK_TOKENS) for n in inp.seq_lens]
    ids = np.concatenate([pool.block_table[b, :k] for b, k in enumerate(nblk)])
    assert sorted(ids.tolist()) == list(range(sum(nblk)))           # a permutation
    for b, k in enumerate(nblk):
        assert np.all(pool.block_table[b, k:] == -1)
    used = np.zeros(pool.rows.shape[0], bool)
    for b in range(cfg.batch):
        rows, _ = inp.cache_stored(b)
        for t in range(int(inp.seq_lens[b])):
            r = pool.row_index(b, t)
            assert np.array_equal(pool.rows[r], rows[t])
            used[r] = True
    assert np.all(pool.rows[~used] == 0x7FC0)                       # bf16 NaN poison


def test_contiguous_pool_fp8_and_scales():
    cfg = scaled(CONFIGS["fp8_b128_l16k_q2"], batch=2, seq_len=70, heads=32)
    inp = MLAInputs(cfg)
    pool = inp.pool()
    assert pool.rows.dtype == np.uint8 and pool.rows.shape == (2 * 70, 576)
    for b in range(2):
        rows, sc = inp.cache_stored(b)
        r0 = b * 70
        assert np.array_equal(pool.rows[r0:r0 + 70], rows)
        assert np.array_equal(pool.kv_scale[r0:r0 + 70], sc)


def test_outlier_rows():
    cfg = scaled(CONFIGS["long_b4_l128k"], batch=1, seq_len=1000, heads=32)
    x = MLAInputs(cfg).cache_source(0)
    big = np.sqrt((x.astype(np.float64) ** 2).mean(1)) > 4.0
    assert big.sum() == 10                                           # ceil(1% of 1000)


def test_value_distribution():
    cfg = scaled(CONFIGS["dsv3_b16_l4k"], batch=2, seq_len=512)
    inp = MLAInputs(cfg)
    from oracle import bf16_to_f64
    w = bf16_to_f64(inp.w_uk)
    assert abs(w.std() * np.sqrt(512) - 1.0) < 0.01
    x = bf16_to_f64(inp.cache_stored(0)[0])
    assert abs(x.std() - 1.0) < 0.01 and abs(x.mean()) < 0.01
