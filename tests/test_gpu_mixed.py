"""GPU parity on mixed small cases: head counts, query lengths, causal
masks, paged and contiguous pools, bf16 and fp8 caches and split counts
combined, each case checked stage by stage against the float64 oracle.

The cases are fixed (seeded); each one crosses several dimensions that the
other parity tests vary one at a time: head counts that are not a multiple of
128 (16, 48, 80 — a partial row group of the decode kernel), 1-3 query
tokens with and without the causal mask, split counts from 1 to more units
than tiles, and ragged lengths with an empty sequence where the contract
allows one (a single query per sequence).
"""

import numpy as np
import pytest

from mla_inputs import CONFIGS, MLAInputs, scaled
from tests.test_gpu_parity import check_all_stages, run_gpu

pytestmark = pytest.mark.gpu

BF16 = CONFIGS["dsv3_b16_l4k"]
FP8 = CONFIGS["fp8_b128_l16k_q2"]

# name, base, heads, q_len, causal, paged, batch, len_lo, len_hi, splits, seed
CASES = [
    ("h16_q1_paged", BF16, 16, 1, False, True, 4, 1, 400, 5, 101),
    ("h48_q2_causal", BF16, 48, 2, True, False, 3, 2, 500, 17, 102),
    ("h64_q3_causal_paged", BF16, 64, 3, True, True, 2, 3, 300, 64, 103),
    ("h128_q1_many_units", BF16, 128, 1, False, False, 2, 100, 600, 256, 104),
    ("h80_q1_units_past_tiles", BF16, 80, 1, False, True, 3, 1, 700, 300, 105),
    ("h32_q3_one_unit", BF16, 32, 3, True, False, 5, 3, 200, 1, 106),
    ("fp8_h16_q2_causal_paged", FP8, 16, 2, True, True, 3, 2, 300, 3, 107),
    ("fp8_h48_q1_paged", FP8, 48, 1, False, True, 4, 1, 600, 40, 108),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_mixed_case(case):
    name, base, heads, q_len, causal, paged, batch, lo, hi, splits, seed = case
    cfg = scaled(base, name=name, heads=heads, q_len=q_len, causal=causal,
                 query_in_cache=causal, paged=paged, batch=batch, seq_len=0,
                 len_lo=lo, len_hi=hi, seed=seed)
    inp = MLAInputs(cfg)
    if q_len == 1 and batch > 2:
        # an empty sequence: its rows give o = 0 and lse = -inf
        inp.seq_lens[1] = 0
        inp.positions[1, 0] = 0
    print(f"[mixed] {name}: lens {inp.seq_lens.tolist()} splits {splits}", flush=True)
    out = run_gpu(inp, num_splits=splits)
    check_all_stages(inp, out)
    if q_len == 1 and batch > 2:
        assert np.all(out["o"][1] == 0) and np.all(np.isneginf(out["lse"][1]))
