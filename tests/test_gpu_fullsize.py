"""GPU parity at the full sizes of all five workloads, in the launch
configuration the benchmark times (split count from mla_num_splits_hint).

The oracle cannot afford every row of a 64 x 8192-token batch, so each case
compares sampled (b, i, h) rows stage by stage (q_abs, o_lat, lse, o): the
first, middle and last sequences plus the longest and shortest, eight heads
spread over the 128, every query token; at 131072 tokens (four sequences)
every sixteenth head of every sequence.  The tiny workload is compared
in full.  On all rows, two properties that hold at any size are checked:
outputs are finite, and a different split count gives the same result.
"""

import numpy as np
import pytest

from mla_inputs import CONFIGS, MLAInputs
from mla_inputs.device import to_device
from tests._metrics import row_rel_err, tol_for
from tests.test_gpu_parity import check_all_stages, check_rows, run_gpu

pytestmark = pytest.mark.gpu

FULL = ["dsv3_b16_l4k", "dsv3_b64_ragged_paged", "dsv3_b64_l8k_paged", "long_b4_l128k",
        "fp8_b128_l16k_q2", "dsv3_b64_l8k_paged_mtp2"]


def sample_rows(inp):
    c = inp.cfg
    lens = inp.seq_lens
    if c.max_seq_len > 65536:
        seqs = list(range(c.batch))
        heads = list(range(0, c.heads, 16))
    else:
        seqs = sorted({0, c.batch // 2, c.batch - 1, int(np.argmax(lens)), int(np.argmin(lens))})
        heads = sorted({*np.linspace(0, c.heads - 1, 8).astype(int).tolist()})
    return [(b, i, h) for b in seqs for i in range(c.q_len) for h in heads]


def test_full_size_tiny_f32():
    inp = MLAInputs(CONFIGS["tiny_f32"])
    check_all_stages(inp, run_gpu(inp))


# the float64 oracle on 32 rows of 131072 tokens takes about a minute of host time
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    cfg = CONFIGS[name]
    inp = MLAInputs(cfg)
    print(f"[fullsize] {name}: inputs ready", flush=True)
    dev = to_device(inp)
    out = run_gpu(inp, dev=dev)
    tol = tol_for(cfg)

    # properties on every row
    assert np.isfinite(out["o"]).all() and np.isfinite(out["o_lat"]).all()
    assert np.isfinite(out["lse"]).all()
    other = max(1, out["num_splits"] // 3 + 1)
    out2 = run_gpu(inp, dev=dev, num_splits=other)
    assert row_rel_err(out2["o_lat"], out["o_lat"]) <= tol
    assert float(np.max(np.abs(out2["lse"] - out["lse"]))) <= tol

    # sampled rows against the oracle
    check_rows(inp, out, sample_rows(inp), tol,
               label=f"full size {name}, splits {out['num_splits']} / {other}")
