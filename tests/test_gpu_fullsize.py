"""GPU parity at the full sizes of all five workloads, in the launch
configuration the benchmark times (split count from mla_num_splits_hint).

The oracle cannot afford every row of a 64 x 8192-token batch, so each case
compares sampled (b, i, h) rows stage by stage (q_abs, o_lat, lse, o): the
first, middle and last sequences plus the longest and shortest, three heads
(two at 131072 tokens), every query token.  The tiny workload is compared
in full.  On all rows, two properties that hold at any size are checked:
outputs are finite, and a different split count gives the same result.
"""

import numpy as np
import pytest

from mla_inputs import CONFIGS, MLAInputs
from mla_inputs.device import to_device
from oracle import mla_absorbed, mla_decode
from tests._metrics import row_rel_err, tol_for
from tests.test_gpu_parity import check_all_stages, run_gpu

pytestmark = pytest.mark.gpu

FULL = ["dsv3_b16_l4k", "dsv3_b64_ragged_paged", "dsv3_b64_l8k_paged", "long_b4_l128k",
        "fp8_b128_l16k_q2", "dsv3_b64_l8k_paged_mtp2"]


def sample_rows(inp):
    c = inp.cfg
    lens = inp.seq_lens
    seqs = sorted({0, c.batch // 2, c.batch - 1, int(np.argmax(lens)), int(np.argmin(lens))})
    heads = [0, c.heads - 1] if c.max_seq_len > 65536 else [0, c.heads // 3, c.heads - 1]
    return [(b, i, h) for b in seqs for i in range(c.q_len) for h in heads]


def test_full_size_tiny_f32():
    inp = MLAInputs(CONFIGS["tiny_f32"])
    check_all_stages(inp, run_gpu(inp))


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
    rows = sample_rows(inp)
    idx = tuple(np.array(rows).T)
    ab = mla_absorbed(inp, rows=rows)
    ref = mla_decode(inp, rows=rows)
    errs = {
        "q_lat": row_rel_err(out["q_abs"][..., :cfg.d_latent][idx], ab["q_lat"][idx]),
        "q_pe": row_rel_err(out["q_abs"][..., cfg.d_latent:][idx], ab["q_pe"][idx]),
        "o_lat": row_rel_err(out["o_lat"][idx], ab["o_lat"][idx]),
        "o": row_rel_err(out["o"][idx], ref["o"][idx]),
        "lse": float(np.max(np.abs(out["lse"][idx] - ref["lse"][idx]))),
    }
    print(f"[fullsize] {name}: {len(rows)} rows, splits {out['num_splits']} / {other}:",
          {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, v in errs.items():
        assert v <= tol, (k, v, tol)
