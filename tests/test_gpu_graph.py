"""A decode step recorded in a HIP graph replays to the eager result.

The graph holds the kernel launches of one step, or of three consecutive
steps on the same inputs (as the benchmark records them).  It is replayed three
times; before each replay the outputs are cleared and an unrelated eager step
runs on other buffers, and every replay must reproduce the eager outputs
bit for bit (the kernels are deterministic).
"""

import pytest
import torch

import mla_latent_kv_lat_amd as mla
from mla_inputs import CONFIGS, MLAInputs, scaled
from mla_inputs.device import to_device

pytestmark = pytest.mark.gpu

DT = {"f32": mla.F32, "bf16": mla.BF16, "fp8": mla.FP8_E4M3}


def _step(inp, splits):
    c = inp.cfg
    d = mla.dims(c.batch, c.q_len, c.heads, c.d_nope, c.d_rope, c.d_latent, c.d_v,
                 DT[c.q_dtype], DT[c.kv_dtype])
    dev = to_device(inp)
    args = dict(q_nope=dev.q_nope, q_rope=dev.q_rope, positions=dev.positions, w_uk=dev.w_uk,
                w_uv=dev.w_uv, latent=dev.latent, rope=dev.rope, kv_row_stride=dev.kv_row_stride,
                kv_scale=dev.kv_scale, seq_lens=dev.seq_lens, block_table=dev.block_table,
                max_blocks_per_seq=dev.max_blocks_per_seq, max_seq_len=dev.max_seq_len,
                causal=dev.causal, softmax_scale=dev.softmax_scale, rope_base=dev.rope_base)
    return mla.DecodeStep(d, num_splits=splits), args


@pytest.mark.parametrize("steps", [1, 3])
@pytest.mark.parametrize("name", ["dsv3_b64_ragged_paged", "fp8_b128_l16k_q2"])
def test_graph_replay_matches_eager(name, steps):
    cfg = scaled(CONFIGS[name], batch=5, seq_len=0, len_lo=300, len_hi=3000)
    step, args = _step(MLAInputs(cfg), splits=37)
    other, other_args = _step(MLAInputs(scaled(cfg, seed=cfg.seed + 1)), splits=11)

    step.run(**args)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (step.q_abs, step.o_lat, step.lse, step.o)]

    graph = step.capture(steps=steps, **args)
    for _ in range(3):
        other.run(**other_args)
        for t in (step.q_abs, step.o_lat, step.lse, step.o):
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip((step.q_abs, step.o_lat, step.lse, step.o), ref):
            assert torch.equal(got, want)
