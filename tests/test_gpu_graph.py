"""Calls recorded in a HIP graph replay to the eager result: a decode step,
and the prefill, cache-append and fused output projection calls.

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


# ---------------------------------------------------------------- other calls
# The same protocol for the calls outside the decode step: record once,
# replay three times with unrelated eager work and cleared outputs between
# replays, bit-identical to the eager call every time.

def _record(fn):
    """One eager call on a side stream, then fn recorded in a HIP graph."""
    cur = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(cur)
    with torch.cuda.stream(side):
        fn()
    cur.wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    return graph


def _replays_match(graph, outs, other):
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    for _ in range(3):
        other()
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert torch.equal(got, want)


def test_graph_prefill_matches_eager():
    from mla_inputs import PREFILL_CONFIGS

    def setup(seed):
        c = scaled(PREFILL_CONFIGS["prefill_b4_s4k"], name="pf_graph", batch=3, seq_len=0,
                   len_lo=1, len_hi=300, q_len=200, heads=4, seed=seed)
        dev = to_device(MLAInputs(c))
        d = mla.dims(c.batch, c.q_len, c.heads, c.d_nope, c.d_rope, c.d_latent, c.d_v,
                     mla.BF16, mla.BF16)
        T = dev.max_seq_len
        bufs = [torch.zeros((c.batch, T, c.heads, c.d_nope), dtype=torch.bfloat16, device="cuda"),
                torch.zeros((c.batch, T, c.heads, c.d_v), dtype=torch.bfloat16, device="cuda"),
                torch.zeros((c.batch, c.q_len, c.heads, c.d_v), dtype=torch.bfloat16, device="cuda"),
                torch.zeros((c.batch, c.q_len, c.heads), dtype=torch.float32, device="cuda")]

        def run():
            mla.mla_prefill_expand(d, dev.latent, dev.kv_row_stride, dev.seq_lens, dev.block_table,
                                   dev.max_blocks_per_seq, mla.TILE_TOKENS, T, dev.w_uk, dev.w_uv,
                                   bufs[0], bufs[1])
            mla.mla_prefill_attn(d, dev.q_nope, dev.q_rope, dev.positions, dev.rope_base, bufs[0],
                                 bufs[1], dev.rope, dev.kv_row_stride, dev.seq_lens, dev.block_table,
                                 dev.max_blocks_per_seq, mla.TILE_TOKENS, T, dev.causal,
                                 dev.softmax_scale, bufs[2], bufs[3])
        return run, bufs

    run, bufs = setup(41)
    other, _ = setup(42)
    _replays_match(_record(run), bufs, other)


def test_graph_kv_append_matches_eager():
    import numpy as np
    from mla_inputs import AppendInputs

    def setup(n, seed):
        inp = AppendInputs(n, 7168, seed=seed)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a.view(np.int16))).cuda().view(torch.bfloat16)
        h, wd, wr, wn = t(inp.h), t(inp.w_dkv), t(inp.w_kr), t(inp.kv_norm_w)
        pos = torch.from_numpy(inp.positions).cuda()
        rows = torch.from_numpy(inp.rows).cuda()
        pool = torch.zeros((inp.pool_rows, 576), dtype=torch.bfloat16, device="cuda")
        d = mla.append_dims(n, 7168)
        ws = torch.empty(mla.mla_kv_append_workspace_bytes(d) // 4, dtype=torch.float32, device="cuda")

        def run():
            mla.mla_kv_append(d, h, wd, wn, wr, pos, 10000.0, 1e-6, rows, pool,
                              pool.view(-1)[512:].data_ptr(), 576, None, ws)
        return run, [pool]

    run, bufs = setup(64, 20261480)
    other, _ = setup(37, 20261481)
    _replays_match(_record(run), bufs, other)


def test_graph_out_fused_matches_eager():
    import numpy as np
    from mla_inputs import OutProjInputs

    def setup(m, seed):
        inp = OutProjInputs(m, 4, 1000, seed=seed)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        o_lat, w_o, w_uv = t(inp.o_lat), t(inp.w_o), t(inp.w_uv)
        d = mla.dims(m, 1, 4, 128, 64, inp.d_latent, inp.d_v, mla.BF16, mla.BF16)
        w_f = torch.zeros((mla.mla_fused_out_weight_bytes(d, 1000) // 2,), dtype=torch.bfloat16,
                          device="cuda")
        out = torch.zeros((m, 1000), dtype=torch.bfloat16, device="cuda")
        ws = torch.empty(mla.mla_out_proj_fused_workspace_bytes(d, 1000) // 4, dtype=torch.float32,
                         device="cuda")

        def run():
            mla.mla_fuse_out_weight(d, 1000, w_o, w_uv, w_f)
            mla.mla_out_proj_fused(d, 1000, o_lat, w_f, ws, out)
        return run, [w_f, out]

    run, bufs = setup(64, 20261490)
    other, _ = setup(7, 20261491)
    _replays_match(_record(run), bufs, other)
