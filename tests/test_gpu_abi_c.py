"""A decode step through the C ABI from a plain C program (no torch in its
process): tests/abi_c_decode.c reads seeded inputs from files, allocates
with hipMalloc, runs mla_absorb_q, mla_decode_attn and mla_combine_out_proj
on the null stream with the split count mla_num_splits_hint gives, and
writes o and lse back.  They must match the float64 oracle at the bf16 gate
and equal, bit for bit, the same step run through the Python binding."""

import os
import subprocess

import numpy as np
import pytest
import torch

import mla_latent_kv_lat_amd as mla
from mla_inputs import CONFIGS, MLAInputs, scaled
from mla_inputs.device import to_device
from oracle import mla_decode
from tests._cprog import program
from tests._metrics import record, row_rel_err, tol_for

pytestmark = pytest.mark.gpu


def _bf16(u16):
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("paged", [True, False])
def test_decode_step_from_c(tmp_path, paged):
    cfg = scaled(CONFIGS["dsv3_b16_l4k"], name="c_abi", batch=3, seq_len=0, len_lo=1, len_hi=700,
                 paged=paged, seed=20261500 + int(paged))
    inp = MLAInputs(cfg)
    pool = inp.pool()
    c = inp.cfg
    d = str(tmp_path)
    for name, arr in (("q_nope", inp.q_nope), ("q_rope", inp.q_rope), ("positions", inp.positions),
                      ("w_uk", inp.w_uk), ("w_uv", inp.w_uv), ("rows", pool.rows),
                      ("seq_lens", inp.seq_lens)):
        np.ascontiguousarray(arr).tofile(os.path.join(d, name + ".bin"))
    if paged:
        np.ascontiguousarray(pool.block_table, np.int32).tofile(os.path.join(d, "block_table.bin"))
    with open(os.path.join(d, "meta.txt"), "w") as f:
        f.write(f"{c.batch} {c.q_len} {c.heads} {c.d_nope} {c.d_rope} {c.d_latent} {c.d_v} "
                f"{mla.BF16} {mla.BF16} {c.row_width} {pool.max_blocks_per_seq} {pool.max_seq_len} "
                f"{int(c.causal)} {int(paged)} {inp.softmax_scale!r} {inp.rope_base!r}\n")
    exe = program("abi_c_decode", d)
    if exe is None:
        pytest.skip("no C compiler")
    print(f"[c abi] running the C decode step ({exe}), paged={paged}", flush=True)
    r = subprocess.run([exe, d], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    G = int(r.stdout.split()[1])

    shape = (c.batch, c.q_len, c.heads)
    o = _bf16(np.fromfile(os.path.join(d, "o.bin"), np.uint16)).reshape(*shape, c.d_v)
    lse = np.fromfile(os.path.join(d, "lse.bin"), np.float32).astype(np.float64).reshape(shape)

    ref = mla_decode(inp)
    fin = np.isfinite(ref["lse"])
    assert np.array_equal(fin, np.isfinite(lse))
    errs = {"o": row_rel_err(o, ref["o"]),
            "lse": float(np.max(np.abs(lse[fin] - ref["lse"][fin]))) if fin.any() else 0.0}
    tol = tol_for(c)
    record(f"C caller, paged={paged}, splits {G}", errs, tol)
    for k, v in errs.items():
        assert v <= tol, (k, v, tol)

    # the same step through the Python binding, same split count: same bits
    dev = to_device(inp)
    dims = mla.dims(c.batch, c.q_len, c.heads, c.d_nope, c.d_rope, c.d_latent, c.d_v,
                    mla.BF16, mla.BF16)
    step = mla.DecodeStep(dims, num_splits=G, keep_o_lat=False)
    step.run(q_nope=dev.q_nope, q_rope=dev.q_rope, positions=dev.positions, w_uk=dev.w_uk,
             w_uv=dev.w_uv, latent=dev.latent, rope=dev.rope, kv_row_stride=dev.kv_row_stride,
             kv_scale=dev.kv_scale, seq_lens=dev.seq_lens, block_table=dev.block_table,
             max_blocks_per_seq=dev.max_blocks_per_seq, max_seq_len=dev.max_seq_len,
             causal=dev.causal, softmax_scale=dev.softmax_scale, rope_base=dev.rope_base)
    torch.cuda.synchronize()
    o_py = step.o.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(np.fromfile(os.path.join(d, "o.bin"), np.uint16).reshape(o_py.shape), o_py)
    assert np.array_equal(np.fromfile(os.path.join(d, "lse.bin"), np.float32).reshape(shape),
                          step.lse.cpu().numpy())
