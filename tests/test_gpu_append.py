"""Cache-append producer on the GPU against the float64 oracle.

mla_kv_append writes [RMSNorm(W_DKV h) * w | RoPE(W_KR h, pos)] of each new
token into its destination row of a cache pool.  Every other row of the pool
is poisoned with NaN beforehand and must stay untouched.  Gate: 2e-2
row-normwise (bf16), separately for the latent and the RoPE part of each row;
the errors are bf16 rounding of the output (~2e-3).
"""

import numpy as np
import pytest
import torch

import mla_latent_kv_lat_amd as mla
from mla_inputs import AppendInputs
from oracle import bf16_to_f64, kv_append

pytestmark = pytest.mark.gpu

NAN_BITS = 0x7FC0


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("n,d_model,stride,split_pools", [
    (1, 512, 576, False),       # one token, one hidden chunk
    (5, 1024, 576, False),      # fewer tokens than one MFMA block
    (64, 7168, 576, False),     # DeepSeek-V3 width, a batch of 64 new tokens
    (130, 7168, 640, False),    # three token groups, padded rows
    (37, 5120, 576, True),      # DeepSeek-V2 width, latent and RoPE in two pools
])
def test_kv_append_matches_oracle(n, d_model, stride, split_pools):
    inp = AppendInputs(n, d_model, seed=20261210 + n)
    dev = torch.device("cuda")
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).view(dt)
    h = t(inp.h.view(np.int16), torch.bfloat16)
    wd = t(inp.w_dkv.view(np.int16), torch.bfloat16)
    wr = t(inp.w_kr.view(np.int16), torch.bfloat16)
    wn = t(inp.kv_norm_w.view(np.int16), torch.bfloat16)
    pos = torch.from_numpy(inp.positions).to(dev)
    rows = torch.from_numpy(inp.rows).to(dev)
    P = inp.pool_rows
    pool = torch.full((P, stride), NAN_BITS, dtype=torch.int16, device=dev).view(torch.bfloat16)
    if split_pools:
        rpool = torch.full((P, stride), NAN_BITS, dtype=torch.int16, device=dev).view(torch.bfloat16)
        lat_ptr, rope_ptr = pool, rpool
    else:
        rpool = pool
        lat_ptr, rope_ptr = pool, pool.view(-1)[512:]
    d = mla.append_dims(n, d_model)
    ws = torch.empty(mla.mla_kv_append_workspace_bytes(d) // 4, dtype=torch.float32, device=dev)
    mla.mla_kv_append(d, h, wd, wn, wr, pos, 10000.0, 1e-6, rows, lat_ptr, rope_ptr.data_ptr(),
                      stride, None, ws)
    torch.cuda.synchronize()

    ckv, kr = kv_append(bf16_to_f64(inp.h), bf16_to_f64(inp.w_dkv), bf16_to_f64(inp.kv_norm_w),
                        bf16_to_f64(inp.w_kr), inp.positions, 10000.0, 1e-6)
    lat = _bits(pool)
    rop = _bits(rpool)
    got_l = bf16_to_f64(lat[inp.rows, :512])
    got_r = bf16_to_f64(rop[inp.rows, 512:576] if not split_pools else rop[inp.rows, :64])
    for got, want in ((got_l, ckv), (got_r, kr)):
        err = np.abs(got - want).max(axis=1) / np.abs(want).max(axis=1)
        assert np.isfinite(got).all()
        assert err.max() < 2e-2, err.max()
    # nothing else was written
    mask = np.ones(P, bool)
    mask[inp.rows] = False
    assert (lat[mask] == NAN_BITS).all()
    if split_pools:
        assert (rop[mask] == NAN_BITS).all()
        assert (lat[inp.rows, 512:] == NAN_BITS).all()
        assert (rop[inp.rows, 64:] == NAN_BITS).all()
    else:
        assert (lat[inp.rows, 576:] == NAN_BITS).all()
