"""mla_kv_append_noalloc (partial sums in the library's static device
scratch) against mla_kv_append (caller workspace) through the C ABI: the same
kernels, so the written rows must be bit-identical.  Two calls in a row, the
second with fewer tokens and a different hidden width, so that a stale
scratch from the first call would show; bf16 and fp8 caches."""

import numpy as np
import pytest
import torch

import mla_latent_kv_lat_amd as mla
from mla_inputs import AppendInputs

pytestmark = pytest.mark.gpu

NAN_BITS = 0x7FC0


def _run(inp, n, d_model, kv_dtype, noalloc):
    dev = torch.device("cuda")
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).view(dt)
    h = t(inp.h.view(np.int16), torch.bfloat16)
    wd = t(inp.w_dkv.view(np.int16), torch.bfloat16)
    wr = t(inp.w_kr.view(np.int16), torch.bfloat16)
    wn = t(inp.kv_norm_w.view(np.int16), torch.bfloat16)
    pos = torch.from_numpy(inp.positions).to(dev)
    rows = torch.from_numpy(inp.rows).to(dev)
    P = inp.pool_rows
    f8 = kv_dtype == mla.FP8_E4M3
    d = mla.append_dims(n, d_model, kv_dtype=kv_dtype)
    if f8:
        pool = torch.full((P, 576), 0x7F, dtype=torch.uint8, device=dev)
        scale = torch.full((P,), float("nan"), dtype=torch.float32, device=dev)
        rope = pool.view(-1)[512:].data_ptr()
    else:
        pool = torch.full((P, 576), NAN_BITS, dtype=torch.int16, device=dev).view(torch.bfloat16)
        scale = None
        rope = pool.view(-1)[512:].data_ptr()
    if noalloc:
        mla.mla_kv_append_noalloc(d, h, wd, wn, wr, pos, 10000.0, 1e-6, rows, pool, rope, 576, scale)
    else:
        ws = torch.empty(mla.mla_kv_append_workspace_bytes(d) // 4, dtype=torch.float32, device=dev)
        mla.mla_kv_append(d, h, wd, wn, wr, pos, 10000.0, 1e-6, rows, pool, rope, 576, scale, ws)
    torch.cuda.synchronize()
    out = pool.view(torch.uint8).cpu().numpy().copy()
    return out, (None if scale is None else scale.cpu().numpy().copy())


@pytest.mark.parametrize("kv_dtype", [mla.BF16, mla.FP8_E4M3])
def test_kv_append_noalloc_matches_workspace_call(kv_dtype):
    # first call: 260 tokens at width 7168, the largest batch the scratch holds
    # at that width; second call: 37 tokens at width 5120
    for n, d_model, seed in ((260, 7168, 31), (37, 5120, 32)):
        inp = AppendInputs(n, d_model, seed=20261300 + seed)
        print(f"[no_alloc] kv_dtype {kv_dtype} n {n} d_model {d_model}", flush=True)
        want, want_s = _run(inp, n, d_model, kv_dtype, noalloc=False)
        got, got_s = _run(inp, n, d_model, kv_dtype, noalloc=True)
        assert np.array_equal(got, want)
        if want_s is not None:
            assert np.array_equal(got_s[inp.rows], want_s[inp.rows])
            assert np.isnan(np.delete(got_s, inp.rows)).all()
