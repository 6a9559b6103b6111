"""Cache-append producer on the GPU against the float64 oracle.

mla_kv_append writes [RMSNorm(W_DKV h) * w | RoPE(W_KR h, pos)] of each new
token into its destination row of a cache pool.  Every other row of the pool
is poisoned with NaN beforehand and must stay untouched.  Gate: 2e-2
row-normwise (bf16), separately for the latent and the RoPE part of each row;
the errors are bf16 rounding of the output (~2e-3).

The fp8 form stores e4m3 codes of the row divided by its scale amax/448.
The code is an integer decided in floating point, so the reference takes that
decision as the kernel does, in fp32, from the oracle's row: the scales must
agree to 1e-5, at most 1% of the codes may differ, each by one step (a value
within fp32 rounding of a rounding boundary), and the dequantised row must
match the float64 row within the fp8 gate, 5e-2 row-normwise.
"""

import numpy as np
import pytest
import torch

import mla_latent_kv_lat_amd as mla
from mla_inputs import AppendInputs
from mla_inputs.generate import fp8_codes_from_f32
from oracle import bf16_to_f64, e4m3_to_f64, kv_append

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


@pytest.mark.parametrize("n,d_model,split_pools", [(64, 7168, False), (37, 5120, True), (3, 512, False)])
def test_kv_append_fp8_matches_oracle(n, d_model, split_pools):
    inp = AppendInputs(n, d_model, seed=20261220 + n)
    dev = torch.device("cuda")
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).view(dt)
    h = t(inp.h.view(np.int16), torch.bfloat16)
    wd = t(inp.w_dkv.view(np.int16), torch.bfloat16)
    wr = t(inp.w_kr.view(np.int16), torch.bfloat16)
    wn = t(inp.kv_norm_w.view(np.int16), torch.bfloat16)
    pos = torch.from_numpy(inp.positions).to(dev)
    rows = torch.from_numpy(inp.rows).to(dev)
    P, stride = inp.pool_rows, 576
    pool = torch.full((P, stride), 0x7F, dtype=torch.uint8, device=dev)   # e4m3 NaN
    rpool = torch.full((P, stride), 0x7F, dtype=torch.uint8, device=dev) if split_pools else pool
    scales = torch.full((P,), float("nan"), dtype=torch.float32, device=dev)
    rope_ptr = rpool.data_ptr() if split_pools else pool.data_ptr() + 512
    d = mla.append_dims(n, d_model, kv_dtype=mla.FP8_E4M3)
    ws = torch.empty(mla.mla_kv_append_workspace_bytes(d) // 4, dtype=torch.float32, device=dev)
    mla.mla_kv_append(d, h, wd, wn, wr, pos, 10000.0, 1e-6, rows, pool, rope_ptr, stride, scales, ws)
    torch.cuda.synchronize()

    ckv, kr = kv_append(bf16_to_f64(inp.h), bf16_to_f64(inp.w_dkv), bf16_to_f64(inp.kv_norm_w),
                        bf16_to_f64(inp.w_kr), inp.positions, 10000.0, 1e-6)
    want = np.concatenate([ckv, kr], axis=1)
    lat = pool.cpu().numpy()
    rop = rpool.cpu().numpy()
    codes = np.concatenate([lat[inp.rows, :512],
                            rop[inp.rows, :64] if split_pools else lat[inp.rows, 512:576]], axis=1)
    sc = scales.cpu().numpy()[inp.rows]
    # the reference decision, in fp32 as the kernel takes it
    r32 = want.astype(np.float32)
    am = np.abs(r32).max(axis=1)
    sc_ref = (am / np.float32(448)).astype(np.float32)
    ref_codes = fp8_codes_from_f32((r32 / sc_ref[:, None]).astype(np.float32))
    assert np.all(np.abs(sc - sc_ref) <= 1e-5 * sc_ref)
    diff = codes != ref_codes
    assert diff.mean() <= 0.01, diff.mean()
    c1, c2 = codes[diff].astype(int), ref_codes[diff].astype(int)
    assert np.all((c1 >> 7) == (c2 >> 7)) and np.all(np.abs((c1 & 0x7F) - (c2 & 0x7F)) == 1)
    got = e4m3_to_f64(codes) * sc[:, None].astype(np.float64)
    err = np.abs(got - want).max(axis=1) / np.abs(want).max(axis=1)
    assert err.max() < 5e-2, err.max()
    mask = np.ones(P, bool)
    mask[inp.rows] = False
    assert (lat[mask] == 0x7F).all() and np.isnan(scales.cpu().numpy()[mask]).all()
    if split_pools:
        assert (rop[mask] == 0x7F).all() and (lat[inp.rows, 512:] == 0x7F).all()


def test_producer_rows_feed_the_decode_path():
    """End to end: mla_kv_append writes every cached row of a small paged
    batch (ragged lengths, permuted 64-token blocks), then the decode step
    (absorb, split-K decode, combine + W_UV) attends over that pool.  The
    oracle builds the same rows with kv_append and attends over them by the
    non-absorbed definition; nothing on the reference side comes from the GPU.
    Gate 2e-2 row-normwise (bf16 cache and queries)."""
    from mla_inputs.generate import bf16_bits_from_f32
    from tests._fake import ArrayInputs
    from oracle import mla_decode

    lens, H, d_model = [100, 64, 257], 16, 1024
    B, n = len(lens), sum(lens)
    app = AppendInputs(n, d_model, seed=20261230)
    pos = np.concatenate([np.arange(L) for L in lens]).astype(np.int32)
    nblk = [(L + 63) // 64 for L in lens]
    perm = np.random.default_rng(5).permutation(sum(nblk))
    mbps = max(nblk)
    bt = np.full((B, mbps), -1, np.int32)
    k = 0
    for b in range(B):
        bt[b, :nblk[b]] = perm[k:k + nblk[b]]
        k += nblk[b]
    rows = np.concatenate([bt[b][np.arange(L) // 64].astype(np.int64) * 64 + np.arange(L) % 64
                           for b, L in enumerate(lens)])
    dev = torch.device("cuda")
    tb = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
    pool = torch.full((sum(nblk) * 64, 576), NAN_BITS, dtype=torch.int16, device=dev).view(torch.bfloat16)
    d_app = mla.append_dims(n, d_model)
    ws = torch.empty(mla.mla_kv_append_workspace_bytes(d_app) // 4, dtype=torch.float32, device=dev)
    mla.mla_kv_append(d_app, tb(app.h), tb(app.w_dkv), tb(app.kv_norm_w), tb(app.w_kr),
                      torch.from_numpy(pos).to(dev), 10000.0, 1e-6, torch.from_numpy(rows).to(dev),
                      pool, pool.view(-1)[512:].data_ptr(), 576, None, ws)

    g = np.random.default_rng(6)
    bits = lambda *s, sd=1.0: bf16_bits_from_f32((g.standard_normal(s) * sd).astype(np.float32))
    qn, qr = bits(B, 1, H, 128), bits(B, 1, H, 64)
    wuk, wuv = bits(H, 128, 512, sd=512 ** -0.5), bits(H, 128, 512, sd=512 ** -0.5)
    qpos = np.array(lens, np.int32)[:, None]
    d = mla.dims(B, 1, H, 128, 64, 512, 128, mla.BF16, mla.BF16)
    step = mla.DecodeStep(d)
    step.run(q_nope=tb(qn), q_rope=tb(qr), positions=torch.from_numpy(qpos).to(dev), w_uk=tb(wuk),
             w_uv=tb(wuv), latent=pool, rope=pool[:, 512:], kv_row_stride=576, kv_scale=None,
             seq_lens=torch.tensor(lens, dtype=torch.int32, device=dev),
             block_table=torch.from_numpy(bt).to(dev), max_blocks_per_seq=mbps,
             max_seq_len=max(lens), causal=False, softmax_scale=192 ** -0.5, rope_base=10000.0)
    torch.cuda.synchronize()
    got = step.o.float().cpu().numpy().astype(np.float64)

    ckv, kr = kv_append(bf16_to_f64(app.h), bf16_to_f64(app.w_dkv), bf16_to_f64(app.kv_norm_w),
                        bf16_to_f64(app.w_kr), pos, 10000.0, 1e-6)
    rows64 = np.concatenate([ckv, kr], axis=1)
    starts = np.cumsum([0] + lens)
    inp = ArrayInputs(q_nope=bf16_to_f64(qn), q_rope=bf16_to_f64(qr), w_uk=bf16_to_f64(wuk),
                      w_uv=bf16_to_f64(wuv), caches=[rows64[starts[b]:starts[b + 1]] for b in range(B)],
                      positions=qpos)
    want = mla_decode(inp)["o"]
    err = np.abs(got - want).max(axis=-1) / np.abs(want).max(axis=-1)
    assert err.max() < 2e-2, err.max()
