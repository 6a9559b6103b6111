"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Each case runs the four calls of one decode step on seeded inputs and
compares every stage with the oracle: q_abs with the absorbed query and the
rotated RoPE query, o_lat and lse with the absorbed intermediates, and o
with the non-absorbed definition.  Gates (row-normwise max relative error):
1e-5 fp32, 2e-2 bf16, 5e-2 fp8 cache.
"""

import os

import numpy as np
import pytest
import torch

import mla_latent_kv_lat_amd as mla
from mla_inputs import CONFIGS, MLAInputs, scaled
from mla_inputs.device import to_device
from oracle import mla_absorbed, mla_decode
from tests._metrics import record, row_rel_err, tol_for

pytestmark = pytest.mark.gpu

DT = {"f32": mla.F32, "bf16": mla.BF16, "fp8": mla.FP8_E4M3}


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_gpu(inp, *, flags=0, num_splits=None, dev=None):
    c = inp.cfg
    dev = dev or to_device(inp)
    d = mla.dims(c.batch, c.q_len, c.heads, c.d_nope, c.d_rope, c.d_latent, c.d_v,
                 DT[c.q_dtype], DT[c.kv_dtype], flags)
    step = mla.DecodeStep(d, num_splits=num_splits)
    step.run(q_nope=dev.q_nope, q_rope=dev.q_rope, positions=dev.positions, w_uk=dev.w_uk,
             w_uv=dev.w_uv, latent=dev.latent, rope=dev.rope, kv_row_stride=dev.kv_row_stride,
             kv_scale=dev.kv_scale, seq_lens=dev.seq_lens, block_table=dev.block_table,
             max_blocks_per_seq=dev.max_blocks_per_seq, max_seq_len=dev.max_seq_len,
             causal=dev.causal, softmax_scale=dev.softmax_scale, rope_base=dev.rope_base)
    torch.cuda.synchronize()
    return {"q_abs": _np(step.q_abs), "o_lat": _np(step.o_lat), "lse": _np(step.lse),
            "o": _np(step.o), "num_splits": step.num_splits}


def check_all_stages(inp, out, tol=None):
    c = inp.cfg
    tol = tol or tol_for(c)
    ab = mla_absorbed(inp)
    ref = mla_decode(inp)
    errs = {
        "q_lat": row_rel_err(out["q_abs"][..., :c.d_latent], ab["q_lat"]),
        "q_pe": row_rel_err(out["q_abs"][..., c.d_latent:], ab["q_pe"]),
        "o_lat": row_rel_err(out["o_lat"], ab["o_lat"]),
        "o": row_rel_err(out["o"], ref["o"]),
    }
    fin = np.isfinite(ref["lse"])
    assert np.array_equal(fin, np.isfinite(out["lse"])), "lse -inf pattern differs"
    errs["lse"] = float(np.max(np.abs(out["lse"][fin] - ref["lse"][fin]))) if fin.any() else 0.0
    print(c.name, {k: f"{v:.2e}" for k, v in errs.items()}, "splits", out["num_splits"], flush=True)
    record(_label(c, out), errs, tol)
    for k, v in errs.items():
        assert v <= tol, (k, v, tol)
    return errs


def _label(cfg, out):
    t = os.environ.get("PYTEST_CURRENT_TEST", cfg.name).split(" ")[0].split("::")[-1]
    return f"{t} [{cfg.name}, splits {out['num_splits']}]"


def check_rows(inp, out, rows, tol=None, label=None):
    """Stage-by-stage comparison on the (b, i, h) rows given (the oracle's
    cost grows with the rows it computes; large cases sample them)."""
    c = inp.cfg
    tol = tol or tol_for(c)
    idx = tuple(np.array(rows).T)
    ab = mla_absorbed(inp, rows=rows)
    ref = mla_decode(inp, rows=rows)
    fin = np.isfinite(ref["lse"][idx])
    assert np.array_equal(fin, np.isfinite(out["lse"][idx])), "lse -inf pattern differs"
    errs = {
        "q_lat": row_rel_err(out["q_abs"][..., :c.d_latent][idx], ab["q_lat"][idx]),
        "q_pe": row_rel_err(out["q_abs"][..., c.d_latent:][idx], ab["q_pe"][idx]),
        "o_lat": row_rel_err(out["o_lat"][idx], ab["o_lat"][idx]),
        "o": row_rel_err(out["o"][idx], ref["o"][idx]),
        "lse": float(np.max(np.abs(out["lse"][idx][fin] - ref["lse"][idx][fin]))) if fin.any() else 0.0,
    }
    label = label or _label(c, out)
    print(f"{label}: {len(rows)} rows", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    record(f"{label} ({len(rows)} rows)", errs, tol)
    for k, v in errs.items():
        assert v <= tol, (k, v, tol)
    return errs


def spread_rows(inp, n_heads=3, full_seqs=2):
    """Every query of a few heads (first, last and one between) of every
    sequence, plus all heads of the longest and of a middle sequence."""
    c = inp.cfg
    heads = sorted({0, c.heads - 1, *np.linspace(0, c.heads - 1, n_heads).astype(int).tolist()})
    rows = {(b, i, h) for b in range(c.batch) for i in range(c.q_len) for h in heads}
    for b in sorted({int(np.argmax(inp.seq_lens)), c.batch // 2})[:full_seqs]:
        rows |= {(b, i, h) for i in range(c.q_len) for h in range(c.heads)}
    return sorted(rows)


# ---------------------------------------------------------------- fp32

@pytest.mark.parametrize("splits", [None, 1, 2, 5])
def test_tiny_f32(splits):
    inp = MLAInputs(CONFIGS["tiny_f32"])
    check_all_stages(inp, run_gpu(inp, num_splits=splits))


F32_SMALL = scaled(CONFIGS["tiny_f32"], name="f32_ragged", batch=4, seq_len=0, len_lo=1, len_hi=300,
                   heads=6, d_nope=24, d_rope=16, d_latent=40, d_v=20)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("q_len,causal", [(1, False), (2, True), (3, False)])
@pytest.mark.parametrize("splits", [1, 3, 64])
def test_f32_ragged(paged, q_len, causal, splits):
    cfg = scaled(F32_SMALL, paged=paged, q_len=q_len, causal=causal, query_in_cache=causal)
    inp = MLAInputs(cfg)
    check_all_stages(inp, run_gpu(inp, num_splits=splits))


def test_f32_split_invariance_and_paged_equals_contiguous():
    base = scaled(F32_SMALL, batch=3)
    outs = []
    for paged in (False, True):
        inp = MLAInputs(scaled(base, paged=paged))
        for g in (1, 2, 7, 40):
            outs.append(run_gpu(inp, num_splits=g))
    for o in outs[1:]:
        assert row_rel_err(o["o"], outs[0]["o"]) < 2e-6
        assert np.max(np.abs(o["lse"] - outs[0]["lse"])) < 2e-6


def test_f32_empty_sequence_and_single_token():
    cfg = scaled(F32_SMALL, batch=3, len_lo=1, len_hi=65)
    inp = MLAInputs(cfg)
    inp.seq_lens[:] = [0, 1, 65]
    inp.positions[:, 0] = inp.seq_lens
    out = run_gpu(inp, num_splits=4)
    assert np.all(out["o"][0] == 0) and np.all(out["lse"][0] == -np.inf)
    ref = mla_decode(inp, rows=[(b, 0, h) for b in (1, 2) for h in range(cfg.heads)])
    assert row_rel_err(out["o"][1:], ref["o"][1:]) < 1e-5


# ---------------------------------------------------------------- bf16 / fp8

DSV3_SMALL = scaled(CONFIGS["dsv3_b16_l4k"], name="dsv3_small", batch=2, seq_len=0,
                    len_lo=65, len_hi=333)


@pytest.mark.parametrize("flags", [mla.FLAG_GENERIC, 0])
@pytest.mark.parametrize("paged", [False, True])
def test_bf16_dsv3_small(flags, paged):
    inp = MLAInputs(scaled(DSV3_SMALL, paged=paged))
    check_all_stages(inp, run_gpu(inp, flags=flags, num_splits=5))


FP8_SMALL = scaled(CONFIGS["fp8_b128_l16k_q2"], name="fp8_small", batch=2, seq_len=0,
                   len_lo=70, len_hi=200)


@pytest.mark.parametrize("flags", [mla.FLAG_GENERIC, 0])
@pytest.mark.parametrize("paged", [False, True])
def test_fp8_small_causal(flags, paged):
    inp = MLAInputs(scaled(FP8_SMALL, paged=paged))
    check_all_stages(inp, run_gpu(inp, flags=flags, num_splits=3))


# ------------------------------------------------------- MFMA decode path

BF16_RAGGED = scaled(CONFIGS["dsv3_b16_l4k"], name="bf16_ragged", batch=3, seq_len=0,
                     len_lo=1, len_hi=700)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("q_len,causal", [(1, False), (2, True)])
@pytest.mark.parametrize("splits", [1, 7, 300])
def test_bf16_mfma_ragged(paged, q_len, causal, splits):
    cfg = scaled(BF16_RAGGED, paged=paged, q_len=q_len, causal=causal, query_in_cache=causal)
    inp = MLAInputs(cfg)
    check_all_stages(inp, run_gpu(inp, num_splits=splits))


def test_bf16_mfma_matches_generic_kernels():
    inp = MLAInputs(scaled(BF16_RAGGED, paged=True, seed=99))
    dev = to_device(inp)
    a = run_gpu(inp, num_splits=5, dev=dev)
    b = run_gpu(inp, flags=mla.FLAG_GENERIC, num_splits=5, dev=dev)
    assert row_rel_err(a["o_lat"], b["o_lat"]) < 1e-2
    assert np.max(np.abs(a["lse"] - b["lse"])) < 1e-2


FP8_RAGGED = scaled(CONFIGS["fp8_b128_l16k_q2"], name="fp8_ragged", batch=3, seq_len=0,
                    len_lo=2, len_hi=700)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("splits", [1, 7, 300])
def test_fp8_mfma_ragged_causal(paged, splits):
    # two causal queries per sequence, the shortest sequence holding just them
    inp = MLAInputs(scaled(FP8_RAGGED, paged=paged))
    inp.seq_lens[0] = 2
    inp.positions[0] = [0, 1]
    check_all_stages(inp, run_gpu(inp, num_splits=splits))


# More than two draft tokens per sequence (multi-token prediction or
# speculative decoding): 3 and 4 causal queries, 384 and 512 query rows over
# 128 heads, the shortest sequence holding just its queries.
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("q_len", [3, 4])
@pytest.mark.parametrize("splits", [1, 7])
def test_mfma_multi_token_causal(kv, q_len, splits):
    base = BF16_RAGGED if kv == "bf16" else FP8_RAGGED
    cfg = scaled(base, paged=True, q_len=q_len, causal=True, query_in_cache=True, len_lo=q_len,
                 seed=base.seed + q_len)
    inp = MLAInputs(cfg)
    inp.seq_lens[0] = q_len
    inp.positions[0] = np.arange(q_len)
    check_all_stages(inp, run_gpu(inp, num_splits=splits))


def test_fp8_mfma_matches_generic_kernels():
    inp = MLAInputs(scaled(FP8_RAGGED, paged=True, seed=77))
    dev = to_device(inp)
    a = run_gpu(inp, num_splits=5, dev=dev)
    b = run_gpu(inp, flags=mla.FLAG_GENERIC, num_splits=5, dev=dev)
    assert row_rel_err(a["o_lat"], b["o_lat"]) < 2e-2
    assert np.max(np.abs(a["lse"] - b["lse"])) < 2e-2


def test_bf16_mfma_32_heads_and_empty_sequence():
    cfg = scaled(BF16_RAGGED, heads=32, batch=4, len_lo=1, len_hi=200)
    inp = MLAInputs(cfg)
    inp.seq_lens[:] = [130, 0, 64, 1]
    inp.positions[:, 0] = inp.seq_lens
    out = run_gpu(inp, num_splits=3)
    assert np.all(out["o"][1] == 0) and np.all(out["lse"][1] == -np.inf)
    rows = [(b, 0, h) for b in (0, 2, 3) for h in range(32)]
    ref = mla_decode(inp, rows=rows)
    for b in (0, 2, 3):
        assert row_rel_err(out["o"][b], ref["o"][b]) < 2e-2


# Batches of more than 64 sequences take the decode kernels' general setup
# (tile totals summed over lane chunks, the unit's first sequence found by a
# scan, the descriptor window built chunk by chunk).  Short ragged sequences
# keep the oracle cheap; one split makes a unit walk all ~780 tiles and 7
# splits ~110, so the 64-tile window slides many times.
@pytest.mark.parametrize("splits", [None, 7, 1])
@pytest.mark.parametrize("q_len", [1, 2])
def test_bf16_batch_over_64(splits, q_len):
    cfg = scaled(BF16_RAGGED, batch=130, paged=True, q_len=q_len, causal=q_len > 1,
                 query_in_cache=q_len > 1, len_lo=max(1, q_len), len_hi=700, seed=4242 + q_len)
    inp = MLAInputs(cfg)
    inp.seq_lens[5] = q_len      # a sequence holding only its queries
    inp.positions[5] = np.arange(q_len) if q_len > 1 else [q_len]
    out = run_gpu(inp, num_splits=splits)
    check_rows(inp, out, spread_rows(inp))


# Batches of at most 64 whose units span more than 64 tiles: the descriptor
# window slides inside the unit (one split over two ~5000-token sequences).
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("splits", [1, 2])
def test_bf16_long_unit_window_slides(paged, splits):
    cfg = scaled(BF16_RAGGED, batch=2, paged=paged, len_lo=4700, len_hi=5200, seed=515)
    inp = MLAInputs(cfg)
    out = run_gpu(inp, num_splits=splits)
    rows = [(b, 0, h) for b in range(2) for h in (0, 5, 64, 127)]
    check_rows(inp, out, rows)


# ------------------------------------------------ fused combine + W_UV

# batch 130 / 70: 130 and 140 query rows, where the fused kernel takes 64 rows
# per workgroup (64 and 32 sequences per block)
@pytest.mark.parametrize("q_len,causal,batch", [(1, False, 5), (2, True, 5), (1, False, 130),
                                                (2, True, 70)])
def test_combine_out_proj_matches_two_calls(q_len, causal, batch):
    cfg = scaled(BF16_RAGGED, batch=batch, heads=64, paged=True, q_len=q_len, causal=causal,
                 query_in_cache=causal)
    inp = MLAInputs(cfg)
    dev = to_device(inp)
    c = cfg
    d = mla.dims(c.batch, c.q_len, c.heads, c.d_nope, c.d_rope, c.d_latent, c.d_v,
                 DT[c.q_dtype], DT[c.kv_dtype])
    step = mla.DecodeStep(d, num_splits=9)
    step.run(q_nope=dev.q_nope, q_rope=dev.q_rope, positions=dev.positions, w_uk=dev.w_uk,
             w_uv=dev.w_uv, latent=dev.latent, rope=dev.rope, kv_row_stride=dev.kv_row_stride,
             kv_scale=dev.kv_scale, seq_lens=dev.seq_lens, block_table=dev.block_table,
             max_blocks_per_seq=dev.max_blocks_per_seq, max_seq_len=dev.max_seq_len,
             causal=dev.causal, softmax_scale=dev.softmax_scale, rope_base=dev.rope_base)
    torch.cuda.synchronize()
    o_fused, lse_fused, o_lat_fused = step.o.clone(), step.lse.clone(), step.o_lat.clone()
    # the same partials without writing o_lat: identical results
    o2 = torch.empty_like(step.o)
    mla.mla_combine_out_proj(d, 9, dev.seq_lens, step.o_part, step.lse_part, dev.w_uv, o2)
    # the two separate calls on the same partials
    o_lat3 = torch.empty_like(step.o_lat)
    lse3 = torch.empty_like(step.lse)
    o3 = torch.empty_like(step.o)
    mla.mla_combine(d, 9, dev.seq_lens, step.o_part, step.lse_part, o_lat3, lse3)
    mla.mla_out_proj(d, o_lat3, dev.w_uv, o3)
    torch.cuda.synchronize()
    assert torch.equal(o2, o_fused)
    assert row_rel_err(_np(o_lat_fused), _np(o_lat3)) < 1e-2
    assert row_rel_err(_np(o_fused), _np(o3)) < 1e-2
    assert float(torch.max(torch.abs(lse_fused - lse3))) < 1e-5
    # the two separate calls (mla_combine, then mla_out_proj's MFMA kernel)
    # and the fused call, each against the oracle on sampled rows
    q_abs = _np(step.q_abs)
    rows = spread_rows(inp)
    sep = {"q_abs": q_abs, "o_lat": _np(o_lat3), "lse": _np(lse3), "o": _np(o3), "num_splits": 9}
    check_rows(inp, sep, rows, label=f"two calls q_len {q_len} batch {batch}")
    fus = {"q_abs": q_abs, "o_lat": _np(o_lat_fused), "lse": _np(lse_fused), "o": _np(o_fused),
           "num_splits": 9}
    check_rows(inp, fus, rows, label=f"fused call q_len {q_len} batch {batch}")
