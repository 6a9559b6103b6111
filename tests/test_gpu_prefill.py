"""GPU parity of the MHA-form prefill: mla_prefill_expand and
mla_prefill_attn through the C ABI against the float64 oracle.

The expand step (per-head keys W_UK c and values W_UV c of every cached
token) is compared with ``oracle.mla_expand``; the attention output and LSE
with ``oracle.mla_decode`` on the same inputs (a prompt of q_len tokens is a
multi-token query whose tokens are the last q_len cached ones, causal).
Gates as for decode: row-normwise 2e-2 for bf16, LSE absolute.
"""

import numpy as np
import pytest
import torch

import mla_latent_kv_lat_amd as mla
from mla_inputs import MLAInputs, PREFILL_CONFIGS, scaled
from mla_inputs.device import to_device
from oracle import mla_decode, mla_expand
from tests._metrics import record, row_rel_err, tol_for

pytestmark = pytest.mark.gpu

PF = PREFILL_CONFIGS["prefill_b4_s4k"]


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_prefill(inp, dev=None):
    c = inp.cfg
    dev = dev or to_device(inp)
    d = mla.dims(c.batch, c.q_len, c.heads, c.d_nope, c.d_rope, c.d_latent, c.d_v, mla.BF16, mla.BF16)
    T = dev.max_seq_len
    # rows past a sequence's end are never written; NaN there would reach
    # the outputs if the attention read them
    k_nope = torch.full((c.batch, T, c.heads, c.d_nope), float("nan"), dtype=torch.bfloat16, device="cuda")
    v = torch.full((c.batch, T, c.heads, c.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    o = torch.full((c.batch, c.q_len, c.heads, c.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((c.batch, c.q_len, c.heads), float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_prefill_expand(d, dev.latent, dev.kv_row_stride, dev.seq_lens, dev.block_table,
                           dev.max_blocks_per_seq, mla.TILE_TOKENS, T, dev.w_uk, dev.w_uv, k_nope, v)
    mla.mla_prefill_attn(d, dev.q_nope, dev.q_rope, dev.positions, dev.rope_base, k_nope, v,
                         dev.rope, dev.kv_row_stride, dev.seq_lens, dev.block_table,
                         dev.max_blocks_per_seq, mla.TILE_TOKENS, T, dev.causal, dev.softmax_scale,
                         o, lse)
    torch.cuda.synchronize()
    return {"k_nope": k_nope, "v": v, "o": _np(o), "lse": _np(lse)}


def check_expand(inp, out, tokens_per_seq=None, label=""):
    """k_nope and v against the oracle's expand step on every (or sampled)
    token of each sequence; rows past the end stay untouched."""
    c = inp.cfg
    worst = 0.0
    for b in range(c.batch):
        n = int(inp.seq_lens[b])
        if n == 0:
            continue
        k_ref, v_ref = mla_expand(inp, b)
        ts = np.arange(n) if tokens_per_seq is None else np.unique(
            np.r_[0, n - 1, np.random.default_rng(b).integers(0, n, tokens_per_seq)])
        kt = _np(out["k_nope"][b, torch.from_numpy(ts).cuda()])
        vt = _np(out["v"][b, torch.from_numpy(ts).cuda()])
        worst = max(worst, row_rel_err(kt, k_ref[ts]), row_rel_err(vt, v_ref[ts]))
        if n < out["k_nope"].shape[1]:
            assert torch.isnan(out["k_nope"][b, n:].float()).all(), "rows past the end written"
    record(f"prefill expand {label}", {"k_v": worst}, 1e-2)
    print(f"prefill expand {label}: k/v {worst:.2e}", flush=True)
    assert worst <= 1e-2
    return worst


def check_attn(inp, out, rows=None, label=""):
    c = inp.cfg
    tol = tol_for(c)
    ref = mla_decode(inp, rows=rows)
    if rows is None:
        idx = (slice(None),)
        got_o, ref_o, got_l, ref_l = out["o"], ref["o"], out["lse"], ref["lse"]
    else:
        idx = tuple(np.array(rows).T)
        got_o, ref_o, got_l, ref_l = out["o"][idx], ref["o"][idx], out["lse"][idx], ref["lse"][idx]
    fin = np.isfinite(ref_l)
    assert np.array_equal(fin, np.isfinite(got_l)), "lse -inf pattern differs"
    assert np.isfinite(got_o).all()
    errs = {"o": row_rel_err(got_o, ref_o),
            "lse": float(np.max(np.abs(got_l[fin] - ref_l[fin]))) if fin.any() else 0.0}
    print(f"prefill attn {label}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    record(f"prefill attn {label}", errs, tol)
    for k, e in errs.items():
        assert e <= tol, (k, e, tol)
    return errs


SMALL = {
    # ragged lengths 1..300, a 200-token prompt: sequences shorter than the
    # prompt have queries that see nothing; paged
    "ragged_paged": scaled(PF, name="pf_ragged", batch=3, seq_len=0, len_lo=1, len_hi=300,
                           q_len=200, heads=4, seed=31),
    # the whole sequence is the prompt, three 256-row query blocks, contiguous
    "full_contig": scaled(PF, name="pf_full", batch=2, seq_len=600, q_len=600, heads=2,
                          paged=False, seed=32),
    # no causal mask: every query sees every cached token
    "noncausal": scaled(PF, name="pf_noncausal", batch=2, seq_len=130, q_len=70, heads=3,
                        causal=False, seed=33),
    # a prompt longer than the cache: the first 230 queries see nothing
    "prompt_longer": scaled(PF, name="pf_longer", batch=1, seq_len=70, q_len=300, heads=2,
                            seed=34),
}


@pytest.mark.parametrize("case", sorted(SMALL))
def test_prefill_small(case):
    inp = MLAInputs(SMALL[case])
    out = run_prefill(inp)
    check_expand(inp, out, label=case)
    check_attn(inp, out, label=case)


def test_prefill_lse_optional_and_repeatable():
    """lse may be NULL; two runs on the same inputs give the same bits."""
    inp = MLAInputs(SMALL["ragged_paged"])
    dev = to_device(inp)
    a = run_prefill(inp, dev=dev)
    b = run_prefill(inp, dev=dev)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])
    c = inp.cfg
    d = mla.dims(c.batch, c.q_len, c.heads, c.d_nope, c.d_rope, c.d_latent, c.d_v, mla.BF16, mla.BF16)
    o = torch.empty((c.batch, c.q_len, c.heads, c.d_v), dtype=torch.bfloat16, device="cuda")
    mla.mla_prefill_attn(d, dev.q_nope, dev.q_rope, dev.positions, dev.rope_base, a["k_nope"], a["v"],
                         dev.rope, dev.kv_row_stride, dev.seq_lens, dev.block_table,
                         dev.max_blocks_per_seq, mla.TILE_TOKENS, dev.max_seq_len, dev.causal,
                         dev.softmax_scale, o, None)
    torch.cuda.synchronize()
    assert np.array_equal(_np(o), a["o"])


@pytest.mark.timeout(900)
def test_prefill_full_size_sampled():
    """4 prompts of 4096 tokens, 128 heads: sampled rows against the oracle
    (first and last query of every sequence, queries at block boundaries)."""
    inp = MLAInputs(PF)
    print("[prefill fullsize] inputs ready", flush=True)
    out = run_prefill(inp)
    assert np.isfinite(out["o"]).all() and np.isfinite(out["lse"]).all()
    rng = np.random.default_rng(5)
    rows = set()
    for b in range(PF.batch):
        for i in (0, 1, 255, 256, 4095):
            rows.add((b, i, int(rng.integers(0, PF.heads))))
    for _ in range(12):
        rows.add((int(rng.integers(0, PF.batch)), int(rng.integers(0, PF.q_len)),
                  int(rng.integers(0, PF.heads))))
    rows.update({(1, 1000, h) for h in (0, 127)})
    check_attn(inp, out, rows=sorted(rows), label="prefill_b4_s4k (sampled)")
    check_expand(inp, out, tokens_per_seq=24, label="prefill_b4_s4k (sampled)")
