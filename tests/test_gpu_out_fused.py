"""GPU parity of the output-side absorption: mla_fuse_out_weight and
mla_out_proj_fused through the C ABI against the float64 oracle
(``oracle.fuse_out_weight``, ``oracle.out_proj_fused``).

Gates, from the arithmetic: each fused weight element is an fp32 sum of
d_v exact bf16 products, rounded once to bf16, so it lies within half a
bf16 ulp of its exact value plus the fp32 sum's error, at most
d_v 2^-24 sum_k |w_o||w_uv|; the test takes, element by element, the error
in units of ulp(exact) + 2 d_v 2^-24 sum_k |w_o||w_uv|.  A correctly
rounded result stays at or below 0.5 of that unit (half an ulp plus at
most half of the sum term), rounding toward zero reaches ~1 and a dropped
product far more: gate 0.75.  A row-normwise bound cannot
give such a margin: one correct rounding of an element near its row's
maximum already moves the row by up to 2^-8.  The projection adds
K = 512 H products of that rounded weight in fp32 and rounds the result to
bf16 (~2e-3 from the weight's independent roundings plus up to 2^-8 from
the output's: gate 1e-2, row-normwise over each query token's outputs).
"""

import numpy as np
import pytest
import torch

import mla_latent_kv_lat_amd as mla
from mla_inputs import OutProjInputs
from oracle import bf16_to_f64, fuse_out_weight, out_proj_fused
from tests._metrics import record, row_rel_err

pytestmark = pytest.mark.gpu

TOL_W_ULPS = 0.75
TOL_OUT = 1e-2


def _dev(u16):
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _dims(inp):
    return mla.dims(inp.m, 1, inp.heads, 128, 64, inp.d_latent, inp.d_v, mla.BF16, mla.BF16)


def run_fused(inp, tensors=None):
    """Fuse the weight, project the latent outputs; returns (w_fused, out)."""
    d = _dims(inp)
    t = tensors or {"o_lat": _dev(inp.o_lat), "w_o": _dev(inp.w_o), "w_uv": _dev(inp.w_uv)}
    H, dc = inp.heads, inp.d_latent
    w_f = torch.full((mla.mla_fused_out_weight_bytes(d, inp.d_model) // 2,), float("nan"),
                     dtype=torch.bfloat16, device="cuda")
    out = torch.full((inp.m, inp.d_model), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mla.mla_out_proj_fused_workspace_bytes(d, inp.d_model) // 4,
                     dtype=torch.float32, device="cuda")
    ws.fill_(float("nan"))  # no initial contents are needed
    mla.mla_fuse_out_weight(d, inp.d_model, t["w_o"], t["w_uv"], w_f)
    mla.mla_out_proj_fused(d, inp.d_model, t["o_lat"], w_f, ws, out)
    torch.cuda.synchronize()
    return w_f, out, t


def fused_rows(inp, w_f, ns):
    """Rows ns of the fused weight, [len(ns), H, d_c], gathered from its
    packed 1 KB blocks (element (n, k) at ((n/32 K/16 + k/16) 64 +
    ((k/8) % 2) 32 + n % 32) 8 + k % 8)."""
    K = inp.heads * inp.d_latent
    w5 = w_f.view(-1, K // 16, 2, 32, 8)
    nb = torch.from_numpy(np.asarray(ns) // 32).cuda()
    r = torch.from_numpy(np.asarray(ns) % 32).cuda()
    return w5[nb, :, :, r, :].reshape(len(ns), inp.heads, inp.d_latent)


def check(inp, w_f, out, rows=None, label=""):
    """w_fused rows `rows` (all if None) against the oracle's fused weight,
    and out[:, rows] against the oracle's projection through it."""
    H = inp.heads
    ns = np.arange(inp.d_model) if rows is None else np.asarray(rows)
    w_o, w_uv = bf16_to_f64(inp.w_o[ns]), bf16_to_f64(inp.w_uv)
    w_ref = fuse_out_weight(w_o, w_uv, H)
    idx = torch.from_numpy(ns).cuda()
    w_got = _np(fused_rows(inp, w_f, ns))
    pad = np.arange(inp.d_model, -(-inp.d_model // 32) * 32)
    if len(pad):
        assert not fused_rows(inp, w_f, pad).float().abs().sum().item(), "padding rows not zero"
    # element-wise, in units of one bf16 ulp of the exact value plus twice
    # the fp32 sum's error bound (the same sums over |w_o| and |w_uv|)
    mag = fuse_out_weight(np.abs(w_o), np.abs(w_uv), H)
    a = np.abs(w_ref)
    ulp = np.where(a > 0, np.exp2(np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7), 2.0 ** -133)
    err_w = float(np.max(np.abs(w_got - w_ref) / (ulp + 2 * inp.d_v * 2.0 ** -24 * mag)))
    err_w_norm = row_rel_err(w_got.reshape(len(ns) * H, -1), w_ref.reshape(len(ns) * H, -1))
    o_ref = out_proj_fused(bf16_to_f64(inp.o_lat), w_ref)
    o_got = _np(out[:, idx])
    assert np.isfinite(_np(out)).all(), "an output was not written"
    err_o = row_rel_err(o_got, o_ref)
    errs = {"w_fused_ulps": err_w, "out": err_o}
    print(f"out_fused {label}: w_fused={err_w:.3f} of the rounding bound (row-normwise "
          f"{err_w_norm:.2e}) out={err_o:.2e}", flush=True)
    record(f"out_fused weight {label}", {"w_fused_ulps": err_w}, TOL_W_ULPS)
    record(f"out_fused out {label}", {"out": err_o}, TOL_OUT)
    assert err_w <= TOL_W_ULPS, err_w
    assert err_o <= TOL_OUT, err_o
    return errs


SMALL = {
    # (query tokens, heads, d_v, d_model); kernel paths: up to 32 rows, up to
    # 64, 128 rows per pass (and several passes); a ragged last feature block
    "m1_h2_d200": (1, 2, 128, 200),
    "m5_h1_dv32": (5, 1, 32, 64),
    "m33_h3_dv64": (33, 3, 64, 256),
    "m64_h4_d1000": (64, 4, 128, 1000),
    "m100_h2_dv96": (100, 2, 96, 130),
    "m300_h1_d129": (300, 1, 128, 129),
}


@pytest.mark.parametrize("case", sorted(SMALL))
def test_out_fused_small(case):
    m, H, dv, dm = SMALL[case]
    inp = OutProjInputs(m, H, dm, seed=20261400 + m + dm, d_v=dv)
    w_f, out, _ = run_fused(inp)
    check(inp, w_f, out, label=case)


def test_out_fused_repeatable_and_workspace_reuse():
    """Same bits on a second run; a smaller call after a larger one on the
    same workspace gives that smaller call's own result."""
    inp = OutProjInputs(64, 4, 1000, seed=20261450)
    w_f, out, t = run_fused(inp)
    w_f2, out2, _ = run_fused(inp, tensors=t)
    assert torch.equal(w_f, w_f2) and torch.equal(out, out2)
    small = OutProjInputs(7, 4, 1000, seed=20261451)
    d = _dims(small)
    ws = torch.empty(mla.mla_out_proj_fused_workspace_bytes(_dims(inp), 1000) // 4,
                     dtype=torch.float32, device="cuda")
    o_big = torch.empty((64, 1000), dtype=torch.bfloat16, device="cuda")
    o_small = torch.empty((7, 1000), dtype=torch.bfloat16, device="cuda")
    mla.mla_out_proj_fused(_dims(inp), 1000, t["o_lat"], w_f, ws, o_big)
    mla.mla_out_proj_fused(d, 1000, _dev(small.o_lat), w_f, ws, o_small)
    torch.cuda.synchronize()
    assert torch.equal(o_big, out)
    ref = out_proj_fused(bf16_to_f64(small.o_lat),
                         fuse_out_weight(bf16_to_f64(inp.w_o), bf16_to_f64(inp.w_uv), 4))
    assert row_rel_err(_np(o_small), ref) <= TOL_OUT


@pytest.mark.timeout(600)
@pytest.mark.parametrize("m", [64, 128])
def test_out_fused_full_size_sampled(m):
    """DeepSeek-V3 shape (128 heads, d_v 128, hidden 7168): one decode
    step's query tokens at batch 64 (one or two tokens per sequence);
    sampled fused-weight rows and every query token's outputs at them."""
    inp = OutProjInputs(m, 128, 7168, seed=20261460 + m)
    print(f"[out_fused fullsize m={m}] inputs ready", flush=True)
    w_f, out, _ = run_fused(inp)
    rng = np.random.default_rng(m)
    rows = np.unique(np.r_[0, 127, 128, 4095, 7167, rng.integers(0, 7168, 19)])
    check(inp, w_f, out, rows=rows, label=f"dsv3 m={m} (sampled)")
