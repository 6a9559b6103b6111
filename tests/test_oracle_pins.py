"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test ties one part of the oracle to the mathematics (closed forms,
invariants, special cases), to a library routine, to brute force on tiny
inputs, or to numbers printed on the pages.  The dimensions are chosen all
distinct (d_nope != d_latent != d_v, ...) so that a transposed weight, a
dropped term or a swapped operand fails on shape or on value.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from mla_inputs import CONFIGS, MLAInputs, scaled
from mla_inputs.generate import bf16_bits_from_f32
from oracle import (bf16_to_f64, e4m3_to_f64, fuse_out_weight, kv_cache_bytes_per_token,
                    mla_absorbed, mla_decode, mla_expand, out_proj_fused, rope_interleaved)
from tests._fake import ArrayInputs, random_arrays

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# all-distinct small dims: H=3, d_nope=12, d_rope=8, d_latent=24, d_v=20
DIMS = dict(H=3, d_n=12, d_R=8, d_c=24, d_v=20)


def _arrays(seed, B=2, Lq=1, lens=(7, 5), **kw):
    d = dict(DIMS)
    d.update(kw)
    rng = np.random.default_rng(seed)
    return random_arrays(rng, B, Lq, d["H"], d["d_n"], d["d_R"], d["d_c"], d["d_v"], list(lens))


# ---------------------------------------------------------------- codecs

def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(3.0),
        np.array([0.0, -0.0, 1.0, -2.5, 3.3895314e38, 1e-40, -1e-45, 1.00390625, 1.01171875],
                 np.float32)])
    ours = bf16_to_f64(bf16_bits_from_f32(x))
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_e4m3_all_256_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    np.testing.assert_array_equal(ours[~np.isnan(ours)], ref[~np.isnan(ref)])
    # format landmarks: largest finite 448, smallest normal 2^-6, smallest subnormal 2^-9
    assert ours[0x7E] == 448.0 and ours[0x08] == 2.0 ** -6 and ours[0x01] == 2.0 ** -9
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF]) and ours[0x80] == 0.0


# ------------------------------------------------------------------ RoPE

def test_rope_position_zero_is_identity():
    x = np.random.default_rng(2).standard_normal((5, 16))
    np.testing.assert_array_equal(rope_interleaved(x, 0, 10000.0), x)


def test_rope_rotation_direction_and_pairing():
    # pair 0 has frequency 1: (1, 0) -> (cos p, sin p), (0, 1) -> (-sin p, cos p)
    d = 8
    e0 = np.zeros(d); e0[0] = 1.0
    e1 = np.zeros(d); e1[1] = 1.0
    for p in (1, 3, 64):
        r0 = rope_interleaved(e0, p, 10000.0)
        r1 = rope_interleaved(e1, p, 10000.0)
        np.testing.assert_allclose(r0[:2], [math.cos(p), math.sin(p)], rtol=0, atol=1e-15)
        np.testing.assert_allclose(r1[:2], [-math.sin(p), math.cos(p)], rtol=0, atol=1e-15)
        assert np.all(r0[2:] == 0) and np.all(r1[2:] == 0)


def test_rope_frequency_schedule():
    # pair k of a 16-wide vector turns by base^(-2k/16) per position step
    d, base = 16, 10000.0
    for k in range(d // 2):
        x = np.zeros(d); x[2 * k] = 1.0
        r = rope_interleaved(x, 1, base)
        ang = math.atan2(r[2 * k + 1], r[2 * k])
        assert abs(ang - base ** (-2.0 * k / d)) < 1e-15
    assert abs(10000.0 ** (-1.0 / 8.0) - 0.31622776601683794) < 1e-15


def test_rope_preserves_norm_and_is_relative():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m, n in [(131072, 5), (700, 699), (9, 130000)]:
        rq, rk = rope_interleaved(q, m, 10000.0), rope_interleaved(k, n, 10000.0)
        assert abs(np.linalg.norm(rq) - np.linalg.norm(q)) < 1e-12
        lhs = rq @ rk
        rhs = rope_interleaved(q, m - n, 10000.0) @ k
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(lhs))


# ------------------------------------------------------- closed forms

@pytest.mark.parametrize("Lq,causal", [(1, False), (2, True)])
def test_absorbed_equals_unabsorbed(Lq, causal):
    """[ARCH] 3.1/3.2: (W^T q).c == q.(W c) and W_UV sum p c == sum p W_UV c."""
    arr = _arrays(5, B=3, Lq=Lq, lens=(9, 1, 17))
    inp = ArrayInputs(**arr, causal=causal)
    ref = mla_decode(inp)
    ab = mla_absorbed(inp)
    fin = np.isfinite(ref["lse"])
    np.testing.assert_allclose(ab["lse"][fin], ref["lse"][fin], rtol=1e-12, atol=0)
    num = np.max(np.abs(ab["o"] - ref["o"]), axis=-1)
    den = np.max(np.abs(ref["o"]), axis=-1)
    assert np.all(num <= 1e-12 * den)


def _brute(inp):
    """Per-element definition with scalar Python loops (tiny inputs only)."""
    cfg = inp.cfg
    out = {}
    for b in range(cfg.batch):
        rows = [list(map(float, r)) for r in inp.caches[b]]
        L = len(rows)
        for i in range(cfg.q_len):
            pos = int(inp.positions[b, i])
            for h in range(cfg.heads):
                qn = [float(v) for v in inp.q_nope[b, i, h]]
                qr_raw = [float(v) for v in inp.q_rope[b, i, h]]
                qr = [0.0] * cfg.d_rope
                for k in range(cfg.d_rope // 2):
                    a = pos * cfg.rope_base ** (-2.0 * k / cfg.d_rope)
                    x0, x1 = qr_raw[2 * k], qr_raw[2 * k + 1]
                    qr[2 * k] = x0 * math.cos(a) - x1 * math.sin(a)
                    qr[2 * k + 1] = x0 * math.sin(a) + x1 * math.cos(a)
                scores, vals = [], []
                for t in range(L):
                    if cfg.causal and t > L - cfg.q_len + i:
                        continue
                    c = rows[t][:cfg.d_latent]
                    kr = rows[t][cfg.d_latent:]
                    s = 0.0
                    for d in range(cfg.d_nope):
                        kd = sum(float(inp.w_uk[h, d, j]) * c[j] for j in range(cfg.d_latent))
                        s += qn[d] * kd
                    s += sum(qr[j] * kr[j] for j in range(cfg.d_rope))
                    scores.append(s / math.sqrt(cfg.d_nope + cfg.d_rope))
                    vals.append([sum(float(inp.w_uv[h, v, j]) * c[j] for j in range(cfg.d_latent))
                                 for v in range(cfg.d_v)])
                m = max(scores)
                w = [math.exp(s - m) for s in scores]
                z = sum(w)
                o = [sum(w[t] * vals[t][v] for t in range(len(w))) / z for v in range(cfg.d_v)]
                out[(b, i, h)] = (np.array(o), m + math.log(z))
    return out


@pytest.mark.parametrize("Lq,causal", [(1, False), (2, True)])
def test_oracle_matches_brute_force(Lq, causal):
    arr = _arrays(6, B=2, Lq=Lq, lens=(5, 3), H=2)
    inp = ArrayInputs(**arr, causal=causal)
    ref = mla_decode(inp)
    for (b, i, h), (o, lse) in _brute(inp).items():
        np.testing.assert_allclose(ref["o"][b, i, h], o, rtol=1e-12, atol=1e-14)
        assert abs(ref["lse"][b, i, h] - lse) < 1e-12


@pytest.mark.parametrize("Lq,causal", [(1, False), (2, True), (2, False)])
def test_oracle_matches_torch_sdpa(Lq, causal):
    """torch's float64 scaled_dot_product_attention on explicitly built K, V."""
    arr = _arrays(7, B=2, Lq=Lq, lens=(33, 8))
    inp = ArrayInputs(**arr, causal=causal)
    ref = mla_decode(inp)
    d = DIMS
    for b in range(2):
        cache = torch.from_numpy(inp.caches[b]).double()
        L = cache.shape[0]
        c, kr = cache[:, :d["d_c"]], cache[:, d["d_c"]:]
        for h in range(d["H"]):
            wk = torch.from_numpy(inp.w_uk[h]).double()
            wv = torch.from_numpy(inp.w_uv[h]).double()
            K = torch.cat([c @ wk.T, kr], dim=1)
            V = c @ wv.T
            qn = torch.from_numpy(inp.q_nope[b, :, h]).double()
            qr = torch.from_numpy(np.stack([rope_interleaved(inp.q_rope[b, i, h], inp.positions[b, i], 10000.0)
                                            for i in range(Lq)]))
            Q = torch.cat([qn, qr], dim=1)
            mask = torch.ones(Lq, L, dtype=torch.bool)
            if causal:
                t = torch.arange(L)[None, :]
                i = torch.arange(Lq)[:, None]
                mask = t <= (L - Lq + i)
            o = torch.nn.functional.scaled_dot_product_attention(
                Q[None], K[None], V[None], attn_mask=mask[None], scale=1.0 / math.sqrt(12 + 8))
            np.testing.assert_allclose(ref["o"][b, :, h], o[0].numpy(), rtol=1e-11, atol=1e-13)


# ------------------------------------------------ prefill in MHA form


def test_expand_matches_brute_force():
    """k_nope[t, h, j] = sum_c W_UK[h][j][c] c_t[c] and the same with W_UV,
    element by element with scalar loops."""
    arr = _arrays(11, B=2, lens=(5, 3))
    inp = ArrayInputs(**arr)
    d = DIMS
    for b in range(2):
        k, v = mla_expand(inp, b)
        assert k.shape == (len(inp.caches[b]), d["H"], d["d_n"])
        assert v.shape == (len(inp.caches[b]), d["H"], d["d_v"])
        c = inp.caches[b]
        for t in range(len(c)):
            for h in range(d["H"]):
                for j in range(d["d_n"]):
                    ref = sum(float(inp.w_uk[h, j, cc]) * float(c[t, cc]) for cc in range(d["d_c"]))
                    assert abs(k[t, h, j] - ref) < 1e-12
                for j in range(d["d_v"]):
                    ref = sum(float(inp.w_uv[h, j, cc]) * float(c[t, cc]) for cc in range(d["d_c"]))
                    assert abs(v[t, h, j] - ref) < 1e-12


def test_prefill_is_causal_self_attention():
    """A prompt of q_len = len tokens that are all cached: the oracle's output
    equals torch's float64 causal attention (is_causal, no explicit mask) over
    keys [W_UK c ; k_rope] and values W_UV c built from the expand step."""
    L = 9
    arr = _arrays(12, B=2, Lq=L, lens=(L, L))
    arr["positions"] = np.tile(np.arange(L), (2, 1))
    inp = ArrayInputs(**arr, causal=True)
    ref = mla_decode(inp)
    d = DIMS
    for b in range(2):
        k, v = mla_expand(inp, b)
        kr = inp.caches[b][:, d["d_c"]:].astype(np.float64)
        for h in range(d["H"]):
            K = torch.from_numpy(np.concatenate([k[:, h], kr], axis=1))
            V = torch.from_numpy(v[:, h])
            qr = np.stack([rope_interleaved(inp.q_rope[b, i, h], inp.positions[b, i], 10000.0)
                           for i in range(L)])
            Q = torch.from_numpy(np.concatenate([inp.q_nope[b, :, h].astype(np.float64), qr], axis=1))
            o = torch.nn.functional.scaled_dot_product_attention(
                Q[None], K[None], V[None], is_causal=True, scale=1.0 / math.sqrt(12 + 8))
            np.testing.assert_allclose(ref["o"][b, :, h], o[0].numpy(), rtol=1e-11, atol=1e-13)


# --------------------------------------------------------- special cases

def test_single_token_gives_value_exactly():
    arr = _arrays(8, B=1, lens=(1,))
    inp = ArrayInputs(**arr)
    ref = mla_decode(inp)
    c0 = inp.caches[0][0, :DIMS["d_c"]].astype(np.float64)
    for h in range(DIMS["H"]):
        np.testing.assert_allclose(ref["o"][0, 0, h], inp.w_uv[h].astype(np.float64) @ c0, rtol=1e-15, atol=1e-15)


def test_identical_rows_give_uniform_weights():
    arr = _arrays(9, B=1, lens=(11,))
    row = arr["caches"][0][3].copy()
    arr["caches"] = [np.tile(row, (11, 1))]
    inp = ArrayInputs(**arr)
    ref = mla_decode(inp)
    c = row[:DIMS["d_c"]].astype(np.float64)
    for h in range(DIMS["H"]):
        np.testing.assert_allclose(ref["o"][0, 0, h], inp.w_uv[h].astype(np.float64) @ c, rtol=1e-13, atol=1e-14)
        # lse = s + log(11) where s is the common score
        ab = mla_absorbed(inp)
        s = ab["lse"][0, 0, h] - math.log(11)
        assert np.isfinite(s)


def test_two_tokens_logistic():
    arr = _arrays(10, B=1, lens=(2,), H=1)
    inp = ArrayInputs(**arr)
    ref = mla_decode(inp)
    ab = mla_absorbed(inp)
    # recover the two scores through one-token runs on the same query
    s = []
    for t in range(2):
        one = dict(arr)
        one["caches"] = [arr["caches"][0][t:t + 1]]
        s.append(mla_decode(ArrayInputs(**one))["lse"][0, 0, 0])
    p0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
    c = inp.caches[0][:, :DIMS["d_c"]].astype(np.float64)
    v = c @ inp.w_uv[0].astype(np.float64).T
    np.testing.assert_allclose(ref["o"][0, 0, 0], p0 * v[0] + (1 - p0) * v[1], rtol=1e-13, atol=1e-14)
    assert abs(ab["lse"][0, 0, 0] - (max(s) + math.log(1 + math.exp(min(s) - max(s))))) < 1e-13


def test_zero_query_averages_values():
    arr = _arrays(11, B=1, lens=(13,))
    arr["q_nope"][:] = 0
    arr["q_rope"][:] = 0
    inp = ArrayInputs(**arr)
    ref = mla_decode(inp)
    c = inp.caches[0][:, :DIMS["d_c"]].astype(np.float64)
    for h in range(DIMS["H"]):
        np.testing.assert_allclose(ref["o"][0, 0, h], (c @ inp.w_uv[h].astype(np.float64).T).mean(0),
                                   rtol=1e-13, atol=1e-14)
        assert abs(ref["lse"][0, 0, h] - math.log(13)) < 1e-14


def test_weights_sum_to_one():
    """Make latent column 0 the constant 1 and read it through a selector row
    of W_UV: the output then equals the sum of the attention weights."""
    arr = _arrays(12, B=2, Lq=2, lens=(40, 3))
    for c in arr["caches"]:
        c[:, 0] = 1.0
    arr["w_uv"][:, 0, :] = 0.0
    arr["w_uv"][:, 0, 0] = 1.0
    inp = ArrayInputs(**arr, causal=True)
    ref = mla_decode(inp)
    assert np.all(np.abs(ref["o"][..., 0] - 1.0) < 1e-14)


def test_causal_query_equals_shorter_single_query():
    """Query i of a causal q_len=2 call sees the first len-2+i+1 tokens."""
    arr = _arrays(13, B=2, Lq=2, lens=(20, 2))
    arr["positions"] = np.array([[18, 19], [0, 1]])
    inp = ArrayInputs(**arr, causal=True)
    ref = mla_decode(inp)
    for b in range(2):
        L = len(arr["caches"][b])
        for i in range(2):
            one = dict(q_nope=arr["q_nope"][b:b + 1, i:i + 1], q_rope=arr["q_rope"][b:b + 1, i:i + 1],
                       w_uk=arr["w_uk"], w_uv=arr["w_uv"], caches=[arr["caches"][b][:L - 2 + i + 1]],
                       positions=arr["positions"][b:b + 1, i:i + 1])
            r1 = mla_decode(ArrayInputs(**one))
            np.testing.assert_allclose(ref["o"][b, i], r1["o"][0, 0], rtol=1e-14, atol=1e-15)


def test_query_seeing_nothing_gives_zero_and_neg_inf():
    arr = _arrays(14, B=1, Lq=2, lens=(1,))
    inp = ArrayInputs(**arr, causal=True)
    ref = mla_decode(inp)
    assert np.all(ref["o"][0, 0] == 0) and np.all(ref["lse"][0, 0] == -np.inf)
    assert np.all(np.isfinite(ref["o"][0, 1]))


# ----------------------------------------------------- generated inputs

def test_tiny_config_matches_pages_scale_and_dims():
    inp = MLAInputs(CONFIGS["tiny_f32"])
    assert inp.softmax_scale == pytest.approx(1 / math.sqrt(48), rel=1e-15)
    assert CONFIGS["dsv3_b16_l4k"].softmax_scale == pytest.approx(1 / math.sqrt(192), rel=1e-15)
    ref = mla_decode(inp)
    ab = mla_absorbed(inp)
    assert np.all(np.isfinite(ref["o"]))
    np.testing.assert_allclose(ab["o"], ref["o"], rtol=1e-12, atol=1e-14)


def test_fp8_dequant_uses_token_scale():
    cfg = scaled(CONFIGS["fp8_b128_l16k_q2"], batch=2, seq_len=70, heads=32)
    inp = MLAInputs(cfg)
    from oracle import cache_f64
    for b in range(2):
        src = inp.cache_source(b).astype(np.float64)
        deq = cache_f64(inp, b)
        # E4M3 keeps 3 mantissa bits: relative error <= 2^-4 for normals
        amax = np.abs(src).max(1, keepdims=True)
        assert np.all(np.abs(deq - src) <= 2.0 ** -4 * np.abs(src) + amax / 448 * 2.0 ** -9 + 1e-12)
        assert np.allclose(np.abs(deq).max(1), amax[:, 0], rtol=1e-7)


# ------------------------------------------------------- pages' numbers

def test_cache_bytes_match_pages_tables():
    with open(os.path.join(GOLDEN, "cache_bytes_per_token.json")) as f:
        g = json.load(f)
    for e in g["entries"]:
        kw = {k: e[k] for k in ("n_kv_heads", "d_head", "d_latent", "d_rope") if k in e}
        got = kv_cache_bytes_per_token(e["kind"], elem_bytes=e["elem_bytes"], **kw)
        assert got == e["bytes"], e["cite"]
        assert got / e["elem_bytes"] == e["elements"], e["cite"]
    mla = kv_cache_bytes_per_token("mla", d_latent=512, d_rope=64, elem_bytes=2)
    mha64 = kv_cache_bytes_per_token("mha", n_kv_heads=64, d_head=128, elem_bytes=2)
    mha128 = kv_cache_bytes_per_token("mha", n_kv_heads=128, d_head=128, elem_bytes=2)
    gqa8 = kv_cache_bytes_per_token("gqa", n_kv_heads=8, d_head=128, elem_bytes=2)
    r = {r_.get("num", ""): r_ for r_ in g["ratios"]}
    assert abs(mha64 / mla - r["mha64_bytes"]["value"]) < r["mha64_bytes"]["tol"]
    assert abs(mha128 / mla - r["mha128_bytes"]["value"]) < r["mha128_bytes"]["tol"]
    assert abs(1 - mla / gqa8 - g["ratios"][2]["value"]) < g["ratios"][2]["tol"]
    # the configs' storage per token: 1152 B bf16, 576 + 4 B fp8 + scale, 192 B tiny fp32
    assert CONFIGS["dsv3_b64_l8k_paged"].storage_bytes_per_token() == 1152
    assert CONFIGS["fp8_b128_l16k_q2"].storage_bytes_per_token() == 580
    assert CONFIGS["tiny_f32"].storage_bytes_per_token() == 192


# --------------------------------------------------- cache-append producer


def _append_case(n=3, d=10, dc=6, dr=4, seed=7):
    g = np.random.default_rng(seed)
    return (g.standard_normal((n, d)), g.standard_normal((dc, d)) / math.sqrt(d),
            1.0 + 0.1 * g.standard_normal(dc), g.standard_normal((dr, d)) / math.sqrt(d),
            np.array([0, 5, 130][:n]))


def test_kv_append_brute_force():
    """Scalar loops straight from the definitions: c = W_DKV h, RMSNorm with
    a weight, k = RoPE(W_KR h) with pair k turned by pos * base^(-2k/d_R)."""
    from oracle import kv_append

    h, wd, gam, wr, pos = _append_case()
    eps, base = 1e-6, 10000.0
    ckv, kr = kv_append(h, wd, gam, wr, pos, base, eps)
    n, d = h.shape
    for t in range(n):
        c = [sum(wd[j][i] * h[t][i] for i in range(d)) for j in range(wd.shape[0])]
        ms = sum(x * x for x in c) / len(c)
        for j in range(len(c)):
            assert abs(ckv[t][j] - c[j] / math.sqrt(ms + eps) * gam[j]) <= 1e-12 * (1 + abs(ckv[t][j]))
        r = [sum(wr[j][i] * h[t][i] for i in range(d)) for j in range(wr.shape[0])]
        dr = len(r)
        for k in range(dr // 2):
            a = pos[t] * base ** (-2.0 * k / dr)
            x0, x1 = r[2 * k], r[2 * k + 1]
            assert abs(kr[t][2 * k] - (x0 * math.cos(a) - x1 * math.sin(a))) <= 1e-12
            assert abs(kr[t][2 * k + 1] - (x0 * math.sin(a) + x1 * math.cos(a))) <= 1e-12


def test_kv_append_norm_invariants():
    """With a unit weight and eps = 0 the cached latent has mean square 1 per
    token and does not change when the hidden state is scaled; the key at
    position 0 is the plain projection."""
    from oracle import kv_append

    h, wd, _, wr, _ = _append_case(n=3, d=16, dc=8, dr=6, seed=3)
    ones = np.ones(wd.shape[0])
    ckv, kr = kv_append(h, wd, ones, wr, np.zeros(3), 10000.0, 0.0)
    np.testing.assert_allclose(np.mean(ckv * ckv, axis=-1), 1.0, rtol=1e-13)
    ckv3, kr3 = kv_append(3.0 * h, wd, ones, wr, np.zeros(3), 10000.0, 0.0)
    np.testing.assert_allclose(ckv3, ckv, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(kr, h @ wr.T, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(kr3, 3.0 * kr, rtol=1e-13, atol=1e-15)


# ------------------------------------------------- output-side absorption


def test_fused_output_weight_equals_unfused_projection():
    """u[m] = sum_i W~_O,i o_lat[m, i] with the pre-fused weight equals the
    unfused definition, per-head values v_i = W_UV,i o_lat[m, i] and then W_O
    over their concatenation, written out with scalar loops."""
    rng = np.random.default_rng(41)
    H, d_v, d_c, d, M = 3, 4, 5, 7, 2
    w_o = rng.standard_normal((d, H * d_v))
    w_uv = rng.standard_normal((H, d_v, d_c))
    o_lat = rng.standard_normal((M, H, d_c))
    got = out_proj_fused(o_lat, fuse_out_weight(w_o, w_uv, H))
    assert got.shape == (M, d)
    for m in range(M):
        concat = []
        for i in range(H):
            for j in range(d_v):
                concat.append(sum(w_uv[i, j, c] * o_lat[m, i, c] for c in range(d_c)))
        for n in range(d):
            ref = sum(w_o[n, k] * concat[k] for k in range(H * d_v))
            assert abs(got[m, n] - ref) < 1e-12


def test_fused_output_weight_with_identity_w_o():
    """With W_O the identity (d = H d_v) the fused weight of head i is W_UV,i
    placed in rows i d_v .. (i+1) d_v, and the fused projection returns the
    concatenated per-head values."""
    rng = np.random.default_rng(42)
    H, d_v, d_c = 4, 3, 6
    w_uv = rng.standard_normal((H, d_v, d_c))
    wf = fuse_out_weight(np.eye(H * d_v), w_uv, H)
    for i in range(H):
        np.testing.assert_array_equal(wf[i * d_v:(i + 1) * d_v, i, :], w_uv[i])
        others = [k for k in range(H * d_v) if not (i * d_v <= k < (i + 1) * d_v)]
        assert np.all(wf[others, i, :] == 0.0)
    o_lat = rng.standard_normal((5, H, d_c))
    got = out_proj_fused(o_lat, wf)
    ref = np.concatenate([o_lat[:, i, :] @ w_uv[i].T for i in range(H)], axis=1)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_fused_output_projection_of_the_attention_output():
    """Applied to the absorbed latent output of the attention, the fused path
    gives W_O times the concatenated non-absorbed head outputs (the oracle's
    decode output, pinned separately)."""
    arr = _arrays(43, B=2, Lq=2, lens=(6, 4))
    inp = ArrayInputs(**arr, causal=True)
    d = DIMS
    o = mla_decode(inp)["o"]             # [B, Lq, H, d_v]
    o_lat = mla_absorbed(inp)["o_lat"]   # [B, Lq, H, d_c]
    rng = np.random.default_rng(44)
    d_model = 9
    w_o = rng.standard_normal((d_model, d["H"] * d["d_v"]))
    wf = fuse_out_weight(w_o, inp.w_uv, d["H"])
    got = out_proj_fused(o_lat.reshape(-1, d["H"], d["d_c"]), wf)
    ref = o.reshape(-1, d["H"] * d["d_v"]) @ w_o.T
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-10)
