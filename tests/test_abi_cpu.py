"""C ABI checks that need no GPU: the library loads, every declared entry
point is exported, host validation rejects bad arguments before any HIP
call, and the split-K division is a partition with distinct slots."""

import ctypes
import os
import re

import numpy as np
import pytest

import mla_latent_kv_lat_amd as mla
from mla_latent_kv_lat_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "mla.h")).read()
    return sorted(set(re.findall(r"^(?:int|const char\*)\s+(mla_\w+)\(", txt, re.M)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert {"mla_absorb_q", "mla_decode_attn", "mla_combine", "mla_out_proj"} <= set(names)
    lib = binding.library()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = binding.library()
    for code in range(6):
        assert lib.mla_status_string(code).decode().startswith("MLA_")


DSV3 = dict(batch=2, q_len=1, heads=128, d_nope=128, d_rope=64, d_latent=512, d_v=128,
            q_dtype=mla.BF16, kv_dtype=mla.BF16)


def _d(**kw):
    a = dict(DSV3)
    a.update(kw)
    return mla.dims(**a)


def _decode(d, **kw):
    a = dict(q_abs=16, latent_cache=16, rope_cache=16 + 1024, kv_row_stride=576, kv_scale=None,
             seq_lens=16, block_table=None, max_blocks_per_seq=0, block_size=64, max_seq_len=64,
             causal=0, softmax_scale=0.07, num_splits=4, o_part=16, lse_part=16)
    a.update(kw)
    return binding._lib.mla_decode_attn(ctypes.byref(d), a["q_abs"], a["latent_cache"],
                                        a["rope_cache"], a["kv_row_stride"], a["kv_scale"],
                                        a["seq_lens"], a["block_table"], a["max_blocks_per_seq"],
                                        a["block_size"], a["max_seq_len"], a["causal"],
                                        a["softmax_scale"], a["num_splits"], a["o_part"],
                                        a["lse_part"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q_len=0), 1), (dict(heads=0), 1), (dict(d_rope=63), 1), (dict(d_latent=500), 1),
    (dict(q_dtype=7), 1), (dict(kv_dtype=9), 1), (dict(flags=8), 1),
    (dict(q_dtype=mla.F32), 2), (dict(kv_dtype=mla.F32), 2),
])
def test_bad_dims_rejected(kw, status):
    assert _decode(_d(**kw)) == status


@pytest.mark.parametrize("kw,status", [
    (dict(q_abs=None), 1), (dict(seq_lens=None), 1), (dict(o_part=None), 3),
    (dict(lse_part=None), 3), (dict(q_abs=8), 1), (dict(kv_row_stride=100), 1),
    (dict(num_splits=0), 1), (dict(num_splits=70000), 1), (dict(causal=2), 1),
    (dict(softmax_scale=0.0), 1), (dict(softmax_scale=float("nan")), 1),
    (dict(max_seq_len=0), 1), (dict(kv_scale=16), 1),
    (dict(block_table=16, block_size=32, max_blocks_per_seq=1), 1),
    (dict(block_table=16, block_size=64, max_blocks_per_seq=1, max_seq_len=65), 1),
])
def test_bad_decode_args_rejected(kw, status):
    assert _decode(_d(), **kw) == status


def test_fp8_needs_scale():
    assert _decode(_d(kv_dtype=mla.FP8_E4M3)) == 1


def test_empty_batch_is_a_noop():
    assert _decode(_d(batch=0)) == 0
    d = _d(batch=0)
    assert binding._lib.mla_combine(ctypes.byref(d), 4, 16, 16, 16, 16, None, None) == 0
    assert binding._lib.mla_out_proj(ctypes.byref(d), 16, 16, 16, None) == 0
    assert binding._lib.mla_absorb_q(ctypes.byref(d), 16, 16, 16, 10000.0, 16, 16, None) == 0


def test_other_entry_points_validate():
    d = _d()
    lib = binding._lib
    assert lib.mla_absorb_q(ctypes.byref(d), None, 16, 16, 10000.0, 16, 16, None) == 1
    assert lib.mla_absorb_q(ctypes.byref(d), 16, 16, 16, -1.0, 16, 16, None) == 1
    assert lib.mla_combine(ctypes.byref(d), 4, 16, None, 16, 16, None, None) == 3
    assert lib.mla_combine(ctypes.byref(d), 0, 16, 16, 16, 16, None, None) == 1
    assert lib.mla_out_proj(ctypes.byref(d), 16, None, 16, None) == 1
    with pytest.raises(mla.MLAError):
        mla.mla_out_proj(d, 16, None, 16, stream=0)


def test_workspace_elems():
    d = _d(batch=64, q_len=2)
    o, l = mla.mla_workspace_elems(d, 128)
    assert l == (128 + 64 - 1) * 256 and o == l * 512


@pytest.mark.parametrize("q_dtype,o_bytes", [(mla.BF16, 2), (mla.F32, 4)])
def test_workspace_bytes(q_dtype, o_bytes):
    # fp16 partials except on the fp32 path; LSEs always fp32
    d = _d(batch=5, q_len=1, q_dtype=q_dtype, kv_dtype=q_dtype)
    o, l = mla.mla_workspace_elems(d, 7)
    ob, lb = mla.mla_workspace_bytes(d, 7)
    assert ob == o * o_bytes and lb == l * 4


@pytest.mark.parametrize("seed", range(20))
def test_split_plan_is_a_partition(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    lens = rng.integers(0, 2000, size=B) * (rng.random(B) > 0.2)
    G = int(rng.integers(1, 300))
    fu, lu, ft = mla.mla_split_plan(lens, G)
    tiles = -(-lens // 64)
    T = int(tiles.sum())
    begin = [u * T // G for u in range(G + 1)]
    assert np.array_equal(ft, np.concatenate([[0], np.cumsum(tiles)[:-1]]))
    slots = set()
    for b in range(B):
        if tiles[b] == 0:
            assert fu[b] == -1 and lu[b] == -1
            continue
        lo, hi = ft[b], ft[b] + tiles[b]
        touching = [u for u in range(G) if begin[u] < begin[u + 1] and begin[u] < hi and begin[u + 1] > lo]
        assert touching[0] == fu[b] and touching[-1] == lu[b]
        covered = sum(min(hi, begin[u + 1]) - max(lo, begin[u]) for u in touching)
        assert covered == tiles[b]
        for u in touching:
            assert u + b not in slots
            slots.add(u + b)
    assert all(s < G + B - 1 for s in slots)


def test_kv_append_validation():
    """The cache-append producer's host checks (no kernel is launched)."""
    lib = binding._lib
    d = mla.append_dims(4, 7168)
    ws = ctypes.c_int64()
    assert lib.mla_kv_append_workspace_bytes(ctypes.byref(d), ctypes.byref(ws)) == 0
    assert ws.value == 14 * 4 * 576 * 4
    ok = dict(h=16, w_dkv=16, kv_norm_w=16, w_kr=16, positions=16, rope_base=10000.0, eps=1e-6,
              cache_rows=16, latent_cache=16, rope_cache=16, kv_row_stride=576, kv_scale=None,
              workspace=16)

    def call(dd, **kw):
        a = dict(ok, **kw)
        return lib.mla_kv_append(ctypes.byref(dd), a["h"], a["w_dkv"], a["kv_norm_w"], a["w_kr"],
                                 a["positions"], a["rope_base"], a["eps"], a["cache_rows"],
                                 a["latent_cache"], a["rope_cache"], a["kv_row_stride"],
                                 a["kv_scale"], a["workspace"], None)

    assert call(mla.append_dims(4, 7000)) == 2          # hidden width not a multiple of 512
    assert call(mla.append_dims(4, 16896)) == 2         # wider than 16384
    assert call(mla.append_dims(4, 7168, d_latent=256)) == 2
    assert call(mla.append_dims(4, 7168, kv_dtype=mla.FP8_E4M3)) == 1  # fp8 needs kv_scale
    assert call(mla.append_dims(4, 7168, kv_dtype=mla.F32)) == 2
    assert call(mla.append_dims(0, 7168)) == 0           # nothing to append
    assert call(d, h=None) == 1
    assert call(d, cache_rows=None) == 1
    assert call(d, workspace=None) == 3
    assert call(d, h=8) == 1                              # misaligned
    assert call(d, kv_row_stride=100) == 1
    assert call(d, rope_base=-1.0) == 1
    assert call(d, eps=float("nan")) == 1
    assert call(d, kv_scale=16) == 1
    assert lib.mla_kv_append_workspace_bytes(None, ctypes.byref(ws)) == 1


def test_kv_append_noalloc_validation():
    """The static-scratch variant: the same host checks, and requests beyond
    its fixed buffer rejected before anything touches the GPU."""
    lib = binding._lib
    ok = dict(h=16, w_dkv=16, kv_norm_w=16, w_kr=16, positions=16, rope_base=10000.0, eps=1e-6,
              cache_rows=16, latent_cache=16, rope_cache=16, kv_row_stride=576, kv_scale=None)

    def call(dd, **kw):
        a = dict(ok, **kw)
        return lib.mla_kv_append_noalloc(ctypes.byref(dd), a["h"], a["w_dkv"], a["kv_norm_w"],
                                         a["w_kr"], a["positions"], a["rope_base"], a["eps"],
                                         a["cache_rows"], a["latent_cache"], a["rope_cache"],
                                         a["kv_row_stride"], a["kv_scale"], None)

    limit = binding.KV_APPEND_NOALLOC_SCRATCH_BYTES
    # the largest batch that fits at width 7168: 14 chunks x n x 576 fp32
    n_max = limit // (14 * 576 * 4)
    assert n_max == 260
    assert call(mla.append_dims(n_max + 1, 7168)) == 5    # MLA_ERR_TOO_LARGE
    assert call(mla.append_dims(4096, 16384)) == 5
    assert call(mla.append_dims(4, 7000)) == 2
    assert call(mla.append_dims(0, 7168)) == 0
    d = mla.append_dims(4, 7168)
    assert call(d, h=None) == 1
    assert call(d, h=8) == 1
    assert call(d, kv_row_stride=100) == 1
    assert call(mla.append_dims(4, 7168, kv_dtype=mla.FP8_E4M3)) == 1
    assert "MLA_ERR_TOO_LARGE" in lib.mla_status_string(5).decode()


def test_prefill_validation():
    """The MHA-form prefill calls: host checks before anything is enqueued,
    and shapes or types they are not built for rejected as unsupported."""
    lib = binding._lib
    ok = dict(q_nope=16, q_rope=16, positions=16, rope_base=10000.0, k_nope=16, v=16,
              rope_cache=16, latent_cache=16, kv_row_stride=576, seq_lens=16, block_table=None,
              max_blocks_per_seq=0, block_size=64, max_seq_len=256, causal=1,
              softmax_scale=0.07, o=16, lse=None, w_uk=16, w_uv=16)

    def attn(dd, **kw):
        a = dict(ok, **kw)
        return lib.mla_prefill_attn(ctypes.byref(dd), a["q_nope"], a["q_rope"], a["positions"],
                                    a["rope_base"], a["k_nope"], a["v"], a["rope_cache"],
                                    a["kv_row_stride"], a["seq_lens"], a["block_table"],
                                    a["max_blocks_per_seq"], a["block_size"], a["max_seq_len"],
                                    a["causal"], a["softmax_scale"], a["o"], a["lse"], None)

    def expand(dd, **kw):
        a = dict(ok, **kw)
        return lib.mla_prefill_expand(ctypes.byref(dd), a["latent_cache"], a["kv_row_stride"],
                                      a["seq_lens"], a["block_table"], a["max_blocks_per_seq"],
                                      a["block_size"], a["max_seq_len"], a["w_uk"], a["w_uv"],
                                      a["k_nope"], a["v"], None)

    d = _d(q_len=256)
    for call in (attn, expand):
        assert call(_d(batch=0)) == 0                            # nothing to do
        assert call(d, seq_lens=None) == 1
        assert call(d, kv_row_stride=100) == 1
        assert call(d, max_seq_len=0) == 1
        assert call(d, block_table=16, block_size=32, max_blocks_per_seq=4) == 1
        assert call(d, block_table=16, block_size=64, max_blocks_per_seq=3) == 1  # 3 x 64 < 256
        assert call(d, k_nope=8) == 1                            # misaligned
        assert call(_d(q_len=256, kv_dtype=mla.FP8_E4M3)) == 2
        assert call(_d(q_len=256, d_nope=64)) == 2
        assert call(_d(q_len=256, d_latent=256)) == 2
        assert call(d, max_seq_len=262145) == 2
        assert call(d, kv_row_stride=580) == 2                   # rows not 16-byte aligned
    assert attn(d, q_rope=None) == 1
    assert attn(d, o=None) == 1
    assert attn(d, causal=2) == 1
    assert attn(d, softmax_scale=0.0) == 1
    assert attn(d, rope_base=float("inf")) == 1
    assert expand(d, w_uv=None) == 1
    assert attn(_d(q_len=256, q_dtype=mla.F32, kv_dtype=mla.F32)) == 2


def test_out_fused_validation():
    """Output-side absorption calls: host checks before anything is enqueued
    (every pointer here is a fake, so any launch would fault)."""
    lib = binding.library()
    d = _d(batch=64)

    def fuse(dd, d_model=7168, w_o=16, w_uv=16, w_fused=16):
        return lib.mla_fuse_out_weight(ctypes.byref(dd), d_model, w_o, w_uv, w_fused, None)

    def proj(dd, d_model=7168, o_lat=16, w_fused=16, workspace=16, out=16):
        return lib.mla_out_proj_fused(ctypes.byref(dd), d_model, o_lat, w_fused, workspace, out, None)

    assert fuse(d, w_o=None) == 1
    assert fuse(d, w_fused=8) == 1                               # misaligned
    assert fuse(d, d_model=0) == 1
    assert fuse(_d(d_latent=256)) == 2
    assert fuse(_d(d_v=256)) == 2
    assert fuse(_d(q_dtype=mla.F32, kv_dtype=mla.F32)) == 2
    assert fuse(d, d_model=65537) == 2
    assert proj(_d(batch=0)) == 0                                # nothing to do
    assert proj(d, workspace=None) == 3
    assert proj(d, out=None) == 1
    assert proj(d, o_lat=24) == 1
    assert proj(_d(d_latent=256)) == 2
    assert proj(_d(batch=1 << 20)) == 2                          # rows x d_model past 2^31
    n = ctypes.c_int64()
    assert lib.mla_out_proj_fused_workspace_bytes(ctypes.byref(d), 7168, ctypes.byref(n)) == 0
    assert n.value == 8 * 64 * 7168 * 4 + 64 * 128 * 512 * 2
    assert mla.mla_out_proj_fused_workspace_bytes(_d(batch=3, q_len=2), 100) == \
        8 * 6 * 100 * 4 + 32 * 128 * 512 * 2
    assert mla.mla_fused_out_weight_bytes(_d(batch=3), 100) == 128 * 128 * 512 * 2  # rows to 128
    assert mla.mla_fused_out_weight_bytes(_d(batch=3, heads=2), 7168) == 7168 * 2 * 512 * 2
