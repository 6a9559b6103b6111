"""ctypes binding of libmla.so: argument marshalling only.

Every function here has the name and argument order of the C entry point
in include/mla.h.  Tensor arguments are torch tensors on the GPU (or None
for NULL); their data pointers and the current HIP stream are passed to the
library, which does all of the work in its kernels.  A non-zero status
raises MLAError.  If the library has not been built, importing this module
raises ImportError: there is no other implementation to fall back to.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

# torch first: it loads its own HIP runtime (same soname as ROCm's), and the
# library must bind to that one instance rather than bring in a second.
import torch  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
FLAG_GENERIC = 1
TILE_TOKENS = 64

KV_APPEND_NOALLOC_SCRATCH_BYTES = 8 << 20  # MLA_KV_APPEND_NOALLOC_SCRATCH_BYTES

STATUS = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_UNSUPPORTED",
          3: "MLA_ERR_WORKSPACE", 4: "MLA_ERR_HIP", 5: "MLA_ERR_TOO_LARGE"}


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.mla_status_string(status).decode()}")


class MLADims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "q_len", "heads", "d_nope", "d_rope", "d_latent", "d_v",
        "q_dtype", "kv_dtype", "flags")]


class MLAAppendDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_tokens", "d_model", "d_latent", "d_rope", "kv_dtype")]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with "
                          "`python mla_latent_kv_lat_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F, VP = (ctypes.POINTER(MLADims), ctypes.c_int32, ctypes.c_int64,
                          ctypes.c_float, ctypes.c_void_p)
    sig = {
        "mla_absorb_q": [P, VP, VP, VP, F, VP, VP, VP],
        "mla_decode_attn": [P, VP, VP, VP, I64, VP, VP, VP, I32, I32, I32, I32, F, I32, VP, VP, VP],
        "mla_combine": [P, I32, VP, VP, VP, VP, VP, VP],
        "mla_out_proj": [P, VP, VP, VP, VP],
        "mla_combine_out_proj": [P, I32, VP, VP, VP, VP, VP, VP, VP, VP],
        "mla_workspace_elems": [P, I32, ctypes.POINTER(I64), ctypes.POINTER(I64)],
        "mla_workspace_bytes": [P, I32, ctypes.POINTER(I64), ctypes.POINTER(I64)],
        "mla_num_splits_hint": [P, I32, ctypes.POINTER(I32)],
        "mla_split_plan": [I32, VP, I32, VP, VP, VP],
        "mla_kv_append_workspace_bytes": [ctypes.POINTER(MLAAppendDims), ctypes.POINTER(I64)],
        "mla_kv_append": [ctypes.POINTER(MLAAppendDims), VP, VP, VP, VP, VP, F, F, VP, VP, VP,
                          I64, VP, VP, VP],
        "mla_kv_append_noalloc": [ctypes.POINTER(MLAAppendDims), VP, VP, VP, VP, VP, F, F, VP, VP,
                                  VP, I64, VP, VP],
        "mla_prefill_expand": [P, VP, I64, VP, VP, I32, I32, I32, VP, VP, VP, VP, VP],
        "mla_prefill_attn": [P, VP, VP, VP, F, VP, VP, VP, I64, VP, VP, I32, I32, I32, I32, F, VP,
                             VP, VP],
        "mla_fuse_out_weight": [P, I32, VP, VP, VP, VP],
        "mla_out_proj_fused_workspace_bytes": [P, I32, ctypes.POINTER(I64)],
        "mla_fused_out_weight_bytes": [P, I32, ctypes.POINTER(I64)],
        "mla_out_proj_fused": [P, I32, VP, VP, VP, VP, VP],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    return lib


_lib = _load()


def library():
    """The loaded ctypes library (for symbol checks)."""
    return _lib


def dims(batch, q_len, heads, d_nope, d_rope, d_latent, d_v, q_dtype, kv_dtype, flags=0) -> MLADims:
    return MLADims(batch, q_len, heads, d_nope, d_rope, d_latent, d_v, q_dtype, kv_dtype, flags)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor arguments must live on the GPU")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(st: int, where: str):
    if st != 0:
        raise MLAError(st, where)


def mla_absorb_q(d: MLADims, q_nope, q_rope, positions, rope_base, w_uk, q_abs, stream=None):
    _check(_lib.mla_absorb_q(ctypes.byref(d), _ptr(q_nope), _ptr(q_rope), _ptr(positions),
                             float(rope_base), _ptr(w_uk), _ptr(q_abs), _stream(stream)),
           "mla_absorb_q")


def mla_decode_attn(d: MLADims, q_abs, latent_cache, rope_cache, kv_row_stride, kv_scale,
                    seq_lens, block_table, max_blocks_per_seq, block_size, max_seq_len,
                    causal, softmax_scale, num_splits, o_part, lse_part, stream=None):
    _check(_lib.mla_decode_attn(ctypes.byref(d), _ptr(q_abs), _ptr(latent_cache),
                                _ptr(rope_cache), int(kv_row_stride), _ptr(kv_scale),
                                _ptr(seq_lens), _ptr(block_table), int(max_blocks_per_seq),
                                int(block_size), int(max_seq_len), int(causal),
                                float(softmax_scale), int(num_splits), _ptr(o_part),
                                _ptr(lse_part), _stream(stream)),
           "mla_decode_attn")


def mla_combine(d: MLADims, num_splits, seq_lens, o_part, lse_part, o_lat, lse_out=None,
                stream=None):
    _check(_lib.mla_combine(ctypes.byref(d), int(num_splits), _ptr(seq_lens), _ptr(o_part),
                            _ptr(lse_part), _ptr(o_lat), _ptr(lse_out), _stream(stream)),
           "mla_combine")


def mla_out_proj(d: MLADims, o_lat, w_uv, o, stream=None):
    _check(_lib.mla_out_proj(ctypes.byref(d), _ptr(o_lat), _ptr(w_uv), _ptr(o), _stream(stream)),
           "mla_out_proj")


def mla_combine_out_proj(d: MLADims, num_splits, seq_lens, o_part, lse_part, w_uv, o,
                         lse_out=None, o_lat=None, stream=None):
    _check(_lib.mla_combine_out_proj(ctypes.byref(d), int(num_splits), _ptr(seq_lens),
                                     _ptr(o_part), _ptr(lse_part), _ptr(w_uv), _ptr(o),
                                     _ptr(lse_out), _ptr(o_lat), _stream(stream)),
           "mla_combine_out_proj")


def mla_workspace_elems(d: MLADims, num_splits: int):
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.mla_workspace_elems(ctypes.byref(d), int(num_splits), ctypes.byref(a),
                                    ctypes.byref(b)), "mla_workspace_elems")
    return a.value, b.value


def mla_workspace_bytes(d: MLADims, num_splits: int):
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.mla_workspace_bytes(ctypes.byref(d), int(num_splits), ctypes.byref(a),
                                    ctypes.byref(b)), "mla_workspace_bytes")
    return a.value, b.value


def mla_num_splits_hint(d: MLADims, device: int = 0) -> int:
    out = ctypes.c_int32()
    _check(_lib.mla_num_splits_hint(ctypes.byref(d), int(device), ctypes.byref(out)),
           "mla_num_splits_hint")
    return out.value


def mla_split_plan(seq_lens, num_splits: int):
    """Host-only: (first_unit[B], last_unit[B], first_tile[B]) as numpy arrays."""
    import numpy as np
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    B = lens.shape[0]
    fu = np.zeros(B, np.int32)
    lu = np.zeros(B, np.int32)
    ft = np.zeros(B, np.int64)
    _check(_lib.mla_split_plan(B, lens.ctypes.data if B else None, int(num_splits),
                               fu.ctypes.data if B else None, lu.ctypes.data if B else None,
                               ft.ctypes.data if B else None), "mla_split_plan")
    return fu, lu, ft


def append_dims(n_tokens, d_model, d_latent=512, d_rope=64, kv_dtype=BF16) -> MLAAppendDims:
    return MLAAppendDims(n_tokens, d_model, d_latent, d_rope, kv_dtype)


def mla_kv_append_workspace_bytes(d: MLAAppendDims) -> int:
    out = ctypes.c_int64()
    _check(_lib.mla_kv_append_workspace_bytes(ctypes.byref(d), ctypes.byref(out)),
           "mla_kv_append_workspace_bytes")
    return out.value


def mla_kv_append(d: MLAAppendDims, h, w_dkv, kv_norm_w, w_kr, positions, rope_base, eps,
                  cache_rows, latent_cache, rope_cache, kv_row_stride, kv_scale, workspace,
                  stream=None):
    _check(_lib.mla_kv_append(ctypes.byref(d), _ptr(h), _ptr(w_dkv), _ptr(kv_norm_w), _ptr(w_kr),
                              _ptr(positions), float(rope_base), float(eps), _ptr(cache_rows),
                              _ptr(latent_cache), _ptr(rope_cache), int(kv_row_stride),
                              _ptr(kv_scale), _ptr(workspace), _stream(stream)),
           "mla_kv_append")


def mla_kv_append_noalloc(d: MLAAppendDims, h, w_dkv, kv_norm_w, w_kr, positions, rope_base, eps,
                          cache_rows, latent_cache, rope_cache, kv_row_stride, kv_scale,
                          stream=None):
    _check(_lib.mla_kv_append_noalloc(ctypes.byref(d), _ptr(h), _ptr(w_dkv), _ptr(kv_norm_w),
                                      _ptr(w_kr), _ptr(positions), float(rope_base), float(eps),
                                      _ptr(cache_rows), _ptr(latent_cache), _ptr(rope_cache),
                                      int(kv_row_stride), _ptr(kv_scale), _stream(stream)),
           "mla_kv_append_noalloc")


def mla_prefill_expand(d: MLADims, latent_cache, kv_row_stride, seq_lens, block_table,
                       max_blocks_per_seq, block_size, max_seq_len, w_uk, w_uv, k_nope, v,
                       stream=None):
    _check(_lib.mla_prefill_expand(ctypes.byref(d), _ptr(latent_cache), int(kv_row_stride),
                                   _ptr(seq_lens), _ptr(block_table), int(max_blocks_per_seq),
                                   int(block_size), int(max_seq_len), _ptr(w_uk), _ptr(w_uv),
                                   _ptr(k_nope), _ptr(v), _stream(stream)),
           "mla_prefill_expand")


def mla_prefill_attn(d: MLADims, q_nope, q_rope, positions, rope_base, k_nope, v, rope_cache,
                     kv_row_stride, seq_lens, block_table, max_blocks_per_seq, block_size,
                     max_seq_len, causal, softmax_scale, o, lse=None, stream=None):
    _check(_lib.mla_prefill_attn(ctypes.byref(d), _ptr(q_nope), _ptr(q_rope), _ptr(positions),
                                 float(rope_base), _ptr(k_nope), _ptr(v), _ptr(rope_cache),
                                 int(kv_row_stride), _ptr(seq_lens), _ptr(block_table),
                                 int(max_blocks_per_seq), int(block_size), int(max_seq_len),
                                 int(causal), float(softmax_scale), _ptr(o), _ptr(lse),
                                 _stream(stream)),
           "mla_prefill_attn")


def mla_fuse_out_weight(d: MLADims, d_model, w_o, w_uv, w_fused, stream=None):
    _check(_lib.mla_fuse_out_weight(ctypes.byref(d), int(d_model), _ptr(w_o), _ptr(w_uv),
                                    _ptr(w_fused), _stream(stream)),
           "mla_fuse_out_weight")


def mla_fused_out_weight_bytes(d: MLADims, d_model) -> int:
    out = ctypes.c_int64()
    _check(_lib.mla_fused_out_weight_bytes(ctypes.byref(d), int(d_model), ctypes.byref(out)),
           "mla_fused_out_weight_bytes")
    return out.value


def mla_out_proj_fused_workspace_bytes(d: MLADims, d_model) -> int:
    out = ctypes.c_int64()
    _check(_lib.mla_out_proj_fused_workspace_bytes(ctypes.byref(d), int(d_model), ctypes.byref(out)),
           "mla_out_proj_fused_workspace_bytes")
    return out.value


def mla_out_proj_fused(d: MLADims, d_model, o_lat, w_fused, workspace, out, stream=None):
    _check(_lib.mla_out_proj_fused(ctypes.byref(d), int(d_model), _ptr(o_lat), _ptr(w_fused),
                                   _ptr(workspace), _ptr(out), _stream(stream)),
           "mla_out_proj_fused")
