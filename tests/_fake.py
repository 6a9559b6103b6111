"""Hand-built inputs exposing the attributes the oracle reads.

Used for special cases (one token, identical rows, two tokens, zero query)
whose answers follow from the mathematics alone.  Values are float32 so the
oracle's float64 arithmetic sees them exactly.
"""

import numpy as np

from mla_inputs import MLAConfig


class ArrayInputs:
    def __init__(self, *, q_nope, q_rope, w_uk, w_uv, caches, positions,
                 causal=False, rope_base=10000.0):
        q_nope = np.asarray(q_nope, np.float32)
        B, Lq, H, d_n = q_nope.shape
        d_R = np.asarray(q_rope).shape[-1]
        d_v, d_c = np.asarray(w_uv).shape[1:]
        self.cfg = MLAConfig(name="array", batch=B, q_len=Lq, heads=H, d_nope=d_n,
                             d_rope=d_R, d_latent=d_c, d_v=d_v,
                             seq_len=max(1, max(len(c) for c in caches)),
                             q_dtype="f32", kv_dtype="f32", causal=causal,
                             rope_base=rope_base)
        self.q_nope = q_nope
        self.q_rope = np.asarray(q_rope, np.float32)
        self.w_uk = np.asarray(w_uk, np.float32)
        self.w_uv = np.asarray(w_uv, np.float32)
        self.caches = [np.asarray(c, np.float32).reshape(-1, d_c + d_R) for c in caches]
        self.seq_lens = np.array([len(c) for c in self.caches], np.int32)
        self.positions = np.asarray(positions, np.int32).reshape(B, Lq)
        self.softmax_scale = float((d_n + d_R) ** -0.5)
        self.rope_base = rope_base

    def cache_stored(self, b):
        return self.caches[b], None


def random_arrays(rng, B, Lq, H, d_n, d_R, d_c, d_v, lens, w_std=None):
    w_std = w_std if w_std else d_c ** -0.5
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return dict(
        q_nope=f(B, Lq, H, d_n), q_rope=f(B, Lq, H, d_R),
        w_uk=(f(H, d_n, d_c) * w_std).astype(np.float32),
        w_uv=(f(H, d_v, d_c) * w_std).astype(np.float32),
        caches=[f(n, d_c + d_R) for n in lens],
        positions=np.array([[n + i for i in range(Lq)] for n in lens]),
    )
