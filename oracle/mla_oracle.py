"""Plain float64 CPU oracle for MLA decode -- test infrastructure.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module.  It shares no code with the HIP path.

It follows the *non-absorbed* definition: per head it materialises the
content keys K = W_UK c and values V = W_UV c of every cached token, appends
the shared post-RoPE key, and runs textbook two-pass softmax attention.
A separate routine (``mla_absorbed``) computes the absorbed intermediates
(q_lat, o_lat) for per-stage checks.

Pages cited (by title, section):
  [ARCH]  "Model Architecture Driving Inference Systems: From MHA/GQA to
          DeepSeek MLA Matrix Absorption and Memory Minimalism"
  [MATH]  "Multi-Head Latent Attention (MLA): Mathematical Foundations,
          Low-Rank KV Compression, Decoupled Rotary Positional Embeddings,
          and Inference Matrix Absorption"
  [RADAR] "Tech Radar: DeepSeek-V3 Multi-Head Latent Attention (MLA)
          Architecture & KV Cache Compression"

Readings where the pages leave a step open:
  * RoPE pairs are interleaved (x[2k], x[2k+1]) and rotate by
    pos * base**(-2k/d_R), the RoFormer schedule [MATH] cites.
  * The cached keys are stored post-RoPE and used as given.
  * With q_len > 1 and ``causal``, query i sees cached tokens
    t <= len - q_len + i (bottom-right aligned).
  * A row that sees no token gets o = 0 and lse = -inf.
  * fp8 rows are OCP E4M3 codes times one fp32 scale per token.
  * Prefill in MHA form (``mla_expand`` then ``mla_decode``): the prompt's
    q_len tokens are the last q_len of the sequence's cached tokens and see
    them causally, as any multi-token query does.
  * The cache-append producer (``kv_append``): RMSNorm with eps as given by
    the caller (the module on [MATH] uses the framework default); the new
    token's key is rotated at its own position.
  * Output-side absorption (``fuse_out_weight``, ``out_proj_fused``): W_O is
    d x (H d_v) with head i's block in columns i d_v .. (i+1) d_v; the fused
    weight is kept as [d, H, d_c].
"""

from __future__ import annotations

import math
from typing import Iterable, Optional

import numpy as np

# --------------------------------------------------------------- codecs


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly: a bf16 value is the
    float32 whose upper 16 bits are the pattern and lower 16 bits zero."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 ("fn": no infinities) codes -> float64 from the format's
    definition: sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent field 0 is subnormal (m/8 * 2**-6); S.1111.111 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = np.where(e == 0, sub, normal) * sign
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, val)


def stored_to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f64(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "fp8":
        return e4m3_to_f64(arr)
    raise ValueError(dtype)


# ----------------------------------------------------------------- RoPE


def rope_interleaved(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotary embedding of the decoupled query part.

    [ARCH] 2.2-2.3: the positional part is rotated by a position-dependent
    block-diagonal matrix of 2x2 rotations.  [MATH] reference module
    (apply_rope): consecutive pairs are read as complex numbers and multiplied
    by a unit complex number per pair, i.e. (x0, x1) -> (x0 cos a - x1 sin a,
    x0 sin a + x1 cos a).  The angle of pair k at position p is
    p * base**(-2k/d) (RoFormer, the source [MATH] cites for RoPE).

    x: [..., d] float64, pos: broadcastable to x.shape[:-1].
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    k = np.arange(d // 2, dtype=np.float64)
    theta = base ** (-2.0 * k / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


# ---------------------------------------------------------------- inputs


def cache_f64(inp, b: int) -> np.ndarray:
    """Cached rows of sequence b as float64 [len_b, d_latent + d_rope]:
    latent c_kv then the post-RoPE key ([ARCH] 2.4: the cache of one token is
    the 512-wide latent plus the 64-wide decoupled key).  fp8 rows are
    decoded and multiplied by their token's scale."""
    rows, scale = inp.cache_stored(b)
    x = stored_to_f64(rows, inp.cfg.kv_dtype)
    if scale is not None:
        x = x * np.asarray(scale, dtype=np.float64)[:, None]
    return x


def _visible(cfg, length: int, i: int) -> int:
    """Number of leading cached tokens query i may attend to."""
    if cfg.causal:
        return max(0, length - cfg.q_len + i + 1)
    return length


def _rows_by_seq(cfg, rows: Optional[Iterable]):
    B, Lq, H = cfg.batch, cfg.q_len, cfg.heads
    if rows is None:
        rows = [(b, i, h) for b in range(B) for i in range(Lq) for h in range(H)]
    by = {}
    for b, i, h in rows:
        by.setdefault(int(b), {}).setdefault(int(h), []).append(int(i))
    return by


# ------------------------------------------------------- the definition


def mla_decode(inp, rows: Optional[Iterable] = None):
    """Decode attention output o[b, i, h, :d_v] and lse[b, i, h] by the
    non-absorbed definition.

    Steps, for each sequence b, head h, query i:
      1. q = [q_nope ; RoPE(q_rope, pos)]  ([ARCH] 2.3, decoupled query).
      2. Materialise every cached token's key and value for head h:
         k_t = [W_UK[h] c_t ; k_rope_t],  v_t = W_UV[h] c_t
         ([ARCH] 2.3 content key k^C = W^UK c; 3.2 value v^C = W^UV c;
         W^UK_i is d_h x d_c, W^UV_i is d_v x d_c).
      3. s_t = (q . k_t) / sqrt(d_nope + d_rope)  ([ARCH] 3.1 score
         definition; [RADAR] 2).
      4. p = softmax over the visible tokens (two passes: max, then
         normalised exponentials)  ([MATH] value absorption).
      5. o = sum_t p_t v_t;  lse = max + log(sum exp(s - max)).

    rows: optional iterable of (b, i, h) to compute; others stay NaN.
    Returns dict(o=[B, Lq, H, d_v], lse=[B, Lq, H]) float64.
    """
    cfg = inp.cfg
    B, Lq, H = cfg.batch, cfg.q_len, cfg.heads
    dc = cfg.d_latent
    o = np.full((B, Lq, H, cfg.d_v), np.nan)
    lse = np.full((B, Lq, H), np.nan)
    scale = 1.0 / math.sqrt(cfg.d_nope + cfg.d_rope)
    q_nope = stored_to_f64(inp.q_nope, cfg.q_dtype)
    q_rope = stored_to_f64(inp.q_rope, cfg.q_dtype)
    w_uk = stored_to_f64(inp.w_uk, cfg.q_dtype)
    w_uv = stored_to_f64(inp.w_uv, cfg.q_dtype)

    for b, heads in _rows_by_seq(cfg, rows).items():
        length = int(inp.seq_lens[b])
        cache = cache_f64(inp, b)
        c_kv, k_rope = cache[:, :dc], cache[:, dc:]
        for h, qs in heads.items():
            k_content = c_kv @ w_uk[h].T            # [len, d_nope]
            keys = np.concatenate([k_content, k_rope], axis=1)
            values = c_kv @ w_uv[h].T               # [len, d_v]
            for i in qs:
                q = np.concatenate([q_nope[b, i, h],
                                    rope_interleaved(q_rope[b, i, h], inp.positions[b, i], cfg.rope_base)])
                n = _visible(cfg, length, i)
                if n == 0:
                    o[b, i, h] = 0.0
                    lse[b, i, h] = -np.inf
                    continue
                s = (keys[:n] @ q) * scale
                m = np.max(s)
                e = np.exp(s - m)
                z = np.sum(e)
                p = e / z
                o[b, i, h] = p @ values[:n]
                lse[b, i, h] = m + np.log(z)
    return {"o": o, "lse": lse}


def mla_expand(inp, b: int):
    """Per-head content keys and values of sequence b's cached latents, the
    first step of the MHA form used for prefill ("DeepSeek's attention
    evolution - [MLA]" 2.5; [ARCH] 2.3 content key W^UK c, 3.2 value W^UV c):

      k_nope[t, h, :] = W_UK[h] c_t      (d_nope)
      v[t, h, :]      = W_UV[h] c_t      (d_v)

    Returns (k_nope [len_b, H, d_nope], v [len_b, H, d_v]) float64.  The
    attention that follows is ``mla_decode`` itself: with q_len prompt tokens
    and ``causal`` it scores exactly these keys and values.
    """
    cfg = inp.cfg
    dc = cfg.d_latent
    c_kv = cache_f64(inp, b)[:, :dc]
    w_uk = stored_to_f64(inp.w_uk, cfg.q_dtype)
    w_uv = stored_to_f64(inp.w_uv, cfg.q_dtype)
    k_nope = np.einsum("hdc,tc->thd", w_uk, c_kv)
    v = np.einsum("hdc,tc->thd", w_uv, c_kv)
    return k_nope, v


def mla_absorbed(inp, rows: Optional[Iterable] = None):
    """Absorbed intermediates, for per-stage checks only.

      q_lat = W_UK[h]^T q_nope                ([ARCH] 3.1 absorbed query)
      q_pe  = RoPE(q_rope, pos)
      s_t   = (q_lat . c_t + q_pe . k_rope_t) / sqrt(d_nope + d_rope)
      p     = softmax(s) over visible tokens
      o_lat = sum_t p_t c_t                   ([ARCH] 3.2, latent sum)
      o     = W_UV[h] o_lat
    Returns dict(q_lat, q_pe, o_lat, lse, o) float64.
    """
    cfg = inp.cfg
    B, Lq, H = cfg.batch, cfg.q_len, cfg.heads
    dc = cfg.d_latent
    q_nope = stored_to_f64(inp.q_nope, cfg.q_dtype)
    q_rope = stored_to_f64(inp.q_rope, cfg.q_dtype)
    w_uk = stored_to_f64(inp.w_uk, cfg.q_dtype)
    w_uv = stored_to_f64(inp.w_uv, cfg.q_dtype)
    scale = 1.0 / math.sqrt(cfg.d_nope + cfg.d_rope)

    q_lat = np.einsum("bihd,hdc->bihc", q_nope, w_uk)
    q_pe = rope_interleaved(q_rope, inp.positions[:, :, None], cfg.rope_base)
    o_lat = np.full((B, Lq, H, dc), np.nan)
    lse = np.full((B, Lq, H), np.nan)
    o = np.full((B, Lq, H, cfg.d_v), np.nan)
    for b, heads in _rows_by_seq(cfg, rows).items():
        length = int(inp.seq_lens[b])
        cache = cache_f64(inp, b)
        c_kv, k_rope = cache[:, :dc], cache[:, dc:]
        for h, qs in heads.items():
            for i in qs:
                n = _visible(cfg, length, i)
                if n == 0:
                    o_lat[b, i, h] = 0.0
                    o[b, i, h] = 0.0
                    lse[b, i, h] = -np.inf
                    continue
                s = (c_kv[:n] @ q_lat[b, i, h] + k_rope[:n] @ q_pe[b, i, h]) * scale
                m = np.max(s)
                e = np.exp(s - m)
                z = np.sum(e)
                o_lat[b, i, h] = (e / z) @ c_kv[:n]
                lse[b, i, h] = m + np.log(z)
                o[b, i, h] = w_uv[h] @ o_lat[b, i, h]
    return {"q_lat": q_lat, "q_pe": q_pe, "o_lat": o_lat, "lse": lse, "o": o}


# ------------------------------------------------- cache-append producer


def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """Root-mean-square normalisation over the last axis with a learned
    per-channel weight ([MATH] reference module: the latent passes through
    an RMSNorm, kv_norm, before it is cached): x / sqrt(mean(x**2) + eps) * w."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(weight, np.float64)


def kv_append(h, w_dkv, kv_norm_w, w_kr, pos, rope_base: float, eps: float):
    """The cache row of each new token (the producer of the cached latent).

    [ARCH] 2.1: the hidden state is down-projected to the latent,
    c = W_DKV h (d_c = 512 wide); [MATH] reference module: the cached latent
    is kv_norm(W_DKV h).  [ARCH] 2.3: the decoupled key is projected on its
    own and rotated at the token's position, k_R = RoPE(W_KR h), shared by
    all heads.

    h: [N, d] (one row per new token); w_dkv: [d_c, d]; w_kr: [d_R, d]
    (one row per output channel, the Linear-weight layout of the module);
    kv_norm_w: [d_c]; pos: [N].  Returns c_kv [N, d_c] and k_rope [N, d_R]
    in float64.
    """
    h = np.asarray(h, dtype=np.float64)
    c = h @ np.asarray(w_dkv, np.float64).T
    c_kv = rms_norm(c, kv_norm_w, eps)
    k_rope = rope_interleaved(h @ np.asarray(w_kr, np.float64).T, np.asarray(pos), rope_base)
    return c_kv, k_rope


# ------------------------------------------- output-side absorption


def fuse_out_weight(w_o, w_uv, heads: int):
    """The pre-fused output weight of each head ([ARCH] 3.2: W~_O,i =
    W_O,i W_UV,i in R^{d x d_c}; [MATH] value output matrix absorption:
    W_O = [W_O^1, ..., W_O^{n_h}] in R^{d x (n_h d_v)}).

    w_o: [d, H * d_v] (column block i is W_O,i); w_uv: [H, d_v, d_c].
    Returns [d, H, d_c] float64 (the layout of a map from the H x d_c latent
    outputs to the d-wide hidden state).
    """
    w_o = np.asarray(w_o, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    d = w_o.shape[0]
    d_v = w_uv.shape[1]
    out = np.empty((d, heads, w_uv.shape[2]))
    for i in range(heads):
        out[:, i, :] = w_o[:, i * d_v:(i + 1) * d_v] @ w_uv[i]
    return out


def out_proj_fused(o_lat, w_fused):
    """The hidden-state contribution of the attention block straight from the
    latent outputs ([ARCH] 3.2: u_t = sum_i W~_O,i o~_{t,i}).

    o_lat: [M, H, d_c] (one row per query token); w_fused: [d, H, d_c].
    Returns [M, d] float64.
    """
    o = np.asarray(o_lat, np.float64)
    w = np.asarray(w_fused, np.float64)
    return o.reshape(o.shape[0], -1) @ w.reshape(w.shape[0], -1).T


# ------------------------------------------------------- byte accounting


def kv_cache_bytes_per_token(kind: str, *, n_kv_heads: int = 0, d_head: int = 0,
                             d_latent: int = 0, d_rope: int = 0,
                             elem_bytes: float = 2, scale_bytes: int = 0) -> float:
    """Per-token, per-layer cache bytes.

    Head-based caches store one key and one value per KV head
    (2 * n_kv_heads * d_head elements; [ARCH] introduction, [MATH] cache
    footprint mechanics).  MLA stores the latent and the decoupled key only
    (d_latent + d_rope elements; [ARCH] 2.4), plus any per-token scale.
    """
    if kind in ("mha", "gqa", "mqa"):
        return 2 * n_kv_heads * d_head * elem_bytes
    if kind == "mla":
        return (d_latent + d_rope) * elem_bytes + scale_bytes
    raise ValueError(kind)
