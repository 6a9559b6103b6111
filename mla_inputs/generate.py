"""Seeded generator of MLA decode inputs.

Everything is drawn from numpy's PCG64 with one independent stream per
(config seed, tensor id, index), so any single sequence's cache can be
regenerated without drawing the others.  Values are drawn in float32, scaled,
then rounded once to the storage format:

* bf16: round-to-nearest-even on the float32 bit pattern;
* fp32: as drawn;
* fp8:  OCP E4M3 ("e4m3fn": bias 7, max 448, no infinities) with one fp32
  scale per cached token, scale = amax(row)/448, codes = RNE(row/scale) via
  torch's float8_e4m3fn cast.

Cached keys are stored after RoPE ("Multi-Head Latent Attention (MLA):
Mathematical Foundations ...", reference module, cache append).  The values
drawn here *are* those stored post-rotation values: a rotation of an isotropic
Gaussian pair is again an isotropic Gaussian pair, so drawing the stored value
directly gives the distribution a rotated draw would have, and no rotation is
computed here.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import BLOCK_TOKENS, MLAConfig

# Tensor ids of the independent random streams.
_T_LENS, _T_QNOPE, _T_QROPE, _T_WUK, _T_WUV, _T_CACHE, _T_OUTLIER, _T_PERM = range(1, 9)

BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)


def _rng(seed: int, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *ids])))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # (u + 0x7FFF + lsb) >> 16, with lsb the bit that becomes the last kept
    # one; computed in place (one temporary) since caches run to 10^8 values
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def fp8_codes_from_f32(x: np.ndarray) -> np.ndarray:
    """Encode float32 values (|x| <= 448) as OCP E4M3 codes (uint8)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_from_f32(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


@dataclass
class Pool:
    """Cached rows as the GPU sees them.

    rows:        [n_rows, d_latent + d_rope] in the storage format (uint16 bf16
                 bits, float32, or uint8 E4M3 codes); row r holds the latent
                 at columns [0, d_latent) and the post-RoPE key after it.
    kv_scale:    [n_rows] float32 per-token scale (fp8 only).
    block_table: [batch, max_blocks_per_seq] int32 physical block ids, -1 for
                 unused entries (paged only).
    Rows that belong to no cached token (tails of the last block, or past the
    end of a sequence in the contiguous layout) hold NaN.
    """

    rows: np.ndarray
    kv_scale: Optional[np.ndarray]
    block_table: Optional[np.ndarray]
    max_blocks_per_seq: int
    max_seq_len: int

    def row_index(self, b: int, t: int) -> int:
        if self.block_table is not None:
            return int(self.block_table[b, t // BLOCK_TOKENS]) * BLOCK_TOKENS + t % BLOCK_TOKENS
        return b * self.max_seq_len + t


class MLAInputs:
    """All inputs of one decode step for ``cfg``, drawn from ``cfg.seed``."""

    def __init__(self, cfg: MLAConfig, seed: Optional[int] = None):
        self.cfg = cfg
        self.seed = cfg.seed if seed is None else seed
        c = cfg
        B, Lq, H = c.batch, c.q_len, c.heads

        if c.ragged:
            lens = _rng(self.seed, _T_LENS).integers(c.len_lo, c.len_hi + 1, size=B)
        else:
            lens = np.full(B, c.seq_len)
        self.seq_lens = lens.astype(np.int32)

        i = np.arange(Lq, dtype=np.int64)[None, :]
        L = self.seq_lens.astype(np.int64)[:, None]
        pos = (L - Lq + i) if c.query_in_cache else (L + i)
        self.positions = pos.astype(np.int32)

        def draw(tid, shape, std=1.0):
            return _rng(self.seed, tid).standard_normal(shape, dtype=np.float32) * np.float32(std)

        self.q_nope = _store(draw(_T_QNOPE, (B, Lq, H, c.d_nope)), c.q_dtype)
        self.q_rope = _store(draw(_T_QROPE, (B, Lq, H, c.d_rope)), c.q_dtype)
        self.w_uk = _store(draw(_T_WUK, (H, c.d_nope, c.d_latent), c.w_std), c.q_dtype)
        self.w_uv = _store(draw(_T_WUV, (H, c.d_v, c.d_latent), c.w_std), c.q_dtype)
        self.softmax_scale = c.softmax_scale
        self.rope_base = c.rope_base
        self._pool: Optional[Pool] = None

    # ------------------------------------------------------------------ cache
    def cache_source(self, b: int) -> np.ndarray:
        """float32 [len_b, d_latent + d_rope] values before storage rounding."""
        c = self.cfg
        n = int(self.seq_lens[b])
        x = _rng(self.seed, _T_CACHE, b).standard_normal((n, c.row_width), dtype=np.float32)
        if c.outlier_frac > 0.0 and n > 0:
            k = int(np.ceil(c.outlier_frac * n))
            idx = _rng(self.seed, _T_OUTLIER, b).permutation(n)[:k]
            x[idx] *= np.float32(c.outlier_scale)
        return x

    def cache_stored(self, b: int):
        """(rows [len_b, W] in storage format, per-token fp32 scale or None)."""
        x = self.cache_source(b)
        if self.cfg.kv_dtype == "fp8":
            amax = np.max(np.abs(x), axis=1) if x.shape[0] else np.zeros(0, np.float32)
            scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
            codes = fp8_codes_from_f32(x / scale[:, None])
            return codes, scale
        return _store(x, self.cfg.kv_dtype), None

    # ------------------------------------------------------------------- pool
    def pool(self) -> Pool:
        if self._pool is None:
            self._pool = self._build_pool()
        return self._pool

    def _build_pool(self) -> Pool:
        c = self.cfg
        W = c.row_width
        B = c.batch
        store_dt = {"bf16": np.uint16, "f32": np.float32, "fp8": np.uint8}[c.kv_dtype]
        nan = {"bf16": BF16_NAN, "f32": np.float32(np.nan), "fp8": FP8_NAN}[c.kv_dtype]
        fp8 = c.kv_dtype == "fp8"
        max_blocks = -(-c.max_seq_len // BLOCK_TOKENS)

        if c.paged:
            nblk = [-(-int(n) // BLOCK_TOKENS) for n in self.seq_lens]
            total = int(sum(nblk))
            perm = _rng(self.seed, _T_PERM).permutation(total).astype(np.int32)
            table = np.full((B, max_blocks), -1, dtype=np.int32)
            n_rows = total * BLOCK_TOKENS
        else:
            table = None
            n_rows = B * c.max_seq_len
        rows = np.empty((n_rows, W), dtype=store_dt)
        rows[...] = nan
        scale = np.full(n_rows, np.nan, dtype=np.float32) if fp8 else None

        off = 0
        for b in range(B):
            n = int(self.seq_lens[b])
            vals, sc = self.cache_stored(b)
            if c.paged:
                k = nblk[b]
                ids = perm[off:off + k]
                off += k
                table[b, :k] = ids
                full = n // BLOCK_TOKENS
                if full:
                    blk = rows.reshape(-1, BLOCK_TOKENS, W)
                    blk[ids[:full]] = vals[: full * BLOCK_TOKENS].reshape(full, BLOCK_TOKENS, W)
                    if fp8:
                        scale.reshape(-1, BLOCK_TOKENS)[ids[:full]] = sc[: full * BLOCK_TOKENS].reshape(full, BLOCK_TOKENS)
                if n % BLOCK_TOKENS:
                    r0 = int(ids[full]) * BLOCK_TOKENS
                    tail = n - full * BLOCK_TOKENS
                    rows[r0:r0 + tail] = vals[full * BLOCK_TOKENS:]
                    if fp8:
                        scale[r0:r0 + tail] = sc[full * BLOCK_TOKENS:]
            else:
                r0 = b * c.max_seq_len
                rows[r0:r0 + n] = vals
                if fp8:
                    scale[r0:r0 + n] = sc
        return Pool(rows=rows, kv_scale=scale, block_table=table,
                    max_blocks_per_seq=max_blocks, max_seq_len=c.max_seq_len)


# Tensor ids of the cache-append producer's streams.
_T_APP_H, _T_APP_WDKV, _T_APP_WKR, _T_APP_NORM, _T_APP_POS, _T_APP_ROWS = range(101, 107)


@dataclass
class AppendInputs:
    """Seeded inputs of the cache-append producer (bf16 bit patterns).

    h ~ N(0, 1) [n, d]; w_dkv ~ N(0, 1/d) [d_c, d]; w_kr ~ N(0, 1/d)
    [d_R, d]; the RMSNorm weight ~ 1 + 0.1 N(0, 1) [d_c]; positions uniform
    in [0, max_pos); destination rows a seeded choice of n distinct rows of
    a pool of ``pool_rows``.
    """
    n: int
    d_model: int
    seed: int
    d_latent: int = 512
    d_rope: int = 64
    max_pos: int = 131072
    pool_rows: int = 0

    def __post_init__(self):
        n, d, dc, dr = self.n, self.d_model, self.d_latent, self.d_rope
        f32 = np.float32
        self.h = bf16_bits_from_f32(_rng(self.seed, _T_APP_H).standard_normal((n, d), dtype=f32))
        self.w_dkv = bf16_bits_from_f32(
            _rng(self.seed, _T_APP_WDKV).standard_normal((dc, d), dtype=f32) / f32(np.sqrt(d)))
        self.w_kr = bf16_bits_from_f32(
            _rng(self.seed, _T_APP_WKR).standard_normal((dr, d), dtype=f32) / f32(np.sqrt(d)))
        self.kv_norm_w = bf16_bits_from_f32(
            f32(1.0) + f32(0.1) * _rng(self.seed, _T_APP_NORM).standard_normal(dc, dtype=f32))
        self.positions = _rng(self.seed, _T_APP_POS).integers(0, self.max_pos, n).astype(np.int32)
        if n:
            self.positions[0] = 0
        pool = self.pool_rows or 2 * n + 1
        self.pool_rows = pool
        self.rows = _rng(self.seed, _T_APP_ROWS).permutation(pool)[:n].astype(np.int64)


# Tensor ids of the output-side absorption's streams.
_T_OUT_OLAT, _T_OUT_WO, _T_OUT_WUV = range(201, 204)


@dataclass
class OutProjInputs:
    """Seeded inputs of the output-side absorption (bf16 bit patterns).

    o_lat ~ N(0, 1) [m, heads, d_latent] (the attention's latent outputs of
    m query tokens); w_o ~ N(0, 1/(heads d_v)) [d_model, heads d_v];
    w_uv ~ N(0, 1/d_latent) [heads, d_v, d_latent].
    """
    m: int
    heads: int
    d_model: int
    seed: int
    d_v: int = 128
    d_latent: int = 512

    def __post_init__(self):
        f32 = np.float32
        H, dv, dc = self.heads, self.d_v, self.d_latent
        self.o_lat = bf16_bits_from_f32(
            _rng(self.seed, _T_OUT_OLAT).standard_normal((self.m, H, dc), dtype=f32))
        self.w_o = bf16_bits_from_f32(
            _rng(self.seed, _T_OUT_WO).standard_normal((self.d_model, H * dv), dtype=f32)
            / f32(np.sqrt(H * dv)))
        self.w_uv = bf16_bits_from_f32(
            _rng(self.seed, _T_OUT_WUV).standard_normal((H, dv, dc), dtype=f32) / f32(np.sqrt(dc)))
