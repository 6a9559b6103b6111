"""One decode step: buffers and the library calls in order.

Argument marshalling only: torch allocates the caller-owned outputs and
split-K workspaces once; ``run`` enqueues mla_absorb_q, mla_decode_attn and
mla_combine_out_proj (the combine and the W_UV projection in one call) on the
current stream.  ``capture`` records the
same three launches (for one or more consecutive steps) in a HIP graph, whose
replay skips the per-launch host overhead (the library records kernel
launches only, no memset nodes).
"""

from __future__ import annotations

import torch

from . import binding as _b

TORCH_DTYPE = {_b.F32: torch.float32, _b.BF16: torch.bfloat16}


class DecodeStep:
    def __init__(self, d: _b.MLADims, *, num_splits: int | None = None, device="cuda",
                 keep_o_lat: bool = True):
        self.d = d
        self.keep_o_lat = keep_o_lat  # also write the latent output o_lat
        self.device = torch.device(device)
        self.num_splits = int(num_splits) if num_splits else _b.mla_num_splits_hint(
            d, self.device.index or 0)
        qt = TORCH_DTYPE[d.q_dtype]
        B, Lq, H = d.batch, d.q_len, d.heads
        W = d.d_latent + d.d_rope
        n_o, n_l = _b.mla_workspace_elems(d, self.num_splits)
        kw = dict(device=self.device)
        # the absorbed query: fp32 on the fp32 path, fp16 for bf16 queries (mla.h)
        self.q_abs = torch.empty((B, Lq, H, W), dtype=torch.float32 if d.q_dtype == _b.F32
                                 else torch.float16, **kw)
        # normalised partials: fp32 on the fp32 path, fp16 otherwise (mla.h)
        pt = torch.float32 if d.q_dtype == _b.F32 else torch.float16
        self.o_part = torch.empty(max(n_o, 1), dtype=pt, **kw)
        self.lse_part = torch.empty(max(n_l, 1), dtype=torch.float32, **kw)
        self.o_lat = torch.empty((B, Lq, H, d.d_latent), dtype=qt, **kw)
        self.lse = torch.empty((B, Lq, H), dtype=torch.float32, **kw)
        self.o = torch.empty((B, Lq, H, d.d_v), dtype=qt, **kw)

    def run(self, *, q_nope, q_rope, positions, w_uk, w_uv, latent, rope, kv_row_stride,
            kv_scale, seq_lens, block_table, max_blocks_per_seq, max_seq_len, causal,
            softmax_scale, rope_base=10000.0, stream=None):
        d = self.d
        _b.mla_absorb_q(d, q_nope, q_rope, positions, rope_base, w_uk, self.q_abs, stream)
        _b.mla_decode_attn(d, self.q_abs, latent, rope, kv_row_stride, kv_scale, seq_lens,
                           block_table, max_blocks_per_seq, _b.TILE_TOKENS, max_seq_len,
                           causal, softmax_scale, self.num_splits, self.o_part, self.lse_part,
                           stream)
        # o_lat may be skipped only where the combine and projection run fused
        fused = (d.q_dtype == _b.BF16 and d.d_latent == 512 and d.d_v % 32 == 0
                 and not d.flags & _b.FLAG_GENERIC)
        _b.mla_combine_out_proj(d, self.num_splits, seq_lens, self.o_part, self.lse_part, w_uv,
                                self.o, self.lse,
                                self.o_lat if (self.keep_o_lat or not fused) else None, stream)
        return self.o

    def capture(self, steps: int = 1, **kwargs) -> torch.cuda.CUDAGraph:
        """Record ``steps`` consecutive steps of ``run(**kwargs)`` (without
        ``stream``) in one HIP graph; ``replay()`` re-runs them on the same
        inputs and buffers.  Several steps per graph (as a model's layers
        would share one graph) spread the per-replay launch cost over them."""
        if steps < 1:
            raise ValueError("steps must be >= 1")
        cur = torch.cuda.current_stream(self.device)
        side = torch.cuda.Stream(device=self.device)
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            self.run(**kwargs)  # first launches outside the capture
        cur.wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(steps):
                self.run(**kwargs)
        return graph
