// Kernel launchers of the MLA decode library (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

struct DecodeArgs {
  const void* q_abs;
  const void* latent;
  const void* rope;
  int64_t row_stride;      // elements between consecutive cache rows
  const float* kv_scale;   // fp8 per-row scale, else nullptr
  const int32_t* seq_lens;
  const int32_t* block_table;
  int mbps;                // max_blocks_per_seq
  int max_seq_len;
  int batch, q_len, heads, d_c, d_r;
  int causal;
  float softmax_scale;
  int num_splits;
  void* o_part;            // normalised partials: fp16 if part_f16, else fp32
  int part_f16;
  float* lse_part;
};

// MHA-form prefill (bf16, d_nope = d_v = 128, d_rope = 64, d_latent = 512).
struct PrefillArgs {
  const void* latent;       // cache rows, as for decode
  const void* rope;
  int64_t row_stride;       // elements
  const int32_t* seq_lens;
  const int32_t* block_table;
  int mbps, max_seq_len;
  int batch, q_len, heads;
  int causal;
  float softmax_scale;
  const uint16_t* w_uk;     // [H, 128, 512]
  const uint16_t* w_uv;     // [H, 128, 512]
  void* k_nope;             // [B, max_seq_len, H, 128]
  void* v;                  // [B, max_seq_len, H, 128]
  const void* q_nope;       // [B, Lq, H, 128]
  const void* q_rope;       // [B, Lq, H, 64], before rotation
  const int32_t* positions; // [B, Lq]
  float rope_base;
  void* o;                  // [B, Lq, H, 128]
  float* lse;               // [B, Lq, H] or nullptr
  int ntile;                // set by the expand launcher
};

hipError_t launch_absorb_generic(const mla_dims_t& d, const void* q_nope, const void* q_rope,
                                 const int32_t* positions, float rope_base, const void* w_uk,
                                 void* q_abs, hipStream_t s);
bool generic_decode_supports(const mla_dims_t& d);
hipError_t launch_decode_generic(const mla_dims_t& d, const DecodeArgs& a, hipStream_t s);
hipError_t launch_out_proj_generic(const mla_dims_t& d, const void* o_lat, const void* w_uv,
                                   void* o, hipStream_t s);
hipError_t launch_combine(const mla_dims_t& d, int num_splits, const int32_t* seq_lens,
                          const void* o_part, const float* lse_part, void* o_lat,
                          float* lse_out, hipStream_t s);

// MFMA kernels (bf16 queries and weights, gfx950).
bool mfma_absorb_supports(const mla_dims_t& d);
hipError_t launch_absorb_mfma(const mla_dims_t& d, const void* q_nope, const void* q_rope,
                              const int32_t* positions, float rope_base, const void* w_uk,
                              void* q_abs, hipStream_t s);
bool mfma_decode_supports(const mla_dims_t& d, int64_t row_stride, const void* latent,
                          const void* rope);
hipError_t launch_decode_mfma(const mla_dims_t& d, const DecodeArgs& a, hipStream_t s);
bool mfma_out_proj_supports(const mla_dims_t& d);
bool combine_proj_supports(const mla_dims_t& d);
bool prefill_supports(const mla_dims_t& d, int64_t row_stride, int max_seq_len);
hipError_t launch_prefill_expand(const mla_dims_t& d, const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_attn(const mla_dims_t& d, const PrefillArgs& a, hipStream_t s);
hipError_t launch_combine_proj(const mla_dims_t& d, int num_splits, const int32_t* seq_lens,
                               const void* o_part, const float* lse_part, const void* w_uv,
                               void* o, float* lse_out, void* o_lat, hipStream_t s);
hipError_t launch_out_proj_mfma(const mla_dims_t& d, const void* o_lat, const void* w_uv,
                                void* o, hipStream_t s);

// Output-side absorption (bf16, latent 512, d_v <= 128).
bool out_fused_supports(const mla_dims_t& d, int d_model);
hipError_t launch_fuse_out(const mla_dims_t& d, int d_model, const void* w_o, const void* w_uv,
                           void* w_fused, hipStream_t s);
int64_t fused_out_weight_elems(const mla_dims_t& d, int d_model);
int64_t out_fused_workspace_bytes(const mla_dims_t& d, int d_model);
hipError_t launch_out_fused(const mla_dims_t& d, int d_model, const void* o_lat, const void* w_fused,
                            float* workspace, void* out, hipStream_t s);

}  // namespace mla
