// C ABI entry points: host-side validation, then dispatch to the MFMA
// kernels (bf16 queries/weights at the widths they are built for) or to the
// plain SIMT kernels.  Nothing here allocates or synchronises.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.hpp"
#include "kernels.hpp"

using namespace mla;

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_dims(const mla_dims_t* d) {
  if (!d) return MLA_ERR_INVALID_ARG;
  if (d->batch < 0 || d->q_len < 1 || d->heads < 1 || d->d_nope < 1 || d->d_rope < 0 ||
      (d->d_rope & 1) || d->d_latent < 8 || (d->d_latent % 8) || d->d_v < 1)
    return MLA_ERR_INVALID_ARG;
  if (d->flags & ~(int32_t)MLA_FLAG_GENERIC) return MLA_ERR_INVALID_ARG;
  if (d->q_dtype != MLA_F32 && d->q_dtype != MLA_BF16) return MLA_ERR_INVALID_ARG;
  if (d->kv_dtype != MLA_F32 && d->kv_dtype != MLA_BF16 && d->kv_dtype != MLA_FP8_E4M3)
    return MLA_ERR_INVALID_ARG;
  const bool ok_mix = d->q_dtype == MLA_F32 ? d->kv_dtype == MLA_F32 : d->kv_dtype != MLA_F32;
  if (!ok_mix) return MLA_ERR_UNSUPPORTED;
  // row counts must fit the grid dimensions used below
  if ((int64_t)d->batch * d->q_len * d->heads > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

bool use_mfma(const mla_dims_t* d) { return !(d->flags & MLA_FLAG_GENERIC); }

int launched(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

int check_cache_args(const mla_dims_t* dims, int64_t kv_row_stride, const int32_t* seq_lens,
                     const int32_t* block_table, int32_t max_blocks_per_seq, int32_t block_size,
                     int32_t max_seq_len) {
  if (!seq_lens) return MLA_ERR_INVALID_ARG;
  if (kv_row_stride < dims->d_latent || kv_row_stride < dims->d_rope) return MLA_ERR_INVALID_ARG;
  if (max_seq_len < 1) return MLA_ERR_INVALID_ARG;
  if (block_table) {
    if (block_size != MLA_TILE_TOKENS) return MLA_ERR_INVALID_ARG;
    if ((int64_t)max_blocks_per_seq * MLA_TILE_TOKENS < max_seq_len) return MLA_ERR_INVALID_ARG;
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: invalid argument";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: combination not built";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: split-K workspace missing";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime or launch failure";
    case MLA_ERR_TOO_LARGE: return "MLA_ERR_TOO_LARGE: request exceeds a fixed internal buffer";
    default: return "unknown MLA status";
  }
}

int mla_absorb_q(const mla_dims_t* dims, const void* q_nope, const void* q_rope,
                 const int32_t* positions, float rope_base, const void* w_uk, void* q_abs,
                 void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->batch == 0) return MLA_OK;
  if (!q_nope || !w_uk || !q_abs || (dims->d_rope && (!q_rope || !positions)))
    return MLA_ERR_INVALID_ARG;
  if (!aligned16(q_nope) || !aligned16(w_uk) || !aligned16(q_abs) ||
      (q_rope && !aligned16(q_rope)))
    return MLA_ERR_INVALID_ARG;
  if (!(rope_base > 0.f) || !isfinite(rope_base)) return MLA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  if (use_mfma(dims) && mfma_absorb_supports(*dims))
    return launched(launch_absorb_mfma(*dims, q_nope, q_rope, positions, rope_base, w_uk, q_abs, s));
  return launched(launch_absorb_generic(*dims, q_nope, q_rope, positions, rope_base, w_uk, q_abs, s));
}

int mla_decode_attn(const mla_dims_t* dims, const void* q_abs, const void* latent_cache,
                    const void* rope_cache, int64_t kv_row_stride, const float* kv_scale,
                    const int32_t* seq_lens, const int32_t* block_table,
                    int32_t max_blocks_per_seq, int32_t block_size, int32_t max_seq_len,
                    int32_t causal, float softmax_scale, int32_t num_splits, void* o_part,
                    float* lse_part, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->batch == 0) return MLA_OK;
  if (!q_abs || !latent_cache || (dims->d_rope && !rope_cache) || !seq_lens)
    return MLA_ERR_INVALID_ARG;
  if (!o_part || !lse_part) return MLA_ERR_WORKSPACE;
  if (!aligned16(q_abs) || !aligned16(o_part) || !aligned16(lse_part))
    return MLA_ERR_INVALID_ARG;
  if (kv_row_stride < dims->d_latent || kv_row_stride < dims->d_rope) return MLA_ERR_INVALID_ARG;
  if (max_seq_len < 1 || num_splits < 1 || num_splits > 65536) return MLA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return MLA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return MLA_ERR_INVALID_ARG;
  if ((dims->kv_dtype == MLA_FP8_E4M3) != (kv_scale != nullptr)) return MLA_ERR_INVALID_ARG;
  if (block_table) {
    if (block_size != MLA_TILE_TOKENS) return MLA_ERR_INVALID_ARG;
    if ((int64_t)max_blocks_per_seq * MLA_TILE_TOKENS < max_seq_len) return MLA_ERR_INVALID_ARG;
  }
  DecodeArgs a;
  a.q_abs = q_abs;
  a.latent = latent_cache;
  a.rope = rope_cache;
  a.row_stride = kv_row_stride;
  a.kv_scale = kv_scale;
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.mbps = max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  a.batch = dims->batch;
  a.q_len = dims->q_len;
  a.heads = dims->heads;
  a.d_c = dims->d_latent;
  a.d_r = dims->d_rope;
  a.causal = causal;
  a.softmax_scale = softmax_scale;
  a.num_splits = num_splits;
  a.o_part = o_part;
  a.part_f16 = dims->q_dtype != MLA_F32;
  a.lse_part = lse_part;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  if (use_mfma(dims) && mfma_decode_supports(*dims, kv_row_stride, latent_cache, rope_cache))
    return launched(launch_decode_mfma(*dims, a, s));
  if (!generic_decode_supports(*dims)) return MLA_ERR_UNSUPPORTED;
  return launched(launch_decode_generic(*dims, a, s));
}

int mla_combine(const mla_dims_t* dims, int32_t num_splits, const int32_t* seq_lens,
                const void* o_part, const float* lse_part, void* o_lat, float* lse_out,
                void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->batch == 0) return MLA_OK;
  if (!seq_lens || !o_lat) return MLA_ERR_INVALID_ARG;
  if (!o_part || !lse_part) return MLA_ERR_WORKSPACE;
  if (num_splits < 1 || num_splits > 65536) return MLA_ERR_INVALID_ARG;
  if (!aligned16(o_part) || !aligned16(o_lat)) return MLA_ERR_INVALID_ARG;
  (void)hipGetLastError();
  return launched(launch_combine(*dims, num_splits, seq_lens, o_part, lse_part, o_lat, lse_out,
                                 (hipStream_t)stream));
}

int mla_out_proj(const mla_dims_t* dims, const void* o_lat, const void* w_uv, void* o,
                 void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->batch == 0) return MLA_OK;
  if (!o_lat || !w_uv || !o) return MLA_ERR_INVALID_ARG;
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(o)) return MLA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  if (use_mfma(dims) && mfma_out_proj_supports(*dims))
    return launched(launch_out_proj_mfma(*dims, o_lat, w_uv, o, s));
  return launched(launch_out_proj_generic(*dims, o_lat, w_uv, o, s));
}

int mla_combine_out_proj(const mla_dims_t* dims, int32_t num_splits, const int32_t* seq_lens,
                         const void* o_part, const float* lse_part, const void* w_uv, void* o,
                         float* lse_out, void* o_lat, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->batch == 0) return MLA_OK;
  if (!seq_lens || !w_uv || !o) return MLA_ERR_INVALID_ARG;
  if (!o_part || !lse_part) return MLA_ERR_WORKSPACE;
  if (num_splits < 1 || num_splits > 65536) return MLA_ERR_INVALID_ARG;
  if (!aligned16(o_part) || !aligned16(w_uv) || !aligned16(o) || !aligned16(o_lat))
    return MLA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();
  if (use_mfma(dims) && combine_proj_supports(*dims))
    return launched(launch_combine_proj(*dims, num_splits, seq_lens, o_part, lse_part, w_uv, o,
                                        lse_out, o_lat, s));
  // the two kernels in turn: the latent output goes through o_lat
  if (!o_lat) return MLA_ERR_INVALID_ARG;
  st = launched(launch_combine(*dims, num_splits, seq_lens, o_part, lse_part, o_lat, lse_out, s));
  if (st) return st;
  if (use_mfma(dims) && mfma_out_proj_supports(*dims))
    return launched(launch_out_proj_mfma(*dims, o_lat, w_uv, o, s));
  return launched(launch_out_proj_generic(*dims, o_lat, w_uv, o, s));
}

int mla_workspace_elems(const mla_dims_t* dims, int32_t num_splits, int64_t* o_part_elems,
                        int64_t* lse_part_elems) {
  int st = check_dims(dims);
  if (st) return st;
  if (num_splits < 1 || num_splits > 65536 || !o_part_elems || !lse_part_elems)
    return MLA_ERR_INVALID_ARG;
  const int64_t slots = dims->batch ? (int64_t)num_splits + dims->batch - 1 : 0;
  const int64_t rows = (int64_t)dims->q_len * dims->heads;
  *o_part_elems = slots * rows * dims->d_latent;
  *lse_part_elems = slots * rows;
  return MLA_OK;
}

int mla_workspace_bytes(const mla_dims_t* dims, int32_t num_splits, int64_t* o_part_bytes,
                        int64_t* lse_part_bytes) {
  if (!o_part_bytes || !lse_part_bytes) return MLA_ERR_INVALID_ARG;
  int64_t no = 0, nl = 0;
  const int st = mla_workspace_elems(dims, num_splits, &no, &nl);
  if (st) return st;
  *o_part_bytes = no * (dims->q_dtype == MLA_F32 ? 4 : 2);
  *lse_part_bytes = nl * 4;
  return MLA_OK;
}

int mla_num_splits_hint(const mla_dims_t* dims, int32_t device, int32_t* num_splits) {
  int st = check_dims(dims);
  if (st) return st;
  if (!num_splits) return MLA_ERR_INVALID_ARG;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
    return MLA_ERR_HIP;
  // one workgroup per (split unit, block of 128 query rows) on every
  // compute unit
  const int rows = dims->q_len * dims->heads;
  const int groups = (rows + 127) / 128;
  int g = cus / (groups > 0 ? groups : 1);
  *num_splits = g > 0 ? g : 1;
  return MLA_OK;
}

int mla_split_plan(int32_t batch, const int32_t* seq_lens_host, int32_t num_splits,
                   int32_t* first_unit, int32_t* last_unit, int64_t* first_tile) {
  if (batch < 0 || num_splits < 1 || num_splits > 65536) return MLA_ERR_INVALID_ARG;
  if (batch && (!seq_lens_host || !first_unit || !last_unit || !first_tile))
    return MLA_ERR_INVALID_ARG;
  int64_t T = 0;
  for (int b = 0; b < batch; ++b) {
    if (seq_lens_host[b] < 0) return MLA_ERR_INVALID_ARG;
    T += tiles_of(seq_lens_host[b]);
  }
  int64_t pb = 0;
  for (int b = 0; b < batch; ++b) {
    const int64_t tb = tiles_of(seq_lens_host[b]);
    first_tile[b] = pb;
    if (tb == 0) {
      first_unit[b] = last_unit[b] = -1;
    } else {
      first_unit[b] = (int32_t)unit_of_tile(pb, T, num_splits);
      last_unit[b] = (int32_t)unit_of_tile(pb + tb - 1, T, num_splits);
    }
    pb += tb;
  }
  return MLA_OK;
}


// ------------------------------------------------------------- prefill


int mla_prefill_expand(const mla_dims_t* dims, const void* latent_cache, int64_t kv_row_stride,
                       const int32_t* seq_lens, const int32_t* block_table,
                       int32_t max_blocks_per_seq, int32_t block_size, int32_t max_seq_len,
                       const void* w_uk, const void* w_uv, void* k_nope, void* v, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->batch == 0) return MLA_OK;
  if (!latent_cache || !w_uk || !w_uv || !k_nope || !v) return MLA_ERR_INVALID_ARG;
  st = check_cache_args(dims, kv_row_stride, seq_lens, block_table, max_blocks_per_seq, block_size,
                        max_seq_len);
  if (st) return st;
  if (!aligned16(latent_cache) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(k_nope) ||
      !aligned16(v))
    return MLA_ERR_INVALID_ARG;
  if (!prefill_supports(*dims, kv_row_stride, max_seq_len)) return MLA_ERR_UNSUPPORTED;
  PrefillArgs a{};
  a.latent = latent_cache;
  a.row_stride = kv_row_stride;
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.mbps = max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  a.batch = dims->batch;
  a.q_len = dims->q_len;
  a.heads = dims->heads;
  a.w_uk = (const uint16_t*)w_uk;
  a.w_uv = (const uint16_t*)w_uv;
  a.k_nope = k_nope;
  a.v = v;
  (void)hipGetLastError();
  return launched(launch_prefill_expand(*dims, a, (hipStream_t)stream));
}

int mla_prefill_attn(const mla_dims_t* dims, const void* q_nope, const void* q_rope,
                     const int32_t* positions, float rope_base, const void* k_nope,
                     const void* v, const void* rope_cache, int64_t kv_row_stride,
                     const int32_t* seq_lens, const int32_t* block_table,
                     int32_t max_blocks_per_seq, int32_t block_size, int32_t max_seq_len,
                     int32_t causal, float softmax_scale, void* o, float* lse, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (dims->batch == 0) return MLA_OK;
  if (!q_nope || !q_rope || !positions || !k_nope || !v || !rope_cache || !o)
    return MLA_ERR_INVALID_ARG;
  st = check_cache_args(dims, kv_row_stride, seq_lens, block_table, max_blocks_per_seq, block_size,
                        max_seq_len);
  if (st) return st;
  if (causal != 0 && causal != 1) return MLA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return MLA_ERR_INVALID_ARG;
  if (!(rope_base > 0.f) || !isfinite(rope_base)) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(k_nope) || !aligned16(v) ||
      !aligned16(rope_cache) || !aligned16(o))
    return MLA_ERR_INVALID_ARG;
  if (!prefill_supports(*dims, kv_row_stride, max_seq_len)) return MLA_ERR_UNSUPPORTED;
  PrefillArgs a{};
  a.rope = rope_cache;
  a.row_stride = kv_row_stride;
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.mbps = max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  a.batch = dims->batch;
  a.q_len = dims->q_len;
  a.heads = dims->heads;
  a.causal = causal;
  a.softmax_scale = softmax_scale;
  a.k_nope = const_cast<void*>(k_nope);
  a.v = const_cast<void*>(v);
  a.q_nope = q_nope;
  a.q_rope = q_rope;
  a.positions = positions;
  a.rope_base = rope_base;
  a.o = o;
  a.lse = lse;
  (void)hipGetLastError();
  return launched(launch_prefill_attn(*dims, a, (hipStream_t)stream));
}

// ---- Output-side absorption ----

int mla_fuse_out_weight(const mla_dims_t* dims, int32_t d_model, const void* w_o, const void* w_uv,
                        void* w_fused, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (d_model < 1 || !w_o || !w_uv || !w_fused) return MLA_ERR_INVALID_ARG;
  if (!aligned16(w_o) || !aligned16(w_uv) || !aligned16(w_fused)) return MLA_ERR_INVALID_ARG;
  if (!out_fused_supports(*dims, d_model)) return MLA_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  return launched(launch_fuse_out(*dims, d_model, w_o, w_uv, w_fused, (hipStream_t)stream));
}

int mla_fused_out_weight_bytes(const mla_dims_t* dims, int32_t d_model, int64_t* bytes) {
  int st = check_dims(dims);
  if (st) return st;
  if (d_model < 1 || !bytes) return MLA_ERR_INVALID_ARG;
  if (!out_fused_supports(*dims, d_model)) return MLA_ERR_UNSUPPORTED;
  *bytes = fused_out_weight_elems(*dims, d_model) * 2;
  return MLA_OK;
}

int mla_out_proj_fused_workspace_bytes(const mla_dims_t* dims, int32_t d_model, int64_t* bytes) {
  int st = check_dims(dims);
  if (st) return st;
  if (d_model < 1 || !bytes) return MLA_ERR_INVALID_ARG;
  if (!out_fused_supports(*dims, d_model)) return MLA_ERR_UNSUPPORTED;
  *bytes = out_fused_workspace_bytes(*dims, d_model);
  return MLA_OK;
}

int mla_out_proj_fused(const mla_dims_t* dims, int32_t d_model, const void* o_lat,
                       const void* w_fused, void* workspace, void* out, void* stream) {
  int st = check_dims(dims);
  if (st) return st;
  if (d_model < 1) return MLA_ERR_INVALID_ARG;
  if (!out_fused_supports(*dims, d_model)) return MLA_ERR_UNSUPPORTED;
  if (dims->batch == 0) return MLA_OK;
  if (!o_lat || !w_fused || !out) return MLA_ERR_INVALID_ARG;
  if (!workspace) return MLA_ERR_WORKSPACE;
  if (!aligned16(o_lat) || !aligned16(w_fused) || !aligned16(workspace) || !aligned16(out))
    return MLA_ERR_INVALID_ARG;
  (void)hipGetLastError();
  return launched(launch_out_fused(*dims, d_model, o_lat, w_fused, (float*)workspace, out,
                                   (hipStream_t)stream));
}

}  // extern "C"
