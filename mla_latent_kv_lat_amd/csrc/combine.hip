// Log-sum-exp merge of the split-K partials.  One wave per (sequence, query
// row); lanes stream the 512-wide partial rows with 16-byte loads.
#include <hip/hip_runtime.h>
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace mla {

template <typename OT> struct Store4;
template <> struct Store4<float> {
  __device__ static void run(float* p, float4 v) { *(float4*)p = v; }
};
template <> struct Store4<uint16_t> {
  __device__ static void run(uint16_t* p, float4 v) {
    ushort4 r;
    r.x = f32_to_bf16(v.x);
    r.y = f32_to_bf16(v.y);
    r.z = f32_to_bf16(v.z);
    r.w = f32_to_bf16(v.w);
    *(ushort4*)p = r;
  }
};

template <typename OT>
__global__ __launch_bounds__(256) void combine_kernel(int B, int R, int d_c, int G,
                                                      const int32_t* __restrict__ seq_lens,
                                                      const float* __restrict__ o_part,
                                                      const float* __restrict__ lse_part,
                                                      OT* __restrict__ o_lat,
                                                      float* __restrict__ lse_out) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (row >= R) return;
  int64_t T, pb;
  wave_tile_sums(seq_lens, B, b, T, pb);
  const int64_t tb = tiles_of(seq_lens[b]);
  OT* out = o_lat + ((int64_t)b * R + row) * d_c;

  float mx = -INFINITY;
  int64_t u0 = 0, u1 = -1;
  if (tb > 0) {
    u0 = unit_of_tile(pb, T, G);
    u1 = unit_of_tile(pb + tb - 1, T, G);
    for (int64_t u = u0 + lane; u <= u1; u += 64)
      if (unit_begin(u, T, G) < unit_begin(u + 1, T, G))
        mx = fmaxf(mx, lse_part[(u + b) * R + row]);
    mx = wave_max(mx);
  }
  if (mx == -INFINITY) {  // no token seen: zero output
    for (int c = lane * 4; c < d_c; c += 256) Store4<OT>::run(out + c, make_float4(0, 0, 0, 0));
    if (lse_out && lane == 0) lse_out[(int64_t)b * R + row] = -INFINITY;
    return;
  }
  float z = 0.f;
  for (int64_t u = u0 + lane; u <= u1; u += 64)
    if (unit_begin(u, T, G) < unit_begin(u + 1, T, G))
      z += expf(lse_part[(u + b) * R + row] - mx);
  z = wave_sum(z);
  const float inv_z = 1.f / z;
  for (int c = lane * 4; c < d_c; c += 256) {
    float4 acc = make_float4(0, 0, 0, 0);
    for (int64_t u = u0; u <= u1; ++u) {
      if (!(unit_begin(u, T, G) < unit_begin(u + 1, T, G))) continue;
      const float w = expf(lse_part[(u + b) * R + row] - mx) * inv_z;
      const float4 v = *(const float4*)(o_part + ((u + b) * R + row) * d_c + c);
      acc.x = fmaf(w, v.x, acc.x);
      acc.y = fmaf(w, v.y, acc.y);
      acc.z = fmaf(w, v.z, acc.z);
      acc.w = fmaf(w, v.w, acc.w);
    }
    Store4<OT>::run(out + c, acc);
  }
  if (lse_out && lane == 0) lse_out[(int64_t)b * R + row] = mx + logf(z);
}

hipError_t launch_combine(const mla_dims_t& d, int num_splits, const int32_t* seq_lens,
                          const float* o_part, const float* lse_part, void* o_lat,
                          float* lse_out, hipStream_t s) {
  const int R = d.q_len * d.heads;
  dim3 grid((unsigned)((R + 3) / 4), (unsigned)d.batch);
  if (d.q_dtype == MLA_F32)
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, s, d.batch, R, d.d_latent,
                       num_splits, seq_lens, o_part, lse_part, (float*)o_lat, lse_out);
  else
    hipLaunchKernelGGL(combine_kernel<uint16_t>, grid, dim3(256), 0, s, d.batch, R, d.d_latent,
                       num_splits, seq_lens, o_part, lse_part, (uint16_t*)o_lat, lse_out);
  return hipGetLastError();
}

}  // namespace mla
