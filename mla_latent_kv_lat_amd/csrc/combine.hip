// Log-sum-exp merge of the split-K partials.  One wave per (sequence, query
// row); lanes stream the 512-wide partial rows (fp16, or fp32 for the fp32
// path) four elements at a time.
#include <hip/hip_runtime.h>
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace mla {

// four consecutive partial elements as floats (16-byte or 8-byte load)
template <typename PT> struct Load4;
template <> struct Load4<float> {
  __device__ static float4 run(const float* p) { return *(const float4*)p; }
};
template <> struct Load4<_Float16> {
  __device__ static float4 run(const _Float16* p) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    const h4 v = *(const h4*)p;
    return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
  }
};

// one 16-byte load of partial elements (4 fp32 or 8 fp16) as floats
template <typename PT> struct Load16;
template <> struct Load16<float> {
  static constexpr int kE = 4;
  __device__ static void run(const float* p, float (&o)[4]) {
    const float4 v = *(const float4*)p;
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
};
template <> struct Load16<_Float16> {
  static constexpr int kE = 8;
  __device__ static void run(const _Float16* p, float (&o)[8]) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const h8 v = *(const h8*)p;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (float)v[i];
  }
};

// kE consecutive outputs from floats: fp32 (4 -> 16 bytes) or bf16 (8 -> 16 bytes)
template <typename OT, int kE> struct StoreE;
template <int kE> struct StoreE<float, kE> {
  __device__ static void run(float* p, const float (&v)[kE]) {
#pragma unroll
    for (int i = 0; i < kE; i += 4) *(float4*)(p + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
  }
};
template <int kE> struct StoreE<uint16_t, kE> {
  __device__ static void run(uint16_t* p, const float (&v)[kE]) {
#pragma unroll
    for (int i = 0; i < kE; i += 4) {
      ushort4 r;
      r.x = f32_to_bf16(v[i]);
      r.y = f32_to_bf16(v[i + 1]);
      r.z = f32_to_bf16(v[i + 2]);
      r.w = f32_to_bf16(v[i + 3]);
      *(ushort4*)(p + i) = r;
    }
  }
};

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

// One wave per (sequence, query row).  The lanes first turn the partials'
// LSEs into normalised weights (one unit per lane, 64 at a time), then stream
// the 512-wide partial rows with 16-byte loads, keeping up to 8 units' loads
// in flight per lane.
template <typename PT, typename OT>
__global__ __launch_bounds__(256) void combine_kernel(int B, int R, int d_c, int G,
                                                      const int32_t* __restrict__ seq_lens,
                                                      const PT* __restrict__ o_part,
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

  // units touching b: u0..u1 (empty units hold no partial: weight 0)
  int64_t u0 = 0, u1 = -1;
  if (tb > 0) {
    u0 = unit_of_tile(pb, T, G);
    u1 = unit_of_tile(pb + tb - 1, T, G);
  }
  const int n = (int)(u1 - u0 + 1);
  auto live = [&](int64_t u) { return unit_begin(u, T, G) < unit_begin(u + 1, T, G); };

  // Fast path (at most 8 units, d_c <= 512): every load of the row -- the
  // partials and their LSEs -- is issued before any of them is needed; each
  // lane loads 16 bytes per partial per pass.
  constexpr int kU = 8, kE = Load16<PT>::kE, kC = 512 / (64 * kE);
  if (n <= kU && d_c <= 64 * kE * kC) {
    float v[kU][kC][kE];
    float lu = -INFINITY;  // lane k < n holds unit u0 + k's LSE
    if (lane < n && live(u0 + lane)) lu = lse_part[(u0 + lane + b) * R + row];
#pragma unroll
    for (int k = 0; k < kU; ++k) {
      const int64_t u = u0 + k;
      const bool ok = k < n && live(u);
#pragma unroll
      for (int j = 0; j < kC; ++j) {
        const int c = lane * kE + 64 * kE * j;
        if (ok && c < d_c) {
          Load16<PT>::run(o_part + ((u + b) * R + row) * d_c + c, v[k][j]);
        } else {
#pragma unroll
          for (int i = 0; i < kE; ++i) v[k][j][i] = 0.f;
        }
      }
    }
    const float mx = wave_max(lu);
    float acc[kC][kE];
#pragma unroll
    for (int j = 0; j < kC; ++j)
#pragma unroll
      for (int i = 0; i < kE; ++i) acc[j][i] = 0.f;
    float z = 1.f;
    if (mx != -INFINITY) {  // else no token seen: zero output
      const float el = lu == -INFINITY ? 0.f : expf(lu - mx);
      z = wave_sum(el);
      const float wl = el / z;
#pragma unroll
      for (int k = 0; k < kU; ++k) {
        const float w = __shfl(wl, k, 64);
#pragma unroll
        for (int j = 0; j < kC; ++j)
#pragma unroll
          for (int i = 0; i < kE; ++i) acc[j][i] = fmaf(w, v[k][j][i], acc[j][i]);
      }
    }
#pragma unroll
    for (int j = 0; j < kC; ++j) {
      const int c = lane * kE + 64 * kE * j;
      if (c < d_c) StoreE<OT, kE>::run(out + c, acc[j]);
    }
    if (lse_out && lane == 0)
      lse_out[(int64_t)b * R + row] = mx == -INFINITY ? -INFINITY : mx + logf(z);
    return;
  }

  // General path: many units or wide rows.
  float mx = -INFINITY;
  for (int k = lane; k < n; k += 64)
    if (live(u0 + k)) mx = fmaxf(mx, lse_part[(u0 + k + b) * R + row]);
  mx = wave_max(mx);
  if (mx == -INFINITY) {
    for (int c = lane * 4; c < d_c; c += 256) Store4<OT>::run(out + c, make_float4(0, 0, 0, 0));
    if (lse_out && lane == 0) lse_out[(int64_t)b * R + row] = -INFINITY;
    return;
  }
  float z = 0.f;
  for (int k = lane; k < n; k += 64)
    if (live(u0 + k)) z += expf(lse_part[(u0 + k + b) * R + row] - mx);
  z = wave_sum(z);
  const float inv_z = 1.f / z;
  for (int c0 = 0; c0 < d_c; c0 += 256 * kC) {
    float4 acc[kC];
#pragma unroll
    for (int j = 0; j < kC; ++j) acc[j] = make_float4(0, 0, 0, 0);
    for (int k0 = 0; k0 < n; k0 += 64) {
      float wl = 0.f;
      if (k0 + lane < n && live(u0 + k0 + lane))
        wl = expf(lse_part[(u0 + k0 + lane + b) * R + row] - mx) * inv_z;
      const int m = n - k0 < 64 ? n - k0 : 64;
      for (int k1 = 0; k1 < m; k1 += kU) {
        float4 v[kU][kC];
#pragma unroll
        for (int k2 = 0; k2 < kU; ++k2) {
          const int64_t u = u0 + k0 + k1 + k2;
          const bool ok = k1 + k2 < m && live(u);
#pragma unroll
          for (int j = 0; j < kC; ++j) {
            const int c = c0 + lane * 4 + 256 * j;
            v[k2][j] = (ok && c < d_c) ? Load4<PT>::run(o_part + ((u + b) * R + row) * d_c + c)
                                       : make_float4(0, 0, 0, 0);
          }
        }
#pragma unroll
        for (int k2 = 0; k2 < kU; ++k2) {
          const float w = __shfl(wl, k1 + k2, 64);
#pragma unroll
          for (int j = 0; j < kC; ++j) {
            acc[j].x = fmaf(w, v[k2][j].x, acc[j].x);
            acc[j].y = fmaf(w, v[k2][j].y, acc[j].y);
            acc[j].z = fmaf(w, v[k2][j].z, acc[j].z);
            acc[j].w = fmaf(w, v[k2][j].w, acc[j].w);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kC; ++j) {
      const int c = c0 + lane * 4 + 256 * j;
      if (c < d_c) Store4<OT>::run(out + c, acc[j]);
    }
  }
  if (lse_out && lane == 0) lse_out[(int64_t)b * R + row] = mx + logf(z);
}

hipError_t launch_combine(const mla_dims_t& d, int num_splits, const int32_t* seq_lens,
                          const void* o_part, const float* lse_part, void* o_lat,
                          float* lse_out, hipStream_t s) {
  const int R = d.q_len * d.heads;
  dim3 grid((unsigned)((R + 3) / 4), (unsigned)d.batch);
  if (d.q_dtype == MLA_F32)  // fp32 partials, fp32 output
    hipLaunchKernelGGL((combine_kernel<float, float>), grid, dim3(256), 0, s, d.batch, R,
                       d.d_latent, num_splits, seq_lens, (const float*)o_part, lse_part,
                       (float*)o_lat, lse_out);
  else  // fp16 partials, bf16 output
    hipLaunchKernelGGL((combine_kernel<_Float16, uint16_t>), grid, dim3(256), 0, s, d.batch, R,
                       d.d_latent, num_splits, seq_lens, (const _Float16*)o_part, lse_part,
                       (uint16_t*)o_lat, lse_out);
  return hipGetLastError();
}

}  // namespace mla
