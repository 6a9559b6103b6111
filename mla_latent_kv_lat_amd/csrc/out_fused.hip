// MLA output-side absorption for gfx950 (bf16; d_latent = 512).
//
// Pages cited (title, section):
//   [ARCH] "Model Architecture Driving Inference Systems: From MHA/GQA to
//          DeepSeek MLA Matrix Absorption and Memory Minimalism" 3.2 (the
//          value up-projection folds into the output projection: the fused
//          weight of head i is W~_O,i = W_O,i W_UV,i, d x d_c, and the block
//          output is u_t = sum_i W~_O,i o~_{t,i}), 4.2 (the fusion is done
//          once, when the model is loaded)
//   [MATH] "Multi-Head Latent Attention (MLA): Mathematical Foundations,
//          Low-Rank KV Compression, Decoupled Rotary Positional Embeddings,
//          and Inference Matrix Absorption" (value output matrix absorption:
//          W_O = [W_O^1, ..., W_O^{n_h}], d x (n_h d_v))
//
// Two kernels, one per ABI call:
//
// fuse_out_kernel (load time): W~[n][i][c] = sum_j W_O[n][i d_v + j] W_UV[i][j][c],
//   one d x d_v by d_v x d_c product per head.  Not on the decode path: a
//   plain LDS-tiled fp32 SIMT product, 64 x 64 outputs per workgroup with
//   the whole K = d_v staged, rounded to bf16 once.
//
// out_fused_kernel + out_sum_kernel (decode): u[m][n] = sum_k o~[m][k] W~[n][k]
//   over k = (i, c), K = H d_c, for the M = B Lq query tokens.  Both operands
//   are K-contiguous rows, so the 32x32x16 bf16 MFMA operands come straight
//   from global memory (lane l: row l%32, 8 consecutive k).  The kernel
//   streams the fused weight, H x d x d_c bf16 (940 MB at H = 128,
//   d = 7168), once per 128 query rows; at decode sizes it is bound by that
//   stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_common.hpp"

namespace mla {
namespace {

using namespace mfma;

constexpr int kFoMaxDv = 128;

__global__ __launch_bounds__(256) void fuse_out_kernel(const uint16_t* __restrict__ w_o,
                                                       const uint16_t* __restrict__ w_uv,
                                                       uint16_t* __restrict__ w_f, int d_model, int H,
                                                       int d_v, int d_c) {
  __shared__ float As[64][kFoMaxDv + 1];  // W_O,i rows n0.., all d_v columns
  __shared__ float Bs[kFoMaxDv][64 + 1];  // W_UV,i all d_v rows, columns c0..
  const int c0 = blockIdx.x * 64, n0 = blockIdx.y * 64, i = blockIdx.z;
  const int tid = threadIdx.x;
  for (int e = tid; e < 64 * d_v; e += 256) {
    const int r = e / d_v, j = e - r * d_v;
    const int n = min(n0 + r, d_model - 1);
    As[r][j] = bf16_to_f32(w_o[(int64_t)n * H * d_v + (int64_t)i * d_v + j]);
  }
  for (int e = tid; e < d_v * 64; e += 256) {
    const int j = e >> 6, cc = e & 63;
    const int c = min(c0 + cc, d_c - 1);
    Bs[j][cc] = bf16_to_f32(w_uv[((int64_t)i * d_v + j) * d_c + c]);
  }
  __syncthreads();
  const int ty = tid >> 4, tx = tid & 15;  // outputs rows 4ty.., columns 4tx..
  float acc[4][4] = {};
  for (int j = 0; j < d_v; ++j) {
    float a[4], b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = As[4 * ty + r][j];
#pragma unroll
    for (int q = 0; q < 4; ++q) b[q] = Bs[j][4 * tx + q];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[r][q] = fmaf(a[r], b[q], acc[r][q]);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int n = n0 + 4 * ty + r;
    if (n >= d_model) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = c0 + 4 * tx + q;
      if (c < d_c) w_f[((int64_t)n * H + i) * d_c + c] = f32_to_bf16(acc[r][q]);
    }
  }
}

// K = H d_c is cut into kOfSplit chunks, one per XCD (workgroup id mod 8 is
// the XCD the dispatcher places it on), so a chunk's rows of o~ are fetched
// into that XCD's L2 once and shared by its workgroups.  Each workgroup
// owns 128 output features (32 per wave) of one chunk and writes fp32
// partial sums; out_sum_kernel adds the chunks in a fixed order.
constexpr int kOfSplit = 8;

// RT row tiles of 32 query rows per pass, PF k-steps of loads in flight.
template <int RT, int PF>
__global__ __launch_bounds__(256) void out_fused_kernel(const uint16_t* __restrict__ o_lat,
                                                        const uint16_t* __restrict__ w_f,
                                                        float* __restrict__ part, int M,
                                                        int d_model, int K) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int chunk = blockIdx.x & (kOfSplit - 1);
  const int n0 = (blockIdx.x / kOfSplit) * 128 + 32 * w;
  const int l32 = lane & 31, hk = lane >> 5;
  // features past the end re-read the last row (their results are not stored)
  const int n = min(n0 + l32, d_model - 1);
  const int kc = K / kOfSplit;  // a multiple of 16 (K = 512 H)
  const int steps = kc >> 4;
  // k-step s of the chunk: elements chunk kc + 16 s + 8 hk .. +7, i.e. the
  // 8-element unit kb + 2 s of a K-contiguous row
  const int kb = chunk * (kc >> 3) + hk;
  const bf16x8* brow = (const bf16x8*)(w_f + (int64_t)n * K) + kb;
  float* pout = part + (int64_t)chunk * M * d_model;
  for (int mg = blockIdx.y * 32 * RT; mg < M; mg += gridDim.y * 32 * RT) {
    const bf16x8* arow[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t)
      arow[t] = (const bf16x8*)(o_lat + (int64_t)min(mg + 32 * t + l32, M - 1) * K) + kb;
    bf16x8 a[PF][RT], b[PF];
#pragma unroll
    for (int d = 0; d < PF; ++d) {
      if (d < steps) {
        b[d] = brow[2 * d];
#pragma unroll
        for (int t = 0; t < RT; ++t) a[d][t] = arow[t][2 * d];
      }
    }
    f32x16 acc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) acc[t] = f32x16{};
    for (int s0 = 0; s0 < steps; s0 += PF) {
#pragma unroll
      for (int d = 0; d < PF; ++d) {
        if (s0 + d < steps) {
          const bf16x8 bv = b[d];
          bf16x8 av[RT];
#pragma unroll
          for (int t = 0; t < RT; ++t) av[t] = a[d][t];
          const int sn = s0 + d + PF;
          if (sn < steps) {
            b[d] = brow[2 * sn];
#pragma unroll
            for (int t = 0; t < RT; ++t) a[d][t] = arow[t][2 * sn];
          }
#pragma unroll
          for (int t = 0; t < RT; ++t) acc[t] = mfma32(av[t], bv, acc[t]);
        }
      }
    }
    // D (32 x 32) of row tile t: lane l holds feature n0 + l%32 and rows
    // mg + 32 t + 8(r/4) + 4(l/32) + r%4
    if (n0 + l32 < d_model) {
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = mg + 32 * t + 8 * (r >> 2) + 4 * hk + (r & 3);
          if (m < M) pout[(int64_t)m * d_model + n0 + l32] = acc[t][r];
        }
    }
  }
}

// out = bf16(sum over chunks 0..7 of part[chunk]), in that order.
__global__ __launch_bounds__(256) void out_sum_kernel(const float* __restrict__ part,
                                                      uint16_t* __restrict__ out, int64_t total) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    float v = part[i];
#pragma unroll
    for (int c = 1; c < kOfSplit; ++c) v += part[c * total + i];
    out[i] = f32_to_bf16(v);
  }
}

}  // namespace

bool out_fused_supports(const mla_dims_t& d, int d_model) {
  return d.q_dtype == MLA_BF16 && d.d_latent == 512 && d.d_v >= 1 && d.d_v <= kFoMaxDv &&
         d_model >= 1 && d_model <= 65536 && d.heads <= 1024 &&
         (int64_t)d.batch * d.q_len * d_model <= INT32_MAX;
}

hipError_t launch_fuse_out(const mla_dims_t& d, int d_model, const void* w_o, const void* w_uv,
                           void* w_fused, hipStream_t s) {
  dim3 grid((unsigned)((d.d_latent + 63) / 64), (unsigned)((d_model + 63) / 64), (unsigned)d.heads);
  hipLaunchKernelGGL(fuse_out_kernel, grid, dim3(256), 0, s, (const uint16_t*)w_o,
                     (const uint16_t*)w_uv, (uint16_t*)w_fused, d_model, d.heads, d.d_v, d.d_latent);
  return hipGetLastError();
}

int64_t out_fused_workspace_floats(const mla_dims_t& d, int d_model) {
  return (int64_t)kOfSplit * d.batch * d.q_len * d_model;
}

hipError_t launch_out_fused(const mla_dims_t& d, int d_model, const void* o_lat, const void* w_fused,
                            float* workspace, void* out, hipStream_t s) {
  const int M = d.batch * d.q_len, K = d.heads * d.d_latent;
  if (M == 0) return hipSuccess;
  const unsigned gx = (unsigned)(((d_model + 127) / 128) * kOfSplit);
  if (M <= 32) {
    hipLaunchKernelGGL((out_fused_kernel<1, 8>), dim3(gx), dim3(256), 0, s, (const uint16_t*)o_lat,
                       (const uint16_t*)w_fused, workspace, M, d_model, K);
  } else if (M <= 64) {
    hipLaunchKernelGGL((out_fused_kernel<2, 8>), dim3(gx), dim3(256), 0, s, (const uint16_t*)o_lat,
                       (const uint16_t*)w_fused, workspace, M, d_model, K);
  } else {
    // 128 rows per pass; passes beyond the grid's rows loop inside
    const unsigned gy = (unsigned)min((M + 127) / 128, 65535);
    hipLaunchKernelGGL((out_fused_kernel<4, 4>), dim3(gx, gy), dim3(256), 0, s,
                       (const uint16_t*)o_lat, (const uint16_t*)w_fused, workspace, M, d_model, K);
  }
  const int64_t total = (int64_t)M * d_model;
  const unsigned gs = (unsigned)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
  hipLaunchKernelGGL(out_sum_kernel, dim3(gs), dim3(256), 0, s, workspace, (uint16_t*)out, total);
  return hipGetLastError();
}

}  // namespace mla
