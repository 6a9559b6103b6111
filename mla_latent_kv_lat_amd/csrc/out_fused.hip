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
//   the whole K = d_v staged, rounded to bf16 once.  It writes the weight in
//   the order the projection's MFMAs consume it: 1 KB blocks of 32 features
//   x 16 consecutive k, 16 bytes per lane, so that every load of the
//   projection is one contiguous 1 KB and each wave streams a contiguous
//   range (rows of a plain [d, H d_c] layout are 2 H d_c bytes apart, and
//   32 of them per load instruction spread the stream thinly over memory).
//
// out_fused_kernel + out_sum_kernel (decode): u[m][n] = sum_k o~[m][k] W~[n][k]
//   over k = (i, c), K = H d_c, for the M = B Lq query tokens.  Both operands
//   are K-contiguous rows, so the 32x32x16 bf16 MFMA operands come straight
//   from global memory (lane l: row l%32, 8 consecutive k; the weight's
//   from its packed blocks, read non-temporally).  The kernel
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
  // packed store: element (n, k = i d_c + c) of the [d, H d_c] product goes to
  // 1 KB block (n / 32, k / 16), lane 32 ((k % 16) / 8) + n % 32, slot k % 8;
  // rows from d_model up to the next multiple of 32 are zero
  const int64_t ksteps = (int64_t)H * d_c / 16;
  const int npad = (d_model + 31) & ~31;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int n = n0 + 4 * ty + r;
    if (n >= npad) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = c0 + 4 * tx + q;
      if (c >= d_c) continue;
      const int64_t k = (int64_t)i * d_c + c;
      const int64_t off = (((int64_t)(n >> 5) * ksteps + (k >> 4)) * 64 + ((k >> 3) & 1) * 32 +
                           (n & 31)) * 8 + (k & 7);
      w_f[off] = n < d_model ? f32_to_bf16(acc[r][q]) : (uint16_t)0;
    }
  }
}

constexpr int kOfSplit = 8;

// A workgroup (4 waves) owns 64 FT features of one chunk: wave w takes the
// FT 32-feature blocks of group w & 1 and half w >> 1 of the chunk's k-steps
// (the halves are added through LDS), RT row tiles of 32 query rows per
// pass and PF k-steps of loads in flight.  Each k-step loads RT tiles of o~
// and FT blocks of the weight for RT x FT MFMAs.
template <int RT, int FT, int PF>
__global__ __launch_bounds__(256, 2) void out_fused_kernel(const uint16_t* __restrict__ a_pk,
                                                        const uint16_t* __restrict__ w_f,
                                                        float* __restrict__ part, int M,
                                                        int d_model, int K) {
  static_assert(RT * FT <= 8, "LDS holds eight accumulators per lane");
  __shared__ f32x16 red[2][8][64];  // half 1's accumulators, per feature group
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int fg = w & 1, kh = w >> 1;
  const int chunk = blockIdx.x & (kOfSplit - 1);
  const int nbase = (blockIdx.x / kOfSplit) * 2 * FT + fg * FT;  // first 32-feature block
  const int nblocks = (d_model + 31) >> 5;
  const int l32 = lane & 31, hk = lane >> 5;
  const int kc = K / kOfSplit;  // a multiple of 64 (K = 512 H)
  const int steps = kc >> 5;    // per half
  // k-step s of this half is k-step chunk kc/16 + kh steps + s of K; both
  // operands are packed in 1 KB blocks per (32-row tile, k-step), lane l's
  // 16 bytes holding row l%32, k 16 s + 8 (l/32) .. +7
  const int64_t sbase = (int64_t)chunk * (kc >> 4) + kh * steps;
  const int ntiles = (M + 31) >> 5;
  const bf16x8* brow[FT];
#pragma unroll
  for (int f = 0; f < FT; ++f) {
    // blocks past the last (their results are not stored) re-read the last one
    const int nbl = min(nbase + f, nblocks - 1);
    brow[f] = (const bf16x8*)w_f + ((int64_t)nbl * (K >> 4) + sbase) * 64 + lane;
  }
  float* pout = part + (int64_t)chunk * M * d_model;
  for (int mg = blockIdx.y * 32 * RT; mg < M; mg += gridDim.y * 32 * RT) {
    const bf16x8* arow[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      // tiles past the last (their results are not stored) re-read the last one
      const int tile = min((mg >> 5) + t, ntiles - 1);
      arow[t] = (const bf16x8*)a_pk + ((int64_t)tile * (K >> 4) + sbase) * 64 + lane;
    }
    bf16x8 a[PF][RT], b[PF][FT];
#pragma unroll
    for (int d = 0; d < PF; ++d) {
      if (d < steps) {
#pragma unroll
        for (int f = 0; f < FT; ++f) b[d][f] = __builtin_nontemporal_load(brow[f] + 64 * d);
#pragma unroll
        for (int t = 0; t < RT; ++t) a[d][t] = arow[t][64 * d];
      }
    }
    f32x16 acc[RT][FT];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int f = 0; f < FT; ++f) acc[t][f] = f32x16{};
    for (int s0 = 0; s0 < steps; s0 += PF) {
#pragma unroll
      for (int d = 0; d < PF; ++d) {
        if (s0 + d < steps) {
          bf16x8 av[RT], bv[FT];
#pragma unroll
          for (int t = 0; t < RT; ++t) av[t] = a[d][t];
#pragma unroll
          for (int f = 0; f < FT; ++f) bv[f] = b[d][f];
          const int sn = s0 + d + PF;
          if (sn < steps) {
#pragma unroll
            for (int f = 0; f < FT; ++f) b[d][f] = __builtin_nontemporal_load(brow[f] + 64 * sn);
#pragma unroll
            for (int t = 0; t < RT; ++t) a[d][t] = arow[t][64 * sn];
          }
#pragma unroll
          for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int f = 0; f < FT; ++f) acc[t][f] = mfma32(av[t], bv[f], acc[t][f]);
        }
      }
    }
    if (kh == 1) {
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int f = 0; f < FT; ++f) red[fg][t * FT + f][lane] = acc[t][f];
    }
    __syncthreads();
    if (kh == 0) {
      // D (32 x 32) of (row tile t, block f): lane l holds feature
      // 32 (nbase + f) + l%32 and rows mg + 32 t + 8(r/4) + 4(l/32) + r%4
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int f = 0; f < FT; ++f) {
          const f32x16 v = acc[t][f] + red[fg][t * FT + f][lane];
          const int n = 32 * (nbase + f) + l32;
          if (n >= d_model) continue;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int m = mg + 32 * t + 8 * (r >> 2) + 4 * hk + (r & 3);
            if (m < M) pout[(int64_t)m * d_model + n] = v[r];
          }
        }
    }
    __syncthreads();  // red is free for the next pass
  }
}

// o~ [M, K] into the operand blocks out_fused_kernel reads: 16-byte unit
// (tile, s, l) holds row 32 tile + l%32, k 16 s + 8 (l/32) .. +7; rows from
// M up to the next multiple of 32 are zero.
__global__ __launch_bounds__(256) void pack_rows_kernel(const uint16_t* __restrict__ o_lat,
                                                        bf16x8* __restrict__ a_pk, int M, int K,
                                                        int64_t units) {
  const int ks = K >> 4;
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * 256) {
    const int l = (int)(u & 63);
    const int64_t ts = u >> 6;
    const int64_t tile = ts / ks;
    const int st = (int)(ts - tile * ks);
    const int64_t m = tile * 32 + (l & 31);
    bf16x8 v = bf16x8{};
    if (m < M) v = *(const bf16x8*)(o_lat + m * K + 16 * st + 8 * (l >> 5));
    a_pk[u] = v;
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

int64_t fused_out_weight_elems(const mla_dims_t& d, int d_model) {
  return (int64_t)((d_model + 31) / 32) * 32 * d.heads * d.d_latent;
}

// workspace: kOfSplit partial sums [M, d] (fp32), then the packed o~
// (ceil(M/32) 32 x K bf16)
int64_t out_fused_workspace_bytes(const mla_dims_t& d, int d_model) {
  const int64_t M = (int64_t)d.batch * d.q_len;
  return (int64_t)kOfSplit * M * d_model * 4 + (M + 31) / 32 * 32 * d.heads * d.d_latent * 2;
}

hipError_t launch_out_fused(const mla_dims_t& d, int d_model, const void* o_lat, const void* w_fused,
                            float* workspace, void* out, hipStream_t s) {
  const int M = d.batch * d.q_len, K = d.heads * d.d_latent;
  if (M == 0) return hipSuccess;
  const int nblocks = (d_model + 31) / 32;
  bf16x8* apk = (bf16x8*)(workspace + (int64_t)kOfSplit * M * d_model);
  const int64_t units = (int64_t)(M + 31) / 32 * 32 * K / 8;
  const unsigned gp = (unsigned)((units + 255) / 256 < 2048 ? (units + 255) / 256 : 2048);
  hipLaunchKernelGGL(pack_rows_kernel, dim3(gp), dim3(256), 0, s, (const uint16_t*)o_lat, apk, M, K,
                     units);
  const uint16_t* a = (const uint16_t*)apk;
  const uint16_t* w = (const uint16_t*)w_fused;
  if (M <= 32) {
    const unsigned gx = (unsigned)((nblocks + 3) / 4 * kOfSplit);
    hipLaunchKernelGGL((out_fused_kernel<1, 2, 4>), dim3(gx), dim3(256), 0, s, a, w, workspace, M,
                       d_model, K);
  } else if (M <= 64) {
    const unsigned gx = (unsigned)((nblocks + 3) / 4 * kOfSplit);
    hipLaunchKernelGGL((out_fused_kernel<2, 2, 4>), dim3(gx), dim3(256), 0, s, a, w, workspace, M,
                       d_model, K);
  } else {
    // 128 rows per pass; passes beyond the grid's rows loop inside
    const unsigned gx = (unsigned)((nblocks + 3) / 4 * kOfSplit);
    const unsigned gy = (unsigned)min((M + 127) / 128, 65535);
    hipLaunchKernelGGL((out_fused_kernel<4, 2, 2>), dim3(gx, gy), dim3(256), 0, s, a, w, workspace,
                       M, d_model, K);
  }
  const int64_t total = (int64_t)M * d_model;
  const unsigned gs = (unsigned)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
  hipLaunchKernelGGL(out_sum_kernel, dim3(gs), dim3(256), 0, s, workspace, (uint16_t*)out, total);
  return hipGetLastError();
}

}  // namespace mla
