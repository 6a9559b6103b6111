// Matrix-core (MFMA) kernels for gfx950 around the attention: query
// absorption of W_UK with RoPE, and the W_UV output projection (bf16).
// The split-K decode itself lives in decode_split.hip.
//
// Pages cited (title, section):
//   [ARCH] "Model Architecture Driving Inference Systems: From MHA/GQA to
//          DeepSeek MLA Matrix Absorption and Memory Minimalism"
//   [MATH] "Multi-Head Latent Attention (MLA): Mathematical Foundations, ..."
//
// MFMA operand layouts used below (v_mfma_f32_32x32x16_bf16, wave64):
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) .. +7
//   B (16 x 32): lane l holds column l%32, k = 8*(l/32) .. +7
//   C (32 x 32): lane l holds column l%32, rows 8*(r/4) + 4*(l/32) + r%4
//
// ds_read_b64_tr_b16: in each group of 16 lanes, lane i names 4 consecutive
// 16-bit elements (row i/4, columns 4*(i%4)..+3 of a 4 x 16 block) and gets
// back column i of that block, rows 0..3.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_common.hpp"

namespace mla {
namespace {

using namespace mfma;

// ===================================================================== absorb
// q_abs[m, h, 0:d_c] = q_nope[m, h, :] W_UK[h]   ([ARCH] 3.1 absorbed query)
// One wave per (head, 128-column block).  The wave stages its 128 columns of
// W_UK[h] (d_n rows) in LDS with all loads in flight, then reads them back
// transposed as the MFMA B operand; q_nope rows are the A operand straight
// from memory.  The RoPE part (pair k turns by pos * base^(-2k/d_r), angle
// in fp64) is split over the head's column blocks by rows.
constexpr int kAbsCols = 128;
constexpr int kAbsPitch = 320;  // bytes per staged W row: 256 + 64 keeps tr reads conflict-free
constexpr int kAbsMaxDn = 128;

__global__ __launch_bounds__(64) void absorb_mfma_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
    const int32_t* __restrict__ positions, double rope_base, const uint16_t* __restrict__ w_uk,
    uint16_t* __restrict__ q_abs, int M, int H, int d_n, int d_r, int d_c) {
  __shared__ __attribute__((aligned(16))) char wsm[kAbsMaxDn * kAbsPitch];
  const int h = blockIdx.x;
  const int cb = blockIdx.y;
  const int lane = threadIdx.x;
  const int W = d_c + d_r;

  // stage W_UK[h][:, cb*128 .. +128]: lane reads chunk lane%16 of rows lane/16 + 4i
  const char* wsrc = (const char*)(w_uk + (int64_t)h * d_n * d_c + cb * kAbsCols);
  {
    // rows past d_n re-read the last row and land in LDS rows nobody reads
    uint4 st[kAbsMaxDn / 4];
#pragma unroll
    for (int i = 0; i < kAbsMaxDn / 4; ++i) {
      const int r = (lane >> 4) + 4 * i;
      const int rs = r < d_n ? r : d_n - 1;
      st[i] = *(const uint4*)(wsrc + (int64_t)rs * d_c * 2 + (lane & 15) * 16);
    }
#pragma unroll
    for (int i = 0; i < kAbsMaxDn / 4; ++i)
      *(uint4*)(wsm + ((lane >> 4) + 4 * i) * kAbsPitch + (lane & 15) * 16) = st[i];
  }
  __syncthreads();

  const int hf = lane >> 5, n32 = lane & 31;
  const int li = lane & 15, ch = (lane >> 4) & 1;
  constexpr int kK = kAbsMaxDn / 16;  // k-steps (rows past d_n are multiplied by zero A)
  for (int mb = 0; mb < M; mb += 64) {
    // all A loads of two 32-row blocks in flight at once
    bf16x8 av[2][kK];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int m = mb + 32 * t + n32;
#pragma unroll
      for (int k = 0; k < kK; ++k)
        av[t][k] = (m < M && 16 * k < d_n)
                       ? *(const bf16x8*)(q_nope + ((int64_t)m * H + h) * d_n + 16 * k + 8 * hf)
                       : bf16x8{};
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (mb + 32 * t >= M) break;
      f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
#pragma unroll
      for (int k = 0; k < kK; ++k) {
        if (16 * k >= d_n) break;
        const int r0 = 16 * k + 8 * hf + (li >> 2);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const uint32_t off0 = (uint32_t)(r0 * kAbsPitch + (nb * 32 + 16 * ch + 4 * (li & 3)) * 2);
          acc[nb] = mfma32(av[t][k], cat(lds_tr4(wsm, off0), lds_tr4(wsm, off0 + 4 * kAbsPitch)), acc[nb]);
        }
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int mr = mb + 32 * t + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (mr < M)
            q_abs[((int64_t)mr * H + h) * W + cb * kAbsCols + nb * 32 + n32] = f32_to_bf16(acc[nb][r]);
        }
    }
  }

  // RoPE of rows m = cb, cb + nblocks, ... of this head: lane -> (pair k, row
  // offset); d_r <= 128, so one pass covers 64 / (d_r/2) rows.
  const int half = d_r / 2;
  if (half > 0) {
    const int nblocks = gridDim.y;
    const int rows_per_pass = 64 / half;
    const int k = lane % half, rsub = lane / half;
    if (rsub < rows_per_pass) {
      const double theta = pow(rope_base, -2.0 * k / d_r);
      for (int m = cb + rsub * nblocks; m < M; m += rows_per_pass * nblocks) {
        double sn, cs;
        sincos((double)positions[m] * theta, &sn, &cs);
        const int64_t src = ((int64_t)m * H + h) * d_r + 2 * k;
        const float x0 = bf16_to_f32(q_rope[src]), x1 = bf16_to_f32(q_rope[src + 1]);
        const int64_t dst = ((int64_t)m * H + h) * W + d_c + 2 * k;
        q_abs[dst] = f32_to_bf16(x0 * (float)cs - x1 * (float)sn);
        q_abs[dst + 1] = f32_to_bf16(x0 * (float)sn + x1 * (float)cs);
      }
    }
  }
}

// =================================================================== out proj
// o[m, h, v] = sum_c W_UV[h][v][c] o_lat[m, h, c]   ([ARCH] 3.2)
// One workgroup per head, one wave per 32 output columns.  Both operands have
// the contracted latent index contiguous in memory, so they load straight
// into MFMA registers.  Each wave keeps its 32 rows of W_UV[h] in registers
// (512-wide latent: 32 steps of 16) and reuses them for every 32-row block.
constexpr int kOutMaxDc = 512;

__global__ __launch_bounds__(256) void out_proj_mfma_kernel(
    const uint16_t* __restrict__ o_lat, const uint16_t* __restrict__ w_uv,
    uint16_t* __restrict__ o, int M, int H, int d_c, int d_v) {
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63, hf = lane >> 5, n32 = lane & 31;
  const int vb = (blockIdx.y * 4 + (threadIdx.x >> 6)) * 32;
  if (vb >= d_v) return;
  const bf16x8* bp = (const bf16x8*)(w_uv + ((int64_t)h * d_v + vb + n32) * d_c);
  const int nk = d_c / 16;
  constexpr int kK = kOutMaxDc / 16;
  bf16x8 bw[kK];
#pragma unroll
  for (int k = 0; k < kK; ++k) bw[k] = k < nk ? bp[2 * k + hf] : bf16x8{};
  for (int mb = 0; mb < M; mb += 32) {
    const int m = mb + n32;
    const bf16x8* ap = (const bf16x8*)(o_lat + ((int64_t)(m < M ? m : 0) * H + h) * d_c);
    f32x16 acc = f32x16{};
    // the row block's A operand in two halves, each with all loads in flight
#pragma unroll
    for (int k0 = 0; k0 < kK; k0 += kK / 2) {
      bf16x8 av[kK / 2];
#pragma unroll
      for (int j = 0; j < kK / 2; ++j)
        av[j] = (k0 + j < nk && m < M) ? ap[2 * (k0 + j) + hf] : bf16x8{};
#pragma unroll
      for (int j = 0; j < kK / 2; ++j) acc = mfma32(av[j], bw[k0 + j], acc);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int mr = mb + 8 * (r >> 2) + 4 * hf + (r & 3);
      if (mr < M) o[((int64_t)mr * H + h) * d_v + vb + n32] = f32_to_bf16(acc[r]);
    }
  }
}

}  // namespace

// ================================================================= launchers

bool mfma_absorb_supports(const mla_dims_t& d) {
  return d.q_dtype == MLA_BF16 && d.d_nope % 16 == 0 && d.d_nope <= kAbsMaxDn &&
         d.d_latent % kAbsCols == 0 && d.d_rope <= 128;
}

hipError_t launch_absorb_mfma(const mla_dims_t& d, const void* q_nope, const void* q_rope,
                              const int32_t* positions, float rope_base, const void* w_uk,
                              void* q_abs, hipStream_t s) {
  const int M = d.batch * d.q_len;
  dim3 grid((unsigned)d.heads, (unsigned)(d.d_latent / kAbsCols));
  hipLaunchKernelGGL(absorb_mfma_kernel, grid, dim3(64), 0, s,
                     (const uint16_t*)q_nope, (const uint16_t*)q_rope, positions,
                     (double)rope_base, (const uint16_t*)w_uk, (uint16_t*)q_abs, M, d.heads,
                     d.d_nope, d.d_rope, d.d_latent);
  return hipGetLastError();
}

bool mfma_out_proj_supports(const mla_dims_t& d) {
  return d.q_dtype == MLA_BF16 && d.d_latent % 16 == 0 && d.d_latent <= kOutMaxDc &&
         d.d_v % 32 == 0;
}

hipError_t launch_out_proj_mfma(const mla_dims_t& d, const void* o_lat, const void* w_uv,
                                void* o, hipStream_t s) {
  const int M = d.batch * d.q_len;
  dim3 grid((unsigned)d.heads, (unsigned)((d.d_v / 32 + 3) / 4));
  hipLaunchKernelGGL(out_proj_mfma_kernel, grid, dim3(256), 0, s, (const uint16_t*)o_lat,
                     (const uint16_t*)w_uv, (uint16_t*)o, M, d.heads, d.d_latent, d.d_v);
  return hipGetLastError();
}

}  // namespace mla
