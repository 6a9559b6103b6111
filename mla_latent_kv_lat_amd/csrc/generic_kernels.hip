// Plain SIMT kernels for every step of the decode path, for any widths and
// element types.  They serve the fp32 workloads and any shape the MFMA
// kernels are not built for, and give a second GPU implementation to test
// the MFMA kernels against.  Pages: see include/mla.h.
#include <hip/hip_runtime.h>
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace mla {

// ------------------------------------------------------------ absorb + RoPE
// One block per query row (b, i, h); threads over latent columns, then over
// RoPE pairs.  q_lat[c] = sum_d w_uk[h][d][c] q_nope[d]   (key absorption:
// the content key W_UK c is never formed, its transpose moves to the query).
// T: inputs (fp32 or bf16 bits); QA: q_abs (fp32, or fp16 for bf16 inputs).
template <typename T, typename QA>
__global__ __launch_bounds__(256) void absorb_generic_kernel(
    const T* __restrict__ q_nope, const T* __restrict__ q_rope,
    const int32_t* __restrict__ positions, double rope_base, const T* __restrict__ w_uk,
    QA* __restrict__ q_abs, int H, int d_n, int d_r, int d_c) {
  const int64_t row = blockIdx.x;  // ((b*Lq)+i)*H + h
  const int h = (int)(row % H);
  const int64_t bi = row / H;
  const int W = d_c + d_r;
  for (int c = threadIdx.x; c < d_c; c += blockDim.x) {
    float acc = 0.f;
    for (int d = 0; d < d_n; ++d)
      acc = fmaf(Elem<T>::load(q_nope, row * d_n + d),
                 Elem<T>::load(w_uk, ((int64_t)h * d_n + d) * d_c + c), acc);
    Elem<QA>::store(q_abs, row * W + c, acc);
  }
  // RoPE: pair k turns by pos * base^(-2k/d_r); angle and its sine/cosine in fp64.
  const double pos = (double)positions[bi];
  for (int k = threadIdx.x; k < d_r / 2; k += blockDim.x) {
    const double ang = pos * pow(rope_base, -2.0 * k / d_r);
    double s, c;
    sincos(ang, &s, &c);
    const float x0 = Elem<T>::load(q_rope, row * d_r + 2 * k);
    const float x1 = Elem<T>::load(q_rope, row * d_r + 2 * k + 1);
    const float cs = (float)c, sn = (float)s;
    Elem<QA>::store(q_abs, row * W + d_c + 2 * k, x0 * cs - x1 * sn);
    Elem<QA>::store(q_abs, row * W + d_c + 2 * k + 1, x0 * sn + x1 * cs);
  }
}

// ------------------------------------------------------------- decode
// One wave per query row and unit; 4 waves per block.  Per 64-token tile:
// each token's score is a wave-wide dot product over the 576-wide row, the
// tile's softmax is folded into a running (max, sum, accumulator), and the
// accumulator gathers the weighted raw latents.
constexpr int kGenMaxW = 1280;   // max d_latent + d_rope
constexpr int kGenMaxC = 1024;   // max d_latent

template <typename QT, typename KT>
__global__ __launch_bounds__(256) void decode_generic_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int R = a.q_len * a.heads;
  const int64_t u = blockIdx.x;
  if (row >= R) return;
  int64_t T, unused;
  wave_tile_sums(a.seq_lens, a.batch, 0, T, unused);
  const int64_t x0 = unit_begin(u, T, a.num_splits);
  const int64_t x1 = unit_begin(u + 1, T, a.num_splits);
  if (x0 >= x1) return;
  const int i = row / a.heads;
  const int W = a.d_c + a.d_r;
  const QT* q_abs = (const QT*)a.q_abs;
  const KT* lat = (const KT*)a.latent;
  const KT* rope = (const KT*)a.rope;

  int b;
  int64_t pb;
  find_sequence(a.seq_lens, a.batch, x0, b, pb);
  int64_t x = x0;
  while (x < x1 && b < a.batch) {
    const int len = a.seq_lens[b];
    const int64_t tb = tiles_of(len);
    if (tb == 0) { ++b; continue; }
    const int64_t seg_end = x1 < pb + tb ? x1 : pb + tb;
    int n_vis = a.causal ? len - a.q_len + i + 1 : len;
    if (n_vis < 0) n_vis = 0;

    float q[kGenMaxW / 64];
    const int64_t qrow = ((int64_t)b * a.q_len + i) * a.heads + (row % a.heads);
#pragma unroll
    for (int k = 0; k < kGenMaxW / 64; ++k) {
      const int c = lane + 64 * k;
      q[k] = c < W ? Elem<QT>::load(q_abs, qrow * W + c) : 0.f;
    }
    float acc[kGenMaxC / 64];
#pragma unroll
    for (int k = 0; k < kGenMaxC / 64; ++k) acc[k] = 0.f;
    float m = -INFINITY, l = 0.f;

    for (int64_t xt = x; xt < seg_end; ++xt) {
      const int t0 = (int)(xt - pb) * kTile;
      if (t0 >= n_vis) break;
      const int tn = n_vis - t0 < kTile ? n_vis - t0 : kTile;
      float s_mine = -INFINITY;
      for (int j = 0; j < tn; ++j) {
        const int64_t r = cache_row(b, t0 + j, a.block_table, a.mbps, a.max_seq_len);
        const float sc = a.kv_scale ? a.kv_scale[r] : 1.f;
        float part = 0.f;
#pragma unroll
        for (int k = 0; k < kGenMaxW / 64; ++k) {
          const int c = lane + 64 * k;
          if (c < a.d_c)
            part = fmaf(q[k], Elem<KT>::load(lat, r * a.row_stride + c), part);
          else if (c < W)
            part = fmaf(q[k], Elem<KT>::load(rope, r * a.row_stride + (c - a.d_c)), part);
        }
        const float s = wave_sum(part) * sc * a.softmax_scale;
        if (lane == j) s_mine = s;
      }
      const float m_new = fmaxf(m, wave_max(s_mine));
      const float alpha = expf(m - m_new);  // m = -inf -> 0
      const float p_mine = lane < tn ? expf(s_mine - m_new) : 0.f;
      l = l * alpha + wave_sum(p_mine);
#pragma unroll
      for (int k = 0; k < kGenMaxC / 64; ++k) acc[k] *= alpha;
      for (int j = 0; j < tn; ++j) {
        const int64_t r = cache_row(b, t0 + j, a.block_table, a.mbps, a.max_seq_len);
        const float p = __shfl(p_mine, j, 64) * (a.kv_scale ? a.kv_scale[r] : 1.f);
#pragma unroll
        for (int k = 0; k < kGenMaxC / 64; ++k) {
          const int c = lane + 64 * k;
          if (c < a.d_c) acc[k] = fmaf(p, Elem<KT>::load(lat, r * a.row_stride + c), acc[k]);
        }
      }
      m = m_new;
    }
    const int64_t slot = u + b;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t ob = (slot * R + row) * a.d_c;
#pragma unroll
    for (int k = 0; k < kGenMaxC / 64; ++k) {
      const int c = lane + 64 * k;
      if (c < a.d_c) {
        if (a.part_f16)
          ((_Float16*)a.o_part)[ob + c] = (_Float16)(acc[k] * inv);
        else
          ((float*)a.o_part)[ob + c] = acc[k] * inv;
      }
    }
    if (lane == 0) a.lse_part[slot * R + row] = l > 0.f ? m + logf(l) : -INFINITY;
    x = seg_end;
    pb += tb;
    ++b;
  }
}

// --------------------------------------------------------------- out proj
// o[row][v] = sum_c w_uv[h][v][c] o_lat[row][c]; one block per row.
template <typename T>
__global__ __launch_bounds__(256) void out_proj_generic_kernel(
    const T* __restrict__ o_lat, const T* __restrict__ w_uv, T* __restrict__ o, int H, int d_c,
    int d_v) {
  const int64_t row = blockIdx.x;
  const int h = (int)(row % H);
  for (int v = threadIdx.x; v < d_v; v += blockDim.x) {
    float acc = 0.f;
    for (int c = 0; c < d_c; ++c)
      acc = fmaf(Elem<T>::load(w_uv, ((int64_t)h * d_v + v) * d_c + c),
                 Elem<T>::load(o_lat, row * d_c + c), acc);
    Elem<T>::store(o, row * d_v + v, acc);
  }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_absorb_generic(const mla_dims_t& d, const void* q_nope, const void* q_rope,
                                 const int32_t* positions, float rope_base, const void* w_uk,
                                 void* q_abs, hipStream_t s) {
  const int64_t rows = (int64_t)d.batch * d.q_len * d.heads;
  if (d.q_dtype == MLA_F32)
    hipLaunchKernelGGL((absorb_generic_kernel<float, float>), dim3((unsigned)rows), dim3(256), 0, s,
                       (const float*)q_nope, (const float*)q_rope, positions, (double)rope_base,
                       (const float*)w_uk, (float*)q_abs, d.heads, d.d_nope, d.d_rope,
                       d.d_latent);
  else
    hipLaunchKernelGGL((absorb_generic_kernel<uint16_t, _Float16>), dim3((unsigned)rows), dim3(256),
                       0, s, (const uint16_t*)q_nope, (const uint16_t*)q_rope, positions,
                       (double)rope_base, (const uint16_t*)w_uk, (_Float16*)q_abs, d.heads,
                       d.d_nope, d.d_rope, d.d_latent);
  return hipGetLastError();
}

bool generic_decode_supports(const mla_dims_t& d) {
  return d.d_latent + d.d_rope <= kGenMaxW && d.d_latent <= kGenMaxC;
}

hipError_t launch_decode_generic(const mla_dims_t& d, const DecodeArgs& a, hipStream_t s) {
  const int R = d.q_len * d.heads;
  dim3 grid((unsigned)a.num_splits, (unsigned)((R + 3) / 4));
  if (d.q_dtype == MLA_F32)
    hipLaunchKernelGGL((decode_generic_kernel<float, float>), grid, dim3(256), 0, s, a);
  else if (d.kv_dtype == MLA_BF16)  // fp16 absorbed query, bf16 cache
    hipLaunchKernelGGL((decode_generic_kernel<_Float16, uint16_t>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_generic_kernel<_Float16, uint8_t>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_out_proj_generic(const mla_dims_t& d, const void* o_lat, const void* w_uv,
                                   void* o, hipStream_t s) {
  const int64_t rows = (int64_t)d.batch * d.q_len * d.heads;
  if (d.q_dtype == MLA_F32)
    hipLaunchKernelGGL(out_proj_generic_kernel<float>, dim3((unsigned)rows), dim3(256), 0, s,
                       (const float*)o_lat, (const float*)w_uv, (float*)o, d.heads, d.d_latent,
                       d.d_v);
  else
    hipLaunchKernelGGL(out_proj_generic_kernel<uint16_t>, dim3((unsigned)rows), dim3(256), 0, s,
                       (const uint16_t*)o_lat, (const uint16_t*)w_uv, (uint16_t*)o, d.heads,
                       d.d_latent, d.d_v);
  return hipGetLastError();
}

}  // namespace mla
