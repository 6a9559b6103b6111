// Fused log-sum-exp combine and W_UV projection for gfx950 (bf16 queries,
// fp16 partials, latent 512).
//
// Pages cited (title, section):
//   [ARCH] "Model Architecture Driving Inference Systems: From MHA/GQA to
//          DeepSeek MLA Matrix Absorption and Memory Minimalism"
//   [MATH] "Multi-Head Latent Attention (MLA): Mathematical Foundations, ..."
//
// One workgroup of 8 waves per (head h, 32 or 64 query rows m = (b, i));
// wave w owns rows w, w + 8, w + 16, ... in phases 0-1:
//   phase 0  each wave on its own: the split-K units that touched each of
//            its rows' sequence b (a lane scan over seq_lens, whose load is
//            the kernel's first), then the log-sum-exp of their partials,
//            lse = log sum_u exp(lse_u); lane k of the wave keeps the weight
//            exp(lse_u - lse) of the row's k-th unit;
//   phase 1  o_lat = sum_u exp(lse_u - lse) o_u ([MATH] value absorption:
//            softmax weights on the cached latents), rounded to bf16 into an
//            LDS tile (and to memory when asked for).  The partial loads of
//            all four rows are issued together with their LSE loads, so a
//            row spanning up to kCPChunk units costs one memory round trip
//            after the one for seq_lens; W_UV streams in meanwhile;
//   phase 2  o = o_lat W_UV[h]^T on v_mfma_f32_32x32x16_bf16 ([ARCH] 3.2):
//            wave w takes the 32 v-columns 32 (w & 3) + 128 j and half w >> 2
//            of the 512 latent columns, with its rows of W_UV[h] loaded into
//            registers early; the two halves meet in LDS.  When two
//            workgroups share a head (all rows in one block), each takes two
//            of every four 32-column blocks and a wave a quarter of the
//            latent columns; the four quarters meet in LDS.
// The latent output never makes an HBM round trip between the two steps.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_common.hpp"

namespace mla {
namespace {

using namespace mfma;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kCPWaves = 8;
constexpr int kCPPitch = 1040;  // bytes per bf16 o_lat row in LDS: 1024 + 16 (conflict-free A reads)
constexpr int kCPChunk = 4;     // partials per row loaded per pass

__device__ inline float lane_value(float v, int k) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), k));
}
__device__ inline int64_t lane_i64(int64_t v, int k) {  // k wave-uniform
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, k);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), k);
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ROWS query rows per workgroup; VS workgroups (blockIdx.z = vpart) share a head's
// v-columns when one row block holds every row, so that W_UV[h] is pulled
// into VS CUs in parts instead of into one CU whole.  Each of them combines
// the same rows (the partials are read VS times).
template <int ROWS, int VS>
__global__ __launch_bounds__(512) void combine_proj_kernel(
    int B, int Lq, int H, int G, const int32_t* __restrict__ seq_lens,
    const _Float16* __restrict__ o_part, const float* __restrict__ lse_part,
    const uint16_t* __restrict__ w_uv, int d_v, uint16_t* __restrict__ o,
    float* __restrict__ lse_out, uint16_t* __restrict__ o_lat) {
  __shared__ __attribute__((aligned(16))) char lat[ROWS * kCPPitch];
  // v-column blocks per pass and latent parts per block: 4 x 2 or 2 x 4 waves
  constexpr int kNC = 4 / VS, kNK = kCPWaves / kNC, kSteps = 32 / kNK;
  __shared__ __attribute__((aligned(16))) float red[(kNK - 1) * kNC * 64 * 16];

  constexpr int kRowsPerWave = ROWS / kCPWaves;
  const int h = blockIdx.x;
  const int M = B * Lq, R = Lq * H;
  const int mb0 = blockIdx.y * ROWS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int vpart = blockIdx.z;  // which of the VS workgroups of this head
  const int cq = w % kNC, kh = w / kNC;
  const int hf = lane >> 5, n32 = lane & 31;

  // ---- phase 0, by every wave for its own rows (no barrier): the lengths
  // of the first 64 sequences load first.  With 32 rows W_UV[h] rows
  // 32 (kNC vpart + cq) + n32 of latent part kh stream in behind them; with
  // 64 rows the partials are twice the bytes and go first (measured 30.0
  // against 34.2 us at 128 rows).
  constexpr bool kWeightsFirst = ROWS <= 32;
  const int len0 = seq_lens[lane < B ? lane : B - 1];
  __builtin_amdgcn_sched_barrier(0);  // the load above stays ahead of the weights: its wait leaves them in flight
  bf16x8 bw[kSteps];
  auto load_w = [&]() {
    const int vb = 32 * (kNC * vpart + cq);
    const bf16x8* bp = (const bf16x8*)(w_uv + ((int64_t)h * d_v + (vb < d_v ? vb : 0) + n32) * 512);
#pragma unroll
    for (int k = 0; k < kSteps; ++k) bw[k] = bp[2 * (kSteps * kh + k) + hf];
  };
  if (kWeightsFirst) load_w();
  // total tiles T, and in lane i < kRowsPerWave the first tile pb and tile
  // count tb of the sequence of this wave's row i (a lane scan per 64
  // sequences); the rows' unit arithmetic below then runs once, in lanes
  const int m_l = mb0 + w + kCPWaves * (lane < kRowsPerWave ? lane : 0);
  const int b_l = (m_l < M ? m_l : M - 1) / Lq;
  int64_t pb_l = 0, tb_l = 0, T = 0;
  auto scan_chunk = [&](int c0, int len) {  // sequences c0 .. c0 + 63, lane bb - c0 holds len(bb)
    const int64_t t = c0 + lane < B ? tiles_of(len) : 0;
    int64_t incl = t;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t x = __shfl_up(incl, d, 64);
      if (lane >= d) incl += x;
    }
    const int src = b_l - c0;
    const int64_t e = __shfl(incl - t, src & 63, 64), tt = __shfl(t, src & 63, 64);
    if (src >= 0 && src < 64) {
      pb_l = T + e;
      tb_l = tt;
    }
    T += lane_i64(incl, 63);
  };
  scan_chunk(0, len0);
  for (int c0 = 64; c0 < B; c0 += 64) scan_chunk(c0, seq_lens[c0 + lane < B ? c0 + lane : B - 1]);
  // with G <= T no unit is empty
  const bool may_be_empty = G > T;
  const bool small = T * (int64_t)G < ((int64_t)1 << 32);
  auto nonempty = [&](int64_t u) -> bool {
    if (!may_be_empty) return true;
    return small ? ((uint32_t)u * (uint32_t)T) / (uint32_t)G <
                       ((uint32_t)u * (uint32_t)T + (uint32_t)T) / (uint32_t)G
                 : unit_begin(u, T, G) < unit_begin(u + 1, T, G);
  };
  auto unit_of = [&](int64_t x) -> int64_t {  // unit holding tile x
    return small ? (int64_t)(((uint32_t)x * (uint32_t)G + (uint32_t)G - 1u) / (uint32_t)T)
                 : unit_of_tile(x, T, G);
  };
  // lane i: row i's first unit u0, unit count n and first partial slot
  // (u0 + b) R + r
  int64_t u0_l = 0;
  int n_l = 0;
  if (m_l < M && tb_l > 0) {
    u0_l = unit_of(pb_l);
    n_l = (int)(unit_of(pb_l + tb_l - 1) - u0_l + 1);
  }
  const int64_t slot_l = (u0_l + b_l) * R + (m_l < M ? (m_l % Lq) * H + h : h);

  // ---- the rows' LSEs and first kCPChunk partials.  The partial loads are
  // buffer loads bounded to the row's units: a chunk past them reads zeros
  // without touching memory (the kernel is bound by the bytes each CU pulls
  // in), and no branch splits the loads
  const int c = 8 * lane;  // latent columns of this lane in phase 1
  int64_t u0[kRowsPerWave], slot0[kRowsPerWave];
  int n[kRowsPerWave];
  float lv[kRowsPerWave];
  h8 v[kRowsPerWave][kCPChunk];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    u0[i] = lane_i64(u0_l, i);
    n[i] = __builtin_amdgcn_readlane(n_l, i);
    slot0[i] = lane_i64(slot_l, i);
    lv[i] = lse_part[slot0[i] + (int64_t)(lane < n[i] ? lane : 0) * R];
    const int nk = n[i] < kCPChunk ? n[i] : kCPChunk;
    const __amdgpu_buffer_rsrc_t rs =
        buffer_rsrc((void*)(o_part + slot0[i] * 512), nk > 0 ? ((uint32_t)(nk - 1) * (uint32_t)R + 1u) * 1024u : 0u);
#pragma unroll
    for (int k = 0; k < kCPChunk; ++k)
      v[i][k] = __builtin_bit_cast(h8, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs, (int)((uint32_t)k * (uint32_t)R * 1024u + 2u * c), 0, 0));
  }
  if (!kWeightsFirst) load_w();

  // ---- phase 0c / 1: LSE, weights, weighted sum of the partials
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int j = w + kCPWaves * i, m = mb0 + j;
    const int ni = n[i];
    // empty units wrote no partial (weight 0); a row may span more than 64 units
    const bool ne = lane < ni && nonempty(u0[i] + lane);
    const float x = ne ? lv[i] : -INFINITY;
    float mx = x;
    for (int k = lane + 64; k < ni; k += 64)
      if (nonempty(u0[i] + k))
        mx = fmaxf(mx, lse_part[slot0[i] + (int64_t)k * R]);
    mx = wave_max(mx);
    float z = (mx != -INFINITY && x != -INFINITY) ? expf(x - mx) : 0.f;
    if (mx != -INFINITY)
      for (int k = lane + 64; k < ni; k += 64)
        if (nonempty(u0[i] + k))
          z += expf(lse_part[slot0[i] + (int64_t)k * R] - mx);
    z = wave_sum(z);
    const float lse = mx == -INFINITY ? -INFINITY : mx + logf(z);
    const float wt = (lse != -INFINITY && x != -INFINITY) ? expf(x - lse) : 0.f;
    if (lse_out && vpart == 0 && m < M && lane == 0) lse_out[(int64_t)m * H + h] = lse;

    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int k = 0; k < kCPChunk; ++k) {
      const float wk = k < ni ? lane_value(wt, k) : 0.f;
      if (wk != 0.f)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(wk, (float)v[i][k][e], acc[e]);
    }
    for (int k0 = kCPChunk; k0 < ni; k0 += kCPChunk) {  // rows spanning more units
      h8 vv[kCPChunk];
      float wv[kCPChunk];
#pragma unroll
      for (int k = 0; k < kCPChunk; ++k) {
        const int kk = k0 + k;
        float wk = 0.f;
        if (kk < ni) {
          if (kk < 64) {
            wk = lane_value(wt, kk);
          } else if (lse != -INFINITY && nonempty(u0[i] + kk)) {
            wk = expf(lse_part[slot0[i] + (int64_t)kk * R] - lse);
          }
        }
        wv[k] = wk;
        vv[k] = wk != 0.f ? *(const h8*)(o_part + (slot0[i] + (int64_t)kk * R) * 512 + c) : h8{};
      }
#pragma unroll
      for (int k = 0; k < kCPChunk; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(wv[k], (float)vv[k][e], acc[e]);
    }
    bf16x8 ov;
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[e] = (__bf16)acc[e];
    *(bf16x8*)(lat + j * kCPPitch + 16 * lane) = ov;  // rows past M hold zeros
    if (o_lat && vpart == 0 && m < M) *(bf16x8*)(o_lat + ((int64_t)m * H + h) * 512 + c) = ov;
  }
  __syncthreads();

  // ---- phase 2: o[m, h, vb..vb+31] = o_lat[m] W_UV[h][vb..]^T; the wave sums
  // latent part kh, parts 1.. hand their sums to part 0 through LDS
  const int nvb = d_v / 32;
  for (int base = 0; base < nvb; base += 4) {
    const int cb = base + kNC * vpart + cq;
    const bool act = cb < nvb;
    if (base > 0 && act) {
      const bf16x8* bp = (const bf16x8*)(w_uv + ((int64_t)h * d_v + 32 * cb + n32) * 512);
#pragma unroll
      for (int k = 0; k < kSteps; ++k) bw[k] = bp[2 * (kSteps * kh + k) + hf];
    }
    for (int rb = 0; rb < ROWS / 32; ++rb) {  // 32-row blocks of the tile
      f32x16 acc2[2] = {f32x16{}, f32x16{}};  // even / odd k-steps: two chains
      if (act) {
#pragma unroll
        for (int k = 0; k < kSteps; ++k) {
          const bf16x8 av = *(const bf16x8*)(lat + (32 * rb + n32) * kCPPitch +
                                             (16 * (kSteps * kh + k) + 8 * hf) * 2);
          acc2[k & 1] = mfma32(av, bw[k], acc2[k & 1]);
        }
      }
      mfma_settle(acc2[0]);
      mfma_settle(acc2[1]);
      f32x16 acc = acc2[0] + acc2[1];
      if (kh >= 1 && act) {
        f32x4* rp = (f32x4*)(red + (((kh - 1) * kNC + cq) * 64 + lane) * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) rp[q] = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
      }
      __syncthreads();
      if (kh == 0 && act) {
#pragma unroll
        for (int p = 1; p < kNK; ++p) {
          const f32x4* rp = (const f32x4*)(red + (((p - 1) * kNC + cq) * 64 + lane) * 16);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 t = rp[q];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[4 * q + e] += t[e];
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int mr = mb0 + 32 * rb + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (mr < M) o[((int64_t)mr * H + h) * d_v + 32 * cb + n32] = f32_to_bf16(acc[r]);
        }
      }
      __syncthreads();
    }
  }
}

}  // namespace

bool combine_proj_supports(const mla_dims_t& d) {
  // Lq H <= 2^20 keeps the buffer ranges of a row's first partials in 32 bits
  return d.q_dtype == MLA_BF16 && d.d_latent == 512 && d.d_v % 32 == 0 &&
         (int64_t)d.q_len * d.heads <= (1 << 20);
}

hipError_t launch_combine_proj(const mla_dims_t& d, int num_splits, const int32_t* seq_lens,
                               const void* o_part, const float* lse_part, const void* w_uv,
                               void* o, float* lse_out, void* o_lat, hipStream_t s) {
  const int M = d.batch * d.q_len;
  // 32 query rows per workgroup up to 64 rows (every CU busy), 64 from 128
  // rows on: the workgroup holds one CU, so fewer, larger ones halve the
  // rounds of workgroups and the re-reads of W_UV[h].  Up to 32 rows one
  // workgroup per head would leave half the CUs idle: two share its
  // v-columns.
  if (M >= 128) {
    dim3 grid((unsigned)d.heads, (unsigned)((M + 63) / 64));
    hipLaunchKernelGGL((combine_proj_kernel<64, 1>), grid, dim3(512), 0, s, d.batch, d.q_len, d.heads,
                       num_splits, seq_lens, (const _Float16*)o_part, lse_part,
                       (const uint16_t*)w_uv, d.d_v, (uint16_t*)o, lse_out, (uint16_t*)o_lat);
  } else if (M > 32) {
    dim3 grid((unsigned)d.heads, (unsigned)((M + 31) / 32));
    hipLaunchKernelGGL((combine_proj_kernel<32, 1>), grid, dim3(512), 0, s, d.batch, d.q_len, d.heads,
                       num_splits, seq_lens, (const _Float16*)o_part, lse_part,
                       (const uint16_t*)w_uv, d.d_v, (uint16_t*)o, lse_out, (uint16_t*)o_lat);
  } else {
    dim3 grid((unsigned)d.heads, 1u, 2u);
    hipLaunchKernelGGL((combine_proj_kernel<32, 2>), grid, dim3(512), 0, s, d.batch, d.q_len, d.heads,
                       num_splits, seq_lens, (const _Float16*)o_part, lse_part,
                       (const uint16_t*)w_uv, d.d_v, (uint16_t*)o, lse_out, (uint16_t*)o_lat);
  }
  return hipGetLastError();
}

}  // namespace mla
