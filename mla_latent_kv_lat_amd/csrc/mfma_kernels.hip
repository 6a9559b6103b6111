// Matrix-core (MFMA) kernels for gfx950 around the attention: query
// absorption of W_UK with RoPE, and the W_UV output projection (bf16).
// The split-K decode itself lives in decode_split.hip.
//
// Pages cited (title, section):
//   [ARCH] "Model Architecture Driving Inference Systems: From MHA/GQA to
//          DeepSeek MLA Matrix Absorption and Memory Minimalism"
//   [MATH] "Multi-Head Latent Attention (MLA): Mathematical Foundations, ..."
//
// The absorbed query q_abs is written in fp16 (saturating at +-65504): its
// 11-bit significand is what keeps scores against long contexts with large
// cached values accurate (a bf16 query moves such scores by ~1e-2).
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
// One workgroup of 4 waves per (head, 128-column block).  The block of
// W_UK[h] (d_n rows x 128 columns) is staged in LDS once; each wave then
// owns 16 query rows of every 64-row block and computes the transposed
// product q_abs^T = W^T q^T with v_mfma_f32_16x16x32_bf16:
//   A (16 x 32) = W^T: lane l holds output column l%16, k 8(l/16)..+7,
//                 read transposed from LDS with ds_read_b64_tr_b16;
//   B (32 x 16) = q^T: lane l holds query row l%16, k 8(l/16)..+7, one
//                 16-byte load straight from q_nope;
//   C (16 x 16): lane l holds row m = l%16, output columns 4(l/16)..+3,
//                 stored as 8 contiguous bytes.
// The RoPE part ([ARCH] 2.3: pair k of the query turns by pos * base^(-2k/d_r))
// is spread over all threads of the head's workgroups: the angle is formed
// and reduced modulo 2 pi in double precision, then sin/cos in single.
constexpr int kAbsCols = 128;
constexpr int kAbsPitch = 320;  // bytes per staged W row: 256 + 64 keeps tr reads conflict-free
constexpr int kAbsMaxDn = 128;
constexpr int kRopeAhead = 4;  // RoPE pairs per thread whose inputs load before W

__global__ __launch_bounds__(256) void absorb_mfma_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_rope,
    const int32_t* __restrict__ positions, double rope_base, const uint16_t* __restrict__ w_uk,
    uint16_t* __restrict__ q_abs, int M, int H, int d_n, int d_r, int d_c) {
  __shared__ __attribute__((aligned(16))) char wsm[kAbsMaxDn * kAbsPitch];
  const int h = blockIdx.x;
  const int cb = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int W = d_c + d_r;

  const int g = lane >> 4, li = lane & 15;
  const int ksteps = (d_n + 31) / 32;
  // B operand (q rows m = mb + lane%16, k 8(lane/16).. of each 32-step);
  // the first block's loads go out together with the W loads below
  // (unconditional loads from clamped indices: a row past M is never
  // stored, and a k past d_n meets a zero row of W)
  auto load_q = [&](int mb, bf16x8 (&qb)[kAbsMaxDn / 32]) {
    const int m = min(mb + li, M - 1);
#pragma unroll
    for (int ks = 0; ks < kAbsMaxDn / 32; ++ks) {
      const int k0 = min(32 * ks + 8 * g, d_n - 8);
      if (ks < ksteps)  // uniform
        qb[ks] = *(const bf16x8*)(q_nope + ((int64_t)m * H + h) * d_n + k0);
    }
  };
  bf16x8 qb[kAbsMaxDn / 32];

  // RoPE work of this thread: pairs p = cb*256 + tid + i * rstride of the
  // M * half pairs; angle pos * base^(-2k/d_r) in double, reduced into
  // [-pi, pi], then sin/cos in single precision
  const int half = d_r / 2, np = M * half;
  const int rstride = (int)gridDim.y * 256;
  int rp[kRopeAhead], rpos[kRopeAhead];
  uint32_t rq[kRopeAhead];
#pragma unroll
  for (int j = 0; j < kRopeAhead; ++j) rp[j] = cb * 256 + tid + j * rstride;
  const double l2b = half > 0 ? log2(rope_base) : 0.0;
  auto rope_pair = [&](int p, int pos, uint32_t xq) {
    const int m = p / half, k = p % half;
    const double theta = exp2(-2.0 * k / d_r * l2b);
    double ang = (double)pos * theta;
    ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);  // into [-pi, pi]
    float sn, cs;
    __sincosf((float)ang, &sn, &cs);
    const float x0 = bf16_to_f32((uint16_t)(xq & 0xffffu)), x1 = bf16_to_f32((uint16_t)(xq >> 16));
    const int64_t dst = ((int64_t)m * H + h) * W + d_c + 2 * k;
    *(uint32_t*)(q_abs + dst) = (uint32_t)f32_to_f16_sat_bits(x0 * cs - x1 * sn) |
                                ((uint32_t)f32_to_f16_sat_bits(x0 * sn + x1 * cs) << 16);
  };

  // inputs of this thread's first RoPE pairs, issued first so that their
  // arithmetic below overlaps the W_UK and q loads; the loads are
  // unconditional (indices clamped) so that no branch puts a wait between
  // them and the W_UK loads
  if (np > 0) {  // uniform
#pragma unroll
    for (int j = 0; j < kRopeAhead; ++j) {
      const int pj = rp[j] < np ? rp[j] : np - 1;
      const int m = pj / half, k = pj % half;
      rpos[j] = positions[m];
      rq[j] = *(const uint32_t*)(q_rope + ((int64_t)m * H + h) * d_r + 2 * k);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // stage W_UK[h][:, cb*128 .. +128]: thread reads chunk tid%16 of rows
  // tid/16 + 16i; rows past d_n are zero (they meet zero-padded k of q)
  {
    const char* wsrc = (const char*)(w_uk + (int64_t)h * d_n * d_c + cb * kAbsCols);
    uint4 st[kAbsMaxDn / 16];
#pragma unroll
    for (int i = 0; i < kAbsMaxDn / 16; ++i) {  // rows clamped here, zeroed at the LDS store
      const int r = min((tid >> 4) + 16 * i, d_n - 1);
      st[i] = *(const uint4*)(wsrc + (int64_t)r * d_c * 2 + (tid & 15) * 16);
    }
    load_q(16 * w, qb);
    __builtin_amdgcn_sched_barrier(0);

    // RoPE pairs of this head, spread over its column-block workgroups
#pragma unroll
    for (int j = 0; j < kRopeAhead; ++j)
      if (rp[j] < np) rope_pair(rp[j], rpos[j], rq[j]);
    for (int p = rp[kRopeAhead - 1] + rstride; p < np; p += rstride)
      rope_pair(p, positions[p / half],
                *(const uint32_t*)(q_rope + ((int64_t)(p / half) * H + h) * d_r + 2 * (p % half)));

#pragma unroll
    for (int i = 0; i < kAbsMaxDn / 16; ++i) {
      const int r = (tid >> 4) + 16 * i;
      *(uint4*)(wsm + r * kAbsPitch + (tid & 15) * 16) = r < d_n ? st[i] : make_uint4(0, 0, 0, 0);
    }
  }
  __syncthreads();

  for (int mb = 16 * w; mb < M; mb += 64) {
    const int m = mb + li;
    const bool mv = m < M;
    f32x4 acc[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[nb] = f32x4{};
#pragma unroll
    for (int ks = 0; ks < kAbsMaxDn / 32; ++ks) {
      if (ks >= ksteps) break;
      const int r0 = 32 * ks + 8 * g + (li >> 2);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const uint32_t off = (uint32_t)(r0 * kAbsPitch + (nb * 16 + 4 * (li & 3)) * 2);
        const bf16x8 wa = cat(lds_tr4(wsm, off), lds_tr4(wsm, off + 4 * kAbsPitch));
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa, qb[ks], acc[nb], 0, 0, 0);
      }
    }
    if (mv) {
      uint16_t* dst = q_abs + ((int64_t)m * H + h) * W + cb * kAbsCols + 4 * g;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const uint2 v = make_uint2(
            (uint32_t)f32_to_f16_sat_bits(acc[nb][0]) | ((uint32_t)f32_to_f16_sat_bits(acc[nb][1]) << 16),
            (uint32_t)f32_to_f16_sat_bits(acc[nb][2]) | ((uint32_t)f32_to_f16_sat_bits(acc[nb][3]) << 16));
        *(uint2*)(dst + nb * 16) = v;
      }
    }
    if (mb + 64 < M) load_q(mb + 64, qb);
  }
}

// =================================================================== out proj
// o[m, h, v] = sum_c W_UV[h][v][c] o_lat[m, h, c]   ([ARCH] 3.2)
// One workgroup per (head, 32 query rows), one wave per 32 output columns.
// Both operands have the contracted latent index contiguous in memory, so
// they load straight into MFMA registers: the wave's 32 rows of W_UV[h]
// (512-wide latent: 32 steps of 16) and its 32 rows of o_lat.
constexpr int kOutMaxDc = 512;

__global__ __launch_bounds__(256) void out_proj_mfma_kernel(
    const uint16_t* __restrict__ o_lat, const uint16_t* __restrict__ w_uv,
    uint16_t* __restrict__ o, int M, int H, int d_c, int d_v) {
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63, hf = lane >> 5, n32 = lane & 31;
  const int nvg = (d_v / 32 + 3) / 4;  // groups of 4 v-blocks
  const int vb = ((blockIdx.y % nvg) * 4 + (threadIdx.x >> 6)) * 32;
  const int mb0 = (blockIdx.y / nvg) * 32;  // this workgroup's 32 query rows
  if (vb >= d_v) return;
  const bf16x8* bp = (const bf16x8*)(w_uv + ((int64_t)h * d_v + vb + n32) * d_c);
  const int nk = d_c / 16;
  constexpr int kK = kOutMaxDc / 16;
  bf16x8 bw[kK];
#pragma unroll
  for (int k = 0; k < kK; ++k) bw[k] = k < nk ? bp[2 * k + hf] : bf16x8{};
  {
    const int mb = mb0;
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
  // d_rope % 4: q_abs rows then start 8-byte aligned for the vector stores
  return d.q_dtype == MLA_BF16 && d.d_nope % 16 == 0 && d.d_nope <= kAbsMaxDn &&
         d.d_latent % kAbsCols == 0 && d.d_rope % 4 == 0 && d.d_rope <= 128;
}

hipError_t launch_absorb_mfma(const mla_dims_t& d, const void* q_nope, const void* q_rope,
                              const int32_t* positions, float rope_base, const void* w_uk,
                              void* q_abs, hipStream_t s) {
  const int M = d.batch * d.q_len;
  dim3 grid((unsigned)d.heads, (unsigned)(d.d_latent / kAbsCols));
  hipLaunchKernelGGL(absorb_mfma_kernel, grid, dim3(256), 0, s,
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
  dim3 grid((unsigned)d.heads, (unsigned)(((d.d_v / 32 + 3) / 4) * ((M + 31) / 32)));
  hipLaunchKernelGGL(out_proj_mfma_kernel, grid, dim3(256), 0, s, (const uint16_t*)o_lat,
                     (const uint16_t*)w_uv, (uint16_t*)o, M, d.heads, d.d_latent, d.d_v);
  return hipGetLastError();
}

}  // namespace mla
