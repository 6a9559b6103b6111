// Matrix-core (MFMA) kernels for gfx950: bf16 queries and weights, bf16 or
// fp8 cache, DeepSeek-V3 widths (latent 512, RoPE 64).
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
// The order of k inside one instruction is immaterial as long as A and B
// agree, which lets P stay in the registers the score MFMA wrote it to.
//
// ds_read_b64_tr_b16: in each group of 16 lanes, lane i names 4 consecutive
// 16-bit elements (row i/4, columns 4*(i%4)..+3 of a 4 x 16 block) and gets
// back column i of that block, rows 0..3.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.hpp"
#include "kernels.hpp"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 lds_tr4(const char* base, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)((lds_char*)base + off));
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// One 16-byte direct global->LDS load per lane: lane i reads 16 bytes at
// sbase + voff (sbase wave-uniform, voff per lane) and the wave's 64 lanes fill
// the 1 KB of LDS starting at byte address m0 in lane order.  Issued as
// inline assembly so that waits on it are placed by hand (vmcnt), instead of
// the compiler's blanket wait before every later LDS read.
__device__ __forceinline__ void lds_dma16(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(voff),
               "s"(sbase)
               : "memory", "m0");
}
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
// vmcnt(0) through the builtin, so the compiler's own wait bookkeeping also
// sees every earlier vector load as complete (and places no later waits for
// them, which would otherwise land on the next tile's prefetch).
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0f70); }
__device__ __forceinline__ void block_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ===================================================================== decode
//
// One workgroup = one split-K unit x one group of 128 query rows (rows are
// (query i, head h) pairs, i*H + h).  8 waves, each owning 16 rows: the heads
// sit on an MFMA dimension, so one pass over a cached tile in LDS serves all
// 128 heads ([ARCH] 3.1: every head scores the same raw cached latent).
//
// Per 64-token tile (bf16: 64 rows x 576 = 72 KB, double-buffered in LDS),
// in two halves of 32 tokens:
//   S^T[t, h] = sum_c K[t, c] Q[h, c]   K = tile (LDS), Q = q_abs (registers)
//   online softmax over t (per head), in log2 units
//   O[h, c]  += sum_t P[h, t] V[t, c]   V = tile latent part (LDS, transposed
//                                        reads), O = fp32 accumulators
// with v_mfma_f32_16x16x32_bf16, whose operand layouts are
//   A (16 x 32): lane l holds row l%16, k = 8*(l/16) .. +7
//   B (32 x 16): lane l holds column l%16, k = 8*(l/16) .. +7
//   C (16 x 16): lane l holds column l%16, rows 4*(l/16) .. +3
// The order of k inside one instruction is immaterial as long as A and B
// agree, so P is used as the A operand right where the score MFMA left it.
//
// LDS tile layout: 1 KB blocks of 8 rows x 8 chunks (chunk = 16 bytes), block
// (cg, rg) at ((cg*8 + rg) KB) for chunk group cg (0..8) and row group rg
// (0..7).  Inside a block, row rho / chunk kappa sits at entry
//   8*(kappa ^ (rg&1)) + (rho ^ 4*((kappa ^ kappa>>1) & 1))
// which keeps both the score reads (16 rows x one chunk) and the transposed
// value reads (8 rows x 2 chunks) free of bank conflicts.  One block is
// exactly one wave-wide 16-byte direct load: 8 rows x 128 contiguous bytes.

constexpr int kRowsPerWG = 128;
constexpr int kWaves = 8;
constexpr int kTileBytesBF16 = kTile * 576 * 2;  // 73728

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct TileRef {
  int t0;       // first token of the tile
  int n_tok;    // cached tokens of the sequence (rows past it are clamped)
  int64_t row0; // cache row of token t0
};

__device__ __forceinline__ TileRef tile_ref(const DecodeArgs& a, int b, int64_t tile_in_seq) {
  TileRef r;
  r.t0 = (int)tile_in_seq * kTile;
  r.n_tok = a.seq_lens[b];
  r.row0 = a.block_table ? (int64_t)a.block_table[(int64_t)b * a.mbps + tile_in_seq] * kTile
                         : (int64_t)b * a.max_seq_len + r.t0;
  return r;
}

// Issue this wave's 9 of the tile's 72 block loads (bf16 cache): row group
// rg = w, all 9 chunk groups.  Rows past the end of the sequence are clamped
// to its last row, so poisoned tail slots of a page are never read.
__device__ __forceinline__ void issue_tile_bf16(const DecodeArgs& a, const TileRef& tr,
                                                uint32_t lds_base, int w, int lane) {
  const int kappa = (lane >> 3) ^ (w & 1);
  const int rho = (lane & 7) ^ (4 * ((kappa ^ (kappa >> 1)) & 1));
  const int nvalid = tr.n_tok - tr.t0;  // >= 1
  int r = w * 8 + rho;
  r = r < nvalid ? r : nvalid - 1;
  const int64_t stride = a.row_stride * 2;  // bytes
  const char* lat = (const char*)a.latent + tr.row0 * stride;  // uniform
  const char* rop = (const char*)a.rope + tr.row0 * stride;    // uniform
  const uint32_t voff = (uint32_t)(r * stride) + (uint32_t)(kappa * 16);
#pragma unroll
  for (int cg = 0; cg < 8; ++cg)
    lds_dma16(lat, voff + cg * 128, lds_base + (uint32_t)((cg * 8 + w) * 1024));
  lds_dma16(rop, voff, lds_base + (uint32_t)((64 + w) * 1024));
}

template <int KV>  // KV: MLA_BF16
__global__ __launch_bounds__(512, 1) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kTileBytesBF16];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;     // lane group (k slice of the MFMA operands)
  const int li = lane & 15;    // this lane's head (column) within the wave
  const int R = a.q_len * a.heads;
  const int u = blockIdx.x;
  const int row0 = blockIdx.y * kRowsPerWG + w * 16;  // first query row of this wave
  const bool active = row0 < R;
  const int qi = active ? row0 / a.heads : 0;          // query token of this wave
  const int h0 = active ? row0 % a.heads : 0;

  int64_t T, unused;
  wave_tile_sums(a.seq_lens, a.batch, 0, T, unused);
  T = uniform64(T);
  const int64_t x0 = unit_begin(u, T, a.num_splits);
  const int64_t x1 = unit_begin(u + 1, T, a.num_splits);
  if (x0 >= x1) return;  // uniform across the workgroup

  int cur_b;
  int64_t cur_pb;
  find_sequence(a.seq_lens, a.batch, x0, cur_b, cur_pb);
  cur_b = __builtin_amdgcn_readfirstlane(cur_b);
  cur_pb = uniform64(cur_pb);

  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)smem;
  const float sl2 = a.softmax_scale * kLog2e;

  // ---- per-lane constant parts of the LDS read addresses --------------------
  // score reads: token row 16*j + li, chunk 4*kk + g
  const int fq = (g ^ (g >> 1)) & 1;
  const uint32_t qk_off = (uint32_t)(((li >> 3) & 1) * 1024 + 128 * (g ^ ((li >> 3) & 1)) +
                                     16 * ((lane & 7) ^ (4 * fq)));
  // value reads (transposed): token row 16*rd + 4*g + li/4, column 16*nb + 4*(li%4)
  const int bq = (li & 3) >> 1;
  const int rho_v = 4 * (g & 1) + (li >> 2);
  uint32_t pv_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par)
    pv_off[par] = (uint32_t)((g >> 1) * 1024 + 128 * (bq ^ (g >> 1)) +
                             16 * (rho_v ^ (4 * (bq ^ par))) + 8 * (li & 1));

  // ---- first tile of the unit ------------------------------------------------
  int64_t x = x0;
  issue_tile_bf16(a, tile_ref(a, cur_b, x - cur_pb), lds0, w, lane);

  bf16x8 q[18];
  f32x4 o[32];
  float m_run = -INFINITY, l_run = 0.f;
  bool new_seg = true;
  int buf = 0;

  while (x < x1) {
    const int len = a.seq_lens[cur_b];
    const int64_t tb = tiles_of(len);
    const int64_t tis = x - cur_pb;  // tile index within the sequence
    if (new_seg) {
      // new segment: load this wave's 16 query rows, reset the state
      new_seg = false;
      const bf16x8* qp = (const bf16x8*)((const uint16_t*)a.q_abs +
                                          (((int64_t)cur_b * a.q_len + qi) * a.heads + h0 + li) * 576);
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) q[kk] = qp[4 * kk + g];
#pragma unroll
      for (int nb = 0; nb < 32; ++nb) o[nb] = f32x4{};
      m_run = -INFINITY;
      l_run = 0.f;
    }
    const int n_vis = a.causal ? len - a.q_len + qi + 1 : len;
    int nv = n_vis - (int)tis * kTile;  // visible tokens of this tile for this wave
    nv = nv < 0 ? 0 : (nv > kTile ? kTile : nv);

    // next tile of the unit (possibly in a later sequence)
    const int64_t xn = x + 1;
    const bool seg_end = xn >= x1 || xn >= cur_pb + tb;
    int nb_b = cur_b;
    int64_t nb_pb = cur_pb;
    if (xn < x1 && xn >= cur_pb + tb) {
      nb_pb = cur_pb + tb;
      ++nb_b;
      while (tiles_of(a.seq_lens[nb_b]) == 0) ++nb_b;
    }

    wait_vm0();     // this wave's loads of tile x have landed
    block_sync();   // ... and everyone's; everyone also finished tile x-1
    if (xn < x1)
      issue_tile_bf16(a, tile_ref(a, nb_b, xn - nb_pb),
                      lds0 + (uint32_t)((buf ^ 1) * kTileBytesBF16), w, lane);

    const char* tile = smem + buf * kTileBytesBF16;
    if (active && nv > 0) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        if (32 * h2 >= nv) break;
        // ---------------- scores for tokens 32*h2 .. +31: two 16 x 16 blocks,
        // interleaved, with the tile reads issued kPf steps ahead
        constexpr int kPf = 2;
        f32x4 s[2] = {f32x4{}, f32x4{}};
        bf16x8 ka[kPf + 1][2];
        auto kload = [&](int kk, int j) {
          const uint32_t off = (uint32_t)((kk >> 1) * 8192 + (2 * h2 + j) * 2048 +
                                          512 * (kk & 1)) + qk_off;
          return *(const bf16x8*)(tile + off);
        };
#pragma unroll
        for (int kk = 0; kk < kPf; ++kk) {
          ka[kk][0] = kload(kk, 0);
          ka[kk][1] = kload(kk, 1);
        }
#pragma unroll
        for (int kk = 0; kk < 18; ++kk) {
          if (kk + kPf < 18) {
            ka[(kk + kPf) % (kPf + 1)][0] = kload(kk + kPf, 0);
            ka[(kk + kPf) % (kPf + 1)][1] = kload(kk + kPf, 1);
          }
          s[0] = mfma16(ka[kk % (kPf + 1)][0], q[kk], s[0]);
          s[1] = mfma16(ka[kk % (kPf + 1)][1], q[kk], s[1]);
          __builtin_amdgcn_sched_barrier(0);  // keep each prefetch in its step
        }
        // ---------------- online softmax (log2 domain)
        float mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 32 * h2 + 16 * j + 4 * g + r;
            const float v = t < nv ? s[j][r] * sl2 : -INFINITY;
            s[j][r] = v;
            mt = fmaxf(mt, v);
          }
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m_run, mt);
        // Rescale only when the running max grows by more than 2^8: the
        // exponentials stay <= 256, and the final normalisation uses the
        // same reference max for numerator and denominator, so the result
        // is unchanged.
        const bool rescale = __ballot(m_new > m_run + 8.f) != 0;
        f32x4 a4 = f32x4{1.f, 1.f, 1.f, 1.f};
        if (rescale) {
          // 0 when m_run = -inf; 1 for a head that has seen no token yet
          const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int r = 0; r < 4; ++r) a4[r] = __shfl(alpha, 4 * g + r, 64);
        }
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        bf16x8 p;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = exp2f(s[j][r] - m_use);
            l_run += e;
            p[4 * j + r] = (__bf16)e;
          }
        // ---------------- O = a4 * O + P V for tokens 32*h2 .. +31; the
        // rescaling pass only runs when some head's running max moved.
        if (rescale) {
#pragma unroll
          for (int nb = 0; nb < 32; ++nb) o[nb] *= a4;
        }
        const uint32_t kbase = (uint32_t)(h2 * 4096);
        constexpr int kPv = 3;
        bf16x8 vb[kPv + 1];
        auto vload = [&](int nb) {
          const uint32_t cb = (uint32_t)((nb >> 2) * 8192 + 256 * (nb & 3)) + kbase;
          return cat(lds_tr4(tile, cb + pv_off[nb & 1]), lds_tr4(tile, cb + 2048 + pv_off[nb & 1]));
        };
#pragma unroll
        for (int nb = 0; nb < kPv; ++nb) vb[nb] = vload(nb);
#pragma unroll
        for (int nb = 0; nb < 32; ++nb) {
          if (nb + kPv < 32) vb[(nb + kPv) % (kPv + 1)] = vload(nb + kPv);
          o[nb] = mfma16(p, vb[nb % (kPv + 1)], o[nb]);
          __builtin_amdgcn_sched_barrier(0);  // keep each prefetch in its step
        }
      }
    }

    if (seg_end) {
      if (active) {
        const int64_t slot = (int64_t)u + cur_b;
        float l_tot = l_run + __shfl_xor(l_run, 16, 64);
        l_tot += __shfl_xor(l_tot, 32, 64);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        if (g == 0)
          a.lse_part[slot * R + row0 + li] =
              l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
        float* op = a.o_part + (slot * R + row0) * 512;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int hr = 4 * g + r;
          const float ir = __shfl(inv, hr, 64);
#pragma unroll
          for (int nb = 0; nb < 32; ++nb) op[(int64_t)hr * 512 + nb * 16 + li] = o[nb][r] * ir;
        }
      }
      new_seg = true;
    }
    x = xn;
    cur_b = nb_b;
    cur_pb = nb_pb;
    buf ^= 1;
  }
}

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

bool mfma_decode_supports(const mla_dims_t& d, int64_t row_stride, const void* latent,
                          const void* rope) {
  return d.q_dtype == MLA_BF16 && d.kv_dtype == MLA_BF16 && d.d_latent == 512 &&
         d.d_rope == 64 && d.heads % 16 == 0 && (row_stride * 2) % 16 == 0 &&
         ((uintptr_t)latent & 15) == 0 && ((uintptr_t)rope & 15) == 0;
}

hipError_t launch_decode_mfma(const mla_dims_t& d, const DecodeArgs& a, hipStream_t s) {
  const int R = d.q_len * d.heads;
  dim3 grid((unsigned)a.num_splits, (unsigned)((R + kRowsPerWG - 1) / kRowsPerWG));
  hipLaunchKernelGGL(decode_mfma_kernel<MLA_BF16>, grid, dim3(kWaves * 64), 0, s, a);
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
