// MLA prefill in MHA form for gfx950 (bf16; d_nope = d_v = 128, d_rope = 64,
// d_latent = 512).
//
// Pages cited (title, section):
//   [ARCH] "Model Architecture Driving Inference Systems: From MHA/GQA to
//          DeepSeek MLA Matrix Absorption and Memory Minimalism" (FAQ on
//          prefill: absorbing there multiplies the attention flops by the
//          ratio of latent to head width, ~4x)
//   [DUAL] "DeepSeek's attention evolution - [MLA]" 2.5 (prefill runs the
//          "MHA form": the latent is expanded into per-head keys and values;
//          decode runs the absorbed "MQA form")
//
// Two kernels, one per ABI call:
//
// prefill_expand_kernel: k_nope[b,t,h,:] = W_UK,h c_t and v[b,t,h,:] = W_UV,h c_t
//   for every cached token, one GEMM of the tokens' latents (K = 512) against
//   the 2H x 128 rows of W_UK and W_UV.  Workgroup = 128 tokens of one
//   sequence x one head's 128 k or v channels, 4 waves of 64 x 64 on
//   v_mfma_f32_32x32x16_bf16; both operands stream through LDS in 64-wide k
//   chunks (direct global->LDS loads, double buffered).
//
// prefill_attn_kernel: causal attention of the Lq prompt tokens of each
//   sequence over its keys [k_nope ; k_rope] (192 wide, the decoupled RoPE
//   key shared by the heads) and values (128 wide).  Workgroup = 256 query
//   rows of one (sequence, head), 16 waves of 16 rows; the keys and values of
//   64 tokens (one page) at a time are filled into LDS once for all 256 rows.  Each wave
//   computes S^T = K Q^T, the online softmax and O^T += V^T P^T on
//   v_mfma_f32_16x16x32_bf16 with P fed from the score registers, exactly as
//   the decode kernel does with the latent (same LDS layout and operand
//   addressing).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "common.hpp"
#include "decode_common.hpp"
#include "kernels.hpp"
#include "mfma_common.hpp"

namespace mla {
namespace {

using namespace mfma;
using namespace dec;

// Workgroups are dispatched to the 8 XCDs round-robin by linear id (id % 8).
// Map id to an item so that XCD x gets the contiguous items
// [x q + min(x, r), ...) of n = 8 q + r, in dispatch order: a bijection of
// [0, n), since id = 8 k + x has k < q + (x < r).
__device__ __forceinline__ uint32_t xcd_item(uint32_t id, uint32_t n) {
  const uint32_t q = n >> 3, r = n & 7, x = id & 7;
  return x * q + min(x, r) + (id >> 3);
}

// ------------------------------------------------------------------ expand

constexpr int kExTok = 128;                  // tokens per workgroup
constexpr int kExKc = 64;                    // k per LDS chunk
constexpr int kExOpBytes = 128 * kExKc * 2;  // 16 KB: one operand's chunk
constexpr int kExBytes = 2 * 2 * kExOpBytes; // two buffers of A and B

// 1 KB LDS block j = rows 8j..8j+7 x 8 16-byte chunks; row rho, chunk kappa
// at entry 8 rho + (kappa ^ rho ^ (j & 1)).  A 32x32x16 operand read (32
// rows, one chunk) is served 16 lanes at a time: rows 8j.. and 8(j+1).. of
// one group then fall in complementary halves of the 64 banks.  The
// wave-wide fill writes lane e at entry e, so it loads chunk
// (e%8) ^ row ^ (j & 1).
__device__ __forceinline__ uint32_t ex_entry(int row, int kap) {
  return (uint32_t)((row >> 3) * 1024 + 16 * (8 * (row & 7) + (kap ^ (row & 7) ^ ((row >> 3) & 1))));
}

__global__ __launch_bounds__(256) void prefill_expand_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kExBytes];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = a.heads;
  // Work order: workgroups reach the 8 XCDs round-robin by linear id, so
  // XCD x is given the contiguous item range x*N/8.. (xcd_item).  Items run
  // channel-block-fastest within groups of HG channel blocks, then token
  // tiles, then groups: the workgroups an XCD runs at once share one token
  // tile's latents and the group's HG x 128 KB of weights stay in its L2.
  const uint32_t T = gridDim.y;
  const uint32_t item = xcd_item(blockIdx.x + gridDim.x * blockIdx.y, gridDim.x * T);
  const uint32_t HG = (2 * H) % 8 == 0 ? 8 : ((2 * H) % 4 == 0 ? 4 : 2);
  const uint32_t rest = item / HG, tile = rest % T;
  const int cb = (int)((rest / T) * HG + item % HG);  // channel block: W_UK,h (cb < H) or W_UV,h
  const int b = (int)(tile / a.ntile);
  const int t0 = (int)(tile % a.ntile) * kExTok;
  const int len = a.seq_lens[b];
  if (t0 >= len) return;  // uniform across the workgroup
  const bool is_v = cb >= H;
  const int h = is_v ? cb - H : cb;
  const uint16_t* wsrc = (is_v ? a.w_uv : a.w_uk) + (int64_t)h * 128 * 512;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)smem;

  // first cache row of the tile's two 64-token pages (the second only when
  // the sequence reaches it)
  auto page_row = [&](int page) -> int64_t {
    return a.block_table ? (int64_t)a.block_table[(int64_t)b * a.mbps + page] * kTile
                         : (int64_t)b * a.max_seq_len + (int64_t)page * kTile;
  };
  const int pg0 = t0 >> 6;
  const int64_t prow0 = page_row(pg0);
  const int64_t prow1 = t0 + kTile < len ? page_row(pg0 + 1) : prow0;

  // fill lane: row e/8 of a block, chunk (e%8) ^ row
  const int frow = lane >> 3, fkap = (lane & 7) ^ frow ^ (w & 1);
  // block j of a chunk: j < 16 the tokens' latents (rows 8j..), else the
  // weight rows 8(j-16)..; wave w issues j = w, w+4, .., w+28
  auto issue = [&](int kc, int buf) {
    const uint32_t dst = lds0 + (uint32_t)(buf * 2 * kExOpBytes);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = w + 4 * i;
      if (j < 16) {
        // the block's rows, clamped to the sequence's last token (a whole
        // block past the end re-reads it); all in one page
        const int tb = min(t0 + 8 * j, len - 1);
        const int ps = tb & ~(kTile - 1);
        const int64_t r0 = (tb >> 6) == pg0 ? prow0 : prow1;
        const int tl = min(t0 + 8 * j + frow, len - 1) - ps;
        const char* base = (const char*)a.latent + r0 * a.row_stride * 2;
        const uint32_t voff = (uint32_t)(tl * a.row_stride * 2) + (uint32_t)((kc * kExKc + fkap * 8) * 2);
        lds_dma16(base, voff, dst + (uint32_t)(j * 1024));
      } else {
        const int jr = j - 16;
        const uint32_t voff = (uint32_t)(((8 * jr + frow) * 512 + kc * kExKc + fkap * 8) * 2);
        lds_dma16(wsrc, voff, dst + (uint32_t)(kExOpBytes + jr * 1024));
      }
    }
  };

  const int wr = w >> 1, wc = w & 1;  // wave tile: tokens 64 wr.., channels 64 wc..
  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16{};

  issue(0, 0);
  constexpr int kChunks = 512 / kExKc;
  for (int kc = 0; kc < kChunks; ++kc) {
    if (kc + 1 < kChunks) issue(kc + 1, (kc + 1) & 1);
    if (kc + 1 < kChunks)
      wait_vm(8);  // this wave's loads of chunk kc landed (those of kc+1 in flight)
    else
      wait_vm(0);
    block_sync();
    const char* A = smem + (kc & 1) * 2 * kExOpBytes;
    const char* Bm = A + kExOpBytes;
    const int l32 = lane & 31, hk = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < kExKc / 16; ++ks) {
      const int kap = 2 * ks + hk;
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        av[mi] = *(const bf16x8*)(A + ex_entry(64 * wr + 32 * mi + l32, kap));
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        bv[ni] = *(const bf16x8*)(Bm + ex_entry(64 * wc + 32 * ni + l32, kap));
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma32(av[mi], bv[ni], acc[mi][ni]);
    }
    block_sync();  // the buffer is refilled by the loads of chunk kc+2
  }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) mfma_settle(acc[mi][ni]);

  // C (32 x 32): lane l holds channel l%32, tokens 8(r/4) + 4(l/32) + r%4
  uint16_t* dst = (uint16_t*)(is_v ? a.v : a.k_nope);
  const int ch = lane & 31, hr = lane >> 5;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = t0 + 64 * wr + 32 * mi + 8 * (r >> 2) + 4 * hr + (r & 3);
      if (t < len) {
        uint16_t* row = dst + (((int64_t)b * a.max_seq_len + t) * H + h) * 128 + 64 * wc + ch;
        row[0] = f32_to_bf16(acc[mi][0][r]);
        row[32] = f32_to_bf16(acc[mi][1][r]);
      }
    }
}

// --------------------------------------------------------------- attention

constexpr int kAtWaves = 16;
constexpr int kAtRows = 16 * kAtWaves;          // 256 query rows per workgroup
constexpr int kAtSub = 64;                      // tokens per LDS sub-tile (one page)
constexpr int kAtCg = kAtSub * 128;             // 8 KB: one 64-column group of the sub-tile
constexpr int kAtKBytes = 3 * kAtCg;            // 24 KB: keys, column groups 0-2
constexpr int kAtSubBytes = kAtKBytes + 2 * kAtCg;  // + 16 KB values
constexpr int kAtRing = 3;
constexpr int kAtMaxPages = 4096;               // 262144 tokens
constexpr int kAtPageOff = kAtRing * kAtSubBytes;
constexpr int kAtThetaOff = kAtPageOff + kAtMaxPages * 4;
constexpr int kAtBytes = kAtThetaOff + 32 * 8;
static_assert(kAtBytes <= 163840, "LDS budget");

__global__ __launch_bounds__(1024) void prefill_attn_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kAtBytes];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = a.heads, Lq = a.q_len;
  const int nqb = (Lq + kAtRows - 1) / kAtRows;
  const int64_t Tmax = a.max_seq_len;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)smem;
  int* prow = (int*)(smem + kAtPageOff);  // block id (paged) of each page of the item

  // RoPE frequencies base^(-2p/64) of the 32 pairs, once (the first
  // item's barrier orders them before use)
  double* theta = (double*)(smem + kAtThetaOff);
  if (threadIdx.x < 32) theta[threadIdx.x] = exp2(-2.0 * (int)threadIdx.x / 64.0 * log2((double)a.rope_base));

  // Persistent workgroups, one per compute unit: the items, (sequence,
  // head, query block) with the query blocks of a head consecutive and the
  // longest causal range first, are cut into P = min(8, grid) contiguous
  // ranges; workgroup g takes range g % P, which is its XCD's when the
  // grid is a multiple of 8 (workgroups reach the XCDs round-robin), so
  // the query blocks of one head share an L2.  Its nx workgroups deal the
  // range out in rounds of nx items, the order reversed every other round
  // so that the long and short blocks of the heads even out.
  const uint32_t n_items = (uint32_t)nqb * (uint32_t)H * (uint32_t)a.batch;
  const uint32_t G = gridDim.x, g = blockIdx.x;
  const uint32_t P = G < 8 ? G : 8, pi = g % P, rank = g / P, nx = (G - pi + P - 1) / P;
  const uint32_t cnt = n_items / P + (pi < n_items % P ? 1u : 0u);
  const uint32_t beg = pi * (n_items / P) + min(pi, n_items % P);

  for (uint32_t rd = 0;; ++rd) {
  const uint32_t loc = rd * nx + ((rd & 1) ? nx - 1 - rank : rank);
  if (loc >= cnt) break;  // uniform
  const uint32_t item = beg + loc;
  const int qb = nqb - 1 - (int)(item % (uint32_t)nqb);
  const int h = (int)((item / (uint32_t)nqb) % (uint32_t)H), b = (int)(item / ((uint32_t)nqb * (uint32_t)H));
  const int len = a.seq_lens[b];
  const int i0 = qb * kAtRows;

  // visible tokens of query i: t < len - Lq + i + 1 (causal) or t < len
  auto n_vis = [&](int i) { return a.causal ? len - Lq + i + 1 : len; };
  const int i_last = min(Lq, i0 + kAtRows) - 1;
  const int n_end = min(len, max(0, n_vis(i_last)));  // tokens the workgroup reads
  const int nsub = (n_end + kAtSub - 1) / kAtSub;

  // rows of this wave; lane l holds row i0 + 16w + l%16
  const int wrow0 = i0 + 16 * w;
  const bool active = wrow0 < Lq;  // uniform per wave
  const int wave_vis = active ? min(len, max(0, n_vis(min(wrow0 + 15, Lq - 1)))) : 0;

  // page table of the tokens this item reads; the barrier also ends the
  // previous item's use of the ring
  if (a.block_table) {
    const int npg = (n_end + kTile - 1) / kTile;
    for (int pg = (int)threadIdx.x; pg < npg; pg += 1024) prow[pg] = a.block_table[(int64_t)b * a.mbps + pg];
  }
  block_sync();

  // ---- fills: 40 blocks of 1 KB per sub-tile (keys: column groups 0-1
  // k_nope, 2 the RoPE key; values: 0-1; 8 row groups each), block k by
  // wave k % 16; all of a wave's blocks are row group w & 7
  const int n_share = w < 8 ? 3 : 2;
  const int rg = w & 7;
  int pz = 0;  // next sub-tile to fill
  auto issue = [&]() {
    // lane offsets from an opaque lane id: recomputed here, not kept live
    // across the item loop
    const int fl = fresh_lane();
    const int kap = (fl >> 3) ^ (rg & 1);
    const int rho = (fl & 7) ^ (4 * ((kap ^ (kap >> 1)) & 1));
    const int t0 = pz * kAtSub;
    const uint32_t slot = lds0 + (uint32_t)((pz % kAtRing) * kAtSubBytes);
    const int tl = min(t0 + 8 * rg + rho, len - 1) - t0;  // clamped rows are masked
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int k = w + 16 * i;
      if (k >= 40) break;  // uniform
      if (k < 16 || k >= 24) {  // k_nope or v: [B, Tmax, H, 128]
        const int cg = (k < 16 ? k : k - 24) >> 3;
        const char* base = (const char*)(k < 16 ? a.k_nope : a.v) + (((int64_t)b * Tmax + t0) * H + h) * 256;
        const uint32_t voff = (uint32_t)(tl * H * 256) + (uint32_t)((cg * 64 + kap * 8) * 2);
        lds_dma16_stream((const char*)uniform64((int64_t)base), voff,
                         __builtin_amdgcn_readfirstlane(slot + (uint32_t)((k < 16 ? 0 : kAtKBytes) + cg * kAtCg + rg * 1024)));
      } else {  // RoPE key of the cache rows (the sub-tile is one page)
        const int64_t r0 = a.block_table ? (int64_t)prow[t0 >> 6] * kTile : (int64_t)b * Tmax + t0;
        const char* base = (const char*)a.rope + r0 * a.row_stride * 2;
        const uint32_t voff = (uint32_t)(tl * a.row_stride * 2) + (uint32_t)(kap * 16);
        lds_dma16_stream((const char*)uniform64((int64_t)base), voff,
                         __builtin_amdgcn_readfirstlane(slot + (uint32_t)(2 * kAtCg + rg * 1024)));
      }
    }
    ++pz;
  };

  // the first sub-tiles go out before the query loads, so both latencies
  // overlap
  for (int z = 0; z < kAtRing - 1 && z < nsub; ++z) issue();

  // ---- the wave's query rows: q_nope in k-slices 0-3, RoPE(q_rope) in 4-5
  bf16x8 q[6];
  {
    const int fl = fresh_lane();
    const int li = fl & 15, gq = fl >> 4;
    const int i = min(wrow0 + li, Lq - 1);
    const int64_t qrow = ((int64_t)b * Lq + i) * H + h;
    const bf16x8* qn = (const bf16x8*)((const uint16_t*)a.q_nope + qrow * 128);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) q[kk] = qn[4 * kk + gq];
    const bf16x8* qr = (const bf16x8*)((const uint16_t*)a.q_rope + qrow * 64);
    const double pos = (double)a.positions[(int64_t)b * Lq + i];
#pragma unroll
    for (int kk = 4; kk < 6; ++kk) {
      const bf16x8 x = qr[4 * (kk - 4) + gq];
      bf16x8 y;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        // pair p = 16 (kk-4) + 4 gq + m turns by pos * base^(-2p/64); the
        // angle is reduced modulo 2 pi in double, sin/cos in single
        const int pr = 16 * (kk - 4) + 4 * gq + m;
        double ang = pos * theta[pr];
        ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
        float sn, cs;
        __sincosf((float)ang, &sn, &cs);
        const float x0 = (float)x[2 * m], x1 = (float)x[2 * m + 1];
        y[2 * m] = (__bf16)(x0 * cs - x1 * sn);
        y[2 * m + 1] = (__bf16)(x0 * sn + x1 * cs);
      }
      q[kk] = y;
    }
    // taken here: the compiler's waits for the query (it does not count
    // the direct loads issued before them) then also cover sub-tiles 0-1
#pragma unroll
    for (int kk = 0; kk < 6; ++kk) asm volatile("" ::"v"(q[kk]));
  }
  if (nsub > 0) wait_vm(n_share * (pz - 1));
  block_sync();

  f32x4 o[8];  // O^T: block nb holds value columns 16 nb + 4(l/16)..+3 of row l%16
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) o[nb] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.softmax_scale * kLog2e;

  for (int s = 0; s < nsub; ++s) {
    if (s + kAtRing - 1 < nsub) issue();  // into the slot every wave finished with
    const char* tile = smem + (s % kAtRing) * kAtSubBytes;
    const int t0 = s * kAtSub;
    if (active && t0 < wave_vis) {  // uniform per wave
      f32x4 sc[4];  // token block jt: tokens 16 jt + 4(l/16)..+3
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) sc[jt] = f32x4{};
      {
        constexpr int kPf = 2;
        const uint32_t o_qk = off_qk(fresh_lane());
        bf16x8 ka[kPf + 1][4];
        auto kload = [&](int kk) {
          const int e = kk % (kPf + 1);
#pragma unroll
          for (int jt = 0; jt < 4; ++jt)
            ka[e][jt] = *(const bf16x8*)(tile + (uint32_t)((kk >> 1) * kAtCg + 2048 * jt + 512 * (kk & 1)) + o_qk);
        };
#pragma unroll
        for (int kk = 0; kk < kPf; ++kk) kload(kk);
#pragma unroll
        for (int kk = 0; kk < 6; ++kk) {
          if (kk + kPf < 6) kload(kk + kPf);
          const int e = kk % (kPf + 1);
#pragma unroll
          for (int jt = 0; jt < 4; ++jt) sc[jt] = mfma16(ka[e][jt], q[kk], sc[jt]);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) mfma_settle(sc[jt]);
      }
      const int ln = fresh_lane();
      const int nv = min(len, n_vis(wrow0 + (ln & 15)));  // this lane's row
      if (t0 + kAtSub > nv) {  // mask past the visible end
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (t0 + 16 * jt + 4 * (ln >> 4) + r >= nv) sc[jt][r] = -INFINITY;
      }
      // lazy rescale: the reference max moves only when a score passes it
      // by more than 2^8 (log2 units)
      float lm = sc[0][0];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) lm = fmaxf(lm, sc[jt][r]);
      lm *= sl2;
      if (__ballot(lm > m_run + 8.f) != 0) {
        float mt = fmaxf(lm, __shfl_xor(lm, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) o[nb] *= alpha;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      // P^T operands of the two 32-token halves ks: tokens
      // {32 ks + 4(l/16)..+3, 32 ks + 16 + 4(l/16)..+3} of row l%16
      bf16x8 p[2];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sc[jt][r], sl2, -m_use));
          l_run += e;
          p[jt >> 1][4 * (jt & 1) + r] = (__bf16)e;
        }
      // O^T += V^T P^T, V^T read transposed from the values' blocks (the
      // second half's row groups sit 4 KB after the first's)
      const char* vt = tile + kAtKBytes;
      const int lv = fresh_lane();
      const uint32_t vb00 = vt_base(lv, 0, 0), vb01 = vt_base(lv, 0, 1);
      const uint32_t vb10 = vt_base(lv, 1, 0), vb11 = vt_base(lv, 1, 1);
      auto vload = [&](int n) {  // n = 2 nb + ks
        const int nb = n >> 1, ks = n & 1;
        const uint32_t cb = (uint32_t)((nb >> 2) * kAtCg + ks * 4096 + (nb & 3) * 256);
        return cat(lds_tr4(vt, cb + ((nb & 1) ? vb01 : vb00)), lds_tr4(vt, cb + ((nb & 1) ? vb11 : vb10)));
      };
      bf16x8 va = vload(0), vn = vload(1);
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        const bf16x8 vnn = n + 2 < 16 ? vload(n + 2) : vn;
        o[n >> 1] = mfma16(va, p[n & 1], o[n >> 1]);
        __builtin_amdgcn_sched_barrier(0);
        va = vn;
        vn = vnn;
      }
    }
    // this wave's fills of sub-tile s+1 landed (later ones may stay in flight)
    if (s + 1 < nsub) wait_vm(n_share * (pz - 1 - (s + 1)));
    block_sync();  // sub-tile s+1 complete for everyone; the slot of s free
  }
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) mfma_settle(o[nb]);

  // ---- outputs: o = O / l (0 where no token was visible), lse
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const int lw = fresh_lane();
  const int i = wrow0 + (lw & 15);
  if (active && i < Lq) {
    const int64_t row = ((int64_t)b * Lq + i) * H + h;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (a.lse && (lw >> 4) == 0) a.lse[row] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    uint16_t* orow = (uint16_t*)a.o + row * 128 + 4 * (lw >> 4);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const bf16x4 v4 = {(__bf16)(o[nb][0] * inv), (__bf16)(o[nb][1] * inv), (__bf16)(o[nb][2] * inv),
                         (__bf16)(o[nb][3] * inv)};
      *(bf16x4*)(orow + 16 * nb) = v4;
    }
  }
  }  // items
}

}  // namespace

// compute units of the current device, looked up once per device
static int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool prefill_supports(const mla_dims_t& d, int64_t row_stride, int max_seq_len) {
  return d.q_dtype == MLA_BF16 && d.kv_dtype == MLA_BF16 && d.d_nope == 128 && d.d_v == 128 &&
         d.d_rope == 64 && d.d_latent == 512 && row_stride % 8 == 0 && row_stride <= (1 << 16) &&
         (int64_t)d.heads * 256 * 32 < ((int64_t)1 << 31) && max_seq_len <= kAtMaxPages * kTile &&
         (int64_t)d.batch * ((max_seq_len + kExTok - 1) / kExTok) <= 65535 && d.heads <= 32767 &&
         // the work-order maps index all workgroups of a launch in 32 bits
         (int64_t)d.batch * d.heads * ((d.q_len + kAtRows - 1) / kAtRows) < ((int64_t)1 << 31);
}

hipError_t launch_prefill_expand(const mla_dims_t& d, const PrefillArgs& a, hipStream_t s) {
  PrefillArgs x = a;
  x.ntile = (a.max_seq_len + kExTok - 1) / kExTok;
  dim3 grid((unsigned)(2 * d.heads), (unsigned)(d.batch * x.ntile));
  hipLaunchKernelGGL(prefill_expand_kernel, grid, dim3(256), 0, s, x);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const mla_dims_t& d, const PrefillArgs& a, hipStream_t s) {
  // one persistent workgroup per compute unit (fewer when there are fewer items)
  const int64_t items = (int64_t)((d.q_len + kAtRows - 1) / kAtRows) * d.heads * d.batch;
  const int64_t cus = cu_count();
  const unsigned grid = (unsigned)(items < cus ? items : cus);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3(grid), dim3(1024), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
