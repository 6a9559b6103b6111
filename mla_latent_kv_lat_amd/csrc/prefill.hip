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
//   the 2H x 128 rows of W_UK and W_UV.  Workgroup = 256 tokens of one
//   sequence x one head's 256 k and v channels, 16 waves of 64 x 64 on
//   v_mfma_f32_32x32x16_bf16; both operands stream through a 4-stage LDS
//   ring in 32-wide k chunks (direct global->LDS loads), and the outputs
//   leave through LDS as whole 256-byte rows.
//
// prefill_attn_kernel: causal attention of the Lq prompt tokens of each
//   sequence over its keys [k_nope ; k_rope] (192 wide, the decoupled RoPE
//   key shared by the heads) and values (128 wide).  Persistent workgroups
//   (one per compute unit) take items of 256 query rows of one (sequence,
//   head), 8 waves of 32 rows; the keys and values of 64 tokens (one page)
//   at a time are filled into LDS once for all 256 rows (the decode
//   kernel's block layout).  Each wave computes S^T = K Q^T, the online
//   softmax and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16 with P fed from
//   the score registers, so every key and value operand read from LDS
//   serves 32 rows.
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

constexpr int kExTok = 256;                  // tokens per workgroup (four pages)
constexpr int kExCh = 256;                   // output channels: one head's k_nope and v
constexpr int kExKc = 32;                    // k per LDS chunk
constexpr int kExOpBytes = 256 * kExKc * 2;  // 16 KB: one operand's chunk
constexpr int kExStage = 2 * kExOpBytes;     // weights then latents
constexpr int kExRing = 4;                   // chunks kc .. kc+3
constexpr int kExPitch = 528;                // bytes per token row of the staged outputs
constexpr int kExBytes = kExTok * kExPitch > kExRing * kExStage ? kExTok * kExPitch : kExRing * kExStage;
static_assert(kExBytes <= 163840, "LDS budget");

// 1 KB LDS block j = rows 16j..16j+15 of 64 bytes (four 16-byte chunks of
// 8 k); row rho, chunk kappa at entry 4 rho + (kappa ^ ((rho >> 2) & 3)).
// A 32x32x16 operand read (one chunk of 32 rows) is served 16 lanes at a
// time; rows 4m..4m+3 fill the 64 banks once each.  The wave-wide fill
// writes lane e at entry e, so it loads chunk (e%4) ^ ((e/16) & 3).
__device__ __forceinline__ uint32_t ex_entry(int row, int kap) {
  return (uint32_t)(row * 64 + 16 * (kap ^ ((row >> 2) & 3)));
}

// One GEMM per (sequence, 256-token tile, head): C^T = [W_UK,h ; W_UV,h] X^T
// with X the tiles' cached latents (K = 512).  16 waves of 64 channels x 64
// tokens on v_mfma_f32_32x32x16_bf16; the outputs are staged in LDS as
// bf16 token rows and leave as 16-byte row pieces.
__global__ __launch_bounds__(1024) void prefill_expand_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kExBytes];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = a.heads;
  // Work order: workgroups reach the 8 XCDs round-robin by linear id, so
  // XCD x is given the contiguous item range x*N/8.. (xcd_item).  Items run
  // head-fastest within groups of HG heads, then token tiles, then groups:
  // the workgroups an XCD runs at once share a few token tiles' latents and
  // the group's HG x 256 KB of weights stay in its L2.
  const uint32_t T = (uint32_t)a.batch * (uint32_t)a.ntile;
  const uint32_t item = xcd_item(blockIdx.x, gridDim.x);
  const uint32_t HG = H % 8 == 0 ? 8 : (H % 4 == 0 ? 4 : (H % 2 == 0 ? 2 : 1));
  const uint32_t rest = item / HG, tile = rest % T;
  const int h = (int)((rest / T) * HG + item % HG);
  const int b = (int)(tile / a.ntile);
  const int t0 = (int)(tile % a.ntile) * kExTok;
  const int len = a.seq_lens[b];
  if (t0 >= len) return;  // uniform across the workgroup
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)smem;

  // fills: per chunk, wave w loads weight rows 16w.. (block w) and token
  // rows 16w.. (block w); the token block lies in one page
  const int fr = lane >> 2;                       // row in the block
  const int fk = (lane & 3) ^ ((lane >> 4) & 3);  // chunk this lane loads
  // weight rows 16w.. = output channels: W_UK,h rows for w < 8, W_UV,h after
  const uint16_t* wsrc = (w < 8 ? a.w_uk : a.w_uv) + ((int64_t)h * 128 + ((16 * w) & 127)) * 512;
  const int tb = min(t0 + 16 * w, len - 1);       // the block's rows, clamped to the last token
  const int64_t prow = a.block_table ? (int64_t)a.block_table[(int64_t)b * a.mbps + (tb >> 6)] * kTile
                                     : (int64_t)b * a.max_seq_len + (tb & ~(kTile - 1));
  const int tl = min(t0 + 16 * w + fr, len - 1) - (tb & ~(kTile - 1));
  const char* xbase = (const char*)a.latent + prow * a.row_stride * 2;
  const uint32_t xoff = (uint32_t)(tl * a.row_stride * 2) + (uint32_t)(fk * 16);
  const uint32_t woff = (uint32_t)(fr * 1024 + fk * 16);
  auto issue = [&](int kc) {
    const uint32_t dst = lds0 + (uint32_t)((kc % kExRing) * kExStage + w * 1024);
    lds_dma16((const char*)wsrc, woff + (uint32_t)(kc * kExKc * 2), dst);
    lds_dma16((const char*)uniform64((int64_t)xbase), xoff + (uint32_t)(kc * kExKc * 2), dst + kExOpBytes);
  };

  const int wch = w & 3, wtk = w >> 2;  // wave tile: channels 64 wch.., tokens 64 wtk..
  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = f32x16{};

  // operands of k-step half kh (16 k) of chunk kc
  auto kread = [&](int kc, int kh, bf16x8 (&wv)[2], bf16x8 (&xv)[2]) {
    const char* Wm = smem + (kc % kExRing) * kExStage;
    const char* Xm = Wm + kExOpBytes;
    const int lr = fresh_lane();
    const int l32 = lr & 31, kap = 2 * kh + (lr >> 5);
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) wv[mi] = *(const bf16x8*)(Wm + ex_entry(64 * wch + 32 * mi + l32, kap));
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) xv[ni] = *(const bf16x8*)(Xm + ex_entry(64 * wtk + 32 * ni + l32, kap));
  };
  auto kmul = [&](const bf16x8 (&wv)[2], const bf16x8 (&xv)[2]) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma32(wv[mi], xv[ni], acc[mi][ni]);
  };

  // The operands of the next k-step are read while the current one
  // multiplies; a chunk's barrier comes right after its predecessor's last
  // products are issued, so the matrix cores stay busy across it.  After
  // the barrier for chunk m every wave has read chunk m-1 into registers,
  // and chunk m+3 goes into its stage.
  constexpr int kChunks = 512 / kExKc;
#pragma unroll
  for (int kc = 0; kc < kExRing; ++kc) issue(kc);
  wait_vm(2 * (kExRing - 1));  // this wave's loads of chunk 0 landed
  block_sync();
  bf16x8 cw[2], cx[2], nw[2], nx[2];
  kread(0, 0, cw, cx);
  for (int kc = 0; kc < kChunks; ++kc) {
    kread(kc, 1, nw, nx);
    kmul(cw, cx);
    // chunk kc+3 into the stage of kc-1 (read by everyone before the last
    // barrier); issued once products are queued, so that the wait for a
    // free slot in the load queue overlaps them
    __builtin_amdgcn_sched_barrier(0);
    if (kc >= 1 && kc + kExRing - 1 < kChunks) issue(kc + kExRing - 1);
    kmul(nw, nx);
    __builtin_amdgcn_sched_barrier(0);  // the products go out before the wait and the barrier
    if (kc + 1 < kChunks) {
      const int m = kc + 1;
      const int later = min(2, kChunks - 1 - m);  // chunks after m already issued
      if (later == 2) wait_vm(4); else if (later == 1) wait_vm(2); else wait_vm(0);
      block_sync();  // chunk m complete for everyone; chunk m-1 read by everyone
      kread(m, 0, cw, cx);
    }
  }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) mfma_settle(acc[mi][ni]);
  block_sync();  // every wave's last operand reads done: the ring becomes the staging area

  // C^T (32 x 32): lane l holds token l%32 and channels 8(r/4) + 4(l/32) + r%4
  {
    const int ls = fresh_lane();
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int tok = 64 * wtk + 32 * ni + (ls & 31);
          const int ch = 64 * wch + 32 * mi + 8 * g4 + 4 * (ls >> 5);
          const bf16x4 v4 = {(__bf16)acc[mi][ni][4 * g4], (__bf16)acc[mi][ni][4 * g4 + 1],
                             (__bf16)acc[mi][ni][4 * g4 + 2], (__bf16)acc[mi][ni][4 * g4 + 3]};
          *(bf16x4*)(smem + tok * kExPitch + ch * 2) = v4;
        }
  }
  block_sync();
  // token rows out: 32 pieces of 16 bytes per token (16 of k_nope, 16 of v)
  const int64_t T2 = a.max_seq_len;
#pragma unroll
  for (int j = 0; j < kExTok * 32 / 1024; ++j) {
    const int e = (int)threadIdx.x + 1024 * j;
    const int tk = e >> 5, cc = e & 31;
    if (t0 + tk < len) {
      const uint4 v = *(const uint4*)(smem + tk * kExPitch + cc * 16);
      char* dst = (char*)(cc < 16 ? a.k_nope : a.v) + (((int64_t)b * T2 + t0 + tk) * H + h) * 256 + (cc & 15) * 16;
      *(uint4*)dst = v;
    }
  }
}

// --------------------------------------------------------------- attention

constexpr int kAtWaves = 8;
constexpr int kAtRows = 32 * kAtWaves;          // 256 query rows per workgroup
constexpr int kAtThreads = 64 * kAtWaves;
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

__global__ __launch_bounds__(kAtThreads) void prefill_attn_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kAtBytes];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = a.heads, Lq = a.q_len;
  const int nqb = (Lq + kAtRows - 1) / kAtRows;
  const int64_t Tmax = a.max_seq_len;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)smem;
  int* prow = (int*)(smem + kAtPageOff);  // block id (paged) of each page of the item

  // RoPE frequencies base^(-2p/64) of the 32 pairs, once
  double* theta = (double*)(smem + kAtThetaOff);
  if (threadIdx.x < 32) theta[threadIdx.x] = exp2(-2.0 * (int)threadIdx.x / 64.0 * log2((double)a.rope_base));
  block_sync();

  // Persistent workgroups, one per compute unit.  An item is a pair of
  // query blocks of one (sequence, head), p and nqb-1-p, whose causal
  // ranges add up to the same length for every p, so all items cost the
  // same when the sequences do.  The items, those of a head consecutive,
  // are cut into P = min(8, grid) contiguous ranges; workgroup g takes
  // range g % P, which is its XCD's when the grid is a multiple of 8
  // (workgroups reach the XCDs round-robin), and its nx workgroups deal the
  // range out in rounds of nx items.  Equal items keep the workgroups of an
  // XCD in step, so the blocks of the few heads they work on share its L2.
  const uint32_t npair = (uint32_t)(nqb + 1) / 2;
  const uint32_t n_items = npair * (uint32_t)H * (uint32_t)a.batch;
  const uint32_t G = gridDim.x, g = blockIdx.x;
  const uint32_t P = G < 8 ? G : 8, pi = g % P, rank = g / P, nx = (G - pi + P - 1) / P;
  const uint32_t cnt = n_items / P + (pi < n_items % P ? 1u : 0u);
  const uint32_t beg = pi * (n_items / P) + min(pi, n_items % P);

  int table_b = -1;  // sequence whose page table is in LDS
  for (uint32_t rd = 0;; ++rd) {
  const uint32_t loc = rd * nx + rank;
  if (loc >= cnt) break;  // uniform
  const uint32_t item = beg + loc;
  const int pr = (int)(item % npair);
  const int h = (int)((item / npair) % (uint32_t)H), b = (int)(item / (npair * (uint32_t)H));
  for (int half = 0; half < 2; ++half) {
  const int qb = half == 0 ? nqb - 1 - pr : pr;  // the longer causal range first
  if (half == 1 && qb == nqb - 1 - pr) break;    // odd nqb: the middle block once
  const int len = a.seq_lens[b];
  const int i0 = qb * kAtRows;

  // visible tokens of query i: t < len - Lq + i + 1 (causal) or t < len
  auto n_vis = [&](int i) { return a.causal ? len - Lq + i + 1 : len; };
  const int i_last = min(Lq, i0 + kAtRows) - 1;
  const int n_end = min(len, max(0, n_vis(i_last)));  // tokens the workgroup reads
  const int nsub = (n_end + kAtSub - 1) / kAtSub;

  // rows of this wave; lane l holds row i0 + 32w + l%32
  const int wrow0 = i0 + 32 * w;
  const bool active = wrow0 < Lq;  // uniform per wave
  const int wave_vis = active ? min(len, max(0, n_vis(min(wrow0 + 31, Lq - 1)))) : 0;

  // page table of the whole sequence, when it changes (consecutive items
  // mostly share the sequence).  The previous block's last barrier already
  // ended every wave's use of the ring, so with the table in place the
  // first fills can go out at once.
  if (a.block_table && b != table_b) {
    const int npg = (len + kTile - 1) / kTile;
    for (int pg = (int)threadIdx.x; pg < npg; pg += kAtThreads) prow[pg] = a.block_table[(int64_t)b * a.mbps + pg];
    table_b = b;
    block_sync();
  }

  // ---- fills: 40 blocks of 1 KB per sub-tile (keys: column groups 0-1
  // k_nope, 2 the RoPE key; values: 0-1; 8 row groups each); wave w issues
  // blocks w + 8i, all of row group w
  constexpr int n_share = 5;
  const int rg = w;
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
    for (int i = 0; i < n_share; ++i) {
      const int k = w + 8 * i;
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

  // ---- the wave's query rows as the B operand of the score products: lane
  // l holds row l%32 and, for k-step k (16 dims), dims 16k + 8(l/32)..+7:
  // q_nope for k < 8, RoPE(q_rope) for k = 8..11
  bf16x8 q[12];
  {
    const int fl = fresh_lane();
    const int li = fl & 31, hq = fl >> 5;
    const int i = min(wrow0 + li, Lq - 1);
    const int64_t qrow = ((int64_t)b * Lq + i) * H + h;
    const bf16x8* qn = (const bf16x8*)((const uint16_t*)a.q_nope + qrow * 128);
#pragma unroll
    for (int k = 0; k < 8; ++k) q[k] = qn[2 * k + hq];
    const bf16x8* qr = (const bf16x8*)((const uint16_t*)a.q_rope + qrow * 64);
    const double pos = (double)a.positions[(int64_t)b * Lq + i];
#pragma unroll
    for (int k = 8; k < 12; ++k) {
      const int un = 2 * (k - 8) + hq;  // 8-dim unit of q_rope
      const bf16x8 x = qr[un];
      bf16x8 y;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        // pair p = 4 un + m turns by pos * base^(-2p/64); the angle is
        // reduced modulo 2 pi in double, sin/cos in single
        double ang = pos * theta[4 * un + m];
        ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
        float sn, cs;
        __sincosf((float)ang, &sn, &cs);
        const float x0 = (float)x[2 * m], x1 = (float)x[2 * m + 1];
        y[2 * m] = (__bf16)(x0 * cs - x1 * sn);
        y[2 * m + 1] = (__bf16)(x0 * sn + x1 * cs);
      }
      q[k] = y;
    }
    // taken here: the compiler's waits for the query (it does not count
    // the direct loads issued before them) then also cover sub-tiles 0-1
#pragma unroll
    for (int k = 0; k < 12; ++k) asm volatile("" ::"v"(q[k]));
  }
  if (nsub > 0) wait_vm(n_share * (pz - 1));
  block_sync();

  f32x16 o[4];  // O^T tile ct: value columns 32 ct + 8(r/4) + 4(l/32) + r%4 of row l%32
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) o[ct] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.softmax_scale * kLog2e;

  for (int s = 0; s < nsub; ++s) {
    if (s + kAtRing - 1 < nsub) issue();  // into the slot every wave finished with
    const char* tile = smem + (s % kAtRing) * kAtSubBytes;
    const int t0 = s * kAtSub;
    if (active && t0 < wave_vis) {  // uniform per wave
      // ---- S^T = K Q^T on v_mfma_f32_32x32x16_bf16, two 32-token tiles jt:
      // lane l ends with row l%32 and tokens 32 jt + 8(r/4) + 4(l/32) + r%4
      f32x16 sc[2] = {f32x16{}, f32x16{}};
      {
        const int lk = fresh_lane();
        const int tk = lk & 31, hk = lk >> 5, rgk = tk >> 3, rhk = tk & 7;
        // K operand of k-step k, tile jt: token 32 jt + tk, dims 16k + 8hk..+7,
        // at kb[k % 4] + (k / 4) * 8 KB + jt * 4 KB
        uint32_t kb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kap = 2 * j + hk;
          kb[j] = (uint32_t)(rgk * 1024 + 16 * (8 * (kap ^ (rgk & 1)) + (rhk ^ (4 * ((kap ^ (kap >> 1)) & 1)))));
        }
        auto kaddr = [&](int k, int jt) { return kb[k & 3] + (uint32_t)((k >> 2) * kAtCg + jt * 4096); };
        constexpr int kPf = 2;
        bf16x8 ka[kPf + 1][2];
#pragma unroll
        for (int k = 0; k < kPf; ++k)
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) ka[k][jt] = *(const bf16x8*)(tile + kaddr(k, jt));
#pragma unroll
        for (int k = 0; k < 12; ++k) {
          if (k + kPf < 12)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) ka[(k + kPf) % (kPf + 1)][jt] = *(const bf16x8*)(tile + kaddr(k + kPf, jt));
#pragma unroll
          for (int jt = 0; jt < 2; ++jt) sc[jt] = mfma32(ka[k % (kPf + 1)][jt], q[k], sc[jt]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      const int ln = fresh_lane();
      const int hk = ln >> 5;
      const int nv = min(len, n_vis(wrow0 + (ln & 31)));  // this lane's row
      if (t0 + kAtSub > nv) {  // mask past the visible end
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (t0 + 32 * jt + 8 * (r >> 2) + 4 * hk + (r & 3) >= nv) sc[jt][r] = -INFINITY;
      }
      // lazy rescale: the reference max moves only when a score passes it
      // by more than 2^8 (log2 units); a row's scores sit in lanes l, l^32
      float lm = sc[0][0];
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int r = 0; r < 16; ++r) lm = fmaxf(lm, sc[jt][r]);
      lm *= sl2;
      if (__ballot(lm > m_run + 8.f) != 0) {
        const float mt = fmaxf(lm, __shfl_xor(lm, 32, 64));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) o[ct] *= alpha;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      // P^T operand of value k-step ks (16 tokens): registers 8(ks%2)..+7 of
      // tile ks/2, i.e. tokens 16 ks + 4(l/32) + {0..3, 8..11}
      bf16x8 p[4];
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sc[jt][r], sl2, -m_use));
          l_run += e;
          p[2 * jt + (r >> 3)][r & 7] = (__bf16)e;
        }
      // ---- O^T += V^T P^T: V^T (32 columns x 16 tokens) read transposed.
      // Lane l (G = l/16, i = l%16) names token 16 ks + 8 sub + 4(G/2) + i/4
      // and columns 32 ct + 16(G&1) + 4(i%4)..+3, and then holds column
      // 32 ct + l%32 and 4 consecutive tokens; the address is
      // vb[ct % 2][sub] + (ct / 2) * 8 KB + ks * 2 KB.
      const char* vt = tile + kAtKBytes;
      const int lv = fresh_lane();
      const int G = lv >> 4, i16 = lv & 15;
      uint32_t vb[2][2];
#pragma unroll
      for (int par = 0; par < 2; ++par)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const int kap = 4 * par + 2 * (G & 1) + ((i16 & 3) >> 1);
          const int rho = 4 * (G >> 1) + (i16 >> 2);
          vb[par][sub] = (uint32_t)(sub * 1024 + 16 * (8 * (kap ^ sub) + (rho ^ (4 * ((kap ^ (kap >> 1)) & 1)))) +
                                    8 * (i16 & 1));
        }
      auto vload = [&](int n) {  // n = 4 ks + ct
        const int ks = n >> 2, ct = n & 3;
        const uint32_t off = (uint32_t)((ct >> 1) * kAtCg + ks * 2048);
        return cat(lds_tr4(vt, vb[ct & 1][0] + off), lds_tr4(vt, vb[ct & 1][1] + off));
      };
      bf16x8 va = vload(0), vn = vload(1);
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        const bf16x8 vnn = n + 2 < 16 ? vload(n + 2) : vn;
        o[n & 3] = mfma32(va, p[n >> 2], o[n & 3]);
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
  for (int ct = 0; ct < 4; ++ct) mfma_settle(o[ct]);

  // ---- outputs: o = O / l (0 where no token was visible), lse
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const int lw = fresh_lane();
  const int i = wrow0 + (lw & 31);
  if (active && i < Lq) {
    const int64_t row = ((int64_t)b * Lq + i) * H + h;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (a.lse && (lw >> 5) == 0) a.lse[row] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
    uint16_t* orow = (uint16_t*)a.o + row * 128 + 4 * (lw >> 5);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x4 v4 = {(__bf16)(o[ct][4 * g] * inv), (__bf16)(o[ct][4 * g + 1] * inv),
                           (__bf16)(o[ct][4 * g + 2] * inv), (__bf16)(o[ct][4 * g + 3] * inv)};
        *(bf16x4*)(orow + 32 * ct + 8 * g) = v4;
      }
  }
  }  // the pair's two blocks
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
         d.heads <= 32767 &&
         // the work-order maps index all workgroups of a launch in 32 bits
         (int64_t)d.batch * d.heads * ((max_seq_len + kExTok - 1) / kExTok) < ((int64_t)1 << 31) &&
         (int64_t)d.batch * d.heads * ((d.q_len + kAtRows - 1) / kAtRows) < ((int64_t)1 << 31);
}

hipError_t launch_prefill_expand(const mla_dims_t& d, const PrefillArgs& a, hipStream_t s) {
  PrefillArgs x = a;
  x.ntile = (a.max_seq_len + kExTok - 1) / kExTok;
  const int64_t n = (int64_t)d.heads * d.batch * x.ntile;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_expand_kernel, dim3((unsigned)n), dim3(1024), 0, s, x);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const mla_dims_t& d, const PrefillArgs& a, hipStream_t s) {
  // one persistent workgroup per compute unit (fewer when there are fewer items)
  const int64_t items = (int64_t)((d.q_len + kAtRows - 1) / kAtRows + 1) / 2 * d.heads * d.batch;
  const int64_t cus = cu_count();
  const unsigned grid = (unsigned)(items < cus ? items : cus);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3(grid), dim3(kAtThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
