// Split-K MLA decode for gfx950, latent 512 + RoPE 64, two kernels.
//
// Pages cited (title, section):
//   [ARCH] "Model Architecture Driving Inference Systems: From MHA/GQA to
//          DeepSeek MLA Matrix Absorption and Memory Minimalism"
//
// Query rows are (query i, head h) pairs, row i*H + h.  The cache is walked
// in 32-token sub-tiles, each staged once in LDS for all the workgroup's rows
// ([ARCH] 3.1: every head scores the same raw latent).
//
// decode_hs_kernel (bf16 cache): one workgroup = one split-K unit x 64 rows,
// 8 waves with fixed roles, the two roles working on consecutive sub-tiles:
//
//   scores   waves 0-3, wave v owns rows 16v..16v+15: S^T = K Q^T with
//            v_mfma_f32_16x16x32_bf16 (K = tile rows from LDS as A, the
//            wave's 18 k-slices of absorbed query in registers as B);
//            online softmax in log2 units with a lazy rescale; P (bf16) to
//            one of two LDS buffers.
//   values   waves 4-7, wave c owns latent columns 128c..128c+127 of all 64
//            rows: O[:, cols] += P V[:, cols] with v_mfma_f32_32x32x16_bf16
//            (P from LDS as A, V = the tile's latent part read transposed
//            with ds_read_b64_tr_b16 as B); they also issue the direct loads.
//
// decode_fp8_kernel (fp8 e4m3 cache with per-token scales): one workgroup =
// one split-K unit x 128 rows, every wave in both roles in turn (wave w
// scores rows 16w.. with 11 k-slices in registers and 7 in LDS, then sums
// latent columns 64w.. for all 128 rows); each staged sub-tile is first
// converted exactly to bf16 in LDS, and the scales enter the scores and P.
//
// Operand layouts:
//   16x16x32  A: lane l row l%16, k 8(l/16)..+7; B: column l%16, same k;
//             C: column l%16, rows 4(l/16)..+3
//   32x32x16  A: lane l row l%32, k 8(l/32)..+7; B: column l%32, same k;
//             C: column l%32, rows 8(r/4) + 4(l/32) + r%4, r = 0..15
// The order of k inside one MFMA is immaterial when A and B agree; P is
// stored so that each lane's 16-byte A operand holds tokens
// {16ks + 4hf + 0..3, 16ks + 8 + 4hf + 0..3}, the rows its two transposed V
// reads return.
//
// Sub-tile LDS layout (32 rows x 72 16-byte chunks = 36 KB): 1 KB blocks of
// 8 rows x 8 chunks, block (cg, rg) at (cg*4 + rg) KB; inside, row rho /
// chunk kappa at entry 8*(kappa ^ (rg&1)) + (rho ^ 4*((kappa ^ kappa>>1)&1)),
// which keeps the score reads and the transposed value reads free of bank
// conflicts.  Each block is one wave-wide direct global->LDS load.  Rings of
// 4 (bf16) and 3 (fp8 staging) sub-tiles keep two loads in flight.
//
// The loop is latency-bound before it is bandwidth-bound, so it avoids
// anything that stalls a wave on memory: the unit's tile descriptors
// (sequence, tokens left, first cache row) sit in the lanes of a VGPR window
// and are read with v_readlane; the waits on the direct loads are counted by
// hand; no register is spilled (a scratch reload would force a wait on every
// load in flight).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_common.hpp"
#include "decode_common.hpp"

namespace mla {
namespace {

using namespace mfma;
using namespace dec;

constexpr int kSub = 32;                       // tokens per LDS sub-tile
constexpr int kSubBytes = kSub * 576 * 2;      // 36864
constexpr int kRing = 3;
constexpr int kPPitch = 80;                    // bytes per row of P (32 bf16 + pad)
constexpr int kPBytes = 128 * kPPitch;         // 10240
constexpr int kF8Stage = 32 * 512 + 32 * 64 + 256;  // 18688: fp8 rows + scales

// LDS map of the fp8 kernel: the ring stages raw e4m3 rows and per-token
// scales, and one bf16 tile receives the exact conversion of the sub-tile in
// use.
struct LdsF8 {
  // k-slices of Q (32 columns each) kept in registers; the rest live in LDS
  static constexpr int kQReg = 11;
  static constexpr int kQLds = 18 - kQReg;
  static constexpr int kStage = kF8Stage;             // bytes per ring slot
  static constexpr int kConv = kRing * kStage;        // the converted tile
  static constexpr int kOffP = kConv + kSubBytes;
  static constexpr int kOffAlpha = kOffP + kPBytes;
  static constexpr int kOffL = kOffAlpha + 512;
  static constexpr int kOffFlag = kOffL + 512;
  static constexpr int kOffQ = kOffFlag + 128;
  static constexpr int kBytes = kOffQ + kQLds * 8192;  // 161664
};

// Next 32-token sub-tile: second half of the tile, or the next tile.
__device__ __forceinline__ void step_sub(int64_t& x, int& hh) {
  if (hh) {
    hh = 0;
    ++x;
  } else {
    hh = 1;
  }
}

// The direct loads of half hh of tile t (bf16 cache) into LDS at `dst`:
// wave w loads row group w&3, nine 1 KB blocks (block (cg, rg) = 4 cg + rg;
// cg 8 is the RoPE part).  Rows past the sequence end re-read its last row
// (poisoned page tails are never touched); an empty second half re-reads the
// first half's last row.
struct DmaPlan {
  const char* lat;
  const char* rop;
  uint32_t voff;
  uint32_t dst;
};

__device__ __forceinline__ DmaPlan plan_sub(const DecodeArgs& a, const TileInfo& t, int hh,
                                            uint32_t dst, int w, int lane) {
  const int in_page = min(kTile, t.rem);  // >= 1
  const int kappa = (lane >> 3) ^ (w & 1);
  const int rho = (lane & 7) ^ (4 * ((kappa ^ (kappa >> 1)) & 1));
  int r = 32 * hh + (w & 3) * 8 + rho;
  r = r < in_page ? r : in_page - 1;
  const int64_t stride = a.row_stride * 2;
  DmaPlan p;
  p.lat = (const char*)a.latent + t.row0 * stride;
  p.rop = (const char*)a.rope + t.row0 * stride;
  p.voff = (uint32_t)(r * stride) + (uint32_t)(kappa * 16);
  p.dst = dst;
  return p;
}

// fp8 cache: staging slot = latent rows (32 x 512 B) at 0, RoPE rows
// (32 x 64 B) at 16384, the 32 per-token scales (then repeated) at 18432.
// 19 wave loads per sub-tile: k < 16 latent rows 2k, 2k+1; k = 16, 17 RoPE
// rows 16(k-16)..+15; k = 18 the scales (4 bytes per lane).  Wave w issues
// k = w, w + 8, w + 16: waves 0-2 three loads, waves 3-7 two.
struct F8Plan {
  const char* lat;
  const char* rop;
  const float* scl;
  uint32_t voff[3];
  uint32_t dst;
};

__device__ __forceinline__ F8Plan plan_sub_f8(const DecodeArgs& a, const TileInfo& t, int hh,
                                              uint32_t dst, int w, int lane) {
  const int in_page = min(kTile, t.rem);  // >= 1
  const int64_t stride = a.row_stride;    // bytes
  F8Plan p;
  p.lat = (const char*)a.latent + t.row0 * stride;
  p.rop = (const char*)a.rope + t.row0 * stride;
  p.scl = a.kv_scale + t.row0;
  p.dst = dst;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int k = w + 8 * i;
    int r, col;
    if (k < 16) {
      r = 2 * k + (lane >> 5);
      col = lane & 31;
    } else if (k < 18) {
      r = 16 * (k - 16) + (lane >> 2);
      col = lane & 3;
    } else {
      r = lane & 31;
      col = 0;
    }
    r += 32 * hh;
    r = r < in_page ? r : in_page - 1;  // past the end: re-read the last row
    p.voff[i] = k < 18 ? (uint32_t)(r * stride) + (uint32_t)(col * 16) : (uint32_t)(r * 4);
  }
  return p;
}

__device__ __forceinline__ void issue_all_f8(const F8Plan& p, int w) {
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int k = w + 8 * i;
    if (k < 16)
      lds_dma16_stream(p.lat, p.voff[i], p.dst + (uint32_t)(k * 1024));
    else if (k < 18)
      lds_dma16_stream(p.rop, p.voff[i], p.dst + (uint32_t)(k * 1024));
    else if (k == 18)
      lds_dma4(p.scl, p.voff[i], p.dst + 18432u);
  }
}

// Exact e4m3 -> bf16 conversion of a staged sub-tile into the bf16 tile
// layout (every e4m3 value is a bf16 value, so the unit-scale hardware
// conversion is exact).  512 threads, 2304 chunks of 8: thread t takes chunks
// t + 512 i, i.e. row r0 + 7 i (+1 when the chunk index wraps) of 72 chunks.
__device__ __forceinline__ void convert_f8(const char* stage, char* tile, int tid) {
  int r = tid / 72, kap = tid - 72 * (tid / 72);
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    if (i < 4 || tid < 2304 - 4 * 512) {
      const uint2 raw = *(const uint2*)(stage + (kap < 64 ? r * 512 + kap * 8
                                                          : 16384 + r * 64 + (kap - 64) * 8));
      const bf16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.x, 1.0f, false);
      const bf16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.x, 1.0f, true);
      const bf16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.y, 1.0f, false);
      const bf16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)raw.y, 1.0f, true);
      const bf16x8 v = {v0.x, v0.y, v1.x, v1.y, v2.x, v2.y, v3.x, v3.y};
      const int cg = kap >> 3, kc = kap & 7, rg = r >> 3, rho = r & 7;
      const int entry = 8 * (kc ^ (rg & 1)) + (rho ^ (4 * ((kc ^ (kc >> 1)) & 1)));
      *(bf16x8*)(tile + (cg * 4 + rg) * 1024 + entry * 16) = v;
    }
    // next chunk: + 512 = 7 rows + 8 chunks
    r += 7;
    kap += 8;
    if (kap >= 72) {
      kap -= 72;
      r += 1;
    }
  }
}

// Per-lane LDS byte offsets of the operand reads, computed where they are
// used from fresh_lane().
// Score A operand inside a sub-tile.  Sub-tile blocks of 8 rows x 8 chunks:
// row rho / chunk kappa of block (cg, rg) at entry
// 8*(kappa ^ (rg&1)) + (rho ^ 4*((kappa ^ kappa>>1)&1)).
__device__ __forceinline__ uint32_t off_qk(int lane) {
  const int g = lane >> 4, li = lane & 15;
  const int g1 = (li >> 3) & 1;
  const int fq = (g ^ (g >> 1)) & 1;
  return (uint32_t)(g1 * 1024 + 128 * (g ^ g1) + 16 * ((lane & 7) ^ (4 * fq)));
}

// Value B operand: the two transposed 8-byte reads rd = 0, 1.
__device__ __forceinline__ uint32_t off_pv(int lane, int w, int rd) {
  const int li = lane & 15, hf = lane >> 5;
  const int ch = (lane >> 4) & 1, bq = (li & 3) >> 1;
  const int rho_v = 4 * hf + (li >> 2);
  return (uint32_t)(w * 4096 + rd * 1024 + 256 * ch + 128 * (bq ^ rd) +
                    16 * (rho_v ^ (4 * (bq ^ ch))) + 8 * (li & 1));
}

// This lane's P write and P (A operand) read.
__device__ __forceinline__ uint32_t off_pw(int lane, int w) {
  const int g = lane >> 4, li = lane & 15;
  return (uint32_t)((16 * w + li) * kPPitch + (g & 1) * 16 + (g >> 1) * 8);
}
__device__ __forceinline__ uint32_t off_pr(int lane) {
  return (uint32_t)((lane & 31) * kPPitch + (lane >> 5) * 16);
}

// Q k-slices held in LDS: rows of 64 B (row 16w + lane%16, chunk lane/16),
// 16-byte chunk c of row r stored at chunk c ^ ((r >> 1) & 3).
__device__ __forceinline__ uint32_t off_ql(int lane, int w) {
  const int g = lane >> 4, li = lane & 15;
  return (uint32_t)(LdsF8::kOffQ + (16 * w + li) * 64 + 16 * (g ^ ((li >> 1) & 3)));
}

__global__ __launch_bounds__(512, 1) void decode_fp8_kernel(DecodeArgs a) {
  using L = LdsF8;
  __shared__ __attribute__((aligned(1024))) char smem[L::kBytes];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, li = lane & 15;    // 16x16 operand coordinates
  const int hf = lane >> 5, n32 = lane & 31;  // 32x32 operand coordinates
  const int R = a.q_len * a.heads;
  const int rowg = blockIdx.y * 128;
  const int qrow0 = rowg + 16 * w;            // rows this wave scores
  const bool qk_active = qrow0 < R;
  const int qi = qk_active ? qrow0 / a.heads : 0;
  const int h0 = qk_active ? qrow0 % a.heads : 0;
  const int u = blockIdx.x;
  const int my_loads = w < 3 ? 3 : 2;  // direct loads per sub-tile

  int64_t x0, x1;  // this unit's tiles
  TileWin win;
  if (a.batch <= 64) {
    if (!unit_window_small(a, u, lane, x0, x1, win)) return;  // uniform across the workgroup
  } else {
    int64_t T, unused;
    wave_tile_sums(a.seq_lens, a.batch, 0, T, unused);
    T = uniform64(T);
    x0 = unit_begin(u, T, a.num_splits);
    x1 = unit_begin(u + 1, T, a.num_splits);
    if (x0 >= x1) return;  // uniform across the workgroup
    int b;
    int64_t pb;
    find_sequence(a.seq_lens, a.batch, x0, b, pb);
    build_window(a, x0, x1, __builtin_amdgcn_readfirstlane(b), uniform64(pb), lane, win);
  }

  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)smem;
  char* pbuf = smem + L::kOffP;
  float* alpha_buf = (float*)(smem + L::kOffAlpha);
  float* lbuf = (float*)(smem + L::kOffL);
  uint8_t* flags = (uint8_t*)(smem + L::kOffFlag);
  // issue the direct loads of (tile x, half hh) into ring slot `sl`
  auto issue = [&](const TileInfo& t, int hh, int sl, int lane_) {
    const uint32_t dst = lds0 + (uint32_t)(sl * L::kStage);
    issue_all_f8(plan_sub_f8(a, t, hh, dst, w, lane_), w);
  };
  const float sl2 = a.softmax_scale * kLog2e;

  // ---- prologue: sub-tiles 0 and 1 of the unit (a unit has >= 1 tile = 2 subs)
  const int64_t nsub = 2 * (x1 - x0);
  int64_t cx = x0, px = x0;  // tile of the sub-tile in use / next to issue
  int chh = 0, phh = 0;      // and its half
  issue(tile_info(win, px), phh, 0, lane);
  step_sub(px, phh);
  issue(tile_info(win, px), phh, 1, lane);
  step_sub(px, phh);

  constexpr int kQReg = L::kQReg;
  bf16x8 q[kQReg];
  f32x16 o[4][2];
  float m_run = -INFINITY, l_run = 0.f;
  bool new_seg = true;
  int slot = 0;

  for (int64_t y = 0; y < nsub; ++y) {
    const int ln = fresh_lane();
    const TileInfo ci = tile_info(win, cx);
    if (new_seg) {
      new_seg = false;
      {  // unconditional (inactive waves read row 0) so q is dead between segments
        const bf16x8* qp = (const bf16x8*)((const uint16_t*)a.q_abs +
                                            (((int64_t)ci.b * a.q_len + qi) * a.heads + h0 + li) * 576);
#pragma unroll
        for (int kk = 0; kk < kQReg; ++kk) q[kk] = qp[4 * kk + g];
#pragma unroll
        for (int kk = kQReg; kk < 18; ++kk)
          *(bf16x8*)(smem + off_ql(ln, w) + (kk - kQReg) * 8192) = qp[4 * kk + g];
      }
      wait_vm0();
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) o[mb][0] = o[mb][1] = f32x16{};
      m_run = -INFINITY;
      l_run = 0.f;
    }
    // sub-tile y has landed (the only newer loads are sub-tile y+1's)
    if (y + 1 < nsub)
      wait_vm(my_loads);
    else
      wait_vm(0);
    block_sync();  // visible to all; everyone also finished sub-tile y-1
    // the loads of sub-tile y+2, into the slot every wave finished with
    if (y + 2 < nsub) {
      const int s2 = slot + 2 >= kRing ? slot + 2 - kRing : slot + 2;
      if (px >= win.wx + win.wn)  // slide the window to start at the tile in use
        build_window(a, cx, x1, win.b0, win.pb0, ln, win);
      issue(tile_info(win, px), phh, s2, ln);
      step_sub(px, phh);
    }

    const char* stage = smem + slot * L::kStage;
    const bool has_tokens = 32 * chh < ci.rem;  // uniform: an empty second half does nothing
    if (has_tokens) {  // every wave converts its share, then all may read the tile
      int tid = (int)threadIdx.x;
      asm volatile("" : "+v"(tid));  // recompute the addresses, do not keep them live
      convert_f8(stage, smem + L::kConv, tid);
      block_sync();
    }
    const char* tile = smem + L::kConv;
    char* pb = pbuf;  // one P buffer: the barrier at the top of the next
                      // sub-tile orders its reuse after every wave's reads
    // visible tokens of this sub-tile: all up to the sequence end, or with
    // the causal mask those up to the query's own position
    int nv = ci.rem - 32 * chh - (a.causal ? a.q_len - 1 - qi : 0);
    nv = nv < 0 ? 0 : (nv > kSub ? kSub : nv);
    const bool scores = has_tokens && qk_active && nv > 0;  // uniform per wave
    if (has_tokens) {
      // ---------------- scores and softmax for this wave's 16 rows
      bf16x8 pw = bf16x8{};
      bool need = false;
      float alpha = 1.f;
      if (scores) {
        f32x4 s[2] = {f32x4{}, f32x4{}};
        constexpr int kPf = 2;
        const int lq = fresh_lane();
        const uint32_t o_qk = off_qk(lq), o_ql = off_ql(lq, w);
        bf16x8 ka[kPf + 1][2], qb[kPf + 1];
        auto kload = [&](int kk) {
          const int e = kk % (kPf + 1);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            ka[e][j] = *(const bf16x8*)(tile + (uint32_t)((kk >> 1) * 4096 + 2048 * j + 512 * (kk & 1)) + o_qk);
          if (kk >= kQReg) qb[e] = *(const bf16x8*)(smem + o_ql + (kk - kQReg) * 8192);
        };
#pragma unroll
        for (int kk = 0; kk < kPf; ++kk) kload(kk);
#pragma unroll
        for (int kk = 0; kk < 18; ++kk) {
          if (kk + kPf < 18) kload(kk + kPf);
          const int e = kk % (kPf + 1);
          const bf16x8 qk = kk < kQReg ? q[kk < kQReg ? kk : 0] : qb[e];
          s[0] = mfma16(ka[e][0], qk, s[0]);
          s[1] = mfma16(ka[e][1], qk, s[1]);
          __builtin_amdgcn_sched_barrier(0);
        }
        mfma_settle(s[0]);
        mfma_settle(s[1]);
        // the tokens' dequantisation scales
        const float* scl = (const float*)(stage + 18432);
        const f32x4 sc[2] = {*(const f32x4*)(scl + 4 * (ln >> 4)), *(const f32x4*)(scl + 16 + 4 * (ln >> 4))};
        s[0] *= sc[0];
        s[1] *= sc[1];
        if (nv < kSub) {  // mask the tokens past the visible end
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (16 * j + 4 * (ln >> 4) + r >= nv) s[j][r] = -INFINITY;
        }
        // this lane's max over its 8 scores, in log2 units
        const float lm = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                               fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3]))) * sl2;
        // Rescale only when some score passes its row's running max by more
        // than 2^8 (log2 units): the exponentials stay <= 256 and the final
        // normalisation uses the same reference max for numerator and
        // denominator.  Only then is the row max reduced across lanes.
        need = __ballot(lm > m_run + 8.f) != 0;
        if (need) {
          float mt = fmaxf(lm, __shfl_xor(lm, 16, 64));
          mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
          const float m_new = fmaxf(m_run, mt);
          alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
        }
        // exponent arguments are <= 8; results under 2^-126 flush to zero
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = __builtin_amdgcn_exp2f(fmaf(s[j][r], sl2, -m_use));
            l_run += e;
            // fp8: the value rows in LDS are unscaled, so P carries the scale
            pw[4 * j + r] = (__bf16)(e * sc[j][r]);
          }
      }
      // P rows of this wave's heads (zeros when it has nothing to score)
      {
        const uint32_t o_pw = off_pw(fresh_lane(), w);
        *(bf16x4*)(pb + o_pw) = __builtin_shufflevector(pw, pw, 0, 1, 2, 3);
        *(bf16x4*)(pb + o_pw + 32) = __builtin_shufflevector(pw, pw, 4, 5, 6, 7);
      }
      // every wave publishes its factors (1 when unchanged): a rescale reads all rows
      if ((ln >> 4) == 0) alpha_buf[16 * w + (ln & 15)] = alpha;
      if (lane == 0) flags[w] = need ? 1 : 0;
      block_sync();

      // ---------------- rescale (rare), then O[:, 64w..] += P V
      const uint64_t fl = *(const uint64_t*)flags;
      if (fl != 0) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          f32x16 a16;
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 a4 = *(const f32x4*)(alpha_buf + mb * 32 + 8 * r4 + 4 * (ln >> 5));
#pragma unroll
            for (int i = 0; i < 4; ++i) a16[4 * r4 + i] = a4[i];
          }
          o[mb][0] *= a16;
          o[mb][1] *= a16;
          __builtin_amdgcn_sched_barrier(0);  // one block's factors live at a time
        }
      }
      const int lv = fresh_lane();
      const uint32_t o_pr = off_pr(lv), o_pv0 = off_pv(lv, w, 0), o_pv1 = off_pv(lv, w, 1);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 pa[4], vb[2];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          pa[mb] = *(const bf16x8*)(pb + o_pr + (uint32_t)(mb * 32 * kPPitch + ks * 32));
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const uint32_t cb = (uint32_t)(2048 * ks + 512 * nb);
          vb[nb] = cat(lds_tr4(tile, cb + o_pv0), lds_tr4(tile, cb + o_pv1));
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) o[mb][nb] = mfma32(pa[mb], vb[nb], o[mb][nb]);
      }
    }


    // ---- end of this unit's part of the sequence: write the partial
    const bool last = y + 1 >= nsub || (chh == 1 && ci.rem <= kTile);
    if (last) {
      float l_tot = l_run + __shfl_xor(l_run, 16, 64);
      l_tot += __shfl_xor(l_tot, 32, 64);
      const int64_t sl = (int64_t)u + ci.b;
      if ((ln >> 4) == 0) {
        lbuf[16 * w + (ln & 15)] = l_tot;
        if (qk_active)
          a.lse_part[sl * R + qrow0 + (ln & 15)] =
              l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
      }
      block_sync();
      // fp16 partial rows of 1 KB; rows past R fall outside the resource
      // and are dropped
      const int rows_here = min(128, R - rowg);
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(
          (_Float16*)a.o_part + (sl * R + rowg) * 512, (uint32_t)rows_here * 1024u);
      const uint32_t vo = (uint32_t)((4 * hf * 512 + 64 * w + n32) * 2);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        f32x16 inv16;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 l4 = *(const f32x4*)(lbuf + mb * 32 + 8 * r4 + 4 * hf);
#pragma unroll
          for (int i = 0; i < 4; ++i) inv16[4 * r4 + i] = l4[i] > 0.f ? 1.f / l4[i] : 0.f;
        }
        const f32x16 v0 = o[mb][0] * inv16, v1 = o[mb][1] * inv16;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t so = (uint32_t)((mb * 32 + 8 * (r >> 2) + (r & 3)) * 1024);
          buffer_store_f16(v0[r], rs, vo, so);
          buffer_store_f16(v1[r], rs, vo + 64, so);
        }
      }
      new_seg = true;
    }
    step_sub(cx, chh);
    slot = slot + 1 >= kRing ? 0 : slot + 1;
  }
}


// ---------------------------------------------------------------------------
// bf16 cache, head-split kernel with specialised waves.  A workgroup takes
// 64 of the query rows (two workgroups per 128: the second one, 128 units
// later in launch order, runs on the same XCD and finds the tiles its sibling
// just read in L2).  Waves 0-3 only score: wave v holds all 18 k-slices of
// its 16 rows' absorbed query in registers and runs the online softmax;
// waves 4-7 only sum values (wave c: the 64 rows x latent columns
// 128c..128c+127) and issue the direct loads.  The roles overlap in time:
//
//   phase k   score waves: S, P of sub-tile k      value waves: P V of k-1,
//                                                  loads of sub-tile k+2
//
// with P, the rescale factors and the row totals double-buffered by sub-tile
// parity and a ring of four sub-tiles (k+2 loading, k+1 landed, k scored,
// k-1 summed).  Each role runs its own loop over the nsub + 1 phases with one
// barrier per phase, so a wave only keeps its own role's state live.
constexpr int kHsRows = 64;
constexpr int kHsRing = 4;
struct LdsHS {
  static constexpr int kPBuf = kHsRows * kPPitch;       // 5120
  static constexpr int kOffP = kHsRing * kSubBytes;     // 147456: two P buffers
  static constexpr int kOffAlpha = kOffP + 2 * kPBuf;   // 2 x 64 floats
  static constexpr int kOffInvL = kOffAlpha + 512;      // 2 x 64 floats: 1/l or 0
  static constexpr int kOffLse = kOffInvL + 512;        // 2 x 64 floats
  static constexpr int kOffFlag = kOffLse + 512;        // 2 x 4 bytes
  static constexpr int kBytes = kOffFlag + 64;          // 159296
};
static_assert(LdsHS::kBytes <= 163840, "LDS budget");

// All nine direct loads of row group (w & 3) of a sub-tile (value waves).
__device__ __forceinline__ void issue_rows(const DmaPlan& p, int w) {
  const uint32_t m0 = p.dst + (uint32_t)((w & 3) * 1024);
#pragma unroll
  for (int cg = 0; cg < 8; ++cg) lds_dma16_stream(p.lat, p.voff + cg * 128, m0 + cg * 4096);
  lds_dma16_stream(p.rop, p.voff, m0 + 8 * 4096);
}

// Load cg (0-7 latent, 8 RoPE) of row group (w & 3).
__device__ __forceinline__ void issue_cg(const DmaPlan& p, int w, int cg) {
  const uint32_t m0 = p.dst + (uint32_t)((w & 3) * 1024) + (uint32_t)(cg * 4096);
  if (cg < 8)
    lds_dma16_stream(p.lat, p.voff + cg * 128, m0);
  else
    lds_dma16_stream(p.rop, p.voff, m0);
}

__global__ __launch_bounds__(512, 1) void decode_hs_kernel(DecodeArgs a) {
  using L = LdsHS;
  __shared__ __attribute__((aligned(1024))) char smem[L::kBytes];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int R = a.q_len * a.heads;
  const int rowb = blockIdx.y * kHsRows;  // first query row of this workgroup
  const int u = blockIdx.x;

  int64_t x0, x1;  // this unit's tiles
  TileWin win;
  if (a.batch <= 64) {
    if (!unit_window_small(a, u, lane, x0, x1, win)) return;  // uniform across the workgroup
  } else {
    int64_t T, unused;
    wave_tile_sums(a.seq_lens, a.batch, 0, T, unused);
    T = uniform64(T);
    x0 = unit_begin(u, T, a.num_splits);
    x1 = unit_begin(u + 1, T, a.num_splits);
    if (x0 >= x1) return;  // uniform across the workgroup
    int b;
    int64_t pb;
    find_sequence(a.seq_lens, a.batch, x0, b, pb);
    build_window(a, x0, x1, __builtin_amdgcn_readfirstlane(b), uniform64(pb), lane, win);
  }

  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)smem;
  float* alpha_buf = (float*)(smem + L::kOffAlpha);
  float* invl_buf = (float*)(smem + L::kOffInvL);
  float* lse_buf = (float*)(smem + L::kOffLse);
  uint8_t* flags = (uint8_t*)(smem + L::kOffFlag);
  const int64_t nsub = 2 * (x1 - x0);  // a unit has >= 1 tile = 2 sub-tiles
  int64_t cx = x0;  // tile of this wave's current sub-tile
  int chh = 0;      // and its half

  if (w >= 4) {
    // ======================= value waves: loads, then O[:, 128c..] += P V
    const int c = w - 4;
    int64_t px = x0;  // next sub-tile to load
    int phh = 0;
    issue_rows(plan_sub(a, tile_info(win, px), phh, lds0, w, lane), w);
    step_sub(px, phh);
    issue_rows(plan_sub(a, tile_info(win, px), phh, lds0 + (uint32_t)kSubBytes, w, lane), w);
    step_sub(px, phh);
    wait_vm(9);
    block_sync();  // sub-tile 0 in LDS

    f32x16 o[2][4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) o[mb][nb] = f32x16{};

    for (int64_t k = 0; k <= nsub; ++k) {
      // the loads of sub-tile k+2, into the slot sub-tile k-2 used, go out
      // between the value MFMAs so that their issue stalls overlap them
      const bool more = k + 2 < nsub;
      DmaPlan plan{};
      int issued = more ? 0 : 9;
      if (more) {
        const int ln = fresh_lane();
        if (px >= win.wx + win.wn)  // slide the window to start at the tile in use
          build_window(a, cx, x1, win.b0, win.pb0, ln, win);
        plan = plan_sub(a, tile_info(win, px), phh, lds0 + (uint32_t)(((k + 2) & 3) * kSubBytes),
                        w, ln);
        step_sub(px, phh);
      }
      if (k >= 1) {  // sub-tile j = k-1, scored in the previous phase
        const int64_t j = k - 1;
        const int jb = (int)(j & 1);
        const TileInfo ci = tile_info(win, cx);
        const char* tile = smem + (int)(j & 3) * kSubBytes;
        const char* pb = smem + L::kOffP + jb * L::kPBuf;
        if (32 * chh < ci.rem) {
          const uint32_t fl = *(const uint32_t*)(flags + 4 * jb);
          if (fl != 0) {  // rare: some row moved its reference max
            const int lr = fresh_lane();
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
              f32x16 a16;
#pragma unroll
              for (int r4 = 0; r4 < 4; ++r4) {
                const f32x4 a4 = *(const f32x4*)(alpha_buf + 64 * jb + mb * 32 + 8 * r4 + 4 * (lr >> 5));
#pragma unroll
                for (int i = 0; i < 4; ++i) a16[4 * r4 + i] = a4[i];
              }
#pragma unroll
              for (int nb = 0; nb < 4; ++nb) o[mb][nb] *= a16;
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          // the RoPE block's load first, the eight latent blocks' between the
          // MFMAs (all nine at the top, or two per MFMA slot, measured slower)
          if (more) issue_cg(plan, w, 8);
          const int lv = fresh_lane();
          const uint32_t o_pr = off_pr(lv);
          const uint32_t o_pv0 = off_pv(lv, 2 * c, 0), o_pv1 = off_pv(lv, 2 * c, 1);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            bf16x8 pa[2], vb[4];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
              pa[mb] = *(const bf16x8*)(pb + o_pr + (uint32_t)(mb * 32 * kPPitch + ks * 32));
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
              const uint32_t cb = (uint32_t)(2048 * ks + 4096 * (nb >> 1) + 512 * (nb & 1));
              vb[nb] = cat(lds_tr4(tile, cb + o_pv0), lds_tr4(tile, cb + o_pv1));
            }
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
              if (more) issue_cg(plan, w, 4 * ks + nb);
#pragma unroll
              for (int mb = 0; mb < 2; ++mb) o[mb][nb] = mfma32(pa[mb], vb[nb], o[mb][nb]);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          issued = 9;
        }
        const bool last = j + 1 >= nsub || (chh == 1 && ci.rem <= kTile);
        if (last) {  // end of this unit's part of the sequence: write the partial
          const int64_t sl = (int64_t)u + ci.b;
          const int lw = fresh_lane();
          if ((lw >> 4) == 0 && rowb + 16 * c + (lw & 15) < R)
            a.lse_part[sl * R + rowb + 16 * c + (lw & 15)] = lse_buf[64 * jb + 16 * c + (lw & 15)];
          // fp16 partial rows of 1 KB; rows past R fall outside the resource
          // and are dropped
          const int rows_here = min(kHsRows, R - rowb);
          const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(
              (_Float16*)a.o_part + (sl * R + rowb) * 512, (uint32_t)rows_here * 1024u);
          const uint32_t vo = (uint32_t)((4 * (lw >> 5) * 512 + 128 * c + (lw & 31)) * 2);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            f32x16 inv16;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const f32x4 l4 = *(const f32x4*)(invl_buf + 64 * jb + mb * 32 + 8 * r4 + 4 * (lw >> 5));
#pragma unroll
              for (int i = 0; i < 4; ++i) inv16[4 * r4 + i] = l4[i];
            }
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
              const f32x16 vv = o[mb][nb] * inv16;
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const uint32_t so = (uint32_t)((mb * 32 + 8 * (r >> 2) + (r & 3)) * 1024);
                buffer_store_f16(vv[r], rs, vo + 64 * nb, so);
              }
              o[mb][nb] = f32x16{};
            }
          }
          wait_vm0();  // keeps the hand-counted load waits exact
        }
        step_sub(cx, chh);
      }
      for (int cg = issued; cg < 9; ++cg) issue_cg(plan, w, cg);  // the rest (all, without a value sum)
      if (k + 1 < nsub) wait_vm(more ? 9 : 0);  // sub-tile k+1 landed
      block_sync();
    }
  } else {
    // ======================= score waves: S = Q K^T, online softmax, P
    // Each SIMD runs one score wave and one value wave; the next phase waits
    // on this wave's P, so its instructions go first when both are ready.
    __builtin_amdgcn_s_setprio(3);
    const int qrow0 = rowb + 16 * w;  // rows this wave scores
    const bool qk_active = qrow0 < R;
    const int qi = qk_active ? qrow0 / a.heads : 0;
    const int h0 = qk_active ? qrow0 % a.heads : 0;
    const float sl2 = a.softmax_scale * kLog2e;
    bf16x8 q[18];
    float m_run = -INFINITY, l_run = 0.f;
    bool new_seg = true;
    block_sync();  // pairs with the value waves' first barrier

    for (int64_t k = 0; k <= nsub; ++k) {
      if (k < nsub) {
        int ln = fresh_lane();
        if (cx >= win.wx + win.wn) build_window(a, cx, x1, win.b0, win.pb0, ln, win);
        const TileInfo ci = tile_info(win, cx);
        if (new_seg) {
          new_seg = false;
          // unconditional (inactive waves read row 0) so q is dead between segments
          const int li = ln & 15, g = ln >> 4;
          const bf16x8* qp = (const bf16x8*)((const uint16_t*)a.q_abs +
                                              (((int64_t)ci.b * a.q_len + qi) * a.heads + h0 + li) * 576);
#pragma unroll
          for (int kk = 0; kk < 18; ++kk) q[kk] = qp[4 * kk + g];
          m_run = -INFINITY;
          l_run = 0.f;
        }
        const int kb = (int)(k & 1);
        const char* tile = smem + (int)(k & 3) * kSubBytes;
        const bool has_tokens = 32 * chh < ci.rem;  // uniform: an empty second half does nothing
        int nv = ci.rem - 32 * chh - (a.causal ? a.q_len - 1 - qi : 0);
        nv = nv < 0 ? 0 : (nv > kSub ? kSub : nv);
        const bool scores = has_tokens && qk_active && nv > 0;  // uniform per wave
        const bool last = k + 1 >= nsub || (chh == 1 && ci.rem <= kTile);
        if (has_tokens) {
          bf16x8 pw = bf16x8{};
          bool need = false;
          float alpha = 1.f;
          if (scores) {
            // token block j x k-slice parity: four accumulator chains
            f32x4 s[2][2] = {{f32x4{}, f32x4{}}, {f32x4{}, f32x4{}}};
            constexpr int kPf = 4;
            const uint32_t o_qk = off_qk(fresh_lane());
            bf16x8 ka[kPf + 1][2];
            auto kload = [&](int kk) {
              const int e = kk % (kPf + 1);
#pragma unroll
              for (int jt = 0; jt < 2; ++jt)
                ka[e][jt] = *(const bf16x8*)(tile + (uint32_t)((kk >> 1) * 4096 + 2048 * jt + 512 * (kk & 1)) + o_qk);
            };
#pragma unroll
            for (int kk = 0; kk < kPf; ++kk) kload(kk);
#pragma unroll
            for (int kk = 0; kk < 18; ++kk) {
              if (kk + kPf < 18) kload(kk + kPf);
              const int e = kk % (kPf + 1);
              s[0][kk & 1] = mfma16(ka[e][0], q[kk], s[0][kk & 1]);
              s[1][kk & 1] = mfma16(ka[e][1], q[kk], s[1][kk & 1]);
              __builtin_amdgcn_sched_barrier(0);
            }
            asm volatile("s_nop 15\n\ts_nop 7" : "+v"(s[0][0]), "+v"(s[0][1]), "+v"(s[1][0]), "+v"(s[1][1]));
            s[0][0] += s[0][1];
            s[1][0] += s[1][1];
            ln = fresh_lane();
            if (nv < kSub) {  // mask the tokens past the visible end
#pragma unroll
              for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (16 * jt + 4 * (ln >> 4) + r >= nv) s[jt][0][r] = -INFINITY;
            }
            // this lane's max over its 8 scores, in log2 units; the reference
            // max moves only when a score passes it by more than 2^8
            const float lm = fmaxf(fmaxf(fmaxf(s[0][0][0], s[0][0][1]), fmaxf(s[0][0][2], s[0][0][3])),
                                   fmaxf(fmaxf(s[1][0][0], s[1][0][1]), fmaxf(s[1][0][2], s[1][0][3]))) * sl2;
            need = __ballot(lm > m_run + 8.f) != 0;
            if (need) {
              float mt = fmaxf(lm, __shfl_xor(lm, 16, 64));
              mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
              const float m_new = fmaxf(m_run, mt);
              alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
              m_run = m_new;
              l_run *= alpha;
            }
            const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float e = __builtin_amdgcn_exp2f(fmaf(s[jt][0][r], sl2, -m_use));
                l_run += e;
                pw[4 * jt + r] = (__bf16)e;
              }
          }
          // P rows of this wave (zeros when it has nothing to score)
          char* pb = smem + L::kOffP + kb * L::kPBuf;
          const uint32_t o_pw = off_pw(fresh_lane(), w);
          *(bf16x4*)(pb + o_pw) = __builtin_shufflevector(pw, pw, 0, 1, 2, 3);
          *(bf16x4*)(pb + o_pw + 32) = __builtin_shufflevector(pw, pw, 4, 5, 6, 7);
          ln = fresh_lane();
          if ((ln >> 4) == 0) alpha_buf[64 * kb + 16 * w + (ln & 15)] = alpha;
          if (ln == 0) flags[4 * kb + w] = need ? 1 : 0;
        }
        if (last) {  // the segment's row totals, for the value waves
          float l_tot = l_run + __shfl_xor(l_run, 16, 64);
          l_tot += __shfl_xor(l_tot, 32, 64);
          ln = fresh_lane();
          if ((ln >> 4) == 0) {
            invl_buf[64 * kb + 16 * w + (ln & 15)] = l_tot > 0.f ? 1.f / l_tot : 0.f;
            lse_buf[64 * kb + 16 * w + (ln & 15)] =
                l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
          }
          new_seg = true;
        }
        step_sub(cx, chh);
      }
      block_sync();
    }
  }
}

}  // namespace

bool mfma_decode_supports(const mla_dims_t& d, int64_t row_stride, const void* latent,
                          const void* rope) {
  const int64_t row_bytes = row_stride * (d.kv_dtype == MLA_BF16 ? 2 : 1);
  return d.q_dtype == MLA_BF16 && (d.kv_dtype == MLA_BF16 || d.kv_dtype == MLA_FP8_E4M3) &&
         d.d_latent == 512 && d.d_rope == 64 && d.heads % 16 == 0 && row_bytes % 16 == 0 &&
         ((uintptr_t)latent & 15) == 0 && ((uintptr_t)rope & 15) == 0;
}

hipError_t launch_decode_mfma(const mla_dims_t& d, const DecodeArgs& a, hipStream_t s) {
  const int R = d.q_len * d.heads;
  if (d.kv_dtype == MLA_FP8_E4M3) {
    dim3 grid((unsigned)a.num_splits, (unsigned)((R + 127) / 128));
    hipLaunchKernelGGL(decode_fp8_kernel, grid, dim3(512), 0, s, a);
  } else {
    dim3 grid((unsigned)a.num_splits, (unsigned)((R + kHsRows - 1) / kHsRows));
    hipLaunchKernelGGL(decode_hs_kernel, grid, dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace mla
