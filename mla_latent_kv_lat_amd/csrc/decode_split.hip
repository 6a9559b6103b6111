// Split-K MLA decode for gfx950, latent 512 + RoPE 64.
//
// Pages cited (title, section):
//   [ARCH] "Model Architecture Driving Inference Systems: From MHA/GQA to
//          DeepSeek MLA Matrix Absorption and Memory Minimalism"
//   [MATH] "Multi-Head Latent Attention (MLA): Mathematical Foundations, ..."
//          (section on high-throughput serving kernels: fp8 latent cache)
//
// Query rows are (query i, head h) pairs, row i*H + h.  The cache is walked
// in 32-token sub-tiles, each staged once in LDS for all the workgroup's rows
// ([ARCH] 3.1: every head scores the same raw latent).  The kernel computes
// in fp16: the absorbed query arrives in fp16, and the staged cache rows are
// converted exactly to fp16 in LDS (every bf16 value of magnitude 2^-17 ..
// 65504 and every e4m3 value is an fp16 value), so scores against long
// contexts with large cached values keep the query's 11-bit significand.
//
// decode_sf_kernel<F8>: one workgroup = one split-K unit x 128 rows, 8
// waves, each owning 16 rows for both products (see the kernel).  bf16
// cache: the sub-tiles land in a 4-slot ring and are converted in place,
// each wave converting the rows it loaded.  fp8 e4m3 cache with per-token
// fp32 scales ([MATH]): the raw rows of 4 sub-tiles are staged, and all 512
// threads convert the next one into one of 2 fp16 slots; the scales multiply
// the scores and ride in P for the value product.
//
// Operand layouts:
//   16x16x32  A: lane l row l%16, k 8(l/16)..+7; B: column l%16, same k;
//             C: column l%16, rows 4(l/16)..+3
//   32x32x16  A: lane l row l%32, k 8(l/32)..+7; B: column l%32, same k;
//             C: column l%32, rows 8(r/4) + 4(l/32) + r%4, r = 0..15
// The order of k inside one MFMA is immaterial when A and B agree.
//
// Sub-tile LDS layout (32 rows x 72 16-byte chunks = 36 KB): 1 KB blocks of
// 8 rows x 8 chunks, block (cg, rg) at (cg*4 + rg) KB; inside, row rho /
// chunk kappa at entry 8*(kappa ^ (rg&1)) + (rho ^ 4*((kappa ^ kappa>>1)&1)),
// which keeps the score reads and the transposed value reads free of bank
// conflicts.  Each block is one wave-wide direct global->LDS load.
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
constexpr int kF8Stage = 32 * 512 + 32 * 64 + 256;  // 18688: fp8 rows + scales

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

// Exact e4m3 -> fp16 conversion of a staged sub-tile into the tile layout
// (every e4m3 value is an fp16 value, so the unit-scale hardware conversion
// is exact).  512 threads, 2304 chunks of 8: thread t takes chunks
// t + 512 i, i.e. row r0 + 7 i (+1 when the chunk index wraps) of 72 chunks.
__device__ __forceinline__ void convert_f8(const char* stage, char* tile, int tid) {
  int r = tid / 72, kap = tid - 72 * (tid / 72);
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    if (i < 4 || tid < 2304 - 4 * 512) {
      const uint2 raw = *(const uint2*)(stage + (kap < 64 ? r * 512 + kap * 8
                                                          : 16384 + r * 64 + (kap - 64) * 8));
      const f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)raw.x, 1.0f, false);
      const f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)raw.x, 1.0f, true);
      const f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)raw.y, 1.0f, false);
      const f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)raw.y, 1.0f, true);
      const f16x8 v = {v0.x, v0.y, v1.x, v1.y, v2.x, v2.y, v3.x, v3.y};
      const int cg = kap >> 3, kc = kap & 7, rg = r >> 3, rho = r & 7;
      const int entry = 8 * (kc ^ (rg & 1)) + (rho ^ (4 * ((kc ^ (kc >> 1)) & 1)));
      *(f16x8*)(tile + (cg * 4 + rg) * 1024 + entry * 16) = v;
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

// ---------------------------------------------------------------------------
// bf16 cache, single-fill kernel.  One workgroup per split-K unit holds a
// block of 128 query rows, so every 32-token sub-tile is loaded into LDS
// once for all of them ([ARCH] 3.1: every head scores the same raw latent).
// Each of the 8 waves owns 16 rows for the whole walk:
//
//   scores  S^T = K Q^T on v_mfma_f32_16x16x32_f16 (K from LDS as A, the
//           wave's 18 k-slices of fp16 query in registers as B); lane l
//           holds row l%16 and tokens 4(l/16)..+3 of each 16-token block;
//           online softmax in log2 units with a lazy rescale;
//   values  O^T += V^T P^T on the same instruction: V^T (16 latent columns
//           x 32 tokens) read transposed from LDS with ds_read_b64_tr_b16 as
//           A, and P^T straight from the score registers as B (the k order
//           of one MFMA only has to agree between A and B: lane l supplies
//           tokens {4(l/16)..+3, 16+4(l/16)..+3}, the two transposed reads
//           return the same tokens).  Lane l accumulates row l%16, so the
//           rescale factor and 1/l are per-lane scalars.
//
// Waves never exchange data; they meet at one barrier per sub-tile, after
// which the next sub-tile is complete in LDS and the oldest ring slot is
// free.  In the value part of sub-tile s each wave issues its share of the
// direct loads of sub-tile s+3 (row group w&3; column groups 0-4 for waves
// 0-3, 5-8 for waves 4-7) and converts, bf16 -> fp16 in place, the chunks
// it loaded of sub-tile s+1 after waiting for them itself: waves 0-3 after
// their value part, waves 4-7 before their score part (measured 2-5%
// faster than both at the end).
constexpr int kSfRows = 128;
constexpr int kSfRing = 4;
constexpr int kSfSplit = 5;      // column groups [0, 5) loaded by waves 0-3, [5, 9) by waves 4-7
constexpr int kSfKPrefetch = 2;  // K operands read ahead of the score MFMAs
constexpr int kSfBytes = kSfRing * kSubBytes;  // 147456
static_assert(kSfBytes <= 163840, "LDS budget");
// fp8: 2 converted sub-tiles, 4 staged raw sub-tiles, 2 x 32 token scales
constexpr int kSf8Stage0 = 2 * kSubBytes;
constexpr int kSf8Scale0 = kSf8Stage0 + 4 * kF8Stage;
constexpr int kSf8Bytes = kSf8Scale0 + 256;  // 148736
static_assert(kSf8Bytes <= 163840, "LDS budget");

// Load cg (0-7 latent, 8 RoPE) of row group (w & 3).
__device__ __forceinline__ void issue_cg(const DmaPlan& p, int w, int cg) {
  const uint32_t m0 = p.dst + (uint32_t)((w & 3) * 1024) + (uint32_t)(cg * 4096);
  if (cg < 8)
    lds_dma16_stream(p.lat, p.voff + cg * 128, m0);
  else
    lds_dma16_stream(p.rop, p.voff, m0);
}

// Two bf16 values -> fp16 (exact for magnitudes 2^-17 .. 65504; the
// round-toward-zero conversion saturates larger ones at 65504).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t d) {
  typedef __fp16 fp16x2_t __attribute__((ext_vector_type(2)));
  const fp16x2_t h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(d << 16), __uint_as_float(d & 0xffff0000u));
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 c) {
  return make_uint4(bf16x2_to_f16x2(c.x), bf16x2_to_f16x2(c.y), bf16x2_to_f16x2(c.z),
                    bf16x2_to_f16x2(c.w));
}

template <bool F8>
__global__ __launch_bounds__(512, 1) void decode_sf_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[F8 ? kSf8Bytes : kSfBytes];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int R = a.q_len * a.heads;
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
  const int64_t nsub = 2 * (x1 - x0);  // a unit has >= 1 tile = 2 sub-tiles
  const int cg0 = w < 4 ? 0 : kSfSplit, cg1 = w < 4 ? kSfSplit : 9;
  // direct loads per sub-tile of this wave (fp8: loads k = w, w + 8, w + 16 of 19)
  const int n_share = F8 ? (w < 3 ? 3 : 2) : cg1 - cg0;
  // bf16: ring of 4 sub-tiles converted in place.  fp8: the raw rows of 4
  // sub-tiles are staged (issued 4 ahead), 2 converted sub-tiles and their
  // token scales are read by the products.
  auto tile_of = [&](int64_t z) -> char* {
    return smem + (F8 ? (int)(z & 1) : (int)(z & 3)) * kSubBytes;
  };
  auto stage_of = [&](int64_t z) -> char* { return smem + kSf8Stage0 + (int)(z & 3) * kF8Stage; };
  auto scales_of = [&](int64_t z) -> float* { return (float*)(smem + kSf8Scale0 + (int)(z & 1) * 128); };
  constexpr int kAhead = F8 ? 4 : 3;  // sub-tiles issued ahead of the one in use

  // rows of this wave
  const int qrow0 = blockIdx.y * kSfRows + 16 * w;
  const bool active = qrow0 < R;  // uniform per wave
  const int qi = active ? qrow0 / a.heads : 0;
  const int h0 = active ? qrow0 % a.heads : 0;
  const float sl2 = a.softmax_scale * kLog2e;

  // next sub-tile to load: tile px, half phh, ring index pz
  int64_t px = x0, pz = 0;
  int phh = 0;
  auto slide = [&](int ln) {
    if (px >= win.wx + win.wn)  // slide the window to start at the tile in use
      build_window(a, px - 2, x1, win.b0, win.pb0, ln, win);
  };
  auto plan_next = [&](int ln) {
    slide(ln);
    const DmaPlan plan = plan_sub(a, tile_info(win, px), phh, lds0 + (uint32_t)((pz & 3) * kSubBytes), w, ln);
    step_sub(px, phh);
    ++pz;
    return plan;
  };
  auto plan_next_f8 = [&](int ln) {
    slide(ln);
    const F8Plan plan = plan_sub_f8(a, tile_info(win, px), phh,
                                    lds0 + (uint32_t)(kSf8Stage0 + (pz & 3) * kF8Stage), w, ln);
    step_sub(px, phh);
    ++pz;
    return plan;
  };
  // this wave's loaded chunks of sub-tile z, bf16 -> fp16 in place, once
  // they have landed (its loads of later sub-tiles may stay in flight)
  // fp8: this thread's chunks of sub-tile z (staged by all waves, whose
  // loads of z landed before the last barrier), e4m3 -> fp16, and its token
  // scales (wave 4)
  auto convert_sub_f8 = [&](int64_t z, int ln) {
    int tid = (int)threadIdx.x;
    asm volatile("" : "+v"(tid));  // recompute the addresses, do not keep them live
    convert_f8(stage_of(z), tile_of(z), tid);
    if (w == 4 && ln < 32) scales_of(z)[ln] = ((const float*)(stage_of(z) + 18432))[ln];
  };
  auto convert_sub = [&](int64_t z, int ln) {
    if (F8) {
      convert_sub_f8(z, ln);
      return;
    }
    wait_vm((int)(n_share * (pz - 1 - z)));
    char* base = smem + (int)(z & 3) * kSubBytes + (w & 3) * 1024 + 16 * ln;
    uint4 c[kSfSplit];
#pragma unroll
    for (int i = 0; i < kSfSplit; ++i)
      if (i < n_share) c[i] = *(const uint4*)(base + (cg0 + i) * 4096);
#pragma unroll
    for (int i = 0; i < kSfSplit; ++i)
      if (i < n_share) *(uint4*)(base + (cg0 + i) * 4096) = bf16x8_to_f16x8(c[i]);
  };

  f16x8 q[18];
  auto load_q = [&](int b, int ln) {
    // unconditional (inactive waves read row 0) so q is dead between segments
    const int li = ln & 15, gq = ln >> 4;
    const f16x8* qp = (const f16x8*)((const _Float16*)a.q_abs +
                                     (((int64_t)b * a.q_len + qi) * a.heads + h0 + li) * 576);
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) q[kk] = qp[4 * kk + gq];
    // The compiler counts only its own loads: left pending, each score
    // MFMA would get a wait for its q slice, and since the counter is in
    // order that wait also covers every direct cache load issued after the
    // query (the last one drains them all, every sub-tile).  Taking q here
    // puts one wait at the segment start instead.
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) asm volatile("" ::"v"(q[kk]));
  };

  // ---- prologue: the first sub-tiles in flight, this wave's query, sub-tile
  // 0 converted (fp8: and sub-tile 1 landed)
  for (int z = 0; z < kAhead && z < nsub; ++z) {
    if (F8) {
      issue_all_f8(plan_next_f8(lane), w);
    } else {
      const DmaPlan plan = plan_next(lane);
      for (int cg = cg0; cg < cg1; ++cg) issue_cg(plan, w, cg);
    }
  }
  load_q(tile_info(win, x0).b, lane);
  wait_vm0();
  if (F8) block_sync();  // every wave's rows of the first sub-tiles in LDS
  convert_sub(0, lane);
  block_sync();

  f32x4 o[32];  // O^T: column block nb holds latent columns 16 nb + 4(l/16)..+3 of row l%16
#pragma unroll
  for (int nb = 0; nb < 32; ++nb) o[nb] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  bool new_seg = false;  // the first segment's query is loaded
  int64_t cx = x0;       // tile of the current sub-tile
  int chh = 0;           // and its half

  for (int64_t s = 0; s < nsub; ++s) {
    // waves 4-7 convert their chunks of the next sub-tile first, waves 0-3
    // last, so that between two barriers the two waves sharing a SIMD reach
    // their MFMA phases at different times (and 4-7, the waves the barrier
    // waits for, find their loads landed)
    if (w >= 4 && s + 1 < nsub) convert_sub(s + 1, fresh_lane());
    int ln = fresh_lane();
    const TileInfo ci = tile_info(win, cx);
    if (new_seg) {
      new_seg = false;
      load_q(ci.b, ln);
      m_run = -INFINITY;
      l_run = 0.f;
    }
    const char* tile = tile_of(s);
    // visible tokens of this sub-tile: all up to the sequence end, or with
    // the causal mask those up to the query's own position
    int nv = ci.rem - 32 * chh - (a.causal ? a.q_len - 1 - qi : 0);
    nv = nv < 0 ? 0 : (nv > kSub ? kSub : nv);
    const bool work = active && nv > 0;  // uniform per wave
    const bool last = s + 1 >= nsub || (chh == 1 && ci.rem <= kTile);
    const bool more = s + kAhead < nsub;
    DmaPlan plan{};
    F8Plan plan8{};
    if (more) {
      if (F8)
        plan8 = plan_next_f8(ln);
      else
        plan = plan_next(ln);
    }
    int issued = cg0;  // column groups of sub-tile s+3 issued so far (bf16)
    bool issued8 = false;

    if (work) {
      // ------------------------------------------------ scores and softmax
      f32x4 sc[2] = {f32x4{}, f32x4{}};  // token block jt: tokens 16 jt + 4(l/16)..+3
      {
        constexpr int kPf = kSfKPrefetch;
        const uint32_t o_qk = off_qk(fresh_lane());
        f16x8 ka[kPf + 1][2];
        auto kload = [&](int kk) {
          const int e = kk % (kPf + 1);
#pragma unroll
          for (int jt = 0; jt < 2; ++jt)
            ka[e][jt] = *(const f16x8*)(tile + (uint32_t)((kk >> 1) * 4096 + 2048 * jt + 512 * (kk & 1)) + o_qk);
        };
#pragma unroll
        for (int kk = 0; kk < kPf; ++kk) kload(kk);
#pragma unroll
        for (int kk = 0; kk < 18; ++kk) {
          if (kk + kPf < 18) kload(kk + kPf);
          const int e = kk % (kPf + 1);
          sc[0] = mfma16h(ka[e][0], q[kk], sc[0]);
          sc[1] = mfma16h(ka[e][1], q[kk], sc[1]);
          __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("s_nop 15\n\ts_nop 7" : "+v"(sc[0]), "+v"(sc[1]));
      }
      ln = fresh_lane();
      f32x4 tsc[2];  // fp8: the tokens' dequantisation scales
      if (F8) {
        tsc[0] = *(const f32x4*)(scales_of(s) + 4 * (ln >> 4));
        tsc[1] = *(const f32x4*)(scales_of(s) + 16 + 4 * (ln >> 4));
        sc[0] *= tsc[0];
        sc[1] *= tsc[1];
      }
      if (nv < kSub) {  // mask the tokens past the visible end
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * jt + 4 * (ln >> 4) + r >= nv) sc[jt][r] = -INFINITY;
      }
      // this lane's max over its 8 scores, in log2 units; the reference max
      // of a row moves only when one of its scores passes it by more than 2^8
      // (exponentials stay <= 256, and the final normalisation uses the same
      // reference for numerator and denominator)
      const float lm = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                             fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3]))) * sl2;
      if (__ballot(lm > m_run + 8.f) != 0) {
        float mt = fmaxf(lm, __shfl_xor(lm, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int nb = 0; nb < 32; ++nb) o[nb] *= alpha;  // lane l holds row l%16's accumulators
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      f16x8 p;  // P^T operand: tokens {4(l/16)..+3, 16+4(l/16)..+3} of row l%16
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sc[jt][r], sl2, -m_use));
          l_run += e;
          // fp8: the value rows in LDS are unscaled, so P carries the scale
          p[4 * jt + r] = (_Float16)(F8 ? e * tsc[jt][r] : e);
        }

      // ------------------------------------------------ O^T += V^T P^T
      const int lv = fresh_lane();
      const uint32_t vb00 = vt_base(lv, 0, 0), vb01 = vt_base(lv, 0, 1);
      const uint32_t vb10 = vt_base(lv, 1, 0), vb11 = vt_base(lv, 1, 1);
      auto vload = [&](int nb) {
        const uint32_t cb = (uint32_t)((nb >> 2) * 4096 + (nb & 3) * 256);
        return cath(lds_tr4h(tile, cb + ((nb & 1) ? vb01 : vb00)),
                    lds_tr4h(tile, cb + ((nb & 1) ? vb11 : vb10)));
      };
      f16x8 va = vload(0), vn = vload(1);
#pragma unroll
      for (int nb = 0; nb < 32; ++nb) {
        const f16x8 vnn = nb + 2 < 32 ? vload(nb + 2) : vn;
        // this sub-tile's share of the loads of sub-tile s+3 goes out between
        // the MFMAs, so that the issue stalls overlap the matrix core's work
        if (F8) {
          if (nb == 3 && more) {
            issue_all_f8(plan8, w);
            issued8 = true;
          }
        } else if ((nb & 3) == 3 && more && issued < cg1) {
          issue_cg(plan, w, issued++);
        }
        o[nb] = mfma16h(va, p, o[nb]);
        __builtin_amdgcn_sched_barrier(0);
        va = vn;
        vn = vnn;
      }
    }
    if (more) {  // the rest (all, without a value sum)
      if (F8) {
        if (!issued8) issue_all_f8(plan8, w);
      } else {
        for (; issued < cg1; ++issued) issue_cg(plan, w, issued);
      }
    }

    if (last) {  // end of this unit's part of the sequence: write the partial
      float l_tot = l_run + __shfl_xor(l_run, 16, 64);
      l_tot += __shfl_xor(l_tot, 32, 64);
      const int lw = fresh_lane();
      if (active) {
        const int64_t sl = (int64_t)u + ci.b;
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        if ((lw >> 4) == 0)
          a.lse_part[sl * R + qrow0 + (lw & 15)] =
              l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
        // fp16 partial row of 1 KB per query row; lane l writes columns
        // 16 nb + 4(l/16)..+3 of row l%16
        _Float16* prow = (_Float16*)a.o_part + (sl * R + qrow0 + (lw & 15)) * 512 + 4 * (lw >> 4);
#pragma unroll
        for (int nb = 0; nb < 32; ++nb) {
          const f16x4 hv = {(_Float16)(o[nb][0] * inv), (_Float16)(o[nb][1] * inv),
                            (_Float16)(o[nb][2] * inv), (_Float16)(o[nb][3] * inv)};
          *(f16x4*)(prow + 16 * nb) = hv;
        }
      }
#pragma unroll
      for (int nb = 0; nb < 32; ++nb) o[nb] = f32x4{};
      new_seg = true;
      wait_vm0();  // keeps the hand-counted load waits exact
    }
    // this wave's chunks of the next sub-tile, once they have landed
    if (w < 4 && s + 1 < nsub) convert_sub(s + 1, fresh_lane());
    // fp8: this wave's rows of sub-tile s+2 landed, for its conversion in
    // the next pass (the loads of s+3 and s+4 may stay in flight)
    if (F8 && s + 2 < nsub) wait_vm((int)(n_share * (pz - 1 - (s + 2))));
    step_sub(cx, chh);
    block_sync();  // sub-tile s+1 complete for everyone; slot of s free
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
    dim3 grid((unsigned)a.num_splits, (unsigned)((R + kSfRows - 1) / kSfRows));
    hipLaunchKernelGGL(decode_sf_kernel<true>, grid, dim3(512), 0, s, a);
  } else {
    dim3 grid((unsigned)a.num_splits, (unsigned)((R + kSfRows - 1) / kSfRows));
    hipLaunchKernelGGL(decode_sf_kernel<false>, grid, dim3(512), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace mla
