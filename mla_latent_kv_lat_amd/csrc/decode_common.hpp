// Device helpers shared by the split-K decode kernels (internal): the
// lane-resident window of tile descriptors that replaces scalar-memory
// walks over seq_lens / block_table inside the loops.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_common.hpp"

namespace mla {
namespace dec {

using namespace mfma;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Lane-resident descriptors of tiles wx .. wx+wn-1 of a unit's walk over
// the cache: lane i describes tile wx+i (its sequence, the tokens from the
// tile's start to the sequence end, and the tile's first cache row).  The hot
// loop reads them with v_readlane, so no scalar-memory round trip sits on the
// path from one sub-tile to the next.  Cache rows fit in 32 bits: 2^31 rows
// of >= 1 KB would exceed any HBM.
struct TileWin {
  int64_t wx;      // first tile (uniform)
  int wn;          // tiles described (uniform, 1..64)
  int b0;          // sequence of tile wx ...
  int64_t pb0;     // ... and the global index of its first tile (uniform)
  int b, rem, row0;  // per lane
};

struct TileInfo {
  int b;
  int rem;       // tokens from the tile's first row to the sequence end (>= 1)
  int64_t row0;  // first cache row of the tile
};

__device__ __forceinline__ int64_t readlane64(int64_t v, int i) {
  const int lo = __builtin_amdgcn_readlane((int)(uint32_t)v, i);
  const int hi = __builtin_amdgcn_readlane((int)(v >> 32), i);
  return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}

// Describe tiles wx .. min(wx+64, x1)-1.  (b_s, pb_s): any sequence at or
// before the one holding tile wx, and the global index of its first tile.
// Sequence b ends at global tile E_b = sum of tiles of sequences <= b; tile x
// lies in the first sequence with E_b > x, which is b_s plus the number of
// sequences from b_s on that end at or before x (empty ones included).
// Ends with all vector memory drained.
__device__ void build_window(const DecodeArgs& a, int64_t wx, int64_t x1, int b_s, int64_t pb_s,
                             int lane, TileWin& win) {
  const int64_t x = wx + lane;
  int cnt = 0;
  int64_t start = pb_s, carry = pb_s;
  for (int cb = b_s; cb < a.batch; cb += 64) {
    const int seq = cb + lane;
    int64_t incl = seq < a.batch ? tiles_of(a.seq_lens[seq]) : 0;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    const int64_t e = carry + incl;
    for (int j = 0; j < 64; ++j) {
      const int64_t ej = readlane64(e, j);
      if (ej <= x) {
        ++cnt;
        start = ej;
      }
    }
    carry = readlane64(e, 63);
    if (carry > wx + 63) break;
  }
  const bool ok = x < x1;  // then b < batch: tile x belongs to a real sequence
  const int b = b_s + cnt;
  const int tis = (int)(x - start);
  const int len = ok ? a.seq_lens[b] : 0;
  const int page = ok && a.block_table ? a.block_table[(int64_t)b * a.mbps + tis] : 0;
  win.wx = wx;
  win.wn = (int)min((int64_t)64, x1 - wx);
  win.b0 = __builtin_amdgcn_readfirstlane(b);
  win.pb0 = uniform64(start);
  win.b = b;
  win.rem = len - tis * kTile;
  win.row0 = a.block_table ? page * kTile : (int)((int64_t)b * a.max_seq_len + (int64_t)tis * kTile);
  wait_vm0();
}

// Batches of at most 64 sequences: the unit's tile range [x0, x1) of G over
// all T tiles and the window of its first tiles from one load of seq_lens
// (one sequence per lane) and one of block_table, instead of separate passes
// for T, for the sequence holding x0 and for the window.  False: the unit
// is empty.  Ends with all vector memory drained.
__device__ bool unit_window_small(const DecodeArgs& a, int u, int lane, int64_t& x0,
                                  int64_t& x1, TileWin& win) {
  const int len_l = lane < a.batch ? a.seq_lens[lane] : 0;  // sequence `lane`
  const int64_t t_l = tiles_of(len_l);
  int64_t e = t_l;  // end tile (exclusive) of sequence `lane`
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t o = __shfl_up(e, d, 64);
    if (lane >= d) e += o;
  }
  const int64_t T = readlane64(e, 63);
  x0 = unit_begin(u, T, a.num_splits);
  x1 = unit_begin(u + 1, T, a.num_splits);
  if (x0 >= x1) return false;
  // lane i describes tile x = x0 + i: its sequence is the number of
  // sequences that end at or before x (empty ones included)
  const int64_t x = x0 + lane;
  int cnt = 0;
  for (int j = 0; j < a.batch; ++j) cnt += readlane64(e, j) <= x ? 1 : 0;
  const bool ok = x < x1;  // then cnt < batch: tile x belongs to a real sequence
  const int b = ok ? cnt : 0;
  const int64_t start = __shfl(e - t_l, b, 64);  // first tile of sequence b
  const int tis = (int)(x - start);
  const int len = __shfl(len_l, b, 64);
  const int page = ok && a.block_table ? a.block_table[(int64_t)b * a.mbps + tis] : 0;
  win.wx = x0;
  win.wn = (int)min((int64_t)64, x1 - x0);
  win.b0 = __builtin_amdgcn_readfirstlane(b);
  win.pb0 = uniform64(start);
  win.b = b;
  win.rem = ok ? len - tis * kTile : 0;
  win.row0 = a.block_table ? page * kTile : (int)((int64_t)b * a.max_seq_len + (int64_t)tis * kTile);
  wait_vm0();
  return true;
}

__device__ __forceinline__ TileInfo tile_info(const TileWin& win, int64_t x) {
  const int i = (int)(x - win.wx);
  TileInfo t;
  t.b = __builtin_amdgcn_readlane(win.b, i);
  t.rem = __builtin_amdgcn_readlane(win.rem, i);
  t.row0 = (int64_t)(uint32_t)__builtin_amdgcn_readlane(win.row0, i);
  return t;
}

// An opaque copy of the lane id: offsets derived from it are recomputed where
// they are used (a handful of VALU ops) instead of being kept live across a
// loop in registers the accumulators need.
__device__ __forceinline__ int fresh_lane() {
  int l = (int)(threadIdx.x & 63);
  asm volatile("" : "+v"(l));
  return l;
}

// ---- operand addresses in the sub-tile LDS layout (1 KB blocks of 8 rows x
// 8 16-byte chunks; block (cg, rg) at (cg*4 + rg) KB; row rho / chunk kappa
// of a block at entry 8*(kappa ^ (rg&1)) + (rho ^ 4*((kappa ^ kappa>>1)&1)))

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


// Lane part of the V^T operand address (16x16x32 A: lane l holds latent
// column 16 nb + l%16, tokens 4(l/16)..+3 for rd = 0, 16 + 4(l/16)..+3 for
// rd = 1).  Lane l names token 16 rd + 4g + i/4 and columns
// 16 nb + 4(i%4)..+3 (g = l/16, i = l%16); in the sub-tile layout that
// address is this base (which depends on nb only through its parity) plus
// (nb/4) * 4096 + (nb%4) * 256.  The reads are free of bank conflicts.
__device__ __forceinline__ uint32_t vt_base(int lane, int rd, int par) {
  const int g = lane >> 4, i = lane & 15;
  const int rg = 2 * rd + (g >> 1);
  const int rho = 4 * (g & 1) + (i >> 2);
  const int b = (i >> 1) & 1;
  return (uint32_t)(rg * 1024 + 128 * (b ^ (rg & 1)) + 16 * (rho ^ (4 * ((b ^ par) & 1))) + 8 * (i & 1));
}


}  // namespace dec
}  // namespace mla
