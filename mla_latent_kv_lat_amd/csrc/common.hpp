// Shared device/host helpers of the MLA decode library: element codecs,
// cache-row addressing and the split-K division of the cached tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

constexpr int kTile = MLA_TILE_TOKENS;  // tokens per tile and per page block

// ---------------------------------------------------------------- codecs

__host__ __device__ inline float bf16_to_f32(uint16_t b) {
  union { uint32_t u; float f; } v;
  v.u = (uint32_t)b << 16;
  return v.f;
}

// Round to nearest, ties to even; NaN stays NaN.
__host__ __device__ inline uint16_t f32_to_bf16(float f) {
  union { uint32_t u; float f; } v;
  v.f = f;
  if ((v.u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((v.u >> 16) | 0x40u);
  uint32_t r = v.u + 0x7fffu + ((v.u >> 16) & 1u);
  return (uint16_t)(r >> 16);
}

// OCP E4M3 ("fn"): sign, 4-bit exponent with bias 7, 3-bit mantissa;
// exponent 0 is subnormal; S.1111.111 is NaN; no infinities.
__host__ __device__ inline float e4m3_to_f32(uint8_t c) {
  const int e = (c >> 3) & 0xf;
  const int m = c & 7;
  float v;
  if (e == 0)
    v = ldexpf((float)m, -9);
  else if (e == 15 && m == 7)
    v = __builtin_nanf("");
  else
    v = ldexpf((float)(8 + m), e - 10);
  return (c & 0x80) ? -v : v;
}

// IEEE binary16 with saturation: finite values beyond +-65504 become
// +-65504 (the absorbed query is carried in fp16; its 11-bit significand
// keeps the scores of long, outlier-heavy contexts accurate, and the clamp
// keeps an out-of-range query finite instead of turning scores into NaN).
__device__ inline _Float16 f32_to_f16_sat(float f) {
  return (_Float16)fminf(fmaxf(f, -65504.f), 65504.f);
}
__device__ inline uint16_t f32_to_f16_sat_bits(float f) {
  return __builtin_bit_cast(uint16_t, f32_to_f16_sat(f));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {  // bf16 bits
  __device__ static float load(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ static void store(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};
template <> struct Elem<_Float16> {
  __device__ static float load(const _Float16* p, int64_t i) { return (float)p[i]; }
  __device__ static void store(_Float16* p, int64_t i, float v) { p[i] = f32_to_f16_sat(v); }
};
template <> struct Elem<uint8_t> {  // e4m3 codes
  __device__ static float load(const uint8_t* p, int64_t i) { return e4m3_to_f32(p[i]); }
};

// ------------------------------------------------------- cache addressing

// Row of cached token t of sequence b (paged through block_table when given).
__device__ inline int64_t cache_row(int b, int t, const int32_t* block_table, int mbps,
                                    int max_seq_len) {
  if (block_table)
    return (int64_t)block_table[(int64_t)b * mbps + (t >> 6)] * kTile + (t & (kTile - 1));
  return (int64_t)b * max_seq_len + t;
}

// ------------------------------------------------------- split-K division
// The cached tiles of all sequences, in order, form one list of T tiles.
// Unit u of G covers tiles [begin(u), begin(u+1)).  A unit writes one partial
// per sequence it touches, into slot u + b; since units and sequences are
// both in order, (u, b) pairs that touch are distinct in u + b.

__host__ __device__ inline int64_t tiles_of(int32_t len) {
  return len > 0 ? ((int64_t)len + kTile - 1) / kTile : 0;
}
__host__ __device__ inline int64_t unit_begin(int64_t u, int64_t T, int64_t G) {
  return u * T / G;
}
// Unit whose range holds global tile x (0 <= x < T).
__host__ __device__ inline int64_t unit_of_tile(int64_t x, int64_t T, int64_t G) {
  return ((x + 1) * G - 1) / T;
}

// Wave-cooperative search (all 64 lanes call it with the same x): the
// sequence b whose tiles hold global tile x, and its first tile Pb.
// Sums tiles over sequences in chunks of 64 with a lane scan.
__device__ inline void find_sequence(const int32_t* seq_lens, int B, int64_t x, int& b_out,
                                     int64_t& pb_out) {
  const int lane = threadIdx.x & 63;
  int64_t base = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const int64_t t = b < B ? tiles_of(seq_lens[b]) : 0;
    int64_t incl = t;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    const int64_t chunk_total = __shfl(incl, 63, 64);
    if (x < base + chunk_total) {
      // first lane whose inclusive prefix exceeds x - base
      const unsigned long long hit = __ballot(base + incl > x && b < B);
      const int l = __ffsll((long long)hit) - 1;
      b_out = b0 + l;
      pb_out = base + __shfl(incl - t, l, 64);
      return;
    }
    base += chunk_total;
  }
  b_out = B;
  pb_out = base;
}

// Wave-cooperative: total tile count T over all sequences, and the tiles
// of the sequences before b_query.
__device__ inline void wave_tile_sums(const int32_t* seq_lens, int B, int b_query,
                                      int64_t& total, int64_t& before) {
  const int lane = threadIdx.x & 63;
  int64_t t_all = 0, t_before = 0;
  for (int b = lane; b < B; b += 64) {
    const int64_t t = tiles_of(seq_lens[b]);
    t_all += t;
    if (b < b_query) t_before += t;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    t_all += __shfl_xor(t_all, d, 64);
    t_before += __shfl_xor(t_before, d, 64);
  }
  total = t_all;
  before = t_before;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}
__device__ inline float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  return v;
}

}  // namespace mla
