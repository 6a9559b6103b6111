// Device helpers shared by the gfx950 MFMA kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __fp16 fp16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) fp16x4_t lds_f16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 lds_tr4(const char* base, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)((lds_char*)base + off));
}

// fp16 forms: the decode kernels score and sum in fp16 (an exact image of
// the bf16 or e4m3 cache values, and an 11-bit-significand query)
__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16h(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x4 lds_tr4h(const char* base, uint32_t off) {
  return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_f16x4*)((lds_char*)base + off)));
}
__device__ __forceinline__ f16x8 cath(f16x4 a, f16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// One 16-byte direct global->LDS load per lane: lane i reads 16 bytes at
// sbase + voff (sbase wave-uniform, voff per lane) and the wave's 64 lanes fill
// the 1 KB of LDS starting at byte address m0 in lane order.  Issued as
// inline assembly so that waits on it are placed by hand (vmcnt), instead of
// the compiler's blanket wait before every later LDS read.  An SALU write of
// m0 needs one wait state before a load with LDS = 1 reads it (the compiler
// cannot pad inside the asm): without the s_nop the load may take the
// previous m0 and fill the previous block's LDS.
__device__ __forceinline__ void lds_dma16(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0),
               "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// As lds_dma16 for data read once (the cache rows of a decode step): the
// non-temporal hint keeps the stream from displacing data that later
// kernels reuse (weights, partials) from the caches.
__device__ __forceinline__ void lds_dma16_stream(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(m0),
               "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// As lds_dma16 with 4 bytes per lane (256 bytes of LDS per wave).
__device__ __forceinline__ void lds_dma4(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(m0),
               "v"(voff), "s"(sbase)
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
// s_waitcnt vmcnt(n) for n in 0..9 (tile loads still allowed in flight).
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
    case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
  }
}
__device__ __forceinline__ void block_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}


// Raw buffer resource over `bytes` bytes at `base`: stores at offsets past
// the end are dropped by the hardware range check.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void buffer_store_f32(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)voff, (int)soff, 0);
}

__device__ __forceinline__ void buffer_store_f16(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 uint32_t soff) {
  const _Float16 h = (_Float16)v;
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, h), r, (int)voff, (int)soff, 0);
}


// Let the last MFMA into `v` finish before VALU code reads it: 24 wait
// states, more than an 8-pass MFMA result needs.  The compiler's hazard
// padding is missing when the first read sits behind a branch join, and a
// read that early sees a stale accumulator.  The in/out operand orders every
// later use of `v` after the wait.
template <typename V>
__device__ __forceinline__ void mfma_settle(V& v) {
  asm volatile("s_nop 15\n\ts_nop 7" : "+v"(v));
}

}  // namespace mfma
}  // namespace mla
