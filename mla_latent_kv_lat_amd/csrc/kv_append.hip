// Cache-append producer for gfx950: the cached row [c_kv | k_rope] of each
// new token, written into the latent cache at a caller-given row.
//
// Pages cited (title, section):
//   [ARCH] "Model Architecture Driving Inference Systems: From MHA/GQA to
//          DeepSeek MLA Matrix Absorption and Memory Minimalism"
//   [MATH] "Multi-Head Latent Attention (MLA): Mathematical Foundations, ..."
//
//   c_kv   = RMSNorm(W_DKV h) * w_norm    ([ARCH] 2.1 down-projection; the
//                                          [MATH] reference module normalises
//                                          the latent before caching it)
//   k_rope = RoPE(W_KR h, pos)             ([ARCH] 2.3 decoupled key)
//
// Two kernels:
//   kv_down_kernel    the 576 output channels (512 of W_DKV, 64 of W_KR)
//                     as one GEMM on v_mfma_f32_16x16x32_bf16, split over
//                     the hidden width: workgroup (channel block, chunk)
//                     computes 32 channels of every token over 512 hidden
//                     columns (4 waves x 128), the waves' sums meet in LDS,
//                     and one fp32 partial per chunk goes to the workspace.  Both
//                     operands have the contracted index contiguous, so
//                     they load straight into MFMA registers; every weight
//                     byte is read once.
//   kv_finish_kernel  one single-wave workgroup per token (spreading the
//                     partial loads over as many CUs as there are tokens):
//                     adds the chunks' partials,
//                     normalises the latent (mean square over 512 channels,
//                     fp32), applies the norm weight, rotates the key at the
//                     token's position (angle reduced in double precision),
//                     and stores the bf16 row, or the e4m3 codes of the row
//                     divided by its scale amax/448 and the scale (the fp8
//                     cache the decode kernel reads: one fp32 scale per token
//                     over its 576 values).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "common.hpp"
#include "../../include/mla.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kAppN = 576;      // output channels: latent 512 + RoPE 64
constexpr int kAppLat = 512;
constexpr int kAppChunk = 512;  // hidden columns per workgroup (4 waves x 128)
constexpr int kAppMaxChunks = 32;  // hidden width up to 16384 (API limit)

// 16x16x32 operands: A lane l = row l%16, k 8(l/16)..+7; B lane l = column
// l%16, same k; C lane l = column l%16, rows 4(l/16)..+3.
__global__ __launch_bounds__(256) void kv_down_kernel(const uint16_t* __restrict__ h,
                                                      const uint16_t* __restrict__ w_dkv,
                                                      const uint16_t* __restrict__ w_kr,
                                                      int n_tok, int d_model, int n_chunks,
                                                      float* __restrict__ part) {
  __shared__ f32x4 red[3][2][4][64];
  // Work item p = (chunk s, channel block xb), chunk-major.  Workgroups are
  // dealt to the 8 XCDs round-robin, so workgroup i takes item
  // (i % 8) * per_xcd + i / 8: the channel blocks of one chunk then run on
  // one or two XCDs and that chunk's hidden-state columns are fetched into
  // one or two L2s instead of all eight.
  const int n_items = (kAppN / 32) * n_chunks;
  const int per_xcd = (n_items + 7) / 8;
  const int p = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (p >= n_items) return;  // uniform across the workgroup
  const int s = p / (kAppN / 32);   // hidden columns [512 s, 512 s + 512)
  const int xb = p % (kAppN / 32);  // output channels 32 xb .. 32 xb + 31
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int li = lane & 15, g = lane >> 4;
  const int k0 = kAppChunk * s + 128 * w + 8 * g;
  // output channels 32 blockIdx.x + 16 j + li, j = 0, 1 (never straddling 512)
  bf16x8 bw[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = 32 * xb + 16 * j + li;
    const uint16_t* wrow = n < kAppLat ? w_dkv + (int64_t)n * d_model
                                       : w_kr + (int64_t)(n - kAppLat) * d_model;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) bw[j][ks] = *(const bf16x8*)(wrow + k0 + 32 * ks);
  }

  for (int m0 = 0; m0 < n_tok; m0 += 64) {  // four 16-token blocks at a time
    bf16x8 ha[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + 16 * mb + li;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        ha[mb][ks] = m < n_tok ? *(const bf16x8*)(h + (int64_t)m * d_model + k0 + 32 * ks) : bf16x8{};
    }
    f32x4 acc[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        acc[j][mb] = f32x4{};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          acc[j][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ha[mb][ks], bw[j][ks], acc[j][mb], 0, 0, 0);
      }
    if (w > 0)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) red[w - 1][j][mb][lane] = acc[j][mb];
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = 32 * xb + 16 * j + li;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const f32x4 t = acc[j][mb] + red[0][j][mb][lane] + red[1][j][mb][lane] + red[2][j][mb][lane];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = m0 + 16 * mb + 4 * g + r;
            if (m < n_tok) part[((int64_t)s * n_tok + m) * kAppN + n] = t[r];
          }
        }
      }
    }
    __syncthreads();  // red is reused by the next token group
  }
}

// F8: e4m3 codes (OCP) of row / scale with scale = amax / 448 over the
// token's 576 values, and the scale to kv_scale[row]; else bf16 values.
template <bool F8>
__global__ __launch_bounds__(64) void kv_finish_kernel(
    const float* __restrict__ part, int n_chunks, int n_tok, const uint16_t* __restrict__ w_norm,
    const int32_t* __restrict__ positions, double log2_base, float eps,
    const int64_t* __restrict__ rows, char* __restrict__ latent, char* __restrict__ rope,
    int64_t stride_bytes, float* __restrict__ kv_scale) {
  const int t = blockIdx.x;  // one wave per token
  const int lane = threadIdx.x & 63;
  f32x4 v0 = f32x4{}, v1 = f32x4{};  // latent channels 8 lane .. 8 lane + 7
  float r0 = 0.f, r1 = 0.f;          // RoPE pair `lane` (lanes < 32)
  // eight chunks' loads in flight at once (sixteen measured slower): indices
  // past the last chunk are clamped and the duplicates are not added, so the
  // loads need no branches
  constexpr int kG = 8;
  for (int s0 = 0; s0 < n_chunks; s0 += kG) {
    f32x4 a[kG], b[kG];
    float2 c[kG];
#pragma unroll
    for (int i = 0; i < kG; ++i) {
      const int sc = min(s0 + i, n_chunks - 1);
      const float* p = part + ((int64_t)sc * n_tok + t) * kAppN;
      a[i] = *(const f32x4*)(p + 8 * lane);
      b[i] = *(const f32x4*)(p + 8 * lane + 4);
      c[i] = *(const float2*)(p + kAppLat + 2 * (lane & 31));
    }
#pragma unroll
    for (int i = 0; i < kG; ++i) {
      const float m = s0 + i < n_chunks ? 1.f : 0.f;
      v0 += m * a[i];
      v1 += m * b[i];
      r0 += m * c[i].x;
      r1 += m * c[i].y;
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) ss += v0[i] * v0[i] + v1[i] * v1[i];
  ss = wave_sum(ss);
  const float inv = 1.f / sqrtf(ss * (1.f / kAppLat) + eps);
  const uint4 wn = *(const uint4*)(w_norm + 8 * lane);
  const uint32_t wv[4] = {wn.x, wn.y, wn.z, wn.w};
  const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
  float y[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[2 * i] = v[2 * i] * inv * bf16_to_f32((uint16_t)(wv[i] & 0xffffu));
    y[2 * i + 1] = v[2 * i + 1] * inv * bf16_to_f32((uint16_t)(wv[i] >> 16));
  }
  // pair k = lane turns by pos * base^(-2k/64); the angle is reduced into
  // [-pi, pi] in double so that long positions keep their accuracy
  float x0 = 0.f, x1 = 0.f;
  if (lane < 32) {
    const double theta = exp2(-2.0 * lane / (2 * 32) * log2_base);
    double ang = (double)positions[t] * theta;
    ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
    float sn, cs;
    __sincosf((float)ang, &sn, &cs);
    x0 = r0 * cs - r1 * sn;
    x1 = r0 * sn + r1 * cs;
  }
  const int64_t row = rows[t];
  if constexpr (F8) {
    float am = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(y[i]));
    am = wave_max(am);
    const float sc = am > 0.f ? am / 448.f : 1.f;
    int lo = 0, hi = 0;
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0] / sc, y[1] / sc, lo, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2] / sc, y[3] / sc, lo, true);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4] / sc, y[5] / sc, hi, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6] / sc, y[7] / sc, hi, true);
    *(uint2*)(latent + row * stride_bytes + 8 * lane) = make_uint2((uint32_t)lo, (uint32_t)hi);
    if (lane < 32) {
      const int pr = __builtin_amdgcn_cvt_pk_fp8_f32(x0 / sc, x1 / sc, 0, false);
      *(uint16_t*)(rope + row * stride_bytes + 2 * lane) = (uint16_t)(pr & 0xffff);
    }
    if (lane == 0) kv_scale[row] = sc;
  } else {
    uint32_t ob[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ob[i] = (uint32_t)f32_to_bf16(y[2 * i]) | ((uint32_t)f32_to_bf16(y[2 * i + 1]) << 16);
    *(uint4*)(latent + row * stride_bytes + 16 * lane) = make_uint4(ob[0], ob[1], ob[2], ob[3]);
    if (lane < 32)
      *(uint32_t*)(rope + row * stride_bytes + 4 * lane) =
          (uint32_t)f32_to_bf16(x0) | ((uint32_t)f32_to_bf16(x1) << 16);
  }
}

bool app_dims_ok(const mla_append_dims_t* d) {
  return d && d->n_tokens >= 0 && d->d_model > 0 && d->d_latent > 0 && d->d_rope >= 0;
}

// Host validation shared by both entry points: 0, or the status to return.
int app_check(const mla_append_dims_t* dims, const void* h, const void* w_dkv,
              const void* kv_norm_w, const void* w_kr, const int32_t* positions, float rope_base,
              float eps, const int64_t* cache_rows, const void* latent_cache,
              const void* rope_cache, int64_t kv_row_stride, const float* kv_scale) {
  if (!app_dims_ok(dims)) return MLA_ERR_INVALID_ARG;
  if (dims->d_latent != kAppLat || dims->d_rope != kAppN - kAppLat || dims->d_model % kAppChunk ||
      dims->d_model > kAppChunk * kAppMaxChunks ||
      (dims->kv_dtype != MLA_BF16 && dims->kv_dtype != MLA_FP8_E4M3))
    return MLA_ERR_UNSUPPORTED;
  if (dims->n_tokens == 0) return MLA_OK;
  const bool f8 = dims->kv_dtype == MLA_FP8_E4M3;
  if (!h || !w_dkv || !kv_norm_w || !w_kr || !positions || !cache_rows || !latent_cache ||
      !rope_cache || (kv_scale != nullptr) != f8)
    return MLA_ERR_INVALID_ARG;
  auto al = [](const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; };
  if (!al(h, 16) || !al(w_dkv, 16) || !al(w_kr, 16) || !al(kv_norm_w, 16) ||
      !al(latent_cache, f8 ? 8 : 16) || !al(rope_cache, f8 ? 2 : 4) || (f8 && !al(kv_scale, 4)))
    return MLA_ERR_INVALID_ARG;
  if (kv_row_stride < kAppLat || kv_row_stride % 8) return MLA_ERR_INVALID_ARG;
  if (!(rope_base > 0.f) || !isfinite(rope_base) || !(eps >= 0.f) || !isfinite(eps))
    return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

// The two kernels in turn; `workspace` holds the partial sums (16-byte aligned).
int app_launch(const mla_append_dims_t* dims, const void* h, const void* w_dkv,
               const void* kv_norm_w, const void* w_kr, const int32_t* positions, float rope_base,
               float eps, const int64_t* cache_rows, void* latent_cache, void* rope_cache,
               int64_t kv_row_stride, float* kv_scale, float* workspace, hipStream_t s) {
  const bool f8 = dims->kv_dtype == MLA_FP8_E4M3;
  (void)hipGetLastError();
  const int chunks = dims->d_model / kAppChunk;
  const int items = (kAppN / 32) * chunks;
  hipLaunchKernelGGL(kv_down_kernel, dim3(8 * ((items + 7) / 8)), dim3(256), 0, s,
                     (const uint16_t*)h, (const uint16_t*)w_dkv, (const uint16_t*)w_kr,
                     dims->n_tokens, dims->d_model, chunks, workspace);
  if (hipGetLastError() != hipSuccess) return MLA_ERR_HIP;
  const dim3 fg(dims->n_tokens);
  if (f8)
    hipLaunchKernelGGL(kv_finish_kernel<true>, fg, dim3(64), 0, s, (const float*)workspace,
                       chunks, dims->n_tokens, (const uint16_t*)kv_norm_w, positions,
                       log2((double)rope_base), eps, cache_rows, (char*)latent_cache,
                       (char*)rope_cache, kv_row_stride, kv_scale);
  else
    hipLaunchKernelGGL(kv_finish_kernel<false>, fg, dim3(64), 0, s, (const float*)workspace,
                       chunks, dims->n_tokens, (const uint16_t*)kv_norm_w, positions,
                       log2((double)rope_base), eps, cache_rows, (char*)latent_cache,
                       (char*)rope_cache, kv_row_stride * 2, nullptr);
  return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// Scratch of mla_kv_append_noalloc: kv_down_kernel's fp32 partial sums in
// a file-scope device array, one copy per GPU the library runs on, held
// until the process ends.  Host code never passes `scratch` itself (its
// host-side name is only a stand-in for the device object): the device
// address comes from hipGetSymbolAddress, once per device.
constexpr int64_t kAppScratchBytes = MLA_KV_APPEND_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kAppScratchBytes / 4];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null: not looked up)

// The device address of `scratch` on the current device, looked up on the
// first call on that device (with it current).  Null on failure.
float* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = (float*)ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace mla

using namespace mla;

extern "C" {

int mla_kv_append_workspace_bytes(const mla_append_dims_t* dims, int64_t* bytes) {
  if (!app_dims_ok(dims) || !bytes) return MLA_ERR_INVALID_ARG;
  if (dims->d_latent != kAppLat || dims->d_rope != kAppN - kAppLat || dims->d_model % kAppChunk ||
      dims->d_model > kAppChunk * kAppMaxChunks)
    return MLA_ERR_UNSUPPORTED;
  *bytes = (int64_t)(dims->d_model / kAppChunk) * dims->n_tokens * kAppN * 4;
  return MLA_OK;
}

int mla_kv_append(const mla_append_dims_t* dims, const void* h, const void* w_dkv,
                  const void* kv_norm_w, const void* w_kr, const int32_t* positions,
                  float rope_base, float eps, const int64_t* cache_rows, void* latent_cache,
                  void* rope_cache, int64_t kv_row_stride, float* kv_scale, void* workspace,
                  void* stream) {
  const int st = app_check(dims, h, w_dkv, kv_norm_w, w_kr, positions, rope_base, eps, cache_rows,
                           latent_cache, rope_cache, kv_row_stride, kv_scale);
  if (st != MLA_OK || dims->n_tokens == 0) return st;
  if (!workspace) return MLA_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 15) != 0) return MLA_ERR_INVALID_ARG;
  return app_launch(dims, h, w_dkv, kv_norm_w, w_kr, positions, rope_base, eps, cache_rows,
                    latent_cache, rope_cache, kv_row_stride, kv_scale, (float*)workspace,
                    (hipStream_t)stream);
}

int mla_kv_append_noalloc(const mla_append_dims_t* dims, const void* h, const void* w_dkv,
                          const void* kv_norm_w, const void* w_kr, const int32_t* positions,
                          float rope_base, float eps, const int64_t* cache_rows,
                          void* latent_cache, void* rope_cache, int64_t kv_row_stride,
                          float* kv_scale, void* stream) {
  const int st = app_check(dims, h, w_dkv, kv_norm_w, w_kr, positions, rope_base, eps, cache_rows,
                           latent_cache, rope_cache, kv_row_stride, kv_scale);
  if (st != MLA_OK || dims->n_tokens == 0) return st;
  // the partial sums must fit the static scratch
  const int64_t need = (int64_t)(dims->d_model / kAppChunk) * dims->n_tokens * kAppN * 4;
  if (need > kAppScratchBytes) return MLA_ERR_TOO_LARGE;
  float* ws = scratch_on_current_device();
  if (!ws) return MLA_ERR_HIP;
  return app_launch(dims, h, w_dkv, kv_norm_w, w_kr, positions, rope_base, eps, cache_rows,
                    latent_cache, rope_cache, kv_row_stride, kv_scale, ws, (hipStream_t)stream);
}

}  // extern "C"
