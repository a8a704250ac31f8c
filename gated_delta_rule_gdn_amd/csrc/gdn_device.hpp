// gdn_device.hpp -- device-side helpers shared by the gfx950 kernels of
// libgdn.so: element types, vector loads/stores and MFMA fragment wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

using bf16 = __bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Debug build (-DGDN_CHECK, libgdn_check.so).  A kernel first fills its LDS
// with 0xFF bytes, a NaN in fp32, bf16 and fp16, so that a read of LDS that
// nothing wrote reaches the outputs as NaN; and every LDS access through the
// checked helpers (lds_check) is compared with the kernel's static LDS size.
// An access past the end is counted in the module's device counter, which
// the C ABI of that build reads after each launch (take_check_violations).
// In the normal build both helpers compile to nothing.
// ---------------------------------------------------------------------------
#ifdef GDN_CHECK
static __device__ unsigned int g_check_violations;
__device__ __forceinline__ void lds_check(const void* p, int bytes) {
#if __HIP_DEVICE_COMPILE__   // (the builtins exist only in the device pass)
  if (__builtin_amdgcn_is_shared((const __attribute__((address_space(0))) void*)p)) {
    const auto lp = (const __attribute__((address_space(3))) char*)p;
    const uint32_t off = (uint32_t)(uintptr_t)lp;
    if (off + (uint32_t)bytes > __builtin_amdgcn_groupstaticsize())
      atomicAdd(&g_check_violations, 1u);
  }
#else
  (void)p; (void)bytes;
#endif
}
// A condition the caller's indices must meet (counted when they do not).
__device__ __forceinline__ void check_true(bool ok) {
  if (!ok) atomicAdd(&g_check_violations, 1u);
}
__device__ __forceinline__ void lds_nan_fill(void* base, int bytes) {
  uint32_t* w = static_cast<uint32_t*>(base);
  for (int i = (int)threadIdx.x; i < bytes / 4; i += (int)blockDim.x) w[i] = 0xFFFFFFFFu;
  __syncthreads();
}
// Host side: the module's count since the last call (all its work finished),
// reset to zero; ~0u if the counter cannot be read.
static inline unsigned take_check_violations() {
  unsigned v = 0, z = 0;
  if (hipDeviceSynchronize() != hipSuccess) return ~0u;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_check_violations), sizeof v) != hipSuccess) return ~0u;
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_check_violations), &z, sizeof z) != hipSuccess) return ~0u;
  return v;
}
#else
__device__ __forceinline__ void lds_check(const void*, int) {}
__device__ __forceinline__ void check_true(bool) {}
__device__ __forceinline__ void lds_nan_fill(void*, int) {}
#endif

// ---------------------------------------------------------------------------
// Scalar conversions.  bf16 -> fp32 is exact; fp32 -> bf16 rounds to nearest
// even (v_cvt_pk_bf16_f32 on gfx950).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// ---------------------------------------------------------------------------
// Loads of N consecutive elements (N * sizeof(T) bytes, naturally aligned)
// converted to fp32.
// ---------------------------------------------------------------------------
template <int N, typename T>
__device__ __forceinline__ void load_f32(const T* __restrict__ p, float* out);

template <>
__device__ __forceinline__ void load_f32<8, bf16>(const bf16* __restrict__ p, float* out) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load_f32<4, bf16>(const bf16* __restrict__ p, float* out) {
  uint2 u = *reinterpret_cast<const uint2*>(p);
  out[0] = __uint_as_float(u.x << 16);
  out[1] = __uint_as_float(u.x & 0xffff0000u);
  out[2] = __uint_as_float(u.y << 16);
  out[3] = __uint_as_float(u.y & 0xffff0000u);
}
template <>
__device__ __forceinline__ void load_f32<8, float>(const float* __restrict__ p, float* out) {
  float4 a = reinterpret_cast<const float4*>(p)[0];
  float4 b = reinterpret_cast<const float4*>(p)[1];
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}
template <>
__device__ __forceinline__ void load_f32<4, float>(const float* __restrict__ p, float* out) {
  float4 a = *reinterpret_cast<const float4*>(p);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
}

// Store 4 consecutive elements from fp32 (rounded to T).
template <typename T>
__device__ __forceinline__ void store4(T* __restrict__ p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* __restrict__ p, float a, float b, float c,
                                              float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* __restrict__ p, float a, float b, float c,
                                             float d) {
  bf16x4 h = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  *reinterpret_cast<bf16x4*>(p) = h;
}

// 2^x on the hardware exp unit (v_exp_f32).  Arguments are kept in the range
// where the result is a normal float or an exact 0/inf by the callers.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Gate activations, on the hardware exp / log / reciprocal:
//   sigmoid(x)  = 1 / (1 + 2^(-x log2 e))   (0 and 1 at the saturated ends)
//   softplus(x) = max(x, 0) + log(1 + t),  t = e^-|x| in (0, 1]; for
//                 t < 2^-10 the series t - t^2/2 replaces the log, which
//                 would lose t's low bits in 1 + t.
// The Mamba-2 log-decay is g = -exp(A_log) softplus(a + dt_bias); callers
// that reuse a column's -exp(A_log) pass it as neg_A.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sigmoid_f(float x) {
  return __builtin_amdgcn_rcpf(1.f + exp2_fast(-x * kLog2e));
}
__device__ __forceinline__ float softplus_f(float x) {
  const float t = exp2_fast(-fabsf(x) * kLog2e);
  const float l = t < 0x1p-10f ? t - 0.5f * t * t
                               : __builtin_amdgcn_logf(1.f + t) * 0.6931471805599453f;
  return fmaxf(x, 0.f) + l;
}
__device__ __forceinline__ float neg_exp_f(float A_log) { return -exp2_fast(A_log * kLog2e); }
__device__ __forceinline__ float log_decay_f(float a, float neg_A, float dt) {
  return neg_A * softplus_f(a + dt);
}

// ---------------------------------------------------------------------------
// MFMA fragments (wave64, 16x16 output tiles).
//
// For D[16x16] += A[16xK] * B[Kx16] a lane l = 16*g + j (g = 0..3, j = 0..15)
// holds  A row j / B column j, 8 (K=32) or 4 (K=16) k-values, and the
// accumulator rows 4g..4g+3 of column j.  Which k-values a lane supplies
// only has to agree between A and B, so every K-block here is fed in one
// fixed order on both sides (see the kernels).
//
// Frag8<T>: 8 elements of one K=32 block.  bf16 -> one
// v_mfma_f32_16x16x32_bf16; fp32 -> eight v_mfma_f32_16x16x4_f32, the i-th
// taking element i of every lane (each covers 4 distinct k of the block).
// Frag4<T>: 4 elements of a K=16 block.  bf16 -> v_mfma_f32_16x16x16_bf16;
// fp32 -> four v_mfma_f32_16x16x4_f32.
// ---------------------------------------------------------------------------
template <typename T> struct Frag8;
template <> struct Frag8<bf16> { bf16x8 v; };
template <> struct Frag8<float> { float v[8]; };
template <typename T> struct Frag4;
template <> struct Frag4<bf16> { bf16x4 v; };
template <> struct Frag4<float> { float v[4]; };

__device__ __forceinline__ void mma32(f32x4& acc, const Frag8<bf16>& a, const Frag8<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32(f32x4& acc, const Frag8<float>& a, const Frag8<float>& b) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& acc, const Frag4<bf16>& a, const Frag4<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4v, a.v),
                                                  __builtin_bit_cast(short4v, b.v), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16(f32x4& acc, const Frag4<float>& a, const Frag4<float>& b) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], acc, 0, 0, 0);
}

}  // namespace gdn
