// chunk_common.hpp -- helpers shared by the chunkwise forward kernels
// (chunk_fwd.hip: sequential-phase kernel, fp32 operands; chunk_fwd_sb.hip:
// sub-block kernel, bf16 operands) and the backward.  Device code only;
// internal linkage in each unit.
#pragma once

#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

namespace gdn {
namespace {

constexpr int kC = 64;          // tokens per chunk

// Position of index x inside its 32-block when stored in accumulator-row
// order: k = 4g+i (k < 16) -> 8g+i, k = 16+4g+i -> 8g+4+i.
__device__ __forceinline__ int sig(int x) {
  const int k = x & 31;
  const int p = (k < 16) ? (((k >> 2) << 3) + (k & 3)) : ((((k - 16) >> 2) << 3) + 4 + (k & 3));
  return (x & ~31) + p;
}

__device__ __forceinline__ float dpp_row_shr(float x, int n) {
  int v = __builtin_bit_cast(int, x);
  int r;
  switch (n) {
    case 1: r = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false); break;
    case 4: r = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false); break;
    default: r = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false); break;
  }
  return __builtin_bit_cast(float, r);
}

// Value of lane n of each 16-lane row, broadcast to the whole row.
template <int N>
__device__ __forceinline__ float dpp_row_bcast(float x) {
  static_assert(N >= 0 && N < 16, "lane");
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0x150 + N, 0xf, 0xf, false));
}

// NB bytes loaded as packed 32-bit words (one or two vector loads).
template <int NB>
struct Raw {
  uint32_t w[NB / 4];
};
template <int NB>
__device__ __forceinline__ void ld_raw(const void* p, Raw<NB>& r) {
  if constexpr (NB == 8) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    r.w[0] = u.x; r.w[1] = u.y;
  } else if constexpr (NB == 16) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    r.w[0] = u.x; r.w[1] = u.y; r.w[2] = u.z; r.w[3] = u.w;
  } else {
    static_assert(NB == 32, "raw size");
    const uint4 u = reinterpret_cast<const uint4*>(p)[0];
    const uint4 v = reinterpret_cast<const uint4*>(p)[1];
    r.w[0] = u.x; r.w[1] = u.y; r.w[2] = u.z; r.w[3] = u.w;
    r.w[4] = v.x; r.w[5] = v.y; r.w[6] = v.z; r.w[7] = v.w;
  }
}
// Unpack N elements of type E to fp32, zeroed when !valid.
template <typename E, int N, int NB>
__device__ __forceinline__ void unpack(const Raw<NB>& r, bool valid, float* out) {
  static_assert(N * (int)sizeof(E) == NB, "raw size");
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float x;
    if constexpr (sizeof(E) == 2) {
      const uint32_t w = r.w[i >> 1];
      x = __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
      x = __uint_as_float(r.w[i]);
    }
    out[i] = valid ? x : 0.f;
  }
}

// Unpack N elements of type E to fp32 (no masking: callers zero the raw words
// of absent tokens).
template <typename E, int N, int NB>
__device__ __forceinline__ void unpack(const Raw<NB>& r, float* out) {
  static_assert(N * (int)sizeof(E) == NB, "raw size");
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if constexpr (sizeof(E) == 2) {
      const uint32_t w = r.w[i >> 1];
      out[i] = __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
      out[i] = __uint_as_float(r.w[i]);
    }
  }
}
template <int NB>
__device__ __forceinline__ void zero_raw(Raw<NB>& r) {
#pragma unroll
  for (int i = 0; i < NB / 4; ++i) r.w[i] = 0u;
}

// One gate element of type E kept as its raw bits in a 32-bit word (the
// load is not waited for until the word is converted).
template <typename E>
__device__ __forceinline__ uint32_t ld_word(const void* p) {
  if constexpr (sizeof(E) == 2) return (uint32_t)(*reinterpret_cast<const unsigned short*>(p));
  else return *reinterpret_cast<const uint32_t*>(p);
}
template <typename E>
__device__ __forceinline__ float word_f32(uint32_t w) {
  if constexpr (sizeof(E) == 2) return __uint_as_float(w << 16);
  else return __uint_as_float(w);
}

// Store 4 consecutive fp32 values as T.
template <typename T>
__device__ __forceinline__ void st4(T* p, float a, float b, float c, float d) {
  lds_check(p, 4 * (int)sizeof(T));
  if constexpr (sizeof(T) == 2) {
    bf16x4 h = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
    *reinterpret_cast<bf16x4*>(p) = h;
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
}

template <typename T>
__device__ __forceinline__ Frag8<T> ld_frag8(const T* p) {
  lds_check(p, 8 * (int)sizeof(T));
  Frag8<T> f;
  if constexpr (sizeof(T) == 2) {
    f.v = *reinterpret_cast<const bf16x8*>(p);
  } else {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  }
  return f;
}

template <typename T>
__device__ __forceinline__ Frag4<T> ld_frag4(const T* p) {
  lds_check(p, 4 * (int)sizeof(T));
  Frag4<T> f;
  if constexpr (sizeof(T) == 2) {
    f.v = *reinterpret_cast<const bf16x4*>(p);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  }
  return f;
}

// K=32 fragment from two accumulator tiles (rows 0-15 and 16-31 of a block).
// bf16 values are rounded in pairs (one v_cvt_pk_bf16_f32 per two).
template <typename T>
__device__ __forceinline__ Frag8<T> frag8_from_acc(const f32x4& lo, const f32x4& hi) {
  Frag8<T> f;
  if constexpr (sizeof(T) == 2) {
    const bf16x2 a = {(bf16)lo[0], (bf16)lo[1]}, b = {(bf16)lo[2], (bf16)lo[3]};
    const bf16x2 c = {(bf16)hi[0], (bf16)hi[1]}, d = {(bf16)hi[2], (bf16)hi[3]};
    const bf16x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    const bf16x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    f.v = __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f.v[i] = lo[i];
      f.v[4 + i] = hi[i];
    }
  }
  return f;
}

template <typename T>
__device__ __forceinline__ Frag4<T> frag4_from_acc(const f32x4& x) {
  Frag4<T> f;
  if constexpr (sizeof(T) == 2) {
    const bf16x2 a = {(bf16)x[0], (bf16)x[1]}, b = {(bf16)x[2], (bf16)x[3]};
    f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f.v[i] = x[i];
  }
  return f;
}

// ---------------------------------------------------------------------------
// Inverse of a 16x16 unit triangular block on the fp16 MFMA (the forward's
// diagonal blocks, and the backward's with bf16 operands).
// ---------------------------------------------------------------------------
typedef _Float16 sb_h4 __attribute__((ext_vector_type(4)));
typedef _Float16 sb_h2 __attribute__((ext_vector_type(2)));
typedef float sb_f2 __attribute__((ext_vector_type(2)));

// Largest entry of N the fp16 inverse accepts.  With |N| <= m entrywise, an
// entry of N^k is at most m^k C(14, k - 1) (paths of k strictly descending
// steps), so every power and partial product below stays under
// m (1 + m)^14 = 4.3e4 for m = 1.125, inside fp16's 65504; above it the
// caller takes another path (the forward: the exact token recurrence; the
// backward: the fp32 chain).  Unit keys with gates in [0, 1] and decay <= 1
// give |N| <= 1.
constexpr float kNBig = 1.125f;

// (I + A)^{-1} of a 16x16 unit lower-triangular matrix from N = -A (strictly
// lower, N^16 = 0):  (I + A)^{-1} = (I + N)(I + N^2)(I + N^4)(I + N^8), on the
// fp16 MFMA with fp32 accumulation (one v_mfma_f32_16x16x16_f16 per product;
// fp16 operands carry 11 significant bits, finer than the bf16 in which T is
// stored).  Layouts (lane = 16 g + j):
//   rowL(X): X[j][4g + i]      accL(X): X[4g + i][j]
// mma(acc, rowL(X), accL(Y)) adds accL(X Y); accL(X) = rowL(X^T).
// In: nr = rowL(N), nc = accL(N).  Out: rowL(T), T = (I + A)^{-1}, and nmax =
// the lane's largest |N| entry.
__device__ __forceinline__ Frag4<float> unit_lower_inverse(const Frag4<float>& nr,
                                                           const Frag4<float>& nc, int g, int j,
                                                           float& nmax) {
  auto h = [](float a, float b, float c, float d) {
    const sb_h2 lo = __builtin_convertvector((sb_f2){a, b}, sb_h2);
    const sb_h2 hi = __builtin_convertvector((sb_f2){c, d}, sb_h2);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
  };
  nmax = fmaxf(fmaxf(fabsf(nr.v[0]), fabsf(nr.v[1])), fmaxf(fabsf(nr.v[2]), fabsf(nr.v[3])));
  auto hv = [&h](const f32x4& x) { return h(x[0], x[1], x[2], x[3]); };
  auto mma = [](const sb_h4& a, const sb_h4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  };
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  const sb_h4 hr = h(nr.v[0], nr.v[1], nr.v[2], nr.v[3]);
  const sb_h4 hc = h(nc.v[0], nc.v[1], nc.v[2], nc.v[3]);
  const sb_h4 n2c = hv(mma(hr, hc, z));    // accL(N^2)
  const sb_h4 n2r = hv(mma(hc, hr, z));    // rowL(N^2)
  const sb_h4 n4c = hv(mma(n2r, n2c, z));  // accL(N^4)
  const sb_h4 n4r = hv(mma(n2c, n2r, z));  // rowL(N^4)
  const sb_h4 n8c = hv(mma(n4r, n4c, z));  // accL(N^8)
  // accL(T^T), T^T = (I + N^8)^T (I + N^4)^T (I + N^2)^T (I + N)^T, by left
  // products C + X C starting from accL((I + N)^T) = rowL(I + N); C enters
  // the accumulator in fp32 and only the product X C is rounded
  f32x4 t;
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = nr.v[i] + ((4 * g + i == j) ? 1.f : 0.f);
  t = mma(n2c, hv(t), t);
  t = mma(n4c, hv(t), t);
  t = mma(n8c, hv(t), t);
  Frag4<float> r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.v[i] = t[i];
  return r;  // accL(T^T) = rowL(T)
}


struct Params {
  int64_t B, T;      // sequences, tokens per sequence (packed total when cu is set)
  const int64_t* cu; // packed sequences: [B + 1] token offsets, or nullptr
  int Hk, Hv;
  float scale;
  const void *q, *k, *v, *b, *w, *g;
  const float* state_in;
  float* state_out;
  void* o;
  // Raw gate projections (the kernel applies the activations): b, g and w
  // are then the projections of beta|b, of the decay and of w, read with
  // these row strides (elements); A_log and dt_bias are per column of g's
  // projection, or nullptr (0).
  int64_t ld_b = 0, ld_g = 0, ld_w = 0;
  const float* A_log = nullptr;
  const float* dt_bias = nullptr;
  // Optional (nullptr: not written): the state entering every 16-token block
  // and every u, bf16, in the layouts the backward's reverse walk reads (see
  // backward.hip); ck_slots and ck_nblk are its slot count and blocks per
  // sequence.
  bf16* ck = nullptr;
  bf16* u = nullptr;
  int64_t ck_slots = 0, ck_nblk = 0;
};

}  // namespace
}  // namespace gdn
