// layer_ops.hip -- the memory-bound operations around the recurrence in a
// Gated DeltaNet block, on gfx950:
//
//   short_conv  : q, k, v branch -- depthwise causal convolution of kernel 4,
//                 SiLU, and an L2 norm per head for q and k (notes "Gated
//                 DeltaNet", Figure 1 block; architecture notes §La
//                 convolution causale).
//   gates       : beta = sigmoid(b), Mamba-2 decay g = log(alpha) =
//                 -exp(A_log) softplus(a + dt_bias), and the GDN-2 write gate
//                 w = sigmoid(w_raw).
//   output_gate : RMS norm of each value head's output times swish(z)
//                 (architecture notes §La porte de sortie).
//
// All three stream their operands once through HBM at a few flops per byte,
// so each is laid out for coalesced 16-byte accesses and enough loads in
// flight; none uses LDS or a scratch buffer.
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

#include <type_traits>

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kConvTokens = 128;  // tokens per short-conv workgroup

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* out) {
  load_f32<8, T>(p, out);
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float* v) {
  store4<T>(p, v[0], v[1], v[2], v[3]);
  store4<T>(p + 4, v[4], v[5], v[6], v[7]);
}

// x * sigmoid(x) with the hardware exp and reciprocal: exp(-x) overflows to
// +inf for x < -88, where the result is then -0 as it should be.
__device__ __forceinline__ float silu(float x) {
  const float e = exp2_fast(-x * kLog2e);
  return x * __builtin_amdgcn_rcpf(1.f + e);
}

// Sum over the L consecutive lanes (L = 8 or 16, aligned) that hold one row,
// as a butterfly of DPP moves inside each 16-lane row: swap neighbours, swap
// pairs, then fold the 8-lane halves and the 16-lane row onto their mirrors.
template <int L>
__device__ __forceinline__ float row_sum(float s) {
  static_assert(L == 8 || L == 16, "row width");
  auto dpp = [](float v, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), decltype(ctrl)::value, 0xf, 0xf, false));
  };
  s += dpp(s, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  s += dpp(s, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  s += dpp(s, std::integral_constant<int, 0x141>{});  // row_half_mirror
  if constexpr (L == 16) s += dpp(s, std::integral_constant<int, 0x140>{});  // row_mirror
  return s;
}

// 8 consecutive elements kept as loaded (converted when used), so that many
// rows can be in flight at the cost of 4 (bf16) or 8 (fp32) registers each.
template <typename T> struct Raw8;
template <> struct Raw8<bf16> { uint4 u; };
template <> struct Raw8<float> { float4 a, b; };

__device__ __forceinline__ void ld_raw8(const bf16* p, Raw8<bf16>& r) {
  r.u = *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void ld_raw8(const float* p, Raw8<float>& r) {
  r.a = reinterpret_cast<const float4*>(p)[0];
  r.b = reinterpret_cast<const float4*>(p)[1];
}
__device__ __forceinline__ void unpack8(const Raw8<bf16>& r, float* out) {
  const uint32_t w[4] = {r.u.x, r.u.y, r.u.z, r.u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack8(const Raw8<float>& r, float* out) {
  out[0] = r.a.x; out[1] = r.a.y; out[2] = r.a.z; out[3] = r.a.w;
  out[4] = r.b.x; out[5] = r.b.y; out[6] = r.b.z; out[7] = r.b.w;
}

// ---------------------------------------------------------------------------
// Short causal convolution.
//
// Grid: x = heads of the branch (q heads, then k heads, then v heads), y =
// blocks of kConvTokens packed tokens, so that the workgroups running
// together read whole rows of x (all heads of the same tokens) rather than
// one head's 256-byte piece of many rows (measured 1.4x faster).  A head of
// width D is covered by D/8 lanes with 8 channels each (one 16-byte bf16
// access per row); the workgroup's 256 threads form 2048/D streams that each
// walk kConvTokens*D/2048 consecutive tokens (8 for D = 128, the fastest of
// 4, 8, 16 and 32), keeping the three previous inputs in registers so every
// input row is read once from HBM (the 3-row halo of a stream is its
// neighbour's rows, served by L2).  A stream that lies
// inside one sequence with its halo takes a branch-free path; a stream that
// touches a sequence start fetches the history from the carried conv state.
// ---------------------------------------------------------------------------
struct SeqPos {
  int64_t n, start, end;
  bool hist;  // the tokens before `start` come from the carried state
};

__device__ __forceinline__ int64_t clamp_off(const int64_t* cu, int64_t i, int64_t total) {
  const int64_t c = cu[i];
  return c < 0 ? 0 : (c > total ? total : c);
}

// Sequence of token r: N equal sequences, or the last n with cu[n] <= r
// (offsets clamped into [0, total]).  For well-formed offsets this is the
// sequence that holds r; for malformed ones it is some n whose range keeps
// every access inside the tensors.
__device__ SeqPos find_seq(const ConvArgs& p, int64_t r) {
  SeqPos s;
  if (!p.cu_seqlens) {
    s.n = r / p.Tseq;
    s.start = s.n * p.Tseq;
    s.end = s.start + p.Tseq;
    s.hist = true;
    return s;
  }
  int64_t lo = 0, hi = p.N;
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) >> 1;
    if (clamp_off(p.cu_seqlens, mid, p.total_T) <= r) lo = mid; else hi = mid;
  }
  s.n = lo;
  s.start = clamp_off(p.cu_seqlens, lo, p.total_T);
  s.end = clamp_off(p.cu_seqlens, lo + 1, p.total_T);
  s.hist = true;
  if (s.start > r) { s.start = r; s.hist = false; }  // before the first sequence
  if (s.end <= r) s.end = r + 1;
  return s;
}

template <typename T, int D, bool NORM>
__device__ __forceinline__ void conv_head(const ConvArgs& p, int64_t blk, int64_t col,
                                          T* __restrict__ out, int64_t out_ld) {
  constexpr int TPR = D / 8;              // lanes per token row
  constexpr int TB = kConvTokens * TPR / kThreads;  // tokens per stream
  const int tid = threadIdx.x;
  const int l8 = tid % TPR;
  const int stream = tid / TPR;
  const int64_t c = col + 8 * l8;         // first channel of this lane
  const int64_t C = p.C;
  const T* __restrict__ x = static_cast<const T*>(p.x);
  const T* __restrict__ s_in = static_cast<const T*>(p.s_in);

  float w[4][8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 t = *reinterpret_cast<const float4*>(p.w + (c + i) * 4);
    w[0][i] = t.x; w[1][i] = t.y; w[2][i] = t.z; w[3][i] = t.w;
  }

  const int64_t r0 = blk * kConvTokens + (int64_t)stream * TB;
  if (r0 >= p.total_T) return;

  auto finish = [&](int64_t r, float* acc) {
    float y[8];
    if constexpr (NORM) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) { y[i] = silu(acc[i]); ss += y[i] * y[i]; }
      ss = row_sum<TPR>(ss);
      const float inv = __builtin_amdgcn_rsqf(ss + p.eps);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] *= inv;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = silu(acc[i]);
    }
    store8<T>(out + r * out_ld + 8 * l8, y);
  };

  SeqPos sp = find_seq(p, r0);
  if (sp.hist && sp.start <= r0 - 3 && r0 + TB <= sp.end) {
    // Whole stream and its halo inside one sequence.  Every row load is
    // issued before any arithmetic (the scheduling barrier keeps the
    // compiler from spreading them over the token loop).
    Raw8<T> H[3], X[TB];
#pragma unroll
    for (int j = 0; j < 3; ++j) ld_raw8(x + (r0 - 3 + j) * p.ld_x + c, H[j]);
#pragma unroll
    for (int t = 0; t < TB; ++t) ld_raw8(x + (r0 + t) * p.ld_x + c, X[t]);
    __builtin_amdgcn_sched_barrier(0);
    float h[3][8];
#pragma unroll
    for (int j = 0; j < 3; ++j) unpack8(H[j], h[j]);
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      float xt[8], acc[8];
      unpack8(X[t], xt);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc[i] = w[0][i] * h[0][i] + w[1][i] * h[1][i] + w[2][i] * h[2][i] + w[3][i] * xt[i];
#pragma unroll
      for (int i = 0; i < 8; ++i) { h[0][i] = h[1][i]; h[1][i] = h[2][i]; h[2][i] = xt[i]; }
      finish(r0 + t, acc);
    }
    return;
  }
  // A sequence starts inside the stream or its halo, or the stream ends the
  // tensor: fetch every tap on its own.  Every lane of a row takes the same
  // path (the branch depends on the token only), so the row sum stays whole.
  for (int t = 0; t < TB; ++t) {
    const int64_t r = r0 + t;
    if (r >= p.total_T) break;
    if (r >= sp.end) sp = find_seq(p, r);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t pp = r - 3 + j;
      float xv[8];
      if (pp >= sp.start) {
        load8<T>(x + pp * p.ld_x + c, xv);
      } else if (sp.hist && s_in) {
        load8<T>(s_in + (sp.n * 3 + (pp - sp.start + 3)) * C + c, xv);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[i] = 0.f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += w[j][i] * xv[i];
    }
    finish(r, acc);
  }
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(kThreads) void short_conv_kernel(ConvArgs p) {
  const int hh = blockIdx.x;
  const int64_t nblk = (p.total_T + kConvTokens - 1) / kConvTokens;
  for (int64_t blk = blockIdx.y; blk < nblk; blk += gridDim.y) {
    if (hh < p.Hk) {
      conv_head<T, DK, true>(p, blk, (int64_t)hh * DK, static_cast<T*>(p.q) + (int64_t)hh * DK,
                             (int64_t)p.Hk * DK);
    } else if (hh < 2 * p.Hk) {
      const int h = hh - p.Hk;
      conv_head<T, DK, true>(p, blk, (int64_t)(p.Hk + h) * DK,
                             static_cast<T*>(p.k) + (int64_t)h * DK, (int64_t)p.Hk * DK);
    } else {
      const int h = hh - 2 * p.Hk;
      conv_head<T, DV, false>(p, blk, (int64_t)2 * p.Hk * DK + (int64_t)h * DV,
                              static_cast<T*>(p.v) + (int64_t)h * DV, (int64_t)p.Hv * DV);
    }
  }
}

// New conv state of every sequence: its last three inputs, the older entries
// of its carried state filling in for a sequence shorter than three tokens.
// One thread per (sequence, channel) reads all three entries before it
// writes any, so the state may be updated in place.  Runs after the
// convolution on the same stream, which has finished reading the old state.
template <typename T>
__global__ __launch_bounds__(kThreads) void conv_state_kernel(ConvArgs p) {
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (c >= p.C) return;
  const T* x = static_cast<const T*>(p.x);
  const T* s_in = static_cast<const T*>(p.s_in);
  T* s_out = static_cast<T*>(p.s_out);
  for (int64_t n = blockIdx.y; n < p.N; n += gridDim.y) {
    int64_t a0, a1;
    if (p.cu_seqlens) {
      a0 = clamp_off(p.cu_seqlens, n, p.total_T);
      a1 = clamp_off(p.cu_seqlens, n + 1, p.total_T);
      if (a1 < a0) a1 = a0;
    } else {
      a0 = n * p.Tseq;
      a1 = a0 + p.Tseq;
    }
    const int64_t L = a1 - a0;
    T vals[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int64_t i = L + j;  // position in [carried state (3), sequence inputs]
      if (i >= 3) vals[j] = x[(a0 + i - 3) * p.ld_x + c];
      else vals[j] = s_in ? s_in[(n * 3 + i) * p.C + c] : from_f32<T>(0.f);
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) s_out[(n * 3 + j) * p.C + c] = vals[j];
  }
}

// ---------------------------------------------------------------------------
// Gate activations (sigmoid_f, softplus_f: gdn_device.hpp).  The vector
// kernel handles 8 consecutive columns per thread (every row stride a
// multiple of 8 and the pointers 16-byte aligned); the scalar kernel one
// element.  Flat indices are 32-bit (the host checks the counts fit).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float decay_f(float a, float A_log, float dt) {
  return log_decay_f(a, neg_exp_f(A_log), dt);
}

template <typename TI, typename TO>
__global__ __launch_bounds__(kThreads) void gates_kernel(GateArgs p) {
  const uint32_t e = blockIdx.x * kThreads + threadIdx.x;
  const TI* a = static_cast<const TI*>(p.a);
  const TI* b = static_cast<const TI*>(p.b);
  if (e < p.n_ab_total) {
    const uint32_t r = e / p.n_ab, col = e - r * p.n_ab;
    const float av = to_f32(a[(int64_t)r * p.ld_a + col]);
    const float bv = to_f32(b[(int64_t)r * p.ld_b + col]);
    const float Al = p.A_log ? p.A_log[col] : 0.f;
    const float dt = p.dt_bias ? p.dt_bias[col] : 0.f;
    static_cast<TO*>(p.g)[e] = from_f32<TO>(decay_f(av, Al, dt));
    static_cast<TO*>(p.beta)[e] = from_f32<TO>(sigmoid_f(bv));
  }
  if (e < p.n_w_total) {
    const uint32_t r = e / p.n_w, col = e - r * p.n_w;
    const float wv = to_f32(static_cast<const TI*>(p.w_raw)[(int64_t)r * p.ld_w + col]);
    static_cast<TO*>(p.w)[e] = from_f32<TO>(sigmoid_f(wv));
  }
}

__device__ __forceinline__ void ld_params8(const float* p, int64_t col, float dflt, float* out) {
  if (p) {
    const float4 u = *reinterpret_cast<const float4*>(p + col);
    const float4 v = *reinterpret_cast<const float4*>(p + col + 4);
    out[0] = u.x; out[1] = u.y; out[2] = u.z; out[3] = u.w;
    out[4] = v.x; out[5] = v.y; out[6] = v.z; out[7] = v.w;
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = dflt;
  }
}

template <typename TI, typename TO>
__global__ __launch_bounds__(kThreads) void gates_vec_kernel(GateArgs p) {
  const uint32_t e = blockIdx.x * kThreads + threadIdx.x;   // group of 8 elements
  const uint32_t nab8 = p.n_ab >> 3, nw8 = p.n_w >> 3;
  Raw8<TI> ra, rb, rw;
  uint32_t r = 0, c8 = 0, rw_ = 0, cw8 = 0;
  const bool ab = e < (p.n_ab_total >> 3), ww = e < (p.n_w_total >> 3);
  if (ab) {
    r = e / nab8; c8 = e - r * nab8;
    ld_raw8(static_cast<const TI*>(p.a) + (int64_t)r * p.ld_a + 8 * c8, ra);
    ld_raw8(static_cast<const TI*>(p.b) + (int64_t)r * p.ld_b + 8 * c8, rb);
  }
  if (ww) {
    rw_ = e / nw8; cw8 = e - rw_ * nw8;
    ld_raw8(static_cast<const TI*>(p.w_raw) + (int64_t)rw_ * p.ld_w + 8 * cw8, rw);
  }
  if (ab) {
    float av[8], bv[8], Al[8], dt[8], g[8], be[8];
    unpack8(ra, av);
    unpack8(rb, bv);
    ld_params8(p.A_log, 8 * (int64_t)c8, 0.f, Al);
    ld_params8(p.dt_bias, 8 * (int64_t)c8, 0.f, dt);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      g[i] = decay_f(av[i], Al[i], dt[i]);
      be[i] = sigmoid_f(bv[i]);
    }
    store8<TO>(static_cast<TO*>(p.g) + 8 * (int64_t)e, g);
    store8<TO>(static_cast<TO*>(p.beta) + 8 * (int64_t)e, be);
  }
  if (ww) {
    float wv[8];
    unpack8(rw, wv);
#pragma unroll
    for (int i = 0; i < 8; ++i) wv[i] = sigmoid_f(wv[i]);
    store8<TO>(static_cast<TO*>(p.w) + 8 * (int64_t)e, wv);
  }
}

// ---------------------------------------------------------------------------
// Output norm and gate.  A (token, value head) row of DV elements is held by
// DV/8 lanes; a workgroup covers 2048/DV rows per pass and kOutPasses passes,
// with every pass's loads issued before the first row is reduced.  y may
// alias o: each lane reads its own elements before it writes them.
// ---------------------------------------------------------------------------
constexpr int kOutPasses = 4;

template <typename T, int DV>
__global__ __launch_bounds__(kThreads) void output_gate_kernel(NormArgs p) {
  constexpr int TPR = DV / 8;
  constexpr int G = kThreads / TPR;       // rows per pass
  const int l8 = threadIdx.x % TPR;
  const int grp = threadIdx.x / TPR;
  const int64_t nrows = p.rows * p.Hv;
  const T* o = static_cast<const T*>(p.o);
  const T* z = static_cast<const T*>(p.z);
  T* y = static_cast<T*>(p.y);

  float wt[8];
  {
    const float4 a = *reinterpret_cast<const float4*>(p.weight + 8 * l8);
    const float4 b = *reinterpret_cast<const float4*>(p.weight + 8 * l8 + 4);
    wt[0] = a.x; wt[1] = a.y; wt[2] = a.z; wt[3] = a.w;
    wt[4] = b.x; wt[5] = b.y; wt[6] = b.z; wt[7] = b.w;
  }
  float ov[kOutPasses][8], zv[kOutPasses][8];
  int64_t row[kOutPasses];
#pragma unroll
  for (int it = 0; it < kOutPasses; ++it) {
    int64_t pr = ((int64_t)blockIdx.x * kOutPasses + it) * G + grp;
    row[it] = pr;
    if (pr >= nrows) pr = nrows - 1;      // loads stay in bounds; the store is skipped
    const int64_t tok = pr / p.Hv;
    const int64_t h = pr - tok * p.Hv;
    load8<T>(o + pr * DV + 8 * l8, ov[it]);
    load8<T>(z + tok * p.ld_z + h * DV + 8 * l8, zv[it]);
  }
#pragma unroll
  for (int it = 0; it < kOutPasses; ++it) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += ov[it][i] * ov[it][i];
    ss = row_sum<TPR>(ss);
    const float inv = __builtin_amdgcn_rsqf(ss * (1.f / DV) + p.eps);
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = ov[it][i] * inv * wt[i] * silu(zv[it][i]);
    if (row[it] < nrows) store8<T>(y + row[it] * DV + 8 * l8, r);
  }
}

template <typename T>
hipError_t launch_short_conv_t(const ConvArgs& a, hipStream_t stream) {
  const int heads = 2 * a.Hk + a.Hv;
  if (a.total_T > 0) {
    const int64_t blocks = (a.total_T + kConvTokens - 1) / kConvTokens;
    const dim3 grid((unsigned)heads, (unsigned)(blocks < 65535 ? blocks : 65535));
    if (a.dk == 128 && a.dv == 128) short_conv_kernel<T, 128, 128><<<grid, kThreads, 0, stream>>>(a);
    else if (a.dk == 128) short_conv_kernel<T, 128, 64><<<grid, kThreads, 0, stream>>>(a);
    else if (a.dv == 128) short_conv_kernel<T, 64, 128><<<grid, kThreads, 0, stream>>>(a);
    else short_conv_kernel<T, 64, 64><<<grid, kThreads, 0, stream>>>(a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.s_out) {
    const dim3 grid((unsigned)((a.C + kThreads - 1) / kThreads),
                    (unsigned)(a.N < 65535 ? a.N : 65535));
    conv_state_kernel<T><<<grid, kThreads, 0, stream>>>(a);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename TI, typename TO>
hipError_t launch_gates_t(const GateArgs& a, hipStream_t stream) {
  const int64_t n = a.n_ab_total > a.n_w_total ? a.n_ab_total : a.n_w_total;
  auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  const bool vec = a.n_ab % 8 == 0 && a.n_w % 8 == 0 && a.ld_a % 8 == 0 && a.ld_b % 8 == 0 &&
                   a.ld_w % 8 == 0 && al16(a.a) && al16(a.b) && al16(a.g) && al16(a.beta) &&
                   (!a.w_raw || (al16(a.w_raw) && al16(a.w))) &&
                   (!a.A_log || al16(a.A_log)) && (!a.dt_bias || al16(a.dt_bias));
  if (vec) {
    const int64_t n8 = n / 8;
    gates_vec_kernel<TI, TO><<<dim3((unsigned)((n8 + kThreads - 1) / kThreads)), kThreads, 0,
                               stream>>>(a);
  } else {
    gates_kernel<TI, TO><<<dim3((unsigned)((n + kThreads - 1) / kThreads)), kThreads, 0,
                           stream>>>(a);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_output_gate_t(const NormArgs& a, hipStream_t stream) {
  const int64_t nrows = a.rows * a.Hv;
  const int64_t per_block = (int64_t)kOutPasses * (kThreads / (a.dv / 8));
  const dim3 grid((unsigned)((nrows + per_block - 1) / per_block));
  if (a.dv == 128) output_gate_kernel<T, 128><<<grid, kThreads, 0, stream>>>(a);
  else output_gate_kernel<T, 64><<<grid, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_short_conv(const ConvArgs& a, hipStream_t stream) {
  return a.io == DType::F32 ? launch_short_conv_t<float>(a, stream)
                            : launch_short_conv_t<bf16>(a, stream);
}

hipError_t launch_gates(const GateArgs& a, hipStream_t stream) {
  if (a.n_ab_total == 0 && a.n_w_total == 0) return hipSuccess;
  if (a.in == DType::F32)
    return a.out == DType::F32 ? launch_gates_t<float, float>(a, stream)
                               : launch_gates_t<float, bf16>(a, stream);
  return a.out == DType::F32 ? launch_gates_t<bf16, float>(a, stream)
                             : launch_gates_t<bf16, bf16>(a, stream);
}

hipError_t launch_output_gate(const NormArgs& a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  return a.io == DType::F32 ? launch_output_gate_t<float>(a, stream)
                            : launch_output_gate_t<bf16>(a, stream);
}

}  // namespace gdn
