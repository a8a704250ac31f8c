// decode.hip -- single-token decode step of the gated delta rule on gfx950.
//
// Per (sequence n, value head h) the d_k x d_v fp32 state S is streamed once
// from HBM and once back.  Expanding the update ("Gated DeltaNet-2",
// Methodologie §1) with S_bar = Diag(alpha) S:
//
//   r   = S_bar^T e          = sum_i alpha_i e_i S_i,:           (e = b (.) k)
//   S'  = S_bar + k (z - r)^T                                     (z = w (.) v)
//   o   = scale * S'^T q     = scale * (sum_i alpha_i q_i S_i,: + (q.k)(z - r))
//
// so both row reductions (r and the alpha-weighted q read) come from ONE read
// of S, and S' is written from the registers that hold it.  The kernel is
// bound by HBM bandwidth: 2 * 4 * d_k * d_v bytes of state per head against
// about 6 flops per state element.
//
// Layout: one 256-thread workgroup per (n, h).  A thread owns 4 consecutive
// columns (one 16-byte access per row) and DK*DV/1024 consecutive rows; a
// wave's load instruction touches whole 512-byte (or 256-byte) row segments.
// Column partial sums are reduced across the row groups of a wave with
// cross-lane shuffles, then across the 4 waves through LDS.
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

namespace gdn {
namespace {

constexpr int kDecodeThreads = 256;

template <typename GT>
__device__ __forceinline__ float gate_val(const GT* p, int64_t i) {
  return to_f32(p[i]);
}

template <int DK, int DV, bool CHANNEL, bool HAS_G, typename IO, typename GT>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    int Hk, int Hv, float scale, const IO* __restrict__ q, const IO* __restrict__ k,
    const IO* __restrict__ v, const GT* __restrict__ bb, const GT* __restrict__ ww,
    const GT* __restrict__ gg, float* __restrict__ S, IO* __restrict__ o) {
  constexpr int CG = DV / 4;               // column groups of 4 floats
  constexpr int RG = kDecodeThreads / CG;  // row groups
  constexpr int RPT = DK / RG;             // rows per thread
  constexpr int WAVES = kDecodeThreads / 64;
  constexpr int RG_PER_WAVE = 64 / CG;
  static_assert(RPT >= 1 && DK % RG == 0, "shape");

  const int64_t head = blockIdx.x;  // n * Hv + h
  const int64_t n = head / Hv;
  const int h = (int)(head - n * Hv);
  const int hk = h / (Hv / Hk);
  const int tid = threadIdx.x;
  const int cg = tid % CG;
  const int rg = tid / CG;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)

  float* __restrict__ Sh = S + head * (int64_t)(DK * DV);

  // 1. Issue the state loads first: they are the whole cost of the kernel.
  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg * RPT + i;
    s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sh + row * DV + 4 * cg));
  }

  // 2. Per-row factors into LDS: alpha_i, alpha_i e_i, alpha_i q_i, k_i; and q.k.
  __shared__ float s_alpha[DK], s_ae[DK], s_aq[DK], s_k[DK];
  __shared__ float s_qk[WAVES];
  __shared__ float s_red[WAVES][CG][8];
  lds_nan_fill(s_alpha, sizeof s_alpha);
  lds_nan_fill(s_ae, sizeof s_ae);
  lds_nan_fill(s_aq, sizeof s_aq);
  lds_nan_fill(s_k, sizeof s_k);
  lds_nan_fill(s_qk, sizeof s_qk);
  lds_nan_fill(s_red, sizeof s_red);

  const IO* qh = q + (n * Hk + hk) * (int64_t)DK;
  const IO* kh = k + (n * Hk + hk) * (int64_t)DK;
  float qk_part = 0.f;
  if (tid < DK) {
    const float qi = to_f32(qh[tid]);
    const float ki = to_f32(kh[tid]);
    float bi, gi;
    if constexpr (CHANNEL) {
      bi = gate_val(bb, head * DK + tid);
      gi = HAS_G ? gate_val(gg, head * DK + tid) : 0.f;
    } else {
      bi = gate_val(bb, head);
      gi = HAS_G ? gate_val(gg, head) : 0.f;
    }
    const float ai = HAS_G ? exp2_fast(gi * kLog2e) : 1.f;
    s_alpha[tid] = ai;
    s_ae[tid] = ai * bi * ki;
    s_aq[tid] = ai * qi;
    s_k[tid] = ki;
    qk_part = qi * ki;
  }
  // q.k over the first DK threads (whole waves, DK is 64 or 128).
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) qk_part += __shfl_xor(qk_part, off);
  if (lane == 0) s_qk[wave] = qk_part;
  __syncthreads();

  // 3. Column partial sums over this thread's rows.
  float r[4] = {0.f, 0.f, 0.f, 0.f};
  float p[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg * RPT + i;
    const float ae = s_ae[row];
    const float aq = s_aq[row];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[j] += ae * s[i][j];
      p[j] += aq * s[i][j];
    }
  }
  // Reduce over the row groups inside the wave (lanes CG apart).
#pragma unroll
  for (int off = CG; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[j] += __shfl_xor(r[j], off);
      p[j] += __shfl_xor(p[j], off);
    }
  }
  if (lane < CG) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s_red[wave][cg][j] = r[j];
      s_red[wave][cg][4 + j] = p[j];
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float rs = 0.f, ps = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      rs += s_red[w][cg][j];
      ps += s_red[w][cg][4 + j];
    }
    r[j] = rs;
    p[j] = ps;
  }
  (void)RG_PER_WAVE;

  // 4. Gated write target for this thread's columns: z = w (.) v.
  float vz[4];
  load_f32<4, IO>(v + head * (int64_t)DV + 4 * cg, vz);
  if constexpr (CHANNEL) {
    float wz[4];
    load_f32<4, GT>(ww + head * (int64_t)DV + 4 * cg, wz);
#pragma unroll
    for (int j = 0; j < 4; ++j) vz[j] *= wz[j];
  } else {
    const float beta = gate_val(bb, head);
#pragma unroll
    for (int j = 0; j < 4; ++j) vz[j] *= beta;
  }
  float d[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) d[j] = vz[j] - r[j];  // z - r

  // 5. Write S' = Diag(alpha) S + k (z - r)^T back in place.
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg * RPT + i;
    const float a = s_alpha[row];
    const float kr = s_k[row];
    f32x4 out;
#pragma unroll
    for (int j = 0; j < 4; ++j) out[j] = a * s[i][j] + kr * d[j];
    __builtin_nontemporal_store(out, reinterpret_cast<f32x4*>(Sh + row * DV + 4 * cg));
  }

  // 6. o = scale * (p + (q.k)(z - r)), one row group writes it.
  if (rg == 0) {
    float qk = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) qk += (w * 64 < DK) ? s_qk[w] : 0.f;
    float ov[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ov[j] = scale * (p[j] + qk * d[j]);
    store4<IO>(o + head * (int64_t)DV + 4 * cg, ov[0], ov[1], ov[2], ov[3]);
  }
}

template <int DK, int DV, bool CH, bool HG, typename IO, typename GT>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  const int64_t heads = a.N * a.Hv;
  decode_kernel<DK, DV, CH, HG, IO, GT><<<dim3((unsigned)heads), dim3(kDecodeThreads), 0, stream>>>(
      a.Hk, a.Hv, a.scale, static_cast<const IO*>(a.q), static_cast<const IO*>(a.k),
      static_cast<const IO*>(a.v), static_cast<const GT*>(a.b), static_cast<const GT*>(a.w),
      static_cast<const GT*>(a.g), a.state, static_cast<IO*>(a.o));
  return hipGetLastError();
}

template <int DK, int DV, bool CH, bool HG>
hipError_t pick_types(const DecodeArgs& a, hipStream_t s) {
  if (a.io == DType::BF16 && a.gate == DType::BF16) return launch_typed<DK, DV, CH, HG, bf16, bf16>(a, s);
  if (a.io == DType::BF16 && a.gate == DType::F32) return launch_typed<DK, DV, CH, HG, bf16, float>(a, s);
  return launch_typed<DK, DV, CH, HG, float, float>(a, s);
}

template <int DK, int DV>
hipError_t pick_gates(const DecodeArgs& a, hipStream_t s) {
  const bool hg = a.g != nullptr;
  if (a.channel) return hg ? pick_types<DK, DV, true, true>(a, s) : pick_types<DK, DV, true, false>(a, s);
  return hg ? pick_types<DK, DV, false, true>(a, s) : pick_types<DK, DV, false, false>(a, s);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.dk == 128 && a.dv == 128) return pick_gates<128, 128>(a, stream);
  if (a.dk == 128 && a.dv == 64) return pick_gates<128, 64>(a, stream);
  if (a.dk == 64 && a.dv == 128) return pick_gates<64, 128>(a, stream);
  return pick_gates<64, 64>(a, stream);
}

#ifdef GDN_CHECK
unsigned check_violations_decode() { return take_check_violations(); }
#endif

}  // namespace gdn
