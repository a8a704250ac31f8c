// backward.hip -- gradients of the gated delta rule on gfx950 (reverse mode
// through the token recurrence).
//
// With P_t the state before token t, abar = exp(g_t), e = b (.) k,
// z = w (.) v, the forward step is
//   Sbar = Diag(abar) P_t,  r = Sbar^T e,  u = z - r,
//   P_{t+1} = Sbar + k u^T,  o_t = scale P_{t+1}^T q_t,
// and the reverse step, with D the gradient w.r.t. P_{t+1}:
//   D += scale q dO^T;  dq = scale P_{t+1} dO;  du = D^T k;
//   dv = w (.) du;  dw = v (.) du;  de = -Sbar du;
//   dk = D u + b (.) de;  db = k (.) de;  dSbar = D - e du^T;
//   dg = abar (.) rowsum(dSbar (.) P_t);  D <- Diag(abar) dSbar.
// The pages give the forward update ("Gated DeltaNet-2", Methodologie §1)
// and name the gate-aware gradient as what makes training work (§3); the
// formulas above are the chain rule through that update.
//
// Layout: one workgroup per (sequence, value head, block of 64 value
// columns); the fp32 state slice is DK x 64, 4 rows x 4 columns per thread
// (DK * 4 threads).  The 16 lanes of a DPP row hold the 64 columns of 4 rows,
// so sums over columns are DPP butterflies; sums over rows take two
// cross-lane shuffles and one LDS exchange (one barrier).
//
// Phase 1 runs the recurrence forward from the initial state, storing the
// state every kCkpt tokens and every u_t in the workspace.  Phase 2 walks the
// checkpoint blocks backwards: it rebuilds a block's states from its
// checkpoint with the stored u (no reduction is needed: P_{t+1} = abar P_t +
// k u^T), keeps the starts of its sub-blocks in LDS (each thread its own
// tile) and the states of one sub-block in registers, and runs the reverse
// step token by token.  The per-row gradients (dq, dk, db, dg) are partial
// over the column block; they go to the workspace and a second kernel sums
// them over column blocks and over the value heads of a key head.
#include "gdn_device.hpp"
#include "gdn_kernels.hpp"

#include <type_traits>

namespace gdn {
namespace {

constexpr int kCkpt = 16;            // tokens between stored states
constexpr int kSub = 4;              // tokens per register-resident sub-block
constexpr int kSubs = kCkpt / kSub;  // sub-blocks per checkpoint block
constexpr int kCols = 64;            // value columns per workgroup

// Sum over the 16 lanes of a DPP row (all lanes get the sum).
__device__ __forceinline__ float row16_sum(float s) {
  auto dpp = [](float v, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), decltype(ctrl)::value, 0xf, 0xf, false));
  };
  s += dpp(s, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  s += dpp(s, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  s += dpp(s, std::integral_constant<int, 0x141>{});  // row_half_mirror
  s += dpp(s, std::integral_constant<int, 0x140>{});  // row_mirror
  return s;
}

template <typename T>
__device__ __forceinline__ void ld4(const T* p, float* o) {
  if constexpr (sizeof(T) == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    o[0] = __uint_as_float(u.x << 16); o[1] = __uint_as_float(u.x & 0xffff0000u);
    o[2] = __uint_as_float(u.y << 16); o[3] = __uint_as_float(u.y & 0xffff0000u);
  } else {
    const float4 f = *reinterpret_cast<const float4*>(p);
    o[0] = f.x; o[1] = f.y; o[2] = f.z; o[3] = f.w;
  }
}
__device__ __forceinline__ void st4f(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

typedef float Tile[4][4];

// Row-side inputs of token t for a thread's 4 rows: k, e = b (.) k, b, abar.
template <int DK, bool CHANNEL, bool HAS_G, typename IO, typename GT>
__device__ __forceinline__ void load_rows(const BwdArgs& p, int64_t bt, int64_t bth, int hk,
                                          int r0, float* k, float* e, float* bb, float* a) {
  ld4<IO>(static_cast<const IO*>(p.k) + (bt * p.Hk + hk) * DK + r0, k);
  if constexpr (CHANNEL) {
    ld4<GT>(static_cast<const GT*>(p.b) + bth * DK + r0, bb);
    if constexpr (HAS_G) {
      float gg[4];
      ld4<GT>(static_cast<const GT*>(p.g) + bth * DK + r0, gg);
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = exp2_fast(gg[i] * kLog2e);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = 1.f;
    }
  } else {
    const float beta = to_f32(static_cast<const GT*>(p.b)[bth]);
    float av = 1.f;
    if constexpr (HAS_G) av = exp2_fast(to_f32(static_cast<const GT*>(p.g)[bth]) * kLog2e);
#pragma unroll
    for (int i = 0; i < 4; ++i) { bb[i] = beta; a[i] = av; }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) e[i] = bb[i] * k[i];
}

// Column-side write gate of token t for a thread's 4 columns.
template <bool CHANNEL, typename GT>
__device__ __forceinline__ void load_wgate(const BwdArgs& p, int64_t bth, int64_t c0, float* w) {
  if constexpr (CHANNEL) {
    ld4<GT>(static_cast<const GT*>(p.w) + bth * p.dv + c0, w);
  } else {
    const float beta = to_f32(static_cast<const GT*>(p.b)[bth]);
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = beta;
  }
}

// Sum of v[4] over all DK rows of the workgroup for each of the thread's 4
// columns: across the 4 row groups of a wave by shuffles, then across the
// waves through LDS (double-buffered, so one barrier per call).
template <int NW>
__device__ __forceinline__ void row_reduce(float* v, float (*red)[NW][kCols], int& buf, int lane,
                                           int wave, int cg) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[j] += __shfl_xor(v[j], 16);
    v[j] += __shfl_xor(v[j], 32);
  }
  if (lane < 16) st4f(&red[buf][wave][4 * cg], v);
  __syncthreads();
  float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float4 x = *reinterpret_cast<const float4*>(&red[buf][w][4 * cg]);
    s[0] += x.x; s[1] += x.y; s[2] += x.z; s[3] += x.w;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = s[j];
  buf ^= 1;
}

template <int DK, bool CHANNEL, bool HAS_G, typename IO, typename GT>
__global__ __launch_bounds__(DK * 4) void bwd_kernel(BwdArgs p) {
  constexpr int NT = DK * 4;
  constexpr int NW = NT / 64;
  __shared__ float red[2][NW][kCols];
  __shared__ float4 subs[kSubs][4][NT];     // sub-block start states, private per thread

  const int64_t head = blockIdx.x;          // b * Hv + hv
  const int cb = blockIdx.y;
  const int ncb = p.dv / kCols;
  const int64_t b = head / p.Hv;
  const int hv = (int)(head - b * p.Hv);
  const int hk = hv / (p.Hv / p.Hk);
  const int tid = threadIdx.x;
  const int rg = tid >> 4, cg = tid & 15;
  const int lane = tid & 63, wave = tid >> 6;
  const int r0 = 4 * rg;
  const int64_t c0 = (int64_t)cb * kCols + 4 * cg;
  const int64_t T = p.T;
  const int64_t NR = p.B * T * p.Hv;        // gradient rows (b, t, hv)
  const float scale = p.scale;
  int buf = 0;

  float* ck = p.ckpt + ((head * ncb + cb) * p.nblk) * (int64_t)DK * kCols;
  auto ck_at = [&](int64_t m, int i) { return ck + (m * DK + r0 + i) * kCols + 4 * cg; };

  // ---- phase 1: forward, storing checkpoints and u ----
  Tile P;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (p.state_in) {
      const float4 x = *reinterpret_cast<const float4*>(p.state_in + (head * DK + r0 + i) * p.dv + c0);
      P[i][0] = x.x; P[i][1] = x.y; P[i][2] = x.z; P[i][3] = x.w;
    } else {
      P[i][0] = P[i][1] = P[i][2] = P[i][3] = 0.f;
    }
  }
  for (int64_t t = 0; t < T; ++t) {
    if (t % kCkpt == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) st4f(ck_at(t / kCkpt, i), P[i]);
    }
    const int64_t bt = b * T + t, bth = bt * p.Hv + hv;
    float k[4], e[4], bb[4], a[4], w[4], v[4];
    load_rows<DK, CHANNEL, HAS_G, IO, GT>(p, bt, bth, hk, r0, k, e, bb, a);
    load_wgate<CHANNEL, GT>(p, bth, c0, w);
    ld4<IO>(static_cast<const IO*>(p.v) + bth * p.dv + c0, v);
    float r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) s += a[i] * P[i][j] * e[i];
      r[j] = s;
    }
    row_reduce<NW>(r, red, buf, lane, wave, cg);
    float u[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = w[j] * v[j] - r[j];
    if (rg == 0) st4f(p.u + bth * p.dv + c0, u);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) P[i][j] = a[i] * P[i][j] + k[i] * u[j];
  }

  // ---- phase 2: reverse ----
  Tile D, Pn;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) Pn[i][j] = P[i][j];
    if (p.d_state_out) {
      const float4 x = *reinterpret_cast<const float4*>(p.d_state_out + (head * DK + r0 + i) * p.dv + c0);
      D[i][0] = x.x; D[i][1] = x.y; D[i][2] = x.z; D[i][3] = x.w;
    } else {
      D[i][0] = D[i][1] = D[i][2] = D[i][3] = 0.f;
    }
  }

  // P_{t+1} = abar P_t + k u^T with the stored u.
  auto advance = [&](Tile& X, int64_t t) {
    const int64_t bt = b * T + t, bth = bt * p.Hv + hv;
    float k[4], e[4], bb[4], a[4], u[4];
    load_rows<DK, CHANNEL, HAS_G, IO, GT>(p, bt, bth, hk, r0, k, e, bb, a);
    const float4 uu = *reinterpret_cast<const float4*>(p.u + bth * p.dv + c0);
    u[0] = uu.x; u[1] = uu.y; u[2] = uu.z; u[3] = uu.w;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) X[i][j] = a[i] * X[i][j] + k[i] * u[j];
  };

  // Reverse step of token t: Pb = P_t, Pa = P_{t+1}, D = dL/dP_{t+1} -> dL/dP_t.
  auto reverse = [&](const Tile& Pb, const Tile& Pa, int64_t t) {
    const int64_t bt = b * T + t, bth = bt * p.Hv + hv;
    float k[4], e[4], bb[4], a[4], w[4], v[4], dO[4], q[4], u[4];
    load_rows<DK, CHANNEL, HAS_G, IO, GT>(p, bt, bth, hk, r0, k, e, bb, a);
    load_wgate<CHANNEL, GT>(p, bth, c0, w);
    ld4<IO>(static_cast<const IO*>(p.v) + bth * p.dv + c0, v);
    ld4<IO>(static_cast<const IO*>(p.d_o) + bth * p.dv + c0, dO);
    ld4<IO>(static_cast<const IO*>(p.q) + (bt * p.Hk + hk) * DK + r0, q);
    {
      const float4 uu = *reinterpret_cast<const float4*>(p.u + bth * p.dv + c0);
      u[0] = uu.x; u[1] = uu.y; u[2] = uu.z; u[3] = uu.w;
    }
    float dq[4], du[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        D[i][j] += scale * q[i] * dO[j];
        s += Pa[i][j] * dO[j];
      }
      dq[i] = scale * s;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) s += D[i][j] * k[i];
      du[j] = s;
    }
    row_reduce<NW>(du, red, buf, lane, wave, cg);
    if (rg == 0) {
      float dvv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) dvv[j] = w[j] * du[j];
      st4f(p.dv_out + bth * p.dv + c0, dvv);
      if constexpr (CHANNEL) {
        float dww[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) dww[j] = v[j] * du[j];
        st4f(p.dw + bth * p.dv + c0, dww);
      }
    }
    if constexpr (!CHANNEL) {
      float ws = v[0] * du[0] + v[1] * du[1] + v[2] * du[2] + v[3] * du[3];
      ws = row16_sum(ws);
      if (tid == 0) p.part[(int64_t)ncb * 4 * NR * DK + (int64_t)cb * NR + bth] = ws;
    }
    float de[4], dk[4], da[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float s = 0.f, sk = 0.f, sa = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s += Pb[i][j] * du[j];
        sk += D[i][j] * u[j];
        const float dsb = D[i][j] - e[i] * du[j];
        sa += dsb * Pb[i][j];
        D[i][j] = a[i] * dsb;
      }
      de[i] = -a[i] * s;
      dk[i] = sk;
      da[i] = sa;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dq[i] = row16_sum(dq[i]);
      de[i] = row16_sum(de[i]);
      dk[i] = row16_sum(dk[i]);
      da[i] = row16_sum(da[i]);
    }
    if (cg < 4) {
      float out[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[i] = cg == 0 ? dq[i]
               : cg == 1 ? dk[i] + bb[i] * de[i]
               : cg == 2 ? k[i] * de[i]
                         : a[i] * da[i];
      }
      st4f(p.part + (((int64_t)cb * 4 + cg) * NR + bth) * DK + r0, out);
    }
  };

  for (int64_t m = p.nblk - 1; m >= 0; --m) {
    const int64_t t0 = m * kCkpt;
    const int64_t t1 = (t0 + kCkpt < T) ? t0 + kCkpt : T;
    Tile X;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 x = *reinterpret_cast<const float4*>(ck_at(m, i));
      X[i][0] = x.x; X[i][1] = x.y; X[i][2] = x.z; X[i][3] = x.w;
    }
    // starts of the sub-blocks (each thread keeps its own tile)
    for (int s = 0; s < kSubs; ++s) {
      const int64_t ts = t0 + s * kSub;
      if (ts >= t1) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) subs[s][i][tid] = make_float4(X[i][0], X[i][1], X[i][2], X[i][3]);
      if (ts + kSub < t1)
        for (int j = 0; j < kSub; ++j) advance(X, ts + j);
    }
    for (int s = kSubs - 1; s >= 0; --s) {
      const int64_t ts = t0 + s * kSub;
      if (ts >= t1) continue;
      const int n = (int)((t1 - ts) < kSub ? (t1 - ts) : kSub);
      Tile R[kSub];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 x = subs[s][i][tid];
        R[0][i][0] = x.x; R[0][i][1] = x.y; R[0][i][2] = x.z; R[0][i][3] = x.w;
      }
#pragma unroll
      for (int j = 1; j < kSub; ++j) {
        if (j < n) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) R[j][i][c] = R[j - 1][i][c];
          advance(R[j], ts + j - 1);
        }
      }
#pragma unroll
      for (int j = kSub - 1; j >= 0; --j) {
        if (j < n) {
          reverse(R[j], Pn, ts + j);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) Pn[i][c] = R[j][i][c];
        }
      }
    }
  }
  if (p.d_state_in) {
#pragma unroll
    for (int i = 0; i < 4; ++i) st4f(p.d_state_in + (head * DK + r0 + i) * p.dv + c0, D[i]);
  }
}

// Sums the per-column-block partials: dq, dk over the value heads of each key
// head; db, dg per value head (summed over d_k in scalar mode, where the
// write-gate sums are added to dbeta).  One workgroup per (b, t).
template <int DK, bool CHANNEL>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdArgs p) {
  const int64_t bt = blockIdx.x;
  const int ncb = p.dv / kCols;
  const int G = p.Hv / p.Hk;
  const int64_t NR = p.B * p.T * p.Hv;
  auto part = [&](int cb, int vec, int64_t row, int i) {
    return p.part[(((int64_t)cb * 4 + vec) * NR + row) * DK + i];
  };
  for (int idx = threadIdx.x; idx < p.Hk * DK; idx += blockDim.x) {
    const int hk = idx / DK, i = idx - hk * DK;
    float sq = 0.f, sk = 0.f;
    for (int gi = 0; gi < G; ++gi) {
      const int64_t row = bt * p.Hv + hk * G + gi;
      for (int cb = 0; cb < ncb; ++cb) { sq += part(cb, 0, row, i); sk += part(cb, 1, row, i); }
    }
    p.dq_out[(bt * p.Hk + hk) * DK + i] = sq;
    p.dk_out[(bt * p.Hk + hk) * DK + i] = sk;
  }
  if constexpr (CHANNEL) {
    for (int idx = threadIdx.x; idx < p.Hv * DK; idx += blockDim.x) {
      const int hv = idx / DK, i = idx - hv * DK;
      const int64_t row = bt * p.Hv + hv;
      float sb = 0.f, sg = 0.f;
      for (int cb = 0; cb < ncb; ++cb) { sb += part(cb, 2, row, i); sg += part(cb, 3, row, i); }
      p.db[row * DK + i] = sb;
      if (p.dg) p.dg[row * DK + i] = sg;
    }
  } else {
    for (int hv = threadIdx.x; hv < p.Hv; hv += blockDim.x) {
      const int64_t row = bt * p.Hv + hv;
      float sb = 0.f, sg = 0.f;
      for (int cb = 0; cb < ncb; ++cb) {
        for (int i = 0; i < DK; ++i) { sb += part(cb, 2, row, i); sg += part(cb, 3, row, i); }
        sb += p.part[(int64_t)ncb * 4 * NR * DK + (int64_t)cb * NR + row];
      }
      p.db[row] = sb;
      if (p.dg) p.dg[row] = sg;
    }
  }
}

template <int DK, bool CHANNEL, bool HAS_G, typename IO, typename GT>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.B * a.Hv), (unsigned)(a.dv / kCols));
  bwd_kernel<DK, CHANNEL, HAS_G, IO, GT><<<grid, DK * 4, 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_reduce_kernel<DK, CHANNEL><<<dim3((unsigned)(a.B * a.T)), 256, 0, stream>>>(a);
  return hipGetLastError();
}

template <int DK, typename IO, typename GT>
hipError_t launch_bwd_dk(const BwdArgs& a, hipStream_t stream) {
  const bool hg = a.g != nullptr;
  if (a.channel)
    return hg ? launch_bwd_t<DK, true, true, IO, GT>(a, stream)
              : launch_bwd_t<DK, true, false, IO, GT>(a, stream);
  return hg ? launch_bwd_t<DK, false, true, IO, GT>(a, stream)
            : launch_bwd_t<DK, false, false, IO, GT>(a, stream);
}

template <typename IO, typename GT>
hipError_t launch_bwd_types(const BwdArgs& a, hipStream_t stream) {
  return a.dk == 128 ? launch_bwd_dk<128, IO, GT>(a, stream) : launch_bwd_dk<64, IO, GT>(a, stream);
}

}  // namespace

int64_t bwd_checkpoint_blocks(int64_t T) { return (T + kCkpt - 1) / kCkpt; }

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
  if (a.io == DType::F32) return launch_bwd_types<float, float>(a, stream);
  if (a.gate == DType::F32) return launch_bwd_types<bf16, float>(a, stream);
  return launch_bwd_types<bf16, bf16>(a, stream);
}

}  // namespace gdn
