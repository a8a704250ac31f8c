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
// state every kCkpt tokens, the final state and every u_t in the workspace;
// it uses a layout of its own in which the read r needs no barrier.  Phase 2 walks the
// checkpoint blocks backwards: for each sub-block of kSub tokens it rebuilds
// the states from the block's checkpoint with the stored u (no reduction is
// needed: P_{t+1} = abar P_t + k u^T), keeps the sub-block's states in
// registers and runs the reverse step token by token.  Both phases read a
// block's token inputs from LDS, where they were staged while the previous
// block was computed (global loads issued a block ahead, LDS-only barriers in
// between so they stay in flight).  The per-row gradients (dq, dk, db, dg)
// are partial over the column block; they go to the workspace and a second
// kernel sums them over column blocks and over the value heads of a key head.
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

typedef float Tile[4][4];

// Barrier for LDS traffic only: waits for this wave's LDS operations, not
// for its global loads, so prefetches stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ void st4f(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void ld4f(const float* p, float* v) {
  const float4 x = *reinterpret_cast<const float4*>(p);
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}

// N consecutive elements of T kept as loaded (converted when stored to LDS,
// so that the load is not waited for where it is issued).
template <typename T, int N> struct RawN;
template <int N> struct RawN<bf16, N> { uint32_t w[N / 2]; };
template <int N> struct RawN<float, N> { float w[N]; };

template <typename T, int N>
__device__ __forceinline__ void load_raw(const T* p, RawN<T, N>& r) {
  if constexpr (sizeof(T) == 2) {
    if constexpr (N == 4) { const uint2 u = *reinterpret_cast<const uint2*>(p); r.w[0] = u.x; r.w[1] = u.y; }
    else { static_assert(N == 2, "N"); r.w[0] = *reinterpret_cast<const uint32_t*>(p); }
  } else {
    if constexpr (N == 4) { const float4 u = *reinterpret_cast<const float4*>(p); r.w[0] = u.x; r.w[1] = u.y; r.w[2] = u.z; r.w[3] = u.w; }
    else { static_assert(N == 2, "N"); const float2 u = *reinterpret_cast<const float2*>(p); r.w[0] = u.x; r.w[1] = u.y; }
  }
}
template <typename T, int N>
__device__ __forceinline__ void zero_raw(RawN<T, N>& r) {
#pragma unroll
  for (int i = 0; i < (sizeof(T) == 2 ? N / 2 : N); ++i) r.w[i] = 0;
}
template <typename T, int N>
__device__ __forceinline__ void unpack_raw(const RawN<T, N>& r, float* o) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if constexpr (sizeof(T) == 2) {
      const uint32_t w = r.w[i >> 1];
      o[i] = __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
      o[i] = r.w[i];
    }
  }
}

// One checkpoint block's token inputs in LDS: the row side (q, k, b, abar)
// over all DK rows and the column side (v, w, dO, u) over the workgroup's 64
// columns; scalar gates per token.
template <int DK>
struct Stage {
  float k[kCkpt][DK], q[kCkpt][DK], b[kCkpt][DK], a[kCkpt][DK];
  float v[kCkpt][kCols], w[kCkpt][kCols], dO[kCkpt][kCols], u[kCkpt][kCols];
  float sb[kCkpt], sa[kCkpt];
};

// A thread's share of loading one block into a Stage: 4 row elements of one
// token, CPT column elements of one token.
template <int DK, bool CHANNEL, bool HAS_G, bool REV, typename IO, typename GT>
struct BlockLoad {
  static constexpr int NT = DK * 4;
  static constexpr int TPR = DK / 4;                // threads per token (rows)
  static constexpr int CPT = kCkpt * kCols / NT;    // column elements per thread
  static constexpr int TPC = kCols / CPT;           // threads per token (columns)
  RawN<IO, 4> k, q;
  RawN<GT, 4> b, g;
  RawN<IO, CPT> v, dO;
  RawN<GT, CPT> w;
  float u[CPT];
  float sb, sg;
  bool rv, cv;   // the row / column token exists (loads past T read token T-1)

  // Every load is issued unconditionally (token index clamped into the
  // sequence), so the compiler's count of outstanding loads is the same on
  // every path and nothing waits for them before store().
  __device__ __forceinline__ void issue(const BwdArgs& p, int64_t tok0, int64_t Tn, int hv,
                                        int hk, int cb, int64_t t0, int tid) {
    const int tr = tid / TPR, i0 = 4 * (tid % TPR);
    const int tc = tid / TPC, j0 = CPT * (tid % TPC);
    const int64_t trr = t0 + tr, tcc = t0 + tc;
    rv = trr < Tn;
    cv = tcc < Tn;
    {
      const int64_t t = rv ? trr : Tn - 1;
      const int64_t bt = tok0 + t, bth = bt * p.Hv + hv;
      load_raw<IO, 4>(static_cast<const IO*>(p.k) + (bt * p.Hk + hk) * DK + i0, k);
      if constexpr (REV) load_raw<IO, 4>(static_cast<const IO*>(p.q) + (bt * p.Hk + hk) * DK + i0, q);
      if constexpr (CHANNEL) {
        load_raw<GT, 4>(static_cast<const GT*>(p.b) + bth * DK + i0, b);
        if constexpr (HAS_G) load_raw<GT, 4>(static_cast<const GT*>(p.g) + bth * DK + i0, g);
      } else {
        sb = to_f32(static_cast<const GT*>(p.b)[bth]);
        sg = HAS_G ? to_f32(static_cast<const GT*>(p.g)[bth]) : 0.f;
      }
    }
    {
      const int64_t t = cv ? tcc : Tn - 1;
      const int64_t bth = (tok0 + t) * p.Hv + hv;
      const int64_t off = bth * p.dv + (int64_t)cb * kCols + j0;
      load_raw<IO, CPT>(static_cast<const IO*>(p.v) + off, v);
      if constexpr (CHANNEL) load_raw<GT, CPT>(static_cast<const GT*>(p.w) + off, w);
      if constexpr (REV) {
        load_raw<IO, CPT>(static_cast<const IO*>(p.d_o) + off, dO);
#pragma unroll
        for (int j = 0; j < CPT; ++j) u[j] = p.u[off + j];
      }
    }
  }

  // Writes the block to LDS; tokens past T are stored as zeros.
  __device__ __forceinline__ void store(Stage<DK>& st, int tid) const {
    const int tr = tid / TPR, i0 = 4 * (tid % TPR);
    const int tc = tid / TPC, j0 = CPT * (tid % TPC);
    const float mr = rv ? 1.f : 0.f, mc = cv ? 1.f : 0.f;
    float x[4];
    unpack_raw<IO, 4>(k, x);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] *= mr;
    st4f(&st.k[tr][i0], x);
    if constexpr (REV) {
      unpack_raw<IO, 4>(q, x);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] *= mr;
      st4f(&st.q[tr][i0], x);
    }
    if constexpr (CHANNEL) {
      unpack_raw<GT, 4>(b, x);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] *= mr;
      st4f(&st.b[tr][i0], x);
      if constexpr (HAS_G) {
        unpack_raw<GT, 4>(g, x);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = exp2_fast(x[i] * kLog2e);
      } else {
        x[0] = x[1] = x[2] = x[3] = 1.f;
      }
      st4f(&st.a[tr][i0], x);
    } else if (i0 == 0) {
      st.sb[tr] = sb * mr;
      st.sa[tr] = HAS_G ? exp2_fast(sg * kLog2e) : 1.f;
    }
    float y[CPT];
    unpack_raw<IO, CPT>(v, y);
#pragma unroll
    for (int j = 0; j < CPT; ++j) st.v[tc][j0 + j] = y[j] * mc;
    if constexpr (CHANNEL) {
      unpack_raw<GT, CPT>(w, y);
#pragma unroll
      for (int j = 0; j < CPT; ++j) st.w[tc][j0 + j] = y[j] * mc;
    }
    if constexpr (REV) {
      unpack_raw<IO, CPT>(dO, y);
#pragma unroll
      for (int j = 0; j < CPT; ++j) { st.dO[tc][j0 + j] = y[j] * mc; st.u[tc][j0 + j] = u[j] * mc; }
    }
  }
};

// Token tl of a staged block, seen by one thread: its 4 rows and 4 columns.
template <int DK, bool CHANNEL>
__device__ __forceinline__ void rows_of(const Stage<DK>& st, int tl, int r0, float* k, float* e,
                                        float* bb, float* a) {
  ld4f(&st.k[tl][r0], k);
  if constexpr (CHANNEL) {
    ld4f(&st.b[tl][r0], bb);
    ld4f(&st.a[tl][r0], a);
  } else {
    const float sb = st.sb[tl], sa = st.sa[tl];
#pragma unroll
    for (int i = 0; i < 4; ++i) { bb[i] = sb; a[i] = sa; }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) e[i] = bb[i] * k[i];
}
template <int DK, bool CHANNEL>
__device__ __forceinline__ void wgate_of(const Stage<DK>& st, int tl, int cl, float* w) {
  if constexpr (CHANNEL) {
    ld4f(&st.w[tl][cl], w);
  } else {
    const float sb = st.sb[tl];
    w[0] = w[1] = w[2] = w[3] = sb;
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
  lds_barrier();
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
  __shared__ Stage<DK> stg[2];

  const int64_t head = blockIdx.x;          // b * Hv + hv
  const int cb = blockIdx.y;
  const int ncb = p.dv / kCols;
  const int64_t b = head / p.Hv;
  const int hv = (int)(head - b * p.Hv);
  const int hk = hv / (p.Hv / p.Hk);
  const int tid = threadIdx.x;
  const int rg = tid >> 4, cg = tid & 15;
  const int lane = tid & 63, wave = tid >> 6;
  const int r0 = 4 * rg, cl = 4 * cg;       // first row; first column inside the block
  const int64_t c0 = (int64_t)cb * kCols + cl;
  const int64_t NR = p.rows * p.Hv;         // gradient rows (token, hv)
  const float scale = p.scale;
  // This workgroup's sequence: tokens [tok0, tok0 + T) of the packed rows,
  // and its run of checkpoint slots (packed sequences: floor(tok0/16) + 2b,
  // which leaves room for the ceil(T/16) + 1 slots of every sequence).
  int64_t tok0 = b * p.T, T = p.T, slot0 = b * (p.nblk + 1);
  if (p.cu) {
    int64_t a0 = p.cu[b], a1 = p.cu[b + 1];
    a0 = a0 < 0 ? 0 : (a0 > p.rows ? p.rows : a0);
    a1 = a1 < a0 ? a0 : (a1 > p.rows ? p.rows : a1);
    tok0 = a0;
    T = a1 - a0;
    slot0 = a0 / kCkpt + 2 * b;
  }
  const int64_t nblk = (T + kCkpt - 1) / kCkpt;
  if (T == 0) {  // no token: the state gradient passes through
    if (p.d_state_in) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x[4] = {0.f, 0.f, 0.f, 0.f};
        if (p.d_state_out) ld4f(p.d_state_out + (head * DK + r0 + i) * p.dv + c0, x);
        st4f(p.d_state_in + (head * DK + r0 + i) * p.dv + c0, x);
      }
    }
    return;
  }
  int buf = 0;

  // nblk checkpoints (state before each 16-token block) + the final state
  float* ck = p.ckpt + (((int64_t)hv * ncb + cb) * p.slots + slot0) * (int64_t)DK * kCols;
  auto ck_at = [&](int64_t m, int i) { return ck + (m * DK + r0 + i) * kCols + cl; };

  // ---- phase 1: forward, storing checkpoints and u ----
  // Its own layout: a wave holds all DK rows of CW columns, a lane RPL rows
  // x CPL columns (the 16 lanes of a DPP row share the columns), so the read
  // r = Sbar^T e is an in-wave butterfly and the token loop has no barrier.
  {
    constexpr int RPL = DK / 16;             // rows per lane
    constexpr int CPL = 256 / DK;            // columns per lane
    constexpr int CW = 4 * CPL;              // columns per wave
    const int rl = lane & 15, dr = lane >> 4;
    const int pr0 = rl * RPL;                // first row
    const int pc0 = wave * CW + dr * CPL;    // first column inside the block
    const int64_t pcg = (int64_t)cb * kCols + pc0;
    auto ldn = [](const float* src, float* out, int n) {
      for (int i = 0; i < n; i += 4) ld4f(src + i, out + i);
    };
    auto ldc = [](const float* src, float* out) {
      if constexpr (CPL == 2) {
        const float2 x = *reinterpret_cast<const float2*>(src);
        out[0] = x.x; out[1] = x.y;
      } else {
        ld4f(src, out);
      }
    };
    auto stc = [](float* dst, const float* v) {
      if constexpr (CPL == 2) *reinterpret_cast<float2*>(dst) = make_float2(v[0], v[1]);
      else st4f(dst, v);
    };
    float P1[RPL][CPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      if (p.state_in) {
        ldc(p.state_in + (head * DK + pr0 + i) * p.dv + pcg, P1[i]);
      } else {
#pragma unroll
        for (int j = 0; j < CPL; ++j) P1[i][j] = 0.f;
      }
    }
    BlockLoad<DK, CHANNEL, HAS_G, false, IO, GT> ld;
    ld.issue(p, tok0, T, hv, hk, cb, 0, tid);
    ld.store(stg[0], tid);
    lds_barrier();
    for (int64_t m = 0; m < nblk; ++m) {
      const int cur = (int)(m & 1);
      const bool more = m + 1 < nblk;
      ld.issue(p, tok0, T, hv, hk, cb, (more ? m + 1 : m) * kCkpt, tid);
#pragma unroll
      for (int i = 0; i < RPL; ++i) stc(ck + (m * DK + pr0 + i) * kCols + pc0, P1[i]);
      const int64_t t0 = m * kCkpt;
      const int nt = (int)((T - t0) < kCkpt ? (T - t0) : kCkpt);
      const Stage<DK>& st = stg[cur];
      for (int tl = 0; tl < nt; ++tl) {
        float k[RPL], bb[RPL], a[RPL], w[CPL], v[CPL], r[CPL];
        ldn(&st.k[tl][pr0], k, RPL);
        if constexpr (CHANNEL) {
          ldn(&st.b[tl][pr0], bb, RPL);
          ldn(&st.a[tl][pr0], a, RPL);
          ldc(&st.w[tl][pc0], w);
        } else {
          const float sb = st.sb[tl], sa = st.sa[tl];
#pragma unroll
          for (int i = 0; i < RPL; ++i) { bb[i] = sb; a[i] = sa; }
#pragma unroll
          for (int j = 0; j < CPL; ++j) w[j] = sb;
        }
        ldc(&st.v[tl][pc0], v);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          float sacc = 0.f;
#pragma unroll
          for (int i = 0; i < RPL; ++i) sacc += a[i] * P1[i][j] * (bb[i] * k[i]);
          r[j] = row16_sum(sacc);
        }
        float u[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) u[j] = w[j] * v[j] - r[j];
        if (rl == 0) stc(p.u + ((tok0 + t0 + tl) * p.Hv + hv) * p.dv + pcg, u);
#pragma unroll
        for (int i = 0; i < RPL; ++i)
#pragma unroll
          for (int j = 0; j < CPL; ++j) P1[i][j] = a[i] * P1[i][j] + k[i] * u[j];
      }
      ld.store(stg[cur ^ 1], tid);   // (the last block stores a copy nobody reads)
      lds_barrier();
    }
    // the final state, read back below in the reverse layout
#pragma unroll
    for (int i = 0; i < RPL; ++i) stc(ck + (nblk * DK + pr0 + i) * kCols + pc0, P1[i]);
  }
  // The u and the final state written above are read back below through
  // global memory by other threads of this workgroup: make them visible.
  __threadfence_block();
  __syncthreads();

  // ---- phase 2: reverse ----
  Tile D, Pn;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ld4f(ck_at(nblk, i), Pn[i]);
    if (p.d_state_out) ld4f(p.d_state_out + (head * DK + r0 + i) * p.dv + c0, D[i]);
    else D[i][0] = D[i][1] = D[i][2] = D[i][3] = 0.f;
  }

  // P_{t+1} = abar P_t + k u^T with the staged u.
  auto advance = [&](const Stage<DK>& st, Tile& X, int tl) {
    float k[4], e[4], bb[4], a[4], u[4];
    rows_of<DK, CHANNEL>(st, tl, r0, k, e, bb, a);
    ld4f(&st.u[tl][cl], u);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) X[i][j] = a[i] * X[i][j] + k[i] * u[j];
  };

  // Reverse step of token t: Pb = P_t, Pa = P_{t+1}, D = dL/dP_{t+1} -> dL/dP_t.
  auto reverse = [&](const Stage<DK>& st, const Tile& Pb, const Tile& Pa, int tl, int64_t t) {
    const int64_t bth = (tok0 + t) * p.Hv + hv;
    float k[4], e[4], bb[4], a[4], w[4], v[4], dO[4], q[4], u[4];
    rows_of<DK, CHANNEL>(st, tl, r0, k, e, bb, a);
    wgate_of<DK, CHANNEL>(st, tl, cl, w);
    ld4f(&st.v[tl][cl], v);
    ld4f(&st.dO[tl][cl], dO);
    ld4f(&st.q[tl][r0], q);
    ld4f(&st.u[tl][cl], u);
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

  {
    BlockLoad<DK, CHANNEL, HAS_G, true, IO, GT> ld;
    ld.issue(p, tok0, T, hv, hk, cb, (nblk - 1) * kCkpt, tid);
    ld.store(stg[0], tid);
    Tile Ck, Cn;
#pragma unroll
    for (int i = 0; i < 4; ++i) ld4f(ck_at(nblk - 1, i), Ck[i]);
    // Wait here for everything loaded so far (D, Ck, the first block): the
    // block loop below then holds no value whose load is still pending on
    // entry, so the compiler need not drain the prefetches of each block
    // before its token loop.
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    for (int64_t mm = 0; mm < nblk; ++mm) {
      const int64_t m = nblk - 1 - mm;
      const int cur = (int)(mm & 1);
      const bool more = m > 0;
      const int64_t mp = more ? m - 1 : m;   // the next block (or this one again)
      ld.issue(p, tok0, T, hv, hk, cb, mp * kCkpt, tid);
#pragma unroll
      for (int i = 0; i < 4; ++i) ld4f(ck_at(mp, i), Cn[i]);
      const Stage<DK>& st = stg[cur];
      const int64_t t0 = m * kCkpt;
      const int nt = (int)((T - t0) < kCkpt ? (T - t0) : kCkpt);
      for (int s = kSubs - 1; s >= 0; --s) {
        const int ts = s * kSub;                // first token of the sub-block (local)
        if (ts >= nt) continue;
        const int n = (nt - ts) < kSub ? (nt - ts) : kSub;
        Tile R[kSub];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int c = 0; c < 4; ++c) R[0][i][c] = Ck[i][c];
        for (int tl = 0; tl < ts; ++tl) advance(st, R[0], tl);
#pragma unroll
        for (int j = 1; j < kSub; ++j) {
          if (j < n) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int c = 0; c < 4; ++c) R[j][i][c] = R[j - 1][i][c];
            advance(st, R[j], ts + j - 1);
          }
        }
#pragma unroll
        for (int j = kSub - 1; j >= 0; --j) {
          if (j < n) {
            reverse(st, R[j], Pn, ts + j, t0 + ts + j);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int c = 0; c < 4; ++c) Pn[i][c] = R[j][i][c];
          }
        }
      }
      ld.store(stg[cur ^ 1], tid);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) Ck[i][c] = Cn[i][c];
      lds_barrier();
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
  const int64_t NR = p.rows * p.Hv;
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
  bwd_reduce_kernel<DK, CHANNEL><<<dim3((unsigned)a.rows), 256, 0, stream>>>(a);
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
