// backward.hip -- gradients of the gated delta rule on gfx950 (reverse mode
// through the recurrence, in 16-token blocks on MFMA).
//
// With P_t the state before token t, abar = exp(g_t), e = b (.) k,
// z = w (.) v, the forward step is
//   Sbar = Diag(abar) P_t,  r = Sbar^T e,  u = z - r,
//   P_{t+1} = Sbar + k u^T,  o_t = scale P_{t+1}^T q_t.
// The pages give the forward update ("Gated DeltaNet-2", Methodologie §1)
// and name the gate-aware gradient as what makes training work (§3); the
// gradients below are the chain rule through that update, gathered over a
// block of C = 16 tokens so that they become matrix products.
//
// Block form.  For a block with entry state S, exit-state gradient D and,
// per channel i, the inclusive cumulative log-decay G_s (from the block
// start), write Gamma_st = exp(G_s - G_t) (s >= t; <= 1), gs = exp(G_s),
// ge = exp(G_end - G_s), gend = exp(G_end).  With
//   A[s][t] = sum_i e_s Gamma_st k_t (s > t),  Pm[s][t] = sum_i q_s Gamma_st k_t (s >= t),
//   RHS = (k ge) D + scale Pm^T dO,  DU = (I + A^T)^{-1} RHS   (du per token),
//   M3 = U dO^T,  M4 = U DU^T                                  (over columns),
// the gradients are
//   dq = scale (gs (.) dO S^T + [sum_{t<=s} M3[t][s] Gamma_st k_t])
//   de = -(gs (.) DU S^T + [sum_{t<s} M4[t][s] Gamma_st k_t])
//   dk = ge (.) U D^T + [sum_{s>=t} (scale M3[t][s] q_s - [s>t] M4[t][s] e_s) Gamma_st] + b (.) de
//   db = k (.) de,  dv = w (.) DU,  dw = v (.) DU,
//   dG_s = q dq + e de - k dk1 (+ rowsum(D (.) P_end) at the last token),
//   dg = reverse cumulative sum of dG over the block
//   (evaluated without the pairs of terms that cancel identically; see the
//   combine step),
//   D <- Diag(gend) D + scale (gs q)^T dO - (gs e)^T DU.
// The bracketed sums are intra-block.  They and A, Pm are products over the
// channel with a per-channel decay; they factor as exp(G_s - ref) exp(ref - G_t)
// around a per-channel reference and then run on the
// MFMA.  The reference is the midpoint of the channel's range of G over the
// block, which makes max |G_s - ref| half that range; a block whose range
// would still take the factors past the bound below computes them term by
// term on the vector units instead.  With scalar
// gates the decay is a 16 x 16 mask and the factors are 1.
//
// Layout: one workgroup per (sequence, value head, block of 64 value
// columns), DK * 4 threads; waves 0-3 are "column waves", one per 16-column
// tile.  Phase 1 runs the forward in the same 16-token blocks from the
// initial state -- U = (I + A)^{-1} (Z - (gs e) S), S' = Diag(gend) S +
// (ge k)^T U, the state tiles in the column waves' MFMA accumulators -- and
// stores the entry state of every block, the final state and every u_t in
// the workspace, in the operand type (phase 2 reads them as MFMA operands;
// only the row sum of D (.) S at the block end sees the rounded state).
// Phase 2 walks the blocks backwards with the exit-state
// gradient D held by every wave w as D^T tiles of rows 16w..16w+15 (bf16
// operands: also as a bf16 copy in LDS for the column waves' (k ge) D) and
// evaluates the block form above.  The per-row gradients (dq, dk, db, dg) are
// partial over the column block.  With channel gates, one value head per key
// head and at most two column blocks, each block adds its part straight into
// the outputs (cleared first): a sum of two addends is the same in either
// order, so the result stays deterministic.  Otherwise the parts go to the
// workspace and a second kernel sums them over column blocks and over the
// value heads of a key head.
// Only the first block walked in each phase can be short, so the others are
// compiled without per-token guards.
#include "chunk_common.hpp"

#include <type_traits>

namespace gdn {
namespace {

constexpr int kCkpt = 16;            // tokens per block (and between stored states)
constexpr int kCols = 64;            // value columns per workgroup
// Largest |G_s - ref| (log2 units) on the MFMA path.  The factored operands
// are at most 2^96 |k| (and 2^96 |q|, |e|), well inside fp32 and bf16.  An
// intra-block bracketed sum adds 16 terms M[t][s] Kf_t with |Kf_t| <= 2^96
// before the 2^(G_s - ref) factor brings it back, so it stays finite while
// |M| < 2^28: M3 and M4 are products of per-token vectors (U dO^T, U DU^T)
// and reach large values when a slowly decaying channel lets the state
// gradient D grow over a long sequence, so the bound is kept well below
// 2^127 / 16.  The masked-out entries of A and Pm (s < t) can overflow to
// inf; they are dropped with selects, never multiplied by zero.
constexpr float kSafeLog2 = 96.f;

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
__device__ __forceinline__ void ld4f(const bf16* p, float* v) {
  const uint2 x = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(x.x << 16); v[1] = __uint_as_float(x.x & 0xffff0000u);
  v[2] = __uint_as_float(x.y << 16); v[3] = __uint_as_float(x.y & 0xffff0000u);
}

// Adds one of exactly two addends into an fp32 output that starts at zero.
// Subnormal addends are flushed first, so that 0 + x is x exactly; the result
// is then the rounded sum of the two whichever lands first (and whatever the
// atomic unit does with subnormals), so it is bitwise deterministic.
__device__ __forceinline__ void add_pair(float* p, float x) {
  x = fabsf(x) < 1.17549435e-38f ? 0.f : x;
  unsafeAtomicAdd(p, x);
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

// ---------------------------------------------------------------------------
// Phase 1 (forward rebuild) in LDS: one block's row inputs, the gated
// operands of U = (I + A)^{-1} (Z - (gs e) S) and S' = Diag(gend) S +
// (ge k)^T U, and the cumulative decay.  Fragment layouts as in phase 2
// (below).
// ---------------------------------------------------------------------------
template <int DK, typename T>
struct FwdLds {
  static constexpr int RP = DK + 4;
  static constexpr int OP = DK + 16 / (int)sizeof(T);
  static constexpr int TP = 20;
  float k[kCkpt][RP], b[kCkpt][RP], gl[kCkpt][RP];   // inputs (fp32)
  T Kf[kCkpt][OP], Ef[kCkpt][OP], Egm[kCkpt][OP];    // k fk, e fq, -e gs  [token][channel]
  T KgT[DK][TP];                                     // k ge  [channel][token]
  float Gl[DK][TP];                                  // cumulative log2-decay
  float gend[DK];
  float A[kCkpt][kCkpt + 1];                         // exact channels' share of A
  float sb[kCkpt], sgl[kCkpt];
  uint32_t badm[DK / 32];                            // channels taken term by term
  int unsafe;                                        // some channel is
};

// A thread's share of one block's row inputs (4 channels of one token).
template <int DK, bool CHANNEL, bool HAS_G, typename IO, typename GT>
struct FwdLoad {
  static constexpr int TPR = DK / 4;
  RawN<IO, 4> k;
  RawN<GT, 4> b, g;
  float sb, sg;
  bool rv;

  __device__ __forceinline__ void issue(const BwdArgs& p, int64_t tok0, int64_t Tn, int hv,
                                        int hk, int64_t t0, int tid) {
    const int tr = tid / TPR, i0 = 4 * (tid % TPR);
    const int64_t trr = t0 + tr;
    rv = trr < Tn;
    const int64_t t = rv ? trr : Tn - 1;
    const int64_t bt = tok0 + t, bth = bt * p.Hv + hv;
    load_raw<IO, 4>(static_cast<const IO*>(p.k) + (bt * p.Hk + hk) * DK + i0, k);
    if constexpr (CHANNEL) {
      load_raw<GT, 4>(static_cast<const GT*>(p.b) + bth * DK + i0, b);
      if constexpr (HAS_G) load_raw<GT, 4>(static_cast<const GT*>(p.g) + bth * DK + i0, g);
    } else {
      sb = to_f32(static_cast<const GT*>(p.b)[bth]);
      sg = HAS_G ? to_f32(static_cast<const GT*>(p.g)[bth]) : 0.f;
    }
  }

  // Tokens past T are stored as zeros with zero log-decay.
  template <typename T>
  __device__ __forceinline__ void store(FwdLds<DK, T>& F, int tid) const {
    const int tr = tid / TPR, i0 = 4 * (tid % TPR);
    const float mr = rv ? 1.f : 0.f;
    float x[4];
    unpack_raw<IO, 4>(k, x);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] *= mr;
    st4f(&F.k[tr][i0], x);
    if constexpr (CHANNEL) {
      unpack_raw<GT, 4>(b, x);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] *= mr;
      st4f(&F.b[tr][i0], x);
      if constexpr (HAS_G) {
        unpack_raw<GT, 4>(g, x);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] *= kLog2e * mr;
      } else {
        x[0] = x[1] = x[2] = x[3] = 0.f;
      }
      st4f(&F.gl[tr][i0], x);
    } else if (i0 == 0) {
      F.sb[tr] = sb * mr;
      F.sgl[tr] = HAS_G ? sg * kLog2e * mr : 0.f;
    }
  }
};

// ---------------------------------------------------------------------------
// Phase 2: one block in LDS.  Fragment layouts (lane = 16 g + n): rowL(X)
// holds X[n][4g .. 4g+3], accL(X) holds X[4g .. 4g+3][n]; mma16(acc,
// rowL(X), accL(Y)) adds accL(X Y), and accL(X) = rowL(X^T).  Operands read
// with the channel as the contraction index are [token][channel] arrays;
// those read with the token as the contraction index are [channel][token]
// arrays (names ending in T).
// ---------------------------------------------------------------------------
template <int DK, typename T>
struct RevLds {
  static constexpr int RP = DK + 4;                    // fp32 [16][DK] pitch
  static constexpr int OP = DK + 16 / (int)sizeof(T);  // T [16][DK] pitch
  static constexpr int CPd = kCols + 16 / (int)sizeof(T);
  static constexpr int TP = 20;                        // [*][16] pitch
  float k[kCkpt][RP], q[kCkpt][RP], b[kCkpt][RP], gl[kCkpt][RP];  // inputs (fp32)
  T Kg[kCkpt][OP], Kf[kCkpt][OP], Qf[kCkpt][OP], Ef[kCkpt][OP];
  T KfT[DK][TP], QfT[DK][TP], EfT[DK][TP], QgT[DK][TP], EgT[DK][TP];
  T dOr[kCkpt][CPd], Ur[kCkpt][CPd], DUr[kCkpt][CPd];  // [token][column]
  T dOt[kCols][TP], DUt[kCols][TP];                     // [column][token]
  float Gl[DK][TP];                                     // cumulative log2-decay
  float ref[DK], lend[DK], gend[DK];
  float A[kCkpt][kCkpt + 1], P[kCkpt][kCkpt + 1];       // exact channels' share of A, Pm
  float M3[kCkpt][kCkpt + 1], M4[kCkpt][kCkpt + 1];
  float vs[4][kCkpt];                                   // scalar gates: sum_j v du per tile
  float sb[kCkpt], sgl[kCkpt];
  uint32_t badm[DK / 32];                               // channels taken term by term
  int unsafe;                                           // some channel is
  // bf16 operands: the exit-state gradient as D^T [column][row], the X1
  // operand of the column waves (fp32 operands keep D tiles in registers).
  static constexpr bool kDl = sizeof(T) == 2;
  T Dl[kDl ? kCols : 1][DK + 8];
};

// A thread's share of one block's row inputs (4 channels of one token) and
// column inputs (CPT columns of one token), issued a block ahead.
template <int DK, bool CHANNEL, bool HAS_G, typename IO, typename GT>
struct RevLoad {
  static constexpr int NT = DK * 4;
  static constexpr int TPR = DK / 4;
  static constexpr int CPT = kCkpt * kCols / NT;
  static constexpr int TPC = kCols / CPT;
  RawN<IO, 4> k, q;
  RawN<GT, 4> b, g;
  RawN<IO, CPT> dO, u;
  float sb, sg;
  bool rv, cv;

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
      load_raw<IO, 4>(static_cast<const IO*>(p.q) + (bt * p.Hk + hk) * DK + i0, q);
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
      const int64_t off = ((tok0 + t) * p.Hv + hv) * p.dv + (int64_t)cb * kCols + j0;
      load_raw<IO, CPT>(static_cast<const IO*>(p.d_o) + off, dO);
      load_raw<IO, CPT>(static_cast<const IO*>(p.u) + off, u);
    }
  }

  // Writes the block to LDS; tokens past T are stored as zeros, with zero
  // log-decay so that the cumulative decay stays put past the end.
  template <typename T>
  __device__ __forceinline__ void store(RevLds<DK, T>& L, int tid) const {
    const int tr = tid / TPR, i0 = 4 * (tid % TPR);
    const int tc = tid / TPC, j0 = CPT * (tid % TPC);
    const float mr = rv ? 1.f : 0.f, mc = cv ? 1.f : 0.f;
    float x[4];
    unpack_raw<IO, 4>(k, x);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] *= mr;
    st4f(&L.k[tr][i0], x);
    unpack_raw<IO, 4>(q, x);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] *= mr;
    st4f(&L.q[tr][i0], x);
    if constexpr (CHANNEL) {
      unpack_raw<GT, 4>(b, x);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] *= mr;
      st4f(&L.b[tr][i0], x);
      if constexpr (HAS_G) {
        unpack_raw<GT, 4>(g, x);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] *= kLog2e * mr;
      } else {
        x[0] = x[1] = x[2] = x[3] = 0.f;
      }
      st4f(&L.gl[tr][i0], x);
    } else if (i0 == 0) {
      L.sb[tr] = sb * mr;
      L.sgl[tr] = HAS_G ? sg * kLog2e * mr : 0.f;
    }
    float y[CPT], yu[CPT];
    unpack_raw<IO, CPT>(dO, y);
    unpack_raw<IO, CPT>(u, yu);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const T d = from_f32<T>(y[j] * mc);
      L.dOr[tc][j0 + j] = d;
      L.dOt[j0 + j][tc] = d;
      L.Ur[tc][j0 + j] = from_f32<T>(yu[j] * mc);
    }
  }
};

template <typename T>
__device__ __forceinline__ Frag4<T> frag4_of(const float* x) {
  Frag4<T> f;
#pragma unroll
  for (int i = 0; i < 4; ++i) f.v[i] = from_f32<T>(x[i]);
  return f;
}
__device__ __forceinline__ Frag4<float> f32frag(const f32x4& a) {
  Frag4<float> f;
#pragma unroll
  for (int i = 0; i < 4; ++i) f.v[i] = a[i];
  return f;
}

// 2^(Gl_s - Gl_t) for scalar gates (the per-token cumulative log2-decay is
// the same in every channel's row of Gl).
template <typename Lds>
__device__ __forceinline__ float token_decay(const Lds& L, int s, int t) {
  return exp2_fast(L.Gl[0][s] - L.Gl[0][t]);
}

// REV_ONLY: the checkpoints and u are in the workspace already (written by
// the chunk forward); only phase 2 runs.  Otherwise p.phases selects.
template <int DK, bool CHANNEL, bool HAS_G, typename IO, typename GT, bool REV_ONLY>
__global__ __launch_bounds__(DK * 4) void bwd_kernel(BwdArgs p) {
  constexpr int RB = DK / 16;               // 16-row blocks of the state
  using TO = IO;                            // MFMA operand type
  union Smem {
    FwdLds<DK, TO> fwd;
    RevLds<DK, TO> rev;
  };
  __shared__ Smem sm;
  lds_nan_fill(&sm, (int)sizeof(Smem));

  const int64_t head = blockIdx.x;          // b * Hv + hv
  const int cb = blockIdx.y;
  const int ncb = p.dv / kCols;
  const int64_t b = head / p.Hv;
  const int hv = (int)(head - b * p.Hv);
  const int hk = hv / (p.Hv / p.Hk);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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
      const int r0 = 4 * (tid >> 4), c0 = cb * kCols + 4 * (tid & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x[4] = {0.f, 0.f, 0.f, 0.f};
        if (p.d_state_out) ld4f(p.d_state_out + (head * DK + r0 + i) * p.dv + c0, x);
        st4f(p.d_state_in + (head * DK + r0 + i) * p.dv + c0, x);
      }
    }
    return;
  }

  // nblk checkpoints (state before each 16-token block) + the final state,
  // each stored [column][channel] (kCols rows of DK), in the operand type
  // (phase 2 uses them as MFMA operands and in one row sum)
  TO* ck = static_cast<TO*>(p.ckpt) + (((int64_t)hv * ncb + cb) * p.slots + slot0) * (int64_t)DK * kCols;

  const int g4 = lane >> 4, n = lane & 15;
  const bool colw = wave < 4;                // column waves own state tiles of columns 16 wave..
  const int ct = wave & 3;                   // a column wave's column tile
  const int64_t colg = (int64_t)cb * kCols;  // first value column of the workgroup
  // A column wave's v, w of its column tile (4 tokens per lane), a block ahead.
  IO vr[4];
  GT wr[4];
  auto issue_vw = [&](int64_t t0) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      int64_t t = t0 + 4 * g4 + ii;
      t = t < T ? t : T - 1;
      const int64_t off = ((tok0 + t) * p.Hv + hv) * p.dv + colg + 16 * ct + n;
      vr[ii] = static_cast<const IO*>(p.v)[off];
      if constexpr (CHANNEL) wr[ii] = static_cast<const GT*>(p.w)[off];
    }
  };

  // ---- phase 1: forward in blocks, storing checkpoints and u ----
  // Column wave ct holds the state's columns 16 ct.. over all rows as accL
  // tiles Sc[rb] (S[16rb + 4 g4 + ii][16 ct + n]) and per block solves
  // U = (I + A)^{-1} (Z - (gs e) S) and updates S' = Diag(gend) S + (ge k)^T U.
  // (Skipped when the forward kernel has stored the checkpoints and u.)
  if (!REV_ONLY && (p.phases & 1)) {
    FwdLds<DK, TO>& F = sm.fwd;
    f32x4 Sc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
        Sc[rb][ii] = (colw && p.state_in)
                         ? p.state_in[(head * DK + 16 * rb + 4 * g4 + ii) * p.dv + colg + 16 * ct + n]
                         : 0.f;
    FwdLoad<DK, CHANNEL, HAS_G, IO, GT> ld;
    ld.issue(p, tok0, T, hv, hk, 0, tid);
    issue_vw(0);
    __builtin_amdgcn_s_waitcnt(0);
    // One block of the forward walk (FULL: all 16 tokens; only the last can be short).
    auto fwd_block = [&](auto full_tag, int64_t m) __attribute__((always_inline)) {
      constexpr bool FULL = decltype(full_tag)::value;
      const int64_t t0 = m * kCkpt;
      const int nt = FULL ? kCkpt : (int)((T - t0) < kCkpt ? (T - t0) : kCkpt);
      const int64_t mn = m + 1 < nblk ? m + 1 : m;   // the next block (or this one again)
      ld.store(F, tid);
      if (tid < DK / 32) F.badm[tid] = 0u;
      if (tid == 0) F.unsafe = 0;
      float vv[4], wv[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        vv[ii] = to_f32(vr[ii]);
        wv[ii] = CHANNEL ? to_f32(wr[ii]) : 0.f;
      }
      lds_barrier();
      ld.issue(p, tok0, T, hv, hk, mn * kCkpt, tid);
      if (colw) issue_vw(mn * kCkpt);
      {
        const int i = tid % DK, qt = tid / DK;
        float acc = 0.f, gmax = -INFINITY, gmin = INFINITY, G[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < kCkpt; ++r) {
          acc += CHANNEL ? F.gl[r][i] : F.sgl[r];
          gmax = fmaxf(gmax, acc);
          gmin = fminf(gmin, acc);
          if ((r >> 2) == qt) G[r & 3] = acc;
        }
        const float ref = 0.5f * (gmax + gmin);   // midpoint of the block's range
        const float lend = acc;
        if (qt == 0) F.gend[i] = exp2_fast(lend);
        st4f(&F.Gl[i][4 * qt], G);
        // a channel whose range takes the factors past the bound leaves the
        // factored products (zero operands) and is added term by term
        const bool bad = CHANNEL && 0.5f * (gmax - gmin) > kSafeLog2;
        float kg[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int s = 4 * qt + ii;
          const float kk = F.k[s][i];
          const float e = (CHANNEL ? F.b[s][i] : F.sb[s]) * kk;
          const float fq = CHANNEL ? exp2_fast(G[ii] - ref) : 1.f;
          const float fk = CHANNEL ? exp2_fast(ref - G[ii]) : 1.f;
          kg[ii] = kk * exp2_fast(lend - G[ii]);
          F.Kf[s][i] = from_f32<TO>(bad ? 0.f : kk * fk);
          F.Ef[s][i] = from_f32<TO>(bad ? 0.f : e * fq);
          F.Egm[s][i] = from_f32<TO>(-e * exp2_fast(G[ii]));
        }
        st4<TO>(&F.KgT[i][4 * qt], kg[0], kg[1], kg[2], kg[3]);
        if (bad && qt == 0) {
          atomicOr(&F.badm[i >> 5], 1u << (i & 31));
          F.unsafe = 1;
        }
      }
      lds_barrier();
      const bool exact = CHANNEL && F.unsafe != 0;   // uniform over the workgroup
      if (exact) {
        // the term-by-term channels' share of A[s][t] = sum_i e_s k_t 2^(Gl_s - Gl_t)
        if (tid < kCkpt * kCkpt) {
          const int s = tid >> 4, t = tid & 15;
          float sa = 0.f;
          if (s > t) {
#pragma unroll 1
            for (int w = 0; w < DK / 32; ++w)
              for (uint32_t m = F.badm[w]; m != 0u; m &= m - 1u) {
                const int i = 32 * w + __builtin_ctz(m);
                sa += F.b[s][i] * F.k[s][i] * F.k[t][i] * exp2_fast(F.Gl[i][s] - F.Gl[i][t]);
              }
          }
          F.A[s][t] = sa;
        }
        lds_barrier();
      }
      if (colw) {
        // the block's entry state
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          st4<TO>(ck + (m * kCols + 16 * ct + n) * DK + 16 * rb + 4 * g4, Sc[rb][0], Sc[rb][1],
                  Sc[rb][2], Sc[rb][3]);
        Frag4<float> nr, nc;   // rowL(N), accL(N), N = -A
        {
          f32x4 aA = {0.f, 0.f, 0.f, 0.f}, aAt = aA;
#pragma unroll
          for (int kb = 0; kb < RB; ++kb) {
            const Frag4<TO> ef = ld_frag4<TO>(&F.Ef[n][16 * kb + 4 * g4]);
            const Frag4<TO> kf = ld_frag4<TO>(&F.Kf[n][16 * kb + 4 * g4]);
            mma16(aA, ef, kf);    // A[4g+ii][n]
            mma16(aAt, kf, ef);   // A[n][4g+ii]
          }
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int r = 4 * g4 + ii;
            float grn = 1.f, gnr = 1.f;
            if constexpr (!CHANNEL) {
              grn = r >= n ? token_decay(F, r, n) : 0.f;
              gnr = n >= r ? token_decay(F, n, r) : 0.f;
            }
            float xc = aA[ii] * grn, xr = aAt[ii] * gnr;
            if (exact) {
              xc += F.A[r][n];
              xr += F.A[n][r];
            }
            nc.v[ii] = n < r ? -xc : 0.f;
            nr.v[ii] = r < n ? -xr : 0.f;
          }
        }
        // rowL((I + A)^{-1}) = accL(T^T), T = (I + N)(I + N^2)(I + N^4)(I + N^8):
        // bf16 operands take the fp16 products while |N| allows them (one
        // MFMA per product), otherwise (and for fp32 operands) the fp32 chain
        f32x4 trow;
        bool have_t = false;
        if constexpr (!std::is_same<TO, float>::value) {
          float nmax;
          const Frag4<float> tt = unit_lower_inverse(nr, nc, g4, n, nmax);
          if (!__any(!(nmax <= kNBig))) {   // uniform over the wave
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) trow[ii] = tt.v[ii];
            have_t = true;
          }
        }
        if (!have_t) {
          auto prod = [](const Frag4<float>& x, const Frag4<float>& y) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
            mma16(a, x, y);
            return f32frag(a);
          };
          const Frag4<float> n2c = prod(nr, nc), n2r = prod(nc, nr);
          const Frag4<float> n4c = prod(n2r, n2c), n4r = prod(n2c, n2r);
          const Frag4<float> n8r = prod(n4c, n4r);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) trow[ii] = n8r.v[ii] + (4 * g4 + ii == n ? 1.f : 0.f);
          mma16(trow, n4c, f32frag(trow));
          mma16(trow, n2c, f32frag(trow));
          mma16(trow, nc, f32frag(trow));
        }
        // W = Z - (gs e) S, U = T W
        f32x4 wt;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int s = 4 * g4 + ii;
          wt[ii] = s < nt ? (CHANNEL ? wv[ii] : F.sb[s]) * vv[ii] : 0.f;
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          mma16(wt, ld_frag4<TO>(&F.Egm[n][16 * rb + 4 * g4]), frag4_from_acc<TO>(Sc[rb]));
        f32x4 ut = {0.f, 0.f, 0.f, 0.f};
        mma16(ut, f32frag(trow), f32frag(wt));
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int s = 4 * g4 + ii;
          if (s < nt)
            static_cast<TO*>(p.u)[((tok0 + t0 + s) * p.Hv + hv) * p.dv + colg + 16 * ct + n] =
                from_f32<TO>(ut[ii]);
        }
        const Frag4<TO> uf = frag4_from_acc<TO>(ut);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const float4 ge4 = *reinterpret_cast<const float4*>(&F.gend[16 * rb + 4 * g4]);
          Sc[rb][0] *= ge4.x; Sc[rb][1] *= ge4.y; Sc[rb][2] *= ge4.z; Sc[rb][3] *= ge4.w;
          mma16(Sc[rb], ld_frag4<TO>(&F.KgT[16 * rb + n][4 * g4]), uf);
        }
      }
      lds_barrier();   // the block's LDS is rewritten by the next one
    };
    for (int64_t m = 0; m + 1 < nblk; ++m) fwd_block(std::true_type{}, m);
    fwd_block(std::false_type{}, nblk - 1);
    // the final state
    if (colw) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        st4<TO>(ck + (nblk * kCols + 16 * ct + n) * DK + 16 * rb + 4 * g4, Sc[rb][0], Sc[rb][1],
                Sc[rb][2], Sc[rb][3]);
    }
  }
  if (!REV_ONLY && !(p.phases & 2)) return;
  // The u and the states written above are read back below through global
  // memory by other threads of this workgroup: make them visible.
  __threadfence_block();
  __syncthreads();

  // ---- phase 2: reverse, one block at a time in matrix form ----
  RevLds<DK, TO>& L = sm.rev;
  const int ch = 16 * wave + n;              // this lane's channel in the row-gradient tiles

  // Dt[c]: accL(D^T) tile (columns 16c.., rows 16 wave..): D[ch][16c + 4 g4 + ii].
  // Dc[rb]: accL(D) tile (rows 16rb.., columns 16 ct..): D[16rb + 4 g4 + ii][16 ct + n]
  // (fp32 operands; with bf16 operands the column waves read D from LDS).
  constexpr bool DL = RevLds<DK, TO>::kDl;
  f32x4 Dt[4], Dc[DL ? 1 : RB];
  float Sf[4][4];                            // S[ch][16c + 4 g4 + ii]: the block's entry state
  auto ld_ck = [&](int64_t blk, int c, float* x) {
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) x[ii] = to_f32(ck[(blk * kCols + 16 * c + 4 * g4 + ii) * DK + ch]);
  };
  {
    const float* dso = p.d_state_out ? p.d_state_out + head * (int64_t)DK * p.dv + colg : nullptr;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float x[4] = {0.f, 0.f, 0.f, 0.f};
      if (dso) ld4f(dso + (int64_t)ch * p.dv + 16 * c + 4 * g4, x);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) Dt[c][ii] = x[ii];
      ld_ck(nblk - 1, c, Sf[c]);
    }
    if constexpr (!DL) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          Dc[rb][ii] = (dso && colw) ? dso[(int64_t)(16 * rb + 4 * g4 + ii) * p.dv + 16 * ct + n] : 0.f;
    }
  }
  auto put_dl = [&]() {   // D^T into LDS for the next block's X1 (bf16 operands)
    if constexpr (DL) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) L.Dl[16 * c + 4 * g4 + ii][ch] = from_f32<TO>(Dt[c][ii]);
    }
  };
  put_dl();
  RevLoad<DK, CHANNEL, HAS_G, IO, GT> ld;
  ld.issue(p, tok0, T, hv, hk, cb, (nblk - 1) * kCkpt, tid);
  issue_vw((nblk - 1) * kCkpt);
  // Wait here for everything loaded so far: the block loop then holds no
  // value whose load is still pending on entry, so the compiler need not
  // drain each block's prefetches at its top.
  __builtin_amdgcn_s_waitcnt(0);

  // One block of the reverse walk; FULL blocks have all 16 tokens, so none
  // of their stores is conditional (only the first block walked can be short).
  auto rev_block = [&](auto full_tag, int64_t mm) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
    const int64_t m = nblk - 1 - mm;
    const int64_t t0 = m * kCkpt;
    const int nt = FULL ? kCkpt : (int)((T - t0) < kCkpt ? (T - t0) : kCkpt);
    const int64_t mp = m > 0 ? m - 1 : 0;    // the next block (or this one again)

    // rowsum(D (.) S) of the incoming D with the entry state
    float dps = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) dps += Dt[c][ii] * Sf[c][ii];
    dps += __shfl_xor(dps, 16);
    dps += __shfl_xor(dps, 32);

    ld.store(L, tid);
    if (tid < DK / 32) L.badm[tid] = 0u;
    if (tid == 0) L.unsafe = 0;
    float vv[4], wv[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      vv[ii] = to_f32(vr[ii]);
      wv[ii] = CHANNEL ? to_f32(wr[ii]) : 0.f;
    }
    lds_barrier();
    ld.issue(p, tok0, T, hv, hk, cb, mp * kCkpt, tid);
    if (colw) issue_vw(mp * kCkpt);

    // ---- cumulative decay, factors and gated operands (thread: channel i, tokens 4 qt..) ----
    {
      const int i = tid % DK, qt = tid / DK;
      float acc = 0.f, gmax = -INFINITY, gmin = INFINITY, G[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < kCkpt; ++r) {
        acc += CHANNEL ? L.gl[r][i] : L.sgl[r];
        gmax = fmaxf(gmax, acc);
        gmin = fminf(gmin, acc);
        if ((r >> 2) == qt) G[r & 3] = acc;
      }
      const float ref = 0.5f * (gmax + gmin);   // midpoint of the block's range
      const float lend = acc;
      if (qt == 0) {
        L.ref[i] = ref;
        L.lend[i] = lend;
        L.gend[i] = exp2_fast(lend);
      }
      st4f(&L.Gl[i][4 * qt], G);
      // as in the forward walk: a channel out of range has zero factored
      // operands and is added term by term
      const bool bad = CHANNEL && 0.5f * (gmax - gmin) > kSafeLog2;
      float kf[4], qf[4], ef[4], qg[4], eg[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int s = 4 * qt + ii;
        const float kk = L.k[s][i], qq = L.q[s][i];
        const float e = (CHANNEL ? L.b[s][i] : L.sb[s]) * kk;
        const float gs = exp2_fast(G[ii]), ge = exp2_fast(lend - G[ii]);
        const float fq = CHANNEL ? exp2_fast(G[ii] - ref) : 1.f;
        const float fk = CHANNEL ? exp2_fast(ref - G[ii]) : 1.f;
        kf[ii] = bad ? 0.f : kk * fk;
        qf[ii] = bad ? 0.f : qq * fq;
        ef[ii] = bad ? 0.f : e * fq;
        qg[ii] = scale * qq * gs;
        eg[ii] = -e * gs;
        L.Kg[s][i] = from_f32<TO>(kk * ge);
        L.Kf[s][i] = from_f32<TO>(kf[ii]);
        L.Qf[s][i] = from_f32<TO>(qf[ii]);
        L.Ef[s][i] = from_f32<TO>(ef[ii]);
      }
      st4<TO>(&L.KfT[i][4 * qt], kf[0], kf[1], kf[2], kf[3]);
      st4<TO>(&L.QfT[i][4 * qt], qf[0], qf[1], qf[2], qf[3]);
      st4<TO>(&L.EfT[i][4 * qt], ef[0], ef[1], ef[2], ef[3]);
      st4<TO>(&L.QgT[i][4 * qt], qg[0], qg[1], qg[2], qg[3]);
      st4<TO>(&L.EgT[i][4 * qt], eg[0], eg[1], eg[2], eg[3]);
      if (bad && qt == 0) {
        atomicOr(&L.badm[i >> 5], 1u << (i & 31));
        L.unsafe = 1;
      }
    }
    lds_barrier();
    const bool exact = CHANNEL && L.unsafe != 0;   // uniform over the workgroup

    if (exact) {
      // the term-by-term channels' share of A[s][t] = sum_i e_s k_t 2^(Gl_s - Gl_t)
      // and of Pm (q_s in place of e_s)
      if (tid < kCkpt * kCkpt) {
        const int s = tid >> 4, t = tid & 15;
        float sa = 0.f, sp = 0.f;
        if (s >= t) {
#pragma unroll 1
          for (int w = 0; w < DK / 32; ++w)
            for (uint32_t m = L.badm[w]; m != 0u; m &= m - 1u) {
              const int i = 32 * w + __builtin_ctz(m);
              const float kt = L.k[t][i] * exp2_fast(L.Gl[i][s] - L.Gl[i][t]);
              sa += L.b[s][i] * L.k[s][i] * kt;
              sp += L.q[s][i] * kt;
            }
        }
        L.A[s][t] = s > t ? sa : 0.f;
        L.P[s][t] = s >= t ? sp : 0.f;
      }
      lds_barrier();
    }

    // ---- column waves: DU tile = (I + A^T)^{-1} RHS, dv, dw, D tiles ----
    f32x4 du = {0.f, 0.f, 0.f, 0.f};
    if (colw) {
      Frag4<float> nr, nc;   // rowL(N), accL(N), N = -A
      Frag4<TO> pT;          // rowL(scale Pm^T) = scale accL(Pm)
      {
        f32x4 aA = {0.f, 0.f, 0.f, 0.f}, aAt = aA, aP = aA;
#pragma unroll
        for (int kb = 0; kb < RB; ++kb) {
          const Frag4<TO> ef = ld_frag4<TO>(&L.Ef[n][16 * kb + 4 * g4]);
          const Frag4<TO> kf = ld_frag4<TO>(&L.Kf[n][16 * kb + 4 * g4]);
          const Frag4<TO> qf = ld_frag4<TO>(&L.Qf[n][16 * kb + 4 * g4]);
          mma16(aA, ef, kf);    // A[4g+ii][n]
          mma16(aAt, kf, ef);   // A[n][4g+ii]
          mma16(aP, qf, kf);    // Pm[4g+ii][n]
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int r = 4 * g4 + ii;
          float grn = 1.f, gnr = 1.f;
          if constexpr (!CHANNEL) {
            grn = r >= n ? token_decay(L, r, n) : 0.f;
            gnr = n >= r ? token_decay(L, n, r) : 0.f;
          }
          float xc = aA[ii] * grn, xr = aAt[ii] * gnr, xp = aP[ii] * grn;
          if (exact) {
            xc += L.A[r][n];
            xr += L.A[n][r];
            xp += L.P[r][n];
          }
          nc.v[ii] = n < r ? -xc : 0.f;
          nr.v[ii] = r < n ? -xr : 0.f;
          pT.v[ii] = from_f32<TO>(r >= n ? scale * xp : 0.f);
        }
      }
      // (I + A)^{-1} = (I + N)(I + N^2)(I + N^4)(I + N^8) (N^16 = 0), as accL.
      // accL(T) = rowL(T^T), and T^T is the same product of N^T, so bf16
      // operands take the fp16 products on (accL(N), rowL(N)) while |N|
      // allows them; otherwise (and for fp32 operands) the fp32 chain.
      f32x4 tinv;
      bool have_t = false;
      if constexpr (!std::is_same<TO, float>::value) {
        float nmax;
        const Frag4<float> tt = unit_lower_inverse(nc, nr, g4, n, nmax);
        if (!__any(!(nmax <= kNBig))) {   // uniform over the wave
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) tinv[ii] = tt.v[ii];
          have_t = true;
        }
      }
      if (!have_t) {
        auto prod = [](const Frag4<float>& x, const Frag4<float>& y) {
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
          mma16(a, x, y);
          return f32frag(a);
        };
        const Frag4<float> n2c = prod(nr, nc), n2r = prod(nc, nr);
        const Frag4<float> n4c = prod(n2r, n2c), n4r = prod(n2c, n2r);
        const Frag4<float> n8c = prod(n4r, n4c);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) tinv[ii] = n8c.v[ii] + (4 * g4 + ii == n ? 1.f : 0.f);
        mma16(tinv, n4r, f32frag(tinv));
        mma16(tinv, n2r, f32frag(tinv));
        mma16(tinv, nr, f32frag(tinv));
      }
      // RHS = (k ge) D + scale Pm^T dO for this column tile
      f32x4 rhs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        Frag4<TO> dfr;
        if constexpr (DL) dfr = ld_frag4<TO>(&L.Dl[16 * ct + n][16 * rb + 4 * g4]);
        else dfr = frag4_from_acc<TO>(Dc[rb]);
        mma16(rhs, ld_frag4<TO>(&L.Kg[n][16 * rb + 4 * g4]), dfr);
      }
      const Frag4<TO> dot = ld_frag4<TO>(&L.dOt[16 * ct + n][4 * g4]);   // accL(dO tile)
      mma16(rhs, pT, dot);
      mma16(du, f32frag(tinv), f32frag(rhs));   // DU = Tinv^T RHS
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) L.DUr[4 * g4 + ii][16 * ct + n] = from_f32<TO>(du[ii]);
      st4<TO>(&L.DUt[16 * ct + n][4 * g4], du[0], du[1], du[2], du[3]);
      if constexpr (!CHANNEL) {   // sum_j v du of the tile goes to dbeta
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float x = row16_sum(vv[ii] * du[ii]);
          if (n == 0) L.vs[ct][4 * g4 + ii] = x;
        }
      }
    }

    // ---- every wave: row-gradient tiles of channels 16 wave .. (tokens 4 g4 + ii) ----
    Frag4<TO> sfr[4], ua[4], doa[4];
    f32x4 dQi = {0.f, 0.f, 0.f, 0.f}, dKi = dQi, m3 = dQi, m3t = dQi, dQa = dQi, dKa = dQi;
#pragma unroll
    for (int c = 0; c < 4; ++c) sfr[c] = frag4_of<TO>(Sf[c]);   // accL(S^T) tile
#pragma unroll
    for (int c = 0; c < 4; ++c)   // the next block's entry state
      ld_ck(mp, c, Sf[c]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ua[c] = ld_frag4<TO>(&L.Ur[n][16 * c + 4 * g4]);     // rowL(U)
      doa[c] = ld_frag4<TO>(&L.dOr[n][16 * c + 4 * g4]);   // rowL(dO)
      mma16(dQi, doa[c], sfr[c]);                          // dO S^T
      mma16(dKi, ua[c], frag4_from_acc<TO>(Dt[c]));        // U D^T
      mma16(m3, ua[c], doa[c]);                            // M3[4g+ii][n]
      mma16(m3t, doa[c], ua[c]);                           // M3[n][4g+ii]
    }
    // M3[s][s] for this lane's tokens (the diagonal pairs are added apart)
    float d3[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) d3[ii] = __shfl(m3[ii], 20 * g4 + ii);
    const Frag4<TO> kfb = ld_frag4<TO>(&L.KfT[ch][4 * g4]);   // accL(Kf) tile
    const Frag4<TO> qfb = ld_frag4<TO>(&L.QfT[ch][4 * g4]);
    const Frag4<TO> efb = ld_frag4<TO>(&L.EfT[ch][4 * g4]);
    {
      Frag4<TO> a1, a2;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = 4 * g4 + ii;
        float gnr = 1.f, grn = 1.f;
        if constexpr (!CHANNEL) {
          gnr = n >= r ? token_decay(L, n, r) : 0.f;
          grn = r >= n ? token_decay(L, r, n) : 0.f;
        }
        a1.v[ii] = from_f32<TO>(r < n ? m3[ii] * gnr : 0.f);            // X[s=n][t=r]
        a2.v[ii] = from_f32<TO>(r > n ? scale * m3t[ii] * grn : 0.f);   // Y[t=n][s=r]
      }
      mma16(dQa, a1, kfb);
      mma16(dKa, a2, qfb);
    }
    if (exact && wave == 0) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) L.M3[4 * g4 + ii][n] = m3[ii];
    }
    lds_barrier();   // DU tiles (and M3 for the term-by-term channels) visible

    if (colw) {
      // dv = w du, dw = v du (scalar gates: w = beta)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int s = 4 * g4 + ii;
        const float wgt = CHANNEL ? wv[ii] : L.sb[s];
        if (s < nt) {
          const int64_t o = ((tok0 + t0 + s) * p.Hv + hv) * p.dv + colg + 16 * ct + n;
          p.dv_out[o] = wgt * du[ii];
          if constexpr (CHANNEL) p.dw[o] = vv[ii] * du[ii];
        }
      }
      if constexpr (!DL) {
        // D tiles: D <- Diag(gend) D + (scale gs q)^T dO - (gs e)^T DU
        const Frag4<TO> dot = ld_frag4<TO>(&L.dOt[16 * ct + n][4 * g4]);
        const Frag4<TO> duf = ld_frag4<TO>(&L.DUt[16 * ct + n][4 * g4]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const float4 ge4 = *reinterpret_cast<const float4*>(&L.gend[16 * rb + 4 * g4]);
          Dc[rb][0] *= ge4.x; Dc[rb][1] *= ge4.y; Dc[rb][2] *= ge4.z; Dc[rb][3] *= ge4.w;
          mma16(Dc[rb], ld_frag4<TO>(&L.QgT[16 * rb + n][4 * g4]), dot);
          mma16(Dc[rb], ld_frag4<TO>(&L.EgT[16 * rb + n][4 * g4]), duf);
        }
      }
    }

    f32x4 dEi = {0.f, 0.f, 0.f, 0.f}, m4 = dEi, m4t = dEi, dEa = dEi;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const Frag4<TO> dua = ld_frag4<TO>(&L.DUr[n][16 * c + 4 * g4]);
      mma16(dEi, dua, sfr[c]);     // DU S^T
      mma16(m4, ua[c], dua);       // M4[4g+ii][n]
      mma16(m4t, dua, ua[c]);      // M4[n][4g+ii]
    }
    {
      Frag4<TO> a3, a4;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int r = 4 * g4 + ii;
        float gnr = 1.f, grn = 1.f;
        if constexpr (!CHANNEL) {
          gnr = n >= r ? token_decay(L, n, r) : 0.f;
          grn = r >= n ? token_decay(L, r, n) : 0.f;
        }
        a3.v[ii] = from_f32<TO>(r < n ? m4[ii] * gnr : 0.f);     // X[s=n][t=r]
        a4.v[ii] = from_f32<TO>(r > n ? -m4t[ii] * grn : 0.f);   // Y[t=n][s=r]
      }
      mma16(dEa, a3, kfb);
      mma16(dKa, a4, efb);
    }
    // D^T tiles: D^T <- D^T Diag(gend) + dO^T (scale gs q) - DU^T (gs e)
    {
      const Frag4<TO> qgb = ld_frag4<TO>(&L.QgT[ch][4 * g4]);
      const Frag4<TO> egb = ld_frag4<TO>(&L.EgT[ch][4 * g4]);
      const float gi = L.gend[ch];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) Dt[c][ii] *= gi;
        mma16(Dt[c], ld_frag4<TO>(&L.dOt[16 * c + n][4 * g4]), qgb);
        mma16(Dt[c], ld_frag4<TO>(&L.DUt[16 * c + n][4 * g4]), egb);
      }
      put_dl();   // read by the next block's column waves, after the end barrier
    }
    // this lane's channel is taken term by term (its factored operands were
    // zero, so the products above left nothing for it)
    const bool bad_ch = exact && ((L.badm[ch >> 5] >> (ch & 31)) & 1u);
    if (exact) {
      if (wave == 0) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) L.M4[4 * g4 + ii][n] = m4[ii];
      }
      lds_barrier();
      // Intra-block terms of this wave's term-by-term channels, one channel
      // at a time by the whole wave: lane 4 s + j takes token s against the
      // partners t = 4 j .. 4 j + 3, with 2^(Gl_s - Gl_t) for s > t; the
      // lane quad sums them and the channel's own lanes pick up their tokens.
      const int sl = lane >> 2, jq = lane & 3;
      const uint32_t wm = (L.badm[(16 * wave) >> 5] >> ((16 * wave) & 31)) & 0xffffu;
#pragma unroll 1
      for (uint32_t m = wm; m != 0u; m &= m - 1u) {   // uniform over the wave
        const int c = 16 * wave + __builtin_ctz(m);
        const float Gs = L.Gl[c][sl];
        float aq = 0.f, ae = 0.f, ak = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int t2 = 4 * jq + u;
          const float Gt = L.Gl[c][t2];
          if (t2 < sl) {
            const float kg = L.k[t2][c] * exp2_fast(Gs - Gt);
            aq += L.M3[t2][sl] * kg;
            ae += L.M4[t2][sl] * kg;
          }
          if (t2 > sl) {
            const float x = scale * L.M3[sl][t2] * L.q[t2][c] -
                            L.M4[sl][t2] * L.b[t2][c] * L.k[t2][c];
            ak += x * exp2_fast(Gt - Gs);
          }
        }
        aq += __shfl_xor(aq, 1);
        ae += __shfl_xor(ae, 1);
        ak += __shfl_xor(ak, 1);
        aq += __shfl_xor(aq, 2);
        ae += __shfl_xor(ae, 2);
        ak += __shfl_xor(ak, 2);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int src = 4 * (4 * g4 + ii);
          const float vq = __shfl(aq, src), ve = __shfl(ae, src), vk = __shfl(ak, src);
          if (ch == c) {
            dQa[ii] = vq;
            dEa[ii] = ve;
            dKa[ii] = vk;
          }
        }
      }
    }

    // ---- combine and write the partial row gradients ----
    {
      const float4 G4 = *reinterpret_cast<const float4*>(&L.Gl[ch][4 * g4]);
      const float Gv[4] = {G4.x, G4.y, G4.z, G4.w};
      const float ref = L.ref[ch], lend = L.lend[ch];
      const bool fac = CHANNEL && !bad_ch;
      const int send = nt - 1;   // the block's last token
      // dG: every pair of terms that share a decay factor contributes once
      // at each end, so the pairs whose factor is identically 1 -- the
      // diagonal (s, s) and the last token's own share of the exit state --
      // are left out of both ends; with them in, dG would be a difference
      // of O(1) terms where the true value underflows.
      float dq[4], dk[4], db[4], dG[4], pend = 0.f;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int s = 4 * g4 + ii;
        const float G = Gv[ii];
        const float gs = exp2_fast(G), ge = exp2_fast(lend - G);
        const float fq = fac ? exp2_fast(G - ref) : 1.f;
        const float fk = fac ? exp2_fast(ref - G) : 1.f;
        const float kk = L.k[s][ch], qq = L.q[s][ch];
        const float bb = CHANNEL ? L.b[s][ch] : L.sb[s];
        const float dQo = scale * (gs * dQi[ii] + fq * dQa[ii]);   // off-diagonal part
        const float dE = -(gs * dEi[ii] + fq * dEa[ii]);
        const float K1i = ge * dKi[ii], K1a = fk * dKa[ii];
        const float dgn = scale * d3[ii];                          // diagonal: scale M3[s][s]
        dq[ii] = dQo + dgn * kk;
        dk[ii] = K1i + K1a + dgn * qq + bb * dE;
        db[ii] = kk * dE;
        dG[ii] = qq * dQo + bb * kk * dE - kk * (K1a + (s == send ? 0.f : K1i));
        if (s < send) pend += kk * K1i;   // the exit state's k u^T terms
      }
      pend += __shfl_xor(pend, 16);
      pend += __shfl_xor(pend, 32);
      if (g4 == 3) dG[3] += L.gend[ch] * dps + pend;
      // dg = reverse cumulative sum of dG over the block's tokens
      dG[2] += dG[3];
      dG[1] += dG[2];
      dG[0] += dG[1];
      const float t1 = __shfl(dG[0], n + 16), t2 = __shfl(dG[0], n + 32);
      const float t3 = __shfl(dG[0], n + 48);
      const float after = (g4 < 1 ? t1 : 0.f) + (g4 < 2 ? t2 : 0.f) + (g4 < 3 ? t3 : 0.f);
      if (CHANNEL && p.direct) {
        // (token, key head) rows are (token, value head) rows here; one
        // column block stores, two add into outputs cleared beforehand
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int s = 4 * g4 + ii;
          if (s < nt) {
            const int64_t o = ((tok0 + t0 + s) * p.Hv + hv) * DK + ch;
            if (ncb == 1) {
              p.dq_out[o] = dq[ii];
              p.dk_out[o] = dk[ii];
              p.db[o] = db[ii];
              if (p.dg) p.dg[o] = dG[ii] + after;
            } else {
              add_pair(p.dq_out + o, dq[ii]);
              add_pair(p.dk_out + o, dk[ii]);
              add_pair(p.db + o, db[ii]);
              if (p.dg) add_pair(p.dg + o, dG[ii] + after);
            }
          }
        }
      } else {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int s = 4 * g4 + ii;
          if (s < nt) {
            const int64_t row = (tok0 + t0 + s) * p.Hv + hv;
            float* pp = p.part + ((int64_t)cb * 4 * NR + row) * DK + ch;
            pp[0] = dq[ii];
            pp[NR * DK] = dk[ii];
            pp[2 * NR * DK] = db[ii];
            pp[3 * NR * DK] = dG[ii] + after;
          }
        }
      }
    }
    if constexpr (!CHANNEL) {
      if (tid < nt) {
        const int64_t row = (tok0 + t0 + tid) * p.Hv + hv;
        p.part[(int64_t)ncb * 4 * NR * DK + (int64_t)cb * NR + row] =
            L.vs[0][tid] + L.vs[1][tid] + L.vs[2][tid] + L.vs[3][tid];
      }
    }
    lds_barrier();   // the block's LDS is rewritten by the next one
  };
  rev_block(std::false_type{}, 0);
  for (int64_t mm = 1; mm < nblk; ++mm) rev_block(std::true_type{}, mm);
  if (p.d_state_in) {
    float* dsi = p.d_state_in + head * (int64_t)DK * p.dv + colg;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float x[4] = {Dt[c][0], Dt[c][1], Dt[c][2], Dt[c][3]};
      st4f(dsi + (int64_t)ch * p.dv + 16 * c + 4 * g4, x);
    }
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

// Clears up to four fp32 arrays of n4 float4 each (a null pointer is
// skipped); a kernel rather than a memset, so that the call can be captured
// into a graph.
__global__ __launch_bounds__(256) void zero4_kernel(float* a, float* b, float* c, float* d,
                                                    int64_t n4) {
  float* const ptr[4] = {a, b, c, d};
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (!ptr[j]) continue;
    float4* q = reinterpret_cast<float4*>(ptr[j]);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) q[i] = z;
  }
}

template <int DK, bool CHANNEL, bool HAS_G, typename IO, typename GT>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  const int ncb = a.dv / kCols;
  hipError_t e;
  if (a.direct && ncb == 2 && (a.phases & 2)) {
    const int64_t n4 = a.rows * a.Hv * DK / 4;
    const int64_t want = (n4 + 255) / 256;
    zero4_kernel<<<dim3((unsigned)(want < 16384 ? want : 16384)), 256, 0, stream>>>(
        a.dq_out, a.dk_out, a.db, a.dg, n4);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)(a.B * a.Hv), (unsigned)ncb);
  if (a.phases == 2) bwd_kernel<DK, CHANNEL, HAS_G, IO, GT, true><<<grid, DK * 4, 0, stream>>>(a);
  else bwd_kernel<DK, CHANNEL, HAS_G, IO, GT, false><<<grid, DK * 4, 0, stream>>>(a);
  e = hipGetLastError();
  if (e != hipSuccess || a.direct || !(a.phases & 2)) return e;
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

#ifdef GDN_CHECK
unsigned check_violations_backward() { return take_check_violations(); }
#endif

}  // namespace gdn
