// chunk_fwd.hip -- chunkwise forward of the gated delta rule on gfx950.
//
// Method ("Gated DeltaNet-2", §3 "Entrainement Parallele Efficace par Blocs";
// "Gated DeltaNet", §Rendre l'entrainement parallele): inside a chunk of
// C = 64 tokens the cumulative decay G_t = sum_{tau<=t} g_tau is absorbed into
// the erase/write factors, a unit lower-triangular system (I + A) resolves the
// intra-chunk dependencies, and the d_k x d_v state is passed from chunk to
// chunk.  With S the state entering the chunk:
//
//   A[t,s] = sum_c e_t,c k_s,c exp(G_t,c - G_s,c)    s < t     (e = b (.) k)
//   P[t,s] = sum_c q_t,c k_s,c exp(G_t,c - G_s,c)    s <= t
//   U      = (I + A)^{-1} (Z - E_bar S)               Z_t = w_t (.) v_t,
//                                                     E_bar_t = exp(G_t) (.) e_t
//   O      = Q_bar S + P U                            Q_bar_t = exp(G_t) (.) q_t
//   S'     = Diag(exp(G_C)) S + K_hat^T U             K_hat_s = exp(G_C - G_s) (.) k_s
//
// Design for CDNA4 (one workgroup = 4 waves per (sequence, value head, slice
// of d_v); the chunks of a head are walked in order):
//  * Every d_v column evolves independently, so a workgroup owns DVS columns
//    and the state slice stays in MFMA accumulator registers for the whole
//    sequence (wave w owns 16 columns, all d_k rows).
//  * The channel decay is factored around a per-channel reference r_c (the
//    cumulative log-decay at the middle of the chunk):
//      exp(G_t - G_s) = exp(G_t - r) * exp(r - G_s),
//    so A and P become plain MFMA products of L = e exp(G - r),
//    M = q exp(G - r) and R = k exp(r - G).  Carrying the state as
//    S~ = Diag(exp(r)) S turns E_bar S into L S~ and Q_bar S into M S~.  A
//    chunk whose |G_t - r| would leave the normal fp32 range instead runs the
//    token-by-token recurrence on the register-resident state (exact, slower).
//  * Operands live in LDS in the element type of the io tensors (bf16 -> the
//    16x16x32 bf16 MFMA; fp32 -> the 16x16x4 fp32 MFMA).  Along every
//    contraction axis each 32-wide block is stored in the order in which an
//    MFMA accumulator holds its rows (lane group g: rows 4g..4g+3 of the upper
//    and of the lower 16), so register-resident results (S, X, U) feed the
//    next MFMA directly and every LDS fragment read is one 16-byte access.
//  * (I + A)^{-1} is applied by block forward substitution over four 16-token
//    blocks: the 16x16 diagonal inverses are formed in fp32 on the VALU, the
//    off-diagonal updates and the diagonal applications run on MFMA with the
//    intermediate blocks kept in registers.
#include "chunk_common.hpp"

namespace gdn {
namespace {

constexpr int kThreads = 256;   // 4 waves

// LDS plan (byte offsets) for one instantiation.
template <typename T, int DK, int DVS>
struct Lds {
  static constexpr int ES = (int)sizeof(T);
  static constexpr int PADT = 16 / ES;
  static constexpr int DKP = DK + PADT;  // pitch of [64][DK] operand arrays
  static constexpr int CP = kC + PADT;   // pitch of [*][64] operand arrays
  static constexpr int TDP = 16 + PADT;  // pitch of the 16x16 diagonal inverses
  static constexpr int ZP = kC + 4;      // pitch of Z^T (fp32)
  static constexpr int rnd(int x) { return (x + 15) & ~15; }
  static constexpr int kLn = 0;
  static constexpr int kM = kLn + rnd(kC * DKP * ES);
  static constexpr int kRK = kM + rnd(kC * DKP * ES);  // R, later K_hat^T
  static constexpr int kRKsz = rnd((kC * DKP > DK * CP ? kC * DKP : DK * CP) * ES);
  static constexpr int kP = kRK + kRKsz;
  static constexpr int kAo = kP + rnd(kC * CP * ES);
  static constexpr int kTd = kAo + rnd(kC * CP * ES);
  static constexpr int kAd = kTd + rnd(4 * 16 * TDP * ES);
  static constexpr int kOpEnd = kAd + 4 * 16 * 16 * 4;
  // token-by-token path: four [32][DK] fp32 arrays over the operand area
  static constexpr int kFb = 32 * DK * 4;
  static_assert(4 * kFb <= kOpEnd, "fallback buffers must fit in the operand area");
  static constexpr int kZ = kOpEnd;
  static constexpr int kVec = kZ + rnd(DVS * ZP * 4);
  static constexpr int kBase = kVec + 2 * DK * 4 + 16;
  // K_hat^T gets its own region when it fits (written with the other
  // operands); otherwise it reuses R's region once the Gram tiles are done.
  static constexpr int kKtSz = rnd(DK * CP * ES);
  static constexpr bool kKtSeparate = kBase + kKtSz <= 160 * 1024;
  static constexpr int kKt = kKtSeparate ? kBase : kRK;
  static constexpr int kTotal = kKtSeparate ? kBase + kKtSz : kBase;
  static_assert(kTotal <= 160 * 1024, "LDS budget");
};

template <typename T, typename GT, int DK, int DV, int DVS, bool CHANNEL, bool HAS_G>
__global__ __launch_bounds__(kThreads, 1) void chunk_fwd_kernel(Params p) {
  using L = Lds<T, DK, DVS>;
  constexpr int NSPLIT = DV / DVS;
  constexpr int NWC = DVS / 16;   // waves that own state columns
  constexpr int CPT = DK / 16;    // channels per thread in the elementwise phase
  constexpr int KB = DK / 32;     // 32-wide blocks along d_k
  constexpr int MT = DK / 16;     // 16-row tiles of the state
  constexpr float kRange = 90.f;  // |G - r| bound (log2 units) of the factored path
  static_assert(CPT % 4 == 0 && NWC >= 1 && NWC <= 4, "shape");

  __shared__ __attribute__((aligned(16))) char smem[L::kTotal];
  lds_nan_fill(smem, L::kTotal);
  T* sLn = reinterpret_cast<T*>(smem + L::kLn);
  T* sM = reinterpret_cast<T*>(smem + L::kM);
  T* sR = reinterpret_cast<T*>(smem + L::kRK);
  T* sKt = reinterpret_cast<T*>(smem + L::kKt);
  T* sP = reinterpret_cast<T*>(smem + L::kP);
  T* sAo = reinterpret_cast<T*>(smem + L::kAo);
  T* sTd = reinterpret_cast<T*>(smem + L::kTd);
  float* sAd = reinterpret_cast<float*>(smem + L::kAd);
  float* sZ = reinterpret_cast<float*>(smem + L::kZ);
  float* sR2 = reinterpret_cast<float*>(smem + L::kVec);  // exp(r), per channel
  float* sGC = sR2 + DK;                                    // exp(G_C), per channel
  float* fQ = reinterpret_cast<float*>(smem);               // token-by-token path
  float* fK = fQ + 32 * DK;
  float* fE = fK + 32 * DK;
  float* fA = fE + 32 * DK;

  const T* __restrict__ gq = static_cast<const T*>(p.q);
  const T* __restrict__ gk = static_cast<const T*>(p.k);
  const T* __restrict__ gv = static_cast<const T*>(p.v);
  const GT* __restrict__ gb = static_cast<const GT*>(p.b);
  const GT* __restrict__ gw = static_cast<const GT*>(p.w);
  const GT* __restrict__ gg = static_cast<const GT*>(p.g);
  T* __restrict__ go = static_cast<T*>(p.o);

  // Workgroup -> (head, slice).  Dispatch places workgroup i on XCD i % 8;
  // remap so that consecutive logical indices (the slices of one head, and the
  // value heads that share a key head) land on the same XCD and its L2.
  const int64_t nwg = (int64_t)gridDim.x;
  int64_t lid = blockIdx.x;
  if ((nwg & 7) == 0) lid = (lid & 7) * (nwg >> 3) + (lid >> 3);
  const int64_t head = lid / NSPLIT;  // b * Hv + hv
  const int split = (int)(lid - head * NSPLIT);
  const int64_t bidx = head / p.Hv;
  const int hv = (int)(head - bidx * p.Hv);
  const int hk = hv / (p.Hv / p.Hk);
  const int c0 = split * DVS;  // first value column of this workgroup
  // Token range of this sequence: [tok0, tok0 + Tn) in the token-major
  // tensors.  Packed sequences read their range from cu (clamped into the
  // tensor, so malformed offsets cannot reach outside it; an empty range only
  // passes the state through).
  int64_t tok0 = bidx * p.T, Tn = p.T;
  if (p.cu) {
    int64_t a0 = p.cu[bidx], a1 = p.cu[bidx + 1];
    a0 = a0 < 0 ? 0 : (a0 > p.T ? p.T : a0);
    a1 = a1 < a0 ? a0 : (a1 > p.T ? p.T : a1);
    tok0 = a0;
    Tn = a1 - a0;
  }

  const int tid = threadIdx.x;
  if (Tn == 0) {  // an empty packed sequence only passes its state through
    if (p.state_out) {
      const int64_t base = head * (int64_t)DK * DV + c0;
      for (int idx = tid; idx < DK * DVS; idx += (int)blockDim.x) {
        const int64_t e = base + (int64_t)(idx / DVS) * DV + (idx % DVS);
        p.state_out[e] = p.state_in ? p.state_in[e] : 0.f;
      }
    }
    return;
  }
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int j = lane & 15;   // MFMA: row/column within a 16x16 tile
  const int g = lane >> 4;   // MFMA: lane group
  const bool colwave = wave < NWC;

  // ---- state slice in accumulator layout: S[16mt + 4g + i][c0 + 16*wave + j]
  f32x4 S[MT];
  {
    const float* sin = p.state_in ? p.state_in + head * (int64_t)DK * DV : nullptr;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[mt][i] = (sin && colwave) ? sin[(16 * mt + 4 * g + i) * DV + c0 + 16 * wave + j] : 0.f;
  }

  // elementwise-phase mapping: 4 consecutive tokens x CPT consecutive channels
  const int tg = lane & 15;
  const int cg = wave * 4 + (lane >> 4);
  const int ch0 = cg * CPT;
  // Z^T mapping: 4 consecutive value columns x TPZ consecutive tokens
  constexpr int ZCG = DVS / 4;
  constexpr int TPZ = kC / (kThreads / ZCG);
  const int zc = tid % ZCG;
  const int zt = (tid / ZCG) * TPZ;

  // Raw inputs of one chunk in packed registers.  Every load is issued
  // unconditionally (the token index is clamped into the sequence; values of
  // tokens past the end are zeroed when unpacked) so that the whole chunk is
  // in flight at once, and the next chunk is requested while this one computes.
  constexpr int QB = CPT * (int)sizeof(T);
  constexpr int GB = CPT * (int)sizeof(GT);
  constexpr int VB = 4 * (int)sizeof(T);
  constexpr int WB = 4 * (int)sizeof(GT);
  Raw<QB> rq[4], rk[4];
  Raw<GB> rb[4], rg[4];
  float sb[4], sg[4];
  Raw<VB> rv[TPZ];
  Raw<WB> rw[TPZ];
  float zb[TPZ];
  auto load_chunk = [&](int64_t tc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t tok = tc + 4 * tg + i;
      tok = tok < Tn ? tok : Tn - 1;
      const int64_t qk_off = ((tok0 + tok) * p.Hk + hk) * (int64_t)DK + ch0;
      ld_raw<QB>(gq + qk_off, rq[i]);
      ld_raw<QB>(gk + qk_off, rk[i]);
      if constexpr (CHANNEL) {
        const int64_t g_off = ((tok0 + tok) * p.Hv + hv) * (int64_t)DK + ch0;
        ld_raw<GB>(gb + g_off, rb[i]);
        if constexpr (HAS_G) ld_raw<GB>(gg + g_off, rg[i]);
      } else {
        const int64_t s_off = (tok0 + tok) * p.Hv + hv;
        sb[i] = to_f32(gb[s_off]);
        sg[i] = HAS_G ? to_f32(gg[s_off]) : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < TPZ; ++i) {
      int64_t tok = tc + zt + i;
      tok = tok < Tn ? tok : Tn - 1;
      const int64_t v_off = ((tok0 + tok) * p.Hv + hv) * (int64_t)DV + c0 + 4 * zc;
      ld_raw<VB>(gv + v_off, rv[i]);
      if constexpr (CHANNEL) ld_raw<WB>(gw + v_off, rw[i]);
      else zb[i] = to_f32(gb[(tok0 + tok) * p.Hv + hv]);
    }
  };

  const int64_t nchunks = (Tn + kC - 1) / kC;
  load_chunk(0);  // nchunks >= 1: empty sequences returned above
  for (int64_t ci = 0; ci < nchunks; ++ci) {
    const int64_t t0 = ci * kC;
    const bool has_next = ci + 1 < nchunks;

    // ================= elementwise phase: unpack, cumulative decay, operands
    float qv[4][CPT], kv[4][CPT], bv[4][CPT], G[4][CPT], graw[4][CPT];
    auto unpack_chunk = [&]() {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool valid = t0 + 4 * tg + i < Tn;
        unpack<T, CPT>(rq[i], valid, qv[i]);
        unpack<T, CPT>(rk[i], valid, kv[i]);
        if constexpr (CHANNEL) {
          unpack<GT, CPT>(rb[i], valid, bv[i]);
          if constexpr (HAS_G) {
            unpack<GT, CPT>(rg[i], valid, graw[i]);
          } else {
#pragma unroll
            for (int e = 0; e < CPT; ++e) graw[i][e] = 0.f;
          }
        } else {
#pragma unroll
          for (int e = 0; e < CPT; ++e) {
            bv[i][e] = valid ? sb[i] : 0.f;
            graw[i][e] = valid ? sg[i] : 0.f;
          }
        }
#pragma unroll
        for (int e = 0; e < CPT; ++e) graw[i][e] *= kLog2e;  // log2 units
      }
    };
    unpack_chunk();
    float zv[TPZ][4];
#pragma unroll
    for (int i = 0; i < TPZ; ++i) {
      const bool valid = t0 + zt + i < Tn;
      unpack<T, 4>(rv[i], valid, zv[i]);
      if constexpr (CHANNEL) {
        float wz[4];
        unpack<GT, 4>(rw[i], valid, wz);
#pragma unroll
        for (int e = 0; e < 4; ++e) zv[i][e] *= wz[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) zv[i][e] *= zb[i];
      }
    }
    // inclusive prefix over the chunk: in-thread over 4 tokens, then across
    // the 16 token groups of the DPP row
    float rr[CPT], gc[CPT];
    bool bad = false;
    if constexpr (HAS_G) {
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        G[0][e] = graw[0][e];
#pragma unroll
        for (int i = 1; i < 4; ++i) G[i][e] = G[i - 1][e] + graw[i][e];
        const float tot = G[3][e];
        float x = tot;
        x += dpp_row_shr(x, 1);
        x += dpp_row_shr(x, 2);
        x += dpp_row_shr(x, 4);
        x += dpp_row_shr(x, 8);
        const float excl = x - tot;
#pragma unroll
        for (int i = 0; i < 4; ++i) G[i][e] += excl;
        rr[e] = dpp_row_bcast<7>(G[3][e]);   // G at token 31
        gc[e] = dpp_row_bcast<15>(G[3][e]);  // G at token 63 (chunk end)
#pragma unroll
        for (int i = 0; i < 4; ++i) bad |= !(fabsf(G[i][e] - rr[e]) <= kRange);
        bad |= !(rr[e] >= -100.f);
      }
    } else {
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        rr[e] = 0.f; gc[e] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) G[i][e] = 0.f;
      }
    }
    const bool slow = HAS_G ? (__syncthreads_or(bad) != 0) : false;

    // Z^T = (w (.) v)^T for this workgroup's columns (both paths read it)
#pragma unroll
    for (int i = 0; i < TPZ; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) sZ[(4 * zc + e) * L::ZP + zt + i] = zv[i][e];

    if (!slow) {
      // ---------------- factored path ----------------
      float kh[4][CPT];
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        const float cC = HAS_G ? exp2_fast(gc[e] - rr[e]) : 1.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = G[i][e] - rr[e];
          const float e1 = HAS_G ? exp2_fast(x) : 1.f;
          const float e2 = HAS_G ? exp2_fast(-x) : 1.f;
          const float ev = bv[i][e] * kv[i][e];
          bv[i][e] = -ev * e1;           // Ln = -e exp(G - r)
          qv[i][e] = qv[i][e] * e1;      // M  =  q exp(G - r)
          kh[i][e] = kv[i][e] * e2;      // R  =  k exp(r - G)
          kv[i][e] = kh[i][e];
          kh[i][e] *= cC;                // K_hat = k exp(G_C - G)
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * tg + i;
#pragma unroll
        for (int u = 0; u < CPT / 4; ++u) {
          const int pos = sig(ch0 + 4 * u);
          st4<T>(sLn + t * L::DKP + pos, bv[i][4 * u], bv[i][4 * u + 1], bv[i][4 * u + 2], bv[i][4 * u + 3]);
          st4<T>(sM + t * L::DKP + pos, qv[i][4 * u], qv[i][4 * u + 1], qv[i][4 * u + 2], qv[i][4 * u + 3]);
          st4<T>(sR + t * L::DKP + pos, kv[i][4 * u], kv[i][4 * u + 1], kv[i][4 * u + 2], kv[i][4 * u + 3]);
        }
      }
      if constexpr (L::kKtSeparate) {
#pragma unroll
        for (int e = 0; e < CPT; ++e)
          st4<T>(sKt + (ch0 + e) * L::CP + sig(4 * tg), kh[0][e], kh[1][e], kh[2][e], kh[3][e]);
      }
      if (tg == 0) {
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
          sR2[ch0 + e] = HAS_G ? exp2_fast(rr[e]) : 1.f;
          sGC[ch0 + e] = HAS_G ? exp2_fast(gc[e]) : 1.f;
        }
      }
      __syncthreads();  // B1
      if (has_next) load_chunk(t0 + kC);

      // ---- A and P tiles: D[s][t] = sum_c R[s][c] X[t][c], X = Ln (gives -A) or M (gives P)
#pragma unroll
      for (int it = 0; it < 5; ++it) {
        const int tile = wave + 4 * it;
        const bool isP = tile >= 10;
        const int tt = isP ? tile - 10 : tile;
        // (ms, nt) enumeration of the lower block triangle
        const int nt = tt >= 6 ? 3 : (tt >= 3 ? 2 : (tt >= 1 ? 1 : 0));
        const int ms = tt - (nt * (nt + 1)) / 2;
        const T* X = isP ? sM : sLn;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const Frag8<T> a = ld_frag8<T>(sR + (16 * ms + j) * L::DKP + 32 * kb + 8 * g);
          const Frag8<T> bq = ld_frag8<T>(X + (16 * nt + j) * L::DKP + 32 * kb + 8 * g);
          mma32(acc, a, bq);
        }
        const int t = 16 * nt + j;
        if (isP) {
          float pv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[i] = (16 * ms + 4 * g + i <= t) ? acc[i] : 0.f;
          st4<T>(sP + t * L::CP + sig(16 * ms + 4 * g), pv[0], pv[1], pv[2], pv[3]);
          // The causal product reads whole 32-token blocks: the block above
          // an even diagonal block is read too and must be zero.
          if (ms == nt && (nt & 1) == 0)
            st4<T>(sP + t * L::CP + sig(16 * (ms + 1) + 4 * g), 0.f, 0.f, 0.f, 0.f);
        } else if (ms == nt) {
          // diagonal block, fp32, stored transposed: sAd[blk][s][t] = A[t][s]
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int sl = 4 * g + i;
            sAd[(ms * 16 + sl) * 16 + j] = (sl < j) ? -acc[i] : 0.f;
          }
        } else {
          // off-diagonal block of -A, natural order within the 16-block
          st4<T>(sAo + t * L::CP + 16 * ms + 4 * g, acc[0], acc[1], acc[2], acc[3]);
        }
      }
      __syncthreads();  // B2: R is dead, A/P written

      // K_hat^T over R's space: sKt[c][sig(s)]
      if constexpr (!L::kKtSeparate) {
#pragma unroll
        for (int e = 0; e < CPT; ++e)
          st4<T>(sKt + (ch0 + e) * L::CP + sig(4 * tg), kh[0][e], kh[1][e], kh[2][e], kh[3][e]);
      }

      // S~ = Diag(exp(r)) S as K=32 fragments; X' = Z + Ln S~ (= Z - E_bar S);
      // O^T = S~^T M^T (= (Q_bar S)^T).
      f32x4 X[4], O[4];
      Frag8<T> sf[KB];
      if (colwave) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          f32x4 lo = S[2 * kb], hi = S[2 * kb + 1];
          if constexpr (HAS_G) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              lo[i] *= sR2[32 * kb + 4 * g + i];
              hi[i] *= sR2[32 * kb + 16 + 4 * g + i];
            }
          }
          sf[kb] = frag8_from_acc<T>(lo, hi);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const float4 z = *reinterpret_cast<const float4*>(sZ + (16 * wave + j) * L::ZP + 16 * mt + 4 * g);
          X[mt][0] = z.x; X[mt][1] = z.y; X[mt][2] = z.z; X[mt][3] = z.w;
          O[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            const Frag8<T> a = ld_frag8<T>(sLn + (16 * mt + j) * L::DKP + 32 * kb + 8 * g);
            mma32(X[mt], a, sf[kb]);
            const Frag8<T> bm = ld_frag8<T>(sM + (16 * mt + j) * L::DKP + 32 * kb + 8 * g);
            mma32(O[mt], sf[kb], bm);
          }
        }
      }
      // 16x16 diagonal inverses T_bb = (I + A_bb)^{-1} in fp32, wave w forming
      // block w (issued after this wave's MFMAs above, which run meanwhile).
      // Row form, each row independent: T[r][r] = 1 and, for s = r-1 .. 0,
      // T[r][s] = -sum_{u>s} T[r][u] A[u][s].  Lane j forms row j (the four
      // lane groups compute the same rows); column s of A is read as 4 x 16 B
      // one step ahead of its use.
      {
        const int r = j;
        const float* ad = sAd + wave * 256;  // ad[s * 16 + u] = A[u][s]
        float trow[16];
        float cur[16], nxt[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 c4 = *reinterpret_cast<const float4*>(ad + 15 * 16 + 4 * q4);
          cur[4 * q4] = c4.x; cur[4 * q4 + 1] = c4.y; cur[4 * q4 + 2] = c4.z; cur[4 * q4 + 3] = c4.w;
        }
#pragma unroll
        for (int s = 15; s >= 0; --s) {
          if (s > 0) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const float4 c4 = *reinterpret_cast<const float4*>(ad + (s - 1) * 16 + 4 * q4);
              nxt[4 * q4] = c4.x; nxt[4 * q4 + 1] = c4.y; nxt[4 * q4 + 2] = c4.z; nxt[4 * q4 + 3] = c4.w;
            }
          }
          float a0 = 0.f, a1 = 0.f;
#pragma unroll
          for (int u = s + 1; u < 16; ++u) {
            if (u & 1) a1 -= trow[u] * cur[u];
            else a0 -= trow[u] * cur[u];
          }
          trow[s] = (s > r) ? 0.f : ((s == r) ? 1.f : a0 + a1);
#pragma unroll
          for (int u = 0; u < 16; ++u) cur[u] = nxt[u];
        }
        if (g == 0) {
          T* dst = sTd + (wave * 16 + r) * L::TDP;
#pragma unroll
          for (int u = 0; u < 4; ++u)
            st4<T>(dst + 4 * u, trow[4 * u], trow[4 * u + 1], trow[4 * u + 2], trow[4 * u + 3]);
        }
      }
      __syncthreads();  // B3: K_hat^T and the diagonal inverses are visible

      if (colwave) {
        // U = (I + A)^{-1} X' by block forward substitution (K = 16 MFMAs)
        f32x4 U[4];
        Frag4<T> uf[4];
#pragma unroll
        for (int bi = 0; bi < 4; ++bi) {
          f32x4 acc = X[bi];
#pragma unroll
          for (int bj = 0; bj < bi; ++bj) {
            const Frag4<T> a = ld_frag4<T>(sAo + (16 * bi + j) * L::CP + 16 * bj + 4 * g);
            mma16(acc, a, uf[bj]);
          }
          const Frag4<T> xf = frag4_from_acc<T>(acc);
          const Frag4<T> td = ld_frag4<T>(sTd + (bi * 16 + j) * L::TDP + 4 * g);
          U[bi] = f32x4{0.f, 0.f, 0.f, 0.f};
          mma16(U[bi], td, xf);
          uf[bi] = frag4_from_acc<T>(U[bi]);
        }
        Frag8<T> u8[2];
        u8[0] = frag8_from_acc<T>(U[0], U[1]);
        u8[1] = frag8_from_acc<T>(U[2], U[3]);

        // O^T += U^T P^T  (causal: token block kb contributes to t-tile nt when 32kb <= 16nt+15)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
            if (32 * kb <= 16 * nt + 15) {
              const Frag8<T> bp = ld_frag8<T>(sP + (16 * nt + j) * L::CP + 32 * kb + 8 * g);
              mma32(O[nt], u8[kb], bp);
            }

        // S <- Diag(exp(G_C)) S + K_hat^T U
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if constexpr (HAS_G) {
#pragma unroll
            for (int i = 0; i < 4; ++i) S[mt][i] *= sGC[16 * mt + 4 * g + i];
          }
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const Frag8<T> a = ld_frag8<T>(sKt + (16 * mt + j) * L::CP + 32 * kb + 8 * g);
            mma32(S[mt], a, u8[kb]);
          }
        }

        // o[t][c0 + 16 wave + 4g + i] = scale * O^T[4g + i][t]
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int64_t tok = t0 + 16 * nt + j;
          if (tok < Tn) {
            T* dst = go + ((tok0 + tok) * p.Hv + hv) * (int64_t)DV + c0 + 16 * wave + 4 * g;
            st4<T>(dst, p.scale * O[nt][0], p.scale * O[nt][1], p.scale * O[nt][2], p.scale * O[nt][3]);
          }
        }
      }
      __syncthreads();  // B4: LDS free for the next chunk
    } else {
      // ---------------- token-by-token path (exact in fp32) ----------------
      // Used when the factored operands would leave the fp32 range.  Two
      // halves of 32 tokens are staged in LDS; the state stays in registers.
      // The chunk is read again (this path is rare) rather than holding its
      // unpacked values live through the common path.
      load_chunk(t0);
      unpack_chunk();
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if ((tg >> 3) == half) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tl = 4 * tg + i - 32 * half;
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
              fQ[tl * DK + ch0 + e] = qv[i][e];
              fK[tl * DK + ch0 + e] = kv[i][e];
              fE[tl * DK + ch0 + e] = bv[i][e] * kv[i][e];
              fA[tl * DK + ch0 + e] = HAS_G ? exp2_fast(graw[i][e]) : 1.f;
            }
          }
        }
        __syncthreads();
        if (colwave) {
          for (int tl = 0; tl < 32; ++tl) {
            const int64_t tok = t0 + 32 * half + tl;
            if (tok >= Tn) break;
            float rp = 0.f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int row = 16 * mt + 4 * g + i;
                S[mt][i] *= fA[tl * DK + row];
                rp += fE[tl * DK + row] * S[mt][i];
              }
            rp += __shfl_xor(rp, 16);
            rp += __shfl_xor(rp, 32);
            const float d = sZ[(16 * wave + j) * L::ZP + 32 * half + tl] - rp;
            float op = 0.f;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int row = 16 * mt + 4 * g + i;
                S[mt][i] += fK[tl * DK + row] * d;
                op += fQ[tl * DK + row] * S[mt][i];
              }
            op += __shfl_xor(op, 16);
            op += __shfl_xor(op, 32);
            if (g == 0)
              go[((tok0 + tok) * p.Hv + hv) * (int64_t)DV + c0 + 16 * wave + j] = from_f32<T>(p.scale * op);
          }
        }
        __syncthreads();
      }
      if (has_next) load_chunk(t0 + kC);
    }
  }

  // ---- final state
  if (p.state_out && colwave) {
    float* sout = p.state_out + head * (int64_t)DK * DV;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sout[(16 * mt + 4 * g + i) * DV + c0 + 16 * wave + j] = S[mt][i];
  }
}

template <typename T, typename GT, int DK, int DV, int DVS, bool CH, bool HG>
hipError_t launch_typed(const ChunkArgs& a, hipStream_t stream) {
  Params p;
  p.B = a.B; p.T = a.T; p.cu = a.cu_seqlens; p.Hk = a.Hk; p.Hv = a.Hv; p.scale = a.scale;
  p.q = a.q; p.k = a.k; p.v = a.v; p.b = a.b; p.w = a.w; p.g = a.g;
  p.state_in = a.state_in; p.state_out = a.state_out; p.o = a.o;
  const int64_t nwg = a.B * a.Hv * (DV / DVS);
  chunk_fwd_kernel<T, GT, DK, DV, DVS, CH, HG><<<dim3((unsigned)nwg), dim3(kThreads), 0, stream>>>(p);
  return hipGetLastError();
}

template <typename T, typename GT, int DK, int DV, int DVS>
hipError_t pick_gates(const ChunkArgs& a, hipStream_t s) {
  const bool hg = a.g != nullptr;
  if (a.channel) return hg ? launch_typed<T, GT, DK, DV, DVS, true, true>(a, s)
                           : launch_typed<T, GT, DK, DV, DVS, true, false>(a, s);
  return hg ? launch_typed<T, GT, DK, DV, DVS, false, true>(a, s)
            : launch_typed<T, GT, DK, DV, DVS, false, false>(a, s);
}

// d_v slice per workgroup: 64 columns (4 waves x 16); fp32 operands with
// d_k = 128 take 32 columns so that the LDS plan fits.
template <typename T, typename GT>
hipError_t pick_dims(const ChunkArgs& a, hipStream_t s) {
  constexpr bool F32 = sizeof(T) == 4;
  if (a.dk == 128 && a.dv == 128) return pick_gates<T, GT, 128, 128, F32 ? 32 : 64>(a, s);
  if (a.dk == 128 && a.dv == 64) return pick_gates<T, GT, 128, 64, F32 ? 32 : 64>(a, s);
  if (a.dk == 64 && a.dv == 128) return pick_gates<T, GT, 64, 128, 64>(a, s);
  return pick_gates<T, GT, 64, 64, 64>(a, s);
}

__global__ void state_copy_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src ? src[i] : 0.f;
}

}  // namespace

// bf16 operands run the sub-block kernel (chunk_fwd_sb.hip); fp32
// operands run the sequential-phase kernel of this file.
hipError_t launch_chunk_fwd(const ChunkArgs& a, hipStream_t stream) {
  if (a.io == DType::BF16) return launch_chunk_fwd_sb(a, stream);
  return pick_dims<float, float>(a, stream);
}

hipError_t launch_state_copy(const float* state_in, float* state_out, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  state_copy_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(state_in, state_out, n);
  return hipGetLastError();
}

#ifdef GDN_CHECK
unsigned check_violations_chunk() { return take_check_violations(); }
#endif

}  // namespace gdn
