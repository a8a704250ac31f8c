// chunk_fwd_pipe.hip -- producer/consumer chunkwise forward (bf16 operands).
//
// Same mathematics as chunk_fwd.hip ("Gated DeltaNet-2", §3 "Entrainement
// Parallele Efficace par Blocs"): per chunk of 64 tokens, with S the state
// entering the chunk and r_c a per-channel reference of the cumulative
// log-decay,
//   L = -e exp(G - r), M = q exp(G - r), R = k exp(r - G)    (elementwise)
//   A = strict_lower(L R^T), P = lower(M R^T)                (Gram tiles)
//   X = Z + L S~,  S~ = Diag(exp(r)) S                       (S-dependent)
//   U = (I + A)^{-1} X                                        (forward subst.)
//   O = M S~ + P U,  S' = Diag(exp(G_C)) S + K_hat^T U.
//
// Work split inside one workgroup of 8 waves (two per SIMD):
//   consumer waves 0-3 own the fp32 state slice (16 value columns each, in
//     MFMA accumulators); they run the S-dependent MFMA chain and, in the
//     same pass over the operands, the 16 off-diagonal Gram tiles of A and P
//     (their MFMA pipe would otherwise wait for the producers);
//   producer waves 4-7 run the VALU side: loads (prefetched a chunk ahead),
//     the cumulative decay, the exponentials and gated operands, and the four
//     16x16 diagonal blocks of A with their fp32 inverses.
// With scalar gates (Gated DeltaNet, DeltaNet) the decay factors out of the
// Gram matrices ("Gated DeltaNet-2", §3; the GDN-1 form of the scope): the
// producers store raw q and k, and the per-token factors exp(G_t - r),
// exp(r - G_t), beta_t are applied as a 64x64 mask on the Gram tiles and as
// row scales of the MFMA results, so the producers do no per-element math.
//
// Two workgroup barriers per chunk c:
//
//   interval 2(c): consumers  X, O (c); off-diagonal A, P tiles (c)
//                  producers  diagonal A blocks + inverses (c);
//                             decay prefix, flags, Z^T (c+1); load g, v, w (c+2)
//   ---- barrier A
//   interval 1(c): consumers  U, O += P U, S', store o (c)
//                  producers  gated operands L, M, R, K_hat^T (c+1); load q, k, b (c+2)
//   ---- barrier B
//
// L, M and R are written in interval 1 and read only in interval 2, so they
// are single buffered; Z^T, K_hat^T, the per-channel vectors and the flags
// are written one interval ahead of a reader of the previous chunk and are
// double buffered.  A chunk whose decay range would leave the fp32 range of
// the factored operands is run token by token by the consumers instead.
#include "chunk_common.hpp"

namespace gdn {
namespace {

constexpr int kPipeThreads = 512;  // 4 consumer + 4 producer waves

template <int N>
struct IntTag {
  static constexpr int value = N;
};

template <typename T, int DK, int DVS>
struct PipeLds {
  static constexpr int ES = (int)sizeof(T);
  static constexpr int PADT = 16 / ES;
  static constexpr int DKP = DK + PADT;  // pitch of [64][DK] operand arrays
  // Element offset of (row, pos) in a [64][DK] operand array.  The 16-byte
  // column blocks of each row are XOR-swizzled by (row / 8) mod 8: the
  // producers store rows four tokens apart and the consumers read sixteen
  // consecutive rows, and both then spread over all banks.
  __device__ static constexpr int at(int row, int pos) {
    return row * DKP + (pos ^ (8 * ((row >> 3) & 7)));
  }
  static constexpr int CP = kC + PADT;   // pitch of [*][64] operand arrays
  static constexpr int TDP = 16 + PADT;  // pitch of the diagonal inverses
  static constexpr int ZP = kC + 4;      // pitch of Z^T (fp32)
  static constexpr int rnd(int x) { return (x + 15) & ~15; }
  static constexpr int kLn = 0;
  static constexpr int kM = kLn + rnd(kC * DKP * ES);
  static constexpr int kR = kM + rnd(kC * DKP * ES);
  static constexpr int kKt = kR + rnd(kC * DKP * ES);  // two buffers
  static constexpr int kKtSz = rnd(DK * CP * ES);
  static constexpr int kP = kKt + 2 * kKtSz;
  static constexpr int kAo = kP + rnd(kC * CP * ES);
  static constexpr int kTd = kAo + rnd(kC * CP * ES);
  static constexpr int kZ = kTd + rnd(4 * 16 * TDP * ES);  // two buffers
  static constexpr int kZSz = rnd(DVS * ZP * 4);
  static constexpr int kVec = kZ + 2 * kZSz;           // two buffers of [exp(r) | exp(G_C)]
  static constexpr int kTok = kVec + 2 * 2 * DK * 4;   // two buffers of [8][64] per-token factors
  static constexpr int kFlag = kTok + 2 * 8 * kC * 4;  // two buffers of 4 ints
  static constexpr int kTotal = kFlag + 2 * 4 * 4;
  static_assert(kTotal <= 160 * 1024, "LDS budget");
};

template <typename T, typename GT, int DK, int DV, int DVS, bool CHANNEL, bool HAS_G>
__global__ __launch_bounds__(kPipeThreads, 1) void chunk_fwd_pipe_kernel(Params p) {
  using L = PipeLds<T, DK, DVS>;
  constexpr int NSPLIT = DV / DVS;
  constexpr int CPT = DK / 16;  // channels per producer thread
  constexpr int KB = DK / 32;
  constexpr int MT = DK / 16;
  constexpr float kRange = 90.f;  // |G - r| bound (log2 units) of the factored form
  static_assert(DVS == 64 && CPT % 4 == 0, "shape");

  __shared__ __attribute__((aligned(16))) char smem[L::kTotal];
  T* sLn = reinterpret_cast<T*>(smem + L::kLn);
  T* sM = reinterpret_cast<T*>(smem + L::kM);
  T* sR = reinterpret_cast<T*>(smem + L::kR);
  T* sKt0 = reinterpret_cast<T*>(smem + L::kKt);
  T* sP = reinterpret_cast<T*>(smem + L::kP);
  T* sAo = reinterpret_cast<T*>(smem + L::kAo);
  T* sTd = reinterpret_cast<T*>(smem + L::kTd);
  float* sZ0 = reinterpret_cast<float*>(smem + L::kZ);
  float* sVec0 = reinterpret_cast<float*>(smem + L::kVec);
  int* sFlag = reinterpret_cast<int*>(smem + L::kFlag);
  float* sTok0 = reinterpret_cast<float*>(smem + L::kTok);
  // Scalar gates: per-token factors of chunk ci in sTok0 + (ci & 1) * 512,
  // each a [64] vector (x_t = (G_t - r) log2 e, r = G at token 31):
  constexpr int kFE1 = 0;  // exp2(x_t)
  constexpr int kFE2 = 1;  // exp2(-x_t)
  constexpr int kFNB = 2;  // -beta_t exp2(x_t)
  constexpr int kFX = 3;   // -beta_t exp(G_t): X = Z + diag(FX) K S
  constexpr int kFO = 4;   // exp(G_t):         O = diag(FO) Q S + P U
  constexpr int kFK = 5;   // exp(G_C - G_t):   S' = exp(G_C) S + K^T diag(FK) U
  constexpr int kFG = 6;   // [0] = exp(G_C)

  const T* __restrict__ gq = static_cast<const T*>(p.q);
  const T* __restrict__ gk = static_cast<const T*>(p.k);
  const T* __restrict__ gv = static_cast<const T*>(p.v);
  const GT* __restrict__ gb = static_cast<const GT*>(p.b);
  const GT* __restrict__ gw = static_cast<const GT*>(p.w);
  const GT* __restrict__ gg = static_cast<const GT*>(p.g);
  T* __restrict__ go = static_cast<T*>(p.o);

  // Workgroup -> (head, d_v slice), XCD-aware (workgroup i runs on XCD i % 8;
  // the slices of one head land on the same XCD and share its L2).
  const int64_t nwg = (int64_t)gridDim.x;
  int64_t lid = blockIdx.x;
  if ((nwg & 7) == 0) lid = (lid & 7) * (nwg >> 3) + (lid >> 3);
  const int64_t head = lid / NSPLIT;
  const int split = (int)(lid - head * NSPLIT);
  const int64_t bidx = head / p.Hv;
  const int hv = (int)(head - bidx * p.Hv);
  const int hk = hv / (p.Hv / p.Hk);
  const int c0 = split * DVS;
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
  const int64_t nchunks = (Tn + kC - 1) / kC;

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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool consumer = wave < 4;
  const int j = lane & 15;
  const int g = lane >> 4;

  // =====================================================================
  // Producer side (waves 4-7): thread ptid handles 4 consecutive tokens x
  // CPT consecutive channels of the chunk, and 4 value columns x TPZ tokens.
  // =====================================================================
  const int pw = wave - 4;
  const int ptid = tid - 256;
  const int tg = lane & 15;
  const int ch0 = (pw * 4 + (lane >> 4)) * CPT;
  constexpr int ZCG = DVS / 4;
  constexpr int TPZ = kC / (256 / ZCG);
  const int zc = ptid % ZCG;
  const int zt = (ptid / ZCG) * TPZ;

  constexpr int QB = CPT * (int)sizeof(T);
  constexpr int GB = CPT * (int)sizeof(GT);
  constexpr int VB = 4 * (int)sizeof(T);
  constexpr int WB = 4 * (int)sizeof(GT);
  // raw words of the chunk being prefetched / consumed
  Raw<QB> rq[4], rk[4];
  Raw<GB> rb[4], rg[4];     // channel gates
  uint32_t ub[4], ug[4];    // scalar gates
  Raw<VB> rv[TPZ];
  Raw<WB> rw[TPZ];          // channel write gate
  uint32_t uz[TPZ];         // scalar beta for the write side

  // Load addressing: a wave-uniform 64-bit base per chunk (SGPRs) plus a
  // per-thread 32-bit byte offset that is the same for every chunk.  Only a
  // partial last chunk clamps the token index (tokens past the end re-read
  // the last token) and then zeroes the raw words of the absent tokens, so
  // full chunks need no masking anywhere.
  const uint32_t qk_tok = (uint32_t)(p.Hk * DK * (int)sizeof(T));    // bytes per token
  const uint32_t gc_tok = (uint32_t)(p.Hv * DK * (int)sizeof(GT));   // channel gates
  const uint32_t gs_tok = (uint32_t)(p.Hv * (int)sizeof(GT));        // scalar gates
  const uint32_t v_tok = (uint32_t)(p.Hv * DV * (int)sizeof(T));
  const uint32_t w_tok = (uint32_t)(p.Hv * DV * (int)sizeof(GT));
  const char* bq = reinterpret_cast<const char*>(gq) + ((uint64_t)tok0 * qk_tok + (uint32_t)(hk * DK * (int)sizeof(T)));
  const char* bk = reinterpret_cast<const char*>(gk) + ((uint64_t)tok0 * qk_tok + (uint32_t)(hk * DK * (int)sizeof(T)));
  const char* bbc = reinterpret_cast<const char*>(gb) + ((uint64_t)tok0 * gc_tok + (uint32_t)(hv * DK * (int)sizeof(GT)));
  const char* bgc = reinterpret_cast<const char*>(gg) + ((uint64_t)tok0 * gc_tok + (uint32_t)(hv * DK * (int)sizeof(GT)));
  const char* bbs = reinterpret_cast<const char*>(gb) + ((uint64_t)tok0 * gs_tok + (uint32_t)(hv * (int)sizeof(GT)));
  const char* bgs = reinterpret_cast<const char*>(gg) + ((uint64_t)tok0 * gs_tok + (uint32_t)(hv * (int)sizeof(GT)));
  const char* bv = reinterpret_cast<const char*>(gv) + ((uint64_t)tok0 * v_tok + (uint32_t)((hv * DV + c0) * (int)sizeof(T)));
  const char* bw = reinterpret_cast<const char*>(gw) + ((uint64_t)tok0 * w_tok + (uint32_t)((hv * DV + c0) * (int)sizeof(GT)));
  const uint32_t oq = (uint32_t)(ch0 * (int)sizeof(T));
  const uint32_t og = (uint32_t)(ch0 * (int)sizeof(GT));
  const uint32_t ov = (uint32_t)(4 * zc * (int)sizeof(T));
  const uint32_t ow = (uint32_t)(4 * zc * (int)sizeof(GT));

  // Decay, value and write gate of the chunk starting at token tc.
  auto load_gvw = [&](int64_t tc) {
    const bool full = tc + kC <= Tn;  // wave-uniform
    const int64_t last = Tn - 1 - tc;
    const uint64_t tcu = (uint64_t)tc;
    const char* cgc = bgc + tcu * gc_tok;
    const char* cgs = bgs + tcu * gs_tok;
    const char* cbs = bbs + tcu * gs_tok;
    const char* cv = bv + tcu * v_tok;
    const char* cw = bw + tcu * w_tok;
    if constexpr (HAS_G) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t t = (uint32_t)(4 * tg + i);
        if (!full) t = (int64_t)t < last ? t : (uint32_t)last;
        if constexpr (CHANNEL) ld_raw<GB>(cgc + (t * gc_tok + og), rg[i]);
        else ug[i] = ld_word<GT>(cgs + t * gs_tok);
      }
    }
#pragma unroll
    for (int i = 0; i < TPZ; ++i) {
      uint32_t t = (uint32_t)(zt + i);
      if (!full) t = (int64_t)t < last ? t : (uint32_t)last;
      ld_raw<VB>(cv + (t * v_tok + ov), rv[i]);
      if constexpr (CHANNEL) ld_raw<WB>(cw + (t * w_tok + ow), rw[i]);
      else uz[i] = ld_word<GT>(cbs + t * gs_tok);
    }
    if (!full) {  // absent tokens: g = 0 (no decay), z = 0
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((int64_t)(4 * tg + i) > last) {
          if constexpr (HAS_G) {
            if constexpr (CHANNEL) zero_raw(rg[i]);
            else ug[i] = 0u;
          }
        }
#pragma unroll
      for (int i = 0; i < TPZ; ++i)
        if ((int64_t)(zt + i) > last) zero_raw(rv[i]);
    }
  };
  // Query, key and erase gate of the chunk starting at token tc.
  auto load_qkb = [&](int64_t tc) {
    const bool full = tc + kC <= Tn;
    const int64_t last = Tn - 1 - tc;
    const uint64_t tcu = (uint64_t)tc;
    const char* cq = bq + tcu * qk_tok;
    const char* ck = bk + tcu * qk_tok;
    const char* cbc = bbc + tcu * gc_tok;
    const char* cbs = bbs + tcu * gs_tok;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t t = (uint32_t)(4 * tg + i);
      if (!full) t = (int64_t)t < last ? t : (uint32_t)last;
      ld_raw<QB>(cq + (t * qk_tok + oq), rq[i]);
      ld_raw<QB>(ck + (t * qk_tok + oq), rk[i]);
      if constexpr (CHANNEL) ld_raw<GB>(cbc + (t * gc_tok + og), rb[i]);
      else ub[i] = ld_word<GT>(cbs + t * gs_tok);
    }
    if (!full) {  // absent tokens: q = k = 0, b = 0
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((int64_t)(4 * tg + i) > last) {
          zero_raw(rq[i]);
          zero_raw(rk[i]);
          if constexpr (CHANNEL) zero_raw(rb[i]);
          else ub[i] = 0u;
        }
    }
  };

  // Decay prefix of chunk ci, carried from part 1 to part 2 in registers:
  // x = G - r (log2 units) per token and channel, and exp2(G_C - r).
  float X2[4][CPT], cC[CPT];

  // Part 1 of the operands of chunk ci: cumulative decay, range flag,
  // per-channel vectors and Z^T (producer interval 2 of chunk ci - 1).
  auto produce_decay = [&](int64_t ci) {
    const int slot = (int)(ci & 1);
    float* sZ = sZ0 + slot * (L::kZSz / 4);
    float* sR2 = sVec0 + slot * 2 * DK;
    float* sGC = sR2 + DK;
    // Z^T = (w (.) v)^T for this workgroup's columns: the TPZ = 4
    // consecutive tokens of a column go out as one 16-byte store
    static_assert(TPZ == 4, "Z^T store");
    float zz[4][TPZ];
#pragma unroll
    for (int i = 0; i < TPZ; ++i) {
      float zv[4];
      unpack<T, 4>(rv[i], zv);
      if constexpr (CHANNEL) {
        float wz[4];
        unpack<GT, 4>(rw[i], wz);
#pragma unroll
        for (int e = 0; e < 4; ++e) zv[e] *= wz[e];
      } else {
        const float beta = word_f32<GT>(uz[i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) zv[e] *= beta;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) zz[e][i] = zv[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      *reinterpret_cast<float4*>(sZ + (4 * zc + e) * L::ZP + zt) = make_float4(zz[e][0], zz[e][1], zz[e][2], zz[e][3]);
    if constexpr (!CHANNEL) {
      // one decay per token: prefix over the 4 tokens of the thread and the
      // 16 token groups of the DPP row; every lane row computes the same.
      float gt[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) gt[i] = HAS_G ? word_f32<GT>(ug[i]) : 0.f;
#pragma unroll
      for (int i = 1; i < 4; ++i) gt[i] += gt[i - 1];
      float x = gt[3];
      x += dpp_row_shr(x, 1);
      x += dpp_row_shr(x, 2);
      x += dpp_row_shr(x, 4);
      x += dpp_row_shr(x, 8);
      const float rr = dpp_row_bcast<7>(x);
      const float gc = dpp_row_bcast<15>(x);
      const float sh = (x - gt[3] - rr) * kLog2e;
      float xt[4];
      float worst = -100.f - rr * kLog2e + kRange;  // > kRange iff r < -100 (log2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xt[i] = fmaf(gt[i], kLog2e, sh);
        worst = fmaxf(worst, fabsf(xt[i]));
      }
      const bool any_bad = __any(!(worst <= kRange));
      if (lane == 0) sFlag[slot * 4 + pw] = any_bad ? 1 : 0;
      // Every lane computes the factors (the same instructions either way);
      // only the stores are masked.  Reading beta outside a branch also keeps
      // the compiler's view of the outstanding loads exact.
      float* tok = sTok0 + slot * 8 * kC;
      const float r2 = exp2_fast(rr * kLog2e);
      const float cC = exp2_fast((gc - rr) * kLog2e);
      const float gC = exp2_fast(gc * kLog2e);
      float f[6][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e1 = exp2_fast(xt[i]);
        const float e2 = exp2_fast(-xt[i]);
        const float nb = -word_f32<GT>(ub[i]) * e1;
        f[kFE1][i] = e1;
        f[kFE2][i] = e2;
        f[kFNB][i] = nb;
        f[kFX][i] = nb * r2;
        f[kFO][i] = e1 * r2;
        f[kFK][i] = cC * e2;
      }
      if (g == 0) {  // lanes 0-15 hold tokens 4 tg .. 4 tg + 3
#pragma unroll
        for (int a = 0; a < 6; ++a)
          *reinterpret_cast<float4*>(tok + a * kC + 4 * tg) = make_float4(f[a][0], f[a][1], f[a][2], f[a][3]);
        if (tg == 0 && pw == 0) tok[kFG * kC] = gC;
      }
    } else if constexpr (HAS_G) {
      // cumulative log2-decay over the chunk (4 tokens in-thread, then the
      // 16 token groups of the DPP row); reference r = G at token 31
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (CHANNEL) {
          unpack<GT, CPT>(rg[i], X2[i]);
        } else {
          const float gi = word_f32<GT>(ug[i]);
#pragma unroll
          for (int e = 0; e < CPT; ++e) X2[i][e] = gi;
        }
      }
      float worst = 0.f;
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        X2[0][e] *= kLog2e;
#pragma unroll
        for (int i = 1; i < 4; ++i) X2[i][e] = X2[i - 1][e] + X2[i][e] * kLog2e;
        const float tot = X2[3][e];
        float x = tot;
        x += dpp_row_shr(x, 1);
        x += dpp_row_shr(x, 2);
        x += dpp_row_shr(x, 4);
        x += dpp_row_shr(x, 8);
        const float excl = x - tot;
        const float rr = dpp_row_bcast<7>(x);
        const float gc = dpp_row_bcast<15>(x);
        // x = G - r; the range test needs only the largest |x| of the thread
#pragma unroll
        for (int i = 0; i < 4; ++i) X2[i][e] += excl - rr;
        worst = fmaxf(worst, fmaxf(fmaxf(fabsf(X2[0][e]), fabsf(X2[1][e])),
                                   fmaxf(fabsf(X2[2][e]), fabsf(X2[3][e]))));
        worst = fmaxf(worst, -100.f - rr + kRange);  // > kRange iff r < -100
        cC[e] = exp2_fast(gc - rr);
        if (tg == 0) {
          sR2[ch0 + e] = exp2_fast(rr);
          sGC[ch0 + e] = exp2_fast(gc);
        }
      }
      const bool any_bad = __any(!(worst <= kRange));
      if (lane == 0) sFlag[slot * 4 + pw] = any_bad ? 1 : 0;
    } else {
      if (lane == 0) sFlag[slot * 4 + pw] = 0;
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        if (tg == 0) {
          sR2[ch0 + e] = 1.f;
          sGC[ch0 + e] = 1.f;
        }
      }
    }
  };

  // Part 2: gated operands of chunk ci (producer interval 1 of chunk ci - 1).
  auto produce_operands = [&](int64_t ci) {
    const int slot = (int)(ci & 1);
    T* sKt = sKt0 + slot * (L::kKtSz / L::ES);
    if constexpr (!CHANNEL) {
      // raw q and k rows (each run of 4 channels at its accumulator-order
      // position) and raw k^T (4 tokens per channel, repacked with v_perm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * tg + i;
#pragma unroll
        for (int u = 0; u < CPT / 4; ++u) {
          const int pos = sig(ch0 + 4 * u);
          *reinterpret_cast<uint2*>(sM + L::at(t, pos)) = make_uint2(rq[i].w[2 * u], rq[i].w[2 * u + 1]);
          *reinterpret_cast<uint2*>(sR + L::at(t, pos)) = make_uint2(rk[i].w[2 * u], rk[i].w[2 * u + 1]);
        }
      }
#pragma unroll
      for (int m = 0; m < CPT / 2; ++m) {
        const uint32_t lo01 = __builtin_amdgcn_perm(rk[1].w[m], rk[0].w[m], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(rk[3].w[m], rk[2].w[m], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(rk[1].w[m], rk[0].w[m], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(rk[3].w[m], rk[2].w[m], 0x07060302u);
        *reinterpret_cast<uint2*>(sKt + (ch0 + 2 * m) * L::CP + sig(4 * tg)) = make_uint2(lo01, lo23);
        *reinterpret_cast<uint2*>(sKt + (ch0 + 2 * m + 1) * L::CP + sig(4 * tg)) = make_uint2(hi01, hi23);
      }
      return;
    }
    float kh[4][CPT];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float qv[CPT], kv[CPT], bv[CPT];
      unpack<T, CPT>(rq[i], qv);
      unpack<T, CPT>(rk[i], kv);
      if constexpr (CHANNEL) {
        unpack<GT, CPT>(rb[i], bv);
      } else {
        const float beta = word_f32<GT>(ub[i]);
#pragma unroll
        for (int e = 0; e < CPT; ++e) bv[e] = beta;
      }
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        const float e1 = HAS_G ? exp2_fast(X2[i][e]) : 1.f;
        const float e2 = HAS_G ? exp2_fast(-X2[i][e]) : 1.f;
        bv[e] = -(bv[e] * kv[e]) * e1;          // Ln = -e exp(G - r)
        qv[e] = qv[e] * e1;                     // M  =  q exp(G - r)
        kv[e] = kv[e] * e2;                     // R  =  k exp(r - G)
        kh[i][e] = HAS_G ? kv[e] * cC[e] : kv[e];  // K_hat = k exp(G_C - G)
      }
      const int t = 4 * tg + i;
#pragma unroll
      for (int u = 0; u < CPT / 4; ++u) {
        const int pos = sig(ch0 + 4 * u);
        st4<T>(sLn + L::at(t, pos), bv[4 * u], bv[4 * u + 1], bv[4 * u + 2], bv[4 * u + 3]);
        st4<T>(sM + L::at(t, pos), qv[4 * u], qv[4 * u + 1], qv[4 * u + 2], qv[4 * u + 3]);
        st4<T>(sR + L::at(t, pos), kv[4 * u], kv[4 * u + 1], kv[4 * u + 2], kv[4 * u + 3]);
      }
    }
#pragma unroll
    for (int e = 0; e < CPT; ++e)
      st4<T>(sKt + (ch0 + e) * L::CP + sig(4 * tg), kh[0][e], kh[1][e], kh[2][e], kh[3][e]);
  };

  // Diagonal block pw of A and its inverse (producer interval 2).  With
  // N = -A (strictly lower, so N^16 = 0),
  //   (I + A)^{-1} = I + N + ... + N^15 = (I + N)(I + N^2)(I + N^4)(I + N^8),
  // four levels of 16x16 products on the fp32 MFMA instead of a 16-step
  // substitution.  Fragment layouts (lane = 16 g + j):
  //   row form  rowL(X): X[j][4g + i]   (A operand of mma16)
  //   acc form  accL(X): X[4g + i][j]   (B operand and result of mma16)
  // mma16(acc, rowL(X), accL(Y)) adds accL(X Y); accL(X) = rowL(X^T).
  auto diag_inverse = [&](int slot) {
    Frag4<float> nr, nc;
    if constexpr (CHANNEL) {
      f32x4 nrow = {0.f, 0.f, 0.f, 0.f}, ncol = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const Frag8<T> a = ld_frag8<T>(sR + L::at(16 * pw + j, 32 * kb + 8 * g));
        const Frag8<T> b = ld_frag8<T>(sLn + L::at(16 * pw + j, 32 * kb + 8 * g));
        mma32(nrow, a, b);  // [4g+i][j] of R Ln^T = N[j][4g+i]
        mma32(ncol, b, a);  // [4g+i][j] of Ln R^T = N[4g+i][j]
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        nr.v[i] = (4 * g + i < j) ? nrow[i] : 0.f;  // rowL(N)
        nc.v[i] = (j < 4 * g + i) ? ncol[i] : 0.f;  // accL(N)
      }
    } else {
      // K K^T is symmetric: one product gives both orientations; the mask
      // -beta_t exp(G_t - G_s) = FNB[t] FE2[s] makes N[t][s] = -A[t][s].
      const float* tok = sTok0 + slot * 8 * kC;
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const Frag8<T> a = ld_frag8<T>(sR + L::at(16 * pw + j, 32 * kb + 8 * g));
        mma32(d, a, a);  // [4g+i][j] = k_(16pw+4g+i) . k_(16pw+j)
      }
      const float4 nb4 = *reinterpret_cast<const float4*>(tok + kFNB * kC + 16 * pw + 4 * g);
      const float4 e24 = *reinterpret_cast<const float4*>(tok + kFE2 * kC + 16 * pw + 4 * g);
      const float nbj = tok[kFNB * kC + 16 * pw + j];
      const float e2j = tok[kFE2 * kC + 16 * pw + j];
      const float nbv[4] = {nb4.x, nb4.y, nb4.z, nb4.w};
      const float e2v[4] = {e24.x, e24.y, e24.z, e24.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        nr.v[i] = (4 * g + i < j) ? nbj * e2v[i] * d[i] : 0.f;
        nc.v[i] = (j < 4 * g + i) ? nbv[i] * e2j * d[i] : 0.f;
      }
    }
    auto prod = [](const Frag4<float>& x, const Frag4<float>& y) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      mma16(acc, x, y);
      Frag4<float> f;
#pragma unroll
      for (int i = 0; i < 4; ++i) f.v[i] = acc[i];
      return f;
    };
    const Frag4<float> n2c = prod(nr, nc);    // accL(N^2)
    const Frag4<float> n2r = prod(nc, nr);    // rowL(N^2) = accL(N^T N^T)
    const Frag4<float> n4c = prod(n2r, n2c);  // accL(N^4)
    const Frag4<float> n4r = prod(n2c, n2r);  // rowL(N^4)
    const Frag4<float> n8c = prod(n4r, n4c);  // accL(N^8)
    // accL(T^T), T^T = (I + N^8)^T (I + N^4)^T (I + N^2)^T (I + N)^T, built
    // by left products starting from accL((I + N)^T) = rowL(I + N).
    Frag4<float> t;
#pragma unroll
    for (int i = 0; i < 4; ++i) t.v[i] = nr.v[i] + ((4 * g + i == j) ? 1.f : 0.f);
    auto step = [](const Frag4<float>& x, const Frag4<float>& c) {  // accL(C + X C), x = rowL(X)
      f32x4 acc = {c.v[0], c.v[1], c.v[2], c.v[3]};
      mma16(acc, x, c);
      Frag4<float> f;
#pragma unroll
      for (int i = 0; i < 4; ++i) f.v[i] = acc[i];
      return f;
    };
    t = step(n2c, t);  // rowL((N^2)^T) = accL(N^2)
    t = step(n4c, t);
    t = step(n8c, t);
    // t = accL(T^T) = rowL(T): lane (g, j) holds T[j][4g .. 4g+3]
    st4<T>(sTd + (pw * 16 + j) * L::TDP + 4 * g, t.v[0], t.v[1], t.v[2], t.v[3]);
  };

  // =====================================================================
  // Consumer side (waves 0-3): the state slice S[16mt + 4g + i][col],
  // col = c0 + 16 * wave + j, in accumulator layout.
  // =====================================================================
  const int col = c0 + 16 * wave + j;
  f32x4 S[MT], X[4], O[4];
  if (consumer) {
    const float* sin = p.state_in ? p.state_in + head * (int64_t)DK * DV : nullptr;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[mt][i] = sin ? sin[(16 * mt + 4 * g + i) * DV + col] : 0.f;
  }

  // X = Z + Ln S~ (= Z - E_bar S), O^T = S~^T M^T (= (Q_bar S)^T), and the
  // Gram tiles of this wave w: P(ms = w, nt = n) for n >= w and
  // A(ms = n, nt = w) for n < w (four tiles per wave, ten P and six
  // off-diagonal A tiles in all), sharing the operand fragment loads.
  auto consume_first = [&](int slot, auto wave_tag) {
    constexpr int w = decltype(wave_tag)::value;  // == wave
    const float* sR2 = sVec0 + slot * 2 * DK;
    const float* sZ = sZ0 + slot * (L::kZSz / 4);
    Frag8<T> sf[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f32x4 lo = S[2 * kb], hi = S[2 * kb + 1];
      if constexpr (HAS_G && CHANNEL) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lo[i] *= sR2[32 * kb + 4 * g + i];
          hi[i] *= sR2[32 * kb + 16 + 4 * g + i];
        }
      }
      sf[kb] = frag8_from_acc<T>(lo, hi);
    }
    f32x4 tacc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if constexpr (CHANNEL) {
        const float4 z = *reinterpret_cast<const float4*>(sZ + (16 * wave + j) * L::ZP + 16 * mt + 4 * g);
        X[mt][0] = z.x; X[mt][1] = z.y; X[mt][2] = z.z; X[mt][3] = z.w;
      } else {
        X[mt] = f32x4{0.f, 0.f, 0.f, 0.f};  // K S first, then Z + diag(FX) K S
      }
      O[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      tacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // scalar gates: L is raw k (sR) and the decay is applied afterwards
    const T* sL = CHANNEL ? sLn : sR;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      Frag8<T> ln[4], mm[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        ln[mt] = ld_frag8<T>(sL + L::at(16 * mt + j, 32 * kb + 8 * g));
        mm[mt] = ld_frag8<T>(sM + L::at(16 * mt + j, 32 * kb + 8 * g));
      }
      // Gram operands: with scalar gates L is raw k, so R(w) and R(n) are
      // the L fragments already loaded; Ln(w) is always ln[w]
      const Frag8<T> rw = CHANNEL ? ld_frag8<T>(sR + L::at(16 * w + j, 32 * kb + 8 * g)) : ln[w];
      const Frag8<T> lw = ln[w];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        mma32(X[mt], ln[mt], sf[kb]);
        mma32(O[mt], sf[kb], mm[mt]);
      }
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        if (n >= w) {
          mma32(tacc[n], rw, mm[n]);
        } else {
          const Frag8<T> rn = CHANNEL ? ld_frag8<T>(sR + L::at(16 * n + j, 32 * kb + 8 * g)) : ln[n];
          mma32(tacc[n], rn, lw);
        }
      }
    }
    if constexpr (!CHANNEL) {
      // keep the factor loads below out of the MFMA loop (register budget)
      __builtin_amdgcn_sched_barrier(0);
      const float* tok = sTok0 + slot * 8 * kC;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const float4 z = *reinterpret_cast<const float4*>(sZ + (16 * wave + j) * L::ZP + 16 * mt + 4 * g);
        const float4 fx = *reinterpret_cast<const float4*>(tok + kFX * kC + 16 * mt + 4 * g);
        const float fo = tok[kFO * kC + 16 * mt + j];  // O^T: token 16 mt + j of this lane
        X[mt][0] = fmaf(fx.x, X[mt][0], z.x); X[mt][1] = fmaf(fx.y, X[mt][1], z.y);
        X[mt][2] = fmaf(fx.z, X[mt][2], z.z); X[mt][3] = fmaf(fx.w, X[mt][3], z.w);
#pragma unroll
        for (int i = 0; i < 4; ++i) O[mt][i] *= fo;
      }
      // Gram masks: P[t][s] *= FE1[t] FE2[s], -A[t][s] = FNB[t] FE2[s] (k_t . k_s)
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int t = (n >= w) ? 16 * n + j : 16 * w + j;
        const int s0 = (n >= w) ? 16 * w + 4 * g : 16 * n + 4 * g;
        const float ft = tok[((n >= w) ? kFE1 : kFNB) * kC + t];
        const float4 fs = *reinterpret_cast<const float4*>(tok + kFE2 * kC + s0);
        tacc[n][0] *= ft * fs.x; tacc[n][1] *= ft * fs.y;
        tacc[n][2] *= ft * fs.z; tacc[n][3] *= ft * fs.w;
      }
    }
    // tacc[n][i] = D[s][t]: P tiles s = 16w + 4g + i, t = 16n + j;
    //                       A tiles s = 16n + 4g + i, t = 16w + j (= -A[t][s])
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      if (n >= w) {
        const int t = 16 * n + j;
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = (16 * w + 4 * g + i <= t) ? tacc[n][i] : 0.f;
        st4<T>(sP + t * L::CP + sig(16 * w + 4 * g), pv[0], pv[1], pv[2], pv[3]);
        if (n == w && (w & 1) == 0)  // the causal product reads whole 32-token blocks
          st4<T>(sP + t * L::CP + sig(16 * (w + 1) + 4 * g), 0.f, 0.f, 0.f, 0.f);
      } else {
        const int t = 16 * w + j;
        st4<T>(sAo + t * L::CP + 16 * n + 4 * g, tacc[n][0], tacc[n][1], tacc[n][2], tacc[n][3]);
      }
    }
  };

  // U = (I + A)^{-1} X, O^T += U^T P^T, S' = Diag(exp(G_C)) S + K_hat^T U, store o.
  auto consume_second = [&](int64_t ci) {
    const int slot = (int)(ci & 1);
    const T* sKt = sKt0 + slot * (L::kKtSz / L::ES);
    const float* sGC = sVec0 + slot * 2 * DK + DK;
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
    // state update operand: U itself (channel gates, K_hat^T holds the
    // decay) or diag(FK) U with raw k^T (scalar gates)
    Frag8<T> uk[2] = {u8[0], u8[1]};
    float gC = 1.f;
    if constexpr (!CHANNEL) {
      const float* tok = sTok0 + slot * 8 * kC;
      f32x4 us[4];
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        const float4 fk = *reinterpret_cast<const float4*>(tok + kFK * kC + 16 * bi + 4 * g);
        us[bi] = f32x4{U[bi][0] * fk.x, U[bi][1] * fk.y, U[bi][2] * fk.z, U[bi][3] * fk.w};
      }
      uk[0] = frag8_from_acc<T>(us[0], us[1]);
      uk[1] = frag8_from_acc<T>(us[2], us[3]);
      gC = tok[kFG * kC];
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        if (32 * kb <= 16 * nt + 15) {
          const Frag8<T> bp = ld_frag8<T>(sP + (16 * nt + j) * L::CP + 32 * kb + 8 * g);
          mma32(O[nt], u8[kb], bp);
        }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if constexpr (HAS_G && CHANNEL) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[mt][i] *= sGC[16 * mt + 4 * g + i];
      } else if constexpr (HAS_G) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[mt][i] *= gC;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const Frag8<T> a = ld_frag8<T>(sKt + (16 * mt + j) * L::CP + 32 * kb + 8 * g);
        mma32(S[mt], a, uk[kb]);
      }
    }
    const int64_t t0 = ci * kC;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t tok = t0 + 16 * nt + j;
      if (tok < Tn) {
        T* dst = go + ((tok0 + tok) * p.Hv + hv) * (int64_t)DV + c0 + 16 * wave + 4 * g;
        st4<T>(dst, p.scale * O[nt][0], p.scale * O[nt][1], p.scale * O[nt][2], p.scale * O[nt][3]);
      }
    }
  };

  // Exact token-by-token recurrence for one chunk, straight from global
  // memory (chunks whose decay range the factored form cannot represent).
  auto consume_tokens = [&](int64_t ci) {
    const int64_t t0 = ci * kC;
    for (int tl = 0; tl < kC; ++tl) {
      const int64_t tok = t0 + tl;
      if (tok >= Tn) break;
      const int64_t qk_off = ((tok0 + tok) * p.Hk + hk) * (int64_t)DK;
      const int64_t gt = (tok0 + tok) * p.Hv + hv;
      float sbeta = 0.f, salpha = 1.f;
      if constexpr (!CHANNEL) {
        sbeta = to_f32(gb[gt]);
        if constexpr (HAS_G) salpha = exp2_fast(to_f32(gg[gt]) * kLog2e);
      }
      float rp = 0.f;
      float kr[MT][4], qr[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = 16 * mt + 4 * g;
        float er[4], ar[4];
        load_f32<4, T>(gk + qk_off + row, kr[mt]);
        load_f32<4, T>(gq + qk_off + row, qr[mt]);
        if constexpr (CHANNEL) {
          load_f32<4, GT>(gb + gt * DK + row, er);
          if constexpr (HAS_G) {
            load_f32<4, GT>(gg + gt * DK + row, ar);
#pragma unroll
            for (int i = 0; i < 4; ++i) ar[i] = exp2_fast(ar[i] * kLog2e);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) ar[i] = 1.f;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) { er[i] = sbeta; ar[i] = salpha; }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          S[mt][i] *= ar[i];
          rp += er[i] * kr[mt][i] * S[mt][i];
        }
      }
      rp += __shfl_xor(rp, 16);
      rp += __shfl_xor(rp, 32);
      float z = to_f32(gv[gt * DV + col]);
      if constexpr (CHANNEL) z *= to_f32(gw[gt * DV + col]);
      else z *= sbeta;
      const float d = z - rp;
      float op = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          S[mt][i] += kr[mt][i] * d;
          op += qr[mt][i] * S[mt][i];
        }
      op += __shfl_xor(op, 16);
      op += __shfl_xor(op, 32);
      if (g == 0) go[gt * DV + col] = from_f32<T>(p.scale * op);
    }
  };

  // The two roles run separate loops with the same barrier sequence (one
  // before the first chunk, two per chunk), so that each role's registers are
  // allocated for its own live values only.
  if (consumer) {
    __syncthreads();  // operands of chunk 0 are ready
    for (int64_t ci = 0; ci < nchunks; ++ci) {
      const int slot = (int)(ci & 1);
      const bool slow = (sFlag[slot * 4] | sFlag[slot * 4 + 1] | sFlag[slot * 4 + 2] |
                         sFlag[slot * 4 + 3]) != 0;
      if (slow) {
        consume_tokens(ci);
      } else {
        // one instantiation per wave, so the tile choice is resolved at
        // compile time and the MFMA sequence has no branches
        switch (wave) {
          case 0: consume_first(slot, IntTag<0>{}); break;
          case 1: consume_first(slot, IntTag<1>{}); break;
          case 2: consume_first(slot, IntTag<2>{}); break;
          default: consume_first(slot, IntTag<3>{}); break;
        }
      }
      __syncthreads();  // barrier A
      if (!slow) consume_second(ci);
      __syncthreads();  // barrier B
    }
    if (p.state_out) {
      float* sout = p.state_out + head * (int64_t)DK * DV;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sout[(16 * mt + 4 * g + i) * DV + col] = S[mt][i];
    }
  } else {
    // (nchunks >= 1 here.  The prologue stays unconditional: loads issued
    // under a branch would leave the compiler unsure of the outstanding
    // loads at the loop head, and its waits there would drain them.)
    load_gvw(0);
    load_qkb(0);
    produce_decay(0);
    produce_operands(0);
    load_gvw(nchunks > 1 ? kC : 0);
    load_qkb(nchunks > 1 ? kC : 0);
    __syncthreads();
    // The prefetch of chunk ci + 2 is issued on every iteration (the last
    // two re-read the final chunk): with a fixed number of loads in flight
    // the wait for the older half of the registers does not drain the
    // younger loads, whose latency would otherwise be exposed.
    for (int64_t ci = 0; ci < nchunks; ++ci) {
      const int slot = (int)(ci & 1);
      const bool slow = (sFlag[slot * 4] | sFlag[slot * 4 + 1] | sFlag[slot * 4 + 2] |
                         sFlag[slot * 4 + 3]) != 0;
      const int64_t pre = (ci + 2 < nchunks ? ci + 2 : nchunks - 1) * kC;
      if (!slow) diag_inverse(slot);
      if (ci + 1 < nchunks) produce_decay(ci + 1);
      load_gvw(pre);
      __syncthreads();  // barrier A
      if (ci + 1 < nchunks) produce_operands(ci + 1);
      load_qkb(pre);
      __syncthreads();  // barrier B
    }
  }
}

template <typename T, typename GT, int DK, int DV, bool CH, bool HG>
hipError_t launch_pipe_typed(const ChunkArgs& a, hipStream_t stream) {
  Params p;
  p.B = a.B; p.T = a.T; p.cu = a.cu_seqlens; p.Hk = a.Hk; p.Hv = a.Hv; p.scale = a.scale;
  p.q = a.q; p.k = a.k; p.v = a.v; p.b = a.b; p.w = a.w; p.g = a.g;
  p.state_in = a.state_in; p.state_out = a.state_out; p.o = a.o;
  const int64_t nwg = a.B * a.Hv * (DV / 64);
  chunk_fwd_pipe_kernel<T, GT, DK, DV, 64, CH, HG><<<dim3((unsigned)nwg), dim3(kPipeThreads), 0, stream>>>(p);
  return hipGetLastError();
}

template <typename GT, int DK, int DV>
hipError_t pipe_gates(const ChunkArgs& a, hipStream_t s) {
  const bool hg = a.g != nullptr;
  if (a.channel) return hg ? launch_pipe_typed<bf16, GT, DK, DV, true, true>(a, s)
                           : launch_pipe_typed<bf16, GT, DK, DV, true, false>(a, s);
  return hg ? launch_pipe_typed<bf16, GT, DK, DV, false, true>(a, s)
            : launch_pipe_typed<bf16, GT, DK, DV, false, false>(a, s);
}

template <typename GT>
hipError_t pipe_dims(const ChunkArgs& a, hipStream_t s) {
  if (a.dk == 128 && a.dv == 128) return pipe_gates<GT, 128, 128>(a, s);
  if (a.dk == 128 && a.dv == 64) return pipe_gates<GT, 128, 64>(a, s);
  if (a.dk == 64 && a.dv == 128) return pipe_gates<GT, 64, 128>(a, s);
  return pipe_gates<GT, 64, 64>(a, s);
}

}  // namespace

// bf16 operands: producer/consumer kernel.
hipError_t launch_chunk_fwd_pipe(const ChunkArgs& a, hipStream_t stream) {
  if (a.gate == DType::F32) return pipe_dims<float>(a, stream);
  return pipe_dims<bf16>(a, stream);
}

}  // namespace gdn
