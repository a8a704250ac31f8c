// chunk_fwd_sb.hip -- chunkwise forward on bf16 MFMA operands, each 64-token
// chunk solved in four 16-token sub-blocks.
//
// Method ("Gated DeltaNet-2", Methodologie §3 "Entrainement Parallele Efficace
// par Blocs"; "Gated DeltaNet", §Rendre l'entrainement parallele).  Inside a
// chunk of C = 64 tokens the unit lower-triangular system (I + A) U = Z - E S
// is solved by block forward substitution over four 16x16 diagonal blocks.
// The off-diagonal blocks A_bb' (b' < b) are applied in factored form through
// the running state: with S_b the state entering sub-block b and G the
// cumulative log-decay counted from the first token of the sub-block,
//
//   X_b     = Z_b + Ln_b S_b          Ln_t = -(b_t (.) k_t) exp(G_t)
//   U_b     = (I + A_bb)^{-1} X_b
//   O_b     = Qb_b S_b + P_bb U_b     Qb_t = q_t (.) exp(G_t)
//   S_{b+1} = Diag(exp(G_15)) S_b + Kh_b^T U_b,   Kh_s = k_s (.) exp(G_15 - G_s)
//
// which is the chunk's block substitution (A_bb' U_b' enters through
// Ln_b S_b).  For alpha <= 1 every exponential above is at most 1, so the
// state-side operands never overflow however strong the decay.
//
// Inside a diagonal block, A[t,s] = sum_c e_t,c k_s,c exp(G_t,c - G_s,c)
// (s < t) and P[t,s] (s <= t) are MFMA products of factored operands around
// one reference per channel, the cumulative log-decay at the block's middle
// token (m = G_7), so a factor spans at most eight tokens of decay:
//   L = -e exp(G - m),  M = q exp(G - m),  R = k exp(m - G)
// and A = L R^T, P = M R^T below the diagonal (each product there is
// exp(G_t - G_s) <= 1 times the operands; the products above it are never
// used).  The factors must stay finite: a sub-block whose decays put some
// |G - m| above kRange (log2 units) is redone with every per-token decay
// raised to at least 2^-kFloor.  A term that crosses such a token then
// carries 2^-kFloor = 2^-13 in place of a smaller true factor, a change of at
// most 2^-13 of its undecayed size, well under the rounding of the bf16
// operands (2^-9).  Floored, eight tokens span at most 104 < kRange, so the
// retry always fits when alpha <= 1; only a rising state (alpha > 1) can
// still leave the range, and such a sub-block runs the exact token
// recurrence.
//
// With scalar gates (Gated DeltaNet, DeltaNet) the decay factors out of the
// Gram matrices exactly: A[t,s] = beta_t exp(G_t - G_s) (k_t . k_s), applied
// as an element-wise mask, and as row scales of K S, Q S and U, so the
// operands are the raw q and k and no sub-block ever leaves the MFMA path
// when alpha <= 1.
//
// Workgroup: 512 threads per (sequence, value head, 64 columns of d_v).
//   Consumer waves 0-3 own 16 state columns each (all d_k rows, fp32, in MFMA
//     accumulator registers for the whole sequence) and walk the sub-blocks.
//   Producer wave 4 + p prepares sub-block p of the next chunk on its own:
//     loads, decay prefix, gated operands, the 16x16 Gram blocks, the inverse
//     (I + A_bb)^{-1} and the flags.  Nothing crosses producer waves, so
//     one workgroup barrier per chunk hands a whole chunk over.
// State rows in registers: accumulator tile 2kb + h, row 4g + i holds channel
// 32kb + 8g + 4h + i.  With that order the B fragment of a 32-channel block
// is 8 consecutive channels per lane, so every operand is stored with its
// channels in natural order: X and O read 16-byte fragments, and the state
// update reads Kh^T with the gfx950 transposing LDS read (ds_read_b64_tr_b16).
#include "chunk_common.hpp"

namespace gdn {
namespace {

template <int N>
struct IntTag {
  static constexpr int value = N;
};

constexpr int kSB = 16;           // tokens per sub-block
constexpr int kRankMax = 256;     // packed sequences ranked by length in the kernel
constexpr int kSbThreads = 512;   // 4 consumer + 4 producer waves
constexpr float kRange = 110.f;   // largest |G - m| (log2) of the factored form
constexpr float kFloor = 13.f;    // per-token decay floor (log2) of the second scan
static_assert(8.f * kFloor <= kRange, "a floored sub-block fits the factored form");

// One [16][DK] bf16 operand block.  Rows are DK contiguous channels in
// 16-byte chunks of 8; the chunks of a row are XOR-permuted by the row, in
// one of three placements, each chosen for the LDS accesses that touch the
// block (on gfx950, measured with the bank-conflict counter; for DK = 128):
//   ax:  chunk ^ r.  Fragment reads (lane 16 g + j: row j, chunk 4 kb + g)
//        and stores of that shape are conflict free.
//   at:  chunk ^ s(r), s(4x + y) = 4 (x ^ y) + x.  Row-quad stores (lane
//        4 cg + qd: row 4 qd + i, chunk cg) are conflict free.
//   ath: at, with the two 8-byte halves of each chunk exchanged in rows
//        4..7 and 12..15; the transposing reads (lane 16 g + j: row
//        4 g + j / 4, a half chunk) are then conflict free.
// DK = 64 (two rows per bank period) keeps one placement, chunk ^ (r/2) % 8.
template <int DK>
struct Blk {
  static constexpr int NCH = DK / 8;
  static constexpr int BYTES = 16 * DK * 2;
  static constexpr bool kWide = NCH >= 16;
  __host__ __device__ static constexpr int sw(int r) {
    if constexpr (kWide) return 4 * ((r >> 2) ^ (r & 3)) + (r >> 2);
    else return (r >> 1) % NCH;
  }
  __host__ __device__ static constexpr int at(int r, int c) {
    return r * DK + ((((c >> 3) ^ sw(r))) << 3) + (c & 7);
  }
  __host__ __device__ static constexpr int ax(int r, int c) {
    if constexpr (kWide) return r * DK + ((((c >> 3) ^ r)) << 3) + (c & 7);
    else return at(r, c);
  }
  __host__ __device__ static constexpr int ath(int r, int c) {
    if constexpr (kWide) return at(r, c) ^ (((r >> 2) & 1) << 2);
    else return at(r, c);
  }
  // does row r hold its chunks' halves exchanged (ath)?
  __host__ __device__ static constexpr bool half_swapped(int r) { return kWide && ((r >> 2) & 1); }
};

// Element (r, c) of a [64][64] bf16 tile of v or o rows (token r, column c
// of the workgroup's slice): the 32-byte column segments of a row are
// XOR-permuted by r / 2, so that accesses of 4 rows x 16 columns (the
// transposing reads of v, the output fragments) spread over the banks.
__host__ __device__ constexpr int vo_at(int r, int c) {
  return r * 64 + (((c >> 4) ^ ((r >> 1) & 3)) << 4) + (c & 15);
}

// Element (r, c) of a 16x16 bf16 block (T, P), read and written as four
// consecutive columns per lane: the 4-column group is XOR-permuted by r / 4
// (conflict-free 8-byte accesses for lane 16 g + j at row j, group g).
__host__ __device__ constexpr int tp_at(int r, int c) {
  return r * 16 + (((c >> 2) ^ ((r >> 2) & 3)) << 2) + (c & 3);
}

// Compile-time check of a placement: every (row, column) of a ROWS x COLS
// block lands inside the block, on an element of its own (a permutation), so
// no access through it can leave its LDS block or alias another element.
template <int ROWS, int COLS, typename F>
constexpr bool is_permutation(F f) {
  bool seen[ROWS * COLS] = {};
  for (int r = 0; r < ROWS; ++r)
    for (int c = 0; c < COLS; ++c) {
      const int o = f(r, c);
      if (o < 0 || o >= ROWS * COLS || seen[o]) return false;
      seen[o] = true;
    }
  return true;
}
template <int DK>
constexpr bool blk_placements_ok() {
  using B = Blk<DK>;
  return is_permutation<16, DK>([](int r, int c) { return B::at(r, c); }) &&
         is_permutation<16, DK>([](int r, int c) { return B::ax(r, c); }) &&
         is_permutation<16, DK>([](int r, int c) { return B::ath(r, c); });
}
static_assert(blk_placements_ok<64>() && blk_placements_ok<128>(), "operand block placements");
static_assert(is_permutation<64, 64>([](int r, int c) { return vo_at(r, c); }), "v/o tile placement");
static_assert(is_permutation<16, 16>([](int r, int c) { return tp_at(r, c); }), "T/P block placement");

template <int DK, bool CHANNEL>
struct SbLds {
  static constexpr int NOPS = 3;                 // Ln|k, Qb|q, Kh|k (transposing placement)
  static constexpr int BLK = Blk<DK>::BYTES;
  static constexpr int TPB = 16 * 16 * 2;       // one 16x16 bf16 block
  static constexpr int kOps = 0;                 // [NOPS][4 sub-blocks] blocks
  static constexpr int kT = kOps + NOPS * 4 * BLK;
  static constexpr int kP = kT + 4 * TPB;
  static constexpr int kVec = kP + 4 * TPB;      // channel: D [4][DK]; scalar: [4][6][16]
  static constexpr int VEC = CHANNEL ? 4 * DK * 4 : 4 * 6 * 16 * 4;
  static constexpr int kFlag = kVec + VEC;
  // scalar gates: the v rows and the o rows of the chunk's 64 tokens for the
  // workgroup's 64 columns, [64][64] bf16 each
  static constexpr int VO = CHANNEL ? 0 : 64 * 64 * 2;
  static constexpr int kVt = kFlag + 16;
  static constexpr int kOt = kVt + VO;
  static constexpr int SLOT = kOt + VO;
  static constexpr int kPriv = 2 * SLOT;         // channel: per producer wave L, M, R
  static constexpr int PRIV = CHANNEL ? 3 * BLK : 0;
  static constexpr int kTotal = kPriv + 4 * PRIV;
  static_assert(kTotal <= 160 * 1024, "LDS budget");
  // every region starts 16-byte aligned (whole-chunk accesses) and ends
  // before the next begins
  static_assert(kOps % 16 == 0 && kT % 16 == 0 && kP % 16 == 0 && kVec % 16 == 0 &&
                    kFlag % 16 == 0 && kVt % 16 == 0 && kOt % 16 == 0 && SLOT % 16 == 0 &&
                    kPriv % 16 == 0 && PRIV % 16 == 0,
                "LDS regions 16-byte aligned");
  static_assert(kOps + NOPS * 4 * BLK <= kT && kT + 4 * TPB <= kP && kP + 4 * TPB <= kVec &&
                    kVec + VEC <= kFlag && kFlag + 16 <= kVt && kVt + VO <= kOt &&
                    kOt + VO <= SLOT && 2 * SLOT <= kPriv,
                "LDS regions disjoint");
};

// Scalar-gate factor arrays of one sub-block, [6][16] floats.
constexpr int kFX = 0;    // -beta_t exp(G_t):   X = Z + diag(FX) K S
constexpr int kFO = 1;    // exp(G_t):           O = diag(FO) Q S + P U
constexpr int kFK = 2;    // exp(G_15 - G_t):    S' = D S + K^T diag(FK) U
constexpr int kFB = 3;    // beta_t:             Z = diag(beta) V
constexpr int kFG = 4;    // G_t (log2)
constexpr int kFD = 5;    // [0] = D = exp(G_15)

__device__ __forceinline__ float quad_perm(float x, int pat) {
  // every lane reads a lane of its own quad, so no lane keeps an old value
  int v = __builtin_bit_cast(int, x);
  int r;
  switch (pat) {
    case 0x00: r = __builtin_amdgcn_mov_dpp(v, 0x00, 0xf, 0xf, false); break;
    case 0x55: r = __builtin_amdgcn_mov_dpp(v, 0x55, 0xf, 0xf, false); break;
    case 0x90: r = __builtin_amdgcn_mov_dpp(v, 0x90, 0xf, 0xf, false); break;
    case 0x44: r = __builtin_amdgcn_mov_dpp(v, 0x44, 0xf, 0xf, false); break;
    case 0xAA: r = __builtin_amdgcn_mov_dpp(v, 0xAA, 0xf, 0xf, false); break;
    default: r = __builtin_amdgcn_mov_dpp(v, 0xFF, 0xf, 0xf, false); break;
  }
  return __builtin_bit_cast(float, r);
}

// Row shift right by n inside 16-lane rows; lanes shifted in take +inf.
__device__ __forceinline__ float dpp_row_shr_inf(float x, int n) {
  const int inf = 0x7f800000;
  int v = __builtin_bit_cast(int, x);
  int r;
  switch (n) {
    case 1: r = __builtin_amdgcn_update_dpp(inf, v, 0x111, 0xf, 0xf, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(inf, v, 0x112, 0xf, 0xf, false); break;
    case 4: r = __builtin_amdgcn_update_dpp(inf, v, 0x114, 0xf, 0xf, false); break;
    default: r = __builtin_amdgcn_update_dpp(inf, v, 0x118, 0xf, 0xf, false); break;
  }
  return __builtin_bit_cast(float, r);
}

// Two fp32 values rounded to bf16 (nearest even) in one 32-bit word.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 h = {(bf16)a, (bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// N packed words to LDS in one store (16 or 8 bytes).
template <int N>
__device__ __forceinline__ void st_words(bf16* p, const uint32_t* w) {
  lds_check(p, 4 * N);
  if constexpr (N == 4) *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  else *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
}

typedef short sb_v4s __attribute__((ext_vector_type(4)));

// Four 16-bit elements of one row read transposed: within each 16-lane group
// the lanes' 8-byte reads of 4 rows x 16 columns come back as lane l holding
// column l of the 4 rows.
__device__ __forceinline__ Frag4<bf16> ld_tr16(const bf16* p) {
  lds_check(p, 8);
  const sb_v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) sb_v4s*)(p));
  Frag4<bf16> f;
  f.v = __builtin_bit_cast(bf16x4, r);
  return f;
}

// RAW: b, g and w are the raw gate projections (row strides p.ld_b, p.ld_g,
// p.ld_w) and the kernel applies the activations where it reads them:
// sigmoid for beta|b and w, the Mamba-2 log-decay for g.
// SAVE: also store each 16-token block's entry state and every u (p.ck, p.u).
template <typename GT, int DK, int DV, bool CHANNEL, bool HAS_G, bool RAW, bool SAVE>
__global__ __launch_bounds__(kSbThreads, 1) void chunk_fwd_sb_kernel(Params p) {
  using T = bf16;
  using L = SbLds<DK, CHANNEL>;
  using B = Blk<DK>;
  constexpr int DVS = 64;
  constexpr int NSPLIT = DV / DVS;
  constexpr int KB = DK / 32;
  constexpr int MT = DK / 16;
  constexpr int CPL = DK / 16;   // channels per producer lane (channel gates)
  constexpr int NSB = kC / kSB;  // 4

  __shared__ __attribute__((aligned(16))) char smem[L::kTotal];
  lds_nan_fill(smem, L::kTotal);

  const T* __restrict__ gq = static_cast<const T*>(p.q);
  const T* __restrict__ gk = static_cast<const T*>(p.k);
  const T* __restrict__ gv = static_cast<const T*>(p.v);
  const GT* __restrict__ gb = static_cast<const GT*>(p.b);
  const GT* __restrict__ gw = static_cast<const GT*>(p.w);
  const GT* __restrict__ gg = static_cast<const GT*>(p.g);
  T* __restrict__ go = static_cast<T*>(p.o);

  const int tid = threadIdx.x;
  // packed sequences: clamped token range of sequence n, so malformed offsets
  // stay inside the tensors
  auto seq_range = [&](int64_t n, int64_t& a0, int64_t& a1) {
    a0 = p.cu[n];
    a1 = p.cu[n + 1];
    a0 = a0 < 0 ? 0 : (a0 > p.T ? p.T : a0);
    a1 = a1 < a0 ? a0 : (a1 > p.T ? p.T : a1);
  };
  // Workgroup -> (sequence, value head, d_v slice).  Equal-length sequences:
  // XCD-aware (workgroup i runs on XCD i % 8; the slices of one head, and
  // the value heads that share a key head, land on the same XCD and share its
  // L2).  Packed sequences: workgroups start in dispatch order with the
  // longest sequence first (ties by index), so that the short ones fill in
  // behind; the rank is computed here when there are at most kRankMax
  // sequences.  Within each run of 16 workgroups the two slices of a head
  // are 8 apart, so they too share an XCD while the order stays longest
  // first.
  const int64_t nwg = (int64_t)gridDim.x;
  int64_t lid = blockIdx.x;
  if (!p.cu && (nwg & 7) == 0) {
    lid = (lid & 7) * (nwg >> 3) + (lid >> 3);
  } else if (p.cu && NSPLIT == 2 && (nwg & 15) == 0) {
    const int64_t r = lid & 15;
    lid = (lid - r) + 2 * (r & 7) + (r >> 3);
  }
  const int64_t slot_head = lid / NSPLIT;
  const int split = (int)(lid - slot_head * NSPLIT);
  int64_t bidx = slot_head / p.Hv;
  const int hv = (int)(slot_head - bidx * p.Hv);
  if (p.cu && p.B <= kRankMax) {
    int* lens = reinterpret_cast<int*>(smem);   // LDS is free until the pipeline starts
    int* pick = lens + kRankMax;
    for (int n = tid; n < (int)p.B; n += (int)blockDim.x) {
      int64_t a0, a1;
      seq_range(n, a0, a1);
      lens[n] = (int)(a1 - a0);
    }
    __syncthreads();
    for (int n = tid; n < (int)p.B; n += (int)blockDim.x) {
      const int ln = lens[n];
      int rank = 0;
      for (int m = 0; m < (int)p.B; ++m) {
        const int lm = lens[m];
        rank += (lm > ln || (lm == ln && m < n)) ? 1 : 0;
      }
      if (rank == (int)bidx) *pick = n;   // exactly one sequence has each rank
    }
    __syncthreads();
    bidx = *pick;
    __syncthreads();
  }
  const int64_t head = bidx * p.Hv + hv;   // state index
  const int hk = hv / (p.Hv / p.Hk);
  const int c0 = split * DVS;
  int64_t tok0 = bidx * p.T, Tn = p.T;
  if (p.cu) {
    int64_t a0, a1;
    seq_range(bidx, a0, a1);
    tok0 = a0;
    Tn = a1 - a0;
  }
  const int64_t nchunks = (Tn + kC - 1) / kC;
  if (Tn == 0) {  // an empty sequence only passes its state through
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
  const int j = lane & 15;
  const int g = lane >> 4;

  // (the debug build checks every block index against the layout)
  auto opblk = [&](int slot, int op, int sb) -> T* {
    check_true(slot >= 0 && slot < 2 && op >= 0 && op < L::NOPS && sb >= 0 && sb < NSB);
    return reinterpret_cast<T*>(smem + slot * L::SLOT + L::kOps + (op * NSB + sb) * L::BLK);
  };
  auto tblk = [&](int slot, int sb) -> T* {
    check_true(slot >= 0 && slot < 2 && sb >= 0 && sb < NSB);
    return reinterpret_cast<T*>(smem + slot * L::SLOT + L::kT + sb * L::TPB);
  };
  auto pblk = [&](int slot, int sb) -> T* {
    check_true(slot >= 0 && slot < 2 && sb >= 0 && sb < NSB);
    return reinterpret_cast<T*>(smem + slot * L::SLOT + L::kP + sb * L::TPB);
  };
  auto vecp = [&](int slot) -> float* {
    check_true(slot >= 0 && slot < 2);
    return reinterpret_cast<float*>(smem + slot * L::SLOT + L::kVec);
  };
  auto flagp = [&](int slot) -> int* {
    check_true(slot >= 0 && slot < 2);
    return reinterpret_cast<int*>(smem + slot * L::SLOT + L::kFlag);
  };
  auto vtile = [&](int slot) -> T* {
    check_true(!CHANNEL && slot >= 0 && slot < 2);
    return reinterpret_cast<T*>(smem + slot * L::SLOT + L::kVt);
  };
  auto otile = [&](int slot) -> T* {
    check_true(!CHANNEL && slot >= 0 && slot < 2);
    return reinterpret_cast<T*>(smem + slot * L::SLOT + L::kOt);
  };
  const uint32_t v_tok = (uint32_t)(p.Hv * DV * 2);   // bytes per token of v (and o)

  const uint32_t qk_tok = (uint32_t)(p.Hk * DK * (int)sizeof(T));   // bytes per token
  // bytes per token of beta|b and of g (the projections' row strides when raw)
  const uint32_t gb_tok = RAW ? (uint32_t)(p.ld_b * (int64_t)sizeof(GT))
                              : (uint32_t)(p.Hv * (CHANNEL ? DK : 1) * (int)sizeof(GT));
  const uint32_t gg_tok = RAW ? (uint32_t)(p.ld_g * (int64_t)sizeof(GT)) : gb_tok;
  const char* bq = reinterpret_cast<const char*>(gq) + ((uint64_t)tok0 * qk_tok + (uint32_t)(hk * DK * (int)sizeof(T)));
  const char* bk = reinterpret_cast<const char*>(gk) + ((uint64_t)tok0 * qk_tok + (uint32_t)(hk * DK * (int)sizeof(T)));
  const char* bbc = reinterpret_cast<const char*>(gb) + ((uint64_t)tok0 * gb_tok + (uint32_t)(hv * DK * (int)sizeof(GT)));
  const char* bgc = reinterpret_cast<const char*>(gg) + ((uint64_t)tok0 * gg_tok + (uint32_t)(hv * DK * (int)sizeof(GT)));
  const char* bbs = reinterpret_cast<const char*>(gb) + ((uint64_t)tok0 * gb_tok + (uint32_t)(hv * (int)sizeof(GT)));
  const char* bgs = reinterpret_cast<const char*>(gg) + ((uint64_t)tok0 * gg_tok + (uint32_t)(hv * (int)sizeof(GT)));
  // raw gates: the gate projections' token offsets (rows of the exact path)
  auto gate_row = [&](int64_t tok, int64_t ld) -> int64_t { return (tok0 + tok) * ld; };

  if (wave >= 4) {
    if constexpr (!CHANNEL) __builtin_amdgcn_s_setprio(3);
    // =================================================================
    // Producer wave 4 + pw: sub-block pw of every chunk.
    // =================================================================
    const int pw = wave - 4;
    if constexpr (CHANNEL) {
      // lane = 4 cg + qd: tokens 4 qd .. 4 qd + 3 of the sub-block,
      // channels cg * CPL .. cg * CPL + CPL - 1
      const int qd = lane & 3;
      const int cg = lane >> 2;
      const int ch0 = cg * CPL;
      constexpr int QB = CPL * 2;
      constexpr int GB = CPL * (int)sizeof(GT);
      Raw<QB> rq[4], rk[4];
      Raw<GB> rb[4], rg[4];
      const uint32_t oq = (uint32_t)(ch0 * 2);
      const uint32_t og = (uint32_t)(ch0 * (int)sizeof(GT));
      // addressing: a wave-uniform 64-bit base per sub-block plus a per-lane
      // 32-bit offset.  A sub-block that is not whole (the last chunk; it may
      // even start past the end) clamps absolute token indices to the last
      // token instead.  load_tok issues token i's q, k and b (qkb) and/or g
      // (gg).  With bf16 gates each register is reloaded for the next chunk as
      // soon as its values have been consumed, so the loads have the element
      // work to land (measured: 7 % on the GDN-2 B8 shape).  With fp32 gates,
      // whose raw registers are twice as wide, only q and k reload early and b
      // and g after the element work (all four early spilled 60 VGPRs and took
      // 45 % longer; q and k early gained 3.6 %).
      auto load_tok = [&](int64_t ci, int i, bool qkb, bool gg) {
        const int64_t t0 = ci * kC + kSB * pw;          // first token of the sub-block
        if (t0 + kSB <= Tn) {                           // wave-uniform
          const uint64_t tu = (uint64_t)t0;
          const uint32_t tl = (uint32_t)(4 * qd + i);
          if (qkb) {
            ld_raw<QB>(bq + tu * qk_tok + (tl * qk_tok + oq), rq[i]);
            ld_raw<QB>(bk + tu * qk_tok + (tl * qk_tok + oq), rk[i]);
            ld_raw<GB>(bbc + tu * gb_tok + (tl * gb_tok + og), rb[i]);
          }
          if constexpr (HAS_G)
            if (gg) ld_raw<GB>(bgc + tu * gg_tok + (tl * gg_tok + og), rg[i]);
        } else {
          int64_t t = t0 + 4 * qd + i;
          t = t < Tn - 1 ? t : Tn - 1;
          const uint64_t tu = (uint64_t)t;
          if (qkb) {
            ld_raw<QB>(bq + (tu * qk_tok + oq), rq[i]);
            ld_raw<QB>(bk + (tu * qk_tok + oq), rk[i]);
            ld_raw<GB>(bbc + (tu * gb_tok + og), rb[i]);
          }
          if constexpr (HAS_G)
            if (gg) ld_raw<GB>(bgc + (tu * gg_tok + og), rg[i]);
        }
      };
      auto load = [&](int64_t ci) {
#pragma unroll
        for (int i = 0; i < 4; ++i) load_tok(ci, i, true, true);
      };
      constexpr bool kEarly = sizeof(GT) == 2;
      // fp32 gates: q and k of token i early, b and g after the element work
      auto load_qk_tok = [&](int64_t ci, int i) {
        const int64_t t0 = ci * kC + kSB * pw;
        int64_t t = t0 + 4 * qd + i;
        t = t < Tn - 1 ? t : Tn - 1;
        const uint64_t tu = (uint64_t)t;
        ld_raw<QB>(bq + (tu * qk_tok + oq), rq[i]);
        ld_raw<QB>(bk + (tu * qk_tok + oq), rk[i]);
      };
      auto load_bg = [&](int64_t ci) {
        const int64_t t0 = ci * kC + kSB * pw;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int64_t t = t0 + 4 * qd + i;
          t = t < Tn - 1 ? t : Tn - 1;
          const uint64_t tu = (uint64_t)t;
          ld_raw<GB>(bbc + (tu * gb_tok + og), rb[i]);
          if constexpr (HAS_G) ld_raw<GB>(bgc + (tu * gg_tok + og), rg[i]);
        }
      };
      // raw gates: A_log and dt_bias of the lane's channels (read where used)
      const float* pA = RAW && p.A_log ? p.A_log + hv * DK + ch0 : nullptr;
      const float* pD = RAW && p.dt_bias ? p.dt_bias + hv * DK + ch0 : nullptr;
      check_true(pw >= 0 && pw < 4);
      T* priv = reinterpret_cast<T*>(smem + L::kPriv + pw * L::PRIV);
      T* sL = priv;               // L (rows 0..15)
      T* sM = priv + 16 * DK;     // M
      T* sR = priv + 32 * DK;     // R

      auto produce = [&](int64_t ci) {
        const int slot = (int)(ci & 1);
        // absent tokens of a partial last chunk: q = k = b = 0, g = 0
        if (ci * kC + kSB * pw + kSB > Tn) {
          const int64_t tb = ci * kC + kSB * pw + 4 * qd;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tb + i >= Tn) {
              zero_raw(rq[i]); zero_raw(rk[i]); zero_raw(rb[i]);
              if constexpr (HAS_G) zero_raw(rg[i]);
            }
        }
        float* dvec = vecp(slot) + pw * DK + ch0;
        const bool partial = ci * kC + kSB * pw + kSB > Tn;   // wave-uniform
        const int64_t tq = ci * kC + kSB * pw + 4 * qd;       // first token of the lane
        (void)tq;
        float G[4][CPL], fln[CPL], fkh[CPL];
        float worst;
        // cumulative log2-decay over the sub-block (4 tokens in-thread, then
        // an exclusive scan over the 4 token quads of the lane quad), the
        // references and factors, and the largest exponent the factored form
        // would meet.  Pass 0 takes the exact decays; a sub-block they put out
        // of range is scanned again with each per-token decay raised to at
        // least 2^-kFloor.  One that still fails (a rising state) keeps its
        // flag and runs the exact recurrence.
        auto scan = [&](const bool floored) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (HAS_G) {
              unpack<GT, CPL>(rg[i], G[i]);
              if constexpr (RAW) {
                // the decay of an absent token must stay 1 (g = 0)
                const bool here = !partial || tq + i < Tn;
#pragma unroll
                for (int e = 0; e < CPL; ++e) {
                  const float nA = neg_exp_f(pA ? pA[e] : 0.f), dt = pD ? pD[e] : 0.f;
                  G[i][e] = here ? log_decay_f(G[i][e], nA, dt) : 0.f;
                }
              }
            } else {
#pragma unroll
              for (int e = 0; e < CPL; ++e) G[i][e] = 0.f;
            }
          }
          worst = 0.f;
#pragma unroll
          for (int e = 0; e < CPL; ++e) {
            if (!floored) {
              G[0][e] *= kLog2e;
#pragma unroll
              for (int i = 1; i < 4; ++i) G[i][e] = fmaf(G[i][e], kLog2e, G[i - 1][e]);
            } else {
              float acc = 0.f;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float lg = G[i][e] * kLog2e;
                acc += lg < -kFloor ? -kFloor : lg;   // (a NaN stays NaN)
                G[i][e] = acc;
              }
            }
            // (every lane evaluates the DPP reads: a read under a branch
            // would see the lanes that took the other side as inactive)
            const float tot = G[3][e];
            const float sh1 = quad_perm(tot, 0x90);
            float s = tot + (qd >= 1 ? sh1 : 0.f);
            const float sh2 = quad_perm(s, 0x44);
            s = s + (qd >= 2 ? sh2 : 0.f);
            const float excl = s - tot;
            const float g3 = G[3][e] + excl;             // G at the lane's last token
            const float m = quad_perm(g3, 0x55);         // the reference, G at token 7
            const float g15 = quad_perm(g3, 0xFF);
            // from here on G holds the exponents G - m of the factors
            const float c = excl - m;
#pragma unroll
            for (int i = 0; i < 4; ++i) G[i][e] += c;
            fln[e] = exp2_fast(m);
            fkh[e] = exp2_fast(g15 - m);
            // channel decay of the whole sub-block (one lane per channel group)
            if (qd == 0) dvec[e] = fln[e] * fkh[e];
            // the lane's tokens against the reference: |G - m| <= kRange
#pragma unroll
            for (int i = 0; i < 4; ++i) worst = fmaxf(worst, fabsf(G[i][e]));
            // per-channel factors that exceed 1 only when some g > 0; each
            // may reach 2^10 so that no product of two factors overflows
            worst = fmaxf(worst, fmaxf(fmaxf(m, g15 - m), g15) + (kRange - 10.f));
          }
        };
        scan(false);
        if (__any(!(worst <= kRange))) scan(true);
        // the next chunk's g (the last chunk re-reads itself)
        const int64_t cn = ci + 1 < nchunks ? ci + 1 : ci;
        if constexpr (HAS_G && kEarly) {
#pragma unroll
          for (int i = 0; i < 4; ++i) load_tok(cn, i, false, true);
        }
        // gated operands, token by token; each operand row of the lane's
        // CPL channels goes out as one store
        T* sLn = opblk(slot, 0, pw);
        T* sQb = opblk(slot, 1, pw);
        T* sKh = opblk(slot, 2, pw);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float qv[CPL], kv[CPL], bv[CPL];
          unpack<T, CPL>(rq[i], qv);
          unpack<T, CPL>(rk[i], kv);
          unpack<GT, CPL>(rb[i], bv);
          if constexpr (kEarly) load_tok(cn, i, true, false);   // the next chunk's q, k, b
          else load_qk_tok(cn, i);                              // the next chunk's q, k
          if constexpr (RAW) {
#pragma unroll
            for (int e = 0; e < CPL; ++e) bv[e] = sigmoid_f(bv[e]);   // absent tokens: k = 0
          }
          uint32_t wLn[CPL / 2], wQb[CPL / 2], wKh[CPL / 2], wL[CPL / 2], wM[CPL / 2], wR[CPL / 2];
#pragma unroll
          for (int e2 = 0; e2 < CPL / 2; ++e2) {
            float Lv[2], Mv[2], Rv[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int e = 2 * e2 + h;
              const float x = G[i][e];
              const float e1 = exp2_fast(x);
              const float e2v = exp2_fast(-x);
              Lv[h] = -(bv[e] * kv[e]) * e1;
              Mv[h] = qv[e] * e1;
              Rv[h] = kv[e] * e2v;
            }
            const int e = 2 * e2;
            wLn[e2] = pack_bf16x2(Lv[0] * fln[e], Lv[1] * fln[e + 1]);
            wQb[e2] = pack_bf16x2(Mv[0] * fln[e], Mv[1] * fln[e + 1]);
            wKh[e2] = pack_bf16x2(Rv[0] * fkh[e], Rv[1] * fkh[e + 1]);
            wL[e2] = pack_bf16x2(Lv[0], Lv[1]);
            wM[e2] = pack_bf16x2(Mv[0], Mv[1]);
            wR[e2] = pack_bf16x2(Rv[0], Rv[1]);
          }
          const int r = 4 * qd + i;
          st_words<CPL / 2>(sLn + B::ax(r, ch0), wLn);
          st_words<CPL / 2>(sQb + B::ax(r, ch0), wQb);
          if constexpr (B::kWide) {   // (a lane's row piece is one 16-byte chunk)
            if (B::half_swapped(r)) {
              const uint32_t a0 = wKh[0], a1 = wKh[1];
              wKh[0] = wKh[2]; wKh[1] = wKh[3]; wKh[2] = a0; wKh[3] = a1;
            }
          }
          st_words<CPL / 2>(sKh + B::at(r, ch0), wKh);
          st_words<CPL / 2>(sL + B::at(r, ch0), wL);
          st_words<CPL / 2>(sM + B::at(r, ch0), wM);
          st_words<CPL / 2>(sR + B::at(r, ch0), wR);
        }
        if constexpr (!kEarly) load_bg(cn);   // the next chunk's b and g

        // Gram blocks; L carries the sign, so L . R = -A = N.  Layouts
        // (lane = 16 g + j):
        //   ac = L_{4g+i} . R_j = N[t][s], t = 4g+i, s = j
        //   ar = R_{4g+i} . L_j = N[t][s], t = j, s = 4g+i
        //   pr = R_{4g+i} . M_j = P[t][s], t = j, s = 4g+i
        // (this wave's LDS operations run in order, so its own stores above
        // complete before these reads)
        f32x4 ac = {0.f, 0.f, 0.f, 0.f}, ar = ac, pr = ac;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const Frag8<T> rf = ld_frag8<T>(sR + B::at(j, 32 * kb + 8 * g));
          const Frag8<T> lf = ld_frag8<T>(sL + B::at(j, 32 * kb + 8 * g));
          const Frag8<T> mf = ld_frag8<T>(sM + B::at(j, 32 * kb + 8 * g));
          mma32(ac, lf, rf);
          mma32(ar, rf, lf);
          mma32(pr, rf, mf);
        }
        // N strictly lower in both layouts; P lower incl. diagonal.  Selects
        // (not products) drop the entries above the diagonal, whose factors'
        // products may be inf or NaN.
        Frag4<float> nr, nc;
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tc = 4 * g + i;  // t of ac, s of ar
          nc.v[i] = (j < tc) ? ac[i] : 0.f;
          nr.v[i] = (tc < j) ? ar[i] : 0.f;
          pv[i] = (tc <= j) ? pr[i] : 0.f;
        }
        float nmax;
        const Frag4<float> tt = unit_lower_inverse(nr, nc, g, j, nmax);
        st4<T>(tblk(slot, pw) + tp_at(j, 4 * g), tt.v[0], tt.v[1], tt.v[2], tt.v[3]);
        st4<T>(pblk(slot, pw) + tp_at(j, 4 * g), pv[0], pv[1], pv[2], pv[3]);
        const bool bad = __any(!(worst <= kRange) || !(nmax <= kNBig));
        if (lane == 0) flagp(slot)[pw] = bad ? 1 : 0;
      };

      load(0);
      produce(0);
      __syncthreads();
      for (int64_t ci = 0; ci < nchunks; ++ci) {
        if (ci + 1 < nchunks) produce(ci + 1);
        __syncthreads();
      }
    } else {
      // Scalar gates.  lane (g, j): token j of the sub-block, channels
      // 32 kb + 8 g .. + 7 of every 32-channel block (the MFMA fragment).
      Raw<16> rq[KB], rk[KB], rv[2];
      uint32_t ub = 0u, ug = 0u;
      // raw gates: -exp(A_log) and dt_bias of the head
      const float nAs = RAW ? neg_exp_f(p.A_log ? p.A_log[hv] : 0.f) : 0.f;
      const float dts = RAW && p.dt_bias ? p.dt_bias[hv] : 0.f;
      // v rows of the sub-block for the consumers, whole 16-byte pieces:
      // lane l takes token 8 h + l / 8 and columns 8 (l % 8) .. + 7
      const char* bvs = reinterpret_cast<const char*>(gv) + ((uint64_t)tok0 * v_tok + (uint32_t)((hv * DV + c0) * 2));
      auto load = [&](int64_t ci) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          int64_t tv = ci * kC + kSB * pw + 8 * h + (lane >> 3);
          tv = tv < Tn - 1 ? tv : Tn - 1;
          ld_raw<16>(bvs + ((uint64_t)tv * v_tok + (uint32_t)((lane & 7) * 16)), rv[h]);
        }
        int64_t t = ci * kC + kSB * pw + j;
        t = t < Tn - 1 ? t : Tn - 1;
        const uint64_t tu = (uint64_t)t;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          ld_raw<16>(bq + (tu * qk_tok + (uint32_t)((32 * kb + 8 * g) * 2)), rq[kb]);
          ld_raw<16>(bk + (tu * qk_tok + (uint32_t)((32 * kb + 8 * g) * 2)), rk[kb]);
        }
        ub = ld_word<GT>(bbs + tu * gb_tok);
        if constexpr (HAS_G) ug = ld_word<GT>(bgs + tu * gg_tok);
      };
      auto produce = [&](int64_t ci) {
        const int slot = (int)(ci & 1);
        const bool present = ci * kC + kSB * pw + j < Tn;
        Frag8<T> kf[KB], qf[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          if (!present) { zero_raw(rq[kb]); zero_raw(rk[kb]); }
          kf[kb].v = __builtin_bit_cast(bf16x8, make_uint4(rk[kb].w[0], rk[kb].w[1], rk[kb].w[2], rk[kb].w[3]));
          qf[kb].v = __builtin_bit_cast(bf16x8, make_uint4(rq[kb].w[0], rq[kb].w[1], rq[kb].w[2], rq[kb].w[3]));
        }
        float beta = present ? word_f32<GT>(ub) : 0.f;
        float x = (HAS_G && present) ? word_f32<GT>(ug) : 0.f;
        if constexpr (RAW) {
          beta = present ? sigmoid_f(beta) : 0.f;
          x = (HAS_G && present) ? log_decay_f(x, nAs, dts) : 0.f;
        }
        x *= kLog2e;
        // inclusive prefix over the 16 tokens of the row
        x += dpp_row_shr(x, 1);
        x += dpp_row_shr(x, 2);
        x += dpp_row_shr(x, 4);
        x += dpp_row_shr(x, 8);
        const float G = x;
        const float g15 = dpp_row_bcast<15>(G);
        // largest rise G_t - min_{s<=t} G_s (0 when alpha <= 1)
        float mn = G;
        mn = fminf(mn, dpp_row_shr_inf(mn, 1));
        mn = fminf(mn, dpp_row_shr_inf(mn, 2));
        mn = fminf(mn, dpp_row_shr_inf(mn, 4));
        mn = fminf(mn, dpp_row_shr_inf(mn, 8));
        const float worst = fmaxf(fmaxf(G, g15 - G), G - mn);
        const float fo = exp2_fast(G);
        float* fv = vecp(slot) + pw * 6 * 16;
        if (g == 0) {
          fv[kFX * 16 + j] = -beta * fo;
          fv[kFO * 16 + j] = fo;
          fv[kFK * 16 + j] = exp2_fast(g15 - G);
          fv[kFB * 16 + j] = beta;
          fv[kFG * 16 + j] = G;
          if (j == 0) fv[kFD * 16] = exp2_fast(g15);
        }
        // raw k and q rows for the consumers: k twice, in the fragment
        // placement and in the transposing one
        T* sK = opblk(slot, 0, pw);
        T* sQ = opblk(slot, 1, pw);
        T* sKt = opblk(slot, 2, pw);
        const bool hs = B::half_swapped(j);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          *reinterpret_cast<uint4*>(sK + B::ax(j, 32 * kb + 8 * g)) =
              make_uint4(rk[kb].w[0], rk[kb].w[1], rk[kb].w[2], rk[kb].w[3]);
          *reinterpret_cast<uint4*>(sQ + B::ax(j, 32 * kb + 8 * g)) =
              make_uint4(rq[kb].w[0], rq[kb].w[1], rq[kb].w[2], rq[kb].w[3]);
          *reinterpret_cast<uint4*>(sKt + B::at(j, 32 * kb + 8 * g)) =
              hs ? make_uint4(rk[kb].w[2], rk[kb].w[3], rk[kb].w[0], rk[kb].w[1])
                 : make_uint4(rk[kb].w[0], rk[kb].w[1], rk[kb].w[2], rk[kb].w[3]);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = kSB * pw + 8 * h + (lane >> 3);
          const bool pres = ci * kC + r < Tn;   // absent tokens: v = 0
          *reinterpret_cast<uint4*>(vtile(slot) + vo_at(r, 8 * (lane & 7))) =
              pres ? make_uint4(rv[h].w[0], rv[h].w[1], rv[h].w[2], rv[h].w[3]) : make_uint4(0u, 0u, 0u, 0u);
        }
        load(ci + 1 < nchunks ? ci + 1 : ci);
        // Gram blocks: kk[4g+i][j] = k_{4g+i} . k_j, pq[4g+i][j] = k_{4g+i} . q_j
        f32x4 kk = {0.f, 0.f, 0.f, 0.f}, pq = kk;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          mma32(kk, kf[kb], kf[kb]);
          mma32(pq, kf[kb], qf[kb]);
        }
        const float4 G4 = *reinterpret_cast<const float4*>(fv + kFG * 16 + 4 * g);
        const float4 B4 = *reinterpret_cast<const float4*>(fv + kFB * 16 + 4 * g);
        const float Gs[4] = {G4.x, G4.y, G4.z, G4.w};
        const float Bs[4] = {B4.x, B4.y, B4.z, B4.w};
        Frag4<float> nr, nc;
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tc = 4 * g + i;
          // exponents are taken only where t >= s, so they are <= the rise
          const float dcol = exp2_fast((j < tc) ? Gs[i] - G : 0.f);   // t = tc, s = j
          const float drow = exp2_fast((tc <= j) ? G - Gs[i] : 0.f);  // t = j, s = tc
          nc.v[i] = (j < tc) ? -Bs[i] * dcol * kk[i] : 0.f;
          nr.v[i] = (tc < j) ? -beta * drow * kk[i] : 0.f;
          pv[i] = (tc <= j) ? drow * pq[i] : 0.f;
        }
        float nmax;
        const Frag4<float> tt = unit_lower_inverse(nr, nc, g, j, nmax);
        st4<T>(tblk(slot, pw) + tp_at(j, 4 * g), tt.v[0], tt.v[1], tt.v[2], tt.v[3]);
        st4<T>(pblk(slot, pw) + tp_at(j, 4 * g), pv[0], pv[1], pv[2], pv[3]);
        const bool bad = __any(!(worst <= kRange) || !(nmax <= kNBig));
        if (lane == 0) flagp(slot)[pw] = bad ? 1 : 0;
      };
      load(0);
      produce(0);
      __syncthreads();
      for (int64_t ci = 0; ci < nchunks; ++ci) {
        if (ci + 1 < nchunks) produce(ci + 1);
        __syncthreads();
      }
    }
    return;
  }

  // ===================================================================
  // Consumer wave w: state columns col = c0 + 16 w + j; accumulator tile
  // 2kb + h, row 4g + i <-> channel 32kb + 8g + 4h + i.
  // ===================================================================
  // Issue priority: with channel gates the consumers' state chain goes
  // first and the producer wave on the same SIMD fills the gaps; with scalar
  // gates, whose producers wait mostly on their loads, the producers go first
  // (measured: each order is a few per cent faster on its own gate mode).
  if constexpr (CHANNEL) __builtin_amdgcn_s_setprio(3);
  const int col = c0 + 16 * wave + j;
  f32x4 S[MT];
  {
    const float* sin = p.state_in ? p.state_in + head * (int64_t)DK * DV : nullptr;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 32 * (t >> 1) + 8 * g + 4 * (t & 1) + i;
        S[t][i] = sin ? sin[row * DV + col] : 0.f;
      }
  }
  // Saved for the backward (when asked): block m's entry state as the
  // [column][channel] row of this lane's column (16-byte pieces of 8
  // channels), and u of every token.
  T* ckb = nullptr;
  if constexpr (SAVE) {
    const int64_t slot0 = p.cu ? tok0 / kSB + 2 * bidx : bidx * (p.ck_nblk + 1);
    ckb = p.ck + (((int64_t)hv * NSPLIT + split) * p.ck_slots + slot0) * (int64_t)DK * DVS +
          (int64_t)(16 * wave + j) * DK + 8 * g;
  }
  auto save_state = [&](int64_t tb, const Frag8<T>* sf) {
    T* dst = ckb + (tb / kSB) * (int64_t)DVS * DK;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) *reinterpret_cast<Frag8<T>*>(dst + 32 * kb) = sf[kb];
  };
  const uint32_t w_tok = RAW ? (uint32_t)(p.ld_w * (int64_t)sizeof(GT))
                             : (uint32_t)(p.Hv * DV * (int)sizeof(GT));
  // v (and w) of the 16 tokens 16 sb + 4 g + i of a chunk for this column,
  // two tokens per register: zv/zw are prefetched a chunk ahead, cv/cw hold
  // the chunk being consumed (fp32 write gates keep one per word).  The reads
  // go through buffer descriptors based at the chunk's first token: one
  // 32-bit lane offset (the lane's column) and the token offset as a scalar.
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  constexpr int WPW = sizeof(GT) == 2 ? 2 : 1;  // w tokens per word
  u16x2 zv[NSB][2], cv[NSB][2];
  uint32_t zw[NSB][4 / WPW], cw[NSB][4 / WPW];
  const char* bv0 = reinterpret_cast<const char*>(gv) + (uint64_t)tok0 * v_tok;
  const char* bw0 = reinterpret_cast<const char*>(gw) + (uint64_t)tok0 * w_tok;
  const int cvo = (hv * DV + col) * 2;
  const int cwo = (hv * DV + col) * (int)sizeof(GT);
  auto rsrc = [](const char* base, uint32_t bytes) {
    // the base is the same in every lane; say so, so that it stays scalar
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    char* u = reinterpret_cast<char*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, (int)bytes, 0x00020000);
  };
  auto load_z = [&](int64_t ci) {
    const int64_t t0 = ci * kC;
    const auto rv = rsrc(bv0 + (uint64_t)t0 * v_tok, (uint32_t)kC * v_tok);
    const auto rw = rsrc(CHANNEL ? bw0 + (uint64_t)t0 * w_tok : bv0, CHANNEL ? (uint32_t)kC * w_tok : 0u);
    // tokens a and b (chunk-relative) of the pair (sb, h): lane term la / lb
    // plus scalar term sa / sb (bytes of v); w likewise
    auto fetch = [&](int sb, int h, int lva, int lvb, int sva, int svb, int lwa, int lwb, int swa,
                     int swb) {
      u16x2 pv;
      pv.x = __builtin_amdgcn_raw_buffer_load_b16(rv, lva, sva, 0);
      pv.y = __builtin_amdgcn_raw_buffer_load_b16(rv, lvb, svb, 0);
      zv[sb][h] = pv;
      if constexpr (CHANNEL) {
        if constexpr (WPW == 2) {
          u16x2 pw2;
          pw2.x = __builtin_amdgcn_raw_buffer_load_b16(rw, lwa, swa, 0);
          pw2.y = __builtin_amdgcn_raw_buffer_load_b16(rw, lwb, swb, 0);
          zw[sb][h] = __builtin_bit_cast(uint32_t, pw2);
        } else {
          zw[sb][2 * h] = __builtin_amdgcn_raw_buffer_load_b32(rw, lwa, swa, 0);
          zw[sb][2 * h + 1] = __builtin_amdgcn_raw_buffer_load_b32(rw, lwb, swb, 0);
        }
      }
    };
    if (t0 + kC <= Tn) {
      // full chunk: token 16 sb + 4 g + 2 h (+1); the 4g term is the lane's
      const int lv = cvo + 4 * g * (int)v_tok, lw = cwo + 4 * g * (int)w_tok;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int u = kSB * sb + 2 * h;
          fetch(sb, h, lv, lv, u * (int)v_tok, (u + 1) * (int)v_tok, lw, lw, u * (int)w_tok,
                (u + 1) * (int)w_tok);
        }
    } else {
      // the partial last chunk clamps every token to the last one and zeroes
      // the values of tokens past the end, so that their rows of X (and U)
      // vanish
      const int lastl = (int)(Tn - 1 - t0);
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          int l0 = kSB * sb + 4 * g + 2 * h, l1 = l0 + 1;
          const bool p0 = l0 <= lastl, p1 = l1 <= lastl;
          l0 = p0 ? l0 : lastl;
          l1 = p1 ? l1 : lastl;
          fetch(sb, h, cvo + l0 * (int)v_tok, cvo + l1 * (int)v_tok, 0, 0, cwo + l0 * (int)w_tok,
                cwo + l1 * (int)w_tok, 0, 0);
          if (!p0) zv[sb][h].x = 0;
          if (!p1) zv[sb][h].y = 0;
        }
    }
  };
  // value of token 4g + i of sub-block sb from the packed words
  auto zval = [&](int sb, int i) -> float {
    const u16x2 pv = cv[sb][i >> 1];
    return __uint_as_float(((uint32_t)((i & 1) ? pv.y : pv.x)) << 16);
  };
  auto wval = [&](int sb, int i) -> float {
    if constexpr (WPW == 2) {
      const uint32_t w = cw[sb][i >> 1];
      return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
      return __uint_as_float(cw[sb][i]);
    }
  };

  // Exact token-by-token recurrence for tokens [tb, min(tb + 16, Tn)) of the
  // chunk in the given slot that starts at token cb.
  auto tokens_path = [&](int slot, int64_t cb, int64_t tb) {
    if constexpr (SAVE) {
      Frag8<T> sf[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sf[kb] = frag8_from_acc<T>(S[2 * kb], S[2 * kb + 1]);
      save_state(tb, sf);
    }
    for (int tl = 0; tl < kSB; ++tl) {
      const int64_t tok = tb + tl;
      if (tok >= Tn) break;
      const int64_t qk_off = ((tok0 + tok) * p.Hk + hk) * (int64_t)DK;
      const int64_t gt = (tok0 + tok) * p.Hv + hv;
      float sbeta = 0.f, salpha = 1.f;
      // raw channel gates: the token's activated b and alpha, computed by the
      // wave (two channels per lane) into its quarter of the flagged
      // sub-block's first operand block, which nothing reads in this chunk
      // (a wave's LDS accesses complete in order, so no barrier is needed)
      const float* gact = nullptr;
      if constexpr (CHANNEL && RAW) {
        float* gsc = reinterpret_cast<float*>(opblk(slot, 0, (int)((tb - cb) / kSB))) + wave * 2 * DK;
#pragma unroll
        for (int c = lane; c < DK; c += 64) {
          gsc[c] = sigmoid_f(to_f32(gb[gate_row(tok, p.ld_b) + hv * DK + c]));
          float al = 1.f;
          if constexpr (HAS_G) {
            const int col = hv * DK + c;
            al = exp2_fast(log_decay_f(to_f32(gg[gate_row(tok, p.ld_g) + col]),
                                       neg_exp_f(p.A_log ? p.A_log[col] : 0.f),
                                       p.dt_bias ? p.dt_bias[col] : 0.f) * kLog2e);
          }
          gsc[DK + c] = al;
        }
        gact = gsc;
      }
      if constexpr (!CHANNEL) {
        if constexpr (RAW) {
          sbeta = sigmoid_f(to_f32(gb[gate_row(tok, p.ld_b) + hv]));
          if constexpr (HAS_G)
            salpha = exp2_fast(log_decay_f(to_f32(gg[gate_row(tok, p.ld_g) + hv]),
                                           neg_exp_f(p.A_log ? p.A_log[hv] : 0.f),
                                           p.dt_bias ? p.dt_bias[hv] : 0.f) * kLog2e);
        } else {
          sbeta = to_f32(gb[gt]);
          if constexpr (HAS_G) salpha = exp2_fast(to_f32(gg[gt]) * kLog2e);
        }
      }
      float rp = 0.f;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int row = 32 * (t >> 1) + 8 * g + 4 * (t & 1);
        float kr[4], er[4], ar[4];
        load_f32<4, T>(gk + qk_off + row, kr);
        if constexpr (CHANNEL) {
          if constexpr (RAW) {
            const float4 e4 = *reinterpret_cast<const float4*>(gact + row);
            const float4 a4 = *reinterpret_cast<const float4*>(gact + DK + row);
            er[0] = e4.x; er[1] = e4.y; er[2] = e4.z; er[3] = e4.w;
            ar[0] = a4.x; ar[1] = a4.y; ar[2] = a4.z; ar[3] = a4.w;
          } else if constexpr (HAS_G) {
            load_f32<4, GT>(gb + gt * DK + row, er);
            load_f32<4, GT>(gg + gt * DK + row, ar);
#pragma unroll
            for (int i = 0; i < 4; ++i) ar[i] = exp2_fast(ar[i] * kLog2e);
          } else {
            load_f32<4, GT>(gb + gt * DK + row, er);
#pragma unroll
            for (int i = 0; i < 4; ++i) ar[i] = 1.f;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) { er[i] = sbeta; ar[i] = salpha; }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          S[t][i] *= ar[i];
          rp += er[i] * kr[i] * S[t][i];
        }
      }
      rp += __shfl_xor(rp, 16);
      rp += __shfl_xor(rp, 32);
      float z = to_f32(gv[gt * DV + col]);
      if constexpr (CHANNEL) {
        if constexpr (RAW) z *= sigmoid_f(to_f32(gw[gate_row(tok, p.ld_w) + hv * DV + col]));
        else z *= to_f32(gw[gt * DV + col]);
      }
      else z *= sbeta;
      const float d = z - rp;
      if (SAVE && g == 0) p.u[gt * DV + col] = from_f32<T>(d);
      float op = 0.f;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int row = 32 * (t >> 1) + 8 * g + 4 * (t & 1);
        float kr[4], qr[4];
        load_f32<4, T>(gk + qk_off + row, kr);
        load_f32<4, T>(gq + qk_off + row, qr);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          S[t][i] += kr[i] * d;
          op += qr[i] * S[t][i];
        }
      }
      op += __shfl_xor(op, 16);
      op += __shfl_xor(op, 32);
      if (g == 0) {
        if constexpr (CHANNEL) go[gt * DV + col] = from_f32<T>(p.scale * op);
        else otile(slot)[vo_at((int)(tok - cb), 16 * wave + j)] = from_f32<T>(p.scale * op);
      }
    }
    (void)slot; (void)cb;
  };

  // The state-independent operands of one sub-block, read from LDS ahead of
  // their use (the common loop reads sub-block sb + 1 while sb computes).
  struct Ops {
    Frag8<T> af[KB], qf[KB];
    Frag4<T> td, pf;
    float4 fx, fb, f4;
    float fo, dsc;
  };
  auto ld_ops = [&](int slot, int sb) {
    Ops o;
    const T* sA = opblk(slot, 0, sb);   // Ln | k
    const T* sQ = opblk(slot, 1, sb);   // Qb | q
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      o.af[kb] = ld_frag8<T>(sA + B::ax(j, 32 * kb + 8 * g));
      o.qf[kb] = ld_frag8<T>(sQ + B::ax(j, 32 * kb + 8 * g));
    }
    o.td = ld_frag4<T>(tblk(slot, sb) + tp_at(j, 4 * g));
    o.pf = ld_frag4<T>(pblk(slot, sb) + tp_at(j, 4 * g));
    o.fo = 1.f;
    o.dsc = 1.f;
    if constexpr (!CHANNEL) {
      const float* fv = vecp(slot) + sb * 6 * 16;
      o.fx = *reinterpret_cast<const float4*>(fv + kFX * 16 + 4 * g);
      o.fb = *reinterpret_cast<const float4*>(fv + kFB * 16 + 4 * g);
      o.f4 = *reinterpret_cast<const float4*>(fv + kFK * 16 + 4 * g);
      o.fo = fv[kFO * 16 + j];
      o.dsc = fv[kFD * 16];
    }
    return o;
  };

  // One sub-block on the MFMA path.  zpre: take v (and w) from the
  // prefetched words (the unrolled common loop) or load them here (the loop
  // of a chunk that holds a sub-block on the exact path).
  auto sub_block = [&](int slot, int sb, int64_t tb, auto zpre, const Ops& op) {
    const T* sK = opblk(slot, 2, sb);   // Kh | k, transposing placement
    const float* fv = vecp(slot) + (CHANNEL ? sb * DK : sb * 6 * 16);
    Frag4<T> kt[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
      kt[t] = ld_tr16(sK + B::ath(4 * g + (j >> 2), 32 * (t >> 1) + 8 * (j & 3) + 4 * (t & 1)));
    const Frag8<T>* af = op.af;
    const Frag8<T>* qf = op.qf;
    const Frag4<T>& td = op.td;
    const Frag4<T>& pf = op.pf;
    const float4 fx = op.fx, fb = op.fb, f4 = op.f4;
    const float fo = op.fo, dsc = op.dsc;
    Frag8<T> sf[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sf[kb] = frag8_from_acc<T>(S[2 * kb], S[2 * kb + 1]);
    if constexpr (SAVE) save_state(tb, sf);
    f32x4 X, O = {0.f, 0.f, 0.f, 0.f};
    float zz[4], ww[4];
    const bool full_sb = tb + kSB <= Tn;  // wave-uniform
    Frag4<T> vz;
    if constexpr (!CHANNEL)  // v rows 16 sb + 4 g + i, column 16 wave + j
      vz = ld_tr16(vtile(slot) + vo_at(16 * sb + 4 * g + (j >> 2), 16 * wave + 4 * (j & 3)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (!CHANNEL) {
        // absent tokens hold zero in the tile
        zz[i] = (float)vz.v[i];
        ww[i] = 0.f;
      } else if constexpr (decltype(zpre)::value) {
        // prefetched words: tokens past the end already hold zero
        zz[i] = zval(sb, i);
        ww[i] = RAW ? sigmoid_f(wval(sb, i)) : wval(sb, i);
      } else {
        const int64_t t = tb + 4 * g + i;
        const int64_t tc = t < Tn - 1 ? t : Tn - 1;
        zz[i] = t < Tn ? to_f32(gv[((tok0 + tc) * p.Hv + hv) * (int64_t)DV + col]) : 0.f;
        if constexpr (CHANNEL) {
          if constexpr (RAW) ww[i] = sigmoid_f(to_f32(gw[gate_row(tc, p.ld_w) + hv * DV + col]));
          else ww[i] = to_f32(gw[((tok0 + tc) * p.Hv + hv) * (int64_t)DV + col]);
        } else {
          ww[i] = 0.f;
        }
      }
    }
    if constexpr (CHANNEL) {
#pragma unroll
      for (int i = 0; i < 4; ++i) X[i] = zz[i] * ww[i];
    } else {
      X = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      mma32(X, af[kb], sf[kb]);   // X[4g+i][j]: token 4g+i, column j
      mma32(O, sf[kb], qf[kb]);   // O[4g+i][j]: column 4g+i, token j
    }
    // the state decays while the products run: S = Diag(D) S + Kh^T U
    if constexpr (CHANNEL) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const float4 d4 = *reinterpret_cast<const float4*>(fv + 32 * (t >> 1) + 8 * g + 4 * (t & 1));
        S[t][0] *= d4.x; S[t][1] *= d4.y; S[t][2] *= d4.z; S[t][3] *= d4.w;
      }
    } else if constexpr (HAS_G) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[t][i] *= dsc;
    }
    float fk[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (!CHANNEL) {
      X[0] = fmaf(fx.x, X[0], fb.x * zz[0]);
      X[1] = fmaf(fx.y, X[1], fb.y * zz[1]);
      X[2] = fmaf(fx.z, X[2], fb.z * zz[2]);
      X[3] = fmaf(fx.w, X[3], fb.w * zz[3]);
#pragma unroll
      for (int i = 0; i < 4; ++i) O[i] *= fo;
      fk[0] = f4.x; fk[1] = f4.y; fk[2] = f4.z; fk[3] = f4.w;
    }
    const Frag4<T> xf = frag4_from_acc<T>(X);
    f32x4 U = {0.f, 0.f, 0.f, 0.f};
    mma16(U, td, xf);  // U[4g+i][j]
    const Frag4<T> uo = frag4_from_acc<T>(U);
    if constexpr (SAVE) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = tb + 4 * g + i;
        if (full_sb || t < Tn) p.u[((tok0 + t) * p.Hv + hv) * (int64_t)DV + col] = uo.v[i];
      }
    }
    Frag4<T> uk = uo;
    if constexpr (!CHANNEL) {
      f32x4 us = {U[0] * fk[0], U[1] * fk[1], U[2] * fk[2], U[3] * fk[3]};
      uk = frag4_from_acc<T>(us);
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) mma16(S[t], kt[t], uk);
    mma16(O, uo, pf);
    if constexpr (CHANNEL) {
      const int64_t tok = tb + j;
      if (full_sb || tok < Tn) {
        T* dst = go + ((tok0 + tok) * p.Hv + hv) * (int64_t)DV + c0 + 16 * wave + 4 * g;
        st4<T>(dst, p.scale * O[0], p.scale * O[1], p.scale * O[2], p.scale * O[3]);
      }
    } else {
      // token 16 sb + j, columns 16 wave + 4 g .. + 3, into the o tile
      st4<T>(otile(slot) + vo_at(16 * sb + j, 16 * wave + 4 * g), p.scale * O[0], p.scale * O[1],
             p.scale * O[2], p.scale * O[3]);
    }
  };

  // Scalar gates: o rows of a finished chunk from its tile to memory, whole
  // 16-byte pieces (consumer wave w: tokens 16 w .. 16 w + 15).
  auto flush_o = [&](int64_t ci) {
    const int slot = (int)(ci & 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 16 * wave + 8 * h + (lane >> 3);
      const int64_t tok = ci * kC + r;
      if (tok < Tn) {
        const uint4 val = *reinterpret_cast<const uint4*>(otile(slot) + vo_at(r, 8 * (lane & 7)));
        *reinterpret_cast<uint4*>(go + ((tok0 + tok) * p.Hv + hv) * (int64_t)DV + c0 + 8 * (lane & 7)) = val;
      }
    }
  };

  if constexpr (CHANNEL) load_z(0);
  __syncthreads();  // chunk 0 is ready
  for (int64_t ci = 0; ci < nchunks; ++ci) {
    const int slot = (int)(ci & 1);
    if constexpr (CHANNEL) {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
        for (int h = 0; h < 2; ++h) cv[sb][h] = zv[sb][h];
#pragma unroll
        for (int h = 0; h < 4 / WPW; ++h) cw[sb][h] = zw[sb][h];
      }
      load_z(ci + 1 < nchunks ? ci + 1 : ci);
    } else if (ci > 0) {
      flush_o(ci - 1);  // the previous chunk's rows, complete since the barrier
    }
    const int* fl = flagp(slot);
    if ((fl[0] | fl[1] | fl[2] | fl[3]) == 0) {
      Ops cur = ld_ops(slot, 0);
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const int64_t tb = ci * kC + kSB * sb;
        Ops nxt;
        if (sb + 1 < NSB) nxt = ld_ops(slot, sb + 1);
        if (tb < Tn) sub_block(slot, sb, tb, IntTag<1>{}, cur);
        if (sb + 1 < NSB) cur = nxt;
      }
    } else {
      // a chunk with a sub-block whose decay range the factored form cannot
      // hold: that sub-block runs the exact recurrence, the others as usual
#pragma unroll 1
      for (int sb = 0; sb < NSB; ++sb) {
        const int64_t tb = ci * kC + kSB * sb;
        if (tb < Tn) {
          if (fl[sb]) tokens_path(slot, ci * kC, tb);
          else sub_block(slot, sb, tb, IntTag<0>{}, ld_ops(slot, sb));
        }
      }
    }
    __syncthreads();
  }
  if constexpr (!CHANNEL) flush_o(nchunks - 1);
  if (p.state_out) {
    float* sout = p.state_out + head * (int64_t)DK * DV;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 32 * (t >> 1) + 8 * g + 4 * (t & 1) + i;
        sout[row * DV + col] = S[t][i];
      }
  }
}

template <typename GT, int DK, int DV, bool CH, bool HG, bool RAW = false>
hipError_t launch_sb_typed(const ChunkArgs& a, hipStream_t stream) {
  const bool save = a.ck != nullptr;
  Params p;
  p.B = a.B; p.T = a.T; p.cu = a.cu_seqlens; p.Hk = a.Hk; p.Hv = a.Hv; p.scale = a.scale;
  p.q = a.q; p.k = a.k; p.v = a.v; p.b = a.b; p.w = a.w; p.g = a.g;
  p.state_in = a.state_in; p.state_out = a.state_out; p.o = a.o;
  p.ld_b = a.ld_b; p.ld_g = a.ld_g; p.ld_w = a.ld_w; p.A_log = a.A_log; p.dt_bias = a.dt_bias;
  p.ck = static_cast<bf16*>(a.ck); p.u = static_cast<bf16*>(a.u);
  p.ck_slots = a.ck_slots; p.ck_nblk = a.ck_nblk;
  const int64_t nwg = a.B * a.Hv * (DV / 64);
  if constexpr (RAW) {
    if (save) return hipErrorNotSupported;
    chunk_fwd_sb_kernel<GT, DK, DV, CH, HG, true, false>
        <<<dim3((unsigned)nwg), dim3(kSbThreads), 0, stream>>>(p);
  } else if (save) {
    chunk_fwd_sb_kernel<GT, DK, DV, CH, HG, false, true>
        <<<dim3((unsigned)nwg), dim3(kSbThreads), 0, stream>>>(p);
  } else {
    chunk_fwd_sb_kernel<GT, DK, DV, CH, HG, false, false>
        <<<dim3((unsigned)nwg), dim3(kSbThreads), 0, stream>>>(p);
  }
  return hipGetLastError();
}

template <typename GT, int DK, int DV>
hipError_t sb_gates(const ChunkArgs& a, hipStream_t s) {
  const bool hg = a.g != nullptr;
  if (a.channel) return hg ? launch_sb_typed<GT, DK, DV, true, true>(a, s)
                           : launch_sb_typed<GT, DK, DV, true, false>(a, s);
  return hg ? launch_sb_typed<GT, DK, DV, false, true>(a, s)
            : launch_sb_typed<GT, DK, DV, false, false>(a, s);
}

template <typename GT>
hipError_t sb_dims(const ChunkArgs& a, hipStream_t s) {
  if (a.dk == 128 && a.dv == 128) return sb_gates<GT, 128, 128>(a, s);
  if (a.dk == 128 && a.dv == 64) return sb_gates<GT, 128, 64>(a, s);
  if (a.dk == 64 && a.dv == 128) return sb_gates<GT, 64, 128>(a, s);
  return sb_gates<GT, 64, 64>(a, s);
}

// Raw gate projections: bf16 projections, d_k = d_v = 128.
hipError_t sb_raw(const ChunkArgs& a, hipStream_t s) {
  if (a.gate != DType::BF16 || a.dk != 128 || a.dv != 128) return hipErrorNotSupported;
  const bool hg = a.g != nullptr;
  if (a.channel) return hg ? launch_sb_typed<bf16, 128, 128, true, true, true>(a, s)
                           : launch_sb_typed<bf16, 128, 128, true, false, true>(a, s);
  return hg ? launch_sb_typed<bf16, 128, 128, false, true, true>(a, s)
            : launch_sb_typed<bf16, 128, 128, false, false, true>(a, s);
}

}  // namespace

// bf16 operands: sub-block producer/consumer kernel.
hipError_t launch_chunk_fwd_sb(const ChunkArgs& a, hipStream_t stream) {
  if (a.raw_gates) return sb_raw(a, stream);
  if (a.gate == DType::F32) return sb_dims<float>(a, stream);
  return sb_dims<bf16>(a, stream);
}

#ifdef GDN_CHECK
unsigned check_violations_chunk_sb() { return take_check_violations(); }

namespace {
__global__ __launch_bounds__(64) void check_selftest_kernel(float* out) {
  __shared__ float buf[64];
  lds_nan_fill(buf, (int)sizeof buf);
  const int l = (int)threadIdx.x;
  out[l] = buf[l];                        // in bounds, never written
  lds_check(buf + 64 + l, 4);             // one past the end: counted, not made
}
}  // namespace

hipError_t launch_check_selftest(float* out, hipStream_t stream) {
  check_selftest_kernel<<<1, 64, 0, stream>>>(out);
  return hipGetLastError();
}
#endif

}  // namespace gdn
