// gdn_kernels.hpp -- host-side launch interface between the C ABI layer
// (gdn_api.cpp) and the kernel translation units.  Arguments arrive already
// validated; each launcher only picks the template instantiation and launches
// on the given stream, returning the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

enum class DType : int { F32 = 0, BF16 = 1 };

struct DecodeArgs {
  int64_t N;
  int Hk, Hv, dk, dv;
  DType io, gate;
  bool channel;
  float scale;
  const void *q, *k, *v, *b, *w, *g;
  float* state;
  void* o;
};

struct ChunkArgs {
  int64_t B, T;                       // sequences; tokens each (packed total with cu_seqlens)
  const int64_t* cu_seqlens = nullptr;  // device [B + 1] offsets of packed sequences
  int Hk, Hv, dk, dv;
  DType io, gate;
  bool channel;
  float scale;
  const void *q, *k, *v, *b, *w, *g;
  const float* state_in;
  float* state_out;
  void* o;
  // raw gate projections (b, g, w hold the projections; see chunk_common.hpp)
  bool raw_gates = false;
  int64_t ld_b = 0, ld_g = 0, ld_w = 0;
  const float* A_log = nullptr;
  const float* dt_bias = nullptr;
  // optional: what the backward's forward rebuild stores (BwdArgs ckpt and u,
  // bf16, in the backward's layout; ck_slots and ck_nblk as there)
  void* ck = nullptr;
  void* u = nullptr;
  int64_t ck_slots = 0, ck_nblk = 0;
};

// Short causal convolution of the q, k, v branch (+ SiLU, L2 norm of q, k).
struct ConvArgs {
  int64_t N, total_T;
  int64_t Tseq;                       // tokens per sequence when cu_seqlens is NULL
  const int64_t* cu_seqlens;          // device [N + 1] offsets, or NULL
  int Hk, Hv, dk, dv;
  int64_t C;                          // 2 Hk dk + Hv dv channels
  int64_t ld_x;                       // row stride of x (elements)
  DType io;
  float eps;
  const void* x;
  const float* w;                     // [C, 4]
  const void* s_in;                   // [N, 3, C] or NULL
  void* s_out;                        // [N, 3, C] or NULL
  void *q, *k, *v;
};

// Gate activations; element totals fit in 32 bits (checked by the caller).
struct GateArgs {
  uint32_t n_ab, n_w;                 // columns of a/b and of w (0: no w)
  uint32_t n_ab_total, n_w_total;     // rows * columns
  int64_t ld_a, ld_b, ld_w;
  DType in, out;
  const void *a, *b, *w_raw;
  const float *A_log, *dt_bias;       // [n_ab] or NULL
  void *g, *beta, *w;
};

// Output RMS norm times swish(z).
struct NormArgs {
  int64_t rows;
  int Hv, dv;
  int64_t ld_z;
  DType io;
  float eps;
  const void *o, *z;
  const float* weight;                // [dv]
  void* y;
};

// Gradients of the recurrence.  Workspace: ckpt [Hv][dv/64][slots][dk][64],
// the states every 16 tokens and the final state of each sequence;
// u [rows*Hv][dv]; part [dv/64][4][rows*Hv][dk] per-column-block row
// gradients followed by [dv/64][rows*Hv] write-gate sums (scalar gates).
struct BwdArgs {
  int64_t B, T;                       // sequences; tokens each (packed total with cu)
  const int64_t* cu = nullptr;        // device [B + 1] offsets of packed sequences
  int64_t rows;                       // token rows of q, k, v, ... (B*T, or packed total)
  int64_t slots;                      // checkpoint slots per (value head, 64 columns)
  int Hk, Hv, dk, dv;
  DType io, gate;
  bool channel;
  float scale;
  const void *q, *k, *v, *b, *w, *g, *d_o;
  const float *state_in, *d_state_out;
  // checkpoint states and u in the MFMA operand type (io), partial row
  // gradients in fp32; with `direct` the row gradients go straight to the
  // outputs (channel gates, H_v == H_k, at most two column blocks) and
  // `part` is unused
  void *ckpt, *u;
  float* part;
  bool direct;
  int phases = 3;                     // 1: forward rebuild only, 2: reverse walk only
  int64_t nblk;
  float *dq_out, *dk_out, *dv_out, *db, *dw, *dg, *d_state_in;
};
int64_t bwd_checkpoint_blocks(int64_t T);
hipError_t launch_backward(const BwdArgs& a, hipStream_t stream);

hipError_t launch_short_conv(const ConvArgs& a, hipStream_t stream);
hipError_t launch_gates(const GateArgs& a, hipStream_t stream);
hipError_t launch_output_gate(const NormArgs& a, hipStream_t stream);

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_chunk_fwd(const ChunkArgs& a, hipStream_t stream);
// bf16-operand sub-block variant (called by launch_chunk_fwd).
hipError_t launch_chunk_fwd_sb(const ChunkArgs& a, hipStream_t stream);

#ifdef GDN_CHECK
// Debug build: LDS accesses out of range counted by each module's kernels
// since the previous call (after all work on the device has finished).
unsigned check_violations_decode();
unsigned check_violations_chunk();
unsigned check_violations_chunk_sb();
unsigned check_violations_backward();
// One block: out[l] = never-written LDS word l, and one counted (unmade)
// access past the kernel's LDS per lane (64 in all).
hipError_t launch_check_selftest(float* out, hipStream_t stream);
#endif
// state_out = state_in (or 0 when state_in is NULL) for n floats; used when
// there are no tokens to process.
hipError_t launch_state_copy(const float* state_in, float* state_out, int64_t n,
                             hipStream_t stream);

}  // namespace gdn
