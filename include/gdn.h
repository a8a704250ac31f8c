/*
 * gdn.h -- C ABI of libgdn.so: the gated delta rule (GDN-2, with Gated DeltaNet
 * and DeltaNet as special cases) on AMD Instinct MI355X (gfx950).
 *
 * The operation (per value head; S is the d_k x d_v state, fp32, row-major):
 *
 *   e_t = b_t (.) k_t                     erase/read direction
 *   z_t = w_t (.) v_t                     gated write target
 *   S_t = (I - k_t e_t^T) Diag(alpha_t) S_{t-1} + k_t z_t^T
 *   o_t = scale * S_t^T q_t               read-out after the update
 *
 * defined by "Gated DeltaNet-2: Decoupling Erase and Write in Linear
 * Attention" (gist.science summary), Methodologie §1 (update equation, erase
 * gate b_t in [0,1]^{d_k}, write gate w_t in [0,1]^{d_v}, channel decay
 * D_t = Diag(alpha_t)), and by the news page on the same paper (zubnet.ai),
 * which restates the equation and the gate roles.  With b_t = w_t = beta_t
 * (a scalar per token and head) and a scalar alpha_t it is the gated delta
 * rule of "Gated DeltaNet" (docsaid.org notes, §Reunir les deux); with
 * alpha = 1 it is DeltaNet (same notes, §DeltaNet).  The read-out is the
 * notes' o_t = S_t q_t (§L'attention lineaire) in the transposed storage used
 * here.
 *
 * Conventions shared by every entry point:
 *  - Memory: every tensor pointer is a DEVICE pointer (hipMalloc'd or from the
 *    caller's allocator), dense, row-major in the order given, contiguous, and
 *    16-byte aligned.  Descriptors are HOST pointers, read during the call only.
 *    The caller owns all memory; the library allocates nothing and keeps no
 *    mutable global state, so calls are reentrant and thread-safe.
 *  - Decay is passed in log space: g = log(alpha) (alpha = exp(g)); a NULL g
 *    means alpha = 1 (DeltaNet).  Gates are not clamped: any finite b, w, g is
 *    accepted (beta in (0, 2) is allowed); non-finite inputs give undefined
 *    results.
 *  - Key/value head grouping: value head h reads key head h / (H_v / H_k)
 *    (architecture notes page "Gated DeltaNet", §La dissymetrie 16 / 128: eight
 *    value heads share one key head).
 *  - Asynchrony: work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream).  GDN_OK means the launch succeeded, not that the work finished.
 *  - Errors: arguments are validated synchronously before anything is
 *    enqueued.  On GDN_ERR_INVALID_ARG or GDN_ERR_UNSUPPORTED nothing is
 *    enqueued and no output is touched.  GDN_ERR_HIP reports a failed launch
 *    (hipGetLastError).  Nothing is printed and no exception crosses the ABI.
 *  - Aliasing: outputs must not overlap inputs, except state_out == state_in
 *    exactly (in-place chaining), which is allowed.  Partial overlap is
 *    rejected.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 9  /* 2: adds gdn_chunk_fwd_varlen; 3: adds gdn_short_conv,
                              gdn_gates, gdn_output_gate; 4: adds gdn_backward;
                              5: adds gdn_backward_varlen; 6: adds
                              gdn_backward_noalloc; 7: adds gdn_chunk_fwd_gated;
                              8: adds gdn_chunk_fwd_save, gdn_backward_saved and
                              their packed forms gdn_chunk_fwd_varlen_save,
                              gdn_backward_varlen_saved; 9: adds
                              GDN_ERR_CHECK and gdn_check_selftest */

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARG = 1, /* NULL/misaligned/overlapping pointer, bad shape  */
  GDN_ERR_UNSUPPORTED = 2, /* valid request this build does not implement      */
  GDN_ERR_HIP = 3,         /* the HIP runtime reported an error at launch      */
  GDN_ERR_CHECK = 4        /* debug build libgdn_check.so only (-DGDN_CHECK):
                              a kernel of the call accessed LDS outside its
                              layout; that build waits for every launch to
                              finish and reads its device counters, which the
                              normal libgdn.so never does */
} gdn_status;

typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef enum gdn_gate_mode {
  /* Gated DeltaNet / DeltaNet: beta [.., H_v], g [.., H_v]; w must be NULL.  */
  GDN_GATES_SCALAR = 0,
  /* GDN-2: b [.., H_v, d_k], w [.., H_v, d_v], g [.., H_v, d_k].             */
  GDN_GATES_CHANNEL = 1
} gdn_gate_mode;

/* Chunked forward over a sequence batch. */
typedef struct gdn_fwd_desc {
  int64_t B;          /* batch, >= 0 (0: nothing to do)                          */
  int64_t T;          /* tokens per sequence, >= 0 (0: state_out = state_in)     */
  int32_t H_k, H_v;   /* >= 1, H_v % H_k == 0                                    */
  int32_t d_k, d_v;   /* each 64 or 128                                          */
  int32_t io_dtype;   /* gdn_dtype of q, k, v, o                                 */
  int32_t gate_dtype; /* gdn_dtype of beta|b, w, g: equal to io_dtype, or F32    */
  int32_t gate_mode;  /* gdn_gate_mode                                           */
  int32_t chunk;      /* tokens per chunk; must be 64                            */
  float scale;        /* finite; o = scale * S_t^T q_t                           */
} gdn_fwd_desc;

/*
 * gdn_chunk_fwd -- o and the final state of the recurrence above for every
 * token of a batch of sequences, computed chunkwise (64 tokens per chunk):
 * inside a chunk the cumulative channel decay is absorbed into the erase and
 * write factors and a unit lower-triangular system is solved; the fp32 state
 * is passed from chunk to chunk ("Gated DeltaNet-2", §3 "Entrainement
 * Parallele Efficace par Blocs"; "Gated DeltaNet", §Rendre l'entrainement
 * parallele).  The result equals the token-by-token recurrence up to rounding.
 *
 *   q, k       [B, T, H_k, d_k]  io_dtype
 *   v          [B, T, H_v, d_v]  io_dtype
 *   beta_or_b  SCALAR: [B, T, H_v]        CHANNEL: [B, T, H_v, d_k]   gate_dtype
 *   w          SCALAR: NULL               CHANNEL: [B, T, H_v, d_v]   gate_dtype
 *   g          same shape as beta_or_b, gate_dtype; NULL => alpha = 1
 *   state_in   [B, H_v, d_k, d_v] fp32, or NULL => zero initial state
 *   state_out  [B, H_v, d_k, d_v] fp32, or NULL => final state not stored;
 *              may equal state_in
 *   o          [B, T, H_v, d_v]  io_dtype (output; rounded to nearest even)
 *   stream     hipStream_t or NULL
 */
gdn_status gdn_chunk_fwd(const gdn_fwd_desc* desc, const void* q, const void* k,
                         const void* v, const void* beta_or_b, const void* w,
                         const void* g, const float* state_in, float* state_out,
                         void* o, void* stream);

/* Raw gate projections for gdn_chunk_fwd_gated. */
typedef struct gdn_raw_gates {
  const void* a;         /* decay projection [B*T, ld_a] gate_dtype, or NULL => alpha = 1 */
  const void* b;         /* beta|b projection [B*T, ld_b] gate_dtype                        */
  const void* w;         /* CHANNEL: write-gate projection [B*T, ld_w]; SCALAR: NULL        */
  const float* A_log;    /* [columns of a] fp32, or NULL (0)                                */
  const float* dt_bias;  /* [columns of a] fp32, or NULL (0)                                */
  int64_t ld_a, ld_b, ld_w;  /* row strides in elements (>= columns, <= 2^24)               */
} gdn_raw_gates;

/*
 * gdn_chunk_fwd_gated -- gdn_chunk_fwd with the gate activations of
 * gdn_gates applied inside the recurrence kernel, where it reads each gate
 * (the notes page "Gated DeltaNet", §Architecture et versions hybrides,
 * Figure 1: the gates come from plain projections; alpha takes the Mamba-2
 * parameterisation):
 *
 *   g = log(alpha) = -exp(A_log[j]) * softplus(a[r][j] + dt_bias[j])
 *   beta_or_b = sigmoid(b[r][j]),  w = sigmoid(w[r][j])   (CHANNEL)
 *
 * The result is that of gdn_gates followed by gdn_chunk_fwd, except that the
 * activated gates are not rounded to gate_dtype in between.  Columns per row
 * r = token: SCALAR H_v (a, b); CHANNEL H_v d_k (a, b) and H_v d_v (w), in
 * the layouts of gdn_chunk_fwd's gates; the projections are read with their
 * row strides, so they may be column blocks of one projection output.
 * Supported: io_dtype = gate_dtype = BF16, d_k = d_v = 128, equal-length
 * sequences (else GDN_ERR_UNSUPPORTED).  CHANNEL gates read a and b rows in
 * 16-byte pieces: those two need ld % 8 == 0 and 16-byte aligned pointers;
 * otherwise projections are 2-byte and A_log, dt_bias 4-byte aligned.
 * Arguments q, k, v, state_in, state_out, o, stream: as gdn_chunk_fwd.
 */
gdn_status gdn_chunk_fwd_gated(const gdn_fwd_desc* desc, const void* q, const void* k,
                               const void* v, const gdn_raw_gates* gates,
                               const float* state_in, float* state_out, void* o, void* stream);

/* Chunked forward over packed sequences of different lengths. */
typedef struct gdn_varlen_desc {
  int64_t N;          /* sequences, >= 0 (0: nothing to do)                      */
  int64_t total_T;    /* packed tokens of all sequences, >= 0                    */
  int32_t H_k, H_v;   /* >= 1, H_v % H_k == 0                                    */
  int32_t d_k, d_v;   /* each 64 or 128                                          */
  int32_t io_dtype;   /* gdn_dtype of q, k, v, o                                 */
  int32_t gate_dtype; /* equal to io_dtype, or F32                               */
  int32_t gate_mode;  /* gdn_gate_mode                                           */
  int32_t chunk;      /* must be 64                                              */
  float scale;        /* finite                                                  */
} gdn_varlen_desc;

/*
 * gdn_chunk_fwd_varlen -- gdn_chunk_fwd over N sequences packed along the
 * token axis (prefill of a serving batch).  Sequence n is the packed tokens
 * [cu_seqlens[n], cu_seqlens[n+1]); it starts from state_in[n] (or zero) and
 * leaves its final state in state_out[n], the layout gdn_decode_step updates
 * in place, so a prefill hands over to decoding without a copy.  The state is
 * what the recurrence carries from token to token, whatever the context
 * length (architecture notes page "Gated DeltaNet", §L'etat, en memoire); the
 * pages describe no batching of sequences, and this entry point is the
 * packed form of gdn_chunk_fwd with the same per-sequence result.
 *
 *   cu_seqlens [N + 1] int64, DEVICE pointer, 8-byte aligned; expected
 *              non-decreasing with cu_seqlens[0] = 0 and cu_seqlens[N] =
 *              total_T.  Each range is clamped into [0, total_T] on the
 *              device, and an empty or reversed range is a sequence of no
 *              token (its state passes through), so malformed offsets never
 *              make the kernels touch memory outside the tensors; tokens that
 *              no range covers keep their previous o.
 *   q, k       [total_T, H_k, d_k]  io_dtype
 *   v          [total_T, H_v, d_v]  io_dtype
 *   beta_or_b  SCALAR: [total_T, H_v]   CHANNEL: [total_T, H_v, d_k]  gate_dtype
 *   w          SCALAR: NULL             CHANNEL: [total_T, H_v, d_v]  gate_dtype
 *   g          same shape as beta_or_b; NULL => alpha = 1
 *   state_in   [N, H_v, d_k, d_v] fp32, or NULL => zero initial states
 *   state_out  [N, H_v, d_k, d_v] fp32, or NULL; may equal state_in
 *   o          [total_T, H_v, d_v]  io_dtype (output)
 *   stream     hipStream_t or NULL
 */
gdn_status gdn_chunk_fwd_varlen(const gdn_varlen_desc* desc, const int64_t* cu_seqlens,
                                const void* q, const void* k, const void* v,
                                const void* beta_or_b, const void* w, const void* g,
                                const float* state_in, float* state_out, void* o,
                                void* stream);

/* Single-token decode step over N independent sequences. */
typedef struct gdn_decode_desc {
  int64_t N;          /* sequences, >= 0 (0: nothing to do)                      */
  int32_t H_k, H_v;   /* >= 1, H_v % H_k == 0                                    */
  int32_t d_k, d_v;   /* each 64 or 128                                          */
  int32_t io_dtype;   /* gdn_dtype of q, k, v, o                                 */
  int32_t gate_dtype; /* equal to io_dtype, or F32                               */
  int32_t gate_mode;  /* gdn_gate_mode                                           */
  float scale;        /* finite                                                  */
} gdn_decode_desc;

/*
 * gdn_decode_step -- one step of the recurrence for one new token per
 * sequence, updating the fp32 state IN PLACE.  The state is constant-size
 * whatever the context length (architecture notes page "Gated DeltaNet",
 * §L'etat, en memoire: 128 heads x 128 x 128 fp32 per layer), so the step
 * streams the state once from and once to HBM.
 *
 *   q, k       [N, H_k, d_k]  io_dtype
 *   v          [N, H_v, d_v]  io_dtype
 *   beta_or_b  SCALAR: [N, H_v]   CHANNEL: [N, H_v, d_k]   gate_dtype
 *   w          SCALAR: NULL       CHANNEL: [N, H_v, d_v]   gate_dtype
 *   g          same shape as beta_or_b; NULL => alpha = 1
 *   state      [N, H_v, d_k, d_v] fp32, read and overwritten
 *   o          [N, H_v, d_v]  io_dtype (output)
 *   stream     hipStream_t or NULL
 */
gdn_status gdn_decode_step(const gdn_decode_desc* desc, const void* q, const void* k,
                           const void* v, const void* beta_or_b, const void* w,
                           const void* g, float* state, void* o, void* stream);

/* Gradients of the recurrence over a sequence batch. */
typedef struct gdn_bwd_desc {
  int64_t B;          /* batch, >= 0 (0: nothing to do)                          */
  int64_t T;          /* tokens per sequence, >= 0                               */
  int32_t H_k, H_v;   /* >= 1, H_v % H_k == 0                                    */
  int32_t d_k, d_v;   /* each 64 or 128                                          */
  int32_t io_dtype;   /* gdn_dtype of q, k, v, d_o                               */
  int32_t gate_dtype; /* gdn_dtype of beta|b, w, g: equal to io_dtype, or F32    */
  int32_t gate_mode;  /* gdn_gate_mode                                           */
  float scale;        /* finite; the forward's o = scale * S_t^T q_t             */
} gdn_bwd_desc;

/*
 * gdn_backward_workspace_size -- bytes of device workspace gdn_backward needs
 * for this descriptor (0 for an invalid descriptor or when there is no
 * token): the states every 16 tokens and the final state
 * (B H_v (ceil(T/16) + 1) d_k d_v elements of io_dtype), the per-token
 * vectors u (B T H_v d_v elements of io_dtype) and, unless the gates are
 * CHANNEL with H_v == H_k and d_v <= 128 (then the row gradients go straight
 * to the outputs), per-64-column partial row gradients
 * (d_v/64 * B T H_v (4 d_k + 1) fp32), each rounded up to 256 bytes.
 * 1.35 GB at B 8, T 4096, H 16, d_k = d_v = 128, bf16, channel gates.
 */
size_t gdn_backward_workspace_size(const gdn_bwd_desc* desc);

/*
 * gdn_backward -- gradients of the recurrence of gdn_chunk_fwd for upstream
 * gradients d_o (of o) and d_state_out (of the final state), i.e. of the
 * loss L = sum(o * d_o) + sum(S_T * d_state_out).  The pages give the update
 * ("Gated DeltaNet-2", Methodologie §1) and stress that training needs its
 * gate-aware gradient (§3); the gradients here are the chain rule through
 * that update, run in reverse over blocks of 16 tokens (the block form is
 * written out in backward.hip).  The kernels recompute the forward states
 * from checkpoints kept in the workspace: states and accumulation in fp32,
 * matrix-product operands and stored checkpoints in io_dtype.
 *
 *   q, k, v, beta_or_b, w, g, state_in   as for gdn_chunk_fwd (inputs)
 *   d_o          [B, T, H_v, d_v]  io_dtype
 *   d_state_out  [B, H_v, d_k, d_v] fp32, or NULL (no gradient on S_T)
 *   workspace    DEVICE, >= gdn_backward_workspace_size(desc) bytes, 16-byte
 *                aligned; owned by the caller, contents undefined on return
 *   gradients, all fp32, DEVICE, dense:
 *     dq, dk     [B, T, H_k, d_k]  (summed over the value heads of a key head)
 *     dv         [B, T, H_v, d_v]
 *     db         shape of beta_or_b (SCALAR: d beta, which also collects the
 *                write side, since b = w = beta there)
 *     dw         CHANNEL: [B, T, H_v, d_v]; SCALAR: must be NULL
 *     dg         shape of g (the gradient w.r.t. g = log alpha), or NULL;
 *                must be NULL when g is NULL
 *     d_state_in [B, H_v, d_k, d_v], or NULL; may equal d_state_out
 *   stream     hipStream_t or NULL
 * Outputs must not overlap the inputs, the workspace or each other (except
 * d_state_in == d_state_out).
 */
gdn_status gdn_backward(const gdn_bwd_desc* desc, const void* q, const void* k, const void* v,
                        const void* beta_or_b, const void* w, const void* g,
                        const float* state_in, const void* d_o, const float* d_state_out,
                        void* workspace, size_t workspace_bytes, float* dq, float* dk,
                        float* dv, float* db, float* dw, float* dg, float* d_state_in,
                        void* stream);

/*
 * gdn_backward_noalloc -- gdn_backward for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments and results, without the
 * workspace.  The workspace is a static device array inside the library,
 * gdn_backward_noalloc_max_bytes() bytes (64 MiB) on each GPU it runs on,
 * held until the process ends; the call allocates nothing.  A descriptor
 * whose gdn_backward_workspace_size exceeds that returns GDN_ERR_UNSUPPORTED
 * (for example B 1, T 1792, H 16, d_k = d_v = 128 with bf16 inputs and
 * channel gates fits; the B 8, T 4096 training shape does not).  All calls on one GPU share its array: calls that
 * overlap on one GPU (other streams or host threads) race, and must be
 * serialised by the caller.
 */
gdn_status gdn_backward_noalloc(const gdn_bwd_desc* desc, const void* q, const void* k,
                                const void* v, const void* beta_or_b, const void* w,
                                const void* g, const float* state_in, const void* d_o,
                                const float* d_state_out, float* dq, float* dk, float* dv,
                                float* db, float* dw, float* dg, float* d_state_in,
                                void* stream);

/* Bytes of the static workspace gdn_backward_noalloc uses on each GPU. */
size_t gdn_backward_noalloc_max_bytes(void);

/*
 * gdn_chunk_fwd_save -- gdn_chunk_fwd that also leaves in `workspace` what
 * gdn_backward otherwise recomputes first: the state entering every 16-token
 * block and every token's u = z - Sbar^T e (the recurrence of backward.hip),
 * so that a training step runs the recurrence forward once ("Gated
 * DeltaNet-2", Methodologie §3: the backward pass needs the forward's
 * states).  With bf16 io the chunk kernel stores them as it goes (the state
 * as bf16, the operand precision of the backward's products); with fp32 io
 * the backward's own rebuild runs after the forward.
 *
 *   desc, q, k, v, beta_or_b, w, g, state_in, state_out, o, stream
 *                 as gdn_chunk_fwd
 *   workspace     DEVICE, >= gdn_backward_workspace_size() bytes of the
 *                 gdn_bwd_desc with the same B, T, heads, dims, dtypes, gate
 *                 mode and scale; 16-byte aligned; must not overlap any
 *                 tensor of the call.  Its contents are for
 *                 gdn_backward_saved only.
 * Returns as gdn_chunk_fwd, and GDN_ERR_INVALID_ARG for a missing, short or
 * overlapping workspace.
 */
gdn_status gdn_chunk_fwd_save(const gdn_fwd_desc* desc, const void* q, const void* k,
                              const void* v, const void* beta_or_b, const void* w,
                              const void* g, const float* state_in, float* state_out, void* o,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_backward_saved -- gdn_backward for a workspace that gdn_chunk_fwd_save
 * filled for the same descriptor and the same q, k, v, gates and state_in:
 * only the reverse walk runs.  Arguments and results as gdn_backward; the
 * workspace's saved contents are read (and the rest overwritten).  A
 * workspace that does not hold them gives meaningless gradients, never an
 * access outside the arguments.
 */
gdn_status gdn_backward_saved(const gdn_bwd_desc* desc, const void* q, const void* k,
                              const void* v, const void* beta_or_b, const void* w,
                              const void* g, const float* state_in, const void* d_o,
                              const float* d_state_out, void* workspace, size_t workspace_bytes,
                              float* dq, float* dk, float* dv, float* db, float* dw, float* dg,
                              float* d_state_in, void* stream);

/* Gradients over packed sequences of different lengths. */
typedef struct gdn_bwd_varlen_desc {
  int64_t N;          /* sequences, >= 0 (0: nothing to do)                      */
  int64_t total_T;    /* packed tokens of all sequences, >= 0                    */
  int32_t H_k, H_v;   /* >= 1, H_v % H_k == 0                                    */
  int32_t d_k, d_v;   /* each 64 or 128                                          */
  int32_t io_dtype;   /* gdn_dtype of q, k, v, d_o                               */
  int32_t gate_dtype; /* equal to io_dtype, or F32                               */
  int32_t gate_mode;  /* gdn_gate_mode                                           */
  float scale;        /* finite                                                  */
} gdn_bwd_varlen_desc;

/*
 * gdn_backward_varlen_workspace_size -- workspace bytes for gdn_backward_varlen
 * (0 for an invalid descriptor or when there is no token): as for
 * gdn_backward with total_T token rows, the checkpoints taking
 * H_v (floor(total_T/16) + 2 N + 2) d_k d_v fp32.
 */
size_t gdn_backward_varlen_workspace_size(const gdn_bwd_varlen_desc* desc);

/*
 * gdn_backward_varlen -- gdn_backward over the packed sequences of
 * gdn_chunk_fwd_varlen: sequence n is the tokens [cu_seqlens[n],
 * cu_seqlens[n+1]) (device offsets, clamped on the device as for the forward;
 * malformed offsets never make the kernels touch memory outside the tensors
 * and the workspace, though their gradients are then unspecified).  The
 * result for each sequence is that of gdn_backward on it alone; an empty
 * sequence passes d_state_out[n] to d_state_in[n].
 *
 *   cu_seqlens        [N + 1] int64, DEVICE, 8-byte aligned
 *   q, k, v, gates, d_o, dq, dk, dv, db, dw, dg   [total_T, ...] packed, as
 *                     for gdn_chunk_fwd_varlen
 *   state_in, d_state_out, d_state_in             [N, H_v, d_k, d_v] fp32
 *   workspace         >= gdn_backward_varlen_workspace_size(desc) bytes
 */
gdn_status gdn_backward_varlen(const gdn_bwd_varlen_desc* desc, const int64_t* cu_seqlens,
                               const void* q, const void* k, const void* v,
                               const void* beta_or_b, const void* w, const void* g,
                               const float* state_in, const void* d_o, const float* d_state_out,
                               void* workspace, size_t workspace_bytes, float* dq, float* dk,
                               float* dv, float* db, float* dw, float* dg, float* d_state_in,
                               void* stream);

/*
 * gdn_chunk_fwd_varlen_save -- gdn_chunk_fwd_varlen that also leaves in
 * `workspace` the states and u gdn_backward_varlen_saved reads, as
 * gdn_chunk_fwd_save does for equal-length sequences.
 *
 *   desc, cu_seqlens, q, k, v, beta_or_b, w, g, state_in, state_out, o, stream
 *                 as gdn_chunk_fwd_varlen
 *   workspace     DEVICE, >= gdn_backward_varlen_workspace_size() bytes of the
 *                 gdn_bwd_varlen_desc with the same N, total_T, heads, dims,
 *                 dtypes, gate mode and scale; 16-byte aligned; must not
 *                 overlap any tensor of the call
 * Returns as gdn_chunk_fwd_varlen, and GDN_ERR_INVALID_ARG for a missing,
 * short or overlapping workspace.
 */
gdn_status gdn_chunk_fwd_varlen_save(const gdn_varlen_desc* desc, const int64_t* cu_seqlens,
                                     const void* q, const void* k, const void* v,
                                     const void* beta_or_b, const void* w, const void* g,
                                     const float* state_in, float* state_out, void* o,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_backward_varlen_saved -- gdn_backward_varlen for a workspace that
 * gdn_chunk_fwd_varlen_save filled for the same descriptor, offsets and
 * inputs: only the reverse walk runs.  Arguments and results as
 * gdn_backward_varlen; a workspace that does not hold them gives meaningless
 * gradients, never an access outside the arguments.
 */
gdn_status gdn_backward_varlen_saved(const gdn_bwd_varlen_desc* desc, const int64_t* cu_seqlens,
                                     const void* q, const void* k, const void* v,
                                     const void* beta_or_b, const void* w, const void* g,
                                     const float* state_in, const void* d_o,
                                     const float* d_state_out, void* workspace,
                                     size_t workspace_bytes, float* dq, float* dk, float* dv,
                                     float* db, float* dw, float* dg, float* d_state_in,
                                     void* stream);

/* ------------------------------------------------------------------------
 * The operations around the recurrence in a Gated DeltaNet block (notes page
 * "Gated DeltaNet", §Architecture et versions hybrides, Figure 1 right-hand
 * block): q, k, v pass through a short convolution and SiLU, q and k are
 * then L2-normalised; alpha and beta come from a plain projection, alpha
 * with the Mamba-2 parameterisation; the recurrence output is normalised and
 * multiplied by a gate branch.  The projections themselves are plain GEMMs
 * and are not part of this library.  The pages leave the exact forms open;
 * the ones computed here are stated with each entry point.
 * ------------------------------------------------------------------------ */

/* Short causal convolution of the q, k, v branch. */
typedef struct gdn_conv_desc {
  int64_t N;          /* sequences, >= 0 (0: nothing to do)                      */
  int64_t total_T;    /* packed tokens = rows of x, >= 0                         */
  int64_t ld_x;       /* elements from one row of x to the next: >= C, % 8 == 0  */
  int32_t H_k, H_v;   /* >= 1                                                    */
  int32_t d_k, d_v;   /* each 64 or 128                                          */
  int32_t io_dtype;   /* gdn_dtype of x, the conv states, q, k, v                */
  float eps;          /* L2-norm epsilon, finite, >= 0                           */
} gdn_conv_desc;

/*
 * gdn_short_conv -- the q, k, v branch: a depthwise causal convolution of
 * kernel 4 along the tokens of each sequence (architecture notes page "Gated
 * DeltaNet", §La convolution causale: a token's output combines its own
 * input with those of the three tokens before it; the notes count 4 weights
 * per channel, so there is no bias), SiLU, and for q and k an L2
 * norm over the d_k channels of each head.  With C = 2 H_k d_k + H_v d_v and
 * u the conv input of one channel,
 *
 *   a_t   = w[c][0] u_{t-3} + w[c][1] u_{t-2} + w[c][2] u_{t-1} + w[c][3] u_t
 *   v_t   = silu(a_t)                        silu(x) = x / (1 + e^-x)
 *   q_t   = silu(a_t) / sqrt(sum_head silu(a_t)^2 + eps)     (same for k)
 *
 * where u_{t-j} before a sequence's first token is the carried conv state
 * (the sequence's 3 previous inputs) or 0.
 *
 *   cu_seqlens      [N + 1] int64 DEVICE offsets of packed sequences (as in
 *                   gdn_chunk_fwd_varlen, clamped on the device), or NULL for
 *                   N sequences of total_T / N tokens (total_T % N == 0)
 *   x               [total_T, ld_x] io_dtype; columns [0, H_k d_k) are q, the
 *                   next H_k d_k are k, the next H_v d_v are v; later columns
 *                   (e.g. the output-gate branch) are not read
 *   conv_w          [C, 4] fp32; tap 3 multiplies the current token
 *   conv_state_in   [N, 3, C] io_dtype, oldest input first, or NULL (zeros)
 *   conv_state_out  [N, 3, C] io_dtype, or NULL; receives each sequence's
 *                   last 3 inputs (the older carried entries where a sequence
 *                   is shorter); may equal conv_state_in
 *   q, k            [total_T, H_k, d_k]  io_dtype (outputs)
 *   v               [total_T, H_v, d_v]  io_dtype (output)
 *   stream          hipStream_t or NULL
 * A decode step is the same call with one token per sequence and the state
 * updated in place.  Pointers are 16-byte aligned (conv_w too).
 */
gdn_status gdn_short_conv(const gdn_conv_desc* desc, const int64_t* cu_seqlens,
                          const void* x, const float* conv_w, const void* conv_state_in,
                          void* conv_state_out, void* q, void* k, void* v, void* stream);

/* Gate activations. */
typedef struct gdn_gate_desc {
  int64_t rows;       /* tokens, >= 0                                            */
  int64_t ld_a, ld_b; /* row strides (elements) of a_raw and b_raw, >= columns   */
  int64_t ld_w;       /* row stride of w_raw (CHANNEL), >= H_v d_v               */
  int32_t H_v;        /* >= 1                                                    */
  int32_t d_k, d_v;   /* >= 1 (CHANNEL only; ignored for SCALAR)                 */
  int32_t gate_mode;  /* gdn_gate_mode                                           */
  int32_t in_dtype;   /* gdn_dtype of the raw projections                        */
  int32_t gate_dtype; /* gdn_dtype of g, beta_or_b, w                            */
} gdn_gate_desc;

/*
 * gdn_gates -- gate activations from the raw projections.  The notes page
 * "Gated DeltaNet" (§Architecture et versions hybrides) gives alpha the
 * Mamba-2 parameterisation and the architecture notes page (§La recurrence)
 * puts alpha and beta in ]0,1[; computed here, per column j:
 *
 *   g[r][j]         = log(alpha) = -exp(A_log[j]) * softplus(a_raw[r][j] + dt_bias[j])
 *   beta_or_b[r][j] = sigmoid(b_raw[r][j])
 *   w[r][j]         = sigmoid(w_raw[r][j])          (CHANNEL: the GDN-2 write gate)
 *
 * in the layouts gdn_chunk_fwd and gdn_decode_step take.  Columns: SCALAR
 * H_v (a, b); CHANNEL H_v d_k (a, b) and H_v d_v (w).  The raw inputs are
 * read with row strides, so they may be column blocks of one projection
 * output; outputs are dense.
 *
 *   a_raw, b_raw   [rows, ld_a], [rows, ld_b]  in_dtype
 *   w_raw          [rows, ld_w] in_dtype (CHANNEL), NULL for SCALAR
 *   A_log, dt_bias [columns of a] fp32, or NULL (0)
 *   g, beta_or_b   [rows, columns of a] gate_dtype (outputs)
 *   w              [rows, H_v d_v] gate_dtype (CHANNEL output), NULL for SCALAR
 * Pointers are aligned to their element size; rows * columns < 2^32.
 */
gdn_status gdn_gates(const gdn_gate_desc* desc, const void* a_raw, const void* b_raw,
                     const void* w_raw, const float* A_log, const float* dt_bias, void* g,
                     void* beta_or_b, void* w, void* stream);

/* Output normalisation and gate. */
typedef struct gdn_norm_desc {
  int64_t rows;       /* tokens, >= 0                                            */
  int64_t ld_z;       /* elements from one row of z to the next: >= H_v d_v, % 8 == 0 */
  int32_t H_v;        /* >= 1                                                    */
  int32_t d_v;        /* 64 or 128                                               */
  int32_t io_dtype;   /* gdn_dtype of o, z, y                                    */
  float eps;          /* finite, >= 0                                            */
} gdn_norm_desc;

/*
 * gdn_output_gate -- the block's output: each value head's recurrence output
 * normalised, then multiplied by swish of the gate branch z (notes page
 * "Gated DeltaNet", Figure 1; architecture notes page, §La porte de sortie:
 * y = o (.) swish(z), swish(x) = x sigmoid(x)).  The norm is an RMS norm over
 * the d_v channels with one weight vector shared by all heads (the
 * architecture notes count d_v normalisation parameters per layer):
 *
 *   y[r][h][:] = o[r][h][:] / sqrt(mean(o[r][h][:]^2) + eps) * weight[:] * swish(z[r][h][:])
 *
 *   o       [rows, H_v, d_v] io_dtype
 *   z       [rows, ld_z] io_dtype; columns [h d_v, (h+1) d_v) gate head h
 *   weight  [d_v] fp32
 *   y       [rows, H_v, d_v] io_dtype (output); may equal o
 * Pointers are 16-byte aligned.
 */
gdn_status gdn_output_gate(const gdn_norm_desc* desc, const void* o, const void* z,
                           const float* weight, void* y, void* stream);

/* Self-test of the debug build libgdn_check.so (not an operation of the
 * method: it proves that build's LDS checks fire).  One small kernel on
 * `stream` writes to out64 (64 fp32, device memory, caller-owned) what it
 * reads from LDS that it never wrote, and computes (without making) one
 * address past the end of its LDS per lane, which the check must count.
 * Returns GDN_OK when the count is exactly 64 (the caller then expects
 * out64 to hold NaN, the fill pattern), GDN_ERR_CHECK otherwise; waits for
 * the kernel.  NULL out64: GDN_ERR_INVALID_ARG.  The normal libgdn.so
 * returns GDN_ERR_UNSUPPORTED and touches nothing. */
gdn_status gdn_check_selftest(float* out64, void* stream);

/* Static, never-NULL description of a status code. */
const char* gdn_status_string(gdn_status s);

/* Returns GDN_ABI_VERSION of the loaded library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
