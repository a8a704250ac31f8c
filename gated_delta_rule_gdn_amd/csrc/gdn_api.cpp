// gdn_api.cpp -- the C ABI of libgdn.so (declared in include/gdn.h).
//
// Every argument is validated on the host before anything is enqueued; on a
// validation error nothing is launched and no output is touched.  The layer
// then fills a plain launch struct and hands it to the kernel translation
// unit, which launches on the caller's stream.
#include "gdn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>

#include "gdn_kernels.hpp"

namespace {

// Status of a call whose launches returned e.  The debug build (-DGDN_CHECK)
// also waits for the work to finish and reads the kernels' LDS-check
// counters (all modules, so that they are reset for the next call).
gdn_status launched(hipError_t e) {
  if (e != hipSuccess) return GDN_ERR_HIP;
#ifdef GDN_CHECK
  const unsigned long long v = (unsigned long long)gdn::check_violations_decode() +
                               gdn::check_violations_chunk() + gdn::check_violations_chunk_sb() +
                               gdn::check_violations_backward();
  if (v != 0) {
    fprintf(stderr, "libgdn_check: %llu LDS accesses outside the layout\n", v);
    return GDN_ERR_CHECK;
  }
#endif
  return GDN_OK;
}

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
  bool valid() const { return hi > lo; }
};

Span span(const void* p, int64_t elems, int64_t elem_bytes) {
  Span s{0, 0};
  if (p && elems > 0) {
    s.lo = reinterpret_cast<uintptr_t>(p);
    s.hi = s.lo + static_cast<uintptr_t>(elems * elem_bytes);
  }
  return s;
}

bool overlaps(const Span& a, const Span& b) {
  return a.valid() && b.valid() && a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t dtype_bytes(int32_t d) { return d == GDN_F32 ? 4 : 2; }

// Common shape/type checks shared by both entry points.
gdn_status check_common(int32_t Hk, int32_t Hv, int32_t dk, int32_t dv, int32_t io,
                        int32_t gate, int32_t mode, float scale) {
  if (Hk < 1 || Hv < 1 || Hv % Hk != 0) return GDN_ERR_INVALID_ARG;
  if (io != GDN_F32 && io != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (gate != GDN_F32 && gate != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (mode != GDN_GATES_SCALAR && mode != GDN_GATES_CHANNEL) return GDN_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return GDN_ERR_INVALID_ARG;
  if (dk < 1 || dv < 1) return GDN_ERR_INVALID_ARG;
  if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return GDN_ERR_UNSUPPORTED;
  // Token rows of at most 2^22 elements (the kernels address a 64-token chunk
  // of any tensor with 32-bit byte offsets).
  if ((int64_t)Hk * dk > (int64_t(1) << 22) || (int64_t)Hv * dv > (int64_t(1) << 22))
    return GDN_ERR_UNSUPPORTED;
  // Gate storage must match the io type or be fp32; fp32 io with bf16 gates
  // is not built.
  if (!(gate == io || gate == GDN_F32)) return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

gdn::DType to_dtype(int32_t d) { return d == GDN_F32 ? gdn::DType::F32 : gdn::DType::BF16; }

// Checks pointer presence, alignment and overlap.  `rows` is the number of
// (token, head)-independent rows of the leading dims: B*T for the forward,
// N for decode.
gdn_status check_pointers(int64_t rows, int64_t heads_state, int32_t Hk, int32_t Hv,
                          int32_t dk, int32_t dv, int32_t io, int32_t gate, int32_t mode,
                          const void* q, const void* k, const void* v, const void* b,
                          const void* w, const void* g, const float* s_in, const float* s_out,
                          const void* o, bool decode) {
  if (!q || !k || !v || !b || !o) return GDN_ERR_INVALID_ARG;
  if (mode == GDN_GATES_CHANNEL && !w) return GDN_ERR_INVALID_ARG;
  if (mode == GDN_GATES_SCALAR && w) return GDN_ERR_INVALID_ARG;
  if (decode && !s_in) return GDN_ERR_INVALID_ARG;
  const void* all[] = {q, k, v, b, w, g, s_in, s_out, o};
  for (const void* p : all)
    if (p && !aligned16(p)) return GDN_ERR_INVALID_ARG;

  const int64_t ib = dtype_bytes(io), gb = dtype_bytes(gate);
  const bool ch = mode == GDN_GATES_CHANNEL;
  const Span sq = span(q, rows * Hk * dk, ib);
  const Span sk = span(k, rows * Hk * dk, ib);
  const Span sv = span(v, rows * Hv * dv, ib);
  const Span sb = span(b, rows * Hv * (ch ? dk : 1), gb);
  const Span sw = span(w, rows * Hv * dv, gb);
  const Span sg = span(g, rows * Hv * (ch ? dk : 1), gb);
  const Span si = span(s_in, heads_state * dk * dv, 4);
  const Span so = span(s_out, heads_state * dk * dv, 4);
  const Span sO = span(o, rows * Hv * dv, ib);
  const Span inputs[] = {sq, sk, sv, sb, sw, sg, si};
  // o must not overlap any input nor the state output.
  for (const Span& in : inputs)
    if (overlaps(sO, in)) return GDN_ERR_INVALID_ARG;
  if (overlaps(sO, so)) return GDN_ERR_INVALID_ARG;
  // state_out may equal state_in exactly, and must not overlap anything else.
  if (!decode && so.valid()) {
    const Span others[] = {sq, sk, sv, sb, sw, sg};
    for (const Span& in : others)
      if (overlaps(so, in)) return GDN_ERR_INVALID_ARG;
    if (si.valid() && overlaps(so, si) && !(si.lo == so.lo && si.hi == so.hi))
      return GDN_ERR_INVALID_ARG;
  }
  if (decode) {  // the state is read and written in place
    const Span others[] = {sq, sk, sv, sb, sw, sg};
    for (const Span& in : others)
      if (overlaps(si, in)) return GDN_ERR_INVALID_ARG;
  }
  return GDN_OK;
}

}  // namespace

namespace {

struct BwdLayout {
  int64_t nblk, slots, ckpt_elems, u_elems, part_floats;
  bool direct;   // row gradients written straight to the outputs, no partials
  size_t ckpt_off, u_off, part_off, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// What the backward runs on: N sequences over `rows` token rows, either of T
// tokens each (cu == nullptr) or packed by the device offsets cu.
struct BwdShape {
  int64_t N, rows, T;
  const int64_t* cu;
  int32_t Hk, Hv, dk, dv, io, gate, mode;
  float scale;
};

BwdLayout bwd_layout(const BwdShape& d) {
  BwdLayout L;
  const int64_t hrows = d.rows * d.Hv;
  const int64_t ncb = d.dv / 64;
  L.nblk = d.cu ? 0 : gdn::bwd_checkpoint_blocks(d.T);
  // packed sequences: sequence n uses slots floor(start/16) + 2n onwards
  L.slots = d.cu ? d.rows / 16 + 2 * d.N + 2 : d.N * (L.nblk + 1);
  // checkpoints and u are kept in the io type (the matrix-product operand type)
  const size_t eb = d.io == GDN_BF16 ? 2 : 4;
  L.ckpt_elems = (int64_t)d.Hv * L.slots * d.dk * d.dv;
  L.u_elems = hrows * d.dv;
  L.direct = d.mode == GDN_GATES_CHANNEL && d.Hv == d.Hk && ncb <= 2;
  L.part_floats = L.direct ? 0 : ncb * 4 * hrows * d.dk + ncb * hrows;
  L.ckpt_off = 0;
  L.u_off = align256((size_t)L.ckpt_elems * eb);
  L.part_off = L.u_off + align256((size_t)L.u_elems * eb);
  L.total = L.part_off + align256((size_t)L.part_floats * 4);
  return L;
}

gdn_status check_bwd_shape(const BwdShape& d) {
  if (d.N < 0 || d.rows < 0 || d.T < 0) return GDN_ERR_INVALID_ARG;
  if ((double)d.T > 2.0e9 || (double)d.rows > 2.0e9) return GDN_ERR_UNSUPPORTED;
  gdn_status st = check_common(d.Hk, d.Hv, d.dk, d.dv, d.io, d.gate, d.mode, d.scale);
  if (st != GDN_OK) return st;
  const double elems = (double)d.rows * (double)d.Hv * (double)(4 * d.dk + 2 * d.dv + 2);
  const double ck = (double)d.Hv * ((double)d.rows / 16.0 + 2.0 * (double)d.N + 2.0) *
                    (double)d.dk * (double)d.dv;
  if (elems > 2.0e15 || ck > 2.0e15) return GDN_ERR_INVALID_ARG;
  if ((double)d.N * (double)d.Hv > 2.0e9 || (double)d.rows > 2.0e9)
    return GDN_ERR_UNSUPPORTED;  // grid sizes
  return GDN_OK;
}

BwdShape shape_of(const gdn_bwd_desc* d) {
  // rows = B T, or -1 (rejected by check_bwd_shape) when a factor is negative
  // or the product overflows
  int64_t rows = -1;
  if (d->B >= 0 && d->T >= 0 && __builtin_mul_overflow(d->B, d->T, &rows)) rows = -1;
  if (d->B < 0 || d->T < 0) rows = -1;
  return BwdShape{d->B, rows, d->T, nullptr, d->H_k, d->H_v, d->d_k, d->d_v,
                  d->io_dtype, d->gate_dtype, d->gate_mode, d->scale};
}
BwdShape shape_of(const gdn_bwd_varlen_desc* d, const int64_t* cu) {
  return BwdShape{d->N, d->total_T, 0, cu, d->H_k, d->H_v, d->d_k, d->d_v,
                  d->io_dtype, d->gate_dtype, d->gate_mode, d->scale};
}

gdn_status run_backward(const BwdShape& d, const void* q, const void* k, const void* v,
                        const void* beta_or_b, const void* w, const void* g,
                        const float* state_in, const void* d_o, const float* d_state_out,
                        void* workspace, size_t workspace_bytes, float* dq, float* dk,
                        float* dv, float* db, float* dw, float* dg, float* d_state_in,
                        void* stream, int phases = 3) {
  gdn_status st = check_bwd_shape(d);
  if (st != GDN_OK) return st;
  if (d.N == 0) return GDN_OK;
  const int64_t heads = d.N * d.Hv;
  const int64_t S = heads * d.dk * d.dv;
  const Span sdsi = span(d_state_in, S, 4), sdso = span(d_state_out, S, 4);
  if ((d_state_in && !aligned16(d_state_in)) || (d_state_out && !aligned16(d_state_out)))
    return GDN_ERR_INVALID_ARG;
  if (overlaps(sdsi, sdso) && !(sdsi.lo == sdso.lo && sdsi.hi == sdso.hi))
    return GDN_ERR_INVALID_ARG;
  const Span scu = span(d.cu, d.N + 1, 8);
  if (d.cu && ((reinterpret_cast<uintptr_t>(d.cu) & 7u) != 0 || overlaps(scu, sdsi)))
    return GDN_ERR_INVALID_ARG;
  if (d.rows == 0) {
    // No token: the gradient only passes from the final to the initial state.
    if (!d_state_in || d_state_in == d_state_out) return GDN_OK;
    hipError_t e = gdn::launch_state_copy(d_state_out, d_state_in, S,
                                          static_cast<hipStream_t>(stream));
    return launched(e);
  }
  const int64_t rows = d.rows;
  st = check_pointers(rows, heads, d.Hk, d.Hv, d.dk, d.dv, d.io, d.gate, d.mode, q, k, v,
                      beta_or_b, w, g, state_in, nullptr, d_o, false);
  if (st != GDN_OK) return st;
  const bool ch = d.mode == GDN_GATES_CHANNEL;
  if (!dq || !dk || !dv || !db) return GDN_ERR_INVALID_ARG;
  if (ch != (dw != nullptr)) return GDN_ERR_INVALID_ARG;
  if (dg && !g) return GDN_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace)) return GDN_ERR_INVALID_ARG;
  const BwdLayout L = bwd_layout(d);
  if (workspace_bytes < L.total) return GDN_ERR_INVALID_ARG;
  const float* outs[] = {dq, dk, dv, db, dw, dg, d_state_in};
  for (const float* p : outs)
    if (p && !aligned16(p)) return GDN_ERR_INVALID_ARG;
  // outputs: no overlap with inputs, the workspace or each other
  const int64_t ib = dtype_bytes(d.io), gb = dtype_bytes(d.gate);
  const int64_t gcols = ch ? d.dk : 1;
  const Span in_sp[] = {
      span(q, rows * d.Hk * d.dk, ib), span(k, rows * d.Hk * d.dk, ib),
      span(v, rows * d.Hv * d.dv, ib), span(beta_or_b, rows * d.Hv * gcols, gb),
      span(w, rows * d.Hv * d.dv, gb), span(g, rows * d.Hv * gcols, gb),
      span(state_in, S, 4), span(d_o, rows * d.Hv * d.dv, ib), sdso, scu,
      span(workspace, (int64_t)L.total, 1)};
  const Span out_sp[] = {
      span(dq, rows * d.Hk * d.dk, 4), span(dk, rows * d.Hk * d.dk, 4),
      span(dv, rows * d.Hv * d.dv, 4), span(db, rows * d.Hv * gcols, 4),
      span(dw, rows * d.Hv * d.dv, 4), span(dg, rows * d.Hv * gcols, 4), sdsi};
  const int n_out = sizeof(out_sp) / sizeof(out_sp[0]);
  for (int i = 0; i < n_out; ++i) {
    for (const Span& in : in_sp) {
      if (i == n_out - 1 && in.lo == sdso.lo && in.hi == sdso.hi && sdso.valid()) continue;
      if (overlaps(out_sp[i], in)) return GDN_ERR_INVALID_ARG;
    }
    for (int j = i + 1; j < n_out; ++j)
      if (overlaps(out_sp[i], out_sp[j])) return GDN_ERR_INVALID_ARG;
  }
  if (workspace_bytes && overlaps(span(workspace, (int64_t)L.total, 1), scu))
    return GDN_ERR_INVALID_ARG;

  gdn::BwdArgs a;
  a.B = d.N; a.T = d.T; a.cu = d.cu; a.rows = rows; a.slots = L.slots;
  a.Hk = d.Hk; a.Hv = d.Hv; a.dk = d.dk; a.dv = d.dv;
  a.io = to_dtype(d.io); a.gate = to_dtype(d.gate); a.channel = ch;
  a.scale = d.scale;
  a.q = q; a.k = k; a.v = v; a.b = beta_or_b; a.w = w; a.g = g; a.d_o = d_o;
  a.state_in = state_in; a.d_state_out = d_state_out;
  char* ws = static_cast<char*>(workspace);
  a.ckpt = ws + L.ckpt_off;
  a.u = ws + L.u_off;
  a.part = reinterpret_cast<float*>(ws + L.part_off);
  a.direct = L.direct;
  a.nblk = L.nblk;
  a.dq_out = dq; a.dk_out = dk; a.dv_out = dv; a.db = db; a.dw = dw; a.dg = dg;
  a.d_state_in = d_state_in;
  a.phases = phases;
  hipError_t e = gdn::launch_backward(a, static_cast<hipStream_t>(stream));
  return launched(e);
}

// Checks of gdn_chunk_fwd's descriptor that come before any pointer is read.
gdn_status check_fwd_desc(const gdn_fwd_desc* d) {
  if (!d) return GDN_ERR_INVALID_ARG;
  if (d->B < 0 || d->T < 0) return GDN_ERR_INVALID_ARG;
  gdn_status st = check_common(d->H_k, d->H_v, d->d_k, d->d_v, d->io_dtype, d->gate_dtype,
                               d->gate_mode, d->scale);
  if (st != GDN_OK) return st;
  if (d->chunk != 64) return GDN_ERR_UNSUPPORTED;
  // Guard index arithmetic: every element count must fit comfortably in int64.
  const double elems = (double)d->B * (double)d->T * (double)d->H_v * (double)(d->d_k + d->d_v);
  if (elems > 9.0e15) return GDN_ERR_INVALID_ARG;
  if ((double)d->T > 2.0e9) return GDN_ERR_UNSUPPORTED;
  if ((double)d->B * (double)d->H_v * 2.0 > 2.0e9) return GDN_ERR_UNSUPPORTED;  // grid size
  return GDN_OK;
}

// The chunk forward over the shape bs (equal-length or packed by bs.cu) with
// the backward's checkpoints and u left in `workspace`; the forward's own
// argument checks have passed.  The bf16 chunk kernel stores them as it goes;
// other configurations run the backward's forward rebuild after the forward.
gdn_status run_fwd_save(const BwdShape& bs, const void* q, const void* k, const void* v,
                        const void* beta_or_b, const void* w, const void* g,
                        const float* state_in, float* state_out, void* o, void* workspace,
                        size_t workspace_bytes, void* stream) {
  gdn_status st = check_bwd_shape(bs);
  if (st != GDN_OK) return st;
  const BwdLayout L = bwd_layout(bs);
  if (!workspace || !aligned16(workspace) || workspace_bytes < L.total) return GDN_ERR_INVALID_ARG;
  // the workspace is written: it overlaps no tensor of the call
  const int64_t rows = bs.rows, heads = bs.N * bs.Hv;
  const int64_t ib = dtype_bytes(bs.io), gb = dtype_bytes(bs.gate);
  const int64_t gcols = bs.mode == GDN_GATES_CHANNEL ? bs.dk : 1;
  const int64_t S = heads * bs.dk * bs.dv;
  const Span sws = span(workspace, (int64_t)L.total, 1);
  const Span all[] = {span(q, rows * bs.Hk * bs.dk, ib), span(k, rows * bs.Hk * bs.dk, ib),
                      span(v, rows * bs.Hv * bs.dv, ib), span(beta_or_b, rows * bs.Hv * gcols, gb),
                      span(w, rows * bs.Hv * bs.dv, gb), span(g, rows * bs.Hv * gcols, gb),
                      span(state_in, S, 4), span(state_out, S, 4),
                      span(o, rows * bs.Hv * bs.dv, ib), span(bs.cu, bs.N + 1, 8)};
  for (const Span& x : all)
    if (overlaps(sws, x)) return GDN_ERR_INVALID_ARG;

  gdn::ChunkArgs a;
  a.B = bs.N; a.T = bs.cu ? rows : bs.T; a.cu_seqlens = bs.cu;
  a.Hk = bs.Hk; a.Hv = bs.Hv; a.dk = bs.dk; a.dv = bs.dv;
  a.io = to_dtype(bs.io); a.gate = to_dtype(bs.gate);
  a.channel = bs.mode == GDN_GATES_CHANNEL; a.scale = bs.scale;
  a.q = q; a.k = k; a.v = v; a.b = beta_or_b; a.w = w; a.g = g;
  a.state_in = state_in; a.state_out = state_out; a.o = o;
  char* ws = static_cast<char*>(workspace);
  const bool in_kernel = bs.io == GDN_BF16;
  if (in_kernel) {
    a.ck = ws + L.ckpt_off;
    a.u = ws + L.u_off;
    a.ck_slots = L.slots;
    a.ck_nblk = L.nblk;
  }
  hipError_t e = gdn::launch_chunk_fwd(a, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return GDN_ERR_UNSUPPORTED;
  if (e != hipSuccess) return GDN_ERR_HIP;
  if (in_kernel) return GDN_OK;
  gdn::BwdArgs b;
  b.B = bs.N; b.T = bs.T; b.cu = bs.cu; b.rows = rows; b.slots = L.slots;
  b.Hk = bs.Hk; b.Hv = bs.Hv; b.dk = bs.dk; b.dv = bs.dv;
  b.io = a.io; b.gate = a.gate; b.channel = a.channel; b.scale = bs.scale;
  b.q = q; b.k = k; b.v = v; b.b = beta_or_b; b.w = w; b.g = g; b.d_o = nullptr;
  b.state_in = state_in; b.d_state_out = nullptr;
  b.ckpt = ws + L.ckpt_off; b.u = ws + L.u_off;
  b.part = reinterpret_cast<float*>(ws + L.part_off);
  b.direct = L.direct;
  b.phases = 1;
  b.nblk = L.nblk;
  b.dq_out = b.dk_out = b.dv_out = b.db = b.dw = b.dg = b.d_state_in = nullptr;
  e = gdn::launch_backward(b, static_cast<hipStream_t>(stream));
  return launched(e);
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "GDN_OK: success";
    case GDN_ERR_INVALID_ARG: return "GDN_ERR_INVALID_ARG: invalid argument";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: configuration not supported";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: HIP runtime error at launch";
    case GDN_ERR_CHECK: return "GDN_ERR_CHECK: LDS access outside the kernel's layout (debug build)";
  }
  return "GDN_ERR_UNKNOWN: unknown status code";
}

gdn_status gdn_chunk_fwd(const gdn_fwd_desc* d, const void* q, const void* k, const void* v,
                         const void* beta_or_b, const void* w, const void* g,
                         const float* state_in, float* state_out, void* o, void* stream) {
  gdn_status st = check_fwd_desc(d);
  if (st != GDN_OK) return st;
  if (d->B == 0) return GDN_OK;  // nothing to read or write
  const int64_t rows = d->B * d->T;
  const int64_t heads = d->B * d->H_v;
  if (d->T == 0) {
    // No token: only the state passes through (o is empty).
    if (state_out && state_in && state_out != state_in) {
      const Span si = span(state_in, heads * d->d_k * d->d_v, 4);
      const Span so = span(state_out, heads * d->d_k * d->d_v, 4);
      if (overlaps(si, so)) return GDN_ERR_INVALID_ARG;
    }
    if ((state_in && !aligned16(state_in)) || (state_out && !aligned16(state_out)))
      return GDN_ERR_INVALID_ARG;
    if (!state_out || state_out == state_in) return GDN_OK;
    hipError_t e = gdn::launch_state_copy(state_in, state_out, heads * d->d_k * d->d_v,
                                          static_cast<hipStream_t>(stream));
    return launched(e);
  }
  st = check_pointers(rows, heads, d->H_k, d->H_v, d->d_k, d->d_v, d->io_dtype, d->gate_dtype,
                      d->gate_mode, q, k, v, beta_or_b, w, g, state_in, state_out, o, false);
  if (st != GDN_OK) return st;

  gdn::ChunkArgs a;
  a.B = d->B; a.T = d->T; a.Hk = d->H_k; a.Hv = d->H_v; a.dk = d->d_k; a.dv = d->d_v;
  a.io = to_dtype(d->io_dtype); a.gate = to_dtype(d->gate_dtype);
  a.channel = d->gate_mode == GDN_GATES_CHANNEL; a.scale = d->scale;
  a.q = q; a.k = k; a.v = v; a.b = beta_or_b; a.w = w; a.g = g;
  a.state_in = state_in; a.state_out = state_out; a.o = o;
  hipError_t e = gdn::launch_chunk_fwd(a, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return GDN_ERR_UNSUPPORTED;
  return launched(e);
}

gdn_status gdn_chunk_fwd_save(const gdn_fwd_desc* d, const void* q, const void* k,
                              const void* v, const void* beta_or_b, const void* w, const void* g,
                              const float* state_in, float* state_out, void* o, void* workspace,
                              size_t workspace_bytes, void* stream) {
  gdn_status st = check_fwd_desc(d);
  if (st != GDN_OK) return st;
  if (d->B == 0 || d->T == 0)   // nothing for a backward to read
    return gdn_chunk_fwd(d, q, k, v, beta_or_b, w, g, state_in, state_out, o, stream);
  const int64_t rows = d->B * d->T, heads = d->B * d->H_v;
  st = check_pointers(rows, heads, d->H_k, d->H_v, d->d_k, d->d_v, d->io_dtype, d->gate_dtype,
                      d->gate_mode, q, k, v, beta_or_b, w, g, state_in, state_out, o, false);
  if (st != GDN_OK) return st;
  const BwdShape bs{d->B, rows, d->T, nullptr, d->H_k, d->H_v, d->d_k, d->d_v,
                    d->io_dtype, d->gate_dtype, d->gate_mode, d->scale};
  return run_fwd_save(bs, q, k, v, beta_or_b, w, g, state_in, state_out, o, workspace,
                      workspace_bytes, stream);
}

gdn_status gdn_chunk_fwd_gated(const gdn_fwd_desc* d, const void* q, const void* k, const void* v,
                               const gdn_raw_gates* gt, const float* state_in, float* state_out,
                               void* o, void* stream) {
  if (!d || !gt) return GDN_ERR_INVALID_ARG;
  if (d->B < 0 || d->T < 0) return GDN_ERR_INVALID_ARG;
  gdn_status st = check_common(d->H_k, d->H_v, d->d_k, d->d_v, d->io_dtype, d->gate_dtype,
                               d->gate_mode, d->scale);
  if (st != GDN_OK) return st;
  if (d->chunk != 64) return GDN_ERR_UNSUPPORTED;
  if (d->io_dtype != GDN_BF16 || d->gate_dtype != GDN_BF16 || d->d_k != 128 || d->d_v != 128)
    return GDN_ERR_UNSUPPORTED;
  const double elems = (double)d->B * (double)d->T * (double)d->H_v * (double)(d->d_k + d->d_v);
  if (elems > 9.0e15) return GDN_ERR_INVALID_ARG;
  if ((double)d->T > 2.0e9) return GDN_ERR_UNSUPPORTED;
  if ((double)d->B * (double)d->H_v * 2.0 > 2.0e9) return GDN_ERR_UNSUPPORTED;  // grid size
  const bool ch = d->gate_mode == GDN_GATES_CHANNEL;
  const int64_t ncol = ch ? (int64_t)d->H_v * d->d_k : d->H_v;   // columns of a and b
  const int64_t nw = (int64_t)d->H_v * d->d_v;                     // columns of w
  if (!gt->b || (ch ? !gt->w : gt->w != nullptr)) return GDN_ERR_INVALID_ARG;
  if (gt->ld_b < ncol || (gt->a && gt->ld_a < ncol) || (ch && gt->ld_w < nw))
    return GDN_ERR_INVALID_ARG;
  // a 64-token chunk of a projection is addressed with 32-bit byte offsets
  const int64_t ld_max = int64_t(1) << 24;
  if (gt->ld_b > ld_max || gt->ld_a > ld_max || gt->ld_w > ld_max) return GDN_ERR_UNSUPPORTED;
  // channel gates: a and b rows are read in 16-byte pieces
  if (ch && ((gt->ld_b % 8) != 0 || !aligned16(gt->b) ||
             (gt->a && ((gt->ld_a % 8) != 0 || !aligned16(gt->a)))))
    return GDN_ERR_INVALID_ARG;
  auto al2 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; };
  auto al4 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; };
  if (!al2(gt->b) || (gt->a && !al2(gt->a)) || (gt->w && !al2(gt->w))) return GDN_ERR_INVALID_ARG;
  if ((gt->A_log && !al4(gt->A_log)) || (gt->dt_bias && !al4(gt->dt_bias)))
    return GDN_ERR_INVALID_ARG;
  if (d->B == 0) return GDN_OK;
  const int64_t rows = d->B * d->T;
  const int64_t heads = d->B * d->H_v;
  const int64_t nstate = heads * d->d_k * d->d_v;
  if ((state_in && !aligned16(state_in)) || (state_out && !aligned16(state_out)))
    return GDN_ERR_INVALID_ARG;
  const Span si = span(state_in, nstate, 4), so = span(state_out, nstate, 4);
  if (si.valid() && overlaps(so, si) && !(si.lo == so.lo && si.hi == so.hi))
    return GDN_ERR_INVALID_ARG;
  if (d->T == 0) {
    if (!state_out || state_out == state_in) return GDN_OK;
    hipError_t e = gdn::launch_state_copy(state_in, state_out, nstate,
                                          static_cast<hipStream_t>(stream));
    return launched(e);
  }
  if (!q || !k || !v || !o) return GDN_ERR_INVALID_ARG;
  const void* a16[] = {q, k, v, o};
  for (const void* p : a16)
    if (!aligned16(p)) return GDN_ERR_INVALID_ARG;
  // row-strided projections: from the first element to the last row's end
  auto pspan = [&](const void* p, int64_t ld, int64_t cols) {
    return span(p, p ? (rows - 1) * ld + cols : 0, 2);
  };
  const Span sq = span(q, rows * d->H_k * d->d_k, 2), sk = span(k, rows * d->H_k * d->d_k, 2);
  const Span sv = span(v, rows * d->H_v * d->d_v, 2), sO = span(o, rows * d->H_v * d->d_v, 2);
  const Span sa = pspan(gt->a, gt->ld_a, ncol), sb = pspan(gt->b, gt->ld_b, ncol);
  const Span sw = pspan(gt->w, gt->ld_w, nw);
  const Span sA = span(gt->A_log, ncol, 4), sD = span(gt->dt_bias, ncol, 4);
  const Span inputs[] = {sq, sk, sv, sa, sb, sw, sA, sD};
  for (const Span& in : inputs)
    if (overlaps(sO, in) || overlaps(so, in)) return GDN_ERR_INVALID_ARG;
  if (overlaps(sO, si) || overlaps(sO, so)) return GDN_ERR_INVALID_ARG;

  gdn::ChunkArgs a;
  a.B = d->B; a.T = d->T; a.Hk = d->H_k; a.Hv = d->H_v; a.dk = d->d_k; a.dv = d->d_v;
  a.io = gdn::DType::BF16; a.gate = gdn::DType::BF16;
  a.channel = ch; a.scale = d->scale;
  a.q = q; a.k = k; a.v = v; a.b = gt->b; a.w = gt->w; a.g = gt->a;
  a.state_in = state_in; a.state_out = state_out; a.o = o;
  a.raw_gates = true;
  a.ld_b = gt->ld_b; a.ld_g = gt->ld_a; a.ld_w = gt->ld_w;
  a.A_log = gt->A_log; a.dt_bias = gt->dt_bias;
  hipError_t e = gdn::launch_chunk_fwd(a, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return GDN_ERR_UNSUPPORTED;
  return launched(e);
}

gdn_status gdn_chunk_fwd_varlen(const gdn_varlen_desc* d, const int64_t* cu_seqlens,
                                const void* q, const void* k, const void* v,
                                const void* beta_or_b, const void* w, const void* g,
                                const float* state_in, float* state_out, void* o,
                                void* stream) {
  if (!d) return GDN_ERR_INVALID_ARG;
  if (d->N < 0 || d->total_T < 0) return GDN_ERR_INVALID_ARG;
  gdn_status st = check_common(d->H_k, d->H_v, d->d_k, d->d_v, d->io_dtype, d->gate_dtype,
                               d->gate_mode, d->scale);
  if (st != GDN_OK) return st;
  if (d->chunk != 64) return GDN_ERR_UNSUPPORTED;
  const double elems = (double)d->total_T * (double)d->H_v * (double)(d->d_k + d->d_v);
  if (elems > 9.0e15) return GDN_ERR_INVALID_ARG;
  if ((double)d->total_T > 2.0e9 || (double)d->N * (double)d->H_v * 2.0 > 2.0e9)
    return GDN_ERR_UNSUPPORTED;
  if (d->N == 0) return GDN_OK;
  if (!cu_seqlens || (reinterpret_cast<uintptr_t>(cu_seqlens) & 7u) != 0) return GDN_ERR_INVALID_ARG;
  const int64_t heads = d->N * d->H_v;
  const Span scu = span(cu_seqlens, d->N + 1, 8);
  const Span so = span(state_out, heads * d->d_k * d->d_v, 4);
  const Span sO = span(o, d->total_T * d->H_v * d->d_v, dtype_bytes(d->io_dtype));
  if (overlaps(scu, so) || overlaps(scu, sO)) return GDN_ERR_INVALID_ARG;
  if (d->total_T == 0) {
    // Every sequence is empty: only the states pass through.
    const Span si = span(state_in, heads * d->d_k * d->d_v, 4);
    if (overlaps(si, so) && !(si.lo == so.lo && si.hi == so.hi)) return GDN_ERR_INVALID_ARG;
    if ((state_in && !aligned16(state_in)) || (state_out && !aligned16(state_out)))
      return GDN_ERR_INVALID_ARG;
    if (!state_out || state_out == state_in) return GDN_OK;
    hipError_t e = gdn::launch_state_copy(state_in, state_out, heads * d->d_k * d->d_v,
                                          static_cast<hipStream_t>(stream));
    return launched(e);
  }
  st = check_pointers(d->total_T, heads, d->H_k, d->H_v, d->d_k, d->d_v, d->io_dtype,
                      d->gate_dtype, d->gate_mode, q, k, v, beta_or_b, w, g, state_in, state_out,
                      o, false);
  if (st != GDN_OK) return st;

  gdn::ChunkArgs a;
  a.B = d->N; a.T = d->total_T; a.cu_seqlens = cu_seqlens;
  a.Hk = d->H_k; a.Hv = d->H_v; a.dk = d->d_k; a.dv = d->d_v;
  a.io = to_dtype(d->io_dtype); a.gate = to_dtype(d->gate_dtype);
  a.channel = d->gate_mode == GDN_GATES_CHANNEL; a.scale = d->scale;
  a.q = q; a.k = k; a.v = v; a.b = beta_or_b; a.w = w; a.g = g;
  a.state_in = state_in; a.state_out = state_out; a.o = o;
  hipError_t e = gdn::launch_chunk_fwd(a, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return GDN_ERR_UNSUPPORTED;
  return launched(e);
}

gdn_status gdn_chunk_fwd_varlen_save(const gdn_varlen_desc* d, const int64_t* cu_seqlens,
                                     const void* q, const void* k, const void* v,
                                     const void* beta_or_b, const void* w, const void* g,
                                     const float* state_in, float* state_out, void* o,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!d) return GDN_ERR_INVALID_ARG;
  if (d->N <= 0 || d->total_T <= 0)   // nothing for a backward to read
    return gdn_chunk_fwd_varlen(d, cu_seqlens, q, k, v, beta_or_b, w, g, state_in, state_out, o,
                                stream);
  gdn_status st = check_common(d->H_k, d->H_v, d->d_k, d->d_v, d->io_dtype, d->gate_dtype,
                               d->gate_mode, d->scale);
  if (st != GDN_OK) return st;
  if (d->chunk != 64) return GDN_ERR_UNSUPPORTED;
  const double elems = (double)d->total_T * (double)d->H_v * (double)(d->d_k + d->d_v);
  if (elems > 9.0e15) return GDN_ERR_INVALID_ARG;
  if ((double)d->total_T > 2.0e9 || (double)d->N * (double)d->H_v * 2.0 > 2.0e9)
    return GDN_ERR_UNSUPPORTED;
  if (!cu_seqlens || (reinterpret_cast<uintptr_t>(cu_seqlens) & 7u) != 0) return GDN_ERR_INVALID_ARG;
  const int64_t heads = d->N * d->H_v;
  const Span scu = span(cu_seqlens, d->N + 1, 8);
  const Span so = span(state_out, heads * d->d_k * d->d_v, 4);
  const Span sO = span(o, d->total_T * d->H_v * d->d_v, dtype_bytes(d->io_dtype));
  if (overlaps(scu, so) || overlaps(scu, sO)) return GDN_ERR_INVALID_ARG;
  st = check_pointers(d->total_T, heads, d->H_k, d->H_v, d->d_k, d->d_v, d->io_dtype,
                      d->gate_dtype, d->gate_mode, q, k, v, beta_or_b, w, g, state_in, state_out,
                      o, false);
  if (st != GDN_OK) return st;
  const BwdShape bs{d->N, d->total_T, 0, cu_seqlens, d->H_k, d->H_v, d->d_k, d->d_v,
                    d->io_dtype, d->gate_dtype, d->gate_mode, d->scale};
  return run_fwd_save(bs, q, k, v, beta_or_b, w, g, state_in, state_out, o, workspace,
                      workspace_bytes, stream);
}

size_t gdn_backward_workspace_size(const gdn_bwd_desc* d) {
  if (!d) return 0;
  const BwdShape sh = shape_of(d);
  if (check_bwd_shape(sh) != GDN_OK || sh.N == 0 || sh.rows == 0) return 0;
  return bwd_layout(sh).total;
}

gdn_status gdn_backward(const gdn_bwd_desc* d, const void* q, const void* k, const void* v,
                        const void* beta_or_b, const void* w, const void* g,
                        const float* state_in, const void* d_o, const float* d_state_out,
                        void* workspace, size_t workspace_bytes, float* dq, float* dk,
                        float* dv, float* db, float* dw, float* dg, float* d_state_in,
                        void* stream) {
  if (!d) return GDN_ERR_INVALID_ARG;
  return run_backward(shape_of(d), q, k, v, beta_or_b, w, g, state_in, d_o, d_state_out,
                      workspace, workspace_bytes, dq, dk, dv, db, dw, dg, d_state_in, stream);
}

gdn_status gdn_backward_saved(const gdn_bwd_desc* d, const void* q, const void* k, const void* v,
                              const void* beta_or_b, const void* w, const void* g,
                              const float* state_in, const void* d_o, const float* d_state_out,
                              void* workspace, size_t workspace_bytes, float* dq, float* dk,
                              float* dv, float* db, float* dw, float* dg, float* d_state_in,
                              void* stream) {
  if (!d) return GDN_ERR_INVALID_ARG;
  return run_backward(shape_of(d), q, k, v, beta_or_b, w, g, state_in, d_o, d_state_out,
                      workspace, workspace_bytes, dq, dk, dv, db, dw, dg, d_state_in, stream,
                      /*phases=*/2);
}

size_t gdn_backward_varlen_workspace_size(const gdn_bwd_varlen_desc* d) {
  if (!d) return 0;
  const int64_t dummy = 0;
  const BwdShape sh = shape_of(d, &dummy);
  if (check_bwd_shape(sh) != GDN_OK || sh.N == 0 || sh.rows == 0) return 0;
  return bwd_layout(sh).total;
}

gdn_status gdn_backward_varlen(const gdn_bwd_varlen_desc* d, const int64_t* cu_seqlens,
                               const void* q, const void* k, const void* v,
                               const void* beta_or_b, const void* w, const void* g,
                               const float* state_in, const void* d_o, const float* d_state_out,
                               void* workspace, size_t workspace_bytes, float* dq, float* dk,
                               float* dv, float* db, float* dw, float* dg, float* d_state_in,
                               void* stream) {
  if (!d) return GDN_ERR_INVALID_ARG;
  if (d->N > 0 && !cu_seqlens) return GDN_ERR_INVALID_ARG;
  return run_backward(shape_of(d, cu_seqlens), q, k, v, beta_or_b, w, g, state_in, d_o,
                      d_state_out, workspace, workspace_bytes, dq, dk, dv, db, dw, dg,
                      d_state_in, stream);
}

gdn_status gdn_backward_varlen_saved(const gdn_bwd_varlen_desc* d, const int64_t* cu_seqlens,
                                     const void* q, const void* k, const void* v,
                                     const void* beta_or_b, const void* w, const void* g,
                                     const float* state_in, const void* d_o,
                                     const float* d_state_out, void* workspace,
                                     size_t workspace_bytes, float* dq, float* dk, float* dv,
                                     float* db, float* dw, float* dg, float* d_state_in,
                                     void* stream) {
  if (!d) return GDN_ERR_INVALID_ARG;
  if (d->N > 0 && !cu_seqlens) return GDN_ERR_INVALID_ARG;
  return run_backward(shape_of(d, cu_seqlens), q, k, v, beta_or_b, w, g, state_in, d_o,
                      d_state_out, workspace, workspace_bytes, dq, dk, dv, db, dw, dg,
                      d_state_in, stream, /*phases=*/2);
}

gdn_status gdn_short_conv(const gdn_conv_desc* d, const int64_t* cu_seqlens, const void* x,
                          const float* conv_w, const void* conv_state_in, void* conv_state_out,
                          void* q, void* k, void* v, void* stream) {
  if (!d) return GDN_ERR_INVALID_ARG;
  if (d->N < 0 || d->total_T < 0) return GDN_ERR_INVALID_ARG;
  if (d->H_k < 1 || d->H_v < 1 || d->d_k < 1 || d->d_v < 1) return GDN_ERR_INVALID_ARG;
  if (d->io_dtype != GDN_F32 && d->io_dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if ((d->d_k != 64 && d->d_k != 128) || (d->d_v != 64 && d->d_v != 128))
    return GDN_ERR_UNSUPPORTED;
  if (!std::isfinite(d->eps) || d->eps < 0.f) return GDN_ERR_INVALID_ARG;
  const int64_t C = 2 * (int64_t)d->H_k * d->d_k + (int64_t)d->H_v * d->d_v;
  if (d->ld_x < C || d->ld_x % 8 != 0) return GDN_ERR_INVALID_ARG;
  if ((double)d->total_T * (double)d->ld_x > 9.0e15 || (double)d->N * 3.0 * (double)C > 9.0e15)
    return GDN_ERR_INVALID_ARG;
  if (2.0 * d->H_k + d->H_v > 2.0e9) return GDN_ERR_UNSUPPORTED;  // grid limit
  if (d->N == 0) return GDN_OK;
  if (!cu_seqlens && d->total_T % d->N != 0) return GDN_ERR_INVALID_ARG;
  if (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 7u) != 0) return GDN_ERR_INVALID_ARG;
  const bool tokens = d->total_T > 0;
  if (tokens && (!x || !conv_w || !q || !k || !v)) return GDN_ERR_INVALID_ARG;
  if (!tokens && !conv_state_out) return GDN_OK;
  if (conv_state_out && !tokens && conv_state_out == conv_state_in) return GDN_OK;
  const void* all[] = {x, conv_w, conv_state_in, conv_state_out, q, k, v};
  for (const void* p : all)
    if (p && !aligned16(p)) return GDN_ERR_INVALID_ARG;

  const int64_t eb = dtype_bytes(d->io_dtype);
  const int64_t T = d->total_T;
  const Span sx = tokens ? span(x, (T - 1) * d->ld_x + C, eb) : Span{0, 0};
  const Span sw = tokens ? span(conv_w, C * 4, 4) : Span{0, 0};
  const Span scu = span(cu_seqlens, d->N + 1, 8);
  const Span si = span(conv_state_in, d->N * 3 * C, eb);
  const Span so = span(conv_state_out, d->N * 3 * C, eb);
  const Span sq = tokens ? span(q, T * d->H_k * d->d_k, eb) : Span{0, 0};
  const Span sk = tokens ? span(k, T * d->H_k * d->d_k, eb) : Span{0, 0};
  const Span sv = tokens ? span(v, T * d->H_v * d->d_v, eb) : Span{0, 0};
  const Span outs[] = {sq, sk, sv};
  const Span ins[] = {sx, sw, scu, si};
  for (const Span& o : outs) {
    for (const Span& in : ins)
      if (overlaps(o, in)) return GDN_ERR_INVALID_ARG;
    if (overlaps(o, so)) return GDN_ERR_INVALID_ARG;
  }
  if (overlaps(sq, sk) || overlaps(sq, sv) || overlaps(sk, sv)) return GDN_ERR_INVALID_ARG;
  if (overlaps(so, sx) || overlaps(so, sw) || overlaps(so, scu)) return GDN_ERR_INVALID_ARG;
  if (overlaps(so, si) && !(so.lo == si.lo && so.hi == si.hi)) return GDN_ERR_INVALID_ARG;

  gdn::ConvArgs a;
  a.N = d->N; a.total_T = T; a.Tseq = cu_seqlens ? 0 : T / d->N; a.cu_seqlens = cu_seqlens;
  a.Hk = d->H_k; a.Hv = d->H_v; a.dk = d->d_k; a.dv = d->d_v; a.C = C; a.ld_x = d->ld_x;
  a.io = to_dtype(d->io_dtype); a.eps = d->eps;
  a.x = x; a.w = conv_w; a.s_in = conv_state_in; a.s_out = conv_state_out;
  a.q = q; a.k = k; a.v = v;
  hipError_t e = gdn::launch_short_conv(a, static_cast<hipStream_t>(stream));
  return launched(e);
}

gdn_status gdn_gates(const gdn_gate_desc* d, const void* a_raw, const void* b_raw,
                     const void* w_raw, const float* A_log, const float* dt_bias, void* g,
                     void* beta_or_b, void* w, void* stream) {
  if (!d) return GDN_ERR_INVALID_ARG;
  if (d->rows < 0 || d->H_v < 1) return GDN_ERR_INVALID_ARG;
  if (d->gate_mode != GDN_GATES_SCALAR && d->gate_mode != GDN_GATES_CHANNEL)
    return GDN_ERR_INVALID_ARG;
  if (d->in_dtype != GDN_F32 && d->in_dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (d->gate_dtype != GDN_F32 && d->gate_dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  const bool ch = d->gate_mode == GDN_GATES_CHANNEL;
  if (ch && (d->d_k < 1 || d->d_v < 1)) return GDN_ERR_INVALID_ARG;
  const int64_t n_ab = ch ? (int64_t)d->H_v * d->d_k : d->H_v;
  const int64_t n_w = ch ? (int64_t)d->H_v * d->d_v : 0;
  if (d->ld_a < n_ab || d->ld_b < n_ab || (ch && d->ld_w < n_w)) return GDN_ERR_INVALID_ARG;
  if ((double)d->rows * (double)(n_ab > n_w ? n_ab : n_w) >= 4294967040.0)
    return GDN_ERR_UNSUPPORTED;  // 32-bit element indices
  if (!a_raw || !b_raw || !g || !beta_or_b) return GDN_ERR_INVALID_ARG;
  if (ch != (w_raw != nullptr) || ch != (w != nullptr)) return GDN_ERR_INVALID_ARG;
  const int64_t ib = dtype_bytes(d->in_dtype), ob = dtype_bytes(d->gate_dtype);
  const void* in_ptrs[] = {a_raw, b_raw, w_raw};
  for (const void* p : in_ptrs)
    if (p && (reinterpret_cast<uintptr_t>(p) % ib) != 0) return GDN_ERR_INVALID_ARG;
  const void* out_ptrs[] = {g, beta_or_b, w};
  for (const void* p : out_ptrs)
    if (p && (reinterpret_cast<uintptr_t>(p) % ob) != 0) return GDN_ERR_INVALID_ARG;
  if ((A_log && (reinterpret_cast<uintptr_t>(A_log) & 3u)) ||
      (dt_bias && (reinterpret_cast<uintptr_t>(dt_bias) & 3u)))
    return GDN_ERR_INVALID_ARG;
  if (d->rows == 0) return GDN_OK;
  const int64_t R = d->rows;
  const Span sa = span(a_raw, (R - 1) * d->ld_a + n_ab, ib);
  const Span sb = span(b_raw, (R - 1) * d->ld_b + n_ab, ib);
  const Span swr = ch ? span(w_raw, (R - 1) * d->ld_w + n_w, ib) : Span{0, 0};
  const Span sA = span(A_log, n_ab, 4), sdt = span(dt_bias, n_ab, 4);
  const Span sg = span(g, R * n_ab, ob), sbe = span(beta_or_b, R * n_ab, ob);
  const Span sw = span(w, R * n_w, ob);
  const Span ins[] = {sa, sb, swr, sA, sdt};
  const Span outs[] = {sg, sbe, sw};
  for (const Span& o : outs)
    for (const Span& in : ins)
      if (overlaps(o, in)) return GDN_ERR_INVALID_ARG;
  if (overlaps(sg, sbe) || overlaps(sg, sw) || overlaps(sbe, sw)) return GDN_ERR_INVALID_ARG;

  gdn::GateArgs a;
  a.n_ab = (uint32_t)n_ab; a.n_w = (uint32_t)n_w;
  a.n_ab_total = (uint32_t)(R * n_ab); a.n_w_total = (uint32_t)(R * n_w);
  a.ld_a = d->ld_a; a.ld_b = d->ld_b; a.ld_w = d->ld_w;
  a.in = to_dtype(d->in_dtype); a.out = to_dtype(d->gate_dtype);
  a.a = a_raw; a.b = b_raw; a.w_raw = w_raw; a.A_log = A_log; a.dt_bias = dt_bias;
  a.g = g; a.beta = beta_or_b; a.w = w;
  hipError_t e = gdn::launch_gates(a, static_cast<hipStream_t>(stream));
  return launched(e);
}

gdn_status gdn_output_gate(const gdn_norm_desc* d, const void* o, const void* z,
                           const float* weight, void* y, void* stream) {
  if (!d) return GDN_ERR_INVALID_ARG;
  if (d->rows < 0 || d->H_v < 1 || d->d_v < 1) return GDN_ERR_INVALID_ARG;
  if (d->io_dtype != GDN_F32 && d->io_dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (d->d_v != 64 && d->d_v != 128) return GDN_ERR_UNSUPPORTED;
  if (!std::isfinite(d->eps) || d->eps < 0.f) return GDN_ERR_INVALID_ARG;
  const int64_t width = (int64_t)d->H_v * d->d_v;
  if (d->ld_z < width || d->ld_z % 8 != 0) return GDN_ERR_INVALID_ARG;
  if ((double)d->rows * (double)d->ld_z > 9.0e15) return GDN_ERR_INVALID_ARG;
  if ((double)d->rows * (double)d->H_v / 64.0 > 2.0e9) return GDN_ERR_UNSUPPORTED;  // grid
  if (d->rows == 0) return GDN_OK;
  if (!o || !z || !weight || !y) return GDN_ERR_INVALID_ARG;
  const void* all[] = {o, z, weight, y};
  for (const void* p : all)
    if (!aligned16(p)) return GDN_ERR_INVALID_ARG;
  const int64_t eb = dtype_bytes(d->io_dtype);
  const Span so = span(o, d->rows * width, eb);
  const Span sz = span(z, (d->rows - 1) * d->ld_z + width, eb);
  const Span sw = span(weight, d->d_v, 4);
  const Span sy = span(y, d->rows * width, eb);
  if (overlaps(sy, sz) || overlaps(sy, sw)) return GDN_ERR_INVALID_ARG;
  if (overlaps(sy, so) && !(sy.lo == so.lo && sy.hi == so.hi)) return GDN_ERR_INVALID_ARG;

  gdn::NormArgs a;
  a.rows = d->rows; a.Hv = d->H_v; a.dv = d->d_v; a.ld_z = d->ld_z;
  a.io = to_dtype(d->io_dtype); a.eps = d->eps;
  a.o = o; a.z = z; a.weight = weight; a.y = y;
  hipError_t e = gdn::launch_output_gate(a, static_cast<hipStream_t>(stream));
  return launched(e);
}

gdn_status gdn_check_selftest(float* out64, void* stream) {
#ifdef GDN_CHECK
  if (!out64) return GDN_ERR_INVALID_ARG;
  unsigned long long before = (unsigned long long)gdn::check_violations_decode() +
                              gdn::check_violations_chunk() + gdn::check_violations_chunk_sb() +
                              gdn::check_violations_backward();
  (void)before;   // whatever an earlier call left is cleared first
  if (gdn::launch_check_selftest(out64, static_cast<hipStream_t>(stream)) != hipSuccess)
    return GDN_ERR_HIP;
  const unsigned v = gdn::check_violations_chunk_sb();
  return v == 64u ? GDN_OK : GDN_ERR_CHECK;
#else
  (void)out64;
  (void)stream;
  return GDN_ERR_UNSUPPORTED;
#endif
}

gdn_status gdn_decode_step(const gdn_decode_desc* d, const void* q, const void* k,
                           const void* v, const void* beta_or_b, const void* w, const void* g,
                           float* state, void* o, void* stream) {
  if (!d) return GDN_ERR_INVALID_ARG;
  if (d->N < 0) return GDN_ERR_INVALID_ARG;
  gdn_status st = check_common(d->H_k, d->H_v, d->d_k, d->d_v, d->io_dtype, d->gate_dtype,
                               d->gate_mode, d->scale);
  if (st != GDN_OK) return st;
  if ((double)d->N * (double)d->H_v > 2.0e9) return GDN_ERR_UNSUPPORTED;  // grid size
  if (d->N == 0) return GDN_OK;
  st = check_pointers(d->N, d->N * d->H_v, d->H_k, d->H_v, d->d_k, d->d_v, d->io_dtype,
                      d->gate_dtype, d->gate_mode, q, k, v, beta_or_b, w, g, state, state, o,
                      true);
  if (st != GDN_OK) return st;
  gdn::DecodeArgs a;
  a.N = d->N; a.Hk = d->H_k; a.Hv = d->H_v; a.dk = d->d_k; a.dv = d->d_v;
  a.io = to_dtype(d->io_dtype); a.gate = to_dtype(d->gate_dtype);
  a.channel = d->gate_mode == GDN_GATES_CHANNEL; a.scale = d->scale;
  a.q = q; a.k = k; a.v = v; a.b = beta_or_b; a.w = w; a.g = g;
  a.state = state; a.o = o;
  hipError_t e = gdn::launch_decode(a, static_cast<hipStream_t>(stream));
  return launched(e);
}

}  // extern "C"
