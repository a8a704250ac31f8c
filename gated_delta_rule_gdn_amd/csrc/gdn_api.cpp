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

#include "gdn_kernels.hpp"

namespace {

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

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "GDN_OK: success";
    case GDN_ERR_INVALID_ARG: return "GDN_ERR_INVALID_ARG: invalid argument";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: configuration not supported";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: HIP runtime error at launch";
  }
  return "GDN_ERR_UNKNOWN: unknown status code";
}

gdn_status gdn_chunk_fwd(const gdn_fwd_desc* d, const void* q, const void* k, const void* v,
                         const void* beta_or_b, const void* w, const void* g,
                         const float* state_in, float* state_out, void* o, void* stream) {
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
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
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
  return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
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
    return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
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
  return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
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
  return e == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // extern "C"
