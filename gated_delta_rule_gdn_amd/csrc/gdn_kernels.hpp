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
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_chunk_fwd(const ChunkArgs& a, hipStream_t stream);
// bf16-operand producer/consumer variant (called by launch_chunk_fwd).
hipError_t launch_chunk_fwd_pipe(const ChunkArgs& a, hipStream_t stream);
// state_out = state_in (or 0 when state_in is NULL) for n floats; used when
// there are no tokens to process.
hipError_t launch_state_copy(const float* state_in, float* state_out, int64_t n,
                             hipStream_t stream);

}  // namespace gdn
