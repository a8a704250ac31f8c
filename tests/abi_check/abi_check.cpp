// Drives every entry point of the C ABI layer (gdn_api.cpp, built with the
// launch stubs of launch_stubs.cpp) over a grid of descriptors, from valid to
// absurd (negative, zero, huge and overflowing sizes, unknown dtypes and
// modes, non-finite scales), with distinct fake device addresses and with
// exact-size host buffers.  Under -fsanitize=address,undefined any
// out-of-bounds access or signed overflow in the validation aborts the run.
// It also checks that a call that returns an error has launched nothing, and
// that each small valid call launches.  Prints "ok <calls>" on success.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "gdn.h"

extern long g_launches;

namespace {

long calls = 0, failures = 0;

// Fake device addresses: 16-byte aligned, 2^40 bytes apart.
void* P(int i) { return reinterpret_cast<void*>((uintptr_t)(i + 1) << 40); }
float* F(int i) { return static_cast<float*>(P(i)); }

void check(gdn_status st, long before, const char* what) {
  ++calls;
  if (st < GDN_OK || st > GDN_ERR_HIP) {
    std::printf("%s: status %d out of range\n", what, (int)st);
    ++failures;
  }
  if (st != GDN_OK && g_launches != before) {
    std::printf("%s: launched on error %d\n", what, (int)st);
    ++failures;
  }
}

const int64_t kSizes[] = {-1, 0, 1, 17, 4096, (int64_t)1 << 31, (int64_t)1 << 62};
const int32_t kHeads[] = {0, 1, 3, 4, 65536, 2147483647};
const int32_t kDims[] = {0, 64, 128, 256};
const int32_t kTypes[] = {-1, GDN_F32, GDN_BF16, 5};
const int32_t kModes[] = {-1, GDN_GATES_SCALAR, GDN_GATES_CHANNEL, 3};
const float kScales[] = {1.f, NAN, INFINITY};

template <typename Fn>
void grid(Fn fn) {
  for (int64_t a : kSizes)
    for (int64_t t : kSizes)
      for (int32_t hk : kHeads)
        for (int hvm : {1, 2})
          for (int32_t d : kDims)
            for (int32_t io : kTypes)
              for (int32_t mode : kModes)
                for (float sc : kScales) {
                  const int64_t hv64 = (int64_t)hk * hvm;
                  const int32_t hv = hv64 > 2147483647 ? 2147483647 : (int32_t)hv64;
                  fn(a, t, hk, hv, d, io, mode, sc);
                }
}

void fuzz() {
  grid([](int64_t B, int64_t T, int32_t hk, int32_t hv, int32_t d, int32_t io, int32_t mode,
          float sc) {
    const bool ch = mode == GDN_GATES_CHANNEL;
    void* w = ch ? P(4) : nullptr;
    for (int32_t gate : {io, (int32_t)GDN_F32}) {
      gdn_fwd_desc f{B, T, hk, hv, d, d, io, gate, mode, 64, sc};
      long b0 = g_launches;
      check(gdn_chunk_fwd(&f, P(0), P(1), P(2), P(3), w, P(5), F(6), F(7), P(8), nullptr), b0,
            "chunk_fwd");
      b0 = g_launches;
      check(gdn_chunk_fwd_save(&f, P(0), P(1), P(2), P(3), w, P(5), F(6), F(7), P(8), P(9),
                               (size_t)1 << 40, nullptr),
            b0, "chunk_fwd_save");
      gdn_raw_gates rg{P(10), P(3), w, F(11), F(12), (int64_t)hv * d, (int64_t)hv * d,
                       (int64_t)hv * d};
      b0 = g_launches;
      check(gdn_chunk_fwd_gated(&f, P(0), P(1), P(2), &rg, F(6), F(7), P(8), nullptr), b0,
            "chunk_fwd_gated");
      gdn_varlen_desc vl{B, T, hk, hv, d, d, io, gate, mode, 64, sc};
      const int64_t* cu = static_cast<const int64_t*>(P(13));
      b0 = g_launches;
      check(gdn_chunk_fwd_varlen(&vl, cu, P(0), P(1), P(2), P(3), w, P(5), F(6), F(7), P(8),
                                 nullptr),
            b0, "chunk_fwd_varlen");
      b0 = g_launches;
      check(gdn_chunk_fwd_varlen_save(&vl, cu, P(0), P(1), P(2), P(3), w, P(5), F(6), F(7),
                                      P(8), P(9), (size_t)1 << 40, nullptr),
            b0, "chunk_fwd_varlen_save");
      gdn_decode_desc dd{B, hk, hv, d, d, io, gate, mode, sc};
      b0 = g_launches;
      check(gdn_decode_step(&dd, P(0), P(1), P(2), P(3), w, P(5), F(6), P(8), nullptr), b0,
            "decode_step");
      gdn_bwd_desc bd{B, T, hk, hv, d, d, io, gate, mode, sc};
      (void)gdn_backward_workspace_size(&bd);
      float* dw = ch ? F(18) : nullptr;
      b0 = g_launches;
      check(gdn_backward(&bd, P(0), P(1), P(2), P(3), w, P(5), F(6), P(8), F(7), P(9),
                         (size_t)1 << 40, F(14), F(15), F(16), F(17), dw, F(19), F(20), nullptr),
            b0, "backward");
      b0 = g_launches;
      check(gdn_backward_saved(&bd, P(0), P(1), P(2), P(3), w, P(5), F(6), P(8), F(7), P(9),
                               (size_t)1 << 40, F(14), F(15), F(16), F(17), dw, F(19), F(20),
                               nullptr),
            b0, "backward_saved");
      gdn_bwd_varlen_desc bv{B, T, hk, hv, d, d, io, gate, mode, sc};
      (void)gdn_backward_varlen_workspace_size(&bv);
      b0 = g_launches;
      check(gdn_backward_varlen(&bv, cu, P(0), P(1), P(2), P(3), w, P(5), F(6), P(8), F(7),
                                P(9), (size_t)1 << 40, F(14), F(15), F(16), F(17), dw, F(19),
                                F(20), nullptr),
            b0, "backward_varlen");
      b0 = g_launches;
      check(gdn_backward_varlen_saved(&bv, cu, P(0), P(1), P(2), P(3), w, P(5), F(6), P(8),
                                      F(7), P(9), (size_t)1 << 40, F(14), F(15), F(16), F(17),
                                      dw, F(19), F(20), nullptr),
            b0, "backward_varlen_saved");
    }
    // block operations
    gdn_conv_desc cd{B, T, (int64_t)2 * hk * d + (int64_t)hv * d, hk, hv, d, d, io, 1e-6f};
    long b0 = g_launches;
    check(gdn_short_conv(&cd, static_cast<const int64_t*>(P(13)), P(0), F(1), P(2), P(3), P(4),
                         P(5), P(6), nullptr),
          b0, "short_conv");
    gdn_gate_desc gd{T, (int64_t)hv * d, (int64_t)hv * d, (int64_t)hv * d, hv, d, d, mode, io,
                     io};
    b0 = g_launches;
    check(gdn_gates(&gd, P(0), P(1), mode == GDN_GATES_CHANNEL ? P(2) : nullptr, F(3), F(4),
                    P(5), P(6), mode == GDN_GATES_CHANNEL ? P(7) : nullptr, nullptr),
          b0, "gates");
    gdn_norm_desc nd{T, (int64_t)hv * d, hv, d, io, std::isfinite(sc) ? 1e-6f : sc};
    b0 = g_launches;
    check(gdn_output_gate(&nd, P(0), P(1), F(2), P(3), nullptr), b0, "output_gate");
  });
}

// A small valid call of each kind on exact-size host buffers launches.
void exact_buffers() {
  const int64_t B = 2, T = 37, hk = 1, hv = 2, d = 64;
  auto buf = [](int64_t bytes) { return std::malloc((size_t)bytes); };
  const int64_t qk = B * T * hk * d * 2, vb = B * T * hv * d * 2, S = B * hv * d * d * 4;
  void *q = buf(qk), *k = buf(qk), *v = buf(vb), *bb = buf(vb), *w = buf(vb), *g = buf(vb);
  void *o = buf(vb), *si = buf(S), *so = buf(S);
  gdn_fwd_desc f{B, T, (int32_t)hk, (int32_t)hv, (int32_t)d, (int32_t)d, GDN_BF16, GDN_BF16,
                 GDN_GATES_CHANNEL, 64, 1.f};
  long b0 = g_launches;
  gdn_status st = gdn_chunk_fwd(&f, q, k, v, bb, w, g, static_cast<float*>(si),
                                static_cast<float*>(so), o, nullptr);
  if (st != GDN_OK || g_launches != b0 + 1) {
    std::printf("exact-buffer chunk_fwd: %d\n", (int)st);
    ++failures;
  }
  gdn_bwd_desc bd{B, T, (int32_t)hk, (int32_t)hv, (int32_t)d, (int32_t)d, GDN_BF16, GDN_BF16,
                  GDN_GATES_CHANNEL, 1.f};
  const size_t nws = gdn_backward_workspace_size(&bd);
  void* ws = buf((int64_t)nws);
  const int64_t gq = B * T * hk * d * 4, gv = B * T * hv * d * 4;
  void *dq = buf(gq), *dk = buf(gq), *dv = buf(gv), *db = buf(gv), *dwg = buf(gv),
       *dg = buf(gv), *dsi = buf(S), *dso = buf(S), *dO = buf(vb);
  b0 = g_launches;
  st = gdn_chunk_fwd_save(&f, q, k, v, bb, w, g, static_cast<float*>(si), static_cast<float*>(so),
                          o, ws, nws, nullptr);
  if (st != GDN_OK || g_launches != b0 + 1) {
    std::printf("exact-buffer chunk_fwd_save: %d\n", (int)st);
    ++failures;
  }
  b0 = g_launches;
  st = gdn_backward_saved(&bd, q, k, v, bb, w, g, static_cast<float*>(si), dO,
                          static_cast<float*>(dso), ws, nws, static_cast<float*>(dq),
                          static_cast<float*>(dk), static_cast<float*>(dv),
                          static_cast<float*>(db), static_cast<float*>(dwg),
                          static_cast<float*>(dg), static_cast<float*>(dsi), nullptr);
  if (st != GDN_OK || g_launches != b0 + 1) {
    std::printf("exact-buffer backward_saved: %d\n", (int)st);
    ++failures;
  }
  calls += 3;
  for (void* p : {q, k, v, bb, w, g, o, si, so, ws, dq, dk, dv, db, dwg, dg, dsi, dso, dO})
    std::free(p);
}

}  // namespace

int main() {
  fuzz();
  exact_buffers();
  if (failures) {
    std::printf("FAILED %ld of %ld calls\n", failures, calls);
    return 1;
  }
  std::printf("ok %ld calls, %ld launches\n", calls, g_launches);
  return 0;
}
