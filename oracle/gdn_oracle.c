/*
 * gdn_oracle.c -- CPU oracle for the gated delta rule (GDN-1 / GDN-2).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * reference that the GPU library is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark load it; the
 * product library never links, calls or falls back to it.  It shares no code,
 * header or constant with the HIP library.
 *
 * Arithmetic is IEEE double throughout.  Inputs arrive as double arrays that
 * the caller up-converted exactly from the bytes handed to the GPU
 * (bf16 -> fp32 -> double is exact).
 *
 * Sources (the web pages on the gated delta rule):
 *  - "Gated DeltaNet-2: Decoupling Erase and Write in Linear Attention"
 *    (gist.science summary), Methodologie §1 "Regle Delta Portee-2": the
 *    erase gate b_t in [0,1]^{d_k} forms the read direction e_t = b_t (.) k_t,
 *    the write gate w_t in [0,1]^{d_v} forms the target z_t = w_t (.) v_t, and
 *    the state update is S_t = (I - k_t e_t^T) D_t S_{t-1} + k_t z_t^T with
 *    D_t = Diag(alpha_t).  §2 "Perspective de Mise a Jour des Poids Rapides":
 *    the update corrects the read of the decayed memory, S_bar^T e_t, toward
 *    z_t -- so decay comes first, then read, then erase+write.
 *  - Same page, §3 "Entrainement Parallele Efficace par Blocs": the chunkwise
 *    form absorbs the cumulative channel decay into the erase matrix (E_bar)
 *    and the write matrix (Z) and solves a lower-triangular system (I+T)^{-1}
 *    for the auxiliary matrices Y (erase side) and U (write side).
 *  - "Gated DeltaNet" (docsaid.org notes), §"L'attention lineaire": the read
 *    of the memory is o_t = S_t q_t in that page's (transposed) orientation;
 *    with S stored d_k x d_v here, that read is o_t = S_t^T q_t, taken after
 *    the update of token t.
 *
 * Reading of the pages taken where they are silent:
 *  - alpha is passed in log space, g = log(alpha); g == NULL means alpha = 1.
 *  - the output scale is an explicit argument (1.0 in every workload).
 *  - value head h reads key head h / (H_v / H_k) (contiguous grouping).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_ABI 2

int gdn_oracle_abi(void) { return ORACLE_ABI; }

/* Gate accessors: scalar mode holds one value per (b,t,h), channel mode one
 * per (b,t,h,channel). */
static inline double gate_at(const double* p, int channel_mode, long bt_h,
                             int width, int c) {
  return channel_mode ? p[bt_h * (long)width + c] : p[bt_h];
}

/*
 * One head, token by token.  S is d_k x d_v, row-major, d_v contiguous.
 *   a     = exp(g_t)                  (decay, per key channel or scalar)
 *   e     = b_t (.) k_t               (read / erase direction)
 *   z     = w_t (.) v_t               (gated write target)
 *   S    <- Diag(a) S                 (decay)
 *   r     = S^T e                     (read of the decayed memory)
 *   S    <- S + k_t (z - r)^T         (erase along k, write z)
 *   o_t   = scale * S^T q_t           (read-out after the update)
 * In scalar mode b and w are the same scalar beta_t.
 */
static void run_head(long T, int dk, int dv, int channel_mode,
                     const double* q, long q_stride,   /* &q[b,0,hk,0], stride per token */
                     const double* k, long k_stride,
                     const double* v, long v_stride,   /* &v[b,0,hv,0] */
                     const double* bb, const double* ww, const double* gg,
                     int Hv, int hv, long bT,          /* gate row = (b*T + t)*Hv + hv */
                     double scale, double* S, double* o, long o_stride,
                     double* a, double* e, double* z, double* r) {
  for (long t = 0; t < T; ++t) {
    const double* qt = q + t * q_stride;
    const double* kt = k + t * k_stride;
    const double* vt = v + t * v_stride;
    long bth = (bT + t) * (long)Hv + hv;
    for (int i = 0; i < dk; ++i) {
      a[i] = gg ? exp(gate_at(gg, channel_mode, bth, dk, i)) : 1.0;
      e[i] = gate_at(bb, channel_mode, bth, dk, i) * kt[i];
    }
    for (int j = 0; j < dv; ++j) {
      double wj = channel_mode ? ww[bth * (long)dv + j] : bb[bth];
      z[j] = wj * vt[j];
    }
    /* decay */
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[(long)i * dv + j] *= a[i];
    /* read of the decayed memory */
    for (int j = 0; j < dv; ++j) r[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) r[j] += S[(long)i * dv + j] * e[i];
    /* erase along k and write z: rank-1 correction */
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[(long)i * dv + j] += kt[i] * (z[j] - r[j]);
    /* read-out with the query after the update */
    double* ot = o + t * o_stride;
    for (int j = 0; j < dv; ++j) ot[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) ot[j] += S[(long)i * dv + j] * qt[i];
    for (int j = 0; j < dv; ++j) ot[j] *= scale;
  }
}

static int check_dims(long B, long T, int Hk, int Hv, int dk, int dv) {
  if (B < 0 || T < 0 || Hk <= 0 || Hv <= 0 || dk <= 0 || dv <= 0) return 1;
  if (Hv % Hk != 0) return 1;
  return 0;
}

/*
 * Token-by-token recurrence over a batch.
 *   q, k      [B, T, Hk, dk]
 *   v, o      [B, T, Hv, dv]
 *   scalar mode (gate_mode 0): beta [B, T, Hv]; w must be NULL; g [B, T, Hv] or NULL
 *   channel mode (gate_mode 1): b [B, T, Hv, dk]; w [B, T, Hv, dv]; g [B, T, Hv, dk] or NULL
 *   state_in  [B, Hv, dk, dv] or NULL (zeros); state_out same shape or NULL.
 * Returns 0 on success, 1 on bad arguments.
 */
int gdn_ref_recurrent(long B, long T, int Hk, int Hv, int dk, int dv, int gate_mode,
                      const double* q, const double* k, const double* v,
                      const double* beta_or_b, const double* w, const double* g,
                      double scale, const double* state_in, double* state_out,
                      double* o, int nthreads) {
  if (check_dims(B, T, Hk, Hv, dk, dv)) return 1;
  if (gate_mode != 0 && gate_mode != 1) return 1;
  if (!q || !k || !v || !beta_or_b || !o) return 1;
  if (gate_mode == 1 && !w) return 1;
  if (gate_mode == 0 && w) return 1;
  const int group = Hv / Hk;
  const long n_heads = B * (long)Hv;
  int bad = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (long bh = 0; bh < n_heads; ++bh) {
    long b = bh / Hv;
    int hv = (int)(bh % Hv);
    int hk = hv / group;
    double* S = (double*)calloc((size_t)dk * dv, sizeof(double));
    double* scratch = (double*)malloc(sizeof(double) * (size_t)(2 * dk + 2 * dv));
    if (!S || !scratch) { bad |= 1; free(S); free(scratch); continue; }
    if (state_in)
      memcpy(S, state_in + bh * (long)dk * dv, sizeof(double) * (size_t)dk * dv);
    run_head(T, dk, dv, gate_mode,
             q + (b * T * Hk + hk) * (long)dk, (long)Hk * dk,
             k + (b * T * Hk + hk) * (long)dk, (long)Hk * dk,
             v + (b * T * Hv + hv) * (long)dv, (long)Hv * dv,
             beta_or_b, w, g, Hv, hv, b * T,
             scale, S, o + (b * T * Hv + hv) * (long)dv, (long)Hv * dv,
             scratch, scratch + dk, scratch + 2 * dk, scratch + 2 * dk + dv);
    if (state_out)
      memcpy(state_out + bh * (long)dk * dv, S, sizeof(double) * (size_t)dk * dv);
    free(S);
    free(scratch);
  }
  return bad ? 1 : 0;
}

/*
 * Single-token decode step: the same recurrence with T = 1, state updated in
 * place.  q, k [N, Hk, dk]; v, o [N, Hv, dv]; gates [N, Hv] (scalar) or
 * [N, Hv, dk] / [N, Hv, dv] (channel); state [N, Hv, dk, dv].
 */
int gdn_ref_decode(long N, int Hk, int Hv, int dk, int dv, int gate_mode,
                   const double* q, const double* k, const double* v,
                   const double* beta_or_b, const double* w, const double* g,
                   double scale, double* state, double* o, int nthreads) {
  if (!state) return 1;
  return gdn_ref_recurrent(N, 1, Hk, Hv, dk, dv, gate_mode, q, k, v, beta_or_b, w, g,
                           scale, state, state, o, nthreads);
}

/*
 * Naive chunkwise form, used only to check that the chunk decomposition the
 * pages describe reaches the recurrence's result.  For a chunk of C tokens
 * entering with state S (local index t = 0..C-1):
 *   G_t      = sum_{tau <= t} g_tau                 (cumulative log-decay)
 *   T[t,s]   = sum_c e_t,c k_s,c exp(G_t,c - G_s,c)  s < t (strictly lower)
 *   P[t,s]   = sum_c q_t,c k_s,c exp(G_t,c - G_s,c)  s <= t
 *   E_bar_t  = exp(G_t) (.) e_t        Z_t = z_t     (decay absorbed)
 *   (I + T) [Y | U0] = [E_bar | Z]                   (forward substitution)
 *   U        = U0 - Y S
 *   o_t      = scale * ( sum_c q_t,c exp(G_t,c) S[c,:] + sum_{s<=t} P[t,s] U_s )
 *   S_next   = Diag(exp(G_{C-1})) S + sum_s (exp(G_{C-1} - G_s) (.) k_s) U_s^T
 * Every exponent is formed from a difference G_t - G_s with s <= t, so
 * nothing overflows.  The last chunk may be shorter than C.
 */
int gdn_ref_chunkwise(long B, long T, int Hk, int Hv, int dk, int dv, int gate_mode,
                      const double* q, const double* k, const double* v,
                      const double* beta_or_b, const double* w, const double* g,
                      double scale, const double* state_in, double* state_out,
                      double* o, int C, int nthreads) {
  if (check_dims(B, T, Hk, Hv, dk, dv) || C <= 0) return 1;
  if (gate_mode != 0 && gate_mode != 1) return 1;
  if (!q || !k || !v || !beta_or_b || !o) return 1;
  if (gate_mode == 1 && !w) return 1;
  if (gate_mode == 0 && w) return 1;
  const int group = Hv / Hk;
  const long n_heads = B * (long)Hv;
  int bad = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (long bh = 0; bh < n_heads; ++bh) {
    long b = bh / Hv;
    int hv = (int)(bh % Hv);
    int hk = hv / group;
    size_t need = (size_t)dk * dv          /* S */
                + (size_t)C * dk * 4       /* G, e, Ebar, Y */
                + (size_t)C * dv * 3       /* Z, U0/U, Onew */
                + (size_t)C * C * 2;       /* T, P */
    double* mem = (double*)calloc(need, sizeof(double));
    if (!mem) { bad |= 1; continue; }
    double* S = mem;
    double* G = S + (size_t)dk * dv;
    double* e = G + (size_t)C * dk;
    double* Eb = e + (size_t)C * dk;
    double* Y = Eb + (size_t)C * dk;
    double* Z = Y + (size_t)C * dk;
    double* U = Z + (size_t)C * dv;
    double* On = U + (size_t)C * dv;
    double* Tm = On + (size_t)C * dv;
    double* P = Tm + (size_t)C * C;
    if (state_in)
      memcpy(S, state_in + bh * (long)dk * dv, sizeof(double) * (size_t)dk * dv);

    for (long t0 = 0; t0 < T; t0 += C) {
      int n = (int)((T - t0) < C ? (T - t0) : C);
      /* per-token operands of this chunk */
      for (int t = 0; t < n; ++t) {
        long tok = t0 + t;
        long bth = (b * T + tok) * (long)Hv + hv;
        const double* kt = k + ((b * T + tok) * Hk + hk) * (long)dk;
        const double* vt = v + ((b * T + tok) * Hv + hv) * (long)dv;
        for (int c = 0; c < dk; ++c) {
          double gv = g ? gate_at(g, gate_mode, bth, dk, c) : 0.0;
          G[(size_t)t * dk + c] = (t == 0 ? 0.0 : G[(size_t)(t - 1) * dk + c]) + gv;
          e[(size_t)t * dk + c] = gate_at(beta_or_b, gate_mode, bth, dk, c) * kt[c];
        }
        for (int j = 0; j < dv; ++j) {
          double wj = gate_mode ? w[bth * (long)dv + j] : beta_or_b[bth];
          Z[(size_t)t * dv + j] = wj * vt[j];
        }
        for (int c = 0; c < dk; ++c)
          Eb[(size_t)t * dk + c] = exp(G[(size_t)t * dk + c]) * e[(size_t)t * dk + c];
      }
      /* T (strictly lower) and P (lower incl. diagonal) */
      for (int t = 0; t < n; ++t) {
        const double* qt = q + ((b * T + t0 + t) * Hk + hk) * (long)dk;
        for (int s = 0; s < n; ++s) {
          const double* ks = k + ((b * T + t0 + s) * Hk + hk) * (long)dk;
          double ta = 0.0, pa = 0.0;
          if (s <= t) {
            for (int c = 0; c < dk; ++c) {
              double dec = exp(G[(size_t)t * dk + c] - G[(size_t)s * dk + c]);
              if (s < t) ta += e[(size_t)t * dk + c] * ks[c] * dec;
              pa += qt[c] * ks[c] * dec;
            }
          }
          Tm[(size_t)t * C + s] = ta;
          P[(size_t)t * C + s] = pa;
        }
      }
      /* forward substitution: (I + T) [Y | U0] = [E_bar | Z] */
      for (int t = 0; t < n; ++t) {
        for (int c = 0; c < dk; ++c) {
          double acc = Eb[(size_t)t * dk + c];
          for (int s = 0; s < t; ++s) acc -= Tm[(size_t)t * C + s] * Y[(size_t)s * dk + c];
          Y[(size_t)t * dk + c] = acc;
        }
        for (int j = 0; j < dv; ++j) {
          double acc = Z[(size_t)t * dv + j];
          for (int s = 0; s < t; ++s) acc -= Tm[(size_t)t * C + s] * U[(size_t)s * dv + j];
          U[(size_t)t * dv + j] = acc;
        }
      }
      /* U = U0 - Y S */
      for (int t = 0; t < n; ++t)
        for (int j = 0; j < dv; ++j) {
          double acc = 0.0;
          for (int c = 0; c < dk; ++c) acc += Y[(size_t)t * dk + c] * S[(size_t)c * dv + j];
          U[(size_t)t * dv + j] -= acc;
        }
      /* outputs: inter-chunk term through S plus intra-chunk causal term */
      for (int t = 0; t < n; ++t) {
        const double* qt = q + ((b * T + t0 + t) * Hk + hk) * (long)dk;
        for (int j = 0; j < dv; ++j) {
          double acc = 0.0;
          for (int c = 0; c < dk; ++c)
            acc += qt[c] * exp(G[(size_t)t * dk + c]) * S[(size_t)c * dv + j];
          for (int s = 0; s <= t; ++s) acc += P[(size_t)t * C + s] * U[(size_t)s * dv + j];
          On[(size_t)t * dv + j] = scale * acc;
        }
      }
      for (int t = 0; t < n; ++t) {
        double* ot = o + ((b * T + t0 + t) * Hv + hv) * (long)dv;
        memcpy(ot, On + (size_t)t * dv, sizeof(double) * (size_t)dv);
      }
      /* state passed to the next chunk */
      for (int c = 0; c < dk; ++c) {
        double GC = G[(size_t)(n - 1) * dk + c];
        for (int j = 0; j < dv; ++j) {
          double acc = exp(GC) * S[(size_t)c * dv + j];
          for (int s = 0; s < n; ++s) {
            const double* ks = k + ((b * T + t0 + s) * Hk + hk) * (long)dk;
            acc += exp(GC - G[(size_t)s * dk + c]) * ks[c] * U[(size_t)s * dv + j];
          }
          S[(size_t)c * dv + j] = acc;
        }
      }
    }
    if (state_out)
      memcpy(state_out + bh * (long)dk * dv, S, sizeof(double) * (size_t)dk * dv);
    free(mem);
  }
  return bad ? 1 : 0;
}

/*
 * Gradients of the recurrence (reverse mode, token by token) -- the backward
 * pass that training needs ("Gated DeltaNet-2", §3: the gate-aware gradient
 * accumulation of the auxiliary matrices; "Gated DeltaNet", §Rendre
 * l'entrainement parallele).  The pages give no gradient formulas; these
 * are the chain rule applied to the per-token steps of run_head, taken in
 * reverse order.  With P_t the state before token t (P_0 = state_in),
 * abar = exp(g_t), e = b (.) k, z = w (.) v:
 *
 *   Sbar = Diag(abar) P_t,  r = Sbar^T e,  u = z - r,
 *   P_{t+1} = Sbar + k u^T,  o_t = scale P_{t+1}^T q_t.
 *
 * Reverse step, with D the gradient w.r.t. P_{t+1} (D = d_state_out after the
 * last token, or 0):
 *   D     += scale q_t dO_t^T
 *   dq_t  += scale P_{t+1} dO_t
 *   du     = D^T k_t                 (dz = du, dr = -du)
 *   dv_t   = w (.) du,  dw_t = v (.) du
 *   de     = -Sbar du
 *   dk_t  += D u + b (.) de,  db_t = k (.) de
 *   dSbar  = D - e du^T
 *   dg_t   = abar (.) rowsum(dSbar (.) P_t)
 *   D      = Diag(abar) dSbar        (the gradient w.r.t. P_t)
 * and d_state_in = D after token 0.  In scalar mode b = w = beta_t, so
 * dbeta_t = sum(k (.) de) + sum(v (.) du), and dg_t is the sum over channels.
 * dq and dk sum over the value heads that share a key head.
 *
 *   d_o          [B, T, Hv, dv]
 *   d_state_out  [B, Hv, dk, dv] or NULL (no gradient flows into the final state)
 *   outputs: dq, dk [B,T,Hk,dk]; dv [B,T,Hv,dv]; db like beta_or_b; dw like w
 *   (NULL in scalar mode); dg like beta_or_b (NULL allowed, and required to be
 *   NULL when g is NULL); d_state_in [B,Hv,dk,dv] or NULL.
 * All states of a head are kept (T+1 matrices), so this is for small T.
 * Returns 0 on success, 1 on bad arguments or allocation failure.
 */
int gdn_ref_backward(long B, long T, int Hk, int Hv, int dk, int dv, int gate_mode,
                     const double* q, const double* k, const double* v,
                     const double* beta_or_b, const double* w, const double* g,
                     double scale, const double* state_in, const double* d_o,
                     const double* d_state_out, double* dq, double* dk_out,
                     double* dv_out, double* db, double* dw, double* dg,
                     double* d_state_in, int nthreads) {
  if (check_dims(B, T, Hk, Hv, dk, dv)) return 1;
  if (gate_mode != 0 && gate_mode != 1) return 1;
  if (!q || !k || !v || !beta_or_b || !d_o || !dq || !dk_out || !dv_out || !db) return 1;
  if (gate_mode == 1 && (!w || !dw)) return 1;
  if (gate_mode == 0 && (w || dw)) return 1;
  if (!g && dg) return 1;
  const int group = Hv / Hk;
  const int ch = gate_mode == 1;
  const long n_groups = B * (long)Hk;
  const size_t SS = (size_t)dk * dv;
  int bad = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  /* dq, dk are sums over the value heads of a key head: one thread per
   * (sequence, key head) owns them. */
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (long bg = 0; bg < n_groups; ++bg) {
    long b = bg / Hk;
    int hk = (int)(bg % Hk);
    for (long t = 0; t < T; ++t) {
      long row = (b * T + t) * Hk + hk;
      memset(dq + row * dk, 0, sizeof(double) * dk);
      memset(dk_out + row * dk, 0, sizeof(double) * dk);
    }
    double* P = (double*)malloc(sizeof(double) * SS * (size_t)(T + 1));
    double* U = (double*)malloc(sizeof(double) * (size_t)dv * (size_t)(T > 0 ? T : 1));
    double* D = (double*)malloc(sizeof(double) * SS);
    double* tmp = (double*)malloc(sizeof(double) * (size_t)(3 * dk + 3 * dv));
    if (!P || !U || !D || !tmp) { bad |= 1; free(P); free(U); free(D); free(tmp); continue; }
    double* a = tmp;             /* abar   [dk] */
    double* e = a + dk;          /* e      [dk] */
    double* de = e + dk;         /* de     [dk] */
    double* z = de + dk;         /* z      [dv] */
    double* r = z + dv;          /* r      [dv] */
    double* du = r + dv;         /* du     [dv] */
    for (int hv = hk * group; hv < (hk + 1) * group; ++hv) {
      const long bh = b * Hv + hv;
      /* forward, keeping every state and every u */
      if (state_in) memcpy(P, state_in + bh * (long)SS, sizeof(double) * SS);
      else memset(P, 0, sizeof(double) * SS);
      for (long t = 0; t < T; ++t) {
        const long bth = (b * T + t) * (long)Hv + hv;
        const double* kt = k + ((b * T + t) * Hk + hk) * (long)dk;
        const double* vt = v + bth * (long)dv;
        const double* Pt = P + (size_t)t * SS;
        double* Pn = P + (size_t)(t + 1) * SS;
        for (int i = 0; i < dk; ++i) {
          a[i] = g ? exp(gate_at(g, ch, bth, dk, i)) : 1.0;
          e[i] = gate_at(beta_or_b, ch, bth, dk, i) * kt[i];
        }
        for (int j = 0; j < dv; ++j) {
          z[j] = (ch ? w[bth * (long)dv + j] : beta_or_b[bth]) * vt[j];
          r[j] = 0.0;
        }
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < dv; ++j) r[j] += a[i] * Pt[(size_t)i * dv + j] * e[i];
        double* ut = U + (size_t)t * dv;
        for (int j = 0; j < dv; ++j) ut[j] = z[j] - r[j];
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < dv; ++j)
            Pn[(size_t)i * dv + j] = a[i] * Pt[(size_t)i * dv + j] + kt[i] * ut[j];
      }
      /* reverse */
      if (d_state_out) memcpy(D, d_state_out + bh * (long)SS, sizeof(double) * SS);
      else memset(D, 0, sizeof(double) * SS);
      for (long t = T - 1; t >= 0; --t) {
        const long bth = (b * T + t) * (long)Hv + hv;
        const long krow = (b * T + t) * Hk + hk;
        const double* qt = q + krow * (long)dk;
        const double* kt = k + krow * (long)dk;
        const double* vt = v + bth * (long)dv;
        const double* dot = d_o + bth * (long)dv;
        const double* Pt = P + (size_t)t * SS;
        const double* Pn = P + (size_t)(t + 1) * SS;
        const double* ut = U + (size_t)t * dv;
        double* dqt = dq + krow * (long)dk;
        double* dkt = dk_out + krow * (long)dk;
        double bsum = 0.0, gsum = 0.0;
        for (int i = 0; i < dk; ++i) {
          a[i] = g ? exp(gate_at(g, ch, bth, dk, i)) : 1.0;
          e[i] = gate_at(beta_or_b, ch, bth, dk, i) * kt[i];
        }
        /* o_t = scale P_{t+1}^T q_t */
        for (int i = 0; i < dk; ++i) {
          double acc = 0.0;
          for (int j = 0; j < dv; ++j) {
            D[(size_t)i * dv + j] += scale * qt[i] * dot[j];
            acc += Pn[(size_t)i * dv + j] * dot[j];
          }
          dqt[i] += scale * acc;
        }
        /* P_{t+1} = Sbar + k u^T */
        for (int j = 0; j < dv; ++j) du[j] = 0.0;
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < dv; ++j) du[j] += D[(size_t)i * dv + j] * kt[i];
        for (int j = 0; j < dv; ++j) {
          const long idx = bth * (long)dv + j;
          if (ch) {
            dv_out[idx] = w[idx] * du[j];
            dw[idx] = vt[j] * du[j];
          } else {
            dv_out[idx] = beta_or_b[bth] * du[j];
            bsum += vt[j] * du[j];
          }
        }
        for (int i = 0; i < dk; ++i) {
          double s = 0.0, du_dot = 0.0;
          for (int j = 0; j < dv; ++j) {
            s += a[i] * Pt[(size_t)i * dv + j] * du[j];
            du_dot += D[(size_t)i * dv + j] * ut[j];
          }
          de[i] = -s;
          const double bi = gate_at(beta_or_b, ch, bth, dk, i);
          dkt[i] += du_dot + bi * de[i];
          if (ch) db[bth * (long)dk + i] = kt[i] * de[i];
          else bsum += kt[i] * de[i];
        }
        /* Sbar = Diag(abar) P_t:  dSbar = D - e du^T */
        for (int i = 0; i < dk; ++i) {
          double da = 0.0;
          for (int j = 0; j < dv; ++j) {
            const double dsb = D[(size_t)i * dv + j] - e[i] * du[j];
            da += dsb * Pt[(size_t)i * dv + j];
            D[(size_t)i * dv + j] = a[i] * dsb;
          }
          if (dg && ch) dg[bth * (long)dk + i] = a[i] * da;
          gsum += a[i] * da;
        }
        if (!ch) {
          db[bth] = bsum;
          if (dg) dg[bth] = gsum;
        }
      }
      if (d_state_in) memcpy(d_state_in + bh * (long)SS, D, sizeof(double) * SS);
    }
    free(P); free(U); free(D); free(tmp);
  }
  return bad ? 1 : 0;
}
