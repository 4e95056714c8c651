/*
 * ram_oracle.c -- plain, slow CPU oracle for the RAM-Net attention core.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file.  Only the test suite, the smoke check of the package entry
 * module and the CPU-baseline leg of the benchmark use it.  It shares no code,
 * header, table or helper with the HIP library.
 *
 * What it computes, and where the pages define it:
 *   - Sources: "RAM-Net: Linear-Time Sequence Modeling with Sparsely
 *     Addressable State" (paper page) and the "ramnet-ops 0.1.0rc0" PyPI page.
 *   - Address decoding (paper §3.1, §3.2 "Address Decoder", App. B.1): per
 *     token, head and side, a softmax over each of U digits of size P; the
 *     probability of slot a = (a_0..a_{U-1}) is the product of its digit
 *     probabilities (Kronecker product), the K most probable slots are kept
 *     with their un-renormalised probabilities (paper App. B.2 "Addressing";
 *     ramnet-ops "Arguments", top_k_re_norm defaults to False).
 *   - Gated Sparse Update (paper §3.4, properties (i)-(iii) and the TTT
 *     remark): per addressed slot, retention lambda = sigmoid(logit(1-w) -
 *     gamma), mass m <- lambda*m + w, step eta = w/(m+eps), content
 *     s <- (1-eta)*s + eta*v.  The printed equations did not survive in the
 *     pages; this is the reading that satisfies every stated property.
 *   - Read-out (paper §3.4 "Read-out"): o_t = sum_a r_t[a] s_t[a], with S_t
 *     the state after token t's writes.
 *   - CAPE (ramnet-ops "Quick start": the first embed_num heads cyclically
 *     shift read and write slot indices by token position; paper App. C: the
 *     index of given content moves by one per step).
 *   - Token mask (ramnet-ops "Arguments", mask): a masked token is not
 *     written and its output is to be ignored; read here as a token absent
 *     from the computation (no write, no read, output 0, zero gradients).
 *   - Read epilogue (paper §3.4 "Read-out", its last sentence, and Fig. 2):
 *     y = sigmoid(g) * RMSNorm(o), RMSNorm head-wise: over the d_v channels
 *     of one (token, head), o / sqrt(mean(o^2) + eps_n) times a gain vector
 *     of d_v entries; g are the gate pre-activations (x W_g).  The output
 *     projection W_o is outside.
 *   - First-order gradients (ramnet-ops "Autograd and compile").
 *
 * Arithmetic: every floating-point value is held and computed in IEEE double.
 * Inputs arrive as double arrays (bf16 and fp32 io values convert exactly).
 * One decision is taken in float, by reading: for U >= 2 the ranking key of a
 * slot is the float32 sum of its raw digit logits, taken in ascending u
 * starting from 0.  The pages rank slots by a sum of per-digit log-scores
 * (paper §4 "Efficient Address Decoding"; the slot probability is the
 * product of the digit softmaxes, App. B.1) but fix neither the precision
 * nor the order of that sum; near-ties rank one way or the other depending
 * on both, so the reading fixes them (float32, the precision of the state
 * and of all arithmetic on the path; ascending u, the digits' order).  For
 * U = 1 the key is the logit itself, exact.
 *
 * Parallelism: OpenMP over independent (batch, head) pairs or rows only.
 * Compile with -ffp-contract=off so no fused multiply-add changes rounding.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int32_t B, H, T;      /* batch, heads, tokens in this call               */
  int32_t U, P;         /* digits per address and digit size; S = P^U      */
  int32_t k_w, k_r;     /* top-K of the write and read side                */
  int32_t d_v;          /* slot / value width                              */
  double eps;           /* GSU epsilon (> 0 in the paper; 0 allowed here)  */
  int32_t renorm_w, renorm_r; /* renormalise the kept weights per side     */
  int32_t cape_heads;   /* heads h < cape_heads use CAPE                    */
  int32_t pad_;
  int64_t t0;           /* absolute position of token 0 of this call       */
} orc_problem;

enum { ORC_OK = 0, ORC_EINVAL = -1, ORC_ENOMEM = -2 };

static int64_t slots_of(const orc_problem* p) {
  int64_t s = 1;
  for (int u = 0; u < p->U; ++u) s *= p->P;
  return s;
}

static int check_problem(const orc_problem* p) {
  if (!p || p->B < 0 || p->H < 1 || p->T < 0 || p->U < 1 || p->P < 1) return ORC_EINVAL;
  if (p->d_v < 1 || p->k_w < 1 || p->k_r < 1) return ORC_EINVAL;
  double s = pow((double)p->P, (double)p->U);
  if (s > 2147483647.0) return ORC_EINVAL;
  if (p->k_w > (int64_t)s || p->k_r > (int64_t)s) return ORC_EINVAL;
  if (p->cape_heads < 0 || p->cape_heads > p->H || p->t0 < 0) return ORC_EINVAL;
  if (!(p->eps >= 0.0)) return ORC_EINVAL;
  return ORC_OK;
}

int orc_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Address decoding of one row (one token, one head, one side).             */
/* ------------------------------------------------------------------------ */

/* Per digit u: lse_u = log sum_i exp(l_u[i]), max-shifted, i ascending. */
static void digit_lse(const double* l, int U, int P, double* lse) {
  for (int u = 0; u < U; ++u) {
    const double* d = l + (int64_t)u * P;
    double mx = -INFINITY;
    for (int i = 0; i < P; ++i) if ((double)d[i] > mx) mx = (double)d[i];
    double sum = 0.0;
    for (int i = 0; i < P; ++i) sum += exp((double)d[i] - mx);
    lse[u] = mx + log(sum);
  }
}

/* Ranking key of flat slot a: the float sum of its digit logits, u ascending.
 * Digits are big-endian: a = sum_u a_u * P^(U-1-u) (Kronecker order). */
static float slot_key(const double* l, int U, int P, int64_t a) {
  float key = 0.0f;
  int64_t stride = 1;
  for (int u = 1; u < U; ++u) stride *= P;
  for (int u = 0; u < U; ++u) {
    int64_t au = (a / stride) % P;
    key = key + (float)l[(int64_t)u * P + au];
    stride /= P;
  }
  return key;
}

/* Top-k of one row: scan the S slots in ascending index order and keep the k
 * best by (key descending, index ascending).  A later slot enters only if its
 * key is strictly larger than the current k-th, so among equal keys the
 * lower index stays ahead.  Output is sorted by that order.  Weights are the
 * slot probabilities exp(sum_u (l_u[a_u] - lse_u)), optionally renormalised.
 * Returns the un-renormalised sum in *wsum_out (used by the backward). */
static void decode_row(const double* l, int U, int P, int k, int renorm,
                       int32_t* idx, double* w, double* lse, double* wsum_out) {
  const int64_t S = (int64_t)pow((double)P, (double)U) + 0.5;
  float* best = (float*)malloc(sizeof(float) * k);
  int n = 0;
  for (int64_t a = 0; a < S; ++a) {
    float key = slot_key(l, U, P, a);
    if (n == k && !(key > best[k - 1])) continue;
    int pos = (n < k) ? n : k - 1;
    /* shift right while the new key beats the entry in front of it */
    while (pos > 0 && key > best[pos - 1]) {
      if (pos < k) { best[pos] = best[pos - 1]; idx[pos] = idx[pos - 1]; }
      --pos;
    }
    best[pos] = key;
    idx[pos] = (int32_t)a;
    if (n < k) ++n;
  }
  free(best);
  digit_lse(l, U, P, lse);
  double wsum = 0.0;
  for (int j = 0; j < k; ++j) {
    /* log-probability of the slot: sum_u (l_u[a_u] - lse_u), in double */
    int64_t a = idx[j], stride = 1;
    for (int u = 1; u < U; ++u) stride *= P;
    double lp = 0.0;
    for (int u = 0; u < U; ++u) {
      int64_t au = (a / stride) % P;
      lp += (double)l[(int64_t)u * P + au] - lse[u];
      stride /= P;
    }
    w[j] = exp(lp);
    wsum += w[j];
  }
  if (renorm)
    for (int j = 0; j < k; ++j) w[j] = w[j] / wsum;
  if (wsum_out) *wsum_out = wsum;
}

/* CAPE: heads h < cape_heads shift the selected flat index cyclically by the
 * absolute token position (t0 + t).  Selection (and its tie order) is on the
 * content logits; the shift is applied to the chosen index. */
static int32_t cape_shift(const orc_problem* p, int h, int64_t t, int32_t a, int64_t S) {
  if (h >= p->cape_heads) return a;
  int64_t pos = p->t0 + t;
  return (int32_t)(((int64_t)a + pos % S) % S);
}

/* Decode every row (b, t, h) of one side.  logits: (B,T,H,U,P); outputs
 * idx (B,T,H,k) holding the final slot (after CAPE), w (B,T,H,k),
 * lse (B,T,H,U). */
int orc_decode(const orc_problem* p, int side, const double* logits,
               int32_t* idx, double* w, double* lse) {
  if (check_problem(p) != ORC_OK || (side != 0 && side != 1)) return ORC_EINVAL;
  const int k = side == 0 ? p->k_w : p->k_r;
  const int renorm = side == 0 ? p->renorm_w : p->renorm_r;
  const int64_t S = slots_of(p);
  const int64_t rows = (int64_t)p->B * p->T * p->H;
  const int64_t rowlen = (int64_t)p->U * p->P;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t row = 0; row < rows; ++row) {
    int h = (int)(row % p->H);
    int64_t t = (row / p->H) % p->T;
    decode_row(logits + row * rowlen, p->U, p->P, k, renorm,
               idx + row * k, w + row * k, lse + row * p->U, NULL);
    for (int j = 0; j < k; ++j) idx[row * k + j] = cape_shift(p, h, t, idx[row * k + j], S);
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Gated Sparse Update on one slot.                                          */
/* ------------------------------------------------------------------------ */

/* Retention lambda = sigmoid(logit(1-w) - gamma) = (1-w)/((1-w) + w e^gamma),
 * evaluated in the form that stays finite for large |gamma|: for gamma >= 0
 * numerator and denominator are multiplied by q = e^-gamma.  Also returns
 * d lambda / d w = -e^gamma / D^2 in the matching form.  w = 0 gives
 * lambda = 1 (logit(1) = +inf), w = 1 gives lambda = 0 (logit(0) = -inf). */
static void retention(double w, double g, double* lam, double* dlam_dw) {
  double num, den, c;
  if (g >= 0.0) {
    c = exp(-g);
    num = (1.0 - w) * c;
    den = num + w;
  } else {
    c = exp(g);
    num = 1.0 - w;
    den = num + w * c;
  }
  if (w <= 0.0) *lam = 1.0;
  else if (w >= 1.0) *lam = 0.0;
  else *lam = num / den;
  if (dlam_dw) *dlam_dw = -c / (den * den);
}

/* One write of value v (d_v doubles) with weight w and modulator g into
 * slot content s and mass *m. */
static void gsu_write(double* s, double* m, const double* v, int d_v,
                      double w, double g, double eps) {
  double lam;
  retention(w, g, &lam, NULL);
  double m_new = lam * (*m) + w;
  double eta = (w > 0.0) ? w / (m_new + eps) : 0.0;
  for (int c = 0; c < d_v; ++c) s[c] = (1.0 - eta) * s[c] + eta * v[c];
  *m = m_new;
}

/* ------------------------------------------------------------------------ */
/* Forward: token-by-token over the slot array of each (b, h).              */
/* ------------------------------------------------------------------------ */

static void decode_token(const orc_problem* p, const double* wl, const double* rl,
                         int64_t t, int h, int32_t* iw, double* ww, double* lw, double* sw,
                         int32_t* ir, double* wr, double* lr, double* sr) {
  const int64_t S = slots_of(p);
  decode_row(wl, p->U, p->P, p->k_w, p->renorm_w, iw, ww, lw, sw);
  decode_row(rl, p->U, p->P, p->k_r, p->renorm_r, ir, wr, lr, sr);
  for (int j = 0; j < p->k_w; ++j) iw[j] = cape_shift(p, h, t, iw[j], S);
  for (int j = 0; j < p->k_r; ++j) ir[j] = cape_shift(p, h, t, ir[j], S);
}

/* Runs one (b, h): state s (S x d_v) and m (S) are updated in place; writes
 * o rows for every token.  When hist_* are given, records for the backward:
 * the pre-write content and mass of every write and the content read by
 * every read. */
static void forward_bh(const orc_problem* p, int b, int h,
                       const double* wlogits, const double* rlogits,
                       const double* vin, const double* gamma, const uint8_t* mask,
                       double* s, double* m, double* o,
                       double* hist_s_old, double* hist_m_old, double* hist_read,
                       int32_t* hid_w, double* hw_w, double* hl_w, double* hs_w,
                       int32_t* hid_r, double* hw_r, double* hl_r, double* hs_r) {
  const int d_v = p->d_v, kw = p->k_w, kr = p->k_r;
  const int64_t rowlen = (int64_t)p->U * p->P;
  double* v = (double*)malloc(sizeof(double) * d_v);
  int32_t* iw = (int32_t*)malloc(sizeof(int32_t) * kw);
  int32_t* ir = (int32_t*)malloc(sizeof(int32_t) * kr);
  double* ww = (double*)malloc(sizeof(double) * kw);
  double* wr = (double*)malloc(sizeof(double) * kr);
  double* lw = (double*)malloc(sizeof(double) * p->U);
  double* lr = (double*)malloc(sizeof(double) * p->U);
  double sw = 0.0, sr = 0.0;
  for (int64_t t = 0; t < p->T; ++t) {
    const int64_t row = ((int64_t)b * p->T + t) * p->H + h;
    if (mask && !mask[(int64_t)b * p->T + t]) {
      /* a masked token is absent: no write, no read, output 0 */
      if (o)
        for (int c = 0; c < d_v; ++c) o[row * d_v + c] = 0.0;
      continue;
    }
    decode_token(p, wlogits + row * rowlen, rlogits + row * rowlen, t, h,
                 iw, ww, lw, &sw, ir, wr, lr, &sr);
    for (int c = 0; c < d_v; ++c) v[c] = (double)vin[row * d_v + c];
    const double g = (double)gamma[row];
    /* writes of token t (distinct slots, so their order does not matter) */
    for (int j = 0; j < kw; ++j) {
      double* sa = s + (int64_t)iw[j] * d_v;
      if (hist_s_old) {
        memcpy(hist_s_old + ((int64_t)t * kw + j) * d_v, sa, sizeof(double) * d_v);
        hist_m_old[(int64_t)t * kw + j] = m[iw[j]];
      }
      gsu_write(sa, &m[iw[j]], v, d_v, ww[j], g, p->eps);
    }
    /* reads of token t see its own writes */
    for (int j = 0; j < kr; ++j) {
      const double* sa = s + (int64_t)ir[j] * d_v;
      if (hist_read) memcpy(hist_read + ((int64_t)t * kr + j) * d_v, sa, sizeof(double) * d_v);
    }
    if (o) {
      double* orow = o + row * d_v;
      for (int c = 0; c < d_v; ++c) orow[c] = 0.0;
      for (int j = 0; j < kr; ++j) {
        const double* sa = s + (int64_t)ir[j] * d_v;
        for (int c = 0; c < d_v; ++c) orow[c] += wr[j] * sa[c];
      }
    }
    if (hid_w) {
      memcpy(hid_w + t * kw, iw, sizeof(int32_t) * kw);
      memcpy(hw_w + t * kw, ww, sizeof(double) * kw);
      memcpy(hl_w + t * p->U, lw, sizeof(double) * p->U);
      hs_w[t] = sw;
      memcpy(hid_r + t * kr, ir, sizeof(int32_t) * kr);
      memcpy(hw_r + t * kr, wr, sizeof(double) * kr);
      memcpy(hl_r + t * p->U, lr, sizeof(double) * p->U);
      hs_r[t] = sr;
    }
  }
  free(v); free(iw); free(ir); free(ww); free(wr); free(lw); free(lr);
}

/* Forward over all (b, h).  Shapes: logits (B,T,H,U,P), v (B,T,H,d_v),
 * gamma (B,T,H), slot0/slot1 (B,H,S,d_v), mass0/mass1 (B,H,S), o (B,T,H,d_v).
 * slot0 / mass0 may be NULL (every slot starts empty: content 0, mass 0).
 * mask (B,T) uint8, nonzero = valid token, or NULL (all valid). */
int orc_forward(const orc_problem* p, const double* wlogits, const double* rlogits,
                const double* v, const double* gamma, const uint8_t* mask,
                const double* slot0, const double* mass0,
                double* o, double* slot1, double* mass1) {
  if (check_problem(p) != ORC_OK || !wlogits || !rlogits || !v || !gamma || !o || !slot1 || !mass1)
    return ORC_EINVAL;
  if ((slot0 == NULL) != (mass0 == NULL)) return ORC_EINVAL;
  const int64_t S = slots_of(p);
  const int64_t nbh = (int64_t)p->B * p->H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < nbh; ++bh) {
    const int b = (int)(bh / p->H), h = (int)(bh % p->H);
    double* s = slot1 + bh * S * p->d_v;
    double* m = mass1 + bh * S;
    if (slot0) {
      memmove(s, slot0 + bh * S * p->d_v, sizeof(double) * S * p->d_v);
      memmove(m, mass0 + bh * S, sizeof(double) * S);
    } else {
      memset(s, 0, sizeof(double) * S * p->d_v);
      memset(m, 0, sizeof(double) * S);
    }
    forward_bh(p, b, h, wlogits, rlogits, v, gamma, mask, s, m, o,
               NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL);
  }
  return ORC_OK;
}

/* Autoregressive step (ramnet-ops "CUDA execution", autoregressive mode):
 * one token per (b, h), state (B,H,S,d_v) / (B,H,S) updated in place.
 * p->T must be 1; p->t0 is the position of that token.  mask (B) or NULL. */
int orc_decode_step(const orc_problem* p, const double* wlogits, const double* rlogits,
                    const double* v, const double* gamma, const uint8_t* mask,
                    double* slot, double* mass, double* o) {
  if (check_problem(p) != ORC_OK || p->T != 1 || !slot || !mass || !o) return ORC_EINVAL;
  const int64_t S = slots_of(p);
  const int64_t nbh = (int64_t)p->B * p->H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < nbh; ++bh) {
    const int b = (int)(bh / p->H), h = (int)(bh % p->H);
    forward_bh(p, b, h, wlogits, rlogits, v, gamma, mask, slot + bh * S * p->d_v, mass + bh * S, o,
               NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL);
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Backward: reverse token loop (first-order gradients).                    */
/* ------------------------------------------------------------------------ */

/* Gradient of the decoded weights of one row with respect to its logits.
 * g[j] is dL/dw_j of the weights as output (renormalised if renorm).  With
 * renormalisation w~_j = w_j / W: dL/dw_j = (g_j - sum_i g_i w~_i) / W.
 * Then dl_u[i] = sum_j gw_j [a_{j,u} = i] - p_u[i] sum_j gw_j, with
 * gw_j = (dL/dw_j) w_j and p_u the digit softmax. */
static void decode_row_backward(const double* l, int U, int P, int k, int renorm,
                                const int32_t* idx_content, const double* w_out,
                                const double* lse, double wsum, const double* g,
                                double* dl) {
  double* gw = (double*)malloc(sizeof(double) * k);
  double dot = 0.0;
  if (renorm) for (int j = 0; j < k; ++j) dot += g[j] * w_out[j];
  double tot = 0.0;
  for (int j = 0; j < k; ++j) {
    double wj = renorm ? w_out[j] * wsum : w_out[j];  /* un-renormalised weight */
    double dj = renorm ? (g[j] - dot) / wsum : g[j];
    gw[j] = dj * wj;
    tot += gw[j];
  }
  for (int u = 0; u < U; ++u)
    for (int i = 0; i < P; ++i)
      dl[(int64_t)u * P + i] = -exp((double)l[(int64_t)u * P + i] - lse[u]) * tot;
  int64_t top = 1;
  for (int u = 1; u < U; ++u) top *= P;
  for (int j = 0; j < k; ++j) {
    int64_t a = idx_content[j], stride = top;
    for (int u = 0; u < U; ++u) {
      int64_t au = (a / stride) % P;
      dl[(int64_t)u * P + au] += gw[j];
      stride /= P;
    }
  }
  free(gw);
}

/* Backward over all (b, h).  d_o (B,T,H,d_v) is the gradient of o; d_slot1
 * and d_mass1 (may be NULL = zero) the gradients of the final state.
 * Outputs: d_wlogits, d_rlogits (B,T,H,U,P), d_v (B,T,H,d_v), d_gamma
 * (B,T,H), d_slot0 (B,H,S,d_v), d_mass0 (B,H,S) (both may be NULL).
 * Optional dw_out (B,T,H,k_w) and dr_out (B,T,H,k_r): gradients of the
 * decoded weights (the values fed to the decode backward).  mask as in
 * orc_forward. */
int orc_backward(const orc_problem* p, const double* wlogits, const double* rlogits,
                 const double* vin, const double* gamma, const uint8_t* mask,
                 const double* slot0, const double* mass0,
                 const double* d_o, const double* d_slot1, const double* d_mass1,
                 double* d_wlogits, double* d_rlogits, double* d_v, double* d_gamma,
                 double* d_slot0, double* d_mass0, double* dw_out, double* dr_out) {
  if (check_problem(p) != ORC_OK || !wlogits || !rlogits || !vin || !gamma || !d_o ||
      !d_wlogits || !d_rlogits || !d_v || !d_gamma)
    return ORC_EINVAL;
  if ((slot0 == NULL) != (mass0 == NULL)) return ORC_EINVAL;
  const int64_t S = slots_of(p);
  const int64_t nbh = (int64_t)p->B * p->H;
  const int d_v_ = p->d_v, kw = p->k_w, kr = p->k_r, U = p->U, P = p->P;
  const int64_t rowlen = (int64_t)U * P;
  int status = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < nbh; ++bh) {
    const int b = (int)(bh / p->H), h = (int)(bh % p->H);
    const int64_t T = p->T;
    double* s = (double*)malloc(sizeof(double) * S * d_v_);
    double* m = (double*)malloc(sizeof(double) * S);
    double* hs_old = (double*)malloc(sizeof(double) * (T * kw * d_v_ + 1));
    double* hm_old = (double*)malloc(sizeof(double) * (T * kw + 1));
    double* hread = (double*)malloc(sizeof(double) * (T * kr * d_v_ + 1));
    int32_t* iw = (int32_t*)malloc(sizeof(int32_t) * (T * kw + 1));
    int32_t* ir = (int32_t*)malloc(sizeof(int32_t) * (T * kr + 1));
    double* ww = (double*)malloc(sizeof(double) * (T * kw + 1));
    double* wr = (double*)malloc(sizeof(double) * (T * kr + 1));
    double* lw = (double*)malloc(sizeof(double) * (T * U + 1));
    double* lr = (double*)malloc(sizeof(double) * (T * U + 1));
    double* sw = (double*)malloc(sizeof(double) * (T + 1));
    double* sr = (double*)malloc(sizeof(double) * (T + 1));
    double* sh = (double*)malloc(sizeof(double) * S * d_v_);  /* content adjoint */
    double* mh = (double*)malloc(sizeof(double) * S);         /* mass adjoint    */
    double* gwv = (double*)malloc(sizeof(double) * (kw + kr + 1));
    int32_t* ic = (int32_t*)malloc(sizeof(int32_t) * (kw + kr + 1));
    if (!s || !m || !hs_old || !hm_old || !hread || !iw || !ir || !ww || !wr ||
        !lw || !lr || !sw || !sr || !sh || !mh || !gwv || !ic) {
#pragma omp atomic write
      status = ORC_ENOMEM;
    } else {
      /* 1. forward replay with history */
      if (slot0) {
        memcpy(s, slot0 + bh * S * d_v_, sizeof(double) * S * d_v_);
        memcpy(m, mass0 + bh * S, sizeof(double) * S);
      } else {
        memset(s, 0, sizeof(double) * S * d_v_);
        memset(m, 0, sizeof(double) * S);
      }
      forward_bh(p, b, h, wlogits, rlogits, vin, gamma, mask, s, m, NULL,
                 hs_old, hm_old, hread, iw, ww, lw, sw, ir, wr, lr, sr);
      /* 2. reverse sweep */
      for (int64_t a = 0; a < S; ++a) {
        for (int c = 0; c < d_v_; ++c)
          sh[a * d_v_ + c] = d_slot1 ? d_slot1[(bh * S + a) * d_v_ + c] : 0.0;
        mh[a] = d_mass1 ? d_mass1[bh * S + a] : 0.0;
      }
      for (int64_t t = T - 1; t >= 0; --t) {
        const int64_t row = ((int64_t)b * T + t) * p->H + h;
        if (mask && !mask[(int64_t)b * T + t]) {
          /* a masked token takes no part: every gradient of it is zero */
          for (int64_t i = 0; i < rowlen; ++i) d_wlogits[row * rowlen + i] = 0.0;
          for (int64_t i = 0; i < rowlen; ++i) d_rlogits[row * rowlen + i] = 0.0;
          for (int c = 0; c < d_v_; ++c) d_v[row * d_v_ + c] = 0.0;
          d_gamma[row] = 0.0;
          if (dw_out) for (int j = 0; j < kw; ++j) dw_out[row * kw + j] = 0.0;
          if (dr_out) for (int j = 0; j < kr; ++j) dr_out[row * kr + j] = 0.0;
          continue;
        }
        const double* dO = d_o + row * d_v_;
        const double* vv = vin + row * d_v_;
        const double g = (double)gamma[row];
        /* reads of token t: o_t = sum_j r_j s[a_j] */
        double* drow_r = gwv + kw;
        for (int j = 0; j < kr; ++j) {
          const int32_t a = ir[t * kr + j];
          const double* snap = hread + (t * kr + j) * d_v_;
          double dr = 0.0;
          for (int c = 0; c < d_v_; ++c) dr += (double)dO[c] * snap[c];
          drow_r[j] = dr;
          for (int c = 0; c < d_v_; ++c) sh[(int64_t)a * d_v_ + c] += wr[t * kr + j] * (double)dO[c];
        }
        /* writes of token t, reversed */
        double dgam = 0.0;
        for (int c = 0; c < d_v_; ++c) d_v[row * d_v_ + c] = 0.0;
        for (int j = kw - 1; j >= 0; --j) {
          const int32_t a = iw[t * kw + j];
          const double w = ww[t * kw + j];
          const double m_old = hm_old[t * kw + j];
          const double* s_old = hs_old + (t * kw + j) * d_v_;
          double lam, dlam_dw;
          retention(w, g, &lam, &dlam_dw);
          const double m_new = lam * m_old + w;
          const double eta = (w > 0.0) ? w / (m_new + p->eps) : 0.0;
          double* sha = sh + (int64_t)a * d_v_;
          double deta = 0.0;
          for (int c = 0; c < d_v_; ++c) {
            d_v[row * d_v_ + c] += eta * sha[c];
            deta += sha[c] * ((double)vv[c] - s_old[c]);
          }
          for (int c = 0; c < d_v_; ++c) sha[c] = (1.0 - eta) * sha[c];
          const double den = m_new + p->eps;
          /* eta = w / (m_new + eps), m_new = lam(w, g) m_old + w */
          const double M = mh[a] - ((w > 0.0) ? deta * w / (den * den) : 0.0);
          const double dw = ((w > 0.0) ? deta / den : 0.0) + M + M * m_old * dlam_dw;
          dgam += M * m_old * (-lam * (1.0 - lam));
          mh[a] = lam * M;
          gwv[j] = dw;
        }
        d_gamma[row] = dgam;
        if (dw_out) for (int j = 0; j < kw; ++j) dw_out[row * kw + j] = gwv[j];
        if (dr_out) for (int j = 0; j < kr; ++j) dr_out[row * kr + j] = drow_r[j];
        /* decoded weights back to logits; CAPE does not change the content
         * index, so undo the shift to find the selected digits */
        const int64_t Sx = S;
        for (int j = 0; j < kw; ++j) {
          int32_t a = iw[t * kw + j];
          if (h < p->cape_heads) a = (int32_t)((((int64_t)a - (p->t0 + t) % Sx) % Sx + Sx) % Sx);
          ic[j] = a;
        }
        decode_row_backward(wlogits + row * rowlen, U, P, kw, p->renorm_w, ic, ww + t * kw,
                            lw + t * U, sw[t], gwv, d_wlogits + row * rowlen);
        for (int j = 0; j < kr; ++j) {
          int32_t a = ir[t * kr + j];
          if (h < p->cape_heads) a = (int32_t)((((int64_t)a - (p->t0 + t) % Sx) % Sx + Sx) % Sx);
          ic[j] = a;
        }
        decode_row_backward(rlogits + row * rowlen, U, P, kr, p->renorm_r, ic, wr + t * kr,
                            lr + t * U, sr[t], drow_r, d_rlogits + row * rowlen);
      }
      if (d_slot0) memcpy(d_slot0 + bh * S * d_v_, sh, sizeof(double) * S * d_v_);
      if (d_mass0) memcpy(d_mass0 + bh * S, mh, sizeof(double) * S);
    }
    free(s); free(m); free(hs_old); free(hm_old); free(hread);
    free(iw); free(ir); free(ww); free(wr); free(lw); free(lr); free(sw); free(sr);
    free(sh); free(mh); free(gwv); free(ic);
  }
  return status;
}

/* ------------------------------------------------------------------------ */
/* Event / segment view of slot-parallel execution (paper §4 "Slot-Parallel  */
/* Execution"; ramnet-ops "CUDA execution", parallel mode).                  */
/* ------------------------------------------------------------------------ */

/* Every selected write or read of token t is one event.  Events of the same
 * (b, h, slot) form one segment; segments are laid out by flat id
 * g = (b*H + h)*S + a, and inside a segment events are in time order with
 * the write of a token before its read.  Outputs: seg_offset (B*H*S + 1,
 * exclusive prefix of the segment sizes) and, per event position, its token
 * t, side (0 write, 1 read) and rank j inside that side's top-K.
 * idx_w (B,T,H,k_w), idx_r (B,T,H,k_r) hold final slots. */
int orc_bucket(const orc_problem* p, const int32_t* idx_w, const int32_t* idx_r,
               int64_t* seg_offset, int32_t* ev_t, int32_t* ev_side, int32_t* ev_j) {
  if (check_problem(p) != ORC_OK || !idx_w || !idx_r || !seg_offset) return ORC_EINVAL;
  const int64_t S = slots_of(p);
  const int64_t nseg = (int64_t)p->B * p->H * S;
  int64_t* fill = (int64_t*)calloc((size_t)nseg + 1, sizeof(int64_t));
  if (!fill) return ORC_ENOMEM;
  for (int64_t g = 0; g <= nseg; ++g) seg_offset[g] = 0;
  /* sizes */
  for (int b = 0; b < p->B; ++b)
    for (int64_t t = 0; t < p->T; ++t)
      for (int h = 0; h < p->H; ++h) {
        const int64_t row = ((int64_t)b * p->T + t) * p->H + h;
        const int64_t base = ((int64_t)b * p->H + h) * S;
        for (int j = 0; j < p->k_w; ++j) seg_offset[base + idx_w[row * p->k_w + j] + 1] += 1;
        for (int j = 0; j < p->k_r; ++j) seg_offset[base + idx_r[row * p->k_r + j] + 1] += 1;
      }
  for (int64_t g = 0; g < nseg; ++g) seg_offset[g + 1] += seg_offset[g];
  /* place events in time order; write before read */
  for (int b = 0; b < p->B; ++b)
    for (int64_t t = 0; t < p->T; ++t)
      for (int h = 0; h < p->H; ++h) {
        const int64_t row = ((int64_t)b * p->T + t) * p->H + h;
        const int64_t base = ((int64_t)b * p->H + h) * S;
        for (int side = 0; side < 2; ++side) {
          const int k = side == 0 ? p->k_w : p->k_r;
          const int32_t* id = side == 0 ? idx_w : idx_r;
          for (int j = 0; j < k; ++j) {
            const int64_t g = base + id[row * k + j];
            const int64_t pos = seg_offset[g] + fill[g]++;
            if (ev_t) ev_t[pos] = (int32_t)t;
            if (ev_side) ev_side[pos] = side;
            if (ev_j) ev_j[pos] = j;
          }
        }
      }
  free(fill);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Read epilogue (paper §3.4 "Read-out", last sentence; Fig. 2): per row of  */
/* d_v channels (one token and head), n = o / sqrt(mean_c o_c^2 + eps),      */
/* z = n * gain, y = sigmoid(g) * z.  gain may be NULL (all ones).           */
/* ------------------------------------------------------------------------ */

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static double inv_rms(const double* o, int d_v, double eps) {
  double ss = 0.0;
  for (int c = 0; c < d_v; ++c) ss += o[c] * o[c];
  return 1.0 / sqrt(ss / d_v + eps);
}

int orc_epilogue_forward(int64_t rows, int d_v, const double* o, const double* g,
                         const double* gain, double eps, double* y) {
  if (rows < 0 || d_v < 1 || !(eps >= 0.0) || (rows > 0 && (!o || !g || !y))) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const double* orow = o + r * d_v;
    const double rstd = inv_rms(orow, d_v, eps);
    for (int c = 0; c < d_v; ++c) {
      const double z = orow[c] * rstd * (gain ? gain[c] : 1.0);
      y[r * d_v + c] = sigmoid(g[r * d_v + c]) * z;
    }
  }
  return ORC_OK;
}

/* Gradients of the epilogue: given dL/dy, writes dL/do, dL/dg and (when
 * d_gain is non-NULL) dL/dgain summed over all rows.  With s = sigmoid(g),
 * dz = dy * s, dg = dy * z * s * (1 - s), dn = dz * gain, and the
 * normalisation's Jacobian: do = rstd * (dn - n * mean_c(dn_c * n_c)). */
int orc_epilogue_backward(int64_t rows, int d_v, const double* o, const double* g,
                          const double* gain, double eps, const double* d_y, double* d_o,
                          double* d_g, double* d_gain) {
  if (rows < 0 || d_v < 1 || !(eps >= 0.0) ||
      (rows > 0 && (!o || !g || !d_y || !d_o || !d_g)))
    return ORC_EINVAL;
  if (d_gain) for (int c = 0; c < d_v; ++c) d_gain[c] = 0.0;
  double* n = (double*)malloc(sizeof(double) * d_v);
  double* dn = (double*)malloc(sizeof(double) * d_v);
  if (!n || !dn) { free(n); free(dn); return ORC_ENOMEM; }
  for (int64_t r = 0; r < rows; ++r) {
    const double* orow = o + r * d_v;
    const double rstd = inv_rms(orow, d_v, eps);
    double dot = 0.0;
    for (int c = 0; c < d_v; ++c) {
      const double gc = gain ? gain[c] : 1.0;
      const double s = sigmoid(g[r * d_v + c]);
      n[c] = orow[c] * rstd;
      const double z = n[c] * gc;
      const double dz = d_y[r * d_v + c] * s;
      d_g[r * d_v + c] = d_y[r * d_v + c] * z * s * (1.0 - s);
      if (d_gain) d_gain[c] += dz * n[c];
      dn[c] = dz * gc;
      dot += dn[c] * n[c];
    }
    dot /= d_v;
    for (int c = 0; c < d_v; ++c) d_o[r * d_v + c] = rstd * (dn[c] - n[c] * dot);
  }
  free(n);
  free(dn);
  return ORC_OK;
}
