// Product-softmax row decoder (U >= 2 address digits), shared by the decode
// kernels and the autoregressive step kernel.
//
// A row holds U digit distributions of P logits each (paper §3.2 "Product
// Softmax"; App. B.1): the slot a = sum_u a_u P^(U-1-u) has probability
// prod_u softmax(l_u)[a_u] and is ranked by its key, the float sum of its
// digit logits taken in ascending u starting from 0 (a sum of logs instead of
// a product, paper §4 "Efficient Address Decoding").  The K best slots by
// (key descending, index ascending) are found by a level-by-level prefix
// search (paper §3.2 top-K prefix tree):
//
//   level u extends every kept prefix by the P values of digit u.  The best
//   key any completion of a prefix can reach is its key with the maxima of
//   the remaining digits added in the same order; float addition rounds
//   monotonically, so this bound is exact, and it is the key of a real slot.
//   tau = the K-th largest per-lane maximum of these bounds is the key of K
//   distinct slots, hence at most the K-th best key of the row; every prefix
//   whose bound reaches tau is kept (at least K, more on ties).  No prefix of
//   a top-K slot is ever dropped, whatever the rounding.  At the last level
//   the bound is the key itself and the kept slots are ranked exactly.
//
// Rows whose kept list would overflow KEEP_CAP (massive ties) take K exact
// passes over all P^U slots instead.  Two digits of at most 64 values take
// a shorter register-resident search first (decode_row_u2).
#pragma once
#include "decode.hpp"

namespace ramk {

constexpr int MAX_DIGITS = 14;   // P >= 2 and P^U <= 16384; P = 1 allows U <= 14
constexpr int MAX_ROW = 256;     // U * P of a product row (P <= 128 when U >= 2)
constexpr int KEEP_CAP = 128;    // prefixes kept per level

struct ProdScratch {
  float dig[MAX_ROW];            // the row's logits as float, digit-major
  float dmax[MAX_DIGITS];        // per digit: largest logit
  float dlse[MAX_DIGITS];        //            logsumexp
  float kk[2][KEEP_CAP];         // kept prefixes of the current / next level: key
  int ki[2][KEEP_CAP];           //                                            flat prefix
  float sv[MAX_K];               // selection, in order
  int si[MAX_K];
};

namespace {

// Best key reachable from a prefix of key `key` that ends at digit u.
__device__ __forceinline__ float completion_bound(const ProdScratch& sc, float key, int u, int U) {
  for (int v = u + 1; v < U; ++v) key += sc.dmax[v];
  return key;
}

// Exact rank of each of the `count` candidates (cv, ci) among them; the K best
// go to sv / si in order.  Indices are distinct, so ranks are too.
__device__ __forceinline__ void rank_list(const float* cv, const int* ci, int count, int k,
                                          float* sv, int* si) {
  for (int c = lane_id(); c < count; c += WAVE) {
    const float v = cv[c];
    const int id = ci[c];
    int rank = 0;
    for (int o = 0; o < count; ++o) rank += before(cv[o], ci[o], v, id) ? 1 : 0;
    if (rank < k) { sv[rank] = v; si[rank] = id; }
  }
}

// K exact passes over all S = P^U slots (keys from the digits in LDS), each
// taking the best slot after the previous pick (NaN keys below every
// number, as in exact_k_passes).  Out of line so that its registers do not
// count against the common path.
__device__ __noinline__ void product_k_passes(ProdScratch& sc, int U, int P, int S, int k) {
  const int lane = lane_id();
  const int top = S / P;   // P^(U-1)
  uint32_t pk = 0xFFFFFFFFu;
  int pi = -1;
  for (int r = 0; r < k; ++r) {
    uint32_t bk = 0u;
    int bi = 0x7fffffff;
    float bv = -INFINITY;
    for (int a = lane; a < S; a += WAVE) {
      float key = 0.f;
      int rem = a, stride = top;
      for (int u = 0; u < U; ++u) {
        const int du = rem / stride;
        rem -= du * stride;
        key += sc.dig[u * P + du];
        stride /= P;
      }
      const uint32_t kb = sel_key(key);
      if (key_before(pk, pi, kb, a) && key_before(kb, a, bk, bi)) { bk = kb; bi = a; bv = key; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const uint32_t ok = (uint32_t)__shfl_xor((int)bk, o, WAVE);
      const int oi = __shfl_xor(bi, o, WAVE);
      const float ov = __shfl_xor(bv, o, WAVE);
      if (key_before(ok, oi, bk, bi)) { bk = ok; bi = oi; bv = ov; }
    }
    if (lane == 0) { sc.sv[r] = bv; sc.si[r] = bi; }
    pk = bk;
    pi = bi;
  }
}

// Two digits of at most 64 values, in registers (lane L holds l0[L] and
// l1[L], -inf past P).  The best key with digit-1 value L is fl(M0 + l1[L])
// (M0 the largest digit-0 logit); tau = the K-th largest of these over the
// lanes is the key of K distinct slots, so at most the K-th best key.  As
// fl(M0 + x) is non-decreasing in x, tau = fl(M0 + the K-th largest l1),
// which for bf16 logits is found by a 16-bit search.  Only digit-1 values
// whose bound reaches tau can appear in the top K; for each of them one
// wave-wide add gives the keys of all its slots, and those reaching tau are
// listed and ranked exactly (from registers when at most 64 are listed).
// Returns false, having written nothing to sel_i / sel_w, when the list
// would overflow (massive ties) or hold fewer than K slots (NaN logits).
__device__ __forceinline__ bool decode_row_u2_vals(float l0, float l1, int P, int k, int renorm,
                                                   bool bf16_logits, ProdScratch& sc,
                                                   int* sel_i, float* sel_w) {
  const int lane = lane_id();
  const bool in = lane < P;
  const float M0 = wave_max(l0), M1 = wave_max(l1);
  float s0 = 0.f, s1 = 0.f;
  if (M0 != -INFINITY) s0 = fast_exp2(fmaf(l0, LOG2E, -M0 * LOG2E));
  if (M1 != -INFINITY) s1 = fast_exp2(fmaf(l1, LOG2E, -M1 * LOG2E));
  const float lse0 = M0 + logf(wave_sum(s0));
  const float lse1 = M1 + logf(wave_sum(s1));
  if (lane == 0) {
    sc.dmax[0] = M0;
    sc.dmax[1] = M1;
    sc.dlse[0] = lse0;
    sc.dlse[1] = lse1;
  }
  const float b1 = in ? M0 + l1 : -INFINITY;
  const float l1k = bf16_logits ? kth_lane_max_bf16(l1, k) : kth_lane_max(l1, k);
  const float tau = (l1k == -INFINITY) ? -INFINITY : M0 + l1k;
  uint64_t qual = __ballot(in && b1 >= tau);
  const uint64_t lt = lanemask_lt();
  int count = 0;
  while (qual) {
    const int L = (int)__builtin_ctzll(qual);
    qual &= qual - 1;
    const float l1L = readlane_f(l1, L);
    const float key = l0 + l1L;
    const bool c = in && key >= tau;
    const uint64_t bal = __ballot(c);
    const int pos = count + __popcll(bal & lt);
    if (c && pos < KEEP_CAP) {
      sc.kk[0][pos] = key;
      sc.ki[0][pos] = lane * P + L;
      sc.kk[1][pos] = (l0 - lse0) + (l1L - lse1);   // log-probability of the slot
    }
    count += __popcll(bal);
  }
  if (count > KEEP_CAP || count < k) return false;
  wave_sync();
  // exact rank of every listed slot; the K best to sv / si with their
  // log-probabilities
  if (count <= WAVE) {
    float v = -INFINITY, lpv = 0.f;
    int id = 0x7fffffff;
    if (lane < count) {
      v = sc.kk[0][lane];
      id = sc.ki[0][lane];
      lpv = sc.kk[1][lane];
    }
    int rank = 0;
    for (int o = 0; o < count; ++o)
      rank += before(readlane_f(v, o), readlane_i(id, o), v, id) ? 1 : 0;
    if (lane < count && rank < k) {
      sc.si[rank] = id;
      sc.sv[rank] = lpv;
    }
  } else {
    for (int c = lane; c < count; c += WAVE) {
      const float v = sc.kk[0][c];
      const int id = sc.ki[0][c];
      int rank = 0;
      for (int o = 0; o < count; ++o) rank += before(sc.kk[0][o], sc.ki[0][o], v, id) ? 1 : 0;
      if (rank < k) {
        sc.si[rank] = id;
        sc.sv[rank] = sc.kk[1][c];
      }
    }
  }
  wave_sync();
  float w = 0.f;
  int id = 0;
  if (lane < k) {
    id = sc.si[lane];
    w = expf(sc.sv[lane]);
  }
  if (renorm) {
    const float tot = wave_sum(lane < k ? w : 0.f);
    w = w / tot;
  }
  if (lane < k) { sel_i[lane] = id; sel_w[lane] = w; }
  return true;
}

template <typename IO>
__device__ bool decode_row_u2(const IO* __restrict__ row, int P, int k, int renorm,
                              ProdScratch& sc, int* sel_i, float* sel_w) {
  const int lane = lane_id();
  const bool in = lane < P;
  const float l0 = in ? to_f32(row[lane]) : -INFINITY;
  const float l1 = in ? to_f32(row[P + lane]) : -INFINITY;
  return decode_row_u2_vals(l0, l1, P, k, renorm, sizeof(IO) == 2, sc, sel_i, sel_w);
}

}  // namespace

// Decodes one product row (U * P logits) with the calling wave: the K
// selected flat slots and their probabilities exp(sum_u (l_u[a_u] - lse_u))
// (renormalised if asked) to sel_i / sel_w (lanes < k), and the per-digit
// maxima and logsumexps to sc.dmax / sc.dlse.  Visible to the wave on return.
// try_u2: rows of two digits of at most 64 first take the register search
// (callers that already tried it pass false).
template <typename IO>
__device__ void decode_row_product(const IO* __restrict__ row, int U, int P, int k, int renorm,
                                   ProdScratch& sc, int* sel_i, float* sel_w, bool try_u2 = true) {
  if (try_u2 && U == 2 && P <= WAVE) {
    if (decode_row_u2<IO>(row, P, k, renorm, sc, sel_i, sel_w)) return;
    wave_sync();
  }
  const int lane = lane_id();
  const int UP = U * P;
  for (int e = lane; e < UP; e += WAVE) sc.dig[e] = to_f32(row[e]);
  if (lane == 0) { sc.kk[0][0] = 0.f; sc.ki[0][0] = 0; }
  wave_sync();

  // per digit: maximum and logsumexp (P <= 128: two values per lane)
  for (int u = 0; u < U; ++u) {
    const float x0 = lane < P ? sc.dig[u * P + lane] : -INFINITY;
    const float x1 = lane + WAVE < P ? sc.dig[u * P + lane + WAVE] : -INFINITY;
    const float M = wave_max(fmaxf(x0, x1));
    float s = 0.f;
    if (M != -INFINITY) {
      const float nm = -M * LOG2E;
      s = fast_exp2(fmaf(x0, LOG2E, nm)) + fast_exp2(fmaf(x1, LOG2E, nm));
    }
    const float lse = M + logf(wave_sum(s));
    if (lane == 0) { sc.dmax[u] = M; sc.dlse[u] = lse; }
  }
  wave_sync();

  // candidate c of a level is (kept prefix c / P, digit c % P); a lane walks
  // c = lane, lane + 64, ... keeping (r, d) = (c / P, c % P) by increments
  const uint64_t lt = lanemask_lt();
  const int step_r = WAVE / P, step_d = WAVE % P;
  const int r0 = lane / P, d0 = lane % P;
  int cur = 0, nk = 1;
  bool overflow = false;
  for (int u = 0; u < U; ++u) {
    const int nc = nk * P;
    const float* dg = sc.dig + u * P;
    const float* kk = sc.kk[cur];
    const int* ki = sc.ki[cur];
    float lm = -INFINITY;
    {
      int r = r0, d = d0;
      for (int c = lane; c < nc; c += WAVE) {
        lm = fmaxf(lm, completion_bound(sc, kk[r] + dg[d], u, U));
        r += step_r;
        d += step_d;
        if (d >= P) { d -= P; ++r; }
      }
    }
    const float tau = kth_lane_max(lm, k);
    const int nxt = cur ^ 1;
    int count = 0;
    int r = r0, d = d0;
    for (int c0 = 0; c0 < nc; c0 += WAVE) {
      const bool in = c0 + lane < nc;
      float key = 0.f;
      bool keep = false;
      if (in) {
        key = kk[r] + dg[d];
        keep = completion_bound(sc, key, u, U) >= tau;
      }
      const uint64_t bal = __ballot(keep);
      const int pos = count + __popcll(bal & lt);
      if (keep && pos < KEEP_CAP) {
        sc.kk[nxt][pos] = key;
        sc.ki[nxt][pos] = ki[r] * P + d;
      }
      count += __popcll(bal);
      r += step_r;
      d += step_d;
      if (d >= P) { d -= P; ++r; }
    }
    wave_sync();
    cur = nxt;
    nk = count;
    if (count > KEEP_CAP) { overflow = true; break; }
  }
  if (nk < k) overflow = true;   // NaN logits: fewer than K slots survive
  if (!overflow) {
    rank_list(sc.kk[cur], sc.ki[cur], nk, k, sc.sv, sc.si);
  } else {
    int S = 1;
    for (int u = 0; u < U; ++u) S *= P;
    product_k_passes(sc, U, P, S, k);
  }
  wave_sync();

  float w = 0.f;
  int id = 0;
  if (lane < k) {
    id = sc.si[lane];
    float lp = 0.f;
    int rem = id;
    for (int u = U - 1; u >= 0; --u) {
      const int du = rem % P;
      rem /= P;
      lp += sc.dig[u * P + du] - sc.dlse[u];
    }
    w = expf(lp);
  }
  if (renorm) {
    const float tot = wave_sum(lane < k ? w : 0.f);
    w = w / tot;
  }
  if (lane < k) { sel_i[lane] = id; sel_w[lane] = w; }
}

}  // namespace ramk
