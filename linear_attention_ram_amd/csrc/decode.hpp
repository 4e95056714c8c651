// Row decoder of the RAM-Net attention core, shared by the decode kernels and
// the autoregressive step kernel.  See decode.hip for the algorithm.
#pragma once
#include <type_traits>

#include "common.hpp"

namespace ramk {

constexpr int CAND_CAP = 256;   // candidates kept in LDS per row
constexpr int MAX_K = 64;       // largest top-K per side

// Per-wave LDS work area of the row decoder.
constexpr int STAGE_CAP = 64;   // 16-byte vectors staged per row by the resident decoder

struct DecodeScratch {
  uint64_t ck[CAND_CAP];   // candidate words: cand_word(value, index)
  uint4 stage[STAGE_CAP];
  int stage_c[STAGE_CAP];
  float sv[MAX_K];
  int si[MAX_K];
  int lanes[WAVE];
};

struct DecodeFwdArgs {
  const void* logits[2];   // (N, U * P) io per side
  int32_t* idx[2];         // (N, k) per side
  float* w[2];             // (N, k) per side
  float* lse[2];           // (N, U) per side: logsumexp of each digit
  int k[2];
  int renorm[2];
  int64_t N;               // rows per side
  int S;                   // slots, P^U
  int U, P;                // address digits and digit size
  int nsides;              // 1 or 2 (side 0 = first pointer set)
  int H, T;                // row r is token (r / H) % T of head r % H
  int cape_heads;          // heads h < cape_heads shift the chosen slot by (t0 + t) mod S
  int64_t t0;              // reduced mod S
};

// CAPE (ramnet-ops "Quick start", embed_num; paper App. C): for the first
// cape_heads heads the slot addressed by a token is its content-selected
// index shifted cyclically by the token's absolute position.  The shift of
// row r, or -1 for heads without CAPE.  t0 is already reduced mod S; the
// rows of one call number less than 2^31 (the event count is checked on the
// host), so 32-bit arithmetic suffices.
__device__ __forceinline__ int cape_shift_of(int64_t r, int H, int T, int S, int cape_heads,
                                             int64_t t0) {
  if (cape_heads == 0) return -1;
  const uint32_t r32 = (uint32_t)r;
  const uint32_t q = r32 / (uint32_t)H;           // token row b * T + t
  if ((int)(r32 - q * (uint32_t)H) >= cape_heads) return -1;
  return (int)(((uint32_t)t0 + q % (uint32_t)T) % (uint32_t)S);
}

// Token index b * T + t of row r = (b * T + t) * H + h (the mask index).
__device__ __forceinline__ uint32_t token_of(int64_t r, int H) {
  return (uint32_t)r / (uint32_t)H;
}

struct DecodeBwdArgs {
  const void* logits[2];   // (N, U * P) io
  const float* lse[2];     // (N, U)
  const int32_t* idx[2];
  const float* w[2];
  const float* g[2];       // gradient of the output weights (N, k)
  void* dlogits[2];        // (N, U * P) io
  int k[2];
  int renorm[2];
  int64_t N;
  int S;
  int U, P;
  int nsides;
  int H, T;                // as in DecodeFwdArgs: idx holds shifted slots of CAPE heads
  int cape_heads;
  int64_t t0;
  const uint8_t* mask;     // (B, T) or null: rows of masked tokens get zero gradients
};

hipError_t launch_decode_fwd(const DecodeFwdArgs& a, bool bf16, hipStream_t st);
hipError_t launch_decode_bwd(const DecodeBwdArgs& a, bool bf16, hipStream_t st);

namespace {

// Pairwise sum of an array of 4 or 8 values.
template <int N>
__device__ __forceinline__ float tree_sum(const float (&x)[N]) {
  static_assert(N == 4 || N == 8, "vector of 4 or 8");
  if constexpr (N == 4) return (x[0] + x[1]) + (x[2] + x[3]);
  else return ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
}

// (value, index) order of the selection: larger value first, then lower index.
__device__ __forceinline__ bool before(float v, int i, float v2, int i2) {
  return (v > v2) || (v == v2 && i < i2);
}

template <typename IO>
__device__ __forceinline__ uint4 load_vec(const IO* row, int c, int nvec) {
  return (c < nvec) ? *reinterpret_cast<const uint4*>(row + (int64_t)c * vec16<IO>::E)
                    : neg_inf16<IO>();
}
// Same for a row that is read exactly once.  The load itself is
// unconditional (a clamped address), so all of a lane's loads stay in flight
// together; FULL: the caller knows c < nvec.
template <typename IO, bool FULL>
__device__ __forceinline__ uint4 load_vec_nt(const IO* row, int c, int nvec) {
  if constexpr (FULL) return ld_nt16(row + (int64_t)c * vec16<IO>::E);
  const uint4 t = ld_nt16(row + (int64_t)min(c, nvec - 1) * vec16<IO>::E);
  return (c < nvec) ? t : neg_inf16<IO>();
}

// Makes the compiler forget what it knows about q (emits no code), so values
// unpacked from q earlier are not kept alive for reuse after this point.
template <int NV>
__device__ __forceinline__ void hide_regs(uint4 (&q)[NV]) {
#pragma unroll
  for (int u = 0; u < NV; ++u) asm volatile("" : "+v"(q[u].x), "+v"(q[u].y), "+v"(q[u].z), "+v"(q[u].w));
}

// Order-preserving map of a float to an unsigned integer, and back
// (negative values reversed below the positive ones; -0 just below +0).
__device__ __forceinline__ uint32_t ordered_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// tau = K-th largest lane value m (counted with multiplicity).  Every top-K
// element of the row is >= tau, and lies in a lane whose maximum is >= tau.
// Found bit by bit, from the top, as the largest ordered threshold that K
// lanes reach: one compare and a ballot count per bit, no cross-lane moves.
__device__ __forceinline__ float kth_lane_max(float m, int k) {
  const uint32_t mb = ordered_bits(m);
  const int ku = __builtin_amdgcn_readfirstlane(k);   // uniform: kept in scalar registers
  uint32_t t = 0;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = t | (1u << b);
    t = (__popcll(__ballot(mb >= c)) >= ku) ? c : t;
    t = __builtin_amdgcn_readfirstlane(t);
  }
  return from_ordered(t);
}

// K-th largest lane value with multiplicity, for values that are bf16
// numbers (their ordered bit patterns end in 16 zero bits, or 16 one bits
// for negative values): the same search as kth_lane_max over the upper 16
// bits only.
__device__ __forceinline__ float kth_lane_max_bf16(float m, int k) {
  const uint32_t mb = ordered_bits(m) >> 16;
  const int ku = __builtin_amdgcn_readfirstlane(k);
  uint32_t t = 0;
#pragma unroll
  for (int b = 15; b >= 0; --b) {
    const uint32_t c = t | (1u << b);
    t = (__popcll(__ballot(mb >= c)) >= ku) ? c : t;
    t = __builtin_amdgcn_readfirstlane(t);
  }
  return from_ordered((t << 16) | ((t & 0x8000u) ? 0u : 0xFFFFu));
}

// tau of a row of io values: for bf16 rows the lane maxima are bf16 numbers
// and the 16-bit search finds the same value in half the rounds.
template <typename IO>
__device__ __forceinline__ float kth_lane_max_io(float m, int k) {
  if constexpr (std::is_same<IO, bf16_t>::value) return kth_lane_max_bf16(m, k);
  else return kth_lane_max(m, k);
}

// Exact rank of every one of the `count` candidates in sc among the
// candidates; the K best go to sc.sv / sc.si in order.  A candidate is
// ranked by its word (cand_word): the larger word is the earlier entry in
// (value descending, index ascending) order, and the words of distinct
// indices are distinct, so the rank is the number of larger words.
__device__ __forceinline__ void rank_candidates(DecodeScratch& sc, int count, int k) {
  for (int ci = lane_id(); ci < count; ci += WAVE) {
    const uint64_t mine = sc.ck[ci];
    int rank = 0;
#pragma unroll 4
    for (int o = 0; o < count; ++o) rank += (sc.ck[o] > mine) ? 1 : 0;
    if (rank < k) {
      sc.sv[rank] = from_ordered((uint32_t)(mine >> 32));
      sc.si[rank] = (int)(0xFFFFFFFFu - (uint32_t)mine);
    }
  }
}

// Total order of the exact passes: the ordered bits of a value, with -0 and
// +0 equal and NaN below every number (0), so that a row holding NaN still
// yields K distinct in-range slots.
__device__ __forceinline__ uint32_t sel_key(float x) {
  if (x != x) return 0u;
  return ordered_bits(x == 0.f ? 0.f : x);
}
// Word of a candidate (value x, not NaN, at index i): the ordered bits of x
// (+0 for -0) above the complemented index.
__device__ __forceinline__ uint64_t cand_word(float x, int i) {
  return ((uint64_t)ordered_bits(x == 0.f ? 0.f : x) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
}
__device__ __forceinline__ bool key_before(uint32_t v, int i, uint32_t v2, int i2) {
  return (v > v2) || (v == v2 && i < i2);
}

// Rows with more than CAND_CAP candidates (massive ties), or fewer than K
// (NaN logits): K exact passes over the row in memory, each taking the best
// element after the previous pick in (value desc, index asc) order, to
// sc.sv / sc.si.  Kept out of line so its registers do not count against the
// common path.
template <typename IO>
__device__ __noinline__ void exact_k_passes(const IO* __restrict__ row, int nvec, int k,
                                            DecodeScratch& sc) {
  constexpr int E = vec16<IO>::E;
  const int lane = lane_id();
  uint32_t pk = 0xFFFFFFFFu;   // above every key: the first pass may take any element
  int pi = -1;
  for (int r = 0; r < k; ++r) {
    uint32_t bk = 0u;
    int bi = 0x7fffffff;
    float bv = -INFINITY;
    for (int c = lane; c < nvec; c += WAVE) {
      float x[E];
      unpack16(load_vec<IO>(row, c, nvec), x);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int id = c * E + e;
        const uint32_t key = sel_key(x[e]);
        if (key_before(pk, pi, key, id) && key_before(key, id, bk, bi)) {
          bk = key;
          bi = id;
          bv = x[e];
        }
      }
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

// Weights exp(l - lse) of the K selected entries (optionally renormalised)
// to sel_i / sel_w, lanes < k.
__device__ __forceinline__ void finish_weights(const DecodeScratch& sc, int k, float lse,
                                               int renorm, int* sel_i, float* sel_w) {
  const int lane = lane_id();
  float w = 0.f;
  int id = 0;
  if (lane < k) {
    id = sc.si[lane];
    w = expf(sc.sv[lane] - lse);
  }
  if (renorm) {
    const float tot = wave_sum(lane < k ? w : 0.f);
    w = w / tot;
  }
  if (lane < k) { sel_i[lane] = id; sel_w[lane] = w; }
}

}  // namespace

// Decodes one row of at most NV * 64 16-byte vectors with the calling wave,
// holding the whole row in registers (lane l: vectors l, l + 64, ...):
// one read of the row from memory, then every pass works on registers.
// FULL: the row has exactly NV * 64 vectors.
template <typename IO, int NV, bool FULL>
__device__ __forceinline__ float decode_row_resident(const IO* __restrict__ row, int S, int k, int renorm,
                                     DecodeScratch& sc, int* sel_i, float* sel_w) {
  constexpr int E = vec16<IO>::E;
  const int lane = lane_id();
  const int nvec = FULL ? NV * WAVE : S / E;
  uint4 q[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) q[u] = load_vec_nt<IO, FULL>(row, u * WAVE + lane, nvec);
  float vm[NV];            // maximum of each of the lane's vectors
  float m = -INFINITY;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    float x[E];
    unpack16(q[u], x);
    vm[u] = x[0];
#pragma unroll
    for (int e = 1; e < E; ++e) vm[u] = fmaxf(vm[u], x[e]);
    m = fmaxf(m, vm[u]);
  }
  const float M = wave_max(m);
  // each pass unpacks the packed row again instead of keeping the floats
  hide_regs(q);
  float s = 0.f;
  if (M != -INFINITY) {
    const float nm = -M * LOG2E;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      float x[E];
      unpack16(q[u], x);
      // all exponentials of the vector first, then a tree sum: no sum waits
      // on the exponential just issued
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = fast_exp2(fmaf(x[e], LOG2E, nm));
      s += tree_sum(x);
    }
  }
  const float lse = M + logf(wave_sum(s));
  const float tau = kth_lane_max_io<IO>(m, k);

  // stage the vectors whose maximum reaches tau (they hold every top-K
  // element), then compact their elements >= tau into the candidate list
  const uint64_t lt = lanemask_lt();
  int nq = 0;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int c = u * WAVE + lane;
    const bool qual = c < nvec && vm[u] >= tau;
    const uint64_t bal = __ballot(qual);
    const int pos = nq + __popcll(bal & lt);
    if (qual && pos < STAGE_CAP) {
      sc.stage[pos] = q[u];
      sc.stage_c[pos] = c;
    }
    nq += __popcll(bal);
  }
  wave_sync();
  int count = 0;
  bool overflow = nq > STAGE_CAP;
  if (!overflow) {
    float x[E];
    int base = 0, mine = 0;
    if (lane < nq) {
      unpack16(sc.stage[lane], x);
      base = sc.stage_c[lane] * E;
#pragma unroll
      for (int e = 0; e < E; ++e) mine += (x[e] >= tau) ? 1 : 0;
    }
    const int incl = wave_incl_scan(mine);
    count = readlane_i(incl, WAVE - 1);
    overflow = count > CAND_CAP;
    if (!overflow && lane < nq) {
      int pos = incl - mine;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (x[e] >= tau) { sc.ck[pos] = cand_word(x[e], base + e); ++pos; }
    }
  }
  // fewer than K candidates: NaN logits (they compare false with tau)
  if (count < k) overflow = true;
  wave_sync();
  if (!overflow) rank_candidates(sc, count, k);
  else exact_k_passes<IO>(row, nvec, k, sc);
  wave_sync();
  finish_weights(sc, k, lse, renorm, sel_i, sel_w);
  return lse;
}

// Decodes one row with the calling wave.  Results go to sel_i / sel_w
// (k entries, LDS or registers visible to the wave after the call) and the
// returned lse.  scratch: this wave's LDS area.
template <typename IO>
__device__ float decode_row_wave(const IO* __restrict__ row, int S, int k, int renorm,
                                 DecodeScratch& sc, int* sel_i, float* sel_w) {
  constexpr int E = vec16<IO>::E;
  constexpr int TILE = 8;                 // 16-byte vectors per lane held at once
  const int lane = lane_id();
  const int nvec = S / E;

  // pass 1: online max / sum of exp per lane
  float m = -INFINITY, s = 0.f;
  for (int c0 = 0; c0 < nvec; c0 += WAVE * TILE) {
    uint4 q[TILE];
#pragma unroll
    for (int u = 0; u < TILE; ++u) q[u] = load_vec<IO>(row, c0 + u * WAVE + lane, nvec);
    float tmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < TILE; ++u) {
      float x[E];
      unpack16(q[u], x);
#pragma unroll
      for (int e = 0; e < E; ++e) tmax = fmaxf(tmax, x[e]);
    }
    const float mn = fmaxf(m, tmax);
    if (mn != -INFINITY) {
      s *= (m == -INFINITY) ? 0.f : fast_exp2((m - mn) * LOG2E);
      const float nml = -mn * LOG2E;
#pragma unroll
      for (int u = 0; u < TILE; ++u) {
        float x[E];
        unpack16(q[u], x);
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = fast_exp2(fmaf(x[e], LOG2E, nml));
        s += tree_sum(x);
      }
      m = mn;
    }
  }
  const float M = wave_max(m);
  const float part = (m == -INFINITY) ? 0.f : s * fast_exp2((m - M) * LOG2E);
  const float lse = M + logf(wave_sum(part));

  const float tau = kth_lane_max_io<IO>(m, k);

  // lanes that may hold top-K elements
  const bool winner = (m >= tau);
  const uint64_t wmask = __ballot(winner);
  const int nw = __popcll(wmask);
  if (winner) sc.lanes[__popcll(wmask & lanemask_lt())] = lane;
  wave_sync();

  // compact every element >= tau of those lanes into LDS
  const int per_lane = (nvec + WAVE - 1) / WAVE;
  const int items = nw * per_lane;
  int count = 0;
  bool overflow = false;
  for (int it0 = 0; it0 < items; it0 += WAVE) {
    const int it = it0 + lane;
    float x[E];
    int base = -1, mine = 0;
    if (it < items) {
      const int c = (it % per_lane) * WAVE + sc.lanes[it / per_lane];
      if (c < nvec) {
        unpack16(load_vec<IO>(row, c, nvec), x);
        base = c * E;
#pragma unroll
        for (int e = 0; e < E; ++e) mine += (x[e] >= tau);
      }
    }
    const int incl = wave_incl_scan(mine);
    const int total = readlane_i(incl, WAVE - 1);
    if (count + total > CAND_CAP) { overflow = true; break; }
    int pos = count + incl - mine;
    if (base >= 0) {
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (x[e] >= tau) { sc.ck[pos] = cand_word(x[e], base + e); ++pos; }
    }
    count += total;
  }
  if (count < k) overflow = true;   // NaN logits
  wave_sync();

  if (!overflow) {
    rank_candidates(sc, count, k);
  } else {
    exact_k_passes<IO>(row, nvec, k, sc);
  }
  wave_sync();
  finish_weights(sc, k, lse, renorm, sel_i, sel_w);
  return lse;
}

}  // namespace ramk
