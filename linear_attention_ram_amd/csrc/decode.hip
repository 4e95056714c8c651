// Address decoding of the RAM-Net attention core (paper §3.1-3.2).  Rows of
// U >= 2 digits go through the product decoder of decode_prod.hpp; the rest
// of this comment is the one-digit case (U = 1).
// Per (token, head, side) row of S logits, lse = logsumexp, the K
// largest logits by (value descending, index ascending), and their
// un-renormalised probabilities exp(l - lse), optionally renormalised
// (paper App. B.2 "Addressing"; ramnet-ops "Arguments", top_k_re_norm).
//
// One wavefront decodes one row.  Lane l owns the 16-byte vectors
// l, l + 64, l + 128, ... of the row, so every load instruction of the wave
// reads 1 KiB of contiguous HBM.
//   pass 1  streaming: per-lane running max and sum of exp (online softmax),
//           then a wave reduction gives lse;
//   select  the K-th largest per-lane maximum tau is a lower bound of the
//           row's K-th largest value, so every top-K element lies in a lane
//           whose maximum is >= tau and is itself >= tau.  Those lanes'
//           vectors are re-read (they were just streamed, so they come from
//           cache), the elements >= tau are compacted into LDS, and each
//           candidate's rank is counted exactly.  Rows with more than
//           CAND_CAP candidates (massive ties) take an exact K-pass fallback.
#include <type_traits>
#include <utility>

#include "decode.hpp"
#include "decode_prod.hpp"

namespace ramk {

// One wave per row; rows of side 0 first, then side 1.  The stored index is
// the slot the token addresses (CAPE-shifted for CAPE heads).  NV > 0: rows of at
// most NV * 64 vectors, held in registers; NV = 0: any length, streamed.
// For rows of up to 16 KiB the results of the workgroup's rows are gathered
// in LDS and written as contiguous pieces (k indices, k weights and one lse
// per row) with streaming stores: small stores scattered through the read
// stream cost far more HBM time than their bytes.
constexpr int FWD_ROWS = 4;   // rows (waves) per decode_fwd workgroup
constexpr int U2_ROWS = 4;    // two-digit rows per wave of the U = 2 kernels

template <typename IO, int NV, bool FULL = false>
__global__ __launch_bounds__(FWD_ROWS * WAVE) void decode_fwd_kernel(DecodeFwdArgs a) {
  // rows of up to 16 KiB: their results are a large enough share of the
  // traffic to be worth the workgroup barrier
  constexpr bool STAGED = NV > 0 && NV <= 16;
  __shared__ DecodeScratch scratch[FWD_ROWS];
  __shared__ int s_idx[FWD_ROWS][MAX_K];
  __shared__ float s_w[FWD_ROWS][MAX_K];
  __shared__ float s_lse[FWD_ROWS];
  const int wv = threadIdx.x >> 6;
  const int lane = lane_id();
  const int64_t total = (int64_t)a.nsides * a.N;
  const int64_t r0 = (int64_t)blockIdx.x * FWD_ROWS;
  const int64_t grow = r0 + wv;
  const int side = grow >= a.N ? 1 : 0;   // nsides <= 2
  const int64_t row = grow - (int64_t)side * a.N;
  const int k = a.k[side];
  if (grow < total) {
    const IO* src = reinterpret_cast<const IO*>(a.logits[side]) + row * (int64_t)a.S;
    float lse;
    if constexpr (NV > 0)
      lse = decode_row_resident<IO, NV, FULL>(src, a.S, k, a.renorm[side], scratch[wv],
                                              s_idx[wv], s_w[wv]);
    else
      lse = decode_row_wave<IO>(src, a.S, k, a.renorm[side], scratch[wv], s_idx[wv], s_w[wv]);
    wave_sync();
    if (lane < k) {
      const int shift = cape_shift_of(row, a.H, a.T, a.S, a.cape_heads, a.t0);
      const int id = s_idx[wv][lane];
      s_idx[wv][lane] = (shift < 0) ? id : (id + shift) % a.S;
    }
    if (lane == 0) s_lse[wv] = lse;
  }
  if constexpr (STAGED) __syncthreads();
  else wave_sync();
  const int side_last = r0 + FWD_ROWS - 1 >= a.N ? 1 : 0;
  if (STAGED && r0 + FWD_ROWS - 1 < total && side_last == (r0 >= a.N ? 1 : 0)) {
    // all rows of one side: FWD_ROWS * k entries of idx and of w from row0 * k, FWD_ROWS of lse
    const int sd = side_last;
    const int kk = a.k[sd];
    const int64_t row0 = r0 - (int64_t)sd * a.N;
    for (int e = threadIdx.x; e < 2 * FWD_ROWS * kk; e += FWD_ROWS * WAVE) {
      const int f = e < FWD_ROWS * kk ? e : e - FWD_ROWS * kk;
      const int j = f / kk, c = f - j * kk;
      if (e < FWD_ROWS * kk) __builtin_nontemporal_store(s_idx[j][c], a.idx[sd] + row0 * kk + f);
      else __builtin_nontemporal_store(s_w[j][c], a.w[sd] + row0 * kk + f);
    }
    if (threadIdx.x < FWD_ROWS) __builtin_nontemporal_store(s_lse[threadIdx.x], a.lse[sd] + row0 + threadIdx.x);
  } else if (grow < total) {
    if (lane < k) {
      a.idx[side][row * k + lane] = s_idx[wv][lane];
      a.w[side][row * k + lane] = s_w[wv][lane];
    }
    if (lane == 0) a.lse[side][row] = s_lse[wv];
  }
}

// gw_j = g_j w_j of lane j < k (0 in the other lanes, where g and w are 0).
// Renormalised weights w = p / sum p: the gradient reaching the
// un-renormalised p_j times p_j is (g_j - sum_i g_i w_i) w_j.
__device__ __forceinline__ float decode_gw(float gj, float wj, int renorm) {
  if (renorm) return (gj - wave_sum(gj * wj)) * wj;
  return gj * wj;
}

// Decode backward: with g_j the gradient of the j-th output weight,
// gw_j = g_j w_j (renormalised: gw_j = (g_j - sum_i g_i w_i) w_j),
// dl_i = [i = a_j] gw_j - p_i sum_j gw_j, p = softmax(l) = exp(l - lse).
// One wave per 1 KiB vector row (64 lanes x 16 bytes) of a logits row, and
// one wave per workgroup: the row's scalars (lse and lanes j < k: g_j, w_j,
// a_j) are requested together with the wave's one vector, so every load of
// the wave is in flight at once.  A selected entry a_j inside the wave's
// vector row takes gw_j added to its streamed value -p_i sum_j gw_j (the
// same sum, in the same order, as gw_j + (-sum) p_{a_j}).
template <typename IO>
__global__ __launch_bounds__(WAVE) void decode_bwd_vec_kernel(DecodeBwdArgs a) {
  constexpr int E = vec16<IO>::E;
  const int lane = lane_id();
  const int nvec = a.S / E;
  const int vrows = (nvec + WAVE - 1) / WAVE;
  const int64_t grow = (int64_t)blockIdx.x / vrows;
  const int part = (int)((int64_t)blockIdx.x - grow * vrows);
  if (grow >= (int64_t)a.nsides * a.N) return;
  const int side = grow >= a.N ? 1 : 0;   // nsides <= 2
  const int64_t row = grow - (int64_t)side * a.N;
  const int k = a.k[side];
  const IO* __restrict__ src = reinterpret_cast<const IO*>(a.logits[side]) + row * (int64_t)a.S;
  IO* __restrict__ dst = reinterpret_cast<IO*>(a.dlogits[side]) + row * (int64_t)a.S;
  const int c = part * WAVE + lane;
  const bool has = c < nvec;
  if (a.mask && !a.mask[token_of(row, a.H)]) {
    // a masked token takes no part in the computation: zero gradient
    if (has) st_nt16(dst + (int64_t)c * E, make_uint4(0, 0, 0, 0));
    return;
  }
  uint4 q = ld_nt16(src + (int64_t)min(c, nvec - 1) * E);   // clamped: in bounds
  float gj = 0.f, wj = 0.f;
  int aj = -1;
  if (lane < k) {
    gj = a.g[side][row * k + lane];
    wj = a.w[side][row * k + lane];
    aj = a.idx[side][row * k + lane];
  }
  const float nl = -a.lse[side][row] * LOG2E;
  if (lane < k) {
    // the logit behind a CAPE slot is the content index (slot - shift)
    const int shift = cape_shift_of(row, a.H, a.T, a.S, a.cape_heads, a.t0);
    if (shift >= 0) aj = (aj - shift + a.S) % a.S;
  }
  const float gw = decode_gw(gj, wj, a.renorm[side]);
  const float ntot = -wave_sum(gw);
  float x[E];
  unpack16(q, x);
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = ntot * fast_exp2(fmaf(x[e], LOG2E, nl));
  // selected entries inside this vector row (usually none)
  uint64_t fixes = __ballot(lane < k && aj / (E * WAVE) == part);
  while (fixes) {
    const int j = (int)__builtin_ctzll(fixes);
    fixes &= fixes - 1;
    const int id = readlane_i(aj, j);
    const float gwj = readlane_f(gw, j);
    const bool mine = lane == (id / E) % WAVE;
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = (mine && id % E == e) ? gwj + x[e] : x[e];
  }
  if (has) st_nt16(dst + (int64_t)c * E, pack16(x));
}

// Product rows (U >= 2 digits, see decode_prod.hpp): one wave per row, rows
// of side 0 first.  lse holds the U per-digit logsumexps of each row.
template <typename IO>
__global__ __launch_bounds__(256) void decode_fwd_prod_kernel(DecodeFwdArgs a) {
  __shared__ ProdScratch scratch[4];
  __shared__ int s_idx[4][MAX_K];
  __shared__ float s_w[4][MAX_K];
  const int wv = threadIdx.x >> 6;
  const int lane = lane_id();
  const int64_t grow = (int64_t)blockIdx.x * 4 + wv;
  if (grow >= (int64_t)a.nsides * a.N) return;
  const int side = grow >= a.N ? 1 : 0;   // nsides <= 2
  const int64_t row = grow - (int64_t)side * a.N;
  const int UP = a.U * a.P;
  const IO* src = reinterpret_cast<const IO*>(a.logits[side]) + row * (int64_t)UP;
  const int k = a.k[side];
  decode_row_product<IO>(src, a.U, a.P, k, a.renorm[side], scratch[wv], s_idx[wv], s_w[wv]);
  wave_sync();
  if (lane < k) {
    const int shift = cape_shift_of(row, a.H, a.T, a.S, a.cape_heads, a.t0);
    const int id = s_idx[wv][lane];
    a.idx[side][row * k + lane] = (shift < 0) ? id : (id + shift) % a.S;
    a.w[side][row * k + lane] = s_w[wv][lane];
  }
  if (lane < a.U) a.lse[side][row * a.U + lane] = scratch[wv].dlse[lane];
}

// Two-digit rows of at most 64 logits per digit (decode_row_u2_vals): R rows
// per wave, every row's logits requested before the first row is decoded,
// so the R rows share one memory round trip.  A row whose register search
// gives up (massive ties, NaN) takes the general prefix search.
template <typename IO, int R>
__global__ __launch_bounds__(256) void decode_fwd_u2_kernel(DecodeFwdArgs a) {
  __shared__ ProdScratch scratch[4];
  __shared__ int s_idx[4][MAX_K];
  __shared__ float s_w[4][MAX_K];
  const int wv = threadIdx.x >> 6;
  const int lane = lane_id();
  const int64_t total = (int64_t)a.nsides * a.N;
  const int64_t g0 = ((int64_t)blockIdx.x * 4 + wv) * R;
  const int P = a.P;
  const bool in = lane < P;
  float l0[R], l1[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t grow = g0 + r;
    const bool valid = grow < total;
    const int side = grow >= a.N ? 1 : 0;
    const int64_t row = grow - (int64_t)side * a.N;
    const IO* src = reinterpret_cast<const IO*>(a.logits[side]) + row * (int64_t)(2 * P);
    l0[r] = (valid && in) ? to_f32(src[lane]) : -INFINITY;
    l1[r] = (valid && in) ? to_f32(src[P + lane]) : -INFINITY;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t grow = g0 + r;
    if (grow >= total) break;
    const int side = grow >= a.N ? 1 : 0;
    const int64_t row = grow - (int64_t)side * a.N;
    const int k = a.k[side];
    if (!decode_row_u2_vals(l0[r], l1[r], P, k, a.renorm[side], sizeof(IO) == 2, scratch[wv],
                            s_idx[wv], s_w[wv])) {
      wave_sync();
      const IO* src = reinterpret_cast<const IO*>(a.logits[side]) + row * (int64_t)(2 * P);
      decode_row_product<IO>(src, 2, P, k, a.renorm[side], scratch[wv], s_idx[wv], s_w[wv], false);
    }
    wave_sync();
    if (lane < k) {
      const int shift = cape_shift_of(row, a.H, a.T, a.S, a.cape_heads, a.t0);
      const int id = s_idx[wv][lane];
      a.idx[side][row * k + lane] = (shift < 0) ? id : (id + shift) % a.S;
      a.w[side][row * k + lane] = s_w[wv][lane];
    }
    if (lane < 2) a.lse[side][row * 2 + lane] = scratch[wv].dlse[lane];
    wave_sync();   // the next row rewrites the scratch
  }
}

// Decode backward of U = 2 rows of P <= 64 (P a multiple of 4) with k <= 16,
// four rows per wave: DPP row r (lanes 16r .. 16r + 15) takes logits row r,
// lane p of it holds entries 4p .. 4p + 3 of each digit (one 8- or 16-byte
// vector per digit), and lane j < k of it holds selection j, broadcast to its
// row with row_newbcast.  The same terms in the same order as the one-row
// kernel below: dl_u[i] = -p_u[i] sum_j gw_j, then gw_j added in ascending j
// to the entry holding digit u of a_j.
constexpr int U2_BWD_K = 16;
template <int J>
__device__ __forceinline__ int row_bcast_i(int x) {
  return __builtin_amdgcn_mov_dpp(x, 0x150 + J, 0xF, 0xF, true);
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<DPP_XOR1>(x);
  x += dpp<DPP_XOR2>(x);
  x += dpp<DPP_HALF_MIRROR>(x);
  return x + dpp<DPP_MIRROR>(x);
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t row16_sum_u(uint32_t x) {
  x += dpp_u<DPP_XOR1>(x);
  x += dpp_u<DPP_XOR2>(x);
  x += dpp_u<DPP_HALF_MIRROR>(x);
  return x + dpp_u<DPP_MIRROR>(x);
}
template <typename IO> struct Vec4;
template <> struct Vec4<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float (&x)[4]) {
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    x[0] = __uint_as_float(q.x << 16);
    x[1] = __uint_as_float(q.x & 0xffff0000u);
    x[2] = __uint_as_float(q.y << 16);
    x[3] = __uint_as_float(q.y & 0xffff0000u);
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float (&x)[4]) {
    *reinterpret_cast<uint2*>(p) = make_uint2(cvt2bf(x[0], x[1]), cvt2bf(x[2], x[3]));
  }
};
template <> struct Vec4<float> {
  static __device__ __forceinline__ void load(const float* p, float (&x)[4]) {
    const float4 q = *reinterpret_cast<const float4*>(p);
    x[0] = q.x; x[1] = q.y; x[2] = q.z; x[3] = q.w;
  }
  static __device__ __forceinline__ void store(float* p, const float (&x)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
};
template <typename IO>
__global__ __launch_bounds__(256) void decode_bwd_u2_kernel(DecodeBwdArgs a) {
  const int lane = lane_id();
  const int p = lane & 15;
  const int64_t grow = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  const bool live = grow < (int64_t)a.nsides * a.N;
  const int side = (live && grow >= a.N) ? 1 : 0;   // nsides <= 2
  const int64_t row = live ? grow - (int64_t)side * a.N : 0;
  const int k = a.k[side];
  const int P = a.P;
  const bool own = live && 4 * p < P;
  const bool masked = live && a.mask && !a.mask[token_of(row, a.H)];
  float gj = 0.f, wj = 0.f;
  int aj0 = -1, aj1 = -1;
  if (live && p < k) {
    gj = a.g[side][row * k + p];
    wj = a.w[side][row * k + p];
    int aj = a.idx[side][row * k + p];
    const int shift = cape_shift_of(row, a.H, a.T, a.S, a.cape_heads, a.t0);
    if (shift >= 0) aj = (aj - shift + a.S) % a.S;
    aj0 = aj / P;
    aj1 = aj - aj0 * P;
  }
  // the row sums run with every lane active (lanes past k hold zeros)
  const float gwr = a.renorm[side] ? (gj - row16_sum(gj * wj)) * wj : gj * wj;
  const float gw = masked ? 0.f : gwr;
  const float ntot = -row16_sum(gw);
  float x0[4] = {0.f, 0.f, 0.f, 0.f}, x1[4] = {0.f, 0.f, 0.f, 0.f};
  float nl0 = 0.f, nl1 = 0.f;
  const IO* src = reinterpret_cast<const IO*>(a.logits[side]) + row * (int64_t)(2 * P);
  IO* dst = reinterpret_cast<IO*>(a.dlogits[side]) + row * (int64_t)(2 * P);
  if (own) {
    Vec4<IO>::load(src + 4 * p, x0);
    Vec4<IO>::load(src + P + 4 * p, x1);
    nl0 = -a.lse[side][row * 2] * LOG2E;
    nl1 = -a.lse[side][row * 2 + 1] * LOG2E;
  }
  float acc0[4], acc1[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc0[e] = ntot * fast_exp2(fmaf(x0[e], LOG2E, nl0));
    acc1[e] = ntot * fast_exp2(fmaf(x1[e], LOG2E, nl1));
  }
  const int base = 4 * p;
  auto add = [&](auto J) {
    constexpr int j = decltype(J)::value;
    const float g = dpp<0x150 + j>(gw);
    const int d0 = row_bcast_i<j>(aj0) - base, d1 = row_bcast_i<j>(aj1) - base;
    if (j < k) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc0[e] = (d0 == e) ? acc0[e] + g : acc0[e];
        acc1[e] = (d1 == e) ? acc1[e] + g : acc1[e];
      }
    }
  };
  add(std::integral_constant<int, 0>{});  add(std::integral_constant<int, 1>{});
  add(std::integral_constant<int, 2>{});  add(std::integral_constant<int, 3>{});
  add(std::integral_constant<int, 4>{});  add(std::integral_constant<int, 5>{});
  add(std::integral_constant<int, 6>{});  add(std::integral_constant<int, 7>{});
  add(std::integral_constant<int, 8>{});  add(std::integral_constant<int, 9>{});
  add(std::integral_constant<int, 10>{}); add(std::integral_constant<int, 11>{});
  add(std::integral_constant<int, 12>{}); add(std::integral_constant<int, 13>{});
  add(std::integral_constant<int, 14>{}); add(std::integral_constant<int, 15>{});
  if (own) {
    if (masked) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc0[e] = acc1[e] = 0.f;
    }
    Vec4<IO>::store(dst + 4 * p, acc0);
    Vec4<IO>::store(dst + P + 4 * p, acc1);
  }
}

// U = 2 rows of P <= 64 (P a multiple of 4, at least 4K entries) with K <= 16,
// four rows per wave in the layout of decode_bwd_u2_kernel (DPP row r takes
// logits row r, lane p entries 4p .. 4p + 3 of each digit).  The selection is
// that of decode_row_u2_vals, made with row-local steps:
//   tau = max(fl(M0 + v1), fl(v0 + M1)), v_u a lower bound of the K-th
//   largest logit of digit u (the largest 16-bit prefix of the ordered bits
//   that K of its values reach; for bf16 logits that value itself), so K
//   distinct slots reach tau and tau is at most the K-th best key;
//   every slot with key fl(l0[a] + l1[b]) >= tau is listed (only a digit-0
//   value with fl(l0[a] + M1) >= tau and a digit-1 value with
//   fl(M0 + l1[b]) >= tau can give one, so those pairs are tried) as a
//   64-bit word: its
//   ordered key, then its index complemented in 16 bits, then its list
//   position, so that the larger word is the earlier slot in (key
//   descending, index ascending) and names its log-probability in the list;
//   the K best in order: where every row of the wave lists at most 32 slots,
//   by each word's rank (the number of larger words of its row, the words
//   being distinct); otherwise by K rounds of a row maximum over the words.
// Rows whose list would overflow or hold fewer than K slots (NaN logits, a
// bound that is no number) are marked and redone by the whole-wave path in a
// second kernel, whose registers then do not limit this one's occupancy.
constexpr int U2X_CAP = 64;    // listed slots per row
constexpr int U2X_QCAP = 24;   // listed values of each digit per row (at most 32)
constexpr int U2X_K = 16;
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<DPP_XOR1>(x));
  x = fmaxf(x, dpp<DPP_XOR2>(x));
  x = fmaxf(x, dpp<DPP_HALF_MIRROR>(x));
  return fmaxf(x, dpp<DPP_MIRROR>(x));
}
// Inclusive sum of x over the lanes of the DPP row up to this one.
__device__ __forceinline__ int row16_incl(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);
  return x;
}
__device__ __forceinline__ int row16_last(int x) {   // lane 15 of the row
  return __builtin_amdgcn_mov_dpp(x, 0x15F, 0xF, 0xF, true);
}
// Larger of two 64-bit words over the lanes of the DPP row (every lane gets it).
template <int CTRL>
__device__ __forceinline__ uint64_t max64_step(uint64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)x, CTRL, 0xF, 0xF, true);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(x >> 32), CTRL, 0xF, 0xF, true);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > x ? o : x;
}
__device__ __forceinline__ uint64_t row16_max64(uint64_t x) {
  x = max64_step<DPP_XOR1>(x);
  x = max64_step<DPP_XOR2>(x);
  x = max64_step<DPP_HALF_MIRROR>(x);
  return max64_step<DPP_MIRROR>(x);
}
// A 64-bit word of the lane S places further along the DPP row (rotating).
template <int S>
__device__ __forceinline__ uint64_t row_ror64(uint64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)x, 0x120 + S, 0xF, 0xF, true);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(x >> 32), 0x120 + S, 0xF, 0xF, true);
  return ((uint64_t)hi << 32) | lo;
}
// Ranks of two words per lane among the 32 words of the lane's DPP row: the
// number of words of the row larger than each (distinct words get distinct
// ranks; a zero word is larger than none).
template <int... S>
__device__ __forceinline__ void row32_ranks(uint64_t w0, uint64_t w1, int& n0, int& n1,
                                            std::integer_sequence<int, S...>) {
  n0 = (w1 > w0) ? 1 : 0;
  n1 = (w0 > w1) ? 1 : 0;
  auto step = [&](auto R) {
    constexpr int s = decltype(R)::value + 1;
    const uint64_t o0 = row_ror64<s>(w0), o1 = row_ror64<s>(w1);
    n0 += ((o0 > w0) ? 1 : 0) + ((o1 > w0) ? 1 : 0);
    n1 += ((o0 > w1) ? 1 : 0) + ((o1 > w1) ? 1 : 0);
    // one rotation at a time (the counts are taken after each, so the
    // compiler keeps no more than one rotation's words live)
    asm volatile("" : "+v"(n0), "+v"(n1));
  };
  (step(std::integral_constant<int, S>{}), ...);
}

template <typename IO>
__global__ __launch_bounds__(256) void decode_fwd_u2x_kernel(DecodeFwdArgs a) {
  // per wave: the lists of its four rows
  struct Lists {
    uint64_t c_word[4][U2X_CAP];   // [row][slot]: ordered key, complemented index, position
    float c_lp[4][U2X_CAP];        // log-probability of the slot
    float a_v[4][U2X_QCAP];        // A: qualifying digit-0 values
    int a_i[4][U2X_QCAP];          //    and their indices
    float b_v[4][U2X_QCAP];        // B: qualifying digit-1 values
    int b_i[4][U2X_QCAP];          //    and their indices
    uint32_t top[4][U2X_K];        // low halves of the K best words, in order
  };
  __shared__ Lists lds[4];
  const int wv = threadIdx.x >> 6;
  Lists& L = lds[wv];
  const int lane = lane_id();
  const int r = lane >> 4, p = lane & 15;
  const int64_t total = (int64_t)a.nsides * a.N;
  const int64_t g0 = ((int64_t)blockIdx.x * 4 + wv) * 4;
  const int64_t grow = g0 + r;
  const bool live = grow < total;
  const int side = (live && grow >= a.N) ? 1 : 0;   // nsides <= 2
  const int64_t row = live ? grow - (int64_t)side * a.N : 0;
  const int k = a.k[side];
  const int P = a.P;
  const bool own = live && 4 * p < P;
  float x0[4], x1[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) x0[e] = x1[e] = -INFINITY;
  if (own) {
    const IO* src = reinterpret_cast<const IO*>(a.logits[side]) + row * (int64_t)(2 * P);
    Vec4<IO>::load(src + 4 * p, x0);
    Vec4<IO>::load(src + P + 4 * p, x1);
  }
  // digit maxima and logsumexps over the row
  const float m0 = fmaxf(fmaxf(x0[0], x0[1]), fmaxf(x0[2], x0[3]));
  const float m1 = fmaxf(fmaxf(x1[0], x1[1]), fmaxf(x1[2], x1[3]));
  const float M0 = row16_max(m0), M1 = row16_max(m1);
  float s0 = 0.f, s1 = 0.f;
  if (M0 != -INFINITY) {
    const float n = -M0 * LOG2E;
#pragma unroll
    for (int e = 0; e < 4; ++e) s0 += fast_exp2(fmaf(x0[e], LOG2E, n));
  }
  if (M1 != -INFINITY) {
    const float n = -M1 * LOG2E;
#pragma unroll
    for (int e = 0; e < 4; ++e) s1 += fast_exp2(fmaf(x1[e], LOG2E, n));
  }
  const float lse0 = M0 + logf(row16_sum(s0));
  const float lse1 = M1 + logf(row16_sum(s1));
  // v0, v1: the largest 16-bit ordered prefixes that K values of digit 0 and
  // of digit 1 reach (for bf16 logits the K-th largest values themselves);
  // the two searches share one loop, their counts one row sum
  uint32_t ob0[4], ob1[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ob0[e] = ordered_bits(x0[e]) >> 16;
    ob1[e] = ordered_bits(x1[e]) >> 16;
  }
  uint32_t t0 = 0, t1 = 0;
#pragma unroll
  for (int b = 15; b >= 0; --b) {
    const uint32_t c0 = t0 | (1u << b), c1 = t1 | (1u << b);
    uint32_t n0 = 0, n1 = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      n0 += (ob0[e] >= c0) ? 1u : 0u;
      n1 += (ob1[e] >= c1) ? 1u : 0u;
    }
    const uint32_t tot = row16_sum_u(n0 | (n1 << 8));   // count0 + 256 count1, both <= 64
    t0 = ((tot & 0xFFu) >= (uint32_t)k) ? c0 : t0;
    t1 = ((tot >> 8) >= (uint32_t)k) ? c1 : t1;
  }
  // K distinct slots (argmax l0, b) reach fl(M0 + v1) and K distinct slots
  // (a, argmax l1) reach fl(v0 + M1): either is at most the K-th best key
  // (fmaxf keeps the number when one bound is NaN)
  const float tau = fmaxf(M0 + from_ordered(t1 << 16), from_ordered(t0 << 16) + M1);
  // A: the row's digit-0 values that reach tau together with the largest
  // digit-1 value; B: its digit-1 values that reach tau together with the
  // largest digit-0 value.  Float addition is monotone, so every slot whose
  // key reaches tau pairs an entry of A with one of B.  Both are listed in LDS.
  auto list_reaching = [&](const float (&x)[4], float best_other, float* vals, int* ids) {
    bool f[4];
    int n = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = own && x[e] + best_other >= tau;
      n += f[e] ? 1 : 0;
    }
    const int incl = row16_incl(n);
    int pos = incl - n;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (f[e]) {
        if (pos < U2X_QCAP) {
          vals[pos] = x[e];
          ids[pos] = 4 * p + e;
        }
        ++pos;
      }
    }
    return row16_last(incl);
  };
  int na = list_reaching(x0, M1, L.a_v[r], L.a_i[r]);
  int nb = list_reaching(x1, M0, L.b_v[r], L.b_i[r]);
  const bool q_over = na > U2X_QCAP || nb > U2X_QCAP;   // such a row takes the whole-wave path
  if (q_over) na = nb = 0;
  wave_sync();
  // every slot reaching tau: lane p holds entries p and p + 16 of B and
  // meets the entries of A one after another
  const bool has0 = p < nb, has1 = p + 16 < nb;
  const float bv0 = has0 ? L.b_v[r][p] : 0.f, bv1 = has1 ? L.b_v[r][p + 16] : 0.f;
  const int bi0 = has0 ? L.b_i[r][p] : 0, bi1 = has1 ? L.b_i[r][p + 16] : 0;
  const int na_max = __builtin_amdgcn_readfirstlane((int)wave_max((float)na));
  int count = 0;
  auto put = [&](float av, int ai, float bv, int bi, int pos) {
    const float key = av + bv;
    const uint32_t id = (uint32_t)(ai * P + bi);   // < 2^12
    L.c_word[r][pos] = ((uint64_t)sel_key(key) << 32) | ((uint32_t)(0xFFFFu - id) << 16) |
                       (uint32_t)pos;
    L.c_lp[r][pos] = (av - lse0) + (bv - lse1);
  };
  for (int i = 0; i < na_max; ++i) {
    const bool ok = i < na;
    const float av = ok ? L.a_v[r][i] : 0.f;
    const int ai = ok ? L.a_i[r][i] : 0;
    const bool f0 = ok && has0 && av + bv0 >= tau;
    const bool f1 = ok && has1 && av + bv1 >= tau;
    const int nc = (f0 ? 1 : 0) + (f1 ? 1 : 0);
    const int incl = row16_incl(nc);
    int pos = count + incl - nc;
    if (f0) {
      if (pos < U2X_CAP) put(av, ai, bv0, bi0, pos);
      ++pos;
    }
    if (f1 && pos < U2X_CAP) put(av, ai, bv1, bi1, pos);
    count += row16_last(incl);
  }
  const bool failed = live && (q_over || count > U2X_CAP || count < k);
  wave_sync();
  uint32_t my_word = 0;   // lane p: low half of the p-th best word
  const int listed = (live && !failed) ? count : 0;
  const int n_max = __builtin_amdgcn_readfirstlane((int)wave_max((float)listed));
  if (n_max <= 32) {
    // lane p holds listed words p and p + 16 (a missing one is 0); the word
    // of rank n < K goes to entry n of the row's top list
    const uint64_t w0 = (p < listed) ? L.c_word[r][p] : 0ull;
    const uint64_t w1 = (p + 16 < listed) ? L.c_word[r][p + 16] : 0ull;
    int n0, n1;
    row32_ranks(w0, w1, n0, n1, std::make_integer_sequence<int, 15>{});
    if (w0 != 0ull && n0 < k) L.top[r][n0] = (uint32_t)w0;
    if (w1 != 0ull && n1 < k) L.top[r][n1] = (uint32_t)w1;
    wave_sync();
    if (listed > 0 && p < k) my_word = L.top[r][p];
  } else {
    // K rounds of the row maximum over the listed words (lane p holds the
    // listed slots p, p + 16, ...; a taken or missing slot is 0)
    constexpr int PER_LANE = U2X_CAP / 16;
    static_assert(U2X_CAP % 16 == 0, "lanes hold whole shares of the list");
    uint64_t wd[PER_LANE];
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) {
      const int c = p + 16 * j;
      wd[j] = (c < listed) ? L.c_word[r][c] : 0ull;
    }
    const int k_max = __builtin_amdgcn_readfirstlane((int)wave_max((float)(live ? k : 0)));
    uint64_t best = wd[0];
#pragma unroll
    for (int j = 1; j < PER_LANE; ++j) best = wd[j] > best ? wd[j] : best;
    for (int rnd = 0; rnd < k_max; ++rnd) {
      const uint64_t win = row16_max64(best);
      if (p == rnd) my_word = (uint32_t)win;
      if (win != 0ull && best == win) {   // this lane held it: take it out
#pragma unroll
        for (int j = 0; j < PER_LANE; ++j) wd[j] = (wd[j] == win) ? 0ull : wd[j];
        best = wd[0];
#pragma unroll
        for (int j = 1; j < PER_LANE; ++j) best = wd[j] > best ? wd[j] : best;
      }
    }
  }
  if (live && !failed) {
    float w = 0.f;
    if (p < k) w = expf(L.c_lp[r][my_word & 0xFFFFu]);
    const float tot = row16_sum(w);
    if (a.renorm[side]) w = w / tot;
    if (p < k) {
      const int shift = cape_shift_of(row, a.H, a.T, a.S, a.cape_heads, a.t0);
      const int id = (int)(0xFFFFu - (my_word >> 16));
      a.idx[side][row * k + p] = (shift < 0) ? id : (id + shift) % a.S;
      a.w[side][row * k + p] = w;
    }
    if (p == 0) a.lse[side][row * 2] = lse0;
    if (p == 1) a.lse[side][row * 2 + 1] = lse1;
  }
  // a row that needs the whole-wave path is marked by index -1 in its first
  // entry; decode_fwd_u2_fix redoes it
  if (failed && p == 0) a.idx[side][row * k] = -1;
}

// The rows decode_fwd_u2x_kernel marked, by the whole-wave path, one at a
// time: a wave looks at 64 consecutive rows.
template <typename IO>
__global__ __launch_bounds__(256) void decode_fwd_u2_fix_kernel(DecodeFwdArgs a) {
  __shared__ ProdScratch scratch[4];
  __shared__ int s_idx[4][MAX_K];
  __shared__ float s_w[4][MAX_K];
  const int wv = threadIdx.x >> 6;
  const int lane = lane_id();
  const int64_t total = (int64_t)a.nsides * a.N;
  const int64_t g0 = ((int64_t)blockIdx.x * 4 + wv) * WAVE;
  const int64_t grow = g0 + lane;
  bool marked = false;
  if (grow < total) {
    const int side = grow >= a.N ? 1 : 0;
    const int64_t row = grow - (int64_t)side * a.N;
    marked = a.idx[side][row * a.k[side]] == -1;
  }
  uint64_t fm = __ballot(marked);
  while (fm) {
    const int l = (int)__builtin_ctzll(fm);
    fm &= fm - 1;
    const int64_t fg = g0 + l;
    const int side = fg >= a.N ? 1 : 0;
    const int64_t row = fg - (int64_t)side * a.N;
    const int k = a.k[side];
    const IO* src = reinterpret_cast<const IO*>(a.logits[side]) + row * (int64_t)(2 * a.P);
    decode_row_product<IO>(src, 2, a.P, k, a.renorm[side], scratch[wv], s_idx[wv], s_w[wv]);
    wave_sync();
    if (lane < k) {
      const int shift = cape_shift_of(row, a.H, a.T, a.S, a.cape_heads, a.t0);
      const int id = s_idx[wv][lane];
      a.idx[side][row * k + lane] = (shift < 0) ? id : (id + shift) % a.S;
      a.w[side][row * k + lane] = s_w[wv][lane];
    }
    if (lane < 2) a.lse[side][row * 2 + lane] = scratch[wv].dlse[lane];
    wave_sync();   // the next row rewrites the scratch
  }
}

// Decode backward of product rows (one wave per row): with gw_j as for one
// digit, dl_u[i] = sum_j gw_j [digit u of a_j = i] - p_u[i] sum_j gw_j,
// p_u = exp(l_u - lse_u) the digit softmax (paper App. B.1: the slot
// probability is the product of the digit softmaxes).  The selected-slot
// terms are added in ascending j.
template <typename IO>
__global__ __launch_bounds__(256) void decode_bwd_prod_kernel(DecodeBwdArgs a) {
  __shared__ int s_pos[4][MAX_K * MAX_DIGITS];   // element u * P + a_{j,u} of each (j, u)
  __shared__ float s_gw[4][MAX_K];
  const int wv = threadIdx.x >> 6;
  const int lane = lane_id();
  const int64_t grow = (int64_t)blockIdx.x * 4 + wv;
  if (grow >= (int64_t)a.nsides * a.N) return;
  const int side = grow >= a.N ? 1 : 0;   // nsides <= 2
  const int64_t row = grow - (int64_t)side * a.N;
  const int k = a.k[side];
  const int U = a.U, P = a.P, UP = U * P;
  const IO* __restrict__ src = reinterpret_cast<const IO*>(a.logits[side]) + row * (int64_t)UP;
  IO* __restrict__ dst = reinterpret_cast<IO*>(a.dlogits[side]) + row * (int64_t)UP;
  if (a.mask && !a.mask[token_of(row, a.H)]) {
    for (int e = lane; e < UP; e += WAVE) dst[e] = from_f32<IO>(0.f);
    return;
  }
  float gj = 0.f, wj = 0.f;
  int aj = 0;
  if (lane < k) {
    gj = a.g[side][row * k + lane];
    wj = a.w[side][row * k + lane];
    aj = a.idx[side][row * k + lane];
    const int shift = cape_shift_of(row, a.H, a.T, a.S, a.cape_heads, a.t0);
    if (shift >= 0) aj = (aj - shift + a.S) % a.S;
  }
  const float gw = decode_gw(gj, wj, a.renorm[side]);
  const float ntot = -wave_sum(gw);
  if (U == 2 && P <= WAVE) {
    // two digits: lane i holds element i of each; the selected slots' terms
    // are added in ascending j, each to the lane that holds its digit value
    const bool in = lane < P;
    const float* lse = a.lse[side] + row * 2;
    const float x0 = in ? to_f32(src[lane]) : 0.f;
    const float x1 = in ? to_f32(src[P + lane]) : 0.f;
    float acc0 = ntot * fast_exp2(fmaf(x0, LOG2E, -lse[0] * LOG2E));
    float acc1 = ntot * fast_exp2(fmaf(x1, LOG2E, -lse[1] * LOG2E));
    const int aj0 = aj / P;
    const int aj1 = aj - aj0 * P;
    for (int j = 0; j < k; ++j) {
      const float g = readlane_f(gw, j);
      if (lane == readlane_i(aj0, j)) acc0 += g;
      if (lane == readlane_i(aj1, j)) acc1 += g;
    }
    if (in) {
      dst[lane] = from_f32<IO>(acc0);
      dst[P + lane] = from_f32<IO>(acc1);
    }
    return;
  }
  if (lane < k) {
    s_gw[wv][lane] = gw;
    int rem = aj;
    for (int u = U - 1; u >= 0; --u) {
      s_pos[wv][lane * U + u] = u * P + rem % P;
      rem /= P;
    }
  }
  wave_sync();
  const float* lse = a.lse[side] + row * U;
  for (int e = lane; e < UP; e += WAVE) {
    const int u = e / P;
    const float x = to_f32(src[e]);
    float acc = ntot * fast_exp2(fmaf(x, LOG2E, -lse[u] * LOG2E));
    for (int j = 0; j < k; ++j)
      if (s_pos[wv][j * U + u] == e) acc += s_gw[wv][j];
    dst[e] = from_f32<IO>(acc);
  }
}

hipError_t launch_decode_fwd(const DecodeFwdArgs& a, bool bf16, hipStream_t st) {
  const int64_t rows = (int64_t)a.nsides * a.N;
  if (rows == 0) return hipSuccess;
  if (a.U == 2 && a.P <= WAVE && a.P % 4 == 0 && a.k[0] <= U2X_K && 4 * a.k[0] <= a.P &&
      (a.nsides < 2 || (a.k[1] <= U2X_K && 4 * a.k[1] <= a.P))) {
    const dim3 grid((unsigned)((rows + 15) / 16)), block(256);
    const dim3 fgrid((unsigned)((rows + 4 * WAVE - 1) / (4 * WAVE)));
    if (bf16) {
      hipLaunchKernelGGL(decode_fwd_u2x_kernel<bf16_t>, grid, block, 0, st, a);
      hipLaunchKernelGGL(decode_fwd_u2_fix_kernel<bf16_t>, fgrid, block, 0, st, a);
    } else {
      hipLaunchKernelGGL(decode_fwd_u2x_kernel<float>, grid, block, 0, st, a);
      hipLaunchKernelGGL(decode_fwd_u2_fix_kernel<float>, fgrid, block, 0, st, a);
    }
    return hipGetLastError();
  }
  if (a.U == 2 && a.P <= WAVE) {
    const dim3 grid((unsigned)((rows + 4 * U2_ROWS - 1) / (4 * U2_ROWS))), block(256);
    if (bf16) hipLaunchKernelGGL((decode_fwd_u2_kernel<bf16_t, U2_ROWS>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((decode_fwd_u2_kernel<float, U2_ROWS>), grid, block, 0, st, a);
    return hipGetLastError();
  }
  if (a.U > 1) {
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    if (bf16) hipLaunchKernelGGL(decode_fwd_prod_kernel<bf16_t>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(decode_fwd_prod_kernel<float>, grid, block, 0, st, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((rows + FWD_ROWS - 1) / FWD_ROWS)), block(FWD_ROWS * WAVE);
  const int nvec = a.S / (bf16 ? 8 : 4);
  if (bf16) {
    if (nvec == 512) hipLaunchKernelGGL((decode_fwd_kernel<bf16_t, 8, true>), grid, block, 0, st, a);
    else if (nvec == 2048) hipLaunchKernelGGL((decode_fwd_kernel<bf16_t, 32, true>), grid, block, 0, st, a);
    else if (nvec == 1024) hipLaunchKernelGGL((decode_fwd_kernel<bf16_t, 16, true>), grid, block, 0, st, a);
    else if (nvec <= 64) hipLaunchKernelGGL((decode_fwd_kernel<bf16_t, 1>), grid, block, 0, st, a);
    else if (nvec <= 128) hipLaunchKernelGGL((decode_fwd_kernel<bf16_t, 2>), grid, block, 0, st, a);
    else if (nvec <= 256) hipLaunchKernelGGL((decode_fwd_kernel<bf16_t, 4>), grid, block, 0, st, a);
    else if (nvec <= 512) hipLaunchKernelGGL((decode_fwd_kernel<bf16_t, 8>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((decode_fwd_kernel<bf16_t, 0>), grid, block, 0, st, a);
  } else {
    if (nvec == 512) hipLaunchKernelGGL((decode_fwd_kernel<float, 8, true>), grid, block, 0, st, a);
    else if (nvec <= 64) hipLaunchKernelGGL((decode_fwd_kernel<float, 1>), grid, block, 0, st, a);
    else if (nvec <= 128) hipLaunchKernelGGL((decode_fwd_kernel<float, 2>), grid, block, 0, st, a);
    else if (nvec <= 256) hipLaunchKernelGGL((decode_fwd_kernel<float, 4>), grid, block, 0, st, a);
    else if (nvec <= 512) hipLaunchKernelGGL((decode_fwd_kernel<float, 8>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((decode_fwd_kernel<float, 0>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_decode_bwd(const DecodeBwdArgs& a, bool bf16, hipStream_t st) {
  const int64_t rows = (int64_t)a.nsides * a.N;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (a.U == 2 && a.P <= WAVE && a.P % 4 == 0 && a.k[0] <= U2_BWD_K &&
      (a.nsides < 2 || a.k[1] <= U2_BWD_K)) {
    const dim3 grid2((unsigned)((rows + 15) / 16));
    if (bf16) hipLaunchKernelGGL(decode_bwd_u2_kernel<bf16_t>, grid2, block, 0, st, a);
    else hipLaunchKernelGGL(decode_bwd_u2_kernel<float>, grid2, block, 0, st, a);
    return hipGetLastError();
  }
  if (a.U > 1) {
    if (bf16) hipLaunchKernelGGL(decode_bwd_prod_kernel<bf16_t>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(decode_bwd_prod_kernel<float>, grid, block, 0, st, a);
    return hipGetLastError();
  }
  // One wave per 1 KiB of a row, one wave per workgroup (the fastest copy
  // layout measured on this device).
  const int nvec = a.S / (bf16 ? vec16<bf16_t>::E : vec16<float>::E);
  const int64_t waves = rows * ((nvec + WAVE - 1) / WAVE);
  if (waves > 0x7FFFFFFFll) return hipErrorInvalidValue;
  const dim3 gv((unsigned)waves), bv(WAVE);
  if (bf16) hipLaunchKernelGGL(decode_bwd_vec_kernel<bf16_t>, gv, bv, 0, st, a);
  else hipLaunchKernelGGL(decode_bwd_vec_kernel<float>, gv, bv, 0, st, a);
  return hipGetLastError();
}

}  // namespace ramk
