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

// Decode backward (one wave per row): with g_j the gradient of the j-th
// output weight, gw_j = g_j w_j (renormalised: gw_j = (g_j - sum_i g_i w_i) w_j),
// dl_i = [i = a_j] gw_j - p_i sum_j gw_j, p = softmax(l) = exp(l - lse).
// The row streams through in tiles of TILE 16-byte vectors per lane (all
// loads of a tile in flight before the first store).  Lane j < k gathers its
// selected logit and forms the full value of entry a_j; the lane that owns
// that entry's vector puts it into the vector before the vector is stored
// (scattered 2-byte stores after the stream cost more than the stream's
// own writes would suggest).
template <typename IO>
__global__ __launch_bounds__(256) void decode_bwd_kernel(DecodeBwdArgs a) {
  constexpr int E = vec16<IO>::E;
  constexpr int TILE = 8;
  const int lane = lane_id();
  const int64_t grow = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (grow >= (int64_t)a.nsides * a.N) return;
  const int side = grow >= a.N ? 1 : 0;   // nsides <= 2
  const int64_t row = grow - (int64_t)side * a.N;
  const int k = a.k[side];
  const IO* __restrict__ src = reinterpret_cast<const IO*>(a.logits[side]) + row * (int64_t)a.S;
  IO* __restrict__ dst = reinterpret_cast<IO*>(a.dlogits[side]) + row * (int64_t)a.S;
  if (a.mask && !a.mask[token_of(row, a.H)]) {
    // a masked token takes no part in the computation: zero gradient
    for (int c = lane; c < a.S / E; c += WAVE) st_nt16(dst + (int64_t)c * E, make_uint4(0, 0, 0, 0));
    return;
  }
  float gw = 0.f, wj = 0.f, gj = 0.f, lj = 0.f;
  int aj = 0;
  if (lane < k) {
    gj = a.g[side][row * k + lane];
    wj = a.w[side][row * k + lane];
    aj = a.idx[side][row * k + lane];
    // the logit behind a CAPE slot is the content index (slot - shift)
    const int shift = cape_shift_of(row, a.H, a.T, a.S, a.cape_heads, a.t0);
    if (shift >= 0) aj = (aj - shift + a.S) % a.S;
    lj = to_f32(src[aj]);
  }
  if (a.renorm[side]) {
    const float dot = wave_sum(gj * wj);
    gw = (gj - dot) * wj;
  } else {
    gw = gj * wj;
  }
  const float tot = wave_sum(gw);
  const float nl = -a.lse[side][row] * LOG2E;
  const float ntot = -tot;
  const float fix = gw + ntot * fast_exp2(fmaf(lj, LOG2E, nl));
  const int fix_row = (lane < k) ? aj / (E * WAVE) : -1;   // vector row of the wave holding a_j
  const int nvec = a.S / E;
  for (int c0 = 0; c0 < nvec; c0 += WAVE * TILE) {
    uint4 q[TILE];
#pragma unroll
    for (int u = 0; u < TILE; ++u) {
      const int c = c0 + u * WAVE + lane;
      if (c < nvec) q[u] = ld_nt16(src + (int64_t)c * E);
    }
    // every vector of the tile is finished before the first store: loads and
    // stores share one completion counter, so a store between two vectors
    // would make the next vector wait for it
#pragma unroll
    for (int u = 0; u < TILE; ++u) {
      float x[E];
      unpack16(q[u], x);
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = ntot * fast_exp2(fmaf(x[e], LOG2E, nl));
      // selected entries inside this vector row of the wave (usually none)
      uint64_t fixes = __ballot(fix_row == c0 / WAVE + u);
      while (fixes) {
        const int j = (int)__builtin_ctzll(fixes);
        fixes &= fixes - 1;
        const int id = readlane_i(aj, j);
        const float v = readlane_f(fix, j);
        const bool mine = lane == (id / E) % WAVE;
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = (mine && id % E == e) ? v : x[e];
      }
      q[u] = pack16(x);
    }
#pragma unroll
    for (int u = 0; u < TILE; ++u) {
      const int c = c0 + u * WAVE + lane;
      if (c < nvec) st_nt16(dst + (int64_t)c * E, q[u]);
    }
  }
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
  float gw;
  if (a.renorm[side]) {
    const float dot = wave_sum(gj * wj);
    gw = (gj - dot) * wj;
  } else {
    gw = gj * wj;
  }
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
  if (a.U > 1) {
    if (bf16) hipLaunchKernelGGL(decode_bwd_prod_kernel<bf16_t>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(decode_bwd_prod_kernel<float>, grid, block, 0, st, a);
    return hipGetLastError();
  }
  if (bf16) hipLaunchKernelGGL(decode_bwd_kernel<bf16_t>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(decode_bwd_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace ramk
