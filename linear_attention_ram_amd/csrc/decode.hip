// Address decoding of the RAM-Net attention core (paper §3.1-3.2, one digit:
// U = 1): per (token, head, side) row of S logits, lse = logsumexp, the K
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

namespace ramk {

// One wave per row; rows of side 0 first, then side 1.
template <typename IO>
__global__ __launch_bounds__(256) void decode_fwd_kernel(DecodeFwdArgs a) {
  __shared__ DecodeScratch scratch[4];
  __shared__ int s_idx[4][MAX_K];
  __shared__ float s_w[4][MAX_K];
  const int wv = threadIdx.x >> 6;
  const int lane = lane_id();
  const int64_t grow = (int64_t)blockIdx.x * 4 + wv;
  if (grow >= (int64_t)a.nsides * a.N) return;
  const int side = (int)(grow / a.N);
  const int64_t row = grow - (int64_t)side * a.N;
  const IO* src = reinterpret_cast<const IO*>(a.logits[side]) + row * (int64_t)a.S;
  const int k = a.k[side];
  const float lse = decode_row_wave<IO>(src, a.S, k, a.renorm[side], scratch[wv], s_idx[wv], s_w[wv]);
  wave_sync();
  if (lane < k) {
    a.idx[side][row * k + lane] = s_idx[wv][lane];
    a.w[side][row * k + lane] = s_w[wv][lane];
  }
  if (lane == 0) a.lse[side][row] = lse;
  if (a.zero_rows && side == a.nsides - 1) {
    float* z = a.zero_rows + row * (int64_t)a.zero_width;
    for (int c = lane; c < a.zero_width; c += WAVE) z[c] = 0.f;
  }
}

// Decode backward (one wave per row): with g_j the gradient of the j-th
// output weight, gw_j = g_j w_j (renormalised: gw_j = (g_j - sum_i g_i w_i) w_j),
// dl_i = [i = a_j] gw_j - p_i sum_j gw_j, p = softmax(l) = exp(l - lse).
template <typename IO>
__global__ __launch_bounds__(256) void decode_bwd_kernel(DecodeBwdArgs a) {
  constexpr int E = vec16<IO>::E;
  const int wv = threadIdx.x >> 6;
  const int lane = lane_id();
  const int64_t grow = (int64_t)blockIdx.x * 4 + wv;
  if (grow >= (int64_t)a.nsides * a.N) return;
  (void)wv;
  const int side = (int)(grow / a.N);
  const int64_t row = grow - (int64_t)side * a.N;
  const int k = a.k[side];
  const IO* src = reinterpret_cast<const IO*>(a.logits[side]) + row * (int64_t)a.S;
  IO* dst = reinterpret_cast<IO*>(a.dlogits[side]) + row * (int64_t)a.S;
  float gw = 0.f, wj = 0.f, gj = 0.f;
  int aj = 0;
  if (lane < k) {
    gj = a.g[side][row * k + lane];
    wj = a.w[side][row * k + lane];
    aj = a.idx[side][row * k + lane];
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
  const int nvec = a.S / E;
  for (int c = lane; c < nvec; c += WAVE) {
    float x[E];
    unpack16(*reinterpret_cast<const uint4*>(src + (int64_t)c * E), x);
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = ntot * exp2f(fmaf(x[e], LOG2E, nl));
    *reinterpret_cast<uint4*>(dst + (int64_t)c * E) = pack16(x);
  }
  // the selected entries get their extra term; each is rewritten by the lane
  // that wrote its vector above, so program order keeps the later store
  for (int j = 0; j < k; ++j) {
    const int id = readlane_i(aj, j);
    const float g = readlane_f(gw, j);
    if (lane == (id / E) % WAVE) {
      const float p = exp2f(fmaf(to_f32(src[id]), LOG2E, nl));
      dst[id] = from_f32<IO>(g + ntot * p);
    }
  }
}

hipError_t launch_decode_fwd(const DecodeFwdArgs& a, bool bf16, hipStream_t st) {
  const int64_t rows = (int64_t)a.nsides * a.N;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (bf16) hipLaunchKernelGGL(decode_fwd_kernel<bf16_t>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(decode_fwd_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode_bwd(const DecodeBwdArgs& a, bool bf16, hipStream_t st) {
  const int64_t rows = (int64_t)a.nsides * a.N;
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
  if (bf16) hipLaunchKernelGGL(decode_bwd_kernel<bf16_t>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(decode_bwd_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace ramk
