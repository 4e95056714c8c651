// Autoregressive step of the RAM-Net attention core (ramnet-ops "CUDA
// execution", autoregressive mode; paper §4: during decoding each new token
// updates and reads its own K slots).  One workgroup of two waves per
// (b, h): wave 0 decodes the write row, wave 1 the read row; then the k_w
// selected slots are updated in place (GSU, paper §3.4), the updated rows are
// kept in LDS, and wave 0 reads the k_r selected slots, taking rows written by
// this token from LDS so the read sees the write.
#include <type_traits>

#include "decode.hpp"
#include "decode_prod.hpp"
#include "kernels.hpp"

namespace ramk {

constexpr int STEP_ROW_CAP = 8192;  // k_w * d_v floats kept in LDS

// PROD: rows of U >= 2 address digits (product decoder)
template <typename IO, bool PROD>
__global__ __launch_bounds__(128) void decode_step_kernel(StepArgs a) {
  using Scratch = typename std::conditional<PROD, ProdScratch, DecodeScratch>::type;
  __shared__ Scratch scratch[2];
  __shared__ int sel_i[2][MAX_K];
  __shared__ float sel_w[2][MAX_K];
  __shared__ float rows[STEP_ROW_CAP];
  const int bh = blockIdx.x;
  const int wv = threadIdx.x >> 6;
  const int lane = lane_id();
  if (a.mask && !a.mask[bh / a.H]) {
    // masked sequence: state untouched, output 0
    if (wv == 0) {
      IO* o = reinterpret_cast<IO*>(a.o) + (int64_t)bh * a.d_v;
      for (int c = lane; c < a.d_v; c += WAVE) o[c] = from_f32<IO>(0.f);
    }
    return;
  }
  const IO* logits =
      reinterpret_cast<const IO*>(wv == 0 ? a.wl : a.rl) + (int64_t)bh * a.U * a.P;
  if constexpr (PROD)
    decode_row_product<IO>(logits, a.U, a.P, wv == 0 ? a.k_w : a.k_r,
                           wv == 0 ? a.renorm_w : a.renorm_r, scratch[wv], sel_i[wv], sel_w[wv]);
  else
    decode_row_wave<IO>(logits, a.S, wv == 0 ? a.k_w : a.k_r, wv == 0 ? a.renorm_w : a.renorm_r,
                        scratch[wv], sel_i[wv], sel_w[wv]);
  // CAPE heads address the content index shifted by the token's position
  // (each lane rewrites the entry it wrote)
  if ((bh % a.H) < a.cape_heads && lane < (wv == 0 ? a.k_w : a.k_r))
    sel_i[wv][lane] = (int)((sel_i[wv][lane] + a.t0 % a.S) % a.S);
  __syncthreads();

  const int d_v = a.d_v;
  const IO* v = reinterpret_cast<const IO*>(a.v) + (int64_t)bh * d_v;
  const float g = to_f32(reinterpret_cast<const IO*>(a.gamma)[bh]);
  for (int j = wv; j < a.k_w; j += 2) {
    const int slot = sel_i[0][j];
    const float w = sel_w[0][j];
    const int64_t gs = (int64_t)bh * a.S + slot;
    const float lam = retention(w, g, nullptr);
    const float m = lam * a.mass[gs] + w;
    const float eta = (w > 0.f) ? w / (m + a.eps) : 0.f;
    float* srow = a.slot + gs * d_v;
    for (int c = lane; c < d_v; c += WAVE) {
      const float s = fmaf(1.f - eta, srow[c], eta * to_f32(v[c]));
      srow[c] = s;
      rows[j * d_v + c] = s;
    }
    if (lane == 0) a.mass[gs] = m;
  }
  __syncthreads();

  if (wv == 0) {
    IO* o = reinterpret_cast<IO*>(a.o) + (int64_t)bh * d_v;
    for (int c = lane; c < d_v; c += WAVE) {
      float acc = 0.f;
      for (int j = 0; j < a.k_r; ++j) {
        const int slot = sel_i[1][j];
        int hit = -1;
        for (int i = 0; i < a.k_w; ++i) hit = (sel_i[0][i] == slot) ? i : hit;
        const float s = (hit >= 0) ? rows[hit * d_v + c]
                                   : a.slot[((int64_t)bh * a.S + slot) * d_v + c];
        acc = fmaf(sel_w[1][j], s, acc);
      }
      o[c] = from_f32<IO>(acc);
    }
  }
}

hipError_t launch_step(const StepArgs& a, bool bf16, hipStream_t st) {
  const int BH = a.B * a.H;
  if (BH == 0) return hipSuccess;
  if (a.U > 1) {
    if (bf16) hipLaunchKernelGGL((decode_step_kernel<bf16_t, true>), dim3(BH), dim3(128), 0, st, a);
    else hipLaunchKernelGGL((decode_step_kernel<float, true>), dim3(BH), dim3(128), 0, st, a);
  } else {
    if (bf16) hipLaunchKernelGGL((decode_step_kernel<bf16_t, false>), dim3(BH), dim3(128), 0, st, a);
    else hipLaunchKernelGGL((decode_step_kernel<float, false>), dim3(BH), dim3(128), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace ramk
