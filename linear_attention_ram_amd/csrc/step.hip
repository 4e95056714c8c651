// Autoregressive step of the RAM-Net attention core (ramnet-ops "CUDA
// execution", autoregressive mode; paper §4: during decoding each new token
// updates and reads its own K slots).  One workgroup of two waves per
// (b, h): wave 0 decodes the write row, wave 1 the read row (the
// register-resident decoder when the row fits, one pass over HBM); then the
// k_w selected slots are updated in place (GSU, paper §3.4), each wave taking
// every other slot with all of its row loads in flight together, and the
// updated rows are kept in LDS; last, wave 1 reads the k_r selected slots,
// taking rows written by this token from LDS so the read sees the write.
// Wave 1 requests its first read rows as soon as its own decode is done, so
// those loads overlap the write phase (a row this token writes is taken from
// LDS instead, and its early copy is dropped).
#include <type_traits>

#include "decode.hpp"
#include "decode_prod.hpp"
#include "kernels.hpp"

namespace ramk {

constexpr int STEP_ROW_CAP = 8192;  // k_w * d_v floats kept in LDS
constexpr int STEP_BATCH = 4;       // slot rows per wave with loads in flight together
constexpr int STEP_PREFETCH = 8;    // read rows requested before the write phase

// DEC: -1 product rows (U >= 2); 0 flat rows of any length, streamed;
// NV > 0 flat rows of at most NV * 64 16-byte vectors held in registers
// (FULL: exactly that many).
template <typename IO, int DEC, bool FULL>
__global__ __launch_bounds__(128) void decode_step_kernel(StepArgs a) {
  using Scratch = typename std::conditional<(DEC < 0), ProdScratch, DecodeScratch>::type;
  __shared__ Scratch scratch[2];
  __shared__ int sel_i[2][MAX_K];
  __shared__ float sel_w[2][MAX_K];
  __shared__ int hit_of[MAX_K];       // read j: index of the write of the same slot, or -1
  extern __shared__ float rows[];     // (k_w, d_v): the rows this token wrote
  const int bh = blockIdx.x;
  const int wv = threadIdx.x >> 6;
  const int lane = lane_id();
  const int d_v = a.d_v;
  if (a.mask && !a.mask[bh / a.H]) {
    // masked sequence: state untouched, output 0
    IO* o = reinterpret_cast<IO*>(a.o) + (int64_t)bh * d_v;
    for (int c = threadIdx.x; c < d_v; c += 2 * WAVE) o[c] = from_f32<IO>(0.f);
    return;
  }
  const int k = wv == 0 ? a.k_w : a.k_r;
  const int renorm = wv == 0 ? a.renorm_w : a.renorm_r;
  const IO* logits =
      reinterpret_cast<const IO*>(wv == 0 ? a.wl : a.rl) + (int64_t)bh * a.U * a.P;
  if constexpr (DEC < 0)
    decode_row_product<IO>(logits, a.U, a.P, k, renorm, scratch[wv], sel_i[wv], sel_w[wv]);
  else if constexpr (DEC == 0)
    decode_row_wave<IO>(logits, a.S, k, renorm, scratch[wv], sel_i[wv], sel_w[wv]);
  else
    decode_row_resident<IO, DEC, FULL>(logits, a.S, k, renorm, scratch[wv], sel_i[wv],
                                       sel_w[wv]);
  wave_sync();
  // CAPE heads address the content index shifted by the token's position
  // (each lane rewrites the entry it wrote)
  if ((bh % a.H) < a.cape_heads && lane < k)
    sel_i[wv][lane] = (int)((sel_i[wv][lane] + a.t0 % a.S) % a.S);
  wave_sync();
  const int c0 = lane, c1 = lane + WAVE;
  const bool ok0 = c0 < d_v, ok1 = c1 < d_v;
  float* const slot_bh = a.slot + (int64_t)bh * a.S * d_v;
  float* const mass_bh = a.mass + (int64_t)bh * a.S;
  // wave 1: the first read rows, channels c0 and c1
  float pre0[STEP_PREFETCH], pre1[STEP_PREFETCH];
  if (wv == 1) {
#pragma unroll
    for (int u = 0; u < STEP_PREFETCH; ++u) {
      const float* srow = slot_bh + (int64_t)sel_i[1][min(u, a.k_r - 1)] * d_v;
      pre0[u] = ok0 ? srow[c0] : 0.f;
      pre1[u] = ok1 ? srow[c1] : 0.f;
    }
  }
  __syncthreads();
  if (wv == 1 && lane < a.k_r) {
    const int slot = sel_i[1][lane];
    int hit = -1;
    for (int i = 0; i < a.k_w; ++i) hit = (sel_i[0][i] == slot) ? i : hit;
    hit_of[lane] = hit;
  }

  // GSU writes: wave wv updates rows j = wv, wv + 2, ...
  const IO* v = reinterpret_cast<const IO*>(a.v) + (int64_t)bh * d_v;
  const float g = to_f32(reinterpret_cast<const IO*>(a.gamma)[bh]);
  const float v0 = ok0 ? to_f32(v[c0]) : 0.f;
  const float v1 = ok1 ? to_f32(v[c1]) : 0.f;
  for (int j0 = wv; j0 < a.k_w; j0 += 2 * STEP_BATCH) {
    float m_old[STEP_BATCH], x0[STEP_BATCH], x1[STEP_BATCH];
    int slot[STEP_BATCH];
#pragma unroll
    for (int u = 0; u < STEP_BATCH; ++u) {
      const int j = min(j0 + 2 * u, a.k_w - 1);     // clamped: the load stays in bounds
      slot[u] = sel_i[0][j];
      const float* srow = slot_bh + (int64_t)slot[u] * d_v;
      m_old[u] = mass_bh[slot[u]];
      x0[u] = ok0 ? srow[c0] : 0.f;
      x1[u] = ok1 ? srow[c1] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < STEP_BATCH; ++u) {
      const int j = j0 + 2 * u;
      if (j >= a.k_w) break;
      const float w = sel_w[0][j];
      const float lam = retention(w, g, nullptr);
      const float m = lam * m_old[u] + w;
      const float eta = (w > 0.f) ? w / (m + a.eps) : 0.f;
      float* srow = slot_bh + (int64_t)slot[u] * d_v;
      if (ok0) {
        const float s = fmaf(1.f - eta, x0[u], eta * v0);
        srow[c0] = s;
        rows[j * d_v + c0] = s;
      }
      if (ok1) {
        const float s = fmaf(1.f - eta, x1[u], eta * v1);
        srow[c1] = s;
        rows[j * d_v + c1] = s;
      }
      if (lane == 0) mass_bh[slot[u]] = m;
    }
  }
  __syncthreads();

  // read-out by wave 1: o = sum_j r_j s_j in ascending j, channels c0 and c1
  if (wv == 1) {
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int u = 0; u < STEP_PREFETCH; ++u) {
      if (u < a.k_r) {
        const int hit = hit_of[u];
        const float r = sel_w[1][u];
        const float s0 = (hit >= 0 && ok0) ? rows[hit * d_v + c0] : pre0[u];
        const float s1 = (hit >= 0 && ok1) ? rows[hit * d_v + c1] : pre1[u];
        acc0 = fmaf(r, s0, acc0);
        acc1 = fmaf(r, s1, acc1);
      }
    }
    for (int j0 = STEP_PREFETCH; j0 < a.k_r; j0 += STEP_BATCH) {
      float s0[STEP_BATCH], s1[STEP_BATCH];
#pragma unroll
      for (int u = 0; u < STEP_BATCH; ++u) {
        const int j = min(j0 + u, a.k_r - 1);
        const int hit = hit_of[j];
        const float* srow = slot_bh + (int64_t)sel_i[1][j] * d_v;
        s0[u] = !ok0 ? 0.f : (hit >= 0) ? rows[hit * d_v + c0] : srow[c0];
        s1[u] = !ok1 ? 0.f : (hit >= 0) ? rows[hit * d_v + c1] : srow[c1];
      }
#pragma unroll
      for (int u = 0; u < STEP_BATCH; ++u)
        if (j0 + u < a.k_r) {
          acc0 = fmaf(sel_w[1][j0 + u], s0[u], acc0);
          acc1 = fmaf(sel_w[1][j0 + u], s1[u], acc1);
        }
    }
    IO* o = reinterpret_cast<IO*>(a.o) + (int64_t)bh * d_v;
    if (ok0) o[c0] = from_f32<IO>(acc0);
    if (ok1) o[c1] = from_f32<IO>(acc1);
  }
}

template <typename IO>
static void launch_step_io(const StepArgs& a, hipStream_t st) {
  const dim3 grid(a.B * a.H), block(128);
  const size_t lds = sizeof(float) * (size_t)a.k_w * a.d_v;
  if (a.U > 1) {
    hipLaunchKernelGGL((decode_step_kernel<IO, -1, false>), grid, block, lds, st, a);
    return;
  }
  const int nvec = a.S / vec16<IO>::E;
  if (nvec == 512) hipLaunchKernelGGL((decode_step_kernel<IO, 8, true>), grid, block, lds, st, a);
  else if (nvec <= 64) hipLaunchKernelGGL((decode_step_kernel<IO, 1, false>), grid, block, lds, st, a);
  else if (nvec <= 128) hipLaunchKernelGGL((decode_step_kernel<IO, 2, false>), grid, block, lds, st, a);
  else if (nvec <= 256) hipLaunchKernelGGL((decode_step_kernel<IO, 4, false>), grid, block, lds, st, a);
  else if (nvec <= 512) hipLaunchKernelGGL((decode_step_kernel<IO, 8, false>), grid, block, lds, st, a);
  else hipLaunchKernelGGL((decode_step_kernel<IO, 0, false>), grid, block, lds, st, a);
}

hipError_t launch_step(const StepArgs& a, bool bf16, hipStream_t st) {
  if (a.B * a.H == 0) return hipSuccess;
  if ((int64_t)a.k_w * a.d_v > STEP_ROW_CAP) return hipErrorInvalidValue;
  if (bf16) launch_step_io<bf16_t>(a, st);
  else launch_step_io<float>(a, st);
  return hipGetLastError();
}

}  // namespace ramk
