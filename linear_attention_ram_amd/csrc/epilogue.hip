// Read epilogue of the RAM-Net attention core (paper §3.4 "Read-out", its
// last step, and Fig. 2): y = sigmoid(g) * RMSNorm(o), the norm head-wise over
// the d_v channels of one (token, head), n = o / sqrt(mean(o^2) + eps),
// times a gain vector; the output projection stays outside.
//
// Fused into the read-out: one wave per (token, head) row sums the row's k_r
// read contributions from the stash (the same float32 sum, in the same order,
// as the plain read-out) and normalises and gates it in registers, so o never
// goes to memory.  The backward recomputes o the same way from the stash,
// which still holds the forward's contributions when the backward starts,
// and writes d_o (the input of the reverse scan) and d_gate; the gain
// gradient is summed per wave over its rows and the per-wave partial sums
// are added in a fixed order by a second kernel (deterministic).
//
// Two layouts.  Vector rows (d_v io values a multiple of 16 bytes, and a power
// of two number L of 16-byte vectors per row): each lane holds one vector,
// a wave 64 / L rows, and the norms reduce across the L lanes of a row.
// Other rows: one wave per row, lane l holds channels 2l and 2l + 1.
#include "common.hpp"
#include "kernels.hpp"

namespace ramk {

namespace {

__device__ __forceinline__ float sigmoidf(float x) { return 1.f / (1.f + expf(-x)); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Channels c, c + 1 of an io row as one access when the row width is even
// (both exist, and the pair is aligned), else element by element.
template <typename IO> struct Pair;
template <> struct Pair<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, bool even, int c, int d_v,
                                              float& a, float& b) {
    if (even) {
      const uint32_t u = c < d_v ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p + c)) : 0u;
      a = __uint_as_float(u << 16);
      b = __uint_as_float(u & 0xFFFF0000u);
    } else {
      a = c < d_v ? to_f32(p[c]) : 0.f;
      b = c + 1 < d_v ? to_f32(p[c + 1]) : 0.f;
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, bool even, int c, int d_v, float a, float b) {
    if (even) {
      if (c < d_v)
        *reinterpret_cast<uint32_t*>(p + c) =
            (uint32_t)from_f32<bf16_t>(a) | ((uint32_t)from_f32<bf16_t>(b) << 16);
    } else {
      if (c < d_v) p[c] = from_f32<bf16_t>(a);
      if (c + 1 < d_v) p[c + 1] = from_f32<bf16_t>(b);
    }
  }
};
template <> struct Pair<float> {
  static __device__ __forceinline__ void load(const float* p, bool even, int c, int d_v,
                                              float& a, float& b) {
    if (even) {
      const f32x2_t u = c < d_v ? __builtin_nontemporal_load(reinterpret_cast<const f32x2_t*>(p + c))
                                : f32x2_t{0.f, 0.f};
      a = u.x;
      b = u.y;
    } else {
      a = c < d_v ? p[c] : 0.f;
      b = c + 1 < d_v ? p[c + 1] : 0.f;
    }
  }
  static __device__ __forceinline__ void store(float* p, bool even, int c, int d_v, float a, float b) {
    if (even) {
      if (c < d_v) *reinterpret_cast<f32x2_t*>(p + c) = f32x2_t{a, b};
    } else {
      if (c < d_v) p[c] = a;
      if (c + 1 < d_v) p[c + 1] = b;
    }
  }
};

// o of one row: channels c and c + 1, the k contributions summed in j order
// (loads of RB contributions in flight together).
template <typename IO>
__device__ __forceinline__ void read_out_pair(const IO* __restrict__ st, int64_t row, int k,
                                              int d_v, bool even, int c, float& o0, float& o1) {
  constexpr int RB = 8;
  o0 = 0.f;
  o1 = 0.f;
  const IO* base = st + row * k * d_v;
  for (int j0 = 0; j0 < k; j0 += RB) {
    float x0[RB], x1[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u)
      Pair<IO>::load(base + (int64_t)min(j0 + u, k - 1) * d_v, even, c, d_v, x0[u], x1[u]);
#pragma unroll
    for (int u = 0; u < RB; ++u)
      if (j0 + u < k) {
        o0 += x0[u];
        o1 += x1[u];
      }
  }
}

template <typename IO>
__device__ __forceinline__ void load_pair(const IO* p, bool even, int c, int d_v, float& a, float& b) {
  Pair<IO>::load(p, even, c, d_v, a, b);
}

template <typename IO>
__device__ __forceinline__ void store_pair(IO* p, bool even, int c, int d_v, float a, float b) {
  Pair<IO>::store(p, even, c, d_v, a, b);
}

__device__ __forceinline__ bool row_valid(const EpilogueArgs& a, int64_t row) {
  // row = (b * T + t) * H + h; rows of one call number less than 2^31
  return !a.mask || a.mask[(uint32_t)row / (uint32_t)a.H];
}

}  // namespace

template <typename IO>
__global__ __launch_bounds__(256) void epilogue_fwd_kernel(EpilogueArgs a) {
  const int lane = lane_id();
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.N) return;
  const int d_v = a.d_v, c = 2 * lane;
  const bool even = (d_v & 1) == 0;
  const IO* st = reinterpret_cast<const IO*>(a.stash);
  float o0, o1;
  read_out_pair(st, row, a.k, d_v, even, c, o0, o1);
  const float rstd = 1.f / sqrtf(wave_sum(o0 * o0 + o1 * o1) / d_v + a.eps);
  float g0, g1;
  load_pair(reinterpret_cast<const IO*>(a.gate) + row * d_v, even, c, d_v, g0, g1);
  const float w0 = a.gain && c < d_v ? a.gain[c] : 1.f;
  const float w1 = a.gain && c + 1 < d_v ? a.gain[c + 1] : 1.f;
  store_pair(reinterpret_cast<IO*>(a.y) + row * d_v, even, c, d_v, sigmoidf(g0) * (o0 * rstd * w0),
             sigmoidf(g1) * (o1 * rstd * w1));
}

// Grid-stride over rows with a fixed number of waves; wave w leaves its gain
// gradient partial sums in part[w * d_v + c].
template <typename IO>
__global__ __launch_bounds__(256) void epilogue_bwd_kernel(EpilogueArgs a) {
  const int lane = lane_id();
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const int d_v = a.d_v, c = 2 * lane;
  const bool even = (d_v & 1) == 0;
  const IO* st = reinterpret_cast<const IO*>(a.stash);
  const float w0 = a.gain && c < d_v ? a.gain[c] : 1.f;
  const float w1 = a.gain && c + 1 < d_v ? a.gain[c + 1] : 1.f;
  float p0 = 0.f, p1 = 0.f;
  for (int64_t row = wave; row < a.N; row += nwaves) {
    IO* d_o = reinterpret_cast<IO*>(a.d_o) + row * d_v;
    IO* d_g = reinterpret_cast<IO*>(a.d_gate) + row * d_v;
    if (!row_valid(a, row)) {
      // a masked token takes no part: zero gradients
      store_pair(d_o, even, c, d_v, 0.f, 0.f);
      store_pair(d_g, even, c, d_v, 0.f, 0.f);
      continue;
    }
    float o0, o1, g0, g1, dy0, dy1;
    read_out_pair(st, row, a.k, d_v, even, c, o0, o1);
    load_pair(reinterpret_cast<const IO*>(a.gate) + row * d_v, even, c, d_v, g0, g1);
    load_pair(reinterpret_cast<const IO*>(a.d_y) + row * d_v, even, c, d_v, dy0, dy1);
    const float rstd = 1.f / sqrtf(wave_sum(o0 * o0 + o1 * o1) / d_v + a.eps);
    const float n0 = o0 * rstd, n1 = o1 * rstd;
    const float s0 = sigmoidf(g0), s1 = sigmoidf(g1);
    const float dz0 = dy0 * s0, dz1 = dy1 * s1;
    store_pair(d_g, even, c, d_v, dy0 * (n0 * w0) * s0 * (1.f - s0), dy1 * (n1 * w1) * s1 * (1.f - s1));
    p0 += dz0 * n0;
    p1 += dz1 * n1;
    const float dn0 = dz0 * w0, dn1 = dz1 * w1;
    const float dot = wave_sum(dn0 * n0 + dn1 * n1) / d_v;
    store_pair(d_o, even, c, d_v, rstd * (dn0 - n0 * dot), rstd * (dn1 - n1 * dot));
  }
  if (a.part) {
    float* part = a.part + wave * d_v;
    if (c < d_v) part[c] = p0;
    if (c + 1 < d_v) part[c + 1] = p1;
  }
}

// Sum of x over the L lanes of each row group (L a power of two <= 64).
__device__ __forceinline__ float group_sum(float x, int L) {
  for (int o = L >> 1; o > 0; o >>= 1) x += __shfl_xor(x, o, WAVE);
  return x;
}

template <typename IO>
__device__ __forceinline__ void read_out_vec(const IO* __restrict__ st, int64_t row, int k,
                                             int d_v, int vcol, float (&o)[vec16<IO>::E]) {
  constexpr int E = vec16<IO>::E, RB = 8;
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  const IO* base = st + row * k * d_v + vcol * E;
  for (int j0 = 0; j0 < k; j0 += RB) {
    uint4 q[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) q[u] = ld_nt16(base + (int64_t)min(j0 + u, k - 1) * d_v);
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      if (j0 + u >= k) break;
      float x[E];
      unpack16(q[u], x);
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] += x[e];
    }
  }
}

// Vector rows, forward: row = wave * (64 / L) + lane / L, vector lane % L.
template <typename IO>
__global__ __launch_bounds__(256) void epilogue_fwd_vec_kernel(EpilogueArgs a, int L) {
  constexpr int E = vec16<IO>::E;
  const int lane = lane_id();
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t row = wave * (WAVE / L) + lane / L;
  const int vcol = lane % L;
  const bool live = row < a.N;
  const int64_t r = live ? row : a.N - 1;    // clamped: loads stay in bounds
  const int d_v = a.d_v;
  float o[E], g[E];
  read_out_vec(reinterpret_cast<const IO*>(a.stash), r, a.k, d_v, vcol, o);
  unpack16(ld_nt16(reinterpret_cast<const IO*>(a.gate) + r * d_v + vcol * E), g);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) ss += o[e] * o[e];
  const float rstd = 1.f / sqrtf(group_sum(ss, L) / d_v + a.eps);
  float y[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float w = a.gain ? a.gain[vcol * E + e] : 1.f;
    y[e] = sigmoidf(g[e]) * (o[e] * rstd * w);
  }
  if (live) st_nt16(reinterpret_cast<IO*>(a.y) + r * d_v + vcol * E, pack16(y));
}

// Vector rows, backward: grid-stride over row groups of 64 / L rows with a
// fixed number of waves; the lanes of one vector column add their gain
// partial sums, and lanes < L of wave w leave them in part[w * d_v + c].
template <typename IO>
__global__ __launch_bounds__(256) void epilogue_bwd_vec_kernel(EpilogueArgs a, int L) {
  constexpr int E = vec16<IO>::E;
  const int lane = lane_id();
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const int rpw = WAVE / L;
  const int vcol = lane % L;
  const int d_v = a.d_v;
  float w[E], p[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    w[e] = a.gain ? a.gain[vcol * E + e] : 1.f;
    p[e] = 0.f;
  }
  for (int64_t g0 = wave * rpw; g0 < a.N; g0 += nwaves * rpw) {
    const int64_t row = g0 + lane / L;
    const bool live = row < a.N;
    const int64_t r = live ? row : a.N - 1;
    const bool valid = live && row_valid(a, r);
    float o[E], g[E], dy[E];
    read_out_vec(reinterpret_cast<const IO*>(a.stash), r, a.k, d_v, vcol, o);
    unpack16(ld_nt16(reinterpret_cast<const IO*>(a.gate) + r * d_v + vcol * E), g);
    unpack16(ld_nt16(reinterpret_cast<const IO*>(a.d_y) + r * d_v + vcol * E), dy);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) ss += o[e] * o[e];
    const float rstd = 1.f / sqrtf(group_sum(ss, L) / d_v + a.eps);
    float n[E], dn[E], dg[E], dot = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      n[e] = o[e] * rstd;
      const float s = sigmoidf(g[e]);
      const float dz = dy[e] * s;
      dg[e] = dy[e] * (n[e] * w[e]) * s * (1.f - s);
      if (valid) p[e] += dz * n[e];
      dn[e] = dz * w[e];
      dot += dn[e] * n[e];
    }
    dot = group_sum(dot, L) / d_v;
    float d_o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      d_o[e] = valid ? rstd * (dn[e] - n[e] * dot) : 0.f;
      dg[e] = valid ? dg[e] : 0.f;
    }
    if (live) {
      st_nt16(reinterpret_cast<IO*>(a.d_o) + r * d_v + vcol * E, pack16(d_o));
      st_nt16(reinterpret_cast<IO*>(a.d_gate) + r * d_v + vcol * E, pack16(dg));
    }
  }
  if (a.part) {
#pragma unroll
    for (int e = 0; e < E; ++e)
      for (int off = L; off < WAVE; off <<= 1) p[e] += __shfl_xor(p[e], off, WAVE);
    if (lane < L) {
      float* part = a.part + wave * d_v + vcol * E;
#pragma unroll
      for (int e = 0; e < E; ++e) part[e] = p[e];
    }
  }
}

// d_gain[c] = sum over the waves' partial sums, in wave order within each
// thread's share and a fixed tree across the workgroup.
__global__ __launch_bounds__(256) void gain_reduce_kernel(const float* __restrict__ part,
                                                          int nparts, int d_v, float* d_gain) {
  __shared__ float red[256];
  const int c = blockIdx.x;
  float s = 0.f;
  for (int w = threadIdx.x; w < nparts; w += 256) s += part[(int64_t)w * d_v + c];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) d_gain[c] = red[0];
}

// Lanes per row of the vector layout, or 0 when the rows do not fit it (or a
// row pointer the caller gave is not 16-byte aligned).
static int vec_lanes(const EpilogueArgs& a, bool bf16) {
  const int E = bf16 ? 8 : 4, d_v = a.d_v;
  const uintptr_t ptrs = (uintptr_t)a.gate | (uintptr_t)a.y | (uintptr_t)a.d_y |
                         (uintptr_t)a.d_gate | (uintptr_t)a.d_o | (uintptr_t)a.stash;
  if (d_v % E != 0 || (ptrs & 15u) != 0) return 0;
  const int L = d_v / E;
  return (L & (L - 1)) == 0 && L <= WAVE ? L : 0;
}

hipError_t launch_epilogue_fwd(const EpilogueArgs& a, bool bf16, hipStream_t st) {
  if (a.N == 0) return hipSuccess;
  const int L = vec_lanes(a, bf16);
  if (L > 0) {
    const int64_t rows_per_block = 4 * (WAVE / L);
    const dim3 grid((unsigned)((a.N + rows_per_block - 1) / rows_per_block)), block(256);
    if (bf16) hipLaunchKernelGGL(epilogue_fwd_vec_kernel<bf16_t>, grid, block, 0, st, a, L);
    else hipLaunchKernelGGL(epilogue_fwd_vec_kernel<float>, grid, block, 0, st, a, L);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((a.N + 3) / 4)), block(256);
  if (bf16) hipLaunchKernelGGL(epilogue_fwd_kernel<bf16_t>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(epilogue_fwd_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_epilogue_bwd(const EpilogueArgs& a, bool bf16, hipStream_t st) {
  if (a.N > 0) {
    const dim3 grid(EPI_BWD_WAVES / 4), block(256);
    const int L = vec_lanes(a, bf16);
    if (L > 0) {
      if (bf16) hipLaunchKernelGGL(epilogue_bwd_vec_kernel<bf16_t>, grid, block, 0, st, a, L);
      else hipLaunchKernelGGL(epilogue_bwd_vec_kernel<float>, grid, block, 0, st, a, L);
    } else {
      if (bf16) hipLaunchKernelGGL(epilogue_bwd_kernel<bf16_t>, grid, block, 0, st, a);
      else hipLaunchKernelGGL(epilogue_bwd_kernel<float>, grid, block, 0, st, a);
    }
  }
  if (a.d_gain)
    hipLaunchKernelGGL(gain_reduce_kernel, dim3(a.d_v), dim3(256), 0, st, a.part,
                       a.N > 0 ? EPI_BWD_WAVES : 0, a.d_v, a.d_gain);
  return hipGetLastError();
}

}  // namespace ramk
