// HBM streaming ceilings of gfx950, measured with the access patterns of the
// decoders: a wave owns one contiguous row of ROW_VECS * 64 16-byte vectors
// (lane l holds vectors l, l + 64, ...), a workgroup holds WAVES
// consecutive rows, and all of a wave's loads are in flight before its first
// store.  Read mode folds the loaded words into one value per lane (stored
// only if it matches a value no input produces, so the loads stay live);
// copy mode stores the row back to the destination.  These are the two
// roofs of the decoders: decode_fwd reads its rows once, decode_bwd reads a
// row and writes a row of the same size.
#include "../../include/ramnet.h"
#include "common.hpp"

namespace ramk {

namespace {

template <int ROW_VECS, int WAVES, bool NT, bool COPY>
__global__ __launch_bounds__(WAVES * WAVE) void stream_kernel(const uint4* __restrict__ src,
                                                              uint4* __restrict__ dst) {
  const int lane = lane_id();
  const int64_t row = (int64_t)blockIdx.x * WAVES + (threadIdx.x >> 6);
  const uint4* s = src + row * ROW_VECS * WAVE;
  uint4 q[ROW_VECS];
#pragma unroll
  for (int u = 0; u < ROW_VECS; ++u) q[u] = NT ? ld_nt16(s + u * WAVE + lane) : s[u * WAVE + lane];
  if constexpr (COPY) {
    uint4* d = dst + row * ROW_VECS * WAVE;
#pragma unroll
    for (int u = 0; u < ROW_VECS; ++u) {
      if constexpr (NT) st_nt16(d + u * WAVE + lane, q[u]);
      else d[u * WAVE + lane] = q[u];
    }
  } else {
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < ROW_VECS; ++u) acc ^= q[u].x ^ q[u].y ^ q[u].z ^ q[u].w;
    if (acc == 0x9E3779B9u) dst[row * WAVE + lane] = q[0];
  }
}

struct Variant {
  int row_vecs, waves;
  bool nt;
};
// 0: the forward decoder's pattern (8 KiB rows, 4 waves, nontemporal); 1: the
// same with plain loads and stores; 2: 16 KiB rows; 3: 4 KiB rows; 4: 8 waves;
// 5: 1 KiB rows, one wave per workgroup (the decode backward's pattern);
// 6: 2 KiB rows, one wave per workgroup
constexpr Variant VARIANTS[] = {{8, 4, true}, {8, 4, false}, {16, 4, true}, {4, 4, true},
                                {8, 8, true}, {1, 1, true},  {2, 1, true}};
constexpr int NVARIANTS = (int)(sizeof(VARIANTS) / sizeof(VARIANTS[0]));

template <int RV, int W, bool NT>
hipError_t launch_v(bool copy, const void* src, void* dst, size_t bytes, hipStream_t st) {
  const size_t tile = (size_t)RV * WAVE * 16 * W;
  const dim3 grid((unsigned)(bytes / tile)), block(W * WAVE);
  if (copy)
    hipLaunchKernelGGL((stream_kernel<RV, W, NT, true>), grid, block, 0, st, (const uint4*)src,
                       (uint4*)dst);
  else
    hipLaunchKernelGGL((stream_kernel<RV, W, NT, false>), grid, block, 0, st, (const uint4*)src,
                       (uint4*)dst);
  return hipGetLastError();
}

}  // namespace

}  // namespace ramk

extern "C" int ram_stream_probe(int mode, int variant, const void* src, void* dst, size_t bytes,
                                void* stream) {
  using namespace ramk;
  if (mode != 0 && mode != 1) return RAM_EINVAL;
  if (variant < 0 || variant >= NVARIANTS) return RAM_EINVAL;
  const Variant v = VARIANTS[variant];
  const size_t tile = (size_t)v.row_vecs * WAVE * 16 * v.waves;
  if (!src || !dst || bytes == 0 || bytes % tile != 0 || bytes / tile > 0x7FFFFFFFu)
    return RAM_EINVAL;
  if (((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return RAM_EINVAL;
  const bool copy = mode == 1;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  switch (variant) {
    case 0: e = launch_v<8, 4, true>(copy, src, dst, bytes, st); break;
    case 1: e = launch_v<8, 4, false>(copy, src, dst, bytes, st); break;
    case 2: e = launch_v<16, 4, true>(copy, src, dst, bytes, st); break;
    case 3: e = launch_v<4, 4, true>(copy, src, dst, bytes, st); break;
    case 4: e = launch_v<8, 8, true>(copy, src, dst, bytes, st); break;
    case 5: e = launch_v<1, 1, true>(copy, src, dst, bytes, st); break;
    default: e = launch_v<2, 1, true>(copy, src, dst, bytes, st); break;
  }
  return e == hipSuccess ? RAM_OK : RAM_EHIP;
}
