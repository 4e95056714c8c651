// Device helpers shared by the gfx950 kernels of the RAM-Net attention core.
// Wave64 throughout: one wavefront = 64 lanes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ramk {

constexpr int WAVE = 64;
constexpr float LOG2E = 1.4426950408889634f;

// bf16 is carried as its 16-bit pattern.
typedef uint16_t bf16_t;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float(((uint32_t)x) << 16); }

template <typename IO> __device__ __forceinline__ IO from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
// Round to nearest even; NaN stays NaN (quietened).
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// Number of io elements in one 16-byte vector.
template <typename IO> struct vec16 { static constexpr int E = 16 / (int)sizeof(IO); };

// Unpack a 16-byte vector of io values to float (memory order).
__device__ __forceinline__ void unpack16(const uint4 q, float (&v)[4]) {
  v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
  v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
}
__device__ __forceinline__ void unpack16(const uint4 q, float (&v)[8]) {
  v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xffff0000u);
  v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xffff0000u);
  v[4] = __uint_as_float(q.z << 16); v[5] = __uint_as_float(q.z & 0xffff0000u);
  v[6] = __uint_as_float(q.w << 16); v[7] = __uint_as_float(q.w & 0xffff0000u);
}
__device__ __forceinline__ uint4 pack16(const float (&v)[4]) {
  return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                    __float_as_uint(v[3]));
}
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  return (uint32_t)from_f32<bf16_t>(lo) | ((uint32_t)from_f32<bf16_t>(hi) << 16);
}
// Two floats to packed bf16 with the gfx950 conversion (round to nearest
// even, like from_f32; a NaN stays a NaN).
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt2bf(float lo, float hi) {
  const f32x2_hw x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_hw));
}
__device__ __forceinline__ uint4 pack16(const float (&v)[8]) {
  return make_uint4(cvt2bf(v[0], v[1]), cvt2bf(v[2], v[3]), cvt2bf(v[4], v[5]),
                    cvt2bf(v[6], v[7]));
}

// Streaming 16-byte load / store (nontemporal hint: the line is not kept in
// the caches for reuse).  Rows that are read or written exactly once go
// through these; on gfx950 they reach a markedly higher share of HBM
// bandwidth than plain accesses.
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt16(const void* p) {
  const u32x4_nt t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt*>(p));
  return make_uint4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void st_nt16(void* p, uint4 v) {
  const u32x4_nt t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x4_nt*>(p));
}

// Loads and stores through a pointer the compiler can no longer trace to a
// kernel argument (it then emits flat accesses, which also count on the LDS
// counter, so every LDS wait would wait for them too): the access is made in
// the global address space explicitly.
template <typename T>
__device__ __forceinline__ T ld_global(const T* p) {
  return *(const T __attribute__((address_space(1)))*)p;
}
template <typename T>
__device__ __forceinline__ void st_global(T* p, T v) {
  *(T __attribute__((address_space(1)))*)p = v;
}

// 16-byte vector of -inf in the io type (pads a row past its end).
template <typename IO> __device__ __forceinline__ uint4 neg_inf16();
template <> __device__ __forceinline__ uint4 neg_inf16<float>() {
  return make_uint4(0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u);
}
template <> __device__ __forceinline__ uint4 neg_inf16<bf16_t>() {
  return make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u);
}

// 2^x with the hardware instruction alone: results below 2^-126 flush to 0
// (exp2f adds a range reduction to keep them), which only drops softmax
// terms more than 87 nats below the row maximum.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (WAVE - 1)); }
__device__ __forceinline__ uint64_t lanemask_lt() {
  return (1ull << lane_id()) - 1ull;
}

// Orders LDS traffic between the lanes of one wave.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Cross-lane moves without LDS: DPP within rows of 16 lanes and the gfx950
// permlane swaps across rows.  All callers run with every lane active.
//   quad_perm [1,0,3,2] = lane ^ 1      quad_perm [2,3,0,1] = lane ^ 2
//   row_half_mirror: lane i <-> 7 - i in groups of 8
//   row_mirror:      lane i <-> 15 - i in rows of 16
//   row_ror:8 = lane ^ 8;  row_shl:k: lane i reads i + k;  row_shr:k: i - k
//   permlane16_swap(A, B): even row r gets {A_r, A_r+1}, odd row gets
//   {B_r-1, B_r};  permlane32_swap(A, B): lane l < 32 gets {A_l, A_l+32},
//   lane l >= 32 gets {B_l-32, B_l}.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
// Same move, but a lane whose source lane lies outside its row keeps `old`
// (row shifts: the lanes at the row's edge).
template <int CTRL>
__device__ __forceinline__ float dpp_or(float old, float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), CTRL,
                                                    0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
constexpr int DPP_ROR8 = 0x128, DPP_SHL1 = 0x101, DPP_SHL4 = 0x104, DPP_SHR1 = 0x111;
constexpr int DPP_SHR4 = 0x114;
template <int K> struct DppShr;
template <> struct DppShr<1> { static constexpr int v = 0x111; };
template <> struct DppShr<2> { static constexpr int v = 0x112; };
template <> struct DppShr<4> { static constexpr int v = 0x114; };
template <> struct DppShr<8> { static constexpr int v = 0x118; };
template <int K> struct DppShl;
template <> struct DppShl<1> { static constexpr int v = 0x101; };
template <> struct DppShl<2> { static constexpr int v = 0x102; };
template <> struct DppShl<4> { static constexpr int v = 0x104; };
template <> struct DppShl<8> { static constexpr int v = 0x108; };

// Sum of a and the value of the lane that differs in bit 4 (or bit 5).
__device__ __forceinline__ float xor16_pair(float a, float b) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float xor32_pair(float a, float b) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<DPP_XOR1>(x);
  x += dpp<DPP_XOR2>(x);
  x += dpp<DPP_HALF_MIRROR>(x);
  x += dpp<DPP_MIRROR>(x);
  x = xor16_pair(x, x);
  return xor32_pair(x, x);
}
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<DPP_XOR1>(x));
  x = fmaxf(x, dpp<DPP_XOR2>(x));
  x = fmaxf(x, dpp<DPP_HALF_MIRROR>(x));
  x = fmaxf(x, dpp<DPP_MIRROR>(x));
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, WAVE);
  return x;
}
// Inclusive prefix sum over the lanes of a wave, without LDS: row shifts
// by 1, 2, 4 and 8 sum inside each row of 16 lanes (a lane with no source
// in its row adds 0), then row_bcast:15 adds row 0's total to row 1 and
// row 2's to row 3, and row_bcast:31 adds the total of rows 0-1 to rows 2-3.
// Every lane must be active.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
  return x;
}

__device__ __forceinline__ float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ int readlane_i(int x, int l) { return __builtin_amdgcn_readlane(x, l); }

// Retention lambda = sigmoid(logit(1-w) - g) = (1-w)/((1-w) + w e^g) of the
// Gated Sparse Update, in the form that stays finite for large |g|: for
// g >= 0 numerator and denominator are multiplied by e^-g.  w <= 0 gives 1
// (unaddressed), w >= 1 gives 0.  Optionally d lambda / d w = -e^g / D^2.
__device__ __forceinline__ float retention(float w, float g, float* dlam_dw) {
  float c, num, den;
  if (g >= 0.f) {
    c = expf(-g);
    num = (1.f - w) * c;
    den = num + w;
  } else {
    c = expf(g);
    num = 1.f - w;
    den = num + w * c;
  }
  float lam = (w <= 0.f) ? 1.f : ((w >= 1.f) ? 0.f : num / den);
  if (dlam_dw) *dlam_dw = -c / (den * den);
  return lam;
}

}  // namespace ramk
