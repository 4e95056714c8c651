// Segmented GSU scan of the RAM-Net attention core (paper §3.4 "Gated Sparse
// Update" and "Read-out"; paper §4 "Slot-Parallel Execution": slots and their
// d_v channels in parallel, each slot's events in time order, each read
// accumulated back to its token).
//
// One wavefront owns one segment (b, h, slot): lane l holds channels
// [l*CPL, l*CPL + CPL) of the slot's content in registers.  Events are taken
// in chunks of up to CHUNK = 32, aligned to multiples of 32 in the global
// event list:
//   * lane i of the wave decodes event i of the chunk and computes its
//     retention; the mass recurrence m <- lambda*m + w is an affine map, so
//     the chunk's masses come from one inclusive scan of (lambda, w) pairs
//     across lanes, then eta_i = w_i / (m_i + eps);
//   * the v rows of the chunk's writes are loaded together, then the content
//     chain s <- (1-eta)*s + eta*v runs event by event with the scalars read
//     from their lanes; a read adds r*s into the token's float accumulator.
// The state before every 32-aligned event is saved (checkpoint), so the
// reverse pass can restart any chunk without replaying the whole segment.
#include "common.hpp"
#include "kernels.hpp"

namespace ramk {

namespace {

// CPL io values of one row slice, loaded with one instruction.
template <typename IO, int CPL> struct Slice;
template <> struct Slice<bf16_t, 1> {
  uint16_t r;
  __device__ __forceinline__ void load(const bf16_t* p) { r = *p; }
  __device__ __forceinline__ void get(float (&f)[1]) const { f[0] = to_f32((bf16_t)r); }
};
template <> struct Slice<bf16_t, 2> {
  uint32_t r;
  __device__ __forceinline__ void load(const bf16_t* p) { r = *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ void get(float (&f)[2]) const {
    f[0] = __uint_as_float(r << 16);
    f[1] = __uint_as_float(r & 0xffff0000u);
  }
};
template <> struct Slice<float, 1> {
  float r;
  __device__ __forceinline__ void load(const float* p) { r = *p; }
  __device__ __forceinline__ void get(float (&f)[1]) const { f[0] = r; }
};
template <> struct Slice<float, 2> {
  float2 r;
  __device__ __forceinline__ void load(const float* p) { r = *reinterpret_cast<const float2*>(p); }
  __device__ __forceinline__ void get(float (&f)[2]) const { f[0] = r.x; f[1] = r.y; }
};

struct EventInfo {
  int row;    // token row (b*T + t)*H + h
  int side;   // 0 write, 1 read
  int j;      // rank inside the side's top-K
};

__device__ __forceinline__ EventInfo decode_event(int code, int b, int h, int T, int H) {
  EventInfo e;
  const int t = code >> 7;
  e.side = (code >> 6) & 1;
  e.j = code & 63;
  e.row = (int)(((int64_t)b * T + t) * H + h);
  return e;
}

// Inclusive scan across lanes of affine maps x -> A*x + B (earlier lanes
// applied first).  Lanes past the chunk carry the identity.
__device__ __forceinline__ void affine_scan(float& A, float& B) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < CHUNK; o <<= 1) {
    const float Ap = __shfl_up(A, o, WAVE);
    const float Bp = __shfl_up(B, o, WAVE);
    if (lane >= o) {
      B = fmaf(A, Bp, B);
      A = A * Ap;
    }
  }
}

}  // namespace

template <typename IO, int CPL>
__global__ __launch_bounds__(64) void scan_fwd_kernel(ScanFwdArgs a) {
  const int64_t g = blockIdx.x;
  const int lane = lane_id();
  const int64_t bh = g / a.S;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int c0 = lane * CPL;
  const bool active = c0 < a.d_v;
  const int beg = a.seg_offset[g], end = a.seg_offset[g + 1];
  const IO* vb = reinterpret_cast<const IO*>(a.v);
  const IO* gb = reinterpret_cast<const IO*>(a.gamma);

  float s[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) s[c] = (active && a.slot0) ? a.slot0[g * a.d_v + c0 + c] : 0.f;
  float m = a.mass0 ? a.mass0[g] : 0.f;

  for (int p0 = beg; p0 < end;) {
    const int p1 = min(end, (p0 / CHUNK + 1) * CHUNK);
    const int n = p1 - p0;
    if (p0 != beg) {
      float* ck = a.ckpt_s + (int64_t)(p0 / CHUNK) * a.d_v;
      if (active) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) ck[c0 + c] = s[c];
      }
      if (lane == 0) a.ckpt_m[p0 / CHUNK] = m;
    }
    // scalars of event lane
    EventInfo ev{0, 1, 0};
    float wt = 0.f, lam = 1.f;
    if (lane < n) {
      ev = decode_event(a.events[p0 + lane], b, h, a.T, a.H);
      if (ev.side == 0) {
        wt = a.w_w[(int64_t)ev.row * a.k_w + ev.j];
        lam = retention(wt, to_f32(gb[ev.row]), nullptr);
      } else {
        wt = a.w_r[(int64_t)ev.row * a.k_r + ev.j];
      }
    }
    float A = (ev.side == 0) ? lam : 1.f;
    float Bm = (ev.side == 0) ? wt : 0.f;
    affine_scan(A, Bm);
    const float mi = fmaf(A, m, Bm);
    const float eta = (ev.side == 0 && wt > 0.f) ? wt / (mi + a.eps) : 0.f;
    m = readlane_f(mi, n - 1);

    Slice<IO, CPL> raw[CHUNK];
#pragma unroll
    for (int i = 0; i < CHUNK; ++i) {
      raw[i].r = {};
      if (i < n && readlane_i(ev.side, i) == 0 && active)
        raw[i].load(vb + (int64_t)readlane_i(ev.row, i) * a.d_v + c0);
    }
#pragma unroll
    for (int i = 0; i < CHUNK; ++i) {
      if (i < n) {
        if (readlane_i(ev.side, i) == 0) {
          const float e = readlane_f(eta, i);
          float vv[CPL];
          raw[i].get(vv);
#pragma unroll
          for (int c = 0; c < CPL; ++c) s[c] = fmaf(1.f - e, s[c], e * vv[c]);
        } else if (active) {
          const float r = readlane_f(wt, i);
          float* dst = a.acc + (int64_t)readlane_i(ev.row, i) * a.d_v + c0;
#pragma unroll
          for (int c = 0; c < CPL; ++c) unsafeAtomicAdd(dst + c, r * s[c]);
        }
      }
    }
    p0 = p1;
  }
  if (active) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) a.slot1[g * a.d_v + c0 + c] = s[c];
  }
  if (lane == 0) a.mass1[g] = m;
}

// Reverse pass, one wave per segment, chunks in reverse order.  Each chunk
// restarts from its checkpoint (or the initial state), replays its events
// forward to recover the content before every write and to form the read
// gradients dr = <dO_t, s>, then walks the events backwards:
//   read  (weight r):  s_hat += r * dO_t
//   write (w, gamma):  dv_t += eta * s_hat;  deta = <s_hat, v_t - s_old>;
//                      s_hat <- (1 - eta) s_hat;
//                      M = m_hat - deta * w / (m' + eps)^2;
//                      dw = deta / (m' + eps) + M + M * m_old * dlambda/dw;
//                      dgamma part = M * m_old * (-lambda (1 - lambda));
//                      m_hat <- lambda * M.
template <typename IO, int CPL>
__global__ __launch_bounds__(64) void scan_bwd_kernel(ScanBwdArgs a) {
  const int64_t g = blockIdx.x;
  const int lane = lane_id();
  const int64_t bh = g / a.S;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int c0 = lane * CPL;
  const bool active = c0 < a.d_v;
  const int beg = a.seg_offset[g], end = a.seg_offset[g + 1];
  const IO* vb = reinterpret_cast<const IO*>(a.v);
  const IO* ob = reinterpret_cast<const IO*>(a.d_o);
  const IO* gb = reinterpret_cast<const IO*>(a.gamma);

  float sh[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) sh[c] = (active && a.d_slot1) ? a.d_slot1[g * a.d_v + c0 + c] : 0.f;
  float mh = a.d_mass1 ? a.d_mass1[g] : 0.f;

  if (beg < end) {
    int cs = max(beg, ((end - 1) / CHUNK) * CHUNK);
    while (true) {
      const int ce = min(end, (cs / CHUNK + 1) * CHUNK);
      const int n = ce - cs;
      float s[CPL];
      float m;
      if (cs == beg) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) s[c] = (active && a.slot0) ? a.slot0[g * a.d_v + c0 + c] : 0.f;
        m = a.mass0 ? a.mass0[g] : 0.f;
      } else {
        const float* ck = a.ckpt_s + (int64_t)(cs / CHUNK) * a.d_v;
#pragma unroll
        for (int c = 0; c < CPL; ++c) s[c] = active ? ck[c0 + c] : 0.f;
        m = a.ckpt_m[cs / CHUNK];
      }
      EventInfo ev{0, 1, 0};
      float wt = 0.f, lam = 1.f, dl = 0.f;
      if (lane < n) {
        ev = decode_event(a.events[cs + lane], b, h, a.T, a.H);
        if (ev.side == 0) {
          wt = a.w_w[(int64_t)ev.row * a.k_w + ev.j];
          lam = retention(wt, to_f32(gb[ev.row]), &dl);
        } else {
          wt = a.w_r[(int64_t)ev.row * a.k_r + ev.j];
        }
      }
      float A = (ev.side == 0) ? lam : 1.f;
      float Bm = (ev.side == 0) ? wt : 0.f;
      affine_scan(A, Bm);
      const float mi = fmaf(A, m, Bm);                     // mass after event
      float mo = __shfl_up(mi, 1, WAVE);                   // mass before event
      if (lane == 0) mo = m;
      const float eta = (ev.side == 0 && wt > 0.f) ? wt / (mi + a.eps) : 0.f;

      Slice<IO, CPL> raw[CHUNK];
#pragma unroll
      for (int i = 0; i < CHUNK; ++i) {
        raw[i].r = {};
        if (i < n && active) {
          const IO* src = (readlane_i(ev.side, i) == 0) ? vb : ob;
          raw[i].load(src + (int64_t)readlane_i(ev.row, i) * a.d_v + c0);
        }
      }
      // forward replay
      float so[CHUNK][CPL];
#pragma unroll
      for (int i = 0; i < CHUNK; ++i) {
        if (i < n) {
          float x[CPL];
          raw[i].get(x);
          if (readlane_i(ev.side, i) == 0) {
            const float e = readlane_f(eta, i);
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              so[i][c] = s[c];
              s[c] = fmaf(1.f - e, s[c], e * x[c]);
            }
          } else {
            float d = 0.f;
            if (active) {
#pragma unroll
              for (int c = 0; c < CPL; ++c) d = fmaf(x[c], s[c], d);
            }
            d = wave_sum(d);
            if (lane == 0) {
              const int ri = readlane_i(ev.row, i);
              a.dr[(int64_t)ri * a.k_r + readlane_i(ev.j, i)] = d;
            }
          }
        }
      }
      // reverse walk
#pragma unroll
      for (int i = CHUNK - 1; i >= 0; --i) {
        if (i < n) {
          float x[CPL];
          raw[i].get(x);
          const int ri = readlane_i(ev.row, i);
          if (readlane_i(ev.side, i) == 1) {
            const float r = readlane_f(wt, i);
#pragma unroll
            for (int c = 0; c < CPL; ++c) sh[c] = fmaf(r, x[c], sh[c]);
          } else {
            const float e = readlane_f(eta, i);
            float d = 0.f;
            if (active) {
              float* dst = a.acc + (int64_t)ri * a.d_v + c0;
#pragma unroll
              for (int c = 0; c < CPL; ++c) {
                unsafeAtomicAdd(dst + c, e * sh[c]);
                d = fmaf(sh[c], x[c] - so[i][c], d);
              }
            }
            d = wave_sum(d);
#pragma unroll
            for (int c = 0; c < CPL; ++c) sh[c] = (1.f - e) * sh[c];
            const float w = readlane_f(wt, i);
            const float mnew = readlane_f(mi, i);
            const float mold = readlane_f(mo, i);
            const float li = readlane_f(lam, i);
            const float dli = readlane_f(dl, i);
            const float den = mnew + a.eps;
            const float M = (w > 0.f) ? mh - d * w / (den * den) : mh;
            const float dwi = ((w > 0.f) ? d / den : 0.f) + M + M * mold * dli;
            const float dgi = M * mold * (-li * (1.f - li));
            mh = li * M;
            if (lane == 0) {
              const int64_t o = (int64_t)ri * a.k_w + readlane_i(ev.j, i);
              a.dw[o] = dwi;
              a.dgam[o] = dgi;
            }
          }
        }
      }
      if (cs == beg) break;
      cs = max(beg, cs - CHUNK);
    }
  }
  if (a.d_slot0 && active) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) a.d_slot0[g * a.d_v + c0 + c] = sh[c];
  }
  if (a.d_mass0 && lane == 0) a.d_mass0[g] = mh;
}

// acc -> io output (cleared afterwards, so the accumulator is zero between
// calls); optionally d_gamma[row] = sum_j dgam[row, j].
template <typename IO>
__global__ __launch_bounds__(256) void finalize_kernel(FinalizeArgs a) {
  IO* out = reinterpret_cast<IO*>(a.out);
  const int64_t total = a.N * a.d_v;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    out[i] = from_f32<IO>(a.acc[i]);
    a.acc[i] = 0.f;
  }
  if (a.dgam) {
    IO* dg = reinterpret_cast<IO*>(a.d_gamma);
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < a.N; r += stride) {
      float sum = 0.f;
      for (int j = 0; j < a.k_w; ++j) sum += a.dgam[r * a.k_w + j];
      dg[r] = from_f32<IO>(sum);
    }
  }
}

hipError_t launch_scan_fwd(const ScanFwdArgs& a, bool bf16, hipStream_t st) {
  const int64_t nseg = (int64_t)a.B * a.H * a.S;
  if (nseg == 0) return hipSuccess;
  const dim3 grid((unsigned)nseg), block(64);
  if (bf16) {
    if (a.d_v > 64) hipLaunchKernelGGL((scan_fwd_kernel<bf16_t, 2>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((scan_fwd_kernel<bf16_t, 1>), grid, block, 0, st, a);
  } else {
    if (a.d_v > 64) hipLaunchKernelGGL((scan_fwd_kernel<float, 2>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((scan_fwd_kernel<float, 1>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_scan_bwd(const ScanBwdArgs& a, bool bf16, hipStream_t st) {
  const int64_t nseg = (int64_t)a.B * a.H * a.S;
  if (nseg == 0) return hipSuccess;
  const dim3 grid((unsigned)nseg), block(64);
  if (bf16) {
    if (a.d_v > 64) hipLaunchKernelGGL((scan_bwd_kernel<bf16_t, 2>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((scan_bwd_kernel<bf16_t, 1>), grid, block, 0, st, a);
  } else {
    if (a.d_v > 64) hipLaunchKernelGGL((scan_bwd_kernel<float, 2>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((scan_bwd_kernel<float, 1>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeArgs& a, bool bf16, hipStream_t st) {
  const int64_t total = a.N * a.d_v;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (bf16) hipLaunchKernelGGL(finalize_kernel<bf16_t>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(finalize_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace ramk
