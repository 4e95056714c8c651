// Segmented GSU scan of the RAM-Net attention core (paper §3.4 "Gated Sparse
// Update" and "Read-out"; paper §4 "Slot-Parallel Execution": slots and their
// d_v channels in parallel, each slot's events in time order, each read
// accumulated back to its token).
//
// A segment (b, h, slot) keeps its content in registers: lane l holds channels
// [l*CPL, l*CPL + CPL).  Events are taken in chunks of up to CHUNK = 16 that
// are aligned to multiples of 16 in the global event list; the state before
// every aligned event inside a segment is saved as a checkpoint for the
// reverse pass.  Inside a chunk:
//   * lane i loads event record i (code, weight, retention); the mass recurrence
//     m <- lambda*m + w is affine, so one inclusive scan of (lambda, w) pairs
//     across lanes gives every event's mass, then eta_i = w_i / (m_i + eps);
//   * the chunk's v rows are loaded together and the content chain
//     s <- (1-eta)*s + eta*v runs event by event; a read stores its
//     contribution r*s, in the io dtype, to its own (token, j) row of a stash.
//     A token-major pass later sums the K rows of each token.  No atomics:
//     the read-out scatter is plain stores.
// Short segments (<= LONG_EVENTS events) take one wave each.  Long segments
// (hot slots) take a workgroup of NW waves that advance NW chunks at a time:
// each wave forms its chunk's mass map and, once its incoming mass is known,
// its content map s -> P*s + b (computed from s = 0); the maps are combined
// through LDS, then each wave replays its chunk from its true start state.
#include "common.hpp"
#include "kernels.hpp"

namespace ramk {

namespace {

// CPL io values of one row slice, loaded or stored with one instruction.
template <typename IO, int CPL> struct Slice;
template <> struct Slice<bf16_t, 1> {
  uint16_t r;
  __device__ __forceinline__ void load(const bf16_t* p) { r = *p; }
  __device__ __forceinline__ void get(float (&f)[1]) const { f[0] = to_f32((bf16_t)r); }
  static __device__ __forceinline__ void store(bf16_t* p, const float (&f)[1]) {
    *p = from_f32<bf16_t>(f[0]);
  }
};
template <> struct Slice<bf16_t, 2> {
  uint32_t r;
  __device__ __forceinline__ void load(const bf16_t* p) { r = *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ void get(float (&f)[2]) const {
    f[0] = __uint_as_float(r << 16);
    f[1] = __uint_as_float(r & 0xffff0000u);
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float (&f)[2]) {
    *reinterpret_cast<uint32_t*>(p) = pack2bf(f[0], f[1]);
  }
};
template <> struct Slice<float, 1> {
  float r;
  __device__ __forceinline__ void load(const float* p) { r = *p; }
  __device__ __forceinline__ void get(float (&f)[1]) const { f[0] = r; }
  static __device__ __forceinline__ void store(float* p, const float (&f)[1]) { *p = f[0]; }
};
template <> struct Slice<float, 2> {
  float2 r;
  __device__ __forceinline__ void load(const float* p) { r = *reinterpret_cast<const float2*>(p); }
  __device__ __forceinline__ void get(float (&f)[2]) const { f[0] = r.x; f[1] = r.y; }
  static __device__ __forceinline__ void store(float* p, const float (&f)[2]) {
    *reinterpret_cast<float2*>(p) = make_float2(f[0], f[1]);
  }
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

// Inclusive scan across the CHUNK = 16 lanes of each row of affine maps
// x -> A*x + B (earlier lanes applied first), with DPP row shifts.  Lanes
// past the chunk carry the identity.
template <int O>
__device__ __forceinline__ void affine_step(float& A, float& B) {
  const float Ap = dpp<DppShr<O>::v>(A);
  const float Bp = dpp<DppShr<O>::v>(B);
  const bool take = (lane_id() & (CHUNK - 1)) >= O;
  B = take ? fmaf(A, Bp, B) : B;
  A = take ? A * Ap : A;
}
__device__ __forceinline__ void affine_scan(float& A, float& B) {
  static_assert(CHUNK == 16, "scans are written for rows of 16 lanes");
  affine_step<1>(A, B);
  affine_step<2>(A, B);
  affine_step<4>(A, B);
  affine_step<8>(A, B);
}

// Per-event scalars of one chunk: lane i < n holds event cs + i.
struct ChunkScalars {
  EventInfo ev;
  float wt;   // write weight or read weight
  float lam;  // retention (writes), 1 for reads
  float dl;   // d lambda / d w (writes), 0 for reads
};

// Event record cs + lane for lanes < n (one 16-byte load; issued early so
// the next chunk's records arrive while the current chunk computes).
__device__ __forceinline__ float4 load_rec(const EventRec* events, int cs, int n) {
  return (lane_id() < n) ? *reinterpret_cast<const float4*>(events + cs + lane_id())
                         : make_float4(__int_as_float(1 << 6), 0.f, 1.f, 0.f);
}

__device__ __forceinline__ ChunkScalars chunk_scalars(float4 r, int b, int h, int T, int H) {
  ChunkScalars c;
  c.ev = decode_event(__float_as_int(r.x), b, h, T, H);
  c.wt = r.y;
  c.lam = r.z;
  c.dl = r.w;
  return c;
}

// Start of chunk k of the chunk sequence that begins at position p (p is the
// segment start or a multiple of CHUNK), clamped to end.
__device__ __forceinline__ int chunk_start(int p, int k, int end) {
  if (k == 0) return min(p, end);
  return min(end, (p / CHUNK + k) * CHUNK);
}

}  // namespace

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------

template <typename IO, int CPL>
__device__ void scan_fwd_short(const ScanFwdArgs& a, int64_t g) {
  const int lane = lane_id();
  const int64_t bh = g / a.S;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int c0 = lane * CPL;
  const bool active = c0 < a.d_v;
  const int beg = a.seg_offset[g], end = a.seg_offset[g + 1];
  const IO* vb = reinterpret_cast<const IO*>(a.v);
  IO* stash = reinterpret_cast<IO*>(a.stash);

  float s[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) s[c] = (active && a.slot0) ? a.slot0[g * a.d_v + c0 + c] : 0.f;
  float m = a.mass0 ? a.mass0[g] : 0.f;

  float4 rec = load_rec(a.events, beg, min(end, (beg / CHUNK + 1) * CHUNK) - beg);
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
    const ChunkScalars cs = chunk_scalars(rec, b, h, a.T, a.H);
    float A = (cs.ev.side == 0) ? cs.lam : 1.f;
    float Bm = (cs.ev.side == 0) ? cs.wt : 0.f;
    affine_scan(A, Bm);
    const float mi = fmaf(A, m, Bm);
    const float eta = (cs.ev.side == 0 && cs.wt > 0.f) ? cs.wt / (mi + a.eps) : 0.f;
    m = readlane_f(mi, n - 1);

    Slice<IO, CPL> raw[CHUNK];
#pragma unroll
    for (int i = 0; i < CHUNK; ++i) {
      raw[i].r = {};
      if (i < n) {
        const int si = readlane_i(cs.ev.side, i);
        const int64_t ri = readlane_i(cs.ev.row, i);
        if (si == 0 && active) raw[i].load(vb + ri * a.d_v + c0);
      }
    }
    rec = load_rec(a.events, p1, min(end, (p1 / CHUNK + 1) * CHUNK) - p1);   // next chunk
#pragma unroll
    for (int i = 0; i < CHUNK; ++i) {
      if (i < n) {
        if (readlane_i(cs.ev.side, i) == 0) {
          const float e = readlane_f(eta, i);
          float vv[CPL];
          raw[i].get(vv);
#pragma unroll
          for (int c = 0; c < CPL; ++c) s[c] = fmaf(1.f - e, s[c], e * vv[c]);
        } else {
          const float r = readlane_f(cs.wt, i);
          const int64_t slot_row = (int64_t)readlane_i(cs.ev.row, i) * a.k_r + readlane_i(cs.ev.j, i);
          float contrib[CPL];
#pragma unroll
          for (int c = 0; c < CPL; ++c) contrib[c] = r * s[c];
          if (active) Slice<IO, CPL>::store(stash + slot_row * a.d_v + c0, contrib);
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

template <typename IO, int CPL>
__device__ void scan_fwd_long(const ScanFwdArgs& a, int64_t g) {
  __shared__ float mapA[NW], mapB[NW], mapP[NW];
  __shared__ float mapb[NW][MAX_DV];
  const int lane = lane_id();
  const int w = threadIdx.x / WAVE;
  const int64_t bh = g / a.S;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int c0 = lane * CPL;
  const bool active = c0 < a.d_v;
  const int beg = a.seg_offset[g], end = a.seg_offset[g + 1];
  const IO* vb = reinterpret_cast<const IO*>(a.v);
  IO* stash = reinterpret_cast<IO*>(a.stash);

  float s_carry[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
    s_carry[c] = (active && a.slot0) ? a.slot0[g * a.d_v + c0 + c] : 0.f;
  float m_carry = a.mass0 ? a.mass0[g] : 0.f;

  float4 rec = load_rec(a.events, chunk_start(beg, w, end),
                        chunk_start(beg, w + 1, end) - chunk_start(beg, w, end));
  for (int p = beg; p < end;) {
    const int cs = chunk_start(p, w, end);
    const int n = chunk_start(p, w + 1, end) - cs;
    const int pn = chunk_start(p, NW, end);
    const ChunkScalars sc = chunk_scalars(rec, b, h, a.T, a.H);
    float A = (sc.ev.side == 0) ? sc.lam : 1.f;
    float Bm = (sc.ev.side == 0) ? sc.wt : 0.f;
    affine_scan(A, Bm);
    // cross-lane reads stay outside lane-dependent branches
    const float A_tot = readlane_f(A, max(n, 1) - 1);
    const float B_tot = readlane_f(Bm, max(n, 1) - 1);
    if (lane == 0) {
      mapA[w] = n > 0 ? A_tot : 1.f;
      mapB[w] = n > 0 ? B_tot : 0.f;
    }
    // content loads do not depend on the mass: issue them before the barrier
    Slice<IO, CPL> raw[CHUNK];
#pragma unroll
    for (int i = 0; i < CHUNK; ++i) {
      raw[i].r = {};
      if (i < n) {
        const int si = readlane_i(sc.ev.side, i);
        const int64_t ri = readlane_i(sc.ev.row, i);
        if (si == 0 && active) raw[i].load(vb + ri * a.d_v + c0);
      }
    }
    if (pn < end)   // next super-chunk's records for this wave
      rec = load_rec(a.events, chunk_start(pn, w, end),
                     chunk_start(pn, w + 1, end) - chunk_start(pn, w, end));
    __syncthreads();
    float m_in = m_carry, m_next = m_carry;
    for (int k = 0; k < NW; ++k) {
      if (k == w) m_in = m_next;
      m_next = fmaf(mapA[k], m_next, mapB[k]);
    }
    const float mi = fmaf(A, m_in, Bm);
    const float eta = (sc.ev.side == 0 && sc.wt > 0.f) ? sc.wt / (mi + a.eps) : 0.f;
    // content map of the chunk from a zero start
    float sz[CPL], P = 1.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) sz[c] = 0.f;
#pragma unroll
    for (int i = 0; i < CHUNK; ++i) {
      if (i < n && readlane_i(sc.ev.side, i) == 0) {
        const float e = readlane_f(eta, i);
        float vv[CPL];
        raw[i].get(vv);
#pragma unroll
        for (int c = 0; c < CPL; ++c) sz[c] = fmaf(1.f - e, sz[c], e * vv[c]);
        P *= 1.f - e;
      }
    }
    if (active) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) mapb[w][c0 + c] = sz[c];
    }
    if (lane == 0) mapP[w] = P;
    __syncthreads();
    float s[CPL], s_next[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) s_next[c] = s_carry[c];
    for (int k = 0; k < NW; ++k) {
      const float Pk = mapP[k];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        if (k == w) s[c] = s_next[c];
        s_next[c] = fmaf(Pk, s_next[c], active ? mapb[k][c0 + c] : 0.f);
      }
    }
    if (n > 0 && cs != beg) {
      float* ck = a.ckpt_s + (int64_t)(cs / CHUNK) * a.d_v;
      if (active) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) ck[c0 + c] = s[c];
      }
      if (lane == 0) a.ckpt_m[cs / CHUNK] = m_in;
    }
    // replay from the true start state; reads store their contributions
#pragma unroll
    for (int i = 0; i < CHUNK; ++i) {
      if (i < n) {
        if (readlane_i(sc.ev.side, i) == 0) {
          const float e = readlane_f(eta, i);
          float vv[CPL];
          raw[i].get(vv);
#pragma unroll
          for (int c = 0; c < CPL; ++c) s[c] = fmaf(1.f - e, s[c], e * vv[c]);
        } else {
          const float r = readlane_f(sc.wt, i);
          const int64_t slot_row = (int64_t)readlane_i(sc.ev.row, i) * a.k_r + readlane_i(sc.ev.j, i);
          float contrib[CPL];
#pragma unroll
          for (int c = 0; c < CPL; ++c) contrib[c] = r * s[c];
          if (active) Slice<IO, CPL>::store(stash + slot_row * a.d_v + c0, contrib);
        }
      }
    }
    m_carry = m_next;
#pragma unroll
    for (int c = 0; c < CPL; ++c) s_carry[c] = s_next[c];
    p = pn;
    __syncthreads();
  }
  if (w == 0) {
    if (active) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) a.slot1[g * a.d_v + c0 + c] = s_carry[c];
    }
    if (lane == 0) a.mass1[g] = m_carry;
  }
}

// Blocks [0, long_blocks) walk the list of long segments; every other block
// takes NW consecutive segments, one per wave, and skips the long ones.
template <typename IO, int CPL>
__global__ __launch_bounds__(NW * WAVE) void scan_fwd_kernel(ScanFwdArgs a) {
  if ((int)blockIdx.x < a.long_blocks) {
    const int count = a.use_long ? *a.long_count : 0;
    for (int i = blockIdx.x; i < count; i += a.long_blocks)
      scan_fwd_long<IO, CPL>(a, a.long_list[i]);
    return;
  }
  const int64_t g = ((int64_t)blockIdx.x - a.long_blocks) * NW + threadIdx.x / WAVE;
  if (g >= a.nseg) return;
  if (a.use_long && a.seg_offset[g + 1] - a.seg_offset[g] > LONG_EVENTS) return;
  scan_fwd_short<IO, CPL>(a, g);
}

// ---------------------------------------------------------------------------
// reverse
// ---------------------------------------------------------------------------
//
// Per chunk: restart from its checkpoint (or the initial state), replay the
// events forward to recover the content before every write, then walk the
// events backwards with the content adjoint s_hat:
//   read  (weight r):  s_hat += r * dO_t;               dr   = <dO_t, s>
//   write (w, gamma):  dv_t += eta * s_hat (io stash);  deta = <s_hat, v_t - s_old>;
//                      s_hat <- (1 - eta) s_hat
// The inner products are accumulated lane-locally for all events of the
// chunk and summed in one batched transpose-reduction.  The mass adjoint
// then follows m_hat_before = lambda * (m_hat_after - g * deta), with
// g = w / (m' + eps)^2, which is affine in m_hat: an inclusive suffix scan
// across lanes gives it for every event at once, and each lane forms
//   M = m_hat_after - g * deta
//   dw = deta / (m' + eps) + M + M * m_old * dlambda/dw
//   dgamma part = M * m_old * (-lambda (1 - lambda))
// for its own event and stores it.

template <typename IO, int CPL>
struct BwdChunk {
  ChunkScalars sc;
  float mi, mo, eta;       // mass after / before the event, step size
  Slice<IO, CPL> raw[CHUNK];
  float so[CHUNK][CPL];    // content before each write
};

// Sums x[i] over the 64 lanes for every i < CHUNK; lane i < CHUNK receives
// the total of index i.  Each halving step exchanges the half of the values a
// lane does not keep (permlane swaps across rows, DPP inside rows), so 16
// sums cost 15 cross-lane moves plus one final gather.
__device__ __forceinline__ float batched_sum(const float (&x)[CHUNK]) {
  static_assert(CHUNK == 16, "batched_sum is written for 16 values");
  const int lane = lane_id();
  float y8[8], y4[4], y2[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) y8[i] = xor32_pair(x[i], x[i + 8]);   // index i + 8*b5
#pragma unroll
  for (int i = 0; i < 4; ++i) y4[i] = xor16_pair(y8[i], y8[i + 4]); // + 4*b4
  const bool b3 = lane & 8, b2 = lane & 4;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float send = b3 ? y4[i] : y4[i + 2];
    y2[i] = (b3 ? y4[i + 2] : y4[i]) + dpp<DPP_ROR8>(send);           // + 2*b3
  }
  // row_half_mirror pairs lane i with 7 - i, whose bit 2 is the opposite one.
  // (Each cross-lane move is evaluated unconditionally: a DPP move inside one
  // arm of a ?: would run with the other lanes inactive and read zeros.)
  const float send = b2 ? y2[0] : y2[1];
  const float recv = dpp<DPP_HALF_MIRROR>(send);
  float y = (b2 ? y2[1] : y2[0]) + recv;                              // + b2
  y += dpp<DPP_XOR2>(y);
  y += dpp<DPP_XOR1>(y);
  // lane l now holds the total of index l >> 2
  return __shfl(y, (lane & (CHUNK - 1)) * 4, WAVE);
}

// Inclusive suffix scan across the 16 lanes of each row of affine maps
// x -> A*x + B, later lanes applied first (lane i ends with F_i o F_i+1 o
// ...).  Lanes past the chunk carry the identity.
template <int O>
__device__ __forceinline__ void affine_suffix_step(float& A, float& B) {
  const float An = dpp<DppShl<O>::v>(A);
  const float Bn = dpp<DppShl<O>::v>(B);
  const bool take = (lane_id() & (CHUNK - 1)) + O < CHUNK;
  B = take ? fmaf(A, Bn, B) : B;
  A = take ? A * An : A;
}
__device__ __forceinline__ void affine_suffix_scan(float& A, float& B) {
  affine_suffix_step<1>(A, B);
  affine_suffix_step<2>(A, B);
  affine_suffix_step<4>(A, B);
  affine_suffix_step<8>(A, B);
}

// Loads a chunk and replays it forward from (s, m): fills the chunk's
// scalars, rows and pre-write contents, and part[i] = <dO_i, s> (lane-local
// partial) for the reads.  s ends as the content after the chunk.
template <typename IO, int CPL>
__device__ __forceinline__ void bwd_load_replay(const ScanBwdArgs& a, BwdChunk<IO, CPL>& ck,
                                                int b, int h, float4 rec, int n, float (&s)[CPL],
                                                float m, bool active, int c0,
                                                float (&part)[CHUNK]) {
  const IO* vb = reinterpret_cast<const IO*>(a.v);
  const IO* ob = reinterpret_cast<const IO*>(a.d_o);
  ck.sc = chunk_scalars(rec, b, h, a.T, a.H);
#pragma unroll
  for (int i = 0; i < CHUNK; ++i) {
    ck.raw[i].r = {};
    if (i < n) {
      const IO* src = (readlane_i(ck.sc.ev.side, i) == 0) ? vb : ob;
      const int64_t ri = readlane_i(ck.sc.ev.row, i);
      if (active) ck.raw[i].load(src + ri * a.d_v + c0);
    }
  }
  float A = (ck.sc.ev.side == 0) ? ck.sc.lam : 1.f;
  float Bm = (ck.sc.ev.side == 0) ? ck.sc.wt : 0.f;
  affine_scan(A, Bm);
  ck.mi = fmaf(A, m, Bm);
  const float up = dpp<DPP_SHR1>(ck.mi);
  ck.mo = ((lane_id() & (CHUNK - 1)) == 0) ? m : up;
  ck.eta = (ck.sc.ev.side == 0 && ck.sc.wt > 0.f) ? ck.sc.wt / (ck.mi + a.eps) : 0.f;
#pragma unroll
  for (int i = 0; i < CHUNK; ++i) {
    part[i] = 0.f;
    if (i < n) {
      float x[CPL];
      ck.raw[i].get(x);
      if (readlane_i(ck.sc.ev.side, i) == 0) {
        const float e = readlane_f(ck.eta, i);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          ck.so[i][c] = s[c];
          s[c] = fmaf(1.f - e, s[c], e * x[c]);
        }
      } else if (active) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) part[i] = fmaf(x[c], s[c], part[i]);
      }
    }
  }
}

// Reverse walk of the content adjoint from sh (after the chunk) to sh (before
// it): stores the dv contributions and puts <s_hat_after, v - s_old> partials
// of the writes into part[i].
template <typename IO, int CPL>
__device__ __forceinline__ void bwd_walk_content(const ScanBwdArgs& a, const BwdChunk<IO, CPL>& ck,
                                                 int n, float (&sh)[CPL], bool active, int c0,
                                                 float (&part)[CHUNK]) {
  IO* stash = reinterpret_cast<IO*>(a.stash);
#pragma unroll
  for (int i = CHUNK - 1; i >= 0; --i) {
    if (i < n) {
      float x[CPL];
      ck.raw[i].get(x);
      const float r_or_w = readlane_f(ck.sc.wt, i);
      if (readlane_i(ck.sc.ev.side, i) == 1) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) sh[c] = fmaf(r_or_w, x[c], sh[c]);
      } else {
        const float e = readlane_f(ck.eta, i);
        const int64_t srow = (int64_t)readlane_i(ck.sc.ev.row, i) * a.k_w + readlane_i(ck.sc.ev.j, i);
        float contrib[CPL];
        float d = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          contrib[c] = e * sh[c];
          d = fmaf(sh[c], x[c] - ck.so[i][c], d);
          sh[c] = (1.f - e) * sh[c];
        }
        if (active) {
          Slice<IO, CPL>::store(stash + srow * a.d_v + c0, contrib);
          part[i] = d;
        }
      }
    }
  }
}

// Lane-parallel scalar part of a chunk's reverse step.  red (lane i) holds
// dr_i for a read and deta_i for a write.  Stores dr, dw and the gamma parts;
// mh goes from the mass adjoint after the chunk to the one before it.
template <typename IO, int CPL>
__device__ __forceinline__ void bwd_scalars(const ScanBwdArgs& a, const BwdChunk<IO, CPL>& ck,
                                            int n, float red, float& mh) {
  const int lane = lane_id();
  const bool ev = lane < n;
  const bool wr = ev && ck.sc.ev.side == 0;
  const float den = ck.mi + a.eps;
  const float g = (wr && ck.sc.wt > 0.f) ? ck.sc.wt / (den * den) : 0.f;
  const float deta = wr ? red : 0.f;
  float A = wr ? ck.sc.lam : 1.f;
  float B = wr ? -ck.sc.lam * g * deta : 0.f;
  affine_suffix_scan(A, B);
  const float before = fmaf(A, mh, B);
  const float after_n = dpp<DPP_SHL1>(before);
  const float after = ((lane & (CHUNK - 1)) == CHUNK - 1) ? mh : after_n;
  if (wr) {
    const float M = after - g * deta;
    const float dwi = ((ck.sc.wt > 0.f) ? deta / den : 0.f) + M + M * ck.mo * ck.sc.dl;
    const float dgi = M * ck.mo * (-ck.sc.lam * (1.f - ck.sc.lam));
    const int64_t o = (int64_t)ck.sc.ev.row * a.k_w + ck.sc.ev.j;
    a.dw[o] = dwi;
    a.dgam[o] = dgi;
  } else if (ev) {
    a.dr[(int64_t)ck.sc.ev.row * a.k_r + ck.sc.ev.j] = red;
  }
  mh = readlane_f(before, 0);
}

// State at the start of chunk cs of segment g: the initial state for the
// segment's first chunk, else the checkpoint the forward saved.
template <int CPL>
__device__ __forceinline__ void chunk_state(const ScanBwdArgs& a, int64_t g, int beg, int cs,
                                            bool active, int c0, float (&s)[CPL], float& m) {
  if (cs == beg) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) s[c] = (active && a.slot0) ? a.slot0[g * a.d_v + c0 + c] : 0.f;
    m = a.mass0 ? a.mass0[g] : 0.f;
  } else {
    const float* cp = a.ckpt_s + (int64_t)(cs / CHUNK) * a.d_v;
#pragma unroll
    for (int c = 0; c < CPL; ++c) s[c] = active ? cp[c0 + c] : 0.f;
    m = a.ckpt_m[cs / CHUNK];
  }
}

template <typename IO, int CPL>
__device__ void scan_bwd_short(const ScanBwdArgs& a, int64_t g) {
  const int lane = lane_id();
  const int64_t bh = g / a.S;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int c0 = lane * CPL;
  const bool active = c0 < a.d_v;
  const int beg = a.seg_offset[g], end = a.seg_offset[g + 1];

  float sh[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) sh[c] = (active && a.d_slot1) ? a.d_slot1[g * a.d_v + c0 + c] : 0.f;
  float mh = a.d_mass1 ? a.d_mass1[g] : 0.f;

  if (beg < end) {
    BwdChunk<IO, CPL> ck;
    float part[CHUNK];
    int cs = max(beg, ((end - 1) / CHUNK) * CHUNK);
    float4 rec = load_rec(a.events, cs, end - cs);
    while (true) {
      const int n = min(end, (cs / CHUNK + 1) * CHUNK) - cs;
      const int cp = max(beg, cs - CHUNK);
      float s[CPL], m;
      chunk_state<CPL>(a, g, beg, cs, active, c0, s, m);
      const float4 rec_cur = rec;
      if (cs != beg) rec = load_rec(a.events, cp, cs - cp);   // previous chunk
      bwd_load_replay<IO, CPL>(a, ck, b, h, rec_cur, n, s, m, active, c0, part);
      bwd_walk_content<IO, CPL>(a, ck, n, sh, active, c0, part);
      bwd_scalars<IO, CPL>(a, ck, n, batched_sum(part), mh);
      if (cs == beg) break;
      cs = cp;
    }
  }
  if (a.d_slot0 && active) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) a.d_slot0[g * a.d_v + c0 + c] = sh[c];
  }
  if (a.d_mass0 && lane == 0) a.d_mass0[g] = mh;
}

// Long segments: a workgroup of NWB waves takes NWB consecutive chunks at a
// time, from the end of the segment.  Each wave replays its chunk from its
// checkpoint and forms the chunk's adjoint map from a symbolic zero at its end
//   s_hat_in = Q * s_hat_out + q
//   m_hat_in = L * m_hat_out + <s_hat_out, U> + K
// (Q = prod (1-eta), L = prod lambda over the writes; U and K collect the
// mass terms), the maps of the later chunks are folded to give each wave its
// true adjoints after its chunk, and each wave then runs the exact reverse
// step.  Wave 0's result is the carry into the previous NW chunks.
template <typename IO, int CPL>
__device__ void scan_bwd_long(const ScanBwdArgs& a, int64_t g) {
  constexpr int NW = NWB;
  __shared__ float mQ[NW], mL[NW], mK[NW];
  __shared__ float mq[NW][MAX_DV], mU[NW][MAX_DV];
  __shared__ float carry_s[MAX_DV];
  __shared__ float carry_m;
  const int lane = lane_id();
  const int w = threadIdx.x / WAVE;
  const int64_t bh = g / a.S;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int c0 = lane * CPL;
  const bool active = c0 < a.d_v;
  const int beg = a.seg_offset[g], end = a.seg_offset[g + 1];
  const int nchunks = (end - 1) / CHUNK - beg / CHUNK + 1;

  float sh_carry[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
    sh_carry[c] = (active && a.d_slot1) ? a.d_slot1[g * a.d_v + c0 + c] : 0.f;
  float mh_carry = a.d_mass1 ? a.d_mass1[g] : 0.f;

  BwdChunk<IO, CPL> ck;
  float part[CHUNK];
  auto chunk_of = [&](int k, int& cs, int& n) {
    cs = end;
    n = 0;
    if (k < nchunks) {
      cs = chunk_start(beg, k, end);
      n = chunk_start(beg, k + 1, end) - cs;
    }
  };
  float4 rec;
  {
    int cs0, n0;
    chunk_of(((nchunks - 1) / NW) * NW + w, cs0, n0);
    rec = load_rec(a.events, cs0, n0);
  }
  for (int u0 = ((nchunks - 1) / NW) * NW; u0 >= 0; u0 -= NW) {
    int cs, n;
    chunk_of(u0 + w, cs, n);
    float s[CPL], m = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) s[c] = 0.f;
    if (n > 0) chunk_state<CPL>(a, g, beg, cs, active, c0, s, m);
    const float4 rec_cur = rec;
    if (u0 >= NW) {   // this wave's chunk of the previous super-chunk
      int csp, np;
      chunk_of(u0 - NW + w, csp, np);
      rec = load_rec(a.events, csp, np);
    }
    bwd_load_replay<IO, CPL>(a, ck, b, h, rec_cur, n, s, m, active, c0, part);
    // adjoint map of the chunk (reverse walk from zero); write partials
    // <q_after_i, u_i> join the read partials in part[]
    float Lp = (lane < n && ck.sc.ev.side == 0) ? ck.sc.lam : 1.f;
    {                                                        // prefix products of lambda
      float dummy = 0.f;
      affine_scan(Lp, dummy);
    }
    const float den = ck.mi + a.eps;
    const float gq = (ck.sc.ev.side == 0 && ck.sc.wt > 0.f) ? ck.sc.wt / (den * den) : 0.f;
    float Q = 1.f, q[CPL], U[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) { q[c] = 0.f; U[c] = 0.f; }
#pragma unroll
    for (int i = CHUNK - 1; i >= 0; --i) {
      if (i < n) {
        float x[CPL];
        ck.raw[i].get(x);
        const float r_or_w = readlane_f(ck.sc.wt, i);
        if (readlane_i(ck.sc.ev.side, i) == 1) {
#pragma unroll
          for (int c = 0; c < CPL; ++c) q[c] = fmaf(r_or_w, x[c], q[c]);
        } else {
          const float e = readlane_f(ck.eta, i);
          const float coef = -readlane_f(Lp, i) * readlane_f(gq, i) * Q;
          float d = 0.f;
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const float u = active ? x[c] - ck.so[i][c] : 0.f;
            d = fmaf(q[c], u, d);
            U[c] = fmaf(coef, u, U[c]);
            q[c] = (1.f - e) * q[c];
          }
          part[i] = active ? d : 0.f;
          Q *= 1.f - e;
        }
      }
    }
    const float red1 = batched_sum(part);     // dr (reads), <q_after, u> (writes)
    const bool wr = lane < n && ck.sc.ev.side == 0;
    const float K = wave_sum(wr ? -Lp * gq * red1 : 0.f);
    const float L = readlane_f(Lp, max(n, 1) - 1);
    if (active) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) { mq[w][c0 + c] = q[c]; mU[w][c0 + c] = U[c]; }
    }
    if (lane == 0) { mQ[w] = Q; mL[w] = (n > 0) ? L : 1.f; mK[w] = K; }
    __syncthreads();
    // adjoints after this wave's chunk: fold the maps of the later chunks
    float sh[CPL];
    float mh = mh_carry;
#pragma unroll
    for (int c = 0; c < CPL; ++c) sh[c] = sh_carry[c];
    for (int kk = NW - 1; kk > w; --kk) {
      float d = 0.f;
      if (active) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) d = fmaf(sh[c], mU[kk][c0 + c], d);
      }
      d = wave_sum(d);
      mh = fmaf(mL[kk], mh, d + mK[kk]);
      const float Qk = mQ[kk];
#pragma unroll
      for (int c = 0; c < CPL; ++c) sh[c] = fmaf(Qk, sh[c], active ? mq[kk][c0 + c] : 0.f);
    }
    // exact reverse step of this wave's chunk
#pragma unroll
    for (int i = 0; i < CHUNK; ++i) part[i] = 0.f;
    bwd_walk_content<IO, CPL>(a, ck, n, sh, active, c0, part);
    const float red2 = batched_sum(part);     // deta (writes)
    {
      // bwd_scalars stores dr for reads too; keep the values from red1 there
      const bool rd = lane < n && ck.sc.ev.side == 1;
      bwd_scalars<IO, CPL>(a, ck, n, rd ? red1 : red2, mh);
    }
    if (w == 0) {
      if (active) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) carry_s[c0 + c] = sh[c];
      }
      if (lane == 0) carry_m = mh;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < CPL; ++c) sh_carry[c] = active ? carry_s[c0 + c] : 0.f;
    mh_carry = carry_m;
    __syncthreads();
  }
  if (w == 0) {
    if (a.d_slot0 && active) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) a.d_slot0[g * a.d_v + c0 + c] = sh_carry[c];
    }
    if (a.d_mass0 && lane == 0) a.d_mass0[g] = mh_carry;
  }
}

// Long segments: NWB waves per workgroup, the workgroups walk the long list.
template <typename IO, int CPL>
__global__ __launch_bounds__(NWB * WAVE) void scan_bwd_long_kernel(ScanBwdArgs a) {
  const int count = a.use_long ? *a.long_count : 0;
  for (int i = blockIdx.x; i < count; i += gridDim.x) scan_bwd_long<IO, CPL>(a, a.long_list[i]);
}

// Short segments: one wave each, four per workgroup.
template <typename IO, int CPL>
__global__ __launch_bounds__(4 * WAVE) void scan_bwd_short_kernel(ScanBwdArgs a) {
  const int64_t g = (int64_t)blockIdx.x * 4 + threadIdx.x / WAVE;
  if (g >= a.nseg) return;
  if (a.use_long && a.seg_offset[g + 1] - a.seg_offset[g] > LONG_EVENTS) return;
  scan_bwd_short<IO, CPL>(a, g);
}

// ---------------------------------------------------------------------------
// token-major sums of the stash rows
// ---------------------------------------------------------------------------

// out[row] = sum_j stash[row, j] (float accumulation, j ascending).  With
// d_v a multiple of one 16-byte vector, a thread sums one vector column.
template <typename IO>
__global__ __launch_bounds__(256) void finalize_kernel(FinalizeArgs a) {
  constexpr int E = vec16<IO>::E;
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const IO* st = reinterpret_cast<const IO*>(a.stash);
  IO* out = reinterpret_cast<IO*>(a.out);
  if (a.d_v % E == 0) {
    const int vpr = a.d_v / E;
    if (tid < a.N * vpr) {
      const int64_t row = tid / vpr;
      const int vcol = (int)(tid % vpr);
      float acc[E];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = 0.f;
      const IO* base = st + row * a.k * a.d_v + vcol * E;
      for (int j = 0; j < a.k; ++j) {
        float x[E];
        unpack16(*reinterpret_cast<const uint4*>(base + (int64_t)j * a.d_v), x);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += x[e];
      }
      *reinterpret_cast<uint4*>(out + row * a.d_v + vcol * E) = pack16(acc);
    }
  } else if (tid < a.N * a.d_v) {
    const int64_t row = tid / a.d_v;
    const int c = (int)(tid % a.d_v);
    float acc = 0.f;
    for (int j = 0; j < a.k; ++j) acc += to_f32(st[(row * a.k + j) * a.d_v + c]);
    out[row * a.d_v + c] = from_f32<IO>(acc);
  }
  if (a.dgam && tid < a.N) {
    float sum = 0.f;
    for (int j = 0; j < a.k; ++j) sum += a.dgam[tid * a.k + j];
    reinterpret_cast<IO*>(a.d_gamma)[tid] = from_f32<IO>(sum);
  }
}

// ---------------------------------------------------------------------------

hipError_t launch_scan_fwd(const ScanFwdArgs& a, bool bf16, hipStream_t st) {
  if (a.nseg == 0) return hipSuccess;
  const dim3 grid((unsigned)(a.long_blocks + (a.nseg + NW - 1) / NW)), block(NW * WAVE);
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
  if (a.nseg == 0) return hipSuccess;
  const dim3 lgrid((unsigned)a.long_blocks), lblock(NWB * WAVE);
  const dim3 sgrid((unsigned)((a.nseg + 3) / 4)), sblock(4 * WAVE);
  if (a.use_long) {
    if (bf16) {
      if (a.d_v > 64) hipLaunchKernelGGL((scan_bwd_long_kernel<bf16_t, 2>), lgrid, lblock, 0, st, a);
      else hipLaunchKernelGGL((scan_bwd_long_kernel<bf16_t, 1>), lgrid, lblock, 0, st, a);
    } else {
      if (a.d_v > 64) hipLaunchKernelGGL((scan_bwd_long_kernel<float, 2>), lgrid, lblock, 0, st, a);
      else hipLaunchKernelGGL((scan_bwd_long_kernel<float, 1>), lgrid, lblock, 0, st, a);
    }
  }
  if (bf16) {
    if (a.d_v > 64) hipLaunchKernelGGL((scan_bwd_short_kernel<bf16_t, 2>), sgrid, sblock, 0, st, a);
    else hipLaunchKernelGGL((scan_bwd_short_kernel<bf16_t, 1>), sgrid, sblock, 0, st, a);
  } else {
    if (a.d_v > 64) hipLaunchKernelGGL((scan_bwd_short_kernel<float, 2>), sgrid, sblock, 0, st, a);
    else hipLaunchKernelGGL((scan_bwd_short_kernel<float, 1>), sgrid, sblock, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeArgs& a, bool bf16, hipStream_t st) {
  if (a.N == 0) return hipSuccess;
  const int E = bf16 ? 8 : 4;
  int64_t threads = (a.d_v % E == 0) ? a.N * (a.d_v / E) : a.N * a.d_v;
  if (threads < a.N) threads = a.N;
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (bf16) hipLaunchKernelGGL(finalize_kernel<bf16_t>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(finalize_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace ramk
