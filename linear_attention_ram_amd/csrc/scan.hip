// Segmented GSU scan of the RAM-Net attention core (paper §3.4 "Gated Sparse
// Update" and "Read-out"; paper §4 "Slot-Parallel Execution": slots and their
// d_v channels in parallel, each slot's events in time order, each read
// accumulated back to its token).
//
// A segment (b, h, slot) keeps its content in registers: lane l holds channels
// [l*CPL, l*CPL + CPL).  Events are taken in chunks of CHUNK = 16 from the
// segment's start (the last chunk may be shorter); the state before every
// chunk but the first is saved as a checkpoint for the reverse pass, at index
// (chunk start) / 16 of the checkpoint array: chunk starts of one segment are
// 16 apart and those of later segments lie more than 16 beyond, so no two
// share an index.
//
// Lane layout of a chunk.  Lane l also holds the scalars of event (l & 15):
// the four 16-lane rows of the wave carry identical copies, so the DPP
// row_newbcast:i move hands every lane the scalars of event i without a trip
// through a scalar register, and every per-row DPP scan or reduction sees all
// 16 events.  Lanes past the chunk's end hold a read of weight 0.
//
// Event loops.  The row loads and stores go through buffer resources whose
// range check turns an offset of OOB into a load of zero or a dropped store,
// so a chunk's row loads are issued for all 16 events at once without
// branches (the load of an event that has no such row reads nothing).  The
// arithmetic of event i then runs under a branch on its kind, which is the
// same in every lane (all lanes work on the same event), so each event does
// only its own kind's work and padding does none.
//
// Inside a chunk:
//   * the mass recurrence m <- lambda*m + w is affine, so one inclusive scan
//     of (lambda, w) pairs across each row gives every event's mass, then
//     eta_i = w_i / (m_i + eps);
//   * the content chain s <- (1-eta)*s + eta*v runs event by event (eta = 1
//     replaces the content exactly); a read
//     stores its contribution r*s, in the io dtype, to its own (token, j) row
//     of a stash.  A token-major pass later sums the K rows of each token.
//     No atomics: the read-out scatter is plain stores.
// Short segments (1 to LONG_EVENTS events) take one wave each, found through
// the bucketing's list of them where most segments have no events (a hot
// slot layout leaves most slots untouched).  Long segments
// (hot slots) take a workgroup of NWL waves that advance NWL chunks at a
// time: each wave forms its chunk's mass map and, once its incoming mass is
// known, its content map s -> P*s + b (computed from s = 0); the maps are
// combined through LDS, then each wave replays its chunk from its true start
// state.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace ramk {

namespace {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
// Byte offsets that fall outside every buffer (load 0, drop the store).  An
// access offset is event offset + lane offset; buffers hold at most
// MAX_BUF_BYTES (checked on the host), and the two sentinels are chosen so
// that no sum wraps around 2^32:
//   OOB (event): + a lane offset < 2^20 stays in [OOB, 2^31)
//   OOB_LANE:    + an event offset < 2^31 stays in [2^31, 2^32)
constexpr uint32_t OOB = 0x7FF00000u;
constexpr uint32_t OOB_LANE = 0x80000000u;
static_assert(OOB >= MAX_BUF_BYTES, "event sentinel inside a buffer");
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Raw buffer of `bytes` bytes (<= MAX_BUF_BYTES) at base.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Waits until every vector memory access the wave has issued is complete
// (s_waitcnt vmcnt(0); the other counters are left alone).  Loads and stores
// share that counter, so once a chunk's row loads are known to be done, the
// stores of its event loop are never waited on inside it.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Kernel arguments are read with wide scalar loads, and the registers of one
// load stay allocated together while any of its fields is in use.  fresh()
// turns a field into a value of its own (an empty asm the compiler cannot see
// through), so a long loop that needs a few fields keeps only those, and the
// rest are freed instead of spilled.
template <typename T>
__device__ __forceinline__ void fresh(T& x) { asm volatile("" : "+s"(x)); }

// Index of the wave in its workgroup, as a value the compiler knows to be
// uniform (buffer resources built from it stay in scalar registers).
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / WAVE));
}

// Value of event I of the lane's row (DPP row_newbcast:I).
template <int I>
__device__ __forceinline__ float bc(float x) { return dpp<0x150 + I>(x); }
template <int I>
__device__ __forceinline__ uint32_t bcu(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x150 + I, 0xF, 0xF, true);
}

// Compile-time loops over the events of a chunk.
template <int I, int N, typename F>
__device__ __forceinline__ void for_up(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>());
    for_up<I + 1, N>(f);
  }
}
template <int I, typename F>
__device__ __forceinline__ void for_down(F&& f) {   // I-1, I-2, ..., 0
  if constexpr (I > 0) {
    f(std::integral_constant<int, I - 1>());
    for_down<I - 1>(f);
  }
}

// Scheduling fence every SCHED_EVENTS events of a chunk loop: keeps the
// compiler from hoisting the loads and broadcasts of all 16 events at once,
// which would cost more registers than the latency it hides.
constexpr int SCHED_EVENTS = 4;
template <int I>
__device__ __forceinline__ void sched_fence() {
  if constexpr (I % SCHED_EVENTS == SCHED_EVENTS - 1) __builtin_amdgcn_sched_barrier(0);
}

// CPL io values of one row slice at a byte offset of a buffer.
template <typename IO, int CPL> struct Lanes;
template <> struct Lanes<bf16_t, 1> {
  typedef uint32_t Raw;
  static __device__ __forceinline__ Raw load(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  }
  static __device__ __forceinline__ void get(Raw x, float (&f)[1]) { f[0] = __uint_as_float(x << 16); }
  static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, const float (&f)[1]) {
    const f32x2_t x = {f[0], 0.f};
    const uint32_t u = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)u, r, off, 0, 0);
  }
};
template <> struct Lanes<bf16_t, 2> {
  typedef uint32_t Raw;
  static __device__ __forceinline__ Raw load(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
  static __device__ __forceinline__ void get(Raw x, float (&f)[2]) {
    f[0] = __uint_as_float(x << 16);
    f[1] = __uint_as_float(x & 0xffff0000u);
  }
  static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, const float (&f)[2]) {
    const f32x2_t x = {f[0], f[1]};
    __builtin_amdgcn_raw_buffer_store_b32(
        __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t)), r, off, 0, 0);
  }
};
template <> struct Lanes<float, 1> {
  typedef uint32_t Raw;
  static __device__ __forceinline__ Raw load(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
  static __device__ __forceinline__ void get(Raw x, float (&f)[1]) { f[0] = __uint_as_float(x); }
  static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, const float (&f)[1]) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(f[0]), r, off, 0, 0);
  }
};
template <> struct Lanes<float, 2> {
  typedef uint2 Raw;
  static __device__ __forceinline__ Raw load(rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return make_uint2(v[0], v[1]);
  }
  static __device__ __forceinline__ void get(Raw x, float (&f)[2]) {
    f[0] = __uint_as_float(x.x);
    f[1] = __uint_as_float(x.y);
  }
  static __device__ __forceinline__ void store(rsrc_t r, uint32_t off, const float (&f)[2]) {
    typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t v = {__float_as_uint(f[0]), __float_as_uint(f[1])};
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
  }
};

// Where a segment's lanes read and write: buffers of its batch b, the lane's
// byte offset inside a row (OOB for lanes past d_v) and the row pitch.
template <typename IO, int CPL>
struct SegCtx {
  int b, h;
  int c0;             // first channel of the lane
  bool active;        // c0 < d_v
  uint32_t lb;        // c0 * sizeof(IO), or OOB_LANE
  uint32_t pitch;     // d_v * sizeof(IO)
  int64_t row0;       // first token row of batch b: b * T * H
};

template <typename IO, int CPL>
__device__ __forceinline__ SegCtx<IO, CPL> seg_ctx(int64_t g, int S, int H, int T, int d_v) {
  SegCtx<IO, CPL> c;
  const int64_t bh = g / S;
  c.b = (int)(bh / H);
  c.h = (int)(bh % H);
  c.c0 = lane_id() * CPL;
  c.active = c.c0 < d_v;
  c.lb = c.active ? (uint32_t)(c.c0 * sizeof(IO)) : OOB_LANE;
  c.pitch = (uint32_t)(d_v * sizeof(IO));
  c.row0 = (int64_t)c.b * T * H;
  return c;
}

// Scalars of event (lane & 15) of a chunk.
struct Ev {
  bool valid;   // the chunk has this event
  bool live;    // not the no-op event of a masked token (its rows are never loaded)
  int side;     // 0 write, 1 read (padding: read of weight 0)
  int rb;       // token row inside the batch: t*H + h
  int j;        // rank inside the side's top-K
  float wt;     // write weight or read weight
  float lam;    // retention (writes), 1 for reads
  float dl;     // d lambda / d w (writes), 0 for reads
};

// Raw record of event cs + (lane & 15), clamped into the segment's non-empty
// range [beg, end).  The load is unconditional and its value is only
// inspected when the chunk is decoded (lanes past the chunk then become a
// read of weight 0), so an early load of the next chunk's records stays in
// flight while the current chunk computes.
__device__ __forceinline__ float4 load_rec(const EventRec* events, int cs, int n, int beg, int end) {
  (void)n;
  const int at = min(max(cs + (lane_id() & (CHUNK - 1)), beg), end - 1);
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const f32x4 r = ld_global(reinterpret_cast<const f32x4*>(events + at));
  return make_float4(r[0], r[1], r[2], r[3]);
}

__device__ __forceinline__ Ev decode_rec(float4 raw, int n, int h, int H) {
  Ev e;
  e.valid = (lane_id() & (CHUNK - 1)) < n;
  const float4 r = e.valid ? raw : make_float4(__int_as_float(1 << 6), 0.f, 1.f, 0.f);
  const int code = __float_as_int(r.x);
  e.live = code >= 0;
  e.side = (code >> 6) & 1;
  e.j = code & 63;
  e.rb = ((code & 0x7FFFFFFF) >> 7) * H + h;
  e.wt = r.y;
  e.lam = r.z;
  e.dl = r.w;
  return e;
}

// Inclusive scan across the 16 lanes of each row of affine maps x -> A*x + B
// (earlier lanes applied first), with DPP row shifts; the first O lanes of a
// row receive the identity map (A, B finite).
template <int O>
__device__ __forceinline__ void affine_step(float& A, float& B) {
  const float Ap = dpp_or<DppShr<O>::v>(1.f, A);
  // B's identity is 0, which the zero-filling move gives for free (it then
  // folds into the fma as a DPP operand)
  const float Bp = dpp<DppShr<O>::v>(B);
  B = fmaf(A, Bp, B);
  A = A * Ap;
}
__device__ __forceinline__ void affine_scan(float& A, float& B) {
  static_assert(CHUNK == 16, "scans are written for rows of 16 lanes");
  affine_step<1>(A, B);
  affine_step<2>(A, B);
  affine_step<4>(A, B);
  affine_step<8>(A, B);
}

// Inclusive suffix scan of the same maps, later lanes applied first (lane i
// ends with F_i o F_i+1 o ... o F_15).
template <int O>
__device__ __forceinline__ void affine_suffix_step(float& A, float& B) {
  const float An = dpp_or<DppShl<O>::v>(1.f, A);
  const float Bn = dpp<DppShl<O>::v>(B);
  B = fmaf(A, Bn, B);
  A = A * An;
}
__device__ __forceinline__ void affine_suffix_scan(float& A, float& B) {
  affine_suffix_step<1>(A, B);
  affine_suffix_step<2>(A, B);
  affine_suffix_step<4>(A, B);
  affine_suffix_step<8>(A, B);
}

// Inclusive suffix product across the 16 lanes of each row (lane i ends with
// x_i * x_i+1 * ... * x_15), in the same order as the A part of
// affine_suffix_scan.
__device__ __forceinline__ float suffix_prod(float A) {
  A = A * dpp_or<DppShl<1>::v>(1.f, A);
  A = A * dpp_or<DppShl<2>::v>(1.f, A);
  A = A * dpp_or<DppShl<4>::v>(1.f, A);
  A = A * dpp_or<DppShl<8>::v>(1.f, A);
  return A;
}

// Inclusive prefix product across the 16 lanes of each row (lane i ends with
// x_0 * x_1 * ... * x_i).
__device__ __forceinline__ float prefix_prod(float A) {
  A = A * dpp_or<DppShr<1>::v>(1.f, A);
  A = A * dpp_or<DppShr<2>::v>(1.f, A);
  A = A * dpp_or<DppShr<4>::v>(1.f, A);
  A = A * dpp_or<DppShr<8>::v>(1.f, A);
  return A;
}

// Product of x over the 16 lanes of each row (every lane gets it).
__device__ __forceinline__ float row_prod(float x) {
  x *= dpp<DPP_XOR1>(x);
  x *= dpp<DPP_XOR2>(x);
  x *= dpp<DPP_HALF_MIRROR>(x);
  return x * dpp<DPP_MIRROR>(x);
}
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<DPP_XOR1>(x);
  x += dpp<DPP_XOR2>(x);
  x += dpp<DPP_HALF_MIRROR>(x);
  return x + dpp<DPP_MIRROR>(x);
}

// Sums x[i] over the 64 lanes for every i < CHUNK; lane l receives the total
// of index l & 15.  Each halving step exchanges the half of the values a
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
  // lane l (of each row) now holds the total of index (l & 15) >> 2
  return __shfl(y, (lane & (CHUNK - 1)) * 4, WAVE);
}

// Start of chunk k of the chunk sequence that begins at position p (a chunk
// start), clamped to end.
__device__ __forceinline__ int chunk_start(int p, int k, int end) {
  return min(end, p + k * CHUNK);
}

// Entry counts of the long-segment list's length classes, read once per
// workgroup (independent loads).
struct LongCounts {
  int n[NBIN];
  int total;
};
__device__ __forceinline__ LongCounts long_counts(const int32_t* count) {
  LongCounts L;
  L.total = 0;
#pragma unroll
  for (int c = 0; c < NBIN; ++c) L.n[c] = count[c];
#pragma unroll
  for (int c = 0; c < NBIN; ++c) L.total += L.n[c];
  return L;
}
// Entry i < total of the list, longest class first.
__device__ __forceinline__ int64_t long_entry(const int32_t* list, const LongCounts& L, int cap,
                                              int i) {
  int64_t pos = 0;
  bool found = false;
#pragma unroll
  for (int c = NBIN - 1; c >= 0; --c) {
    if (!found) {
      if (i < L.n[c]) { pos = (int64_t)c * cap + i; found = true; }
      else i -= L.n[c];
    }
  }
  return list[pos];
}

// Work queue of the long-segment kernels.  A workgroup takes list entries one
// at a time from a ticket counter (longest class first), so the entries
// spread over the resident workgroups by their length rather than by a
// fixed stride.  The counter is zero at launch; the last workgroup to run
// out of entries clears it, and its finished count, for the next launch.
__device__ __forceinline__ int take_ticket(int32_t* queue) {
  __shared__ int ticket;
  __syncthreads();   // the previous ticket has been read by every wave
  if (threadIdx.x == 0) ticket = atomicAdd(queue, 1);
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(ticket);
}
__device__ __forceinline__ void release_queue(int32_t* queue) {
  if (threadIdx.x == 0 && atomicAdd(queue + 1, 1) == (int)gridDim.x - 1) {
    atomicExch(queue, 0);
    atomicExch(queue + 1, 0);
  }
}

// Per-event mass of a chunk from the incoming mass m: mi after the event,
// mo before it, and the write step size eta (0 for reads and padding).
struct Mass {
  float A, B;     // inclusive affine prefix of the chunk's mass maps
  float mi, mo, eta;
  float keep;     // 1 - eta
};
__device__ __forceinline__ Mass mass_prefix(const Ev& ev) {
  Mass M;
  M.A = (ev.side == 0) ? ev.lam : 1.f;
  M.B = (ev.side == 0) ? ev.wt : 0.f;
  affine_scan(M.A, M.B);
  return M;
}
__device__ __forceinline__ void mass_apply(Mass& M, const Ev& ev, float m, float eps) {
  M.mi = fmaf(M.A, m, M.B);
  M.mo = dpp_or<DPP_SHR1>(m, M.mi);   // lane 0 of a row: the incoming mass
  M.eta = (ev.side == 0 && ev.wt > 0.f) ? ev.wt / (M.mi + eps) : 0.f;
  M.keep = 1.f - M.eta;
}

// Forward pass over a chunk from s: a write (bit i of wm) moves the content
// toward its v row, s <- (1 - eta) s + eta v; a read (bit i of rm) stores
// r * s to its own stash row.  The kind of event i is the same in every lane,
// so each event runs only its kind's arithmetic; padding runs none.
template <typename IO, int CPL>
__device__ __forceinline__ void fwd_replay(const typename Lanes<IO, CPL>::Raw (&x)[CHUNK],
                                           const Mass& M, float rr, uint32_t so, uint32_t wm,
                                           uint32_t rm, rsrc_t rs, uint32_t lb, float (&s)[CPL]) {
  using LN = Lanes<IO, CPL>;
  for_up<0, CHUNK>([&](auto I) {
    if ((wm >> I) & 1u) {
      float xf[CPL];
      LN::get(x[I], xf);
      const float e = bc<I>(M.eta), om = bc<I>(M.keep);
#pragma unroll
      for (int k = 0; k < CPL; ++k) s[k] = fmaf(om, s[k], e * xf[k]);
    } else if ((rm >> I) & 1u) {
      const float r = bc<I>(rr);
      float ctr[CPL];
#pragma unroll
      for (int k = 0; k < CPL; ++k) ctr[k] = r * s[k];
      LN::store(rs, bcu<I>(so) + lb, ctr);
    }
    sched_fence<I>();
  });
}

}  // namespace

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------

template <typename IO, int CPL>
__device__ void scan_fwd_short(const ScanFwdArgs& a, int64_t g, int beg, int end) {
  using LN = Lanes<IO, CPL>;
  const SegCtx<IO, CPL> c = seg_ctx<IO, CPL>(g, a.S, a.H, a.T, a.d_v);
  const int lane = lane_id();
  const uint32_t nrow = (uint32_t)a.T * a.H;
  const rsrc_t rv = make_rsrc(reinterpret_cast<const IO*>(a.v) + c.row0 * a.d_v, nrow * c.pitch);
  const rsrc_t rs = make_rsrc(reinterpret_cast<IO*>(a.stash) + c.row0 * a.k_r * a.d_v,
                              nrow * a.k_r * c.pitch);

  float s[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) s[k] = (c.active && a.slot0) ? a.slot0[g * a.d_v + c.c0 + k] : 0.f;
  float m = a.mass0 ? a.mass0[g] : 0.f;

  float4 rec = make_float4(0.f, 0.f, 0.f, 0.f);
  if (beg < end) rec = load_rec(a.events, beg, min(end, beg + CHUNK) - beg, beg, end);
  for (int p0 = beg; p0 < end;) {
    const int p1 = min(end, p0 + CHUNK);
    const int n = p1 - p0;
    if (p0 != beg) {
      float* ck = a.ckpt_s + (int64_t)(p0 / CHUNK) * a.d_v;
      if (c.active) {
#pragma unroll
        for (int k = 0; k < CPL; ++k) ck[c.c0 + k] = s[k];
      }
      if (lane == 0) a.ckpt_m[p0 / CHUNK] = m;
    }
    const Ev ev = decode_rec(rec, n, c.h, a.H);
    Mass M = mass_prefix(ev);
    mass_apply(M, ev, m, a.eps);
    m = readlane_f(M.mi, n - 1);
    const float rr = (ev.side == 1) ? ev.wt : 0.f;
    const uint32_t xo = (ev.valid && ev.live && ev.side == 0) ? (uint32_t)ev.rb * c.pitch : OOB;
    const uint32_t so = (ev.valid && ev.side == 1) ? ((uint32_t)ev.rb * a.k_r + ev.j) * c.pitch : OOB;
    rec = load_rec(a.events, p1, min(end, p1 + CHUNK) - p1, beg, end);   // next chunk

    const uint32_t wm = (uint32_t)__ballot(ev.valid && ev.side == 0) & 0xFFFFu;
    const uint32_t rm = (uint32_t)__ballot(ev.valid && ev.side == 1) & 0xFFFFu;

    typename LN::Raw x[CHUNK];
    for_up<0, CHUNK>([&](auto I) { x[I] = LN::load(rv, bcu<I>(xo) + c.lb); });
    wait_vmem();
    fwd_replay<IO, CPL>(x, M, rr, so, wm, rm, rs, c.lb, s);
    p0 = p1;
  }
  if (c.active) {
#pragma unroll
    for (int k = 0; k < CPL; ++k) a.slot1[g * a.d_v + c.c0 + k] = s[k];
  }
  if (lane == 0) a.mass1[g] = m;
}

template <typename IO, int CPL>
__device__ void scan_fwd_long(const ScanFwdArgs& a, int64_t g) {
  constexpr int NW = NWL;
  using LN = Lanes<IO, CPL>;
  __shared__ float mapA[NW], mapB[NW], mapP[NW];
  __shared__ float mapb[NW][MAX_DV];
  const SegCtx<IO, CPL> c = seg_ctx<IO, CPL>(g, a.S, a.H, a.T, a.d_v);
  const int lane = lane_id();
  const int w = wave_index();
  const uint32_t nrow = (uint32_t)a.T * a.H;
  const rsrc_t rv = make_rsrc(reinterpret_cast<const IO*>(a.v) + c.row0 * a.d_v, nrow * c.pitch);
  const rsrc_t rs = make_rsrc(reinterpret_cast<IO*>(a.stash) + c.row0 * a.k_r * a.d_v,
                              nrow * a.k_r * c.pitch);
  const int beg = a.seg_offset[g], end = a.seg_offset[g + 1];

  float s_carry[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k)
    s_carry[k] = (c.active && a.slot0) ? a.slot0[g * a.d_v + c.c0 + k] : 0.f;
  float m_carry = a.mass0 ? a.mass0[g] : 0.f;

  // the v rows of a wave's next chunk are requested as soon as its replay of
  // the current chunk is done, so the loads overlap the closing barrier and
  // the next chunk's mass fold
  float4 rec = load_rec(a.events, chunk_start(beg, w, end),
                        chunk_start(beg, w + 1, end) - chunk_start(beg, w, end), beg, end);
  typename LN::Raw x[CHUNK];
  {
    const int n0 = chunk_start(beg, w + 1, end) - chunk_start(beg, w, end);
    const Ev ev0 = decode_rec(rec, n0, c.h, a.H);
    const uint32_t xo0 = (ev0.valid && ev0.live && ev0.side == 0) ? (uint32_t)ev0.rb * c.pitch : OOB;
    for_up<0, CHUNK>([&](auto I) { x[I] = LN::load(rv, bcu<I>(xo0) + c.lb); });
  }
  for (int p = beg; p < end;) {
    const int cs = chunk_start(p, w, end);
    const int n = chunk_start(p, w + 1, end) - cs;
    const int pn = chunk_start(p, NW, end);
    const Ev ev = decode_rec(rec, n, c.h, a.H);
    Mass M = mass_prefix(ev);
    // padded lanes carry the identity, so lane 15 holds the chunk's map
    const float A_tot = bc<15>(M.A), B_tot = bc<15>(M.B);
    if (lane == 0) {
      mapA[w] = A_tot;
      mapB[w] = B_tot;
    }
    const float rr = (ev.side == 1) ? ev.wt : 0.f;
    const uint32_t so = (ev.valid && ev.side == 1) ? ((uint32_t)ev.rb * a.k_r + ev.j) * c.pitch : OOB;
    const uint32_t wm = (uint32_t)__ballot(ev.valid && ev.side == 0) & 0xFFFFu;
    const uint32_t rm = (uint32_t)__ballot(ev.valid && ev.side == 1) & 0xFFFFu;
    // next super-chunk's records for this wave (unconditional: past the end
    // it reloads the last event, unused)
    rec = load_rec(a.events, chunk_start(pn, w, end),
                   chunk_start(pn, w + 1, end) - chunk_start(pn, w, end), beg, end);
    __syncthreads();
    float m_in = m_carry, m_next = m_carry;
    for (int k = 0; k < NW; ++k) {
      if (k == w) m_in = m_next;
      m_next = fmaf(mapA[k], m_next, mapB[k]);
    }
    mass_apply(M, ev, m_in, a.eps);
    // the chunk from a zero content: sz after each event (kept at every
    // event for the reads) and the chunk's map s -> P*s + sz, which the
    // later waves fold
    float sz[CPL], szr[CHUNK][CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) sz[k] = 0.f;
    for_up<0, CHUNK>([&](auto I) {
      if ((wm >> I) & 1u) {
        float xf[CPL];
        LN::get(x[I], xf);
        const float e = bc<I>(M.eta), om = bc<I>(M.keep);
#pragma unroll
        for (int k = 0; k < CPL; ++k) sz[k] = fmaf(om, sz[k], e * xf[k]);
      }
#pragma unroll
      for (int k = 0; k < CPL; ++k) szr[I][k] = sz[k];
      sched_fence<I>();
    });
    const float Pi = prefix_prod(M.keep);   // lane i: product of (1 - eta) over events 0..i
    const float P = bc<15>(Pi);
    if (c.active) {
#pragma unroll
      for (int k = 0; k < CPL; ++k) mapb[w][c.c0 + k] = sz[k];
    }
    if (lane == 0) mapP[w] = P;
    __syncthreads();
    // the rows and records requested before the barriers have arrived by now
    wait_vmem();
    // this wave's start state: the carry through the earlier chunks' maps
    float s[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) s[k] = s_carry[k];
    for (int kk = 0; kk < w; ++kk) {
      const float Pk = mapP[kk];
#pragma unroll
      for (int k = 0; k < CPL; ++k) s[k] = fmaf(Pk, s[k], c.active ? mapb[kk][c.c0 + k] : 0.f);
    }
    if (n > 0 && cs != beg) {
      float* ck = a.ckpt_s + (int64_t)(cs / CHUNK) * a.d_v;
      if (c.active) {
#pragma unroll
        for (int k = 0; k < CPL; ++k) ck[c.c0 + k] = s[k];
      }
      if (lane == 0) a.ckpt_m[cs / CHUNK] = m_in;
    }
    // each read sees P_i * s + sz_i (a read's own factor is 1) and stores
    // r times it to its stash row
    for_up<0, CHUNK>([&](auto I) {
      if ((rm >> I) & 1u) {
        const float r = bc<I>(rr), pi = bc<I>(Pi);
        float ctr[CPL];
#pragma unroll
        for (int k = 0; k < CPL; ++k) ctr[k] = r * fmaf(pi, s[k], szr[I][k]);
        LN::store(rs, bcu<I>(so) + c.lb, ctr);
      }
      sched_fence<I>();
    });
    {   // rows of this wave's next chunk (past the end: no valid event, no load)
      const int n_n = chunk_start(pn, w + 1, end) - chunk_start(pn, w, end);
      const Ev ev_n = decode_rec(rec, n_n, c.h, a.H);
      const uint32_t xo_n = (ev_n.valid && ev_n.live && ev_n.side == 0) ? (uint32_t)ev_n.rb * c.pitch : OOB;
      for_up<0, CHUNK>([&](auto I) { x[I] = LN::load(rv, bcu<I>(xo_n) + c.lb); });
    }
    // the carry into the next chunks: this wave's own map, then the later
    // waves' maps (every wave computes it, in the same order of operations)
#pragma unroll
    for (int k = 0; k < CPL; ++k) s_carry[k] = fmaf(P, s[k], sz[k]);
    for (int kk = w + 1; kk < NW; ++kk) {
      const float Pk = mapP[kk];
#pragma unroll
      for (int k = 0; k < CPL; ++k)
        s_carry[k] = fmaf(Pk, s_carry[k], c.active ? mapb[kk][c.c0 + k] : 0.f);
    }
    m_carry = m_next;
    p = pn;
  }
  if (w == 0) {
    if (c.active) {
#pragma unroll
      for (int k = 0; k < CPL; ++k) a.slot1[g * a.d_v + c.c0 + k] = s_carry[k];
    }
    if (lane == 0) a.mass1[g] = m_carry;
  }
}

// The segment wave i of a short-segment kernel scans (-1: none) and its
// event range.  When at most half of the segments are in the bucketing's
// short list (hot slots take most events, most slots none), wave i takes
// list entry i, so the waves with work are the grid's first and the rest
// end at once; otherwise it takes segment i itself when that one is short,
// which saves the list's extra dependent load where nearly every segment
// has a few events; a wave without work then ends after reading the list
// length alone.  Segments without events are left to fill_empty_kernel.
template <typename Args>
__device__ __forceinline__ int64_t short_segment(const Args& a, int64_t i, int& beg, int& end) {
  const int64_t n = a.use_long ? *a.short_count : 0;
  if (2 * n <= a.nseg) {
    if (i >= n) return -1;
    const int64_t g = a.short_list[i];
    beg = a.seg_offset[g];
    end = a.seg_offset[g + 1];
    return g;
  }
  beg = a.seg_offset[i];
  end = a.seg_offset[i + 1];
  return (end > beg && end - beg <= LONG_EVENTS) ? i : -1;
}

// Segments of 1 to LONG_EVENTS events: one wave each (short_segment).
template <typename IO, int CPL>
__global__ __launch_bounds__(SHORT_WAVES * WAVE) void scan_fwd_short_kernel(ScanFwdArgs a) {
  const int64_t i = (int64_t)blockIdx.x * SHORT_WAVES + wave_index();
  if (i >= a.nseg) return;
  int beg, end;
  const int64_t g = short_segment(a, i, beg, end);
  if (g >= 0) scan_fwd_short<IO, CPL>(a, g, beg, end);
}

// Long segments: a resident grid of NWL-wave workgroups takes the list's
// entries from the work queue, longest class first.
template <typename IO, int CPL>
__global__ __launch_bounds__(NWL * WAVE) void scan_fwd_long_kernel(ScanFwdArgs a) {
  const LongCounts L = long_counts(a.long_count);
  if (L.total == 0) return;   // the queue stays at zero
  for (int i = take_ticket(a.queue); i < L.total; i = take_ticket(a.queue))
    scan_fwd_long<IO, CPL>(a, long_entry(a.long_list, L, a.long_cap, i));
  release_queue(a.queue);
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
// chunk and summed in batched transpose-reductions.  The mass adjoint then
// follows m_hat_before = lambda * (m_hat_after - g * deta), with
// g = w / (m' + eps)^2, which is affine in m_hat: an inclusive suffix scan
// across lanes gives it for every event at once, and each lane forms
//   M = m_hat_after - g * deta
//   dw = deta / (m' + eps) + M + M * m_old * dlambda/dw
//   dgamma part = M * m_old * (-lambda (1 - lambda))
// for its own event and stores it.

// One chunk of the reverse pass: scalars, the event rows x (v for a write,
// dO for a read) and the content before each event, kept in registers or
// (SO_LDS, where registers are short) in this wave's block of LDS.
template <typename IO, int CPL, bool SO_LDS>
struct BwdChunk {
  Ev ev;
  Mass M;
  float rr;                        // read weight, 0 for writes and padding
  uint32_t sw;                     // stash offset of a write's dv row, else OOB
  uint32_t wm, rm;                 // bit i: event i is a write / a read (wave-uniform)
  float rden;                      // 1 / (m' + eps): mass after the event plus eps
  float gq;                        // w / (m' + eps)^2 of a write, else 0
  typename Lanes<IO, CPL>::Raw x[CHUNK];
  // rows in float, unpacked once for both passes where registers allow
  // (the LDS variant: its workgroups are held to four per CU by LDS)
  static constexpr bool UNPACKED = SO_LDS && sizeof(IO) == 2;
  float xf[UNPACKED ? CHUNK : 1][CPL];
  float so_reg[SO_LDS ? 1 : CHUNK][CPL];
  float* so_lds;                   // [CHUNK][MAX_DV] floats at the lane's channel c0

  __device__ __forceinline__ void unpack_rows() {
    if constexpr (UNPACKED) {
#pragma unroll
      for (int i = 0; i < CHUNK; ++i) Lanes<IO, CPL>::get(x[i], xf[i]);
    }
  }
  template <int I>
  __device__ __forceinline__ void get_x(float (&f)[CPL]) const {
    if constexpr (UNPACKED) {
#pragma unroll
      for (int k = 0; k < CPL; ++k) f[k] = xf[I][k];
    } else {
      Lanes<IO, CPL>::get(x[I], f);
    }
  }
  template <int I>
  __device__ __forceinline__ void put_so(const float (&s)[CPL]) {
    if constexpr (SO_LDS) {
      if constexpr (CPL == 2) *reinterpret_cast<float2*>(so_lds + I * MAX_DV) = make_float2(s[0], s[1]);
      else so_lds[I * MAX_DV] = s[0];
    } else {
#pragma unroll
      for (int k = 0; k < CPL; ++k) so_reg[I][k] = s[k];
    }
  }
  template <int I>
  __device__ __forceinline__ void get_so(float (&o)[CPL]) const {
    if constexpr (SO_LDS) {
      if constexpr (CPL == 2) {
        const float2 t = *reinterpret_cast<const float2*>(so_lds + I * MAX_DV);
        o[0] = t.x;
        o[1] = t.y;
      } else {
        o[0] = so_lds[I * MAX_DV];
      }
    } else {
#pragma unroll
      for (int k = 0; k < CPL; ++k) o[k] = so_reg[I][k];
    }
  }
};

// Row gathers of a chunk: the v row of each write and the dO row of each read.
// The kind of event i is the same in every lane, so its one load takes the
// buffer of its kind (a scalar select); padding and the no-op events of
// masked tokens (whose rows may hold anything) load nothing.
template <typename IO, int CPL>
__device__ __forceinline__ void bwd_gather_rows(const ScanBwdArgs& a, const SegCtx<IO, CPL>& c,
                                                rsrc_t rv, rsrc_t ro,
                                                typename Lanes<IO, CPL>::Raw (&x)[CHUNK],
                                                float4 rec, int n) {
  using LN = Lanes<IO, CPL>;
  const Ev ev = decode_rec(rec, n, c.h, a.H);
  const uint32_t xo = (ev.valid && ev.live) ? (uint32_t)ev.rb * c.pitch : OOB;
  const uint32_t wm = (uint32_t)__ballot(ev.valid && ev.side == 0) & 0xFFFFu;
  for_up<0, CHUNK>([&](auto I) {
    x[I] = LN::load(((wm >> I) & 1u) ? rv : ro, bcu<I>(xo) + c.lb);
  });
}
template <typename IO, int CPL, bool SO>
__device__ __forceinline__ void bwd_gather(const ScanBwdArgs& a, const SegCtx<IO, CPL>& c,
                                           rsrc_t rv, rsrc_t ro, BwdChunk<IO, CPL, SO>& ck,
                                           float4 rec, int n) {
  bwd_gather_rows<IO, CPL>(a, c, rv, ro, ck.x, rec, n);
}

// Scalars of a chunk whose rows are gathered: event fields, masses and step
// sizes, read weights and stash offsets.
template <typename IO, int CPL, bool SO>
__device__ __forceinline__ void bwd_prepare(const ScanBwdArgs& a, const SegCtx<IO, CPL>& c,
                                            BwdChunk<IO, CPL, SO>& ck, float4 rec, int n,
                                            float m) {
  ck.ev = decode_rec(rec, n, c.h, a.H);
  const Ev& ev = ck.ev;
  ck.M = mass_prefix(ev);
  mass_apply(ck.M, ev, m, a.eps);
  ck.rr = (ev.side == 1) ? ev.wt : 0.f;
  ck.sw = (ev.valid && ev.side == 0) ? ((uint32_t)ev.rb * a.k_w + ev.j) * c.pitch : OOB;
  ck.wm = (uint32_t)__ballot(ev.valid && ev.side == 0) & 0xFFFFu;
  ck.rm = (uint32_t)__ballot(ev.valid && ev.side == 1) & 0xFFFFu;
  // the gradient scalars divide by m' + eps through its reciprocal (the
  // hardware instruction, within 1 ulp); eta keeps the exact quotient the
  // forward used, so the replay reproduces the forward's contents
  ck.rden = __builtin_amdgcn_rcpf(ck.M.mi + a.eps);
  ck.gq = (ev.valid && ev.side == 0 && ev.wt > 0.f) ? ck.M.eta * ck.rden : 0.f;
}

template <typename IO, int CPL, bool SO>
__device__ __forceinline__ void bwd_setup(const ScanBwdArgs& a, const SegCtx<IO, CPL>& c,
                                          rsrc_t rv, rsrc_t ro, BwdChunk<IO, CPL, SO>& ck, float4 rec,
                                          int n, float m) {
  bwd_gather(a, c, rv, ro, ck, rec, n);
  bwd_prepare(a, c, ck, rec, n, m);
}

// Forward replay of a chunk from s: keeps the content before each write
// and pr[i] = <x_i, s_i> (lane-local) of each read, its dr partial.  An
// event is either a write (step eta, no read weight) or a read (the
// reverse), and its kind is the same in every lane, so each event takes only
// its kind's arithmetic; the results equal those of the common form with
// the other kind's terms zero.
template <typename IO, int CPL, bool SO>
__device__ __forceinline__ void bwd_replay(BwdChunk<IO, CPL, SO>& ck, float (&s)[CPL],
                                           float (&pr)[CHUNK]) {
  using LN = Lanes<IO, CPL>;
  for_up<0, CHUNK>([&](auto I) {
    if ((ck.wm >> I) & 1u) {
      float xf[CPL];
      ck.template get_x<I>(xf);
      const float e = bc<I>(ck.M.eta), om = bc<I>(ck.M.keep);
      ck.template put_so<I>(s);
#pragma unroll
      for (int k = 0; k < CPL; ++k) s[k] = fmaf(om, s[k], e * xf[k]);
    } else if ((ck.rm >> I) & 1u) {
      float xf[CPL];
      ck.template get_x<I>(xf);
      float d = 0.f;
#pragma unroll
      for (int k = 0; k < CPL; ++k) d = fmaf(xf[k], s[k], d);
      pr[I] = d;
    }
    sched_fence<I>();
  });
}

// The same replay, which also forms the chunk's content adjoint map from a
// zero adjoint at its end: walking back, a read adds r_i x_i and a write
// scales by (1 - eta_j), so the adjoint at the chunk's start is
//   q = sum over reads i of c_i x_i,  c_i = r_i * prod over writes j < i of (1 - eta_j)
// (cq holds c_i in lane i) and the map is s_hat -> Q s_hat + q with Q the
// product of all (1 - eta).
template <typename IO, int CPL, bool SO>
__device__ __forceinline__ void bwd_replay_map(BwdChunk<IO, CPL, SO>& ck, float (&s)[CPL],
                                               float (&pr)[CHUNK], float cq, float (&q)[CPL]) {
  using LN = Lanes<IO, CPL>;
#pragma unroll
  for (int k = 0; k < CPL; ++k) q[k] = 0.f;
  for_up<0, CHUNK>([&](auto I) {
    if ((ck.wm >> I) & 1u) {
      float xf[CPL];
      ck.template get_x<I>(xf);
      const float e = bc<I>(ck.M.eta), om = bc<I>(ck.M.keep);
      ck.template put_so<I>(s);
#pragma unroll
      for (int k = 0; k < CPL; ++k) s[k] = fmaf(om, s[k], e * xf[k]);
    } else if ((ck.rm >> I) & 1u) {
      float xf[CPL];
      ck.template get_x<I>(xf);
      const float ci = bc<I>(cq);
      float d = 0.f;
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        d = fmaf(xf[k], s[k], d);
        q[k] = fmaf(ci, xf[k], q[k]);
      }
      pr[I] = d;
    }
    sched_fence<I>();
  });
}

// Reverse walk of the content adjoint from sh (after the chunk) to sh (before
// it): stores the dv contributions e * s_hat of the writes and leaves in pw
// the lane-local partials of each event's scalar gradient: <s_hat_after,
// x - s_old> (the deta of a write), or the replay's partial pr of a read (its
// dr), so that one batched reduction serves both kinds.
// DEFER (contents in LDS only): each write's contribution is left in its
// event's LDS slot, whose pre-write content the walk no longer needs, and
// stored later by flush_dv.
template <typename IO, int CPL, bool SO, bool DEFER = false>
__device__ __forceinline__ void bwd_walk(BwdChunk<IO, CPL, SO>& ck, const SegCtx<IO, CPL>& c,
                                         rsrc_t rs, float (&sh)[CPL], const float (&pr)[CHUNK],
                                         float (&pw)[CHUNK]) {
  static_assert(!DEFER || SO, "deferred stores keep the contributions in LDS");
  using LN = Lanes<IO, CPL>;
  // each event's pre-write content is read from LDS one event ahead, outside
  // the per-kind branches, so the read has an event's work to complete in
  float so_n[CPL];
  ck.template get_so<CHUNK - 1>(so_n);
  for_down<CHUNK>([&](auto I) {
    float so[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) so[k] = so_n[k];
    if constexpr (I > 0) ck.template get_so<I - 1>(so_n);
    pw[I] = 0.f;
    if ((ck.wm >> I) & 1u) {
      float xf[CPL], ctr[CPL];
      ck.template get_x<I>(xf);
      const float e = bc<I>(ck.M.eta);
      float d = 0.f;
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        ctr[k] = e * sh[k];
        d = fmaf(sh[k], xf[k] - so[k], d);
        sh[k] = fmaf(-e, sh[k], sh[k]);
      }
      if constexpr (DEFER) ck.template put_so<I>(ctr);
      else LN::store(rs, bcu<I>(ck.sw) + c.lb, ctr);
      pw[I] = d;
    } else if ((ck.rm >> I) & 1u) {
      float xf[CPL];
      ck.template get_x<I>(xf);
      const float r = bc<I>(ck.rr);
#pragma unroll
      for (int k = 0; k < CPL; ++k) sh[k] = fmaf(r, xf[k], sh[k]);
      pw[I] = pr[I];
    }
    sched_fence<I>();
  });
}

// Stores the dv contributions a deferred walk left in LDS (sw: the chunk's
// per-event stash offsets, OOB for all but writes, so those stores drop).
template <typename IO, int CPL>
__device__ __forceinline__ void flush_dv(const BwdChunk<IO, CPL, true>& ck, rsrc_t rs, uint32_t sw,
                                         uint32_t lb) {
  using LN = Lanes<IO, CPL>;
  for_up<0, CHUNK>([&](auto I) {
    float v[CPL];
    ck.template get_so<I>(v);
    LN::store(rs, bcu<I>(sw) + lb, v);
  });
}

// Lane-parallel scalar part of a chunk's reverse step, in two halves.  red
// (lane i) holds dr_i for a read and deta_i for a write.  The mass adjoint
// m_hat_before = lambda * (m_hat_after - g * deta) of a write is affine in
// m_hat; bwd_mass_maps composes these maps over the later events of the chunk
// (lane i: F_i o ... o F_15, so lane 0 holds the whole chunk's map), and
// bwd_mass_grads, given the mass adjoint after the chunk, forms dr, dw and
// the gamma parts (ChunkGrads, stored by store_grads) and returns the adjoint
// before the chunk.
struct MassAdj {
  float A, B, deta;
};
template <typename IO, int CPL, bool SO>
__device__ __forceinline__ MassAdj bwd_mass_maps(const BwdChunk<IO, CPL, SO>& ck, float red) {
  const Ev& ev = ck.ev;
  const bool wr = ev.valid && ev.side == 0;
  MassAdj ma;
  ma.deta = wr ? red : 0.f;
  ma.A = wr ? ev.lam : 1.f;
  ma.B = wr ? -ev.lam * ck.gq * ma.deta : 0.f;
  affine_suffix_scan(ma.A, ma.B);
  return ma;
}
// Lane i < 16: the gradients of event i, at byte offsets inside its batch's
// rows of dw and dgam (a write) or dr (a read); OOB where there is none.
struct ChunkGrads {
  float dw, dg, dr;
  uint32_t ow, orr;
};
template <typename IO, int CPL, bool SO>
__device__ __forceinline__ float bwd_mass_grads(const ScanBwdArgs& a, const BwdChunk<IO, CPL, SO>& ck,
                                                const MassAdj& ma, float red, float mh,
                                                ChunkGrads& gr) {
  const Ev& ev = ck.ev;
  const bool wr = ev.valid && ev.side == 0;
  const float before = fmaf(ma.A, mh, ma.B);
  const float after = dpp_or<DPP_SHL1>(mh, before);   // lane 15: the chunk's m_hat
  const float M = after - ck.gq * ma.deta;
  // dw = deta * d eta/dw + M * dm'/dw with dm'/dw = 1 + m * dlambda/dw.  The
  // part of deta * d eta/dw that goes through m' is taken together with the
  // direct one: 1/(m'+eps) - w/(m'+eps)^2 = (lambda m + eps)/(m'+eps)^2,
  // which keeps the small eps of a first write to an empty slot exact where
  // the difference of the two terms (both about 1/w) would lose it.
  const float dm = fmaf(ck.M.mo, ev.dl, 1.f);
  const float deta_dw = (ev.wt > 0.f) ? fmaf(ev.lam, ck.M.mo, a.eps) * ck.rden * ck.rden : 0.f;
  gr.dw = ma.deta * (deta_dw - ck.gq * ck.M.mo * ev.dl) + after * dm;
  // d lambda / d gamma = -lambda (1 - lambda) = (d lambda / d w) w (1 - w):
  // the first form where lambda < 1/2, the second (1 - w close to 1) where
  // 1 - lambda would be the difference of two numbers close to 1
  const float lam1 = (ev.lam < 0.5f) ? -ev.lam * (1.f - ev.lam) : ev.dl * ev.wt * (1.f - ev.wt);
  gr.dg = M * ck.M.mo * lam1;
  gr.dr = red;
  if (!ev.live) {
    // a masked token's no-op event stands for no event at all: no gradients
    gr.dw = 0.f;
    gr.dg = 0.f;
    gr.dr = 0.f;
  }
  const bool mine = lane_id() < CHUNK;
  gr.ow = (mine && wr) ? ((uint32_t)ev.rb * a.k_w + ev.j) * 4u : OOB;
  gr.orr = (mine && !wr && ev.valid) ? ((uint32_t)ev.rb * a.k_r + ev.j) * 4u : OOB;
  return readlane_f(before, 0);
}
// Stores a chunk's gradients (three stores, each dropped where its offset is
// OOB).
template <typename IO, int CPL>
__device__ __forceinline__ void store_grads(const ScanBwdArgs& a, const SegCtx<IO, CPL>& c,
                                            const ChunkGrads& gr) {
  const uint32_t nrow = (uint32_t)a.T * a.H;
  const rsrc_t rdw = make_rsrc(a.dw + c.row0 * a.k_w, nrow * a.k_w * 4u);
  const rsrc_t rdg = make_rsrc(a.dgam + c.row0 * a.k_w, nrow * a.k_w * 4u);
  const rsrc_t rdr = make_rsrc(a.dr + c.row0 * a.k_r, nrow * a.k_r * 4u);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gr.dw), rdw, gr.ow, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gr.dg), rdg, gr.ow, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gr.dr), rdr, gr.orr, 0, 0);
}
template <typename IO, int CPL, bool SO>
__device__ __forceinline__ void bwd_scalars(const ScanBwdArgs& a, const SegCtx<IO, CPL>& c,
                                            const BwdChunk<IO, CPL, SO>& ck, float red, float& mh) {
  ChunkGrads gr;
  mh = bwd_mass_grads(a, ck, bwd_mass_maps(ck, red), red, mh, gr);
  store_grads(a, c, gr);
}

// State at the start of chunk cs of segment g: the initial state for the
// segment's first chunk, else the checkpoint the forward saved.
// The loads are unconditional (a valid address is always chosen: an
// inactive lane reads the row's last channels, a missing initial state reads
// checkpoint 0) and the value is selected afterwards, so no wait sits inside
// a branch.  cs may be the segment end (an empty chunk of the long path):
// checkpoint cs / 16 <= E / 16 exists.
// The loaded values and the selection are kept apart (ChunkStart holds the
// raw loads), so a caller can carry the loads in flight across a loop
// iteration and select once they have arrived.
template <int CPL>
struct ChunkStart {
  float t[CPL], tm;   // loaded content and mass
  bool zero;          // the segment's first chunk with no initial state
};
template <typename IO, int CPL>
__device__ __forceinline__ void chunk_state_load(const ScanBwdArgs& a, const SegCtx<IO, CPL>& c,
                                                 int64_t g, int beg, int cs, ChunkStart<CPL>& st) {
  const bool first = cs == beg;
  st.zero = first && !a.slot0;
  const float* sp = first ? (a.slot0 ? a.slot0 + g * a.d_v : a.ckpt_s)
                          : a.ckpt_s + (int64_t)(cs / CHUNK) * a.d_v;
  const float* mp = first ? (a.mass0 ? a.mass0 + g : a.ckpt_m) : a.ckpt_m + cs / CHUNK;
  const int cc = min(c.c0, a.d_v - CPL);
#pragma unroll
  for (int k = 0; k < CPL; ++k) st.t[k] = ld_global(sp + cc + k);
  st.tm = ld_global(mp);
}
template <typename IO, int CPL>
__device__ __forceinline__ void chunk_state_take(const SegCtx<IO, CPL>& c, const ChunkStart<CPL>& st,
                                                 float (&s)[CPL], float& m) {
#pragma unroll
  for (int k = 0; k < CPL; ++k) s[k] = (st.zero || !c.active) ? 0.f : st.t[k];
  m = st.zero ? 0.f : st.tm;
}
template <typename IO, int CPL>
__device__ __forceinline__ void chunk_state(const ScanBwdArgs& a, const SegCtx<IO, CPL>& c,
                                            int64_t g, int beg, int cs, float (&s)[CPL],
                                            float& m) {
  ChunkStart<CPL> st;
  chunk_state_load(a, c, g, beg, cs, st);
  chunk_state_take(c, st, s, m);
}

template <typename IO, int CPL>
__device__ void scan_bwd_short(const ScanBwdArgs& a, int64_t g, int beg, int end) {
  const SegCtx<IO, CPL> c = seg_ctx<IO, CPL>(g, a.S, a.H, a.T, a.d_v);
  const int lane = lane_id();
  const uint32_t nrow = (uint32_t)a.T * a.H;
  const rsrc_t rv = make_rsrc(reinterpret_cast<const IO*>(a.v) + c.row0 * a.d_v, nrow * c.pitch);
  const rsrc_t ro = make_rsrc(reinterpret_cast<const IO*>(a.d_o) + c.row0 * a.d_v, nrow * c.pitch);
  const rsrc_t rs = make_rsrc(reinterpret_cast<IO*>(a.stash) + c.row0 * a.k_w * a.d_v,
                              nrow * a.k_w * c.pitch);

  float sh[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k)
    sh[k] = (c.active && a.d_slot1) ? a.d_slot1[g * a.d_v + c.c0 + k] : 0.f;
  float mh = a.d_mass1 ? a.d_mass1[g] : 0.f;

  if (beg < end) {
    BwdChunk<IO, CPL, false> ck;
    float pr[CHUNK], pw[CHUNK];
    int cs = beg + ((end - 1 - beg) / CHUNK) * CHUNK;
    float4 rec = load_rec(a.events, cs, end - cs, beg, end);
    while (true) {
      const int n = min(end, cs + CHUNK) - cs;
      const int cp = max(beg, cs - CHUNK);
      float s[CPL], m;
      chunk_state<IO, CPL>(a, c, g, beg, cs, s, m);
      const float4 rec_cur = rec;
      rec = load_rec(a.events, cp, cs - cp, beg, end);   // previous chunk (unused after the first)
      bwd_setup(a, c, rv, ro, ck, rec_cur, n, m);
      // the row loads are done before the event loops, whose stores then
      // never wait (a padded event's load is never consumed)
      wait_vmem();
      bwd_replay(ck, s, pr);
      bwd_walk(ck, c, rs, sh, pr, pw);
      bwd_scalars(a, c, ck, batched_sum(pw), mh);
      if (cs == beg) break;
      cs = cp;
    }
  }
  if (a.d_slot0 && c.active) {
#pragma unroll
    for (int k = 0; k < CPL; ++k) a.d_slot0[g * a.d_v + c.c0 + k] = sh[k];
  }
  if (a.d_mass0 && lane == 0) a.d_mass0[g] = mh;
}

// Long segments: a workgroup of NWL waves takes NWL consecutive chunks at a
// time, from the end of the segment.  Each wave replays its chunk from its
// checkpoint and, in the same pass, forms the chunk's content adjoint map
// from a zero adjoint at its end, s_hat_in = Q * s_hat_out + q (Q = prod
// (1 - eta); q a weighted sum of the chunk's read rows).  Folding the later
// chunks' maps onto the carry gives each wave its true s_hat after its chunk,
// and it runs the exact reverse walk from there, which fixes every deta of
// the chunk.  The mass adjoint is then affine in m_hat with known
// coefficients: each wave composes its chunk's scalar map, the maps are
// folded the same way, and each wave finishes its own chunk's gradients.
// Two workgroup barriers per NWL chunks; wave 0's walk gives the content
// carry into the previous NWL chunks, the folded mass maps the mass carry.
template <typename IO, int CPL>
__device__ void scan_bwd_long(const ScanBwdArgs& args, int64_t g) {
  ScanBwdArgs a = args;
  fresh(a.events), fresh(a.ckpt_s), fresh(a.ckpt_m), fresh(a.slot0), fresh(a.mass0);
  fresh(a.dw), fresh(a.dr), fresh(a.dgam), fresh(a.d_slot0), fresh(a.d_mass0);
  fresh(a.d_slot1), fresh(a.d_mass1), fresh(a.stash), fresh(a.v), fresh(a.d_o);
  fresh(a.seg_offset);
  constexpr int NW = NWL;
  using LN = Lanes<IO, CPL>;
  __shared__ float mQ[NW], mA[NW], mB[NW];
  __shared__ float mq[NW][MAX_DV];
  __shared__ float carry_s[MAX_DV];
  const SegCtx<IO, CPL> c = seg_ctx<IO, CPL>(g, a.S, a.H, a.T, a.d_v);
  const int lane = lane_id();
  const int w = wave_index();
  const uint32_t nrow = (uint32_t)a.T * a.H;
  const rsrc_t rv = make_rsrc(reinterpret_cast<const IO*>(a.v) + c.row0 * a.d_v, nrow * c.pitch);
  const rsrc_t ro = make_rsrc(reinterpret_cast<const IO*>(a.d_o) + c.row0 * a.d_v, nrow * c.pitch);
  const rsrc_t rs = make_rsrc(reinterpret_cast<IO*>(a.stash) + c.row0 * a.k_w * a.d_v,
                              nrow * a.k_w * c.pitch);
  const int beg = ld_global(a.seg_offset + g), end = ld_global(a.seg_offset + g + 1);
  const int nchunks = (end - beg + CHUNK - 1) / CHUNK;

  float sh_carry[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k)
    sh_carry[k] = (c.active && a.d_slot1) ? ld_global(a.d_slot1 + g * a.d_v + c.c0 + k) : 0.f;
  float mh_carry = a.d_mass1 ? ld_global(a.d_mass1 + g) : 0.f;

  __shared__ float so_lds[NW][CHUNK][MAX_DV];   // pre-write contents, per wave
  BwdChunk<IO, CPL, true> ck;
  ck.so_lds = &so_lds[w][0][0] + c.c0;
  float pr[CHUNK], pw[CHUNK];
  auto chunk_of = [&](int k, int& cs, int& n) {
    cs = end;
    n = 0;
    if (k < nchunks) {
      cs = chunk_start(beg, k, end);
      n = chunk_start(beg, k + 1, end) - cs;
    }
  };
  // The rows and the start state of a wave's next chunk are requested at the
  // start of the current chunk's work, into a second set of registers, so
  // that the loads are in flight during the whole iteration.
  typename LN::Raw xn[CHUNK];
  // a chunk's stores are issued at the start of the next iteration, a whole
  // iteration before the wait for that iteration's loads, so no wait ever
  // covers a store just issued: its dv contributions stay in the wave's LDS
  // slots, its gradients in gr, its stash offsets in sw_prev
  uint32_t sw_prev = OOB;
  ChunkGrads gr;
  gr.dw = gr.dg = gr.dr = 0.f;
  gr.ow = gr.orr = OOB;
  float4 rec, rec_next;
  ChunkStart<CPL> st;
  int cs, n;
  {
    const int u_first = ((nchunks - 1) / NW) * NW;
    chunk_of(u_first + w, cs, n);
    rec = load_rec(a.events, cs, n, beg, end);
    int csp, np;
    chunk_of(max(u_first - NW, 0) + w, csp, np);
    rec_next = load_rec(a.events, csp, np, beg, end);
    chunk_state_load<IO, CPL>(a, c, g, beg, cs, st);
    bwd_gather_rows<IO, CPL>(a, c, rv, ro, xn, rec, n);
  }
  for (int u0 = ((nchunks - 1) / NW) * NW; u0 >= 0; u0 -= NW) {
    // this chunk's rows and start state, requested at the start of the
    // previous iteration, are in by now; once they are known to be done the
    // event loops' stores never wait
    wait_vmem();
    for_up<0, CHUNK>([&](auto I) { ck.x[I] = xn[I]; });
    ck.unpack_rows();
    float s[CPL], m;
    chunk_state_take(c, st, s, m);
    flush_dv(ck, rs, sw_prev, c.lb);
    store_grads(a, c, gr);
    bwd_prepare(a, c, ck, rec, n, m);
    sw_prev = ck.sw;
    // next chunk of this wave: rows, start state and the record after it
    // (unconditional: past the segment's start the chunk is empty)
    int csn, nn;
    chunk_of(max(u0 - NW, 0) + w, csn, nn);
    if (u0 < NW) { csn = end; nn = 0; }
    const float4 rec_n = rec_next;
    {
      int csp, np;
      chunk_of(max(u0 - 2 * NW, 0) + w, csp, np);
      rec_next = load_rec(a.events, csp, np, beg, end);
    }
    chunk_state_load<IO, CPL>(a, c, g, beg, csn, st);
    bwd_gather_rows<IO, CPL>(a, c, rv, ro, xn, rec_n, nn);
    // content adjoint map of the chunk from a zero adjoint at its end,
    // formed during the replay (the weights of its reads are prefix
    // products of 1 - eta over the chunk's earlier writes)
    const float Pk = prefix_prod(ck.M.keep);
    const float cq = ck.rr * dpp_or<DPP_SHR1>(1.f, Pk);
    const float Qw = bc<15>(Pk);   // every lane: the broadcast reads lane 15
    float q[CPL];
    bwd_replay_map(ck, s, pr, cq, q);
    if (c.active) {
#pragma unroll
      for (int k = 0; k < CPL; ++k) mq[w][c.c0 + k] = q[k];
    }
    if (lane == 0) mQ[w] = Qw;
    __syncthreads();
    // content adjoint after this wave's chunk: the later chunks' maps
    // folded onto the carry; then the exact reverse walk from it
    float sh[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) sh[k] = sh_carry[k];
    for (int kk = NW - 1; kk > w; --kk) {
      const float Qk = mQ[kk];
#pragma unroll
      for (int k = 0; k < CPL; ++k) sh[k] = fmaf(Qk, sh[k], c.active ? mq[kk][c.c0 + k] : 0.f);
    }
    bwd_walk<IO, CPL, true, true>(ck, c, rs, sh, pr, pw);
    if (w == 0 && c.active) {
#pragma unroll
      for (int k = 0; k < CPL; ++k) carry_s[c.c0 + k] = sh[k];
    }
    // the mass adjoint, now that every deta is known: each chunk's map,
    // folded the same way
    const float red = batched_sum(pw);   // deta of the writes, dr of the reads
    const MassAdj ma = bwd_mass_maps(ck, red);
    if (lane == 0) { mA[w] = ma.A; mB[w] = ma.B; }
    __syncthreads();
    float mh = mh_carry;
    for (int kk = NW - 1; kk > w; --kk) mh = fmaf(mA[kk], mh, mB[kk]);
    bwd_mass_grads(a, ck, ma, red, mh, gr);
    for (int kk = w; kk >= 0; --kk) mh = fmaf(mA[kk], mh, mB[kk]);
    mh_carry = mh;
#pragma unroll
    for (int k = 0; k < CPL; ++k) sh_carry[k] = c.active ? carry_s[c.c0 + k] : 0.f;
    rec = rec_n;
    cs = csn;
    n = nn;
  }
  flush_dv(ck, rs, sw_prev, c.lb);
  store_grads(a, c, gr);
  if (w == 0) {
    if (a.d_slot0 && c.active) {
#pragma unroll
      for (int k = 0; k < CPL; ++k) st_global(a.d_slot0 + g * a.d_v + c.c0 + k, sh_carry[k]);
    }
    if (a.d_mass0 && lane == 0) st_global(a.d_mass0 + g, mh_carry);
  }
}

// Same split as the forward.  Held to five waves per SIMD (96 registers,
// three of them spilled): its waves are bound by dependent memory round
// trips, and the fifth wave measured 3-4% faster where short segments carry
// the pass (1.3B shape without bias: 1.108 -> 1.074 ms; as U = 2 x 64:
// 1.056 -> 1.016 ms); six or eight waves spill 18 or 34 registers and are
// 20-50% slower.
template <typename IO, int CPL>
__global__ __launch_bounds__(SHORT_WAVES * WAVE) __attribute__((amdgpu_waves_per_eu(5, 8)))
void scan_bwd_short_kernel(ScanBwdArgs a) {
  const int64_t i = (int64_t)blockIdx.x * SHORT_WAVES + wave_index();
  if (i >= a.nseg) return;
  int beg, end;
  const int64_t g = short_segment(a, i, beg, end);
  if (g >= 0) scan_bwd_short<IO, CPL>(a, g, beg, end);
}

// Segments without events keep their state: dst = src bit for bit, or 0
// where src is null (forward: slot1 / mass1 from slot0 / mass0; reverse:
// d_slot0 / d_mass0 from d_slot1 / d_mass1).  One wave per 64 consecutive
// segments: lane l checks segment g0 + l, then the wave writes the rows of
// the empty ones item by item (16-byte vectors when VEC, else floats), four
// items per lane at a time, every load before any store.
struct FillArgs {
  int64_t nseg;
  int d_v;
  const int32_t* seg_offset;
  const float* src_s;     // (nseg, d_v) or null
  const float* src_m;     // (nseg) or null
  float* dst_s;           // (nseg, d_v) or null: nothing to write
  float* dst_m;           // (nseg) or null
};

template <bool VEC>
__global__ __launch_bounds__(256) void fill_empty_kernel(FillArgs f) {
  using T = typename std::conditional<VEC, float4, float>::type;
  const int lane = lane_id();
  const int64_t g0 = ((int64_t)blockIdx.x * 4 + wave_index()) * WAVE;
  if (g0 >= f.nseg) return;
  const int64_t g = g0 + lane;
  const bool empty = g < f.nseg && f.seg_offset[g + 1] == f.seg_offset[g];
  const uint64_t em = __ballot(empty);
  if (em == 0) return;
  if (empty && f.dst_m) f.dst_m[g] = f.src_m ? f.src_m[g] : 0.f;
  if (!f.dst_s) return;
  const uint32_t per = VEC ? f.d_v / 4 : f.d_v;   // items per row
  const uint32_t items = WAVE * per;
  const T* src = reinterpret_cast<const T*>(f.src_s);
  T* dst = reinterpret_cast<T*>(f.dst_s);
  for (uint32_t it0 = 0; it0 < items; it0 += 4 * WAVE) {
    T x[4];
    int64_t at[4];
    bool ok[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t it = it0 + u * WAVE + lane;
      const uint32_t r = it / per;
      ok[u] = it < items && ((em >> r) & 1);
      at[u] = (g0 + r) * per + (it - r * per);
      if (src && ok[u]) x[u] = src[at[u]];
      else x[u] = T{};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (ok[u]) dst[at[u]] = x[u];
  }
}

// At most 128 registers, so that 4 workgroups fit on a CU (the rows of the
// next chunk held in flight take 16 of them).
template <typename IO, int CPL>
__global__ __launch_bounds__(NWL * WAVE, 4) void scan_bwd_long_kernel(ScanBwdArgs a) {
  const LongCounts L = long_counts(a.long_count);
  if (L.total == 0) return;   // the queue stays at zero
  for (int i = take_ticket(a.queue); i < L.total; i = take_ticket(a.queue))
    scan_bwd_long<IO, CPL>(a, long_entry(a.long_list, L, a.long_cap, i));
  release_queue(a.queue);
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
        unpack16(ld_nt16(base + (int64_t)j * a.d_v), x);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += x[e];
      }
      st_nt16(out + row * a.d_v + vcol * E, pack16(acc));
    }
  } else if (tid < a.N * a.d_v) {
    const int64_t row = tid / a.d_v;
    const int c = (int)(tid % a.d_v);
    float acc = 0.f;
    for (int j = 0; j < a.k; ++j) acc += to_f32(st[(row * a.k + j) * a.d_v + c]);
    out[row * a.d_v + c] = from_f32<IO>(acc);
  }
  if (a.dgam) {
    // the thread of a row's first column also sums the row's dgam, so that
    // the sums spread over the grid with the rows
    const int per_row = (a.d_v % E == 0) ? a.d_v / E : a.d_v;
    const int64_t row = tid / per_row;
    if (tid - row * per_row == 0 && row < a.N) {
      float sum = 0.f;
      for (int j = 0; j < a.k; ++j) sum += a.dgam[row * a.k + j];
      reinterpret_cast<IO*>(a.d_gamma)[row] = from_f32<IO>(sum);
    }
  }
}

// ---------------------------------------------------------------------------

namespace {
// Long-kernel workgroups per CU at most.  The long kernel pulls work until
// its queue is empty, so the wave slots and registers it leaves free are the
// ones the short-segment kernel beside it runs in.  Measured on the
// 1.3B-layer shape: 4 for the forward (3, 5 and 6 are slower), 4 for the
// reverse (its LDS allows no more; at 128 registers its 4 workgroups then
// hold all of a CU's registers until their queue runs dry, and 3 is slower).
constexpr int LONG_GROUPS_FWD = 4;
constexpr int LONG_GROUPS_BWD = 4;

// Workgroups of the long kernel that run at once: as many as fit, at most
// `cap` per CU.
template <typename Args>
int resident_blocks(void (*kern)(Args), int threads, int cap) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, 0) != hipSuccess)
    return 0;
  if (per_cu > cap) per_cu = cap;
  return cus > 0 && per_cu > 0 ? cus * per_cu : 0;
}

// Long kernel on `st`, short kernel on `side` (the caller orders the two
// streams).  The long grid is the resident count above, capped by the list
// capacity: the work queue needs no more.  The long kernel is enqueued
// first so that its workgroups, which hold the critical path, are resident
// before the short kernel's many small ones fill the device.  The short
// kernel has a wave per segment.
template <typename Args>
hipError_t launch_pair(void (*shortk)(Args), void (*longk)(Args), int& resident, int per_cu,
                       const Args& a, hipStream_t st, hipStream_t side) {
  if (a.use_long) {
    if (resident == 0) resident = resident_blocks(longk, NWL * WAVE, per_cu);
    if (resident == 0) return hipErrorInvalidDeviceFunction;
    const int64_t cap = (int64_t)a.long_cap * NBIN;
    const unsigned lgrid = (unsigned)(cap < resident ? cap : resident);
    hipLaunchKernelGGL(longk, dim3(lgrid), dim3(NWL * WAVE), 0, st, a);
  }
  const unsigned sgrid = (unsigned)((a.nseg + SHORT_WAVES - 1) / SHORT_WAVES);
  hipLaunchKernelGGL(shortk, dim3(sgrid), dim3(SHORT_WAVES * WAVE), 0, side, a);
  return hipGetLastError();
}

// The state of the segments without events, on `st` after the long kernel
// (beside the short kernel it held that one up): nothing to do when dst is
// null or the same arrays as src.
hipError_t launch_fill(const FillArgs& f, hipStream_t st) {
  if (!f.dst_s && !f.dst_m) return hipSuccess;
  if (f.dst_s == f.src_s && f.dst_m == f.src_m) return hipSuccess;
  const bool vec = f.d_v % 4 == 0 && (((uintptr_t)f.src_s | (uintptr_t)f.dst_s) & 15u) == 0;
  const unsigned groups = (unsigned)((f.nseg + 4 * WAVE - 1) / (4 * WAVE));
  if (vec) hipLaunchKernelGGL(fill_empty_kernel<true>, dim3(groups), dim3(256), 0, st, f);
  else hipLaunchKernelGGL(fill_empty_kernel<false>, dim3(groups), dim3(256), 0, st, f);
  return hipGetLastError();
}

template <typename Args>
hipError_t launch_scan(void (*shortk)(Args), void (*longk)(Args), int& resident, int per_cu,
                       const Args& a, const FillArgs& f, hipStream_t st, hipStream_t side) {
  const hipError_t e = launch_pair(shortk, longk, resident, per_cu, a, st, side);
  return e != hipSuccess ? e : launch_fill(f, st);
}
}  // namespace

hipError_t launch_scan_fwd(const ScanFwdArgs& a, bool bf16, hipStream_t st, hipStream_t side) {
  if (a.nseg == 0) return hipSuccess;
  static int res[4] = {0, 0, 0, 0};
  const FillArgs f{a.nseg, a.d_v, a.seg_offset, a.slot0, a.mass0, a.slot1, a.mass1};
  if (bf16) {
    if (a.d_v > 64)
      return launch_scan(scan_fwd_short_kernel<bf16_t, 2>, scan_fwd_long_kernel<bf16_t, 2>, res[0], LONG_GROUPS_FWD, a, f, st, side);
    return launch_scan(scan_fwd_short_kernel<bf16_t, 1>, scan_fwd_long_kernel<bf16_t, 1>, res[1], LONG_GROUPS_FWD, a, f, st, side);
  }
  if (a.d_v > 64)
    return launch_scan(scan_fwd_short_kernel<float, 2>, scan_fwd_long_kernel<float, 2>, res[2], LONG_GROUPS_FWD, a, f, st, side);
  return launch_scan(scan_fwd_short_kernel<float, 1>, scan_fwd_long_kernel<float, 1>, res[3], LONG_GROUPS_FWD, a, f, st, side);
}

hipError_t launch_scan_bwd(const ScanBwdArgs& a, bool bf16, hipStream_t st, hipStream_t side) {
  if (a.nseg == 0) return hipSuccess;
  static int res[4] = {0, 0, 0, 0};
  const FillArgs f{a.nseg, a.d_v, a.seg_offset, a.d_slot1, a.d_mass1, a.d_slot0, a.d_mass0};
  if (bf16) {
    if (a.d_v > 64)
      return launch_scan(scan_bwd_short_kernel<bf16_t, 2>, scan_bwd_long_kernel<bf16_t, 2>, res[0], LONG_GROUPS_BWD, a, f, st, side);
    return launch_scan(scan_bwd_short_kernel<bf16_t, 1>, scan_bwd_long_kernel<bf16_t, 1>, res[1], LONG_GROUPS_BWD, a, f, st, side);
  }
  if (a.d_v > 64)
    return launch_scan(scan_bwd_short_kernel<float, 2>, scan_bwd_long_kernel<float, 2>, res[2], LONG_GROUPS_BWD, a, f, st, side);
  return launch_scan(scan_bwd_short_kernel<float, 1>, scan_bwd_long_kernel<float, 1>, res[3], LONG_GROUPS_BWD, a, f, st, side);
}

hipError_t launch_finalize(const FinalizeArgs& a, bool bf16, hipStream_t st) {
  if (a.N == 0) return hipSuccess;
  const int E = bf16 ? 8 : 4;
  const int64_t threads = (a.d_v % E == 0) ? a.N * (a.d_v / E) : a.N * a.d_v;
  // one-wave workgroups: a read-heavy stream runs faster in them on this
  // device than in four-wave ones
  const dim3 grid((unsigned)((threads + WAVE - 1) / WAVE)), block(WAVE);
  if (bf16) hipLaunchKernelGGL(finalize_kernel<bf16_t>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(finalize_kernel<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace ramk
