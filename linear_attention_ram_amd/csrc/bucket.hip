// Event bucketing (paper §4 "Slot-Parallel Execution": all read and write
// events are sorted by slot so each slot gets a time-ordered list; ramnet-ops
// "CUDA execution": events of the same (batch, head, slot) form a segment).
//
// A stable counting sort per (b, h), in three kernels:
//   hist     one block per (b, h, tile of `tile` tokens): slot histogram
//            of the tile's events in LDS;
//   scan     one workgroup per (b, h, block of SCAN_SLOTS slots): per slot,
//            exclusive prefix of the tile counts (in place), and the slot's
//            offset inside its block, which takes the place of tile 0's
//            entry (always 0); the block's event count goes to blk_tot.
//            Segments with more than LONG_EVENTS events are listed for the
//            cooperative scan path, in NBIN classes of doubling length (any
//            order inside a class), and segments with 1 to LONG_EVENTS
//            events in the short list (slot order inside a block, blocks
//            in any order).  Every (b, h) holds exactly
//            T*(k_w+k_r) events, so segment offsets need no scan across
//            (b, h);
//   scatter  one workgroup per (b, h, tile): its waves set up the tile's
//            per-slot write positions in LDS (the (b, h) base, the event
//            counts of the earlier blocks, the offset inside the block and
//            the tile prefix; the tile-0 workgroup also stores the segment
//            offsets).  The tile's events, in order (t ascending, write side
//            before read side), are ranked among equal slots inside each
//            64-event batch with ballots (all waves), given positions batch
//            after batch (one wave), and written as 16-byte records (code,
//            weight, retention lambda and d lambda / d w of a write) to their
//            final positions (all waves), so the scans read their events
//            with one coalesced load and gather nothing.
#include "common.hpp"
#include "kernels.hpp"

namespace ramk {

namespace {

__device__ __forceinline__ int event_slot(const BucketArgs& a, int b, int h, int t, int p) {
  const int64_t row = ((int64_t)b * a.T + t) * a.H + h;
  return (p < a.k_w) ? a.idx_w[row * a.k_w + p] : a.idx_r[row * a.k_r + (p - a.k_w)];
}

}  // namespace

__global__ __launch_bounds__(256) void bucket_hist_kernel(BucketArgs a) {
  extern __shared__ int hist[];
  const int tile = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int K = a.k_w + a.k_r;
  const int t_lo = tile * a.tile;
  const int t_hi = min(a.T, t_lo + a.tile);
  for (int s = threadIdx.x; s < a.S; s += blockDim.x) hist[s] = 0;
  if (tile == 0 && bh == 0 && threadIdx.x < LONG_WORDS) a.long_count[threadIdx.x] = 0;
  __syncthreads();
  const int n = (t_hi - t_lo) * K;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const int slot = event_slot(a, b, h, t_lo + e / K, e % K);
    if ((unsigned)slot < (unsigned)a.S) atomicAdd(&hist[slot], 1);
  }
  __syncthreads();
  int32_t* out = a.tile_hist + ((int64_t)bh * a.ntiles + tile) * a.S;
  for (int s = threadIdx.x; s < a.S; s += blockDim.x) out[s] = hist[s];
}

__global__ __launch_bounds__(SCAN_SLOTS) void bucket_scan_kernel(BucketArgs a) {
  static_assert(SCAN_SLOTS == 16 * WAVE, "one slot per thread, 16 waves");
  __shared__ int wave_tot[16], wave_short[16];
  __shared__ int cls_n[NBIN], cls_at[NBIN];   // long segments of the block per class
  __shared__ int short_at;                    // the block's place in the short list
  const int blk = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x;
  if (tid < NBIN) cls_n[tid] = 0;
  const int S = a.S;
  const int s = blk * SCAN_SLOTS + tid;
  int32_t* th = a.tile_hist + (int64_t)bh * a.ntiles * S;
  int cnt = 0;
  if (s < S) {
    // exclusive prefix over the tiles, in place; loads in groups of TG so
    // that a group costs one memory round trip
    constexpr int TG = 8;
    for (int t0 = 0; t0 < a.ntiles; t0 += TG) {
      int c[TG];
#pragma unroll
      for (int u = 0; u < TG; ++u)
        c[u] = (t0 + u < a.ntiles) ? th[(int64_t)(t0 + u) * S + s] : 0;
#pragma unroll
      for (int u = 0; u < TG; ++u) {
        if (t0 + u < a.ntiles) th[(int64_t)(t0 + u) * S + s] = cnt;
        cnt += c[u];
      }
    }
  }
  const int incl = wave_incl_scan(cnt);
  // segments with 1 to LONG_EVENTS events: listed for the short-segment
  // scans (slots without events need no scan), in slot order inside the
  // block, the block's share reserved with one global counter update
  const bool shrt = s < S && cnt > 0 && cnt <= LONG_EVENTS;
  const uint64_t sbal = __ballot(shrt);
  if (lane_id() == WAVE - 1) {
    wave_tot[tid / WAVE] = incl;
    wave_short[tid / WAVE] = __popcll(sbal);
  }
  __syncthreads();
  int before = 0, all = 0, s_before = 0, s_all = 0;
  for (int w = 0; w < 16; ++w) {
    const int wt = wave_tot[w], ws = wave_short[w];
    if (w < tid / WAVE) {
      before += wt;
      s_before += ws;
    }
    all += wt;
    s_all += ws;
  }
  // long segments: a place in the block's share of their class, then one
  // global counter update per class and block (hot slots make the global
  // counters contended)
  const bool lng = s < S && cnt > LONG_EVENTS;
  const int cls = lng ? min(NBIN - 1, 31 - __clz(cnt / (LONG_EVENTS + 1))) : 0;
  const int rank = lng ? atomicAdd(&cls_n[cls], 1) : 0;
  if (s < S) {
    if (a.ntiles > 0) th[s] = before + incl - cnt;   // offset inside the block
    else a.seg_offset[(int64_t)bh * S + s] = (int32_t)a.ev_base;   // no events at all
  }
  __syncthreads();
  if (tid < NBIN && cls_n[tid] > 0) cls_at[tid] = atomicAdd(&a.long_count[tid], cls_n[tid]);
  if (tid == NBIN && s_all > 0) short_at = atomicAdd(&a.long_count[SHORT_WORD], s_all);
  __syncthreads();
  if (lng) a.long_list[(int64_t)cls * a.long_cap + cls_at[cls] + rank] = (int32_t)((int64_t)bh * S + s);
  if (shrt)
    a.short_list[short_at + s_before + __popcll(sbal & lanemask_lt())] = (int32_t)((int64_t)bh * S + s);
  if (tid == 0) a.blk_tot[(int64_t)bh * a.nblk + blk] = all;
  if (blk == 0 && bh == a.B * a.H - 1 && tid == 0)
    a.seg_offset[(int64_t)a.B * a.H * S] =
        (int32_t)(a.ev_base + (int64_t)a.B * a.H * a.T * (a.k_w + a.k_r));
}

constexpr int SCATTER_THREADS = 256;
constexpr int SCATTER_CHUNK = 4096;   // events of a tile ranked per round (LDS)
constexpr int SCATTER_PER = SCATTER_CHUNK / SCATTER_THREADS;   // events per thread and round

// Slot of event e of a tile (-1 past the tile's events).
__device__ __forceinline__ int tile_event_slot(const BucketArgs& a, int b, int h, int t_lo, int K,
                                               int n, int e) {
  if (e >= n) return -1;
  const int t = t_lo + e / K, p = e % K;
  const int64_t row = ((int64_t)b * a.T + t) * a.H + h;
  return (p < a.k_w) ? a.idx_w[row * a.k_w + p] : a.idx_r[row * a.k_r + (p - a.k_w)];
}

// 16-byte record of event e (< n) of a tile.  A masked token keeps its
// events with weight 0, flagged by bit 31 of the code: an exact no-op write
// (retention 1, step 0) and a read that contributes 0, neither of which loads
// the token's rows.
template <typename IO>
__device__ __forceinline__ EventRec tile_event_rec(const BucketArgs& a, int b, int h, int t_lo,
                                                   int K, int e) {
  const int t = t_lo + e / K, p = e % K;
  const int64_t row = ((int64_t)b * a.T + t) * a.H + h;
  const bool live = !a.mask || a.mask[(int64_t)b * a.T + t];
  EventRec rec{0, 0.f, 1.f, 0.f};
  if (p < a.k_w) {
    rec.code = (t << 7) | p;
    rec.w = live ? a.w_w[row * a.k_w + p] : 0.f;
    if (live) rec.lam = retention(rec.w, to_f32(reinterpret_cast<const IO*>(a.gamma)[row]), &rec.dlam);
  } else {
    rec.code = (t << 7) | (1 << 6) | (p - a.k_w);
    rec.w = live ? a.w_r[row * a.k_r + (p - a.k_w)] : 0.f;
  }
  if (!live) rec.code = (int32_t)((uint32_t)rec.code | 0x80000000u);
  return rec;
}

// Per tile, in rounds of SCATTER_CHUNK events:
//   1. every wave ranks batches of 64 events: lanes with equal slots find
//      each other with one ballot per slot bit, giving each event its rank
//      among its batch's events of the same slot and their number;
//   2. one wave takes the batches in order and turns (slot, rank) into a
//      final position from the running per-slot counts in LDS;
//   3. every wave writes the records of its batches to their positions.
// Only step 2 is serial, and it is a few LDS operations per batch.
template <typename IO>
__global__ __launch_bounds__(SCATTER_THREADS) void bucket_scatter_kernel(BucketArgs a) {
  extern __shared__ int lds[];
  const int S = a.S;
  int* next = lds;                                        // S write positions
  uint32_t* ev = reinterpret_cast<uint32_t*>(lds + S);    // SCATTER_CHUNK per-event words
  const int tile = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int lane = lane_id();
  const int wave = threadIdx.x / WAVE;
  constexpr int NWAVES = SCATTER_THREADS / WAVE;
  const int32_t* th0 = a.tile_hist + (int64_t)bh * a.ntiles * S;   // offsets inside the blocks
  const int32_t* th = th0 + (int64_t)tile * S;                       // tile prefixes
  // event counts of the (at most 16) slot blocks, requested together
  static_assert(16 * SCAN_SLOTS >= 16384, "S <= 16384 has at most 16 blocks");
  int bt[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) bt[k] = k < a.nblk ? a.blk_tot[(int64_t)bh * a.nblk + k] : 0;
  // per block, each thread's SCAN_SLOTS / SCATTER_THREADS slots, their loads
  // requested together
  constexpr int SPT = SCAN_SLOTS / SCATTER_THREADS;
  static_assert(SPT * SCATTER_THREADS == SCAN_SLOTS, "whole slots per thread");
  int start = (int)(a.ev_base + (int64_t)bh * a.T * (a.k_w + a.k_r));   // of the block
#pragma unroll
  for (int blk = 0; blk < 16; ++blk) {
    if (blk < a.nblk) {
      int off[SPT], pre[SPT];
#pragma unroll
      for (int u = 0; u < SPT; ++u) {
        const int s = blk * SCAN_SLOTS + u * SCATTER_THREADS + (int)threadIdx.x;
        off[u] = s < S ? th0[s] : 0;
        pre[u] = (s < S && tile > 0) ? th[s] : 0;
      }
#pragma unroll
      for (int u = 0; u < SPT; ++u) {
        const int s = blk * SCAN_SLOTS + u * SCATTER_THREADS + (int)threadIdx.x;
        if (s < S) {
          const int seg = start + off[u];
          next[s] = seg + pre[u];
          if (tile == 0) a.seg_offset[(int64_t)bh * S + s] = seg;
        }
      }
    }
    start += bt[blk];
  }
  const int K = a.k_w + a.k_r;
  const int t_lo = tile * a.tile;
  const int t_hi = min(a.T, t_lo + a.tile);
  const int n = (t_hi - t_lo) * K;
  const uint64_t lt = lanemask_lt();
  constexpr uint32_t NONE = 0xFFFFFFFFu;
  for (int c0 = 0; c0 < n; c0 += SCATTER_CHUNK) {
    const int cn = min(SCATTER_CHUNK, n - c0);
    // 1. slot | rank << 14 | count << 21 of every event (slots < 2^14, ranks
    //    and counts <= 64); the wave's batches are e0 = (j * NWAVES + wave) *
    //    WAVE, their slots all requested before the first is ranked
    constexpr int NB = SCATTER_CHUNK / (NWAVES * WAVE);
    int sl[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
      sl[j] = tile_event_slot(a, b, h, t_lo, K, c0 + cn, c0 + (j * NWAVES + wave) * WAVE + lane);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int e0 = (j * NWAVES + wave) * WAVE;
      if (e0 < cn) {
        const int slot = sl[j];
        const bool valid = e0 + lane < cn && (unsigned)slot < (unsigned)S;
        uint64_t peers = __ballot(valid);
        for (int bit = 0; bit < a.nbits; ++bit) {
          const bool one = (slot >> bit) & 1;
          const uint64_t bal = __ballot(valid && one);
          peers &= one ? bal : ~bal;
        }
        const uint32_t rank = (uint32_t)__popcll(peers & lt);
        const uint32_t tot = (uint32_t)__popcll(peers);
        if (e0 + lane < cn) ev[e0 + lane] = valid ? ((uint32_t)slot | rank << 14 | tot << 21) : NONE;
      }
    }
    __syncthreads();   // (also orders the initial positions before the first round)
    // 2. positions, batch after batch
    if (wave == 0) {
      for (int e0 = 0; e0 < cn; e0 += WAVE) {
        const bool in = e0 + lane < cn;
        const uint32_t q = in ? ev[e0 + lane] : NONE;
        const bool valid = q != NONE;
        const int slot = (int)(q & 0x3FFFu);
        const int rank = (int)((q >> 14) & 0x7Fu), tot = (int)((q >> 21) & 0x7Fu);
        const int base = valid ? next[slot] : 0;
        wave_sync();
        if (valid && rank == 0) next[slot] = base + tot;
        wave_sync();
        if (in) ev[e0 + lane] = valid ? (uint32_t)(base + rank) : NONE;
      }
    }
    __syncthreads();
    // 3. records, in groups of REC_GROUP per thread whose inputs are all
    //    requested before the first record is formed
    constexpr int REC_GROUP = 8;
    static_assert(SCATTER_PER % REC_GROUP == 0, "whole groups");
    for (int j0 = 0; j0 < SCATTER_PER; j0 += REC_GROUP) {
      uint32_t pos[REC_GROUP];
      EventRec rec[REC_GROUP];
#pragma unroll
      for (int j = 0; j < REC_GROUP; ++j) {
        const int e = (j0 + j) * SCATTER_THREADS + (int)threadIdx.x;
        pos[j] = e < cn ? ev[e] : NONE;
        if (pos[j] != NONE) rec[j] = tile_event_rec<IO>(a, b, h, t_lo, K, c0 + e);
      }
#pragma unroll
      for (int j = 0; j < REC_GROUP; ++j)
        if (pos[j] != NONE) a.events[pos[j]] = rec[j];
    }
    __syncthreads();   // ev is rewritten by the next round
  }
}

hipError_t launch_bucket(const BucketArgs& a, bool bf16, hipStream_t st,
                         void (*before)(const char*, hipStream_t),
                         void (*after)(const char*, hipStream_t)) {
  const int BH = a.B * a.H;
  if (BH == 0) return hipSuccess;
  const size_t lds = (size_t)a.S * sizeof(int);
  if (a.ntiles > 0) {
    before("bucket_hist", st);
    hipLaunchKernelGGL(bucket_hist_kernel, dim3(a.ntiles, BH), dim3(256), lds, st, a);
    after("bucket_hist", st);
  }
  before("bucket_scan", st);
  hipLaunchKernelGGL(bucket_scan_kernel, dim3(a.nblk, BH), dim3(SCAN_SLOTS), 0, st, a);
  after("bucket_scan", st);
  if (a.ntiles > 0) {
    before("bucket_scatter", st);
    const dim3 grid(a.ntiles, BH), block(SCATTER_THREADS);
    const int64_t n = (int64_t)a.tile * (a.k_w + a.k_r);
    const size_t slds = lds + sizeof(uint32_t) * (size_t)(n < SCATTER_CHUNK ? n : SCATTER_CHUNK);
    if (bf16) hipLaunchKernelGGL(bucket_scatter_kernel<bf16_t>, grid, block, slds, st, a);
    else hipLaunchKernelGGL(bucket_scatter_kernel<float>, grid, block, slds, st, a);
    after("bucket_scatter", st);
  }
  return hipGetLastError();
}

}  // namespace ramk
