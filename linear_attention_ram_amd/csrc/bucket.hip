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
//            order inside a class).  Every (b, h) holds exactly
//            T*(k_w+k_r) events, so segment offsets need no scan across
//            (b, h);
//   scatter  one workgroup per (b, h, tile): all its waves set up the
//            tile's per-slot write positions in LDS (the (b, h) base, the
//            event counts of the earlier blocks, the offset inside the
//            block and the tile prefix; the tile-0 workgroup also stores the
//            segment offsets), then one wave walks the tile's events in order
//            (t ascending, write side before read side), ranks equal slots
//            inside each 64-event batch with ballots, and writes each event
//            as a 16-byte record (code, weight, retention lambda and
//            d lambda / d w of a write) to its final position, so the scans
//            read their events with one coalesced load and gather nothing.
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
  __shared__ int wave_tot[16];
  __shared__ int cls_n[NBIN], cls_at[NBIN];   // long segments of the block per class
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
  if (lane_id() == WAVE - 1) wave_tot[tid / WAVE] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < 16; ++w) {
    const int wt = wave_tot[w];
    if (w < tid / WAVE) before += wt;
    all += wt;
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
  __syncthreads();
  if (lng) a.long_list[(int64_t)cls * a.long_cap + cls_at[cls] + rank] = (int32_t)((int64_t)bh * S + s);
  if (tid == 0) a.blk_tot[(int64_t)bh * a.nblk + blk] = all;
  if (blk == 0 && bh == a.B * a.H - 1 && tid == 0)
    a.seg_offset[(int64_t)a.B * a.H * S] =
        (int32_t)(a.ev_base + (int64_t)a.B * a.H * a.T * (a.k_w + a.k_r));
}

constexpr int SCATTER_THREADS = 256;

template <typename IO>
__global__ __launch_bounds__(SCATTER_THREADS) void bucket_scatter_kernel(BucketArgs a) {
  extern __shared__ int next[];   // S write positions
  const int tile = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.H, h = bh % a.H;
  const int lane = lane_id();
  const int S = a.S;
  const int32_t* th0 = a.tile_hist + (int64_t)bh * a.ntiles * S;   // offsets inside the blocks
  const int32_t* th = th0 + (int64_t)tile * S;                       // tile prefixes
  const IO* gam = reinterpret_cast<const IO*>(a.gamma);
  int start = (int)(a.ev_base + (int64_t)bh * a.T * (a.k_w + a.k_r));   // of the block
  for (int blk = 0; blk < a.nblk; ++blk) {
    const int s1 = min(S, (blk + 1) * SCAN_SLOTS);
    for (int s = blk * SCAN_SLOTS + (int)threadIdx.x; s < s1; s += SCATTER_THREADS) {
      const int seg = start + th0[s];
      next[s] = seg + (tile > 0 ? th[s] : 0);
      if (tile == 0) a.seg_offset[(int64_t)bh * S + s] = seg;
    }
    start += a.blk_tot[(int64_t)bh * a.nblk + blk];
  }
  __syncthreads();
  if (threadIdx.x >= WAVE) return;   // the ranking below is one wave's walk
  const int K = a.k_w + a.k_r;
  const int t_lo = tile * a.tile;
  const int t_hi = min(a.T, t_lo + a.tile);
  const int n = (t_hi - t_lo) * K;
  const uint64_t lt = lanemask_lt();
  for (int e0 = 0; e0 < n; e0 += WAVE) {
    const int e = e0 + lane;
    bool valid = e < n;
    int slot = 0;
    EventRec rec{0, 0.f, 1.f, 0.f};
    if (valid) {
      const int t = t_lo + e / K, p = e % K;
      const int64_t row = ((int64_t)b * a.T + t) * a.H + h;
      // a masked token keeps its events with weight 0: an exact no-op write
      // (retention 1, step 0) and a read that contributes 0
      const bool live = !a.mask || a.mask[(int64_t)b * a.T + t];
      if (p < a.k_w) {
        slot = a.idx_w[row * a.k_w + p];
        rec.code = (t << 7) | p;
        rec.w = live ? a.w_w[row * a.k_w + p] : 0.f;
        rec.lam = live ? retention(rec.w, to_f32(gam[row]), &rec.dlam) : 1.f;
        if (!live) rec.dlam = 0.f;
      } else {
        slot = a.idx_r[row * a.k_r + (p - a.k_w)];
        rec.code = (t << 7) | (1 << 6) | (p - a.k_w);
        rec.w = live ? a.w_r[row * a.k_r + (p - a.k_w)] : 0.f;
      }
      valid = (unsigned)slot < (unsigned)S;   // decoded slots are always < S
    }
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < a.nbits; ++bit) {
      const bool one = (slot >> bit) & 1;
      const uint64_t bal = __ballot(valid && one);
      peers &= one ? bal : ~bal;
    }
    const int rank = __popcll(peers & lt);
    const int tot = __popcll(peers);
    const int base = valid ? next[slot] : 0;
    wave_sync();
    if (valid && rank == 0) next[slot] = base + tot;
    wave_sync();
    if (valid) a.events[base + rank] = rec;
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
    if (bf16) hipLaunchKernelGGL(bucket_scatter_kernel<bf16_t>, grid, block, lds, st, a);
    else hipLaunchKernelGGL(bucket_scatter_kernel<float>, grid, block, lds, st, a);
    after("bucket_scatter", st);
  }
  return hipGetLastError();
}

}  // namespace ramk
