// C ABI of the RAM-Net attention core: validation, workspace layout and the
// launch sequence of each entry point.  See include/ramnet.h for the contract.
#include <algorithm>
#include <mutex>
#include <string.h>
#include <string>
#include <unordered_set>
#include <vector>

#include "../../include/ramnet.h"
#include "decode.hpp"
#include "decode_prod.hpp"
#include "kernels.hpp"

using namespace ramk;

namespace {

constexpr size_t ALIGN = 256;
size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

struct Dims {
  int64_t S, N, E, nseg, nck;
  int64_t row;   // logits per (token, head, side): U * P
  int tile, ntiles, nbits;
  size_t io_bytes;
};

int check_problem(const ram_problem* p, Dims* d) {
  if (!p) return RAM_EINVAL;
  if (p->io_dtype != RAM_F32 && p->io_dtype != RAM_BF16) return RAM_EDTYPE;
  if (p->reserved != 0) return RAM_EINVAL;
  if (p->B < 1 || p->H < 1 || p->T < 0 || p->P < 1 || p->U < 1) return RAM_EINVAL;
  if (p->cape_heads < 0 || p->cape_heads > p->H || p->t0 < 0) return RAM_EINVAL;
  if (p->U > MAX_DIGITS) return RAM_EUNSUPPORTED;
  int64_t S = 1;
  for (int u = 0; u < p->U; ++u) {
    S *= p->P;
    if (S > 16384) return RAM_EUNSUPPORTED;
  }
  const size_t io = p->io_dtype == RAM_F32 ? 4 : 2;
  // flat rows are read in 16-byte vectors
  if (p->U == 1 && (S * (int64_t)io) % 16 != 0) return RAM_EINVAL;
  if (p->k_w < 1 || p->k_r < 1 || p->k_w > 64 || p->k_r > 64 || p->k_w > S || p->k_r > S)
    return RAM_EINVAL;
  if (p->d_v < 1 || p->d_v > 128 || (p->d_v > 64 && (p->d_v % 2) != 0)) return RAM_EINVAL;
  if (!(p->eps >= 0.f) || p->eps > 3.0e38f) return RAM_EINVAL;
  if (p->renorm_w < 0 || p->renorm_w > 1 || p->renorm_r < 0 || p->renorm_r > 1) return RAM_EINVAL;
  if (p->T >= (1 << 24)) return RAM_ECAPACITY;
  const int64_t N = (int64_t)p->B * p->T * p->H;
  const int64_t E = N * (p->k_w + p->k_r);
  const int64_t nseg = (int64_t)p->B * p->H * S;
  if (E >= ((int64_t)1 << 31) || nseg >= ((int64_t)1 << 31) || N * p->d_v >= ((int64_t)1 << 40))
    return RAM_ECAPACITY;
  // the scans address one batch's rows of v, dO and the stash through
  // buffer resources of at most MAX_BUF_BYTES
  const int64_t kmax = p->k_w > p->k_r ? p->k_w : p->k_r;
  if ((int64_t)p->T * p->H * kmax * p->d_v * (int64_t)io > (int64_t)MAX_BUF_BYTES)
    return RAM_ECAPACITY;
  if (d) {
    d->S = S;
    d->row = (int64_t)p->U * p->P;
    d->N = N;
    d->E = E;
    d->nseg = nseg;
    d->nck = E / CHUNK + 1;
    // bucketing tiles of 256 tokens, or 128 when 256 would leave fewer than
    // 1024 scatter workgroups (measured: 1.3B layer 256, long-context chunk 128)
    d->tile = 256;
    if ((int64_t)p->B * p->H * ((p->T + 255) / 256) < 1024) d->tile = 128;
    d->ntiles = (p->T + d->tile - 1) / d->tile;
    int nb = 0;
    while ((1ll << nb) < S) ++nb;
    d->nbits = nb;
    d->io_bytes = io;
  }
  return RAM_OK;
}

// Workgroups of the bucketing scan per (b, h): blocks of SCAN_SLOTS slots.
int scan_blocks(int64_t S) { return (int)((S + SCAN_SLOTS - 1) / SCAN_SLOTS); }

// Entries per length class of the long-segment list: every long segment has
// more than LONG_EVENTS events.
int long_cap(const Dims& d) {
  const int64_t c = d.E / (LONG_EVENTS + 1) + 1;
  return (int)(c < d.nseg ? c : d.nseg);
}


void make_layout(const ram_problem* p, const Dims& d, ram_ws_layout* L) {
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  L->idx_w = take(sizeof(int32_t) * d.N * p->k_w);
  L->w_w = take(sizeof(float) * d.N * p->k_w);
  L->lse_w = take(sizeof(float) * d.N * p->U);
  L->idx_r = take(sizeof(int32_t) * d.N * p->k_r);
  L->w_r = take(sizeof(float) * d.N * p->k_r);
  L->lse_r = take(sizeof(float) * d.N * p->U);
  L->seg_offset = take(sizeof(int32_t) * (d.nseg + 1));
  L->events = take(sizeof(EventRec) * d.E);
  L->ckpt_s = take(sizeof(float) * d.nck * p->d_v);
  L->ckpt_m = take(sizeof(float) * d.nck);
  L->stash = take(d.io_bytes * d.N * p->k_r * p->d_v);
  // tile histograms, then the per-block event counts of the bucketing scan
  L->tile_hist = take(sizeof(int32_t) * (size_t)p->B * p->H *
                      ((size_t)d.ntiles * d.S + scan_blocks(d.S)));
  L->long_list = take(sizeof(int32_t) * NBIN * long_cap(d));
  L->long_count = take(sizeof(int32_t) * LONG_WORDS);
  L->short_list = take(sizeof(int32_t) * (d.E < d.nseg ? d.E : d.nseg));
  L->fwd_bytes = off;
  L->stash_b = take(d.io_bytes * d.N * p->k_w * p->d_v);
  L->dw = take(sizeof(float) * d.N * p->k_w);
  L->dr = take(sizeof(float) * d.N * p->k_r);
  L->dgam = take(sizeof(float) * d.N * p->k_w);
  L->epi_d_o = take(d.io_bytes * d.N * p->d_v);
  L->epi_part = take(sizeof(float) * EPI_BWD_WAVES * p->d_v);
  L->total_bytes = off;
}

bool aligned16(const void* q) { return ((uintptr_t)q & 15u) == 0; }

// ---- optional per-kernel timing -------------------------------------------
struct ProfRec { hipEvent_t a, b; int kind; };
std::mutex prof_mu;
bool prof_on = false;
std::vector<ProfRec> prof_recs;
std::vector<hipEvent_t> prof_pool;
size_t prof_used = 0;
std::vector<std::string> prof_names;

int prof_kind(const char* name) {
  for (size_t i = 0; i < prof_names.size(); ++i)
    if (prof_names[i] == name) return (int)i;
  prof_names.emplace_back(name);
  return (int)prof_names.size() - 1;
}

hipEvent_t prof_event() {
  if (prof_used == prof_pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    prof_pool.push_back(e);
  }
  return prof_pool[prof_used++];
}

void prof_before(const char* name, hipStream_t st) {
  if (!prof_on) return;
  std::lock_guard<std::mutex> lk(prof_mu);
  ProfRec r{prof_event(), nullptr, prof_kind(name)};
  if (r.a) (void)hipEventRecord(r.a, st);
  prof_recs.push_back(r);
}

void prof_after(const char*, hipStream_t st) {
  if (!prof_on) return;
  std::lock_guard<std::mutex> lk(prof_mu);
  if (prof_recs.empty()) return;
  ProfRec& r = prof_recs.back();
  r.b = prof_event();
  if (r.b) (void)hipEventRecord(r.b, st);
}

void prof_none(const char*, hipStream_t) {}

int hip_status(hipError_t e) { return e == hipSuccess ? RAM_OK : RAM_EHIP; }

// ---- library streams ---------------------------------------------------------
// The kernels of a call run on the caller's stream and on one library
// stream of the same device (default priority, non-blocking with respect to
// the null stream).  Every dependency goes through an event: the library
// streams first wait for everything already on the caller's stream (fork),
// and the caller's stream ends waiting for the library streams' work
// (join), so the call as a whole is ordered on the caller's stream.
constexpr int EV_POOL = 16;
struct Sched {
  hipStream_t side[1] = {nullptr};
  hipEvent_t ev[EV_POOL] = {};
  int used = 0;
  hipError_t err = hipSuccess;
  // `waiter` waits for all work enqueued on `signaler` so far.
  void dep(hipStream_t waiter, hipStream_t signaler) {
    if (err != hipSuccess || waiter == signaler) return;
    if (used == EV_POOL) { err = hipErrorOutOfMemory; return; }
    hipEvent_t e = ev[used++];
    err = hipEventRecord(e, signaler);
    if (err == hipSuccess) err = hipStreamWaitEvent(waiter, e, 0);
  }
};
std::mutex sched_mu;   // held for a whole call: one call uses the event pool at a time
std::vector<Sched> scheds;

hipError_t get_sched(Sched** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((int)scheds.size() <= dev) scheds.resize(dev + 1);
  Sched& S = scheds[dev];
  if (!S.ev[0]) {
    for (auto& ev : S.ev)
      if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) return e;
  }
  // the stream is created on first use only: it takes a hardware queue, and
  // a stream that shares its queue with the caller's serialises with it
  if (!S.side[0] && (e = hipStreamCreateWithFlags(&S.side[0], hipStreamNonBlocking)) != hipSuccess)
    return e;
  S.used = 0;
  S.err = hipSuccess;
  *out = &S;
  return hipSuccess;
}

// Byte offset helper: p advanced by n elements of `bytes` bytes.
template <typename T>
T* adv(T* q, int64_t n, size_t bytes) {
  return q ? (T*)((const char*)q + n * (int64_t)bytes) : nullptr;
}

}  // namespace

extern "C" {

const char* ram_status_string(int status) {
  switch (status) {
    case RAM_OK: return "ok";
    case RAM_EINVAL: return "invalid argument (shape, pointer, k, d_v, alignment)";
    case RAM_EDTYPE: return "unsupported io dtype";
    case RAM_ECAPACITY: return "capacity exceeded (events, tokens or workspace size)";
    case RAM_EUNSUPPORTED: return "unsupported configuration (S = P^U > 16384 or U > 14)";
    case RAM_EHIP: return "HIP runtime or launch error";
    default: return "unknown status";
  }
}

int ram_workspace_layout(const ram_problem* p, ram_ws_layout* out) {
  Dims d;
  const int st = check_problem(p, &d);
  if (st != RAM_OK) return st;
  if (!out) return RAM_EINVAL;
  make_layout(p, d, out);
  return RAM_OK;
}

int ram_workspace_size(const ram_problem* p, int with_backward, size_t* bytes) {
  ram_ws_layout L;
  const int st = ram_workspace_layout(p, &L);
  if (st != RAM_OK) return st;
  if (!bytes) return RAM_EINVAL;
  *bytes = with_backward ? L.total_bytes : L.fwd_bytes;
  return RAM_OK;
}

int ram_decode(const ram_problem* p, int side, const void* logits, int32_t* idx, float* weight,
               float* lse, void* stream) {
  Dims d;
  int st = check_problem(p, &d);
  if (st != RAM_OK) return st;
  if ((side != 0 && side != 1) || !logits || !idx || !weight || !lse || !aligned16(logits))
    return RAM_EINVAL;
  DecodeFwdArgs a{};
  a.logits[0] = logits;
  a.idx[0] = idx;
  a.w[0] = weight;
  a.lse[0] = lse;
  a.k[0] = side == 0 ? p->k_w : p->k_r;
  a.renorm[0] = side == 0 ? p->renorm_w : p->renorm_r;
  a.N = d.N;
  a.S = (int)d.S;
  a.U = p->U;
  a.P = p->P;
  a.nsides = 1;
  a.H = p->H;
  a.T = p->T;
  a.cape_heads = p->cape_heads;
  a.t0 = p->t0 % d.S;
  hipStream_t s = (hipStream_t)stream;
  prof_before("decode_fwd", s);
  hipError_t e = launch_decode_fwd(a, p->io_dtype == RAM_BF16, s);
  prof_after("decode_fwd", s);
  return hip_status(e);
}

}  // extern "C"

namespace {

bool epilogue_ok(const ram_epilogue* ep, int64_t N) {
  return ep && (N == 0 || ep->gate) && ep->eps >= 0.f && ep->eps <= 3.0e38f;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// In-place continuation (ramnet-ops "Arguments", inplace: no gradients): a
// forward whose final state overlaps its initial state overwrites what a
// backward would need.  The library keeps the workspace addresses whose last
// forward ran in place; ram_backward on such a workspace returns RAM_EINVAL
// before it enqueues anything.
std::mutex alias_mu;
std::unordered_set<uintptr_t> inplace_ws;

void note_forward(const void* ws, bool inplace) {
  std::lock_guard<std::mutex> lk(alias_mu);
  if (inplace) inplace_ws.insert((uintptr_t)ws);
  else inplace_ws.erase((uintptr_t)ws);
}

bool ran_in_place(const void* ws) {
  std::lock_guard<std::mutex> lk(alias_mu);
  return inplace_ws.count((uintptr_t)ws) != 0;
}

// ram_forward, or with ep the gated read-out y = sigmoid(gate) * RMSNorm(o)
// written to o.  one_stream: every kernel on the caller's stream, and no
// library stream, event or timing record is created or used.
int forward_impl(const ram_problem* p, const ram_epilogue* ep, const void* wlogits,
                 const void* rlogits, const void* v, const void* gamma, const uint8_t* mask,
                 const float* slot0, const float* mass0, void* o, float* slot1, float* mass1,
                 void* ws, size_t ws_bytes, void* stream, bool one_stream) {
  Dims d;
  int st = check_problem(p, &d);
  if (st != RAM_OK) return st;
  if (!slot1 || !mass1 || !ws) return RAM_EINVAL;
  if (ep && !epilogue_ok(ep, d.N)) return RAM_EINVAL;
  if (d.N > 0 && (!wlogits || !rlogits || !v || !gamma || !o)) return RAM_EINVAL;
  if ((slot0 == nullptr) != (mass0 == nullptr)) return RAM_EINVAL;
  if (d.N > 0 && (!aligned16(wlogits) || !aligned16(rlogits))) return RAM_EINVAL;
  ram_ws_layout L;
  make_layout(p, d, &L);
  if (ws_bytes < L.fwd_bytes) return RAM_ECAPACITY;
  const size_t sb = (size_t)d.nseg * p->d_v * sizeof(float), mb = (size_t)d.nseg * sizeof(float);
  note_forward(ws, overlaps(slot1, sb, slot0, sb) || overlaps(mass1, mb, mass0, mb) ||
                       overlaps(slot1, sb, mass0, mb) || overlaps(mass1, mb, slot0, sb));
  char* w = (char*)ws;
  hipStream_t s = (hipStream_t)stream;
  const bool bf = p->io_dtype == RAM_BF16;
  const int cap = long_cap(d);

  void (*before)(const char*, hipStream_t) = one_stream ? prof_none : prof_before;
  void (*after)(const char*, hipStream_t) = one_stream ? prof_none : prof_after;
  std::lock_guard<std::mutex> lk(sched_mu);
  Sched local;
  Sched* S = &local;
  if (!one_stream && get_sched(&S) != hipSuccess) return RAM_EHIP;
  // the short-segment scans run beside the long-segment ones on a library
  // stream; everything else on the caller's stream
  hipStream_t b = one_stream ? s : S->side[0];
  hipError_t e = hipSuccess;

  DecodeFwdArgs da{};
  da.logits[0] = wlogits;
  da.logits[1] = rlogits;
  da.idx[0] = (int32_t*)(w + L.idx_w);
  da.idx[1] = (int32_t*)(w + L.idx_r);
  da.w[0] = (float*)(w + L.w_w);
  da.w[1] = (float*)(w + L.w_r);
  da.lse[0] = (float*)(w + L.lse_w);
  da.lse[1] = (float*)(w + L.lse_r);
  da.k[0] = p->k_w;
  da.k[1] = p->k_r;
  da.renorm[0] = p->renorm_w;
  da.renorm[1] = p->renorm_r;
  da.N = d.N;
  da.S = (int)d.S;
  da.U = p->U;
  da.P = p->P;
  da.nsides = 2;
  da.H = p->H;
  da.T = p->T;
  da.cape_heads = p->cape_heads;
  da.t0 = p->t0 % d.S;
  before("decode_fwd", s);
  e = launch_decode_fwd(da, bf, s);
  after("decode_fwd", s);
  if (e != hipSuccess) return RAM_EHIP;

  BucketArgs ba{};
  ba.idx_w = da.idx[0];
  ba.idx_r = da.idx[1];
  ba.w_w = da.w[0];
  ba.w_r = da.w[1];
  ba.gamma = gamma;
  ba.mask = mask;
  ba.B = p->B;
  ba.H = p->H;
  ba.T = p->T;
  ba.S = (int)d.S;
  ba.k_w = p->k_w;
  ba.k_r = p->k_r;
  ba.tile = d.tile;
  ba.ntiles = d.ntiles;
  ba.nbits = d.nbits;
  ba.tile_hist = (int32_t*)(w + L.tile_hist);
  ba.nblk = scan_blocks(d.S);
  ba.blk_tot = (int32_t*)(w + L.tile_hist) + (int64_t)p->B * p->H * d.ntiles * d.S;
  ba.seg_offset = (int32_t*)(w + L.seg_offset);
  ba.ev_base = 0;
  ba.events = (EventRec*)(w + L.events);
  ba.long_list = (int32_t*)(w + L.long_list);
  ba.long_count = (int32_t*)(w + L.long_count);
  ba.long_cap = cap;
  ba.short_list = (int32_t*)(w + L.short_list);
  e = launch_bucket(ba, bf, s, before, after);
  if (e != hipSuccess) return RAM_EHIP;

  ScanFwdArgs sa{};
  sa.B = p->B;
  sa.H = p->H;
  sa.T = p->T;
  sa.S = (int)d.S;
  sa.d_v = p->d_v;
  sa.k_w = p->k_w;
  sa.k_r = p->k_r;
  sa.eps = p->eps;
  sa.nseg = d.nseg;
  sa.long_list = ba.long_list;
  sa.long_count = ba.long_count;
  sa.queue = ba.long_count + NBIN;
  sa.long_cap = cap;
  sa.use_long = d.ntiles > 0;
  sa.short_list = ba.short_list;
  sa.short_count = ba.long_count + SHORT_WORD;
  sa.seg_offset = ba.seg_offset;
  sa.events = ba.events;
  sa.v = v;
  sa.slot0 = slot0;
  sa.mass0 = mass0;
  sa.slot1 = slot1;
  sa.mass1 = mass1;
  sa.stash = w + L.stash;
  sa.ckpt_s = (float*)(w + L.ckpt_s);
  sa.ckpt_m = (float*)(w + L.ckpt_m);
  // The short-segment stream forks off just before the launch and joins
  // right after it; the timing events bracket the fork and the join (an
  // event recorded between the launch and the join slows the scans down).
  before("scan_fwd", s);
  S->dep(b, s);
  e = launch_scan_fwd(sa, bf, s, b);
  S->dep(s, b);
  after("scan_fwd", s);
  if (e != hipSuccess || S->err != hipSuccess) return RAM_EHIP;

  if (ep) {
    EpilogueArgs ea{};
    ea.N = d.N;
    ea.d_v = p->d_v;
    ea.k = p->k_r;
    ea.T = p->T;
    ea.H = p->H;
    ea.stash = sa.stash;
    ea.gate = ep->gate;
    ea.gain = ep->gain;
    ea.eps = ep->eps;
    ea.y = o;
    before("epilogue_fwd", s);
    e = launch_epilogue_fwd(ea, bf, s);
    after("epilogue_fwd", s);
  } else {
    FinalizeArgs fa{};
    fa.N = d.N;
    fa.d_v = p->d_v;
    fa.k = p->k_r;
    fa.stash = sa.stash;
    fa.out = o;
    before("finalize_o", s);
    e = launch_finalize(fa, bf, s);
    after("finalize_o", s);
  }
  return e == hipSuccess ? RAM_OK : RAM_EHIP;
}

// ram_backward, or with ep the backward of the gated read-out: d_o is then
// the gradient of y, and d_gate / d_gain receive the epilogue's gradients.
// The reverse scan runs its long-segment kernel on the caller's stream and
// its short-segment kernel beside it on a library stream; the decode
// backward of both sides and the d_v / d_gamma sums follow.
int backward_impl(const ram_problem* p, const ram_epilogue* ep, void* ws, size_t ws_bytes,
                  const void* wlogits, const void* rlogits, const void* v, const void* gamma,
                  const uint8_t* mask, const float* slot0, const float* mass0, const void* d_o,
                  const float* d_slot1, const float* d_mass1, void* d_wlogits, void* d_rlogits,
                  void* d_v, void* d_gamma, void* d_gate, float* d_gain, float* d_slot0,
                  float* d_mass0, void* stream) {
  Dims d;
  int st = check_problem(p, &d);
  if (st != RAM_OK) return st;
  if (!ws) return RAM_EINVAL;
  if (ep && (!epilogue_ok(ep, d.N) || (d.N > 0 && !d_gate))) return RAM_EINVAL;
  if (d.N > 0 && (!wlogits || !rlogits || !v || !gamma || !d_o || !d_wlogits || !d_rlogits ||
                  !d_v || !d_gamma))
    return RAM_EINVAL;
  if ((slot0 == nullptr) != (mass0 == nullptr)) return RAM_EINVAL;
  if (d.N > 0 && (!aligned16(wlogits) || !aligned16(rlogits) || !aligned16(d_wlogits) ||
                  !aligned16(d_rlogits)))
    return RAM_EINVAL;
  ram_ws_layout L;
  make_layout(p, d, &L);
  if (ws_bytes < L.total_bytes) return RAM_ECAPACITY;
  if (ran_in_place(ws)) return RAM_EINVAL;
  char* w = (char*)ws;
  hipStream_t s = (hipStream_t)stream;
  const bool bf = p->io_dtype == RAM_BF16;
  const int cap = long_cap(d);
  (void)gamma;   // the event records carry lambda and d lambda / d w

  std::lock_guard<std::mutex> lk(sched_mu);
  Sched* S = nullptr;
  if (get_sched(&S) != hipSuccess) return RAM_EHIP;
  hipStream_t b = S->side[0];
  hipError_t e = hipSuccess;
  const void* dO = d_o;
  if (ep) {
    // gradient of o from that of y; o is recomputed from the forward's read
    // contributions, which the backward never overwrites
    EpilogueArgs ea{};
    ea.N = d.N;
    ea.d_v = p->d_v;
    ea.k = p->k_r;
    ea.T = p->T;
    ea.H = p->H;
    ea.stash = w + L.stash;
    ea.gate = ep->gate;
    ea.gain = ep->gain;
    ea.eps = ep->eps;
    ea.d_y = d_o;
    ea.d_o = w + L.epi_d_o;
    ea.d_gate = d_gate;
    ea.part = (float*)(w + L.epi_part);
    ea.d_gain = d_gain;
    ea.mask = mask;
    prof_before("epilogue_bwd", s);
    e = launch_epilogue_bwd(ea, bf, s);
    prof_after("epilogue_bwd", s);
    if (e != hipSuccess) return RAM_EHIP;
    dO = w + L.epi_d_o;
  }

  ScanBwdArgs sb{};
  sb.B = p->B;
  sb.H = p->H;
  sb.T = p->T;
  sb.S = (int)d.S;
  sb.d_v = p->d_v;
  sb.k_w = p->k_w;
  sb.k_r = p->k_r;
  sb.eps = p->eps;
  sb.nseg = d.nseg;
  sb.long_list = (const int32_t*)(w + L.long_list);
  sb.long_count = (const int32_t*)(w + L.long_count);
  sb.queue = (int32_t*)(w + L.long_count) + NBIN + 2;
  sb.long_cap = cap;
  sb.use_long = d.ntiles > 0;
  sb.short_list = (const int32_t*)(w + L.short_list);
  sb.short_count = (const int32_t*)(w + L.long_count) + SHORT_WORD;
  sb.seg_offset = (const int32_t*)(w + L.seg_offset);
  sb.events = (const EventRec*)(w + L.events);
  sb.v = v;
  sb.d_o = dO;
  sb.slot0 = slot0;
  sb.mass0 = mass0;
  sb.ckpt_s = (const float*)(w + L.ckpt_s);
  sb.ckpt_m = (const float*)(w + L.ckpt_m);
  sb.d_slot1 = d_slot1;
  sb.d_mass1 = d_mass1;
  sb.d_slot0 = d_slot0;
  sb.d_mass0 = d_mass0;
  sb.stash = w + L.stash_b;
  sb.dw = (float*)(w + L.dw);
  sb.dr = (float*)(w + L.dr);
  sb.dgam = (float*)(w + L.dgam);
  prof_before("scan_bwd", s);
  S->dep(b, s);
  e = launch_scan_bwd(sb, bf, s, b);
  S->dep(s, b);
  prof_after("scan_bwd", s);
  if (e != hipSuccess || S->err != hipSuccess) return RAM_EHIP;

  DecodeBwdArgs db{};
  db.logits[0] = wlogits;
  db.logits[1] = rlogits;
  db.lse[0] = (const float*)(w + L.lse_w);
  db.lse[1] = (const float*)(w + L.lse_r);
  db.idx[0] = (const int32_t*)(w + L.idx_w);
  db.idx[1] = (const int32_t*)(w + L.idx_r);
  db.w[0] = (const float*)(w + L.w_w);
  db.w[1] = (const float*)(w + L.w_r);
  db.g[0] = sb.dw;
  db.g[1] = sb.dr;
  db.dlogits[0] = d_wlogits;
  db.dlogits[1] = d_rlogits;
  db.k[0] = p->k_w;
  db.k[1] = p->k_r;
  db.renorm[0] = p->renorm_w;
  db.renorm[1] = p->renorm_r;
  db.N = d.N;
  db.S = (int)d.S;
  db.U = p->U;
  db.P = p->P;
  db.nsides = 2;
  db.H = p->H;
  db.T = p->T;
  db.cape_heads = p->cape_heads;
  db.t0 = p->t0 % d.S;
  db.mask = mask;
  prof_before("decode_bwd", s);
  e = launch_decode_bwd(db, bf, s);
  prof_after("decode_bwd", s);
  if (e != hipSuccess) return RAM_EHIP;

  FinalizeArgs fa{};
  fa.N = d.N;
  fa.d_v = p->d_v;
  fa.k = p->k_w;
  fa.stash = sb.stash;
  fa.out = d_v;
  fa.dgam = sb.dgam;
  fa.d_gamma = d_gamma;
  prof_before("finalize_bwd", s);
  e = launch_finalize(fa, bf, s);
  prof_after("finalize_bwd", s);
  return e == hipSuccess ? RAM_OK : RAM_EHIP;
}

// ---- allocation-free forward -------------------------------------------------
// The workspace of ram_forward_noalloc: one array per device in the library's
// code object (allocated when the library is loaded on a device, held until
// the process ends).  Host code never uses the array's name as an address:
// its device address comes from hipGetSymbolAddress, once per device, with
// that device current.
static __device__ __align__(256) unsigned char scratch[RAM_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES] = {};

hipError_t device_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int ram_forward_noalloc(const ram_problem* p, const void* wlogits, const void* rlogits,
                        const void* v, const void* gamma, const uint8_t* mask, const float* slot0,
                        const float* mass0, void* o, float* slot1, float* mass1, void* stream) {
  Dims d;
  const int st = check_problem(p, &d);
  if (st != RAM_OK) return st;
  ram_ws_layout L;
  make_layout(p, d, &L);
  if (L.fwd_bytes > RAM_NOALLOC_SCRATCH_BYTES) return RAM_ECAPACITY;
  void* ws = nullptr;
  if (device_scratch(&ws) != hipSuccess) return RAM_EHIP;
  return forward_impl(p, nullptr, wlogits, rlogits, v, gamma, mask, slot0, mass0, o, slot1, mass1,
                      ws, RAM_NOALLOC_SCRATCH_BYTES, stream, true);
}

int ram_forward(const ram_problem* p, const void* wlogits, const void* rlogits, const void* v,
                const void* gamma, const uint8_t* mask, const float* slot0, const float* mass0,
                void* o, float* slot1, float* mass1, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(p, nullptr, wlogits, rlogits, v, gamma, mask, slot0, mass0, o, slot1, mass1,
                      ws, ws_bytes, stream, false);
}

int ram_forward_gated(const ram_problem* p, const ram_epilogue* ep, const void* wlogits,
                      const void* rlogits, const void* v, const void* gamma, const uint8_t* mask,
                      const float* slot0, const float* mass0, void* y, float* slot1, float* mass1,
                      void* ws, size_t ws_bytes, void* stream) {
  if (!ep) return RAM_EINVAL;
  return forward_impl(p, ep, wlogits, rlogits, v, gamma, mask, slot0, mass0, y, slot1, mass1, ws,
                      ws_bytes, stream, false);
}

int ram_backward(const ram_problem* p, void* ws, size_t ws_bytes, const void* wlogits,
                 const void* rlogits, const void* v, const void* gamma, const uint8_t* mask,
                 const float* slot0, const float* mass0, const void* d_o, const float* d_slot1,
                 const float* d_mass1, void* d_wlogits, void* d_rlogits, void* d_v, void* d_gamma,
                 float* d_slot0, float* d_mass0, void* stream) {
  return backward_impl(p, nullptr, ws, ws_bytes, wlogits, rlogits, v, gamma, mask, slot0, mass0,
                       d_o, d_slot1, d_mass1, d_wlogits, d_rlogits, d_v, d_gamma, nullptr, nullptr,
                       d_slot0, d_mass0, stream);
}

int ram_backward_gated(const ram_problem* p, const ram_epilogue* ep, void* ws, size_t ws_bytes,
                       const void* wlogits, const void* rlogits, const void* v, const void* gamma,
                       const uint8_t* mask, const float* slot0, const float* mass0,
                       const void* d_y, const float* d_slot1, const float* d_mass1,
                       void* d_wlogits, void* d_rlogits, void* d_v, void* d_gamma, void* d_gate,
                       float* d_gain, float* d_slot0, float* d_mass0, void* stream) {
  if (!ep) return RAM_EINVAL;
  return backward_impl(p, ep, ws, ws_bytes, wlogits, rlogits, v, gamma, mask, slot0, mass0, d_y,
                       d_slot1, d_mass1, d_wlogits, d_rlogits, d_v, d_gamma, d_gate, d_gain,
                       d_slot0, d_mass0, stream);
}

int ram_decode_step(const ram_problem* p, const void* wlogits, const void* rlogits, const void* v,
                    const void* gamma, const uint8_t* mask, float* slot, float* mass, void* o,
                    void* stream) {
  Dims d;
  int st = check_problem(p, &d);
  if (st != RAM_OK) return st;
  if (p->T != 1) return RAM_EINVAL;
  if ((int64_t)p->k_w * p->d_v > 8192) return RAM_EUNSUPPORTED;
  if (!wlogits || !rlogits || !v || !gamma || !slot || !mass || !o) return RAM_EINVAL;
  if (!aligned16(wlogits) || !aligned16(rlogits)) return RAM_EINVAL;
  StepArgs a{};
  a.B = p->B;
  a.H = p->H;
  a.S = (int)d.S;
  a.U = p->U;
  a.P = p->P;
  a.d_v = p->d_v;
  a.k_w = p->k_w;
  a.k_r = p->k_r;
  a.renorm_w = p->renorm_w;
  a.renorm_r = p->renorm_r;
  a.cape_heads = p->cape_heads;
  a.t0 = p->t0 % d.S;
  a.mask = mask;
  a.eps = p->eps;
  a.wl = wlogits;
  a.rl = rlogits;
  a.v = v;
  a.gamma = gamma;
  a.slot = slot;
  a.mass = mass;
  a.o = o;
  hipStream_t s = (hipStream_t)stream;
  prof_before("decode_step", s);
  hipError_t e = launch_step(a, p->io_dtype == RAM_BF16, s);
  prof_after("decode_step", s);
  return hip_status(e);
}

int ram_prof_enable(int on) {
  std::lock_guard<std::mutex> lk(prof_mu);
  prof_recs.clear();
  prof_used = 0;
  prof_on = on != 0;
  return RAM_OK;
}

int ram_prof_collect(ram_prof_entry* out, int max_entries, int* n_entries) {
  std::lock_guard<std::mutex> lk(prof_mu);
  std::vector<double> ms(prof_names.size(), 0.0);
  std::vector<int64_t> cnt(prof_names.size(), 0);
  for (const ProfRec& r : prof_recs) {
    if (!r.a || !r.b) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return RAM_EHIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return RAM_EHIP;
    ms[r.kind] += t;
    cnt[r.kind] += 1;
  }
  int n = 0;
  for (size_t i = 0; i < prof_names.size() && n < max_entries; ++i) {
    if (cnt[i] == 0) continue;
    if (out) {
      strncpy(out[n].name, prof_names[i].c_str(), sizeof(out[n].name) - 1);
      out[n].name[sizeof(out[n].name) - 1] = 0;
      out[n].launches = cnt[i];
      out[n].total_ms = ms[i];
    }
    ++n;
  }
  if (n_entries) *n_entries = n;
  return RAM_OK;
}

}  // extern "C"
