// C ABI of the RAM-Net attention core: validation, workspace layout and the
// launch sequence of each entry point.  See include/ramnet.h for the contract.
#include <mutex>
#include <string.h>
#include <string>
#include <vector>

#include "../../include/ramnet.h"
#include "decode.hpp"
#include "kernels.hpp"

using namespace ramk;

namespace {

constexpr size_t ALIGN = 256;
size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

struct Dims {
  int64_t S, N, E, nseg, nck;
  int ntiles, nbits;
  size_t io_bytes;
};

int check_problem(const ram_problem* p, Dims* d) {
  if (!p) return RAM_EINVAL;
  if (p->io_dtype != RAM_F32 && p->io_dtype != RAM_BF16) return RAM_EDTYPE;
  if (p->cape_heads != 0) return RAM_EUNSUPPORTED;
  if (p->U != 1) return RAM_EUNSUPPORTED;
  if (p->reserved != 0) return RAM_EINVAL;
  if (p->B < 1 || p->H < 1 || p->T < 0 || p->P < 1) return RAM_EINVAL;
  const int64_t S = p->P;
  if (S > 16384) return RAM_EUNSUPPORTED;
  const size_t io = p->io_dtype == RAM_F32 ? 4 : 2;
  if ((S * (int64_t)io) % 16 != 0) return RAM_EINVAL;
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
    d->N = N;
    d->E = E;
    d->nseg = nseg;
    d->nck = E / CHUNK + 1;
    d->ntiles = (p->T + TILE_TOKENS - 1) / TILE_TOKENS;
    int nb = 0;
    while ((1ll << nb) < S) ++nb;
    d->nbits = nb;
    d->io_bytes = io;
  }
  return RAM_OK;
}

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
  L->lse_w = take(sizeof(float) * d.N);
  L->idx_r = take(sizeof(int32_t) * d.N * p->k_r);
  L->w_r = take(sizeof(float) * d.N * p->k_r);
  L->lse_r = take(sizeof(float) * d.N);
  L->seg_offset = take(sizeof(int32_t) * (d.nseg + 1));
  L->events = take(sizeof(EventRec) * d.E);
  L->ckpt_s = take(sizeof(float) * d.nck * p->d_v);
  L->ckpt_m = take(sizeof(float) * d.nck);
  L->stash = take(d.io_bytes * d.N * (p->k_w > p->k_r ? p->k_w : p->k_r) * p->d_v);
  L->tile_hist = take(sizeof(int32_t) * (size_t)p->B * p->H * d.ntiles * d.S);
  L->long_list = take(sizeof(int32_t) * NBIN * long_cap(d));
  L->long_count = take(sizeof(int32_t) * NBIN);
  L->fwd_bytes = off;
  L->dw = take(sizeof(float) * d.N * p->k_w);
  L->dr = take(sizeof(float) * d.N * p->k_r);
  L->dgam = take(sizeof(float) * d.N * p->k_w);
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

int hip_status(hipError_t e) { return e == hipSuccess ? RAM_OK : RAM_EHIP; }

// ---- a second stream per device ---------------------------------------------
// Independent kernels of one call (the short- and the long-segment scans) run
// on the caller's stream and on a library stream at the same time.  The
// library stream waits for everything enqueued on the caller's stream before
// the call (fork event), and the caller's stream waits for the library
// stream's part (join event), so the call stays ordered on the caller's
// stream.  Default priority; non-blocking with respect to the null stream.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex side_mu;
std::vector<SideStream> side_streams;

// Runs launch(main, side) between a fork and a join.  Holds side_mu so the
// pair of events is not shared by two calls at once.
template <typename F>
hipError_t forked(hipStream_t st, F&& launch) {
  std::lock_guard<std::mutex> lk(side_mu);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((int)side_streams.size() <= dev) side_streams.resize(dev + 1);
  SideStream& ss = side_streams[dev];
  if (!ss.s) {
    if ((e = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming)) != hipSuccess) return e;
  }
  if ((e = hipEventRecord(ss.fork, st)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(ss.s, ss.fork, 0)) != hipSuccess) return e;
  const hipError_t le = launch(st, ss.s);
  if ((e = hipEventRecord(ss.join, ss.s)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(st, ss.join, 0)) != hipSuccess) return e;
  return le;
}

}  // namespace

extern "C" {

const char* ram_status_string(int status) {
  switch (status) {
    case RAM_OK: return "ok";
    case RAM_EINVAL: return "invalid argument (shape, pointer, k, d_v, alignment)";
    case RAM_EDTYPE: return "unsupported io dtype";
    case RAM_ECAPACITY: return "capacity exceeded (events, tokens or workspace size)";
    case RAM_EUNSUPPORTED: return "unsupported configuration (U > 1, CAPE or S > 16384)";
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
  a.nsides = 1;
  hipStream_t s = (hipStream_t)stream;
  prof_before("decode_fwd", s);
  hipError_t e = launch_decode_fwd(a, p->io_dtype == RAM_BF16, s);
  prof_after("decode_fwd", s);
  return hip_status(e);
}

int ram_forward(const ram_problem* p, const void* wlogits, const void* rlogits, const void* v,
                const void* gamma, const float* slot0, const float* mass0, void* o, float* slot1,
                float* mass1, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int st = check_problem(p, &d);
  if (st != RAM_OK) return st;
  if (!slot1 || !mass1 || !ws) return RAM_EINVAL;
  if (d.N > 0 && (!wlogits || !rlogits || !v || !gamma || !o)) return RAM_EINVAL;
  if ((slot0 == nullptr) != (mass0 == nullptr)) return RAM_EINVAL;
  if (d.N > 0 && (!aligned16(wlogits) || !aligned16(rlogits))) return RAM_EINVAL;
  ram_ws_layout L;
  make_layout(p, d, &L);
  if (ws_bytes < L.fwd_bytes) return RAM_ECAPACITY;
  char* w = (char*)ws;
  hipStream_t s = (hipStream_t)stream;
  const bool bf = p->io_dtype == RAM_BF16;
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
  da.nsides = 2;
  prof_before("decode_fwd", s);
  e = launch_decode_fwd(da, bf, s);
  prof_after("decode_fwd", s);
  if (e != hipSuccess) return RAM_EHIP;

  BucketArgs ba{};
  ba.idx_w = da.idx[0];
  ba.idx_r = da.idx[1];
  ba.w_w = da.w[0];
  ba.w_r = da.w[1];
  ba.gamma = gamma;
  ba.B = p->B;
  ba.H = p->H;
  ba.T = p->T;
  ba.S = (int)d.S;
  ba.k_w = p->k_w;
  ba.k_r = p->k_r;
  ba.ntiles = d.ntiles;
  ba.nbits = d.nbits;
  ba.tile_hist = (int32_t*)(w + L.tile_hist);
  ba.seg_offset = (int32_t*)(w + L.seg_offset);
  ba.events = (EventRec*)(w + L.events);
  ba.long_list = (int32_t*)(w + L.long_list);
  ba.long_count = (int32_t*)(w + L.long_count);
  ba.long_cap = long_cap(d);
  e = launch_bucket(ba, bf, s, prof_before, prof_after);
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
  sa.long_cap = ba.long_cap;
  sa.use_long = d.ntiles > 0;
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
  prof_before("scan_fwd", s);
  e = forked(s, [&](hipStream_t m, hipStream_t x) { return launch_scan_fwd(sa, bf, m, x); });
  prof_after("scan_fwd", s);
  if (e != hipSuccess) return RAM_EHIP;

  FinalizeArgs fa{};
  fa.N = d.N;
  fa.d_v = p->d_v;
  fa.k = p->k_r;
  fa.stash = sa.stash;
  fa.out = o;
  prof_before("finalize_o", s);
  e = launch_finalize(fa, bf, s);
  prof_after("finalize_o", s);
  return hip_status(e);
}

int ram_backward(const ram_problem* p, void* ws, size_t ws_bytes, const void* wlogits,
                 const void* rlogits, const void* v, const void* gamma, const float* slot0,
                 const float* mass0, const void* d_o, const float* d_slot1, const float* d_mass1,
                 void* d_wlogits, void* d_rlogits, void* d_v, void* d_gamma, float* d_slot0,
                 float* d_mass0, void* stream) {
  Dims d;
  int st = check_problem(p, &d);
  if (st != RAM_OK) return st;
  if (!ws) return RAM_EINVAL;
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
  char* w = (char*)ws;
  hipStream_t s = (hipStream_t)stream;
  const bool bf = p->io_dtype == RAM_BF16;
  hipError_t e;

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
  sb.long_cap = long_cap(d);
  sb.use_long = d.ntiles > 0;
  sb.seg_offset = (const int32_t*)(w + L.seg_offset);
  sb.events = (const EventRec*)(w + L.events);
  sb.v = v;
  sb.d_o = d_o;
  sb.slot0 = slot0;
  sb.mass0 = mass0;
  sb.ckpt_s = (const float*)(w + L.ckpt_s);
  sb.ckpt_m = (const float*)(w + L.ckpt_m);
  sb.d_slot1 = d_slot1;
  sb.d_mass1 = d_mass1;
  sb.d_slot0 = d_slot0;
  sb.d_mass0 = d_mass0;
  sb.stash = w + L.stash;
  sb.dw = (float*)(w + L.dw);
  sb.dr = (float*)(w + L.dr);
  sb.dgam = (float*)(w + L.dgam);
  prof_before("scan_bwd", s);
  e = forked(s, [&](hipStream_t m, hipStream_t x) { return launch_scan_bwd(sb, bf, m, x); });
  prof_after("scan_bwd", s);
  if (e != hipSuccess) return RAM_EHIP;

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
  db.nsides = 2;
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
  return hip_status(e);
}

int ram_decode_step(const ram_problem* p, const void* wlogits, const void* rlogits, const void* v,
                    const void* gamma, float* slot, float* mass, void* o, void* stream) {
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
  a.d_v = p->d_v;
  a.k_w = p->k_w;
  a.k_r = p->k_r;
  a.renorm_w = p->renorm_w;
  a.renorm_r = p->renorm_r;
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
