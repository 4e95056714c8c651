// Argument blocks and host launchers of the bucketing, scan and step kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ramk {

constexpr int CHUNK = 16;        // scan chunk: 16 events from the segment start
constexpr int NWL = 4;           // waves per long-segment scan workgroup
constexpr int SHORT_WAVES = 4;   // waves (one short segment each) per short-segment workgroup
constexpr int LONG_EVENTS = 128; // segments with more events take the cooperative path
constexpr int NBIN = 8;          // length classes of the long-segment list: class c holds
                                 // segments of [129 * 2^c, 129 * 2^(c+1)) events (the last
                                 // class is open-ended); scans take the longest first
constexpr int SHORT_WORD = 32;        // a 128-byte line of its own: the work queues' atomics
                                      // would hold up its many reads
constexpr int LONG_WORDS = SHORT_WORD + 1;  // int32 words per long-segment list header:
                                      //   [0, NBIN)  entries per class
                                      //   NBIN, +1   forward scan: next ticket, finished workgroups
                                      //   NBIN+2, +3 reverse scan: the same
                                      //   SHORT_WORD entries of the short-segment list
constexpr int SCAN_SLOTS = 1024; // slots per workgroup of the bucketing scan
constexpr int MAX_DV = 128;      // widest slot
constexpr uint32_t MAX_BUF_BYTES = 0x7FE00000u;  // one batch's v, dO or stash rows (scans)

// One event of the segment lists: 16 bytes, read with one vector load.
struct EventRec {
  int32_t code;           // (t << 7) | (side << 6) | j; bit 31: a masked token's no-op event
  float w;                // write weight or read weight
  float lam;              // retention of a write (1 for a read)
  float dlam;             // d lambda / d w of a write (0 for a read)
};

struct BucketArgs {
  const int32_t* idx_w;   // (N, k_w)
  const int32_t* idx_r;   // (N, k_r)
  const float* w_w;       // (N, k_w)
  const float* w_r;       // (N, k_r)
  const void* gamma;      // (N) io
  const uint8_t* mask;    // (B, T): nonzero = valid token, or null (all valid)
  int B, H, T, S, k_w, k_r;
  int tile;               // tokens per bucketing tile
  int ntiles;             // ceil(T / tile)
  int nbits;              // bits needed for a slot index
  int32_t* tile_hist;     // (B*H, ntiles, S)
  int32_t* blk_tot;       // (B*H, nblk): events of each block of SCAN_SLOTS slots
  int nblk;               // ceil(S / SCAN_SLOTS)
  int32_t* seg_offset;    // (B*H*S + 1): absolute positions in `events`
  int64_t ev_base;        // position of these rows' first event (B counts the batches
                          // of this call's piece; events is the whole list)
  EventRec* events;       // (all events of the call)
  int32_t* long_list;     // (NBIN, long_cap): segments with more than LONG_EVENTS events
  int32_t* long_count;    // (LONG_WORDS): entries per class, the scans' work queues, the
                          // short-list length
  int long_cap;
  int32_t* short_list;    // (B*H*S at most): segments with 1 to LONG_EVENTS events
};

struct ScanFwdArgs {
  int B, H, T, S, d_v, k_w, k_r;
  float eps;
  int64_t nseg;
  const int32_t* long_list;   // (NBIN, long_cap)
  const int32_t* long_count;  // (NBIN)
  int32_t* queue;             // (2): next ticket, finished workgroups; zero at launch
  int long_cap;
  int use_long;           // long_list / long_count / short_list are valid
  const int32_t* short_list;  // segments with 1 to LONG_EVENTS events
  const int32_t* short_count; // its length
  const int32_t* seg_offset;
  const EventRec* events;
  const void* v;          // (N, d_v) io
  const float* slot0;     // (B*H*S, d_v) or null
  const float* mass0;     // (B*H*S) or null
  float* slot1;
  float* mass1;
  void* stash;            // (N, k_r, d_v) io: read contributions r*s
  float* ckpt_s;          // (E/CHUNK + 1, d_v)
  float* ckpt_m;          // (E/CHUNK + 1)
};

struct ScanBwdArgs {
  int B, H, T, S, d_v, k_w, k_r;
  float eps;
  int64_t nseg;
  const int32_t* long_list;
  const int32_t* long_count;
  int32_t* queue;         // (2), as in the forward
  int long_cap;
  int use_long;
  const int32_t* short_list;
  const int32_t* short_count;
  const int32_t* seg_offset;
  const EventRec* events;
  const void* v;          // io
  const void* d_o;        // (N, d_v) io
  const float* slot0;     // or null
  const float* mass0;     // or null
  const float* ckpt_s;
  const float* ckpt_m;
  const float* d_slot1;   // or null
  const float* d_mass1;   // or null
  float* d_slot0;         // or null
  float* d_mass0;         // or null
  void* stash;            // (N, k_w, d_v) io: dv contributions eta*s_hat
  float* dw;              // (N, k_w)
  float* dr;              // (N, k_r)
  float* dgam;            // (N, k_w) per-write gamma gradient parts
};

struct FinalizeArgs {
  int64_t N;
  int d_v, k;
  const void* stash;      // (N, k, d_v) io
  void* out;              // (N, d_v) io
  const float* dgam;      // (N, k) or null
  void* d_gamma;          // (N) io or null
};

// Read epilogue y = sigmoid(gate) * RMSNorm(o) fused into the read-out.
constexpr int EPI_BWD_WAVES = 8192;   // waves of the epilogue backward (gain partial sums)
struct EpilogueArgs {
  int64_t N;              // (token, head) rows
  int d_v, k;             // k = k_r: read contributions per row in the stash
  int T, H;               // row r is token (r / H) % T of batch r / (T * H)
  const void* stash;      // (N, k, d_v) io: read contributions of the forward
  const void* gate;       // (N, d_v) io: gate pre-activations
  const float* gain;      // (d_v) or null (ones)
  float eps;
  void* y;                // forward: (N, d_v) io
  const void* d_y;        // backward: (N, d_v) io
  void* d_o;              // backward: (N, d_v) io, input of the reverse scan
  void* d_gate;           // backward: (N, d_v) io
  float* part;            // backward: (EPI_BWD_WAVES, d_v) gain partial sums
  float* d_gain;          // backward: (d_v) or null
  const uint8_t* mask;    // (B, T) or null: masked rows get zero gradients
};

struct StepArgs {
  int B, H, S, d_v, k_w, k_r, renorm_w, renorm_r;
  int U, P;               // address digits and digit size (S = P^U)
  int cape_heads;         // heads h < cape_heads address (content index + t0) mod S
  int64_t t0;             // absolute position of the token
  const uint8_t* mask;    // (B): nonzero = valid token, or null
  float eps;
  const void* wl;         // (B*H, U * P) io
  const void* rl;
  const void* v;          // (B*H, d_v) io
  const void* gamma;      // (B*H) io
  float* slot;            // (B*H*S, d_v)
  float* mass;            // (B*H*S)
  void* o;                // (B*H, d_v) io
};

hipError_t launch_bucket(const BucketArgs& a, bool bf16, hipStream_t st,
                         void (*before)(const char*, hipStream_t),
                         void (*after)(const char*, hipStream_t));
// Short-segment kernel on `side`, long-segment kernel on `st`; the caller
// makes both streams wait for the inputs and joins them afterwards.
hipError_t launch_scan_fwd(const ScanFwdArgs& a, bool bf16, hipStream_t st, hipStream_t side);
hipError_t launch_scan_bwd(const ScanBwdArgs& a, bool bf16, hipStream_t st, hipStream_t side);
hipError_t launch_finalize(const FinalizeArgs& a, bool bf16, hipStream_t st);
hipError_t launch_step(const StepArgs& a, bool bf16, hipStream_t st);
hipError_t launch_epilogue_fwd(const EpilogueArgs& a, bool bf16, hipStream_t st);
hipError_t launch_epilogue_bwd(const EpilogueArgs& a, bool bf16, hipStream_t st);

}  // namespace ramk
