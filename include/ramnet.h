/*
 * ramnet.h -- C ABI of the RAM-Net attention core on AMD Instinct MI355X
 * (gfx950).  Plain pointers and sizes only; no framework types.
 *
 * What the calls compute (sources: the paper page "RAM-Net: Linear-Time
 * Sequence Modeling with Sparsely Addressable State", and the "ramnet-ops
 * 0.1.0rc0" PyPI project page):
 *
 *   state       per (batch b, head h) an array of S slots; slot a holds a
 *               content row s[a] (d_v floats) and a mass m[a] (paper §3.1;
 *               ramnet-ops "Quick start": slot (B,H,P^U,C), mass (B,H,P^U)).
 *   decode      per token, head and side (write side from the key logits,
 *               read side from the query logits): softmax over the S slots,
 *               keep the K most probable by (logit descending, slot index
 *               ascending), weights = their probabilities, optionally
 *               renormalised to sum 1 (paper §3.2, App. B.2 "Addressing";
 *               ramnet-ops "Arguments": top_k, top_k_re_norm).
 *               With U >= 2 digits (product softmax, paper §3.2 and App.
 *               B.1) a row holds U digit logit vectors of P entries; slot
 *               a = sum_u a_u P^(U-1-u) has probability prod_u
 *               softmax(l_u)[a_u] and is ranked by its key, the float32 sum
 *               l_0[a_0] + l_1[a_1] + ... taken in ascending u from 0
 *               (log-space score, paper §4 "Efficient Address Decoding");
 *               the K best by (key desc, index asc) are found exactly by a
 *               pruned prefix search.
 *   write (GSU) for each selected write slot a with weight w and the token's
 *               forgetting modulator gamma (paper §3.4 "Gated Sparse Update"):
 *                 lambda = sigmoid(logit(1-w) - gamma)
 *                 m[a]   <- lambda * m[a] + w
 *                 eta    = w / (m[a] + eps)
 *                 s[a]   <- (1 - eta) * s[a] + eta * v_t
 *               every other slot is left bit-for-bit unchanged.
 *   read        o_t = sum_j r_j * s[a_j] over the selected read slots, with
 *               the state after token t's writes (paper §3.4 "Read-out").
 *   order       tokens in time order; slot-parallel execution groups the
 *               events of each (b, h, slot) and applies them in time order
 *               (paper §4 "Slot-Parallel Execution"; ramnet-ops "CUDA
 *               execution", parallel and autoregressive modes).
 *
 *   CAPE        heads h < cape_heads address slot (a + t0 + t) mod S for the
 *               content-selected index a of token t (ramnet-ops "Quick start",
 *               embed_num; paper App. C); selection and its tie order stay on
 *               the content logits, gradients flow to logit a.
 *
 * Supported: 1 <= U <= 14 digits with S = P^U <= 16384.  One batch's rows of v (and of the read-out
 * and gradient staging, T*H*max(k_w, k_r)*d_v io values) must fit in
 * 0x7FE00000 bytes, else RAM_ECAPACITY (split T over calls).
 *
 * Layouts (all row-major, contiguous, device memory):
 *   logits  (B, T, H, U, P)  io dtype     wlogits: write side, rlogits: read side
 *                                         (U = 1: (B, T, H, S))
 *   v, o    (B, T, H, d_v)   io dtype
 *   gamma   (B, T, H)        io dtype
 *   slot    (B, H, S, d_v)   float32
 *   mass    (B, H, S)        float32
 * io dtype is float32 or bfloat16 (RAM_F32 / RAM_BF16); all arithmetic is
 * float32 and the state is float32.  o and d_v are sums over the K selected
 * slots of one token; each of the K terms is rounded to the io dtype before
 * the float32 sum, which is then rounded (to nearest even) once more.
 *
 * Ownership and streams: the caller allocates every buffer, including the
 * workspace (size from ram_workspace_size).  The library never allocates or
 * frees device memory and never blocks the host.  All work is ordered on the
 * given HIP stream (a hipStream_t passed as void*, NULL = default stream):
 * parts of ram_forward and ram_backward run on a library-owned stream of the
 * same device, which first waits for the work already on the given stream
 * and which the given stream then waits for (event fork and join;
 * capturable in a graph); calls from several host threads are serialised
 * inside the library.  Pointers to logits must be 16-byte aligned; with
 * U = 1, S times the io size must be a multiple of 16.
 *
 * Errors: every call returns RAM_OK (0) or a negative code; nothing is
 * enqueued when validation fails.  There is no fallback path.
 */
#ifndef RAMNET_H
#define RAMNET_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RAM_OK 0
#define RAM_EINVAL (-1)       /* bad shape, null pointer, k > S, misalignment  */
#define RAM_EDTYPE (-2)       /* io_dtype not RAM_F32 / RAM_BF16               */
#define RAM_ECAPACITY (-3)    /* too many events or tokens, workspace too small */
#define RAM_EUNSUPPORTED (-4) /* S = P^U > 16384 or U > 14                       */
#define RAM_EHIP (-5)         /* HIP launch or runtime error                    */

#define RAM_F32 0
#define RAM_BF16 1

/* One problem description, passed to every call. */
typedef struct ram_problem {
  int32_t B, H, T;      /* batch, heads, tokens in this call (T = 1 for ram_decode_step) */
  int32_t U, P;         /* address digits (1..14) and digit size; S = P^U <= 16384 slots */
  int32_t k_w, k_r;     /* top-K of the write and read side: 1 <= k <= min(S, 64)        */
  int32_t d_v;          /* slot / value width: 1..64, or an even number 66..128          */
  int32_t io_dtype;     /* RAM_F32 or RAM_BF16 for logits, v, gamma, o and gradients    */
  float eps;            /* GSU epsilon (finite, >= 0; the paper's default reading 1e-6) */
  int32_t renorm_w;     /* 1: renormalise the kept write weights to sum 1               */
  int32_t renorm_r;     /* 1: same for the read side                                    */
  int32_t cape_heads;   /* heads h < cape_heads use CAPE, 0 <= cape_heads <= H          */
  int32_t reserved;     /* must be 0                                                    */
  int64_t t0;           /* absolute position (>= 0) of token 0 (CAPE only)              */
} ram_problem;

/* Byte offsets of the arrays that ram_forward leaves in the workspace for
 * ram_backward (and for inspection).  N = B*T*H rows, E = N*(k_w+k_r) events. */
typedef struct ram_ws_layout {
  size_t idx_w;       /* int32 (N, k_w): selected write slots, sorted by (logit desc, index asc) */
  size_t w_w;         /* float (N, k_w): their weights                                          */
  size_t lse_w;       /* float (N, U): logsumexp of each digit of the write logits             */
  size_t idx_r;       /* int32 (N, k_r)                                                           */
  size_t w_r;         /* float (N, k_r)                                                           */
  size_t lse_r;       /* float (N, U)                                                             */
  size_t seg_offset;  /* int32 (B*H*S + 1): first event of segment g = (b*H + h)*S + a          */
  size_t events;      /* (E) 16-byte records {int32 code, float weight, float lambda, float
                         d lambda/d w}; code = (t << 7) | (side << 6) | j, bit 31 set for
                         the (weight 0, no-op) events of masked tokens; segment-major, time
                         order inside a segment, a token's write before its read            */
  size_t ckpt_s;      /* float (E/16 + 1, d_v): slot content before every 16-event chunk of a
                         segment but its first (chunks counted from the segment's first
                         event), at index (chunk's first event) / 16                         */
  size_t ckpt_m;      /* float (E/16 + 1): slot mass at the same points                      */
  size_t stash;       /* io (N, k_r, d_v): read contributions r_j * s_t[a_j] of each (token, j) */
  size_t tile_hist;   /* int32: bucketing scratch                                              */
  size_t long_list;   /* int32: segments that take the cooperative scan path                   */
  size_t long_count;  /* int32: their number per length class, the scans' work counters, and
                         the length of short_list                                              */
  size_t short_list;  /* int32: segments with 1 to 128 events (slots without events need no
                         scan)                                                                 */
  size_t stash_b;     /* io (N, k_w, d_v): backward scratch, d_v contributions of each write     */
  size_t dw;          /* float (N, k_w): gradient of each write weight                          */
  size_t dr;          /* float (N, k_r): gradient of each read weight                           */
  size_t dgam;        /* float (N, k_w): gamma gradient part of each write                      */
  size_t epi_d_o;     /* io (N, d_v): gated backward, gradient of o                              */
  size_t epi_part;    /* float (8192, d_v): gated backward, gain gradient partial sums           */
  size_t fwd_bytes;   /* workspace bytes ram_forward needs                                      */
  size_t total_bytes; /* workspace bytes ram_forward + ram_backward need                       */
} ram_ws_layout;

/* Workspace size for a forward (with_backward = 0) or a forward that a
 * backward will follow (with_backward = 1). */
int ram_workspace_size(const ram_problem* p, int with_backward, size_t* bytes);

/* Offsets of the saved arrays inside the workspace. */
int ram_workspace_layout(const ram_problem* p, ram_ws_layout* out);

/* Address decode of one side (paper §3.2): for every row (b, t, h) of
 * logits (B,T,H,U,P), writes idx (B,T,H,k) int32 with the K selected flat
 * slots in (key desc, index asc) order (U = 1: the key is the logit; CAPE
 * heads: the addressed slot, i.e. the selected index shifted as above),
 * weight (B,T,H,k) float with their probabilities exp(sum_u (l_u[a_u] -
 * lse_u)) (renormalised if the side's renorm flag is set) and lse (B,T,H,U)
 * float, the logsumexp of each digit.  side: 0 write (k_w, renorm_w), 1 read. */
int ram_decode(const ram_problem* p, int side, const void* logits, int32_t* idx, float* weight,
               float* lse, void* stream);

/* Parallel (training / prefill) forward over T tokens: decode both sides,
 * bucket events into per-slot segments, run the GSU scan per segment and
 * accumulate the reads into o.  slot0 / mass0: initial state, or both NULL
 * for empty slots (content 0, mass 0) (ramnet-ops "Arguments": init_ram).
 * mask: (B, T) uint8, nonzero = valid token, or NULL for all valid
 * (ramnet-ops "Arguments": masked tokens are not written and their outputs
 * are to be ignored); a masked token is absent: it writes and reads nothing
 * and its o row is 0.  Allocations do not depend on the mask.
 * Writes o, slot1, mass1.  slot1 / mass1 may alias slot0 / mass0 (in-place
 * continuation, ramnet-ops inplace) only when no ram_backward follows.
 * ws: workspace of at least ram_workspace_size bytes; it keeps what the
 * backward needs and must stay untouched until then. */
int ram_forward(const ram_problem* p, const void* wlogits, const void* rlogits, const void* v,
                const void* gamma, const uint8_t* mask, const float* slot0, const float* mass0,
                void* o, float* slot1, float* mass1, void* ws, size_t ws_bytes, void* stream);

/* First-order backward (ramnet-ops "Autograd and compile") of the forward
 * that filled ws (same problem, same inputs, mask, slot0 / mass0 as given to
 * it); masked tokens get zero gradients.
 * d_o: gradient of o; d_slot1 / d_mass1: gradients of the final state, NULL
 * for zero.  Writes d_wlogits, d_rlogits (B,T,H,U,P) io, d_v (B,T,H,d_v) io,
 * d_gamma (B,T,H) io, and, when non-NULL, d_slot0 (B,H,S,d_v) / d_mass0
 * (B,H,S) float.  ws must have been sized with with_backward = 1.  The
 * backward keeps its own scratch and work counters in ws, which it leaves
 * as it found them: several ram_backward calls after one ram_forward each
 * give the same result, but calls that share one workspace must not overlap
 * on the device (order them on one stream). */
int ram_backward(const ram_problem* p, void* ws, size_t ws_bytes, const void* wlogits,
                 const void* rlogits, const void* v, const void* gamma, const uint8_t* mask,
                 const float* slot0, const float* mass0, const void* d_o, const float* d_slot1,
                 const float* d_mass1, void* d_wlogits, void* d_rlogits, void* d_v, void* d_gamma,
                 float* d_slot0, float* d_mass0, void* stream);

/* Gated read-out (paper §3.4 "Read-out", last step; Fig. 2): the read o of
 * each (token, head) goes through a head-wise RMSNorm and a sigmoid output
 * gate, y = sigmoid(gate) * (o / sqrt(mean_c o_c^2 + eps) * gain), the mean
 * over the d_v channels of the row.  The output projection is the caller's.
 *   gate  (B,T,H,d_v) io: gate pre-activations (x W_g plus its bias)
 *   gain  (d_v) float32, or NULL for all ones
 *   eps   RMSNorm epsilon, finite and >= 0 */
typedef struct ram_epilogue {
  const void* gate;
  const float* gain;
  float eps;
} ram_epilogue;

/* ram_forward with the gated read-out fused into the read: writes y
 * (B,T,H,d_v) io instead of o (o itself is not written; the arithmetic of o
 * is that of ram_forward, kept in float32 for the norm).  A masked token's
 * y row is 0.  ws as for ram_forward. */
int ram_forward_gated(const ram_problem* p, const ram_epilogue* ep, const void* wlogits,
                      const void* rlogits, const void* v, const void* gamma, const uint8_t* mask,
                      const float* slot0, const float* mass0, void* y, float* slot1, float* mass1,
                      void* ws, size_t ws_bytes, void* stream);

/* Backward of ram_forward_gated (same problem, ep, inputs and ws): d_y is
 * the gradient of y; writes everything ram_backward writes, plus d_gate
 * (B,T,H,d_v) io and, when non-NULL, d_gain (d_v) float32 summed over all
 * rows in a fixed order (deterministic).  o is recomputed from the read
 * contributions the forward left in ws.  Masked tokens get zero d_gate and
 * add nothing to d_gain. */
int ram_backward_gated(const ram_problem* p, const ram_epilogue* ep, void* ws, size_t ws_bytes,
                       const void* wlogits, const void* rlogits, const void* v, const void* gamma,
                       const uint8_t* mask, const float* slot0, const float* mass0,
                       const void* d_y, const float* d_slot1, const float* d_mass1,
                       void* d_wlogits, void* d_rlogits, void* d_v, void* d_gamma, void* d_gate,
                       float* d_gain, float* d_slot0, float* d_mass0, void* stream);

/* Autoregressive step (ramnet-ops "CUDA execution", autoregressive mode;
 * paper §4: each new token updates and reads its own K slots): p->T == 1;
 * decode both sides of the one token per (b, h), apply its k_w writes to
 * slot / mass in place, then read its k_r slots into o (B,1,H,d_v); o is
 * the float32 sum of the K terms, rounded once to the io dtype.  For CAPE,
 * t0 is the position of this token.  mask: (B) uint8 or NULL; a masked
 * sequence's state is untouched and its o rows are 0.  Needs
 * k_w * d_v <= 8192.  No workspace. */
int ram_decode_step(const ram_problem* p, const void* wlogits, const void* rlogits, const void* v,
                    const void* gamma, const uint8_t* mask, float* slot, float* mass, void* o,
                    void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments (less the workspace), kernels and results as
 * ram_forward.  Its workspace is an array of RAM_NOALLOC_SCRATCH_BYTES that
 * the library holds on each device it runs on, from the library's load on
 * that device until the process ends; the call itself allocates nothing and
 * creates no stream or event, and every kernel runs on the given stream.
 * A problem whose forward workspace (ram_workspace_size with
 * with_backward = 0) exceeds the array returns RAM_ECAPACITY with nothing
 * enqueued (64 MiB holds the 340M-layer shape, B=4, H=8, T=2048, S=1024,
 * k=4, d_v=64, and 1,024 tokens of 16 heads at S=4096, k=8, d_v=128).
 * Every call on a device shares that device's array and leaves its contents
 * to the next call: calls that overlap on one device (several streams or
 * host threads) race and must be ordered by the caller, and no ram_backward
 * can follow (use ram_forward with a workspace for training). */
#define RAM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int ram_forward_noalloc(const ram_problem* p, const void* wlogits, const void* rlogits,
                        const void* v, const void* gamma, const uint8_t* mask, const float* slot0,
                        const float* mass0, void* o, float* slot1, float* mass1, void* stream);

/* Text of a status code (static storage). */
const char* ram_status_string(int status);

/* Measurement only (not part of the method): the HBM streaming roofs the
 * decoders work against.  Streams `bytes` from src with the decoders' access
 * pattern (a wave reads one contiguous row with 16-byte vector loads, all of
 * its loads in flight at once) and, with mode 1, writes it to dst (a copy,
 * the pattern of a decode backward row: read a row, write a row); mode 0
 * only reads.  variant: 0 = 8 KiB rows, 4 waves per workgroup, nontemporal
 * loads and stores (the forward decoder's own); 1 = the same with plain
 * loads and stores; 2 = 16 KiB rows; 3 = 4 KiB rows; 4 = 8 waves per
 * workgroup; 5 = 1 KiB rows, one wave per workgroup (the decode backward's
 * own); 6 = 2 KiB rows, one wave per workgroup.  src
 * and dst are device buffers of `bytes` each, 16-byte aligned; bytes must be a
 * multiple of the variant's workgroup tile (128 KiB covers every variant),
 * else RAM_EINVAL.  Asynchronous on the given stream. */
int ram_stream_probe(int mode, int variant, const void* src, void* dst, size_t bytes,
                     void* stream);

/* Optional kernel timing: while enabled, every kernel the library launches
 * is bracketed by HIP events on its stream.  ram_prof_collect waits for
 * those events and returns, per kernel name, the launch count and summed
 * milliseconds since the last enable. */
typedef struct ram_prof_entry {
  char name[32];
  int64_t launches;
  double total_ms;
} ram_prof_entry;
int ram_prof_enable(int on);
int ram_prof_collect(ram_prof_entry* out, int max_entries, int* n_entries);

#ifdef __cplusplus
}
#endif

#endif /* RAMNET_H */
